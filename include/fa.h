/*
 * fa.h - exact attention forward and backward passes on AMD Instinct MI355X (gfx950).
 *
 * Computes, for every batch b and head h,
 *
 *     O = softmax(scale * Q K^T) V,      LSE_i = ln( sum_j exp(scale * q_i . k_j) )
 *
 * tile by tile with an online softmax, so the N x N score and probability
 * matrices never reach device memory. Definitions: the three-step attention of
 * the introduction of "FlashAttention · InkStack" (S = QK^T, P = softmax(S),
 * O = PV) and of the MUSA guide "FlashAttention 优化"; the per-row statistic
 * L = m + log(l) of "FlashAttention · InkStack" section 2.1, written here in
 * natural log of the scaled logits; the causal mask of section 1.1.3 of the
 * same page, with key j hidden from query i when j > i.
 *
 * Layout (all tensors dense, row-major, no strides):
 *     q, k, v, o : [B][H][N][d], head dimension innermost (each row holds one
 *                  head's d elements, the convention of the FA3 walkthrough
 *                  "FlashAttention 完全拆解（三）", FP8 layout section)
 *     lse        : [B][H][N] float32, natural log
 *
 * Ownership: the caller owns every buffer (device memory). The library never
 * allocates, frees or keeps a pointer after the call returns. Outputs must not
 * overlap inputs. Every base pointer must be 16-byte aligned.
 *
 * Streams: `stream` is a hipStream_t (NULL = the default stream). Calls are
 * asynchronous: they enqueue their kernels (one; two for a split-KV call; three
 * for the backward) on `stream` and return. The library may be called from
 * several threads at once. Its only global state is the per-device scratch
 * array of fa_fwd_kv_noalloc and the cached device addresses of that array.
 *
 * Errors: arguments are validated on the host before any HIP call, so
 * FA_ERR_INVALID_ARG (and FA_ERR_UNSUPPORTED for a shape) means nothing was
 * launched and nothing was written. A launch failure in a call of several
 * kernels (FA_ERR_LAUNCH, or FA_ERR_UNSUPPORTED when the device has no gfx950
 * code) stops at the failing kernel; the outputs are then undefined.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* return codes */
#define FA_OK               0
#define FA_ERR_INVALID_ARG (-1)  /* null pointer, negative size, bad scale, misaligned, bad dtype/causal */
#define FA_ERR_UNSUPPORTED (-2)  /* head dimension not in {64, 128}; no gfx950 code for this device */
#define FA_ERR_LAUNCH      (-3)  /* the HIP launch itself failed */
#define FA_ERR_TOO_LARGE   (-4)  /* fa_fwd_kv_noalloc: partials exceed FA_NOALLOC_SCRATCH_BYTES */

/* bytes of the static per-device scratch array of fa_fwd_kv_noalloc */
#define FA_NOALLOC_SCRATCH_BYTES (16u << 20)

/* element types of q, k, v */
#define FA_F16       0   /* IEEE binary16; o is f16 */
#define FA_BF16      1   /* bfloat16;      o is bf16 */
#define FA_FP8_E4M3  2   /* OCP e4m3fn;    only through fa_fwd_fp8, o is bf16 */

#define FA_VERSION 120   /* 1.2.0 */

/*
 * fa_fwd - attention forward for f16 or bf16 inputs.
 *
 *   q, k, v  device pointers to B*H*N*d elements of `dtype`
 *   o        device pointer to B*H*N*d elements of `dtype` (written)
 *   lse      device pointer to B*H*N float32 (written), natural log
 *   B, H, N  batch, heads, sequence length (queries = keys = N); any value
 *            >= 0; if any is 0 the call returns FA_OK and launches nothing
 *   d        head dimension, 64 or 128
 *   scale    logit multiplier, finite and > 0 (usually 1/sqrt(d))
 *   causal   0 = full attention, 1 = key j is masked for query i when j > i
 *   dtype    FA_F16 or FA_BF16 (FA_FP8_E4M3 returns FA_ERR_UNSUPPORTED:
 *            use fa_fwd_fp8, which carries the per-tensor descales)
 *   stream   hipStream_t or NULL
 *
 * Inside, the scores are accumulated in fp32, the probabilities are rounded to
 * `dtype` (round to nearest even) before the second product, the row sums
 * l are accumulated from the unrounded fp32 probabilities, and O is rounded
 * to `dtype` once, after the single division by l (deferred normalisation,
 * "FlashAttention · InkStack" section 2.1).
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, int dtype,
           void* stream);

/*
 * fa_fwd_fp8 - attention forward for OCP e4m3fn inputs with per-tensor scales.
 *
 * The real inputs are q8 * q_descale, k8 * k_descale, v8 * v_descale, where
 * each descale is the tensor's amax / 448 (per-tensor scaling, "FlashAttention
 * · InkStack" section 3.3.3). Both products run on the fp8 matrix cores with
 * fp32 accumulation; the probabilities are quantised to e4m3fn with unit
 * scale before the second product; o is bf16 (B*H*N*d elements), lse is
 * float32 as for fa_fwd. Descales must be finite and > 0. Other arguments,
 * layout and errors as fa_fwd.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               float q_descale, float k_descale, float v_descale,
               int B, int H, int N, int d, float scale, int causal,
               void* stream);

/*
 * fa_fwd_fp8_block - fa_fwd_fp8 with one scale per block instead of per
 * tensor (block quantisation: "FlashAttention · InkStack" 3.3.1, the FP8
 * section of the FA3 walkthrough).
 *
 *   q_scale  device pointer, B*H*ceil(N/128) float32: the scale of each
 *            128-row query block, [B][H][N/128]
 *   k_scale, v_scale   device pointers, B*H*ceil(N/64) float32: the scale of
 *            each 64-row key and value block, [B][H][N/64]
 *   q, k, v  e4m3 codes; element (b, h, i, c) stands for code * the scale of
 *            its block. All scales must be positive and finite.
 *
 * The per-block factors enter the logit multiplier (q and k) and the
 * probabilities of each key tile (v, relative to the head's largest v
 * scale). N is limited to 131072 (FA_ERR_UNSUPPORTED above). Other arguments,
 * layout, ownership, errors and rounding as fa_fwd_fp8; the scale arrays must
 * not overlap o or lse.
 */
int fa_fwd_fp8_block(const void* q, const void* k, const void* v, void* o, float* lse,
                     const float* q_scale, const float* k_scale, const float* v_scale,
                     int B, int H, int N, int d, float scale, int causal, void* stream);

/*
 * fa_quantize_fp8 - f16/bf16 -> OCP e4m3 codes with one scale per block of
 * rows, optionally after the incoherent transform ("FlashAttention ·
 * InkStack" 3.3.1-3.3.3).
 *
 *   x        device pointer, B*H*N*d elements of `dtype` (FA_F16 or
 *            FA_BF16), [B][H][N][d]
 *   x8       device pointer, B*H*N*d bytes (written): e4m3 codes
 *   scales   device pointer, B*H*ceil(N/block_rows) float32 (written), one
 *            per block of block_rows rows of each (b, h): s = amax / 448
 *            (1 for an all-zero block); code = e4m3(y / s), rounded to
 *            nearest even, with y / s and s formed by IEEE float32 division
 *   signs    NULL: y = x. Else a device pointer to d float32 values, each +1
 *            or -1: y = x diag(signs) H_d / sqrt(d), with H_d the
 *            Sylvester-Hadamard matrix (fast Walsh-Hadamard transform in
 *            float32). Applied with the same signs to q and k, Q K^T is
 *            unchanged; v must not be transformed.
 *   block_rows  64 or 128 (FA_ERR_UNSUPPORTED otherwise): use 128 for q and
 *            64 for k and v to feed fa_fwd_fp8_block
 *   d        64 or 128
 *
 * x, x8 and signs 16-byte aligned, scales 4-byte aligned; outputs must not
 * overlap the inputs or each other. One kernel is queued on `stream`;
 * nothing is launched on an error, and B*H*N = 0 returns FA_OK.
 */
int fa_quantize_fp8(const void* x, void* x8, float* scales, const float* signs,
                    int B, int H, int N, int d, int block_rows, int dtype,
                    void* stream);

/*
 * fa_fwd_kv - attention forward with grouped key/value heads and a key/value
 * history, optionally split over key ranges (decoding).
 *
 *   q, o   [B][H][Nq][d] elements of `dtype`;  lse [B][H][Nq] float32
 *   k, v   [B][Hkv][Nk][d] elements of `dtype`; H must be a multiple of Hkv,
 *          and query head h reads key/value head h / (H / Hkv) (grouped- and
 *          multi-query attention, the "qhead_per_kvhead" sharing of the FA4
 *          walkthrough, section 3.3)
 *   Nq, Nk the queries are the last Nq of Nk positions: with causal = 1, query
 *          i sees key j only if j <= i + (Nk - Nq) (requires Nq <= Nk); for
 *          Nq = Nk, H = Hkv this is fa_fwd
 *   num_splits  1: one pass per query tile. >1: the keys are cut into that many
 *          ranges computed in parallel, each giving a partial O and LSE, then
 *          merged as LSE = log sum exp(LSE_s), O = sum exp(LSE_s - LSE) O_s
 *          (split-KV decoding, same walkthrough section; the merge of
 *          "FlashAttention · InkStack" 2.2). Between 1 and 1024.
 *   workspace   num_splits > 1: device memory of fa_fwd_kv_workspace(B, H, Nq,
 *          d, num_splits) bytes, owned by the caller, overwritten; else unused
 *          (may be NULL)
 *   other arguments, ownership, errors and rounding as fa_fwd. Query heads
 *   sharing a K/V head are processed together, so each K/V tile read from
 *   memory serves all of them.
 */
size_t fa_fwd_kv_workspace(int B, int H, int Nq, int d, int num_splits);
int fa_fwd_kv(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int H, int Hkv, int Nq, int Nk, int d, float scale,
              int causal, int dtype, int num_splits, float* workspace,
              void* stream);

/*
 * fa_fwd_kv_noalloc - fa_fwd_kv with no workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc). It calls no allocating routine: the
 * key-range partials go to a static device array of FA_NOALLOC_SCRATCH_BYTES
 * (16 MiB) that the library's code object holds on every GPU it runs on,
 * until the process ends. Results equal fa_fwd_kv's with the same num_splits
 * bit for bit (the same kernels run).
 *
 *   arguments   as fa_fwd_kv, without `workspace`
 *   limit       fa_fwd_kv_workspace(B, H, Nq, d, num_splits) must not exceed
 *               FA_NOALLOC_SCRATCH_BYTES, else FA_ERR_TOO_LARGE (checked on the
 *               host, nothing launched). num_splits = 1 needs no scratch.
 *   device      the scratch of the device `stream` belongs to (the current
 *               device for a NULL stream); its address is looked up once per
 *               device, on the first call there
 *   concurrency every call on a GPU shares that GPU's array: calls that can
 *               overlap in time on one GPU (other streams, other threads)
 *               race and must be serialised by the caller
 */
int fa_fwd_kv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int Hkv, int Nq, int Nk, int d, float scale,
                      int causal, int dtype, int num_splits, void* stream);

/*
 * fa_fwd_varlen - fa_fwd_kv over a batch of sequences of different lengths,
 * packed token-major without padding (variable-length batching; the query
 * heads of one K/V head are processed together as in fa_fwd_kv).
 *
 *   q, o   [total_q][H][d] elements of `dtype`;  lse [total_q][H] float32
 *   k, v   [total_k][Hkv][d] elements of `dtype`; H a multiple of Hkv
 *   cu_seqlens_q, cu_seqlens_k   device pointers to B+1 int32 offsets each:
 *          sequence b owns query tokens cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1
 *          and key tokens cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1; offsets are
 *          nondecreasing from 0 to total_q (total_k). The kernels read them on
 *          the device and clamp every offset to [0, total] and every length to
 *          max_seqlen_q (max_seqlen_k), so malformed offsets give wrong results,
 *          never accesses outside the tensors
 *   order  NULL, or a device pointer to B int32: a permutation of 0..B-1 that
 *          the kernel walks instead of the input order (virtual sequence v runs
 *          sequence order[v]), normally written by fa_varlen_order so that the
 *          heaviest tiles start first. The results do not depend on it: every
 *          output row is computed the same way in any order. Entries are
 *          clamped to 0..B-1; an order that is not a permutation leaves some
 *          sequences unwritten
 *   max_seqlen_q, max_seqlen_k   upper bounds of the sequence lengths (they size
 *          the grid)
 *   causal within each sequence, bottom-right aligned as fa_fwd_kv: query i of
 *          sequence b sees key j when j <= i + (Nk_b - Nq_b). A query that sees
 *          no key (Nk_b = 0, or causal with Nq_b > Nk_b) gets O = 0 and
 *          LSE = -inf
 *   num_splits, workspace   as fa_fwd_kv, with fa_fwd_varlen_workspace(total_q,
 *          H, d, num_splits) bytes
 *   q, k, v, o, workspace 16-byte aligned; lse, the offsets and order 4-byte
 *   aligned;
 *   other arguments, ownership, errors and rounding as fa_fwd_kv. B = 0,
 *   total_q = 0 or max_seqlen_q = 0 queue nothing and return FA_OK.
 */
size_t fa_fwd_varlen_workspace(int total_q, int H, int d, int num_splits);
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int* cu_seqlens_q, const int* cu_seqlens_k, const int* order,
                  int B, int H, int Hkv, int max_seqlen_q, int max_seqlen_k,
                  int total_q, int total_k, int d, float scale, int causal, int dtype,
                  int num_splits, float* workspace, void* stream);

/*
 * fa_varlen_order - longest-first order of a variable-length batch, for the
 * `order` argument of fa_fwd_varlen (the batch-order preprocessing of the FA4
 * walkthrough, variable-length section: the sequences are ranked by the
 * estimated time of their heaviest work tile, heaviest first, and the kernel
 * reads sequence order[v] where it would read sequence v).
 *
 *   cu_seqlens_q, cu_seqlens_k, B, max_seqlen_q, max_seqlen_k, total_q,
 *   total_k, num_splits   as for the fa_fwd_varlen call the order is for
 *   order  device pointer to B int32 (written): order[v] is the sequence that
 *          virtual sequence v runs
 *
 * The weight of sequence b is the number of 64-key blocks its heaviest query
 * tile streams: ceil(min(Nk_b, split_keys) / 64) when Nq_b > 0 (with the
 * bottom-right causal mask the last query row sees every key), 0 otherwise,
 * where split_keys is the key range of one split (all keys for one split).
 * Lengths are clamped exactly as fa_fwd_varlen clamps them. Sequences of
 * equal weight keep their input order, so the result is unique. One kernel,
 * O(B^2) comparisons; B at most 2^20. B = 0 queues nothing and returns FA_OK.
 * Pointers 4-byte aligned; order must not overlap the offsets.
 */
int fa_varlen_order(const int* cu_seqlens_q, const int* cu_seqlens_k, int B,
                    int max_seqlen_q, int max_seqlen_k, int total_q, int total_k,
                    int num_splits, int* order, void* stream);

/*
 * fa_bwd - attention backward for f16 or bf16 inputs (gradients of fa_fwd).
 *
 * Given the forward's inputs q, k, v, its outputs o and lse, and the gradient
 * dout = dL/dO, writes dq, dk, dv (each B*H*N*d elements of `dtype`):
 *
 *     P = exp(scale * Q K^T - LSE)  (rebuilt from the saved statistic,
 *                                    "FlashAttention · InkStack" 1.2.2)
 *     dV = P^T dO,   dP = dO V^T,   D = rowsum(dO * O),
 *     dS = P * (dP - D),   dQ = scale * dS K,   dK = scale * dS^T Q
 *                                   ("FlashAttention · InkStack" 1.2.1)
 *
 * with the same causal convention as fa_fwd. Products accumulate in fp32; P
 * and dS are rounded to `dtype` before the products that consume them; each
 * gradient is rounded to `dtype` once. Every output element is written by
 * exactly one thread (no atomics), so results are deterministic.
 *
 *   q, k, v, o, dout  device pointers, B*H*N*d elements of `dtype`, [B][H][N][d]
 *   lse               device pointer, B*H*N float32 (natural log), as fa_fwd wrote it
 *   dq, dk, dv        device pointers, B*H*N*d elements of `dtype` (written)
 *   workspace         device pointer to 2*B*H*N float32, scratch owned by the
 *                     caller; on return its first B*H*N values hold -D
 *   B, H, N, d, scale, causal, dtype, stream   as fa_fwd (FA_FP8_E4M3 returns
 *                     FA_ERR_UNSUPPORTED)
 *
 * Three kernels are queued on `stream`. Outputs and workspace must not
 * overlap each other or any input; all pointers 16-byte aligned.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const void* dout, const float* lse, void* dq, void* dk, void* dv,
           float* workspace, int B, int H, int N, int d, float scale,
           int causal, int dtype, void* stream);

/* Static description of a return code (never NULL). */
const char* fa_strerror(int code);

/* FA_VERSION of the built library. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
