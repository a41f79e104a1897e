// Attention forward pass for gfx950 (MI355X, CDNA4): C ABI and kernels.
//
// O = softmax(scale * Q K^T) V and LSE = m + ln(l), computed one query tile
// per workgroup with an online softmax, so the score and probability tiles
// live only in registers ("FlashAttention · InkStack" sections 1.1 and 2.1-2.3;
// MUSA guide "FlashAttention 优化", complete-algorithm section).
//
// Work decomposition (sequence parallelism, "FlashAttention · InkStack" 2.2):
// one workgroup per (batch, head, query tile); each wave owns 32 query rows
// outright (split-Q, section 2.3), so no cross-wave reduction; at d = 64
// without a mask a wave owns 64 rows as two 32-column query blocks, so that
// each K and V operand it reads from LDS feeds two matrix instructions. Each
// SIMD runs two waves: while one issues matrix instructions the other's
// softmax VALU work fills the gaps, the hardware counterpart of the pingpong
// schedule of the FA3 walkthrough ("FlashAttention 完全拆解（三）", pingpong
// section). Tiles of 128 rows (four waves, two workgroups per CU) serve the
// fp8, grouped-query and variable-length forms, causal d = 64 and short
// causal d = 128 problems; the plain forward otherwise takes tiles of 256
// rows (eight waves of 32 rows at d = 128, one workgroup per CU; four waves
// of 64 rows at d = 64), which halves the K/V copies per FLOP. Causal d = 64
// waves need under 144 registers, so a CU holds three of its workgroups.
//
// Keys and values stream through LDS in 64-key tiles, double buffered, copied
// global -> LDS directly (no register staging) one tile ahead of the compute.
// Both tiles keep their row-major [key][dim] layout with a 16-byte-chunk XOR
// swizzle; GEMM1 reads V with the transposing LDS read, so no transpose pass
// is needed (the in-kernel V transpose of the FA3 walkthrough, FP8 layout
// section, done by the LDS read itself on gfx950).
//
// Both products run on MFMA 32x32x16 (f16/bf16 in, fp32 accumulate):
//   GEMM0  S^T[key][query] = K[key][:] . Q[query][:]            (A = K from LDS, B = Q in VGPRs)
//   GEMM1  O^T[dim][query] += V^T[dim][key] . P^T[key][query]   (A = V from LDS, B = P in VGPRs)
// Computing the transposed products puts one query column in each lane, so a
// row reduction over keys is 16 in-lane values plus one swap with the lane 32
// away, and per-query factors are per-lane scalars. The fp32 score
// accumulator becomes GEMM1's B operand in place; the key order this implies
// is matched by the rows the V read selects, so the two permutations cancel
// (the register-permutation idea of the same FA3 walkthrough section).
//
// Softmax in base 2: p = exp2(s * scale * log2(e) - m) on v_exp_f32. The
// reference value m of a row is moved only when the row's probabilities in a
// tile would sum past 256 (so every p stays <= 256): then the tile's row max
// is taken, O~ and l are rescaled by exp2(m_old - m_new) and the tile is
// recomputed, decided once per wave. This is the rescale skip of the FA4
// walkthrough, section 3.1.4, driven by the row sums the kernel keeps anyway
// instead of a row max per tile. Any reference m gives the same O = O~ / l and
// LSE = m + log l, so the skip changes rounding only. 1/l and LSE are applied
// once, in the epilogue (deferred normalisation, "FlashAttention · InkStack"
// 2.1).

#include "fa_common.h"

#include <atomic>
#include <mutex>

namespace {

constexpr int kWaves = 4;              // wave64s per workgroup (fp8, grouped, variable-length)
constexpr int kThreads = 64 * kWaves;
constexpr int kBlocksPerCU = 8 / kWaves;  // two waves per SIMD
constexpr int kBr = 32 * kWaves;       // query rows per workgroup
// The plain f16/bf16 forward at d = 128 runs eight waves (256 query rows) per
// workgroup, one workgroup per CU: still two waves per SIMD, but each K/V
// tile copied into LDS serves twice the rows, so the copies per FLOP halve.
// Measured against four waves on one box: +3% at N = 8192 and +4% at
// N = 32768 non-causal, +3% causal at N >= 32768, +1.5% causal at 8192 and
// 15% slower causal at N = 2048 (the larger tile wastes more of the
// diagonal), so causal problems shorter than 8192 keep four waves. The
// plain d = 64 forward takes 256 rows without a mask (+2% at B=4 H=16
// N=2048, neutral at N=8192) and 128 with one (-6% at N=16384 with 256).
// Causal d = 128 takes the 256-row tiles from N = 8192 (with the early stop
// below: +1.9% at B=2 H=32 N=8192 against 128-row tiles, one box, three runs
// each; 128-row tiles stay shorter, where the larger tile wastes more of the
// diagonal: -2% at N=4096).
#ifndef FA_WIDE_CAUSAL_MIN_N
#define FA_WIDE_CAUSAL_MIN_N 8192
#endif
constexpr int kWidePlainMinCausalN = FA_WIDE_CAUSAL_MIN_N;
#ifndef FA_CAUSAL_EARLY_STOP
#define FA_CAUSAL_EARLY_STOP 1
#endif
// Grouped-query attention without a mask, in one key range, takes the same
// 256-row tiles from 1024 rows per K/V head (+3% at B=2 H=32 Hkv=8
// N=8192); causal grouped and variable-length problems keep 128-row tiles
// (variable-length causal measured 6% slower with 256).
constexpr int kWideKvMinRows = 1024;
constexpr int kWaveRows = 32;          // query rows per wave (one 32-column MFMA block)
constexpr int kBc = 64;                // keys per KV tile
constexpr float kSumLimit = 256.0f;    // per-lane tile row-sum that forces a rescale
constexpr float kMinit = -1.0e30f;     // finite "no key seen yet" reference value

// Optional software exponential (the FMA-pipe exp2 of the FA4 walkthrough,
// section 3.1.3), for a measurement variant of the library only: with
// FA_SWEXP2_EVERY = k > 0 the f16/bf16 kernels compute every k-th
// probability of a lane with exp2_fma below instead of v_exp_f32. The
// default build (k = 0) does not use it: on gfx950 the transcendental issues
// on the VALU like an FMA (about 1.6 FMA slots per v_exp_f32, measured), so
// nine VALU instructions per emulated element cost more than they free.
// The plain forward at d = 128 without a mask runs on the 16x16x32 matrix
// instruction (fa_fwd16_kernel below); FA_M16 = 0 builds the library with
// the 32x32x16 kernel there instead, for measurement.
#ifndef FA_M16
#define FA_M16 1
#endif
#ifndef FA_SWEXP2_EVERY
#define FA_SWEXP2_EVERY 0
#endif

// 2^x without the transcendental unit: x = n + f with n = round(x) (the
// 1.5 * 2^23 shift, exact for |x| < 2^22) and f = x - n in [-1/2, 1/2]
// exact; 2^f by the cubic minimax fit of csrc/fit_exp2.py (relative error
// 7.5e-5, below half an f16 ulp); 2^n applied by v_ldexp_f32, which
// underflows to 0, so masked scores (-inf, clamped to -1000) give exactly 0.
__device__ __forceinline__ float exp2_fma(float x) {
  const float xc = fmaxf(x, -1000.0f);
  const float y = xc + 12582912.0f;
  const float r = y - 12582912.0f;
  const float f = xc - r;
  float p = __builtin_fmaf(5.517166853e-02f, f, 2.426111251e-01f);
  p = __builtin_fmaf(p, f, 6.932609677e-01f);
  p = __builtin_fmaf(p, f, 9.999280572e-01f);
  return __builtin_ldexpf(p, (int)(__float_as_uint(y) - 0x4B400000u));
}

// Software pipeline. Keys are processed in 32-key units u (two per 64-key
// tile). In the region of unit u a wave issues, back to back,
//   GEMM0 of unit u+1 (scores S_{u+1}),  GEMM1 of unit u-1 (O~ += V P_{u-1}),
// and between those matrix instructions the VALU softmax of unit u (P_u from
// S_u). The three are independent, so one wave's instruction stream carries
// both matrix and vector work (the two-stage GEMM/softmax pipeline of
// "FlashAttention · InkStack" 3.2.2 and the FA3 walkthrough's Algorithm 2,
// at 32-key granularity). K and V tiles have separate double buffers: K_j is
// read in regions 2j-1 and 2j, V_j in regions 2j+1 and 2j+2, so after the
// barrier that ends region 2j the copies of K_{j+2} and V_{j+1} can start and
// have two regions to land.
//
// The general form (GEN) runs grouped-query attention over a key/value
// history, optionally split over key ranges. Query heads that share a K/V
// head are contiguous in memory, so their rows are taken as one "virtual
// head" of group*Nq rows over that K/V head (the packing of query heads per
// K/V head of the FA4 walkthrough, section 3.3): every K/V tile read serves
// all of them. Row r of a virtual head is query position r % Nq, which sees
// key j when j <= r % Nq + (Nk - Nq). With several splits, each workgroup
// covers one range of keys and writes its O (normalised by its own l) and
// LSE in fp32 for the merge kernel below (the split-KV decoding of the same
// walkthrough section).
//
// The variable-length form (VL, with GEN) packs B sequences of different
// lengths token-major: q and o are [total_q][H][d], k and v [total_k][Hkv][d],
// lse [total_q][H], and sequence b owns query tokens cu_q[b]..cu_q[b+1]-1 and
// key tokens cu_k[b]..cu_k[b+1]-1 (the "varlen" batching of the vLLM deep
// dive and the FA4 walkthrough's variable sequence lengths). A virtual head is
// then (sequence, K/V head); the grid covers the longest sequence and tiles
// past a shorter one return at once. Offsets are clamped to the totals and
// lengths to the stated maxima, so malformed offsets cannot address memory
// outside the tensors. A query that sees no key (an empty key sequence, or
// causal with more queries than keys) gets O = 0 and LSE = -inf.
struct KvArgs {
  int nk;          // keys per K/V head (VL: the longest key sequence)
  int nq;          // query positions per query head (VL: the longest query sequence)
  int coff;        // Nk - Nq (VL: per sequence)
  int splits;      // key ranges per (virtual head, query tile)
  int split_keys;  // keys per range, a multiple of the 64-key tile
  float* part;     // splits > 1: O [splits][rows_total][d] fp32, then LSE [splits][rows_total]
  size_t rows_total;   // output rows (B*H*Nq, VL: total_q*H); partials are indexed by output row
  const int* cu_q;     // VL: [B+1] query token offsets
  const int* cu_k;     // VL: [B+1] key token offsets
  int hkv;             // VL: K/V heads
  int group;           // VL: query heads per K/V head
  int total_q, total_k;
  int stream_kv;       // 1: every K/V byte is read by one workgroup only (one query
                       // tile per virtual head): copy with the non-temporal hint
  const int* order;    // VL: virtual -> actual sequence (heaviest first), or null
  int nb;              // VL: sequences in the batch
};

template <int DT, int D, bool CAUSAL, bool GEN = false, bool VL = false, int W = kWaves,
          int QB = 1>
__global__ __launch_bounds__(64 * W, 8 / W)
void fa_fwd_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
                   const uint16_t* __restrict__ Vg, uint16_t* __restrict__ Og,
                   float* __restrict__ LSEg, int N, int n_qtiles, int n_tiles,
                   float c_log2, KvArgs kva) {
  using E = Elt<DT>;
  constexpr int KCH = D / 8;                     // 16-byte chunks per row
  constexpr int KS = D / 16;                     // GEMM0 k-steps
  constexpr int DB = D / 32;                     // 32-row blocks of O^T
  constexpr int TILE = kBc * D;                  // elements of one K or V tile
  constexpr int ROWS_PER_LOAD = 64 / KCH;        // rows one wave-wide 1 KB copy covers
  constexpr int WR = kWaveRows * QB;             // query rows per wave
  constexpr int kBrW = WR * W;                   // query rows per workgroup
  constexpr int LPW = kBc / ROWS_PER_LOAD / W;   // 1 KB copies per wave, tile and tensor
  static_assert(LPW * W * ROWS_PER_LOAD == kBc, "tile must split over the waves");
  static_assert(QB == 1 || !GEN, "two query blocks per wave: plain forward only");

  __shared__ __attribute__((aligned(1024))) uint16_t k_lds[2][TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds[2][TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  int bh, qt, sp = 0;
  if constexpr (GEN) {
    int qs;
    // grouped causal prefill in one key range: the plain kernel's head bundles
    const int hb = (!CAUSAL || VL || kva.splits != 1 || kva.nk > (1 << 20) / D)
                       ? 1 : max(1, min((n_tiles / n_qtiles) >> 3, max(4, (1 << 20) / (kva.nk * D))));
    tile_of<CAUSAL, VL>(blockIdx.x, n_tiles, n_qtiles * kva.splits, bh, qs, hb);
    qt = qs / kva.splits;
    sp = qs - qt * kva.splits;
  } else {
    // causal: bundles of heads whose K and V (4 N D bytes each) fill at most
    // 4 MB, an XCD's L2 (+21% at B=4 H=16 N=2048 d=64, +2-4% at d=128 and
    // N <= 4096), and at least 4 heads while one head's K and V fit it:
    // B=2 H=32 N=8192 d=128 measured +1.6%, +2.0% and +2.0% on three boxes
    // against one head per bundle (bundles of 2: +1.6%, of 8: +-0; neutral
    // at N=4096 and 16384). The L2 hit rate falls with the bundles (87.5% ->
    // 77%, the misses served by the MALL), so the gain is not L2 reuse. One
    // head per bundle for longer heads.
    const int hb = (!CAUSAL || N > (1 << 20) / D)
                       ? 1 : max(1, min((n_tiles / n_qtiles) >> 3, max(4, (1 << 20) / (N * D))));
    tile_of<CAUSAL>(blockIdx.x, n_tiles, n_qtiles, bh, qt, hb);
  }
  // Nr rows per (virtual) head, nq query positions per query head, Nk keys
  // per K/V head; K/V rows krs elements apart
  int Nr = N, nq = GEN ? kva.nq : N, Nk = GEN ? kva.nk : N, coff = GEN ? kva.coff : 0;
  const uint16_t* K = Kg + (size_t)bh * (size_t)Nk * D;
  const uint16_t* V = Vg + (size_t)bh * (size_t)Nk * D;
  int krs = D;
  int vl_tok0 = 0, vl_h0 = 0;   // VL: first query token and first query head
  if constexpr (VL) {
    // virtual sequence bv runs sequence order[bv] when the caller passes the
    // longest-first order (a permutation, so every sequence still runs once)
    const int bv = bh / kva.hkv, hk = bh - bv * kva.hkv;
    const int b = kva.order ? min(max(kva.order[bv], 0), kva.nb - 1) : bv;
    const int q0 = min(max(kva.cu_q[b], 0), kva.total_q);
    const int q1 = min(max(kva.cu_q[b + 1], q0), kva.total_q);
    const int k0 = min(max(kva.cu_k[b], 0), kva.total_k);
    const int k1 = min(max(kva.cu_k[b + 1], k0), kva.total_k);
    nq = min(q1 - q0, kva.nq);
    Nk = min(k1 - k0, kva.nk);
    coff = Nk - nq;
    Nr = kva.group * nq;
    if (qt * kBrW >= Nr) return;   // past this sequence's rows
    K = Kg + ((size_t)k0 * kva.hkv + hk) * D;
    V = Vg + ((size_t)k0 * kva.hkv + hk) * D;
    krs = kva.hkv * D;
    vl_tok0 = q0;
    vl_h0 = hk * kva.group;
  }

  const int q_wave = qt * kBrW + wave * WR;
  const int q_lane = q_wave + l32;   // this lane's row in query block 0 (block qb: + 32 qb)
  // query position of this lane's row and the lowest one in the wave (the
  // causal diagonal), and the keys this workgroup covers: [kbeg, kend)
  const int q_pos = GEN ? q_lane % nq : q_lane;
  const int wave_pos = GEN ? ((q_wave / nq == min(q_wave + 31, Nr - 1) / nq) ? q_wave % nq : 0)
                           : q_wave;
  // output row of this lane's query (units of D): also its Q row and LSE index
  size_t orow = (size_t)bh * (size_t)Nr + q_lane;
  if constexpr (VL)
    orow = (size_t)(vl_tok0 + q_pos) * (size_t)(kva.hkv * kva.group) + vl_h0 + q_lane / nq;
  const int kbeg = GEN ? sp * kva.split_keys : 0;
  int kend = GEN ? min(Nk, kbeg + kva.split_keys) : Nk;
  if (CAUSAL) {
    const int first = qt * kBrW, last = min(Nr, qt * kBrW + kBrW) - 1;
    const int max_pos = GEN ? ((first / nq != last / nq) ? nq - 1 : last % nq) : last;
    kend = min(kend, max_pos + coff + 1);
  }
  // KV tiles the workgroup streams; every wave runs every unit (units past a
  // wave's causal diagonal are fully masked and contribute nothing)
  const int n_kv_real = kend > kbeg ? (kend - kbeg + kBc - 1) / kBc : 0;
  const int n_kv = n_kv_real + (n_kv_real & 1);
  const int n_units = 2 * n_kv;
  const int jbeg = kbeg / kBc;   // first key tile
  if constexpr (GEN) {
    if (n_kv_real == 0) {
      // no key to see (a key range wholly past the causal diagonal, or an
      // empty key sequence): O = 0 and LSE = -inf, which the merge ignores
      if (q_lane < Nr && hi == 0) {
        if (kva.splits > 1) {
          const size_t prow = (size_t)sp * kva.rows_total + orow;
          float* po = kva.part + prow * D;
          for (int c = 0; c < D; c += 4) *(float4*)(po + c) = float4{0.0f, 0.0f, 0.0f, 0.0f};
          kva.part[(size_t)kva.splits * kva.rows_total * D + prow] = -INFINITY;
        } else {
          uint16_t* po = Og + orow * D;
          for (int c = 0; c < D; c += 8) *(u32x4*)(po + c) = u32x4{0u, 0u, 0u, 0u};
          LSEg[orow] = -INFINITY;
        }
      }
      return;
    }
  }

  // ---- Q tile -> registers (GEMM0 B operand), loaded once
  u32x4 qreg[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const uint16_t* Q = Qg + (orow + 32 * qb) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 z = {0u, 0u, 0u, 0u};
      qreg[qb][ks] = q_lane + 32 * qb < Nr ? *(const u32x4*)(Q + ks * 16 + hi * 8) : z;
    }
  }

  // ---- global -> LDS copies: per-lane byte offsets within a tile
  int src_off[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int r = (wave * LPW + i) * ROWS_PER_LOAD + lane / KCH;
    // row r, chunk swizzled (the swizzle is an involution)
    src_off[i] = r * (krs * 2) + swz<KCH>(r, lane % KCH) * 16;
  }
  // copy of tile j (keys 64j..64j+63): a buffer load ranged over the tile's
  // rows inside the tensor, so rows past the end of the range (ragged or
  // padded tiles, tiles past the end) read as zero with no bounds branch
  auto copy_tile = [&](const uint16_t* src, uint16_t* dst, int j) {
    const int key0 = min((jbeg + j) * kBc, kend);
    const int rows = min(kend - key0, kBc);
    uint32_t bytes = (uint32_t)rows * (D * 2);
    if constexpr (VL) bytes = rows > 0 ? (uint32_t)((rows - 1) * krs + D) * 2 : 0u;
    const i32x4 rs = buffer_rsrc(src + (size_t)key0 * krs, bytes);
    const uint32_t dst0 = lds_addr(dst) + wave * LPW * 1024;
    if (GEN && kva.stream_kv) {
#pragma unroll
      for (int i = 0; i < LPW; ++i) copy16_buf_to_lds_nt(rs, src_off[i], dst0 + i * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < LPW; ++i) copy16_buf_to_lds(rs, src_off[i], dst0 + i * 1024);
    }
  };

  // ---- per-lane LDS read offsets (elements)
  // GEMM0 A operand: K row l32 (+32 for the second unit of a tile), chunk 2*ks + hi
  int k_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) k_off[ks] = l32 * D + swz<KCH>(l32, 2 * ks + hi) * 8;
  // GEMM1 A operand, transposing read: 16-lane group g covers 4 keys x 16 dims;
  // lane jj of the group points at key k0 + jj/4, dims d0 + 4*(jj%4) .. +3.
  int v_off[2][DB];
  {
    const int g = lane >> 4, jj = lane & 15;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int row = 8 * h2 + 4 * (g >> 1) + (jj >> 2);
        const int dim = db * 32 + 16 * (g & 1) + 4 * (jj & 3);
        v_off[h2][db] = row * D + swz<KCH>(row, dim >> 3) * 8 + (dim & 7);
      }
  }

  // Per query block qb of the wave (QB blocks of 32 rows; lane l32 holds row
  // q_lane + 32 qb of block qb): O^T accumulators, the double-buffered score
  // tiles and packed P, and the online-softmax state.
  f32x16 oacc[QB][DB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qb][db][r] = 0.0f;
  f32x16 sacc[2][QB];
  u32x4 pk[2][QB][2];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[b][qb][r] = 0.0f;
      pk[b][qb][0] = pk[b][qb][1] = u32x4{0u, 0u, 0u, 0u};
    }
  float m_run[QB];          // reference value of this lane's query row (log2 units)
  float l_run[QB];          // this lane's partial row sum
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = kMinit;
    l_run[qb] = 0.0f;
  }

  // GEMM0 of one unit: S^T (32 keys x 32 queries per block) = K_unit Q^T;
  // each K operand read serves every query block
  auto gemm0 = [&](auto kst, auto kkb, f32x16 (&acc)[QB]) {
    const uint16_t* base = &k_lds[decltype(kst)::value][decltype(kkb)::value * 32 * D];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[qb][r] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 a = *(const u32x4*)(base + k_off[ks]);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) acc[qb] = E::mma(a, qreg[qb][ks], acc[qb]);
    }
  };
  // GEMM1 of one unit: O^T += V_unit^T P^T, two 16-key steps; each V operand
  // read serves every query block
  auto gemm1 = [&](auto vst, auto vkb, const u32x4 (&p)[QB][2]) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const uint16_t* base =
          &v_lds[decltype(vst)::value][(decltype(vkb)::value * 32 + s2 * 16) * D];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x2 lo = E::read_tr(base + v_off[0][db]);
        const u32x2 hi2 = E::read_tr(base + v_off[1][db]);
        const u32x4 a = {lo[0], lo[1], hi2[0], hi2[1]};
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) oacc[qb][db] = E::mma(a, p[qb][s2], oacc[qb][db]);
      }
    }
  };
  // p = exp2(s*c - m) packed into GEMM1's B operand; returns this lane's row sum
  auto softmax = [&](const f32x16& sv, u32x4 (&p)[2], int qb) -> float {
    const float neg_m = -m_run[qb];
    float e[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float x = __builtin_fmaf(sv[r], c_log2, neg_m);
      if constexpr (FA_SWEXP2_EVERY > 0)
        e[r] = r % FA_SWEXP2_EVERY == FA_SWEXP2_EVERY - 1 ? exp2_fma(x) : __builtin_amdgcn_exp2f(x);
      else
        e[r] = __builtin_amdgcn_exp2f(x);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 w = {E::pack(e[8 * h + 0], e[8 * h + 1]), E::pack(e[8 * h + 2], e[8 * h + 3]),
                 E::pack(e[8 * h + 4], e[8 * h + 5]), E::pack(e[8 * h + 6], e[8 * h + 7])};
      p[h] = w;
    }
    // row sum as a tree (a short dependency chain)
    float t[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) t[r] = e[2 * r] + e[2 * r + 1];
    return ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
  };
  // mask keys past the covered range and, when causal, keys after the query
  auto mask = [&](f32x16& sv, int u, int qb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kbeg + 32 * u + 8 * (r >> 2) + 4 * hi + (r & 3);
      if (key >= kend || (CAUSAL && key > q_pos + 32 * qb + coff)) sv[r] = -INFINITY;
    }
  };

  // Rare path: a row's reference value must move (always after the first
  // unit). Take the unit's row max, rescale O~ and l, recompute P and its sum.
  auto rescale = [&](const f32x16& sv, u32x4 (&p)[2], float& tsum, int qb) {
    float mx = sv[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sv[r]);
    mx = fmaxf(mx, other_half(mx));
    const float m_new = fmaxf(m_run[qb], mx * c_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
    l_run[qb] *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qb][db][r] *= alpha;
    m_run[qb] = m_new;
    tsum = softmax(sv, p, qb);
  };
  // row-sum partials of the unit whose P awaits its check
  float tsum_prev[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) tsum_prev[qb] = 0.0f;
  // the check of a unit's P, per query block: rescale the block when any of its
  // rows' tile sums passed the limit, then add the sums into l
  auto check = [&](f32x16 (&sv)[QB], u32x4 (&p)[QB][2]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (__builtin_amdgcn_ballot_w64(!(tsum_prev[qb] <= kSumLimit)) != 0)
        rescale(sv[qb], p[qb], tsum_prev[qb], qb);
      l_run[qb] += tsum_prev[qb];
    }
  };

  // Region u. The check of P_{u-1} sits at the top, after the first LDS reads
  // of the region are in flight and before GEMM1 consumes P_{u-1} (and before
  // GEMM0 of unit u+1 overwrites S_{u-1}), so no region ends in a branch
  // that waits on its own VALU work.
  // A wave whose 32 rows all lie past the (virtual) head's rows has no work
  // (a decode step fills only the first rows of the tile): it still issues its
  // share of the copies and meets every barrier, but skips the products and
  // the softmax.
  const bool active = !GEN || q_wave < Nr;
  auto region = [&](auto kst, auto kkb, auto vst, auto vkb, auto sb, int u) {
    constexpr int SB = decltype(sb)::value;
    if (GEN && !active) return;
    const uint16_t* kbase = &k_lds[decltype(kst)::value][decltype(kkb)::value * 32 * D];
    const u32x4 a0 = *(const u32x4*)(kbase + k_off[0]);
    const u32x4 a1 = *(const u32x4*)(kbase + k_off[1]);
    check(sacc[SB ^ 1], pk[SB ^ 1]);
    if ((kbeg + 32 * u + 32 > kend) || (CAUSAL && kbeg + 32 * u + 31 > wave_pos + coff)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) mask(sacc[SB][qb], u, qb);
    }

    f32x16 (&acc)[QB] = sacc[SB ^ 1];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[qb][r] = 0.0f;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) acc[qb] = E::mma(a0, qreg[qb][0], acc[qb]);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) acc[qb] = E::mma(a1, qreg[qb][1], acc[qb]);
#pragma unroll
    for (int ks = 2; ks < KS; ++ks) {
      const u32x4 a = *(const u32x4*)(kbase + k_off[ks]);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) acc[qb] = E::mma(a, qreg[qb][ks], acc[qb]);
    }
    gemm1(vst, vkb, pk[SB ^ 1]);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      tsum_prev[qb] = softmax(sacc[SB][qb], pk[SB][qb], qb);
      // P is needed only where the next region does not rescale; without this
      // use the compiler would move its packing past that branch, out of reach
      // of this region's matrix instructions
      asm volatile("" ::"v"(pk[SB][qb][0]), "v"(pk[SB][qb][1]), "v"(tsum_prev[qb]));
    }
    // interleave: per matrix instruction 2 LDS reads and 3 VALU (measured
    // against 1, 2 reads and 2, 4, 5 VALU, and 2 matrix instructions per
    // group: 1-2% ahead of the next best). With two query blocks the matrix
    // instructions keep their order and the compiler places the rest: fixed
    // groups of 1 read with 5, 7 or 9 VALU, or 2 with 7, measured 0-4% slower.
    constexpr int NM = QB * (KS + 2 * DB);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (QB == 1) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
      }
    }
  };
  // after region 2j: every wave is done with K_j and V_{j-1}; start K_{j+2}, V_{j+1}
  auto sync = [&]() {
    wait_copies();
    __syncthreads();
  };
  auto copy_k = [&](auto kst, int j) { copy_tile(K, k_lds[decltype(kst)::value], j + 2); };
  auto copy_v = [&](auto kst, int j) { copy_tile(V, v_lds[decltype(kst)::value ^ 1], j + 1); };
  auto sync_and_copy = [&](auto kst, int j) {
    sync();
    copy_k(kst, j);
    copy_v(kst, j);
  };

  // ---- prologue: zero both V stages (region 0's GEMM1 adds P = 0 times the
  // second; rows a copy leaves alone must be finite), then K_0, V_0, K_1; S_0
#pragma unroll
  for (int i = 0; i < 2 * TILE; i += 64 * W * 8)
    *(u32x4*)(&v_lds[0][0] + i + tid * 8) = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
  copy_tile(K, k_lds[0], 0);
  copy_tile(V, v_lds[0], 0);
  copy_tile(K, k_lds[1], 1);
  wait_copies();
  __syncthreads();
  gemm0(IC<0>(), IC<0>(), sacc[0]);

  // A causal wave whose rows end before the workgroup's last keys stops
  // computing after the trip that holds the region doing GEMM1 of its last
  // unit with a visible key; it still issues its share of the copies and
  // meets every barrier. The units it skips are fully masked for all its rows
  // (P = 0), and so is the unit the final check and GEMM1 below then take.
  int u_stop = n_units;
  if constexpr (CAUSAL && !GEN && FA_CAUSAL_EARLY_STOP) {
    const int need = (min(kend, wave_pos + coff + WR) - kbeg + 31) / 32;
    u_stop = __builtin_amdgcn_readfirstlane(min(n_units, (need / 4 + 1) * 4));
  }
  // ---- steady state, four units (two tiles) per trip so that every buffer
  // index is a constant; the tile count is padded to even (a padded tile is
  // all keys >= N, fully masked). The K copies start right after each barrier
  // and the V copies one region later: both land before the wait ahead of the
  // next barrier, and no region reads the stages they fill (K_{j+2} replaces
  // K_j, last read in region 2j; V_{j+1} replaces V_{j-1}, last read in region
  // 2j). Spreading the copies over two regions instead of issuing all of a
  // wave's copies after the barrier (all eight waves at once) measured +2.2 to
  // +2.6% non-causal and +2.0 to +2.5% causal at B=2 H=32 N=8192 d=128 (two
  // boxes, three runs each; V first and K one region later: +2.4%; half of each
  // at both points: +1.9%; all of them one region later: +1.6%), +-0 at d=64.
  for (int u = 0; u < n_units; u += 4) {
    if (!(CAUSAL && !GEN && FA_CAUSAL_EARLY_STOP) || u < u_stop) {
      region(IC<0>(), IC<1>(), IC<1>(), IC<1>(), IC<0>(), u);
      sync();
      copy_k(IC<0>(), u >> 1);
      region(IC<1>(), IC<0>(), IC<0>(), IC<0>(), IC<1>(), u + 1);
      copy_v(IC<0>(), u >> 1);
      region(IC<1>(), IC<1>(), IC<0>(), IC<1>(), IC<0>(), u + 2);
      sync();
      copy_k(IC<1>(), (u >> 1) + 1);
      region(IC<0>(), IC<0>(), IC<1>(), IC<0>(), IC<1>(), u + 3);
      copy_v(IC<1>(), (u >> 1) + 1);
    } else {
      sync_and_copy(IC<0>(), u >> 1);
      sync_and_copy(IC<1>(), (u >> 1) + 1);
    }
  }
  // copies of tiles past the end are still in flight; the LDS must not be
  // released under them
  wait_copies();
  // ---- check and GEMM1 of the last unit (second half of the last tile, odd index)
  check(sacc[1], pk[1]);
  gemm1(IC<1>(), IC<1>(), pk[1]);
  // Matrix instructions need every lane enabled (each lane supplies an operand
  // slice). These accumulators are used only inside the lane-divergent
  // epilogue, and the compiler would otherwise sink the last GEMM1 into it,
  // where idle lanes drop their slices; an empty volatile use keeps it here.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) asm volatile("" ::"v"(oacc[qb][db][r]));

  // ---- epilogue: O = O~ / l, LSE = ln2 * (m + log2 l)
  if (q_wave < Nr) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float l_tot = l_run[qb] + other_half(l_run[qb]);
      float inv = __builtin_amdgcn_rcpf(l_tot);
      float lse_v = (m_run[qb] + __builtin_amdgcn_logf(l_tot)) * kLn2;
      if constexpr (VL) {
        // a causal row of a sequence with fewer keys than queries may see none
        inv = l_tot > 0.0f ? inv : 0.0f;
        lse_v = l_tot > 0.0f ? lse_v : -INFINITY;
      }
      const f32x16 (&oa)[DB] = oacc[qb];
      if (GEN && kva.splits > 1) {
        // partial of key range sp, fp32, for the merge
        if (q_lane < Nr) {
          const size_t prow = (size_t)sp * kva.rows_total + orow;
          float* po = kva.part + prow * D;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4)
              *(float4*)(po + db * 32 + 8 * g4 + 4 * hi) =
                  float4{oa[db][4 * g4 + 0] * inv, oa[db][4 * g4 + 1] * inv,
                         oa[db][4 * g4 + 2] * inv, oa[db][4 * g4 + 3] * inv};
          if (hi == 0) kva.part[(size_t)kva.splits * kva.rows_total * D + prow] = lse_v;
        }
      } else if (q_lane + 32 * qb < Nr) {
        uint16_t* op = Og + (orow + 32 * qb) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            u32x2 w = {E::pack(oa[db][4 * g4 + 0] * inv, oa[db][4 * g4 + 1] * inv),
                       E::pack(oa[db][4 * g4 + 2] * inv, oa[db][4 * g4 + 3] * inv)};
            *(u32x2*)(op + db * 32 + 8 * g4 + 4 * hi) = w;
          }
        if (hi == 0) LSEg[orow + 32 * qb] = lse_v;
      }
    }
  }
}

// -------------------------------------------------------------- fp8 kernel --
//
// OCP e4m3 inputs with per-tensor descales (per-tensor scaling,
// "FlashAttention · InkStack" section 3.3.3). Both products run on the
// 32x32x64 fp8 matrix instruction with unit block scales and fp32
// accumulation; the logit multiplier carries scale * s_q * s_k * log2(e) and
// the epilogue multiplies by s_v. P is quantised to e4m3 (round to nearest
// even) before GEMM1; l sums the unquantised fp32 P. Because one GEMM1
// instruction consumes 64 keys, the pipeline unit here is a whole 64-key
// tile: region j issues GEMM0 of tile j+1 and GEMM1 of tile j-1 around the
// softmax of tile j. K and V tiles sit in four-stage rings, so a copy has
// three regions to land.
//
// V is read with the 8-bit transposing LDS read, which hands each lane 8
// consecutive LDS rows of one dimension. The score accumulator gives lane
// half h the keys whose bit 2 equals h, so V rows are written to LDS with
// key bits 2 and 3 swapped: 8 consecutive LDS rows then hold exactly the
// keys one lane half owns, in accumulator order (the V-side permutation that
// cancels the P-side one, FA3 walkthrough, FP8 layout section).

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ u32x2 read_tr8(const uint8_t* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2*)p));
}

// LDS swizzles for fp8 tiles (rows of RB bytes, 16-byte chunks, 64 banks).
// K: the GEMM0 read has 16 lanes per cycle on 16 consecutive rows at one
// chunk. V: the 8-bit transposing read has 32 lanes per cycle on 8
// consecutive rows x 2 adjacent chunks (an aligned chunk pair).
template <int RB>
__device__ __forceinline__ int swz_k8(int r, int c) {
  if (RB == 128) return c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  return c ^ ((r >> 2) & 3);
}
template <int RB>
__device__ __forceinline__ int swz_v8(int r, int c) {
  if (RB == 128) return c ^ (((r >> 1) & 3) << 1);
  return c ^ (((r >> 2) & 1) << 1);
}

// key bits 2 and 3 swapped (an involution)
__device__ __forceinline__ int swap23(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// Block scales (BS): one scale per 128-row query tile, per 64-key K tile and
// per 64-key V tile (block quantisation, InkStack 3.3.1 and the FA3
// walkthrough's FP8 section). The product of the Q and K scales enters the
// logit multiplier of each tile, so m and l stay in units of the true
// scores. A V tile's scale s_j is folded into P: with s* the head's largest V
// scale, the tile's P is formed as exp2(t - m + log2(s_j / s*)) (at most the
// unscaled P, so no e4m3 overflow), l adds the unscaled sum (the tile sum
// times s* / s_j), and the epilogue multiplies by s*. The per-tile factors are
// staged in LDS once per workgroup.
constexpr int kMaxScaleTiles = 2048;   // keys <= 131072 per head with block scales

// The non-causal per-tensor fp8 kernel at d = 128 runs 8 waves (256 query
// rows) per workgroup, as the f16/bf16 forward does: the K/V copies per FLOP
// halve and the engine clock rises 8%, but the per-tile barriers over 8
// waves take most of it back: +1.0% at B=4 H=16 N=8192 (1919 -> 1938
// TFLOP/s, one box, four runs each). Block scales keep 128-row tiles (one Q
// scale per tile), and so does causal.
#ifndef FA_FP8_WIDE
#define FA_FP8_WIDE 1
#endif
#ifndef FA_FP8_INTERLEAVE
#define FA_FP8_INTERLEAVE 1
#endif
#ifndef FA_FP8_LDS
#define FA_FP8_LDS 3
#endif
#ifndef FA_FP8_VALU
#define FA_FP8_VALU 14
#endif

template <int D, bool CAUSAL, bool BS = false, int W = kWaves>
__global__ __launch_bounds__(64 * W, 8 / W)
void fa_fwd_fp8_kernel(const uint8_t* __restrict__ Qg, const uint8_t* __restrict__ Kg,
                       const uint8_t* __restrict__ Vg, uint16_t* __restrict__ Og,
                       float* __restrict__ LSEg, int N, int n_qtiles, int n_tiles,
                       float c_log2, float v_descale, const float* __restrict__ qsc,
                       const float* __restrict__ ksc, const float* __restrict__ vsc) {
  using Out = Elt<FA_BF16>;
  constexpr int CH = D / 16;                     // 16-byte chunks per row
  constexpr int KS = D / 64;                     // GEMM0 k-steps
  constexpr int DB = D / 32;                     // 32-row blocks of O^T
  constexpr int TILE = kBc * D;                  // bytes of one K or V tile
  constexpr int ROWS_PER_LOAD = 64 / CH;         // rows one wave-wide 1 KB copy covers
  constexpr int LPW = kBc / ROWS_PER_LOAD / W;
  constexpr int kBrW = 32 * W;                   // query rows per workgroup
  constexpr int kThreadsW = 64 * W;
  static_assert(!BS || W == kWaves, "block scales are per 128-row query tile");
  constexpr int NST = 4;                         // ring stages
  static_assert(LPW * W * ROWS_PER_LOAD == kBc, "tile must split over the waves");

  __shared__ __attribute__((aligned(1024))) uint8_t k_lds[NST][TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds[NST][TILE];
  // BS: per key tile {logit multiplier, log2(s_j / s*)}
  __shared__ float2 sc_lds[BS ? kMaxScaleTiles : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  int bh, qt;
  // causal: the f16/bf16 kernel's head bundles, sized to the XCD's L2 for
  // one-byte K and V (2 N D bytes per head)
  const int hb = (!CAUSAL || N > (1 << 21) / D)
                     ? 1 : max(1, min((n_tiles / n_qtiles) >> 3, max(4, (1 << 21) / (N * D))));
  tile_of<CAUSAL>(blockIdx.x, n_tiles, n_qtiles, bh, qt, hb);

  const size_t head = (size_t)bh * (size_t)N * D;
  const uint8_t* K = Kg + head;
  const uint8_t* V = Vg + head;

  const int q_wave = qt * kBrW + wave * kWaveRows;
  const int q_lane = q_wave + l32;
  const int kv_len = CAUSAL ? min(N, qt * kBrW + kBrW) : N;
  const int n_kv_real = (kv_len + kBc - 1) / kBc;
  const int n_kv = (n_kv_real + 3) & ~3;         // whole trips of the 4-tile loop

  if constexpr (BS) {
    // s* = the head's largest V scale, then the per-tile factors
    const int nkb = (N + kBc - 1) / kBc;
    const float* vs = vsc + (size_t)bh * nkb;
    const float* ks = ksc + (size_t)bh * nkb;
    float mx = 0.0f;
    for (int t = tid; t < nkb; t += kThreadsW) mx = fmaxf(mx, vs[t]);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
    if (lane == 0) sc_lds[wave].x = mx;      // the table's first entries as scratch
    __syncthreads();
    mx = fmaxf(fmaxf(sc_lds[0].x, sc_lds[1].x), fmaxf(sc_lds[2].x, sc_lds[3].x));
    mx = mx > 0.0f ? mx : 1.0f;
    __syncthreads();
    v_descale = mx;
    const float c_q = c_log2 * qsc[(size_t)bh * n_qtiles + qt];
    for (int t = tid; t < n_kv_real; t += kThreadsW)
      sc_lds[t] = float2{c_q * ks[t], fmaxf(__builtin_amdgcn_logf(vs[t] / mx), -100.0f)};
    __syncthreads();
  }

  // ---- Q -> registers: lane half h holds dims 64*ks + 32*h .. +31
  i32x8 qreg[KS];
  {
    const uint8_t* Q = Qg + head;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 lo = {0u, 0u, 0u, 0u}, hi4 = {0u, 0u, 0u, 0u};
      if (q_lane < N) {
        const uint8_t* src = Q + (size_t)q_lane * D + ks * 64 + hi * 32;
        lo = *(const u32x4*)src;
        hi4 = *(const u32x4*)(src + 16);
      }
      qreg[ks] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                       (int)hi4[0], (int)hi4[1], (int)hi4[2], (int)hi4[3]};
    }
  }

  // ---- copies: per-lane (row, column) of the slot each lane fills
  int k_row[LPW], k_colb[LPW], v_row[LPW], v_colb[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int slot = (wave * LPW + i) * 64 + lane;
    const int r = slot / CH, p = slot % CH;
    k_row[i] = r;
    k_colb[i] = swz_k8<D>(r, p) * 16;
    v_row[i] = swap23(r);
    v_colb[i] = swz_v8<D>(r, p) * 16;
  }
  auto copy_tile = [&](const uint8_t* src, uint8_t* dst, int key0, const int (&row)[LPW],
                       const int (&colb)[LPW]) {
    const uint32_t dst0 = lds_addr(dst) + wave * LPW * 1024;
    if (key0 + kBc <= N) {
      const uint8_t* g = src + (size_t)key0 * D;
#pragma unroll
      for (int i = 0; i < LPW; ++i) copy16_to_lds(g, row[i] * D + colb[i], dst0 + i * 1024);
    } else {
      // rows past N repeat row N-1; offsets are taken from the tile's first
      // row so that the 32-bit offset stays below 64 rows at any N
      const int r0 = min(key0, N - 1);
      const uint8_t* g = src + (size_t)r0 * D;
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int r = min(key0 + row[i], N - 1) - r0;
        copy16_to_lds(g, r * D + colb[i], dst0 + i * 1024);
      }
    }
  };
  auto copy_k = [&](int j, int st) { copy_tile(K, k_lds[st], j * kBc, k_row, k_colb); };
  auto copy_v = [&](int j, int st) { copy_tile(V, v_lds[st], j * kBc, v_row, v_colb); };

  // ---- LDS read offsets (bytes)
  int k_off[KS][2];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
      k_off[ks][h2] = l32 * D + swz_k8<D>(l32, 4 * ks + 2 * hi + h2) * 16;
  int v_off[DB];
  {
    const int g = lane >> 4, jj = lane & 15;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int row = 8 * (g >> 1) + (jj >> 1);
      v_off[db] = row * D + swz_v8<D>(row, 2 * db + (g & 1)) * 16 + 8 * (jj & 1);
    }
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
  f32x16 sacc[2][2];      // [tile parity][32-key half]
  i32x8 pk[2];            // P of a tile, e4m3, GEMM1 B operand
#pragma unroll
  for (int b = 0; b < 2; ++b) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[b][kb][r] = 0.0f;
#pragma unroll
    for (int w = 0; w < 8; ++w) pk[b][w] = 0;
  }
  float m_run = kMinit;
  float l_run = 0.0f;
  float tsum_prev = 0.0f;

  // GEMM0 of one tile; the operand of its first instruction (key half 0,
  // k-step 0) may be read ahead by the caller
  auto gemm0 = [&](auto kst, f32x16 (&acc)[2], const u32x4* first = nullptr) {
    const uint8_t* base = k_lds[decltype(kst)::value];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[kb][r] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bool ahead = first && kb == 0 && ks == 0;
        const u32x4 a0 = ahead ? first[0] : *(const u32x4*)(base + kb * 32 * D + k_off[ks][0]);
        const u32x4 a1 = ahead ? first[1] : *(const u32x4*)(base + kb * 32 * D + k_off[ks][1]);
        const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                         (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
        acc[kb] = mma_fp8(a, qreg[ks], acc[kb]);
      }
    }
  };
  auto gemm1 = [&](auto vst, const i32x8& p) {
    const uint8_t* base = v_lds[decltype(vst)::value];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      u32x2 r[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) r[q] = read_tr8(base + q * 16 * D + v_off[db]);
      const i32x8 a = {(int)r[0][0], (int)r[0][1], (int)r[1][0], (int)r[1][1],
                       (int)r[2][0], (int)r[2][1], (int)r[3][0], (int)r[3][1]};
      oacc[db] = mma_fp8(a, p, oacc[db]);
    }
  };
  // tile parameters (BS): logit multiplier and log2 of the V-scale ratio of the
  // tile in softmax (cur) and of the tile before it (prev)
  float2 sc_cur = float2{c_log2, 0.0f}, sc_prev = sc_cur;
  auto softmax = [&](const f32x16 (&sv)[2], i32x8& p, const float2& sc) -> float {
    const float neg_m = BS ? sc.y - m_run : -m_run;
    const float c = BS ? sc.x : c_log2;
    float half[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float e[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) e[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[kb][r], c, neg_m));
#pragma unroll
      for (int w = 0; w < 4; ++w)
        p[4 * kb + w] = (int)pack_e4m3x4(e[4 * w], e[4 * w + 1], e[4 * w + 2], e[4 * w + 3]);
      // row sum as a tree (a short dependency chain)
      float t[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) t[r] = e[2 * r] + e[2 * r + 1];
      half[kb] = ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
    }
    const float sum = half[0] + half[1];
    // the unscaled row sum (P before the V-scale factor)
    return BS ? sum * __builtin_amdgcn_exp2f(-sc.y) : sum;
  };
  auto mask = [&](f32x16 (&sv)[2], int j) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j * kBc + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (key >= N || (CAUSAL && key > q_lane)) sv[kb][r] = -INFINITY;
      }
  };
  auto rescale = [&](const f32x16 (&sv)[2], i32x8& p, float& tsum, const float2& sc) {
    float mx = sv[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sv[kb][r]);
    mx = fmaxf(mx, other_half(mx));
    const float m_new = fmaxf(m_run, mx * (BS ? sc.x : c_log2));
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    m_run = m_new;
    tsum = softmax(sv, p, sc);
  };

  // region j: check P_{j-1}, mask S_j; GEMM0 of tile j+1, GEMM1 of tile j-1,
  // softmax of tile j. The operand of the first matrix instruction is read
  // before the check, and the region's LDS reads, matrix instructions and
  // softmax are interleaved (below); left to itself the compiler issued all
  // 24 reads at the end of the region and their matrix instructions after
  // the barrier, so every wave waited out the reads' latency at the barrier.
  auto region = [&](auto kst, auto vst, auto sb, int j) {
    constexpr int SB = decltype(sb)::value;
    if constexpr (BS) {
      // padded tiles past n_kv_real are all masked; the values are uniform (SGPRs)
      const float2 t = sc_lds[min(j, n_kv_real - 1)];
      sc_cur = float2{__int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(t.x))),
                      __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(t.y)))};
    }
    const uint8_t* kbase = k_lds[decltype(kst)::value];
    const u32x4 first[2] = {*(const u32x4*)(kbase + k_off[0][0]), *(const u32x4*)(kbase + k_off[0][1])};
    if (__builtin_amdgcn_ballot_w64(!(tsum_prev <= kSumLimit)) != 0)
      rescale(sacc[SB ^ 1], pk[SB ^ 1], tsum_prev, sc_prev);
    l_run += tsum_prev;
    if ((j * kBc + kBc > N) || (CAUSAL && j * kBc + kBc - 1 > q_wave)) mask(sacc[SB], j);
    gemm0(kst, sacc[SB ^ 1], first);
    gemm1(vst, pk[SB ^ 1]);
    tsum_prev = softmax(sacc[SB], pk[SB], sc_cur);
    if constexpr (BS) sc_prev = sc_cur;
#if FA_FP8_INTERLEAVE
    // keep P's packing and both products in this region: their results are
    // first used in the next region, behind its check, and the compiler
    // would otherwise sink them there, away from this region's LDS reads
    // (element by element: the host pass rejects wide vector operands)
    asm volatile("" ::"v"(tsum_prev));
#pragma unroll
    for (int w = 0; w < 8; ++w) asm volatile("" ::"v"(pk[SB][w]));
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      asm volatile("" ::"v"(sacc[SB ^ 1][0][r]), "v"(sacc[SB ^ 1][1][r]));
#pragma unroll
      for (int db = 0; db < DB; ++db) asm volatile("" ::"v"(oacc[db][r]));
    }
    // per matrix instruction: FA_FP8_LDS LDS reads and FA_FP8_VALU VALU
    // instructions (8 matrix instructions, 22 reads, ~115 VALU per region)
#pragma unroll
    for (int i = 0; i < 2 * KS + DB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, FA_FP8_LDS, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, FA_FP8_VALU, 0);
    }
#endif
  };
  // after region j: K_{j+1} and V_{j-1} are done; the copies issued after
  // region j-3 (K_{j+2}, V_j) must have landed. Start K_{j+5} and V_{j+3}.
  auto sync_and_copy = [&](auto kst_free, auto vst_free, int j) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * LPW) : "memory");
    __syncthreads();
    copy_k(j + 5, decltype(kst_free)::value);
    copy_v(j + 3, decltype(vst_free)::value);
  };

  // ---- prologue
  copy_k(0, 0);
  copy_k(1, 1);
  copy_k(2, 2);
  copy_k(3, 3);
  copy_v(0, 0);
  copy_v(1, 1);
#pragma unroll
  for (int i = tid * 16; i < TILE; i += kThreadsW * 16) *(u32x4*)(&v_lds[3][i]) = u32x4{0u, 0u, 0u, 0u};
  wait_copies();
  __syncthreads();
  gemm0(IC<0>(), sacc[0]);
  __syncthreads();                       // every wave is done with K_0
  copy_k(4, 0);
  copy_v(2, 2);

  for (int j = 0; j < n_kv; j += 4) {
    region(IC<1>(), IC<3>(), IC<0>(), j);
    sync_and_copy(IC<1>(), IC<3>(), j);
    region(IC<2>(), IC<0>(), IC<1>(), j + 1);
    sync_and_copy(IC<2>(), IC<0>(), j + 1);
    region(IC<3>(), IC<1>(), IC<0>(), j + 2);
    sync_and_copy(IC<3>(), IC<1>(), j + 2);
    region(IC<0>(), IC<2>(), IC<1>(), j + 3);
    sync_and_copy(IC<0>(), IC<2>(), j + 3);
  }
  // ---- last tile (n_kv - 1, odd parity, V stage 3)
  if (__builtin_amdgcn_ballot_w64(!(tsum_prev <= kSumLimit)) != 0)
    rescale(sacc[1], pk[1], tsum_prev, sc_prev);
  l_run += tsum_prev;
  wait_copies();                          // no copy may land after the workgroup ends
  gemm1(IC<3>(), pk[1]);
  // Matrix instructions need every lane enabled (each lane supplies an operand
  // slice). These accumulators are used only inside the lane-divergent
  // epilogue, and the compiler would otherwise sink the last GEMM1 into it,
  // where idle lanes drop their slices; an empty volatile use keeps it here.
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) asm volatile("" ::"v"(oacc[db][r]));

  if (q_wave < N) {
    const float l_tot = l_run + other_half(l_run);
    const float inv = v_descale * __builtin_amdgcn_rcpf(l_tot);
    if (q_lane < N) {
      uint16_t* orow = Og + head + (size_t)q_lane * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          u32x2 w = {Out::pack(oacc[db][4 * g4 + 0] * inv, oacc[db][4 * g4 + 1] * inv),
                     Out::pack(oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv)};
          *(u32x2*)(orow + db * 32 + 8 * g4 + 4 * hi) = w;
        }
      if (hi == 0) LSEg[(size_t)bh * N + q_lane] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
  }
}

// ------------------------------------------------------ variable-length order --
//
// Longest-first order of a variable-length batch (the FA4 walkthrough's
// variable-length preprocessing): every sequence's heaviest work tile is
// weighted by the 64-key K/V blocks it streams, ceil(min(Nk_b, split_keys) /
// 64) when the sequence has queries and 0 otherwise (with the bottom-right
// causal mask the last query row sees every key); the sequences are ranked
// heaviest first, equal weights in input order, and order[rank] = b gives the
// permutation virtual -> actual. Lengths are taken as the attention kernel
// takes them (offsets clamped to the totals, lengths to the maxima). One
// thread per sequence counts the sequences ranked before it, reading the
// weights a workgroup-wide chunk at a time from LDS: O(B^2) comparisons, small
// next to the attention call for the batch sizes a serving step holds.
constexpr int kOrderThreads = 256;
constexpr int kMaxOrderSeqs = 1 << 20;

__global__ __launch_bounds__(kOrderThreads)
void fa_varlen_order_kernel(const int* __restrict__ cu_q, const int* __restrict__ cu_k, int B,
                            int max_q, int max_k, int total_q, int total_k, int split_keys,
                            int* __restrict__ order) {
  __shared__ int wl[kOrderThreads];
  auto weight = [&](int s) -> int {
    const int q0 = min(max(cu_q[s], 0), total_q), q1 = min(max(cu_q[s + 1], q0), total_q);
    const int k0 = min(max(cu_k[s], 0), total_k), k1 = min(max(cu_k[s + 1], k0), total_k);
    const int nq = min(q1 - q0, max_q), nk = min(k1 - k0, max_k);
    return nq <= 0 ? 0 : (min(nk, split_keys) + kBc - 1) / kBc;
  };
  const int b = blockIdx.x * kOrderThreads + threadIdx.x;
  const int wb = b < B ? weight(b) : -1;
  int rank = 0;
  for (int c0 = 0; c0 < B; c0 += kOrderThreads) {
    const int s = c0 + threadIdx.x;
    wl[threadIdx.x] = s < B ? weight(s) : -1;
    __syncthreads();
    const int n = min(kOrderThreads, B - c0);
    for (int i = 0; i < n; ++i) {
      const int w2 = wl[i];
      rank += (w2 > wb) || (w2 == wb && c0 + i < b);
    }
    __syncthreads();
  }
  if (b < B) order[rank] = b;
}

// ------------------------------------------------ 16x16x32 forward kernel --
//
// The plain forward on the 16x16x32 matrix instruction. On random bf16
// operands a loop of 16x16x32 instructions sustains about 14% more TFLOP/s
// than one of 32x32x16 instructions on this part: the chip runs power-limited,
// and the smaller instruction moves fewer accumulator bytes per FLOP. The
// structure is the kernel above (32-key units, 64-key double-buffered K/V
// tiles, one barrier per tile, the same regions); the fragments differ:
//   GEMM0: S^T (16 keys x 16 queries per instruction, 32 dims per step) =
//     K Q^T; lane l holds, for query l%16 of each 16-query block, keys
//     16 kb + 4 (l/16) + r of the unit (kb = 0, 1; r = 0..3).
//   GEMM1: O^T (16 dims x 16 queries) += V^T P^T over the unit's 32 keys in
//     one step, its k index taken in the order k = 8 (l/16) + j <-> key
//     16 (j/4) + 4 (l/16) + j%4, so that a lane's own eight P values are its
//     B operand and the two transposing V reads (4 keys each) its A operand.
// A query's row sum and maximum are spread over the four lanes l%16 + 16 i.
// The K and V tiles use their own swizzle (swz16) for these read patterns.

// Physical 16-byte chunk of logical chunk c in row r (256-byte rows, d = 128)
// of this kernel's K and V tiles: c ^ f(r) with f linear over the bits of
// r % 16, f = 2 r0 ^ 4 r1 ^ 8 r2 ^ 9 r3 (r_i bit i of r). Its two read
// patterns: the K read gives lane l row l%16 of a 16-key block at chunk
// 4 ks + l/16; the transposing V read serves the 32 lanes of each wave half
// on 8 consecutive rows x 2 adjacent chunks (c, c^1), conflict-free when f/2
// is distinct over each aligned 8 rows (it is: 0..7 on rows 0-7 and 4..7,
// 0..3 on rows 8-15). For the K read, 64 candidate f with that property were
// measured with the LDS bank-conflict counter on gfx950: only this one is
// conflict-free (the others, among them 2 (r%8) + (r/8)%2, take 4 extra
// cycles per read).
__device__ __forceinline__ int swz16(int r, int c) {
  return c ^ ((r & 7) << 1) ^ ((r & 8) ? 9 : 0);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int DT>
__device__ __forceinline__ f32x4 mma16(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (DT == FA_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// value of lane l ^ 16 (within each 32-lane half)
__device__ __forceinline__ float xor16(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401f));
}

template <int DT, int D, bool CAUSAL, int W, int NQ>
__global__ __launch_bounds__(64 * W, 8 / W)
void fa_fwd16_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
                     const uint16_t* __restrict__ Vg, uint16_t* __restrict__ Og,
                     float* __restrict__ LSEg, int N, int n_qtiles, int n_tiles, float c_log2) {
  using E = Elt<DT>;
  constexpr int KCH = D / 8;                     // 16-byte chunks per row
  constexpr int KS = D / 32;                     // GEMM0 k-steps
  constexpr int DB = D / 16;                     // 16-dim blocks of O^T
  constexpr int TILE = kBc * D;
  constexpr int ROWS_PER_LOAD = 64 / KCH;
  constexpr int WR = 16 * NQ;                    // query rows per wave
  constexpr int kBrW = WR * W;                   // query rows per workgroup
  constexpr int LPW = kBc / ROWS_PER_LOAD / W;
  static_assert(LPW * W * ROWS_PER_LOAD == kBc, "tile must split over the waves");
  static_assert(D == 128, "the swizzle is laid out for 256-byte rows");

  __shared__ __attribute__((aligned(1024))) uint16_t k_lds[2][TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds[2][TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int g = lane >> 4;

  int bh, qt;
  {
    const int hb = (!CAUSAL || N > (1 << 20) / D)
                       ? 1 : max(1, min((n_tiles / n_qtiles) >> 3, max(4, (1 << 20) / (N * D))));
    tile_of<CAUSAL>(blockIdx.x, n_tiles, n_qtiles, bh, qt, hb);
  }
  const uint16_t* K = Kg + (size_t)bh * (size_t)N * D;
  const uint16_t* V = Vg + (size_t)bh * (size_t)N * D;
  const int q_wave = qt * kBrW + wave * WR;
  const int q_lane = q_wave + l16;   // this lane's query in block 0 (block nq: + 16 nq)
  const size_t orow = (size_t)bh * (size_t)N + q_lane;
  int kend = N;
  if (CAUSAL) kend = min(N, qt * kBrW + kBrW);
  const int n_kv_real = (kend + kBc - 1) / kBc;
  const int n_kv = n_kv_real + (n_kv_real & 1);
  const int n_units = 2 * n_kv;

  // ---- Q -> registers (GEMM0 B operand): query q_lane + 16 nq, dims 32 ks + 8 g ..
  u32x4 qreg[NQ][KS];
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) {
    const uint16_t* Q = Qg + (orow + 16 * nq) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 z = {0u, 0u, 0u, 0u};
      qreg[nq][ks] = q_lane + 16 * nq < N ? *(const u32x4*)(Q + 32 * ks) : z;
    }
  }

  // ---- global -> LDS copies (as in the kernel above, swizzled by swz16)
  int src_off[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int r = (wave * LPW + i) * ROWS_PER_LOAD + lane / KCH;
    src_off[i] = r * (D * 2) + swz16(r, lane % KCH) * 16;
  }
  auto copy_tile = [&](const uint16_t* src, uint16_t* dst, int j) {
    const int key0 = min(j * kBc, kend);
    const int rows = min(kend - key0, kBc);
    const i32x4 rs = buffer_rsrc(src + (size_t)key0 * D, (uint32_t)rows * (D * 2));
    const uint32_t dst0 = lds_addr(dst) + wave * LPW * 1024;
#pragma unroll
    for (int i = 0; i < LPW; ++i) copy16_buf_to_lds(rs, src_off[i], dst0 + i * 1024);
  };

  // ---- per-lane LDS read offsets (elements)
  // GEMM0 A operand: K row 16 kb + l16 of the unit, chunk 4 ks + g
  int k_off[2][KS];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int row = 16 * kb + l16;
      k_off[kb][ks] = row * D + swz16(row, 4 * ks + g) * 8;
    }
  // GEMM1 A operand, transposing reads: half h covers keys 16 h + 4 g .. +3;
  // lane l16 of group g points at key 16 h + 4 g + l16/4, dims 16 db + 4 (l16%4) .. +3
  int v_off[2][DB];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int row = 16 * h + 4 * g + (l16 >> 2);
      const int dim = 16 * db + 4 * (l16 & 3);
      v_off[h][db] = row * D + swz16(row, dim >> 3) * 8 + (dim & 7);
    }

  f32x4 oacc[NQ][DB];
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq)
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[nq][db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  f32x4 sacc[2][NQ][2];     // [buffer][query block][key block]
  u32x4 pk[2][NQ];          // packed P, GEMM1's B operand
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) {
      sacc[b][nq][0] = sacc[b][nq][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      pk[b][nq] = u32x4{0u, 0u, 0u, 0u};
    }
  float m_run[NQ], l_run[NQ], tsum_prev[NQ];
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) {
    m_run[nq] = kMinit;
    l_run[nq] = 0.0f;
    tsum_prev[nq] = 0.0f;
  }

  auto gemm0 = [&](auto kst, auto kkb, f32x4 (&acc)[NQ][2]) {
    const uint16_t* base = &k_lds[decltype(kst)::value][decltype(kkb)::value * 32 * D];
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) acc[nq][0] = acc[nq][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 a = *(const u32x4*)(base + k_off[kb][ks]);
#pragma unroll
        for (int nq = 0; nq < NQ; ++nq) acc[nq][kb] = mma16<DT>(a, qreg[nq][ks], acc[nq][kb]);
      }
  };
  auto gemm1 = [&](auto vst, auto vkb, const u32x4 (&p)[NQ]) {
    const uint16_t* base = &v_lds[decltype(vst)::value][decltype(vkb)::value * 32 * D];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const u32x2 lo = E::read_tr(base + v_off[0][db]);
      const u32x2 hi2 = E::read_tr(base + v_off[1][db]);
      const u32x4 a = {lo[0], lo[1], hi2[0], hi2[1]};
#pragma unroll
      for (int nq = 0; nq < NQ; ++nq) oacc[nq][db] = mma16<DT>(a, p[nq], oacc[nq][db]);
    }
  };
  // p = exp2(s*c - m) packed as GEMM1's B operand; returns this lane's part of the row sum
  auto softmax = [&](const f32x4 (&sv)[2], u32x4& p, int nq) -> float {
    const float neg_m = -m_run[nq];
    float e[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        e[4 * kb + r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[kb][r], c_log2, neg_m));
    p = u32x4{E::pack(e[0], e[1]), E::pack(e[2], e[3]), E::pack(e[4], e[5]), E::pack(e[6], e[7])};
    return ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
  };
  auto mask = [&](f32x4 (&sv)[2], int u, int nq) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = 32 * u + 16 * kb + 4 * g + r;
        if (key >= kend || (CAUSAL && key > q_lane + 16 * nq)) sv[kb][r] = -INFINITY;
      }
  };
  // Rare path: the reference value of a query block must move. The unit's row
  // maximum over the four lanes of each query, then rescale O~ and l.
  auto rescale = [&](const f32x4 (&sv)[2], u32x4& p, float& tsum, int nq) {
    float mx = fmaxf(fmaxf(fmaxf(sv[0][0], sv[0][1]), fmaxf(sv[0][2], sv[0][3])),
                     fmaxf(fmaxf(sv[1][0], sv[1][1]), fmaxf(sv[1][2], sv[1][3])));
    mx = fmaxf(mx, xor16(mx));
    mx = fmaxf(mx, other_half(mx));
    const float m_new = fmaxf(m_run[nq], mx * c_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run[nq] - m_new);
    l_run[nq] *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[nq][db] *= alpha;
    m_run[nq] = m_new;
    tsum = softmax(sv, p, nq);
  };
  auto check = [&](f32x4 (&sv)[NQ][2], u32x4 (&p)[NQ]) {
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) {
      if (__builtin_amdgcn_ballot_w64(!(tsum_prev[nq] <= kSumLimit)) != 0)
        rescale(sv[nq], p[nq], tsum_prev[nq], nq);
      l_run[nq] += tsum_prev[nq];
    }
  };

  const int wave_pos = q_wave;
  auto region = [&](auto kst, auto kkb, auto vst, auto vkb, auto sb, int u) {
    constexpr int SB = decltype(sb)::value;
    const uint16_t* kbase = &k_lds[decltype(kst)::value][decltype(kkb)::value * 32 * D];
    const u32x4 a0 = *(const u32x4*)(kbase + k_off[0][0]);
    const u32x4 a1 = *(const u32x4*)(kbase + k_off[1][0]);
    check(sacc[SB ^ 1], pk[SB ^ 1]);
    if ((32 * u + 32 > kend) || (CAUSAL && 32 * u + 31 > wave_pos)) {
#pragma unroll
      for (int nq = 0; nq < NQ; ++nq) mask(sacc[SB][nq], u, nq);
    }
    f32x4 (&acc)[NQ][2] = sacc[SB ^ 1];
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) acc[nq][0] = acc[nq][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) acc[nq][0] = mma16<DT>(a0, qreg[nq][0], acc[nq][0]);
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) acc[nq][1] = mma16<DT>(a1, qreg[nq][0], acc[nq][1]);
#pragma unroll
    for (int ks = 1; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 a = *(const u32x4*)(kbase + k_off[kb][ks]);
#pragma unroll
        for (int nq = 0; nq < NQ; ++nq) acc[nq][kb] = mma16<DT>(a, qreg[nq][ks], acc[nq][kb]);
      }
    gemm1(vst, vkb, pk[SB ^ 1]);
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) {
      tsum_prev[nq] = softmax(sacc[SB][nq], pk[SB][nq], nq);
      asm volatile("" ::"v"(pk[SB][nq]), "v"(tsum_prev[nq]));
    }
    // interleave: per matrix instruction one LDS read until the region's
    // reads are placed, and one VALU instruction in the GEMM0 half of the
    // region, two in the GEMM1 half. At B=2 H=32 N=8192: +0.7% over a read
    // at three matrix instructions in four, +0.5% more over one VALU
    // throughout. Two VALU throughout, two in the GEMM0 half, three in the
    // GEMM1 half, no pinned order, the matrix instructions pinned alone, the
    // reads front-loaded two per matrix instruction or issued 4 to 8 ahead of
    // the first one each measured 1-5% slower.
    constexpr int NM = NQ * (2 * KS + DB);
    constexpr int NL = 2 * KS + 2 * DB - 2;   // reads after the two ahead of the check
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < NL) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (i >= NM / 2) __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      else __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
    }
  };
  auto sync = [&]() {
    wait_copies();
    __syncthreads();
  };
  auto copy_k = [&](auto kst, int j) { copy_tile(K, k_lds[decltype(kst)::value], j + 2); };
  auto copy_v = [&](auto kst, int j) { copy_tile(V, v_lds[decltype(kst)::value ^ 1], j + 1); };

  // ---- prologue (as in the kernel above)
#pragma unroll
  for (int i = 0; i < 2 * TILE; i += 64 * W * 8)
    *(u32x4*)(&v_lds[0][0] + i + tid * 8) = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
  copy_tile(K, k_lds[0], 0);
  copy_tile(V, v_lds[0], 0);
  copy_tile(K, k_lds[1], 1);
  wait_copies();
  __syncthreads();
  gemm0(IC<0>(), IC<0>(), sacc[0]);

  int u_stop = n_units;
  if constexpr (CAUSAL && FA_CAUSAL_EARLY_STOP) {
    const int need = (min(kend, wave_pos + WR) + 31) / 32;
    u_stop = __builtin_amdgcn_readfirstlane(min(n_units, (need / 4 + 1) * 4));
  }
  for (int u = 0; u < n_units; u += 4) {
    if (!(CAUSAL && FA_CAUSAL_EARLY_STOP) || u < u_stop) {
      region(IC<0>(), IC<1>(), IC<1>(), IC<1>(), IC<0>(), u);
      sync();
      copy_k(IC<0>(), u >> 1);
      region(IC<1>(), IC<0>(), IC<0>(), IC<0>(), IC<1>(), u + 1);
      copy_v(IC<0>(), u >> 1);
      region(IC<1>(), IC<1>(), IC<0>(), IC<1>(), IC<0>(), u + 2);
      sync();
      copy_k(IC<1>(), (u >> 1) + 1);
      region(IC<0>(), IC<0>(), IC<1>(), IC<0>(), IC<1>(), u + 3);
      copy_v(IC<1>(), (u >> 1) + 1);
    } else {
      sync();
      copy_k(IC<0>(), u >> 1);
      copy_v(IC<0>(), u >> 1);
      sync();
      copy_k(IC<1>(), (u >> 1) + 1);
      copy_v(IC<1>(), (u >> 1) + 1);
    }
  }
  wait_copies();
  check(sacc[1], pk[1]);
  gemm1(IC<1>(), IC<1>(), pk[1]);
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) asm volatile("" ::"v"(oacc[nq][db][r]));

  // ---- epilogue: O = O~ / l, LSE = ln2 * (m + log2 l); l summed over the
  // four lanes of each query
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) {
    float l_tot = l_run[nq] + xor16(l_run[nq]);
    l_tot += other_half(l_tot);
    const float inv = __builtin_amdgcn_rcpf(l_tot);
    const float lse_v = (m_run[nq] + __builtin_amdgcn_logf(l_tot)) * kLn2;
    if (q_lane + 16 * nq < N) {
      uint16_t* op = Og + (orow + 16 * nq) * D + 4 * g;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const f32x4 o = oacc[nq][db];
        *(u32x2*)(op + 16 * db) = u32x2{E::pack(o[0] * inv, o[1] * inv), E::pack(o[2] * inv, o[3] * inv)};
      }
      if (g == 0) LSEg[orow + 16 * nq] = lse_v;
    }
  }
}

// ------------------------------------------------------------------- host --


// The 16x16x32 plain forward: W waves of 16 NQ query rows each.
template <int DT, int D, bool CAUSAL, int W, int NQ>
int launch_m16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int N, float scale, hipStream_t stream) {
  const int n_qtiles = (N + 16 * NQ * W - 1) / (16 * NQ * W);
  const int n_tiles = B * H * n_qtiles;
  const float c_log2 = (float)((double)scale * kLog2e);
  const uint16_t* qp = static_cast<const uint16_t*>(q);
  const uint16_t* kp = static_cast<const uint16_t*>(k);
  const uint16_t* vp = static_cast<const uint16_t*>(v);
  uint16_t* op = static_cast<uint16_t*>(o);
  void* args[] = {&qp, &kp, &vp, &op, &lse, &N, (void*)&n_qtiles, (void*)&n_tiles, (void*)&c_log2};
  hipError_t e =
      hipLaunchKernel(reinterpret_cast<const void*>(&fa_fwd16_kernel<DT, D, CAUSAL, W, NQ>),
                      dim3(n_tiles), dim3(64 * W), args, 0, stream);
  return map_launch_error(e);
}

template <int DT, int D, bool CAUSAL, int W = kWaves, int QB = 1>
int launch16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int N, float scale, hipStream_t stream) {
  if constexpr (FA_M16 && D == 128 && !CAUSAL && W == kWaves && QB == 1) {
    // eight waves of 32 rows (256-row tiles). Measured against the 32x32x16
    // kernel: +0.3% to +2.2% here on five boxes; causal at N=8192 -0.5 to
    // -1% (1104-1110 vs 1111-1119 TFLOP/s), so the causal launch keeps it.
    return launch_m16<DT, D, CAUSAL, 8, 2>(q, k, v, o, lse, B, H, N, scale, stream);
  }
  if constexpr (W == kWaves && QB == 1) {
    if constexpr (D == 64 && !CAUSAL) {
      // d=64 without a mask: 64 query rows per wave, four waves (256 rows)
      return launch16<DT, D, CAUSAL, 4, 2>(q, k, v, o, lse, B, H, N, scale, stream);
    } else {
      // d=64 causal keeps 128-row tiles at every N (256 rows: -6% at N=16384)
      if (!CAUSAL || (D == 128 && N >= kWidePlainMinCausalN))
        return launch16<DT, D, CAUSAL, 8>(q, k, v, o, lse, B, H, N, scale, stream);
    }
  }
  const int n_qtiles = (N + 32 * QB * W - 1) / (32 * QB * W);
  const int n_tiles = B * H * n_qtiles;
  const float c_log2 = (float)((double)scale * kLog2e);
  const uint16_t* qp = static_cast<const uint16_t*>(q);
  const uint16_t* kp = static_cast<const uint16_t*>(k);
  const uint16_t* vp = static_cast<const uint16_t*>(v);
  uint16_t* op = static_cast<uint16_t*>(o);
  KvArgs none = {N, N, 0, 1, 0, nullptr};
  void* args[] = {&qp, &kp, &vp, &op, &lse, &N, (void*)&n_qtiles, (void*)&n_tiles,
                  (void*)&c_log2, &none};
  hipError_t e =
      hipLaunchKernel(reinterpret_cast<const void*>(&fa_fwd_kernel<DT, D, CAUSAL, false, false, W, QB>),
                      dim3(n_tiles), dim3(64 * W), args, 0, stream);
  return map_launch_error(e);
}

// Merge of the key-range partials: per row, LSE = log sum_s exp(LSE_s) and
// O = sum_s exp(LSE_s - LSE) O_s (the associative merge of per-block softmax
// statistics, "FlashAttention · InkStack" section 2.2). One thread per four
// dims of a row; rows = every (virtual head, row).
template <int DT, int D>
__global__ __launch_bounds__(256)
void fa_merge_kernel(const float* __restrict__ part, uint16_t* __restrict__ Og,
                     float* __restrict__ LSEg, size_t rows, int splits) {
  using E = Elt<DT>;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t row = idx / (D / 4);
  const int c = (int)(idx % (D / 4)) * 4;
  if (row >= rows) return;
  const float* lp = part + (size_t)splits * rows * D;
  // ranges are read U at a time, all loads of a group issued before any is
  // used, so a row costs one memory latency per group instead of one per range
  constexpr int U = 8;
  float m = -INFINITY;
  for (int b = 0; b < splits; b += U) {
    float l[U];
#pragma unroll
    for (int u = 0; u < U; ++u) l[u] = b + u < splits ? lp[(size_t)(b + u) * rows + row] : -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) m = fmaxf(m, l[u]);
  }
  float w_sum = 0.0f, a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
  for (int b = 0; b < splits; b += U) {
    float l[U];
    float4 o[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = b + u < splits;
      l[u] = in ? lp[(size_t)(b + u) * rows + row] : -INFINITY;
      o[u] = in ? *(const float4*)(part + ((size_t)(b + u) * rows + row) * D + c)
                : float4{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w = l[u] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((l[u] - m) * (float)kLog2e);
      a0 = __builtin_fmaf(w, o[u].x, a0);
      a1 = __builtin_fmaf(w, o[u].y, a1);
      a2 = __builtin_fmaf(w, o[u].z, a2);
      a3 = __builtin_fmaf(w, o[u].w, a3);
      w_sum += w;
    }
  }
  // w_sum = 0 only when no range saw a key (variable-length rows without keys)
  const float inv = w_sum > 0.0f ? 1.0f / w_sum : 0.0f;
  *(u32x2*)(Og + row * D + c) = u32x2{E::pack(a0 * inv, a1 * inv), E::pack(a2 * inv, a3 * inv)};
  if (c == 0) LSEg[row] = m + __builtin_amdgcn_logf(w_sum) * kLn2;
}

template <int DT, int D>
int launch_merge(const float* wsc, uint16_t* op, float* lse, size_t rows, int splits,
                 hipStream_t stream);

template <int DT, int D, bool CAUSAL, int W = kWaves>
int launch_kv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
              int Hkv, int Nq, int Nk, float scale, int splits, float* ws, hipStream_t stream) {
  const int group = H / Hkv;
  int N = group * Nq;                       // rows per virtual head
  if constexpr (W == kWaves && D == 128 && !CAUSAL) {
    if (splits == 1 && N >= kWideKvMinRows)
      return launch_kv<DT, D, CAUSAL, 8>(q, k, v, o, lse, B, H, Hkv, Nq, Nk, scale, splits, ws,
                                         stream);
  }
  const int heads = B * Hkv;
  const int n_qtiles = (N + 32 * W - 1) / (32 * W);
  const int n_tiles = heads * n_qtiles * splits;
  const int per = (Nk + splits - 1) / splits;
  KvArgs kva = {Nk, Nq, Nk - Nq, splits, (per + kBc - 1) / kBc * kBc, ws, (size_t)heads * N};
  kva.stream_kv = n_qtiles == 1;
  const float c_log2 = (float)((double)scale * kLog2e);
  const uint16_t* qp = static_cast<const uint16_t*>(q);
  const uint16_t* kp = static_cast<const uint16_t*>(k);
  const uint16_t* vp = static_cast<const uint16_t*>(v);
  uint16_t* op = static_cast<uint16_t*>(o);
  void* args[] = {&qp, &kp, &vp, &op, &lse, &N, (void*)&n_qtiles, (void*)&n_tiles,
                  (void*)&c_log2, &kva};
  hipError_t e = hipLaunchKernel(
      reinterpret_cast<const void*>(&fa_fwd_kernel<DT, D, CAUSAL, true, false, W>), dim3(n_tiles),
      dim3(64 * W), args, 0, stream);
  if (e != hipSuccess || splits == 1) return map_launch_error(e);
  return launch_merge<DT, D>(ws, op, lse, kva.rows_total, splits, stream);
}

template <int DT, int D, bool CAUSAL>
int launch_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int* cu_q, const int* cu_k, const int* order, int B, int H, int Hkv,
                  int max_q, int max_k, int total_q, int total_k, float scale, int splits,
                  float* ws, hipStream_t stream) {
  const int group = H / Hkv;
  int N = group * max_q;                    // rows of the largest virtual head
  const int heads = B * Hkv;
  const int n_qtiles = (N + kBr - 1) / kBr;
  const int n_tiles = heads * n_qtiles * splits;
  const int per = (max_k + splits - 1) / splits;
  KvArgs kva = {max_k, max_q, 0, splits, (per + kBc - 1) / kBc * kBc, ws,
                (size_t)total_q * H, cu_q, cu_k, Hkv, group, total_q, total_k, n_qtiles == 1,
                order, B};
  const float c_log2 = (float)((double)scale * kLog2e);
  const uint16_t* qp = static_cast<const uint16_t*>(q);
  const uint16_t* kp = static_cast<const uint16_t*>(k);
  const uint16_t* vp = static_cast<const uint16_t*>(v);
  uint16_t* op = static_cast<uint16_t*>(o);
  void* args[] = {&qp, &kp, &vp, &op, &lse, &N, (void*)&n_qtiles, (void*)&n_tiles,
                  (void*)&c_log2, &kva};
  hipError_t e = hipLaunchKernel(
      reinterpret_cast<const void*>(&fa_fwd_kernel<DT, D, CAUSAL, true, true>), dim3(n_tiles),
      dim3(kThreads), args, 0, stream);
  if (e != hipSuccess || splits == 1) return map_launch_error(e);
  return launch_merge<DT, D>(ws, op, lse, kva.rows_total, splits, stream);
}

template <int DT, int D>
int launch_merge(const float* wsc, uint16_t* op, float* lse, size_t rows, int splits,
                 hipStream_t stream) {
  void* margs[] = {&wsc, &op, &lse, &rows, &splits};
  const unsigned blocks = (unsigned)((rows * (D / 4) + 255) / 256);
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&fa_merge_kernel<DT, D>),
                                 dim3(blocks), dim3(256), margs, 0, stream);
  return map_launch_error(e);
}

template <int D, bool CAUSAL, bool BS = false, int W = kWaves>
int launch_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int N, float c_log2, float v_descale, hipStream_t stream,
               const float* qsc = nullptr, const float* ksc = nullptr,
               const float* vsc = nullptr) {
  if constexpr (W == kWaves && D == 128 && !BS && !CAUSAL && FA_FP8_WIDE)
    return launch_fp8<D, CAUSAL, BS, 8>(q, k, v, o, lse, B, H, N, c_log2, v_descale, stream);
  const int n_qtiles = (N + 32 * W - 1) / (32 * W);
  const int n_tiles = B * H * n_qtiles;
  const uint8_t* qp = static_cast<const uint8_t*>(q);
  const uint8_t* kp = static_cast<const uint8_t*>(k);
  const uint8_t* vp = static_cast<const uint8_t*>(v);
  uint16_t* op = static_cast<uint16_t*>(o);
  void* args[] = {&qp, &kp, &vp, &op, &lse, &N, (void*)&n_qtiles, (void*)&n_tiles,
                  (void*)&c_log2, (void*)&v_descale, (void*)&qsc, (void*)&ksc, (void*)&vsc};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&fa_fwd_fp8_kernel<D, CAUSAL, BS, W>),
                                 dim3(n_tiles), dim3(64 * W), args, 0, stream);
  return map_launch_error(e);
}

template <int DT>
int dispatch16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int N, int d, float scale, int causal, hipStream_t s) {
  if (d == 64)
    return causal ? launch16<DT, 64, true>(q, k, v, o, lse, B, H, N, scale, s)
                  : launch16<DT, 64, false>(q, k, v, o, lse, B, H, N, scale, s);
  return causal ? launch16<DT, 128, true>(q, k, v, o, lse, B, H, N, scale, s)
                : launch16<DT, 128, false>(q, k, v, o, lse, B, H, N, scale, s);
}


// Host-side checks of fa_fwd_kv and fa_fwd_kv_noalloc (everything but the
// workspace); returns FA_OK or an error.
int kv_validate(const void* q, const void* k, const void* v, const void* o, const float* lse,
                int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal, int dtype,
                int num_splits) {
  if (dtype != FA_F16 && dtype != FA_BF16 && dtype != FA_FP8_E4M3) return FA_ERR_INVALID_ARG;
  if (B < 0 || H < 0 || Hkv < 0 || Nq < 0 || Nk < 0 || d <= 0) return FA_ERR_INVALID_ARG;
  if (!(scale > 0.0f) || !isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (num_splits < 1 || num_splits > 1024) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (dtype == FA_FP8_E4M3) return FA_ERR_UNSUPPORTED;
  if ((unsigned __int128)B * (unsigned)H * (unsigned)Nq == 0) return FA_OK;
  if (Hkv == 0 || H % Hkv != 0 || Nk == 0) return FA_ERR_INVALID_ARG;
  if (causal && Nq > Nk) return FA_ERR_INVALID_ARG;
  const unsigned __int128 rows_v = (unsigned __int128)(H / Hkv) * (unsigned)Nq;
  const unsigned __int128 tiles = (unsigned __int128)B * (unsigned)Hkv * ((rows_v + 127) / 128) *
                                  (unsigned)num_splits;
  if (tiles > 0x7FFFFFFFu || rows_v > 0x7FFFFFFFu || (unsigned __int128)Nk * d > 0x7FFFFFFFu)
    return FA_ERR_INVALID_ARG;
  const void* ptrs[5] = {q, k, v, o, lse};
  for (const void* p : ptrs)
    if (!p || misaligned(p)) return FA_ERR_INVALID_ARG;
  const size_t qb = (size_t)B * H * Nq * d * 2, kb = (size_t)B * Hkv * Nk * d * 2;
  const size_t lb = (size_t)B * H * Nq * sizeof(float);
  const void* ins[3] = {q, k, v};
  const size_t in_b[3] = {qb, kb, kb};
  for (int i = 0; i < 3; ++i)
    if (overlaps(ins[i], in_b[i], o, qb) || overlaps(ins[i], in_b[i], lse, lb)) return FA_ERR_INVALID_ARG;
  if (overlaps(o, qb, lse, lb)) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

int kv_dispatch(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                int Hkv, int Nq, int Nk, int d, float scale, int causal, int dtype, int num_splits,
                float* ws, hipStream_t s) {
#define FA_KV(DT_, D_, C_) launch_kv<DT_, D_, C_>(q, k, v, o, lse, B, H, Hkv, Nq, Nk, scale, num_splits, ws, s)
  if (dtype == FA_F16) {
    if (d == 64) return causal ? FA_KV(FA_F16, 64, true) : FA_KV(FA_F16, 64, false);
    return causal ? FA_KV(FA_F16, 128, true) : FA_KV(FA_F16, 128, false);
  }
  if (d == 64) return causal ? FA_KV(FA_BF16, 64, true) : FA_KV(FA_BF16, 64, false);
  return causal ? FA_KV(FA_BF16, 128, true) : FA_KV(FA_BF16, 128, false);
#undef FA_KV
}

// ----------------------------------------------- allocation-free split-KV --
//
// fa_fwd_kv_noalloc keeps the key-range partials (fp32 O and LSE of every
// range, fa_fwd_kv_workspace bytes) in this file-scope device array instead of
// a caller workspace, for callers that cannot allocate. Every GPU the library
// runs on holds its own copy for the life of the process. Each call writes
// every partial it later reads (every range of every row, empty ranges
// included), so nothing has to start at zero; calls that overlap in time on
// one GPU share the array and race.
static __device__ __align__(256) float scratch[FA_NOALLOC_SCRATCH_BYTES / sizeof(float)];

constexpr int kMaxDevices = 256;
std::atomic<float*> g_scratch[kMaxDevices];   // device address of `scratch`, per device
std::mutex g_scratch_mu;

// Device address of this library's `scratch` on the device `stream` belongs to
// (the current device for the null stream). In host code the array's name is
// a host-side stand-in, so the address is taken once per device, with that
// device current, and only this address is handed to kernels.
int scratch_of_stream(hipStream_t stream, float** out) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return FA_ERR_LAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
  float* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) {
    *out = p;
    return FA_OK;
  }
  std::lock_guard<std::mutex> guard(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (!p) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return FA_ERR_LAUNCH;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return FA_ERR_LAUNCH;
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !a) return map_launch_error(e != hipSuccess ? e : hipErrorUnknown);
    p = static_cast<float*>(a);
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
           int d, float scale, int causal, int dtype, void* stream) {
  if (dtype != FA_F16 && dtype != FA_BF16 && dtype != FA_FP8_E4M3) return FA_ERR_INVALID_ARG;
  int rc = validate(q, k, v, o, lse, B, H, N, d, scale, causal, 2, 2);
  if (rc != FA_OK) return rc;
  if (dtype == FA_FP8_E4M3) return FA_ERR_UNSUPPORTED;
  if ((size_t)B * H * N == 0) return FA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return dtype == FA_F16 ? dispatch16<FA_F16>(q, k, v, o, lse, B, H, N, d, scale, causal, s)
                         : dispatch16<FA_BF16>(q, k, v, o, lse, B, H, N, d, scale, causal, s);
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, float q_descale,
               float k_descale, float v_descale, int B, int H, int N, int d, float scale,
               int causal, void* stream) {
  int rc = validate(q, k, v, o, lse, B, H, N, d, scale, causal, 1, 2);
  if (rc != FA_OK) return rc;
  const float ds[3] = {q_descale, k_descale, v_descale};
  for (float x : ds)
    if (!(x > 0.0f) || !isfinite(x)) return FA_ERR_INVALID_ARG;
  if ((size_t)B * H * N == 0) return FA_OK;
  const float c_log2 = (float)((double)scale * q_descale * k_descale * kLog2e);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d == 64)
    return causal ? launch_fp8<64, true>(q, k, v, o, lse, B, H, N, c_log2, v_descale, s)
                  : launch_fp8<64, false>(q, k, v, o, lse, B, H, N, c_log2, v_descale, s);
  return causal ? launch_fp8<128, true>(q, k, v, o, lse, B, H, N, c_log2, v_descale, s)
                : launch_fp8<128, false>(q, k, v, o, lse, B, H, N, c_log2, v_descale, s);
}

int fa_fwd_fp8_block(const void* q, const void* k, const void* v, void* o, float* lse,
                     const float* q_scale, const float* k_scale, const float* v_scale, int B,
                     int H, int N, int d, float scale, int causal, void* stream) {
  int rc = validate(q, k, v, o, lse, B, H, N, d, scale, causal, 1, 2);
  if (rc != FA_OK) return rc;
  if ((size_t)B * H * N == 0) return FA_OK;
  if (N > kMaxScaleTiles * kBc) return FA_ERR_UNSUPPORTED;
  const float* scs[3] = {q_scale, k_scale, v_scale};
  const size_t rows = (size_t)B * H;
  const size_t sb[3] = {rows * ((N + kBr - 1) / kBr) * sizeof(float),
                        rows * ((N + kBc - 1) / kBc) * sizeof(float),
                        rows * ((N + kBc - 1) / kBc) * sizeof(float)};
  const size_t ob = rows * N * d * 2, lb = rows * N * sizeof(float);
  for (int i = 0; i < 3; ++i) {
    if (!scs[i] || ((uintptr_t)scs[i] & 3)) return FA_ERR_INVALID_ARG;
    if (overlaps(scs[i], sb[i], o, ob) || overlaps(scs[i], sb[i], lse, lb)) return FA_ERR_INVALID_ARG;
  }
  const float c_log2 = (float)((double)scale * kLog2e);
  hipStream_t s = static_cast<hipStream_t>(stream);
#define FA_B8(D_, C_) \
  launch_fp8<D_, C_, true>(q, k, v, o, lse, B, H, N, c_log2, 1.0f, s, q_scale, k_scale, v_scale)
  if (d == 64) return causal ? FA_B8(64, true) : FA_B8(64, false);
  return causal ? FA_B8(128, true) : FA_B8(128, false);
#undef FA_B8
}

size_t fa_fwd_kv_workspace(int B, int H, int Nq, int d, int num_splits) {
  if (B <= 0 || H <= 0 || Nq <= 0 || d <= 0 || num_splits <= 1) return 0;
  return (size_t)num_splits * B * H * Nq * (size_t)(d + 1) * sizeof(float);
}

int fa_fwd_kv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
              int Hkv, int Nq, int Nk, int d, float scale, int causal, int dtype, int num_splits,
              float* workspace, void* stream) {
  int rc = kv_validate(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, dtype, num_splits);
  if (rc != FA_OK || (unsigned __int128)B * (unsigned)H * (unsigned)Nq == 0) return rc;
  const size_t qb = (size_t)B * H * Nq * d * 2, kb = (size_t)B * Hkv * Nk * d * 2;
  const size_t lb = (size_t)B * H * Nq * sizeof(float);
  const size_t wb = fa_fwd_kv_workspace(B, H, Nq, d, num_splits);
  if (num_splits > 1 && (!workspace || misaligned(workspace))) return FA_ERR_INVALID_ARG;
  const void* ins[3] = {q, k, v};
  const size_t in_b[3] = {qb, kb, kb};
  for (int i = 0; i < 3; ++i)
    if (wb && overlaps(ins[i], in_b[i], workspace, wb)) return FA_ERR_INVALID_ARG;
  if (wb && (overlaps(o, qb, workspace, wb) || overlaps(lse, lb, workspace, wb)))
    return FA_ERR_INVALID_ARG;
  return kv_dispatch(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, dtype, num_splits,
                     num_splits > 1 ? workspace : nullptr, static_cast<hipStream_t>(stream));
}

int fa_fwd_kv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int Hkv, int Nq, int Nk, int d, float scale, int causal, int dtype,
                      int num_splits, void* stream) {
  int rc = kv_validate(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, dtype, num_splits);
  if (rc != FA_OK || (unsigned __int128)B * (unsigned)H * (unsigned)Nq == 0) return rc;
  if (fa_fwd_kv_workspace(B, H, Nq, d, num_splits) > FA_NOALLOC_SCRATCH_BYTES)
    return FA_ERR_TOO_LARGE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* ws = nullptr;
  if (num_splits > 1) {
    rc = scratch_of_stream(s, &ws);
    if (rc != FA_OK) return rc;
  }
  return kv_dispatch(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, dtype, num_splits, ws,
                     s);
}

size_t fa_fwd_varlen_workspace(int total_q, int H, int d, int num_splits) {
  if (total_q <= 0 || H <= 0 || d <= 0 || num_splits <= 1) return 0;
  return (size_t)num_splits * total_q * H * (size_t)(d + 1) * sizeof(float);
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int* cu_seqlens_q, const int* cu_seqlens_k, const int* order, int B,
                  int H, int Hkv, int max_seqlen_q, int max_seqlen_k, int total_q, int total_k,
                  int d, float scale, int causal, int dtype, int num_splits, float* workspace,
                  void* stream) {
  if (dtype != FA_F16 && dtype != FA_BF16 && dtype != FA_FP8_E4M3) return FA_ERR_INVALID_ARG;
  if (B < 0 || H <= 0 || Hkv <= 0 || H % Hkv != 0 || max_seqlen_q < 0 || max_seqlen_k < 0 ||
      total_q < 0 || total_k < 0 || d <= 0)
    return FA_ERR_INVALID_ARG;
  if (!(scale > 0.0f) || !isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (num_splits < 1 || num_splits > 1024) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (dtype == FA_FP8_E4M3) return FA_ERR_UNSUPPORTED;
  if (B == 0 || total_q == 0 || max_seqlen_q == 0) return FA_OK;
  const unsigned __int128 rows_v = (unsigned __int128)(H / Hkv) * (unsigned)max_seqlen_q;
  const unsigned __int128 tiles = (unsigned __int128)B * (unsigned)Hkv * ((rows_v + 127) / 128) *
                                  (unsigned)num_splits;
  if (tiles > 0x7FFFFFFFu || rows_v > 0x7FFFFFFFu ||
      (unsigned __int128)total_k * (unsigned)Hkv * (unsigned)d > 0x7FFFFFFFu ||
      (unsigned __int128)total_q * (unsigned)H > 0x7FFFFFFFu)
    return FA_ERR_INVALID_ARG;
  const void* ptrs[7] = {q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k};
  for (const void* p : ptrs)
    if (!p) return FA_ERR_INVALID_ARG;
  const void* aligned16[4] = {q, k, v, o};
  for (const void* p : aligned16)
    if (misaligned(p)) return FA_ERR_INVALID_ARG;
  if (((uintptr_t)lse | (uintptr_t)cu_seqlens_q | (uintptr_t)cu_seqlens_k | (uintptr_t)order) & 3)
    return FA_ERR_INVALID_ARG;
  const size_t qb = (size_t)total_q * H * d * 2, kb = (size_t)total_k * Hkv * d * 2;
  const size_t lb = (size_t)total_q * H * sizeof(float), cb = (size_t)(B + 1) * sizeof(int);
  const size_t wb = fa_fwd_varlen_workspace(total_q, H, d, num_splits);
  if (num_splits > 1 && (!workspace || misaligned(workspace))) return FA_ERR_INVALID_ARG;
  // the order, when given, is read like the offsets (B int32)
  const void* ins[6] = {q, k, v, cu_seqlens_q, cu_seqlens_k, order};
  const size_t in_b[6] = {qb, kb, kb, cb, cb, order ? (size_t)B * sizeof(int) : 0};
  for (int i = 0; i < 6; ++i) {
    if (overlaps(ins[i], in_b[i], o, qb) || overlaps(ins[i], in_b[i], lse, lb)) return FA_ERR_INVALID_ARG;
    if (wb && overlaps(ins[i], in_b[i], workspace, wb)) return FA_ERR_INVALID_ARG;
  }
  if (overlaps(o, qb, lse, lb)) return FA_ERR_INVALID_ARG;
  if (wb && (overlaps(o, qb, workspace, wb) || overlaps(lse, lb, workspace, wb)))
    return FA_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* ws = num_splits > 1 ? workspace : nullptr;
#define FA_VL(DT_, D_, C_)                                                                 \
  launch_varlen<DT_, D_, C_>(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, order, B, H, Hkv, \
                             max_seqlen_q, max_seqlen_k, total_q, total_k, scale, num_splits, \
                             ws, s)
  if (dtype == FA_F16) {
    if (d == 64) return causal ? FA_VL(FA_F16, 64, true) : FA_VL(FA_F16, 64, false);
    return causal ? FA_VL(FA_F16, 128, true) : FA_VL(FA_F16, 128, false);
  }
  if (d == 64) return causal ? FA_VL(FA_BF16, 64, true) : FA_VL(FA_BF16, 64, false);
  return causal ? FA_VL(FA_BF16, 128, true) : FA_VL(FA_BF16, 128, false);
#undef FA_VL
}

int fa_varlen_order(const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int max_seqlen_q,
                    int max_seqlen_k, int total_q, int total_k, int num_splits, int* order,
                    void* stream) {
  if (B < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || total_q < 0 || total_k < 0)
    return FA_ERR_INVALID_ARG;
  if (num_splits < 1 || num_splits > 1024 || B > kMaxOrderSeqs) return FA_ERR_INVALID_ARG;
  if (B == 0) return FA_OK;
  if (!cu_seqlens_q || !cu_seqlens_k || !order) return FA_ERR_INVALID_ARG;
  if (((uintptr_t)cu_seqlens_q | (uintptr_t)cu_seqlens_k | (uintptr_t)order) & 3)
    return FA_ERR_INVALID_ARG;
  const size_t cb = (size_t)(B + 1) * sizeof(int), ob = (size_t)B * sizeof(int);
  if (overlaps(order, ob, cu_seqlens_q, cb) || overlaps(order, ob, cu_seqlens_k, cb))
    return FA_ERR_INVALID_ARG;
  const int per = (max_seqlen_k + num_splits - 1) / num_splits;
  int split_keys = (per + kBc - 1) / kBc * kBc;
  int nb = B, mq = max_seqlen_q, mk = max_seqlen_k, tq = total_q, tk = total_k;
  void* args[] = {&cu_seqlens_q, &cu_seqlens_k, &nb, &mq, &mk, &tq, &tk, &split_keys, &order};
  const unsigned blocks = (unsigned)((B + kOrderThreads - 1) / kOrderThreads);
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&fa_varlen_order_kernel),
                                 dim3(blocks), dim3(kOrderThreads), args, 0,
                                 static_cast<hipStream_t>(stream));
  return map_launch_error(e);
}

const char* fa_strerror(int code) {
  switch (code) {
    case FA_OK: return "success";
    case FA_ERR_INVALID_ARG: return "invalid argument (null, misaligned or overlapping pointer, "
                                    "negative size, bad scale, dtype or causal flag)";
    case FA_ERR_UNSUPPORTED: return "unsupported (head dimension not 64 or 128, fp8 through "
                                    "fa_fwd, or no gfx950 code for this device)";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_TOO_LARGE: return "the key-range partials need more than the allocation-free "
                                  "entry point's scratch holds (FA_NOALLOC_SCRATCH_BYTES): pass a "
                                  "workspace to fa_fwd_kv, or use fewer splits";
    default: return "unknown error code";
  }
}

int fa_version(void) { return FA_VERSION; }

}  // extern "C"
