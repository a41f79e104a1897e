// Attention forward pass for gfx950 (MI355X, CDNA4): C ABI and kernels.
//
// O = softmax(scale * Q K^T) V and LSE = m + ln(l), computed one query tile
// per workgroup with an online softmax, so the score and probability tiles
// live only in registers ("FlashAttention · InkStack" sections 1.1 and 2.1-2.3;
// MUSA guide "FlashAttention 优化", complete-algorithm section).
//
// Work decomposition (sequence parallelism, "FlashAttention · InkStack" 2.2):
// one workgroup per (batch, head, 256-query tile); four waves, each owning 64
// query rows outright (split-Q, section 2.3), so no cross-wave reduction.
// Keys and values stream through LDS in 64-key tiles, double buffered: the
// global loads of tile j+1 are in flight while tile j is computed.
//
// Both products run on MFMA 32x32x16 (f16/bf16 in, fp32 accumulate):
//   GEMM0  S^T[key][query] = K[key][:] . Q[query][:]   (A = K from LDS, B = Q in VGPRs)
//   GEMM1  O^T[dim][query] += V^T[dim][key] . P^T[key][query]  (A = V^T from LDS, B = P in VGPRs)
// Computing the transposed products puts one query column in each lane, so a
// row max or row sum over keys is 16 in-lane values plus one swap with the
// lane 32 away, and the per-query rescale factor is a per-lane scalar.
// The fp32 score accumulator is turned into GEMM1's B operand in place; the
// key order this implies is matched by the order V^T is written to LDS, so the
// two permutations cancel (the register-permutation idea of the FA3
// walkthrough "FlashAttention 完全拆解（三）", FP8 layout section).
//
// Softmax in base 2: t = s * scale * log2(e); p = exp2(t - m) on v_exp_f32.
// The running max is moved only when a row's tile max exceeds it by more than
// 8 (a factor 256), decided once per wave (the rescale skip of the FA4
// walkthrough, section 3.1.4). Any reference value m gives the same O = O~/l
// and LSE = m + log l, so the skip changes rounding only; p stays <= 256.
// Normalisation by 1/l and the LSE write happen once, in the epilogue
// (deferred normalisation, "FlashAttention · InkStack" 2.1).

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "fa.h"

namespace {

typedef float    f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4  __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2  __attribute__((ext_vector_type(2)));
typedef __bf16   bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16   bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8  __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2  __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;          // four wave64s
constexpr int kBr = 256;               // query rows per workgroup
constexpr int kWaveRows = 64;          // query rows per wave (two 32-column MFMA blocks)
constexpr int kBc = 64;                // keys per KV tile
constexpr float kRescaleThreshold = 8.0f;   // log2 units: rescale only past a factor 256
constexpr float kLn2 = 0.693147180559945309f;
constexpr double kLog2e = 1.4426950408889634074;

// ------------------------------------------------------------ element types --

template <int DT> struct Elt;

template <> struct Elt<FA_F16> {
  static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  // two fp32 -> packed f16 pair, round to nearest even
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    f16x2 h = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, h);
  }
};

template <> struct Elt<FA_BF16> {
  static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    bf16x2 h = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, h);
  }
};

__device__ __forceinline__ float xor32(float x) {
  return __shfl_xor(x, 32, 64);
}

// Workgroup -> tile. Workgroups are dealt round-robin to the 8 XCDs; give each
// XCD a contiguous range of tiles so the query tiles of one head (which all
// stream the same K/V) share that XCD's L2.
__device__ __forceinline__ int xcd_tile(int b, int n) {
  if ((n & 7) != 0) return b;
  return (b & 7) * (n >> 3) + (b >> 3);
}

// Position of key `k` (0..63) of a KV tile inside a V^T row in LDS: bits 2 and
// 3 swapped, which is the key order of GEMM1's B operand taken straight from
// GEMM0's accumulator (lane half h holds keys {4h..4h+3, 8+4h..8+4h+3} of
// each 16-key step).
__device__ __forceinline__ int vt_pos(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// ------------------------------------------------------------------ kernel --

template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1)
void fa_fwd_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
                   const uint16_t* __restrict__ Vg, uint16_t* __restrict__ Og,
                   float* __restrict__ LSEg, int N, int n_qtiles, int n_tiles,
                   float c_log2) {
  using E = Elt<DT>;
  constexpr int KCH = D / 8;          // 16-byte chunks per K row
  constexpr int KS = D / 16;          // GEMM0 k-steps
  constexpr int DB = D / 32;          // 32-row blocks of O^T
  constexpr int K_ELEMS = kBc * D;    // one K stage, elements
  constexpr int V_ELEMS = D * kBc;    // one V^T stage, elements
  constexpr int K_LOADS = kBc * KCH / kThreads;          // 16-byte K loads per thread
  constexpr int V_UNITS = (kBc / 4) * KCH;               // (4 keys x 8 dims) units
  constexpr int V_LOADS = (V_UNITS + kThreads - 1) / kThreads;
  static_assert(K_LOADS * kThreads == kBc * KCH, "K tile must split evenly");

  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * (K_ELEMS + V_ELEMS)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const int t = xcd_tile(blockIdx.x, n_tiles);
  const int bh = t / n_qtiles;
  int qt = t - bh * n_qtiles;
  if (CAUSAL) qt = n_qtiles - 1 - qt;     // longest tiles of a head first

  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* Q = Qg + head;
  const uint16_t* K = Kg + head;
  const uint16_t* V = Vg + head;
  uint16_t* O = Og + head;
  float* LSE = LSEg + (size_t)bh * N;

  const int q_wave = qt * kBr + wave * kWaveRows;
  const bool wave_live = q_wave < N;

  // KV tiles this workgroup streams, and the ones this wave needs
  const int kv_len = CAUSAL ? min(N, qt * kBr + kBr) : N;
  const int n_kv = (kv_len + kBc - 1) / kBc;
  const int wave_kv_len = !wave_live ? 0 : (CAUSAL ? min(N, q_wave + kWaveRows) : N);
  const int wave_n_kv = (wave_kv_len + kBc - 1) / kBc;

  // ---- Q tile -> registers (GEMM0 B operand), loaded once
  u32x4 qreg[2][KS];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int row = q_wave + 32 * c + l32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 z = {0u, 0u, 0u, 0u};
      qreg[c][ks] = row < N ? *(const u32x4*)(Q + (size_t)row * D + ks * 16 + hi * 8) : z;
    }
  }

  f32x16 oacc[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][c][r] = 0.0f;
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.0f, 0.0f};

  // ---- K/V staging: global -> registers -> LDS
  u32x4 kbuf[K_LOADS];
  u32x4 vbuf[V_LOADS][4];

  auto load_tile = [&](int j) {
    const int key0 = j * kBc;
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) {
      const int ci = tid + i * kThreads;
      const int row = ci / KCH, ch = ci % KCH;
      u32x4 z = {0u, 0u, 0u, 0u};
      kbuf[i] = (key0 + row < N) ? *(const u32x4*)(K + (size_t)(key0 + row) * D + ch * 8) : z;
    }
#pragma unroll
    for (int i = 0; i < V_LOADS; ++i) {
      const int u = tid + i * kThreads;
      const int kg = u / KCH, ch = u % KCH;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = key0 + 4 * kg + r;
        u32x4 z = {0u, 0u, 0u, 0u};
        vbuf[i][r] = (u < V_UNITS && key < N) ? *(const u32x4*)(V + (size_t)key * D + ch * 8) : z;
      }
    }
  };

  auto store_tile = [&](int stage) {
    uint16_t* ks_ = lds + stage * (K_ELEMS + V_ELEMS);
    uint16_t* vs_ = ks_ + K_ELEMS;
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) {
      const int ci = tid + i * kThreads;
      const int row = ci / KCH, ch = ci % KCH;
      *(u32x4*)(ks_ + row * D + ((ch ^ (row % KCH)) * 8)) = kbuf[i];
    }
#pragma unroll
    for (int i = 0; i < V_LOADS; ++i) {
      const int u = tid + i * kThreads;
      if (u < V_UNITS) {
        const int kg = u / KCH, ch = u % KCH;
        const int pos = vt_pos(4 * kg);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int dd = ch * 8 + e;
          const int sh = (e & 1) * 16;
          const uint32_t x0 = (vbuf[i][0][e >> 1] >> sh) & 0xFFFFu;
          const uint32_t x1 = (vbuf[i][1][e >> 1] >> sh) & 0xFFFFu;
          const uint32_t x2 = (vbuf[i][2][e >> 1] >> sh) & 0xFFFFu;
          const uint32_t x3 = (vbuf[i][3][e >> 1] >> sh) & 0xFFFFu;
          u32x2 w = {x0 | (x1 << 16), x2 | (x3 << 16)};
          *(u32x2*)(vs_ + dd * kBc + (((pos >> 3) ^ (dd & 7)) * 8) + (pos & 7)) = w;
        }
      }
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < n_kv; ++j) {
    if (j + 1 < n_kv) load_tile(j + 1);

    if (j < wave_n_kv) {
      const uint16_t* ks_ = lds + (j & 1) * (K_ELEMS + V_ELEMS);
      const uint16_t* vs_ = ks_ + K_ELEMS;
      const int key0 = j * kBc;

      // ---- GEMM0: S^T = K Q^T for 64 keys x 64 queries
      f32x16 sacc[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[kb][c][r] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int row = kb * 32 + l32;
          const u32x4 a = *(const u32x4*)(ks_ + row * D + (((2 * ks + hi) ^ (row % KCH)) * 8));
#pragma unroll
          for (int c = 0; c < 2; ++c) sacc[kb][c] = E::mma(a, qreg[c][ks], sacc[kb][c]);
        }
      }

      // ---- mask (ragged tail, causal diagonal)
      const bool need_mask = (key0 + kBc > N) || (CAUSAL && key0 + kBc - 1 > q_wave);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int qi = q_wave + 32 * c + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
              if (key >= N || (CAUSAL && key > qi)) sacc[kb][c][r] = -INFINITY;
            }
          }
      }

      // ---- online softmax statistics
      float mt[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float mx = sacc[0][c][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][c][r]);
        mx = fmaxf(mx, xor32(mx));
        mt[c] = mx * c_log2;
      }
      const bool grow = (mt[0] > m_run[0] + kRescaleThreshold) ||
                        (mt[1] > m_run[1] + kRescaleThreshold);
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          float m_new = fmaxf(m_run[c], mt[c]);
          if (m_new == -INFINITY) m_new = 0.0f;   // no visible key yet: nothing to rescale
          const float alpha = __builtin_amdgcn_exp2f(m_run[c] - m_new);
          l_run[c] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][c][r] *= alpha;
          m_run[c] = m_new;
        }
      }

      // ---- P = exp2(s*c - m), row-sum partials, pack to GEMM1's B operand
      u32x4 pk[2][2][2];   // [kb][c][16-key half]
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const float neg_m = -m_run[c];
        float sum = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          float p[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][c][r], c_log2, neg_m));
            sum += p[r];
          }
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            u32x4 w = {E::pack(p[8 * h + 0], p[8 * h + 1]), E::pack(p[8 * h + 2], p[8 * h + 3]),
                       E::pack(p[8 * h + 4], p[8 * h + 5]), E::pack(p[8 * h + 6], p[8 * h + 7])};
            pk[kb][c][h] = w;
          }
        }
        l_run[c] += sum;
      }

      // ---- GEMM1: O^T += V^T P^T
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int row = db * 32 + l32;
#pragma unroll
        for (int kv = 0; kv < 4; ++kv) {
          const u32x4 a = *(const u32x4*)(vs_ + row * kBc + (((2 * kv + hi) ^ (row & 7)) * 8));
#pragma unroll
          for (int c = 0; c < 2; ++c)
            oacc[db][c] = E::mma(a, pk[kv >> 1][c][kv & 1], oacc[db][c]);
        }
      }
    }

    if (j + 1 < n_kv) store_tile((j + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: O = O~ / l, LSE = ln2 * (m + log2 l)
  if (wave_live) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const float l_tot = l_run[c] + xor32(l_run[c]);
      const float inv = __builtin_amdgcn_rcpf(l_tot);
      const int qi = q_wave + 32 * c + l32;
      if (qi < N) {
        uint16_t* orow = O + (size_t)qi * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            u32x2 w = {E::pack(oacc[db][c][4 * g + 0] * inv, oacc[db][c][4 * g + 1] * inv),
                       E::pack(oacc[db][c][4 * g + 2] * inv, oacc[db][c][4 * g + 3] * inv)};
            *(u32x2*)(orow + db * 32 + 8 * g + 4 * hi) = w;
          }
        if (hi == 0) LSE[qi] = (m_run[c] + __builtin_amdgcn_logf(l_tot)) * kLn2;
      }
    }
  }
}

// ------------------------------------------------------------------- host --

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Host-side checks shared by both entry points; returns FA_OK or an error.
int validate(const void* q, const void* k, const void* v, const void* o, const void* lse,
             int B, int H, int N, int d, float scale, int causal, size_t in_esz,
             size_t out_esz) {
  if (B < 0 || H < 0 || N < 0 || d <= 0) return FA_ERR_INVALID_ARG;
  if (!(scale > 0.0f) || !isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if ((unsigned __int128)B * (unsigned)H * (unsigned)N == 0) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(lse))
    return FA_ERR_INVALID_ARG;
  // the grid (one workgroup per 256 query rows of a head) must fit a launch and
  // every byte count below must fit size_t
  const unsigned __int128 tiles =
      (unsigned __int128)B * (unsigned)H * (((unsigned)N + kBr - 1) / kBr);
  if (tiles > 0x7FFFFFFFu) return FA_ERR_INVALID_ARG;
  const size_t rows = (size_t)B * (size_t)H * (size_t)N;
  const size_t in_bytes = rows * d * in_esz, out_bytes = rows * d * out_esz;
  const size_t lse_bytes = rows * sizeof(float);
  const void* ins[3] = {q, k, v};
  for (const void* p : ins)
    if (overlaps(p, in_bytes, o, out_bytes) || overlaps(p, in_bytes, lse, lse_bytes))
      return FA_ERR_INVALID_ARG;
  if (overlaps(o, out_bytes, lse, lse_bytes)) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

int map_launch_error(hipError_t e) {
  if (e == hipSuccess) return FA_OK;
  if (e == hipErrorNoBinaryForGpu || e == hipErrorInvalidDeviceFunction) return FA_ERR_UNSUPPORTED;
  return FA_ERR_LAUNCH;
}

template <int DT, int D, bool CAUSAL>
int launch16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int N, float scale, hipStream_t stream) {
  const int n_qtiles = (N + kBr - 1) / kBr;
  const int n_tiles = B * H * n_qtiles;
  const float c_log2 = (float)((double)scale * kLog2e);
  const uint16_t* qp = static_cast<const uint16_t*>(q);
  const uint16_t* kp = static_cast<const uint16_t*>(k);
  const uint16_t* vp = static_cast<const uint16_t*>(v);
  uint16_t* op = static_cast<uint16_t*>(o);
  void* args[] = {&qp, &kp, &vp, &op, &lse, &N, (void*)&n_qtiles, (void*)&n_tiles,
                  (void*)&c_log2};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&fa_fwd_kernel<DT, D, CAUSAL>),
                                 dim3(n_tiles), dim3(kThreads), args, 0, stream);
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
  (void)stream;
  return FA_ERR_UNSUPPORTED;
}

const char* fa_strerror(int code) {
  switch (code) {
    case FA_OK: return "success";
    case FA_ERR_INVALID_ARG: return "invalid argument (null, misaligned or overlapping pointer, "
                                    "negative size, bad scale, dtype or causal flag)";
    case FA_ERR_UNSUPPORTED: return "unsupported (head dimension not 64 or 128, fp8 through "
                                    "fa_fwd, or no gfx950 code for this device)";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown error code";
  }
}

int fa_version(void) { return FA_VERSION; }

}  // extern "C"
