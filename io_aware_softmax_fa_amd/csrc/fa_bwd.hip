// Attention backward pass for gfx950 (MI355X, CDNA4): kernels and C ABI.
//
// Gradients of O = softmax(scale * Q K^T) V for an upstream gradient dO
// ("FlashAttention · InkStack" section 1.2.1), with P rebuilt from the scores
// and the forward's saved statistic, P = exp(S - LSE) (section 1.2.2):
//   dV = P^T dO,   dP = dO V^T,   D_i = rowsum(dO * O)_i,
//   dS = P * (dP - D),   dQ = scale * dS K,   dK = scale * dS^T Q.
//
// Three launches on the caller's stream:
//   1. bwd_prep:  -D = -rowsum(dO * O) and LSE in base-2 units, into the
//                 caller's workspace (one pass over O and dO);
//   2. bwd_dkdv:  one workgroup per 128 keys of a head (four waves x 32 keys,
//                 each wave holding its K and V rows in registers) streams
//                 the query tiles through LDS and accumulates dK and dV (the
//                 key-parallel loop of section 1.2.3, the outer loop over
//                 K/V blocks); d = 128 takes an eight-wave form with 256
//                 keys per workgroup and V in LDS (bwd_dkdv_wide);
//   3. bwd_dq:    one workgroup per 128 queries (four waves x 32 queries,
//                 each holding its Q and dO rows in registers) streams the
//                 key tiles through LDS and accumulates dQ.
// Splitting dQ into its own query-parallel pass replaces the cross-block
// atomic accumulation of dQ (section 2.2) with plain stores: every output
// element is written once, by one lane, and the result is deterministic.
//
// All products run on MFMA 32x32x16 (f16/bf16 in, fp32 accumulate); P and dS
// are rounded to the input type before the products that consume them. The
// layouts are the forward's: a wave's 32-row block is one MFMA column block,
// the accumulator of a score-shaped product becomes the B operand of the next
// product in place, and the A operand of that product is read from LDS with
// the transposing read in the matching row order (the register-permutation
// idea of the FA3 walkthrough, FP8 layout section).

#include "fa_common.h"

namespace {

constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = 64 * kBwdWaves;
constexpr int kBwdRows = 32 * kBwdWaves;   // keys (dk/dv pass) or queries (dq pass) per workgroup
constexpr int kTile = 64;                  // rows of a streamed LDS tile

// Causal launches take an XCD's heads in bundles whose K and V (4 N d bytes
// each) fill at most 4 MB, its L2, and at least 4 heads while one head's
// fit, with the bundle's tiles interleaved longest first: the forward's order
// (tile_of). One head per bundle, in each head longest first, for longer
// heads and without a mask.
__device__ __forceinline__ int bwd_bundle(bool causal, int heads, int N, int D) {
  return (!causal || N > (1 << 20) / D) ? 1 : max(1, min(heads >> 3, max(4, (1 << 20) / (N * D))));
}
// key tile of workgroup b: a dK/dV workgroup's work shrinks with its key
// tile under the causal mask, so the longest-first rank maps to kt = rank
__device__ __forceinline__ void bwd_key_tile(bool causal, int b, int n_tiles, int n_ktiles, int N,
                                             int D, int& bh, int& kt) {
  if (!causal) {
    tile_of<false>(b, n_tiles, n_ktiles, bh, kt);
    return;
  }
  int r;
  tile_of<true>(b, n_tiles, n_ktiles, bh, r, bwd_bundle(true, n_tiles / n_ktiles, N, D));
  kt = n_ktiles - 1 - r;
}

// two packed 16-bit values -> fp32
template <int DT>
__device__ __forceinline__ void unpack2(uint32_t w, float& lo, float& hi) {
  if constexpr (DT == FA_BF16) {
    lo = __uint_as_float(w << 16);
    hi = __uint_as_float(w & 0xffff0000u);
  } else {
    const f16x2 h = __builtin_bit_cast(f16x2, w);
    lo = (float)h[0];
    hi = (float)h[1];
  }
}

// Lane i's 4 bytes at buffer offset `off` land at LDS byte `lds + 4 * i`.
__device__ __forceinline__ void copy4_buf_to_lds(i32x4 rsrc, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(off), "s"(rsrc), "s"(lds)
               : "memory", "m0");
}

// ---------------------------------------------------------------- prep --
// D_i = sum_d dO[i][d] * O[i][d] in fp32, stored negated (the later kernels
// start their dP accumulators at -D_i), and L2_i = LSE_i * log2(e).
// D/8 lanes share a row (one 16-byte chunk each) and reduce with lane shuffles.
template <int DT, int D>
__global__ __launch_bounds__(256)
void bwd_prep_kernel(const uint16_t* __restrict__ Og, const uint16_t* __restrict__ dOg,
                     const float* __restrict__ LSEg, float* __restrict__ ws, size_t rows) {
  constexpr int LPR = D / 8;                     // lanes per row
  const size_t row = ((size_t)blockIdx.x * 256 + threadIdx.x) / LPR;
  const int part = threadIdx.x % LPR;
  float acc = 0.0f;
  if (row < rows) {
    const u32x4 o = *(const u32x4*)(Og + row * D + part * 8);
    const u32x4 g = *(const u32x4*)(dOg + row * D + part * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float o0, o1, g0, g1;
      unpack2<DT>(o[w], o0, o1);
      unpack2<DT>(g[w], g0, g1);
      acc = __builtin_fmaf(o0, g0, acc);
      acc = __builtin_fmaf(o1, g1, acc);
    }
  }
#pragma unroll
  for (int s = LPR / 2; s >= 1; s >>= 1) acc += __shfl_xor(acc, s, LPR);
  if (row < rows && part == 0) {
    ws[row] = -acc;
    ws[rows + row] = LSEg[row] * (float)kLog2e;
  }
}

// ------------------------------------------------------------ dK and dV --
//
// Per 32-query unit of a streamed query tile, wave w (keys kt*128 + 32w ..):
//   S  = Q_u K^T      (A = Q rows from LDS, B = this wave's K rows)
//   dP = dO_u V^T     (A = dO rows from LDS, B = this wave's V rows)
//   P  = exp2(S * scale*log2e - L2_row),  dS = P * (dP - D_row)
//   dV^T += dO_u^T P  (A = dO^T by transposing LDS read, B = P)
//   dK^T += Q_u^T dS  (A = Q^T by transposing LDS read, B = dS)
// The accumulators put one query row per register and one key per lane
// column, so L2 and D vary per register: they are staged in LDS with the tile
// and read four rows at a time. Rows past N read as zero (Q = dO = L2 = D =
// 0), which makes P = 1 and dS = 0 there and adds nothing.
template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, 1)
void bwd_dkdv_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
                     const uint16_t* __restrict__ Vg, const uint16_t* __restrict__ dOg,
                     const float* __restrict__ ws, uint16_t* __restrict__ dKg,
                     uint16_t* __restrict__ dVg, int N, int n_ktiles, int n_tiles, size_t rows,
                     float c_log2, float scale) {
  using E = Elt<DT>;
  constexpr int KCH = D / 8;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILE = kTile * D;
  constexpr int ROWS_PER_LOAD = 64 / KCH;
  constexpr int LPW = kTile / ROWS_PER_LOAD / kBwdWaves;
  static_assert(LPW * kBwdWaves * ROWS_PER_LOAD == kTile, "tile must split over the waves");

  // Q stages [0], [1] and dO stages [2], [3] in one array: every operand
  // read of a unit is then one of a few lane offsets plus an immediate
  __shared__ __attribute__((aligned(1024))) uint16_t qd_lds[4][TILE];
  __shared__ __attribute__((aligned(256))) float l2_lds[2][kTile];
  __shared__ __attribute__((aligned(256))) float dl_lds[2][kTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  int bh, kt;
  bwd_key_tile(CAUSAL, blockIdx.x, n_tiles, n_ktiles, N, D, bh, kt);
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* Q = Qg + head;
  const uint16_t* dO = dOg + head;
  const float* dlg = ws + (size_t)bh * N;
  const float* l2g = ws + rows + (size_t)bh * N;

  const int key = kt * kBwdRows + wave * 32 + l32;   // this lane's key (B operand column)
  // a query sees key j only if j <= query: causal tiles start at the first
  // query tile that reaches this workgroup's first key
  const int i0 = CAUSAL ? (kt * kBwdRows) / kTile : 0;
  const int n_qt = (N + kTile - 1) / kTile;

  // ---- K and V rows of this lane's key -> registers (B operands)
  u32x4 kreg[KS], vreg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    kreg[ks] = key < N ? *(const u32x4*)(Kg + head + (size_t)key * D + ks * 16 + hi * 8) : z;
    vreg[ks] = key < N ? *(const u32x4*)(Vg + head + (size_t)key * D + ks * 16 + hi * 8) : z;
  }

  // ---- copies of query tile i: Q and dO rows (swizzled as in the forward),
  // L2 and D (wave 0); ranged buffer loads, rows past N read as zero
  uint32_t src_off[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int r = (wave * LPW + i) * ROWS_PER_LOAD + lane / KCH;
    src_off[i] = r * (D * 2) + swz<KCH>(r, lane % KCH) * 16;
  }
  auto copy_tile = [&](int i, int st) {
    const int r0 = min(i * kTile, N);
    const int nr = min(N - r0, kTile);
    const i32x4 rq = buffer_rsrc(Q + (size_t)r0 * D, (uint32_t)nr * (D * 2));
    const i32x4 rd = buffer_rsrc(dO + (size_t)r0 * D, (uint32_t)nr * (D * 2));
    const uint32_t dq0 = lds_addr(&qd_lds[st][0]) + wave * LPW * 1024;
    const uint32_t dd0 = lds_addr(&qd_lds[2 + st][0]) + wave * LPW * 1024;
#pragma unroll
    for (int k = 0; k < LPW; ++k) {
      copy16_buf_to_lds(rq, src_off[k], dq0 + k * 1024);
      copy16_buf_to_lds(rd, src_off[k], dd0 + k * 1024);
    }
    if (wave == 0) {
      copy4_buf_to_lds(buffer_rsrc(l2g + r0, (uint32_t)nr * 4), lane * 4, lds_addr(&l2_lds[st][0]));
      copy4_buf_to_lds(buffer_rsrc(dlg + r0, (uint32_t)nr * 4), lane * 4, lds_addr(&dl_lds[st][0]));
    }
  };

  // ---- LDS read offsets (elements): row-major operand reads (rows l32) and
  // transposing reads (the forward's V-read pattern)
  int k_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) k_off[ks] = l32 * D + swz<KCH>(l32, 2 * ks + hi) * 8;
  int t_off[2][DB];
  {
    const int g = lane >> 4, jj = lane & 15;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int row = 8 * h2 + 4 * (g >> 1) + (jj >> 2);
        const int dim = db * 32 + 16 * (g & 1) + 4 * (jj & 3);
        t_off[h2][db] = row * D + swz<KCH>(row, dim >> 3) * 8 + (dim & 7);
      }
  }

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[db][r] = dv[db][r] = 0.0f;

  // st (LDS stage) and ub (unit of the tile) are compile-time constants
  auto unit = [&](auto ST, auto UB, int q0) {
    constexpr int st = decltype(ST)::value;
    constexpr int ub = decltype(UB)::value;
    const uint16_t* qb = &qd_lds[st][ub * 32 * D];
    const uint16_t* db_ = &qd_lds[2 + st][ub * 32 * D];
    // One wave per SIMD: issue every operand read of the unit up front so
    // their latency overlaps the matrix work instead of stalling each product.
    u32x4 qa[KS], da[KS], ta[2][2][DB];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qa[ks] = *(const u32x4*)(qb + k_off[ks]);
      da[ks] = *(const u32x4*)(db_ + k_off[ks]);
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int d2 = 0; d2 < DB; ++d2) {
        const u32x2 a0 = E::read_tr(db_ + s2 * 16 * D + t_off[0][d2]);
        const u32x2 a1 = E::read_tr(db_ + s2 * 16 * D + t_off[1][d2]);
        ta[0][s2][d2] = u32x4{a0[0], a0[1], a1[0], a1[1]};
        const u32x2 b0 = E::read_tr(qb + s2 * 16 * D + t_off[0][d2]);
        const u32x2 b1 = E::read_tr(qb + s2 * 16 * D + t_off[1][d2]);
        ta[1][s2][d2] = u32x4{b0[0], b0[1], b1[0], b1[1]};
      }
    // row statistics: register r holds query row 8*(r/4) + 4*hi + r%4; the
    // dP accumulator starts at -D of its row (the workspace holds -D), so
    // the chain yields dP - D
    f32x16 s = {}, dp;
    float l2v[16];
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int o = ub * 32 + 8 * g4 + 4 * hi;
      const float4 a = *(const float4*)&l2_lds[st][o];
      const float4 b = *(const float4*)&dl_lds[st][o];
      l2v[4 * g4 + 0] = a.x; l2v[4 * g4 + 1] = a.y; l2v[4 * g4 + 2] = a.z; l2v[4 * g4 + 3] = a.w;
      dp[4 * g4 + 0] = b.x; dp[4 * g4 + 1] = b.y; dp[4 * g4 + 2] = b.z; dp[4 * g4 + 3] = b.w;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = E::mma(qa[ks], kreg[ks], s);
      dp = E::mma(da[ks], vreg[ks], dp);
    }
    float p[16], ds[16];
    // only a unit on the causal diagonal (a query of the unit before one of
    // the wave's keys) needs the per-element mask (wave-uniform branch)
    const bool diag = CAUSAL && kt * kBwdRows + wave * 32 + 31 > q0;
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c_log2, -l2v[r]));
    if (diag) {
      asm volatile("");   // keeps the block a branch (not speculated into selects)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (key > q0 + 8 * (r >> 2) + 4 * hi + (r & 3)) p[r] = 0.0f;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      ds[r] = p[r] * dp[r];
    }
    u32x4 ppk[2], spk[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      ppk[h] = u32x4{E::pack(p[8 * h + 0], p[8 * h + 1]), E::pack(p[8 * h + 2], p[8 * h + 3]),
                     E::pack(p[8 * h + 4], p[8 * h + 5]), E::pack(p[8 * h + 6], p[8 * h + 7])};
      spk[h] = u32x4{E::pack(ds[8 * h + 0], ds[8 * h + 1]), E::pack(ds[8 * h + 2], ds[8 * h + 3]),
                     E::pack(ds[8 * h + 4], ds[8 * h + 5]), E::pack(ds[8 * h + 6], ds[8 * h + 7])};
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int d2 = 0; d2 < DB; ++d2) {
        dv[d2] = E::mma(ta[0][s2][d2], ppk[s2], dv[d2]);
        dk[d2] = E::mma(ta[1][s2][d2], spk[s2], dk[d2]);
      }
  };

  // ---- query-tile loop, double buffered, two tiles per iteration (the
  // stages compile-time constants): after the barrier that publishes tile i,
  // every wave is done with tile i-1, whose stage takes tile i+1
  auto tile = [&](auto ST, int i) {
    wait_copies();
    __syncthreads();
    if (i + 1 < n_qt) copy_tile(i + 1, decltype(ST)::value ^ 1);
    unit(ST, IC<0>{}, i * kTile);
    unit(ST, IC<1>{}, i * kTile + 32);
  };
  if (i0 < n_qt) {
    copy_tile(i0, 0);
    int i = i0;
    for (; i + 1 < n_qt; i += 2) {
      tile(IC<0>{}, i);
      tile(IC<1>{}, i + 1);
    }
    if (i < n_qt) tile(IC<0>{}, i);
  }
  wait_copies();

  // ---- epilogue: lane holds dK^T / dV^T column `key`; rows are dims
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) asm volatile("" ::"v"(dk[db][r]), "v"(dv[db][r]));
  if (key < N) {
    uint16_t* krow = dKg + head + (size_t)key * D;
    uint16_t* vrow = dVg + head + (size_t)key * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int dim = db * 32 + 8 * g4 + 4 * hi;
        *(u32x2*)(krow + dim) = u32x2{E::pack(dk[db][4 * g4 + 0] * scale, dk[db][4 * g4 + 1] * scale),
                                      E::pack(dk[db][4 * g4 + 2] * scale, dk[db][4 * g4 + 3] * scale)};
        *(u32x2*)(vrow + dim) = u32x2{E::pack(dv[db][4 * g4 + 0], dv[db][4 * g4 + 1]),
                                      E::pack(dv[db][4 * g4 + 2], dv[db][4 * g4 + 3])};
      }
  }
}

// Eight-wave form of the dK/dV kernel: 256 keys per workgroup, two waves per
// SIMD. The one-wave-per-SIMD form above holds K and V of its keys in
// registers (64 of them at d = 128) next to the dK and dV accumulators (128),
// which leaves no room for a second wave per SIMD; here V of the workgroup's
// keys sits in LDS instead (64 KB, rows in the forward's K-tile swizzle, so
// that the dP product reads its B operand with the same conflict-free pattern
// as the Q and dO reads), and each query tile copied into LDS serves twice
// the keys. Wave w copies and reads only the V rows of its own 32 keys, so no
// barrier is needed for them. Units before a wave's first key (causal) are
// skipped by that wave.
// Dispatched for d = 128, measured against the one-wave forms (whole
// backward, B=2 H=32 N=8192, four runs each on one box): causal +7.4%
// (+9.2% on another lease), non-causal +9.2% against the software-pipelined
// one-wave form it replaces. The loop takes two tiles per iteration (LDS
// stages as compile-time constants) with a scheduling fence between units:
// left to interleave two units, the scheduler overlaps their live ranges and
// the kernel spills. At d = 64 the plain form, already at two waves per SIMD,
// stays (this form measured -4% non-causal, -20% causal).
#ifndef FA_BWD_WIDE
#define FA_BWD_WIDE 1
#endif
constexpr int kBwd2Waves = 8;
constexpr int kBwd2Rows = 32 * kBwd2Waves;   // keys per workgroup

template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kBwd2Waves, 1)
void bwd_dkdv_wide_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
                          const uint16_t* __restrict__ Vg, const uint16_t* __restrict__ dOg,
                          const float* __restrict__ ws, uint16_t* __restrict__ dKg,
                          uint16_t* __restrict__ dVg, int N, int n_ktiles, int n_tiles,
                          size_t rows, float c_log2, float scale) {
  using E = Elt<DT>;
  constexpr int KCH = D / 8;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILE = kTile * D;
  constexpr int ROWS_PER_LOAD = 64 / KCH;
  constexpr int LPW = kTile / ROWS_PER_LOAD / kBwd2Waves;
  constexpr int VPW = 32 / ROWS_PER_LOAD;          // V copies per wave (its 32 keys)
  static_assert(LPW * kBwd2Waves * ROWS_PER_LOAD == kTile, "tile must split over the waves");

  // Q stages [0], [1] and dO stages [2], [3] in one array: every operand
  // read of a unit is then one of a few lane offsets plus an immediate
  __shared__ __attribute__((aligned(1024))) uint16_t qd_lds[4][TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds[kBwd2Rows * D];
  __shared__ __attribute__((aligned(256))) float l2_lds[2][kTile];
  __shared__ __attribute__((aligned(256))) float dl_lds[2][kTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  int bh, kt;
  bwd_key_tile(CAUSAL, blockIdx.x, n_tiles, n_ktiles, N, D, bh, kt);
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* Q = Qg + head;
  const uint16_t* dO = dOg + head;
  const float* dlg = ws + (size_t)bh * N;
  const float* l2g = ws + rows + (size_t)bh * N;

  const int key0 = kt * kBwd2Rows;                   // the workgroup's first key
  const int wkey0 = key0 + wave * 32;                // this wave's first key
  const int key = wkey0 + l32;                       // this lane's key (B operand column)
  const int i0 = CAUSAL ? key0 / kTile : 0;
  const int n_qt = (N + kTile - 1) / kTile;

  // ---- K rows of this lane's key -> registers (B operand of S)
  u32x4 kreg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    kreg[ks] = key < N ? *(const u32x4*)(Kg + head + (size_t)key * D + ks * 16 + hi * 8) : z;
  }
  // ---- V rows of this wave's keys -> LDS (rows past N read as zero)
  {
    // (both uniform; spelled out so the resource lands in scalar registers)
    const int nr = __builtin_amdgcn_readfirstlane(max(min(N - wkey0, 32), 0));
    const int vr0 = __builtin_amdgcn_readfirstlane(min(wkey0, N));
    const i32x4 rv = buffer_rsrc(Vg + head + (size_t)vr0 * D, (uint32_t)nr * (D * 2));
    const uint32_t dv0 = lds_addr(&v_lds[wave * 32 * D]);
#pragma unroll
    for (int i = 0; i < VPW; ++i) {
      const int r = i * ROWS_PER_LOAD + lane / KCH;   // row within the wave's 32
      copy16_buf_to_lds(rv, r * (D * 2) + swz<KCH>(r, lane % KCH) * 16, dv0 + i * 1024);
    }
  }

  // ---- copies of query tile i: Q and dO rows, L2 and D (wave 0)
  uint32_t src_off[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int r = (wave * LPW + i) * ROWS_PER_LOAD + lane / KCH;
    src_off[i] = r * (D * 2) + swz<KCH>(r, lane % KCH) * 16;
  }
  auto copy_tile = [&](int i, int st) {
    const int r0 = min(i * kTile, N);
    const int nr = min(N - r0, kTile);
    const i32x4 rq = buffer_rsrc(Q + (size_t)r0 * D, (uint32_t)nr * (D * 2));
    const i32x4 rd = buffer_rsrc(dO + (size_t)r0 * D, (uint32_t)nr * (D * 2));
    const uint32_t dq0 = lds_addr(&qd_lds[st][0]) + wave * LPW * 1024;
    const uint32_t dd0 = lds_addr(&qd_lds[2 + st][0]) + wave * LPW * 1024;
#pragma unroll
    for (int k = 0; k < LPW; ++k) {
      copy16_buf_to_lds(rq, src_off[k], dq0 + k * 1024);
      copy16_buf_to_lds(rd, src_off[k], dd0 + k * 1024);
    }
    if (wave == 0) {
      copy4_buf_to_lds(buffer_rsrc(l2g + r0, (uint32_t)nr * 4), lane * 4, lds_addr(&l2_lds[st][0]));
      copy4_buf_to_lds(buffer_rsrc(dlg + r0, (uint32_t)nr * 4), lane * 4, lds_addr(&dl_lds[st][0]));
    }
  };

  // ---- LDS read offsets (elements)
  int k_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) k_off[ks] = l32 * D + swz<KCH>(l32, 2 * ks + hi) * 8;
  int t_off[2][DB];
  {
    const int g = lane >> 4, jj = lane & 15;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int row = 8 * h2 + 4 * (g >> 1) + (jj >> 2);
        const int dim = db * 32 + 16 * (g & 1) + 4 * (jj & 3);
        t_off[h2][db] = row * D + swz<KCH>(row, dim >> 3) * 8 + (dim & 7);
      }
  }
  const uint16_t* vbase = &v_lds[wave * 32 * D];

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[db][r] = dv[db][r] = 0.0f;

  // st (LDS stage) and ub (unit of the tile) are compile-time constants, so
  // every operand read's address is a loop-invariant lane offset plus an
  // immediate
  auto unit = [&](auto ST, auto UB, int q0) {
    constexpr int st = decltype(ST)::value;
    constexpr int ub = decltype(UB)::value;
    // a causal unit wholly before the wave's keys adds nothing
    if (CAUSAL && q0 + 31 < wkey0) return;
    const uint16_t* qb = &qd_lds[st][ub * 32 * D];
    const uint16_t* db_ = &qd_lds[2 + st][ub * 32 * D];
    // register r holds query row 8*(r/4) + 4*hi + r%4; the dP accumulator
    // starts at -D of its row (the workspace holds -D), so the chain yields
    // dP - D
    f32x16 s = {}, dp;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const float4 b = *(const float4*)&dl_lds[st][ub * 32 + 8 * g4 + 4 * hi];
      dp[4 * g4 + 0] = b.x; dp[4 * g4 + 1] = b.y; dp[4 * g4 + 2] = b.z; dp[4 * g4 + 3] = b.w;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = E::mma(*(const u32x4*)(qb + k_off[ks]), kreg[ks], s);
      dp = E::mma(*(const u32x4*)(db_ + k_off[ks]), *(const u32x4*)(vbase + k_off[ks]), dp);
    }
    float p[16], ds[16];
    const bool diag = CAUSAL && wkey0 + 31 > q0;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const float4 a = *(const float4*)&l2_lds[st][ub * 32 + 8 * g4 + 4 * hi];
      const float l2v[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * g4 + j;
        const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c_log2, -l2v[j]));
        p[r] = pr;
        ds[r] = pr * dp[r];
      }
    }
    // the mask, on the diagonal unit only (a wave-uniform branch; folded
    // into the loop above it would cost three VALU instructions per score
    // on every unit): P and dS of a key after its query are zero, whatever
    // the unmasked score gave (inf and NaN included)
    if (diag) {
      asm volatile("");   // keeps the block a branch (not speculated into selects)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (key > q0 + 8 * (r >> 2) + 4 * hi + (r & 3)) p[r] = ds[r] = 0.0f;
    }
    u32x4 ppk[2], spk[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      ppk[h] = u32x4{E::pack(p[8 * h + 0], p[8 * h + 1]), E::pack(p[8 * h + 2], p[8 * h + 3]),
                     E::pack(p[8 * h + 4], p[8 * h + 5]), E::pack(p[8 * h + 6], p[8 * h + 7])};
      spk[h] = u32x4{E::pack(ds[8 * h + 0], ds[8 * h + 1]), E::pack(ds[8 * h + 2], ds[8 * h + 3]),
                     E::pack(ds[8 * h + 4], ds[8 * h + 5]), E::pack(ds[8 * h + 6], ds[8 * h + 7])};
    }
    // keep the transposing reads of the dV/dK products after the scores'
    // products: issued earlier they hold 64 registers across them and spill
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int d2 = 0; d2 < DB; ++d2) {
        const u32x2 a0 = E::read_tr(db_ + s2 * 16 * D + t_off[0][d2]);
        const u32x2 a1 = E::read_tr(db_ + s2 * 16 * D + t_off[1][d2]);
        dv[d2] = E::mma(u32x4{a0[0], a0[1], a1[0], a1[1]}, ppk[s2], dv[d2]);
        const u32x2 b0 = E::read_tr(qb + s2 * 16 * D + t_off[0][d2]);
        const u32x2 b1 = E::read_tr(qb + s2 * 16 * D + t_off[1][d2]);
        dk[d2] = E::mma(u32x4{b0[0], b0[1], b1[0], b1[1]}, spk[s2], dk[d2]);
      }
  };

  // ---- query-tile loop, double buffered, two tiles (four 32-query units)
  // per iteration: after the barrier that publishes tile i, every wave is
  // done with tile i-1, whose stage takes tile i+1 (the first barrier also
  // publishes each wave's V rows to itself). The scheduling fences keep the
  // units apart: interleaved, their live ranges overlap and spill.
  auto tile = [&](auto ST, int i) {
    wait_copies();
    __syncthreads();
    if (i + 1 < n_qt) copy_tile(i + 1, decltype(ST)::value ^ 1);
    unit(ST, IC<0>{}, 64 * i);
    __builtin_amdgcn_sched_barrier(0);
    unit(ST, IC<1>{}, 64 * i + 32);
    __builtin_amdgcn_sched_barrier(0);
  };
  if (i0 < n_qt) {
    copy_tile(i0, 0);
    int i = i0;
    for (; i + 1 < n_qt; i += 2) {
      tile(IC<0>{}, i);
      tile(IC<1>{}, i + 1);
    }
    if (i < n_qt) tile(IC<0>{}, i);
  }
  wait_copies();

  // ---- epilogue: lane holds dK^T / dV^T column `key`; rows are dims
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) asm volatile("" ::"v"(dk[db][r]), "v"(dv[db][r]));
  if (key < N) {
    uint16_t* krow = dKg + head + (size_t)key * D;
    uint16_t* vrow = dVg + head + (size_t)key * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int dim = db * 32 + 8 * g4 + 4 * hi;
        *(u32x2*)(krow + dim) = u32x2{E::pack(dk[db][4 * g4 + 0] * scale, dk[db][4 * g4 + 1] * scale),
                                      E::pack(dk[db][4 * g4 + 2] * scale, dk[db][4 * g4 + 3] * scale)};
        *(u32x2*)(vrow + dim) = u32x2{E::pack(dv[db][4 * g4 + 0], dv[db][4 * g4 + 1]),
                                      E::pack(dv[db][4 * g4 + 2], dv[db][4 * g4 + 3])};
      }
  }
}

// ------------------------------------------------------------------ dQ --
//
// Per 32-key unit of a streamed K/V tile, wave w (queries qt*128 + 32w ..):
//   S^T  = K_u Q^T     (A = K rows from LDS, B = this wave's Q rows)
//   dP^T = V_u dO^T    (A = V rows from LDS, B = this wave's dO rows)
//   P^T  = exp2(S^T * scale*log2e - L2_q),  dS^T = P^T * (dP^T - D_q)
//   dQ^T += K_u^T dS^T (A = K^T by transposing LDS read, B = dS^T)
// One query per lane column, so L2 and D are per-lane scalars. Keys past N
// and, when causal, keys after the query are masked to P = 0.
template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, 2)
void bwd_dq_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
                   const uint16_t* __restrict__ Vg, const uint16_t* __restrict__ dOg,
                   const float* __restrict__ ws, uint16_t* __restrict__ dQg, int N,
                   int n_qtiles, int n_tiles, size_t rows, float c_log2, float scale) {
  using E = Elt<DT>;
  constexpr int KCH = D / 8;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILE = kTile * D;
  constexpr int ROWS_PER_LOAD = 64 / KCH;
  constexpr int LPW = kTile / ROWS_PER_LOAD / kBwdWaves;
  static_assert(LPW * kBwdWaves * ROWS_PER_LOAD == kTile, "tile must split over the waves");

  // K stages [0], [1] and V stages [2], [3] in one array: every operand read
  // of a unit is then one of a few lane offsets plus an immediate
  __shared__ __attribute__((aligned(1024))) uint16_t kv_lds[4][TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  int bh, qt;
  tile_of<CAUSAL>(blockIdx.x, n_tiles, n_qtiles, bh, qt, bwd_bundle(CAUSAL, n_tiles / n_qtiles, N, D));
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* K = Kg + head;
  const uint16_t* V = Vg + head;

  const int q_wave = qt * kBwdRows + wave * 32;
  const int q_lane = q_wave + l32;
  const int kv_len = CAUSAL ? min(N, qt * kBwdRows + kBwdRows) : N;
  const int n_kv = (kv_len + kTile - 1) / kTile;

  u32x4 qreg[KS], dreg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    qreg[ks] = q_lane < N ? *(const u32x4*)(Qg + head + (size_t)q_lane * D + ks * 16 + hi * 8) : z;
    dreg[ks] = q_lane < N ? *(const u32x4*)(dOg + head + (size_t)q_lane * D + ks * 16 + hi * 8) : z;
  }
  // -D of this lane's query (the workspace holds -D): the first dP product
  // of every unit accumulates onto it, so the chain yields dP - D
  const float ndl = q_lane < N ? ws[(size_t)bh * N + q_lane] : 0.0f;
  f32x16 ndl16;
#pragma unroll
  for (int r = 0; r < 16; ++r) ndl16[r] = ndl;
  const float l2 = q_lane < N ? ws[rows + (size_t)bh * N + q_lane] : 0.0f;

  uint32_t src_off[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int r = (wave * LPW + i) * ROWS_PER_LOAD + lane / KCH;
    src_off[i] = r * (D * 2) + swz<KCH>(r, lane % KCH) * 16;
  }
  auto copy_tile = [&](int j, int st) {
    const int r0 = min(j * kTile, N);
    const int nr = min(N - r0, kTile);
    const i32x4 rk = buffer_rsrc(K + (size_t)r0 * D, (uint32_t)nr * (D * 2));
    const i32x4 rv = buffer_rsrc(V + (size_t)r0 * D, (uint32_t)nr * (D * 2));
    const uint32_t dk0 = lds_addr(&kv_lds[st][0]) + wave * LPW * 1024;
    const uint32_t dv0 = lds_addr(&kv_lds[2 + st][0]) + wave * LPW * 1024;
#pragma unroll
    for (int k = 0; k < LPW; ++k) {
      copy16_buf_to_lds(rk, src_off[k], dk0 + k * 1024);
      copy16_buf_to_lds(rv, src_off[k], dv0 + k * 1024);
    }
  };

  int k_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) k_off[ks] = l32 * D + swz<KCH>(l32, 2 * ks + hi) * 8;
  int t_off[2][DB];
  {
    const int g = lane >> 4, jj = lane & 15;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int row = 8 * h2 + 4 * (g >> 1) + (jj >> 2);
        const int dim = db * 32 + 16 * (g & 1) + 4 * (jj & 3);
        t_off[h2][db] = row * D + swz<KCH>(row, dim >> 3) * 8 + (dim & 7);
      }
  }

  f32x16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[db][r] = 0.0f;

  // st (LDS stage) and ub (unit of the tile) are compile-time constants
  auto unit = [&](auto ST, auto UB, int k0) {
    constexpr int st = decltype(ST)::value;
    constexpr int ub = decltype(UB)::value;
    const uint16_t* kb = &kv_lds[st][ub * 32 * D];
    const uint16_t* vb = &kv_lds[2 + st][ub * 32 * D];
    f32x16 s = {}, dp = ndl16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = E::mma(*(const u32x4*)(kb + k_off[ks]), qreg[ks], s);
      dp = E::mma(*(const u32x4*)(vb + k_off[ks]), dreg[ks], dp);
    }
    float ds[16];
    // keys past N or after a query exist only in the last unit and on the
    // causal diagonal: the per-element mask is applied there alone
    // (wave-uniform branch)
    if (k0 + 32 > N || (CAUSAL && k0 + 31 > q_wave)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = k0 + 8 * (r >> 2) + 4 * hi + (r & 3);
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c_log2, -l2));
        if (kk >= N || (CAUSAL && kk > q_lane)) p = 0.0f;
        ds[r] = p * dp[r];
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        ds[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c_log2, -l2)) * dp[r];
    }
    u32x4 spk[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      spk[h] = u32x4{E::pack(ds[8 * h + 0], ds[8 * h + 1]), E::pack(ds[8 * h + 2], ds[8 * h + 3]),
                     E::pack(ds[8 * h + 4], ds[8 * h + 5]), E::pack(ds[8 * h + 6], ds[8 * h + 7])};
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const uint16_t* kt_ = kb + s2 * 16 * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x2 a0 = E::read_tr(kt_ + t_off[0][db]);
        const u32x2 a1 = E::read_tr(kt_ + t_off[1][db]);
        dq[db] = E::mma(u32x4{a0[0], a0[1], a1[0], a1[1]}, spk[s2], dq[db]);
      }
    }
  };

  // double-buffered key tiles, two per iteration so that the stages are
  // compile-time constants
  auto tile = [&](auto ST, int j) {
    wait_copies();
    __syncthreads();
    if (j + 1 < n_kv) copy_tile(j + 1, decltype(ST)::value ^ 1);
    unit(ST, IC<0>{}, j * kTile);
    unit(ST, IC<1>{}, j * kTile + 32);
  };
  copy_tile(0, 0);
  int j = 0;
  for (; j + 1 < n_kv; j += 2) {
    tile(IC<0>{}, j);
    tile(IC<1>{}, j + 1);
  }
  if (j < n_kv) tile(IC<0>{}, j);
  wait_copies();

#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) asm volatile("" ::"v"(dq[db][r]));
  if (q_lane < N) {
    uint16_t* qrow = dQg + head + (size_t)q_lane * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *(u32x2*)(qrow + db * 32 + 8 * g4 + 4 * hi) =
            u32x2{E::pack(dq[db][4 * g4 + 0] * scale, dq[db][4 * g4 + 1] * scale),
                  E::pack(dq[db][4 * g4 + 2] * scale, dq[db][4 * g4 + 3] * scale)};
  }
}

// ---------------------------------------------------------------- host --

template <int DT, int D, bool CAUSAL>
int launch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
               const float* lse, void* dq, void* dk, void* dv, float* ws, int B, int H, int N,
               float scale, hipStream_t stream) {
  const size_t rows = (size_t)B * H * N;
  const float c_log2 = (float)((double)scale * kLog2e);
  const uint16_t* qp = static_cast<const uint16_t*>(q);
  const uint16_t* kp = static_cast<const uint16_t*>(k);
  const uint16_t* vp = static_cast<const uint16_t*>(v);
  const uint16_t* op = static_cast<const uint16_t*>(o);
  const uint16_t* gp = static_cast<const uint16_t*>(dout);
  uint16_t* dqp = static_cast<uint16_t*>(dq);
  uint16_t* dkp = static_cast<uint16_t*>(dk);
  uint16_t* dvp = static_cast<uint16_t*>(dv);
  const float* wsc = ws;

  const unsigned prep_blocks = (unsigned)((rows * (D / 8) + 255) / 256);
  void* a0[] = {&op, &gp, &lse, &ws, (void*)&rows};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_prep_kernel<DT, D>),
                                 dim3(prep_blocks), dim3(256), a0, 0, stream);
  if (e != hipSuccess) return map_launch_error(e);

  int n_k = (N + kBwdRows - 1) / kBwdRows;
  int nt = B * H * n_k;
  if constexpr (FA_BWD_WIDE && D == 128) {
    int n_k2 = (N + kBwd2Rows - 1) / kBwd2Rows;
    int nt2 = B * H * n_k2;
    void* a1[] = {&qp, &kp, &vp, &gp, &wsc, &dkp, &dvp, &N, &n_k2, &nt2, (void*)&rows,
                  (void*)&c_log2, &scale};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dkdv_wide_kernel<DT, D, CAUSAL>),
                        dim3(nt2), dim3(64 * kBwd2Waves), a1, 0, stream);
  } else {
    void* a1[] = {&qp, &kp, &vp, &gp, &wsc, &dkp, &dvp, &N, &n_k, &nt, (void*)&rows,
                  (void*)&c_log2, &scale};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dkdv_kernel<DT, D, CAUSAL>), dim3(nt),
                        dim3(kBwdThreads), a1, 0, stream);
  }
  if (e != hipSuccess) return map_launch_error(e);

  void* a2[] = {&qp, &kp, &vp, &gp, &wsc, &dqp, &N, &n_k, &nt, (void*)&rows, (void*)&c_log2,
                &scale};
  e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dq_kernel<DT, D, CAUSAL>),
                      dim3(nt), dim3(kBwdThreads), a2, 0, stream);
  return map_launch_error(e);
}

template <int DT>
int dispatch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, float* ws, int B, int H, int N,
                 int d, float scale, int causal, hipStream_t s) {
  if (d == 64)
    return causal ? launch_bwd<DT, 64, true>(q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, N, scale, s)
                  : launch_bwd<DT, 64, false>(q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, N, scale, s);
  return causal ? launch_bwd<DT, 128, true>(q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, N, scale, s)
                : launch_bwd<DT, 128, false>(q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, N, scale, s);
}

}  // namespace

extern "C" int fa_bwd(const void* q, const void* k, const void* v, const void* o,
                      const void* dout, const float* lse, void* dq, void* dk, void* dv,
                      float* workspace, int B, int H, int N, int d, float scale, int causal,
                      int dtype, void* stream) {
  if (dtype != FA_F16 && dtype != FA_BF16 && dtype != FA_FP8_E4M3) return FA_ERR_INVALID_ARG;
  if (B < 0 || H < 0 || N < 0 || d <= 0) return FA_ERR_INVALID_ARG;
  if (!(scale > 0.0f) || !isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (dtype == FA_FP8_E4M3) return FA_ERR_UNSUPPORTED;
  if ((unsigned __int128)B * (unsigned)H * (unsigned)N == 0) return FA_OK;
  const void* all[10] = {q, k, v, o, dout, lse, dq, dk, dv, workspace};
  for (const void* p : all)
    if (!p || misaligned(p)) return FA_ERR_INVALID_ARG;
  const unsigned __int128 tiles = (unsigned __int128)B * (unsigned)H * (((unsigned)N + 63) / 64);
  if (tiles > 0x7FFFFFFFu) return FA_ERR_INVALID_ARG;
  const size_t rows = (size_t)B * H * N;
  const size_t tb = rows * d * 2;
  // outputs (dq, dk, dv, workspace) must not overlap each other or any input
  const void* outs[4] = {dq, dk, dv, workspace};
  const size_t out_b[4] = {tb, tb, tb, 2 * rows * sizeof(float)};
  const void* ins[6] = {q, k, v, o, dout, lse};
  const size_t in_b[6] = {tb, tb, tb, tb, tb, rows * sizeof(float)};
  for (int a = 0; a < 4; ++a) {
    for (int b = 0; b < 6; ++b)
      if (overlaps(outs[a], out_b[a], ins[b], in_b[b])) return FA_ERR_INVALID_ARG;
    for (int b = a + 1; b < 4; ++b)
      if (overlaps(outs[a], out_b[a], outs[b], out_b[b])) return FA_ERR_INVALID_ARG;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  return dtype == FA_F16
             ? dispatch_bwd<FA_F16>(q, k, v, o, dout, lse, dq, dk, dv, workspace, B, H, N, d, scale, causal, s)
             : dispatch_bwd<FA_BF16>(q, k, v, o, dout, lse, dq, dk, dv, workspace, B, H, N, d, scale, causal, s);
}
