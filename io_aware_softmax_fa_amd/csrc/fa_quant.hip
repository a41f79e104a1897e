// FP8 (OCP e4m3) block quantisation for the attention kernels, gfx950.
//
// Each workgroup takes one block of `ROWS` rows of one (batch, head) matrix
// [N][D] in f16/bf16 and writes its e4m3 codes and one fp32 scale
// s = amax / 448, so that a code c stands for c * s (the per-tile scaling of
// "FlashAttention · InkStack" 3.3.1 and 3.3.3; block quantisation in the FP8
// section of the FA3 walkthrough). With a sign vector it first applies the
// incoherent transform x -> x diag(signs) H_D / sqrt(D) to every row, H_D the
// Sylvester-Hadamard matrix, as a fast Walsh-Hadamard transform
// (InkStack 3.3.2: the same orthogonal M on Q and K leaves Q K^T unchanged
// and spreads outlier dimensions over all D).
//
// The pass is bound by HBM: 2 bytes read and 1 byte written per element.
// Lanes hold 8 consecutive elements of a row (16-byte loads, D/8 lanes per
// row, 32 elements per thread, so ROWS * D / 32 threads per workgroup); the
// transform's first three butterfly stages run inside a lane, the remaining
// log2(D/8) across lanes (DPP moves, one LDS-crossbar permute). The whole
// block stays in registers between the amax reduction and the encoding.

#include "fa_common.h"

namespace {

constexpr float kE4m3Max = 448.0f;

// threads of a workgroup: 32 elements (four 16-byte chunks) per thread
template <int D, int ROWS> constexpr int quant_threads() { return ROWS * D / 32; }

// value of lane (lane ^ M) within groups of 16 lanes: M = 1, 2 by a quad
// permutation, M = 8 by a row rotation (DPP, no LDS traffic), M = 4 by a
// bpermute through the LDS crossbar
template <int M>
__device__ __forceinline__ float lane_xor(float v, int lane) {
  const int iv = __float_as_int(v);
  if constexpr (M == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(iv, 0xB1, 0xf, 0xf, false));
  if constexpr (M == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(iv, 0x4E, 0xf, 0xf, false));
  if constexpr (M == 8) return __int_as_float(__builtin_amdgcn_mov_dpp(iv, 0x128, 0xf, 0xf, false));
  return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ M) << 2, iv));
}

template <int DT>
__device__ __forceinline__ void unpack8(u32x4 w, float (&x)[8]) {
  if constexpr (DT == FA_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    // the whole vector reinterpreted at once (a per-element reinterpretation
    // of w[i] inside the unrolled loop was compiled to reads of w[0] only)
    const f16x8 h = __builtin_bit_cast(f16x8, w);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)h[i];
  }
}

// a, b -> a + b, a - b
__device__ __forceinline__ void bfly(float& a, float& b) {
  const float s = a + b, d = a - b;
  a = s;
  b = d;
}

template <int DT, int D, int ROWS, bool HAD>
__global__ __launch_bounds__((quant_threads<D, ROWS>()))
void fa_quant_kernel(const uint16_t* __restrict__ X, uint8_t* __restrict__ X8,
                     float* __restrict__ S, const float* __restrict__ signs, int N, int nblk) {
  constexpr int kQThreads = quant_threads<D, ROWS>();
  constexpr int CPR = D / 8;                   // lanes per row
  constexpr int RPP = kQThreads / CPR;         // rows per pass of the workgroup
  constexpr int PASSES = ROWS / RPP;
  static_assert(PASSES * RPP == ROWS, "block must be whole passes");
  __shared__ float red[kQThreads / 64];

  const int tid = threadIdx.x;
  const size_t bh = blockIdx.x / nblk;
  const int blk = blockIdx.x - (int)bh * nblk;
  const int c = tid % CPR;                     // this lane's 8-element chunk of its row
  const int r0 = blk * ROWS + tid / CPR;
  const size_t head = bh * (size_t)N * D;

  float sg[8];
  if constexpr (HAD) {
    const float4 a = *(const float4*)(signs + c * 8);
    const float4 b = *(const float4*)(signs + c * 8 + 4);
    sg[0] = a.x; sg[1] = a.y; sg[2] = a.z; sg[3] = a.w;
    sg[4] = b.x; sg[5] = b.y; sg[6] = b.z; sg[7] = b.w;
  }

  float x[PASSES][8];
  float amax = 0.0f;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = r0 + p * RPP;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (row < N) w = *(const u32x4*)(X + head + (size_t)row * D + c * 8);
    unpack8<DT>(w, x[p]);
    if constexpr (HAD) {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[p][i] *= sg[i];
      // element strides 1, 2, 4 inside the lane
#pragma unroll
      for (int st = 1; st < 8; st <<= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if ((i & st) == 0) bfly(x[p][i], x[p][i + st]);
      // element strides 8, 16, ... : the partner chunk is lane ^ m
      auto cross = [&](auto mc) {
        constexpr int M = decltype(mc)::value;
        const bool upper = (c & M) != 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float o = lane_xor<M>(x[p][i], tid & 63);
          x[p][i] = upper ? o - x[p][i] : x[p][i] + o;
        }
      };
      cross(IC<1>());
      cross(IC<2>());
      cross(IC<4>());
      if constexpr (CPR == 16) cross(IC<8>());
      constexpr float inv_sqrt_d = D == 64 ? 0.125f : 0.0883883476483184405f;
#pragma unroll
      for (int i = 0; i < 8; ++i) x[p][i] *= inv_sqrt_d;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[p][i]));
  }
  // block amax: across the wave, then across the workgroup's waves
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = red[0];
#pragma unroll
  for (int w = 1; w < kQThreads / 64; ++w) amax = fmaxf(amax, red[w]);
  const float s = amax > 0.0f ? amax / kE4m3Max : 1.0f;
  // x / s correctly rounded without a division per element: with r = RN(1/s)
  // and q0 = RN(x r) (within an ulp of x / s), q0 + RN-fma of the exact
  // residual (x - q0 s) times r is the correctly rounded quotient (Markstein's
  // theorem for binary floating point, no overflow or underflow here)
  const float r = 1.0f / s;

#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = r0 + p * RPP;
    if (row < N) {
      float y[8];
      // |x / s| can round a hair above 448 for the block's largest element;
      // saturate explicitly rather than rely on the conversion's overflow rule
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float q0 = x[p][i] * r;
        const float q = __builtin_fmaf(__builtin_fmaf(-q0, s, x[p][i]), r, q0);
        y[i] = fminf(fmaxf(q, -kE4m3Max), kE4m3Max);
      }
      const u32x2 w = {pack_e4m3x4(y[0], y[1], y[2], y[3]), pack_e4m3x4(y[4], y[5], y[6], y[7])};
      *(u32x2*)(X8 + head + (size_t)row * D + c * 8) = w;
    }
  }
  if (tid == 0) S[bh * nblk + blk] = s;
}

template <int DT, int D>
int launch_quant(const void* x, void* x8, float* scales, const float* signs, int heads, int N,
                 int block_rows, hipStream_t stream) {
  int nblk = (N + block_rows - 1) / block_rows;
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  uint8_t* op = static_cast<uint8_t*>(x8);
  void* args[] = {&xp, &op, &scales, &signs, &N, &nblk};
  const void* fn;
  if (block_rows == 64)
    fn = signs ? reinterpret_cast<const void*>(&fa_quant_kernel<DT, D, 64, true>)
               : reinterpret_cast<const void*>(&fa_quant_kernel<DT, D, 64, false>);
  else
    fn = signs ? reinterpret_cast<const void*>(&fa_quant_kernel<DT, D, 128, true>)
               : reinterpret_cast<const void*>(&fa_quant_kernel<DT, D, 128, false>);
  const unsigned threads = block_rows == 64 ? quant_threads<D, 64>() : quant_threads<D, 128>();
  hipError_t e = hipLaunchKernel(fn, dim3((unsigned)heads * (unsigned)nblk), dim3(threads), args,
                                 0, stream);
  return map_launch_error(e);
}

}  // namespace

extern "C" {

int fa_quantize_fp8(const void* x, void* x8, float* scales, const float* signs, int B, int H,
                    int N, int d, int block_rows, int dtype, void* stream) {
  if (dtype != FA_F16 && dtype != FA_BF16 && dtype != FA_FP8_E4M3) return FA_ERR_INVALID_ARG;
  if (B < 0 || H < 0 || N < 0 || d <= 0 || block_rows <= 0) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (block_rows != 64 && block_rows != 128) return FA_ERR_UNSUPPORTED;
  if (dtype == FA_FP8_E4M3) return FA_ERR_UNSUPPORTED;
  if ((unsigned __int128)B * (unsigned)H * (unsigned)N == 0) return FA_OK;
  const unsigned __int128 blocks =
      (unsigned __int128)B * (unsigned)H * (((unsigned)N + block_rows - 1) / block_rows);
  if (blocks > 0x7FFFFFFFu) return FA_ERR_INVALID_ARG;
  if (!x || !x8 || !scales) return FA_ERR_INVALID_ARG;
  if (misaligned(x) || misaligned(x8) || ((uintptr_t)scales & 3) || (signs && misaligned(signs)))
    return FA_ERR_INVALID_ARG;
  const size_t elems = (size_t)B * H * N * d;
  const size_t xb = elems * 2, cb = elems, sb = (size_t)blocks * sizeof(float);
  if (overlaps(x, xb, x8, cb) || overlaps(x, xb, scales, sb) || overlaps(x8, cb, scales, sb))
    return FA_ERR_INVALID_ARG;
  if (signs && (overlaps(signs, d * sizeof(float), x8, cb) ||
                overlaps(signs, d * sizeof(float), scales, sb)))
    return FA_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int heads = B * H;
  if (dtype == FA_F16)
    return d == 64 ? launch_quant<FA_F16, 64>(x, x8, scales, signs, heads, N, block_rows, s)
                   : launch_quant<FA_F16, 128>(x, x8, scales, signs, heads, N, block_rows, s);
  return d == 64 ? launch_quant<FA_BF16, 64>(x, x8, scales, signs, heads, N, block_rows, s)
                 : launch_quant<FA_BF16, 128>(x, x8, scales, signs, heads, N, block_rows, s);
}

}  // extern "C"
