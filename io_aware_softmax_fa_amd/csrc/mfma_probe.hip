// Matrix-pipe ceiling probe for gfx950 (MI355X): a measurement kernel, not
// part of the attention library's C ABI.
//
// Every wave issues only v_mfma_f32_32x32x16_bf16 on four independent
// accumulators, cycling through eight pseudo-random operand pairs held in
// registers (the dynamic power of the matrix pipe depends on how often its
// inputs toggle; constant operands let the chip clock far higher than any
// real kernel), with two waves per SIMD (eight waves per workgroup, one
// workgroup per CU) as the attention forward runs: no LDS, no global traffic
// in the loop and no VALU work beyond the loop counter. Its rate, at the
// engine clock the chip holds under that load, is the dense bf16 ceiling the
// attention kernel's throughput is compared with.
//
// The co-issue probe below runs the same matrix loop with K vector
// operations after each matrix instruction, independent of the matrix work
// and of each other across groups: plain FMAs, v_exp_f32 on fresh arguments,
// or the softmax chain of one score (FMA -> v_exp_f32 -> add into a row sum),
// so that the matrix rate lost to a given VALU mix can be read off directly.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kChains = 4;
constexpr int kSets = 8;           // operand pairs cycled per chain

// pseudo-random bf16 of either sign and magnitude about 2^-4 .. 2^3 (a hash of
// the index), so the multiplier inputs toggle like attention's operands do
__device__ __forceinline__ __bf16 rnd_bf16(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  const uint32_t bits = (x & 0x807fu) | ((0x7Bu + ((x >> 8) & 7u)) << 7);   // sign, exp 123..130, 7-bit mantissa
  return __builtin_bit_cast(__bf16, (uint16_t)bits);
}

__global__ __launch_bounds__(512, 1) void mfma_probe_kernel(float* __restrict__ out, int iters) {
  // eight operand pairs per lane, cycled so every instruction sees new inputs
  bf16x8 a[kSets], b[kSets];
#pragma unroll
  for (int s = 0; s < kSets; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t id = ((blockIdx.x * 512u + threadIdx.x) * kSets + s) * 16u + i;
      a[s][i] = rnd_bf16(id);
      b[s][i] = rnd_bf16(id + 8u);
    }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  for (int i = 0; i < iters; i += kSets) {
#pragma unroll
    for (int s = 0; s < kSets; ++s)
#pragma unroll
      for (int c = 0; c < kChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], b[(s + c) % kSets], acc[c], 0, 0, 0);
  }
  float sum = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += acc[c][r];
  // keeps the loop live (never true for a finite sum)
  if (sum != sum) out[blockIdx.x * blockDim.x + threadIdx.x] = sum;
}


// The same loop on the 16x16x32 bf16 instruction (16384 FLOP each), with
// eight accumulator chains so that the instruction count per FLOP is the
// only difference: half the accumulator bytes per FLOP of the 32x32x16 form.
typedef float f32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(512, 1) void mfma16_probe_kernel(float* __restrict__ out, int iters) {
  constexpr int kChains16 = 2 * kChains;
  bf16x8 a[kSets], b[kSets];
#pragma unroll
  for (int s = 0; s < kSets; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t id = ((blockIdx.x * 512u + threadIdx.x) * kSets + s) * 16u + i;
      a[s][i] = rnd_bf16(id);
      b[s][i] = rnd_bf16(id + 8u);
    }
  f32x4 acc[kChains16];
#pragma unroll
  for (int c = 0; c < kChains16; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[c][r] = 0.0f;
  for (int i = 0; i < iters; i += kSets) {
#pragma unroll
    for (int s = 0; s < kSets; ++s)
#pragma unroll
      for (int c = 0; c < kChains16; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], b[(s + c) % kSets], acc[c], 0, 0, 0);
  }
  float sum = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains16; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) sum += acc[c][r];
  if (sum != sum) out[blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

// Matrix loop with K VALU operations per matrix instruction. OP 0: K
// independent FMAs; OP 1: K v_exp_f32, each of an argument formed by one add
// (2K instructions); OP 2: K scores per matrix instruction, each an FMA, a
// v_exp_f32 of its result and an add into one of four running sums (3K
// instructions).
// The scheduling hints put each group right after its matrix instruction.
template <int K, int OP>
__global__ __launch_bounds__(512, 1) void coissue_probe_kernel(float* __restrict__ out, int iters) {
  bf16x8 a[kSets], b[kSets];
#pragma unroll
  for (int s = 0; s < kSets; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t id = ((blockIdx.x * 512u + threadIdx.x) * kSets + s) * 16u + i;
      a[s][i] = rnd_bf16(id);
      b[s][i] = rnd_bf16(id + 8u);
    }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  constexpr int NV = (OP == 2 && K > 2) ? 32 * K : 64;   // VALU operand slots per lane
  float v[NV], lsum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int r = 0; r < NV; ++r) v[r] = (float)((threadIdx.x * 7u + 3u * r) & 255u) * -0.03125f;
  const float cm = 0.999f, ca = 1.0e-4f;
  for (int i = 0; i < iters; i += kSets) {
    // a per-iteration offset keeps the exponentials from being hoisted
    const float fi = -(float)(i & 63) * 1.0e-3f;
#pragma unroll
    for (int s = 0; s < kSets; ++s)
#pragma unroll
      for (int c = 0; c < kChains; ++c) {
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], b[(s + c) % kSets], acc[c], 0, 0, 0);
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const int r = ((s * kChains + c) * K + k) % NV;
          if constexpr (OP == 0) {
            v[r] = __builtin_fmaf(v[r], cm, ca);
          } else if constexpr (OP == 1) {
            v[r] = __builtin_amdgcn_exp2f(v[r] + fi);
          } else {
            lsum[k & 3] += __builtin_amdgcn_exp2f(__builtin_fmaf(v[r], cm, fi));
          }
        }
        if constexpr (K > 0) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, OP == 2 ? 3 * K : (OP == 1 ? 2 * K : K), 0);
        }
      }
  }
  float sum = lsum[0] + lsum[1] + lsum[2] + lsum[3];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += acc[c][r];
#pragma unroll
  for (int r = 0; r < NV; ++r) sum += v[r];
  // keeps the loop live (never true for a finite sum)
  if (sum != sum) out[blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

// The fp8 matrix-pipe ceiling: the same loop on the 32x32x64 e4m3 matrix
// instruction (unit block scales, as the fp8 attention kernel issues it),
// operands random e4m3 bytes of either sign and exponents 5..10 (magnitudes
// about 2^-2 .. 2^3), so the multiplier inputs toggle like attention's.
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t rnd_e4m3x4(uint32_t x) {
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t h = x * 0x9E3779B1u + 0x7F4A7C15u * (uint32_t)(i + 1);
    h ^= h >> 15;
    h *= 0x2C1B3C6Du;
    h ^= h >> 12;
    const uint32_t byte = (h & 0x87u) | ((5u + (h >> 8) % 6u) << 3);   // sign, exponent 5..10, 3-bit mantissa
    w |= (byte & 0xFFu) << (8 * i);
  }
  return w;
}

__global__ __launch_bounds__(512, 1) void mfma_fp8_probe_kernel(float* __restrict__ out, int iters) {
  i32x8 a[kSets], b[kSets];
#pragma unroll
  for (int s = 0; s < kSets; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t id = ((blockIdx.x * 512u + threadIdx.x) * kSets + s) * 16u + i;
      a[s][i] = (int)rnd_e4m3x4(id);
      b[s][i] = (int)rnd_e4m3x4(id + 8u);
    }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  for (int i = 0; i < iters; i += kSets) {
#pragma unroll
    for (int s = 0; s < kSets; ++s)
#pragma unroll
      for (int c = 0; c < kChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[s], b[(s + c) % kSets], acc[c],
                                                                0, 0, 0, 127, 0, 127);
  }
  float sum = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += acc[c][r];
  if (sum != sum) out[blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

}  // namespace

extern "C" {

// Runs `blocks` workgroups of 512 threads, each wave issuing iters * 4 matrix
// instructions of 32x32x16 (32768 FLOP each; iters a multiple of 8), on
// `stream`. `out` (device, blocks * 512 floats) is written only if a sum is
// NaN, which it cannot be. Returns 0, or -1 for bad arguments, -3 if the
// launch failed.
int fa_probe_mfma(float* out, int blocks, int iters, void* stream) {
  if (!out || blocks <= 0 || iters <= 0 || iters % kSets != 0) return -1;
  void* args[] = {&out, &iters};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&mfma_probe_kernel), dim3(blocks),
                                 dim3(512), args, 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? 0 : -3;
}

// The co-issue probe: the matrix loop of fa_probe_mfma with K VALU
// operations of kind `op` per matrix instruction (op 0: FMA, K in
// {2, 4, 8}; op 1: add and v_exp_f32, K in {2, 4}; op 2: softmax chain of K
// scores, K in {1, 2, 3}). Same grid, arguments and return codes as fa_probe_mfma;
// -2 for an (op, K) pair that is not built.
int fa_probe_coissue(float* out, int blocks, int iters, int op, int k, void* stream) {
  if (!out || blocks <= 0 || iters <= 0 || iters % kSets != 0) return -1;
  const void* f = nullptr;
  if (op == 0 && k == 2) f = reinterpret_cast<const void*>(&coissue_probe_kernel<2, 0>);
  if (op == 0 && k == 4) f = reinterpret_cast<const void*>(&coissue_probe_kernel<4, 0>);
  if (op == 0 && k == 8) f = reinterpret_cast<const void*>(&coissue_probe_kernel<8, 0>);
  if (op == 1 && k == 2) f = reinterpret_cast<const void*>(&coissue_probe_kernel<2, 1>);
  if (op == 1 && k == 4) f = reinterpret_cast<const void*>(&coissue_probe_kernel<4, 1>);
  if (op == 2 && k == 1) f = reinterpret_cast<const void*>(&coissue_probe_kernel<1, 2>);
  if (op == 2 && k == 2) f = reinterpret_cast<const void*>(&coissue_probe_kernel<2, 2>);
  if (op == 2 && k == 3) f = reinterpret_cast<const void*>(&coissue_probe_kernel<3, 2>);
  if (!f) return -2;
  void* args[] = {&out, &iters};
  hipError_t e = hipLaunchKernel(f, dim3(blocks), dim3(512), args, 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? 0 : -3;
}

// The fp8 ceiling probe: fa_probe_mfma's loop on the 32x32x64 e4m3 matrix
// instruction (131072 FLOP each; fa_probe_mfma_flops(blocks, iters) * 4).
// Same grid, arguments and return codes as fa_probe_mfma.
int fa_probe_mfma_fp8(float* out, int blocks, int iters, void* stream) {
  if (!out || blocks <= 0 || iters <= 0 || iters % kSets != 0) return -1;
  void* args[] = {&out, &iters};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&mfma_fp8_probe_kernel), dim3(blocks),
                                 dim3(512), args, 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? 0 : -3;
}

// The ceiling loop on the 16x16x32 bf16 instruction: twice the instructions
// of fa_probe_mfma at half the FLOPs each, so the same FLOPs per call
// (fa_probe_mfma_flops). Same grid, arguments and return codes.
int fa_probe_mfma16(float* out, int blocks, int iters, void* stream) {
  if (!out || blocks <= 0 || iters <= 0 || iters % kSets != 0) return -1;
  void* args[] = {&out, &iters};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&mfma16_probe_kernel), dim3(blocks),
                                 dim3(512), args, 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? 0 : -3;
}

// FLOPs one call of fa_probe_mfma or fa_probe_coissue performs.
double fa_probe_mfma_flops(int blocks, int iters) {
  return (double)blocks * 8.0 * (double)iters * kChains * 32768.0;
}

}  // extern "C"
