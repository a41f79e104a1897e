// Pieces shared by the forward and backward kernels of the attention library
// for gfx950 (MI355X): vector types, the f16/bf16 matrix-instruction and
// transposing-LDS-read wrappers, the global -> LDS copy helpers, the LDS
// swizzle, the workgroup -> tile map, and the host-side argument checks.
// Each translation unit gets its own copy (anonymous namespace).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include <type_traits>

#include "fa.h"

namespace {

typedef float    f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4  __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2  __attribute__((ext_vector_type(2)));
typedef __bf16   bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16   bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8  __attribute__((ext_vector_type(8)));
typedef __fp16   fp16x4_tr __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __bf16   bf16x4_tr __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef _Float16 f16x2  __attribute__((ext_vector_type(2)));
typedef int      i32x4  __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))
#define GLOBAL_AS __attribute__((address_space(1)))

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
  // transposing LDS read of 4 16-bit elements
  static __device__ __forceinline__ u32x2 read_tr(const uint16_t* p) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4f16((LDS_AS fp16x4_tr*)p));
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
  static __device__ __forceinline__ u32x2 read_tr(const uint16_t* p) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_tr*)p));
  }
};

// four fp32 -> four OCP e4m3 bytes in order (round to nearest even; |x| <= 448).
// Each conversion writes one 16-bit half of its destination and keeps the
// other; the second overwrites the half the first kept, so the first one's
// incoming value may be anything. An empty asm statement hands it a fresh
// register with no defined contents (a constant 0, or a copy of a live
// value, costs a v_mov per packed register).
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  int any;
  asm volatile("" : "=v"(any));
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, any, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// One wave-wide 16-byte-per-lane copy global -> LDS: lane i's 16 bytes at
// `base + off` land at LDS byte address `lds + 16 * i`. Issued as inline
// assembly so the compiler does not treat every later LDS read as dependent
// on it (it would wait for the copy before the next read of any LDS buffer);
// the kernel orders the copies itself with an explicit vmcnt wait before the
// barrier that publishes a tile. The s_nop covers the M0-write hazard. These
// copy helpers and the backward's 4-byte copy are the only code in the
// library that writes M0; the build checks that on the generated code
// (no compiler-generated instruction reads or writes M0).
__device__ __forceinline__ void copy16_to_lds(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}

constexpr int kRsrcWord3 = 0x00020000;     // raw buffer, 32-bit data format

// Buffer resource over [base, base + bytes): loads at offsets >= bytes return
// zero and touch no memory.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return i32x4{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), (int)bytes, kRsrcWord3};
}

// Lane i's 16 bytes at buffer offset `off` land at LDS byte `lds + 16 * i`
// (the buffer form of copy16_to_lds, same ordering rules).
__device__ __forceinline__ void copy16_buf_to_lds(i32x4 rsrc, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(off), "s"(rsrc), "s"(lds)
               : "memory", "m0");
}

// The same with the non-temporal hint, for data read exactly once (the K/V
// history of a decode step): it streams past the caches instead of
// displacing lines that other workgroups will read again.
__device__ __forceinline__ void copy16_buf_to_lds_nt(i32x4 rsrc, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
               :
               : "v"(off), "s"(rsrc), "s"(lds)
               : "memory", "m0");
}

__device__ __forceinline__ void wait_copies() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(LDS_AS const void*)p;
}

// value of lane (l ^ 32)
__device__ __forceinline__ float other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  return __uint_as_float(lane < 32 ? r[1] : r[0]);
}

// Workgroup -> (head, query tile). Workgroups are dealt round-robin to the 8
// XCDs. When the heads split evenly over the XCDs, each XCD gets a contiguous
// range of whole heads, so the query tiles of one head (which all stream the
// same K/V) share that XCD's L2; causal tiles of a head run longest first
// (the longest-processing-time order of the FA4 walkthrough, section 3.3).
// Otherwise (few heads) a causal launch runs all heads' tiles longest first,
// so every XCD gets the same mix of long and short tiles.
// With DEAL, XCD x takes heads x, x+8, x+16, ... instead of a contiguous
// range: heads of unequal work (sequences of different lengths, laid out
// sequence-major with 8 or a multiple of 8 heads each) are then spread evenly
// over the XCDs, while each head still stays on one XCD.
// With hb > 1 (causal), an XCD takes its heads hb at a time and runs the
// tiles of those hb heads interleaved, longest first, so that the longest
// tiles of a later head do not start behind the short tiles of an earlier
// one; hb is chosen so that the bundle's K and V still fit the XCD's L2.
template <bool CAUSAL, bool DEAL = false>
__device__ __forceinline__ void tile_of(int b, int n_tiles, int n_qtiles, int& bh, int& qt,
                                        int hb = 1) {
  const int heads = n_tiles / n_qtiles;
  if (DEAL && (heads & 7) == 0) {
    const int i = (b >> 3) / n_qtiles;   // the XCD's i-th head
    qt = (b >> 3) - i * n_qtiles;
    bh = (b & 7) + 8 * i;
    if (CAUSAL) qt = n_qtiles - 1 - qt;
  } else if (CAUSAL && (heads & 7) == 0 && hb > 1) {
    const int hx = heads >> 3, i = b >> 3;   // the XCD's heads and its i-th tile
    const int bundle = i / (hb * n_qtiles), j = i - bundle * hb * n_qtiles;
    const int hbb = min(hb, hx - bundle * hb);   // heads in this bundle (the last may be short)
    const int r = j / hbb;                        // length rank, 0 = longest
    bh = (b & 7) * hx + bundle * hb + (j - r * hbb);
    qt = n_qtiles - 1 - r;
  } else if ((heads & 7) == 0 || !CAUSAL) {
    const int t = (n_tiles & 7) == 0 ? (b & 7) * (n_tiles >> 3) + (b >> 3) : b;
    bh = t / n_qtiles;
    qt = t - bh * n_qtiles;
    if (CAUSAL) qt = n_qtiles - 1 - qt;
  } else {
    const int rank = b / heads;
    bh = b - rank * heads;
    qt = n_qtiles - 1 - rank;
  }
}

// Physical 16-byte chunk of logical chunk c in row r of a K or V tile in LDS
// (64 banks of 4 bytes). The GEMM0 K read has 16 lanes per LDS cycle on 16
// consecutive rows at one logical chunk: f(r) must differ over any 16
// consecutive rows. The transposing V read has 32 lanes per cycle on 4
// consecutive rows x 4 consecutive chunks: f(r)/4 must differ over any 4
// aligned rows. 256-byte rows (d = 128): f = 4*(r%4) + (r/4)%4. 128-byte
// rows (d = 64, two rows per bank line): f = 4*((r/2)%2) + (r/4)%4, which
// makes the rows of each parity class differ in the same two senses.
template <int KCH>
__device__ __forceinline__ int swz(int r, int c) {
  if (KCH == 16) return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
  return c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

template <int V_> using IC = std::integral_constant<int, V_>;

// ---------------------------------------------------------------- host --

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Host-side checks shared by the forward entry points; returns FA_OK or an error.
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
  // the grid (one workgroup per 64 or more rows of a head) must fit a launch and
  // every byte count below must fit size_t
  const unsigned __int128 tiles =
      (unsigned __int128)B * (unsigned)H * (((unsigned)N + 63) / 64);
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

}  // namespace
