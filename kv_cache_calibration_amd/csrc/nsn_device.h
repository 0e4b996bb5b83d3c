// Device helpers shared by the NSNQuant HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include <type_traits>

#include "nsn_launch.h"

namespace nsn {

constexpr int kD = 128;      // head_dim
constexpr int kCodes = 256;  // codebook entries
constexpr int kWave = 64;

// Prepared-codebook blob layout (bytes).  Written by nsn_prepare_codebook.
//   [0, 8192)        float32 codebook [256][m], m in {4, 8}
//   [8192, 9216)     float32 squared norms [256]
//   [9216, 13312)    fp16 codebook [256][m] (exact: entries are fp16 values
//                    when built by nsn_build_codebook; otherwise rounded)
//   [16384, 17408)   u8 bin of each fine cell of [-4.5, 4.5) (1024 cells)
//   [17408, 17508)   float32 bin edges [25]
//   kTabMain         u64 per 4-d grid cell: eight candidate codes (below)
// The 4-d search tables exist for m = 4 only.
constexpr size_t kTabCodebook = 0;
constexpr size_t kTabNorm2 = 8192;
constexpr size_t kTabCodebookH = 9216;
constexpr size_t kTabBinLut = 16384;
constexpr size_t kTabEdges = 17408;
constexpr int kNB = 24;                          // quantile bins per coordinate
constexpr int kCells = kNB * kNB * kNB * kNB;    // 331776
constexpr int kFine = 1024;                      // fine cells of [-4.5, 4.5)
constexpr float kGridLo = -4.5f;
constexpr float kFineW = 9.0f / 1024.0f;         // exact binary fraction
constexpr float kFineInv = 1024.0f / 9.0f;
constexpr size_t kTabMain = 18432;
constexpr size_t kTabBytes = kTabMain + size_t(kCells) * 8;

// Candidate word of a grid cell (little-endian bytes b0..b7):
//  * <= 4 candidates: b0..b3 ascending, padded by repeating the last; b4..b7 = b0..b3
//  * 5..8: b0..b3 = the four lowest, stored descending (b0 > b1 flags "more
//          than four"); b4..b7 the rest ascending, padded by repeating the last
//  * > 8:  as 5..8 for the first eight, but b4..b7 stored descending
//          (b4 > b5 flags "more than eight": the caller scans all codes)
__device__ __forceinline__ bool cand_more_than_4(uint64_t w) {
  return (w & 0xffu) > ((w >> 8) & 0xffu);
}
__device__ __forceinline__ bool cand_more_than_8(uint64_t w) {
  return ((w >> 32) & 0xffu) > ((w >> 40) & 0xffu);
}
// The same tests on the low (b0..b3) and high (b4..b7) 32-bit halves.
__device__ __forceinline__ bool cand_more_than_4_lo(uint32_t lo) {
  return (lo & 0xffu) > ((lo >> 8) & 0xffu);
}
__device__ __forceinline__ bool cand_more_than_8_hi(uint32_t hi) {
  return (hi & 0xffu) > ((hi >> 8) & 0xffu);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) 16-byte load: data read once should not evict
// reused lines from L2/MALL.
__device__ __forceinline__ u32x4 load_nt16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ float h2f(uint16_t b) {
  return __half2float(__ushort_as_half(b));
}
__device__ __forceinline__ uint16_t f2h(float f) {
  // round to nearest even (v_cvt_f16_f32 in the default mode)
  return __half_as_ushort(__float2half_rn(f));
}

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<__half>(__half v) {
  return __half2float(v);
}

// Channel signs of the randomized Hadamard rotation R = H D / sqrt(d)
// (RhtSigns): bit c (word c / 32, bit c % 32) set means channel c is negated
// before H.  All zero for the plain rotation.
typedef RhtSigns Signs;
__device__ __forceinline__ bool any_sign(const Signs& s) {
  return (s.w[0] | s.w[1] | s.w[2] | s.w[3]) != 0u;
}
// Word i of the mask for an index that may differ between lanes (a select,
// never an indexed array: that would go through scratch memory).
__device__ __forceinline__ uint32_t sign_word(const Signs& s, int i) {
  return i == 0 ? s.w[0] : (i == 1 ? s.w[1] : (i == 2 ? s.w[2] : s.w[3]));
}
// 0x80000000 if channel c is negated, else 0.
__device__ __forceinline__ uint32_t sign_bit(const Signs& s, int c) {
  return (sign_word(s, c >> 5) << (31 - (c & 31))) & 0x80000000u;
}
__device__ __forceinline__ float flip_sign(float v, uint32_t bit) {
  return __uint_as_float(__float_as_uint(v) ^ bit);
}

// In-register unnormalized Walsh-Hadamard transform of N values in Sylvester
// (natural) order: v <- H_N v.  Every index is a compile-time constant once
// the loops are unrolled, so the array stays in VGPRs.
template <int N>
__device__ __forceinline__ void fwht_regs(float (&v)[N]) {
#pragma unroll
  for (int h = 1; h < N; h <<= 1) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if ((i & h) == 0) {
        const float a = v[i];
        const float b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
}

// Wave-wide all-reduce on the VALU: DPP within rows of 16 lanes (xor 1,
// xor 2, rotate 4, rotate 8), then gfx950 permlane swaps across the row pairs
// and the two halves.  Every lane ends with the full result.
template <typename Op>
__device__ __forceinline__ float wave_allreduce_dpp(float x, Op op) {
  auto dpp = [](float v, auto ctrl_c) {
    constexpr int ctrl = decltype(ctrl_c)::value;
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xf, 0xf, false));
  };
  x = op(x, dpp(x, std::integral_constant<int, 0xB1>{}));   // quad_perm [1,0,3,2]
  x = op(x, dpp(x, std::integral_constant<int, 0x4E>{}));   // quad_perm [2,3,0,1]
  x = op(x, dpp(x, std::integral_constant<int, 0x124>{}));  // row_ror:4
  x = op(x, dpp(x, std::integral_constant<int, 0x128>{}));  // row_ror:8
  {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  return x;
}
__device__ __forceinline__ float wave_sum_fast(float x) {
  return wave_allreduce_dpp(x, [](float a, float b) { return a + b; });
}
__device__ __forceinline__ float wave_max_fast(float x) {
  return wave_allreduce_dpp(x, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ float wave_min_fast(float x) {
  return wave_allreduce_dpp(x, [](float a, float b) { return fminf(a, b); });
}
// Decoding of a double-quantized group record (4-bit codes, two per byte,
// the low nibble first).  o': (code - 8) * sc, a code of 0 decodes to 0.
// s1: lo + code * (hi - lo) / 15.
__device__ __forceinline__ float dq_nibble_o(uint32_t byte, int high, float sc) {
  const int c = static_cast<int>((byte >> (4 * high)) & 15u);
  return c ? static_cast<float>(c - 8) * sc : 0.f;
}
__device__ __forceinline__ float dq_s1(uint32_t code, float lo, float step) {
  return fmaf(static_cast<float>(code), step, lo);
}
__device__ __forceinline__ float dq_step(float lo, float hi) { return (hi - lo) / 15.0f; }
__device__ __forceinline__ float dq_nibble_s1(uint32_t byte, int high, float lo, float hi) {
  return dq_s1((byte >> (4 * high)) & 15u, lo, dq_step(lo, hi));
}
// x(lane) + x(lane ^ 32) on the VALU (permlane32 swap of x with itself
// yields the lower half in one result and the upper half in the other).
__device__ __forceinline__ float half_pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, kWave));
  return x;
}

}  // namespace nsn
