// MXFP8 quantisation of activation rows (E4M3 codes + one E8M0 exponent per
// 32 consecutive elements), shared by the grouped path's quantiser, the
// grouped gate_up epilogue and the fused front end of the layer.
#pragma once

#include "device.h"

namespace moe {
namespace {

typedef short s16x2 __attribute__((ext_vector_type(2)));

// Four floats, already divided by their block scale, -> four E4M3FN codes in
// one dword (byte i = element i).  They are saturated to +-448 first (the
// conversion itself gives NaN past the top of the format); the gfx950
// conversion then rounds to nearest, ties to even, and keeps the sign of
// values that round to zero.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  s16x2 r = {0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f),
                                                __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f), 1.0f, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f),
                                                __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f), 1.0f, true);
  uint32_t u;
  __builtin_memcpy(&u, &r, 4);
  return u;
}

// Shared MX exponent of a block with maximum magnitude amax:
// floor(log2 amax) - 8, clamped to [-127, 127]; -127 for amax == 0.
__device__ __forceinline__ int mx_exponent(float amax) {
  const uint32_t u = __float_as_uint(amax);
  const int ef = (int)(u >> 23);
  int l2;
  if (amax == 0.0f) return -127;
  if (ef == 0) {
    l2 = (31 - __clz(u & 0x7fffffu)) - 149;  // subnormal amax
  } else {
    l2 = ef - 127;
  }
  return max(-127, min(127, l2 - 8));
}

// 2^-e for e in [-127, 127] as a float (exact: 2^127 .. 2^-127).
__device__ __forceinline__ float pow2_neg(int e) {
  const int p = -e;
  if (p >= -126) return __uint_as_float((uint32_t)(p + 127) << 23);
  return __uint_as_float(0x00400000u >> (-126 - p - 1));   // p == -127 only
}

__device__ __forceinline__ float pow2(int e) { return pow2_neg(-e); }

// Quantises token row t of x [T][H] (FP32 or BF16) into xq [T][H] and xs
// [T][H/32]; one wavefront, each lane taking whole 32-element blocks.
template <bool XF32>
__device__ __forceinline__ void quant_row(const void* __restrict__ x, int t, int H,
                                          uint8_t* __restrict__ xq, uint8_t* __restrict__ xs,
                                          int lane) {
  const int nblk = H >> 5;
  for (int b = lane; b < nblk; b += kWave) {
    float v[32];
    if constexpr (XF32) {
      const float* p = reinterpret_cast<const float*>(x) + (size_t)t * H + b * 32;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        u32x4 q = load16(p + 4 * i);
        v[4 * i + 0] = __uint_as_float(q[0]);
        v[4 * i + 1] = __uint_as_float(q[1]);
        v[4 * i + 2] = __uint_as_float(q[2]);
        v[4 * i + 3] = __uint_as_float(q[3]);
      }
    } else {
      const uint16_t* p = reinterpret_cast<const uint16_t*>(x) + (size_t)t * H + b * 32;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x4 q = load16(p + 8 * i);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          v[8 * i + 2 * w] = bf16_lo(q[w]);
          v[8 * i + 2 * w + 1] = bf16_hi(q[w]);
        }
      }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const int e = mx_exponent(amax);
    const float inv = pow2_neg(e);
    u32x4 out[2];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      out[i >> 2][i & 3] = e4m3x4(v[4 * i] * inv, v[4 * i + 1] * inv, v[4 * i + 2] * inv,
                                  v[4 * i + 3] * inv);
    uint8_t* dq = xq + (size_t)t * H + b * 32;
    *reinterpret_cast<u32x4*>(dq) = out[0];
    *reinterpret_cast<u32x4*>(dq + 16) = out[1];
    xs[(size_t)t * nblk + b] = (uint8_t)(e + 127);
  }
}

}  // namespace
}  // namespace moe
