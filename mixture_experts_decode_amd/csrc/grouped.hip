// Expert-centric (grouped) path: gather + MXFP8 activation quantisation,
// grouped gate_up / down GEMMs on gfx950 block-scaled MFMA, ordered combine.

#include "device.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kGqBlock = 256;

// E4M3FN code of a float already divided by its block scale: saturate to
// +-448, round to nearest, ties to even; the sign bit follows the input.
__device__ __forceinline__ uint32_t encode_e4m3(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fminf(fabsf(v), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {                       // below 2^-6: subnormal step 2^-9
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    uint32_t u = __float_as_uint(a);
    u += 0x7ffffu + ((u >> 20) & 1u);        // keep 3 mantissa bits, ties to even
    code = (u >> 20) - ((127u - 7u) << 3);   // rebias the exponent 127 -> 7
  }
  return sign | code;
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

// One wavefront per sorted row; each lane quantises whole 32-element blocks.
template <bool XF32>
__global__ __launch_bounds__(kGqBlock) void gather_quant_kernel(
    const void* __restrict__ x, int H, int slots, int sentinel, const int32_t* __restrict__ sorted,
    const int32_t* __restrict__ npp, int capacity, uint8_t* __restrict__ xq,
    uint8_t* __restrict__ xs) {
  const int lane = threadIdx.x & (kWave - 1);
  const int r = blockIdx.x * (kGqBlock / kWave) + (threadIdx.x >> 6);
  if (r >= capacity || r >= *npp) return;
  const int ent = sorted[r];
  const bool pad = ent < 0 || ent >= sentinel;
  const int t = pad ? 0 : ent / slots;
  const int nblk = H >> 5;
  for (int b = lane; b < nblk; b += kWave) {
    float v[32];
    if (pad) {
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = 0.0f;
    } else if constexpr (XF32) {
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
    for (int i = 0; i < 8; ++i) {
      const uint32_t c0 = encode_e4m3(v[4 * i + 0] * inv);
      const uint32_t c1 = encode_e4m3(v[4 * i + 1] * inv);
      const uint32_t c2 = encode_e4m3(v[4 * i + 2] * inv);
      const uint32_t c3 = encode_e4m3(v[4 * i + 3] * inv);
      out[i >> 2][i & 3] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
    }
    uint8_t* dq = xq + (size_t)r * H + b * 32;
    *reinterpret_cast<u32x4*>(dq) = out[0];
    *reinterpret_cast<u32x4*>(dq + 16) = out[1];
    xs[(size_t)r * nblk + b] = (uint8_t)(e + 127);
  }
}

template <bool YBF16>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ so, int T,
                                                      int slots, int H, void* __restrict__ y) {
  const int h4 = H >> 2;
  const size_t n = (size_t)T * h4;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const size_t t = i / h4;
    const size_t c = i - t * h4;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < slots; ++j) {
      const float4 v = reinterpret_cast<const float4*>(so + ((t * slots + j) * H))[c];
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    if constexpr (YBF16) {
      uint2 o;
      o.x = f32_to_bf16_bits(acc.x) | (f32_to_bf16_bits(acc.y) << 16);
      o.y = f32_to_bf16_bits(acc.z) | (f32_to_bf16_bits(acc.w) << 16);
      reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + t * H)[c] = o;
    } else {
      reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + t * H)[c] = acc;
    }
  }
}

}  // namespace

hipError_t launch_gather_quant(const void* x, int x_dtype, int T, int H, int slots,
                               const int32_t* sorted, const int32_t* npp, int capacity,
                               uint8_t* xq, uint8_t* xs, hipStream_t s) {
  const int rows_per_block = kGqBlock / kWave;
  const int blocks = (capacity + rows_per_block - 1) / rows_per_block;
  const int sentinel = T * slots;
  if (x_dtype == MOE_DT_F32)
    hipLaunchKernelGGL(gather_quant_kernel<true>, dim3(blocks), dim3(kGqBlock), 0, s, x, H, slots,
                       sentinel, sorted, npp, capacity, xq, xs);
  else
    hipLaunchKernelGGL(gather_quant_kernel<false>, dim3(blocks), dim3(kGqBlock), 0, s, x, H,
                       slots, sentinel, sorted, npp, capacity, xq, xs);
  return hipGetLastError();
}

hipError_t launch_combine(const float* slot_out, int T, int slots, int H, void* y, int y_dtype,
                          hipStream_t s) {
  if (H % 4) return hipErrorNotSupported;
  const size_t n = (size_t)T * (H / 4);
  const int blocks = (int)std::min<size_t>((n + 255) / 256, (size_t)device_num_cus() * 16);
  if (y_dtype == MOE_DT_BF16)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(blocks), dim3(256), 0, s, slot_out, T, slots, H, y);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(blocks), dim3(256), 0, s, slot_out, T, slots, H, y);
  return hipGetLastError();
}

hipError_t launch_grouped_gate_up(const moe_weights&, const uint8_t*, const uint8_t*,
                                  const int32_t*, const int32_t*, int, int, uint8_t*, uint8_t*,
                                  hipStream_t) {
  return hipErrorNotSupported;
}

hipError_t launch_grouped_down(const moe_weights&, const uint8_t*, const uint8_t*, const int32_t*,
                               const int32_t*, const int32_t*, int, int, const float*, int, int,
                               float*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace moe
