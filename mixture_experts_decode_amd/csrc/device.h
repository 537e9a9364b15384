// Device-side helpers shared by the HIP kernels of this library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum WFormat { W_F32 = 0, W_MXFP8 = 1, W_MXFP4 = 2, W_FP8B128 = 3 };

constexpr int kWave = 64;

// Index of the calling wavefront inside its workgroup, as a scalar: the
// compiler cannot prove threadIdx.x / 64 uniform by itself and would keep
// everything derived from it (row addresses, 64-bit multiplies) per lane.
__device__ __forceinline__ int wave_in_block() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// ---------------------------------------------------------------------------
// loads
// ---------------------------------------------------------------------------

// 16-byte load that bypasses reuse-oriented cache allocation: for data each
// call reads exactly once (expert weight rows in the expert-major kernels).
__device__ __forceinline__ u32x4 load_stream16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Empty register barrier: the compiler must assume v changed here.  Used on
// weight registers inside per-token loops so the format conversion is redone
// per token (a few VALU ops) instead of being hoisted into 2-4x more registers.
__device__ __forceinline__ void opaque(u32x4& v) {
  uint32_t a = v[0], b = v[1], c = v[2], d = v[3];
  asm volatile("" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
  v = u32x4{a, b, c, d};
}

// ---------------------------------------------------------------------------
// number formats
// ---------------------------------------------------------------------------

// E8M0 scale byte -> float 2^(b-127); b = 0 is the subnormal 2^-127, b = 255 NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  uint32_t bits = b ? (b << 23) : 0x00400000u;
  bits = (b == 255u) ? 0x7fc00000u : bits;
  return __uint_as_float(bits);
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two E4M3 bytes (low or high half-word of v) -> two exact bf16 values.
template <bool HI>
__device__ __forceinline__ bf16x2 fp8x2_to_bf16x2(uint32_t v) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, HI);
}

// Two E2M1 nibbles (byte `sel` of v) -> two exact bf16 values.
template <int SEL>
__device__ __forceinline__ bf16x2 fp4x2_to_bf16x2(uint32_t v) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, SEL);
}

// Two E4M3 bytes -> two exact floats.
template <bool HI>
__device__ __forceinline__ f32x2 fp8x2_to_f32x2(uint32_t v) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v, 1.0f, HI);
}

template <int SEL>
__device__ __forceinline__ f32x2 fp4x2_to_f32x2(uint32_t v) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, SEL);
}

__device__ __forceinline__ float dot2_bf16(bf16x2 a, bf16x2 b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}

// ---------------------------------------------------------------------------
// 16-byte weight chunk . activation chunk, FP32 accumulation
// ---------------------------------------------------------------------------
// Elements per 16-byte weight chunk: 16 (E4M3), 32 (E2M1), 4 (F32).
template <int FMT> struct Chunk;
template <> struct Chunk<W_MXFP8> { static constexpr int kElems = 16; };
template <> struct Chunk<W_FP8B128> { static constexpr int kElems = 16; };
template <> struct Chunk<W_MXFP4> { static constexpr int kElems = 32; };
template <> struct Chunk<W_F32> { static constexpr int kElems = 4; };

// Weight chunk w against bf16 activations xs (kElems/2 dwords, element 2i in
// the low half of dword i).  Returns the unscaled partial dot product.
template <int FMT>
__device__ __forceinline__ float chunk_dot_bf16(const u32x4 w, const uint32_t* xs) {
  float acc = 0.f;
  if constexpr (FMT == W_MXFP8 || FMT == W_FP8B128) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      acc = dot2_bf16(fp8x2_to_bf16x2<false>(w[d]), as_bf16x2(xs[2 * d]), acc);
      acc = dot2_bf16(fp8x2_to_bf16x2<true>(w[d]), as_bf16x2(xs[2 * d + 1]), acc);
    }
  } else if constexpr (FMT == W_MXFP4) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      acc = dot2_bf16(fp4x2_to_bf16x2<0>(w[d]), as_bf16x2(xs[4 * d + 0]), acc);
      acc = dot2_bf16(fp4x2_to_bf16x2<1>(w[d]), as_bf16x2(xs[4 * d + 1]), acc);
      acc = dot2_bf16(fp4x2_to_bf16x2<2>(w[d]), as_bf16x2(xs[4 * d + 2]), acc);
      acc = dot2_bf16(fp4x2_to_bf16x2<3>(w[d]), as_bf16x2(xs[4 * d + 3]), acc);
    }
  } else {  // F32 weights, bf16 activations
    acc = fmaf(__uint_as_float(w[0]), bf16_lo(xs[0]), acc);
    acc = fmaf(__uint_as_float(w[1]), bf16_hi(xs[0]), acc);
    acc = fmaf(__uint_as_float(w[2]), bf16_lo(xs[1]), acc);
    acc = fmaf(__uint_as_float(w[3]), bf16_hi(xs[1]), acc);
  }
  return acc;
}

// Weight chunk w against float activations xs (kElems floats).
template <int FMT>
__device__ __forceinline__ float chunk_dot_f32(const u32x4 w, const float* xs) {
  float acc = 0.f;
  if constexpr (FMT == W_MXFP8 || FMT == W_FP8B128) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      f32x2 a = fp8x2_to_f32x2<false>(w[d]);
      f32x2 b = fp8x2_to_f32x2<true>(w[d]);
      acc = fmaf(a.x, xs[4 * d + 0], acc);
      acc = fmaf(a.y, xs[4 * d + 1], acc);
      acc = fmaf(b.x, xs[4 * d + 2], acc);
      acc = fmaf(b.y, xs[4 * d + 3], acc);
    }
  } else if constexpr (FMT == W_MXFP4) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      f32x2 a = fp4x2_to_f32x2<0>(w[d]);
      f32x2 b = fp4x2_to_f32x2<1>(w[d]);
      f32x2 c = fp4x2_to_f32x2<2>(w[d]);
      f32x2 e = fp4x2_to_f32x2<3>(w[d]);
      acc = fmaf(a.x, xs[8 * d + 0], acc);
      acc = fmaf(a.y, xs[8 * d + 1], acc);
      acc = fmaf(b.x, xs[8 * d + 2], acc);
      acc = fmaf(b.y, xs[8 * d + 3], acc);
      acc = fmaf(c.x, xs[8 * d + 4], acc);
      acc = fmaf(c.y, xs[8 * d + 5], acc);
      acc = fmaf(e.x, xs[8 * d + 6], acc);
      acc = fmaf(e.y, xs[8 * d + 7], acc);
    }
  } else {
    acc = fmaf(__uint_as_float(w[0]), xs[0], acc);
    acc = fmaf(__uint_as_float(w[1]), xs[1], acc);
    acc = fmaf(__uint_as_float(w[2]), xs[2], acc);
    acc = fmaf(__uint_as_float(w[3]), xs[3], acc);
  }
  return acc;
}

// ---------------------------------------------------------------------------
// wave64 sum: rotations inside each 16-lane row (DPP), then the gfx950 row
// swaps across rows (permlane16/32 swap).  Fixed order; every lane ends with
// the same total.  No LDS, no barrier.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over the 16 lanes of each DPP row; every lane of the row gets it.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f32<0x128>(x);  // row_ror:8
  x += dpp_f32<0x124>(x);  // row_ror:4
  x += dpp_f32<0x122>(x);  // row_ror:2
  x += dpp_f32<0x121>(x);  // row_ror:1
  return x;
}

// Maximum over the whole wave (unsigned), every lane gets it: DPP row
// rotations, then the row swaps across rows, as wave_sum.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf, false);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, dpp_u32<0x128>(x));
  x = max(x, dpp_u32<0x124>(x));
  x = max(x, dpp_u32<0x122>(x));
  x = max(x, dpp_u32<0x121>(x));
  auto r16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = max((uint32_t)r16[0], (uint32_t)r16[1]);
  auto r32 = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return max((uint32_t)r32[0], (uint32_t)r32[1]);
}

// Sum over each half wave (two DPP rows); every lane of the half gets it.
__device__ __forceinline__ float half32_sum(float x) {
  x = row16_sum(x);
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over each aligned group of 8 lanes (half a DPP row).
__device__ __forceinline__ float group8_sum(float x) {
  x += dpp_f32<0x141>(x);  // row_half_mirror: lane i <- 7 - i within the half row
  x += dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2]
  return x;
}

// Sum over each aligned group of 4 lanes (a DPP quad).
__device__ __forceinline__ float group4_sum(float x) {
  x += dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2]
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
  x = row16_sum(x);
  uint32_t u = __float_as_uint(x);
  auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
  u = __float_as_uint(x);
  auto r32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

// Four wave sums at once: on return DPP row 0 holds sum(a), row 1 sum(b),
// row 2 sum(c), row 3 sum(d) (every lane of the row).  The halves are folded
// with permlane32 swaps (a with c, b with d), the row pairs with a
// permlane16 swap, then each row is finished with DPP rotations.
__device__ __forceinline__ float wave_sum4_rows(float a, float b, float c, float d) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(c), false, false);
  const float u = __uint_as_float(p[0]) + __uint_as_float(p[1]);   // lo: a, hi: c
  auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(b), __float_as_uint(d), false, false);
  const float v = __uint_as_float(q[0]) + __uint_as_float(q[1]);   // lo: b, hi: d
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(u), __float_as_uint(v), false, false);
  return row16_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

// Two wave sums at once: rows 0-1 hold sum(a), rows 2-3 sum(b).
__device__ __forceinline__ float wave_sum2_halves(float a, float b) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  const float u = __uint_as_float(p[0]) + __uint_as_float(p[1]);   // lo: a, hi: b
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(u), __float_as_uint(u), false, false);
  return row16_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

__device__ __forceinline__ float lane_value(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// SiLU(g) * u in FP32: g * sigmoid(g) with the hardware reciprocal (about
// one ulp) instead of an IEEE division, which costs a dozen instructions per
// output.  As g -> -inf, 1 + e^-g -> inf and the reciprocal -> 0, so the
// product goes to (signed) zero as SiLU does.
__device__ __forceinline__ float swiglu(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// ---------------------------------------------------------------------------
// XCD-aware block order.  Workgroups are dispatched round-robin over the
// XCDs (block b runs on XCD b % nxcd).  The returned logical index makes
// consecutive logical blocks share an XCD (and therefore its L2), so blocks
// that reuse the same rows sit on one L2 (align-and-sort article, Triton
// section: pid remapping on XCDs).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int xcd_logical_block(int b, int nblocks, int nxcd) {
  int per = nblocks / nxcd;            // full rounds
  int full = per * nxcd;
  if (b >= full) return b;             // ragged tail keeps its order
  return (b % nxcd) * per + b / nxcd;
}

}  // namespace moe
