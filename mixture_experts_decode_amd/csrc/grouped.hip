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

__device__ __forceinline__ float pow2(int e) { return pow2_neg(-e); }

// E4M3FN code -> float (finite codes): e == 0 subnormal m * 2^-9.
__device__ __forceinline__ float decode_e4m3(uint32_t c) {
  const uint32_t sign = (c & 0x80u) << 24;
  const uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return __uint_as_float(__float_as_uint(mag) | sign);
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

// ---------------------------------------------------------------------------
// grouped GEMMs on v_mfma_scale_f32_32x32x64_f8f6f4
// ---------------------------------------------------------------------------

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kGemmBlock = 256;          // 4 wavefronts
constexpr int kKStep = 64;               // K per MFMA
constexpr int kARowPitch = 80;           // LDS bytes per staged A row (64 + pad)

struct GemmArgs {
  const uint8_t* a;        // activations [cap][K] E4M3 (the hi term for down)
  const uint8_t* as;       // [cap][K/32] E8M0
  const uint8_t* a_lo;     // down: lo term of h [cap][K]
  const uint8_t* as_lo;    // down: [cap][K/32]
  const uint8_t* b;        // expert weights, rows of K (E4M3 or packed E2M1)
  const void* bs;          // weight scales (E8M0 bytes or float tiles)
  const int32_t* expert_ids;
  const int32_t* npp;
  const int32_t* sorted;   // down: entry of each sorted row
  const float* wts;        // down: routing weights
  uint8_t* hq;             // gate_up out [2][cap][I]: hi term, then lo term
  uint8_t* hs;             // gate_up out [2][cap][I/32]
  int cap;
  float* out;              // down out: slot_out [T*slots][H]
  int K, N;                // reduction length, output columns (neurons or H)
  int I, H;
  int b_row_bytes;
  int rows_per_expert;     // 2I (gate_up) or H (down)
  int n_ntiles;            // workgroup tiles along N
  int k, slots, sentinel;
  int nxcd;
};

// Max over the 32 lanes of each half wave.
__device__ __forceinline__ float half32_max(float x) {
  x = fmaxf(x, dpp_f32<0x128>(x));
  x = fmaxf(x, dpp_f32<0x124>(x));
  x = fmaxf(x, dpp_f32<0x122>(x));
  x = fmaxf(x, dpp_f32<0x121>(x));
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// B fragment of one K step for the weight row of this lane.  8-bit elements:
// bytes [16h, 16h+16) and [32+16h, 32+16h+16) of the step (the gfx950 lane
// layout of 8-bit MFMA operands); E2M1: 16 bytes holding K [32h, 32h+32).
template <int BFMT>
__device__ __forceinline__ i32x8 load_b_frag(const uint8_t* row, int step, int h) {
  i32x8 v;
  if constexpr (BFMT == W_MXFP4) {
    const u32x4 q = load_stream16(row + step * (kKStep / 2) + 16 * h);
    v = i32x8{(int)q[0], (int)q[1], (int)q[2], (int)q[3], 0, 0, 0, 0};
  } else {
    const u32x4 q0 = load_stream16(row + step * kKStep + 16 * h);
    const u32x4 q1 = load_stream16(row + step * kKStep + 32 + 16 * h);
    v = i32x8{(int)q0[0], (int)q0[1], (int)q0[2], (int)q0[3],
              (int)q1[0], (int)q1[1], (int)q1[2], (int)q1[3]};
  }
  return v;
}

template <int BFMT, bool GATEUP, int MF, int NF>
__global__ __launch_bounds__(kGemmBlock) void grouped_gemm_kernel(const GemmArgs g) {
  constexpr int BS = MF * 32;
  constexpr bool kTile128 = BFMT == W_FP8B128;   // float 128x128 weight scales
  constexpr int TERMS = GATEUP ? 1 : 2;          // down reads h as hi + lo
  __shared__ __attribute__((aligned(16))) uint8_t s_a[2][TERMS][BS * kARowPitch];
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x >> 6;
  const int r32 = lane & 31, h = lane >> 5;

  const int lb = xcd_logical_block(blockIdx.x, gridDim.x, g.nxcd);
  const int mb = lb / g.n_ntiles;
  const int nt = lb - mb * g.n_ntiles;
  if (mb * BS >= *g.npp) return;
  const int e = g.expert_ids[mb];
  const int row0 = mb * BS;
  const int nsteps = g.K / kKStep;

  // this wavefront's NF fragments of 32 weight rows
  int col[NF];           // output column (neuron or H index) of the lane's row
  const uint8_t* brow[NF];
  long long bidx[NF];    // global weight row index
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    int c, proj = 0;
    if constexpr (GATEUP) {
      const int nb = nt * (4 * (NF / 2) * 32) + w * ((NF / 2) * 32);
      proj = f < NF / 2 ? 0 : 1;
      c = nb + 32 * (f % (NF / 2)) + r32;
    } else {
      c = nt * (4 * NF * 32) + w * (NF * 32) + 32 * f + r32;
    }
    col[f] = c;
    const int cc = min(c, g.N - 1);
    bidx[f] = (long long)e * g.rows_per_expert + (long long)proj * g.I + cc;
    brow[f] = g.b + bidx[f] * g.b_row_bytes;
  }
  const int k_blocks = g.K >> 5;
  const int k_tiles = g.K >> 7;

  f32x16 acc[MF][NF];
#pragma unroll
  for (int m = 0; m < MF; ++m)
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[m][f] = f32x16{0};
  f32x16 part[kTile128 ? MF : 1][kTile128 ? NF : 1];
  if constexpr (kTile128) {
#pragma unroll
    for (int m = 0; m < MF; ++m)
#pragma unroll
      for (int f = 0; f < NF; ++f) part[m][f] = f32x16{0};
  }

  // ---- staging of the activation tile(s) (BS rows x 64 bytes per step)
  constexpr int kAChunks = BS * 4;                       // 16-byte chunks per step
  constexpr int kAPerThread = (kAChunks + kGemmBlock - 1) / kGemmBlock;
  u32x4 a_stage[TERMS][kAPerThread];
  auto load_a = [&](int step) {
#pragma unroll
    for (int tm = 0; tm < TERMS; ++tm) {
      const uint8_t* src = tm == 0 ? g.a : g.a_lo;
#pragma unroll
      for (int i = 0; i < kAPerThread; ++i) {
        const int c = threadIdx.x + i * kGemmBlock;
        if (c < kAChunks) {
          const int r = c >> 2, sg = c & 3;
          a_stage[tm][i] = load16(src + (size_t)(row0 + r) * g.K + step * kKStep + sg * 16);
        }
      }
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int tm = 0; tm < TERMS; ++tm) {
#pragma unroll
      for (int i = 0; i < kAPerThread; ++i) {
        const int c = threadIdx.x + i * kGemmBlock;
        if (c < kAChunks) {
          const int r = c >> 2, sg = c & 3;
          *reinterpret_cast<u32x4*>(&s_a[buf][tm][r * kARowPitch + sg * 16]) = a_stage[tm][i];
        }
      }
    }
  };
  auto load_scales = [&](int step, int (&sa)[TERMS][MF], int (&sb)[NF]) {
#pragma unroll
    for (int tm = 0; tm < TERMS; ++tm) {
      const uint8_t* src = tm == 0 ? g.as : g.as_lo;
#pragma unroll
      for (int m = 0; m < MF; ++m)
        sa[tm][m] = src[(size_t)(row0 + m * 32 + r32) * k_blocks + 2 * step + h];
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      if constexpr (kTile128) {
        sb[f] = 127;
      } else {
        sb[f] = reinterpret_cast<const uint8_t*>(g.bs)[bidx[f] * k_blocks + 2 * step + h];
      }
    }
  };

  i32x8 bcur[NF], bnxt[NF];
  int sa_cur[TERMS][MF], sb_cur[NF], sa_nxt[TERMS][MF], sb_nxt[NF];
  load_a(0);
#pragma unroll
  for (int f = 0; f < NF; ++f) bcur[f] = load_b_frag<BFMT>(brow[f], 0, h);
  load_scales(0, sa_cur, sb_cur);
  store_a(0);
  __syncthreads();

  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    const bool more = s + 1 < nsteps;
    if (more) {
      load_a(s + 1);
#pragma unroll
      for (int f = 0; f < NF; ++f) bnxt[f] = load_b_frag<BFMT>(brow[f], s + 1, h);
      load_scales(s + 1, sa_nxt, sb_nxt);
    }
#pragma unroll
    for (int m = 0; m < MF; ++m) {
#pragma unroll
      for (int tm = 0; tm < TERMS; ++tm) {
        const uint8_t* ap = &s_a[buf][tm][(m * 32 + r32) * kARowPitch];
        const u32x4 q0 = *reinterpret_cast<const u32x4*>(ap + 16 * h);
        const u32x4 q1 = *reinterpret_cast<const u32x4*>(ap + 32 + 16 * h);
        const i32x8 afrag = {(int)q0[0], (int)q0[1], (int)q0[2], (int)q0[3],
                             (int)q1[0], (int)q1[1], (int)q1[2], (int)q1[3]};
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          if constexpr (kTile128) {
            part[m][f] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                afrag, bcur[f], part[m][f], 0, 0, 0, sa_cur[tm][m], 0, sb_cur[f]);
          } else {
            acc[m][f] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                afrag, bcur[f], acc[m][f], 0, BFMT == W_MXFP4 ? 4 : 0, 0, sa_cur[tm][m], 0,
                sb_cur[f]);
          }
        }
      }
    }
    if constexpr (kTile128) {
      if (s & 1) {   // a 128-wide K tile is complete: promote with its scale
        const float* ts = reinterpret_cast<const float*>(g.bs);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const float sc = ts[(bidx[f] >> 7) * k_tiles + (s >> 1)];
#pragma unroll
          for (int m = 0; m < MF; ++m) {
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[m][f][q] = fmaf(part[m][f][q], sc, acc[m][f][q]);
            part[m][f] = f32x16{0};
          }
        }
      }
    }
    if (more) {
      store_a(buf ^ 1);
#pragma unroll
      for (int f = 0; f < NF; ++f) bcur[f] = bnxt[f];
#pragma unroll
      for (int tm = 0; tm < TERMS; ++tm)
#pragma unroll
        for (int m = 0; m < MF; ++m) sa_cur[tm][m] = sa_nxt[tm][m];
#pragma unroll
      for (int f = 0; f < NF; ++f) sb_cur[f] = sb_nxt[f];
    }
    __syncthreads();
  }

  // ---- epilogue.  Accumulator element q of a 32x32 tile sits at row
  // 8*(q/4) + 4*h + q%4 and column r32 of the tile.
  if constexpr (GATEUP) {
#pragma unroll
    for (int m = 0; m < MF; ++m) {
#pragma unroll
      for (int f = 0; f < NF / 2; ++f) {
        const int n = col[f];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int row = row0 + m * 32 + 8 * (q >> 2) + 4 * h + (q & 3);
          const float hv = swiglu(acc[m][f][q], acc[m][f + NF / 2][q]);
          // hi = Q(h) per 32 neurons (the 32 lanes of this half wave), then
          // lo = Q(h - hi): the residual is exact in FP32
          const float amax = half32_max(n < g.N ? fabsf(hv) : 0.0f);
          const int e1 = mx_exponent(amax);
          const uint32_t c1 = encode_e4m3(hv * pow2_neg(e1));
          const float res = hv - decode_e4m3(c1) * pow2(e1);
          const float rmax = half32_max(n < g.N ? fabsf(res) : 0.0f);
          const int e2 = mx_exponent(rmax);
          const uint32_t c2 = encode_e4m3(res * pow2_neg(e2));
          if (n < g.N) {
            const size_t o = (size_t)row * g.I + n;
            const size_t os = (size_t)row * (g.I >> 5) + (n >> 5);
            g.hq[o] = (uint8_t)c1;
            g.hq[(size_t)g.cap * g.I + o] = (uint8_t)c2;
            if (r32 == 0) {
              g.hs[os] = (uint8_t)(e1 + 127);
              g.hs[(size_t)g.cap * (g.I >> 5) + os] = (uint8_t)(e2 + 127);
            }
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int m = 0; m < MF; ++m) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = row0 + m * 32 + 8 * (q >> 2) + 4 * h + (q & 3);
        const int ent = g.sorted[row];
        if (ent < 0 || ent >= g.sentinel) continue;
        const int t = ent / g.slots, j = ent - t * g.slots;
        const float wgt = j < g.k ? g.wts[t * g.k + j] : 1.0f;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          if (col[f] < g.N) g.out[(size_t)ent * g.H + col[f]] = __fmul_rn(acc[m][f][q], wgt);
        }
      }
    }
  }
}

template <int BFMT, bool GATEUP>
hipError_t gemm_dispatch(const GemmArgs& a, int bs, int capacity, hipStream_t s) {
  const int n_mblocks = capacity / bs;
  if (n_mblocks == 0) return hipSuccess;
  const dim3 grid(n_mblocks * a.n_ntiles), block(kGemmBlock);
#define MOE_GG(MF, NF) hipLaunchKernelGGL((grouped_gemm_kernel<BFMT, GATEUP, MF, NF>), grid, block, 0, s, a)
  if constexpr (BFMT == W_FP8B128) {
    if (bs == 32) MOE_GG(1, 4);
    else if (bs == 64) MOE_GG(2, 2);
    else if (!GATEUP) MOE_GG(4, 1);
    else return hipErrorNotSupported;
  } else {
    if (bs == 32) MOE_GG(1, 8);
    else if (bs == 64) MOE_GG(2, 4);
    else MOE_GG(4, 2);
  }
#undef MOE_GG
  return hipGetLastError();
}

// fragments per wavefront for a block size (as dispatched above)
int gemm_nf(int fmt, int bs) {
  if (fmt == W_FP8B128) return bs == 32 ? 4 : bs == 64 ? 2 : 1;
  return bs == 32 ? 8 : bs == 64 ? 4 : 2;
}

}  // namespace

hipError_t launch_grouped_gate_up(const moe_weights& W, const uint8_t* xq, const uint8_t* xs,
                                  const int32_t* expert_ids, const int32_t* npp, int capacity,
                                  int bs, uint8_t* hq, uint8_t* hs, hipStream_t s) {
  GemmArgs a{};
  a.a = xq;
  a.as = xs;
  a.b = reinterpret_cast<const uint8_t*>(W.w13);
  a.bs = W.w13_scale;
  a.expert_ids = expert_ids;
  a.npp = npp;
  a.hq = hq;
  a.hs = hs;
  a.cap = capacity;
  a.K = W.hidden;
  a.N = W.inter;
  a.I = W.inter;
  a.H = W.hidden;
  a.b_row_bytes = W.format == W_MXFP4 ? W.hidden / 2 : W.hidden;
  a.rows_per_expert = 2 * W.inter;
  const int nf = gemm_nf(W.format, bs);
  const int per_wg = 4 * (nf / 2) * 32;                   // neurons per workgroup
  if (nf < 2) return hipErrorNotSupported;
  a.n_ntiles = (W.inter + per_wg - 1) / per_wg;
  a.nxcd = device_num_xcds();
  switch (W.format) {
    case W_MXFP8: return gemm_dispatch<W_MXFP8, true>(a, bs, capacity, s);
    case W_MXFP4: return gemm_dispatch<W_MXFP4, true>(a, bs, capacity, s);
    case W_FP8B128: return gemm_dispatch<W_FP8B128, true>(a, bs, capacity, s);
    default: return hipErrorNotSupported;
  }
}

hipError_t launch_grouped_down(const moe_weights& W, const uint8_t* hq, const uint8_t* hs,
                               const int32_t* sorted, const int32_t* expert_ids,
                               const int32_t* npp, int capacity, int bs, const float* wts, int T,
                               int k, float* slot_out, hipStream_t s) {
  GemmArgs a{};
  a.a = hq;
  a.as = hs;
  a.a_lo = hq + (size_t)capacity * W.inter;
  a.as_lo = hs + (size_t)capacity * (W.inter / 32);
  a.cap = capacity;
  a.b = reinterpret_cast<const uint8_t*>(W.w2);
  a.bs = W.w2_scale;
  a.expert_ids = expert_ids;
  a.npp = npp;
  a.sorted = sorted;
  a.wts = wts;
  a.out = slot_out;
  a.K = W.inter;
  a.N = W.hidden;
  a.I = W.inter;
  a.H = W.hidden;
  a.b_row_bytes = W.format == W_MXFP4 ? W.inter / 2 : W.inter;
  a.rows_per_expert = W.hidden;
  const int nf = gemm_nf(W.format, bs);
  const int per_wg = 4 * nf * 32;
  a.n_ntiles = (W.hidden + per_wg - 1) / per_wg;
  a.k = k;
  a.slots = k + W.num_shared;
  a.sentinel = T * a.slots;
  a.nxcd = device_num_xcds();
  switch (W.format) {
    case W_MXFP8: return gemm_dispatch<W_MXFP8, false>(a, bs, capacity, s);
    case W_MXFP4: return gemm_dispatch<W_MXFP4, false>(a, bs, capacity, s);
    case W_FP8B128: return gemm_dispatch<W_FP8B128, false>(a, bs, capacity, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace moe
