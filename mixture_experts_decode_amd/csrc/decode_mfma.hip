// Decode gate_up on the matrix cores.
//
// The warp-decode post (sections on how the kernels work and on hardware
// efficiency) computes every output with one wavefront's vector dot products.
// On gfx950 the vector work of that scheme -- E4M3/E2M1 -> BF16 conversion,
// the dot products and a cross-lane reduction per (token, neuron) -- takes
// about as long as streaming the weights, and the two overlap only in part.
// Here the products go to v_mfma_f32_16x16x32_bf16 instead: the weights are
// still converted exactly to BF16 in registers (once per call), but the
// multiply-adds and the K reduction run on the matrix cores, which the
// decode shapes leave idle.  The arithmetic is unchanged: exact BF16 x BF16
// products accumulated in FP32, each output owned by one workgroup, no
// atomics.
//
// Work split.  A workgroup owns 16 neurons of one touched expert (their 16
// gate and 16 up rows of W13) and every token routed to that expert, 16
// tokens (MFMA columns) per pass.  Its KW wavefronts split the H reduction
// into contiguous ranges; each wavefront walks its range in 64-byte stages:
// lane (r, q) = (lane % 16, lane / 16) loads 16 bytes of gate row r and of
// up row r at byte 64*stage + 16*q, so a stage covers 64 bytes of all 32
// rows.  The matching activations of the lane's token column come from x.
// The MFMA pairs K index i of lane group q in the A operand with the same
// index of the same lane group in B, so which K a (lane group, element)
// stands for is free as long as A and B agree; here it is the byte order of
// the row.  The partial 16x16 results of the wavefronts are added in LDS in
// wavefront order, SiLU(g) * u is applied and h is stored.
//
// Scales.  MX scales (powers of two) enter the BF16 conversion as its scale
// operand, which keeps the product exact for scale exponents that leave the
// result in the normal BF16 range; FP8 128x128 tile scales (arbitrary FP32)
// multiply each stage's FP32 partial before it is added, as in the vector
// kernel.

#include <algorithm>

#include "device.h"
#include "internal.h"

namespace moe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kCols = 16;   // tokens per MFMA pass

struct GateUpMfmaArgs {
  const uint8_t* w13;
  const void* w13s;
  const uint16_t* x;      // [T][H] bf16
  const int32_t* ids;
  void* h;                // [T*slots][I] bf16 or f32
  int T, k, slots, E, H, I;
  int row_bytes;          // bytes of one w13 row
  int spw;                // 64-byte stages per wavefront
  int n_blocks;           // 16-neuron blocks per expert
  int n_words;            // 32-bit words of the touched-expert mask
  int n_entries;          // T * slots
  uint32_t slots_magic;
};

__device__ __forceinline__ int div_slots_m(int v, uint32_t magic) {
  return (int)(((unsigned long long)(unsigned)v * magic) >> 32);
}

__device__ __forceinline__ int routed_expert(const GateUpMfmaArgs& a, int v) {
  const int t = div_slots_m(v, a.slots_magic), j = v - t * a.slots;
  if (j >= a.k) return a.E;
  const int e = a.ids[t * a.k + j];
  return (unsigned)e < (unsigned)a.E ? e : 0;
}

__device__ __forceinline__ uint32_t bf16x2_bits(bf16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// 16 weight bytes -> BF16 A operands (two for E4M3, four for E2M1), each
// value multiplied exactly by the power-of-two scale `sc`.
template <int FMT>
__device__ __forceinline__ void chunk_to_a(const u32x4 q, float sc, bf16x8 (&A)[FMT == W_MXFP4 ? 4 : 2]) {
  if constexpr (FMT == W_MXFP4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t b0 = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[j], sc, 0));
      const uint32_t b1 = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[j], sc, 1));
      const uint32_t b2 = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[j], sc, 2));
      const uint32_t b3 = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[j], sc, 3));
      A[j] = __builtin_bit_cast(bf16x8, u32x4{b0, b1, b2, b3});
    }
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t b0 = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[2 * j], sc, false));
      const uint32_t b1 = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[2 * j], sc, true));
      const uint32_t b2 = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[2 * j + 1], sc, false));
      const uint32_t b3 = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[2 * j + 1], sc, true));
      A[j] = __builtin_bit_cast(bf16x8, u32x4{b0, b1, b2, b3});
    }
  }
}

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// KW wavefronts per workgroup; CH stages in flight per wavefront.
template <int FMT, int KW, int CH, bool HBF16>
__global__ __launch_bounds__(64 * KW) __attribute__((amdgpu_waves_per_eu(4)))
void gate_up_mfma_kernel(const GateUpMfmaArgs a) {
  constexpr int NT = 64 * KW;
  constexpr int MAXR = (kDecodeMaxEntries + NT - 1) / NT;
  constexpr int NSTEP = FMT == W_MXFP4 ? 4 : 2;   // MFMA K-steps per 16-byte chunk
  __shared__ uint32_t s_mask[kMaxExpertsTotal / 32];
  __shared__ int s_list[kDecodeMaxEntries];
  __shared__ int s_cnt[MAXR][KW];
  __shared__ f32x4 s_part[KW][2][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_in_block();
  const int r = lane & 15, q = lane >> 4;

  // touched experts of the batch (LDS bitmask), then this workgroup's expert
  for (int i = tid; i < a.n_words; i += NT) s_mask[i] = 0;
  __syncthreads();
  for (int v = tid; v < a.n_entries; v += NT) {
    const int e = routed_expert(a, v);
    atomicOr(&s_mask[e >> 5], 1u << (e & 31));
  }
  __syncthreads();
  const int rank = blockIdx.x / a.n_blocks;
  const int nb = blockIdx.x - rank * a.n_blocks;
  int e = -1;
  {
    int rr = rank;
    for (int i = 0; i < a.n_words; ++i) {
      const uint32_t m = s_mask[i];
      const int c = __popc(m);
      if (rr < c) {
        uint32_t mm = m;
        for (int j = 0; j < rr; ++j) mm &= mm - 1;
        e = i * 32 + __ffs(mm) - 1;
        break;
      }
      rr -= c;
    }
  }
  e = __builtin_amdgcn_readfirstlane(e);
  if (e < 0) return;   // fewer touched experts than the grid assumed (uniform)

  // entries routed to e, in ascending entry order
  const int rounds = (a.n_entries + NT - 1) / NT;
  unsigned long long bal[MAXR];
  bool hit[MAXR];
#pragma unroll
  for (int rd = 0; rd < MAXR; ++rd) {
    const int v = rd * NT + tid;
    hit[rd] = rd < rounds && v < a.n_entries && routed_expert(a, v) == e;
    bal[rd] = __ballot(hit[rd]);
    if (rd < rounds && lane == 0) s_cnt[rd][w] = __popcll(bal[rd]);
  }
  __syncthreads();
  int m = 0;   // entries routed to e
  {
    int base = 0;
#pragma unroll
    for (int rd = 0; rd < MAXR; ++rd) {
      if (rd >= rounds) break;
      int off = base;
      for (int ww = 0; ww < w; ++ww) off += s_cnt[rd][ww];
      if (hit[rd]) {
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal[rd] >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)bal[rd], 0));
        s_list[off + below] = rd * NT + tid;
      }
      for (int ww = 0; ww < KW; ++ww) base += s_cnt[rd][ww];
    }
    m = __builtin_amdgcn_readfirstlane(base);
  }
  __syncthreads();

  const int n0 = nb * 16;
  const long long grow = (long long)e * 2 * a.I + n0;          // first gate row
  const uint8_t* gbase = a.w13 + grow * a.row_bytes;
  const uint8_t* ubase = gbase + (long long)a.I * a.row_bytes;  // first up row
  const int s0 = w * a.spw;                                     // first stage of this wavefront
  const uint32_t wlane = (uint32_t)r * a.row_bytes + 16u * q;   // lane offset inside the row block

  for (int p0 = 0; p0 < m; p0 += kCols) {
    const int col = min(p0 + r, m - 1);        // clamped columns compute, never store
    const int tok = div_slots_m(s_list[col], a.slots_magic);
    const uint16_t* xrow = a.x + (size_t)tok * a.H;
    f32x4 accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};

    for (int c0 = 0; c0 < a.spw; c0 += CH) {
      const int nst = min(CH, a.spw - c0);
      u32x4 xv[CH][NSTEP];
      u32x4 wg[CH], wu[CH];
      float sg[CH], su[CH];
#pragma unroll
      for (int s = 0; s < CH; ++s) {
        if (s < nst) {
          const int st = s0 + c0 + s;
          const int cidx = 4 * st + q;                    // 16-byte chunk of the row
          const int kel = cidx * (FMT == W_MXFP4 ? 32 : 16);
#pragma unroll
          for (int j = 0; j < NSTEP; ++j) xv[s][j] = load16(xrow + kel + 8 * j);
        }
      }
#pragma unroll
      for (int s = 0; s < CH; ++s) {
        if (s < nst) {
          const int st = s0 + c0 + s;
          const uint32_t off = wlane + 64u * st;
          wg[s] = load_stream16(gbase + off);
          wu[s] = load_stream16(ubase + off);
          const int cidx = 4 * st + q;
          if constexpr (FMT == W_MXFP8 || FMT == W_MXFP4) {
            const int srow = a.H >> 5;
            const uint8_t* sc = reinterpret_cast<const uint8_t*>(a.w13s);
            const long long rg = (grow + r) * srow, ru = (grow + a.I + r) * srow;
            const int blk = FMT == W_MXFP8 ? (cidx >> 1) : cidx;
            sg[s] = e8m0_to_f32(sc[rg + blk]);
            su[s] = e8m0_to_f32(sc[ru + blk]);
          } else {
            const int srow = a.H >> 7;
            const float* sc = reinterpret_cast<const float*>(a.w13s);
            const long long tg = ((long long)e * 2 * (a.I >> 7) + (n0 >> 7)) * srow;
            const long long tu = tg + (long long)(a.I >> 7) * srow;
            sg[s] = sc[tg + (st >> 1)];
            su[s] = sc[tu + (st >> 1)];
          }
        }
      }
#pragma unroll
      for (int s = 0; s < CH; ++s) {
        if (s < nst) {
          bf16x8 ag[NSTEP], au[NSTEP];
          if constexpr (FMT == W_FP8B128) {
            chunk_to_a<FMT>(wg[s], 1.0f, ag);
            chunk_to_a<FMT>(wu[s], 1.0f, au);
            f32x4 pg = {0.f, 0.f, 0.f, 0.f}, pu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < NSTEP; ++j) {
              const bf16x8 b = __builtin_bit_cast(bf16x8, xv[s][j]);
              pg = mfma_bf16(ag[j], b, pg);
              pu = mfma_bf16(au[j], b, pu);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              accg[i] = fmaf(pg[i], sg[s], accg[i]);
              accu[i] = fmaf(pu[i], su[s], accu[i]);
            }
          } else {
            chunk_to_a<FMT>(wg[s], sg[s], ag);
            chunk_to_a<FMT>(wu[s], su[s], au);
#pragma unroll
            for (int j = 0; j < NSTEP; ++j) {
              const bf16x8 b = __builtin_bit_cast(bf16x8, xv[s][j]);
              accg = mfma_bf16(ag[j], b, accg);
              accu = mfma_bf16(au[j], b, accu);
            }
          }
        }
      }
    }

    // add the wavefronts' partials in wavefront order; lane (col, q) holds
    // rows 4q..4q+3 of its token column
    s_part[w][0][lane] = accg;
    s_part[w][1][lane] = accu;
    __syncthreads();
    if (w == 0) {
      f32x4 g = s_part[0][0][lane], u = s_part[0][1][lane];
      for (int ww = 1; ww < KW; ++ww) {
        const f32x4 pg = s_part[ww][0][lane], pu = s_part[ww][1][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          g[i] = __fadd_rn(g[i], pg[i]);
          u[i] = __fadd_rn(u[i], pu[i]);
        }
      }
      if (p0 + r < m) {
        const int pe = s_list[p0 + r];
        const size_t off = (size_t)pe * a.I + n0 + 4 * q;
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = swiglu(g[i], u[i]);
        if constexpr (HBF16) {
          const uint32_t lo = f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16);
          const uint32_t hi = f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16);
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.h) + off) = uint2{lo, hi};
        } else {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.h) + off) =
              float4{o[0], o[1], o[2], o[3]};
        }
      }
    }
    __syncthreads();
  }
}

template <int FMT, int KW, bool HBF16>
hipError_t gate_up_mfma_go(const GateUpMfmaArgs& a, int blocks, hipStream_t s) {
  constexpr int CH = FMT == W_MXFP4 ? (KW == 8 ? 1 : 2) : (KW == 8 ? 2 : 4);
  hipLaunchKernelGGL((gate_up_mfma_kernel<FMT, KW, CH, HBF16>), dim3(blocks), dim3(64 * KW), 0, s, a);
  return hipGetLastError();
}

template <int FMT>
hipError_t gate_up_mfma_fmt(const GateUpMfmaArgs& a, int kw, bool hbf, int blocks, hipStream_t s) {
  if (kw == 8) return hbf ? gate_up_mfma_go<FMT, 8, true>(a, blocks, s)
                          : gate_up_mfma_go<FMT, 8, false>(a, blocks, s);
  return hbf ? gate_up_mfma_go<FMT, 4, true>(a, blocks, s)
             : gate_up_mfma_go<FMT, 4, false>(a, blocks, s);
}

}  // namespace

// Shapes this kernel takes: quantised weights, BF16 activations, I a
// multiple of 16, rows a whole number of 64-byte stages that split evenly
// over 4 or 8 wavefronts.  Anything else returns hipErrorNotSupported and
// the caller uses the vector kernel.
hipError_t launch_gate_up_mfma(const moe_weights& W, const void* x, int x_dtype,
                               const int32_t* ids, int T, int k, void* h, int h_dtype,
                               hipStream_t s) {
  if (x_dtype != MOE_DT_BF16) return hipErrorNotSupported;
  if (W.format != W_MXFP8 && W.format != W_MXFP4 && W.format != W_FP8B128)
    return hipErrorNotSupported;
  GateUpMfmaArgs a;
  a.w13 = reinterpret_cast<const uint8_t*>(W.w13);
  a.w13s = W.w13_scale;
  a.x = reinterpret_cast<const uint16_t*>(x);
  a.ids = ids;
  a.h = h;
  a.T = T;
  a.k = k;
  a.slots = k + W.num_shared;
  a.E = W.num_experts;
  a.H = W.hidden;
  a.I = W.inter;
  a.row_bytes = W.format == W_MXFP4 ? W.hidden / 2 : W.hidden;
  if (a.I % 16 || a.row_bytes % 64) return hipErrorNotSupported;
  const int stages = a.row_bytes / 64;
  const int kw_max = env_int("MOE_TUNE_GUM_KW", 8);
  const int kw = stages % 8 == 0 && kw_max >= 8 ? 8 : stages % 4 == 0 ? 4 : 0;
  if (kw == 0) return hipErrorNotSupported;
  a.spw = stages / kw;
  a.n_blocks = a.I / 16;
  const int n_exp = W.num_experts + W.num_shared;
  a.n_words = (n_exp + 31) / 32;
  a.n_entries = T * a.slots;
  if (a.n_entries > kDecodeMaxEntries) return hipErrorNotSupported;
  a.slots_magic = (uint32_t)(((1ull << 32) + a.slots - 1) / a.slots);
  const long long blocks = (long long)std::min(n_exp, a.n_entries) * a.n_blocks;
  if (blocks > 0x7fffffffll) return hipErrorNotSupported;
  const bool hbf = h_dtype == MOE_DT_BF16;
  switch (W.format) {
    case W_MXFP8: return gate_up_mfma_fmt<W_MXFP8>(a, kw, hbf, (int)blocks, s);
    case W_MXFP4: return gate_up_mfma_fmt<W_MXFP4>(a, kw, hbf, (int)blocks, s);
    default: return gate_up_mfma_fmt<W_FP8B128>(a, kw, hbf, (int)blocks, s);
  }
}

}  // namespace moe
