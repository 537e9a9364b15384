// Output-centric decode kernels: gate_up and down.
//
// Both follow the warp-decode post (sections on how the two kernels work and
// on warp independence): every output scalar is owned by exactly one 64-lane
// wavefront, which streams the expert weight rows it needs, converts the
// stored format to FP32/BF16 in registers, keeps FP32 accumulators and finishes
// with a wave reduction; nothing is staged between kernels except h itself.
//
// gfx950-specific choices (not on the pages):
//  * gate_up is expert-major: a wavefront owns NR neurons (gate + up rows) of
//    one touched expert and produces them for every (token, slot) routed to
//    that expert in the batch, so each weight row is read from HBM once per
//    call even when several tokens share an expert.  Each workgroup finds the
//    touched experts itself from the routed ids (an LDS bitmask), so no
//    pre-pass kernel and no host sync are needed; waves loop over
//    (expert rank, neuron group) items with a static stride.
//  * down is token-major as on the page, with the (slot, K-chunk) pairs of a
//    token flattened across the 64 lanes, and workgroups of one output group
//    ordered onto one XCD so tokens sharing an expert hit that XCD's L2.
//  * 16-byte loads per lane; E4M3 / E2M1 are converted to exact BF16 and
//    multiplied with BF16 activations by v_dot2_f32_bf16 (FP32 accumulate); the
//    MX / tile scale multiplies each 16-byte chunk's partial sum.

#include "device.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kMaskWords = kMaxExpertsTotal / 32;

struct GateUpArgs {
  const uint8_t* w13;
  const void* w13s;
  const void* x;
  const int32_t* ids;
  void* h;
  int T, k, slots, E, H, I;
  int row_bytes;    // bytes of one w13 row
  int chunks;       // 16-byte chunks per row
  int n_groups;     // neuron groups per expert
  int n_words;      // 32-bit words of the touched-expert mask
  int n_entries;    // T * slots
};

struct DownArgs {
  const uint8_t* w2;
  const void* w2s;
  const void* h;
  const int32_t* ids;
  const float* wts;
  void* y;
  int T, k, slots, E, H, I;
  int row_bytes;    // bytes of one w2 row
  int chunks;       // 16-byte chunks per w2 row
  int F;            // slots * chunks (flattened per-token chunks)
  int n_dgroups;    // output groups of ND rows
  int nxcd;
};

__device__ __forceinline__ int clamp_expert(int e, int n) {
  return (unsigned)e < (unsigned)n ? e : 0;
}

// Scale of 16-byte chunk c of weight row `row` (global row index over
// [experts][projections][rows]); `blk_row` is the row's 128-tile row index for
// FP8B128, `blk_rows_base` the tile-row base of its matrix.
template <int FMT>
__device__ __forceinline__ float chunk_scale(const void* scales, long long row, int c,
                                             int scale_row_len, long long tile_row) {
  if constexpr (FMT == W_MXFP8) {
    return e8m0_to_f32(reinterpret_cast<const uint8_t*>(scales)[row * scale_row_len + (c >> 1)]);
  } else if constexpr (FMT == W_MXFP4) {
    return e8m0_to_f32(reinterpret_cast<const uint8_t*>(scales)[row * scale_row_len + c]);
  } else if constexpr (FMT == W_FP8B128) {
    return reinterpret_cast<const float*>(scales)[tile_row * scale_row_len + (c >> 3)];
  } else {
    return 1.0f;
  }
}

// Activation chunk matching weight chunk c: Chunk<FMT>::kElems elements.
template <int FMT, bool XF32>
struct XChunk {
  static constexpr int kElems = Chunk<FMT>::kElems;
  static constexpr int kWords = XF32 ? kElems : kElems / 2;
  uint32_t v[kWords];
};

template <int FMT, bool XF32>
__device__ __forceinline__ void load_x_chunk(XChunk<FMT, XF32>& xc, const void* xrow, int c) {
  constexpr int W = XChunk<FMT, XF32>::kWords;
  const uint32_t* p = reinterpret_cast<const uint32_t*>(xrow) + (size_t)c * W;
  if constexpr (W >= 4) {
#pragma unroll
    for (int i = 0; i < W / 4; ++i) {
      u32x4 q = load16(p + 4 * i);
      xc.v[4 * i + 0] = q[0];
      xc.v[4 * i + 1] = q[1];
      xc.v[4 * i + 2] = q[2];
      xc.v[4 * i + 3] = q[3];
    }
  } else {
    const uint2 q = *reinterpret_cast<const uint2*>(p);
    xc.v[0] = q.x;
    xc.v[1] = q.y;
  }
}

template <int FMT, bool XF32>
__device__ __forceinline__ float chunk_dot(const u32x4 w, const XChunk<FMT, XF32>& xc) {
  if constexpr (XF32) {
    return chunk_dot_f32<FMT>(w, reinterpret_cast<const float*>(xc.v));
  } else {
    return chunk_dot_bf16<FMT>(w, xc.v);
  }
}

// r-th set bit over the LDS mask words (uniform inputs).
__device__ __forceinline__ int select_rank(const uint32_t* mask, int n_words, int r) {
  int q = 0;
  uint32_t m = 0;
  for (; q < n_words; ++q) {
    m = mask[q];
    int c = __popc(m);
    if (r < c) break;
    r -= c;
  }
  for (int i = 0; i < r; ++i) m &= m - 1;
  return q * 32 + __ffs(m) - 1;
}

template <int FMT, int NR, int MCH, bool XF32, bool HBF16>
__global__ __launch_bounds__(kBlock) void gate_up_decode_kernel(const GateUpArgs a) {
  __shared__ int s_ids[kDecodeMaxEntries];
  __shared__ uint32_t s_mask[kMaskWords];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int n_exp = a.E + (a.slots - a.k);

  for (int q = tid; q < a.n_words; q += kBlock) s_mask[q] = 0;
  __syncthreads();
  for (int v = tid; v < a.n_entries; v += kBlock) {
    const int t = v / a.slots, j = v - t * a.slots;
    const int e = j < a.k ? clamp_expert(a.ids[t * a.k + j], a.E) : a.E;
    s_ids[v] = e;
    atomicOr(&s_mask[e >> 5], 1u << (e & 31));
  }
  __syncthreads();

  int U = 0;
  for (int q = 0; q < a.n_words; ++q) U += __popc(s_mask[q]);
  const int n_items = U * a.n_groups;
  const int n_waves = gridDim.x * kWavesPerBlock;
  constexpr int EPC = Chunk<FMT>::kElems;
  (void)n_exp;

  for (int it = blockIdx.x * kWavesPerBlock + (tid >> 6); it < n_items; it += n_waves) {
    const int r = it / a.n_groups;
    const int g = it - r * a.n_groups;
    const int e = select_rank(s_mask, a.n_words, r);
    const int n0 = g * NR;

    // gate rows [0, NR), up rows [NR, 2NR): load every chunk of the lane once
    u32x4 wv[2 * NR][MCH];
    float sc[2 * NR][MCH];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
#pragma unroll
      for (int rr = 0; rr < NR; ++rr) {
        const int n = min(n0 + rr, a.I - 1);
        const long long row = ((long long)e * 2 + p) * a.I + n;
        const long long tile_row = ((long long)e * 2 + p) * (a.I >> 7) + (n >> 7);
        const uint8_t* base = a.w13 + row * a.row_bytes;
#pragma unroll
        for (int m = 0; m < MCH; ++m) {
          const int c = lane + m * kWave;
          if (c < a.chunks) {
            wv[p * NR + rr][m] = load_stream16(base + (size_t)c * 16);
            sc[p * NR + rr][m] = chunk_scale<FMT>(a.w13s, row, c,
                                                  FMT == W_FP8B128 ? (a.H >> 7) : (a.H >> 5),
                                                  tile_row);
          } else {
            wv[p * NR + rr][m] = u32x4{0, 0, 0, 0};
            sc[p * NR + rr][m] = 0.f;
          }
        }
      }
    }

    for (int base = 0; base < a.n_entries; base += kWave) {
      const int v = base + lane;
      const bool hit = v < a.n_entries && s_ids[v] == e;
      unsigned long long bm = __ballot(hit);
      while (bm) {
        const int b = __ffsll((long long)bm) - 1;
        bm &= bm - 1;
        const int pe = base + b;                    // entry index = t*slots + j
        const int t = pe / a.slots;
        const char* xrow = reinterpret_cast<const char*>(a.x) +
                           (size_t)t * a.H * (XF32 ? 4 : 2);
        float acc[2 * NR];
#pragma unroll
        for (int q = 0; q < 2 * NR; ++q) acc[q] = 0.f;
#pragma unroll
        for (int m = 0; m < MCH; ++m) {
          const int c = lane + m * kWave;
          if (c < a.chunks) {
            XChunk<FMT, XF32> xc;
            load_x_chunk<FMT, XF32>(xc, xrow, c);
#pragma unroll
            for (int q = 0; q < 2 * NR; ++q)
              acc[q] = fmaf(chunk_dot<FMT, XF32>(wv[q][m], xc), sc[q][m], acc[q]);
          }
        }
        float out = 0.f;
#pragma unroll
        for (int rr = 0; rr < NR; ++rr) {
          const float gsum = wave_sum(acc[rr]);
          const float usum = wave_sum(acc[NR + rr]);
          if (lane == rr) out = swiglu(gsum, usum);
        }
        if (lane < NR && n0 + lane < a.I) {
          const size_t off = (size_t)pe * a.I + n0 + lane;
          if constexpr (HBF16) {
            reinterpret_cast<uint16_t*>(a.h)[off] = (uint16_t)f32_to_bf16_bits(out);
          } else {
            reinterpret_cast<float*>(a.h)[off] = out;
          }
        }
      }
    }
  }
  (void)EPC;
}

// h chunk matching w2 chunk c of slot j: Chunk<FMT>::kElems elements.
template <int FMT, bool HBF16>
using HChunk = XChunk<FMT, !HBF16>;

template <int FMT, int ND, bool HBF16, bool YBF16>
__global__ __launch_bounds__(kBlock) void down_decode_kernel(const DownArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x, a.nxcd);
  const int item = lb * kWavesPerBlock + (threadIdx.x >> 6);
  if (item >= a.T * a.n_dgroups) return;
  const int dg = item / a.T;
  const int t = item - dg * a.T;
  const int d0 = dg * ND;

  int my_e = 0;
  float my_w = 0.f;
  if (lane < a.slots) {
    if (lane < a.k) {
      my_e = clamp_expert(a.ids[t * a.k + lane], a.E);
      my_w = a.wts[t * a.k + lane];
    } else {
      my_e = a.E;
      my_w = 1.0f;
    }
  }

  float acc[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) acc[d] = 0.f;

  const int n_m = (a.F + kWave - 1) / kWave;
  const size_t h_row_bytes = (size_t)a.I * (HBF16 ? 2 : 4);
  const char* hbase = reinterpret_cast<const char*>(a.h) + (size_t)t * a.slots * h_row_bytes;
  const int scale_len = FMT == W_FP8B128 ? (a.I >> 7) : (a.I >> 5);
  for (int m = 0; m < n_m; ++m) {
    const int f = m * kWave + lane;
    const bool valid = f < a.F;
    const int fj = valid ? f / a.chunks : 0;
    const int c = valid ? f - fj * a.chunks : 0;
    const int e = __shfl(my_e, fj);
    const float w = __shfl(my_w, fj);
    if (valid) {
      HChunk<FMT, HBF16> hc;
      load_x_chunk<FMT, !HBF16>(hc, hbase + (size_t)fj * h_row_bytes, c);
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        const int dd = min(d0 + d, a.H - 1);
        const long long row = (long long)e * a.H + dd;
        const long long tile_row = (long long)e * (a.H >> 7) + (dd >> 7);
        const u32x4 wq = load16(a.w2 + row * a.row_bytes + (size_t)c * 16);
        const float s = chunk_scale<FMT>(a.w2s, row, c, scale_len, tile_row);
        acc[d] = fmaf(chunk_dot<FMT, !HBF16>(wq, hc), s * w, acc[d]);
      }
    }
  }

  float out = 0.f;
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    const float v = wave_sum(acc[d]);
    if (lane == d) out = v;
  }
  if (lane < ND && d0 + lane < a.H) {
    const size_t off = (size_t)t * a.H + d0 + lane;
    if constexpr (YBF16) {
      reinterpret_cast<uint16_t*>(a.y)[off] = (uint16_t)f32_to_bf16_bits(out);
    } else {
      reinterpret_cast<float*>(a.y)[off] = out;
    }
  }
}

int row_bytes_of(int fmt, int k_elems) {
  switch (fmt) {
    case W_F32: return k_elems * 4;
    case W_MXFP4: return k_elems / 2;
    default: return k_elems;
  }
}

// ---- dispatch ------------------------------------------------------------

template <int FMT, int NR, bool XF32, bool HBF16>
hipError_t gate_up_mch(const GateUpArgs& a, int mch, int blocks, hipStream_t s) {
  dim3 g(blocks), b(kBlock);
  switch (mch) {
    case 1: hipLaunchKernelGGL((gate_up_decode_kernel<FMT, NR, 1, XF32, HBF16>), g, b, 0, s, a); break;
    case 2: hipLaunchKernelGGL((gate_up_decode_kernel<FMT, NR, 2, XF32, HBF16>), g, b, 0, s, a); break;
    case 4: hipLaunchKernelGGL((gate_up_decode_kernel<FMT, NR, 4, XF32, HBF16>), g, b, 0, s, a); break;
    case 8: hipLaunchKernelGGL((gate_up_decode_kernel<FMT, NR, 8, XF32, HBF16>), g, b, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int FMT, bool XF32, bool HBF16>
hipError_t gate_up_nr(const GateUpArgs& a, int nr, int mch, int blocks, hipStream_t s) {
  if (nr == 1) return gate_up_mch<FMT, 1, XF32, HBF16>(a, mch, blocks, s);
  return gate_up_mch<FMT, 2, XF32, HBF16>(a, mch, blocks, s);
}

template <int FMT, int ND, bool HBF16>
hipError_t down_y(const DownArgs& a, int ybf16, int blocks, hipStream_t s) {
  dim3 g(blocks), b(kBlock);
  if (ybf16) hipLaunchKernelGGL((down_decode_kernel<FMT, ND, HBF16, true>), g, b, 0, s, a);
  else hipLaunchKernelGGL((down_decode_kernel<FMT, ND, HBF16, false>), g, b, 0, s, a);
  return hipGetLastError();
}

template <int FMT, bool HBF16>
hipError_t down_nd(const DownArgs& a, int nd, int ybf16, int blocks, hipStream_t s) {
  switch (nd) {
    case 1: return down_y<FMT, 1, HBF16>(a, ybf16, blocks, s);
    case 2: return down_y<FMT, 2, HBF16>(a, ybf16, blocks, s);
    case 4: return down_y<FMT, 4, HBF16>(a, ybf16, blocks, s);
    default: return down_y<FMT, 8, HBF16>(a, ybf16, blocks, s);
  }
}

}  // namespace

hipError_t launch_gate_up_decode(const moe_weights& W, const void* x, int x_dtype,
                                 const int32_t* ids, int T, int k, void* h, int h_dtype,
                                 hipStream_t s) {
  GateUpArgs a;
  a.w13 = reinterpret_cast<const uint8_t*>(W.w13);
  a.w13s = W.w13_scale;
  a.x = x;
  a.ids = ids;
  a.h = h;
  a.T = T;
  a.k = k;
  a.slots = k + W.num_shared;
  a.E = W.num_experts;
  a.H = W.hidden;
  a.I = W.inter;
  a.row_bytes = row_bytes_of(W.format, W.hidden);
  a.chunks = a.row_bytes / 16;
  const int n_exp = W.num_experts + W.num_shared;
  a.n_words = (n_exp + 31) / 32;
  a.n_entries = T * a.slots;
  // wider neuron groups amortise the activation reads; one row pair when a
  // lane already holds many chunks of a long row
  const int lane_chunks = (a.chunks + kWave - 1) / kWave;
  const int mch = lane_chunks <= 1 ? 1 : lane_chunks <= 2 ? 2 : lane_chunks <= 4 ? 4 : 8;
  const int nr = mch >= 8 ? 1 : 2;
  a.n_groups = (W.inter + nr - 1) / nr;
  const long long max_items = (long long)std::min(n_exp, a.n_entries) * a.n_groups;
  const long long want = (max_items + kWavesPerBlock - 1) / kWavesPerBlock;
  const int cap = device_num_cus() * 4;
  const int blocks = (int)std::max<long long>(1, std::min<long long>(want, cap));
  const bool xf32 = x_dtype == MOE_DT_F32;
  const bool hbf = h_dtype == MOE_DT_BF16;
  switch (W.format) {
    case W_F32:
      if (xf32) return hbf ? gate_up_nr<W_F32, true, true>(a, nr, mch, blocks, s)
                           : gate_up_nr<W_F32, true, false>(a, nr, mch, blocks, s);
      return hbf ? gate_up_nr<W_F32, false, true>(a, nr, mch, blocks, s)
                 : gate_up_nr<W_F32, false, false>(a, nr, mch, blocks, s);
    case W_MXFP8:
      return hbf ? gate_up_nr<W_MXFP8, false, true>(a, nr, mch, blocks, s)
                 : gate_up_nr<W_MXFP8, false, false>(a, nr, mch, blocks, s);
    case W_MXFP4:
      return hbf ? gate_up_nr<W_MXFP4, false, true>(a, nr, mch, blocks, s)
                 : gate_up_nr<W_MXFP4, false, false>(a, nr, mch, blocks, s);
    case W_FP8B128:
      return hbf ? gate_up_nr<W_FP8B128, false, true>(a, nr, mch, blocks, s)
                 : gate_up_nr<W_FP8B128, false, false>(a, nr, mch, blocks, s);
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_down_decode(const moe_weights& W, const void* h, int h_dtype,
                              const int32_t* ids, const float* wts, int T, int k, void* y,
                              int y_dtype, hipStream_t s) {
  DownArgs a;
  a.w2 = reinterpret_cast<const uint8_t*>(W.w2);
  a.w2s = W.w2_scale;
  a.h = h;
  a.ids = ids;
  a.wts = wts;
  a.y = y;
  a.T = T;
  a.k = k;
  a.slots = k + W.num_shared;
  a.E = W.num_experts;
  a.H = W.hidden;
  a.I = W.inter;
  a.row_bytes = row_bytes_of(W.format, W.inter);
  a.chunks = a.row_bytes / 16;
  a.F = a.slots * a.chunks;
  a.nxcd = device_num_xcds();
  // output rows per wave: enough waves to fill the chip at small T, more
  // reuse of the staged h chunk at large T
  const long long target_waves = (long long)device_num_cus() * 8;
  int nd = 8;
  while (nd > 1 && (long long)T * ((W.hidden + nd - 1) / nd) < target_waves) nd >>= 1;
  a.n_dgroups = (W.hidden + nd - 1) / nd;
  const long long items = (long long)T * a.n_dgroups;
  const int blocks = (int)((items + kWavesPerBlock - 1) / kWavesPerBlock);
  const bool hbf = h_dtype == MOE_DT_BF16;
  const int ybf = y_dtype == MOE_DT_BF16;
  switch (W.format) {
    case W_F32:
      return hbf ? down_nd<W_F32, true>(a, nd, ybf, blocks, s) : down_nd<W_F32, false>(a, nd, ybf, blocks, s);
    case W_MXFP8:
      return hbf ? down_nd<W_MXFP8, true>(a, nd, ybf, blocks, s) : down_nd<W_MXFP8, false>(a, nd, ybf, blocks, s);
    case W_MXFP4:
      return hbf ? down_nd<W_MXFP4, true>(a, nd, ybf, blocks, s) : down_nd<W_MXFP4, false>(a, nd, ybf, blocks, s);
    case W_FP8B128:
      return hbf ? down_nd<W_FP8B128, true>(a, nd, ybf, blocks, s) : down_nd<W_FP8B128, false>(a, nd, ybf, blocks, s);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace moe
