// Output-centric decode kernels: gate_up and down.
//
// Both follow the warp-decode post (sections on how the two kernels work and
// on warp independence): every output scalar is owned by exactly one 64-lane
// wavefront, which streams the expert weight rows it needs, converts the
// stored format to BF16/FP32 in registers, keeps FP32 accumulators and
// finishes with a fixed-order cross-lane reduction.
//
// gfx950-specific choices (not on the pages):
//  * gate_up is expert-major: a wavefront owns NR neurons (their gate and up
//    rows) of one touched expert and produces them for every (token, slot)
//    routed to that expert in the batch, so each weight row is read from HBM
//    once per call even when several tokens share an expert.  Each workgroup
//    finds the touched experts itself from the routed ids (LDS bitmask), so
//    no pre-pass kernel and no host sync are needed; wavefronts loop over
//    (expert rank, neuron group) items with a static stride.  Rows of up to
//    four chunks per lane are converted to BF16 once per item and reused for
//    every routed token; longer rows are converted per token.
//  * down has two variants with bitwise-identical results.  In both, a row of
//    W_down is split over LPR lanes (8 or 16) so one wavefront covers 64/LPR
//    output rows and every dot product is reduced inside a DPP row.
//      - token-major (as on the page): a wavefront owns (token, output rows)
//        and folds the token's slots in slot order into y; no buffer at all.
//      - expert-major: a wavefront owns (expert, output rows), reads those
//        rows once and writes w * dot for every (token, slot) routed to the
//        expert; a small combine kernel then sums the slots in slot order.
//        Used from a number of routed entries up (see down_variant_for),
//        where it was measured faster: rows shared by several tokens are
//        read once instead of once per (token, slot).
//  * MXFP4 gate_up (E2M1 rows, BF16 activations) runs on the matrix cores
//    instead: a wavefront owns (expert, 16 neurons) with the expert's routed
//    entries as MFMA columns, and streams 128-byte row slices through an LDS
//    ring by direct-to-LDS loads; MXFP4 expert-major down likewise (see
//    mx4_mfma_kernel).
//  * 16-byte loads per lane; E4M3 / E2M1 are converted exactly to BF16 and
//    multiplied with BF16 activations by v_dot2_f32_bf16, or converted to FP32
//    for FP32 intermediates; the MX / tile scale multiplies each 16-byte
//    chunk's partial sum, except in gate_up rows converted once per item,
//    where an MX scale (a power of two) enters the conversion itself.

#include <algorithm>
#include <cmath>

#include "device.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kMaskWords = kMaxExpertsTotal / 32;
constexpr int kDownTokenMajor = MOE_DOWN_TOKEN_MAJOR;
constexpr int kDownExpertMajor = MOE_DOWN_EXPERT_MAJOR;

// Occupancy floor for the streaming kernels: at least WPE wavefronts per SIMD
// (4 -> <= 128 VGPRs), so latency is hidden by resident waves rather than by
// registers the compiler would otherwise spend on hoisted loads; 2 for the
// shapes that keep long rows (or a prefetched second item) in registers.
#define MOE_STREAM_KERNEL(WPE) \
  __global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(WPE)))

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
  uint32_t slots_magic;  // ceil(2^32 / slots): entry / slots by a multiply-high
  int sscl;         // MXFP8 neuron pairs: the rows' scales as one dword per lane
};

struct DownArgs {
  const uint8_t* w2;
  const void* w2s;
  const void* h;
  const int32_t* ids;
  const float* wts;
  void* y;          // token-major: y [T][H]; expert-major: slot_out [T*slots][H] f32
  int T, k, slots, E, H, I;
  int row_bytes;    // bytes of one w2 row
  int chunks;       // 16-byte chunks per w2 row
  int cpl;          // chunks per lane = chunks / LPR
  int n_dgroups;    // output groups of 64/LPR rows
  int n_words;
  int n_entries;
  int nxcd;
  uint32_t slots_magic;
  int rpl;          // rows per lane group in the expert-major kernel
  int sscl;         // expert-major MXFP8: stage each item's scale bytes in LDS
};

// entry / slots for entry < 2^24 (slots <= 64): exact with a 32-bit reciprocal.
__device__ __forceinline__ int div_slots(int v, uint32_t magic) {
  return (int)(((unsigned long long)(unsigned)v * magic) >> 32);
}

__device__ __forceinline__ int clamp_expert(int e, int n) {
  return (unsigned)e < (unsigned)n ? e : 0;
}

// Stage the batch's routed experts in LDS (entry index t*slots + j -> expert,
// the shared slot being expert E) and the bitmask of touched experts.
// Returns the number of touched experts.  Whole workgroup; two barriers.
__device__ __forceinline__ int stage_routing(const int32_t* ids, int k, int slots, int E,
                                             int n_words, int n_entries, int* s_ids,
                                             uint32_t* s_mask) {
  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  for (int q = tid; q < n_words; q += nt) s_mask[q] = 0;
  __syncthreads();
  for (int v = tid; v < n_entries; v += nt) {
    const int t = v / slots, j = v - t * slots;
    const int e = j < k ? clamp_expert(ids[t * k + j], E) : E;
    s_ids[v] = e;
    atomicOr(&s_mask[e >> 5], 1u << (e & 31));
  }
  __syncthreads();
  int u = 0;
  for (int q = 0; q < n_words; ++q) u += __popc(s_mask[q]);
  return u;
}

// r-th set bit over the LDS mask words (uniform inputs).
__device__ __forceinline__ int select_rank(const uint32_t* mask, int n_words, int r) {
  int q = 0;
  uint32_t m = 0;
  for (; q < n_words; ++q) {
    m = mask[q];
    const int c = __popc(m);
    if (r < c) break;
    r -= c;
  }
  for (int i = 0; i < r; ++i) m &= m - 1;
  return __builtin_amdgcn_readfirstlane(q * 32 + __ffs(m) - 1);
}

// Walks the entries routed to one expert, in ascending entry order.
struct PairIter {
  int base;
  unsigned long long bm;
};

__device__ __forceinline__ void pairs_begin(PairIter& it, const int* s_ids, int n, int e) {
  const int lane = threadIdx.x & (kWave - 1);
  it.base = 0;
  it.bm = __ballot(lane < n && s_ids[lane] == e);
}

__device__ __forceinline__ int pairs_next(PairIter& it, const int* s_ids, int n, int e) {
  const int lane = threadIdx.x & (kWave - 1);
  while (it.bm == 0) {
    it.base += kWave;
    if (it.base >= n) return -1;
    const int v = it.base + lane;
    it.bm = __ballot(v < n && s_ids[v] == e);
  }
  const int b = __ffsll((long long)it.bm) - 1;
  it.bm &= it.bm - 1;
  return it.base + b;
}

// Scale of 16-byte chunk c of weight row `row`; `tile_row` is the row's
// 128-tile row (FP8 with 128x128 tiles).
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
      const u32x4 q = load16(p + 4 * i);
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

// ---------------------------------------------------------------------------
// gate_up
// ---------------------------------------------------------------------------

// Rows of one item.  PRE: held as exact BF16 pairs (converted once per item,
// reused by every token routed to the expert); otherwise the raw 16-byte
// chunks, converted per token.
template <int FMT, int NR, int MCH, bool PRE>
struct GateRows {
  static constexpr int kWords = PRE ? Chunk<FMT>::kElems / 2 : 4;
  uint32_t w[2 * NR][MCH][kWords];
  float s[2 * NR][MCH];
};

// The conversion multiplies by `sc`: 1 for unscaled use, or an MX block
// scale (a power of two, so the BF16 result stays exact while it is a
// normal BF16 number).
template <int FMT>
__device__ __forceinline__ void chunk_to_bf16(const u32x4 q, uint32_t* out, float sc) {
  if constexpr (FMT == W_MXFP4) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      out[4 * d + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[d], sc, 0));
      out[4 * d + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[d], sc, 1));
      out[4 * d + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[d], sc, 2));
      out[4 * d + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[d], sc, 3));
    }
  } else {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      out[2 * d + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[d], sc, false));
      out[2 * d + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[d], sc, true));
    }
  }
}

// PRE rows of MX formats carry their block scale inside the converted BF16
// values, so the per-token dot products need no scale multiply.
template <int FMT, bool PRE>
constexpr bool scale_folded() { return PRE && (FMT == W_MXFP8 || FMT == W_MXFP4); }

// For MXFP8 neuron pairs (rows of MCH <= 2 whole 64-lane passes) the four
// rows' E8M0 scales are two runs of 2 * H/32 bytes, the gate rows n0, n0 + 1
// and the up rows n0, n0 + 1: 32 * MCH dwords.  In the DW instantiation (the
// host's a.sscl: I even, so n0 + 1 < I, and the scales 4-byte aligned) each
// lane loads one dword of them, ahead of the rows, and every lane takes its
// chunks' scale bytes from the lanes holding them (ds_bpermute), in place of
// a byte load per row and chunk.  Same scale values, same bits.
template <int FMT, int NR, int MCH, bool GUARD>
constexpr bool gate_scales_by_dword() {
  return FMT == W_MXFP8 && NR == 2 && MCH <= 2 && !GUARD;
}

// GUARD: the row has fewer than 64*MCH chunks, lanes past the end hold zeros.
template <int FMT, int NR, int MCH, bool PRE, bool GUARD, bool DW>
__device__ __forceinline__ void load_gate_rows(GateRows<FMT, NR, MCH, PRE>& R,
                                               const GateUpArgs& a, int e, int n0, int lane) {
  static_assert(!DW || gate_scales_by_dword<FMT, NR, MCH, GUARD>(), "dword scale shape");
  constexpr int kRun = 16 * MCH;                  // dwords of two rows' scales
  const int srow = a.H >> 5;                      // scale bytes per row
  uint32_t sdw = 0;
  if constexpr (DW) {
    if (lane < 2 * kRun) {
      const int p = lane / kRun, k = lane - p * kRun;
      sdw = reinterpret_cast<const uint32_t*>(
          reinterpret_cast<const uint8_t*>(a.w13s) + (((long long)e * 2 + p) * a.I + n0) * srow)[k];
    }
  }
  u32x4 raw[2 * NR][MCH];
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
        if (!GUARD || c < a.chunks) {
          raw[p * NR + rr][m] = load_stream16(base + (size_t)c * 16);
          if constexpr (!DW)
            R.s[p * NR + rr][m] = chunk_scale<FMT>(
                a.w13s, row, c, FMT == W_FP8B128 ? (a.H >> 7) : (a.H >> 5), tile_row);
        } else {
          raw[p * NR + rr][m] = u32x4{0, 0, 0, 0};
          R.s[p * NR + rr][m] = 0.f;
        }
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 2 * NR; ++q)
#pragma unroll
    for (int m = 0; m < MCH; ++m) {
      if constexpr (DW) {
        // chunk lane + 64 m of row q uses the row's scale byte (lane + 64 m) / 2;
        // row q starts q * srow bytes into the two runs, and lane i holds dword i
        const int off = q * srow + ((lane + m * kWave) >> 1);
        const uint32_t v = (uint32_t)__builtin_amdgcn_ds_bpermute((off >> 2) << 2, (int)sdw);
        R.s[q][m] = e8m0_to_f32((v >> (8 * (off & 3))) & 0xffu);
      }
      if constexpr (PRE) {
        chunk_to_bf16<FMT>(raw[q][m], R.w[q][m], scale_folded<FMT, PRE>() ? R.s[q][m] : 1.0f);
      } else {
        R.w[q][m][0] = raw[q][m][0];
        R.w[q][m][1] = raw[q][m][1];
        R.w[q][m][2] = raw[q][m][2];
        R.w[q][m][3] = raw[q][m][3];
      }
    }
}

template <int FMT, int NR, int MCH, bool PRE, bool XF32>
__device__ __forceinline__ float gate_chunk_dot(GateRows<FMT, NR, MCH, PRE>& R, int q, int m,
                                                const XChunk<FMT, XF32>& xc) {
  if constexpr (PRE) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < GateRows<FMT, NR, MCH, PRE>::kWords; ++i)
      acc = dot2_bf16(as_bf16x2(R.w[q][m][i]), as_bf16x2(xc.v[i]), acc);
    return acc;
  } else {
    u32x4 w = {R.w[q][m][0], R.w[q][m][1], R.w[q][m][2], R.w[q][m][3]};
    opaque(w);   // keep the conversion per token (registers), see PRE
    return chunk_dot<FMT, XF32>(w, xc);
  }
}

// The MCH activation chunks of token entry pe, all requested together.
template <int FMT, int MCH, bool XF32, bool GUARD>
__device__ __forceinline__ void load_token_x(XChunk<FMT, XF32> (&xc)[MCH], const GateUpArgs& a,
                                             int pe, int lane) {
  const char* xrow = reinterpret_cast<const char*>(a.x) +
                     (size_t)div_slots(pe, a.slots_magic) * a.H * (XF32 ? 4 : 2);
#pragma unroll
  for (int m = 0; m < MCH; ++m) {
    const int c = lane + m * kWave;
    load_x_chunk<FMT, XF32>(xc[m], xrow, GUARD ? min(c, a.chunks - 1) : c);
  }
}

template <int FMT, int NR, int MCH, bool PRE, bool XF32, bool HBF16, bool GUARD>
__device__ __forceinline__ void gate_up_pair(GateRows<FMT, NR, MCH, PRE>& R, const GateUpArgs& a,
                                             const XChunk<FMT, XF32> (&xc)[MCH], int pe, int n0,
                                             int lane) {
  float acc[2 * NR];
#pragma unroll
  for (int q = 0; q < 2 * NR; ++q) {
    acc[q] = 0.f;
    if constexpr (scale_folded<FMT, PRE>()) {
#pragma unroll
      for (int m = 0; m < MCH; ++m)
#pragma unroll
        for (int i = 0; i < GateRows<FMT, NR, MCH, PRE>::kWords; ++i)
          acc[q] = dot2_bf16(as_bf16x2(R.w[q][m][i]), as_bf16x2(xc[m].v[i]), acc[q]);
    } else {
#pragma unroll
      for (int m = 0; m < MCH; ++m)
        acc[q] = fmaf(gate_chunk_dot<FMT, NR, MCH, PRE, XF32>(R, q, m, xc[m]), R.s[q][m], acc[q]);
    }
  }
  float out;
  if constexpr (NR == 2) {
    const float r = wave_sum4_rows(acc[0], acc[1], acc[2], acc[3]);
    const float g0 = lane_value(r, 0), g1 = lane_value(r, 16);
    const float u0 = lane_value(r, 32), u1 = lane_value(r, 48);
    out = lane == 0 ? swiglu(g0, u0) : swiglu(g1, u1);
  } else {
    const float r = wave_sum2_halves(acc[0], acc[1]);
    out = swiglu(lane_value(r, 0), lane_value(r, 32));
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

template <int FMT, int NR, int MCH, bool PRE, bool XF32, bool HBF16, bool GUARD, bool DW>
MOE_STREAM_KERNEL(MCH >= 7 ? 2 : 4) void gate_up_decode_kernel(const GateUpArgs a) {
  __shared__ int s_ids[kDecodeMaxEntries];
  __shared__ uint32_t s_mask[kMaskWords];
  const int lane = threadIdx.x & (kWave - 1);
  const int U = stage_routing(a.ids, a.k, a.slots, a.E, a.n_words, a.n_entries, s_ids, s_mask);
  const int n_items = U * a.n_groups;
  const int n_waves = gridDim.x * kWavesPerBlock;
  for (int it = blockIdx.x * kWavesPerBlock + wave_in_block(); it < n_items; it += n_waves) {
    const int e = select_rank(s_mask, a.n_words, it / a.n_groups);
    const int n0 = (it % a.n_groups) * NR;
    // the first routed token's activations are requested together with the
    // rows, so they arrive in the same memory round trip
    PairIter pi;
    pairs_begin(pi, s_ids, a.n_entries, e);
    int pe = pairs_next(pi, s_ids, a.n_entries, e);
    XChunk<FMT, XF32> xc[MCH];
    load_token_x<FMT, MCH, XF32, GUARD>(xc, a, pe, lane);
    GateRows<FMT, NR, MCH, PRE> rows;
    load_gate_rows<FMT, NR, MCH, PRE, GUARD, DW>(rows, a, e, n0, lane);
    while (true) {
      gate_up_pair<FMT, NR, MCH, PRE, XF32, HBF16, GUARD>(rows, a, xc, pe, n0, lane);
      pe = pairs_next(pi, s_ids, a.n_entries, e);
      if (pe < 0) break;
      load_token_x<FMT, MCH, XF32, GUARD>(xc, a, pe, lane);
    }
  }
}

// ---------------------------------------------------------------------------
// down: shared per-row dot product over LPR lanes
// ---------------------------------------------------------------------------

template <int FMT, int CPL>
struct DownRow {
  u32x4 w[CPL];
  float s[CPL];
};

// Row d of expert e's W_down.  e is uniform, so the expert's weight and scale
// bases are scalar; only the offset of the lane's row inside the expert (below
// 2^31 bytes, checked at launch) is per lane, in 32-bit arithmetic.
template <int FMT, int LPR, int CPL, bool SCALES = true>
__device__ __forceinline__ void load_down_row(DownRow<FMT, CPL>& R, const DownArgs& a, int e,
                                              int d, int gl, bool stream) {
  const uint8_t* base = a.w2 + (size_t)e * a.H * a.row_bytes + (uint32_t)d * (uint32_t)a.row_bytes;
  const int scale_len = FMT == W_FP8B128 ? (a.I >> 7) : (a.I >> 5);
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = gl + LPR * i;
    R.w[i] = stream ? load_stream16(base + (uint32_t)c * 16) : load16(base + (uint32_t)c * 16);
    if constexpr (!SCALES) {
      R.s[i] = 0.0f;   // set by the caller
    } else if constexpr (FMT == W_MXFP8 || FMT == W_MXFP4) {
      const uint8_t* sb = reinterpret_cast<const uint8_t*>(a.w2s) + (size_t)e * a.H * scale_len;
      R.s[i] = e8m0_to_f32(sb[(uint32_t)d * scale_len + (FMT == W_MXFP8 ? (c >> 1) : c)]);
    } else if constexpr (FMT == W_FP8B128) {
      const float* sb = reinterpret_cast<const float*>(a.w2s) + (size_t)e * (a.H >> 7) * scale_len;
      R.s[i] = sb[(d >> 7) * scale_len + (c >> 3)];
    } else {
      R.s[i] = 1.0f;
    }
  }
}

// dot(row r, h[pe]) for the lane's RPL rows, each reduced over its LPR lanes
// (every lane of the group gets the totals).  Fixed order per row: chunk by
// chunk per lane, then the DPP tree; the staged h chunks serve all RPL rows.
template <int FMT, int LPR, int CPL, bool HBF16>
__device__ __forceinline__ void load_h_chunks(XChunk<FMT, !HBF16> (&hc)[CPL], const DownArgs& a,
                                              int pe, int gl) {
  const size_t h_row_bytes = (size_t)a.I * (HBF16 ? 2 : 4);
  const char* hrow = reinterpret_cast<const char*>(a.h) + (size_t)pe * h_row_bytes;
#pragma unroll
  for (int i = 0; i < CPL; ++i) load_x_chunk<FMT, !HBF16>(hc[i], hrow, gl + LPR * i);
}

template <int FMT, int LPR, int CPL, int RPL, bool HBF16>
__device__ __forceinline__ void rows_dot_staged(DownRow<FMT, CPL> (&R)[RPL],
                                                const XChunk<FMT, !HBF16> (&hc)[CPL],
                                                float (&out)[RPL]) {
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) opaque(R[r].w[i]);
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < CPL; ++i)
      acc = fmaf(chunk_dot<FMT, !HBF16>(R[r].w[i], hc[i]), R[r].s[i], acc);
    if constexpr (LPR == 32) out[r] = half32_sum(acc);
    else if constexpr (LPR == 16) out[r] = row16_sum(acc);
    else if constexpr (LPR == 8) out[r] = group8_sum(acc);
    else out[r] = group4_sum(acc);
  }
}

template <int FMT, int LPR, int CPL, int RPL, bool HBF16>
__device__ __forceinline__ void down_rows_dot(DownRow<FMT, CPL> (&R)[RPL], const DownArgs& a,
                                              int pe, int gl, float (&out)[RPL]) {
  XChunk<FMT, !HBF16> hc[CPL];
  load_h_chunks<FMT, LPR, CPL, HBF16>(hc, a, pe, gl);
  rows_dot_staged<FMT, LPR, CPL, RPL, HBF16>(R, hc, out);
}

__device__ __forceinline__ float slot_weight(const DownArgs& a, int pe) {
  const int t = div_slots(pe, a.slots_magic), j = pe - t * a.slots;
  return j < a.k ? a.wts[t * a.k + j] : 1.0f;
}

// VGPRs the staged h chunks of one lane take.
template <int FMT, int CPL, bool HBF16>
constexpr int h_regs() { return CPL * Chunk<FMT>::kElems * (HBF16 ? 2 : 4) / 4; }

// Expert-major: slot_out[pe][d] = w_pe * dot(Wd[e][d], h[pe]).  A wavefront
// item is RPL * 64/LPR output rows of one expert.
template <int FMT, int LPR, int CPL, int RPL, bool HBF16>
MOE_STREAM_KERNEL((h_regs<FMT, CPL, HBF16>() > 48 || CPL >= 12) ? 2 : 4) void down_expert_kernel(
    const DownArgs a) {
  __shared__ int s_ids[kDecodeMaxEntries];
  __shared__ uint32_t s_mask[kMaskWords];
  constexpr int ND = kWave / LPR;
  const int lane = threadIdx.x & (kWave - 1);
  const int grp = lane / LPR, gl = lane % LPR;
  const int U = stage_routing(a.ids, a.k, a.slots, a.E, a.n_words, a.n_entries, s_ids, s_mask);
  const int n_items = U * a.n_dgroups;
  const int n_waves = gridDim.x * kWavesPerBlock;
  float* out = reinterpret_cast<float*>(a.y);
  for (int it = blockIdx.x * kWavesPerBlock + wave_in_block(); it < n_items; it += n_waves) {
    const int e = select_rank(s_mask, a.n_words, it / a.n_dgroups);
    const int d0 = (it % a.n_dgroups) * ND * RPL + grp;
    DownRow<FMT, CPL> rows[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r)
      load_down_row<FMT, LPR, CPL>(rows[r], a, e, min(d0 + r * ND, a.H - 1), gl, true);
    PairIter pi;
    pairs_begin(pi, s_ids, a.n_entries, e);
    for (int pe = pairs_next(pi, s_ids, a.n_entries, e); pe >= 0;
         pe = pairs_next(pi, s_ids, a.n_entries, e)) {
      float dot[RPL];
      down_rows_dot<FMT, LPR, CPL, RPL, HBF16>(rows, a, pe, gl, dot);
      const float w = slot_weight(a, pe);
#pragma unroll
      for (int r = 0; r < RPL; ++r)
        if (gl == 0 && d0 + r * ND < a.H)
          out[(size_t)pe * a.H + d0 + r * ND] = __fmul_rn(dot[r], w);
    }
  }
}

// Expert-major down with the item's E4M3 rows converted to BF16 once instead
// of once per routed entry.  The conversion is exact and unscaled, and each
// chunk's partial sum is still a fresh dot2 chain over the same pairs in the
// same order, multiplied into the accumulator by the chunk's scale, then the
// same lane reduction: y keeps the bits of the other two down kernels.  Per
// entry only the dot products remain.  With SSCL (MXFP8 rows, when the host
// finds the item's scale bytes whole and 16-byte aligned) the item's rows are
// consecutive rows of W_down, so their E8M0 scales are one run of
// ND*RPL*I/32 bytes: one 16-byte load per lane brings the run into the
// wavefront's LDS slice, in place of one byte load per row and chunk.
template <int LPR>
__device__ __forceinline__ float lane_group_sum(float acc) {
  if constexpr (LPR == 32) return half32_sum(acc);
  else if constexpr (LPR == 16) return row16_sum(acc);
  else if constexpr (LPR == 8) return group8_sum(acc);
  else return group4_sum(acc);
}

constexpr int kPreScaleBytes = 1024;   // per wavefront: a 16-byte load per lane

template <int FMT, int LPR, int CPL, int RPL, bool SSCL>
MOE_STREAM_KERNEL(RPL * CPL >= 8 ? 3 : 4) void down_expert_pre_kernel(const DownArgs a) {
  static_assert(FMT == W_MXFP8 || FMT == W_FP8B128, "E4M3 rows");
  static_assert(!SSCL || FMT == W_MXFP8, "staged E8M0 scales");
  __shared__ int s_ids[kDecodeMaxEntries];
  __shared__ uint32_t s_mask[kMaskWords];
  __shared__ __attribute__((aligned(16))) uint8_t s_scl[SSCL ? kWavesPerBlock * kPreScaleBytes : 16];
  constexpr int ND = kWave / LPR;
  const int lane = threadIdx.x & (kWave - 1);
  const int grp = lane / LPR, gl = lane % LPR;
  const int U = stage_routing(a.ids, a.k, a.slots, a.E, a.n_words, a.n_entries, s_ids, s_mask);
  const int n_items = U * a.n_dgroups;
  const int n_waves = gridDim.x * kWavesPerBlock;
  float* out = reinterpret_cast<float*>(a.y);
  for (int it = blockIdx.x * kWavesPerBlock + wave_in_block(); it < n_items; it += n_waves) {
    const int e = select_rank(s_mask, a.n_words, it / a.n_dgroups);
    const int row0 = (it % a.n_dgroups) * ND * RPL;
    const int d0 = row0 + grp;
    DownRow<FMT, CPL> raw[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r)
      load_down_row<FMT, LPR, CPL, !SSCL>(raw[r], a, e, min(d0 + r * ND, a.H - 1), gl, true);
    // SSCL: the host checked that H is a multiple of ND*RPL (no partial
    // item), that the run is a multiple of 16 bytes and at most
    // kPreScaleBytes, and that every run starts 16-byte aligned
    const int scale_len = a.I >> 5;
    const bool s_lane = SSCL && lane * 16 < ND * RPL * scale_len;
    u32x4 sv = {0u, 0u, 0u, 0u};
    if (s_lane)
      sv = load16(reinterpret_cast<const uint8_t*>(a.w2s) + ((size_t)e * a.H + row0) * scale_len +
                  lane * 16);
    // wb[r][i][2d], [2d + 1]: the two BF16 pairs of byte pairs 0-1 and 2-3 of dword d
    uint32_t wb[RPL][CPL][8];
#pragma unroll
    for (int r = 0; r < RPL; ++r)
#pragma unroll
      for (int i = 0; i < CPL; ++i)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          wb[r][i][2 * d] = __builtin_bit_cast(uint32_t, fp8x2_to_bf16x2<false>(raw[r].w[i][d]));
          wb[r][i][2 * d + 1] = __builtin_bit_cast(uint32_t, fp8x2_to_bf16x2<true>(raw[r].w[i][d]));
        }
    if constexpr (SSCL) {
      uint8_t* sl = s_scl + wave_in_block() * kPreScaleBytes;
      if (s_lane) *reinterpret_cast<u32x4*>(sl + lane * 16) = sv;
      // the same wavefront wrote the slice: its LDS accesses stay in order
#pragma unroll
      for (int r = 0; r < RPL; ++r)
#pragma unroll
        for (int i = 0; i < CPL; ++i)
          raw[r].s[i] = e8m0_to_f32(sl[(grp + r * ND) * scale_len + ((gl + LPR * i) >> 1)]);
    }
    PairIter pi;
    pairs_begin(pi, s_ids, a.n_entries, e);
    for (int pe = pairs_next(pi, s_ids, a.n_entries, e); pe >= 0;
         pe = pairs_next(pi, s_ids, a.n_entries, e)) {
      XChunk<FMT, false> hc[CPL];
      load_h_chunks<FMT, LPR, CPL, true>(hc, a, pe, gl);
      const float w = slot_weight(a, pe);
#pragma unroll
      for (int r = 0; r < RPL; ++r) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          float part = 0.f;
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            part = dot2_bf16(as_bf16x2(wb[r][i][2 * d]), as_bf16x2(hc[i].v[2 * d]), part);
            part = dot2_bf16(as_bf16x2(wb[r][i][2 * d + 1]), as_bf16x2(hc[i].v[2 * d + 1]), part);
          }
          acc = fmaf(part, raw[r].s[i], acc);
        }
        const float dot = lane_group_sum<LPR>(acc);
        if (gl == 0 && d0 + r * ND < a.H) out[(size_t)pe * a.H + d0 + r * ND] = __fmul_rn(dot, w);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// gate_up and down on the matrix cores for E2M1 rows and BF16 activations
// ---------------------------------------------------------------------------
//
// With E2M1 rows the vector kernels convert every row again for each routed
// token (BF16 copies of the rows do not fit in registers), so their work grows
// with the tokens per expert.  These kernels put the rows on the matrix
// cores instead.  A wavefront owns a unit: 32 weight rows of one expert (the
// gate and up rows of 16 neurons, or 32 consecutive rows of W_down), as two
// 16-row operand blocks of v_mfma_f32_16x16x32_bf16, against up to TC of the
// expert's routed entries as the columns.  An expert with more than TC entries
// is split into "virtual experts" (passes of TC entries), each a separate run
// of units, so a heavily routed expert is spread over many wavefronts.  Units
// are dealt to the wavefronts in contiguous ranges (consecutive units share
// the expert and its entry list, and read adjacent rows).
// The rows are cut into 128-byte slices (256 K values).  A slice of the 32
// rows, the columns' BF16 activations over the same K range and the rows'
// E8M0 scales travel HBM -> LDS by direct-to-LDS loads into a ring of NS
// stages per wavefront: NS - 1 stages are in flight while one is consumed,
// and no registers hold staged data.  Each slice is converted to BF16 once
// (the MX scale, a power of two, enters the conversion exactly) and feeds
// every column.  A lane's A and B operands take the same K values in the same
// order (a permutation of K that keeps each 16-byte chunk in one lane), so
// each column is an exact-product FP32 accumulation over K in a fixed order
// that depends neither on the other columns nor on TC or NS: results do not
// depend on the batch (tested bitwise).
//   gate_up: h[pe][n] = SiLU(gate . x) * (up . x), x the entry's token row.
//   down:    slot_out[pe][d] = w_pe * (Wd[d] . h[pe]), summed in slot order
//            by the combine kernel.

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMx4SliceBytes = 128;   // bytes of a row per stage (256 K values)
constexpr int kMx4XBytes = 512;       // BF16 activations of one column per stage

struct Mx4Args {
  const uint8_t* w;       // gate_up: w13 [E+S][2I][H/2]; down: w2 [E+S][H][I/2]
  const uint8_t* ws;      // E8M0 scales, K/32 per row
  const uint8_t* act;     // gate_up: x [T][H]; down: h [T*slots][I] (BF16)
  const int32_t* ids;
  const float* wts;       // down only
  void* out;              // gate_up: h [T*slots][I]; down: slot_out [T*slots][H] FP32
  int T, k, slots, E, n_words, n_entries;
  int K, N;               // reduction length; gate_up: neurons I, down: rows H
  int row_bytes;          // K / 2
  int n_groups;           // units per virtual expert: I / 16 or H / 32
  uint32_t slots_magic;
};

// LDS layout of one instantiation: the ring, then the work map.
template <int TC, int NS, bool DOWN>
struct Mx4Lds {
  static constexpr int X = 32 * kMx4SliceBytes;        // stage: W [32 rows][128 B] (chunks
  static constexpr int S = X + TC * kMx4XBytes;        //  swizzled by row) | X [TC][512 B]
  static constexpr int STAGE = S + 256;                //  (pieces swizzled by column) | S
  static constexpr int XI = TC * kMx4XBytes / 1024;    // activation loads per stage
  static constexpr int OPS = 4 + XI + 1;               // direct-to-LDS loads per stage
  static constexpr int RING = kWavesPerBlock * NS * STAGE;
  static constexpr int IDS = RING;                                  // int16 [entries]
  static constexpr int CNT = IDS + 2 * kDecodeMaxEntries;           // int32 [experts]
  static constexpr int REXP = CNT + 4 * kMaxExpertsTotal;           // int16 [experts]
  static constexpr int VSTART = REXP + 2 * kMaxExpertsTotal;        // int16 [experts + 1]
  static constexpr int MASK = VSTART + 2 * kMaxExpertsTotal + 16;   // uint32 [words]
  static constexpr int LISTS = MASK + 4 * kMaskWords;               // int32 [waves][2][TC]
  static constexpr int WTS = LISTS + 4 * kWavesPerBlock * 2 * TC;   // float [entries] (down)
  static constexpr int TOT = WTS + (DOWN ? 4 * kDecodeMaxEntries : 0);
  static constexpr int BYTES = TOT + 16;
  static_assert(XI >= 1 && TC * kMx4XBytes % 1024 == 0, "whole activation loads");
  static_assert(TC <= 16, "at most the MFMA's 16 columns");
  static_assert((NS - 2) * OPS < 64, "vmcnt range");
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ void dma16_lds(const void* src, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4_lds(const void* src, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
}
// Until at most N vector-memory operations of this wavefront are outstanding
// (they complete in issue order) and all its LDS reads have returned.
template <int N>
__device__ __forceinline__ void wait_vmem_and_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  asm volatile("" ::: "memory");
}
// LDS slot of 16-byte chunk c of row r inside a 128-byte slice: a bijection
// per row under which 16 consecutive rows reading one chunk hit distinct banks.
__device__ __forceinline__ int mx4_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Entries of expert e with rank [TC * pass, TC * (pass + 1)) in entry order
// -> list[0 .. TC).  Whole wavefront.
template <int TC>
__device__ __forceinline__ void pass_entries(const int16_t* s_ids, int n_entries, int e, int pass,
                                             int* list) {
  const int lane = threadIdx.x & (kWave - 1);
  int seen = 0;
  for (int b = 0; b < n_entries; b += kWave) {
    const int v = b + lane;
    const bool m = v < n_entries && s_ids[v] == e;
    const unsigned long long bm = __ballot(m);
    if (m) {
      const int r = seen + __popcll(bm & ((1ull << lane) - 1ull)) - TC * pass;
      if (r >= 0 && r < TC) list[r] = v;
    }
    seen += __popcll(bm);
  }
}

// Last rank r with vstart[r] <= v (uniform inputs; vstart strictly increases).
__device__ __forceinline__ int rank_of(const int16_t* vstart, int U, int v) {
  int lo = 0, hi = U - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (vstart[mid] <= v) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

template <int TC, int NS, bool DOWN, bool HBF16>
__global__ __launch_bounds__(kBlock) void mx4_mfma_kernel(const Mx4Args a) {
  using L = Mx4Lds<TC, NS, DOWN>;
  // one LDS array: the compiler then orders LDS reads against the
  // direct-to-LDS loads only through the explicit waits below
  __shared__ __attribute__((aligned(1024))) uint8_t lds[L::BYTES];
  int16_t* s_ids = reinterpret_cast<int16_t*>(lds + L::IDS);
  int* s_cnt = reinterpret_cast<int*>(lds + L::CNT);
  int16_t* s_rexp = reinterpret_cast<int16_t*>(lds + L::REXP);
  int16_t* s_vstart = reinterpret_cast<int16_t*>(lds + L::VSTART);
  uint32_t* s_mask = reinterpret_cast<uint32_t*>(lds + L::MASK);
  float* s_wts = reinterpret_cast<float*>(lds + L::WTS);
  int* s_tot = reinterpret_cast<int*>(lds + L::TOT);
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wv = wave_in_block();

  // ---- work map (whole workgroup): entry -> expert, entries per expert, the
  // touched experts in ascending order and each one's first virtual expert ----
  const int n_exp = a.n_words * 32;
  for (int q = tid; q < a.n_words; q += blockDim.x) s_mask[q] = 0;
  for (int e = tid; e < n_exp; e += blockDim.x) s_cnt[e] = 0;
  __syncthreads();
  for (int v = tid; v < a.n_entries; v += blockDim.x) {
    const int t = div_slots(v, a.slots_magic), j = v - t * a.slots;
    const int e = j < a.k ? clamp_expert(a.ids[t * a.k + j], a.E) : a.E;
    s_ids[v] = (int16_t)e;
    atomicOr(&s_mask[e >> 5], 1u << (e & 31));
    atomicAdd(&s_cnt[e], 1);
    // routing weights go to LDS too: a global load inside the loop below
    // would wait for every stage in flight (loads complete in issue order)
    if constexpr (DOWN) s_wts[v] = j < a.k ? a.wts[t * a.k + j] : 1.0f;
  }
  __syncthreads();
  if (wv == 0) {
    int rank0 = 0, v0 = 0;
    for (int e0 = 0; e0 < n_exp; e0 += kWave) {
      const int e = e0 + lane;
      const bool touched = e < n_exp && ((s_mask[e >> 5] >> (e & 31)) & 1u);
      const unsigned long long bm = __ballot(touched);
      const int r = rank0 + __popcll(bm & ((1ull << lane) - 1ull));
      const int p = touched ? (s_cnt[e] + TC - 1) / TC : 0;
      int incl = p;
      for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += y;
      }
      if (touched) {
        s_rexp[r] = (int16_t)e;
        s_vstart[r] = (int16_t)(v0 + incl - p);
      }
      v0 += __shfl(incl, kWave - 1, kWave);
      rank0 += __popcll(bm);
    }
    if (lane == 0) {
      s_vstart[rank0] = (int16_t)v0;
      s_tot[0] = rank0;
      s_tot[1] = v0;
    }
  }
  __syncthreads();
  const int U = s_tot[0];
  const int n_units = s_tot[1] * a.n_groups;
  const long long gw = (long long)blockIdx.x * kWavesPerBlock + wv;
  const long long nw = (long long)gridDim.x * kWavesPerBlock;
  const int u_first = (int)(gw * n_units / nw), u_end = (int)((gw + 1) * n_units / nw);
  if (u_first >= u_end) return;

  const int S = a.row_bytes / kMx4SliceBytes;   // stages per unit
  const int n = lane & 15, g = lane >> 4;       // MFMA column / K group of this lane
  const int scale_len = a.K >> 5;               // E8M0 bytes per row
  int* list_i = reinterpret_cast<int*>(lds + L::LISTS) + wv * 2 * TC;   // columns being loaded
  int* list_c = list_i + TC;                                            // columns being computed
  uint8_t* const ring = lds + wv * NS * L::STAGE;

  // Per-lane source offsets, fixed for the whole kernel.  Rows: load j fills
  // stage rows 8j .. 8j+7 (0-15 the first operand block, 16-31 the second),
  // lane -> row 8j + lane/8, LDS slot lane%8 holding chunk (lane%8) ^ swz(row).
  // Scales: lane -> row lane/2, dword lane%2 of the row's 8 bytes of the slice.
  uint32_t w_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 8 * j + (lane >> 3);
    w_off[j] = (uint32_t)(r & 15) * a.row_bytes + 16u * (uint32_t)((lane & 7) ^ mx4_swz(r));
  }
  const int s_row = lane >> 1, s_dw = lane & 1;

  // a unit's two 16-row blocks of expert e: gate / up rows of neurons
  // 16 grp .. 16 grp + 15, or rows 32 grp .. 32 grp + 31 of W_down
  auto row_block = [&](int e, int grp, int blk) -> long long {
    if constexpr (DOWN) return (long long)e * a.N + 32 * grp + 16 * blk;
    else return ((long long)e * 2 + blk) * a.N + 16 * grp;
  };

  // ---- load cursor ----
  int iu = u_first, is = 0, iv = -1, ie = 0, ihave = 0;
  bool idone = false;
  const uint8_t* iw0 = nullptr;
  const uint8_t* iw1 = nullptr;
  const uint8_t* i_scale = nullptr;
  const uint8_t* ix[L::XI];
  auto enter_unit_i = [&]() {
    const int v = iu / a.n_groups, grp = iu - v * a.n_groups;
    if (v != iv) {   // a new virtual expert: its columns
      iv = v;
      const int r = rank_of(s_vstart, U, v);
      ie = s_rexp[r];
      const int pass = v - s_vstart[r];
      ihave = min(s_cnt[ie] - TC * pass, TC);
      pass_entries<TC>(s_ids, a.n_entries, ie, pass, list_i);
      // activations: load j, lane -> column t = (64j + lane) / 32, piece
      // p = lane % 32 of its 512-byte slice, stored at piece slot p holding
      // piece p ^ (t % 16)
#pragma unroll
      for (int j = 0; j < L::XI; ++j) {
        const int idx = 64 * j + lane;
        const int t = idx >> 5, p = idx & 31;
        const int pe = list_i[t < ihave ? t : 0];
        const int row = DOWN ? pe : div_slots(pe, a.slots_magic);
        ix[j] = a.act + (size_t)row * a.K * 2 + 16 * (p ^ (t & 15));
      }
    }
    const long long r0 = row_block(ie, grp, 0), r1 = row_block(ie, grp, 1);
    iw0 = a.w + r0 * a.row_bytes;
    iw1 = a.w + r1 * a.row_bytes;
    i_scale = a.ws + ((s_row < 16 ? r0 : r1) + (s_row & 15)) * scale_len + 4 * s_dw;
  };
  enter_unit_i();

  // Every call issues L::OPS loads (after the last stage the cursor stays put
  // and the loads repeat its addresses, which are in L2), so the waits below
  // are exact.
  auto issue = [&](int q) {
    const uint32_t so = (uint32_t)is * kMx4SliceBytes;
    uint8_t* dst = ring + q * L::STAGE;
    dma16_lds(iw0 + so + w_off[0], dst);
    dma16_lds(iw0 + so + w_off[1], dst + 1024);
    dma16_lds(iw1 + so + w_off[2], dst + 2048);
    dma16_lds(iw1 + so + w_off[3], dst + 3072);
#pragma unroll
    for (int j = 0; j < L::XI; ++j)
      dma16_lds(ix[j] + (size_t)is * kMx4XBytes, dst + L::X + 1024 * j);
    dma4_lds(i_scale + 8 * is, dst + L::S);
    asm volatile("" ::: "memory");
    if (!idone && ++is == S) {
      if (iu + 1 < u_end) {
        is = 0;
        ++iu;
        enter_unit_i();
      } else {
        idone = true;
        is = S - 1;
      }
    }
  };

  // ---- compute cursor ----
  int cu = u_first, cs = 0, cv = -1, chave = 0, cgrp = 0;
  auto enter_unit_c = [&]() {
    const int v = cu / a.n_groups;
    cgrp = cu - v * a.n_groups;
    if (v != cv) {
      cv = v;
      const int r = rank_of(s_vstart, U, v);
      const int e = s_rexp[r];
      const int pass = v - s_vstart[r];
      chave = min(s_cnt[e] - TC * pass, TC);
      pass_entries<TC>(s_ids, a.n_entries, e, pass, list_c);
    }
  };
  enter_unit_c();

#pragma unroll
  for (int q = 0; q < NS - 1; ++q) issue(q);

  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  const int xt = n % TC;   // column slot this lane reads (columns >= TC repeat)
  bool cdone = false;
  while (!cdone) {
#pragma unroll
    for (int q = 0; q < NS; ++q) {
      if (cdone) break;
      wait_vmem_and_lds<(NS - 2) * L::OPS>();
      issue((q + NS - 1) % NS);
      const uint8_t* st = ring + q * L::STAGE;
      const uint32_t* sc = reinterpret_cast<const uint32_t*>(st + L::S);
      const uint8_t* xrow = st + L::X + xt * kMx4XBytes;
#pragma unroll
      for (int p = 0; p < 2; ++p) {            // operand blocks: rows 0-15, 16-31
        const int row = 16 * p + n;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int c = 4 * jj + g;            // 16-byte chunk: K 32c .. 32c+31 of the slice
          const u32x4 w = *reinterpret_cast<const u32x4*>(st + row * kMx4SliceBytes +
                                                          16 * (c ^ mx4_swz(row)));
          const float scl = e8m0_to_f32((sc[2 * row + (c >> 2)] >> (8 * (c & 3))) & 0xffu);
#pragma unroll
          for (int i = 0; i < 4; ++i) {        // dword i: K 32c + 8i .. 32c + 8i + 7
            const bf16x2 e0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scl, 0);
            const bf16x2 e1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scl, 1);
            const bf16x2 e2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scl, 2);
            const bf16x2 e3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scl, 3);
            const bf16x8 av = {e0[0], e0[1], e1[0], e1[1], e2[0], e2[1], e3[0], e3[1]};
            const int piece = 4 * c + i;
            const bf16x8 xv = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4*>(xrow + 16 * (piece ^ (xt & 15))));
            if (p == 0) acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, xv, acc0, 0, 0, 0);
            else acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, xv, acc1, 0, 0, 0);
          }
        }
      }
      if (++cs == S) {
        // lane (n, g) holds rows 4g .. 4g+3 of each operand block for column n
        cs = 0;
        if (n < chave) {
          const int pe = list_c[n];
          if constexpr (DOWN) {
            const float wt = s_wts[pe];
            float* o = reinterpret_cast<float*>(a.out) + (size_t)pe * a.N + 32 * cgrp + 4 * g;
            *reinterpret_cast<float4*>(o) =
                make_float4(__fmul_rn(acc0[0], wt), __fmul_rn(acc0[1], wt),
                            __fmul_rn(acc0[2], wt), __fmul_rn(acc0[3], wt));
            *reinterpret_cast<float4*>(o + 16) =
                make_float4(__fmul_rn(acc1[0], wt), __fmul_rn(acc1[1], wt),
                            __fmul_rn(acc1[2], wt), __fmul_rn(acc1[3], wt));
          } else {
            const size_t off = (size_t)pe * a.N + 16 * cgrp + 4 * g;
            float o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = swiglu(acc0[i], acc1[i]);
            if constexpr (HBF16) {
              const uint32_t lo = f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16);
              const uint32_t hi = f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16);
              *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + off) = make_uint2(lo, hi);
            } else {
              *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + off) =
                  make_float4(o[0], o[1], o[2], o[3]);
            }
          }
        }
        acc0 = f32x4{0.f, 0.f, 0.f, 0.f};
        acc1 = f32x4{0.f, 0.f, 0.f, 0.f};
        if (cu + 1 < u_end) {
          ++cu;
          enter_unit_c();
        } else {
          cdone = true;
        }
      }
    }
  }
  wait_vmem_and_lds<0>();   // no direct-to-LDS load may land after the wavefront ends
}

// Shapes they take: whole 16-neuron / 32-row units and whole 128-byte row
// slices of both matrices.
bool mx4_mfma_fits(const moe_weights& W) {
  return W.format == W_MXFP4 && W.inter % 256 == 0 && W.hidden % 256 == 0;
}

// Columns per pass and ring depth, from the expected entries per touched
// expert under uniform routing: 2 columns and a 6-stage ring for (nearly) one
// entry per expert, 8 and 4 up to four (one pass for almost every expert),
// 12 and 3 beyond.  Results do not depend on the choice.
int mx4_mode(const moe_weights& W, int T, int k) {
  const double n = W.num_experts;
  const double p = std::min(1.0, (double)k / n);
  const double u = n * (1.0 - std::pow(1.0 - p, (double)T)) + W.num_shared;
  const double per = (double)T * (k + W.num_shared) / std::max(1.0, u);
  return per <= 1.5 ? 0 : per <= 4.0 ? 1 : 2;
}

Mx4Args mx4_args_gate_up(const GateUpArgs& g) {
  Mx4Args m{};
  m.w = g.w13;
  m.ws = reinterpret_cast<const uint8_t*>(g.w13s);
  m.act = reinterpret_cast<const uint8_t*>(g.x);
  m.ids = g.ids;
  m.wts = nullptr;
  m.out = g.h;
  m.T = g.T, m.k = g.k, m.slots = g.slots, m.E = g.E, m.n_words = g.n_words;
  m.n_entries = g.n_entries;
  m.K = g.H, m.N = g.I, m.row_bytes = g.row_bytes, m.n_groups = g.I / 16;
  m.slots_magic = g.slots_magic;
  return m;
}

Mx4Args mx4_args_down(const DownArgs& d) {
  Mx4Args m{};
  m.w = d.w2;
  m.ws = reinterpret_cast<const uint8_t*>(d.w2s);
  m.act = reinterpret_cast<const uint8_t*>(d.h);
  m.ids = d.ids;
  m.wts = d.wts;
  m.out = d.y;   // the slot buffer
  m.T = d.T, m.k = d.k, m.slots = d.slots, m.E = d.E, m.n_words = d.n_words;
  m.n_entries = d.n_entries;
  m.K = d.I, m.N = d.H, m.row_bytes = d.row_bytes, m.n_groups = d.H / 32;
  m.slots_magic = d.slots_magic;
  return m;
}

template <bool DOWN, bool HBF16>
hipError_t launch_mx4(const Mx4Args& a, int mode, hipStream_t s) {
  // one persistent workgroup per CU (the stage ring takes most of the LDS)
  const dim3 g(device_num_cus()), b(kBlock);
  if (mode == 0) hipLaunchKernelGGL((mx4_mfma_kernel<2, 6, DOWN, HBF16>), g, b, 0, s, a);
  else if (mode == 1) hipLaunchKernelGGL((mx4_mfma_kernel<8, 4, DOWN, HBF16>), g, b, 0, s, a);
  else hipLaunchKernelGGL((mx4_mfma_kernel<12, 3, DOWN, HBF16>), g, b, 0, s, a);
  return hipGetLastError();
}

// Token-major: y[t][d] = sum over slots j (in order) of w_tj * dot(Wd[e_tj][d], h[t][j]).
// A workgroup owns one (token, output group); its 4 wavefronts take the slots
// j = w, w+4, ... and park w * dot in LDS; wavefront 0 adds them in slot order.
template <int FMT, int LPR, int CPL, bool HBF16, bool YBF16>
MOE_STREAM_KERNEL((h_regs<FMT, CPL, HBF16>() > 48 || CPL >= 12) ? 2 : 4) void down_token_kernel(const DownArgs a) {
  constexpr int ND = kWave / LPR;
  __shared__ float s_part[64][ND];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = wave_in_block();
  const int grp = lane / LPR, gl = lane % LPR;
  const int item = xcd_logical_block(blockIdx.x, gridDim.x, a.nxcd);
  const int dg = item / a.T;
  const int t = item - dg * a.T;
  const int d = dg * ND + grp;   // token-major items are one row per lane group
  const int dd = min(d, a.H - 1);

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
  for (int j = wv; j < a.slots; j += kWavesPerBlock) {
    DownRow<FMT, CPL> R[1];
    load_down_row<FMT, LPR, CPL>(R[0], a, __builtin_amdgcn_readlane(my_e, j), dd, gl, false);
    float dot[1];
    down_rows_dot<FMT, LPR, CPL, 1, HBF16>(R, a, t * a.slots + j, gl, dot);
    if (gl == 0) s_part[j][grp] = __fmul_rn(dot[0], lane_value(my_w, j));
  }
  __syncthreads();
  if (wv == 0 && gl == 0 && d < a.H) {
    float y = 0.f;
    for (int j = 0; j < a.slots; ++j) y = __fadd_rn(y, s_part[j][grp]);
    const size_t off = (size_t)t * a.H + d;
    if constexpr (YBF16) {
      reinterpret_cast<uint16_t*>(a.y)[off] = (uint16_t)f32_to_bf16_bits(y);
    } else {
      reinterpret_cast<float*>(a.y)[off] = y;
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

// Shapes the launch rules below can pick (two neurons per wavefront only
// while a row is at most two chunks per lane, BF16 rows only up to four);
// nothing else is compiled.
template <int NR, int MCH, bool PRE>
constexpr bool gate_up_shape_ok() { return (NR == 1 || MCH <= 2) && (!PRE || MCH <= 4); }

template <int FMT, int NR, bool PRE, bool XF32, bool HBF16>
hipError_t gate_up_mch(const GateUpArgs& a, int mch, bool guard, int blocks, hipStream_t s) {
  dim3 g(blocks), b(kBlock);
#define MOE_GU(M, G)                                                                         \
  do {                                                                                       \
    if constexpr (!gate_up_shape_ok<NR, M, PRE>())                                           \
      return hipErrorNotSupported;                                                           \
    else if constexpr (gate_scales_by_dword<FMT, NR, M, G>()) {                              \
      if (a.sscl)                                                                            \
        hipLaunchKernelGGL((gate_up_decode_kernel<FMT, NR, M, PRE, XF32, HBF16, G, true>), g, b, \
                           0, s, a);                                                         \
      else                                                                                   \
        hipLaunchKernelGGL((gate_up_decode_kernel<FMT, NR, M, PRE, XF32, HBF16, G, false>), g, \
                           b, 0, s, a);                                                      \
    } else                                                                                   \
      hipLaunchKernelGGL((gate_up_decode_kernel<FMT, NR, M, PRE, XF32, HBF16, G, false>), g, b, 0, \
                         s, a);                                                              \
  } while (0)
  if (!guard) {
    switch (mch) {
      case 1: MOE_GU(1, false); break;
      case 2: MOE_GU(2, false); break;
      case 4: MOE_GU(4, false); break;
      case 7: MOE_GU(7, false); break;
      case 8: MOE_GU(8, false); break;
      default: return hipErrorNotSupported;
    }
  } else {
    switch (mch) {
      case 1: MOE_GU(1, true); break;
      case 2: MOE_GU(2, true); break;
      case 4: MOE_GU(4, true); break;
      case 8: MOE_GU(8, true); break;
      default: return hipErrorNotSupported;
    }
  }
#undef MOE_GU
  return hipGetLastError();
}

template <int FMT, bool XF32, bool HBF16>
hipError_t gate_up_nr(const GateUpArgs& a, int nr, bool pre, int mch, bool guard, int blocks,
                      hipStream_t s) {
  if constexpr (FMT == W_F32) {
    if (nr == 1) return gate_up_mch<FMT, 1, false, XF32, HBF16>(a, mch, guard, blocks, s);
    return gate_up_mch<FMT, 2, false, XF32, HBF16>(a, mch, guard, blocks, s);
  } else {
    if (nr == 1)
      return pre ? gate_up_mch<FMT, 1, true, XF32, HBF16>(a, mch, guard, blocks, s)
                 : gate_up_mch<FMT, 1, false, XF32, HBF16>(a, mch, guard, blocks, s);
    return pre ? gate_up_mch<FMT, 2, true, XF32, HBF16>(a, mch, guard, blocks, s)
               : gate_up_mch<FMT, 2, false, XF32, HBF16>(a, mch, guard, blocks, s);
  }
}

template <int FMT, int LPR, int CPL, bool HBF16>
hipError_t down_launch(const DownArgs& a, int variant, int ybf16, int blocks, hipStream_t s) {
  dim3 g(blocks), b(kBlock);
  const bool expert_major = variant == kDownExpertMajor;
  // rows per lane group as the register rule allows (4 up to 3 chunks per
  // lane, 2 up to 4); nothing wider is compiled.  E4M3 rows with BF16 h take
  // the kernel that converts each item's rows once.
  if constexpr ((FMT == W_MXFP8 || FMT == W_FP8B128) && HBF16 && CPL <= 4) {
    if (expert_major && (a.rpl == 4 || a.rpl == 2)) {
      constexpr bool kCanStage = FMT == W_MXFP8;
      if constexpr (CPL <= 3) {
        if (a.rpl == 4) {
          if (kCanStage && a.sscl)
            hipLaunchKernelGGL((down_expert_pre_kernel<FMT, LPR, CPL, 4, kCanStage>), g, b, 0, s, a);
          else
            hipLaunchKernelGGL((down_expert_pre_kernel<FMT, LPR, CPL, 4, false>), g, b, 0, s, a);
          return hipGetLastError();
        }
      }
      if (kCanStage && a.sscl)
        hipLaunchKernelGGL((down_expert_pre_kernel<FMT, LPR, CPL, 2, kCanStage>), g, b, 0, s, a);
      else
        hipLaunchKernelGGL((down_expert_pre_kernel<FMT, LPR, CPL, 2, false>), g, b, 0, s, a);
      return hipGetLastError();
    }
  }
  if constexpr (CPL <= 3) {
    if (expert_major && a.rpl == 4) {
      hipLaunchKernelGGL((down_expert_kernel<FMT, LPR, CPL, 4, HBF16>), g, b, 0, s, a);
      return hipGetLastError();
    }
  }
  if constexpr (CPL <= 4) {
    if (expert_major && a.rpl == 2) {
      hipLaunchKernelGGL((down_expert_kernel<FMT, LPR, CPL, 2, HBF16>), g, b, 0, s, a);
      return hipGetLastError();
    }
  }
  if (expert_major)
    hipLaunchKernelGGL((down_expert_kernel<FMT, LPR, CPL, 1, HBF16>), g, b, 0, s, a);
  else if (ybf16)
    hipLaunchKernelGGL((down_token_kernel<FMT, LPR, CPL, HBF16, true>), g, b, 0, s, a);
  else
    hipLaunchKernelGGL((down_token_kernel<FMT, LPR, CPL, HBF16, false>), g, b, 0, s, a);
  return hipGetLastError();
}

template <int FMT, int LPR, bool HBF16>
hipError_t down_cpl(const DownArgs& a, int em, int ybf16, int blocks, hipStream_t s) {
  switch (a.cpl) {
    case 2: return down_launch<FMT, LPR, 2, HBF16>(a, em, ybf16, blocks, s);
    case 3: return down_launch<FMT, LPR, 3, HBF16>(a, em, ybf16, blocks, s);
    case 4: return down_launch<FMT, LPR, 4, HBF16>(a, em, ybf16, blocks, s);
    case 6: return down_launch<FMT, LPR, 6, HBF16>(a, em, ybf16, blocks, s);
    case 8: return down_launch<FMT, LPR, 8, HBF16>(a, em, ybf16, blocks, s);
    case 12: return down_launch<FMT, LPR, 12, HBF16>(a, em, ybf16, blocks, s);
    case 16: return down_launch<FMT, LPR, 16, HBF16>(a, em, ybf16, blocks, s);
    default: return hipErrorNotSupported;
  }
}

template <int FMT, bool HBF16>
hipError_t down_shape(const DownArgs& a, int lpr, int em, int ybf16, int blocks, hipStream_t s) {
  if (lpr == 4) return down_cpl<FMT, 4, HBF16>(a, em, ybf16, blocks, s);
  if (lpr == 8) return down_cpl<FMT, 8, HBF16>(a, em, ybf16, blocks, s);
  if (lpr == 16) return down_cpl<FMT, 16, HBF16>(a, em, ybf16, blocks, s);
  return down_cpl<FMT, 32, HBF16>(a, em, ybf16, blocks, s);
}

}  // namespace

// ---- host planning: every refusal is decided here, before any launch -----

namespace {

int lanes_per_row_for(int fmt, int inter, int h_dtype) {
  const int chunks = row_bytes_of(fmt, inter) / 16;
  const int elems = fmt == W_F32 ? 4 : fmt == W_MXFP4 ? 32 : 16;
  const int hwords = elems * (h_dtype == MOE_DT_BF16 ? 2 : 4) / 4;
  auto inst = [&](int lpr) {
    if (chunks % lpr) return false;
    const int c = chunks / lpr;
    return c == 2 || c == 3 || c == 4 || c == 6 || c == 8 || c == 12 || c == 16;
  };
  for (int lpr : {4, 8, 16, 32}) {
    const int c = chunks / lpr;
    if (inst(lpr) && (lpr >= 8 || chunks < 16) && 2 * c * 5 + c * hwords <= 80) return lpr;
  }
  for (int budget = 48; budget <= 128; budget *= 2)
    for (int lpr : {4, 8, 16, 32})
      if (inst(lpr) && (lpr >= 8 || chunks < 16) && (chunks / lpr) * hwords <= budget) return lpr;
  return 0;
}

struct GateUpPlan {
  GateUpArgs a;
  int nr, mch, blocks;
  bool pre, guard;
};

struct DownPlan {
  DownArgs a;
  int lpr, blocks;
  int variant;     // kDownTokenMajor or kDownExpertMajor
};

hipError_t plan_gate_up(const moe_weights& W, const void* x, const int32_t* ids, int T, int k,
                        void* h, GateUpPlan& p) {
  GateUpArgs& a = p.a;
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
  if (a.n_entries > kDecodeMaxEntries) return hipErrorNotSupported;
  // chunks per lane: exact when the row is a whole number of 64-lane passes
  // (loads then batch without guards), else the next instantiated size
  const int lane_chunks = (a.chunks + kWave - 1) / kWave;
  if (lane_chunks > 8) return hipErrorNotSupported;
  p.guard = a.chunks % kWave != 0 ||
            !(lane_chunks == 1 || lane_chunks == 2 || lane_chunks == 4 || lane_chunks == 7 ||
              lane_chunks == 8);
  p.mch = !p.guard ? lane_chunks
                   : lane_chunks <= 1 ? 1 : lane_chunks <= 2 ? 2 : lane_chunks <= 4 ? 4 : 8;
  // neurons per wavefront: two while the rows stay small in registers; rows
  // converted to BF16 once per item while that takes at most 64 VGPRs
  p.nr = p.mch <= 2 ? 2 : 1;
  const int elems = W.format == W_MXFP4 ? 32 : 16;
  p.pre = W.format != W_F32 && p.mch <= 4 && 2 * p.nr * p.mch * elems / 2 <= 64;
  a.slots_magic = (uint32_t)(((1ull << 32) + a.slots - 1) / a.slots);
  a.n_groups = (W.inter + p.nr - 1) / p.nr;
  // neuron pairs never straddle the end of I, and the scales load as dwords
  a.sscl = W.format == W_MXFP8 && W.inter % 2 == 0 &&
           (reinterpret_cast<uintptr_t>(W.w13_scale) & 3) == 0;
  const long long max_items = (long long)std::min(n_exp, a.n_entries) * a.n_groups;
  const long long want = (max_items + kWavesPerBlock - 1) / kWavesPerBlock;
  p.blocks = (int)std::max<long long>(1, std::min<long long>(want, device_num_cus() * 16LL));
  return hipSuccess;
}

}  // namespace

hipError_t launch_gate_up_decode(const moe_weights& W, const void* x, int x_dtype,
                                 const int32_t* ids, int T, int k, void* h, int h_dtype,
                                 hipStream_t s) {
  GateUpPlan p;
  hipError_t e = plan_gate_up(W, x, ids, T, k, h, p);
  if (e != hipSuccess) return e;
  const GateUpArgs& a = p.a;
  const bool xf32 = x_dtype == MOE_DT_F32;
  const bool hbf = h_dtype == MOE_DT_BF16;
  const int nr = p.nr, mch = p.mch, blocks = p.blocks;
  const bool pre = p.pre, guard = p.guard;
  switch (W.format) {
    case W_F32:
      if (xf32) return hbf ? gate_up_nr<W_F32, true, true>(a, nr, pre, mch, guard, blocks, s)
                           : gate_up_nr<W_F32, true, false>(a, nr, pre, mch, guard, blocks, s);
      return hbf ? gate_up_nr<W_F32, false, true>(a, nr, pre, mch, guard, blocks, s)
                 : gate_up_nr<W_F32, false, false>(a, nr, pre, mch, guard, blocks, s);
    case W_MXFP8:
      return hbf ? gate_up_nr<W_MXFP8, false, true>(a, nr, pre, mch, guard, blocks, s)
                 : gate_up_nr<W_MXFP8, false, false>(a, nr, pre, mch, guard, blocks, s);
    case W_MXFP4:
      if (!xf32 && mx4_mfma_fits(W)) {
        const Mx4Args m = mx4_args_gate_up(a);
        return hbf ? launch_mx4<false, true>(m, mx4_mode(W, T, k), s)
                   : launch_mx4<false, false>(m, mx4_mode(W, T, k), s);
      }
      return hbf ? gate_up_nr<W_MXFP4, false, true>(a, nr, pre, mch, guard, blocks, s)
                 : gate_up_nr<W_MXFP4, false, false>(a, nr, pre, mch, guard, blocks, s);
    case W_FP8B128:
      return hbf ? gate_up_nr<W_FP8B128, false, true>(a, nr, pre, mch, guard, blocks, s)
                 : gate_up_nr<W_FP8B128, false, false>(a, nr, pre, mch, guard, blocks, s);
    default:
      return hipErrorInvalidValue;
  }
}

// Lanes that share one W_down row.  It depends only on the format, the row
// length and the h dtype (both down variants use it, so their bits agree):
// the fewest lanes such that the row splits into an instantiated number of
// chunks per lane and two rows per lane group fit the register budget
// (weights + scales ~5 VGPRs per chunk, plus the staged h chunks); failing
// that, one row per group with at most 48 (then 96) VGPRs of h.  0 if none.
int down_lanes_per_row(int fmt, int inter, int h_dtype) {
  return lanes_per_row_for(fmt, inter, h_dtype);
}

namespace {

hipError_t plan_down(const moe_weights& W, const void* h, int h_dtype, const int32_t* ids,
                     const float* wts, int T, int k, void* y, int variant, float* slot_out,
                     DownPlan& p) {
  DownArgs& a = p.a;
  a.w2 = reinterpret_cast<const uint8_t*>(W.w2);
  a.w2s = W.w2_scale;
  a.h = h;
  a.ids = ids;
  a.wts = wts;
  a.T = T;
  a.k = k;
  a.slots = k + W.num_shared;
  a.E = W.num_experts;
  a.H = W.hidden;
  a.I = W.inter;
  a.row_bytes = row_bytes_of(W.format, W.inter);
  a.chunks = a.row_bytes / 16;
  // one slot per lane in the token-major kernel
  if (a.slots > kWave) return hipErrorNotSupported;
  if (variant == kDownExpertMajor && slot_out == nullptr) return hipErrorInvalidValue;
  p.variant = variant;
  const bool em = variant == kDownExpertMajor;
  p.lpr = lanes_per_row_for(W.format, W.inter, h_dtype);
  if (p.lpr == 0) return hipErrorNotSupported;
  // row offsets inside one expert are 32-bit in the kernels
  if ((long long)a.H * a.row_bytes >= (1ll << 32)) return hipErrorNotSupported;
  a.n_entries = T * a.slots;
  // the expert-major kernel stages the routed ids on chip
  if (em && a.n_entries > kDecodeMaxEntries) return hipErrorNotSupported;
  a.cpl = a.chunks / p.lpr;
  const int nd = kWave / p.lpr;
  a.slots_magic = (uint32_t)(((1ull << 32) + a.slots - 1) / a.slots);
  // two or four rows per lane group in the expert-major kernel (more bytes in
  // flight per item, each staged h chunk used for every row) as the register
  // budget allows, within the compiled shapes
  const int elems = W.format == W_F32 ? 4 : W.format == W_MXFP4 ? 32 : 16;
  const int hregs = a.cpl * elems * (h_dtype == MOE_DT_BF16 ? 2 : 4) / 4;
  const int rpl_fit = 4 * a.cpl * 5 + hregs <= 96 ? 4 : 2 * a.cpl * 5 + hregs <= 80 ? 2 : 1;
  const int rpl_max = a.cpl <= 3 ? 4 : a.cpl <= 4 ? 2 : 1;
  a.rpl = em ? std::min(rpl_fit, rpl_max) : 1;
  a.n_dgroups = (W.hidden + nd * a.rpl - 1) / (nd * a.rpl);
  {
    // an item's rows' E8M0 scales as one 16-byte-aligned run (see
    // down_expert_pre_kernel)
    const long long run = (long long)nd * a.rpl * (W.inter / 32);
    a.sscl = W.format == W_MXFP8 && em && W.hidden % (nd * a.rpl) == 0 && run % 16 == 0 &&
             run <= 1024 && (reinterpret_cast<uintptr_t>(W.w2_scale) & 15) == 0;
  }
  const int n_exp = W.num_experts + W.num_shared;
  a.n_words = (n_exp + 31) / 32;
  a.nxcd = device_num_xcds();
  if (em) {
    a.y = slot_out;
    const long long max_items = (long long)std::min(n_exp, a.n_entries) * a.n_dgroups;
    const long long want = (max_items + kWavesPerBlock - 1) / kWavesPerBlock;
    p.blocks = (int)std::max<long long>(1, std::min<long long>(want, device_num_cus() * 8LL));
  } else {
    a.y = y;
    const long long blocks = (long long)T * a.n_dgroups;   // one workgroup per (token, output group)
    if (blocks > 0x7fffffffLL) return hipErrorNotSupported;
    p.blocks = (int)blocks;
  }
  return hipSuccess;
}

}  // namespace

// AUTO: token-major for small batches, expert-major from a number of routed
// entries on (within the entries it stages).  The token-major kernel reads a
// routed expert's rows once per (token, slot), from L2 after the first, and a
// wavefront holds 64/LPR rows of one entry; the expert-major kernel reads them
// once per call and holds 64/LPR x 2-4 rows, at the price of the slot buffer
// and the combine kernel.  The crossover follows the lanes per row (BF16 h;
// FP32 h with FP32 weights).  Measured, down alone, graph-replayed, MI355X,
// token-major / expert-major:
//  * 16 lanes per row (Qwen3-style layer, I = 768): 13 tokens 29.1 / 29.4 us,
//    14 tokens 30.8 / 30.3 us, 16 tokens 35.0 / 32.2, 32 tokens 56.6 / 44.1:
//    expert-major from 112 entries;
//  * 32 lanes per row (MXFP8, I = 1536: 2 tokens 22.3 / 24.4 us, 4 tokens
//    37.5 / 34.0; DeepSeek-V3-shaped, 9 slots: 1 token 29.2 / 30.2, 2 tokens
//    52.4 / 48.5): expert-major from 18 entries.
// The two give identical bits, so the switch does not change any result.
// MXFP4 rows that fit the matrix-core kernel take expert-major at every batch
// size, so that a token's y does not change with the batch size there either.
int down_variant_for(const moe_weights& W, int T, int k) {
  const long long entries = (long long)T * (k + W.num_shared);
  if (entries > kDecodeMaxEntries) return kDownTokenMajor;
  if (mx4_mfma_fits(W)) return kDownExpertMajor;
  const int lpr = lanes_per_row_for(W.format, W.inter, W.format == W_F32 ? MOE_DT_F32 : MOE_DT_BF16);
  return entries >= (lpr >= 32 ? 18 : 112) ? kDownExpertMajor : kDownTokenMajor;
}

hipError_t launch_down_decode(const moe_weights& W, const void* h, int h_dtype,
                              const int32_t* ids, const float* wts, int T, int k, void* y,
                              int y_dtype, int variant, float* slot_out, hipStream_t s) {
  if (variant == MOE_DOWN_AUTO) variant = down_variant_for(W, T, k);
  DownPlan p;
  hipError_t err = plan_down(W, h, h_dtype, ids, wts, T, k, y, variant, slot_out, p);
  if (err != hipSuccess) return err;
  const DownArgs& a = p.a;
  const bool hbf = h_dtype == MOE_DT_BF16;
  const int ybf = y_dtype == MOE_DT_BF16;
  const int em = p.variant;
  switch (W.format) {
    case W_F32:
      err = hbf ? down_shape<W_F32, true>(a, p.lpr, em, ybf, p.blocks, s)
                : down_shape<W_F32, false>(a, p.lpr, em, ybf, p.blocks, s);
      break;
    case W_MXFP8:
      err = hbf ? down_shape<W_MXFP8, true>(a, p.lpr, em, ybf, p.blocks, s)
                : down_shape<W_MXFP8, false>(a, p.lpr, em, ybf, p.blocks, s);
      break;
    case W_MXFP4:
      if (hbf && em == kDownExpertMajor && mx4_mfma_fits(W)) {
        err = launch_mx4<true, false>(mx4_args_down(a), mx4_mode(W, T, k), s);
      } else {
        err = hbf ? down_shape<W_MXFP4, true>(a, p.lpr, em, ybf, p.blocks, s)
                  : down_shape<W_MXFP4, false>(a, p.lpr, em, ybf, p.blocks, s);
      }
      break;
    case W_FP8B128:
      err = hbf ? down_shape<W_FP8B128, true>(a, p.lpr, em, ybf, p.blocks, s)
                : down_shape<W_FP8B128, false>(a, p.lpr, em, ybf, p.blocks, s);
      break;
    default:
      return hipErrorInvalidValue;
  }
  if (err != hipSuccess || p.variant != kDownExpertMajor) return err;
  return launch_combine(slot_out, MOE_DT_F32, T, a.slots, W.hidden, y, y_dtype, s);
}

hipError_t decode_supported(const moe_weights& W, int T, int k, int h_dtype) {
  GateUpPlan g;
  hipError_t e = plan_gate_up(W, nullptr, nullptr, T, k, nullptr, g);
  if (e != hipSuccess) return e;
  DownPlan d;
  static float slot_dummy;   // stands for a slot buffer; nothing is launched
  return plan_down(W, nullptr, h_dtype, nullptr, nullptr, T, k, nullptr, down_variant_for(W, T, k),
                   &slot_dummy, d);
}

int down_auto_variant(const moe_weights& W, int T, int k) { return down_variant_for(W, T, k); }

bool decode_on_matrix_cores(const moe_weights& W) { return mx4_mfma_fits(W); }

// Expected number of passes (virtual experts) of the matrix-core kernels
// under uniform routing: each expert's entry count is Binomial(T, k/E), and an
// expert with c entries takes ceil(c / TC) passes; shared experts take every
// token.
double decode_matrix_core_passes(const moe_weights& W, int T, int k) {
  static const int kTc[3] = {2, 8, 12};
  const int tc = kTc[mx4_mode(W, T, k)];
  const double p = std::min(1.0, (double)k / W.num_experts);
  const double all = (double)((T + tc - 1) / tc);   // passes of an expert every token uses
  double per = all;
  if (p < 1.0) {
    per = 0.0;
    double pmf = std::pow(1.0 - p, (double)T);         // P(c = 0)
    for (int c = 1; c <= T; ++c) {
      pmf *= (double)(T - c + 1) / c * (p / (1.0 - p));
      per += pmf * ((c + tc - 1) / tc);
    }
  }
  return W.num_experts * per + W.num_shared * all;
}

}  // namespace moe
