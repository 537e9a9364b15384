// Internal host interface between the C ABI layer (api.hip) and the kernel
// translation units.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_mi355x.h"

namespace moe {

constexpr int kDecodeMaxEntries = 2048;   // T * slots staged in LDS by gate_up
constexpr int kMaxExpertsTotal = 1024;    // E + S

int device_num_cus();
int device_num_xcds();

// decode.hip
hipError_t launch_gate_up_decode(const moe_weights& W, const void* x, int x_dtype,
                                 const int32_t* ids, int T, int k, void* h, int h_dtype,
                                 hipStream_t s);
// variant: a moe_down_variant; MOE_DOWN_AUTO picks one.  The expert-major
// variant needs slot_out (T*slots*H floats); all variants give identical bits.
hipError_t launch_down_decode(const moe_weights& W, const void* h, int h_dtype,
                              const int32_t* ids, const float* wts, int T, int k, void* y,
                              int y_dtype, int variant, float* slot_out, hipStream_t s);
int down_lanes_per_row(int fmt, int inter, int h_dtype);
// hipSuccess if both decode kernels accept this shape (the down kernel in the
// variant MOE_DOWN_AUTO picks), else hipErrorNotSupported; launches nothing
hipError_t decode_supported(const moe_weights& W, int T, int k, int h_dtype);
// the moe_down_variant MOE_DOWN_AUTO runs for T tokens
int down_auto_variant(const moe_weights& W, int T, int k);
// MXFP4 decode runs on the matrix cores for these weights; expected passes
// over the touched experts' rows at T tokens (path-choice model).
bool decode_on_matrix_cores(const moe_weights& W);
double decode_matrix_core_passes(const moe_weights& W, int T, int k);

// align_sort.hip
size_t align_sort_workspace_bytes(int n_entries, int n_experts);
hipError_t launch_align_sort(const int32_t* ids, int T, int k, int E, int S, int bs,
                             int32_t* sorted, int32_t* expert_ids, int32_t* offsets,
                             int32_t* npp, void* ws, hipStream_t s);
// moe_layer's grouped front end: the align-sort above and the MXFP8
// quantisation of the token rows (launch_quant_rows), as one launch up to the
// single-workgroup sort's entry limit, else the separate launches
hipError_t launch_front_end(const int32_t* ids, int T, int k, int E, int S, int bs,
                            int32_t* sorted, int32_t* expert_ids, int32_t* offsets, int32_t* npp,
                            void* ws, const void* x, int x_dtype, int H, uint8_t* xq, uint8_t* xs,
                            hipStream_t s);

// grouped.hip
hipError_t launch_quant_rows(const void* x, int x_dtype, int T, int H, uint8_t* xq, uint8_t* xs,
                             hipStream_t s);
hipError_t launch_grouped_gate_up(const moe_weights& W, const uint8_t* xq, const uint8_t* xs,
                                  int T, int slots, const int32_t* sorted,
                                  const int32_t* expert_ids, const int32_t* npp, int capacity,
                                  int bs, uint8_t* hq, uint8_t* hs, hipStream_t s);
hipError_t launch_grouped_down(const moe_weights& W, const uint8_t* hq, const uint8_t* hs,
                               const int32_t* sorted, const int32_t* expert_ids,
                               const int32_t* npp, int capacity, int bs, const float* wts,
                               int T, int k, uint16_t* slot_out, hipStream_t s);
hipError_t launch_topk_route(const float* scores, const float* bias, int T, int E, int k,
                             int32_t* ids, float* wts, hipStream_t s);
// out[0] = ids outside [0, E) among ids[0 .. n), out[1] = the first (-1: none)
hipError_t launch_check_routing(const int32_t* ids, int n, int E, int32_t* out, hipStream_t s);
// slot_dtype MOE_DT_F32 (decode path) or MOE_DT_BF16 (grouped path)
hipError_t launch_combine(const void* slot_out, int slot_dtype, int T, int slots, int H, void* y,
                          int y_dtype, hipStream_t s);

// util.hip
hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t s);
hipError_t launch_read(const void* src, size_t bytes, float* sink, hipStream_t s);
hipError_t launch_fill(void* dst, size_t bytes, uint32_t value, hipStream_t s);
constexpr int kReadSinkLen = 4096;

}  // namespace moe
