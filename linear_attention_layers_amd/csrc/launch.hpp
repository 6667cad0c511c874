// Host-side launchers of the GDN kernels (internal to libgdn.so).  Arguments
// are validated by api.cpp before these are called; each returns the HIP
// status of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gdn.h"

namespace gdn {

hipError_t launch_make_chunks(const int32_t* cu, int nseq, int chunk_len, gdn_chunk* out,
                              int cap, hipStream_t st);

hipError_t launch_conv(const void* x, int64_t xs, int act, const float* w, const float* bias,
                       float* conv_state, const uint8_t* has_init, const int32_t* cu,
                       const gdn_chunk* chunks, int nchunks, int nseq, int C, int write_state, void* y,
                       hipStream_t st);
// The conv with the post-conv step fused (q, k, v written instead of y;
// bitwise equal to launch_conv followed by the post-conv with out = act).
hipError_t launch_conv_postconv(const void* x, int64_t xs, int act, const float* w, const float* bias,
                                float* conv_state, const uint8_t* has_init, const int32_t* cu,
                                const gdn_chunk* chunks, int nchunks, int nseq, int Hk, int Hv, float eps,
                                int write_state, void* q, void* k, void* v, hipStream_t st);

hipError_t launch_gates(const void* ba, int gate_act, const float* A_log, const float* dt_bias, int rows,
                        int Hv, float* g, float* beta, hipStream_t st);
hipError_t launch_out_norm(const void* o, const void* z, int act, const float* w, int rows, float eps,
                           void* y, hipStream_t st);
hipError_t launch_postconv(const void* y, int64_t ys, int in, int N, int Hk, int Hv, float eps,
                           void* q, void* k, void* v, int out, hipStream_t st);

hipError_t launch_step(const void* q, const void* k, const void* v, int act, const float* g,
                       const float* beta, const int32_t* cu, int nseq, int Hk, int Hv,
                       float* state, const uint8_t* has_init, void* o, int commit_state,
                       hipStream_t st);

hipError_t launch_decode_fused(const void* x, int64_t xs, int act, const float* w, const float* bias,
                               float* conv_state, const int32_t* cu, int nseq, int Hk, int Hv, float eps,
                               const float* g, const float* beta, float* state, const uint8_t* has_init,
                               void* o, void* k_out, void* v_out, int write_conv_state, int commit_state,
                               hipStream_t st);
hipError_t launch_commit(const gdn_layer_io* layers, int L, const int32_t* cu,
                         const int32_t* n_keep, const uint8_t* has_init, int nseq, int C,
                         int Hk, int Hv, int act, hipStream_t st);

// Segment-parallel prefill (bf16 activations): two passes of the
// warp-specialised prefill with the segment chain between them; ws holds
// 3 * nseq * nseg * Hv float32 128 x 128 matrices.
hipError_t launch_prefill_segmented(const void* q, const void* k, const void* v, const float* g,
                                    const float* beta, const int32_t* cu, int nseq, int Hk, int Hv,
                                    float* state, const uint8_t* has_init, void* o, int nseg,
                                    float* ws, hipStream_t st);
// Device address of the no-allocation scratch (GDN_NOALLOC_SCRATCH_BYTES)
// on the stream's device (the current device for a NULL stream), looked up
// once per device.
hipError_t noalloc_scratch(hipStream_t st, float** out);
hipError_t launch_prefill(const void* q, const void* k, const void* v, int act, const float* g,
                          const float* beta, const int32_t* cu, int nseq, int Hk, int Hv,
                          float* state, const uint8_t* has_init, void* o, hipStream_t st);

}  // namespace gdn
