// Host-side launcher interface between the C ABI (api.hip) and the kernel files.
#pragma once

#include <stdint.h>
#include <type_traits>
#include <hip/hip_runtime_api.h>

#include "linattn.h"

namespace la {

struct PrefillArgs {
    const void *Q, *K, *V, *alpha;
    int64_t n_heads;  // B * H
    int64_t T;
    int32_t d, dv;
    double eps;
    int32_t chunk;
    void *Y, *S, *z;
    int phi = LA_PHI_ELU1;  // an la_feature_map
};

struct DecodeArgs {
    const void *q, *k, *v, *alpha;
    int64_t n_states;
    int32_t d, dv;
    double eps;
    void *y, *S, *z;
    int phi = LA_PHI_ELU1;  // an la_feature_map
};

struct DeltaArgs {
    const void *q, *k, *v, *beta;
    int64_t n_states;
    int32_t d, dv;
    void *y, *S;
};

struct SoftmaxDecodeArgs {
    const void *q, *k, *v;
    int64_t n_heads;
    int32_t d, dv;
    int64_t pos, capacity;
    void *K_cache, *V_cache;
    double scale;
    void *y;
    void *workspace;
};

// Calls f(std::integral_constant<int, FM>{}) for the feature map `phi` (an
// la_feature_map the C ABI has already checked), so launchers pick a kernel
// instantiation per map.
template <typename F>
hipError_t dispatch_feature_map(int phi, F &&f)
{
    switch (phi) {
    case LA_PHI_RELU1:
        return f(std::integral_constant<int, LA_PHI_RELU1>{});
    case LA_PHI_RELU_EPS:
        return f(std::integral_constant<int, LA_PHI_RELU_EPS>{});
    case LA_PHI_SIGMOID_EPS:
        return f(std::integral_constant<int, LA_PHI_SIGMOID_EPS>{});
    default:
        return f(std::integral_constant<int, LA_PHI_ELU1>{});
    }
}

// Each launcher enqueues its kernels on `stream` and returns the HIP status of
// the launch (hipSuccess or the runtime's refusal).  Arguments are already valid.
hipError_t launch_state_init(void *S, void *z, int64_t n_states, int32_t r, int32_t dv,
                             la_dtype state_dtype, hipStream_t stream);
hipError_t launch_prefill_general(const PrefillArgs &a, la_dtype io_dtype, hipStream_t stream);
hipError_t launch_prefill_mfma_bf16(const PrefillArgs &a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, la_dtype io_dtype, hipStream_t stream);
// Non-causal form (PrefillArgs without alpha and chunk): S, z += the whole sequence,
// then every query reads the final state.
hipError_t launch_noncausal_general(const PrefillArgs &a, la_dtype io_dtype, hipStream_t stream);
hipError_t launch_noncausal_mfma_bf16(const PrefillArgs &a, hipStream_t stream);
hipError_t launch_delta_decode(const DeltaArgs &a, la_dtype io_dtype, hipStream_t stream);
hipError_t launch_softmax_decode(const SoftmaxDecodeArgs &a, la_dtype io_dtype, hipStream_t stream);
// history pieces (workgroups per head) of the softmax decode for L attended rows
int64_t softmax_decode_splits(int64_t L);
// Device address of the softmax decode's fixed scratch array on the current device
// (LA_SOFTMAX_STATIC_WORKSPACE_BYTES bytes), looked up once per device.
hipError_t softmax_static_workspace(void **ptr);

// True when the bf16 MFMA prefill kernel handles the request.
bool mfma_prefill_supported(la_dtype io_dtype, int32_t d, int32_t dv, int32_t chunk);
// The MFMA prefills' cut of each sequence into segments (chunk 64 or 128; rows of row_bytes
// bytes of Q; a state slot of slot_bytes): false when the grid would not fit a launch.
bool plan_segments(int64_t n_heads, int64_t T, int32_t chunk, int64_t row_bytes, int64_t slot_bytes, int64_t *nseg,
                   int64_t *seg_len);
// True when the fp32-arithmetic MFMA prefill kernel handles the request (chunk 64; fp32
// inputs at d = dv = 64 or 128, bf16 inputs at d = dv = 64); its launcher.
bool mfma_f32_prefill_supported(la_dtype io_dtype, int32_t d, int32_t dv, int32_t chunk);
hipError_t launch_prefill_mfma_f32(const PrefillArgs &a, la_dtype io_dtype, hipStream_t stream);
// Bytes of the state (S, z, a gate product, padded) each segment after the first parks in
// Y at its first rows, at width d = dv.
int64_t segment_slot_bytes(int32_t d);
bool mfma_noncausal_supported(la_dtype io_dtype, int32_t d, int32_t dv);

}  // namespace la
