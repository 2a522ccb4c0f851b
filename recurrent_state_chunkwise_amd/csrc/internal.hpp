// Host-side launcher interface between the C ABI (api.hip) and the kernel files.
#pragma once

#include <stdint.h>
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
};

struct DecodeArgs {
    const void *q, *k, *v, *alpha;
    int64_t n_states;
    int32_t d, dv;
    double eps;
    void *y, *S, *z;
};

struct DeltaArgs {
    const void *q, *k, *v, *beta;
    int64_t n_states;
    int32_t d, dv;
    void *y, *S;
};

// Each launcher enqueues its kernels on `stream` and returns the HIP status of
// the launch (hipSuccess or the runtime's refusal).  Arguments are already valid.
hipError_t launch_state_init(void *S, void *z, int64_t n_states, int32_t r, int32_t dv,
                             la_dtype state_dtype, hipStream_t stream);
hipError_t launch_prefill_general(const PrefillArgs &a, la_dtype io_dtype, hipStream_t stream);
hipError_t launch_prefill_mfma_bf16(const PrefillArgs &a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, la_dtype io_dtype, hipStream_t stream);
hipError_t launch_delta_decode(const DeltaArgs &a, la_dtype io_dtype, hipStream_t stream);

// True when the bf16 MFMA prefill kernel handles the request.
bool mfma_prefill_supported(la_dtype io_dtype, int32_t d, int32_t dv, int32_t chunk);

}  // namespace la
