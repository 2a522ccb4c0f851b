// bf16 MFMA chunked prefill for d = dv = 128 (placeholder until the kernel lands).
#include "device_common.hpp"
#include "internal.hpp"

namespace la {

bool mfma_prefill_supported(la_dtype, int32_t, int32_t, int32_t) { return false; }

hipError_t launch_prefill_mfma_bf16(const PrefillArgs &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace la
