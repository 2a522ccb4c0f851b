// Device-side helpers shared by the gfx950 kernels of the linear-attention library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef __bf16 bf16;

// ---------------------------------------------------------------- feature map
// phi(x) = ELU(x) + 1 with ELU's scale 1: x + 1 above zero, exp(x) at or below
// (page "Linear attention：把历史写进状态", section "关键改写").  phi(0) = 1 from both
// branches and phi(-inf) = 0 exactly.
__device__ __forceinline__ float phi_accurate(float x) { return x > 0.f ? x + 1.f : expf(x); }
__device__ __forceinline__ double phi_accurate(double x) { return x > 0.0 ? x + 1.0 : exp(x); }
// Hardware exp2 path; its few-ulp error is far below the bf16 rounding that follows.
__device__ __forceinline__ float phi_fast(float x) { return x > 0.f ? x + 1.f : __expf(x); }

// ---------------------------------------------------------------- io conversions
template <typename TA, typename TI>
__device__ __forceinline__ TA to_acc(TI x) { return static_cast<TA>(x); }

template <typename TI, typename TA>
__device__ __forceinline__ TI from_acc(TA x) { return static_cast<TI>(x); }

// bf16 -> double goes through float (exact).
template <>
__device__ __forceinline__ double to_acc<double, bf16>(bf16 x) { return static_cast<double>(static_cast<float>(x)); }
template <>
__device__ __forceinline__ bf16 from_acc<bf16, double>(double x) { return static_cast<bf16>(static_cast<float>(x)); }

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ double wave_sum(double v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

}  // namespace la
