// Device-side helpers shared by the gfx950 kernels of the linear-attention library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "linattn.h"

namespace la {

typedef __bf16 bf16;

// ---------------------------------------------------------------- feature maps
// FM is an la_feature_map value:
//   LA_PHI_ELU1         ELU(x) + 1 with ELU's scale 1: x + 1 above zero, exp(x) at or
//                       below (page "Linear attention：把历史写进状态", section "关键改写");
//                       phi(0) = 1 from both branches and phi(-inf) = 0 exactly
//   LA_PHI_RELU1        max(x, 0) + 1 (the positive map of the datawhalechina chapter
//                       "Linear Attention and Recurrent State", Step 4)
//   LA_PHI_RELU_EPS     max(x, 0) + 1e-5   (the switchable maps of the pluggable module
//   LA_PHI_SIGMOID_EPS  sigmoid(x) + 1e-5   on the page "线性注意力架构演进", ai-master.cc)
// Arithmetic in the type of x.
__device__ __forceinline__ float exp_of(float x) { return expf(x); }
__device__ __forceinline__ double exp_of(double x) { return exp(x); }

template <int FM, typename T>
__device__ __forceinline__ T phi_accurate(T x)
{
    if constexpr (FM == LA_PHI_RELU1)
        return (x > T(0) ? x : T(0)) + T(1);
    else if constexpr (FM == LA_PHI_RELU_EPS)
        return (x > T(0) ? x : T(0)) + T(1e-5);
    else if constexpr (FM == LA_PHI_SIGMOID_EPS)
        return T(1) / (T(1) + exp_of(-x)) + T(1e-5);
    else
        return x > T(0) ? x + T(1) : exp_of(x);
}

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
