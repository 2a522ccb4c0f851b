// Delta-rule decode step: for each independent memory S [d, dv] (feature-major),
//   p = S^T k,  e = v - p,  S <- S + beta k e^T,  y = S^T q  (read after the write),
// the fast-weight memory of the page "Linear attention：把历史写进状态", section
// "Delta rule：先读旧答案，再写误差" (the write S' = S + beta k (v - k^T S) of its
// derivation "key 的范数决定了纠错力度").  Keys and queries enter as given; the page's
// delta examples apply no feature map.  Like the accumulating decode step this streams
// every state once per step: it reads S, forms the prediction, and writes S back.
#include "device_common.hpp"
#include "internal.hpp"

namespace la {
namespace {

constexpr int kDeltaThreads = 512;  // per state, as for the accumulating decode step
constexpr int kGeneralThreads = 256;

// d = dv = 128: thread (rg, cg) owns VEC consecutive columns (cg) of rows rg, rg + NRG,
// ..., so each wave reads adjacent full rows; all of a thread's rows are loaded before
// any is used, with non-temporal hints (each state is touched once per step).  The
// read-out of the written state needs no second pass over it: with e the error,
//   S_new^T q = S^T q + beta (k . q) e,
// so S^T k and S^T q are reduced together from the state as loaded, and the write
// follows (one reduction round per step instead of two; the same values up to the
// order of fp rounding).
template <typename TI, typename TA, int VEC>
__global__ __launch_bounds__(kDeltaThreads) void delta_w128_kernel(
    const TI *__restrict__ q, const TI *__restrict__ k, const TI *__restrict__ v, const TA *__restrict__ beta,
    TI *__restrict__ y, TA *__restrict__ S)
{
    constexpr int D = 128, DV = 128, NCG = DV / VEC, NRG = kDeltaThreads / NCG, ROWS = D / NRG;
    typedef TA vec_t __attribute__((ext_vector_type(VEC)));
    __shared__ TA kf[D], qf[D], be[DV];
    __shared__ TA redk[NRG][DV], redq[NRG][DV];
    __shared__ TA kq[2];

    const int tid = threadIdx.x;
    const int64_t n = blockIdx.x;
    const int cg = tid % NCG, rg = tid / NCG;
    vec_t *Sv = reinterpret_cast<vec_t *>(S + n * (int64_t)(D * DV));

    vec_t s[ROWS];
#pragma unroll
    for (int i = 0; i < ROWS; ++i)
        s[i] = __builtin_nontemporal_load(&Sv[(rg + i * NRG) * NCG + cg]);
    TA kqp = TA(0);
    if (tid < D) {
        const TA kv = to_acc<TA>(k[n * D + tid]), qv = to_acc<TA>(q[n * D + tid]);
        kf[tid] = kv;
        qf[tid] = qv;
        kqp = kv * qv;
    }
    const TA vv = tid < DV ? to_acc<TA>(v[n * DV + tid]) : TA(0);
    const TA b = beta[n];
    kqp = wave_sum(kqp);  // waves 0 and 1 hold k . q over their 64 features
    if (tid < D && (tid & 63) == 0)
        kq[tid >> 6] = kqp;
    __syncthreads();

    // S^T k and S^T q: partial sums over this thread's rows of the state as loaded
    TA pk[VEC], pq[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e)
        pk[e] = pq[e] = TA(0);
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        const TA kv = kf[rg + i * NRG], qv = qf[rg + i * NRG];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            pk[e] += kv * s[i][e];
            pq[e] += qv * s[i][e];
        }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        redk[rg][cg * VEC + e] = pk[e];
        redq[rg][cg * VEC + e] = pq[e];
    }
    __syncthreads();
    if (tid < DV) {
        TA p = TA(0), o = TA(0);
#pragma unroll
        for (int r = 0; r < NRG; ++r) {
            p += redk[r][tid];
            o += redq[r][tid];
        }
        const TA bev = b * (vv - p);  // beta * error
        be[tid] = bev;
        y[n * DV + tid] = from_acc<TI>(o + (kq[0] + kq[1]) * bev);
    }
    __syncthreads();

    // write S += k (beta e)^T
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        const int f = rg + i * NRG;
        const TA kv = kf[f];
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            s[i][e] += kv * be[cg * VEC + e];
        __builtin_nontemporal_store(s[i], &Sv[f * NCG + cg]);
    }
}

// Any d, dv <= 128: thread (rg, c) owns column c of rows rg, rg + nrg, ...; the state
// is read twice (prediction, then write and read-out), so this path is for odd shapes.
template <typename TI, typename TA>
__global__ __launch_bounds__(kGeneralThreads) void delta_general_kernel(
    const TI *__restrict__ q, const TI *__restrict__ k, const TI *__restrict__ v, const TA *__restrict__ beta,
    int d, int dv, TI *__restrict__ y, TA *__restrict__ S)
{
    __shared__ TA kf[LA_MAX_WIDTH], qf[LA_MAX_WIDTH], vs[LA_MAX_WIDTH], be[LA_MAX_WIDTH];
    __shared__ TA red[kGeneralThreads];
    const int tid = threadIdx.x;
    const int64_t n = blockIdx.x;
    if (tid < d) {
        kf[tid] = to_acc<TA>(k[n * d + tid]);
        qf[tid] = to_acc<TA>(q[n * d + tid]);
    }
    if (tid < dv)
        vs[tid] = to_acc<TA>(v[n * dv + tid]);
    const TA b = beta[n];
    __syncthreads();

    const int nrg = kGeneralThreads / dv;
    const int c = tid % dv, rg = tid / dv;
    TA *Sn = S + n * (int64_t)d * dv;
    TA part = TA(0);
    if (rg < nrg)
        for (int f = rg; f < d; f += nrg)
            part += kf[f] * Sn[(int64_t)f * dv + c];
    red[tid] = part;
    __syncthreads();
    if (tid < dv) {
        TA p = TA(0);
        for (int r = 0; r < nrg; ++r)
            p += red[r * dv + tid];
        be[tid] = b * (vs[tid] - p);
    }
    __syncthreads();
    part = TA(0);
    if (rg < nrg) {
        for (int f = rg; f < d; f += nrg) {
            const TA s = Sn[(int64_t)f * dv + c] + kf[f] * be[c];
            Sn[(int64_t)f * dv + c] = s;
            part += qf[f] * s;
        }
    }
    red[tid] = part;
    __syncthreads();
    if (tid < dv) {
        TA acc = TA(0);
        for (int r = 0; r < nrg; ++r)
            acc += red[r * dv + tid];
        y[n * dv + tid] = from_acc<TI>(acc);
    }
}

template <typename TI, typename TA>
hipError_t launch_delta_typed(const DeltaArgs &a, hipStream_t stream)
{
    constexpr int VEC = 16 / sizeof(TA);
    const bool aligned = (reinterpret_cast<uintptr_t>(a.S) % 16) == 0;
    if (a.d == 128 && a.dv == 128 && aligned) {
        delta_w128_kernel<TI, TA, VEC><<<dim3((unsigned)a.n_states), dim3(kDeltaThreads), 0, stream>>>(
            static_cast<const TI *>(a.q), static_cast<const TI *>(a.k), static_cast<const TI *>(a.v),
            static_cast<const TA *>(a.beta), static_cast<TI *>(a.y), static_cast<TA *>(a.S));
    } else {
        delta_general_kernel<TI, TA><<<dim3((unsigned)a.n_states), dim3(kGeneralThreads), 0, stream>>>(
            static_cast<const TI *>(a.q), static_cast<const TI *>(a.k), static_cast<const TI *>(a.v),
            static_cast<const TA *>(a.beta), a.d, a.dv, static_cast<TI *>(a.y), static_cast<TA *>(a.S));
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_delta_decode(const DeltaArgs &a, la_dtype io_dtype, hipStream_t stream)
{
    switch (io_dtype) {
    case LA_F64:
        return launch_delta_typed<double, double>(a, stream);
    case LA_F32:
        return launch_delta_typed<float, float>(a, stream);
    default:
        return launch_delta_typed<bf16, float>(a, stream);
    }
}

}  // namespace la
