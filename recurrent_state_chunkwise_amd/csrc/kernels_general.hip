// General kernels: state initialisation, the general chunked prefill (any d, dv <= 128,
// chunk <= 128, f64/f32/bf16 io, arithmetic in the state dtype), the general non-causal
// form and the batched decode step.
//
// The operation is the one of page "Linear attention：把历史写进状态"
// (hs-black.github.io): phi = ELU+1, gated write S = a*S + k~ v^T, z = a*z + k~, then
// y = q~^T S / (q~^T z + eps).  Every kernel takes the feature map FM (an
// la_feature_map) as a template parameter.
#include "device_common.hpp"
#include "internal.hpp"

namespace la {
namespace {

constexpr int kThreads = 256;

// ===================================================================== state init
// One launch zeroes up to two byte ranges (S and z).  Each range is cut into an
// unaligned head, a bulk of aligned 16-byte stores and a tail; the first blocks of the
// grid take the first range and the rest the second.
struct FillRange {
    unsigned char *head;
    int64_t n_head;
    uint4 *bulk;
    int64_t n_bulk;
    unsigned char *tail;
    int64_t n_tail;
    int64_t blocks;  // blocks of the grid given to this range
};

FillRange make_fill_range(void *p, int64_t nbytes)
{
    FillRange r;
    unsigned char *b = static_cast<unsigned char *>(p);
    r.n_head = (int64_t)((16 - (reinterpret_cast<uintptr_t>(b) & 15)) & 15);
    if (r.n_head > nbytes)
        r.n_head = nbytes;
    r.n_bulk = (nbytes - r.n_head) / 16;
    r.n_tail = nbytes - r.n_head - r.n_bulk * 16;
    r.head = b;
    r.bulk = reinterpret_cast<uint4 *>(b + r.n_head);
    r.tail = b + r.n_head + r.n_bulk * 16;
    int64_t work = r.n_bulk > r.n_head ? r.n_bulk : r.n_head;
    if (r.n_tail > work)
        work = r.n_tail;
    r.blocks = (work + kThreads - 1) / kThreads;
    if (r.blocks > 8192)
        r.blocks = 8192;
    return r;
}

__global__ __launch_bounds__(kThreads) void zero_fill_kernel(FillRange r0, FillRange r1)
{
    const bool first = (int64_t)blockIdx.x < r0.blocks;
    const FillRange &r = first ? r0 : r1;
    const int64_t blk = first ? (int64_t)blockIdx.x : (int64_t)blockIdx.x - r0.blocks;
    const int64_t stride = r.blocks * kThreads;
    const int64_t i0 = blk * kThreads + threadIdx.x;
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
    for (int64_t i = i0; i < r.n_bulk; i += stride)
        r.bulk[i] = zero;
    for (int64_t i = i0; i < r.n_head; i += stride)
        r.head[i] = 0;
    for (int64_t i = i0; i < r.n_tail; i += stride)
        r.tail[i] = 0;
}

hipError_t zero_fill2(void *p0, int64_t n0, void *p1, int64_t n1, hipStream_t stream)
{
    const FillRange r0 = make_fill_range(p0, n0);
    const FillRange r1 = make_fill_range(p1, n1);
    const int64_t blocks = r0.blocks + r1.blocks;
    if (blocks == 0)
        return hipSuccess;
    zero_fill_kernel<<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(r0, r1);
    return hipGetLastError();
}

// ===================================================================== general prefill
constexpr int kRB = 16;        // query rows per block
constexpr int kIB = 16;        // key tokens per block (kRB * kIB == kThreads)
constexpr int kMaxSlice = 32;  // value columns per workgroup
constexpr int kPairs = kRB * kMaxSlice / kThreads;
constexpr int kStateRegs = LA_MAX_WIDTH * kMaxSlice / kThreads;
static_assert(kRB * kIB == kThreads, "one score per thread");

__device__ __forceinline__ float log_acc(float x) { return logf(x); }
__device__ __forceinline__ double log_acc(double x) { return log(x); }
__device__ __forceinline__ float exp_acc(float x) { return expf(x); }
__device__ __forceinline__ double exp_acc(double x) { return exp(x); }

template <typename TA>
size_t general_prefill_lds_bytes(int d, int slice)
{
    const int dp = d + 1;
    return sizeof(TA) * (size_t)(d * slice + d + kRB * dp + kIB * dp + kIB * slice + kRB * kIB +
                                 LA_MAX_CHUNK + kRB + kIB) +
           sizeof(int) * LA_MAX_CHUNK;
}

// One workgroup per (sequence, slice of value columns).  The sequence is walked
// chunk by chunk; inside a chunk the outputs are produced kRB rows at a time from
// the inter-chunk read of the previous state plus the masked intra-chunk scores,
// then the chunk is written into the state.  Gates enter through the log-sum of
// the gates since the last zero gate (lg) and the position of that zero gate (zp):
// the product of gates over (i, j] is 0 when a zero gate lies in (i, j], else
// exp(lg[j] - lg[i]).
template <typename TI, typename TA, int FM>
__global__ __launch_bounds__(kThreads) void prefill_general_kernel(
    const TI *__restrict__ Q, const TI *__restrict__ K, const TI *__restrict__ V, const TA *__restrict__ alpha,
    int64_t T, int d, int dv, int slice, TA eps, int chunk, TI *__restrict__ Y, TA *__restrict__ S,
    TA *__restrict__ z)
{
    const int tid = threadIdx.x;
    const int64_t h = blockIdx.x;
    const int c0 = blockIdx.y * slice;
    const int nc = min(slice, dv - c0);
    const int dp = d + 1;  // padded row stride of the Q~ and K~ tiles

    const TI *Qh = Q + h * T * d;
    const TI *Kh = K + h * T * d;
    const TI *Vh = V + h * T * dv;
    const TA *Ah = alpha ? alpha + h * T : nullptr;
    TI *Yh = Y + h * T * dv;
    TA *Sh = S + h * (int64_t)d * dv;
    TA *zh = z + h * d;

    extern __shared__ __align__(16) unsigned char smem_raw[];
    TA *Ss = reinterpret_cast<TA *>(smem_raw);  // [d][slice] state slice
    TA *zs = Ss + d * slice;                     // [d]
    TA *Qt = zs + d;                             // [kRB][dp] phi(q) rows
    TA *Kt = Qt + kRB * dp;                      // [kIB][dp] phi(k) rows
    TA *Vt = Kt + kIB * dp;                      // [kIB][slice]
    TA *At = Vt + kIB * slice;                   // [kRB][kIB] masked, gated scores
    TA *lg = At + kRB * kIB;                     // [LA_MAX_CHUNK]
    TA *den_s = lg + LA_MAX_CHUNK;               // [kRB]
    TA *wk = den_s + kRB;                        // [kIB] weight of a write at the chunk end
    int *zp = reinterpret_cast<int *>(wk + kIB); // [LA_MAX_CHUNK]

    // product of the gates of tokens i+1..j of the chunk (i <= j)
    auto pair_decay = [&](int j, int i) -> TA {
        if (!Ah)
            return TA(1);
        if (zp[j] > i)
            return TA(0);
        return exp_acc(lg[j] - lg[i]);
    };
    // product of the gates of tokens 0..j of the chunk: what is left of the incoming state
    auto start_decay = [&](int j) -> TA {
        if (!Ah)
            return TA(1);
        if (zp[j] >= 0)
            return TA(0);
        return exp_acc(lg[j]);
    };

    for (int e = tid; e < d * nc; e += kThreads) {
        const int f = e / nc, c = e - f * nc;
        Ss[f * slice + c] = Sh[(int64_t)f * dv + c0 + c];
    }
    for (int f = tid; f < d; f += kThreads)
        zs[f] = zh[f];
    __syncthreads();

    for (int64_t t0 = 0; t0 < T; t0 += chunk) {
        const int n = (int)min((int64_t)chunk, T - t0);
        if (Ah && tid == 0) {
            TA acc = 0;
            int last = -1;
            for (int j = 0; j < n; ++j) {
                const TA a = Ah[t0 + j];
                if (a == TA(0)) {
                    last = j;
                    acc = TA(0);
                } else {
                    acc += log_acc(a);
                }
                lg[j] = acc;
                zp[j] = last;
            }
        }

        // ---------------- outputs of the chunk, kRB rows at a time
        for (int j0 = 0; j0 < n; j0 += kRB) {
            const int rb = min(kRB, n - j0);
            for (int e = tid; e < rb * d; e += kThreads) {
                const int jj = e / d, f = e - jj * d;
                Qt[jj * dp + f] = phi_accurate<FM>(to_acc<TA>(Qh[(t0 + j0 + jj) * d + f]));
            }
            __syncthreads();

            // inter-chunk read: what is left of the previous state, seen by q~
            TA num[kPairs];
#pragma unroll
            for (int p = 0; p < kPairs; ++p) {
                num[p] = TA(0);
                const int e = tid + p * kThreads, jj = e / slice, c = e - jj * slice;
                if (jj < rb && c < nc) {
                    TA acc = 0;
                    for (int f = 0; f < d; ++f)
                        acc += Qt[jj * dp + f] * Ss[f * slice + c];
                    num[p] = start_decay(j0 + jj) * acc;
                }
            }
            if (tid < rb) {
                TA acc = 0;
                for (int f = 0; f < d; ++f)
                    acc += Qt[tid * dp + f] * zs[f];
                den_s[tid] = start_decay(j0 + tid) * acc;
            }

            // intra-chunk part: scores masked to i <= j and weighted by the gates
            const int jmax = j0 + rb - 1;
            for (int i0 = 0; i0 <= jmax; i0 += kIB) {
                const int ib = min(kIB, n - i0);
                __syncthreads();
                for (int e = tid; e < ib * d; e += kThreads) {
                    const int ii = e / d, f = e - ii * d;
                    Kt[ii * dp + f] = phi_accurate<FM>(to_acc<TA>(Kh[(t0 + i0 + ii) * d + f]));
                }
                for (int e = tid; e < ib * nc; e += kThreads) {
                    const int ii = e / nc, c = e - ii * nc;
                    Vt[ii * slice + c] = to_acc<TA>(Vh[(t0 + i0 + ii) * dv + c0 + c]);
                }
                __syncthreads();
                {
                    const int jj = tid / kIB, ii = tid - jj * kIB;
                    const int j = j0 + jj, i = i0 + ii;
                    TA a = TA(0);
                    if (jj < rb && ii < ib && i <= j) {
                        TA acc = 0;
                        for (int f = 0; f < d; ++f)
                            acc += Qt[jj * dp + f] * Kt[ii * dp + f];
                        a = acc * pair_decay(j, i);
                    }
                    At[jj * kIB + ii] = a;
                }
                __syncthreads();
#pragma unroll
                for (int p = 0; p < kPairs; ++p) {
                    const int e = tid + p * kThreads, jj = e / slice, c = e - jj * slice;
                    if (jj < rb && c < nc) {
                        TA acc = 0;
                        for (int ii = 0; ii < ib; ++ii)
                            acc += At[jj * kIB + ii] * Vt[ii * slice + c];
                        num[p] += acc;
                    }
                }
                if (tid < rb) {
                    TA acc = 0;
                    for (int ii = 0; ii < ib; ++ii)
                        acc += At[tid * kIB + ii];
                    den_s[tid] += acc;
                }
            }
            __syncthreads();
#pragma unroll
            for (int p = 0; p < kPairs; ++p) {
                const int e = tid + p * kThreads, jj = e / slice, c = e - jj * slice;
                if (jj < rb && c < nc)
                    Yh[(t0 + j0 + jj) * dv + c0 + c] = from_acc<TI>(num[p] / (den_s[jj] + eps));
            }
            __syncthreads();
        }

        // ---------------- write the chunk into the state
        const TA g_end = start_decay(n - 1);
        TA sreg[kStateRegs];
#pragma unroll
        for (int p = 0; p < kStateRegs; ++p) {
            const int e = tid + p * kThreads;
            sreg[p] = TA(0);
            if (e < d * nc) {
                const int f = e / nc, c = e - f * nc;
                sreg[p] = g_end * Ss[f * slice + c];
            }
        }
        TA zreg = tid < d ? g_end * zs[tid] : TA(0);
        for (int i0 = 0; i0 < n; i0 += kIB) {
            const int ib = min(kIB, n - i0);
            __syncthreads();
            for (int e = tid; e < ib * d; e += kThreads) {
                const int ii = e / d, f = e - ii * d;
                Kt[ii * dp + f] = phi_accurate<FM>(to_acc<TA>(Kh[(t0 + i0 + ii) * d + f]));
            }
            for (int e = tid; e < ib * nc; e += kThreads) {
                const int ii = e / nc, c = e - ii * nc;
                Vt[ii * slice + c] = to_acc<TA>(Vh[(t0 + i0 + ii) * dv + c0 + c]);
            }
            if (tid < ib)
                wk[tid] = pair_decay(n - 1, i0 + tid);
            __syncthreads();
#pragma unroll
            for (int p = 0; p < kStateRegs; ++p) {
                const int e = tid + p * kThreads;
                if (e < d * nc) {
                    const int f = e / nc, c = e - f * nc;
                    TA acc = 0;
                    for (int ii = 0; ii < ib; ++ii)
                        acc += (wk[ii] * Kt[ii * dp + f]) * Vt[ii * slice + c];
                    sreg[p] += acc;
                }
            }
            if (tid < d) {
                TA acc = 0;
                for (int ii = 0; ii < ib; ++ii)
                    acc += wk[ii] * Kt[ii * dp + tid];
                zreg += acc;
            }
        }
        __syncthreads();
#pragma unroll
        for (int p = 0; p < kStateRegs; ++p) {
            const int e = tid + p * kThreads;
            if (e < d * nc) {
                const int f = e / nc, c = e - f * nc;
                Ss[f * slice + c] = sreg[p];
            }
        }
        if (tid < d)
            zs[tid] = zreg;
        __syncthreads();
    }

    for (int e = tid; e < d * nc; e += kThreads) {
        const int f = e / nc, c = e - f * nc;
        Sh[(int64_t)f * dv + c0 + c] = Ss[f * slice + c];
    }
    // z is left to z_finish_kernel: other slices of this sequence may still be about to
    // read the incoming z
}

// The final z of each sequence, z_out = (product of all gates) z_in + sum over i of
// (product of the gates after i) phi(k_i), as the plain recurrence z = alpha z + phi(k)
// (page "Linear attention：把历史写进状态", sections "每来一个 token" and "加一个门")
// walked over kZStripes stretches of the sequence at once and composed in order.  It runs
// after the kernel whose value slices all read the incoming z, so it is the only writer
// of z.  One workgroup per sequence; thread (p, f) walks stretch p for feature f.
constexpr int kZThreads = 1024;

template <typename TI, typename TA, int FM>
__global__ __launch_bounds__(kZThreads) void z_finish_kernel(const TI *__restrict__ K, const TA *__restrict__ alpha,
                                                             int64_t T, int d, TA *__restrict__ z)
{
    __shared__ TA zl[kZThreads];
    __shared__ TA gp[kZThreads];
    const int tid = threadIdx.x;
    const int64_t h = blockIdx.x;
    const int stripes = kZThreads / d;  // d <= 128: at least 8 stretches
    const int p = tid / d, f = tid - p * d;
    const int64_t len = (T + stripes - 1) / stripes;
    if (p < stripes) {
        const int64_t t0 = p * len, t1 = min(T, t0 + len);
        const TI *Kh = K + h * T * d;
        const TA *Ah = alpha ? alpha + h * T : nullptr;
        TA acc = TA(0), g = TA(1);
#pragma unroll 8
        for (int64_t t = t0; t < t1; ++t) {
            const TA kf = phi_accurate<FM>(to_acc<TA>(Kh[t * d + f]));
            const TA a = Ah ? Ah[t] : TA(1);
            acc = a * acc + kf;
            g *= a;
        }
        zl[tid] = acc;
        gp[tid] = g;
    }
    __syncthreads();
    if (tid < d) {
        TA run = z[h * d + tid];
        for (int q = 0; q < stripes; ++q)
            run = gp[q * d + tid] * run + zl[q * d + tid];
        z[h * d + tid] = run;
    }
}

template <typename TI, typename TA, int FM>
hipError_t launch_z_finish(const PrefillArgs &a, hipStream_t stream)
{
    z_finish_kernel<TI, TA, FM><<<dim3((unsigned)a.n_heads), dim3(kZThreads), 0, stream>>>(
        static_cast<const TI *>(a.K), static_cast<const TA *>(a.alpha), a.T, a.d, static_cast<TA *>(a.z));
    return hipGetLastError();
}

template <typename TI, typename TA, int FM>
hipError_t launch_general_typed(const PrefillArgs &a, hipStream_t stream)
{
    // widest value slice whose working set fits a 64 KiB LDS budget
    int slice = a.dv < kMaxSlice ? a.dv : kMaxSlice;
    while (slice > 1 && general_prefill_lds_bytes<TA>(a.d, slice) > 65536)
        slice /= 2;
    const size_t lds = general_prefill_lds_bytes<TA>(a.d, slice);
    const unsigned n_slices = (unsigned)((a.dv + slice - 1) / slice);
    prefill_general_kernel<TI, TA, FM><<<dim3((unsigned)a.n_heads, n_slices), dim3(kThreads), lds, stream>>>(
        static_cast<const TI *>(a.Q), static_cast<const TI *>(a.K), static_cast<const TI *>(a.V),
        static_cast<const TA *>(a.alpha), a.T, a.d, a.dv, slice, static_cast<TA>(a.eps), a.chunk,
        static_cast<TI *>(a.Y), static_cast<TA *>(a.S), static_cast<TA *>(a.z));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    return launch_z_finish<TI, TA, FM>(a, stream);
}

// ===================================================================== general non-causal form
template <typename TA>
size_t noncausal_general_lds_bytes(int d, int slice)
{
    const int dp = d + 1;
    return sizeof(TA) * (size_t)(d * slice + d + kRB * dp + kIB * dp + kIB * slice + kRB);
}

// One workgroup per (sequence, slice of value columns).  First the whole sequence is
// written into the workgroup's slice of the state (and into all of z, which every
// slice needs), kIB tokens at a time; the state goes back to the caller; then every
// query is read against it, kRB rows at a time.  No slice writes z: z_finish_kernel
// does, once every slice has read the incoming z.
template <typename TI, typename TA, int FM>
__global__ __launch_bounds__(kThreads) void noncausal_general_kernel(
    const TI *__restrict__ Q, const TI *__restrict__ K, const TI *__restrict__ V, int64_t T, int d, int dv,
    int slice, TA eps, TI *__restrict__ Y, TA *__restrict__ S, TA *__restrict__ z)
{
    const int tid = threadIdx.x;
    const int64_t h = blockIdx.x;
    const int c0 = blockIdx.y * slice;
    const int nc = min(slice, dv - c0);
    const int dp = d + 1;

    const TI *Qh = Q + h * T * d;
    const TI *Kh = K + h * T * d;
    const TI *Vh = V + h * T * dv;
    TI *Yh = Y + h * T * dv;
    TA *Sh = S + h * (int64_t)d * dv;
    TA *zh = z + h * d;

    extern __shared__ __align__(16) unsigned char smem_raw[];
    TA *Ss = reinterpret_cast<TA *>(smem_raw);  // [d][slice] the full-sequence state slice
    TA *zs = Ss + d * slice;                     // [d]
    TA *Qt = zs + d;                             // [kRB][dp] phi(q) rows
    TA *Kt = Qt + kRB * dp;                      // [kIB][dp] phi(k) rows
    TA *Vt = Kt + kIB * dp;                      // [kIB][slice]
    TA *den_s = Vt + kIB * slice;                // [kRB]

    // ---------------- write: S_in + sum of k~ v^T, z_in + sum of k~
    TA sreg[kStateRegs];
#pragma unroll
    for (int p = 0; p < kStateRegs; ++p) {
        const int e = tid + p * kThreads;
        sreg[p] = TA(0);
        if (e < d * nc) {
            const int f = e / nc, c = e - f * nc;
            sreg[p] = Sh[(int64_t)f * dv + c0 + c];
        }
    }
    TA zreg = tid < d ? zh[tid] : TA(0);
    for (int64_t i0 = 0; i0 < T; i0 += kIB) {
        const int ib = (int)min((int64_t)kIB, T - i0);
        __syncthreads();
        for (int e = tid; e < ib * d; e += kThreads) {
            const int ii = e / d, f = e - ii * d;
            Kt[ii * dp + f] = phi_accurate<FM>(to_acc<TA>(Kh[(i0 + ii) * d + f]));
        }
        for (int e = tid; e < ib * nc; e += kThreads) {
            const int ii = e / nc, c = e - ii * nc;
            Vt[ii * slice + c] = to_acc<TA>(Vh[(i0 + ii) * dv + c0 + c]);
        }
        __syncthreads();
#pragma unroll
        for (int p = 0; p < kStateRegs; ++p) {
            const int e = tid + p * kThreads;
            if (e < d * nc) {
                const int f = e / nc, c = e - f * nc;
                TA acc = sreg[p];
                for (int ii = 0; ii < ib; ++ii)
                    acc += Kt[ii * dp + f] * Vt[ii * slice + c];
                sreg[p] = acc;
            }
        }
        if (tid < d) {
            TA acc = zreg;
            for (int ii = 0; ii < ib; ++ii)
                acc += Kt[ii * dp + tid];
            zreg = acc;
        }
    }
#pragma unroll
    for (int p = 0; p < kStateRegs; ++p) {
        const int e = tid + p * kThreads;
        if (e < d * nc) {
            const int f = e / nc, c = e - f * nc;
            Ss[f * slice + c] = sreg[p];
            Sh[(int64_t)f * dv + c0 + c] = sreg[p];
        }
    }
    if (tid < d)
        zs[tid] = zreg;  // z goes out through z_finish_kernel, after every slice has read z_in

    // ---------------- read: every query against the full state
    for (int64_t j0 = 0; j0 < T; j0 += kRB) {
        const int rb = (int)min((int64_t)kRB, T - j0);
        __syncthreads();
        for (int e = tid; e < rb * d; e += kThreads) {
            const int jj = e / d, f = e - jj * d;
            Qt[jj * dp + f] = phi_accurate<FM>(to_acc<TA>(Qh[(j0 + jj) * d + f]));
        }
        __syncthreads();
        if (tid < rb) {
            TA acc = 0;
            for (int f = 0; f < d; ++f)
                acc += Qt[tid * dp + f] * zs[f];
            den_s[tid] = acc;
        }
        TA num[kPairs];
#pragma unroll
        for (int p = 0; p < kPairs; ++p) {
            num[p] = TA(0);
            const int e = tid + p * kThreads, jj = e / slice, c = e - jj * slice;
            if (jj < rb && c < nc) {
                TA acc = 0;
                for (int f = 0; f < d; ++f)
                    acc += Qt[jj * dp + f] * Ss[f * slice + c];
                num[p] = acc;
            }
        }
        __syncthreads();
#pragma unroll
        for (int p = 0; p < kPairs; ++p) {
            const int e = tid + p * kThreads, jj = e / slice, c = e - jj * slice;
            if (jj < rb && c < nc)
                Yh[(j0 + jj) * dv + c0 + c] = from_acc<TI>(num[p] / (den_s[jj] + eps));
        }
    }
}

template <typename TI, typename TA, int FM>
hipError_t launch_noncausal_typed(const PrefillArgs &a, hipStream_t stream)
{
    int slice = a.dv < kMaxSlice ? a.dv : kMaxSlice;
    while (slice > 1 && noncausal_general_lds_bytes<TA>(a.d, slice) > 65536)
        slice /= 2;
    const size_t lds = noncausal_general_lds_bytes<TA>(a.d, slice);
    const unsigned n_slices = (unsigned)((a.dv + slice - 1) / slice);
    noncausal_general_kernel<TI, TA, FM><<<dim3((unsigned)a.n_heads, n_slices), dim3(kThreads), lds, stream>>>(
        static_cast<const TI *>(a.Q), static_cast<const TI *>(a.K), static_cast<const TI *>(a.V), a.T, a.d, a.dv,
        slice, static_cast<TA>(a.eps), static_cast<TI *>(a.Y), static_cast<TA *>(a.S), static_cast<TA *>(a.z));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    return launch_z_finish<TI, TA, FM>(a, stream);  // PrefillArgs of the non-causal form carry no alpha
}

// ===================================================================== decode
constexpr int kDecodeThreads = 512;

// d = dv = D (64 or 128): one workgroup of 512 threads per state (measured faster than
// 256 or 1024 on this streaming update at width 128).  Thread (rg, cg) owns VEC
// consecutive columns (cg) of the rows rg, rg + NRG, ..., so each wave reads adjacent
// full rows; all of a thread's rows are loaded before any is used.
// Each state is touched once per step, so its loads and stores are marked
// non-temporal to keep it from displacing other lines in the caches.
template <typename TI, typename TA, int VEC, int FM, int D>
__global__ __launch_bounds__(kDecodeThreads) void decode_wide_kernel(
    const TI *__restrict__ q, const TI *__restrict__ k, const TI *__restrict__ v, const TA *__restrict__ alpha,
    TA eps, TI *__restrict__ y, TA *__restrict__ S, TA *__restrict__ z)
{
    constexpr int DV = D, NCG = DV / VEC, NRG = kDecodeThreads / NCG, ROWS = D / NRG;
    static_assert(ROWS >= 1 && D * NCG * VEC == D * DV, "whole rows per thread group");
    typedef TA vec_t __attribute__((ext_vector_type(VEC)));
    __shared__ TA kf[D], qf[D], vs[DV];
    __shared__ TA red[NRG][DV];
    __shared__ TA dred[kDecodeThreads / 64];

    const int tid = threadIdx.x;
    const int64_t n = blockIdx.x;
    const int cg = tid % NCG, rg = tid / NCG;
    vec_t *Sv = reinterpret_cast<vec_t *>(S + n * (int64_t)(D * DV));

    vec_t s[ROWS];
#pragma unroll
    for (int i = 0; i < ROWS; ++i)
        s[i] = __builtin_nontemporal_load(&Sv[(rg + i * NRG) * NCG + cg]);
    const TA zf = tid < D ? z[n * D + tid] : TA(0);
    if (tid < D) {
        kf[tid] = phi_accurate<FM>(to_acc<TA>(k[n * D + tid]));
        qf[tid] = phi_accurate<FM>(to_acc<TA>(q[n * D + tid]));
        vs[tid] = to_acc<TA>(v[n * DV + tid]);
    }
    const TA a = alpha ? alpha[n] : TA(1);
    __syncthreads();

    TA part[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e)
        part[e] = TA(0);
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        const int f = rg + i * NRG;
        const TA kv = kf[f], qv = qf[f];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            s[i][e] = a * s[i][e] + kv * vs[cg * VEC + e];
            part[e] += qv * s[i][e];
        }
        __builtin_nontemporal_store(s[i], &Sv[f * NCG + cg]);
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e)
        red[rg][cg * VEC + e] = part[e];

    TA dpart = TA(0);
    if (tid < D) {
        const TA zn = a * zf + kf[tid];
        z[n * D + tid] = zn;
        dpart = qf[tid] * zn;
    }
    dpart = wave_sum(dpart);
    if ((tid & 63) == 0)
        dred[tid >> 6] = dpart;
    __syncthreads();
    if (tid < DV) {
        TA num = TA(0);
#pragma unroll
        for (int r = 0; r < NRG; ++r)
            num += red[r][tid];
        TA den = TA(0);
#pragma unroll
        for (int w = 0; w < kDecodeThreads / 64; ++w)
            den += dred[w];
        y[n * DV + tid] = from_acc<TI>(num / (den + eps));
    }
}

// Any d, dv <= 128: thread (rg, c) owns column c of rows rg, rg + nrg, ...
template <typename TI, typename TA, int FM>
__global__ __launch_bounds__(kThreads) void decode_general_kernel(
    const TI *__restrict__ q, const TI *__restrict__ k, const TI *__restrict__ v, const TA *__restrict__ alpha,
    int d, int dv, TA eps, TI *__restrict__ y, TA *__restrict__ S, TA *__restrict__ z)
{
    __shared__ TA kf[LA_MAX_WIDTH], qf[LA_MAX_WIDTH], vs[LA_MAX_WIDTH];
    __shared__ TA red[kThreads];
    __shared__ TA dred[kThreads / 64];
    const int tid = threadIdx.x;
    const int64_t n = blockIdx.x;
    if (tid < d) {
        kf[tid] = phi_accurate<FM>(to_acc<TA>(k[n * d + tid]));
        qf[tid] = phi_accurate<FM>(to_acc<TA>(q[n * d + tid]));
    }
    if (tid < dv)
        vs[tid] = to_acc<TA>(v[n * dv + tid]);
    const TA a = alpha ? alpha[n] : TA(1);
    __syncthreads();

    const int nrg = kThreads / dv;
    const int c = tid % dv, rg = tid / dv;
    TA *Sn = S + n * (int64_t)d * dv;
    TA part = TA(0);
    if (rg < nrg) {
        for (int f = rg; f < d; f += nrg) {
            const TA s = a * Sn[(int64_t)f * dv + c] + kf[f] * vs[c];
            Sn[(int64_t)f * dv + c] = s;
            part += qf[f] * s;
        }
    }
    red[tid] = part;
    TA dpart = TA(0);
    if (tid < d) {
        const TA zn = a * z[n * d + tid] + kf[tid];
        z[n * d + tid] = zn;
        dpart = qf[tid] * zn;
    }
    dpart = wave_sum(dpart);
    if ((tid & 63) == 0)
        dred[tid >> 6] = dpart;
    __syncthreads();
    if (tid < dv) {
        TA num = TA(0);
        for (int r = 0; r < nrg; ++r)
            num += red[r * dv + tid];
        TA den = TA(0);
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w)
            den += dred[w];
        y[n * dv + tid] = from_acc<TI>(num / (den + eps));
    }
}

template <typename TI, typename TA, int FM>
hipError_t launch_decode_typed(const DecodeArgs &a, hipStream_t stream)
{
    constexpr int VEC = 16 / sizeof(TA);
    const bool aligned = (reinterpret_cast<uintptr_t>(a.S) % 16) == 0;
    if (a.d == 128 && a.dv == 128 && aligned) {
        decode_wide_kernel<TI, TA, VEC, FM, 128><<<dim3((unsigned)a.n_states), dim3(kDecodeThreads), 0, stream>>>(
            static_cast<const TI *>(a.q), static_cast<const TI *>(a.k), static_cast<const TI *>(a.v),
            static_cast<const TA *>(a.alpha), static_cast<TA>(a.eps), static_cast<TI *>(a.y),
            static_cast<TA *>(a.S), static_cast<TA *>(a.z));
    } else if (a.d == 64 && a.dv == 64 && aligned) {
        decode_wide_kernel<TI, TA, VEC, FM, 64><<<dim3((unsigned)a.n_states), dim3(kDecodeThreads), 0, stream>>>(
            static_cast<const TI *>(a.q), static_cast<const TI *>(a.k), static_cast<const TI *>(a.v),
            static_cast<const TA *>(a.alpha), static_cast<TA>(a.eps), static_cast<TI *>(a.y),
            static_cast<TA *>(a.S), static_cast<TA *>(a.z));
    } else {
        decode_general_kernel<TI, TA, FM><<<dim3((unsigned)a.n_states), dim3(kThreads), 0, stream>>>(
            static_cast<const TI *>(a.q), static_cast<const TI *>(a.k), static_cast<const TI *>(a.v),
            static_cast<const TA *>(a.alpha), a.d, a.dv, static_cast<TA>(a.eps), static_cast<TI *>(a.y),
            static_cast<TA *>(a.S), static_cast<TA *>(a.z));
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_state_init(void *S, void *z, int64_t n_states, int32_t r, int32_t dv, la_dtype state_dtype,
                             hipStream_t stream)
{
    const int64_t es = state_dtype == LA_F64 ? 8 : 4;
    return zero_fill2(S, n_states * r * dv * es, z, n_states * r * es, stream);
}

hipError_t launch_prefill_general(const PrefillArgs &a, la_dtype io_dtype, hipStream_t stream)
{
    return dispatch_feature_map(a.phi, [&](auto fm) {
        constexpr int FM = decltype(fm)::value;
        switch (io_dtype) {
        case LA_F64:
            return launch_general_typed<double, double, FM>(a, stream);
        case LA_F32:
            return launch_general_typed<float, float, FM>(a, stream);
        default:
            return launch_general_typed<bf16, float, FM>(a, stream);
        }
    });
}

hipError_t launch_noncausal_general(const PrefillArgs &a, la_dtype io_dtype, hipStream_t stream)
{
    return dispatch_feature_map(a.phi, [&](auto fm) {
        constexpr int FM = decltype(fm)::value;
        switch (io_dtype) {
        case LA_F64:
            return launch_noncausal_typed<double, double, FM>(a, stream);
        case LA_F32:
            return launch_noncausal_typed<float, float, FM>(a, stream);
        default:
            return launch_noncausal_typed<bf16, float, FM>(a, stream);
        }
    });
}

hipError_t launch_decode(const DecodeArgs &a, la_dtype io_dtype, hipStream_t stream)
{
    return dispatch_feature_map(a.phi, [&](auto fm) {
        constexpr int FM = decltype(fm)::value;
        switch (io_dtype) {
        case LA_F64:
            return launch_decode_typed<double, double, FM>(a, stream);
        case LA_F32:
            return launch_decode_typed<float, float, FM>(a, stream);
        default:
            return launch_decode_typed<bf16, float, FM>(a, stream);
        }
    });
}

}  // namespace la
