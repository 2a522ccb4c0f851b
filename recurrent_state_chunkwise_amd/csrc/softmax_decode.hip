// Softmax attention decode over an explicit K/V history: the comparator of the
// datawhalechina chapter "Linear Attention and Recurrent State", Step 5, which sets a
// full K/V history against the fixed recurrent state.  The row is the one of the page
// "Linear attention：把历史写进状态" (hs-black.github.io), section "先看普通 attention 在读
// 什么": the query scores every history key, softmax normalises the scores, and the
// values are summed with those weights.
//
// One step for each head h: the new (k, v) is written to row `pos` of the caches, and
//   y_h = sum_{i <= pos} softmax_i(scale * q_h . K_h[i]) V_h[i].
// The history is split into kSplit-token pieces, one workgroup each (enough workgroups
// to spread a long history over the compute units): a workgroup keeps the maximum
// score m, the sum l of exp(s - m) and the weighted value sum o of its piece, and a
// second kernel combines the pieces of a head with the usual rescaling by exp(m - M).
// The workgroup that owns row `pos` takes that row's key and value from the inputs and
// writes them to the caches; no other workgroup reads it.
#include <mutex>

#include "device_common.hpp"
#include "internal.hpp"

namespace la {
namespace {

constexpr int kSmThreads = 256;
constexpr int kSplit = 256;  // history rows per workgroup

template <typename TA>
__device__ __forceinline__ TA wave_max(TA v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const TA o = __shfl_xor(v, off, 64);
        v = o > v ? o : v;
    }
    return v;
}

template <typename TI>
struct SmArgs {
    const TI *q, *k, *v;
    TI *Kc, *Vc;
    int64_t capacity, L;  // L = pos + 1 rows attended
    int d, dv, n_splits;
    double scale;
    void *ws;  // [head][split][2 + dv] of TA: m, l, o
    TI *y;
};

// Any width and dtype, element by element: thread t scores history row t, then each
// column's weighted sum walks the piece's rows.
template <typename TI, typename TA>
__global__ __launch_bounds__(kSmThreads) void softmax_split_kernel(SmArgs<TI> a)
{
    __shared__ TA qs[LA_MAX_WIDTH];
    __shared__ TA p[kSplit];
    __shared__ TA red[kSmThreads / 64];

    const int tid = threadIdx.x;
    const int64_t h = blockIdx.y;
    const int sp = blockIdx.x;
    const int64_t i0 = (int64_t)sp * kSplit;
    const int n = (int)min((int64_t)kSplit, a.L - i0);
    const int64_t pos = a.L - 1;
    const int d = a.d, dv = a.dv;
    const TI *Kh = a.Kc + h * a.capacity * d;
    const TI *Vh = a.Vc + h * a.capacity * dv;
    const TI *kn = a.k + h * d;
    const TI *vn = a.v + h * dv;

    for (int c = tid; c < d; c += kSmThreads)
        qs[c] = to_acc<TA>(a.q[h * d + c]);
    if (pos >= i0 && pos < i0 + n) {  // this piece holds the new row: it joins the caches
        TI *kdst = a.Kc + (h * a.capacity + pos) * d;
        TI *vdst = a.Vc + (h * a.capacity + pos) * dv;
        for (int c = tid; c < d; c += kSmThreads)
            kdst[c] = kn[c];
        for (int c = tid; c < dv; c += kSmThreads)
            vdst[c] = vn[c];
    }
    __syncthreads();

    TA s = -INFINITY;
    if (tid < n) {
        const int64_t i = i0 + tid;
        const TI *kr = i == pos ? kn : Kh + i * d;
        TA acc = 0;
        for (int c = 0; c < d; ++c)
            acc += qs[c] * to_acc<TA>(kr[c]);
        s = static_cast<TA>(a.scale) * acc;
    }
    TA m = wave_max(s);
    if ((tid & 63) == 0)
        red[tid >> 6] = m;
    __syncthreads();
    m = red[0];
#pragma unroll
    for (int w = 1; w < kSmThreads / 64; ++w)
        m = red[w] > m ? red[w] : m;
    const TA e = tid < n ? exp_of(s - m) : TA(0);
    p[tid] = e;
    TA l = wave_sum(e);
    __syncthreads();  // everyone has read red[] for m; p[] is complete
    if ((tid & 63) == 0)
        red[tid >> 6] = l;
    __syncthreads();
    l = red[0];
#pragma unroll
    for (int w = 1; w < kSmThreads / 64; ++w)
        l += red[w];

    const bool direct = a.n_splits == 1;
    TA *ws = static_cast<TA *>(a.ws) + (h * a.n_splits + sp) * (int64_t)(2 + dv);
    for (int c = tid; c < dv; c += kSmThreads) {
        TA acc = 0;
        for (int t = 0; t < n; ++t) {
            const int64_t i = i0 + t;
            acc += p[t] * to_acc<TA>(i == pos ? vn[c] : Vh[i * dv + c]);
        }
        if (direct)
            a.y[h * dv + c] = from_acc<TI>(acc / l);
        else
            ws[2 + c] = acc;
    }
    if (!direct && tid == 0) {
        ws[0] = m;
        ws[1] = l;
    }
}

// bf16 rows with d and dv = 8 G multiples of 8 (G a power of two, 16-byte aligned rows): all
// of a workgroup's key and value loads are issued before any is used, so a piece costs
// one trip to memory.  Thread t scores row t; for the value sums thread (tg, gr) takes
// granule gr (8 columns) of rows tg, tg + TG, ... (TG = 256 / G, so G rows per thread).
template <int G>
__global__ __launch_bounds__(kSmThreads) void softmax_split_bf16_kernel(SmArgs<bf16> a)
{
    constexpr int TG = kSmThreads / G;
    __shared__ float qs[LA_MAX_WIDTH];
    __shared__ float p[kSplit];
    __shared__ float red[kSmThreads / 64];
    __shared__ float ored[kSmThreads * 8];

    const int tid = threadIdx.x;
    const int64_t h = blockIdx.y;
    const int sp = blockIdx.x;
    const int64_t i0 = (int64_t)sp * kSplit;
    const int n = (int)min((int64_t)kSplit, a.L - i0);
    const int64_t pos = a.L - 1;
    const int d = a.d, dv = a.dv;
    const bf16 *Kh = a.Kc + h * a.capacity * d;
    const bf16 *Vh = a.Vc + h * a.capacity * dv;
    const bf16 *kn = a.k + h * d;
    const bf16 *vn = a.v + h * dv;
    const int gr = tid % G, tg = tid / G;

    // every load first: the value granules, then the key row
    uint4 vr[G];
#pragma unroll
    for (int r = 0; r < G; ++r) {
        const int t = tg + r * TG;
        const int64_t i = i0 + t;
        vr[r] = make_uint4(0u, 0u, 0u, 0u);
        if (t < n)
            vr[r] = *reinterpret_cast<const uint4 *>((i == pos ? vn : Vh + i * dv) + 8 * gr);
    }
    uint4 kr[LA_MAX_WIDTH / 8];
    {
        const int64_t i = i0 + tid;
        const bf16 *row = i == pos ? kn : Kh + i * d;
#pragma unroll
        for (int c8 = 0; c8 < LA_MAX_WIDTH / 8; ++c8) {
            kr[c8] = make_uint4(0u, 0u, 0u, 0u);
            if (tid < n && 8 * c8 < d)
                kr[c8] = *reinterpret_cast<const uint4 *>(row + 8 * c8);
        }
    }
    for (int c = tid; c < d; c += kSmThreads)
        qs[c] = static_cast<float>(a.q[h * d + c]);
    if (pos >= i0 && pos < i0 + n) {  // this piece holds the new row: it joins the caches
        bf16 *kdst = a.Kc + (h * a.capacity + pos) * d;
        bf16 *vdst = a.Vc + (h * a.capacity + pos) * dv;
        for (int c = tid; c < d; c += kSmThreads)
            kdst[c] = kn[c];
        for (int c = tid; c < dv; c += kSmThreads)
            vdst[c] = vn[c];
    }
    __syncthreads();

    float s = -INFINITY;
    if (tid < n) {
        float acc = 0.f;
#pragma unroll
        for (int c8 = 0; c8 < LA_MAX_WIDTH / 8; ++c8) {
            if (8 * c8 < d) {
                const unsigned w[4] = {kr[c8].x, kr[c8].y, kr[c8].z, kr[c8].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc += qs[8 * c8 + 2 * e] * __uint_as_float(w[e] << 16);
                    acc += qs[8 * c8 + 2 * e + 1] * __uint_as_float(w[e] & 0xffff0000u);
                }
            }
        }
        s = static_cast<float>(a.scale) * acc;
    }
    float m = wave_max(s);
    if ((tid & 63) == 0)
        red[tid >> 6] = m;
    __syncthreads();
    m = red[0];
#pragma unroll
    for (int w = 1; w < kSmThreads / 64; ++w)
        m = red[w] > m ? red[w] : m;
    const float e = tid < n ? __expf(s - m) : 0.f;
    p[tid] = e;
    float l = wave_sum(e);
    __syncthreads();
    if ((tid & 63) == 0)
        red[tid >> 6] = l;

    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < G; ++r) {
        const float pt = p[tg + r * TG];  // 0 past the end of the piece
        const unsigned w[4] = {vr[r].x, vr[r].y, vr[r].z, vr[r].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            o[2 * j] += pt * __uint_as_float(w[j] << 16);
            o[2 * j + 1] += pt * __uint_as_float(w[j] & 0xffff0000u);
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
        ored[tid * 8 + j] = o[j];
    __syncthreads();
    l = red[0];
#pragma unroll
    for (int w = 1; w < kSmThreads / 64; ++w)
        l += red[w];

    const bool direct = a.n_splits == 1;
    float *ws = static_cast<float *>(a.ws) + (h * a.n_splits + sp) * (int64_t)(2 + dv);
    for (int c = tid; c < dv; c += kSmThreads) {
        const int g = c / 8, j = c % 8;
        float acc = 0.f;
        for (int t = 0; t < TG; ++t)
            acc += ored[(t * G + g) * 8 + j];
        if (direct)
            a.y[h * dv + c] = static_cast<bf16>(acc / l);
        else
            ws[2 + c] = acc;
    }
    if (!direct && tid == 0) {
        ws[0] = m;
        ws[1] = l;
    }
}

// y_h = sum_s o_s exp(m_s - M) / sum_s l_s exp(m_s - M), M = max_s m_s.  The pieces'
// maxima and sums are read by all threads at once and the factors exp(m_s - M) kept in
// LDS (recomputed past kFac pieces); thread (sg, c) then sums column c over the pieces
// s = sg, sg + SG, ..., four loads in flight at a time, and the SG partial sums of a
// column are added through LDS.
constexpr int kFac = 2048;

template <typename TA>
__device__ TA block_reduce(TA v, bool is_max, TA *red)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const TA o = __shfl_xor(v, off, 64);
        v = is_max ? (o > v ? o : v) : v + o;
    }
    __syncthreads();
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = v;
    __syncthreads();
    TA r = red[0];
#pragma unroll
    for (int w = 1; w < kSmThreads / 64; ++w)
        r = is_max ? (red[w] > r ? red[w] : r) : r + red[w];
    return r;
}

template <typename TI, typename TA>
__global__ __launch_bounds__(kSmThreads) void softmax_combine_kernel(SmArgs<TI> a)
{
    __shared__ TA fac[kFac];
    __shared__ TA red[kSmThreads / 64];
    __shared__ TA part[kSmThreads];
    const int tid = threadIdx.x;
    const int64_t h = blockIdx.x;
    const int ns = a.n_splits, dv = a.dv, stride = 2 + dv;
    const TA *ws = static_cast<const TA *>(a.ws) + h * ns * (int64_t)stride;

    TA mloc = -INFINITY;
    for (int s = tid; s < ns; s += kSmThreads)
        mloc = ws[(int64_t)s * stride] > mloc ? ws[(int64_t)s * stride] : mloc;
    const TA M = block_reduce(mloc, true, red);
    TA lloc = 0;
    for (int s = tid; s < ns; s += kSmThreads) {
        const TA f = exp_of(ws[(int64_t)s * stride] - M);
        if (s < kFac)
            fac[s] = f;
        lloc += ws[(int64_t)s * stride + 1] * f;
    }
    const TA lsum = block_reduce(lloc, false, red);  // its barriers also publish fac[]

    const int SG = kSmThreads / dv;  // dv <= 128, so at least 2 groups
    const int c = tid % dv, sg = tid / dv;
    TA acc = 0;
    if (sg < SG) {
        auto factor = [&](int s) { return s < kFac ? fac[s] : exp_of(ws[(int64_t)s * stride] - M); };
        int s = sg;
        for (; s + 3 * SG < ns; s += 4 * SG) {
            const TA o0 = ws[(int64_t)s * stride + 2 + c];
            const TA o1 = ws[(int64_t)(s + SG) * stride + 2 + c];
            const TA o2 = ws[(int64_t)(s + 2 * SG) * stride + 2 + c];
            const TA o3 = ws[(int64_t)(s + 3 * SG) * stride + 2 + c];
            acc += o0 * factor(s) + o1 * factor(s + SG) + o2 * factor(s + 2 * SG) + o3 * factor(s + 3 * SG);
        }
        for (; s < ns; s += SG)
            acc += ws[(int64_t)s * stride + 2 + c] * factor(s);
    }
    part[tid] = acc;
    __syncthreads();
    if (tid < dv) {
        TA y = 0;
        for (int g = 0; g < SG; ++g)
            y += part[g * dv + tid];
        a.y[h * dv + tid] = from_acc<TI>(y / lsum);
    }
}

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <typename TI, typename TA>
hipError_t launch_softmax_typed(const SoftmaxDecodeArgs &s, hipStream_t stream)
{
    SmArgs<TI> a;
    a.q = static_cast<const TI *>(s.q);
    a.k = static_cast<const TI *>(s.k);
    a.v = static_cast<const TI *>(s.v);
    a.Kc = static_cast<TI *>(s.K_cache);
    a.Vc = static_cast<TI *>(s.V_cache);
    a.capacity = s.capacity;
    a.L = s.pos + 1;
    a.d = s.d;
    a.dv = s.dv;
    a.n_splits = (int)softmax_decode_splits(a.L);
    a.scale = s.scale;
    a.ws = s.workspace;
    a.y = static_cast<TI *>(s.y);
    const dim3 grid((unsigned)a.n_splits, (unsigned)s.n_heads);
    const bool vec = std::is_same<TI, bf16>::value && s.d % 8 == 0 && s.dv % 8 == 0 && pow2(s.dv / 8) &&
                     aligned16(s.q) && aligned16(s.k) && aligned16(s.v) && aligned16(s.K_cache) &&
                     aligned16(s.V_cache);
    if constexpr (std::is_same<TI, bf16>::value) {
        if (vec) {
            switch (s.dv / 8) {
            case 1:
                softmax_split_bf16_kernel<1><<<grid, dim3(kSmThreads), 0, stream>>>(a);
                break;
            case 2:
                softmax_split_bf16_kernel<2><<<grid, dim3(kSmThreads), 0, stream>>>(a);
                break;
            case 4:
                softmax_split_bf16_kernel<4><<<grid, dim3(kSmThreads), 0, stream>>>(a);
                break;
            case 8:
                softmax_split_bf16_kernel<8><<<grid, dim3(kSmThreads), 0, stream>>>(a);
                break;
            default:
                softmax_split_bf16_kernel<16><<<grid, dim3(kSmThreads), 0, stream>>>(a);
                break;
            }
        } else {
            softmax_split_kernel<TI, TA><<<grid, dim3(kSmThreads), 0, stream>>>(a);
        }
    } else {
        softmax_split_kernel<TI, TA><<<grid, dim3(kSmThreads), 0, stream>>>(a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.n_splits == 1)
        return e;
    softmax_combine_kernel<TI, TA><<<dim3((unsigned)s.n_heads), dim3(kSmThreads), 0, stream>>>(a);
    return hipGetLastError();
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

}  // namespace

// The fixed scratch of la_softmax_decode_step_static.  In host code `scratch` names a
// host-side stand-in, not device memory: kernels get the address that
// hipGetSymbolAddress returns for the current device (each GPU holds its own copy).
static __device__ __align__(256) unsigned char scratch[LA_SOFTMAX_STATIC_WORKSPACE_BYTES];

hipError_t softmax_static_workspace(void **ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

int64_t softmax_decode_splits(int64_t L) { return (L + kSplit - 1) / kSplit; }

hipError_t launch_softmax_decode(const SoftmaxDecodeArgs &a, la_dtype io_dtype, hipStream_t stream)
{
    switch (io_dtype) {
    case LA_F64:
        return launch_softmax_typed<double, double>(a, stream);
    case LA_F32:
        return launch_softmax_typed<float, float>(a, stream);
    default:
        return launch_softmax_typed<bf16, float>(a, stream);
    }
}

}  // namespace la
