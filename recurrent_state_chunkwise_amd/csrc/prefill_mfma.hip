// bf16 MFMA chunked prefill for d = dv = 128, chunk 64 or 128, fp32 state.
//
// Computes, per chunk c with carried state S_prev, z_prev, the chunk equations of the
// page "Linear attention：把历史写进状态" (hs-black.github.io), section "一个 chunk 的
// 输出由两部分组成":
//   numerator   = Q~c S_prev + [(Q~c K~c^T) . M] Vc
//   denominator = Q~c z_prev + rowsum[(Q~c K~c^T) . M]
//   S_next = S_prev + K~c^T Vc,   z_next = z_prev + sum of the rows of K~c
// and y = numerator / (denominator + eps).  The gate of section "加一个门" enters as the
// page asks ("门控版本要加入门乘积"): with L_j the sum of log(alpha) over the chunk up to
// token j, score (j, i) is weighted by exp(L_j - L_i), the read of S_prev and z_prev by
// exp(L_j), the write of token i by exp(L_last - L_i) and the carried state by
// exp(L_last); a zero gate inside (i, j] makes the weight exactly 0.
//
// Parallel structure.  A sequence is cut into segments.  Because one gated update is
// the affine map S -> a S + k~ v^T and such maps compose associatively (section "门控
// 递推为什么能做并行 scan"), the state entering each segment is obtained by
//   pass 1  summarise: each (sequence, segment) computes its own map (G, dS, dz) by
//           running the chunk write from a zero state;
//   pass 2  scan:      the entering state of segment p is G_{p-1} S_in(p-1) + dS_{p-1};
//   pass 3  prefill:   each (sequence, segment) runs the chunk equations from its
//           entering state, writing y and, for the last segment, the final S and z.
// phi is evaluated once per token and pass, every compute unit gets a whole
// (sequence, segment), and the segment maps and entering states are parked in the
// caller's output buffer Y inside the segment they belong to (each needs 66 KB, less
// than one segment's share of Y); pass 3 reads its slot before it writes any output.
//
// Inside a workgroup (8 waves, all 128 value columns) every product is
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation:
//   (1) A^T = K~ Q~^T, 16x16 tiles on or below the diagonal spread over the waves; the
//       fp32 tile is masked and gate-weighted, its row sums feed the denominator and
//       its accumulator layout is stored per lane as the A operand of (3);
//   (2) N  = Q~ S_prev with S_prev taken from the fp32 state accumulators of the wave
//   (3) N += A V
//   (4) S  = g_last S + (w K~)^T V
// Wave w owns value columns 16w..16w+15 of N and of S, so S never leaves registers.
#include "device_common.hpp"
#include "internal.hpp"

namespace la {
namespace {

typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;          // feature width d = r and value width dv
constexpr int kThreads = 512;    // 8 waves
constexpr float kLog2e = 1.4426950408889634f;

// (sequence, segment) workgroups aimed for, per chunk size: one or two per compute unit
#ifndef LA_SEGMENT_TARGET_C64
#define LA_SEGMENT_TARGET_C64 256
#endif
#ifndef LA_SEGMENT_TARGET_C128
#define LA_SEGMENT_TARGET_C128 256
#endif

// per-(sequence, segment) slot in Y: S [128][128], z [128], segment gate product, pad
constexpr int kSlotFloats = kD * kD + kD + 4;
constexpr int64_t kMinSegTokens = (kSlotFloats * 4 + kD * 2 - 1) / (kD * 2);

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 8 packed bf16 -> 8 floats
__device__ __forceinline__ void unpack8(uint4 u, float *f)
{
    const unsigned w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

// phi = ELU + 1 as the median of (x + 1, e^x, 1): x + 1 for x > 0 (where e^x > x + 1 > 1)
// and e^x for x <= 0 (where x + 1 <= e^x <= 1); e^x on the hardware exp2
__device__ __forceinline__ float phi(float x)
{
    return __builtin_amdgcn_fmed3f(x + 1.f, __builtin_amdgcn_exp2f(x * kLog2e), 1.f);
}

// Buffer resources (gfx9 raw buffers): an access at or past num_records bytes reads
// zeros and drops writes, which is how the last, partial chunk of a segment is handled.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(rsrc_t r, int off)
{
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// low / high bf16 halves of two dwords packed into one dword (x in the low half)
__device__ __forceinline__ unsigned pack_lo(unsigned x, unsigned y) { return __builtin_amdgcn_perm(y, x, 0x05040100u); }
__device__ __forceinline__ unsigned pack_hi(unsigned x, unsigned y) { return __builtin_amdgcn_perm(y, x, 0x07060302u); }

template <int C>
struct Cfg {
    static constexpr int NTJ = C / 16;                 // 16-token tiles per chunk
    static constexpr int NKI = C / 32;                 // 32-token MFMA steps per chunk
    static constexpr int TPT = C / 32;                 // tokens per staging thread
    static constexpr int NPT = NTJ * (NTJ + 1) / 2;    // tiles on or below the diagonal
};

// LDS.  Row-major tiles (Qs, Ks) hold 128 features per token; the token-major tiles
// (KwT: features x tokens, VT: values x tokens) are the K-contiguous operands of the
// contractions over tokens.  16-byte granules are XOR-swizzled per row so that the
// 16 rows read by one MFMA operand land in distinct banks.
template <int C, bool SUMMARY>
struct alignas(16) Smem {
    typedef Cfg<C> G;
    static constexpr int QN = SUMMARY ? 1 : C * kD;
    static constexpr int PN = SUMMARY ? 1 : G::NPT;
    alignas(16) bf16 Qs[1][QN];             // phi(q) rows
    alignas(16) bf16 Ks[1][QN];             // phi(k) rows; after the scores, output staging
    alignas(16) bf16 KwT[1][kD * C];
    alignas(16) bf16 VT[1][kD * C];
    alignas(16) uint2 P[PN * 64];           // bf16 A tiles, one 4-value group per lane
    alignas(16) float rs[PN * 16];          // row sums of each A tile
    alignas(16) float zpart[1][8 * kD];     // per-wave partial sums of w phi(k)
    alignas(16) float zs[kD];
    alignas(16) float den_q[1][C];          // phi(q_j) . z_prev
    alignas(16) float ivd[C];               // 1 / (denominator + eps)
    alignas(16) float lg[2][C];             // in-chunk prefix sum of log(alpha) (0 at zero gates)
    alignas(16) float gj[2][C];             // product of the chunk's gates up to j
    alignas(16) int zp[2][C];               // last zero gate at or before j, -1 if none
};

// Sum over the 16 lanes of a DPP row, result in every lane of the row.
__device__ __forceinline__ float row_sum16(float v)
{
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false));  // row_ror:8
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, false));  // row_ror:4
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xf, 0xf, false));  // row_ror:2
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xf, 0xf, false));  // row_ror:1
    return v;
}
// v[l] + v[l ^ 16] and v[l] + v[l ^ 32] with the gfx950 lane-swap instructions
__device__ __forceinline__ float xor16_sum(float v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// swizzled element offsets
__device__ __forceinline__ int qk_off(int row, int col)  // [C][128]
{
    return row * kD + ((((col >> 3) ^ (row & 15)) << 3) | (col & 7));
}
template <int C>
__device__ __forceinline__ int tm_off(int row, int tok)  // [128][C]
{
    int h;
    if constexpr (C == 128)
        h = (row + (row >> 4)) & 15;
    else
        h = (row >> 1) & 7;
    return row * C + ((((tok >> 3) ^ h) << 3) | (tok & 7));
}

struct Args {
    const bf16 *Q, *K, *V;
    const float *alpha;
    bf16 *Y;
    float *S, *z;
    int64_t T;
    int64_t seg_len;
    int nseg;
    float eps;
};

__device__ __forceinline__ float *slot_ptr(const Args &a, int64_t head, int p)
{
    return reinterpret_cast<float *>(a.Y + (head * a.T + (int64_t)p * a.seg_len) * kD);
}

// SUMMARY: pass 1 (segment map from a zero state, written to the next segment's slot).
// FULL:    pass 3 (outputs from the entering state; the last segment writes S, z).
template <int C, bool GATED, bool SUMMARY>
__global__ __launch_bounds__(kThreads) void chunk_kernel(Args a)
{
    typedef Cfg<C> G;
    __shared__ Smem<C, SUMMARY> sm;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lr = lane & 15;   // row / column inside a 16x16 tile
    const int lg4 = lane >> 4;  // lane group

    const int64_t head = blockIdx.x / a.nseg;
    const int seg = blockIdx.x % a.nseg;
    if (SUMMARY && seg == a.nseg - 1)
        return;  // the last segment's map is never needed
    const int64_t s0 = (int64_t)seg * a.seg_len;
    const int64_t s1 = seg == a.nseg - 1 ? a.T : s0 + a.seg_len;
    const int64_t len = s1 - s0;
    const int n_chunks = (int)((len + C - 1) / C);
    auto chunk_len = [&](int c) { return (int)min((int64_t)C, len - (int64_t)c * C); };

    // this segment's rows of Q, K, V, Y (256 bytes per token) and of alpha (4 bytes)
    const int64_t row0 = head * a.T + s0;
    const rsrc_t rQ = make_rsrc(a.Q + row0 * kD, len * kD * 2);
    const rsrc_t rK = make_rsrc(a.K + row0 * kD, len * kD * 2);
    const rsrc_t rV = make_rsrc(a.V + row0 * kD, len * kD * 2);
    const rsrc_t rY = make_rsrc(a.Y + row0 * kD, len * kD * 2);
    const rsrc_t rA = make_rsrc(GATED ? a.alpha + row0 : a.S, GATED ? len * 4 : 0);

    // ---------------------------------------------------------------- entering state
    // wave w owns value columns c = 16w + lr; tile tf holds rows f = 16tf + 4lg4 + r
    f32x4 sacc[8];
    const int cw = wave * 16 + lr;
    if (SUMMARY) {
#pragma unroll
        for (int tf = 0; tf < 8; ++tf)
            sacc[tf] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (tid < kD)
            sm.zs[tid] = 0.f;
    } else {
        const float *Sin = a.nseg == 1 ? a.S + head * kD * kD : slot_ptr(a, head, seg);
        const float *zin = a.nseg == 1 ? a.z + head * kD : Sin + kD * kD;
#pragma unroll
        for (int tf = 0; tf < 8; ++tf)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sacc[tf][r] = Sin[(tf * 16 + lg4 * 4 + r) * kD + cw];
        if (tid < kD)
            sm.zs[tid] = zin[tid];
    }
    float g_seg = 1.f;  // product of all gates of the segment (SUMMARY)

    // ---------------------------------------------------------------- loads
    // every thread stages TPT consecutive tokens of one 8-wide granule of Q, K and V:
    // thread (fg, tg) holds granule fg of tokens tg*TPT .. tg*TPT + TPT - 1
    const int fg = tid & 15, tg = tid >> 4;
    uint4 raw_q[G::TPT], raw_k[G::TPT], raw_v[G::TPT];
    float araw[C / 64];
    const int ld_off = (tg * G::TPT) * kD * 2 + fg * 16;  // byte offset of this thread's first row

    auto prefetch_k = [&](int chunk) {
        const int off = chunk * C * kD * 2 + ld_off;
#pragma unroll
        for (int p = 0; p < G::TPT; ++p)
            raw_k[p] = bload16(rK, off + p * kD * 2);
    };
    auto prefetch_qv = [&](int chunk) {
        const int off = chunk * C * kD * 2 + ld_off;
#pragma unroll
        for (int p = 0; p < G::TPT; ++p) {
            if (!SUMMARY)
                raw_q[p] = bload16(rQ, off + p * kD * 2);
            raw_v[p] = bload16(rV, off + p * kD * 2);
        }
    };
    auto prefetch_a = [&](int chunk) {
        if (GATED && wave == 0) {
#pragma unroll
            for (int h = 0; h < C / 64; ++h)
                araw[h] = __uint_as_float(
                    (unsigned)__builtin_amdgcn_raw_buffer_load_b32(rA, (chunk * C + h * 64 + lane) * 4, 0, 0));
        }
    };

    // ---------------------------------------------------------------- gates
    // wave 0: inclusive scans of log(alpha) and of the last zero-gate position
    auto gate_scan = [&](int n, int gs) {
        if (GATED && wave == 0) {
            float carry = 0.f;
            int zcarry = -1;
#pragma unroll
            for (int h = 0; h < C / 64; ++h) {
                const int j = h * 64 + lane;
                const float av = j < n ? araw[h] : 1.f;
                float s = av > 0.f ? __logf(av) : 0.f;
                int zf = av == 0.f ? j : -1;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const float s2 = __shfl_up(s, off, 64);
                    const int z2 = __shfl_up(zf, off, 64);
                    if (lane >= off) {
                        s += s2;
                        zf = max(zf, z2);
                    }
                }
                s += carry;
                zf = max(zf, zcarry);
                sm.lg[gs][j] = s;
                sm.zp[gs][j] = zf;
                sm.gj[gs][j] = zf >= 0 ? 0.f : __expf(s);
                carry = __shfl(s, 63, 64);
                zcarry = __shfl(zf, 63, 64);
            }
        }
    };
    auto pair_decay = [&](int gs, int j, int i) -> float {  // gates of tokens i+1..j
        return sm.zp[gs][j] > i ? 0.f : __expf(sm.lg[gs][j] - sm.lg[gs][i]);
    };

    // ---------------------------------------------------------------- staging
    // keys: phi, row-major K~ for the scores, gate-weighted token-major K~ for the state
    // write, and the partial normaliser sums.  Tokens past the end of the segment load as
    // zeros: their V rows are zero, so they add nothing to the state; they are masked in
    // the scores by causality and in the normaliser by w = 0.
    auto stage_k = [&](int n, int gs, int buf) {
        float zacc[8];
#pragma unroll
        for (int s = 0; s < 8; ++s)
            zacc[s] = 0.f;
        unsigned kwp[G::TPT][4];  // bf16 pairs of w*phi(k)
#pragma unroll
        for (int p = 0; p < G::TPT; ++p) {
            const int j = tg * G::TPT + p;
            const float w = j >= n ? 0.f : (GATED ? pair_decay(gs, n - 1, j) : 1.f);
            float x[8];
            unpack8(raw_k[p], x);
            bf16x8 kb;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const float f = phi(x[s]);
                kb[s] = static_cast<bf16>(f);
                zacc[s] = fmaf(w, f, zacc[s]);
                if (GATED)
                    x[s] = w * f;
            }
            if (!SUMMARY)
                *reinterpret_cast<bf16x8 *>(&sm.Ks[buf][qk_off(j, fg * 8)]) = kb;
            uint4 u;
            if (GATED) {
                bf16x8 kwb;
#pragma unroll
                for (int s = 0; s < 8; ++s)
                    kwb[s] = static_cast<bf16>(x[s]);
                u = *reinterpret_cast<uint4 *>(&kwb);
            } else {
                u = *reinterpret_cast<uint4 *>(&kb);
            }
            kwp[p][0] = u.x, kwp[p][1] = u.y, kwp[p][2] = u.z, kwp[p][3] = u.w;
        }
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int row = fg * 8 + s;
            unsigned o[G::TPT / 2];
#pragma unroll
            for (int q = 0; q < G::TPT / 2; ++q)
                o[q] = (s & 1) ? pack_hi(kwp[2 * q][s >> 1], kwp[2 * q + 1][s >> 1])
                               : pack_lo(kwp[2 * q][s >> 1], kwp[2 * q + 1][s >> 1]);
            if constexpr (G::TPT == 2)
                *reinterpret_cast<unsigned *>(&sm.KwT[buf][tm_off<C>(row, tg * 2)]) = o[0];
            else
                *reinterpret_cast<uint2 *>(&sm.KwT[buf][tm_off<C>(row, tg * 4)]) = make_uint2(o[0], o[1]);
            zacc[s] = xor32_sum(xor16_sum(zacc[s]));
        }
        if (lg4 == 0) {
#pragma unroll
            for (int s = 0; s < 8; ++s)
                sm.zpart[buf][wave * kD + fg * 8 + s] = zacc[s];
        }
    };
    // queries: phi, row-major Q~ and the read of z_prev (z in sm.zs)
    auto stage_q = [&](int buf) {
#pragma unroll
        for (int p = 0; p < G::TPT; ++p) {
            const int j = tg * G::TPT + p;
            float x[8];
            unpack8(raw_q[p], x);
            bf16x8 qb;
            float dot = 0.f;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const float f = phi(x[s]);
                qb[s] = static_cast<bf16>(f);
                dot = fmaf(f, sm.zs[fg * 8 + s], dot);
            }
            *reinterpret_cast<bf16x8 *>(&sm.Qs[buf][qk_off(j, fg * 8)]) = qb;
            dot = row_sum16(dot);
            if (fg == 0)
                sm.den_q[buf][j] = dot;
        }
    };
    // values -> token-major VT: value column 8fg+s gets this thread's TPT tokens
    auto stage_v = [&](int buf) {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int row = fg * 8 + s;
            unsigned o[G::TPT / 2];
#pragma unroll
            for (int q = 0; q < G::TPT / 2; ++q) {
                const unsigned lo = (&raw_v[2 * q].x)[s >> 1], hi = (&raw_v[2 * q + 1].x)[s >> 1];
                o[q] = (s & 1) ? pack_hi(lo, hi) : pack_lo(lo, hi);
            }
            if constexpr (G::TPT == 2)
                *reinterpret_cast<unsigned *>(&sm.VT[buf][tm_off<C>(row, tg * 2)]) = o[0];
            else
                *reinterpret_cast<uint2 *>(&sm.VT[buf][tm_off<C>(row, tg * 4)]) = make_uint2(o[0], o[1]);
        }
    };

    // ---------------------------------------------------------------- chunk products
    // (1) A tiles on or below the diagonal, distributed over the waves
    auto scores = [&](int buf, int gs) {
        for (int k = wave; k < G::NPT; k += 8) {
            int tj = 0;
            while ((tj + 1) * (tj + 2) / 2 <= k)
                ++tj;
            const int ti = k - tj * (tj + 1) / 2;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kf = 0; kf < 4; ++kf) {
                const bf16x8 ka =
                    *reinterpret_cast<const bf16x8 *>(&sm.Ks[buf][qk_off(ti * 16 + lr, kf * 32 + lg4 * 8)]);
                const bf16x8 qb =
                    *reinterpret_cast<const bf16x8 *>(&sm.Qs[buf][qk_off(tj * 16 + lr, kf * 32 + lg4 * 8)]);
                acc = mfma(ka, qb, acc);
            }
            // acc[r] = A[j][i], j = 16tj + lr, i = 16ti + 4lg4 + r
            const int j = tj * 16 + lr;
            float rsum = 0.f;
            bf16x4 pk;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = ti * 16 + lg4 * 4 + r;
                float v = i <= j ? acc[r] : 0.f;
                if (GATED && i <= j)
                    v *= pair_decay(gs, j, i);
                rsum += v;
                pk[r] = static_cast<bf16>(v);
            }
            sm.P[k * 64 + lane] = *reinterpret_cast<uint2 *>(&pk);
            rsum = xor32_sum(xor16_sum(rsum));
            if (lg4 == 0)
                sm.rs[k * 16 + lr] = rsum;
        }
    };
    // 1 / (denominator + eps) for chunk rows j0, j0 + step, ...
    auto inv_den = [&](int buf, int gs, float *dst, int j0, int step) {
        for (int j = j0; j < C; j += step) {
            const int tj = j >> 4, jr = j & 15;
            float d = 0.f;
            for (int ti = 0; ti <= tj; ++ti)
                d += sm.rs[(tj * (tj + 1) / 2 + ti) * 16 + jr];
            const float inter = GATED ? sm.gj[gs][j] * sm.den_q[buf][j] : sm.den_q[buf][j];
            dst[j] = 1.f / (inter + d + a.eps);
        }
    };
    // (2) + (3) for this wave's 16 value columns, outputs through the dead K~ tile
    auto outputs = [&](int buf, int gs, int64_t t0, const float *ivd) {
        bf16 *ystage = sm.Ks[buf] + wave * (C * 16);
        // S_prev as the B operand: K step kf takes feature tiles 2kf and 2kf+1, whose
        // accumulator rows 4lg4..4lg4+3 give the permuted k order used on both sides
        bf16x8 sb[4];
#pragma unroll
        for (int kf = 0; kf < 4; ++kf)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sb[kf][r] = static_cast<bf16>(sacc[2 * kf][r]);
                sb[kf][4 + r] = static_cast<bf16>(sacc[2 * kf + 1][r]);
            }
#pragma unroll 1
        for (int tj = 0; tj < G::NTJ; ++tj) {
            const int j = tj * 16 + lr;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kf = 0; kf < 4; ++kf) {
                const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(&sm.Qs[buf][qk_off(j, kf * 32 + lg4 * 4)]);
                const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(&sm.Qs[buf][qk_off(j, kf * 32 + 16 + lg4 * 4)]);
                const bf16x8 qa = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                acc = mfma(qa, sb[kf], acc);
            }
            if (GATED) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[r] *= sm.gj[gs][tj * 16 + lg4 * 4 + r];
            }
            for (int ki = 0; 2 * ki <= tj; ++ki) {
                const int k1 = tj * (tj + 1) / 2 + 2 * ki;
                const uint2 p1 = sm.P[k1 * 64 + lane];
                const uint2 p2 = 2 * ki + 1 <= tj ? sm.P[(k1 + 1) * 64 + lane] : make_uint2(0u, 0u);
                const bf16x4 a1 = *reinterpret_cast<const bf16x4 *>(&p1);
                const bf16x4 a2 = *reinterpret_cast<const bf16x4 *>(&p2);
                const bf16x8 pa = {a1[0], a1[1], a1[2], a1[3], a2[0], a2[1], a2[2], a2[3]};
                const bf16x4 vlo = *reinterpret_cast<const bf16x4 *>(&sm.VT[buf][tm_off<C>(cw, ki * 32 + lg4 * 4)]);
                const bf16x4 vhi =
                    *reinterpret_cast<const bf16x4 *>(&sm.VT[buf][tm_off<C>(cw, ki * 32 + 16 + lg4 * 4)]);
                const bf16x8 vb = {vlo[0], vlo[1], vlo[2], vlo[3], vhi[0], vhi[1], vhi[2], vhi[3]};
                acc = mfma(pa, vb, acc);
            }
            // stage the 16 columns of this wave: row j, 16-byte granule (col >> 3)
            // swapped on odd multiples of 8 rows to spread the rows over the banks
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int jj = tj * 16 + lg4 * 4 + r;
                const int g = (lr >> 3) ^ ((jj >> 3) & 1);
                ystage[jj * 16 + g * 8 + (lr & 7)] = static_cast<bf16>(acc[r] * ivd[jj]);
            }
        }
        // write this wave's C x 16 block as 16-byte row segments; rows past the end of
        // the segment fall outside rY and are dropped
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int q = 0; q < C / 32; ++q) {
            const int idx = q * 64 + lane;
            const int jj = idx >> 1, g = idx & 1;
            const uint4 v = *reinterpret_cast<const uint4 *>(&ystage[jj * 16 + ((g ^ ((jj >> 3) & 1)) * 8)]);
            const int off = (int)((t0 + jj) * kD + wave * 16 + g * 8) * 2;
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, v), rY, off, 0, 0);
        }
    };
    // (4) S = g_end S + (w K~)^T V for this wave's columns
    auto state_write = [&](int buf, float g_end) {
        if (GATED) {
#pragma unroll
            for (int tf = 0; tf < 8; ++tf)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sacc[tf][r] *= g_end;
        }
#pragma unroll
        for (int ki = 0; ki < G::NKI; ++ki) {
            const bf16x8 vb = *reinterpret_cast<const bf16x8 *>(&sm.VT[buf][tm_off<C>(cw, ki * 32 + lg4 * 8)]);
#pragma unroll
            for (int tf = 0; tf < 8; ++tf) {
                const bf16x8 ka =
                    *reinterpret_cast<const bf16x8 *>(&sm.KwT[buf][tm_off<C>(tf * 16 + lr, ki * 32 + lg4 * 8)]);
                sacc[tf] = mfma(ka, vb, sacc[tf]);
            }
        }
    };
    // z = g_end z + sum of this chunk's w phi(k) (threads 0..127)
    auto z_update = [&](int buf, float g_end) {
        if (tid < kD) {
            float zsum = 0.f;
#pragma unroll
            for (int w8 = 0; w8 < 8; ++w8)
                zsum += sm.zpart[buf][w8 * kD + tid];
            sm.zs[tid] = g_end * sm.zs[tid] + zsum;
        }
    };

    // ---------------------------------------------------------------- walk: stage, then multiply
    prefetch_k(0);
    prefetch_qv(0);
    prefetch_a(0);
    gate_scan(chunk_len(0), 0);
    __syncthreads();

    for (int c = 0; c < n_chunks; ++c) {
        const int64_t t0 = (int64_t)c * C;
        const int n = chunk_len(c);
        const int gs = c & 1;
        const bool more = c + 1 < n_chunks;

        stage_k(n, gs, 0);
        if (!SUMMARY)
            stage_q(0);
        stage_v(0);
        if (more) {
            prefetch_k(c + 1);
            prefetch_qv(c + 1);
            prefetch_a(c + 1);
        }
        __syncthreads();  // A: chunk staged

        if (!SUMMARY) {
            scores(0, gs);
            __syncthreads();  // B: A tiles and row sums ready
            inv_den(0, gs, sm.ivd, tid, kThreads);
            __syncthreads();  // B': denominators ready
            outputs(0, gs, t0, sm.ivd);
        }
        const float g_end = GATED ? sm.gj[gs][n - 1] : 1.f;
        if (GATED)
            g_seg *= g_end;
        state_write(0, g_end);
        z_update(0, g_end);
        if (more)
            gate_scan(chunk_len(c + 1), gs ^ 1);
        __syncthreads();  // C: chunk done
    }

    // ---------------------------------------------------------------- leaving state
    float *Sout, *zout;
    if (SUMMARY) {
        Sout = slot_ptr(a, head, seg + 1);
        zout = Sout + kD * kD;
        if (tid == 0)
            Sout[kD * kD + kD] = g_seg;
    } else {
        if (seg != a.nseg - 1)
            return;
        Sout = a.S + head * kD * kD;
        zout = a.z + head * kD;
    }
#pragma unroll
    for (int tf = 0; tf < 8; ++tf)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            Sout[(tf * 16 + lg4 * 4 + r) * kD + cw] = sacc[tf][r];
    if (tid < kD)
        zout[tid] = sm.zs[tid];
}

// Pass 2: entering state of every segment, in place over the segment maps.
// slot 0 <- (S0, z0); slot p <- G_{p-1} slot(p-1) + dS_{p-1}   (p = 1 .. nseg-1)
// The maps are read 8 at a time before the chain runs, so the loads overlap.
__global__ __launch_bounds__(256) void segment_scan_kernel(Args a)
{
    const int64_t head = blockIdx.y;
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= kD * kD + kD)
        return;
    float run = e < kD * kD ? a.S[head * kD * kD + e] : a.z[head * kD + (e - kD * kD)];
    slot_ptr(a, head, 0)[e] = run;
    constexpr int kBatch = 8;
    for (int p0 = 1; p0 < a.nseg; p0 += kBatch) {
        float d[kBatch], g[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            if (p0 + q < a.nseg) {
                const float *sl = slot_ptr(a, head, p0 + q);
                d[q] = sl[e];
                g[q] = sl[kD * kD + kD];
            }
        }
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            if (p0 + q < a.nseg) {
                run = g[q] * run + d[q];
                slot_ptr(a, head, p0 + q)[e] = run;
            }
        }
    }
}

template <int C, bool GATED>
hipError_t launch_c(const Args &a, int64_t n_heads, hipStream_t stream)
{
    const unsigned blocks = (unsigned)(n_heads * a.nseg);
    if (a.nseg > 1) {
        // pass 1 walks 128-token chunks whatever the caller's chunk: its chunking only
        // changes the rounding of the segment maps, and longer chunks keep more bytes
        // in flight
        chunk_kernel<128, GATED, true><<<dim3(blocks), dim3(kThreads), 0, stream>>>(a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        segment_scan_kernel<<<dim3((kD * kD + kD + 255) / 256, (unsigned)n_heads), dim3(256), 0, stream>>>(a);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    chunk_kernel<C, GATED, false><<<dim3(blocks), dim3(kThreads), 0, stream>>>(a);
    return hipGetLastError();
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

bool mfma_prefill_supported(la_dtype io_dtype, int32_t d, int32_t dv, int32_t chunk)
{
    return io_dtype == LA_BF16 && d == kD && dv == kD && (chunk == 64 || chunk == 128);
}

hipError_t launch_prefill_mfma_bf16(const PrefillArgs &pa, hipStream_t stream)
{
    if (!aligned16(pa.Q) || !aligned16(pa.K) || !aligned16(pa.V) || !aligned16(pa.Y))
        return launch_prefill_general(pa, LA_BF16, stream);
    Args a;
    a.Q = static_cast<const bf16 *>(pa.Q);
    a.K = static_cast<const bf16 *>(pa.K);
    a.V = static_cast<const bf16 *>(pa.V);
    a.alpha = static_cast<const float *>(pa.alpha);
    a.Y = static_cast<bf16 *>(pa.Y);
    a.S = static_cast<float *>(pa.S);
    a.z = static_cast<float *>(pa.z);
    a.T = pa.T;
    a.eps = (float)pa.eps;

    // Segments: enough (sequence, segment) workgroups to give every compute unit
    // work (two resident workgroups per unit at chunk 64, one at chunk 128), each
    // segment a whole number of chunks and long enough to hold its slot in Y.
    const int C = pa.chunk;
    const int64_t target = C == 64 ? LA_SEGMENT_TARGET_C64 : LA_SEGMENT_TARGET_C128;
    int64_t nseg = (target + pa.n_heads - 1) / pa.n_heads;
    const int64_t min_len = ((kMinSegTokens + C - 1) / C) * C;
    if (nseg > pa.T / min_len)
        nseg = pa.T / min_len;
    // buffer offsets are 32-bit: keep every segment (the last may be up to twice as
    // long) below 2^31 bytes of Q
    const int64_t max_len = ((int64_t)1 << 31) / (kD * 2) / 2;
    if (nseg < (pa.T + max_len - 1) / max_len)
        nseg = (pa.T + max_len - 1) / max_len;
    if (nseg < 1)
        nseg = 1;
    if (pa.n_heads * nseg > INT32_MAX)
        return hipErrorInvalidValue;
    a.nseg = (int)nseg;
    a.seg_len = nseg == 1 ? pa.T : ((pa.T / nseg) / C) * C;  // the last segment takes the rest

    if (C == 64)
        return pa.alpha ? launch_c<64, true>(a, pa.n_heads, stream) : launch_c<64, false>(a, pa.n_heads, stream);
    return pa.alpha ? launch_c<128, true>(a, pa.n_heads, stream) : launch_c<128, false>(a, pa.n_heads, stream);
}

}  // namespace la
