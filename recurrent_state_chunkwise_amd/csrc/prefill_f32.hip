// fp32-arithmetic MFMA chunked prefill at chunk 64, fp32 state: d = dv = 128 with fp32
// inputs, and d = dv = 64 with fp32 or bf16 inputs (bf16 values widen to fp32 exactly).
//
// The chunk equations of the page "Linear attention：把历史写进状态" (hs-black.github.io),
// section "一个 chunk 的输出由两部分组成", with the gate products of section "加一个门" folded
// in as in the bf16 kernels (log-sums of alpha inside a chunk, zero gates exact), over the
// same segment-parallel structure (section "门控递推为什么能做并行 scan"): pass 1 forms each
// segment's map (G, dS, dz) from a zero state, pass 2 (segment_scan_kernel) chains them
// into the state entering every segment, pass 3 runs the chunks of every segment from its
// entering state, writing y and, for the last segment, the final S and z.
//
// Every product is v_mfma_f32_16x16x4_f32 on fp32 operands with fp32 accumulation, so
// nothing is rounded below fp32 before y is stored.  Lane (lr, g) of a 16x16x4 product
// supplies A[lr][g] and B[g][lr]; lane (lr, g) of its 16x16 result holds rows 4g .. 4g+3
// of column lr.  The contraction order is permuted so that the operands come straight out
// of registers or one 16-byte LDS read serves four products:
//   (2) N^T = S_prev^T Q~^T: K step (tf, r) takes features 16tf + 4g + r, whose S_prev
//       values are exactly the wave's accumulator register sacc[tf][r];
//   (1) scores K~ Q~^T and the denominator part phi(q) . z_prev: the same feature order;
//   (3) N^T += V^T P^T: K step (ti, r) takes tokens 16ti + 4g + r, whose score values are
//       register r of the score tile's accumulator lane (lr, g), kept in LDS in that layout;
//   (4) S += (w K~)^T V: K step (u, r) takes tokens 16u + 4g + r.
// Q~ and K~ are staged token-major (rows of D floats), V and the write weights
// feature-major (rows of 64 tokens), each row padded by 4 floats, so that every operand
// is a float4 per lane and each 16-lane group reads 64 distinct banks.
//
// One workgroup of D/16 waves per (sequence, segment); wave w owns value columns
// 16w .. 16w+15 of S and of the outputs.  Per chunk all waves first stage the chunk
// (feature map, write weights, transposes) from the registers into which its raw rows were
// loaded during the previous chunk's products, then do the products; the products take
// several times the memory time of a chunk, so the loads have that long to arrive.  The row
// sums of the masked scores (the intra-chunk denominator) are formed in fp32 from the
// scores, z from the fp32 write weights.  At D = 64 the tiles take under 80 KB of LDS, so
// two workgroups share a compute unit.
#include <type_traits>

#include "device_common.hpp"
#include "internal.hpp"
#include "prefill_common.hpp"

namespace la {
namespace {

constexpr int kFC = 64;      // chunk
constexpr int kTRow = kFC + 4;  // row of the feature-major tiles, in floats (272 bytes)
constexpr int kFTiles = 10;  // 16x16 score tiles on or below the diagonal of a chunk

template <int D>
struct FShape {
    static_assert(D == 64 || D == 128, "the fp32-arithmetic prefill takes d = dv = 64 or 128");
    static constexpr int tiles = D / 16;    // 16-wide feature or value tiles, = waves
    static constexpr int threads = 64 * tiles;
    static constexpr int quads = D / 4;     // 4-feature pieces of a row
    static constexpr int qrow = D + 4;      // row of the token-major tiles, in floats
};

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <typename TI, int D>
struct FArgs {
    const TI *Q, *K, *V;
    const float *alpha;
    TI *Y;
    float *S, *z;
    int64_t T;
    int64_t seg_len;
    int nseg;
    float eps;
};

// slot p of a sequence: S [D][D], z [D] and the segment's gate product, parked in the first
// rows of segment p of Y
template <typename TI, int D>
__device__ __forceinline__ float *slot_ptr(const FArgs<TI, D> &a, int64_t head, int p)
{
    return reinterpret_cast<float *>(a.Y + (head * a.T + (int64_t)p * a.seg_len) * D);
}

// Raw rows of one chunk held in registers between their load and their staging: thread
// (fq, tq) holds features 4fq .. 4fq+3 of tokens 4tq .. 4tq+3 (fq = tid mod D/4,
// tq = tid div D/4, 0 .. 15), so that the feature-major tiles are written as float4 runs of
// 4 tokens.
struct Quad {
    f32x4 x[4];  // x[s] = the 4 features of token 4tq + s
};

template <typename TI, int D>
__device__ __forceinline__ void load_quad(rsrc_t r, int c, int fq, int tq, Quad &q)
{
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int e = (c * kFC + 4 * tq + s) * D + 4 * fq;  // element offset in the segment
        if constexpr (std::is_same_v<TI, float>) {
            const uint4 u = bload16(r, e * 4);
            q.x[s] = f32x4{__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w)};
        } else {
            const auto u = __builtin_amdgcn_raw_buffer_load_b64(r, e * 2, 0, 0);
            q.x[s] = f32x4{__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xffff0000u),
                           __uint_as_float(u[1] << 16), __uint_as_float(u[1] & 0xffff0000u)};
        }
    }
}

template <int FM>
__device__ __forceinline__ f32x4 phi4(f32x4 x)
{
    return f32x4{phi<FM>(x[0]), phi<FM>(x[1]), phi<FM>(x[2]), phi<FM>(x[3])};
}

// Gates of the chunk of n tokens from alpha of token `lane` (one wave): inclusive scans of
// log(alpha) (zero gates left out) and of the last zero-gate position, and the product of
// the gates from the chunk start, 0 after a zero gate.
__device__ __forceinline__ void scan_gates(float av_raw, int n, int lane, float *lg, int *zp, float *gj)
{
    const float av = lane < n ? av_raw : 1.f;
    float s = av > 0.f ? __logf(av) : 0.f;
    int zf = av == 0.f ? lane : -1;
    s = wave_scan_add(s);
    zf = wave_scan_max(zf);
    lg[lane] = s;
    zp[lane] = zf;
    gj[lane] = zf >= 0 ? 0.f : __expf(s);
}

// Write weights of one token quad: w phi(k) feature-major into KwT, and phi(k) token-major
// into Ks when given.  Tokens past the end of the segment (whose K rows load as zeros)
// weigh 0.
template <int D, bool GATED, int FM>
__device__ __forceinline__ void stage_weights(const Quad &rk, const float *lg, const int *zp, int n, int fq,
                                              int tq, float *KwT, float *Ks)
{
    f32x4 f[4];
    float w[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        f[s] = phi4<FM>(rk.x[s]);
        w[s] = write_weight<GATED>(lg, zp, n, 4 * tq + s);
        if (Ks)
            *reinterpret_cast<f32x4 *>(&Ks[(4 * tq + s) * FShape<D>::qrow + 4 * fq]) = f[s];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
        *reinterpret_cast<f32x4 *>(&KwT[(4 * fq + e) * kTRow + 4 * tq]) =
            f32x4{w[0] * f[0][e], w[1] * f[1][e], w[2] * f[2][e], w[3] * f[3][e]};
}

// V rows of one token quad, feature-major into VT
__device__ __forceinline__ void stage_values(const Quad &rv, int fq, int tq, float *VT)
{
#pragma unroll
    for (int e = 0; e < 4; ++e)
        *reinterpret_cast<f32x4 *>(&VT[(4 * fq + e) * kTRow + 4 * tq]) =
            f32x4{rv.x[0][e], rv.x[1][e], rv.x[2][e], rv.x[3][e]};
}

// The chunk's write to z of feature f: the sum of row f of KwT, by token quads in order
// (each quad summed pairwise)
__device__ __forceinline__ float chunk_dz(const float *KwT, int f)
{
    float dz = 0.f;
#pragma unroll
    for (int u = 0; u < kFC / 4; ++u) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(&KwT[f * kTRow + 4 * u]);
        dz += (v[0] + v[1]) + (v[2] + v[3]);
    }
    return dz;
}

// (4) of wave w: S[16tf + 4g + r][16w + lr] (sacc[tf][r] of lane (lr, g)) += sum over the 64
// tokens i of w_i phi(k_i)[f] v_i[c], with K step (u, r) taking tokens 16u + 4g + r
template <int D>
__device__ __forceinline__ void state_write(f32x4 (&sacc)[D / 16], const float *KwT, const float *VT, int wave,
                                            int lr, int g)
{
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const f32x4 vb = *reinterpret_cast<const f32x4 *>(&VT[(16 * wave + lr) * kTRow + 16 * u + 4 * g]);
#pragma unroll
        for (int tf = 0; tf < D / 16; ++tf) {
            const f32x4 ka = *reinterpret_cast<const f32x4 *>(&KwT[(16 * tf + lr) * kTRow + 16 * u + 4 * g]);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sacc[tf] = mfma4(ka[r], vb[r], sacc[tf]);
        }
    }
}

// ============================================================================ pass 1
template <int D>
struct alignas(16) F32SumSmem {
    alignas(16) float VT[D * kTRow];
    alignas(16) float KwT[D * kTRow];
    alignas(16) float lg[2][kFC];
    alignas(16) float gj[2][kFC];
    alignas(16) int zp[2][kFC];
};

// Segment map of every non-final segment (from a zero state): S and z, then the product of
// the segment's gates, into the next segment's slot.  Segment-major block order spreads the
// idle last-segment workgroups over the XCDs.
template <typename TI, int D, bool GATED, int FM>
__global__ __launch_bounds__(FShape<D>::threads) void summary_f32_kernel(FArgs<TI, D> a)
{
    using Sh = FShape<D>;
    __shared__ F32SumSmem<D> sm;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lr = lane & 15, g = lane >> 4;
    const int fq = tid % Sh::quads, tq = tid / Sh::quads;

    const int64_t n_heads = gridDim.x / a.nseg;
    const int64_t head = blockIdx.x % n_heads;
    const int seg = (int)(blockIdx.x / n_heads);
    if (seg == a.nseg - 1)
        return;  // the last segment's map is never needed
    const int64_t s0 = (int64_t)seg * a.seg_len;
    const int64_t len = a.seg_len;
    const int n_chunks = (int)((len + kFC - 1) / kFC);
    auto chunk_len = [&](int c) { return (int)min((int64_t)kFC, len - (int64_t)c * kFC); };
    const int64_t row0 = head * a.T + s0;
    const int64_t seg_bytes = len * D * (int64_t)sizeof(TI);
    const rsrc_t rK = make_rsrc(a.K + row0 * D, seg_bytes);
    const rsrc_t rV = make_rsrc(a.V + row0 * D, seg_bytes);
    const rsrc_t rA = make_rsrc(GATED ? a.alpha + row0 : a.S, GATED ? len * 4 : 0);

    f32x4 sacc[Sh::tiles];
#pragma unroll
    for (int tf = 0; tf < Sh::tiles; ++tf)
        sacc[tf] = f32x4{0.f, 0.f, 0.f, 0.f};
    float zreg = 0.f, g_seg = 1.f;
    Quad rk, rv;
    float ar = 0.f;
    load_quad<TI, D>(rK, 0, fq, tq, rk);
    load_quad<TI, D>(rV, 0, fq, tq, rv);
    if (GATED && wave == 0)
        ar = __uint_as_float((unsigned)__builtin_amdgcn_raw_buffer_load_b32(rA, lane * 4, 0, 0));

    for (int c = 0; c < n_chunks; ++c) {
        const int gs = c & 1;
        const int n = chunk_len(c);
        if (GATED && wave == 0)
            scan_gates(ar, n, lane, sm.lg[gs], sm.zp[gs], sm.gj[gs]);
        wg_barrier();  // gates visible; the previous chunk's products are done with the tiles
        stage_weights<D, GATED, FM>(rk, sm.lg[gs], sm.zp[gs], n, fq, tq, sm.KwT, nullptr);
        stage_values(rv, fq, tq, sm.VT);
        load_quad<TI, D>(rK, c + 1, fq, tq, rk);  // past the end of the segment these read zeros
        load_quad<TI, D>(rV, c + 1, fq, tq, rv);
        if (GATED && wave == 0)
            ar = __uint_as_float(
                (unsigned)__builtin_amdgcn_raw_buffer_load_b32(rA, ((c + 1) * kFC + lane) * 4, 0, 0));
        wg_barrier();  // chunk staged
        const float g_end = GATED ? sm.gj[gs][n - 1] : 1.f;
        if (GATED) {
            g_seg *= g_end;
#pragma unroll
            for (int tf = 0; tf < Sh::tiles; ++tf)
                sacc[tf] *= g_end;
        }
        state_write<D>(sacc, sm.KwT, sm.VT, wave, lr, g);
        if (tid < D)
            zreg = g_end * zreg + chunk_dz(sm.KwT, tid);
    }

    float *Sout = slot_ptr(a, head, seg + 1);
    if (tid == 0)
        Sout[D * D + D] = g_seg;
#pragma unroll
    for (int tf = 0; tf < Sh::tiles; ++tf)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            Sout[(16 * tf + 4 * g + r) * D + 16 * wave + lr] = sacc[tf][r];
    if (tid < D)
        Sout[D * D + tid] = zreg;
}

// ============================================================================ pass 3
// The gates need one buffer: they are rewritten (by wave 0, at the top of the next chunk)
// only after every wave has passed the barrier between the products, and what the second
// half of the products needs of them is read into registers before it.
template <int D>
struct alignas(16) F32Smem {
    alignas(16) float Qs[kFC * FShape<D>::qrow];  // phi(q), token-major
    alignas(16) float Ks[kFC * FShape<D>::qrow];  // phi(k), token-major
    alignas(16) float VT[D * kTRow];              // v, feature-major
    alignas(16) float KwT[D * kTRow];             // w phi(k), feature-major; 0 past the end of the segment
    alignas(16) f32x4 P[kFTiles * 64];            // masked, gate-weighted scores, accumulator layout
    alignas(16) float rs[kFTiles * 16];           // rs[16k + lr]: score tile k's sum over its 16 tokens i
    alignas(16) float zs[D];                      // z entering the chunk
    alignas(16) float dq[kFC];                    // phi(q_j) . z_prev
    alignas(16) float lg[kFC];
    alignas(16) float gj[kFC];
    alignas(16) int zp[kFC];
};
static_assert(sizeof(F32Smem<128>) <= 160 * 1024, "the fp32 tiles must fit in the 160 KB of LDS");
static_assert(sizeof(F32Smem<64>) <= 80 * 1024, "two workgroups of the d = 64 tiles must share the LDS");

template <typename TI, int D, bool GATED, int FM>
__global__ __launch_bounds__(FShape<D>::threads) void prefill_f32_kernel(FArgs<TI, D> a)
{
    using Sh = FShape<D>;
    constexpr int QR = Sh::qrow;
    __shared__ F32Smem<D> sm;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lr = lane & 15, g = lane >> 4;
    const int fq = tid % Sh::quads, tq = tid / Sh::quads;

    const int64_t head = blockIdx.x / a.nseg;
    const int seg = blockIdx.x % a.nseg;
    const int64_t s0 = (int64_t)seg * a.seg_len;
    const int64_t s1 = seg == a.nseg - 1 ? a.T : s0 + a.seg_len;
    const int64_t len = s1 - s0;
    const int n_chunks = (int)((len + kFC - 1) / kFC);
    auto chunk_len = [&](int c) { return (int)min((int64_t)kFC, len - (int64_t)c * kFC); };
    const int64_t row0 = head * a.T + s0;
    const int64_t seg_bytes = len * D * (int64_t)sizeof(TI);
    const rsrc_t rQ = make_rsrc(a.Q + row0 * D, seg_bytes);
    const rsrc_t rK = make_rsrc(a.K + row0 * D, seg_bytes);
    const rsrc_t rV = make_rsrc(a.V + row0 * D, seg_bytes);
    const rsrc_t rA = make_rsrc(GATED ? a.alpha + row0 : a.S, GATED ? len * 4 : 0);
    const rsrc_t rY = make_rsrc(a.Y + row0 * D, seg_bytes);

    // wave w owns columns 16w + lr of S: sacc[tf][r] = S[16tf + 4g + r][16w + lr]
    f32x4 sacc[Sh::tiles];
    float zreg = 0.f;  // threads tid < D: z of feature tid
    {
        const float *Sin = a.nseg == 1 ? a.S + head * D * D : slot_ptr(a, head, seg);
        const float *zin = a.nseg == 1 ? a.z + head * D : Sin + D * D;
#pragma unroll
        for (int tf = 0; tf < Sh::tiles; ++tf)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sacc[tf][r] = Sin[(16 * tf + 4 * g + r) * D + 16 * wave + lr];
        if (tid < D) {
            zreg = zin[tid];
            sm.zs[tid] = zreg;
        }
    }
    Quad rq, rk, rv;
    float ar = 0.f;
    load_quad<TI, D>(rQ, 0, fq, tq, rq);
    load_quad<TI, D>(rK, 0, fq, tq, rk);
    load_quad<TI, D>(rV, 0, fq, tq, rv);
    if (GATED && wave == 0)
        ar = __uint_as_float((unsigned)__builtin_amdgcn_raw_buffer_load_b32(rA, lane * 4, 0, 0));

    for (int c = 0; c < n_chunks; ++c) {
        const int n = chunk_len(c);
        if (GATED && wave == 0)
            scan_gates(ar, n, lane, sm.lg, sm.zp, sm.gj);
        wg_barrier();  // gates visible; the previous chunk's products are done with the tiles
        // ---- staging: phi(q) and phi(k) token-major, the write weights and V feature-major
#pragma unroll
        for (int s = 0; s < 4; ++s)
            *reinterpret_cast<f32x4 *>(&sm.Qs[(4 * tq + s) * QR + 4 * fq]) = phi4<FM>(rq.x[s]);
        stage_weights<D, GATED, FM>(rk, sm.lg, sm.zp, n, fq, tq, sm.KwT, sm.Ks);
        stage_values(rv, fq, tq, sm.VT);
        load_quad<TI, D>(rQ, c + 1, fq, tq, rq);  // past the end of the segment these read zeros
        load_quad<TI, D>(rK, c + 1, fq, tq, rk);
        load_quad<TI, D>(rV, c + 1, fq, tq, rv);
        if (GATED && wave == 0)
            ar = __uint_as_float(
                (unsigned)__builtin_amdgcn_raw_buffer_load_b32(rA, ((c + 1) * kFC + lane) * 4, 0, 0));
        wg_barrier();  // chunk staged

        // ---- part a: (2) for the four token tiles; phi(q) . z_prev (waves 0-3, token tile
        //      `wave`); the score tiles k = wave (mod waves) with their row sums
        float gjr[4], g_end = 1.f;  // gate products the part b below needs
        if (GATED) {
#pragma unroll
            for (int tj = 0; tj < 4; ++tj)
                gjr[tj] = sm.gj[16 * tj + lr];
            g_end = sm.gj[n - 1];
        }
        f32x4 acc[4];
#pragma unroll
        for (int tj = 0; tj < 4; ++tj)
            acc[tj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int tf = 0; tf < Sh::tiles; ++tf) {
#pragma unroll
            for (int tj = 0; tj < 4; ++tj) {
                const f32x4 qv = *reinterpret_cast<const f32x4 *>(&sm.Qs[(16 * tj + lr) * QR + 16 * tf + 4 * g]);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[tj] = mfma4(sacc[tf][r], qv[r], acc[tj]);
            }
        }
        if (wave < 4) {
            f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int tf = 0; tf < Sh::tiles; ++tf) {
                const f32x4 zv = *reinterpret_cast<const f32x4 *>(&sm.zs[16 * tf + 4 * g]);
                const f32x4 qv = *reinterpret_cast<const f32x4 *>(&sm.Qs[(16 * wave + lr) * QR + 16 * tf + 4 * g]);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    d = mfma4(zv[r], qv[r], d);
            }
            if (g == 0)
                sm.dq[16 * wave + lr] = d[0];
        }
        for (int k = wave; k < kFTiles; k += Sh::tiles) {
            const int tj = k >= 6 ? 3 : k >= 3 ? 2 : k >= 1 ? 1 : 0;
            const int ti = k - tj * (tj + 1) / 2;
            // sc[r] = score (i = 16ti + 4g + r, j = 16tj + lr)
            const int j = 16 * tj + lr;
            f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < Sh::tiles; ++t) {
                const f32x4 ka = *reinterpret_cast<const f32x4 *>(&sm.Ks[(16 * ti + lr) * QR + 16 * t + 4 * g]);
                const f32x4 qb = *reinterpret_cast<const f32x4 *>(&sm.Qs[j * QR + 16 * t + 4 * g]);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sc = mfma4(ka[r], qb[r], sc);
            }
            int ii[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                ii[r] = 16 * ti + 4 * g + r;
            float dec[4];
            pair_decays<GATED>(sm.lg, sm.zp, j, ii, dec);
            f32x4 p;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                p[r] = ii[r] <= j ? sc[r] * dec[r] : 0.f;
            sm.P[k * 64 + lane] = p;
            // row sum over the tile's 16 tokens i, in a fixed order: own 4, then across g
            float rsum = (p[0] + p[1]) + (p[2] + p[3]);
            rsum += __shfl_xor(rsum, 16, 64);
            rsum += __shfl_xor(rsum, 32, 64);
            if (g == 0)
                sm.rs[16 * k + lr] = rsum;
        }
        wg_barrier();  // a | b

        // ---- part b: (3) and the outputs of the four token tiles, then (4)
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) {
            const int j = 16 * tj + lr;
            float den = sm.dq[j];
            if (GATED) {
                acc[tj] *= gjr[tj];
                den *= gjr[tj];
            }
#pragma unroll
            for (int ti = 0; ti <= tj; ++ti) {
                const int k = tj * (tj + 1) / 2 + ti;
                den += sm.rs[16 * k + lr];
                const f32x4 pv = sm.P[k * 64 + lane];
                const f32x4 va = *reinterpret_cast<const f32x4 *>(&sm.VT[(16 * wave + lr) * kTRow + 16 * ti + 4 * g]);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[tj] = mfma4(va[r], pv[r], acc[tj]);
            }
            const float inv = 1.f / (den + a.eps);
            const f32x4 y = acc[tj] * inv;
            // columns 16w + 4g .. + 3 of token j; rows past the end fall outside rY
            const int e = (c * kFC + j) * D + 16 * wave + 4 * g;
            if constexpr (std::is_same_v<TI, float>) {
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, y),
                                                       rY, e * 4, 0, 0);
            } else {
                const bf16x4 yb = {static_cast<bf16>(y[0]), static_cast<bf16>(y[1]), static_cast<bf16>(y[2]),
                                   static_cast<bf16>(y[3])};
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, yb),
                                                      rY, e * 2, 0, 0);
            }
        }
        if (GATED) {
#pragma unroll
            for (int tf = 0; tf < Sh::tiles; ++tf)
                sacc[tf] *= g_end;
        }
        state_write<D>(sacc, sm.KwT, sm.VT, wave, lr, g);
        if (tid < D) {
            zreg = g_end * zreg + chunk_dz(sm.KwT, tid);
            sm.zs[tid] = zreg;  // read again only after the next chunk's two barriers
        }
    }

    if (seg != a.nseg - 1)
        return;
    float *Sout = a.S + head * D * D;
#pragma unroll
    for (int tf = 0; tf < Sh::tiles; ++tf)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            Sout[(16 * tf + 4 * g + r) * D + 16 * wave + lr] = sacc[tf][r];
    if (tid < D)
        a.z[head * D + tid] = zreg;
}

template <typename TI, int D, bool GATED, int FM>
hipError_t launch_f32(const FArgs<TI, D> &a, int64_t n_heads, hipStream_t stream)
{
    constexpr int NT = FShape<D>::threads;
    const unsigned blocks = (unsigned)(n_heads * a.nseg);
    if (a.nseg > 1) {
        summary_f32_kernel<TI, D, GATED, FM><<<dim3(blocks), dim3(NT), 0, stream>>>(a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        segment_scan_kernel<FArgs<TI, D>, D>
            <<<dim3((D * D + D + 255) / 256, (unsigned)n_heads), dim3(256), 0, stream>>>(a);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    prefill_f32_kernel<TI, D, GATED, FM><<<dim3(blocks), dim3(NT), 0, stream>>>(a);
    return hipGetLastError();
}

template <typename TI, int D>
hipError_t launch_typed(const PrefillArgs &pa, hipStream_t stream)
{
    FArgs<TI, D> a;
    a.Q = static_cast<const TI *>(pa.Q);
    a.K = static_cast<const TI *>(pa.K);
    a.V = static_cast<const TI *>(pa.V);
    a.alpha = static_cast<const float *>(pa.alpha);
    a.Y = static_cast<TI *>(pa.Y);
    a.S = static_cast<float *>(pa.S);
    a.z = static_cast<float *>(pa.z);
    a.T = pa.T;
    a.eps = (float)pa.eps;
    int64_t nseg, seg_len;
    if (!plan_segments(pa.n_heads, pa.T, kFC, D * (int64_t)sizeof(TI), segment_slot_bytes(D), &nseg, &seg_len))
        return hipErrorInvalidValue;
    a.nseg = (int)nseg;
    a.seg_len = seg_len;
    return dispatch_feature_map(pa.phi, [&](auto fm) {
        constexpr int FM = decltype(fm)::value;
        return pa.alpha ? launch_f32<TI, D, true, FM>(a, pa.n_heads, stream)
                        : launch_f32<TI, D, false, FM>(a, pa.n_heads, stream);
    });
}

bool aligned(const void *p, uintptr_t bytes) { return (reinterpret_cast<uintptr_t>(p) & (bytes - 1)) == 0; }

}  // namespace

bool mfma_f32_prefill_supported(la_dtype io_dtype, int32_t d, int32_t dv, int32_t chunk)
{
    if (chunk != kFC || d != dv)
        return false;
    return (io_dtype == LA_F32 && (d == 64 || d == 128)) || (io_dtype == LA_BF16 && d == 64);
}

hipError_t launch_prefill_mfma_f32(const PrefillArgs &pa, la_dtype io_dtype, hipStream_t stream)
{
    // rows are read and written 4 elements at a time: 16 bytes for fp32, 8 for bf16
    const uintptr_t al = io_dtype == LA_F32 ? 16 : 8;
    if (!aligned(pa.Q, al) || !aligned(pa.K, al) || !aligned(pa.V, al) || !aligned(pa.Y, al))
        return launch_prefill_general(pa, io_dtype, stream);
    if (io_dtype == LA_BF16)
        return launch_typed<bf16, 64>(pa, stream);
    return pa.d == 64 ? launch_typed<float, 64>(pa, stream) : launch_typed<float, 128>(pa, stream);
}

}  // namespace la
