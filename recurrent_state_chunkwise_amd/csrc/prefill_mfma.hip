// bf16 MFMA chunked prefill for d = dv = 128, chunk 64 or 128, fp32 state.
//
// Computes, per chunk c with carried state S_prev, z_prev, the chunk equations of the
// page "Linear attention：把历史写进状态" (hs-black.github.io), section "一个 chunk 的
// 输出由两部分组成":
//   numerator   = Q~c S_prev + [(Q~c K~c^T) . M] Vc
//   denominator = Q~c z_prev + rowsum[(Q~c K~c^T) . M]
//   S_next = S_prev + K~c^T Vc,   z_next = z_prev + sum of the rows of K~c
// and y = numerator / (denominator + eps).  The gate of section "加一个门" enters through
// gate products, which the page names without a formula: with L_j the sum of log(alpha)
// over the chunk up to token j, score (j, i) is weighted by exp(L_j - L_i), the read of
// S_prev and z_prev by exp(L_j), the write of token i by exp(L_last - L_i) and the
// carried state by exp(L_last); a zero gate inside (i, j] makes the weight exactly 0.
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
// Inside a workgroup (8 consumer waves for all 128 value columns, and producer waves that
// stage the tiles) every product is v_mfma_f32_16x16x32_bf16 with fp32 accumulation:
//   (1) scores K~ Q~^T, 16x16 tiles on or below the diagonal spread over the waves; the
//       fp32 tile is masked, gate-weighted and kept in LDS as bf16 in accumulator layout;
//   (2) N^T  = S_prev^T Q~^T  and  D = z_prev^T Q~^T (z_prev as bf16 high and low parts),
//       both scaled by exp(L_j);
//   (3) N^T += V^T P^T        and  D += 1^T P^T (the row sums of the masked scores);
//   (4) S = g_last S + (w K~)^T V.
// Wave w owns value columns 16w..16w+15 of N and of S, so S never leaves registers.  z is
// kept by the producers: the fp32 sum of the write weights w phi(k) they form, before the
// rounding to bf16 that S's operand takes.  The outputs are computed transposed so that a
// lane holds four adjacent columns of one token together with that token's denominator.
#include "device_common.hpp"
#include "internal.hpp"
#include "prefill_common.hpp"

namespace la {
namespace {

// (sequence, segment) workgroups aimed for: one per compute unit (twice as many, two
// rounds of workgroups, and half as many, twice the chunks per workgroup, both measured
// slower)
constexpr int64_t kSegmentTarget = 256;

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

// slot p of a sequence: S [128][128], z [128] and the segment's gate product (padded), in
// the first rows of segment p of Y
__device__ __forceinline__ float *slot_ptr(const Args &a, int64_t head, int p)
{
    return reinterpret_cast<float *>(a.Y + (head * a.T + (int64_t)p * a.seg_len) * kD);
}

// ============================================================================ pass 3, chunk 64
// Producer / consumer form of the full pass at chunk 64: 12 waves, of which waves 0-7
// (consumers) hold S and do every product, while waves 8-11 (producers) turn the raw Q,
// K, V and alpha of the next chunk into staged tiles in the other half of a
// double-buffered LDS and keep z.  Two workgroup barriers per chunk i:
//   part a   consumers: scores of chunk i; N^T = S_prev^T Q~^T; waves 4-7 D = z_prev^T Q~^T
//            producers: z entering chunk i+1; y of chunk i-1 to HBM; gate scan (and write
//            weights) of chunk i+1; phi(q) and V of chunk i+1
//   part b   consumers: gates, V^T P^T and 1^T P^T, y into LDS, state update
//            producers: phi(k), the write weights and their fp32 sums for z, of chunk i+1
// Each raw load is issued two chunks ahead of its use, except K in the gated form, which
// has one register set and is loaded one chunk ahead: the gated producers also hold the
// fp32 sums of the z update, and a second K set would not fit in their registers.  The two
// roles run their own loops with the same number of barriers, which keeps their registers
// apart.
//
// Every staged tile is token-major (one row of 128 bf16 per token, rows padded to
// 272 bytes), written with 16-byte row stores.  Operands that contract over tokens (V^T
// for (3), the write weights and V for (4)) are read with the gfx950 transposing LDS
// load: within each 16-lane group, lane 4e + q supplies the address of 4 adjacent
// columns of token row t(e) and lane i receives column i of rows t(0..3).  With the
// padded rows every row store, row read and transposing read of a wave hits distinct
// banks as long as each transposing load takes only even or only odd token rows per
// 32 lanes; the scores therefore feed K~ rows to the MFMA in the order sigma (even
// tokens first), which makes the score tiles, and so V^T in (3), come in that order.
// The two score tiles that one K step of (3) needs sit side by side, so that step reads
// them with one 16-byte load per lane.  Paired 8-byte LDS loads (which the compiler forms
// from loads a known distance apart) run at half the rate of two single loads on gfx950,
// so the two 8-byte halves of a (2) operand are kept from being fused.
constexpr int kPcC = 64;
constexpr int kPcConsumers = 512;
// Producer waves: 4 in the output pass (8 measured slower), 8 in the segment-map pass,
// whose consumers only fold and whose registers fit 16 waves; the segment-map producers
// keep 2 chunks of K and V in flight per thread (4 measured no faster).
constexpr int kPcProducers = 4;
constexpr int kPcThreads = kPcConsumers + 64 * kPcProducers;
constexpr int kSumProducers = 8;
constexpr int kSumThreads = kPcConsumers + 64 * kSumProducers;
constexpr int kSumSets = 2;

constexpr int kRow = kD + 8;  // padded token row, in elements
__device__ __forceinline__ int pr_off(int row, int col) { return row * kRow + col; }
// token order of the K~ rows in the score tiles: even tokens of the 16-token tile first
__device__ __forceinline__ int sigma(int m) { return 2 * (m & 7) + (m >> 3); }
// y tile: 16-byte granule g of row j sits at granule g ^ (j & 15)
__device__ __forceinline__ int ys_off(int row, int col)
{
    return row * kD + ((((col >> 3) ^ (row & 15)) << 3) | (col & 7));
}
// 4 bf16 of one lane from the transposing LDS load
__device__ __forceinline__ bf16x4 ld_tr(const bf16 *p)
{
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
    return __builtin_bit_cast(bf16x4, v);
}
// x, hidden from the optimiser (which then cannot fuse loads addressed from it with others)
__device__ __forceinline__ int opaque(int x)
{
    asm volatile("" : "+v"(x));
    return x;
}
__device__ __forceinline__ bf16x8 cat8(bf16x4 lo, bf16x4 hi)
{
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// z in bf16 high and low parts: hi = bf16(z), lo = bf16(z - hi), so that hi + lo carries
// about 16 bits of z
__device__ __forceinline__ void split_store(float z, bf16 *hi, bf16 *lo)
{
    const bf16 h = static_cast<bf16>(z);
    *hi = h;
    *lo = static_cast<bf16>(z - static_cast<float>(h));
}
// A-operands of the denominator product phi(q) . z from the high and low parts zhl[0],
// zhl[1]: features f0 .. f0 + 3 and f0 + 16 .. f0 + 19 (the k order of the Q~ operand)
__device__ __forceinline__ void z_operand(const bf16 (&zhl)[2][kD], int f0, bf16x8 &zh, bf16x8 &zl)
{
    zh = cat8(*reinterpret_cast<const bf16x4 *>(&zhl[0][f0]), *reinterpret_cast<const bf16x4 *>(&zhl[0][f0 + 16]));
    zl = cat8(*reinterpret_cast<const bf16x4 *>(&zhl[1][f0]), *reinterpret_cast<const bf16x4 *>(&zhl[1][f0 + 16]));
}

// score tile (tj, ti) lives in half ti & 1 of pair slot kPairBase[tj] + ti / 2
constexpr int kPairBase[4] = {0, 1, 2, 4};
constexpr int kPairSlots = 6;

template <bool GATED>
struct alignas(16) PcSmem {
    alignas(16) bf16 Qs[2][kPcC * kRow];           // phi(q)
    alignas(16) bf16 Ks[2][kPcC * kRow];           // phi(k); ungated, also the write weights
    alignas(16) bf16 Vs[2][kPcC * kRow];           // v
    alignas(16) bf16 Kw[GATED ? 2 : 1][GATED ? kPcC * kRow : 8];  // w phi(k) (gated)
    // y of the last finished chunk, 16-byte granules XOR-swizzled by row.  Gated, it lives
    // in that chunk's phi(k) buffer, dead from the scores until the producers stage the
    // chunk after next into it (after the y of this chunk has gone out).
    alignas(16) bf16 Ys[GATED ? 8 : kPcC * kD];
    alignas(16) uint4 P[kPairSlots * 64];          // bf16 score tiles in pairs, 4 values of each per lane
    alignas(16) float zs[2][kD];                   // z entering the chunk, by chunk parity
    alignas(16) bf16 zhl[2][2][kD];                // the same as bf16 high and low parts
    alignas(16) float zred[16][kD];                // fp32 z update of the staged chunk, per token group
    alignas(16) float dq[kPcC];                    // phi(q_j) . z_prev
    alignas(16) float lg[2][kPcC];
    alignas(16) float gj[2][kPcC];
    alignas(16) int zp[2][kPcC];
    alignas(16) float wt[GATED ? 2 : 1][GATED ? kPcC : 4];  // write weights of the staged chunk (gated)
};

template <bool GATED, int FM>
__global__ __launch_bounds__(kPcThreads) void prefill_pc_kernel(Args a)
{
    constexpr int C = kPcC;
    typedef Cfg<C> G;
    __shared__ PcSmem<GATED> sm;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lr = lane & 15;
    const int lg4 = lane >> 4;

    const int64_t head = blockIdx.x / a.nseg;
    const int seg = blockIdx.x % a.nseg;
    const int64_t s0 = (int64_t)seg * a.seg_len;
    const int64_t s1 = seg == a.nseg - 1 ? a.T : s0 + a.seg_len;
    const int64_t len = s1 - s0;
    const int n_chunks = (int)((len + C - 1) / C);
    const int n_steps = (n_chunks + 1) & ~1;  // both roles walk an even number of chunk steps
    auto chunk_len = [&](int c) { return (int)min((int64_t)C, len - (int64_t)c * C); };
    const int64_t row0 = head * a.T + s0;

    if (wave >= 8) {
        // ============================================================ producers
        const rsrc_t rQ = make_rsrc(a.Q + row0 * kD, len * kD * 2);
        const rsrc_t rK = make_rsrc(a.K + row0 * kD, len * kD * 2);
        const rsrc_t rV = make_rsrc(a.V + row0 * kD, len * kD * 2);
        const rsrc_t rA = make_rsrc(GATED ? a.alpha + row0 : a.S, GATED ? len * 4 : 0);
        const rsrc_t rY = make_rsrc(a.Y + row0 * kD, len * kD * 2);
        const int pt = tid - kPcConsumers;
        // the gate scan runs on a wave that does not also finish z (waves 8 and 9 do), so
        // that neither job lengthens the other's wave
        const bool scanner = wave == 10;
        // thread (fg, tg) stages granule fg (8 features) of tokens TPT tg .. TPT tg + TPT - 1
        constexpr int TPT = 16 / kPcProducers;
        const int fg = pt & 15, tg = pt >> 4;
        const int ld_off = tg * TPT * kD * 2 + fg * 16;
        // two register sets: chunk c is loaded into set c & 1 two chunks before it is staged
        uint4 rq0[TPT], rk0[TPT], rv0[TPT], rq1[TPT], rk1[TPT], rv1[TPT];
        float ar0 = 0.f, ar1 = 0.f;
        // z of feature pt (threads pt < 128): z = g_end z + sum of w phi(k) over each chunk,
        // from the fp32 write weights before their rounding to bf16.  The running value
        // stays in sm.zs (only this same thread writes and reads it), so it takes no register
        // across the loop; the consumers read its bf16 high and low parts in sm.zhl.
        auto z_update = [&](int c) {  // chunk c staged: z entering chunk c + 1, for part a
            if (pt < kD) {
                float dz = 0.f;
#pragma unroll
                for (int t = 0; t < 16; ++t)
                    dz += sm.zred[t][pt];
                const float g = GATED ? sm.gj[c & 1][chunk_len(c) - 1] : 1.f;
                const float zn = g * sm.zs[c & 1][pt] + dz;
                sm.zs[(c + 1) & 1][pt] = zn;
                split_store(zn, &sm.zhl[(c + 1) & 1][0][pt], &sm.zhl[(c + 1) & 1][1][pt]);
            }
        };

        auto load_qv = [&](int c, uint4 (&rq)[TPT], uint4 (&rv)[TPT]) {
#pragma unroll
            for (int p = 0; p < TPT; ++p) {
                rq[p] = bload16<kNT>(rQ, c * C * kD * 2 + ld_off + p * kD * 2);
                rv[p] = bload16<kNT>(rV, c * C * kD * 2 + ld_off + p * kD * 2);
            }
        };
        auto load_k = [&](int c, uint4 (&rk)[TPT]) {
#pragma unroll
            for (int p = 0; p < TPT; ++p)
                rk[p] = bload16<kNT>(rK, c * C * kD * 2 + ld_off + p * kD * 2);
        };
        auto load_a = [&](int c, float &ar) {  // every producer wave loads; the scanner uses it
            if (GATED)
                ar = __uint_as_float((unsigned)__builtin_amdgcn_raw_buffer_load_b32(rA, (c * C + lane) * 4, 0, kNT));
        };
        // inclusive scans of log(alpha) and of the last zero-gate position, and the write
        // weights they give (one wave)
        auto scan = [&](int n, int gs, float ar) {
            if (GATED && scanner) {
                const float av = lane < n ? ar : 1.f;
                float s = av > 0.f ? __logf(av) : 0.f;
                int zf = av == 0.f ? lane : -1;
                s = wave_scan_add(s);
                zf = wave_scan_max(zf);
                sm.lg[gs][lane] = s;
                sm.zp[gs][lane] = zf;
                sm.gj[gs][lane] = zf >= 0 ? 0.f : __expf(s);
                sm.wt[gs][lane] = lane_write_weight(s, zf, n, lane);
            }
        };
        // phi(q) rows and V rows
        auto stage_qv = [&](int buf, const uint4 (&rq)[TPT], const uint4 (&rv)[TPT]) {
#pragma unroll
            for (int p = 0; p < TPT; ++p) {
                const int j = tg * TPT + p;
                float x[8];
                unpack8(rq[p], x);
                bf16x8 qb;
#pragma unroll
                for (int s = 0; s < 8; ++s)
                    qb[s] = static_cast<bf16>(phi<FM>(x[s]));
                *reinterpret_cast<bf16x8 *>(&sm.Qs[buf][pr_off(j, fg * 8)]) = qb;
                *reinterpret_cast<uint4 *>(&sm.Vs[buf][pr_off(j, fg * 8)]) = rv[p];
            }
        };
        // phi(k) rows and the write weights w_j phi(k_j); w_j = gates after j to the
        // chunk end, 0 past the end of the segment (whose tokens load as zeros).  The
        // ungated weights are phi(k) itself, so those rows of Ks are zeroed instead (the
        // scores never use them: they lie above the diagonal of every kept row).
        auto stage_k = [&](int buf, int gs, int n, const uint4 (&rk)[TPT]) {
            float zp8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < TPT; ++p) {
                const int j = tg * TPT + p;
                float x[8];
                unpack8(rk[p], x);
                bf16x8 kb, kwb;
                const float w = GATED ? sm.wt[gs][j] : write_weight<false>(nullptr, nullptr, n, j);
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const float f = phi<FM>(x[s]);
                    kb[s] = static_cast<bf16>(f);
                    if (GATED)
                        kwb[s] = static_cast<bf16>(w * f);
                    zp8[s] += GATED ? w * f : (j < n ? f : 0.f);
                }
                uint4 u = *reinterpret_cast<uint4 *>(&kb);
                if (!GATED && j >= n)
                    u = make_uint4(0u, 0u, 0u, 0u);
                *reinterpret_cast<uint4 *>(&sm.Ks[buf][pr_off(j, fg * 8)]) = u;
                if (GATED)
                    *reinterpret_cast<bf16x8 *>(&sm.Kw[buf][pr_off(j, fg * 8)]) = kwb;
            }
            *reinterpret_cast<f32x4 *>(&sm.zred[tg][fg * 8]) = f32x4{zp8[0], zp8[1], zp8[2], zp8[3]};
            *reinterpret_cast<f32x4 *>(&sm.zred[tg][fg * 8 + 4]) = f32x4{zp8[4], zp8[5], zp8[6], zp8[7]};
        };
        // y of chunk c from the LDS tile to HBM as whole 256-byte rows: producer wave pw
        // takes rows 4 TPT pw .. 4 TPT pw + 4 TPT - 1, four rows per store; rows past the end
        // of the segment fall outside rY and are dropped
        const int pw = wave - 8;
        auto flush_y = [&](int c) {
#pragma unroll
            for (int u = 0; u < TPT; ++u) {
                const int row = pw * 4 * TPT + u * 4 + (lane >> 4), g = lane & 15;
                const bf16 *ys = GATED ? sm.Ks[c & 1] : sm.Ys;
                const uint4 v = *reinterpret_cast<const uint4 *>(&ys[row * kD + g * 8]);
                const int off = ((c * C + row) * kD + ((g ^ (row & 15)) << 3)) * 2;
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, v), rY, off, 0, kNT);
            }
        };
        // one chunk interval: write out y of chunk i - 1, stage chunk cn = i + 1 from its
        // register set, then refill that set with chunk cn + 2
        // Loads and stores past the end of the segment read zeros or are dropped by the
        // buffer resources; they are issued unconditionally so that every wait on them is
        // a counted one.  Step 0 flushes to chunk n_chunks, which is such a store.
        auto step = [&](int i, uint4 (&rq)[TPT], uint4 (&rk)[TPT], uint4 (&rv)[TPT], float &ar) {
            const int cn = i + 1;
            const bool work = cn < n_chunks;
            if (i < n_chunks)
                z_update(i);
            flush_y(i > 0 ? i - 1 : n_chunks);
            if (work)
                scan(chunk_len(cn), cn & 1, ar);
            load_a(cn + 2, ar);
            if (work)
                stage_qv(cn & 1, rq, rv);
            load_qv(cn + 2, rq, rv);
            wg_barrier();  // a | b
            if (work)
                stage_k(cn & 1, cn & 1, chunk_len(cn), GATED ? rk0 : rk);
            if (GATED)
                load_k(cn + 1, rk0);
            else
                load_k(cn + 2, rk);
            wg_barrier();  // chunk i done
        };

        // prologue: chunk 0 staged whole, chunks 1 and 2 in flight
        load_qv(0, rq0, rv0);
        load_k(0, rk0);
        load_a(0, ar0);
        load_qv(1, rq1, rv1);
        if (!GATED)
            load_k(1, rk1);
        load_a(1, ar1);
        scan(chunk_len(0), 0, ar0);
        load_a(2, ar0);
        wg_barrier();
        stage_qv(0, rq0, rv0);
        load_qv(2, rq0, rv0);
        stage_k(0, 0, chunk_len(0), rk0);
        load_k(GATED ? 1 : 2, rk0);
        wg_barrier();

        for (int i = 0; i < n_steps; i += 2) {
            step(i, rq1, rk1, rv1, ar1);      // stages chunk i + 1 (odd)
            step(i + 1, rq0, rk0, rv0, ar0);  // stages chunk i + 2 (even)
        }
        // the last chunk's y, complete since the last barrier (already written by the
        // trailing empty step when the chunk count is odd)
        flush_y(n_steps == n_chunks ? n_chunks - 1 : n_chunks);
        if (seg == a.nseg - 1 && pt < kD)
            a.z[head * kD + pt] = sm.zs[n_chunks & 1][pt];
        return;
    }

    // ================================================================ consumers
    bf16x8 ones;
#pragma unroll
    for (int s = 0; s < 8; ++s)
        ones[s] = static_cast<bf16>(1.f);
    // wave w owns value columns c = 16w + lr of S (tile tf holds rows f = 16tf + 4lg4 + r);
    // z lives with the producers, which pass each chunk's entering z through sm.zhl
    f32x4 sacc[8];
    const int cw = wave * 16 + lr;
    const int fw = wave * 16 + lg4 * 4;
    {
        const float *Sin = a.nseg == 1 ? a.S + head * kD * kD : slot_ptr(a, head, seg);
        const float *zin = a.nseg == 1 ? a.z + head * kD : Sin + kD * kD;
#pragma unroll
        for (int tf = 0; tf < 8; ++tf)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sacc[tf][r] = Sin[(tf * 16 + lg4 * 4 + r) * kD + cw];
        if (tid < kD) {
            sm.zs[0][tid] = zin[tid];
            split_store(zin[tid], &sm.zhl[0][0][tid], &sm.zhl[0][1][tid]);
        }
    }
    // transposing-load addresses: this lane supplies 4 adjacent columns (4 (lr & 3) ..)
    // of token row e = lr >> 2 of its group's set
    const int te = lr >> 2, tc = 4 * (lr & 3);
    // the second halves of the pair slots of tiles (0, 0) and (2, 2) hold no tile: zero,
    // they stand for the tiles above the diagonal in the K steps of (3)
    if (wave == 0) {
        reinterpret_cast<uint2 *>(&sm.P[kPairBase[0] * 64 + lane])[1] = make_uint2(0u, 0u);
        reinterpret_cast<uint2 *>(&sm.P[(kPairBase[2] + 1) * 64 + lane])[1] = make_uint2(0u, 0u);
    }
    wg_barrier();
    wg_barrier();

    for (int i = 0; i < n_chunks; ++i) {
        const int buf = i & 1;
        const int n = chunk_len(i);
        const bf16 *Qb = sm.Qs[buf];
        const bf16 *Kb = sm.Ks[buf];
        const bf16 *Vb = sm.Vs[buf];
        const bf16 *Wb = GATED ? sm.Kw[buf] : sm.Ks[buf];

        // ---- part a: scores (1), then (2) for all four token tiles
        for (int k = wave; k < G::NPT; k += 8) {
            int tj = 0;
            while ((tj + 1) * (tj + 2) / 2 <= k)
                ++tj;
            const int ti = k - tj * (tj + 1) / 2;
            // acc[r] = score (j = 16tj + lr, i = 16ti + sigma(4lg4 + r))
            const int j = tj * 16 + lr;
            int ii[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                ii[r] = ti * 16 + sigma(lg4 * 4 + r);
            float dec[4];
            pair_decays<GATED>(sm.lg[buf], sm.zp[buf], j, ii, dec);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kf = 0; kf < 4; ++kf) {
                const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(&Kb[pr_off(ti * 16 + sigma(lr), kf * 32 + lg4 * 8)]);
                const bf16x8 qb = *reinterpret_cast<const bf16x8 *>(&Qb[pr_off(tj * 16 + lr, kf * 32 + lg4 * 8)]);
                acc = mfma(ka, qb, acc);
            }
            bf16x4 pk;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                pk[r] = static_cast<bf16>(ii[r] <= j ? acc[r] * dec[r] : 0.f);
            reinterpret_cast<uint2 *>(&sm.P[(kPairBase[tj] + (ti >> 1)) * 64 + lane])[ti & 1] =
                *reinterpret_cast<uint2 *>(&pk);
        }
        // waves 4-7: phi(q_j) . z_prev for the token tile tj = wave - 4, with z_prev
        // spread over 16 identical columns and split into bf16 high and low parts (about
        // 16 bits of z_prev reach the product)
        if (wave >= 4) {
            const int j = (wave - 4) * 16 + lr;
            f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kf = 0; kf < 4; ++kf) {
                bf16x8 zh, zl;
                z_operand(sm.zhl[buf], kf * 32 + lg4 * 4, zh, zl);
                const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(&Qb[pr_off(j, kf * 32 + lg4 * 4)]);
                const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(&Qb[pr_off(j, opaque(kf * 32 + 16 + lg4 * 4))]);
                const bf16x8 qv = cat8(lo, hi);
                d = mfma(zh, qv, d);
                d = mfma(zl, qv, d);
            }
            if (lg4 == 0)
                sm.dq[j] = d[0];
        }
        f32x4 acc[G::NTJ];
#pragma unroll
        for (int tj = 0; tj < G::NTJ; ++tj)
            acc[tj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kf = 0; kf < 4; ++kf) {
            // K step kf: feature tiles 2kf and 2kf+1 of S_prev in bf16; their accumulator
            // rows 4lg4..4lg4+3 give the permuted k order used on both sides
            bf16x8 sb;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sb[r] = static_cast<bf16>(sacc[2 * kf][r]);
                sb[4 + r] = static_cast<bf16>(sacc[2 * kf + 1][r]);
            }
            const int hi_col = opaque(kf * 32 + 16 + lg4 * 4);
#pragma unroll
            for (int tj = 0; tj < G::NTJ; ++tj) {
                const int j = tj * 16 + lr;
                const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(&Qb[pr_off(j, kf * 32 + lg4 * 4)]);
                const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(&Qb[pr_off(j, hi_col)]);
                acc[tj] = mfma(sb, cat8(lo, hi), acc[tj]);
            }
        }
        wg_barrier();  // a | b

        // ---- part b: (3) with V^T in the score tiles' k order (tokens sigma(4lg4 + e)
        //      and 16 + sigma(4lg4 + e) of the 32-token step), outputs, then (4).  The V^T
        //      operand of each 32-token step is loaded once and serves every token tile.
        bf16x8 vt[G::NKI];
#pragma unroll
        for (int ki = 0; ki < G::NKI; ++ki) {
            const int tb = ki * 32 + sigma(lg4 * 4 + te);
            vt[ki] = cat8(ld_tr(&Vb[pr_off(tb, wave * 16 + tc)]), ld_tr(&Vb[pr_off(tb + 16, wave * 16 + tc)]));
        }
#pragma unroll
        for (int tj = 0; tj < G::NTJ; ++tj) {
            const int j = tj * 16 + lr;
            // only element 0 of the denominator accumulator is read
            f32x4 dac = {sm.dq[j], 0.f, 0.f, 0.f};
            if (GATED) {
                const float g = sm.gj[buf][j];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[tj][r] *= g;
                dac[0] *= g;
            }
#pragma unroll
            for (int ki = 0; 2 * ki <= tj; ++ki) {
                const bf16x8 pb = __builtin_bit_cast(bf16x8, sm.P[(kPairBase[tj] + ki) * 64 + lane]);
                acc[tj] = mfma(vt[ki], pb, acc[tj]);
                dac = mfma(ones, pb, dac);
            }
            const float inv = __builtin_amdgcn_rcpf(dac[0] + a.eps);
            bf16x4 yb;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                yb[r] = static_cast<bf16>(acc[tj][r] * inv);
            *reinterpret_cast<bf16x4 *>(&(GATED ? sm.Ks[buf] : sm.Ys)[ys_off(j, fw)]) = yb;
        }
        const float g_end = GATED ? sm.gj[buf][n - 1] : 1.f;
        if (GATED) {
#pragma unroll
            for (int tf = 0; tf < 8; ++tf)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sacc[tf][r] *= g_end;
        }
        // (4) in k order: lane group lg4 takes tokens 8lg4 + 2e (first load) and
        //     8lg4 + 2e + 1 (second) of each 32-token step, alike for both operands
#pragma unroll
        for (int ki = 0; ki < G::NKI; ++ki) {
            const int tb = ki * 32 + lg4 * 8 + 2 * te;
            const bf16x8 vb = cat8(ld_tr(&Vb[pr_off(tb, wave * 16 + tc)]), ld_tr(&Vb[pr_off(tb + 1, wave * 16 + tc)]));
#pragma unroll
            for (int tf = 0; tf < 8; ++tf) {
                const bf16x8 ka = cat8(ld_tr(&Wb[pr_off(tb, tf * 16 + tc)]), ld_tr(&Wb[pr_off(tb + 1, tf * 16 + tc)]));
                sacc[tf] = mfma(ka, vb, sacc[tf]);
            }
        }
        wg_barrier();  // chunk i done
    }
    if (n_steps > n_chunks) {  // the trailing empty step of an odd chunk count
        wg_barrier();
        wg_barrier();
    }

    if (seg != a.nseg - 1)
        return;
    float *Sout = a.S + head * kD * kD;  // the final z leaves from the producers
#pragma unroll
    for (int tf = 0; tf < 8; ++tf)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            Sout[(tf * 16 + lg4 * 4 + r) * kD + cw] = sacc[tf][r];
}

// ============================================================================ pass 3, chunk 128
// Producer / consumer form at chunk 128.  Two buffers of every 128-token tile do not fit
// in LDS, so each tile has one buffer and the producers stage it in the half of the chunk
// in which the consumers do not read it:
//   part A (consumers: (2), phi(q).z_prev, scores (1); read Q~, K~)  producers stage V and
//          the write weights of this chunk;
//   part B (consumers: (3), outputs, (4); read V, the write weights, the score tiles)
//          producers scan the gates of the next chunk and stage its Q~ and K~.
// Q and V registers are refilled right after they are staged, so those loads have a whole
// chunk to arrive.  The raw K rows stay in registers from the staging of K~ to that of the
// write weights, so w phi(k) is formed in fp32 and rounded once, as in the chunk-64 form;
// K is then loaded for the next chunk, with the compute of part A to arrive.
// y leaves straight from the consumers, 8 bytes per lane.  Unlike the chunk-64 passes this
// one keeps the default cache policy on its streams: marked non-temporal (loads and y
// stores) it was 45 us slower per call on a 4.3 GB gated workload.
constexpr int kP8C = 128;
constexpr int kP8Producers = 4;
constexpr int kP8Threads = kPcConsumers + 64 * kP8Producers;

struct alignas(16) P8Smem {
    alignas(16) bf16 Qs[kP8C * kRow];  // phi(q)
    alignas(16) bf16 Ks[kP8C * kRow];  // phi(k), rows of the scores
    alignas(16) bf16 Vs[kP8C * kRow];  // v
    alignas(16) bf16 Kw[kP8C * kRow];  // write weights w phi(k), 0 past the end of the segment
    alignas(16) uint2 P[Cfg<kP8C>::NPT * 64];  // bf16 score tile (tj, ti) at tj (tj + 1) / 2 + ti
    alignas(16) bf16 zhl[2][2][kD];    // z entering the chunk in bf16 high and low parts, by parity
    alignas(16) float zred[3][kD];     // fp32 z update of the chunk from producer waves 9-11
    alignas(16) float dq[kP8C];        // phi(q_j) . z_prev
    // Gate scans of chunk c: lg, zp and the write weights wt are read only in part A of
    // chunk c (producers' write weights, consumers' score weights) and rewritten for chunk
    // c + 1 in part B, so one buffer each; the consumers read gj in part B too, so two.
    alignas(16) float lg[kP8C];
    alignas(16) int zp[kP8C];
    alignas(16) float wt[kP8C];
    alignas(16) float gj[2][kP8C];
};
static_assert(sizeof(P8Smem) <= 160 * 1024, "the chunk-128 tiles must fit in the 160 KB of LDS");

template <bool GATED, int FM>
__global__ __launch_bounds__(kP8Threads) void prefill_p8_kernel(Args a)
{
    constexpr int C = kP8C;
    typedef Cfg<C> G;
    static_assert(G::NTJ == 8 && G::NKI == 4, "8 token tiles, one per consumer wave");
    __shared__ P8Smem sm;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lr = lane & 15;
    const int lg4 = lane >> 4;

    const int64_t head = blockIdx.x / a.nseg;
    const int seg = blockIdx.x % a.nseg;
    const int64_t s0 = (int64_t)seg * a.seg_len;
    const int64_t s1 = seg == a.nseg - 1 ? a.T : s0 + a.seg_len;
    const int64_t len = s1 - s0;
    const int n_chunks = (int)((len + C - 1) / C);
    auto chunk_len = [&](int c) { return (int)min((int64_t)C, len - (int64_t)c * C); };
    const int64_t row0 = head * a.T + s0;

    if (wave >= 8) {
        // ============================================================ producers
        const rsrc_t rQ = make_rsrc(a.Q + row0 * kD, len * kD * 2);
        const rsrc_t rK = make_rsrc(a.K + row0 * kD, len * kD * 2);
        const rsrc_t rV = make_rsrc(a.V + row0 * kD, len * kD * 2);
        const rsrc_t rA = make_rsrc(GATED ? a.alpha + row0 : a.S, GATED ? len * 4 : 0);
        const int pt = tid - kPcConsumers;
        const bool scanner = wave == 9;  // not wave 8, which keeps z
        // thread (fg, tg) stages granule fg (8 features) of tokens TPT tg .. TPT tg + TPT - 1
        constexpr int TPT = C / 16;
        const int fg = pt & 15, tg = pt >> 4;
        const int ld_off = tg * TPT * kD * 2 + fg * 16;
        uint4 rq[TPT], rk[TPT], rv[TPT];
        float ar[2] = {0.f, 0.f};  // alpha of the next chunk to scan: tokens lane, 64 + lane
        // z: lanes 0-15 of wave 8 hold features 8 lane .. 8 lane + 7; each chunk adds the sum
        // of its fp32 write weights w phi(k), formed before their rounding to bf16
        float zreg[8], zsum[8];
        if (wave == 8 && lane < 16) {
            const float *zin = a.nseg == 1 ? a.z + head * kD : slot_ptr(a, head, seg) + kD * kD;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                zreg[e] = zin[8 * lane + e];
        }

        auto load = [&](const rsrc_t &r, int c, uint4 (&x)[TPT]) {
#pragma unroll
            for (int p = 0; p < TPT; ++p)
                x[p] = bload16(r, c * C * kD * 2 + ld_off + p * kD * 2);
        };
        auto load_a = [&](int c) {
            if (GATED) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    ar[h] = __uint_as_float(
                        (unsigned)__builtin_amdgcn_raw_buffer_load_b32(rA, (c * C + h * 64 + lane) * 4, 0, 0));
            }
        };
        // inclusive scans of log(alpha) and of the last zero-gate position over the chunk
        auto scan = [&](int n, int gs) {
            if (GATED && scanner) {
                float carry = 0.f;
                int zcarry = -1;
                float sv2[2];
                int zf2[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int j = h * 64 + lane;
                    const int jo = opaque(j);  // addresses formed here, not held across the loop
                    const float av = j < n ? ar[h] : 1.f;
                    float sv = av > 0.f ? __logf(av) : 0.f;
                    int zf = av == 0.f ? j : -1;
                    sv = wave_scan_add(sv) + carry;
                    zf = max(wave_scan_max(zf), zcarry);
                    sm.lg[jo] = sv;
                    sm.zp[jo] = zf;
                    sm.gj[gs][j] = zf >= 0 ? 0.f : __expf(sv);
                    carry = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sv), 63));
                    zcarry = __builtin_amdgcn_readlane(zf, 63);
                    sv2[h] = sv;
                    zf2[h] = zf;
                }
                // the write weights, from the scans at the chunk's last token n - 1
                const int l = n - 1;
                const float s_last = __builtin_bit_cast(
                    float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l >= 64 ? sv2[1] : sv2[0]), l & 63));
                const int z_last = __builtin_amdgcn_readlane(l >= 64 ? zf2[1] : zf2[0], l & 63);
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    sm.wt[opaque(h * 64 + lane)] = scanned_write_weight(s_last, z_last, sv2[h], n, h * 64 + lane);
            }
        };
        // phi(q) and phi(k) rows
        auto stage_qk = [&]() {
#pragma unroll
            for (int p = 0; p < TPT; ++p) {
                const int j = tg * TPT + p;
                float x[8];
                unpack8(rq[p], x);
                bf16x8 qb;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    qb[e] = static_cast<bf16>(phi<FM>(x[e]));
                *reinterpret_cast<bf16x8 *>(&sm.Qs[pr_off(j, fg * 8)]) = qb;
                unpack8(rk[p], x);
                bf16x8 kb;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    kb[e] = static_cast<bf16>(phi<FM>(x[e]));
                *reinterpret_cast<bf16x8 *>(&sm.Ks[pr_off(j, fg * 8)]) = kb;
            }
        };
        // V rows and the write weights w_j phi(k_j) (w_j = gates after j to the chunk end,
        // 0 past the end of the segment)
        auto stage_vw = [&](int n) {
            const float *wts = sm.wt + opaque(0);  // addressed afresh each chunk
#pragma unroll
            for (int e = 0; e < 8; ++e)
                zsum[e] = 0.f;
#pragma unroll
            for (int p = 0; p < TPT; ++p) {
                const int j = tg * TPT + p;
                *reinterpret_cast<uint4 *>(&sm.Vs[pr_off(j, fg * 8)]) = rv[p];
                const float w = GATED ? wts[j] : write_weight<false>(nullptr, nullptr, n, j);
                float x[8];
                unpack8(rk[p], x);
                bf16x8 kwb;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float wf = w * phi<FM>(x[e]);
                    kwb[e] = static_cast<bf16>(wf);
                    zsum[e] += wf;
                }
                *reinterpret_cast<bf16x8 *>(&sm.Kw[pr_off(j, fg * 8)]) = kwb;
            }
            // the wave's four token groups (lanes 16 t + fg) summed into every lane, in a
            // fixed order; waves 9-11 hand theirs to wave 8 through sm.zred
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                zsum[e] += __shfl_xor(zsum[e], 16, 64);
                zsum[e] += __shfl_xor(zsum[e], 32, 64);
            }
            if (wave > 8 && lane < 16) {
                *reinterpret_cast<f32x4 *>(&sm.zred[wave - 9][8 * lane]) = f32x4{zsum[0], zsum[1], zsum[2], zsum[3]};
                *reinterpret_cast<f32x4 *>(&sm.zred[wave - 9][8 * lane + 4]) = f32x4{zsum[4], zsum[5], zsum[6], zsum[7]};
            }
        };
        // after stage_vw(c) and a barrier: z entering chunk c + 1, for part A of that chunk
        auto z_update = [&](int c) {
            if (wave == 8 && lane < 16) {
                const float g = GATED ? sm.gj[c & 1][chunk_len(c) - 1] : 1.f;
                bf16x8 zh, zl;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float dz = zsum[e] + sm.zred[0][8 * lane + e] + sm.zred[1][8 * lane + e] +
                                     sm.zred[2][8 * lane + e];
                    zreg[e] = g * zreg[e] + dz;
                    zh[e] = static_cast<bf16>(zreg[e]);
                    zl[e] = static_cast<bf16>(zreg[e] - static_cast<float>(zh[e]));
                }
                *reinterpret_cast<bf16x8 *>(&sm.zhl[(c + 1) & 1][0][8 * lane]) = zh;
                *reinterpret_cast<bf16x8 *>(&sm.zhl[(c + 1) & 1][1][8 * lane]) = zl;
            }
        };

        // prologue: chunk 0's Q~ and K~ staged, its gates scanned; chunk 1's Q in flight
        load(rQ, 0, rq);
        load(rK, 0, rk);
        load(rV, 0, rv);
        load_a(0);
        scan(chunk_len(0), 0);
        load_a(1);
        stage_qk();
        load(rQ, 1, rq);
        wg_barrier();
        // Loads past the end of the segment read zeros through the buffer resources; they
        // are issued unconditionally so that every wait on them is a counted one.
        for (int c = 0; c < n_chunks; ++c) {
            // part A of chunk c
            stage_vw(chunk_len(c));
            load(rV, c + 1, rv);
            load(rK, c + 1, rk);
            wg_barrier();  // a | b
            // part B of chunk c
            z_update(c);
            if (c + 1 < n_chunks)
                scan(chunk_len(c + 1), (c + 1) & 1);
            load_a(c + 2);
            stage_qk();
            load(rQ, c + 2, rq);
            wg_barrier();  // chunk c done
        }
        if (seg == a.nseg - 1 && wave == 8 && lane < 16) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                a.z[head * kD + 8 * lane + e] = zreg[e];
        }
        return;
    }

    // ================================================================ consumers
    bf16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        ones[e] = static_cast<bf16>(1.f);
    f32x4 sacc[8];  // z lives with the producers, which pass each chunk's entering z through sm.zhl
    const int cw = wave * 16 + lr;
    const int fw = wave * 16 + lg4 * 4;
    {
        const float *Sin = a.nseg == 1 ? a.S + head * kD * kD : slot_ptr(a, head, seg);
        const float *zin = a.nseg == 1 ? a.z + head * kD : Sin + kD * kD;
#pragma unroll
        for (int tf = 0; tf < 8; ++tf)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sacc[tf][r] = Sin[(tf * 16 + lg4 * 4 + r) * kD + cw];
        if (tid < kD)
            split_store(zin[tid], &sm.zhl[0][0][tid], &sm.zhl[0][1][tid]);
    }
    const rsrc_t rY = make_rsrc(a.Y + row0 * kD, len * kD * 2);
    // transposing-load addresses: this lane supplies 4 adjacent columns (4 (lr & 3) ..)
    // of token row e = lr >> 2 of its group's set
    const int te = lr >> 2, tc = 4 * (lr & 3);
    wg_barrier();

    for (int c = 0; c < n_chunks; ++c) {
        const int buf = c & 1;
        const int n = chunk_len(c);

        // ---- part A: (2) for the eight token tiles, phi(q) . z_prev for tile `wave`, scores
        f32x4 acc[G::NTJ];
#pragma unroll
        for (int tj = 0; tj < G::NTJ; ++tj)
            acc[tj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kf = 0; kf < 4; ++kf) {
            // K step kf: feature tiles 2kf and 2kf+1 of S_prev in bf16; their accumulator
            // rows 4lg4..4lg4+3 give the permuted k order used on both sides
            bf16x8 sb;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sb[r] = static_cast<bf16>(sacc[2 * kf][r]);
                sb[4 + r] = static_cast<bf16>(sacc[2 * kf + 1][r]);
            }
            const int hi_col = opaque(kf * 32 + 16 + lg4 * 4);
#pragma unroll
            for (int tj = 0; tj < G::NTJ; ++tj) {
                const int j = tj * 16 + lr;
                const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(&sm.Qs[pr_off(j, kf * 32 + lg4 * 4)]);
                const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(&sm.Qs[pr_off(j, hi_col)]);
                acc[tj] = mfma(sb, cat8(lo, hi), acc[tj]);
            }
        }
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
        {
            const int j = wave * 16 + lr;
#pragma unroll
            for (int kf = 0; kf < 4; ++kf) {
                bf16x8 zh, zl;  // z_prev in bf16 high and low parts
                z_operand(sm.zhl[buf], kf * 32 + lg4 * 4, zh, zl);
                const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(&sm.Qs[pr_off(j, kf * 32 + lg4 * 4)]);
                const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(&sm.Qs[pr_off(j, opaque(kf * 32 + 16 + lg4 * 4))]);
                const bf16x8 qv = cat8(lo, hi);
                d = mfma(zh, qv, d);
                d = mfma(zl, qv, d);
            }
        }
        // the score tiles k = wave + 8m of the 36 on or below the diagonal: two at a time with
        // interleaved product chains (k and k + 8 for k = wave, wave + 16), then the fifth of
        // waves 0-3 (k = wave + 32) alone
        auto score_tiles = [&](auto npair, int k0) {
            constexpr int NP = decltype(npair)::value;
            int tj[NP], ti[NP];
#pragma unroll
            for (int u = 0; u < NP; ++u) {
                const int k = k0 + 8 * u;
                tj[u] = 0;
                while ((tj[u] + 1) * (tj[u] + 2) / 2 <= k)
                    ++tj[u];
                ti[u] = k - tj[u] * (tj[u] + 1) / 2;
            }
            f32x4 sc[NP];
#pragma unroll
            for (int u = 0; u < NP; ++u)
                sc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kf = 0; kf < 4; ++kf)
#pragma unroll
                for (int u = 0; u < NP; ++u) {
                    const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(&sm.Ks[pr_off(ti[u] * 16 + sigma(lr), kf * 32 + lg4 * 8)]);
                    const bf16x8 qb = *reinterpret_cast<const bf16x8 *>(&sm.Qs[pr_off(tj[u] * 16 + lr, kf * 32 + lg4 * 8)]);
                    sc[u] = mfma(ka, qb, sc[u]);
                }
#pragma unroll
            for (int u = 0; u < NP; ++u) {
                // sc[u][r] = score (j = 16tj + lr, i = 16ti + sigma(4lg4 + r))
                const int j = tj[u] * 16 + lr;
                int ii[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    ii[r] = ti[u] * 16 + sigma(lg4 * 4 + r);
                float dec[4];
                pair_decays<GATED>(sm.lg + opaque(0), sm.zp + opaque(0), j, ii, dec);
                bf16x4 pk;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    pk[r] = static_cast<bf16>(ii[r] <= j ? sc[u][r] * dec[r] : 0.f);
                sm.P[(k0 + 8 * u) * 64 + lane] = *reinterpret_cast<uint2 *>(&pk);
            }
        };
        static_assert(G::NPT == 36, "four pairs and four lone tiles over the eight waves");
        score_tiles(std::integral_constant<int, 2>{}, wave);
        score_tiles(std::integral_constant<int, 2>{}, wave + 16);
        if (wave < 4)
            score_tiles(std::integral_constant<int, 1>{}, wave + 32);
        if (lg4 == 0)
            sm.dq[wave * 16 + lr] = d[0];
        wg_barrier();  // a | b

        // ---- part B: (3) with V^T in the score tiles' k order (tokens sigma(4lg4 + e) and
        //      16 + sigma(4lg4 + e) of the 32-token step), outputs, then (4)
        auto out_begin = [&](int tj, f32x4 &dac) {
            const int j = tj * 16 + lr;
            dac = f32x4{sm.dq[j], 0.f, 0.f, 0.f};  // only element 0 is read
            if (GATED) {
                const float g = sm.gj[buf][j];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[tj][r] *= g;
                dac[0] *= g;
            }
        };
        auto out_end = [&](int tj, const f32x4 &dac) {
            const int j = tj * 16 + lr;
            const float inv = __builtin_amdgcn_rcpf(dac[0] + a.eps);
            bf16x4 yb;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                yb[r] = static_cast<bf16>(acc[tj][r] * inv);
            // rows past the end of the segment fall outside rY and are dropped
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, yb),
                                                  rY, ((c * C + j) * kD + fw) * 2, 0, 0);
        };
        auto pair = [&](int k0, int k1) {
            return cat8(__builtin_bit_cast(bf16x4, sm.P[k0 * 64 + lane]), __builtin_bit_cast(bf16x4, sm.P[k1 * 64 + lane]));
        };
        // token tiles in pairs (2m, 2m + 1), both fed from each 32-token step's V^T operand:
        // tile 2m + 1 has m + 1 full pairs of score tiles, tile 2m has m full pairs and the
        // diagonal tile alone, taken in the last step
#pragma unroll
        for (int m = 0; m < G::NTJ / 2; ++m) {
            const int t0 = 2 * m, t1 = 2 * m + 1;
            const int kb0 = t0 * (t0 + 1) / 2, kb1 = t1 * (t1 + 1) / 2;
            f32x4 dac0, dac1;
            out_begin(t0, dac0);
            out_begin(t1, dac1);
            auto vstep = [&](int ki) {
                const int tb = ki * 32 + sigma(lg4 * 4 + te);
                return cat8(ld_tr(&sm.Vs[pr_off(tb, wave * 16 + tc)]), ld_tr(&sm.Vs[pr_off(tb + 16, wave * 16 + tc)]));
            };
            for (int ki = 0; ki < m; ++ki) {
                const bf16x8 va = vstep(ki);
                const bf16x8 pb0 = pair(kb0 + 2 * ki, kb0 + 2 * ki + 1);
                const bf16x8 pb1 = pair(kb1 + 2 * ki, kb1 + 2 * ki + 1);
                acc[t0] = mfma(va, pb0, acc[t0]);
                dac0 = mfma(ones, pb0, dac0);
                acc[t1] = mfma(va, pb1, acc[t1]);
                dac1 = mfma(ones, pb1, dac1);
            }
            {
                const bf16x8 va = vstep(m);
                const bf16x8 pb0 = cat8(__builtin_bit_cast(bf16x4, sm.P[(kb0 + 2 * m) * 64 + lane]),
                                        __builtin_bit_cast(bf16x4, make_uint2(0u, 0u)));
                const bf16x8 pb1 = pair(kb1 + 2 * m, kb1 + 2 * m + 1);
                acc[t0] = mfma(va, pb0, acc[t0]);
                dac0 = mfma(ones, pb0, dac0);
                acc[t1] = mfma(va, pb1, acc[t1]);
                dac1 = mfma(ones, pb1, dac1);
            }
            out_end(t0, dac0);
            out_end(t1, dac1);
        }
        const float g_end = GATED ? sm.gj[buf][n - 1] : 1.f;
        if (GATED) {
#pragma unroll
            for (int tf = 0; tf < 8; ++tf)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sacc[tf][r] *= g_end;
        }
        // (4) in k order: lane group lg4 takes tokens 8lg4 + 2e (first load) and
        //     8lg4 + 2e + 1 (second) of each 32-token step, alike for both operands
#pragma unroll
        for (int ki = 0; ki < G::NKI; ++ki) {
            const int tb = ki * 32 + lg4 * 8 + 2 * te;
            const bf16x8 vb = cat8(ld_tr(&sm.Vs[pr_off(tb, wave * 16 + tc)]), ld_tr(&sm.Vs[pr_off(tb + 1, wave * 16 + tc)]));
#pragma unroll
            for (int tf = 0; tf < 8; ++tf) {
                const bf16x8 ka = cat8(ld_tr(&sm.Kw[pr_off(tb, tf * 16 + tc)]), ld_tr(&sm.Kw[pr_off(tb + 1, tf * 16 + tc)]));
                sacc[tf] = mfma(ka, vb, sacc[tf]);
            }
        }
        wg_barrier();  // chunk c done
    }

    if (seg != a.nseg - 1)
        return;
    float *Sout = a.S + head * kD * kD;  // the final z leaves from the producers
#pragma unroll
    for (int tf = 0; tf < 8; ++tf)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            Sout[(tf * 16 + lg4 * 4 + r) * kD + cw] = sacc[tf][r];
}

// ============================================================================ pass 1, chunk 64
// Segment maps in the same producer / consumer form: producers stage the write weights
// w phi(k) and V of the next chunk as token rows, consumers fold each chunk into
// (S, z) with transposing loads, one workgroup barrier per chunk.  The gate scan runs
// two chunks ahead of the consumers, so its results are kept for three chunks.  This
// pass has 8 producer waves (16 in all): its consumers only do the state write, so the
// staging sets the pace, and the registers of both roles fit 4 waves per SIMD.
template <bool GATED>
struct alignas(16) SumSmem {
    alignas(16) bf16 Ws[2][kPcC * kRow];  // w phi(k) (ungated: phi(k), zero past the end)
    alignas(16) bf16 Vs[2][kPcC * kRow];
    alignas(16) float zred[2][kSumProducers * 4][kD];  // fp32 z update per token group, by chunk parity
    alignas(16) float lg[3][kPcC];
    alignas(16) float gj[3][kPcC];
    alignas(16) int zp[3][kPcC];
    alignas(16) float wt[GATED ? 3 : 1][GATED ? kPcC : 4];  // write weights (gated)
};

// NONCAUSAL (ungated): every segment's map is needed, including the last one's, and it
// goes to the segment's own slot; with a single segment it is added straight into the
// caller's S and z.
template <bool GATED, int FM, bool NONCAUSAL>
__global__ __launch_bounds__(kSumThreads) void summary_pc_kernel(Args a)
{
    static_assert(!(GATED && NONCAUSAL), "the non-causal form has no gate");
    constexpr int C = kPcC;
    typedef Cfg<C> G;
    __shared__ SumSmem<GATED> sm;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lr = lane & 15;
    const int lg4 = lane >> 4;

    // Segment-major block order: workgroup b runs on XCD b mod 8, so numbering
    // (sequence, segment) head-major would put every idle last-segment workgroup on the
    // same XCDs whenever the segment count divides 8; segment-major spreads them evenly.
    const int64_t n_heads = gridDim.x / a.nseg;
    const int64_t head = blockIdx.x % n_heads;
    const int seg = (int)(blockIdx.x / n_heads);
    if (!NONCAUSAL && seg == a.nseg - 1)
        return;  // the last segment's map is never needed
    const int64_t s0 = (int64_t)seg * a.seg_len;
    const int64_t len = seg == a.nseg - 1 ? a.T - s0 : a.seg_len;
    const int n_chunks = (int)((len + C - 1) / C);
    // both roles walk the same number of chunk steps, a multiple of the register sets
    const int n_steps = (n_chunks + kSumSets - 1) / kSumSets * kSumSets;
    auto chunk_len = [&](int c) { return (int)min((int64_t)C, len - (int64_t)c * C); };
    const int64_t row0 = head * a.T + s0;

    if (wave >= 8) {
        // ============================================================ producers
        const rsrc_t rK = make_rsrc(a.K + row0 * kD, len * kD * 2);
        const rsrc_t rV = make_rsrc(a.V + row0 * kD, len * kD * 2);
        const rsrc_t rA = make_rsrc(GATED ? a.alpha + row0 : a.S, GATED ? len * 4 : 0);
        const int pt = tid - kPcConsumers;
        const bool scanner = wave == 8;
        constexpr int TPT = 16 / kSumProducers;  // tokens per thread and chunk
        const int fg = pt & 15, tg = pt >> 4;    // granule fg of tokens TPT tg .. TPT tg + TPT - 1
        const int ld_off = tg * TPT * kD * 2 + fg * 16;
        uint4 rk[kSumSets][TPT], rv[kSumSets][TPT];  // chunk c in set c % kSumSets
        float ar[2] = {0.f, 0.f};                      // alpha of even / odd chunks

        auto load_kv = [&](int c, uint4 (&rkx)[TPT], uint4 (&rvx)[TPT]) {
#pragma unroll
            for (int p = 0; p < TPT; ++p) {
                rkx[p] = bload16<NONCAUSAL ? kNT : 0>(rK, c * C * kD * 2 + ld_off + p * kD * 2);
                rvx[p] = bload16<NONCAUSAL ? kNT : 0>(rV, c * C * kD * 2 + ld_off + p * kD * 2);
            }
        };
        auto load_a = [&](int c, float &arx) {  // every producer wave loads; the scanner uses it
            if (GATED)
                arx = __uint_as_float((unsigned)__builtin_amdgcn_raw_buffer_load_b32(rA, (c * C + lane) * 4, 0, 0));
        };
        auto scan = [&](int n, int gs, float arx) {
            if (GATED && scanner) {
                const float av = lane < n ? arx : 1.f;
                float s = av > 0.f ? __logf(av) : 0.f;
                int zf = av == 0.f ? lane : -1;
                s = wave_scan_add(s);
                zf = wave_scan_max(zf);
                sm.lg[gs][lane] = s;
                sm.zp[gs][lane] = zf;
                sm.gj[gs][lane] = zf >= 0 ? 0.f : __expf(s);
                sm.wt[gs][lane] = lane_write_weight(s, zf, n, lane);
            }
        };
        // write weights w phi(k) in bf16 (Ws, the operand of S), 0 past the end of the
        // segment, and their fp32 sums over this thread's tokens for z (zred)
        auto stage = [&](int buf, int gs, int n, const uint4 (&rkx)[TPT], const uint4 (&rvx)[TPT]) {
            float zp8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < TPT; ++p) {
                const int j = tg * TPT + p;
                const float w = GATED ? sm.wt[gs][j] : write_weight<false>(nullptr, nullptr, n, j);
                float x[8];
                unpack8(rkx[p], x);
                bf16x8 kb;
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const float wf = GATED ? w * phi<FM>(x[s]) : (j < n ? phi<FM>(x[s]) : 0.f);
                    kb[s] = static_cast<bf16>(wf);
                    zp8[s] += wf;
                }
                *reinterpret_cast<uint4 *>(&sm.Ws[buf][pr_off(j, fg * 8)]) = *reinterpret_cast<uint4 *>(&kb);
                *reinterpret_cast<uint4 *>(&sm.Vs[buf][pr_off(j, fg * 8)]) = rvx[p];
            }
            *reinterpret_cast<f32x4 *>(&sm.zred[buf][tg][fg * 8]) = f32x4{zp8[0], zp8[1], zp8[2], zp8[3]};
            *reinterpret_cast<f32x4 *>(&sm.zred[buf][tg][fg * 8 + 4]) = f32x4{zp8[4], zp8[5], zp8[6], zp8[7]};
        };
        // interval i: stage chunk i + 1 from its set and refill the set with chunk
        // i + 1 + kSumSets; scan the gates of chunk i + 2 and load the alpha of chunk i + 4
        // in its place.  Loads past the end of the segment read zeros through the buffer
        // resource; they are issued unconditionally so that every wait on them is a
        // counted one.
        auto step = [&](int i, uint4 (&rkx)[TPT], uint4 (&rvx)[TPT], float &arx) {
            const int cn = i + 1;
            if (cn < n_chunks)
                stage(cn & 1, cn % 3, chunk_len(cn), rkx, rvx);
            load_kv(cn + kSumSets, rkx, rvx);
            if (i + 2 < n_chunks)
                scan(chunk_len(i + 2), (i + 2) % 3, arx);
            load_a(i + 4, arx);
            wg_barrier();  // chunk i done, chunk i + 1 staged
        };

#pragma unroll
        for (int c = 0; c < kSumSets; ++c) {
            load_kv(c, rk[c], rv[c]);
            if (c < 2)
                load_a(c, ar[c]);
        }
        scan(chunk_len(0), 0, ar[0]);
        if (n_chunks > 1)
            scan(chunk_len(1), 1, ar[1]);
        load_a(2, ar[0]);
        load_a(3, ar[1]);
        wg_barrier();
        stage(0, 0, chunk_len(0), rk[0], rv[0]);
        load_kv(kSumSets, rk[0], rv[0]);
        wg_barrier();
        for (int i = 0; i < n_steps; i += kSumSets) {
#pragma unroll
            for (int u = 0; u < kSumSets; ++u)  // stages chunk i + u + 1, scans chunk i + u + 2
                step(i + u, rk[(u + 1) % kSumSets], rv[(u + 1) % kSumSets], ar[u & 1]);
        }
        return;
    }

    // ================================================================ consumers
    f32x4 sacc[8];
#pragma unroll
    for (int tf = 0; tf < 8; ++tf)
        sacc[tf] = f32x4{0.f, 0.f, 0.f, 0.f};
    float zf = 0.f;  // threads tid < 128: z of feature tid, from the producers' fp32 sums
    float g_seg = 1.f;
    const int cw = wave * 16 + lr;
    const int te = lr >> 2, tc = 4 * (lr & 3);
    wg_barrier();
    wg_barrier();
    for (int i = 0; i < n_chunks; ++i) {
        const int buf = i & 1;
        const bf16 *Wb = sm.Ws[buf];
        const bf16 *Vb = sm.Vs[buf];
        if (GATED) {
            const float g_end = sm.gj[i % 3][chunk_len(i) - 1];
            g_seg *= g_end;
#pragma unroll
            for (int tf = 0; tf < 8; ++tf)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sacc[tf][r] *= g_end;
            zf *= g_end;
        }
        if (tid < kD) {
            float dz = 0.f;
#pragma unroll
            for (int t = 0; t < kSumProducers * 4; ++t)
                dz += sm.zred[buf][t][tid];
            zf += dz;
        }
#pragma unroll
        for (int ki = 0; ki < G::NKI; ++ki) {
            const int tb = ki * 32 + lg4 * 8 + 2 * te;
            const bf16x8 vb = cat8(ld_tr(&Vb[pr_off(tb, wave * 16 + tc)]), ld_tr(&Vb[pr_off(tb + 1, wave * 16 + tc)]));
#pragma unroll
            for (int tf = 0; tf < 8; ++tf) {
                const bf16x8 ka = cat8(ld_tr(&Wb[pr_off(tb, tf * 16 + tc)]), ld_tr(&Wb[pr_off(tb + 1, tf * 16 + tc)]));
                sacc[tf] = mfma(ka, vb, sacc[tf]);
            }
        }
        wg_barrier();  // chunk i folded
    }
    for (int i = n_chunks; i < n_steps; ++i)  // trailing empty steps up to a multiple of the register sets
        wg_barrier();

    // causal: the map goes to the next segment's slot: S, z, then the product of the gates
    float *Sout = slot_ptr(a, head, NONCAUSAL ? seg : seg + 1);
    float *zout = Sout + kD * kD;
    bool add_in = false;
    if (NONCAUSAL && a.nseg == 1) {
        Sout = a.S + head * kD * kD;
        zout = a.z + head * kD;
        add_in = true;
    }
    if (!NONCAUSAL && tid == 0)
        Sout[kD * kD + kD] = g_seg;
#pragma unroll
    for (int tf = 0; tf < 8; ++tf)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float *o = &Sout[(tf * 16 + lg4 * 4 + r) * kD + cw];
            *o = sacc[tf][r] + (add_in ? *o : 0.f);
        }
    if (tid < kD)
        zout[tid] = zf + (add_in ? zout[tid] : 0.f);
}

template <int C, bool GATED, int FM>
hipError_t launch_c(const Args &a, int64_t n_heads, hipStream_t stream)
{
    const unsigned blocks = (unsigned)(n_heads * a.nseg);
    if (a.nseg > 1) {
        // pass 1 walks 64-token chunks whatever the caller's chunk: its chunking only
        // changes the rounding of the segment maps
        summary_pc_kernel<GATED, FM, false><<<dim3(blocks), dim3(kSumThreads), 0, stream>>>(a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        segment_scan_kernel<Args><<<dim3((kD * kD + kD + 255) / 256, (unsigned)n_heads), dim3(256), 0, stream>>>(a);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    if constexpr (C == kPcC)
        prefill_pc_kernel<GATED, FM><<<dim3(blocks), dim3(kPcThreads), 0, stream>>>(a);
    else
        prefill_p8_kernel<GATED, FM><<<dim3(blocks), dim3(kP8Threads), 0, stream>>>(a);
    return hipGetLastError();
}

// ============================================================================ non-causal form
// Non-causal form (page "线性注意力架构演进", ai-master.cc: K~^T V and the key sum are
// formed once and every query reads them):
//   pass 1  summary_pc_kernel<false, FM, true>: each (sequence, segment) folds its tokens
//           into (dS, dz) in its own slot (a single segment adds into S, z directly);
//   pass 2  segment_sum_kernel: S = S_in + sum of the slots, same for z;
//   pass 3  noncausal_readout_kernel: y_t = q~_t^T S / (q~_t^T z + eps) for every t.

// S_out = S_in + sum over segments of dS (and z likewise), in the caller's S and z.
__global__ __launch_bounds__(256) void segment_sum_kernel(Args a)
{
    const int64_t head = blockIdx.y;
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= kD * kD + kD)
        return;
    float *dst = e < kD * kD ? &a.S[head * kD * kD + e] : &a.z[head * kD + (e - kD * kD)];
    float run = *dst;
    constexpr int kBatch = 8;
    for (int p0 = 0; p0 < a.nseg; p0 += kBatch) {
        float d[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q)
            d[q] = p0 + q < a.nseg ? slot_ptr(a, head, p0 + q)[e] : 0.f;
#pragma unroll
        for (int q = 0; q < kBatch; ++q)
            run += d[q];
    }
    *dst = run;
}

// Read-out: one workgroup of 8 waves per (sequence, block of kNcBlockTokens tokens).
// The workgroup converts S to bf16 once, transposed into LDS, with z split into bf16
// high and low parts (so the denominator keeps about 16 bits of z); every wave then
// keeps S^T in registers as 32 MFMA A-operands and streams 16-token tiles of Q through
// v_mfma_f32_16x16x32_bf16: the transposed numerator N^T = S^T Q~^T and the
// denominator 1 z^T Q~^T, so a lane ends with eight adjacent output columns of one
// token and that token's denominator.
// Q and Y move between HBM and registers as whole 256-byte rows (16 lanes per row,
// four rows per instruction) and are rearranged through a wave-private LDS tile into
// and out of the MFMA layouts; the tiles' 16-byte granules are XOR-swizzled by row so
// that both sides of the rearrangement are free of bank conflicts.  The first tiles'
// loads are issued before the staging, and three register sets keep up to three
// tiles in flight per wave.
constexpr int kNcWaves = 8;
constexpr int kNcThreads = 64 * kNcWaves;
constexpr int kNcTilesPerWave = 8;
constexpr int kNcSets = 3;
constexpr int kNcBlockTokens = 16 * kNcWaves * kNcTilesPerWave;
constexpr int kStRow = kD + 8;  // bf16 row stride of S^T in LDS (272 bytes)

// byte offset of 16-byte granule `gran` of row `row` in a swizzled 16 x 256-byte tile
__device__ __forceinline__ int sw_off(int row, int gran) { return row * 256 + ((gran ^ row) & 15) * 16; }

template <int FM>
__global__ __launch_bounds__(kNcThreads) void noncausal_readout_kernel(Args a, int blocks_per_head)
{
    __shared__ __align__(16) bf16 St[kD * kStRow];             // St[f][r] = S[r][f]
    __shared__ __align__(16) bf16x8 Zs[2][4][4];                // [hi/lo][k-step][lane group]: z of 8 features
    __shared__ __align__(16) unsigned char Qt[kNcWaves][4096];  // per wave: a Q tile, swizzled
    __shared__ __align__(16) unsigned char Yt[kNcWaves][4096];  // per wave: a Y tile, swizzled

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int m = lane & 15;  // A-operand row / B-operand column (token) / output column
    const int g = lane >> 4;  // lane group: k = 8g .. 8g+7 of each 32-wide step
    const int64_t head = blockIdx.x / blocks_per_head;
    const int64_t t0 = (int64_t)(blockIdx.x % blocks_per_head) * kNcBlockTokens;
    const int len = (int)min((int64_t)kNcBlockTokens, a.T - t0);

    // this block's rows of Q and Y; reads past the end give zeros, writes are dropped
    const int64_t row0 = head * a.T + t0;
    const rsrc_t rQ = make_rsrc(a.Q + row0 * kD, (int64_t)len * kD * 2);
    const rsrc_t rY = make_rsrc(a.Y + row0 * kD, (int64_t)len * kD * 2);
    const float eps = a.eps;
    unsigned char *qt = Qt[wave];
    unsigned char *yt = Yt[wave];
    auto tile_of = [&](int it) { return wave + it * kNcWaves; };  // tiles wave, wave + 8, ...
    // row-major transfers: lane takes granule m of rows g, g + 4, g + 8, g + 12
    auto load = [&](int tile, uint4 (&q)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            q[i] = bload16(rQ, ((tile * 16 + 4 * i + g) * kD + 8 * m) * 2);
    };
    uint4 qr[kNcSets][4];
#pragma unroll
    for (int it = 0; it < kNcSets; ++it)
        load(tile_of(it), qr[it]);

    // S (fp32, [r][f]) -> bf16 S^T in LDS: a thread takes rows r, r+1 of four columns
    const float *Sh = a.S + head * kD * kD;
    for (int e = tid; e < kD * kD / 8; e += kNcThreads) {
        const int r = 2 * (e >> 5), f = 4 * (e & 31);
        const float4 s0 = *reinterpret_cast<const float4 *>(&Sh[r * kD + f]);
        const float4 s1 = *reinterpret_cast<const float4 *>(&Sh[(r + 1) * kD + f]);
        const float lo[4] = {s0.x, s0.y, s0.z, s0.w}, hi[4] = {s1.x, s1.y, s1.z, s1.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            bf16x2 pr;
            pr[0] = static_cast<bf16>(lo[i]);
            pr[1] = static_cast<bf16>(hi[i]);
            *reinterpret_cast<bf16x2 *>(&St[(f + i) * kStRow + r]) = pr;
        }
    }
    // z as A operands (every row the same): k-step ks, lane group gg holds features
    // 32 ks + 8 gg .. + 7
    if (tid < 16) {
        const int ks = tid >> 2, gg = tid & 3;
        const float *zh = a.z + head * kD + 32 * ks + 8 * gg;
        const float4 z0 = *reinterpret_cast<const float4 *>(zh);
        const float4 z1 = *reinterpret_cast<const float4 *>(zh + 4);
        const float zv[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
        bf16x8 h, l;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            h[s] = static_cast<bf16>(zv[s]);
            l[s] = static_cast<bf16>(zv[s] - static_cast<float>(h[s]));
        }
        Zs[0][ks][gg] = h;
        Zs[1][ks][gg] = l;
    }
    __syncthreads();

    // S^T operands: tile ft, row m holds column f(ft, m) = 32 (ft/2) + 8 (m/4) + 4 (ft%2) + m%4,
    // so output row 4g + i of tiles 2j and 2j+1 are columns 32 j + 8 g + 0..7 (granule 4j + g)
    bf16x8 sa[8][4];
#pragma unroll
    for (int ft = 0; ft < 8; ++ft) {
        const int f = 32 * (ft >> 1) + 8 * (m >> 2) + 4 * (ft & 1) + (m & 3);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            sa[ft][ks] = *reinterpret_cast<const bf16x8 *>(&St[f * kStRow + 32 * ks + 8 * g]);
    }

    auto compute = [&](int tile, const uint4 (&q)[4]) {
        // rows into the wave's Q tile, then the B operands: token m, granule 4 ks + g
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<uint4 *>(&qt[sw_off(4 * i + g, m)]) = q[i];
        bf16x8 qb[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            float x[8];
            unpack8(*reinterpret_cast<const uint4 *>(&qt[sw_off(m, 4 * ks + g)]), x);
#pragma unroll
            for (int s = 0; s < 8; ++s)
                qb[ks][s] = static_cast<bf16>(phi<FM>(x[s]));
        }
        f32x4 acc[8], den = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ft = 0; ft < 8; ++ft)
            acc[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int ft = 0; ft < 8; ++ft)
                acc[ft] = mfma(sa[ft][ks], qb[ks], acc[ft]);
            den = mfma(Zs[0][ks][g], qb[ks], den);
            den = mfma(Zs[1][ks][g], qb[ks], den);
        }
        const float rd = 1.f / (den[0] + eps);
        // token m's columns 32 j + 8 g .. + 7 into the wave's Y tile, then out as rows
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bf16x8 yb;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                yb[i] = static_cast<bf16>(acc[2 * j][i] * rd);
                yb[4 + i] = static_cast<bf16>(acc[2 * j + 1][i] * rd);
            }
            *reinterpret_cast<bf16x8 *>(&yt[sw_off(m, 4 * j + g)]) = yb;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 u = *reinterpret_cast<const uint4 *>(&yt[sw_off(4 * i + g, m)]);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, u),
                                                   rY, ((tile * 16 + 4 * i + g) * kD + 8 * m) * 2, 0, 0);
        }
    };

    // tile it is computed from set it % kNcSets, which is then refilled with tile
    // it + kNcSets; tiles past the block compute nothing (loads past it read zeros)
    const int n_tiles = (len + 15) / 16;
#pragma unroll
    for (int it = 0; it < kNcTilesPerWave; ++it) {
        if (tile_of(it) < n_tiles)
            compute(tile_of(it), qr[it % kNcSets]);
        if (it + kNcSets < kNcTilesPerWave)
            load(tile_of(it + kNcSets), qr[it % kNcSets]);
    }
}

template <int FM>
hipError_t launch_nc(const Args &a, int64_t n_heads, hipStream_t stream)
{
    summary_pc_kernel<false, FM, true><<<dim3((unsigned)(n_heads * a.nseg)), dim3(kSumThreads), 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    if (a.nseg > 1) {
        segment_sum_kernel<<<dim3((kD * kD + kD + 255) / 256, (unsigned)n_heads), dim3(256), 0, stream>>>(a);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    const int64_t bph = (a.T + kNcBlockTokens - 1) / kNcBlockTokens;
    noncausal_readout_kernel<FM><<<dim3((unsigned)(n_heads * bph)), dim3(kNcThreads), 0, stream>>>(a, (int)bph);
    return hipGetLastError();
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Segments per sequence: enough (sequence, segment) workgroups to give every compute
// unit work, each segment a whole number of chunks and long enough to hold its slot of
// slot_bytes in its rows of Y, every segment (the last may be up to twice as long) below
// 2^31 bytes of Q rows of row_bytes each so that buffer offsets stay 32-bit.
// Returns 0 when the grid would not fit or a segment could not be kept that short.
int64_t choose_segments(int64_t T, int64_t n_heads, int C, int64_t target, int64_t row_bytes, int64_t slot_bytes)
{
    int64_t nseg = (target + n_heads - 1) / n_heads;
    const int64_t min_tokens = (slot_bytes + row_bytes - 1) / row_bytes;
    const int64_t min_len = ((min_tokens + C - 1) / C) * C;
    if (nseg > T / min_len)
        nseg = T / min_len;
    const int64_t max_len = ((int64_t)1 << 31) / row_bytes / 2;
    if (nseg < (T + max_len - 1) / max_len)
        nseg = (T + max_len - 1) / max_len;
    if (nseg < 1)
        nseg = 1;
    if (n_heads * nseg > INT32_MAX)
        return 0;
    const int64_t seg_len = nseg == 1 ? T : ((T / nseg) / C) * C;
    if ((T - (nseg - 1) * seg_len) * row_bytes >= ((int64_t)1 << 31))
        return 0;
    return nseg;
}

}  // namespace

bool plan_segments(int64_t n_heads, int64_t T, int32_t chunk, int64_t row_bytes, int64_t slot_bytes, int64_t *nseg,
                   int64_t *seg_len)
{
    *nseg = choose_segments(T, n_heads, chunk, kSegmentTarget, row_bytes, slot_bytes);
    if (*nseg == 0)
        return false;
    *seg_len = *nseg == 1 ? T : ((T / *nseg) / chunk) * chunk;  // the last segment takes the rest
    return true;
}

int64_t segment_slot_bytes(int32_t d) { return ((int64_t)d * d + d + 4) * 4; }

bool mfma_prefill_supported(la_dtype io_dtype, int32_t d, int32_t dv, int32_t chunk)
{
    return io_dtype == LA_BF16 && d == kD && dv == kD && (chunk == 64 || chunk == 128);
}

bool mfma_noncausal_supported(la_dtype io_dtype, int32_t d, int32_t dv)
{
    return io_dtype == LA_BF16 && d == kD && dv == kD;
}

hipError_t launch_noncausal_mfma_bf16(const PrefillArgs &pa, hipStream_t stream)
{
    if (!aligned16(pa.Q) || !aligned16(pa.K) || !aligned16(pa.V) || !aligned16(pa.Y) || !aligned16(pa.S) ||
        !aligned16(pa.z))
        return launch_noncausal_general(pa, LA_BF16, stream);
    Args a;
    a.Q = static_cast<const bf16 *>(pa.Q);
    a.K = static_cast<const bf16 *>(pa.K);
    a.V = static_cast<const bf16 *>(pa.V);
    a.alpha = nullptr;
    a.Y = static_cast<bf16 *>(pa.Y);
    a.S = static_cast<float *>(pa.S);
    a.z = static_cast<float *>(pa.z);
    a.T = pa.T;
    a.eps = (float)pa.eps;
    int64_t nseg, seg_len;
    const int64_t bph = (pa.T + kNcBlockTokens - 1) / kNcBlockTokens;
    if (!plan_segments(pa.n_heads, pa.T, kPcC, kD * 2, segment_slot_bytes(kD), &nseg, &seg_len) || pa.n_heads * bph > INT32_MAX)
        return hipErrorInvalidValue;
    a.nseg = (int)nseg;
    a.seg_len = seg_len;
    return dispatch_feature_map(pa.phi, [&](auto fm) { return launch_nc<decltype(fm)::value>(a, pa.n_heads, stream); });
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

    const int C = pa.chunk;
    int64_t nseg, seg_len;
    if (!plan_segments(pa.n_heads, pa.T, C, kD * 2, segment_slot_bytes(kD), &nseg, &seg_len))
        return hipErrorInvalidValue;
    a.nseg = (int)nseg;
    a.seg_len = seg_len;

    return dispatch_feature_map(pa.phi, [&](auto fm) {
        constexpr int FM = decltype(fm)::value;
        if (C == 64)
            return pa.alpha ? launch_c<64, true, FM>(a, pa.n_heads, stream)
                            : launch_c<64, false, FM>(a, pa.n_heads, stream);
        return pa.alpha ? launch_c<128, true, FM>(a, pa.n_heads, stream)
                        : launch_c<128, false, FM>(a, pa.n_heads, stream);
    });
}

}  // namespace la
