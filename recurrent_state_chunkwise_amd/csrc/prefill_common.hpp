// Device helpers shared by the MFMA prefill kernels (bf16 and fp32 inputs): vector types,
// the fast feature map, buffer resources, the in-chunk gate weights, wave scans and the
// workgroup barrier.
#pragma once

#include "device_common.hpp"

namespace la {
namespace {

typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;          // feature width d = r and value width dv
constexpr float kLog2e = 1.4426950408889634f;

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

// The feature map on the values the kernels stage as bf16 operands, where the few-ulp
// error of the hardware exp2 and reciprocal is far below the bf16 rounding that follows.
// ELU + 1 is the median of (x + 1, e^x, 1): x + 1 for x > 0 (where e^x > x + 1 > 1) and
// e^x for x <= 0 (where x + 1 <= e^x <= 1).  The other maps are those of la_feature_map.
template <int FM>
__device__ __forceinline__ float phi(float x)
{
    if constexpr (FM == LA_PHI_RELU1)
        return __builtin_fmaxf(x, 0.f) + 1.f;
    else if constexpr (FM == LA_PHI_RELU_EPS)
        return __builtin_fmaxf(x, 0.f) + 1e-5f;
    else if constexpr (FM == LA_PHI_SIGMOID_EPS)
        return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-x * kLog2e)) + 1e-5f;
    else
        return __builtin_amdgcn_fmed3f(x + 1.f, __builtin_amdgcn_exp2f(x * kLog2e), 1.f);
}

// Buffer resources (gfx9 raw buffers): an access at or past num_records bytes reads
// zeros and drops writes, which is how the last, partial chunk of a segment is handled.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
// Cache policy operand of the buffer accesses: kNT marks an access non-temporal (the `nt`
// bit), for data read for the last time or written and not read back by the library:
// such lines are not kept in the caches, where the output rows would otherwise wait,
// dirty, to be written back during the next kernel.
constexpr int kNT = 2;
template <int POL = 0>
__device__ __forceinline__ uint4 bload16(rsrc_t r, int off)
{
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POL);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// Gate weights inside a chunk, from lg (the in-chunk prefix sums of log alpha, zero gates
// left out) and zp (the position of the last zero gate at or before each token, -1 if
// none).  The weight of token i's write as token j reads it (i <= j) is the product of
// the gates of tokens i+1..j: 0 if one of them is zero, else exp(lg_j - lg_i).  Both
// helpers read everything they need and evaluate the exponentials unconditionally, then
// select, so that their LDS reads are issued together rather than one behind another in
// branches; for i > j the exponential may overflow and is discarded by the caller.
template <bool GATED>
__device__ __forceinline__ void pair_decays(const float *lg, const int *zp, int j, const int (&i)[4], float (&dec)[4])
{
    if (!GATED) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            dec[r] = 1.f;
        return;
    }
    const float lgj = lg[j];
    const int zpj = zp[j];
    float lgi[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
        lgi[r] = lg[i[r]];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float e = __expf(lgj - lgi[r]);
        dec[r] = zpj > i[r] ? 0.f : e;
        asm volatile("" : "+v"(dec[r]));  // computed here, not sunk into the caller's i <= j branch
    }
}
// write weight of token j of a chunk of n tokens: the gates after j to the chunk end;
// 0 past the end of the chunk (where the tokens read as zeros)
template <bool GATED>
__device__ __forceinline__ float write_weight(const float *lg, const int *zp, int n, int j)
{
    float w = 1.f;
    if (GATED) {
        const float e = __expf(lg[n - 1] - lg[j]);
        w = zp[n - 1] > j ? 0.f : e;
    }
    return j >= n ? 0.f : w;
}

// The same write weight for token `lane` of a chunk of n tokens, formed by the wave that
// has just scanned the chunk's gates (s: this lane's prefix sum of log alpha, zf: its last
// zero-gate position), so that the staging reads one stored value instead of two scans and
// an exponential: the operands and the arithmetic are those of write_weight, bitwise.
// s_last, z_last: the scans at the chunk's last token n - 1; s: the scan at token j.
__device__ __forceinline__ float scanned_write_weight(float s_last, int z_last, float s, int n, int j)
{
    const float e = __expf(s_last - s);
    const float w = z_last > j ? 0.f : e;
    return j >= n ? 0.f : w;
}
__device__ __forceinline__ float lane_write_weight(float s, int zf, int n, int lane)
{
    const float s_last = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), n - 1));
    return scanned_write_weight(s_last, __builtin_amdgcn_readlane(zf, n - 1), s, n, lane);
}

// Inclusive scans over the 64 lanes of a wave with data-parallel moves (DPP): shifts by 1,
// 2, 4 and 8 lanes inside each row of 16, then the row totals carried from lane 15 to rows
// 1 and 3 and from lane 31 to rows 2 and 3.  A lane whose source falls outside its row, or
// whose row is masked off, receives the identity.  Full-rate VALU moves, no LDS round trip.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_move(int identity, int v)
{
    return __builtin_amdgcn_update_dpp(identity, v, CTRL, ROWS, 0xf, false);
}
__device__ __forceinline__ float wave_scan_add(float x)
{
    const auto step = [](float v, int moved) { return v + __builtin_bit_cast(float, moved); };
    const auto bits = [](float v) { return __builtin_bit_cast(int, v); };
    x = step(x, dpp_move<0x111, 0xf>(0, bits(x)));  // row_shr:1
    x = step(x, dpp_move<0x112, 0xf>(0, bits(x)));  // row_shr:2
    x = step(x, dpp_move<0x114, 0xf>(0, bits(x)));  // row_shr:4
    x = step(x, dpp_move<0x118, 0xf>(0, bits(x)));  // row_shr:8
    x = step(x, dpp_move<0x142, 0xa>(0, bits(x)));  // row_bcast:15
    x = step(x, dpp_move<0x143, 0xc>(0, bits(x)));  // row_bcast:31
    return x;
}
__device__ __forceinline__ int wave_scan_max(int x)  // identity -1
{
    x = max(x, dpp_move<0x111, 0xf>(-1, x));
    x = max(x, dpp_move<0x112, 0xf>(-1, x));
    x = max(x, dpp_move<0x114, 0xf>(-1, x));
    x = max(x, dpp_move<0x118, 0xf>(-1, x));
    x = max(x, dpp_move<0x142, 0xa>(-1, x));
    x = max(x, dpp_move<0x143, 0xc>(-1, x));
    return x;
}

template <int C>
struct Cfg {
    static constexpr int NTJ = C / 16;                 // 16-token tiles per chunk
    static constexpr int NKI = C / 32;                 // 32-token MFMA steps per chunk
    static constexpr int NPT = NTJ * (NTJ + 1) / 2;    // tiles on or below the diagonal
};

// workgroup barrier with LDS visibility; reached the same number of times by every
// wave, from the producer and the consumer loops alike
__device__ __forceinline__ void wg_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Pass 2: entering state of every segment, in place over the segment maps.
// slot 0 <- (S0, z0); slot p <- G_{p-1} slot(p-1) + dS_{p-1}   (p = 1 .. nseg-1)
// The maps are read 8 at a time before the chain runs, so the loads overlap.
// A is the argument block of the pass; slot_ptr(a, head, p) locates slot p: S [D][D], z [D],
// then the segment's gate product.
template <typename A, int D = kD>
__global__ __launch_bounds__(256) void segment_scan_kernel(A a)
{
    const int64_t head = blockIdx.y;
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= D * D + D)
        return;
    float run = e < D * D ? a.S[head * D * D + e] : a.z[head * D + (e - D * D)];
    slot_ptr(a, head, 0)[e] = run;
    constexpr int kBatch = 8;
    for (int p0 = 1; p0 < a.nseg; p0 += kBatch) {
        float d[kBatch], g[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            if (p0 + q < a.nseg) {
                const float *sl = slot_ptr(a, head, p0 + q);
                d[q] = sl[e];
                g[q] = sl[D * D + D];
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

}  // namespace
}  // namespace la
