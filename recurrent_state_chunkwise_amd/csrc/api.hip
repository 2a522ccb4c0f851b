// C ABI of the linear-attention library: argument checks, kernel choice, launch.
// Every check runs on the host before anything is enqueued, so a rejected call
// has no side effect.
#include <math.h>
#include <stdint.h>

#include "internal.hpp"
#include "linattn.h"

namespace {

bool known_dtype(la_dtype t) { return t == LA_F64 || t == LA_F32 || t == LA_BF16; }

int64_t dtype_bytes(la_dtype t) { return t == LA_F64 ? 8 : t == LA_F32 ? 4 : 2; }

// io bf16/f32 carry an f32 state, f64 io an f64 state.
bool valid_pair(la_dtype io, la_dtype st)
{
    if (!known_dtype(io) || !known_dtype(st))
        return false;
    return io == LA_F64 ? st == LA_F64 : st == LA_F32;
}

// a*b with an overflow check against INT64_MAX / 16 (so byte counts stay representable).
bool mul_ok(int64_t a, int64_t b, int64_t *out)
{
    const int64_t lim = INT64_MAX / 16;
    if (a < 0 || b < 0 || (a != 0 && b > lim / a))
        return false;
    *out = a * b;
    return true;
}

bool prod_ok(std::initializer_list<int64_t> xs, int64_t *out)
{
    int64_t p = 1;
    for (int64_t x : xs)
        if (!mul_ok(p, x, &p))
            return false;
    *out = p;
    return true;
}

struct Range {
    const void *p;
    int64_t bytes;
};

bool overlap(Range a, Range b)
{
    if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0)
        return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + (uintptr_t)b.bytes && b0 < a0 + (uintptr_t)a.bytes;
}

// outputs must not overlap inputs or each other
bool any_alias(std::initializer_list<Range> outs, std::initializer_list<Range> ins)
{
    for (auto o = outs.begin(); o != outs.end(); ++o) {
        for (const Range &i : ins)
            if (overlap(*o, i))
                return true;
        for (auto o2 = o + 1; o2 != outs.end(); ++o2)
            if (overlap(*o, *o2))
                return true;
    }
    return false;
}

bool eps_ok(double eps) { return isfinite(eps) && eps >= 0.0; }

bool phi_ok(la_feature_map phi)
{
    return phi == LA_PHI_ELU1 || phi == LA_PHI_RELU1 || phi == LA_PHI_RELU_EPS || phi == LA_PHI_SIGMOID_EPS;
}

la_status launched(hipError_t e) { return e == hipSuccess ? LA_OK : LA_ERR_LAUNCH; }

// Scalar checks shared by la_prefill_chunked and la_prefill_variant.
la_status check_prefill_scalars(la_dtype io, int32_t d, int32_t dv, int32_t chunk, la_dtype st)
{
    if (d < 1 || dv < 1)
        return LA_ERR_SHAPE;
    if (!valid_pair(io, st))
        return LA_ERR_DTYPE;
    if (chunk < 1)
        return LA_ERR_CHUNK;
    if (d > LA_MAX_WIDTH || dv > LA_MAX_WIDTH || chunk > LA_MAX_CHUNK)
        return LA_ERR_UNSUPPORTED;
    return LA_OK;
}

// Checks shared by the softmax decode entry points; *need receives the scratch bytes.
la_status check_softmax(const void *q, const void *k, const void *v, la_dtype io_dtype, int64_t n_heads, int32_t d,
                        int32_t dv, int64_t pos, int64_t capacity, void *K_cache, void *V_cache, double scale,
                        void *y, int64_t *need)
{
    if (!q || !k || !v || !K_cache || !V_cache || !y)
        return LA_ERR_NULL;
    if (n_heads < 1 || d < 1 || dv < 1 || pos < 0 || capacity <= pos || n_heads > INT32_MAX)
        return LA_ERR_SHAPE;
    if (!known_dtype(io_dtype))
        return LA_ERR_DTYPE;
    if (d > LA_MAX_WIDTH || dv > LA_MAX_WIDTH)
        return LA_ERR_UNSUPPORTED;
    if (!isfinite(scale))
        return LA_ERR_SCALE;
    int64_t qk, vy, kc, vc;
    const int64_t ei = dtype_bytes(io_dtype);
    if (!prod_ok({n_heads, d, ei}, &qk) || !prod_ok({n_heads, dv, ei}, &vy) ||
        !prod_ok({n_heads, capacity, d, ei}, &kc) || !prod_ok({n_heads, capacity, dv, ei}, &vc) ||
        la::softmax_decode_splits(pos + 1) > INT32_MAX)
        return LA_ERR_SHAPE;
    *need = la_softmax_decode_workspace_bytes(io_dtype, n_heads, pos + 1, dv);
    if (*need < 0)
        return LA_ERR_SHAPE;
    if (any_alias({{K_cache, kc}, {V_cache, vc}, {y, vy}}, {{q, qk}, {k, qk}, {v, vy}}))
        return LA_ERR_ALIAS;
    return LA_OK;
}

// The caller's workspace must not overlap the caches, y or the inputs.
bool softmax_outputs_alias(const void *q, const void *k, const void *v, la_dtype io_dtype, int64_t n_heads, int32_t d,
                           int32_t dv, int64_t capacity, void *K_cache, void *V_cache, void *y, Range ws)
{
    const int64_t ei = dtype_bytes(io_dtype);
    const int64_t qk = n_heads * d * ei, vy = n_heads * dv * ei;
    const int64_t kc = n_heads * capacity * d * ei, vc = n_heads * capacity * dv * ei;
    return any_alias({ws}, {{q, qk}, {k, qk}, {v, vy}, {K_cache, kc}, {V_cache, vc}, {y, vy}});
}

}  // namespace

extern "C" {

const char *la_status_str(la_status s)
{
    switch (s) {
    case LA_OK:
        return "ok";
    case LA_ERR_NULL:
        return "a required pointer is NULL";
    case LA_ERR_SHAPE:
        return "a size is < 1 or too large";
    case LA_ERR_DTYPE:
        return "unknown dtype or io/state dtype pairing not allowed";
    case LA_ERR_EPS:
        return "eps must be finite and >= 0";
    case LA_ERR_CHUNK:
        return "chunk must be >= 1";
    case LA_ERR_UNSUPPORTED:
        return "no kernel for this request (d, dv and chunk must be <= 128)";
    case LA_ERR_LAUNCH:
        return "the HIP runtime refused a kernel launch";
    case LA_ERR_ALIAS:
        return "an output buffer overlaps an input or another output";
    case LA_ERR_PHI:
        return "unknown feature map";
    case LA_ERR_WORKSPACE:
        return "workspace missing or smaller than la_softmax_decode_workspace_bytes (static variant: the call "
               "needs more than LA_SOFTMAX_STATIC_WORKSPACE_BYTES)";
    case LA_ERR_SCALE:
        return "scale must be finite";
    }
    return "unknown status";
}

la_status la_state_init(void *S, void *z, int64_t n_states, int32_t r, int32_t dv, la_dtype state_dtype,
                        hipStream_t stream)
{
    if (!S || !z)
        return LA_ERR_NULL;
    if (n_states < 1 || r < 1 || dv < 1)
        return LA_ERR_SHAPE;
    if (state_dtype != LA_F32 && state_dtype != LA_F64)
        return LA_ERR_DTYPE;
    const int64_t es = dtype_bytes(state_dtype);
    int64_t sb, zb;
    if (!prod_ok({n_states, r, dv, es}, &sb) || !prod_ok({n_states, r, es}, &zb))
        return LA_ERR_SHAPE;
    if (overlap({S, sb}, {z, zb}))
        return LA_ERR_ALIAS;
    (void)hipGetLastError();
    return launched(la::launch_state_init(S, z, n_states, r, dv, state_dtype, stream));
}

int32_t la_prefill_variant(la_dtype io_dtype, int32_t d, int32_t dv, int32_t chunk, int32_t gated,
                           la_dtype state_dtype)
{
    (void)gated;
    if (check_prefill_scalars(io_dtype, d, dv, chunk, state_dtype) != LA_OK)
        return -1;
    if (la::mfma_prefill_supported(io_dtype, d, dv, chunk))
        return 1;
    return la::mfma_f32_prefill_supported(io_dtype, d, dv, chunk) ? 2 : 0;
}

int64_t la_prefill_segments(la_dtype io_dtype, int32_t d, int64_t n_heads, int64_t T, int32_t chunk,
                            int64_t *seg_len)
{
    if (!seg_len || n_heads < 1 || T < 1)
        return -1;
    if (!la::mfma_prefill_supported(io_dtype, d, d, chunk) && !la::mfma_f32_prefill_supported(io_dtype, d, d, chunk))
        return -1;
    int64_t nseg, len;
    if (!la::plan_segments(n_heads, T, chunk, d * dtype_bytes(io_dtype), la::segment_slot_bytes(d), &nseg, &len))
        return 0;
    *seg_len = len;
    return nseg;
}

int64_t la_prefill_segment_slot_bytes(int32_t d)
{
    return d == 64 || d == 128 ? la::segment_slot_bytes(d) : -1;
}

la_status la_prefill_chunked_fm(const void *Q, const void *K, const void *V, const void *alpha, la_dtype io_dtype,
                                int64_t B, int64_t H, int64_t T, int32_t d, int32_t dv, double eps, int32_t chunk,
                                void *Y, void *S, void *z, la_dtype state_dtype, la_feature_map phi,
                                hipStream_t stream)
{
    if (!Q || !K || !V || !Y || !S || !z)
        return LA_ERR_NULL;
    if (B < 1 || H < 1 || T < 1 || d < 1 || dv < 1)
        return LA_ERR_SHAPE;
    if (!known_dtype(io_dtype) || !known_dtype(state_dtype) || !valid_pair(io_dtype, state_dtype))
        return LA_ERR_DTYPE;
    if (!eps_ok(eps))
        return LA_ERR_EPS;
    la_status st = check_prefill_scalars(io_dtype, d, dv, chunk, state_dtype);
    if (st != LA_OK)
        return st;
    int64_t heads, qk, vy, sb, zb, ab;
    const int64_t ei = dtype_bytes(io_dtype), es = dtype_bytes(state_dtype);
    if (!mul_ok(B, H, &heads) || heads > INT32_MAX || !prod_ok({heads, T, d, ei}, &qk) ||
        !prod_ok({heads, T, dv, ei}, &vy) || !prod_ok({heads, d, dv, es}, &sb) || !prod_ok({heads, d, es}, &zb) ||
        !prod_ok({heads, T, es}, &ab))
        return LA_ERR_SHAPE;
    if (any_alias({{Y, vy}, {S, sb}, {z, zb}}, {{Q, qk}, {K, qk}, {V, vy}, {alpha, alpha ? ab : 0}}))
        return LA_ERR_ALIAS;
    if (!phi_ok(phi))
        return LA_ERR_PHI;

    la::PrefillArgs a{Q, K, V, alpha, heads, T, d, dv, eps, chunk, Y, S, z, phi};
    (void)hipGetLastError();
    if (la::mfma_prefill_supported(io_dtype, d, dv, chunk))
        return launched(la::launch_prefill_mfma_bf16(a, stream));
    if (la::mfma_f32_prefill_supported(io_dtype, d, dv, chunk))
        return launched(la::launch_prefill_mfma_f32(a, io_dtype, stream));
    return launched(la::launch_prefill_general(a, io_dtype, stream));
}

la_status la_prefill_chunked(const void *Q, const void *K, const void *V, const void *alpha, la_dtype io_dtype,
                             int64_t B, int64_t H, int64_t T, int32_t d, int32_t dv, double eps, int32_t chunk,
                             void *Y, void *S, void *z, la_dtype state_dtype, hipStream_t stream)
{
    return la_prefill_chunked_fm(Q, K, V, alpha, io_dtype, B, H, T, d, dv, eps, chunk, Y, S, z, state_dtype,
                                 LA_PHI_ELU1, stream);
}

la_status la_prefill_noncausal(const void *Q, const void *K, const void *V, la_dtype io_dtype, int64_t B, int64_t H,
                               int64_t T, int32_t d, int32_t dv, double eps, void *Y, void *S, void *z,
                               la_dtype state_dtype, la_feature_map phi, hipStream_t stream)
{
    if (!Q || !K || !V || !Y || !S || !z)
        return LA_ERR_NULL;
    if (B < 1 || H < 1 || T < 1 || d < 1 || dv < 1)
        return LA_ERR_SHAPE;
    if (!valid_pair(io_dtype, state_dtype))
        return LA_ERR_DTYPE;
    if (!eps_ok(eps))
        return LA_ERR_EPS;
    if (d > LA_MAX_WIDTH || dv > LA_MAX_WIDTH)
        return LA_ERR_UNSUPPORTED;
    int64_t heads, qk, vy, sb, zb;
    const int64_t ei = dtype_bytes(io_dtype), es = dtype_bytes(state_dtype);
    if (!mul_ok(B, H, &heads) || heads > INT32_MAX || !prod_ok({heads, T, d, ei}, &qk) ||
        !prod_ok({heads, T, dv, ei}, &vy) || !prod_ok({heads, d, dv, es}, &sb) || !prod_ok({heads, d, es}, &zb))
        return LA_ERR_SHAPE;
    if (any_alias({{Y, vy}, {S, sb}, {z, zb}}, {{Q, qk}, {K, qk}, {V, vy}}))
        return LA_ERR_ALIAS;
    if (!phi_ok(phi))
        return LA_ERR_PHI;

    la::PrefillArgs a{Q, K, V, nullptr, heads, T, d, dv, eps, 0, Y, S, z, phi};
    (void)hipGetLastError();
    if (la::mfma_noncausal_supported(io_dtype, d, dv))
        return launched(la::launch_noncausal_mfma_bf16(a, stream));
    return launched(la::launch_noncausal_general(a, io_dtype, stream));
}

la_status la_decode_step_fm(const void *q, const void *k, const void *v, const void *alpha, la_dtype io_dtype,
                            int64_t n_states, int32_t d, int32_t dv, double eps, void *y, void *S, void *z,
                            la_dtype state_dtype, la_feature_map phi, hipStream_t stream)
{
    if (!q || !k || !v || !y || !S || !z)
        return LA_ERR_NULL;
    if (n_states < 1 || d < 1 || dv < 1 || n_states > INT32_MAX)
        return LA_ERR_SHAPE;
    if (!valid_pair(io_dtype, state_dtype))
        return LA_ERR_DTYPE;
    if (!eps_ok(eps))
        return LA_ERR_EPS;
    if (d > LA_MAX_WIDTH || dv > LA_MAX_WIDTH)
        return LA_ERR_UNSUPPORTED;
    int64_t qk, vy, sb, zb, ab;
    const int64_t ei = dtype_bytes(io_dtype), es = dtype_bytes(state_dtype);
    if (!prod_ok({n_states, d, ei}, &qk) || !prod_ok({n_states, dv, ei}, &vy) ||
        !prod_ok({n_states, d, dv, es}, &sb) || !prod_ok({n_states, d, es}, &zb) || !prod_ok({n_states, es}, &ab))
        return LA_ERR_SHAPE;
    if (any_alias({{y, vy}, {S, sb}, {z, zb}}, {{q, qk}, {k, qk}, {v, vy}, {alpha, alpha ? ab : 0}}))
        return LA_ERR_ALIAS;
    if (!phi_ok(phi))
        return LA_ERR_PHI;

    la::DecodeArgs a{q, k, v, alpha, n_states, d, dv, eps, y, S, z, phi};
    (void)hipGetLastError();
    return launched(la::launch_decode(a, io_dtype, stream));
}

la_status la_decode_step(const void *q, const void *k, const void *v, const void *alpha, la_dtype io_dtype,
                         int64_t n_states, int32_t d, int32_t dv, double eps, void *y, void *S, void *z,
                         la_dtype state_dtype, hipStream_t stream)
{
    return la_decode_step_fm(q, k, v, alpha, io_dtype, n_states, d, dv, eps, y, S, z, state_dtype, LA_PHI_ELU1,
                             stream);
}

la_status la_delta_decode_step(const void *q, const void *k, const void *v, const void *beta, la_dtype io_dtype,
                               int64_t n_states, int32_t d, int32_t dv, void *y, void *S, la_dtype state_dtype,
                               hipStream_t stream)
{
    if (!q || !k || !v || !beta || !y || !S)
        return LA_ERR_NULL;
    if (n_states < 1 || d < 1 || dv < 1 || n_states > INT32_MAX)
        return LA_ERR_SHAPE;
    if (!valid_pair(io_dtype, state_dtype))
        return LA_ERR_DTYPE;
    if (d > LA_MAX_WIDTH || dv > LA_MAX_WIDTH)
        return LA_ERR_UNSUPPORTED;
    int64_t qk, vy, sb, bb;
    const int64_t ei = dtype_bytes(io_dtype), es = dtype_bytes(state_dtype);
    if (!prod_ok({n_states, d, ei}, &qk) || !prod_ok({n_states, dv, ei}, &vy) ||
        !prod_ok({n_states, d, dv, es}, &sb) || !prod_ok({n_states, es}, &bb))
        return LA_ERR_SHAPE;
    if (any_alias({{y, vy}, {S, sb}}, {{q, qk}, {k, qk}, {v, vy}, {beta, bb}}))
        return LA_ERR_ALIAS;

    la::DeltaArgs a{q, k, v, beta, n_states, d, dv, y, S};
    (void)hipGetLastError();
    return launched(la::launch_delta_decode(a, io_dtype, stream));
}

int64_t la_softmax_decode_workspace_bytes(la_dtype io_dtype, int64_t n_heads, int64_t L, int32_t dv)
{
    if (!known_dtype(io_dtype) || n_heads < 1 || L < 1 || dv < 1 || dv > LA_MAX_WIDTH)
        return -1;
    const int64_t splits = la::softmax_decode_splits(L);
    if (splits == 1)
        return 0;
    int64_t b;
    if (!prod_ok({n_heads, splits, 2 + (int64_t)dv, io_dtype == LA_F64 ? 8 : 4}, &b))
        return -1;
    return b;
}

la_status la_softmax_decode_step(const void *q, const void *k, const void *v, la_dtype io_dtype, int64_t n_heads,
                                 int32_t d, int32_t dv, int64_t pos, int64_t capacity, void *K_cache, void *V_cache,
                                 double scale, void *y, void *workspace, int64_t workspace_bytes, hipStream_t stream)
{
    int64_t need = 0;
    la_status st = check_softmax(q, k, v, io_dtype, n_heads, d, dv, pos, capacity, K_cache, V_cache, scale, y, &need);
    if (st != LA_OK)
        return st;
    if (need > 0 && (!workspace || workspace_bytes < need))
        return LA_ERR_WORKSPACE;
    if (need > 0 && softmax_outputs_alias(q, k, v, io_dtype, n_heads, d, dv, capacity, K_cache, V_cache, y,
                                          {workspace, need}))
        return LA_ERR_ALIAS;

    la::SoftmaxDecodeArgs a{q, k, v, n_heads, d, dv, pos, capacity, K_cache, V_cache, scale, y, workspace};
    (void)hipGetLastError();
    return launched(la::launch_softmax_decode(a, io_dtype, stream));
}

la_status la_softmax_decode_step_static(const void *q, const void *k, const void *v, la_dtype io_dtype,
                                        int64_t n_heads, int32_t d, int32_t dv, int64_t pos, int64_t capacity,
                                        void *K_cache, void *V_cache, double scale, void *y, hipStream_t stream)
{
    int64_t need = 0;
    la_status st = check_softmax(q, k, v, io_dtype, n_heads, d, dv, pos, capacity, K_cache, V_cache, scale, y, &need);
    if (st != LA_OK)
        return st;
    if (need > LA_SOFTMAX_STATIC_WORKSPACE_BYTES)
        return LA_ERR_WORKSPACE;
    void *scratch = nullptr;
    if (need > 0 && la::softmax_static_workspace(&scratch) != hipSuccess)
        return LA_ERR_LAUNCH;

    la::SoftmaxDecodeArgs a{q, k, v, n_heads, d, dv, pos, capacity, K_cache, V_cache, scale, y, scratch};
    (void)hipGetLastError();
    return launched(la::launch_softmax_decode(a, io_dtype, stream));
}

}  // extern "C"
