/*
 * linattn.h -- C ABI of the causal kernelized linear-attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (page "Linear attention：把历史写进状态", hs-black.github.io):
 *   features      q~ = phi(q), k~ = phi(k), phi(x) = ELU(x)+1 = x+1 (x > 0), exp(x) (x <= 0)
 *                 (section "关键改写：让求和先发生")
 *   state write   S_t = alpha_t * S_{t-1} + k~_t v_t^T     S is r x dv, feature-major
 *                 z_t = alpha_t * z_{t-1} + k~_t           z is r
 *                 (sections "公式里的每个维度" and "加一个门"; alpha == 1 when ungated)
 *   read-out      y_t = (q~_t^T S_t) / (q~_t^T z_t + eps)  -- the state is written
 *                 first, so y_t includes token t; eps is added to the denominator,
 *                 never max(den, eps) (sections "每来一个 token…" and "ε 是数值保护")
 * Prefill evaluates this over a whole sequence chunk by chunk (section "一个 chunk
 * 的输出由两部分组成"); decode applies one step per call (section "训练时，状态更新
 * 也能按块并行": the token recurrence is the decode form).  Here the feature width r
 * equals the key width d, since phi is elementwise.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers to dense, contiguous, row-major
 *     arrays owned by the caller.  The library allocates nothing, keeps nothing
 *     between calls and never synchronises: work is enqueued on `stream`
 *     (a hipStream_t; NULL means the default stream) and the caller synchronises.
 *     (One exception: la_softmax_decode_step_static keeps its scratch in a fixed
 *     device array of the library's own, see there.)
 *   - Arguments are checked on the host before anything is enqueued.  On any
 *     status other than LA_OK nothing has been launched and no output has been
 *     written.  Faults inside a kernel surface at the caller's next
 *     synchronisation.
 *   - Outputs must not overlap inputs or each other (LA_ERR_ALIAS).
 *   - dtypes: the io dtype (q, k, v and the output y) is LA_BF16, LA_F32 or
 *     LA_F64.  The state dtype (S, z and the gate alpha) is LA_F32 for bf16 and
 *     f32 io, LA_F64 for f64 io; any other pairing is LA_ERR_DTYPE.
 *   - alpha, when given, must lie in [0, 1] (section "加一个门"); alpha = 0 resets
 *     the state exactly.  Values outside [0, 1] are not checked and give
 *     unspecified results.
 *   - Calls are thread-safe; calls that share output buffers on concurrent
 *     streams race.
 */
#ifndef LINATTN_H
#define LINATTN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum la_status {
    LA_OK = 0,
    LA_ERR_NULL = 1,        /* a required pointer is NULL */
    LA_ERR_SHAPE = 2,       /* a size is < 1, or too large to index */
    LA_ERR_DTYPE = 3,       /* unknown dtype, or an io/state pairing that is not allowed */
    LA_ERR_EPS = 4,         /* eps is negative, NaN or infinite (0 is allowed) */
    LA_ERR_CHUNK = 5,       /* chunk < 1 */
    LA_ERR_UNSUPPORTED = 6, /* valid request with no kernel: d or dv > 128, chunk > 128 */
    LA_ERR_LAUNCH = 7,      /* the HIP runtime refused a launch (or a set-up call) */
    LA_ERR_ALIAS = 8,       /* an output overlaps an input or another output */
    LA_ERR_PHI = 9,         /* unknown feature map */
    LA_ERR_WORKSPACE = 10,  /* workspace missing or too small */
    LA_ERR_SCALE = 11       /* scale is NaN or infinite */
} la_status;

typedef enum la_dtype {
    LA_F64 = 0,
    LA_F32 = 1,
    LA_BF16 = 2
} la_dtype;

/*
 * Feature maps phi, applied elementwise to queries and keys.  Every entry point without
 * an la_feature_map argument uses LA_PHI_ELU1.
 *   LA_PHI_ELU1         ELU(x) + 1 = x + 1 (x > 0), exp(x) (x <= 0)     (hs-black.github.io
 *                       page, section "关键改写：让求和先发生")
 *   LA_PHI_RELU1        max(x, 0) + 1       (datawhalechina chapter "Linear Attention and
 *                       Recurrent State", Step 4: its positive feature map)
 *   LA_PHI_RELU_EPS     max(x, 0) + 1e-5    (page "线性注意力架构演进", ai-master.cc: the
 *   LA_PHI_SIGMOID_EPS  sigmoid(x) + 1e-5    feature-map switch of its pluggable module)
 * In exact arithmetic all four are strictly positive for finite x.  In the arithmetic type
 * (fp32 for bf16 and f32 io, fp64 for f64 io) ELU(x) + 1 = exp(x) underflows to 0 for x
 * below about -87 (fp32; -708 in fp64), while the other three never fall below 1e-5.  With
 * eps = 0, a query whose every feature maps to 0 then reads 0 / 0 = NaN where exact
 * arithmetic gives a finite value; with eps > 0 its output is 0, within rounding of the
 * exact value.  Inputs that can reach that range should use eps > 0.
 */
typedef enum la_feature_map {
    LA_PHI_ELU1 = 0,
    LA_PHI_RELU1 = 1,
    LA_PHI_RELU_EPS = 2,
    LA_PHI_SIGMOID_EPS = 3
} la_feature_map;

/* Largest feature width d (= r), value width dv and chunk any kernel handles. */
#define LA_MAX_WIDTH 128
#define LA_MAX_CHUNK 128

/*
 * la_state_init -- S_0 = 0, z_0 = 0 for n_states independent states
 * (section "每来一个 token，更新两个累加器": both accumulators start at zero).
 *   S  [n_states, r, dv]  state_dtype, written
 *   z  [n_states, r]      state_dtype, written
 * Errors: LA_ERR_NULL, LA_ERR_SHAPE (n_states, r or dv < 1), LA_ERR_DTYPE
 * (state_dtype not LA_F32/LA_F64), LA_ERR_ALIAS (S and z overlap), LA_ERR_LAUNCH.
 * Enqueues a fill kernel (not a memset node), so it may be captured in a graph.
 */
la_status la_state_init(void *S, void *z, int64_t n_states, int32_t r, int32_t dv,
                        la_dtype state_dtype, hipStream_t stream);

/*
 * la_prefill_chunked -- run B*H independent sequences of T tokens through the
 * recurrence, continuing from the state in S and z, and return every output
 * and the final state.  The work is organised chunk by chunk (section "一个 chunk
 * 的输出由两部分组成"): for each chunk, the inter-chunk read Q~c S_prev and
 * Q~c z_prev, the intra-chunk masked (Q~c K~c^T . M) Vc and its row sums, and the
 * state write S_next = S_prev + K~c^T Vc, z_next = z_prev + sum of K~c rows; with a
 * gate, the cumulative gate products inside the chunk weight the mask, the read
 * of S_prev and the write.  `chunk` changes only the rounding, never the result.
 *   Q, K   [B, H, T, d]   io_dtype, read
 *   V      [B, H, T, dv]  io_dtype, read
 *   alpha  [B, H, T]      state_dtype, read; NULL = ungated (alpha == 1)
 *   Y      [B, H, T, dv]  io_dtype, written
 *   S      [B, H, d, dv]  state_dtype, read (state before token 0) and overwritten
 *                         with the state after token T-1
 *   z      [B, H, d]      state_dtype, same as S
 *   eps    >= 0, added to every denominator
 *   chunk  tokens per chunk, 1..128 (the last chunk of a sequence may be shorter)
 * Kernels (la_prefill_variant tells which a request takes):
 *   - bf16 io, d = dv = 128, chunk 64 or 128: bf16 MFMA products with fp32
 *     accumulation and fp32 state;
 *   - chunk 64 with f32 io at d = dv = 64 or 128, or bf16 io at d = dv = 64: fp32 MFMA
 *     products on fp32 operands (bf16 inputs widen exactly), fp32 state;
 *   - every other valid request, and the two above when Q, K, V or Y is not aligned as
 *     la_prefill_variant states: a general kernel that computes in the state dtype.  It
 *     uses no matrix instructions and is about two orders of magnitude slower (bf16,
 *     B=4, H=16, T=4096, d = dv = 128: about 12 ms per call at chunk 32 against 0.09 ms
 *     at chunk 64 on an MI355X), so callers free to pick the chunk should pick 64.
 * The MFMA paths split long sequences into segments (la_prefill_segments) and keep
 * each segment's entering state (la_prefill_segment_slot_bytes(d) bytes) in that
 * segment's rows of Y until they are overwritten with its outputs, so Y is working
 * memory for the duration of the call: its contents are defined only once the call's
 * work on `stream` has finished.  No other memory is used.
 * Errors: LA_ERR_NULL, LA_ERR_SHAPE (B, H, T, d, dv < 1), LA_ERR_DTYPE, LA_ERR_EPS,
 * LA_ERR_CHUNK, LA_ERR_UNSUPPORTED (d or dv > 128, chunk > 128), LA_ERR_ALIAS,
 * LA_ERR_LAUNCH.
 */
la_status la_prefill_chunked(const void *Q, const void *K, const void *V, const void *alpha,
                             la_dtype io_dtype, int64_t B, int64_t H, int64_t T,
                             int32_t d, int32_t dv, double eps, int32_t chunk,
                             void *Y, void *S, void *z, la_dtype state_dtype,
                             hipStream_t stream);

/*
 * la_decode_step -- one token for each of n_states independent states, updated in
 * place: S <- alpha*S + k~ v^T, z <- alpha*z + k~, then y = q~^T S / (q~^T z + eps)
 * (the minimal per-token loop of section "最小递推里，每一行都有张量意义", gated as
 * in section "加一个门").  A state can be a (request, layer, head) slot of a batch.
 *   q, k   [n_states, d]      io_dtype, read
 *   v      [n_states, dv]     io_dtype, read
 *   alpha  [n_states]         state_dtype, read; NULL = ungated
 *   y      [n_states, dv]     io_dtype, written
 *   S      [n_states, d, dv]  state_dtype, read and written in place
 *   z      [n_states, d]      state_dtype, read and written in place
 * Errors: LA_ERR_NULL, LA_ERR_SHAPE, LA_ERR_DTYPE, LA_ERR_EPS,
 * LA_ERR_UNSUPPORTED (d or dv > 128), LA_ERR_ALIAS, LA_ERR_LAUNCH.
 */
la_status la_decode_step(const void *q, const void *k, const void *v, const void *alpha,
                         la_dtype io_dtype, int64_t n_states, int32_t d, int32_t dv,
                         double eps, void *y, void *S, void *z, la_dtype state_dtype,
                         hipStream_t stream);

/*
 * la_delta_decode_step -- one delta-rule step for each of n_states independent
 * memories, updated in place (the fast-weight memory of section "Delta rule：先读旧答案，
 * 再写误差", written as S' = S + beta k (v - k^T S) under "key 的范数决定了纠错力度"):
 *   p = S^T k,  e = v - p,  S <- S + beta k e^T,  then y = S^T q.
 * The memory has no normaliser and q, k enter as given (no feature map): the page's
 * delta examples use raw keys, and normalised keys keep beta's meaning stable (a step
 * contracts the error along k by 1 - beta |k|^2).
 *   q, k   [n_states, d]      io_dtype, read
 *   v      [n_states, dv]     io_dtype, read
 *   beta   [n_states]         state_dtype, read (required)
 *   y      [n_states, dv]     io_dtype, written
 *   S      [n_states, d, dv]  state_dtype, read and written in place
 * Same dtype pairs as la_decode_step.  Errors: LA_ERR_NULL, LA_ERR_SHAPE, LA_ERR_DTYPE,
 * LA_ERR_UNSUPPORTED (d or dv > 128), LA_ERR_ALIAS, LA_ERR_LAUNCH.
 */
la_status la_delta_decode_step(const void *q, const void *k, const void *v, const void *beta,
                               la_dtype io_dtype, int64_t n_states, int32_t d, int32_t dv,
                               void *y, void *S, la_dtype state_dtype, hipStream_t stream);

/*
 * la_prefill_chunked_fm, la_decode_step_fm -- la_prefill_chunked and la_decode_step with
 * the feature map chosen by `phi` (same arguments, then `phi` before the stream).
 * An unknown `phi` is LA_ERR_PHI; everything else is as for the call without _fm.
 */
la_status la_prefill_chunked_fm(const void *Q, const void *K, const void *V, const void *alpha,
                                la_dtype io_dtype, int64_t B, int64_t H, int64_t T,
                                int32_t d, int32_t dv, double eps, int32_t chunk,
                                void *Y, void *S, void *z, la_dtype state_dtype,
                                la_feature_map phi, hipStream_t stream);

la_status la_decode_step_fm(const void *q, const void *k, const void *v, const void *alpha,
                            la_dtype io_dtype, int64_t n_states, int32_t d, int32_t dv,
                            double eps, void *y, void *S, void *z, la_dtype state_dtype,
                            la_feature_map phi, hipStream_t stream);

/*
 * la_prefill_noncausal -- the non-causal form: every token of a sequence is written into
 * the state first, then every query reads that full state (page "线性注意力架构演进",
 * ai-master.cc: its linear-attention module's parallel form and its pluggable module
 * form K~^T V and the key sum once and read each query against them; eps is added to
 * the denominator as in the causal read-out):
 *   S_out = S_in + sum_t k~_t v_t^T,   z_out = z_in + sum_t k~_t
 *   y_t   = (q~_t^T S_out) / (q~_t^T z_out + eps)        for every t
 * With S_in = z_in = 0 (la_state_init) this is unmasked attention with weights
 * q~_t . k~_i; a nonzero incoming state is context that every query also sees.  There
 * is no gate: a decay has no direction in this form.
 *   Q, K   [B, H, T, d]   io_dtype, read
 *   V      [B, H, T, dv]  io_dtype, read
 *   Y      [B, H, T, dv]  io_dtype, written
 *   S      [B, H, d, dv]  state_dtype, read (S_in) and overwritten with S_out
 *   z      [B, H, d]      state_dtype, same as S
 * bf16 io with d = dv = 128 runs on bf16 MFMA (fp32 accumulation, the state rounded
 * to bf16 for the read as in the causal inter-chunk read); other valid requests run a
 * general kernel in the state dtype.
 * Errors: LA_ERR_NULL, LA_ERR_SHAPE, LA_ERR_DTYPE, LA_ERR_EPS, LA_ERR_UNSUPPORTED
 * (d or dv > 128), LA_ERR_ALIAS, LA_ERR_PHI, LA_ERR_LAUNCH.
 */
la_status la_prefill_noncausal(const void *Q, const void *K, const void *V, la_dtype io_dtype,
                               int64_t B, int64_t H, int64_t T, int32_t d, int32_t dv,
                               double eps, void *Y, void *S, void *z, la_dtype state_dtype,
                               la_feature_map phi, hipStream_t stream);

/*
 * la_softmax_decode_step -- one decode step of softmax attention over an explicit K/V
 * history, the comparator that the datawhalechina chapter "Linear Attention and
 * Recurrent State" (Step 5) sets against the fixed recurrent state.  The row is the one
 * of section "先看普通 attention 在读什么" of the hs-black.github.io page: every history key
 * is scored against the query, the scores are normalised by softmax and the values are
 * summed with those weights.  For each head h:
 *   K_cache[h][pos] = k[h], V_cache[h][pos] = v[h]   (the new token joins the history)
 *   y[h] = sum_{i=0..pos} w_i V_cache[h][i],  w = softmax_i(scale * q[h] . K_cache[h][i])
 *   q, k      [n_heads, d]            io_dtype, read
 *   v         [n_heads, dv]           io_dtype, read
 *   K_cache   [n_heads, capacity, d]  io_dtype, rows 0..pos-1 read, row pos written
 *   V_cache   [n_heads, capacity, dv] io_dtype, same
 *   y         [n_heads, dv]           io_dtype, written
 *   scale     any finite value (1/sqrt(d) for the page's row)
 *   workspace device buffer of at least la_softmax_decode_workspace_bytes(io_dtype,
 *             n_heads, pos + 1, dv) bytes (NULL allowed when that is 0), overwritten
 * Arithmetic in fp32 (fp64 for f64 io).  Errors: LA_ERR_NULL, LA_ERR_SHAPE (sizes < 1,
 * pos < 0 or pos >= capacity), LA_ERR_DTYPE, LA_ERR_UNSUPPORTED (d or dv > 128),
 * LA_ERR_SCALE, LA_ERR_WORKSPACE, LA_ERR_ALIAS, LA_ERR_LAUNCH.
 */
la_status la_softmax_decode_step(const void *q, const void *k, const void *v, la_dtype io_dtype,
                                 int64_t n_heads, int32_t d, int32_t dv, int64_t pos, int64_t capacity,
                                 void *K_cache, void *V_cache, double scale, void *y,
                                 void *workspace, int64_t workspace_bytes, hipStream_t stream);

/* Workspace bytes la_softmax_decode_step needs for a history of L rows (L = pos + 1);
 * 0 when none is needed, -1 for invalid arguments. */
int64_t la_softmax_decode_workspace_bytes(la_dtype io_dtype, int64_t n_heads, int64_t L, int32_t dv);

/*
 * la_softmax_decode_step_static -- la_softmax_decode_step with no workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It runs the same kernels on the same arguments
 * (minus workspace and workspace_bytes) and gives bitwise the same y and caches.
 *   Scratch: the per-piece partials live in a device array of the library's own,
 *   LA_SOFTMAX_STATIC_WORKSPACE_BYTES bytes on each GPU the call runs on, set up on the
 *   first call on that device (with it current) and held until the process ends.  The
 *   call allocates nothing (no hipMalloc, hipFree or allocating library routine).  Every
 *   entry of the array that a call reads was written earlier in the same call, so
 *   nothing needs clearing between calls.
 *   Concurrency: every call on one GPU shares that GPU's array.  Calls whose execution
 *   overlaps on one GPU (different streams without ordering between them) race and may
 *   return wrong results; serialise them (one stream, or events).
 * Errors: those of la_softmax_decode_step, with LA_ERR_WORKSPACE when
 * la_softmax_decode_workspace_bytes(io_dtype, n_heads, pos + 1, dv) exceeds
 * LA_SOFTMAX_STATIC_WORKSPACE_BYTES (nothing launched), and LA_ERR_LAUNCH when the runtime
 * does not give the array's device address on the first call on a device.
 */
#define LA_SOFTMAX_STATIC_WORKSPACE_BYTES ((int64_t)32 << 20)
la_status la_softmax_decode_step_static(const void *q, const void *k, const void *v, la_dtype io_dtype,
                                        int64_t n_heads, int32_t d, int32_t dv, int64_t pos,
                                        int64_t capacity, void *K_cache, void *V_cache, double scale,
                                        void *y, hipStream_t stream);

/* Static description of a status code; never NULL. */
const char *la_status_str(la_status status);

/*
 * Which prefill kernel a request would run, without running it:
 *   1 = bf16 MFMA chunked kernel (bf16 io, d = dv = 128, chunk 64 or 128),
 *   2 = fp32-arithmetic MFMA chunked kernel (chunk 64: f32 io at d = dv = 64 or 128, bf16 io
 *       at d = dv = 64),
 *   0 = general kernel, -1 = the request is rejected (the same checks as
 *   la_prefill_chunked on the scalar arguments).
 * Variants 1 and 2 fall back to the general kernel at run time when Q, K, V or Y is not
 * aligned to 16 bytes (8 bytes for bf16 io in variant 2).
 */
int32_t la_prefill_variant(la_dtype io_dtype, int32_t d, int32_t dv, int32_t chunk,
                           int32_t gated, la_dtype state_dtype);

/*
 * How the MFMA prefills (variants 1 and 2 of la_prefill_variant, at d = dv) cut each of
 * n_heads sequences of T tokens, without running anything: the plan la_prefill_chunked
 * uses for those requests (la_prefill_noncausal: bf16 at d = 128 and chunk 64).  Sequences
 * are cut into segments so that the (sequence, segment) workgroups give every compute
 * unit work; the state entering each segment follows from the segments before it by the
 * associative composition of gated updates (section "门控递推为什么能做并行 scan").  Returns
 * the number of segments per sequence and sets *seg_len to the length of every segment
 * but the last, which takes the rest (*seg_len = T for one segment).  Every segment but
 * the last is a whole number of chunks; with more than one segment, each segment is long
 * enough to hold, in its own rows of Y, a slot of la_prefill_segment_slot_bytes(d) bytes
 * where the state entering it is parked before its outputs overwrite those rows, and
 * every segment stays below 2^31 bytes of Q.  Returns 0 when n_heads x segments would not
 * fit one launch (the prefill then fails with LA_ERR_LAUNCH) and -1 for seg_len NULL,
 * n_heads or T < 1, or an (io_dtype, d, chunk) the MFMA prefills do not take.
 */
int64_t la_prefill_segments(la_dtype io_dtype, int32_t d, int64_t n_heads, int64_t T, int32_t chunk,
                            int64_t *seg_len);
/* Bytes of one segment's state slot at d = dv = d (S, z and the segment's gate product in
 * fp32, padded to 16 bytes): (d*d + d + 4) * 4; -1 for a width no MFMA prefill takes
 * (d other than 64 or 128). */
int64_t la_prefill_segment_slot_bytes(int32_t d);

#ifdef __cplusplus
}
#endif

#endif /* LINATTN_H */
