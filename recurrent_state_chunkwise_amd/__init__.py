"""Causal kernelized linear attention on AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of ``liblinattn.so`` (declared in
``include/linattn.h``).  It only marshals arguments: torch tensors already on
the GPU become device pointers and sizes, the current torch stream becomes the
``hipStream_t``, and status codes become exceptions (``ValueError`` for a
rejected argument, ``RuntimeError`` for a refused launch).  Every step of the
computation runs in the library's HIP kernels; there is no other path, and
the binding fails loudly when the library is missing.

The operation (page "Linear attention：把历史写进状态", hs-black.github.io):
phi = ELU+1 on queries and keys; S_t = alpha_t S_{t-1} + phi(k_t) v_t^T and
z_t = alpha_t z_{t-1} + phi(k_t); y_t = phi(q_t)^T S_t / (phi(q_t)^T z_t + eps).
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = [
    "LA_F64", "LA_F32", "LA_BF16", "LA_PHI_ELU1", "LA_PHI_RELU1", "LA_PHI_RELU_EPS", "LA_PHI_SIGMOID_EPS",
    "FEATURE_MAPS", "LaArgumentError", "LaLaunchError",
    "la_state_init", "la_prefill_chunked", "la_prefill_chunked_fm", "la_prefill_noncausal", "la_decode_step",
    "la_decode_step_fm", "la_delta_decode_step", "la_softmax_decode_step", "la_softmax_decode_workspace_bytes",
    "la_softmax_decode_step_static", "LA_SOFTMAX_STATIC_WORKSPACE_BYTES",
    "la_status_str", "la_prefill_variant", "la_prefill_segments", "la_prefill_segment_slot_bytes", "library",
    "library_path",
]

LA_F64, LA_F32, LA_BF16 = 0, 1, 2
LA_PHI_ELU1, LA_PHI_RELU1, LA_PHI_RELU_EPS, LA_PHI_SIGMOID_EPS = 0, 1, 2, 3
# feature-map names accepted by the *_fm calls and la_prefill_noncausal
FEATURE_MAPS = {"elu1": LA_PHI_ELU1, "relu1": LA_PHI_RELU1, "relu_eps": LA_PHI_RELU_EPS,
                "sigmoid_eps": LA_PHI_SIGMOID_EPS}

STATUS = {
    0: "LA_OK", 1: "LA_ERR_NULL", 2: "LA_ERR_SHAPE", 3: "LA_ERR_DTYPE", 4: "LA_ERR_EPS",
    5: "LA_ERR_CHUNK", 6: "LA_ERR_UNSUPPORTED", 7: "LA_ERR_LAUNCH", 8: "LA_ERR_ALIAS", 9: "LA_ERR_PHI",
    10: "LA_ERR_WORKSPACE", 11: "LA_ERR_SCALE",
}
LA_ERR_LAUNCH = 7
LA_SOFTMAX_STATIC_WORKSPACE_BYTES = 32 << 20  # the library's fixed scratch per GPU (linattn.h)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liblinattn.so")
_lib = None
_lock = threading.Lock()


class LaArgumentError(ValueError):
    """The library rejected an argument (nothing was launched)."""

    def __init__(self, status: int, what: str):
        super().__init__("%s (%s)" % (what, STATUS.get(status, status)))
        self.status = status


class LaLaunchError(RuntimeError):
    """The HIP runtime refused a launch."""

    def __init__(self, status: int, what: str):
        super().__init__("%s (%s)" % (what, STATUS.get(status, status)))
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def library() -> ctypes.CDLL:
    """The loaded ``liblinattn.so``; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise RuntimeError(
                    "liblinattn.so is not built (python -m recurrent_state_chunkwise_amd.build); "
                    "there is no other implementation to fall back to")
            lib = ctypes.CDLL(_LIB_PATH)
            vp, i64, i32, f64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
            lib.la_status_str.restype = ctypes.c_char_p
            lib.la_status_str.argtypes = [ctypes.c_int]
            lib.la_state_init.restype = ctypes.c_int
            lib.la_state_init.argtypes = [vp, vp, i64, i32, i32, ctypes.c_int, vp]
            lib.la_prefill_chunked.restype = ctypes.c_int
            lib.la_prefill_chunked.argtypes = [vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i32, i32, f64, i32,
                                               vp, vp, vp, ctypes.c_int, vp]
            lib.la_decode_step.restype = ctypes.c_int
            lib.la_decode_step.argtypes = [vp, vp, vp, vp, ctypes.c_int, i64, i32, i32, f64, vp, vp, vp,
                                           ctypes.c_int, vp]
            lib.la_delta_decode_step.restype = ctypes.c_int
            lib.la_delta_decode_step.argtypes = [vp, vp, vp, vp, ctypes.c_int, i64, i32, i32, vp, vp,
                                                 ctypes.c_int, vp]
            lib.la_prefill_chunked_fm.restype = ctypes.c_int
            lib.la_prefill_chunked_fm.argtypes = [vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i32, i32, f64, i32,
                                                  vp, vp, vp, ctypes.c_int, ctypes.c_int, vp]
            lib.la_decode_step_fm.restype = ctypes.c_int
            lib.la_decode_step_fm.argtypes = [vp, vp, vp, vp, ctypes.c_int, i64, i32, i32, f64, vp, vp, vp,
                                              ctypes.c_int, ctypes.c_int, vp]
            lib.la_prefill_noncausal.restype = ctypes.c_int
            lib.la_prefill_noncausal.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64, i64, i32, i32, f64, vp, vp, vp,
                                                 ctypes.c_int, ctypes.c_int, vp]
            lib.la_softmax_decode_step.restype = ctypes.c_int
            lib.la_softmax_decode_step.argtypes = [vp, vp, vp, ctypes.c_int, i64, i32, i32, i64, i64, vp, vp, f64,
                                                   vp, vp, i64, vp]
            lib.la_softmax_decode_step_static.restype = ctypes.c_int
            lib.la_softmax_decode_step_static.argtypes = [vp, vp, vp, ctypes.c_int, i64, i32, i32, i64, i64, vp, vp,
                                                          f64, vp, vp]
            lib.la_softmax_decode_workspace_bytes.restype = i64
            lib.la_softmax_decode_workspace_bytes.argtypes = [ctypes.c_int, i64, i64, i32]
            lib.la_prefill_segments.restype = i64
            lib.la_prefill_segments.argtypes = [ctypes.c_int, i32, i64, i64, i32, ctypes.POINTER(i64)]
            lib.la_prefill_segment_slot_bytes.restype = i64
            lib.la_prefill_segment_slot_bytes.argtypes = [i32]
            lib.la_prefill_variant.restype = ctypes.c_int32
            lib.la_prefill_variant.argtypes = [ctypes.c_int, i32, i32, i32, i32, ctypes.c_int]
            _lib = lib
    return _lib


def la_status_str(status: int) -> str:
    return library().la_status_str(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status == 0:
        return
    msg = "%s: %s" % (what, la_status_str(status))
    if status == LA_ERR_LAUNCH:
        raise LaLaunchError(status, msg)
    raise LaArgumentError(status, msg)


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    codes = {torch.float64: LA_F64, torch.float32: LA_F32, torch.bfloat16: LA_BF16}
    if t.dtype not in codes:
        raise ValueError("unsupported dtype %s (float64, float32 or bfloat16)" % t.dtype)
    return codes[t.dtype]


def _same_dtype(name, tensors):
    dts = {t.dtype for t in tensors if t is not None}
    if len(dts) != 1:
        raise ValueError("%s must share one dtype, got %s" % (name, sorted(map(str, dts))))


def _device_ptrs(*tensors):
    """Device pointers of contiguous GPU tensors (None -> NULL)."""
    out = []
    for t in tensors:
        if t is None:
            out.append(None)
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous (row-major)")
        out.append(ctypes.c_void_p(t.data_ptr()))
    return out


def _stream_ptr(t, stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(s.cuda_stream)


def la_state_init(S, z, stream=None) -> None:
    """S_0 = 0, z_0 = 0.  S: [..., r, dv], z: [..., r] (float32 or float64)."""
    if S.dim() < 2 or z.dim() < 1 or tuple(S.shape[:-1]) != tuple(z.shape):
        raise ValueError("S must be [..., r, dv] and z [..., r] with the same leading shape")
    r, dv = S.shape[-2], S.shape[-1]
    n = S.numel() // (r * dv) if r * dv else 0
    _same_dtype("S, z", (S, z))
    st = _dtype_code(S)
    pS, pz = _device_ptrs(S, z)
    _check(library().la_state_init(pS, pz, n, r, dv, st, _stream_ptr(S, stream)), "la_state_init")


def _phi_code(phi) -> int:
    """A feature-map name of FEATURE_MAPS or an la_feature_map code (an unknown code is
    passed through, for the library to reject)."""
    if isinstance(phi, str):
        if phi not in FEATURE_MAPS:
            raise ValueError("unknown feature map %r (one of %s)" % (phi, ", ".join(FEATURE_MAPS)))
        return FEATURE_MAPS[phi]
    return int(phi)


def _prefill_shapes(Q, K, V, Y, S, z):
    if Q.dim() != 4 or tuple(K.shape) != tuple(Q.shape):
        raise ValueError("Q and K must both be [B, H, T, d] with the same shape")
    B, H, T, d = Q.shape
    if V.dim() != 4 or tuple(V.shape[:3]) != (B, H, T):
        raise ValueError("V must be [B, H, T, dv] with Q's B, H, T")
    dv = V.shape[3]
    if tuple(Y.shape) != tuple(V.shape):
        raise ValueError("Y must have V's shape")
    if tuple(S.shape) != (B, H, d, dv) or tuple(z.shape) != (B, H, d):
        raise ValueError("S must be [B, H, d, dv] and z [B, H, d]")
    return B, H, T, d, dv


def _gated_prefill_args(Q, K, V, alpha, Y, S, z):
    """Shape and dtype checks of the causal prefill calls: (B, H, T, d, dv, io, st, ptrs)."""
    B, H, T, d, dv = _prefill_shapes(Q, K, V, Y, S, z)
    if alpha is not None and tuple(alpha.shape) != (B, H, T):
        raise ValueError("alpha must be [B, H, T]")
    _same_dtype("Q, K, V, Y", (Q, K, V, Y))
    _same_dtype("S, z, alpha", (S, z, alpha))
    return B, H, T, d, dv, _dtype_code(Q), _dtype_code(S), _device_ptrs(Q, K, V, alpha, Y, S, z)


def la_prefill_chunked_fm(Q, K, V, alpha, eps: float, chunk: int, Y, S, z, phi="elu1", stream=None) -> None:
    """:func:`la_prefill_chunked` with the feature map ``phi`` (a FEATURE_MAPS name or code)."""
    B, H, T, d, dv, io, st, ptrs = _gated_prefill_args(Q, K, V, alpha, Y, S, z)
    rc = library().la_prefill_chunked_fm(ptrs[0], ptrs[1], ptrs[2], ptrs[3], io, B, H, T, d, dv, float(eps),
                                         int(chunk), ptrs[4], ptrs[5], ptrs[6], st, _phi_code(phi),
                                         _stream_ptr(Q, stream))
    _check(rc, "la_prefill_chunked_fm")


def la_prefill_noncausal(Q, K, V, eps: float, Y, S, z, phi="elu1", stream=None) -> None:
    """Non-causal form of B*H sequences: (S, z) += the whole sequence, then every query
    reads the final state: Y_t = q~_t^T S / (q~_t^T z + eps).

    Q, K: [B, H, T, d]; V, Y: [B, H, T, dv]; S: [B, H, d, dv], z: [B, H, d] in/out.
    """
    B, H, T, d, dv = _prefill_shapes(Q, K, V, Y, S, z)
    _same_dtype("Q, K, V, Y", (Q, K, V, Y))
    _same_dtype("S, z", (S, z))
    io, st = _dtype_code(Q), _dtype_code(S)
    ptrs = _device_ptrs(Q, K, V, Y, S, z)
    rc = library().la_prefill_noncausal(ptrs[0], ptrs[1], ptrs[2], io, B, H, T, d, dv, float(eps), ptrs[3],
                                        ptrs[4], ptrs[5], st, _phi_code(phi), _stream_ptr(Q, stream))
    _check(rc, "la_prefill_noncausal")


def la_prefill_chunked(Q, K, V, alpha, eps: float, chunk: int, Y, S, z, stream=None) -> None:
    """Chunked prefill of B*H sequences, continuing from (S, z), writing Y and the final (S, z).

    Q, K: [B, H, T, d]; V, Y: [B, H, T, dv] (one io dtype); alpha: [B, H, T] or None;
    S: [B, H, d, dv], z: [B, H, d] (state dtype: float32 for bf16/f32 io, float64 for f64 io).
    """
    B, H, T, d, dv, io, st, ptrs = _gated_prefill_args(Q, K, V, alpha, Y, S, z)
    rc = library().la_prefill_chunked(ptrs[0], ptrs[1], ptrs[2], ptrs[3], io, B, H, T, d, dv, float(eps),
                                      int(chunk), ptrs[4], ptrs[5], ptrs[6], st, _stream_ptr(Q, stream))
    _check(rc, "la_prefill_chunked")


def _decode_args(q, k, v, alpha, y, S, z):
    """Shape and dtype checks of the decode calls: (N, d, dv, io, st, ptrs)."""
    if q.dim() != 2 or tuple(k.shape) != tuple(q.shape):
        raise ValueError("q and k must both be [N, d] with the same shape")
    N, d = q.shape
    if v.dim() != 2 or v.shape[0] != N:
        raise ValueError("v must be [N, dv] with q's N")
    dv = v.shape[1]
    if tuple(y.shape) != (N, dv) or tuple(S.shape) != (N, d, dv) or tuple(z.shape) != (N, d):
        raise ValueError("y must be [N, dv], S [N, d, dv] and z [N, d]")
    if alpha is not None and tuple(alpha.shape) != (N,):
        raise ValueError("alpha must be [N]")
    _same_dtype("q, k, v, y", (q, k, v, y))
    _same_dtype("S, z, alpha", (S, z, alpha))
    return N, d, dv, _dtype_code(q), _dtype_code(S), _device_ptrs(q, k, v, alpha, y, S, z)


def la_decode_step(q, k, v, alpha, eps: float, y, S, z, stream=None) -> None:
    """One decode step for N independent states, S and z updated in place.

    q, k: [N, d]; v, y: [N, dv]; alpha: [N] or None; S: [N, d, dv]; z: [N, d].
    """
    N, d, dv, io, st, ptrs = _decode_args(q, k, v, alpha, y, S, z)
    rc = library().la_decode_step(ptrs[0], ptrs[1], ptrs[2], ptrs[3], io, N, d, dv, float(eps),
                                  ptrs[4], ptrs[5], ptrs[6], st, _stream_ptr(q, stream))
    _check(rc, "la_decode_step")


def la_decode_step_fm(q, k, v, alpha, eps: float, y, S, z, phi="elu1", stream=None) -> None:
    """:func:`la_decode_step` with the feature map ``phi`` (a FEATURE_MAPS name or code)."""
    N, d, dv, io, st, ptrs = _decode_args(q, k, v, alpha, y, S, z)
    rc = library().la_decode_step_fm(ptrs[0], ptrs[1], ptrs[2], ptrs[3], io, N, d, dv, float(eps),
                                     ptrs[4], ptrs[5], ptrs[6], st, _phi_code(phi), _stream_ptr(q, stream))
    _check(rc, "la_decode_step_fm")


def la_delta_decode_step(q, k, v, beta, y, S, stream=None) -> None:
    """One delta-rule step for N independent memories, S updated in place:
    e = v - S^T k, S <- S + beta k e^T, y = S^T q (no feature map, no normaliser).

    q, k: [N, d]; v, y: [N, dv]; beta: [N]; S: [N, d, dv].
    """
    if q.dim() != 2 or tuple(k.shape) != tuple(q.shape):
        raise ValueError("q and k must both be [N, d] with the same shape")
    N, d = q.shape
    if v.dim() != 2 or v.shape[0] != N:
        raise ValueError("v must be [N, dv] with q's N")
    dv = v.shape[1]
    if tuple(y.shape) != (N, dv) or tuple(S.shape) != (N, d, dv):
        raise ValueError("y must be [N, dv] and S [N, d, dv]")
    if beta is None or tuple(beta.shape) != (N,):
        raise ValueError("beta must be [N]")
    _same_dtype("q, k, v, y", (q, k, v, y))
    _same_dtype("S, beta", (S, beta))
    io, st = _dtype_code(q), _dtype_code(S)
    ptrs = _device_ptrs(q, k, v, beta, y, S)
    rc = library().la_delta_decode_step(ptrs[0], ptrs[1], ptrs[2], ptrs[3], io, N, d, dv, ptrs[4], ptrs[5], st,
                                        _stream_ptr(q, stream))
    _check(rc, "la_delta_decode_step")


def la_softmax_decode_workspace_bytes(io_dtype: int, n_heads: int, L: int, dv: int) -> int:
    """Workspace bytes of la_softmax_decode_step for a history of L rows (0: none needed)."""
    return int(library().la_softmax_decode_workspace_bytes(int(io_dtype), int(n_heads), int(L), int(dv)))


def _softmax_shapes(q, k, v, K_cache, V_cache, y):
    """(H, d, dv, capacity, io) of a softmax decode call, after the shape checks."""
    if q.dim() != 2 or tuple(k.shape) != tuple(q.shape):
        raise ValueError("q and k must both be [H, d] with the same shape")
    H, d = q.shape
    if v.dim() != 2 or v.shape[0] != H or tuple(y.shape) != tuple(v.shape):
        raise ValueError("v and y must be [H, dv] with q's H")
    dv = v.shape[1]
    if K_cache.dim() != 3 or tuple(K_cache.shape[::2]) != (H, d):
        raise ValueError("K_cache must be [H, capacity, d]")
    cap = K_cache.shape[1]
    if tuple(V_cache.shape) != (H, cap, dv):
        raise ValueError("V_cache must be [H, capacity, dv] with K_cache's capacity")
    _same_dtype("q, k, v, y, K_cache, V_cache", (q, k, v, y, K_cache, V_cache))
    return H, d, dv, cap, _dtype_code(q)


def la_softmax_decode_step(q, k, v, pos: int, K_cache, V_cache, y, scale=None, workspace=None,
                           stream=None) -> None:
    """Softmax attention decode over an explicit history: row `pos` of the caches takes
    (k, v), then y = softmax(scale * K_cache[:pos+1] q) V_cache[:pos+1] per head.

    q, k: [H, d]; v, y: [H, dv]; K_cache: [H, capacity, d]; V_cache: [H, capacity, dv];
    scale defaults to 1/sqrt(d).  A workspace (uint8 device tensor) is allocated here
    when the call needs one and none is given.
    """
    H, d, dv, cap, io = _softmax_shapes(q, k, v, K_cache, V_cache, y)
    sc = 1.0 / d ** 0.5 if scale is None else float(scale)
    need = la_softmax_decode_workspace_bytes(io, H, int(pos) + 1, dv) if 0 <= int(pos) < cap else 0
    if need > 0 and workspace is None:
        workspace = _torch().empty(need, dtype=_torch().uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ptrs = _device_ptrs(q, k, v, K_cache, V_cache, y, workspace)
    rc = library().la_softmax_decode_step(ptrs[0], ptrs[1], ptrs[2], io, H, d, dv, int(pos), cap, ptrs[3], ptrs[4],
                                          sc, ptrs[5], ptrs[6], wbytes, _stream_ptr(q, stream))
    _check(rc, "la_softmax_decode_step")


def la_softmax_decode_step_static(q, k, v, pos: int, K_cache, V_cache, y, scale=None, stream=None) -> None:
    """la_softmax_decode_step without a workspace: the library's fixed per-GPU scratch
    (LA_SOFTMAX_STATIC_WORKSPACE_BYTES) holds the partials, so the call allocates nothing.
    Calls that overlap in time on one GPU share that scratch and race."""
    H, d, dv, cap, io = _softmax_shapes(q, k, v, K_cache, V_cache, y)
    sc = 1.0 / d ** 0.5 if scale is None else float(scale)
    ptrs = _device_ptrs(q, k, v, K_cache, V_cache, y)
    rc = library().la_softmax_decode_step_static(ptrs[0], ptrs[1], ptrs[2], io, H, d, dv, int(pos), cap, ptrs[3],
                                                 ptrs[4], sc, ptrs[5], _stream_ptr(q, stream))
    _check(rc, "la_softmax_decode_step_static")


def la_prefill_variant(io_dtype: int, d: int, dv: int, chunk: int, gated: bool, state_dtype: int) -> int:
    """1 = bf16 MFMA kernel, 2 = fp32-arithmetic MFMA kernel (chunk 64: fp32 io at d = 64 or 128,
    bf16 io at d = 64), 0 = general kernel, -1 = rejected."""
    return int(library().la_prefill_variant(io_dtype, d, dv, chunk, int(bool(gated)), state_dtype))


def la_prefill_segments(n_heads: int, T: int, chunk: int, io_dtype: int = LA_BF16, d: int = 128):
    """(segments per sequence, length of all but the last) of the MFMA prefills' plan at
    d = dv = d; segments = 0 when the grid would not fit a launch, -1 for invalid arguments."""
    seg_len = ctypes.c_int64(0)
    n = int(library().la_prefill_segments(int(io_dtype), int(d), int(n_heads), int(T), int(chunk),
                                          ctypes.byref(seg_len)))
    return n, int(seg_len.value)


def la_prefill_segment_slot_bytes(d: int = 128) -> int:
    """Bytes of the state each segment after the first parks in its own rows of Y (-1 for a
    width no MFMA prefill takes)."""
    return int(library().la_prefill_segment_slot_bytes(int(d)))
