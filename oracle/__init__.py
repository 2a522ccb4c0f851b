"""Oracle for causal kernelized linear attention (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never links, loads
or calls it, and it shares no code with the HIP path: the seeded input
generators live in a module of their own and hold none of the method's
arithmetic.

Source of truth is the page "Linear attention：把历史写进状态"
(hs-black.github.io/posts/linear-attention).  Contents:

* :func:`recurrence` -- the oracle proper, the plain FP64 token-by-token
  recurrence (sections "每来一个 token，更新两个累加器", "查询时，分子和分母一起读",
  "ε 是数值保护", "加一个门" and "最小递推里，每一行都有张量意义"), written in
  plain C (``linattn_oracle.c``) and called through ctypes.
* :func:`quadratic_masked` -- the quadratic masked form A = (Q~K~^T) * M,
  Y = AV / rowsum(A) of section "先确认我们在重排哪一种 attention", with the gate
  entering as the products of later gates (exercise 2's coefficients
  [a2*a3, a3, 1]).  Brute force; an independent formula used to pin the
  recurrence.
* :func:`chunkwise` -- the chunk equations of section "一个 chunk 的输出由两部分
  组成", with the gated extension that the page leaves open (it only says that
  the gated form needs the gate products) written as explicit gate products.
* :func:`scan_prefix` -- the affine composition (a2, B2) o (a1, B1) =
  (a2 a1, a2 B1 + B2) of section "门控递推为什么能做并行 scan", combined in
  tree order.
* :func:`delta_steps` -- the delta rule of section "Delta rule：先读旧答案，再写误差"
  (S <- S + beta k (v - S^T k), read y = S^T q after the write), also in C.
* :func:`noncausal` -- the non-causal form of the page "线性注意力架构演进"
  (ai-master.cc): all keys and values are written into the state first, then
  every query reads the full state (eps added to the denominator), in C;
  :func:`quadratic_unmasked` is its brute-force unmasked counterpart.
* :func:`softmax_decode` -- the softmax attention row y = sum softmax(q.k_i/sqrt(d)) v_i
  of section "先看普通 attention 在读什么" (hs-black page), the explicit-history
  comparator of the datawhalechina chapter's Step 5, in C.

Feature maps (``phi_mode``): ``"elu1"`` (ELU+1, the default), ``"relu1"``
(max(x,0)+1, the positive map of the datawhalechina chapter "Linear Attention and
Recurrent State"), ``"relu_eps"`` and ``"sigmoid_eps"`` (max(x,0)+1e-5 and
sigmoid(x)+1e-5, the switchable maps of the ai-master.cc page's pluggable module)
and ``"identity"`` (the inputs already are features, for worked examples).

Every function here is pinned by the CPU tests against the page's worked
examples, closed forms and brute force (see ``tests/test_oracle_pins.py``).
"""
from __future__ import annotations

import concurrent.futures
import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "linattn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liblinattn_oracle.so")
# A build of the same source to load instead (the sanitizer test points this at a build
# with AddressSanitizer and UndefinedBehaviorSanitizer); it must exist, nothing is built.
_ALT_LIB = os.environ.get("LINATTN_ORACLE_LIB")
SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=all"]

PHI_ELU1 = 0
PHI_IDENTITY = 1
PHI_RELU1 = 2
PHI_RELU_EPS = 3
PHI_SIGMOID_EPS = 4
_PHI_MODES = {"elu1": PHI_ELU1, "identity": PHI_IDENTITY, "relu1": PHI_RELU1,
              "relu_eps": PHI_RELU_EPS, "sigmoid_eps": PHI_SIGMOID_EPS}
PHI_MODES = tuple(_PHI_MODES)

_lib = None
_lib_lock = threading.Lock()


def build_oracle(force: bool = True) -> str:
    """Compile ``linattn_oracle.c`` into ``liblinattn_oracle.so`` with gcc.

    No fast-math and no floating-point contraction: the C arithmetic is the
    arithmetic written in the source.
    """
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def build_oracle_sanitized(path: str) -> str:
    """Compile the same source with AddressSanitizer and UndefinedBehaviorSanitizer into
    ``path`` (host code, gcc; loaded through LINATTN_ORACLE_LIB with libasan preloaded)."""
    cmd = ["gcc", *SANITIZE_FLAGS, "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", path, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return path


def loaded_library() -> str:
    """Path of the oracle library this process uses."""
    return _ALT_LIB or _LIB_PATH


def _load():
    global _lib
    with _lib_lock:
        if _lib is None:
            if _ALT_LIB:
                if not os.path.exists(_ALT_LIB):
                    raise RuntimeError("LINATTN_ORACLE_LIB names a missing file: %s" % _ALT_LIB)
                lib = ctypes.CDLL(_ALT_LIB)
            else:
                build_oracle(force=False)
                lib = ctypes.CDLL(_LIB_PATH)
            dp = ctypes.POINTER(ctypes.c_double)
            lib.oracle_recurrence.restype = ctypes.c_int
            lib.oracle_recurrence.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                              dp, dp, dp, dp, ctypes.c_double, ctypes.c_int32,
                                              dp, dp, dp, dp]
            lib.oracle_phi.restype = ctypes.c_double
            lib.oracle_phi.argtypes = [ctypes.c_double]
            lib.oracle_phi_mode.restype = ctypes.c_double
            lib.oracle_phi_mode.argtypes = [ctypes.c_double, ctypes.c_int32]
            lib.oracle_noncausal.restype = ctypes.c_int
            lib.oracle_noncausal.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                             dp, dp, dp, ctypes.c_double, ctypes.c_int32,
                                             dp, dp, dp, dp]
            lib.oracle_softmax_decode.restype = ctypes.c_int
            lib.oracle_softmax_decode.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, dp, dp, dp,
                                                  ctypes.c_double, dp, dp]
            lib.oracle_delta_steps.restype = ctypes.c_int
            lib.oracle_delta_steps.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                               dp, dp, dp, dp, dp, dp, dp]
            _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def phi(x) -> np.ndarray:
    """ELU(x)+1 with ELU's scale 1: x+1 for x > 0, exp(x) otherwise."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0.0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def phi_scalar_c(x: float, phi_mode: str = "elu1") -> float:
    """The C oracle's own feature map, for pinning it to the closed form."""
    if phi_mode == "elu1":
        return _load().oracle_phi(float(x))
    return _load().oracle_phi_mode(float(x), _mode_code(phi_mode))


def _mode_code(phi_mode: str) -> int:
    if phi_mode not in _PHI_MODES:
        raise ValueError("phi_mode must be one of %s" % ", ".join(PHI_MODES))
    return _PHI_MODES[phi_mode]


def _features(x: np.ndarray, phi_mode: str) -> np.ndarray:
    """The feature maps in NumPy (used by the matrix forms; the C oracle has its own)."""
    x = np.asarray(x, dtype=np.float64)
    if phi_mode == "identity":
        return x
    if phi_mode == "elu1":
        return phi(x)
    if phi_mode == "relu1":
        return np.maximum(x, 0.0) + 1.0
    if phi_mode == "relu_eps":
        return np.maximum(x, 0.0) + 1e-5
    if phi_mode == "sigmoid_eps":
        with np.errstate(over="ignore"):
            return 1.0 / (1.0 + np.exp(-x)) + 1e-5
    raise ValueError("phi_mode must be one of %s" % ", ".join(PHI_MODES))


def features(x, phi_mode: str = "elu1") -> np.ndarray:
    """phi applied elementwise, for any of the modes."""
    return _features(x, phi_mode)


def recurrence(q, k, v, alpha=None, eps: float = 1e-6, S0=None, z0=None,
               phi_mode: str = "elu1"):
    """The oracle: FP64 token-by-token recurrence for one sequence.

    q, k: [T, r]; v: [T, dv]; alpha: [T] or None (ungated); S0: [r, dv] and
    z0: [r] (default zero).  Returns ``(Y [T, dv], S [r, dv], z [r], den [T])``
    where ``den`` is phi(q_t)^T z_t before eps is added.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 2 or k.shape != q.shape or v.ndim != 2 or v.shape[0] != q.shape[0] or q.shape[0] == 0:
        raise ValueError("q, k must be [T, r] of equal shape and v [T, dv] with the same T >= 1")
    T, r = q.shape
    dv = v.shape[1]
    if r == 0 or dv == 0:
        raise ValueError("feature and value widths must be >= 1")
    a = None if alpha is None else _f64(alpha).reshape(T)
    S = np.zeros((r, dv)) if S0 is None else _f64(S0).reshape(r, dv).copy()
    z = np.zeros(r) if z0 is None else _f64(z0).reshape(r).copy()
    y = np.empty((T, dv))
    den = np.empty(T)
    rc = _load().oracle_recurrence(T, r, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(a), float(eps),
                                   _mode_code(phi_mode), _ptr(S), _ptr(z), _ptr(y), _ptr(den))
    if rc != 0:
        raise RuntimeError("oracle_recurrence rejected its arguments")
    return y, S, z, den


def recurrence_heads(Q, K, V, alpha=None, eps: float = 1e-6, S0=None, z0=None,
                     phi_mode: str = "elu1", threads: int = 1):
    """:func:`recurrence` over independent heads.

    Q, K: [..., T, r]; V: [..., T, dv]; alpha: [..., T] or None; S0: [..., r, dv];
    z0: [..., r].  Heads are independent, so ``threads`` > 1 runs them on a
    thread pool (ctypes releases the GIL during the C call).
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    lead = Q.shape[:-2]
    T, r = Q.shape[-2:]
    dv = V.shape[-1]
    n = int(np.prod(lead)) if lead else 1
    Qf, Kf, Vf = Q.reshape(n, T, r), K.reshape(n, T, r), V.reshape(n, T, dv)
    Af = None if alpha is None else _f64(alpha).reshape(n, T)
    Sf = None if S0 is None else _f64(S0).reshape(n, r, dv)
    zf = None if z0 is None else _f64(z0).reshape(n, r)
    Y = np.empty((n, T, dv))
    S = np.empty((n, r, dv))
    z = np.empty((n, r))
    den = np.empty((n, T))

    def one(h):
        Y[h], S[h], z[h], den[h] = recurrence(
            Qf[h], Kf[h], Vf[h], None if Af is None else Af[h], eps,
            None if Sf is None else Sf[h], None if zf is None else zf[h], phi_mode)

    if threads <= 1 or n == 1:
        for h in range(n):
            one(h)
    else:
        with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, range(n)))
    return (Y.reshape(*lead, T, dv), S.reshape(*lead, r, dv), z.reshape(*lead, r),
            den.reshape(*lead, T))


def gate_products(alpha, T: int) -> np.ndarray:
    """D[t, i] = alpha[i+1] * ... * alpha[t] for i <= t (empty product 1), 0 above.

    The weight the gate leaves on token i's write when token t reads (the
    coefficients [a2*a3, a3, 1] of exercise 2).  Built by explicit products.
    """
    D = np.zeros((T, T))
    for i in range(T):
        D[i, i] = 1.0
        for t in range(i + 1, T):
            D[t, i] = D[t - 1, i] * (1.0 if alpha is None else float(alpha[t]))
    return D


def decay_from_start(alpha, T: int) -> np.ndarray:
    """c[t] = alpha[0] * ... * alpha[t]: the weight left on the incoming state at token t."""
    c = np.empty(T)
    acc = 1.0
    for t in range(T):
        acc = acc * (1.0 if alpha is None else float(alpha[t]))
        c[t] = acc
    return c


def quadratic_masked(q, k, v, alpha=None, eps: float = 1e-6, S0=None, z0=None,
                     phi_mode: str = "elu1"):
    """Brute-force quadratic form: A = (Q~ K~^T) * M (times gate products),
    Y = (c * Q~ S0 + A V) / (c * Q~ z0 + rowsum(A) + eps).

    With S0 = z0 = 0 and no gate this is exactly Y = AV / (rowsum(A) + eps).
    Returns ``(Y, den)``.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    T = q.shape[0]
    qf, kf = _features(q, phi_mode), _features(k, phi_mode)
    A = (qf @ kf.T) * gate_products(alpha, T)
    num = A @ v
    den = A.sum(axis=1)
    if S0 is not None or z0 is not None:
        c = decay_from_start(alpha, T)
        if S0 is not None:
            num = num + c[:, None] * (qf @ _f64(S0))
        if z0 is not None:
            den = den + c * (qf @ _f64(z0))
    return num / (den + eps)[:, None], den


def chunkwise(q, k, v, alpha=None, eps: float = 1e-6, chunk: int = 64, S0=None, z0=None,
              phi_mode: str = "elu1"):
    """FP64 chunkwise form.  Per chunk c with incoming S_prev, z_prev:

    num    = g * (Q~c S_prev) + [(Q~c K~c^T) * D] Vc
    den    = g * (Q~c z_prev) + rowsum[(Q~c K~c^T) * D]
    S_next = g_last * S_prev + K~c^T (w * Vc)
    z_next = g_last * z_prev + sum_i w_i K~c[i]

    where D holds the in-chunk gate products (the causal mask M when ungated),
    g[j] the product of the chunk's gates up to token j, and w[i] = D[last, i].
    Returns ``(Y, S, z, den)``.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, r = q.shape
    dv = v.shape[1]
    if chunk < 1:
        raise ValueError("chunk must be >= 1")
    qf, kf = _features(q, phi_mode), _features(k, phi_mode)
    S = np.zeros((r, dv)) if S0 is None else _f64(S0).copy()
    z = np.zeros(r) if z0 is None else _f64(z0).copy()
    Y = np.empty((T, dv))
    den_all = np.empty(T)
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        n = t1 - t0
        a = None if alpha is None else np.asarray(alpha, dtype=np.float64)[t0:t1]
        D = gate_products(a, n)
        g = decay_from_start(a, n)
        Qc, Kc, Vc = qf[t0:t1], kf[t0:t1], v[t0:t1]
        A = (Qc @ Kc.T) * D
        num = g[:, None] * (Qc @ S) + A @ Vc
        den = g * (Qc @ z) + A.sum(axis=1)
        Y[t0:t1] = num / (den + eps)[:, None]
        den_all[t0:t1] = den
        w = D[n - 1]
        S = g[n - 1] * S + Kc.T @ (w[:, None] * Vc)
        z = g[n - 1] * z + (w[:, None] * Kc).sum(axis=0)
    return Y, S, z, den_all


def compose(later, earlier):
    """(a2, B2, b2) o (a1, B1, b1) = (a2 a1, a2 B1 + B2, a2 b1 + b2).

    Applying ``earlier`` then ``later`` to a state; b is the normaliser part
    (B with k~ in place of k~ v^T).
    """
    a2, B2, b2 = later
    a1, B1, b1 = earlier
    return (a2 * a1, a2 * B1 + B2, a2 * b1 + b2)


def scan_prefix(q, k, v, alpha=None, eps: float = 1e-6, S0=None, z0=None,
                phi_mode: str = "elu1", order: str = "correct"):
    """Inclusive prefix of the per-token affine maps by recursive doubling
    (a tree order of composition, not the sequential one), then the read-out.

    ``order='swapped'`` composes earlier o later instead; it exists only so
    the tests can show that the order of composition matters.
    Returns ``(Y, S, z, den)``.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, r = q.shape
    dv = v.shape[1]
    qf, kf = _features(q, phi_mode), _features(k, phi_mode)
    cur = []
    for t in range(T):
        a_t = 1.0 if alpha is None else float(alpha[t])
        cur.append((a_t, np.outer(kf[t], v[t]), kf[t].copy()))
    off = 1
    while off < T:
        nxt = list(cur)
        for t in range(off, T):
            if order == "correct":
                nxt[t] = compose(cur[t], cur[t - off])
            else:
                nxt[t] = compose(cur[t - off], cur[t])
        cur = nxt
        off *= 2
    S_in = np.zeros((r, dv)) if S0 is None else _f64(S0)
    z_in = np.zeros(r) if z0 is None else _f64(z0)
    Y = np.empty((T, dv))
    den = np.empty(T)
    for t in range(T):
        a_t, B_t, b_t = cur[t]
        S_t = a_t * S_in + B_t
        z_t = a_t * z_in + b_t
        den[t] = qf[t] @ z_t
        Y[t] = (qf[t] @ S_t) / (den[t] + eps)
    a_T, B_T, b_T = cur[T - 1]
    return Y, a_T * S_in + B_T, a_T * z_in + b_T, den


def delta_steps(q, k, v, beta, S0=None):
    """Delta-rule oracle for one memory: T steps of p = S^T k, e = v - p,
    S <- S + beta k e^T, y = S^T q (after the write); raw q and k.

    q, k: [T, r]; v: [T, dv]; beta: [T]; S0: [r, dv] (default zero).
    Returns ``(Y [T, dv], S [r, dv], P [T, dv])`` with P the predictions before each write.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 2 or k.shape != q.shape or v.ndim != 2 or v.shape[0] != q.shape[0] or q.shape[0] == 0:
        raise ValueError("q, k must be [T, r] of equal shape and v [T, dv] with the same T >= 1")
    T, r = q.shape
    dv = v.shape[1]
    b = _f64(beta).reshape(T)
    S = np.zeros((r, dv)) if S0 is None else _f64(S0).reshape(r, dv).copy()
    y = np.empty((T, dv))
    P = np.empty((T, dv))
    rc = _load().oracle_delta_steps(T, r, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(b), _ptr(S), _ptr(y), _ptr(P))
    if rc != 0:
        raise RuntimeError("oracle_delta_steps rejected its arguments")
    return y, S, P


def delta_steps_states(Q, K, V, beta, S0, threads: int = 1):
    """:func:`delta_steps` over independent memories: Q, K [n, T, r]; V [n, T, dv];
    beta [n, T]; S0 [n, r, dv].  Returns ``(Y [n, T, dv], S [n, r, dv])``."""
    Q, K, V, B, S0 = _f64(Q), _f64(K), _f64(V), _f64(beta), _f64(S0)
    n, T, r = Q.shape
    dv = V.shape[-1]
    Y = np.empty((n, T, dv))
    S = np.empty((n, r, dv))

    def one(h):
        Y[h], S[h], _ = delta_steps(Q[h], K[h], V[h], B[h], S0[h])

    if threads <= 1 or n == 1:
        for h in range(n):
            one(h)
    else:
        with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, range(n)))
    return Y, S


def noncausal(q, k, v, eps: float = 1e-6, S0=None, z0=None, phi_mode: str = "elu1"):
    """Non-causal oracle for one sequence: S = S0 + sum_t k~_t v_t^T, z = z0 + sum_t k~_t
    over the whole sequence, then y_t = q~_t^T S / (q~_t^T z + eps) for every t.

    Shapes as :func:`recurrence`.  Returns ``(Y [T, dv], S [r, dv], z [r], den [T])``.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 2 or k.shape != q.shape or v.ndim != 2 or v.shape[0] != q.shape[0] or q.shape[0] == 0:
        raise ValueError("q, k must be [T, r] of equal shape and v [T, dv] with the same T >= 1")
    T, r = q.shape
    dv = v.shape[1]
    if r == 0 or dv == 0:
        raise ValueError("feature and value widths must be >= 1")
    S = np.zeros((r, dv)) if S0 is None else _f64(S0).reshape(r, dv).copy()
    z = np.zeros(r) if z0 is None else _f64(z0).reshape(r).copy()
    y = np.empty((T, dv))
    den = np.empty(T)
    rc = _load().oracle_noncausal(T, r, dv, _ptr(q), _ptr(k), _ptr(v), float(eps), _mode_code(phi_mode),
                                  _ptr(S), _ptr(z), _ptr(y), _ptr(den))
    if rc != 0:
        raise RuntimeError("oracle_noncausal rejected its arguments")
    return y, S, z, den


def noncausal_heads(Q, K, V, eps: float = 1e-6, S0=None, z0=None, phi_mode: str = "elu1",
                    threads: int = 1):
    """:func:`noncausal` over independent heads (shapes as :func:`recurrence_heads`)."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    lead = Q.shape[:-2]
    T, r = Q.shape[-2:]
    dv = V.shape[-1]
    n = int(np.prod(lead)) if lead else 1
    Qf, Kf, Vf = Q.reshape(n, T, r), K.reshape(n, T, r), V.reshape(n, T, dv)
    Sf = None if S0 is None else _f64(S0).reshape(n, r, dv)
    zf = None if z0 is None else _f64(z0).reshape(n, r)
    Y = np.empty((n, T, dv))
    S = np.empty((n, r, dv))
    z = np.empty((n, r))
    den = np.empty((n, T))

    def one(h):
        Y[h], S[h], z[h], den[h] = noncausal(Qf[h], Kf[h], Vf[h], eps, None if Sf is None else Sf[h],
                                             None if zf is None else zf[h], phi_mode)

    if threads <= 1 or n == 1:
        for h in range(n):
            one(h)
    else:
        with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, range(n)))
    return (Y.reshape(*lead, T, dv), S.reshape(*lead, r, dv), z.reshape(*lead, r),
            den.reshape(*lead, T))


def quadratic_unmasked(q, k, v, eps: float = 1e-6, S0=None, z0=None, phi_mode: str = "elu1"):
    """Brute-force unmasked form: A = Q~ K~^T over all pairs (no causal mask),
    Y = (Q~ S0 + A V) / (Q~ z0 + rowsum(A) + eps).  Returns ``(Y, den)``."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    qf, kf = _features(q, phi_mode), _features(k, phi_mode)
    A = qf @ kf.T
    num = A @ v
    den = A.sum(axis=1)
    if S0 is not None:
        num = num + qf @ _f64(S0)
    if z0 is not None:
        den = den + qf @ _f64(z0)
    return num / (den + eps)[:, None], den


def softmax_decode(q, K, V, scale=None):
    """Softmax attention of one query over an explicit history: y = sum_i w_i v_i with
    w = softmax(scale * K q) (scale defaults to 1/sqrt(r)).

    q: [r]; K: [L, r]; V: [L, dv].  Returns ``(y [dv], w [L])``.
    """
    q, K, V = _f64(q).reshape(-1), _f64(K), _f64(V)
    if K.ndim != 2 or V.ndim != 2 or K.shape[0] != V.shape[0] or K.shape[1] != q.shape[0] or K.shape[0] == 0:
        raise ValueError("q must be [r], K [L, r] and V [L, dv] with L >= 1")
    L, r = K.shape
    dv = V.shape[1]
    if r == 0 or dv == 0:
        raise ValueError("feature and value widths must be >= 1")
    sc = 1.0 / np.sqrt(r) if scale is None else float(scale)
    y = np.empty(dv)
    w = np.empty(L)
    rc = _load().oracle_softmax_decode(L, r, dv, _ptr(q), _ptr(K), _ptr(V), sc, _ptr(y), _ptr(w))
    if rc != 0:
        raise RuntimeError("oracle_softmax_decode rejected its arguments")
    return y, w


def softmax_decode_heads(q, K, V, scale=None, threads: int = 1):
    """:func:`softmax_decode` over independent heads: q [n, r]; K [n, L, r]; V [n, L, dv].
    Returns ``y [n, dv]``."""
    q, K, V = _f64(q), _f64(K), _f64(V)
    n = q.shape[0]
    Y = np.empty((n, V.shape[-1]))

    def one(h):
        Y[h] = softmax_decode(q[h], K[h], V[h], scale)[0]

    if threads <= 1 or n == 1:
        for h in range(n):
            one(h)
    else:
        with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, range(n)))
    return Y
