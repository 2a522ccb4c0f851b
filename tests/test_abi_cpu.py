"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments with the documented status codes
before anything is launched (so no call here reaches the device)."""
import ctypes
import math
import os
import re

import pytest

import recurrent_state_chunkwise_amd as la

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "linattn.h")

OK, NULL, SHAPE, DTYPE, EPS, CHUNK, UNSUP, LAUNCH, ALIAS, PHI, WORKSPACE, SCALE = range(12)
F64, F32, BF16 = la.LA_F64, la.LA_F32, la.LA_BF16


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(la.library_path()):
        from recurrent_state_chunkwise_amd import build
        build.build()
    return la.library()


def _declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(la_[a-z_]+)\s*\(", text)))


def test_header_symbols_exported(lib):
    names = _declared_functions()
    assert set(names) >= {"la_state_init", "la_prefill_chunked", "la_decode_step", "la_delta_decode_step",
                          "la_status_str", "la_prefill_variant", "la_prefill_chunked_fm", "la_decode_step_fm",
                          "la_prefill_noncausal", "la_softmax_decode_step", "la_softmax_decode_workspace_bytes"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in range(12):
        s = la.la_status_str(code)
        assert isinstance(s, str) and s
    assert la.la_status_str(0) == "ok"
    assert la.la_status_str(99) == "unknown status"


# fake, distinct, non-overlapping device addresses: validation fails before any use
P = [ctypes.c_void_p(0x100000000 + i * 0x10000000) for i in range(8)]


def prefill(lib, Q=P[0], K=P[1], V=P[2], alpha=None, io=BF16, B=1, H=1, T=8, d=4, dv=4, eps=1e-6, chunk=4,
            Y=P[3], S=P[4], z=P[5], st=F32):
    return lib.la_prefill_chunked(Q, K, V, alpha, io, B, H, T, d, dv, eps, chunk, Y, S, z, st, None)


def decode(lib, q=P[0], k=P[1], v=P[2], alpha=None, io=BF16, N=4, d=4, dv=4, eps=1e-6, y=P[3], S=P[4],
           z=P[5], st=F32):
    return lib.la_decode_step(q, k, v, alpha, io, N, d, dv, eps, y, S, z, st, None)


def test_prefill_rejections(lib):
    assert prefill(lib, Q=None) == NULL
    assert prefill(lib, Y=None) == NULL
    assert prefill(lib, z=None) == NULL
    assert prefill(lib, T=0) == SHAPE            # empty sequence (ch. 45 input contract)
    assert prefill(lib, B=0) == SHAPE
    assert prefill(lib, H=-1) == SHAPE
    assert prefill(lib, d=0) == SHAPE
    assert prefill(lib, dv=0) == SHAPE
    assert prefill(lib, io=7) == DTYPE
    assert prefill(lib, io=BF16, st=F64) == DTYPE
    assert prefill(lib, io=F64, st=F32) == DTYPE
    assert prefill(lib, io=F32, st=BF16) == DTYPE
    assert prefill(lib, eps=-1e-9) == EPS
    assert prefill(lib, eps=math.nan) == EPS
    assert prefill(lib, eps=math.inf) == EPS
    assert prefill(lib, chunk=0) == CHUNK
    assert prefill(lib, chunk=129) == UNSUP
    assert prefill(lib, d=129) == UNSUP
    assert prefill(lib, dv=256) == UNSUP
    assert prefill(lib, B=1 << 40, H=1 << 40) == SHAPE
    # outputs overlapping inputs or each other
    assert prefill(lib, Y=P[0]) == ALIAS
    assert prefill(lib, S=ctypes.c_void_p(P[2].value + 8)) == ALIAS
    assert prefill(lib, z=P[4]) == ALIAS
    assert prefill(lib, alpha=P[4]) == ALIAS


def test_decode_rejections(lib):
    assert decode(lib, q=None) == NULL
    assert decode(lib, S=None) == NULL
    assert decode(lib, N=0) == SHAPE
    assert decode(lib, N=1 << 33) == SHAPE
    assert decode(lib, d=0) == SHAPE
    assert decode(lib, io=BF16, st=F64) == DTYPE
    assert decode(lib, eps=-1.0) == EPS
    assert decode(lib, d=200) == UNSUP
    assert decode(lib, y=P[1]) == ALIAS
    assert decode(lib, S=P[5]) == ALIAS
    assert decode(lib, alpha=P[3]) == ALIAS


def delta(lib, q=P[0], k=P[1], v=P[2], beta=P[6], io=BF16, N=4, d=4, dv=4, y=P[3], S=P[4], st=F32):
    return lib.la_delta_decode_step(q, k, v, beta, io, N, d, dv, y, S, st, None)


def test_delta_decode_rejections(lib):
    assert delta(lib, q=None) == NULL
    assert delta(lib, beta=None) == NULL          # beta is required
    assert delta(lib, S=None) == NULL
    assert delta(lib, N=0) == SHAPE
    assert delta(lib, N=1 << 33) == SHAPE
    assert delta(lib, dv=0) == SHAPE
    assert delta(lib, io=BF16, st=F64) == DTYPE
    assert delta(lib, io=F64, st=F32) == DTYPE
    assert delta(lib, d=129) == UNSUP
    assert delta(lib, y=P[1]) == ALIAS
    assert delta(lib, S=P[3]) == ALIAS
    assert delta(lib, beta=P[4]) == ALIAS


def test_state_init_rejections(lib):
    assert lib.la_state_init(None, P[1], 1, 4, 4, F32, None) == NULL
    assert lib.la_state_init(P[0], P[1], 0, 4, 4, F32, None) == SHAPE
    assert lib.la_state_init(P[0], P[1], 1, 4, 4, BF16, None) == DTYPE
    assert lib.la_state_init(P[0], P[0], 1, 4, 4, F32, None) == ALIAS


def test_prefill_variant(lib):
    assert la.la_prefill_variant(BF16, 16, 16, 16, False, F32) == 0
    assert la.la_prefill_variant(F64, 16, 16, 16, False, F64) == 0
    assert la.la_prefill_variant(F32, 128, 128, 64, True, F32) == 2   # the fp32 MFMA kernel
    assert la.la_prefill_variant(F32, 128, 128, 128, True, F32) == 0  # fp32 at chunk 128: general
    assert la.la_prefill_variant(F32, 64, 64, 64, False, F32) == 2     # d = 64: fp32 MFMA, either io
    assert la.la_prefill_variant(BF16, 64, 64, 64, True, F32) == 2
    assert la.la_prefill_variant(BF16, 64, 64, 128, True, F32) == 0
    assert la.la_prefill_variant(F32, 64, 128, 64, True, F32) == 0
    assert la.la_prefill_variant(F64, 64, 64, 64, True, F64) == 0
    assert la.la_prefill_variant(BF16, 96, 96, 64, False, F32) == 0
    assert la.la_prefill_variant(BF16, 128, 128, 64, False, F32) == 1
    assert la.la_prefill_variant(BF16, 128, 128, 128, True, F32) == 1
    assert la.la_prefill_variant(BF16, 128, 128, 32, True, F32) == 0
    assert la.la_prefill_variant(BF16, 64, 128, 64, True, F32) == 0
    assert la.la_prefill_variant(BF16, 129, 128, 64, False, F32) == -1
    assert la.la_prefill_variant(BF16, 128, 128, 0, False, F32) == -1
    assert la.la_prefill_variant(BF16, 128, 128, 64, False, F64) == -1


def test_binding_shape_contract_cpu():
    """The binding rejects Q/K width mismatches and empty sequences (ValueError,
    the first page's convention) before touching any device."""
    import torch
    q = torch.zeros(1, 1, 2, 2)
    with pytest.raises(ValueError):
        la.la_prefill_chunked(q, torch.zeros(1, 1, 2, 3), torch.zeros(1, 1, 2, 1), None, 1e-6, 4,
                              torch.zeros(1, 1, 2, 1), torch.zeros(1, 1, 2, 1), torch.zeros(1, 1, 2))
    e = torch.zeros(1, 1, 0, 2)
    with pytest.raises(ValueError):
        la.la_prefill_chunked(e, e, torch.zeros(1, 1, 0, 1), None, 1e-6, 4, torch.zeros(1, 1, 0, 1),
                              torch.zeros(1, 1, 2, 1), torch.zeros(1, 1, 2))
    with pytest.raises(ValueError):
        la.la_decode_step(torch.zeros(2, 3), torch.zeros(2, 4), torch.zeros(2, 1), None, 1e-6,
                          torch.zeros(2, 1), torch.zeros(2, 3, 1), torch.zeros(2, 3))
    with pytest.raises(ValueError):
        la.la_delta_decode_step(torch.zeros(2, 3), torch.zeros(2, 3), torch.zeros(2, 1), None,
                                torch.zeros(2, 1), torch.zeros(2, 3, 1))


def prefill_fm(lib, phi=0, **kw):
    a = dict(Q=P[0], K=P[1], V=P[2], alpha=None, io=BF16, B=1, H=1, T=8, d=4, dv=4, eps=1e-6, chunk=4, Y=P[3],
             S=P[4], z=P[5], st=F32)
    a.update(kw)
    return lib.la_prefill_chunked_fm(a["Q"], a["K"], a["V"], a["alpha"], a["io"], a["B"], a["H"], a["T"], a["d"],
                                     a["dv"], a["eps"], a["chunk"], a["Y"], a["S"], a["z"], a["st"], phi, None)


def decode_fm(lib, phi=0, **kw):
    a = dict(q=P[0], k=P[1], v=P[2], alpha=None, io=BF16, N=4, d=4, dv=4, eps=1e-6, y=P[3], S=P[4], z=P[5], st=F32)
    a.update(kw)
    return lib.la_decode_step_fm(a["q"], a["k"], a["v"], a["alpha"], a["io"], a["N"], a["d"], a["dv"], a["eps"],
                                 a["y"], a["S"], a["z"], a["st"], phi, None)


def noncausal(lib, Q=P[0], K=P[1], V=P[2], io=BF16, B=1, H=1, T=8, d=4, dv=4, eps=1e-6, Y=P[3], S=P[4], z=P[5],
              st=F32, phi=0):
    return lib.la_prefill_noncausal(Q, K, V, io, B, H, T, d, dv, eps, Y, S, z, st, phi, None)


def test_feature_map_rejections(lib):
    # an unknown map is LA_ERR_PHI; the other checks are those of the calls without _fm
    for bad in (-1, 4, 99):
        assert prefill_fm(lib, phi=bad) == PHI
        assert decode_fm(lib, phi=bad) == PHI
        assert noncausal(lib, phi=bad) == PHI
    assert prefill_fm(lib, phi=1, Q=None) == NULL
    assert prefill_fm(lib, phi=2, T=0) == SHAPE
    assert prefill_fm(lib, phi=3, chunk=0) == CHUNK
    assert prefill_fm(lib, phi=3, Y=P[0]) == ALIAS
    assert decode_fm(lib, phi=1, N=0) == SHAPE
    assert decode_fm(lib, phi=2, eps=-1.0) == EPS
    assert decode_fm(lib, phi=3, y=P[1]) == ALIAS


def test_noncausal_rejections(lib):
    assert noncausal(lib, Q=None) == NULL
    assert noncausal(lib, z=None) == NULL
    assert noncausal(lib, T=0) == SHAPE
    assert noncausal(lib, B=0) == SHAPE
    assert noncausal(lib, dv=0) == SHAPE
    assert noncausal(lib, B=1 << 40, H=1 << 40) == SHAPE
    assert noncausal(lib, io=7) == DTYPE
    assert noncausal(lib, io=BF16, st=F64) == DTYPE
    assert noncausal(lib, io=F64, st=F32) == DTYPE
    assert noncausal(lib, eps=math.nan) == EPS
    assert noncausal(lib, eps=-1e-3) == EPS
    assert noncausal(lib, d=129) == UNSUP
    assert noncausal(lib, Y=P[2]) == ALIAS
    assert noncausal(lib, S=ctypes.c_void_p(P[0].value + 16)) == ALIAS
    assert noncausal(lib, z=P[4]) == ALIAS


def test_binding_feature_map_names():
    """Names map to the header's codes; an unknown name is a ValueError before any call."""
    import torch
    assert la.FEATURE_MAPS == {"elu1": 0, "relu1": 1, "relu_eps": 2, "sigmoid_eps": 3}
    q = torch.zeros(1, 1, 2, 2)
    with pytest.raises(ValueError):
        la.la_prefill_noncausal(q, q, torch.zeros(1, 1, 2, 1), 1e-6, torch.zeros(1, 1, 2, 1),
                                torch.zeros(1, 1, 2, 1), torch.zeros(1, 1, 2), phi="softplus")
    with pytest.raises(ValueError):
        la.la_prefill_noncausal(q, torch.zeros(1, 1, 2, 3), torch.zeros(1, 1, 2, 1), 1e-6, torch.zeros(1, 1, 2, 1),
                                torch.zeros(1, 1, 2, 1), torch.zeros(1, 1, 2))


def softmax(lib, q=P[0], k=P[1], v=P[2], io=BF16, H=2, d=64, dv=64, pos=10, cap=16, Kc=P[3], Vc=P[4],
            scale=0.125, y=P[5], ws=P[6], wbytes=1 << 20):
    return lib.la_softmax_decode_step(q, k, v, io, H, d, dv, pos, cap, Kc, Vc, scale, y, ws, wbytes, None)


def test_softmax_decode_workspace_bytes(lib):
    # one 256-row piece needs no workspace; then n_heads * pieces * (2 + dv) accumulators
    assert la.la_softmax_decode_workspace_bytes(BF16, 8, 256, 64) == 0
    assert la.la_softmax_decode_workspace_bytes(BF16, 8, 257, 64) == 8 * 2 * 66 * 4
    assert la.la_softmax_decode_workspace_bytes(F64, 8, 8192, 64) == 8 * 32 * 66 * 8
    assert la.la_softmax_decode_workspace_bytes(BF16, 0, 8, 64) == -1
    assert la.la_softmax_decode_workspace_bytes(BF16, 1, 8, 129) == -1


def test_softmax_decode_rejections(lib):
    assert softmax(lib, q=None) == NULL
    assert softmax(lib, Kc=None) == NULL
    assert softmax(lib, y=None) == NULL
    assert softmax(lib, H=0) == SHAPE
    assert softmax(lib, pos=-1) == SHAPE
    assert softmax(lib, pos=16, cap=16) == SHAPE     # pos must lie inside the caches
    assert softmax(lib, d=0) == SHAPE
    assert softmax(lib, io=9) == DTYPE
    assert softmax(lib, d=200) == UNSUP
    assert softmax(lib, scale=math.nan) == SCALE
    assert softmax(lib, scale=math.inf) == SCALE
    # pos = 300: two pieces, so a workspace is required
    assert softmax(lib, pos=300, cap=512, ws=None) == WORKSPACE
    assert softmax(lib, pos=300, cap=512, wbytes=100) == WORKSPACE
    assert softmax(lib, pos=10, ws=None, wbytes=0, y=P[0]) == ALIAS  # no workspace needed at pos 10
    assert softmax(lib, y=P[0]) == ALIAS
    assert softmax(lib, Kc=ctypes.c_void_p(P[2].value + 8)) == ALIAS
    assert softmax(lib, Vc=P[3]) == ALIAS
    assert softmax(lib, pos=300, cap=512, ws=P[5]) == ALIAS


def softmax_static(lib, q=P[0], k=P[1], v=P[2], io=BF16, H=2, d=64, dv=64, pos=10, cap=16, Kc=P[3], Vc=P[4],
                   scale=0.125, y=P[5]):
    return lib.la_softmax_decode_step_static(q, k, v, io, H, d, dv, pos, cap, Kc, Vc, scale, y, None)


def test_softmax_decode_static_rejections(lib):
    """The allocation-free variant checks its arguments like la_softmax_decode_step and
    refuses, before any launch, a call whose partials exceed its fixed scratch."""
    assert la.LA_SOFTMAX_STATIC_WORKSPACE_BYTES == 32 << 20
    assert softmax_static(lib, q=None) == NULL
    assert softmax_static(lib, Vc=None) == NULL
    assert softmax_static(lib, H=0) == SHAPE
    assert softmax_static(lib, pos=16, cap=16) == SHAPE
    assert softmax_static(lib, io=9) == DTYPE
    assert softmax_static(lib, dv=129) == UNSUP
    assert softmax_static(lib, scale=math.inf) == SCALE
    assert softmax_static(lib, y=P[1]) == ALIAS
    # 4,096 heads over 8,192 rows at dv = 128: 4096 x 32 pieces x 130 floats = 68 MB of
    # partials, beyond the 32 MiB array (buffers placed 1 TiB apart so none overlap)
    far = [ctypes.c_void_p((1 << 40) * (i + 1)) for i in range(6)]
    big = dict(q=far[0], k=far[1], v=far[2], Kc=far[3], Vc=far[4], y=far[5], H=4096, d=128, dv=128,
               pos=8191, cap=8192)
    need = la.la_softmax_decode_workspace_bytes(BF16, 4096, 8192, 128)
    assert need == 4096 * 32 * 130 * 4 > la.LA_SOFTMAX_STATIC_WORKSPACE_BYTES
    assert softmax_static(lib, **big) == WORKSPACE


# ---------------------------------------------------------------- the segment plan
PLAN_T = [1, 2, 63, 64, 65, 258, 259, 319, 320, 321, 383, 384, 385, 1000, 4096, 16384, 131072, 1 << 20,
          (1 << 22) - 1, 1 << 22, (1 << 22) + 1, 1 << 23, (1 << 24) + 17, 3 * (1 << 24) + 5]
PLAN_H = [1, 2, 3, 4, 31, 32, 64, 100, 255, 256, 257, 4096, 65536, 1 << 20, (1 << 31) - 1]
INT32_MAX = (1 << 31) - 1


# (io dtype, width d = dv, chunk, bytes of one row of Q) of every MFMA prefill plan
PLANS = [(BF16, 128, 64, 256), (BF16, 128, 128, 256), (F32, 128, 64, 512), (F32, 64, 64, 256),
         (BF16, 64, 64, 128)]


@pytest.mark.parametrize("io,d,chunk,row", PLANS)
def test_segment_plan_invariants(lib, io, d, chunk, row):
    """The plan of the MFMA prefills at extreme lengths and head counts: whole chunks, every
    segment's own rows of Y hold its state slot, 32-bit offsets inside every segment, a grid
    that fits one launch, the compute units filled when the length allows, and no more
    segments than needed."""
    slot = la.la_prefill_segment_slot_bytes(d)
    assert slot == (d * d + d + 4) * 4       # S, z and the segment's gate product, padded
    min_len = -(-(-(-slot // row)) // chunk) * chunk  # shortest segment that holds a slot
    max_len = (1 << 31) // row // 2            # longest segment but the last: below 2^30 bytes
    for T in PLAN_T:
        for H in PLAN_H:
            nseg, seg_len = la.la_prefill_segments(H, T, chunk, io, d)
            if nseg == 0:  # refused: even the fewest segments would not fit one grid
                assert H * -(-T // max_len) > INT32_MAX, (T, H)
                continue
            assert 1 <= nseg and H * nseg <= INT32_MAX, (T, H, nseg)
            last = T - (nseg - 1) * seg_len
            if nseg == 1:
                assert seg_len == T and T * row < (1 << 31), (T, H)
                continue
            assert seg_len % chunk == 0 and seg_len >= min_len, (T, H, seg_len)
            assert seg_len * row >= slot                 # slot p sits in segment p's own rows
            assert seg_len <= last, (T, H, seg_len, last)  # the last segment takes the rest
            assert last * row < (1 << 31) and seg_len * row < (1 << 31)
            want = -(-256 // H)                          # workgroups to fill 256 compute units
            if T // min_len >= want:
                assert H * nseg >= 256 or nseg >= want, (T, H, nseg)
            assert nseg <= max(want, -(-T // max_len)), (T, H, nseg)


def test_segment_plan_rejections(lib):
    assert la.la_prefill_segments(0, 100, 64)[0] == -1
    assert la.la_prefill_segments(4, 0, 64)[0] == -1
    assert la.la_prefill_segments(4, 100, 32)[0] == -1
    assert lib.la_prefill_segments(BF16, 128, 4, 100, 64, None) == -1
    assert la.la_prefill_segments(4, 100, 64, BF16, 96)[0] == -1   # no MFMA prefill at d = 96
    assert la.la_prefill_segments(4, 100, 128, BF16, 64)[0] == -1  # d = 64 runs chunk 64 only
    assert la.la_prefill_segment_slot_bytes(96) == -1
    # the full workloads: one segment per compute unit (or per sequence past 256 sequences)
    assert la.la_prefill_segments(64, 4096, 64) == (4, 1024)
    assert la.la_prefill_segments(32, 16384, 64) == (8, 2048)
    assert la.la_prefill_segments(32, 131072, 128) == (8, 16384)
    assert la.la_prefill_segments(65536, 256, 64) == (1, 256)
    # the fp32 kernel plans with its own 512-byte rows, at chunk 64 only
    assert la.la_prefill_segments(64, 4096, 64, F32) == (4, 1024)
    assert la.la_prefill_segments(64, 4096, 128, F32)[0] == -1
    assert la.la_prefill_segments(64, 4096, 64, F64)[0] == -1
    # d = 64 (16,656-byte slots): the state builds of the history-against-state comparison,
    # 8 sequences of 8,191 tokens cut into 32 segments of 192, and 1,024 sequences uncut
    assert la.la_prefill_segments(8, 8191, 64, BF16, 64) == (32, 192)
    assert la.la_prefill_segments(1024, 8191, 64, BF16, 64) == (1, 8191)
    assert la.la_prefill_segments(8, 8191, 64, F32, 64) == (32, 192)


def test_segment_plan_f32_rows(lib):
    # fp32 rows are 512 bytes: every segment, the last included, stays below 2^31 bytes of Q
    for T in PLAN_T:
        for H in (1, 3, 64, 256, 65536):
            nseg, seg_len = la.la_prefill_segments(H, T, 64, F32)
            if nseg <= 0:
                assert nseg == 0 and H * -(-T // ((1 << 31) // 512 // 2)) > INT32_MAX
                continue
            last = T - (nseg - 1) * seg_len
            assert last * 512 < (1 << 31) and seg_len * 512 < (1 << 31), (T, H, nseg, seg_len)
            if nseg > 1:
                assert seg_len % 64 == 0 and seg_len * 512 >= la.la_prefill_segment_slot_bytes(128)
