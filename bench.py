"""Benchmark of the linear-attention hot path on one MI355X.

One step = one state initialisation plus one la_prefill_chunked call over the
ungated prefill workload B=4, H=16, T=4096, d=dv=128, chunk 64, bf16 inputs
resident in HBM (the workload the prefill metric is quoted on).  `value` is
whole-job prefill throughput in tokens/s (B*T tokens per step).  The same JSON
line also carries:
  roofline      the timed prefill call against the HBM roofline (algorithmic bytes:
                Q, K, V read and Y written in bf16, 1,024 B per head-token, plus the
                fp32 state read and written, 2 x 66,048 B per head), and its useful
                MFMA flops against the bf16 dense peak;
  decode        the batched decode workload (65,536 fp32 states seeded by 256
                writes, 1,024 sequential steps) in state-steps/s with its HBM roofline
                (133,120 B per state-step);
  noncausal     la_prefill_noncausal on the ungated prefill shape (every query reads
                the state of the whole sequence), timed the same way, same roofline bytes;
  kv_vs_state   an explicit K/V history (softmax decode over L rows) against the fixed
                recurrent state (one decode step), 8 heads x 64, bf16, L = 512, 2048,
                8192: state bytes, step time, peak memory; also at 128 sequences;
  other         the gated prefill workloads, timed the same way;
  measured_ceilings  what torch's own copy, reduction, fill and bf16 matmul reach on this GPU; the
                prefill and decode rooflines also carry their fraction of the measured stream rate
                for their read/write mix (`frac_of_measured`);
  cpu_baseline  the FP64 oracle timed on this host's cores on a sample of the
                prefill workload.
Run: python bench.py [--gpus 1] [--steps K] [--warmup W]
     python bench.py --only prefill|noncausal|gated|long|decode|delta|kvstate|copy   (one workload, for profiler runs; `copy`
     is a plain 1 GiB device-to-device copy used to calibrate the HBM byte counters)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 matrix (and packed vector) peak
STATE_BYTES = 128 * 128 * 4 + 128 * 4


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.txt")
_BF16_PREFILL = ["prefill_mfma.hip", "prefill_common.hpp", "kernels_general.hip"]
KERNEL_SOURCES = {
    "prefill": _BF16_PREFILL,
    "gated": _BF16_PREFILL,
    "long": _BF16_PREFILL,
    "noncausal": _BF16_PREFILL,
    "fp32": ["prefill_f32.hip", "prefill_common.hpp", "kernels_general.hip"],
    "decode": ["kernels_general.hip"],
    "delta": ["delta_decode.hip"],
}


_T0 = time.perf_counter()


def progress(msg):
    """One line on stderr per finished leg, so that a long run shows where it is."""
    print("[bench %6.1f s] %s" % (time.perf_counter() - _T0, msg), file=sys.stderr, flush=True)


def source_digest(kind):
    """sha256 over the kernel sources of a path; counters taken on other sources are stale."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "recurrent_state_chunkwise_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kind):
    """HBM bytes per call from the committed counter summary, if it matches these sources."""
    try:
        with open(TRAFFIC_FILE, encoding="utf-8") as f:
            for line in f:
                line = line.strip()
                if line.startswith("{"):
                    rec = json.loads(line)
                    if rec.get("kind") == kind and rec.get("source_sha256") == source_digest(kind):
                        return rec["hbm_bytes_per_call"]
    except (OSError, ValueError, KeyError):
        pass
    return None


def prefill_bytes(B, H, T, gated, io_bytes=2):
    # Q, K, V read and Y written (4 x 128 elements per head-token in the io dtype), alpha (fp32)
    # when gated, the fp32 state read and written once per head
    return B * H * T * (512 * io_bytes + (4 if gated else 0)) + 2 * B * H * STATE_BYTES


def prefill_useful_flops(B, H, T, C, d=128, dv=128):
    # per head-token: causal intra-chunk scores and A V ((C+1)(d+dv)), inter-chunk read
    # and state write (4 d dv)
    return B * H * T * ((C + 1) * (d + dv) + 4 * d * dv)


# The clock under load: kernel times change over the first tens of milliseconds of
# back-to-back work, so every timing warms up for at least WARMUP_FLOOR_S of calls and
# every mean per call is taken over at least TIMED_FLOOR_S, whatever --warmup and
# --steps ask for (the timed steps behind `value` are still exactly --steps).
WARMUP_FLOOR_S = 0.040
TIMED_FLOOR_S = 0.025


def run_for(torch, fn, at_least_calls, floor_s):
    """Call fn(0), fn(1), ... back to back: at least `at_least_calls` calls and at least
    `floor_s` seconds of wall time, the device drained before each reading of the clock.
    Returns (calls, seconds)."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n, batch = 0, max(int(at_least_calls), 1)
    while True:
        for i in range(batch):
            fn(n + i)
        n += batch
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        if n >= at_least_calls and el >= floor_s:
            return n, el
        batch = max(1, int((floor_s - el) / (el / n) * 1.1) + 1)


def time_prefill(torch, la, wl, cfg, steps, warmup, sets=2, noncausal=False, phi=None):
    """Time la_prefill_chunked (or la_prefill_noncausal); step i uses input set i % sets.
    Two sets of the ungated workload (2 x 201 MB of Q, K, V) exceed the 256 MB last-level
    cache, so a timed call cannot find its inputs left there by the previous call.
    phi: a feature-map name for la_prefill_chunked_fm (None: la_prefill_chunked, ELU+1).

    Returns a dict:
      total_ms  exactly `steps` steps of state initialisation + call, events only around
                the loop (after a warm-up of at least `warmup` steps and WARMUP_FLOOR_S);
      call_ms   mean time of one call over `call_calls` back-to-back calls (at least
                `steps` and at least TIMED_FLOOR_S) bracketed by events; the state buffers
                carry over from call to call, which leaves the work identical.
    Events are kept out of the loops: each recorded timing event costs several microseconds
    of device time between the kernels it separates."""
    inputs = [wl.prefill_inputs(cfg, "cuda", seed=cfg.seed + 1000 * i) for i in range(sets)]
    Y = torch.empty_like(inputs[0][2])
    S = torch.empty((cfg.B, cfg.H, cfg.d, cfg.dv), device="cuda")
    z = torch.empty((cfg.B, cfg.H, cfg.d), device="cuda")

    def call(i):
        Q, K, V, A = inputs[i % sets]
        if noncausal:
            la.la_prefill_noncausal(Q, K, V, cfg.eps, Y, S, z)
        elif phi is not None:
            la.la_prefill_chunked_fm(Q, K, V, A, cfg.eps, cfg.chunk, Y, S, z, phi=phi)
        else:
            la.la_prefill_chunked(Q, K, V, A, cfg.eps, cfg.chunk, Y, S, z)

    def step(i):
        la.la_state_init(S, z)
        call(i)

    w_calls, w_s = run_for(torch, step, warmup, WARMUP_FLOOR_S)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record()
    for i in range(steps):
        step(i)
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    # the warm-up steps include the state initialisation: 1.5x margin over the call count
    n_calls = max(steps, int(1.5 * TIMED_FLOOR_S / (w_s / w_calls)) + 1)
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record()
    for i in range(n_calls):
        call(i)
    c1.record()
    torch.cuda.synchronize()
    region_ms = c0.elapsed_time(c1)
    del inputs, Y, S, z
    return {"total_ms": total_ms, "call_ms": region_ms / n_calls, "warmup_steps_run": w_calls,
            "warmup_ms": w_s * 1e3, "call_calls": n_calls, "call_region_ms": region_ms}


def time_decode(torch, la, wl, cfg, warmup=10, steps=None):
    N = cfg.n_states
    # seed every state with 256 writes through the prefill path (untimed)
    ks, vs = wl.decode_seed_inputs(cfg, "cuda")
    S = torch.empty((N, 1, cfg.d, cfg.dv), device="cuda")
    z = torch.empty((N, 1, cfg.d), device="cuda")
    la.la_state_init(S, z)
    Ys = torch.empty_like(vs)
    la.la_prefill_chunked(ks, ks, vs, None, cfg.eps, 64, Ys, S, z)
    del ks, vs, Ys
    S, z = S.view(N, cfg.d, cfg.dv), z.view(N, cfg.d)
    steps = cfg.steps if steps is None else steps
    inputs = [wl.decode_step_inputs(cfg, i, "cuda") for i in range(max(steps, warmup))]
    y = torch.empty((N, cfg.dv), device="cuda", dtype=torch.bfloat16)
    Sw, zw = S.clone(), z.clone()

    def warm(i):  # on a scratch copy of the state
        q, k, v = inputs[i % len(inputs)]
        la.la_decode_step(q, k, v, None, cfg.eps, y, Sw, zw)

    run_for(torch, warm, warmup, WARMUP_FLOOR_S)
    del Sw, zw
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        q, k, v = inputs[i]
        la.la_decode_step(q, k, v, None, cfg.eps, y, S, z)
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    call_ms = total_ms / steps  # back-to-back calls, events only around the loop
    del inputs, S, z, y
    return total_ms, call_ms


DELTA_STATE_STEP_BYTES = 2 * 128 * 128 * 4 + 4 * 256 + 4  # S read and written, q k v y bf16, beta


def time_delta(torch, la, wl, cfg, warmup=10, steps=None):
    """Delta-rule decode: `steps` sequential steps over all memories, inputs pre-generated."""
    N = cfg.n_states
    S = wl.delta_seed_state(cfg, "cuda")
    steps = cfg.steps if steps is None else steps
    inputs = [wl.delta_step_inputs(cfg, i, "cuda") for i in range(max(steps, warmup))]
    y = torch.empty((N, cfg.dv), device="cuda", dtype=torch.bfloat16)
    Sw = S.clone()

    def warm(i):  # on a scratch copy of the memories
        q, k, v, b = inputs[i % len(inputs)]
        la.la_delta_decode_step(q, k, v, b, y, Sw)

    run_for(torch, warm, warmup, WARMUP_FLOOR_S)
    del Sw
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        q, k, v, b = inputs[i]
        la.la_delta_decode_step(q, k, v, b, y, S)
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    call_ms = total_ms / steps  # back-to-back calls, events only around the loop
    del inputs, S, y
    return total_ms, call_ms


def time_kv_state(torch, la, wl, cfg):
    """The history path and the state path at each length L, P1's protocol: `warmup` steps,
    then `repeats` steps bracketed by events, mean per step.  Memory: what each path holds
    during its steps (peak over the timed loop) and, for the state path, the peak of
    building the state from the same L-1 earlier rows (a prefill whose outputs are
    discarded)."""
    H, d = cfg.n_heads, cfg.d
    bf16 = torch.bfloat16
    rows = []

    def timed(step_fn, steps):
        """(eager ms, graph ms) per step: P1's protocol with the steps launched one by one
        from Python (at these sizes the launch rate can set the pace), then the same
        `repeats` steps captured once into a HIP graph and replayed (device time)."""
        for i in range(cfg.warmup):
            step_fn(*steps[i])
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(cfg.repeats):
            step_fn(*steps[cfg.warmup + i])
        t1.record()
        torch.cuda.synchronize()
        eager = t0.elapsed_time(t1) / cfg.repeats
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(cfg.repeats):
                step_fn(*steps[cfg.warmup + i])
        graph.replay()
        torch.cuda.synchronize()
        t0.record()
        graph.replay()
        t1.record()
        torch.cuda.synchronize()
        replay = t0.elapsed_time(t1) / cfg.repeats
        del graph
        return eager, replay

    for L in cfg.lengths:
        hk, hv = wl.kv_state_history(cfg, L, "cuda")
        steps = wl.kv_state_steps(cfg, L, cfg.warmup + cfg.repeats, "cuda")
        # explicit history: caches of L rows, the step writes row L-1 and attends over all
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        Kc = torch.empty((H, L, d), device="cuda", dtype=bf16)
        Vc = torch.empty((H, L, d), device="cuda", dtype=bf16)
        Kc[:, :L - 1].copy_(hk)
        Vc[:, :L - 1].copy_(hv)
        y = torch.empty((H, d), device="cuda", dtype=bf16)
        need = la.la_softmax_decode_workspace_bytes(la.LA_BF16, H, L, d)
        ws = torch.empty(max(need, 1), device="cuda", dtype=torch.uint8)
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        hist_ms, hist_graph_ms = timed(
            lambda q, k, v: la.la_softmax_decode_step(q, k, v, L - 1, Kc, Vc, y, workspace=ws), steps)
        hist_peak = torch.cuda.max_memory_allocated() - base
        hist_finite = bool(torch.isfinite(y.float()).all())
        del Kc, Vc, ws, y
        # fixed state: S, z built from the same L-1 rows, then one decode step per call
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        S = torch.empty((H, 1, d, d), device="cuda")
        z = torch.empty((H, 1, d), device="cuda")
        la.la_state_init(S, z)
        Yseed = torch.empty((H, 1, L - 1, d), device="cuda", dtype=bf16)
        hk4, hv4 = hk.view(H, 1, L - 1, d), hv.view(H, 1, L - 1, d)
        la.la_prefill_chunked(hk4, hk4, hv4, None, cfg.eps, 64, Yseed, S, z)
        torch.cuda.synchronize()
        setup_peak = torch.cuda.max_memory_allocated() - base
        # the build itself, timed over 5 more builds from a zero state (device time)
        b0 = torch.cuda.Event(enable_timing=True)
        b1 = torch.cuda.Event(enable_timing=True)
        b0.record()
        for _ in range(5):
            la.la_state_init(S, z)
            la.la_prefill_chunked(hk4, hk4, hv4, None, cfg.eps, 64, Yseed, S, z)
        b1.record()
        torch.cuda.synchronize()
        build_ms = b0.elapsed_time(b1) / 5
        del Yseed
        S2, z2 = S.view(H, d, d), z.view(H, d)
        y = torch.empty((H, d), device="cuda", dtype=bf16)
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        state_ms, state_graph_ms = timed(lambda q, k, v: la.la_decode_step(q, k, v, None, cfg.eps, y, S2, z2), steps)
        state_peak = torch.cuda.max_memory_allocated() - base
        state_finite = bool(torch.isfinite(y.float()).all())
        del S, z, S2, z2, y, hk, hv, hk4, hv4, steps
        hist_bytes = 2 * H * L * d * 2
        state_bytes = H * (d * d + d) * 4
        rows.append({
            "L": L, "history_bytes": hist_bytes, "state_bytes": state_bytes,
            "history_step_ms": hist_ms, "state_step_ms": state_ms, "state_over_history_time": state_ms / hist_ms,
            "history_step_ms_graph": hist_graph_ms, "state_step_ms_graph": state_graph_ms,
            "state_over_history_time_graph": state_graph_ms / hist_graph_ms,
            "history_peak_bytes": hist_peak, "state_peak_bytes": state_peak, "state_setup_peak_bytes": setup_peak,
            "state_build_ms": build_ms,
            "state_build_variant": la.la_prefill_variant(la.LA_BF16, d, d, 64, False, la.LA_F32),
            "history_read_GBps_graph": hist_bytes / (hist_graph_ms / 1e3) / 1e9,
            "finite": hist_finite and state_finite,
        })
    return {"workload": cfg.name, "heads": H, "d": d, "dtype": "bf16",
            "protocol": "warmup %d, repeats %d, events around the repeats, mean per step; *_graph: the same "
                        "repeats captured in one HIP graph and replayed" % (cfg.warmup, cfg.repeats),
            "rows": rows}


def measured_ceilings(torch, reps=10):
    """What this GPU reaches on plain streams and a dense product, with torch's own kernels:
    a 1:1 device copy, a read-only reduction and a fill over 4 GiB, and an 8192^3 bf16 matmul.
    Rates are per second of device time between events around `reps` repetitions."""
    n = 1 << 30  # fp32 elements: 4 GiB
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    out = torch.empty((), device="cuda")

    def timed(fn):
        for _ in range(3):
            fn()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / 1e3 / reps

    nb = 4 * n
    rows = torch.empty(n // 4096, device="cuda")
    # the faster of two kernels each for the copy and the read-only stream
    copy_s = min(timed(lambda: dst.copy_(src)), timed(lambda: torch.mul(src, 1.0, out=dst)))
    read_s = min(timed(lambda: torch.sum(src, 0, out=out)),
                 timed(lambda: torch.sum(src.view(-1, 4096), 1, out=rows)))
    write_s = timed(lambda: dst.fill_(2.0))
    del rows
    del src, dst
    m = 8192
    a = torch.randn((m, m), device="cuda").to(torch.bfloat16)
    b = torch.randn((m, m), device="cuda").to(torch.bfloat16)
    c = torch.empty((m, m), device="cuda", dtype=torch.bfloat16)
    gemm_s = timed(lambda: torch.matmul(a, b, out=c))
    del a, b, c
    torch.cuda.empty_cache()
    return {
        "copy_GBps": 2 * nb / copy_s / 1e9,  # bytes read + written
        "read_GBps": nb / read_s / 1e9,
        "write_GBps": nb / write_s / 1e9,
        "gemm_bf16_TFLOPs": 2.0 * m ** 3 / gemm_s / 1e12,
        "method": "torch kernels on 4 GiB fp32 (copy: the faster of copy_ and mul by 1; read: the faster of a "
                  "full sum and a sum of 4096-element rows; write: fill_) and an 8192^3 bf16 matmul, %d "
                  "repetitions each after 3 untimed" % reps,
    }


def mix_ceiling(ceil, read_bytes, write_bytes):
    """Rate of a stream with these read and write bytes if its reads ran at the measured
    read-only rate and its writes at the measured write-only rate, one after the other."""
    t = read_bytes / ceil["read_GBps"] + write_bytes / ceil["write_GBps"]
    return (read_bytes + write_bytes) / t


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _time_oracle(fn, min_s=0.5, max_reps=5):
    """Mean wall seconds of fn() over repeats until about min_s (at least one, at most max_reps)."""
    reps, t0 = 0, time.perf_counter()
    while reps < max_reps and (reps == 0 or time.perf_counter() - t0 < min_s):
        fn()
        reps += 1
    return (time.perf_counter() - t0) / reps, reps


def cpu_baseline(wl, torch):
    """The FP64 oracle on this host's cores (one GPU's share: at most 16 threads), on the
    workloads or bounded samples of them, inputs drawn on the host with the same recipes.
    The headline entry is the ungated prefill workload in full; `configs` times every
    workload, with the decode and long-sequence ones on samples and their full-workload
    times extrapolated (states and heads are independent) and labelled as such."""
    import numpy as np
    import oracle
    threads = min(16, len(os.sched_getaffinity(0)))
    f64 = lambda t: t.to(torch.float64).numpy()
    rows = []

    def prefill_row(cfg, heads_total, H_sample, label):
        Q, K, V, A = wl.prefill_inputs(cfg, "cpu", B=1, H=H_sample)
        q, k, v = f64(Q), f64(K), f64(V)
        a = None if A is None else f64(A)
        th = min(threads, H_sample)
        dt, reps = _time_oracle(lambda: oracle.recurrence_heads(q, k, v, a, eps=cfg.eps, threads=th))
        rate = H_sample * cfg.T / dt  # head-tokens/s
        row = {"workload": cfg.name, "sample": label, "threads": th, "runs": reps, "seconds_per_run": dt,
               "head_tokens_per_s": rate}
        if H_sample < heads_total:
            # the remaining heads run on the same threads, th at a time
            full = dt * heads_total / H_sample * th / min(threads, heads_total)
            row["full_workload_seconds_extrapolated"] = full
        else:
            full = row["full_workload_seconds"] = dt
        row["tokens_per_s"] = cfg.B * cfg.T / full  # of the whole workload, on `threads` threads
        return row

    cfg2 = wl.PREFILL_UNGATED
    rows.append(prefill_row(wl.SINGLE_HEAD_F64, 1, 1, "the whole workload (1 head x 64 tokens, fp64)"))
    rows.append(prefill_row(cfg2, cfg2.B * cfg2.H, cfg2.B * cfg2.H, "the whole workload (64 heads x 4096 tokens)"))
    g3 = wl.PREFILL_GATED
    rows.append(prefill_row(g3, g3.B * g3.H, g3.B * g3.H, "the whole workload (32 heads x 16384 tokens)"))
    g5 = wl.PREFILL_LONG
    rows.append(prefill_row(g5, g5.B * g5.H, 4, "4 of the 32 heads x 131072 tokens (extrapolated to 32 heads)"))
    # decode: 2048 states seeded by 256 writes (untimed), then 128 of the 1024 steps timed
    dcfg = wl.DECODE
    n_s, n_steps = 2048, 128
    ks, vs = wl.decode_seed_inputs(dcfg, "cpu", n_states=n_s)
    _, S0, z0, _ = oracle.recurrence_heads(f64(ks), f64(ks), f64(vs), eps=dcfg.eps, threads=threads)
    steps = [wl.decode_step_inputs(dcfg, i, "cpu", n_states=n_s) for i in range(n_steps)]
    st = lambda j: np.stack([f64(x[j]) for x in steps], axis=1)[:, None]
    q, k, v = st(0), st(1), st(2)
    dt, reps = _time_oracle(lambda: oracle.recurrence_heads(q, k, v, eps=dcfg.eps, S0=S0[:, None], z0=z0[:, None],
                                                            threads=threads))
    rate = n_s * n_steps / dt
    rows.append({"workload": dcfg.name, "sample": "2048 of the 65536 states x 128 of the 1024 steps, from states "
                 "seeded by 256 writes (extrapolated to the whole workload)", "threads": threads, "runs": reps,
                 "seconds_per_run": dt, "state_steps_per_s": rate,
                 "full_workload_seconds_extrapolated": dcfg.n_states * dcfg.steps / rate})
    main_row = rows[1]
    return {
        "value": main_row["tokens_per_s"],
        "unit": "tokens/s",
        "cores": main_row["threads"],
        "kind": "oracle",
        "sample": "all 64 heads x 4096 tokens of the B=4,H=16,T=4096 ungated workload, %d runs of %.2f s wall "
                  "(inputs drawn on the host); tokens/s = head-tokens/s / H" % (main_row["runs"],
                                                                             main_row["seconds_per_run"]),
        "cpu_model": cpu_model(),
        "threads_available": len(os.sched_getaffinity(0)),
        "configs": rows,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the decode and gated workloads")
    ap.add_argument("--only", choices=["prefill", "noncausal", "gated", "long", "fp32", "decode", "delta", "kvstate",
                                       "copy"],
                    default=None,
                    help="run one workload only and print its timing (for profiler runs)")
    ap.add_argument("--decode-steps", type=int, default=None,
                    help="steps to time with --only decode or --only delta (default: the workload's)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the data-parallel step shards by sequence with no communication); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import recurrent_state_chunkwise_amd as la
    from recurrent_state_chunkwise_amd import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    la.library()
    if args.only == "copy":
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"only": "copy", "bytes_read_per_copy": n, "bytes_written_per_copy": n, "copies": 5}))
        return
    if args.only == "decode":
        steps = args.decode_steps or wl.DECODE.steps
        d_total, d_call = time_decode(torch, la, wl, wl.DECODE, steps=steps)
        print(json.dumps({"only": "decode", "steps": steps, "ms_per_step": d_total / steps, "call_ms": d_call}))
        return
    if args.only == "delta":
        steps = args.decode_steps or wl.DELTA_DECODE.steps
        d_total, d_call = time_delta(torch, la, wl, wl.DELTA_DECODE, steps=steps)
        print(json.dumps({"only": "delta", "steps": steps, "ms_per_step": d_total / steps, "call_ms": d_call}))
        return
    if args.only == "kvstate":
        print(json.dumps({"only": "kvstate", "kv_vs_state": time_kv_state(torch, la, wl, wl.KV_STATE),
                          "kv_vs_state_batched": time_kv_state(torch, la, wl, wl.KV_STATE_BATCHED)}))
        return
    if args.only in ("gated", "long", "fp32"):
        ocfg = {"gated": wl.PREFILL_GATED, "long": wl.PREFILL_LONG, "fp32": wl.PREFILL_UNGATED_F32}[args.only]
        r = time_prefill(torch, la, wl, ocfg, args.steps, args.warmup)
        print(json.dumps({"only": args.only, "workload": ocfg.name, "steps": args.steps,
                          "ms_per_step": r["total_ms"] / args.steps, **r}))
        return
    cfg = wl.PREFILL_UNGATED
    if args.only == "noncausal":
        r = time_prefill(torch, la, wl, cfg, args.steps, args.warmup, noncausal=True)
        print(json.dumps({"only": "noncausal", "steps": args.steps, "ms_per_step": r["total_ms"] / args.steps,
                          **r}))
        return
    torch.cuda.synchronize()
    main_t = time_prefill(torch, la, wl, cfg, args.steps, args.warmup)
    total_ms, call_ms = main_t["total_ms"], main_t["call_ms"]
    progress("ungated prefill timed")
    # the same call on one input set, whose inputs may stay in the last-level cache (reported only)
    warm_call_ms = None
    if args.only is None:
        warm_call_ms = time_prefill(torch, la, wl, cfg, args.steps, args.warmup, sets=1)["call_ms"]
    ms_per_step = total_ms / args.steps
    tokens = cfg.B * cfg.T
    value = tokens * args.steps / (total_ms / 1e3)
    nbytes = prefill_bytes(cfg.B, cfg.H, cfg.T, cfg.gated)
    flops = prefill_useful_flops(cfg.B, cfg.H, cfg.T, cfg.chunk)
    achieved = nbytes / (call_ms / 1e3) / 1e9
    out = {
        "metric": "prefill tokens/s + %MFMA peak; decode state-steps/s + %HBM GB/s",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "timing": {"warmup_steps_run": main_t["warmup_steps_run"], "warmup_ms": main_t["warmup_ms"],
                   "timed_steps": args.steps, "timed_ms": total_ms,
                   "call_ms_calls": main_t["call_calls"], "call_ms_region_ms": main_t["call_region_ms"],
                   "floors": "warm-up until >= %d ms of back-to-back steps (and >= --warmup steps); call_ms "
                             "over >= %d ms of back-to-back calls (and >= --steps calls)"
                             % (WARMUP_FLOOR_S * 1e3, TIMED_FLOOR_S * 1e3)},
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "H": cfg.H, "T": cfg.T, "d": cfg.d, "dv": cfg.dv,
                   "chunk": cfg.chunk, "gated": cfg.gated, "eps": cfg.eps, "state": "fp32",
                   "input_sets": 2, "parallelism": "single GPU"},
        "roofline": {
            "kernel": "la_prefill_chunked (segment maps + scan + chunked prefill)",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic("prefill"),
            "call_ms": call_ms,
            "warm_call_ms": warm_call_ms,
            "algorithmic_bytes": nbytes,
            "useful_mfma_tflops": flops / (call_ms / 1e3) / 1e12,
            "mfma_frac": flops / (call_ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS,
        },
    }
    if args.only == "prefill":
        print(json.dumps(out), flush=True)
        return
    if not args.no_extra:
        dcfg = wl.DECODE
        d_total, d_call = time_decode(torch, la, wl, dcfg)
        progress("decode timed")
        d_bytes = dcfg.n_states * (2 * STATE_BYTES + 3 * 256 + 256)
        out["decode"] = {
            "workload": dcfg.name, "steps": dcfg.steps,
            "value": dcfg.n_states * dcfg.steps / (d_total / 1e3), "unit": "state-steps/s",
            "ms_per_step": d_total / dcfg.steps,
            "roofline": {"kernel": "la_decode_step", "bound": "hbm",
                         "achieved": d_bytes / (d_call / 1e3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": d_bytes / (d_call / 1e3) / 1e9 / HBM_PEAK_GBS,
                         "traffic": measured_traffic("decode"),
                         "call_ms": d_call, "algorithmic_bytes": d_bytes},
        }
        xcfg = wl.DELTA_DECODE
        x_total, x_call = time_delta(torch, la, wl, xcfg)
        progress("delta-rule decode timed")
        x_bytes = xcfg.n_states * DELTA_STATE_STEP_BYTES
        out["delta_decode"] = {
            "workload": xcfg.name, "steps": xcfg.steps,
            "value": xcfg.n_states * xcfg.steps / (x_total / 1e3), "unit": "state-steps/s",
            "ms_per_step": x_total / xcfg.steps,
            "roofline": {"kernel": "la_delta_decode_step", "bound": "hbm",
                         "achieved": x_bytes / (x_call / 1e3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": x_bytes / (x_call / 1e3) / 1e9 / HBM_PEAK_GBS,
                         "traffic": measured_traffic("delta"),
                         "call_ms": x_call, "algorithmic_bytes": x_bytes},
        }
        n_call = time_prefill(torch, la, wl, cfg, args.steps, args.warmup, noncausal=True)["call_ms"]
        progress("non-causal form timed")
        out["noncausal"] = {
            "workload": "noncausal_" + cfg.name, "value": tokens / (n_call / 1e3), "unit": "tokens/s",
            "roofline": {"kernel": "la_prefill_noncausal (segment sums + read-out)", "bound": "hbm",
                         "achieved": nbytes / (n_call / 1e3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": nbytes / (n_call / 1e3) / 1e9 / HBM_PEAK_GBS,
                         "traffic": measured_traffic("noncausal"),
                         "call_ms": n_call, "algorithmic_bytes": nbytes},
        }
        # the other feature maps on the same call (template instantiations of the same kernels)
        out["feature_maps"] = {"workload": cfg.name, "unit": "ms per call", "elu1": call_ms}
        for fm in ("relu1", "relu_eps", "sigmoid_eps"):
            out["feature_maps"][fm] = time_prefill(torch, la, wl, cfg, args.steps, args.warmup, phi=fm)["call_ms"]
        progress("feature maps timed")
        out["kv_vs_state"] = time_kv_state(torch, la, wl, wl.KV_STATE)
        out["kv_vs_state_batched"] = time_kv_state(torch, la, wl, wl.KV_STATE_BATCHED)
        progress("history-against-state comparison timed")
        other = []
        for kind, ocfg in (("gated", wl.PREFILL_GATED), ("long", wl.PREFILL_LONG)):
            o_call = time_prefill(torch, la, wl, ocfg, args.steps, args.warmup)["call_ms"]
            ob = prefill_bytes(ocfg.B, ocfg.H, ocfg.T, ocfg.gated)
            of = prefill_useful_flops(ocfg.B, ocfg.H, ocfg.T, ocfg.chunk)
            other.append({"workload": ocfg.name, "value": ocfg.B * ocfg.T / (o_call / 1e3), "unit": "tokens/s",
                          "call_ms": o_call, "hbm_frac": ob / (o_call / 1e3) / 1e9 / HBM_PEAK_GBS,
                          "mfma_frac": of / (o_call / 1e3) / 1e12 / BF16_PEAK_TFLOPS,
                          "algorithmic_bytes": ob, "traffic": measured_traffic(kind)})
            progress("%s timed" % ocfg.name)
        # the fp32-input path on the ungated shape: its useful flops at the fp32 matrix peak
        # take longer than its bytes at the HBM peak, so that is its roofline
        fcfg = wl.PREFILL_UNGATED_F32
        f_call = time_prefill(torch, la, wl, fcfg, args.steps, args.warmup, sets=1)["call_ms"]
        fb = prefill_bytes(fcfg.B, fcfg.H, fcfg.T, fcfg.gated, io_bytes=4)
        ff = prefill_useful_flops(fcfg.B, fcfg.H, fcfg.T, fcfg.chunk)
        other.append({"workload": fcfg.name, "value": fcfg.B * fcfg.T / (f_call / 1e3), "unit": "tokens/s",
                      "call_ms": f_call, "dtype": "f32",
                      "roofline": {"bound": "mfma", "achieved": ff / (f_call / 1e3) / 1e12, "peak": FP32_PEAK_TFLOPS,
                                   "unit": "TFLOP/s", "frac": ff / (f_call / 1e3) / 1e12 / FP32_PEAK_TFLOPS,
                                   "hbm_frac": fb / (f_call / 1e3) / 1e9 / HBM_PEAK_GBS,
                                   "algorithmic_bytes": fb, "useful_flops": ff,
                                   "traffic": measured_traffic("fp32")}})
        out["other"] = other
        progress("fp32-input prefill timed")
    if not args.no_extra:
        ceil = measured_ceilings(torch)
        out["measured_ceilings"] = ceil
        # the prefill moves its algorithmic bytes as reads of Q, K, V (+ state) and writes of Y (+ state)
        pr = cfg.B * cfg.H * (cfg.T * 768 + STATE_BYTES)
        pw = cfg.B * cfg.H * (cfg.T * 256 + STATE_BYTES)
        m = mix_ceiling(ceil, pr, pw)
        out["roofline"]["measured_ceiling_GBps"] = m
        out["roofline"]["frac_of_measured"] = achieved / m
        out["decode"]["roofline"]["measured_ceiling_GBps"] = ceil["copy_GBps"]
        out["decode"]["roofline"]["frac_of_measured"] = out["decode"]["roofline"]["achieved"] / ceil["copy_GBps"]
    if not args.no_cpu_baseline:
        progress("timing the oracle on the host")
        out["cpu_baseline"] = cpu_baseline(wl, torch)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
