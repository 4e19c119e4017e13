#!/usr/bin/env python3
"""Benchmark of the SANATAN p=1 attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extras]

A step is one chunked causal prefill (phase table, featurize, intra-chunk product, inter-chunk
readout, state update, boundary scan, normalisation) over the B=8, H=12, T=2048, d=64 bf16
workload with chunk 64; its throughput in tokens/s (B*T tokens per step) is `value`.
Decode (12 layers x 12 heads of fp32 state, batch 1 and 64), the long prefill (B=1, H=12,
T=32768, chunk 128) and the p=2 quadratic form (B=4, H=12, T=4096) are timed after it and
reported in `extras`.  Inputs are seeded synthetic N(0,1) values (sanatan_inputs), resident in
HBM before timing starts.  Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
D, DV, F = 64, 64, 384
STATE_BYTES = (F * DV + F) * 4


def prefill_flops(B, H, T, C, causal=True):
    """Algorithmic FLOPs (multiply-add = 2) of the chunked p=1 prefill."""
    per_head = 0
    for c0 in range(0, T, C):
        n = min(C, T - c0)
        pairs = n * (n + 1) // 2 if causal else n * n
        per_head += 2 * pairs * (F + DV)          # A = Phi(Q) Phi(K)^T over s <= t, then A V
        per_head += 2 * n * F * DV * 2            # readout Phi(Q) S and update Phi(K)^T V
    return B * H * per_head


def prefill_bytes(B, H, T, el=2):
    return B * H * T * (3 * D * el + DV * el)   # q, k, v in; out


def quadratic_flops(B, H, T, features=F):
    """Causal pairs x (score over the features + weighted value sum); features = 4d for the four-channel kernel."""
    pairs = T * (T + 1) // 2
    return B * H * pairs * 2 * (features + DV)


PREFILL_SOURCES = ("api.hip", "featurize.hip", "prefill.hip", "prefill_grp.hip", "prefill_common.h", "launchers.h",
                   "sanatan_device.h")
PREFILL_KERNELS = ("phase_table_kernel", "prefill_grp_kernel", "prefill_grp128_kernel", "prefill_state8_kernel", "prefill_scan_kernel",
                   "prefill4_kernel")
CAL_BYTES = 256 << 20       # plain device copy used to calibrate the memory counters


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "root_parity_gated_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel_key, src_hash):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they match the current source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path)).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


def _counter_rows(d):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    return rows


def traffic_summary(fetch_dir, write_dir, key):
    """Per-call HBM bytes of the prefill from two rocprofv3 --pmc runs of `bench.py --calibrate-copy`
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each scaled so that the calibration copy of
    CAL_BYTES reads / writes exactly CAL_BYTES.  Writes profiles/traffic.json[key]."""
    out = {}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _counter_rows(d) if r["Counter_Name"] == name]
        # the calibration copies are the run's first three copy dispatches (workloads may copy buffers later)
        cal_rows = sorted((r for r in rows if "copyBuffer" in r["Kernel_Name"]), key=lambda r: int(r["Dispatch_Id"]))
        cal = [float(r["Counter_Value"]) for r in cal_rows[:3]]
        if not cal:
            raise SystemExit(f"no calibration copy found in {d}")
        scale = CAL_BYTES / (max(cal) * 1024.0)
        per_kernel = {}
        for r in rows:
            kn = r["Kernel_Name"]
            hit = next((k for k in PREFILL_KERNELS if k in kn), None)
            if hit is None:
                continue
            m = re.search(r"(\w+_kernel(<[^>]*>)?)", kn)
            label = m.group(1) if m else kn
            per_kernel.setdefault(label, []).append(float(r["Counter_Value"]) * 1024.0 * scale)
        calls = len(per_kernel.get("phase_table_kernel", [])) or max(len(v) for v in per_kernel.values())
        out[name] = {"scale": scale, "calibration_kib": max(cal),
                     "per_kernel_bytes_avg": {k: sum(v) / len(v) for k, v in per_kernel.items()},
                     "bytes_per_call": sum(sum(v) for v in per_kernel.values()) / calls}
    rec = {"source_hash": source_hash(*PREFILL_SOURCES),
           "bytes_per_launch": out["FETCH_SIZE"]["bytes_per_call"] + out["WRITE_SIZE"]["bytes_per_call"],
           "fetch": out["FETCH_SIZE"], "write": out["WRITE_SIZE"]}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        allrec = json.load(open(path))
    except (OSError, ValueError):
        allrec = {}
    allrec[key] = rec
    with open(path, "w") as f:
        json.dump(allrec, f, indent=1, sort_keys=True)
    print(json.dumps(rec, indent=1))


def log(msg):
    print(f"# {msg}", file=sys.stderr, flush=True)


def timed_loop(torch, fn, steps, warmup):
    """Run fn warmup times, then time `steps` calls with HIP events on the current stream (the stream the
    library launches on), bracketed by device synchronisations.  Returns ms per call."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(steps):
        fn()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def per_call_ms(torch, fn, steps):
    """Each of `steps` calls timed on its own (an event pair around every call, on the current stream);
    returns (median, mean) in ms.  Used beside timed_loop's whole-loop figure."""
    st = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record(st)
        fn()
        b.record(st)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    return ms[len(ms) // 2] if len(ms) % 2 else 0.5 * (ms[len(ms) // 2 - 1] + ms[len(ms) // 2]), sum(ms) / len(ms)


def graph_of(torch, fn):
    """One call of fn captured as a HIP graph (replayed on the current stream); None if capture fails."""
    try:
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=torch.cuda.Stream()):
            fn()
        torch.cuda.synchronize()
        return g
    except Exception as ex:  # the eager timing stands on its own
        log(f"graph capture skipped: {ex}")
        return None


def host_cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, budget_s=8.0):
    """The fp64 oracle (recurrent form, all host threads) on a bounded sample of the prefill workload, timed
    three times (the median is reported)."""
    import oracle
    import sanatan_inputs as si

    q, k, v, om = si.workload_inputs(w)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    # calibrate on one head, then size the sample to roughly `budget_s`
    t0 = time.perf_counter()
    oracle.recurrent(q[0, 0, :256], k[0, 0, :256], v[0, 0, :256], om[0])
    per_head_tok = (time.perf_counter() - t0) / 256
    nth = oracle.num_threads()
    n_heads = int(round(budget_s * nth / (per_head_tok * w.T)))
    n_heads = max(1, min(len(heads), n_heads))
    sel = heads[:n_heads]
    qs = np.stack([q[b, h] for b, h in sel])
    ks = np.stack([k[b, h] for b, h in sel])
    vs = np.stack([v[b, h] for b, h in sel])
    oms = np.stack([om[h] for _, h in sel])
    runs = []
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.recurrent_heads(qs, ks, vs, oms)
        runs.append(time.perf_counter() - t0)
    dt = sorted(runs)[1]
    tokens = n_heads * w.T / w.H  # a token carries H heads
    return {"value": tokens / dt, "unit": "tokens/s", "cores": nth, "kind": "oracle", "cpu_model": host_cpu_model(),
            "sample": f"recurrent fp64 oracle over {n_heads} of {len(heads)} (b,h) sequences x {w.T} tokens, "
                      f"median of 3 runs ({', '.join(f'{r:.1f}' for r in runs)} s wall)"}


def cpu_oracle_extras(si):
    """The fp64 oracle timed beside the other workloads, each on a bounded sample (a few seconds at most):
    the recurrent form for decode and the long prefill, the direct-kappa form for the p=2 quadratic."""
    import oracle

    nth = oracle.num_threads()
    res = {}
    # decode: 144 head-states, 128 tokens from an empty state (the per-token cost does not depend on the fill)
    w = si.DECODE
    steps = 128
    om, _, (sq, sk, sv) = si.decode_inputs_numpy(w.seed, w.H, 1, steps)
    t0 = time.perf_counter()
    oracle.recurrent_heads(sq.transpose(1, 0, 2), sk.transpose(1, 0, 2), sv.transpose(1, 0, 2), om, pos0=w.T)
    dt = time.perf_counter() - t0
    res["decode"] = {"value": dt / steps * 1e6, "unit": "us/token", "cores": nth, "kind": "oracle",
                     "sample": f"recurrent fp64 oracle, {w.H} head-states x {steps} tokens ({dt:.2f} s wall)"}
    # long prefill: the recurrence over every head and the first 4096 tokens (cost per token is constant)
    w = si.LONG
    n_tok = min(w.T, 4096)
    q, k, v, om = si.attention_inputs(w.seed, 1, w.H, n_tok, "bf16")
    t0 = time.perf_counter()
    oracle.recurrent_heads(q[0], k[0], v[0], om, want_out=True)
    dt = time.perf_counter() - t0
    res["long_prefill"] = {"value": n_tok / dt, "unit": "tokens/s", "cores": nth, "kind": "oracle",
                           "sample": f"recurrent fp64 oracle, {w.H} heads x the first {n_tok} of {w.T} tokens "
                                     f"({dt:.2f} s wall)"}
    # the headline prefill in its direct-kappa form: 128 query rows spread over one head, extrapolated by pairs
    w = si.PREFILL
    q, k, v, om = si.attention_inputs(w.seed, 1, 1, w.T, "bf16")
    rows = np.linspace(0, w.T - 1, 128).astype(np.int64)
    pairs = float((rows + 1).sum())
    t0 = time.perf_counter()
    oracle.attention_direct(q[0, 0], k[0, 0], v[0, 0], om[0], p=1, rows=rows)
    dt = time.perf_counter() - t0
    full_s = dt / pairs * (w.B * w.H * w.T * (w.T + 1) / 2)
    res["prefill_direct_kappa"] = {
        "value": w.B * w.T / full_s, "unit": "tokens/s", "cores": nth, "kind": "oracle",
        "sample": f"direct-kappa fp64 oracle, {rows.size} query rows of one head ({int(pairs)} pairs, {dt:.2f} s "
                  f"wall), extrapolated by causal pairs to the whole headline workload"}
    # quadratic p=2: direct kappa on 256 query rows spread over one head, extrapolated by causal pairs
    w = si.QUAD_P2
    q, k, v, om = si.attention_inputs(w.seed, 1, 1, w.T, "bf16")
    rows = np.linspace(0, w.T - 1, 256).astype(np.int64)
    pairs = float((rows + 1).sum())
    t0 = time.perf_counter()
    oracle.attention_direct(q[0, 0], k[0, 0], v[0, 0], om[0], p=w.p, rows=rows)
    dt = time.perf_counter() - t0
    full_s = dt / pairs * (w.B * w.H * w.T * (w.T + 1) / 2)
    res["quadratic_p2"] = {"value": w.B * w.T / full_s, "unit": "tokens/s", "cores": nth, "kind": "oracle",
                           "sample": f"direct-kappa fp64 oracle, {rows.size} query rows of one head ({int(pairs)} pairs, "
                                     f"{dt:.2f} s wall), extrapolated by causal pairs to the whole workload"}
    return res


def bench_decode(torch, rpg, si, batch, steps_timed, warmup, positions=False, compact=False):
    """fp32 decode: 144 head-states per sequence, state filled by 4096 tokens, then sequential steps.
    With `positions`, each sequence continues at its own position (4096 plus a seeded offset below 4096)
    through the per-head-state entry point; the position arrays of every step are built before timing.
    With `compact`, the filled state is converted to the compact layout ((5d+1) rows: the d equal channel-0
    rows kept once) and the compact decode is timed on its own bytes."""
    w = si.DECODE
    nh, fill = w.H, w.T
    N = batch * nh
    if batch == 1:
        om, (fq, fk, fv), (sq, sk, sv) = si.decode_inputs_numpy(w.seed, nh, fill, steps_timed + warmup)
        dv = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
        fq, fk, fv, sq, sk, sv = map(dv, (fq, fk, fv, sq, sk, sv))
    else:
        om, (fq, fk, fv), (sq, sk, sv) = si.decode_inputs_torch(w.seed + batch, batch, nh, fill,
                                                                steps_timed + warmup, "cuda")
    p = rpg.Params(omega=torch.from_numpy(om).cuda())
    S = torch.zeros((N, F, DV), device="cuda")
    z = torch.zeros((N, F), device="cuda")
    # fill the state with the chunked prefill (fp32), in slices of sequences
    sl = 1152
    for i in range(0, N, sl):
        j = min(N, i + sl)
        rpg.sanatan_prefill_chunked(fq[i:j].unsqueeze(0), fk[i:j].unsqueeze(0), fv[i:j].unsqueeze(0), 64,
                                    rpg.Params(omega=p.omega), S=S[i:j].unsqueeze(0), z=z[i:j].unsqueeze(0))
    del fq, fk, fv
    if compact:
        S, z = rpg.sanatan_state_compact(S, z)
        torch.cuda.synchronize()
    out = torch.empty((N, DV), device="cuda")
    posv = None
    if positions:
        seq_off = np.repeat(si.decode_positions(w.seed + 7 * batch, batch, 0, fill), nh)
        posv = torch.from_numpy(fill + seq_off[None, :] + np.arange(steps_timed + warmup)[:, None]).cuda()

    def dec(i, S_, z_):
        if compact:
            rpg.sanatan_decode_step_compact(sq[i], sk[i], sv[i], fill + i if posv is None else posv[i], p, S_, z_,
                                            out)
        elif posv is None:
            rpg.sanatan_decode_step(sq[i], sk[i], sv[i], fill + i, p, S_, z_, out)
        else:
            rpg.sanatan_decode_step_positions(sq[i], sk[i], sv[i], posv[i], p, S_, z_, out)

    torch.cuda.synchronize()
    step = [0]

    def one():
        dec(step[0], S, z)
        step[0] += 1

    ms = timed_loop(torch, one, steps_timed, warmup)
    # graph-replayed variant: the same steps captured once (launch overhead removed)
    g_ms = None
    try:
        S2, z2 = S.clone(), z.clone()
        gstream = torch.cuda.Stream()
        graph = torch.cuda.CUDAGraph()
        n_cap = min(steps_timed, 256)
        with torch.cuda.graph(graph, stream=gstream):
            for i in range(n_cap):
                dec(i, S2, z2)
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        g_ms = e0.elapsed_time(e1) / n_cap
    except Exception as ex:  # graph capture is an optional view of the same kernel
        g_ms = None
        print(f"# decode graph capture skipped: {ex}", file=sys.stderr)
    state_bytes = rpg.sanatan_compact_state_bytes(D, DV) if compact else STATE_BYTES
    bytes_step = N * (2 * state_bytes + 3 * D * 4 + DV * 4)
    best_ms = min(ms, g_ms) if g_ms else ms
    # reference for what an in-place read-and-write-back stream of the same state bytes reaches on this
    # device: torch's vectorized in-place add over the state tensor (one read and one write per element)
    ref_tbs = None
    if batch > 1:
        flat = S.view(-1)
        ref_ms = timed_loop(torch, lambda: flat.add_(0.0), 10, 2)
        ref_tbs = 2 * flat.numel() * 4 / (ref_ms * 1e-3) / 1e12
    return {
        "batch": batch, "head_states": N, "steps": steps_timed,
        "us_per_step_eager": ms * 1e3, "us_per_step_graph": (g_ms * 1e3) if g_ms else None,
        "us_per_token": best_ms * 1e3 / batch,
        "bytes_per_step": bytes_step,
        "roofline": {"bound": "hbm", "achieved": bytes_step / (best_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": bytes_step / (best_ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
        "note": ("state (14.4 MB, 12.0 MB compact) is resident in the 256 MB Infinity Cache between steps"
                 if batch == 1
                 else "state exceeds the Infinity Cache; HBM-bound")
                + ("; one position per sequence (sanatan_decode_step_positions)" if positions else "")
                + ("; compact state, (5d+1) x (d_v+1) floats per head-state: roofline on its own bytes, not on"
                   " the 6d state's" if compact else ""),
        "rmw_stream_reference_TBps": ref_tbs,
    }


def bench_prefill_like(torch, rpg, si, w, steps, warmup, quadratic=False, four_channel=False, per_call=None,
                       train=False):
    """ms per call: (eager, graph-replayed).  Each call is one complete library call on resident inputs;
    the graph variant replays that call captured once, which removes the host launch overhead."""
    q, k, v, om = si.workload_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    qd, kd, vd = (torch.from_numpy(x).cuda().to(dt) for x in (q, k, v))
    del q, k, v
    p = rpg.Params(omega=torch.from_numpy(om).cuda(), gamma=w.gamma, eps=w.eps, lambda_base=w.lambda_base)
    out = torch.empty_like(vd)
    if quadratic:
        code = rpg.SANATAN_BF16 if w.dtype == "bf16" else rpg.SANATAN_F32
        ws = torch.empty((rpg.sanatan_quadratic_workspace_bytes(w.B, w.H, w.T, code, p),), dtype=torch.uint8,
                         device="cuda")
        if train:  # the training forward: also saves the backward pass's statistics
            saved = torch.empty((rpg.lib().sanatan_quadratic_saved_bytes(w.B, w.H, w.T, None) // 4,),
                                dtype=torch.float32, device="cuda")
            fn = lambda: rpg.sanatan_quadratic_train(qd, kd, vd, w.p, p, out=out, saved=saved, ws=ws)
        else:
            fn = lambda: rpg.sanatan_quadratic_ref_p2(qd, kd, vd, w.p, p, out=out, ws=ws, four_channel=four_channel)
    else:
        ws = torch.empty((rpg.sanatan_prefill_workspace_bytes(w.B, w.H, w.T, w.chunk, p),), dtype=torch.uint8,
                         device="cuda")
        fn = lambda: rpg.sanatan_prefill_chunked(qd, kd, vd, w.chunk, p, out=out, ws=ws)
    eager = timed_loop(torch, fn, steps, warmup)
    if per_call is not None:  # each call timed on its own as well: median and mean
        per_call["median"], per_call["mean"] = per_call_ms(torch, fn, steps)
    g = graph_of(torch, fn)
    graph = timed_loop(torch, g.replay, steps, warmup) if g is not None else None
    return eager, graph


def backward_flops(B, H, T):
    """Algorithmic FLOPs of the attention backward: per causal pair the score kappa (2 x 6d), <g_t, v_s>
    (2 d_v), and the three gradient products dPhi(q) (2 x 6d), dPhi(k) (2 x 6d) and dv (2 d_v)."""
    pairs = T * (T + 1) // 2
    return B * H * pairs * 2 * (3 * F + 2 * DV)


def backward_p1_flops(B, H, T, C=32):
    """Algorithmic FLOPs of the p = 1 backward as the library computes it, as chunked recurrences in 32-token chunks
    (statistics included).  Per token the state products S g, Phi(K)^T V (forward), R v, R^T Phi(k) and
    Phi(Q)^T (G / Dn) (reverse), 2 x 6d x d_v each, and the statistics' dot products Phi(q) . S g and Phi(q) . z
    (2 x 6d each); per causal pair inside a chunk <g_t, v_s> twice (2 d_v each), the scores twice, A Phi(K) and
    Phi(Q) A (2 x 6d each), and the chunk's part of dv (2 d_v)."""
    chunk_pairs = (T // C) * C * (C + 1) // 2 + (T % C) * (T % C + 1) // 2
    linear = T * (5 * 2 * F * DV + 2 * 2 * F)
    intra = chunk_pairs * 2 * (3 * DV + 4 * F)
    return B * H * (linear + intra)


def bench_backward(torch, rpg, si, w, p_exp, steps, warmup, saved=False):
    """ms per call (eager, graph-replayed) of sanatan_attention_backward on workload w's inputs with p = p_exp,
    dout ~ N(0, 1) in the same dtype.  saved: sanatan_attention_backward_saved instead, given the statistics one
    sanatan_quadratic_train call saved before the timed region (a training step's forward pass; the forward itself
    is timed as the quadratic workload)."""
    q, k, v, om = si.workload_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    qd, kd, vd = (torch.from_numpy(x).cuda().to(dt) for x in (q, k, v))
    del q, k, v
    g = torch.randn(vd.shape, generator=torch.Generator(device="cuda").manual_seed(w.seed), device="cuda").to(dt)
    p = rpg.Params(omega=torch.from_numpy(om).cuda(), gamma=w.gamma, eps=w.eps, lambda_base=w.lambda_base)
    code = rpg.SANATAN_BF16 if w.dtype == "bf16" else rpg.SANATAN_F32
    ws = torch.empty((rpg.sanatan_attention_backward_workspace_bytes(w.B, w.H, w.T, code, p),), dtype=torch.uint8,
                     device="cuda")
    outs = (torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd),
            torch.empty((om.shape[0], D), dtype=torch.float32, device="cuda"))
    if saved:
        _, saved_stats = rpg.sanatan_quadratic_train(qd, kd, vd, p_exp, p)
        fn = lambda: rpg.sanatan_attention_backward_saved(qd, kd, vd, g, saved_stats, p_exp, p, dq=outs[0],
                                                          dk=outs[1], dv=outs[2], domega=outs[3], ws=ws)
    else:
        fn = lambda: rpg.sanatan_attention_backward(qd, kd, vd, g, p_exp, p, dq=outs[0], dk=outs[1], dv=outs[2],
                                                    domega=outs[3], ws=ws)
    eager = timed_loop(torch, fn, steps, warmup)
    gr = graph_of(torch, fn)
    graph = timed_loop(torch, gr.replay, steps, warmup) if gr is not None else None
    return eager, graph


def bench_featurize(torch, rpg, si, w, steps, warmup):
    """Standalone feature map of one [B,H,T,64] operand (the keys of workload w) into [B,H,T,384], same dtype.
    HBM-bound: the algorithmic bytes are the input read once and Phi written once."""
    _, k, _, om = si.workload_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    kd = torch.from_numpy(k).cuda().to(dt)
    del k
    p = rpg.Params(omega=torch.from_numpy(om).cuda(), gamma=w.gamma, eps=w.eps, lambda_base=w.lambda_base)
    phi = torch.empty((w.B, w.H, w.T, 6 * 64), dtype=dt, device="cuda")
    fn = lambda: rpg.sanatan_featurize(kd, 0, p, out=phi)
    eager = timed_loop(torch, fn, steps, warmup)
    g = graph_of(torch, fn)
    graph = timed_loop(torch, g.replay, steps, warmup) if g is not None else None
    el = 2 if w.dtype == "bf16" else 4
    return eager, graph, w.B * w.H * w.T * 64 * el * 7


def bench_feature_map(torch, rpg, si, w, nh, steps, warmup):
    """ms per call (eager, graph-replayed) of the materialized-feature chunked prefill on workload w's inputs:
    the spectral-harmonic map with nh harmonics, or (nh = 0) the unclipped four-channel map."""
    q, k, v, om = si.workload_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    qd, kd, vd = (torch.from_numpy(x).cuda().to(dt) for x in (q, k, v))
    del q, k, v
    p = rpg.Params(omega=torch.from_numpy(om).cuda(), gamma=w.gamma, eps=w.eps, lambda_base=w.lambda_base)
    code = rpg.SANATAN_BF16 if w.dtype == "bf16" else rpg.SANATAN_F32
    if nh > 0:
        need = rpg.sanatan_prefill_harmonics_workspace_bytes(w.B, w.H, w.T, code, nh, p)
    else:
        need = rpg.sanatan_prefill_four_channel_workspace_bytes(w.B, w.H, w.T, code, p)
    ws = torch.empty((int(need),), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(vd)
    if nh > 0:
        fn = lambda: rpg.sanatan_prefill_harmonics(qd, kd, vd, nh, p, out=out, ws=ws)
    else:
        fn = lambda: rpg.sanatan_prefill_four_channel(qd, kd, vd, p, out=out, ws=ws)
    eager = timed_loop(torch, fn, steps, warmup)
    g = graph_of(torch, fn)
    graph = timed_loop(torch, g.replay, steps, warmup) if g is not None else None
    return eager, graph


def bench_ragged(torch, rpg, si, w, steps, warmup):
    """The headline shape as a batch of prompts of seeded lengths in [T/8, T]: one ragged prefill call, and
    for comparison one uniform call per prompt (what a caller without per-element lengths would run).
    Returns (lengths, (eager, graph) of the ragged call, (eager, graph) of the per-prompt calls)."""
    import numpy as np

    q, k, v, om = si.workload_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    qd, kd, vd = (torch.from_numpy(x).cuda().to(dt) for x in (q, k, v))
    del q, k, v
    p = rpg.Params(omega=torch.from_numpy(om).cuda(), gamma=w.gamma, eps=w.eps, lambda_base=w.lambda_base)
    lens = np.random.default_rng(w.seed + 99).integers(w.T // 8, w.T + 1, w.B).astype(np.int32)
    lens_d = torch.from_numpy(lens).cuda()
    out = torch.zeros_like(vd)
    ws = torch.empty((rpg.sanatan_prefill_workspace_bytes(w.B, w.H, w.T, w.chunk, p),), dtype=torch.uint8,
                     device="cuda")
    fn = lambda: rpg.sanatan_prefill_chunked_ragged(qd, kd, vd, lens_d, w.chunk, p, out=out, ws=ws)
    eager = timed_loop(torch, fn, steps, warmup)
    g = graph_of(torch, fn)
    graph = timed_loop(torch, g.replay, steps, warmup) if g is not None else None
    # one uniform call per prompt, on contiguous copies of its rows
    per = []
    for b, L in enumerate(lens):
        xs = [x[b:b + 1, :, :L].contiguous() for x in (qd, kd, vd)]
        o = torch.empty_like(xs[2])
        wsb = torch.empty((rpg.sanatan_prefill_workspace_bytes(1, w.H, int(L), w.chunk, p),), dtype=torch.uint8,
                          device="cuda")
        per.append((xs, o, wsb))

    def fn_per():
        for xs, o, wsb in per:
            rpg.sanatan_prefill_chunked(xs[0], xs[1], xs[2], w.chunk, p, out=o, ws=wsb)

    eager_p = timed_loop(torch, fn_per, steps, warmup)
    gp = graph_of(torch, fn_per)
    graph_p = timed_loop(torch, gp.replay, steps, warmup) if gp is not None else None
    return lens, (eager, graph), (eager_p, graph_p)


def chunked_flops(B, H, T, C, F_, DV_=DV):
    """Causal FLOPs of a chunked p = 1 prefill with F_ features per head (causal pairs inside chunks, readout
    and update per token)."""
    per_head = 0
    for c0 in range(0, T, C):
        n = min(C, T - c0)
        per_head += 2 * (n * (n + 1) // 2) * (F_ + DV_) + 2 * n * F_ * DV_ * 2
    return B * H * per_head


def mfma_line(fl, ms):
    return {"bound": "mfma", "achieved": fl / (ms * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


ONLY = ("prefill", "decode1", "decode64", "long", "quad", "quad4", "backward_p2", "backward_p2_saved", "backward_p1",
        "featurize", "harmonics", "four_channel", "ragged")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--only", choices=ONLY,
                    help="time one workload and print its own JSON line (for profiling runs), not the headline line")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a plain %d MiB device copy first (reference kernel for memory counters)" % (CAL_BYTES >> 20))
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) into profiles/traffic.json")
    ap.add_argument("--traffic-key", default="prefill_b8h12_t2048")
    args = ap.parse_args()
    if args.traffic:
        traffic_summary(args.traffic[0], args.traffic[1], args.traffic_key)
        return
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(pass --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import root_parity_gated_amd as rpg
    import sanatan_inputs as si

    rpg.lib()  # raises if the HIP library is not built
    if args.calibrate_copy:
        src_buf = torch.empty(CAL_BYTES, dtype=torch.uint8, device="cuda")
        dst_buf = torch.empty_like(src_buf)
        for _ in range(3):
            dst_buf.copy_(src_buf)
        torch.cuda.synchronize()
        del src_buf, dst_buf
    w = si.PREFILL
    small = max(5, args.steps // 5)
    if args.only:
        rec = {"only": args.only}
        if args.only == "prefill":
            rec["ms"] = bench_prefill_like(torch, rpg, si, w, args.steps, args.warmup)
        elif args.only in ("decode1", "decode64"):
            b = 1 if args.only == "decode1" else 64
            rec.update(bench_decode(torch, rpg, si, b, args.decode_steps, 16))
        elif args.only == "long":
            rec["ms"] = bench_prefill_like(torch, rpg, si, si.LONG, small, 3)
        elif args.only in ("quad", "quad4"):
            rec["ms"] = bench_prefill_like(torch, rpg, si, si.QUAD_P2, small, 3, quadratic=True,
                                           four_channel=args.only == "quad4")
        elif args.only.startswith("backward"):
            wb, pb = (w, 1) if args.only == "backward_p1" else (si.QUAD_P2, 2)
            rec["ms"] = bench_backward(torch, rpg, si, wb, pb, max(3, args.steps // 10), 2,
                                       saved=args.only == "backward_p2_saved")
        elif args.only == "featurize":
            rec["ms"] = bench_featurize(torch, rpg, si, w, small, 3)[:2]
        elif args.only == "ragged":
            lens, r, pp = bench_ragged(torch, rpg, si, w, small, 3)
            rec.update({"lengths": lens.tolist(), "ms": r, "ms_per_prompt_calls": pp})
        elif args.only in ("harmonics", "four_channel"):
            rec["ms"] = bench_feature_map(torch, rpg, si, w, 2 if args.only == "harmonics" else 0, small, 3)
        print(json.dumps(rec))
        return

    log(f"prefill {w.name}: {args.warmup} warmup + {args.steps} timed steps")
    per_call = {}
    eager_ms, graph_ms = bench_prefill_like(torch, rpg, si, w, args.steps, args.warmup, per_call=per_call)
    use_graph = graph_ms is not None and graph_ms < eager_ms
    ms = graph_ms if use_graph else eager_ms
    log(f"prefill: {eager_ms * 1e3:.1f} us/step eager, "
        f"{graph_ms * 1e3 if graph_ms is not None else float('nan'):.1f} us/step graph-replayed")
    call_ms = ms
    tokens = w.B * w.T
    fl = prefill_flops(w.B, w.H, w.T, w.chunk)
    fl_dense = prefill_flops(w.B, w.H, w.T, w.chunk, causal=False)
    nbytes = prefill_bytes(w.B, w.H, w.T)
    achieved_tf = fl / (call_ms * 1e-3) / 1e12
    achieved_gbs = nbytes / (call_ms * 1e-3) / 1e9
    src = source_hash(*PREFILL_SOURCES)
    result = {
        "metric": "prefill tokens/s (12h x d64, T=2K, p=1)",
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: q,k,v ~ N(0,1) rounded to bf16, omega ~ U(-pi,pi), seeded (sanatan_inputs)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "d": D, "d_v": DV, "chunk": w.chunk,
                   "p": 1, "gamma": w.gamma, "lambda_base": w.lambda_base},
        # At about 249 flop per algorithmic byte the workload sits below the bf16 ridge (~312 flop/byte): the HBM
        # roof (12.6 us) binds before the MFMA roof (10.0 us), so the line is priced against HBM, with the MFMA
        # fraction beside it.
        "roofline": {
            "bound": "hbm", "achieved": achieved_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved_gbs / PEAK_HBM_GBS,
            "traffic": traffic_from_profiles("prefill_b8h12_t2048", src),
            "kernel": "sanatan_prefill_chunked: phase table + pass 1 (state increments) + pass 3 (outputs), "
                      "timed as one launch sequence",
            "timing": "graph-replayed call" if use_graph else "eager call",
            "ms_per_call_eager": eager_ms, "ms_per_call_graph": graph_ms,
            "ms_per_call_eager_median": per_call.get("median"), "ms_per_call_eager_mean_single": per_call.get("mean"),
            "hbm_bytes_algorithmic": nbytes,
            "mfma_achieved_tflops": achieved_tf, "mfma_peak_tflops": PEAK_BF16_TFLOPS,
            "mfma_frac": achieved_tf / PEAK_BF16_TFLOPS,
            "flops_per_launch": fl, "flops_dense_tile": fl_dense,
            "source_hash": src,
        },
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(w)
        log(f"cpu baseline: {result['cpu_baseline']['sample']}")
    if not args.no_extras:
        extras = {}
        for b in (1, 64):
            log(f"decode batch {b}")
            extras[f"decode_batch{b}"] = bench_decode(torch, rpg, si, b, args.decode_steps, 16)
            if b > 1:
                log(f"decode batch {b}, one position per sequence")
                extras[f"decode_batch{b}_positions"] = bench_decode(torch, rpg, si, b, args.decode_steps, 16,
                                                                    positions=True)
            log(f"decode batch {b}, compact state")
            extras[f"decode_batch{b}_compact"] = bench_decode(torch, rpg, si, b, args.decode_steps, 16, compact=True)
            log(f"decode batch {b}: {extras[f'decode_batch{b}']['us_per_token']:.2f} us/token")
        wl = si.LONG
        log(f"long prefill {wl.name}")
        lms_e, lms_g = bench_prefill_like(torch, rpg, si, wl, small, 3)
        lms = min(lms_e, lms_g) if lms_g is not None else lms_e
        extras["long_prefill"] = {"workload": wl.name, "tokens_per_s": wl.B * wl.T / (lms * 1e-3), "ms": lms,
                                  "ms_eager": lms_e, "ms_graph": lms_g,
                                  "roofline": mfma_line(prefill_flops(wl.B, wl.H, wl.T, wl.chunk), lms)}
        wq = si.QUAD_P2
        log(f"quadratic {wq.name}")
        qms_e, qms_g = bench_prefill_like(torch, rpg, si, wq, small, 3, quadratic=True)
        qms = min(qms_e, qms_g) if qms_g is not None else qms_e
        extras["quadratic_p2"] = {"workload": wq.name, "tokens_per_s": wq.B * wq.T / (qms * 1e-3), "ms": qms,
                                  "ms_eager": qms_e, "ms_graph": qms_g,
                                  "roofline": mfma_line(quadratic_flops(wq.B, wq.H, wq.T), qms)}
        log(f"quadratic {wq.name}, training forward (saves the backward pass's statistics)")
        qt_e, qt_g = bench_prefill_like(torch, rpg, si, wq, small, 3, quadratic=True, train=True)
        qt = min(qt_e, qt_g) if qt_g is not None else qt_e
        extras["quadratic_p2_train"] = {
            "workload": wq.name + "_train", "tokens_per_s": wq.B * wq.T / (qt * 1e-3), "ms": qt, "ms_eager": qt_e,
            "ms_graph": qt_g, "roofline": mfma_line(quadratic_flops(wq.B, wq.H, wq.T), qt),
            "note": "sanatan_quadratic_train: the p=2 forward plus its saved fp32 output rows and 1/Dn, the input "
                    "of backward_p2_saved"}
        log(f"quadratic {wq.name}, unclipped four-channel kernel")
        q4_e, q4_g = bench_prefill_like(torch, rpg, si, wq, small, 3, quadratic=True, four_channel=True)
        q4 = min(q4_e, q4_g) if q4_g is not None else q4_e
        extras["quadratic_p2_four_channel"] = {
            "workload": wq.name + "_four_channel", "tokens_per_s": wq.B * wq.T / (q4 * 1e-3), "ms": q4,
            "ms_eager": q4_e, "ms_graph": q4_g,
            "roofline": mfma_line(quadratic_flops(wq.B, wq.H, wq.T, features=4 * D), q4),
            "note": "unclipped four-channel kernel: 2 (4d + d_v) flops per causal pair"}
        for key, wb, pb, sv in (("backward_p2", si.QUAD_P2, 2, False), ("backward_p2_saved", si.QUAD_P2, 2, True),
                                ("backward_p1", w, 1, False)):
            log(f"backward {wb.name}, p={pb}" + (", saved statistics" if sv else ""))
            be, bg = bench_backward(torch, rpg, si, wb, pb, max(3, args.steps // 10), 2, saved=sv)
            bms = min(be, bg) if bg is not None else be
            bfl = backward_flops(wb.B, wb.H, wb.T) if pb == 2 else backward_p1_flops(wb.B, wb.H, wb.T)
            note = ("gradients of q, k, v, omega (sanatan_attention_backward, masked quadratic form); "
                    "flops: 2 (3 x 6d + 2 d_v) per causal pair") if pb == 2 and not sv else (
                    "sanatan_attention_backward_saved: the same gradients given the fp32 output rows and 1/Dn "
                    "saved by sanatan_quadratic_train (no statistics pass); flops as backward_p2") if pb == 2 else (
                    "gradients of q, k, v, omega (sanatan_attention_backward: statistics, feature gradients and dv "
                    "as chunked recurrences, linear in T); flops as backward_p1_flops states")
            extras[key] = {"workload": f"{wb.name}_backward_p{pb}" + ("_saved" if sv else ""), "ms": bms,
                           "ms_eager": be, "ms_graph": bg,
                           "tokens_per_s": wb.B * wb.T / (bms * 1e-3), "flops_per_call": bfl,
                           "roofline": mfma_line(bfl, bms), "note": note}
        for key, nh, feats in (("harmonics_nh2_prefill", 2, 10 * D), ("four_channel_prefill", 0, 3 * D + 1)):
            log(f"{key} {w.name}")
            he, hg = bench_feature_map(torch, rpg, si, w, nh, small, 3)
            hms = min(he, hg) if hg is not None else he
            extras[key] = {"workload": f"{w.name}_{key}", "ms": hms, "ms_eager": he, "ms_graph": hg,
                           "tokens_per_s": w.B * w.T / (hms * 1e-3),
                           "roofline": mfma_line(chunked_flops(w.B, w.H, w.T, 32, feats), hms),
                           "note": f"materialized-feature chunked prefill, {feats} features per head, chunk 32, "
                                   "one workgroup per sequence"}
        log(f"featurize {w.name} keys")
        fms_e, fms_g, fbytes = bench_featurize(torch, rpg, si, w, small, 3)
        fms = min(fms_e, fms_g) if fms_g is not None else fms_e
        extras["featurize"] = {"workload": f"featurize_keys_of_{w.name}", "ms": fms, "ms_eager": fms_e,
                               "ms_graph": fms_g, "bytes_per_call": fbytes,
                               "roofline": {"bound": "hbm", "achieved": fbytes / (fms * 1e-3) / 1e9,
                                            "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                            "frac": fbytes / (fms * 1e-3) / 1e9 / PEAK_HBM_GBS}}
        log(f"ragged prefill {w.name}")
        lens, (re_, rg_), (pe_, pg_) = bench_ragged(torch, rpg, si, w, small, 3)
        rms = min(re_, rg_) if rg_ is not None else re_
        pms = min(pe_, pg_) if pg_ is not None else pe_
        rtok = int(lens.sum())
        rbytes = prefill_bytes(1, w.H, rtok)
        extras["ragged_prefill"] = {
            "workload": f"{w.name}_ragged", "lengths": lens.tolist(), "tokens_per_s": rtok / (rms * 1e-3),
            "ms": rms, "ms_eager": re_, "ms_graph": rg_,
            "ms_one_call_per_prompt": pms, "ms_one_call_per_prompt_eager": pe_, "ms_one_call_per_prompt_graph": pg_,
            "roofline": {"bound": "hbm", "achieved": rbytes / (rms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": rbytes / (rms * 1e-3) / 1e9 / PEAK_HBM_GBS},
            "note": "one sanatan_prefill_chunked_ragged call over prompts of seeded lengths in [T/8, T]; "
                    "algorithmic bytes: q, k, v read and out written for the valid rows only"}
        if not args.no_cpu_baseline:
            log("cpu oracle beside the other workloads")
            for key, rec in cpu_oracle_extras(si).items():
                extras.setdefault("cpu_oracle", {})[key] = rec
        result["extras"] = extras
    print(json.dumps(result))


if __name__ == "__main__":
    main()
