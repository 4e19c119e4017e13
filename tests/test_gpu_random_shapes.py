"""Seeded random shapes through the prefill entry points (against the fp64 oracle's recurrence) and the masked
quadratic form (against its direct form).

Each case draws B, H, T, the chunk, the element type, a start position, whether a caller state is passed, and
either a forced workgroup count (the partition test hook: from one workgroup for the whole call to one per
chunk) or per-element lengths for the ragged call.  Every output row below each sequence's length and every
final state is compared.  Bars: 1e-4 (fp32 inputs), 2e-2 (bf16).  The draws are fixed by the case number, so a
failure names a reproducible configuration.
"""
import numpy as np
import pytest

import oracle
import sanatan_inputs as si
from parity_log import record

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module")
def torch_dev():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import root_parity_gated_amd as rpg

    rpg.lib()
    return torch


def draw(case):
    rng = np.random.default_rng(4000 + case)
    dtype = ["f32", "bf16"][rng.integers(2)]
    chunk = int(rng.choice([16, 32, 64] + ([128] if dtype == "bf16" else [])))
    B, H = int(rng.integers(1, 5)), int(rng.integers(1, 7))
    T = int(rng.integers(1, 5 * chunk + 40))
    pos0 = int(rng.choice([0, 1, int(rng.integers(2, 1 << 20))]))
    with_state = bool(rng.integers(2))
    ragged = bool(rng.integers(2))
    nch = B * H * ((T + chunk - 1) // chunk)
    wgs = 0 if ragged else int(rng.choice([0, 1, int(rng.integers(1, nch + 1)), nch]))
    lengths = rng.integers(0, T + 1, B) if ragged else None
    return dict(dtype=dtype, chunk=chunk, B=B, H=H, T=T, pos0=pos0, with_state=with_state, wgs=wgs,
                lengths=lengths)


@pytest.mark.parametrize("case", range(64))
def test_prefill_random_shape(torch_dev, case):
    import root_parity_gated_amd as rpg

    torch = torch_dev
    c = draw(case)
    dtype, chunk, B, H, T, pos0 = c["dtype"], c["chunk"], c["B"], c["H"], c["T"], c["pos0"]
    print(f"case {case}: {c}", flush=True)
    q, k, v, om = si.attention_inputs(4100 + case, B, H, T + 8, dtype)
    dev = lambda x: (lambda t: t.to(torch.bfloat16) if dtype == "bf16" else t)(
        torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda())
    prm = rpg.Params(omega=torch.from_numpy(np.ascontiguousarray(om, dtype=np.float32)).cuda())
    S0 = z0 = None
    S = z = None
    if c["with_state"]:
        # the state after 8 earlier tokens (positions pos0 - 8 .. pos0 - 1, or from 0 when pos0 < 8)
        p_hist = pos0 - 8
        _, S0, z0 = oracle.recurrent_heads(q[:, :, T:].reshape(B * H, 8, -1), k[:, :, T:].reshape(B * H, 8, -1),
                                           v[:, :, T:].reshape(B * H, 8, -1), np.tile(om, (B, 1)), pos0=p_hist)
        S0 = S0.reshape(B, H, 384, 64).astype(np.float32)
        z0 = z0.reshape(B, H, 384).astype(np.float32)
        S, z = torch.from_numpy(S0).cuda(), torch.from_numpy(z0).cuda()
    args = [dev(x[:, :, :T]) for x in (q, k, v)]
    if c["lengths"] is not None:
        lens = torch.from_numpy(c["lengths"].astype(np.int32)).cuda()
        out = torch.zeros((B, H, T, 64), device="cuda", dtype=args[0].dtype)
        rpg.sanatan_prefill_chunked_ragged(*args, lens, chunk, prm, pos0=pos0, S=S, z=z, out=out)
        lengths = [int(x) for x in c["lengths"]]
    else:
        out = rpg.sanatan_prefill_chunked_partitioned(*args, chunk, c["wgs"], prm, pos0=pos0, S=S, z=z)
        lengths = [T] * B
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    Sg = S.cpu().numpy() if S is not None else None
    zg = z.cpu().numpy() if z is not None else None
    err = serr = 0.0
    for b in range(B):
        L = lengths[b]
        for h in range(H):
            want, Sw, zw = oracle.recurrent(q[b, h, :L], k[b, h, :L], v[b, h, :L], om[h], pos0=pos0,
                                            S=None if S0 is None else S0[b, h], z=None if z0 is None else z0[b, h])
            if L:
                d = np.abs(got[b, h, :L] - want).max(1) / np.maximum(np.abs(want).max(1), 1e-12)
                err = max(err, float(d.max()))
            if Sg is not None:
                serr = max(serr, np.abs(Sg[b, h] - Sw).max() / max(np.abs(Sw).max(), 1e-30),
                           np.abs(zg[b, h] - zw).max() / max(np.abs(zw).max(), 1e-30))
    print(f"case {case}: output {err:.3e}, state {serr:.3e}")
    assert record(f"random prefill shapes {dtype}: output", err, TOL[dtype]) <= TOL[dtype]
    assert record(f"random prefill shapes {dtype}: state", serr, TOL[dtype]) <= TOL[dtype]


@pytest.mark.parametrize("case", range(16))
def test_quadratic_random_shape(torch_dev, case):
    """The masked quadratic form (p = 1 or 2, six- or four-channel) at seeded random shapes."""
    import root_parity_gated_amd as rpg

    torch = torch_dev
    rng = np.random.default_rng(4500 + case)
    dtype = ["f32", "bf16"][rng.integers(2)]
    # the unclipped four-channel kernel only at p = 2: at p = 1 its weights, and so a denominator, can be near
    # zero, where a row's relative error measures the row's conditioning rather than the kernel
    p = int(rng.integers(1, 3))
    four = bool(rng.integers(2)) and p == 2
    B, H, T = int(rng.integers(1, 4)), int(rng.integers(1, 5)), int(rng.integers(1, 300))
    print(f"case {case}: {dtype} p={p} four_channel={four} B={B} H={H} T={T}", flush=True)
    q, k, v, om = si.attention_inputs(4600 + case, B, H, T, dtype)
    dev = lambda x: (lambda t: t.to(torch.bfloat16) if dtype == "bf16" else t)(
        torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda())
    prm = rpg.Params(omega=torch.from_numpy(np.ascontiguousarray(om, dtype=np.float32)).cuda())
    out = rpg.sanatan_quadratic_ref_p2(dev(q), dev(k), dev(v), p, prm, four_channel=four)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    err = 0.0
    for b in range(B):
        for h in range(H):
            want = oracle.attention_direct(q[b, h], k[b, h], v[b, h], om[h], p=p, four_channel=four)
            d = np.abs(got[b, h] - want).max(1) / np.maximum(np.abs(want).max(1), 1e-12)
            err = max(err, float(d.max()))
    print(f"case {case}: {err:.3e}")
    assert record(f"random quadratic shapes {dtype}", err, TOL[dtype]) <= TOL[dtype]


@pytest.mark.parametrize("case", range(12))
def test_backward_random_shape(torch_dev, case):
    """The backward pass (p = 1 or 2) at seeded random shapes, heads sharing omega rows at random."""
    import root_parity_gated_amd as rpg

    torch = torch_dev
    rng = np.random.default_rng(4700 + case)
    dtype = ["f32", "bf16"][rng.integers(2)]
    p = int(rng.integers(1, 3))
    B, H, T = int(rng.integers(1, 3)), int(rng.integers(1, 5)), int(rng.integers(2, 260))
    nph = int(rng.integers(1, H + 1))
    print(f"case {case}: {dtype} p={p} B={B} H={H} T={T} nph={nph}", flush=True)
    q, k, v, om = si.attention_inputs(4800 + case, B, H, T, dtype)
    g = np.random.default_rng(4900 + case).standard_normal((B, H, T, 64)).astype(np.float32)
    if dtype == "bf16":
        g = si.bf16_round(g)
    om = om[:nph]
    dev = lambda x: (lambda t: t.to(torch.bfloat16) if dtype == "bf16" else t)(
        torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda())
    prm = rpg.Params(omega=torch.from_numpy(np.ascontiguousarray(om, dtype=np.float32)).cuda())
    dq, dk, dv, dom = rpg.sanatan_attention_backward(dev(q), dev(k), dev(v), dev(g), p, prm)
    torch.cuda.synchronize()
    host = lambda t: t.float().cpu().numpy().astype(np.float64)
    dq, dk, dv, dom = host(dq), host(dk), host(dv), host(dom)

    def rel(got, want):  # the backward tests' metric: rows floored at 1 % of the largest row
        got, want = got.reshape(-1, want.shape[-1]), want.reshape(-1, want.shape[-1])
        sc = np.abs(want).max(1)
        sc = np.maximum(sc, 1e-2 * sc.max())
        return float((np.abs(got - want).max(1) / sc).max())

    want_dom = np.zeros_like(dom)
    errs = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    for b in range(B):
        for h in range(H):
            wq, wk, wv, wo = oracle.attention_direct_grad(q[b, h], k[b, h], v[b, h], g[b, h], om[h % nph], p=p)
            errs["dq"] = max(errs["dq"], rel(dq[b, h], wq))
            errs["dk"] = max(errs["dk"], rel(dk[b, h], wk))
            errs["dv"] = max(errs["dv"], rel(dv[b, h], wv))
            want_dom[h % nph] += wo
    errs["domega"] = rel(dom, want_dom)
    err = max(errs.values())
    print(f"case {case}: " + ", ".join(f"{n} {e:.3e}" for n, e in errs.items()))
    assert record(f"random backward shapes {dtype}", err, TOL[dtype]) <= TOL[dtype]


@pytest.mark.parametrize("case", range(12))
def test_decode_random_shape(torch_dev, case):
    """Decode steps from a prefilled state at seeded random sizes: one position for all head-states or one each,
    on the full or the compact state."""
    import root_parity_gated_amd as rpg

    torch = torch_dev
    rng = np.random.default_rng(5000 + case)
    N, steps, fill = int(rng.integers(1, 300)), int(rng.integers(1, 9)), int(rng.integers(1, 200))
    per_state, compact = bool(rng.integers(2)), bool(rng.integers(2))
    print(f"case {case}: N={N} steps={steps} fill={fill} per_state={per_state} compact={compact}", flush=True)
    q, k, v, om = si.attention_inputs(5100 + case, 1, N, fill + steps, "f32")
    q, k, v = q[0], k[0], v[0]
    base = rng.integers(0, 1 << 20, N) if per_state else np.full(N, int(rng.integers(0, 1 << 20)))
    prm = rpg.Params(omega=torch.from_numpy(np.ascontiguousarray(om, dtype=np.float32)).cuda())
    # the starting state: the oracle's recurrence over the fill tokens of each head-state, from its own position
    S0 = np.zeros((N, 384, 64), np.float32)
    z0 = np.zeros((N, 384), np.float32)
    for i in range(N):
        _, s_, z_ = oracle.recurrent(q[i, :fill], k[i, :fill], v[i, :fill], om[i], pos0=int(base[i]), want_out=False)
        S0[i], z0[i] = s_, z_
    S, z = torch.from_numpy(S0).cuda(), torch.from_numpy(z0).cuda()
    if compact:
        Sc = torch.empty((N, 5 * 64 + 1, 64), device="cuda")
        zc = torch.empty((N, 5 * 64 + 1), device="cuda")
        rpg.sanatan_state_compact(S, z, Sc, zc)
    outs = []
    for j in range(steps):
        pos = torch.from_numpy((base + fill + j).astype(np.int64)).cuda() if per_state else int(base[0] + fill + j)
        args = [torch.from_numpy(np.ascontiguousarray(x[:, fill + j], dtype=np.float32)).cuda() for x in (q, k, v)]
        if compact:
            outs.append(rpg.sanatan_decode_step_compact(*args, pos, prm, Sc, zc).clone())
        elif per_state:
            outs.append(rpg.sanatan_decode_step_positions(*args, pos, prm, S, z).clone())
        else:
            outs.append(rpg.sanatan_decode_step(*args, pos, prm, S, z).clone())
    torch.cuda.synchronize()
    err = 0.0
    for i in range(N):
        want, _, _ = oracle.recurrent(q[i, fill:], k[i, fill:], v[i, fill:], om[i], pos0=int(base[i] + fill),
                                      S=S0[i], z=z0[i])
        got = np.stack([o[i].cpu().numpy() for o in outs]).astype(np.float64)
        d = np.abs(got - want).max(1) / np.maximum(np.abs(want).max(1), 1e-12)
        err = max(err, float(d.max()))
    print(f"case {case}: {err:.3e}")
    assert record("random decode shapes f32", err, TOL["f32"]) <= TOL["f32"]
