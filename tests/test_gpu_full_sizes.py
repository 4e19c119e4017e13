"""Parity at the benchmark's full sizes and launch configuration, on outputs the oracle can afford:
whole sampled sequences (recurrent oracle) or sampled rows (direct oracle)."""
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


def row_rel_err(got, want):
    got = np.asarray(got, np.float64).reshape(-1, want.shape[-1])
    want = np.asarray(want, np.float64).reshape(-1, want.shape[-1])
    return float((np.abs(got - want).max(1) / np.maximum(np.abs(want).max(1), 1e-12)).max())


def run_workload(torch, w, quadratic=False):
    import root_parity_gated_amd as rpg

    q, k, v, om = si.workload_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    qd, kd, vd = (torch.from_numpy(x).cuda().to(dt) for x in (q, k, v))
    p = rpg.Params(omega=torch.from_numpy(om).cuda(), gamma=w.gamma, eps=w.eps, lambda_base=w.lambda_base)
    if quadratic:
        out = rpg.sanatan_quadratic_ref_p2(qd, kd, vd, w.p, p)
    else:
        out = rpg.sanatan_prefill_chunked(qd, kd, vd, w.chunk, p)
    torch.cuda.synchronize()
    return (q, k, v, om), out.float().cpu().numpy()


def test_prefill_b8h12_t2048(torch_dev):
    w = si.PREFILL
    (q, k, v, om), got = run_workload(torch_dev, w)
    assert np.isfinite(got).all()
    for b, h in [(0, 0), (3, 7), (7, 11)]:
        want, _, _ = oracle.recurrent(q[b, h], k[b, h], v[b, h], om[h])
        err = record(f"prefill {w.name} (3 sequences)", row_rel_err(got[b, h], want), TOL[w.dtype])
        assert err <= TOL[w.dtype], (b, h)


def test_long_prefill_b1h12_t32768(torch_dev):
    w = si.LONG
    (q, k, v, om), got = run_workload(torch_dev, w)
    assert np.isfinite(got).all()
    heads = [0, 11]
    want, _, _ = oracle.recurrent_heads(q[0, heads], k[0, heads], v[0, heads], om[heads])
    for j, h in enumerate(heads):
        err = record(f"long prefill {w.name} (heads 0, 11)", row_rel_err(got[0, h], want[j]), TOL[w.dtype])
        assert err <= TOL[w.dtype], h
    # explicitly the chunk-boundary rows, the first rows and the last row
    C = w.chunk
    rows = sorted(set([0, 1, w.T - 1] + [t for j in range(1, w.T // C) for t in (C * j - 1, C * j)]))
    assert row_rel_err(got[0, 0, rows], want[0, rows]) <= TOL[w.dtype]


def test_quadratic_p2_b4h12_t4096(torch_dev):
    w = si.QUAD_P2
    (q, k, v, om), got = run_workload(torch_dev, w, quadratic=True)
    assert np.isfinite(got).all()
    rng = np.random.default_rng(77)
    for b, h in [(0, 0), (2, 5), (3, 11)]:
        rows = sorted(set([0, 1, 63, 64, 127, 128, w.T - 1] + list(rng.integers(0, w.T, 12))))
        want = oracle.attention_direct(q[b, h], k[b, h], v[b, h], om[h], p=w.p, rows=rows)
        err = record(f"quadratic {w.name} (sampled rows)", row_rel_err(got[b, h, rows], want), TOL[w.dtype])
        assert err <= TOL[w.dtype], (b, h)


@pytest.mark.parametrize("batch", [1, 64])
def test_decode_after_4096_token_fill(torch_dev, batch):
    import root_parity_gated_amd as rpg

    torch = torch_dev
    w = si.DECODE
    nh, fill, steps = w.H, w.T, w.extra["steps"]
    N = batch * nh
    if batch == 1:
        om, (fq, fk, fv), (sq, sk, sv) = si.decode_inputs_numpy(w.seed, nh, fill, steps)
        fq, fk, fv, sq, sk, sv = (torch.from_numpy(x).cuda() for x in (fq, fk, fv, sq, sk, sv))
    else:
        om, (fq, fk, fv), (sq, sk, sv) = si.decode_inputs_torch(w.seed + batch, batch, nh, fill, steps, "cuda")
    p = rpg.Params(omega=torch.from_numpy(om).cuda())
    S = torch.zeros((N, 384, 64), device="cuda")
    z = torch.zeros((N, 384), device="cuda")
    for i in range(0, N, 1152):
        j = min(N, i + 1152)
        rpg.sanatan_prefill_chunked(fq[i:j].unsqueeze(0), fk[i:j].unsqueeze(0), fv[i:j].unsqueeze(0), 64, p,
                                    S=S[i:j].unsqueeze(0), z=z[i:j].unsqueeze(0))
    sample = [0, 77, 143] if batch == 1 else [5, 144 * 31 + 100, N - 1]
    outs = torch.empty((steps, len(sample), 64), device="cuda")
    out = torch.empty((N, 64), device="cuda")
    idx = torch.tensor(sample, device="cuda")
    for i in range(steps):
        rpg.sanatan_decode_step(sq[i], sk[i], sv[i], fill + i, p, S, z, out)
        outs[i] = out[idx]
    torch.cuda.synchronize()
    got = outs.cpu().numpy().transpose(1, 0, 2)
    hs = [i % nh for i in sample]
    cpu = lambda x: x[sample].cpu().numpy() if hasattr(x, "cpu") else x[sample]
    Fq, Fk, Fv = cpu(fq), cpu(fk), cpu(fv)
    Dq = (sq[:, sample].cpu().numpy() if hasattr(sq, "cpu") else sq[:, sample]).transpose(1, 0, 2)
    Dk = (sk[:, sample].cpu().numpy() if hasattr(sk, "cpu") else sk[:, sample]).transpose(1, 0, 2)
    Dv = (sv[:, sample].cpu().numpy() if hasattr(sv, "cpu") else sv[:, sample]).transpose(1, 0, 2)
    _, S0, z0 = oracle.recurrent_heads(Fq, Fk, Fv, om[hs], want_out=False)
    want, Sw, zw = oracle.recurrent_heads(Dq, Dk, Dv, om[hs], pos0=fill, S=S0, z=z0)
    err = record(f"decode {w.name} batch {batch} (sampled head-states)", row_rel_err(got, want), TOL["f32"])
    assert err <= TOL["f32"]
    Sg = S[idx].cpu().numpy()
    assert np.abs(Sg - Sw).max() <= 1e-4 * np.abs(Sw).max()


def test_tiny_config_three_forms(torch_dev):
    """The tiny workload's own seeded inputs (B1 H1 T256 fp32, seed 1000, positions from 0) through all three GPU
    forms -- the chunked prefill at chunk 64, the masked quadratic form at p = 1 and 256 decode steps from an
    empty state -- each against the oracle on the same inputs ([N] §2.7: the parallel and recurrent forms are the
    same function)."""
    import root_parity_gated_amd as rpg

    torch = torch_dev
    w = si.TINY
    q, k, v, om = si.workload_inputs(w)
    want = oracle.attention_direct(q[0, 0], k[0, 0], v[0, 0], om[0])
    want_rec, Sw, zw = oracle.recurrent(q[0, 0], k[0, 0], v[0, 0], om[0])
    assert row_rel_err(want_rec, want) <= 1e-12  # the two oracle forms agree
    d = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    p = rpg.Params(omega=d(om), gamma=w.gamma, eps=w.eps, lambda_base=w.lambda_base)
    chunked = rpg.sanatan_prefill_chunked(d(q), d(k), d(v), w.chunk, p).cpu().numpy()[0, 0]
    quad = rpg.sanatan_quadratic_ref_p2(d(q), d(k), d(v), 1, p).cpu().numpy()[0, 0]
    S = torch.zeros((1, 384, 64), device="cuda")
    z = torch.zeros((1, 384), device="cuda")
    rec = np.stack([rpg.sanatan_decode_step(d(q[0, 0, t:t + 1]), d(k[0, 0, t:t + 1]), d(v[0, 0, t:t + 1]), t, p, S,
                                            z).cpu().numpy()[0] for t in range(w.T)])
    torch.cuda.synchronize()
    for form, got in (("chunked C=64", chunked), ("quadratic p=1", quad), ("recurrent (256 decode steps)", rec)):
        err = record(f"tiny {w.name}: {form}", row_rel_err(got, want), TOL["f32"])
        assert err <= TOL["f32"], form
    assert np.abs(S.cpu().numpy()[0] - Sw).max() <= 1e-4 * np.abs(Sw).max()
