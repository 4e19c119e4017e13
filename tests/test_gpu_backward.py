"""The backward pass on the GPU against the oracle's fp64 gradient of the direct form.

For L = sum(dout * o) with o the normalised causal power attention (p = 1 or 2), the GPU's dq, dk, dv and
domega are compared with oracle.attention_direct_grad on the same seeded inputs (the oracle consumes the
bf16-rounded values for bf16 cases).  Metric: per token row, max |error| / max |reference| over that row's
components, maximised over rows (the forward's metric), with each row's scale floored at 1% of the largest
row's in that tensor (a gradient row can vanish: dq of the first token is exactly 0 at eps = 0), and a tensor
that vanishes as a whole (every gradient but dv of a single token) compared absolutely; domega per parameter
row the same way.  Bars: the forward's, 1e-4 for fp32 inputs and 2e-2 for bf16 inputs.
"""
import math

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


def dev(torch, x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def rounded(x, dtype):
    """The values the GPU sees: bf16 inputs are rounded to bf16 (round to nearest even)."""
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    import torch

    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)


def row_rel_err(got, want, floor=1e-2):
    """Per-row max |error| / max |reference|, the row's scale floored at `floor` times the largest row's.
    Gradient rows can vanish: dq of the first token is exactly 0 at eps = 0 (o_0 = v_0), so without a floor
    the metric would divide rounding noise by ~0."""
    got = np.asarray(got, np.float64).reshape(-1, want.shape[-1])
    want = np.asarray(want, np.float64).reshape(-1, want.shape[-1])
    scale = np.abs(want).max(1)
    if scale.max() < 1e-4:
        # the whole tensor is an eps-sized signal (one token: o_0 = v_0 w / (w + eps), so dq, dk and domega are
        # ~1e-6, below what fp32 resolves relative to <g, v> ~ 1): compare absolutely, against the unit scale of
        # the N(0, 1) inputs
        return float(np.abs(got - want).max())
    scale = np.maximum(scale, floor * scale.max())
    return float((np.abs(got - want).max(1) / scale).max())


def run_case(torch, seed, B, H, T, dtype, p, nph=None, pos0=0, heads=None, saved=False):
    """saved: the training pair, the statistics sanatan_quadratic_train saved fed to
    sanatan_attention_backward_saved, instead of the backward pass that recomputes them."""
    import root_parity_gated_amd as rpg

    q, k, v, om = si.attention_inputs(seed, B, H, T, dtype)
    rng = np.random.default_rng(seed + 17)
    g = rounded(rng.standard_normal((B, H, T, 64)), dtype)
    nph = H if nph is None else nph
    om = om[:nph]
    prm = rpg.Params(omega=torch.from_numpy(np.ascontiguousarray(om, dtype=np.float32)).cuda())
    qd, kd, vd, gd = dev(torch, q, dtype), dev(torch, k, dtype), dev(torch, v, dtype), dev(torch, g, dtype)
    if saved:
        _, sv = rpg.sanatan_quadratic_train(qd, kd, vd, p, prm, pos0=pos0)
        dq, dk, dv, dom = rpg.sanatan_attention_backward_saved(qd, kd, vd, gd, sv, p, prm, pos0=pos0)
    else:
        dq, dk, dv, dom = rpg.sanatan_attention_backward(qd, kd, vd, gd, p, prm, pos0=pos0)
    torch.cuda.synchronize()
    dq, dk, dv, dom = host(dq), host(dk), host(dv), host(dom)
    want_dom = np.zeros_like(dom)
    errs = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    for b in range(B):
        for h in range(H):
            if heads is not None and (b, h) not in heads:
                continue
            wq, wk, wv, wo = oracle.attention_direct_grad(q[b, h], k[b, h], v[b, h], g[b, h], om[h % nph], p=p)
            errs["dq"] = max(errs["dq"], row_rel_err(dq[b, h], wq))
            errs["dk"] = max(errs["dk"], row_rel_err(dk[b, h], wk))
            errs["dv"] = max(errs["dv"], row_rel_err(dv[b, h], wv))
            want_dom[h % nph] += wo
    if heads is None:
        errs["domega"] = row_rel_err(dom, want_dom)
    tag = " (saved statistics)" if saved else ""
    print(f"backward{tag} B{B} H{H} T{T} {dtype} p={p} nph={nph}: " +
          ", ".join(f"{k} {v:.3e}" for k, v in errs.items()))
    if T > 1:
        for name, e in errs.items():
            record(f"backward{tag} {dtype} p={p}: {name}", e, TOL[dtype])
    return errs


@pytest.mark.parametrize("p", [1, 2])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_small(torch_dev, dtype, p):
    """Several key and query tiles, a ragged last tile, every head its own omega row."""
    errs = run_case(torch_dev, 800 + p, 1, 3, 200, dtype, p)
    for name, e in errs.items():
        assert e <= TOL[dtype], (name, e)


@pytest.mark.parametrize("T", [1, 31, 33, 129])
def test_backward_edge_lengths(torch_dev, T):
    """One token, and lengths around the 32-token block and 128-token tile edges."""
    for p in (1, 2):
        errs = run_case(torch_dev, 810 + T, 1, 2, T, "f32", p)
        for name, e in errs.items():
            assert e <= TOL["f32"], (name, p, e)


@pytest.mark.parametrize("p", [1, 2])
def test_backward_shared_omega_rows(torch_dev, p):
    """Two batches and six heads over two omega rows: each row's gradient sums over every head using it."""
    errs = run_case(torch_dev, 820, 2, 6, 96, "f32", p, nph=2, pos0=12345)
    for name, e in errs.items():
        assert e <= TOL["f32"], (name, e)


def test_backward_p1_one_piece_per_sequence(torch_dev):
    """p = 1 with enough sequences (128) that each runs its recurrences whole, in one piece per direction (the
    smaller cases above split every sequence into pieces that start from their neighbours' states)."""
    errs = run_case(torch_dev, 825, 2, 64, 70, "f32", 1)
    for name, e in errs.items():
        assert e <= TOL["f32"], (name, e)


@pytest.mark.parametrize("p", [1, 2])
def test_backward_long_bf16(torch_dev, p):
    """1000 tokens in bf16: 8 query tiles, the heaviest first."""
    errs = run_case(torch_dev, 830 + p, 1, 2, 1000, "bf16", p)
    for name, e in errs.items():
        assert e <= TOL["bf16"], (name, e)


def test_backward_p1_long_many_pieces(torch_dev):
    """p = 1 at 4096 tokens in bf16: on 256 compute units the 256 chunks of the two sequences run as 256
    one-chunk ranges, so a range's start state sums up to 127 slots of the ranges before (forward) or after
    (reverse) it."""
    errs = run_case(torch_dev, 835, 1, 2, 4096, "bf16", 1)
    for name, e in errs.items():
        assert e <= TOL["bf16"], (name, e)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_p1_range_across_sequences(torch_dev, dtype):
    """p = 1 at 2020 tokens (a 4-token last chunk) over five heads: on 256 compute units the 320 chunks run as
    ranges of one or two chunks, one of which holds the last chunk of one sequence and the first of the next, so
    a workgroup runs two segments of different sequences in turn."""
    errs = run_case(torch_dev, 837, 1, 5, 2020, dtype, 1)
    for name, e in errs.items():
        assert e <= TOL[dtype], (name, e)


@pytest.mark.parametrize("p", [1, 2])
def test_backward_deterministic(torch_dev, p):
    import root_parity_gated_amd as rpg

    torch = torch_dev
    q, k, v, om = si.attention_inputs(840, 1, 2, 300, "bf16")
    prm = rpg.Params(omega=torch.from_numpy(om).cuda())
    g = dev(torch, np.random.default_rng(1).standard_normal((1, 2, 300, 64)), "bf16")
    args = [dev(torch, x, "bf16") for x in (q, k, v)] + [g]
    a = [x.clone() for x in rpg.sanatan_attention_backward(*args, p, prm)]
    b = [x.clone() for x in rpg.sanatan_attention_backward(*args, p, prm)]
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("p", [1, 2])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_saved_statistics(torch_dev, dtype, p):
    """The training pair: the statistics sanatan_quadratic_train saved fed to sanatan_attention_backward_saved
    (at p = 2 delta comes from the saved fp32 output rows instead of a statistics pass; at p = 1 the saved
    values are not read), against the oracle at the same bars, with several tiles, a ragged last one and heads
    sharing omega rows."""
    errs = run_case(torch_dev, 850 + p, 2, 3, 200, dtype, p, nph=2, pos0=77, saved=True)
    for name, e in errs.items():
        assert e <= TOL[dtype], (name, e)


def test_backward_saved_statistics_long_bf16(torch_dev):
    """p = 2, bf16, 1000 tokens: delta over a long causal prefix (from a bf16-rounded output instead, dq reached
    2.5e-2 here)."""
    errs = run_case(torch_dev, 860, 1, 2, 1000, "bf16", 2, saved=True)
    for name, e in errs.items():
        assert e <= TOL["bf16"], (name, e)


@pytest.mark.parametrize("p", [1, 2])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quadratic_train_outputs(torch_dev, dtype, p):
    """sanatan_quadratic_train's output is bitwise sanatan_quadratic_ref_p2's; the saved fp32 rows round to it;
    the saved normaliser is 1 / (sum_{s<=t} kappa_ts^p + eps c^p) with kappa from the oracle's features
    ([N] §2.3, §2.6), per row; and the saved rows match the oracle's output at the forward's bar."""
    import root_parity_gated_amd as rpg

    torch = torch_dev
    B, H, T, pos0 = 1, 2, 150, 5
    q, k, v, om = si.attention_inputs(870 + p, B, H, T, dtype)
    prm = rpg.Params(omega=torch.from_numpy(np.ascontiguousarray(om, dtype=np.float32)).cuda())
    qd, kd, vd = dev(torch, q, dtype), dev(torch, k, dtype), dev(torch, v, dtype)
    out, sv = rpg.sanatan_quadratic_train(qd, kd, vd, p, prm, pos0=pos0)
    ref = rpg.sanatan_quadratic_ref_p2(qd, kd, vd, p, prm, pos0=pos0)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    o32 = sv[: B * H * T * 64].view(B, H, T, 64)
    inv_dn = sv[B * H * T * 64:].view(B, H, T)
    assert torch.equal(o32.to(out.dtype), out)
    c = 4.0 * 64
    worst, worst_o = 0.0, 0.0
    for h in range(H):
        fq = oracle.features(q[0, h], pos0, om[h])
        fk = oracle.features(k[0, h], pos0, om[h])
        kap = np.tril(fq @ fk.T) ** p
        want = 1.0 / (kap.sum(1) + 1e-6 * c ** p)
        got = host(inv_dn[0, h])
        worst = max(worst, float(np.max(np.abs(got - want) / want)))
        wo = oracle.attention_direct(q[0, h], k[0, h], v[0, h], om[h], pos0=pos0, p=p)
        worst_o = max(worst_o, row_rel_err(host(o32[0, h]), wo))
    print(f"saved statistics {dtype} p={p}: 1/Dn max relative error {worst:.3e}, fp32 rows {worst_o:.3e}")
    record(f"saved normaliser 1/Dn {dtype} p={p}", worst, TOL[dtype])
    record(f"saved fp32 output rows {dtype} p={p}", worst_o, TOL[dtype])
    assert worst <= TOL[dtype], worst
    assert worst_o <= TOL[dtype], worst_o
