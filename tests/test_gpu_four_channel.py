"""The masked quadratic form on the unclipped four-channel kernel (SANATAN reading notes §2.5: [1, r, r cos,
r sin] per dim, kappa4 = sum_a 1 + r_q r_k (1 + cos dtheta), no clipping) against the fp64 oracle's direct form.

Element by element on seeded inputs, p = 1 and 2, fp32 and bf16, from one token to several key blocks with a
ragged tail; at a longer sequence on sampled rows.  Bars: row-wise max relative error <= 1e-4 (fp32 inputs),
<= 2e-2 (bf16 inputs), as for the six-channel form.
"""
import numpy as np
import pytest

import oracle
import sanatan_inputs as si

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


def row_rel_err(got, want):
    got = np.asarray(got, np.float64).reshape(-1, want.shape[-1])
    want = np.asarray(want, np.float64).reshape(-1, want.shape[-1])
    return float((np.abs(got - want).max(1) / np.maximum(np.abs(want).max(1), 1e-12)).max())


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("p", [1, 2])
@pytest.mark.parametrize("T", [1, 33, 200])
def test_four_channel_matches_oracle(torch_dev, dtype, p, T):
    import root_parity_gated_amd as rpg

    torch = torch_dev
    B, H = 1, 2
    q, k, v, om = si.attention_inputs(700 + T + 10 * p, B, H, T, dtype)
    par = rpg.Params(omega=torch.from_numpy(om).cuda())
    out = rpg.sanatan_quadratic_four_channel(dev(torch, q, dtype), dev(torch, k, dtype), dev(torch, v, dtype), p,
                                             par)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    for h in range(H):
        want = oracle.attention_direct(q[0, h], k[0, h], v[0, h], om[h], p=p, four_channel=True)
        assert row_rel_err(got[0, h], want) <= TOL[dtype], h


@pytest.mark.parametrize("p", [1, 2])
def test_four_channel_long_sampled_rows(torch_dev, p):
    """B=2, H=3, T=1500 bf16: 40 sampled rows per head (block edges, the ends, seeded rows)."""
    import root_parity_gated_amd as rpg

    torch = torch_dev
    B, H, T = 2, 3, 1500
    q, k, v, om = si.attention_inputs(720 + p, B, H, T, "bf16")
    par = rpg.Params(omega=torch.from_numpy(om).cuda())
    out = rpg.sanatan_quadratic_four_channel(dev(torch, q, "bf16"), dev(torch, k, "bf16"), dev(torch, v, "bf16"),
                                             p, par)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    rng = np.random.default_rng(730 + p)
    rows = np.unique(np.concatenate([[0, 1, 31, 32, 127, 128, T - 1], rng.integers(0, T, 33)]))
    for b in range(B):
        for h in range(H):
            want = oracle.attention_direct(q[b, h], k[b, h], v[b, h], om[h], p=p, four_channel=True, rows=rows)
            assert row_rel_err(got[b, h][rows], want) <= TOL["bf16"], (b, h)


def test_four_channel_differs_from_six_channel(torch_dev):
    """The two kernels are different functions: on the same inputs their outputs are far apart."""
    import root_parity_gated_amd as rpg

    torch = torch_dev
    q, k, v, om = si.attention_inputs(740, 1, 1, 64, "f32")
    par = rpg.Params(omega=torch.from_numpy(om).cuda())
    a = rpg.sanatan_quadratic_four_channel(dev(torch, q, "f32"), dev(torch, k, "f32"), dev(torch, v, "f32"), 2, par)
    b = rpg.sanatan_quadratic_ref_p2(dev(torch, q, "f32"), dev(torch, k, "f32"), dev(torch, v, "f32"), 2, par)
    torch.cuda.synchronize()
    assert row_rel_err(a.cpu().numpy(), b.cpu().numpy().astype(np.float64)) > 1e-2


@pytest.mark.parametrize("per_head", [False, True])
def test_four_channel_decode_matches_direct_form(torch_dev, per_head):
    """37 head-states, eight tokens from an empty state on the four-channel kernel's state ((3d+1) rows).  The
    outputs equal the direct p=1 form's rows (the recurrence is exact for the unclipped kernel); the state equals
    the six-channel recurrence's rows of channels 0, 3, 4, 5 (the same features), channel 0 kept once."""
    import root_parity_gated_amd as rpg

    torch = torch_dev
    N, steps, nph = 37, 8, 12
    om, _, (sq, sk, sv) = si.decode_inputs_numpy(750, N, 1, steps)
    om = om[:nph]
    par = rpg.Params(omega=torch.from_numpy(om).cuda())
    pos0 = si.decode_positions(751, N, 0, 1 << 16) if per_head else np.full(N, 300, dtype=np.int64)
    S4 = torch.zeros((N, 193, 64), device="cuda")
    z4 = torch.zeros((N, 193), device="cuda")
    outs = []
    for s in range(steps):
        pos = torch.from_numpy(pos0 + s).cuda() if per_head else 300 + s
        outs.append(rpg.sanatan_decode_step_four_channel(dev(torch, sq[s], "f32"), dev(torch, sk[s], "f32"),
                                                         dev(torch, sv[s], "f32"), pos, par, S4, z4).clone())
    torch.cuda.synchronize()
    got = np.stack([o.cpu().numpy() for o in outs], 1)
    Sg, zg = S4.cpu().numpy().astype(np.float64), z4.cpu().numpy().astype(np.float64)
    rows6 = np.concatenate([[0], np.arange(3 * 64, 6 * 64)])
    for i in range(N):
        q, k, v = sq[:, i], sk[:, i], sv[:, i]
        want = oracle.attention_direct(q, k, v, om[i % nph], p=1, four_channel=True)
        assert row_rel_err(got[i], want) <= 1e-4, i
        _, S6, z6 = oracle.recurrent_heads(q[None], k[None], v[None], om[i % nph:i % nph + 1], pos0=int(pos0[i]))
        assert np.abs(Sg[i] - S6[0][rows6]).max() <= 1e-4 * max(1.0, np.abs(S6).max()), i
        assert np.abs(zg[i] - z6[0][rows6]).max() <= 1e-4 * max(1.0, np.abs(z6).max()), i
