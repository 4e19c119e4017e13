"""Serving-side decode against the fp64 oracle: one position per head-state (a batch whose sequences have
reached different lengths), and the handoff from prefill to decode for prompts of different lengths.

The position of a token sets the rotation of both of its feature maps (SANATAN reading notes §2.2); the state
carries everything else (§2.7), so a head-state continued at its own position must match the recurrence run
over its whole sequence.  Tolerances are the parity bars of the other GPU tests: row-wise max relative error
<= 1e-4 where every input is fp32, <= 2e-2 where the prompt went through the bf16 prefill.
"""
import numpy as np
import pytest

import oracle
import sanatan_inputs as si

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import root_parity_gated_amd as rpg

    rpg.lib()
    return torch


def dev(torch, x, dtype="f32"):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def params(torch, omega):
    import root_parity_gated_amd as rpg

    return rpg.Params(omega=torch.from_numpy(np.ascontiguousarray(omega, dtype=np.float32)).cuda())


def row_rel_err(got, want):
    got = np.asarray(got, np.float64).reshape(-1, want.shape[-1])
    want = np.asarray(want, np.float64).reshape(-1, want.shape[-1])
    return float((np.abs(got - want).max(1) / np.maximum(np.abs(want).max(1), 1e-12)).max())


@pytest.mark.parametrize("N,nph", [(1, 1), (37, 12)])
def test_decode_positions_per_head_state(torch_dev, N, nph):
    """Every head-state at its own position (0 and up to 2^20), six steps from an empty state."""
    import root_parity_gated_amd as rpg

    torch = torch_dev
    steps = 6
    om, _, (sq, sk, sv) = si.decode_inputs_numpy(500 + N, N, 1, steps)
    om = om[:nph]
    pos = si.decode_positions(510 + N, N)
    pos[0] = 0
    p = params(torch, om)
    S = torch.zeros((N, 384, 64), device="cuda")
    z = torch.zeros((N, 384), device="cuda")
    outs = []
    for s in range(steps):
        pd = torch.from_numpy(pos + s).cuda()
        outs.append(rpg.sanatan_decode_step_positions(dev(torch, sq[s]), dev(torch, sk[s]), dev(torch, sv[s]), pd, p,
                                                      S, z).clone())
    torch.cuda.synchronize()
    got = np.stack([host(o) for o in outs], 1)  # [N, steps, dv]
    Sg, zg = host(S), host(z)
    for i in range(N):
        want, Sw, zw = oracle.recurrent_heads(sq[:, i:i + 1].transpose(1, 0, 2), sk[:, i:i + 1].transpose(1, 0, 2),
                                              sv[:, i:i + 1].transpose(1, 0, 2), om[i % nph:i % nph + 1],
                                              pos0=int(pos[i]))
        assert row_rel_err(got[i], want[0]) <= 1e-4, (i, int(pos[i]))
        assert np.abs(Sg[i] - Sw[0]).max() <= 1e-4 * max(1.0, np.abs(Sw).max())
        assert np.abs(zg[i] - zw[0]).max() <= 1e-4 * max(1.0, np.abs(zw).max())


def test_decode_positions_equal_is_the_single_position_call(torch_dev):
    """All entries equal to one position: bitwise the same outputs and state as the single-position call."""
    import root_parity_gated_amd as rpg

    torch = torch_dev
    N, steps = 24, 3
    om, _, (sq, sk, sv) = si.decode_inputs_numpy(520, N, 1, steps)
    p = params(torch, om)
    S1 = torch.zeros((N, 384, 64), device="cuda")
    z1 = torch.zeros((N, 384), device="cuda")
    S2, z2 = S1.clone(), z1.clone()
    for s in range(steps):
        a = rpg.sanatan_decode_step(dev(torch, sq[s]), dev(torch, sk[s]), dev(torch, sv[s]), 4096 + s, p, S1, z1)
        pd = torch.full((N,), 4096 + s, dtype=torch.int64, device="cuda")
        b = rpg.sanatan_decode_step_positions(dev(torch, sq[s]), dev(torch, sk[s]), dev(torch, sv[s]), pd, p, S2, z2)
        assert torch.equal(a, b)
    assert torch.equal(S1, S2) and torch.equal(z1, z2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_decode_handoff_ragged_prompts(torch_dev, dtype):
    """Three sequences of 2 heads with prompts of 37, 128 and 300 tokens, each prefilled with its final state
    (one call per prompt length), then decoded together for five steps, each head-state at its own position.
    Decode outputs and final states against the recurrence over prompt + decoded tokens."""
    import root_parity_gated_amd as rpg

    torch = torch_dev
    H, steps, lens = 2, 5, [37, 128, 300]
    nb = len(lens)
    N = nb * H
    om = si.attention_inputs(530, 1, H, 1, dtype)[3]
    p = params(torch, om)
    S = torch.zeros((nb, H, 384, 64), device="cuda")
    z = torch.zeros((nb, H, 384), device="cuda")
    prompts = []
    for b, T in enumerate(lens):
        q, k, v, _ = si.attention_inputs(531 + b, 1, H, T, dtype)
        prompts.append((q[0], k[0], v[0]))
        rpg.sanatan_prefill_chunked(dev(torch, q, dtype), dev(torch, k, dtype), dev(torch, v, dtype), 64, p,
                                    S=S[b:b + 1], z=z[b:b + 1])
    _, _, (sq, sk, sv) = si.decode_inputs_numpy(540, N, 1, steps)
    pos = np.repeat(np.asarray(lens, dtype=np.int64), H)  # head-state b*H + h continues sequence b
    Sf, zf = S.view(N, 384, 64), z.view(N, 384)
    outs = []
    for s in range(steps):
        pd = torch.from_numpy(pos + s).cuda()
        outs.append(rpg.sanatan_decode_step_positions(dev(torch, sq[s]), dev(torch, sk[s]), dev(torch, sv[s]), pd, p,
                                                      Sf, zf).clone())
    torch.cuda.synchronize()
    got = np.stack([host(o) for o in outs], 1).reshape(nb, H, steps, -1)
    tol = 1e-4 if dtype == "f32" else 2e-2
    for b, T in enumerate(lens):
        pq, pk, pv = prompts[b]
        dq = sq[:, b * H:(b + 1) * H].transpose(1, 0, 2)
        dk = sk[:, b * H:(b + 1) * H].transpose(1, 0, 2)
        dvv = sv[:, b * H:(b + 1) * H].transpose(1, 0, 2)
        want, Sw, zw = oracle.recurrent_heads(np.concatenate([pq, dq], 1), np.concatenate([pk, dk], 1),
                                              np.concatenate([pv, dvv], 1), om)
        assert row_rel_err(got[b], want[:, T:]) <= tol, (b, T)
        assert np.abs(host(S[b]) - Sw).max() <= tol * np.abs(Sw).max()
        assert np.abs(host(z[b]) - zw).max() <= tol * np.abs(zw).max()


# ---- compact state: the d equal channel-0 rows of S (and entries of z) kept once, (5d+1) rows


def test_compact_expand_round_trip_is_bitwise(torch_dev):
    """Compacting keeps row 0 and rows d..6d-1; expanding writes the shared row into all d channel-0 rows."""
    import root_parity_gated_amd as rpg

    torch = torch_dev
    N = 5
    g = torch.Generator(device="cuda").manual_seed(600)
    S = torch.randn((N, 384, 64), device="cuda", generator=g)
    z = torch.rand((N, 384), device="cuda", generator=g)
    S[:, 1:64] = S[:, :1]
    z[:, 1:64] = z[:, :1]
    Sc, zc = rpg.sanatan_state_compact(S, z)
    assert Sc.shape == (N, 321, 64) and zc.shape == (N, 321)
    assert torch.equal(Sc[:, 0], S[:, 0]) and torch.equal(Sc[:, 1:], S[:, 64:])
    assert torch.equal(zc[:, 0], z[:, 0]) and torch.equal(zc[:, 1:], z[:, 64:])
    S2, z2 = rpg.sanatan_state_expand(Sc, zc)
    assert torch.equal(S2, S) and torch.equal(z2, z)


@pytest.mark.parametrize("per_head", [False, True])
def test_decode_compact_matches_recurrence(torch_dev, per_head):
    """37 head-states continued from a 200-token fp32 prefill: the compact decode for six steps (one position
    for all, or one per head-state) against the recurrence over the whole sequence; the expanded final
    state against the recurrence's state."""
    import root_parity_gated_amd as rpg

    torch = torch_dev
    N, T, steps = 37, 200, 6
    q, k, v, om = si.attention_inputs(610, 1, N, T, "f32")
    p = params(torch, om)
    S = torch.zeros((1, N, 384, 64), device="cuda")
    z = torch.zeros((1, N, 384), device="cuda")
    rpg.sanatan_prefill_chunked(dev(torch, q), dev(torch, k), dev(torch, v), 64, p, S=S, z=z)
    Sc, zc = rpg.sanatan_state_compact(S[0], z[0])
    _, _, (sq, sk, sv) = si.decode_inputs_numpy(611, N, 1, steps)
    outs = []
    for s in range(steps):
        pos = torch.full((N,), T + s, dtype=torch.int64, device="cuda") if per_head else T + s
        outs.append(rpg.sanatan_decode_step_compact(dev(torch, sq[s]), dev(torch, sk[s]), dev(torch, sv[s]), pos, p,
                                                    Sc, zc).clone())
    S2, z2 = rpg.sanatan_state_expand(Sc, zc)
    torch.cuda.synchronize()
    got = np.stack([host(o) for o in outs], 1)
    want, Sw, zw = oracle.recurrent_heads(np.concatenate([q[0], sq.transpose(1, 0, 2)], 1),
                                          np.concatenate([k[0], sk.transpose(1, 0, 2)], 1),
                                          np.concatenate([v[0], sv.transpose(1, 0, 2)], 1), om)
    assert row_rel_err(got, want[:, T:]) <= 1e-4
    assert np.abs(host(S2) - Sw).max() <= 1e-4 * np.abs(Sw).max()
    assert np.abs(host(z2) - zw).max() <= 1e-4 * np.abs(zw).max()


def test_decode_compact_streamed_equals_full(torch_dev):
    """1700 head-states (a 142 MB compact state, streamed with non-temporal accesses) at their own positions,
    three steps from an empty state: the expanded compact state equals the full-state call's bit for bit (the
    updates are the same operations), the outputs agree to the rounding of the channel-0 readout, and eight
    sampled head-states match the recurrence."""
    import root_parity_gated_amd as rpg

    torch = torch_dev
    N, steps = 1700, 3
    om, _, (sq, sk, sv) = si.decode_inputs_numpy(620, N, 1, steps)
    om = om[:12]
    p = params(torch, om)
    pos = si.decode_positions(621, N, 0, 1 << 16)
    S = torch.zeros((N, 384, 64), device="cuda")
    z = torch.zeros((N, 384), device="cuda")
    Sc = torch.zeros((N, 321, 64), device="cuda")
    zc = torch.zeros((N, 321), device="cuda")
    full, comp = [], []
    for s in range(steps):
        pd = torch.from_numpy(pos + s).cuda()
        a = (dev(torch, sq[s]), dev(torch, sk[s]), dev(torch, sv[s]))
        full.append(rpg.sanatan_decode_step_positions(*a, pd, p, S, z).clone())
        comp.append(rpg.sanatan_decode_step_compact(*a, pd, p, Sc, zc).clone())
    S2, z2 = rpg.sanatan_state_expand(Sc, zc)
    torch.cuda.synchronize()
    assert torch.equal(S2, S) and torch.equal(z2, z)
    gf = np.stack([host(o) for o in full], 1)
    gc = np.stack([host(o) for o in comp], 1)
    assert row_rel_err(gc, gf) <= 1e-5
    for i in np.random.default_rng(622).choice(N, 8, replace=False):
        want, _, _ = oracle.recurrent_heads(sq[:, i:i + 1].transpose(1, 0, 2), sk[:, i:i + 1].transpose(1, 0, 2),
                                            sv[:, i:i + 1].transpose(1, 0, 2), om[i % 12:i % 12 + 1],
                                            pos0=int(pos[i]))
        assert row_rel_err(gc[i], want[0]) <= 1e-4, int(i)
