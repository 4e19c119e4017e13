"""The spectral-harmonic and the unclipped four-channel maps on the GPU, against the oracle.

Spectral harmonics (the notes' Appendix B outlook; reading: harmonics n = 1..nh of the rotated angle, gated by
the root label): the chunked prefill against the oracle's direct kappa_h form and its recurrence (outputs and
final state), the decode step continuing a prefilled state against the recurrence, and nh = 1 against the
six-channel oracle.  Unclipped four-channel kernel ([N] §2.5): the chunked prefill against the oracle's
four-channel direct form, its compact final state against the six-channel recurrence's rows of the same
features, and the handoff to sanatan_decode_step_four_channel.  Bars: 1e-4 (fp32 inputs), 2e-2 (bf16).
"""
import numpy as np
import pytest

import oracle
import sanatan_inputs as si
from parity_log import record

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
D = 64


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


def params(torch, omega, **kw):
    import root_parity_gated_amd as rpg

    return rpg.Params(omega=torch.from_numpy(np.ascontiguousarray(omega, dtype=np.float32)).cuda(), **kw)


def row_rel_err(got, want):
    got = np.asarray(got, np.float64).reshape(-1, want.shape[-1])
    want = np.asarray(want, np.float64).reshape(-1, want.shape[-1])
    return float((np.abs(got - want).max(1) / np.maximum(np.abs(want).max(1), 1e-12)).max())


@pytest.mark.parametrize("nh", [1, 2])
@pytest.mark.parametrize("dtype,T", [("f32", 150), ("bf16", 300)])
def test_harmonics_prefill(torch_dev, nh, dtype, T):
    """Outputs against the direct kappa_h form (the six-channel oracle at nh = 1), final state against the
    recurrence, with a nonzero initial state for half of the heads' history."""
    import root_parity_gated_amd as rpg

    torch = torch_dev
    B, H = 1, 3
    q, k, v, om = si.attention_inputs(900 + nh, B, H, T, dtype)
    rows = (2 + 4 * nh) * D
    S = torch.zeros((B, H, rows, 64), device="cuda")
    z = torch.zeros((B, H, rows), device="cuda")
    p = params(torch, om)
    half = T // 2
    out1 = rpg.sanatan_prefill_harmonics(dev(torch, q[:, :, :half], dtype), dev(torch, k[:, :, :half], dtype),
                                         dev(torch, v[:, :, :half], dtype), nh, p, S=S, z=z)
    out2 = rpg.sanatan_prefill_harmonics(dev(torch, q[:, :, half:], dtype), dev(torch, k[:, :, half:], dtype),
                                         dev(torch, v[:, :, half:], dtype), nh, p, pos0=half, S=S, z=z)
    torch.cuda.synchronize()
    got = np.concatenate([host(out1), host(out2)], 2)
    err = 0.0
    for h in range(H):
        if nh == 1:
            want = oracle.attention_direct(q[0, h], k[0, h], v[0, h], om[h])
        else:
            want = oracle.attention_direct_h(q[0, h], k[0, h], v[0, h], om[h], nh)
        err = max(err, row_rel_err(got[0, h], want))
        _, Sw, zw = oracle.recurrent_h(q[0, h], k[0, h], v[0, h], om[h], nh, want_out=False)
        assert np.abs(host(S)[0, h] - Sw).max() <= TOL[dtype] * np.abs(Sw).max()
        assert np.abs(host(z)[0, h] - zw).max() <= TOL[dtype] * np.abs(zw).max()
    print(f"harmonics nh={nh} {dtype} T={T}: max row error {err:.3e}")
    assert record(f"harmonics prefill nh={nh} {dtype}", err, TOL[dtype]) <= TOL[dtype]


@pytest.mark.parametrize("nh", [1, 2])
def test_harmonics_decode_continues_prefill(torch_dev, nh):
    """A 100-token fp32 prefill, then 6 decode steps (one position for all, then one per head-state), against
    the recurrence over the whole sequence."""
    import root_parity_gated_amd as rpg

    torch = torch_dev
    N, T, steps = 5, 100, 6
    q, k, v, om = si.attention_inputs(910 + nh, 1, N, T + steps, "f32")
    rows = (2 + 4 * nh) * D
    p = params(torch, om)
    S = torch.zeros((1, N, rows, 64), device="cuda")
    z = torch.zeros((1, N, rows), device="cuda")
    rpg.sanatan_prefill_harmonics(dev(torch, q[:, :, :T], "f32"), dev(torch, k[:, :, :T], "f32"),
                                  dev(torch, v[:, :, :T], "f32"), nh, p, S=S, z=z)
    got = []
    for i in range(steps):
        pos = T + i if i < 3 else torch.full((N,), T + i, dtype=torch.int64, device="cuda")
        o = rpg.sanatan_decode_step_harmonics(dev(torch, q[0, :, T + i], "f32"), dev(torch, k[0, :, T + i], "f32"),
                                              dev(torch, v[0, :, T + i], "f32"), pos, nh, p, S[0], z[0])
        got.append(host(o))
    torch.cuda.synchronize()
    err = 0.0
    for h in range(N):
        want, Sw, zw = oracle.recurrent_h(q[0, h], k[0, h], v[0, h], om[h], nh)
        err = max(err, row_rel_err(np.stack(got, 1)[h], want[T:]))
        assert np.abs(host(S)[0, h] - Sw).max() <= 1e-4 * np.abs(Sw).max()
        assert np.abs(host(z)[0, h] - zw).max() <= 1e-4 * np.abs(zw).max()
    print(f"harmonics decode nh={nh}: max row error {err:.3e}")
    assert record(f"harmonics decode nh={nh} f32", err, TOL["f32"]) <= TOL["f32"]


@pytest.mark.parametrize("dtype,T", [("f32", 97), ("bf16", 260)])
def test_four_channel_prefill(torch_dev, dtype, T):
    """Outputs against the oracle's four-channel direct form; the compact final state (before the decode steps)
    against the six-channel recurrence's rows of the same features (channel 0 once, then r, r cos, r sin); then
    two decode steps continuing it."""
    import root_parity_gated_amd as rpg

    torch = torch_dev
    B, H = 1, 2
    q, k, v, om = si.attention_inputs(930, B, H, T + 2, dtype)
    p = params(torch, om)
    S4 = torch.zeros((B, H, 3 * D + 1, 64), device="cuda")
    z4 = torch.zeros((B, H, 3 * D + 1), device="cuda")
    out = rpg.sanatan_prefill_four_channel(dev(torch, q[:, :, :T], dtype), dev(torch, k[:, :, :T], dtype),
                                           dev(torch, v[:, :, :T], dtype), p, S4=S4, z4=z4)
    S4_after, z4_after = host(S4), host(z4)
    dec = []
    for i in range(2):
        dec.append(host(rpg.sanatan_decode_step_four_channel(
            torch.from_numpy(q[0, :, T + i].astype(np.float32)).cuda(),
            torch.from_numpy(k[0, :, T + i].astype(np.float32)).cuda(),
            torch.from_numpy(v[0, :, T + i].astype(np.float32)).cuda(), T + i, p, S4[0], z4[0])))
    torch.cuda.synchronize()
    got = host(out)
    err = errd = 0.0
    for h in range(H):
        want = oracle.attention_direct(q[0, h], k[0, h], v[0, h], om[h], four_channel=True)
        err = max(err, row_rel_err(got[0, h], want[:T]))
        errd = max(errd, row_rel_err(np.stack([dd[h] for dd in dec]), want[T:]))
        _, S6, z6 = oracle.recurrent(q[0, h, :T], k[0, h, :T], v[0, h, :T], om[h], want_out=False)
        rows6 = [0] + list(range(3 * D, 6 * D))
        Sw, zw = S6[rows6], z6[rows6]
        assert np.abs(S4_after[0, h] - Sw).max() <= TOL[dtype] * np.abs(Sw).max()
        assert np.abs(z4_after[0, h] - zw).max() <= TOL[dtype] * np.abs(zw).max()
    print(f"four-channel prefill {dtype} T={T}: max row error {err:.3e}, decode after it {errd:.3e}")
    assert record(f"four-channel chunked prefill {dtype}", err, TOL[dtype]) <= TOL[dtype]
    assert record(f"four-channel decode (fp32) after a {dtype} prefill", errd, TOL[dtype]) <= TOL[dtype]


@pytest.mark.parametrize("kind", ["nh1", "nh2", "four"])
def test_feature_prefill_split_and_unsplit(torch_dev, kind):
    """The sequence split (pieces of whole chunks over several workgroups, a state pass that may cut each piece
    into parts, and a start state summed from the parts' slots) and the unsplit form (at least as many sequences as compute units), both
    with a caller state, against the oracle; every sequence's outputs and final state are checked."""
    import root_parity_gated_amd as rpg

    torch = torch_dev
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    # split into up to 8 pieces; at T = 1000 (8 pieces of 4 chunks, the last ragged) the state pass runs each
    # piece as 4 one-chunk parts with a slot each; then unsplit
    for B, H, T in ((1, 2, 333), (1, 2, 1000), (2, (n_cu + 1) // 2, 70)):
        q, k, v, om = si.attention_inputs(950 + T, B, H, T + 20, "bf16")
        p = params(torch, om)
        nh = {"nh1": 1, "nh2": 2, "four": 0}[kind]
        rows = (2 + 4 * nh) * D if nh else 3 * D + 1
        # caller state: the prefill of 20 earlier tokens (positions 0..19), checked through the outputs below
        S = torch.zeros((B, H, rows, 64), device="cuda")
        z = torch.zeros((B, H, rows), device="cuda")
        pre, main = slice(0, 20), slice(20, 20 + T)
        run = (lambda a, b, c, **kw: rpg.sanatan_prefill_harmonics(a, b, c, nh, p, **kw)) if nh else (
            lambda a, b, c, **kw: rpg.sanatan_prefill_four_channel(a, b, c, p, S4=kw.pop("S"), z4=kw.pop("z"), **kw))
        run(dev(torch, q[:, :, pre], "bf16"), dev(torch, k[:, :, pre], "bf16"), dev(torch, v[:, :, pre], "bf16"),
            S=S, z=z)
        out = run(dev(torch, q[:, :, main], "bf16"), dev(torch, k[:, :, main], "bf16"),
                  dev(torch, v[:, :, main], "bf16"), pos0=20, S=S, z=z)
        torch.cuda.synchronize()
        got, Sg, zg = host(out), host(S), host(z)
        err = serr = 0.0
        for b in range(B):
            for h in range(H):
                if nh:
                    want = oracle.attention_direct_h(q[b, h], k[b, h], v[b, h], om[h], nh)[20:]
                    _, Sw, zw = oracle.recurrent_h(q[b, h], k[b, h], v[b, h], om[h], nh, want_out=False)
                else:
                    want = oracle.attention_direct(q[b, h], k[b, h], v[b, h], om[h], four_channel=True)[20:]
                    _, S6, z6 = oracle.recurrent(q[b, h], k[b, h], v[b, h], om[h], want_out=False)
                    rows6 = [0] + list(range(3 * D, 6 * D))
                    Sw, zw = S6[rows6], z6[rows6]
                err = max(err, row_rel_err(got[b, h], want))
                serr = max(serr, np.abs(Sg[b, h] - Sw).max() / np.abs(Sw).max(), np.abs(zg[b, h] - zw).max() / np.abs(zw).max())
        print(f"feature prefill {kind} B{B} H{H} T{T}: output {err:.3e}, state {serr:.3e}")
        assert record(f"feature-map prefill {kind} bf16 (split and unsplit)", err, TOL["bf16"]) <= TOL["bf16"]
        assert serr <= TOL["bf16"]
