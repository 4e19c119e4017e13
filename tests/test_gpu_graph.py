"""Replays of captured HIP graphs give the eager results (bit for bit: the kernels are deterministic).

The prefill (phase table, pass 1, pass 3), a run of decode steps and the backward pass are captured once; each
replay is separated by unrelated eager work and a synchronisation, and every replay is compared with the eager
output of the same call.  bench.py times graph replays of the same calls.
"""
import numpy as np
import pytest

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


def test_prefill_graph_replays_match_eager(torch_dev):
    import root_parity_gated_amd as rpg

    torch = torch_dev
    B, H, T, C = 2, 4, 1000, 64  # 32 chunks over at most #CU workgroups: several pieces per sequence
    q, k, v, om = si.attention_inputs(31, B, H, T, "bf16")
    qd, kd, vd = (torch.from_numpy(x).cuda().to(torch.bfloat16) for x in (q, k, v))
    p = rpg.Params(omega=torch.from_numpy(om).cuda())
    ws = torch.empty((rpg.sanatan_prefill_workspace_bytes(B, H, T, C, p),), dtype=torch.uint8, device="cuda")
    S = torch.zeros((B, H, 384, 64), device="cuda")
    z = torch.zeros((B, H, 384), device="cuda")
    eager = torch.empty_like(vd)
    rpg.sanatan_prefill_chunked(qd, kd, vd, C, p, out=eager, ws=ws, S=S, z=z)
    S_eager, z_eager = S.clone(), z.clone()
    torch.cuda.synchronize()

    out = torch.empty_like(vd)
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    S.zero_()
    z.zero_()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        rpg.sanatan_prefill_chunked(qd, kd, vd, C, p, out=out, ws=ws, S=S, z=z)
    other = torch.empty((B, H, T, 64), device="cuda", dtype=torch.bfloat16)
    for rep in range(3):
        S.zero_()
        z.zero_()
        out.fill_(float("nan"))
        other.normal_()  # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep
        assert torch.equal(S, S_eager) and torch.equal(z, z_eager), rep


def test_decode_graph_replays_match_eager(torch_dev):
    import root_parity_gated_amd as rpg

    torch = torch_dev
    nh, steps = 144, 4
    om, (fq, fk, fv), (sq, sk, sv) = si.decode_inputs_numpy(57, nh, 8, steps)
    dv = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    sq, sk, sv = map(dv, (sq, sk, sv))
    p = rpg.Params(omega=dv(om))
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    S0 = torch.randn((nh, 384, 64), device="cuda", generator=g) * 0.01
    z0 = torch.rand((nh, 384), device="cuda", generator=g) + 1.0
    S, z = S0.clone(), z0.clone()
    eager = torch.empty((steps, nh, 64), device="cuda")
    for i in range(steps):
        rpg.sanatan_decode_step(sq[i], sk[i], sv[i], 4096 + i, p, S, z, eager[i])
    S_eager, z_eager = S.clone(), z.clone()

    out = torch.empty_like(eager)
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    S.copy_(S0)
    z.copy_(z0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(steps):
            rpg.sanatan_decode_step(sq[i], sk[i], sv[i], 4096 + i, p, S, z, out[i])
    for rep in range(3):
        S.copy_(S0)
        z.copy_(z0)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep
        assert torch.equal(S, S_eager) and torch.equal(z, z_eager), rep


def test_serving_decode_graph_replays_match_eager(torch_dev):
    """The per-head-state-position decode and the compact-state decode, four steps each, captured once and
    replayed three times with unrelated eager work in between: every replay bitwise equal to the eager run."""
    import root_parity_gated_amd as rpg

    torch = torch_dev
    nh, steps = 144, 4
    om, _, (sq, sk, sv) = si.decode_inputs_numpy(58, nh, 1, steps)
    dv = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    sq, sk, sv = map(dv, (sq, sk, sv))
    p = rpg.Params(omega=dv(om))
    pos = dv(si.decode_positions(59, nh) + np.arange(steps)[:, None])  # [steps, nh]
    g = torch.Generator(device="cuda")
    g.manual_seed(6)
    S0 = torch.randn((nh, 384, 64), device="cuda", generator=g) * 0.01
    z0 = torch.rand((nh, 384), device="cuda", generator=g) + 1.0
    S0[:, 1:64] = S0[:, :1]
    z0[:, 1:64] = z0[:, :1]
    Sc0, zc0 = rpg.sanatan_state_compact(S0, z0)

    def run(S, z, Sc, zc, o1, o2):
        for i in range(steps):
            rpg.sanatan_decode_step_positions(sq[i], sk[i], sv[i], pos[i], p, S, z, o1[i])
            rpg.sanatan_decode_step_compact(sq[i], sk[i], sv[i], pos[i], p, Sc, zc, o2[i])

    S, z, Sc, zc = S0.clone(), z0.clone(), Sc0.clone(), zc0.clone()
    e1, e2 = torch.empty((steps, nh, 64), device="cuda"), torch.empty((steps, nh, 64), device="cuda")
    run(S, z, Sc, zc, e1, e2)
    want = [t.clone() for t in (S, z, Sc, zc)]

    o1, o2 = torch.empty_like(e1), torch.empty_like(e2)
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    for t, t0 in zip((S, z, Sc, zc), (S0, z0, Sc0, zc0)):
        t.copy_(t0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        run(S, z, Sc, zc, o1, o2)
    for rep in range(3):
        for t, t0 in zip((S, z, Sc, zc), (S0, z0, Sc0, zc0)):
            t.copy_(t0)
        o1.fill_(float("nan"))
        o2.fill_(float("nan"))
        torch.randn((1 << 20,), device="cuda").sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o1, e1) and torch.equal(o2, e2), rep
        for got, w in zip((S, z, Sc, zc), want):
            assert torch.equal(got, w), rep


@pytest.mark.parametrize("p", [1, 2])
def test_backward_graph_replays_match_eager(torch_dev, p):
    """The backward pass captured once (at p = 1 several pieces per sequence: increments, forward direction,
    increments, reverse direction), replayed three times between unrelated eager work."""
    import root_parity_gated_amd as rpg

    torch = torch_dev
    B, H, T = 1, 3, 700
    q, k, v, om = si.attention_inputs(41 + p, B, H, T, "bf16")
    qd, kd, vd = (torch.from_numpy(x).cuda().to(torch.bfloat16) for x in (q, k, v))
    g = torch.from_numpy(np.random.default_rng(43).standard_normal((B, H, T, 64)).astype(np.float32)).cuda()
    g = g.to(torch.bfloat16)
    prm = rpg.Params(omega=torch.from_numpy(om).cuda())
    ws = torch.empty((rpg.sanatan_attention_backward_workspace_bytes(B, H, T, rpg.SANATAN_BF16, prm),),
                     dtype=torch.uint8, device="cuda")
    outs = [torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd),
            torch.empty((H, 64), dtype=torch.float32, device="cuda")]
    call = lambda: rpg.sanatan_attention_backward(qd, kd, vd, g, p, prm, dq=outs[0], dk=outs[1], dv=outs[2],
                                                  domega=outs[3], ws=ws)
    call()
    torch.cuda.synchronize()
    eager = [x.clone() for x in outs]
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        call()
    other = torch.empty((B, H, T, 64), device="cuda")
    for rep in range(3):
        for x in outs:
            x.fill_(float("nan"))
        other.normal_()  # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, x, y in zip(("dq", "dk", "dv", "domega"), outs, eager):
            assert torch.equal(x, y), (rep, name)
