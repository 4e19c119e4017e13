"""Prefill with a caller state when sequences are split into pieces over workgroups, and positions at the edge
of the accepted range.

A sequence whose chunks span several workgroups is a chain of pieces; its final piece writes the caller's
state back in place.  Every piece must have read the initial state before that write, whichever workgroup
runs first.  These tests take more sequences than workgroups (so that a workgroup's range holds the final
piece of one sequence and the head piece of the next), a nonzero initial state, and check every output row
of every sequence, not only the final state.

Positions enter only through t - s ([N] §2.2, rotation), so a prefill or decode run near the largest accepted
position |pos| < 2^53 must match the oracle run at small positions.
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


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def params(torch, omega, **kw):
    import root_parity_gated_amd as rpg

    return rpg.Params(omega=torch.from_numpy(np.ascontiguousarray(omega, dtype=np.float32)).cuda(), **kw)


def row_rel_err(got, want):
    got = np.asarray(got, np.float64).reshape(-1, want.shape[-1])
    want = np.asarray(want, np.float64).reshape(-1, want.shape[-1])
    return float((np.abs(got - want).max(1) / np.maximum(np.abs(want).max(1), 1e-12)).max())


def oracle_heads(q, k, v, omega, pos0=0, **kw):
    B, H, T, d = q.shape
    out, S, z = oracle.recurrent_heads(q.reshape(B * H, T, d), k.reshape(B * H, T, d), v.reshape(B * H, T, -1),
                                       np.tile(omega, (B, 1)), pos0=pos0, **kw)
    return out.reshape(B, H, T, -1), S.reshape(B, H, *S.shape[1:]), z.reshape(B, H, -1)


def _run_with_state(torch, B, H, T, chunk, dtype, seed, workgroups):
    import root_parity_gated_amd as rpg

    q, k, v, om = si.attention_inputs(seed, B, H, T, dtype)
    pq, pk, pv, _ = si.attention_inputs(seed + 1, B, H, 96, dtype)
    _, S0, z0 = oracle_heads(pq, pk, pv, om)
    S = torch.from_numpy(S0.astype(np.float32)).cuda()
    z = torch.from_numpy(z0.astype(np.float32)).cuda()
    out = rpg.sanatan_prefill_chunked_partitioned(dev(torch, q, dtype), dev(torch, k, dtype), dev(torch, v, dtype),
                                                  chunk, workgroups, params(torch, om), pos0=96, S=S, z=z)
    torch.cuda.synchronize()
    want, Sw, zw = oracle_heads(np.concatenate([pq, q], 2), np.concatenate([pk, k], 2),
                                np.concatenate([pv, v], 2), om)
    err = row_rel_err(host(out), want[:, :, 96:])
    print(f"prefill with state B{B} H{H} T{T} chunk {chunk} {dtype} workgroups {workgroups}: "
          f"max row error {err:.3e}")
    assert err <= TOL[dtype]
    assert np.abs(host(S) - Sw).max() <= TOL[dtype] * np.abs(Sw).max()
    assert np.abs(host(z) - zw).max() <= TOL[dtype] * np.abs(zw).max()


def test_state_more_sequences_than_workgroups_default_split(torch_dev):
    """384 sequences over one workgroup per CU: ranges hold a final piece, then the next head piece."""
    _run_with_state(torch_dev, 32, 12, 512, 64, "bf16", 610, 0)


@pytest.mark.parametrize("dtype,chunk,workgroups", [("bf16", 64, 20), ("bf16", 128, 7), ("bf16", 32, 37),
                                                    ("f32", 64, 20), ("f32", 16, 11)])
def test_state_forced_splits(torch_dev, dtype, chunk, workgroups):
    """48 sequences over a forced workgroup count that does not divide the chunk list."""
    _run_with_state(torch_dev, 4, 12, 384 + 17, chunk, dtype, 620 + workgroups, workgroups)


@pytest.mark.parametrize("dtype,chunk", [("f32", 64), ("bf16", 64), ("bf16", 128)])
def test_prefill_at_largest_position(torch_dev, dtype, chunk):
    """Positions up to 2^53 - 1: the output equals the oracle's at positions 0..T-1."""
    import root_parity_gated_amd as rpg

    torch = torch_dev
    T = 300
    q, k, v, om = si.attention_inputs(640, 1, 3, T, dtype)
    pos0 = (1 << 53) - T
    out = rpg.sanatan_prefill_chunked(dev(torch, q, dtype), dev(torch, k, dtype), dev(torch, v, dtype), chunk,
                                      params(torch, om), pos0=pos0)
    torch.cuda.synchronize()
    want, _, _ = oracle_heads(q, k, v, om)
    err = row_rel_err(host(out), want)
    print(f"prefill at pos0 = 2^53 - {T}, {dtype} chunk {chunk}: max row error {err:.3e}")
    assert err <= TOL[dtype]


def test_decode_at_largest_position(torch_dev):
    """A history prefilled on the GPU at positions 2^53 - 72 .. 2^53 - 9, then decode steps at
    2^53 - 8 .. 2^53 - 1: the outputs equal the recurrence at positions 0 .. 71 (only t - s matters)."""
    import root_parity_gated_amd as rpg

    torch = torch_dev
    N, T, steps = 5, 64, 8
    q, k, v, om = si.attention_inputs(650, 1, N, T + steps, "f32")
    base = (1 << 53) - steps
    p = params(torch, om)
    S = torch.zeros((1, N, 384, 64), device="cuda")
    z = torch.zeros((1, N, 384), device="cuda")
    rpg.sanatan_prefill_chunked(dev(torch, q[:, :, :T], "f32"), dev(torch, k[:, :, :T], "f32"),
                                dev(torch, v[:, :, :T], "f32"), 64, p, pos0=base - T, S=S, z=z)
    got = []
    for i in range(steps):
        o = rpg.sanatan_decode_step(dev(torch, q[0, :, T + i], "f32"), dev(torch, k[0, :, T + i], "f32"),
                                    dev(torch, v[0, :, T + i], "f32"), base + i, p, S[0], z[0])
        got.append(host(o))
    torch.cuda.synchronize()
    want, _, _ = oracle.recurrent_heads(q[0], k[0], v[0], om)
    err = row_rel_err(np.stack(got, 1), want[:, T:])
    print(f"decode at 2^53 - {steps}: max row error {err:.3e}")
    assert err <= TOL["f32"]
