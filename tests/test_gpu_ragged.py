"""A batch of sequences of different lengths in one prefill call (sanatan_prefill_chunked_ragged), against the
fp64 oracle's recurrence run on each sequence alone.

Batch element b uses the first lengths[b] rows of every head; the oracle runs the recurrence of each (b, h) over
exactly those rows, from the same initial state.  Checked: the output rows below each length (row-wise max
relative error, 1e-4 for fp32 inputs and 2e-2 for bf16 inputs), that the rows from each length on are left as
they were, and the final state of every sequence (a length of 0 leaves the caller's state bit for bit).
"""
import numpy as np
import pytest

import oracle
import sanatan_inputs as si
from parity_log import record

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
SENTINEL = 7.0


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


def row_rel_err(got, want):
    got = np.asarray(got, np.float64).reshape(-1, want.shape[-1])
    want = np.asarray(want, np.float64).reshape(-1, want.shape[-1])
    if want.shape[0] == 0:
        return 0.0
    return float((np.abs(got - want).max(1) / np.maximum(np.abs(want).max(1), 1e-12)).max())


def run_ragged(torch, seed, dtype, chunk, B, H, T, lengths, pos0=0, with_state=False):
    """One ragged call; returns the worst output row error and the worst state error over all sequences."""
    import root_parity_gated_amd as rpg

    q, k, v, om = si.attention_inputs(seed, B, H, T + 24, dtype)
    S0 = z0 = None
    if with_state:
        # the caller's state: the recurrence over 24 earlier tokens (positions pos0 - 24 .. pos0 - 1)
        hist = slice(T, T + 24)
        _, S0, z0 = oracle.recurrent_heads(q[:, :, hist].reshape(B * H, 24, -1), k[:, :, hist].reshape(B * H, 24, -1),
                                           v[:, :, hist].reshape(B * H, 24, -1), np.tile(om, (B, 1)),
                                           pos0=pos0 - 24)
        S0 = S0.reshape(B, H, 384, 64).astype(np.float32)
        z0 = z0.reshape(B, H, 384).astype(np.float32)
    q, k, v = q[:, :, :T], k[:, :, :T], v[:, :, :T]
    prm = rpg.Params(omega=torch.from_numpy(np.ascontiguousarray(om, dtype=np.float32)).cuda())
    lens = torch.tensor(np.asarray(lengths, dtype=np.int32), device="cuda")
    out = torch.full((B, H, T, 64), SENTINEL, device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
    Sg = torch.from_numpy(S0).cuda() if with_state else None
    zg = torch.from_numpy(z0).cuda() if with_state else None
    # a workspace full of NaNs: a slot read before it is written shows up in the outputs
    ws = torch.full((rpg.sanatan_prefill_workspace_bytes(B, H, T, chunk, prm),), 0xFF, dtype=torch.uint8,
                    device="cuda")
    rpg.sanatan_prefill_chunked_ragged(dev(torch, q, dtype), dev(torch, k, dtype), dev(torch, v, dtype), lens, chunk,
                                       prm, pos0=pos0, S=Sg, z=zg, out=out, ws=ws)
    torch.cuda.synchronize()
    got = host(out)
    Sgot = host(Sg) if with_state else None
    zgot = host(zg) if with_state else None
    err = serr = 0.0
    for b in range(B):
        L = min(max(int(lengths[b]), 0), T)
        assert np.all(got[b, :, L:] == SENTINEL), f"rows from the length on were written (b={b}, L={L})"
        for h in range(H):
            want, Sw, zw = oracle.recurrent(q[b, h, :L], k[b, h, :L], v[b, h, :L], om[h], pos0=pos0,
                                            S=None if S0 is None else S0[b, h], z=None if z0 is None else z0[b, h])
            err = max(err, row_rel_err(got[b, h, :L], want))
            if with_state:
                if L == 0:
                    assert np.array_equal(Sgot[b, h], S0[b, h]) and np.array_equal(zgot[b, h], z0[b, h])
                else:
                    serr = max(serr, np.abs(Sgot[b, h] - Sw).max() / np.abs(Sw).max(),
                               np.abs(zgot[b, h] - zw).max() / np.abs(zw).max())
    return err, serr


@pytest.mark.parametrize("dtype,chunk", [("f32", 16), ("f32", 32), ("f32", 64), ("bf16", 16), ("bf16", 32),
                                         ("bf16", 64), ("bf16", 128)])
def test_ragged_small(torch_dev, dtype, chunk):
    """Lengths of 0, 1, a chunk's edges and the full T in one batch; a caller state and a position offset."""
    T = 300
    lengths = [T, 0, 1, chunk - 1, chunk, chunk + 1, 199, 2 * chunk + 5]
    err, serr = run_ragged(torch_dev, 1300 + chunk, dtype, chunk, len(lengths), 2, T, lengths, pos0=57,
                           with_state=True)
    print(f"ragged {dtype} chunk {chunk}: output {err:.3e}, state {serr:.3e}")
    assert record(f"ragged prefill {dtype}: output", err, TOL[dtype]) <= TOL[dtype]
    assert record(f"ragged prefill {dtype}: state", serr, TOL[dtype]) <= TOL[dtype]


def test_ragged_no_state_and_clamped_lengths(torch_dev):
    """No caller state; lengths beyond T and below 0 are clamped to T and 0."""
    T = 130
    lengths = [T + 1000, -5, 64, 3]
    err, _ = run_ragged(torch_dev, 1310, "bf16", 64, len(lengths), 3, T, lengths)
    assert record("ragged prefill bf16: output", err, TOL["bf16"]) <= TOL["bf16"]


def test_ragged_all_empty(torch_dev):
    """Every length 0: nothing is written, the state stays as it was."""
    err, serr = run_ragged(torch_dev, 1320, "bf16", 64, 3, 2, 64, [0, 0, 0], with_state=True)
    assert err == 0.0 and serr == 0.0


def test_ragged_large_batch_with_state(torch_dev):
    """384 sequences (more than the compute units) of seeded lengths up to 512: ranges cross sequence
    boundaries and the head piece of one sequence can share a workgroup with the final piece of another."""
    rng = np.random.default_rng(1330)
    B, H, T = 32, 12, 512
    lengths = rng.integers(0, T + 1, B)
    lengths[:3] = [T, 0, 1]
    err, serr = run_ragged(torch_dev, 1331, "bf16", 64, B, H, T, lengths, pos0=1000, with_state=True)
    print(f"ragged large batch: output {err:.3e}, state {serr:.3e}")
    assert record("ragged prefill bf16: output", err, TOL["bf16"]) <= TOL["bf16"]
    assert record("ragged prefill bf16: state", serr, TOL["bf16"]) <= TOL["bf16"]


def test_ragged_equals_uniform_when_lengths_are_full(torch_dev):
    """All lengths T: the same outputs as the uniform call up to the pieces' rounding order."""
    import root_parity_gated_amd as rpg

    torch = torch_dev
    B, H, T = 4, 6, 1000
    q, k, v, om = si.attention_inputs(1340, B, H, T, "bf16")
    prm = rpg.Params(omega=torch.from_numpy(om).cuda())
    args = [dev(torch, x, "bf16") for x in (q, k, v)]
    lens = torch.full((B,), T, dtype=torch.int32, device="cuda")
    a = rpg.sanatan_prefill_chunked_ragged(*args, lens, 64, prm)
    b = rpg.sanatan_prefill_chunked(*args, 64, prm)
    torch.cuda.synchronize()
    assert row_rel_err(host(a), host(b)) <= TOL["bf16"]


def test_ragged_many_short_prompts(torch_dev):
    """256 prompts of seeded lengths 0..100 (many sequences per workgroup, many of them empty or one chunk long),
    fp32 with a caller state."""
    rng = np.random.default_rng(1350)
    B, H, T = 256, 2, 100
    lengths = rng.integers(0, T + 1, B)
    lengths[::17] = 0
    err, serr = run_ragged(torch_dev, 1351, "f32", 32, B, H, T, lengths, pos0=3, with_state=True)
    print(f"ragged many short prompts: output {err:.3e}, state {serr:.3e}")
    assert record("ragged prefill f32: output", err, TOL["f32"]) <= TOL["f32"]
    assert record("ragged prefill f32: state", serr, TOL["f32"]) <= TOL["f32"]
