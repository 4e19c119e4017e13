"""The no-allocation prefill entry point (library-held device workspace) against the allocating prefill.

sanatan_prefill_chunked_noalloc runs the same kernels with the same partition on a fixed device array, so
its outputs and final states must equal those of sanatan_prefill_chunked bit for bit.  Two calls in a row,
the second on a smaller input, check that nothing left in the array by the first call leaks into the second.
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


def _inputs(torch, seed, B, H, T, dtype):
    import root_parity_gated_amd as rpg

    q, k, v, om = si.attention_inputs(seed, B, H, T, dtype)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda().to(dt)
    p = rpg.Params(omega=torch.from_numpy(om).cuda())
    g = torch.Generator().manual_seed(seed)
    S0 = torch.randn((B, H, 384, 64), generator=g).cuda()
    z0 = torch.rand((B, H, 384), generator=g).cuda() * 50.0
    return dev(q), dev(k), dev(v), p, S0, z0


@pytest.mark.parametrize("dtype,chunk", [("bf16", 64), ("bf16", 128), ("f32", 32)])
def test_noalloc_matches_allocating_prefill(torch_dev, dtype, chunk):
    import root_parity_gated_amd as rpg

    torch = torch_dev
    # first a large call (many pieces per sequence, scan kernel, a caller state), then a smaller one
    for seed, B, H, T in ((700, 8, 12, 2048 + 37), (701, 1, 3, 200)):
        q, k, v, p, S0, z0 = _inputs(torch, seed, B, H, T, dtype)
        S_a, z_a = S0.clone(), z0.clone()
        S_b, z_b = S0.clone(), z0.clone()
        out_a = rpg.sanatan_prefill_chunked(q, k, v, chunk, p, pos0=11, S=S_a, z=z_a)
        out_b = torch.empty_like(out_a)
        rpg.sanatan_prefill_chunked_noalloc(q, k, v, chunk, p, pos0=11, S=S_b, z=z_b, out=out_b)
        # and without a state
        out_c = rpg.sanatan_prefill_chunked(q, k, v, chunk, p, pos0=11)
        out_d = rpg.sanatan_prefill_chunked_noalloc(q, k, v, chunk, p, pos0=11)
        torch.cuda.synchronize()
        print(f"noalloc B{B} H{H} T{T} {dtype} chunk {chunk}: "
              f"max |diff| {float((out_a.float() - out_b.float()).abs().max()):.3e}")
        assert torch.equal(out_a, out_b)
        assert torch.equal(S_a, S_b) and torch.equal(z_a, z_b)
        assert torch.equal(out_c, out_d)


def test_noalloc_rejects_oversized_workspace(torch_dev):
    """More sequences than the fixed array can hold boundary states for: a clear WORKSPACE status."""
    import root_parity_gated_amd as rpg

    torch = torch_dev
    B, H, T = 40, 12, 2048
    p = rpg.Params(omega=torch.zeros((H, 64), device="cuda"))
    assert rpg.sanatan_prefill_workspace_bytes(B, H, T, 64, p) > 48 << 20
    x = torch.zeros((B, H, T, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(rpg.SanatanError) as e:
        rpg.sanatan_prefill_chunked_noalloc(x, x, x, 64, p)
    assert e.value.status == rpg.SANATAN_ERR_WORKSPACE
