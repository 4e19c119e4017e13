"""The backward pass at the benchmark's full sizes and launch configuration, against the oracle's fp64 gradient
on sampled sequences.

The GPU computes dq, dk, dv and domega for every sequence of the headline prefill shape (p = 1: B=8, H=12,
T=2048, bf16) and of the quadratic-form shape (p = 2: B=4, H=12, T=4096, bf16), exactly as bench.py times it
(one omega row per head).  The oracle's direct-form gradient of two whole sequences per shape, (0, 0) and
(B - 1, H - 1), is compared row by row with the metric of test_gpu_backward (per token row max |error| / max
|reference|, each row's scale floored at 1 % of the largest row's).  domega sums over the B sequences of a head,
which the oracle cannot afford at these sizes; it is compared at smaller sizes in test_gpu_backward.  Bar: 2e-2
(bf16 inputs).
"""
import numpy as np
import pytest

import oracle
import sanatan_inputs as si
from parity_log import record

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module")
def torch_dev():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import root_parity_gated_amd as rpg

    rpg.lib()
    return torch


def row_rel_err(got, want, floor=1e-2):
    got = np.asarray(got, np.float64).reshape(-1, want.shape[-1])
    want = np.asarray(want, np.float64).reshape(-1, want.shape[-1])
    scale = np.abs(want).max(1)
    scale = np.maximum(scale, floor * scale.max())
    return float((np.abs(got - want).max(1) / scale).max())


@pytest.mark.parametrize("shape,p", [("prefill", 1), ("quadratic", 2)])
def test_backward_full_size_two_sequences(torch_dev, shape, p):
    import root_parity_gated_amd as rpg

    torch = torch_dev
    w = si.PREFILL if shape == "prefill" else si.QUAD_P2
    q, k, v, om = si.workload_inputs(w)
    g = si.bf16_round(np.random.default_rng(w.seed + 31).standard_normal(v.shape).astype(np.float32))
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda().to(torch.bfloat16)
    prm = rpg.Params(omega=torch.from_numpy(om).cuda(), gamma=w.gamma, eps=w.eps, lambda_base=w.lambda_base)
    dq, dk, dv, dom = rpg.sanatan_attention_backward(dev(q), dev(k), dev(v), dev(g), p, prm)
    torch.cuda.synchronize()
    host = lambda t: t.float().cpu().numpy().astype(np.float64)
    dq, dk, dv, dom = host(dq), host(dk), host(dv), host(dom)
    errs = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    for b, h in ((0, 0), (w.B - 1, w.H - 1)):
        wq, wk, wv, _ = oracle.attention_direct_grad(q[b, h], k[b, h], v[b, h], g[b, h], om[h], p=p, gamma=w.gamma,
                                                     eps=w.eps, lambda_base=w.lambda_base)
        errs["dq"] = max(errs["dq"], row_rel_err(dq[b, h], wq))
        errs["dk"] = max(errs["dk"], row_rel_err(dk[b, h], wk))
        errs["dv"] = max(errs["dv"], row_rel_err(dv[b, h], wv))
    print(f"backward full size {w.name} p={p}: " + ", ".join(f"{n} {e:.3e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert record(f"backward {w.name} p={p} (two whole sequences): {n}", e, TOL) <= TOL, (n, e)
