"""The Python binding refuses tensors whose shapes or element types do not match before anything reaches the
library: the C ABI takes bare pointers and cannot see a short buffer, so these checks are what keeps a wrong
shape from turning into an out-of-bounds access.  Nothing is launched by any call here."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import root_parity_gated_amd as rpg

    rpg.lib()
    return torch, rpg, rpg.Params(omega=torch.zeros((2, 64), device="cuda"))


def z(torch, *shape, dtype=None):
    return torch.zeros(shape, device="cuda", dtype=dtype or torch.float32)


def test_prefill_and_quadratic_shapes(env):
    torch, rpg, p = env
    q, k, v = z(torch, 1, 2, 16, 64), z(torch, 1, 2, 16, 64), z(torch, 1, 2, 16, 64)
    with pytest.raises(ValueError):
        rpg.sanatan_prefill_chunked(q, z(torch, 1, 2, 15, 64), v, 16, p)
    with pytest.raises(ValueError):
        rpg.sanatan_prefill_chunked(q, k, z(torch, 1, 2, 16, 32), 16, p)
    with pytest.raises(ValueError):
        rpg.sanatan_prefill_chunked(q, k, v.to(torch.bfloat16), 16, p)
    with pytest.raises(ValueError):
        rpg.sanatan_prefill_chunked(q, k, v, 16, p, S=z(torch, 1, 2, 383, 64), z=z(torch, 1, 2, 384))
    with pytest.raises(ValueError):
        rpg.sanatan_prefill_chunked(q, k, v, 16, p, out=z(torch, 1, 2, 16, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        rpg.sanatan_quadratic_ref_p2(q, k, z(torch, 1, 1, 16, 64), 2, p)
    with pytest.raises(ValueError):
        rpg.sanatan_featurize(z(torch, 1, 2, 16, 32), 0, p)
    with pytest.raises(ValueError):
        rpg.sanatan_prefill_chunked(q, k, v, 16, rpg.Params(omega=z(torch, 2, 32)))


def test_decode_shapes(env):
    torch, rpg, p = env
    N = 3
    q, k, v = z(torch, N, 64), z(torch, N, 64), z(torch, N, 64)
    S, zz = z(torch, N, 384, 64), z(torch, N, 384)
    with pytest.raises(ValueError):
        rpg.sanatan_decode_step(q, k, v, 0, p, z(torch, N - 1, 384, 64), zz)
    with pytest.raises(ValueError):
        rpg.sanatan_decode_step(q, z(torch, N + 1, 64), v, 0, p, S, zz)
    with pytest.raises(ValueError):
        rpg.sanatan_decode_step(q, k, v, 0, p, S, zz, out=z(torch, N, 32))
    with pytest.raises(ValueError):
        rpg.sanatan_decode_step_positions(q, k, v, z(torch, N + 1, dtype=torch.int64), p, S, zz)
    with pytest.raises(ValueError):
        rpg.sanatan_decode_step_compact(q, k, v, 0, p, S, zz)  # full-size state where the compact one belongs
    with pytest.raises(ValueError):
        rpg.sanatan_state_compact(S, z(torch, N, 383))
    with pytest.raises(ValueError):
        rpg.sanatan_state_expand(z(torch, N, 321, 64), z(torch, N, 321), S=z(torch, N, 321, 64))
