"""C-ABI checks that need no GPU: the library loads, exports every function declared in
include/sanatan.h, and rejects bad arguments with the documented status codes before any launch.
Pointers passed here are never dereferenced on the host (validation fails first)."""
import ctypes
import json
import os
import re

import pytest

import root_parity_gated_amd as rpg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sanatan.h")
FAKE = ctypes.c_void_p(0x1000)  # non-null, never dereferenced by the validation paths exercised here
GOLD = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_values.json")))


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sanatan_\w+)\s*\(", src)))


def params(**kw):
    p = dict(d=64, d_v=64, gamma=4.0, c=256.0, eps=1e-6, lambda_base=10000.0, omega=0x2000, n_param_heads=1)
    p.update(kw)
    return rpg.sanatan_params(p["d"], p["d_v"], p["gamma"], p["c"], p["eps"], p["lambda_base"], p["omega"],
                              p["n_param_heads"])


@pytest.fixture(scope="module")
def L():
    return rpg.lib()


def test_every_declared_function_is_exported(L):
    names = declared_functions()
    assert set(names) == set(rpg.EXPORTED), names
    for n in names:
        assert hasattr(L, n), n


def test_state_bytes_matches_pages(L):
    assert L.sanatan_state_bytes(64, 64) == GOLD["state_bytes_per_head_d64"]["value"]
    assert 144 * L.sanatan_state_bytes(64, 64) == GOLD["state_bytes_12layers_12heads_d64"]["value"]
    assert L.sanatan_state_bytes(0, 64) == 0


def test_compact_state_bytes(L):
    """(5d+1)(d_v+1) floats: the d equal channel-0 rows of S and entries of z kept once."""
    assert L.sanatan_compact_state_bytes(64, 64) == 321 * 65 * 4
    assert L.sanatan_state_bytes(64, 64) - L.sanatan_compact_state_bytes(64, 64) == 63 * 65 * 4
    assert L.sanatan_compact_state_bytes(64, 0) == 0


def test_status_strings(L):
    for s in range(5):
        assert L.sanatan_status_string(s)
    assert b"unknown" in L.sanatan_status_string(99)


def _prefill(L, p, q=FAKE, t=rpg.SANATAN_BF16, B=1, H=1, T=128, chunk=64, S=None, z=None, ws=FAKE, ws_bytes=1 << 40):
    return L.sanatan_prefill_chunked(q, FAKE, FAKE, t, B, H, T, chunk, 0, ctypes.byref(p), S, z, FAKE, ws, ws_bytes,
                                     None)


def test_prefill_validation(L):
    p = params()
    assert _prefill(L, p, q=None) == rpg.SANATAN_ERR_INVALID_ARG
    assert _prefill(L, p, T=0) == rpg.SANATAN_ERR_INVALID_ARG
    assert _prefill(L, p, B=-1) == rpg.SANATAN_ERR_INVALID_ARG
    assert _prefill(L, p, chunk=0) == rpg.SANATAN_ERR_INVALID_ARG
    assert _prefill(L, p, t=7) == rpg.SANATAN_ERR_INVALID_ARG
    assert _prefill(L, p, S=FAKE, z=None) == rpg.SANATAN_ERR_INVALID_ARG
    assert _prefill(L, p, chunk=48) == rpg.SANATAN_ERR_UNSUPPORTED
    assert _prefill(L, p, chunk=24) == rpg.SANATAN_ERR_UNSUPPORTED
    assert _prefill(L, p, chunk=128, t=rpg.SANATAN_F32) == rpg.SANATAN_ERR_UNSUPPORTED
    assert _prefill(L, params(d=32)) == rpg.SANATAN_ERR_UNSUPPORTED
    assert _prefill(L, params(d_v=128)) == rpg.SANATAN_ERR_UNSUPPORTED
    assert _prefill(L, p, ws=None) == rpg.SANATAN_ERR_WORKSPACE
    assert _prefill(L, p, ws_bytes=16) == rpg.SANATAN_ERR_WORKSPACE


def test_ragged_prefill_validation(L):
    p = params()

    def rg(q=FAKE, lengths=FAKE, T=128, chunk=64, S=None, z=None, ws=FAKE, ws_bytes=1 << 40, pos0=0):
        return L.sanatan_prefill_chunked_ragged(q, FAKE, FAKE, rpg.SANATAN_BF16, 2, 1, T, chunk, lengths, pos0,
                                                ctypes.byref(p), S, z, FAKE, ws, ws_bytes, None)

    assert rg(lengths=None) == rpg.SANATAN_ERR_INVALID_ARG
    assert rg(q=None) == rpg.SANATAN_ERR_INVALID_ARG
    assert rg(T=0) == rpg.SANATAN_ERR_INVALID_ARG
    assert rg(S=FAKE) == rpg.SANATAN_ERR_INVALID_ARG
    assert rg(pos0=(1 << 53) - 10) == rpg.SANATAN_ERR_INVALID_ARG
    assert rg(chunk=48) == rpg.SANATAN_ERR_UNSUPPORTED
    assert rg(T=(1 << 22) + 1) == rpg.SANATAN_ERR_UNSUPPORTED
    assert rg(ws=None) == rpg.SANATAN_ERR_WORKSPACE
    assert rg(ws_bytes=16) == rpg.SANATAN_ERR_WORKSPACE


@pytest.mark.parametrize("bad", [dict(omega=0), dict(n_param_heads=0), dict(gamma=-1.0), dict(gamma=float("nan")),
                                 dict(c=0.0), dict(c=float("inf")), dict(eps=-1e-3), dict(lambda_base=0.0),
                                 dict(d=0)])
def test_param_validation(L, bad):
    assert _prefill(L, params(**bad)) == rpg.SANATAN_ERR_INVALID_ARG


def test_featurize_decode_quadratic_validation(L):
    p = params()
    assert L.sanatan_featurize(None, 0, 1, 1, 8, 0, ctypes.byref(p), FAKE, 0, None) == rpg.SANATAN_ERR_INVALID_ARG
    assert L.sanatan_featurize(FAKE, 0, 1, 1, 0, 0, ctypes.byref(p), FAKE, 0, None) == rpg.SANATAN_ERR_INVALID_ARG
    assert L.sanatan_featurize(FAKE, 0, 1, 1, 8, 0, ctypes.byref(params(d=16)), FAKE, 0,
                               None) == rpg.SANATAN_ERR_UNSUPPORTED
    assert L.sanatan_decode_step(FAKE, FAKE, FAKE, 0, 0, ctypes.byref(p), FAKE, FAKE, FAKE,
                                 None) == rpg.SANATAN_ERR_INVALID_ARG
    assert L.sanatan_decode_step(FAKE, FAKE, FAKE, 4, 0, ctypes.byref(p), None, FAKE, FAKE,
                                 None) == rpg.SANATAN_ERR_INVALID_ARG
    assert L.sanatan_decode_step(FAKE, FAKE, FAKE, 4, 0, None, FAKE, FAKE, FAKE, None) == rpg.SANATAN_ERR_INVALID_ARG
    dp = L.sanatan_decode_step_positions
    assert dp(FAKE, FAKE, FAKE, 4, None, ctypes.byref(p), FAKE, FAKE, FAKE, None) == rpg.SANATAN_ERR_INVALID_ARG
    assert dp(FAKE, FAKE, FAKE, 0, FAKE, ctypes.byref(p), FAKE, FAKE, FAKE, None) == rpg.SANATAN_ERR_INVALID_ARG
    assert dp(FAKE, FAKE, FAKE, 4, FAKE, ctypes.byref(p), FAKE, None, FAKE, None) == rpg.SANATAN_ERR_INVALID_ARG
    assert dp(FAKE, FAKE, FAKE, 4, FAKE, ctypes.byref(params(d=32)), FAKE, FAKE, FAKE,
              None) == rpg.SANATAN_ERR_UNSUPPORTED
    dc = L.sanatan_decode_step_compact
    assert dc(FAKE, FAKE, FAKE, 0, 0, None, ctypes.byref(p), FAKE, FAKE, FAKE, None) == rpg.SANATAN_ERR_INVALID_ARG
    assert dc(FAKE, FAKE, FAKE, 4, 0, None, ctypes.byref(p), None, FAKE, FAKE, None) == rpg.SANATAN_ERR_INVALID_ARG
    assert dc(FAKE, FAKE, FAKE, 4, 0, FAKE, None, FAKE, FAKE, FAKE, None) == rpg.SANATAN_ERR_INVALID_ARG
    assert dc(FAKE, FAKE, FAKE, 4, 0, None, ctypes.byref(params(d_v=32)), FAKE, FAKE, FAKE,
              None) == rpg.SANATAN_ERR_UNSUPPORTED
    d4 = L.sanatan_decode_step_four_channel
    assert d4(FAKE, FAKE, FAKE, 0, 0, None, ctypes.byref(p), FAKE, FAKE, FAKE, None) == rpg.SANATAN_ERR_INVALID_ARG
    assert d4(FAKE, FAKE, FAKE, 4, 0, None, ctypes.byref(p), FAKE, None, FAKE, None) == rpg.SANATAN_ERR_INVALID_ARG
    assert d4(FAKE, FAKE, FAKE, 4, 0, None, ctypes.byref(params(d=32)), FAKE, FAKE, FAKE,
              None) == rpg.SANATAN_ERR_UNSUPPORTED
    assert L.sanatan_four_channel_state_bytes(64, 64) == 193 * 65 * 4
    for conv in (L.sanatan_state_compact, L.sanatan_state_expand):
        assert conv(FAKE, FAKE, 0, FAKE, FAKE, None) == rpg.SANATAN_ERR_INVALID_ARG
        assert conv(FAKE, None, 3, FAKE, FAKE, None) == rpg.SANATAN_ERR_INVALID_ARG
        assert conv(FAKE, FAKE, 3, FAKE, None, None) == rpg.SANATAN_ERR_INVALID_ARG
    for pe in (0, 3):
        assert L.sanatan_quadratic_ref_p2(FAKE, FAKE, FAKE, 1, 1, 1, 64, pe, 0, ctypes.byref(p), FAKE, FAKE, 1 << 40,
                                          None) == rpg.SANATAN_ERR_INVALID_ARG
    assert L.sanatan_quadratic_ref_p2(FAKE, FAKE, FAKE, 1, 1, 1, 64, 2, 0, ctypes.byref(p), FAKE, FAKE, 10,
                                      None) == rpg.SANATAN_ERR_WORKSPACE
    for pe in (0, 3):
        assert L.sanatan_quadratic_four_channel(FAKE, FAKE, FAKE, 1, 1, 1, 64, pe, 0, ctypes.byref(p), FAKE, FAKE,
                                                1 << 40, None) == rpg.SANATAN_ERR_INVALID_ARG
    assert L.sanatan_quadratic_four_channel(FAKE, FAKE, FAKE, 1, 1, 1, 64, 1, 0, ctypes.byref(p), FAKE, FAKE, 10,
                                            None) == rpg.SANATAN_ERR_WORKSPACE
    assert L.sanatan_quadratic_four_channel(None, FAKE, FAKE, 1, 1, 1, 64, 1, 0, ctypes.byref(p), FAKE, FAKE,
                                            1 << 40, None) == rpg.SANATAN_ERR_INVALID_ARG
    # the training forward: the quadratic form's checks, and its saved-statistics output is required
    qt = lambda pe, sv, ws_bytes=1 << 40: L.sanatan_quadratic_train(FAKE, FAKE, FAKE, 1, 1, 1, 64, pe, 0,
                                                                    ctypes.byref(p), FAKE, sv, FAKE, ws_bytes, None)
    assert qt(2, None) == rpg.SANATAN_ERR_INVALID_ARG
    assert qt(3, FAKE) == rpg.SANATAN_ERR_INVALID_ARG
    assert qt(2, FAKE, ws_bytes=10) == rpg.SANATAN_ERR_WORKSPACE
    # saved statistics: the fp32 output row and 1 / Dn per query row
    assert L.sanatan_quadratic_saved_bytes(2, 3, 100, ctypes.byref(p)) == 2 * 3 * 100 * 65 * 4
    assert L.sanatan_quadratic_saved_bytes(2, 3, 0, ctypes.byref(p)) == 0


def test_backward_saved_validation(L):
    """The backward pass from saved statistics: the saved buffer is required, and the rest is checked as in
    sanatan_attention_backward."""
    p = params()
    def bs(saved=FAKE, pe=2, T=64, ws_bytes=1 << 40, dq=FAKE):
        return L.sanatan_attention_backward_saved(FAKE, FAKE, FAKE, FAKE, saved, 1, 1, 1, T, pe, 0, ctypes.byref(p),
                                                  dq, FAKE, FAKE, FAKE, FAKE, ws_bytes, None)
    assert bs(saved=None) == rpg.SANATAN_ERR_INVALID_ARG
    assert bs(dq=None) == rpg.SANATAN_ERR_INVALID_ARG
    assert bs(pe=3) == rpg.SANATAN_ERR_INVALID_ARG
    assert bs(T=0) == rpg.SANATAN_ERR_INVALID_ARG
    assert bs(T=(1 << 20) + 1) == rpg.SANATAN_ERR_UNSUPPORTED
    assert bs(ws_bytes=10) == rpg.SANATAN_ERR_WORKSPACE


def test_workspace_sizes(L):
    p = params()
    assert L.sanatan_prefill_workspace_bytes(0, 1, 64, 64, ctypes.byref(p)) == 0
    assert L.sanatan_prefill_workspace_bytes(1, 1, 64, 0, ctypes.byref(p)) == 0
    assert L.sanatan_quadratic_workspace_bytes(1, 1, 0, 1, ctypes.byref(p)) == 0
    # quadratic: phase table [T][64] fp32 (256-byte aligned), then Phi(K) in the element type, [B,H,T,384]
    assert L.sanatan_quadratic_workspace_bytes(4, 12, 4096, rpg.SANATAN_BF16, ctypes.byref(p)) == \
        4096 * 64 * 4 + 4 * 12 * 4096 * 384 * 2
    assert L.sanatan_quadratic_workspace_bytes(1, 1, 255, rpg.SANATAN_F32, ctypes.byref(p)) == \
        (255 * 64 * 4 + 255) // 256 * 256 + 255 * 384 * 4
    # prefill: phase table [T][64] fp32 (256-byte aligned) + one boundary state per (sequence + range - 1)
    ws = L.sanatan_prefill_workspace_bytes(8, 12, 2048, 64, ctypes.byref(p))
    state = L.sanatan_state_bytes(64, 64)
    rho = 2048 * 64 * 4
    G = (ws - rho) // state - 96 + 1
    assert (ws - rho) % state == 0 and 1 <= G <= 3072


def test_position_and_length_ranges(L):
    """Positions must satisfy |pos| < 2^53 (the exact fp64 reduction's range); the prefill takes T <= 2^22 and
    the quadratic form T <= 2^20 (buffer-descriptor byte ranges)."""
    p = params()
    big = 1 << 53
    pf = lambda pos0, T=128: L.sanatan_prefill_chunked(FAKE, FAKE, FAKE, 1, 1, 1, T, 64, pos0, ctypes.byref(p), None,
                                                       None, FAKE, FAKE, 1 << 40, None)
    assert pf(big) == rpg.SANATAN_ERR_INVALID_ARG
    assert pf(big - 127) == rpg.SANATAN_ERR_INVALID_ARG      # the last token reaches 2^53
    assert pf(-big) == rpg.SANATAN_ERR_INVALID_ARG
    assert pf(0, T=(1 << 22) + 1) == rpg.SANATAN_ERR_UNSUPPORTED
    assert L.sanatan_prefill_workspace_bytes(1, 1, (1 << 22) + 1, 64, ctypes.byref(p)) == 0
    assert L.sanatan_featurize(FAKE, 0, 1, 1, 8, big - 4, ctypes.byref(p), FAKE, 0, None) == \
        rpg.SANATAN_ERR_INVALID_ARG
    assert L.sanatan_decode_step(FAKE, FAKE, FAKE, 4, big, ctypes.byref(p), FAKE, FAKE, FAKE, None) == \
        rpg.SANATAN_ERR_INVALID_ARG
    assert L.sanatan_decode_step_compact(FAKE, FAKE, FAKE, 4, -big, None, ctypes.byref(p), FAKE, FAKE, FAKE,
                                         None) == rpg.SANATAN_ERR_INVALID_ARG
    q2 = lambda T, pos0=0: L.sanatan_quadratic_ref_p2(FAKE, FAKE, FAKE, 1, 1, 1, T, 2, pos0, ctypes.byref(p), FAKE,
                                                      FAKE, 1 << 62, None)
    assert q2((1 << 20) + 1) == rpg.SANATAN_ERR_UNSUPPORTED
    assert q2(64, pos0=big) == rpg.SANATAN_ERR_INVALID_ARG
    assert L.sanatan_quadratic_workspace_bytes(1, 1, (1 << 20) + 1, 1, ctypes.byref(p)) == 0


def test_partitioned_prefill_validation(L):
    """The partition test hook: a negative workgroup count is refused, and the workspace follows the count."""
    p = params()
    part = lambda wgs, ws_bytes=1 << 40: L.sanatan_prefill_chunked_partitioned(
        FAKE, FAKE, FAKE, 1, 1, 1, 128, 64, wgs, 0, ctypes.byref(p), None, None, FAKE, FAKE, ws_bytes, None)
    assert part(-1) == rpg.SANATAN_ERR_INVALID_ARG
    state = L.sanatan_state_bytes(64, 64)
    w1 = L.sanatan_prefill_workspace_bytes_partitioned(2, 3, 1000, 64, 1, ctypes.byref(p))
    w5 = L.sanatan_prefill_workspace_bytes_partitioned(2, 3, 1000, 64, 5, ctypes.byref(p))
    assert w5 - w1 == 4 * state
    assert part(2, ws_bytes=16) == rpg.SANATAN_ERR_WORKSPACE
    assert L.sanatan_prefill_workspace_bytes_partitioned(2, 3, 1000, 64, -2, ctypes.byref(p)) == 0
