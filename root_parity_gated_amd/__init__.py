"""Thin ctypes binding of libsanatan.so -- SANATAN root-parity gated attention on MI355X (gfx950).

Every function here has the name of the C entry point it wraps and only marshals arguments:
checks that tensors are contiguous CUDA/HIP tensors of the expected dtype, allocates outputs and
workspaces with torch when the caller passes none, and forwards raw pointers plus the current
stream.  All arithmetic runs in the library's kernels.  If the library has not been built this
module raises instead of falling back to anything else.

Build the library with ``python -m root_parity_gated_amd.build``.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsanatan.so")

SANATAN_OK, SANATAN_ERR_INVALID_ARG, SANATAN_ERR_UNSUPPORTED, SANATAN_ERR_WORKSPACE, SANATAN_ERR_HIP = range(5)
SANATAN_F32, SANATAN_BF16 = 0, 1
D = 64
DV = 64


class SanatanError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {sanatan_status_string(status)} (status {status})")


class sanatan_params(ctypes.Structure):
    _fields_ = [
        ("d", ctypes.c_int),
        ("d_v", ctypes.c_int),
        ("gamma", ctypes.c_float),
        ("c", ctypes.c_float),
        ("eps", ctypes.c_float),
        ("lambda_base", ctypes.c_double),
        ("omega", ctypes.c_void_p),
        ("n_param_heads", ctypes.c_int),
    ]


_lib = None


def lib():
    """The loaded library (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m root_parity_gated_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        pp = ctypes.POINTER(sanatan_params)
        L.sanatan_state_bytes.restype = sz
        L.sanatan_state_bytes.argtypes = [i32, i32]
        L.sanatan_status_string.restype = ctypes.c_char_p
        L.sanatan_status_string.argtypes = [i32]
        L.sanatan_featurize.restype = i32
        L.sanatan_featurize.argtypes = [vp, i32, i32, i32, i32, i64, pp, vp, i32, vp]
        L.sanatan_prefill_workspace_bytes.restype = sz
        L.sanatan_prefill_workspace_bytes.argtypes = [i32, i32, i32, i32, pp]
        L.sanatan_prefill_chunked.restype = i32
        L.sanatan_prefill_chunked.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i64, pp, vp, vp, vp, vp, sz, vp]
        L.sanatan_prefill_workspace_bytes_partitioned.restype = sz
        L.sanatan_prefill_workspace_bytes_partitioned.argtypes = [i32, i32, i32, i32, i32, pp]
        L.sanatan_prefill_chunked_partitioned.restype = i32
        L.sanatan_prefill_chunked_partitioned.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i64, pp, vp, vp,
                                                          vp, vp, sz, vp]
        L.sanatan_prefill_chunked_ragged.restype = i32
        L.sanatan_prefill_chunked_ragged.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, vp, i64, pp, vp, vp, vp,
                                                     vp, sz, vp]
        L.sanatan_prefill_chunked_noalloc.restype = i32
        L.sanatan_prefill_chunked_noalloc.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i64, pp, vp, vp, vp, vp]
        L.sanatan_decode_step.restype = i32
        L.sanatan_decode_step.argtypes = [vp, vp, vp, i32, i64, pp, vp, vp, vp, vp]
        L.sanatan_decode_step_positions.restype = i32
        L.sanatan_decode_step_positions.argtypes = [vp, vp, vp, i32, vp, pp, vp, vp, vp, vp]
        L.sanatan_compact_state_bytes.restype = sz
        L.sanatan_compact_state_bytes.argtypes = [i32, i32]
        L.sanatan_state_compact.restype = i32
        L.sanatan_state_compact.argtypes = [vp, vp, i32, vp, vp, vp]
        L.sanatan_state_expand.restype = i32
        L.sanatan_state_expand.argtypes = [vp, vp, i32, vp, vp, vp]
        L.sanatan_decode_step_compact.restype = i32
        L.sanatan_decode_step_compact.argtypes = [vp, vp, vp, i32, i64, vp, pp, vp, vp, vp, vp]
        L.sanatan_four_channel_state_bytes.restype = sz
        L.sanatan_four_channel_state_bytes.argtypes = [i32, i32]
        L.sanatan_decode_step_four_channel.restype = i32
        L.sanatan_decode_step_four_channel.argtypes = L.sanatan_decode_step_compact.argtypes
        L.sanatan_quadratic_workspace_bytes.restype = sz
        L.sanatan_quadratic_workspace_bytes.argtypes = [i32, i32, i32, i32, pp]
        L.sanatan_quadratic_ref_p2.restype = i32
        L.sanatan_quadratic_ref_p2.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i64, pp, vp, vp, sz, vp]
        L.sanatan_harmonics_state_bytes.restype = sz
        L.sanatan_harmonics_state_bytes.argtypes = [i32, i32, i32]
        L.sanatan_prefill_harmonics_workspace_bytes.restype = sz
        L.sanatan_prefill_harmonics_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, pp]
        L.sanatan_prefill_harmonics.restype = i32
        L.sanatan_prefill_harmonics.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i64, pp, vp, vp, vp, vp, sz, vp]
        L.sanatan_decode_step_harmonics.restype = i32
        L.sanatan_decode_step_harmonics.argtypes = [vp, vp, vp, i32, i64, vp, i32, pp, vp, vp, vp, vp]
        L.sanatan_prefill_four_channel_workspace_bytes.restype = sz
        L.sanatan_prefill_four_channel_workspace_bytes.argtypes = [i32, i32, i32, i32, pp]
        L.sanatan_prefill_four_channel.restype = i32
        L.sanatan_prefill_four_channel.argtypes = [vp, vp, vp, i32, i32, i32, i32, i64, pp, vp, vp, vp, vp, sz, vp]
        L.sanatan_attention_backward_workspace_bytes.restype = sz
        L.sanatan_attention_backward_workspace_bytes.argtypes = [i32, i32, i32, i32, pp]
        L.sanatan_attention_backward.restype = i32
        L.sanatan_attention_backward.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i64, pp, vp, vp, vp, vp, vp,
                                                 sz, vp]
        L.sanatan_quadratic_four_channel.restype = i32
        L.sanatan_quadratic_four_channel.argtypes = L.sanatan_quadratic_ref_p2.argtypes
        L.sanatan_quadratic_saved_bytes.restype = sz
        L.sanatan_quadratic_saved_bytes.argtypes = [i32, i32, i32, pp]
        L.sanatan_quadratic_train.restype = i32
        L.sanatan_quadratic_train.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i64, pp, vp, vp, vp, sz, vp]
        L.sanatan_attention_backward_saved.restype = i32
        L.sanatan_attention_backward_saved.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i64, pp, vp, vp,
                                                       vp, vp, vp, sz, vp]
        _lib = L
    return _lib


EXPORTED = [
    "sanatan_state_bytes", "sanatan_status_string", "sanatan_featurize", "sanatan_prefill_workspace_bytes",
    "sanatan_prefill_chunked", "sanatan_prefill_workspace_bytes_partitioned", "sanatan_prefill_chunked_partitioned",
    "sanatan_prefill_chunked_noalloc", "sanatan_prefill_chunked_ragged", "sanatan_decode_step", "sanatan_decode_step_positions",
    "sanatan_compact_state_bytes", "sanatan_state_compact", "sanatan_state_expand", "sanatan_decode_step_compact",
    "sanatan_four_channel_state_bytes", "sanatan_decode_step_four_channel",
    "sanatan_quadratic_workspace_bytes",
    "sanatan_quadratic_ref_p2", "sanatan_quadratic_four_channel", "sanatan_quadratic_saved_bytes",
    "sanatan_quadratic_train",
    "sanatan_attention_backward_workspace_bytes", "sanatan_attention_backward", "sanatan_attention_backward_saved",
    "sanatan_harmonics_state_bytes", "sanatan_prefill_harmonics_workspace_bytes", "sanatan_prefill_harmonics",
    "sanatan_decode_step_harmonics", "sanatan_prefill_four_channel_workspace_bytes", "sanatan_prefill_four_channel",
]


@dataclass
class Params:
    """Method parameters; `omega` is a device fp32 tensor [n_param_heads, d]."""
    omega: object
    gamma: float = 4.0
    c: float | None = None
    eps: float = 1e-6
    lambda_base: float = 10000.0
    d: int = D
    d_v: int = DV

    def struct(self) -> sanatan_params:
        om = self.omega
        if om is None:
            ptr, nph = None, 1
        else:
            _check_tensor(om, "omega", dtypes=("float32",))
            if om.dim() not in (1, 2) or om.shape[-1] != self.d:
                raise ValueError(f"omega must be [n_param_heads, {self.d}] (got {tuple(om.shape)})")
            ptr, nph = om.data_ptr(), int(om.shape[0]) if om.dim() == 2 else 1
        c = float(4 * self.d) if self.c is None else float(self.c)
        return sanatan_params(int(self.d), int(self.d_v), float(self.gamma), c, float(self.eps),
                              float(self.lambda_base), ptr, nph)


def sanatan_status_string(status: int) -> str:
    return lib().sanatan_status_string(int(status)).decode()


def sanatan_state_bytes(d: int = D, d_v: int = DV) -> int:
    return int(lib().sanatan_state_bytes(int(d), int(d_v)))


def _check(status: int, where: str):
    if status != SANATAN_OK:
        raise SanatanError(status, where)


def _check_tensor(t, name, dtypes=("float32", "bfloat16")):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if str(t.dtype).replace("torch.", "") not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")


def _check_shape(t, name, shape):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_same_dtype(ref, *named):
    for name, t in named:
        if t.dtype != ref.dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, expected {ref.dtype} (as q)")


def _dtype_code(t) -> int:
    import torch

    return SANATAN_BF16 if t.dtype == torch.bfloat16 else SANATAN_F32


def _stream():
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def sanatan_featurize(u, pos0: int, params: Params, out_dtype=None, out=None):
    """Phi of u [B,H,T,64] at positions pos0.. -> [B,H,T,384] (channel-major feature rows)."""
    import torch

    _check_tensor(u, "u")
    if u.dim() != 4:
        raise ValueError(f"u must be [B,H,T,d] (got {tuple(u.shape)})")
    B, H, T, d = u.shape
    _check_shape(u, "u", (B, H, T, params.d))
    out_dtype = u.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, H, T, 6 * d), dtype=out_dtype, device=u.device)
    _check_tensor(out, "phi")
    _check_shape(out, "phi", (B, H, T, 6 * d))
    p = params.struct()
    _check(lib().sanatan_featurize(_ptr(u), _dtype_code(u), B, H, T, int(pos0), ctypes.byref(p), _ptr(out),
                                   _dtype_code(out), _stream()), "sanatan_featurize")
    return out


def _attention_shape(q, k, v, params):
    """q, k [B,H,T,d] and v [B,H,T,d_v] (d, d_v of params) of one element type -> (B, H, T)."""
    if q.dim() != 4:
        raise ValueError(f"q must be [B,H,T,d] (got {tuple(q.shape)})")
    B, H, T = q.shape[:3]
    _check_shape(q, "q", (B, H, T, params.d))
    _check_shape(k, "k", (B, H, T, params.d))
    _check_shape(v, "v", (B, H, T, params.d_v))
    _check_same_dtype(q, ("k", k), ("v", v))
    return B, H, T


def _decode_shapes(q, k, v, S, z, rows, params):
    """q, k [N,d], v [N,d_v], S [N,rows,d_v], z [N,rows] (d, d_v of params) -> N."""
    if q.dim() != 2:
        raise ValueError(f"q must be [N,d] (got {tuple(q.shape)})")
    N = q.shape[0]
    _check_shape(q, "q", (N, params.d))
    _check_shape(k, "k", (N, params.d))
    _check_shape(v, "v", (N, params.d_v))
    _check_shape(S, "S", (N, rows, params.d_v))
    _check_shape(z, "z", (N, rows))
    return N


def sanatan_prefill_workspace_bytes(B: int, H: int, T: int, chunk: int, params: Params | None = None) -> int:
    p = params.struct() if params is not None else None
    return int(lib().sanatan_prefill_workspace_bytes(B, H, T, chunk, ctypes.byref(p) if p is not None else None))


def sanatan_prefill_workspace_bytes_partitioned(B: int, H: int, T: int, chunk: int, workgroups: int,
                                                params: Params | None = None) -> int:
    p = params.struct() if params is not None else None
    return int(lib().sanatan_prefill_workspace_bytes_partitioned(B, H, T, chunk, int(workgroups),
                                                                  ctypes.byref(p) if p is not None else None))


def sanatan_prefill_chunked(q, k, v, chunk: int, params: Params, pos0: int = 0, S=None, z=None, out=None, ws=None):
    """Chunked causal p=1 attention; S, z (fp32, in/out) optional.  Returns out [B,H,T,64]."""
    return sanatan_prefill_chunked_partitioned(q, k, v, chunk, 0, params, pos0=pos0, S=S, z=z, out=out, ws=ws,
                                               _entry="sanatan_prefill_chunked")


def sanatan_prefill_chunked_partitioned(q, k, v, chunk: int, workgroups: int, params: Params, pos0: int = 0, S=None,
                                        z=None, out=None, ws=None, _entry="sanatan_prefill_chunked_partitioned"):
    """Test hook: the prefill with the chunk list split over `workgroups` workgroups (0 = one per CU)."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(t, name)
    B, H, T = _attention_shape(q, k, v, params)
    d, dv = params.d, params.d_v
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    _check_tensor(out, "out")
    _check_shape(out, "out", (B, H, T, dv))
    _check_same_dtype(q, ("out", out))
    for name, t, shape in (("S", S, (B, H, 6 * d, dv)), ("z", z, (B, H, 6 * d))):
        if t is not None:
            _check_tensor(t, name, dtypes=("float32",))
            _check_shape(t, name, shape)
    p = params.struct()
    need = int(lib().sanatan_prefill_workspace_bytes_partitioned(B, H, T, chunk, int(workgroups), ctypes.byref(p)))
    if ws is None:
        ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=q.device)
    if _entry == "sanatan_prefill_chunked":
        st = lib().sanatan_prefill_chunked(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, H, T, int(chunk), int(pos0),
                                           ctypes.byref(p), _ptr(S), _ptr(z), _ptr(out), _ptr(ws), ws.numel(),
                                           _stream())
    else:
        st = lib().sanatan_prefill_chunked_partitioned(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, H, T,
                                                       int(chunk), int(workgroups), int(pos0), ctypes.byref(p),
                                                       _ptr(S), _ptr(z), _ptr(out), _ptr(ws), ws.numel(), _stream())
    _check(st, _entry)
    return out


def sanatan_prefill_chunked_ragged(q, k, v, lengths, chunk: int, params: Params, pos0: int = 0, S=None, z=None,
                                   out=None, ws=None):
    """One prefill call over sequences of different lengths: batch element b uses its first lengths[b] rows
    (lengths: int32 device tensor [B], clamped to [0, T] by the kernels).  Output rows from lengths[b] on are
    left as they are (zeros when `out` is allocated here); S, z (fp32, in/out) end at each element's length."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(t, name)
    B, H, T = _attention_shape(q, k, v, params)
    d, dv = params.d, params.d_v
    _check_tensor(lengths, "lengths", dtypes=("int32",))
    _check_shape(lengths, "lengths", (B,))
    if out is None:
        out = torch.zeros((B, H, T, dv), dtype=q.dtype, device=q.device)
    _check_tensor(out, "out")
    _check_shape(out, "out", (B, H, T, dv))
    _check_same_dtype(q, ("out", out))
    for name, t, shape in (("S", S, (B, H, 6 * d, dv)), ("z", z, (B, H, 6 * d))):
        if t is not None:
            _check_tensor(t, name, dtypes=("float32",))
            _check_shape(t, name, shape)
    p = params.struct()
    need = int(lib().sanatan_prefill_workspace_bytes(B, H, T, chunk, ctypes.byref(p)))
    if ws is None:
        ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=q.device)
    _check(lib().sanatan_prefill_chunked_ragged(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, H, T, int(chunk),
                                                _ptr(lengths), int(pos0), ctypes.byref(p), _ptr(S), _ptr(z),
                                                _ptr(out), _ptr(ws), ws.numel(), _stream()),
           "sanatan_prefill_chunked_ragged")
    return out


def sanatan_prefill_chunked_noalloc(q, k, v, chunk: int, params: Params, pos0: int = 0, S=None, z=None, out=None):
    """sanatan_prefill_chunked with the library's fixed device workspace (no workspace argument).  `out` is
    allocated here when not given; pass it to keep the call itself free of allocation."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(t, name)
    B, H, T = _attention_shape(q, k, v, params)
    d, dv = params.d, params.d_v
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    _check_tensor(out, "out")
    _check_shape(out, "out", (B, H, T, dv))
    _check_same_dtype(q, ("out", out))
    for name, t, shape in (("S", S, (B, H, 6 * d, dv)), ("z", z, (B, H, 6 * d))):
        if t is not None:
            _check_tensor(t, name, dtypes=("float32",))
            _check_shape(t, name, shape)
    p = params.struct()
    _check(lib().sanatan_prefill_chunked_noalloc(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, H, T, int(chunk),
                                                 int(pos0), ctypes.byref(p), _ptr(S), _ptr(z), _ptr(out), _stream()),
           "sanatan_prefill_chunked_noalloc")
    return out


def sanatan_decode_step(q, k, v, pos: int, params: Params, S, z, out=None):
    """One token for N head-states: q,k [N,64], v [N,64] fp32; S [N,384,64], z [N,384] in/out."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v), ("S", S), ("z", z)):
        _check_tensor(t, name, dtypes=("float32",))
    N = _decode_shapes(q, k, v, S, z, 6 * params.d, params)
    if out is None:
        out = torch.empty((N, v.shape[-1]), dtype=torch.float32, device=q.device)
    _check_tensor(out, "out", dtypes=("float32",))
    _check_shape(out, "out", (N, v.shape[-1]))
    p = params.struct()
    _check(lib().sanatan_decode_step(_ptr(q), _ptr(k), _ptr(v), N, int(pos), ctypes.byref(p), _ptr(S), _ptr(z),
                                     _ptr(out), _stream()), "sanatan_decode_step")
    return out


def sanatan_decode_step_positions(q, k, v, pos, params: Params, S, z, out=None):
    """As sanatan_decode_step, with pos a device int64 tensor [N]: one position per head-state."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v), ("S", S), ("z", z)):
        _check_tensor(t, name, dtypes=("float32",))
    _check_tensor(pos, "pos", dtypes=("int64",))
    N = _decode_shapes(q, k, v, S, z, 6 * params.d, params)
    if pos.numel() != N:
        raise ValueError(f"pos has {pos.numel()} entries for {N} head-states")
    if out is None:
        out = torch.empty((N, v.shape[-1]), dtype=torch.float32, device=q.device)
    _check_tensor(out, "out", dtypes=("float32",))
    _check_shape(out, "out", (N, v.shape[-1]))
    p = params.struct()
    _check(lib().sanatan_decode_step_positions(_ptr(q), _ptr(k), _ptr(v), N, _ptr(pos), ctypes.byref(p), _ptr(S),
                                               _ptr(z), _ptr(out), _stream()), "sanatan_decode_step_positions")
    return out


COMPACT_ROWS = 5 * 64 + 1  # compact state rows at d = 64: the d equal channel-0 rows kept once


def sanatan_compact_state_bytes(d: int = 64, d_v: int = 64) -> int:
    return int(lib().sanatan_compact_state_bytes(d, d_v))


def _state_lead(S, z, rows):
    """S [...,rows,64] and z [...,rows] with the same leading shape (at least one head-state) -> that shape."""
    if S.dim() < 3 or tuple(S.shape[-2:]) != (rows, 64):
        raise ValueError(f"state has shape {tuple(S.shape)}, expected [..., {rows}, 64]")
    lead = tuple(S.shape[:-2])
    _check_shape(z, "z", (*lead, rows))
    if math.prod(lead) == 0:
        raise ValueError("state holds no head-states")
    return lead


def sanatan_state_compact(S, z, Sc=None, zc=None):
    """Full state S [...,384,64], z [...,384] -> compact Sc [...,321,64], zc [...,321] (pure copies)."""
    import torch

    for name, t in (("S", S), ("z", z)):
        _check_tensor(t, name, dtypes=("float32",))
    lead = _state_lead(S, z, 6 * 64)
    N = math.prod(lead)
    if Sc is None:
        Sc = torch.empty((*lead, COMPACT_ROWS, 64), dtype=torch.float32, device=S.device)
    if zc is None:
        zc = torch.empty((*lead, COMPACT_ROWS), dtype=torch.float32, device=z.device)
    for name, t in (("Sc", Sc), ("zc", zc)):
        _check_tensor(t, name, dtypes=("float32",))
    _check_shape(Sc, "Sc", (*lead, COMPACT_ROWS, 64))
    _check_shape(zc, "zc", (*lead, COMPACT_ROWS))
    _check(lib().sanatan_state_compact(_ptr(S), _ptr(z), N, _ptr(Sc), _ptr(zc), _stream()), "sanatan_state_compact")
    return Sc, zc


def sanatan_state_expand(Sc, zc, S=None, z=None):
    """Compact Sc [...,321,64], zc [...,321] -> full S [...,384,64], z [...,384] (pure copies)."""
    import torch

    for name, t in (("Sc", Sc), ("zc", zc)):
        _check_tensor(t, name, dtypes=("float32",))
    lead = _state_lead(Sc, zc, COMPACT_ROWS)
    N = math.prod(lead)
    if S is None:
        S = torch.empty((*lead, 6 * 64, 64), dtype=torch.float32, device=Sc.device)
    if z is None:
        z = torch.empty((*lead, 6 * 64), dtype=torch.float32, device=zc.device)
    for name, t in (("S", S), ("z", z)):
        _check_tensor(t, name, dtypes=("float32",))
    _check_shape(S, "S", (*lead, 6 * 64, 64))
    _check_shape(z, "z", (*lead, 6 * 64))
    _check(lib().sanatan_state_expand(_ptr(Sc), _ptr(zc), N, _ptr(S), _ptr(z), _stream()), "sanatan_state_expand")
    return S, z


def sanatan_decode_step_compact(q, k, v, pos, params: Params, Sc, zc, out=None, _entry="sanatan_decode_step_compact"):
    """sanatan_decode_step on the compact state; pos is an int (every head-state) or a device int64 tensor [N]."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v), ("Sc", Sc), ("zc", zc)):
        _check_tensor(t, name, dtypes=("float32",))
    rows = 3 * params.d + 1 if _entry == "sanatan_decode_step_four_channel" else 5 * params.d + 1
    N = _decode_shapes(q, k, v, Sc, zc, rows, params)
    posv = None
    if isinstance(pos, torch.Tensor):
        _check_tensor(pos, "pos", dtypes=("int64",))
        if pos.numel() != N:
            raise ValueError(f"pos has {pos.numel()} entries for {N} head-states")
        posv, pos = pos, 0
    if out is None:
        out = torch.empty((N, v.shape[-1]), dtype=torch.float32, device=q.device)
    _check_tensor(out, "out", dtypes=("float32",))
    _check_shape(out, "out", (N, v.shape[-1]))
    p = params.struct()
    _check(getattr(lib(), _entry)(_ptr(q), _ptr(k), _ptr(v), N, int(pos), _ptr(posv) if posv is not None else None,
                                  ctypes.byref(p), _ptr(Sc), _ptr(zc), _ptr(out), _stream()), _entry)
    return out


FOUR_ROWS = 3 * 64 + 1  # four-channel state rows at d = 64: shared channel 0, then r, r cos, r sin


def sanatan_four_channel_state_bytes(d: int = 64, d_v: int = 64) -> int:
    return int(lib().sanatan_four_channel_state_bytes(d, d_v))


def sanatan_decode_step_four_channel(q, k, v, pos, params: Params, S4, z4, out=None):
    """One token on the unclipped four-channel kernel's state S4 [N,193,64], z4 [N,193]; pos an int or [N] int64."""
    return sanatan_decode_step_compact(q, k, v, pos, params, S4, z4, out=out,
                                       _entry="sanatan_decode_step_four_channel")


def sanatan_quadratic_workspace_bytes(B: int, H: int, T: int, dtype_code: int, params: Params | None = None) -> int:
    p = params.struct() if params is not None else None
    return int(lib().sanatan_quadratic_workspace_bytes(B, H, T, dtype_code, ctypes.byref(p) if p is not None else None))


def sanatan_quadratic_ref_p2(q, k, v, p_exp: int, params: Params, pos0: int = 0, out=None, ws=None,
                             four_channel: bool = False):
    """Masked quadratic normalised power attention (p = 1 or 2).  Returns out [B,H,T,64].  With four_channel,
    the unclipped four-channel kernel (sanatan_quadratic_four_channel) replaces the six-channel one."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(t, name)
    B, H, T = _attention_shape(q, k, v, params)
    if out is None:
        out = torch.empty((B, H, T, params.d_v), dtype=q.dtype, device=q.device)
    _check_tensor(out, "out")
    _check_shape(out, "out", (B, H, T, params.d_v))
    _check_same_dtype(q, ("out", out))
    p = params.struct()
    need = int(lib().sanatan_quadratic_workspace_bytes(B, H, T, _dtype_code(q), ctypes.byref(p)))
    if ws is None:
        ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=q.device)
    name = "sanatan_quadratic_four_channel" if four_channel else "sanatan_quadratic_ref_p2"
    _check(getattr(lib(), name)(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, H, T, int(p_exp), int(pos0),
                                ctypes.byref(p), _ptr(out), _ptr(ws), ws.numel(), _stream()), name)
    return out


def sanatan_quadratic_train(q, k, v, p_exp: int, params: Params, pos0: int = 0, out=None, saved=None, ws=None):
    """sanatan_quadratic_ref_p2 that also saves what sanatan_attention_backward_saved needs (fp32 output rows, then
    1 / Dn per row).  Returns (out [B,H,T,64] in the input dtype, saved: fp32 1-D tensor)."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(t, name)
    B, H, T = _attention_shape(q, k, v, params)
    if out is None:
        out = torch.empty((B, H, T, params.d_v), dtype=q.dtype, device=q.device)
    _check_tensor(out, "out")
    _check_shape(out, "out", (B, H, T, params.d_v))
    _check_same_dtype(q, ("out", out))
    p = params.struct()
    nsaved = int(lib().sanatan_quadratic_saved_bytes(B, H, T, ctypes.byref(p))) // 4
    if saved is None:
        saved = torch.empty((nsaved,), dtype=torch.float32, device=q.device)
    _check_tensor(saved, "saved", dtypes=("float32",))
    _check_shape(saved, "saved", (nsaved,))
    need = int(lib().sanatan_quadratic_workspace_bytes(B, H, T, _dtype_code(q), ctypes.byref(p)))
    if ws is None:
        ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=q.device)
    _check(lib().sanatan_quadratic_train(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, H, T, int(p_exp), int(pos0),
                                         ctypes.byref(p), _ptr(out), _ptr(saved), _ptr(ws), ws.numel(), _stream()),
           "sanatan_quadratic_train")
    return out, saved


def sanatan_quadratic_four_channel(q, k, v, p_exp: int, params: Params, pos0: int = 0, out=None, ws=None):
    """The masked quadratic form on the unclipped four-channel kernel.  Returns out [B,H,T,64]."""
    return sanatan_quadratic_ref_p2(q, k, v, p_exp, params, pos0=pos0, out=out, ws=ws, four_channel=True)


def sanatan_attention_backward_workspace_bytes(B: int, H: int, T: int, dtype_code: int,
                                               params: Params | None = None) -> int:
    p = params.struct() if params is not None else None
    return int(lib().sanatan_attention_backward_workspace_bytes(B, H, T, dtype_code,
                                                                ctypes.byref(p) if p is not None else None))


def sanatan_attention_backward(q, k, v, dout, p_exp: int, params: Params, pos0: int = 0, dq=None, dk=None, dv=None,
                               domega=None, ws=None):
    """Gradient of sum(dout * o) for the normalised causal power attention o (p = 1: the chunked prefill's
    output; p = 2: the quadratic form's).  Returns (dq, dk, dv [B,H,T,64] in the input dtype, domega fp32
    [n_param_heads, 64])."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _check_tensor(t, name)
    B, H, T = _attention_shape(q, k, v, params)
    _check_shape(dout, "dout", (B, H, T, params.d_v))
    _check_same_dtype(q, ("dout", dout))
    pr = params.struct()
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_tensor(t, name)
        _check_shape(t, name, tuple(ref.shape))
        _check_same_dtype(q, (name, t))
    nph = pr.n_param_heads
    if domega is None:
        domega = torch.empty((nph, params.d), dtype=torch.float32, device=q.device)
    _check_tensor(domega, "domega", dtypes=("float32",))
    _check_shape(domega, "domega", (nph, params.d))
    need = int(lib().sanatan_attention_backward_workspace_bytes(B, H, T, _dtype_code(q), ctypes.byref(pr)))
    if ws is None:
        ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=q.device)
    _check(lib().sanatan_attention_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _dtype_code(q), B, H, T, int(p_exp),
                                            int(pos0), ctypes.byref(pr), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(domega),
                                            _ptr(ws), ws.numel(), _stream()), "sanatan_attention_backward")
    return dq, dk, dv, domega


def sanatan_attention_backward_saved(q, k, v, dout, saved, p_exp: int, params: Params, pos0: int = 0,
                                     dq=None, dk=None, dv=None, domega=None, ws=None):
    """sanatan_attention_backward given the statistics sanatan_quadratic_train saved (same q, k, v, p, pos0,
    params).  Returns (dq, dk, dv, domega) as sanatan_attention_backward."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _check_tensor(t, name)
    B, H, T = _attention_shape(q, k, v, params)
    _check_shape(dout, "dout", (B, H, T, params.d_v))
    _check_same_dtype(q, ("dout", dout))
    pr = params.struct()
    _check_tensor(saved, "saved", dtypes=("float32",))
    _check_shape(saved, "saved", (int(lib().sanatan_quadratic_saved_bytes(B, H, T, ctypes.byref(pr))) // 4,))
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_tensor(t, name)
        _check_shape(t, name, tuple(ref.shape))
        _check_same_dtype(q, (name, t))
    nph = pr.n_param_heads
    if domega is None:
        domega = torch.empty((nph, params.d), dtype=torch.float32, device=q.device)
    _check_tensor(domega, "domega", dtypes=("float32",))
    _check_shape(domega, "domega", (nph, params.d))
    need = int(lib().sanatan_attention_backward_workspace_bytes(B, H, T, _dtype_code(q), ctypes.byref(pr)))
    if ws is None:
        ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=q.device)
    _check(lib().sanatan_attention_backward_saved(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(saved),
                                                  _dtype_code(q), B, H, T, int(p_exp), int(pos0), ctypes.byref(pr),
                                                  _ptr(dq), _ptr(dk), _ptr(dv), _ptr(domega), _ptr(ws), ws.numel(),
                                                  _stream()), "sanatan_attention_backward_saved")
    return dq, dk, dv, domega


def sanatan_harmonics_state_bytes(d: int = D, d_v: int = DV, nh: int = 2) -> int:
    return int(lib().sanatan_harmonics_state_bytes(int(d), int(d_v), int(nh)))


def sanatan_prefill_harmonics_workspace_bytes(B: int, H: int, T: int, dtype_code: int, nh: int,
                                              params: Params | None = None) -> int:
    p = params.struct() if params is not None else None
    return int(lib().sanatan_prefill_harmonics_workspace_bytes(B, H, T, dtype_code, int(nh),
                                                               ctypes.byref(p) if p is not None else None))


def sanatan_prefill_four_channel_workspace_bytes(B: int, H: int, T: int, dtype_code: int,
                                                 params: Params | None = None) -> int:
    p = params.struct() if params is not None else None
    return int(lib().sanatan_prefill_four_channel_workspace_bytes(B, H, T, dtype_code,
                                                                  ctypes.byref(p) if p is not None else None))


def _ext_prefill(entry, q, k, v, params: Params, pos0, S, z, out, ws, rows, ws_fn):
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(t, name)
    B, H, T = _attention_shape(q, k, v, params)
    if out is None:
        out = torch.empty((B, H, T, params.d_v), dtype=q.dtype, device=q.device)
    _check_tensor(out, "out")
    _check_shape(out, "out", (B, H, T, params.d_v))
    _check_same_dtype(q, ("out", out))
    for name, t, shape in (("S", S, (B, H, rows, params.d_v)), ("z", z, (B, H, rows))):
        if t is not None:
            _check_tensor(t, name, dtypes=("float32",))
            _check_shape(t, name, shape)
    p = params.struct()
    need = ws_fn(B, H, T, _dtype_code(q), p)
    if ws is None:
        ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=q.device)
    return B, H, T, p, out, ws


def sanatan_prefill_harmonics(q, k, v, nh: int, params: Params, pos0: int = 0, S=None, z=None, out=None, ws=None):
    """Chunked p = 1 prefill on the spectral-harmonic map with nh harmonics; S [B,H,(2+4nh)d,64], z optional."""
    rows = (2 + 4 * nh) * params.d
    ws_fn = lambda B, H, T, t, p: int(lib().sanatan_prefill_harmonics_workspace_bytes(B, H, T, t, int(nh),
                                                                                        ctypes.byref(p)))
    B, H, T, p, out, ws = _ext_prefill("harmonics", q, k, v, params, pos0, S, z, out, ws, rows, ws_fn)
    _check(lib().sanatan_prefill_harmonics(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, H, T, int(nh), int(pos0),
                                           ctypes.byref(p), _ptr(S), _ptr(z), _ptr(out), _ptr(ws), ws.numel(),
                                           _stream()), "sanatan_prefill_harmonics")
    return out


def sanatan_prefill_four_channel(q, k, v, params: Params, pos0: int = 0, S4=None, z4=None, out=None, ws=None):
    """Chunked p = 1 prefill on the unclipped four-channel kernel; S4 [B,H,3d+1,64], z4 [B,H,3d+1] optional."""
    rows = 3 * params.d + 1
    ws_fn = lambda B, H, T, t, p: int(lib().sanatan_prefill_four_channel_workspace_bytes(B, H, T, t, ctypes.byref(p)))
    B, H, T, p, out, ws = _ext_prefill("four", q, k, v, params, pos0, S4, z4, out, ws, rows, ws_fn)
    _check(lib().sanatan_prefill_four_channel(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, H, T, int(pos0),
                                              ctypes.byref(p), _ptr(S4), _ptr(z4), _ptr(out), _ptr(ws), ws.numel(),
                                              _stream()), "sanatan_prefill_four_channel")
    return out


def sanatan_decode_step_harmonics(q, k, v, pos, nh: int, params: Params, S, z, out=None):
    """One token of the spectral-harmonic recurrence for N head-states: S [N,(2+4nh)d,64], z [N,(2+4nh)d]."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v), ("S", S), ("z", z)):
        _check_tensor(t, name, dtypes=("float32",))
    rows = (2 + 4 * nh) * params.d
    N = _decode_shapes(q, k, v, S, z, rows, params)
    if out is None:
        out = torch.empty((N, params.d_v), dtype=torch.float32, device=q.device)
    _check_tensor(out, "out", dtypes=("float32",))
    _check_shape(out, "out", (N, params.d_v))
    p = params.struct()
    posv = None
    if isinstance(pos, torch.Tensor):
        _check_tensor(pos, "pos", dtypes=("int64",))
        _check_shape(pos, "pos", (N,))
        posv, pos = pos, 0
    _check(lib().sanatan_decode_step_harmonics(_ptr(q), _ptr(k), _ptr(v), N, int(pos), _ptr(posv), int(nh),
                                               ctypes.byref(p), _ptr(S), _ptr(z), _ptr(out), _stream()),
           "sanatan_decode_step_harmonics")
    return out
