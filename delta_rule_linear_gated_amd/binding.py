"""ctypes binding of ``libdn.so`` (declared in ``include/dn.h``).

Argument marshalling only: every step of the operator runs in the HIP kernels
behind the C ABI.  PyTorch supplies device memory and the stream.  When the
library is not built this module raises -- there is no fallback path.

Low level (same names as the C ABI): ``dn_states_bytes``, ``dn_states_layout``,
``dn_workspace_bytes``, ``dn_workspace_layout``, ``dn_chunk_fwd``, ``dn_chunk_bwd``,
``dn_status_string``, ``dn_last_error``.  Convenience: ``chunk_fwd`` / ``chunk_bwd`` allocate outputs
and workspace with torch and call the above; ``DeltaRule`` is a
``torch.autograd.Function`` over them.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdn.so")

DN_OK, DN_ERR_INVALID, DN_ERR_SHAPE, DN_ERR_DTYPE, DN_ERR_WORKSPACE, DN_ERR_UNSUPPORTED, DN_ERR_HIP = (
    0, -1, -2, -3, -4, -5, -6)
DN_F32, DN_BF16 = 0, 1
DN_GATE_NONE, DN_GATE_SCALAR, DN_GATE_VECTOR = 0, 1, 2
DN_PASS_FWD, DN_PASS_BWD, DN_PASS_BWD_RECOMPUTE = 0, 1, 2
DN_FLAG_KACZMARZ, DN_FLAG_NO_SCAN = 1, 2
DN_NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTS = ("dn_states_bytes", "dn_states_layout", "dn_workspace_bytes", "dn_workspace_layout", "dn_chunk_fwd",
           "dn_chunk_fwd_noalloc", "dn_chunk_bwd", "dn_recurrent_fwd", "dn_recurrent_phase_fwd", "dn_phase_states_bytes",
           "dn_phase_workspace_bytes", "dn_chunk_phase_fwd", "dn_chunk_phase_bwd", "dn_status_string", "dn_last_error",
           "dn_profile_enable", "dn_profile_collect")


class DnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("C", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("gate", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("eps", ctypes.c_float)]


_lib = None


def lib():
    """Open libdn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m delta_rule_linear_gated_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    sp = ctypes.POINTER(Shape)
    L.dn_states_bytes.argtypes = [sp]
    L.dn_states_bytes.restype = sz
    L.dn_workspace_bytes.argtypes = [sp, i32]
    L.dn_workspace_bytes.restype = sz
    L.dn_workspace_layout.argtypes = [sp, i32, ctypes.POINTER(ctypes.c_size_t)]
    L.dn_workspace_layout.restype = i32
    L.dn_states_layout.argtypes = [sp, ctypes.POINTER(ctypes.c_size_t)]
    L.dn_states_layout.restype = i32
    L.dn_recurrent_fwd.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.dn_recurrent_fwd.restype = i32
    L.dn_recurrent_phase_fwd.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.dn_recurrent_phase_fwd.restype = i32
    L.dn_chunk_fwd.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.dn_chunk_fwd.restype = i32
    L.dn_chunk_fwd_noalloc.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.dn_chunk_fwd_noalloc.restype = i32
    L.dn_chunk_bwd.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.dn_chunk_bwd.restype = i32
    L.dn_phase_states_bytes.argtypes = [sp]
    L.dn_phase_states_bytes.restype = sz
    L.dn_phase_workspace_bytes.argtypes = [sp, i32]
    L.dn_phase_workspace_bytes.restype = sz
    L.dn_chunk_phase_fwd.argtypes = [sp] + [vp] * 13 + [sz, vp]
    L.dn_chunk_phase_fwd.restype = i32
    L.dn_chunk_phase_bwd.argtypes = [sp] + [vp] * 21 + [sz, vp]
    L.dn_chunk_phase_bwd.restype = i32
    L.dn_status_string.argtypes = [i32]
    L.dn_status_string.restype = ctypes.c_char_p
    L.dn_last_error.argtypes = []
    L.dn_last_error.restype = ctypes.c_char_p
    L.dn_profile_enable.argtypes = [i32]
    L.dn_profile_enable.restype = i32
    L.dn_profile_collect.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_int), i32]
    L.dn_profile_collect.restype = i32
    _lib = L
    return L


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _check(status: int):
    if status != DN_OK:
        L = lib()
        raise DnError(status, f"{L.dn_status_string(status).decode()}: {L.dn_last_error().decode()}")


def make_shape(B, H, T, dk, dv, C, dtype, gate, kaczmarz_eps=None, no_scan=False) -> Shape:
    """``kaczmarz_eps`` not None sets DN_FLAG_KACZMARZ with that eps (beta then carries eta);
    ``no_scan`` sets DN_FLAG_NO_SCAN (one sequential state pass, never the chunk-parallel scan)."""
    dt = {torch.float32: DN_F32, torch.bfloat16: DN_BF16, "fp32": DN_F32, "bf16": DN_BF16}.get(dtype, dtype)
    gt = {None: DN_GATE_NONE, "none": DN_GATE_NONE, "scalar": DN_GATE_SCALAR,
          "vector": DN_GATE_VECTOR}.get(gate, gate)
    flags, eps = (0, 0.0) if kaczmarz_eps is None else (DN_FLAG_KACZMARZ, float(kaczmarz_eps))
    if no_scan:
        flags |= DN_FLAG_NO_SCAN
    return Shape(int(B), int(H), int(T), int(dk), int(dv), int(C), int(dt), int(gt), flags, eps)


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


# ------------------------------------------------------------------ C-ABI mirrors


def dn_states_bytes(shape: Shape) -> int:
    return lib().dn_states_bytes(ctypes.byref(shape))


def dn_states_layout(shape: Shape):
    out = (ctypes.c_size_t * 7)()
    _check(lib().dn_states_layout(ctypes.byref(shape), out))
    return dict(zip(("states", "T", "P", "U", "gam", "kz", "total"), list(out)))


def dn_workspace_bytes(shape: Shape, pass_: int) -> int:
    return lib().dn_workspace_bytes(ctypes.byref(shape), int(pass_))


def dn_workspace_layout(shape: Shape, pass_: int):
    out = (ctypes.c_size_t * 10)()
    _check(lib().dn_workspace_layout(ctypes.byref(shape), int(pass_), out))
    return dict(zip(("gam", "T", "P", "lam", "dS1", "states", "kz", "seg_end", "seg_start", "total"), list(out)))


def dn_status_string(status: int) -> str:
    return lib().dn_status_string(int(status)).decode()


def dn_last_error() -> str:
    return lib().dn_last_error().decode()


def dn_profile_enable(on: bool) -> None:
    _check(lib().dn_profile_enable(1 if on else 0))


def dn_profile_collect(max_kernels: int = 16) -> dict:
    """{kernel name: (total ms, launches)} of the launches since the last collect."""
    names = ctypes.create_string_buffer(32 * max_kernels)
    ms = (ctypes.c_double * max_kernels)()
    cnt = (ctypes.c_int * max_kernels)()
    n = lib().dn_profile_collect(names, ms, cnt, max_kernels)
    raw = names.raw
    out = {}
    for i in range(n):
        nm = raw[32 * i: 32 * i + 32].split(b"\0", 1)[0].decode()
        out[nm] = (ms[i], cnt[i])
    return out


def dn_chunk_fwd(shape, q, k, v, beta, g, h0, o, hT, states, ws, ws_bytes, stream=None) -> int:
    """Raw call; returns the dn_status (no exception)."""
    return lib().dn_chunk_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
                              _ptr(h0), _ptr(o), _ptr(hT), _ptr(states), _ptr(ws), int(ws_bytes),
                              _stream(stream))


def dn_chunk_fwd_noalloc(shape, q, k, v, beta, g, h0, o, hT, stream=None) -> int:
    """Raw call; returns the dn_status (no exception).  The forward without saved
    states, its scratch in the library's per-device array (no workspace)."""
    return lib().dn_chunk_fwd_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
                                      _ptr(h0), _ptr(o), _ptr(hT), _stream(stream))


def dn_chunk_bwd(shape, q, k, v, beta, g, h0, dout, dhT, states, dq, dk, dv, dbeta, dg, dh0, ws,
                 ws_bytes, stream=None) -> int:
    """Raw call; returns the dn_status (no exception)."""
    return lib().dn_chunk_bwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
                              _ptr(h0), _ptr(dout), _ptr(dhT), _ptr(states), _ptr(dq), _ptr(dk),
                              _ptr(dv), _ptr(dbeta), _ptr(dg), _ptr(dh0), _ptr(ws), int(ws_bytes),
                              _stream(stream))


def dn_recurrent_fwd(shape, q, k, v, beta, g, state, o, stream=None) -> int:
    """Raw call; returns the dn_status (no exception)."""
    return lib().dn_recurrent_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
                                  _ptr(state), _ptr(o), _stream(stream))


def dn_recurrent_phase_fwd(shape, q, k, v, beta, g, theta, state_re, state_im, o, stream=None) -> int:
    """Raw call; returns the dn_status (no exception)."""
    return lib().dn_recurrent_phase_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
                                        _ptr(theta), _ptr(state_re), _ptr(state_im), _ptr(o), _stream(stream))


def dn_phase_states_bytes(shape: Shape) -> int:
    return lib().dn_phase_states_bytes(ctypes.byref(shape))


def dn_phase_workspace_bytes(shape: Shape, pass_: int) -> int:
    return lib().dn_phase_workspace_bytes(ctypes.byref(shape), pass_)


def dn_chunk_phase_fwd(shape, q, k, v, beta, g, theta, h0_re, h0_im, o, hT_re, hT_im, states, ws=None, ws_bytes=0,
                       stream=None) -> int:
    """Raw call; returns the dn_status (no exception)."""
    return lib().dn_chunk_phase_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(theta),
                                    _ptr(h0_re), _ptr(h0_im), _ptr(o), _ptr(hT_re), _ptr(hT_im), _ptr(states),
                                    _ptr(ws), ws_bytes, _stream(stream))


def dn_chunk_phase_bwd(shape, q, k, v, beta, g, theta, h0_re, h0_im, dout, dhT_re, dhT_im, states, dq, dk, dv, dbeta,
                       dg, dtheta, dh0_re, dh0_im, ws=None, ws_bytes=0, stream=None) -> int:
    """Raw call; returns the dn_status (no exception).  states NULL: recompute
    (h0_re / h0_im used, workspace of DN_PASS_BWD_RECOMPUTE)."""
    return lib().dn_chunk_phase_bwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(theta),
                                    _ptr(h0_re), _ptr(h0_im), _ptr(dout), _ptr(dhT_re), _ptr(dhT_im), _ptr(states),
                                    _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbeta), _ptr(dg), _ptr(dtheta), _ptr(dh0_re),
                                    _ptr(dh0_im), _ptr(ws), ws_bytes, _stream(stream))


# ------------------------------------------------------------------ convenience


def _gate_kind(g, dk):
    if g is None:
        return DN_GATE_NONE
    return DN_GATE_VECTOR if g.dim() == 4 else DN_GATE_SCALAR


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


_IO_DTYPES = (torch.float32, torch.bfloat16)


def _validate(q, k, v, beta, g, h0=None, do=None, dhT=None, states=None, state=None, theta=None,
              state_im=None):
    """Check what the C ABI cannot: element types, shapes and devices of the
    tensors (it sizes every buffer from q's shape and the dtype field, so a
    mismatched tensor would be read past its end).  Raises ValueError.
      q, k [B,H,T,dk], v and do [B,H,T,dv]: one I/O type (fp32 or bf16)
      beta [B,H,T]; g [B,H,T] or [B,H,T,dk]; theta [B,H,T,dk]: fp32
      h0, dhT, state, state_im [B,H,dv,dk]: fp32;  states: uint8
    Every tensor contiguous and on q's CUDA device."""
    if q.dim() != 4:
        raise ValueError(f"q must be [B,H,T,dk], got shape {tuple(q.shape)}")
    Bq, Hq, Tq, dk = q.shape
    if q.dtype not in _IO_DTYPES:
        raise ValueError(f"q must be float32 or bfloat16, got {q.dtype}")
    if v.dim() != 4:
        raise ValueError(f"v must be [B,H,T,dv], got shape {tuple(v.shape)}")
    dv = v.shape[-1]
    want = {"k": (k, q.dtype, (Bq, Hq, Tq, dk)), "v": (v, q.dtype, (Bq, Hq, Tq, dv)),
            "beta": (beta, torch.float32, (Bq, Hq, Tq)), "do": (do, q.dtype, (Bq, Hq, Tq, dv)),
            "h0": (h0, torch.float32, (Bq, Hq, dv, dk)), "dhT": (dhT, torch.float32, (Bq, Hq, dv, dk)),
            "state": (state, torch.float32, (Bq, Hq, dv, dk)),
            "state_im": (state_im, torch.float32, (Bq, Hq, dv, dk)),
            "theta": (theta, torch.float32, (Bq, Hq, Tq, dk))}
    for name, (t, dt, shp) in want.items():
        if t is None:
            continue
        if t.dtype != dt:
            raise ValueError(f"{name} must be {dt} (q is {q.dtype}), got {t.dtype}")
        if tuple(t.shape) != shp:
            raise ValueError(f"{name} must have shape {shp}, got {tuple(t.shape)}")
    if g is not None:
        if g.dtype != torch.float32:
            raise ValueError(f"g must be torch.float32, got {g.dtype}")
        if tuple(g.shape) not in ((Bq, Hq, Tq), (Bq, Hq, Tq, dk)):
            raise ValueError(f"g must have shape {(Bq, Hq, Tq)} or {(Bq, Hq, Tq, dk)}, got {tuple(g.shape)}")
    if states is not None and states.dtype != torch.uint8:
        raise ValueError(f"states must be the uint8 buffer chunk_fwd returns, got {states.dtype}")
    ts = [q, k, v, beta, g, h0, do, dhT, states, state, theta, state_im]
    _contig(*ts)
    if q.device.type != "cuda":
        raise ValueError(f"tensors must be on a CUDA device, q is on {q.device}")
    for t in ts:
        if t is not None and t.device != q.device:
            raise ValueError(f"every tensor must be on {q.device}, found one on {t.device}")


def shape_of(q, v, g, C, kaczmarz_eps=None, no_scan=False) -> Shape:
    B, H, T, dk = q.shape
    return make_shape(B, H, T, dk, v.shape[-1], C, q.dtype, _gate_kind(g, dk), kaczmarz_eps, no_scan)


def workspace(shape: Shape, pass_: int, device) -> torch.Tensor:
    n = dn_workspace_bytes(shape, pass_)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def saved_buffer(shape: Shape, device) -> torch.Tensor:
    """Byte buffer for the forward's saved states, T, P, U and log-decay."""
    return torch.empty(max(dn_states_bytes(shape), 1), dtype=torch.uint8, device=device)


def saved_regions(buf: torch.Tensor, shape: Shape) -> dict:
    """Views of a saved buffer: states [B,H,NT,dv,dk], T and P [B,H,NT,C,C], U
    [B,H,NT,C,dv] (io type), gam like g (fp32; None without a gate), and with the Kaczmarz flag
    kz_beta and kz_rn [B,H,T] (fp32; else None)."""
    lay = dn_states_layout(shape)
    io = torch.bfloat16 if shape.dtype == DN_BF16 else torch.float32
    E = 2 if shape.dtype == DN_BF16 else 4
    B, H, T, dk, dv, C = shape.B, shape.H, shape.T, shape.dk, shape.dv, shape.C
    NT = -(-T // C) if T > 0 else 0

    def view(off, dims, dt, e):
        n = 1
        for x in dims:
            n *= x
        return buf[off:off + n * e].view(dt).reshape(dims)

    out = {"states": view(lay["states"], (B, H, NT, dv, dk), io, E),
           "T": view(lay["T"], (B, H, NT, C, C), io, E),
           "P": view(lay["P"], (B, H, NT, C, C), io, E), "U": view(lay["U"], (B, H, NT, C, dv), io, E),
           "gam": None, "kz_beta": None, "kz_rn": None}
    if shape.gate != DN_GATE_NONE:
        gw = (dk,) if shape.gate == DN_GATE_VECTOR else ()
        out["gam"] = view(lay["gam"], (B, H, T) + gw, torch.float32, 4)
    if shape.flags & DN_FLAG_KACZMARZ:
        out["kz_beta"] = view(lay["kz"], (B, H, T), torch.float32, 4)
        out["kz_rn"] = view(lay["kz"] + B * H * T * 4, (B, H, T), torch.float32, 4)
    return out


def chunk_fwd(q, k, v, beta, g=None, h0=None, C=64, save_states=True, want_hT=True, ws=None,
              stream=None, kaczmarz_eps=None, no_scan=False):
    """Returns (o, hT or None, saved buffer or None); saved_regions() views the buffer.
    With ``kaczmarz_eps`` set, ``beta`` is eta (Kaczmarz step)."""
    _validate(q, k, v, beta, g, h0)
    sh = shape_of(q, v, g, C, kaczmarz_eps, no_scan)
    o = torch.empty_like(v)
    hT = torch.empty(q.shape[0], q.shape[1], v.shape[-1], q.shape[-1], dtype=torch.float32,
                     device=q.device) if want_hT else None
    states = saved_buffer(sh, q.device) if save_states else None
    if ws is None:
        ws = workspace(sh, DN_PASS_FWD, q.device)
    _check(dn_chunk_fwd(sh, q, k, v, beta, g, h0, o, hT, states, ws, ws.numel(), stream))
    return o, hT, states


def chunk_bwd(q, k, v, beta, g, h0, do, dhT=None, states=None, C=64, want_dh0=True, ws=None,
              stream=None, kaczmarz_eps=None, no_scan=False):
    """Returns dict dq, dk, dv, dbeta, dg (None without a gate), dh0 (or None).  With
    ``kaczmarz_eps`` set, ``beta`` is eta and "dbeta" holds d eta."""
    _validate(q, k, v, beta, g, h0, do, dhT, states)
    sh = shape_of(q, v, g, C, kaczmarz_eps, no_scan)
    if states is not None and states.numel() < dn_states_bytes(sh):
        raise ValueError(f"states holds {states.numel()} bytes, this shape saves {dn_states_bytes(sh)}")
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dbeta = torch.empty_like(beta)
    dg = None if g is None else torch.empty_like(g)
    dh0 = torch.empty(q.shape[0], q.shape[1], v.shape[-1], q.shape[-1], dtype=torch.float32,
                      device=q.device) if want_dh0 else None
    if ws is None:
        ws = workspace(sh, DN_PASS_BWD if states is not None else DN_PASS_BWD_RECOMPUTE, q.device)
    _check(dn_chunk_bwd(sh, q, k, v, beta, g, h0, do, dhT, states, dq, dk, dv, dbeta, dg, dh0, ws,
                        ws.numel(), stream))
    return {"dq": dq, "dk": dk, "dv": dv, "dbeta": dbeta, "dg": dg, "dh0": dh0}


def recurrent_fwd(q, k, v, beta, g, state, stream=None, kaczmarz_eps=None):
    """T recurrent steps (decode); `state` (fp32 [B,H,dv,dk]) is updated in place.
    Returns o.  With ``kaczmarz_eps`` set, ``beta`` is eta."""
    _validate(q, k, v, beta, g, state=state)
    B, H, T, dk = q.shape
    sh = make_shape(B, H, T, dk, v.shape[-1], 64, q.dtype, _gate_kind(g, dk), kaczmarz_eps)
    o = torch.empty_like(v)
    _check(dn_recurrent_fwd(sh, q, k, v, beta, g, state, o, stream))
    return o


def recurrent_phase_fwd(q, k, v, beta, g, theta, state_re, state_im, gate=None, stream=None, kaczmarz_eps=None):
    """T recurrent steps with the phase-controlled gate; the complex state
    (state_re, state_im, fp32 [B,H,dv,dk]) is updated in place.  ``gate`` names
    how g is laid out when it is 4-D or 3-D (default: from g's rank).  Returns o."""
    _validate(q, k, v, beta, g, state=state_re, theta=theta, state_im=state_im)
    B, H, T, dk = q.shape
    sh = make_shape(B, H, T, dk, v.shape[-1], 64, q.dtype, gate if gate is not None else _gate_kind(g, dk),
                    kaczmarz_eps)
    o = torch.empty_like(v)
    _check(dn_recurrent_phase_fwd(sh, q, k, v, beta, g, theta, state_re, state_im, o, stream))
    return o


def chunk_phase_fwd(q, k, v, beta, g, theta, h0_re=None, h0_im=None, gate=None, save_states=True, stream=None):
    """Chunkwise forward of the phase-controlled gate (chunks of 16).  ``gate``
    names how g is laid out (default: from its rank).  Returns (o, hT_re, hT_im,
    states or None)."""
    _validate(q, k, v, beta, g, h0=h0_re, state_im=h0_im, theta=theta)
    B, H, T, dk = q.shape
    sh = make_shape(B, H, T, dk, v.shape[-1], 16, q.dtype, gate if gate is not None else _gate_kind(g, dk))
    o = torch.empty_like(v)
    hT_re = torch.empty(B, H, v.shape[-1], dk, dtype=torch.float32, device=q.device)
    hT_im = torch.empty_like(hT_re)
    states = (torch.empty(max(dn_phase_states_bytes(sh) // 4, 1), dtype=torch.float32, device=q.device)
              if save_states else None)
    nws = 0 if save_states else dn_phase_workspace_bytes(sh, DN_PASS_FWD)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=q.device) if nws else None
    _check(dn_chunk_phase_fwd(sh, q, k, v, beta, g, theta, h0_re, h0_im, o, hT_re, hT_im, states, ws, nws, stream))
    return o, hT_re, hT_im, states


def chunk_phase_bwd(q, k, v, beta, g, theta, do, dhT_re, dhT_im, states, h0_re=None, h0_im=None, gate=None,
                    stream=None):
    """Backward of chunk_phase_fwd from its saved states, or (states None) with the
    states recomputed from h0_re / h0_im.  Returns a dict dq, dk, dv, dbeta, dg
    (None without a gate), dtheta, dh0_re, dh0_im."""
    _validate(q, k, v, beta, g, h0_re, do=do, dhT=dhT_re, state_im=dhT_im, theta=theta)
    if h0_im is not None:
        _validate(q, k, v, beta, g, h0_im)
    B, H, T, dk = q.shape
    sh = make_shape(B, H, T, dk, v.shape[-1], 16, q.dtype, gate if gate is not None else _gate_kind(g, dk))
    if states is not None and (states.dtype != torch.float32 or states.numel() * 4 < dn_phase_states_bytes(sh)):
        raise ValueError("states must be the float32 buffer chunk_phase_fwd saved")
    out = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
           "dbeta": torch.empty_like(beta), "dg": None if g is None else torch.empty_like(g),
           "dtheta": torch.empty_like(theta),
           "dh0_re": torch.empty(B, H, v.shape[-1], dk, dtype=torch.float32, device=q.device)}
    out["dh0_im"] = torch.empty_like(out["dh0_re"])
    nws = dn_phase_workspace_bytes(sh, DN_PASS_BWD if states is not None else DN_PASS_BWD_RECOMPUTE)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=q.device)
    _check(dn_chunk_phase_bwd(sh, q, k, v, beta, g, theta, h0_re, h0_im, do, dhT_re, dhT_im, states, out["dq"],
                              out["dk"], out["dv"], out["dbeta"], out["dg"], out["dtheta"], out["dh0_re"],
                              out["dh0_im"], ws, nws, stream))
    return out


class DeltaRule(torch.autograd.Function):
    """o, hT = DeltaRule.apply(q, k, v, beta, g, h0, C, recompute, kaczmarz_eps); with
    kaczmarz_eps set, the fourth argument is eta."""

    @staticmethod
    def forward(ctx, q, k, v, beta, g, h0, C=64, recompute=False, kaczmarz_eps=None):
        o, hT, states = chunk_fwd(q, k, v, beta, g, h0, C=C, save_states=not recompute,
                                  kaczmarz_eps=kaczmarz_eps)
        ctx.C = C
        ctx.kz = kaczmarz_eps
        ctx.save_for_backward(q, k, v, beta, g, h0, states)
        return o, hT

    @staticmethod
    def backward(ctx, do, dhT):
        q, k, v, beta, g, h0, states = ctx.saved_tensors
        gr = chunk_bwd(q, k, v, beta, g, h0, do.contiguous(),
                       None if dhT is None else dhT.contiguous(), states, C=ctx.C, kaczmarz_eps=ctx.kz)
        return (gr["dq"], gr["dk"], gr["dv"], gr["dbeta"], gr["dg"], (gr["dh0"] if h0 is not None else None),
                None, None, None)
