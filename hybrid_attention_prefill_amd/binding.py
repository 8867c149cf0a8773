"""Thin ctypes binding of libhypic.so (include/hypic.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their device pointers and the current HIP stream are passed to the
C ABI, and a non-OK status raises.  Every step of the computation runs in the
library's HIP kernels; there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhypic.so")

HYPIC_OK, HYPIC_E_INVALID, HYPIC_E_UNSUPPORTED, HYPIC_E_DEVICE = 0, 1, 2, 3
GATE_HEAD, GATE_TOKEN, GATE_DIAG = 0, 1, 2
F32, BF16 = 0, 1
T_DENSE, T_SCALAR, T_SPLIT, T_DIAG = 0, 1, 2, 3

EXPORTED = ("hypic_segment_build", "hypic_build_workspace_bytes", "hypic_segment_prefill", "hypic_compose",
            "hypic_seam_advance", "hypic_seam_advance_noalloc",
            "hypic_seam_workspace_bytes", "hypic_last_error", "hypic_abi_version", "hypic_selftest_layouts")
NOALLOC_SCRATCH_BYTES = 128 << 20


class HypicError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"hypic status {status}: {msg}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("gate", ctypes.c_int32), ("delta", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
                ("t_layout", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libhypic.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m hybrid_attention_prefill_amd.build_lib`")
    lib = ctypes.CDLL(path)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    D = ctypes.POINTER(Dims)
    lib.hypic_segment_build.argtypes = [D, I32, P, P, I64, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.hypic_segment_build.restype = ctypes.c_int
    lib.hypic_build_workspace_bytes.argtypes = [D, I32, I64]
    lib.hypic_segment_prefill.argtypes = [D, I32, P, P, I64, P, P, P, P, P, ctypes.c_float, P, P, P, P]
    lib.hypic_segment_prefill.restype = ctypes.c_int
    lib.hypic_build_workspace_bytes.restype = ctypes.c_size_t
    lib.hypic_compose.argtypes = [D, I32, I32, P, I32, P, P, P, P]
    lib.hypic_compose.restype = ctypes.c_int
    lib.hypic_seam_advance.argtypes = [D, I32, I32, I32, P, I64, P, P, P, P, P, ctypes.c_float, P, I32,
                                       P, P, P, P, P, ctypes.c_size_t, P]
    lib.hypic_seam_advance.restype = ctypes.c_int
    lib.hypic_seam_advance_noalloc.argtypes = [D, I32, I32, I32, P, I64, P, P, P, P, P, ctypes.c_float, P, I32,
                                               P, P, P, P, P]
    lib.hypic_seam_advance_noalloc.restype = ctypes.c_int
    lib.hypic_seam_workspace_bytes.argtypes = [D, I32, I32, I32]
    lib.hypic_seam_workspace_bytes.restype = ctypes.c_size_t
    lib.hypic_last_error.restype = ctypes.c_char_p
    lib.hypic_abi_version.restype = ctypes.c_int32
    lib.hypic_selftest_layouts.argtypes = [P, P, P]
    lib.hypic_selftest_layouts.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status):
    if status != HYPIC_OK:
        raise HypicError(status, load_library().hypic_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, name, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _in_dtype(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise ValueError(f"inputs must be bfloat16 or float32, got {t.dtype}")


def _t_shape(t_layout, n, H, dk):
    return {T_DENSE: (n, H, dk, dk), T_SCALAR: (n, H), T_SPLIT: (n, H, 2, dk * dk), T_DIAG: (n, H, dk)}[t_layout]


def _t_dtype(t_layout):
    return torch.bfloat16 if t_layout == T_SPLIT else torch.float32


def t_layout_of(T):
    """Layout of a T cache tensor: bf16 [n,H,2,d*d] SPLIT, fp32 [n,H] SCALAR, fp32 [n,H,d] DIAG,
    fp32 [n,H,d,d] DENSE."""
    if T.dtype == torch.bfloat16 and T.dim() == 4:
        return T_SPLIT
    if T.dtype == torch.float32 and T.dim() == 2:
        return T_SCALAR
    if T.dtype == torch.float32 and T.dim() == 3:
        return T_DIAG
    if T.dtype == torch.float32 and T.dim() == 4:
        return T_DENSE
    raise ValueError(f"T cache of dtype {T.dtype} and shape {tuple(T.shape)} matches no T layout")


def make_dims(H, dk, dv, *, gate, delta, in_dtype, t_layout=T_DENSE):
    """delta: False/0 plain write, True/1 erase then gate, 2 gate then erase."""
    return Dims(int(H), int(dk), int(dv), int(gate), int(delta), int(in_dtype), int(t_layout))


def abi_version() -> int:
    return int(load_library().hypic_abi_version())


def build_workspace_bytes(H, dk, dv, n_seg, n_tokens, *, gate=GATE_TOKEN, delta=True, in_dtype=BF16):
    d = make_dims(H, dk, dv, gate=gate, delta=delta, in_dtype=in_dtype)
    return int(load_library().hypic_build_workspace_bytes(ctypes.byref(d), n_seg, n_tokens))


def segment_build(k, v, g, beta, seg_begin, seg_end, *, gate, delta, t_layout=T_DENSE,
                  want_T=True, T_out=None, S_out=None, workspace="auto", stream=None):
    """(T_C, S(C|0)) for every (segment, head) -- hypic_segment_build.
    workspace: "auto" allocates the build workspace (long segments are cut into pieces
    built in parallel), None builds every segment as one chain, or a uint8 device tensor."""
    lib = load_library()
    _dev(k, "k")
    n_tok, H, dk = k.shape
    dv = v.shape[2]
    dt = _in_dtype(k)
    _dev(v, "v", k.dtype, (n_tok, H, dv))
    if gate == GATE_HEAD:
        _dev(g, "g", torch.float32, (H,))
    elif gate == GATE_TOKEN:
        _dev(g, "g", k.dtype, (n_tok, H))
    else:
        _dev(g, "g", k.dtype, (n_tok, H, dk))
    if delta:
        _dev(beta, "beta", k.dtype, (n_tok, H))
    _dev(seg_begin, "seg_begin", torch.int64)
    n_seg = seg_begin.shape[0]
    _dev(seg_end, "seg_end", torch.int64, (n_seg,))
    if S_out is None:
        S_out = torch.empty((n_seg, H, dk, dv), device=k.device, dtype=torch.float32)
    _dev(S_out, "S_out", torch.float32, (n_seg, H, dk, dv))
    if want_T and T_out is None:
        T_out = torch.empty(_t_shape(t_layout, n_seg, H, dk), device=k.device, dtype=_t_dtype(t_layout))
    if T_out is not None:
        _dev(T_out, "T_out", _t_dtype(t_layout), _t_shape(t_layout, n_seg, H, dk))
    d = make_dims(H, dk, dv, gate=gate, delta=delta, in_dtype=dt, t_layout=t_layout)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError(f"workspace must be 'auto', None or a tensor (got {workspace!r})")
        need = int(lib.hypic_build_workspace_bytes(ctypes.byref(d), n_seg, n_tok))
        workspace = torch.empty(need, device=k.device, dtype=torch.uint8) if need > 0 else None
    if workspace is not None:
        _dev(workspace, "workspace", torch.uint8)
    _check(lib.hypic_segment_build(ctypes.byref(d), n_seg, _ptr(seg_begin), _ptr(seg_end), n_tok, _ptr(k),
                                   _ptr(v), _ptr(g), _ptr(beta) if delta else None, _ptr(T_out),
                                   _ptr(S_out), _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                   _stream(stream)))
    return T_out, S_out


def segment_prefill(q, k, v, g, beta, seg_begin, seg_end, *, scale, t_layout=T_DENSE, want_T=True, T_out=None,
                    S_out=None, out=None, stream=None):
    """Cold prefill of every segment in isolation -- hypic_segment_prefill: the pair
    (T_C, S(C|0)) and every token's output out[t] = S_t^T (scale q_t) (fp32 [n_tok][H][d_v];
    rows of tokens outside the segments are left as they are)."""
    lib = load_library()
    _dev(k, "k")
    n_tok, H, dk = k.shape
    dv = v.shape[2]
    dt = _in_dtype(k)
    _dev(q, "q", k.dtype, (n_tok, H, dk))
    _dev(v, "v", k.dtype, (n_tok, H, dv))
    _dev(g, "g", k.dtype, (n_tok, H))
    _dev(beta, "beta", k.dtype, (n_tok, H))
    _dev(seg_begin, "seg_begin", torch.int64)
    n_seg = seg_begin.shape[0]
    _dev(seg_end, "seg_end", torch.int64, (n_seg,))
    if S_out is None:
        S_out = torch.empty((n_seg, H, dk, dv), device=k.device, dtype=torch.float32)
    _dev(S_out, "S_out", torch.float32, (n_seg, H, dk, dv))
    if want_T and T_out is None:
        T_out = torch.empty(_t_shape(t_layout, n_seg, H, dk), device=k.device, dtype=_t_dtype(t_layout))
    if T_out is not None:
        _dev(T_out, "T_out", _t_dtype(t_layout), _t_shape(t_layout, n_seg, H, dk))
    if out is None:
        out = torch.zeros((n_tok, H, dv), device=k.device, dtype=torch.float32)
    _dev(out, "out", torch.float32, (n_tok, H, dv))
    d = make_dims(H, dk, dv, gate=GATE_TOKEN, delta=True, in_dtype=dt, t_layout=t_layout)
    _check(lib.hypic_segment_prefill(ctypes.byref(d), n_seg, _ptr(seg_begin), _ptr(seg_end), n_tok, _ptr(q), _ptr(k),
                                     _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(T_out), _ptr(S_out), _ptr(out),
                                     _stream(stream)))
    return T_out, S_out, out


def compose(T_cache, S_cache, pair_id, S_run, *, t_layout=None, stream=None):
    """In place: S_run[c] <- T[id] S_run[c] + S[id] along each chain -- hypic_compose.
    The T layout is taken from T_cache's dtype and rank unless given."""
    lib = load_library()
    _dev(S_cache, "S_cache", torch.float32)
    n_pair, H, dk, dv = S_cache.shape
    if t_layout is None:
        t_layout = t_layout_of(T_cache)
    _dev(T_cache, "T_cache", _t_dtype(t_layout), _t_shape(t_layout, n_pair, H, dk))
    _dev(pair_id, "pair_id", torch.int32)
    n_chain, n_step = pair_id.shape
    _dev(S_run, "S_run", torch.float32, (n_chain, H, dk, dv))
    gate = {T_SCALAR: GATE_HEAD, T_DIAG: GATE_DIAG}.get(t_layout, GATE_TOKEN)
    d = make_dims(H, dk, dv, gate=gate, delta=0, in_dtype=F32, t_layout=t_layout)
    _check(lib.hypic_compose(ctypes.byref(d), n_chain, n_step, _ptr(pair_id), n_pair, _ptr(T_cache),
                             _ptr(S_cache), _ptr(S_run), _stream(stream)))
    return S_run


def seam_workspace_bytes(H, dk, dv, n_chain, n_step, w, *, gate=GATE_TOKEN, delta=True, in_dtype=BF16):
    d = make_dims(H, dk, dv, gate=gate, delta=delta, in_dtype=in_dtype)
    return int(load_library().hypic_seam_workspace_bytes(ctypes.byref(d), n_chain, n_step, w))


def seam_advance(q, k, v, g, beta, seam_start, S_run, out, *, gate, delta, w, scale, pair_id=None,
                 T_cache=None, S_cache=None, workspace=None, stream=None):
    """Seam windows then composition along each chain -- hypic_seam_advance (in place on S_run, out)."""
    lib = load_library()
    _dev(k, "k")
    n_tok, H, dk = k.shape
    dv = v.shape[2]
    dt = _in_dtype(k)
    _dev(q, "q", k.dtype, (n_tok, H, dk))
    _dev(v, "v", k.dtype, (n_tok, H, dv))
    _dev(seam_start, "seam_start", torch.int64)
    n_chain, n_step = seam_start.shape
    _dev(S_run, "S_run", torch.float32, (n_chain, H, dk, dv))
    _dev(out, "out", torch.float32, (n_chain, n_step, w, H, dv))
    n_pair, t_layout = 0, T_DENSE
    if pair_id is not None:
        _dev(pair_id, "pair_id", torch.int32, (n_chain, n_step))
        _dev(S_cache, "S_cache", torch.float32)
        n_pair = S_cache.shape[0]
        t_layout = t_layout_of(T_cache)
        if t_layout in (T_SCALAR, T_DIAG):
            raise ValueError("seam_advance needs a dense T cache (DENSE or SPLIT layout)")
        _dev(T_cache, "T_cache", _t_dtype(t_layout), _t_shape(t_layout, n_pair, H, dk))
    need = seam_workspace_bytes(H, dk, dv, n_chain, n_step, w, gate=gate, delta=delta, in_dtype=dt)
    if workspace is None and need > 0:
        workspace = torch.empty(need, device=k.device, dtype=torch.uint8)
    d = make_dims(H, dk, dv, gate=gate, delta=delta, in_dtype=dt, t_layout=t_layout)
    _check(lib.hypic_seam_advance(ctypes.byref(d), n_chain, n_step, w, _ptr(seam_start), n_tok, _ptr(q),
                                  _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(pair_id), n_pair,
                                  _ptr(T_cache), _ptr(S_cache), _ptr(S_run), _ptr(out), _ptr(workspace),
                                  0 if workspace is None else workspace.numel(), _stream(stream)))
    return S_run, out


def seam_advance_noalloc(q, k, v, g, beta, seam_start, S_run, out, *, gate, delta, w, scale, pair_id=None,
                         T_cache=None, S_cache=None, stream=None):
    """hypic_seam_advance_noalloc: seam_advance with the library's static device scratch instead of
    a workspace (nothing is allocated; calls that overlap on one device race)."""
    lib = load_library()
    _dev(k, "k")
    n_tok, H, dk = k.shape
    dv = v.shape[2]
    dt = _in_dtype(k)
    _dev(q, "q", k.dtype, (n_tok, H, dk))
    _dev(v, "v", k.dtype, (n_tok, H, dv))
    _dev(seam_start, "seam_start", torch.int64)
    n_chain, n_step = seam_start.shape
    _dev(S_run, "S_run", torch.float32, (n_chain, H, dk, dv))
    _dev(out, "out", torch.float32, (n_chain, n_step, w, H, dv))
    n_pair, t_layout = 0, T_DENSE
    if pair_id is not None:
        _dev(pair_id, "pair_id", torch.int32, (n_chain, n_step))
        _dev(S_cache, "S_cache", torch.float32)
        n_pair = S_cache.shape[0]
        t_layout = t_layout_of(T_cache)
        _dev(T_cache, "T_cache", _t_dtype(t_layout), _t_shape(t_layout, n_pair, H, dk))
    d = make_dims(H, dk, dv, gate=gate, delta=delta, in_dtype=dt, t_layout=t_layout)
    _check(lib.hypic_seam_advance_noalloc(ctypes.byref(d), n_chain, n_step, w, _ptr(seam_start), n_tok, _ptr(q),
                                          _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(pair_id),
                                          n_pair, _ptr(T_cache), _ptr(S_cache), _ptr(S_run), _ptr(out),
                                          _stream(stream)))
    return S_run, out


def selftest_layouts(device="cuda"):
    """Run the lane-layout self-test kernel on in = [0, 1, ..., 255]; returns its 2112 raw floats (host)."""
    lib = load_library()
    inp = torch.arange(256, device=device, dtype=torch.float32)
    out = torch.full((2112,), float("nan"), device=device, dtype=torch.float32)
    _check(lib.hypic_selftest_layouts(_ptr(inp), _ptr(out), _stream(None)))
    torch.cuda.synchronize()
    return out.cpu().numpy()
