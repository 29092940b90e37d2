"""Python binding of the MI355X Mamba2 selective-state scan library.

Argument marshalling only: every step of the scan, of the conv1d + SiLU
and gated RMSNorm beside it, and of the gated delta-rule recurrence runs in the HIP kernels of ``libssmscan.so``
(built from ``csrc/`` by ``build.py``), reached through its C ABI
(``include/ssm_scan.h``, ``include/ssm_conv_norm.h``, ``include/ssm_gdn.h``).  torch supplies device memory and the current
stream; tensors are passed as raw device pointers.  There is no CPU fallback:
if the library is missing, importing this package raises.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libssmscan.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "ssm_scan.h")
HEADERS = [HEADER] + [os.path.join(os.path.dirname(PKG), "include", h)
                      for h in ("ssm_conv_norm.h", "ssm_gdn.h")]

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
        "or `python mamba2_selective_scan_amd/build.py` first")

# torch ships its own HIP runtime under the same soname (libamdhip64.so.7).
# Importing torch first makes the library bind to that runtime, so torch's
# device pointers and stream handles are valid in our calls.  Loading the
# library first would bring in a second runtime and every launch would fail.
import torch  # noqa: E402,F401  (load order matters, see above)

_lib = ctypes.CDLL(LIB_PATH)


def hip_runtimes_loaded() -> list:
    """Paths of the HIP runtime libraries mapped into this process (Linux)."""
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


if len(hip_runtimes_loaded()) > 1:
    raise ImportError("two HIP runtimes are loaded in this process "
                      f"({hip_runtimes_loaded()}); import torch before anything that "
                      "links /opt/rocm's libamdhip64, and before this package")

SSM_OK = 0
SSM_ERR_NULL = -1
SSM_ERR_DIMS = -2
SSM_ERR_UNSUPPORTED = -3
SSM_ERR_ALIGN = -4
SSM_ERR_LAUNCH = -5
SSM_ERR_METADATA = -6
SSM_ERR_SCRATCH = -7
MAX_D_STATE = 1024
STATIC_SCRATCH_BYTES = 48 << 20     # SSM_SCAN_STATIC_SCRATCH_BYTES


class Dims(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("d_state", ctypes.c_int32), ("n_groups", ctypes.c_int32)]


class Options(ctypes.Structure):
    _fields_ = [("dt_bias", ctypes.c_void_p), ("dt_softplus", ctypes.c_int32),
                ("a_per_state", ctypes.c_int32), ("snapshots", ctypes.c_void_p)]


class Geometry(ctypes.Structure):
    _fields_ = [("lanes_per_row", ctypes.c_int32), ("elems_per_lane", ctypes.c_int32),
                ("rows_per_block", ctypes.c_int32), ("chunk_tokens", ctypes.c_int32),
                ("threads_per_block", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
                ("blocks", ctypes.c_int64), ("vector_path", ctypes.c_int32),
                ("segments", ctypes.c_int32), ("segment_tokens", ctypes.c_int32)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_lib.ssm_scan_prefill.argtypes = [ctypes.POINTER(Dims), _i32, _i32] + [_vp] * 9 + [_i32, _vp, _vp]
_lib.ssm_scan_prefill.restype = ctypes.c_int
_lib.ssm_scan_decode.argtypes = [ctypes.POINTER(Dims), _i32] + [_vp] * 8 + [_i32, _vp, _vp]
_lib.ssm_scan_decode.restype = ctypes.c_int
_lib.ssm_scan_strerror.argtypes = [ctypes.c_int]
_lib.ssm_scan_strerror.restype = ctypes.c_char_p
_lib.ssm_scan_version.argtypes = []
_lib.ssm_scan_version.restype = ctypes.c_int
_lib.ssm_scan_last_hip_error.argtypes = []
_lib.ssm_scan_last_hip_error.restype = ctypes.c_int
_lib.ssm_scan_last_hip_error_string.argtypes = []
_lib.ssm_scan_last_hip_error_string.restype = ctypes.c_char_p
_lib.ssm_scan_check_metadata.argtypes = [_i32, _i32, _vp, _vp, _i32, _vp]
_lib.ssm_scan_check_metadata.restype = ctypes.c_int
_lib.ssm_scan_check_metadata_host.argtypes = [_i32, _i32, _vp, _vp, _i32]
_lib.ssm_scan_check_metadata_host.restype = ctypes.c_int
_lib.ssm_scan_query_geometry.argtypes = [ctypes.POINTER(Dims), _i32, _i32, _i32,
                                         ctypes.POINTER(Geometry)]
_lib.ssm_scan_query_geometry.restype = ctypes.c_int
_lib.ssm_scan_query_prefill_plan.argtypes = [ctypes.POINTER(Dims), _i32, _i32, _i32, _i32,
                                             ctypes.POINTER(Geometry)]
_lib.ssm_scan_query_prefill_plan.restype = ctypes.c_int
_lib.ssm_scan_prefill_workspace_size.argtypes = [ctypes.POINTER(Dims), _i32, _i32, _i32, _i32,
                                                 ctypes.POINTER(ctypes.c_size_t)]
_lib.ssm_scan_prefill_workspace_size.restype = ctypes.c_int
_lib.ssm_scan_prefill_ws.argtypes = ([ctypes.POINTER(Dims), _i32, _i32, _i32, _i32] + [_vp] * 9
                                     + [_i32, _vp, _vp, ctypes.c_size_t, _vp])
_lib.ssm_scan_prefill_ws.restype = ctypes.c_int
_lib.ssm_scan_prefill_static.argtypes = ([ctypes.POINTER(Dims), _i32, _i32, _i32, _i32] + [_vp] * 9
                                         + [_i32, _vp, _vp])
_lib.ssm_scan_prefill_static.restype = ctypes.c_int
_lib.ssm_scan_prefill_opt.argtypes = ([ctypes.POINTER(Dims), ctypes.POINTER(Options), _i32, _i32,
                                       _i32, _i32] + [_vp] * 9
                                      + [_i32, _vp, _vp, ctypes.c_size_t, _vp])
_lib.ssm_scan_prefill_opt.restype = ctypes.c_int
_lib.ssm_scan_decode_opt.argtypes = ([ctypes.POINTER(Dims), ctypes.POINTER(Options), _i32]
                                     + [_vp] * 8 + [_i32, _vp, _vp])
_lib.ssm_scan_decode_opt.restype = ctypes.c_int


class ConvDims(ctypes.Structure):
    _fields_ = [("channels", ctypes.c_int32), ("kernel", ctypes.c_int32)]


MAX_CONV_KERNEL = 4
_lib.ssm_conv1d_silu_prefill.argtypes = ([ctypes.POINTER(ConvDims), _i32, _i32] + [_vp] * 6
                                         + [_i32, _vp, _vp, _vp])
_lib.ssm_conv1d_silu_prefill.restype = ctypes.c_int
_lib.ssm_conv1d_silu_decode.argtypes = ([ctypes.POINTER(ConvDims), _i32] + [_vp] * 5
                                        + [_i32, _vp, _vp])
_lib.ssm_conv1d_silu_decode.restype = ctypes.c_int
_lib.ssm_gated_rmsnorm.argtypes = [ctypes.c_int64, _i32, _vp, _vp, _vp, ctypes.c_float, _vp, _vp]
_lib.ssm_gated_rmsnorm.restype = ctypes.c_int


class GdnDims(ctypes.Structure):
    _fields_ = [("n_v_heads", ctypes.c_int32), ("n_k_heads", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32)]


MAX_GDN_DK = 256
_lib.ssm_gdn_prefill.argtypes = ([ctypes.POINTER(GdnDims), _i32, _i32] + [_vp] * 8
                                 + [ctypes.c_float, _vp, _i32, _vp, _vp, _vp])
_lib.ssm_gdn_prefill.restype = ctypes.c_int
_lib.ssm_gdn_prefill_ws.argtypes = ([ctypes.POINTER(GdnDims), _i32, _i32] + [_vp] * 8
                                    + [ctypes.c_float, _vp, _i32, _vp, _i32, _vp, ctypes.c_size_t,
                                       _vp])
_lib.ssm_gdn_prefill_ws.restype = ctypes.c_int
_lib.ssm_gdn_prefill_workspace_size.argtypes = [ctypes.POINTER(GdnDims), _i32, _i32,
                                                ctypes.POINTER(ctypes.c_size_t)]
_lib.ssm_gdn_prefill_workspace_size.restype = ctypes.c_int
_lib.ssm_gdn_decode.argtypes = ([ctypes.POINTER(GdnDims), _i32] + [_vp] * 7
                                + [ctypes.c_float, _vp, _i32, _vp, _vp, _vp])
_lib.ssm_gdn_decode.restype = ctypes.c_int


class ScanError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = f"{where}: {strerror(code)} (status {code})"
        if code == SSM_ERR_LAUNCH:
            self.hip_error = int(_lib.ssm_scan_last_hip_error())
            msg += (f"; HIP error {self.hip_error}: "
                    f"{_lib.ssm_scan_last_hip_error_string().decode()}")
        super().__init__(msg)


def lib() -> ctypes.CDLL:
    """The loaded C library (for callers that want the raw ABI)."""
    return _lib


def header_symbols() -> list:
    """Names of the functions the headers under include/ declare."""
    names = set()
    for h in HEADERS:
        text = open(h).read()
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ssm_\w+)\s*\(", text, re.M))
    return sorted(names)


def strerror(code: int) -> str:
    return _lib.ssm_scan_strerror(int(code)).decode()


def version() -> int:
    return int(_lib.ssm_scan_version())


def _check(rc: int, where: str) -> None:
    if rc != SSM_OK:
        raise ScanError(rc, where)


def geometry(H, P, N, G, n_seqs, decode=False, aligned=True) -> dict:
    out = Geometry()
    _check(_lib.ssm_scan_query_geometry(ctypes.byref(Dims(H, P, N, G)), int(n_seqs),
                                        int(bool(decode)), int(bool(aligned)),
                                        ctypes.byref(out)), "ssm_scan_query_geometry")
    return out.as_dict()


def prefill_plan(H, P, N, G, n_seqs, max_seqlen, segments=0, aligned=True) -> dict:
    """Geometry of the segment scan ``prefill_ws`` would launch (segments == 1:
    it would not split)."""
    out = Geometry()
    _check(_lib.ssm_scan_query_prefill_plan(ctypes.byref(Dims(H, P, N, G)), int(n_seqs),
                                            int(max_seqlen), int(segments), int(bool(aligned)),
                                            ctypes.byref(out)), "ssm_scan_query_prefill_plan")
    return out.as_dict()


def workspace_size(H, P, N, G, n_seqs, n_tokens, max_seqlen, segments=0) -> int:
    """Bytes of device workspace ``prefill_ws`` needs (0: it would not split)."""
    b = ctypes.c_size_t()
    _check(_lib.ssm_scan_prefill_workspace_size(ctypes.byref(Dims(H, P, N, G)), int(n_seqs),
                                                int(n_tokens), int(max_seqlen), int(segments),
                                                ctypes.byref(b)), "ssm_scan_prefill_workspace_size")
    return int(b.value)


def check_metadata(cu_seqlens, slot, n_tokens: int, n_slots: int, stream=None) -> int:
    """Check a batch's metadata; returns the status code (SSM_OK or SSM_ERR_*).

    ``slot`` as a CUDA int32 tensor (and ``cu_seqlens`` as one, or None for a
    decode batch): ``ssm_scan_check_metadata`` copies them to the host on
    ``stream`` (default: the current stream) and waits.  Host arrays (numpy
    or CPU tensors): ``ssm_scan_check_metadata_host``."""
    import numpy as np
    if hasattr(slot, "is_cuda") and slot.is_cuda:
        import torch
        dev = slot.device
        slot_p = _dev_ptr(slot, torch.int32, "slot", dev)
        cu_p = None if cu_seqlens is None else _dev_ptr(cu_seqlens, torch.int32, "cu_seqlens", dev)
        if cu_seqlens is not None and tuple(cu_seqlens.shape) != (int(slot.shape[0]) + 1,):
            raise ValueError("cu_seqlens must have n_seqs + 1 entries")
        return int(_lib.ssm_scan_check_metadata(int(slot.shape[0]), int(n_tokens), cu_p, slot_p,
                                                int(n_slots), _stream_handle(stream, dev)))
    slot_h = np.ascontiguousarray(_to_host(slot), dtype=np.int32)
    cu_h = None if cu_seqlens is None else np.ascontiguousarray(_to_host(cu_seqlens),
                                                                 dtype=np.int32)
    return int(_lib.ssm_scan_check_metadata_host(
        int(slot_h.shape[0]), int(n_tokens),
        None if cu_h is None else cu_h.ctypes.data, slot_h.ctypes.data, int(n_slots)))


def _to_host(a):
    if hasattr(a, "detach"):
        return a.detach().cpu().numpy()
    return a


# ------------------------------------------------------------------ torch side
def _dev_ptr(t, dtype, name, device):
    import torch
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr() if t.numel() else None


def _options(dev, T, H, P, N, dt_bias, dt_softplus, A_per_state, snapshots):
    """The ssm_scan_options struct for these keyword options, or None if all
    are off."""
    import torch
    if dt_bias is None and not dt_softplus and not A_per_state and snapshots is None:
        return None
    if dt_bias is not None and tuple(dt_bias.shape) != (H,):
        raise ValueError("dt_bias must have shape [H]")
    if snapshots is not None and tuple(snapshots.shape) != (T, H, P, N):
        raise ValueError("snapshots must have shape [T, H, P, N]")
    return Options(_dev_ptr(dt_bias, torch.float32, "dt_bias", dev), int(bool(dt_softplus)),
                   int(bool(A_per_state)), _dev_ptr(snapshots, torch.float32, "snapshots", dev))


def _stream_handle(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def prefill(x, dt, A, B, C, state, cu_seqlens, slot, fresh, y=None, stream=None,
            dt_bias=None, dt_softplus=False, A_per_state=False, snapshots=None):
    """Scan a packed batch on the GPU (``ssm_scan_prefill``), one pass per
    sequence.

    x [T, H, P], dt [T, H], A [H] (or [H, N] with ``A_per_state``), B and C
    [T, G, N] fp32; state [n_slots, H, P, N] fp32 (updated in place);
    cu_seqlens [n_seqs+1] and slot [n_seqs] int32; fresh [n_seqs] uint8.
    Options (``ssm_scan_prefill_opt``): ``dt_bias`` [H], ``dt_softplus``,
    ``A_per_state``, ``snapshots`` [T, H, P, N] fp32 output.  Returns y
    [T, H, P] (``y`` if given).  Enqueued on ``stream`` (default: the current
    stream), no sync.
    """
    return _prefill_any(x, dt, A, B, C, state, cu_seqlens, slot, fresh, 0, 1, None, y, stream,
                        dt_bias, dt_softplus, A_per_state, snapshots)


def _prefill_any(x, dt, A, B, C, state, cu_seqlens, slot, fresh, max_seqlen, segments,
                 workspace, y, stream, dt_bias, dt_softplus, A_per_state, snapshots):
    import torch
    n_slots, H, P, N = (int(v) for v in state.shape)
    T = int(x.shape[0])
    G = int(B.shape[1])
    n_seqs = int(slot.shape[0])
    a_shape = (H, N) if A_per_state else (H,)
    if tuple(x.shape) != (T, H, P) or tuple(dt.shape) != (T, H) or tuple(A.shape) != a_shape:
        raise ValueError("x, dt or A has the wrong shape")
    if tuple(B.shape) != (T, G, N) or tuple(C.shape) != (T, G, N):
        raise ValueError("B or C has the wrong shape")
    if tuple(cu_seqlens.shape) != (n_seqs + 1,) or tuple(fresh.shape) != (n_seqs,):
        raise ValueError("cu_seqlens or fresh has the wrong shape")
    dev = state.device
    if y is None:
        y = torch.empty((T, H, P), dtype=torch.float32, device=dev)
    elif tuple(y.shape) != (T, H, P):
        raise ValueError("y has the wrong shape")
    opts = _options(dev, T, H, P, N, dt_bias, dt_softplus, A_per_state, snapshots)
    f32, i32 = torch.float32, torch.int32
    args = (_dev_ptr(cu_seqlens, i32, "cu_seqlens", dev), _dev_ptr(slot, i32, "slot", dev),
            _dev_ptr(fresh, torch.uint8, "fresh", dev), _dev_ptr(x, f32, "x", dev),
            _dev_ptr(dt, f32, "dt", dev), _dev_ptr(A, f32, "A", dev), _dev_ptr(B, f32, "B", dev),
            _dev_ptr(C, f32, "C", dev), _dev_ptr(state, f32, "state", dev), n_slots,
            _dev_ptr(y, f32, "y", dev))
    if opts is None and max_seqlen == 0:
        rc = _lib.ssm_scan_prefill(ctypes.byref(Dims(H, P, N, G)), n_seqs, T, *args,
                                   _stream_handle(stream, dev))
        _check(rc, "ssm_scan_prefill")
        return y
    ws_ptr, ws_bytes = None, 0
    if max_seqlen:
        need = workspace_size(H, P, N, G, n_seqs, T, max_seqlen, segments)
        if workspace is None and need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        if workspace is not None:
            ws_ptr = _dev_ptr(workspace, torch.uint8, "workspace", dev)
            ws_bytes = int(workspace.numel())
    rc = _lib.ssm_scan_prefill_opt(ctypes.byref(Dims(H, P, N, G)),
                                   None if opts is None else ctypes.byref(opts), n_seqs, T,
                                   int(max_seqlen), int(segments), *args, ws_ptr, ws_bytes,
                                   _stream_handle(stream, dev))
    _check(rc, "ssm_scan_prefill_opt")
    return y


def prefill_ws(x, dt, A, B, C, state, cu_seqlens, slot, fresh, max_seqlen, segments=0,
               workspace=None, y=None, stream=None, dt_bias=None, dt_softplus=False,
               A_per_state=False, snapshots=None):
    """``ssm_scan_prefill_opt`` / ``ssm_scan_prefill_ws``: like ``prefill``, but
    long sequences may be split over time when the batch is too small to fill
    the GPU.  ``max_seqlen`` (host int) bounds the sequence lengths;
    ``segments`` 0 = automatic, 1 = never split, k = about k segments.
    ``workspace`` (a uint8 CUDA tensor of at least ``workspace_size(...)``
    bytes) is allocated here when not given.  Options as for ``prefill``."""
    return _prefill_any(x, dt, A, B, C, state, cu_seqlens, slot, fresh, max(int(max_seqlen), 0),
                        segments, workspace, y, stream, dt_bias, dt_softplus, A_per_state,
                        snapshots)


def prefill_static(x, dt, A, B, C, state, cu_seqlens, slot, fresh, max_seqlen, segments=0,
                   y=None, stream=None):
    """``ssm_scan_prefill_static``: ``prefill_ws`` with the library's own
    static device scratch (no workspace, nothing allocated in the call; only
    ``y`` is allocated here when not given).  Raises ``ScanError`` with
    ``SSM_ERR_SCRATCH`` when the split would need more than the scratch holds."""
    import torch
    n_slots, H, P, N = (int(v) for v in state.shape)
    T = int(x.shape[0])
    G = int(B.shape[1])
    n_seqs = int(slot.shape[0])
    if tuple(x.shape) != (T, H, P) or tuple(dt.shape) != (T, H) or tuple(A.shape) != (H,):
        raise ValueError("x, dt or A has the wrong shape")
    if tuple(B.shape) != (T, G, N) or tuple(C.shape) != (T, G, N):
        raise ValueError("B or C has the wrong shape")
    if tuple(cu_seqlens.shape) != (n_seqs + 1,) or tuple(fresh.shape) != (n_seqs,):
        raise ValueError("cu_seqlens or fresh has the wrong shape")
    dev = state.device
    if y is None:
        y = torch.empty((T, H, P), dtype=torch.float32, device=dev)
    elif tuple(y.shape) != (T, H, P):
        raise ValueError("y has the wrong shape")
    f32, i32 = torch.float32, torch.int32
    rc = _lib.ssm_scan_prefill_static(
        ctypes.byref(Dims(H, P, N, G)), n_seqs, T, max(int(max_seqlen), 0), int(segments),
        _dev_ptr(cu_seqlens, i32, "cu_seqlens", dev), _dev_ptr(slot, i32, "slot", dev),
        _dev_ptr(fresh, torch.uint8, "fresh", dev), _dev_ptr(x, f32, "x", dev),
        _dev_ptr(dt, f32, "dt", dev), _dev_ptr(A, f32, "A", dev), _dev_ptr(B, f32, "B", dev),
        _dev_ptr(C, f32, "C", dev), _dev_ptr(state, f32, "state", dev), n_slots,
        _dev_ptr(y, f32, "y", dev), _stream_handle(stream, dev))
    _check(rc, "ssm_scan_prefill_static")
    return y


def decode(x, dt, A, B, C, state, slot, fresh, y=None, stream=None, dt_bias=None,
           dt_softplus=False, A_per_state=False, snapshots=None):
    """One token per sequence on the GPU (``ssm_scan_decode``, or
    ``ssm_scan_decode_opt`` with options).

    x [S, H, P], dt [S, H], A [H] (or [H, N]), B and C [S, G, N]; state as for
    prefill; slot [S] int32, fresh [S] uint8; snapshots [S, H, P, N].
    Returns y [S, H, P].
    """
    import torch
    n_slots, H, P, N = (int(v) for v in state.shape)
    S = int(slot.shape[0])
    G = int(B.shape[1])
    a_shape = (H, N) if A_per_state else (H,)
    if tuple(x.shape) != (S, H, P) or tuple(dt.shape) != (S, H) or tuple(A.shape) != a_shape:
        raise ValueError("x, dt or A has the wrong shape")
    if tuple(B.shape) != (S, G, N) or tuple(C.shape) != (S, G, N):
        raise ValueError("B or C has the wrong shape")
    if tuple(fresh.shape) != (S,):
        raise ValueError("fresh has the wrong shape")
    dev = state.device
    if y is None:
        y = torch.empty((S, H, P), dtype=torch.float32, device=dev)
    elif tuple(y.shape) != (S, H, P):
        raise ValueError("y has the wrong shape")
    opts = _options(dev, S, H, P, N, dt_bias, dt_softplus, A_per_state, snapshots)
    f32 = torch.float32
    args = (_dev_ptr(slot, torch.int32, "slot", dev), _dev_ptr(fresh, torch.uint8, "fresh", dev),
            _dev_ptr(x, f32, "x", dev), _dev_ptr(dt, f32, "dt", dev), _dev_ptr(A, f32, "A", dev),
            _dev_ptr(B, f32, "B", dev), _dev_ptr(C, f32, "C", dev),
            _dev_ptr(state, f32, "state", dev), n_slots, _dev_ptr(y, f32, "y", dev),
            _stream_handle(stream, dev))
    if opts is None:
        rc = _lib.ssm_scan_decode(ctypes.byref(Dims(H, P, N, G)), S, *args)
        _check(rc, "ssm_scan_decode")
    else:
        rc = _lib.ssm_scan_decode_opt(ctypes.byref(Dims(H, P, N, G)), ctypes.byref(opts), S, *args)
        _check(rc, "ssm_scan_decode_opt")
    return y


# ------------------------------------------------------------ beside the scan
def conv1d_silu(x, weight, conv_state, cu_seqlens, slot, fresh, out=None, snapshots=None,
                stream=None):
    """Causal depthwise conv1d + SiLU over a packed batch
    (``ssm_conv1d_silu_prefill``).

    x [T, D], weight [D, K] (K <= 4), conv_state [n_slots, D, K-1] fp32
    (updated in place); cu_seqlens [n_seqs+1] and slot [n_seqs] int32, fresh
    [n_seqs] uint8; ``snapshots`` [T, D, K-1] fp32 receives the history after
    every token.  Returns out [T, D] (``out`` if given)."""
    import torch
    T, D = (int(v) for v in x.shape)
    K = int(weight.shape[1])
    n_slots = int(conv_state.shape[0])
    n_seqs = int(slot.shape[0])
    if tuple(weight.shape) != (D, K) or tuple(conv_state.shape) != (n_slots, D, K - 1):
        raise ValueError("weight or conv_state has the wrong shape")
    if tuple(cu_seqlens.shape) != (n_seqs + 1,) or tuple(fresh.shape) != (n_seqs,):
        raise ValueError("cu_seqlens or fresh has the wrong shape")
    if snapshots is not None and tuple(snapshots.shape) != (T, D, K - 1):
        raise ValueError("snapshots must have shape [T, D, K-1]")
    dev = x.device
    if out is None:
        out = torch.empty((T, D), dtype=torch.float32, device=dev)
    elif tuple(out.shape) != (T, D):
        raise ValueError("out has the wrong shape")
    f32 = torch.float32
    rc = _lib.ssm_conv1d_silu_prefill(
        ctypes.byref(ConvDims(D, K)), n_seqs, T, _dev_ptr(cu_seqlens, torch.int32, "cu_seqlens", dev),
        _dev_ptr(slot, torch.int32, "slot", dev), _dev_ptr(fresh, torch.uint8, "fresh", dev),
        _dev_ptr(x, f32, "x", dev), _dev_ptr(weight, f32, "weight", dev),
        _dev_ptr(conv_state, f32, "conv_state", dev), n_slots, _dev_ptr(out, f32, "out", dev),
        _dev_ptr(snapshots, f32, "snapshots", dev), _stream_handle(stream, dev))
    _check(rc, "ssm_conv1d_silu_prefill")
    return out


def conv1d_silu_decode(x, weight, conv_state, slot, fresh, out=None, stream=None):
    """One token per sequence (``ssm_conv1d_silu_decode``): x [S, D], the rest
    as for ``conv1d_silu``.  Returns out [S, D]."""
    import torch
    S, D = (int(v) for v in x.shape)
    K = int(weight.shape[1])
    n_slots = int(conv_state.shape[0])
    if tuple(weight.shape) != (D, K) or tuple(conv_state.shape) != (n_slots, D, K - 1):
        raise ValueError("weight or conv_state has the wrong shape")
    if tuple(slot.shape) != (S,) or tuple(fresh.shape) != (S,):
        raise ValueError("slot or fresh has the wrong shape")
    dev = x.device
    if out is None:
        out = torch.empty((S, D), dtype=torch.float32, device=dev)
    elif tuple(out.shape) != (S, D):
        raise ValueError("out has the wrong shape")
    f32 = torch.float32
    rc = _lib.ssm_conv1d_silu_decode(
        ctypes.byref(ConvDims(D, K)), S, _dev_ptr(slot, torch.int32, "slot", dev),
        _dev_ptr(fresh, torch.uint8, "fresh", dev), _dev_ptr(x, f32, "x", dev),
        _dev_ptr(weight, f32, "weight", dev), _dev_ptr(conv_state, f32, "conv_state", dev),
        n_slots, _dev_ptr(out, f32, "out", dev), _stream_handle(stream, dev))
    _check(rc, "ssm_conv1d_silu_decode")
    return out


def gated_rmsnorm(y, z, weight, eps, out=None, stream=None):
    """Gated RMSNorm over the last axis (``ssm_gated_rmsnorm``): y, z [..., L]
    fp32, weight [L] shared by every row.  Returns out shaped like y."""
    import torch
    L = int(weight.shape[0])
    if tuple(z.shape) != tuple(y.shape) or int(y.shape[-1]) != L or weight.dim() != 1:
        raise ValueError("y, z and weight shapes disagree")
    dev = y.device
    if out is None:
        out = torch.empty(y.shape, dtype=torch.float32, device=dev)
    elif tuple(out.shape) != tuple(y.shape):
        raise ValueError("out has the wrong shape")
    f32 = torch.float32
    rc = _lib.ssm_gated_rmsnorm(y.numel() // L, L, _dev_ptr(y, f32, "y", dev),
                                _dev_ptr(z, f32, "z", dev), _dev_ptr(weight, f32, "weight", dev),
                                float(eps), _dev_ptr(out, f32, "out", dev),
                                _stream_handle(stream, dev))
    _check(rc, "ssm_gated_rmsnorm")
    return out


# ------------------------------------------------------------ gated delta rule
def _gdn_args(q, k, v, g, beta, state, y, snapshots, T):
    import torch
    n_slots, Hv, Dv, Dk = (int(d) for d in state.shape)
    Hk = int(k.shape[1])
    if tuple(q.shape) != (T, Hk, Dk) or tuple(k.shape) != (T, Hk, Dk):
        raise ValueError("q and k must have shape [T, Hk, Dk]")
    if tuple(v.shape) != (T, Hv, Dv) or tuple(g.shape) != (T, Hv) or tuple(beta.shape) != (T, Hv):
        raise ValueError("v, g or beta has the wrong shape")
    if snapshots is not None and tuple(snapshots.shape) != (T, Hv, Dv, Dk):
        raise ValueError("snapshots must have shape [T, Hv, Dv, Dk]")
    dev = state.device
    if y is None:
        y = torch.empty((T, Hv, Dv), dtype=torch.float32, device=dev)
    elif tuple(y.shape) != (T, Hv, Dv):
        raise ValueError("y has the wrong shape")
    f32 = torch.float32
    ptrs = [_dev_ptr(t, f32, n, dev) for t, n in ((q, "q"), (k, "k"), (v, "v"), (g, "g"),
                                                   (beta, "beta"))]
    return GdnDims(Hv, Hk, Dk, Dv), n_slots, dev, y, ptrs


def gdn_prefill(q, k, v, g, beta, state, cu_seqlens, slot, fresh, scale=None, y=None,
                snapshots=None, stream=None):
    """Gated delta-rule recurrence over a packed batch (``ssm_gdn_prefill``).

    q, k [T, Hk, Dk]; v [T, Hv, Dv]; g (log decay) and beta [T, Hv]; state
    [n_slots, Hv, Dv, Dk] fp32, updated in place; cu_seqlens [n_seqs+1] and
    slot [n_seqs] int32, fresh [n_seqs] uint8; ``scale`` defaults to
    1/sqrt(Dk); ``snapshots`` [T, Hv, Dv, Dk] receives the state after every
    token.  Returns y [T, Hv, Dv]."""
    import math
    import torch
    T = int(v.shape[0])
    n_seqs = int(slot.shape[0])
    dims, n_slots, dev, y, ptrs = _gdn_args(q, k, v, g, beta, state, y, snapshots, T)
    if tuple(cu_seqlens.shape) != (n_seqs + 1,) or tuple(fresh.shape) != (n_seqs,):
        raise ValueError("cu_seqlens or fresh has the wrong shape")
    sc = 1.0 / math.sqrt(dims.d_k) if scale is None else float(scale)
    rc = _lib.ssm_gdn_prefill(ctypes.byref(dims), n_seqs, T,
                              _dev_ptr(cu_seqlens, torch.int32, "cu_seqlens", dev),
                              _dev_ptr(slot, torch.int32, "slot", dev),
                              _dev_ptr(fresh, torch.uint8, "fresh", dev), *ptrs, sc,
                              _dev_ptr(state, torch.float32, "state", dev), n_slots,
                              _dev_ptr(y, torch.float32, "y", dev),
                              _dev_ptr(snapshots, torch.float32, "snapshots", dev),
                              _stream_handle(stream, dev))
    _check(rc, "ssm_gdn_prefill")
    return y


def gdn_workspace_size(Hv, Hk, Dk, Dv, n_seqs, max_seqlen) -> int:
    """Bytes of device workspace ``gdn_prefill_ws`` needs (0: it would run the
    per-token kernel)."""
    b = ctypes.c_size_t()
    _check(_lib.ssm_gdn_prefill_workspace_size(ctypes.byref(GdnDims(Hv, Hk, Dk, Dv)), int(n_seqs),
                                               int(max_seqlen), ctypes.byref(b)),
           "ssm_gdn_prefill_workspace_size")
    return int(b.value)


def gdn_prefill_ws(q, k, v, g, beta, state, cu_seqlens, slot, fresh, max_seqlen, scale=None,
                   y=None, workspace=None, stream=None):
    """``ssm_gdn_prefill_ws``: the recurrence with long sequences in chunked
    matrix form.  ``max_seqlen`` (host int) bounds every length;
    ``workspace`` (a uint8 CUDA tensor of at least ``gdn_workspace_size(...)``
    bytes) is allocated here when not given.  Otherwise as ``gdn_prefill``
    (no snapshots)."""
    import math
    import torch
    T = int(v.shape[0])
    n_seqs = int(slot.shape[0])
    dims, n_slots, dev, y, ptrs = _gdn_args(q, k, v, g, beta, state, y, None, T)
    if tuple(cu_seqlens.shape) != (n_seqs + 1,) or tuple(fresh.shape) != (n_seqs,):
        raise ValueError("cu_seqlens or fresh has the wrong shape")
    sc = 1.0 / math.sqrt(dims.d_k) if scale is None else float(scale)
    need = gdn_workspace_size(dims.n_v_heads, dims.n_k_heads, dims.d_k, dims.d_v, n_seqs,
                              max_seqlen)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if workspace.dtype != torch.uint8 or workspace.device != dev:
        raise ValueError("workspace must be a uint8 tensor on the device of the state")
    rc = _lib.ssm_gdn_prefill_ws(ctypes.byref(dims), n_seqs, T,
                                 _dev_ptr(cu_seqlens, torch.int32, "cu_seqlens", dev),
                                 _dev_ptr(slot, torch.int32, "slot", dev),
                                 _dev_ptr(fresh, torch.uint8, "fresh", dev), *ptrs, sc,
                                 _dev_ptr(state, torch.float32, "state", dev), n_slots,
                                 _dev_ptr(y, torch.float32, "y", dev), int(max_seqlen),
                                 ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                                 _stream_handle(stream, dev))
    _check(rc, "ssm_gdn_prefill_ws")
    return y


def gdn_decode(q, k, v, g, beta, state, slot, fresh, scale=None, y=None, snapshots=None,
               stream=None):
    """One token per sequence (``ssm_gdn_decode``): the token arrays are
    indexed by sequence; the rest as for ``gdn_prefill``."""
    import math
    import torch
    S = int(slot.shape[0])
    dims, n_slots, dev, y, ptrs = _gdn_args(q, k, v, g, beta, state, y, snapshots, S)
    if tuple(fresh.shape) != (S,):
        raise ValueError("fresh has the wrong shape")
    sc = 1.0 / math.sqrt(dims.d_k) if scale is None else float(scale)
    rc = _lib.ssm_gdn_decode(ctypes.byref(dims), S, _dev_ptr(slot, torch.int32, "slot", dev),
                             _dev_ptr(fresh, torch.uint8, "fresh", dev), *ptrs, sc,
                             _dev_ptr(state, torch.float32, "state", dev), n_slots,
                             _dev_ptr(y, torch.float32, "y", dev),
                             _dev_ptr(snapshots, torch.float32, "snapshots", dev),
                             _stream_handle(stream, dev))
    _check(rc, "ssm_gdn_decode")
    return y


def to_device(case, device="cuda:0"):
    """Copy an ``ssm_inputs.ScanCase``'s arrays to ``device`` as torch tensors."""
    import torch
    d = {}
    for f in ("x", "dt", "A", "B", "C", "state", "cu_seqlens", "slot", "fresh"):
        d[f] = torch.from_numpy(getattr(case, f)).to(device)
    return d
