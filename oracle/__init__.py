"""CPU oracle for the Mamba2 selective-state scan, its neighbouring steps
(causal conv1d + SiLU, gated RMSNorm) and the gated delta-rule recurrence --
TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The GPU library never calls it and shares no code
with it.  The arithmetic lives in ``ssm_oracle.c`` (plain sequential C, built
by ``oracle/build.py``); this module only marshals numpy arrays.

Every function here is pinned by ``tests/test_oracle_pins.py`` against things
other than itself: a brute-force unrolled closed form, hand-worked fixtures,
prefix sums, T=1 dot products, decay-only powers and invariants.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_LIB = os.path.join(HERE, "libssm_oracle.so")

_i32p = ctypes.POINTER(ctypes.c_int32)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)


def default_threads() -> int:
    """Host threads the oracle uses when not told: the CPUs this process may
    run on, capped by OMP_NUM_THREADS when that is set (a shared host's share
    can be far below what os.cpu_count() reports)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def _ptr(a: np.ndarray, t):
    return a.ctypes.data_as(t)


class Oracle:
    """Binds one build of the oracle library (the default one, or a test build)."""

    def __init__(self, path: str = DEFAULT_LIB):
        if not os.path.exists(path):
            raise FileNotFoundError(
                f"{path} is missing: build it with `python oracle/build.py`")
        self.path = path
        self.lib = ctypes.CDLL(path)
        common = [ctypes.c_int32] * 5 + [_i32p, _i32p, _u8p] + [_f32p] * 5
        opts = [_f32p, ctypes.c_int32, ctypes.c_int32]
        self.lib.ssm_oracle_scan_opt_f32.argtypes = (common + [_f32p, _f32p, ctypes.c_int32]
                                                     + opts + [_f32p])
        self.lib.ssm_oracle_scan_opt_f32.restype = ctypes.c_int
        self.lib.ssm_oracle_scan_opt_f64.argtypes = (common + [_f64p, _f64p, ctypes.c_int32]
                                                     + opts + [_f64p])
        self.lib.ssm_oracle_scan_opt_f64.restype = ctypes.c_int
        meta = [ctypes.c_int32] * 3 + [_i32p, _i32p, _u8p, _f32p, _f32p]
        self.lib.ssm_oracle_conv1d_silu_f32.argtypes = meta + [_f32p] * 3 + [ctypes.c_int32]
        self.lib.ssm_oracle_conv1d_silu_f32.restype = ctypes.c_int
        self.lib.ssm_oracle_conv1d_silu_f64.argtypes = meta + [_f64p] * 3 + [ctypes.c_int32]
        self.lib.ssm_oracle_conv1d_silu_f64.restype = ctypes.c_int
        norm = [ctypes.c_int64, ctypes.c_int32, _f32p, _f32p, _f32p]
        self.lib.ssm_oracle_gated_rmsnorm_f32.argtypes = norm + [ctypes.c_float, _f32p,
                                                                 ctypes.c_int32]
        self.lib.ssm_oracle_gated_rmsnorm_f32.restype = ctypes.c_int
        self.lib.ssm_oracle_gated_rmsnorm_f64.argtypes = norm + [ctypes.c_double, _f64p,
                                                                 ctypes.c_int32]
        self.lib.ssm_oracle_gated_rmsnorm_f64.restype = ctypes.c_int
        gdn = [ctypes.c_int32] * 5 + [_i32p, _i32p, _u8p] + [_f32p] * 5
        self.lib.ssm_oracle_gdn_f32.argtypes = gdn + [ctypes.c_float] + [_f32p] * 3 + [ctypes.c_int32]
        self.lib.ssm_oracle_gdn_f32.restype = ctypes.c_int
        self.lib.ssm_oracle_gdn_f64.argtypes = gdn + [ctypes.c_double] + [_f64p] * 3 + [ctypes.c_int32]
        self.lib.ssm_oracle_gdn_f64.restype = ctypes.c_int

    def scan(self, H, P, N, G, cu_seqlens, slot, fresh, x, dt, A, B, C, state,
             precision="f32", threads=None, dt_bias=None, dt_softplus=False,
             A_per_state=False, snapshots=False):
        """Run the scan on a packed batch.

        Returns ``(y, state_out)``, or ``(y, state_out, snapshots)`` with
        ``snapshots=True``; the input ``state`` is not modified.  precision
        "f32": fp32 arithmetic; "f64": double arithmetic on the same fp32
        inputs (outputs are float64 then).  Options: ``dt_bias`` [H] is added
        to dt, ``dt_softplus`` applies softplus (identity above 20),
        ``A_per_state`` takes A as [H][N], ``snapshots`` returns the state
        after every token, [T][H][P][N].
        """
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        slot = np.ascontiguousarray(slot, dtype=np.int32)
        fresh = np.ascontiguousarray(fresh, dtype=np.uint8)
        x = np.ascontiguousarray(x, dtype=np.float32)
        dt = np.ascontiguousarray(dt, dtype=np.float32)
        A = np.ascontiguousarray(A, dtype=np.float32)
        B = np.ascontiguousarray(B, dtype=np.float32)
        C = np.ascontiguousarray(C, dtype=np.float32)
        n_seqs = slot.shape[0]
        T = int(cu[-1]) if cu.shape[0] else 0
        assert cu.shape[0] == n_seqs + 1
        assert x.shape == (T, H, P) and dt.shape == (T, H)
        assert A.shape == ((H, N) if A_per_state else (H,))
        assert B.shape == (T, G, N) and C.shape == (T, G, N)
        assert state.ndim == 4 and state.shape[1:] == (H, P, N)
        bias = None
        if dt_bias is not None:
            bias = np.ascontiguousarray(dt_bias, dtype=np.float32)
            assert bias.shape == (H,)
        if threads is None:
            threads = default_threads()
        if precision == "f32":
            dtype, fn, fp = np.float32, self.lib.ssm_oracle_scan_opt_f32, _f32p
        elif precision == "f64":
            dtype, fn, fp = np.float64, self.lib.ssm_oracle_scan_opt_f64, _f64p
        else:
            raise ValueError(precision)
        st = np.array(state, dtype=dtype, copy=True, order="C")
        y = np.zeros((T, H, P), dtype=dtype)
        snaps = np.zeros((T, H, P, N), dtype=dtype) if snapshots else None
        rc = fn(H, P, N, G, n_seqs, _ptr(cu, _i32p), _ptr(slot, _i32p),
                _ptr(fresh, _u8p), _ptr(x, _f32p), _ptr(dt, _f32p), _ptr(A, _f32p),
                _ptr(B, _f32p), _ptr(C, _f32p), _ptr(st, fp), _ptr(y, fp), int(threads),
                None if bias is None else _ptr(bias, _f32p), int(bool(dt_softplus)),
                int(bool(A_per_state)), None if snaps is None else _ptr(snaps, fp))
        if rc != 0:
            raise ValueError(f"oracle rejected the dimensions (rc={rc})")
        return (y, st, snaps) if snapshots else (y, st)

    def scan_case(self, case, precision="f32", threads=None, **options):
        """``scan`` on an ``ssm_inputs.ScanCase`` (options as for ``scan``)."""
        return self.scan(case.H, case.P, case.N, case.G, case.cu_seqlens, case.slot,
                         case.fresh, case.x, case.dt, case.A, case.B, case.C,
                         case.state, precision=precision, threads=threads, **options)

    # ------------------------------------------------------------ neighbours
    def conv1d_silu(self, K, cu_seqlens, slot, fresh, x, w, conv_state, precision="f32",
                    threads=None, snapshots=False):
        """Causal depthwise conv1d + SiLU with a rolling history over a packed
        batch.  x [T][D], w [D][K], conv_state [n_slots][D][K-1] (not
        modified).  Returns ``(out, conv_state_out)``, or ``(out, state_out,
        snapshots)`` with ``snapshots=True`` ([T][D][K-1], the history after
        each token)."""
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        slot = np.ascontiguousarray(slot, dtype=np.int32)
        fresh = np.ascontiguousarray(fresh, dtype=np.uint8)
        x = np.ascontiguousarray(x, dtype=np.float32)
        w = np.ascontiguousarray(w, dtype=np.float32)
        n_seqs = slot.shape[0]
        T = int(cu[-1]) if cu.shape[0] else 0
        D = w.shape[0]
        assert cu.shape[0] == n_seqs + 1 and w.shape == (D, K) and x.shape == (T, D)
        assert conv_state.ndim == 3 and conv_state.shape[1:] == (D, K - 1)
        if threads is None:
            threads = default_threads()
        if precision == "f32":
            dtype, fn, fp = np.float32, self.lib.ssm_oracle_conv1d_silu_f32, _f32p
        elif precision == "f64":
            dtype, fn, fp = np.float64, self.lib.ssm_oracle_conv1d_silu_f64, _f64p
        else:
            raise ValueError(precision)
        st = np.array(conv_state, dtype=dtype, copy=True, order="C")
        out = np.zeros((T, D), dtype=dtype)
        snaps = np.zeros((T, D, K - 1), dtype=dtype) if snapshots else None
        rc = fn(D, K, n_seqs, _ptr(cu, _i32p), _ptr(slot, _i32p), _ptr(fresh, _u8p),
                _ptr(x, _f32p), _ptr(w, _f32p), _ptr(st, fp), _ptr(out, fp),
                None if snaps is None else _ptr(snaps, fp), int(threads))
        if rc != 0:
            raise ValueError(f"oracle rejected the dimensions (rc={rc})")
        return (out, st, snaps) if snapshots else (out, st)

    def conv_case(self, case, precision="f32", threads=None, snapshots=False):
        """``conv1d_silu`` on an ``ssm_inputs.ConvCase``."""
        return self.conv1d_silu(case.K, case.cu_seqlens, case.slot, case.fresh, case.x,
                                case.w, case.state, precision=precision, threads=threads,
                                snapshots=snapshots)

    def gated_rmsnorm(self, y, z, w, eps, precision="f32", threads=None):
        """Gated RMSNorm over the last axis: y, z [..., L], w [L]."""
        y = np.ascontiguousarray(y, dtype=np.float32)
        z = np.ascontiguousarray(z, dtype=np.float32)
        w = np.ascontiguousarray(w, dtype=np.float32)
        L = w.shape[0]
        assert y.shape == z.shape and y.shape[-1] == L
        n_rows = y.size // L
        if threads is None:
            threads = default_threads()
        if precision == "f32":
            out = np.zeros(y.shape, dtype=np.float32)
            rc = self.lib.ssm_oracle_gated_rmsnorm_f32(n_rows, L, _ptr(y, _f32p), _ptr(z, _f32p),
                                                       _ptr(w, _f32p), float(eps),
                                                       _ptr(out, _f32p), int(threads))
        elif precision == "f64":
            out = np.zeros(y.shape, dtype=np.float64)
            rc = self.lib.ssm_oracle_gated_rmsnorm_f64(n_rows, L, _ptr(y, _f32p), _ptr(z, _f32p),
                                                       _ptr(w, _f32p), float(eps),
                                                       _ptr(out, _f64p), int(threads))
        else:
            raise ValueError(precision)
        if rc != 0:
            raise ValueError(f"oracle rejected the dimensions (rc={rc})")
        return out

    def norm_case(self, case, precision="f32", threads=None):
        """``gated_rmsnorm`` on an ``ssm_inputs.NormCase``."""
        return self.gated_rmsnorm(case.y, case.z, case.w, case.eps, precision=precision,
                                  threads=threads)

    # ------------------------------------------------------------ delta rule
    def gdn(self, Hv, Hk, Dk, Dv, cu_seqlens, slot, fresh, q, k, v, g, beta, scale, state,
            precision="f32", threads=None, snapshots=False):
        """Gated delta-rule recurrence over a packed batch.  q, k [T][Hk][Dk],
        v [T][Hv][Dv], g and beta [T][Hv], state [n_slots][Hv][Dv][Dk] (not
        modified).  Returns ``(y, state_out)`` or ``(y, state_out, snapshots)``."""
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        slot = np.ascontiguousarray(slot, dtype=np.int32)
        fresh = np.ascontiguousarray(fresh, dtype=np.uint8)
        q, k, v, g, beta = (np.ascontiguousarray(a, dtype=np.float32) for a in (q, k, v, g, beta))
        n_seqs = slot.shape[0]
        T = int(cu[-1]) if cu.shape[0] else 0
        assert cu.shape[0] == n_seqs + 1
        assert q.shape == (T, Hk, Dk) and k.shape == (T, Hk, Dk) and v.shape == (T, Hv, Dv)
        assert g.shape == (T, Hv) and beta.shape == (T, Hv)
        assert state.ndim == 4 and state.shape[1:] == (Hv, Dv, Dk)
        if threads is None:
            threads = default_threads()
        if precision == "f32":
            dtype, fn, fp = np.float32, self.lib.ssm_oracle_gdn_f32, _f32p
        elif precision == "f64":
            dtype, fn, fp = np.float64, self.lib.ssm_oracle_gdn_f64, _f64p
        else:
            raise ValueError(precision)
        st = np.array(state, dtype=dtype, copy=True, order="C")
        y = np.zeros((T, Hv, Dv), dtype=dtype)
        snaps = np.zeros((T, Hv, Dv, Dk), dtype=dtype) if snapshots else None
        rc = fn(Hv, Hk, Dk, Dv, n_seqs, _ptr(cu, _i32p), _ptr(slot, _i32p), _ptr(fresh, _u8p),
                _ptr(q, _f32p), _ptr(k, _f32p), _ptr(v, _f32p), _ptr(g, _f32p),
                _ptr(beta, _f32p), float(scale), _ptr(st, fp), _ptr(y, fp),
                None if snaps is None else _ptr(snaps, fp), int(threads))
        if rc != 0:
            raise ValueError(f"oracle rejected the dimensions (rc={rc})")
        return (y, st, snaps) if snapshots else (y, st)

    def gdn_case(self, case, precision="f32", threads=None, snapshots=False):
        """``gdn`` on an ``ssm_inputs.GdnCase``."""
        return self.gdn(case.Hv, case.Hk, case.Dk, case.Dv, case.cu_seqlens, case.slot,
                        case.fresh, case.q, case.k, case.v, case.g, case.beta, case.scale,
                        case.state, precision=precision, threads=threads, snapshots=snapshots)


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def scan(*args, **kw):
    return default().scan(*args, **kw)


def scan_case(case, **kw):
    return default().scan_case(case, **kw)
