"""Helpers shared by the GPU tests: run a case through the C ABI on cuda:0 and
compare with the oracle.  Every input comes from ssm_inputs (seeded); every
expected value from the oracle or from closed forms -- never from the GPU."""
from __future__ import annotations

import sys

import numpy as np

import ssm_inputs

TOL = 1e-4          # max |gpu - ref| / (1 + |ref|) on y and on the final state


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(a, ref):
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - ref) / (1.0 + np.abs(ref))))


def run_gpu(case, mode="prefill", device="cuda:0", offset_floats=0, max_seqlen=None,
            segments=0, workspace_bytes=None, dt_bias=None, dt_softplus=False,
            A_per_state=False, snapshots=False):
    """Run ``case`` on the GPU; returns (y, state) as numpy.  ``mode`` is
    "prefill" or "decode" (every length must be 1).  ``offset_floats`` > 0
    places every float array at that element offset inside a larger buffer,
    which breaks 16-byte alignment and forces the scalar path.  Mode
    "prefill_ws" calls ssm_scan_prefill_ws with ``max_seqlen`` (default: the
    longest length) and ``segments``; ``workspace_bytes`` overrides the
    workspace size the library asks for.  Options (``dt_bias`` numpy [H],
    ``dt_softplus``, ``A_per_state`` with case.A [H][N], ``snapshots``) go
    through the ``_opt`` entry points; with ``snapshots`` the result is
    (y, state, snapshots)."""
    import torch
    import mamba2_selective_scan_amd as ssm

    def put(arr):
        t = torch.from_numpy(np.ascontiguousarray(arr))
        if offset_floats and t.dtype == torch.float32:
            flat = torch.empty(t.numel() + offset_floats, dtype=t.dtype, device=device)
            view = flat[offset_floats:].view(t.shape)
            view.copy_(t.to(device))
            return view
        return t.to(device)

    x, dt, A, B, C = (put(getattr(case, f)) for f in ("x", "dt", "A", "B", "C"))
    state = put(case.state)
    slot = put(case.slot)
    fresh = put(case.fresh)
    y = put(np.zeros((case.n_tokens, case.H, case.P), np.float32))
    opts = dict(dt_bias=None if dt_bias is None else put(np.asarray(dt_bias, np.float32)),
                dt_softplus=dt_softplus, A_per_state=A_per_state,
                snapshots=put(np.full((case.n_tokens, case.H, case.P, case.N), np.nan, np.float32))
                if snapshots else None)
    if mode == "prefill":
        cu = put(case.cu_seqlens)
        ssm.prefill(x, dt, A, B, C, state, cu, slot, fresh, y=y, **opts)
    elif mode == "prefill_ws":
        cu = put(case.cu_seqlens)
        ms = int(case.lengths.max()) if max_seqlen is None and case.n_seqs else int(max_seqlen or 0)
        need = ssm.workspace_size(case.H, case.P, case.N, case.G, case.n_seqs, case.n_tokens,
                                  ms, segments)
        nbytes = need if workspace_bytes is None else workspace_bytes
        ws = torch.full((max(nbytes, 1),), 0xFF, dtype=torch.uint8, device=device)  # garbage
        ssm.prefill_ws(x, dt, A, B, C, state, cu, slot, fresh, ms, segments=segments,
                       workspace=ws[:nbytes] if nbytes else None, y=y, **opts)
    elif mode == "decode":
        assert np.all(case.lengths == 1)
        ssm.decode(x, dt, A, B, C, state, slot, fresh, y=y, **opts)
    else:
        raise ValueError(mode)
    torch.cuda.synchronize()
    if snapshots:
        return y.cpu().numpy(), state.cpu().numpy(), opts["snapshots"].cpu().numpy()
    return y.cpu().numpy(), state.cpu().numpy()


def assert_parity(case, y_gpu, st_gpu, y_ref, st_ref, tol=TOL, label=""):
    used = np.unique(case.slot)
    e_y = rel_err(y_gpu, y_ref)
    e_s = rel_err(st_gpu[used], st_ref[used]) if used.size else 0.0
    say(f"  {label or case.name}: max rel err y={e_y:.3e} state={e_s:.3e}")
    assert np.all(np.isfinite(y_gpu)), "non-finite y"
    assert e_y <= tol, f"y error {e_y} > {tol}"
    assert e_s <= tol, f"state error {e_s} > {tol}"
    unused = np.setdiff1d(np.arange(case.n_slots), used)
    for k in unused:
        assert np.array_equal(st_gpu[k], case.state[k], equal_nan=True), f"unused slot {k} changed"


def sub_case(case, seqs):
    """The sequences ``seqs`` of a packed case, repacked (same slots)."""
    parts = [(int(case.cu_seqlens[s]), int(case.cu_seqlens[s + 1])) for s in seqs]
    idx = np.concatenate([np.arange(a, b) for a, b in parts]) if parts else np.zeros(0, int)
    lengths = np.array([b - a for a, b in parts], np.int32)
    return ssm_inputs.ScanCase(H=case.H, P=case.P, N=case.N, G=case.G, lengths=lengths,
                               cu_seqlens=ssm_inputs.lengths_to_cu(lengths),
                               slot=case.slot[list(seqs)], fresh=case.fresh[list(seqs)],
                               x=case.x[idx], dt=case.dt[idx], A=case.A, B=case.B[idx],
                               C=case.C[idx], state=case.state, name=case.name + f"[{seqs}]")


def _put(arr, device, offset_floats=0):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(arr))
    if offset_floats and t.dtype == torch.float32:
        flat = torch.empty(t.numel() + offset_floats, dtype=t.dtype, device=device)
        view = flat[offset_floats:].view(t.shape)
        view.copy_(t.to(device))
        return view
    return t.to(device)


def run_conv_gpu(case, mode="prefill", device="cuda:0", offset_floats=0, snapshots=False):
    """Run an ``ssm_inputs.ConvCase`` through the conv1d + SiLU ABI; returns
    (out, state) or (out, state, snapshots) as numpy.  ``mode`` "prefill" or
    "decode" (every length 1); ``offset_floats`` > 0 breaks 16-byte alignment."""
    import torch
    import mamba2_selective_scan_amd as ssm
    put = lambda a: _put(a, device, offset_floats)
    x, w, st = put(case.x), put(case.w), put(case.state)
    slot, fresh = put(case.slot), put(case.fresh)
    out = put(np.full((case.n_tokens, case.D), np.nan, np.float32))
    snaps = (put(np.full((case.n_tokens, case.D, case.K - 1), np.nan, np.float32))
             if snapshots else None)
    if mode == "prefill":
        ssm.conv1d_silu(x, w, st, put(case.cu_seqlens), slot, fresh, out=out, snapshots=snaps)
    elif mode == "decode":
        assert np.all(case.lengths == 1) and not snapshots
        ssm.conv1d_silu_decode(x, w, st, slot, fresh, out=out)
    else:
        raise ValueError(mode)
    torch.cuda.synchronize()
    res = (out.cpu().numpy(), st.cpu().numpy())
    return res + (snaps.cpu().numpy(),) if snapshots else res


def assert_conv_parity(case, out_gpu, st_gpu, out_ref, st_ref, tol=TOL, label=""):
    """out within ``tol``; the history holds raw inputs, so it must match
    bitwise; slots no sequence names come back unchanged."""
    used = np.unique(case.slot)
    e = rel_err(out_gpu, out_ref)
    say(f"  {label or case.name}: max rel err out={e:.3e}")
    assert np.all(np.isfinite(out_gpu)), "non-finite output"
    assert e <= tol, f"output error {e} > {tol}"
    assert np.array_equal(st_gpu[used], st_ref[used]), "history differs"
    for k in np.setdiff1d(np.arange(case.n_slots), used):
        assert np.array_equal(st_gpu[k], case.state[k], equal_nan=True), f"unused slot {k} changed"


def run_norm_gpu(case, device="cuda:0", offset_floats=0, eps=None):
    import torch
    import mamba2_selective_scan_amd as ssm
    put = lambda a: _put(a, device, offset_floats)
    y, z, w = put(case.y), put(case.z), put(case.w)
    out = put(np.full(case.y.shape, np.nan, np.float32))
    ssm.gated_rmsnorm(y, z, w, case.eps if eps is None else eps, out=out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def run_gdn_gpu(case, mode="prefill", device="cuda:0", offset_floats=0, snapshots=False,
                max_seqlen=None):
    """Run an ``ssm_inputs.GdnCase`` through the delta-rule ABI; returns (y,
    state) or (y, state, snapshots) as numpy."""
    import torch
    import mamba2_selective_scan_amd as ssm
    put = lambda a: _put(a, device, offset_floats)
    q, k, v, g, beta = (put(getattr(case, f)) for f in ("q", "k", "v", "g", "beta"))
    st = put(case.state)
    slot, fresh = put(case.slot), put(case.fresh)
    y = put(np.full((case.n_tokens, case.Hv, case.Dv), np.nan, np.float32))
    sn = (put(np.full((case.n_tokens, case.Hv, case.Dv, case.Dk), np.nan, np.float32))
          if snapshots else None)
    if mode == "prefill":
        ssm.gdn_prefill(q, k, v, g, beta, st, put(case.cu_seqlens), slot, fresh, scale=case.scale,
                        y=y, snapshots=sn)
    elif mode == "prefill_ws":
        assert not snapshots
        ms = int(case.lengths.max()) if max_seqlen is None and case.n_seqs else int(max_seqlen or 0)
        ssm.gdn_prefill_ws(q, k, v, g, beta, st, put(case.cu_seqlens), slot, fresh, ms,
                           scale=case.scale, y=y)
    elif mode == "decode":
        assert np.all(case.lengths == 1)
        ssm.gdn_decode(q, k, v, g, beta, st, slot, fresh, scale=case.scale, y=y, snapshots=sn)
    else:
        raise ValueError(mode)
    torch.cuda.synchronize()
    res = (y.cpu().numpy(), st.cpu().numpy())
    return res + (sn.cpu().numpy(),) if snapshots else res
