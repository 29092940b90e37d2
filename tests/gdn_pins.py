"""Pins for the oracle's gated delta-rule recurrence.  Each takes an
``oracle.Oracle`` and raises AssertionError when the oracle disagrees with
something fixed independently of its C loops: the matrix form of the update
M <- alpha M (I - beta k k^T) + beta v k^T computed with numpy in float64, the
delta rule's defining property (with beta = 1 and unit keys a write replaces
the value stored under that key exactly), pure decay, the one-token closed
form, and invariants that hold bitwise (split runs, batch composition, GQA
against explicitly repeated keys, thread count)."""
from __future__ import annotations

import math

import numpy as np

import ssm_inputs


def rel_err(a, ref):
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - ref) / (1.0 + np.abs(ref))))


def small_gdn_case(seed, Hv=4, Hk=2, Dk=5, Dv=3, lengths=(5, 1, 0, 8, 3),
                   fresh=(1, 0, 1, 0, 0)):
    n = len(lengths)
    slots = np.random.Generator(np.random.PCG64(seed + 9)).permutation(n + 2)[:n]
    return ssm_inputs.make_gdn_case(Hv, Hk, Dk, Dv, list(lengths), list(fresh), seed,
                                    slots=slots.astype(np.int32), n_slots=n + 2,
                                    sentinel_unused=True, name="gdn_small")


def matrix_form(case):
    """y and final states in float64 from the matrix form: per (sequence, value
    head) M[j][i] (value j, key i) evolves as M <- alpha M (I - beta k k^T) +
    beta v k^T, and y = scale M q; the key head of value head vh is vh % Hk."""
    y = np.zeros((case.n_tokens, case.Hv, case.Dv))
    st = case.state.astype(np.float64).copy()
    eye = np.eye(case.Dk)
    for s in range(case.n_seqs):
        for vh in range(case.Hv):
            kh = vh % case.Hk
            M = np.zeros((case.Dv, case.Dk)) if case.fresh[s] else st[case.slot[s], vh].copy()
            for t in range(int(case.cu_seqlens[s]), int(case.cu_seqlens[s + 1])):
                k = case.k[t, kh].astype(np.float64)
                q = case.q[t, kh].astype(np.float64)
                b = float(case.beta[t, vh])
                alpha = math.exp(float(case.g[t, vh]))
                M = alpha * M @ (eye - b * np.outer(k, k)) + b * np.outer(case.v[t, vh], k)
                y[t, vh] = case.scale * (M @ q)
            st[case.slot[s], vh] = M
    return y, st


def pin_gdn_matrix_form(orc):
    for seed, shape in ((1, {}), (2, dict(Hv=6, Hk=3, Dk=7, Dv=4)), (3, dict(Hv=2, Hk=2, Dk=1, Dv=5))):
        case = small_gdn_case(seed, **shape)
        y_ref, st_ref = matrix_form(case)
        used = np.unique(case.slot)
        y64, st64 = orc.gdn_case(case, precision="f64", threads=2)
        assert rel_err(y64, y_ref) <= 1e-12 and rel_err(st64[used], st_ref[used]) <= 1e-12, seed
        y32, st32 = orc.gdn_case(case, precision="f32", threads=2)
        assert rel_err(y32, y_ref) <= 1e-5 and rel_err(st32[used], st_ref[used]) <= 1e-5, seed


def pin_gdn_matrix_form_general_keys(orc):
    """Keys and queries of any length (rows rescaled to norms in [0.25, 1.4])
    and write strengths 0, 1/2, 1 and drawn: the oracle still follows the
    matrix form.  The recurrence takes q and k as given, so nothing in it may
    assume unit rows (a kernel that dropped k.k or normalised would fail)."""
    for seed, beta in ((21, None), (22, 0.0), (23, 0.5), (24, 1.0)):
        n = 5
        slots = np.random.Generator(np.random.PCG64(seed + 9)).permutation(n + 2)[:n]
        case = ssm_inputs.make_gdn_case(4, 2, 6, 3, [5, 1, 0, 8, 3], [1, 0, 1, 0, 0], seed,
                                        slots=slots.astype(np.int32), n_slots=n + 2,
                                        sentinel_unused=True, qk_norm=(0.25, 1.4), beta=beta)
        norms = np.linalg.norm(case.k.astype(np.float64), axis=-1)
        assert norms.min() < 0.6 and norms.max() > 1.1, "rows must not be unit length"
        y_ref, st_ref = matrix_form(case)
        used = np.unique(case.slot)
        y64, st64 = orc.gdn_case(case, precision="f64", threads=2)
        assert rel_err(y64, y_ref) <= 1e-12 and rel_err(st64[used], st_ref[used]) <= 1e-12, seed
        y32, st32 = orc.gdn_case(case, precision="f32", threads=2)
        assert rel_err(y32, y_ref) <= 1e-5 and rel_err(st32[used], st_ref[used]) <= 1e-5, seed


def pin_gdn_key_length_overwrite(orc):
    """beta = 1 and a key of length c along e_m: the write leaves the stored
    column at (1 - c^2) times its old value plus c times v (the matrix form
    with k k^T = c^2 e_m e_m^T), exactly for c = 2 and small integers."""
    Dk, Dv, m, c = 4, 3, 2, 2.0
    state0 = np.arange(1, Dv * Dk + 1, dtype=np.float32).reshape(1, 1, Dv, Dk)
    k = np.zeros((1, 1, Dk), np.float32)
    k[0, 0, m] = c
    q = np.zeros((1, 1, Dk), np.float32)
    q[0, 0, m] = 1.0
    v = np.array([[[3.0, -1.0, 5.0]]], np.float32)
    y, st = orc.gdn(1, 1, Dk, Dv, [0, 1], [0], [0], q, k, v, np.zeros((1, 1), np.float32),
                    np.ones((1, 1), np.float32), 1.0, state0, precision="f32", threads=1)
    want = state0[0, 0].copy()
    want[:, m] = (1.0 - c * c) * state0[0, 0, :, m] + c * v[0, 0]
    assert np.array_equal(st[0, 0], want)
    assert np.array_equal(y[0, 0], want[:, m])


def pin_gdn_tiny_workload_matrix_form(orc):
    case = ssm_inputs.gdn_workload("tiny")
    y_ref, st_ref = matrix_form(case)
    y32, st32 = orc.gdn_case(case)
    assert rel_err(y32, y_ref) <= 1e-5 and rel_err(st32[0], st_ref[0]) <= 1e-5


def _one_hot_case(Dk, Dv, writes, state0, scale=0.5):
    """One sequence, one head, no decay (g = 0), beta = 1: token t writes
    value writes[t][1] under key e_{writes[t][0]} and queries key
    e_{writes[t][2]}."""
    T = len(writes)
    k = np.zeros((T, 1, Dk), np.float32)
    q = np.zeros((T, 1, Dk), np.float32)
    v = np.zeros((T, 1, Dv), np.float32)
    for t, (m, val, mq) in enumerate(writes):
        k[t, 0, m] = 1.0
        q[t, 0, mq] = 1.0
        v[t, 0] = val
    return ssm_inputs.GdnCase(Hv=1, Hk=1, Dk=Dk, Dv=Dv, lengths=np.array([T], np.int32),
                              cu_seqlens=np.array([0, T], np.int32),
                              slot=np.array([0], np.int32), fresh=np.array([0], np.uint8),
                              q=q, k=k, v=v, g=np.zeros((T, 1), np.float32),
                              beta=np.ones((T, 1), np.float32),
                              state=state0.astype(np.float32)[None, None], scale=scale)


def pin_gdn_overwrite(orc):
    """With beta = 1, no decay and a unit key e_m, the rank-1 write makes
    column m of the state equal to v (the value stored under key m is
    replaced), other columns are untouched, and a query e_m reads scale * v.
    Small integers keep every step exact, so the check is bitwise."""
    Dk, Dv = 5, 3
    M0 = np.arange(Dv * Dk, dtype=np.float64).reshape(Dv, Dk) - 7.0
    writes = [(1, [3.0, -2.0, 5.0], 1), (3, [1.0, 1.0, -4.0], 1), (1, [-6.0, 0.0, 2.0], 3),
              (4, [9.0, -9.0, 8.0], 0)]
    case = _one_hot_case(Dk, Dv, writes, M0)
    M = M0.copy()
    y_ref = np.zeros((len(writes), 1, Dv))
    for t, (m, val, mq) in enumerate(writes):
        M[:, m] = val
        y_ref[t, 0] = 0.5 * M[:, mq]
    for precision in ("f32", "f64"):
        y, st = orc.gdn_case(case, precision=precision, threads=1)
        assert np.array_equal(st[0, 0], M), precision
        assert np.array_equal(y, y_ref), precision


def pin_gdn_pure_decay(orc):
    """beta = 0: nothing is written, the state only decays:
    M_t = exp(g_1 + ... + g_t) M_0 and y_t = scale * M_t q_t."""
    case = small_gdn_case(11, lengths=(6,), fresh=(0,))
    case.beta[:] = 0.0
    y, st = orc.gdn_case(case, precision="f64", threads=1)
    y32, st32 = orc.gdn_case(case, precision="f32", threads=1)
    s0 = case.state[case.slot[0]].astype(np.float64)
    for t in range(6):
        for vh in range(case.Hv):
            a = math.exp(float(np.sum(case.g[:t + 1, vh].astype(np.float64))))
            ref = case.scale * a * (s0[vh] @ case.q[t, vh % case.Hk].astype(np.float64))
            assert rel_err(y[t, vh], ref) <= 1e-12 and rel_err(y32[t, vh], ref) <= 1e-6, (t, vh)
    for vh in range(case.Hv):
        a = math.exp(float(np.sum(case.g[:, vh].astype(np.float64))))
        assert rel_err(st[case.slot[0], vh], a * s0[vh]) <= 1e-12


def pin_gdn_single_token(orc):
    """One token from zero: the state becomes beta * v k^T and
    y = scale * beta * (k . q) * v (the dot with math.fsum)."""
    case = small_gdn_case(12, Hv=3, Hk=1, Dk=9, Dv=4, lengths=(1, 1), fresh=(1, 1))
    y, st = orc.gdn_case(case, precision="f64", threads=1)
    for s in range(2):
        t = int(case.cu_seqlens[s])
        k = case.k[t, 0].astype(np.float64)
        q = case.q[t, 0].astype(np.float64)
        kq = math.fsum(k * q)
        for vh in range(3):
            b = float(case.beta[t, vh])
            v = case.v[t, vh].astype(np.float64)
            assert rel_err(st[case.slot[s], vh], b * np.outer(v, k)) <= 1e-15
            assert rel_err(y[t, vh], case.scale * b * kq * v) <= 1e-13


def pin_gdn_split_resume(orc):
    case = small_gdn_case(13, lengths=(9,), fresh=(0,))
    y_all, st_all = orc.gdn_case(case, threads=1)
    for cut in (1, 4, 8):
        kw = dict(Hv=case.Hv, Hk=case.Hk, Dk=case.Dk, Dv=case.Dv)
        y1, s1 = orc.gdn(**kw, cu_seqlens=[0, cut], slot=case.slot, fresh=case.fresh,
                         q=case.q[:cut], k=case.k[:cut], v=case.v[:cut], g=case.g[:cut],
                         beta=case.beta[:cut], scale=case.scale, state=case.state, threads=1)
        y2, s2 = orc.gdn(**kw, cu_seqlens=[0, 9 - cut], slot=case.slot, fresh=[0],
                         q=case.q[cut:], k=case.k[cut:], v=case.v[cut:], g=case.g[cut:],
                         beta=case.beta[cut:], scale=case.scale, state=s1, threads=1)
        assert np.array_equal(np.concatenate([y1, y2]), y_all), cut
        assert np.array_equal(s2, st_all), cut


def _sub(case, s):
    a, b = int(case.cu_seqlens[s]), int(case.cu_seqlens[s + 1])
    return dict(Hv=case.Hv, Hk=case.Hk, Dk=case.Dk, Dv=case.Dv, cu_seqlens=[0, b - a],
                slot=case.slot[s:s + 1], fresh=case.fresh[s:s + 1], q=case.q[a:b], k=case.k[a:b],
                v=case.v[a:b], g=case.g[a:b], beta=case.beta[a:b], scale=case.scale,
                state=case.state), a, b


def pin_gdn_batch_independence(orc):
    case = small_gdn_case(14)
    y, st = orc.gdn_case(case, threads=3)
    for s in range(case.n_seqs):
        kw, a, b = _sub(case, s)
        y1, s1 = orc.gdn(**kw, threads=1)
        assert np.array_equal(y1, y[a:b]) and np.array_equal(s1[case.slot[s]], st[case.slot[s]])


def pin_gdn_gqa_interleaved(orc):
    """Hk < Hv equals Hk = Hv with each value head given the keys and queries
    of key head vh % Hk explicitly (bitwise)."""
    case = small_gdn_case(15, Hv=6, Hk=2)
    y, st = orc.gdn_case(case, threads=2)
    rep = [vh % case.Hk for vh in range(case.Hv)]
    y2, st2 = orc.gdn(case.Hv, case.Hv, case.Dk, case.Dv, case.cu_seqlens, case.slot, case.fresh,
                      case.q[:, rep], case.k[:, rep], case.v, case.g, case.beta, case.scale,
                      case.state, threads=2)
    assert np.array_equal(y, y2) and np.array_equal(st, st2)


def pin_gdn_slot_hygiene(orc):
    case = ssm_inputs.make_gdn_case(2, 1, 4, 3, [3, 0, 0, 4], [1, 1, 0, 0], 16,
                                    slots=[5, 1, 3, 0], n_slots=6, poison_fresh=True,
                                    sentinel_unused=True)
    y, st = orc.gdn_case(case, threads=2)
    assert np.all(np.isfinite(y))
    for kk in (2, 4):
        assert np.array_equal(st[kk], case.state[kk])
    assert np.array_equal(st[1], np.zeros_like(st[1]))
    assert np.array_equal(st[3], case.state[3])
    assert np.all(np.isfinite(st[5]))


def pin_gdn_snapshots(orc):
    case = small_gdn_case(17, lengths=(4, 2), fresh=(1, 0))
    y, st, sn = orc.gdn_case(case, snapshots=True, threads=2)
    for s in range(case.n_seqs):
        a, b = int(case.cu_seqlens[s]), int(case.cu_seqlens[s + 1])
        for t in range(a, b):
            kw, _, _ = _sub(case, s)
            kw.update(cu_seqlens=[0, t + 1 - a], q=case.q[a:t + 1], k=case.k[a:t + 1],
                      v=case.v[a:t + 1], g=case.g[a:t + 1], beta=case.beta[a:t + 1])
            _, s1 = orc.gdn(**kw, threads=1)
            assert np.array_equal(sn[t], s1[case.slot[s]]), (s, t)
        assert np.array_equal(sn[b - 1], st[case.slot[s]])


def pin_gdn_thread_count(orc):
    case = ssm_inputs.gdn_workload("mixed")
    y1, s1 = orc.gdn_case(case, threads=1)
    y3, s3 = orc.gdn_case(case, threads=3)
    assert np.array_equal(y1, y3) and np.array_equal(s1, s3, equal_nan=True)


GDN_PINS = [pin_gdn_matrix_form, pin_gdn_matrix_form_general_keys, pin_gdn_key_length_overwrite,
            pin_gdn_tiny_workload_matrix_form, pin_gdn_overwrite,
            pin_gdn_pure_decay, pin_gdn_single_token, pin_gdn_split_resume,
            pin_gdn_batch_independence, pin_gdn_gqa_interleaved, pin_gdn_slot_hygiene,
            pin_gdn_snapshots, pin_gdn_thread_count]
