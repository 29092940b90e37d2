"""Seeded synthetic inputs for the Mamba2 selective-state scan.

This module only draws random numbers and lays them out; it holds none of the
scan's arithmetic.  Both the CPU oracle (through the tests) and the GPU path
(through the tests and the benchmark) receive the very same host arrays from
here, so the two sides see identical input bits.

Shapes follow the operand table of ggml's CPU scan as transcribed on
"The llama journey" (Day 12, the src0..src6 table): state [slot][head][row][n],
x [token][head][row], dt [token][head], A [head] (one scalar per head for
Mamba2), B and C [token][group][n].  Tokens of all sequences are packed one
after another; ``cu_seqlens`` gives where each sequence starts.

Value distributions (the five workloads named below): x, B, C ~ N(0, 1);
dt ~ U[0.001, 0.1]; A = -exp(U[0, ln 16]) per head, so A is log-uniform in
[-16, -1]; a resuming state ~ 0.5 * N(0, 1).  Draw order is fixed: A, dt, x,
B, C, state.  The generator is numpy's PCG64 seeded with the case's seed.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = ["ScanCase", "make_case", "WORKLOADS", "workload", "lengths_to_cu",
           "ConvCase", "make_conv_case", "CONV_WORKLOADS", "conv_workload",
           "NormCase", "make_norm_case", "NORM_WORKLOADS", "norm_workload",
           "GdnCase", "make_gdn_case", "GDN_WORKLOADS", "gdn_workload"]


@dataclass
class ScanCase:
    """One packed batch: dims, per-sequence metadata and the fp32 operands."""

    H: int
    P: int
    N: int
    G: int
    lengths: np.ndarray          # int32 [n_seqs]
    cu_seqlens: np.ndarray       # int32 [n_seqs + 1]
    slot: np.ndarray             # int32 [n_seqs]
    fresh: np.ndarray            # uint8 [n_seqs]
    x: np.ndarray                # f32 [T, H, P]
    dt: np.ndarray               # f32 [T, H]
    A: np.ndarray                # f32 [H]
    B: np.ndarray                # f32 [T, G, N]
    C: np.ndarray                # f32 [T, G, N]
    state: np.ndarray            # f32 [n_slots, H, P, N] (initial contents)
    seed: int = 0
    name: str = ""
    notes: dict = field(default_factory=dict)

    @property
    def n_seqs(self) -> int:
        return int(self.lengths.shape[0])

    @property
    def n_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def n_slots(self) -> int:
        return int(self.state.shape[0])


def lengths_to_cu(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(lengths.shape[0] + 1, dtype=np.int64)
    np.cumsum(lengths, out=cu[1:])
    return cu.astype(np.int32)


def make_case(H, P, N, G, lengths, fresh, seed, *, slots=None, n_slots=None,
              state_std=0.5, dt_lo=0.001, dt_hi=0.1, a_log_hi=math.log(16.0),
              poison_fresh=False, sentinel_unused=False, name="") -> ScanCase:
    """Draw one packed batch.

    ``fresh`` is a sequence of 0/1 flags (1 = start from the zero state).
    ``slots`` defaults to 0..n_seqs-1.  With ``poison_fresh`` the slots of
    fresh sequences are filled with NaN (a correct scan never reads them).
    With ``sentinel_unused`` slots that no sequence names are filled with a
    recognisable finite pattern (they must come back bit-for-bit unchanged).
    """
    lengths = np.asarray(lengths, dtype=np.int32)
    fresh = np.asarray(fresh, dtype=np.uint8)
    n_seqs = lengths.shape[0]
    if slots is None:
        slots = np.arange(n_seqs, dtype=np.int32)
    slots = np.asarray(slots, dtype=np.int32)
    if n_slots is None:
        n_slots = int(slots.max()) + 1 if n_seqs else 0
    cu = lengths_to_cu(lengths)
    T = int(cu[-1])
    rng = np.random.Generator(np.random.PCG64(seed))
    A = (-np.exp(rng.uniform(0.0, a_log_hi, size=H))).astype(np.float32)
    dt = rng.uniform(dt_lo, dt_hi, size=(T, H)).astype(np.float32)
    x = rng.standard_normal((T, H, P), dtype=np.float32)
    B = rng.standard_normal((T, G, N), dtype=np.float32)
    C = rng.standard_normal((T, G, N), dtype=np.float32)
    state = rng.standard_normal((n_slots, H, P, N), dtype=np.float32)
    state *= np.float32(state_std)
    if sentinel_unused:
        used = np.zeros(n_slots, dtype=bool)
        used[slots] = True
        for k in np.nonzero(~used)[0]:
            state[k] = np.float32(1000.0 + k)
    if poison_fresh:
        for s in range(n_seqs):
            if fresh[s]:
                state[slots[s]] = np.nan
    return ScanCase(H=H, P=P, N=N, G=G, lengths=lengths, cu_seqlens=cu, slot=slots,
                    fresh=fresh, x=x, dt=dt, A=A, B=B, C=C, state=state, seed=seed,
                    name=name)


# The five workloads.  Seeds: the tiny scan's seed 0 is given; the others are
# this project's choice (1..4), fixed here.
def _tiny(seed=0):
    return make_case(4, 16, 16, 1, [64], [1], seed, name="tiny_T64_H4_P16_N16_G1")


def _decode16(seed=1, sets=1):
    n = 16
    return make_case(64, 64, 128, 8, [1] * n, [0] * n, seed, n_slots=n * sets,
                     name="decode_16x1_H64_P64_N128_G8")


def _prefill4096(seed=2):
    return make_case(64, 64, 128, 8, [4096], [1], seed,
                     name="prefill_1x4096_H64_P64_N128_G8")


def _mixed(seed=3):
    lengths = [1, 7, 25, 26, 64, 100, 150, 150]
    fresh = [1 - (i % 2) for i in range(8)]          # odd indices resume
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    slots = rng.permutation(10)[:8].astype(np.int32)  # 2 of 10 slots unused
    return make_case(16, 96, 100, 4, lengths, fresh, seed, slots=slots, n_slots=10,
                     poison_fresh=True, sentinel_unused=True,
                     name="mixed_8seq_H16_P96_N100_G4")


def _decode256(seed=4):
    n = 256
    return make_case(64, 64, 128, 8, [1] * n, [0] * n, seed,
                     name="decode_256x1_H64_P64_N128_G8")


WORKLOADS = {
    "tiny": _tiny,
    "decode16": _decode16,
    "prefill4096": _prefill4096,
    "mixed": _mixed,
    "decode256": _decode256,
}


def workload(name: str, **kw) -> ScanCase:
    return WORKLOADS[name](**kw)


# ---------------------------------------------------------------------------
# The steps on either side of the scan.
#
# Causal conv1d + SiLU: x [T][D] token-major (packed like the scan's x), the
# depthwise weight [D][K], the rolling history [n_slots][D][K-1] oldest first
# (the layout of "ssm_gated_delta.cu", fc_ssm_conv1d_silu).  In a Mamba2 layer
# the conv runs over the concatenation of x, B and C, so D = H*P + 2*G*N with
# K = 4.  Values: x and history ~ N(0, 1) (the history holds past raw inputs);
# weights ~ U(-1/sqrt(K), 1/sqrt(K)), the usual fan-in scale of a depthwise
# conv.  Draw order: w, x, state.
#
# Gated RMSNorm: y and z [T][H][P], the shared weight [P] (the layout of
# fc_ssm_gated_norm, one row per head).  Values: y, z ~ N(0, 1), weight
# 1 + 0.1 * N(0, 1), eps 1e-5.  Draw order: w, y, z.
# ---------------------------------------------------------------------------
@dataclass
class ConvCase:
    D: int
    K: int
    lengths: np.ndarray          # int32 [n_seqs]
    cu_seqlens: np.ndarray       # int32 [n_seqs + 1]
    slot: np.ndarray             # int32 [n_seqs]
    fresh: np.ndarray            # uint8 [n_seqs]
    x: np.ndarray                # f32 [T, D]
    w: np.ndarray                # f32 [D, K]
    state: np.ndarray            # f32 [n_slots, D, K - 1]
    seed: int = 0
    name: str = ""

    @property
    def n_seqs(self) -> int:
        return int(self.lengths.shape[0])

    @property
    def n_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def n_slots(self) -> int:
        return int(self.state.shape[0])


def make_conv_case(D, K, lengths, fresh, seed, *, slots=None, n_slots=None,
                   poison_fresh=False, sentinel_unused=False, name="") -> ConvCase:
    """Draw one packed conv batch; ``slots``, ``poison_fresh`` and
    ``sentinel_unused`` mean what they mean for ``make_case``."""
    lengths = np.asarray(lengths, dtype=np.int32)
    fresh = np.asarray(fresh, dtype=np.uint8)
    n_seqs = lengths.shape[0]
    if slots is None:
        slots = np.arange(n_seqs, dtype=np.int32)
    slots = np.asarray(slots, dtype=np.int32)
    if n_slots is None:
        n_slots = int(slots.max()) + 1 if n_seqs else 0
    cu = lengths_to_cu(lengths)
    T = int(cu[-1])
    rng = np.random.Generator(np.random.PCG64(seed))
    bound = 1.0 / math.sqrt(K)
    w = rng.uniform(-bound, bound, size=(D, K)).astype(np.float32)
    x = rng.standard_normal((T, D), dtype=np.float32)
    state = rng.standard_normal((n_slots, D, K - 1), dtype=np.float32)
    if sentinel_unused:
        used = np.zeros(n_slots, dtype=bool)
        used[slots] = True
        for k in np.nonzero(~used)[0]:
            state[k] = np.float32(1000.0 + k)
    if poison_fresh:
        for s in range(n_seqs):
            if fresh[s]:
                state[slots[s]] = np.nan
    return ConvCase(D=D, K=K, lengths=lengths, cu_seqlens=cu, slot=slots, fresh=fresh,
                    x=x, w=w, state=state, seed=seed, name=name)


def conv_channels(H, P, N, G) -> int:
    """Channels of a Mamba2 layer's conv: x, B and C side by side."""
    return H * P + 2 * G * N


CONV_WORKLOADS = {
    "tiny": lambda seed=10: make_conv_case(conv_channels(4, 16, 16, 1), 4, [64], [1], seed,
                                           name="conv_tiny_T64_D96_K4"),
    "decode16": lambda seed=11, sets=1: make_conv_case(
        conv_channels(64, 64, 128, 8), 4, [1] * 16, [0] * 16, seed, n_slots=16 * sets,
        name="conv_decode_16x1_D6144_K4"),
    "prefill4096": lambda seed=12: make_conv_case(
        conv_channels(64, 64, 128, 8), 4, [4096], [1], seed,
        name="conv_prefill_1x4096_D6144_K4"),
    "mixed": lambda seed=13: make_conv_case(
        conv_channels(16, 96, 100, 4), 4, [1, 7, 25, 26, 64, 100, 150, 150],
        [1 - (i % 2) for i in range(8)], seed,
        slots=np.random.Generator(np.random.PCG64(seed + 1000)).permutation(10)[:8]
        .astype(np.int32), n_slots=10, poison_fresh=True, sentinel_unused=True,
        name="conv_mixed_8seq_D2336_K4"),
    "decode256": lambda seed=14: make_conv_case(
        conv_channels(64, 64, 128, 8), 4, [1] * 256, [0] * 256, seed,
        name="conv_decode_256x1_D6144_K4"),
}


def conv_workload(name: str, **kw) -> ConvCase:
    return CONV_WORKLOADS[name](**kw)


@dataclass
class NormCase:
    y: np.ndarray                # f32 [T, H, P]
    z: np.ndarray                # f32 [T, H, P]
    w: np.ndarray                # f32 [P]
    eps: float
    seed: int = 0
    name: str = ""


def make_norm_case(T, H, P, seed, *, eps=1e-5, y_std=1.0, name="") -> NormCase:
    rng = np.random.Generator(np.random.PCG64(seed))
    w = (1.0 + 0.1 * rng.standard_normal(P)).astype(np.float32)
    y = rng.standard_normal((T, H, P), dtype=np.float32)
    y *= np.float32(y_std)
    z = rng.standard_normal((T, H, P), dtype=np.float32)
    return NormCase(y=y, z=z, w=w, eps=float(eps), seed=seed, name=name)


NORM_WORKLOADS = {
    "tiny": lambda seed=20: make_norm_case(64, 4, 16, seed, name="norm_tiny_T64_H4_P16"),
    "decode16": lambda seed=21: make_norm_case(16, 64, 64, seed, name="norm_16x1_H64_P64"),
    "prefill4096": lambda seed=22: make_norm_case(4096, 64, 64, seed,
                                                  name="norm_1x4096_H64_P64"),
    "mixed": lambda seed=23: make_norm_case(523, 16, 96, seed, name="norm_T523_H16_P96"),
    "decode256": lambda seed=24: make_norm_case(256, 64, 64, seed, name="norm_256x1_H64_P64"),
}


def norm_workload(name: str, **kw) -> NormCase:
    return NORM_WORKLOADS[name](**kw)


# ---------------------------------------------------------------------------
# Gated delta-rule recurrence ("ssm_gated_delta.cu").  q, k [T][Hk][Dk] arrive
# L2-normalised per head, as on that page; v [T][Hv][Dv]; the log decay
# g = a[h] * dt with a = -exp(U[0, ln 16]) per head and dt ~ U[0.001, 0.1]
# (the scan's decay distribution, g in [-1.6, -0.001]); beta = sigmoid(N(0,1));
# a resuming state ~ 0.5 * N(0, 1); scale = 1/sqrt(Dk).  Draw order: a, dt, q,
# k, v, beta, state.  The page's model geometry: Hv 32, Hk 16, Dk = Dv = 128.
# ---------------------------------------------------------------------------
@dataclass
class GdnCase:
    Hv: int
    Hk: int
    Dk: int
    Dv: int
    lengths: np.ndarray
    cu_seqlens: np.ndarray
    slot: np.ndarray
    fresh: np.ndarray
    q: np.ndarray                # f32 [T, Hk, Dk], unit rows unless drawn otherwise
    k: np.ndarray                # f32 [T, Hk, Dk], unit rows unless drawn otherwise
    v: np.ndarray                # f32 [T, Hv, Dv]
    g: np.ndarray                # f32 [T, Hv], log decay
    beta: np.ndarray             # f32 [T, Hv]
    state: np.ndarray            # f32 [n_slots, Hv, Dv, Dk]
    scale: float
    seed: int = 0
    name: str = ""

    @property
    def n_seqs(self) -> int:
        return int(self.lengths.shape[0])

    @property
    def n_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def n_slots(self) -> int:
        return int(self.state.shape[0])


def _unit_rows(a):
    n = np.sqrt(np.sum(a.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (a / np.maximum(n, 1e-6)).astype(np.float32)


def make_gdn_case(Hv, Hk, Dk, Dv, lengths, fresh, seed, *, slots=None, n_slots=None,
                  state_std=0.5, poison_fresh=False, sentinel_unused=False, qk_norm=None,
                  beta=None, name="") -> GdnCase:
    """Draw one packed delta-rule batch.  By default q and k rows have unit
    length.  ``qk_norm=(lo, hi)`` rescales every q and k row to a length
    drawn from U[lo, hi]; ``beta`` (a float) replaces the drawn write
    strengths with that constant.  Both are drawn or applied after every
    default draw, so cases without them keep their bits."""
    lengths = np.asarray(lengths, dtype=np.int32)
    fresh = np.asarray(fresh, dtype=np.uint8)
    n_seqs = lengths.shape[0]
    if slots is None:
        slots = np.arange(n_seqs, dtype=np.int32)
    slots = np.asarray(slots, dtype=np.int32)
    if n_slots is None:
        n_slots = int(slots.max()) + 1 if n_seqs else 0
    cu = lengths_to_cu(lengths)
    T = int(cu[-1])
    rng = np.random.Generator(np.random.PCG64(seed))
    a = -np.exp(rng.uniform(0.0, math.log(16.0), size=Hv))
    dt = rng.uniform(0.001, 0.1, size=(T, Hv))
    g = (a[None, :] * dt).astype(np.float32)
    q = _unit_rows(rng.standard_normal((T, Hk, Dk), dtype=np.float32))
    k = _unit_rows(rng.standard_normal((T, Hk, Dk), dtype=np.float32))
    v = rng.standard_normal((T, Hv, Dv), dtype=np.float32)
    beta_drawn = (1.0 / (1.0 + np.exp(-rng.standard_normal((T, Hv))))).astype(np.float32)
    state = rng.standard_normal((n_slots, Hv, Dv, Dk), dtype=np.float32)
    state *= np.float32(state_std)
    if qk_norm is not None:
        lo, hi = qk_norm
        q = (q * rng.uniform(lo, hi, size=(T, Hk, 1))).astype(np.float32)
        k = (k * rng.uniform(lo, hi, size=(T, Hk, 1))).astype(np.float32)
    beta_arr = beta_drawn if beta is None else np.full((T, Hv), beta, dtype=np.float32)
    if sentinel_unused:
        used = np.zeros(n_slots, dtype=bool)
        used[slots] = True
        for kk in np.nonzero(~used)[0]:
            state[kk] = np.float32(1000.0 + kk)
    if poison_fresh:
        for s in range(n_seqs):
            if fresh[s]:
                state[slots[s]] = np.nan
    return GdnCase(Hv=Hv, Hk=Hk, Dk=Dk, Dv=Dv, lengths=lengths, cu_seqlens=cu, slot=slots,
                   fresh=fresh, q=q, k=k, v=v, g=g, beta=beta_arr, state=state,
                   scale=float(np.float32(1.0 / math.sqrt(Dk))), seed=seed, name=name)


GDN_WORKLOADS = {
    "tiny": lambda seed=30: make_gdn_case(4, 2, 16, 16, [64], [1], seed,
                                          name="gdn_tiny_T64_Hv4_Hk2_D16"),
    "decode16": lambda seed=31, sets=1: make_gdn_case(
        32, 16, 128, 128, [1] * 16, [0] * 16, seed, n_slots=16 * sets,
        name="gdn_decode_16x1_Hv32_Hk16_D128"),
    "prefill4096": lambda seed=32: make_gdn_case(32, 16, 128, 128, [4096], [1], seed,
                                                 name="gdn_prefill_1x4096_Hv32_Hk16_D128"),
    "mixed": lambda seed=33: make_gdn_case(
        8, 4, 100, 96, [1, 7, 25, 26, 64, 100, 150, 150], [1 - (i % 2) for i in range(8)], seed,
        slots=np.random.Generator(np.random.PCG64(seed + 1000)).permutation(10)[:8]
        .astype(np.int32), n_slots=10, poison_fresh=True, sentinel_unused=True,
        name="gdn_mixed_8seq_Hv8_Hk4_Dk100_Dv96"),
    "decode256": lambda seed=34: make_gdn_case(32, 16, 128, 128, [1] * 256, [0] * 256, seed,
                                               name="gdn_decode_256x1_Hv32_Hk16_D128"),
}


def gdn_workload(name: str, **kw) -> GdnCase:
    return GDN_WORKLOADS[name](**kw)
