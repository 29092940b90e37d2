"""Independent fp64 formulations used to pin the oracle (test helpers).

None of this calls the oracle or the GPU library.  The brute-force form is the
recurrence unrolled, which the benchmark spec of the scan and the
recurrence on "The llama journey" (Day 14) imply: for one (sequence, head),
with a_k = exp(dt_k * A), u_k = dt_k * x_k and tokens k = 1..t,

    h_t = (prod_{r=1..t} a_r) h_0 + sum_{j=1..t} (prod_{r=j+1..t} a_r) u_j (x) B_j
    y_t = h_t . C_t          (contracted over the state index)

Products are formed by explicit loops over the token pairs; the contraction
uses numpy.einsum.  Heads map to groups contiguously, g = head // (H // G).
"""
from __future__ import annotations

import numpy as np


def brute_force(H, P, N, G, cu_seqlens, slot, fresh, x, dt, A, B, C, state):
    """Return (y, state_out) in float64 from the unrolled closed form."""
    x = np.asarray(x, dtype=np.float64)
    dt = np.asarray(dt, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    st = np.array(state, dtype=np.float64, copy=True)
    T = x.shape[0]
    y = np.zeros((T, H, P), dtype=np.float64)
    hpg = H // G
    for s in range(len(slot)):
        t0, t1 = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        L = t1 - t0
        for hd in range(H):
            g = hd // hpg
            h0 = np.zeros((P, N)) if fresh[s] else st[slot[s], hd].copy()
            if L == 0:
                st[slot[s], hd] = h0
                continue
            a = np.exp(dt[t0:t1, hd] * A[hd])                 # [L]
            u = dt[t0:t1, hd, None] * x[t0:t1, hd, :]          # [L, P]
            Bs = B[t0:t1, g, :]                                # [L, N]
            Cs = C[t0:t1, g, :]
            # decay[k, j] = prod of a over tokens j+1..k (empty product = 1)
            decay = np.zeros((L, L))
            lead = np.zeros(L)                                 # prod a_0..a_k
            for k in range(L):
                lead[k] = np.prod(a[: k + 1])
                for j in range(k + 1):
                    decay[k, j] = np.prod(a[j + 1: k + 1])
            hs = lead[:, None, None] * h0[None] + np.einsum("kj,jp,jn->kpn", decay, u, Bs)
            y[t0:t1, hd, :] = np.einsum("kpn,kn->kp", hs, Cs)
            st[slot[s], hd] = hs[-1]
    return y, st
