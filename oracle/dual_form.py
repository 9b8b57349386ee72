"""Dense quadratic ("dual") form of the SSD scan, materialised in fp64.

Test infrastructure only.  Source: "Compiler-First State Space Duality and
Portable O(1) Autoregressive Caching", Background, Eq. 3 and the "diagonal
state matrix" property: unrolling the diagonal recurrence gives
y = M x with a lower-triangular M whose (i, j) entry is
(C_i . B_j) * exp(sum of A*Delta over tokens j+1..i) * Delta_j.

Here the whole sequence is one block (no chunking), and every segment sum
sum_{k=j+1..i} a_k is accumulated directly along the row (never formed as a
difference of two prefix sums), so this shares neither the recurrence's
token loop nor the chunked algorithm's prefix-sum arithmetic.
Cost is O(T^2 (N + P)) per (b, h): tiny inputs only.
"""
from __future__ import annotations

import numpy as np


def _delta(dt, dt_bias, h, dt_softplus, dt_min, dt_max):
    z = dt.astype(np.float64) + (0.0 if dt_bias is None else float(dt_bias[h]))
    if dt_softplus:
        z = np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))
    return np.clip(z, float(np.float32(dt_min)), float(np.float32(dt_max)))


def dual_form(x, dt, A, B, C, D=None, dt_bias=None, h0=None, *, dt_softplus=True,
              dt_min=1e-4, dt_max=0.5):
    """Returns (y, final_state) in float64; same argument conventions as
    oracle.scan (numpy arrays)."""
    x = np.asarray(x, np.float64)
    Bt, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = H // G
    y = np.zeros((Bt, T, H, P))
    fin = np.zeros((Bt, H, P, N))
    for b in range(Bt):
        for h in range(H):
            g = h // hpg
            d = _delta(np.asarray(dt)[b, :, h], dt_bias, h, dt_softplus, dt_min, dt_max)
            a = d * float(A[h])
            Bg = np.asarray(B, np.float64)[b, :, g, :]       # [T, N]
            Cg = np.asarray(C, np.float64)[b, :, g, :]       # [T, N]
            X = x[b, :, h, :]                                # [T, P]
            M = np.zeros((T, T))
            for i in range(T):
                # seg[j] = sum_{k=j+1..i} a_k for j = i, i-1, ..., 0, summed outward from i
                seg = np.zeros(i + 1)
                run = 0.0
                for j in range(i, -1, -1):
                    seg[j] = run
                    run += a[j]
                M[i, : i + 1] = (Cg[i] @ Bg[: i + 1].T) * np.exp(seg) * d[: i + 1]
            yy = M @ X
            if D is not None:
                yy += float(D[h]) * X
            # state at the end: sum_j exp(sum_{k>j} a_k) d_j x_j (x) B_j
            tail = np.zeros(T)
            run = 0.0
            for j in range(T - 1, -1, -1):
                tail[j] = run
                run += a[j]
            F = (X * (np.exp(tail) * d)[:, None]).T @ Bg     # [P, N]
            if h0 is not None:
                H0 = np.asarray(h0, np.float64)[b, h]
                # contribution of the initial state: decay through tokens 0..i
                pre = np.zeros(T)
                run = 0.0
                for i in range(T):
                    run += a[i]
                    pre[i] = run
                yy += np.exp(pre)[:, None] * (Cg @ H0.T)
                F += np.exp(run) * H0
            y[b, :, h, :] = yy
            fin[b, h] = F
    return y, fin
