"""The token-by-token recurrence at 50 significant digits (mpmath).

Test infrastructure only.  Same definition as the C oracle ("Compiler-First
State Space Duality and Portable O(1) Autoregressive Caching", Background,
Eq. 2 with Abar = exp(Delta A), Bbar = Delta B), evaluated with mpmath so the
C oracle's double rounding can be bounded.  Tiny inputs only (T <= 16,
P, N <= 3).
"""
from __future__ import annotations

import mpmath as mp
import numpy as np


def brute(x, dt, A, B, C, D=None, dt_bias=None, h0=None, *, dt_softplus=True,
          dt_min=1e-4, dt_max=0.5, digits=50):
    with mp.workdps(digits):
        x = np.asarray(x, np.float64)
        Bt, T, H, P = x.shape
        G, N = B.shape[2], B.shape[3]
        hpg = H // G
        lo, hi = mp.mpf(float(np.float32(dt_min))), mp.mpf(float(np.float32(dt_max)))
        y = np.zeros((Bt, T, H, P))
        fin = np.zeros((Bt, H, P, N))
        for b in range(Bt):
            for h in range(H):
                g = h // hpg
                S = [[mp.mpf(0) if h0 is None else mp.mpf(float(h0[b, h, p, n]))
                      for n in range(N)] for p in range(P)]
                for t in range(T):
                    z = mp.mpf(float(dt[b, t, h])) + (mp.mpf(float(dt_bias[h])) if dt_bias is not None else 0)
                    d = mp.log(1 + mp.exp(z)) if dt_softplus else z
                    d = min(max(d, lo), hi)
                    abar = mp.exp(d * mp.mpf(float(A[h])))
                    for p in range(P):
                        acc = mp.mpf(0)
                        for n in range(N):
                            S[p][n] = abar * S[p][n] + d * mp.mpf(float(x[b, t, h, p])) * mp.mpf(float(B[b, t, g, n]))
                            acc += mp.mpf(float(C[b, t, g, n])) * S[p][n]
                        if D is not None:
                            acc += mp.mpf(float(D[h])) * mp.mpf(float(x[b, t, h, p]))
                        y[b, t, h, p] = float(acc)
                for p in range(P):
                    for n in range(N):
                        fin[b, h, p, n] = float(S[p][n])
        return y, fin
