"""The chunked SSD algorithm written out step by step in fp64 (numpy).

Test infrastructure only.  Source: "Compiler-First State Space Duality and
Portable O(1) Autoregressive Caching", Background (Eq. 3 and the inter-chunk
recurrence that follows it) and SSD properties ("diagonal state matrix",
"chunked recurrence").  For each (b, h) the sequence is cut into chunks of L
tokens (the last one may be shorter); within a chunk:

  step 1  d_l = clip(softplus(dt_l + dt_bias))          (Delta preparation)
  step 2  cum_l = sum_{k<=l} d_k A                       (segment prefix sum)
  step 3  Lmat[i,j] = exp(cum_i - cum_j) if j <= i else 0 (mask chosen before exp)
  step 4  S = C_c B_c^T                                  ([L,N] x [N,L])
  step 5  Y_diag = (S o Lmat o d_j) X_c                  ([L,L] x [L,P])
  step 6  S_c = sum_l exp(cum_last - cum_l) d_l x_l (x) B_l  (chunk summary state)
  step 7  h_c = exp(cum_last) h_{c-1} + S_c              (inter-chunk recurrence)
  step 8  Y_off[l] = exp(cum_l) C_l h_{c-1}^T ;  y = Y_diag + Y_off + D x

Every intermediate is returned so that GPU intermediates can be inspected.
"""
from __future__ import annotations

import numpy as np

from .dual_form import _delta


def chunked(x, dt, A, B, C, D=None, dt_bias=None, h0=None, *, chunk=64, dt_softplus=True,
            dt_min=1e-4, dt_max=0.5, keep_intermediates=False):
    x = np.asarray(x, np.float64)
    Bt, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = H // G
    L = int(chunk)
    nc = (T + L - 1) // L
    y = np.zeros((Bt, T, H, P))
    fin = np.zeros((Bt, H, P, N))
    inter = {"cum": {}, "S_c": {}, "h_prev": {}}
    for b in range(Bt):
        for h in range(H):
            g = h // hpg
            d_all = _delta(np.asarray(dt)[b, :, h], dt_bias, h, dt_softplus, dt_min, dt_max)
            hs = np.zeros((P, N)) if h0 is None else np.asarray(h0, np.float64)[b, h].copy()
            for c in range(nc):
                s, e = c * L, min((c + 1) * L, T)
                d = d_all[s:e]
                cum = np.cumsum(d * float(A[h]))                        # step 2
                diff = cum[:, None] - cum[None, :]
                causal = np.tril(np.ones((e - s, e - s), dtype=bool))
                Lmat = np.where(causal, np.exp(np.where(causal, diff, 0.0)), 0.0)  # step 3
                Cc = np.asarray(C, np.float64)[b, s:e, g, :]
                Bc = np.asarray(B, np.float64)[b, s:e, g, :]
                Xc = x[b, s:e, h, :]
                S = Cc @ Bc.T                                           # step 4
                Ydiag = (S * Lmat * d[None, :]) @ Xc                    # step 5
                w = np.exp(cum[-1] - cum) * d
                Sc = (Xc * w[:, None]).T @ Bc                           # step 6
                Yoff = np.exp(cum)[:, None] * (Cc @ hs.T)               # step 8 (uses h_{c-1})
                yy = Ydiag + Yoff
                if D is not None:
                    yy = yy + float(D[h]) * Xc
                y[b, s:e, h, :] = yy
                if keep_intermediates:
                    inter["cum"][(b, h, c)] = cum
                    inter["S_c"][(b, h, c)] = Sc
                    inter["h_prev"][(b, h, c)] = hs.copy()
                hs = np.exp(cum[-1]) * hs + Sc                          # step 7
            fin[b, h] = hs
    if keep_intermediates:
        return y, fin, inter
    return y, fin
