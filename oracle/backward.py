"""fp64 oracle of the mixer's backward pass -- TEST INFRASTRUCTURE ONLY.

Gradients of one mixer call (GTR write-up "端侧实时感知新标杆！通用线性骨干网络GTR开源",
Method §1: S_t = Diag(g_t) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t, then RMSNorm
over dv, the rms_w weight and the SiLU(z) output gate) with respect to q, k,
v, log_g, z and rms_w, given the gradient dout of the output.  Written from
the chain rule, token by token in scan order, with the states kept:

  epilogue:  r_t = (mean(o_t^2) + eps)^(-1/2),  n_t = r_t o_t,  y_t = n_t w silu(z_t)
             dn_t = dy_t w silu(z_t);  do_t = r_t (dn_t - n_t mean(dn_t n_t))
             dz_t = dy_t n_t w silu'(z_t);  drms_w = sum_t dy_t n_t silu(z_t)
  recurrence: dq_t = S_t do_t
             dS_t = q_t do_t^T + Diag(g_{t+1}) dS_{t+1}      (dS_L = 0)
             dk_t = dS_t v_t,  dv_t = dS_t^T k_t
             dlog_g_t = g_t * sum_d dS_t[:, d] S_{t-1}[:, d]  (S_{-1} = 0)

Plain numpy loops (fine for the test sizes).  Imports nothing from the library.
"""
from __future__ import annotations

import numpy as np

RMS_EPS = 1e-5


def _order(gh: int, gw: int, direction: int) -> np.ndarray:
    """Grid index of each scan step (Method §1 directions LR, RL, TB, BT)."""
    L = gh * gw
    t = np.arange(L)
    if direction & 1:
        t = L - 1 - t
    if direction < 2:
        return t
    c, r = t // gh, t % gh
    return r * gw + c


def bwd(q, k, v, log_g, z, rms_w, dout, direction: int, eps: float = RMS_EPS, bh=None):
    """Returns dict dq, dk, dv, dlog_g, dz (shapes of the inputs) and drms_w [dv], fp64.

    The dict also holds ``y``: the forward output that the kept states give
    (o_t = S_t^T q_t, then the epilogue), stored at grid positions, so that the
    forward half of this oracle can be checked against the C oracle.

    ``bh``: optional iterable of b*H + h sequences to differentiate; the other
    sequences' gradients are NaN and drms_w sums over the chosen ones only."""
    q, k, v, log_g, z, w, dy = (np.asarray(a, dtype=np.float64) for a in
                                (q, k, v, log_g, z, rms_w, dout))
    B, gh, gw, H, dk = q.shape
    dv = v.shape[-1]
    L = gh * gw
    order = _order(gh, gw, direction)
    out = {name: np.full(a.shape, np.nan) for name, a in
           (("dq", q), ("dk", k), ("dv", v), ("dlog_g", log_g), ("dz", z), ("y", z))}
    drms = np.zeros(dv)
    seqs = range(B * H) if bh is None else bh
    for s in seqs:
        b, h = divmod(int(s), H)
        Q = q[b].reshape(L, H, dk)[order, h]
        K = k[b].reshape(L, H, dk)[order, h]
        V = v[b].reshape(L, H, dv)[order, h]
        G = np.exp(log_g[b].reshape(L, H, dk)[order, h])
        Z = z[b].reshape(L, H, dv)[order, h]
        DY = dy[b].reshape(L, H, dv)[order, h]
        # forward, keeping every state
        Ss = np.zeros((L + 1, dk, dv))          # Ss[t + 1] = S_t, Ss[0] = S_{-1} = 0
        O = np.zeros((L, dv))
        for t in range(L):
            Ss[t + 1] = G[t][:, None] * Ss[t] + np.outer(K[t], V[t])
            O[t] = Ss[t + 1].T @ Q[t]
        # epilogue backward
        r = 1.0 / np.sqrt((O * O).mean(axis=1) + eps)
        N = O * r[:, None]
        sig = 1.0 / (1.0 + np.exp(-Z))
        silu = Z * sig
        dN = DY * w * silu
        dO = r[:, None] * (dN - N * (dN * N).mean(axis=1)[:, None])
        dZ = DY * N * w * sig * (1.0 + Z * (1.0 - sig))
        drms += (DY * N * silu).sum(axis=0)
        Y = N * w * silu
        # recurrence backward
        dQ = np.einsum("tcd,td->tc", Ss[1:], dO)
        dK, dV, dLG = np.zeros((L, dk)), np.zeros((L, dv)), np.zeros((L, dk))
        dS = np.zeros((dk, dv))
        for t in range(L - 1, -1, -1):
            if t < L - 1:
                dS = G[t + 1][:, None] * dS
            dS = dS + np.outer(Q[t], dO[t])
            dK[t] = dS @ V[t]
            dV[t] = dS.T @ K[t]
            dLG[t] = G[t] * (dS * Ss[t]).sum(axis=1)
        for name, val, d in (("dq", dQ, dk), ("dk", dK, dk), ("dv", dV, dv),
                             ("dlog_g", dLG, dk), ("dz", dZ, dv), ("y", Y, dv)):
            dst = out[name][b].reshape(L, H, d)
            dst[order, h] = val
            out[name][b] = dst.reshape(out[name][b].shape)
    out["drms_w"] = drms
    return out
