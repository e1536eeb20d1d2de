"""Plain fp64 CPU oracle of the gradient of the VDA linear branch.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import or call this module.  It shares no code with the
HIP path and imports nothing from the product package; the forward quantities
it needs come from the forward oracle (oracle.vdn_oracle).

Sources.  [P3] 10100.com article on Video DeltaNet, section 方法概述 part 2
(the frame-level delta rule S_t = (Sbar_t + B_t)(I + A_t)^-1 with
A_t = beta_t K_t^T K_t and B_t = beta_t V_t^T K_t), part 3 (RMSNorm per
direction, summed, before the gate; the staged adaptation that trains the
linear branch) and the 实验结果 figure caption (forward plus backward scan).
The pages give the forward computation only; the gradient below is the
derivative of that forward computation (the forward oracle's readings D-1,
D-2, D-5..D-8 apply unchanged), taken step by step in reverse order:

  readout   o = w * (r_f + r_b), r = u / rho, rho = sqrt(mean(u^2) + eps),
            u = S_t q (per direction, per token):
              dw += (r_f + r_b) * do;   g = w * do;
              du = (g - r * mean(g * r)) / rho;
              dq += S_t^T du;           dS_t += du q^T
  scan      S_t = X_t M_t, X_t = gamma_t S_prev + B_t (S_prev = S_{t-1} for
            the forward scan, S_{t+1} for the backward scan, zero at the
            start); G_t = dS_t + (gradient arriving from the next step of the
            same scan, gamma_next dX_next):
              dX_t = G_t M_t^T;  dM_t += X_t^T G_t;  dB_t += dX_t;
              dgamma_t += <dX_t, S_prev>
  solve     M_t = (I + A_t)^-1:  dA_t = -M_t^T dM_t M_t^T
  Gram      A_t = beta_t K_t^T K_t, B_t = beta_t V_t^T K_t:
              dK_t = beta_t K_t (dA_t + dA_t^T) + beta_t V_t dB_t
              dV_t = beta_t K_t dB_t^T
              dbeta_t = <dA_t, K_t^T K_t> + <dB_t, V_t^T K_t>

Here <X, Y> is the sum of the elementwise products.  The tests pin every
output against central finite differences of the forward oracle and against
invariants of the forward computation.  The gradient of the sigmoid gate and
of the output projections is not part of this module.
"""
from __future__ import annotations

import numpy as np

from oracle.vdn_oracle import frame_stats, transition, vda_states

__all__ = ["readout_backward", "scan_backward", "vda_branch_backward"]


def readout_backward(q_t, s_fwd_t, s_bwd_t, w, eps, do_t):
    """Adjoint of the readout of one frame's tokens.  [P3 方法概述 part 3]

    q_t, do_t: [n, d] queries and the gradient of the ungated branch output;
    s_fwd_t, s_bwd_t: [d, d] states after frame t in the two scans.
    Returns (dq [n, d], dS_fwd [d, d], dS_bwd [d, d], dw [d]).
    """
    q_t = np.asarray(q_t, dtype=np.float64)
    do_t = np.asarray(do_t, dtype=np.float64)
    g = w * do_t
    dq = np.zeros_like(q_t)
    dw = np.zeros(q_t.shape[1])
    ds = []
    for s in (s_fwd_t, s_bwd_t):
        u = q_t @ s.T                                        # row n: S q_n
        rho = np.sqrt(np.mean(u * u, axis=-1, keepdims=True) + eps)
        r = u / rho
        dw += np.sum(r * do_t, axis=0)
        du = (g - r * np.mean(g * r, axis=-1, keepdims=True)) / rho
        dq += du @ s                                         # row n: S^T du_n
        ds.append(du.T @ q_t)                                # sum_n du_n q_n^T
    return dq, ds[0], ds[1], dw


def scan_backward(states, d_states, m, b_mats, gamma, reverse):
    """Adjoint of one scan direction of one (batch, head).  [P3 方法概述 part 2]

    states[t]: S_t of this direction; d_states[t]: gradient of the loss with
    respect to S_t through the readout only; m[t] = (I + A_t)^-1;
    b_mats[t] = B_t.  reverse=False is the forward scan (S_t follows S_{t-1}),
    True the backward scan (S_t follows S_{t+1}).
    Returns (dM [T, d, d], dB [T, d, d], dgamma [T]) of this direction.
    """
    T, d, _ = states.shape
    dM = np.zeros((T, d, d))
    dB = np.zeros((T, d, d))
    dgamma = np.zeros(T)
    # visit the frames against the direction the scan wrote them in
    order = range(T) if reverse else range(T - 1, -1, -1)
    carried = np.zeros((d, d))        # gamma_next * dX_next from the frame written after t
    for t in order:
        prev = t + 1 if reverse else t - 1
        s_prev = states[prev] if 0 <= prev < T else np.zeros((d, d))
        x_t = gamma[t] * s_prev + b_mats[t]
        g_t = d_states[t] + carried
        dx = g_t @ m[t].T
        dM[t] = x_t.T @ g_t
        dB[t] = dx
        dgamma[t] = np.sum(dx * s_prev)
        carried = gamma[t] * dx
    return dM, dB, dgamma


def vda_branch_backward(q, k, v, gamma, beta, rms_w, eps, d_o):
    """Gradient of <d_o, o_l> for the ungated linear-branch output o_l of
    oracle.vdn_oracle.vda_branch.

    q, k, v, d_o: [B, H, T, N, d]; gamma, beta: [B, H, T]; rms_w: [H*d].
    Returns a dict with dq, dk, dv ([B, H, T, N, d]), dgamma, dbeta
    ([B, H, T]) and drms_w ([H*d]), and dbeta_mass ([B, H, T]): the sum of
    the absolute values of the products that make up dbeta, <|dA|, |K^T K|>
    + <|dB|, |V^T K|>.  dbeta can cancel far below that mass, and a
    floating-point evaluation of it carries an error of order unit roundoff
    times the mass (the standard error bound of an inner product).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d_o = np.asarray(d_o, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    rms_w = np.asarray(rms_w, dtype=np.float64)
    B, H, T, N, d = q.shape
    out = {name: np.zeros(q.shape) for name in ("dq", "dk", "dv")}
    out["dgamma"] = np.zeros((B, H, T))
    out["dbeta"] = np.zeros((B, H, T))
    out["dbeta_mass"] = np.zeros((B, H, T))
    out["drms_w"] = np.zeros(H * d)
    for b in range(B):
        for h in range(H):
            kk, vv, gg, bb = k[b, h], v[b, h], gamma[b, h], beta[b, h]
            w_h = rms_w[h * d:(h + 1) * d]
            sf, sb = vda_states(kk, vv, gg, bb)
            stats = [frame_stats(kk[t], vv[t], float(bb[t])) for t in range(T)]
            m = np.stack([transition(a_t) for a_t, _ in stats])
            b_mats = np.stack([b_t for _, b_t in stats])

            dsf = np.zeros((T, d, d))
            dsb = np.zeros((T, d, d))
            for t in range(T):
                dq, dsf[t], dsb[t], dw = readout_backward(q[b, h, t], sf[t], sb[t], w_h, eps,
                                                          d_o[b, h, t])
                out["dq"][b, h, t] = dq
                out["drms_w"][h * d:(h + 1) * d] += dw

            dM_f, dB_f, dg_f = scan_backward(sf, dsf, m, b_mats, gg, reverse=False)
            dM_b, dB_b, dg_b = scan_backward(sb, dsb, m, b_mats, gg, reverse=True)
            dM = dM_f + dM_b
            dB = dB_f + dB_b
            out["dgamma"][b, h] = dg_f + dg_b

            for t in range(T):
                dA = -m[t].T @ dM[t] @ m[t].T
                kt, vt, bt = kk[t], vv[t], float(bb[t])
                out["dk"][b, h, t] = bt * (kt @ (dA + dA.T)) + bt * (vt @ dB[t])
                out["dv"][b, h, t] = bt * (kt @ dB[t].T)
                out["dbeta"][b, h, t] = np.sum(dA * (kt.T @ kt)) + np.sum(dB[t] * (vt.T @ kt))
                out["dbeta_mass"][b, h, t] = (np.sum(np.abs(dA * (kt.T @ kt)))
                                              + np.sum(np.abs(dB[t] * (vt.T @ kt))))
    return out
