"""AdamW step on the fp32 masters and the fused master-weight pass (oracle;
test infrastructure only).

The pages train with fp32 master weights and apply OsciReset to them after the
optimizer update (TetraJet-v2 technical summary, section 2.B); they do not name
the optimizer.  The builder's optimizer is AdamW with decoupled weight decay
(Loshchilov and Hutter), defined here operation by operation in fp32 (every
product, sum, quotient and square root rounded to nearest, no fused
multiply-add), for step t with bias corrections bc1 = 1 - beta1^t and
bc2 = 1 - beta2^t given in fp32:

    m' = fl(fl(beta1 * m) + fl(fl(1 - beta1) * g))
    v' = fl(fl(beta2 * v) + fl(fl(1 - beta2) * fl(g * g)))
    u  = fl(fl(m' / bc1) / fl(sqrt(fl(v' / bc2)) + eps))
    W' = fl(fl(W * fl(1 - fl(lr * wd))) - fl(lr * u))

The fused master-weight pass is this step followed by the OsciReset update of
the new masters (oracle.osci.osci_step) in which the previous master W stands
for W_prev: the distance the master travels is the update itself, so W_prev
is not stored.  With the same inputs it equals the unfused sequence "AdamW,
then OsciReset" whenever the stored W_prev equals the pre-update master.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .osci import OsciState, osci_step

f32 = np.float32


@dataclass
class AdamW:
    lr: float
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.1

    def bias_corrections(self, t: int) -> tuple[np.float32, np.float32]:
        """1 - beta1^t and 1 - beta2^t (fp64 powers, rounded once to fp32)."""
        return f32(1.0 - float(self.beta1) ** t), f32(1.0 - float(self.beta2) ** t)


def adamw_step(W, m, v, g, opt: AdamW, bc1, bc2):
    """Returns (W', m', v') in fp32."""
    W, m, v, g = (np.asarray(a, dtype=f32) for a in (W, m, v, g))
    b1, b2, eps, lr, wd = f32(opt.beta1), f32(opt.beta2), f32(opt.eps), f32(opt.lr), f32(opt.weight_decay)
    bc1, bc2 = f32(bc1), f32(bc2)
    omb1, omb2 = f32(f32(1.0) - b1), f32(f32(1.0) - b2)
    m1 = (b1 * m).astype(f32) + (omb1 * g).astype(f32)
    m1 = m1.astype(f32)
    gg = (g * g).astype(f32)
    v1 = ((b2 * v).astype(f32) + (omb2 * gg).astype(f32)).astype(f32)
    mh = (m1 / bc1).astype(f32)
    vh = (v1 / bc2).astype(f32)
    den = (np.sqrt(vh).astype(f32) + eps).astype(f32)
    u = (mh / den).astype(f32)
    decay = f32(f32(1.0) - f32(lr * wd))
    W1 = ((W * decay).astype(f32) - (lr * u).astype(f32)).astype(f32)
    return W1, m1, v1


def master_step(W, m, v, g, Q_prev, dQ, dM, opt: AdamW, bc1, bc2, tau: float, window_end: bool,
                reset_enabled: bool, diag: dict | None = None, plan=None):
    """Fused pass: AdamW, then OsciReset with W_prev = the pre-update master (oscillation
    diagnostics and the OutControl plan as oracle.osci.osci_step).  Returns (W, m, v, Q_prev, dQ,
    dM, codes, number of resets)."""
    W = np.asarray(W, dtype=f32)
    W1, m1, v1 = adamw_step(W, m, v, g, opt, bc1, bc2)
    st = OsciState(W.copy(), np.asarray(Q_prev, dtype=f32), np.asarray(dQ, dtype=f32), np.asarray(dM, dtype=f32))
    W2, st2, Wq, n = osci_step(W1, st, tau, window_end, reset_enabled, diag, plan)
    return W2, m1, v1, st2.Q_prev, st2.dQ, st2.dM, Wq, n
