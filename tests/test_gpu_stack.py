"""The 370M-style decoder stack (random tokens, every linear on libtj2 with OutControl plans,
fused master pass with OsciReset): linear layers checked inside real training steps.

For sampled linears (a QKV projection, a down projection and the LM head) the stack records the
call's inputs (X, dY, the fp32 masters) and results.  The same library calls on those inputs
reproduce the stack's outputs bit for bit -- in particular the forward codes and the next
backward's operands that the master pass formed -- and the oracle checks them on samples
(tests/_linear_check.py: packed operands bit-exact, Y / dX / dW within 1e-3 relative Frobenius).
The fused master pass (AdamW + OsciReset with the plan) is checked bit-exact against the oracle
across a window end with resets enabled.  Step size: the 370M stack (d 1024, 16 layers, vocab
50304, 8 x 2048 tokens) and a small stack of the same form."""
import numpy as np
import pytest
import torch

from oracle import adamw as oadamw, linear as olinear, osci as oosci, philox, quant

import _helpers as H
from _linear_check import check_linear_sampled

pytestmark = pytest.mark.gpu

tj2 = pytest.importorskip("bit_fully_quantized_amd")
from bit_fully_quantized_amd import decoder  # noqa: E402


def _bits(t):
    return t.detach().cpu().numpy().view(np.uint32)


def _chan(a, oplan):
    """A master-pass state array (compacted channel order: rest, then outlier channels) in channel order."""
    out = np.empty_like(a)
    out[:, np.concatenate([oplan.rest, oplan.outliers])] = a
    return out


def _check_capture(stack, lin, cap, rng):
    """Re-run the captured call through the library, compare with the stack, then with the oracle."""
    X, W, dY = cap["X"], cap["W"], cap["dY"]
    N, K = lin.N, lin.K
    plan = lin.plan
    seed, offset = stack.cfg.seed, cap["offset"]
    assert offset == stack.offset(lin.idx, cap["step"])
    Y, saved = tj2.linear_fwd(X, W, N, plan=plan, y_dtype=torch.bfloat16)
    Y32, _ = tj2.linear_fwd(X, W, N, plan=plan, y_dtype=torch.float32)
    dX, dW, ops = tj2.linear_bwd(dY, saved, K, seed=seed, offset=offset, plan=plan, dx_dtype=torch.bfloat16,
                                 keep_operands=True)
    dX32, _, _ = tj2.linear_bwd(dY, saved, K, seed=seed, offset=offset, plan=plan, dx_dtype=torch.float32)
    torch.cuda.synchronize()
    # the stack computed exactly this: codes from the master pass, re-grouped weights from the master
    # pass (w_given), products and outputs
    for name in ("Xq", "Wq", "X8", "W8"):
        assert torch.equal(saved[name].codes, cap["saved"][name].codes), f"{lin.name}: {name}"
        assert torch.equal(saved[name].scale128, cap["saved"][name].scale128), f"{lin.name}: {name} scales"
    for name in ("dYq", "dYt", "Wt", "Xt", "W8t", "X8t"):
        assert torch.equal(ops[name].codes, cap["ops"][name].codes), f"{lin.name}: {name}"
    assert torch.equal(Y, cap["Y"]) and torch.equal(dX, cap["dX"]) and torch.equal(dW, cap["dW"]), lin.name
    plan_idx = plan.outliers.cpu().numpy().astype(np.int64)
    gpu = dict(saved=saved, ops=ops, Y=Y, dX=dX, dW=dW, Y32=Y32, dX32=dX32)
    return check_linear_sampled(X.float().cpu().numpy(), W.cpu().numpy(), dY.float().cpu().numpy(), plan_idx,
                                seed, offset, gpu, rng, tag=f"{lin.name} step {cap['step']}")


def _run(cfg, steps, capture_names, capture_steps, master_check=None, calib=2):
    torch.manual_seed(0)
    stack = decoder.Decoder(cfg)
    stack.calibrate([decoder.random_tokens(cfg, 100 + b)[0] for b in range(calib)])
    lins = {L.name: L for L in stack.linears}
    rng = np.random.default_rng(0)
    errs, losses = {}, []
    for t in range(steps):
        for n in capture_names:
            lins[n].capture = {} if t in capture_steps else None
        hook = master_check(stack, t) if master_check else None
        tokens, targets = decoder.random_tokens(cfg, t)
        losses.append(float(stack.train_step(tokens, targets, before_update=hook[0] if hook else None)))
        if hook:
            hook[1](stack)
        for n in capture_names:
            if lins[n].capture:
                errs[(n, t)] = _check_capture(stack, lins[n], lins[n].capture, rng)
                lins[n].capture = None
        print(f"[stack] step {t} loss {losses[-1]:.4f} resets {int(stack.reset_count.item())}", flush=True)
    assert all(np.isfinite(losses))
    return stack, errs


def test_small_stack_linears_and_master_pass():
    cfg = decoder.DecoderConfig(vocab=2048, d_model=256, layers=2, heads=4, ffn=1024, seq=256, batch=2,
                                window=2, tau=0.5, reset_lr=1.0, lr_start=2e-3, lr_end=1e-4, total_steps=10)
    checked = {}

    def master_check(stack, t):
        """At the window end (step 1, resets enabled): the fused master pass of two linears against
        the oracle's AdamW + OsciReset with the plan, the codes and the next backward's operands."""
        if t != 1:
            return None
        names = ("0.gate", "head")
        before = {}

        def pre(st):
            for L in st.linears:
                if L.name in names:
                    before[L.name] = [a.detach().cpu().numpy().copy() for a in (L.W, L.m, L.v, L.grad, L.Q_prev,
                                                                                 L.dQ, L.dM)]

        def post(st):
            c = st.cfg
            opt = oadamw.AdamW(lr=c.lr(t), beta1=c.beta1, beta2=c.beta2, eps=c.eps, weight_decay=c.weight_decay)
            bc1, bc2 = np.float32(1.0 - c.beta1 ** (t + 1)), np.float32(1.0 - c.beta2 ** (t + 1))
            for L in st.linears:
                if L.name not in names:
                    continue
                oplan = olinear.Plan.from_outliers(L.K, L.plan.outliers.cpu().numpy())
                W, g = before[L.name][0], before[L.name][3]
                m, v, Qp, dQ, dM = (_chan(before[L.name][i], oplan) for i in (1, 2, 4, 5, 6))
                W2, m2, v2, Qp2, dQ2, dM2, (wq, w8), n = oadamw.master_step(
                    W, m, v, g, Qp, dQ, dM, opt, bc1, bc2, tau=c.tau, window_end=True, reset_enabled=True,
                    plan=oplan)
                np.testing.assert_array_equal(_bits(L.W), W2.view(np.uint32), err_msg=f"{L.name}: W")
                for name, got, ref in (("m", L.m, m2), ("v", L.v, v2), ("Q_prev", L.Q_prev, Qp2), ("dQ", L.dQ, dQ2),
                                       ("dM", L.dM, dM2)):
                    np.testing.assert_array_equal(_chan(got.detach().cpu().numpy(), oplan).view(np.uint32),
                                                  ref.view(np.uint32), err_msg=f"{L.name}: {name}")
                H.assert_q_equal(L.Wq, wq, what=f"{L.name} Wq")
                H.assert_q_equal(L.W8, w8, what=f"{L.name} W8")
                off = st.offset(L.idx, t + 1)
                mask = philox.rht_signs(c.seed, off)
                H.assert_q_equal(L.next.Wt, quant.quantize(quant.dequantize(wq), grouping="col", rounding="sr",
                                                           rht_mask=mask, seed=c.seed, offset=off + 1),
                                 what=f"{L.name} next Wt")
                H.assert_q_equal(L.next.W8t, quant.quantize(quant.dequantize(w8), grouping="col", fmt="fp8",
                                                            rounding="sr", rht_mask=mask, seed=c.seed,
                                                            offset=off + 4), what=f"{L.name} next W8t")
                checked[L.name] = n
        return pre, post

    stack, errs = _run(cfg, 3, ("0.qkv", "1.down", "head"), (0, 1), master_check)
    assert set(checked) == {"0.gate", "head"}
    assert sum(checked.values()) > 0 and int(stack.reset_count.item()) > 0  # resets happened at the window end
    assert len(errs) == 6


def test_370m_stack_sampled_linears():
    cfg = decoder.DecoderConfig()  # the 370M-style stack: 16 layers, d 1024, vocab 50304, 8 x 2048 tokens
    print("[stack] 370M-style stack: calibration, 2 steps, capture 0.qkv / 7.down / head at step 1", flush=True)
    stack, errs = _run(cfg, 2, ("0.qkv", "7.down", "head"), (1,), calib=2)
    assert len(errs) == 3
    for k, e in errs.items():
        print(f"[stack] {k}: rel_fro Y {e['Y']:.2e} dX {e['dX']:.2e} dW {e['dW']:.2e}", flush=True)
