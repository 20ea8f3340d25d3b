"""GPU parity of the linear layer at full workload size (16384 tokens), in the
launch configuration the benchmark times (fp32 masters quantized inside the
forward call, bf16 Y and dX, fp32 dW, caller workspace, RHT on, seed 0).

Workloads: the OLMo-2-70M-style linears (d_model 512, SwiGLU ffn 2048; X
N(0,1) with 0.5% of the channels x32; no outlier plan) and the
OLMo-2-370M-style linears (d_model 1024, ffn 4096; X[t,c] = z * g_c with
lognormal gains sigma 1.5; top-10% channels in FP8 from 8 calibration
batches).  W ~ N(0, 0.02), dY ~ N(0, 0.01).

The oracle computes only what the sampled outputs need (tests/_linear_check.py),
which is exact because every quantizer group is local.  Packed operands are
compared bit for bit on the sampled rows; products on sampled rows x columns
against the fp64 product of the oracle's operands: within 1e-3 relative
Frobenius with fp32 outputs, and the benchmark's bf16 outputs within one bf16
ulp.
"""
import numpy as np
import pytest
import torch

import synthetic
from oracle import calib

import _helpers as H
from _linear_check import check_linear_sampled

pytestmark = pytest.mark.gpu

tj2 = pytest.importorskip("bit_fully_quantized_amd")

SEED = 0
CASES = [("70M", s) for s in synthetic.OLMO70M.linears] + [("370M", s) for s in synthetic.OLMO370M.linears]


def _inputs(family, spec, M, case_seed):
    K, N = spec.K, spec.N
    if family == "70M":
        xb = synthetic.acts_with_outliers_bf16((M, K), 1.0, 0.005, 32.0, synthetic.SEED_X + case_seed)
        plan_idx = None
    else:
        gains = synthetic.lognormal_channel_gains(K, 1.5, synthetic.SEED_GAIN + case_seed)
        xb = synthetic.heavy_tailed_acts_bf16(M, gains, synthetic.SEED_X + case_seed)
        batches = (H.bf16_values(synthetic.heavy_tailed_acts_bf16(M // 8, gains, synthetic.SEED_CALIB + 10 * case_seed + b))
                   for b in range(8))
        plan_idx = calib.select_outliers(calib.channel_scores(batches), 0.10)
    W = synthetic.normal_f32((N, K), 0.02, synthetic.SEED_W + case_seed)
    dyb = synthetic.normal_bf16((M, N), 0.01, synthetic.SEED_DY + case_seed)
    return xb, W, dyb, plan_idx


@pytest.mark.parametrize("family,spec", CASES, ids=[f"{f}-{s.name}" for f, s in CASES])
def test_linear_full_size_sampled(family, spec):
    M, K, N = 16384, spec.K, spec.N
    case_seed = [s.name for s in synthetic.OLMO370M.linears].index(spec.name)
    offset = 8 * (case_seed + 1)
    xb, W, dyb, plan_idx = _inputs(family, spec, M, case_seed)
    print(f"[fullsize] {family} {spec.name} M={M} K={K} N={N} outliers={0 if plan_idx is None else len(plan_idx)}",
          flush=True)
    rng = np.random.default_rng(100 + case_seed)

    # ---------------- GPU, as the benchmark calls it ----------------
    gplan = tj2.OutlierPlan.from_indices(K, plan_idx) if plan_idx is not None else None
    no = 0 if plan_idx is None else len(plan_idx)
    ws = tj2.linear_bwd_workspace(M, N, K, no)
    Y, saved = tj2.linear_fwd(H.bf16_to_device(xb), H.f32_to_device(W), N, plan=gplan, y_dtype=torch.bfloat16)
    dX, dW, ops = tj2.linear_bwd(H.bf16_to_device(dyb), saved, K, seed=SEED, offset=offset, plan=gplan,
                                 dx_dtype=torch.bfloat16, keep_operands=True, workspace=ws)
    # the same kernels with fp32 outputs, for the relative Frobenius bar (bf16 output rounding alone
    # is about 1.7e-3 of it)
    Y32, _ = tj2.linear_fwd(H.bf16_to_device(xb), H.f32_to_device(W), N, plan=gplan, y_dtype=torch.float32)
    dX32, _, _ = tj2.linear_bwd(H.bf16_to_device(dyb), saved, K, seed=SEED, offset=offset, plan=gplan,
                                dx_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()

    # ---------------- oracle on the samples ----------------
    gpu = dict(saved=saved, ops=ops, Y=Y, dX=dX, dW=dW, Y32=Y32, dX32=dX32)
    err = check_linear_sampled(H.bf16_values(xb), W, H.bf16_values(dyb), plan_idx, SEED, offset, gpu, rng,
                               tag=f"{family} {spec.name}")
    print(f"[fullsize] rel_fro Y {err['Y']:.2e} dX {err['dX']:.2e} dW {err['dW']:.2e}", flush=True)
