#!/usr/bin/env python3
"""Benchmark of the TetraJet-v2 NVFP4 linear-layer path on one MI355X.

One step = the whole hot path over one batch of the OLMo-2-370M-style linear
workload: for each of the 16 layers x 5 linears (QKV 1024->3072, O 1024->1024,
gate/up 1024->4096, down 4096->1024) with 16384 tokens,
  forward   RTN quantization of X (NVFP4 + FP8 outlier channels) and of the
            fp32 masters, product on the packed operands;
  backward  SR + Hadamard quantization of dY (both groupings), re-grouping of
            W-hat and X-hat (NVFP4 + FP8 outliers), dX and dW products;
  OsciReset accumulation step on every fp32 master.
Inputs are synthetic and resident in HBM before timing: X[t, c] = z * g_c with
z ~ N(0, 1) and fixed heavy-tailed channel gains g_c = exp(1.5 * zeta_c); the
static FP8 channels are the top 10% of 8 calibration batches; W ~ N(0, 0.02)
fp32; dY ~ N(0, 0.01) bf16.

value = algorithmic product flops per step (6 * M * N * K summed over the
linears) / step time, in TFLOP/s.  Also reported: the product kernel's
roofline (HIP events on its launch stream), the quantizer sweep on the
8192x4096 bf16 tensor (GB/s of algorithmic bytes), OsciReset GB/s, and the CPU
oracle timed on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA, published
SEED = 0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def make_gen(seed):
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return g


class LinearState:
    """Device buffers of one linear layer of the workload.  370M-style (p_outliers > 0): X[t, c] =
    z * g_c with lognormal gains and a static plan from 8 calibration batches; 70M-style
    (p_outliers == 0): X ~ N(0, 1) with 0.5% of the channels x32, no plan."""

    def __init__(self, tj2, layer, spec, M, p_outliers, seed):
        import torch
        self.name, self.K, self.N = spec.name, spec.K, spec.N
        K, N = self.K, self.N
        g = make_gen(seed)
        if p_outliers > 0:
            self.gains = torch.exp(1.5 * torch.randn(K, generator=g, device="cuda"))
        else:
            self.gains = torch.ones(K, device="cuda")
            self.gains[torch.randperm(K, generator=g, device="cuda")[: max(1, round(0.005 * K))]] = 32.0
        self.X = (torch.randn(M, K, generator=g, device="cuda") * self.gains).to(torch.bfloat16)
        self.W = (torch.randn(N, K, generator=g, device="cuda") * 0.02).float().contiguous()
        self.dY = (torch.randn(M, N, generator=g, device="cuda") * 0.01).to(torch.bfloat16)
        self.plan = None
        if p_outliers > 0:
            # static outlier channels from 8 calibration batches (fresh z, same gains)
            from bit_fully_quantized_amd import outcontrol
            calib = ((torch.randn(M // 8, K, generator=g, device="cuda") * self.gains).to(torch.bfloat16)
                     for _ in range(8))
            self.plan = outcontrol.calibrate(calib, p_outliers)
        no = self.plan.n if self.plan is not None else 0
        self.K1 = K - no
        self.Xq = tj2.QTensor(tj2.NVFP4, M, self.K1)
        self.X8 = tj2.QTensor(tj2.FP8, M, no) if no else None
        self.Wq = tj2.QTensor(tj2.NVFP4, N, self.K1)
        self.W8 = tj2.QTensor(tj2.FP8, N, no) if no else None
        self.Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        self.dX = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
        self.dW = torch.empty(N, K, dtype=torch.float32, device="cuda")
        self.state = [torch.empty_like(self.W) for _ in range(4)]
        tj2.osci_reset_step(self.W, *self.state, mode=tj2.OSCI_INIT, plan=self.plan)
        self.saved = None


def run_step(tj2, lins, ws, it):
    for li in lins:
        _, li.saved = tj2.linear_fwd(li.X, li.W, li.N, Wq=li.Wq, W8=li.W8, plan=li.plan, Y=li.Y, Xq=li.Xq,
                                     X8=li.X8)
    for idx in range(len(lins) - 1, -1, -1):
        li = lins[idx]
        tj2.linear_bwd(li.dY, li.saved, li.K, seed=SEED, offset=8 * (it * len(lins) + idx), plan=li.plan,
                       dX=li.dX, dW=li.dW, workspace=ws)
    tj2.osci_reset_step_multi(osci_batch(tj2, lins), mode=tj2.OSCI_ACCUM, tau=4.0)


_OSCI_BATCH = {}


def osci_batch(tj2, lins):
    """The OsciReset descriptors of all linears, built once (one launch per 16 weight matrices), with
    each linear's outlier plan: the state arrays follow the forward's quantizer (FP8 outlier channels,
    NVFP4 over the compacted rest)."""
    key = id(lins)
    if key not in _OSCI_BATCH:
        _OSCI_BATCH[key] = (lins, tj2.OsciBatch([(li.W, *li.state, None, li.plan, None) for li in lins]))
    return _OSCI_BATCH[key][1]


def under_profiler() -> bool:
    """True inside rocprofv3 (its tool library is preloaded into this process and its children)."""
    return "rocprof" in os.environ.get("LD_PRELOAD", "").lower() or any(k.startswith("ROCPROF") for k in os.environ)


def gpu_state_under_load(run, seconds=1.5):
    """GPU clocks, socket power and temperatures (amd-smi, a child process) sampled while `run`
    (untimed steps) keeps the GPU busy; None where amd-smi is missing or fails.  Skipped under a
    profiler: amd-smi is a Python script whose interpreter would start (by exec) inside a child
    that the preloaded profiler library has already attached to the GPU."""
    import subprocess
    import threading

    import torch
    if under_profiler():
        return {"skipped": "under a profiler (amd-smi would start inside its preloaded GPU library)"}
    res = {}

    def sample():
        time.sleep(0.6)  # under load by then
        try:
            out = subprocess.run(["amd-smi", "metric", "-p", "-c", "-t", "--json"], capture_output=True, text=True,
                                 timeout=30)
            res["data"] = json.loads(out.stdout)
        except Exception as e:  # noqa: BLE001 - report, do not fail the benchmark
            res["error"] = str(e)[:200]

    th = threading.Thread(target=sample)
    t_end = time.perf_counter() + seconds
    th.start()
    while th.is_alive() or time.perf_counter() < t_end:
        run()
        torch.cuda.synchronize()
    th.join()
    if "data" not in res:
        return {"error": res.get("error", "no data")}
    try:
        g = res["data"]["gpu_data"][0] if isinstance(res["data"], dict) else res["data"][0]
        val = lambda x: x["value"] if isinstance(x, dict) else None  # noqa: E731
        gfx = [val(v["clk"]) for k, v in g["clock"].items() if k.startswith("gfx_") and isinstance(v, dict)]
        gfx = [c for c in gfx if c is not None]
        return {"what": "amd-smi metric while untimed steps ran right after the timed ones",
                "gfx_clk_mhz_mean": round(sum(gfx) / len(gfx), 1) if gfx else None,
                "gfx_clk_mhz_min_max": [min(gfx), max(gfx)] if gfx else None,
                "mem_clk_mhz": val(g["clock"].get("mem_0", {}).get("clk")) if isinstance(g["clock"].get("mem_0"), dict) else None,
                "socket_power_w": val(g["power"].get("socket_power")),
                "hotspot_c": val(g["temperature"].get("hotspot")), "mem_c": val(g["temperature"].get("mem"))}
    except (KeyError, IndexError, TypeError, ValueError) as e:
        return {"error": f"unexpected amd-smi output: {e}"[:200]}


def time_launches(fn, reps):
    """Average duration (s) of fn() over reps launches, HIP events on the current stream."""
    import torch
    fn()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / 1e3 / reps


def q_bytes(q):
    """Algorithmic bytes of a packed operand: codes, inner and outer scales of its len (not the padding)."""
    per = 0.5 + 1 / 16 + 4 / 128 if q.scale16 is not None else 1 + 4 / 128
    return q.rows * q.len * per


def gemm_roofline(tj2, lins, layers, M, ws, reps=10):
    """Average duration, flops and algorithmic bytes of the product launches of one step
    (one layer's five linears, each product weighted by the number of layers)."""
    tot_flops = 0.0
    tot_time = 0.0
    tot_bytes = 0.0
    launches = 0
    per = {}
    for li in lins[:5]:
        _, _, ops = tj2.linear_bwd(li.dY, li.saved, li.K, seed=SEED, offset=0, plan=li.plan, dX=li.dX, dW=li.dW,
                                   keep_operands=True)
        K, N = li.K, li.N
        calls = product_calls(tj2, li, ops, M, ws)
        for name, fl, by, fn in calls:
            t = time_launches(fn, reps)
            per[f"{li.name}.{name}"] = {"us": round(t * 1e6, 2), "tflops": round(fl / t / 1e12, 1)}
            tot_flops += fl * layers
            tot_time += t * layers
            tot_bytes += by * layers
            launches += layers
    return tot_flops, tot_time, tot_bytes, launches, per


def product_calls(tj2, li, ops, M, ws):
    """The three product launches of one linear's step (as the linear calls issue them):
    (name, flops, algorithmic bytes, launch)."""
    K, N = li.K, li.N
    qb = lambda q: q_bytes(q) if q is not None else 0.0  # noqa: E731
    if li.plan is None:
        return [
            ("fwd", 2.0 * M * N * K, qb(li.Xq) + qb(li.Wq) + 2 * M * N, lambda: tj2.gemm(li.Xq, li.Wq, out=li.Y)),
            ("dX", 2.0 * M * K * N, qb(ops["dYq"]) + qb(ops["Wt"]) + 2 * M * K,
             lambda: tj2.gemm(ops["dYq"], ops["Wt"], out=li.dX, workspace=ws)),
            ("dW", 2.0 * N * K * M, qb(ops["dYt"]) + qb(ops["Xt"]) + 4 * N * K,
             lambda: tj2.gemm(ops["dYt"], ops["Xt"], out=li.dW, workspace=ws)),
        ]
    return [
        ("fwd", 2.0 * M * N * K, qb(li.Xq) + qb(li.Wq) + qb(li.X8) + qb(li.W8) + 2 * M * N,
         lambda: tj2.gemm(li.Xq, li.Wq, li.X8, li.W8, out=li.Y)),
        ("dX", 2.0 * M * K * N, qb(ops["dYq"]) + qb(ops["Wt"]) + qb(ops["W8t"]) + 2 * M * K,
         lambda: tj2.gemm_outlier_cols(ops["dYq"], ops["Wt"], ops["W8t"], li.plan, out=li.dX, workspace=ws)),
        ("dW", 2.0 * N * K * M, qb(ops["dYt"]) + qb(ops["Xt"]) + qb(ops["X8t"]) + 4 * N * K,
         lambda: tj2.gemm_outlier_cols(ops["dYt"], ops["Xt"], ops["X8t"], li.plan, out=li.dW, workspace=ws)),
    ]


def quantizers_in_step(tj2, lins, layers, M, ws, reps=10):
    """Quantizer rates in the step's own launch configuration, from one layer's linears (weighted by
    the number of layers): the forward's quantization of X = (nvfp4_linear_fwd with given weight codes)
    - (its product alone); the backward's quantizers (the fused two-grouping pass of dY and the
    launch of the other column re-groupings) = nvfp4_linear_bwd - (its two products alone).  Algorithmic bytes: inputs read once,
    packed outputs written once."""
    import torch
    per = 0.5 + 1 / 16 + 4 / 128  # NVFP4 bytes per element
    p8 = 1 + 4 / 128              # FP8
    fwd_t = fwd_b = bwd_t = bwd_b = dual_t = dual_b = 0.0
    for li in lins[:5]:
        M_, K, N = M, li.K, li.N
        no = li.plan.n if li.plan is not None else 0
        K1 = K - no
        ops = tj2.bwd_operands(M_, N, K, li.plan)
        _, saved = tj2.linear_fwd(li.X, None, N, Wq=li.Wq, W8=li.W8, plan=li.plan, Y=li.Y, Xq=li.Xq, X8=li.X8)
        t_fwd = time_launches(lambda: tj2.linear_fwd(li.X, None, N, Wq=li.Wq, W8=li.W8, plan=li.plan, Y=li.Y,
                                                     Xq=li.Xq, X8=li.X8), reps)
        calls = product_calls(tj2, li, ops, M_, ws)
        # the forward product as linear_fwd runs it with the weight codes given (no masters to write an
        # image from, so the direct kernel, without a workspace)
        if li.plan is not None:
            t_prod_fwd = time_launches(lambda: tj2.gemm(li.Xq, li.Wq, li.X8, li.W8, out=li.Y, split_k=False), reps)
        else:
            t_prod_fwd = time_launches(lambda: tj2.gemm(li.Xq, li.Wq, out=li.Y, split_k=False), reps)
        t_bwd = time_launches(lambda: tj2.linear_bwd(li.dY, saved, K, seed=SEED, offset=0, plan=li.plan, dX=li.dX,
                                                     dW=li.dW, operands=ops, workspace=ws), reps)
        t_prod_bwd = time_launches(calls[1][3], reps) + time_launches(calls[2][3], reps)
        # the fused dY pass alone (both groupings from one read), into the step's operand buffers
        dual_t += layers * time_launches(lambda: tj2.quantize_dual(li.dY, seed=SEED, row_offset=0, col_offset=2,
                                                                   row_out=ops["dYq"], col_out=ops["dYt"]), reps)
        dual_b += layers * (2.0 * M_ * N + 2 * M_ * N * per)
        fwd_t += layers * max(t_fwd - t_prod_fwd, 0.0)
        fwd_b += layers * (2.0 * M_ * K + M_ * K1 * per + M_ * no * p8)
        bwd_t += layers * max(t_bwd - t_prod_bwd, 0.0)
        # dY read once into both groupings; W-hat, X-hat (and the FP8 slices) re-grouped: read
        # packed, write packed
        bwd_b += layers * (2.0 * M_ * N + 2 * M_ * N * per + 2 * N * K1 * per + 2 * M_ * K1 * per
                           + 2 * (N + M_) * no * p8)
        del ops
    torch.cuda.empty_cache()
    out = {}
    for name, t, b in (("forward_X", fwd_t, fwd_b), ("backward_all", bwd_t, bwd_b), ("backward_dY_dual", dual_t, dual_b),
                       ("backward_regroupings", max(bwd_t - dual_t, 0.0), bwd_b - dual_b)):
        gbs = b / t / 1e9 if t > 0 else 0.0
        out[name] = {"ms_per_step": round(t * 1e3, 3), "GB_per_step": round(b / 1e9, 2), "GB_s": round(gbs, 1),
                     "frac_hbm": round(gbs / HBM_PEAK_GBS, 3)}
    return out


def fp6_backward(tj2, lins, layers, M, ws, reps=5):
    """The FP6 x FP4 variant at the 370M shapes: the backward of one layer's five linears (weighted by
    the number of layers) with FP4 and with FP6 gradient operands (nvfp6x4_linear_bwd), ms per step."""
    import torch
    out = {}
    for name, fmt in (("fp4_grads", tj2.NVFP4), ("fp6_grads", tj2.NVFP6)):
        t = 0.0
        for li in lins[:5]:
            ops = tj2.bwd_operands(M, li.N, li.K, li.plan, grad_fmt=fmt)
            t += layers * time_launches(lambda: tj2.linear_bwd(li.dY, li.saved, li.K, seed=SEED, offset=0, plan=li.plan,
                                                               dX=li.dX, dW=li.dW, operands=ops, workspace=ws,
                                                               grad_fmt=fmt), reps)
            del ops
        out[name] = {"bwd_ms_per_step": round(t * 1e3, 3)}
    torch.cuda.empty_cache()
    out["fp6_over_fp4_time"] = round(out["fp6_grads"]["bwd_ms_per_step"] / out["fp4_grads"]["bwd_ms_per_step"], 3)
    return out


def single_linear_latency(tj2, reps=50):
    """The single-linear workload (X 256x512, W 512x512 fp32 masters, dY 256x512; RHT on, seed 0): latency
    of the forward (quantizers + product), the backward and one OsciReset window-end step, in us."""
    import torch
    import synthetic
    wl = synthetic.SINGLE_LINEAR
    M, K, N = wl.M, wl.linears[0].K, wl.linears[0].N
    g = make_gen(3)
    X = torch.randn(M, K, generator=g, device="cuda").to(torch.bfloat16)
    W = (torch.randn(N, K, generator=g, device="cuda") * 0.02).contiguous()
    dY = (torch.randn(M, N, generator=g, device="cuda") * 0.01).to(torch.bfloat16)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    Xq, Wq = tj2.QTensor(tj2.NVFP4, M, K), tj2.QTensor(tj2.NVFP4, N, K)
    dX = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    dW = torch.empty(N, K, dtype=torch.float32, device="cuda")
    ws = tj2.linear_bwd_workspace(M, N, K)
    fws = tj2.linear_fwd_workspace(M, N, K)
    _, saved = tj2.linear_fwd(X, W, N, Y=Y, Xq=Xq, Wq=Wq, workspace=fws)
    t_fwd = time_launches(lambda: tj2.linear_fwd(X, W, N, Y=Y, Xq=Xq, Wq=Wq, workspace=fws), reps)
    t_bwd = time_launches(lambda: tj2.linear_bwd(dY, saved, K, seed=0, offset=0, dX=dX, dW=dW, workspace=ws), reps)
    st = [torch.empty_like(W) for _ in range(4)]
    Wm = W.clone()
    tj2.osci_reset_step(Wm, *st, mode=tj2.OSCI_INIT)
    t_osci = time_launches(lambda: tj2.osci_reset_step(Wm, *st, mode=tj2.OSCI_WINDOW_END, tau=4.0,
                                                       reset_enabled=True, Wq_out=Wq), reps)
    flops = 2.0 * M * N * K
    return {"workload": wl.name, "fwd_us": round(t_fwd * 1e6, 2), "bwd_us": round(t_bwd * 1e6, 2),
            "osci_reset_window_end_us": round(t_osci * 1e6, 2),
            "fwd_bwd_tflops": round(3 * flops / (t_fwd + t_bwd) / 1e12, 2)}


def olmo70m_rates(tj2, reps=10, steps=5):
    """OLMo-2-70M-style linears (8 layers x QKV/O/gate/up/down, d 512, ffn 2048, 16384 tokens, no plan):
    whole-step TFLOP/s (forward + backward of all 40 linears) and per-product TFLOP/s."""
    import torch
    import synthetic
    wl = synthetic.OLMO70M
    M, layers = wl.M, wl.layers
    lins = [LinearState(tj2, l, spec, M, 0.0, seed=500 + 10 * l + j)
            for l in range(layers) for j, spec in enumerate(wl.linears)]
    ws = torch.empty(max(int(tj2.lib().nvfp4_linear_bwd_workspace_size(M, li.N, li.K, 0)) for li in lins),
                     dtype=torch.uint8, device="cuda")

    def step(it):
        for li in lins:
            _, li.saved = tj2.linear_fwd(li.X, li.W, li.N, Wq=li.Wq, Y=li.Y, Xq=li.Xq)
        for idx in range(len(lins) - 1, -1, -1):
            li = lins[idx]
            tj2.linear_bwd(li.dY, li.saved, li.K, seed=SEED, offset=8 * (it * len(lins) + idx), dX=li.dX, dW=li.dW,
                           workspace=ws)

    step(0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for it in range(steps):
        step(1 + it)
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / steps
    flops = wl.gemm_flops_per_step()
    per = {}
    g_flops = g_time = 0.0
    for li in lins[:5]:
        _, _, ops = tj2.linear_bwd(li.dY, li.saved, li.K, seed=SEED, offset=0, dX=li.dX, dW=li.dW,
                                   keep_operands=True, workspace=ws)
        for name, fl, _, fn in product_calls(tj2, li, ops, M, ws):
            t = time_launches(fn, reps)
            per[f"{li.name}.{name}"] = round(fl / t / 1e12, 1)
            g_flops += fl * layers
            g_time += t * layers
    del lins, ws
    torch.cuda.empty_cache()
    return {"workload": "OLMo-2-70M-style linears: d_model 512, SwiGLU ffn 2048, 8 layers x (QKV, O, gate, up, "
                        "down), 16384 tokens/step, 0.5% channels x32, no outlier plan",
            "ms_per_step": round(step_s * 1e3, 3), "tflops_step": round(flops / step_s / 1e12, 1),
            "gemm_tflop_per_step": round(flops / 1e12, 3), "products_tflops": round(g_flops / g_time / 1e12, 1),
            "products_frac_of_peak": round(g_flops / g_time / 1e12 / MFMA_F16_PEAK_TFLOPS, 3),
            "per_product_tflops": per}


def decoder_stack(steps=3, warmup=2):
    """The 370M-style decoder stack (vocab 50304, 8 x 2048 random tokens, 16 layers; all linears NVFP4 with
    OutControl plans; fused master pass with OsciReset, window 50, LR decaying 1e-4 -> 1e-6), ms per training
    step, and the same stack with bf16 linears (torch.mm / hipBLASLt, AdamW on the masters) as comparator."""
    import torch
    from bit_fully_quantized_amd import decoder
    out = {}
    for kind in ("nvfp4", "bf16"):
        cfg = decoder.DecoderConfig(linear=kind)
        stack = decoder.Decoder(cfg)
        stack.calibrate([decoder.random_tokens(cfg, 100 + b)[0] for b in range(2)])
        batches = [decoder.random_tokens(cfg, b) for b in range(steps + warmup)]
        for b in range(warmup):
            stack.train_step(*batches[b])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for b in range(warmup, warmup + steps):
            loss = stack.train_step(*batches[b])
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / steps * 1e3
        r = {"ms_per_step": round(ms, 2), "loss": round(float(loss), 4),
             "linear_tflops_over_step": round(cfg.linear_flops_per_step() / (ms * 1e-3) / 1e12, 1)}
        if kind == "nvfp4":
            lr = cfg.lr(stack.step)
            t = time_launches(lambda: tj2_master_pass(stack, lr), 2)
            n = stack.linear_params()
            r.update({"master_pass_ms": round(t * 1e3, 3), "linear_params": n,
                      "master_pass_GB_s": round(n * 52.0 / t / 1e9, 1),
                      "resets": int(stack.reset_count.item())})
        out[kind] = r
        del stack, batches
        torch.cuda.empty_cache()
    out["workload"] = ("OLMo-2-370M-style decoder stack: vocab 50304, d_model 1024, 16 layers, 16 heads, SwiGLU ffn "
                       "4096, 8 x 2048 random tokens; pre-norm RMSNorm, RoPE, causal bf16 flash attention, "
                       "cross-entropy; every linear NVFP4 with top-10% FP8 channels; AdamW + OsciReset (window 50)")
    out["linear_tflop_per_step"] = round(decoder.DecoderConfig().linear_flops_per_step() / 1e12, 3)
    out["bf16_over_nvfp4_step_time"] = round(out["bf16"]["ms_per_step"] / out["nvfp4"]["ms_per_step"], 3)
    return out


def tj2_master_pass(stack, lr):
    """One fused master pass over the stack's linears (ACCUM), as its training step issues it."""
    import bit_fully_quantized_amd as tj2
    c = stack.cfg
    tj2.master_update_step_multi(stack.master_batch, lr=lr, bias_correction1=0.5, bias_correction2=0.5,
                                 beta1=c.beta1, beta2=c.beta2, eps=c.eps, weight_decay=c.weight_decay,
                                 mode=tj2.OSCI_ACCUM, tau=c.tau)


def stream_reference(n, reps=3):
    """HBM rate (GB/s) of the OsciReset and master passes' access pattern without their arithmetic
    (libtj2_measure's tj2_stream_probe) over n fp32 elements per array."""
    import torch
    import bit_fully_quantized_amd as tj2
    bufs = [torch.zeros(n, dtype=torch.float32, device="cuda") for _ in range(13)]
    res = {}
    for name, ns, nd in (("osci_5r4w", 5, 4), ("master_7r6w", 7, 6)):
        src, dst = bufs[:ns], bufs[7:7 + nd]
        nbytes = tj2.stream_probe(src, dst)
        t = time_launches(lambda: tj2.stream_probe(src, dst), reps)
        res[name] = round(nbytes / t / 1e9, 1)
    del bufs
    torch.cuda.empty_cache()
    return res


def copy_calibration(nbytes=1 << 30, reps=3):
    """A plain elementwise copy kernel of known size (bf16 negation, 1 GiB read + 1 GiB written per launch).

    Under `rocprofv3 --pmc FETCH_SIZE` / `WRITE_SIZE` its per-dispatch counters give the factor between
    the counters and bytes moved, which scales the product kernel's counters into HBM bytes."""
    import torch
    x = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    for _ in range(reps):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    del x, y
    torch.cuda.empty_cache()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "products_olmo370m_linears_traffic.txt")
GEMM_SOURCES = [os.path.join(ROOT, "bit_fully_quantized_amd", "csrc", f)
                for f in ("gemm.hip", "tj2_device.h", "tj2_internal.h")]


def gemm_source_hash():
    """Hash of the product kernel's code: its sources with // comments and blank lines removed,
    so that a change of comments alone does not invalidate the counter summary."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(f, encoding="utf-8") as fh:
            for line in fh:
                code = re.sub(r"//.*", "", line).rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per product launch from the committed counter summary, or None when it is missing or
    was taken on a different version of the product kernel's sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256_16") != gemm_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def quant_sweep(tj2, reps=24, nbuf=8):
    """8192x4096 bf16 N(0,1), 1% of columns x64; buffers rotated to defeat the 256 MB last-level cache."""
    import torch
    import synthetic
    R, C = synthetic.QUANT_SWEEP_SHAPE
    g = make_gen(77)
    cols = torch.randperm(C, generator=g, device="cuda")[: round(0.01 * C)]
    xs = []
    for _ in range(nbuf):
        x = torch.randn(R, C, generator=g, device="cuda")
        x[:, cols] *= 64.0
        xs.append(x.to(torch.bfloat16))
    outs_r = [tj2.QTensor(tj2.NVFP4, R, C) for _ in range(nbuf)]
    outs_c = [tj2.QTensor(tj2.NVFP4, C, R) for _ in range(nbuf)]
    bytes_per_call = R * C * (2 + 0.5 + 1 / 16 + 4 / 128)  # read bf16; write codes, E4M3, FP32 scales
    signs = tj2.rht_signs(0, 0)
    variants = {
        "row_rtn": dict(grouping=tj2.GROUP_ROW, rounding=tj2.RTN, rht=False),
        "row_sr": dict(grouping=tj2.GROUP_ROW, rounding=tj2.SR, rht=False),
        "row_sr_rht": dict(grouping=tj2.GROUP_ROW, rounding=tj2.SR, rht=True),
        "col_rtn": dict(grouping=tj2.GROUP_COL, rounding=tj2.RTN, rht=False),
        "col_sr_rht": dict(grouping=tj2.GROUP_COL, rounding=tj2.SR, rht=True),
    }
    res = {}
    for name, kw in variants.items():
        outs = outs_r if kw["grouping"] == tj2.GROUP_ROW else outs_c
        state = {"i": 0}

        def fn():
            i = state["i"] % nbuf
            state["i"] += 1
            tj2.quantize(xs[i], signs=signs, seed=0, offset=i, out=outs[i], **kw)

        t = time_launches(fn, reps)
        gbs = bytes_per_call / t / 1e9
        res[name] = {"us": round(t * 1e6, 2), "GB_s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 3)}
    # the fused pass of the backward's output gradient: both groupings (SR + RHT) from one read;
    # algorithmic bytes: one read, both outputs written
    state = {"i": 0}

    def dual_fn():
        i = state["i"] % nbuf
        state["i"] += 1
        tj2.quantize_dual(xs[i], rht=True, seed=0, row_offset=2 * i, col_offset=2 * i + 1, row_out=outs_r[i],
                          col_out=outs_c[i])

    t = time_launches(dual_fn, reps)
    dual_bytes = R * C * (2 + 2 * (0.5 + 1 / 16 + 4 / 128))
    gbs = dual_bytes / t / 1e9
    sep = res["row_sr_rht"]["us"] + res["col_sr_rht"]["us"]
    res["dual_sr_rht"] = {"what": "both groupings (SR + RHT) from one read, as the backward quantizes dY",
                          "us": round(t * 1e6, 2), "GB_s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 3),
                          "separate_row_plus_col_us": round(sep, 2)}
    # achievable reference on the same rotated buffers: a plain elementwise copy (bf16 negation,
    # 64 MiB read + 64 MiB written per call), and each variant's rate as a fraction of it
    ys = [torch.empty_like(xs[0]) for _ in range(2)]
    state = {"i": 0}

    def copy_fn():
        i = state["i"]
        state["i"] += 1
        torch.neg(xs[i % nbuf], out=ys[i % 2])

    t = time_launches(copy_fn, reps)
    copy_gbs = 2 * xs[0].numel() * 2 / t / 1e9
    res["copy_reference"] = {"what": "torch bf16 negation on the same buffers (read + write)", "us": round(t * 1e6, 2),
                             "GB_s": round(copy_gbs, 1), "frac_hbm": round(copy_gbs / HBM_PEAK_GBS, 3)}
    for name in list(variants) + ["dual_sr_rht"]:
        res[name]["frac_of_copy"] = round(res[name]["GB_s"] / copy_gbs, 3)
    del xs, ys, outs_r, outs_c
    torch.cuda.empty_cache()
    return res, bytes_per_call


def library_gemm_reference(M, shapes, reps=10):
    """Achievable dense f16-class MFMA rate on this part, as the vendor library reaches it: torch's bf16
    matrix product (hipBLASLt) on plain contiguous operands of the workload's forward shapes."""
    import torch
    g = make_gen(5)
    res, flops, secs = {}, 0.0, 0.0
    for name, K, N in shapes:
        a = torch.randn(M, K, generator=g, device="cuda").to(torch.bfloat16)
        b = torch.randn(K, N, generator=g, device="cuda").to(torch.bfloat16).contiguous()
        c = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        t = time_launches(lambda: torch.mm(a, b, out=c), reps)
        res[name] = round(2.0 * M * N * K / t / 1e12, 1)
        flops += 2.0 * M * N * K
        secs += t
        del a, b, c
    torch.cuda.empty_cache()
    return res, flops / secs / 1e12


def mfma_reference(reps=3):
    """Achievable dense f16 MFMA rate of the part: the library's MFMA-only measurement loop
    (four independent v_mfma_f32_32x32x16_f16 chains per wave, 2048 workgroups), TFLOP/s."""
    import torch
    import bit_fully_quantized_amd as tj2
    out = torch.empty(2048 * 256, dtype=torch.float32, device="cuda")
    flops = tj2.mfma_peak_probe(out, 1024)
    t = time_launches(lambda: tj2.mfma_peak_probe(out, 1024), reps)
    return flops / t / 1e12


def decode_placement(reps=3):
    """The product's inner loop (no global memory) with B decoded once per workgroup into f16 LDS
    (the product kernel's placement) and with packed B in LDS decoded by every wave after its LDS
    reads: MFMA TFLOP/s of each (libtj2_measure's tj2_decode_probe, 1024 workgroups)."""
    import torch
    import bit_fully_quantized_amd as tj2
    out = torch.empty(1024 * 512, dtype=torch.float32, device="cuda")
    res = {}
    for name, packed in (("b_f16_in_lds", False), ("b_packed_in_lds", True)):
        flops = tj2.decode_probe(out, 256, packed)
        t = time_launches(lambda: tj2.decode_probe(out, 256, packed), reps)
        res[name] = round(flops / t / 1e12, 1)
    return res


def cpu_baseline(M=8192, K=1024, N=3072, p=0.10):
    """The oracle (fp64 products, numpy quantizers) on one QKV-shaped linear with M tokens."""
    import numpy as np
    from threadpoolctl import threadpool_info
    import synthetic
    from oracle import calib as ocalib, linear as olinear
    gains = synthetic.lognormal_channel_gains(K, 1.5, 11)
    X = synthetic.bf16_bits_to_f32(synthetic.heavy_tailed_acts_bf16(M, gains, 12))
    W = synthetic.normal_f32((N, K), 0.02, 13)
    dY = synthetic.bf16_bits_to_f32(synthetic.normal_bf16((M, N), 0.01, 14))
    plan = olinear.Plan.from_outliers(K, ocalib.select_outliers(ocalib.channel_scores([X]), p))
    t0 = time.perf_counter()
    fwd = olinear.linear_fwd(X, W, plan)
    olinear.linear_bwd(dY, fwd, seed=0, offset=0, plan=plan)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    flops = 6.0 * M * N * K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"one QKV-shaped linear (K={K}, N={N}) with M={M} tokens and {plan.outliers.size} FP8 "
                      f"outlier channels: forward + backward incl. every quantizer, fp64 products; "
                      f"{dt:.2f} s for {flops / 1e9:.2f} GFLOP",
            "seconds": round(dt, 2), "host_cpus": len(os.sched_getaffinity(0)),
            "components": cpu_components()}


def cpu_components(rows=8192):
    """The oracle's quantizers (numpy element-wise, one thread) on the quantizer sweep tensor (8192
    rows: in full), its OsciReset accumulate step on 1024x1024 masters, and the single-linear workload
    end to end (forward, backward, one window-end OsciReset)."""
    import numpy as np
    import synthetic
    from oracle import linear as olinear, osci as oosci, quant as oquant
    out = {}
    C = synthetic.QUANT_SWEEP_SHAPE[1]
    x = synthetic.bf16_bits_to_f32(synthetic.acts_with_outliers_bf16((rows, C), 1.0, 0.01, 64.0, 21))
    for name, kw in (("row_rtn", {}), ("row_sr_rht", {"rounding": "sr", "rht_mask": 0x5A5A, "seed": 0, "offset": 0})):
        t0 = time.perf_counter()
        oquant.quantize(x, grouping="row", fmt="nvfp4", **kw)
        dt = time.perf_counter() - t0
        out[f"quantizer_{name}"] = {"elements_per_s": round(rows * C / dt), "GB_s": round(rows * C * 2.59375 / dt / 1e9, 4),
                                    "sample": f"{rows}x{C} bf16 (the sweep recipe)", "seconds": round(dt, 2)}
    W = synthetic.normal_f32((1024, 1024), 0.02, 22)
    st, _ = oosci.osci_init(W)
    W1 = W - np.float32(1e-4) * synthetic.normal_f32((1024, 1024), 1.0, 23)
    t0 = time.perf_counter()
    oosci.osci_step(W1, st, 4.0, False, False)
    dt = time.perf_counter() - t0
    out["osci_reset_accum"] = {"params_per_s": round(W.size / dt), "GB_s": round(W.size * 36.0 / dt / 1e9, 4),
                               "sample": "1024x1024 fp32 masters", "seconds": round(dt, 2)}
    X = synthetic.bf16_bits_to_f32(synthetic.normal_bf16((256, 512), 1.0, 24))
    Wm = synthetic.normal_f32((512, 512), 0.02, 25)
    dY = synthetic.bf16_bits_to_f32(synthetic.normal_bf16((256, 512), 0.01, 26))
    t0 = time.perf_counter()
    fwd = olinear.linear_fwd(X, Wm)
    bwd = olinear.linear_bwd(dY, fwd, seed=0, offset=0)
    st0, _ = oosci.osci_init(Wm)
    oosci.osci_step(Wm - np.float32(1e-4) * bwd["dW"], st0, 4.0, True, True)
    out["single_linear_end_to_end_s"] = round(time.perf_counter() - t0, 3)
    out["threads"] = "quantizers and OsciReset: numpy element-wise (one thread); products: BLAS (cores above)"
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-stack", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the timed 370M-style steps and the product roofline pass (for a kernel trace whose "
                         "product launches are exactly the headline workload's)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; multi-GPU figures are not produced",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import bit_fully_quantized_amd as tj2
    import synthetic

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    wl = synthetic.OLMO370M
    M, layers = wl.M, wl.layers
    log(f"setting up {wl.name}: {layers} layers x {len(wl.linears)} linears, M={M}")
    lins = []
    for l in range(layers):
        for j, spec in enumerate(wl.linears):
            lins.append(LinearState(tj2, l, spec, M, 0.10, seed=1000 * l + j))
    max_ws = max(int(tj2.lib().nvfp4_linear_bwd_workspace_size(M, li.N, li.K, li.plan.n)) for li in lins)
    ws = torch.empty(max_ws, dtype=torch.uint8, device="cuda")
    flops_step = wl.gemm_flops_per_step()
    torch.cuda.synchronize()
    log(f"setup done; warmup {args.warmup} steps")

    for it in range(args.warmup):
        run_step(tj2, lins, ws, it)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for it in range(args.steps):
        run_step(tj2, lins, ws, args.warmup + it)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_s = wall / args.steps
    step_ev = ev0.elapsed_time(ev1) / 1e3 / args.steps
    log(f"step {step_s * 1e3:.2f} ms (events {step_ev * 1e3:.2f} ms)")
    gpu_state = None
    if not args.headline_only:
        log("clocks and power under the step's load")
        n_extra = [0]

        def extra_step():
            run_step(tj2, lins, ws, args.warmup + args.steps + n_extra[0])
            n_extra[0] += 1
        gpu_state = gpu_state_under_load(extra_step)

    log("product roofline pass")
    g_flops, g_time, g_bytes, g_launches, per = gemm_roofline(tj2, lins, layers, M, ws)
    achieved = g_flops / g_time / 1e12
    if args.headline_only:
        print(json.dumps({"metric": "NVFP4 linear fwd+bwd TFLOP/s at 370M shapes", "value": round(flops_step / step_s / 1e12, 2),
                          "unit": "TFLOP/s", "ms_per_step": round(step_s * 1e3, 3), "steps": args.steps,
                          "roofline_achieved_tflops": round(achieved, 1),
                          "roofline_frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
                          "avg_launch_us": round(g_time / g_launches * 1e6, 2),
                          "gemm_gflop_per_launch": round(g_flops / g_launches / 1e9, 3)}), flush=True)
        return
    log("quantizers in the step's launch configuration")
    q_in_step = quantizers_in_step(tj2, lins, layers, M, ws)
    log("FP6 x FP4 backward")
    fp6 = fp6_backward(tj2, lins, layers, M, ws)
    copy_calibration()
    log("OsciReset pass")
    n_params = sum(li.N * li.K for li in lins)
    osci_t = time_launches(lambda: tj2.osci_reset_step_multi(osci_batch(tj2, lins), mode=tj2.OSCI_ACCUM, tau=4.0),
                           3)
    osci_bytes = n_params * 36.0  # read W, W_prev, Q_prev, dQ, dM; write W_prev, Q_prev, dQ, dM (fp32)
    log("fused master-weight pass")
    for li in lins:
        li.m, li.v = torch.zeros_like(li.W), torch.zeros_like(li.W)
    master_batch = tj2.MasterBatch([(li.W, li.m, li.v, li.dW, *li.state[1:], None) for li in lins])
    master_t = time_launches(lambda: tj2.master_update_step_multi(master_batch, lr=1e-6, bias_correction1=0.1,
                                                                  bias_correction2=0.05, mode=tj2.OSCI_ACCUM,
                                                                  tau=4.0), 3)
    # read W, m, v, grad, Q_prev, dQ, dM; write W, m, v, Q_prev, dQ, dM (fp32)
    master_bytes = n_params * 52.0
    master_plan_batch = tj2.MasterBatch([(li.W, li.m, li.v, li.dW, *li.state[1:], None, li.plan, None, None)
                                         for li in lins])
    master_plan_t = time_launches(lambda: tj2.master_update_step_multi(master_plan_batch, lr=1e-6,
                                                                       bias_correction1=0.1, bias_correction2=0.05,
                                                                       mode=tj2.OSCI_ACCUM, tau=4.0), 3)
    log("OsciReset / master access-pattern reference")
    pattern = stream_reference(n_params)
    log("oscillation diagnostics")
    flips = torch.zeros(1, dtype=torch.int64, device="cuda")
    hist = torch.zeros(tj2.RISK_BINS, dtype=torch.int64, device="cuda")

    def master_diag(mode, h):
        tj2.master_update_step_multi(master_batch, lr=1e-6, bias_correction1=0.1, bias_correction2=0.05, mode=mode,
                                     tau=4.0, flips=flips, risk_hist=h)

    diag_accum_t = time_launches(lambda: master_diag(tj2.OSCI_ACCUM, None), 3)
    flips.zero_()
    master_diag(tj2.OSCI_ACCUM, None)
    flips_per_pass = int(flips.item())
    hist.zero_()
    master_diag(tj2.OSCI_WINDOW_END, hist)  # the window so far: every master pass since the state's INIT
    risk_hist = [int(x) for x in hist.cpu().tolist()]
    diag_end_t = time_launches(lambda: master_diag(tj2.OSCI_WINDOW_END, hist), 2)
    del lins, ws
    torch.cuda.empty_cache()

    log("single-linear latency")
    single = single_linear_latency(tj2)
    log("70M-style linears")
    olmo70 = olmo70m_rates(tj2)
    stack = None
    if not args.no_stack:
        log("370M-style decoder stack (NVFP4 linears, then bf16 comparator)")
        stack = decoder_stack()
    log("MFMA-only reference loop")
    mfma_ach = mfma_reference()
    log("decode placement probe")
    placement = decode_placement()
    log("library bf16 product reference")
    lib_ref, lib_all = library_gemm_reference(M, [(f"{spec.name}.fwd", spec.K, spec.N) for spec in wl.linears])
    sweep, sweep_bytes = ({}, 0) if args.no_sweep else quant_sweep(tj2)
    copy_ref = sweep.get("copy_reference", {}).get("GB_s")
    for v in q_in_step.values():  # fraction of the copy reference measured on the sweep buffers
        if isinstance(v, dict) and "GB_s" in v:
            v["frac_of_copy"] = round(v["GB_s"] / copy_ref, 3) if copy_ref else None
    cpu = None if args.no_cpu_baseline else cpu_baseline()

    out = {
        "metric": "NVFP4 linear fwd+bwd TFLOP/s at 370M shapes; quantizer GB/s (% of peak)",
        "value": round(flops_step / step_s / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",  # MFMA arithmetic on exactly decoded NVFP4/FP8 operands, fp32 accumulation
        "data": "synthetic",
        "config": {
            "workload": "OLMo-2-370M-style linears: d_model 1024, SwiGLU ffn 4096, 16 layers x "
                        "(QKV, O, gate, up, down), 16384 tokens/step, heavy-tailed channels "
                        "(lognormal sigma 1.5), OutControl top-10% FP8 channels, OsciReset accumulate",
            "tokens": M, "layers": layers, "linears": len(wl.linears) * layers,
            "gemm_tflop_per_step": round(flops_step / 1e12, 3), "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": "the products, each called on its own (gemm_img_kernel: dX and dW of >= 2048 output rows "
                      "with B from f16 images in LDS; gemm_nt_kernel: fwd with the FP8 segment, the other dW); a call "
                      "includes its split-K reduction and its B decode pass (in the step the quantizations that "
                      "produce B write the images, and the forward runs gemm_img2_kernel from the image the "
                      "weights' split quantization writes)",
            "bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4), "traffic": measured_traffic(),
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-kernel scaled)",
            "algorithmic_bytes_per_launch": round(g_bytes / g_launches),
            "avg_launch_us": round(g_time / g_launches * 1e6, 2), "launches_per_step": g_launches,
            "gemm_share_of_step": round(g_time / step_s, 3), "per_launch": per,
            "achievable_mfma": {"what": "MFMA-only loop (v_mfma_f32_32x32x16_f16, register operands) on this part",
                                "TFLOP_s": round(mfma_ach, 1), "frac_of_peak": round(mfma_ach / MFMA_F16_PEAK_TFLOPS, 3),
                                "products_frac_of_it": round(achieved / mfma_ach, 3)},
            "decode_placement": {"what": "the products' inner loop without global memory (tj2_decode_probe), MFMA "
                                         "TFLOP/s with B decoded once per workgroup into f16 LDS vs packed B in "
                                         "LDS decoded by every wave", **placement},
            "library_bf16_reference": {"what": "torch.mm bf16 (hipBLASLt) on plain operands of each linear's "
                                               "forward shape, TFLOP/s: the achievable dense rate as a vendor "
                                               "library reaches it, without decode or per-128 promotion",
                                       "per_shape": lib_ref, "all_shapes": round(lib_all, 1),
                                       "frac_of_peak": round(lib_all / MFMA_F16_PEAK_TFLOPS, 3),
                                       "products_frac_of_it": round(achieved / lib_all, 3)},
        },
        "quantizers_in_step": {"what": "370M-style step, quantizer time from the step's own calls (linear call "
                                       "minus its products; the fused dY pass timed alone, the re-groupings the "
                                       "rest of the backward), algorithmic bytes (packed operands; the B images the "
                                       "re-groupings and the forward's split also write, 2.125 B per element, are "
                                       "the products' scratch and not counted); frac_of_copy against the copy "
                                       "reference of the quantizer sweep", **q_in_step},
        "fp6x4_backward": {"what": "backward of the 370M-style linears with FP4 vs FP6 (E2M3, NVFP6) gradient "
                                   "operands, the FP6 x FP4 variant", **fp6},
        "single_linear": single,
        "olmo70m_linears": olmo70,
        "stack": stack,
        "quantizer_sweep": {"tensor": "bf16 8192x4096 N(0,1), 1% columns x64", "algorithmic_MB_per_call":
                            round(sweep_bytes / 1e6, 2), "hbm_peak_GB_s": HBM_PEAK_GBS, **sweep},
        "osci_reset": {"what": "OsciReset accumulate over all masters through osci_reset_step_multi (16 weight "
                               "matrices per launch, each with its outlier plan; 36 B/param), as in the step",
                       "GB_s": round(osci_bytes / osci_t / 1e9, 1),
                       "frac_hbm": round(osci_bytes / osci_t / 1e9 / HBM_PEAK_GBS, 3),
                       "access_pattern_GB_s": pattern["osci_5r4w"],
                       "frac_of_access_pattern": round(osci_bytes / osci_t / 1e9 / pattern["osci_5r4w"], 3),
                       "ms_per_step": round(osci_t * 1e3, 3), "params": n_params},
        "master_update": {"what": "fused AdamW + OsciReset accumulate over all masters through "
                                  "master_update_step_multi (16 weight matrices per launch; 52 B/param), without "
                                  "and with the outlier plans (with a plan W and its gradient are gathered through "
                                  "the channel lists)",
                          "GB_s": round(master_bytes / master_t / 1e9, 1),
                          "frac_hbm": round(master_bytes / master_t / 1e9 / HBM_PEAK_GBS, 3),
                          "access_pattern_GB_s": pattern["master_7r6w"],
                          "frac_of_access_pattern": round(master_bytes / master_t / 1e9 / pattern["master_7r6w"], 3),
                          "ms_per_step": round(master_t * 1e3, 3),
                          "with_plans_GB_s": round(master_bytes / master_plan_t / 1e9, 1),
                          "with_plans_ms_per_step": round(master_plan_t * 1e3, 3), "params": n_params},
        "access_pattern_reference": {"what": "libtj2_measure's tj2_stream_probe: the OsciReset pass's loads and "
                                             "stores (5 fp32 reads, 4 writes per element) and the master pass's "
                                             "(7 reads, 6 writes), 8 consecutive elements per thread, no arithmetic, "
                                             "over as many elements as the masters", **pattern},
        "osci_diagnostics": {"what": "fused master pass with oscillation diagnostics: per-pass flip count (ACCUM), "
                                     "window risk histogram in 32 log2 bins (WINDOW_END)",
                             "accum_with_flips_ms": round(diag_accum_t * 1e3, 3),
                             "accum_with_flips_GB_s": round(master_bytes / diag_accum_t / 1e9, 1),
                             "window_end_with_hist_ms": round(diag_end_t * 1e3, 3),
                             "window_end_with_hist_GB_s": round(master_bytes / diag_end_t / 1e9, 1),
                             "flips_per_pass": flips_per_pass, "risk_hist_one_window_end": risk_hist},
        "gpu_state": gpu_state,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
