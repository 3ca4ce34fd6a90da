"""Throughput of the H-BitLinear forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload KEY] [--no-extra]

A step is one H-BitLinear forward call (transform + quantization kernel, then
the ternary product with its fused dequantization) over one batch of seeded
synthetic input already resident in HBM. The headline workload is the decode
GEMV (M=1, K=2560, N=6912, int8 absmax, no Hadamard); its metric is
packed-weight GB/s (N*K/4 bytes per step), timed cold: the step rotates over
enough copies of the packed weights (> 512 MB) that none is served from the
256 MB Infinity Cache.

The JSON line also carries:
  roofline      the dominant kernel (the ternary product) timed per launch with
                HIP events on the launch stream, against the 8 TB/s HBM peak
                (decode) or the 5.03 POP/s dense int8 MFMA peak (prefill);
                `traffic` is the kernel's HBM bytes per launch from the
                committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary under
                profiles/ (copy-kernel calibrated), null once the kernel's
                sources differ from the ones those counters were taken on;
  cpu_baseline  the fp64 CPU oracle on the host cores, on a bounded sample;
  per_workload  every measured workload at full size (prefill TOPS, decode
                GB/s, the on-device ternarize+pack pass, the whole layer
                with its RMSNorm / SwiGLU input prologue, and for the prefill
                shapes the backward: dx and dw from a bf16 gradient);
  kv_cache      the low-bit KV-cache quantizer (3- and 4-bit) in HBM GB/s.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "H-BitLinear fwd: prefill int8-TOPS & decode weight-GB/s, % of MI355X roofline"
HEADLINE = "decode_int8_m1_k2560_n6912"
HBM_PEAK_GBS = 8000.0
INT8_MFMA_PEAK_TOPS = 5033.2  # 256 CU x 2.4 GHz x 8192 int8 ops/clk/CU (dense)
BF16_MFMA_PEAK_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 bf16 flops/clk/CU (dense)
COLD_BYTES = 512 * 2 ** 20


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _dev_x(torch, x_np, x_dtype, dev):
    if x_dtype == "bf16":
        return torch.from_numpy(x_np.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(x_np).to(dev)


def _copies_for_cold(nbytes):
    return max(1, math.ceil(COLD_BYTES / max(nbytes, 1)) + 1)


def _capture(torch, fn, calls):
    """HIP graph of `calls` consecutive calls fn(0) .. fn(calls-1)."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for i in range(calls):
                fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return g


def _time_replays(torch, fn, steps, reps):
    """Per-call ms of `reps` separate replays of one graph of `steps` calls
    (the spread of the timed figure, not of single calls)."""
    g = _capture(torch, fn, steps)
    g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(reps):
        torch.cuda.synchronize()
        if _FLUSH is not None:
            _FLUSH()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        g.replay()
        end.record()
        torch.cuda.synchronize()
        out.append(start.elapsed_time(end) / steps)
    del g
    return out


class CacheFlush:
    """Reads a 1 GiB buffer with the library's plain streaming-read kernel:
    afterwards neither the XCD L2 caches (4 MB each) nor the 256 MB Infinity
    Cache hold any of the timed calls' inputs, whatever they touched before."""

    def __init__(self, torch, bl, dev, nbytes=1 << 30):
        self.bl = bl
        self.buf = torch.zeros((nbytes,), dtype=torch.uint8, device=dev)
        self.sink = torch.zeros((1,), dtype=torch.int32, device=dev)

    def __call__(self):
        self.bl.stream_read(self.buf, self.sink)


_FLUSH = None


def _time_steps(torch, fn, steps, warmup):
    """ms per call over exactly `steps` calls replayed from one HIP graph.

    `warmup` eager calls and one untimed replay come first; then, after a
    synchronization, the caches are flushed (1 GiB streamed through them), so
    that the timed replay starts cold at any step count. The timed replay is
    bracketed by a pair of HIP events on the stream the kernels run on and by
    synchronizations. The host enqueues the flush, the start event and the
    graph back to back: while the GPU streams the flush, the host submits the
    graph, so that the time between the two events is the `steps` calls and
    not the host's submission of them (about 10 us, which at 20 steps would
    add half a microsecond to every step). Within the replay, consecutive
    calls read different weight copies (more than 512 MB of them), so none is
    served from the caches either. Launching from a graph keeps the host's
    per-call Python overhead out of the GPU's timeline."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    g = _capture(torch, fn, steps)
    g.replay()
    torch.cuda.synchronize()
    if _FLUSH is not None:
        _FLUSH()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    g.replay()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    del g
    return ms


class Prepared:
    """Device-resident inputs of one workload."""

    def __init__(self, torch, bl, key, dev, cold=True):
        from bit_activation_linear_amd import workloads
        self.wl = wl = workloads.WORKLOADS[key]
        case = workloads.make_workload(key, seed=0)
        self.case = case
        self.x = _dev_x(torch, case["x"], wl.x_dtype, dev)
        self.W = torch.from_numpy(case["W"]).to(dev)
        Wp, alpha = bl.ternarize_weights(self.W)
        self.alpha = alpha
        wbytes = Wp.numel()
        # Rotate copies only where the weights are big enough to matter; the
        # tiny single-layer case is a latency measurement.
        self.copies = _copies_for_cold(wbytes) if (cold and wbytes >= 2 ** 20) else 1
        self.Wp = [Wp] + [Wp.clone() for _ in range(self.copies - 1)]
        self.y = torch.empty((wl.M, wl.N), dtype=torch.float32, device=dev)
        self.ws = torch.empty((bl.forward_workspace_bytes(wl.M, wl.K, wl.N, wl.bits, wl.hadamard),),
                              dtype=torch.uint8, device=dev)
        self.rowsum = torch.empty((wl.M,), dtype=torch.int32, device=dev)
        self.codes, self.scales = bl.quantize_activations(self.x, wl.bits, wl.hadamard,
                                                          rowsum=self.rowsum)
        self.fused = bl.forward_workspace_bytes(wl.M, wl.K, wl.N, wl.bits, wl.hadamard) == 0
        torch.cuda.synchronize()

    def forward(self, bl, i):
        wl = self.wl
        bl.hbitlinear_forward(self.x, self.Wp[i % self.copies], self.alpha, wl.bits, wl.hadamard,
                              out=self.y, workspace=self.ws if self.ws.numel() else None)

    def stage(self, bl, i, stages):
        """One stage of the forward on its own kernel and workspace (the
        product reads what the quantization stage left in the workspace)."""
        wl = self.wl
        bl.hbitlinear_forward_stages(self.x, self.Wp[i % self.copies], self.alpha, wl.bits,
                                     wl.hadamard, stages, out=self.y, workspace=self.ws)

    def free_latent(self):
        self.W = None


def _work_units(wl):
    return {"weight_bytes": wl.N * wl.K // 4, "ops": 2 * wl.M * wl.N * wl.K}


def _measure_workload(torch, bl, key, dev, steps, warmup):
    p = Prepared(torch, bl, key, dev)
    wl = p.wl
    u = _work_units(wl)
    fwd_ms = _time_steps(torch, lambda i: p.forward(bl, i), steps, warmup)
    quant_ms = None
    if p.fused:
        # the forward is one kernel: it is the product kernel
        mm_mean = fwd_ms
    else:
        # each stage of the forward alone, on the forward's own kernels: the
        # product reads the workspace the quantization stage wrote (for small
        # int4 batches, nibble codes)
        p.stage(bl, 0, 1)
        torch.cuda.synchronize()
        mm_mean = _time_steps(torch, lambda i: p.stage(bl, i, 2), steps, warmup)
        quant_ms = _time_steps(torch, lambda i: p.stage(bl, i, 1), steps, warmup)
    res = {
        "M": wl.M, "K": wl.K, "N": wl.N, "bits": wl.bits, "hadamard": wl.hadamard,
        "x_dtype": wl.x_dtype, "cold_weight_copies": p.copies, "fused_single_kernel": p.fused,
        "forward_us": fwd_ms * 1e3,
        "matmul_kernel_us_mean": mm_mean * 1e3,
        "quantize_stage_us": None if quant_ms is None else quant_ms * 1e3,
        "forward_weight_GBs": u["weight_bytes"] / (fwd_ms * 1e-3) / 1e9,
        "forward_TOPS": u["ops"] / (fwd_ms * 1e-3) / 1e12,
        "matmul_weight_GBs": u["weight_bytes"] / (mm_mean * 1e-3) / 1e9,
        "matmul_TOPS": u["ops"] / (mm_mean * 1e-3) / 1e12,
    }
    if wl.M <= 16:
        res["matmul_hbm_frac"] = res["matmul_weight_GBs"] / HBM_PEAK_GBS
        if p.copies > 1:
            # the plain streaming-read ceiling: the library's read-only kernel
            # over the same cold weight copies, timed the same way
            sink = torch.zeros((1,), dtype=torch.int32, device=dev)
            sr_ms = _time_steps(torch, lambda i: bl.stream_read(p.Wp[i % p.copies], sink), steps,
                                warmup)
            res["stream_read_same_bytes_us"] = sr_ms * 1e3
            res["stream_read_same_bytes_GBs"] = u["weight_bytes"] / (sr_ms * 1e-3) / 1e9
            res["matmul_over_stream_read"] = mm_mean / sr_ms
            # the launch floor: the same read-only kernel over 4 KiB (one
            # workgroup), timed the same way
            tiny = torch.zeros((4096,), dtype=torch.uint8, device=dev)
            res["launch_floor_us"] = _time_steps(torch, lambda i: bl.stream_read(tiny, sink), steps,
                                                 warmup) * 1e3
            # the same forward on one weight copy, served from the caches
            res["forward_us_warm"] = _time_steps(torch, lambda i: p.forward(bl, 0), steps, warmup) * 1e3
        if wl.M > 1 and p.copies > 1:
            # The batched TL2 forward (edge page: TL2 GEMV on a batch; no
            # transform) on the TL2 re-encoding of each cold copy, against the
            # 2-bit forward without the transform on the same input, and the
            # 2-bit product of int8 codes (the TL2 product's code form).
            Wt = [bl.pack_tl2(w) for w in p.Wp]
            tws = torch.empty((bl.tl2_forward_workspace_bytes(wl.M, wl.K),), dtype=torch.uint8,
                              device=dev)
            t_ms = _time_steps(torch, lambda i: bl.hbitlinear_forward_tl2(
                p.x, Wt[i % len(Wt)], p.alpha, wl.bits, out=p.y, workspace=tws), steps, warmup)
            fws = torch.empty((max(1, bl.forward_workspace_bytes(wl.M, wl.K, wl.N, wl.bits, 0)),),
                              dtype=torch.uint8, device=dev)
            f_ms = _time_steps(torch, lambda i: bl.hbitlinear_forward(
                p.x, p.Wp[i % p.copies], p.alpha, wl.bits, 0, out=p.y, workspace=fws), steps, warmup)
            rs = torch.empty((wl.M,), dtype=torch.int32, device=dev)
            c8, s8 = bl.quantize_activations(p.x, wl.bits, 0, rowsum=rs)
            m8_ms = _time_steps(torch, lambda i: bl.ternary_linear_dequant(
                c8, s8, p.Wp[i % p.copies], p.alpha, wl.bits, rowsum=rs, out=p.y), steps, warmup)
            tbytes = Wt[0].numel()
            res["tl2_no_transform"] = {
                "forward_us": t_ms * 1e3,
                "weight_bytes": tbytes,
                "bits_per_weight": tbytes * 8 / (wl.N * wl.K),
                "forward_2bit_us": f_ms * 1e3,
                "product_2bit_int8_codes_us": m8_ms * 1e3,
                "kernels": "quant_rows_kernel (TL2 code order) + tl2_gemv_kernel",
            }
            del Wt, tws, fws
    else:
        res["matmul_mfma_frac"] = res["matmul_TOPS"] / INT8_MFMA_PEAK_TOPS
    # The engine page's whole HBitLinear.forward: RMSNorm (unit weight plus a
    # seeded elementwise weight) in front, and for the transform workloads
    # (the FFN's Wdown) the SwiGLU product silu(gate) * up as the input.
    gamma = torch.from_numpy((np.random.default_rng(1).standard_normal(wl.K) * 0.3 + 1.0)
                             .astype(np.float32)).to(dev)
    up = p.x.flip(0).contiguous() if wl.hadamard else None
    pws = torch.empty((bl.forward_prologue_workspace_bytes(wl.M, wl.K, wl.N, wl.bits, wl.hadamard),),
                      dtype=torch.uint8, device=dev)

    def with_prologue(i):
        bl.hbitlinear_forward_prologue(p.x, p.Wp[i % p.copies], p.alpha, wl.bits, wl.hadamard, up=up,
                                       rmsnorm=True, norm_weight=gamma, out=p.y, workspace=pws)
    pro_ms = _time_steps(torch, with_prologue, steps, warmup)
    res["forward_prologue_us"] = pro_ms * 1e3
    res["prologue"] = ("silu(gate) * up, RMSNorm" if wl.hadamard else "RMSNorm") + " fused into the quantizer"
    if wl.M > 16:
        # Backward (engine page Eq. 8, STE quantizer gradients): dx and dw from
        # a seeded bf16 gradient dy and the forward's codes and scales.
        gen = torch.Generator(device=dev)
        gen.manual_seed(0)
        dy = (torch.randn((wl.M, wl.N), generator=gen, device=dev) * 1e-3).to(torch.bfloat16)
        dx = torch.empty((wl.M, wl.K), dtype=torch.float32, device=dev)
        dw = torch.empty((wl.N, wl.K), dtype=torch.float32, device=dev)
        bws = torch.empty((bl.backward_workspace_bytes(wl.M, wl.K, wl.N, torch.bfloat16),),
                          dtype=torch.uint8, device=dev)

        def bwd(i):
            bl.hbitlinear_backward(dy, p.codes, p.scales, p.Wp[i % p.copies], p.alpha, wl.bits,
                                   wl.hadamard, dx=dx, dw=dw, workspace=bws)
        b_ms = _time_steps(torch, bwd, max(5, steps // 4), 2)
        bflops = 4 * wl.M * wl.N * wl.K  # dx and dw, 2MNK each
        res["backward_us"] = b_ms * 1e3
        res["backward_TFLOPs"] = bflops / (b_ms * 1e-3) / 1e12
        res["backward_bf16_mfma_frac"] = res["backward_TFLOPs"] / BF16_MFMA_PEAK_TFLOPS
        res["backward"] = ("dx = H(alpha dy . t) and dw = dy^T . x_q from a bf16 dy; 4*M*N*K "
                           "algorithmic flops on bf16 MFMA (dw multiplies the hi and lo bf16 "
                           "parts of dy*s/c in one pass, twice the MFMA work of one part)")
        del dy, dx, dw, bws
    if key == "prefill_int8_m8192_k4096_n14336" or key == "int4_hadamard_m4_k256_n256":
        # on-device ternarize + pack: two fp32 reads of W plus the packed write
        Wp = p.Wp[0]
        tws = torch.empty((bl.api._lib.load().bitnet_ternarize_workspace_bytes(wl.N, wl.K),),
                          dtype=torch.uint8, device=dev)
        tern_ms = _time_steps(torch, lambda i: bl.ternarize_weights(p.W, out=Wp, alpha=p.alpha,
                                                                    workspace=tws),
                              max(5, steps // 4), 2)
        tbytes = 2 * wl.N * wl.K * 4 + wl.N * wl.K // 4
        res["ternarize_us"] = tern_ms * 1e3
        res["ternarize_GBs"] = tbytes / (tern_ms * 1e-3) / 1e9
    if key == "int4_hadamard_m4_k256_n256":
        # whole layer including weight preparation, latency only
        tws1 = torch.empty((bl.api._lib.load().bitnet_ternarize_workspace_bytes(wl.N, wl.K),),
                           dtype=torch.uint8, device=dev)

        def full(i):
            bl.ternarize_weights(p.W, out=p.Wp[0], alpha=p.alpha, workspace=tws1)
            p.forward(bl, 0)
        res["ternarize_plus_forward_us"] = _time_steps(torch, full, steps, warmup) * 1e3
    return p, res


def _measure_kv(torch, bl, dev, steps, warmup):
    """Low-bit KV-cache quantizer on a 32-head, 4096-token, head_dim 128 bf16
    cache (seeded N(0,1) values with a few x8 outlier channels): HBM bytes are
    2 read + 1 written per element and 4 written per token; with the codes
    packed, bits/8 written per element."""
    from bit_activation_linear_amd import workloads
    B, H, S, D = 1, 32, 4096, 128
    case = workloads.make_case(B * H * S, D, 1, x_dtype="bf16", n_out=4, factor=8.0, seed=0)
    kv = _dev_x(torch, case["x"], "bf16", dev).view(B, H, S, D)
    nbytes = B * H * S * (3 * D + 4)
    res = {"shape": [B, H, S, D], "x_dtype": "bf16", "bytes_per_call": nbytes, "bits": {}}
    codes = torch.empty(kv.shape, dtype=torch.int8, device=dev)
    scales = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    for bits in (3, 4):
        ms = _time_steps(torch, lambda i, b=bits: bl.kv_quantize(kv, b, codes=codes, scales=scales),
                         steps, warmup)
        res["bits"][bits] = {"us": ms * 1e3, "GBs": nbytes / (ms * 1e-3) / 1e9,
                             "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        # the same codes stored bits/8 bytes per element (BOS rows apart):
        # 2 B read + bits/8 B written per element, 4 B per token, D B per head
        packed = torch.empty((B, H, S, D * bits // 8), dtype=torch.uint8, device=dev)
        bos = torch.empty((B, H, D), dtype=torch.int8, device=dev)
        pbytes = B * H * S * (2 * D + D * bits // 8 + 4) + B * H * D
        ms = _time_steps(torch, lambda i, b=bits: bl.kv_quantize_packed(
            kv, b, packed=packed, bos_codes=bos, scales=scales), steps, warmup)
        res["bits"][bits]["packed"] = {"us": ms * 1e3, "bytes_per_call": pbytes,
                                       "GBs": pbytes / (ms * 1e-3) / 1e9,
                                       "hbm_frac": pbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                       "cache_bytes_per_element": bits / 8}
    return res


def _recorded_traffic(kernel, key):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary of `kernel` on workload `key`, or None when there is none or when
    the kernel's sources have changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}.{key}.pmc_traffic.md")
    if not os.path.exists(path):
        return None, None
    fields = {}
    with open(path) as f:
        for ln in f:
            if ":" in ln and not ln.startswith((" ", "|", "#")):
                k, v = ln.split(":", 1)
                fields[k.strip()] = v.strip()
    try:
        h = hashlib.sha256()
        for rel in fields["source_files"].split():
            with open(os.path.join(ROOT, rel), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != fields["source_sha256"]:
            return None, os.path.relpath(path, ROOT) + " (stale: kernel sources changed)"
        return float(fields["traffic_bytes_per_launch"]), os.path.relpath(path, ROOT)
    except (KeyError, OSError, ValueError):
        return None, None


def _cpu_baseline(key, budget_s):
    """fp64 oracle on a bounded number of whole forward calls of the workload."""
    import oracle
    from bit_activation_linear_amd import workloads
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = 1
    wl = workloads.WORKLOADS[key]
    case = workloads.make_workload(key, seed=0)
    t, alpha, _ = oracle.ternarize(case["W"])
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.forward(case["x"], wl.x_dtype, t, alpha, wl.bits, wl.hadamard)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 10000:
            break
    per = el / reps
    return {
        "value": (wl.N * wl.K / 4) / per / 1e9, "unit": "GB/s", "cores": int(cores),
        "kind": "oracle",
        "sample": f"{reps} whole forward calls of {key} (M={wl.M}, K={wl.K}, N={wl.N}) from "
                  f"ternary int8 weights, fp64 NumPy, {el:.1f} s; weight-prep excluded",
        "seconds_per_call": per,
    }


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _time_oracle_forward(key, budget_s, threads):
    """Seconds per whole oracle forward call of `key` (weight preparation
    excluded), with the BLAS pool limited to `threads`."""
    import oracle
    from bit_activation_linear_amd import workloads
    from threadpoolctl import threadpool_limits
    wl = workloads.WORKLOADS[key]
    case = workloads.make_workload(key, seed=0)
    t, alpha, _ = oracle.ternarize(case["W"])
    with threadpool_limits(limits=threads):
        oracle.forward(case["x"], wl.x_dtype, t, alpha, wl.bits, wl.hadamard)  # warm-up
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.forward(case["x"], wl.x_dtype, t, alpha, wl.bits, wl.hadamard)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s or reps >= 10000:
                break
    return el / reps, reps


def _cpu_other_workloads(budget_s):
    """The oracle on the single-layer, headline and batched-decode workloads,
    on every host core and on one core (a reported baseline, not a target)."""
    from bit_activation_linear_amd import workloads
    cores = len(os.sched_getaffinity(0))
    out = {}
    for key in ("int4_hadamard_m4_k256_n256", "decode_int8_m1_k2560_n6912",
                "decode_int4_hadamard_m16_k16384_n4096"):
        wl = workloads.WORKLOADS[key]
        r = {"weight_bytes": wl.N * wl.K // 4}
        for label, th in (("all_cores", cores), ("one_core", 1)):
            per, reps = _time_oracle_forward(key, budget_s, th)
            r[label] = {"threads": th, "seconds_per_call": per, "calls": reps,
                        "weight_GBs": (wl.N * wl.K / 4) / per / 1e9}
        out[key] = r
    return out


def _clocks():
    """Current GPU core and memory clocks (sysfs DPM tables, else amd-smi as a
    child process); None where neither is readable."""
    import glob
    import subprocess
    res = {}
    for name in ("pp_dpm_sclk", "pp_dpm_mclk"):
        for path in sorted(glob.glob(f"/sys/class/drm/card*/device/{name}")):
            try:
                with open(path) as f:
                    cur = [ln.strip() for ln in f if ln.strip().endswith("*")]
                if cur:
                    res[name] = cur[0]
                    break
            except OSError:
                continue
    if len(res) < 2:
        try:
            out = subprocess.run(["amd-smi", "metric", "--clock", "--json"], capture_output=True,
                                 text=True, timeout=20)
            if out.returncode == 0:
                res["amd_smi_clock"] = json.loads(out.stdout)
        except (OSError, subprocess.SubprocessError, ValueError):
            pass
    return res or None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(sharding is a design note). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_activation_linear_amd as bl
    from bit_activation_linear_amd import _lib, workloads

    _lib.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    global _FLUSH
    _FLUSH = CacheFlush(torch, bl, dev)
    clocks_before = _clocks()

    key = args.workload
    wl = workloads.WORKLOADS[key]
    _log(f"[bench] headline workload {key}")
    p, head = _measure_workload(torch, bl, key, dev, args.steps, args.warmup)
    ms = head["forward_us"] / 1e3
    decode = wl.M <= 16
    # Spread of the timed figure over separate replays, and, as context, a
    # plain device copy of the same (cold) weight bytes.
    reps = _time_replays(torch, lambda i: p.forward(bl, i), args.steps, 7)
    reps_us = sorted(r * 1e3 for r in reps)
    head["forward_us_replays_p10_p50_p90"] = [reps_us[0], reps_us[3], reps_us[-1]]
    stream_us = None
    if decode and p.copies > 1:
        dst = torch.empty_like(p.Wp[0])
        cp_ms = _time_steps(torch, lambda i: dst.copy_(p.Wp[i % p.copies]), args.steps, 5)
        head["copy_same_bytes_us"] = cp_ms * 1e3
        head["copy_same_bytes_read_GBs"] = p.Wp[0].numel() / (cp_ms * 1e-3) / 1e9
        del dst
        stream_us = head.get("stream_read_same_bytes_us")
    if decode:
        value, unit = head["forward_weight_GBs"], "GB/s"
        roof = {"bound": "hbm", "achieved": head["matmul_weight_GBs"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": head["matmul_weight_GBs"] / HBM_PEAK_GBS}
    else:
        value, unit = head["forward_TOPS"], "TOPS"
        roof = {"bound": "mfma", "achieved": head["matmul_TOPS"], "peak": INT8_MFMA_PEAK_TOPS,
                "unit": "TFLOP/s", "frac": head["matmul_TOPS"] / INT8_MFMA_PEAK_TOPS}
    if decode:
        if not head["fused_single_kernel"]:
            roof["kernel"] = "ternary_gemv_kernel"
        else:  # a single token runs the one-wave kernel, a few tokens the multi-wave one
            roof["kernel"] = "wave_decode_kernel" if wl.M == 1 else "fused_decode_kernel"
    else:
        # the library's dispatch: many 256x256 tiles (and the forward's row
        # sums) take the streamed-tile kernel
        tiles = ((wl.M + 255) // 256) * ((wl.N + 255) // 256)
        stream = tiles >= 1024 and wl.K % 128 == 0 and wl.K >= 512 and wl.N % 4 == 0
        roof["kernel"] = "ternary_gemm_stream_kernel" if stream else "ternary_gemm_kernel"
    roof["algorithmic"] = ("N*K/4 packed weight bytes per launch" if decode
                           else "2*M*N*K int8 ops per launch")
    roof["launch_us_mean"] = head["matmul_kernel_us_mean"]
    roof["timing"] = ("HIP events around one HIP-graph replay of back-to-back launches, caches "
                      "flushed before it")
    if stream_us is not None:
        # context, not the denominator: the plain read-only kernel over the
        # same cold bytes, and the product's time relative to it
        roof["stream_read_ceiling_GBs"] = head["stream_read_same_bytes_GBs"]
        roof["launch_us_over_stream_read_us"] = head["matmul_kernel_us_mean"] / stream_us
    traffic, source = _recorded_traffic(roof["kernel"], key)
    roof["traffic"] = traffic
    if source:
        roof["traffic_source"] = source
    _log(f"[bench] {key}: forward {head['forward_us']:.2f} us, matmul {head['matmul_kernel_us_mean']:.2f} us")
    if decode and wl.M == 1 and not wl.hadamard and wl.K <= 4608:
        # The same forward on the TL2 weight code (edge page: 5 bits per 3
        # weights), re-encoded on the device from each cold 2-bit copy.
        Wt = [bl.pack_tl2(w) for w in p.Wp]
        tl2_ms = _time_steps(torch, lambda i: bl.hbitlinear_forward_tl2(
            p.x, Wt[i % len(Wt)], p.alpha, wl.bits, out=p.y), args.steps, args.warmup)
        tbytes = Wt[0].numel()
        head["tl2"] = {
            "forward_us": tl2_ms * 1e3,
            "weight_bytes": tbytes,
            "bits_per_weight": tbytes * 8 / (wl.N * wl.K),
            "weight_GBs": tbytes / (tl2_ms * 1e-3) / 1e9,
            "vs_2bit_forward": head["forward_us"] / (tl2_ms * 1e3),
            "kernel": "tl2_decode_kernel",
        }
        _log(f"[bench] {key}: TL2 forward {tl2_ms * 1e3:.2f} us ({tbytes} weight bytes)")
        del Wt
    del p

    per = {key: head}
    if not args.no_extra:
        for other in workloads.WORKLOAD_ORDER:
            if other == key:
                continue
            _log(f"[bench] workload {other}")
            po, r = _measure_workload(torch, bl, other, dev, max(20, args.steps // 4),
                                      max(5, args.warmup // 2))
            del po
            torch.cuda.empty_cache()
            per[other] = r
            _log(f"[bench] {other}: forward {r['forward_us']:.2f} us, matmul {r['matmul_kernel_us_mean']:.2f} us"
                 + (f", backward {r['backward_us']:.1f} us" if "backward_us" in r else ""))

    kv = None
    if not args.no_extra:
        kv = _measure_kv(torch, bl, dev, max(20, args.steps // 4), max(5, args.warmup // 2))
        _log(f"[bench] kv cache: " + ", ".join(f"{b}-bit {r['us']:.2f} us (packed {r['packed']['us']:.2f} us)"
                                                for b, r in kv["bits"].items()))

    clocks_after = _clocks()
    cpu = None
    if not args.no_cpu:
        _log("[bench] CPU oracle baseline")
        cpu = _cpu_baseline(key, args.cpu_seconds)
        cpu["model"] = _cpu_model()
        if not args.no_extra:
            cpu["other_workloads"] = _cpu_other_workloads(args.cpu_seconds / 4)

    line = {
        "metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "i8", "data": "synthetic",
        "timing": "HIP graph replay of exactly `steps` forward calls, HIP events on the launch stream",
        "config": {"workload": key, "M": wl.M, "K": wl.K, "N": wl.N, "bits": wl.bits,
                   "hadamard": wl.hadamard, "x_dtype": wl.x_dtype,
                   "cold_weight_copies": head["cold_weight_copies"]},
        "roofline": roof, "cpu_baseline": cpu, "per_workload": per, "kv_cache": kv,
        "clocks": {"before": clocks_before, "after": clocks_after},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
