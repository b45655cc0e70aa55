"""Benchmark of the quantized-linear hot path on one MI355X.

Workload: the CogVideoX-2B-shaped QKV projection, M = 17776 tokens (17550
video + 226 text), K = 1920, N = 5760, bf16 activations ~N(0,1) with 1 %
outlier channels x30, weights ~N(0, 0.02^2) quantized to NVFP4 once at set
up.  The pages measure on VBench with trained CogVideoX weights; seeded
synthetic tensors of the same shapes stand in for them.

One step is one pass of the whole hot path over that batch:
  act_quant NVFP4 -> qlinear_nvfp4 ; act_quant INT8 -> qlinear_int8 (integer
  MFMA on the weight's int8 digit planes, made once at set-up) ;
  tdc_update (Delta cache, with Gamma and relative-L2 sums) ;
  tdc_apply (the skip path, with Gamma sums) ;
  copy of the sums to the host, dmpq_mask and tdc_decide.
`value` is the linear FLOPs of both activation paths per second of whole
steps (2 * 2*M*N*K per step).  The GEMM kernel times come from HIP events
that the library's hook attaches to the GEMM dispatches themselves inside
the timed steps (their start and end timestamps, on the launch stream);
the times of the other calls come from event markers around each library
call in as many extra, untimed steps after the timed region.  `cold`
times each bandwidth-bound call alone, after a 1 GiB read that evicts L2
and the Infinity Cache (median of --cold-reps), against the algorithmic
bytes of the call (the NVFP4 amax pre-pass is not counted; the
given-tensor-scale call is the encoder alone).
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"hbm_GBps": 8000.0, "bf16_TFLOPs": 2500.0, "int8_TOPs": 5000.0, "fp4_TFLOPs": 10100.0,
        "fp8_TFLOPs": 5000.0}
M, K, N = 17776, 1920, 5760


class Hip:
    """The few HIP runtime calls the timing needs (events)."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.h.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def record(self, e, stream):
        assert self.h.hipEventRecord(e, ctypes.c_void_p(stream)) == 0

    def ms(self, a, b):
        out = ctypes.c_float()
        assert self.h.hipEventElapsedTime(ctypes.byref(out), a, b) == 0
        return out.value

    def destroy(self, e):
        self.h.hipEventDestroy(e)


def sources_unchanged(rec):
    """True when the kernel sources a profile record names (sha256 over the
    files in order) are those in the tree."""
    h = hashlib.sha256()
    for name in rec.get("sources", [rec["source"]]):
        with open(os.path.join(ROOT, "mixed_precision_quantized_act_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest() == rec["source_sha256"]


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from profiles/traffic.json (two
    rocprofv3 --pmc passes, FETCH_SIZE and WRITE_SIZE, scaled by the same
    counters on a plain device copy of known size), or None when the file
    is missing or the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel)
    if not rec or not sources_unchanged(rec):
        return None
    return rec["hbm_bytes_per_launch"]


def measured_mfma(kernel):
    """MFMA counters of `kernel` from profiles/mfma_counters.json (one
    rocprofv3 --pmc pass: SQ_VALU_MFMA_BUSY_CYCLES over all SIMDs and
    GRBM_GUI_ACTIVE over the 8 XCDs, per dispatch), or None when the file is
    missing or the kernel source changed since: the fraction of the kernel's
    SIMD cycles in which the MFMA unit was busy, and the shader clock
    implied by the GPU-active cycles and the dispatch's duration."""
    path = os.path.join(ROOT, "profiles", "mfma_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel)
    if not rec or not sources_unchanged(rec):
        return None
    return {"mfma_busy_frac": rec["mfma_busy_frac"], "sclk_MHz": rec["sclk_MHz"],
            "issued_TOP_per_s": rec["issued_TOP_per_s"], "duration_us": rec["duration_us"],
            "source": "profiles/mfma_counters.json"}


# The pages' own figures (6Bit-Diffusion, abstract and Table 2): end-to-end
# speed-ups of W4A6 DMPQ and DMPQ + TDC over W16A16, and the memory
# reduction, on a machine the pages do not name.  Context only.
PAGES_CONTEXT = {"dmpq_speedup_vs_w16a16": 1.36, "full_speedup_vs_w16a16": 1.92,
                 "memory_reduction_vs_fp16": 3.32, "hardware": "not stated on the pages",
                 "source": "6Bit-Diffusion abstract; Table 2"}


def cpu_baseline(x, w, x_out, delta_prev, rows):
    """The oracle, untuned, on the first `rows` token rows of the workload."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import gemm as G
    from oracle import quant as Q
    from oracle import tdc as T
    wq = Q.nvfp4_encode(w)                     # set-up, untimed as on the GPU
    wd = Q.nvfp4_decode(*wq)
    xs, xo, dp = x[:rows], x_out[:rows], delta_prev[:rows]
    t0 = time.perf_counter()
    a4 = Q.nvfp4_encode(xs)
    G.linear_ref(Q.nvfp4_decode(*a4), wd)
    a8 = Q.int8_encode(xs)
    G.linear_ref(Q.int8_decode(*a8), wd)
    dn, sums = T.tdc_update(xs.ravel(), xo.ravel(), dp.ravel())
    applied = T.tdc_apply(xs.ravel(), dn)
    T.gamma_sums(xs.ravel(), applied)
    dt = time.perf_counter() - t0
    blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
    cores = max(blas) if blas else 1
    flops = 2 * 2.0 * rows * N * K
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(flops / dt / 1e12, 4), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle", "cpu": model,
            "sample": f"first {rows} of {M} token rows, one full step (both quantizers, both "
                      f"float64 GEMMs, TDC update/apply sums), {dt:.1f} s; element-wise numpy on "
                      f"1 thread, float64 BLAS on {cores} threads; host has {os.cpu_count()} CPUs"}


def layer_rates(qa, torch, np, dev, stream, M, H, F_, reps=5):
    """Per-layer qlinear speed of one block's four linears (QKV H->3H, O
    H->H, up H->F with GELU, down F->H) on M tokens, both activation
    formats: the GEMM call alone (operands quantized beforehand), median of
    `reps` event-timed calls."""
    shapes = {"qkv": (3 * H, H, False), "o": (H, H, False), "up_gelu": (F_, H, True),
              "down": (H, F_, False)}
    gen = torch.Generator(device=dev)
    gen.manual_seed(77)
    out = {}
    for name, (N, K, gelu) in shapes.items():
        w = (torch.randn((N, K), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
        wq, ws_, wts = qa.empty_nvfp4(N, K, dev)
        qa.act_quant(qa.NVFP4, w.view(torch.int16), wq, ws_, wts, 0,
                     qa.workspace(qa.act_quant_workspace(qa.NVFP4, N, K), dev), stream=stream)
        x = torch.randn((M, K), generator=gen, device=dev).to(torch.bfloat16).view(torch.int16)
        aq, asc, ats = qa.empty_nvfp4(M, K, dev)
        qa.act_quant(qa.NVFP4, x, aq, asc, ats, 0,
                     qa.workspace(qa.act_quant_workspace(qa.NVFP4, M, K), dev), stream=stream)
        a8, s8 = qa.empty_int8_act(M, K, dev)
        qa.act_quant(qa.INT8, x, a8, s8, stream=stream)
        w8 = qa.empty_int8_planes(N, K, dev)
        qa.int8_weight_planes(wq, ws_, w8, N, K, stream=stream)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        epi = qa.EPI_GELU_TANH if gelu else qa.EPI_NONE
        g4 = qa.workspace(qa.qlinear_workspace(qa.NVFP4, M, N, K), dev)
        g8 = qa.workspace(qa.qlinear_workspace(qa.INT8, M, N, K), dev)
        calls = {
            "nvfp4": lambda: qa.qlinear_nvfp4(aq, asc, ats, wq, ws_, wts, y, M, N, K, epi=epi,
                                              ws=g4, stream=stream),
            "int8": lambda: qa.qlinear_int8(a8, s8, wq, ws_, wts, y, M, N, K, epi=epi, ws=g8,
                                            stream=stream, w8=w8),
            "int8_fp16_kernel": lambda: qa.qlinear_int8(a8, s8, wq, ws_, wts, y, M, N, K, epi=epi,
                                                        ws=g8, stream=stream)}
        rec = {"N": N, "K": K}
        for fmt, fn in calls.items():
            fn()
            ts = []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                e1.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3)
            us = float(np.median(ts))
            tfs = 2.0 * M * N * K / (us * 1e-6) / 1e12
            own = PEAK["fp4_TFLOPs"] if fmt == "nvfp4" else PEAK["int8_TOPs"]
            rec[fmt] = {"us": round(us, 1), "TFLOP/s": round(tfs, 1),
                        "frac_own_dtype_peak": round(tfs / own, 4),
                        "frac_fp16_peak": round(tfs / PEAK["bf16_TFLOPs"], 4)}
        out[name] = rec
        del w, x, y, aq, asc, a8, g4, g8, w8
    return out


def ffn_section(qa, torch, np, dev, stream, reps=5):
    """The FFN config: 17776 tokens of Student-t(3) activations, 1920 ->
    7680 (GELU-tanh) -> 1920 with NVFP4 weights; a forward pass (activation
    quantization and GEMM of both linears) in each combination of the two
    formats, and the DMPQ choice for it: p_l = 1.0 Gamma_l + 0.01 per linear
    with Gamma_l of a synthetic in/out pair of the linear's input (out = in +
    0.1 N(0,1), block_gamma), tau at the midpoint so that one of the two
    linears is INT8."""
    import synth
    x, wu, wd = synth.ffn_case(3)
    M, K = x.shape
    F_ = wu.shape[0]
    to = lambda a: torch.from_numpy(a.view(np.int16).copy()).to(dev)
    xd = to(x)
    ws = []
    for w in (wu, wd):
        N, KK = w.shape
        q, sc, ts = qa.empty_nvfp4(N, KK, dev)
        qa.act_quant(qa.NVFP4, to(w), q, sc, ts, 0,
                     qa.workspace(qa.act_quant_workspace(qa.NVFP4, N, KK), dev), stream=stream)
        w8 = qa.empty_int8_planes(N, KK, dev)
        qa.int8_weight_planes(q, sc, w8, N, KK, stream=stream)
        ws.append((q, sc, ts, N, KK, w8))
    h = torch.empty((M, F_), dtype=torch.bfloat16, device=dev)
    y = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    a4 = qa.empty_nvfp4(M, F_, dev)
    a8 = qa.empty_int8_act(M, F_, dev)
    qws = qa.workspace(qa.act_quant_workspace(qa.NVFP4, M, F_), dev)
    gws = qa.workspace(max(qa.qlinear_workspace(f, M, w[3], w[4]) for f in (qa.NVFP4, qa.INT8)
                           for w in ws), dev)

    def lin(fmt, xin, w, out, gelu):
        q, sc, ts, N, KK, w8 = w
        epi = qa.EPI_GELU_TANH if gelu else qa.EPI_NONE
        if fmt == 0:
            aq = a4[0].view(-1)[: M * KK // 2].view(M, KK // 2)
            asc = a4[1].view(-1)[: M * KK // 16].view(M, KK // 16)
            qa.act_quant(qa.NVFP4, xin, aq, asc, a4[2], 0, qws, stream=stream)
            qa.qlinear_nvfp4(aq, asc, a4[2], q, sc, ts, out, M, N, KK, epi=epi, ws=gws,
                             stream=stream)
        else:
            aq = a8[0].view(-1)[: M * KK].view(M, KK)
            qa.act_quant(qa.INT8, xin, aq, a8[1], stream=stream)
            qa.qlinear_int8(aq, a8[1], q, sc, ts, out, M, N, KK, epi=epi, ws=gws, stream=stream,
                            w8=w8)

    def ffn(fu, fd):
        lin(fu, xd, ws[0], h, True)
        lin(fd, h.view(torch.int16), ws[1], y, False)

    amax_word = qws[:4096].view(torch.int32)          # the 1024 partial-maximum slots

    def ffn_amax(fu):
        # NVFP4 down projection whose tensor amax comes from the up GEMM's
        # epilogue (qlinear_*_amax into act_quant's workspace, QA_AMAX_GIVEN)
        amax_word.zero_()
        q, sc, ts, N, KK, w8 = ws[0]
        if fu == 0:
            aq = a4[0].view(-1)[: M * K // 2].view(M, K // 2)
            asc = a4[1].view(-1)[: M * K // 16].view(M, K // 16)
            xws = qa.workspace(4096, dev) if not hasattr(ffn_amax, "xws") else ffn_amax.xws
            ffn_amax.xws = xws
            qa.act_quant(qa.NVFP4, xd, aq, asc, a4[2], 0, xws, stream=stream)
            qa.qlinear_nvfp4_amax(aq, asc, a4[2], q, sc, ts, h, amax_word, M, N, KK,
                                  epi=qa.EPI_GELU_TANH, ws=gws, stream=stream)
        else:
            aq = a8[0].view(-1)[: M * K].view(M, K)
            qa.act_quant(qa.INT8, xd, aq, a8[1], stream=stream)
            qa.qlinear_int8_amax(aq, a8[1], q, sc, ts, h, amax_word, M, N, KK,
                                 epi=qa.EPI_GELU_TANH, ws=gws, stream=stream, w8=w8)
        q, sc, ts, N, KK, _ = ws[1]
        aq = a4[0].view(-1)[: M * KK // 2].view(M, KK // 2)
        asc = a4[1].view(-1)[: M * KK // 16].view(M, KK // 16)
        qa.act_quant(qa.NVFP4, h.view(torch.int16), aq, asc, a4[2], qa.AMAX_GIVEN, qws,
                     stream=stream)
        qa.qlinear_nvfp4(aq, asc, a4[2], q, sc, ts, y, M, N, KK, ws=gws, stream=stream)

    flops = 2.0 * M * K * F_ * 2
    res = {}
    for fu in (0, 1):
        for fd in (0, 1):
            ffn(fu, fd)
            ts_ = []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                ffn(fu, fd)
                e1.record()
                e1.synchronize()
                ts_.append(e0.elapsed_time(e1))
            ms = float(np.median(ts_))
            name = f"up_{'int8' if fu else 'nvfp4'}_down_{'int8' if fd else 'nvfp4'}"
            res[name] = {"ms": round(ms, 3), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1)}
    for fu in (0, 1):
        ffn_amax(fu)
        ts_ = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            ffn_amax(fu)
            e1.record()
            e1.synchronize()
            ts_.append(e0.elapsed_time(e1))
        ms = float(np.median(ts_))
        name = f"up_{'int8' if fu else 'nvfp4'}_down_nvfp4_amax_from_up_epilogue"
        res[name] = {"ms": round(ms, 3), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1)}
    # DMPQ choice for the two linears
    rws = qa.workspace(qa.reduce_workspace(M * F_), dev)
    gam = []
    g2 = torch.zeros(2, dtype=torch.float64, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(303)
    for xin in (xd, h.view(torch.int16)):
        xf = xin.view(torch.bfloat16).float()
        out = (xf + 0.1 * torch.randn(xf.shape, generator=gen, device=dev)).to(torch.bfloat16)
        qa.block_gamma(xin.reshape(-1), out.view(torch.int16).reshape(-1), g2, rws, stream=stream)
        gam.append(qa.gamma_from_sums(g2.cpu().numpy()))
        del xf, out
    alpha = np.full(2, 1.0, np.float32)
    beta = np.full(2, 0.01, np.float32)
    p = np.array(gam) * 1.0 + 0.01
    tau = float(0.5 * (p.min() + p.max()))
    mask = qa.dmpq_mask(np.array(gam), alpha, beta, tau, 2, 1)
    res["dmpq"] = {"gamma": [round(float(g), 5) for g in gam], "tau": round(tau, 6),
                   "mask_int8": [int(m) for m in mask],
                   "pass": f"up_{'int8' if mask[0] else 'nvfp4'}_down_{'int8' if mask[1] else 'nvfp4'}"}
    res["config"] = {"tokens": M, "hidden": K, "ffn": F_, "activations": "Student-t(3) bf16",
                     "GFLOP_per_pass": round(flops / 1e9, 1)}
    del h, y, a4, a8, gws, qws
    return res


def stack_section(qa, torch, np, dev, stream, L=30, H=1920, F_=7680, M=17776, steps=10,
                  delta=0.05, cfg=4,
                  modes=("w4a8", "w4a4", "dmpq", "full", "median", "cos", "device")):
    """The CogVideoX-2B-shaped stack (30 blocks; per block the four internal
    linears QKV H->3H, O H->H, up H->F with GELU, down F->H; attention
    replaced by its value slice, no token mixing) over `steps` drifting
    timesteps, entirely through the library, in four modes: uniform W4A8,
    uniform W4A4, DMPQ (masks from the previous step's Gamma, tau set once
    so that half of the linears are INT8) and DMPQ + TDC ("median": TDC
    with delta at the DMPQ run's median d; "cos": the cosine rule at the
    median cosine); other shapes (the 5B-shaped stack: 42 blocks, H 3072,
    FFN 12288) through L, H, F_ and the synthetic config id `cfg`.  Returns
    ms/step (mean of steps 2..), the INT8 share and the skipped blocks."""
    import math
    import synth
    J = 4
    shapes = [(3 * H, H), (H, H), (F_, H), (H, F_)]
    gen = torch.Generator(device=dev)
    gen.manual_seed(1004)
    layers = []
    qw = qa.workspace(qa.act_quant_workspace(qa.NVFP4, F_, F_), dev)
    for _ in range(L):
        lay = []
        for (N, K) in shapes:
            w = (torch.randn((N, K), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
            q, sc, ts = qa.empty_nvfp4(N, K, dev)
            qa.act_quant(qa.NVFP4, w.view(torch.int16), q, sc, ts, 0, qw)
            w8 = qa.empty_int8_planes(N, K, dev)
            qa.int8_weight_planes(q, sc, w8, N, K)
            lay.append((q, sc, ts, N, K, w8))
        layers.append(lay)
    bf = torch.bfloat16
    qkv = torch.empty((M, 3 * H), dtype=bf, device=dev)
    o = torch.empty((M, H), dtype=bf, device=dev)
    x1 = torch.empty((M, H), dtype=bf, device=dev)
    u = torch.empty((M, F_), dtype=bf, device=dev)
    dd = torch.empty((M, H), dtype=bf, device=dev)
    a4 = qa.empty_nvfp4(M, F_, dev)
    a8 = qa.empty_int8_act(M, F_, dev)
    qws = qa.workspace(qa.act_quant_workspace(qa.NVFP4, M, F_), dev)
    gws = qa.workspace(max([qa.qlinear_workspace(f, M, N, K) for f in (qa.NVFP4, qa.INT8)
                            for (N, K) in shapes] +
                           [qa.qlinear_routed_workspace(M, N, K) for (N, K) in shapes]), dev)
    rws = qa.workspace(qa.reduce_workspace(M * H), dev)
    ring = [[torch.empty((M, H), dtype=bf, device=dev) for _ in range(2)] for _ in range(L)]
    sums = torch.zeros((L, 4), dtype=torch.float64, device=dev)
    hsums = torch.zeros((L, 4), dtype=torch.float64).pin_memory()
    alpha = np.full(L * J, 1.0, np.float32)
    beta = np.full(L * J, 0.01, np.float32)
    i16 = lambda t: t.view(torch.int16)

    # Every NVFP4 activation takes its tensor amax from its producer (bit-
    # identical codes): slots[l] holds block l's three 1024-word partial-
    # maximum arrays -- [0] its input (from block l-1's output add), [1] x1
    # (from the residual add), [2] the hidden activation (from the up
    # GEMM's epilogue) -- all zeroed by one fill at the start of a step;
    # block 0's input has no producer.  Each array doubles as the consumer
    # act_quant's 4 KB workspace.
    slots = torch.zeros((L + 1, 3, 1024), dtype=torch.int32, device=dev)
    assert qa.act_quant_workspace(qa.NVFP4, M, F_) == 4096
    sl_w = lambda l, k: slots[l, k]                       # int32 words (producer side)
    sl_ws = lambda l, k: slots[l, k].view(torch.uint8)    # the same 4 KB (consumer ws)
    lay_up = [None, None]

    def linear(fmt, x, ldx, lay, y, gelu, stream=stream, amax_out=None, amax_ws=None):
        q, sc, ts, N, K, w8 = lay
        xv = torch.as_strided(x, (M, K), (ldx, 1))
        epi = qa.EPI_GELU_TANH if gelu else qa.EPI_NONE
        if fmt == 0:
            aq = a4[0].view(-1)[: M * K // 2].view(M, K // 2)
            asc = a4[1].view(-1)[: M * K // 16].view(M, K // 16)
            if amax_ws is not None:
                qa.act_quant(qa.NVFP4, i16(xv), aq, asc, a4[2], qa.AMAX_GIVEN, amax_ws, M=M, K=K,
                             ldx=ldx, stream=stream)
            else:
                qa.act_quant(qa.NVFP4, i16(xv), aq, asc, a4[2], 0, qws, M=M, K=K, ldx=ldx,
                             stream=stream)
            if amax_out is not None:
                qa.qlinear_nvfp4_amax(aq, asc, a4[2], q, sc, ts, y, amax_out, M, N, K, epi=epi,
                                      ws=gws, stream=stream)
            else:
                qa.qlinear_nvfp4(aq, asc, a4[2], q, sc, ts, y, M, N, K, epi=epi, ws=gws,
                                 stream=stream)
        else:
            aq = a8[0].view(-1)[: M * K].view(M, K)
            qa.act_quant(qa.INT8, i16(xv), aq, a8[1], M=M, K=K, ldx=ldx, stream=stream)
            if amax_out is not None:
                qa.qlinear_int8_amax(aq, a8[1], q, sc, ts, y, amax_out, M, N, K, epi=epi, ws=gws,
                                     stream=stream, w8=w8)
            else:
                qa.qlinear_int8(aq, a8[1], q, sc, ts, y, M, N, K, epi=epi, ws=gws, stream=stream,
                                w8=w8)

    def ffn_pair(l, fu, fd, stream=stream):
        """up (GELU) and down projections of block l; the up GEMM also
        produces the hidden activation's |max| for an NVFP4 down projection,
        and the up projection's NVFP4 input takes x1's |max| from the
        residual add."""
        linear(fu, x1, H, lay_up[0], u, True, stream=stream, amax_out=sl_w(l, 2),
               amax_ws=sl_ws(l, 1))
        linear(fd, u, F_, lay_up[1], dd, False, stream=stream, amax_ws=sl_ws(l, 2))

    def apply_amax(a, b, out, target, sums2=None, stream=stream):
        qa.tdc_apply_amax(i16(a), i16(b), i16(out), target, sums2, rws, stream=stream)

    # the drifting stack inputs x_t = bf16(x_{t-1} + 0.02 N(0,1)), made once
    xs = []
    x = synth.activations(cfg, M, H, "normal")
    for t in range(steps):
        x = synth.drift(cfg, t, x)
        xs.append(torch.from_numpy(x.view(np.int16).copy()).to(dev).view(bf))

    csums = torch.zeros((L, 3), dtype=torch.float64, device=dev)
    hcsums = torch.zeros((L, 3), dtype=torch.float64).pin_memory()

    def run(mode, delta=delta, cos_rule=False, cos_probe=False):
        """cos_rule: skip on the cosine of the last two Deltas (> delta);
        cos_probe: record those cosines (DMPQ only, no skips)."""
        last, n_stored = [1] * L, [0] * L
        d_seen, cos_seen = [], []
        cos_prev = np.full(L, -1.0)
        computed_prev = np.zeros(L, np.uint8)
        d_prev = np.full(L, math.inf)
        gamma_prev, tau = None, None
        times, int8_share, skipped = [], [], 0
        for t in range(steps):
            xd = xs[t]
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            if mode == "w4a8":
                mask = np.ones(L * J, np.uint8)
            elif mode == "w4a4":
                mask = np.zeros(L * J, np.uint8)
            else:
                if gamma_prev is not None and tau is None:
                    p = np.repeat(gamma_prev, J) * alpha.astype(np.float64) + beta
                    srt = np.sort(p)
                    tau = 0.5 * (srt[(len(p) - 1) // 2] + srt[len(p) // 2])
                mask = qa.dmpq_mask(gamma_prev, alpha, beta, tau if tau is not None else 0.0, L, J)
            if mode != "full":
                skip = np.zeros(L, np.uint8)
            elif cos_rule:
                skip = qa.tdc_decide_cos(t, cos_prev, computed_prev, delta)
            else:
                skip = qa.tdc_decide(t, d_prev, computed_prev, delta)
            cur = xd
            slots.zero_()                 # one fill for every producer's amax slots
            for l in range(L):
                out = torch.empty_like(cur)
                if skip[l]:
                    apply_amax(cur, ring[l][last[l]], out, sl_w(l + 1, 0), sums[l, :2])
                    computed_prev[l] = 0
                    skipped += 1
                else:
                    m = mask[l * J:(l + 1) * J]
                    linear(m[0], cur, H, layers[l][0], qkv, False,
                           amax_ws=sl_ws(l, 0) if l else None)
                    linear(m[1], qkv.view(-1)[2 * H:], 3 * H, layers[l][1], o, False)
                    apply_amax(cur, o, x1, sl_w(l, 1))
                    lay_up[:] = layers[l][2:4]
                    ffn_pair(l, m[2], m[3])
                    apply_amax(x1, dd, out, sl_w(l + 1, 0))
                    prev = ring[l][last[l]] if n_stored[l] else None
                    nxt = last[l] ^ 1
                    qa.tdc_update(i16(cur), i16(out), None if prev is None else i16(prev),
                                  i16(ring[l][nxt]), sums[l], rws, stream=stream)
                    if (cos_rule or cos_probe) and prev is not None:
                        qa.delta_cosine(i16(ring[l][nxt]), i16(prev), csums[l], rws, stream=stream)
                    last[l] = nxt
                    n_stored[l] = min(n_stored[l] + 1, 2)
                    computed_prev[l] = 1
                cur = out
            hsums.copy_(sums, non_blocking=True)
            if cos_rule or cos_probe:
                hcsums.copy_(csums, non_blocking=True)
            torch.cuda.current_stream(dev).synchronize()
            hs = hsums.numpy()
            if cos_rule or cos_probe:
                for l in range(L):
                    if not skip[l] and n_stored[l] > 1:
                        cos_prev[l] = qa.cosine_from_sums(hcsums.numpy()[l])
                        cos_seen.append(cos_prev[l])
            gamma_prev = np.array([qa.gamma_from_sums(hs[l, :2]) for l in range(L)])
            for l in range(L):
                if not skip[l]:
                    d_prev[l] = qa.rel_l2_from_sums(hs[l]) if n_stored[l] > 1 else math.inf
                    if n_stored[l] > 1:
                        d_seen.append(d_prev[l])
            times.append(time.perf_counter() - t0)
            int8_share.append(float(mask.mean()))
        return {"ms_per_step": round(1e3 * float(np.mean(times[2:])), 2),
                "int8_share": round(float(np.mean(int8_share[2:])), 3),
                "skipped_blocks": int(skipped), "blocks_run": L * steps, "delta": delta,
                "d_median": round(float(np.median(d_seen)), 4) if d_seen else None,
                "cos_median": round(float(np.median(cos_seen)), 4) if cos_seen else None,
                "tau": tau}

    outs = None

    def run_device(tau, delta, graph, routed=True):
        """DMPQ + TDC with the decisions made on the device
        (qa.decide_step) and every path enqueued under its gate: no host
        sync inside a step (routed: the activation quantization, the GEMM and
        the Delta ring calls take their format or slot from the gate byte in
        one launch each; otherwise one gated launch per choice); graph: one step captured as a HIP graph and
        replayed.  Mean ms/step of steps 2.. (one sync around them)."""
        nonlocal outs
        if outs is None:
            outs = [torch.empty((M, H), dtype=bf, device=dev) for _ in range(L)]
        alpha_d = torch.from_numpy(alpha).to(dev)
        beta_d = torch.from_numpy(beta).to(dev)
        t_ctr = torch.zeros(1, dtype=torch.int32, device=dev)
        bstate = torch.zeros((L, 4), dtype=torch.uint8, device=dev)
        d_dev = torch.zeros(L, dtype=torch.float64, device=dev)
        blk = torch.zeros(L, dtype=torch.uint8, device=dev)
        lin = torch.zeros(L * J, dtype=torch.uint8, device=dev)
        skip_o = torch.zeros(L, dtype=torch.uint8, device=dev)
        x_in = torch.empty((M, H), dtype=bf, device=dev)

        def reset():
            for r in ring:
                for b in r:
                    b.zero_()
            for b in (sums, t_ctr, bstate, d_dev):
                b.zero_()

        def gated_linear(j, l, x, ldx, y, gelu, stream, amax_out=None, amax_ws=None):
            flag = lin[l * J + j:]
            if not routed:
                for fmt, bit in ((0, qa.ROUTE_NVFP4), (1, qa.ROUTE_INT8)):
                    with qa.gate(flag, bit):
                        linear(fmt, x, ldx, layers[l][j], y, gelu, stream=stream,
                               amax_out=amax_out, amax_ws=amax_ws)
                return
            q, sc, ts, N, K, w8 = layers[l][j]
            xv = torch.as_strided(x, (M, K), (ldx, 1))
            aq4 = a4[0].view(-1)[: M * K // 2].view(M, K // 2)
            as4 = a4[1].view(-1)[: M * K // 16].view(M, K // 16)
            aq8 = a8[0].view(-1)[: M * K].view(M, K)
            if amax_ws is not None:
                qa.act_quant_routed(flag, i16(xv), aq4, as4, a4[2], qa.AMAX_GIVEN, amax_ws, aq8,
                                    a8[1], M=M, K=K, ldx=ldx, stream=stream)
            else:
                qa.act_quant_routed(flag, i16(xv), aq4, as4, a4[2], 0, qws, aq8, a8[1], M=M, K=K,
                                    ldx=ldx, stream=stream)
            qa.qlinear_routed(flag, aq4, as4, a4[2], aq8, a8[1], q, sc, ts, w8, y, M, N, K,
                              epi=qa.EPI_GELU_TANH if gelu else qa.EPI_NONE, y_amax=amax_out,
                              ws=gws, stream=stream)

        def step(stream):
            qa.decide_step(sums, alpha_d, beta_d, tau, delta, L, J, t_ctr, bstate, d_dev, blk,
                           lin, None, skip_o, stream=stream)
            slots.zero_()                 # (on the capturing stream when captured)
            cur = x_in
            for l in range(L):
                out = outs[l]
                r0, r1 = ring[l]
                if routed:
                    qa.tdc_apply_ring(blk[l:], i16(cur), i16(r0), i16(r1), i16(out), sums[l, :2],
                                      rws, out_amax=sl_w(l + 1, 0), stream=stream)
                else:
                    for slot, bit in ((r0, qa.BLK_SKIP0), (r1, qa.BLK_SKIP1)):
                        with qa.gate(blk[l:], bit):
                            qa.tdc_apply_amax(i16(cur), i16(slot), i16(out), sl_w(l + 1, 0),
                                              sums[l, :2], rws, stream=stream)
                gated_linear(0, l, cur, H, qkv, False, stream,
                             amax_ws=sl_ws(l, 0) if l else None)
                gated_linear(1, l, qkv.view(-1)[2 * H:], 3 * H, o, False, stream)
                with qa.gate(blk[l:], qa.BLK_RUN0 | qa.BLK_RUN1):
                    qa.tdc_apply_amax(i16(cur), i16(o), i16(x1), sl_w(l, 1), None, rws,
                                      stream=stream)
                gated_linear(2, l, x1, H, u, True, stream, amax_out=sl_w(l, 2),
                             amax_ws=sl_ws(l, 1))
                gated_linear(3, l, u, F_, dd, False, stream, amax_ws=sl_ws(l, 2))
                with qa.gate(blk[l:], qa.BLK_RUN0 | qa.BLK_RUN1):
                    qa.tdc_apply_amax(i16(x1), i16(dd), i16(out), sl_w(l + 1, 0), None, rws,
                                      stream=stream)
                if routed:
                    qa.tdc_update_ring(blk[l:], i16(cur), i16(out), i16(r0), i16(r1), sums[l], rws,
                                       stream=stream)
                else:
                    for prev, nxt, bit in ((r0, r1, qa.BLK_RUN0), (r1, r0, qa.BLK_RUN1)):
                        with qa.gate(blk[l:], bit):
                            qa.tdc_update(i16(cur), i16(out), i16(prev), i16(nxt), sums[l], rws,
                                          stream=stream)
                cur = out

        g = None
        if graph:
            s = torch.cuda.Stream(device=dev)
            s.wait_stream(torch.cuda.current_stream(dev))
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(s):
                with torch.cuda.graph(g, stream=s):
                    step(s.cuda_stream)        # every launch on the capturing stream
            torch.cuda.current_stream(dev).wait_stream(s)
        reset()
        skip_acc = torch.zeros(L, dtype=torch.int32, device=dev)
        torch.cuda.synchronize()
        t0 = None
        for t in range(steps):
            if t == 2:
                torch.cuda.synchronize()
                t0 = time.perf_counter()
            x_in.copy_(xs[t])
            if graph:
                g.replay()
            else:
                step(stream)
            skip_acc += skip_o            # (enqueued: no sync)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        del g
        return {"ms_per_step": round(1e3 * dt / (steps - 2), 2), "delta": delta,
                "skipped_blocks": int(skip_acc.sum().item()), "blocks_run": L * steps,
                "decisions": "device", "graph": graph,
                "launches": "routed (one per format/slot choice)" if routed
                            else "one gated launch per choice"}

    res = {m: run(m) for m in ("w4a8", "w4a4", "dmpq", "full") if m in modes}
    # the synthetic trajectory's block updates change by d ~ d_median from
    # step to step; a threshold at that median shows the skip path's speed
    if "median" in modes and res["dmpq"]["d_median"]:
        res["full_delta_at_median_d"] = run("full", delta=res["dmpq"]["d_median"])
    # the same two configurations with the decisions on the device (no
    # per-step host sync), enqueued per step and as a replayed graph
    if "device" in modes and "full" in res:
        tau_d = res["dmpq"]["tau"]
        res["full_device"] = run_device(tau_d, delta, graph=False)
        res["full_device_graph"] = run_device(tau_d, delta, graph=True)
        res["full_device_graph_per_choice_gates"] = run_device(tau_d, delta, graph=True,
                                                               routed=False)
        if "full_delta_at_median_d" in res:
            dm = res["dmpq"]["d_median"]
            res["full_delta_at_median_d_device"] = run_device(tau_d, dm, graph=False)
            res["full_delta_at_median_d_device_graph"] = run_device(tau_d, dm, graph=True)
    # the cosine rule of Fig. 4 (a variant): threshold at the median cosine
    # of the DMPQ run's successive Deltas (an untimed probe run)
    if "cos" in modes:
        probe = run("dmpq", cos_probe=True)
        if probe["cos_median"] is not None:
            res["full_cos_at_median"] = run("full", delta=probe["cos_median"], cos_rule=True)
    res["config"] = {"blocks": L, "hidden": H, "ffn": F_, "tokens": M, "steps": steps,
                     "delta": delta, "alpha": 1.0, "beta": 0.01,
                     "block": "QKV -> value slice -> O (+res) -> up+GELU -> down (+res); "
                              "no attention mixing"}
    res["config"]["linear_TFLOP_per_step_no_skips"] = round(
        L * 2.0 * M * (3 * H * H + H * H + 2 * F_ * H) / 1e12, 2)
    res["full_vs_dmpq_speedup"] = round(res["dmpq"]["ms_per_step"] / res["full"]["ms_per_step"], 3)
    if "full_delta_at_median_d" in res:
        res["full_at_median_d_vs_dmpq_speedup"] = round(
            res["dmpq"]["ms_per_step"] / res["full_delta_at_median_d"]["ms_per_step"], 3)
    if "full_cos_at_median" in res:
        res["full_cos_vs_dmpq_speedup"] = round(
            res["dmpq"]["ms_per_step"] / res["full_cos_at_median"]["ms_per_step"], 3)
    return res


def design_ab(qa, torch, np, dev, stream, iters=2000, blocks=1024, reps=5):
    """The compute stage of the NVFP4 linear's designs on register-resident
    operands (qa_test_stage_ab): 0 = exact fp16 expansion with the group
    scales, fp16 MFMA accumulating (the library's); 1 = design S, codes as
    fp8, one fp8 MFMA per 16-element group from zero and a rescale by
    s_a s_w per output; 2 = S with the activation scale folded into fp16
    operands and a rescale by s_w.  Rates in MAC-equivalent TFLOP/s (2 x
    multiply-accumulates of the tile per second), median of `reps`."""
    rng = np.random.default_rng(7)
    blk = rng.integers(0, 1 << 32, (1024, 64), dtype=np.uint64).astype(np.uint32)
    blk[:, 12:14] = np.float32(1.5).view(np.uint32)               # scales: finite values
    blk[:, 16:64] = np.float32(0.75).view(np.uint32)
    for w in range(4, 12):                                         # fp8 bytes without NaN codes
        blk[:, w] &= 0x77777777
    blk[:, 0:4] &= 0x77777777
    blk[:, 8:16] = 0x38
    inp = torch.from_numpy(blk.view(np.int32).copy()).to(dev)
    out = torch.empty((1024, 256), dtype=torch.float32, device=dev)
    res = {}
    for design, mfmas in ((0, 16), (1, 8), (2, 8)):
        qa._lib.stage_ab(design, 10, blocks, inp, out, stream=stream)
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            qa._lib.stage_ab(design, iters, blocks, inp, out, stream=stream)
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b))
        ms = float(np.median(ts))
        macs = blocks * 4 * iters * mfmas * 32 * 32 * 16
        res[("D_fp16_exact", "S_fp8_rescale", "S_fp16_rescale")[design]] = {
            "ms": round(ms, 3), "TFLOP/s": round(2 * macs / (ms * 1e-3) / 1e12, 1)}
    best = max(res, key=lambda k: res[k]["TFLOP/s"])
    res["winner"] = best
    res["note"] = ("compute stage only, operands in registers; memory traffic is the same "
                   "4-bit codes and E4M3 scales in every design")
    return res


def sections(args, qa, torch, np, hip, dev, stream, to_dev, xd, xod, dpd, wq, wsc, wts, w8,
             aq, asc, ats, qws, a8, s8, y4, y8, ws4, ws8, dnew, applied, s4, s2, rws, M, N, K):
    """The cold bandwidth kernels, the INT8 kernel A/B and the fused FFN
    output: (cold, int8_ab, ffn_fused) of the report."""
    import synth
    n = M * K
    # the bandwidth kernels timed cold: before each rep a 1 GiB device read
    # replaces the contents of L2 and the 256 MB Infinity Cache with clean
    # lines (after a write, the write-back of its dirty lines would land in
    # the timed kernel); median of the reps
    scratch = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    gw = qa.workspace(qa.reduce_workspace(n), dev)
    gsums = torch.zeros(2, dtype=torch.float64, device=dev)
    cold_calls = [
        ("act_quant_nvfp4", 2.5625 * n, lambda: qa.act_quant(qa.NVFP4, xd, aq, asc, ats, 0, qws,
                                                             stream=stream)),
        ("act_quant_nvfp4_given_tscale", 2.5625 * n,
         lambda: qa.act_quant(qa.NVFP4, xd, aq, asc, ats, qa.TSCALE_GIVEN, None, stream=stream)),
        ("act_quant_int8", 3.0 * n + 4 * M, lambda: qa.act_quant(qa.INT8, xd, a8, s8, stream=stream)),
        ("block_gamma", 4.0 * n, lambda: qa.block_gamma(xd, xod, gsums, gw, stream=stream)),
        ("tdc_update", 8.0 * n, lambda: qa.tdc_update(xd, xod, dpd, dnew, s4, rws, stream=stream)),
        ("tdc_apply", 6.0 * n, lambda: qa.tdc_apply(xd, dnew, applied, s2, rws, stream=stream)),
    ]
    cold = {}
    for name, nbytes, fn in cold_calls:
        reps = []
        for r in range(args.cold_reps):
            scratch.sum()
            a, b = hip.event(), hip.event()
            hip.record(a, stream)
            fn()
            hip.record(b, stream)
            torch.cuda.synchronize()
            reps.append(hip.ms(a, b))
            hip.destroy(a)
            hip.destroy(b)
        t = float(np.median(reps))
        cold[name] = {"us": round(t * 1e3, 2), "GB/s": round(nbytes / (t * 1e-3) / 1e9, 1),
                      "frac_hbm": round(nbytes / (t * 1e-3) / 1e9 / PEAK["hbm_GBps"], 4),
                      "algorithmic_bytes": int(nbytes)}
    del scratch

    # the INT8 linear on its two kernels, each GEMM dispatch timed by its own
    # start/end timestamps (median of 9): integer MFMA on the weight's digit
    # planes (the path above) and fp16 MFMA on operands expanded on load
    def gemm_us(fn, reps=9):
        out = []
        for _ in range(reps):
            a, b = hip.event(), hip.event()
            qa.set_gemm_events(a.value, b.value)
            fn()
            qa.set_gemm_events(None, None)
            torch.cuda.synchronize()
            out.append(hip.ms(a, b))
            hip.destroy(a)
            hip.destroy(b)
        return float(np.median(out)) * 1e3
    int8_ab = {
        "i8_mfma_digit_planes_us": round(gemm_us(lambda: qa.qlinear_int8(
            a8, s8, wq, wsc, wts, y8, M, N, K, ws=ws8, stream=stream, w8=w8)), 1),
        "fp16_mfma_expanded_us": round(gemm_us(lambda: qa.qlinear_int8(
            a8, s8, wq, wsc, wts, y8, M, N, K, ws=ws8, stream=stream)), 1),
        "nvfp4_fp16_mfma_us": round(gemm_us(lambda: qa.qlinear_nvfp4(
            aq, asc, ats, wq, wsc, wts, y4, M, N, K, ws=ws4, stream=stream)), 1)}
    for k_ in list(int8_ab):
        int8_ab[k_.replace("_us", "_TOP/s")] = round(2.0 * M * N * K / (int8_ab[k_] * 1e-6) / 1e12, 1)

    # producer-fused activation quantization: the FFN up-projection
    # (17776 x 1920 -> 7680, GELU) writing its output as NVFP4 (given tensor
    # scale) for the down-projection, against the bf16 output followed by
    # act_quant with the same given scale; median of 9 warm calls each
    F_ = 7680
    wu = to_dev(synth.weight(3, 0, F_, K))
    wuq, wus, wuts = qa.empty_nvfp4(F_, K, dev)
    qa.act_quant(qa.NVFP4, wu, wuq, wus, wuts, 0, qa.workspace(qa.act_quant_workspace(qa.NVFP4, F_, K), dev))
    del wu
    h = torch.empty((M, F_), dtype=torch.bfloat16, device=dev)
    hq, hs, hts = qa.empty_nvfp4(M, F_, dev)
    hws = qa.workspace(qa.act_quant_workspace(qa.NVFP4, M, F_), dev)
    uws = qa.workspace(qa.qlinear_workspace(qa.NVFP4, M, F_, K), dev)
    qa.qlinear_nvfp4(aq, asc, ats, wuq, wus, wuts, h, M, F_, K, epi=qa.EPI_GELU_TANH, ws=uws,
                     stream=stream)
    qa.act_quant(qa.NVFP4, h.view(torch.int16), hq, hs, hts, 0, hws, stream=stream)   # a tensor scale
    torch.cuda.synchronize()

    def timed(fn, reps=9):
        out = []
        for _ in range(reps):
            a, b = hip.event(), hip.event()
            hip.record(a, stream)
            fn()
            hip.record(b, stream)
            torch.cuda.synchronize()
            out.append(hip.ms(a, b))
            hip.destroy(a)
            hip.destroy(b)
        return float(np.median(out)) * 1e3

    def unfused():
        qa.qlinear_nvfp4(aq, asc, ats, wuq, wus, wuts, h, M, F_, K, epi=qa.EPI_GELU_TANH, ws=uws,
                         stream=stream)
        qa.act_quant(qa.NVFP4, h.view(torch.int16), hq, hs, hts, qa.TSCALE_GIVEN, None,
                     stream=stream)

    def fused():
        qa.qlinear_nvfp4_q(aq, asc, ats, wuq, wus, wuts, hts, hq, hs, M, F_, K,
                           epi=qa.EPI_GELU_TANH, ws=uws, stream=stream)

    for _ in range(2):
        unfused()
        fused()
    t_un, t_fu = timed(unfused), timed(fused)
    ffn_fused = {"shape": [M, K, F_], "epilogue": "GELU-tanh",
                 "unfused_us": round(t_un, 1), "fused_us": round(t_fu, 1),
                 "unfused_TFLOP/s": round(2.0 * M * F_ * K / (t_un * 1e-6) / 1e12, 1),
                 "fused_TFLOP/s": round(2.0 * M * F_ * K / (t_fu * 1e-6) / 1e12, 1)}
    del h, hq, hs
    return cold, int8_ab, ffn_fused


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-rows", type=int, default=8192)
    ap.add_argument("--stack-steps", type=int, default=10,
                    help="timesteps of the 30-block stack section (0 skips it)")
    ap.add_argument("--stack5-steps", type=int, default=10,
                    help="timesteps of the 42-block 5B-shaped stack section (0 skips it)")
    ap.add_argument("--layer-reps", type=int, default=5,
                    help="timed calls per linear of the per-layer qlinear section (0 skips it)")
    ap.add_argument("--cold-reps", type=int, default=9,
                    help="reps of each bandwidth kernel timed after a 1 GiB cache-evicting read")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--step-only", action="store_true",
                    help="time the step and report it, without the other sections (cold "
                         "kernels, INT8 kernel A/B, fused FFN output, stacks, per-layer rates): "
                         "a short run whose every GEMM launch is the workload's, for profilers")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 256 MiB device-to-device copy first (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the quantized-linear path has no multi-GPU "
              "variant in this library (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mixed_precision_quantized_act_amd as qa
    import synth

    qa.lib()
    hip = Hip()
    dev = torch.device("cuda:0")

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a.copy()).to(dev)

    x, w = synth.linear_case(2)
    x_out = synth.gamma_pair(2, x)                 # the block output paired with x
    delta_prev = synth.bf16_bits(np.random.default_rng([2, 60]).standard_normal(x.shape) * 0.1)
    xd, wd, xod, dpd = to_dev(x), to_dev(w), to_dev(x_out), to_dev(delta_prev)
    n = M * K

    wq, wsc, wts = qa.empty_nvfp4(N, K, dev)
    qa.act_quant(qa.NVFP4, wd, wq, wsc, wts, 0, qa.workspace(qa.act_quant_workspace(qa.NVFP4, N, K), dev))
    w8 = qa.empty_int8_planes(N, K, dev)           # the INT8 path's digit planes (set-up)
    qa.int8_weight_planes(wq, wsc, w8, N, K)
    aq, asc, ats = qa.empty_nvfp4(M, K, dev)
    qws = qa.workspace(qa.act_quant_workspace(qa.NVFP4, M, K), dev)
    a8, s8 = qa.empty_int8_act(M, K, dev)
    y4 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    y8 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws4 = qa.workspace(qa.qlinear_workspace(qa.NVFP4, M, N, K), dev)
    ws8 = qa.workspace(qa.qlinear_workspace(qa.INT8, M, N, K), dev)
    dnew = torch.empty(n, dtype=torch.int16, device=dev)
    applied = torch.empty(n, dtype=torch.int16, device=dev)
    sums = torch.zeros(6, dtype=torch.float64, device=dev)   # tdc_update's 4, tdc_apply's 2
    s4, s2 = sums[:4], sums[4:]
    rws = qa.workspace(qa.reduce_workspace(n), dev)
    host_sums = torch.zeros(6, dtype=torch.float64).pin_memory()
    alpha = np.ones(4, np.float32)
    beta = np.full(4, 0.01, np.float32)
    stream = torch.cuda.current_stream(dev).cuda_stream

    names = ["act_quant_nvfp4", "qlinear_nvfp4", "gemm_nvfp4", "act_quant_int8", "qlinear_int8",
             "gemm_int8", "tdc_update", "tdc_apply"]
    host_np = host_sums.numpy()
    gamma_buf = np.zeros(1, np.float64)
    d_buf = np.zeros(1, np.float64)
    computed = np.ones(1, np.uint8)
    mask_out = np.zeros(4, np.uint8)
    skip_out = np.zeros(1, np.uint8)

    def step(t, ev=None, brackets=False):
        """One pass of the hot path.  `ev`: name -> (start, stop) events,
        created beforehand; the GEMM pairs take the dispatch timestamps of
        the GEMM kernels, the other pairs (only with `brackets`) are
        recorded around whole library calls."""
        def call(name, fn):
            if brackets:
                hip.record(ev[name][0], stream)
            fn()
            if brackets:
                hip.record(ev[name][1], stream)

        def gemm(name, fn):
            if ev is not None:
                qa.set_gemm_events(ev[name][0].value, ev[name][1].value)
            fn()
            if ev is not None:
                qa.set_gemm_events(None, None)

        call("act_quant_nvfp4", lambda: qa.act_quant(qa.NVFP4, xd, aq, asc, ats, 0, qws,
                                                     stream=stream))
        call("qlinear_nvfp4", lambda: gemm("gemm_nvfp4", lambda: qa.qlinear_nvfp4(
            aq, asc, ats, wq, wsc, wts, y4, M, N, K, ws=ws4, stream=stream)))
        call("act_quant_int8", lambda: qa.act_quant(qa.INT8, xd, a8, s8, stream=stream))
        call("qlinear_int8", lambda: gemm("gemm_int8", lambda: qa.qlinear_int8(
            a8, s8, wq, wsc, wts, y8, M, N, K, ws=ws8, stream=stream, w8=w8)))
        call("tdc_update", lambda: qa.tdc_update(xd, xod, dpd, dnew, s4, rws, stream=stream))
        call("tdc_apply", lambda: qa.tdc_apply(xd, dnew, applied, s2, rws, stream=stream))
        host_sums.copy_(sums, non_blocking=True)
        torch.cuda.current_stream(dev).synchronize()
        gamma_buf[0] = qa.gamma_from_sums(host_np[4:6])
        d_buf[0] = qa.rel_l2_from_sums(host_np[:4])
        qa.dmpq_mask(gamma_buf, alpha, beta, 0.1, 1, 4, out=mask_out)
        qa.tdc_decide(t, d_buf, computed, 0.05, out=skip_out)

    def make_events(keys):
        return [{k: (hip.event(), hip.event()) for k in keys} for _ in range(args.steps)]

    if args.calib_copy:
        # a 256 MiB device copy whose source was written and then evicted
        # from the caches by reading 2 GiB of other data
        src = torch.ones(1 << 28, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        flush = torch.ones(1 << 29, dtype=torch.int32, device=dev)
        flush.sum()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst, flush
    for t in range(args.warmup):
        step(t)
    # timed steps: only the two GEMM dispatches carry (in-packet) events
    timed_ev = make_events(["gemm_nvfp4", "gemm_int8"])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(args.steps):
        step(t, timed_ev[t])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # per-call breakdown of the other kernels: as many extra steps, with
    # event markers around every library call (outside the timed region)
    split_ev = make_events(names)
    for t in range(args.steps):
        step(t, split_ev[t], brackets=True)
    torch.cuda.synchronize()
    ev = {k: [] for k in names}
    for evs, keys in ((timed_ev, ("gemm_nvfp4", "gemm_int8")),
                      (split_ev, [k for k in names if not k.startswith("gemm_")])):
        for pairs in evs:
            for k in keys:
                a, b = pairs[k]
                ev[k].append(hip.ms(a, b))
    for evs in (timed_ev, split_ev):
        for pairs in evs:
            for a, b in pairs.values():
                hip.destroy(a)
                hip.destroy(b)
    avg = {k: float(np.mean(v)) for k, v in ev.items() if v}

    cold = int8_ab = ffn_fused = design = None
    if not args.step_only:
        design = design_ab(qa, torch, np, dev, stream)
        cold, int8_ab, ffn_fused = sections(args, qa, torch, np, hip, dev, stream, to_dev, xd, xod,
                                            dpd, wq, wsc, wts, w8, aq, asc, ats, qws, a8, s8,
                                            y4, y8, ws4, ws8, dnew, applied, s4, s2, rws, M, N, K)
    stack = (stack_section(qa, torch, np, dev, stream, steps=args.stack_steps)
             if args.stack_steps > 0 and not args.step_only else None)
    ffn3 = (ffn_section(qa, torch, np, dev, stream)
            if args.layer_reps > 0 and not args.step_only else None)
    layers2b = (layer_rates(qa, torch, np, dev, stream, M, 1920, 7680, reps=args.layer_reps)
                if args.layer_reps > 0 and not args.step_only else None)
    # a launch-bound stack (30 blocks of the single-linear config's width:
    # H 256, FFN 1024, 256 tokens), where the per-step host sync and the
    # launches, not the kernels, set the step time
    small = None
    if args.stack_steps > 0 and not args.step_only:
        small = stack_section(qa, torch, np, dev, stream, L=30, H=256, F_=1024, M=256,
                              steps=args.stack_steps, cfg=1,
                              modes=("dmpq", "full", "median", "device"))
    stack5 = None
    if args.stack5_steps > 0 and not args.step_only:
        stack5 = stack_section(qa, torch, np, dev, stream, L=42, H=3072, F_=12288, M=M,
                               steps=args.stack5_steps, cfg=5,
                               modes=("dmpq", "full", "median", "device"))
        if args.layer_reps > 0:
            stack5["per_layer_qlinear"] = layer_rates(qa, torch, np, dev, stream, M, 3072, 12288,
                                                      reps=args.layer_reps)

    ms_step = wall * 1e3 / args.steps
    flops_step = 2 * 2.0 * M * N * K
    value = flops_step / (ms_step * 1e-3) / 1e12

    def tf(ms):
        return 2.0 * M * N * K / (ms * 1e-3) / 1e12

    def gbs(nbytes, ms):
        return nbytes / (ms * 1e-3) / 1e9

    kern = {
        "gemm_nvfp4": {"us": avg["gemm_nvfp4"] * 1e3, "TFLOP/s": tf(avg["gemm_nvfp4"]),
                       "issued_dtype": "fp16 MFMA on NVFP4 dequantized exactly on load",
                       "frac_fp4_peak": tf(avg["gemm_nvfp4"]) / PEAK["fp4_TFLOPs"],
                       "frac_fp16_peak": tf(avg["gemm_nvfp4"]) / PEAK["bf16_TFLOPs"]},
        "qlinear_nvfp4_call": {"us": avg["qlinear_nvfp4"] * 1e3, "TFLOP/s": tf(avg["qlinear_nvfp4"])},
        "gemm_int8": {"us": avg["gemm_int8"] * 1e3, "TOP/s": tf(avg["gemm_int8"]),
                      "issued_dtype": "i8 MFMA, int32 sums, against the weight's two int8 "
                                      "digit planes (2 issued ops per algorithmic op)",
                      "frac_int8_peak": tf(avg["gemm_int8"]) / PEAK["int8_TOPs"],
                      "frac_int8_peak_issued": 2 * tf(avg["gemm_int8"]) / PEAK["int8_TOPs"]},
        "qlinear_int8_call": {"us": avg["qlinear_int8"] * 1e3, "TOP/s": tf(avg["qlinear_int8"])},
        "act_quant_nvfp4": {"us": avg["act_quant_nvfp4"] * 1e3,
                            "GB/s": gbs(2.5625 * n, avg["act_quant_nvfp4"])},
        "act_quant_int8": {"us": avg["act_quant_int8"] * 1e3,
                           "GB/s": gbs(3.0 * n + 4 * M, avg["act_quant_int8"])},
        "tdc_update": {"us": avg["tdc_update"] * 1e3, "GB/s": gbs(8.0 * n, avg["tdc_update"])},
        "tdc_apply": {"us": avg["tdc_apply"] * 1e3, "GB/s": gbs(6.0 * n, avg["tdc_apply"])},
    }
    for k in ("act_quant_nvfp4", "act_quant_int8", "tdc_update", "tdc_apply"):
        kern[k]["frac_hbm"] = kern[k]["GB/s"] / PEAK["hbm_GBps"]
    for v in kern.values():
        for kk in list(v):
            if isinstance(v[kk], float):
                v[kk] = round(v[kk], 4)

    # dominant kernel: the longer of the two GEMM kernels, against the peak
    # of its own contraction's dtype (INT8: 5.0 POP/s; NVFP4 x NVFP4: the FP4
    # figure, 10.1 PFLOP/s); `issued` gives the fraction of the peak of the
    # MFMA actually issued (INT8: i8 at twice the algorithmic ops; NVFP4:
    # fp16, 2.5 PFLOP/s)
    dom = "gemm_int8" if avg["gemm_int8"] >= avg["gemm_nvfp4"] else "gemm_nvfp4"
    ach = tf(avg[dom])
    if dom == "gemm_int8":
        peak, unit, dt = PEAK["int8_TOPs"], "TOP/s", "int8"
        issued = {"dtype": "i8 (two digit planes)", "peak": PEAK["int8_TOPs"],
                  "frac": round(2 * ach / PEAK["int8_TOPs"], 4)}
    else:
        peak, unit, dt = PEAK["fp4_TFLOPs"], "TFLOP/s", "nvfp4"
        issued = {"dtype": "fp16", "peak": PEAK["bf16_TFLOPs"],
                  "frac": round(ach / PEAK["bf16_TFLOPs"], 4)}
    roofline = {"bound": "mfma", "kernel": dom, "dtype": dt, "achieved": round(ach, 2),
                "peak": peak, "unit": unit, "frac": round(ach / peak, 4),
                "traffic": measured_traffic(dom), "issued": issued,
                "counters": measured_mfma(dom)}
    # memory per weight element: bf16 2 B; NVFP4 0.5 B codes + 1/16 B scales;
    # the INT8 path's digit planes 2 B more (kept beside the NVFP4 weight)
    context = {"pages": PAGES_CONTEXT,
               "this_run": {
                   "weight_bytes_per_param": {"bf16": 2.0, "nvfp4": 0.5625,
                                              "int8_digit_planes": 2.0},
                   "weight_memory_ratio_bf16_over_nvfp4": round(2.0 / 0.5625, 3)}}
    if stack:
        context["this_run"]["stack_2b_full_vs_dmpq_at_delta_0.05"] = stack["full_vs_dmpq_speedup"]
        if "full_at_median_d_vs_dmpq_speedup" in stack:
            context["this_run"]["stack_2b_full_vs_dmpq_at_median_d"] = \
                stack["full_at_median_d_vs_dmpq_speedup"]
        context["this_run"]["stack_2b_dmpq_vs_uniform_w4a8"] = round(
            stack["w4a8"]["ms_per_step"] / stack["dmpq"]["ms_per_step"], 3)

    line = {
        "metric": "qlinear TFLOP/s (NVFP4 & INT8 A-paths) + quant/TDC GB/s, % of roofline",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "nvfp4+int8 (NVFP4: fp16 MFMA on exact values; INT8: i8 MFMA, int32)",
        "data": "synthetic",
        "config": {"workload": "cogvideox2b-qkv", "M": M, "K": K, "N": N,
                   "activations": "N(0,1) bf16, 19 outlier channels x30",
                   "weights": "N(0,0.02^2) -> NVFP4", "parallelism": "none (1 GPU)"},
        "kernels": kern,
        "int8_kernel_ab": int8_ab,
        "cold": cold,
        "ffn_up_fused_nvfp4_output": ffn_fused,
        "nvfp4_design_ab": design,
        "stack_cogvideox2b_shape": stack,
        "per_layer_qlinear_cogvideox2b_shape": layers2b,
        "ffn_student_t": ffn3,
        "stack_cogvideox5b_shape": stack5,
        "stack_launch_bound_256_tokens": small,
        "roofline": roofline,
        "context": context,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(x, w, x_out, delta_prev, args.cpu_rows)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
