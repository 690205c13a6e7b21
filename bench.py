#!/usr/bin/env python3
"""Benchmark: RIB window attention with the CLA gate on one MI355X.

One step = the whole hot path over one batch of resident synthetic input:
rib_encode (positional factors for the window size) + rib_window_attn
(fused window attention, bf16 MFMA).  The headline workload is the SST
training-patch forward: 32 images of 96x96 tokens, C = 180 (6 heads x 30),
R = 16, one 96x96 window per image.  Secondary figures for the 64x64 window
(1x180x320, C = 180), the 640x360 input with 96x96 windows, and the 16x16
window of the SST-lite map (HBM-bound) are reported in the same JSON line, and so is the
CLA gate producer (rib_cla_gate, HBM-bound) and the LayerNorm + Q/K/V projection
(rib_ln_qkv, HBM-bound) on the same maps, that projection with its Q side moved into the
attention (rib_window_attn_lnq) against the unfused pair, space-time windows on an 8-frame
video map (rib_window_attn3d), and the
training iteration of the attention (rib_window_attn_train + rib_window_attn_backward +
rib_encode_backward) on the 96x96 and 64x64 workloads.

Prints ONE JSON line.  Timing: HIP events on the stream the kernels run on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk/CU
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
ATTN_SRC = os.path.join(ROOT, "super_resolution_transformer_amd", "csrc", "attn_bf16.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bf16_train96_traffic.txt")


def algorithmic(B, H, W, heads, dh, R, ws, elt):
    """Score pairs E, flops F and bytes M of one rib_window_attn call (real tokens only)."""
    nwy, nwx = -(-H // ws), -(-W // ws)
    pairs = 0
    for wy in range(nwy):
        for wx in range(nwx):
            n = min(ws, H - wy * ws) * min(ws, W - wx * ws)
            pairs += n * n
    E = B * heads * pairs
    F = E * (2 * (dh + R) + 2 * dh)
    M = B * H * W * heads * dh * 5 * elt + 2 * ws * ws * R * 4
    return E, F, M


def source_sha(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it still
    describes the current kernel source (else None)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != source_sha(ATTN_SRC):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Workload:
    def __init__(self, torch, rib, synthetic, cfg_idx, ws, copies=1):
        c = synthetic.CONFIGS[cfg_idx]
        self.cfg, self.ws = c, ws
        p = synthetic.config_problem(cfg_idx)
        self.p = p
        bf = lambda nm: torch.from_numpy(p.bits[nm].view("int16")).view(torch.bfloat16).cuda()
        base = [bf(n) for n in ("qc", "kc", "v", "g")]
        self.sets = [base] + [[t.clone() for t in base] for _ in range(copies - 1)]
        self.outs = [torch.empty_like(base[0]) for _ in range(copies)]
        self.w = torch.from_numpy(p.weights).cuda()
        n = ws * ws
        self.qp = torch.empty((n, c.R), dtype=torch.float32, device="cuda")
        self.kp = torch.empty_like(self.qp)
        self.rib = rib
        self.k = 0
        self.E, self.F, self.M = algorithmic(c.B, c.H, c.W, c.heads, c.dh, c.R, ws, 2)
        self.tokens = c.B * c.H * c.W

    def encode(self):
        c = self.cfg
        self.rib.encode_into(self.ws, c.L, c.hidden, c.R, self.w, self.qp, self.kp)

    def attn(self):
        c = self.cfg
        i = self.k % len(self.sets)
        self.k += 1
        qc, kc, v, g = self.sets[i]
        self.rib.window_attn_into(qc, kc, v, g, self.qp, self.kp, c.heads, self.ws, self.outs[i])


def time_steps(torch, wl, steps, warmup):
    """Whole-step timing plus per-launch timing of the attention kernel, HIP events on the
    current stream (the stream the library launches on)."""
    for _ in range(warmup):
        wl.encode()
        wl.attn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for a, b, c in ev:
        a.record()
        wl.encode()
        b.record()
        wl.attn()
        c.record()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(stop)
    enc_ms = sorted(a.elapsed_time(b) for a, b, _ in ev)
    attn_ms = sorted(b.elapsed_time(c) for _, b, c in ev)
    return total_ms / steps, sum(enc_ms) / steps, sum(attn_ms) / steps, attn_ms, wall


def time_attn_only(torch, wl, reps, warmup):
    for _ in range(warmup):
        wl.attn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        wl.attn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps


def time_gate(torch, rib, synthetic):
    """CLA gate producer G = PWConv1x1(DWConv3x3(X)) on the workloads' maps (bf16); HBM roofline.
    Algorithmic bytes: X read + G written (bf16) + fp32 weights; input sets rotate so that the
    maps are not served from the 256 MB MALL."""
    res = {}
    for name, (B, H, W, C, copies) in (("32x96x96, C=180", (32, 96, 96, 180, 3)),
                                       ("1x360x640, C=180", (1, 360, 640, 180, 3)),
                                       ("1x180x320, C=48", (1, 180, 320, 48, 40))):
        p = synthetic.make_gate_problem(B, H, W, C, "bf16", seed=7)
        x0 = torch.from_numpy(p.x_bits.view("int16")).view(torch.bfloat16).cuda()
        xs = [x0] + [x0.clone() for _ in range(copies - 1)]
        gs = [torch.empty_like(x0) for _ in range(copies)]
        w = [torch.from_numpy(a).cuda() for a in (p.dw_w, p.dw_b, p.pw_w, p.pw_b)]
        reps = max(100, 2 * copies)
        for i in range(copies):
            rib.cla_gate_into(xs[i], *w, gs[i])
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for i in range(reps):
            rib.cla_gate_into(xs[i % copies], *w, gs[i % copies])
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / reps
        nbytes = 2 * B * H * W * C * 2 + 4 * (C * 9 + C + C * C + C)
        flops = B * H * W * (18 * C + 2 * C * C)
        res[name] = {"ms": ms, "alg_gbs": nbytes / (ms * 1e-3) / 1e9,
                     "pct_hbm": 100 * nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                     "tflops": flops / (ms * 1e-3) / 1e12, "tokens_per_s": B * H * W / (ms * 1e-3)}
        del xs, gs
        torch.cuda.empty_cache()
    return res


def time_space_time(torch, rib, synthetic):
    """Space-time windows on a video map (rib_encode3d once, then rib_window_attn3d timed): 8 frames of the
    SST inference map 180x320, C=180 (6 heads x dh 30), R=16, bf16; windows 2x32x32 and 4x16x16."""
    res = {}
    B, T, H, W, heads, dh, R, L, hidden = 1, 8, 180, 320, 6, 30, 16, 10, 64
    p = synthetic.make_problem(B * T, H, W, heads, dh, R, dtype="bf16", seed=12)
    maps = [torch.from_numpy(p.bits[n].view("int16")).view(torch.bfloat16).cuda().view(B, T, H, W, heads * dh)
            for n in ("qc", "kc", "v", "g")]
    rng = __import__("numpy").random.default_rng(13)
    F = 3 + 6 * L
    w = torch.tensor(rng.standard_normal(F * hidden + hidden + 2 * hidden * R), dtype=torch.float32).cuda() * 0.1
    for wt, ws in ((2, 32), (4, 16)):
        qp, kp = rib.encode3d(wt, ws, L, hidden, R, w)
        for _ in range(5):
            rib.window_attn3d(*maps, qp, kp, heads, wt, ws)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 50
        s.record()
        for _ in range(reps):
            rib.window_attn3d(*maps, qp, kp, heads, wt, ws)
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / reps
        pairs = 0
        for t0 in range(0, T, wt):
            for y0 in range(0, H, ws):
                for x0 in range(0, W, ws):
                    n = (min(T, t0 + wt) - t0) * (min(H, y0 + ws) - y0) * (min(W, x0 + ws) - x0)
                    pairs += n * n
        flops = B * heads * pairs * (2 * (dh + R) + 2 * dh)
        tf = flops / (ms * 1e-3) / 1e12
        res[f"{wt}x{ws}x{ws} windows, 8 x 180x320, C=180"] = {
            "ms_attn": ms, "tokens_per_s": B * T * H * W / (ms * 1e-3), "tflops": tf,
            "pct_bf16_peak": 100 * tf / PEAK_BF16_TFLOPS}
    del maps
    torch.cuda.empty_cache()
    return res


def time_cyclic(torch, rib, synthetic):
    """The cyclic window schedule (16, 32, 64) on the SST-lite shape (1 x 180x320, C=48, 3 heads x dh 16, R=16,
    bf16) and on the inference shape (C=180, 6 heads x dh 30): three independent rib_window_attn calls one
    after another, and the same three calls in one rib_window_attn_multi."""
    res = {}
    for label, heads, dh in (("1x180x320, C=48", 3, 16), ("1x180x320, C=180", 6, 30)):
        calls = []
        pairs = 0
        for k, ws in enumerate((16, 32, 64)):
            p = synthetic.make_problem(1, 180, 320, heads, dh, 16, dtype="bf16", seed=40 + k)
            maps = [torch.from_numpy(p.bits[n].view("int16")).view(torch.bfloat16).cuda() for n in ("qc", "kc", "v", "g")]
            qp, kp = rib.encode(ws, p.L, p.hidden, p.R, torch.from_numpy(p.weights).cuda())
            calls.append((*maps, qp, kp, heads, ws))
            for y0 in range(0, 180, ws):
                for x0 in range(0, 320, ws):
                    n = (min(180, y0 + ws) - y0) * (min(320, x0 + ws) - x0)
                    pairs += n * n
        outs = [torch.empty_like(c[0]) for c in calls]

        def timed(fn, reps=50):
            for _ in range(5):
                fn()
            torch.cuda.synchronize()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(reps):
                fn()
            e.record()
            torch.cuda.synchronize()
            return s.elapsed_time(e) / reps
        ms_sep = timed(lambda: [rib.window_attn_into(*c, o) for c, o in zip(calls, outs)])
        ms_multi = timed(lambda: rib.window_attn_multi_into(calls, outs))
        flops = heads * pairs * (2 * (dh + 16) + 2 * dh)
        res[f"windows 16+32+64, {label}"] = {
            "ms_three_calls": ms_sep, "ms_one_multi_call": ms_multi,
            "tflops_multi": flops / (ms_multi * 1e-3) / 1e12,
            "pct_bf16_peak_multi": 100 * flops / (ms_multi * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        del calls, outs
        torch.cuda.empty_cache()
    return res


def time_ln_qkv(torch, rib, synthetic):
    """Block input projection (rib_ln_qkv: LayerNorm, then x W + b into Q | K | V, plus LN(X) for the
    gate) on the workloads' maps, bf16; HBM roofline.  Algorithmic bytes: X read, Q, K, V and LN(X)
    written (bf16) + fp32 parameters; input sets rotate."""
    res = {}
    for name, (B, H, W, C, copies) in (("32x96x96, C=180", (32, 96, 96, 180, 2)),
                                       ("1x360x640, C=180", (1, 360, 640, 180, 3)),
                                       ("1x180x320, C=48", (1, 180, 320, 48, 40))):
        p = synthetic.make_ln_qkv_problem(B, H, W, C, "bf16", seed=3)
        x0 = torch.from_numpy(p.x_bits.view("int16")).view(torch.bfloat16).cuda()
        xs = [x0] + [x0.clone() for _ in range(copies - 1)]
        outs = [[torch.empty_like(x0) for _ in range(4)] for _ in range(copies)]
        w = [torch.from_numpy(a).cuda() for a in (p.gamma, p.beta, p.w, p.bias)]
        reps = max(100, 2 * copies)
        for i in range(copies):
            rib.ln_qkv_into(xs[i], *w, *outs[i])
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for i in range(reps):
            rib.ln_qkv_into(xs[i % copies], *w, *outs[i % copies])
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / reps
        nbytes = 5 * B * H * W * C * 2 + 4 * (2 * C + 3 * C * C + 3 * C)
        flops = B * H * W * 2 * C * 3 * C
        res[name] = {"ms": ms, "alg_gbs": nbytes / (ms * 1e-3) / 1e9,
                     "pct_hbm": 100 * nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                     "tflops": flops / (ms * 1e-3) / 1e12, "tokens_per_s": B * H * W / (ms * 1e-3)}
        del xs, outs
        torch.cuda.empty_cache()
    return res


def time_backward(torch, rib, synthetic, cfg_idx, ws, reps):
    """Training iteration of the attention on one workload: rib_window_attn_train (O and the row
    log-sum-exp), rib_window_attn_backward (dQc, dKc, dV, dG, dQp, dKp) and rib_encode_backward
    (the encoder's weight gradient).  Inputs, outputs and workspaces are allocated before timing.
    Algorithmic flops of the backward per score pair: recomputed scores 2(dh+R), dP = dA V^T 2dh,
    dV = P^T dA 2dh, dQt = dS Kt 2(dh+R), dKt = dS^T Qt 2(dh+R)."""
    c = synthetic.CONFIGS[cfg_idx]
    p = synthetic.config_problem(cfg_idx)
    bf = lambda bits: torch.from_numpy(bits.view("int16")).view(torch.bfloat16).cuda()
    maps = [bf(p.bits[n]) for n in ("qc", "kc", "v", "g")]
    w = torch.from_numpy(p.weights).cuda()
    qp, kp = rib.encode(ws, c.L, c.hidden, c.R, w)
    _, dbits = synthetic.make_upstream_grad(p.qc.shape, "bf16", seed=1)
    dout = bf(dbits)
    o, lse = rib.window_attn_train(*maps, qp, kp, c.heads, ws)
    grads = [torch.empty_like(maps[0]) for _ in range(4)] + [torch.empty_like(qp), torch.empty_like(kp)]
    work = torch.empty(rib.backward_workspace_bytes(maps[0], qp, c.heads, ws), dtype=torch.uint8, device="cuda")
    dw = torch.empty_like(w)
    ework = torch.empty(max(16, rib.lib().rib_encode_backward_workspace(ws, c.L, c.hidden, c.R)),
                        dtype=torch.uint8, device="cuda")

    def fwd():
        rib.window_attn_train_into(*maps, qp, kp, c.heads, ws, o, lse)

    def bwd():
        rib.window_attn_backward_into(*maps, qp, kp, o, lse, dout, c.heads, ws, *grads, work)

    def ebwd():
        rib.encode_backward_into(ws, c.L, c.hidden, c.R, w, grads[4], grads[5], dw, ework)

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps

    ms_f, ms_b, ms_e = timed(fwd), timed(bwd), timed(ebwd)
    E, F, _ = algorithmic(c.B, c.H, c.W, c.heads, c.dh, c.R, ws, 2)
    Fb = E * (6 * (c.dh + c.R) + 4 * c.dh)
    tf_b = Fb / (ms_b * 1e-3) / 1e12
    tokens = c.B * c.H * c.W
    ms_step = ms_f + ms_b + ms_e
    return {"workload": f"{c.name}: {c.B} x {c.H}x{c.W}, C={c.C} ({c.heads} heads x dh {c.dh}), R={c.R}, "
                        f"{ws}x{ws} windows",
            "ms_train_forward": ms_f, "ms_backward": ms_b, "ms_encode_backward": ms_e,
            "ms_train_step": ms_step, "train_tokens_per_s": tokens / (ms_step * 1e-3),
            "backward_tflops": tf_b, "backward_pct_bf16_peak": 100 * tf_b / PEAK_BF16_TFLOPS,
            "backward_algorithmic_flop": Fb,
            "roofline": {"bound": "mfma", "achieved": tf_b, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": tf_b / PEAK_BF16_TFLOPS, "traffic": None,
                         "kernel": "rib_window_attn_backward (prep, two packs, dq, dkv, table reduce)"}}


def copy_calibration(torch):
    """Three plain device copies of 2^28 float32 (1 GiB read, 1 GiB written): the reference that
    scales rocprofv3's FETCH_SIZE / WRITE_SIZE counters to bytes."""
    x = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    return {"read": x.numel() * 4, "write": y.numel() * 4}


# forward workloads that --only times alone: (label, config index, window, rotating input sets)
ONLY = {
    "sst-train-96": ("96x96 window, 32x96x96, C=180", 4, 96, 1),
    "sst-infer-64": ("64x64 window, 1x180x320, C=180", 3, 64, 1),
    "large-96": ("96x96 window, 1x360x640 (640x360 input), C=180", 5, 96, 1),
    "sst-lite-16": ("16x16 window, 1x180x320, C=48 (40 rotating input sets)", 2, 16, 40),
    "sst-lite-32": ("32x32 window, 1x180x320, C=48", 2, 32, 1),
    "sst-lite-64": ("64x64 window, 1x180x320, C=48", 2, 64, 1),
}


def cpu_baseline(synthetic, cfg_idx, ws, units_sample):
    """The fp64 oracle as it stands, on the host cores, over a bounded sample of
    (image, window, head) units of the same workload, scaled to tokens/s."""
    import oracle
    p = synthetic.config_problem(cfg_idx)
    c = synthetic.CONFIGS[cfg_idx]
    qp, kp = oracle.encode(ws, c.L, c.hidden, c.R, p.weights)
    total_units = oracle.units(c.B, c.H, c.W, c.heads, ws)
    units_sample = min(units_sample, total_units)
    t0 = time.perf_counter()
    oracle.window_attn(p.qc, p.kc, p.v, p.g, qp, kp, c.heads, ws, unit_range=(0, units_sample))
    dt = time.perf_counter() - t0
    full = dt * total_units / units_sample           # all units are full 96x96 windows here
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": c.B * c.H * c.W / full,
        "unit": "tokens/s",
        "cores": oracle.threads(),
        "cpu_model": model,
        "kind": "oracle",
        "sample": f"{units_sample} of {total_units} (image, window, head) units of the same workload "
                  f"(each a full {ws}x{ws} window, 1 head), {dt:.1f} s, scaled by unit count",
    }


def time_fused_q(torch, rib, synthetic):
    """The block's input projection plus the attention, two ways, on the 96x96-window maps:
    unfused = rib_ln_qkv (Q, K, V, LN(X)) then rib_window_attn; fused = rib_ln_qkv without Q then
    rib_window_attn_lnq (LayerNorm and the Q projection inside the attention's query prologue)."""
    res = {}
    for name, (B, H, W, heads, dh, ws, cfg_idx) in (("96x96 window, 32x96x96, C=180", (32, 96, 96, 6, 30, 96, 4)),
                                                   ("96x96 window, 1x360x640, C=180", (1, 360, 640, 6, 30, 96, 5))):
        C = heads * dh
        c = synthetic.CONFIGS[cfg_idx]
        lp = synthetic.make_ln_qkv_problem(B, H, W, C, "bf16", seed=3)
        x = torch.from_numpy(lp.x_bits.view("int16")).view(torch.bfloat16).cuda()
        prm = [torch.from_numpy(a).cuda() for a in (lp.gamma, lp.beta, lp.w, lp.bias)]
        weights = synthetic.make_problem(1, 8, 8, heads, dh, c.R, c.L, c.hidden, "bf16", c.seed).weights
        gen = torch.Generator(device="cuda")
        gen.manual_seed(c.seed)
        g = torch.empty_like(x).normal_(generator=gen)   # gate pre-activation ~ N(0, 1)
        qp, kp = rib.encode(ws, c.L, c.hidden, c.R, torch.from_numpy(weights).cuda())
        q, k, v, xn, o = (torch.empty_like(x) for _ in range(5))
        unfused = lambda: (rib.ln_qkv_into(x, *prm, q, k, v, xn), rib.window_attn_into(q, k, v, g, qp, kp, heads, ws, o))
        fused = lambda: (rib.ln_qkv_into(x, *prm, None, k, v, xn),
                         rib.window_attn_lnq_into(x, *prm, k, v, g, qp, kp, heads, ws, o))
        r = {}
        for tag, fn in (("unfused", unfused), ("fused", fused)):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(20):
                fn()
            e.record()
            torch.cuda.synchronize()
            r["ms_" + tag] = s.elapsed_time(e) / 20
        r["fused_over_unfused"] = r["ms_fused"] / r["ms_unfused"]
        res[name] = r
        del x, q, k, v, xn, o, g
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extra", action="store_true", help="skip the secondary window sizes")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-units", type=int, default=0,
                    help="oracle sample size in window-head units (default: 2 per oracle thread)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for scaling rocprofv3 byte counters)")
    ap.add_argument("--backward-only", action="store_true",
                    help="time only the training iteration (train forward + backward) on the 96x96 workload")
    ap.add_argument("--backward-reps", type=int, default=10, help="timed repetitions per backward call")
    ap.add_argument("--only", choices=sorted(ONLY), default=None,
                    help="time one forward workload alone and print its line (for profiler passes)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        msg = ("bench.py measures one GPU: this path needs no inter-GPU exchange and this build "
               "runs on a single MI355X; --gpus must be 1")
        print(json.dumps({"error": msg, "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch
    import super_resolution_transformer_amd as rib
    from super_resolution_transformer_amd import synthetic
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    rib.lib()

    if args.only:
        name, cfg_idx, ws, copies = ONLY[args.only]
        wl = Workload(torch, rib, synthetic, cfg_idx, ws, copies=copies)
        wl.encode()
        ms = time_attn_only(torch, wl, reps=args.steps, warmup=args.warmup)
        tf = wl.F / (ms * 1e-3) / 1e12
        out = {"only": name, "ms_attn": ms, "tokens_per_s": wl.tokens / (ms * 1e-3), "tflops": tf,
               "pct_bf16_peak": 100 * tf / PEAK_BF16_TFLOPS, "alg_bytes": wl.M,
               "alg_gbs": wl.M / (ms * 1e-3) / 1e9, "pct_hbm": 100 * wl.M / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
        if args.copy_calibration:
            out["copy_calibration_bytes"] = copy_calibration(torch)
        print(json.dumps(out), flush=True)
        return

    if args.backward_only:
        print(json.dumps({"backward": {"96x96 window, 32x96x96": time_backward(torch, rib, synthetic, 4, 96,
                                                                                args.backward_reps)}}), flush=True)
        return

    # ---- headline workload: 32 x 96x96 patches, 96x96 window
    wl = Workload(torch, rib, synthetic, 4, 96)
    ms_step, ms_enc, ms_attn, attn_list, wall = time_steps(torch, wl, args.steps, args.warmup)
    tflops = wl.F / (ms_attn * 1e-3) / 1e12
    traffic = read_traffic()
    out = {
        "metric": "RIB window-attn tokens/s + TFLOP/s (% bf16 MFMA peak) at 64x64 and 96x96 windows",
        "value": wl.tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "sst-train-bf16: 32 x 96x96 map, C=180 (6 heads x dh 30), R=16, "
                               "L=10, hidden 64, one 96x96 window per image",
                   "B": 32, "H": 96, "W": 96, "C": 180, "heads": 6, "dh": 30, "R": 16, "window": 96,
                   "step": "rib_encode + rib_window_attn"},
        "tflops": tflops,
        "pct_bf16_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
        "ms_attn": ms_attn,
        "ms_encode": ms_enc,
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / PEAK_BF16_TFLOPS, "traffic": traffic,
                     "kernel": "attn_bf16_chunk_kernel<30,16,4>", "algorithmic_flop_per_launch": wl.F,
                     "launch_ms_p10_p50_p90": [attn_list[len(attn_list) // 10], attn_list[len(attn_list) // 2],
                                               attn_list[(9 * len(attn_list)) // 10]]},
    }
    del wl
    torch.cuda.empty_cache()

    if not args.no_extra:
        extra = {}
        for name, cfg_idx, ws, copies in (("64x64 window, 1x180x320, C=180", 3, 64, 1),
                                          ("96x96 window, 1x360x640 (640x360 input), C=180", 5, 96, 1),
                                          ("32x32 window, 1x180x320, C=48", 2, 32, 1),
                                          ("64x64 window, 1x180x320, C=48", 2, 64, 1),
                                          ("16x16 window, 1x180x320, C=48 (HBM-bound; 40 rotating input sets)",
                                           2, 16, 40)):
            w2 = Workload(torch, rib, synthetic, cfg_idx, ws, copies=copies)
            w2.encode()
            ms = time_attn_only(torch, w2, reps=max(100, 2 * copies), warmup=max(10, copies))
            tf = w2.F / (ms * 1e-3) / 1e12
            extra[name] = {"ms_attn": ms, "tokens_per_s": w2.tokens / (ms * 1e-3), "tflops": tf,
                           "pct_bf16_peak": 100 * tf / PEAK_BF16_TFLOPS,
                           "alg_gbs": w2.M / (ms * 1e-3) / 1e9,
                           "pct_hbm": 100 * w2.M / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
            del w2
            torch.cuda.empty_cache()
        out["other_windows"] = extra

    if not args.no_extra:
        out["cla_gate"] = time_gate(torch, rib, synthetic)
        out["ln_qkv"] = time_ln_qkv(torch, rib, synthetic)
        out["fused_q_projection"] = time_fused_q(torch, rib, synthetic)
        out["space_time"] = time_space_time(torch, rib, synthetic)
        out["cyclic_schedule"] = time_cyclic(torch, rib, synthetic)
        out["backward"] = {"96x96 window, 32x96x96": time_backward(torch, rib, synthetic, 4, 96, args.backward_reps),
                           "64x64 window, 1x180x320": time_backward(torch, rib, synthetic, 3, 64,
                                                                    3 * args.backward_reps)}
        torch.cuda.empty_cache()

    if args.copy_calibration:
        out["copy_calibration_bytes"] = copy_calibration(torch)

    if not args.no_cpu:
        import oracle
        units = args.cpu_units or 2 * oracle.threads()
        out["cpu_baseline"] = cpu_baseline(synthetic, 4, 96, units)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
