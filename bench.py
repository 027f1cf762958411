#!/usr/bin/env python3
"""Throughput of the little-lm training-step hot path on one MI355X.

A step is one pass of the whole hot path over one micro-batch of 40 x 1024 synthetic tokens:
forward of one 3.8B decoder layer (FP8 e4m3 MLP GEMMs, bf16 elsewhere), the fused linear
cross-entropy (softcap 15, 50304-padded vocab) on its output with loss and both gradients, and the
layer backward from that gradient. Every kernel is libll's (HIP, gfx950); inputs are resident in
HBM before the timed region. Prints one JSON line on stdout; progress goes to stderr.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload layer_lce|layer|layer_swiglu|layer_ve_2k|lce|model|train|muon] [--no-cpu-baseline]
                    [--lce-chunk TOKENS] [--lce-vocab-tile 128|256] [--sweep-lce]

FLOP accounting (algorithmic, not executed work): per token of one layer, fwd + bwd,
6 * P_mm + 6 * Hq * Dh * (T + 1) with P_mm = 100,663,296 matrix weights (causal attention counted
at half of full); the loss adds 6 * N * V * D. 60,000 tokens/s/GPU x 28 layers x that layer count
gives the ~1,047 TFLOP/s per B200 printed on the hn.213312.xyz translation ("结果 / Results"), so
the same formula prices this step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "train tokens/sec per MI355X (3.8B layer fwd+bwd + fused LCE); % dense MFMA peak"
PEAK_BF16 = 2.5e15          # MI355X dense bf16 MFMA, FLOP/s
PEAK_FP8 = 5.0e15           # dense e4m3
PEAK_HBM = 8.0e12           # bytes/s

D, HQ, HKV, DH, F, V, V_REAL = 3072, 24, 8, 128, 12288, 50304, 50257
P_MM = D * (HQ + 2 * HKV) * DH + D * HQ * DH + 2 * D * F          # 100,663,296


# HBM bytes per launch of a kernel from two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) scaled by
# the same counters on a 1 GiB device copy; valid only for the kernel sources they were taken on
# (sha256 of the listed files, first 16 hex digits), else the roofline reports traffic null.
SOURCES = ("transformer_train_step_amd/csrc/gemm.h", "transformer_train_step_amd/csrc/lce.h",
           "transformer_train_step_amd/csrc/common.h", "transformer_train_step_amd/csrc/lce.hip")
# HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE, copy-calibrated (valid while the sources
# hash to sha256_16; otherwise the roofline reports traffic null)
TRAFFIC = {
    "gemm_bf16_lce_grads_kk": {"sources": SOURCES, "sha256_16": "832ac60ae8291f72", "read_bytes": 1.4504e+10,
                               "write_bytes": 6.256e+08,
                               "profile": "profiles/gemm_bf16_lce_grads_kk_hbm_bytes_layer_lce_40x1024.md"},
    "gemm_bf16_lce_logits_kk": {"sources": SOURCES, "sha256_16": "832ac60ae8291f72", "read_bytes": 5.897e+09,
                                "write_bytes": 1.054e+09,
                                "profile": "profiles/gemm_bf16_lce_logits_kk_hbm_bytes_layer_lce_40x1024.md"},
}


def measured_traffic(tag: str):
    import hashlib
    t = TRAFFIC.get(tag)
    if t is None:
        return None
    here = os.path.dirname(os.path.abspath(__file__))
    try:
        src = b"".join(open(os.path.join(here, f), "rb").read() for f in t["sources"])
    except OSError:
        return None
    if hashlib.sha256(src).hexdigest()[:16] != t["sha256_16"]:
        return None
    return {"read_bytes": t["read_bytes"], "write_bytes": t["write_bytes"],
            "bytes": t["read_bytes"] + t["write_bytes"], "profile": t["profile"]}


def layer_flops_per_token(seq: int, hq: int = HQ, dh: int = DH, p_mm: int = P_MM) -> int:
    return 6 * p_mm + 6 * hq * dh * (seq + 1)


def lce_flops(n: int, v: int = V, d: int = D) -> int:
    return 6 * n * v * d


def log(*a):
    print(*a, file=sys.stderr, flush=True)


WORKLOADS = {
    "layer_lce": dict(batch=40, seq=1024, ve=False, layer=True, lce=True,
                      desc="3.8B decoder layer fwd+bwd (40x1024 tokens, FP8 e4m3 MLP, no value embedding) "
                           "+ fused linear cross-entropy fwd+bwd on its output (40960x3072 @ 50304x3072, softcap 15)"),
    "layer": dict(batch=40, seq=1024, ve=False, layer=True, lce=False,
                  desc="3.8B decoder layer fwd+bwd (40x1024 tokens, FP8 e4m3 MLP)"),
    "layer_swiglu": dict(batch=40, seq=1024, ve=False, layer=True, lce=False, mlp="swiglu", d_ff=8448, fp8=False,
                         desc="3.8B-width decoder layer fwd+bwd with the gated variant: bf16 SwiGLU MLP at 2.75x "
                              "(d_ff 8448, W_fc 16896x3072 gate+up, W_proj 3072x8448), 40x1024 tokens"),
    "layer_ve_2k": dict(batch=20, seq=2048, ve=True, layer=True, lce=False,
                        desc="3.8B value-embedding decoder layer fwd+bwd (20x2048 tokens, FP8 e4m3 MLP)"),
    "lce": dict(batch=40, seq=1024, ve=False, layer=False, lce=True,
                desc="fused linear cross-entropy fwd+bwd (hidden 40960x3072 bf16 N(0,1), head 50304x3072 "
                     "N(0,0.02), softcap 15)"),
    "model": dict(batch=40, seq=1024, ve=True, layer=True, lce=True, layers=28,
                  desc="full 3.848B model fwd+bwd (token embedding 50304x3072, 28 decoder layers with value "
                       "embeddings on the 14 even layers, FP8 e4m3 MLPs, final RMSNorm, untied head + fused "
                       "linear cross-entropy softcap 15; 40x1024 tokens)"),
    "train": dict(batch=40, seq=1024, ve=True, layer=True, lce=True, layers=28, accum=7,
                  desc="one optimizer step of the full 3.848B model on one GPU: 7 accumulated micro-batches of "
                       "40x1024 tokens through the whole model (as 'model'), then Muon (5 Newton-Schulz steps) on "
                       "the 112 layer matrices and AdamW on the embedding, head, 14 value-embedding tables, gains "
                       "and residual scalars; bf16 master weights and optimizer state"),
    "muon": dict(batch=0, seq=0, ve=False, layer=False, lce=False, muon=True,
                 desc="Muon step (momentum, 5 Newton-Schulz steps on bf16 MFMA, update) of one decoder layer's "
                      "four matrices: W_qkv 5120x3072, W_o 3072x3072, W_fc 12288x3072, W_proj 3072x12288"),
}
MUON_SHAPES = ((HQ + 2 * HKV) * DH, D), (D, HQ * DH), (F, D), (D, F)


def muon_flops(rows: int, cols: int, steps: int = 5) -> int:
    """Newton-Schulz GEMM work on the wide orientation [m, n]: X X^T, A A, B X per step."""
    m, n = min(rows, cols), max(rows, cols)
    return steps * (2 * m * m * n + 2 * m * m * m + 2 * m * m * n)


def step_flops(w: dict) -> int:
    """Algorithmic FLOPs of one step: layers and loss (the optimizer is not counted, as on the pages;
    the Muon workload counts its Newton-Schulz GEMMs)."""
    if w.get("muon"):
        return sum(muon_flops(r, c) for r, c in MUON_SHAPES)
    n = w["batch"] * w["seq"]
    f = 0
    if w["layer"]:
        ff = w.get("d_ff", F)
        p_mm = P_MM - 2 * D * F + (3 if w.get("mlp") == "swiglu" else 2) * D * ff
        f += w.get("layers", 1) * layer_flops_per_token(w["seq"], p_mm=p_mm) * n
    if w["lce"]:
        f += lce_flops(n)
    return f * w.get("accum", 1)


def cpu_baseline(seq: int, ve: bool, with_layer: bool, with_lce: bool, layers: int = 1, mlp: str = "relu2",
                 d_ff: int = F, fp8: bool = True) -> dict:
    """The oracle, as it stands, on a bounded sample: one sequence of `seq` tokens through the same
    step (layer fwd -> loss -> layer bwd) at full model width, float64 numpy on the host. With
    layers > 1 the layer part is timed once and counted `layers` times (the whole model would not
    finish in minutes on the host)."""
    import synth
    from oracle import lce as olce
    from oracle import model as om
    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or os.cpu_count()
    except Exception:
        threads = os.cpu_count()
    s = synth.LayerShape(batch=1, seq=seq, value_embed=ve, mlp=mlp, d_ff=d_ff, fp8_mlp=fp8)
    inp = synth.layer_inputs(s, seed=0)
    if with_lce:
        w_head = synth.normal((V, D), 0.02, 0, synth.K_WHEAD, "bf16")
        tg = synth.uniform_ints((seq,), V_REAL, 0, synth.K_TARGETS)
    y, dy = inp.x, inp.dy
    t_layer = t_lce = 0.0
    if with_layer:
        t0 = time.perf_counter()                  # inputs drawn; time the oracle only
        p, d = om.params_from_inputs(inp), om.dims_from_shape(s)
        y, cache = om.layer_fwd(p, inp.x, inp.ids, d)
        t_layer += time.perf_counter() - t0
    if with_lce:
        t0 = time.perf_counter()
        dy = olce.lce_fwd_bwd(y, w_head, tg, softcap=15.0, mode="bf16")["dh"]
        t_lce = time.perf_counter() - t0
    if with_layer:
        t0 = time.perf_counter()
        om.layer_bwd(p, cache, dy, d)
        t_layer += time.perf_counter() - t0
    sec = layers * t_layer + t_lce
    what = f"1 sequence x {seq} tokens of the same step at full width (float64 numpy)"
    if layers > 1:
        what += f"; one layer timed ({t_layer:.1f} s) and counted {layers} times, plus the loss ({t_lce:.1f} s)"
    return {"value": round(seq / sec, 3), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{what}, {sec:.1f} s", "seconds": round(sec, 2)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="layer_lce", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-trace", action="store_true", help="skip the traced pass (roofline)")
    ap.add_argument("--kernels", action="store_true",
                    help="print every traced kernel (ms per step, launches, TFLOP/s of its algorithmic work)")
    ap.add_argument("--lce-chunk", type=int, default=10240, metavar="TOKENS",
                    help="tokens per chunk of the fused linear cross-entropy (logits of one chunk are stored)")
    ap.add_argument("--lce-vocab-tile", type=int, default=256, choices=(128, 256),
                    help="vocabulary columns per partial row sum (the logits GEMM's N tile)")
    ap.add_argument("--gemm-config", type=int, default=0, metavar="CFG",
                    help="GEMM block configuration override for every GEMM (llt_set_gemm_config; 0 = automatic)")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph after the warmup and time its replays (the same "
                         "launches without the host's per-launch gaps)")
    ap.add_argument("--sweep-lce", action="store_true",
                    help="also time the loss alone over token_chunk x vocab_tile (reported as lce_sweep)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before the steps, copy a MIB-MiB device buffer once (a plain copy of known size, "
                         "the reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import transformer_train_step_amd as ll
    from transformer_train_step_amd import _lib as L
    from transformer_train_step_amd.ops import FusedLCE, Layer, LayerConfig, Model

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    L.lib()
    if args.gemm_config:
        L.llt_set_gemm_config(args.gemm_config)
    w = WORKLOADS[args.workload]
    B, T = w["batch"], w["seq"]
    N = B * T
    dev = "cuda"
    log(f"[bench] workload {args.workload}: {w['desc']}")

    def to_dev(a, dt=torch.bfloat16):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dt).to(dev)

    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {n} bytes done")
        del src, dst
    t_in = time.perf_counter()
    if args.workload in ("model", "train"):
        step, n_launch_trace = model_step(w, dev, torch, synth, LayerConfig, Model, args.lce_chunk)
    elif args.workload == "muon":
        step, n_launch_trace = muon_step(dev, torch, L)
    else:
        step, n_launch_trace = layer_lce_step(w, dev, torch, synth, LayerConfig, Layer, FusedLCE, to_dev,
                                              args.lce_chunk, args.lce_vocab_tile)
    torch.cuda.synchronize()
    log(f"[bench] inputs resident in HBM ({time.perf_counter() - t_in:.1f} s to generate)")

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"[bench] warmup step {i + 1}/{args.warmup} done")

    run = step
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        run = graph.replay
        log("[bench] step captured in a HIP graph")

    # timed region: K steps, synchronised on both sides
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        run()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    log(f"[bench] timed {args.steps} steps: {ms:.3f} ms/step (wall {wall * 1e3 / args.steps:.3f} ms/step)")
    report(args, w, ms, step, stream, ev0, ev1, L, n_launch_trace)


def layer_lce_step(w, dev, torch, synth, LayerConfig, Layer, FusedLCE, to_dev, lce_chunk, vocab_tile=256):
    """Inputs and the step closure of the layer / loss workloads (inputs drawn by synth)."""
    B, T = w["batch"], w["seq"]
    N = B * T
    mlp, ff, fp8 = w.get("mlp", "relu2"), w.get("d_ff", F), w.get("fp8", True)
    s = synth.LayerShape(batch=B, seq=T, value_embed=w["ve"], mlp=mlp, d_ff=ff, fp8_mlp=fp8)
    inp = synth.layer_inputs(s, seed=0)
    x = to_dev(inp.x)
    ids = torch.from_numpy(inp.ids).to(dev)
    p = None
    layer = None
    if w["layer"]:
        cfg = LayerConfig(batch=B, seq=T, value_embed=w["ve"], mlp=mlp, d_ff=ff, fp8_mlp=fp8)
        layer = Layer(cfg, dev)
        p = {"attn_norm_w": torch.from_numpy(inp.g_attn).to(dev), "mlp_norm_w": torch.from_numpy(inp.g_mlp).to(dev),
             "w_qkv": to_dev(inp.w_qkv), "w_o": to_dev(inp.w_o), "w_fc": to_dev(inp.w_fc), "w_proj": to_dev(inp.w_proj),
             "resid_attn": torch.ones(1, dtype=torch.float32, device=dev),
             "resid_mlp": torch.ones(1, dtype=torch.float32, device=dev)}
        if w["ve"]:
            p["ve_table"] = to_dev(inp.ve_table)
        grads = layer.new_grads()
        y = torch.empty_like(x)
        dx = torch.empty_like(x)
    dy = to_dev(inp.dy)
    lce = None
    if w["lce"]:
        w_head = to_dev(synth.normal((V, D), 0.02, 0, synth.K_WHEAD, "bf16"))
        targets = torch.from_numpy(synth.uniform_ints((N,), V_REAL, 0, synth.K_TARGETS)).to(dev)
        lce = FusedLCE("bf16", N, D, V, token_chunk=lce_chunk, vocab_tile=vocab_tile, device=dev)
        dh_buf = torch.empty_like(x)
        dw_head = torch.empty_like(w_head)
    del inp

    def step():
        h = x
        if layer is not None:
            layer.forward(p, x, ids, y)
            h = y
        g = dy
        if lce is not None:
            lce(h, w_head, targets, d_hidden=dh_buf, d_weight=dw_head)
            g = dh_buf
        if layer is not None:
            layer.backward(p, x, ids, g, dx=dx, grads=grads)

    return step, 4096


def model_step(w, dev, torch, synth, LayerConfig, Model, lce_chunk):
    """Inputs and the step closure of the whole model. Its ~3.9B weights are drawn on the GPU with
    torch's seeded generator (N(0, 0.02), bf16; gains and residual scalars 1); token ids and
    targets come from synth."""
    B, T, n_layers = w["batch"], w["seq"], w["layers"]
    N = B * T
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)

    def rn(*shape):
        t = torch.empty(shape, dtype=torch.float32, device=dev)
        t.normal_(0.0, 0.02, generator=gen)
        return t.to(torch.bfloat16)

    qkv = (HQ + 2 * HKV) * DH
    layers = []
    for i in range(n_layers):
        lp = {"attn_norm_w": torch.ones(D, device=dev), "mlp_norm_w": torch.ones(D, device=dev),
              "w_qkv": rn(qkv, D), "w_o": rn(D, HQ * DH), "w_fc": rn(F, D), "w_proj": rn(D, F),
              "resid_attn": torch.ones(1, device=dev), "resid_mlp": torch.ones(1, device=dev)}
        if i % 2 == 0:
            lp["ve_table"] = rn(V, HKV * DH)
        layers.append(lp)
    params = {"embed": rn(V, D), "layers": layers, "final_norm_w": torch.ones(D, device=dev), "head": rn(V, D)}
    model = Model(LayerConfig(batch=B, seq=T), n_layers, V, token_chunk=lce_chunk, device=dev)
    accum = w.get("accum", 0)
    if accum:
        from transformer_train_step_amd.ops import TrainStep
        ts = TrainStep(model, params, accum=accum)
        batches = [(torch.from_numpy(synth.uniform_ints((N,), V_REAL, k, synth.K_IDS)).to(dev),
                    torch.from_numpy(synth.uniform_ints((N,), V_REAL, k, synth.K_TARGETS)).to(dev))
                   for k in range(accum)]
    else:
        grads = model.new_grads(params)
        ids = torch.from_numpy(synth.uniform_ints((N,), V_REAL, 0, synth.K_IDS)).to(dev)
        targets = torch.from_numpy(synth.uniform_ints((N,), V_REAL, 0, synth.K_TARGETS)).to(dev)
    log(f"[bench] model buffers: saved {model.saved_bytes / 2**30:.1f} GiB, workspace "
        f"{model.ws_bytes / 2**30:.1f} GiB, device memory in use {torch.cuda.memory_allocated() / 2**30:.1f} GiB")

    if accum:
        def step():
            ts(batches)
        return step, 32768

    def step():
        model(params, ids, targets, grads)

    return step, 16384


def muon_step(dev, torch, L):
    """Muon on one layer's four matrices (weights N(0, 0.02), gradients N(0, 1e-3), bf16)."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    mats = []
    for r, c in MUON_SHAPES:
        w = torch.empty((r, c), device=dev).normal_(0, 0.02, generator=gen).to(torch.bfloat16)
        g = torch.empty((r, c), device=dev).normal_(0, 1e-3, generator=gen).to(torch.bfloat16)
        mats.append((w, g, torch.zeros_like(w)))
    wsb = max(L.ll_muon_workspace_bytes(r, c) for r, c in MUON_SHAPES)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)

    def step():
        for w, g, b in mats:
            L.ll_muon_step(L.LL_BF16, w, g, b, w.shape[0], w.shape[1], 0.02, 0.95, 1, 0.0, 5, ws, wsb)

    return step, 4096


def report(args, w, ms, step, stream, ev0, ev1, L, n_launch_trace):
    import torch
    B, T = w["batch"], w["seq"]
    N = B * T * w.get("accum", 1)
    flops = step_flops(w)
    tok_s = N / (ms * 1e-3)
    value, unit = round(tok_s, 1), "tokens/s"
    if w.get("muon"):
        value, unit = round(1e3 / ms, 3), "Muon steps/s (one layer's four matrices)"
    out = {
        "metric": METRIC, "value": value, "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16+e4m3" if w.get("fp8", True) and (w["layer"] or w.get("layers")) else "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights, uniform token ids)",
        "config": {"workload": w["desc"], "tokens_per_step": N, "batch": B, "seq_len": T,
                   "lce_token_chunk": args.lce_chunk, "lce_vocab_tile": args.lce_vocab_tile,
                   "hip_graph": bool(args.graph), "gemm_config_override": args.gemm_config},
        "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
        "pct_bf16_peak": round(100 * flops / (ms * 1e-3) / PEAK_BF16, 2),
        "algorithmic_flops_per_step": flops,
    }

    # traced pass: the same K steps with every launch bracketed by HIP events on its stream
    if not args.no_trace:
        # as many steps as the launch trace holds (the whole model issues ~2,000 launches a step)
        tsteps = args.steps if n_launch_trace == 4096 else 1
        L.llt_trace_begin(n_launch_trace)
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(tsteps):
            step()
        ev1.record(stream)
        torch.cuda.synchronize()
        L.llt_trace_end()
        traced_ms = ev0.elapsed_time(ev1) / tsteps
        recs = L.llt_trace_read()
        per = {}
        for tag, t, mnk in recs:
            e = per.setdefault(tag, {"launches": 0, "ms": 0.0, "flops": 0})
            e["launches"] += 1
            e["ms"] += t
            e["flops"] += 2 * mnk[0] * mnk[1] * mnk[2]
        top = sorted(per.items(), key=lambda kv: -kv[1]["ms"])
        dom_tag, dom = top[0]
        avg_ms = dom["ms"] / dom["launches"]
        flops_launch = dom["flops"] / dom["launches"]
        peak = PEAK_FP8 if "_e4m3_" in dom_tag else PEAK_BF16
        achieved = flops_launch / (avg_ms * 1e-3) / 1e12 if flops_launch else 0.0
        out["roofline"] = {"kernel": dom_tag, "bound": "mfma", "achieved": round(achieved, 1),
                           "peak": peak / 1e12, "unit": "TFLOP/s", "frac": round(achieved * 1e12 / peak, 4),
                           "traffic": None, "avg_launch_ms": round(avg_ms, 4),
                           "flops_per_launch": int(flops_launch), "launches_per_step": dom["launches"] / tsteps}
        tr = measured_traffic(dom_tag)
        if tr is not None:   # HBM bytes per launch (rocprofv3 counters, copy-calibrated)
            out["roofline"].update(traffic=tr["bytes"], traffic_read_bytes=tr["read_bytes"],
                                   traffic_write_bytes=tr["write_bytes"], traffic_profile=tr["profile"])
        out["kernel_breakdown_ms_per_step"] = {k: round(v["ms"] / tsteps, 3) for k, v in top[:12]}
        out["traced_ms_per_step"] = round(traced_ms, 4)
        log("[bench] per-kernel time per step (ms): " +
            ", ".join(f"{k} {v['ms'] / tsteps:.2f}" for k, v in top[:12]))
        if args.kernels:
            for k, v in top:
                tf = f"{v['flops'] / (v['ms'] * 1e-3) / 1e12:8.1f} TFLOP/s" if v["flops"] and v["ms"] > 0 else ""
                log(f"[bench]   {k:40s} {v['ms'] / tsteps:8.3f} ms/step {v['launches'] / tsteps:6.1f} launches {tf}")

    if args.sweep_lce:
        out["lce_sweep"] = lce_sweep(args, torch)
    if not args.no_cpu_baseline and not w.get("muon") and not w.get("accum"):
        log("[bench] timing the oracle on the host (bounded sample)...")
        seq = T if w["layer"] else 1024
        out["cpu_baseline"] = cpu_baseline(seq, w["ve"], w["layer"], w["lce"], w.get("layers", 1),
                                           w.get("mlp", "relu2"), w.get("d_ff", F), w.get("fp8", True))
        log(f"[bench] oracle: {out['cpu_baseline']['value']} tokens/s on {out['cpu_baseline']['cores']} threads")
    print(json.dumps(out), flush=True)


def lce_sweep(args, torch):
    """The loss alone (40960 x 3072 @ 50304 x 3072, bf16) timed per token_chunk x vocab_tile."""
    import synth
    from transformer_train_step_amd.ops import FusedLCE
    n = 40960
    h = torch.empty((n, D), device="cuda").normal_(0, 1, generator=torch.Generator(device="cuda").manual_seed(1))
    h = h.to(torch.bfloat16)
    wt = torch.empty((V, D), device="cuda").normal_(0, 0.02, generator=torch.Generator(device="cuda").manual_seed(2))
    wt = wt.to(torch.bfloat16)
    y = torch.from_numpy(synth.uniform_ints((n,), V_REAL, 0, synth.K_TARGETS)).cuda()
    dh, dw = torch.empty_like(h), torch.empty_like(wt)
    res = []
    for chunk in (8192, 10240, 20480, 40960):
        for tile in (128, 256):
            lce = FusedLCE("bf16", n, D, V, token_chunk=chunk, vocab_tile=tile)
            lce(h, wt, y, d_hidden=dh, d_weight=dw)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(3):
                lce(h, wt, y, d_hidden=dh, d_weight=dw)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 3
            res.append({"token_chunk": chunk, "vocab_tile": tile, "ms": round(ms, 3),
                        "pct_bf16_peak": round(100 * lce_flops(n) / (ms * 1e-3) / PEAK_BF16, 2)})
            log(f"[bench] lce sweep chunk {chunk} tile {tile}: {ms:.3f} ms")
            del lce
    return res


if __name__ == "__main__":
    main()
