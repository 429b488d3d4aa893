"""Benchmark of the GPT-2 Pre-LN forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step = one full forward (embedding, every block, final LayerNorm, tied
lm_head writing the logits) of the workload's batch, from token ids already
resident in HBM to logits in HBM.  Prints one JSON line.  The logits are
stored in the model's arithmetic dtype (bf16 for the bf16 workloads, as a
bf16 GPT2LMHeadModel returns them); --logits-dtype f32 stores fp32 logits,
and for a bf16 run the line also carries the fp32-logits throughput.

Default workload: GPT-2 small shape, bf16 matrices / fp32 accumulation,
B=8, T=1024 (synthetic ids and random-init weights of that architecture).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 (MFMA/vector)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

CLASSES = ["embed", "layernorm", "qkv_gemm", "attention", "attn_proj_gemm", "fc_gemm", "mlp_proj_gemm",
           "lm_head_gemm"]


def forward_flops(shape, B, T):
    """Algorithmic FLOPs of one forward: 2*M*N*K per projection and the lm_head
    (N = vocab, unpadded); causal attention counts only keys j <= i:
    2 products (QK^T and PV) x 2 FLOP x hs x T(T+1)/2 per (b, h)."""
    D, F, L, H, V = shape.d_model, shape.d_ff, shape.n_layer, shape.n_head, shape.vocab
    M = B * T
    hs = D // H
    per_layer = 2 * M * (D * 3 * D + D * D + D * F + F * D)
    attn = 2 * 2 * hs * (T * (T + 1) // 2) * B * H
    return L * (per_layer + attn) + 2 * M * D * V


def backward_block_flops(shape, B, T):
    """Algorithmic FLOPs of one block's backward: the input- and weight-gradient
    products of the four projections (twice their forward FLOPs) and the four
    causal attention products dV = P^T dO, dP = dO V^T, dQ = dS K, dK = dS^T Q
    (keys j <= i only)."""
    D, F, H = shape.d_model, shape.d_ff, shape.n_head
    hs = D // H
    M = B * T
    proj = 2 * M * D * (3 * D + D + F + F)
    attn = 4 * 2 * hs * (T * (T + 1) // 2) * B * H
    return 2 * proj + attn


def class_work(shape, B, T, cls):
    """(algorithmic units per launch, unit, bound) for one kernel class."""
    D, F, H, V = shape.d_model, shape.d_ff, shape.n_head, shape.vocab
    M = B * T
    hs = D // H
    if cls == "qkv_gemm":
        return 2.0 * M * D * 3 * D, "flop", "mfma"
    if cls == "attn_proj_gemm":
        return 2.0 * M * D * D, "flop", "mfma"
    if cls == "fc_gemm":
        return 2.0 * M * D * F, "flop", "mfma"
    if cls == "mlp_proj_gemm":
        return 2.0 * M * F * D, "flop", "mfma"
    if cls == "lm_head_gemm":
        return 2.0 * M * D * V, "flop", "mfma"
    if cls == "attention":
        return 2.0 * 2 * hs * (T * (T + 1) // 2) * B * H, "flop", "mfma"
    if cls == "layernorm":   # read fp32 x, write bf16 h (gamma/beta negligible)
        return float(M * D * (4 + 2)), "byte", "hbm"
    if cls == "embed":       # read two bf16 rows, write fp32 x
        return float(M * D * (2 + 2 + 4)), "byte", "hbm"
    raise KeyError(cls)


# kernel class -> kernel name as rocprofv3 reports it (short form)
# kernel of each class in the traffic summary (the tile and schedule-knob
# fields of the GEMM template may vary)
TRAFFIC_KERNELS = {"lm_head_gemm": r"void gemm_kernel<bf16_t, 256, 256, 2, 4, 2, \d+, EpiLogits<bf16_t> >",
                   "fc_gemm": r"void gemm_kernel<bf16_t, \d+, \d+, \d+, \d+, 2, \d+, EpiGelu<bf16_t, false> >",
                   "qkv_gemm": r"void gemm_kernel<bf16_t, \d+, \d+, \d+, \d+, 2, \d+, EpiQKV<bf16_t> >",
                   "attention": r"void attn_prefill_kernel<bf16_t, 64, \d+>",
                   "layernorm": r"void layernorm_kernel<bf16_t, 3>"}


def measured_traffic(workload, cls):
    """HBM bytes per dispatch of the kernel (read + write) from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or None when there is none for
    this workload or the sources that kernel is built from changed since the
    counters were taken (each entry carries the hash of its own sources)."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", f"traffic_{workload.replace('gpt2-', 'gpt2_').replace('-', '_')}.json")
    if not os.path.exists(path) or cls not in TRAFFIC_KERNELS:
        return None
    with open(path) as f:
        rec = json.load(f)
    hits = [v for k, v in rec["per_dispatch"].items() if re.fullmatch(TRAFFIC_KERNELS[cls], k)]
    if len(hits) != 1 or "sources" not in hits[0]:
        return None
    entry = hits[0]
    h = hashlib.sha256(b"".join(open(os.path.join(ROOT, p), "rb").read() for p in entry["sources"])).hexdigest()[:16]
    if h != entry["source_hash"]:
        return None
    return round(entry["read_bytes"] + entry["write_bytes"])


def host_cpu():
    """(logical CPUs this process may run on, CPU model name) of the host."""
    try:
        n = len(os.sched_getaffinity(0))
    except Exception:
        n = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return n, model


def cpu_baseline(w, budget_s=12.0, gpu_argmax=None):
    """The fp64 oracle, as it stands, on the first sequences of the same batch
    until about `budget_s` seconds of host work have been spent.

    gpu_argmax: {label: int array [B, T]} of the GPU's arg-max token per
    position; for the sequences the oracle computed, the exact agreement with
    the oracle's arg-max (first index on ties, both sides) and the admissible
    agreement (the GPU's token has an oracle logit within 2e-2 * max|logit| of
    the oracle's best) are returned beside the timing."""
    import numpy as np
    import oracle
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    nproc, model = host_cpu()
    blob = W.make_params(w)
    ids = W.make_ids(w)
    P = oracle.prepare_params(blob, w.shape, w.dtype)
    del blob
    agree = {k: [0, 0, 0] for k in (gpu_argmax or {})}   # exact, admissible, rows
    elapsed = 0.0
    n = 0
    while n < w.batch:
        t0 = time.perf_counter()
        ref = oracle.forward(P, ids[n:n + 1])[0]
        elapsed += time.perf_counter() - t0
        if gpu_argmax:
            best = ref.argmax(-1)
            tol = 2e-2 * np.abs(ref).max()
            top = ref[np.arange(ref.shape[0]), best]
            for k, g in gpu_argmax.items():
                gi = np.asarray(g[n], dtype=np.int64)
                agree[k][0] += int((gi == best).sum())
                agree[k][1] += int((top - ref[np.arange(ref.shape[0]), gi] <= tol).sum())
                agree[k][2] += ref.shape[0]
        del ref
        n += 1
        if elapsed >= budget_s:
            break
    out = {"value": n * w.seq_len / elapsed, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "sample": f"first {n} of {w.batch} sequences x {w.seq_len} tokens, full logits, fp64 numpy "
                     f"oracle ({elapsed:.1f} s)",
           "threads_note": "cores = BLAS threads the oracle's matrix products used",
           "nproc": nproc, "cpu_model": model}
    argmax = {k: {"exact": round(a[0] / a[2], 5), "admissible": round(a[1] / a[2], 5), "rows": a[2],
                  "sequences": n} for k, a in agree.items() if a[2]}
    return out, argmax


def time_steps(fn, steps, warmup):
    """Seconds per call of fn over `steps` calls after `warmup` untimed ones,
    bracketed by device synchronisations."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def forward_leg(W, w, steps, warmup, logits_dtype="bf16"):
    """One more forward workload (the GPT-2 medium and XL shapes): ms per
    forward with logits in the padded layout, and the fraction of peak."""
    import torch
    from gpt_pre_ln_amd.model import GPT2
    dev = torch.device("cuda:0")
    B, T = w.batch, w.seq_len
    model = GPT2.from_shape(w.shape, w.dtype, max_batch=B, max_seq=T, logits_dtype=logits_dtype)
    model.load_blob(W.make_params(w))
    ids = torch.from_numpy(W.make_ids(w)).to(dev)
    logits = torch.empty((B, T, model.logits_padded_ld), dtype=model.logits_torch_dtype, device=dev)
    el = time_steps(lambda: model.forward(ids, out_logits=logits, padded_logits=True), steps, warmup)
    flops = forward_flops(w.shape, B, T)
    del model, logits
    torch.cuda.empty_cache()
    print(f"[bench] {w.name} forward done", file=sys.stderr, flush=True)
    return {"workload": w.name, "batch": B, "seq_len": T, "logits_dtype": logits_dtype,
            "ms_per_step": round(el * 1e3, 4), "tokens_per_s": round(B * T / el, 1),
            "algorithmic_tflop_per_step": round(flops / 1e12, 4),
            "frac_of_peak": round(flops / el / (PEAK_BF16_TFLOPS * 1e12), 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gpt2-small-b8t1024")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="headline only: skip the loss, variant, backward, fp32-logits, decode, medium and XL legs")
    ap.add_argument("--logits-dtype", choices=["f32", "bf16"], default=None,
                    help="element type of the logits (default: the workload's arithmetic dtype)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one device-to-device copy of 1 GiB (a plain copy kernel of known size, "
                         "used to scale rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the forward shards by "
              "sequence with no exchange, so N GPUs = N independent copies of this run.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import workloads as W
    from gpt_pre_ln_amd import binding
    from gpt_pre_ln_amd.model import GPT2

    binding.load()
    w = W.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if w.decode:
        print(json.dumps(bench_decode(args, w)), flush=True)
        return

    B, T = w.batch, w.seq_len
    logits_dtype = args.logits_dtype or w.dtype
    blob = W.make_params(w)
    model = GPT2.from_shape(w.shape, w.dtype, max_batch=B, max_seq=T, logits_dtype=logits_dtype)
    model.load_blob(blob)
    ids = torch.from_numpy(W.make_ids(w)).to(dev)
    V = w.shape.vocab
    # logits in the padded layout (rows of logits_padded_ld elements; the
    # caller sees the [B, T, vocab] view): the fast layout of gpt2_forward_strided
    ld = model.logits_padded_ld
    logits = torch.empty((B, T, ld), dtype=model.logits_torch_dtype, device=dev)

    def step():
        model.forward(ids, out_logits=logits, padded_logits=True)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # which kernel class dominates: one step per class with HIP events around
    # each launch of that class (outside the timed region)
    per_class = {}
    for cls in CLASSES:
        binding.gpt2_timing_enable(model.handle, cls, True)
        step()
        ms, n = binding.gpt2_timing_read(model.handle)
        binding.gpt2_timing_enable(model.handle, cls, False)
        per_class[cls] = {"ms_per_step": ms, "launches": n}
    dominant = max(per_class, key=lambda c: per_class[c]["ms_per_step"])

    # timed region: K steps; the dominant class is bracketed by HIP events on its stream
    binding.gpt2_timing_enable(model.handle, dominant, True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    dom_ms, dom_n = binding.gpt2_timing_read(model.handle)
    binding.gpt2_timing_enable(model.handle, dominant, False)

    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = B * T / (elapsed / args.steps)
    flops = forward_flops(w.shape, B, T)
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    units, unit_kind, bound = class_work(w.shape, B, T, dominant)
    avg_s = dom_ms / 1e3 / max(dom_n, 1)
    if unit_kind == "flop":
        achieved = units / avg_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": None}
    else:
        achieved = units / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None}
    roof["kernel"] = dominant
    roof["traffic"] = measured_traffic(w.name, dominant)
    roof["avg_launch_ms"] = round(dom_ms / max(dom_n, 1), 5)
    roof["launches_timed"] = dom_n

    # the GPU's arg-max token per position (outside the timed region), for the
    # agreement with the oracle computed in the CPU-baseline leg
    gpu_argmax = {logits_dtype: logits[..., :V].argmax(-1).cpu().numpy()}

    out = {
        "metric": "forward tokens/s and % bf16 MFMA peak, GPT-2 small B=8 T=1024, 1 GPU",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "seq_len": T, "d_model": w.shape.d_model,
                   "n_layer": w.shape.n_layer, "n_head": w.shape.n_head, "vocab": V,
                   "logits_dtype": logits_dtype, "logits_row_stride": ld},
        "frac_of_peak": round(flops / (elapsed / args.steps) / (peak * 1e12), 4),
        "algorithmic_tflop_per_step": round(flops / 1e12, 4),
        "roofline": roof,
        "per_class_ms": {c: round(v["ms_per_step"], 4) for c, v in per_class.items()},
        "per_class_note": (f"each class timed in a step of its own, with HIP events around each of its launches: "
                           f"the events keep the launches apart, so the classes sum to "
                           f"{sum(v['ms_per_step'] for v in per_class.values()):.3f} ms against "
                           f"{ms_per_step:.3f} ms per step (not additive)"),
    }

    if not args.no_extra:
        # forward + shifted next-token cross-entropy, logits never stored (gpt2_forward_loss)
        loss_mean = torch.empty(1, dtype=torch.float32, device=dev)
        el_loss = time_steps(lambda: model.loss(ids, out_mean=loss_mean), args.steps, args.warmup)
        out["loss_step"] = {"value": round(B * T / el_loss, 1), "unit": "tokens/s",
                            "ms_per_step": round(el_loss * 1e3, 4), "mean_loss": round(float(loss_mean.item()), 5)}

        # the same workload with every variant switch on (Post-LN wiring, per-layer
        # score scaling, erf GELU, separate head): its own weights, same ids
        import dataclasses
        vshape = dataclasses.replace(w.shape, post_ln=True, scale_attn_by_inverse_layer_idx=True, activation="gelu",
                                     tie_word_embeddings=False)
        vmodel = GPT2.from_shape(vshape, w.dtype, max_batch=B, max_seq=T, logits_dtype=logits_dtype)
        vmodel.load_blob(W.make_params(vshape, w.init, w.param_seed))
        el_v = time_steps(lambda: vmodel.forward(ids, out_logits=logits, padded_logits=True), args.steps,
                          args.warmup)
        out["variant_step"] = {"switches": ["post_ln", "scale_attn_by_inverse_layer_idx", "gelu_erf",
                                            "separate_head"],
                               "value": round(B * T / el_v, 1), "unit": "tokens/s", "ms_per_step": round(el_v * 1e3, 4)}
        del vmodel

        # backward of one block (gpt2_block_backward, layer 0) on the same batch:
        # seeded fp32 block input and output gradient
        gen = torch.Generator(device=dev)
        gen.manual_seed(7)
        xb = torch.randn((B, T, w.shape.d_model), generator=gen, device=dev, dtype=torch.float32)
        dyb = torch.randn((B, T, w.shape.d_model), generator=gen, device=dev, dtype=torch.float32)
        dxb, gb = model.block_backward(0, xb, dyb)
        el_b = time_steps(lambda: model.block_backward(0, xb, dyb, out_dx=dxb, out_grads=gb),
                          max(2, args.steps // 4), max(1, args.warmup // 2))
        bflop = backward_block_flops(w.shape, B, T)
        out["block_backward"] = {"layer": 0, "ms_per_call": round(el_b * 1e3, 4),
                                 "algorithmic_tflop": round(bflop / 1e12, 4),
                                 "achieved_tflops": round(bflop / el_b / 1e12, 2),
                                 "note": "includes the recomputed forward of the block"}
        del xb, dyb, dxb, gb
        model._bwd_ws = None

        # the same forward storing fp32 logits: t_fwd of the measurement
        # definition (device ids -> device fp32 logits), beside the headline value
        if logits_dtype != "f32":
            del logits
            model32 = GPT2.from_shape(w.shape, w.dtype, max_batch=B, max_seq=T, logits_dtype="f32")
            model32.load_blob(blob)
            logits32 = torch.empty((B, T, ld), dtype=torch.float32, device=dev)
            el32 = time_steps(lambda: model32.forward(ids, out_logits=logits32, padded_logits=True), args.steps,
                              args.warmup)
            gpu_argmax["f32"] = logits32[..., :V].argmax(-1).cpu().numpy()
            out["fp32_logits"] = {"value": round(B * T / el32, 1), "unit": "tokens/s",
                                  "ms_per_step": round(el32 * 1e3, 4),
                                  "frac_of_peak": round(flops / el32 / (peak * 1e12), 4),
                                  "note": "t_fwd from device token ids to device fp32 logits"}
            del model32, logits32
        del model
        torch.cuda.empty_cache()
        print("[bench] GPT-2 small legs done", file=sys.stderr, flush=True)

        # the other workloads: the decode step, GPT-2 medium and XL forwards
        dw = W.WORKLOADS["gpt2-small-decode-b32p1023"]
        d = bench_decode(args, dw, generation=False)
        out["decode_step"] = {"workload": dw.name, "batch": d["config"]["batch"], "prefix": d["config"]["prefix"],
                              "ms_per_step": d["ms_per_step"], "tokens_per_s": d["value"],
                              "achieved_gbs": d["roofline"]["achieved"], "frac_of_hbm": d["roofline"]["frac"],
                              "algorithmic_bytes": d["roofline"]["algorithmic_bytes"]}
        fsteps, fwarm = max(3, args.steps // 2), max(1, args.warmup // 2)
        out["medium"] = forward_leg(W, W.WORKLOADS["gpt2-medium-b8t1024"], fsteps, fwarm)
        out["xl"] = forward_leg(W, W.WORKLOADS["gpt2-xl-b4t1024"], fsteps, fwarm)

    if not args.no_cpu_baseline:
        cb, agree = cpu_baseline(w, gpu_argmax=gpu_argmax)
        out["cpu_baseline"] = cb
        out["argmax_agreement"] = agree
    print(json.dumps(out), flush=True)


def bench_decode(args, w, generation=True):
    import torch
    import workloads as W
    from gpt_pre_ln_amd.model import GPT2

    dev = torch.device("cuda:0")
    B, P = w.batch, w.seq_len
    logits_dtype = args.logits_dtype or w.dtype
    model = GPT2.from_shape(w.shape, w.dtype, max_batch=B, max_seq=P + 1, logits_dtype=logits_dtype)
    model.load_blob(W.make_params(w))
    prefix, new = W.make_decode_ids(w)
    kv = model.new_kv_cache(B, P + 1)
    model.forward(torch.from_numpy(prefix).to(dev), logits=False, kv=kv)
    torch.cuda.synchronize()
    print(f"[bench] prefill of {P} tokens done", file=sys.stderr, flush=True)
    new_d = torch.from_numpy(new).to(dev)
    logits = torch.empty((B, w.shape.vocab), dtype=model.logits_torch_dtype, device=dev)

    def step():
        kv.view.past_len = P          # re-run the same step: position P, cache slot P
        model.decode_step(kv, new_d, out_logits=logits)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    print(f"[bench] {args.steps} decode steps done", file=sys.stderr, flush=True)
    generate = None
    if generation:
        generate = bench_generation(args, model, kv, prefix, B, P)

    s = w.shape
    D, F, L, V = s.d_model, s.d_ff, s.n_layer, s.vocab
    weights = 2 * (L * (3 * D * D + D * D + 2 * D * F) + V * D)
    kv_bytes = 2 * L * 2 * B * (P + 1) * D
    logit_bytes = (2 if logits_dtype == "bf16" else 4) * B * V
    total = weights + kv_bytes + logit_bytes
    gbs = total / dt / 1e9
    out = {"metric": "decode tokens/s (GPT-2 small, B=32, cached prefix 1023)", "value": round(B / dt, 1),
           "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(dt * 1e3, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": w.dtype, "data": "synthetic",
           "config": {"workload": w.name, "batch": B, "prefix": P, "logits_dtype": logits_dtype},
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                        "kernel": "whole decode step", "algorithmic_bytes": total}}
    if generate is not None:
        out["generate"] = generate
    del model, kv, logits
    torch.cuda.empty_cache()
    return out


def bench_generation(args, model, kv, prefix, B, P):
    """Greedy generation (gpt2_generate): the first 960 tokens as the prompt,
    64 steps chained on the device (positions 959 .. 1022), no logits stored."""
    import torch
    dev = torch.device("cuda:0")
    gen_prompt, gen_steps = min(960, P), min(64, P + 1 - min(960, P))
    gen_first = torch.from_numpy(np.ascontiguousarray(prefix[:, gen_prompt - 1])).to(dev)
    gen_out = torch.empty((B, gen_steps), dtype=torch.int32, device=dev)

    def gen():
        kv.view.past_len = gen_prompt - 1
        model.generate(kv, gen_first, gen_steps, out=gen_out)
        torch.cuda.synchronize()
        print(f"[bench] generation of {gen_steps} steps done", file=sys.stderr, flush=True)

    gen()
    torch.cuda.synchronize()
    reps = max(1, args.steps // 10)
    t1 = time.perf_counter()
    for _ in range(reps):
        gen()
    torch.cuda.synchronize()
    gdt = (time.perf_counter() - t1) / reps
    return {"value": round(B * gen_steps / gdt, 1), "unit": "tokens/s", "batch": B, "prompt": gen_prompt,
            "steps": gen_steps, "ms_per_step": round(gdt * 1e3 / gen_steps, 4)}


if __name__ == "__main__":
    main()
