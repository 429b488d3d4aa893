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
                   "fc_gemm": r"void gemm_kernel<bf16_t, \d+, \d+, 2, 2, 2, \d+, EpiGelu<bf16_t> >",
                   "qkv_gemm": r"void gemm_kernel<bf16_t, \d+, \d+, 2, 2, 2, \d+, EpiQKV<bf16_t> >",
                   "attention": r"void attn_prefill_kernel<bf16_t, 64>",
                   "layernorm": r"void layernorm_kernel<bf16_t, 3>"}


def measured_traffic(workload, cls):
    """HBM bytes per dispatch of the kernel (read + write) from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or None when there is none for
    this workload or the kernel sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{workload.replace('gpt2-', 'gpt2_').replace('-', '_')}.json")
    if not os.path.exists(path) or cls not in TRAFFIC_KERNELS:
        return None
    with open(path) as f:
        rec = json.load(f)
    h = hashlib.sha256(b"".join(open(os.path.join(ROOT, p), "rb").read() for p in rec["sources"])).hexdigest()[:16]
    if h != rec["source_hash"]:
        return None
    import re
    hits = [v for k, v in rec["per_dispatch"].items() if re.fullmatch(TRAFFIC_KERNELS[cls], k)]
    if len(hits) != 1:
        return None
    entry = hits[0]
    return round(entry["read_bytes"] + entry["write_bytes"])


def cpu_baseline(w, budget_s=12.0):
    """The fp64 oracle, as it stands, on the first sequences of the same batch
    until about `budget_s` seconds of host work have been spent."""
    import numpy as np
    import oracle
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    blob = W.make_params(w)
    ids = W.make_ids(w)
    P = oracle.prepare_params(blob, w.shape, w.dtype)
    del blob
    t0 = time.perf_counter()
    n = 0
    while n < w.batch:
        oracle.forward(P, ids[n:n + 1])
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": n * w.seq_len / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n} of {w.batch} sequences x {w.seq_len} tokens, full logits, fp64 numpy "
                      f"oracle ({dt:.1f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gpt2-small-b8t1024")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
        return bench_decode(args, w)

    B, T = w.batch, w.seq_len
    logits_dtype = args.logits_dtype or w.dtype
    blob = W.make_params(w)
    model = GPT2.from_shape(w.shape, w.dtype, max_batch=B, max_seq=T, logits_dtype=logits_dtype)
    model.load_blob(blob)
    ids = torch.from_numpy(W.make_ids(w)).to(dev)
    # logits in the padded layout (rows of logits_padded_ld elements; the
    # caller sees the [B, T, vocab] view): the fast layout of gpt2_forward_strided
    ld = model.logits_padded_ld
    logits = torch.empty((B, T, ld), dtype=model.logits_torch_dtype, device=dev)

    def step():
        model.forward(ids, out_logits=logits, padded_logits=True)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # which kernel class dominates: one timed step per class (outside the timed region)
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

    # forward + shifted next-token cross-entropy, logits never stored
    # (gpt2_forward_loss; reported beside the headline value)
    loss_mean = torch.empty(1, dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        model.loss(ids, out_mean=loss_mean)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(args.steps):
        model.loss(ids, out_mean=loss_mean)
    torch.cuda.synchronize()
    el_loss = (time.perf_counter() - t2) / args.steps
    loss_step = {"value": round(B * T / el_loss, 1), "unit": "tokens/s", "ms_per_step": round(el_loss * 1e3, 4),
                 "mean_loss": round(float(loss_mean.item()), 5)}

    # the same workload with every variant switch on (Post-LN wiring, per-layer
    # score scaling, erf GELU, separate head): its own weights, same ids
    import dataclasses
    vshape = dataclasses.replace(w.shape, post_ln=True, scale_attn_by_inverse_layer_idx=True, activation="gelu",
                                 tie_word_embeddings=False)
    vmodel = GPT2.from_shape(vshape, w.dtype, max_batch=B, max_seq=T, logits_dtype=logits_dtype)
    vmodel.load_blob(W.make_params(vshape, w.init, w.param_seed))
    for _ in range(args.warmup):
        vmodel.forward(ids, out_logits=logits, padded_logits=True)
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    for _ in range(args.steps):
        vmodel.forward(ids, out_logits=logits, padded_logits=True)
    torch.cuda.synchronize()
    el_v = (time.perf_counter() - t3) / args.steps
    variant_step = {"switches": ["post_ln", "scale_attn_by_inverse_layer_idx", "gelu_erf", "separate_head"],
                    "value": round(B * T / el_v, 1), "unit": "tokens/s", "ms_per_step": round(el_v * 1e3, 4)}
    del vmodel

    # backward of one block (gpt2_block_backward, layer 0) on the same batch:
    # seeded fp32 block input and output gradient
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    xb = torch.randn((B, T, w.shape.d_model), generator=gen, device=dev, dtype=torch.float32)
    dyb = torch.randn((B, T, w.shape.d_model), generator=gen, device=dev, dtype=torch.float32)
    dxb, gb = model.block_backward(0, xb, dyb)
    for _ in range(max(1, args.warmup // 2)):
        model.block_backward(0, xb, dyb, out_dx=dxb, out_grads=gb)
    torch.cuda.synchronize()
    nb = max(2, args.steps // 4)
    t4 = time.perf_counter()
    for _ in range(nb):
        model.block_backward(0, xb, dyb, out_dx=dxb, out_grads=gb)
    torch.cuda.synchronize()
    el_b = (time.perf_counter() - t4) / nb
    bflop = backward_block_flops(w.shape, B, T)
    block_backward = {"layer": 0, "ms_per_call": round(el_b * 1e3, 4), "algorithmic_tflop": round(bflop / 1e12, 4),
                      "achieved_tflops": round(bflop / el_b / 1e12, 2),
                      "note": "includes the recomputed forward of the block"}
    del xb, dyb, dxb, gb
    model._bwd_ws = None

    # the same forward storing fp32 logits (reported beside the headline value)
    alt = None
    if logits_dtype != "f32":
        del logits
        model32 = GPT2.from_shape(w.shape, w.dtype, max_batch=B, max_seq=T, logits_dtype="f32")
        model32.load_blob(blob)
        logits32 = torch.empty((B, T, ld), dtype=torch.float32, device=dev)
        for _ in range(args.warmup):
            model32.forward(ids, out_logits=logits32, padded_logits=True)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(args.steps):
            model32.forward(ids, out_logits=logits32, padded_logits=True)
        torch.cuda.synchronize()
        el32 = (time.perf_counter() - t1) / args.steps
        alt = {"value": round(B * T / el32, 1), "ms_per_step": round(el32 * 1e3, 4)}
        del model32, logits32

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
                   "n_layer": w.shape.n_layer, "n_head": w.shape.n_head, "vocab": w.shape.vocab,
                   "logits_dtype": logits_dtype, "logits_row_stride": ld},
        "frac_of_peak": round(flops / (elapsed / args.steps) / (peak * 1e12), 4),
        "algorithmic_tflop_per_step": round(flops / 1e12, 4),
        "roofline": roof,
        "per_class_ms": {c: round(v["ms_per_step"], 4) for c, v in per_class.items()},
    }
    out["loss_step"] = loss_step
    out["variant_step"] = variant_step
    out["block_backward"] = block_backward
    if alt is not None:
        out["fp32_logits"] = alt
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


def bench_decode(args, w):
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
    # greedy generation (gpt2_generate): the first 960 tokens as the prompt,
    # 64 steps chained on the device (positions 959 .. 1022), no logits stored
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
    generate = {"value": round(B * gen_steps / gdt, 1), "unit": "tokens/s", "batch": B, "prompt": gen_prompt,
                "steps": gen_steps, "ms_per_step": round(gdt * 1e3 / gen_steps, 4)}

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
           "dtype": w.dtype, "data": "synthetic", "config": {"workload": w.name, "batch": B, "prefix": P, "logits_dtype": logits_dtype},
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                        "kernel": "whole decode step", "algorithmic_bytes": total},
           "generate": generate}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
