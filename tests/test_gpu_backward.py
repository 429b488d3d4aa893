"""GPU parity of the block backward (gpt2_block_backward) against the fp64
oracle's block_backward: dx and every parameter gradient, normwise, with the
forward's tolerances (fp32 1e-4; bf16 2e-2).  In bf16 mode the error is that
of the bf16 operand pipeline: the fp64 oracle with the same operands rounded
to bf16 at the same points (LayerNorm outputs, q/k/v, the attention output,
dy, dg, dx_h, dO, dqkv) reproduces the GPU's error, and it is dominated by
the forward's LayerNorm-output and q/k/v roundings, which sharp attention
scores amplify.  Shapes span several 64-row attention tiles with ragged
tails, head sizes 16 and 64, d_model 64 / 128 / 192 (the general LayerNorm
path), layers 0 and 1 (the per-layer score scale), both GELU forms; the
GPT-2 small case uses the workload's own initialisation.
Every case prints its name before touching the GPU.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest

import oracle
import workloads as W
from parity import normwise, TOL_F32, TOL_BF16

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _announce(msg):
    print(f"\n[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gpt_pre_ln_amd import binding
    binding.load()


def _init(std=0.08):
    return W.Init(w_std=std, proj_std=std, bias_std=0.05, gamma=(1.0, 0.2), beta=(0.0, 0.2))


def _split_grads(g, D, F, l):
    """The layer's gradient vector (blob order) as a dict keyed like the oracle."""
    sizes = [("ln_1.w", (D,)), ("ln_1.b", (D,)), ("attn.c_attn.w", (D, 3 * D)), ("attn.c_attn.b", (3 * D,)),
             ("attn.c_proj.w", (D, D)), ("attn.c_proj.b", (D,)), ("ln_2.w", (D,)), ("ln_2.b", (D,)),
             ("mlp.c_fc.w", (D, F)), ("mlp.c_fc.b", (F,)), ("mlp.c_proj.w", (F, D)), ("mlp.c_proj.b", (D,))]
    out, off = {}, 0
    for k, shp in sizes:
        n = int(np.prod(shp))
        out[f"h.{l}.{k}"] = g[off:off + n].reshape(shp)
        off += n
    assert off == g.size
    return out


def _run(s, dtype, B, T, layer, seed, init=None):
    from gpt_pre_ln_amd.model import GPT2
    blob = W.make_params(s, init or _init(), seed)
    rng = np.random.default_rng(seed + 1)
    x = rng.normal(0.0, 1.0, size=(B, T, s.d_model)).astype(np.float32)
    dy = rng.normal(0.0, 1.0, size=(B, T, s.d_model)).astype(np.float32)
    m = GPT2.from_shape(s, dtype, max_batch=B, max_seq=T)
    m.load_blob(blob)
    dx, g = m.block_backward(layer, torch.from_numpy(x).to(DEV), torch.from_numpy(dy).to(DEV))
    torch.cuda.synchronize()
    return blob, x, dy, dx.cpu().numpy(), g.cpu().numpy()


def _compare(s, dtype, blob, x, dy, dx, g, layer, label, seqs=None):
    P = oracle.prepare_params(blob, s, dtype)
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    sel = slice(None) if seqs is None else seqs
    rdx, rg = oracle.block_backward_batch(x[sel].astype(np.float64), dy[sel].astype(np.float64), P, layer)
    errs = {"dx": normwise(dx[sel], rdx)}
    if seqs is None:
        for k, v in _split_grads(g, s.d_model, s.d_ff, layer).items():
            errs[k.split(".", 2)[-1]] = normwise(v, rg[k])
    worst = max(errs, key=errs.get)
    print(f"[backward] {label} worst {worst} {errs[worst]:.2e} | " +
          " ".join(f"{k}={v:.1e}" for k, v in errs.items()), flush=True)
    assert np.isfinite(dx).all() and np.isfinite(g).all()
    for k, e in errs.items():
        assert e <= tol, f"{label}: {k} normwise {e:.3e} > {tol}"


CASES = [
    # dtype, d_model, n_head, n_layer, layer, B, T, switches
    ("f32", 64, 4, 2, 1, 2, 37, {}),                                    # head size 16, one ragged tile
    ("f32", 128, 2, 1, 0, 1, 130, {}),                                  # head size 64, three tiles
    ("bf16", 128, 2, 2, 1, 2, 200, {}),
    ("bf16", 192, 3, 1, 0, 3, 65, {}),                                  # general LayerNorm path
    ("bf16", 128, 2, 2, 1, 2, 100, dict(activation="gelu", scale_attn_by_inverse_layer_idx=True)),
    ("bf16", 128, 2, 1, 0, 1, 1, {}),                                   # a single position
    ("bf16", 128, 2, 1, 0, 20, 1000, dict(n_positions=1024)),  # dK/dV grid of 640 blocks: a plain, a reversed and a partial run of 256
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(str(v) for v in c[:7]) + ("-var" if set(c[7]) - {"n_positions"} else ""))
def test_block_backward_matches_oracle(case):
    dtype, D, H, L, layer, B, T, sw = case
    _announce(f"block backward {case}")
    s = dataclasses.replace(W.ModelShape(vocab=300, n_positions=256, d_model=D, n_head=H, n_layer=L, d_ff=4 * D),
                            **sw)
    blob, x, dy, dx, g = _run(s, dtype, B, T, layer, 800 + D + T)
    _compare(s, dtype, blob, x, dy, dx, g, layer, f"{case}")


@pytest.mark.parametrize("D,H,B,T", [(128, 2, 2, 640), (192, 3, 1, 1088)])
def test_block_backward_kmajor_weight_gradients(D, H, B, T):
    """bf16 with B*T a multiple of 64 and k-loops over 1024 positions: the
    weight gradients read the activations K-major (no transposed copies),
    with split-K slices; d_model 192 leaves partial 128-wide tiles."""
    _announce(f"block backward K-major bf16 D={D} H={H} B={B} T={T}")
    s = W.ModelShape(vocab=300, n_positions=2048, d_model=D, n_head=H, n_layer=1, d_ff=4 * D)
    blob, x, dy, dx, g = _run(s, "bf16", B, T, 0, 850 + D + T)
    _compare(s, "bf16", blob, x, dy, dx, g, 0, f"K-major D={D} B={B} T={T}")


def test_block_backward_gpt2_small():
    """GPT-2 small shapes: B=8 T=1024 (the benchmark batch; the weight
    gradients take the split-K products, 4 to 16 slices), dx and every
    gradient against the oracle over all 8 sequences; B=1 T=1024 (2 slices)
    likewise."""
    w = W.WORKLOADS["gpt2-small-b8t1024"]
    s = w.shape
    _announce(f"{w.name} block backward layer 5, B=8 T=1024 and B=1")
    blob, x, dy, dx, g = _run(s, w.dtype, 8, 1024, 5, 901, w.init)
    _compare(s, w.dtype, blob, x, dy, dx, g, 5, "gpt2-small B=8")
    blob, x, dy, dx, g = _run(s, w.dtype, 1, 1024, 5, 903, w.init)
    _compare(s, w.dtype, blob, x, dy, dx, g, 5, "gpt2-small B=1")
