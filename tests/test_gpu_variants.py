"""GPU parity of the model variants (config switches) against the oracle:
Post-LN wiring, per-layer attention score scaling, erf GELU, a separate head,
each alone and all together, through the forward (logits, final hidden
state, per-layer residual trace), the decode step (split-K path at B <= 32,
tiled path beyond), the fused loss and greedy generation.  Same tolerances
as the other parity tests.  Every case prints its name before touching the GPU.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest

import oracle
import workloads as W
from parity import assert_logits, normwise, TOL_F32, TOL_BF16

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

VARIANTS = {
    "post_ln": dict(post_ln=True),
    "layer_scale": dict(scale_attn_by_inverse_layer_idx=True),
    "gelu_erf": dict(activation="gelu"),
    "untied": dict(tie_word_embeddings=False),
    "all": dict(post_ln=True, scale_attn_by_inverse_layer_idx=True, activation="gelu", tie_word_embeddings=False),
}


def _announce(msg):
    print(f"\n[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gpt_pre_ln_amd import binding
    binding.load()


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def _shape(name, V=777, L=3):
    base = W.ModelShape(vocab=V, n_positions=256, d_model=128, n_head=2, n_layer=L, d_ff=512)
    return dataclasses.replace(base, **VARIANTS[name])


def _init():
    return W.Init(w_std=0.08, proj_std=0.08, bias_std=0.05, gamma=(1.0, 0.2), beta=(0.0, 0.2))


def _model(s, dtype, B, T, blob, **kw):
    from gpt_pre_ln_amd.model import GPT2
    m = GPT2.from_shape(s, dtype, max_batch=B, max_seq=T, **kw)
    m.load_blob(blob)
    return m


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name", list(VARIANTS))
def test_variant_forward(name, dtype):
    _announce(f"variant forward {name} {dtype}")
    s = _shape(name)
    B, T = 2, 150
    blob = W.make_params(s, _init(), 71)
    ids = np.random.default_rng(72).integers(0, s.vocab, size=(B, T)).astype(np.int32)
    m = _model(s, dtype, B, T, blob)
    trace = torch.full((s.n_layer, B * T, s.d_model), float("nan"), dtype=torch.float32, device=DEV)
    m.set_trace(trace)
    lg, hid = m.forward(_dev(ids), hidden=True)
    m.set_trace(None)
    torch.cuda.synchronize()
    P = oracle.prepare_params(blob, s, dtype)
    tr = {}
    ref_h = np.stack([oracle.forward_hidden(P, ids[b], trace=tr) for b in range(B)])
    head = P["lm_head.w"] if "lm_head.w" in P else P["wte"]
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    trace_np = trace.cpu().numpy().reshape(s.n_layer, B, T, s.d_model)
    for l in range(s.n_layer):
        ref_l = np.stack([tr["l_out"][b * s.n_layer + l] for b in range(B)])
        e = normwise(trace_np[l], ref_l)
        assert e <= tol, f"layer {l} residual stream normwise {e:.3e}"
    assert normwise(hid.cpu().numpy(), ref_h) <= tol
    assert_logits(lg.float().cpu().numpy(), np.einsum("btd,vd->btv", ref_h, head), dtype, f"variant {name}")


@pytest.mark.parametrize("dtype,Bsz", [("f32", 3), ("bf16", 3), ("bf16", 40)])
@pytest.mark.parametrize("name", ["post_ln", "all"])
def test_variant_decode(name, dtype, Bsz):
    _announce(f"variant decode {name} {dtype} B={Bsz}")
    s = _shape(name)
    Pn, steps, max_T = 33, 3, 40
    blob = W.make_params(s, _init(), 73)
    ids = np.random.default_rng(74).integers(0, s.vocab, size=(Bsz, Pn + steps)).astype(np.int32)
    m = _model(s, dtype, Bsz, Pn, blob)
    kv = m.new_kv_cache(Bsz, max_T)
    m.forward(_dev(ids[:, :Pn]), logits=False, kv=kv)
    P = oracle.prepare_params(blob, s, dtype)
    ref = oracle.forward(P, ids)
    for i in range(steps):
        lg = m.decode_step(kv, _dev(ids[:, Pn + i])).float().cpu().numpy()
        assert_logits(lg, ref[:, Pn + i], dtype, f"variant {name} decode step {i}")


def test_variant_loss_and_generate():
    """All switches on: the fused loss against the oracle cross-entropy of the
    GPU's own fp32 logits and against the oracle; generation bit-exact
    against step-by-step decode arg-max."""
    _announce("variant all: loss and generation")
    s = _shape("all", V=4099)
    B, T = 3, 64
    blob = W.make_params(s, _init(), 75)
    ids = np.random.default_rng(76).integers(0, s.vocab, size=(B, T)).astype(np.int32)
    m = _model(s, "bf16", B, T, blob, logits_dtype="f32")
    mean, per = m.loss(_dev(ids), token_loss=True)
    own = m.forward(_dev(ids))[0].cpu().numpy()
    per = per.cpu().numpy().astype(np.float64)
    _, per_own = oracle.shifted_cross_entropy(own, ids)
    assert np.abs(per - per_own).max() <= 1e-4
    ref = oracle.forward(oracle.prepare_params(blob, s, "bf16"), ids)
    _, per_ref = oracle.shifted_cross_entropy(ref, ids)
    assert np.abs(per - per_ref).max() <= 2 * TOL_BF16 * np.abs(ref).max()
    # generation from the first 20 tokens, 10 steps
    kv = m.new_kv_cache(B, 40)
    m.forward(_dev(ids[:, :19]), logits=False, kv=kv)
    toks = m.generate(kv, _dev(ids[:, 19]), 10).cpu().numpy()
    kv2 = m.new_kv_cache(B, 40)
    m.forward(_dev(ids[:, :19]), logits=False, kv=kv2)
    feed = np.concatenate([ids[:, 19:20], toks[:, :-1]], axis=1)
    for i in range(10):
        lg = m.decode_step(kv2, _dev(feed[:, i])).cpu().numpy()
        np.testing.assert_array_equal(toks[:, i], lg.argmax(axis=-1))
