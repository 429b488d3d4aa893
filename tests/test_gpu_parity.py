"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every case prints its name, shape and dtype before touching the GPU, so a
failure names itself.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as W
from parity import assert_logits, normwise, TOL_F32, TOL_BF16

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
    binding.load()  # fails loudly if the library was not built


def _model(shape, dtype, B, T, blob):
    from gpt_pre_ln_amd.model import GPT2
    m = GPT2.from_shape(shape, dtype, max_batch=B, max_seq=T)
    m.load_blob(blob)
    return m


def _ids_dev(ids):
    return torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).to(DEV)


def _init_small(std=0.2):
    return W.Init(w_std=std, proj_std=std, bias_std=0.05, gamma=(1.0, 0.2), beta=(0.0, 0.2))


# ------------------------------------------------------------------ tiny fp32


def test_tiny_fp32_full_logits():
    w = W.WORKLOADS["gpt2-tiny-fp32-b1t16"]
    _announce(f"{w.name} B={w.batch} T={w.seq_len} dtype={w.dtype}")
    blob = W.make_params(w)
    ids = W.make_ids(w)
    m = _model(w.shape, w.dtype, w.batch, w.seq_len, blob)
    lg, hid = m.forward(_ids_dev(ids), hidden=True)
    torch.cuda.synchronize()
    P = oracle.prepare_params(blob, w.shape, w.dtype)
    ref = oracle.forward(P, ids)
    assert_logits(lg.float().cpu().numpy(), ref, "f32", w.name)
    ref_h = np.stack([oracle.forward_hidden(P, ids[b]) for b in range(w.batch)])
    assert normwise(hid.cpu().numpy(), ref_h) <= TOL_F32


# ------------------------------------------------------------ ragged shapes

RAGGED = [
    # dtype, d_model, n_head, n_layer, vocab, n_positions, B, T
    ("f32", 64, 4, 2, 512, 64, 1, 1),
    ("f32", 64, 4, 2, 300, 64, 3, 37),
    ("f32", 128, 2, 2, 1000, 256, 2, 200),
    ("bf16", 128, 2, 2, 1000, 256, 3, 200),
    ("bf16", 192, 3, 1, 777, 300, 1, 1),
    ("bf16", 192, 3, 1, 777, 300, 2, 129),
    ("bf16", 256, 4, 3, 4099, 300, 2, 300),
    ("bf16", 128, 2, 1, 1000, 1024, 20, 1000),  # attention grid of 640 blocks: a plain, a reversed and a partial run of 256
]


@pytest.mark.parametrize("case", RAGGED, ids=lambda c: "-".join(map(str, c)))
def test_ragged_shapes_logits_hidden_trace(case):
    dtype, D, H, L, V, P_, B, T = case
    _announce(f"ragged {case}")
    s = W.ModelShape(vocab=V, n_positions=P_, d_model=D, n_head=H, n_layer=L, d_ff=4 * D)
    blob = W.make_params(s, _init_small(0.08), 77 + D + T)
    ids = np.random.default_rng(D * 1000 + T).integers(0, V, size=(B, T)).astype(np.int32)
    m = _model(s, dtype, B, T, blob)
    trace = torch.full((L, B * T, D), float("nan"), dtype=torch.float32, device=DEV)
    m.set_trace(trace)
    lg, hid = m.forward(_ids_dev(ids), hidden=True)
    m.set_trace(None)
    torch.cuda.synchronize()
    Pp = oracle.prepare_params(blob, s, dtype)
    tr = {}
    ref_h = np.stack([oracle.forward_hidden(Pp, ids[b], trace=tr) for b in range(B)])
    ref = np.einsum("btd,vd->btv", ref_h, Pp["wte"])
    # per-layer residual stream (X_{l+1}) localises any failure
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    trace_np = trace.cpu().numpy().reshape(L, B, T, D)
    for l in range(L):
        ref_l = np.stack([tr["l_out"][b * L + l] for b in range(B)])
        e = normwise(trace_np[l], ref_l)
        assert e <= tol, f"layer {l} residual stream normwise {e:.3e}"
    assert normwise(hid.cpu().numpy(), ref_h) <= tol
    assert_logits(lg.float().cpu().numpy(), ref, dtype, f"ragged {case}")


# ------------------------------------------------------------ invariants on GPU


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_causality_bitwise_gpu(dtype):
    _announce(f"causality dtype={dtype}")
    s = W.ModelShape(vocab=600, n_positions=512, d_model=128, n_head=2, n_layer=2, d_ff=512)
    blob = W.make_params(s, _init_small(0.08), 5)
    ids = np.random.default_rng(6).integers(0, 600, size=(2, 300)).astype(np.int32)
    m = _model(s, dtype, 2, 300, blob)
    base = m.forward(_ids_dev(ids))[0].float().cpu().numpy()
    for t in (0, 63, 127, 128, 298):
        ids2 = ids.copy()
        ids2[:, t + 1] = (ids2[:, t + 1] + 7) % 600
        out = m.forward(_ids_dev(ids2))[0].float().cpu().numpy()
        np.testing.assert_array_equal(out[:, :t + 1], base[:, :t + 1])
        assert not np.array_equal(out[:, t + 1], base[:, t + 1])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_identity_blocks_gpu(dtype):
    """Zero attn/mlp c_proj weights and biases: logits = LN_f(wte[id] + wpe[t]) @ wte^T."""
    _announce(f"identity blocks dtype={dtype}")
    s = W.ModelShape(vocab=900, n_positions=128, d_model=128, n_head=2, n_layer=3, d_ff=512)
    blob = W.make_params(s, _init_small(0.1), 8)
    view = W.unpack(blob, s)
    for l in range(s.n_layer):
        for k in ("attn.c_proj.w", "attn.c_proj.b", "mlp.c_proj.w", "mlp.c_proj.b"):
            view[f"h.{l}.{k}"][...] = 0.0
    ids = np.random.default_rng(9).integers(0, 900, size=(2, 100)).astype(np.int32)
    m = _model(s, dtype, 2, 100, blob)
    lg = m.forward(_ids_dev(ids))[0].float().cpu().numpy()
    P = oracle.prepare_params(blob, s, dtype)
    x0 = P["wte"][ids] + P["wpe"][:100]
    expect = oracle.layer_norm(x0, P["ln_f.w"], P["ln_f.b"]) @ P["wte"].T
    assert_logits(lg, expect, dtype, "identity")


def test_sharp_attention_scores():
    """Attention scores spread over hundreds of natural-log units within a row.

    The online softmax must take every exponential against a maximum shared by
    all lanes holding a query: a maximum taken over a subset of the keys leaves
    exp() arguments far above 88 and the output overflows.  fp32, exact parity.
    """
    _announce("sharp attention f32")
    s = W.ModelShape(vocab=512, n_positions=256, d_model=128, n_head=2, n_layer=2, d_ff=512)
    blob = W.make_params(s, _init_small(0.08), 15)
    view = W.unpack(blob, s)
    for l in range(s.n_layer):
        view[f"h.{l}.attn.c_attn.w"][...] *= 6.5
    ids = np.random.default_rng(16).integers(0, 512, size=(2, 200)).astype(np.int32)
    P = oracle.prepare_params(blob, s, "f32")
    tr = {}
    ref_h = np.stack([oracle.forward_hidden(P, ids[b], trace=tr) for b in range(2)])
    # the case is only meaningful if the scores really are that spread out
    h0 = tr["attn_norm"][0]
    qkv = h0 @ P["h.0.attn.c_attn.w"] + P["h.0.attn.c_attn.b"]
    q, k = qkv[:, :64], qkv[:, 128:192]
    sc = (q @ k.T) / 8.0
    spread = max(np.ptp(sc[i, :i + 1]) for i in range(1, 200))
    assert spread > 200.0, f"score spread only {spread:.1f}"
    m = _model(s, "f32", 2, 200, blob)
    lg = m.forward(_ids_dev(ids))[0].float().cpu().numpy()
    assert_logits(lg, np.einsum("btd,vd->btv", ref_h, P["wte"]), "f32", "sharp attention")


@pytest.mark.parametrize("dtype,logits_dtype", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32")])
def test_padded_logits_layout(dtype, logits_dtype):
    """gpt2_forward_strided with the padded row stride: the [B,T,V] view holds
    the same values as the contiguous layout (same kernels and accumulators),
    the padding columns hold 0, and nothing past the padded stride is written."""
    from gpt_pre_ln_amd.model import GPT2
    s = W.ModelShape(vocab=777, n_positions=160, d_model=128, n_head=2, n_layer=2, d_ff=512)
    Bsz, T = 3, 150
    _announce(f"padded logits {dtype}/{logits_dtype} V={s.vocab} B={Bsz} T={T}")
    blob = W.make_params(s, _init_small(), 11)
    ids = np.random.default_rng(12).integers(0, s.vocab, size=(Bsz, T)).astype(np.int32)
    m = GPT2.from_shape(s, dtype, max_batch=Bsz, max_seq=T, logits_dtype=logits_dtype)
    m.load_blob(blob)
    ld = m.logits_padded_ld
    assert ld == 1024
    ref = m.forward(_ids_dev(ids))[0]
    buf = torch.full((Bsz, T, ld + 64), 7.0, dtype=ref.dtype, device=DEV)
    view = buf[..., :ld]   # rows ld + 64 apart: columns [ld, ld + 64) must stay untouched
    from gpt_pre_ln_amd import binding as Bn
    Bn.gpt2_forward_strided(m.handle, _ids_dev(ids).data_ptr(), Bsz, T, buf.data_ptr(), ld + 64, None, None, m.stream)
    torch.cuda.synchronize()
    assert torch.equal(view[..., :s.vocab], ref)
    assert (view[..., s.vocab:] == 0).all()
    assert (buf[..., ld:] == 7.0).all()
    lg, _ = m.forward(_ids_dev(ids), padded_logits=True)
    assert lg.shape == (Bsz, T, s.vocab) and torch.equal(lg, ref)


def test_padded_logits_gpt2_small_full_size():
    """The padded layout on the GPT-2 small B=8 T=1024 lm_head (256x256 tiles,
    whole rows): bitwise the contiguous logits, zero padding columns."""
    w = W.WORKLOADS["gpt2-small-b8t1024"]
    _announce(f"{w.name} padded logits")
    m = _model(w.shape, w.dtype, w.batch, w.seq_len, W.make_params(w))
    ids = _ids_dev(W.make_ids(w))
    ref = m.forward(ids)[0]
    lg, _ = m.forward(ids, padded_logits=True)
    torch.cuda.synchronize()
    assert torch.equal(lg, ref)
    base = lg.as_strided((w.batch, w.seq_len, m.logits_padded_ld), lg.stride())
    assert (base[..., w.shape.vocab:] == 0).all()


def test_fp32_logits_from_bf16_model():
    """logits_dtype f32 on a bf16 model: the same lm_head products, stored unrounded."""
    _announce("bf16 model, fp32 logits")
    from gpt_pre_ln_amd.model import GPT2
    s = W.ModelShape(vocab=1001, n_positions=256, d_model=128, n_head=2, n_layer=2, d_ff=512)
    blob = W.make_params(s, _init_small(0.08), 17)
    ids = np.random.default_rng(18).integers(0, 1001, size=(2, 150)).astype(np.int32)
    m32 = GPT2.from_shape(s, "bf16", max_batch=2, max_seq=150, logits_dtype="f32")
    m32.load_blob(blob)
    m16 = _model(s, "bf16", 2, 150, blob)
    lg32 = m32.forward(_ids_dev(ids))[0]
    lg16 = m16.forward(_ids_dev(ids))[0]
    assert lg32.dtype == torch.float32 and lg16.dtype == torch.bfloat16
    # the bf16 logits are the fp32 ones rounded to nearest even
    np.testing.assert_array_equal(lg32.to(torch.bfloat16).float().cpu().numpy(), lg16.float().cpu().numpy())
    P = oracle.prepare_params(blob, s, "bf16")
    ref = oracle.forward(P, ids)
    assert_logits(lg32.cpu().numpy(), ref, "bf16", "fp32 logits")


def test_batch_independence_gpu():
    _announce("batch permutation bf16")
    s = W.ModelShape(vocab=500, n_positions=256, d_model=128, n_head=2, n_layer=2, d_ff=512)
    blob = W.make_params(s, _init_small(0.08), 10)
    ids = np.random.default_rng(11).integers(0, 500, size=(4, 150)).astype(np.int32)
    m = _model(s, "bf16", 4, 150, blob)
    base = m.forward(_ids_dev(ids))[0].float().cpu().numpy()
    perm = [3, 1, 0, 2]
    out = m.forward(_ids_dev(ids[perm]))[0].float().cpu().numpy()
    np.testing.assert_array_equal(out, base[perm])


# ------------------------------------------------------------ decode


@pytest.mark.parametrize("dtype,Bsz", [("f32", 3), ("bf16", 3), ("bf16", 40)])
def test_decode_small_shapes(dtype, Bsz):
    """Prefill P tokens into the cache, then several decode steps; each step must
    match the oracle's row P+i of the plain forward.  Up to 32 sequences the
    residual projections take the split-K path, beyond it the tiled GEMM."""
    _announce(f"decode small dtype={dtype} B={Bsz}")
    s = W.ModelShape(vocab=700, n_positions=300, d_model=128, n_head=2, n_layer=2, d_ff=512)
    blob = W.make_params(s, _init_small(0.08), 12)
    Pn, steps, max_T = 61, 4, 70
    rng = np.random.default_rng(13)
    ids = rng.integers(0, 700, size=(Bsz, Pn + steps)).astype(np.int32)
    m = _model(s, dtype, Bsz, Pn, blob)
    kv = m.new_kv_cache(Bsz, max_T)
    m.forward(_ids_dev(ids[:, :Pn]), logits=False, kv=kv)
    assert kv.past_len == Pn
    P = oracle.prepare_params(blob, s, dtype)
    ref_all = oracle.forward(P, ids)
    for i in range(steps):
        lg = m.decode_step(kv, _ids_dev(ids[:, Pn + i])).float().cpu().numpy()
        assert kv.past_len == Pn + i + 1
        assert_logits(lg, ref_all[:, Pn + i], dtype, f"decode step {i}")


@pytest.mark.parametrize("dtype,d_model,n_head,Pn", [("bf16", 128, 2, 600), ("f32", 64, 4, 700)])
def test_decode_many_heads_sliced_keys(dtype, d_model, n_head, Pn):
    """At least 96 (sequence, head) pairs: decode attention takes one block per
    pair and merges its 256-key slices in LDS.  Prefixes of 600 / 700 keys give
    three slices with a ragged last one; the steps must match the oracle."""
    Bsz = 48
    _announce(f"decode sliced keys dtype={dtype} D={d_model} H={n_head} B={Bsz} prefix={Pn}")
    s = W.ModelShape(vocab=600, n_positions=1024, d_model=d_model, n_head=n_head, n_layer=2, d_ff=4 * d_model)
    blob = W.make_params(s, _init_small(0.08), 15)
    steps, max_T = 2, Pn + 8
    rng = np.random.default_rng(16)
    ids = rng.integers(0, 600, size=(Bsz, Pn + steps)).astype(np.int32)
    m = _model(s, dtype, Bsz, Pn, blob)
    kv = m.new_kv_cache(Bsz, max_T)
    m.forward(_ids_dev(ids[:, :Pn]), logits=False, kv=kv)
    sel = [0, 17, 47]
    P = oracle.prepare_params(blob, s, dtype)
    ref_all = oracle.forward(P, ids[sel])
    for i in range(steps):
        lg = m.decode_step(kv, _ids_dev(ids[:, Pn + i])).float().cpu().numpy()
        assert_logits(lg[sel], ref_all[:, Pn + i], dtype, f"sliced decode step {i}")


def test_decode_capacity_error():
    from gpt_pre_ln_amd import binding
    s = W.ModelShape(vocab=100, n_positions=64, d_model=64, n_head=1, n_layer=1, d_ff=256)
    blob = W.make_params(s, _init_small(0.08), 14)
    m = _model(s, "bf16", 1, 8, blob)
    kv = m.new_kv_cache(1, 8)
    m.forward(_ids_dev(np.arange(8, dtype=np.int32)[None]), logits=False, kv=kv)
    with pytest.raises(binding.GPT2Error) as e:
        m.decode_step(kv, _ids_dev(np.array([1], np.int32)))
    assert e.value.status == binding.GPT2_ERR_CAPACITY


# ------------------------------------------------------------ full-size workloads


def test_gpt2_small_b8t1024():
    w = W.WORKLOADS["gpt2-small-b8t1024"]
    _announce(f"{w.name} B={w.batch} T={w.seq_len}")
    blob = W.make_params(w)
    ids = W.make_ids(w)
    m = _model(w.shape, w.dtype, w.batch, w.seq_len, blob)
    lg = m.forward(_ids_dev(ids))[0]
    torch.cuda.synchronize()
    P = oracle.prepare_params(blob, w.shape, w.dtype)
    # sequences are independent: the oracle runs sequences 0 and 7 in full
    for b in (0, 7):
        ref = oracle.forward(P, ids[b:b + 1])[0]
        assert_logits(lg[b].float().cpu().numpy(), ref, w.dtype, f"{w.name} seq {b}")


def test_gpt2_small_shape_fp32():
    """The GPT-2 small shape in fp32 (fp32 MFMA operands, fp32 logits) at
    B=8 T=1024: the 128x192 (qkv, c_fc) and 128x96 (c_proj) projection tiles
    and the 256x256 lm_head on the
    fp32 path, checked to the fp32 tolerance and exact argmax on one sequence."""
    w = W.WORKLOADS["gpt2-small-b8t1024"]
    _announce(f"{w.name} shape in f32 B={w.batch} T={w.seq_len}")
    blob = W.make_params(w)
    ids = W.make_ids(w)
    m = _model(w.shape, "f32", w.batch, w.seq_len, blob)
    lg = m.forward(_ids_dev(ids))[0]
    torch.cuda.synchronize()
    got = lg[5].cpu().numpy().astype(np.float64)
    del lg, m
    ref = oracle.forward(oracle.prepare_params(blob, w.shape, "f32"), ids[5:6])[0]
    assert_logits(got, ref, "f32", f"{w.name} f32 seq 5")


def test_gpt2_small_b8t1020_ragged_tiles():
    """B*T = 8160 is not a multiple of the 128-row tiles, and T = 1020 puts
    sequence boundaries inside tiles: the 128x192 (qkv, c_fc) and 128x96
    (both c_proj) projections and the 256x256 lm_head with its ragged last
    tile-row."""
    w = W.WORKLOADS["gpt2-small-b8t1024"]
    T = 1020
    _announce(f"{w.name} shape B={w.batch} T={T}")
    blob = W.make_params(w)
    ids = np.ascontiguousarray(W.make_ids(w)[:, :T])
    m = _model(w.shape, w.dtype, w.batch, T, blob)
    lg = m.forward(_ids_dev(ids))[0]
    torch.cuda.synchronize()
    P = oracle.prepare_params(blob, w.shape, w.dtype)
    for b in (3, 7):
        ref = oracle.forward(P, ids[b:b + 1])[0]
        assert_logits(lg[b].float().cpu().numpy(), ref, w.dtype, f"{w.name} T={T} seq {b}")


def test_gpt2_small_decode_b32p1023():
    w = W.WORKLOADS["gpt2-small-decode-b32p1023"]
    _announce(f"{w.name} B={w.batch} prefix={w.seq_len}")
    blob = W.make_params(w)
    prefix, new = W.make_decode_ids(w)
    m = _model(w.shape, w.dtype, w.batch, w.seq_len + 1, blob)
    kv = m.new_kv_cache(w.batch, w.seq_len + 1)
    m.forward(_ids_dev(prefix), logits=False, kv=kv)
    lg = m.decode_step(kv, _ids_dev(new)).float().cpu().numpy()
    # the GPU's own full forward over prefix ++ new, last row, for every sequence
    full = np.concatenate([prefix, new[:, None]], axis=1).astype(np.int32)
    lg_full = m.forward(_ids_dev(full))[0][:, -1].float().cpu().numpy()
    assert normwise(lg, lg_full) <= TOL_BF16
    P = oracle.prepare_params(blob, w.shape, w.dtype)
    sel = [0, 31]
    ref = oracle.decode_logits(P, prefix[sel], new[sel])
    assert_logits(lg[sel], ref, w.dtype, f"{w.name} seqs {sel}")


@pytest.mark.slow
@pytest.mark.parametrize("name,prefix", [("gpt2-medium-b8t1024", 1024), ("gpt2-xl-b4t1024", 256)])
def test_large_workloads(name, prefix):
    """Full-size forward on the GPU; the oracle checks sequence 0 on its first
    `prefix` positions (exact by causality: rows <= t depend on tokens <= t)."""
    w = W.WORKLOADS[name]
    _announce(f"{w.name} B={w.batch} T={w.seq_len} oracle prefix {prefix}")
    blob = W.make_params(w)
    ids = W.make_ids(w)
    m = _model(w.shape, w.dtype, w.batch, w.seq_len, blob)
    lg = m.forward(_ids_dev(ids))[0]
    torch.cuda.synchronize()
    got = lg[0, :prefix].float().cpu().numpy()
    del lg, m
    P = oracle.prepare_params(blob, w.shape, w.dtype)
    del blob
    ref = oracle.forward(P, ids[0:1, :prefix])[0]
    assert_logits(got, ref, w.dtype, f"{w.name} seq 0 rows 0..{prefix - 1}")
