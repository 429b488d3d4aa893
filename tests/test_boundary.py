"""The C-ABI library on the CPU: it loads, exports every declared symbol, and its
host-side checks reject bad arguments before any HIP call (no GPU needed)."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gpt2.h")


@pytest.fixture(scope="module")
def B():
    from gpt_pre_ln_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from gpt_pre_ln_amd.build import build
        build(verbose=False)
    binding.load()
    return binding


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gpt2_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(B):
    names = _declared_functions()
    assert len(names) >= 12
    lib = B.load()
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (gpt2_\w+)", out))
    assert set(names) <= exported
    # the binding wraps every declared entry point under the same name
    for n in names:
        if n not in ("gpt2_status_string", "gpt2_last_error"):
            assert hasattr(B, n), f"binding lacks {n}"


def _cfg(B, shape, dtype):
    return B.make_config(shape.vocab, shape.n_positions, shape.d_model, shape.n_head, shape.n_layer,
                         shape.d_ff, shape.ln_eps, dtype, None, shape.activation,
                         shape.scale_attn_by_inverse_layer_idx, shape.post_ln, shape.tie_word_embeddings)


def test_variant_blob_and_region_sizes(B):
    """A separate head adds V*D floats to the blob and V_pad*D elements to the
    device region; the other switches change no size."""
    import dataclasses
    s = W.ModelShape(vocab=1000, n_positions=128, d_model=128, n_head=2, n_layer=2, d_ff=512)
    base = _cfg(B, s, "bf16")
    for kw in (dict(post_ln=True), dict(activation="gelu"), dict(scale_attn_by_inverse_layer_idx=True)):
        v = _cfg(B, dataclasses.replace(s, **kw), "bf16")
        assert B.gpt2_param_blob_floats(v) == B.gpt2_param_blob_floats(base) == W.param_count(s)
        assert B.gpt2_param_bytes(v) == B.gpt2_param_bytes(base)
    su = dataclasses.replace(s, tie_word_embeddings=False)
    u = _cfg(B, su, "bf16")
    assert B.gpt2_param_blob_floats(u) == W.param_count(su) == W.param_count(s) + 1000 * 128
    assert B.gpt2_param_bytes(u) == B.gpt2_param_bytes(base) + 1024 * 128 * 2
    assert list(W.unpack(W.make_params(su, W.Init(0.02, 0.02, 0.0, (1.0, 0.0), (0.0, 0.0)), 1), su))[-1] == "lm_head.w"


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_blob_size_matches_layout(B, name):
    w = W.WORKLOADS[name]
    cfg = _cfg(B, w.shape, w.dtype)
    assert B.gpt2_param_blob_floats(cfg) == W.param_count(w.shape)
    es = 2 if w.dtype == "bf16" else 4
    # device region: matrices at es bytes, wte padded to 256 rows, vectors fp32
    assert B.gpt2_param_bytes(cfg) >= W.param_count(w.shape) * es


def test_kv_cache_bytes(B):
    s = W.SMALL
    cfg = _cfg(B, s, "bf16")
    # [L][K, V^T][B][H][round_up(max_T, 64)][hs] bf16
    assert B.gpt2_kv_cache_bytes(cfg, 32, 1024) == 12 * 2 * 32 * 1024 * 768 * 2
    assert B.gpt2_kv_cache_bytes(cfg, 2, 65) == 12 * 2 * 2 * 128 * 768 * 2


@pytest.mark.parametrize("change,status", [
    (dict(d_model=96, n_head=3), "GPT2_ERR_UNSUPPORTED"),        # head_dim 32
    (dict(d_model=100, n_head=3), "GPT2_ERR_SHAPE"),             # not divisible
    (dict(d_model=64, n_head=4), "GPT2_ERR_UNSUPPORTED"),        # head_dim 16 in bf16
    (dict(dtype=7), "GPT2_ERR_UNSUPPORTED"),
    (dict(logits_dtype=3), "GPT2_ERR_UNSUPPORTED"),
    (dict(n_layer=0), "GPT2_ERR_SHAPE"),
    (dict(d_ff=100), "GPT2_ERR_UNSUPPORTED"),
    (dict(n_positions=5000), "GPT2_ERR_UNSUPPORTED"),
    (dict(activation=2), "GPT2_ERR_UNSUPPORTED"),
    (dict(post_ln=-1), "GPT2_ERR_UNSUPPORTED"),
    (dict(separate_head=3), "GPT2_ERR_UNSUPPORTED"),
    (dict(scale_attn_by_inverse_layer_idx=2), "GPT2_ERR_UNSUPPORTED"),
])
def test_config_validation(B, change, status):
    base = dict(vocab_size=1000, n_positions=128, d_model=128, n_head=2, n_layer=2, d_ff=512, ln_eps=1e-5,
                dtype=B.GPT2_BF16, logits_dtype=B.GPT2_BF16)
    base.update(change)
    cfg = B.gpt2_config(**base)
    n = ctypes.c_size_t()
    assert B.load().gpt2_param_bytes(ctypes.byref(cfg), ctypes.byref(n)) == getattr(B, status)


def test_logits_dtype_defaults_to_the_arithmetic_dtype(B):
    assert B.make_config(512, 64, 64, 4, 2, 256, 1e-5, "f32").logits_dtype == B.GPT2_F32
    assert B.make_config(512, 64, 64, 2, 2, 256, 1e-5, "bf16").logits_dtype == B.GPT2_BF16
    assert B.make_config(512, 64, 64, 2, 2, 256, 1e-5, "bf16", "f32").logits_dtype == B.GPT2_F32


def test_fp32_head_dim_16_is_supported(B):
    cfg = B.make_config(512, 64, 64, 4, 2, 256, 1e-5, "f32")
    assert B.gpt2_param_blob_floats(cfg) == W.param_count(W.TINY)


FAKE = 1 << 30  # aligned, never dereferenced: only host checks run


@pytest.fixture()
def handle(B):
    cfg = B.make_config(1000, 128, 128, 2, 2, 512, 1e-5, "bf16")
    pb = B.gpt2_param_bytes(cfg)
    wb = B.gpt2_workspace_bytes(cfg, 2, 64)
    h = B.gpt2_create(cfg, FAKE, pb, FAKE + (1 << 28), wb)
    yield h, cfg
    B.gpt2_destroy(h)


def test_create_rejects_bad_arguments(B):
    cfg = B.make_config(1000, 128, 128, 2, 2, 512, 1e-5, "bf16")
    pb = B.gpt2_param_bytes(cfg)
    wb = B.gpt2_workspace_bytes(cfg, 1, 1)
    lib = B.load()
    h = ctypes.c_void_p()
    assert lib.gpt2_create(ctypes.byref(cfg), FAKE + 4, pb, FAKE, wb, ctypes.byref(h)) == B.GPT2_ERR_INVALID_ARG
    assert lib.gpt2_create(ctypes.byref(cfg), FAKE, pb - 1, FAKE, wb, ctypes.byref(h)) == B.GPT2_ERR_WORKSPACE
    assert lib.gpt2_create(ctypes.byref(cfg), FAKE, pb, FAKE, wb - 256, ctypes.byref(h)) == B.GPT2_ERR_WORKSPACE
    assert lib.gpt2_create(ctypes.byref(cfg), None, pb, FAKE, wb, ctypes.byref(h)) == B.GPT2_ERR_INVALID_ARG


def test_forward_host_checks(B, handle):
    h, cfg = handle
    lib = B.load()
    fwd = lambda tok, Bz, T, lg=FAKE, hid=None, kv=None: lib.gpt2_forward(
        h, tok, Bz, T, lg, hid, ctypes.byref(kv) if kv else None, None)
    assert fwd(None, 1, 8) == B.GPT2_ERR_INVALID_ARG
    assert fwd(FAKE, 1, 0) == B.GPT2_ERR_SHAPE
    assert fwd(FAKE, 1, 129) == B.GPT2_ERR_SHAPE           # T > n_positions
    assert fwd(FAKE, 0, 8) == B.GPT2_ERR_SHAPE
    assert fwd(FAKE, 4, 64) == B.GPT2_ERR_WORKSPACE        # workspace sized for (2, 64)
    assert fwd(FAKE + 2, 1, 8) == B.GPT2_ERR_INVALID_ARG   # misaligned ids
    assert fwd(FAKE, 1, 8, lg=FAKE + 1) == B.GPT2_ERR_INVALID_ARG  # bf16 logits need 2-byte alignment
    assert fwd(FAKE, 1, 8, hid=FAKE + 4) == B.GPT2_ERR_INVALID_ARG
    kv = B.gpt2_kv_view(FAKE, 2, 32, 0)
    assert fwd(FAKE, 1, 8, kv=kv) == B.GPT2_ERR_SHAPE      # kv.B != B
    assert fwd(FAKE, 2, 40, kv=kv) == B.GPT2_ERR_CAPACITY  # T > max_T
    kv = B.gpt2_kv_view(None, 2, 32, 0)
    assert fwd(FAKE, 2, 8, kv=kv) == B.GPT2_ERR_INVALID_ARG


def test_forward_strided_host_checks(B, handle):
    h, cfg = handle
    lib = B.load()
    assert B.gpt2_logits_padded_ld(cfg) == 1024                    # vocab 1000 -> multiple of 256
    assert B.gpt2_logits_padded_ld(B.make_config(50257, 1024, 768, 12, 12, 3072, 1e-5, "bf16")) == 50432
    fwd = lambda ld, lg=FAKE, Bz=1, T=8: lib.gpt2_forward_strided(h, FAKE, Bz, T, lg, ld, None, None, None)
    assert fwd(999) == B.GPT2_ERR_SHAPE                          # row stride below the vocabulary
    assert fwd(1 << 31) == B.GPT2_ERR_SHAPE                      # beyond int32
    assert fwd(999, lg=None, Bz=4, T=64) == B.GPT2_ERR_WORKSPACE  # no logits: the stride is not checked
    assert fwd(1024, lg=FAKE + 1) == B.GPT2_ERR_INVALID_ARG       # bf16 logits need 2-byte alignment
    assert fwd(1024, Bz=4, T=64) == B.GPT2_ERR_WORKSPACE
    assert lib.gpt2_forward_strided(h, None, 1, 8, FAKE, 1024, None, None, None) == B.GPT2_ERR_INVALID_ARG


def test_forward_loss_host_checks(B, handle):
    h, cfg = handle
    lib = B.load()
    loss = lambda tok, Bz, T, lab=None, per=None, mean=FAKE: lib.gpt2_forward_loss(h, tok, lab, Bz, T, per, mean, None)
    assert loss(None, 1, 8) == B.GPT2_ERR_INVALID_ARG
    assert loss(FAKE, 1, 8, mean=None) == B.GPT2_ERR_INVALID_ARG     # no output requested
    assert loss(FAKE, 1, 1) == B.GPT2_ERR_SHAPE                      # T = 1: nothing to score
    assert loss(FAKE, 1, 129) == B.GPT2_ERR_SHAPE
    assert loss(FAKE, 0, 8) == B.GPT2_ERR_SHAPE
    assert loss(FAKE, 4, 64) == B.GPT2_ERR_WORKSPACE                 # workspace sized for (2, 64)
    assert loss(FAKE + 2, 1, 8) == B.GPT2_ERR_INVALID_ARG
    assert loss(FAKE, 1, 8, lab=FAKE + 2) == B.GPT2_ERR_INVALID_ARG
    assert loss(FAKE, 1, 8, per=FAKE + 1) == B.GPT2_ERR_INVALID_ARG
    assert loss(FAKE, 1, 8, mean=FAKE + 1) == B.GPT2_ERR_INVALID_ARG


def test_decode_host_checks(B, handle):
    h, cfg = handle
    lib = B.load()
    kv = B.gpt2_kv_view(FAKE, 2, 32, 32)
    assert lib.gpt2_decode_step(h, ctypes.byref(kv), FAKE, FAKE, None) == B.GPT2_ERR_CAPACITY
    kv = B.gpt2_kv_view(FAKE, 2, 200, 0)
    assert lib.gpt2_decode_step(h, ctypes.byref(kv), FAKE, FAKE, None) == B.GPT2_ERR_SHAPE
    kv = B.gpt2_kv_view(FAKE, 2, 32, -1)
    assert lib.gpt2_decode_step(h, ctypes.byref(kv), FAKE, FAKE, None) == B.GPT2_ERR_SHAPE
    kv = B.gpt2_kv_view(FAKE, 2, 32, 3)
    assert lib.gpt2_decode_step(h, ctypes.byref(kv), FAKE, None, None) == B.GPT2_ERR_INVALID_ARG


def test_generate_host_checks(B, handle):
    h, cfg = handle
    lib = B.load()
    gen = lambda kv, n, tok=FAKE, out=FAKE: lib.gpt2_generate(h, ctypes.byref(kv), tok, n, out, None)
    kv = B.gpt2_kv_view(FAKE, 2, 32, 30)
    assert gen(kv, 3) == B.GPT2_ERR_CAPACITY      # 30 + 3 > 32
    assert gen(kv, 0) == B.GPT2_ERR_SHAPE
    assert gen(kv, 2, tok=None) == B.GPT2_ERR_INVALID_ARG
    assert gen(kv, 2, out=FAKE + 2) == B.GPT2_ERR_INVALID_ARG
    kv = B.gpt2_kv_view(FAKE, 2, 200, 0)           # max_T > n_positions
    assert gen(kv, 1) == B.GPT2_ERR_SHAPE
    kv = B.gpt2_kv_view(FAKE, 2, 32, -1)
    assert gen(kv, 1) == B.GPT2_ERR_SHAPE
    kv = B.gpt2_kv_view(None, 2, 32, 0)
    assert gen(kv, 1) == B.GPT2_ERR_INVALID_ARG


def test_block_backward_host_checks(B, handle):
    h, cfg = handle
    lib = B.load()
    wb = B.gpt2_block_backward_workspace_bytes(cfg, 2, 64)
    assert wb > B.gpt2_workspace_bytes(cfg, 2, 64)
    bwd = lambda layer=0, Bz=2, T=64, x=FAKE, dy=FAKE + 4096, dx=FAKE + 8192, g=FAKE + 16384, ws=FAKE, n=wb: \
        lib.gpt2_block_backward(h, layer, Bz, T, x, dy, dx, g, ws, n, None)
    assert bwd(layer=2) == B.GPT2_ERR_SHAPE          # 2 layers
    assert bwd(layer=-1) == B.GPT2_ERR_SHAPE
    assert bwd(T=0) == B.GPT2_ERR_SHAPE
    assert bwd(T=129) == B.GPT2_ERR_SHAPE
    assert bwd(n=wb - 1) == B.GPT2_ERR_WORKSPACE
    assert bwd(x=None) == B.GPT2_ERR_INVALID_ARG
    assert bwd(dx=FAKE) == B.GPT2_ERR_INVALID_ARG     # dx aliases x
    assert bwd(g=FAKE + 16388) == B.GPT2_ERR_INVALID_ARG
    assert bwd(ws=FAKE + 16) == B.GPT2_ERR_INVALID_ARG
    post = B.make_config(1000, 128, 128, 2, 2, 512, 1e-5, "bf16", post_ln=True)
    pb = B.gpt2_param_bytes(post)
    hp = B.gpt2_create(post, FAKE, pb, FAKE + (1 << 28), B.gpt2_workspace_bytes(post, 2, 64))
    try:
        assert lib.gpt2_block_backward(hp, 0, 2, 64, FAKE, FAKE + 4096, FAKE + 8192, FAKE + 16384, FAKE, wb,
                                       None) == B.GPT2_ERR_UNSUPPORTED
    finally:
        B.gpt2_destroy(hp)


def test_init_params_size_check(B, handle):
    h, cfg = handle
    n = B.gpt2_param_blob_floats(cfg)
    assert B.load().gpt2_init_params(h, FAKE, n - 1, None) == B.GPT2_ERR_SHAPE
    assert B.load().gpt2_init_params(h, None, n, None) == B.GPT2_ERR_INVALID_ARG


def test_status_strings(B):
    lib = B.load()
    for s in range(7):
        assert lib.gpt2_status_string(s)
    assert lib.gpt2_last_error() is not None


def test_source_hash_matches_the_sources(B):
    """The loaded library was built from the sources beside it (load() refuses
    a stale build; the digest is compiled in)."""
    from gpt_pre_ln_amd.build import source_hash
    assert B.gpt2_source_hash() == source_hash()
    assert re.fullmatch(r"[0-9a-f]{16}", B.gpt2_source_hash())


@pytest.mark.parametrize("dtype,tied", [("bf16", True), ("bf16", False), ("f32", True)])
def test_param_tensor_table(B, dtype, tied):
    """gpt2_param_tensor lists the blob's tensors in the safetensors key order
    (offsets and shapes as the blob layout of workloads.py), each with a
    device copy that is aligned, inside the region and disjoint from the
    others; matrices and embeddings are bf16 in a bf16 model, everything
    else fp32; Conv1D matrices [in, out] are stored transposed."""
    import dataclasses
    s = dataclasses.replace(W.ModelShape(vocab=1000, n_positions=128, d_model=128, n_head=2, n_layer=3, d_ff=512),
                            tie_word_embeddings=tied)
    cfg = _cfg(B, s, dtype)
    offs = W.param_offsets(s)
    n = B.gpt2_param_tensor_count(cfg)
    assert n == len(offs) == 4 + 12 * s.n_layer + (0 if tied else 1)
    region = B.gpt2_param_bytes(cfg)
    spans = []
    for i, (key, (off, shp)) in enumerate(offs.items()):
        t = B.gpt2_param_tensor(cfg, i)
        rows, cols = (shp[0], shp[1]) if len(shp) == 2 else (1, shp[0])
        assert (t.blob_offset, t.rows, t.cols) == (off, rows, cols), key
        matrix = len(shp) == 2
        assert t.dev_dtype == (B.GPT2_BF16 if (dtype == "bf16" and matrix) else B.GPT2_F32), key
        assert t.transposed == int(matrix and key not in ("wte", "wpe", "lm_head.w")), key
        stored_rows, row_len = (cols, rows) if t.transposed else (rows, cols)
        assert t.dev_ld == row_len and t.dev_rows >= stored_rows, key
        if key in ("wte", "lm_head.w"):
            assert t.dev_rows % 256 == 0 and t.dev_rows - stored_rows < 256
        es = 2 if t.dev_dtype == B.GPT2_BF16 else 4
        assert t.dev_offset % 256 == 0
        end = t.dev_offset + t.dev_rows * t.dev_ld * es
        assert end <= region
        spans.append((t.dev_offset, end, key))
    spans.sort()
    for (a0, a1, ka), (b0, b1, kb) in zip(spans, spans[1:]):
        assert a1 <= b0, (ka, kb)
    for bad in (-1, n):
        with pytest.raises(B.GPT2Error) as e:
            B.gpt2_param_tensor(cfg, bad)
        assert e.value.status == B.GPT2_ERR_SHAPE


def test_kv_stride(B):
    s = W.ModelShape(vocab=1000, n_positions=300, d_model=128, n_head=2, n_layer=2, d_ff=512)
    cfg = _cfg(B, s, "bf16")
    for max_T, want in ((1, 64), (40, 64), (64, 64), (65, 128), (70, 128), (300, 320)):
        assert B.gpt2_kv_stride(cfg, max_T) == want
        # the cache size is n_layer * 2 (K and V^T) * B * S * d_model elements
        assert B.gpt2_kv_cache_bytes(cfg, 3, max_T) == s.n_layer * 2 * 3 * want * s.d_model * 2
    for bad in (0, 301):
        with pytest.raises(B.GPT2Error) as e:
            B.gpt2_kv_stride(cfg, bad)
        assert e.value.status == B.GPT2_ERR_SHAPE


def test_set_id_check_host_checks(B, handle):
    h, _ = handle
    assert B.load().gpt2_set_id_check(None, None) == B.GPT2_ERR_INVALID_ARG
    assert B.load().gpt2_set_id_check(h, 0x1002) == B.GPT2_ERR_INVALID_ARG  # not 4-byte aligned
    assert B.load().gpt2_set_id_check(h, 0x1000) == B.GPT2_OK
    assert B.load().gpt2_set_id_check(h, None) == B.GPT2_OK


def test_token_id_clamp_host_build(tmp_path):
    """The clamp the embedding applies to every id (rowops.h, clamp_token_id),
    compiled for the host with the same header: ids outside [0, V) go to the
    nearest row, ids inside are kept."""
    src = tmp_path / "clamp.hip"
    src.write_text('#include "rowops.h"\n#include <cstdio>\n#include <climits>\n'
                   'int main() { const int V = 50257;\n'
                   '  const int ids[] = {INT_MIN, -50257, -1, 0, 1, 777, V - 2, V - 1, V, V + 1, INT_MAX};\n'
                   '  for (int id : ids) std::printf("%d %d\\n", id, gpt2::clamp_token_id(id, V));\n'
                   '  std::printf("%d %d\\n", 5, gpt2::clamp_token_id(5, 1));\n  return 0; }\n')
    exe = tmp_path / "clamp"
    r = subprocess.run(["/opt/rocm/bin/hipcc", "-std=c++20", "-w", "--offload-arch=gfx950",
                        "-I", os.path.join(ROOT, "gpt_pre_ln_amd", "csrc"), str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    got = [tuple(map(int, l.split())) for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                               check=True).stdout.split("\n") if l]
    V = 50257
    want = [(i, min(max(i, 0), V - 1)) for i in (-2**31, -V, -1, 0, 1, 777, V - 2, V - 1, V, V + 1, 2**31 - 1)]
    assert got == want + [(5, 0)]


def test_decode_noalloc_host_checks(B, handle):
    """The allocation-free decode step rejects what gpt2_decode_step rejects,
    and a batch whose scratch exceeds the per-device array, before any HIP call."""
    h, cfg = handle
    lib = B.load()
    kv = B.gpt2_kv_view(FAKE + (1 << 30), 2, 64, 0)
    assert lib.gpt2_decode_step_noalloc(None, ctypes.byref(kv), FAKE, FAKE, None) == B.GPT2_ERR_INVALID_ARG
    assert lib.gpt2_decode_step_noalloc(h, ctypes.byref(kv), None, FAKE, None) == B.GPT2_ERR_INVALID_ARG
    assert lib.gpt2_decode_step_noalloc(h, ctypes.byref(kv), FAKE, None, None) == B.GPT2_ERR_INVALID_ARG
    full = B.gpt2_kv_view(FAKE + (1 << 30), 2, 64, 64)
    assert lib.gpt2_decode_step_noalloc(h, ctypes.byref(full), FAKE, FAKE, None) == B.GPT2_ERR_CAPACITY
    long = B.gpt2_kv_view(FAKE + (1 << 30), 2, 129, 0)   # n_positions is 128
    assert lib.gpt2_decode_step_noalloc(h, ctypes.byref(long), FAKE, FAKE, None) == B.GPT2_ERR_SHAPE
    need1, limit = B.gpt2_decode_scratch_bytes(cfg, 1)
    assert 0 < need1 < limit == 16 << 20
    big = 1
    while B.gpt2_decode_scratch_bytes(cfg, big)[0] <= limit:
        big *= 2
    huge = B.gpt2_kv_view(FAKE + (1 << 30), big, 64, 0)
    assert lib.gpt2_decode_step_noalloc(h, ctypes.byref(huge), FAKE, FAKE, None) == B.GPT2_ERR_WORKSPACE
    assert "scratch" in lib.gpt2_last_error().decode()
