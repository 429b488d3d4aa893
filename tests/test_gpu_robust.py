"""Robustness of every entry point on the GPU, on paths whose parity is tested
elsewhere: canary-guarded outputs (nothing is written outside what the header
documents), run-twice bitwise determinism, and the token-id check flag with
valid ids.  Ragged shapes, fp32 and bf16."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import workloads as W

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
GUARD = 4096          # bytes of canary on each side of an output (a multiple of 256)
CANARY = 0xA5


def _announce(msg):
    print(f"\n[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gpt_pre_ln_amd import binding
    binding.load()


class Guarded:
    """nbytes of output inside a buffer filled with the canary byte, GUARD bytes
    of canary before and after it."""

    def __init__(self, nbytes: int):
        self.n = nbytes
        self.buf = torch.full((nbytes + 2 * GUARD,), CANARY, dtype=torch.uint8, device=DEV)

    @property
    def ptr(self) -> int:
        return self.buf.data_ptr() + GUARD

    def view(self, dtype, shape):
        return self.buf[GUARD:GUARD + self.n].view(dtype).view(shape)

    def check(self, what: str, untouched_inner: np.ndarray | None = None):
        """Guards unchanged; untouched_inner: byte mask over the output that must
        still hold the canary."""
        h = self.buf.cpu().numpy()
        assert (h[:GUARD] == CANARY).all(), f"{what}: written before the output"
        assert (h[GUARD + self.n:] == CANARY).all(), f"{what}: written after the output"
        if untouched_inner is not None:
            inner = h[GUARD:GUARD + self.n]
            assert (inner[untouched_inner] == CANARY).all(), f"{what}: written inside a region it must not touch"


SHAPES = [
    ("f32", W.ModelShape(vocab=300, n_positions=64, d_model=64, n_head=4, n_layer=2, d_ff=256), 3, 37),
    ("bf16", W.ModelShape(vocab=777, n_positions=300, d_model=192, n_head=3, n_layer=2, d_ff=256), 2, 129),
]
IDS = ["f32-d64-B3T37", "bf16-d192-B2T129"]


def _model(dtype, s, B, T):
    from gpt_pre_ln_amd.model import GPT2
    blob = W.make_params(s, W.Init(w_std=0.2, proj_std=0.2, bias_std=0.05, gamma=(1.0, 0.2), beta=(0.0, 0.2)), 31)
    m = GPT2.from_shape(s, dtype, max_batch=B, max_seq=T)
    m.load_blob(blob)
    return m


def _ids(B, T, V, seed=3):
    ids = np.random.default_rng(seed).integers(0, V, size=(B, T)).astype(np.int32)
    ids[0, 0], ids[-1, -1] = 0, V - 1          # both ends of the vocabulary
    return torch.from_numpy(ids).to(DEV)


def _stream():
    return torch.cuda.current_stream().cuda_stream


@pytest.mark.parametrize("dtype,s,B,T", SHAPES, ids=IDS)
def test_forward_outputs_stay_in_bounds(dtype, s, B, T):
    from gpt_pre_ln_amd import binding
    _announce(f"canary forward {dtype} d={s.d_model} V={s.vocab} B={B} T={T}")
    m = _model(dtype, s, B, T)
    ids = _ids(B, T, s.vocab)
    V, Vp, M = s.vocab, m.logits_padded_ld, B * T
    es = 2 if m.cfg.logits_dtype == binding.GPT2_BF16 else 4
    ref = None
    for ld in (V, V + 5, Vp + 40):
        lg = Guarded(M * ld * es)
        hd = Guarded(M * s.d_model * 4)
        binding.gpt2_forward_strided(m.handle, ids.data_ptr(), B, T, lg.ptr, ld, hd.ptr, None, _stream())
        torch.cuda.synchronize()
        cols = np.arange(ld)
        untouched = (cols >= V) if ld < Vp else (cols >= Vp)
        lg.check(f"logits ld={ld}", np.repeat(np.tile(untouched, M), es))
        hd.check("hidden")
        out = lg.view(torch.uint8, (M, ld * es)).cpu().numpy()
        if ld >= Vp:     # the padding columns receive the zero logits of the zero rows of wte
            assert not out[:, V * es:Vp * es].any()
        body = out[:, :V * es].copy()
        if ref is None:
            ref = body
        assert np.array_equal(body, ref), f"logits at ld={ld} differ from ld={V}"


@pytest.mark.parametrize("dtype,s,B,T", SHAPES, ids=IDS)
def test_kv_cache_decode_and_generation_stay_in_bounds(dtype, s, B, T):
    from gpt_pre_ln_amd import binding
    _announce(f"canary kv/decode/generate {dtype} d={s.d_model} V={s.vocab} B={B} T={T}")
    m = _model(dtype, s, B, T)
    T0, max_T, n_gen = T - 8, T - 2, 3
    S = binding.gpt2_kv_stride(m.cfg, max_T)
    H, hs, L = s.n_head, s.d_model // s.n_head, s.n_layer
    el = 2 if dtype == "bf16" else 4
    kv = Guarded(binding.gpt2_kv_cache_bytes(m.cfg, B, max_T))
    assert kv.n == L * 2 * B * S * s.d_model * el
    view = binding.gpt2_kv_view(kv.ptr, B, max_T, 0)

    def untouched_after(last):          # byte mask: cache slots > last never written
        slot_k = np.broadcast_to(np.arange(S)[None, None, :, None], (B, H, S, hs))
        slot_v = np.broadcast_to(np.arange(S)[None, None, None, :], (B, H, hs, S))
        layer = np.concatenate([slot_k.ravel(), slot_v.ravel()]) > last
        return np.repeat(np.tile(layer, L), el)

    ids = _ids(B, T, s.vocab)
    prefix = ids[:, :T0].contiguous()
    binding.gpt2_forward(m.handle, prefix.data_ptr(), B, T0, None, None, view, _stream())
    torch.cuda.synchronize()
    assert view.past_len == T0
    kv.check("prefill", untouched_after(T0 - 1))

    les = 2 if m.cfg.logits_dtype == binding.GPT2_BF16 else 4
    lg = Guarded(B * s.vocab * les)
    new = ids[:, T0].contiguous()
    binding.gpt2_decode_step(m.handle, view, new.data_ptr(), lg.ptr, _stream())
    torch.cuda.synchronize()
    assert view.past_len == T0 + 1
    kv.check("decode", untouched_after(T0))
    lg.check("decode logits")

    out = Guarded(B * n_gen * 4)
    first = ids[:, T0 + 1].contiguous()
    binding.gpt2_generate(m.handle, view, first.data_ptr(), n_gen, out.ptr, _stream())
    torch.cuda.synchronize()
    assert view.past_len == T0 + 1 + n_gen
    kv.check("generate", untouched_after(T0 + n_gen))
    out.check("generated tokens")
    toks = out.view(torch.int32, (B, n_gen)).cpu().numpy()
    assert ((toks >= 0) & (toks < s.vocab)).all()


@pytest.mark.parametrize("dtype,s,B,T", SHAPES, ids=IDS)
def test_loss_and_backward_outputs_stay_in_bounds(dtype, s, B, T):
    from gpt_pre_ln_amd import binding
    _announce(f"canary loss/backward {dtype} d={s.d_model} V={s.vocab} B={B} T={T}")
    m = _model(dtype, s, B, T)
    ids = _ids(B, T, s.vocab)
    per = Guarded(B * (T - 1) * 4)
    mean = Guarded(4)
    binding.gpt2_forward_loss(m.handle, ids.data_ptr(), None, B, T, per.ptr, mean.ptr, _stream())
    torch.cuda.synchronize()
    per.check("token losses")
    mean.check("mean loss")
    assert np.isfinite(per.view(torch.float32, (B, T - 1)).cpu().numpy()).all()

    gen = torch.Generator(device=DEV)
    gen.manual_seed(5)
    x = torch.randn((B, T, s.d_model), generator=gen, device=DEV)
    dy = torch.randn((B, T, s.d_model), generator=gen, device=DEV)
    dx = Guarded(B * T * s.d_model * 4)
    grads = Guarded(m.layer_param_count() * 4)
    wsb = binding.gpt2_block_backward_workspace_bytes(m.cfg, B, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    binding.gpt2_block_backward(m.handle, 1, B, T, x.data_ptr(), dy.data_ptr(), dx.ptr, grads.ptr, ws.data_ptr(),
                                wsb, _stream())
    torch.cuda.synchronize()
    dx.check("block backward dx")
    grads.check("block backward gradients")


@pytest.mark.parametrize("dtype,s,B,T", SHAPES, ids=IDS)
def test_run_twice_bitwise(dtype, s, B, T):
    """Same inputs, same bits: forward logits and hidden, the loss, the block
    backward and a decode step (no atomics anywhere; every reduction has a
    fixed order)."""
    _announce(f"determinism {dtype} d={s.d_model} V={s.vocab} B={B} T={T}")
    m = _model(dtype, s, B, T)
    ids = _ids(B, T, s.vocab)

    def fwd():
        lg, hd = m.forward(ids, hidden=True)
        return lg.cpu().clone(), hd.cpu().clone()

    def loss():
        mean, per = m.loss(ids, token_loss=True)
        return mean.cpu().clone(), per.cpu().clone()

    gen = torch.Generator(device=DEV)
    gen.manual_seed(9)
    x = torch.randn((B, T, s.d_model), generator=gen, device=DEV)
    dy = torch.randn((B, T, s.d_model), generator=gen, device=DEV)

    def bwd():
        dx, g = m.block_backward(0, x, dy)
        return dx.cpu().clone(), g.cpu().clone()

    kv = m.new_kv_cache(B, T)
    m.forward(ids[:, :T - 1].contiguous(), logits=False, kv=kv)
    new = ids[:, T - 1].contiguous()

    def dec():
        kv.view.past_len = T - 1
        return (m.decode_step(kv, new).cpu().clone(),)

    for f in (fwd, loss, bwd, dec):
        a, b = f(), f()
        for u, v in zip(a, b):
            assert torch.equal(u.view(torch.uint8) if u.dtype == torch.bfloat16 else u,
                               v.view(torch.uint8) if v.dtype == torch.bfloat16 else v), f.__name__


@pytest.mark.parametrize("dtype,s,B,T", SHAPES, ids=IDS)
def test_id_check_flag_stays_clear_for_valid_ids(dtype, s, B, T):
    """With the check on, valid ids (both ends of the vocabulary included) leave
    the flag at 0 and change nothing in the outputs."""
    from gpt_pre_ln_amd import binding
    _announce(f"id check {dtype} d={s.d_model} V={s.vocab} B={B} T={T}")
    m = _model(dtype, s, B, T)
    ids = _ids(B, T, s.vocab)
    ref, _ = m.forward(ids)
    ref = ref.cpu().clone()
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    binding.gpt2_set_id_check(m.handle, flag.data_ptr())
    try:
        lg, _ = m.forward(ids)
        m.loss(ids)
        kv = m.new_kv_cache(B, T)
        m.forward(ids[:, :T - 1].contiguous(), logits=False, kv=kv)
        m.decode_step(kv, ids[:, T - 1].contiguous())
        torch.cuda.synchronize()
        assert int(flag.item()) == 0
        assert torch.equal(lg.cpu().view(torch.uint8) if lg.dtype == torch.bfloat16 else lg.cpu(),
                           ref.view(torch.uint8) if ref.dtype == torch.bfloat16 else ref)
    finally:
        binding.gpt2_set_id_check(m.handle, None)
