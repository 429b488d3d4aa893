"""GPU parity of greedy generation (gpt2_generate) through the C ABI.

The token choice is an integer decided in floating point, so it is checked
where both sides decide in the same precision and elsewhere by validity:
  * bit-exact against the arg-max (first maximum) of the fp32 logits of
    step-by-step gpt2_decode_step calls fed the same tokens (the same lm_head
    tile, hence the same fp32 accumulators);
  * against the oracle, teacher-forced on the GPU's own sequence: the fp32
    logits of those decode steps by the forward parity rule (normwise error,
    exact arg-max in fp32 mode, admissible arg-max in bf16 mode);
  * the closed-form model (greedy token after position p is pi(p)) exactly.
Every case prints its name before touching the GPU.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as W
from parity import assert_logits

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


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def _init(std=0.08):
    return W.Init(w_std=std, proj_std=std, bias_std=0.05, gamma=(1.0, 0.2), beta=(0.0, 0.2))


def _generate(m, prompt, n_steps, max_T):
    """Prefill all but the prompt's last token, then generate from it."""
    Bsz, Pn = prompt.shape
    kv = m.new_kv_cache(Bsz, max_T)
    if Pn > 1:
        m.forward(_dev(prompt[:, :-1]), logits=False, kv=kv)
    out = m.generate(kv, _dev(prompt[:, -1]), n_steps)
    assert kv.past_len == Pn - 1 + n_steps
    return out.cpu().numpy()


def _stepwise_logits(m, prompt, tokens, max_T):
    """fp32 logits [B, n, V] of decode steps fed prompt[-1], tokens[:, 0], ..."""
    Bsz, Pn = prompt.shape
    kv = m.new_kv_cache(Bsz, max_T)
    if Pn > 1:
        m.forward(_dev(prompt[:, :-1]), logits=False, kv=kv)
    feed = np.concatenate([prompt[:, -1:], tokens[:, :-1]], axis=1)
    steps = [m.decode_step(kv, _dev(feed[:, i])).cpu().numpy() for i in range(tokens.shape[1])]
    return np.stack(steps, axis=1)


def _check_against_oracle(P, prompt, tokens, gpu_logits, dtype, label):
    """Teacher-forced on the GPU's sequence: the oracle's logits of positions
    Pn-1 .. Pn+n-2 against the GPU's fp32 logits of the same steps, by the
    forward parity rule (normwise error and arg-max agreement)."""
    Pn, n = prompt.shape[1], tokens.shape[1]
    seq = np.concatenate([prompt, tokens[:, :-1]], axis=1)
    ref = oracle.forward(P, seq, positions=list(range(Pn - 1, Pn - 1 + n)))   # [B, n, V]
    rep = assert_logits(gpu_logits, ref, dtype, f"generate {label}")
    print(f"[generate] {label} normwise {rep['normwise']:.2e} exact {rep['exact_argmax']:.4f} "
          f"admissible {rep['admissible_argmax']:.4f}", flush=True)


CASES = [
    # dtype, d_model, n_head, n_layer, vocab, n_positions, B, prompt, steps
    ("f32", 64, 4, 2, 512, 64, 2, 5, 12),
    ("f32", 128, 2, 2, 1000, 256, 3, 1, 9),       # prompt of one token: no prefill
    ("bf16", 128, 2, 2, 777, 256, 5, 40, 16),
    ("bf16", 192, 3, 2, 4099, 300, 33, 20, 6),    # B = 33: the tiled lm_head (64x64), not 32x64
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_generate_matches_stepwise_and_oracle(case):
    from gpt_pre_ln_amd.model import GPT2
    dtype, D, H, L, V, P_, Bsz, Pn, n = case
    _announce(f"generate {case}")
    s = W.ModelShape(vocab=V, n_positions=P_, d_model=D, n_head=H, n_layer=L, d_ff=4 * D)
    blob = W.make_params(s, _init(0.3 if dtype == "f32" else 0.08), 500 + D + Pn)
    prompt = np.random.default_rng(V + Pn).integers(0, V, size=(Bsz, Pn)).astype(np.int32)
    max_T = Pn + n + 3
    m = GPT2.from_shape(s, dtype, max_batch=Bsz, max_seq=max(Pn, 1), logits_dtype="f32")
    m.load_blob(blob)
    tokens = _generate(m, prompt, n, max_T)
    assert tokens.shape == (Bsz, n) and tokens.min() >= 0 and tokens.max() < V
    lg = _stepwise_logits(m, prompt, tokens, max_T)
    np.testing.assert_array_equal(tokens, lg.argmax(axis=-1))
    _check_against_oracle(oracle.prepare_params(blob, s, dtype), prompt, tokens, lg, dtype, f"{case}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_generate_closed_form(dtype):
    """The model of the oracle pin: the greedy token after position p is pi(p)."""
    from gpt_pre_ln_amd.model import GPT2
    _announce(f"generate closed form {dtype}")
    V, D, NP = 48, 64, 32
    s = W.ModelShape(vocab=V, n_positions=NP, d_model=D, n_head=1, n_layer=2, d_ff=4 * D)
    blob = W.make_params(s, _init(0.2), 39)
    view = W.unpack(blob, s)
    for l in range(s.n_layer):
        for k in ("attn.c_proj.w", "attn.c_proj.b", "mlp.c_proj.w", "mlp.c_proj.b"):
            view[f"h.{l}.{k}"][...] = 0.0
    view["ln_f.w"][...] = 1.0
    view["ln_f.b"][...] = 0.0
    view["wte"][...] = 0.0
    view["wte"][np.arange(V), np.arange(V)] = 1.0
    pi = lambda t: (5 * t + 3) % V
    view["wpe"][...] = 0.0
    view["wpe"][np.arange(NP), [pi(t) for t in range(NP)]] = 3.0
    prompt = np.random.default_rng(40).integers(0, V, size=(2, 7)).astype(np.int32)
    m = GPT2.from_shape(s, dtype, max_batch=2, max_seq=7)
    m.load_blob(blob)
    tokens = _generate(m, prompt, 25, NP)
    np.testing.assert_array_equal(tokens, np.array([[pi(6 + i) for i in range(25)]] * 2))


def test_generate_gpt2_small_b32():
    """The decode workload's model and batch: a 960-token prompt, 64 greedy steps
    (positions 959 .. 1022).  All sequences bit-exact against step-by-step
    decode arg-max; sequence 0 teacher-forced against the oracle."""
    from gpt_pre_ln_amd.model import GPT2
    w = W.WORKLOADS["gpt2-small-decode-b32p1023"]
    Pn, n = 960, 64
    _announce(f"{w.name} generate prompt={Pn} steps={n}")
    blob = W.make_params(w)
    prefix, _ = W.make_decode_ids(w)
    prompt = np.ascontiguousarray(prefix[:, :Pn])
    m = GPT2.from_shape(w.shape, w.dtype, max_batch=w.batch, max_seq=Pn, logits_dtype="f32")
    m.load_blob(blob)
    tokens = _generate(m, prompt, n, Pn + n)
    lg = _stepwise_logits(m, prompt, tokens, Pn + n)
    np.testing.assert_array_equal(tokens, lg.argmax(axis=-1))
    del m
    P = oracle.prepare_params(blob, w.shape, w.dtype)
    _check_against_oracle(P, prompt[0:1], tokens[0:1], lg[0:1], w.dtype, f"{w.name} seq 0")
