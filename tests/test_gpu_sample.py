"""GPU parity of sampled generation (gpt2_generate_sample) through the C ABI.

The drawn token is an integer decided in floating point (fp32 Gumbel noise on
the lm_head's fp32 accumulators against the oracle's fp64 noise on fp64
logits), so it is checked by validity and by distribution:
  * temperature 0 is the greedy gpt2_generate, bit for bit;
  * teacher-forced on the GPU's own sequence, each token must be admissible
    under the oracle's perturbed scores (logit / temperature + G): within the
    logits tolerance / temperature of the oracle's best score; the exact
    agreement is reported (fp32: expected ~100 %);
  * over many independent rows the GPU's draws follow softmax(logits /
    temperature) of the oracle's logits (chi-square), which pins the GPU
    sampler to the mathematics, not to the oracle's code;
  * the same seed reproduces the same tokens, another seed changes them.
Every case prints its name before touching the GPU.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as W
from parity import TOL_BF16, TOL_F32

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


def _sample(m, prompt, n_steps, max_T, temperature, seed):
    """Prefill all but the prompt's last token, then sample from it."""
    Bsz, Pn = prompt.shape
    kv = m.new_kv_cache(Bsz, max_T)
    if Pn > 1:
        m.forward(_dev(prompt[:, :-1]), logits=False, kv=kv)
    out = m.generate_sample(kv, _dev(prompt[:, -1]), n_steps, temperature, seed)
    assert kv.past_len == Pn - 1 + n_steps
    return out.cpu().numpy()


def _admissible(P, prompt, tokens, temperature, seed, tol_rel, rows):
    """Teacher-forced on the GPU's sequence: (exact, admissible) agreement of
    the GPU's tokens with the oracle's draws for the given rows."""
    Pn, n = prompt.shape[1], tokens.shape[1]
    seq = np.concatenate([prompt, tokens[:, :-1]], axis=1)
    exact = adm = total = 0
    for b in rows:
        logits = oracle.forward(P, seq[b:b + 1], positions=list(range(Pn - 1, Pn - 1 + n)))[0]   # [n, V]
        tol = tol_rel * np.abs(logits).max() / temperature + 1e-4
        for i in range(n):
            best, scores = oracle.sample_token(logits[i], temperature, seed, Pn - 1 + i, b)
            g = int(tokens[b, i])
            exact += g == best
            adm += scores[best] - scores[g] <= tol
            total += 1
    return exact / total, adm / total


def _init(std):
    return W.Init(w_std=std, proj_std=std, bias_std=0.05, gamma=(1.0, 0.2), beta=(0.0, 0.2))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_temperature_zero_is_greedy(dtype):
    from gpt_pre_ln_amd.model import GPT2
    _announce(f"sample temperature 0 == greedy {dtype}")
    s = W.ModelShape(vocab=777, n_positions=128, d_model=128, n_head=2, n_layer=2, d_ff=512)
    m = GPT2.from_shape(s, dtype, max_batch=3, max_seq=20)
    m.load_blob(W.make_params(s, _init(0.1), 61))
    prompt = np.random.default_rng(62).integers(0, s.vocab, size=(3, 20)).astype(np.int32)
    a = _sample(m, prompt, 7, 40, 0.0, 5)
    kv = m.new_kv_cache(3, 40)
    m.forward(_dev(prompt[:, :-1]), logits=False, kv=kv)
    g = m.generate(kv, _dev(prompt[:, -1]), 7).cpu().numpy()
    np.testing.assert_array_equal(a, g)


CASES = [
    # dtype, d_model, n_head, n_layer, vocab, n_positions, B, prompt, steps, temperature
    ("f32", 64, 4, 2, 512, 64, 3, 6, 10, 1.0),
    ("f32", 128, 2, 2, 1000, 256, 2, 1, 8, 0.7),
    ("bf16", 128, 2, 2, 777, 256, 5, 40, 12, 1.3),
    ("bf16", 192, 3, 2, 4099, 300, 33, 20, 5, 0.9),   # B = 33: the 64x64 lm_head tile
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_sample_admissible_against_oracle(case):
    from gpt_pre_ln_amd.model import GPT2
    dtype, D, H, L, V, P_, Bsz, Pn, n, temp = case
    _announce(f"sample {case}")
    s = W.ModelShape(vocab=V, n_positions=P_, d_model=D, n_head=H, n_layer=L, d_ff=4 * D)
    blob = W.make_params(s, _init(0.3 if dtype == "f32" else 0.08), 700 + D + Pn)
    prompt = np.random.default_rng(V + Pn + 1).integers(0, V, size=(Bsz, Pn)).astype(np.int32)
    max_T = Pn + n + 2
    m = GPT2.from_shape(s, dtype, max_batch=Bsz, max_seq=max(Pn, 1))
    m.load_blob(blob)
    seed = 1234 + D
    tokens = _sample(m, prompt, n, max_T, temp, seed)
    assert tokens.min() >= 0 and tokens.max() < V
    np.testing.assert_array_equal(tokens, _sample(m, prompt, n, max_T, temp, seed))   # reproducible
    assert (tokens != _sample(m, prompt, n, max_T, temp, seed + 1)).any()             # seed matters
    P = oracle.prepare_params(blob, s, dtype)
    rows = range(min(Bsz, 6))
    exact, adm = _admissible(P, prompt, tokens, temp, seed, TOL_F32 if dtype == "f32" else TOL_BF16, rows)
    print(f"[sample] {case} exact {exact:.4f} admissible {adm:.4f}", flush=True)
    assert adm == 1.0
    if dtype == "f32":
        assert exact >= 0.99


@pytest.mark.parametrize("temperature", [0.6, 1.0])
def test_sample_distribution_is_softmax(temperature):
    """512 identical sequences per call draw independent tokens (the noise is
    keyed by row): four calls with four seeds give 2,048 draws from
    softmax(logits / temperature) of the last position (chi-square)."""
    from scipy import stats
    from gpt_pre_ln_amd.model import GPT2
    _announce(f"sample distribution temperature={temperature}")
    s = W.ModelShape(vocab=16, n_positions=32, d_model=64, n_head=4, n_layer=1, d_ff=256)
    blob = W.make_params(s, W.Init(w_std=0.15, proj_std=0.15, bias_std=0.05, gamma=(1.0, 0.1),
                                   beta=(0.0, 0.1)), 71)
    Bsz, Pn = 512, 6
    prompt1 = np.random.default_rng(72).integers(0, s.vocab, size=(1, Pn)).astype(np.int32)
    prompt = np.repeat(prompt1, Bsz, axis=0)
    m = GPT2.from_shape(s, "f32", max_batch=Bsz, max_seq=Pn)
    m.load_blob(blob)
    draws = np.concatenate([_sample(m, prompt, 1, Pn + 1, temperature, sd)[:, 0] for sd in (1, 2, 3, 4)])
    P = oracle.prepare_params(blob, s, "f32")
    logits = oracle.forward(P, prompt1, positions=[Pn - 1])[0, 0]
    z = logits / temperature
    p = np.exp(z - z.max())
    p /= p.sum()
    counts = np.bincount(draws, minlength=s.vocab).astype(np.float64)
    expected = p * len(draws)
    big = expected >= 5
    obs = np.append(counts[big], counts[~big].sum())
    exp_ = np.append(expected[big], expected[~big].sum())
    if exp_[-1] == 0:
        obs, exp_ = obs[:-1], exp_[:-1]
    pval = stats.chisquare(obs, exp_).pvalue
    print(f"[sample] distribution T={temperature}: {int(big.sum())} bins, chi-square p = {pval:.3g}", flush=True)
    assert pval > 1e-4


def test_sample_gpt2_small_b32():
    """The decode workload's model and batch: a 960-token prompt, 16 sampled
    steps at temperature 0.8; sequences 0 and 1 teacher-forced against the
    oracle's draws (admissible under the bf16 logits tolerance)."""
    from gpt_pre_ln_amd.model import GPT2
    w = W.WORKLOADS["gpt2-small-decode-b32p1023"]
    Pn, n, temp, seed = 960, 16, 0.8, 2024
    _announce(f"{w.name} sample prompt={Pn} steps={n}")
    blob = W.make_params(w)
    prefix, _ = W.make_decode_ids(w)
    prompt = np.ascontiguousarray(prefix[:, :Pn])
    m = GPT2.from_shape(w.shape, w.dtype, max_batch=w.batch, max_seq=Pn)
    m.load_blob(blob)
    tokens = _sample(m, prompt, n, Pn + n, temp, seed)
    del m
    P = oracle.prepare_params(blob, w.shape, w.dtype)
    exact, adm = _admissible(P, prompt, tokens, temp, seed, TOL_BF16, [0, 1])
    print(f"[sample] {w.name} exact {exact:.4f} admissible {adm:.4f}", flush=True)
    assert adm == 1.0
