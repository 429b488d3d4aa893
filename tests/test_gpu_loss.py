"""GPU parity of the fused next-token loss (gpt2_forward_loss) against the oracle.

Two bounds per case:
  * against the oracle's cross-entropy applied to the GPU's own fp32 logits
    (the loss GEMM and the logits GEMM use the same tile shape, so the fp32
    accumulators are identical and only the fp32 reduction differs): 1e-4
    absolute per position;
  * against the fp64 oracle: per position, log-sum-exp and the picked logit
    each move by at most that row's max|delta logit|, so the cross-entropy is
    2-Lipschitz in the row's max-norm: |loss_gpu - loss_oracle| <= OWN_TOL +
    2 * max_v |logit_gpu - logit_oracle| row by row (the GPU's own logits, in
    turn, within the logits tolerance of the oracle's).
Every case prints its name before touching the GPU.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
import workloads as W
from parity import TOL_F32, TOL_BF16, assert_logits

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
OWN_TOL = 1e-4


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


def _check(per_gpu, mean_gpu, own_logits, ref_logits, labels, dtype, label):
    mean_own, per_own = oracle.shifted_cross_entropy(own_logits, labels)
    mean_ref, per_ref = oracle.shifted_cross_entropy(ref_logits, labels)
    # the GPU's own logits against the oracle's, then the Lipschitz bound row by row
    assert_logits(own_logits, ref_logits, dtype, f"{label} logits")
    row_dev = np.abs(own_logits.astype(np.float64) - ref_logits).max(axis=-1)[:, :-1]  # positions scored
    bound = OWN_TOL + 2.0 * row_dev
    e_own = float(np.abs(per_gpu - per_own).max())
    excess = np.abs(per_gpu - per_ref) - bound
    print(f"[loss] {label} mean gpu {mean_gpu:.6f} oracle {mean_ref:.6f} | per-position max err: "
          f"own-logits {e_own:.2e} oracle {float(np.abs(per_gpu - per_ref).max()):.2e} "
          f"(row bounds {float(bound.min()):.2e}..{float(bound.max()):.2e})", flush=True)
    assert np.isfinite(per_gpu).all()
    assert e_own <= OWN_TOL, f"{label}: fused loss vs own logits {e_own:.3e}"
    assert (excess <= 0).all(), f"{label}: loss vs oracle beyond 2 max|d logit| by {float(excess.max()):.3e}"
    assert abs(mean_gpu - mean_own) <= OWN_TOL
    assert abs(mean_gpu - mean_ref) <= OWN_TOL + 2.0 * float(row_dev.max())


CASES = [
    # dtype, d_model, n_head, n_layer, vocab, n_positions, B, T, ignore   (lm_head tile in the comment)
    ("f32", 64, 4, 2, 512, 64, 1, 16, False),        # M = 16: 32x64
    ("f32", 64, 4, 2, 300, 64, 3, 37, True),         # M = 111: 128x128, vocab padded 300 -> 512
    ("bf16", 192, 3, 1, 777, 300, 2, 20, True),      # M = 40: 64x64
    ("bf16", 128, 2, 2, 1000, 256, 3, 200, False),   # M = 600: 128x128
    ("bf16", 256, 4, 3, 4099, 300, 2, 300, True),    # M = 600, ragged vocabulary
    ("bf16", 64, 1, 1, 50257, 1024, 3, 1000, True),  # M = 3000: 256x256 (GPT-2 vocabulary)
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_loss_matches_oracle(case):
    from gpt_pre_ln_amd.model import GPT2
    dtype, D, H, L, V, P_, B, T, ignore = case
    _announce(f"loss {case}")
    s = W.ModelShape(vocab=V, n_positions=P_, d_model=D, n_head=H, n_layer=L, d_ff=4 * D)
    blob = W.make_params(s, _init(), 300 + D + T)
    rng = np.random.default_rng(V + T)
    ids = rng.integers(0, V, size=(B, T)).astype(np.int32)
    labels = rng.integers(0, V, size=(B, T)).astype(np.int32)
    if ignore:
        labels[rng.random((B, T)) < 0.1] = -100
    m = GPT2.from_shape(s, dtype, max_batch=B, max_seq=T, logits_dtype="f32")
    m.load_blob(blob)
    mean, per = m.loss(_dev(ids), _dev(labels), token_loss=True)
    own = m.forward(_dev(ids))[0]
    torch.cuda.synchronize()
    per_gpu = per.cpu().numpy().astype(np.float64)
    own = own.cpu().numpy()
    ref = oracle.forward(oracle.prepare_params(blob, s, dtype), ids)
    _check(per_gpu, float(mean.item()), own, ref, labels, dtype, f"{case}")
    assert (per_gpu[labels[:, 1:] < 0] == 0).all()
    # labels default to the input ids
    mean_d, per_d = m.loss(_dev(ids), token_loss=True)
    _, per_ids = oracle.shifted_cross_entropy(own, ids)
    assert float(np.abs(per_d.cpu().numpy() - per_ids).max()) <= OWN_TOL


def test_loss_label_edge_cases():
    from gpt_pre_ln_amd.model import GPT2
    _announce("loss label edge cases")
    s = W.ModelShape(vocab=300, n_positions=64, d_model=64, n_head=1, n_layer=1, d_ff=256)
    blob = W.make_params(s, _init(), 41)
    ids = np.random.default_rng(42).integers(0, 300, size=(2, 9)).astype(np.int32)
    m = GPT2.from_shape(s, "bf16", max_batch=2, max_seq=9)
    m.load_blob(blob)
    # nothing scored: every position 0, mean NaN
    mean, per = m.loss(_dev(ids), _dev(np.full((2, 9), -100, np.int32)), token_loss=True)
    assert math.isnan(mean.item()) and (per.cpu().numpy() == 0).all()
    # a label outside the vocabulary poisons its position and the mean
    lab = ids.copy()
    lab[1, 4] = 300
    mean, per = m.loss(_dev(ids), _dev(lab), token_loss=True)
    per = per.cpu().numpy()
    assert math.isnan(mean.item()) and np.isnan(per[1, 3])
    assert np.isfinite(np.delete(per.reshape(-1), 8 + 3)).all()
    # T = 2: exactly one scored position per sequence
    mean, per = m.loss(_dev(ids[:, :2]), token_loss=True)
    assert per.shape == (2, 1) and abs(mean.item() - per.mean().item()) <= 1e-6


def test_gpt2_small_loss_b8t1024():
    """The benchmark workload: every position against the oracle cross-entropy
    of the GPU's own fp32 logits, and sequence 0 against the fp64 oracle."""
    from gpt_pre_ln_amd.model import GPT2
    w = W.WORKLOADS["gpt2-small-b8t1024"]
    _announce(f"{w.name} loss B={w.batch} T={w.seq_len}")
    blob = W.make_params(w)
    ids = W.make_ids(w)
    m = GPT2.from_shape(w.shape, w.dtype, max_batch=w.batch, max_seq=w.seq_len, logits_dtype="f32")
    m.load_blob(blob)
    mean, per = m.loss(_dev(ids), token_loss=True)
    own = m.forward(_dev(ids))[0]
    torch.cuda.synchronize()
    per_gpu = per.cpu().numpy().astype(np.float64)
    own = own.cpu().numpy()
    del m
    mean_own, per_own = oracle.shifted_cross_entropy(own, ids)
    e_own = float(np.abs(per_gpu - per_own).max())
    print(f"[loss] {w.name} mean gpu {mean.item():.6f} own-logits {mean_own:.6f} max err {e_own:.2e}", flush=True)
    assert e_own <= OWN_TOL and abs(mean.item() - mean_own) <= OWN_TOL
    P = oracle.prepare_params(blob, w.shape, w.dtype)
    ref0 = oracle.forward(P, ids[0:1])
    assert_logits(own[0], ref0[0], w.dtype, f"{w.name} seq 0 fp32 logits")
    _check(per_gpu[0:1], float(per_gpu[0].mean()), own[0:1], ref0, ids[0:1], w.dtype, f"{w.name} seq 0")
