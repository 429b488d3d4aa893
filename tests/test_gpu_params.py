"""The library's own parameter conversion against the oracle's rounding set.

gpt2_init_params converts the fp32 blob on the device (its own kernels);
oracle.prepare_params rounds the stored matrices and embeddings to bf16 and
keeps biases and LayerNorm parameters fp32 (reading R10 of "bf16 weights").
Reading the device region back through gpt2_param_tensor must give exactly
the oracle's values, bit for bit, for every tensor of the key list (pwwt.cn
"逐行拆GPT-2源码", section on weights and architecture), and zero padding rows.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest

import oracle
import workloads as W

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gpt_pre_ln_amd import binding
    binding.load()


def _device_tensor(region: np.ndarray, t, bf16: bool) -> np.ndarray:
    """The stored copy of one tensor, widened to fp32, as [dev_rows, dev_ld]."""
    es = 2 if bf16 else 4
    raw = region[t.dev_offset:t.dev_offset + t.dev_rows * t.dev_ld * es]
    if bf16:
        f = (raw.view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    else:
        f = raw.view(np.float32)
    return f.reshape(t.dev_rows, t.dev_ld)


CASES = [
    ("bf16", True, W.ModelShape(vocab=1000, n_positions=128, d_model=128, n_head=2, n_layer=2, d_ff=512)),
    ("bf16", False, W.ModelShape(vocab=777, n_positions=300, d_model=192, n_head=3, n_layer=1, d_ff=256)),
    ("f32", True, W.ModelShape(vocab=300, n_positions=64, d_model=64, n_head=4, n_layer=2, d_ff=256)),
    ("bf16", True, W.SMALL),
]


@pytest.mark.parametrize("dtype,tied,shape", CASES, ids=["bf16-tied", "bf16-head", "f32", "bf16-gpt2-small"])
def test_device_parameters_equal_oracle_rounding(dtype, tied, shape):
    from gpt_pre_ln_amd import binding
    from gpt_pre_ln_amd.model import GPT2
    s = dataclasses.replace(shape, tie_word_embeddings=tied)
    _announce(f"param readback dtype={dtype} tied={tied} d_model={s.d_model} vocab={s.vocab}")
    blob = W.make_params(s, W.Init(w_std=0.2, proj_std=0.2, bias_std=0.1, gamma=(1.0, 0.2), beta=(0.0, 0.2)), 21)
    m = GPT2.from_shape(s, dtype, max_batch=1, max_seq=8)
    m.load_blob(blob)
    torch.cuda.synchronize()
    region = m.params.cpu().numpy()
    P = oracle.prepare_params(blob, s, dtype)
    keys = list(W.param_offsets(s))
    assert binding.gpt2_param_tensor_count(m.cfg) == len(keys)
    n_bf16 = 0
    for i, key in enumerate(keys):
        t = binding.gpt2_param_tensor(m.cfg, i)
        bf16 = t.dev_dtype == binding.GPT2_BF16
        n_bf16 += bf16
        dev = _device_tensor(region, t, bf16)
        stored = t.cols if t.transposed else t.rows
        body = dev[:stored].T if t.transposed else dev[:stored]
        want = P[key].astype(np.float32).reshape(t.rows, t.cols)
        assert np.array_equal(body.view(np.uint32), want.view(np.uint32)), key
        assert not dev[stored:].any(), f"{key}: padding rows not zero"
    # the rounded set has the size the key list fixes: every matrix and embedding
    assert n_bf16 == (0 if dtype == "f32" else 2 + 4 * s.n_layer + (0 if tied else 1))
