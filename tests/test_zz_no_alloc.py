"""gpt2_decode_step_noalloc (the decode step on the library's per-device
scratch array, for callers that cannot allocate) against gpt2_decode_step on
the handle's workspace: two calls in a row, the second with fewer sequences,
each compared with the workspace path on the same inputs and caches.  Same
kernels, so the logits and the appended cache slots agree bit for bit (the
parity bar of the decode step is met a fortiori)."""
from __future__ import annotations

import numpy as np
import pytest

import workloads as W

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


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("dtype,shape,batches,prefix", [
    ("bf16", W.SMALL, (32, 5), 300),
    ("f32", W.ModelShape(vocab=300, n_positions=64, d_model=64, n_head=4, n_layer=2, d_ff=256), (7, 3), 40),
], ids=["bf16-gpt2-small", "f32-tiny"])
def test_noalloc_decode_matches_workspace_decode(dtype, shape, batches, prefix):
    from gpt_pre_ln_amd import binding
    from gpt_pre_ln_amd.model import GPT2
    blob = W.make_params(shape, W.Init(w_std=0.02, proj_std=0.02 / np.sqrt(2 * shape.n_layer), bias_std=0.01,
                                       gamma=(1.0, 0.05), beta=(0.0, 0.02)), 41)
    m = GPT2.from_shape(shape, dtype, max_batch=max(batches), max_seq=prefix + 1)
    m.load_blob(blob)
    stream = torch.cuda.current_stream().cuda_stream
    need, limit = binding.gpt2_decode_scratch_bytes(m.cfg, max(batches))
    assert need <= limit
    for call, B in enumerate(batches):
        _announce(f"noalloc decode call {call} dtype={dtype} d_model={shape.d_model} B={B} prefix={prefix}")
        rng = np.random.default_rng(100 + call)
        ids = torch.from_numpy(rng.integers(0, shape.vocab, size=(B, prefix + 1)).astype(np.int32)).to(DEV)
        kv_ws, kv_na = m.new_kv_cache(B, prefix + 1), m.new_kv_cache(B, prefix + 1)
        kv_ws.buf.zero_()          # slots the calls never write compare equal
        kv_na.buf.zero_()
        m.forward(ids[:, :prefix].contiguous(), logits=False, kv=kv_ws)
        m.forward(ids[:, :prefix].contiguous(), logits=False, kv=kv_na)
        new = ids[:, prefix].contiguous()
        ref = m.decode_step(kv_ws, new)
        got = torch.empty_like(ref)
        binding.gpt2_decode_step_noalloc(m.handle, kv_na.view, new.data_ptr(), got.data_ptr(), stream)
        torch.cuda.synchronize()
        assert kv_na.view.past_len == kv_ws.view.past_len == prefix + 1
        assert torch.equal(_bits(got), _bits(ref)), f"call {call}: logits differ"
        assert torch.equal(kv_na.buf, kv_ws.buf), f"call {call}: caches differ"
        assert torch.isfinite(got.float()).all()
