"""Device-buffer owner around the C ABI.

PyTorch allocates the parameter region, workspace, KV caches and outputs and
supplies the stream; every computation is a call into libgpt2.so.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B


class KVCache:
    """A key/value cache in a torch-owned device buffer plus its C view."""

    def __init__(self, cfg, batch: int, max_T: int, device):
        nbytes = B.gpt2_kv_cache_bytes(cfg, batch, max_T)
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.view = B.gpt2_kv_view(self.buf.data_ptr(), batch, max_T, 0)

    @property
    def past_len(self) -> int:
        return self.view.past_len


class GPT2:
    def __init__(self, vocab_size, n_positions, d_model, n_head, n_layer, d_ff, dtype="bf16",
                 max_batch=1, max_seq=None, ln_eps=1e-5, device="cuda:0", logits_dtype=None,
                 activation="gelu_new", scale_attn_by_inverse_layer_idx=False, post_ln=False,
                 tie_word_embeddings=True):
        """logits_dtype: "f32" or "bf16" element type of the logits (default: dtype).
        The remaining switches select the model variants (defaults: GPT-2)."""
        self.device = torch.device(device)
        self.cfg = B.make_config(vocab_size, n_positions, d_model, n_head, n_layer, d_ff, ln_eps, dtype,
                                 logits_dtype, activation, scale_attn_by_inverse_layer_idx, post_ln,
                                 tie_word_embeddings)
        self.dtype = dtype
        self.logits_torch_dtype = torch.bfloat16 if self.cfg.logits_dtype == B.GPT2_BF16 else torch.float32
        max_seq = max_seq or n_positions
        self.param_bytes = B.gpt2_param_bytes(self.cfg)
        self.ws_bytes = max(B.gpt2_workspace_bytes(self.cfg, max_batch, max_seq),
                            B.gpt2_workspace_bytes(self.cfg, max_batch, 1))
        self.params = torch.empty(self.param_bytes, dtype=torch.uint8, device=self.device)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        self.handle = B.gpt2_create(self.cfg, self.params.data_ptr(), self.param_bytes,
                                    self.ws.data_ptr(), self.ws_bytes)
        self._destroy = B.load().gpt2_destroy  # held so that teardown at interpreter exit still works

    @classmethod
    def from_shape(cls, shape, dtype, **kw):
        return cls(shape.vocab, shape.n_positions, shape.d_model, shape.n_head, shape.n_layer,
                   shape.d_ff, dtype=dtype, ln_eps=shape.ln_eps, activation=shape.activation,
                   scale_attn_by_inverse_layer_idx=shape.scale_attn_by_inverse_layer_idx,
                   post_ln=shape.post_ln, tie_word_embeddings=shape.tie_word_embeddings, **kw)

    def __del__(self):
        h = getattr(self, "handle", None)
        destroy = getattr(self, "_destroy", None)
        if h is not None and destroy is not None:
            destroy(h)
            self.handle = None

    @property
    def stream(self) -> int:
        return torch.cuda.current_stream(self.device).cuda_stream

    def load_blob(self, blob) -> None:
        """Convert an fp32 parameter blob (numpy or torch) into the device layout."""
        n = B.gpt2_param_blob_floats(self.cfg)
        if isinstance(blob, np.ndarray):
            d_blob = torch.from_numpy(np.ascontiguousarray(blob, dtype=np.float32)).to(self.device)
        else:
            d_blob = blob.to(self.device, torch.float32).contiguous()
        if d_blob.numel() != n:
            raise ValueError(f"blob has {d_blob.numel()} floats, the config needs {n}")
        B.gpt2_init_params(self.handle, d_blob.data_ptr(), n, self.stream)
        torch.cuda.current_stream(self.device).synchronize()
        del d_blob

    def _logits_out(self, shape, out):
        if out is None:
            return torch.empty(shape, dtype=self.logits_torch_dtype, device=self.device)
        if out.dtype != self.logits_torch_dtype or tuple(out.shape) != tuple(shape) or not out.is_contiguous() \
                or out.device != self.device:
            raise ValueError(f"out_logits must be a contiguous {self.logits_torch_dtype} tensor of shape {shape} "
                             f"on {self.device}")
        return out

    @property
    def logits_padded_ld(self) -> int:
        """Row stride of the padded logits layout (gpt2_logits_padded_ld)."""
        return B.gpt2_logits_padded_ld(self.cfg)

    def forward(self, ids: torch.Tensor, logits: bool = True, hidden: bool = False, kv: KVCache | None = None,
                out_logits: torch.Tensor | None = None, padded_logits: bool = False):
        """ids: int32 [B, T] on the device.
        Returns (logits [B,T,V] of logits_dtype | None, hidden [B,T,D] fp32 | None).

        padded_logits: the logits live in rows of logits_padded_ld elements
        (gpt2_forward_strided, the faster layout); the result is the [B,T,V]
        view of that buffer, and out_logits, when given, is the [B,T,ld] buffer."""
        assert ids.dtype == torch.int32 and ids.is_contiguous() and ids.device == self.device
        Bsz, T = ids.shape
        V = self.cfg.vocab_size
        ld = self.logits_padded_ld if padded_logits else V
        buf = None
        if logits:
            buf = self._logits_out((Bsz, T, ld), out_logits)
        hd = torch.empty((Bsz, T, self.cfg.d_model), dtype=torch.float32, device=self.device) if hidden else None
        B.gpt2_forward_strided(self.handle, ids.data_ptr(), Bsz, T, buf.data_ptr() if buf is not None else None, ld,
                               hd.data_ptr() if hd is not None else None, kv.view if kv is not None else None,
                               self.stream)
        lg = buf[..., :V] if buf is not None and ld != V else buf
        return lg, hd

    def loss(self, ids: torch.Tensor, labels: torch.Tensor | None = None, token_loss: bool = False,
             out_mean: torch.Tensor | None = None):
        """Shifted next-token cross-entropy (gpt2_forward_loss).

        ids, labels: int32 [B, T] on the device (labels default to ids; negative
        labels are not scored).  Returns (mean fp32 [1], per-position fp32
        [B, T-1] | None).  No logits are materialised."""
        assert ids.dtype == torch.int32 and ids.is_contiguous() and ids.device == self.device
        if labels is not None:
            assert labels.dtype == torch.int32 and labels.is_contiguous() and labels.shape == ids.shape
            assert labels.device == self.device
        Bsz, T = ids.shape
        mean = out_mean if out_mean is not None else torch.empty(1, dtype=torch.float32, device=self.device)
        per = torch.empty((Bsz, T - 1), dtype=torch.float32, device=self.device) if token_loss else None
        B.gpt2_forward_loss(self.handle, ids.data_ptr(), labels.data_ptr() if labels is not None else None, Bsz, T,
                            per.data_ptr() if per is not None else None, mean.data_ptr(), self.stream)
        return mean, per

    def new_kv_cache(self, batch: int, max_T: int) -> KVCache:
        return KVCache(self.cfg, batch, max_T, self.device)

    def decode_step(self, kv: KVCache, new_ids: torch.Tensor, out_logits: torch.Tensor | None = None):
        """new_ids: int32 [B] on the device. Returns logits [B, V] of logits_dtype."""
        assert new_ids.dtype == torch.int32 and new_ids.is_contiguous()
        lg = self._logits_out((kv.view.B, self.cfg.vocab_size), out_logits)
        B.gpt2_decode_step(self.handle, kv.view, new_ids.data_ptr(), lg.data_ptr(), self.stream)
        return lg

    def generate(self, kv: KVCache, first_ids: torch.Tensor, n_steps: int, out: torch.Tensor | None = None):
        """Greedy generation (gpt2_generate): first_ids int32 [B] at position
        kv.past_len; returns int32 [B, n_steps], column i the token chosen at step i."""
        assert first_ids.dtype == torch.int32 and first_ids.is_contiguous() and first_ids.device == self.device
        Bsz = kv.view.B
        if out is None:
            out = torch.empty((Bsz, n_steps), dtype=torch.int32, device=self.device)
        assert out.dtype == torch.int32 and out.is_contiguous() and tuple(out.shape) == (Bsz, n_steps)
        B.gpt2_generate(self.handle, kv.view, first_ids.data_ptr(), n_steps, out.data_ptr(), self.stream)
        return out

    def generate_sample(self, kv: KVCache, first_ids: torch.Tensor, n_steps: int, temperature: float = 1.0,
                        seed: int = 0, out: torch.Tensor | None = None):
        """Sampled generation (gpt2_generate_sample): each step draws from
        softmax(logits / temperature); reproducible from (seed, position, row)."""
        assert first_ids.dtype == torch.int32 and first_ids.is_contiguous() and first_ids.device == self.device
        Bsz = kv.view.B
        if out is None:
            out = torch.empty((Bsz, n_steps), dtype=torch.int32, device=self.device)
        assert out.dtype == torch.int32 and out.is_contiguous() and tuple(out.shape) == (Bsz, n_steps)
        B.gpt2_generate_sample(self.handle, kv.view, first_ids.data_ptr(), n_steps, float(temperature),
                               int(seed) & ((1 << 64) - 1), out.data_ptr(), self.stream)
        return out

    def layer_param_count(self) -> int:
        D, F = self.cfg.d_model, self.cfg.d_ff
        return 2 * D + (3 * D * D + 3 * D) + (D * D + D) + 2 * D + (D * F + F) + (F * D + D)

    def block_backward(self, layer: int, x: torch.Tensor, dy: torch.Tensor, out_dx: torch.Tensor | None = None,
                       out_grads: torch.Tensor | None = None):
        """Backward of block `layer` (gpt2_block_backward): x, dy fp32 [B, T, D]
        on the device.  Returns (dx fp32 [B, T, D], grads fp32 [layer parameters]
        in blob order).  The backward workspace is allocated here, outside the
        library, and kept for calls of the same or a smaller size."""
        assert x.dtype == torch.float32 and dy.dtype == torch.float32 and x.shape == dy.shape
        assert x.is_contiguous() and dy.is_contiguous()
        Bsz, T, _ = x.shape
        need = B.gpt2_block_backward_workspace_bytes(self.cfg, Bsz, T)
        if getattr(self, "_bwd_ws", None) is None or self._bwd_ws.numel() < need:
            self._bwd_ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        dx = out_dx if out_dx is not None else torch.empty_like(x)
        grads = out_grads if out_grads is not None else torch.empty(self.layer_param_count(), dtype=torch.float32,
                                                                   device=self.device)
        B.gpt2_block_backward(self.handle, layer, Bsz, T, x.data_ptr(), dy.data_ptr(), dx.data_ptr(), grads.data_ptr(),
                              self._bwd_ws.data_ptr(), self._bwd_ws.numel(), self.stream)
        return dx, grads

    def set_trace(self, trace: torch.Tensor | None):
        B.gpt2_set_trace(self.handle, trace.data_ptr() if trace is not None else None,
                         trace.numel() if trace is not None else 0)
