"""Seeded synthetic workloads for the GPT-2 Pre-LN forward: shapes, init recipe, inputs.

This module only *draws numbers*; it holds none of the model's arithmetic. Both
the HIP path (through its Python binding) and the fp64 oracle are fed from it,
so that they see bit-identical parameters and token ids.

Shapes and the init recipe follow the pages:
  * GPT2Config fields and the default GPT-2 small shape (vocab 50257, 1024
    positions, d_model 768, 12 heads, 12 layers, eps 1e-5, initializer_range
    0.02) -- pwwt.cn "逐行拆GPT-2源码", section GPT2Config.
  * c_proj weights (attention and MLP) drawn with std 0.02/sqrt(2*n_layer) --
    same page, section GPT2LMHeadModel (the _init_weights remark).
  * MLP width 4*d_model -- same page, section GPT2Block (inner_dim).
  * Parameter order: the safetensors key list -- same page, section
    "权重即架构" (weights as architecture).

Parameter blob layout (fp32, one flat array, this exact order):
    wte[V, D], wpe[P, D],
    per layer l = 0..L-1:
        ln_1.w[D], ln_1.b[D],
        attn.c_attn.w[D, 3D], attn.c_attn.b[3D],
        attn.c_proj.w[D, D], attn.c_proj.b[D],
        ln_2.w[D], ln_2.b[D],
        mlp.c_fc.w[D, F], mlp.c_fc.b[F],
        mlp.c_proj.w[F, D], mlp.c_proj.b[D],
    ln_f.w[D], ln_f.b[D],
    lm_head.w[V, D]          (only when tie_word_embeddings is False)
Matrices are stored [in, out] (the Conv1D orientation: y = x @ W + b); the
separate head is stored like wte, [V, D] (nn.Linear's [out, in]).

Random numbers.  Token ids come from numpy's PCG64 (``default_rng``).
Parameters come from a counter-based generator so that large blobs (GPT-2 XL
has 1.56e9 parameters) can be filled in parallel chunks with a result that
does not depend on the chunking: element i of tensor s of a blob with seed S
takes the SplitMix64 output (Steele, Lea & Flood, "Fast Splittable
Pseudorandom Number Generators", OOPSLA 2014) of the counter
    c = (S << 48) | (s << 32) | (i // 2)      (S, s < 2^16; i // 2 < 2^32)
and turns its two 32-bit halves into two standard normals with the
Box-Muller transform (element 2j gets the cosine branch, 2j+1 the sine
branch).
"""
from __future__ import annotations

import math
import os
import threading
from dataclasses import dataclass, field, asdict

import numpy as np

# --------------------------------------------------------------------------
# Model and workload descriptions
# --------------------------------------------------------------------------


@dataclass(frozen=True)
class ModelShape:
    vocab: int
    n_positions: int
    d_model: int
    n_head: int
    n_layer: int
    d_ff: int
    ln_eps: float = 1e-5
    # Variants the pages describe as switches; the defaults are GPT-2 as
    # released (pwwt.cn GPT2Config / GPT2MLP; russellluo.com Pre-Norm;
    # nano-ai.tech Transformer Stack for the separate head).
    activation: str = "gelu_new"                   # "gelu_new" (tanh form) or "gelu" (erf form)
    scale_attn_by_inverse_layer_idx: bool = False  # scores further divided by layer index + 1
    post_ln: bool = False                          # LN(x + Sublayer(x)) instead of x + Sublayer(LN(x))
    tie_word_embeddings: bool = True               # False: a separate head lm_head.w [V, D]

    @property
    def head_dim(self) -> int:
        return self.d_model // self.n_head


@dataclass(frozen=True)
class Init:
    """Normal init recipe: (mean, std) per parameter group; std 0 = constant."""
    w_std: float            # wte, wpe, c_attn.w, c_fc.w
    proj_std: float         # attn.c_proj.w and mlp.c_proj.w
    bias_std: float         # every bias
    gamma: tuple            # (mean, std) of LayerNorm weights
    beta: tuple             # (mean, std) of LayerNorm biases


@dataclass(frozen=True)
class Workload:
    name: str
    shape: ModelShape
    init: Init
    dtype: str              # "f32" or "bf16": arithmetic type of the GPU path
    batch: int
    seq_len: int            # tokens per sequence in the forward (prefill length for decode)
    param_seed: int
    ids_seed: int
    decode: bool = False    # True: one new token per sequence after a prefill of seq_len

    def as_dict(self):
        d = asdict(self)
        return d


def _gpt2_init(n_layer: int) -> Init:
    return Init(w_std=0.02, proj_std=0.02 / math.sqrt(2 * n_layer), bias_std=0.01,
                gamma=(1.0, 0.05), beta=(0.0, 0.02))


TINY = ModelShape(vocab=512, n_positions=64, d_model=64, n_head=4, n_layer=2, d_ff=256)
SMALL = ModelShape(vocab=50257, n_positions=1024, d_model=768, n_head=12, n_layer=12, d_ff=3072)
MEDIUM = ModelShape(vocab=50257, n_positions=1024, d_model=1024, n_head=16, n_layer=24, d_ff=4096)
XL = ModelShape(vocab=50257, n_positions=1024, d_model=1600, n_head=25, n_layer=48, d_ff=6400)

WORKLOADS = {
    "gpt2-tiny-fp32-b1t16": Workload(
        "gpt2-tiny-fp32-b1t16", TINY,
        Init(w_std=0.02, proj_std=0.02 / math.sqrt(2 * TINY.n_layer), bias_std=0.0,
             gamma=(1.0, 0.0), beta=(0.0, 0.0)),
        "f32", batch=1, seq_len=16, param_seed=1000, ids_seed=2000),
    "gpt2-small-b8t1024": Workload(
        "gpt2-small-b8t1024", SMALL, _gpt2_init(12), "bf16", batch=8, seq_len=1024,
        param_seed=1001, ids_seed=2001),
    "gpt2-small-decode-b32p1023": Workload(
        "gpt2-small-decode-b32p1023", SMALL, _gpt2_init(12), "bf16", batch=32, seq_len=1023,
        param_seed=1002, ids_seed=2002, decode=True),
    "gpt2-medium-b8t1024": Workload(
        "gpt2-medium-b8t1024", MEDIUM, _gpt2_init(24), "bf16", batch=8, seq_len=1024,
        param_seed=1003, ids_seed=2003),
    "gpt2-xl-b4t1024": Workload(
        "gpt2-xl-b4t1024", XL, _gpt2_init(48), "bf16", batch=4, seq_len=1024,
        param_seed=1004, ids_seed=2004),
}

# --------------------------------------------------------------------------
# Parameter blob layout
# --------------------------------------------------------------------------

LAYER_TENSORS = ("ln_1.w", "ln_1.b", "attn.c_attn.w", "attn.c_attn.b", "attn.c_proj.w",
                 "attn.c_proj.b", "ln_2.w", "ln_2.b", "mlp.c_fc.w", "mlp.c_fc.b",
                 "mlp.c_proj.w", "mlp.c_proj.b")


def param_specs(s: ModelShape):
    """Ordered list of (key, shape) in blob order."""
    D, F = s.d_model, s.d_ff
    shapes = {"ln_1.w": (D,), "ln_1.b": (D,), "attn.c_attn.w": (D, 3 * D),
              "attn.c_attn.b": (3 * D,), "attn.c_proj.w": (D, D), "attn.c_proj.b": (D,),
              "ln_2.w": (D,), "ln_2.b": (D,), "mlp.c_fc.w": (D, F), "mlp.c_fc.b": (F,),
              "mlp.c_proj.w": (F, D), "mlp.c_proj.b": (D,)}
    out = [("wte", (s.vocab, D)), ("wpe", (s.n_positions, D))]
    for l in range(s.n_layer):
        for k in LAYER_TENSORS:
            out.append((f"h.{l}.{k}", shapes[k]))
    out += [("ln_f.w", (D,)), ("ln_f.b", (D,))]
    if not s.tie_word_embeddings:
        out.append(("lm_head.w", (s.vocab, D)))
    return out


def param_count(s: ModelShape) -> int:
    return sum(int(np.prod(shp)) for _, shp in param_specs(s))


def param_offsets(s: ModelShape):
    """key -> (offset in floats, shape)."""
    off, out = 0, {}
    for k, shp in param_specs(s):
        out[k] = (off, shp)
        off += int(np.prod(shp))
    return out


def unpack(blob: np.ndarray, s: ModelShape) -> dict:
    """Views of the blob, keyed like the safetensors names (without 'transformer.')."""
    out = {}
    for k, (off, shp) in param_offsets(s).items():
        out[k] = blob[off:off + int(np.prod(shp))].reshape(shp)
    return out


def _init_of(key: str, init: Init):
    """(mean, std) for one tensor key."""
    leaf = key.split(".", 2)[-1] if key.startswith("h.") else key
    if leaf in ("wte", "wpe", "lm_head.w", "attn.c_attn.w", "mlp.c_fc.w"):
        return 0.0, init.w_std
    if leaf in ("attn.c_proj.w", "mlp.c_proj.w"):
        return 0.0, init.proj_std
    if leaf.endswith(".b") and not leaf.startswith("ln"):
        return 0.0, init.bias_std
    if leaf.endswith(".w"):        # ln_1.w, ln_2.w, ln_f.w
        return init.gamma
    return init.beta               # ln_*.b


# --------------------------------------------------------------------------
# Counter-based normal generator (SplitMix64 + Box-Muller)
# --------------------------------------------------------------------------

_M64 = np.uint64(0xFFFFFFFFFFFFFFFF)
_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_MIX1 = np.uint64(0xBF58476D1CE4E5B9)
_MIX2 = np.uint64(0x94D049BB133111EB)


def _splitmix64(c: np.ndarray) -> np.ndarray:
    """SplitMix64 output function applied to state c*golden (c uint64 array)."""
    with np.errstate(over="ignore"):
        z = (c + np.uint64(1)) * _GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _MIX1
        z = (z ^ (z >> np.uint64(27))) * _MIX2
        z = z ^ (z >> np.uint64(31))
    return z


def _normals_chunk(seed: int, stream: int, start: int, n: int) -> np.ndarray:
    """Standard normals for element indices [start, start+n) of one stream."""
    p0, p1 = start // 2, (start + n + 1) // 2
    pairs = np.arange(p0, p1, dtype=np.uint64)
    assert p1 <= (1 << 32) and 0 <= seed < (1 << 16) and 0 <= stream < (1 << 16)
    key = np.uint64((seed << 48) | (stream << 32))
    z = _splitmix64(pairs | key)
    # two 32-bit uniforms in (0, 1]: (k + 1) / 2^32
    u1 = ((z >> np.uint64(32)).astype(np.float64) + 1.0) * (1.0 / 4294967296.0)
    u2 = ((z & np.uint64(0xFFFFFFFF)).astype(np.float64) + 1.0) * (1.0 / 4294967296.0)
    r = np.sqrt(-2.0 * np.log(u1))
    th = (2.0 * np.pi) * u2
    out = np.empty(2 * (p1 - p0), dtype=np.float64)
    out[0::2] = r * np.cos(th)
    out[1::2] = r * np.sin(th)
    off = start - 2 * p0
    return out[off:off + n]


def counter_normals(seed: int, stream: int, n: int, mean: float, std: float,
                    out: np.ndarray | None = None, threads: int | None = None) -> np.ndarray:
    """n values mean + std * N(0,1) as float32, filled in parallel chunks."""
    if out is None:
        out = np.empty(n, dtype=np.float32)
    if std == 0.0:
        out[:] = np.float32(mean)
        return out
    chunk = 1 << 21
    starts = list(range(0, n, chunk))

    def work(idx):
        for s0 in starts[idx::nt]:
            m = min(chunk, n - s0)
            out[s0:s0 + m] = (mean + std * _normals_chunk(seed, stream, s0, m)).astype(np.float32)

    nt = max(1, min(threads or os.cpu_count() or 1, 16, len(starts)))
    if nt == 1:
        work(0)
    else:
        ths = [threading.Thread(target=work, args=(i,)) for i in range(nt)]
        for t in ths:
            t.start()
        for t in ths:
            t.join()
    return out


def make_params(w: Workload | ModelShape, init: Init | None = None, seed: int | None = None,
                out: np.ndarray | None = None) -> np.ndarray:
    """The fp32 parameter blob of a workload (or of a shape + init + seed)."""
    if isinstance(w, Workload):
        shape, init, seed = w.shape, w.init, w.param_seed
    else:
        shape = w
    n = param_count(shape)
    if out is None:
        out = np.empty(n, dtype=np.float32)
    for stream, (key, (off, shp)) in enumerate(param_offsets(shape).items()):
        mean, std = _init_of(key, init)
        m = int(np.prod(shp))
        counter_normals(seed, stream, m, mean, std, out=out[off:off + m])
    return out


def make_ids(w: Workload) -> np.ndarray:
    """Token ids int32 [B, T] (uniform over the vocabulary, numpy PCG64)."""
    rng = np.random.default_rng(w.ids_seed)
    return rng.integers(0, w.shape.vocab, size=(w.batch, w.seq_len), dtype=np.int32)


def make_decode_ids(w: Workload) -> tuple[np.ndarray, np.ndarray]:
    """(prefix ids [B, P], new ids [B]) for a decode workload, same PCG64 stream."""
    rng = np.random.default_rng(w.ids_seed)
    prefix = rng.integers(0, w.shape.vocab, size=(w.batch, w.seq_len), dtype=np.int32)
    new = rng.integers(0, w.shape.vocab, size=(w.batch,), dtype=np.int32)
    return prefix, new
