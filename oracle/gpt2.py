"""Plain fp64 reference of the GPT-2 Pre-LN forward pass -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  It shares no code with the HIP path.

Every value is carried in float64.  Matrix products use numpy's ``@`` (a
library primitive); nothing is blocked, fused or reordered beyond the plain
definitions below.  Each function names the page passage it follows; the
pages are cited by title and section:

  [Hidden]  russellluo.com, "从零学大模型：Hidden State 如何流过 GPT-2 Block？"
  [HFsrc]   pwwt.cn, "逐行拆GPT-2源码：GPT2LMHeadModel到Attention"
  [Anatomy] bbs.huaweicloud.com blog 476445 (GPT-2 parameter anatomy)
  [Stack]   nano-ai.tech, "从零手写大模型 · 推理篇 12 - Transformer Stack"
  [llmc]    dpshk.com news 6064214 (llm.c study notes on attention, LN, MLP)

Readings taken where the pages leave a point open (each also listed in the
design notes of the repository):
  * LayerNorm variance is the biased (divide by D) variance, eps = 1e-5 added
    to the variance inside the square root ([llmc] 3.2; [HFsrc] GPT2Config).
  * The causal mask removes keys j > i entirely (weight exactly 0); the row
    maximum is subtracted before exp ([HFsrc] GPT2Attention ``_attn``; [llmc]
    2.3 and 5.3).
  * Attention scores are divided by sqrt(head_dim); no per-layer scaling
    ([HFsrc] GPT2Config, scale_attn_by_inverse_layer_idx = false).
  * The lm_head is tied to wte and has no bias ([HFsrc] GPT2LMHeadModel).
  * Dropout is the identity (inference; [Hidden] Pre-Norm section).
  * "bf16 weights": matrices and wte/wpe are rounded fp32 -> bf16
    (round-to-nearest-even) once; biases and LayerNorm parameters stay fp32.
    After that rounding, every operation is fp64 -- the oracle never rounds
    activations.
"""
from __future__ import annotations

import numpy as np

TRACE_POINTS = ("attn_norm", "ffn_inp", "ffn_norm", "ffn_out", "l_out")

# --------------------------------------------------------------------------
# bf16 rounding of the stored weights
# --------------------------------------------------------------------------


def bf16_round(a: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned as float32 values.

    bf16 keeps the upper 16 bits of an IEEE binary32.  Rounding adds half an
    ulp of the kept part (0x7FFF) plus the kept part's lowest bit (for ties to
    even), then truncates.  NaNs stay NaN (quiet).
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    r = r.astype(np.uint32)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = (u[nan].astype(np.uint32) | 0x00400000) & 0xFFFF0000
    return r.view(np.float32)


# --------------------------------------------------------------------------
# Building blocks
# --------------------------------------------------------------------------


def layer_norm(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float = 1e-5) -> np.ndarray:
    """LN(x) = gamma * (x - mu) / sqrt(var + eps) + beta over the last axis.

    [Hidden] section Pre-Norm (the LN formula, eps inside the root);
    [llmc] 3.2 (two passes: mean, then variance; eps added to the variance).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    mu = x.sum(axis=-1, keepdims=True) / d
    xc = x - mu
    var = (xc * xc).sum(axis=-1, keepdims=True) / d
    return xc / np.sqrt(var + eps) * np.asarray(gamma, np.float64) + np.asarray(beta, np.float64)


def gelu_new(x: np.ndarray) -> np.ndarray:
    """0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))).

    [HFsrc] section GPT2MLP (NewGELUActivation); [llmc] 4.2 (x^3 as x*x*x).
    """
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * (x * x * x))))


def gelu_erf(x: np.ndarray) -> np.ndarray:
    """0.5 x (1 + erf(x / sqrt(2))), the standard GELU the pages contrast with
    gelu_new ([HFsrc] section GPT2MLP).  erf from scipy (a library routine)."""
    from scipy.special import erf
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_offset: int = 0,
                     return_probs: bool = False, scale: float | None = None):
    """softmax(q k^T * scale, keys j <= i) v, per head; scale = 1/sqrt(hs) unless given.

    q: [H, Tq, hs] at absolute positions q_offset .. q_offset+Tq-1;
    k, v: [H, Tk, hs] at positions 0 .. Tk-1.
    [HFsrc] GPT2Attention ``_attn`` (scores, scale by sqrt of the head size,
    lower-triangular mask sliced to the last Tq rows, softmax, weights @ v);
    [llmc] 2.2 (scale), 2.3 (mask before softmax), 5.3 (max subtraction).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    H, Tq, hs = q.shape
    Tk = k.shape[1]
    i = np.arange(Tq)[:, None] + q_offset
    j = np.arange(Tk)[None, :]
    allowed = j <= i                                   # [Tq, Tk]
    out = np.empty((H, Tq, v.shape[2]), dtype=np.float64)
    probs = np.empty((H, Tq, Tk), dtype=np.float64) if return_probs else None
    for h in range(H):
        s = (q[h] @ k[h].T) / np.sqrt(float(hs)) if scale is None else (q[h] @ k[h].T) * scale
        s = np.where(allowed, s, -np.inf)
        s = s - s.max(axis=-1, keepdims=True)
        e = np.where(allowed, np.exp(s), 0.0)
        p = e / e.sum(axis=-1, keepdims=True)
        out[h] = p @ v[h]
        if return_probs:
            probs[h] = p
    return (out, probs) if return_probs else out


# --------------------------------------------------------------------------
# Parameters
# --------------------------------------------------------------------------


def prepare_params(blob: np.ndarray, shape, dtype: str) -> dict:
    """fp64 views of the parameter blob, keyed as in the safetensors list.

    dtype "bf16": matrices and wte/wpe are first rounded to bf16 (see module
    notes); "f32": values used as stored.
    """
    from workloads import unpack  # layout only (offsets of each key)
    raw = unpack(np.asarray(blob, np.float32), shape)
    out = {}
    for key, arr in raw.items():
        is_matrix = key in ("wte", "wpe", "lm_head.w") or key.endswith("c_attn.w") or key.endswith("c_proj.w") \
            or key.endswith("c_fc.w")
        a = bf16_round(arr) if (dtype == "bf16" and is_matrix) else arr
        out[key] = a.astype(np.float64)
    out["_shape"] = shape
    return out


# --------------------------------------------------------------------------
# The stack
# --------------------------------------------------------------------------


def embed(P: dict, ids: np.ndarray, pos0: int = 0) -> np.ndarray:
    """x_t = wte[id_t] + wpe[pos0 + t]  ([HFsrc] GPT2Model; [Stack] GPT.forward)."""
    ids = np.asarray(ids)
    T = ids.shape[-1]
    return P["wte"][ids] + P["wpe"][pos0:pos0 + T]


def block_forward(x: np.ndarray, P: dict, l: int, trace: dict | None = None) -> np.ndarray:
    """One block on one sequence x [T, D].

    Pre-LN (GPT-2):  H = X + Attn(LN_1(X)),  X' = H + MLP(LN_2(H))
    [Hidden] section "GPT-2 Block" (the four-line data flow);
    [HFsrc] GPT2Block.forward (ln_1 -> attn -> residual -> ln_2 -> mlp ->
    residual), GPT2Attention (fused c_attn, split into thirds q|k|v, heads as
    consecutive head_dim-wide column blocks, merge heads, c_proj), GPT2MLP
    (c_fc -> gelu_new -> c_proj).
    Switches of the model shape (defaults as above):
      post_ln: H = LN_1(X + Attn(X)),  X' = LN_2(H + MLP(H)) -- the Post-Norm
        form LN(x + Sublayer(x)) ([Hidden] Pre-Norm section; [llmc] 3.1);
        the same ln_1 / ln_2 parameters, ln_f and the head unchanged.
      scale_attn_by_inverse_layer_idx: scores further divided by l + 1
        ([HFsrc] GPT2Config, the switch of the original TensorFlow code).
      activation "gelu": the erf GELU instead of gelu_new ([HFsrc] GPT2MLP).
    """
    s = P["_shape"]
    D, H = s.d_model, s.n_head
    hs = D // H
    T = x.shape[0]
    pre = f"h.{l}."
    act = gelu_erf if getattr(s, "activation", "gelu_new") == "gelu" else gelu_new
    post = getattr(s, "post_ln", False)
    scale = 1.0 / np.sqrt(float(hs))
    if getattr(s, "scale_attn_by_inverse_layer_idx", False):
        scale = scale / float(l + 1)
    ln1 = lambda z: layer_norm(z, P[pre + "ln_1.w"], P[pre + "ln_1.b"], s.ln_eps)
    ln2 = lambda z: layer_norm(z, P[pre + "ln_2.w"], P[pre + "ln_2.b"], s.ln_eps)
    h = x if post else ln1(x)
    qkv = h @ P[pre + "attn.c_attn.w"] + P[pre + "attn.c_attn.b"]
    q, k, v = qkv[:, :D], qkv[:, D:2 * D], qkv[:, 2 * D:]
    split = lambda t: t.reshape(T, H, hs).transpose(1, 0, 2)   # [H, T, hs]
    a = causal_attention(split(q), split(k), split(v), scale=scale)
    a = a.transpose(1, 0, 2).reshape(T, D)                      # merge heads in order
    x_h = x + (a @ P[pre + "attn.c_proj.w"] + P[pre + "attn.c_proj.b"])
    if post:
        x_h = ln1(x_h)
    h2 = x_h if post else ln2(x_h)
    u = act(h2 @ P[pre + "mlp.c_fc.w"] + P[pre + "mlp.c_fc.b"])
    m = u @ P[pre + "mlp.c_proj.w"] + P[pre + "mlp.c_proj.b"]
    x_out = ln2(x_h + m) if post else x_h + m
    if trace is not None:
        trace.setdefault("attn_norm", []).append(h)
        trace.setdefault("ffn_inp", []).append(x_h)
        trace.setdefault("ffn_norm", []).append(h2)
        trace.setdefault("ffn_out", []).append(m)
        trace.setdefault("l_out", []).append(x_out)
    return x_out


def forward_hidden(P: dict, ids: np.ndarray, n_layers: int | None = None,
                   trace: dict | None = None) -> np.ndarray:
    """ln_f output h_f [T, D] of one sequence ids [T] ([HFsrc] GPT2Model; [Stack])."""
    s = P["_shape"]
    x = embed(P, ids)
    L = s.n_layer if n_layers is None else n_layers
    for l in range(L):
        x = block_forward(x, P, l, trace)
    return layer_norm(x, P["ln_f.w"], P["ln_f.b"], s.ln_eps)


def forward(P: dict, ids: np.ndarray, positions=None, trace: dict | None = None) -> np.ndarray:
    """Logits [B, T, V] (or [B, len(positions), V]) for ids [B, T].

    logits = ln_f(X_L) @ wte^T, the tied head without bias ([HFsrc]
    GPT2LMHeadModel; [Anatomy] LM head; [Stack] final LayerNorm + head);
    with a separate head (tie_word_embeddings False, [Stack]'s nn.Linear
    head) lm_head.w [V, D] takes wte's place.
    ``positions`` selects which rows of every sequence get logits (all when
    None); rows are independent once h_f is known.
    """
    ids = np.atleast_2d(np.asarray(ids))
    head = P["lm_head.w"] if "lm_head.w" in P else P["wte"]   # untied head when present
    outs = []
    for b in range(ids.shape[0]):
        hf = forward_hidden(P, ids[b], trace=trace)
        if positions is not None:
            hf = hf[np.asarray(positions)]
        outs.append(hf @ head.T)
    return np.stack(outs)


def decode_logits(P: dict, prefix: np.ndarray, new_ids: np.ndarray) -> np.ndarray:
    """Logits [B, V] of one new token per sequence after a cached prefix.

    A KV cache only avoids recomputing the prefix's keys and values; the new
    token sits at position len(prefix) ([HFsrc] GPT2Model position_ids from
    past_length; GPT2Attention KV-cache concatenation).  So the result is the
    last row of the plain forward over prefix ++ [new].
    """
    prefix = np.atleast_2d(np.asarray(prefix))
    new_ids = np.asarray(new_ids).reshape(-1)
    full = np.concatenate([prefix, new_ids[:, None]], axis=1)
    T = full.shape[1]
    return forward(P, full, positions=[T - 1])[:, 0, :]


def shifted_cross_entropy(logits: np.ndarray, labels: np.ndarray):
    """Next-token cross-entropy of logits [B, T, V] against labels [B, T].

    Returns (mean, per_position [B, T-1]).  [HFsrc] section GPT2LMHeadModel,
    its second design: the shift happens inside the model -- the logits of
    positions 0..T-2 are scored against the labels of positions 1..T-1, the
    pairs are flattened and averaged by a cross-entropy loss.  Per position t:
    loss_t = log(sum_v exp(logit_t[v])) - logit_t[label_{t+1}], the sum taken
    after subtracting the row maximum.
    Readings: a negative label marks a position that is not scored (loss
    reported as 0, left out of the mean, as the loss's usual ignore index);
    the mean over zero scored positions is NaN.
    """
    logits = np.asarray(logits, dtype=np.float64)[:, :-1, :]     # [B, T-1, V]
    tgt = np.atleast_2d(np.asarray(labels))[:, 1:]                 # [B, T-1]
    mx = logits.max(axis=-1, keepdims=True)
    lse = mx[..., 0] + np.log(np.exp(logits - mx).sum(axis=-1))
    counted = tgt >= 0
    picked = np.take_along_axis(logits, np.where(counted, tgt, 0)[..., None], axis=-1)[..., 0]
    per = np.where(counted, lse - picked, 0.0)
    n = int(counted.sum())
    mean = per.sum() / n if n else float("nan")
    return float(mean), per


def lm_loss(P: dict, ids: np.ndarray, labels: np.ndarray | None = None):
    """Loss of GPT2LMHeadModel called with labels ([HFsrc] GPT2LMHeadModel):
    the forward's logits through shifted_cross_entropy; labels default to the
    input ids, the ordinary call since the shift happens inside."""
    ids = np.atleast_2d(np.asarray(ids))
    labels = ids if labels is None else np.atleast_2d(np.asarray(labels))
    return shifted_cross_entropy(forward(P, ids), labels)


def generate_greedy(P: dict, prompt: np.ndarray, n_steps: int) -> np.ndarray:
    """Greedy continuation of prompt [B, P]: n_steps new tokens per sequence.

    Token-by-token generation ([HFsrc] closing section: embeddings, positions,
    the pre-norm stack, causal attention and generation one token at a time)
    with the token chosen from the head's distribution ([Anatomy] architecture
    overview: LM head, softmax over the vocabulary, pick a token).  Reading:
    the pick is the most probable token -- the argmax of the logits, since
    softmax is monotone -- ties to the lowest index.  Each new token is
    appended and the next one is read off the last row of the plain forward
    over the longer sequence (a cache would only avoid recomputation).
    """
    seq = np.atleast_2d(np.asarray(prompt)).copy()
    out = np.empty((seq.shape[0], n_steps), dtype=np.int64)
    for i in range(n_steps):
        last = forward(P, seq, positions=[seq.shape[1] - 1])[:, 0, :]
        out[:, i] = last.argmax(axis=-1)          # numpy: first maximum wins
        seq = np.concatenate([seq, out[:, i:i + 1]], axis=1)
    return out


_U64 = np.uint64
_M64 = (1 << 64) - 1


def splitmix64(x: np.ndarray) -> np.ndarray:
    """SplitMix64 output function (Steele, Lea and Flood, "Fast splittable
    pseudorandom number generators", OOPSLA 2014): state x advanced by the
    golden-ratio increment 0x9E3779B97F4A7C15, then z ^= z >> 30, z *= 0xBF58476D1CE4E5B9,
    z ^= z >> 27, z *= 0x94D049BB133111EB, z ^= z >> 31, all modulo 2^64."""
    with np.errstate(over="ignore"):
        z = np.asarray(x, dtype=_U64) + _U64(0x9E3779B97F4A7C15)
        z = (z ^ (z >> _U64(30))) * _U64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> _U64(27))) * _U64(0x94D049BB133111EB)
        return z ^ (z >> _U64(31))


def sample_uniforms(seed: int, position: int, row: int, n: int) -> np.ndarray:
    """U_v in (0, 1) for v = 0..n-1 of one row at one position: a counter-based
    draw, U_v = ((splitmix64(key ^ v) >> 40) + 1/2) / 2^24 with
    key = splitmix64(splitmix64(seed) ^ (position << 32) ^ row)."""
    s0 = int(splitmix64(_U64(seed & _M64)))
    key = int(splitmix64(_U64((s0 ^ ((position & 0xFFFFFFFF) << 32) ^ (row & 0xFFFFFFFF)) & _M64)))
    z = splitmix64(_U64(key) ^ np.arange(n, dtype=_U64))
    return ((z >> _U64(40)).astype(np.float64) + 0.5) / float(1 << 24)


def sample_token(logits: np.ndarray, temperature: float, seed: int, position: int, row: int):
    """One token drawn from softmax(logits / temperature): the Gumbel-max
    identity, argmax_v (logit_v / temperature + G_v) with G_v = -ln(-ln U_v)
    standard Gumbel variables, is distributed as that softmax (the pages' last
    step: [Anatomy] architecture overview, softmax over the vocabulary and a
    token picked from it; [Stack]: with random weights the pick is a random
    draw).  Returns (token, the perturbed scores); ties to the lowest index."""
    u = sample_uniforms(seed, position, row, logits.shape[-1])
    scores = np.asarray(logits, np.float64) / temperature - np.log(-np.log(u))
    return int(scores.argmax()), scores


def generate_sample(P: dict, prompt: np.ndarray, n_steps: int, temperature: float, seed: int):
    """Sampled continuation of prompt [B, P]: as generate_greedy, with each
    token drawn by sample_token at the position of the step's input token
    (the last token of the sequence so far) for row b.  Returns (tokens
    [B, n_steps], the perturbed scores [B, n_steps, V])."""
    seq = np.atleast_2d(np.asarray(prompt)).copy()
    Bn = seq.shape[0]
    out = np.empty((Bn, n_steps), dtype=np.int64)
    all_scores = []
    for i in range(n_steps):
        pos = seq.shape[1] - 1
        last = forward(P, seq, positions=[pos])[:, 0, :]
        step_scores = []
        for b in range(Bn):
            out[b, i], sc = sample_token(last[b], temperature, seed, pos, b)
            step_scores.append(sc)
        all_scores.append(np.stack(step_scores))
        seq = np.concatenate([seq, out[:, i:i + 1]], axis=1)
    return out, np.stack(all_scores, axis=1)


# --------------------------------------------------------------------------
# Backward of one block
# --------------------------------------------------------------------------


def gelu_new_grad(x: np.ndarray) -> np.ndarray:
    """d/dx gelu_new(x) = 0.5 (1 + t) + 0.5 x (1 - t^2) sqrt(2/pi) (1 + 3 c x^2),
    t = tanh(sqrt(2/pi) (x + c x^3)), c = 0.044715 (the derivative of [HFsrc]
    GPT2MLP's NewGELUActivation)."""
    x = np.asarray(x, dtype=np.float64)
    k = np.sqrt(2.0 / np.pi)
    t = np.tanh(k * (x + 0.044715 * x * x * x))
    return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * k * (1.0 + 3.0 * 0.044715 * x * x)


def gelu_erf_grad(x: np.ndarray) -> np.ndarray:
    """d/dx 0.5 x (1 + erf(x/sqrt 2)) = Phi(x) + x phi(x) (standard normal cdf / pdf)."""
    from scipy.special import erf
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * (1.0 + erf(x / np.sqrt(2.0))) + x * np.exp(-0.5 * x * x) / np.sqrt(2.0 * np.pi)


def layer_norm_backward(dh: np.ndarray, x: np.ndarray, gamma: np.ndarray, eps: float = 1e-5):
    """Gradients of h = gamma * xhat + beta, xhat = (x - mu) / sqrt(var + eps),
    over the last axis: returns (dx, dgamma, dbeta) with dgamma, dbeta summed
    over every leading axis.  [llmc] 5.3: the mean, the variance and the
    normalised value are coupled --
      dxhat = dh * gamma,
      dx = rstd * (dxhat - mean(dxhat) - xhat * mean(dxhat * xhat)),
    dgamma = sum dh * xhat, dbeta = sum dh."""
    x = np.asarray(x, np.float64)
    dh = np.asarray(dh, np.float64)
    d = x.shape[-1]
    mu = x.sum(axis=-1, keepdims=True) / d
    xc = x - mu
    rstd = 1.0 / np.sqrt((xc * xc).sum(axis=-1, keepdims=True) / d + eps)
    xhat = xc * rstd
    dxhat = dh * np.asarray(gamma, np.float64)
    dx = rstd * (dxhat - dxhat.mean(axis=-1, keepdims=True) - xhat * (dxhat * xhat).mean(axis=-1, keepdims=True))
    lead = tuple(range(dh.ndim - 1))
    return dx, (dh * xhat).sum(axis=lead), dh.sum(axis=lead)


def block_backward(x: np.ndarray, dy: np.ndarray, P: dict, l: int):
    """Backward of Pre-LN block l on one sequence: x [T, D] is the block input,
    dy [T, D] the gradient of a loss with respect to the block output.
    Returns (dx [T, D], grads) with grads keyed like the parameters
    ("h.{l}.ln_1.w", ...), matrices in the blob's [in, out] orientation.

    The forward of block_forward taken in reverse, one step at a time ([llmc]
    5.3 on the two delicate steps):
      MLP:        y = x_h + u W_pr + b_pr,  u = act(g),  g = h2 W_fc + b_fc,
                  h2 = LN_2(x_h)
      attention:  x_h = x + a W_o + b_o,  a = merge_heads(p v),
                  p = softmax(s) over keys j <= i (masked entries exactly 0,
                  so their gradient is exactly 0), s = q k^T * scale,
                  [q | k | v] = h1 W_qkv + b_qkv,  h1 = LN_1(x)
    Softmax backward: ds = p * (dp - sum_j dp * p).
    """
    s = P["_shape"]
    if getattr(s, "post_ln", False):
        raise NotImplementedError("backward of the Post-LN wiring is not built")
    D, H = s.d_model, s.n_head
    hs = D // H
    T = x.shape[0]
    pre = f"h.{l}."
    g_ = lambda k: P[pre + k]
    erf_form = getattr(s, "activation", "gelu_new") == "gelu"
    act = gelu_erf if erf_form else gelu_new
    act_grad = gelu_erf_grad if erf_form else gelu_new_grad
    scale = 1.0 / np.sqrt(float(hs))
    if getattr(s, "scale_attn_by_inverse_layer_idx", False):
        scale = scale / float(l + 1)
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    # forward, keeping what the backward needs
    h1 = layer_norm(x, g_("ln_1.w"), g_("ln_1.b"), s.ln_eps)
    qkv = h1 @ g_("attn.c_attn.w") + g_("attn.c_attn.b")
    split = lambda t: t.reshape(T, H, hs).transpose(1, 0, 2)    # [H, T, hs]
    q, k, v = split(qkv[:, :D]), split(qkv[:, D:2 * D]), split(qkv[:, 2 * D:])
    o, p = causal_attention(q, k, v, scale=scale, return_probs=True)
    a = o.transpose(1, 0, 2).reshape(T, D)
    x_h = x + a @ g_("attn.c_proj.w") + g_("attn.c_proj.b")
    h2 = layer_norm(x_h, g_("ln_2.w"), g_("ln_2.b"), s.ln_eps)
    gpre = h2 @ g_("mlp.c_fc.w") + g_("mlp.c_fc.b")
    u = act(gpre)
    grads = {}
    # MLP
    grads[pre + "mlp.c_proj.b"] = dy.sum(axis=0)
    grads[pre + "mlp.c_proj.w"] = u.T @ dy
    dgpre = (dy @ g_("mlp.c_proj.w").T) * act_grad(gpre)
    grads[pre + "mlp.c_fc.b"] = dgpre.sum(axis=0)
    grads[pre + "mlp.c_fc.w"] = h2.T @ dgpre
    dh2 = dgpre @ g_("mlp.c_fc.w").T
    dxh_ln, grads[pre + "ln_2.w"], grads[pre + "ln_2.b"] = layer_norm_backward(dh2, x_h, g_("ln_2.w"), s.ln_eps)
    dx_h = dy + dxh_ln
    # attention
    grads[pre + "attn.c_proj.b"] = dx_h.sum(axis=0)
    grads[pre + "attn.c_proj.w"] = a.T @ dx_h
    do = split(dx_h @ g_("attn.c_proj.w").T)                      # [H, T, hs]
    dv = np.einsum("hij,hid->hjd", p, do)
    dp = np.einsum("hid,hjd->hij", do, v)
    ds = p * (dp - (dp * p).sum(axis=-1, keepdims=True))           # 0 wherever p is masked
    dq = np.einsum("hij,hjd->hid", ds, k) * scale
    dk = np.einsum("hij,hid->hjd", ds, q) * scale
    merge = lambda t: t.transpose(1, 0, 2).reshape(T, D)
    dqkv = np.concatenate([merge(dq), merge(dk), merge(dv)], axis=1)
    grads[pre + "attn.c_attn.b"] = dqkv.sum(axis=0)
    grads[pre + "attn.c_attn.w"] = h1.T @ dqkv
    dh1 = dqkv @ g_("attn.c_attn.w").T
    dx_ln, grads[pre + "ln_1.w"], grads[pre + "ln_1.b"] = layer_norm_backward(dh1, x, g_("ln_1.w"), s.ln_eps)
    return dx_h + dx_ln, grads


def block_backward_batch(x: np.ndarray, dy: np.ndarray, P: dict, l: int):
    """block_backward over a batch x, dy [B, T, D]: dx [B, T, D] and parameter
    gradients summed over the sequences (sequences are independent)."""
    dxs, total = [], {}
    for b in range(x.shape[0]):
        dx, g = block_backward(x[b], dy[b], P, l)
        dxs.append(dx)
        for k2, v2 in g.items():
            total[k2] = total[k2] + v2 if k2 in total else v2
    return np.stack(dxs), total
