// Causal multi-head attention kernels.
//
// What is computed (pwwt.cn "逐行拆GPT-2源码", GPT2Attention `_attn`; dpshk.com
// llm.c notes 2.2-2.3): for every sequence b and head h,
//   a_i = sum_{j <= i} softmax_j(q_i . k_j / sqrt(head_dim)) v_j,
// keys after the query (j > i) take no part at all.  q arrives already scaled
// by 1/sqrt(head_dim) (folded into the c_attn epilogue; a power of two for
// head_dim 16 and 64, so the fold is exact).  Heads are merged back in order
// into a [B*T, d_model] row-major activation (GPT2Attention `_merge_heads`).
#pragma once

#include "common.h"

namespace gpt2 {

// Prefill / full forward.  q: [B*H][Tq][hs] at positions 0..Tq-1; k: [B*H][kvT][hs];
// vt: [B*H][hs][kvT]; out: [B*Tq][D] with head h in columns h*hs .. h*hs+hs-1.
// lse (optional): [B*H][Tq], log(sum_j exp(s_ij)) of each query's scores
// s = q k^T (q pre-scaled), for the backward pass.
template <typename T>
hipError_t launch_attention_prefill(const T* q, const T* k, const T* vt, T* out, int B, int H, int Tq,
                                    int kvT, int hs, hipStream_t stream, float* lse = nullptr);

// Decode: one query per (b, h) at position pos = n_keys - 1, attending keys
// 0..n_keys-1 of the cache.  q: [B*H][hs]; k: [B*H][kvT][hs]; vt: [B*H][hs][kvT];
// part: scratch floats, at least decode_partials_floats(B, H, hs); out: [B][D].
size_t decode_partials_floats(int B, int H, int hs);
template <typename T>
hipError_t launch_attention_decode(const T* q, const T* k, const T* vt, T* out, float* part, int B,
                                   int H, int n_keys, int kvT, int hs, hipStream_t stream);

}  // namespace gpt2
