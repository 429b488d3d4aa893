// Row-wise HBM-bound kernels: token + position embedding, LayerNorm, and the
// one-time parameter conversion.
#pragma once

#include "common.h"

namespace gpt2 {

// Token id used for the gather: ids outside [0, V) (V = vocab_size, the rows
// of wte holding the vocabulary, pwwt.cn GPT2Config vocab_size) are clamped
// to the nearest valid row, so a bad id can never address memory outside wte.
__host__ __device__ inline int clamp_token_id(int id, int V) { return id < 0 ? 0 : (id >= V ? V - 1 : id); }

// x[m, :] = wte[ids[m], :] + wpe[pos0 + m % T, :] (fp32 out).
// pwwt.cn "逐行拆GPT-2源码", GPT2Model (wte + wpe, positions from past_length).
// ids are clamped by clamp_token_id; when bad is non-null and some id was
// outside [0, V), *bad receives 1 (it is never cleared here).
template <typename T>
hipError_t launch_embed(const int32_t* ids, const T* wte, const T* wpe, float* x, int M, int T_seq,
                        int pos0, int D, int V, int32_t* bad, hipStream_t stream);

// y[m, :] = gamma * (x - mean) / sqrt(var + eps) + beta over D (biased
// variance, two passes over the row held in registers); optional fp32 copy
// y32, which may be x itself (in-place normalisation, the Post-LN wiring).
// russellluo.com "Hidden State 如何流过 GPT-2 Block", Pre-Norm; dpshk.com 3.2.
// prefetch / prefetch_bytes (optional; 16-byte aligned, a multiple of 16): a
// region the kernel also reads and discards, so that the GEMMs that follow
// find their weights in the caches.
// rpart / rks / rbias (optional): first x += (sum_{s<rks} rpart[s][row][:] +
// rbias), the residual add of a split-K projection, written back to x (one
// block of four waves per row; not combined with prefetch).
template <typename T>
hipError_t launch_layernorm(float* x, const float* gamma, const float* beta, T* y, float* y32,
                            int M, int D, float eps, hipStream_t stream, const void* prefetch = nullptr,
                            size_t prefetch_bytes = 0, const float* rpart = nullptr, int rks = 0,
                            const float* rbias = nullptr);

// launch_embed followed by launch_layernorm(x, gamma, beta, y, nullptr, M, D,
// eps, stream, prefetch, prefetch_bytes) in one pass where d_model is 768 or
// 1024 (the row is normalised from the registers it was summed in: the same
// bits, without re-reading x); two launches otherwise.
template <typename T>
hipError_t launch_embed_layernorm(const int32_t* ids, const T* wte, const T* wpe, float* x, int M, int T_seq,
                                  int pos0, int D, int V, int32_t* bad, const float* gamma, const float* beta, T* y,
                                  float eps, hipStream_t stream, const void* prefetch, size_t prefetch_bytes);

// dst[n][k] = convert(src[k][n]) for a [K][N] fp32 source (Conv1D [in, out]
// -> [out, in]); dst rows N..N_pad-1 are zero-filled.
template <typename T>
hipError_t launch_transpose_convert(const float* src, T* dst, int K, int N, int N_pad, hipStream_t stream);

// dst[i] = convert(src[i]) for i < n; dst[n .. n_pad) = 0.
template <typename T>
hipError_t launch_convert(const float* src, T* dst, size_t n, size_t n_pad, hipStream_t stream);

// Next-token cross-entropy (pwwt.cn "逐行拆GPT-2源码", GPT2LMHeadModel: logits
// of position t scored against the label of position t + 1, mean over the
// scored pairs).  part / nseg / tgt are the lm_head's EpiCE partials over
// rows m = b*T + t; loss[b*(T-1) + t] receives each position's loss (0 for a
// negative label, NaN for a label >= V).
hipError_t launch_ce_rows(const float2* part, int nseg, const float* tgt, const int32_t* labels, int B, int T, int V,
                          float* loss, hipStream_t stream);
// out[0] = mean of loss over the positions whose label is >= 0 (NaN if none).
hipError_t launch_ce_mean(const float* loss, const int32_t* labels, int B, int T, float* out, hipStream_t stream);

// Greedy token choice (the generation loop): the largest logit of each row,
// first column on ties, from the lm_head's EpiArgmax partials (part / nseg);
// written to out[row * out_stride] and next[row] (the next step's input).
// Rows without an ordered logit (all NaN) give token 0.
hipError_t launch_argmax_rows(const int2* part, int nseg, int M, int V, int32_t* out, int out_stride, int32_t* next,
                              hipStream_t stream);

}  // namespace gpt2
