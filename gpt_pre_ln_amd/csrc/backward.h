// Kernels of the block backward pass (backward.hip): operand transposes,
// column sums, the LayerNorm backward and the attention backward.  The
// matrix products of the backward run on the GEMM kernel (gemm.h) with the
// EpiStore / EpiGeluSave / EpiGeluBwd epilogues.
#pragma once

#include "common.h"

namespace gpt2 {

// dst[c][r] = convert(src[r][c]) for r < R, c < C (src row-major, ld C); every
// dst row holds ld_dst >= R elements, those past R are set to 0 (the padded
// contraction dimension of the weight-gradient products).
template <typename Tin, typename Tout>
hipError_t launch_transpose(const Tin* src, int R, int C, Tout* dst, int ld_dst, hipStream_t stream);

// out[n] = sum over m < M of src[m][n] (src row-major [M][N]), or, with x / mu /
// rstd given, of src[m][n] * (x[m][n] - mu[m]) * rstd[m] (the LayerNorm gamma
// gradient).  Two passes in a fixed order (row chunks, then chunks): the
// result does not depend on timing.  part: colsum_partial_floats(N) floats.
size_t colsum_partial_floats(int N);
template <typename Tin>
hipError_t launch_colsum(const Tin* src, int M, int N, float* out, float* part, hipStream_t stream,
                         const float* x = nullptr, const float* mu = nullptr, const float* rstd = nullptr);

// The first pass of launch_colsum alone, into part (colsum_partial_floats(N)
// floats); with x / mu / rstd and part_plain given, the same read of src also
// fills part_plain with the plain-sum partials.  launch_colsum_final then
// finishes up to kMaxColsumJobs sums in one launch, each as launch_colsum
// would (same order, same result).
template <typename Tin>
hipError_t launch_colsum_partial(const Tin* src, int M, int N, float* part, hipStream_t stream,
                                 const float* x = nullptr, const float* mu = nullptr, const float* rstd = nullptr,
                                 float* part_plain = nullptr);
constexpr int kMaxColsumJobs = 8;
struct ColsumJob {
  const float* part;  // colsum_partial_floats(N) floats from launch_colsum_partial
  float* out;         // [N]
  int N;
};
hipError_t launch_colsum_final(const ColsumJob* jobs, int n_jobs, hipStream_t stream);

// out[i] = sum_{s < splits} part[s * n + i] in increasing s (the split-K
// partial products of the weight gradients).
hipError_t launch_sum_splits(const float* part, int splits, size_t n, float* out, hipStream_t stream);

// LayerNorm backward (dpshk.com llm.c notes 5.3: mean, variance and the
// normalised value are coupled).  Per row of x [M][D] (the LayerNorm input):
//   xhat = (x - mu) * rstd, g = dh * gamma,
//   out = resid + rstd * (g - mean(g) - xhat * mean(g * xhat)),
// fp32 out [M][D], an optional copy out_t in T, and the row statistics mu /
// rstd [M] (for the gamma gradient).  out must not alias resid or dh.
template <typename T>
hipError_t launch_layernorm_backward(const float* x, const float* dh, const float* gamma, const float* resid,
                                     float* out, T* out_t, float* mu, float* rstd, int M, int D, float eps,
                                     hipStream_t stream);

// Causal attention backward.  q: [B*H][T][hs] (pre-scaled by `scale`),
// k: [B*H][kvT][hs], vt: [B*H][hs][kvT], o and dout: [B*T][H*hs] (the forward
// output and its gradient), lse: [B*H][T] from the forward.  With
// P = exp(q k^T - lse) on keys j <= i (exactly 0 elsewhere) and
// dS = P * (dout v^T - rowsum(dout * o)):
//   dq = scale * dS k,  dk = dS^T q,  dv = P^T dout,
// written in fp32 to dqkv [B*T][3*H*hs] (q | k | v thirds, heads as column
// blocks: the layout of the c_attn output).  dvec: [B*H][T] scratch.
template <typename T>
hipError_t launch_attention_backward(const T* q, const T* k, const T* vt, const T* o, const T* dout,
                                     const float* lse, float* dvec, float* dqkv, int B, int H, int T_seq, int kvT,
                                     int hs, float scale, hipStream_t stream);

}  // namespace gpt2
