// Row-wise kernels (see rowops.h).  One wavefront per row: D <= 2048 floats
// fit in registers (at most 8 float4 per lane), the row statistics are two
// wavefront reductions (mean, then the centred sum of squares) with no LDS.
#include "rowops.h"

#include <algorithm>

namespace gpt2 {

namespace {

constexpr int kMaxV4 = 8;  // float4 per lane -> D <= 2048

// Ids outside [0, V) are clamped to the nearest row of wte, so the gather
// never leaves the matrix; `bad` (optional) then receives 1.
// NV > 0: d_model = 256 NV, all NV chunks of the row requested before the
// first store; NV = 0: any d_model, one chunk at a time.
template <typename T, int NV>
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ ids, const T* __restrict__ wte,
                                                     const T* __restrict__ wpe, float* __restrict__ x, int M,
                                                     int T_seq, int pos0, int D, int V, int32_t* __restrict__ bad) {
  const int row = xcd_block(blockIdx.x, gridDim.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;
  const int raw = ids[row];
  const int id = clamp_token_id(raw, V);
  if (bad && id != raw && lane == 0) *bad = 1;
  const int pos = pos0 + row % T_seq;
  const T* we = wte + (size_t)id * D;
  const T* pe = wpe + (size_t)pos * D;
  float* xr = x + (size_t)row * D;
  if constexpr (NV > 0) {
    float4 a[NV], b[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      a[i] = Elem<T>::load4(we + lane * 4 + i * 256);
      b[i] = Elem<T>::load4(pe + lane * 4 + i * 256);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i)
      *reinterpret_cast<float4*>(xr + lane * 4 + i * 256) =
          make_float4(a[i].x + b[i].x, a[i].y + b[i].y, a[i].z + b[i].z, a[i].w + b[i].w);
  } else {
    for (int c = lane * 4; c < D; c += 256) {
      float4 a = Elem<T>::load4(we + c);
      float4 b = Elem<T>::load4(pe + c);
      *reinterpret_cast<float4*>(xr + c) = make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
    }
  }
}

// Normalises one row held as float4 groups c = lane*4 + i*256 (v) and
// stores it: two wave reductions (mean, then the variance of the centred
// values), then y = (v - mean) * rstd * gamma + beta.
template <typename T, int NV, int NMAX>
__device__ __forceinline__ void layernorm_row(float4 (&v)[NMAX], const float4 (&gv)[NMAX], const float4 (&bv)[NMAX],
                                              int lane, int row, int D, float eps, T* __restrict__ y,
                                              float* y32) {
  auto valid = [&](int i) { return NV > 0 || lane * 4 + i * 256 < D; };
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < NMAX; ++i)
    if (valid(i)) sum += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  const float mean = wave_sum(sum) / (float)D;
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < NMAX; ++i)
    if (valid(i)) {
      v[i].x -= mean;
      v[i].y -= mean;
      v[i].z -= mean;
      v[i].w -= mean;
      sq += (v[i].x * v[i].x + v[i].y * v[i].y) + (v[i].z * v[i].z + v[i].w * v[i].w);
    }
  const float var = wave_sum(sq) / (float)D;
  const float rstd = 1.0f / sqrtf(var + eps);
#pragma unroll
  for (int i = 0; i < NMAX; ++i)
    if (valid(i)) {
      const int c = lane * 4 + i * 256;
      const float4 g = gv[i], b = bv[i];
      const float o0 = v[i].x * rstd * g.x + b.x, o1 = v[i].y * rstd * g.y + b.y;
      const float o2 = v[i].z * rstd * g.z + b.z, o3 = v[i].w * rstd * g.w + b.w;
      Elem<T>::store4(y + (size_t)row * D + c, o0, o1, o2, o3);
      if (y32) *reinterpret_cast<float4*>(y32 + (size_t)row * D + c) = make_float4(o0, o1, o2, o3);
    }
}

// y32 may be x itself (in-place normalisation): a wave loads its whole row
// before it stores anything, and rows are disjoint between waves.
// One wave per row; lane holds float4 groups c = lane*4 + i*256.  NV > 0:
// exactly NV groups per lane (d_model = 256*NV, no bounds tests); NV == 0:
// up to kMaxV4 groups with tests.
template <typename T, int NV>
__global__ __launch_bounds__(256) void layernorm_kernel(const float* x, const float* __restrict__ gamma,
                                                         const float* __restrict__ beta, T* __restrict__ y,
                                                         float* y32, int M, int D, float eps,
                                                         const u32x4_t* __restrict__ pf, size_t pf16) {
  constexpr int NMAX = NV > 0 ? NV : kMaxV4;
  // Optional read-ahead of the next GEMMs' weights (pf16 16-byte chunks),
  // spread over the grid; the values are discarded.
  if (pf16) {
    u32x4_t acc = {0u, 0u, 0u, 0u};
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < pf16; i += (size_t)gridDim.x * 256) acc ^= pf[i];
    asm volatile("" ::"v"(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]));
  }
  const int row = xcd_block(blockIdx.x, gridDim.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;
  const float* xr = x + (size_t)row * D;
  float4 v[NMAX], gv[NMAX], bv[NMAX];
#pragma unroll
  for (int i = 0; i < NMAX; ++i)
    if (NV > 0 || lane * 4 + i * 256 < D) {
      v[i] = *reinterpret_cast<const float4*>(xr + lane * 4 + i * 256);
      gv[i] = *reinterpret_cast<const float4*>(gamma + lane * 4 + i * 256);
      bv[i] = *reinterpret_cast<const float4*>(beta + lane * 4 + i * 256);
    }
  layernorm_row<T, NV>(v, gv, bv, lane, row, D, eps, y, y32);
}

// embed_kernel and layernorm_kernel in one pass (d_model = 256 * NV): the
// row x = wte[id] + wpe[pos] is stored, then normalised from the registers
// holding it, by layernorm_row as in layernorm_kernel (same bits), after the
// same optional read-ahead of the following GEMMs' weights.
template <typename T, int NV>
__global__ __launch_bounds__(256) void embed_layernorm_kernel(const int32_t* __restrict__ ids,
                                                               const T* __restrict__ wte, const T* __restrict__ wpe,
                                                               float* __restrict__ x, int M, int T_seq, int pos0,
                                                               int D, int V, int32_t* __restrict__ bad,
                                                               const float* __restrict__ gamma,
                                                               const float* __restrict__ beta, T* __restrict__ y,
                                                               float eps, const u32x4_t* __restrict__ pf,
                                                               size_t pf16) {
  static_assert(NV > 0, "whole 256-column groups");
  if (pf16) {
    u32x4_t acc = {0u, 0u, 0u, 0u};
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < pf16; i += (size_t)gridDim.x * 256) acc ^= pf[i];
    asm volatile("" ::"v"(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]));
  }
  const int row = xcd_block(blockIdx.x, gridDim.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;
  const int raw = ids[row];
  const int id = clamp_token_id(raw, V);
  if (bad && id != raw && lane == 0) *bad = 1;
  const int pos = pos0 + row % T_seq;
  const T* we = wte + (size_t)id * D;
  const T* pe = wpe + (size_t)pos * D;
  float* xr = x + (size_t)row * D;
  float4 v[NV], gv[NV], bv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const float4 a = Elem<T>::load4(we + lane * 4 + i * 256);
    const float4 b = Elem<T>::load4(pe + lane * 4 + i * 256);
    v[i] = make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
    gv[i] = *reinterpret_cast<const float4*>(gamma + lane * 4 + i * 256);
    bv[i] = *reinterpret_cast<const float4*>(beta + lane * 4 + i * 256);
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) *reinterpret_cast<float4*>(xr + lane * 4 + i * 256) = v[i];
  layernorm_row<T, NV>(v, gv, bv, lane, row, D, eps, y, nullptr);
}

// Residual add fused in front of the LayerNorm, for few rows: one block of
// four waves per row.  x += (sum over s of rpart[s][row] + rbias) is written
// back, then normalised.  Wave w sums the contiguous slices
// [w*q, min((w+1)*q, rks)), q = ceil(rks/4), in increasing s; wave 0 adds the
// four wave sums in order w = 0..3 (so the result does not depend on timing).
template <typename T, int NV>
__global__ __launch_bounds__(256) void layernorm_residual_kernel(float* x,
                                                                  const float* __restrict__ gamma,
                                                                  const float* __restrict__ beta, T* __restrict__ y,
                                                                  float* y32, int M, int D, float eps,
                                                                  const float* __restrict__ rpart, int rks,
                                                                  const float* __restrict__ rbias) {
  constexpr int NMAX = NV > 0 ? NV : kMaxV4;
  __shared__ float4 red[3][NMAX][64];
  const int row = blockIdx.x;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  auto valid = [&](int i) { return NV > 0 || lane * 4 + i * 256 < D; };
  const int q = (rks + 3) / 4;
  const int s0 = w * q, s1 = min(s0 + q, rks);
  const size_t sstride = (size_t)M * D;
  const float* pr = rpart + (size_t)row * D;
  float4 acc[NMAX];
#pragma unroll
  for (int i = 0; i < NMAX; ++i) acc[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (s0 < s1) {
#pragma unroll
    for (int i = 0; i < NMAX; ++i)
      if (valid(i)) acc[i] = *reinterpret_cast<const float4*>(pr + s0 * sstride + lane * 4 + i * 256);
    for (int s = s0 + 1; s < s1; ++s) {
      float4 p[NMAX];
#pragma unroll
      for (int i = 0; i < NMAX; ++i)
        if (valid(i)) p[i] = *reinterpret_cast<const float4*>(pr + s * sstride + lane * 4 + i * 256);
#pragma unroll
      for (int i = 0; i < NMAX; ++i)
        if (valid(i)) acc[i] = make_float4(acc[i].x + p[i].x, acc[i].y + p[i].y, acc[i].z + p[i].z, acc[i].w + p[i].w);
    }
  }
  if (w > 0) {
#pragma unroll
    for (int i = 0; i < NMAX; ++i) red[w - 1][i][lane] = acc[i];
  }
  __syncthreads();
  if (w > 0) return;
  float* xr = x + (size_t)row * D;
  float4 v[NMAX], gv[NMAX], bv[NMAX];
#pragma unroll
  for (int i = 0; i < NMAX; ++i)
    if (valid(i)) {
      const int c = lane * 4 + i * 256;
      float4 a = acc[i];
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const float4 b = red[j][i][lane];
        a = make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
      }
      const float4 rb = *reinterpret_cast<const float4*>(rbias + c);
      const float4 x0 = *reinterpret_cast<const float4*>(xr + c);
      v[i] = make_float4(x0.x + (a.x + rb.x), x0.y + (a.y + rb.y), x0.z + (a.z + rb.z), x0.w + (a.w + rb.w));
      *reinterpret_cast<float4*>(xr + c) = v[i];
      gv[i] = *reinterpret_cast<const float4*>(gamma + c);
      bv[i] = *reinterpret_cast<const float4*>(beta + c);
    }
  layernorm_row<T, NV>(v, gv, bv, lane, row, D, eps, y, y32);
}

// 32x32 tile transpose through LDS; 256 threads = 32 x 8.
template <typename T>
__global__ __launch_bounds__(256) void transpose_convert_kernel(const float* __restrict__ src, T* __restrict__ dst,
                                                                 int K, int N, int N_pad) {
  __shared__ float tile[32][33];
  const int n0 = blockIdx.x * 32, k0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int r = ty; r < 32; r += 8) {
    const int kk = k0 + r, nn = n0 + tx;
    tile[r][tx] = (kk < K && nn < N) ? src[(size_t)kk * N + nn] : 0.f;
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int nn = n0 + r, kk = k0 + tx;
    if (nn < N_pad && kk < K) dst[(size_t)nn * K + kk] = Elem<T>::from_f32(tile[tx][r]);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void convert_kernel(const float* __restrict__ src, T* __restrict__ dst, size_t n,
                                                       size_t n_pad) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n_pad; i += (size_t)gridDim.x * 256)
    dst[i] = Elem<T>::from_f32(i < n ? src[i] : 0.f);
}

// Per-position next-token loss from the lm_head partials (EpiCE): one wave
// per scored position p = b*(T-1) + t (row m = b*T + t of the product).
// Lane l combines slices l, l+64, ... into (max, sum) online -- slices with
// no valid column carry sum 0 and are skipped -- then the wave takes the
// maximum M and S = sum of sum_l * exp(max_l - M):
//   loss = M + log(S) - C[m][label]   (log-sum-exp minus the label's logit).
// Negative labels give 0 (not scored), labels >= V give NaN.
__global__ __launch_bounds__(256) void ce_rows_kernel(const float2* __restrict__ part, int nseg,
                                                       const float* __restrict__ tgt,
                                                       const int32_t* __restrict__ labels, int B, int T, int V,
                                                       float* __restrict__ loss) {
  const int p = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (p >= B * (T - 1)) return;
  const int b = p / (T - 1), t = p - b * (T - 1);
  const int m = b * T + t;
  const int label = labels[m + 1];
  const float2* pr = part + (size_t)m * nseg;
  float mx = -INFINITY, s = 0.f;
  for (int i = lane; i < nseg; i += 64) {
    const float2 q = pr[i];
    if (q.y > 0.f) {
      if (q.x > mx) {
        s = s * __builtin_amdgcn_exp2f((mx - q.x) * kLog2e) + q.y;
        mx = q.x;
      } else {
        s += q.y * __builtin_amdgcn_exp2f((q.x - mx) * kLog2e);
      }
    }
  }
  const float M = wave_max(mx);
  const float S = wave_sum(s > 0.f ? s * __builtin_amdgcn_exp2f((mx - M) * kLog2e) : 0.f);
  if (lane == 0) {
    float v;
    if (label < 0) v = 0.f;
    else if (label >= V) v = __builtin_nanf("");
    else v = M + logf(S) - tgt[m];
    loss[p] = v;
  }
}

// Mean over the scored positions (labels >= 0) of loss[B*(T-1)], one block,
// fixed summation order; NaN when nothing is scored.
__global__ __launch_bounds__(1024) void ce_mean_kernel(const float* __restrict__ loss,
                                                        const int32_t* __restrict__ labels, int B, int T,
                                                        float* __restrict__ out) {
  __shared__ float ssum[16], scnt[16];
  const int n = B * (T - 1);
  float s = 0.f, c = 0.f;
  for (int p = threadIdx.x; p < n; p += 1024) {
    const int b = p / (T - 1), t = p - b * (T - 1);
    if (labels[b * T + t + 1] >= 0) {
      s += loss[p];
      c += 1.f;
    }
  }
  s = wave_sum(s);
  c = wave_sum(c);
  if ((threadIdx.x & 63) == 0) {
    ssum[threadIdx.x >> 6] = s;
    scnt[threadIdx.x >> 6] = c;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float ts = 0.f, tc = 0.f;
    for (int w = 0; w < 16; ++w) {
      ts += ssum[w];
      tc += scnt[w];
    }
    out[0] = ts / tc;
  }
}

// Greedy token per row from the lm_head's EpiArgmax partials: one wave per
// row; lane l scans slices l, l+64, ... in increasing order (strictly larger
// replaces, so the first maximum stays), then the lanes combine pairs
// (larger value, then smaller column).  A row with no ordered value (all NaN)
// gets token 0, so the next step's embedding gather stays inside wte.
__global__ __launch_bounds__(256) void argmax_rows_kernel(const int2* __restrict__ part, int nseg, int M, int V,
                                                           int32_t* __restrict__ out, int out_stride,
                                                           int32_t* __restrict__ next) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;
  const int2* pr = part + (size_t)row * nseg;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  // eight slices per lane requested at once (past the end: the last slice
  // again, not compared), then compared in increasing order
  constexpr int U = 8;
  for (int s0 = lane; s0 < nseg; s0 += 64 * U) {
    int2 q[U];
#pragma unroll
    for (int u = 0; u < U; ++u) q[u] = pr[min(s0 + 64 * u, nseg - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float v = __builtin_bit_cast(float, q[u].x);
      if (s0 + 64 * u < nseg && v > best) {
        best = v;
        bi = q[u].y;
      }
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float v2 = __shfl_xor(best, o, 64);
    const int i2 = __shfl_xor(bi, o, 64);
    if (v2 > best || (v2 == best && i2 < bi)) {
      best = v2;
      bi = i2;
    }
  }
  if (lane == 0) {
    const int tok = (bi >= 0 && bi < V) ? bi : 0;
    out[(size_t)row * out_stride] = tok;
    next[row] = tok;
  }
}

}  // namespace

hipError_t launch_argmax_rows(const int2* part, int nseg, int M, int V, int32_t* out, int out_stride, int32_t* next,
                              hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL(argmax_rows_kernel, dim3((M + 3) / 4), dim3(256), 0, stream, part, nseg, M, V, out, out_stride,
                     next);
  return hipGetLastError();
}

hipError_t launch_ce_rows(const float2* part, int nseg, const float* tgt, const int32_t* labels, int B, int T, int V,
                          float* loss, hipStream_t stream) {
  const int n = B * (T - 1);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(ce_rows_kernel, dim3((n + 3) / 4), dim3(256), 0, stream, part, nseg, tgt, labels, B, T, V,
                     loss);
  return hipGetLastError();
}

hipError_t launch_ce_mean(const float* loss, const int32_t* labels, int B, int T, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(ce_mean_kernel, dim3(1), dim3(1024), 0, stream, loss, labels, B, T, out);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_embed(const int32_t* ids, const T* wte, const T* wpe, float* x, int M, int T_seq, int pos0, int D,
                        int V, int32_t* bad, hipStream_t stream) {
  if (V < 1) return hipErrorInvalidValue;
  const dim3 grid((M + 3) / 4), block(256);
  if (D == 768)
    hipLaunchKernelGGL((embed_kernel<T, 3>), grid, block, 0, stream, ids, wte, wpe, x, M, T_seq, pos0, D, V, bad);
  else if (D == 1024)
    hipLaunchKernelGGL((embed_kernel<T, 4>), grid, block, 0, stream, ids, wte, wpe, x, M, T_seq, pos0, D, V, bad);
  else
    hipLaunchKernelGGL((embed_kernel<T, 0>), grid, block, 0, stream, ids, wte, wpe, x, M, T_seq, pos0, D, V, bad);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_layernorm(float* x, const float* gamma, const float* beta, T* y, float* y32, int M, int D,
                            float eps, hipStream_t stream, const void* prefetch, size_t prefetch_bytes,
                            const float* rpart, int rks, const float* rbias) {
  if (D > 256 * kMaxV4 || D % 4 != 0) return hipErrorInvalidValue;
  if (M == 0) return hipSuccess;
  if (rpart) {
    if (rks < 1 || !rbias || prefetch) return hipErrorInvalidValue;
    const dim3 grid(M), block(256);
    switch (D) {
      case 768:
        hipLaunchKernelGGL((layernorm_residual_kernel<T, 3>), grid, block, 0, stream, x, gamma, beta, y, y32, M, D,
                           eps, rpart, rks, rbias);
        break;
      case 1024:
        hipLaunchKernelGGL((layernorm_residual_kernel<T, 4>), grid, block, 0, stream, x, gamma, beta, y, y32, M, D,
                           eps, rpart, rks, rbias);
        break;
      default:
        hipLaunchKernelGGL((layernorm_residual_kernel<T, 0>), grid, block, 0, stream, x, gamma, beta, y, y32, M, D,
                           eps, rpart, rks, rbias);
    }
    return hipGetLastError();
  }
  const dim3 grid((M + 3) / 4), block(256);
  const u32x4_t* pf = static_cast<const u32x4_t*>(prefetch);
  const size_t pf16 = prefetch ? prefetch_bytes / 16 : 0;
  switch (D) {
    case 768:
      hipLaunchKernelGGL((layernorm_kernel<T, 3>), grid, block, 0, stream, x, gamma, beta, y, y32, M, D, eps, pf,
                         pf16);
      break;
    case 1024:
      hipLaunchKernelGGL((layernorm_kernel<T, 4>), grid, block, 0, stream, x, gamma, beta, y, y32, M, D, eps, pf,
                         pf16);
      break;
    default:
      hipLaunchKernelGGL((layernorm_kernel<T, 0>), grid, block, 0, stream, x, gamma, beta, y, y32, M, D, eps, pf,
                         pf16);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_transpose_convert(const float* src, T* dst, int K, int N, int N_pad, hipStream_t stream) {
  dim3 grid((N_pad + 31) / 32, (K + 31) / 32);
  hipLaunchKernelGGL(transpose_convert_kernel<T>, grid, dim3(256), 0, stream, src, dst, K, N, N_pad);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_convert(const float* src, T* dst, size_t n, size_t n_pad, hipStream_t stream) {
  size_t blocks = (n_pad + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(convert_kernel<T>, dim3((unsigned)blocks), dim3(256), 0, stream, src, dst, n, n_pad);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_embed_layernorm(const int32_t* ids, const T* wte, const T* wpe, float* x, int M, int T_seq,
                                  int pos0, int D, int V, int32_t* bad, const float* gamma, const float* beta, T* y,
                                  float eps, hipStream_t stream, const void* prefetch, size_t prefetch_bytes) {
  if (V < 1) return hipErrorInvalidValue;
  if (D != 768 && D != 1024) {
    hipError_t e = launch_embed<T>(ids, wte, wpe, x, M, T_seq, pos0, D, V, bad, stream);
    if (e != hipSuccess) return e;
    return launch_layernorm<T>(x, gamma, beta, y, nullptr, M, D, eps, stream, prefetch, prefetch_bytes);
  }
  if (M == 0) return hipSuccess;
  const dim3 grid((M + 3) / 4), block(256);
  const u32x4_t* pf = static_cast<const u32x4_t*>(prefetch);
  const size_t pf16 = prefetch ? prefetch_bytes / 16 : 0;
  if (D == 768)
    hipLaunchKernelGGL((embed_layernorm_kernel<T, 3>), grid, block, 0, stream, ids, wte, wpe, x, M, T_seq, pos0, D, V,
                       bad, gamma, beta, y, eps, pf, pf16);
  else
    hipLaunchKernelGGL((embed_layernorm_kernel<T, 4>), grid, block, 0, stream, ids, wte, wpe, x, M, T_seq, pos0, D, V,
                       bad, gamma, beta, y, eps, pf, pf16);
  return hipGetLastError();
}

#define GPT2_ROWOPS(T)                                                                                          \
  template hipError_t launch_embed<T>(const int32_t*, const T*, const T*, float*, int, int, int, int, int, int32_t*,  \
                                      hipStream_t);                                                                 \
  template hipError_t launch_layernorm<T>(float*, const float*, const float*, T*, float*, int, int, float,          \
                                          hipStream_t, const void*, size_t, const float*, int, const float*);       \
  template hipError_t launch_embed_layernorm<T>(const int32_t*, const T*, const T*, float*, int, int, int, int, int, \
                                                int32_t*, const float*, const float*, T*, float, hipStream_t,     \
                                                const void*, size_t);                                               \
  template hipError_t launch_transpose_convert<T>(const float*, T*, int, int, int, hipStream_t);                   \
  template hipError_t launch_convert<T>(const float*, T*, size_t, size_t, hipStream_t);

GPT2_ROWOPS(float)
GPT2_ROWOPS(bf16_t)

}  // namespace gpt2
