// Block backward kernels (see backward.h).
#include "backward.h"

#include <algorithm>
#include <type_traits>

namespace gpt2 {

namespace {

// Row chunks of the first column-sum pass: 256 chunks of 32 rows at B*T =
// 8192 give a 768-column fp32 sum 768 blocks (3 per CU); with 64 chunks its
// 192 blocks kept too few loads in flight (2.9 TB/s).
constexpr int kColChunks = 256;
constexpr int kColFinalBatch = 32;  // partials per column a thread of the second pass has in flight
constexpr int kColBatch = 8;    // rows per thread with loads in flight together

// 32x32 tile transpose through LDS; 256 threads = 32 x 8.  Tiles cover dst
// rows c and dst columns r < ld_dst (the padding columns are written as 0).
template <typename Tin, typename Tout>
__global__ __launch_bounds__(256) void transpose_kernel(const Tin* __restrict__ src, int R, int C,
                                                         Tout* __restrict__ dst, int ld_dst) {
  __shared__ float tile[32][33];
  const int r0 = blockIdx.x * 32, c0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int i = ty; i < 32; i += 8) {
    const int r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < R && c < C) ? Elem<Tin>::to_f32(src[(size_t)r * C + c]) : 0.f;
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int c = c0 + i, r = r0 + tx;
    if (c < C && r < ld_dst) dst[(size_t)c * ld_dst + r] = Elem<Tout>::from_f32(tile[tx][i]);
  }
}

// bf16 -> bf16 transpose on 64x64 tiles with 16-byte global accesses:
// thread t reads 8 consecutive elements (16 bytes) of source row t/8 (+32),
// and writes 8 consecutive destination elements, i.e. one source column over
// 8 consecutive source rows, gathered from the LDS tile.  Needs C and ld_dst
// multiples of 8 and 16-byte aligned pointers; rows r >= R read as 0, so the
// destination columns R .. ld_dst-1 receive zeros.  A tile row is 64 + 2
// elements (132 bytes) so the column gathers of one read instruction fall in
// different banks.
__global__ __launch_bounds__(256) void transpose64_bf16_kernel(const bf16_t* __restrict__ src, int R, int C,
                                                                bf16_t* __restrict__ dst, int ld_dst) {
  __shared__ uint16_t tile[64][66];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int tid = threadIdx.x, cc = (tid & 7) * 8;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int row = (tid >> 3) + 32 * p, r = r0 + row, c = c0 + cc;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (r < R && c < C) v = *reinterpret_cast<const u32x4_t*>(src + (size_t)r * C + c);
    uint32_t* t = reinterpret_cast<uint32_t*>(&tile[row][cc]);
    t[0] = v[0];
    t[1] = v[1];
    t[2] = v[2];
    t[3] = v[3];
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int col = (tid >> 3) + 32 * p, c = c0 + col, r = r0 + cc;  // 8 source rows r .. r+7 of column c
    if (c >= C || r >= ld_dst) continue;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = (uint32_t)tile[cc + 2 * e][col] | ((uint32_t)tile[cc + 2 * e + 1][col] << 16);
    *reinterpret_cast<u32x4_t*>(dst + (size_t)c * ld_dst + r) = u32x4_t{w[0], w[1], w[2], w[3]};
  }
}

// First pass: block (column block nb, row chunk rc); 256 threads = 4 row
// lanes x 64 columns; lane ry adds rows ry, ry+4, ... of the chunk in order,
// then the four lane sums are added in order.
template <typename Tin, bool kXhat>
__global__ __launch_bounds__(256) void colsum_partial_kernel(const Tin* __restrict__ src, int M, int N,
                                                              float* __restrict__ part, const float* __restrict__ x,
                                                              const float* __restrict__ mu,
                                                              const float* __restrict__ rstd) {
  __shared__ float red[4][64];
  const int cx = threadIdx.x & 63, ry = threadIdx.x >> 6;
  const int n = blockIdx.x * 64 + cx, rc = blockIdx.y;
  const int rows = (M + kColChunks - 1) / kColChunks;
  const int m0 = rc * rows, m1 = min(M, m0 + rows);
  float s = 0.f;
  if (n < N) {
    for (int m = m0 + ry; m < m1; m += 4) {
      float v = Elem<Tin>::to_f32(src[(size_t)m * N + n]);
      if constexpr (kXhat) v *= (x[(size_t)m * N + n] - mu[m]) * rstd[m];
      s += v;
    }
  }
  red[ry][cx] = s;
  __syncthreads();
  if (ry == 0 && n < N) part[(size_t)rc * N + n] = ((red[0][cx] + red[1][cx]) + red[2][cx]) + red[3][cx];
}

// As colsum_partial_kernel with VEC consecutive columns per thread read as
// one 16-byte load (8 bf16 or 4 fp32): the block covers 64*VEC columns, and
// every column is summed in the same order as there (rows ry, ry+4, ... of
// the chunk, then the four lane sums in order), so the result is the same.
// Needs N % VEC == 0 and 16-byte aligned rows.  With part2 given (x-hat
// form only) the same pass also writes the plain sums of src to part2 (the
// LayerNorm gamma and beta gradients from one read of the row gradient).
template <typename Tin, bool kXhat>
__global__ __launch_bounds__(256) void colsum_partial_vec_kernel(const Tin* __restrict__ src, int M, int N,
                                                                  float* __restrict__ part, const float* __restrict__ x,
                                                                  const float* __restrict__ mu,
                                                                  const float* __restrict__ rstd,
                                                                  float* __restrict__ part2) {
  constexpr int VEC = 16 / (int)sizeof(Tin);
  __shared__ float red[4][64 * VEC];
  __shared__ float red2[kXhat ? 4 : 1][kXhat ? 64 * VEC : 1];
  float s2[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) s2[e] = 0.f;
  const int cx = threadIdx.x & 63, ry = threadIdx.x >> 6;
  const int n = (blockIdx.x * 64 + cx) * VEC, rc = blockIdx.y;
  const int rows = (M + kColChunks - 1) / kColChunks;
  const int m0 = rc * rows, m1 = min(M, m0 + rows);
  float s[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) s[e] = 0.f;
  if (n < N && m0 + ry < m1) {
    // kColBatch rows per thread in flight: every load unconditional (rows past
    // the chunk read its last row), rows past the chunk add 0 (s never holds
    // -0, so the sums keep their bits), the additions in row order as before
    constexpr int U = kColBatch;
    for (int m = m0 + ry; m < m1; m += 4 * U) {
      u32x4_t raw[U];
      f32x4_t xr[kXhat ? U : 1];
      float mmv[kXhat ? U : 1], rsv[kXhat ? U : 1];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int mc = min(m + 4 * u, m1 - 1);
        raw[u] = *reinterpret_cast<const u32x4_t*>(src + (size_t)mc * N + n);
        if constexpr (kXhat) {
          xr[u] = *reinterpret_cast<const f32x4_t*>(x + (size_t)mc * N + n);
          mmv[u] = mu[mc];
          rsv[u] = rstd[mc];
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // the batch's loads before its first use
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool on = m + 4 * u < m1;
        float v[VEC];
        if constexpr (sizeof(Tin) == 2) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[2 * e] = bf16_to_f32(raw[u][e] & 0xFFFF);
            v[2 * e + 1] = bf16_to_f32(raw[u][e] >> 16);
          }
        } else {
          const f32x4_t f = __builtin_bit_cast(f32x4_t, raw[u]);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = f[e];
        }
        if constexpr (kXhat) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            s2[e] += on ? v[e] : 0.f;
            v[e] *= (xr[u][e] - mmv[u]) * rsv[u];
          }
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) s[e] += on ? v[e] : 0.f;
      }
    }
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) red[ry][cx * VEC + e] = s[e];
  if constexpr (kXhat) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) red2[ry][cx * VEC + e] = s2[e];
  }
  __syncthreads();
  if (ry == 0 && n < N) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const int j = cx * VEC + e;
      part[(size_t)rc * N + n + e] = ((red[0][j] + red[1][j]) + red[2][j]) + red[3][j];
      if constexpr (kXhat) {
        if (part2) part2[(size_t)rc * N + n + e] = ((red2[0][j] + red2[1][j]) + red2[2][j]) + red2[3][j];
      }
    }
  }
}

// Second pass: out[n] = sum over the kColChunks partials part[rc][n].  A
// block takes 64 columns with 4 threads each: thread group g sums chunks
// g*Q .. (g+1)*Q - 1 in increasing rc (Q = kColChunks / 4, loads in flight
// kColFinalBatch at a time), then the four group sums are added in order g =
// 0..3, so the result does not depend on timing.
constexpr int kColFinalGroups = 4;
__device__ __forceinline__ void sum_chunks_block(const float* __restrict__ part, int N, float* __restrict__ out) {
  constexpr int Q = kColChunks / kColFinalGroups;
  static_assert(Q % kColFinalBatch == 0, "whole batches");
  __shared__ float red[kColFinalGroups][64];
  const int c = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int n = blockIdx.x * 64 + c;
  float s = 0.f;
  if (n < N) {
    for (int rc0 = g * Q; rc0 < (g + 1) * Q; rc0 += kColFinalBatch) {
      float v[kColFinalBatch];
#pragma unroll
      for (int u = 0; u < kColFinalBatch; ++u) v[u] = part[(size_t)(rc0 + u) * N + n];
#pragma unroll
      for (int u = 0; u < kColFinalBatch; ++u) s += v[u];
    }
  }
  red[g][c] = s;
  __syncthreads();
  if (g == 0 && n < N) out[n] = ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c];
}

// Second pass for several column sums in one launch (blockIdx.y = job), each
// summed as in sum_chunks_block.
struct ColsumFinalArgs {
  ColsumJob job[kMaxColsumJobs];
};
__global__ __launch_bounds__(256) void colsum_final_group_kernel(ColsumFinalArgs a) {
  const ColsumJob j = a.job[blockIdx.y];
  if ((int)blockIdx.x * 64 >= j.N) return;  // block-uniform
  sum_chunks_block(j.part, j.N, j.out);
}

__global__ __launch_bounds__(256) void colsum_final_kernel(const float* __restrict__ part, int N,
                                                            float* __restrict__ out) {
  sum_chunks_block(part, N, out);
}

// One wave per row; lane holds float4 groups c = lane*4 + i*256 (as the
// forward LayerNorm).
template <typename T, int NV>
__global__ __launch_bounds__(256) void layernorm_backward_kernel(
    const float* __restrict__ x, const float* __restrict__ dh, const float* __restrict__ gamma,
    const float* __restrict__ resid, float* __restrict__ out, T* __restrict__ out_t, float* __restrict__ mu_out,
    float* __restrict__ rstd_out, int M, int D, float eps) {
  constexpr int kMax = 8;
  constexpr int NMAX = NV > 0 ? NV : kMax;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;
  auto valid = [&](int i) { return NV > 0 || lane * 4 + i * 256 < D; };
  const size_t base = (size_t)row * D;
  float4 xv[NMAX], gv[NMAX];
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < NMAX; ++i)
    if (valid(i)) {
      xv[i] = *reinterpret_cast<const float4*>(x + base + lane * 4 + i * 256);
      sum += (xv[i].x + xv[i].y) + (xv[i].z + xv[i].w);
    }
  const float mu = wave_sum(sum) / (float)D;
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < NMAX; ++i)
    if (valid(i)) {
      xv[i] = make_float4(xv[i].x - mu, xv[i].y - mu, xv[i].z - mu, xv[i].w - mu);
      sq += (xv[i].x * xv[i].x + xv[i].y * xv[i].y) + (xv[i].z * xv[i].z + xv[i].w * xv[i].w);
    }
  const float rstd = 1.0f / sqrtf(wave_sum(sq) / (float)D + eps);
  // g = dh * gamma; a = mean(g), b = mean(g * xhat)
  float sa = 0.f, sb = 0.f;
#pragma unroll
  for (int i = 0; i < NMAX; ++i)
    if (valid(i)) {
      const int c = lane * 4 + i * 256;
      const float4 d = *reinterpret_cast<const float4*>(dh + base + c);
      const float4 gm = *reinterpret_cast<const float4*>(gamma + c);
      gv[i] = make_float4(d.x * gm.x, d.y * gm.y, d.z * gm.z, d.w * gm.w);
      xv[i] = make_float4(xv[i].x * rstd, xv[i].y * rstd, xv[i].z * rstd, xv[i].w * rstd);  // xhat
      sa += (gv[i].x + gv[i].y) + (gv[i].z + gv[i].w);
      sb += (gv[i].x * xv[i].x + gv[i].y * xv[i].y) + (gv[i].z * xv[i].z + gv[i].w * xv[i].w);
    }
  const float a = wave_sum(sa) / (float)D, bm = wave_sum(sb) / (float)D;
#pragma unroll
  for (int i = 0; i < NMAX; ++i)
    if (valid(i)) {
      const int c = lane * 4 + i * 256;
      const float4 r = *reinterpret_cast<const float4*>(resid + base + c);
      const float4 o = make_float4(r.x + rstd * (gv[i].x - a - xv[i].x * bm), r.y + rstd * (gv[i].y - a - xv[i].y * bm),
                                   r.z + rstd * (gv[i].z - a - xv[i].z * bm), r.w + rstd * (gv[i].w - a - xv[i].w * bm));
      *reinterpret_cast<float4*>(out + base + c) = o;
      if (out_t) Elem<T>::store4(out_t + base + c, o.x, o.y, o.z, o.w);
    }
  if (lane == 0) {
    if (mu_out) mu_out[row] = mu;
    if (rstd_out) rstd_out[row] = rstd;
  }
}

// dvec[bh][i] = sum_d dout[b*T + i][h*HS + d] * o[b*T + i][h*HS + d]: one wave per (bh, i).
template <typename T, int HS>
__global__ __launch_bounds__(256) void attn_bwd_dvec_kernel(const T* __restrict__ o, const T* __restrict__ dout,
                                                             float* __restrict__ dvec, int B, int H, int T_seq) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= B * H * T_seq) return;
  const int bh = r / T_seq, i = r - bh * T_seq;
  const int b = bh / H, h = bh - b * H;
  const size_t off = ((size_t)b * T_seq + i) * (H * HS) + h * HS + lane;
  const float v = lane < HS ? Elem<T>::to_f32(dout[off]) * Elem<T>::to_f32(o[off]) : 0.f;
  const float s = wave_sum(v);
  if (lane == 0) dvec[r] = s;
}

// bf16 rows of 64: eight lanes per row, 16 bytes each (eight products added
// in order, then the eight lane sums by xor shuffles), 32 rows per block.
__global__ __launch_bounds__(256) void attn_bwd_dvec_bf16_kernel(const bf16_t* __restrict__ o,
                                                                 const bf16_t* __restrict__ dout,
                                                                 float* __restrict__ dvec, int B, int H, int T_seq) {
  const int r = blockIdx.x * 32 + (threadIdx.x >> 3);
  const int sub = threadIdx.x & 7;
  const bool on = r < B * H * T_seq;
  const int rr = on ? r : 0;
  const int bh = rr / T_seq, i = rr - bh * T_seq;
  const int b = bh / H, h = bh - b * H;
  const size_t off = ((size_t)b * T_seq + i) * (H * 64) + h * 64 + sub * 8;
  const u32x4_t a = *reinterpret_cast<const u32x4_t*>(dout + off);
  const u32x4_t c = *reinterpret_cast<const u32x4_t*>(o + off);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    s += __uint_as_float(a[e] << 16) * __uint_as_float(c[e] << 16);
    s += __uint_as_float(a[e] & 0xFFFF0000u) * __uint_as_float(c[e] & 0xFFFF0000u);
  }
  s += __shfl_xor(s, 1, 8);
  s += __shfl_xor(s, 2, 8);
  s += __shfl_xor(s, 4, 8);
  if (on && sub == 0) dvec[r] = s;
}

constexpr int kBT = 64;  // keys per key tile, queries per query tile

// Shared pieces of the two attention-backward kernels: 256 threads,
// ty = tid / 16 owns rows ty*4 .. +3 of a 64 x 64 score tile, tx = tid % 16
// its columns tx*4 .. +3.
template <int HS>
struct AttnBwdSmem {
  float Ks[kBT][HS + 1];
  float Vs[kBT][HS + 1];
  float Qs[kBT][HS + 1];
  float dOs[kBT][HS + 1];
  float Ps[kBT][kBT + 1];
  float dSs[kBT][kBT + 1];
  float lse[kBT];
  float dv[kBT];
};

template <typename T, int HS>
__device__ __forceinline__ void load_kv_tile(AttnBwdSmem<HS>& sm, const T* k, const T* vt, int bh, int kvT, int j0,
                                             int T_seq) {
  for (int e = threadIdx.x; e < kBT * HS; e += 256) {
    const int j = e / HS, d = e - j * HS;  // K rows are HS-contiguous
    sm.Ks[j][d] = j0 + j < T_seq ? Elem<T>::to_f32(k[((size_t)bh * kvT + j0 + j) * HS + d]) : 0.f;
  }
  for (int e = threadIdx.x; e < kBT * HS; e += 256) {
    const int d = e / kBT, j = e - d * kBT;  // V^T rows are key-contiguous
    sm.Vs[j][d] = j0 + j < T_seq ? Elem<T>::to_f32(vt[((size_t)bh * HS + d) * kvT + j0 + j]) : 0.f;
  }
}

template <typename T, int HS>
__device__ __forceinline__ void load_q_tile(AttnBwdSmem<HS>& sm, const T* q, const T* dout, const float* lse,
                                            const float* dvec, int bh, int b, int h, int H, int i0, int T_seq) {
  for (int e = threadIdx.x; e < kBT * HS; e += 256) {
    const int i = e / HS, d = e - i * HS;
    const bool ok = i0 + i < T_seq;
    sm.Qs[i][d] = ok ? Elem<T>::to_f32(q[((size_t)bh * T_seq + i0 + i) * HS + d]) : 0.f;
    sm.dOs[i][d] = ok ? Elem<T>::to_f32(dout[((size_t)b * T_seq + i0 + i) * (H * HS) + h * HS + d]) : 0.f;
  }
  if (threadIdx.x < kBT) {
    const int i = threadIdx.x;
    const bool ok = i0 + i < T_seq;
    sm.lse[i] = ok ? lse[(size_t)bh * T_seq + i0 + i] : 0.f;
    sm.dv[i] = ok ? dvec[(size_t)bh * T_seq + i0 + i] : 0.f;
  }
}

// P and dS of the (query tile i0, key tile j0) pair into Ps / dSs: entries
// with key j > query i, or outside the sequence, are exactly 0.
template <int HS>
__device__ __forceinline__ void score_tiles(AttnBwdSmem<HS>& sm, int i0, int j0, int T_seq) {
  const int ty = threadIdx.x >> 4, tx = threadIdx.x & 15;
  float s[4][4] = {}, dp[4][4] = {};
#pragma unroll 4
  for (int d = 0; d < HS; ++d) {
    float qa[4], oa[4], kb[4], vb[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      qa[a] = sm.Qs[ty * 4 + a][d];
      oa[a] = sm.dOs[ty * 4 + a][d];
      kb[a] = sm.Ks[tx * 4 + a][d];
      vb[a] = sm.Vs[tx * 4 + a][d];
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        s[a][c] += qa[a] * kb[c];
        dp[a][c] += oa[a] * vb[c];
      }
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int ii = ty * 4 + a, jj = tx * 4 + c;
      const int i = i0 + ii, j = j0 + jj;
      const bool ok = j <= i && i < T_seq;
      const float p = ok ? __builtin_amdgcn_exp2f((s[a][c] - sm.lse[ii]) * kLog2e) : 0.f;
      sm.Ps[ii][jj] = p;
      sm.dSs[ii][jj] = ok ? p * (dp[a][c] - sm.dv[ii]) : 0.f;
    }
}

// dK and dV of one key tile: loops over the query tiles at or after it.
template <typename T, int HS>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                             const T* __restrict__ vt, const T* __restrict__ dout,
                                                             const float* __restrict__ lse,
                                                             const float* __restrict__ dvec, float* __restrict__ dqkv,
                                                             int H, int T_seq, int kvT, int n_tiles) {
  constexpr int DPT = HS / 16;
  __shared__ AttnBwdSmem<HS> sm;
  const int bh = blockIdx.x / n_tiles, kt = blockIdx.x - bh * n_tiles;
  const int b = bh / H, h = bh - b * H;
  const int j0 = kt * kBT;
  const int ty = threadIdx.x >> 4, tx = threadIdx.x & 15;
  load_kv_tile<T, HS>(sm, k, vt, bh, kvT, j0, T_seq);
  float dk[4][DPT] = {}, dv[4][DPT] = {};
  for (int qt = kt; qt < n_tiles; ++qt) {
    const int i0 = qt * kBT;
    __syncthreads();  // previous tile's readers are done
    load_q_tile<T, HS>(sm, q, dout, lse, dvec, bh, b, h, H, i0, T_seq);
    __syncthreads();
    score_tiles<HS>(sm, i0, j0, T_seq);
    __syncthreads();
    // dV[j][d] += sum_i P[i][j] dO[i][d];  dK[j][d] += sum_i dS[i][j] Q[i][d]
#pragma unroll 4
    for (int i = 0; i < kBT; ++i) {
      float pj[4], sj[4], od[DPT], qd[DPT];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        pj[a] = sm.Ps[i][ty * 4 + a];
        sj[a] = sm.dSs[i][ty * 4 + a];
      }
#pragma unroll
      for (int c = 0; c < DPT; ++c) {
        od[c] = sm.dOs[i][tx * DPT + c];
        qd[c] = sm.Qs[i][tx * DPT + c];
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < DPT; ++c) {
          dv[a][c] += pj[a] * od[c];
          dk[a][c] += sj[a] * qd[c];
        }
    }
  }
  const int Dm = H * HS;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int j = j0 + ty * 4 + a;
    if (j < T_seq) {
      float* row = dqkv + ((size_t)b * T_seq + j) * (3 * Dm) + h * HS + tx * DPT;
#pragma unroll
      for (int c = 0; c < DPT; ++c) {
        row[Dm + c] = dk[a][c];
        row[2 * Dm + c] = dv[a][c];
      }
    }
  }
}

// dQ of one query tile: loops over the key tiles at or before it.
template <typename T, int HS>
__global__ __launch_bounds__(256) void attn_bwd_dq_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                           const T* __restrict__ vt, const T* __restrict__ dout,
                                                           const float* __restrict__ lse,
                                                           const float* __restrict__ dvec, float* __restrict__ dqkv,
                                                           int H, int T_seq, int kvT, int n_tiles, float scale) {
  constexpr int DPT = HS / 16;
  __shared__ AttnBwdSmem<HS> sm;
  const int bh = blockIdx.x / n_tiles, qt = blockIdx.x - bh * n_tiles;
  const int b = bh / H, h = bh - b * H;
  const int i0 = qt * kBT;
  const int ty = threadIdx.x >> 4, tx = threadIdx.x & 15;
  load_q_tile<T, HS>(sm, q, dout, lse, dvec, bh, b, h, H, i0, T_seq);
  float dq[4][DPT] = {};
  for (int kt = 0; kt <= qt; ++kt) {
    const int j0 = kt * kBT;
    __syncthreads();
    load_kv_tile<T, HS>(sm, k, vt, bh, kvT, j0, T_seq);
    __syncthreads();
    score_tiles<HS>(sm, i0, j0, T_seq);
    __syncthreads();
    // dQ[i][d] += sum_j dS[i][j] K[j][d]
#pragma unroll 4
    for (int j = 0; j < kBT; ++j) {
      float sj[4], kd[DPT];
#pragma unroll
      for (int a = 0; a < 4; ++a) sj[a] = sm.dSs[ty * 4 + a][j];
#pragma unroll
      for (int c = 0; c < DPT; ++c) kd[c] = sm.Ks[j][tx * DPT + c];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < DPT; ++c) dq[a][c] += sj[a] * kd[c];
    }
  }
  const int Dm = H * HS;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int i = i0 + ty * 4 + a;
    if (i < T_seq) {
      float* row = dqkv + ((size_t)b * T_seq + i) * (3 * Dm) + h * HS + tx * DPT;
#pragma unroll
      for (int c = 0; c < DPT; ++c) row[c] = scale * dq[a][c];
    }
  }
}

// ----------------------------------------------------------- bf16, matrix cores
// Head size 64.  Each 64-row operand tile (Q, dO, K: rows of 64 d; V^T: rows
// of 64 keys) sits in LDS as 64 rows of 128 bytes, 16-byte chunk c of row r
// at slot c ^ (r & 7), filled by global_load_lds (one wave instruction = 8
// rows).  Fragments whose contraction index runs along a tile row are plain
// 16-byte reads; fragments whose contraction index runs down the rows are
// read with ds_read_b64_tr_b16 (tr_frag).  The probabilities P and dS stay
// in the registers of the MFMA that produced them: lane (lr, lg) of
// R = X Y^T holds R[4 lg + e][lr], and two 16-row blocks b, b + 1 give it
// rows 16 b + 4 lg + e and 16 (b + 1) + 4 lg + e -- the eight contraction
// slots 8 lg .. 8 lg + 7 of the next product, in the order pslot() names;
// the other operand of that product is read in the same order.
constexpr int kTileBytes = kBT * 128;
typedef short v4i16_t __attribute__((ext_vector_type(4)));

// s_waitcnt vmcnt(N) (N < 16) as the builtin, so the compiler's own wait
// insertion knows which loads it has retired.
template <int N>
__device__ __forceinline__ void wait_vmcnt_bwd() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(N | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ int pslot_row(int s2, int lg, int h) { return 32 * s2 + 16 * h + 4 * lg; }

__device__ __forceinline__ u32x4_t plain_frag(const char* tile, int row, int chunk) {
  return *reinterpret_cast<const u32x4_t*>(tile + row * 128 + ((chunk ^ (row & 7)) << 4));
}

// Four consecutive tile rows row0 .. row0 + 3 of column nb + lr (16-lane
// group semantics of ds_read_b64_tr_b16: lane l names row row0 + l / 4,
// columns nb + 4 (l % 4) .. +3; lane j receives X[row0 + t][nb + j]).
__device__ __forceinline__ u32x2_t tr4(const char* tile, int row0, int nb, int lr) {
  const int row = row0 + (lr >> 2), col = nb + 4 * (lr & 3);
  const char* addr = tile + row * 128 + (((col >> 3) ^ (row & 7)) << 4) + ((col >> 2) & 1) * 8;
  const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16_t*)(const_cast<char*>(addr)));
  return __builtin_bit_cast(u32x2_t, v);
}

// Fragment of column nb + lr over the rows r0 + t and r1 + t (t = 0..3).
__device__ __forceinline__ u32x4_t tr_frag(const char* tile, int r0, int r1, int nb, int lr) {
  const u32x2_t a = tr4(tile, r0, nb, lr), b = tr4(tile, r1, nb, lr);
  return u32x4_t{a[0], a[1], b[0], b[1]};
}

// 64 rows of 128 bytes into a swizzled LDS tile: wave instruction j of 2
// fills slots (2 w + j) * 64 + lane.  Source row r is src + min(r, last) * ld.
__device__ __forceinline__ void dma_tile(char* tile, const bf16_t* src, size_t ld, int last) {
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int si = (2 * w + j) * 64 + lane, row = si >> 3, c = (si & 7) ^ (row & 7);
    const bf16_t* g = src + (size_t)min(row, last) * ld + c * 8;
    __builtin_amdgcn_global_load_lds((const void*)g,
                                     (__attribute__((address_space(3))) void*)(tile + (2 * w + j) * 1024), 16, 0, 0);
  }
}

// A 64-row tile between its global read and its LDS write, so that the next
// tile's reads are in flight while the current one is computed (the loop
// issues no LDS DMA: with one in flight the compiler waits for it before
// every transposing read).  Thread t holds chunks 2 (t % 4) and +1 of row
// t / 4; source row r is src + min(r, last) * ld.
struct TileRegs {
  u32x4_t v[2];
};

__device__ __forceinline__ void fetch_tile(TileRegs& g, const bf16_t* src, size_t ld, int last) {
  const int row = threadIdx.x >> 2, c0 = (threadIdx.x & 3) * 2;
  const bf16_t* p = src + (size_t)min(row, last) * ld + c0 * 8;
  g.v[0] = *reinterpret_cast<const u32x4_t*>(p);
  g.v[1] = *reinterpret_cast<const u32x4_t*>(p + 8);
}

__device__ __forceinline__ void put_tile(char* tile, const TileRegs& g) {
  const int row = threadIdx.x >> 2, c0 = (threadIdx.x & 3) * 2;
#pragma unroll
  for (int j = 0; j < 2; ++j)
    *reinterpret_cast<u32x4_t*>(tile + row * 128 + (((c0 + j) ^ (row & 7)) << 4)) = g.v[j];
}

// dK and dV of one key tile (64 keys): wave w owns keys 16 w .. 16 w + 15,
// whose K and V rows it keeps as MFMA operands in registers.  Per query
// tile at or after it (Q and dO tiles double-buffered in LDS): S and dP of
// the 64 queries against the wave's keys, P = exp(S - lse) and
// dS = P (dP - dvec) (selected to 0 where the key follows the query or the
// query is past the end), then dV^T += dO^T P and dK^T += Q^T dS.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void attn_bwd_dkdv_reg_kernel(const bf16_t* __restrict__ q,
                                                                  const bf16_t* __restrict__ k,
                                                                  const bf16_t* __restrict__ vt,
                                                                  const bf16_t* __restrict__ dout,
                                                                  const float* __restrict__ lse,
                                                                  const float* __restrict__ dvec,
                                                                  float* __restrict__ dqkv, int BH, int H,
                                                                  int T_seq, int kvT, int n_tiles) {
  __shared__ __attribute__((aligned(16))) char sQ[2][kTileBytes];
  __shared__ __attribute__((aligned(16))) char sO[2][kTileBytes];
  __shared__ __attribute__((aligned(16))) float sL[2][kBT];
  __shared__ __attribute__((aligned(16))) float sD[2][kBT];
  // Key tile 0 (the longest) first; within every other run of 256 blocks the
  // order is reversed, so each CU's resident blocks mix long and short tiles.
  int widx = blockIdx.x;
  {
    const int run = widx >> 8, pos = widx & 255;
    if ((run & 1) && (run << 8) + 256 <= (int)gridDim.x) widx = (run << 8) + (255 - pos);
  }
  const int kt = widx / BH, bh = widx - kt * BH;
  const int b = bh / H, h = bh - b * H;
  const int j0 = kt * kBT;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int Dm = H * 64;
  const int key = j0 + 16 * w + lr;  // this lane's key (column of every S block)

  // V^T tile of the key tile -> V rows of the wave's keys (through sQ[1],
  // free until the second query tile); K rows straight from global.
  dma_tile(sQ[1], vt + (size_t)bh * 64 * kvT + j0, kvT, 63);
  u32x4_t kreg[2], vreg[2];
  {
    const bf16_t* kr = k + ((size_t)bh * kvT + min(key, T_seq - 1)) * 64;
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) kreg[sl] = *reinterpret_cast<const u32x4_t*>(kr + sl * 32 + lg * 8);
  }
  const float* lse_bh = lse + (size_t)bh * T_seq;
  const float* dv_bh = dvec + (size_t)bh * T_seq;
  TileRegs gq, go;
  float gl, gd;  // lse (unscaled while in flight), dvec of query threadIdx.x % 64
  auto fetch = [&](int qt) {
    const int i0 = qt * kBT;
    fetch_tile(gq, q + ((size_t)bh * T_seq + i0) * 64, 64, T_seq - 1 - i0);
    fetch_tile(go, dout + ((size_t)b * T_seq + i0) * Dm + h * 64, Dm, T_seq - 1 - i0);
    const int i = min(i0 + (int)(threadIdx.x & 63), T_seq - 1);  // every thread loads (no branch)
    gl = lse_bh[i];
    gd = dv_bh[i];
  };
  wait_vmcnt_bwd<0>();
  __syncthreads();
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) vreg[sl] = tr_frag(sQ[1], 32 * sl + 8 * lg, 32 * sl + 8 * lg + 4, 16 * w, lr);
  fetch(kt);

  f32x4_t dk[4], dv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) dk[i] = dv[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int qt = kt; qt < n_tiles; ++qt) {
    const int buf = (qt - kt) & 1, i0 = qt * kBT;
    // tile qt into buffer buf (last read two tiles ago, before the previous barrier)
    put_tile(sQ[buf], gq);
    put_tile(sO[buf], go);
    if (threadIdx.x < kBT) {
      sL[buf][threadIdx.x] = gl * kLog2e;
      sD[buf][threadIdx.x] = gd;
    }
    __syncthreads();  // tile qt in LDS; everyone is past tile qt - 1
    if (qt + 1 < n_tiles) fetch(qt + 1);
    const char* tQ = sQ[buf];
    const char* tO = sO[buf];
    // S[q = 16 qb + 4 lg + e][key] and dP likewise
    f32x4_t s[4], dp[4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) s[qb] = dp[qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sl = 0; sl < 2; ++sl)
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        Mma<bf16_t>::run(s[qb], plain_frag(tQ, 16 * qb + lr, sl * 4 + lg), kreg[sl]);
        Mma<bf16_t>::run(dp[qb], plain_frag(tO, 16 * qb + lr, sl * 4 + lg), vreg[sl]);
      }
    const bool full = qt > kt && i0 + kBT <= T_seq;  // uniform: every entry of the tile kept
    u32x4_t pf[2], sf[2];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const f32x4_t l4 = *reinterpret_cast<const f32x4_t*>(&sL[buf][16 * qb + 4 * lg]);
      const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(&sD[buf][16 * qb + 4 * lg]);
      float pv[4], sv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int qi = i0 + 16 * qb + 4 * lg + e;
        const bool ok = full || (key <= qi && qi < T_seq);
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][e], kLog2e, -l4[e]));
        const float ds = p * (dp[qb][e] - d4[e]);
        pv[e] = ok ? p : 0.f;
        sv[e] = ok ? ds : 0.f;
      }
      pf[qb >> 1][(qb & 1) * 2] = pack2_bf16(pv[0], pv[1]);
      pf[qb >> 1][(qb & 1) * 2 + 1] = pack2_bf16(pv[2], pv[3]);
      sf[qb >> 1][(qb & 1) * 2] = pack2_bf16(sv[0], sv[1]);
      sf[qb >> 1][(qb & 1) * 2 + 1] = pack2_bf16(sv[2], sv[3]);
    }
    // dV^T[d][key] += sum_q dO^T[d][q] P[q][key]; dK^T likewise with Q, dS
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int r0 = pslot_row(s2, lg, 0), r1 = pslot_row(s2, lg, 1);
        Mma<bf16_t>::run(dv[db], tr_frag(tO, r0, r1, 16 * db, lr), pf[s2]);
        Mma<bf16_t>::run(dk[db], tr_frag(tQ, r0, r1, 16 * db, lr), sf[s2]);
      }
  }
  // lane holds dK^T, dV^T [d = 16 db + 4 lg + e][key]
  if (key < T_seq) {
    float* row = dqkv + ((size_t)b * T_seq + key) * (3 * Dm) + h * 64;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      *reinterpret_cast<f32x4_t*>(row + Dm + 16 * db + 4 * lg) = dk[db];
      *reinterpret_cast<f32x4_t*>(row + 2 * Dm + 16 * db + 4 * lg) = dv[db];
    }
  }
}

// dQ of one query tile: wave w owns queries 16 w .. 16 w + 15, whose Q and
// dO rows (and lse, dvec) it keeps in registers.  Per key tile at or before
// it (K and V^T tiles double-buffered in LDS): S and dP of the 64 keys
// against the wave's queries (lane (lr, lg): keys 16 kb + 4 lg + e, query lr),
// dS = P (dP - dvec) selected to 0 where the key follows the query, then
// dQ^T += K^T dS.
__global__ __launch_bounds__(256) void attn_bwd_dq_reg_kernel(const bf16_t* __restrict__ q,
                                                                const bf16_t* __restrict__ k,
                                                                const bf16_t* __restrict__ vt,
                                                                const bf16_t* __restrict__ dout,
                                                                const float* __restrict__ lse,
                                                                const float* __restrict__ dvec,
                                                                float* __restrict__ dqkv, int BH, int H, int T_seq,
                                                                int kvT, int n_tiles, float scale) {
  __shared__ __attribute__((aligned(16))) char sK[2][kTileBytes];
  __shared__ __attribute__((aligned(16))) char sV[2][kTileBytes];
  const int r = blockIdx.x / BH, bh = blockIdx.x - r * BH;
  const int qt = n_tiles - 1 - r;  // the last query tile (the longest) first
  const int b = bh / H, h = bh - b * H;
  const int i0 = qt * kBT;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int Dm = H * 64;
  const int qi = i0 + 16 * w + lr;  // this lane's query
  const int qc = min(qi, T_seq - 1);
  TileRegs gk, gv;
  auto fetch = [&](int kt) {
    const int j0 = kt * kBT;
    fetch_tile(gk, k + ((size_t)bh * kvT + j0) * 64, 64, T_seq - 1 - j0);
    fetch_tile(gv, vt + (size_t)bh * 64 * kvT + j0, kvT, 63);
  };
  u32x4_t qreg[2], oreg[2];
  {
    const bf16_t* qr = q + ((size_t)bh * T_seq + qc) * 64;
    const bf16_t* orow = dout + ((size_t)b * T_seq + qc) * Dm + h * 64;
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      qreg[sl] = *reinterpret_cast<const u32x4_t*>(qr + sl * 32 + lg * 8);
      oreg[sl] = *reinterpret_cast<const u32x4_t*>(orow + sl * 32 + lg * 8);
    }
  }
  const float lq = lse[(size_t)bh * T_seq + qc];
  const float dvq = dvec[(size_t)bh * T_seq + qc];
  fetch(0);
  const float l2 = lq * kLog2e;
  f32x4_t dq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) dq[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int kt = 0; kt <= qt; ++kt) {
    const int buf = kt & 1, j0 = kt * kBT;
    // tile kt into buffer buf (last read two tiles ago, before the previous barrier)
    put_tile(sK[buf], gk);
    put_tile(sV[buf], gv);
    __syncthreads();  // tile kt in LDS; everyone is past tile kt - 1
    if (kt + 1 <= qt) fetch(kt + 1);
    const char* tK = sK[buf];
    const char* tV = sV[buf];
    // S[key = 16 kb + 4 lg + e][query lr] and dP likewise
    f32x4_t s[4], dp[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) s[kb] = dp[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sl = 0; sl < 2; ++sl)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        Mma<bf16_t>::run(s[kb], plain_frag(tK, 16 * kb + lr, sl * 4 + lg), qreg[sl]);
        Mma<bf16_t>::run(dp[kb], tr_frag(tV, 32 * sl + 8 * lg, 32 * sl + 8 * lg + 4, 16 * kb, lr), oreg[sl]);
      }
    const bool full = kt < qt;  // uniform: every key before every query of the tile
    u32x4_t sf[2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      float sv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kj = j0 + 16 * kb + 4 * lg + e;
        const bool ok = full || kj <= qi;
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][e], kLog2e, -l2));
        const float ds = p * (dp[kb][e] - dvq);
        sv[e] = ok ? ds : 0.f;
      }
      sf[kb >> 1][(kb & 1) * 2] = pack2_bf16(sv[0], sv[1]);
      sf[kb >> 1][(kb & 1) * 2 + 1] = pack2_bf16(sv[2], sv[3]);
    }
    // dQ^T[d][q] += sum_key K^T[d][key] dS[q][key]
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int db = 0; db < 4; ++db)
        Mma<bf16_t>::run(dq[db], tr_frag(tK, pslot_row(s2, lg, 0), pslot_row(s2, lg, 1), 16 * db, lr), sf[s2]);
  }
  // lane holds dQ^T[d = 16 db + 4 lg + e][query]
  if (qi < T_seq) {
    float* row = dqkv + ((size_t)b * T_seq + qi) * (3 * Dm) + h * 64;
#pragma unroll
    for (int db = 0; db < 4; ++db) *reinterpret_cast<f32x4_t*>(row + 16 * db + 4 * lg) = dq[db] * scale;
  }
}

// out[i] = sum over s < splits of part[s * n + i], s in increasing order.
// All MAXS loads of an element go out before the first addition (slices
// past `splits` re-read the last one and are not added).
template <int MAXS>
__global__ __launch_bounds__(256) void sum_splits_kernel(const float* __restrict__ part, int splits, size_t n,
                                                          float* __restrict__ out) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    float v[MAXS];
#pragma unroll
    for (int k = 0; k < MAXS; ++k) v[k] = part[(size_t)min(k, splits - 1) * n + i];
    float s = v[0];
#pragma unroll
    for (int k = 1; k < MAXS; ++k) s = k < splits ? s + v[k] : s;
    out[i] = s;
  }
}

}  // namespace

hipError_t launch_sum_splits(const float* part, int splits, size_t n, float* out, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (splits < 1 || splits > 16) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(256);
  if (splits <= 2)
    hipLaunchKernelGGL(sum_splits_kernel<2>, grid, block, 0, stream, part, splits, n, out);
  else if (splits <= 4)
    hipLaunchKernelGGL(sum_splits_kernel<4>, grid, block, 0, stream, part, splits, n, out);
  else if (splits <= 8)
    hipLaunchKernelGGL(sum_splits_kernel<8>, grid, block, 0, stream, part, splits, n, out);
  else
    hipLaunchKernelGGL(sum_splits_kernel<16>, grid, block, 0, stream, part, splits, n, out);
  return hipGetLastError();
}

template <typename Tin, typename Tout>
hipError_t launch_transpose(const Tin* src, int R, int C, Tout* dst, int ld_dst, hipStream_t stream) {
  if (ld_dst < R) return hipErrorInvalidValue;
  if constexpr (std::is_same_v<Tin, bf16_t> && std::is_same_v<Tout, bf16_t>) {
    if (C % 8 == 0 && ld_dst % 8 == 0 && (reinterpret_cast<uintptr_t>(src) & 15) == 0 &&
        (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
      const dim3 grid((ld_dst + 63) / 64, (C + 63) / 64);
      if (grid.x == 0 || grid.y == 0) return hipSuccess;
      hipLaunchKernelGGL(transpose64_bf16_kernel, grid, dim3(256), 0, stream, src, R, C, dst, ld_dst);
      return hipGetLastError();
    }
  }
  const dim3 grid((ld_dst + 31) / 32, (C + 31) / 32);
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  hipLaunchKernelGGL((transpose_kernel<Tin, Tout>), grid, dim3(256), 0, stream, src, R, C, dst, ld_dst);
  return hipGetLastError();
}

size_t colsum_partial_floats(int N) { return (size_t)kColChunks * N; }

template <typename Tin>
hipError_t launch_colsum(const Tin* src, int M, int N, float* out, float* part, hipStream_t stream, const float* x,
                         const float* mu, const float* rstd) {
  if (N <= 0) return hipSuccess;
  constexpr int VEC = 16 / (int)sizeof(Tin);
  if (N % VEC == 0 && (reinterpret_cast<uintptr_t>(src) & 15) == 0) {
    const dim3 gridv((N / VEC + 63) / 64, kColChunks);
    if (x)
      hipLaunchKernelGGL((colsum_partial_vec_kernel<Tin, true>), gridv, dim3(256), 0, stream, src, M, N, part, x, mu,
                         rstd, nullptr);
    else
      hipLaunchKernelGGL((colsum_partial_vec_kernel<Tin, false>), gridv, dim3(256), 0, stream, src, M, N, part, x,
                         mu, rstd, nullptr);
    hipLaunchKernelGGL(colsum_final_kernel, dim3((N + 63) / 64), dim3(256), 0, stream, part, N, out);
    return hipGetLastError();
  }
  const dim3 grid1((N + 63) / 64, kColChunks);
  if (x)
    hipLaunchKernelGGL((colsum_partial_kernel<Tin, true>), grid1, dim3(256), 0, stream, src, M, N, part, x, mu, rstd);
  else
    hipLaunchKernelGGL((colsum_partial_kernel<Tin, false>), grid1, dim3(256), 0, stream, src, M, N, part, x, mu,
                       rstd);
  hipLaunchKernelGGL(colsum_final_kernel, dim3((N + 63) / 64), dim3(256), 0, stream, part, N, out);
  return hipGetLastError();
}

template <typename Tin>
hipError_t launch_colsum_partial(const Tin* src, int M, int N, float* part, hipStream_t stream, const float* x,
                                 const float* mu, const float* rstd, float* part_plain) {
  if (N <= 0) return hipSuccess;
  if (part_plain && !x) return hipErrorInvalidValue;
  constexpr int VEC = 16 / (int)sizeof(Tin);
  if (N % VEC == 0 && (reinterpret_cast<uintptr_t>(src) & 15) == 0) {
    const dim3 gridv((N / VEC + 63) / 64, kColChunks);
    if (x)
      hipLaunchKernelGGL((colsum_partial_vec_kernel<Tin, true>), gridv, dim3(256), 0, stream, src, M, N, part, x, mu,
                         rstd, part_plain);
    else
      hipLaunchKernelGGL((colsum_partial_vec_kernel<Tin, false>), gridv, dim3(256), 0, stream, src, M, N, part, x,
                         mu, rstd, nullptr);
    return hipGetLastError();
  }
  const dim3 grid1((N + 63) / 64, kColChunks);
  if (x) {
    hipLaunchKernelGGL((colsum_partial_kernel<Tin, true>), grid1, dim3(256), 0, stream, src, M, N, part, x, mu, rstd);
    if (part_plain)
      hipLaunchKernelGGL((colsum_partial_kernel<Tin, false>), grid1, dim3(256), 0, stream, src, M, N, part_plain, x,
                         mu, rstd);
  } else {
    hipLaunchKernelGGL((colsum_partial_kernel<Tin, false>), grid1, dim3(256), 0, stream, src, M, N, part, x, mu,
                       rstd);
  }
  return hipGetLastError();
}

hipError_t launch_colsum_final(const ColsumJob* jobs, int n_jobs, hipStream_t stream) {
  if (n_jobs < 1 || n_jobs > kMaxColsumJobs) return hipErrorInvalidValue;
  ColsumFinalArgs a{};
  int n_max = 0;
  for (int i = 0; i < n_jobs; ++i) {
    a.job[i] = jobs[i];
    n_max = std::max(n_max, jobs[i].N);
  }
  if (n_max <= 0) return hipSuccess;
  hipLaunchKernelGGL(colsum_final_group_kernel, dim3((n_max + 63) / 64, n_jobs), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_layernorm_backward(const float* x, const float* dh, const float* gamma, const float* resid,
                                     float* out, T* out_t, float* mu, float* rstd, int M, int D, float eps,
                                     hipStream_t stream) {
  if (D > 2048 || D % 4 != 0) return hipErrorInvalidValue;
  if (M <= 0) return hipSuccess;
  const dim3 grid((M + 3) / 4), block(256);
  switch (D) {
    case 768:
      hipLaunchKernelGGL((layernorm_backward_kernel<T, 3>), grid, block, 0, stream, x, dh, gamma, resid, out, out_t,
                         mu, rstd, M, D, eps);
      break;
    case 1024:
      hipLaunchKernelGGL((layernorm_backward_kernel<T, 4>), grid, block, 0, stream, x, dh, gamma, resid, out, out_t,
                         mu, rstd, M, D, eps);
      break;
    default:
      hipLaunchKernelGGL((layernorm_backward_kernel<T, 0>), grid, block, 0, stream, x, dh, gamma, resid, out, out_t,
                         mu, rstd, M, D, eps);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_attention_backward(const T* q, const T* k, const T* vt, const T* o, const T* dout,
                                     const float* lse, float* dvec, float* dqkv, int B, int H, int T_seq, int kvT,
                                     int hs, float scale, hipStream_t stream) {
  if (T_seq <= 0) return hipSuccess;
  const int n_tiles = (T_seq + kBT - 1) / kBT;
  if (kvT < T_seq) return hipErrorInvalidValue;
  const int rows = B * H * T_seq;
  const dim3 grid(B * H * n_tiles), block(256);
  if constexpr (sizeof(T) == 2) {
    if (hs == 64) {
      hipLaunchKernelGGL(attn_bwd_dvec_bf16_kernel, dim3((rows + 31) / 32), block, 0, stream, o, dout, dvec, B, H,
                         T_seq);
      hipLaunchKernelGGL(attn_bwd_dkdv_reg_kernel, grid, block, 0, stream, q, k, vt, dout, lse, dvec, dqkv, B * H, H,
                         T_seq, kvT, n_tiles);
      hipLaunchKernelGGL(attn_bwd_dq_reg_kernel, grid, block, 0, stream, q, k, vt, dout, lse, dvec, dqkv, B * H, H,
                         T_seq, kvT, n_tiles, scale);
      return hipGetLastError();
    }
  }
  if (hs == 64) {
    hipLaunchKernelGGL((attn_bwd_dvec_kernel<T, 64>), dim3((rows + 3) / 4), block, 0, stream, o, dout, dvec, B, H,
                       T_seq);
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, 64>), grid, block, 0, stream, q, k, vt, dout, lse, dvec, dqkv, H,
                       T_seq, kvT, n_tiles);
    hipLaunchKernelGGL((attn_bwd_dq_kernel<T, 64>), grid, block, 0, stream, q, k, vt, dout, lse, dvec, dqkv, H, T_seq,
                       kvT, n_tiles, scale);
  } else if (hs == 16) {
    hipLaunchKernelGGL((attn_bwd_dvec_kernel<T, 16>), dim3((rows + 3) / 4), block, 0, stream, o, dout, dvec, B, H,
                       T_seq);
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, 16>), grid, block, 0, stream, q, k, vt, dout, lse, dvec, dqkv, H,
                       T_seq, kvT, n_tiles);
    hipLaunchKernelGGL((attn_bwd_dq_kernel<T, 16>), grid, block, 0, stream, q, k, vt, dout, lse, dvec, dqkv, H, T_seq,
                       kvT, n_tiles, scale);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template hipError_t launch_transpose<float, float>(const float*, int, int, float*, int, hipStream_t);
template hipError_t launch_transpose<float, bf16_t>(const float*, int, int, bf16_t*, int, hipStream_t);
template hipError_t launch_transpose<bf16_t, bf16_t>(const bf16_t*, int, int, bf16_t*, int, hipStream_t);
template hipError_t launch_colsum<float>(const float*, int, int, float*, float*, hipStream_t, const float*,
                                         const float*, const float*);
template hipError_t launch_colsum<bf16_t>(const bf16_t*, int, int, float*, float*, hipStream_t, const float*,
                                          const float*, const float*);
template hipError_t launch_colsum_partial<float>(const float*, int, int, float*, hipStream_t, const float*,
                                                 const float*, const float*, float*);
template hipError_t launch_colsum_partial<bf16_t>(const bf16_t*, int, int, float*, hipStream_t, const float*,
                                                  const float*, const float*, float*);
template hipError_t launch_layernorm_backward<float>(const float*, const float*, const float*, const float*, float*,
                                                     float*, float*, float*, int, int, float, hipStream_t);
template hipError_t launch_layernorm_backward<bf16_t>(const float*, const float*, const float*, const float*, float*,
                                                      bf16_t*, float*, float*, int, int, float, hipStream_t);
template hipError_t launch_attention_backward<float>(const float*, const float*, const float*, const float*,
                                                     const float*, const float*, float*, float*, int, int, int, int,
                                                     int, float, hipStream_t);
template hipError_t launch_attention_backward<bf16_t>(const bf16_t*, const bf16_t*, const bf16_t*, const bf16_t*,
                                                      const bf16_t*, const float*, float*, float*, int, int, int, int,
                                                      int, float, hipStream_t);

}  // namespace gpt2
