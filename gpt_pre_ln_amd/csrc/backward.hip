// Block backward kernels (see backward.h).
#include "backward.h"

#include <algorithm>
#include <type_traits>

namespace gpt2 {

namespace {

constexpr int kColChunks = 64;  // row chunks of the first column-sum pass

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
  if (n < N) {
    for (int m = m0 + ry; m < m1; m += 4) {
      const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(src + (size_t)m * N + n);
      float v[VEC];
      if constexpr (sizeof(Tin) == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[2 * e] = bf16_to_f32(raw[e] & 0xFFFF);
          v[2 * e + 1] = bf16_to_f32(raw[e] >> 16);
        }
      } else {
        const f32x4_t f = __builtin_bit_cast(f32x4_t, raw);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = f[e];
      }
      if constexpr (kXhat) {
        const float mm = mu[m], rs = rstd[m];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          s2[e] += v[e];
          v[e] *= (x[(size_t)m * N + n + e] - mm) * rs;
        }
      }
#pragma unroll
      for (int e = 0; e < VEC; ++e) s[e] += v[e];
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

// Second pass for several column sums in one launch (blockIdx.y = job):
// out[n] = sum over row chunks rc of part[rc][n], in increasing rc.
struct ColsumFinalArgs {
  ColsumJob job[kMaxColsumJobs];
};
__global__ __launch_bounds__(256) void colsum_final_group_kernel(ColsumFinalArgs a) {
  const ColsumJob j = a.job[blockIdx.y];
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= j.N) return;
  float s = 0.f;
  for (int rc = 0; rc < kColChunks; ++rc) s += j.part[(size_t)rc * j.N + n];
  j.out[n] = s;
}

__global__ __launch_bounds__(256) void colsum_final_kernel(const float* __restrict__ part, int N,
                                                            float* __restrict__ out) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  float s = 0.f;
  for (int rc = 0; rc < kColChunks; ++rc) s += part[(size_t)rc * N + n];
  out[n] = s;
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
// Head size 64, 64 x 64 tiles, 4 waves.  R = X Y^T on 16 x 16 blocks with
// v_mfma_f32_16x16x32_bf16 (Mma<bf16_t>::run(acc, X, Y)): lane l supplies
// X[l % 16][8 (l / 16) .. +7] and Y[l % 16][8 (l / 16) .. +7] (16 bytes of a
// row whose contraction index is contiguous) and receives
// R[4 (l / 16) + e][l % 16], e = 0..3.  Every operand therefore lives in LDS
// with its contraction index contiguous: Q, dO, K, V as [row][d] and the
// transposed copies Q^T, dO^T, K^T as [d][row]; P and dS are written by the
// wave that computed them in the layout of the product that reads them.
constexpr int kLdsRow = 64 + 8;  // bf16 per LDS row (16 bytes of padding)

struct alignas(16) MmaTile {
  bf16_t a[kBT][kLdsRow];
};

__device__ __forceinline__ u32x4_t frag(const MmaTile& t, int row, int k8) {
  return *reinterpret_cast<const u32x4_t*>(&t.a[row][k8]);
}

// Row-major copy ([row][d], 16-byte chunks) and, optionally, the transposed
// copy ([d][row]) of 64 rows of 64 bf16 from global rows src + r * ld, rows
// past `valid` zero.
// A 64 x 64 bf16 tile held in registers between its global read and its LDS
// write, so the next tile's reads can be in flight while the current tile is
// computed.  256 threads, two 16-byte chunks each: thread t holds elements
// 8 (t % 8) .. +7 of rows 2 (t / 8) and 2 (t / 8) + 1, so that the transposed
// copy takes one 4-byte LDS write per element pair of the two rows.
struct TileRegs {
  u32x4_t v[2];
};
static_assert(kBT * 8 == 2 * 256, "two 16-byte chunks per thread");

__device__ __forceinline__ void fetch_rows_bf16(TileRegs& g, const bf16_t* src, size_t ld, int valid) {
  const int r0 = 2 * (threadIdx.x >> 3), d8 = (threadIdx.x & 7) * 8;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    g.v[j] = u32x4_t{0u, 0u, 0u, 0u};
    if (r0 + j < valid) g.v[j] = *reinterpret_cast<const u32x4_t*>(src + (size_t)(r0 + j) * ld + d8);
  }
}

// Rows as [row][d] into t and, when tt is given, transposed as [d][row].
__device__ __forceinline__ void put_rows_bf16(MmaTile& t, MmaTile* tt, const TileRegs& g) {
  const int r0 = 2 * (threadIdx.x >> 3), d8 = (threadIdx.x & 7) * 8;
#pragma unroll
  for (int j = 0; j < 2; ++j) *reinterpret_cast<u32x4_t*>(&t.a[r0 + j][d8]) = g.v[j];
  if (tt) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t a = g.v[0][e], b = g.v[1][e];  // rows r0, r0 + 1; elements d8 + 2e, d8 + 2e + 1
      *reinterpret_cast<uint32_t*>(&tt->a[d8 + 2 * e][r0]) = (a & 0xFFFFu) | (b << 16);
      *reinterpret_cast<uint32_t*>(&tt->a[d8 + 2 * e + 1][r0]) = (a >> 16) | (b & 0xFFFF0000u);
    }
  }
}

// Rows r < valid of a [rows][ld] bf16 matrix into t (and transposed into tt),
// rows past `valid` zero.
__device__ __forceinline__ void load_rows_bf16(MmaTile& t, MmaTile* tt, const bf16_t* src, size_t ld, int valid) {
  TileRegs g;
  fetch_rows_bf16(g, src, ld, valid);
  put_rows_bf16(t, tt, g);
}

// V^T rows (global [d][kvT], keys contiguous) into V as [key][d]; keys past
// `valid` zero.  Thread t holds keys k8 .. k8+7 (k8 = 8 (t % 8)) of rows
// d = 2 (t / 8) and d + 1, so each key's two values leave as one 4-byte write.
__device__ __forceinline__ void fetch_vt_bf16(TileRegs& g, const bf16_t* vt, int kvT, int j0, int valid) {
  const int d0 = 2 * (threadIdx.x >> 3), k8 = (threadIdx.x & 7) * 8;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    g.v[j] = u32x4_t{0u, 0u, 0u, 0u};
    if (k8 < valid) g.v[j] = *reinterpret_cast<const u32x4_t*>(vt + (size_t)(d0 + j) * kvT + j0 + k8);
  }
}

__device__ __forceinline__ void put_vt_bf16(MmaTile& t, const TileRegs& g, int valid) {
  const int d0 = 2 * (threadIdx.x >> 3), k8 = (threadIdx.x & 7) * 8;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t a = g.v[0][e], b = g.v[1][e];  // rows d0, d0 + 1; keys k8 + 2e, k8 + 2e + 1
    const bool lo = k8 + 2 * e < valid, hi = k8 + 2 * e + 1 < valid;
    *reinterpret_cast<uint32_t*>(&t.a[k8 + 2 * e][d0]) = lo ? (a & 0xFFFFu) | (b << 16) : 0u;
    *reinterpret_cast<uint32_t*>(&t.a[k8 + 2 * e + 1][d0]) = hi ? (a >> 16) | (b & 0xFFFF0000u) : 0u;
  }
}

__device__ __forceinline__ void load_vt_bf16(MmaTile& t, const bf16_t* vt, int kvT, int j0, int valid) {
  TileRegs g;
  fetch_vt_bf16(g, vt, kvT, j0, valid);
  put_vt_bf16(t, g, valid);
}

// S and dP of one 16-row block (rows `r16` of X-side tiles Qs / dOs) against
// the 64 keys of Ks / Vs, or (keys_by_wave) of 64 query rows against one
// 16-key block: acc[b] covers the b-th 16 x 16 block.
__device__ __forceinline__ void mma_sp(f32x4_t (&s)[4], f32x4_t (&dp)[4], const MmaTile& X1, const MmaTile& Y1,
                                       const MmaTile& X2, const MmaTile& Y2, int xrow0, int yrow0, bool x_varies) {
  const int lr = threadIdx.x & 15, lg = (threadIdx.x >> 4) & 3;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    s[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    dp[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int k8 = ks * 32 + lg * 8;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int xr = x_varies ? b * 16 + lr : xrow0 + lr;
      const int yr = x_varies ? yrow0 + lr : b * 16 + lr;
      Mma<bf16_t>::run(s[b], frag(X1, xr, k8), frag(Y1, yr, k8));
      Mma<bf16_t>::run(dp[b], frag(X2, xr, k8), frag(Y2, yr, k8));
    }
  }
}

struct AttnBwdMmaKV {
  MmaTile K, V, Q, Qt, dO, dOt, Pt, dSt;
  float lse[kBT];
  float dv[kBT];
};

// dK and dV of one key tile (64 keys): wave w owns keys 16w .. 16w+15.  Per
// query tile at or after it: S and dP of all 64 queries against the wave's
// keys; P = exp(S - lse), dS = P (dP - rowsum(dO o)) (exactly 0 where the key
// follows the query or the query is past the end), written as P^T, dS^T
// rows of the wave's keys; then dV += P^T dO and dK += dS^T Q.
__global__ __launch_bounds__(256) void attn_bwd_dkdv_mma_kernel(const bf16_t* __restrict__ q,
                                                                const bf16_t* __restrict__ k,
                                                                const bf16_t* __restrict__ vt,
                                                                const bf16_t* __restrict__ dout,
                                                                const float* __restrict__ lse,
                                                                const float* __restrict__ dvec,
                                                                float* __restrict__ dqkv, int BH, int H, int T_seq,
                                                                int kvT, int n_tiles) {
  __shared__ AttnBwdMmaKV sm;
  const int kt = blockIdx.x / BH, bh = blockIdx.x - kt * BH;  // key tile 0 (the longest) first
  const int b = bh / H, h = bh - b * H;
  const int j0 = kt * kBT;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int Dm = H * 64;
  load_rows_bf16(sm.K, nullptr, k + ((size_t)bh * kvT + j0) * 64, 64, min(kBT, T_seq - j0));
  load_vt_bf16(sm.V, vt + (size_t)bh * 64 * kvT, kvT, j0, min(kBT, T_seq - j0));
  f32x4_t dk[4], dv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) dk[i] = dv[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // The next query tile's Q, dO, lse and dvec are read into registers while
  // the current one is computed.
  TileRegs gq, gdo;
  float glse = 0.f, gdv = 0.f;
  auto fetch_qtile = [&](int qt) {
    const int i0 = qt * kBT, nq = min(kBT, T_seq - i0);
    fetch_rows_bf16(gq, q + ((size_t)bh * T_seq + i0) * 64, 64, nq);
    fetch_rows_bf16(gdo, dout + ((size_t)b * T_seq + i0) * Dm + h * 64, Dm, nq);
    if (threadIdx.x < kBT) {
      const int i = threadIdx.x;
      glse = i < nq ? lse[(size_t)bh * T_seq + i0 + i] : 0.f;
      gdv = i < nq ? dvec[(size_t)bh * T_seq + i0 + i] : 0.f;
    }
  };
  fetch_qtile(kt);
  for (int qt = kt; qt < n_tiles; ++qt) {
    const int i0 = qt * kBT, nq = min(kBT, T_seq - i0);
    __syncthreads();
    put_rows_bf16(sm.Q, &sm.Qt, gq);
    put_rows_bf16(sm.dO, &sm.dOt, gdo);
    if (threadIdx.x < kBT) {
      sm.lse[threadIdx.x] = glse;
      sm.dv[threadIdx.x] = gdv;
    }
    if (qt + 1 < n_tiles) fetch_qtile(qt + 1);
    __syncthreads();
    // R[q][key] for the 4 query blocks (x varies) against this wave's keys
    f32x4_t s[4], dp[4];
    mma_sp(s, dp, sm.Q, sm.K, sm.dO, sm.V, 0, w * 16, true);
    const int key = w * 16 + lr;  // local key of this lane's column
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      uint32_t pw[2], sw[2];
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
        float pv[2], sv[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int e = e2 * 2 + u;
          const int ql = qb * 16 + lg * 4 + e;
          const bool ok = j0 + key <= i0 + ql && ql < nq;
          const float p = ok ? __builtin_amdgcn_exp2f((s[qb][e] - sm.lse[ql]) * kLog2e) : 0.f;
          pv[u] = p;
          sv[u] = ok ? p * (dp[qb][e] - sm.dv[ql]) : 0.f;
        }
        pw[e2] = pack2_bf16(pv[0], pv[1]);
        sw[e2] = pack2_bf16(sv[0], sv[1]);
      }
      // P^T[key][q .. q+3], dS^T likewise: one 8-byte store each
      *reinterpret_cast<u32x2_t*>(&sm.Pt.a[key][qb * 16 + lg * 4]) = u32x2_t{pw[0], pw[1]};
      *reinterpret_cast<u32x2_t*>(&sm.dSt.a[key][qb * 16 + lg * 4]) = u32x2_t{sw[0], sw[1]};
    }
    __syncthreads();
    // dV[key][d] += P^T dO, dK[key][d] += dS^T Q (contraction over the 64 queries)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int k8 = ks * 32 + lg * 8;
      const u32x4_t pf = frag(sm.Pt, w * 16 + lr, k8), sf = frag(sm.dSt, w * 16 + lr, k8);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        Mma<bf16_t>::run(dv[db], pf, frag(sm.dOt, db * 16 + lr, k8));
        Mma<bf16_t>::run(dk[db], sf, frag(sm.Qt, db * 16 + lr, k8));
      }
    }
  }
  // lane holds R[key = 16w + 4 lg + e][d = 16 db + lr]
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int j = j0 + w * 16 + lg * 4 + e;
    if (j < T_seq) {
      float* row = dqkv + ((size_t)b * T_seq + j) * (3 * Dm) + h * 64 + lr;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        row[Dm + db * 16] = dk[db][e];
        row[2 * Dm + db * 16] = dv[db][e];
      }
    }
  }
}

struct AttnBwdMmaQ {
  MmaTile Q, dO, K, Kt, V, dS;
  float lse[kBT];
  float dv[kBT];
};

// dQ of one query tile: wave w owns queries 16w .. 16w+15.  Per key tile at
// or before it: S, dP of the wave's queries against the 64 keys, dS written
// as rows of the wave's queries, then dQ += dS K (against K^T).
__global__ __launch_bounds__(256) void attn_bwd_dq_mma_kernel(const bf16_t* __restrict__ q,
                                                              const bf16_t* __restrict__ k,
                                                              const bf16_t* __restrict__ vt,
                                                              const bf16_t* __restrict__ dout,
                                                              const float* __restrict__ lse,
                                                              const float* __restrict__ dvec,
                                                              float* __restrict__ dqkv, int BH, int H, int T_seq,
                                                              int kvT, int n_tiles, float scale) {
  __shared__ AttnBwdMmaQ sm;
  const int r = blockIdx.x / BH, bh = blockIdx.x - r * BH;
  const int qt = n_tiles - 1 - r;  // the last query tile (the longest) first
  const int b = bh / H, h = bh - b * H;
  const int i0 = qt * kBT, nq = min(kBT, T_seq - i0);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int Dm = H * 64;
  load_rows_bf16(sm.Q, nullptr, q + ((size_t)bh * T_seq + i0) * 64, 64, nq);
  load_rows_bf16(sm.dO, nullptr, dout + ((size_t)b * T_seq + i0) * Dm + h * 64, Dm, nq);
  if (threadIdx.x < kBT) {
    const int i = threadIdx.x;
    sm.lse[i] = i < nq ? lse[(size_t)bh * T_seq + i0 + i] : 0.f;
    sm.dv[i] = i < nq ? dvec[(size_t)bh * T_seq + i0 + i] : 0.f;
  }
  f32x4_t dq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) dq[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // The next key tile's K and V^T are read into registers while the current
  // one is computed.
  TileRegs gk, gv;
  auto fetch_ktile = [&](int kt) {
    const int j0 = kt * kBT, nk = min(kBT, T_seq - j0);
    fetch_rows_bf16(gk, k + ((size_t)bh * kvT + j0) * 64, 64, nk);
    fetch_vt_bf16(gv, vt + (size_t)bh * 64 * kvT, kvT, j0, nk);
  };
  fetch_ktile(0);
  for (int kt = 0; kt <= qt; ++kt) {
    const int j0 = kt * kBT, nk = min(kBT, T_seq - j0);
    __syncthreads();
    put_rows_bf16(sm.K, &sm.Kt, gk);
    put_vt_bf16(sm.V, gv, nk);
    if (kt + 1 <= qt) fetch_ktile(kt + 1);
    __syncthreads();
    // R[q][key] for this wave's queries (y varies over the 4 key blocks)
    f32x4_t s[4], dp[4];
    mma_sp(s, dp, sm.Q, sm.K, sm.dO, sm.V, w * 16, 0, false);
    // lane holds R[q = 16w + 4 lg + e][key = 16 kb + lr]
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ql = w * 16 + lg * 4 + e, key = kb * 16 + lr;
        const bool ok = j0 + key <= i0 + ql && ql < nq;
        const float p = ok ? __builtin_amdgcn_exp2f((s[kb][e] - sm.lse[ql]) * kLog2e) : 0.f;
        sm.dS.a[ql][key].bits = f32_to_bf16(ok ? p * (dp[kb][e] - sm.dv[ql]) : 0.f);
      }
    __syncthreads();
    // dQ[q][d] += dS K  (contraction over the 64 keys; K^T rows are d)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int k8 = ks * 32 + lg * 8;
      const u32x4_t sf = frag(sm.dS, w * 16 + lr, k8);
#pragma unroll
      for (int db = 0; db < 4; ++db) Mma<bf16_t>::run(dq[db], sf, frag(sm.Kt, db * 16 + lr, k8));
    }
  }
  // lane holds R[q = 16w + 4 lg + e][d = 16 db + lr]
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = i0 + w * 16 + lg * 4 + e;
    if (i < T_seq) {
      float* row = dqkv + ((size_t)b * T_seq + i) * (3 * Dm) + h * 64 + lr;
#pragma unroll
      for (int db = 0; db < 4; ++db) row[db * 16] = scale * dq[db][e];
    }
  }
}

// out[i] = sum over s < splits of part[s * n + i], s in increasing order.
__global__ __launch_bounds__(256) void sum_splits_kernel(const float* __restrict__ part, int splits, size_t n,
                                                          float* __restrict__ out) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    float s = part[i];
    for (int k = 1; k < splits; ++k) s += part[(size_t)k * n + i];
    out[i] = s;
  }
}

}  // namespace

hipError_t launch_sum_splits(const float* part, int splits, size_t n, float* out, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, part, splits, n, out);
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
    hipLaunchKernelGGL(colsum_final_kernel, dim3((N + 255) / 256), dim3(256), 0, stream, part, N, out);
    return hipGetLastError();
  }
  const dim3 grid1((N + 63) / 64, kColChunks);
  if (x)
    hipLaunchKernelGGL((colsum_partial_kernel<Tin, true>), grid1, dim3(256), 0, stream, src, M, N, part, x, mu, rstd);
  else
    hipLaunchKernelGGL((colsum_partial_kernel<Tin, false>), grid1, dim3(256), 0, stream, src, M, N, part, x, mu,
                       rstd);
  hipLaunchKernelGGL(colsum_final_kernel, dim3((N + 255) / 256), dim3(256), 0, stream, part, N, out);
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
  hipLaunchKernelGGL(colsum_final_group_kernel, dim3((n_max + 255) / 256, n_jobs), dim3(256), 0, stream, a);
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
      hipLaunchKernelGGL(attn_bwd_dkdv_mma_kernel, grid, block, 0, stream, q, k, vt, dout, lse, dvec, dqkv, B * H, H,
                         T_seq, kvT, n_tiles);
      hipLaunchKernelGGL(attn_bwd_dq_mma_kernel, grid, block, 0, stream, q, k, vt, dout, lse, dvec, dqkv, B * H, H,
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
