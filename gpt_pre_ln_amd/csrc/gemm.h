// Matrix-core GEMM with fused epilogues for the projections of the GPT-2 block
// and the tied lm_head:  C[m, n] = sum_k A[m, k] * B[n, k]   (both K-contiguous)
//
//   c_attn  (pwwt.cn "逐行拆GPT-2源码", GPT2Attention: one fused projection to
//            3*d_model, split into thirds q|k|v, heads = consecutive head_dim
//            column blocks)                        -> EpiQKV (bias, head scatter)
//   c_proj  (GPT2Attention c_proj, then the first residual of GPT2Block.forward)
//                                                   -> EpiResidual (bias, x += .)
//   c_fc    (GPT2MLP c_fc followed by gelu_new, or the erf GELU)  -> EpiGelu
//   mlp.c_proj (GPT2MLP c_proj, second residual)    -> EpiResidual
//   lm_head (GPT2LMHeadModel: tied to wte, no bias) -> EpiLogits
//
// Design (gfx950):
//   * block tile BM x BN, k staged 128 bytes per step (64 bf16 / 32 fp32)
//     through an LDS ring filled by direct global->LDS loads
//     (global_load_lds_dwordx4, no register staging), one fence-free barrier
//     per k step; loads of step k+1 are in flight while step k runs on the
//     matrix cores.
//   * WGM x WGN waves; each wave owns a (BM/WGM) x (BN/WGN) sub-tile built from
//     16x16 MFMA tiles (v_mfma_f32_16x16x32_bf16, or 16x16x4_f32 for fp32).
//   * operands are swapped in the MFMA (B rows first) so that every lane ends
//     with 4 consecutive output columns of one row.
//   * epilogue: bias added in registers, then each wave stages its sub-tile
//     through its own slice of the operand LDS and reads it back so that one
//     store instruction covers whole row segments (or, for the transposed
//     V^T output, whole column segments) instead of 16 rows x 16 columns.
//   * LDS rows are 128 bytes = 8 chunks of 16 bytes; chunk c of row r lives at
//     slot c ^ (r & 7) so the 16 rows read by a lane group fall in distinct
//     bank groups.
//   * blocks are remapped so that each XCD (blockIdx % 8 on MI355X) walks a
//     contiguous range of tiles, grouped GROUP_M tile-rows at a time, which
//     keeps the A row-panels and B column-panels in that XCD's L2.
#pragma once

#include "common.h"

namespace gpt2 {

// Epilogues.  The kernel adds the bias (bias4(n), when kBias) to the
// accumulators first and then hands over 4-element groups:
//   apply(m, n, v, pre)  v = C[m][n .. n+3]; pre = preload(m, n) when kPreload
//                        (the residual), fetched before the group's stores;
//   apply_t(m, n, v)     v = C[m .. m+3][n], only when kTransposed and
//                        transposed(n) holds for the column block of the wave.
// kRowReduce epilogues (EpiCE) instead receive, per row m and per column
// slice s of one wave's width (gemm_slice_width), the maximum and the sum of
// exp(C - maximum) over the slice's columns below n_valid, and the single
// entry C[m][label(m)] from the lane that holds it; kRowArgmax epilogues
// (EpiArgmax) the slice maximum and the first column holding it.

template <typename T>
struct EpiQKV {
  static constexpr bool kPreload = false, kBias = true, kTransposed = true, kRowReduce = false, kRowArgmax = false;
  const float* bias;  // [3D]
  T* q;               // [B][H][Tq][hs], scaled by q_scale
  T* k;               // [B][H][kvT][hs], rows t0 + t
  T* vt;              // [B][H][hs][kvT], columns t0 + t
  FastDiv Tq;         // tokens per sequence in this call (rows m = b*Tq + t)
  FastDiv D;          // d_model (which third of the 3D columns)
  int t0;             // absolute position of row t = 0 (past length)
  int kvT;            // allocated positions per sequence in k / vt
  int H, hs_log2;
  float q_scale;
  int M;              // rows of the product (B * Tq)
  __device__ __forceinline__ float4 bias4(int n) const { return *reinterpret_cast<const float4*>(bias + n); }
  __device__ __forceinline__ float4 preload(int, int) const { return float4{}; }
  // the value third (columns 2D .. 3D) is stored transposed
  __device__ __forceinline__ bool transposed(int n) const { return D.div((uint32_t)n) == 2; }
  __device__ __forceinline__ void apply(int m, int n, const f32x4_t& v, const float4&) const {
    const int which = (int)D.div((uint32_t)n);
    const int hd = n - which * (int)D.d;
    const int head = hd >> hs_log2;
    const int d = hd - (head << hs_log2);
    const int bb = (int)Tq.div((uint32_t)m);
    const int t = m - bb * (int)Tq.d;
    const size_t bh = (size_t)bb * H + head;
    const int hs = 1 << hs_log2;
    if (which == 0) {
      Elem<T>::store4(q + (bh * Tq.d + t) * hs + d, v[0] * q_scale, v[1] * q_scale, v[2] * q_scale, v[3] * q_scale);
    } else if (which == 1) {
      Elem<T>::store4(k + (bh * kvT + t0 + t) * hs + d, v[0], v[1], v[2], v[3]);
    } else {
      T* p = vt + (bh * hs + d) * kvT + t0 + t;
      p[0] = Elem<T>::from_f32(v[0]);
      p[kvT] = Elem<T>::from_f32(v[1]);
      p[2 * (size_t)kvT] = Elem<T>::from_f32(v[2]);
      p[3 * (size_t)kvT] = Elem<T>::from_f32(v[3]);
    }
  }
  // The same stores with the per-column part of the index formed once per
  // lane and tile (col_ctx: n is fixed over the rows a lane stores) and only
  // the row part per group: destination element ((b * R + t) << hs_log2) +
  // off, with R = H * Tq (q) or H * kvT (k).
  struct ColCtx {
    int which, n;
    size_t off;
  };
  __device__ __forceinline__ ColCtx col_ctx(int n) const {
    const int which = (int)D.div((uint32_t)n);
    const int hd = n - which * (int)D.d;
    const int head = hd >> hs_log2;
    const int d = hd - (head << hs_log2);
    const size_t off = which == 0 ? (((size_t)head * Tq.d) << hs_log2) + d
                                  : (((size_t)head * kvT + t0) << hs_log2) + d;
    return ColCtx{which, n, off};
  }
  __device__ __forceinline__ void apply_c(int m, const ColCtx& c, const f32x4_t& v) const {
    if (c.which == 2) {  // value columns of a wave that also holds key columns
      apply(m, c.n, v, float4{});
      return;
    }
    const uint32_t bb = Tq.div((uint32_t)m), t = (uint32_t)m - bb * Tq.d;
    if (c.which == 0) {
      const size_t i = ((size_t)(bb * (uint32_t)H * Tq.d + t) << hs_log2) + c.off;
      Elem<T>::store4(q + i, v[0] * q_scale, v[1] * q_scale, v[2] * q_scale, v[3] * q_scale);
    } else {
      const size_t i = ((size_t)(bb * (uint32_t)H * (uint32_t)kvT + t) << hs_log2) + c.off;
      Elem<T>::store4(k + i, v[0], v[1], v[2], v[3]);
    }
  }
  // Row constants of apply_t (m is fixed over the columns a lane stores):
  // the destination of a whole aligned vector is base + hd * kvT.
  struct RowCtx {
    size_t base;
    bool vec;
  };
  __device__ __forceinline__ RowCtx row_ctx(int m) const {
    const uint32_t bb = Tq.div((uint32_t)m), t = (uint32_t)m - bb * Tq.d;
    const bool vec = m + 3 < M && t + 3 < Tq.d && ((t0 + t) & 3) == 0;
    return RowCtx{((size_t)bb * (uint32_t)H << hs_log2) * (size_t)kvT + t0 + t, vec};
  }
  __device__ __forceinline__ void apply_tc(int m, const RowCtx& r, int n, const f32x4_t& v) const {
    if (r.vec) {
      const int hd = n - 2 * (int)D.d;
      Elem<T>::store4(vt + r.base + (size_t)hd * kvT, v[0], v[1], v[2], v[3]);
    } else {
      apply_t(m, n, v);
    }
  }
  // v = C[m .. m+3][n] with n in the value third: positions t .. t+3 of one
  // V^T row, stored as one vector when they lie in one sequence and aligned.
  __device__ __forceinline__ void apply_t(int m, int n, const f32x4_t& v) const {
    const int hd = n - 2 * (int)D.d;
    const int head = hd >> hs_log2;
    const int d = hd - (head << hs_log2);
    const int hs = 1 << hs_log2;
    const int bb = (int)Tq.div((uint32_t)m);
    const int t = m - bb * (int)Tq.d;
    if (m + 3 < M && t + 3 < (int)Tq.d && ((t0 + t) & 3) == 0) {
      Elem<T>::store4(vt + (((size_t)bb * H + head) * hs + d) * kvT + t0 + t, v[0], v[1], v[2], v[3]);
      return;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int me = m + e;
      if (me >= M) break;
      const int be = (int)Tq.div((uint32_t)me);
      const int te = me - be * (int)Tq.d;
      vt[(((size_t)be * H + head) * hs + d) * kvT + t0 + te] = Elem<T>::from_f32(v[e]);
    }
  }
};

struct EpiResidual {
  static constexpr bool kPreload = true, kBias = true, kTransposed = false, kRowReduce = false, kRowArgmax = false;
  const float* bias;  // [N]
  float* x;           // [M][ldx] fp32 residual stream, updated in place
  int ldx;
  // When set, the residual is read from here ([M][ldx]) and x = xin + C is
  // written: the update goes to a copy without copying first.
  const float* xin = nullptr;
  __device__ __forceinline__ float4 bias4(int n) const { return *reinterpret_cast<const float4*>(bias + n); }
  __device__ __forceinline__ float4 preload(int m, int n) const {
    return *reinterpret_cast<const float4*>((xin ? xin : x) + (size_t)m * ldx + n);
  }
  __device__ __forceinline__ bool transposed(int) const { return false; }
  __device__ __forceinline__ void apply(int m, int n, const f32x4_t& v, const float4& r) const {
    *reinterpret_cast<float4*>(x + (size_t)m * ldx + n) = make_float4(r.x + v[0], r.y + v[1], r.z + v[2], r.w + v[3]);
  }
  __device__ __forceinline__ void apply_t(int, int, const f32x4_t&) const {}
};

// kErf picks the GELU form at compile time (false: gelu_new, the tanh form;
// true: the erf GELU).  As a run-time flag it put both forms and a branch
// around every four outputs of the epilogue, so the compiler could not
// overlap the exponentials and reciprocals of a batch of staged reads.
template <typename T, bool kErf = false>
struct EpiGelu {
  static constexpr bool kPreload = false, kBias = true, kTransposed = false, kRowReduce = false, kRowArgmax = false;
  const float* bias;  // [N]
  T* u;               // [M][ldu]
  int ldu;
  __device__ __forceinline__ float4 bias4(int n) const { return *reinterpret_cast<const float4*>(bias + n); }
  __device__ __forceinline__ float4 preload(int, int) const { return float4{}; }
  __device__ __forceinline__ bool transposed(int) const { return false; }
  __device__ __forceinline__ void apply(int m, int n, const f32x4_t& v, const float4&) const {
    if constexpr (kErf)
      Elem<T>::store4(u + (size_t)m * ldu + n, gelu_erf(v[0]), gelu_erf(v[1]), gelu_erf(v[2]), gelu_erf(v[3]));
    else
      Elem<T>::store4(u + (size_t)m * ldu + n, gelu_tanh(v[0]), gelu_tanh(v[1]), gelu_tanh(v[2]), gelu_tanh(v[3]));
  }
  __device__ __forceinline__ void apply_t(int, int, const f32x4_t&) const {}
};

// Logits rows of ldo elements (ldo >= vocabulary size; rows are only
// element-aligned unless ldo is a multiple of 64), fp32 or bf16 (O): each
// 4-column group goes out as one 16- or 8-byte store (8-column groups as one
// 16-byte store for bf16), masked per element at the n_valid edge.  The whole
// vectors are non-temporal stores: the logits (0.8-1.6 GB at GPT-2 small
// B=8 T=1024) exceed the memory-side cache anyway, and keeping them out of it
// leaves the next kernels' data cached (forward 3.088 -> 3.069 ms, same-box
// A/B; the lm_head itself unchanged).
typedef float f32x4_u4_t __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2_u2_t __attribute__((ext_vector_type(2), aligned(2)));
typedef uint32_t u32x4_u2_t __attribute__((ext_vector_type(4), aligned(2)));
template <typename O>
struct EpiLogits {
  static constexpr bool kPreload = false, kBias = false, kTransposed = false, kRowReduce = false, kRowArgmax = false;
  O* out;       // [M][ldo], only columns n < n_valid are written
  int ldo;
  int n_valid;
  __device__ __forceinline__ float4 bias4(int) const { return float4{}; }
  __device__ __forceinline__ float4 preload(int, int) const { return float4{}; }
  __device__ __forceinline__ bool transposed(int) const { return false; }
  __device__ __forceinline__ void apply(int m, int n, const f32x4_t& v, const float4&) const {
    O* p = out + (size_t)m * ldo + n;
    if (n + 3 < n_valid) {
      if constexpr (sizeof(O) == 4) {
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4_u4_t*>(p));
      } else {
        *reinterpret_cast<u32x2_u2_t*>(p) = u32x2_u2_t{pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3])};
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n + e < n_valid) p[e] = Elem<O>::from_f32(v[e]);
    }
  }
  __device__ __forceinline__ void apply_t(int, int, const f32x4_t&) const {}
  // bf16 logits only: v = C[m][n .. n+7] already packed (two per 32 bits),
  // one 16-byte store
  template <typename Q = O>
    requires(sizeof(Q) == 2)
  __device__ __forceinline__ void store8_packed(int m, int n, const u32x4_t& v) const {
    O* p = out + (size_t)m * ldo + n;
    if (n + 7 < n_valid) {
      __builtin_nontemporal_store(u32x4_u2_t{v[0], v[1], v[2], v[3]}, reinterpret_cast<u32x4_u2_t*>(p));
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (n + e < n_valid) p[e].bits = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
    }
  }
  // bf16 logits only: a = C[m][n .. n+3], b = C[m][n+4 .. n+7], one 16-byte store
  template <typename Q = O>
    requires(sizeof(Q) == 2)
  __device__ __forceinline__ void apply8(int m, int n, const f32x4_t& a, const f32x4_t& b) const {
    O* p = out + (size_t)m * ldo + n;
    if (n + 7 < n_valid) {
      __builtin_nontemporal_store(
          u32x4_u2_t{pack2_bf16(a[0], a[1]), pack2_bf16(a[2], a[3]), pack2_bf16(b[0], b[1]), pack2_bf16(b[2], b[3])},
          reinterpret_cast<u32x4_u2_t*>(p));
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (n + e < n_valid) p[e] = Elem<O>::from_f32(e < 4 ? a[e] : b[e - 4]);
    }
  }
};

// Backward-pass epilogues (block backward).
// Plain store of C (fp32 or T) into out[M][ldo]; in a split-K launch slice y
// stores its partial sum at out + y * split_stride.
template <typename O>
struct EpiStore {
  static constexpr bool kPreload = false, kBias = false, kTransposed = false, kRowReduce = false,
                        kRowArgmax = false;
  O* out;
  int ldo;
  size_t split_stride = 0;
  __device__ __forceinline__ float4 bias4(int) const { return float4{}; }
  __device__ __forceinline__ float4 preload(int, int) const { return float4{}; }
  __device__ __forceinline__ bool transposed(int) const { return false; }
  __device__ __forceinline__ void apply(int m, int n, const f32x4_t& v, const float4&) const {
    Elem<O>::store4(out + blockIdx.y * split_stride + (size_t)m * ldo + n, v[0], v[1], v[2], v[3]);
  }
  __device__ __forceinline__ void apply_t(int, int, const f32x4_t&) const {}
};

// c_fc of the recomputed forward: as EpiGelu, and the pre-activation (with
// bias) kept in fp32 for the derivative.
template <typename T, bool kErf = false>
struct EpiGeluSave {
  static constexpr bool kPreload = false, kBias = true, kTransposed = false, kRowReduce = false,
                        kRowArgmax = false;
  const float* bias;  // [N]
  T* u;               // [M][ld]
  float* g;           // [M][ld]
  int ld;
  __device__ __forceinline__ float4 bias4(int n) const { return *reinterpret_cast<const float4*>(bias + n); }
  __device__ __forceinline__ float4 preload(int, int) const { return float4{}; }
  __device__ __forceinline__ bool transposed(int) const { return false; }
  __device__ __forceinline__ void apply(int m, int n, const f32x4_t& v, const float4&) const {
    *reinterpret_cast<float4*>(g + (size_t)m * ld + n) = make_float4(v[0], v[1], v[2], v[3]);
    if constexpr (kErf)
      Elem<T>::store4(u + (size_t)m * ld + n, gelu_erf(v[0]), gelu_erf(v[1]), gelu_erf(v[2]), gelu_erf(v[3]));
    else
      Elem<T>::store4(u + (size_t)m * ld + n, gelu_tanh(v[0]), gelu_tanh(v[1]), gelu_tanh(v[2]), gelu_tanh(v[3]));
  }
  __device__ __forceinline__ void apply_t(int, int, const f32x4_t&) const {}
};

// dG = dU * act'(G): C is dU = dY W_pr^T, G the kept pre-activation.
template <typename T, bool kErf = false>
struct EpiGeluBwd {
  static constexpr bool kPreload = true, kBias = false, kTransposed = false, kRowReduce = false,
                        kRowArgmax = false;
  const float* g;  // [M][ld]
  T* dg;           // [M][ld]
  int ld;
  __device__ __forceinline__ float4 bias4(int) const { return float4{}; }
  __device__ __forceinline__ float4 preload(int m, int n) const {
    return *reinterpret_cast<const float4*>(g + (size_t)m * ld + n);
  }
  __device__ __forceinline__ bool transposed(int) const { return false; }
  __device__ __forceinline__ void apply(int m, int n, const f32x4_t& v, const float4& x) const {
    float d0, d1, d2, d3;
    if constexpr (kErf) {
      d0 = gelu_erf_grad(x.x), d1 = gelu_erf_grad(x.y), d2 = gelu_erf_grad(x.z), d3 = gelu_erf_grad(x.w);
    } else {
      d0 = gelu_tanh_grad(x.x), d1 = gelu_tanh_grad(x.y), d2 = gelu_tanh_grad(x.z), d3 = gelu_tanh_grad(x.w);
    }
    Elem<T>::store4(dg + (size_t)m * ld + n, v[0] * d0, v[1] * d1, v[2] * d2, v[3] * d3);
  }
  __device__ __forceinline__ void apply_t(int, int, const f32x4_t&) const {}
};

// Next-token cross-entropy partials of the tied lm_head (pwwt.cn
// "逐行拆GPT-2源码", GPT2LMHeadModel: logits of position t are scored against
// the label of position t + 1): the logits are reduced in registers and never
// stored.  Row m = b*T + t of the product has label labels[m + 1] when
// t < T - 1, none otherwise.
struct EpiCE {
  static constexpr bool kPreload = false, kBias = false, kTransposed = false, kRowReduce = true, kRowArgmax = false;
  float2* part;            // [M][nseg]: (max, sum of exp(C - max)) per column slice
  int nseg;                // slices per row
  const int32_t* labels;   // [M]
  FastDiv T;               // positions per sequence
  int n_valid;             // vocabulary size: columns >= n_valid are padding
  float* tgt;              // [M]: C[m][label], written only for labels in [0, n_valid)
  __device__ __forceinline__ float4 bias4(int) const { return float4{}; }
  __device__ __forceinline__ float4 preload(int, int) const { return float4{}; }
  __device__ __forceinline__ bool transposed(int) const { return false; }
  __device__ __forceinline__ void apply(int, int, const f32x4_t&, const float4&) const {}
  __device__ __forceinline__ void apply_t(int, int, const f32x4_t&) const {}
  __device__ __forceinline__ int label(int m) const {
    const int t = m - (int)T.div((uint32_t)m) * (int)T.d;
    return t + 1 < (int)T.d ? labels[m + 1] : -1;
  }
  __device__ __forceinline__ void partial(int m, int s, float mx, float sum) const {
    part[(size_t)m * nseg + s] = make_float2(mx, sum);
  }
  __device__ __forceinline__ void target(int m, float v) const { tgt[m] = v; }
};

// Greedy token choice of the tied lm_head (the generation loop): per row m
// and column slice s, the largest C[m][n] over the slice's columns below
// n_valid and the first column holding it; the logits are not stored.
struct EpiArgmax {
  static constexpr bool kPreload = false, kBias = false, kTransposed = false, kRowReduce = false,
                        kRowArgmax = true;
  int2* part;   // [M][nseg]: (bits of the slice maximum, its first column)
  int nseg;     // slices per row
  int n_valid;  // vocabulary size
  __device__ __forceinline__ float4 bias4(int) const { return float4{}; }
  __device__ __forceinline__ float4 preload(int, int) const { return float4{}; }
  __device__ __forceinline__ bool transposed(int) const { return false; }
  __device__ __forceinline__ void apply(int, int, const f32x4_t&, const float4&) const {}
  __device__ __forceinline__ void apply_t(int, int, const f32x4_t&) const {}
  __device__ __forceinline__ void partial(int m, int s, float v, int col) const {
    part[(size_t)m * nseg + s] = make_int2(__builtin_bit_cast(int, v), col);
  }
  // the value compared for row m, column col: the logit itself
  __device__ __forceinline__ uint64_t row_key(int) const { return 0; }
  __device__ __forceinline__ float score(uint64_t, int, float v) const { return v; }
};

// SplitMix64 output function (Steele, Lea and Flood, "Fast splittable
// pseudorandom number generators", OOPSLA 2014): the state advanced by the
// golden-ratio increment, then two xor-shift-multiply rounds.
__host__ __device__ inline uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Sampling from softmax(logits / temperature) by the Gumbel-max identity:
// argmax_v (logit_v / temperature + G_v) with G_v = -ln(-ln U_v) independent
// standard Gumbel variables is distributed as that softmax (huaweicloud blog
// 476445, architecture overview: softmax over the vocabulary, then a token is
// picked).  U_v comes from a counter-based generator, so the draw depends only
// on (seed, position, row, column):
//   key_row = splitmix64(splitmix64(seed) ^ (position << 32) ^ row)
//   U_v     = ((splitmix64(key_row ^ v) >> 40) + 1/2) / 2^24, in (0, 1).
// Same slice partials as EpiArgmax, with the perturbed score in place of the
// logit.
struct EpiSample {
  static constexpr bool kPreload = false, kBias = false, kTransposed = false, kRowReduce = false,
                        kRowArgmax = true;
  int2* part;       // [M][nseg]: (bits of the slice's largest score, its first column)
  int nseg;
  int n_valid;      // vocabulary size
  uint64_t seed_mix;  // splitmix64(seed)
  int pos;          // position of the step's input token
  float inv_temp;   // 1 / temperature
  __device__ __forceinline__ float4 bias4(int) const { return float4{}; }
  __device__ __forceinline__ float4 preload(int, int) const { return float4{}; }
  __device__ __forceinline__ bool transposed(int) const { return false; }
  __device__ __forceinline__ void apply(int, int, const f32x4_t&, const float4&) const {}
  __device__ __forceinline__ void apply_t(int, int, const f32x4_t&) const {}
  __device__ __forceinline__ void partial(int m, int s, float v, int col) const {
    part[(size_t)m * nseg + s] = make_int2(__builtin_bit_cast(int, v), col);
  }
  __device__ __forceinline__ uint64_t row_key(int m) const {
    return splitmix64(seed_mix ^ ((uint64_t)(uint32_t)pos << 32) ^ (uint64_t)(uint32_t)m);
  }
  __device__ __forceinline__ float score(uint64_t key, int col, float v) const {
    const uint64_t z = splitmix64(key ^ (uint64_t)(uint32_t)col);
    const float u = ((float)(uint32_t)(z >> 40) + 0.5f) * 5.9604644775390625e-8f;  // 2^-24
    // -ln(-ln u) through the hardware base-2 logarithm: ln x = log2(x) ln 2
    const float ln2 = 0.69314718055994531f;
    const float e = -__builtin_amdgcn_logf(u) * ln2;  // -ln u > 0
    return v * inv_temp - __builtin_amdgcn_logf(e) * ln2;
  }
};

// Host launchers (gemm.hip).  Shapes: A [M][lda], B [N][ldb] (K contiguous),
// K % (128 / sizeof(T)) == 0, N % 4 == 0.  `tile` picks the tile shape
// (see gemm.hip); returns hipSuccess or the launch error.
enum GemmTile {
  kTile128x128 = 0,
  kTile256x256 = 1,
  kTile64x64 = 2,
  kTile32x64 = 3,
  kTile64x128 = 4,
  kTile128x96 = 5,
  kTile128x192 = 6  // 8 waves of 64x48, one block per CU
};

// Width of the column slice one wave owns in `tile` (the kRowReduce slice).
int gemm_slice_width(GemmTile tile);

template <typename T, class Epi>
hipError_t launch_gemm(GemmTile tile, const T* A, const T* B, int M, int N, int K, int lda, int ldb,
                       const Epi& epi, hipStream_t stream);

// Split-K: `splits` slices of K_split each (A and B advance by K_split per
// slice; lda, ldb >= splits * K_split); slice y writes its partial product to
// epi.out + y * epi.split_stride (the caller adds the slices).
template <typename T>
hipError_t launch_gemm_splitk(GemmTile tile, const T* A, const T* B, int M, int N, int K_split, int lda, int ldb,
                              int splits, const EpiStore<float>& epi, hipStream_t stream);

// Both operands K-major (bf16): C[m][n] = sum_k A[k][m] B[k][n] with A
// [K][M] (row stride lda) and B [K][N] (row stride ldb), e.g. a weight
// gradient X^T dY straight from the activations as the forward stored them,
// no transposed copies.  128x128 tiles; split-K as launch_gemm_splitk (slice
// y covers rows [y*K_split, (y+1)*K_split) of A and B).  M, N, lda, ldb
// multiples of 8 (whole 16-byte chunks), K_split a multiple of 64.
hipError_t launch_gemm_kmajor(const bf16_t* A, const bf16_t* B, int M, int N, int K_split, int lda, int ldb,
                              int splits, const EpiStore<float>& epi, hipStream_t stream);

// M <= 32 (decode): one kernel for the product and the fused epilogue `epi`;
// K % 32 == 0 (bf16) or K % 16 == 0 (fp32), no workspace.
template <typename T, class Epi>
hipError_t launch_gemm_skinny(const T* A, const T* B, int M, int N, int K, int lda, int ldb, const Epi& epi,
                              hipStream_t stream);

// M <= 32, no epilogue: part[s][m][n] (s < skinny_splits(K, sizeof(T)), fp32)
// receives the partial product of the s-th k range; the consumer adds them.
int skinny_splits(int K, int elem_bytes);
template <typename T>
hipError_t launch_gemm_skinny_splitk(const T* A, const T* B, int M, int N, int K, int lda, int ldb, float* part,
                                     hipStream_t stream);

}  // namespace gpt2
