// Causal attention on gfx950 (see attention.h for what is computed).
//
// Prefill kernel (flash-style):
//   * one block = 4 waves of QW queries (kPrefillQW = 16: 64 queries) of one
//     (b, h); blocks of the longest query tiles are launched first (causal
//     work grows with the tile index).
//   * key tiles (kPrefillKeys: 32 keys for bf16, 64 for fp32) are staged in
//     LDS (K as [key][d], V transposed as [d][key]) through a double-buffered
//     ring; the next tile's global loads are in flight while the current one
//     is on the matrix cores.  32-key bf16 tiles take 16 KB of LDS per block
//     and 71 registers, so 7 waves share a SIMD (64-key tiles: 32 KB, 95
//     registers, 5 waves); that outweighs their twice as many barriers and
//     per-tile reductions.
//   * each wave computes S^T = K Q^T with MFMA (lane l ends with 4 keys of one
//     query), keeps a running max and sum per query (online softmax, fp32,
//     the running max subtracted before exp as the llm.c notes advise), then
//     O^T += V^T P^T with MFMA.  Everything per query stays in the lane that
//     holds that query, so rescaling needs no cross-lane traffic.
//   * key tiles that lie entirely after a wave's last query are skipped; only
//     tiles that straddle the diagonal evaluate the mask.
//   * keys past the last valid position are clamped on load (K) or zeroed in
//     LDS (V), so uninitialised cache rows never reach the arithmetic.
#include "attention.h"

namespace gpt2 {

namespace {

// max over the lanes l, l^16, l^32, l^48 (the four lane groups holding one
// query of an MFMA fragment).
__device__ __forceinline__ float max_over_lane_groups(float v) {
  const auto mx = [](float a, float b) { return fmaxf(a, b); };
  return combine_xor32(combine_xor16(v, mx), mx);
}

template <int CH>
__device__ __forceinline__ int swz_ch(int row, int c) {
  return c ^ (row & ((CH < 8 ? CH : 8) - 1));
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Block barrier without a memory fence (a fence would also wait for the next
// tile's loads in flight); callers wait for their own loads first.
__device__ __forceinline__ void barrier_nofence() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Keys per K/V tile of the prefill kernel (fp32 keeps 64: with 32 keys its
// head_dim-16 V^T tile would not split over the four waves' loads).
template <typename T>
constexpr int kPrefillKeys = sizeof(T) == 2 ? 32 : 64;

template <typename T, int HS, int QW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(QW == 16 ? (sizeof(T) == 2 ? 6 : 5) : 3))) void attn_prefill_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ vt, T* __restrict__ out, int BH, int H,
    int Tq, int kvT, int n_qtiles, float* __restrict__ lse) {
  constexpr int NW = 4, BQ = QW * NW, BKEYS = kPrefillKeys<T>;
  constexpr int ESZ = (int)sizeof(T);
  constexpr int KROWB = HS * ESZ, KCH = KROWB / 16;     // K tile rows (keys)
  constexpr int VROWB = BKEYS * ESZ, VCH = VROWB / 16;  // V^T tile rows (d)
  constexpr int NSLAB = KROWB / 64;
  constexpr int KF = BKEYS / 16, DF = HS / 16, QF = QW / 16;
  constexpr int KPS = Mma<T>::kPerSlab;      // keys per PV matrix step
  constexpr int EPC = 16 / ESZ;              // elements per 16-byte chunk
  constexpr int K_CHUNKS = BKEYS * KCH, V_CHUNKS = HS * VCH;
  // direct global->LDS loads: one instruction fills 64 consecutive chunks
  constexpr int KI = K_CHUNKS / 64 / NW, VI = V_CHUNKS / 64 / NW;  // instructions per wave per tile
  static_assert(NSLAB >= 1 && KROWB % 64 == 0, "head_dim bytes must be a multiple of 64");
  static_assert(KI * 64 * NW == K_CHUNKS && VI * 64 * NW == V_CHUNKS && KI >= 1 && VI >= 1, "tile split");
  static_assert(KI + VI <= 63, "loads in flight must fit the vmcnt counter");

  // Dynamic LDS: with the two buffers in one dynamic allocation the compiler
  // does not wait for the next tile's DMA (in flight into the other buffer)
  // before reading this one; as static arrays it did, every tile.
  extern __shared__ u32x4_t attn_lds[];
  u32x4_t(*sK)[K_CHUNKS] = reinterpret_cast<u32x4_t(*)[K_CHUNKS]>(attn_lds);
  u32x4_t(*sV)[V_CHUNKS] = reinterpret_cast<u32x4_t(*)[V_CHUNKS]>(attn_lds + 2 * K_CHUNKS);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  // Work order: longest query tiles first, reversed within every other run
  // of 256 blocks, so that the blocks one CU receives (one per run when all
  // are resident) pair long tiles with short ones.
  int widx = blockIdx.x;
  {
    const int run = widx >> 8, pos = widx & 255;
    if ((run & 1) && (run << 8) + 256 <= (int)gridDim.x) widx = (run << 8) + (255 - pos);
  }
  const int bh = widx % BH;
  const int qt = n_qtiles - 1 - widx / BH;
  const int b = bh / H, h = bh - b * H;
  const int D = H * HS;

  const int q_blk = qt * BQ;
  const int q0w = q_blk + wave * QW;
  const int q_end = min(q_blk + BQ, Tq);        // exclusive, block's last query + 1
  const int n_kt = (q_end + BKEYS - 1) / BKEYS;  // key tiles this block needs
  const int nkeys = Tq;                           // valid key positions

  const T* qb = q + (size_t)bh * Tq * HS;
  const T* kb = k + (size_t)bh * kvT * HS;
  const T* vb = vt + (size_t)bh * HS * kvT;

  // K tile row r holds key key_of_row(r) of the tile.  For bf16 the rows are
  // permuted within each 32-key group (r = 16h + 4g + i holds key 8g + 4h + i)
  // so that the S^T fragments give lane group g the probabilities of keys
  // 8g .. 8g+7 of the group: exactly the 16 contiguous bytes of a V^T row that
  // the same lane supplies to the P V product.
  auto key_of_row = [](int r) {
    if constexpr (ESZ == 2) return (r & ~31) | (((r >> 2) & 3) << 3) | (((r >> 4) & 1) << 2) | (r & 3);
    else return r;
  };

  // Query fragments stay in registers: lane (lr, lg) holds query q0w+qf*16+lr,
  // bytes slab*64 + lg*16 .. +16 of its row.
  u32x4_t qfrag[QF][NSLAB];
#pragma unroll
  for (int qf = 0; qf < QF; ++qf) {
    int row = min(q0w + qf * 16 + lr, Tq - 1);
    const char* p = reinterpret_cast<const char*>(qb + (size_t)row * HS);
#pragma unroll
    for (int s = 0; s < NSLAB; ++s) qfrag[qf][s] = *reinterpret_cast<const u32x4_t*>(p + s * 64 + lg * 16);
  }

  // Tile loads: wave instruction j fills LDS chunks (j*NW + wave)*64 + lane;
  // chunk slot s of row r holds the row's global chunk swz_ch(r, s) (the XOR
  // swizzle is an involution).  Keys past the end are clamped to the last
  // valid one for K (their scores are masked) and fixed up for V^T below.
  // Per-thread source offsets within a tile (bytes), fixed over the tiles:
  // K row key_of_row(row), swizzled chunk; V^T row d, swizzled chunk.
  int koff[KI], krow[KI], voff[VI], vcol[VI];
#pragma unroll
  for (int j = 0; j < KI; ++j) {
    const int ci = (j * NW + wave) * 64 + lane;
    const int row = ci / KCH, slot = ci % KCH;
    krow[j] = key_of_row(row);
    koff[j] = krow[j] * KROWB + swz_ch<KCH>(row, slot) * 16;
  }
#pragma unroll
  for (int j = 0; j < VI; ++j) {
    const int ci = (j * NW + wave) * 64 + lane;
    const int d = ci / VCH, slot = ci % VCH;
    vcol[j] = swz_ch<VCH>(d, slot) * EPC;
    voff[j] = d * kvT * ESZ + vcol[j] * ESZ;
  }
  auto issue = [&](int kt, int buf) {
    const char* kt_base = reinterpret_cast<const char*>(kb + (size_t)kt * BKEYS * HS);
    const char* vt_base = reinterpret_cast<const char*>(vb + (size_t)kt * BKEYS);
    const bool tail = (kt + 1) * BKEYS > nkeys;  // block-uniform
#pragma unroll
    for (int j = 0; j < KI; ++j) {
      const char* src = kt_base + koff[j];
      if (tail && kt * BKEYS + krow[j] >= nkeys)  // past the last key: read the last valid row (masked)
        src += (nkeys - 1 - kt * BKEYS - krow[j]) * KROWB;
      __builtin_amdgcn_global_load_lds((const void*)src,
                                       (__attribute__((address_space(3))) void*)&sK[buf][(j * NW + wave) * 64], 16,
                                       0, 0);
    }
#pragma unroll
    for (int j = 0; j < VI; ++j) {
      const char* src = vt_base + voff[j];
      // chunks wholly past the end read the tile's first chunk instead (in bounds; zeroed below)
      if (tail && kt * BKEYS + vcol[j] >= nkeys) src -= vcol[j] * ESZ;
      __builtin_amdgcn_global_load_lds((const void*)src,
                                       (__attribute__((address_space(3))) void*)&sV[buf][(j * NW + wave) * 64], 16,
                                       0, 0);
    }
  };
  // V^T of a tile that runs past the last key: zero the keys >= nkeys (their
  // probabilities are 0, but the cache there is uninitialised and 0 * NaN is NaN).
  auto fix_tail = [&](int kt, int buf) {
    const int valid = nkeys - kt * BKEYS;  // 1 .. BKEYS-1
    T* base = reinterpret_cast<T*>(&sV[buf][0]);
    for (int idx = tid; idx < HS * BKEYS; idx += 256) {
      const int d = idx / BKEYS, key = idx % BKEYS;
      if (key >= valid) base[(d * VCH + swz_ch<VCH>(d, key / EPC)) * EPC + key % EPC] = Elem<T>::from_f32(0.f);
    }
  };

  // Running state per query (lane (lr, lg) holds query q0w + qf*16 + lr):
  //   m_run  reference maximum the exponentials are taken against;
  //   o      O^T[d = df*16 + 4*lg + e][query], unnormalised;
  //   lsum   row sums of P, all four elements equal, produced by the matrix
  //          cores as 1^T P^T (a fragment of ones in place of V^T).
  // The reference maximum is only moved when a tile's maximum exceeds it by
  // more than kSlack (so exp2 arguments stay <= kSlack * log2 e, far from
  // overflow): most tiles then need no rescaling of o and lsum at all.
  constexpr float kSlack = 5.5f;
  f32x4_t o[DF][QF], lsum[QF];
  float m_run[QF], mb[QF];
#pragma unroll
  for (int qf = 0; qf < QF; ++qf) {
    m_run[qf] = -INFINITY;
    mb[qf] = -INFINITY;
    lsum[qf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int df = 0; df < DF; ++df) o[df][qf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const u32x4_t ones = ESZ == 2 ? u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u}
                                : u32x4_t{0x3F800000u, 0x3F800000u, 0x3F800000u, 0x3F800000u};

  issue(0, 0);
  wait_vmcnt<0>();
  barrier_nofence();
  if (BKEYS > nkeys) {
    fix_tail(0, 0);
    __syncthreads();
  }

  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    // the other buffer was released by the barrier that ended the previous tile
    if (kt + 1 < n_kt) issue(kt + 1, buf ^ 1);
    const int key0 = kt * BKEYS;
    if (key0 <= q0w + QW - 1) {  // wave-uniform: otherwise the whole tile is masked for this wave
      // S^T = K Q^T: lane holds S^T[key = key0 + key_of_row(kf*16 + 4*lg + e)][query = q0w + qf*16 + lr]
      f32x4_t s[KF][QF];
      u32x4_t kfr[NSLAB][KF];
#pragma unroll
      for (int sl = 0; sl < NSLAB; ++sl)
#pragma unroll
        for (int kf = 0; kf < KF; ++kf) {
          const int row = kf * 16 + lr;
          kfr[sl][kf] = sK[buf][row * KCH + swz_ch<KCH>(row, sl * 4 + lg)];
        }
#pragma unroll
      for (int sl = 0; sl < NSLAB; ++sl) {
#pragma unroll
        for (int kf = 0; kf < KF; ++kf) {
#pragma unroll
          for (int qf = 0; qf < QF; ++qf) {
            if (sl == 0) s[kf][qf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            Mma<T>::run(s[kf][qf], kfr[sl][kf], qfrag[qf][sl]);
          }
        }
      }
      if (key0 + BKEYS - 1 > q0w) {  // the tile straddles this wave's diagonal
#pragma unroll
        for (int qf = 0; qf < QF; ++qf) {
          const int lim = q0w + qf * 16 + lr - key0;  // tile keys > lim are masked
#pragma unroll
          for (int kf = 0; kf < KF; ++kf)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (key_of_row(kf * 16 + 4 * lg + e) > lim) s[kf][qf][e] = -INFINITY;
        }
      }
      // V^T fragments of the first matrix step, read now: their LDS latency
      // then passes under the softmax arithmetic below
      constexpr int NPRE = DF >= 2 ? DF / 2 : 1;
      u32x4_t vpre[NPRE];
#pragma unroll
      for (int df = 0; df < NPRE; ++df) {
        const int d = df * 16 + lr;
        vpre[df] = sV[buf][d * VCH + swz_ch<VCH>(d, lg)];
      }
      // tile maximum per query: 16 values in the lane, then across the four
      // lanes (lr, lr+16, lr+32, lr+48) that hold the same query
      float mx[QF];
      bool grow = false;
#pragma unroll
      for (int qf = 0; qf < QF; ++qf) {
        float m = fmaxf(s[0][qf][0], s[0][qf][1]);
#pragma unroll
        for (int kf = 0; kf < KF; ++kf)
#pragma unroll
          for (int e = (kf == 0 ? 2 : 0); e < 4; ++e) m = fmaxf(m, s[kf][qf][e]);
        m = max_over_lane_groups(m);
        mx[qf] = m;
        grow |= m > m_run[qf] + kSlack;
      }
      if (__any(grow)) {
#pragma unroll
        for (int qf = 0; qf < QF; ++qf) {
          const float m_new = fmaxf(m_run[qf], mx[qf]);
          const float alpha = __builtin_amdgcn_exp2f((m_run[qf] - m_new) * kLog2e);
          m_run[qf] = m_new;
          mb[qf] = m_new * kLog2e;
          lsum[qf] *= alpha;
#pragma unroll
          for (int df = 0; df < DF; ++df) o[df][qf] *= alpha;
        }
      }
#pragma unroll
      for (int qf = 0; qf < QF; ++qf)
#pragma unroll
        for (int kf = 0; kf < KF; ++kf)
#pragma unroll
          for (int e = 0; e < 4; ++e) s[kf][qf][e] = __builtin_amdgcn_exp2f(fmaf(s[kf][qf][e], kLog2e, -mb[qf]));

      // O^T += V^T P^T and lsum += 1^T P^T, KPS keys per matrix step
#pragma unroll
      for (int st = 0; st < BKEYS / KPS; ++st) {
        u32x4_t pf[QF];
#pragma unroll
        for (int qf = 0; qf < QF; ++qf) {
          if constexpr (ESZ == 2) {
            const f32x4_t& p0 = s[st * 2][qf];
            const f32x4_t& p1 = s[st * 2 + 1][qf];
            pf[qf] = u32x4_t{pack2_bf16(p0[0], p0[1]), pack2_bf16(p0[2], p0[3]), pack2_bf16(p1[0], p1[1]),
                             pack2_bf16(p1[2], p1[3])};
          } else {
            pf[qf] = __builtin_bit_cast(u32x4_t, s[st][qf]);
          }
          Mma<T>::run(lsum[qf], ones, pf[qf]);
        }
        u32x4_t vf[DF];
#pragma unroll
        for (int df = 0; df < DF; ++df) {
          const int d = df * 16 + lr;
          // bf16: keys st*32 + 8*lg .. +7; fp32: keys st*16 + 4*lg .. +3 (16 bytes)
          vf[df] = st == 0 && df < NPRE ? vpre[df < NPRE ? df : 0] : sV[buf][d * VCH + swz_ch<VCH>(d, st * 4 + lg)];
        }
#pragma unroll
        for (int df = 0; df < DF; ++df)
#pragma unroll
          for (int qf = 0; qf < QF; ++qf) Mma<T>::run(o[df][qf], vf[df], pf[qf]);
      }
    }
    if (kt + 1 < n_kt) {
      wait_vmcnt<0>();   // this wave's part of the next tile has landed
      barrier_nofence();  // ... everyone's, and everyone is done with this tile
      if ((kt + 2) * BKEYS > nkeys) {
        fix_tail(kt + 1, buf ^ 1);
        __syncthreads();
      }
    }
  }

  // Normalise and merge heads: lane holds O^T[d = df*16 + 4*lg + e][query = q0w + qf*16 + lr]
#pragma unroll
  for (int qf = 0; qf < QF; ++qf) {
    const float inv = 1.0f / lsum[qf][0];
    const int qi = q0w + qf * 16 + lr;
    // optional log-sum-exp of the query's scores (for the backward pass)
    if (lse && lg == 0 && qi < Tq) lse[((size_t)b * H + h) * Tq + qi] = m_run[qf] + logf(lsum[qf][0]);
    if (qi < Tq) {
      T* dst = out + ((size_t)b * Tq + qi) * D + h * HS;
#pragma unroll
      for (int df = 0; df < DF; ++df)
        Elem<T>::store4(dst + df * 16 + 4 * lg, o[df][qf][0] * inv, o[df][qf][1] * inv, o[df][qf][2] * inv,
                        o[df][qf][3] * inv);
    }
  }
}

// ---------------------------------------------------------------- decode

constexpr int kDecKeys = 256;  // keys per slice (256 threads)
constexpr int kDecMaxSlices = 4;  // slices one fused block merges (1024 threads)
constexpr int kDecFusedMinBH = 96;  // (b, h) pairs from which one block per pair fills the chip

template <typename T, int HS>
struct DecSlice {
  static constexpr int EPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  static constexpr int KCH = HS / EPC;             // chunks per K row
  static constexpr int ROWS_K = 256 / KCH;         // K rows per pass
  static constexpr int VCH = kDecKeys / EPC;       // chunks per V^T row (256 keys)
  static constexpr int ROWS_V = 256 / VCH;         // V^T rows per pass
  static constexpr int PK = kDecKeys / ROWS_K, PV = HS / ROWS_V;
  static_assert(KCH >= 1 && KCH <= 64 && (KCH & (KCH - 1)) == 0, "K chunking");
  float sp[kDecKeys];
  float sred[8];
  float so[HS][VCH + 1];
};

// One slice of up to 256 keys [j0, j0 + nj) of one (b, h), taken by 256
// threads (t = 0..255).  Every global read is a 16-byte coalesced run: K rows
// are read KCH lanes per row (each lane a 16-byte chunk of head_dim), V^T rows
// VCH lanes per row (each lane EPC consecutive keys).  q and all K loads of
// the slice are issued at once, the first VP of its V^T passes with them
// (their stream then overlaps the scores and the softmax), the rest after
// the softmax.  VP = PV where registers are plentiful (the split kernel), 0
// where every block must be resident at once (the fused kernel).  The cache
// is read with non-temporal loads: a decode step streams the whole cache
// (1.2 GB at GPT-2 small B=32, prefix 1023) and reads each row once, and
// keeping it out of the caches leaves the layers' weights cached for the
// small products around the attention (decode step 0.597 -> 0.571 ms,
// same-box A/B).  Measured
// and not kept: half of V^T by LDS DMA in the fused kernel (the compiler
// then waits for every load in flight at the first use of any).  Returns the
// slice maximum mx and sum ls (all threads) and o[t] = sum_j e^{s_j - mx}
// v_j[t] (t < HS).
template <typename T, int HS, int VP>
__device__ __forceinline__ void decode_slice(const T* __restrict__ qrow, const T* __restrict__ kb,
                                             const T* __restrict__ vb, int nj, int kvT, int t,
                                             DecSlice<T, HS>& sm, float& mx_out, float& ls_out, float& o_out) {
  using S = DecSlice<T, HS>;
  constexpr int EPC = S::EPC, KCH = S::KCH, ROWS_K = S::ROWS_K, VCH = S::VCH, ROWS_V = S::ROWS_V;
  constexpr int PK = S::PK, PV = S::PV;
  static_assert(VP >= 0 && VP <= PV, "V passes in flight early");
  const int lane = t & 63;
  const int kc = t % KCH;
  const int vc = t % VCH;
  const bool chunk_ok = vc * EPC < nj;  // the chunk holds a key before nj
  // Every load is unconditional (branch-free, so the compiler can count the
  // loads in flight exactly): rows past the last key read the last key's row
  // (its score is masked), chunks wholly past it the row's first chunk (its
  // probabilities are zero and the values are not used).
  auto kload = [&](int p) {
    const int r = min(p * ROWS_K + t / KCH, nj - 1);
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kb + (size_t)r * HS + kc * EPC));
  };
  const int vcol = chunk_ok ? vc * EPC : 0;
  auto vload = [&](int p) {
    const int d = p * ROWS_V + t / VCH;
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vb + (size_t)d * kvT + vcol));
  };
  u32x4_t kraw[PK], vraw[PV];
  const u32x4_t qraw = *reinterpret_cast<const u32x4_t*>(qrow + kc * EPC);
#pragma unroll
  for (int p = 0; p < PK; ++p) kraw[p] = kload(p);
#pragma unroll
  for (int p = 0; p < VP; ++p) vraw[p] = vload(p);
  float qv[EPC];
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qv[2 * e] = bf16_to_f32(qraw[e] & 0xFFFF);
      qv[2 * e + 1] = bf16_to_f32(qraw[e] >> 16);
    }
  } else {
    const f32x4_t f = __builtin_bit_cast(f32x4_t, qraw);
#pragma unroll
    for (int e = 0; e < 4; ++e) qv[e] = f[e];
  }
  // scores: pass p covers rows p*ROWS_K .. +ROWS_K; KCH lanes per row
  // (computed for every row, masked after: no branch around a use of a load)
  auto score = [&](int p) {
    const int r = p * ROWS_K + t / KCH;
    float acc = 0.f;
    const u32x4_t raw = kraw[p];
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc += qv[2 * e] * bf16_to_f32(raw[e] & 0xFFFF) + qv[2 * e + 1] * bf16_to_f32(raw[e] >> 16);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc += qv[e] * __builtin_bit_cast(f32x4_t, raw)[e];
    }
#pragma unroll
    for (int o = KCH / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (t % KCH == 0) sm.sp[r] = r < nj ? acc : -INFINITY;
  };
#pragma unroll
  for (int p = 0; p < PK; ++p) score(p);
  __syncthreads();
  // softmax over the slice
  const float s = sm.sp[t];
  float mx = wave_max(s);
  if (lane == 0) sm.sred[t >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(sm.sred[0], sm.sred[1]), fmaxf(sm.sred[2], sm.sred[3]));
  const float pv = t < nj ? __builtin_amdgcn_exp2f((s - mx) * kLog2e) : 0.f;
  float ls = wave_sum(pv);
  __syncthreads();
  sm.sp[t] = pv;
  if (lane == 0) sm.sred[4 + (t >> 6)] = ls;
  __syncthreads();
  ls = sm.sred[4] + sm.sred[5] + sm.sred[6] + sm.sred[7];

  // o[d] = sum_j p_j V^T[d][j0 + j]: lane owns chunk vc (EPC keys) of rows d
#pragma unroll
  for (int p = VP; p < PV; ++p) vraw[p] = vload(p);
  float pk[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) pk[e] = sm.sp[vc * EPC + e];
  // (every element past the last key is selected to 0, its probability is 0:
  // no branch around a use of a load)
  float accv[PV];
#pragma unroll
  for (int p = 0; p < PV; ++p) {
    float acc = 0.f;
    const u32x4_t raw = vraw[p];
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v0 = vc * EPC + 2 * e < nj ? bf16_to_f32(raw[e] & 0xFFFF) : 0.f;
        const float v1 = vc * EPC + 2 * e + 1 < nj ? bf16_to_f32(raw[e] >> 16) : 0.f;
        acc += pk[2 * e] * v0 + pk[2 * e + 1] * v1;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v0 = vc * EPC + e < nj ? __builtin_bit_cast(f32x4_t, raw)[e] : 0.f;
        acc += pk[e] * v0;
      }
    }
    accv[p] = acc;
  }
#pragma unroll
  for (int p = 0; p < PV; ++p) sm.so[p * ROWS_V + t / VCH][vc] = accv[p];
  __syncthreads();
  float o = 0.f;
  if (t < HS) {
#pragma unroll 8
    for (int c = 0; c < VCH; ++c) o += sm.so[t][c];
  }
  mx_out = mx;
  ls_out = ls;
  o_out = o;
}

// One block per (bh, split) of up to 256 keys; writes the partial
// (o[HS], max, sum) of its split for attn_decode_merge_kernel.
template <typename T, int HS>
__global__ __launch_bounds__(256) void attn_decode_split_kernel(const T* __restrict__ q,
                                                                 const T* __restrict__ k,
                                                                 const T* __restrict__ vt,
                                                                 float* __restrict__ part, int n_keys,
                                                                 int kvT, int nsplit) {
  __shared__ DecSlice<T, HS> sm;
  const int tid = threadIdx.x;
  const int bh = blockIdx.x / nsplit, split = blockIdx.x % nsplit;
  const int j0 = split * kDecKeys;
  const int nj = min(kDecKeys, n_keys - j0);
  float mx, ls, o;
  constexpr int VP = sizeof(T) == 2 ? DecSlice<T, HS>::PV : 0;  // fp32 head_dim 64: too many registers
  decode_slice<T, HS, VP>(q + (size_t)bh * HS, k + ((size_t)bh * kvT + j0) * HS,
                          vt + (size_t)bh * HS * kvT + j0, nj, kvT, tid, sm, mx, ls, o);
  float* dst = part + ((size_t)bh * nsplit + split) * (HS + 2);
  if (tid < HS) dst[tid] = o;
  if (tid == 0) {
    dst[HS] = mx;
    dst[HS + 1] = ls;
  }
}

// One block per (b, h) for up to kDecMaxSlices slices: 256 threads per slice,
// the slices' (o, max, sum) merged in LDS by the same formula as
// attn_decode_merge_kernel, so the result is the same bits as the split +
// merge pair, in one launch and without the partials' round trip.
template <typename T, int HS>
__global__ __launch_bounds__(256 * kDecMaxSlices) __attribute__((amdgpu_waves_per_eu(8))) void attn_decode_fused_kernel(const T* __restrict__ q,
                                                                                const T* __restrict__ k,
                                                                                const T* __restrict__ vt,
                                                                                T* __restrict__ out, int n_keys,
                                                                                int kvT, int H) {
  __shared__ DecSlice<T, HS> sm[kDecMaxSlices];
  __shared__ float so[kDecMaxSlices][HS + 2];
  const int nsl = (int)blockDim.x / kDecKeys;
  const int slice = threadIdx.x / kDecKeys, t = threadIdx.x % kDecKeys;
  const int bh = blockIdx.x;
  const int j0 = slice * kDecKeys;
  const int nj = min(kDecKeys, n_keys - j0);
  float mx, ls, o;
  decode_slice<T, HS, 0>(q + (size_t)bh * HS, k + ((size_t)bh * kvT + j0) * HS,
                             vt + (size_t)bh * HS * kvT + j0, nj, kvT, t, sm[slice], mx, ls, o);
  if (t < HS) so[slice][t] = o;
  if (t == 0) {
    so[slice][HS] = mx;
    so[slice][HS + 1] = ls;
  }
  __syncthreads();
  const int d = threadIdx.x;
  if (d < HS) {
    float M = -INFINITY;
    for (int s = 0; s < nsl; ++s) M = fmaxf(M, so[s][HS]);
    float num = 0.f, den = 0.f;
    for (int s = 0; s < nsl; ++s) {
      const float w = __builtin_amdgcn_exp2f((so[s][HS] - M) * kLog2e);
      den += w * so[s][HS + 1];
      num += w * so[s][d];
    }
    const int b = bh / H, h = bh - b * H;
    out[(size_t)b * H * HS + h * HS + d] = Elem<T>::from_f32(num / den);
  }
}

// Merge the splits of one (b, h): out = sum_s e^{m_s - M} o_s / sum_s e^{m_s - M} l_s.
template <typename T, int HS>
__global__ __launch_bounds__(64) void attn_decode_merge_kernel(const float* __restrict__ part,
                                                                T* __restrict__ out, int H,
                                                                int nsplit) {
  const int bh = blockIdx.x, d = threadIdx.x;
  const float* pb = part + (size_t)bh * nsplit * (HS + 2);
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, pb[s * (HS + 2) + HS]);
  float num = 0.f, den = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float w = __builtin_amdgcn_exp2f((pb[s * (HS + 2) + HS] - M) * kLog2e);
    den += w * pb[s * (HS + 2) + HS + 1];
    if (d < HS) num += w * pb[s * (HS + 2) + d];
  }
  const int b = bh / H, h = bh - b * H;
  if (d < HS) out[(size_t)b * H * HS + h * HS + d] = Elem<T>::from_f32(num / den);
}

}  // namespace

constexpr int kPrefillQW = 16;  // queries per wave (see the kernel's notes)

// Dynamic LDS of attn_prefill_kernel<T, HS, ...>: two K tiles (kPrefillKeys
// keys x HS) and two V^T tiles (HS x kPrefillKeys keys).
template <typename T, int HS>
constexpr size_t prefill_lds_bytes() {
  return 2 * (kPrefillKeys<T> * HS + HS * kPrefillKeys<T>) * sizeof(T);
}

template <typename T>
hipError_t launch_attention_prefill(const T* q, const T* k, const T* vt, T* out, int B, int H, int Tq,
                                    int kvT, int hs, hipStream_t stream, float* lse) {
  constexpr int QW = kPrefillQW;
  const int n_qtiles = (Tq + 4 * QW - 1) / (4 * QW);
  dim3 grid(B * H * n_qtiles), block(256);
  if (hs == 64) {
    const size_t lds = prefill_lds_bytes<T, 64>();
    hipLaunchKernelGGL((attn_prefill_kernel<T, 64, QW>), grid, block, lds, stream, q, k, vt, out, B * H, H, Tq, kvT,
                       n_qtiles, lse);
  } else if (hs == 16 && sizeof(T) == 4) {
    constexpr int HS = sizeof(T) == 4 ? 16 : 64;
    const size_t lds = prefill_lds_bytes<T, HS>();
    hipLaunchKernelGGL((attn_prefill_kernel<T, HS, QW>), grid, block, lds, stream, q, k, vt, out, B * H, H, Tq, kvT,
                       n_qtiles, lse);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

size_t decode_partials_floats(int B, int H, int hs) {
  const int max_split = (4096 + kDecKeys - 1) / kDecKeys;
  return (size_t)B * H * max_split * (hs + 2);
}

template <typename T>
hipError_t launch_attention_decode(const T* q, const T* k, const T* vt, T* out, float* part, int B, int H,
                                   int n_keys, int kvT, int hs, hipStream_t stream) {
  const int nsplit = (n_keys + kDecKeys - 1) / kDecKeys;
  if (n_keys < 1 || nsplit * kDecKeys > 4096 || (hs != 64 && hs != 16)) return hipErrorInvalidValue;
  // Enough (b, h) pairs to fill the chip with one block each: the fused
  // kernel (no partials, no merge launch).  Otherwise, or past
  // kDecMaxSlices slices, one block per slice and a merge launch.
  // (fp32 with head_dim 64 holds too many K chunks for two 1024-thread blocks per CU.)
  const bool fused = nsplit <= kDecMaxSlices && B * H >= kDecFusedMinBH;
  if (hs == 64) {
    if constexpr (sizeof(T) == 2) {
      if (fused) {
        hipLaunchKernelGGL((attn_decode_fused_kernel<T, 64>), dim3(B * H), dim3(kDecKeys * nsplit), 0, stream, q,
                           k, vt, out, n_keys, kvT, H);
        return hipGetLastError();
      }
    }
    {
      hipLaunchKernelGGL((attn_decode_split_kernel<T, 64>), dim3(B * H * nsplit), dim3(256), 0, stream, q, k, vt,
                         part, n_keys, kvT, nsplit);
      hipLaunchKernelGGL((attn_decode_merge_kernel<T, 64>), dim3(B * H), dim3(64), 0, stream, part, out, H, nsplit);
    }
  } else {
    if (fused) {
      hipLaunchKernelGGL((attn_decode_fused_kernel<T, 16>), dim3(B * H), dim3(kDecKeys * nsplit), 0, stream, q, k,
                         vt, out, n_keys, kvT, H);
    } else {
      hipLaunchKernelGGL((attn_decode_split_kernel<T, 16>), dim3(B * H * nsplit), dim3(256), 0, stream, q, k, vt,
                         part, n_keys, kvT, nsplit);
      hipLaunchKernelGGL((attn_decode_merge_kernel<T, 16>), dim3(B * H), dim3(64), 0, stream, part, out, H, nsplit);
    }
  }
  return hipGetLastError();
}

template hipError_t launch_attention_prefill<float>(const float*, const float*, const float*, float*, int, int,
                                                    int, int, int, hipStream_t, float*);
template hipError_t launch_attention_prefill<bf16_t>(const bf16_t*, const bf16_t*, const bf16_t*, bf16_t*, int,
                                                     int, int, int, int, hipStream_t, float*);
template hipError_t launch_attention_decode<float>(const float*, const float*, const float*, float*, float*, int,
                                                   int, int, int, int, hipStream_t);
template hipError_t launch_attention_decode<bf16_t>(const bf16_t*, const bf16_t*, const bf16_t*, bf16_t*,
                                                    float*, int, int, int, int, int, hipStream_t);

}  // namespace gpt2
