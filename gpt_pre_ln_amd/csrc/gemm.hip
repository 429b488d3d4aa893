// Matrix-core GEMM kernel (see gemm.h for the design notes).
#include "gemm.h"

#include <type_traits>

namespace gpt2 {

namespace {

constexpr int kStepBytes = 128;  // k bytes per LDS stage and row (2 MFMA slabs)
constexpr int kChunks = kStepBytes / 16;
constexpr int kGroupM = 8;

// schedule knobs
constexpr int kPrio = 1;        // raise wave priority around each MFMA burst
constexpr int kAllFrags = 2;    // read both slabs' fragments before the first MFMA
constexpr int kSplitIssue = 4;  // issue the next stage's loads in two halves between slabs
constexpr int kInterleave = 8;  // issue the second slab's fragment reads among the first slab's MFMAs
constexpr int kAKM = 16;        // A stored K-major ([K][M], M contiguous): 16-bit elements only
constexpr int kBKM = 32;        // B stored K-major ([K][N], N contiguous): 16-bit elements only

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

// K-major operand tiles: LDS row kr (one k) holds the tile's BM (or BN)
// elements of that k as 16-byte chunks, chunk c at slot c ^ swzk(kr).  A
// transposing read takes 4 consecutive k rows x 32 bytes per 16-lane group;
// the swizzle puts those 4 row segments in distinct 32-byte bank ranges, and
// the groups of lanes 0-15 and 16-31 (k rows 8 apart) in different 128-byte
// halves.  Tiles of 128 columns: 91 us per weight-gradient product with no
// swizzle, 62.7 with the first term, 61.6 with both.
__device__ __forceinline__ int swzk(int kr) { return ((kr & 3) << 1) ^ (((kr >> 3) & 1) << 3); }

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// MFMA operand fragment from a K-major LDS tile (region of CP chunks per k
// row): lane (lr, lg) receives the 8 consecutive k = k0 + 8*lg .. +7 of
// tile column nb + lr.  ds_read_b64_tr_b16 in a 16-lane group: lane l names
// k row kb + l/4, columns nb + 4*(l%4) .. +3, and lane j receives
// X[kb + t][nb + j] for t = 0..3; two reads (kb = k0 + 8*lg and + 4) give
// the lane's 8 k values in order.
template <int CP>
__device__ __forceinline__ u32x4_t read_kmajor(const u32x4_t* region, int nb, int k0, int lr, int lg) {
  const int col = nb + 4 * (lr & 3);
  const int cl = col >> 3, half = (col >> 2) & 1;
  u32x2_t part[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int kr = k0 + 8 * lg + 4 * h + (lr >> 2);
    const char* addr = reinterpret_cast<const char*>(region + kr * CP + (cl ^ swzk(kr))) + half * 8;
    const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16_t*)(const_cast<char*>(addr)));
    part[h] = __builtin_bit_cast(u32x2_t, v);
  }
  return u32x4_t{part[0][0], part[0][1], part[1][0], part[1][1]};
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Staged reads the row-mode epilogue keeps in flight at once.
constexpr int kEpiBatch = 4;

// Map the linear block id to a (tile_m, tile_n) pair: XCD-contiguous ranges,
// then GROUP_M tile-rows per group with tile_m varying fastest.
__device__ __forceinline__ void tile_of_block(int ntm, int ntn, int& tm, int& tn) {
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int per_group = kGroupM * ntn;
  const int group = bid / per_group;
  const int first_m = group * kGroupM;
  const int gsz = min(ntm - first_m, kGroupM);
  const int r = bid - group * per_group;
  tm = first_m + r % gsz;
  tn = r / gsz;
}

// One block computes a BM x BN tile.  Operand tiles travel global -> LDS with
// global_load_lds_dwordx4 (no register staging): one wave instruction fills an
// 8-row x 128-byte block, lane i writing slot i; the lane loads the global
// chunk that belongs in that slot under the XOR swizzle.  S LDS stages form a
// ring; stage kt+S-1 is requested right after the barrier of step kt.
template <typename T, int BM, int BN, int WGM, int WGN, int S, int KNOB, class Epi>
__global__ __launch_bounds__(WGM* WGN * 64) void gemm_kernel(const T* __restrict__ A,
                                                              const T* __restrict__ B, int M, int N,
                                                              int K, int lda, int ldb, Epi epi) {
  constexpr int NW = WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int RB = (BM + BN) / 8;  // 8-row blocks per stage, one wave instruction each
  static_assert(RB % NW == 0, "row blocks must split evenly over waves");
  constexpr int RBW = RB / NW;  // load instructions per wave per stage
  static_assert(!(KNOB & kSplitIssue) || RBW % 2 == 0, "split issue needs an even count");
  constexpr int STAGE = (BM + BN) * kChunks;  // u32x4 per stage
  constexpr int KE = kStepBytes / (int)sizeof(T);
  static_assert(S >= 2 && S <= 4, "2..4 stages");
  constexpr bool AKM = (KNOB & kAKM) != 0, BKM = (KNOB & kBKM) != 0;
  constexpr int CA = BM / 8, CB = BN / 8;  // 16-byte chunks per k row of a K-major tile
  static_assert(!(AKM || BKM) || sizeof(T) == 2, "K-major operands take 16-bit elements");
  static_assert(!AKM || (CA >= 16 && (CA & (CA - 1)) == 0), "K-major A: BM a power of two >= 128");
  static_assert(!BKM || (CB >= 16 && (CB & (CB - 1)) == 0), "K-major B: BN a power of two >= 128");
  static_assert((BM / 8) % NW == 0, "A and B row blocks split at an instruction boundary");

  extern __shared__ u32x4_t smem[];

  // Split-K launches (gridDim.y > 1): slice blockIdx.y covers k in
  // [y*K, (y+1)*K) of both operands; the epilogue places its partial sum.
  A += (size_t)blockIdx.y * K * (AKM ? lda : 1);
  B += (size_t)blockIdx.y * K * (BKM ? ldb : 1);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  int tm, tn;
  tile_of_block((M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // Loader: wave instruction j covers 64-chunk block rb = j*NW + wave of the
  // stage (A's BM*8 chunks first, then B's; j < BM/(8*NW) is A for every
  // wave).  K-contiguous operand: block rb is rows rb*8 .. +7, lane -> row
  // rb*8 + lane/8, slot lane%8.  K-major operand: slot s = rb*64 + lane of
  // the region is k row s / CP, slot s % CP, holding the chunk that the
  // swizzle puts there (clamped to the last whole chunk in range; columns
  // past the edge are never stored).
  constexpr int JA = BM / (8 * NW);  // instructions per wave that load A
  const char* gsrc[RBW];
#pragma unroll
  for (int j = 0; j < RBW; ++j) {
    const int rb = j * NW + wave;
    const char* p;
    if (j < JA) {
      if constexpr (AKM) {
        const int sl = rb * 64 + lane, kr = sl / CA, cl = (sl % CA) ^ swzk(sl / CA);
        p = reinterpret_cast<const char*>(A + (size_t)kr * lda + min(m0 + cl * 8, M - 8));
      } else {
        const int row = rb * 8 + (lane >> 3);
        const int c = (lane & 7) ^ (lane >> 3);  // global chunk that lives in this lane's slot
        p = reinterpret_cast<const char*>(A + (size_t)min(m0 + row, M - 1) * lda) + c * 16;
      }
    } else {
      if constexpr (BKM) {
        const int sl = (rb - BM / 8) * 64 + lane, kr = sl / CB, cl = (sl % CB) ^ swzk(sl / CB);
        p = reinterpret_cast<const char*>(B + (size_t)kr * ldb + min(n0 + cl * 8, N - 8));
      } else {
        const int row = (rb - BM / 8) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ (lane >> 3);
        p = reinterpret_cast<const char*>(B + (size_t)min(n0 + row, N - 1) * ldb) + c * 16;
      }
    }
    gsrc[j] = p;
  }
  const int KT = K / KE;
  // bytes from one k step to the next: 64 k of a row, or 64 k rows
  const size_t stepA = AKM ? (size_t)KE * lda * sizeof(T) : (size_t)kStepBytes;
  const size_t stepB = BKM ? (size_t)KE * ldb * sizeof(T) : (size_t)kStepBytes;
  auto issue = [&](int kt, int j0, int j1) {
    u32x4_t* base = smem + (kt % S) * STAGE;
#pragma unroll
    for (int j = j0; j < j1; ++j) {
      u32x4_t* dst = base + (j * NW + wave) * 64;
      const size_t off = (size_t)kt * (j < JA ? stepA : stepB);
      __builtin_amdgcn_global_load_lds((const void*)(gsrc[j] + off), (__attribute__((address_space(3))) void*)dst,
                                       16, 0, 0);
    }
  };

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < KT) issue(s, 0, RBW);

  const int lr = lane & 15;  // fragment row within a 16-row tile
  const int lg = lane >> 4;  // lane group: 16-byte k-run within a 64-byte slab
  for (int kt = 0; kt < KT; ++kt) {
    // stage kt has landed once at most (later stages issued) * RBW loads are outstanding
    const int later = min(S - 2, KT - 1 - kt);
    if (S >= 4 && later >= 2) wait_vmcnt<2 * RBW>();
    else if (S >= 3 && later >= 1) wait_vmcnt<RBW>();
    else wait_vmcnt<0>();
    // Barrier without a memory fence: the wait above covers this wave's LDS
    // writes, and a fence would drain the loads still in flight.
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const bool more = kt + S - 1 < KT;
    // K-major tiles: every fragment of the step is read before the next
    // stage's loads go out.  The transposing LDS reads carry no alias
    // information, so the compiler waits for all LDS DMA in flight before
    // each of them; issued after them, the loads overlap this step's MFMAs.
    constexpr bool kReadsFirst = AKM || BKM;
    if (!(KNOB & kSplitIssue) && !kReadsFirst && more) issue(kt + S - 1, 0, RBW);

    const u32x4_t* s = smem + (kt % S) * STAGE;
    u32x4_t af[2][FM], bfr[2][FN];
    auto read_frags = [&](int slab) {
      const int c = slab * 4 + lg;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if constexpr (AKM) {
          af[slab][i] = read_kmajor<CA>(s, wm * WTM + i * 16, slab * 32, lr, lg);
        } else {
          const int r = wm * WTM + i * 16 + lr;
          af[slab][i] = s[r * kChunks + swz(r, c)];
        }
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if constexpr (BKM) {
          bfr[slab][j] = read_kmajor<CB>(s + BM * kChunks, wn * WTN + j * 16, slab * 32, lr, lg);
        } else {
          const int r = BM + wn * WTN + j * 16 + lr;
          bfr[slab][j] = s[r * kChunks + swz(r, c)];
        }
      }
    };
    auto mfma_slab = [&](int slab) {
      if (KNOB & kPrio) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) Mma<T>::run(acc[i][j], bfr[slab][j], af[slab][i]);
      if (KNOB & kPrio) __builtin_amdgcn_s_setprio(0);
    };
    read_frags(0);
    if constexpr (kReadsFirst) {
      read_frags(1);
      if (more) issue(kt + S - 1, 0, RBW);
      mfma_slab(0);
      mfma_slab(1);
      continue;
    }
    if (KNOB & kInterleave) {
      if ((KNOB & kSplitIssue) && more) issue(kt + S - 1, 0, RBW / 2);
      if (KNOB & kPrio) __builtin_amdgcn_s_setprio(1);
      read_frags(1);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) Mma<T>::run(acc[i][j], bfr[0][j], af[0][i]);
      // slab-0 MFMAs and slab-1 LDS reads alternate: FM*FN MFMAs over FM+FN reads
      constexpr int NR = FM + FN, MPR = (FM * FN) / NR > 0 ? (FM * FN) / NR : 1;
#pragma unroll
      for (int q = 0; q < NR; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, MPR, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, FM * FN, 0);
      if (KNOB & kPrio) __builtin_amdgcn_s_setprio(0);
    } else {
      if (KNOB & kAllFrags) read_frags(1);
      if ((KNOB & kSplitIssue) && more) issue(kt + S - 1, 0, RBW / 2);
      mfma_slab(0);
      if (!(KNOB & kAllFrags)) read_frags(1);
    }
    if ((KNOB & kSplitIssue) && more) issue(kt + S - 1, RBW / 2, RBW);
    mfma_slab(1);
  }

  // Epilogue.  Lane holds C[m][n .. n+3] of each fragment; the bias is added
  // in that layout first.
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    if constexpr (Epi::kBias) {
      const float4 b = epi.bias4(min(n0 + wn * WTN + j * 16 + lg * 4, N - 4));
#pragma unroll
      for (int i = 0; i < FM; ++i) acc[i][j] += f32x4_t{b.x, b.y, b.z, b.w};
    }
  }

  if constexpr (Epi::kRowReduce) {
    // Straight from the accumulators, no staging: for fragment row i a lane
    // holds row m = .. + i*16 + lr at columns nw + j*16 + lg*4 + e, and the
    // four lanes lr + 16*lg (lg = 0..3) together hold the wave's WTN columns
    // of that row.  Max, then sum of exp(C - max), over the columns below
    // n_valid: in registers, then across those four lanes (row-swap
    // permutes).  Slices entirely inside the vocabulary (all but the last)
    // take the body without per-column tests; the choice is uniform over the
    // wave.  max(a, b) is med3(a, b, +inf): one instruction.
    auto vmax = [](float a, float b) { return __builtin_amdgcn_fmed3f(a, b, INFINITY); };
    auto vadd = [](float a, float b) { return a + b; };
    const int nw = n0 + wn * WTN;
    auto reduce_rows = [&](auto full_tag) {
      constexpr bool kFull = decltype(full_tag)::value;
      auto ok = [&](int j, int e) { return kFull || nw + j * 16 + lg * 4 + e < epi.n_valid; };
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm * WTM + i * 16 + lr;
        const int label = m < M ? epi.label(m) : -1;
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (ok(j, e)) mx = vmax(mx, acc[i][j][e]);
        mx = combine_xor32(combine_xor16(mx, vmax), vmax);
        const float b = mx * kLog2e;
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (ok(j, e)) s += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[i][j][e], kLog2e, -b));
        s = combine_xor32(combine_xor16(s, vadd), vadd);
        if (m < M) {
          if (lg == 0) epi.partial(m, nw / WTN, mx, s);
          // the label's logit, from the one lane that holds it
          const int dl = label - nw;
          if (dl >= 0 && dl < WTN && ((dl >> 2) & 3) == lg && label < epi.n_valid) {
            float t = 0.f;
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if ((dl >> 4) == j && (dl & 3) == e) t = acc[i][j][e];
            epi.target(m, t);
          }
        }
      }
    };
    if (nw + WTN <= epi.n_valid) reduce_rows(std::true_type{});
    else reduce_rows(std::false_type{});
    return;
  }

  if constexpr (Epi::kRowArgmax) {
    // Same lane layout as the kRowReduce path: per fragment row, the lane's
    // columns in increasing order (strictly larger replaces, so the first
    // maximum stays), then across the four lanes holding the row.
    const int nw = n0 + wn * WTN;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int m = m0 + wm * WTM + i * 16 + lr;
      float best = -INFINITY;
      int bi = 0x7fffffff;
      const uint64_t rk = epi.row_key(m);
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int col = nw + j * 16 + lg * 4 + e;
          const float v = epi.score(rk, col, acc[i][j][e]);
          if (col < epi.n_valid && v > best) {
            best = v;
            bi = col;
          }
        }
      argmax_xor<16>(best, bi);
      argmax_xor<32>(best, bi);
      if (m < M && lg == 0) epi.partial(m, nw / WTN, best, bi);
    }
    return;
  }

  // Each wave then stages its WTM x WTN sub-tile through a private slice
  // of the (now idle) operand LDS, R rows at a time, and reads it back so
  // that 16-byte groups of consecutive lanes cover consecutive columns of one
  // row (row mode) or consecutive rows of one column (transposed mode, for
  // outputs stored transposed): each store instruction then writes whole
  // row segments instead of 16 rows x 16 columns.
  constexpr int LDS_F = S * (BM + BN) * kStepBytes / 4;  // floats of LDS
  constexpr int PER_WAVE = LDS_F / NW;
  constexpr int CPR = WTN / 4;  // 16-byte chunks per staged row (row mode)
  // Rows of a power-of-two number of chunks are XOR-swizzled; other widths
  // (48-column waves of the 128x96 tile) are padded by one chunk instead,
  // which puts 8 consecutive rows in distinct bank groups as well.
  constexpr bool kPow2Row = (CPR & (CPR - 1)) == 0;
  constexpr int RS = kPow2Row ? WTN : WTN + 4;  // staged row stride, floats
  constexpr int R = [] {  // rows staged per round: whole fragments that divide WTM
    int r = WTM < PER_WAVE / RS ? WTM : PER_WAVE / RS;
    r -= r % 16;
    while (r > 16 && WTM % r) r -= 16;
    return r;
  }();
  static_assert(R % 16 == 0 && WTM % R == 0, "staging rounds must hold whole fragments");
  constexpr int CPT = R / 4;    // 16-byte chunks per staged column (transposed mode)
  static_assert(CPR <= 16 && CPT <= 16 && (64 % CPR == 0 || !kPow2Row) && 64 % CPT == 0, "lane mapping");
  auto slot = [](int r, int c) { return kPow2Row ? (c ^ (r & (CPR - 1))) : c; };

  // every wave is past its last operand read (its MFMAs consumed them) and
  // the last stage's loads have landed (vmcnt(0) in the last step)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  float* stg = reinterpret_cast<float*>(smem) + wave * PER_WAVE;
  const int mw = m0 + wm * WTM, nw = n0 + wn * WTN;
  const bool tr = Epi::kTransposed && epi.transposed(nw);

  constexpr int CH = WTN / 8;  // 16-byte chunks per row of a bf16-staged sub-tile
  constexpr bool kStageB16 = requires { epi.store8_packed(0, 0, u32x4_t{}); } && WTN % 8 == 0 &&
                             (CH & (CH - 1)) == 0 && CH <= 64 && WTM % (64 / CH) == 0 &&
                             WTM * WTN * 2 <= PER_WAVE * 4;
  if constexpr (kStageB16) {
    // bf16 output staged as bf16: the whole WTM x WTN sub-tile in one round
    // (rows of WTN/8 16-byte chunks, XOR-swizzled by row), half the LDS bytes
    // of fp32 staging; each lane then stores 8 consecutive columns
    char* sb = reinterpret_cast<char*>(stg);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = i * 16 + lr, ch = 2 * j + (lg >> 1);
        *reinterpret_cast<u32x2_t*>(sb + r * (WTN * 2) + ((ch ^ (r & (CH - 1))) << 4) + (lg & 1) * 8) =
            u32x2_t{pack2_bf16(acc[i][j][0], acc[i][j][1]), pack2_bf16(acc[i][j][2], acc[i][j][3])};
      }
    constexpr int RPW = 64 / CH, NQ8 = WTM / RPW, G = NQ8 < kEpiBatch ? NQ8 : kEpiBatch;
    static_assert(NQ8 % G == 0, "whole batches");
    const int cc = lane % CH;
    const int n = nw + cc * 8;
#pragma unroll
    for (int q0 = 0; q0 < NQ8; q0 += G) {
      u32x4_t v[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int r = (q0 + g) * RPW + lane / CH;
        v[g] = *reinterpret_cast<const u32x4_t*>(sb + r * (WTN * 2) + ((cc ^ (r & (CH - 1))) << 4));
      }
      asm volatile("" ::: "memory");  // the batch's reads stay together
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int m = mw + (q0 + g) * RPW + lane / CH;
        if (m < M && n < N) epi.store8_packed(m, n, v[g]);
      }
    }
    return;
  }

#pragma unroll
  for (int rd = 0; rd < WTM / R; ++rd) {
    const int mr = mw + rd * R;  // first row of this round
    if (!tr) {
      // row-major [R][RS] with chunk c of row r at slot(r, c)
#pragma unroll
      for (int i = 0; i < R / 16; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int r = i * 16 + lr, c = j * 4 + lg;
          *reinterpret_cast<f32x4_t*>(stg + r * RS + (slot(r, c) << 2)) = acc[rd * (R / 16) + i][j];
        }
      if constexpr (kPow2Row && requires { epi.apply8(0, 0, f32x4_t{}, f32x4_t{}); }) {
        // 8 columns per lane (two adjacent staged chunks): one 16-byte store
        // per lane, 8 lanes per 64-column row segment (bf16 logits; 736 ->
        // 725 us for the GPT-2 small lm_head standalone)
        constexpr int LPR = CPR / 2, RPW = 64 / LPR;
        static_assert(R % RPW == 0, "whole rows per store instruction");
        const int c2 = (lane % LPR) * 2;
        const int n = nw + c2 * 4;
        if (mr + R <= M && nw + WTN <= N) {
          // whole round inside C (uniform): staged reads in batches, as below
          constexpr int NQ8 = R / RPW, G = NQ8 < kEpiBatch ? NQ8 : kEpiBatch;
          static_assert(NQ8 % G == 0, "whole batches");
#pragma unroll
          for (int q0 = 0; q0 < NQ8; q0 += G) {
            f32x4_t v0[G], v1[G];
#pragma unroll
            for (int g = 0; g < G; ++g) {
              const int r = (q0 + g) * RPW + lane / LPR;
              v0[g] = *reinterpret_cast<const f32x4_t*>(stg + r * RS + (slot(r, c2) << 2));
              v1[g] = *reinterpret_cast<const f32x4_t*>(stg + r * RS + (slot(r, c2 + 1) << 2));
            }
#pragma unroll
            for (int g = 0; g < G; ++g) epi.apply8(mr + (q0 + g) * RPW + lane / LPR, n, v0[g], v1[g]);
          }
          continue;
        }
#pragma unroll
        for (int q = 0; q < R / RPW; ++q) {
          const int r = q * RPW + lane / LPR;
          const f32x4_t v0 = *reinterpret_cast<const f32x4_t*>(stg + r * RS + (slot(r, c2) << 2));
          const f32x4_t v1 = *reinterpret_cast<const f32x4_t*>(stg + r * RS + (slot(r, c2 + 1) << 2));
          const int m = mr + r;
          if (m < M && n < N) epi.apply8(m, n, v0, v1);
        }
        continue;
      }
      constexpr int RPI = 64 / CPR;            // rows per read instruction
      constexpr int NQ = (R + RPI - 1) / RPI;  // read instructions per round
      const int c = lane % CPR;
      const int n = nw + c * 4;
      const bool lane_on = lane < RPI * CPR;   // every lane when CPR divides 64
      // per-lane column constants of the epilogue, formed once per round
      const auto cctx = [&] {
        if constexpr (requires { epi.col_ctx(0); }) return epi.col_ctx(min(n, N - 4));
        else return 0;
      }();
      float4 pre[NQ];
      if constexpr (Epi::kPreload) {
#pragma unroll
        for (int q = 0; q < NQ; ++q)
          pre[q] = epi.preload(min(mr + min(q * RPI + lane / CPR, R - 1), M - 1), min(n, N - 4));
        asm volatile("" ::: "memory");  // every preload issued before the first store
      }
      if constexpr (RPI * CPR == 64 && NQ * RPI == R) {
        // the wave's rows and columns of this round all inside C (uniform):
        // no per-lane conditions, so the staged reads go out in batches of
        // kEpiBatch and their latency is paid once per batch
        if (mr + R <= M && nw + WTN <= N) {
          constexpr int G = NQ < kEpiBatch ? NQ : kEpiBatch;
          static_assert(NQ % G == 0, "whole batches");
#pragma unroll
          for (int q0 = 0; q0 < NQ; q0 += G) {
            f32x4_t v[G];
#pragma unroll
            for (int g = 0; g < G; ++g) {
              const int r = (q0 + g) * RPI + lane / CPR;
              v[g] = *reinterpret_cast<const f32x4_t*>(stg + r * RS + (slot(r, c) << 2));
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
              if constexpr (requires { epi.col_ctx(0); })
                epi.apply_c(mr + (q0 + g) * RPI + lane / CPR, cctx, v[g]);
              else
                epi.apply(mr + (q0 + g) * RPI + lane / CPR, n, v[g], pre[q0 + g]);
            }
          }
          continue;
        }
      }
      // Otherwise the same batches with the per-lane tests on the stores
      // only (rows past the round clamped to its last row).
      constexpr int G = NQ < kEpiBatch ? NQ : kEpiBatch;
#pragma unroll
      for (int q0 = 0; q0 < NQ; q0 += G) {
        f32x4_t v[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          if (q0 + g >= NQ) break;
          const int r = min((q0 + g) * RPI + lane / CPR, R - 1);
          v[g] = *reinterpret_cast<const f32x4_t*>(stg + r * RS + (slot(r, c) << 2));
        }
        asm volatile("" ::: "memory");  // keeps the batch's reads from sinking into the stores' branches
#pragma unroll
        for (int g = 0; g < G; ++g) {
          if (q0 + g >= NQ) break;
          const int r = (q0 + g) * RPI + lane / CPR;
          const int m = mr + r;
          if (lane_on && r < R && m < M && n < N) {
            if constexpr (requires { epi.col_ctx(0); })
              epi.apply_c(m, cctx, v[g]);
            else
              epi.apply(m, n, v[g], pre[q0 + g]);
          }
        }
      }
    } else {
      // column-major [WTN][R] with chunk c of column n at slot c ^ (n % CPT)
#pragma unroll
      for (int i = 0; i < R / 16; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = i * 16 + lr, col = j * 16 + lg * 4 + e;
            stg[col * R + (((r >> 2) ^ (col & (CPT - 1))) << 2) + (r & 3)] = acc[rd * (R / 16) + i][j][e];
          }
      constexpr int CPI = 64 / CPT;  // columns per read instruction
      constexpr int NQT = WTN / CPI;
      constexpr int GT = NQT <= kEpiBatch ? NQT : NQT % kEpiBatch == 0 ? kEpiBatch : NQT % 3 == 0 ? 3 : NQT % 2 == 0 ? 2 : 1;
      static_assert(NQT % GT == 0, "whole batches");
      const int c = lane % CPT;
      const auto rctx = [&] {  // per-lane row constants, once per round
        if constexpr (requires { epi.row_ctx(0); }) return epi.row_ctx(min(mr + c * 4, M - 1));
        else return 0;
      }();
#pragma unroll
      for (int q0 = 0; q0 < NQT; q0 += GT) {
        f32x4_t v[GT];
#pragma unroll
        for (int g = 0; g < GT; ++g) {
          const int col = (q0 + g) * CPI + lane / CPT;
          v[g] = *reinterpret_cast<const f32x4_t*>(stg + col * R + ((c ^ (col & (CPT - 1))) << 2));
        }
        asm volatile("" ::: "memory");  // as in row mode: the batch's reads stay together
#pragma unroll
        for (int g = 0; g < GT; ++g) {
          const int m = mr + c * 4, n = nw + (q0 + g) * CPI + lane / CPT;
          if (m < M && n < N) {
            if constexpr (requires { epi.row_ctx(0); })
              epi.apply_tc(m, rctx, n, v[g]);
            else
              epi.apply_t(m, n, v[g]);
          }
        }
      }
    }
  }
}

template <typename T, int BM, int BN, int WGM, int WGN, int S, int KNOB, class Epi>
hipError_t launch_tile(const T* A, const T* B, int M, int N, int K, int lda, int ldb, const Epi& epi,
                       hipStream_t stream, int splits = 1) {
  constexpr int NT = WGM * WGN * 64;
  const size_t lds = (size_t)S * (BM + BN) * kStepBytes;
  auto kern = gemm_kernel<T, BM, BN, WGM, WGN, S, KNOB, Epi>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int ntm = (M + BM - 1) / BM, ntn = (N + BN - 1) / BN;
  hipLaunchKernelGGL(kern, dim3(ntm * ntn, splits), dim3(NT), lds, stream, A, B, M, N, K, lda, ldb, epi);
  return hipGetLastError();
}

// ------------------------------------------------------------------ skinny
// GEMMs with at most 32 rows (the decode step: one row per sequence) are
// bound by streaming B once and by the fixed cost of each launch.  One kernel
// does the whole product and its epilogue: a block owns 16 columns; its NWS
// waves take the 32-element (bf16) or 16-element (fp32) k steps round-robin,
// reading their 16 B rows and both 16-row A fragments straight from global
// memory (nothing is shared, so nothing is staged), then the block adds the
// wave results in LDS and wave 0 applies the fused epilogue.  N/16 blocks of
// up to 16 waves keep the whole weight matrix in flight.
// Shared body: waves of the block take the k steps of [k0, k1) round-robin;
// the block sum lands in wave 0 (lane holds C[m][n0 + 4*lg .. +3] for
// m = lr in acc0 and m = 16 + lr in acc1); returns false in the other waves.
template <typename T, int NWS>
__device__ __forceinline__ bool skinny_block_product(const T* __restrict__ A, const T* __restrict__ B, int M, int N,
                                                     int lda, int ldb, int n0, int k0, int k1, f32x4_t (*red)[2][64],
                                                     f32x4_t& acc0, f32x4_t& acc1) {
  constexpr int SLAB = Mma<T>::kPerSlab;  // k elements per 16-byte-per-lane fragment step
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const T* brow = B + (size_t)min(n0 + lr, N - 1) * ldb;
  const T* arow0 = A + (size_t)min(lr, M - 1) * lda;
  const T* arow1 = A + (size_t)min(16 + lr, M - 1) * lda;
  const int lofs = lg * (16 / (int)sizeof(T));
  acc0 = f32x4_t{0.f, 0.f, 0.f, 0.f};
  acc1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int k = k0 + wave * SLAB; k < k1; k += NWS * SLAB) {
    const u32x4_t b = *reinterpret_cast<const u32x4_t*>(brow + k + lofs);
    const u32x4_t a0 = *reinterpret_cast<const u32x4_t*>(arow0 + k + lofs);
    const u32x4_t a1 = *reinterpret_cast<const u32x4_t*>(arow1 + k + lofs);
    Mma<T>::run(acc0, b, a0);
    Mma<T>::run(acc1, b, a1);
  }
  red[wave][0][lane] = acc0;
  red[wave][1][lane] = acc1;
  __syncthreads();
  if (wave != 0) return false;
  acc0 = red[0][0][lane];
  acc1 = red[0][1][lane];
#pragma unroll
  for (int w = 1; w < NWS; ++w) {
    acc0 += red[w][0][lane];
    acc1 += red[w][1][lane];
  }
  return true;
}

template <typename T, int NWS, class Epi>
__global__ __launch_bounds__(NWS * 64) void gemm_skinny_kernel(const T* __restrict__ A, const T* __restrict__ B, int M,
                                                                int N, int K, int lda, int ldb, Epi epi) {
  __shared__ f32x4_t red[NWS][2][64];
  const int n0 = blockIdx.x * 16;
  f32x4_t acc0, acc1;
  if (!skinny_block_product<T, NWS>(A, B, M, N, lda, ldb, n0, 0, K, red, acc0, acc1)) return;
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int n = n0 + lg * 4;
  if (n >= N) return;
  if constexpr (Epi::kBias) {
    const float4 b = epi.bias4(n);
    acc0 += f32x4_t{b.x, b.y, b.z, b.w};
    acc1 += f32x4_t{b.x, b.y, b.z, b.w};
  }
  if (lr < M) epi.apply(lr, n, acc0, Epi::kPreload ? epi.preload(lr, n) : float4{});
  if (16 + lr < M) epi.apply(16 + lr, n, acc1, Epi::kPreload ? epi.preload(16 + lr, n) : float4{});
}

// Split-K variant without an epilogue: block (column group, split s) writes
// the partial product of k in [s*kchunk, (s+1)*kchunk) to part[s][m][n].
template <typename T, int NWS>
__global__ __launch_bounds__(NWS * 64) void gemm_skinny_split_kernel(const T* __restrict__ A, const T* __restrict__ B,
                                                                      float* __restrict__ part, int M, int N, int K,
                                                                      int lda, int ldb, int kchunk) {
  __shared__ f32x4_t red[NWS][2][64];
  const int n0 = blockIdx.x * 16, s = blockIdx.y;
  const int k0 = s * kchunk, k1 = min(K, k0 + kchunk);
  f32x4_t acc0, acc1;
  if (!skinny_block_product<T, NWS>(A, B, M, N, lda, ldb, n0, k0, k1, red, acc0, acc1)) return;
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int n = n0 + lg * 4;
  if (n >= N) return;
  if (lr < M) *reinterpret_cast<f32x4_t*>(part + ((size_t)s * M + lr) * N + n) = acc0;
  if (16 + lr < M) *reinterpret_cast<f32x4_t*>(part + ((size_t)s * M + 16 + lr) * N + n) = acc1;
}

}  // namespace

int gemm_slice_width(GemmTile tile) {
  switch (tile) {
    case kTile256x256: return 256 / 4;
    case kTile64x64: return 64 / 2;
    case kTile32x64: return 64 / 2;
    case kTile64x128: return 128 / 2;
    case kTile128x96: return 96 / 2;
    case kTile128x192: return 192 / 4;
    case kTile128x128:
    default: return 128 / 2;
  }
}

template <typename T, class Epi>
hipError_t launch_gemm(GemmTile tile, const T* A, const T* B, int M, int N, int K, int lda, int ldb,
                       const Epi& epi, hipStream_t stream) {
  switch (tile) {
    case kTile256x256:
      return launch_tile<T, 256, 256, 2, 4, 2, kSplitIssue | kInterleave>(A, B, M, N, K, lda, ldb, epi, stream);
    case kTile64x64:
      return launch_tile<T, 64, 64, 2, 2, 2, 0>(A, B, M, N, K, lda, ldb, epi, stream);
    case kTile32x64:
      return launch_tile<T, 32, 64, 2, 2, 2, 0>(A, B, M, N, K, lda, ldb, epi, stream);
    case kTile64x128:
      return launch_tile<T, 64, 128, 2, 2, 2, kPrio | kInterleave>(A, B, M, N, K, lda, ldb, epi, stream);
    case kTile128x96:
      return launch_tile<T, 128, 96, 2, 2, 2, kPrio | kInterleave>(A, B, M, N, K, lda, ldb, epi, stream);
    case kTile128x192:
      return launch_tile<T, 128, 192, 2, 4, 2, kPrio | kInterleave>(A, B, M, N, K, lda, ldb, epi, stream);
    case kTile128x128:
    default:
      return launch_tile<T, 128, 128, 2, 2, 2, kPrio | kInterleave>(A, B, M, N, K, lda, ldb, epi, stream);
  }
}

template <typename T, class Epi>
hipError_t launch_gemm_skinny(const T* A, const T* B, int M, int N, int K, int lda, int ldb, const Epi& epi,
                              hipStream_t stream) {
  if (M > 32 || M < 1) return hipErrorInvalidValue;
  const dim3 grid((N + 15) / 16);
  if (K >= 2048)
    hipLaunchKernelGGL((gemm_skinny_kernel<T, 16, Epi>), grid, dim3(1024), 0, stream, A, B, M, N, K, lda, ldb, epi);
  else
    hipLaunchKernelGGL((gemm_skinny_kernel<T, 8, Epi>), grid, dim3(512), 0, stream, A, B, M, N, K, lda, ldb, epi);
  return hipGetLastError();
}

int skinny_splits(int K, int elem_bytes) {
  const int step = 8 * (elem_bytes == 2 ? Mma<bf16_t>::kPerSlab : Mma<float>::kPerSlab);
  return (K + step - 1) / step;
}

template <typename T>
hipError_t launch_gemm_skinny_splitk(const T* A, const T* B, int M, int N, int K, int lda, int ldb, float* part,
                                     hipStream_t stream) {
  if (M > 32 || M < 1) return hipErrorInvalidValue;
  const int kchunk = 8 * Mma<T>::kPerSlab;  // one k step per wave of an 8-wave block
  const dim3 grid((N + 15) / 16, skinny_splits(K, sizeof(T)));
  hipLaunchKernelGGL((gemm_skinny_split_kernel<T, 8>), grid, dim3(512), 0, stream, A, B, part, M, N, K, lda, ldb,
                     kchunk);
  return hipGetLastError();
}
template hipError_t launch_gemm_skinny_splitk<float>(const float*, const float*, int, int, int, int, int, float*,
                                                     hipStream_t);
template hipError_t launch_gemm_skinny_splitk<bf16_t>(const bf16_t*, const bf16_t*, int, int, int, int, int, float*,
                                                      hipStream_t);

#define GPT2_INSTANTIATE_GEMM(T, ...)                                                                   \
  template hipError_t launch_gemm<T, __VA_ARGS__>(GemmTile, const T*, const T*, int, int, int, int, int, \
                                                  const __VA_ARGS__&, hipStream_t);                      \
  template hipError_t launch_gemm_skinny<T, __VA_ARGS__>(const T*, const T*, int, int, int, int, int,    \
                                                         const __VA_ARGS__&, hipStream_t);

GPT2_INSTANTIATE_GEMM(float, EpiQKV<float>)
GPT2_INSTANTIATE_GEMM(float, EpiResidual)
GPT2_INSTANTIATE_GEMM(float, EpiGelu<float, false>)
GPT2_INSTANTIATE_GEMM(float, EpiGelu<float, true>)
GPT2_INSTANTIATE_GEMM(float, EpiLogits<float>)
GPT2_INSTANTIATE_GEMM(float, EpiLogits<bf16_t>)
GPT2_INSTANTIATE_GEMM(bf16_t, EpiQKV<bf16_t>)
GPT2_INSTANTIATE_GEMM(bf16_t, EpiResidual)
GPT2_INSTANTIATE_GEMM(bf16_t, EpiGelu<bf16_t, false>)
GPT2_INSTANTIATE_GEMM(bf16_t, EpiGelu<bf16_t, true>)
GPT2_INSTANTIATE_GEMM(bf16_t, EpiLogits<float>)
GPT2_INSTANTIATE_GEMM(bf16_t, EpiLogits<bf16_t>)
template <typename T>
hipError_t launch_gemm_splitk(GemmTile tile, const T* A, const T* B, int M, int N, int K_split, int lda, int ldb,
                              int splits, const EpiStore<float>& epi, hipStream_t stream) {
  if (splits < 1 || splits > 65535) return hipErrorInvalidValue;
  switch (tile) {
    case kTile256x256:
      return launch_tile<T, 256, 256, 2, 4, 2, kSplitIssue | kInterleave>(A, B, M, N, K_split, lda, ldb, epi, stream,
                                                                           splits);
    case kTile64x64:
      return launch_tile<T, 64, 64, 2, 2, 2, 0>(A, B, M, N, K_split, lda, ldb, epi, stream, splits);
    case kTile32x64:
      return launch_tile<T, 32, 64, 2, 2, 2, 0>(A, B, M, N, K_split, lda, ldb, epi, stream, splits);
    case kTile64x128:
      return launch_tile<T, 64, 128, 2, 2, 2, kPrio | kInterleave>(A, B, M, N, K_split, lda, ldb, epi, stream, splits);
    case kTile128x96:
      return launch_tile<T, 128, 96, 2, 2, 2, kPrio | kInterleave>(A, B, M, N, K_split, lda, ldb, epi, stream, splits);
    case kTile128x192:
      return launch_tile<T, 128, 192, 2, 4, 2, kPrio | kInterleave>(A, B, M, N, K_split, lda, ldb, epi, stream,
                                                                    splits);
    case kTile128x128:
    default:
      return launch_tile<T, 128, 128, 2, 2, 2, kPrio | kInterleave>(A, B, M, N, K_split, lda, ldb, epi, stream,
                                                                    splits);
  }
}
hipError_t launch_gemm_kmajor(const bf16_t* A, const bf16_t* B, int M, int N, int K_split, int lda, int ldb,
                              int splits, const EpiStore<float>& epi, hipStream_t stream) {
  if (splits < 1 || splits > 65535 || M < 8 || N < 8 || M % 8 || N % 8 || K_split % 64 || lda % 8 || ldb % 8)
    return hipErrorInvalidValue;
  return launch_tile<bf16_t, 128, 128, 2, 2, 2, kPrio | kInterleave | kAKM | kBKM>(A, B, M, N, K_split, lda, ldb, epi,
                                                                                    stream, splits);
}
template hipError_t launch_gemm_splitk<float>(GemmTile, const float*, const float*, int, int, int, int, int, int,
                                              const EpiStore<float>&, hipStream_t);
template hipError_t launch_gemm_splitk<bf16_t>(GemmTile, const bf16_t*, const bf16_t*, int, int, int, int, int, int,
                                               const EpiStore<float>&, hipStream_t);
template hipError_t launch_gemm<float, EpiStore<float>>(GemmTile, const float*, const float*, int, int, int, int,
                                                        int, const EpiStore<float>&, hipStream_t);
template hipError_t launch_gemm<bf16_t, EpiStore<float>>(GemmTile, const bf16_t*, const bf16_t*, int, int, int, int,
                                                         int, const EpiStore<float>&, hipStream_t);
template hipError_t launch_gemm<bf16_t, EpiStore<bf16_t>>(GemmTile, const bf16_t*, const bf16_t*, int, int, int,
                                                          int, int, const EpiStore<bf16_t>&, hipStream_t);
#define GPT2_INSTANTIATE_GEMM_TILED(T, ...)                                                          \
  template hipError_t launch_gemm<T, __VA_ARGS__>(GemmTile, const T*, const T*, int, int, int, int, int, \
                                                  const __VA_ARGS__&, hipStream_t);
GPT2_INSTANTIATE_GEMM_TILED(float, EpiGeluSave<float, false>)
GPT2_INSTANTIATE_GEMM_TILED(float, EpiGeluSave<float, true>)
GPT2_INSTANTIATE_GEMM_TILED(bf16_t, EpiGeluSave<bf16_t, false>)
GPT2_INSTANTIATE_GEMM_TILED(bf16_t, EpiGeluSave<bf16_t, true>)
GPT2_INSTANTIATE_GEMM_TILED(float, EpiGeluBwd<float, false>)
GPT2_INSTANTIATE_GEMM_TILED(float, EpiGeluBwd<float, true>)
GPT2_INSTANTIATE_GEMM_TILED(bf16_t, EpiGeluBwd<bf16_t, false>)
GPT2_INSTANTIATE_GEMM_TILED(bf16_t, EpiGeluBwd<bf16_t, true>)
template hipError_t launch_gemm<float, EpiArgmax>(GemmTile, const float*, const float*, int, int, int, int, int,
                                                  const EpiArgmax&, hipStream_t);
template hipError_t launch_gemm<bf16_t, EpiArgmax>(GemmTile, const bf16_t*, const bf16_t*, int, int, int, int, int,
                                                   const EpiArgmax&, hipStream_t);
template hipError_t launch_gemm<float, EpiSample>(GemmTile, const float*, const float*, int, int, int, int, int,
                                                  const EpiSample&, hipStream_t);
template hipError_t launch_gemm<bf16_t, EpiSample>(GemmTile, const bf16_t*, const bf16_t*, int, int, int, int, int,
                                                   const EpiSample&, hipStream_t);
template hipError_t launch_gemm<float, EpiCE>(GemmTile, const float*, const float*, int, int, int, int, int,
                                              const EpiCE&, hipStream_t);
template hipError_t launch_gemm<bf16_t, EpiCE>(GemmTile, const bf16_t*, const bf16_t*, int, int, int, int, int,
                                               const EpiCE&, hipStream_t);

}  // namespace gpt2
