// Matrix-core GEMM kernel (see gemm.h for the design notes).
#include "gemm.h"

namespace gpt2 {

namespace {

constexpr int kStepBytes = 128;  // k bytes per LDS stage and row (2 MFMA slabs)
constexpr int kChunks = kStepBytes / 16;
constexpr int kGroupM = 8;

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

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

template <typename T, int BM, int BN, int WGM, int WGN, class Epi>
__global__ __launch_bounds__(WGM* WGN * 64) void gemm_kernel(const T* __restrict__ A,
                                                              const T* __restrict__ B, int M, int N,
                                                              int K, int lda, int ldb, Epi epi) {
  constexpr int NT = WGM * WGN * 64;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int CA = BM * kChunks, CB = BN * kChunks;
  static_assert(CA % NT == 0 && CB % NT == 0, "tile chunks must split evenly over threads");
  constexpr int LA = CA / NT, LB = CB / NT;
  constexpr int KE = kStepBytes / (int)sizeof(T);  // k elements per stage

  extern __shared__ u32x4_t smem[];  // [2][(BM + BN) * kChunks]
  constexpr int STAGE = (BM + BN) * kChunks;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  int tm, tn;
  tile_of_block((M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // Per-thread global source pointers and LDS slots (fixed over k).
  const char* ga[LA];
  const char* gb[LB];
  int sa[LA], sb[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    int idx = tid + i * NT;
    int row = idx / kChunks, c = idx % kChunks;
    int gm = min(m0 + row, M - 1);
    ga[i] = reinterpret_cast<const char*>(A + (size_t)gm * lda) + c * 16;
    sa[i] = row * kChunks + swz(row, c);
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    int idx = tid + i * NT;
    int row = idx / kChunks, c = idx % kChunks;
    int gn = min(n0 + row, N - 1);
    gb[i] = reinterpret_cast<const char*>(B + (size_t)gn * ldb) + c * 16;
    sb[i] = BM * kChunks + row * kChunks + swz(row, c);
  }

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  u32x4_t ra[LA], rb[LB];
  auto gload = [&](int kt) {
    const size_t off = (size_t)kt * kStepBytes;
#pragma unroll
    for (int i = 0; i < LA; ++i) ra[i] = *reinterpret_cast<const u32x4_t*>(ga[i] + off);
#pragma unroll
    for (int i = 0; i < LB; ++i) rb[i] = *reinterpret_cast<const u32x4_t*>(gb[i] + off);
  };
  auto sstore = [&](int buf) {
    u32x4_t* s = smem + buf * STAGE;
#pragma unroll
    for (int i = 0; i < LA; ++i) s[sa[i]] = ra[i];
#pragma unroll
    for (int i = 0; i < LB; ++i) s[sb[i]] = rb[i];
  };

  const int KT = K / KE;
  gload(0);
  sstore(0);
  __syncthreads();

  const int lr = lane & 15;   // fragment row within a 16-row tile
  const int lg = lane >> 4;   // lane group: 16-byte k-run within a 64-byte slab

  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT) gload(kt + 1);
    const u32x4_t* s = smem + (kt & 1) * STAGE;
#pragma unroll
    for (int slab = 0; slab < 2; ++slab) {
      const int c = slab * 4 + lg;
      u32x4_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        int r = wm * WTM + i * 16 + lr;
        af[i] = s[r * kChunks + swz(r, c)];
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        int r = wn * WTN + j * 16 + lr;
        bfr[j] = s[BM * kChunks + r * kChunks + swz(r, c)];
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) Mma<T>::run(acc[i][j], bfr[j], af[i]);
    }
    if (kt + 1 < KT) sstore((kt + 1) & 1);
    __syncthreads();
  }

  // Epilogue: lane holds C[m][n .. n+3].
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m0 + wm * WTM + i * 16 + lr;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + wn * WTN + j * 16 + lg * 4;
      if (n < N) epi.apply(m, n, acc[i][j]);
    }
  }
}

template <typename T, int BM, int BN, int WGM, int WGN, class Epi>
hipError_t launch_tile(const T* A, const T* B, int M, int N, int K, int lda, int ldb, const Epi& epi,
                       hipStream_t stream) {
  constexpr int NT = WGM * WGN * 64;
  const size_t lds = 2 * (size_t)(BM + BN) * kStepBytes;
  auto kern = gemm_kernel<T, BM, BN, WGM, WGN, Epi>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int ntm = (M + BM - 1) / BM, ntn = (N + BN - 1) / BN;
  hipLaunchKernelGGL(kern, dim3(ntm * ntn), dim3(NT), lds, stream, A, B, M, N, K, lda, ldb, epi);
  return hipGetLastError();
}

}  // namespace

template <typename T, class Epi>
hipError_t launch_gemm(GemmTile tile, const T* A, const T* B, int M, int N, int K, int lda, int ldb,
                       const Epi& epi, hipStream_t stream) {
  switch (tile) {
    case kTile256x128:
      return launch_tile<T, 256, 128, 2, 2>(A, B, M, N, K, lda, ldb, epi, stream);
    case kTile64x64:
      return launch_tile<T, 64, 64, 2, 2>(A, B, M, N, K, lda, ldb, epi, stream);
    case kTile32x64:
      return launch_tile<T, 32, 64, 2, 2>(A, B, M, N, K, lda, ldb, epi, stream);
    case kTile128x128:
    default:
      return launch_tile<T, 128, 128, 2, 2>(A, B, M, N, K, lda, ldb, epi, stream);
  }
}

#define GPT2_INSTANTIATE_GEMM(T, EPI)                                                               \
  template hipError_t launch_gemm<T, EPI>(GemmTile, const T*, const T*, int, int, int, int, int, \
                                          const EPI&, hipStream_t);

GPT2_INSTANTIATE_GEMM(float, EpiQKV<float>)
GPT2_INSTANTIATE_GEMM(float, EpiResidual)
GPT2_INSTANTIATE_GEMM(float, EpiGelu<float>)
GPT2_INSTANTIATE_GEMM(float, EpiLogits)
GPT2_INSTANTIATE_GEMM(bf16_t, EpiQKV<bf16_t>)
GPT2_INSTANTIATE_GEMM(bf16_t, EpiResidual)
GPT2_INSTANTIATE_GEMM(bf16_t, EpiGelu<bf16_t>)
GPT2_INSTANTIATE_GEMM(bf16_t, EpiLogits)

}  // namespace gpt2
