// Shared device-side helpers of the gfx950 kernels: element types, bf16
// conversion, 16-byte fragments and the MFMA wrappers used by the GEMM and
// attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gpt2 {

constexpr float kLog2e = 1.4426950408889634f;  // exp(x) = 2^(x * log2(e))

// bf16 is stored as raw 16-bit patterns; arithmetic is always fp32.
struct bf16_t {
  uint16_t bits;
};

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
// 16-byte fragment as a native clang vector.  Two compiler pitfalls are avoided
// throughout: HIP's uint4 (a union wrapper) is never used for fragments, and
// __builtin_bit_cast is applied to whole vectors, never to a vector element --
// on this toolchain bit_cast(float, v[e]) reads element 0 for every e.
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}
// Round to nearest even (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// Two floats -> packed pair of bf16 (lo in bits 0..15), one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_vec_t __attribute__((ext_vector_type(2)));
typedef float f32x2_vec_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_vec_t{lo, hi}, bf16x2_vec_t));
}

// Element traits: loading/storing groups of 4 elements as fp32.
template <typename T> struct Elem;

template <> struct Elem<float> {
  static constexpr int kBytes = 4;
  __device__ static __forceinline__ float to_f32(float v) { return v; }
  __device__ static __forceinline__ float from_f32(float v) { return v; }
  __device__ static __forceinline__ void store4(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
  }
  __device__ static __forceinline__ float4 load4(const float* p) {
    return *reinterpret_cast<const float4*>(p);
  }
};

template <> struct Elem<bf16_t> {
  static constexpr int kBytes = 2;
  __device__ static __forceinline__ float to_f32(bf16_t v) { return bf16_to_f32(v.bits); }
  __device__ static __forceinline__ bf16_t from_f32(float v) { return bf16_t{f32_to_bf16(v)}; }
  __device__ static __forceinline__ void store4(bf16_t* p, float a, float b, float c, float d) {
    *reinterpret_cast<u32x2_t*>(p) = u32x2_t{pack2_bf16(a, b), pack2_bf16(c, d)};
  }
  __device__ static __forceinline__ float4 load4(const bf16_t* p) {
    const u32x2_t u = *reinterpret_cast<const u32x2_t*>(p);
    return make_float4(bf16_to_f32(u[0] & 0xFFFF), bf16_to_f32(u[0] >> 16), bf16_to_f32(u[1] & 0xFFFF),
                       bf16_to_f32(u[1] >> 16));
  }
};

// Matrix-core step on one 16-byte fragment per lane.
//
// Fragment convention (both operands): lane l owns matrix row (l % 16) and a
// 16-byte run along k that starts at byte 16*(l / 16) of a 64-byte k-slab.
// Both operands use the same (lane group, element) -> k assignment, so the
// k-sum is complete whatever order the hardware pairs the elements in.
//   bf16: one v_mfma_f32_16x16x32_bf16 covers the 32 k of a slab.
//   f32:  four v_mfma_f32_16x16x4_f32 cover its 16 k (element j of every lane
//         in step j).
// Result (16x16, fp32): lane l holds rows 4*(l/16)+0..3 of column l%16 of
// A_rows x B_rows^T, where A_rows is the matrix whose rows the first operand
// supplies.
template <typename T> struct Mma;

template <> struct Mma<bf16_t> {
  static constexpr int kPerSlab = 32;
  __device__ static __forceinline__ void run(f32x4_t& acc, const u32x4_t& a, const u32x4_t& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  }
};

template <> struct Mma<float> {
  static constexpr int kPerSlab = 16;
  __device__ static __forceinline__ void run(f32x4_t& acc, const u32x4_t& a, const u32x4_t& b) {
    const f32x4_t fa = __builtin_bit_cast(f32x4_t, a);
    const f32x4_t fb = __builtin_bit_cast(f32x4_t, b);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[0], fb[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[1], fb[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[2], fb[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[3], fb[3], acc, 0, 0, 0);
  }
};

// Wave-wide reductions without LDS round trips: DPP exchanges inside each
// 16-lane row (quad swaps, then half-row and row mirrors), then the gfx950
// row-swap permutes across rows.  Every step combines a lane with a partner
// that combines the same two values, so all 64 lanes end with the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// op over the lanes l and l ^ 16 (rows 0/1 and 2/3 of the wave exchanged).
// The two results of a swap are copied to plain scalars before any bit cast
// (bit-casting an element of the returned pair in place reads element 0).
template <class Op>
__device__ __forceinline__ float combine_xor16(float v, Op op) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const unsigned r0 = r[0], r1 = r[1];
  return op(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1));
}
// op over the lanes l and l ^ 32 (the two halves of the wave exchanged).
template <class Op>
__device__ __forceinline__ float combine_xor32(float v, Op op) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned r0 = r[0], r1 = r[1];
  return op(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1));
}
// Arg-max pairs (v, i) over the lanes l and l ^ 16 (X = 16) or l ^ 32 (X = 32):
// the larger v wins, equal values go to the smaller i, so both lanes of a
// pair end with the same pair.  The same row-swap permute moves v and i.
template <int X>
__device__ __forceinline__ void argmax_xor(float& v, int& i) {
  const unsigned u = __builtin_bit_cast(unsigned, v), w = (unsigned)i;
  unsigned a0, a1, b0, b1;
  if constexpr (X == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const auto q = __builtin_amdgcn_permlane16_swap(w, w, false, false);
    a0 = r[0], a1 = r[1], b0 = q[0], b1 = q[1];
  } else {
    static_assert(X == 32, "lane distance");
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const auto q = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    a0 = r[0], a1 = r[1], b0 = q[0], b1 = q[1];
  }
  const float v0 = __builtin_bit_cast(float, a0), v1 = __builtin_bit_cast(float, a1);
  const int i0 = (int)b0, i1 = (int)b1;
  const bool first = v0 > v1 || (v0 == v1 && i0 < i1);
  v = first ? v0 : v1;
  i = first ? i0 : i1;
}
template <class Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
  v = op(v, dpp_f32<0xB1>(v));   // quad_perm [1,0,3,2]: lane ^ 1
  v = op(v, dpp_f32<0x4E>(v));   // quad_perm [2,3,0,1]: lane ^ 2
  v = op(v, dpp_f32<0x141>(v));  // row_half_mirror: the other quad of the 8
  v = op(v, dpp_f32<0x140>(v));  // row_mirror: the other 8 of the 16
  v = combine_xor16(v, op);
  return combine_xor32(v, op);
}
// op over aligned groups of W consecutive lanes (W = 1, 2, 4, 8 or 16): the
// DPP steps of wave_reduce; every lane of a group ends with its result.
template <int W, class Op>
__device__ __forceinline__ float group_reduce(float v, Op op) {
  static_assert(W == 1 || W == 2 || W == 4 || W == 8 || W == 16, "group width");
  if constexpr (W >= 2) v = op(v, dpp_f32<0xB1>(v));
  if constexpr (W >= 4) v = op(v, dpp_f32<0x4E>(v));
  if constexpr (W >= 8) v = op(v, dpp_f32<0x141>(v));
  if constexpr (W >= 16) v = op(v, dpp_f32<0x140>(v));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  return wave_reduce(v, [](float a, float b) { return a + b; });
}
__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}

// exp(x) through the hardware base-2 exponential.
__device__ __forceinline__ float exp_via_exp2(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// gelu_new(x) = 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))).
// Since 0.5 (1 + tanh(y)) = 1 / (1 + exp(-2y)), this is x / (1 + exp(-2y)):
// one base-2 exponential and one hardware reciprocal (v_rcp_f32, 1 ulp), no
// IEEE division.  Saturates to x (large x) and to -0 (very negative x).
__device__ __forceinline__ float gelu_tanh(float x) {
  // -2 * sqrt(2/pi) * log2(e), and the same times 0.044715
  const float c1 = -2.3022081981f, c3 = -0.1029432396f;
  const float x2 = x * x;
  const float z = x * (c1 + c3 * x2);          // -2y * log2(e)
  const float e = __builtin_amdgcn_exp2f(z);   // exp(-2y)
  return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// The erf GELU, 0.5 x (1 + erf(x / sqrt(2))), with the device library's erff.
__device__ __forceinline__ float gelu_erf(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }

// Derivatives for the backward pass:
// gelu_new'(x) = 0.5 (1 + t) + 0.5 x (1 - t^2) k (1 + 3 c x^2),
//   t = tanh(y), y = k (x + c x^3), k = sqrt(2/pi), c = 0.044715.
// With s = (1 + t) / 2 = 1 / (1 + exp(-2y)) (the sigmoid the forward uses)
// and 1 - t^2 = 4 s (1 - s) this is s + 2 x s (1 - s) k (1 + 3 c x^2): one
// exp2 and one reciprocal, as in gelu_tanh; s saturates to 0 or 1 without NaN.
// gelu'(x) = Phi(x) + x phi(x) for the erf form (device library erff / expf).
__device__ __forceinline__ float gelu_tanh_grad(float x) {
  const float k = 0.7978845608028654f, c = 0.044715f;
  const float c1 = -2.3022081981f, c3 = -0.1029432396f;  // -2 k log2(e), times c
  const float x2 = x * x;
  const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * (c1 + c3 * x2)));
  return s + 2.0f * x * s * (1.0f - s) * k * (1.0f + 3.0f * c * x2);
}
__device__ __forceinline__ float gelu_erf_grad(float x) {
  return 0.5f * (1.0f + erff(x * 0.70710678118654752f)) + x * expf(-0.5f * x * x) * 0.3989422804014327f;
}

// Workgroup i of a grid runs on XCD i % 8 (MI355X: 8 accelerator dies, each
// with its own L2; the GEMM tile order relies on the same placement).
// xcd_block renumbers a grid of n blocks so that each XCD takes a contiguous
// eighth of the work: block i handles item (i % 8) * (n / 8) + i / 8 when
// n % 8 == 0 (identity otherwise).  Row kernels use it so that the rows an
// XCD reads are the rows the same XCD wrote in the GEMM before (and writes
// the rows the same XCD reads in the GEMM after): those accesses then hit
// its L2 instead of crossing to another die's data.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_block(int i, int n) {
  return (n % kXcds == 0) ? (i % kXcds) * (n / kXcds) + i / kXcds : i;
}

// Division by a runtime-invariant positive divisor through a precomputed
// multiplier (Granlund & Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994): for 0 <= n < 2^31 and 1 <= d < 2^31,
// n / d = (umulhi(n, magic) + n) >> shift with shift = ceil(log2 d),
// magic = floor(2^32 (2^shift - d) / d) + 1.
struct FastDiv {
  uint32_t d, magic, shift;
  __host__ __device__ FastDiv() : d(1), magic(1), shift(0) {}
  __host__ explicit FastDiv(uint32_t div) : d(div) {
    shift = 0;
    while ((1u << shift) < div) ++shift;
    const uint64_t one = 1;
    magic = (uint32_t)(((one << 32) * ((one << shift) - div)) / div + 1);
  }
  __device__ __forceinline__ uint32_t div(uint32_t n) const {
    return (__umulhi(n, magic) + n) >> shift;
  }
};

}  // namespace gpt2
