// Device helpers shared by the GCA kernels (gfx950 / CDNA4 only).
//
// Matrix-core conventions used throughout (wave64, 32x32 output tiles):
//   * v_mfma_f32_32x32x16_bf16: lane l supplies 8 bf16 of A row (l % 32) and 8 bf16 of B column
//     (l % 32); element e of lane group h = l / 32 of A meets element e of group h of B in the
//     contraction.  Output element r (0..15) of lane l is D[8(r/4) + 4(l/32) + r%4][l % 32].
//   * v_mfma_f32_32x32x2_f32 has the same output layout; one instruction contracts over the two
//     lane groups, so an 8-element fp32 fragment is issued as 8 instructions (element e of both
//     operands in the e-th).  The set of products is the same as for the bf16 form.
//   * Row permutation pi: loading A row pi(rho) into MFMA row rho makes output element r of lane
//     group h hold logical row 16 h + r, so each lane owns 16 consecutive logical rows per tile.
//     pi(8a + 4c + m) = 16c + 4a + m  (a in 0..3, c in 0..1, m in 0..3).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gca {

constexpr int kChunk = 64;   // S
constexpr int kDim = 64;     // d_head == d_lmk
constexpr int kMaxTopk = 16;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

struct bf16_t {  // storage type of one bf16 value
  uint16_t bits;
};

__device__ __forceinline__ int pi_row(int rho) {
  return ((rho >> 2) & 1) * 16 + (rho >> 3) * 4 + (rho & 3);
}

// ------------------------------------------------------------------ conversions
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// ------------------------------------------------------------------ fragments
// Eight operand elements per lane.
template <typename T>
struct Frag;

template <>
struct Frag<bf16_t> {
  u32x4_t v;  // 8 x bf16
  __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const u32x4_t*>(p); }
  __device__ __forceinline__ void set(const float* x) {
    v[0] = pack_bf16x2(x[0], x[1]);
    v[1] = pack_bf16x2(x[2], x[3]);
    v[2] = pack_bf16x2(x[4], x[5]);
    v[3] = pack_bf16x2(x[6], x[7]);
  }
};

template <>
struct Frag<float> {
  f32x4_t v0, v1;
  __device__ __forceinline__ void load(const float* p) {
    v0 = reinterpret_cast<const f32x4_t*>(p)[0];
    v1 = reinterpret_cast<const f32x4_t*>(p)[1];
  }
  __device__ __forceinline__ void set(const float* x) {
    v0 = f32x4_t{x[0], x[1], x[2], x[3]};
    v1 = f32x4_t{x[4], x[5], x[6], x[7]};
  }
};

__device__ __forceinline__ f32x16_t mma(const Frag<bf16_t>& a, const Frag<bf16_t>& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a.v),
                                                 __builtin_bit_cast(bf16x8_t, b.v), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t mma(const Frag<float>& a, const Frag<float>& b, f32x16_t c) {
#pragma unroll
  for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v0[e], b.v0[e], c, 0, 0, 0);
#pragma unroll
  for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v1[e], b.v1[e], c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

// Load/store of 4 consecutive elements.
__device__ __forceinline__ void store4(bf16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<u32x2_t*>(p) = u32x2_t{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4_t*>(p) = f32x4_t{a, b, c, d};
}
__device__ __forceinline__ float to_f32(bf16_t x) { return bf16_to_f32(x.bits); }
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ void from_f32(bf16_t* p, float x) { p->bits = static_cast<uint16_t>(f32_to_bf16_bits(x)); }
__device__ __forceinline__ void from_f32(float* p, float x) { *p = x; }

// ------------------------------------------------------------------ cross-lane
// Combine with the partner lane l ^ 32 through v_permlane32_swap.
__device__ __forceinline__ float xor32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------------ XCD-aware block order
// Workgroups are dispatched round-robin over the 8 XCDs.  Map the hardware block index so
// that each XCD walks one contiguous range of logical work items: items that share data
// (same batch row and head) then run on the same XCD and meet in its L2.
__device__ __forceinline__ int64_t xcd_logical_block(int64_t bid, int64_t nblocks) {
  const int64_t nx = 8;
  const int64_t x = bid % nx, n = bid / nx;
  const int64_t q = nblocks / nx, rem = nblocks % nx;
  return x * q + (x < rem ? x : rem) + n;
}

}  // namespace gca
