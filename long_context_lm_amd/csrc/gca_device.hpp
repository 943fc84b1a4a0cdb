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
typedef int32_t i32x2_t __attribute__((ext_vector_type(2)));
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

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

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2v_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair with round-to-nearest-even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v_t{lo, hi}, bf16x2_t));
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

// An opaque use of a fragment: the value must be in registers at this point of the program.
__device__ __forceinline__ void pin_in_registers(Frag<bf16_t>& f) { asm volatile("" : "+v"(f.v)); }
__device__ __forceinline__ void pin_in_registers(Frag<float>& f) { asm volatile("" : "+v"(f.v0), "+v"(f.v1)); }

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

namespace gca {

// ------------------------------------------------------------------ 64x64 tiles in LDS
// Row-major, 64 elements per row, no padding; the 16-byte chunks of row R sit at chunk position
// c ^ swz(R), swz(R) = ((R & 3) << 1) ^ ((R >> 2) & 7).  Among the swizzles measured on gfx950
// this one leaves both access patterns the kernels use free of LDS bank conflicts: the 16-byte
// reads of MFMA rows pi(rho) and the 4-row x 16-column blocks of the transposing reads.
template <typename T>
struct Tile {
  static constexpr int kElemsPerChunk = 16 / static_cast<int>(sizeof(T));  // 8 bf16 or 4 fp32
  static constexpr int kChunksPerRow = kDim / kElemsPerChunk;
  static constexpr int kRowBytes = kDim * static_cast<int>(sizeof(T));
  static constexpr int kBytes = kChunk * kRowBytes;
  static constexpr int kChunks = kBytes / 16;
  __device__ static __forceinline__ int swz(int row) { return ((row & 3) << 1) ^ ((row >> 2) & 7); }
  __device__ static __forceinline__ int chunk_offset(int row, int chunk) {
    return row * kRowBytes + ((chunk ^ swz(row)) << 4);
  }
  __device__ static __forceinline__ int elem_offset(int row, int col) {
    return chunk_offset(row, col / kElemsPerChunk) + (col % kElemsPerChunk) * static_cast<int>(sizeof(T));
  }
};

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void gbl_void_t;

// Asynchronous copy global -> LDS of 16 bytes per lane: lane l of the wave writes bytes
// [16 l, 16 l + 16) after `lds_wave_base` (which must be the same in every lane).
__device__ __forceinline__ void copy16_async(const void* gsrc, char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)(gsrc), (lds_void_t*)(lds_wave_base), 16, 0, 0);
}

// The same copy issued from inline assembly: the compiler does not see it as a write to LDS, so
// it never makes later LDS reads wait for it.  The caller must order every read of the target
// after the copy itself (wait_vm_outstanding / barrier_copies_landed, then a barrier).  Extra
// vector memory operations the compiler does not count only make its own waits stricter; the
// caller's counted waits, though, hold only while its own copies and stores are the only vector
// memory operations in flight (no scratch, no flat access, no callee touching memory: the build
// checks this for every file that uses the copy).  gbase must already be a wave-uniform scalar
// (the "s" constraint); never force a vector value into it with readfirstlane.
__device__ __forceinline__ void copy16_async_untracked(const void* gbase, uint32_t lane_off, char* lds_wave_base) {
  const uint32_t lds_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)(lds_wave_base)));
  asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(lane_off), "s"(gbase), "{m0}"(lds_addr) : "memory");
}

// The same copy with the LDS destination given as its 32-bit LDS address (see lds_address):
// no generic-pointer round trip, whose null check the backend cannot always fold.
__device__ __forceinline__ void copy16_async_untracked_at(const void* gbase, uint32_t lane_off, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(lane_off), "s"(gbase), "{m0}"(lds_addr) : "memory");
}

// 32-bit LDS address of a __shared__ array.
__device__ __forceinline__ uint32_t lds_address(const char* lds) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)(lds)));
}

// Start copying one 64x64 tile (global row stride 64 elements) into swizzled LDS.  All threads of
// a workgroup of kWaves waves call it; each wave issues its share of the 1 KiB wave copies.  The
// data is usable after wait_async_copies() and a workgroup barrier.
// `wave` is the caller's wave index within the kWaves waves that share the copy.
template <typename T, int kWaves>
__device__ __forceinline__ void tile_load_async(const T* __restrict__ g, char* lds, int wave) {
  using TL = Tile<T>;
  const int lane = threadIdx.x & 63;
  const char* gb = reinterpret_cast<const char*>(g);
#pragma unroll
  for (int n = 0; n < TL::kChunks / 64 / kWaves; ++n) {
    const int blk = n * kWaves + wave;
    const int pos = blk * 64 + lane;
    const int row = pos / TL::kChunksPerRow;
    const int chunk = (pos % TL::kChunksPerRow) ^ TL::swz(row);
    // uniform tile base + 32-bit lane offset, so the copy can use the scalar-base address form
    const uint32_t off = static_cast<uint32_t>(row * TL::kRowBytes + chunk * 16);
    copy16_async(gb + off, lds + blk * 1024);
  }
}

template <typename T, int kWaves>
__device__ __forceinline__ void tile_load_async(const T* __restrict__ g, char* lds) {
  tile_load_async<T, kWaves>(g, lds, __builtin_amdgcn_readfirstlane(threadIdx.x >> 6));
}

__device__ __forceinline__ void wait_async_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait until at most N of this wave's vector memory operations are outstanding.  On gfx950 they
// retire in issue order (loads, stores and LDS copies alike), so this waits for everything
// issued before the N most recent.
template <int N>
__device__ __forceinline__ void wait_vm_outstanding() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barriers without the memory fence of __syncthreads() (which waits for every
// outstanding global access, in-flight prefetch copies included).  Each wave first waits for what
// the other waves rely on: its LDS reads of a buffer about to be refilled, or its own copies
// into a buffer about to be read (all but the N most recent vector memory operations).
__device__ __forceinline__ void barrier_lds_reads_done() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
template <int N>
__device__ __forceinline__ void barrier_copies_landed() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}
// Both: this wave's copies landed (all but the N most recent) and its LDS reads finished.
template <int N>
__device__ __forceinline__ void barrier_copies_landed_reads_done() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// MFMA operand holding 8 consecutive columns of one tile row: lane gets X[row][col0 .. col0+7].
__device__ __forceinline__ Frag<bf16_t> frag_row(const char* lds, int row, int col0, bf16_t*) {
  Frag<bf16_t> f;
  f.v = *reinterpret_cast<const u32x4_t*>(lds + Tile<bf16_t>::chunk_offset(row, col0 >> 3));
  return f;
}
__device__ __forceinline__ Frag<float> frag_row(const char* lds, int row, int col0, float*) {
  Frag<float> f;
  f.v0 = *reinterpret_cast<const f32x4_t*>(lds + Tile<float>::chunk_offset(row, col0 >> 2));
  f.v1 = *reinterpret_cast<const f32x4_t*>(lds + Tile<float>::chunk_offset(row, (col0 >> 2) + 1));
  return f;
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));

// MFMA operand holding 8 consecutive rows of one tile column: lane l (rho = l % 32) gets
// X[r0 + e][c_base + rho], e = 0..7 (r0 the same within each half-wave).  For bf16 the 16 lanes of
// a block read a 4-row x 16-column block in row-major 8-byte pieces with ds_read_b64_tr_b16, which
// hands lane i of the block the four rows of column i.
__device__ __forceinline__ Frag<bf16_t> frag_col(const char* lds, int r0, int c_base, bf16_t*) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, bb = (lane >> 4) & 1;
  const int col = c_base + 16 * bb + 4 * (j & 3);
  const int row = r0 + (j >> 2);
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4_t*)(lds + Tile<bf16_t>::elem_offset(row, col)));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4_t*)(lds + Tile<bf16_t>::elem_offset(row + 4, col)));
  Frag<bf16_t> f;
  const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo);
  const u32x2_t h2 = __builtin_bit_cast(u32x2_t, hi);
  f.v = u32x4_t{l2[0], l2[1], h2[0], h2[1]};
  return f;
}
__device__ __forceinline__ Frag<float> frag_col(const char* lds, int r0, int c_base, float*) {
  const int rho = threadIdx.x & 31;
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = *reinterpret_cast<const float*>(lds + Tile<float>::elem_offset(r0 + e, c_base + rho));
  Frag<float> f;
  f.set(x);
  return f;
}

}  // namespace gca
