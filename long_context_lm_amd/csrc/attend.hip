// Grouped cross-attention over retrieved chunks: forward and backward.
//
// [Notes, Key designs: GCA]: every token of the current chunk attends to each retrieved chunk
// separately, with its own softmax; the per-chunk outputs are fused with weights given by a
// softmax of the retrieval scores, so the scores receive gradients of the language-model loss
// [Notes, Background: entry point].  K/V are shared by all retrieval groups [Notes, Key
// designs: GCA].
//
// Tiles.  A chunk is 64 tokens and the head dim is 64, so one retrieved chunk of one head is a
// 64x64 K tile and a 64x64 V tile, and one (query chunk, head) is a 64x64 Q tile.  A workgroup
// of two waves owns one 64-query tile (forward and query-major backward) or one 64-key tile
// (key-major backward); each wave owns 32 rows and all 64 columns.  Each per-chunk softmax
// covers exactly one 64-key tile, so it is computed whole, without online rescaling.
//
// Data movement.  The tiles a workgroup walks through (K/V of each retrieved chunk, or Q/dO of
// each retrieving chunk) are copied global -> LDS with direct 16-byte-per-lane copies into a
// row-major, XOR-swizzled layout.  The backward passes double-buffer them (the copy of item n+1
// is in flight while item n is computed; one barrier per item publishes the new buffer and
// retires the old); the forward keeps one K and one V buffer, refills each as soon as its
// fragments are in registers, and relies on the other resident workgroups (two waves per SIMD)
// to cover the rest of the copy latency.
// Operands read along a tile row come from ds_read_b128; operands read down a tile column (V in
// the forward, K in dQ, Q and dO in dK/dV) come from transposing LDS reads, so no tile is ever
// stored transposed.
//
// Layout trick (see gca_device.hpp): S^T = K Q^T is computed with the K rows loaded through the
// permutation pi, which leaves each lane holding 16 consecutive keys of one query per 32-key
// tile; that register block is directly the B operand (P^T) of O^T = V^T P^T.
//
// Backward without floating-point atomics.  dQ and the per-slot sums of e = <dO, O_k> are
// produced query-major (one workgroup per query tile).  dK and dV are produced key-major: an
// inverse index lists, per (batch row, key chunk), the (group, row, slot) retrievals that
// selected it in a fixed order; one workgroup per (batch row, head, key chunk) walks that list
// and accumulates in registers.  d(score) sums the per-head partials in a fixed order.
#include <type_traits>

#include "gca_device.hpp"
#include "gca_internal.hpp"

namespace gca {
namespace {

constexpr int kThreads = 128;  // two waves
constexpr int kWaves = 2;
constexpr int kEntRound = 512;  // inverse-index entries staged in LDS at a time
constexpr int64_t kWideMaxTiles = 256;  // query tiles up to which the forward runs one slot per wave
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2f = 0.6931471805599453f;

// Slot table of one retrieval row: valid slots (0 <= j < n_kv) in slot order, with the fusion
// weights w = softmax over the valid slots of the clean scores.
struct SlotTable {
  int32_t j[kMaxTopk];
  int32_t slot[kMaxTopk];
  float w[kMaxTopk];
  float w_all[kMaxTopk];  // by slot, 0 on invalid slots
  uint32_t valid_mask;
  int n;
};

struct WaveSlots {
  int32_t j;        // lane k: chunk of slot k
  float w;          // lane k: fusion weight of slot k (0 if invalid)
  uint32_t valid;   // bit k: slot k valid
};

// Slots of one retrieval row, computed lane-parallel by one wave: lanes < K load the row's index
// and score together (one memory round trip), the maximum over the valid slots is a butterfly
// (exact, so its order does not matter), and the exponentials are summed in slot order.
__device__ __forceinline__ WaveSlots wave_slots(const AttendParams& p, int g, int b, int64_t row) {
  const int lane = threadIdx.x & 63;
  WaveSlots ws{-1, 0.f, 0u};
  if (row < 0) return ws;
  const int64_t base = ((static_cast<int64_t>(g) * p.B + b) * p.n_q + row) * p.K;
  float sc = -__builtin_inff();
  if (lane < p.K) {
    ws.j = p.idx[base + lane];
    sc = p.score[base + lane];
  }
  const bool v = lane < p.K && ws.j >= 0 && ws.j < p.n_kv;
  ws.valid = static_cast<uint32_t>(__ballot(v));
  // maximum over lanes 0..15 (K <= 16): four DPP steps inside the 16-lane row (the swaps of
  // neighbours and of pairs, then the mirrors of each half and of the row), exact in any order
  float mx = v ? sc : -__builtin_inff();
  auto row_max = [](float x, auto ctrl) {
    const int y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value, 0xf, 0xf, true);
    return fmaxf(x, __int_as_float(y));
  };
  mx = row_max(mx, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
  mx = row_max(mx, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
  mx = row_max(mx, std::integral_constant<int, 0x141>{});  // row_half_mirror
  mx = row_max(mx, std::integral_constant<int, 0x140>{});  // row_mirror
  mx = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(mx)));  // lane 0: slots 0..15
  const float e = v ? expf(sc - mx) : 0.f;
  float sum = 0.f;
  for (int k = 0; k < p.K; ++k)
    if ((ws.valid >> k) & 1u) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(e), k));
  ws.w = v ? e / sum : 0.f;
  return ws;
}

// The slot table of one retrieval row in LDS, filled by every lane of one wave from wave_slots:
// valid slot k goes to position popcount(valid below k), so the table keeps slot order.  The
// caller publishes it with a barrier.
__device__ __forceinline__ void fill_slot_table(SlotTable& st, const AttendParams& p, int g, int b, int64_t row) {
  const int lane = threadIdx.x & 63;
  const WaveSlots ws = wave_slots(p, g, b, row);
  if (lane < kMaxTopk) {
    st.w_all[lane] = ws.w;
    if ((ws.valid >> lane) & 1u) {
      const int pos = __popc(ws.valid & ((1u << lane) - 1u));
      st.j[pos] = ws.j;
      st.slot[pos] = lane;
      st.w[pos] = ws.w;
    }
  }
  if (lane == 0) {
    st.n = __popc(ws.valid);
    st.valid_mask = ws.valid;
  }
}

struct QTileCoord {
  int b, h, g;
  int64_t t;
  int64_t gbh;  // (g * B + b) * H + h
};

// Group fastest, then query chunk: both groups' tiles of one (batch row, head) and chunk run side
// by side and share each K/V tile while it is in L2.
// The grid has G B H n_q < 2^31 blocks (checked on the host), so 32-bit divisions suffice.
__device__ __forceinline__ QTileCoord query_tile_coord(const AttendParams& p) {
  const uint32_t lid = static_cast<uint32_t>(xcd_logical_block(blockIdx.x, gridDim.x));
  const uint32_t G = static_cast<uint32_t>(p.G), H = static_cast<uint32_t>(p.H);
  const uint32_t nq = static_cast<uint32_t>(p.n_q);
  QTileCoord c;
  uint32_t rest = lid / G;
  c.g = static_cast<int>(lid - rest * G);
  const uint32_t bh = rest / nq;
  c.t = rest - bh * nq;
  c.b = static_cast<int>(bh / H);
  c.h = static_cast<int>(bh - static_cast<uint32_t>(c.b) * H);
  c.gbh = (static_cast<int64_t>(c.g) * p.B + c.b) * p.H + c.h;
  return c;
}

// Per-(chunk, slot) vectors of 64 floats (lse, e) live at [gbh][t][slot][64].
__device__ __forceinline__ int64_t slot_vec_offset(const AttendParams& p, int64_t gbh, int64_t t, int slot) {
  return ((gbh * p.n_q + t) * p.K + slot) * kChunk;
}

template <typename T>
__device__ __forceinline__ const T* kv_tile(const void* base, const AttendParams& p, int b, int h, int64_t j) {
  return static_cast<const T*>(base) + ((static_cast<int64_t>(b) * p.H + h) * p.n_kv + j) * kChunk * kDim;
}

template <typename T>
__device__ __forceinline__ Frag<T> row_frag(const char* tile, int row, int col0) {
  return frag_row(tile, row, col0, static_cast<T*>(nullptr));
}
template <typename T>
__device__ __forceinline__ Frag<T> col_frag(const char* tile, int r0, int c_base) {
  return frag_col(tile, r0, c_base, static_cast<T*>(nullptr));
}

// ------------------------------------------------------------------------------ forward
// Per-lane LDS offsets of the MFMA operand reads and tile copies.  They do not change from slot
// to slot, so they are computed once and pinned in registers (opaque to the compiler, which would
// otherwise recompute the swizzles in every iteration of the slot loops).  kfrag reads an operand
// along tile rows (rows pi(l % 32), as S^T = X Q^T wants them); vfrag reads one down tile columns
// with the transposing LDS read (X^T as the A operand of O^T = X^T P^T).
template <typename T, int kWaves>
struct TileOffsets {
  // bf16: K row fragments [s] (rows 32..63 at +4096); transposing V reads [(s & 1), dt, lo/hi]
  // (rows 32..63 at +4096); copy offsets of this lane's 16-byte pieces [n] of a tile.
  static constexpr int kCopies = Tile<T>::kChunks / 64 / kWaves;
  uint32_t k[4], v[8], cp[kCopies];

  __device__ __forceinline__ void init(int wave) { init(wave, static_cast<int>(threadIdx.x)); }
  // the same with the thread index given (an opaque copy keeps the offsets from being hoisted
  // out of a loop of walks, where they would stay live across the loop)
  __device__ __forceinline__ void init(int wave, int tid) {
    using TL = Tile<T>;
    const int lane = tid & 63, li = lane & 31, hl = lane >> 5;
#pragma unroll
    for (int n = 0; n < kCopies; ++n) {
      const int pos = (n * kWaves + wave) * 64 + lane;
      const int row = pos / TL::kChunksPerRow;
      cp[n] = static_cast<uint32_t>(TL::chunk_offset(row, pos % TL::kChunksPerRow));
    }
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int s = 0; s < 4; ++s) k[s] = static_cast<uint32_t>(TL::chunk_offset(pi_row(li), 2 * s + hl));
      const int j = lane & 15, bb = (lane >> 4) & 1;
#pragma unroll
      for (int s1 = 0; s1 < 2; ++s1)
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const int row = 16 * hl + 8 * s1 + (j >> 2), col = 32 * dt + 16 * bb + 4 * (j & 3);
          v[4 * s1 + 2 * dt] = static_cast<uint32_t>(TL::elem_offset(row, col));
          v[4 * s1 + 2 * dt + 1] = static_cast<uint32_t>(TL::elem_offset(row + 4, col));
        }
#pragma unroll
      for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(k[i]));
#pragma unroll
      for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(v[i]));
    }
#pragma unroll
    for (int n = 0; n < kCopies; ++n) asm volatile("" : "+v"(cp[n]));
  }

  // Copy one 64x64 tile (global row stride 64; `g` uniform) into swizzled LDS: kCopies vector
  // memory operations per wave, untracked by the compiler (see copy16_async_untracked).
  __device__ __forceinline__ void copy(const T* __restrict__ g, char* lds, int wave) const {
#pragma unroll
    for (int n = 0; n < kCopies; ++n) copy16_async_untracked(g, cp[n], lds + (n * kWaves + wave) * 1024);
  }
  // the same, to the LDS address lds_addr (lds_address of the buffer)
  __device__ __forceinline__ void copy_at(const T* __restrict__ g, uint32_t lds_addr, int wave) const {
#pragma unroll
    for (int n = 0; n < kCopies; ++n)
      copy16_async_untracked_at(g, cp[n], lds_addr + static_cast<uint32_t>((n * kWaves + wave) * 1024));
  }

  __device__ __forceinline__ Frag<T> kfrag(const char* Ks, int tt, int s) const {
    if constexpr (sizeof(T) == 2) {
      Frag<T> f;
      f.v = *reinterpret_cast<const u32x4_t*>(Ks + k[s] + 4096 * tt);
      return f;
    } else {
      const int li = threadIdx.x & 31, hl = (threadIdx.x >> 5) & 1;
      return frag_row(Ks, 32 * tt + pi_row(li), 16 * s + 8 * hl, static_cast<T*>(nullptr));
    }
  }

  // V^T operand: rows 32 (s >> 1) + 16 hl + 8 (s & 1) .. +7 of columns 32 dt .. 32 dt + 31.
  __device__ __forceinline__ Frag<T> vfrag(const char* Vs, int s, int dt) const {
    if constexpr (sizeof(T) == 2) {
      typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
      const char* base = Vs + 4096 * (s >> 1);
      const int i = 4 * (s & 1) + 2 * dt;
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(base + v[i]));
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(base + v[i + 1]));
      const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo);
      const u32x2_t h2 = __builtin_bit_cast(u32x2_t, hi);
      Frag<T> f;
      f.v = u32x4_t{l2[0], l2[1], h2[0], h2[1]};
      return f;
    } else {
      const int hl = (threadIdx.x >> 5) & 1;
      return frag_col(Vs, 32 * (s >> 1) + 16 * hl + 8 * (s & 1), 32 * dt, static_cast<T*>(nullptr));
    }
  }
};

// Softmax of one 64-key tile held as S^T accumulators (16 keys per lane per 32-key half, the
// other 32 keys in lane ^ 32): returns the row maximum; sacc becomes exp2((s - max) * c2) and l
// their sum.
__device__ __forceinline__ float tile_softmax(f32x16_t (&sacc)[2], float c2, float& l) {
  float m0 = fmaxf(sacc[0][0], sacc[0][1]), m1 = fmaxf(sacc[1][0], sacc[1][1]);
#pragma unroll
  for (int r = 2; r < 16; r += 2) {  // three-operand maxima
    m0 = fmaxf(fmaxf(m0, sacc[0][r]), sacc[0][r + 1]);
    m1 = fmaxf(fmaxf(m1, sacc[1][r]), sacc[1][r + 1]);
  }
  const float mx = xor32_max(fmaxf(m0, m1));
  const float bias = -mx * c2;
  float l0 = 0.f, l1 = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    sacc[0][r] = fast_exp2(__builtin_fmaf(sacc[0][r], c2, bias));
    sacc[1][r] = fast_exp2(__builtin_fmaf(sacc[1][r], c2, bias));
    l0 += sacc[0][r];
    l1 += sacc[1][r];
  }
  l = xor32_sum(l0 + l1);
  return mx;
}

// Two waves of 32 queries per query tile (the fp32 forward; bf16 uses the one-wave kernel below).
// Slot loop, software-pipelined over one K and one V buffer (32 KiB of LDS for fp32 tiles; the
// registers allow two waves per SIMD): once every wave has read K(n) for the scores, K(n+1) is copied
// in behind the softmax and P V of slot n; once every wave has read V(n), V(n+1) is copied in
// behind the scores and softmax of slot n+1.  Each wave waits only for its own copies (counted
// with vmcnt, in issue order) and a barrier then publishes them to the other wave.  kLse: the
// log-sum-exp output is written (one store per slot, which the counts include).
template <typename T, bool kLse>
__global__ __launch_bounds__(kThreads) void attend_fwd_kernel(AttendParams p) {
  using TL = Tile<T>;
  using Off = TileOffsets<T, kWaves>;
  constexpr int kC = Off::kCopies;  // copies per wave per tile
  // Separate arrays, so that the compiler's own tracking of LDS copies never makes a read of
  // one buffer wait for the copy into the other.
  __shared__ __align__(1024) char Ks[TL::kBytes];
  __shared__ __align__(1024) char Vs[TL::kBytes];
  __shared__ SlotTable st;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, hl = lane >> 5;
  const QTileCoord c = query_tile_coord(p);
  const int64_t Lq = p.n_q * kChunk;
  const int64_t qrow0 = c.gbh * Lq + c.t * kChunk;
  const int my_q = 32 * wave + li;

  Frag<T> qf[4];
  const T* q = static_cast<const T*>(p.q) + (qrow0 + my_q) * kDim;
#pragma unroll
  for (int s = 0; s < 4; ++s) qf[s].load(q + 16 * s + 8 * hl);
  if (wave == 0) fill_slot_table(st, p, c.g, c.b, c.t - p.shift);  // its loads beside the query's
  Off off;
  off.init(wave);
  __syncthreads();

  const int nslots = st.n;
  float* const lse_q = kLse ? p.lse + slot_vec_offset(p, c.gbh, c.t, 0) + my_q : nullptr;
  if (kLse) {  // invalid slots: -inf (before any copy, so the copy counts below stay exact)
    for (int e = tid; e < p.K * kChunk; e += kThreads)
      if (!((st.valid_mask >> (e / kChunk)) & 1u)) p.lse[slot_vec_offset(p, c.gbh, c.t, 0) + e] = -__builtin_inff();
  }
  auto chunk_of = [&](int n) { return __builtin_amdgcn_readfirstlane(st.j[n]); };  // uniform
  if (nslots > 0) {
    const int32_t j = chunk_of(0);
    off.copy(kv_tile<T>(p.k, p, c.b, c.h, j), Ks, wave);
    off.copy(kv_tile<T>(p.v, p, c.b, c.h, j), Vs, wave);
    barrier_copies_landed<kC>();  // K(0) landed and visible; V(0) may still be in flight
  }
  // The query fragments are pinned here, before the loop, so that the compiler waits for them
  // once (left to their first use in the loop, its vmcnt waits would run in every iteration and
  // also wait for the prefetch copies in flight).
#pragma unroll
  for (int s = 0; s < 4; ++s) pin_in_registers(qf[s]);

  f32x16_t oacc[2] = {zero16(), zero16()};
  const float c2 = p.attn_scale * kLog2e;
  for (int n = 0; n < nslots; ++n) {
    const bool more = n + 1 < nslots;
    f32x16_t sacc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      sacc[tt] = zero16();
#pragma unroll
      for (int s = 0; s < 4; ++s) sacc[tt] = mma(off.kfrag(Ks, tt, s), qf[s], sacc[tt]);
    }
    barrier_lds_reads_done();  // every wave has read K(n)
    if (more) off.copy(kv_tile<T>(p.k, p, c.b, c.h, chunk_of(n + 1)), Ks, wave);

    float l;
    const float mx = tile_softmax(sacc, c2, l);
    const float f = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(st.w[n]))) * __builtin_amdgcn_rcpf(l);
    Frag<T> pf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = sacc[s >> 1][8 * (s & 1) + e] * f;
      pf[s].set(x);
    }
    if (more) barrier_copies_landed<kC>();  // V(n) landed and visible (K(n+1) may be in flight)
    else barrier_copies_landed<0>();
    if (kLse && hl == 0)
      lse_q[__builtin_amdgcn_readfirstlane(st.slot[n]) * kChunk] = mx * p.attn_scale + __builtin_amdgcn_logf(l) * kLn2f;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int s = 0; s < 4; ++s) oacc[dt] = mma(off.vfrag(Vs, s, dt), pf[s], oacc[dt]);
    if (more) {
      barrier_lds_reads_done();  // every wave has read V(n)
      off.copy(kv_tile<T>(p.v, p, c.b, c.h, chunk_of(n + 1)), Vs, wave);
      barrier_copies_landed<kC + (kLse ? 1 : 0)>();  // K(n+1) landed (the lse store, V(n+1) may not)
    }
  }

  T* o = static_cast<T*>(p.o) + (qrow0 + my_q) * kDim;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a)
      store4(o + 32 * dt + 8 * a + 4 * hl, oacc[dt][4 * a], oacc[dt][4 * a + 1], oacc[dt][4 * a + 2],
             oacc[dt][4 * a + 3]);
}

// ------------------------------------------------------------ forward, one wave per tile (bf16)
// One wave owns a whole 64-query tile: K and V fragments are read from LDS once per slot and
// used for both 32-query halves (half the LDS reads of two waves sharing the tile), the two
// halves give the wave independent MFMA and softmax work to interleave, and a single-wave
// workgroup needs no barriers.  The slot list lives in registers (lane k < K holds slot k).  The
// same one-buffer pipeline as above: K(next) is copied in once K(n) is in registers, V(next)
// once V(n) is, each wait counted in vector memory operations (in issue order).
template <bool kLse>
__global__ __launch_bounds__(64) void attend_fwd_wave_kernel(AttendParams p) {
  using T = bf16_t;
  using TL = Tile<T>;
  using Off = TileOffsets<T, 1>;
  constexpr int kC = Off::kCopies;  // 8 copies per tile
  __shared__ __align__(1024) char Ks[TL::kBytes];
  __shared__ __align__(1024) char Vs[TL::kBytes];

  const int lane = threadIdx.x, li = lane & 31, hl = lane >> 5;
  const QTileCoord c = query_tile_coord(p);
  const int64_t Lq = p.n_q * kChunk;
  const int64_t qrow0 = c.gbh * Lq + c.t * kChunk;

  Frag<T> qf[2][4];
#pragma unroll
  for (int qh = 0; qh < 2; ++qh) {
    const T* q = static_cast<const T*>(p.q) + (qrow0 + 32 * qh + li) * kDim;
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[qh][s].load(q + 16 * s + 8 * hl);
  }
  // after the query loads, so that one memory round trip covers both
  const WaveSlots sl = wave_slots(p, c.g, c.b, c.t - p.shift);
  Off off;
  off.init(0);

  // lane (li, hl) writes the lse of query 32 hl + li
  float* const lse_q = kLse ? p.lse + slot_vec_offset(p, c.gbh, c.t, 0) + lane : nullptr;
  if (kLse) {  // invalid slots: -inf (before any copy, so the copy counts below stay exact)
    for (int k = 0; k < p.K; ++k)
      if (!((sl.valid >> k) & 1u)) lse_q[k * kChunk] = -__builtin_inff();
  }
  uint32_t rem = sl.valid;
  int k = rem ? __builtin_ctz(rem) : -1;
  rem &= rem - 1;
  auto tile_of = [&](const void* base, int slot) {
    return kv_tile<T>(base, p, c.b, c.h, __builtin_amdgcn_readlane(sl.j, slot));
  };
  if (k >= 0) {
    off.copy(tile_of(p.k, k), Ks, 0);
    off.copy(tile_of(p.v, k), Vs, 0);
  }

  f32x16_t oacc[2][2] = {{zero16(), zero16()}, {zero16(), zero16()}};
  const float c2 = p.attn_scale * kLog2e;
  bool first = true;
  while (k >= 0) {  // wave-uniform
    const int kn = rem ? __builtin_ctz(rem) : -1;
    rem &= rem - 1;
    if (first) wait_vm_outstanding<kC>();  // K(k) landed: only V(k) may be in flight
    else wait_vm_outstanding<kC + (kLse ? 1 : 0)>();  // only the last lse store and V(k)
    first = false;
    Frag<T> kf[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int s = 0; s < 4; ++s) kf[tt][s] = off.kfrag(Ks, tt, s);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // K(k) in registers: the buffer is free
    if (kn >= 0) off.copy(tile_of(p.k, kn), Ks, 0);

    f32x16_t sacc[2][2];
#pragma unroll
    for (int qh = 0; qh < 2; ++qh)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        sacc[qh][tt] = zero16();
#pragma unroll
        for (int s = 0; s < 4; ++s) sacc[qh][tt] = mma(kf[tt][s], qf[qh][s], sacc[qh][tt]);
      }
    const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sl.w), k));
    float lse_v[2];
    Frag<T> pf[2][4];
    // softmax of half qh -> its P^T operand (scaled by w / l); written per half so that the P V
    // product of half 0 and the softmax of half 1 are independent work side by side
    auto half_softmax = [&](int qh) {
      float l;
      const float mx = tile_softmax(sacc[qh], c2, l);
      lse_v[qh] = mx * p.attn_scale + __builtin_amdgcn_logf(l) * kLn2f;
      const float f = wk * __builtin_amdgcn_rcpf(l);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = sacc[qh][s >> 1][8 * (s & 1) + e] * f;
        pf[qh][s].set(x);
      }
    };
    half_softmax(0);

    if (kn >= 0) wait_vm_outstanding<kC>();  // V(k) landed: K(kn) may not have
    else wait_vm_outstanding<0>();
    Frag<T> vf[4][2];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) vf[s][dt] = off.vfrag(Vs, s, dt);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // V(k) in registers: the buffer is free
    if (kn >= 0) off.copy(tile_of(p.v, kn), Vs, 0);
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int s = 0; s < 4; ++s) oacc[0][dt] = mma(vf[s][dt], pf[0][s], oacc[0][dt]);
    half_softmax(1);
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int s = 0; s < 4; ++s) oacc[1][dt] = mma(vf[s][dt], pf[1][s], oacc[1][dt]);
    if (kLse) lse_q[k * kChunk] = hl ? lse_v[1] : lse_v[0];
    k = kn;
  }

#pragma unroll
  for (int qh = 0; qh < 2; ++qh) {
    T* o = static_cast<T*>(p.o) + (qrow0 + 32 * qh + li) * kDim;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        store4(o + 32 * dt + 8 * a + 4 * hl, oacc[qh][dt][4 * a], oacc[qh][dt][4 * a + 1],
               oacc[qh][dt][4 * a + 2], oacc[qh][dt][4 * a + 3]);
  }
}

// ------------------------------------------------------------------ forward, few queries
// A decode-style step (one query chunk against a long history) gives too few query tiles to
// occupy the chip, and the main forward would walk its K slots one after another, paying the HBM
// latency of each retrieved tile in turn.  Here one workgroup owns 32 queries (half a chunk) of one
// (group, batch row, head, chunk) and each of its kW waves owns one slot (slots w, w + kW, ...):
// every wave reads its slot's index and the row's scores itself, starts its own tile copies at
// once, and computes alone on its LDS region; the waves' weighted partial outputs are summed in
// wave order through LDS at the end (the same sum as the main forward, in another rounding order).
template <typename T>
struct Wide {
  static constexpr int kW = sizeof(T) == 2 ? 8 : 4;  // waves; LDS holds one K and V tile per wave
  static constexpr int kThreads = 64 * kW;
};

// The slots of one retrieval row: lane s < K holds slot s's chunk and score (-1 and -inf on the
// other lanes, and on every lane without a row).  One round trip for both.
struct RowSlots {
  int32_t j;
  float sc;
};

__device__ __forceinline__ RowSlots load_row_slots(const AttendParams& p, int64_t rowbase, int lane, bool has_row) {
  RowSlots r{-1, -__builtin_inff()};
  if (has_row && lane < p.K) {
    r.j = p.idx[rowbase + lane];
    r.sc = p.score[rowbase + lane];
  }
  // both have landed here: a later wait for them would be placed after the caller's untracked
  // tile copies and wait for those as well
  asm volatile("" ::"v"(r.j), "v"(r.sc));
  return r;
}

// Chunk of slot k (k wave-uniform) and whether it is valid.
__device__ __forceinline__ int32_t row_slot_chunk(const AttendParams& p, const RowSlots& r, int k, bool& valid) {
  const int32_t j = __builtin_amdgcn_readlane(r.j, k);
  valid = j >= 0 && j < p.n_kv;
  return j;
}

// Fusion weight of slot k of the row, computed by every lane of the wave (the softmax over the
// valid slots is reduced across lanes 0..15), and the row's valid-slot mask.  Callers issue the
// slot's tile loads first, so that this runs while they are in flight.
__device__ __forceinline__ float row_slot_weight(const AttendParams& p, const RowSlots& r, int k,
                                                 uint32_t& valid_mask) {
  const bool v = r.j >= 0 && r.j < p.n_kv;
  valid_mask = static_cast<uint32_t>(__ballot(v));
  float mx = v ? r.sc : -__builtin_inff();
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 16));  // K <= 16 lanes
  const float e = v ? expf(r.sc - mx) : 0.f;
  float sum = e;
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 16);
  return __shfl(e, k, 64) / __shfl(sum, 0, 64);  // lanes 0..15 hold the row
}

template <typename T>
__global__ __launch_bounds__(Wide<T>::kThreads) void attend_fwd_wide_kernel(AttendParams p) {
  using TL = Tile<T>;
  constexpr int kW = Wide<T>::kW;
  constexpr int kRegion = 2 * TL::kBytes;  // one wave's K and V tiles, later its fp32 partial output
  static_assert(kRegion >= 32 * kDim * 4, "partial output must fit in a wave's region");
  __shared__ __align__(1024) char buf[kW * kRegion];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, hl = lane >> 5;
  // block -> (query half, tile); the tile order is the main forward's
  const int64_t lid = blockIdx.x;
  const int half = static_cast<int>(lid & 1);
  const int64_t tile = lid >> 1;
  QTileCoord c;
  c.t = tile % p.n_q;
  int64_t rest = tile / p.n_q;
  c.g = static_cast<int>(rest % p.G);
  rest /= p.G;
  c.h = static_cast<int>(rest % p.H);
  c.b = static_cast<int>(rest / p.H);
  c.gbh = (static_cast<int64_t>(c.g) * p.B + c.b) * p.H + c.h;
  const int64_t Lq = p.n_q * kChunk;
  const int64_t qrow0 = c.gbh * Lq + c.t * kChunk + 32 * half;
  char* region = buf + wave * kRegion;

  const int64_t row = c.t - p.shift;
  const bool has_row = row >= 0;
  const int64_t rowbase = ((static_cast<int64_t>(c.g) * p.B + c.b) * p.n_q + (has_row ? row : 0)) * p.K;

  Frag<T> qf[4];
  const T* q = static_cast<const T*>(p.q) + (qrow0 + li) * kDim;
#pragma unroll
  for (int s = 0; s < 4; ++s) qf[s].load(q + 16 * s + 8 * hl);

  f32x16_t oacc[2] = {zero16(), zero16()};
  const float c2 = p.attn_scale * kLog2e;
  const RowSlots rs = load_row_slots(p, rowbase, lane, has_row);
  for (int k = wave; k < p.K; k += kW) {  // wave-uniform
    bool valid;
    const int32_t j = row_slot_chunk(p, rs, k, valid);
    float* lse_k = p.lse ? p.lse + slot_vec_offset(p, c.gbh, c.t, k) + 32 * half : nullptr;
    if (!valid) {
      if (lse_k && lane < 32) lse_k[lane] = -__builtin_inff();
      continue;
    }
    tile_load_async<T, 1>(kv_tile<T>(p.k, p, c.b, c.h, j), region, 0);
    tile_load_async<T, 1>(kv_tile<T>(p.v, p, c.b, c.h, j), region + TL::kBytes, 0);
    uint32_t vmask;
    float w = row_slot_weight(p, rs, k, vmask);  // while the tiles are in flight
    asm volatile("" : "+v"(w));  // (computed here, not sunk past the wait below)
    wait_async_copies();  // this wave's own copies: visible to it once they have landed
    const char* Ks = region;
    const char* Vs = region + TL::kBytes;
    f32x16_t sacc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      sacc[tt] = zero16();
#pragma unroll
      for (int s = 0; s < 4; ++s) sacc[tt] = mma(row_frag<T>(Ks, 32 * tt + pi_row(li), 16 * s + 8 * hl), qf[s], sacc[tt]);
    }
    float mx = fmaxf(sacc[0][0], sacc[1][0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(sacc[0][r], sacc[1][r]));
    mx = xor32_max(mx);
    const float bias = -mx * c2;
    float l = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(__builtin_fmaf(sacc[tt][r], c2, bias));
        sacc[tt][r] = e;
        l += e;
      }
    l = xor32_sum(l);
    if (lse_k && hl == 0) lse_k[li] = mx * p.attn_scale + __builtin_amdgcn_logf(l) * kLn2f;
    const float f = w / l;
    Frag<T> pf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = sacc[s >> 1][8 * (s & 1) + e] * f;
      pf[s].set(x);
    }
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        oacc[dt] = mma(col_frag<T>(Vs, 32 * (s >> 1) + 16 * hl + 8 * (s & 1), 32 * dt), pf[s], oacc[dt]);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // tile reads done before the next refill
  }

  // Partial output of this wave, fp32 [32 queries][64], 16-byte chunk ch of query row qq stored at
  // chunk position ch ^ (qq & 15) (conflict-free for these writes and for the reads below).
  __syncthreads();  // (every wave is past its tile reads)
  float* part = reinterpret_cast<float*>(region);
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int ch = 8 * dt + 2 * a + hl;
      *reinterpret_cast<f32x4_t*>(part + li * kDim + 4 * (ch ^ (li & 15))) =
          f32x4_t{oacc[dt][4 * a], oacc[dt][4 * a + 1], oacc[dt][4 * a + 2], oacc[dt][4 * a + 3]};
    }
  __syncthreads();
  T* o = static_cast<T*>(p.o) + qrow0 * kDim;
  for (int e = tid; e < 32 * kDim / 4; e += Wide<T>::kThreads) {
    const int qq = e >> 4, ch = e & 15;
    const int off = qq * kDim + 4 * (ch ^ (qq & 15));
    f32x4_t acc = *reinterpret_cast<const f32x4_t*>(reinterpret_cast<const float*>(buf) + off);
#pragma unroll
    for (int w2 = 1; w2 < kW; ++w2) {
      const f32x4_t x = *reinterpret_cast<const f32x4_t*>(reinterpret_cast<const float*>(buf + w2 * kRegion) + off);
      acc = f32x4_t{acc[0] + x[0], acc[1] + x[1], acc[2] + x[2], acc[3] + x[3]};
    }
    store4(o + qq * kDim + 4 * ch, acc[0], acc[1], acc[2], acc[3]);
  }
}

// ------------------------------------------------------------- sliding-window attention
// Local causal attention beside GCA [Notes, Loss / training strategy: sliding-window
// self-attention with W = 512]: token i attends to tokens max(0, i - W + 1) .. i under one softmax.
// With W = 64 m, query tile t meets key tiles t - m .. t: in tile t - m only keys above the query's
// position inside the tile are in the window (its lower edge), in tile t only keys at or below it
// (causality), the tiles between are whole.  In the S^T accumulators lane (li, hl) holds
// sacc[qh][tt][r] = S[query 32 qh + li][key 32 tt + 16 hl + r], so the masks are per-register
// comparisons.  Masked scores are -inf; a query whose keys in a tile are all masked keeps its
// running maximum (the guards below avoid -inf - -inf).
// (batch row and head, tile) of a sliding-window workgroup; B H n_c < 2^31 blocks (checked on
// the host), so 32-bit divisions suffice.
__device__ __forceinline__ void window_tile(const SwParams& p, int64_t& bh, int64_t& t) {
  const uint32_t lid = static_cast<uint32_t>(xcd_logical_block(blockIdx.x, gridDim.x));
  const uint32_t n = static_cast<uint32_t>(p.n_c);
  const uint32_t q = lid / n;
  bh = q;
  t = lid - q * n;
}

// Masks the 16 elements of one accumulator run in an edge tile of the window: per lane, the
// elements r < t keep their value and the others become -inf when lo_keeps, and the other way
// round otherwise (lo_keeps wave-uniform).  One comparison and one select per element.  t is
// opaque, so the comparisons are made here on every call: hoisted out of the caller's loop, the
// lane masks they give outgrow the scalar registers, and the compiler then parks them in vector
// lanes and turns every select into a branch.
template <bool kOpaque = true>
__device__ __forceinline__ void mask_run(f32x16_t& x, int t, bool lo_keeps) {
  if (kOpaque) asm volatile("" : "+v"(t));
#pragma unroll
  for (int r = 0; r < 16; ++r) x[r] = (r < t) == lo_keeps ? x[r] : -__builtin_inff();
}

// Edge tiles of a query-major pass (the diagonal tile or, exclusively since W >= 64, the tile at
// the window's lower edge): sacc[qh][tt][r] = S[query 32 qh + li][key 32 tt + 16 hl + r].  The key
// lies after the query (masked in the diagonal tile) exactly when r >= t = 32 (qh - tt) + li -
// 16 hl + 1, and at or before it (masked at the lower edge) when r < t.
__device__ __forceinline__ void sw_mask(f32x16_t (&sacc)[2][2], bool diagonal) {
  const int lane = threadIdx.x & 63, li = lane & 31, hl = lane >> 5;
#pragma unroll
  for (int qh = 0; qh < 2; ++qh)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) mask_run<false>(sacc[qh][tt], 32 * (qh - tt) + li - 16 * hl + 1, diagonal);
}

// The same for query-major accumulators of one 32-query half:
// sacc[tt][r] = S[query query_base + li][key 32 tt + 16 hl + r].
__device__ __forceinline__ void sw_mask_keys_major(f32x16_t (&sacc)[2], int query_base, bool diagonal) {
  const int lane = threadIdx.x & 63, li = lane & 31, hl = lane >> 5;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) mask_run(sacc[tt], query_base + li - 32 * tt - 16 * hl + 1, diagonal);
}

// One wave per query tile, as the bf16 GCA forward: K and V tiles stream through single LDS
// buffers with the same counted-copy pipeline, and the softmax is online (running maximum and sum
// per query; the output accumulators are rescaled when the maximum grows).
__global__ __launch_bounds__(64) void sw_fwd_kernel(SwParams p) {
  using T = bf16_t;
  using TL = Tile<T>;
  using Off = TileOffsets<T, 1>;
  constexpr int kC = Off::kCopies;
  __shared__ __align__(1024) char Ks[TL::kBytes];
  __shared__ __align__(1024) char Vs[TL::kBytes];

  const int lane = threadIdx.x, li = lane & 31, hl = lane >> 5;
  int64_t bh, t;
  window_tile(p, bh, t);
  const int64_t row0 = bh * p.n_c * kChunk;  // first token of this (batch row, head)
  const int64_t qrow0 = row0 + t * kChunk;

  Frag<T> qf[2][4];
#pragma unroll
  for (int qh = 0; qh < 2; ++qh) {
    const T* q = static_cast<const T*>(p.q) + (qrow0 + 32 * qh + li) * kDim;
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[qh][s].load(q + 16 * s + 8 * hl);
  }
  Off off;
  off.init(0);
  const int64_t kt0 = t - p.m > 0 ? t - p.m : 0;
  auto tile = [&](const void* base, int64_t kt) {
    return static_cast<const T*>(base) + (row0 + kt * kChunk) * kDim;
  };
  off.copy(tile(p.k, kt0), Ks, 0);
  off.copy(tile(p.v, kt0), Vs, 0);
  // The loads above are pinned here, before the loop, so that the compiler waits for them once:
  // left to their first use in the loop, its vmcnt waits would run in every iteration and also
  // wait for the untracked prefetch copies in flight.  The first K and V tiles are needed at
  // once anyway.
#pragma unroll
  for (int qh = 0; qh < 2; ++qh)
#pragma unroll
    for (int s = 0; s < 4; ++s) pin_in_registers(qf[qh][s]);

  f32x16_t oacc[2][2] = {{zero16(), zero16()}, {zero16(), zero16()}};
  float m_run[2] = {-__builtin_inff(), -__builtin_inff()}, l_run[2] = {0.f, 0.f};
  const float c2 = p.attn_scale * kLog2e;
  for (int64_t kt = kt0; kt <= t; ++kt) {  // wave-uniform
    const bool more = kt < t;
    wait_vm_outstanding<kC>();  // K(kt) landed: only V(kt) may be in flight
    Frag<T> kf[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int s = 0; s < 4; ++s) kf[tt][s] = off.kfrag(Ks, tt, s);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // K(kt) in registers: the buffer is free
    if (more) off.copy(tile(p.k, kt + 1), Ks, 0);

    f32x16_t sacc[2][2];
#pragma unroll
    for (int qh = 0; qh < 2; ++qh)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        sacc[qh][tt] = zero16();
#pragma unroll
        for (int s = 0; s < 4; ++s) sacc[qh][tt] = mma(kf[tt][s], qf[qh][s], sacc[qh][tt]);
      }
    const bool lower_edge = kt == t - p.m, diagonal = kt == t;
    if (lower_edge || diagonal) sw_mask(sacc, diagonal);
    Frag<T> pf[2][4];
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[qh][tt][r]);
      mx = xor32_max(mx) * c2;  // log2 units
      // The running maximum moves only when a new score exceeds it by more than kLazy (or on the
      // first keys): otherwise the exps run against the stale maximum, stay below 2^kLazy, and the
      // rescale of the accumulators is skipped (a wave-uniform decision).
      constexpr float kLazy = 8.f;
      const bool grow = __ballot(mx > m_run[qh] + kLazy) != 0;
      const float m_new = grow ? fmaxf(m_run[qh], mx) : m_run[qh];
      const bool none = m_new == -__builtin_inff();  // no key of the window seen yet
      const float alpha = none ? 1.f : fast_exp2(m_run[qh] - m_new);
      const float bias = none ? 0.f : -m_new;
      float l = 0.f;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sacc[qh][tt][r] = fast_exp2(__builtin_fmaf(sacc[qh][tt][r], c2, bias));
          l += sacc[qh][tt][r];
        }
      l_run[qh] = l_run[qh] * alpha + xor32_sum(l);
      m_run[qh] = m_new;
      if (grow) {
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[qh][dt][r] *= alpha;
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = sacc[qh][s >> 1][8 * (s & 1) + e];
        pf[qh][s].set(x);
      }
    }
    if (more) wait_vm_outstanding<kC>();  // V(kt) landed: K(kt + 1) may not have
    else wait_vm_outstanding<0>();
    Frag<T> vf[4][2];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) vf[s][dt] = off.vfrag(Vs, s, dt);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // V(kt) in registers: the buffer is free
    if (more) off.copy(tile(p.v, kt + 1), Vs, 0);
#pragma unroll
    for (int qh = 0; qh < 2; ++qh)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int s = 0; s < 4; ++s) oacc[qh][dt] = mma(vf[s][dt], pf[qh][s], oacc[qh][dt]);
  }

#pragma unroll
  for (int qh = 0; qh < 2; ++qh) {
    const float f = __builtin_amdgcn_rcpf(l_run[qh]);
    T* o = static_cast<T*>(p.o) + (qrow0 + 32 * qh + li) * kDim;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        store4(o + 32 * dt + 8 * a + 4 * hl, f * oacc[qh][dt][4 * a], f * oacc[qh][dt][4 * a + 1],
               f * oacc[qh][dt][4 * a + 2], f * oacc[qh][dt][4 * a + 3]);
    if (p.lse && hl == qh)  // lane (li, hl) writes query 32 hl + li
      p.lse[qrow0 + 32 * qh + li] = m_run[qh] * kLn2f + __builtin_amdgcn_logf(l_run[qh]) * kLn2f;
  }
}

// Two waves of 32 queries per query tile, for fp32 tiles (the one-wave forward's registers hold
// bf16 fragments only): the pipeline of the two-wave GCA forward, single K and V buffers
// published by barriers, with the same online softmax and edge masks.
template <typename T>
__global__ __launch_bounds__(kThreads) void sw_fwd2_kernel(SwParams p) {
  using TL = Tile<T>;
  using Off = TileOffsets<T, kWaves>;
  constexpr int kC = Off::kCopies;
  __shared__ __align__(1024) char Ks[TL::kBytes];
  __shared__ __align__(1024) char Vs[TL::kBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, hl = lane >> 5;
  int64_t bh, t;
  window_tile(p, bh, t);
  const int64_t row0 = bh * p.n_c * kChunk;
  const int64_t qrow0 = row0 + t * kChunk;
  const int my_q = 32 * wave + li;

  Frag<T> qf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) qf[s].load(static_cast<const T*>(p.q) + (qrow0 + my_q) * kDim + 16 * s + 8 * hl);
  Off off;
  off.init(wave);
  const int64_t kt0 = t - p.m > 0 ? t - p.m : 0;
  auto tile = [&](const void* base, int64_t kt) {
    return static_cast<const T*>(base) + (row0 + kt * kChunk) * kDim;
  };
  off.copy(tile(p.k, kt0), Ks, wave);
  off.copy(tile(p.v, kt0), Vs, wave);
  barrier_copies_landed<kC>();  // K(kt0) landed and visible; V(kt0) may still be in flight
  // The query fragments are pinned here, before the loop, so that the compiler waits for them
  // once (left to their first use in the loop, its vmcnt waits would run in every iteration and
  // also wait for the prefetch copies in flight).
#pragma unroll
  for (int s = 0; s < 4; ++s) pin_in_registers(qf[s]);

  f32x16_t oacc[2] = {zero16(), zero16()};
  float m_run = -__builtin_inff(), l_run = 0.f;
  const float c2 = p.attn_scale * kLog2e;
  for (int64_t kt = kt0; kt <= t; ++kt) {
    const bool more = kt < t;
    f32x16_t sacc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      sacc[tt] = zero16();
#pragma unroll
      for (int s = 0; s < 4; ++s) sacc[tt] = mma(off.kfrag(Ks, tt, s), qf[s], sacc[tt]);
    }
    barrier_lds_reads_done();  // every wave has read K(kt)
    if (more) off.copy(tile(p.k, kt + 1), Ks, wave);
    const bool lower_edge = kt == t - p.m, diagonal = kt == t;
    if (lower_edge || diagonal) sw_mask_keys_major(sacc, 32 * wave, diagonal);
    float mx = -__builtin_inff();
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[tt][r]);
    mx = xor32_max(mx) * c2;
    constexpr float kLazy = 8.f;
    const bool grow = __ballot(mx > m_run + kLazy) != 0;
    const float m_new = grow ? fmaxf(m_run, mx) : m_run;
    const bool none = m_new == -__builtin_inff();
    const float alpha = none ? 1.f : fast_exp2(m_run - m_new);
    const float bias = none ? 0.f : -m_new;
    float l = 0.f;
    Frag<T> pf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = fast_exp2(__builtin_fmaf(sacc[s >> 1][8 * (s & 1) + e], c2, bias));
        l += x[e];
      }
      pf[s].set(x);
    }
    l_run = l_run * alpha + xor32_sum(l);
    m_run = m_new;
    if (grow) {
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
    }
    if (more) barrier_copies_landed<kC>();  // V(kt) landed and visible (K(kt + 1) may be in flight)
    else barrier_copies_landed<0>();
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int s = 0; s < 4; ++s) oacc[dt] = mma(off.vfrag(Vs, s, dt), pf[s], oacc[dt]);
    if (more) {
      barrier_lds_reads_done();  // every wave has read V(kt)
      off.copy(tile(p.v, kt + 1), Vs, wave);
      barrier_copies_landed<kC>();  // K(kt + 1) landed (V(kt + 1) may not)
    }
  }
  const float f = __builtin_amdgcn_rcpf(l_run);
  T* o = static_cast<T*>(p.o) + (qrow0 + my_q) * kDim;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a)
      store4(o + 32 * dt + 8 * a + 4 * hl, f * oacc[dt][4 * a], f * oacc[dt][4 * a + 1], f * oacc[dt][4 * a + 2],
             f * oacc[dt][4 * a + 3]);
  if (p.lse && hl == 0) p.lse[qrow0 + my_q] = m_run * kLn2f + __builtin_amdgcn_logf(l_run) * kLn2f;
}

// ------------------------------------------------------------- token-level decode
// While the tokens of a query chunk are generated one at a time, each new token attends to the
// chunks retrieved once for the chunk's row: one retrieval serves all S tokens of the chunk.  For
// one to a few query tokens the products are matrix-vector sized, so they run on the vector units:
// one workgroup per (group, batch row, head), one wave per retrieval slot (slots k, k + 8, ...),
// lane u holding key u's row for the scores and lane d holding column d of V for P V.  Each slot's
// output, already scaled by w_k / l_k, goes to LDS; the fused output sums the valid slots in slot
// order.  Tokens are processed kDecodeBatch at a time.
constexpr int kDecodeWaves = 8;
constexpr int kDecodeBatch = 4;

template <typename T>
__global__ __launch_bounds__(64 * kDecodeWaves) void decode_tokens_kernel(AttendParams p, int32_t n_tok) {
  __shared__ float q_s[kDecodeBatch][kDim];
  __shared__ float p_s[kDecodeWaves][kChunk];
  __shared__ float o_s[kMaxTopk][kDecodeBatch][kDim];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t gbh = blockIdx.x;  // (g B + b) H + h
  const int h = static_cast<int>(gbh % p.H);
  const int64_t gb = gbh / p.H;
  const int b = static_cast<int>(gb % p.B);
  const int64_t row = -static_cast<int64_t>(p.shift);  // the call's single query chunk is chunk 0
  const bool has_row = row >= 0;
  const int64_t rowbase = (gb * p.n_q + (has_row ? row : 0)) * p.K;
  const T* q = static_cast<const T*>(p.q) + gbh * static_cast<int64_t>(n_tok) * kDim;
  T* o = static_cast<T*>(p.o) + gbh * static_cast<int64_t>(n_tok) * kDim;
  const int rounds = (p.K + kDecodeWaves - 1) / kDecodeWaves;
  const RowSlots rs = load_row_slots(p, rowbase, lane, has_row);
  uint32_t vmask = 0;  // valid slots of the row (wave-uniform, the same in every wave)
  if (has_row) (void)row_slot_weight(p, rs, 0, vmask);

  for (int t0 = 0; t0 < n_tok; t0 += kDecodeBatch) {  // uniform over the workgroup
    const int nb = n_tok - t0 < kDecodeBatch ? n_tok - t0 : kDecodeBatch;
    if (tid < kDecodeBatch * kDim) {
      const int t = tid / kDim, d = tid % kDim;
      q_s[t][d] = t < nb ? to_f32(q[(t0 + t) * kDim + d]) : 0.f;
    }
    __syncthreads();
    for (int rd = 0; rd < rounds; ++rd) {  // uniform
      const int k = rd * kDecodeWaves + wave;
      bool valid = false;
      int32_t j = -1;
      if (k < p.K) j = row_slot_chunk(p, rs, k, valid);
      if (!valid) continue;  // wave-uniform
      const T* kt = kv_tile<T>(p.k, p, b, h, j);
      const T* vt = kv_tile<T>(p.v, p, b, h, j);
      float krow[kDim], vcol[kChunk];
#pragma unroll
      for (int d = 0; d < kDim; ++d) krow[d] = to_f32(kt[lane * kDim + d]);
#pragma unroll
      for (int u = 0; u < kChunk; ++u) vcol[u] = to_f32(vt[u * kDim + lane]);
      uint32_t vm_k;
      float w = row_slot_weight(p, rs, k, vm_k);  // while the tile loads are in flight
      asm volatile("" : "+v"(w));
      for (int t = 0; t < nb; ++t) {
        float z = 0.f;
#pragma unroll
        for (int d = 0; d < kDim; ++d) z = __builtin_fmaf(q_s[t][d], krow[d], z);
        z *= p.attn_scale;
        float mx = z;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
        const float e = expf(z - mx);
        float l = e;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off, 64);
        p_s[wave][lane] = e * (w / l);
        __builtin_amdgcn_wave_barrier();
        float acc = 0.f;
#pragma unroll
        for (int u = 0; u < kChunk; ++u) acc = __builtin_fmaf(p_s[wave][u], vcol[u], acc);
        o_s[k][t][lane] = acc;
        __builtin_amdgcn_wave_barrier();  // p_s is rewritten for the next token
      }
    }
    __syncthreads();
    if (tid < kDecodeBatch * kDim) {
      const int t = tid / kDim, d = tid % kDim;
      if (t < nb) {
        float acc = 0.f;
        for (int k = 0; k < p.K; ++k)
          if ((vmask >> k) & 1u) acc += o_s[k][t][d];
        from_f32(o + (t0 + t) * kDim + d, acc);
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------- backward, query-major (dQ)
// Sum over the 32 queries of a wave of a per-query value (lanes l and l ^ 32 hold the same
// query): DPP steps within each 16-lane row, then the row pair.  Fixed order: deterministic.
__device__ __forceinline__ float sum_queries32(float x) {
  auto dpp = [](float v, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl)::value, 0xf, 0xf, true));
  };
  x += dpp(x, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
  x += dpp(x, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
  x += dpp(x, std::integral_constant<int, 0x141>{});  // row_half_mirror
  x += dpp(x, std::integral_constant<int, 0x140>{});  // row_mirror
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One workgroup of two waves per query tile walks the tile's slots.  Per slot: S = K Q^T and
// dP' = V dO^T from row reads, P = exp(z - lse), e = sum_u P dP', dz = P (w dP' - w e), and
// dQ^T += K^T dz^T from transposing reads of the same K tile.  K is double-buffered (the next
// slot's K copy starts with the slot); V is read only at the start of a slot, so the next V is
// copied into the single V buffer as soon as both waves have read it.
template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_query_kernel(AttendParams p) {
  // the split-list counters of the key-major pass that follows start at zero
  if (blockIdx.x == 0 && threadIdx.x == 0 && p.long_ctl != nullptr) *p.long_ctl = 0;
  using TL = Tile<T>;
  using Off = TileOffsets<T, kWaves>;
  __shared__ __align__(1024) char Ka[TL::kBytes];
  __shared__ __align__(1024) char Kb[TL::kBytes];
  __shared__ __align__(1024) char Vs[TL::kBytes];
  __shared__ float dw_s[2][kMaxTopk];
  __shared__ SlotTable st;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, hl = lane >> 5;
  const QTileCoord c = query_tile_coord(p);
  const int64_t Lq = p.n_q * kChunk;
  const int64_t qrow0 = c.gbh * Lq + c.t * kChunk;
  const int my_q = 32 * wave + li;
  const int64_t row = c.t - p.shift;

  if (tid < 2 * kMaxTopk) dw_s[tid / kMaxTopk][tid % kMaxTopk] = 0.f;
  Frag<T> qf[4], df[4];
  const T* q = static_cast<const T*>(p.q) + (qrow0 + my_q) * kDim;
  const T* dout = static_cast<const T*>(p.dout) + (qrow0 + my_q) * kDim;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    qf[s].load(q + 16 * s + 8 * hl);
    df[s].load(dout + 16 * s + 8 * hl);
  }
  if (wave == 0) fill_slot_table(st, p, c.g, c.b, row);  // its loads beside the query's and dO's
  Off off;
  off.init(wave);
  __syncthreads();

  const int nslots = st.n;
  if (c.h == 0 && row >= 0 && tid < p.K)
    p.wts[((static_cast<int64_t>(c.g) * p.B + c.b) * p.n_q + row) * p.K + tid] = st.w_all[tid];
  const float* lse_q = p.lse_in + slot_vec_offset(p, c.gbh, c.t, 0) + my_q;
  float* delta_q = p.delta + 2 * slot_vec_offset(p, c.gbh, c.t, 0) + 64 * hl + my_q;
  auto chunk_of = [&](int n) { return __builtin_amdgcn_readfirstlane(st.j[n]); };
  auto slot_of = [&](int n) { return __builtin_amdgcn_readfirstlane(st.slot[n]); };
  float lse_cur = 0.f;
  if (nslots > 0) {
    const int32_t j = chunk_of(0);
    off.copy(kv_tile<T>(p.k, p, c.b, c.h, j), Ka, wave);
    off.copy(kv_tile<T>(p.v, p, c.b, c.h, j), Vs, wave);
    lse_cur = lse_q[slot_of(0) * kChunk];
    barrier_copies_landed<0>();
  }
  // Every load above has landed (the barrier's own wait).  Pinning the values here lets the
  // compiler place its waits for them now, where they cost nothing; left to their first use in
  // the slot loop, its vmcnt waits would also wait for the untracked prefetch copies.
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    pin_in_registers(qf[s]);
    pin_in_registers(df[s]);
  }
  asm volatile("" : "+v"(lse_cur));

  f32x16_t dqacc[2] = {zero16(), zero16()};
  const float c2 = p.attn_scale * kLog2e;
  // unrolled twice below, so that both K buffers are fixed LDS bases (immediate offsets)
  auto slot_step = [&](int n, char* const Kc, char* const Kn) {
    const bool more = n + 1 < nslots;
    const int slot = slot_of(n);
    const float w = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(st.w[n])));
    float lse_nxt = 0.f;
    if (more) {  // the other K buffer was released by the previous slot's closing barrier
      off.copy(kv_tile<T>(p.k, p, c.b, c.h, chunk_of(n + 1)), Kn, wave);
      lse_nxt = lse_q[slot_of(n + 1) * kChunk];
    }
    f32x16_t sacc[2], pacc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      sacc[tt] = zero16();
      pacc[tt] = zero16();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        sacc[tt] = mma(off.kfrag(Kc, tt, s), qf[s], sacc[tt]);
        pacc[tt] = mma(off.kfrag(Vs, tt, s), df[s], pacc[tt]);
      }
    }
    barrier_lds_reads_done();  // every wave has read V(n)
    if (more) off.copy(kv_tile<T>(p.v, p, c.b, c.h, chunk_of(n + 1)), Vs, wave);

    // P = exp(z - lse); e = sum_u P dP' = <dO, O_slot>; dz = w P (dP' - e)
    const float bias = -lse_cur * kLog2e;
    float e0 = 0.f, e1 = 0.f;  // two interleaved chains (the key halves)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sacc[0][r] = fast_exp2(__builtin_fmaf(sacc[0][r], c2, bias));
      sacc[1][r] = fast_exp2(__builtin_fmaf(sacc[1][r], c2, bias));
      e0 = __builtin_fmaf(sacc[0][r], pacc[0][r], e0);
      e1 = __builtin_fmaf(sacc[1][r], pacc[1][r], e1);
    }
    const float e = xor32_sum(e0 + e1);
    // for the key-major pass: P_w = exp2(z log2e + bias) with bias = log2 w - lse log2 e, and e
    delta_q[2 * slot * kChunk] = hl ? -e : __builtin_amdgcn_logf(w) + bias;
    const float es = sum_queries32(e);
    if (lane == 0) dw_s[wave][slot] = es;
    const float we = -w * e;
    Frag<T> zf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float x[8];
#pragma unroll
      for (int ee = 0; ee < 8; ++ee) {
        const int tt = s >> 1, r = 8 * (s & 1) + ee;
        x[ee] = sacc[tt][r] * __builtin_fmaf(w, pacc[tt][r], we);
      }
      zf[s].set(x);
    }
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int s = 0; s < 4; ++s) dqacc[dt] = mma(off.vfrag(Kc, s, dt), zf[s], dqacc[dt]);
    // K(n+1), the lse and V(n+1) landed (the delta store may not have): the next slot can start;
    // every wave has also read K(n), whose buffer the next slot refills
    if (more) barrier_copies_landed_reads_done<1>();
    asm volatile("" : "+v"(lse_nxt));  // landed: the compiler's wait for it goes here, not later
    lse_cur = lse_nxt;
  };
  for (int n = 0; n < nslots; n += 2) {
    slot_step(n, Ka, Kb);
    if (n + 1 < nslots) slot_step(n + 1, Kb, Ka);
  }

  T* dq = static_cast<T*>(p.dq) + (qrow0 + my_q) * kDim;
  const float sc = p.attn_scale;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a)
      store4(dq + 32 * dt + 8 * a + 4 * hl, sc * dqacc[dt][4 * a], sc * dqacc[dt][4 * a + 1],
             sc * dqacc[dt][4 * a + 2], sc * dqacc[dt][4 * a + 3]);
  __syncthreads();
  if (row >= 0 && tid < p.K) {
    const int64_t o = (((static_cast<int64_t>(c.g) * p.B + c.b) * p.n_q + row) * p.H + c.h) * p.K + tid;
    p.dw_part[o] = dw_s[0][tid] + dw_s[1][tid];
  }
}

// ------------------------------------------------------------- sliding-window backward
// dS = P (dP - D) with P = exp(z - lse) and D = <dO, O> per query (one softmax over the window),
// then dQ = scale dS K query-major and dK = scale dS^T Q, dV = P^T dO key-major, without atomics.
// The query-major pass walks key tiles t - m .. t exactly as the GCA query-major pass walks its
// slots (double-buffered K, single V, two waves of 32 queries); it first computes D from the
// stored output and writes -lse log2 e and -D per query (per query tile: 64 of each), which the
// key-major pass reads as the GCA key-major pass reads its biases and -e.  Masked scores become
// -inf before the exp, so their P and dS are exactly 0.

// <a, b> over one lane's eight fragment elements
__device__ __forceinline__ float frag_dot(const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
  float acc = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t x = a.v[w], y = b.v[w];
    acc = __builtin_fmaf(__uint_as_float(x << 16), __uint_as_float(y << 16), acc);
    acc = __builtin_fmaf(__uint_as_float(x & 0xffff0000u), __uint_as_float(y & 0xffff0000u), acc);
  }
  return acc;
}
__device__ __forceinline__ float frag_dot(const Frag<float>& a, const Frag<float>& b) {
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = __builtin_fmaf(a.v0[i], b.v0[i], acc);
    acc = __builtin_fmaf(a.v1[i], b.v1[i], acc);
  }
  return acc;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void sw_bwd_query_kernel(SwParams p) {
  using TL = Tile<T>;
  using Off = TileOffsets<T, kWaves>;
  __shared__ __align__(1024) char Ka[TL::kBytes];
  __shared__ __align__(1024) char Kb[TL::kBytes];
  __shared__ __align__(1024) char Vs[TL::kBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, hl = lane >> 5;
  int64_t bh, t;
  window_tile(p, bh, t);
  const int64_t row0 = bh * p.n_c * kChunk;
  const int64_t qrow0 = row0 + t * kChunk;
  const int my_q = 32 * wave + li;

  Frag<T> qf[4], df[4], of[4];
  const int64_t my_row = qrow0 + my_q;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    qf[s].load(static_cast<const T*>(p.q) + my_row * kDim + 16 * s + 8 * hl);
    df[s].load(static_cast<const T*>(p.dout) + my_row * kDim + 16 * s + 8 * hl);
    of[s].load(static_cast<const T*>(p.o_in) + my_row * kDim + 16 * s + 8 * hl);
  }
  // D = <dO, O> of this lane's query (lanes l and l ^ 32 hold its two halves of the dimensions)
  float dd = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s) dd += frag_dot(df[s], of[s]);
  const float D = xor32_sum(dd);
  const float bias = -p.lse_in[my_row] * kLog2e;
  // per query tile: 64 biases, then the 64 negated D (one store: each lane half writes one)
  p.stats[2 * qrow0 + 64 * hl + my_q] = hl ? -D : bias;
  Off off;
  off.init(wave);

  const int64_t kt0 = t - p.m > 0 ? t - p.m : 0;
  const int nt = static_cast<int>(t - kt0 + 1);
  auto tile = [&](const void* base, int64_t kt) {
    return static_cast<const T*>(base) + (row0 + kt * kChunk) * kDim;
  };
  off.copy(tile(p.k, kt0), Ka, wave);
  off.copy(tile(p.v, kt0), Vs, wave);
  barrier_copies_landed<0>();
  // The loads above are pinned here, before the loop, so that the compiler waits for them once:
  // left to their first use in the loop, its vmcnt waits would run in every iteration and also
  // wait for the untracked prefetch copies in flight.  Here they have all landed: the barrier
  // waited.
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    pin_in_registers(qf[s]);
    pin_in_registers(df[s]);
  }
  float bias_pinned = bias;
  asm volatile("" : "+v"(bias_pinned));

  f32x16_t dqacc[2] = {zero16(), zero16()};
  const float c2 = p.attn_scale * kLog2e;
  auto step = [&](int n, char* const Kc, char* const Kn) {
    const int64_t kt = kt0 + n;
    const bool more = n + 1 < nt;
    if (more) off.copy(tile(p.k, kt + 1), Kn, wave);  // the other K buffer is free
    f32x16_t sacc[2], pacc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      sacc[tt] = zero16();
      pacc[tt] = zero16();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        sacc[tt] = mma(off.kfrag(Kc, tt, s), qf[s], sacc[tt]);
        pacc[tt] = mma(off.kfrag(Vs, tt, s), df[s], pacc[tt]);
      }
    }
    barrier_lds_reads_done();  // every wave has read V(kt)
    if (more) off.copy(tile(p.v, kt + 1), Vs, wave);
    const bool lower_edge = kt == t - p.m, diagonal = kt == t;
    if (lower_edge || diagonal) sw_mask_keys_major(sacc, 32 * wave, diagonal);
    Frag<T> zf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tt = s >> 1, r = 8 * (s & 1) + e;
        const float pw = fast_exp2(__builtin_fmaf(sacc[tt][r], c2, bias_pinned));
        x[e] = pw * (pacc[tt][r] - D);
      }
      zf[s].set(x);
    }
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int s = 0; s < 4; ++s) dqacc[dt] = mma(off.vfrag(Kc, s, dt), zf[s], dqacc[dt]);
    // K(kt + 1) and V(kt + 1) landed, and every wave has read K(kt), whose buffer the next step
    // refills
    if (more) barrier_copies_landed_reads_done<0>();
  };
  for (int n = 0; n < nt; n += 2) {
    step(n, Ka, Kb);
    if (n + 1 < nt) step(n + 1, Kb, Ka);
  }

  T* dq = static_cast<T*>(p.dq) + my_row * kDim;
  const float sc = p.attn_scale;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a)
      store4(dq + 32 * dt + 8 * a + 4 * hl, sc * dqacc[dt][4 * a], sc * dqacc[dt][4 * a + 1],
             sc * dqacc[dt][4 * a + 2], sc * dqacc[dt][4 * a + 3]);
}

// Key-major pass: one workgroup of two waves (32 keys each) per key tile kt walks the query tiles
// kt .. kt + m whose windows reach it, double-buffered like the GCA key-major pass (Q tile, dO
// tile and the 64 biases and 64 -D of the next query tile copied in at the start of the current).
template <typename T>
__global__ __launch_bounds__(kThreads) void sw_bwd_key_kernel(SwParams p) {
  using TL = Tile<T>;
  using Off = TileOffsets<T, kWaves>;
  constexpr int kVecBytes = kChunk * 8;
  __shared__ __align__(1024) char buf0[2 * TL::kBytes + kVecBytes];
  __shared__ __align__(1024) char buf1[2 * TL::kBytes + kVecBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, hl = lane >> 5;
  int64_t bh, kt;
  window_tile(p, bh, kt);
  const int64_t row0 = bh * p.n_c * kChunk;
  const int my_u = 32 * wave + li;
  const int64_t krow = row0 + kt * kChunk + my_u;

  Frag<T> kf[4], vf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    kf[s].load(static_cast<const T*>(p.k) + krow * kDim + 16 * s + 8 * hl);
    vf[s].load(static_cast<const T*>(p.v) + krow * kDim + 16 * s + 8 * hl);
  }
  Off off;
  off.init(wave);
  f32x16_t dkacc[2] = {zero16(), zero16()};
  f32x16_t dvacc[2] = {zero16(), zero16()};
  const float c2 = p.attn_scale * kLog2e;
  const int64_t qt_last = kt + p.m < p.n_c - 1 ? kt + p.m : p.n_c - 1;
  const int count = static_cast<int>(qt_last - kt + 1);

  auto fill = [&](int64_t qt, char* buf) {
    const int64_t qrow0 = row0 + qt * kChunk;
    off.copy(static_cast<const T*>(p.q) + qrow0 * kDim, buf, wave);
    off.copy(static_cast<const T*>(p.dout) + qrow0 * kDim, buf + TL::kBytes, wave);
    // wave w copies the biases and the -D of queries 32 w .. 32 w + 31 (16 bytes per lane,
    // lanes < 16): lanes 0-7 the biases, lanes 8-15 the -D, to [32 biases, 32 -D] at 256 w
    const float* src = p.stats + 2 * qrow0 + 32 * wave;
    if (lane < 16)
      copy16_async_untracked(src, 256u * (lane >> 3) + 16u * (lane & 7), buf + 2 * TL::kBytes + 256 * wave);
  };
  auto body = [&](int n, const char* cur, char* nxt) {
    const int64_t qt = kt + n;
    if (n + 1 < count) fill(qt + 1, nxt);
    const char* Qs = cur;
    const char* Ds = cur + TL::kBytes;
    // [32 biases, 32 -D] of queries 0-31, then of queries 32-63; the dP products start from -D
    // of their queries, so they leave dP - D
    const float* vec = reinterpret_cast<const float*>(cur + 2 * TL::kBytes);
    const bool diagonal = qt == kt, lower_edge = qt == kt + p.m;
    // every row fragment of the query tile is read before the first product, so the products
    // wait once for the LDS reads instead of once per product
    Frag<T> qr[2][4], dr[2][4];
    f32x16_t sacc[2], pacc[2];
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        qr[qh][s] = off.kfrag(Qs, qh, s);
        dr[qh][s] = off.kfrag(Ds, qh, s);
      }
      pacc[qh] = *reinterpret_cast<const f32x16_t*>(vec + 64 * qh + 32 + 16 * hl);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the products
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      sacc[qh] = zero16();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        sacc[qh] = mma(qr[qh][s], kf[s], sacc[qh]);
        pacc[qh] = mma(dr[qh][s], vf[s], pacc[qh]);
      }
    }
    if (lower_edge || diagonal) {  // wave-uniform: only the two edge query tiles are masked
      // sacc[qh][r] = S[query 32 qh + 16 hl + r][key my_u]: the query lies before the key
      // (masked in the diagonal tile, kept at the lower edge) exactly when r < my_u - 32 qh - 16 hl
#pragma unroll
      for (int qh = 0; qh < 2; ++qh) mask_run(sacc[qh], my_u - 32 * qh - 16 * hl, lower_edge);
    }
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      // lane holds queries 32 qh + 16 hl + r of key my_u
      Frag<T> pf[2], zf[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const f32x4_t* bq = reinterpret_cast<const f32x4_t*>(vec + 64 * qh + 16 * hl + 8 * half);
        const f32x4_t b0 = bq[0], b1 = bq[1];
        float xp[8], xz[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * half + e;
          const float pw = fast_exp2(__builtin_fmaf(sacc[qh][r], c2, e < 4 ? b0[e] : b1[e - 4]));
          xp[e] = pw;
          xz[e] = pw * pacc[qh][r];
        }
        pf[half].set(xp);
        zf[half].set(xz);
      }
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          dvacc[dt] = mma(off.vfrag(Ds, 2 * qh + half, dt), pf[half], dvacc[dt]);
          dkacc[dt] = mma(off.vfrag(Qs, 2 * qh + half, dt), zf[half], dkacc[dt]);
        }
    }
    // the next query tile's copies landed, and every wave is done with this buffer
    barrier_copies_landed_reads_done<0>();
  };
  fill(kt, buf0);
  barrier_copies_landed_reads_done<0>();
  // The loads above are pinned here, before the loop, so that the compiler waits for them once:
  // left to their first use in the loop, its vmcnt waits would run in every iteration and also
  // wait for the untracked prefetch copies in flight.  Here they have all landed: the barrier
  // waited.
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    pin_in_registers(kf[s]);
    pin_in_registers(vf[s]);
  }
  for (int n = 0; n < count; n += 2) {
    body(n, buf0, buf1);
    if (n + 1 < count) body(n + 1, buf1, buf0);
  }

  T* dk = static_cast<T*>(p.dk) + krow * kDim;
  T* dv = static_cast<T*>(p.dv) + krow * kDim;
  const float sc = p.attn_scale;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d0 = 32 * dt + 8 * a + 4 * hl;
      store4(dk + d0, sc * dkacc[dt][4 * a], sc * dkacc[dt][4 * a + 1], sc * dkacc[dt][4 * a + 2],
             sc * dkacc[dt][4 * a + 3]);
      store4(dv + d0, dvacc[dt][4 * a], dvacc[dt][4 * a + 1], dvacc[dt][4 * a + 2], dvacc[dt][4 * a + 3]);
    }
}

// ------------------------------------------------------------- backward, key-major (dK, dV)
struct PairRef {
  int g, slot;
  int64_t t;
};

// The backward's inverse index stores each entry decoded: {query chunk t, g * 16 + slot}
// (wave-uniform), so the walk needs no integer division per entry.
__device__ __forceinline__ PairRef decode_pair(const i32x2_t ent) {
  const int32_t gs = __builtin_amdgcn_readfirstlane(ent[1]);
  PairRef r;
  r.t = __builtin_amdgcn_readfirstlane(ent[0]);
  r.g = gs >> 4;
  r.slot = gs & 15;
  return r;
}

// Key-major walk of one key chunk's entries e0 .. e1 - 1 (one (batch row, head, key chunk)):
// each wave owns 32 of the chunk's keys and accumulates their dK (unscaled) and dV over the
// entries, double-buffered: the next entry's Q and dO tiles and its 64 biases and 64 -e are
// copied in at the start of the current one.  Every copy has landed and every LDS read is done
// when it returns, so walks can follow one another in the same workgroup.  tid is the thread
// index (threadIdx.x, or an opaque copy of it in a loop of walks).
template <typename T>
__device__ __forceinline__ void key_walk(const AttendParams& p, int64_t bh, int64_t j, int32_t e0, int32_t e1,
                                         char* buf0, char* buf1, i32x2_t* ents, f32x16_t (&dkacc)[2],
                                         f32x16_t (&dvacc)[2], int tid) {
  using TL = Tile<T>;
  using Off = TileOffsets<T, kWaves>;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, hl = lane >> 5;
  const uint32_t H = static_cast<uint32_t>(p.H);
  const int b = static_cast<int>(static_cast<uint32_t>(bh) / H);  // bh < B H < 2^31
  const int h = static_cast<int>(static_cast<uint32_t>(bh) - static_cast<uint32_t>(b) * H);
  const int my_u = 32 * wave + li;

  const int64_t krow = (bh * p.n_kv + j) * kChunk + my_u;
  Frag<T> kf[4], vf[4];
  const T* kp = static_cast<const T*>(p.k) + krow * kDim;
  const T* vp = static_cast<const T*>(p.v) + krow * kDim;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    kf[s].load(kp + 16 * s + 8 * hl);
    vf[s].load(vp + 16 * s + 8 * hl);
  }
  Off off;
  off.init(wave, tid);
  dkacc[0] = dkacc[1] = dvacc[0] = dvacc[1] = zero16();
  const float c2 = p.attn_scale * kLog2e;
  const int64_t Lq = p.n_q * kChunk;
  const int64_t segment = static_cast<int64_t>(b) * p.n_kv + j;
  const i32x2_t* list = reinterpret_cast<const i32x2_t*>(p.pairs) + segment * p.pair_cap;

  // The list is walked in rounds of up to kEntRound entries {code, weight}, staged in LDS.  Each
  // wave issues kCopies per tile plus one vector copy (lanes < 16) per entry.
  auto fill = [&](const i32x2_t ent, char* buf) {
    const PairRef r = decode_pair(ent);
    const int64_t gbh = (static_cast<int64_t>(r.g) * p.B + b) * p.H + h;
    const int64_t qrow0 = gbh * Lq + r.t * kChunk;
    off.copy(static_cast<const T*>(p.q) + qrow0 * kDim, buf, wave);
    off.copy(static_cast<const T*>(p.dout) + qrow0 * kDim, buf + TL::kBytes, wave);
    // wave w copies the biases and the -e of queries 32 w .. 32 w + 31 (16 bytes per lane,
    // lanes < 16): lanes 0-7 the biases, lanes 8-15 the -e, to [32 biases, 32 -e] at 256 w
    const float* src = p.delta + 2 * slot_vec_offset(p, gbh, r.t, r.slot) + 32 * wave;
    if (lane < 16)
      copy16_async_untracked(src, 256u * (lane >> 3) + 16u * (lane & 7), buf + 2 * TL::kBytes + 256 * wave);
  };

  int32_t n = 0;  // entries in the current round
  auto body = [&](int32_t pr, const char* cur, char* nxt) {
    if (pr + 1 < n) fill(ents[pr + 1], nxt);
    const char* Qs = cur;
    const char* Ds = cur + TL::kBytes;
    // [32 biases, 32 -e] of queries 0-31, then of queries 32-63
    const float* vec = reinterpret_cast<const float*>(cur + 2 * TL::kBytes);
    // Both 32-query tiles' scores first, then each tile's elementwise work beside the other
    // tile's matrix-core work (the second tile's S and dP' products run beside the first tile's
    // exp and dz, the first tile's dK and dV products beside the second tile's).  Every row
    // fragment of the entry is read before the first product, so the products wait once for the
    // LDS reads instead of once per product.
    // The dP' products start from -e of their queries, so they leave dP' - e.
    Frag<T> qr[2][4], dr[2][4];
    f32x16_t sacc[2], pacc[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        qr[qt][s] = off.kfrag(Qs, qt, s);
        dr[qt][s] = off.kfrag(Ds, qt, s);
      }
      pacc[qt] = *reinterpret_cast<const f32x16_t*>(vec + 64 * qt + 32 + 16 * hl);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the products
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      sacc[qt] = zero16();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        sacc[qt] = mma(qr[qt][s], kf[s], sacc[qt]);
        pacc[qt] = mma(dr[qt][s], vf[s], pacc[qt]);
      }
    }
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      // lane holds queries 32 qt + 16 hl + r: P_w = w exp(z - lse) = exp2(z log2e + bias)
      Frag<T> pf[2], zf[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const f32x4_t* bq = reinterpret_cast<const f32x4_t*>(vec + 64 * qt + 16 * hl + 8 * half);
        const f32x4_t b0 = bq[0], b1 = bq[1];
        float xp[8], xz[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * half + e;
          const float pw = fast_exp2(__builtin_fmaf(sacc[qt][r], c2, e < 4 ? b0[e] : b1[e - 4]));
          xp[e] = pw;
          xz[e] = pw * pacc[qt][r];
        }
        pf[half].set(xp);
        zf[half].set(xz);
      }
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          dvacc[dt] = mma(off.vfrag(Ds, 2 * qt + half, dt), pf[half], dvacc[dt]);
          dkacc[dt] = mma(off.vfrag(Qs, 2 * qt + half, dt), zf[half], dkacc[dt]);
        }
    }
    // the next entry's copies landed, and every wave is done with this entry's buffer
    barrier_copies_landed_reads_done<0>();
  };
  // ents is read only inside body, before its closing barrier, so when a round (or a walk) ends
  // every wave is done with it and the next round may restage it.
  for (int32_t round0 = e0; round0 < e1; round0 += kEntRound) {
    n = e1 - round0 < kEntRound ? e1 - round0 : kEntRound;
    for (int e = tid; e < n; e += kThreads) ents[e] = list[round0 + e];
    __syncthreads();
    // The K and V fragments are in registers here (the barrier waited for every load), so the
    // compiler has no load of its own left to wait for in the entry loop, where a vmcnt wait
    // would also wait for the untracked prefetch copies.
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      pin_in_registers(kf[s]);
      pin_in_registers(vf[s]);
    }
    fill(ents[0], buf0);
    barrier_copies_landed_reads_done<0>();
    for (int32_t pr = 0; pr < n; pr += 2) {
      body(pr, buf0, buf1);
      if (pr + 1 < n) body(pr + 1, buf1, buf0);
    }
  }
}

// dK, dV of one wave's 32 keys from its accumulators: into the dK, dV tensors (dK scaled by
// attn_scale), or unscaled into a float [2][64 keys][64] partial of a split list.
template <typename D>
__device__ __forceinline__ void store_key_grads(D* dk, D* dv, float sc, const f32x16_t (&dkacc)[2],
                                                const f32x16_t (&dvacc)[2]) {
  const int hl = (threadIdx.x >> 5) & 1;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d0 = 32 * dt + 8 * a + 4 * hl;
      store4(dk + d0, sc * dkacc[dt][4 * a], sc * dkacc[dt][4 * a + 1], sc * dkacc[dt][4 * a + 2],
             sc * dkacc[dt][4 * a + 3]);
      store4(dv + d0, dvacc[dt][4 * a], dvacc[dt][4 * a + 1], dvacc[dt][4 * a + 2], dvacc[dt][4 * a + 3]);
    }
}

// One workgroup of two waves per (batch row, head, key chunk) walks the chunk's entries and
// writes its dK, dV.  With long lists split (long_ctl set), a chunk of more than kSplitMin
// entries is walked in segments instead: the first n_help workgroups of the launch take the work
// items f = q * H + h (the walk of segment slot q, at most kSegEntries entries of one long chunk,
// for head h) in turn and write float partials, which score_grad_kernel sums in segment order;
// with no long list they end at once.  Both kinds run side by side (they write disjoint outputs
// and only read the inverse index).  n_help is a multiple of 8, so the other workgroups keep the
// XCD order of xcd_logical_block.
template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_key_kernel(AttendParams p) {
  using TL = Tile<T>;
  constexpr int kVecBytes = kChunk * 8;  // biases and -e of the 64 queries of one entry
  __shared__ __align__(1024) char buf0[2 * TL::kBytes + kVecBytes];  // [Q tile, dO tile, vectors]
  __shared__ __align__(1024) char buf1[2 * TL::kBytes + kVecBytes];
  __shared__ i32x2_t ents[kEntRound];
  const int my_u = 32 * (threadIdx.x >> 6) + (threadIdx.x & 31);
  if (static_cast<int32_t>(blockIdx.x) < p.n_help) {
    const uint64_t ctl = *p.long_ctl;
    const int32_t n_long = min(static_cast<int32_t>(ctl >> 32), p.long_cap);
    const int32_t n_seg = min(static_cast<int32_t>(ctl & 0xffffffffu), p.seg_cap);
    const int64_t items = static_cast<int64_t>(n_seg) * p.H;
    for (int64_t f = blockIdx.x; f < items; f += p.n_help) {
      const int32_t q = static_cast<int32_t>(f / p.H);
      const int h = static_cast<int>(f - static_cast<int64_t>(q) * p.H);
      const int32_t at = __builtin_amdgcn_readfirstlane(p.long_seg[q]);
      if (at < 0 || at >= n_long) return;  // never, by the capacities' bound (see inverse_index_kernel)
      const i32x4_t ent = reinterpret_cast<const i32x4_t*>(p.long_list)[at];  // {b, j, segments, first slot}
      const int32_t b = __builtin_amdgcn_readfirstlane(ent[0]);
      const int32_t j = __builtin_amdgcn_readfirstlane(ent[1]);
      const int32_t count = p.counts[static_cast<int64_t>(b) * p.n_kv + j];
      const int32_t e0 = (q - __builtin_amdgcn_readfirstlane(ent[3])) * kSegEntries;
      const int32_t e1 = count - e0 < kSegEntries ? count : e0 + kSegEntries;
      if (e0 < 0 || e0 >= e1) return;
      // the thread index, opaque in every item: the walk's per-lane set-up is then recomputed for
      // each walk instead of hoisted out of the loop and held live across it (which costs the
      // second wave per SIMD)
      int tid = static_cast<int>(threadIdx.x);
      asm volatile("" : "+v"(tid));
      f32x16_t dkacc[2], dvacc[2];
      key_walk<T>(p, static_cast<int64_t>(b) * p.H + h, j, e0, e1, buf0, buf1, ents, dkacc, dvacc, tid);
      float* part = p.long_part + f * (2 * kChunk * kDim) + my_u * kDim;
      store_key_grads(part, part + kChunk * kDim, 1.f, dkacc, dvacc);
    }
    return;
  }
  // B H n_kv < 2^31 blocks (checked on the host): 32-bit divisions
  const uint32_t lid = static_cast<uint32_t>(xcd_logical_block(blockIdx.x - p.n_help, gridDim.x - p.n_help));
  const uint32_t nkv = static_cast<uint32_t>(p.n_kv);
  const uint32_t bh32 = lid / nkv;
  const int64_t j = lid - bh32 * nkv;
  const int64_t bh = bh32;
  const int32_t count = p.counts[static_cast<int64_t>(bh32 / static_cast<uint32_t>(p.H)) * p.n_kv + j];
  // a split list is the helpers' work: walk nothing and write nothing (not an early return,
  // which would hold the walk's K/V loads back behind the count's)
  const bool split = p.long_ctl != nullptr && count > kSplitMin;
  f32x16_t dkacc[2], dvacc[2];
  key_walk<T>(p, bh, j, 0, split ? 0 : count, buf0, buf1, ents, dkacc, dvacc, static_cast<int>(threadIdx.x));
  if (split) return;
  const int64_t krow = (bh * p.n_kv + j) * kChunk + my_u;
  store_key_grads(static_cast<T*>(p.dk) + krow * kDim, static_cast<T*>(p.dv) + krow * kDim, p.attn_scale, dkacc,
                  dvacc);
}

// ------------------------------------------------------------- inverse retrieval index
// For one batch row and 64 consecutive key chunks (lane = chunk j), list the retrievals that
// selected each chunk, in (group, row) order, as entries {(group, row, slot) code, entry value}
// (the landmark gradients: the value is d(score)) or, with entry_decoded (the GCA backward's
// key-major pass), {query chunk row + shift, group * 16 + slot}.
// Retrieval rows, flattened as gr = g * n_q + row, are handled kIdxRows at a time as 32-row
// words.  Phase 1: one thread per row ORs the row's bit into the mask of every chunk of this
// block the row names (integer OR: the result does not depend on the order).  Phase 2: a running
// prefix of the masks' popcounts gives every (word, chunk) its first output position.  Phase 3:
// one thread per row writes each of its entries at that position plus the row's rank among the
// word's rows naming the chunk, so each chunk's entries come out in row order.  Only rows that feed a query
// chunk (row + shift < n_q) are marked; with causal_rows (the landmark gradients) also only rows
// that can hold a chunk of this block (global chunk index q_base + row above the block's first
// chunk), a coarse filter that the landmark key pass refines per entry.  The GCA backward lists
// every row, so its key-major pass counts the same slots (0 <= j < n_kv) as its query-major pass.
// Runs after the query-major pass, which writes the fusion weights.
constexpr int kIdxThreads = 256;
constexpr int kIdxWords = 16;
constexpr int kIdxRows = kIdxWords * 32;

__global__ __launch_bounds__(kIdxThreads) void inverse_index_kernel(AttendParams p) {
  __shared__ int32_t idx_s[kIdxRows][kMaxTopk];
  __shared__ float wts_s[kIdxRows][kMaxTopk];
  __shared__ uint32_t mask[kIdxWords][64];
  __shared__ int32_t first[kIdxWords][64];
  __shared__ int32_t total[64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int32_t nblk = static_cast<int32_t>((p.n_kv + 63) / 64);
  const int b = static_cast<int>(blockIdx.x / nblk);
  const int32_t j0 = static_cast<int32_t>(blockIdx.x % nblk) * 64;
  const int32_t j = j0 + lane;
  // chunk ids, row counts and (g, row) indices fit in int32 (checked on the host)
  const int32_t nq = static_cast<int32_t>(p.n_q);
  const int32_t row_lo =
      p.causal_rows ? static_cast<int32_t>(j0 - p.q_base + 1 > 0 ? j0 - p.q_base + 1 : 0) : 0;
  const int32_t row_hi = nq - p.shift;
  const int32_t n_rows = p.G * nq;
  const int K = p.K;
  if (tid < 64) total[tid] = 0;
  i32x2_t* out_b = reinterpret_cast<i32x2_t*>(p.pairs) + static_cast<int64_t>(b) * p.n_kv * p.pair_cap;

  for (int32_t gr0 = 0; gr0 < n_rows; gr0 += kIdxRows) {
    const int32_t nr = n_rows - gr0 < kIdxRows ? n_rows - gr0 : kIdxRows;
    const int nw = (nr + 31) / 32;
    for (int e = tid; e < kIdxWords * 64; e += kIdxThreads) mask[e / 64][e % 64] = 0u;
    __syncthreads();
    // phase 1: one thread per row
    for (int lr = tid; lr < nr; lr += kIdxThreads) {
      const int32_t gr = gr0 + lr;
      const int32_t g = gr / nq, row = gr - g * nq;
      const int64_t rbase = ((static_cast<int64_t>(g) * p.B + b) * nq + row) * K;
      const bool live = row >= row_lo && row < row_hi;
      int32_t jv[kMaxTopk];
      float wv[kMaxTopk];
#pragma unroll
      for (int k = 0; k < kMaxTopk; ++k) {  // all of the row's loads in flight together
        jv[k] = k < K ? p.idx[rbase + k] : -1;
        wv[k] = k < K && !p.entry_decoded ? p.wts[rbase + k] : 0.f;
      }
#pragma unroll
      for (int k = 0; k < kMaxTopk; ++k) {
        if (k >= K) break;
        idx_s[lr][k] = jv[k];
        wts_s[lr][k] = wv[k];
        if (live && jv[k] >= j0 && jv[k] < j0 + 64 && jv[k] < p.n_kv)
          atomicOr(&mask[lr >> 5][jv[k] - j0], 1u << (lr & 31));
      }
    }
    __syncthreads();
    // phase 2: first output position of every word
    if (tid < 64) {
      int32_t run = total[tid];
      for (int wl = 0; wl < nw; ++wl) {
        first[wl][tid] = run;
        run += __popc(mask[wl][tid]);
      }
      total[tid] = run;
    }
    __syncthreads();
    // phase 3: one thread per row writes the entries of its slots that name chunks of this block,
    // each at its chunk's count before the row's word plus the row's rank among the word's rows
    // naming the chunk (the mask bits below it), so every chunk's entries come out in row order.
    // A row counts once per chunk, with its first slot naming it.
    for (int lr = tid; lr < nr; lr += kIdxThreads) {
      const int32_t gr = gr0 + lr;
      const int32_t g = gr / nq;
      const int32_t row = gr - g * nq;
      if (row < row_lo || row >= row_hi) continue;
      const int w = lr >> 5;
      const uint32_t below = (1u << (lr & 31)) - 1u;
      int32_t jv[kMaxTopk];
#pragma unroll
      for (int k = 0; k < kMaxTopk; ++k) jv[k] = k < K ? idx_s[lr][k] : -1;
#pragma unroll
      for (int k = 0; k < kMaxTopk; ++k) {
        const int32_t jk = jv[k];  // -1 beyond K
        bool first_slot = jk >= j0 && jk < j0 + 64 && jk < p.n_kv;
#pragma unroll
        for (int k2 = 0; k2 < k; ++k2) first_slot = first_slot && jv[k2] != jk;
        if (first_slot) {
          const int jj = jk - j0;
          const int32_t pos = first[w][jj] + __popc(mask[w][jj] & below);
          out_b[static_cast<int64_t>(jk) * p.pair_cap + pos] =
              p.entry_decoded ? i32x2_t{row + p.shift, g * 16 + k} : i32x2_t{gr * K + k, __float_as_int(wts_s[lr][k])};
        }
      }
    }
    __syncthreads();
  }
  if (tid < 64 && j < p.n_kv) {
    const int32_t c = total[tid];
    p.counts[static_cast<int64_t>(b) * p.n_kv + j] = c;
    // A list longer than kSplitMin is split for the key-major pass: one 64-bit atomic takes its
    // place in the list of long chunks (high word) and its segment slots (low word), so the
    // list stays in slot order.  The order of the chunks in it varies from run to run; what is
    // computed for each chunk and segment does not.
    if (p.long_ctl != nullptr && c > kSplitMin) {
      const int32_t nseg = (c + kSegEntries - 1) / kSegEntries;
      const unsigned long long old =
          atomicAdd(reinterpret_cast<unsigned long long*>(p.long_ctl), (1ull << 32) | static_cast<unsigned long long>(nseg));
      const int32_t at = static_cast<int32_t>(old >> 32), pos = static_cast<int32_t>(old & 0xffffffffull);
      if (at < p.long_cap && pos + nseg <= p.seg_cap) {  // always, by the capacities' bound
        reinterpret_cast<i32x4_t*>(p.long_list)[at] = i32x4_t{b, j, nseg, pos};
        for (int32_t sg = 0; sg < nseg; ++sg) p.long_seg[pos + sg] = at;
      }
    }
  }
}

// ------------------------------------------------------------- d(score)
// dscore_k = w_k (dw_k - sum_k' w_k' dw_k'), dw_k = sum over heads (in order) of the per-head
// sums of e over the chunk's tokens.  Sixteen lanes per (g, b, row), one lane per slot.
template <typename T>
__global__ __launch_bounds__(256) void score_grad_kernel(AttendParams p) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int k = threadIdx.x & 15;
  const int64_t rows = static_cast<int64_t>(p.G) * p.B * p.n_q;
  const bool in_range = gid < rows && k < p.K;
  const int64_t row = gid % p.n_q;
  bool valid = false;
  float w = 0.f, dw = 0.f;
  if (in_range) {
    const int32_t jj = p.idx[gid * p.K + k];
    valid = row + p.shift < p.n_q && jj >= 0 && jj < p.n_kv;
    if (valid) {
      w = p.wts[gid * p.K + k];
      // eight heads' loads in flight at a time, added in head order
      constexpr int kBatch = 8;
      const float* dp = p.dw_part + gid * p.H * p.K + k;
      for (int h0 = 0; h0 < p.H; h0 += kBatch) {
        float v[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b)
          if (h0 + b < p.H) v[b] = dp[(h0 + b) * p.K];
#pragma unroll
        for (int b = 0; b < kBatch; ++b)
          if (h0 + b < p.H) dw += v[b];
      }
    }
  }
  float wdw = w * dw;
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) wdw += __shfl_xor(wdw, off, 16);
  if (in_range) p.dscore[gid * p.K + k] = valid ? w * (dw - wdw) : 0.f;
  // dK, dV of the chunks whose lists were split: the segments' partials summed in segment order,
  // dK scaled by attn_scale, one (chunk, head) per workgroup in turn
  if (p.long_ctl == nullptr) return;
  const uint64_t ctl = *p.long_ctl;
  const int64_t n_long = min(static_cast<int32_t>(ctl >> 32), p.long_cap);
  constexpr int kPart = 2 * kChunk * kDim;  // floats of one partial: [dK, dV][64 keys][64]
  for (int64_t it = blockIdx.x; it < n_long * p.H; it += gridDim.x) {
    const int64_t li = it / p.H;
    const int h = static_cast<int>(it - li * p.H);
    const i32x4_t ent = reinterpret_cast<const i32x4_t*>(p.long_list)[li];  // {b, j, segments, first slot}
    if (ent[0] < 0 || ent[0] >= p.B || ent[1] < 0 || ent[1] >= p.n_kv || ent[2] < 1 || ent[3] < 0 ||
        ent[3] + ent[2] > p.seg_cap)
      continue;  // never: every entry is written whole before the key-major pass
    const int64_t tile = ((static_cast<int64_t>(ent[0]) * p.H + h) * p.n_kv + ent[1]) * kChunk * kDim;
    const f32x4_t* part = reinterpret_cast<const f32x4_t*>(p.long_part + (static_cast<int64_t>(ent[3]) * p.H + h) * kPart);
    const int64_t stride = static_cast<int64_t>(p.H) * kPart / 4;
    for (int e = threadIdx.x; e < kPart / 4; e += 256) {
      // the segments' loads eight at a time, all in flight, then added in segment order
      constexpr int kBatch = 8;
      f32x4_t acc = part[e];
      for (int32_t s0 = 1; s0 < ent[2]; s0 += kBatch) {
        f32x4_t v[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b)
          if (s0 + b < ent[2]) v[b] = part[(s0 + b) * stride + e];
#pragma unroll
        for (int b = 0; b < kBatch; ++b)
          if (s0 + b < ent[2]) acc += v[b];
      }
      const bool is_v = e >= kPart / 8;
      const float sc = is_v ? 1.f : p.attn_scale;
      T* dst = static_cast<T*>(is_v ? p.dv : p.dk) + tile + 4 * (e & (kPart / 8 - 1));
      store4(dst, sc * acc[0], sc * acc[1], sc * acc[2], sc * acc[3]);
    }
  }
}

// ------------------------------------------------- fused layer attention (window + GCA), forward
// The layers that run GCA also run sliding-window self-attention (W = 512) [Notes, Loss /
// training strategy].  Reading taken: both read the layer's queries and their outputs are summed,
// with one retrieval group per layer:
//   o = SW(q, k_sw, v_sw; W) + GCA(q, k, v, idx, score).
// One query tile t walks one list of items: the window's key tiles kt0 .. t (online softmax, the
// edge tiles masked), then the valid retrieval slots (one softmax each, weighted by w).  One K and
// one V buffer, the copy pipeline running straight through from the last window tile to the first
// retrieved chunk.  After the window's last tile the accumulators are normalized (1 / l per query),
// so they hold the window's output, and each slot adds w_k O_k to them.  The Q tile is loaded
// once and the sum is stored once.

// Fused forward, one wave per 64-query tile (bf16), the pipeline of attend_fwd_wave_kernel.
template <bool kLse>
__global__ __launch_bounds__(64) void fused_fwd_kernel(AttendParams p) {
  using T = bf16_t;
  using TL = Tile<T>;
  using Off = TileOffsets<T, 1>;
  constexpr int kC = Off::kCopies;
  __shared__ __align__(1024) char Ks[TL::kBytes];
  __shared__ __align__(1024) char Vs[TL::kBytes];

  const int lane = threadIdx.x, li = lane & 31, hl = lane >> 5;
  const QTileCoord c = query_tile_coord(p);
  const int64_t Lq = p.n_q * kChunk;
  const int64_t row0 = (static_cast<int64_t>(c.b) * p.H + c.h) * Lq;  // this (batch row, head)
  const int64_t qrow0 = row0 + c.t * kChunk;
  Frag<T> qf[2][4];
#pragma unroll
  for (int qh = 0; qh < 2; ++qh) {
    const T* q = static_cast<const T*>(p.q) + (qrow0 + 32 * qh + li) * kDim;
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[qh][s].load(q + 16 * s + 8 * hl);
  }
  // after the query loads, so that one memory round trip covers both
  const WaveSlots sl = wave_slots(p, c.g, c.b, c.t - p.shift);
  Off off;
  off.init(0);
  // copies address the buffers by their LDS addresses: with the two item loops below, the
  // backend could not fold the null check of the generic pointer round trip of copy()
  const uint32_t ks_addr = lds_address(Ks), vs_addr = lds_address(Vs);
  float* const lse_q = kLse ? p.lse + slot_vec_offset(p, c.gbh, c.t, 0) + lane : nullptr;
  if (kLse) {  // invalid slots: -inf (before any copy, so the copy counts below stay exact)
    for (int k = 0; k < p.K; ++k)
      if (!((sl.valid >> k) & 1u)) lse_q[k * kChunk] = -__builtin_inff();
  }
  const int64_t kt0 = c.t - p.m > 0 ? c.t - p.m : 0;
  const int n_sw = static_cast<int>(c.t - kt0 + 1);
  const int n_items = n_sw + __popc(sl.valid);
  // item i: window tile kt0 + i (i < n_sw), else the next valid slot; separate cursors for the
  // K copies, the V copies and the softmax, which reach each item at different times
  uint32_t rem_k = sl.valid, rem_v = sl.valid, rem_s = sl.valid;
  auto item_tile = [&](const void* sw_base, const void* kv_base, int i, uint32_t& rem) {
    if (i < n_sw) return static_cast<const T*>(sw_base) + (row0 + (kt0 + i) * kChunk) * kDim;
    const int slot = __builtin_ctz(rem);
    rem &= rem - 1;
    return kv_tile<T>(kv_base, p, c.b, c.h, __builtin_amdgcn_readlane(sl.j, slot));
  };
  off.copy_at(item_tile(p.k_sw, p.k, 0, rem_k), ks_addr, 0);
  off.copy_at(item_tile(p.v_sw, p.v, 0, rem_v), vs_addr, 0);
  // The loads above are pinned here, before the loop, so that the compiler waits for them once:
  // left to their first use in the loop, its vmcnt waits would run in every iteration and also
  // wait for the untracked prefetch copies in flight.  The first item's tiles are needed at once
  // anyway.
#pragma unroll
  for (int qh = 0; qh < 2; ++qh)
#pragma unroll
    for (int s = 0; s < 4; ++s) pin_in_registers(qf[qh][s]);

  f32x16_t oacc[2][2] = {{zero16(), zero16()}, {zero16(), zero16()}};
  float m_run[2] = {-__builtin_inff(), -__builtin_inff()}, l_run[2] = {0.f, 0.f};
  const float c2 = p.attn_scale * kLog2e;
  // the window's key tiles: online softmax; per query half, the softmax, then its P V products
  for (int i = 0; i < n_sw; ++i) {  // wave-uniform
    wait_vm_outstanding<kC>();  // K(i) landed: only V(i) may be in flight
    f32x16_t sacc[2][2];
    {  // K(i) into registers; the copy of K(i + 1) started behind it; S(i) = K(i) Q^T
      Frag<T> kf[2][4];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int s = 0; s < 4; ++s) kf[tt][s] = off.kfrag(Ks, tt, s);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // K(i) in registers: the buffer is free
      if (i + 1 < n_items) off.copy_at(item_tile(p.k_sw, p.k, i + 1, rem_k), ks_addr, 0);
#pragma unroll
      for (int qh = 0; qh < 2; ++qh)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          sacc[qh][tt] = zero16();
#pragma unroll
          for (int s = 0; s < 4; ++s) sacc[qh][tt] = mma(kf[tt][s], qf[qh][s], sacc[qh][tt]);
        }
    }
    const int64_t kt = kt0 + i;
    const bool lower_edge = kt == c.t - p.m, diagonal = kt == c.t;
    if (lower_edge || diagonal) sw_mask(sacc, diagonal);
    Frag<T> vf[4][2];
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[qh][tt][r]);
      mx = xor32_max(mx) * c2;  // log2 units
      constexpr float kLazy = 8.f;  // as in sw_fwd_kernel
      const bool grow = __ballot(mx > m_run[qh] + kLazy) != 0;
      const float m_new = grow ? fmaxf(m_run[qh], mx) : m_run[qh];
      const bool none = m_new == -__builtin_inff();
      const float alpha = none ? 1.f : fast_exp2(m_run[qh] - m_new);
      const float bias = none ? 0.f : -m_new;
      float l = 0.f;
      Frag<T> pf[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          x[e] = fast_exp2(__builtin_fmaf(sacc[qh][s >> 1][8 * (s & 1) + e], c2, bias));
          l += x[e];
        }
        pf[s].set(x);
      }
      l_run[qh] = l_run[qh] * alpha + xor32_sum(l);
      m_run[qh] = m_new;
      if (grow) {
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[qh][dt][r] *= alpha;
      }
      if (qh == 0) {  // V(i) into registers (landed: at most the K(i + 1) copies are outstanding);
                      // the copy of V(i + 1) started behind it
        if (i + 1 < n_items) wait_vm_outstanding<kC>();
        else wait_vm_outstanding<0>();
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int dt = 0; dt < 2; ++dt) vf[s][dt] = off.vfrag(Vs, s, dt);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // V(i) in registers: the buffer is free
        if (i + 1 < n_items) off.copy_at(item_tile(p.v_sw, p.v, i + 1, rem_v), vs_addr, 0);
      }
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int s = 0; s < 4; ++s) oacc[qh][dt] = mma(vf[s][dt], pf[s], oacc[qh][dt]);
    }
  }
  // the window is complete: its output, normalized per query
#pragma unroll
  for (int qh = 0; qh < 2; ++qh) {
    const float f = __builtin_amdgcn_rcpf(l_run[qh]);
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qh][dt][r] *= f;
  }
  // the retrieved slots: one softmax each, weighted by w
  bool stored = false;  // the previous slot issued an lse store after its copies
  for (int i = n_sw; i < n_items; ++i) {  // wave-uniform
    if (stored) wait_vm_outstanding<kC + 1>();  // K(i) landed: only V(i) and that store may not have
    else wait_vm_outstanding<kC>();
    f32x16_t sacc[2][2];
    {  // K(i) into registers; the copy of K(i + 1) started behind it; S(i) = K(i) Q^T
      Frag<T> kf[2][4];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int s = 0; s < 4; ++s) kf[tt][s] = off.kfrag(Ks, tt, s);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // K(i) in registers: the buffer is free
      if (i + 1 < n_items) off.copy_at(item_tile(p.k_sw, p.k, i + 1, rem_k), ks_addr, 0);
#pragma unroll
      for (int qh = 0; qh < 2; ++qh)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          sacc[qh][tt] = zero16();
#pragma unroll
          for (int s = 0; s < 4; ++s) sacc[qh][tt] = mma(kf[tt][s], qf[qh][s], sacc[qh][tt]);
        }
    }
    const int slot = __builtin_ctz(rem_s);
    rem_s &= rem_s - 1;
    const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sl.w), slot));
    float lse_v[2];
    Frag<T> vf[4][2];
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      float l;
      const float mx = tile_softmax(sacc[qh], c2, l);
      lse_v[qh] = mx * p.attn_scale + __builtin_amdgcn_logf(l) * kLn2f;
      const float f = wk * __builtin_amdgcn_rcpf(l);
      Frag<T> pf[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = sacc[qh][s >> 1][8 * (s & 1) + e] * f;
        pf[s].set(x);
      }
      if (qh == 0) {  // V(i) into registers (landed: at most the K(i + 1) copies are outstanding);
                      // the copy of V(i + 1) started behind it
        if (i + 1 < n_items) wait_vm_outstanding<kC>();
        else wait_vm_outstanding<0>();
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int dt = 0; dt < 2; ++dt) vf[s][dt] = off.vfrag(Vs, s, dt);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // V(i) in registers: the buffer is free
        if (i + 1 < n_items) off.copy_at(item_tile(p.v_sw, p.v, i + 1, rem_v), vs_addr, 0);
      }
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int s = 0; s < 4; ++s) oacc[qh][dt] = mma(vf[s][dt], pf[s], oacc[qh][dt]);
    }
    if (kLse) lse_q[slot * kChunk] = hl ? lse_v[1] : lse_v[0];
    stored = kLse;
  }

#pragma unroll
  for (int qh = 0; qh < 2; ++qh) {
    T* o = static_cast<T*>(p.o) + (qrow0 + 32 * qh + li) * kDim;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        store4(o + 32 * dt + 8 * a + 4 * hl, oacc[qh][dt][4 * a], oacc[qh][dt][4 * a + 1],
               oacc[qh][dt][4 * a + 2], oacc[qh][dt][4 * a + 3]);
    if (p.lse_sw && hl == qh)  // lane (li, hl) writes query 32 hl + li
      p.lse_sw[qrow0 + 32 * qh + li] = m_run[qh] * kLn2f + __builtin_amdgcn_logf(l_run[qh]) * kLn2f;
  }
}

// Fused forward, two waves of 32 queries per tile (fp32 tiles: the pipeline of attend_fwd_kernel
// and sw_fwd2_kernel, single K and V buffers published by barriers).
template <typename T, bool kLse>
__global__ __launch_bounds__(kThreads) void fused_fwd2_kernel(AttendParams p) {
  using TL = Tile<T>;
  using Off = TileOffsets<T, kWaves>;
  constexpr int kC = Off::kCopies;
  __shared__ __align__(1024) char Ks[TL::kBytes];
  __shared__ __align__(1024) char Vs[TL::kBytes];
  __shared__ SlotTable st;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, hl = lane >> 5;
  const QTileCoord c = query_tile_coord(p);
  const int64_t Lq = p.n_q * kChunk;
  const int64_t row0 = (static_cast<int64_t>(c.b) * p.H + c.h) * Lq;
  const int64_t qrow0 = row0 + c.t * kChunk;
  const int my_q = 32 * wave + li;

  Frag<T> qf[4];
  const T* q = static_cast<const T*>(p.q) + (qrow0 + my_q) * kDim;
#pragma unroll
  for (int s = 0; s < 4; ++s) qf[s].load(q + 16 * s + 8 * hl);
  if (wave == 0) fill_slot_table(st, p, c.g, c.b, c.t - p.shift);  // its loads beside the query's
  Off off;
  off.init(wave);
  __syncthreads();

  const int64_t kt0 = c.t - p.m > 0 ? c.t - p.m : 0;
  const int n_sw = static_cast<int>(c.t - kt0 + 1);
  const int n_items = n_sw + st.n;
  float* const lse_q = kLse ? p.lse + slot_vec_offset(p, c.gbh, c.t, 0) + my_q : nullptr;
  if (kLse) {  // invalid slots: -inf (before any copy, so the copy counts below stay exact)
    for (int e = tid; e < p.K * kChunk; e += kThreads)
      if (!((st.valid_mask >> (e / kChunk)) & 1u)) p.lse[slot_vec_offset(p, c.gbh, c.t, 0) + e] = -__builtin_inff();
  }
  auto item_tile = [&](const void* sw_base, const void* kv_base, int i) {
    if (i < n_sw) return static_cast<const T*>(sw_base) + (row0 + (kt0 + i) * kChunk) * kDim;
    return kv_tile<T>(kv_base, p, c.b, c.h, __builtin_amdgcn_readfirstlane(st.j[i - n_sw]));
  };
  off.copy(item_tile(p.k_sw, p.k, 0), Ks, wave);
  off.copy(item_tile(p.v_sw, p.v, 0), Vs, wave);
  barrier_copies_landed<kC>();  // K(0) landed and visible; V(0) may still be in flight
  // The query fragments are pinned here, before the loop, so that the compiler waits for them
  // once (left to their first use in the loop, its vmcnt waits would run in every iteration and
  // also wait for the prefetch copies in flight).
#pragma unroll
  for (int s = 0; s < 4; ++s) pin_in_registers(qf[s]);

  f32x16_t oacc[2] = {zero16(), zero16()};
  float m_run = -__builtin_inff(), l_run = 0.f;
  const float c2 = p.attn_scale * kLog2e;
  for (int i = 0; i < n_items; ++i) {
    const bool more = i + 1 < n_items, is_sw = i < n_sw;
    f32x16_t sacc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      sacc[tt] = zero16();
#pragma unroll
      for (int s = 0; s < 4; ++s) sacc[tt] = mma(off.kfrag(Ks, tt, s), qf[s], sacc[tt]);
    }
    barrier_lds_reads_done();  // every wave has read K(i)
    if (more) off.copy(item_tile(p.k_sw, p.k, i + 1), Ks, wave);
    Frag<T> pf[4];
    float lse_v = 0.f;
    int slot = 0;
    if (is_sw) {
      const int64_t kt = kt0 + i;
      const bool lower_edge = kt == c.t - p.m, diagonal = kt == c.t;
      if (lower_edge || diagonal) sw_mask_keys_major(sacc, 32 * wave, diagonal);
      float mx = -__builtin_inff();
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[tt][r]);
      mx = xor32_max(mx) * c2;
      constexpr float kLazy = 8.f;
      const bool grow = __ballot(mx > m_run + kLazy) != 0;
      const float m_new = grow ? fmaxf(m_run, mx) : m_run;
      const bool none = m_new == -__builtin_inff();
      const float alpha = none ? 1.f : fast_exp2(m_run - m_new);
      const float bias = none ? 0.f : -m_new;
      float l = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          x[e] = fast_exp2(__builtin_fmaf(sacc[s >> 1][8 * (s & 1) + e], c2, bias));
          l += x[e];
        }
        pf[s].set(x);
      }
      l_run = l_run * alpha + xor32_sum(l);
      m_run = m_new;
      if (grow) {
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
      }
    } else {
      slot = __builtin_amdgcn_readfirstlane(st.slot[i - n_sw]);
      const float w = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(st.w[i - n_sw])));
      float l;
      const float mx = tile_softmax(sacc, c2, l);
      lse_v = mx * p.attn_scale + __builtin_amdgcn_logf(l) * kLn2f;
      const float f = w * __builtin_amdgcn_rcpf(l);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = sacc[s >> 1][8 * (s & 1) + e] * f;
        pf[s].set(x);
      }
    }
    if (more) barrier_copies_landed<kC>();  // V(i) landed and visible (K(i + 1) may be in flight)
    else barrier_copies_landed<0>();
    const bool store = kLse && !is_sw;
    if (store && hl == 0) lse_q[slot * kChunk] = lse_v;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int s = 0; s < 4; ++s) oacc[dt] = mma(off.vfrag(Vs, s, dt), pf[s], oacc[dt]);
    if (is_sw && i + 1 == n_sw) {  // the window is complete: its output, normalized per query
      const float f = __builtin_amdgcn_rcpf(l_run);
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= f;
    }
    if (more) {
      barrier_lds_reads_done();  // every wave has read V(i)
      off.copy(item_tile(p.v_sw, p.v, i + 1), Vs, wave);
      if (store) barrier_copies_landed<kC + 1>();  // K(i + 1) landed (the lse store, V(i + 1) may not)
      else barrier_copies_landed<kC>();
    }
  }

  T* o = static_cast<T*>(p.o) + (qrow0 + my_q) * kDim;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a)
      store4(o + 32 * dt + 8 * a + 4 * hl, oacc[dt][4 * a], oacc[dt][4 * a + 1], oacc[dt][4 * a + 2],
             oacc[dt][4 * a + 3]);
  if (p.lse_sw && hl == 0) p.lse_sw[qrow0 + my_q] = m_run * kLn2f + __builtin_amdgcn_logf(l_run) * kLn2f;
}

// ------------------------------------------------ fused layer attention (window + GCA), backward
// Query-major pass of the fused layer: dq = dq_window + dq_gca for one 64-query tile (two waves
// of 32 queries, the pipeline of bwd_query_kernel: K double-buffered, V single).  The retrieved
// slots come first, as in bwd_query_kernel: each gives e_{t,k} = <dO_t, O_{t,k}>, writes the
// {bias, e} pairs and per-head sums of the key-major GCA pass, and adds its dQ.  Their weighted
// sum is <dO, o_gca>, so the window's D = <dO, o_window> = <dO, o> - sum_k w_k e_k comes from the
// stored fused output o without the window's own output.  Then the window's key tiles, as in
// sw_bwd_query_kernel, add dS K with dS = P (dP - D).  The window's key-major pass reads the
// biases -lse_sw log2 e and the -D written at the end.
template <typename T>
__global__ __launch_bounds__(kThreads) void fused_bwd_query_kernel(AttendParams p) {
  // the split-list counters of the key-major pass that follows start at zero
  if (blockIdx.x == 0 && threadIdx.x == 0 && p.long_ctl != nullptr) *p.long_ctl = 0;
  using TL = Tile<T>;
  using Off = TileOffsets<T, kWaves>;
  __shared__ __align__(1024) char Ka[TL::kBytes];
  __shared__ __align__(1024) char Kb[TL::kBytes];
  __shared__ __align__(1024) char Vs[TL::kBytes];
  __shared__ float dw_s[2][kMaxTopk];
  __shared__ SlotTable st;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, hl = lane >> 5;
  const QTileCoord c = query_tile_coord(p);
  const int64_t Lq = p.n_q * kChunk;
  const int64_t row0 = (static_cast<int64_t>(c.b) * p.H + c.h) * Lq;
  const int64_t qrow0 = row0 + c.t * kChunk;
  const int my_q = 32 * wave + li;
  const int64_t my_row = qrow0 + my_q;
  const int64_t row = c.t - p.shift;

  if (tid < 2 * kMaxTopk) dw_s[tid / kMaxTopk][tid % kMaxTopk] = 0.f;
  Frag<T> qf[4], df[4];
  float dd = 0.f;
  {
    Frag<T> of[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      qf[s].load(static_cast<const T*>(p.q) + my_row * kDim + 16 * s + 8 * hl);
      df[s].load(static_cast<const T*>(p.dout) + my_row * kDim + 16 * s + 8 * hl);
      of[s].load(static_cast<const T*>(p.o) + my_row * kDim + 16 * s + 8 * hl);
    }
    if (wave == 0) fill_slot_table(st, p, c.g, c.b, row);  // its loads beside the tiles'
#pragma unroll
    for (int s = 0; s < 4; ++s) dd += frag_dot(df[s], of[s]);
  }
  const float d_all = xor32_sum(dd);  // <dO, o> of this lane's query (fused output)
  const float bias_sw = -p.lse_sw[my_row] * kLog2e;
  Off off;
  off.init(wave);
  __syncthreads();

  const int nslots = st.n;
  if (c.h == 0 && row >= 0 && tid < p.K)
    p.wts[((static_cast<int64_t>(c.g) * p.B + c.b) * p.n_q + row) * p.K + tid] = st.w_all[tid];
  const float* lse_q = p.lse_in + slot_vec_offset(p, c.gbh, c.t, 0) + my_q;
  float* delta_q = p.delta + 2 * slot_vec_offset(p, c.gbh, c.t, 0) + 64 * hl + my_q;
  const int64_t kt0 = c.t - p.m > 0 ? c.t - p.m : 0;
  const int n_items = nslots + static_cast<int>(c.t - kt0 + 1);
  auto item_tile = [&](const void* kv_base, const void* sw_base, int i) {
    if (i < nslots) return kv_tile<T>(kv_base, p, c.b, c.h, __builtin_amdgcn_readfirstlane(st.j[i]));
    return static_cast<const T*>(sw_base) + (row0 + (kt0 + (i - nslots)) * kChunk) * kDim;
  };
  auto slot_of = [&](int n) { return __builtin_amdgcn_readfirstlane(st.slot[n]); };
  float lse_cur = 0.f;
  off.copy(item_tile(p.k, p.k_sw, 0), Ka, wave);
  off.copy(item_tile(p.v, p.v_sw, 0), Vs, wave);
  if (nslots > 0) lse_cur = lse_q[slot_of(0) * kChunk];
  barrier_copies_landed<0>();
  // The loads above are pinned here, before the loop, so that the compiler waits for them once:
  // left to their first use in the loop, its vmcnt waits would run in every iteration and also
  // wait for the untracked prefetch copies in flight.  Here they have all landed: the barrier
  // waited.
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    pin_in_registers(qf[s]);
    pin_in_registers(df[s]);
  }
  asm volatile("" : "+v"(lse_cur));
  float bias_sw_pinned = bias_sw;
  asm volatile("" : "+v"(bias_sw_pinned));

  f32x16_t dqacc[2] = {zero16(), zero16()};
  float d_gca = 0.f;  // sum over the slots of w_k e_k (this lane's query)
  const float c2 = p.attn_scale * kLog2e;
  auto step = [&](int i, char* const Kc, char* const Kn) {
    const bool more = i + 1 < n_items, is_gca = i < nslots;
    float lse_nxt = 0.f;
    if (more) {  // the other K buffer was released by the previous item's closing barrier
      off.copy(item_tile(p.k, p.k_sw, i + 1), Kn, wave);
      if (i + 1 < nslots) lse_nxt = lse_q[slot_of(i + 1) * kChunk];
    }
    f32x16_t sacc[2], pacc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      sacc[tt] = zero16();
      pacc[tt] = zero16();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        sacc[tt] = mma(off.kfrag(Kc, tt, s), qf[s], sacc[tt]);
        pacc[tt] = mma(off.kfrag(Vs, tt, s), df[s], pacc[tt]);
      }
    }
    barrier_lds_reads_done();  // every wave has read V(i)
    if (more) off.copy(item_tile(p.v, p.v_sw, i + 1), Vs, wave);
    Frag<T> zf[4];
    if (is_gca) {
      // P = exp(z - lse); e = sum_u P dP' = <dO, O_slot>; dz = w P (dP' - e)
      const int slot = slot_of(i);
      const float w = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(st.w[i])));
      const float bias = -lse_cur * kLog2e;
      float e0 = 0.f, e1 = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sacc[0][r] = fast_exp2(__builtin_fmaf(sacc[0][r], c2, bias));
        sacc[1][r] = fast_exp2(__builtin_fmaf(sacc[1][r], c2, bias));
        e0 = __builtin_fmaf(sacc[0][r], pacc[0][r], e0);
        e1 = __builtin_fmaf(sacc[1][r], pacc[1][r], e1);
      }
      const float e = xor32_sum(e0 + e1);
      d_gca = __builtin_fmaf(w, e, d_gca);
      delta_q[2 * slot * kChunk] = hl ? -e : __builtin_amdgcn_logf(w) + bias;
      const float es = sum_queries32(e);
      if (lane == 0) dw_s[wave][slot] = es;
      const float we = -w * e;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float x[8];
#pragma unroll
        for (int ee = 0; ee < 8; ++ee) {
          const int tt = s >> 1, r = 8 * (s & 1) + ee;
          x[ee] = sacc[tt][r] * __builtin_fmaf(w, pacc[tt][r], we);
        }
        zf[s].set(x);
      }
    } else {
      // the window's key tile kt: P = exp(z - lse_sw), dS = P (dP - D), masked on the edge tiles
      const int64_t kt = kt0 + (i - nslots);
      const bool lower_edge = kt == c.t - p.m, diagonal = kt == c.t;
      if (lower_edge || diagonal) sw_mask_keys_major(sacc, 32 * wave, diagonal);
      const float d_sw = d_all - d_gca;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float x[8];
#pragma unroll
        for (int ee = 0; ee < 8; ++ee) {
          const int tt = s >> 1, r = 8 * (s & 1) + ee;
          const float pw = fast_exp2(__builtin_fmaf(sacc[tt][r], c2, bias_sw_pinned));
          x[ee] = pw * (pacc[tt][r] - d_sw);
        }
        zf[s].set(x);
      }
    }
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int s = 0; s < 4; ++s) dqacc[dt] = mma(off.vfrag(Kc, s, dt), zf[s], dqacc[dt]);
    // K(i + 1), its lse and V(i + 1) landed (a slot's delta store may not have); every wave has
    // also read K(i), whose buffer the next item refills
    if (more) {
      if (is_gca) barrier_copies_landed_reads_done<1>();
      else barrier_copies_landed_reads_done<0>();
    }
    // lse_nxt has landed (the barrier's wait): the compiler's wait for it goes here, not later
    // (it also waits for the slot's delta store, which the barrier left in flight)
    asm volatile("" : "+v"(lse_nxt));
    lse_cur = lse_nxt;
  };
  for (int i = 0; i < n_items; i += 2) {
    step(i, Ka, Kb);
    if (i + 1 < n_items) step(i + 1, Kb, Ka);
  }

  T* dq = static_cast<T*>(p.dq) + my_row * kDim;
  const float sc = p.attn_scale;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a)
      store4(dq + 32 * dt + 8 * a + 4 * hl, sc * dqacc[dt][4 * a], sc * dqacc[dt][4 * a + 1],
             sc * dqacc[dt][4 * a + 2], sc * dqacc[dt][4 * a + 3]);
  p.sw_stats[2 * qrow0 + 64 * hl + my_q] = hl ? -(d_all - d_gca) : bias_sw;  // as the window pass
  __syncthreads();
  if (row >= 0 && tid < p.K) {
    const int64_t o = (((static_cast<int64_t>(c.g) * p.B + c.b) * p.n_q + row) * p.H + c.h) * p.K + tid;
    p.dw_part[o] = dw_s[0][tid] + dw_s[1][tid];
  }
}

}  // namespace

hipError_t launch_attend_fwd(const AttendParams& p, bool f32, hipStream_t s) {
  const int64_t blocks = static_cast<int64_t>(p.G) * p.B * p.H * p.n_q;
  if (blocks <= kWideMaxTiles) {  // too few query tiles to fill the chip: one slot per wave
    if (f32)
      hipLaunchKernelGGL(attend_fwd_wide_kernel<float>, dim3(static_cast<uint32_t>(2 * blocks)),
                         dim3(Wide<float>::kThreads), 0, s, p);
    else
      hipLaunchKernelGGL(attend_fwd_wide_kernel<bf16_t>, dim3(static_cast<uint32_t>(2 * blocks)),
                         dim3(Wide<bf16_t>::kThreads), 0, s, p);
    return hipGetLastError();
  }
  const dim3 grid(static_cast<uint32_t>(blocks));
  if (f32) {
    if (p.lse) hipLaunchKernelGGL((attend_fwd_kernel<float, true>), grid, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((attend_fwd_kernel<float, false>), grid, dim3(kThreads), 0, s, p);
  } else {
    if (p.lse) hipLaunchKernelGGL((attend_fwd_wave_kernel<true>), grid, dim3(64), 0, s, p);
    else hipLaunchKernelGGL((attend_fwd_wave_kernel<false>), grid, dim3(64), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_fused_fwd(const AttendParams& p, bool f32, hipStream_t s) {
  const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(p.G) * p.B * p.H * p.n_q));
  if (f32) {
    if (p.lse) hipLaunchKernelGGL((fused_fwd2_kernel<float, true>), grid, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((fused_fwd2_kernel<float, false>), grid, dim3(kThreads), 0, s, p);
  } else {
    if (p.lse) hipLaunchKernelGGL((fused_fwd_kernel<true>), grid, dim3(64), 0, s, p);
    else hipLaunchKernelGGL((fused_fwd_kernel<false>), grid, dim3(64), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_fused_bwd_query(const AttendParams& p, bool f32, hipStream_t s) {
  const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(p.G) * p.B * p.H * p.n_q));
  if (f32) hipLaunchKernelGGL(fused_bwd_query_kernel<float>, grid, dim3(kThreads), 0, s, p);
  else hipLaunchKernelGGL(fused_bwd_query_kernel<bf16_t>, grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_decode_tokens(const AttendParams& p, int32_t n_tok, bool f32, hipStream_t s) {
  const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(p.G) * p.B * p.H)), block(64 * kDecodeWaves);
  if (f32) hipLaunchKernelGGL(decode_tokens_kernel<float>, grid, block, 0, s, p, n_tok);
  else hipLaunchKernelGGL(decode_tokens_kernel<bf16_t>, grid, block, 0, s, p, n_tok);
  return hipGetLastError();
}

hipError_t launch_sw_fwd(const SwParams& p, bool f32, hipStream_t s) {
  const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(p.B) * p.H * p.n_c));
  if (f32) hipLaunchKernelGGL(sw_fwd2_kernel<float>, grid, dim3(kThreads), 0, s, p);
  else hipLaunchKernelGGL(sw_fwd_kernel, grid, dim3(64), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_sw_bwd_query(const SwParams& p, bool f32, hipStream_t s) {
  const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(p.B) * p.H * p.n_c));
  if (f32) hipLaunchKernelGGL(sw_bwd_query_kernel<float>, grid, dim3(kThreads), 0, s, p);
  else hipLaunchKernelGGL(sw_bwd_query_kernel<bf16_t>, grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_sw_bwd_key(const SwParams& p, bool f32, hipStream_t s) {
  const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(p.B) * p.H * p.n_c));
  if (f32) hipLaunchKernelGGL(sw_bwd_key_kernel<float>, grid, dim3(kThreads), 0, s, p);
  else hipLaunchKernelGGL(sw_bwd_key_kernel<bf16_t>, grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_inverse_index(const AttendParams& p, hipStream_t s) {
  const int64_t blocks = static_cast<int64_t>(p.B) * ((p.n_kv + 63) / 64);
  hipLaunchKernelGGL(inverse_index_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kIdxThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_bwd_query(const AttendParams& p, bool f32, hipStream_t s) {
  const int64_t blocks = static_cast<int64_t>(p.G) * p.B * p.H * p.n_q;
  if (f32)
    hipLaunchKernelGGL(bwd_query_kernel<float>, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(bwd_query_kernel<bf16_t>, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_bwd_key(const AttendParams& p, bool f32, hipStream_t s) {
  // the n_help segment walkers first, then one workgroup per (batch row, head, key chunk)
  const int64_t blocks = (p.long_ctl != nullptr ? p.n_help : 0) + static_cast<int64_t>(p.B) * p.H * p.n_kv;
  if (f32)
    hipLaunchKernelGGL(bwd_key_kernel<float>, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(bwd_key_kernel<bf16_t>, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_score_grad(const AttendParams& p, bool f32, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(p.G) * p.B * p.n_q;
  const int64_t blocks = (rows + 15) / 16;
  if (f32)
    hipLaunchKernelGGL(score_grad_kernel<float>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(score_grad_kernel<bf16_t>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace gca
