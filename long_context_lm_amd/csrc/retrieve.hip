// Causal chunk retrieval: exact landmark scores fused with a streaming top-k.
//
// [Notes, Key designs: causal retrieval]: the landmark of chunk i is scored against the
// landmark of every strictly earlier chunk j and the k best are kept.
// [Notes, Key designs: Gumbel top-k]: in training, Gumbel noise is added to the scores before
// the top-k; it only changes which chunks are selected.
//
// Each score is the float64 sequential sum over d of exact products lq[i,d] * lk[j,d]
// (bf16/fp32 products are exact in float64, so a fused multiply-add gives the same bits as a
// multiply followed by an add), rounded once to fp32 and multiplied by score_scale in fp32.
// The selection key packs the order-preserving image of the (possibly perturbed) fp32 score
// above the complement of j, so the largest key is the best score with the lowest j.  Key 0
// never occurs for a finite score and marks an empty slot.
//
// One workgroup scores one block of candidates of one row (cpt candidates per lane, one or four
// waves); each lane keeps a sorted list of its best keys, each wave extracts its top K with K
// rounds of a wave-wide maximum, and the wave lists are merged through LDS.  Rows with more candidates
// than one block are split over several workgroups whose partial top-K lists a second kernel
// merges (the 16M-token history: 262,144 candidates per row, 256 blocks of 1,024).
#include "gca_device.hpp"
#include "gca_internal.hpp"

namespace gca {
namespace {


// --------------------------------------------------------------- Philox4x64-10 (SC'11)
__device__ __forceinline__ uint64_t philox_word0(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                                 uint64_t k0, uint64_t k1) {
  constexpr uint64_t kM0 = 0xD2E7470EE14C6C93ull, kM1 = 0xCA5A826395121157ull;
  constexpr uint64_t kW0 = 0x9E3779B97F4A7C15ull, kW1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint64_t hi0 = __umul64hi(kM0, c0), lo0 = kM0 * c0;
    const uint64_t hi1 = __umul64hi(kM1, c2), lo1 = kM1 * c2;
    const uint64_t n0 = hi1 ^ c1 ^ k0;
    const uint64_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += kW0;
    k1 += kW1;
  }
  return c0;
}

// --------------------------------------------------------------- fixed-order logarithm
// ln(x) = e ln2 + 2 f (1 + z/3 + z^2/5 + ... + z^11/23), f = (m-1)/(m+1), z = f^2, with
// x = m 2^e and m in [sqrt(1/2), sqrt(2)).  Every operation is a single IEEE float64 rounding
// (no contraction into fused multiply-adds), so the result is a fixed function of x.
struct AtanhCoeffs {
  double c[12];
  constexpr AtanhCoeffs() : c() {
    for (int n = 0; n < 12; ++n) c[n] = 1.0 / static_cast<double>(2 * n + 1);
  }
};

__device__ __noinline__ double ln_fixed(double x) {
#pragma clang fp contract(off)
  constexpr AtanhCoeffs kC;
  constexpr double kSqrtHalf = 0x1.6a09e667f3bcdp-1;
  constexpr double kLn2 = 0x1.62e42fefa39efp-1;
  int e = 0;
  double m = frexp(x, &e);
  if (m < kSqrtHalf) {
    m = m * 2.0;
    e = e - 1;
  }
  const double f = (m - 1.0) / (m + 1.0);
  const double z = f * f;
  double p = kC.c[11];
#pragma unroll
  for (int n = 10; n >= 0; --n) p = p * z + kC.c[n];
  const double a = static_cast<double>(e) * kLn2;
  const double b = (2.0 * f) * p;
  return a + b;
}

__device__ float gumbel(uint64_t seed, int g, int b, int64_t i, int64_t j) {
  const uint64_t x = philox_word0(static_cast<uint64_t>(j), static_cast<uint64_t>(i),
                                  (static_cast<uint64_t>(g) << 32) | static_cast<uint32_t>(b), 0ull,
                                  seed, 0ull);
  const double u = (static_cast<double>(x >> 12) + 0.5) * 0x1.0p-52;
  const double y = -ln_fixed(-ln_fixed(u));
  return static_cast<float>(y);
}

__device__ __forceinline__ float canon_zero(float x) { return x == 0.f ? 0.f : x; }

__device__ __forceinline__ uint64_t make_key(float r, int64_t j) {
  const uint32_t u = __float_as_uint(r);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(ord) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(j));
}

__device__ __forceinline__ int32_t key_index(uint64_t key) {
  return key == 0 ? -1 : static_cast<int32_t>(~static_cast<uint32_t>(key));
}

// --------------------------------------------------------------- per-lane sorted list
// LL entries, at least min(K, entries the lane sees), so that no lane drops one of the K best.
template <int LL>
struct TopList {
  uint64_t key[LL];
  float s[LL];
  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int e = 0; e < LL; ++e) {
      key[e] = 0;
      s[e] = 0.f;
    }
  }
  // Insert keeping key[] descending; the smallest entry falls off the end.
  __device__ __forceinline__ void insert(uint64_t k, float sv) {
    if (k <= key[LL - 1]) return;
#pragma unroll
    for (int e = 0; e < LL; ++e) {
      const bool take = k > key[e];
      const uint64_t tk = key[e];
      const float ts = s[e];
      key[e] = take ? k : key[e];
      s[e] = take ? sv : s[e];
      k = take ? tk : k;
      sv = take ? ts : sv;
    }
  }
  __device__ __forceinline__ void pop() {
#pragma unroll
    for (int e = 0; e + 1 < LL; ++e) {
      key[e] = key[e + 1];
      s[e] = s[e + 1];
    }
    key[LL - 1] = 0;
  }
};

// Wave-wide maximum of a 32-bit value, in every lane.  Within each 16-lane row the partners come
// from DPP lane permutations (xor 1, xor 2, then the half-row and row mirrors, which act as xor 4
// and xor 8 once the quads agree); across rows from v_permlane16_swap / v_permlane32_swap.  No
// LDS traffic, so the K selection rounds are not bound by LDS latency.
// (Every lane has a source lane under these permutations; the zero "old" value and bound_ctrl
// let the compiler fold the move into the max as one v_max_u32_dpp.)
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), kCtrl, 0xf, 0xf, true));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = max(v, dpp_u32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = max(v, dpp_u32<0x141>(v));  // row_half_mirror
  v = max(v, dpp_u32<0x140>(v));  // row_mirror
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);  // rows 0<->1, 2<->3
  v = max(r[0], r[1]);
  const auto h = __builtin_amdgcn_permlane32_swap(v, v, false, false);  // halves
  return max(h[0], h[1]);
}

// Top K of the wave's lists; lane k (< K) returns the k-th best key and its clean score.  Each
// round finds the largest head key: first the largest high (score) word, then, only if several
// lanes share it, the largest low word (the lowest chunk index) among those lanes.  A finite score
// never has a zero high word and a chunk index never a zero low word, so zero marks an empty list.
template <int LL>
__device__ __forceinline__ void wave_topk(TopList<LL>& L, int K, uint64_t& my_key, float& my_s) {
  const int lane = threadIdx.x & 63;
  my_key = 0;
  my_s = 0.f;
  for (int k = 0; k < K; ++k) {
    const uint32_t hh = static_cast<uint32_t>(L.key[0] >> 32);
    const uint32_t hl = static_cast<uint32_t>(L.key[0]);
    const uint32_t mh = wave_max_u32(hh);
    if (mh == 0) break;  // wave-uniform: every list is empty
    const bool top = hh == mh;
    uint64_t hit = __ballot(top);
    if (__popcll(hit) > 1) {
      const uint32_t ml = wave_max_u32(top ? hl : 0u);
      hit = __ballot(top && hl == ml);
    }
    const int owner = __ffsll(static_cast<unsigned long long>(hit)) - 1;
    const uint32_t wl = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(hl), owner));
    const float sw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(L.s[0]), owner));
    if (lane == owner) L.pop();
    if (lane == k) {
      my_key = (static_cast<uint64_t>(mh) << 32) | wl;
      my_s = sw;
    }
  }
}

__device__ __forceinline__ double lmk_to_f64(const bf16_t* p, int d) { return static_cast<double>(to_f32(p[d])); }
__device__ __forceinline__ double lmk_to_f64(const float* p, int d) { return static_cast<double>(p[d]); }

// Key-landmark rows move through LDS so that global reads are whole-row coalesced while each lane
// still scores one row in dimension order.  A pass covers 64 consecutive rows (one per lane).
// Wave load k reads rows [kR, kR + R) as one contiguous span (lane i: 16-byte piece i % P of row
// kR + i / P); the pieces are written to the wave's LDS area and lane r then reads row r back.
// Piece p of row r sits in slot p ^ f(r), which keeps both the row-wide writes and the per-lane
// row reads free of bank conflicts (eight lanes of a row cover all slots; rows r and r + 8 use
// different slots).
template <typename T>
struct RowStage {
  static constexpr int P = kDim * static_cast<int>(sizeof(T)) / 16;  // 16-byte pieces per row
  static constexpr int R = 64 / P;                                   // rows per wave load
  static constexpr int kRowBytes = kDim * static_cast<int>(sizeof(T));
  u32x4_t v[P];

  __device__ static __forceinline__ int slot(int r, int piece) {
    const int f = P == 8 ? ((r & 7) ^ ((r >> 3) & 1)) : (r & (P - 1));
    return piece ^ f;
  }
  // Rows [row0, row0 + 64) of lk; rows at or beyond nrows are not read.
  __device__ __forceinline__ void load(const T* lk, int64_t row0, int64_t nrows, int lane) {
    const char* base = reinterpret_cast<const char*>(lk) + (lane % P) * 16;
#pragma unroll
    for (int k = 0; k < P; ++k) {
      const int64_t row = row0 + k * R + lane / P;
      if (row < nrows) v[k] = *reinterpret_cast<const u32x4_t*>(base + row * kRowBytes);
    }
  }
  __device__ __forceinline__ void store(u32x4_t* area, int lane) const {
#pragma unroll
    for (int k = 0; k < P; ++k) {
      const int r = k * R + lane / P;
      area[r * P + slot(r, lane % P)] = v[k];
    }
  }
};

// Exact sequential float64 dot product of row `lane` of the wave's LDS area with the query
// landmark (float64, in LDS).
__device__ __forceinline__ double row_dot(const u32x4_t* area, int lane, const double* lq_s, const bf16_t*) {
  using S = RowStage<bf16_t>;
  double acc = 0.0;
#pragma unroll
  for (int k = 0; k < S::P; ++k) {
    const u32x4_t c = area[lane * S::P + S::slot(lane, k)];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t pair = c[w];
      const double lo = static_cast<double>(__uint_as_float(pair << 16));
      const double hi = static_cast<double>(__uint_as_float(pair & 0xffff0000u));
      acc = __builtin_fma(lq_s[8 * k + 2 * w], lo, acc);
      acc = __builtin_fma(lq_s[8 * k + 2 * w + 1], hi, acc);
    }
  }
  return acc;
}

__device__ __forceinline__ double row_dot(const u32x4_t* area, int lane, const double* lq_s, const float*) {
  using S = RowStage<float>;
  double acc = 0.0;
#pragma unroll
  for (int k = 0; k < S::P; ++k) {
    const u32x4_t c = area[lane * S::P + S::slot(lane, k)];
#pragma unroll
    for (int w = 0; w < 4; ++w) acc = __builtin_fma(lq_s[4 * k + w], static_cast<double>(__uint_as_float(c[w])), acc);
  }
  return acc;
}

constexpr int kMergeThreads = 1024;      // sixteen waves per merged row
constexpr int kMergeWaves = kMergeThreads / 64;
constexpr int kMergeBatch = 8;           // partial entries each merge thread loads at once

// Merge the K-best lists of NWAVES waves (lane k < K of wave w holds entry k) through LDS; wave 0
// returns the top K of the union, lane k holding entry k.  Every thread of the workgroup calls it.
template <int NWAVES>
__device__ __forceinline__ void workgroup_topk(int K, uint64_t key, float sv, uint64_t* lkey, float* ls,
                                               uint64_t& out_key, float& out_s) {
  constexpr int kPerLane = (NWAVES * kMaxTopk + 63) / 64;  // entries each lane of wave 0 takes
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane < K) {
    lkey[wave * K + lane] = key;
    ls[wave * K + lane] = sv;
  }
  __syncthreads();
  out_key = 0;
  out_s = 0.f;
  if (wave == 0) {
    TopList<kPerLane> L;
    L.clear();
    for (int e = lane; e < NWAVES * K; e += 64)
      if (lkey[e] != 0) L.insert(lkey[e], ls[e]);
    wave_topk<kPerLane>(L, K, out_key, out_s);
  }
}

// One workgroup of NW waves per (row, block of 64 NW cpt candidates).  Pass n of wave w scores
// the 64 consecutive candidates starting at block start + 64 (NW n + w), one per lane.  NW = 4
// for a few long rows (a decode step over a long history: many blocks per row, their lists
// merged by the workgroup and then by topk_merge); NW = 1 for many short rows (training: one wave
// per row).  Short rows and fp32 rows load the next pass into registers while the current pass
// is scored: at most 128 VGPRs for bf16 landmarks and lists of 8 (four resident waves per SIMD),
// two waves otherwise.  Long bf16 rows keep two passes in flight per wave in an LDS ring (two
// workgroups per CU, which is what their grid of at most about two waves per SIMD fills).  Each
// lane's list holds LL = min(K, cpt) entries (rounded up to a power of two).
template <typename T, int LL, int NW>
__global__ __launch_bounds__(64 * NW, (sizeof(T) == 2 && LL <= 8 && NW == 1) ? 4 : 2) void score_topk_kernel(RetrieveParams p) {
  using Stage = RowStage<T>;
  constexpr int kBlockCand = 64 * NW;  // candidates of one block per pass (one per lane)
  // bf16 rows of a few long rows (a decode step) are copied straight into a two-stage LDS ring,
  // two passes in flight per wave (64 KiB per workgroup, two workgroups per CU); the others go
  // through registers, one pass ahead
  constexpr bool kRing = NW > 1 && sizeof(T) == 2;
  constexpr int kStages = kRing ? 2 : 1;
  __shared__ double lq_s[kDim];
  __shared__ u32x4_t rows_s[NW][kStages][64 * Stage::P];
  __shared__ uint64_t lkey[NW * kMaxTopk];
  __shared__ float ls[NW * kMaxTopk];
  const int lane = threadIdx.x & 63;
  const int wave = NW > 1 ? __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6)) : 0;
  const int64_t item = blockIdx.x;
  const int blk = static_cast<int>(item % p.nblk);
  const int64_t rowid = item / p.nblk;  // (g * B + b) * n_q + r
  const int64_t r = rowid % p.n_q;
  const int64_t gb = rowid / p.n_q;
  const int b = static_cast<int>(gb % p.B);
  const int g = static_cast<int>(gb / p.B);
  const int64_t i = p.base + r;
  const int64_t ncand = i < p.n_kv ? i : p.n_kv;

  TopList<LL> L;
  L.clear();
  const T* lk = static_cast<const T*>(p.lk) + gb * p.n_kv * kDim;
  const int64_t jw = static_cast<int64_t>(blk) * kBlockCand * p.cpt + 64 * wave;  // first row, pass 0
  int passes = 0;  // wave-uniform
  if (jw < ncand) {
    const int64_t m = (ncand - jw + kBlockCand - 1) / kBlockCand;
    passes = m < p.cpt ? static_cast<int>(m) : p.cpt;
  }
  auto score = [&](const u32x4_t* area, int64_t j0, const double* lqv) {
    const int64_t j = j0 + lane;
    if (j < ncand) {
      const double acc = row_dot(area, lane, lqv, static_cast<const T*>(nullptr));
      const float s = canon_zero(static_cast<float>(acc) * p.score_scale);
      float rkey = s;
      if (p.use_gumbel) {
#pragma clang fp contract(off)
        const float noise = p.tau * gumbel(p.seed, g, b, i, j);
        rkey = canon_zero(s + noise);
      }
      L.insert(make_key(rkey, j), s);
    }
  };

  if constexpr (kRing) {
    // Pass n's 64 rows go to stage n % 2.  Lane l's copy k lands at byte 16 l of the stage's
    // k-th KiB, which is slot l % P of row r = k R + l / P, so it fetches the piece that the
    // swizzle keeps in that slot.  Rows at or past ncand re-read row ncand - 1 (always a
    // candidate here); their scores are never used.
    auto issue = [&](int n, int stage) {  // wave-uniform
      const int64_t j0 = jw + static_cast<int64_t>(n) * kBlockCand;
      const char* g0 = reinterpret_cast<const char*>(lk + j0 * kDim);
      char* dst = reinterpret_cast<char*>(rows_s[wave][stage]);
      const int64_t last = ncand - 1 - j0;  // >= 0: every issued pass starts below ncand
#pragma unroll
      for (int k = 0; k < Stage::P; ++k) {
        const int r = k * Stage::R + lane / Stage::P;
        const int64_t row = r < last ? r : last;
        const uint32_t off = static_cast<uint32_t>(row * Stage::kRowBytes) + 16u * Stage::slot(r, lane % Stage::P);
        copy16_async_untracked(g0, off, dst + 1024 * k);
      }
    };
    if (passes > 0) issue(0, 0);
    if (passes > 1) issue(1, 1);
    if (threadIdx.x < kDim) lq_s[threadIdx.x] = lmk_to_f64(static_cast<const T*>(p.lq) + rowid * kDim, threadIdx.x);
    __syncthreads();
    // the query landmark stays in 128 registers (this variant runs two waves per SIMD), so a pass
    // reads only its rows from LDS
    double lqr[kDim];
#pragma unroll
    for (int d = 0; d < kDim; ++d) lqr[d] = lq_s[d];
    for (int n0 = 0; n0 < passes; n0 += 2) {
#pragma unroll
      for (int stage = 0; stage < 2; ++stage) {
        const int n = n0 + stage;
        if (n >= passes) break;  // wave-uniform
        // pass n landed (only pass n + 1, issued after it, may still be in flight)
        if (n + 1 < passes) wait_vm_outstanding<Stage::P>();
        else wait_vm_outstanding<0>();
        score(rows_s[wave][stage], jw + static_cast<int64_t>(n) * kBlockCand, lqr);
        // every read of this stage has returned (its values are used above): refill it
        if (n + 2 < passes) issue(n + 2, stage);
      }
    }
  } else {
    Stage st;
    if (passes > 0) st.load(lk, jw, ncand, lane);  // in flight while the query landmark is staged
    if (threadIdx.x < kDim) lq_s[threadIdx.x] = lmk_to_f64(static_cast<const T*>(p.lq) + rowid * kDim, threadIdx.x);
    __syncthreads();
    u32x4_t* area = rows_s[wave][0];
    for (int n = 0; n < passes; ++n) {
      const int64_t j0 = jw + static_cast<int64_t>(n) * kBlockCand;
      st.store(area, lane);
      if (n + 1 < passes) st.load(lk, j0 + kBlockCand, ncand, lane);
      // an opaque zero offset keeps the query landmark in LDS (read per candidate) instead of in
      // 128 registers hoisted out of the loop
      int zero = 0;
      asm volatile("" : "+v"(zero));
      score(area, j0, lq_s + zero);
    }
  }

  uint64_t key, bkey;
  float sv, bs;
  wave_topk<LL>(L, p.K, key, sv);
  if constexpr (NW > 1) {
    workgroup_topk<NW>(p.K, key, sv, lkey, ls, bkey, bs);
  } else {
    bkey = key;
    bs = sv;
  }
  if (p.nblk == 1) {
    if (threadIdx.x < p.K) {
      p.idx[rowid * p.K + lane] = key_index(bkey);
      p.score[rowid * p.K + lane] = bkey == 0 ? -__builtin_inff() : bs;
    }
    return;
  }

  if (threadIdx.x < p.K) {
    const int64_t o = (rowid * p.nblk + blk) * p.K + lane;
    p.part_key[o] = bkey;
    p.part_s[o] = bs;
  }
}

// One workgroup of sixteen waves per long row merges the row's nblk partial top-K lists; each
// thread loads its share of the entries in batches whose loads are in flight together.
// Each thread takes entries threadIdx.x + kMergeThreads e of the row's partial lists and keeps the
// best LL of them (LL = min(K, entries per thread), rounded up to a power of two).
template <int LL>
__global__ __launch_bounds__(kMergeThreads) void topk_merge_kernel(RetrieveParams p) {
  __shared__ uint64_t lkey[kMergeWaves * kMaxTopk];
  __shared__ float ls[kMergeWaves * kMaxTopk];
  const int64_t rowid = blockIdx.x;
  const int64_t n_in = static_cast<int64_t>(p.nblk) * p.K;
  const uint64_t* keys = p.part_key + rowid * n_in;
  const float* svals = p.part_s + rowid * n_in;
  TopList<LL> L;
  L.clear();
  for (int64_t c0 = threadIdx.x; c0 < n_in; c0 += static_cast<int64_t>(kMergeThreads) * kMergeBatch) {
    uint64_t kb[kMergeBatch];
    float sb[kMergeBatch];
#pragma unroll
    for (int e = 0; e < kMergeBatch; ++e) {
      const int64_t c = c0 + static_cast<int64_t>(e) * kMergeThreads;
      kb[e] = c < n_in ? keys[c] : 0;
      sb[e] = c < n_in ? svals[c] : 0.f;
    }
#pragma unroll
    for (int e = 0; e < kMergeBatch; ++e)
      if (kb[e] != 0) L.insert(kb[e], sb[e]);
  }
  uint64_t key, bkey;
  float sv, bs;
  wave_topk<LL>(L, p.K, key, sv);
  workgroup_topk<kMergeWaves>(p.K, key, sv, lkey, ls, bkey, bs);
  if (threadIdx.x < p.K) {
    p.idx[rowid * p.K + threadIdx.x] = key_index(bkey);
    p.score[rowid * p.K + threadIdx.x] = bkey == 0 ? -__builtin_inff() : bs;
  }
}

// Entries each lane's list needs: min(K, what the lane sees), as a power of two of at most 16.
int list_len(int K, int64_t per_lane) {
  const int cap = K <= 8 ? 8 : 16;
  int l = 1;
  while (l < per_lane && l < cap) l *= 2;
  return l;
}

template <typename T, int NW>
void launch_scan(const RetrieveParams& p, hipStream_t s) {
  const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(p.G) * p.B * p.n_q * p.nblk)), block(64 * NW);
  switch (list_len(p.K, p.cpt)) {
    case 1: hipLaunchKernelGGL((score_topk_kernel<T, 1, NW>), grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL((score_topk_kernel<T, 2, NW>), grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL((score_topk_kernel<T, 4, NW>), grid, block, 0, s, p); break;
    case 8: hipLaunchKernelGGL((score_topk_kernel<T, 8, NW>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((score_topk_kernel<T, 16, NW>), grid, block, 0, s, p); break;
  }
}

}  // namespace

hipError_t launch_score_topk(const RetrieveParams& p, bool f32, hipStream_t s) {
  if (f32) {
    if (p.nw == 1) launch_scan<float, 1>(p, s);
    else launch_scan<float, 4>(p, s);
  } else {
    if (p.nw == 1) launch_scan<bf16_t, 1>(p, s);
    else launch_scan<bf16_t, 4>(p, s);
  }
  return hipGetLastError();
}

hipError_t launch_topk_merge(const RetrieveParams& p, hipStream_t s) {
  const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(p.G) * p.B * p.n_q)), block(kMergeThreads);
  const int64_t n_in = static_cast<int64_t>(p.nblk) * p.K;
  switch (list_len(p.K, (n_in + kMergeThreads - 1) / kMergeThreads)) {
    case 1: hipLaunchKernelGGL((topk_merge_kernel<1>), grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL((topk_merge_kernel<2>), grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL((topk_merge_kernel<4>), grid, block, 0, s, p); break;
    case 8: hipLaunchKernelGGL((topk_merge_kernel<8>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((topk_merge_kernel<16>), grid, block, 0, s, p); break;
  }
  return hipGetLastError();
}

}  // namespace gca
