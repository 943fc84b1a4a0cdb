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
// One wave scores one block of candidates of one row (cpt candidates per lane); each lane keeps
// a sorted list of its best keys and the wave extracts the top K with K rounds of a wave-wide
// maximum.  Rows with more candidates than one block are split over several waves whose partial
// top-K lists a second kernel merges (the 16M-token history: 262,144 candidates per row).
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
template <int KL>
struct TopList {
  uint64_t key[KL];
  float s[KL];
  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int e = 0; e < KL; ++e) {
      key[e] = 0;
      s[e] = 0.f;
    }
  }
  // Insert keeping key[] descending; the smallest entry falls off the end.
  __device__ __forceinline__ void insert(uint64_t k, float sv) {
    if (k <= key[KL - 1]) return;
#pragma unroll
    for (int e = 0; e < KL; ++e) {
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
    for (int e = 0; e + 1 < KL; ++e) {
      key[e] = key[e + 1];
      s[e] = s[e + 1];
    }
    key[KL - 1] = 0;
  }
};

// Wave-wide maximum of a 64-bit key, in every lane.  Within each 16-lane row the partners come
// from DPP lane permutations (xor 1, xor 2, then the half-row and row mirrors, which act as xor 4
// and xor 8 once the quads agree); across rows from v_permlane16_swap / v_permlane32_swap.  No
// LDS traffic, so the K selection rounds are not bound by LDS latency.
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <int kCtrl>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const int lo = __builtin_amdgcn_mov_dpp(static_cast<int>(v), kCtrl, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_mov_dpp(static_cast<int>(v >> 32), kCtrl, 0xf, 0xf, false);
  return (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
}

__device__ __forceinline__ uint64_t swap_max_u64(uint64_t v, bool rows16) {
  const uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
  auto l = rows16 ? __builtin_amdgcn_permlane16_swap(lo, lo, false, false)
                  : __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  auto h = rows16 ? __builtin_amdgcn_permlane16_swap(hi, hi, false, false)
                  : __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  const uint64_t a = (static_cast<uint64_t>(h[0]) << 32) | l[0];
  const uint64_t b = (static_cast<uint64_t>(h[1]) << 32) | l[1];
  return max_u64(a, b);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = max_u64(v, dpp_u64<0xB1>(v));   // quad_perm [1,0,3,2]
  v = max_u64(v, dpp_u64<0x4E>(v));   // quad_perm [2,3,0,1]
  v = max_u64(v, dpp_u64<0x141>(v));  // row_half_mirror
  v = max_u64(v, dpp_u64<0x140>(v));  // row_mirror
  v = swap_max_u64(v, true);          // rows 0<->1, 2<->3
  v = swap_max_u64(v, false);         // halves
  return v;
}

// Top K of the wave's lists; lane k (< K) returns the k-th best key and its clean score.
template <int KL>
__device__ __forceinline__ void wave_topk(TopList<KL>& L, int K, uint64_t& my_key, float& my_s) {
  const int lane = threadIdx.x & 63;
  my_key = 0;
  my_s = 0.f;
  for (int k = 0; k < K; ++k) {
    const uint64_t m = wave_max_u64(L.key[0]);
    if (m == 0) break;  // wave-uniform
    const uint64_t hit = __ballot(L.key[0] == m);
    const int owner = __ffsll(static_cast<unsigned long long>(hit)) - 1;
    const float sw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(L.s[0]), owner));
    if (lane == owner) L.pop();
    if (lane == k) {
      my_key = m;
      my_s = sw;
    }
  }
}

__device__ __forceinline__ double lmk_to_f64(const bf16_t* p, int d) { return static_cast<double>(to_f32(p[d])); }
__device__ __forceinline__ double lmk_to_f64(const float* p, int d) { return static_cast<double>(p[d]); }

// Exact sequential float64 dot product of one key landmark row with the query row in LDS.
template <typename T>
__device__ __forceinline__ double landmark_dot(const T* __restrict__ row, const double* lq_s);

template <>
__device__ __forceinline__ double landmark_dot<bf16_t>(const bf16_t* __restrict__ row, const double* lq_s) {
  const u32x4_t* r4 = reinterpret_cast<const u32x4_t*>(row);
  u32x4_t chunk[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) chunk[c] = r4[c];
  double acc = 0.0;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t pair = chunk[c][w];
      const double lo = static_cast<double>(__uint_as_float(pair << 16));
      const double hi = static_cast<double>(__uint_as_float(pair & 0xffff0000u));
      acc = __builtin_fma(lq_s[8 * c + 2 * w], lo, acc);
      acc = __builtin_fma(lq_s[8 * c + 2 * w + 1], hi, acc);
    }
  }
  return acc;
}

template <>
__device__ __forceinline__ double landmark_dot<float>(const float* __restrict__ row, const double* lq_s) {
  const f32x4_t* r4 = reinterpret_cast<const f32x4_t*>(row);
  double acc = 0.0;
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const f32x4_t x = r4[c];
#pragma unroll
    for (int w = 0; w < 4; ++w) acc = __builtin_fma(lq_s[4 * c + w], static_cast<double>(x[w]), acc);
  }
  return acc;
}

constexpr int kThreads = 256;  // four waves, each an independent work item

// One wave per (row, candidate block).
template <typename T, int KL>
__global__ __launch_bounds__(kThreads) void score_topk_kernel(RetrieveParams p) {
  __shared__ double lq_all[kThreads / 64][kDim];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + wave;
  const int64_t n_items = static_cast<int64_t>(p.G) * p.B * p.n_q * p.nblk;
  if (item >= n_items) return;  // whole wave; no workgroup barrier below
  const int blk = static_cast<int>(item % p.nblk);
  const int64_t rowid = item / p.nblk;  // (g * B + b) * n_q + r
  const int64_t r = rowid % p.n_q;
  const int64_t gb = rowid / p.n_q;
  const int b = static_cast<int>(gb % p.B);
  const int g = static_cast<int>(gb / p.B);
  const int64_t i = p.base + r;
  const int64_t ncand = i < p.n_kv ? i : p.n_kv;

  double* lq_s = lq_all[wave];
  lq_s[lane] = lmk_to_f64(static_cast<const T*>(p.lq) + rowid * kDim, lane);
  __builtin_amdgcn_wave_barrier();

  TopList<KL> L;
  L.clear();
  const T* lk = static_cast<const T*>(p.lk) + gb * p.n_kv * kDim;
  const int64_t j0 = static_cast<int64_t>(blk) * 64 * p.cpt;
  for (int n = 0; n < p.cpt; ++n) {
    const int64_t j = j0 + static_cast<int64_t>(n) * 64 + lane;
    if (j >= ncand) break;
    const double acc = landmark_dot<T>(lk + j * kDim, lq_s);
    const float s = canon_zero(static_cast<float>(acc) * p.score_scale);
    float rkey = s;
    if (p.use_gumbel) {
#pragma clang fp contract(off)
      const float noise = p.tau * gumbel(p.seed, g, b, i, j);
      rkey = canon_zero(s + noise);
    }
    L.insert(make_key(rkey, j), s);
  }

  uint64_t key;
  float sv;
  wave_topk<KL>(L, p.K, key, sv);
  if (lane < p.K) {
    if (p.nblk == 1) {
      p.idx[rowid * p.K + lane] = key_index(key);
      p.score[rowid * p.K + lane] = key == 0 ? -__builtin_inff() : sv;
    } else {
      const int64_t o = (rowid * p.nblk + blk) * p.K + lane;
      p.part_key[o] = key;
      p.part_s[o] = sv;
    }
  }
}

// One wave per row: merge the row's nblk partial top-K lists.
template <int KL>
__global__ __launch_bounds__(kThreads) void topk_merge_kernel(RetrieveParams p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t rowid = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + wave;
  if (rowid >= static_cast<int64_t>(p.G) * p.B * p.n_q) return;
  const int64_t n_in = static_cast<int64_t>(p.nblk) * p.K;
  const uint64_t* keys = p.part_key + rowid * n_in;
  const float* svals = p.part_s + rowid * n_in;
  TopList<KL> L;
  L.clear();
  for (int64_t c = lane; c < n_in; c += 64) L.insert(keys[c], svals[c]);
  uint64_t key;
  float sv;
  wave_topk<KL>(L, p.K, key, sv);
  if (lane < p.K) {
    p.idx[rowid * p.K + lane] = key_index(key);
    p.score[rowid * p.K + lane] = key == 0 ? -__builtin_inff() : sv;
  }
}

}  // namespace

hipError_t launch_score_topk(const RetrieveParams& p, bool f32, hipStream_t s) {
  const int64_t items = static_cast<int64_t>(p.G) * p.B * p.n_q * p.nblk;
  const dim3 grid(static_cast<uint32_t>((items + 3) / 4));
  const bool small = p.K <= 8;
  if (f32) {
    if (small) hipLaunchKernelGGL((score_topk_kernel<float, 8>), grid, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((score_topk_kernel<float, 16>), grid, dim3(kThreads), 0, s, p);
  } else {
    if (small) hipLaunchKernelGGL((score_topk_kernel<bf16_t, 8>), grid, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((score_topk_kernel<bf16_t, 16>), grid, dim3(kThreads), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_topk_merge(const RetrieveParams& p, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(p.G) * p.B * p.n_q;
  const dim3 grid(static_cast<uint32_t>((rows + 3) / 4));
  if (p.K <= 8) hipLaunchKernelGGL((topk_merge_kernel<8>), grid, dim3(kThreads), 0, s, p);
  else hipLaunchKernelGGL((topk_merge_kernel<16>), grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace gca
