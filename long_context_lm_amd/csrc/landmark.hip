// Landmark gradients: the retrieval scores' gradients carried to the query and key landmarks.
//
// The retrieval scores weight the fused outputs, so the language-model loss differentiates
// them [Notes, Key designs: GCA]; a score relates the landmark of chunk i to the landmark of an
// earlier chunk j [Notes, Key designs: causal retrieval].  With s_ij = score_scale <lq_i, lk_j>
// (the float32 roundings of the canonical score carry no gradient) and the selection fixed:
//   dlq[g,b,r] = score_scale sum_k dscore[g,b,r,k] lk[g,b,idx[g,b,r,k]]
//   dlk[g,b,j] = score_scale sum over the retrievals (r, k) of chunk j, in (row, slot) order,
//                of dscore[g,b,r,k] lq[g,b,r]
// Both sums run in a fixed order, without atomics: dlk walks the inverse retrieval index (the
// lists of (group, row, slot) entries per key chunk) that the backward also uses, built here
// with every row included and d(score) as the entry value.  One wave per output row; lane d holds
// landmark dimension d, so every landmark row is read as one coalesced 128- or 256-byte piece.
#include "gca_device.hpp"
#include "gca_internal.hpp"

namespace gca {
namespace {

constexpr int kThreads = 256;  // four waves, each an independent output row
constexpr int kBatch = 4;      // gathered rows in flight together

template <typename T>
__global__ __launch_bounds__(kThreads) void lmk_query_grad_kernel(LandmarkParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t rowid = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  if (rowid >= static_cast<int64_t>(p.G) * p.B * p.n_q) return;  // whole wave
  const int64_t r = rowid % p.n_q;
  const int64_t gb = rowid / p.n_q;
  const int64_t limit = p.q_base + r < p.n_kv ? p.q_base + r : p.n_kv;  // candidates j < min(i, n_kv)
  const T* lk = static_cast<const T*>(p.lk) + gb * p.n_kv * kDim;
  float acc = 0.f;
  for (int k0 = 0; k0 < p.K; k0 += kBatch) {
    float x[kBatch], d[kBatch];
#pragma unroll
    for (int e = 0; e < kBatch; ++e) {
      const int k = k0 + e;
      const int32_t j = k < p.K ? __builtin_amdgcn_readfirstlane(p.idx[rowid * p.K + k]) : -1;
      const bool use = j >= 0 && j < limit;
      d[e] = use ? p.dscore[rowid * p.K + k] : 0.f;
      x[e] = use ? to_f32(lk[static_cast<int64_t>(j) * kDim + lane]) : 0.f;
    }
#pragma unroll
    for (int e = 0; e < kBatch; ++e) acc = __builtin_fmaf(d[e], x[e], acc);
  }
  from_f32(static_cast<T*>(p.dlq) + rowid * kDim + lane, acc * p.score_scale);
}

// The chunk's entry list is read 64 entries at a time, one per lane (one coalesced load), and
// the entries are then taken in list order from the lanes, eight row gathers in flight at once.
template <typename T>
__global__ __launch_bounds__(kThreads) void lmk_key_grad_kernel(LandmarkParams p) {
  constexpr int kGather = 8;
  const int lane = threadIdx.x & 63;
  const int64_t outid = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  if (outid >= static_cast<int64_t>(p.G) * p.B * p.n_kv) return;  // whole wave
  const int64_t j = outid % p.n_kv;
  const int64_t gb = outid / p.n_kv;
  const int b = static_cast<int>(gb % p.B);
  const int32_t g = static_cast<int32_t>(gb / p.B);
  const int64_t segment = static_cast<int64_t>(b) * p.n_kv + j;
  const int32_t count = p.counts[segment];
  const i32x2_t* list = reinterpret_cast<const i32x2_t*>(p.pairs) + segment * p.pair_cap;
  const T* lq = static_cast<const T*>(p.lq) + gb * p.n_q * kDim;
  const int32_t nqk = static_cast<int32_t>(p.n_q) * p.K;  // entry code = (g n_q + row) K + slot
  float acc = 0.f;
  for (int32_t e0 = 0; e0 < count; e0 += 64) {
    const int32_t n = count - e0 < 64 ? count - e0 : 64;
    // lane e: entry e0 + e, decoded; entries are grouped by g, rows ascending; j < q_base + row
    int32_t row = 0;
    float d = 0.f;
    if (lane < n) {
      const i32x2_t ent = list[e0 + lane];
      row = (ent[0] % nqk) / p.K;
      if (ent[0] / nqk == g && j < p.q_base + row) d = __int_as_float(ent[1]);
    }
    for (int32_t e = 0; e < n; e += kGather) {
      float x[kGather], dd[kGather];
#pragma unroll
      for (int u = 0; u < kGather; ++u) {
        const int src = e + u < n ? e + u : 0;
        dd[u] = e + u < n ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(d), src)) : 0.f;
        const int32_t r = __builtin_amdgcn_readlane(row, src);
        x[u] = dd[u] != 0.f ? to_f32(lq[static_cast<int64_t>(r) * kDim + lane]) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kGather; ++u) acc = __builtin_fmaf(dd[u], x[u], acc);
    }
  }
  from_f32(static_cast<T*>(p.dlk) + outid * kDim + lane, acc * p.score_scale);
}

}  // namespace

hipError_t launch_lmk_query_grad(const LandmarkParams& p, bool f32, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(p.G) * p.B * p.n_q;
  const dim3 grid(static_cast<uint32_t>((rows + 3) / 4));
  if (f32) hipLaunchKernelGGL(lmk_query_grad_kernel<float>, grid, dim3(kThreads), 0, s, p);
  else hipLaunchKernelGGL(lmk_query_grad_kernel<bf16_t>, grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_lmk_key_grad(const LandmarkParams& p, bool f32, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(p.G) * p.B * p.n_kv;
  const dim3 grid(static_cast<uint32_t>((rows + 3) / 4));
  if (f32) hipLaunchKernelGGL(lmk_key_grad_kernel<float>, grid, dim3(kThreads), 0, s, p);
  else hipLaunchKernelGGL(lmk_key_grad_kernel<bf16_t>, grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace gca
