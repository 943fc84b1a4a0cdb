// C ABI of the GCA library: argument validation, workspace carving and kernel launches on the
// caller's stream.  No allocation, no synchronisation, no state between calls (the optional
// kernel timer aside).
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/gca.h"
#include "gca_internal.hpp"

namespace gca {

const char* kernel_name(int id) {
  static const char* names[kNumKernels] = {"score_topk", "topk_merge", "attend_fwd",     "inverse_index",
                                           "bwd_query",  "bwd_key",    "score_grad",     "lmk_query_grad",
                                           "lmk_key_grad", "fetch_chunks", "decode_tokens", "sw_fwd",
                                           "sw_bwd_query", "sw_bwd_key", "fused_fwd", "fused_bwd_query"};
  return (id >= 0 && id < kNumKernels) ? names[id] : "unknown";
}

namespace {

thread_local int t_last_hip_error = 0;

struct ProfRecord {
  int kernel;
  hipEvent_t start, stop;
};
struct ProfState {
  bool on = false;
  std::vector<ProfRecord> records;
};
thread_local ProfState t_prof;

// Retrieval: one workgroup of nw waves scores a block of 64 nw cpt candidates of one row (one
// candidate per lane per pass).  Many rows (training) take one wave per block; few rows (a decode
// step) take four, so that a long history still gives enough waves.  cpt starts at 1 and doubles
// while the grid would exceed kRetrieveMaxWaves waves and a row still spans several blocks; rows
// spanning several blocks are merged by a second kernel.  The 16M-token history (262,144
// candidates per row, two rows) runs as 512 workgroups of four waves, four candidates per lane
// (two resident per CU, all loads in flight at once): half the partial lists of a 4,096-wave
// grid, which the merge pays for, at the same scan time.  The 16K training step runs as 4,096
// single waves of four candidates per lane (one block per row, whatever the cap).
constexpr int64_t kRetrieveMaxWaves = 2048;
constexpr int64_t kRetrieveManyRows = 1024;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Launch `fn` and, when the timer is on, bracket it with events on `stream`.
template <typename F>
gca_status launch(int kernel, hipStream_t stream, F fn) {
  hipEvent_t a = nullptr, b = nullptr;
  if (t_prof.on) {
    if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess ||
        hipEventRecord(a, stream) != hipSuccess) {
      t_last_hip_error = static_cast<int>(hipGetLastError());
      return GCA_ERR_HIP;
    }
  }
  const hipError_t err = fn();
  if (err != hipSuccess) {
    t_last_hip_error = static_cast<int>(err);
    return GCA_ERR_HIP;
  }
  if (t_prof.on) {
    if (hipEventRecord(b, stream) != hipSuccess) {
      t_last_hip_error = static_cast<int>(hipGetLastError());
      return GCA_ERR_HIP;
    }
    t_prof.records.push_back({kernel, a, b});
  }
  return GCA_OK;
}

gca_status validate_problem(const gca_problem* p) {
  if (p == nullptr) return GCA_ERR_INVALID_ARGUMENT;
  if (p->B < 1 || p->G < 1 || p->H < 1) return GCA_ERR_INVALID_ARGUMENT;
  if (p->n_q_chunks < 0 || p->q_chunk_base < 0 || p->n_kv_chunks < 0) return GCA_ERR_INVALID_ARGUMENT;
  if (p->topk < 1) return GCA_ERR_INVALID_ARGUMENT;
  if (p->dtype != GCA_BF16 && p->dtype != GCA_F32) return GCA_ERR_INVALID_ARGUMENT;
  if (p->use_gumbel != 0 && p->use_gumbel != 1) return GCA_ERR_INVALID_ARGUMENT;
  if (p->shift != 0 && p->shift != 1) return GCA_ERR_INVALID_ARGUMENT;
  if (p->reserved != 0) return GCA_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(p->attn_scale) || !std::isfinite(p->score_scale)) return GCA_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(p->gumbel_tau) || p->gumbel_tau < 0.f) return GCA_ERR_INVALID_ARGUMENT;
  if (p->S != 64 || p->d_head != 64 || p->d_lmk != 64) return GCA_ERR_UNSUPPORTED;
  if (p->topk > 16) return GCA_ERR_UNSUPPORTED;
  if (p->G > (1 << 26)) return GCA_ERR_UNSUPPORTED;  // (group, slot) travels as 16 g + slot in int32
  // index ranges: chunk ids travel as int32, grids as 32-bit block counts
  const int64_t big = (int64_t{1} << 31) - 1;
  if (p->n_kv_chunks > big || p->q_chunk_base + p->n_q_chunks > big) return GCA_ERR_UNSUPPORTED;
  const int64_t gbh = static_cast<int64_t>(p->G) * p->B * p->H;
  if (p->n_q_chunks > 0 && gbh > big / p->n_q_chunks) return GCA_ERR_UNSUPPORTED;
  // (the key-major pass launches up to 1024 more workgroups than B H n_kv)
  if (p->n_kv_chunks > 0 && static_cast<int64_t>(p->B) * p->H > (big - 1024) / p->n_kv_chunks)
    return GCA_ERR_UNSUPPORTED;
  // (group, row, slot) codes of the inverse index travel as int32
  if (static_cast<int64_t>(p->G) * p->n_q_chunks * p->topk > big) return GCA_ERR_UNSUPPORTED;
  // so do the split lists' segment slots: at most B (ceil(L / kSegEntries) + L / (kSplitMin + 1)),
  // L = G n_q K, which is below B (L / 32 + 2)
  if (static_cast<int64_t>(p->B) * (static_cast<int64_t>(p->G) * p->n_q_chunks * p->topk / 32 + 2) > big)
    return GCA_ERR_UNSUPPORTED;
  return GCA_OK;
}

struct RetrievePlan {
  int32_t nblk, cpt, nw;
  size_t ws;
};

RetrievePlan plan_retrieve(const gca_problem* p) {
  RetrievePlan r{1, 1, 4, 0};
  if (p->n_q_chunks == 0) return r;
  const int64_t last_row = p->q_chunk_base + p->n_q_chunks - 1;
  const int64_t max_cand = last_row < p->n_kv_chunks ? last_row : p->n_kv_chunks;
  const int64_t rows = static_cast<int64_t>(p->G) * p->B * p->n_q_chunks;
  const int64_t nw = rows >= kRetrieveManyRows ? 1 : 4;
  const int64_t block = 64 * nw;
  int64_t cpt = 1;
  int64_t nblk = max_cand > 0 ? (max_cand + block - 1) / block : 1;
  while (nblk > 1 && rows * nblk * nw > kRetrieveMaxWaves) {
    cpt *= 2;
    nblk = (max_cand + block * cpt - 1) / (block * cpt);
  }
  r.nblk = static_cast<int32_t>(nblk);
  r.cpt = static_cast<int32_t>(cpt);
  r.nw = static_cast<int32_t>(nw);
  if (nblk > 1) {
    const size_t n = static_cast<size_t>(rows) * nblk * p->topk;
    r.ws = align_up(n * sizeof(uint64_t)) + align_up(n * sizeof(float));
  }
  return r;
}

// Landmark gradients: the inverse retrieval index (entry lists per key chunk) and its counts.
struct LandmarkLayout {
  size_t pairs, counts, total;
};

LandmarkLayout plan_landmark(const gca_problem* p) {
  LandmarkLayout l{};
  if (p->n_kv_chunks == 0) return l;  // no key landmarks: only dlq (zeros or gathers) is written
  const size_t G = p->G, B = p->B;
  const size_t nq = static_cast<size_t>(p->n_q_chunks), nkv = static_cast<size_t>(p->n_kv_chunks);
  size_t off = 0;
  l.pairs = off;
  off += align_up(B * nkv * G * nq * 2 * sizeof(int32_t));
  l.counts = off;
  off += align_up(B * nkv * sizeof(int32_t));
  l.total = off;
  return l;
}

struct BackwardLayout {
  size_t delta, dw_part, wts, pairs, counts, long_ctl, long_list, long_seg, long_part, total;
  int64_t long_cap, seg_cap;  // 0: no list can be long, nothing is split
};

BackwardLayout plan_backward(const gca_problem* p) {
  BackwardLayout l{};
  if (p->n_q_chunks == 0 && p->n_kv_chunks == 0) return l;  // nothing to compute or write
  const size_t G = p->G, B = p->B, H = p->H, K = p->topk;
  const size_t nq = static_cast<size_t>(p->n_q_chunks), nkv = static_cast<size_t>(p->n_kv_chunks);
  size_t off = 0;
  l.delta = off;
  off += align_up(G * B * H * nq * 64 * K * 2 * sizeof(float));  // bias and -e per (token, slot)
  l.dw_part = off;
  off += align_up(G * B * nq * H * K * sizeof(float));
  l.wts = off;
  off += align_up(G * B * nq * K * sizeof(float));
  l.pairs = off;
  off += align_up(B * nkv * G * nq * 2 * sizeof(int32_t));
  l.counts = off;
  off += align_up(B * nkv * sizeof(int32_t));
  // Split lists.  A batch row holds at most L = G n_q K entries (each retrieval row names at most
  // K chunks), so at most floor(L / (T + 1)) of its chunks exceed T = kSplitMin entries, and their
  // segments of E = kSegEntries number at most ceil(L / E) + that many.
  const int64_t L = static_cast<int64_t>(G * nq * K);
  if (nkv > 0 && L > kSplitMin) {
    l.long_cap = static_cast<int64_t>(B) * (L / (kSplitMin + 1));
    l.seg_cap = static_cast<int64_t>(B) * ((L + kSegEntries - 1) / kSegEntries + L / (kSplitMin + 1));
    l.long_ctl = off;
    off += align_up(sizeof(uint64_t));
    l.long_list = off;
    off += align_up(static_cast<size_t>(l.long_cap) * 4 * sizeof(int32_t));
    l.long_seg = off;
    off += align_up(static_cast<size_t>(l.seg_cap) * sizeof(int32_t));
    l.long_part = off;
    off += align_up(static_cast<size_t>(l.seg_cap) * H * 2 * 64 * 64 * sizeof(float));
  }
  l.total = off;
  return l;
}

// Points the key-major pass at the split-list areas of the backward workspace (when a list can
// be long and a query-major pass runs first to clear the counter).
void set_long_lists(AttendParams& a, const BackwardLayout& L, char* w, bool any) {
  if (L.seg_cap == 0 || !any) return;
  a.long_ctl = reinterpret_cast<uint64_t*>(w + L.long_ctl);
  a.long_list = reinterpret_cast<int32_t*>(w + L.long_list);
  a.long_seg = reinterpret_cast<int32_t*>(w + L.long_seg);
  a.long_part = reinterpret_cast<float*>(w + L.long_part);
  a.long_cap = static_cast<int32_t>(L.long_cap);
  a.seg_cap = static_cast<int32_t>(L.seg_cap);
  const int64_t items = L.seg_cap * a.H;  // the most segment walks a call can have
  const int64_t help = items < 1024 ? items : 1024;
  a.n_help = static_cast<int32_t>((help + 7) / 8 * 8);  // a multiple of 8: see bwd_key_kernel
}

gca_status check_ws(size_t need, const void* ws, size_t ws_bytes) {
  if (ws_bytes < need) return GCA_ERR_WORKSPACE_TOO_SMALL;
  if (need > 0 && ws == nullptr) return GCA_ERR_INVALID_ARGUMENT;
  if (need > 0 && !aligned(ws, kAlign)) return GCA_ERR_MISALIGNED;
  return GCA_OK;
}

gca_status check_tensor(const void* ptr, bool nonempty, uintptr_t align) {
  if (!nonempty) return GCA_OK;
  if (ptr == nullptr) return GCA_ERR_INVALID_ARGUMENT;
  if (!aligned(ptr, align)) return GCA_ERR_MISALIGNED;
  return GCA_OK;
}

#define GCA_TRY(expr)                   \
  do {                                  \
    const gca_status _s = (expr);       \
    if (_s != GCA_OK) return _s;        \
  } while (0)

AttendParams attend_params(const gca_problem* p) {
  AttendParams a{};
  a.n_q = p->n_q_chunks;
  a.n_kv = p->n_kv_chunks;
  a.G = p->G;
  a.B = p->B;
  a.H = p->H;
  a.K = p->topk;
  a.shift = p->shift;
  a.q_base = p->q_chunk_base;
  a.pair_cap = static_cast<int32_t>(static_cast<int64_t>(p->G) * p->n_q_chunks);
  a.attn_scale = p->attn_scale;
  return a;
}

}  // namespace
}  // namespace gca

using namespace gca;

extern "C" {

gca_status gca_workspace_size(int op, const gca_problem* problem, size_t* bytes) {
  if (bytes == nullptr) return GCA_ERR_INVALID_ARGUMENT;
  GCA_TRY(validate_problem(problem));
  switch (op) {
    case GCA_OP_RETRIEVE: *bytes = plan_retrieve(problem).ws; return GCA_OK;
    case GCA_OP_FORWARD: *bytes = 0; return GCA_OK;
    case GCA_OP_BACKWARD:
      *bytes = plan_backward(problem).total;
      return GCA_OK;
    case GCA_OP_LANDMARK_BACKWARD: *bytes = plan_landmark(problem).total; return GCA_OK;
    case GCA_OP_SW_BACKWARD:
      *bytes = align_up(static_cast<size_t>(problem->B) * problem->H * problem->n_q_chunks * 64 * 8);
      return GCA_OK;
    case GCA_OP_FUSED_BACKWARD:
      *bytes = plan_backward(problem).total +
               align_up(static_cast<size_t>(problem->B) * problem->H * problem->n_q_chunks * 64 * 8);
      return GCA_OK;
    default: return GCA_ERR_INVALID_ARGUMENT;
  }
}

}  // extern "C"

namespace gca {
namespace {

gca_status retrieve_check(const gca_problem* p, const void* lq, const void* lk, const int32_t* idx,
                          const float* score) {
  GCA_TRY(validate_problem(p));
  const bool any = p->n_q_chunks > 0;
  GCA_TRY(check_tensor(lq, any, 16));
  GCA_TRY(check_tensor(lk, any && p->n_kv_chunks > 0, 16));
  GCA_TRY(check_tensor(idx, any, 4));
  GCA_TRY(check_tensor(score, any, 4));
  return GCA_OK;
}

// The launches of a retrieval whose arguments passed retrieve_check, with a workspace of at least
// plan.ws bytes at ws.
gca_status retrieve_launch(const gca_problem* p, const RetrievePlan& plan, const void* lq, const void* lk,
                           int32_t* idx, float* score, void* ws, void* stream) {
  if (p->n_q_chunks == 0) return GCA_OK;

  RetrieveParams rp{};
  rp.lq = lq;
  rp.lk = lk;
  rp.idx = idx;
  rp.score = score;
  rp.n_q = p->n_q_chunks;
  rp.base = p->q_chunk_base;
  rp.n_kv = p->n_kv_chunks;
  rp.G = p->G;
  rp.B = p->B;
  rp.K = p->topk;
  rp.nblk = plan.nblk;
  rp.cpt = plan.cpt;
  rp.nw = plan.nw;
  rp.score_scale = p->score_scale;
  rp.use_gumbel = p->use_gumbel;
  rp.seed = p->seed;
  rp.tau = p->gumbel_tau;
  if (plan.nblk > 1) {
    const size_t n = static_cast<size_t>(p->G) * p->B * p->n_q_chunks * plan.nblk * p->topk;
    rp.part_key = static_cast<uint64_t*>(ws);
    rp.part_s = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up(n * sizeof(uint64_t)));
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool f32 = p->dtype == GCA_F32;
  GCA_TRY(launch(kScoreTopk, s, [&] { return launch_score_topk(rp, f32, s); }));
  if (plan.nblk > 1) GCA_TRY(launch(kTopkMerge, s, [&] { return launch_topk_merge(rp, s); }));
  return GCA_OK;
}

// Scratch of gca_retrieve_static: the partial top-k lists of rows that span several scan blocks.
// The scan grid is capped at kRetrieveMaxWaves waves, so a problem has at most that many
// (row, block) lists of at most 16 {key, score} entries: 2048 * 16 * (8 + 4) bytes = 384 KiB.
// One copy per GPU, held until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: kernels get the device address that hipGetSymbolAddress returns
// for the current device, looked up once per device and kept in scratch_ptr.
constexpr size_t kStaticScratchBytes = size_t{512} << 10;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

gca_status static_scratch(void** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    t_last_hip_error = static_cast<int>(e);
    return GCA_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return GCA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t r = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (r != hipSuccess || ptr == nullptr) {
      t_last_hip_error = static_cast<int>(r != hipSuccess ? r : hipErrorInvalidSymbol);
      return GCA_ERR_HIP;
    }
    scratch_ptr[dev] = ptr;
  }
  *out = scratch_ptr[dev];
  return GCA_OK;
}

}  // namespace
}  // namespace gca

extern "C" {

gca_status gca_retrieve(const gca_problem* problem, const void* lq, const void* lk, int32_t* idx,
                        float* score, void* ws, size_t ws_bytes, void* stream) {
  GCA_TRY(retrieve_check(problem, lq, lk, idx, score));
  const RetrievePlan plan = plan_retrieve(problem);
  GCA_TRY(check_ws(plan.ws, ws, ws_bytes));
  return retrieve_launch(problem, plan, lq, lk, idx, score, ws, stream);
}

gca_status gca_retrieve_static(const gca_problem* problem, const void* lq, const void* lk, int32_t* idx,
                               float* score, void* stream) {
  GCA_TRY(retrieve_check(problem, lq, lk, idx, score));
  const RetrievePlan plan = plan_retrieve(problem);
  if (plan.ws > kStaticScratchBytes) return GCA_ERR_UNSUPPORTED;
  if (problem->n_q_chunks == 0) return GCA_OK;
  void* ws = nullptr;
  if (plan.ws > 0) GCA_TRY(static_scratch(&ws));
  return retrieve_launch(problem, plan, lq, lk, idx, score, ws, stream);
}

gca_status gca_forward(const gca_problem* problem, const void* q, const void* k, const void* v,
                       const int32_t* idx, const float* score, void* o, float* lse, void* ws,
                       size_t ws_bytes, void* stream) {
  GCA_TRY(validate_problem(problem));
  const gca_problem* p = problem;
  const bool any = p->n_q_chunks > 0;
  const bool kv = any && p->n_kv_chunks > 0;
  GCA_TRY(check_tensor(q, any, 16));
  GCA_TRY(check_tensor(k, kv, 16));
  GCA_TRY(check_tensor(v, kv, 16));
  GCA_TRY(check_tensor(idx, any, 4));
  GCA_TRY(check_tensor(score, any, 4));
  GCA_TRY(check_tensor(o, any, 16));
  if (lse != nullptr) GCA_TRY(check_tensor(lse, any, 16));
  GCA_TRY(check_ws(0, ws, ws_bytes));
  if (!any) return GCA_OK;

  AttendParams a = attend_params(p);
  a.q = q;
  a.k = k;
  a.v = v;
  a.idx = idx;
  a.score = score;
  a.o = o;
  a.lse = lse;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool f32 = p->dtype == GCA_F32;
  return launch(kAttendFwd, s, [&] { return launch_attend_fwd(a, f32, s); });
}

gca_status gca_backward(const gca_problem* problem, const void* q, const void* k, const void* v,
                        const int32_t* idx, const float* score, const float* lse, const void* dout,
                        void* dq, void* dk, void* dv, float* dscore, void* ws, size_t ws_bytes,
                        void* stream) {
  GCA_TRY(validate_problem(problem));
  const gca_problem* p = problem;
  const bool any = p->n_q_chunks > 0;
  const bool kv = p->n_kv_chunks > 0;
  GCA_TRY(check_tensor(q, any, 16));
  GCA_TRY(check_tensor(k, kv, 16));
  GCA_TRY(check_tensor(v, kv, 16));
  GCA_TRY(check_tensor(idx, any, 4));
  GCA_TRY(check_tensor(score, any, 4));
  GCA_TRY(check_tensor(lse, any, 16));
  GCA_TRY(check_tensor(dout, any, 16));
  GCA_TRY(check_tensor(dq, any, 16));
  GCA_TRY(check_tensor(dk, kv, 16));
  GCA_TRY(check_tensor(dv, kv, 16));
  GCA_TRY(check_tensor(dscore, any, 4));
  const BackwardLayout L = plan_backward(p);
  GCA_TRY(check_ws(L.total, ws, ws_bytes));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!any && !kv) return GCA_OK;

  AttendParams a = attend_params(p);
  a.q = q;
  a.k = k;
  a.v = v;
  a.idx = idx;
  a.score = score;
  a.lse_in = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dscore = dscore;
  char* w = static_cast<char*>(ws);
  a.delta = reinterpret_cast<float*>(w + L.delta);
  a.dw_part = reinterpret_cast<float*>(w + L.dw_part);
  a.wts = reinterpret_cast<float*>(w + L.wts);
  a.pairs = reinterpret_cast<int32_t*>(w + L.pairs);
  a.counts = reinterpret_cast<int32_t*>(w + L.counts);
  a.entry_decoded = 1;
  set_long_lists(a, L, w, any);
  const bool f32 = p->dtype == GCA_F32;
  // With no query chunk, only the inverse index (empty lists) and the key-major pass (which
  // writes zero dk, dv for chunks nobody retrieved) run.
  if (any) GCA_TRY(launch(kBwdQuery, s, [&] { return launch_bwd_query(a, f32, s); }));
  if (kv) GCA_TRY(launch(kInverseIndex, s, [&] { return launch_inverse_index(a, s); }));
  if (kv) GCA_TRY(launch(kBwdKey, s, [&] { return launch_bwd_key(a, f32, s); }));
  if (any) GCA_TRY(launch(kScoreGrad, s, [&] { return launch_score_grad(a, f32, s); }));
  return GCA_OK;
}

gca_status gca_landmark_backward(const gca_problem* problem, const void* lq, const void* lk,
                                 const int32_t* idx, const float* dscore, void* dlq, void* dlk, void* ws,
                                 size_t ws_bytes, void* stream) {
  GCA_TRY(validate_problem(problem));
  const gca_problem* p = problem;
  const bool any = p->n_q_chunks > 0;
  const bool kv = p->n_kv_chunks > 0;
  GCA_TRY(check_tensor(lq, any, 16));
  GCA_TRY(check_tensor(lk, kv, 16));
  GCA_TRY(check_tensor(idx, any, 4));
  GCA_TRY(check_tensor(dscore, any, 4));
  GCA_TRY(check_tensor(dlq, any, 16));
  GCA_TRY(check_tensor(dlk, kv, 16));
  const LandmarkLayout L = plan_landmark(p);
  GCA_TRY(check_ws(L.total, ws, ws_bytes));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!any && !kv) return GCA_OK;

  char* w = static_cast<char*>(ws);
  const bool f32 = p->dtype == GCA_F32;
  LandmarkParams m{};
  m.lq = lq;
  m.lk = lk;
  m.idx = idx;
  m.dscore = dscore;
  m.dlq = dlq;
  m.dlk = dlk;
  m.n_q = p->n_q_chunks;
  m.n_kv = p->n_kv_chunks;
  m.q_base = p->q_chunk_base;
  m.G = p->G;
  m.B = p->B;
  m.K = p->topk;
  m.pair_cap = static_cast<int32_t>(static_cast<int64_t>(p->G) * p->n_q_chunks);
  m.score_scale = p->score_scale;
  if (kv) {
    m.pairs = reinterpret_cast<const int32_t*>(w + L.pairs);
    m.counts = reinterpret_cast<const int32_t*>(w + L.counts);
    // the backward's inverse index, over every row (shift 0) and with d(score) as the entry value
    AttendParams a = attend_params(p);
    a.idx = idx;
    a.wts = const_cast<float*>(dscore);
    a.shift = 0;
    a.causal_rows = 1;
    a.pairs = reinterpret_cast<int32_t*>(w + L.pairs);
    a.counts = reinterpret_cast<int32_t*>(w + L.counts);
    GCA_TRY(launch(kInverseIndex, s, [&] { return launch_inverse_index(a, s); }));
  }
  if (any) GCA_TRY(launch(kLmkQueryGrad, s, [&] { return launch_lmk_query_grad(m, f32, s); }));
  if (kv) GCA_TRY(launch(kLmkKeyGrad, s, [&] { return launch_lmk_key_grad(m, f32, s); }));
  return GCA_OK;
}

gca_status gca_decode_tokens(const gca_problem* problem, int32_t n_tokens, const void* q, const void* k,
                             const void* v, const int32_t* idx, const float* score, void* o, void* stream) {
  GCA_TRY(validate_problem(problem));
  const gca_problem* p = problem;
  if (p->n_q_chunks != 1 || n_tokens < 1 || n_tokens > p->S) return GCA_ERR_INVALID_ARGUMENT;
  const bool kv = p->n_kv_chunks > 0;
  GCA_TRY(check_tensor(q, true, 16));
  GCA_TRY(check_tensor(k, kv, 16));
  GCA_TRY(check_tensor(v, kv, 16));
  GCA_TRY(check_tensor(idx, true, 4));
  GCA_TRY(check_tensor(score, true, 4));
  GCA_TRY(check_tensor(o, true, 16));
  AttendParams a = attend_params(p);
  a.q = q;
  a.k = k;
  a.v = v;
  a.idx = idx;
  a.score = score;
  a.o = o;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool f32 = p->dtype == GCA_F32;
  return launch(kDecodeTokens, s, [&] { return launch_decode_tokens(a, n_tokens, f32, s); });
}

// Sliding-window attention problems: one sequence of n_q_chunks chunks per (batch row, head).
static gca_status sw_check(const gca_problem* p, int32_t window) {
  GCA_TRY(validate_problem(p));
  if (p->G != 1 || p->n_kv_chunks != p->n_q_chunks) return GCA_ERR_INVALID_ARGUMENT;
  if (window < 64 || window % 64 != 0) return GCA_ERR_INVALID_ARGUMENT;
  return GCA_OK;
}

static SwParams sw_params(const gca_problem* p, int32_t window) {
  SwParams w{};
  w.n_c = p->n_q_chunks;
  w.B = p->B;
  w.H = p->H;
  w.m = window / 64;
  w.attn_scale = p->attn_scale;
  return w;
}

gca_status gca_sw_forward(const gca_problem* problem, int32_t window, const void* q, const void* k, const void* v,
                          void* o, float* lse, void* stream) {
  GCA_TRY(sw_check(problem, window));
  const bool any = problem->n_q_chunks > 0;
  GCA_TRY(check_tensor(q, any, 16));
  GCA_TRY(check_tensor(k, any, 16));
  GCA_TRY(check_tensor(v, any, 16));
  GCA_TRY(check_tensor(o, any, 16));
  if (lse != nullptr) GCA_TRY(check_tensor(lse, any, 4));
  if (!any) return GCA_OK;
  SwParams w = sw_params(problem, window);
  w.q = q;
  w.k = k;
  w.v = v;
  w.o = o;
  w.lse = lse;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool f32 = problem->dtype == GCA_F32;
  return launch(kSwFwd, s, [&] { return launch_sw_fwd(w, f32, s); });
}

gca_status gca_sw_backward(const gca_problem* problem, int32_t window, const void* q, const void* k, const void* v,
                           const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv, void* ws,
                           size_t ws_bytes, void* stream) {
  GCA_TRY(sw_check(problem, window));
  const bool any = problem->n_q_chunks > 0;
  for (const void* t : {q, k, v, o, dout, static_cast<const void*>(dq), static_cast<const void*>(dk),
                        static_cast<const void*>(dv)})
    GCA_TRY(check_tensor(t, any, 16));
  GCA_TRY(check_tensor(lse, any, 4));
  size_t need = 0;
  GCA_TRY(gca_workspace_size(GCA_OP_SW_BACKWARD, problem, &need));
  GCA_TRY(check_ws(need, ws, ws_bytes));
  if (!any) return GCA_OK;
  SwParams w = sw_params(problem, window);
  w.q = q;
  w.k = k;
  w.v = v;
  w.o_in = o;
  w.lse_in = lse;
  w.dout = dout;
  w.dq = dq;
  w.dk = dk;
  w.dv = dv;
  w.stats = static_cast<float*>(ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool f32 = problem->dtype == GCA_F32;
  GCA_TRY(launch(kSwBwdQuery, s, [&] { return launch_sw_bwd_query(w, f32, s); }));
  return launch(kSwBwdKey, s, [&] { return launch_sw_bwd_key(w, f32, s); });
}

// Fused layer attention: one retrieval group, window W = 64 m over the layer's own keys.
static gca_status fused_check(const gca_problem* p, int32_t window) {
  GCA_TRY(validate_problem(p));
  if (p->G != 1) return GCA_ERR_INVALID_ARGUMENT;
  if (window < 64 || window % 64 != 0) return GCA_ERR_INVALID_ARGUMENT;
  return GCA_OK;
}

gca_status gca_fused_forward(const gca_problem* problem, int32_t window, const void* q, const void* k_sw,
                             const void* v_sw, const void* k, const void* v, const int32_t* idx, const float* score,
                             void* o, float* lse_sw, float* lse, void* stream) {
  GCA_TRY(fused_check(problem, window));
  const gca_problem* p = problem;
  const bool any = p->n_q_chunks > 0;
  const bool kv = any && p->n_kv_chunks > 0;
  for (const void* t : {q, k_sw, v_sw, static_cast<const void*>(o)}) GCA_TRY(check_tensor(t, any, 16));
  GCA_TRY(check_tensor(k, kv, 16));
  GCA_TRY(check_tensor(v, kv, 16));
  GCA_TRY(check_tensor(idx, any, 4));
  GCA_TRY(check_tensor(score, any, 4));
  if (lse_sw != nullptr) GCA_TRY(check_tensor(lse_sw, any, 4));
  if (lse != nullptr) GCA_TRY(check_tensor(lse, any, 16));
  if (!any) return GCA_OK;
  AttendParams a = attend_params(p);
  a.q = q;
  a.k = k;
  a.v = v;
  a.k_sw = k_sw;
  a.v_sw = v_sw;
  a.idx = idx;
  a.score = score;
  a.o = o;
  a.lse = lse;
  a.lse_sw = lse_sw;
  a.m = window / 64;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool f32 = p->dtype == GCA_F32;
  return launch(kFusedFwd, s, [&] { return launch_fused_fwd(a, f32, s); });
}

gca_status gca_fused_backward(const gca_problem* problem, int32_t window, const void* q, const void* k_sw,
                              const void* v_sw, const void* k, const void* v, const int32_t* idx,
                              const float* score, const void* o, const float* lse_sw, const float* lse,
                              const void* dout, void* dq, void* dk_sw, void* dv_sw, void* dk, void* dv,
                              float* dscore, void* ws, size_t ws_bytes, void* stream) {
  GCA_TRY(fused_check(problem, window));
  const gca_problem* p = problem;
  const bool any = p->n_q_chunks > 0;
  const bool kv = p->n_kv_chunks > 0;
  for (const void* t : {q, k_sw, v_sw, o, dout, static_cast<const void*>(dq), static_cast<const void*>(dk_sw),
                        static_cast<const void*>(dv_sw)})
    GCA_TRY(check_tensor(t, any, 16));
  GCA_TRY(check_tensor(k, kv, 16));
  GCA_TRY(check_tensor(v, kv, 16));
  GCA_TRY(check_tensor(dk, kv, 16));
  GCA_TRY(check_tensor(dv, kv, 16));
  GCA_TRY(check_tensor(idx, any, 4));
  GCA_TRY(check_tensor(score, any, 4));
  GCA_TRY(check_tensor(dscore, any, 4));
  GCA_TRY(check_tensor(lse_sw, any, 4));
  GCA_TRY(check_tensor(lse, any, 16));
  const BackwardLayout L = plan_backward(p);
  size_t need = 0;
  GCA_TRY(gca_workspace_size(GCA_OP_FUSED_BACKWARD, p, &need));
  GCA_TRY(check_ws(need, ws, ws_bytes));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!any && !kv) return GCA_OK;

  char* w = static_cast<char*>(ws);
  AttendParams a = attend_params(p);
  a.q = q;
  a.k = k;
  a.v = v;
  a.k_sw = k_sw;
  a.v_sw = v_sw;
  a.idx = idx;
  a.score = score;
  a.o = const_cast<void*>(o);
  a.lse_in = lse;
  a.lse_sw = const_cast<float*>(lse_sw);
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dscore = dscore;
  a.m = window / 64;
  a.delta = reinterpret_cast<float*>(w + L.delta);
  a.dw_part = reinterpret_cast<float*>(w + L.dw_part);
  a.wts = reinterpret_cast<float*>(w + L.wts);
  a.pairs = reinterpret_cast<int32_t*>(w + L.pairs);
  a.counts = reinterpret_cast<int32_t*>(w + L.counts);
  a.sw_stats = reinterpret_cast<float*>(w + L.total);
  a.entry_decoded = 1;
  set_long_lists(a, L, w, any);
  const bool f32 = p->dtype == GCA_F32;
  if (any) {
    GCA_TRY(launch(kFusedBwdQuery, s, [&] { return launch_fused_bwd_query(a, f32, s); }));
    SwParams sw = sw_params(p, window);
    sw.q = q;
    sw.k = k_sw;
    sw.v = v_sw;
    sw.dout = dout;
    sw.dk = dk_sw;
    sw.dv = dv_sw;
    sw.stats = a.sw_stats;
    GCA_TRY(launch(kSwBwdKey, s, [&] { return launch_sw_bwd_key(sw, f32, s); }));
  }
  if (kv) GCA_TRY(launch(kInverseIndex, s, [&] { return launch_inverse_index(a, s); }));
  if (kv) GCA_TRY(launch(kBwdKey, s, [&] { return launch_bwd_key(a, f32, s); }));
  if (any) GCA_TRY(launch(kScoreGrad, s, [&] { return launch_score_grad(a, f32, s); }));
  return GCA_OK;
}

// The device address of a K/V source: device memory as it is; pinned host memory (hipHostMalloc)
// through its mapping into the device's address space.  Pageable host memory, which a kernel
// cannot read, is refused.
static gca_status device_address(const void* ptr, const void** out) {
  hipPointerAttribute_t attr{};
  if (hipPointerGetAttributes(&attr, ptr) != hipSuccess) {
    (void)hipGetLastError();
    return GCA_ERR_INVALID_ARGUMENT;
  }
  if (attr.type == hipMemoryTypeDevice) {
    *out = ptr;
    return GCA_OK;
  }
  if (attr.type == hipMemoryTypeHost && attr.devicePointer != nullptr) {
    *out = attr.devicePointer;
    return GCA_OK;
  }
  return GCA_ERR_INVALID_ARGUMENT;
}

gca_status gca_fetch_chunks(const gca_problem* problem, const int32_t* idx, const void* k, const void* v,
                            void* k_out, void* v_out, int32_t* idx_out, void* stream) {
  GCA_TRY(validate_problem(problem));
  const gca_problem* p = problem;
  const bool any = p->n_q_chunks > 0;
  const bool kv = any && p->n_kv_chunks > 0;
  GCA_TRY(check_tensor(idx, any, 4));
  GCA_TRY(check_tensor(idx_out, any, 4));
  GCA_TRY(check_tensor(k, kv, 16));
  GCA_TRY(check_tensor(v, kv, 16));
  GCA_TRY(check_tensor(k_out, any, 16));
  GCA_TRY(check_tensor(v_out, any, 16));
  if (!any) return GCA_OK;
  FetchParams f{};
  f.idx = idx;
  f.k = k;
  f.v = v;
  if (kv) {
    GCA_TRY(device_address(k, &f.k));
    GCA_TRY(device_address(v, &f.v));
  }
  f.k_out = k_out;
  f.v_out = v_out;
  f.idx_out = idx_out;
  f.n_q = p->n_q_chunks;
  f.n_kv = p->n_kv_chunks;
  f.n_c = static_cast<int64_t>(p->G) * p->n_q_chunks * p->topk;
  f.G = p->G;
  f.B = p->B;
  f.H = p->H;
  f.K = p->topk;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool f32 = p->dtype == GCA_F32;
  return launch(kFetchChunks, s, [&] { return launch_fetch_chunks(f, f32, s); });
}

const char* gca_status_string(gca_status status) {
  switch (status) {
    case GCA_OK: return "ok";
    case GCA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case GCA_ERR_UNSUPPORTED: return "unsupported problem size or option";
    case GCA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case GCA_ERR_MISALIGNED: return "misaligned tensor pointer";
    case GCA_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int gca_last_hip_error(void) { return t_last_hip_error; }

gca_status gca_profile_enable(int on) {
  t_prof.on = on != 0;
  return GCA_OK;
}

gca_status gca_profile_collect(int cap, const char** names, double* total_ms, int64_t* counts, int* n) {
  if (n == nullptr || cap < 0 || (cap > 0 && (names == nullptr || total_ms == nullptr || counts == nullptr)))
    return GCA_ERR_INVALID_ARGUMENT;
  double ms[kNumKernels] = {0};
  int64_t cnt[kNumKernels] = {0};
  gca_status st = GCA_OK;
  for (const ProfRecord& r : t_prof.records) {
    float e = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&e, r.start, r.stop) != hipSuccess) {
      t_last_hip_error = static_cast<int>(hipGetLastError());
      st = GCA_ERR_HIP;
    }
    ms[r.kernel] += e;
    cnt[r.kernel] += 1;
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  t_prof.records.clear();
  int m = 0;
  for (int k = 0; k < kNumKernels; ++k) {
    if (cnt[k] == 0) continue;
    if (m < cap) {
      names[m] = kernel_name(k);
      total_ms[m] = ms[k];
      counts[m] = cnt[k];
    }
    ++m;
  }
  *n = m;
  return st;
}

}  // extern "C"
