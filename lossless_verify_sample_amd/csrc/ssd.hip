// C ABI of the verify-and-resample library (declarations and citations in
// include/ssd.h): host-side argument checks, workspace layout and launches.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>

#include <hip/hip_ext.h>

#include "kernels.hpp"
#include "probe.hpp"

using namespace ssd;

// Library-owned scratch for ssd_round_noalloc (callers that cannot allocate
// device memory): the verification's workspace in the first half, the
// sampling's in the second.  Each GPU the library runs on holds its own copy
// until the process ends.
constexpr size_t kScratchHalf = SSD_NOALLOC_HALF_BYTES;
static __device__ __align__(256) unsigned char scratch[2 * kScratchHalf];

namespace {

size_t al256(size_t x) { return (x + 255) & ~size_t(255); }
int dt_size(int dt) { return dt == SSD_F32 ? 4 : 2; }
bool dt_ok(int dt) { return dt == SSD_F32 || dt == SSD_BF16 || dt == SSD_F16; }
int64_t nblocks(int64_t V) { return (V + BLK - 1) / BLK; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Layout {
  size_t part, zcap, gate, total;
};

// Workspace regions (256-byte aligned): block partials of every streamed row;
// for verification the target logits at the drafted tokens and the
// early-exit gate's decisions.  Every region is written before it is read
// within a call, so the workspace needs no initialisation.
bool layout(ssd_op op, int64_t n, int32_t K, int64_t V, Layout* L) {
  if (n < 1 || V < 1 || V > SSD_MAX_V) return false;
  if ((op == SSD_OP_SAMPLE || op == SSD_OP_VERIFY) && (K < 0 || K > SSD_MAX_K)) return false;
  if (op == SSD_OP_VERIFY_TREE && (K < 0 || K >= SSD_MAX_TREE_NODES)) return false;
  if (op != SSD_OP_SOFTMAX_T && op != SSD_OP_TOPF && op != SSD_OP_SAMPLE && op != SSD_OP_VERIFY &&
      op != SSD_OP_VERIFY_TREE)
    return false;
  const int64_t NB = nblocks(V);
  const int64_t rows = (op == SSD_OP_SAMPLE || op == SSD_OP_VERIFY || op == SSD_OP_VERIFY_TREE) ? n * (K + 1) : n;
  L->part = 0;
  L->zcap = L->gate = 0;
  size_t end = al256((size_t)(rows * NB) * sizeof(float4));
  if (op == SSD_OP_VERIFY) {
    L->zcap = end;
    L->gate = L->zcap + al256((size_t)(n * (K > 0 ? K : 1)) * sizeof(float));
    end = L->gate + al256((size_t)(n + 1) * sizeof(int32_t));
  }
  L->total = end;
  return true;
}

bool aligned16(const void* ptr, int64_t ld, int64_t V, int dt) {
  const int sz = dt_size(dt);
  return ((uintptr_t)ptr % 16 == 0) && ((ld * sz) % 16 == 0) && ((V * sz) % 16 == 0);
}

template <template <int, bool> class L, class... A>
hipError_t dispatch(int dt, bool al, A... a) {
  if (dt == SSD_F32) return al ? L<SSD_F32, true>::go(a...) : L<SSD_F32, false>::go(a...);
  if (dt == SSD_BF16) return al ? L<SSD_BF16, true>::go(a...) : L<SSD_BF16, false>::go(a...);
  return al ? L<SSD_F16, true>::go(a...) : L<SSD_F16, false>::go(a...);
}

// Launch on `st`; with timer events the launch itself records them (the
// HIP extension launch stamps the dispatch, adding no packets of its own).
#define SSD_LAUNCHER_T(NAME, KERNEL, THREADS)                                              \
  template <int DT, bool AL>                                                              \
  struct NAME {                                                                           \
    static hipError_t go(int64_t grid, const Params& p, hipStream_t st, hipEvent_t e0 = nullptr, \
                         hipEvent_t e1 = nullptr) {                                       \
      if (e0) {                                                                           \
        hipExtLaunchKernelGGL(KERNEL, dim3((unsigned)grid), dim3(THREADS), 0, st, e0, e1, 0, p); \
      } else {                                                                            \
        KERNEL<<<dim3((unsigned)grid), dim3(THREADS), 0, st>>>(p);                        \
      }                                                                                   \
      return hipGetLastError();                                                           \
    }                                                                                     \
  };
#define SSD_LAUNCHER(NAME, KERNEL) SSD_LAUNCHER_T(NAME, KERNEL, WG)
#define SSD_LAUNCHER_E(NAME, KERNEL) SSD_LAUNCHER_T(NAME, KERNEL, EWG)

SSD_LAUNCHER(LSoftmax, (k_stream<DT, AL, M_SOFTMAX>))
SSD_LAUNCHER(LTopf, (k_stream<DT, AL, M_TOPF>))
SSD_LAUNCHER(LSample, (k_stream<DT, AL, M_SAMPLE>))
SSD_LAUNCHER(LVerify, (k_stream<DT, AL, M_VERIFY>))
SSD_LAUNCHER(LVerifyGated, (k_stream_gated<DT, AL>))
SSD_LAUNCHER_E(LGate, (k_gate<DT, AL>))
SSD_LAUNCHER_E(LSoftmaxEpi, (k_epi<DT, AL, M_SOFTMAX>))
SSD_LAUNCHER_E(LTopfEpi, (k_epi<DT, AL, M_TOPF>))
SSD_LAUNCHER_E(LSampleEpi, (k_epi<DT, AL, M_SAMPLE>))
SSD_LAUNCHER_E(LVerifySeq, (k_verify_seq<DT, AL>))
SSD_LAUNCHER(LProbs, (k_probs<DT, AL>))

template <int DT, bool AL>
struct LTree {
  static hipError_t go(int64_t grid, const Params& p, const TreeArgs& ta, hipStream_t st) {
    k_tree<DT, AL><<<dim3((unsigned)grid), dim3(EWG), 0, st>>>(p, ta);
    return hipGetLastError();
  }
};

// A launch of two parameter sets (verification's kernel beside sampling's).
#define SSD_LAUNCHER2(NAME, KERNEL)                                                          \
  template <int DT, bool AL>                                                              \
  struct NAME {                                                                           \
    static hipError_t go(int64_t grid, const Params& pv, const Params& ps, int nv, hipStream_t st) { \
      KERNEL<<<dim3((unsigned)grid), dim3(EWG), 0, st>>>(pv, ps, nv);                     \
      return hipGetLastError();                                                           \
    }                                                                                     \
  };
SSD_LAUNCHER2(LRoundMid, (k_round_mid<DT, AL>))
SSD_LAUNCHER2(LRoundTails, (k_round_tails<DT, AL>))
// (the streams' launch runs WG threads per workgroup)
template <int DT, bool AL>
struct LRoundStreams {
  static hipError_t go(int64_t grid, const Params& pv, const Params& ps, int nv, hipStream_t st, hipEvent_t e0 = nullptr,
                       hipEvent_t e1 = nullptr) {
    if (e0) {
      hipExtLaunchKernelGGL((k_round_streams<DT, AL>), dim3((unsigned)grid), dim3(WG), 0, st, e0, e1, 0, pv, ps, nv);
    } else {
      k_round_streams<DT, AL><<<dim3((unsigned)grid), dim3(WG), 0, st>>>(pv, ps, nv);
    }
    return hipGetLastError();
  }
};
// The same with the timer's events recorded by the launch.
template <int DT, bool AL>
struct LRoundMidT {
  static hipError_t go(int64_t grid, const Params& pv, const Params& ps, int nv, hipStream_t st, hipEvent_t e0,
                       hipEvent_t e1) {
    hipExtLaunchKernelGGL((k_round_mid<DT, AL>), dim3((unsigned)grid), dim3(EWG), 0, st, e0, e1, 0, pv, ps, nv);
    return hipGetLastError();
  }
};

ssd_status hip_status(hipError_t e) { return e == hipSuccess ? SSD_OK : SSD_ERR_HIP; }

bool ws_ok(const void* ws, size_t bytes, const Layout& L) {
  return ws != nullptr && ((uintptr_t)ws % 256 == 0) && bytes >= L.total;
}

const int64_t kMaxGrid = 0x7fffffff;
// Target rows read with ordinary loads (positions 0 and 1, the likeliest of
// the first rejection, whose re-read by the residual pass may then hit the
// Infinity Cache), while those rows of all sequences fit in this many bytes:
// measured about 1 us less per step at B=64, K=7, V=151936 (39 MB); at 131
// and 311 MB the shared launch slowed by 10-15%.
constexpr int kKeepRows = 2;
// ssd_round runs in two launches (both streaming passes, then the
// verification beside the sampling epilogue) while the sampling's rows are
// at most this many: at small batches the verification of a sequence takes
// longer than the sampling's streaming pass it would otherwise share.
constexpr int64_t kTwoLaunchRows = 256;
constexpr int64_t kKeepBytes = int64_t(64) << 20;

// Depth offsets of a cache descriptor into p (false for a bad fan-out).
bool cache_layout(const ssd_cache* c, int K, int64_t V, Params& p) {
  int off = 0;
  for (int k = 0; k <= K; ++k) {
    const int f = c->fanout[k];
    if (f < 0 || f > SSD_MAX_F || f > V) return false;
    p.koff[k] = off;
    off += f;
  }
  p.koff[K + 1] = off;
  p.Bgt = off;
  return true;
}

// Kernel timer: event pairs around the streaming-pass launches, per op
// (host state, guarded by a mutex: calls from several threads stay safe, the
// counts then mix their launches).
struct Timer {
  int cap = 0;
  int n[4] = {0, 0, 0, 0};
  std::vector<hipEvent_t> ev[4];
};
Timer g_timer;
std::mutex g_timer_mu;

void timer_free() {
  for (auto& v : g_timer.ev) {
    for (hipEvent_t e : v) (void)hipEventDestroy(e);
    v.clear();
  }
  g_timer.cap = 0;
  for (int& c : g_timer.n) c = 0;
}

// The streaming pass of `op`: launch(e0, e1) with the timer's next event
// pair when it is enabled and has room, else with none.
template <class F>
hipError_t timed(ssd_op op, F launch) {
  std::lock_guard<std::mutex> lock(g_timer_mu);
  if (g_timer.cap > 0 && g_timer.n[op] < g_timer.cap) {
    const int i = g_timer.n[op];
    const hipError_t e = launch(g_timer.ev[op][2 * i], g_timer.ev[op][2 * i + 1]);
    if (e == hipSuccess) ++g_timer.n[op];
    return e;
  }
  return launch(nullptr, nullptr);
}

// A checked call: kernel parameters, element type, alignment, grid sizes.
struct Plan {
  Params p{};
  int dt = 0;
  bool al = false;
  int64_t g_stream = 0;  // streaming pass
  int64_t g_tail = 0;    // sampling epilogue / verification after the streaming pass
};

ssd_status plan_sample(const ssd_sample_args& a, Plan& q) {
  const int32_t B = a.B, K = a.K, F = a.F, F_out = a.F_out;
  const int64_t V = a.V, ld = a.ld;
  const float C = a.C;
  if (!a.draft_logits || !a.temperature || !a.out_stats || !dt_ok(a.dt)) return SSD_ERR_INVALID_ARG;
  if (B < 1 || K < 0 || K > SSD_MAX_K || V < 1 || V > SSD_MAX_V || ld < V) return SSD_ERR_INVALID_ARG;
  if (K > 0 && (!a.out_tokens || !a.out_q)) return SSD_ERR_INVALID_ARG;
  if (F < 0 || F > SSD_MAX_F || F > V || F_out < F || F_out > SSD_MAX_F || F_out > V) return SSD_ERR_INVALID_ARG;
  if (F_out > 0 && !a.out_topf_idx && !a.out_topf_val) return SSD_ERR_INVALID_ARG;
  if (!(C > 0.f) || !(C <= 1.f)) return SSD_ERR_INVALID_ARG;
  Params& p = q.p;
  p = Params{};
  const ssd_cache* cache = a.cache;
  if (cache) {
    if (!cache->fanout || !cache->keys || !cache_layout(cache, K, V, p)) return SSD_ERR_INVALID_ARG;
    p.ckeys = cache->keys;
  }
  Layout L;
  if (!layout(SSD_OP_SAMPLE, B, K, V, &L)) return SSD_ERR_INVALID_ARG;
  if (!ws_ok(a.workspace, a.ws_bytes, L)) return SSD_ERR_WORKSPACE;
  const int64_t rows = (int64_t)B * (K + 1);
  const int64_t NB = nblocks(V), nch = cdiv(NB, CH);
  if (rows * nch > kMaxGrid) return SSD_ERR_UNSUPPORTED;
  p.x = (const unsigned char*)a.draft_logits;
  p.V = V; p.ld = ld; p.rows = rows; p.NB = (int)NB; p.nchunk = (int)nch;
  p.K = K; p.B = B;
  p.temp = a.temperature;
  p.F = F; p.F_out = F_out; p.F_sel = F_out > 1 ? F_out : 1;
  if (cache) {
    for (int j = 0; j <= K; ++j)
      if (cache->fanout[j] > p.F_sel) p.kdep[p.nkd++] = j;
  }
  p.C = C; p.seed = a.seed;
  char* ws = (char*)a.workspace;
  p.part = (float4*)(ws + L.part);
  p.stats = a.out_stats;
  p.out_idx = F_out > 0 ? a.out_topf_idx : nullptr;
  p.out_val = F_out > 0 ? a.out_topf_val : nullptr;
  p.tokens = a.out_tokens;
  p.q = a.out_q;
  q.dt = a.dt;
  q.al = aligned16(a.draft_logits, ld, V, a.dt);
  q.g_stream = rows * nch;
  q.g_tail = rows + (int64_t)p.nkd * B;
  return SSD_OK;
}

hipError_t launch_sample(const Plan& q, hipStream_t st) {
  hipError_t e = timed(SSD_OP_SAMPLE, [&](hipEvent_t e0, hipEvent_t e1) {
    return dispatch<LSample>(q.dt, q.al, q.g_stream, q.p, st, e0, e1);
  });
  if (e == hipSuccess) e = dispatch<LSampleEpi>(q.dt, q.al, q.g_tail, q.p, st);
  return e;
}

ssd_status plan_verify(const ssd_verify_args& a, Plan& q) {
  const int32_t B = a.B, K = a.K, F = a.F;
  const int64_t V = a.V, ld = a.ld;
  const float C = a.C;
  if (!a.target_logits || !a.draft_logits || !a.temperature || !dt_ok(a.dt)) return SSD_ERR_INVALID_ARG;
  if (!a.draft_stats || !a.out_accept_len || !a.out_bonus) return SSD_ERR_INVALID_ARG;
  if (B < 1 || K < 0 || K > SSD_MAX_K || V < 1 || V > SSD_MAX_V || ld < V) return SSD_ERR_INVALID_ARG;
  if (K > 0 && (!a.draft_tokens || !a.draft_q || !a.out_p)) return SSD_ERR_INVALID_ARG;
  if (F < 0 || F > SSD_MAX_F || F > V) return SSD_ERR_INVALID_ARG;
  if (F > 0 && (!a.draft_topf_idx || a.ld_topf < F)) return SSD_ERR_INVALID_ARG;
  if (!(C > 0.f) || !(C <= 1.f)) return SSD_ERR_INVALID_ARG;
  Params& p = q.p;
  p = Params{};
  const ssd_cache* cache = a.cache;
  if (cache) {
    if (!cache->fanout || !cache_layout(cache, K, V, p)) return SSD_ERR_INVALID_ARG;
    if (p.Bgt > 0 && !cache->keys) return SSD_ERR_INVALID_ARG;
    if (!cache->out_hit || !cache->out_slot || (K > 0 && !cache->out_tokens)) return SSD_ERR_INVALID_ARG;
    if (cache->miss_fill != 0 && cache->miss_fill != 1) return SSD_ERR_INVALID_ARG;
    p.fill = cache->miss_fill;
    if (K > 0 && p.Bgt > 0 && !cache->payload) return SSD_ERR_INVALID_ARG;
    p.ckeys = cache->keys;
    p.cpay = cache->payload;
    p.chit = cache->out_hit;
    p.cslot = cache->out_slot;
    p.ctok = cache->out_tokens;
    p.lookup = 1;
  }
  Layout L;
  if (!layout(SSD_OP_VERIFY, B, K, V, &L)) return SSD_ERR_INVALID_ARG;
  if (!ws_ok(a.workspace, a.ws_bytes, L)) return SSD_ERR_WORKSPACE;
  const int64_t rows = (int64_t)B * (K + 1);
  const int64_t NB = nblocks(V), nch = cdiv(NB, CH);
  if (rows * nch > kMaxGrid) return SSD_ERR_UNSUPPORTED;
  p.x = (const unsigned char*)a.target_logits;
  p.xd = (const unsigned char*)a.draft_logits;
  p.V = V; p.ld = ld; p.rows = rows; p.NB = (int)NB; p.nchunk = (int)nch;
  p.K = K; p.B = B;
  p.temp = a.temperature;
  p.F = F; p.C = C; p.seed = a.seed;
  char* ws = (char*)a.workspace;
  p.part = (float4*)(ws + L.part);
  p.stats = a.out_target_stats;
  p.dtok = a.draft_tokens;
  p.dq = a.draft_q;
  p.zcap = (float*)(ws + L.zcap);
  p.gate = (int32_t*)(ws + L.gate);
  p.dstats = a.draft_stats;
  p.dtopf = F > 0 ? a.draft_topf_idx : nullptr;
  p.ld_dtopf = a.ld_topf;
  p.acc_len = a.out_accept_len;
  p.bonus = a.out_bonus;
  p.p_out = a.out_p;
  q.dt = a.dt;
  q.al = aligned16(a.target_logits, ld, V, a.dt) && aligned16(a.draft_logits, ld, V, a.dt);
  q.g_stream = rows * nch;
  p.keep = (int64_t)B * kKeepRows * V * dt_size(a.dt) <= kKeepBytes ? kKeepRows : 0;
  q.g_tail = B;
  return SSD_OK;
}

hipError_t launch_verify(const Plan& q, hipStream_t st) {
  Params p = q.p;
  hipError_t e = timed(SSD_OP_VERIFY, [&](hipEvent_t e0, hipEvent_t e1) {
    return dispatch<LVerify>(q.dt, q.al, q.g_stream, p, st, e0, e1);
  });
  if (e == hipSuccess) e = dispatch<LVerifySeq>(q.dt, q.al, q.g_tail, p, st);
  return e;
}

// The two calls of a pipeline step, checked (see ssd_round).
ssd_status plan_round(const ssd_verify_args* v, const ssd_sample_args* s, Plan& qv, Plan& qs) {
  if (!v && !s) return SSD_ERR_INVALID_ARG;
  if (v) {
    const ssd_status e = plan_verify(*v, qv);
    if (e != SSD_OK) return e;
  }
  if (s) {
    const ssd_status e = plan_sample(*s, qs);
    if (e != SSD_OK) return e;
  }
  if (v && s && (v->workspace == s->workspace)) return SSD_ERR_WORKSPACE;
  if (v && s && (qv.g_tail + qs.g_stream > kMaxGrid || qv.g_stream + qs.g_stream > kMaxGrid ||
                 qv.g_tail + qs.g_tail > kMaxGrid))
    return SSD_ERR_UNSUPPORTED;
  if (v && s) {
    // round i+1's sampling must not write what round i's verification reads
    const void* w[] = {s->out_tokens, s->out_q, s->out_stats, s->out_topf_idx};
    const void* r[] = {v->draft_tokens, v->draft_q, v->draft_stats, v->draft_topf_idx};
    for (const void* a : w)
      for (const void* b : r)
        if (a && a == b) return SSD_ERR_INVALID_ARG;
    if (v->cache && s->cache && v->cache->keys && v->cache->keys == s->cache->keys) return SSD_ERR_INVALID_ARG;
  }
  return SSD_OK;
}

// Launches of a planned pipeline step (either plan may be absent).
ssd_status launch_round(const Plan* pqv, const Plan* pqs, hipStream_t st) {
  (void)hipGetLastError();
  if (!pqv) return hip_status(launch_sample(*pqs, st));
  if (!pqs) return hip_status(launch_verify(*pqv, st));
  const Plan& qv = *pqv;
  const Plan& qs = *pqs;
  if (qv.dt != qs.dt || qv.al != qs.al) {
    // kernels of different element types cannot share a launch: in turn
    hipError_t e = launch_verify(qv, st);
    if (e == hipSuccess) e = launch_sample(qs, st);
    return hip_status(e);
  }
  Params pv = qv.p;
  const int64_t nv = qv.g_tail;
  if (qs.p.rows <= kTwoLaunchRows) {
    // both streaming passes in one launch; then the verification of each
    // sequence beside sampling's epilogue
    hipError_t e = timed(SSD_OP_SAMPLE, [&](hipEvent_t e0, hipEvent_t e1) {
      return dispatch<LRoundStreams>(qv.dt, qv.al, qv.g_stream + qs.g_stream, pv, qs.p, (int)qv.g_stream, st, e0, e1);
    });
    if (e == hipSuccess) e = dispatch<LRoundTails>(qv.dt, qv.al, nv + qs.g_tail, pv, qs.p, (int)nv, st);
    return hip_status(e);
  }
  // verification's streaming pass; then the verification of each sequence
  // beside sampling's streaming pass; then sampling's epilogue
  hipError_t e = timed(SSD_OP_VERIFY, [&](hipEvent_t e0, hipEvent_t e1) {
    return dispatch<LVerify>(qv.dt, qv.al, qv.g_stream, pv, st, e0, e1);
  });
  if (e == hipSuccess) {
    e = timed(SSD_OP_SAMPLE, [&](hipEvent_t e0, hipEvent_t e1) {
      return e0 ? dispatch<LRoundMidT>(qv.dt, qv.al, nv + qs.g_stream, pv, qs.p, (int)nv, st, e0, e1)
                : dispatch<LRoundMid>(qv.dt, qv.al, nv + qs.g_stream, pv, qs.p, (int)nv, st);
    });
  }
  if (e == hipSuccess) e = dispatch<LSampleEpi>(qs.dt, qs.al, qs.g_tail, qs.p, st);
  return hip_status(e);
}

// Token-tree verification: checks, kernel parameters and the topology.
ssd_status plan_tree(const ssd_tree_args& a, Plan& q, TreeArgs& ta) {
  const int32_t B = a.B, N = a.N, F = a.F;
  const int64_t V = a.V, ld = a.ld;
  const float C = a.C;
  if (!a.target_logits || !a.draft_logits || !a.temperature || !a.parent || !dt_ok(a.dt)) return SSD_ERR_INVALID_ARG;
  if (!a.draft_stats || !a.out_accept_len || !a.out_last || !a.out_bonus) return SSD_ERR_INVALID_ARG;
  if (B < 1 || N < 0 || N >= SSD_MAX_TREE_NODES || V < 1 || V > SSD_MAX_V || ld < V) return SSD_ERR_INVALID_ARG;
  if (N > 0 && (!a.tokens || !a.draft_q)) return SSD_ERR_INVALID_ARG;
  if (F < 0 || F > SSD_MAX_F || F > V) return SSD_ERR_INVALID_ARG;
  if (F > 0 && (!a.draft_topf_idx || a.ld_topf < F)) return SSD_ERR_INVALID_ARG;
  if (!(C > 0.f) || !(C <= 1.f)) return SSD_ERR_INVALID_ARG;
  if (a.parent[0] != -1) return SSD_ERR_INVALID_ARG;
  ta = TreeArgs{};
  for (int m = 1; m <= N; ++m) {
    const int pm = a.parent[m];
    if (pm < 0 || pm >= m) return SSD_ERR_INVALID_ARG;
    ta.par[m >> 3] |= (uint64_t)(uint8_t)pm << (8 * (m & 7));
  }
  ta.N1 = N + 1;
  ta.last = a.out_last;
  Layout L;
  if (!layout(SSD_OP_VERIFY_TREE, B, N, V, &L)) return SSD_ERR_INVALID_ARG;
  if (!ws_ok(a.workspace, a.ws_bytes, L)) return SSD_ERR_WORKSPACE;
  const int64_t rows = (int64_t)B * (N + 1);
  const int64_t NB = nblocks(V), nch = cdiv(NB, CH);
  if (rows * nch > kMaxGrid) return SSD_ERR_UNSUPPORTED;
  Params& p = q.p;
  p = Params{};
  p.x = (const unsigned char*)a.target_logits;
  p.xd = (const unsigned char*)a.draft_logits;
  p.V = V; p.ld = ld; p.rows = rows; p.NB = (int)NB; p.nchunk = (int)nch;
  p.K = N; p.B = B;
  p.temp = a.temperature;
  p.F = F; p.C = C; p.seed = a.seed;
  p.part = (float4*)((char*)a.workspace + L.part);
  p.dtok = a.tokens;
  p.dq = a.draft_q;
  p.dstats = a.draft_stats;
  p.dtopf = F > 0 ? a.draft_topf_idx : nullptr;
  p.ld_dtopf = a.ld_topf;
  p.acc_len = a.out_accept_len;
  p.bonus = a.out_bonus;
  q.dt = a.dt;
  q.al = aligned16(a.target_logits, ld, V, a.dt) && aligned16(a.draft_logits, ld, V, a.dt);
  q.g_stream = rows * nch;
  q.g_tail = B;
  return SSD_OK;
}

// Scratch of ssd_round_noalloc on each GPU: the array below, whose address
// on device d comes from hipGetSymbolAddress, taken once per device with d
// current and kept (the array's name is a host-side stand-in, never an
// address host code may pass on).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch[kMaxDevices] = {};

ssd_status scratch_of(hipStream_t st, char** out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return SSD_ERR_HIP;
  int dev = cur;
  if (st) {
    hipDevice_t d = 0;
    if (hipStreamGetDevice(st, &d) != hipSuccess) return SSD_ERR_HIP;
    dev = (int)d;
  }
  if (dev < 0 || dev >= kMaxDevices) return SSD_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return SSD_ERR_HIP;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || ptr == nullptr || (uintptr_t)ptr % 256 != 0) return SSD_ERR_HIP;
    g_scratch[dev] = (char*)ptr;
  }
  *out = g_scratch[dev];
  return SSD_OK;
}

}  // namespace

extern "C" {

const char* ssd_status_string(ssd_status s) {
  switch (s) {
    case SSD_OK: return "SSD_OK";
    case SSD_ERR_INVALID_ARG: return "SSD_ERR_INVALID_ARG";
    case SSD_ERR_UNSUPPORTED: return "SSD_ERR_UNSUPPORTED";
    case SSD_ERR_WORKSPACE: return "SSD_ERR_WORKSPACE";
    case SSD_ERR_HIP: return "SSD_ERR_HIP";
    case SSD_ERR_SCRATCH_LIMIT: return "SSD_ERR_SCRATCH_LIMIT";
  }
  return "SSD_ERR_UNKNOWN";
}

size_t ssd_workspace_bytes(ssd_op op, int64_t n, int32_t K, int64_t V) {
  Layout L;
  return layout(op, n, K, V, &L) ? L.total : 0;
}

ssd_status ssd_softmax_t(const void* logits, ssd_dtype dt, int64_t rows, int64_t V, int64_t ld,
                         const float* temperature, ssd_row_stats* out_stats, float* out_probs,
                         void* workspace, size_t ws_bytes, void* stream) {
  if (!logits || !temperature || !out_stats || !dt_ok(dt)) return SSD_ERR_INVALID_ARG;
  if (rows < 1 || V < 1 || V > SSD_MAX_V || ld < V) return SSD_ERR_INVALID_ARG;
  Layout L;
  if (!layout(SSD_OP_SOFTMAX_T, rows, 0, V, &L)) return SSD_ERR_INVALID_ARG;
  if (!ws_ok(workspace, ws_bytes, L)) return SSD_ERR_WORKSPACE;
  const int64_t NB = nblocks(V), nch = cdiv(NB, CH);
  if (rows * nch > kMaxGrid || rows * cdiv(NB, NWAVE) > kMaxGrid) return SSD_ERR_UNSUPPORTED;
  Params p{};
  p.x = (const unsigned char*)logits;
  p.V = V; p.ld = ld; p.rows = rows; p.NB = (int)NB; p.nchunk = (int)nch;
  p.temp = temperature;
  char* ws = (char*)workspace;
  p.part = (float4*)(ws + L.part);
  p.stats = out_stats;
  p.probs = out_probs;
  const bool al = aligned16(logits, ld, V, dt);
  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();
  hipError_t e = timed(SSD_OP_SOFTMAX_T, [&](hipEvent_t e0, hipEvent_t e1) {
    return dispatch<LSoftmax>(dt, al, rows * nch, p, st, e0, e1);
  });
  if (e == hipSuccess) e = dispatch<LSoftmaxEpi>(dt, al, rows, p, st);
  if (e == hipSuccess && out_probs) {
    p.nchunk = (int)cdiv(NB, NWAVE);
    e = dispatch<LProbs>(dt, al, rows * p.nchunk, p, st);
  }
  return hip_status(e);
}

ssd_status ssd_topf(const void* logits, ssd_dtype dt, int64_t rows, int64_t V, int64_t ld, int32_t F,
                    int32_t* out_idx, float* out_val, void* workspace, size_t ws_bytes, void* stream) {
  if (!logits || !out_idx || !dt_ok(dt)) return SSD_ERR_INVALID_ARG;
  if (rows < 1 || V < 1 || V > SSD_MAX_V || ld < V) return SSD_ERR_INVALID_ARG;
  if (F < 1 || F > SSD_MAX_F || F > V) return SSD_ERR_INVALID_ARG;
  Layout L;
  if (!layout(SSD_OP_TOPF, rows, 0, V, &L)) return SSD_ERR_INVALID_ARG;
  if (!ws_ok(workspace, ws_bytes, L)) return SSD_ERR_WORKSPACE;
  const int64_t NB = nblocks(V), nch = cdiv(NB, CH);
  if (rows * nch > kMaxGrid) return SSD_ERR_UNSUPPORTED;
  Params p{};
  p.x = (const unsigned char*)logits;
  p.V = V; p.ld = ld; p.rows = rows; p.NB = (int)NB; p.nchunk = (int)nch;
  p.F = F; p.F_sel = F;
  char* ws = (char*)workspace;
  p.part = (float4*)(ws + L.part);
  p.out_idx = out_idx;
  p.out_val = out_val;
  const bool al = aligned16(logits, ld, V, dt);
  (void)hipGetLastError();
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = timed(SSD_OP_TOPF, [&](hipEvent_t e0, hipEvent_t e1) {
    return dispatch<LTopf>(dt, al, rows * nch, p, st, e0, e1);
  });
  if (e == hipSuccess) e = dispatch<LTopfEpi>(dt, al, rows, p, st);
  return hip_status(e);
}

ssd_status ssd_saguaro_sample(const void* draft_logits, ssd_dtype dt, int32_t B, int32_t K, int64_t V,
                              int64_t ld, const float* temperature, int32_t F, float C, int32_t F_out,
                              uint64_t seed, int32_t* out_tokens, float* out_q, ssd_row_stats* out_stats,
                              int32_t* out_topf_idx, float* out_topf_val, const ssd_cache* cache,
                              void* workspace, size_t ws_bytes, void* stream) {
  const ssd_sample_args a{draft_logits, dt, B, K, V, ld, temperature, F, C, F_out, seed, out_tokens, out_q,
                          out_stats, out_topf_idx, out_topf_val, cache, workspace, ws_bytes};
  Plan q;
  const ssd_status s = plan_sample(a, q);
  if (s != SSD_OK) return s;
  (void)hipGetLastError();
  return hip_status(launch_sample(q, (hipStream_t)stream));
}

ssd_status ssd_verify(const void* target_logits, const void* draft_logits, ssd_dtype dt, int32_t B, int32_t K,
                      int64_t V, int64_t ld, const float* temperature, int32_t F, float C, uint64_t seed,
                      const int32_t* draft_tokens, const float* draft_q, const ssd_row_stats* draft_stats,
                      const int32_t* draft_topf_idx, int32_t ld_topf, int32_t* out_accept_len,
                      int32_t* out_bonus, float* out_p, ssd_row_stats* out_target_stats, const ssd_cache* cache,
                      void* workspace, size_t ws_bytes, void* stream) {
  const ssd_verify_args a{target_logits, draft_logits, dt, B, K, V, ld, temperature, F, C, seed, draft_tokens,
                          draft_q, draft_stats, draft_topf_idx, ld_topf, out_accept_len, out_bonus, out_p,
                          out_target_stats, cache, workspace, ws_bytes};
  Plan q;
  const ssd_status s = plan_verify(a, q);
  if (s != SSD_OK) return s;
  (void)hipGetLastError();
  return hip_status(launch_verify(q, (hipStream_t)stream));
}

// Checks of an early-exit verification on its plan.
ssd_status check_early(const Plan& q, const ssd_verify_args& a, int32_t J) {
  const int K1 = q.p.K + 1;
  if (J < 1 || J > K1 || a.out_target_stats) return SSD_ERR_INVALID_ARG;
  if ((int64_t)q.p.B * K1 * q.p.nchunk > kMaxGrid) return SSD_ERR_UNSUPPORTED;
  return SSD_OK;
}

// The streaming part of an early-exit verification: positions 0 .. J-1 of
// every sequence; the gate, decided once per sequence; then J .. K of the
// sequences with no clear rejection below J.
hipError_t launch_early_streams(const Plan& q, int32_t J, hipStream_t st) {
  const int K1 = q.p.K + 1;
  const int64_t nch = q.p.nchunk;
  Params p = q.p;
  p.early = 1;
  p.jlo = 0;
  p.jn = J;
  p.gate_reset = 1;
  hipError_t e = dispatch<LVerify>(q.dt, q.al, (int64_t)p.B * J * nch, p, st);
  if (e == hipSuccess && J < K1) {
    Params pg = p;
    pg.gate_reset = 0;
    pg.jlo = J;
    pg.jn = K1 - J;
    e = dispatch<LGate>(q.dt, q.al, (int64_t)p.B, pg, st);
    if (e == hipSuccess) e = dispatch<LVerifyGated>(q.dt, q.al, (int64_t)p.B * (K1 - J) * nch, pg, st);
  }
  return e;
}

// An early-exit verification: its streaming part, then the verification of
// each sequence.
hipError_t launch_verify_early(const Plan& q, int32_t J, hipStream_t st) {
  hipError_t e = launch_early_streams(q, J, st);
  Params p = q.p;
  p.early = 1;
  if (e == hipSuccess) e = dispatch<LVerifySeq>(q.dt, q.al, q.g_tail, p, st);
  return e;
}

ssd_status ssd_verify_early(const ssd_verify_args* a, int32_t J, void* stream) {
  if (!a) return SSD_ERR_INVALID_ARG;
  Plan q;
  ssd_status s = plan_verify(*a, q);
  if (s != SSD_OK) return s;
  s = check_early(q, *a, J);
  if (s != SSD_OK) return s;
  (void)hipGetLastError();
  return hip_status(launch_verify_early(q, J, (hipStream_t)stream));
}

ssd_status ssd_round_early(const ssd_verify_args* v, const ssd_sample_args* s, int32_t J, void* stream) {
  Plan qv, qs;
  ssd_status e = plan_round(v, s, qv, qs);
  if (e != SSD_OK) return e;
  if (v) {
    e = check_early(qv, *v, J);
    if (e != SSD_OK) return e;
  }
  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();
  if (!v) return hip_status(launch_sample(qs, st));
  if (!s || qv.dt != qs.dt || qv.al != qs.al || qs.p.rows <= kTwoLaunchRows) {
    // alone, with element types that cannot share a launch, or at small
    // batches (where early exit saves less than its launches cost): in turn
    hipError_t he = launch_verify_early(qv, J, st);
    if (he == hipSuccess && s) he = launch_sample(qs, st);
    return hip_status(he);
  }
  // the early-exit streaming part of round i; then the verification of each
  // sequence beside round i+1's streaming pass; then its epilogue
  hipError_t he = launch_early_streams(qv, J, st);
  Params pv = qv.p;
  pv.early = 1;
  const int64_t nv = qv.g_tail;
  if (he == hipSuccess) {
    he = timed(SSD_OP_SAMPLE, [&](hipEvent_t e0, hipEvent_t e1) {
      return e0 ? dispatch<LRoundMidT>(qv.dt, qv.al, nv + qs.g_stream, pv, qs.p, (int)nv, st, e0, e1)
                : dispatch<LRoundMid>(qv.dt, qv.al, nv + qs.g_stream, pv, qs.p, (int)nv, st);
    });
  }
  if (he == hipSuccess) he = dispatch<LSampleEpi>(qs.dt, qs.al, qs.g_tail, qs.p, st);
  return hip_status(he);
}

ssd_status ssd_round(const ssd_verify_args* v, const ssd_sample_args* s, void* stream) {
  Plan qv, qs;
  const ssd_status e = plan_round(v, s, qv, qs);
  if (e != SSD_OK) return e;
  return launch_round(v ? &qv : nullptr, s ? &qs : nullptr, (hipStream_t)stream);
}

ssd_status ssd_round_noalloc(const ssd_verify_args* v, const ssd_sample_args* s, void* stream) {
  if (!v && !s) return SSD_ERR_INVALID_ARG;
  // every argument is checked before any HIP call: sizes against the scratch
  // halves, then the full plan on stand-in addresses (never dereferenced)
  ssd_verify_args va{};
  ssd_sample_args sa{};
  if (v) {
    const size_t n = ssd_workspace_bytes(SSD_OP_VERIFY, v->B, v->K, v->V);
    if (n == 0) return SSD_ERR_INVALID_ARG;
    if (n > kScratchHalf) return SSD_ERR_SCRATCH_LIMIT;
    va = *v;
    va.workspace = reinterpret_cast<void*>(uintptr_t(256));
    va.ws_bytes = kScratchHalf;
  }
  if (s) {
    const size_t n = ssd_workspace_bytes(SSD_OP_SAMPLE, s->B, s->K, s->V);
    if (n == 0) return SSD_ERR_INVALID_ARG;
    if (n > kScratchHalf) return SSD_ERR_SCRATCH_LIMIT;
    sa = *s;
    sa.workspace = reinterpret_cast<void*>(uintptr_t(512));
    sa.ws_bytes = kScratchHalf;
  }
  Plan qv, qs;
  ssd_status e = plan_round(v ? &va : nullptr, s ? &sa : nullptr, qv, qs);
  if (e != SSD_OK) return e;
  hipStream_t st = (hipStream_t)stream;
  char* base = nullptr;
  e = scratch_of(st, &base);
  if (e != SSD_OK) return e;
  // verification in the first half, sampling in the second
  if (v) va.workspace = base;
  if (s) sa.workspace = base + kScratchHalf;
  e = plan_round(v ? &va : nullptr, s ? &sa : nullptr, qv, qs);
  if (e != SSD_OK) return e;
  return launch_round(v ? &qv : nullptr, s ? &qs : nullptr, st);
}

ssd_status ssd_verify_tree(const ssd_tree_args* a, void* stream) {
  if (!a) return SSD_ERR_INVALID_ARG;
  Plan q;
  TreeArgs ta;
  const ssd_status e0 = plan_tree(*a, q, ta);
  if (e0 != SSD_OK) return e0;
  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();
  // every node's target row streamed once (no drafted-token capture: a
  // node's children are evaluated at its row), then the walk
  Params ps = q.p;
  ps.dtok = nullptr;
  hipError_t e = dispatch<LVerify>(q.dt, q.al, q.g_stream, ps, st);
  if (e == hipSuccess) e = dispatch<LTree>(q.dt, q.al, q.g_tail, q.p, ta, st);
  return hip_status(e);
}

ssd_status ssd_cache_lookup(const int32_t* keys, const int32_t* depth_off, const int32_t* payload, int32_t B,
                            int32_t K, int32_t Bgt, const int32_t* accept_len, const int32_t* bonus,
                            int32_t* out_hit, int32_t* out_slot, int32_t* out_tokens, int32_t miss_fill,
                            int64_t V, uint64_t seed, void* stream) {
  if (B < 1 || K < 0 || K > SSD_MAX_K || Bgt < 0) return SSD_ERR_INVALID_ARG;
  if (miss_fill != 0 && miss_fill != 1) return SSD_ERR_INVALID_ARG;
  if (miss_fill && (V < 1 || V > SSD_MAX_V)) return SSD_ERR_INVALID_ARG;
  if (!depth_off || !accept_len || !bonus || !out_hit || !out_slot) return SSD_ERR_INVALID_ARG;
  if (Bgt > 0 && !keys) return SSD_ERR_INVALID_ARG;
  if (K > 0 && Bgt > 0 && !payload) return SSD_ERR_INVALID_ARG;
  if (K > 0 && !out_tokens) return SSD_ERR_INVALID_ARG;
  (void)hipGetLastError();
  k_lookup<<<dim3((unsigned)cdiv(B, NWAVE)), dim3(WG), 0, (hipStream_t)stream>>>(
      keys, depth_off, payload, B, K, Bgt, accept_len, bonus, out_hit, out_slot, out_tokens, V, seed, miss_fill);
  return hip_status(hipGetLastError());
}

ssd_status ssd_cache_keys(const int32_t* topf_idx, int32_t ld_topf, const int32_t* depth_off, int32_t B,
                          int32_t K, int32_t Bgt, int32_t* out_keys, void* stream) {
  if (B < 1 || K < 0 || K > SSD_MAX_K || Bgt < 0 || ld_topf < 0) return SSD_ERR_INVALID_ARG;
  if (!depth_off || (Bgt > 0 && (!out_keys || (ld_topf > 0 && !topf_idx)))) return SSD_ERR_INVALID_ARG;
  if (Bgt == 0) return SSD_OK;
  const int64_t n = (int64_t)B * Bgt;
  if (cdiv(n, WG) > kMaxGrid) return SSD_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  k_cache_keys<<<dim3((unsigned)cdiv(n, WG)), dim3(WG), 0, (hipStream_t)stream>>>(topf_idx, ld_topf, depth_off,
                                                                                  B, K, Bgt, out_keys);
  return hip_status(hipGetLastError());
}

ssd_status ssd_read_probe(const void* buf, size_t bytes, int32_t variant, uint32_t* out, size_t out_len,
                          void* stream) {
  if (!buf || !out || bytes < 16 || (uintptr_t)buf % 16 != 0) return SSD_ERR_INVALID_ARG;
  const int64_t n16 = (int64_t)(bytes / 16);
  hipStream_t st = (hipStream_t)stream;
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return SSD_ERR_HIP;
  // (threads, loads per thread, nontemporal, grid kind, workgroups per CU)
  struct V { int wgt, l; bool nt; int kind; int per_cu; };
  static const V vs[] = {
      {256, 8, true, 0, 0},  {256, 16, true, 0, 0}, {512, 8, true, 0, 0},  {1024, 8, true, 0, 0},
      {256, 8, false, 0, 0}, {256, 8, true, 2, 8},  {512, 8, true, 2, 4},  {256, 4, true, 0, 0},
      {1024, 4, true, 0, 0}, {1024, 4, true, 2, 2}, {256, 8, true, 1, 0},  {512, 16, true, 0, 0},
  };
  if (variant < 0 || variant >= (int)(sizeof(vs) / sizeof(vs[0]))) return SSD_ERR_INVALID_ARG;
  const V v = vs[variant];
  const int64_t nchunk = cdiv(n16, (int64_t)v.wgt * v.l);
  const int64_t grid = v.kind == 2 ? std::min<int64_t>(nchunk, (int64_t)ncu * v.per_cu) : nchunk;
  if (grid > kMaxGrid || (size_t)grid > out_len) return SSD_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  const u32x4* p = (const u32x4*)buf;
  const dim3 g((unsigned)grid);
#define SSD_PROBE_ONCE(W, LL, N, X) k_probe_once<W, LL, N, X><<<g, dim3(W), 0, st>>>(p, n16, out)
#define SSD_PROBE_PERSIST(W, LL, N) k_probe_persist<W, LL, N><<<g, dim3(W), 0, st>>>(p, n16, nchunk, out)
  switch (variant) {
    case 0: SSD_PROBE_ONCE(256, 8, true, false); break;
    case 1: SSD_PROBE_ONCE(256, 16, true, false); break;
    case 2: SSD_PROBE_ONCE(512, 8, true, false); break;
    case 3: SSD_PROBE_ONCE(1024, 8, true, false); break;
    case 4: SSD_PROBE_ONCE(256, 8, false, false); break;
    case 5: SSD_PROBE_PERSIST(256, 8, true); break;
    case 6: SSD_PROBE_PERSIST(512, 8, true); break;
    case 7: SSD_PROBE_ONCE(256, 4, true, false); break;
    case 8: SSD_PROBE_ONCE(1024, 4, true, false); break;
    case 9: SSD_PROBE_PERSIST(1024, 4, true); break;
    case 10: SSD_PROBE_ONCE(256, 8, true, true); break;
    case 11: SSD_PROBE_ONCE(512, 16, true, false); break;
  }
#undef SSD_PROBE_ONCE
#undef SSD_PROBE_PERSIST
  return hip_status(hipGetLastError());
}

ssd_status ssd_phase_read(int32_t kind, uint64_t* out, int64_t n) {
  if (kind < 0 || kind > 1 || !out || n < 0 || n > (int64_t)PH_ITEMS * PH_N) return SSD_ERR_INVALID_ARG;
#ifdef SSD_PHASES
  const hipError_t e = hipMemcpyFromSymbol(out, HIP_SYMBOL(g_phase), (size_t)n * sizeof(uint64_t),
                                           (size_t)kind * PH_ITEMS * PH_N * sizeof(uint64_t));
  return hip_status(e);
#else
  return SSD_ERR_UNSUPPORTED;
#endif
}

ssd_status ssd_timer_enable(int32_t max_launches) {
  if (max_launches < 0 || max_launches > (1 << 20)) return SSD_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(g_timer_mu);
  timer_free();
  if (max_launches == 0) return SSD_OK;
  for (auto& v : g_timer.ev) {
    v.resize(2 * (size_t)max_launches);
    for (hipEvent_t& e : v) {
      if (hipEventCreate(&e) != hipSuccess) {
        e = nullptr;
        timer_free();
        return SSD_ERR_HIP;
      }
    }
  }
  g_timer.cap = max_launches;
  return SSD_OK;
}

ssd_status ssd_timer_read(ssd_op op, int32_t* launches, double* total_ms) {
  if (op < SSD_OP_SOFTMAX_T || op > SSD_OP_VERIFY || !launches || !total_ms) return SSD_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(g_timer_mu);
  double t = 0.0;
  for (int i = 0; i < g_timer.n[op]; ++i) {
    float ms = 0.f;
    if (hipEventSynchronize(g_timer.ev[op][2 * i + 1]) != hipSuccess ||
        hipEventElapsedTime(&ms, g_timer.ev[op][2 * i], g_timer.ev[op][2 * i + 1]) != hipSuccess)
      return SSD_ERR_HIP;
    t += ms;
  }
  *launches = g_timer.n[op];
  *total_ms = t;
  return SSD_OK;
}

ssd_status ssd_fanout(int32_t Bgt, int32_t K, double ratio, int64_t V, int32_t* out_F) {
  if (!out_F || Bgt < 0 || K < 0 || K > SSD_MAX_K || V < 1) return SSD_ERR_INVALID_ARG;
  if (!isfinite(ratio) || !(ratio > 0.0)) return SSD_ERR_INVALID_ARG;
  if ((int64_t)Bgt > (int64_t)(K + 1) * V) return SSD_ERR_INVALID_ARG;
  double w[SSD_MAX_K + 1], ideal[SSD_MAX_K + 1], frac[SSD_MAX_K + 1];
  int64_t F[SSD_MAX_K + 1];
  double x = 1.0;
  for (int k = 0; k <= K; ++k) {
    w[k] = x;
    x = x * ratio;
  }
  double S = 0.0;
  for (int k = 0; k <= K; ++k) S = S + w[k];
  int64_t used = 0;
  for (int k = 0; k <= K; ++k) {
    ideal[k] = (double)Bgt * w[k] / S;
    const double fl = floor(ideal[k]);
    F[k] = (int64_t)fl;
    frac[k] = ideal[k] - fl;
    used += F[k];
  }
  int64_t rem = (int64_t)Bgt - used;
  bool taken[SSD_MAX_K + 1] = {};
  while (rem > 0) {  // largest fractional part first, ties to the smaller k
    int best = -1;
    for (int k = 0; k <= K; ++k)
      if (!taken[k] && (best < 0 || frac[k] > frac[best])) best = k;
    taken[best] = true;
    F[best] += 1;
    --rem;
  }
  int64_t excess = 0;
  for (int k = 0; k <= K; ++k)
    if (F[k] > V) {
      excess += F[k] - V;
      F[k] = V;
    }
  for (int k = 0; k <= K && excess > 0; ++k) {
    const int64_t give = excess < V - F[k] ? excess : V - F[k];
    F[k] += give;
    excess -= give;
  }
  for (int k = 0; k <= K; ++k) out_F[k] = (int32_t)F[k];
  return SSD_OK;
}

ssd_status ssd_fanout_greedy(const double* a, const double* h, int32_t K, int32_t Fmax, int32_t Bgt,
                             int32_t* out_F) {
  if (!a || !h || !out_F || K < 0 || K > SSD_MAX_K || Fmax < 1 || Fmax > SSD_MAX_F || Bgt < 0)
    return SSD_ERR_INVALID_ARG;
  if ((int64_t)Bgt > (int64_t)(K + 1) * Fmax) return SSD_ERR_INVALID_ARG;
  for (int64_t i = 0; i < (int64_t)(K + 1) * (Fmax + 1); ++i)
    if (!std::isfinite(h[i])) return SSD_ERR_INVALID_ARG;
  for (int k = 0; k <= K; ++k)
    if (!std::isfinite(a[k]) || a[k] < 0.0) return SSD_ERR_INVALID_ARG;
  std::vector<int32_t> F(K + 1, 0);
  for (int32_t n = 0; n < Bgt; ++n) {
    // the slot goes to the largest marginal gain; ties to the smaller depth
    double best = -INFINITY;
    int bk = -1;
    for (int k = 0; k <= K; ++k) {
      if (F[k] >= Fmax) continue;
      const double* hk = h + (int64_t)k * (Fmax + 1);
      const double g = a[k] * (hk[F[k] + 1] - hk[F[k]]);
      if (g > best) {
        best = g;
        bk = k;
      }
    }
    ++F[bk];
  }
  for (int k = 0; k <= K; ++k) out_F[k] = F[k];
  return SSD_OK;
}

ssd_status ssd_backoff(const double* p_hit, int32_t B, const ssd_backoff_cost* c, int32_t* out_use_fast,
                       double* out_gain) {
  if (!p_hit || !c || !out_use_fast || B < 1) return SSD_ERR_INVALID_ARG;
  if (!(c->t_round > 0.0) || !(c->t_slow >= 0.0) || !(c->t_fast >= 0.0) || !(c->e_acc > 0.0) ||
      !(c->e_fast >= 0.0) || !std::isfinite(c->t_round) || !std::isfinite(c->t_slow) || !std::isfinite(c->t_fast) ||
      !std::isfinite(c->e_acc) || !std::isfinite(c->e_fast))
    return SSD_ERR_INVALID_ARG;
  double P = 1.0, mix = 0.0;
  for (int32_t b = 0; b < B; ++b) {
    const double p = p_hit[b];
    if (!(p >= 0.0 && p <= 1.0)) return SSD_ERR_INVALID_ARG;
    P *= p;
    mix += p * c->e_acc + (1.0 - p) * c->e_fast;
  }
  // tokens per unit time with each backup; a round with any miss waits for it
  const double r_acc = (double)B * c->e_acc / (c->t_round + (1.0 - P) * c->t_slow);
  const double r_fast = mix / (c->t_round + (1.0 - P) * c->t_fast);
  const double gain = r_fast / r_acc;
  *out_use_fast = gain > 1.0 ? 1 : 0;
  if (out_gain) *out_gain = gain;
  return SSD_OK;
}

}  // extern "C"
