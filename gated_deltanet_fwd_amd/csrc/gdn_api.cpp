// Host side of the C ABI in include/gdn.h: validation, buffer layouts, saved-set tagging and the
// launch sequence of each call. No device memory is allocated or freed here, no stream is
// created and nothing synchronises (except the gdn_status query). Launches go to the caller's
// stream; when one document's chain work dominates and the caller names an auxiliary stream,
// the other documents' intra and walk launches go to that stream, forked from and joined back
// into the caller's stream with events from a per-thread pool.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "gdn.h"
#include "gdn_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

constexpr int kChunk = 64;
constexpr size_t kAlign = 256;
constexpr size_t kTagBytes = 256;
constexpr uint64_t kMagic = 0x32564153'4e4447ULL; // "GDNSAV2"

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Sizes {
  int64_t T;
  int N, H, HV, D, NT;
};

// Validates the descriptor and its host cu_seqlens; fills sizes. Returns GDN_OK or an error.
int check_problem(const gdn_problem* p, Sizes* s) {
  if (!p) return fail(GDN_EINVAL, "problem descriptor is NULL");
  if (p->n_seqs < 1) return fail(GDN_EINVAL, "n_seqs must be >= 1 (got %d)", p->n_seqs);
  if (p->h_qk < 1 || p->h_v < 1) return fail(GDN_EINVAL, "head counts must be >= 1");
  if (p->h_v % p->h_qk != 0) return fail(GDN_EINVAL, "h_v (%d) must be a multiple of h_qk (%d)", p->h_v, p->h_qk);
  if (p->d != 64 && p->d != 128) return fail(GDN_EUNSUPPORTED, "d must be 64 or 128 (got %d)", p->d);
  if (p->dtype != GDN_DTYPE_BF16 && p->dtype != GDN_DTYPE_F32)
    return fail(GDN_EUNSUPPORTED, "unsupported dtype %d", p->dtype);
  if (p->save_mode != GDN_SAVE_LIGHT && p->save_mode != GDN_SAVE_FULL && p->save_mode != GDN_SAVE_TAPE)
    return fail(GDN_EINVAL, "save_mode must be light (0), full (1) or tape (2)");
  if (p->segments < 0) return fail(GDN_EINVAL, "segments must be >= 0 (got %d)", p->segments);
  if (p->reserved0 != 0) return fail(GDN_EINVAL, "reserved0 must be 0");
  if (!p->cu_seqlens_host) return fail(GDN_EINVAL, "cu_seqlens_host is NULL");
  const int32_t* cu = p->cu_seqlens_host;
  if (cu[0] != 0) return fail(GDN_EINVAL, "cu_seqlens[0] must be 0");
  int64_t nt = 0;
  for (int n = 0; n < p->n_seqs; ++n) {
    if (cu[n + 1] < cu[n]) return fail(GDN_EINVAL, "cu_seqlens decreases at %d", n);
    nt += (cu[n + 1] - cu[n] + kChunk - 1) / kChunk;
  }
  if ((int64_t)cu[p->n_seqs] != p->n_tokens)
    return fail(GDN_EINVAL, "cu_seqlens[N] = %d but n_tokens = %lld", cu[p->n_seqs], (long long)p->n_tokens);
  if (nt > (int64_t)0x7fffffff / 64) return fail(GDN_EINVAL, "too many chunks");
  if ((int64_t)p->n_seqs * p->h_qk > (int64_t)0x0fffffff) return fail(GDN_EINVAL, "too many documents x heads");
  s->T = p->n_tokens;
  s->N = p->n_seqs;
  s->H = p->h_qk;
  s->HV = p->h_v;
  s->D = p->d;
  s->NT = (int)nt;
  return GDN_OK;
}

// The saved set keeps the state tape in the full and the kept-tape forms; the full form also
// keeps v_new, w, u and the q.k rows.
bool keeps_tape(int save_mode) { return save_mode == GDN_SAVE_FULL || save_mode == GDN_SAVE_TAPE; }

struct SavedLayout {
  size_t akk, gcum, gamma, htape, vnew, w, u, aqk, plane, total;
};

SavedLayout saved_layout(const Sizes& s, int save_mode, int plane_slots = 0) {
  SavedLayout L{};
  size_t off = kTagBytes;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L.akk = take((size_t)s.T * s.HV * kChunk * 2);
  L.gcum = take((size_t)s.T * s.HV * 4);
  L.gamma = take((size_t)s.NT * s.HV * 4);
  if (keeps_tape(save_mode)) L.htape = take((size_t)s.NT * s.HV * s.D * s.D * 2);
  if (save_mode == GDN_SAVE_FULL) {
    L.vnew = take((size_t)s.T * s.HV * s.D * 2);
    L.w = take((size_t)s.T * s.HV * s.D * 2);
    L.u = take((size_t)s.T * s.HV * s.D * 2);
    L.aqk = take((size_t)s.T * s.HV * kChunk * 2);
  }
  // segmented walks: the segments' FP32 start states (the carry plane)
  if (plane_slots > 0) L.plane = take((size_t)plane_slots * s.HV * s.D * s.D * 4);
  L.total = off;
  return L;
}

struct WorkLayout {
  size_t seq_c0, c_t0, c_len, seq_order, pair_order, status, rk, rq, qk, htape, dstape, dqacc, dkacc, state,
      carry, queue, total;
};

WorkLayout work_layout(const Sizes& s, int op, int save_mode, int deterministic, int carry_slots = 0) {
  WorkLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L.seq_c0 = take((size_t)(s.N + 1) * 4);
  L.c_t0 = take((size_t)s.NT * 4);
  L.c_len = take((size_t)s.NT * 4);
  L.seq_order = take((size_t)s.N * 4);
  L.pair_order = take(((size_t)(s.N * s.H + 7) / 8 + 1) * 2 * 4);
  L.status = take(4);
  L.rk = take((size_t)s.T * s.H * 4);
  L.rq = take((size_t)s.T * s.H * 4);
  L.qk = take((size_t)s.NT * s.HV * kChunk * kChunk * 2);
  // the state handed from one piece of the longest document's walk to the next
  if (op != GDN_OP_BWD) L.state = take((size_t)s.HV * s.D * s.D * 4);
  // segmented walks: start states, transfer matrices and zero-start end states of the segments
  if (op != GDN_OP_BWD && carry_slots > 0) L.carry = take((size_t)carry_slots * s.HV * s.D * s.D * 4);
  if (op == GDN_OP_BWD) {
    L.queue = take(2 * 4); // chunk-gradient work queues of the two parts
    if (!keeps_tape(save_mode)) L.htape = take((size_t)s.NT * s.HV * s.D * s.D * 2);
    L.dstape = take((size_t)s.NT * s.HV * s.D * s.D * 2);
    if (!deterministic) {
      L.dqacc = take((size_t)s.T * s.H * s.D * 4);
      L.dkacc = take((size_t)s.T * s.H * s.D * 4);
    }
  }
  L.total = off;
  return L;
}

uint64_t fnv(uint64_t h, const void* data, size_t n) {
  const unsigned char* b = (const unsigned char*)data;
  for (size_t i = 0; i < n; ++i) {
    h ^= b[i];
    h *= 1099511628211ULL;
  }
  return h;
}

uint64_t problem_hash(const gdn_problem* p) {
  uint64_t h = 1469598103934665603ULL;
  const int32_t f[] = {p->n_seqs, p->h_qk, p->h_v, p->d, p->dtype, p->l2norm_qk, p->has_h0, p->save_mode};
  h = fnv(h, f, sizeof f);
  h = fnv(h, &p->n_tokens, sizeof p->n_tokens);
  h = fnv(h, p->cu_seqlens_host, sizeof(int32_t) * (size_t)(p->n_seqs + 1));
  return h;
}

// The four words of the saved set's tag for this problem: magic, ABI version, save mode and
// the hash of the problem (sizes, flags, cu_seqlens). gdn_fwd / gdn_fwd_recompute write them,
// the first kernel of gdn_bwd compares them.
void tag_words(const gdn_problem* p, uint64_t w[4]) {
  w[0] = kMagic;
  w[1] = (uint64_t)GDN_ABI_VERSION;
  w[2] = (uint64_t)p->save_mode;
  w[3] = problem_hash(p);
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

int check_ptr(const void* ptr, const char* name) {
  if (!ptr) return fail(GDN_EINVAL, "%s is NULL", name);
  if (!aligned16(ptr)) return fail(GDN_EINVAL, "%s is not 16-byte aligned", name);
  return GDN_OK;
}

#define CHECK(x)                     \
  do {                               \
    const int rc_ = (x);             \
    if (rc_ != GDN_OK) return rc_;   \
  } while (0)

// Optional kernel timing for benchmarks: while enabled, each launch is bracketed by two
// hipEvents recorded on the stream it goes to; gdn_timing_collect waits for them and sums the
// elapsed time per kernel name, gdn_timing_launches returns each launch's start and end.
std::atomic<int> g_timing_on{0};
std::mutex g_timing_mu;
struct PendingEvent {
  const char* name;
  hipEvent_t start, stop;
};
std::vector<PendingEvent> g_pending;
std::map<std::string, std::pair<double, int>> g_totals;

hipEvent_t timing_begin(void* stream) {
  if (!g_timing_on.load(std::memory_order_relaxed)) return nullptr;
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  hipEventRecord(e, (hipStream_t)stream);
  return e;
}

void timing_end(const char* name, hipEvent_t start, void* stream) {
  if (!start) return;
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) {
    hipEventDestroy(start);
    return;
  }
  hipEventRecord(e, (hipStream_t)stream);
  std::lock_guard<std::mutex> lk(g_timing_mu);
  g_pending.push_back({name, start, e});
}

#define LAUNCH_ON(st, name, x)                                                           \
  do {                                                                                   \
    hipEvent_t t0_ = timing_begin(st);                                                   \
    const int e_ = (x);                                                                  \
    timing_end(name, t0_, st);                                                           \
    if (e_ != 0) return fail(GDN_EHIP, "%s: %s", #x, hipGetErrorString((hipError_t)e_)); \
  } while (0)
#define LAUNCH(name, x) LAUNCH_ON(stream, name, x)

// Events for ordering the caller's two streams: a pool per thread and device, reused by every
// call of the thread (a wait enqueued with hipStreamWaitEvent refers to the record made before
// it, so recording the same event again in a later call is safe). The events live until the
// process ends.
struct EventPool {
  std::vector<hipEvent_t> ev;
  size_t next = 0;
};
thread_local std::unordered_map<int, EventPool> t_pools;

struct CallEvents {
  EventPool* pool = nullptr;
  int take(hipEvent_t* out) {
    if (!pool) {
      int dev = 0;
      if (hipGetDevice(&dev) != hipSuccess) return fail(GDN_EHIP, "hipGetDevice failed");
      pool = &t_pools[dev];
      pool->next = 0;
    }
    if (pool->next == pool->ev.size()) {
      hipEvent_t e = nullptr;
      if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess)
        return fail(GDN_EHIP, "hipEventCreate failed");
      pool->ev.push_back(e);
    }
    *out = pool->ev[pool->next++];
    return GDN_OK;
  }
  // Orders `to` after the work enqueued so far on `from`.
  int order(hipStream_t from, hipStream_t to) {
    hipEvent_t e = nullptr;
    CHECK(take(&e));
    hipError_t r = hipEventRecord(e, from);
    if (r == hipSuccess) r = hipStreamWaitEvent(to, e, 0);
    if (r != hipSuccess) return fail(GDN_EHIP, "stream fork/join: %s", hipGetErrorString(r));
    return GDN_OK;
  }
};

void fill_common(gdn::Args& a, const Sizes& s, const gdn_problem* p) {
  std::memset(&a, 0, sizeof a);
  a.N = s.N;
  a.H = s.H;
  a.HV = s.HV;
  a.G = s.HV / s.H;
  a.D = s.D;
  a.NT = s.NT;
  a.T = s.T;
  a.dtype = p->dtype;
  a.l2norm = p->l2norm_qk ? 1 : 0;
  a.has_h0 = p->has_h0 ? 1 : 0;
  a.want_ht = p->want_ht ? 1 : 0;
  a.full = p->save_mode == GDN_SAVE_FULL ? 1 : 0;
  gdn::whole_range(a);
}

// Two-part launch plan. The walks are serial over a document's chunks, so the longest document
// sets their run time while the others' chains finish early and leave CUs idle. When it is
// clearly the longest (at least 5/4 of the next one, and at least 64 chunks) and the caller gave
// an auxiliary stream, its intra and walk launches (part A) run on the caller's stream and the
// other documents' (part B) on the auxiliary stream: its walk then starts after its own intra
// launch rather than after everyone's, and part B fills the CUs that part A leaves free.
struct Split {
  bool on = false;
  int n0 = 0;          // the longest document (ties: the lowest index), rank 0 of the tables
  int cA0 = 0, cA = 0; // its chunks: [cA0, cA0 + cA)
};

Split plan_split(const gdn_problem* p, const Sizes& s) {
  Split sp;
  if (s.N < 2 || s.N > 8192) return sp; // the device tables keep the identity order above 8192
  const int32_t* cu = p->cu_seqlens_host;
  // rank 0 of the device tables: the most tokens, ties to the lowest index
  int len0 = -1;
  for (int n = 0; n < s.N; ++n)
    if (cu[n + 1] - cu[n] > len0) {
      len0 = cu[n + 1] - cu[n];
      sp.n0 = n;
    }
  int c1 = 0;
  for (int n = 0; n < s.N; ++n) {
    const int c = (cu[n + 1] - cu[n] + kChunk - 1) / kChunk;
    if (n < sp.n0) sp.cA0 += c;
    else if (n == sp.n0) sp.cA = c;
    if (n != sp.n0 && c > c1) c1 = c;
  }
  sp.on = sp.cA >= 64 && 4 * sp.cA >= 5 * c1;
  return sp;
}

// Segment plan (problem->segments >= 2, or the library's count for 0). Document n of c_n chunks is
// walked as P_n = min(segments, c_n / kMinSegChunks) segments of about equal length (at least 1).
//   forward: phase 1 walks every document's segment 0 truly (a document of one segment whole),
//     beside the transfer walks of the middle segments 1 .. P_n - 2 (from the identity with v = 0,
//     and from zero); the carry merge composes the middle segments' start states; phase 2 walks
//     segments 1 .. P_n - 1 from them. The start states S_in(1 .. P_n - 1) are the saved set's
//     carry plane (as the pages' saved set keeps its per-segment FP32 carry states at P > 1).
//   light recompute: the plane again (segment 0 walked to its end, the transfer walks, the merge).
//   light backward: the state tape replayed one segment per chain from the saved plane, beside
//     the reverse walk (which walks each document whole).
// If a table of the plan would not hold its units, the largest segment count is lowered; a
// problem with more documents than a table holds is walked unsegmented.
constexpr int kMinSegChunks = 8;

struct SegPlans {
  bool on = false;
  gdn::SegPlan phase1{}, transfer{}, phase2{}, recompute{}, replay{};
  gdn::MergePlan merge{};
  int plane_slots = 0, work_slots = 0;
};

// CUs of the current device (256 when no device can be queried, e.g. a host-only byte query).
int device_cus() {
  static std::mutex mu;
  static std::unordered_map<int, int> cache;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  cache[dev] = n;
  return n;
}

// The segment count of the library's plan (segments = 0), from the problem's shape and the CU
// count only: split only when the unsegmented chains (documents x value heads) fill at most half
// of the CUs, then as many segments (at most 8) as keep phase 1 (every document's first segment
// and the middle segments' two transfer walks, one workgroup per value head each) within about
// 1.25 rounds of the CUs. Measured on one MI355X (forward, bf16, (16, 48), d = 128): the
// 8,192-token document 0.52 -> 0.38 ms at 4 segments; the two-fragment 65,536-token share
// 2.52 -> 2.01 ms at 3; the 4-document 262,144-token pack slower at every count (its 192 chains
// already fill the chip, and its longest document's intra pass hides behind the others' walks
// only unsegmented).
int auto_segments(const Sizes& s, const std::vector<int>& chunks) {
  const int cus = device_cus();
  if ((long)s.N * s.HV * 2 > cus) return 1;
  int long_docs = 0;
  for (int c : chunks) long_docs += c >= 2 * kMinSegChunks ? 1 : 0;
  if (long_docs == 0) return 1;
  int best = 1;
  for (int P = 2; P <= 8; ++P)
    if ((long)s.N * s.HV + 2L * (P - 2) * long_docs * s.HV <= (long)cus * 5 / 4) best = P;
  return best;
}

SegPlans plan_segments(const gdn_problem* p, const Sizes& s) {
  SegPlans sp;
  const int U = gdn::MAX_SEG_UNITS;
  if (p->segments == 1 || s.N > U) return sp;
  const int32_t* cu = p->cu_seqlens_host;
  std::vector<int> chunks(s.N), P(s.N);
  for (int n = 0; n < s.N; ++n) chunks[n] = (cu[n + 1] - cu[n] + kChunk - 1) / kChunk;
  int pmax = p->segments >= 2 ? p->segments : auto_segments(s, chunks);
  for (; pmax >= 2; --pmax) {
    int nt = 0, n2 = 0, nm = 0, nseg = 0;
    for (int n = 0; n < s.N; ++n) {
      P[n] = std::max(1, std::min(pmax, chunks[n] / kMinSegChunks));
      nt += 2 * std::max(0, P[n] - 2);
      n2 += P[n] - 1;
      nm += P[n] >= 3 ? 1 : 0;
      nseg += P[n] >= 2 ? 1 : 0;
    }
    if (nseg == 0) return sp;
    if (nt + nseg <= U && n2 <= U && s.N + n2 <= U && nm <= gdn::MAX_MERGE_DOCS) break;
  }
  if (pmax < 2) return sp;
  auto bound = [&](int n, int i) { return (int)((long)chunks[n] * i / P[n]); };
  auto add = [](gdn::SegPlan& pl, gdn::SegUnit u) { pl.u[pl.n_units++] = u; };
  int plane = 0, work = 0;
  for (int n = 0; n < s.N; ++n) {
    const int Pn = P[n];
    if (Pn == 1) {
      add(sp.phase1, gdn::SegUnit{n, 0, chunks[n], 0, -1, -1, 0, 1});
      add(sp.replay, gdn::SegUnit{n, 0, chunks[n], 0, -1, -1, 0, 0});
      continue;
    }
    const int s_base = plane;
    plane += Pn - 1;
    int m_base = -1, b_base = -1;
    if (Pn >= 3) {
      m_base = work;
      work += Pn - 2;
      b_base = work;
      work += Pn - 2;
      sp.merge.d[sp.merge.n_docs++] = gdn::MergeDoc{s_base, m_base, b_base, Pn - 2};
    }
    const gdn::SegUnit seg0{n, 0, bound(n, 1), 0, -1, s_base, 1, 0};
    add(sp.phase1, seg0);
    add(sp.recompute, seg0);
    add(sp.replay, gdn::SegUnit{n, 0, bound(n, 1), 0, -1, -1, 0, 0});
    for (int i = 1; i + 1 < Pn; ++i) {
      const gdn::SegUnit m{n, bound(n, i), bound(n, i + 1), 1, -1, m_base + i - 1, 0, 0};
      const gdn::SegUnit b{n, bound(n, i), bound(n, i + 1), 2, -1, b_base + i - 1, 0, 0};
      add(sp.transfer, m);
      add(sp.transfer, b);
      add(sp.recompute, m);
      add(sp.recompute, b);
    }
    for (int i = 1; i < Pn; ++i) {
      add(sp.phase2, gdn::SegUnit{n, bound(n, i), bound(n, i + 1), 0, s_base + i - 1, -1, 0, i + 1 == Pn ? 1 : 0});
      add(sp.replay, gdn::SegUnit{n, bound(n, i), bound(n, i + 1), 0, s_base + i - 1, -1, 0, 0});
    }
  }
  // longest units first, so that the workgroups left waiting for a free CU are the shortest
  for (gdn::SegPlan* pl : {&sp.phase1, &sp.transfer, &sp.phase2, &sp.recompute, &sp.replay})
    std::stable_sort(pl->u, pl->u + pl->n_units,
                     [](const gdn::SegUnit& x, const gdn::SegUnit& y) { return x.hi - x.lo > y.hi - y.lo; });
  sp.plane_slots = plane;
  sp.work_slots = work;
  sp.on = true;
  return sp;
}

// The caller's auxiliary stream, or NULL if there is none (or it is `stream` itself).
hipStream_t aux_of(const gdn_problem* p, void* stream) {
  if (!p->aux_stream || p->aux_stream == stream) return nullptr;
  return (hipStream_t)p->aux_stream;
}

void range_a(gdn::Args& a, const Split& sp) {
  a.grp_off = 0;
  a.grp_end = a.H;
  a.pair_off = 2 * ((a.N * a.H - a.H + 7) / 8);
  a.c_base = sp.cA0;
  a.c_skip_at = 0x7fffffff;
  a.c_skip = 0;
  a.c_count = sp.cA;
}

void range_b(gdn::Args& a, const Split& sp) {
  a.grp_off = a.H;
  a.grp_end = a.N * a.H;
  a.pair_off = 0;
  a.c_base = 0;
  a.c_skip_at = sp.cA0;
  a.c_skip = sp.cA;
  a.c_count = a.NT - sp.cA;
}

void bind_workspace(gdn::Args& a, const WorkLayout& W, void* ws) {
  char* b = (char*)ws;
  a.seq_c0 = (int*)(b + W.seq_c0);
  a.c_t0 = (int*)(b + W.c_t0);
  a.c_len = (int*)(b + W.c_len);
  a.seq_order = (int*)(b + W.seq_order);
  a.pair_order = (int*)(b + W.pair_order);
  a.status = (int*)(b + W.status);
  a.rk = (float*)(b + W.rk);
  a.rq = (float*)(b + W.rq);
  a.qk = (uint16_t*)(b + W.qk);
  if (W.htape) a.htape = (uint16_t*)(b + W.htape);
  if (W.dstape) a.dstape = (uint16_t*)(b + W.dstape);
  if (W.dqacc) a.dqacc = (float*)(b + W.dqacc);
  if (W.dkacc) a.dkacc = (float*)(b + W.dkacc);
  if (W.carry) a.carry = (float*)(b + W.carry);
  if (W.queue) a.gq = (int*)(b + W.queue);
}

// Workspace area that holds the state between the pieces of a split walk (forward ops only).
float* piece_state(const WorkLayout& W, void* ws) { return W.state ? (float*)((char*)ws + W.state) : nullptr; }

void bind_saved(gdn::Args& a, const SavedLayout& L, void* saved) {
  char* b = (char*)saved;
  a.akk = (uint16_t*)(b + L.akk);
  a.gcum = (float*)(b + L.gcum);
  a.gamma = (float*)(b + L.gamma);
  if (L.htape) a.htape = (uint16_t*)(b + L.htape);
  if (L.vnew) {
    a.vnew = (uint16_t*)(b + L.vnew);
    a.w = (uint16_t*)(b + L.w);
    a.u = (uint16_t*)(b + L.u);
    a.aqk = (uint16_t*)(b + L.aqk);
  }
  if (L.plane) a.splane = (float*)(b + L.plane);
}

// Per-token tensors may be NULL when there are no tokens.
int check_tok(const void* ptr, const char* name, int64_t T) {
  if (T == 0 && !ptr) return GDN_OK;
  return check_ptr(ptr, name);
}

int check_inputs(const gdn_problem* p, const void* q, const void* k, const void* v, const float* g,
                 const float* beta, const int32_t* cu, const float* h0) {
  const int64_t T = p->n_tokens;
  CHECK(check_tok(q, "q", T));
  CHECK(check_tok(k, "k", T));
  CHECK(check_tok(v, "v", T));
  CHECK(check_tok(g, "g", T));
  CHECK(check_tok(beta, "beta", T));
  CHECK(check_ptr(cu, "cu_seqlens"));
  if (p->has_h0) CHECK(check_ptr(h0, "h0"));
  return GDN_OK;
}

// Forward and recompute share everything but o/ht.
int forward_common(const gdn_problem* p, const void* q, const void* k, const void* v, const float* g,
                   const float* beta, const int32_t* cu, const float* h0, void* o, float* ht, void* saved,
                   void* workspace, size_t workspace_bytes, void* stream, bool write_o) {
  Sizes s;
  CHECK(check_problem(p, &s));
  CHECK(check_inputs(p, q, k, v, g, beta, cu, h0));
  if (write_o) {
    CHECK(check_tok(o, "o", s.T));
    if (p->want_ht) CHECK(check_ptr(ht, "ht"));
  }
  CHECK(check_ptr(saved, "saved"));
  CHECK(check_ptr(workspace, "workspace"));
  const int full = p->save_mode == GDN_SAVE_FULL;
  const bool tape = keeps_tape(p->save_mode);
  const SegPlans seg = plan_segments(p, s);
  // the light recompute of an unsegmented problem runs no walk: its saved set needs only the chunk
  // tables and the intra pass
  const bool walk = write_o || tape || seg.on;
  const WorkLayout W = work_layout(s, write_o ? GDN_OP_FWD : GDN_OP_RECOMPUTE, p->save_mode, p->deterministic,
                                   seg.work_slots);
  if (workspace_bytes < W.total)
    return fail(GDN_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, W.total);
  const SavedLayout L = saved_layout(s, p->save_mode, seg.plane_slots);
  gdn::Args a;
  fill_common(a, s, p);
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.cu = cu;
  a.h0 = p->has_h0 ? h0 : nullptr;
  a.o = o;
  a.ht = (write_o && p->want_ht) ? ht : nullptr;
  if (!write_o) a.want_ht = 0;
  bind_workspace(a, W, workspace);
  bind_saved(a, L, saved);

  const Split sp = walk && !seg.on ? plan_split(p, s) : Split{};
  hipStream_t side = sp.on ? aux_of(p, stream) : nullptr;
  CallEvents ev;
  if (side) a.grp_split = a.H;
  LAUNCH("gdn_tables", gdn::launch_tables(a, nullptr, nullptr, stream));
  const char* walk_name = write_o ? "gdn_walk_fwd" : "gdn_walk_tape";
  if (seg.on && !write_o && !tape) {
    // light recompute of a segmented problem: only the carry plane (segment 0 of each segmented
    // document walked to its end, the transfer walks, the merge)
    LAUNCH("gdn_intra", gdn::launch_intra(a, 0, stream));
    LAUNCH("gdn_walk_transfer", gdn::launch_walk_seg(a, seg.recompute, 0, 0, 0, 1, stream));
    LAUNCH("gdn_seg_merge", gdn::launch_seg_merge(a, seg.merge, stream));
  } else if (seg.on) {
    // segmented: the transfer walks beside phase 1 (on the auxiliary stream when there is one),
    // the carry merge, then phase 2
    LAUNCH("gdn_intra", gdn::launch_intra(a, 0, stream));
    hipStream_t xs = aux_of(p, stream);
    if (seg.transfer.n_units) {
      if (xs) {
        CHECK(ev.order((hipStream_t)stream, xs));
        LAUNCH_ON(xs, "gdn_walk_transfer", gdn::launch_walk_seg(a, seg.transfer, 0, 0, 0, 1, xs));
      } else {
        LAUNCH("gdn_walk_transfer", gdn::launch_walk_seg(a, seg.transfer, 0, 0, 0, 1, stream));
      }
    }
    LAUNCH(walk_name, gdn::launch_walk_seg(a, seg.phase1, write_o, tape, full, 0, stream));
    if (xs && seg.transfer.n_units) CHECK(ev.order(xs, (hipStream_t)stream));
    LAUNCH("gdn_seg_merge", gdn::launch_seg_merge(a, seg.merge, stream));
    LAUNCH(walk_name, gdn::launch_walk_seg(a, seg.phase2, write_o, tape, full, 0, stream));
  } else if (!side) {
    LAUNCH("gdn_intra", gdn::launch_intra(a, 0, stream));
    if (walk) LAUNCH(walk_name, gdn::launch_walk_fwd(a, write_o, tape, full, stream));
  } else {
    gdn::Args aa = a, ab = a;
    range_a(aa, sp);
    range_b(ab, sp);
    // The longest document in up to 4 pieces when it has at least 768 chunks: each piece's walk
    // needs only that piece's intra launch, and starts from the state the previous piece left in
    // the workspace (f32, so the result is the same as one walk over the document). The first
    // piece is short (96 chunks), so that the walk starts after a small intra launch; the next
    // piece's intra launch (a tenth of a walk step per chunk) is done before its walk is due.
    const int pieces = std::max(1, std::min(4, sp.cA / 384));
    const int first = pieces > 1 ? std::min(96, sp.cA / pieces) : sp.cA;
    float* st = piece_state(W, workspace);
    gdn::Args ap[4];
    for (int i = 0; i < pieces; ++i) {
      ap[i] = aa;
      auto bound = [&](int k) {
        return k == 0 ? 0 : first + (int)((long)(sp.cA - first) * (k - 1) / (pieces - 1));
      };
      const int lo = bound(i), hi = i + 1 < pieces ? bound(i + 1) : sp.cA;
      ap[i].c_base = sp.cA0 + lo;
      ap[i].c_count = hi - lo;
      ap[i].piece_lo = lo;
      ap[i].piece_hi = hi;
      ap[i].state_in = i > 0 ? st : nullptr;
      ap[i].state_out = i + 1 < pieces ? st : nullptr;
      if (i + 1 < pieces) ap[i].want_ht = 0;
    }
    LAUNCH("gdn_intra", gdn::launch_intra(ap[0], 0, stream));
    CHECK(ev.order((hipStream_t)stream, side));
    hipEvent_t ready[4] = {nullptr, nullptr, nullptr, nullptr};
    for (int i = 1; i < pieces; ++i) {
      LAUNCH_ON(side, "gdn_intra", gdn::launch_intra(ap[i], 0, side));
      CHECK(ev.take(&ready[i]));
      if (hipEventRecord(ready[i], side) != hipSuccess) return fail(GDN_EHIP, "piece event record failed");
    }
    LAUNCH_ON(side, "gdn_intra", gdn::launch_intra(ab, 0, side));
    LAUNCH_ON(side, walk_name, gdn::launch_walk_fwd(ab, write_o, tape, full, side));
    for (int i = 0; i < pieces; ++i) {
      if (i > 0 && hipStreamWaitEvent((hipStream_t)stream, ready[i], 0) != hipSuccess)
        return fail(GDN_EHIP, "piece event wait failed");
      LAUNCH(walk_name, gdn::launch_walk_fwd(ap[i], write_o, tape, full, stream));
    }
    CHECK(ev.order(side, (hipStream_t)stream));
  }
  if (full) LAUNCH("gdn_wy_full", gdn::launch_wy_full(a, stream));
  uint64_t words[4];
  tag_words(p, words);
  LAUNCH("gdn_write_tag", gdn::launch_write_tag(saved, words, a.status, stream));
  if (write_o) LAUNCH("gdn_poison", gdn::launch_poison(a, GDN_OP_FWD, stream));
  g_err.clear();
  return GDN_OK;
}

} // namespace

extern "C" {

size_t gdn_saved_bytes(const gdn_problem* p) {
  Sizes s;
  if (check_problem(p, &s) != GDN_OK) return 0;
  return saved_layout(s, p->save_mode, plan_segments(p, s).plane_slots).total;
}

size_t gdn_workspace_bytes(const gdn_problem* p, int op) {
  Sizes s;
  if (check_problem(p, &s) != GDN_OK) return 0;
  if (op != GDN_OP_FWD && op != GDN_OP_RECOMPUTE && op != GDN_OP_BWD) {
    fail(GDN_EINVAL, "unknown op %d", op);
    return 0;
  }
  return work_layout(s, op, p->save_mode, p->deterministic, plan_segments(p, s).work_slots).total;
}

int gdn_fwd(const gdn_problem* p, const void* q, const void* k, const void* v, const float* g, const float* beta,
            const int32_t* cu_seqlens, const float* h0, void* o, float* ht, void* saved, void* workspace,
            size_t workspace_bytes, void* stream) {
  return forward_common(p, q, k, v, g, beta, cu_seqlens, h0, o, ht, saved, workspace, workspace_bytes, stream,
                        true);
}

int gdn_fwd_recompute(const gdn_problem* p, const void* q, const void* k, const void* v, const float* g,
                      const float* beta, const int32_t* cu_seqlens, const float* h0, void* saved, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return forward_common(p, q, k, v, g, beta, cu_seqlens, h0, nullptr, nullptr, saved, workspace, workspace_bytes,
                        stream, false);
}

int gdn_bwd(const gdn_problem* p, const void* q, const void* k, const void* v, const float* g, const float* beta,
            const int32_t* cu_seqlens, const float* h0, const void* saved, const void* dO, const float* dht,
            void* dq, void* dk, void* dv, float* dg, float* dbeta, float* dh0, void* workspace,
            size_t workspace_bytes, void* stream) {
  Sizes s;
  CHECK(check_problem(p, &s));
  CHECK(check_inputs(p, q, k, v, g, beta, cu_seqlens, h0));
  CHECK(check_ptr(saved, "saved"));
  CHECK(check_tok(dO, "dO", s.T));
  if (dht) CHECK(check_ptr(dht, "dht"));
  CHECK(check_tok(dq, "dq", s.T));
  CHECK(check_tok(dk, "dk", s.T));
  CHECK(check_tok(dv, "dv", s.T));
  CHECK(check_tok(dg, "dg", s.T));
  CHECK(check_tok(dbeta, "dbeta", s.T));
  if (p->has_h0) CHECK(check_ptr(dh0, "dh0"));
  CHECK(check_ptr(workspace, "workspace"));
  const bool tape = keeps_tape(p->save_mode);
  const WorkLayout W = work_layout(s, GDN_OP_BWD, p->save_mode, p->deterministic);
  if (workspace_bytes < W.total)
    return fail(GDN_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, W.total);
  const SegPlans seg = plan_segments(p, s);
  const SavedLayout L = saved_layout(s, p->save_mode, seg.plane_slots);
  gdn::Args a;
  fill_common(a, s, p);
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.cu = cu_seqlens;
  a.h0 = p->has_h0 ? h0 : nullptr;
  a.dO = dO;
  a.dht = dht;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dg = dg;
  a.dbeta = dbeta;
  a.dh0 = p->has_h0 ? dh0 : nullptr;
  bind_workspace(a, W, workspace);
  bind_saved(a, L, const_cast<void*>(saved));

  const Split sp = seg.on ? Split{} : plan_split(p, s);
  hipStream_t side = sp.on ? aux_of(p, stream) : nullptr;
  CallEvents ev;
  if (side) a.grp_split = a.H;
  // the first kernel compares the saved set's tag with this problem's; on a mismatch it sets the
  // status word, every later kernel skips its work and the last one fills the gradients with NaN
  uint64_t words[4];
  tag_words(p, words);
  LAUNCH("gdn_tables", gdn::launch_tables(a, (const uint64_t*)saved, words, stream));
  // the chunk-gradient launches' work-queue counters, cleared here, ahead of every launch that
  // may run beside them: a one-wave launch queued between a running chunk-gradient launch and
  // the next would wait for a workgroup of the running one to exit (they hold every register)
  LAUNCH("gdn_fill_zero", gdn::launch_fill_zero(reinterpret_cast<float*>(a.gq), 2, stream));
  if (!p->deterministic) { // accumulators of the atomic dq, dk reduction
    LAUNCH("gdn_fill_zero", gdn::launch_fill_zero(a.dqacc, (size_t)s.T * s.H * s.D, stream));
    LAUNCH("gdn_fill_zero", gdn::launch_fill_zero(a.dkacc, (size_t)s.T * s.H * s.D, stream));
  }
  // light: the state tape is replayed; the tape walk and the reverse walk are independent and
  // share one launch. full / kept tape: the tape is in the saved set.
  auto walks = [&](const gdn::Args& x, hipStream_t st) -> int {
    if (!tape) LAUNCH_ON(st, "gdn_walk_pair", gdn::launch_walk_pair(x, st));
    else LAUNCH_ON(st, "gdn_walk_bwd", gdn::launch_walk_bwd(x, st));
    return GDN_OK;
  };
  if (seg.on && !tape) {
    // segmented, light: the state tape replayed one segment per chain from the saved carry plane
    // (on the auxiliary stream when there is one), beside the reverse walk
    LAUNCH("gdn_intra_bwd", gdn::launch_intra(a, 1, stream));
    hipStream_t xs = aux_of(p, stream);
    if (xs) {
      CHECK(ev.order((hipStream_t)stream, xs));
      LAUNCH_ON(xs, "gdn_walk_tape", gdn::launch_walk_seg(a, seg.replay, 0, 1, 0, 0, xs));
    } else {
      LAUNCH("gdn_walk_tape", gdn::launch_walk_seg(a, seg.replay, 0, 1, 0, 0, stream));
    }
    LAUNCH("gdn_walk_bwd", gdn::launch_walk_bwd(a, stream));
    if (xs) CHECK(ev.order(xs, (hipStream_t)stream));
  } else if (!side) {
    LAUNCH("gdn_intra_bwd", gdn::launch_intra(a, 1, stream));
    CHECK(walks(a, (hipStream_t)stream));
  } else {
    // the chunk gradients of the other documents run on the auxiliary stream as soon as their
    // walks end, beside the longest document's walk; the longest document's follow its walk
    gdn::Args aa = a, ab = a;
    range_a(aa, sp);
    range_b(ab, sp);
    ab.gq = a.gq + 1;
    LAUNCH("gdn_intra_bwd", gdn::launch_intra(aa, 1, stream));
    CHECK(ev.order((hipStream_t)stream, side));
    CHECK(walks(aa, (hipStream_t)stream));
    LAUNCH_ON(side, "gdn_intra_bwd", gdn::launch_intra(ab, 1, side));
    CHECK(walks(ab, side));
    LAUNCH_ON(side, "gdn_chunk_grad", gdn::launch_chunk_grad(ab, p->deterministic, side));
    LAUNCH("gdn_chunk_grad", gdn::launch_chunk_grad(aa, p->deterministic, stream));
    CHECK(ev.order(side, (hipStream_t)stream));
  }
  if (!side) LAUNCH("gdn_chunk_grad", gdn::launch_chunk_grad(a, p->deterministic, stream));
  if (!p->deterministic) LAUNCH("gdn_finalize_qk", gdn::launch_finalize_qk(a, stream));
  LAUNCH("gdn_poison", gdn::launch_poison(a, GDN_OP_BWD, stream));
  g_err.clear();
  return GDN_OK;
}

int gdn_status(const gdn_problem* p, int op, const void* workspace, void* stream) {
  Sizes s;
  CHECK(check_problem(p, &s));
  if (op != GDN_OP_FWD && op != GDN_OP_RECOMPUTE && op != GDN_OP_BWD) return fail(GDN_EINVAL, "unknown op %d", op);
  CHECK(check_ptr(workspace, "workspace"));
  const WorkLayout W = work_layout(s, op, p->save_mode, p->deterministic, plan_segments(p, s).work_slots);
  int32_t st = 0;
  hipError_t r = hipMemcpyAsync(&st, (const char*)workspace + W.status, sizeof st, hipMemcpyDeviceToHost,
                                (hipStream_t)stream);
  if (r == hipSuccess) r = hipStreamSynchronize((hipStream_t)stream);
  if (r != hipSuccess) return fail(GDN_EHIP, "status copy: %s", hipGetErrorString(r));
  if (st == 0) {
    g_err.clear();
    return GDN_OK;
  }
  if (st == 2) return fail(GDN_ESAVED, "the saved buffer's tag does not name this problem, save mode and ABI version");
  return fail(GDN_EINVAL, "the device cu_seqlens disagree with the host copy in the problem");
}

void gdn_timing_enable(int on) { g_timing_on.store(on ? 1 : 0); }

int gdn_timing_launches(int max, const char** names, double* start_ms, double* end_ms) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  const int n = (int)g_pending.size();
  if (n == 0) return 0;
  std::vector<double> st(n, 0.0), en(n, 0.0);
  double lo = 0.0;
  for (int i = 0; i < n; ++i) {
    float a = 0.f, b = 0.f;
    hipEventSynchronize(g_pending[i].stop);
    hipEventElapsedTime(&a, g_pending[0].start, g_pending[i].start);
    hipEventElapsedTime(&b, g_pending[0].start, g_pending[i].stop);
    st[i] = a;
    en[i] = b;
    lo = std::min(lo, st[i]);
  }
  for (int i = 0; i < n && i < max; ++i) {
    if (names) names[i] = g_pending[i].name;
    if (start_ms) start_ms[i] = st[i] - lo;
    if (end_ms) end_ms[i] = en[i] - lo;
  }
  return n;
}

int gdn_timing_collect(int max, const char** names, double* total_ms, int* launches) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  for (const PendingEvent& p : g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.stop) == hipSuccess && hipEventElapsedTime(&ms, p.start, p.stop) == hipSuccess) {
      auto& t = g_totals[p.name];
      t.first += ms;
      t.second += 1;
    }
    hipEventDestroy(p.start);
    hipEventDestroy(p.stop);
  }
  g_pending.clear();
  int i = 0;
  for (const auto& kv : g_totals) {
    if (i >= max) break;
    static thread_local std::vector<std::string> keep;
    if ((int)keep.size() < max) keep.resize(max);
    keep[i] = kv.first;
    if (names) names[i] = keep[i].c_str();
    if (total_ms) total_ms[i] = kv.second.first;
    if (launches) launches[i] = kv.second.second;
    ++i;
  }
  return (int)g_totals.size();
}

void gdn_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  for (const PendingEvent& p : g_pending) {
    hipEventDestroy(p.start);
    hipEventDestroy(p.stop);
  }
  g_pending.clear();
  g_totals.clear();
}

const char* gdn_last_error(void) { return g_err.c_str(); }

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

} // extern "C"

namespace gdn {

// Forward with a caller-chosen workspace and no auxiliary stream (the entry point that allocates
// nothing runs every launch on the caller's stream, so it records no events).
int gdn_fwd_single_stream(const gdn_problem* p, const void* q, const void* k, const void* v, const float* g,
                          const float* beta, const int32_t* cu_seqlens, const float* h0, void* o, float* ht,
                          void* saved, void* workspace, size_t workspace_bytes, void* stream) {
  if (!p) return fail(GDN_EINVAL, "problem descriptor is NULL");
  gdn_problem pc = *p;
  pc.aux_stream = nullptr;
  return forward_common(&pc, q, k, v, g, beta, cu_seqlens, h0, o, ht, saved, workspace, workspace_bytes, stream,
                        true);
}

int gdn_set_error(int code, const char* msg) { return fail(code, "%s", msg); }

} // namespace gdn

// ---------------------------------------------------------------------------------------------
// Short causal conv1d + SiLU front-end

namespace {

int check_conv(const gdn_conv_problem* p) {
  if (!p) return fail(GDN_EINVAL, "conv problem descriptor is NULL");
  if (p->n_seqs < 1) return fail(GDN_EINVAL, "n_seqs must be >= 1 (got %d)", p->n_seqs);
  if (p->width < 1 || p->width > 4) return fail(GDN_EUNSUPPORTED, "conv width must be 1..4 (got %d)", p->width);
  if (p->dtype != GDN_DTYPE_BF16 && p->dtype != GDN_DTYPE_F32)
    return fail(GDN_EUNSUPPORTED, "unsupported dtype %d", p->dtype);
  if (p->n_groups < 1 || p->n_groups > 4) return fail(GDN_EINVAL, "n_groups must be 1..4 (got %d)", p->n_groups);
  int64_t c = 0;
  for (int g = 0; g < p->n_groups; ++g) {
    if (p->group_channels[g] < 8 || p->group_channels[g] % 8 != 0)
      return fail(GDN_EINVAL, "group %d has %d channels: each group needs a positive multiple of 8", g,
                  p->group_channels[g]);
    c += p->group_channels[g];
  }
  if (c != p->channels) return fail(GDN_EINVAL, "channels (%d) must equal the sum of group_channels (%lld)",
                                    p->channels, (long long)c);
  if (!p->cu_seqlens_host) return fail(GDN_EINVAL, "cu_seqlens_host is NULL");
  const int32_t* cu = p->cu_seqlens_host;
  if (cu[0] != 0) return fail(GDN_EINVAL, "cu_seqlens[0] must be 0");
  for (int n = 0; n < p->n_seqs; ++n)
    if (cu[n + 1] < cu[n]) return fail(GDN_EINVAL, "cu_seqlens decreases at %d", n);
  if ((int64_t)cu[p->n_seqs] != p->n_tokens)
    return fail(GDN_EINVAL, "cu_seqlens[N] = %d but n_tokens = %lld", cu[p->n_seqs], (long long)p->n_tokens);
  if ((int64_t)gdn::conv_blocks(p->n_tokens) > 65535) return fail(GDN_EINVAL, "too many tokens for one call");
  return GDN_OK;
}

void conv_args(gdn::ConvArgs& a, const gdn_conv_problem* p, const void* x, const float* w, const float* b,
               const int32_t* cu) {
  std::memset(&a, 0, sizeof a);
  a.T = p->n_tokens;
  a.C = p->channels;
  a.W = p->width;
  a.N = p->n_seqs;
  a.silu = p->silu ? 1 : 0;
  a.n_groups = p->n_groups;
  int off = 0;
  for (int g = 0; g < p->n_groups; ++g) {
    a.goff[g] = off;
    off += p->group_channels[g];
  }
  for (int g = p->n_groups; g <= 4; ++g) a.goff[g] = off;
  a.x = x;
  a.w = w;
  a.b = b;
  a.cu = cu;
}

} // namespace

extern "C" {

size_t gdn_conv_workspace_bytes(const gdn_conv_problem* p) {
  if (check_conv(p) != GDN_OK) return 0;
  const size_t n = (size_t)gdn::conv_blocks(p->n_tokens) * p->channels * (p->width + 1) * 4;
  return align_up(n > 0 ? n : 1);
}

int gdn_conv_fwd(const gdn_conv_problem* p, const void* x, const float* weight, const float* bias,
                 const int32_t* cu_seqlens, void* const* y, void* stream) {
  CHECK(check_conv(p));
  const int64_t T = p->n_tokens;
  CHECK(check_tok(x, "x", T));
  CHECK(check_ptr(weight, "weight"));
  if (bias && !aligned16(bias)) return fail(GDN_EINVAL, "bias is not 16-byte aligned");
  CHECK(check_ptr(cu_seqlens, "cu_seqlens"));
  if (!y) return fail(GDN_EINVAL, "y (the array of output pointers) is NULL");
  gdn::ConvArgs a;
  conv_args(a, p, x, weight, bias, cu_seqlens);
  for (int g = 0; g < p->n_groups; ++g) {
    CHECK(check_tok(y[g], "y[g]", T));
    a.y[g] = y[g];
  }
  LAUNCH("gdn_conv_fwd", gdn::launch_conv_fwd(a, p->dtype, stream));
  g_err.clear();
  return GDN_OK;
}

int gdn_conv_bwd(const gdn_conv_problem* p, const void* x, const float* weight, const float* bias,
                 const int32_t* cu_seqlens, const void* const* dy, void* dx, float* dweight, float* dbias,
                 void* workspace, size_t workspace_bytes, void* stream) {
  CHECK(check_conv(p));
  const int64_t T = p->n_tokens;
  CHECK(check_tok(x, "x", T));
  CHECK(check_ptr(weight, "weight"));
  if (bias && !aligned16(bias)) return fail(GDN_EINVAL, "bias is not 16-byte aligned");
  CHECK(check_ptr(cu_seqlens, "cu_seqlens"));
  CHECK(check_tok(dx, "dx", T));
  CHECK(check_ptr(dweight, "dweight"));
  if (dbias && !aligned16(dbias)) return fail(GDN_EINVAL, "dbias is not 16-byte aligned");
  CHECK(check_ptr(workspace, "workspace"));
  if (workspace_bytes < gdn_conv_workspace_bytes(p))
    return fail(GDN_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, gdn_conv_workspace_bytes(p));
  if (!dy) return fail(GDN_EINVAL, "dy (the array of gradient pointers) is NULL");
  gdn::ConvArgs a;
  conv_args(a, p, x, weight, bias, cu_seqlens);
  for (int g = 0; g < p->n_groups; ++g) {
    CHECK(check_tok(dy[g], "dy[g]", T));
    a.dy[g] = dy[g];
  }
  a.dx = dx;
  a.dw = dweight;
  a.db = dbias;
  a.part = (float*)workspace;
  LAUNCH("gdn_conv_bwd", gdn::launch_conv_bwd(a, p->dtype, stream));
  g_err.clear();
  return GDN_OK;
}

} // extern "C"
