// C-ABI layer of libkvevict: argument validation, launch planning and the
// fused decode step. Validation happens on the host before any launch; the
// library never allocates and never synchronises the device.
#include "kvevict.h"

#include <mutex>

#include "kve_internal.h"

namespace {

// Split-K planning constants (rows are cache rows of one slice).
constexpr int kSplitRowQuantum = 16;   // rows per split: a multiple of this
constexpr int kMinRowsPerSplit = 64;   // no split shorter than this
constexpr int kSplitTargetWGs = 4096;  // bound on slices * splits
constexpr int kWgOverheadRows = 32;    // fixed cost of a workgroup, in rows
constexpr int kCombineRows = 64;       // cost of the combine launch, in rows
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int elem_bytes(int dtype) { return dtype == KVE_F32 ? 4 : 2; }

kve_status check_shape(const kve_shape* s) {
  if (!s) return KVE_ERR_INVALID_ARG;
  if (s->batch < 1 || s->n_kv_heads < 1 || s->capacity < 1 || s->group < 1)
    return KVE_ERR_INVALID_ARG;
  if (s->batch > 65535 || s->n_kv_heads > 65535) return KVE_ERR_UNSUPPORTED;
  if (s->group > 8) return KVE_ERR_UNSUPPORTED;
  if (s->head_dim != 64 && s->head_dim != 128) return KVE_ERR_UNSUPPORTED;
  if (s->kv_dtype != KVE_F32 && s->kv_dtype != KVE_BF16)
    return KVE_ERR_UNSUPPORTED;
  // Kernels address the rows of one slice with 32-bit byte offsets and count
  // slices in an int.
  const long long row_bytes = (long long)s->head_dim * elem_bytes(s->kv_dtype);
  if ((long long)s->capacity * row_bytes >= (1LL << 32))
    return KVE_ERR_UNSUPPORTED;
  if ((long long)s->batch * s->n_kv_heads > 0x7fffffffLL)
    return KVE_ERR_UNSUPPORTED;
  return KVE_OK;
}

kve_status check_policy(const kve_policy* p) {
  if (!p) return KVE_ERR_INVALID_ARG;
  if (p->sinks < 0 || p->window < 0 || p->evict_len < 1 || p->budget < 1)
    return KVE_ERR_POLICY;
  if ((long long)p->sinks + p->window > p->budget) return KVE_ERR_POLICY;
  return KVE_OK;
}

// Kernels move rows with 16-byte vector accesses (some straight into LDS),
// so buffers of K, V, q, output rows, hidden states and workspaces must be
// 16-byte aligned, float32 and int32 arrays 4-byte aligned. Null passes
// (nullability is checked where it matters).
bool a16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool a4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

kve_status check_cache(const kve_cache* c) {
  if (!c || !c->k || !c->v || !c->score || !c->pos) return KVE_ERR_INVALID_ARG;
  if (!a16(c->k) || !a16(c->v) || !a4(c->score) || !a4(c->pos) ||
      !a16(c->scorer_state))
    return KVE_ERR_INVALID_ARG;
  return KVE_OK;
}

long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

// Largest split count the planner may choose for a slice of len rows; it
// depends on the shape only (not on the device) and never decreases with
// len, so a workspace sized for max_len serves every len <= max_len.
int split_cap(const kve_shape* s, int len) {
  const long long slices = (long long)s->batch * s->n_kv_heads;
  long long ns = ceil_div(kSplitTargetWGs, slices);
  const long long by_rows = ceil_div(len, kMinRowsPerSplit);
  if (ns > by_rows) ns = by_rows;
  if (ns > kve::kMaxSplit) ns = kve::kMaxSplit;
  if (ns < 1) ns = 1;
  return (int)ns;
}

// Compute units of the current device (cached per device).
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
          hipSuccess || n < 1)
    n = 256;
  if (dev < 64) cached[dev] = n;
  return n;
}

struct SplitPlan {
  int nsplit, rows_per_split;
};

// Split-K plan of one decode-attention launch. One workgroup with its
// non-temporal loads in flight streams at about a CU's share of HBM
// bandwidth, so the model is per CU: the rows its workgroups stream, plus a
// fixed cost per workgroup it runs, plus the combine launch when split. The
// plan minimises that; ties go to fewer splits. (Measured: when slices are
// fewer than CUs the best plan is one workgroup per CU.)
SplitPlan plan_split(const kve_shape* s, int len) {
  const long long slices = (long long)s->batch * s->n_kv_heads;
  const long long cus = device_cus();
  const int cap = split_cap(s, len);
  SplitPlan best{1, len};
  long long best_cost = -1;
  for (int ns = 1; ns <= cap; ++ns) {
    int rps = (int)ceil_div(len, ns);
    rps = (int)ceil_div(rps, kSplitRowQuantum) * kSplitRowQuantum;
    const int eff = (int)ceil_div(len, rps);
    if (eff != ns) continue;  // same as a smaller split count
    const long long per_cu = ceil_div(slices * eff, cus);
    const long long cost = per_cu * (rps + kWgOverheadRows) +
                           (eff > 1 ? kCombineRows : 0);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = SplitPlan{eff, eff == 1 ? len : rps};
    }
  }
  return best;
}

// Workspace: split-K partial results (acc[D], m, l) per query head and split.
size_t ws_bytes_for(const kve_shape* s, int nsplit) {
  const size_t hq = (size_t)s->batch * s->n_kv_heads * s->group;
  return nsplit > 1 ? align_up(hq * nsplit * (s->head_dim + 2) * sizeof(float))
                    : 0;
}

kve_status from_hip(hipError_t e) { return e == hipSuccess ? KVE_OK : KVE_ERR_LAUNCH; }

// Status of a launcher's host-side configuration check (check_only).
kve_status from_check(hipError_t e) {
  return e == hipSuccess ? KVE_OK : KVE_ERR_UNSUPPORTED;
}

kve_status attn_impl(const kve_shape* shape, const kve_cache* cache, int len,
                     const void* q, float* out, float* lse, void* ws,
                     size_t ws_bytes, int new_slot, int new_pos,
                     const void* k_new, const void* v_new, hipStream_t stream,
                     const void* hidden_new = nullptr, void* hidden_buf = nullptr,
                     int hidden_bytes = 0, int hidden_rows = 0,
                     int hidden_row = 0, bool check_only = false) {
  // The attention kernel reads the appended row from k_new / v_new only in
  // the last stage of the last split, so it must be the slice's last row.
  if (new_slot >= 0 && new_slot != len - 1) return KVE_ERR_INVALID_ARG;
  const SplitPlan plan = plan_split(shape, len);
  if (ws_bytes < ws_bytes_for(shape, plan.nsplit) ||
      (plan.nsplit > 1 && !ws))
    return KVE_ERR_WORKSPACE;
  kve::AttnLaunch a{};
  a.k = cache->k;
  a.v = cache->v;
  a.q = q;
  a.out = out;
  a.lse = lse;
  a.partial = (float*)ws;
  a.batch = shape->batch;
  a.H = shape->n_kv_heads;
  a.G = shape->group;
  a.D = shape->head_dim;
  a.cap = shape->capacity;
  a.len = len;
  a.nsplit = plan.nsplit;
  a.rows_per_split = plan.rows_per_split;
  a.is_bf16 = shape->kv_dtype == KVE_BF16;
  a.new_slot = new_slot;
  a.new_pos = new_pos;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_store = cache->k;
  a.v_store = cache->v;
  a.pos = cache->pos;
  if (new_slot >= 0 && hidden_new) {
    a.hidden_new = hidden_new;
    a.hidden_buf = hidden_buf;
    a.hidden_bytes = hidden_bytes;
    a.hidden_rows = hidden_rows;
    a.hidden_row = hidden_row;
  }
  if (check_only) return from_check(kve::launch_attention(a, stream, true));
  return from_hip(kve::launch_attention(a, stream));
}

kve_status check_scorer(const kve_shape* shape, const kve_scorer* sc) {
  if (!sc || !sc->w1) return KVE_ERR_INVALID_ARG;
  if (!a16(sc->w1) || !a4(sc->b1) || !a4(sc->w2) || !a4(sc->b2))
    return KVE_ERR_INVALID_ARG;
  if (sc->kind == KVE_SCORER_MLP_KV) {
    if (sc->in_dim != 2 * shape->head_dim) return KVE_ERR_UNSUPPORTED;
    if (sc->hidden < 1 || sc->hidden > 256) return KVE_ERR_UNSUPPORTED;
    if (sc->wdtype != shape->kv_dtype) return KVE_ERR_UNSUPPORTED;
    if (sc->act != KVE_ACT_RELU && sc->act != KVE_ACT_SILU)
      return KVE_ERR_UNSUPPORTED;
    if (!sc->w2) return KVE_ERR_INVALID_ARG;
    return KVE_OK;
  }
  if (sc->kind == KVE_SCORER_GATE_HIDDEN) {
    if (sc->wdtype != KVE_BF16) return KVE_ERR_UNSUPPORTED;
    if (sc->in_dim < 32 || sc->in_dim % 32 != 0) return KVE_ERR_UNSUPPORTED;
    if (shape->n_kv_heads > 16) return KVE_ERR_UNSUPPORTED;
    return KVE_OK;
  }
  if (sc->kind == KVE_SCORER_SINK_GATE) {
    if (sc->wdtype != KVE_BF16) return KVE_ERR_UNSUPPORTED;
    if (sc->in_dim < 32 || sc->in_dim % 32 != 0) return KVE_ERR_UNSUPPORTED;
    if (sc->hidden != 16) return KVE_ERR_UNSUPPORTED;
    if (shape->group < 1 || shape->group > 8) return KVE_ERR_UNSUPPORTED;
    if (sc->n_sink < 0 || sc->n_sink > 16) return KVE_ERR_UNSUPPORTED;
    if (sc->n_sink > 0 && !sc->w2) return KVE_ERR_INVALID_ARG;
    return KVE_OK;
  }
  if (sc->kind == KVE_SCORER_MLSTM) {
    if (shape->kv_dtype != KVE_BF16 || sc->wdtype != KVE_BF16)
      return KVE_ERR_UNSUPPORTED;
    if (sc->in_dim != 2 * shape->head_dim) return KVE_ERR_UNSUPPORTED;
    if (sc->hidden != shape->head_dim / 2) return KVE_ERR_UNSUPPORTED;
    if (kve::mlstm_state_floats(shape->head_dim) == 0) return KVE_ERR_UNSUPPORTED;
    if (!sc->w2) return KVE_ERR_INVALID_ARG;
    if (sc->delay < 0) return KVE_ERR_INVALID_ARG;
    return KVE_OK;
  }
  return KVE_ERR_UNSUPPORTED;
}

kve_status score_impl(const kve_shape* shape, const kve_scorer* sc,
                      kve_cache* cache, int slot_begin, int slot_end,
                      const void* hidden, long long hidden_batch_stride,
                      hipStream_t stream, bool check_only = false) {
  if (slot_end == slot_begin) return KVE_OK;
  auto done = [check_only](hipError_t e) {
    return check_only ? from_check(e) : from_hip(e);
  };
  if (sc->kind == KVE_SCORER_MLSTM) {
    if (!cache->scorer_state) return KVE_ERR_INVALID_ARG;
    kve::MlstmLaunch m{};
    m.k = cache->k;
    m.v = cache->v;
    m.pos = cache->pos;
    m.score = cache->score;
    m.state = cache->scorer_state;
    m.w = sc->w1;
    m.b = sc->b1;
    m.a = sc->w2;
    m.b2 = sc->b2;
    m.batch = shape->batch;
    m.H = shape->n_kv_heads;
    m.D = shape->head_dim;
    m.cap = shape->capacity;
    m.slot_begin = slot_begin;
    m.slot_end = slot_end;
    m.delay = sc->delay;
    return done(kve::launch_score_mlstm(m, stream, check_only));
  }
  if (sc->kind == KVE_SCORER_MLP_KV) {
    kve::MlpLaunch m{};
    m.k = cache->k;
    m.v = cache->v;
    m.score = cache->score;
    m.w1 = sc->w1;
    m.b1 = sc->b1;
    m.w2 = sc->w2;
    m.b2 = sc->b2;
    m.batch = shape->batch;
    m.H = shape->n_kv_heads;
    m.D = shape->head_dim;
    m.cap = shape->capacity;
    m.hidden = sc->hidden;
    m.act = sc->act;
    m.is_bf16 = shape->kv_dtype == KVE_BF16;
    m.slot_begin = slot_begin;
    m.slot_end = slot_end;
    m.cus = device_cus();
    return done(kve::launch_score_mlp(m, stream, check_only));
  }
  if (sc->kind == KVE_SCORER_SINK_GATE) {
    kve::SinkGateLaunch q{};
    q.hidden = hidden;
    q.batch_stride = hidden_batch_stride;
    q.score = cache->score;
    q.w = sc->w1;
    q.norm = sc->b1;
    q.sinks = sc->w2;
    q.b = sc->b2;
    q.batch = shape->batch;
    q.H = shape->n_kv_heads;
    q.G = shape->group;
    q.cap = shape->capacity;
    q.in_dim = sc->in_dim;
    q.n_sink = sc->n_sink;
    q.slot_begin = slot_begin;
    q.slot_end = slot_end;
    return done(kve::launch_score_sink_gate(q, stream, check_only));
  }
  kve::GateLaunch g{};
  g.hidden = hidden;
  g.batch_stride = hidden_batch_stride;
  g.score = cache->score;
  g.w = sc->w1;
  g.b = sc->b1;
  g.batch = shape->batch;
  g.H = shape->n_kv_heads;
  g.cap = shape->capacity;
  g.in_dim = sc->in_dim;
  g.slot_begin = slot_begin;
  g.slot_end = slot_end;
  return done(kve::launch_score_gate(g, stream, check_only));
}

// Scratch of kve_step_noalloc: the split-K partial results of its
// attention launches live in this file-scope device array (one copy per
// GPU, held until the process ends) instead of a caller workspace.
constexpr size_t kNoallocScratchBytes = KVE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[KVE_NOALLOC_SCRATCH_BYTES];

// Device address of the current device's copy of `scratch`. The array's name
// is a host-side stand-in in host code: the address comes from
// hipGetSymbolAddress, looked up once per device (with that device current)
// and kept. Returns null and sets *st if the lookup fails.
void* noalloc_scratch(kve_status* st) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *st = KVE_ERR_LAUNCH;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      *st = KVE_ERR_LAUNCH;
      return nullptr;
    }
    ptrs[dev] = p;
  }
  return ptrs[dev];
}

// One decode step of one layer (kve_step). With use_scratch the split-K
// partials go to the library's scratch array and ws / ws_bytes are ignored.
kve_status step_impl(const kve_shape* shape, const kve_policy* policy,
                     const kve_scorer* scorer, kve_cache* cache,
                     kve_decode_state* state, const void* k_new,
                     const void* v_new, const void* hidden_new,
                     void* hidden_buf, const void* q, float* out, float* lse,
                     int32_t* keep_slots, void* ws, size_t ws_bytes,
                     bool use_scratch, hipStream_t stream);

}  // namespace

extern "C" {

int32_t kve_version(void) { return 10400; }  // 1.4.0

size_t kve_prefill_workspace_bytes(const kve_shape* shape, int32_t len) {
  if (check_shape(shape) != KVE_OK || len < 1 || len > kve::kMaxPrefillLen)
    return 0;
  return kve::prefill_ws_bytes((long long)shape->batch * shape->n_kv_heads, len);
}

kve_status kve_prefill_select(const kve_shape* shape, const kve_policy* policy,
                              const kve_cache* cache, int32_t len,
                              int32_t* rank, int32_t* tau, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  kve_status st = check_shape(shape);
  if (st != KVE_OK) return st;
  if ((st = check_policy(policy)) != KVE_OK) return st;
  if (policy->gumbel) return KVE_ERR_UNSUPPORTED;  // deterministic ranks only
  if ((st = check_cache(cache)) != KVE_OK) return st;
  if (!rank || !tau) return KVE_ERR_INVALID_ARG;
  if (!a4(rank) || !a4(tau) || !a16(ws)) return KVE_ERR_INVALID_ARG;
  if (len < 1) return KVE_ERR_INVALID_ARG;
  if (len > shape->capacity) return KVE_ERR_CAPACITY;
  if (len > kve::kMaxPrefillLen) return KVE_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < kve_prefill_workspace_bytes(shape, len))
    return KVE_ERR_WORKSPACE;
  if ((long long)shape->batch * shape->n_kv_heads > 65535)
    return KVE_ERR_UNSUPPORTED;  // one grid row per slice
  const int k = policy->budget - policy->sinks - policy->window;
  return from_hip(kve::launch_prefill_select(
      cache->score, policy->log_gamma, shape->n_kv_heads,
      shape->batch * shape->n_kv_heads, shape->capacity, len, policy->sinks,
      policy->window, k, ws, rank, tau, stream));
}

size_t kve_prefill_attn_workspace_bytes(const kve_shape* shape,
                                        const kve_policy* policy, int32_t len) {
  if (check_shape(shape) != KVE_OK || check_policy(policy) != KVE_OK ||
      len < 1 || len > kve::kMaxPrefillLen)
    return 0;
  const int k = policy->budget - policy->sinks - policy->window;
  return kve::prefill_attn_ws_bytes((long long)shape->batch * shape->n_kv_heads,
                                    len, k > 0 ? k : 1, shape->head_dim);
}

kve_status kve_prefill_attn(const kve_shape* shape, const kve_policy* policy,
                            const kve_cache* cache, int32_t len,
                            const int32_t* rank, const int32_t* tau,
                            const void* q, float* out, float* lse, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  kve_status st = check_shape(shape);
  if (st != KVE_OK) return st;
  if ((st = check_policy(policy)) != KVE_OK) return st;
  if (policy->gumbel) return KVE_ERR_UNSUPPORTED;  // deterministic ranks only
  if ((st = check_cache(cache)) != KVE_OK) return st;
  if (!rank || !tau || !q || !out) return KVE_ERR_INVALID_ARG;
  if (!a4(rank) || !a4(tau) || !a16(q) || !a16(out) || !a4(lse) || !a16(ws))
    return KVE_ERR_INVALID_ARG;
  if (len < 1) return KVE_ERR_INVALID_ARG;
  if (len > shape->capacity) return KVE_ERR_CAPACITY;
  if (len > kve::kMaxPrefillLen) return KVE_ERR_UNSUPPORTED;
  if (shape->kv_dtype != KVE_BF16) return KVE_ERR_UNSUPPORTED;
  const size_t need = kve_prefill_attn_workspace_bytes(shape, policy, len);
  if (!ws || ws_bytes < need) return KVE_ERR_WORKSPACE;
  if ((long long)shape->batch * shape->n_kv_heads > 65535)
    return KVE_ERR_UNSUPPORTED;  // one grid row per slice (key lists)
  const int k = policy->budget - policy->sinks - policy->window;
  kve::PrefillAttnLaunch a{};
  a.kmax = k > 0 ? k : 1;
  a.k = cache->k;
  a.v = cache->v;
  a.rank = rank;
  a.tau = tau;
  a.q = q;
  a.out = out;
  a.lse = lse;
  a.batch = shape->batch;
  a.H = shape->n_kv_heads;
  a.G = shape->group;
  a.D = shape->head_dim;
  a.cap = shape->capacity;
  a.n = len;
  a.S = policy->sinks;
  a.W = policy->window;
  // Query heads of a KV head in subsets of at most 2 per workgroup: the
  // kernel then fits two waves per SIMD (measured faster than 4 heads and
  // one wave per SIMD, although each K/V block is read by more workgroups).
  a.nsub = (shape->group + 1) / 2;
  a.gsub = (shape->group + a.nsub - 1) / a.nsub;
  if ((long long)a.H * a.nsub > 65535) return KVE_ERR_UNSUPPORTED;
  return from_hip(kve::launch_prefill_attn(a, ws, stream));
}

const char* kve_status_str(kve_status s) {
  switch (s) {
    case KVE_OK: return "ok";
    case KVE_ERR_INVALID_ARG: return "invalid argument";
    case KVE_ERR_POLICY: return "invalid policy";
    case KVE_ERR_CAPACITY: return "capacity exceeded";
    case KVE_ERR_UNSUPPORTED: return "unsupported shape, dtype or scorer";
    case KVE_ERR_WORKSPACE: return "workspace missing or too small";
    case KVE_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

size_t kve_workspace_bytes(const kve_shape* shape, int32_t max_len) {
  if (check_shape(shape) != KVE_OK || max_len < 1) return 0;
  // At least one aligned block, so a valid workspace pointer always exists.
  const size_t n = ws_bytes_for(shape, split_cap(shape, max_len));
  return n > 0 ? n : kAlign;
}

size_t kve_scorer_state_bytes(const kve_shape* shape,
                              const kve_scorer* scorer) {
  if (check_shape(shape) != KVE_OK || check_scorer(shape, scorer) != KVE_OK)
    return 0;
  if (scorer->kind != KVE_SCORER_MLSTM) return 0;
  return (size_t)shape->batch * shape->n_kv_heads *
         kve::mlstm_state_floats(shape->head_dim) * sizeof(float);
}

kve_status kve_append(const kve_shape* shape, kve_cache* cache, int32_t slot,
                      int32_t position, const void* k_new, const void* v_new,
                      hipStream_t stream) {
  kve_status st = check_shape(shape);
  if (st != KVE_OK) return st;
  if ((st = check_cache(cache)) != KVE_OK) return st;
  if (!k_new || !v_new) return KVE_ERR_INVALID_ARG;
  if (!a16(k_new) || !a16(v_new)) return KVE_ERR_INVALID_ARG;
  if (slot < 0 || slot >= shape->capacity) return KVE_ERR_CAPACITY;
  return from_hip(kve::launch_append(
      cache->k, cache->v, cache->pos, shape->batch, shape->n_kv_heads,
      shape->head_dim, shape->capacity, elem_bytes(shape->kv_dtype), slot,
      position, k_new, v_new, nullptr, nullptr, 0, 0, 0, stream));
}

kve_status kve_score(const kve_shape* shape, const kve_scorer* scorer,
                     kve_cache* cache, int32_t slot_begin, int32_t slot_end,
                     const void* hidden, hipStream_t stream) {
  kve_status st = check_shape(shape);
  if (st != KVE_OK) return st;
  if ((st = check_cache(cache)) != KVE_OK) return st;
  if ((st = check_scorer(shape, scorer)) != KVE_OK) return st;
  if (slot_begin < 0 || slot_end < slot_begin) return KVE_ERR_INVALID_ARG;
  if (slot_end > shape->capacity) return KVE_ERR_CAPACITY;
  const bool gate = scorer->kind == KVE_SCORER_GATE_HIDDEN ||
                    scorer->kind == KVE_SCORER_SINK_GATE;
  if (gate != (hidden != nullptr)) return KVE_ERR_INVALID_ARG;
  if (!a16(hidden)) return KVE_ERR_INVALID_ARG;
  if (scorer->kind == KVE_SCORER_MLSTM && !cache->scorer_state)
    return KVE_ERR_INVALID_ARG;
  const long long stride = (long long)(slot_end - slot_begin) * scorer->in_dim;
  return score_impl(shape, scorer, cache, slot_begin, slot_end, hidden, stride,
                    stream);
}

kve_status kve_select_evict(const kve_shape* shape, const kve_policy* policy,
                            const kve_cache* cache, int32_t len,
                            int32_t n_keep, int32_t* keep_slots,
                            hipStream_t stream) {
  kve_status st = check_shape(shape);
  if (st != KVE_OK) return st;
  if ((st = check_policy(policy)) != KVE_OK) return st;
  if ((st = check_cache(cache)) != KVE_OK) return st;
  if (!keep_slots || !a4(keep_slots)) return KVE_ERR_INVALID_ARG;
  if (len < 0 || n_keep < 0) return KVE_ERR_INVALID_ARG;
  if (len > shape->capacity) return KVE_ERR_CAPACITY;
  if (n_keep > len) return KVE_ERR_POLICY;
  if (n_keep < len && (long long)policy->sinks + policy->window > n_keep)
    return KVE_ERR_POLICY;
  if (len == 0) return KVE_OK;
  return from_hip(kve::launch_select(
      cache->score, cache->pos, policy->log_gamma, policy->gumbel,
      shape->n_kv_heads,
      shape->batch * shape->n_kv_heads, shape->capacity, len, n_keep,
      policy->sinks, policy->window, keep_slots, stream));
}

kve_status kve_compact(const kve_shape* shape, kve_cache* cache, int32_t len,
                       const int32_t* keep_slots, int32_t n_keep,
                       hipStream_t stream) {
  kve_status st = check_shape(shape);
  if (st != KVE_OK) return st;
  if ((st = check_cache(cache)) != KVE_OK) return st;
  if (!keep_slots || !a4(keep_slots)) return KVE_ERR_INVALID_ARG;
  if (len < 0 || n_keep < 0 || n_keep > len) return KVE_ERR_INVALID_ARG;
  if (len > shape->capacity) return KVE_ERR_CAPACITY;
  if (n_keep == 0) return KVE_OK;
  return from_hip(kve::launch_compact(
      cache->k, cache->v, cache->score, cache->pos,
      shape->batch * shape->n_kv_heads, shape->capacity,
      shape->head_dim * elem_bytes(shape->kv_dtype), len, keep_slots, n_keep,
      stream));
}

kve_status kve_decode_attn(const kve_shape* shape, const kve_cache* cache,
                           int32_t len, const void* q, float* out, float* lse,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
  kve_status st = check_shape(shape);
  if (st != KVE_OK) return st;
  if ((st = check_cache(cache)) != KVE_OK) return st;
  if (!q || !out) return KVE_ERR_INVALID_ARG;
  if (!a16(q) || !a16(out) || !a4(lse) || !a16(ws)) return KVE_ERR_INVALID_ARG;
  if (len < 1) return KVE_ERR_INVALID_ARG;
  if (len > shape->capacity) return KVE_ERR_CAPACITY;
  return attn_impl(shape, cache, len, q, out, lse, ws, ws_bytes, -1, 0,
                   nullptr, nullptr, stream);
}


kve_status kve_step(const kve_shape* shape, const kve_policy* policy,
                    const kve_scorer* scorer, kve_cache* cache,
                    kve_decode_state* state, const void* k_new,
                    const void* v_new, const void* hidden_new,
                    void* hidden_buf, const void* q, float* out, float* lse,
                    int32_t* keep_slots, void* ws, size_t ws_bytes,
                    hipStream_t stream) {
  return step_impl(shape, policy, scorer, cache, state, k_new, v_new,
                   hidden_new, hidden_buf, q, out, lse, keep_slots, ws,
                   ws_bytes, false, stream);
}

kve_status kve_step_noalloc(const kve_shape* shape, const kve_policy* policy,
                            const kve_scorer* scorer, kve_cache* cache,
                            kve_decode_state* state, const void* k_new,
                            const void* v_new, const void* hidden_new,
                            void* hidden_buf, const void* q, float* out,
                            float* lse, int32_t* keep_slots,
                            hipStream_t stream) {
  return step_impl(shape, policy, scorer, cache, state, k_new, v_new,
                   hidden_new, hidden_buf, q, out, lse, keep_slots, nullptr,
                   0, true, stream);
}

}  // extern "C"

namespace {

kve_status step_impl(const kve_shape* shape, const kve_policy* policy,
                     const kve_scorer* scorer, kve_cache* cache,
                     kve_decode_state* state, const void* k_new,
                     const void* v_new, const void* hidden_new,
                     void* hidden_buf, const void* q, float* out, float* lse,
                     int32_t* keep_slots, void* ws, size_t ws_bytes,
                     bool use_scratch, hipStream_t stream) {
  kve_status st = check_shape(shape);
  if (st != KVE_OK) return st;
  if ((st = check_policy(policy)) != KVE_OK) return st;
  if ((st = check_cache(cache)) != KVE_OK) return st;
  if ((st = check_scorer(shape, scorer)) != KVE_OK) return st;
  if (!state || !k_new || !v_new || !q || !out || !keep_slots)
    return KVE_ERR_INVALID_ARG;
  if (!a16(k_new) || !a16(v_new) || !a16(q) || !a16(out) || !a4(lse) ||
      !a4(keep_slots) || !a16(hidden_new) || !a16(hidden_buf) || !a16(ws))
    return KVE_ERR_INVALID_ARG;
  const int B = policy->budget, L = policy->evict_len;
  if ((long long)B + L > shape->capacity) return KVE_ERR_CAPACITY;
  const bool gate = scorer->kind == KVE_SCORER_GATE_HIDDEN ||
                    scorer->kind == KVE_SCORER_SINK_GATE;
  if (gate != (hidden_new != nullptr) || gate != (hidden_buf != nullptr))
    return KVE_ERR_INVALID_ARG;
  if (scorer->kind == KVE_SCORER_MLSTM) {
    if (!cache->scorer_state) return KVE_ERR_INVALID_ARG;
    if (scorer->delay != policy->window) return KVE_ERR_POLICY;
  }
  int len = state->len;
  int scored = state->scored_upto;
  if (len < 0 || scored < 0 || scored > len) return KVE_ERR_INVALID_ARG;
  if (len >= shape->capacity) return KVE_ERR_CAPACITY;
  if (len - scored >= L) return KVE_ERR_INVALID_ARG;  // pending buffer full
  // The attention after this step covers len + 1 rows at most, and the
  // split cap never decreases with len.
  if (!use_scratch &&
      (!ws || ws_bytes < ws_bytes_for(shape, split_cap(shape, len + 1))))
    return KVE_ERR_WORKSPACE;

  const int slot = len;
  const int position = state->next_position;
  const int new_len = len + 1;
  const bool evict = new_len >= B + L;
  const bool score_now = evict || (new_len - scored) >= L;
  const int slices = shape->batch * shape->n_kv_heads;
  const int row_bytes = shape->head_dim * elem_bytes(shape->kv_dtype);
  // Launches of this step, in order: append (when a scoring is due: the new
  // row must be in place before it is scored or selected; otherwise the
  // attention launch appends it), scoring of the pending rows, select and
  // compaction (when the count reaches B + L), attention. Pass 0 checks
  // every launch configuration on the host and launches nothing, so a step
  // the kernels cannot run fails before it touches the device; pass 1
  // enqueues them.
  const int att_len = evict ? B : new_len;
  const int att_scored = score_now ? (evict ? B : new_len) : scored;
  if (use_scratch) {
    // The attention plan of this step must fit the scratch array; its
    // address is looked up only then (so argument errors come first).
    if (ws_bytes_for(shape, plan_split(shape, att_len).nsplit) >
        kNoallocScratchBytes)
      return KVE_ERR_WORKSPACE;
    ws = noalloc_scratch(&st);
    if (!ws) return st;
    ws_bytes = kNoallocScratchBytes;
  }
  // An evicting step of a bf16 MLP-scored cache whose pending rows cover
  // every row compaction moves runs append, scoring, select and compaction
  // as one launch (the same results, the moved rows read once).
  const bool fused_mlp =
      evict && scorer->kind == KVE_SCORER_MLP_KV &&
      shape->kv_dtype == KVE_BF16 &&
      kve::evict_mlp_fits(shape->head_dim, scorer->hidden, new_len, B, scored);
  for (int pass = 0; pass < 2; ++pass) {
    const bool chk = pass == 0;
    auto done = [chk](hipError_t e) {
      return chk ? from_check(e) : from_hip(e);
    };
    if (fused_mlp) {
      kve::EvictMlpLaunchArgs e{};
      e.k = cache->k;
      e.v = cache->v;
      e.score = cache->score;
      e.pos = cache->pos;
      e.w1 = scorer->w1;
      e.b1 = scorer->b1;
      e.w2 = scorer->w2;
      e.b2 = scorer->b2;
      e.act = scorer->act;
      e.log_gamma = policy->log_gamma;
      e.gumbel = policy->gumbel;
      e.slices = slices;
      e.H = shape->n_kv_heads;
      e.D = shape->head_dim;
      e.hidden = scorer->hidden;
      e.cap = shape->capacity;
      e.len = new_len;
      e.n_keep = B;
      e.S = policy->sinks;
      e.W = policy->window;
      e.pend0 = scored;
      e.keep = keep_slots;
      e.k_new = k_new;
      e.v_new = v_new;
      e.new_pos = position;
      st = done(kve::launch_evict_mlp(e, stream, chk));
      if (st != KVE_OK) return st;
    } else if (score_now) {
      st = done(kve::launch_append(
          cache->k, cache->v, cache->pos, shape->batch, shape->n_kv_heads,
          shape->head_dim, shape->capacity, elem_bytes(shape->kv_dtype), slot,
          position, k_new, v_new, hidden_new, hidden_buf, scorer->in_dim, L,
          slot - scored, stream, chk));
      if (st != KVE_OK) return st;
      st = score_impl(shape, scorer, cache, scored, new_len, hidden_buf,
                      (long long)L * scorer->in_dim, stream, chk);
      if (st != KVE_OK) return st;
    }
    if (evict && !fused_mlp) {
      st = done(kve::launch_select_compact(
          cache->k, cache->v, cache->score, cache->pos, policy->log_gamma,
          policy->gumbel, shape->n_kv_heads, slices, shape->capacity,
          row_bytes, new_len, B, policy->sinks, policy->window, keep_slots,
          stream, chk));
      if (st != KVE_OK) return st;
    }
    st = attn_impl(shape, cache, att_len, q, out, lse, ws, ws_bytes,
                   score_now ? -1 : slot, position, k_new, v_new, stream,
                   gate ? hidden_new : nullptr, hidden_buf, scorer->in_dim * 2,
                   L, slot - att_scored, chk);
    if (st != KVE_OK) return st;
  }
  state->evicted = evict ? 1 : 0;
  len = att_len;
  scored = att_scored;
  state->len = len;
  state->scored_upto = scored;
  state->next_position = position + 1;
  return KVE_OK;
}

}  // namespace
