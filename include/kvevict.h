/*
 * libkvevict - fixed-budget KV-cache evict-and-attend decode step for
 * AMD Instinct MI355X (gfx950).
 *
 * C ABI. Every tensor argument is a plain device pointer into caller-owned
 * memory (HIP device memory); shape, policy and scorer descriptors are
 * plain host structs. The library allocates nothing, keeps no state between
 * calls and never synchronises the device: every call validates its
 * arguments on the host, enqueues kernels on `stream` and returns. Argument
 * errors are reported by the returned status before anything is launched.
 * Device faults (for example a dangling pointer) surface at the caller's next
 * synchronisation.
 *
 * Method (the pages this library follows):
 *  - KVpop ("KVpop - Key-Value Cache Compression with Predictive Online
 *    Pruning"): per-KV-head budget B = s + w + k (section 3, Eq. 1); sink
 *    tokens, a protected window of the w most recent tokens, and the top-k
 *    eligible tokens E(q) = {t | s <= t <= q - w} (section 3.1, Eq. 4;
 *    Appendix C.1, Eq. 26); stateless head-wise MLP scorer over [k; v]
 *    (section 3.3, Appendix E.1-E.2, Eq. 35-36); decode attention directly
 *    over the compact cache of retained entries (Appendix C), with logits
 *    <q, k>/sqrt(d_k) and log-sum-exp normaliser (Appendix D.1, Eq. 27-29);
 *    ranking in float32 (Appendix F).
 *  - ForesightKV summary page ("ForesightKV: Optimizing KV Cache Eviction for
 *    Reasoning Models by Learning Long-Term Contribution", "Methodology in
 *    plain English"): periodic eviction with budget B and eviction length L;
 *    when the cache reaches B + L the recent tokens are protected and the
 *    lowest-scored pairs are evicted back to the budget.
 *  - Fast KVzip ("Fast KVzip: Efficient and Accurate LLM Inference with Gated
 *    KV Eviction"): per-KV-head gate on the layer's hidden state with output
 *    in [0, 1] (section 3.1 "Formulation"); buffered scoring of the pending
 *    tokens in parallel, then eviction of as many entries (section 3.1 and
 *    Appendix A.5); the low-rank sink-attention gate (section 3.4).
 *  - Optional parts of the path: KVpop's temporal decay in the ranking
 *    (Appendix B.3, Eq. 20), its stateful mLSTM scorer with delayed read-out
 *    (section 3.3, Appendix A and E.3-E.4), its running top-k selection and
 *    masked prefill attention (section 3.2, Appendix C.1-C.2, Eq. 26), and
 *    ForesightKV's stochastic eviction from the 2L lowest-scored candidates
 *    (summary page, "Key Contributions" item 4).
 *
 * Tensor layouts (row-major, innermost last):
 *   K, V        [batch][n_kv_heads][capacity][head_dim]   kv_dtype
 *   score       [batch][n_kv_heads][capacity]             float32
 *   pos         [batch][n_kv_heads][capacity]             int32
 *   q           [batch][n_kv_heads*group][head_dim]       kv_dtype
 *   out         [batch][n_kv_heads*group][head_dim]       float32
 *   lse         [batch][n_kv_heads*group]                 float32
 *   k_new,v_new [batch][n_kv_heads][head_dim]             kv_dtype
 *   keep_slots  [batch][n_kv_heads][n_keep]               int32, ascending
 * Query head j reads KV head j / group (contiguous GQA groups).
 * Every (batch, KV head) slice holds the same number of entries `len` in
 * slots [0, len), with distinct positions in any slot order: new tokens are
 * appended at slot len, and compaction moves entries from the end into the
 * slots it frees.
 * Alignment: kernels move rows with 16-byte vector accesses, so K, V, q,
 * out, k_new, v_new, hidden states, scorer state, the scorer's w1 and
 * workspaces must be 16-byte aligned, and float32 / int32 arrays (score,
 * pos, lse, keep_slots, rank, tau, the scorer's other weights) 4-byte
 * aligned (PyTorch allocations are 512-byte aligned); a
 * misaligned pointer is KVE_ERR_INVALID_ARG.
 */
#ifndef KVEVICT_H
#define KVEVICT_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVE_OK = 0,
  KVE_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad range */
  KVE_ERR_POLICY = 2,      /* B < S + W, L < 1, n_keep out of range */
  KVE_ERR_CAPACITY = 3,    /* len or slot beyond capacity */
  KVE_ERR_UNSUPPORTED = 4, /* head_dim, dtype, group or scorer shape */
  KVE_ERR_WORKSPACE = 5,   /* workspace missing or too small */
  KVE_ERR_LAUNCH = 6       /* the HIP runtime refused a launch */
} kve_status;

typedef enum { KVE_F32 = 0, KVE_BF16 = 1 } kve_dtype;
typedef enum { KVE_ACT_RELU = 0, KVE_ACT_SILU = 1 } kve_act;
typedef enum {
  KVE_SCORER_MLP_KV = 0,
  KVE_SCORER_GATE_HIDDEN = 1,
  KVE_SCORER_MLSTM = 2,
  KVE_SCORER_SINK_GATE = 3
} kve_scorer_kind;

/* Shape of one layer's cache. head_dim in {64, 128}; group in [1, 8];
 * kv_dtype is a kve_dtype. capacity = slots per (batch, KV head) slice.
 * Limits (KVE_ERR_UNSUPPORTED beyond them): batch and n_kv_heads at most
 * 65535, batch * n_kv_heads below 2^31, and one slice's K (or V) rows,
 * capacity * head_dim * element bytes, below 4 GiB. */
typedef struct {
  int32_t batch;
  int32_t n_kv_heads;
  int32_t group;
  int32_t head_dim;
  int32_t capacity;
  int32_t kv_dtype;
} kve_shape;

/* Retention policy: budget B, sinks S, window W, eviction length L.
 * Requires B >= S + W >= 0 and L >= 1 (KVpop Eq. 1: k = B - S - W >= 0).
 * log_gamma: NULL, or a device array [n_kv_heads] of float32 log decay
 * factors (KVpop Eq. 5 with decay step 1, gamma in (0, 1)): eligible entries
 * are then ranked by the static priority score - position * log_gamma[h]
 * (KVpop Appendix B.3, Eq. 20), both operations rounded to float32.
 * gumbel: NULL (deterministic eviction), or a device array
 * [batch][n_kv_heads][capacity] of float32 standard Gumbel noise, one value
 * per cache slot, for ForesightKV's stochastic eviction (summary page, "Key
 * Contributions" item 4): to evict r entries, the 2r lowest-ranked
 * candidates (all candidates if fewer) form a pool and r of them are drawn
 * without replacement with probability proportional to exp(-key). The draw
 * is the Gumbel-top-k one: the r pool entries with the largest float32 sum
 * -key + gumbel[slot] are evicted, equal sums taking the lower position
 * first. Zero noise gives the deterministic rule. The caller refreshes the
 * noise before each evicting call; it must be finite. Used by
 * kve_select_evict and kve_step; the prefill entry points reject it. */
typedef struct {
  int32_t budget;
  int32_t sinks;
  int32_t window;
  int32_t evict_len;
  const float* log_gamma;
  const float* gumbel;
} kve_policy;

/* Device pointers of one layer's cache (layouts above). scorer_state is
 * the recurrent state of a stateful (MLSTM) scorer,
 * kve_scorer_state_bytes() bytes, caller-owned: all-zero bytes are the
 * empty state (no token absorbed), its layout is otherwise private to the
 * library. NULL for stateless scorers. */
typedef struct {
  void* k;
  void* v;
  float* score;
  int32_t* pos;
  float* scorer_state;
} kve_cache;

/* Scorer weights (device pointers).
 *  MLP over [k; v] (KVpop Eq. 35-36): in_dim = 2 * head_dim;
 *    score = w2 . act(W1 x + b1) + b2, x = [k; v] (key first).
 *    w1 [H][hidden][in_dim] in wdtype (row j: input weights of hidden unit j),
 *    b1 [H][hidden] float32 or NULL, w2 [H][hidden] float32,
 *    b2 [H] float32 or NULL. hidden in [1, 256]; wdtype == kv_dtype.
 *  GATE on hidden states (Fast KVzip section 3.1): in_dim = D,
 *    score = sigmoid(w1[h] . x + b1[h]); w1 [H][D] bf16, b1 [H] float32 or
 *    NULL; hidden, w2, b2, act unused. D a multiple of 32, H <= 16.
 *  MLSTM, stateful with delayed read-out (KVpop section 3.3, Appendix E.3-
 *    E.4, Eq. 37-42, Hedgehog features of Appendix A): x = [k; v],
 *    in_dim = 2 * head_dim, hidden = P = head_dim / 2 (projection width; the
 *    features q~, k~ have 2P entries). w1 [H][3P + 2][in_dim] bf16 holds the
 *    rows of W_q (P rows), W_k (P), W_v (P), then w_i and w_f; b1 [H][2]
 *    float32 (b_i, b_f) or NULL; w2 [H][P] float32 is the read-out a, b2 [H]
 *    float32 or NULL its bias. delay = W: after absorbing the token at
 *    position q the scorer scores position q - W (no score while fewer than
 *    W tokens precede q in the state). kv_dtype and wdtype bf16; act unused.
 *  SINK_GATE, low-rank sink attention on hidden states (Fast KVzip section
 *    3.4): in_dim = D (a multiple of 32), hidden = D' = 16, n_sink = S in
 *    [0, 16]. w1 [H*16 + H*G*16][D] bf16 holds the rows of W_k (16 per KV
 *    head) then W_q (16 per query head j = h*G + g); b1 [32] float32 the
 *    normalisation weights of k then q, or NULL (ones); w2 [S][16] float32
 *    the layer's sink keys; b2 [H*G] float32 the denominator terms b_j, or
 *    NULL (zeros). With k = norm(W_k[h] x), q_j = norm(W_q[j] x) (RMS,
 *    eps 1e-6), a_j = q_j . k / 4 and c_jr = q_j . sink_r / 4:
 *    score_h = max_g exp(a_j) / (exp(a_j) + sum_r exp(c_jr) + b_j).
 *    Hidden states are passed as for GATE.
 *  delay is read for MLSTM only, n_sink for SINK_GATE only. */
typedef struct {
  int32_t kind;   /* kve_scorer_kind */
  int32_t act;    /* kve_act (MLP only) */
  int32_t wdtype; /* kve_dtype of w1 */
  int32_t in_dim;
  int32_t hidden;
  const void* w1;
  const float* b1;
  const float* w2;
  const float* b2;
  int32_t delay;
  int32_t n_sink;
} kve_scorer;

/* Host-side decode state of one layer for kve_step (in/out).
 *  len           entries in every slice, slots [0, len)
 *  scored_upto   slots [0, scored_upto) hold scores; [scored_upto, len) are
 *                pending (appended since the last scoring)
 *  next_position absolute position given to the next appended token
 *  evicted       set by kve_step: 1 if this step evicted, else 0 */
typedef struct {
  int32_t len;
  int32_t scored_upto;
  int32_t next_position;
  int32_t evicted;
} kve_decode_state;

/* Bytes of workspace that kve_decode_attn / kve_step need for caches of up
 * to max_len entries: the split-K partial results (per query head and split:
 * head_dim accumulator sums, running maximum and normaliser, float32). The
 * size depends on the shape and max_len only. The workspace needs no
 * initialisation; its contents are scratch and undefined between calls, and
 * calls that share one workspace must be ordered (same stream). Returns 0
 * on invalid arguments. */
size_t kve_workspace_bytes(const kve_shape* shape, int32_t max_len);

/* Bytes of scorer_state that a stateful scorer needs for this shape:
 * batch * n_kv_heads slices of float32 state (matrix memory C [2P][P],
 * normaliser z [2P], log scale and token count). 0 for stateless scorers
 * and on invalid arguments. */
size_t kve_scorer_state_bytes(const kve_shape* shape, const kve_scorer* scorer);

/* a1 Append (KVpop Appendix C): write one new token per slice into `slot`:
 * K[b][h][slot] = k_new[b][h], V likewise, pos[b][h][slot] = position.
 * Requires 0 <= slot < capacity. The score of the slot is left unset
 * (pending) until kve_score covers it. */
kve_status kve_append(const kve_shape* shape, kve_cache* cache, int32_t slot,
                      int32_t position, const void* k_new, const void* v_new,
                      hipStream_t stream);

/* a2 Score the slots [slot_begin, slot_end) of every slice into
 * cache->score (float32). MLP reads the cached K, V rows of those slots
 * (KVpop Eq. 35-36). GATE and SINK_GATE read `hidden`
 * [batch][slot_end-slot_begin][D] bf16, the hidden states of those tokens
 * (Fast KVzip sections 3.1 and 3.4); `hidden` must be NULL for MLP and
 * MLSTM. MLP, GATE and SINK_GATE run as bf16 MFMA GEMMs with float32
 * accumulation (float32 VALU for float32 MLP weights).
 * MLSTM absorbs the cached tokens of those slots into cache->scorer_state in
 * slot order and writes the score of every token it reads out, into that
 * token's slot (KVpop Eq. 41-42). The slots must hold consecutive positions
 * that continue the state's history, every token read out must be cached in
 * a slot below slot_end, and the tokens of slots [0, slot_begin) must be
 * older than those absorbed. Projections on MFMA (bf16, float32
 * accumulation), the recurrence in float32. */
kve_status kve_score(const kve_shape* shape, const kve_scorer* scorer,
                     kve_cache* cache, int32_t slot_begin, int32_t slot_end,
                     const void* hidden, hipStream_t stream);

/* a3 Select (KVpop Eq. 4 and Eq. 26; ForesightKV periodic eviction): cut
 * each slice of `len` entries to `n_keep`. With P the newest position in the
 * slice, entries with position < S (sinks) or > P - W (recent window) are
 * protected; among the eligible entries (S <= position <= P - W) the
 * len - n_keep with the smallest (float32 key, position) are evicted, the
 * key being the score or, with policy->log_gamma, the static priority:
 * equal keys evict the older entry first, and -0.0 ranks as +0.0. Writes
 * the kept slots in ascending order to keep_slots [batch][H][n_keep].
 * Requires 0 <= n_keep <= len <= capacity, and S + W <= n_keep when
 * n_keep < len; n_keep == len writes the identity. Scores must be finite;
 * positions distinct, with the S oldest and W newest present (as the
 * library's own appends and compaction keep them). With policy->gumbel the
 * evicted entries are drawn by ForesightKV's stochastic rule instead (see
 * kve_policy); the same noise and scores give the same kept slots. */
kve_status kve_select_evict(const kve_shape* shape, const kve_policy* policy,
                            const kve_cache* cache, int32_t len,
                            int32_t n_keep, int32_t* keep_slots,
                            hipStream_t stream);

/* a4 Compact in place (KVpop Appendix C: the cache keeps only retained
 * entries) after kve_select_evict: keep_slots lists the n_keep kept slots
 * of each slice in ascending order (each < len <= capacity). Kept entries
 * in slots below n_keep stay in place; the slots below n_keep that were not
 * kept, in ascending order, receive the kept entries from slots at or above
 * n_keep, in ascending order (K, V, score and pos move together). At most
 * min(n_keep, len - n_keep) rows per slice move. Slots >= n_keep are left
 * as they were. */
kve_status kve_compact(const kve_shape* shape, kve_cache* cache, int32_t len,
                       const int32_t* keep_slots, int32_t n_keep,
                       hipStream_t stream);

/* a5 Decode attention (KVpop Appendix C and D.1, Eq. 27-29) of the
 * n_kv_heads*group query heads in q over slots [0, len) of their KV head:
 * out = sum_t softmax_t(<q, k_t> / sqrt(d)) v_t, lse = log sum_t
 * exp(<q, k_t> / sqrt(d)). Float32 math and output. lse may be NULL.
 * Requires 1 <= len <= capacity and ws_bytes >= kve_workspace_bytes(shape,
 * len). */
kve_status kve_decode_attn(const kve_shape* shape, const kve_cache* cache,
                           int32_t len, const void* q, float* out, float* lse,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/* a6 One decode step of one layer, stream-ordered: append the new token at
 * slot state->len with position state->next_position; score the pending
 * slots when an eviction is due or L of them have accumulated (buffered
 * scoring, Fast KVzip section 3.1); when the cache reaches B + L, select
 * and compact it back to B (keep_slots receives the kept slots); then
 * attend over the cache. Updates *state on the host.
 * GATE scorers: hidden_new [batch][D] is the new token's hidden state and
 * hidden_buf [batch][L][D] (bf16, caller-owned) holds the pending tokens'
 * hidden states between calls (SINK_GATE likewise); both must be NULL for
 * MLP and MLSTM.
 * MLSTM scorers absorb the pending tokens at that point (the same scores as
 * absorbing every token as it arrives) and need scorer->delay equal to the
 * policy window. With policy->gumbel the eviction is stochastic, as in
 * kve_select_evict.
 * Requires capacity >= B + L and state->len < capacity.
 * Failure: the step validates its arguments and the launch configuration of
 * every kernel it will enqueue (append, scorer, select, compaction,
 * attention) on the host before it enqueues the first one; any such error
 * is returned with *state, the cache and the outputs untouched, so the
 * call may be corrected and repeated. Only a launch that the HIP runtime
 * itself refuses after that check (KVE_ERR_LAUNCH; the device or the
 * stream is already in an error state) can leave the step part-way: *state
 * is then unchanged, but the layer's cache contents are undefined and it
 * must be rebuilt before the next step. */
kve_status kve_step(const kve_shape* shape, const kve_policy* policy,
                    const kve_scorer* scorer, kve_cache* cache,
                    kve_decode_state* state, const void* k_new,
                    const void* v_new, const void* hidden_new,
                    void* hidden_buf, const void* q, float* out, float* lse,
                    int32_t* keep_slots, void* ws, size_t ws_bytes,
                    hipStream_t stream);

/* Size of the device scratch array that kve_step_noalloc uses, bytes. */
#define KVE_NOALLOC_SCRATCH_BYTES (2u << 20)

/* kve_step for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): no
 * workspace argument; the split-K partial results of the attention launch
 * live in a library-owned device array of KVE_NOALLOC_SCRATCH_BYTES per GPU,
 * held until the process ends (its address is looked up on the first call
 * on each device; nothing is allocated). Arguments, results, updates of
 * *state and the failure contract are those of kve_step. A step whose
 * attention plan needs more partial storage than the array holds returns
 * KVE_ERR_WORKSPACE before any launch (every shape whose
 * kve_workspace_bytes(shape, state->len + 1) is at most
 * KVE_NOALLOC_SCRATCH_BYTES fits; use kve_step with a workspace beyond
 * that). Every call on one GPU shares that GPU's array, and its contents
 * are scratch: calls that overlap on one GPU (on different streams, or from
 * host threads without ordering) race and give undefined results; order
 * them on one stream. */
kve_status kve_step_noalloc(const kve_shape* shape, const kve_policy* policy,
                            const kve_scorer* scorer, kve_cache* cache,
                            kve_decode_state* state, const void* k_new,
                            const void* v_new, const void* hidden_new,
                            void* hidden_buf, const void* q, float* out,
                            float* lse, int32_t* keep_slots,
                            hipStream_t stream);

/* Prefill selection (KVpop section 3.2 "Running top-k sparse attention",
 * Appendix C.1-C.2) for a prompt of len tokens held in slots [0, len) with
 * slot s holding position s, scored in cache->score (by kve_score):
 *  rank [batch][H][len] int32: rank(t) under the static priority, the score
 *    or, with policy->log_gamma, score - t * log_gamma[h] (both rounded to
 *    float32, as in kve_select_evict); rank 0 is the best, equal keys rank
 *    the newer token first;
 *  tau [batch][H][len] int32: for each query position q, the rank of the
 *    k-th best token of E(q) = {S <= t <= q - W}, k = B - S - W; len when
 *    E(q) holds fewer than k tokens, -1 when k = 0.
 * ws: kve_prefill_workspace_bytes(shape, len) bytes of scratch (sorted
 * keys). Requires 1 <= len <= min(capacity, 262144); scores finite;
 * policy->gumbel NULL (KVE_ERR_UNSUPPORTED otherwise: the running top-k is
 * deterministic). */
size_t kve_prefill_workspace_bytes(const kve_shape* shape, int32_t len);
kve_status kve_prefill_select(const kve_shape* shape, const kve_policy* policy,
                              const kve_cache* cache, int32_t len,
                              int32_t* rank, int32_t* tau, void* ws,
                              size_t ws_bytes, hipStream_t stream);

/* Masked prefill attention (KVpop Appendix C.1, Eq. 26, in the attention of
 * Appendix D.1 Eq. 27-29): for every query position q < len and query head
 * j (KV head j / G), attention over the keys t <= q that are sinks (t < S),
 * in the recent window (q - t < W) or eligible with rank(t) <= tau_q, with
 * rank and tau from kve_prefill_select. q [batch][H*G][len][d] bf16; out
 * [batch][H*G][len][d] float32; lse [batch][H*G][len] float32 natural-log
 * normaliser or NULL. bf16 caches only; MFMA with float32 accumulation and
 * softmax: q.k in bf16; the weighted sum of V in float16 (V converted
 * exactly, weights rounded to 11 significant bits) for a (batch, KV head)
 * slice whose largest |v| over positions < len lies in [2^-6, 65280], else
 * in bf16 with each weight as two parts (about 17 significant bits). ws:
 * kve_prefill_attn_workspace_bytes bytes of scratch: per 64-position query
 * block, the at most k long-range keys any of its queries keeps (the
 * attention visits only those, the sinks and the block's recent windows),
 * their count and the block's largest |v|, and V in float16 (len rows of d
 * per slice). policy->gumbel must be NULL, as for kve_prefill_select. */
size_t kve_prefill_attn_workspace_bytes(const kve_shape* shape,
                                        const kve_policy* policy, int32_t len);
kve_status kve_prefill_attn(const kve_shape* shape, const kve_policy* policy,
                            const kve_cache* cache, int32_t len,
                            const int32_t* rank, const int32_t* tau,
                            const void* q, float* out, float* lse, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/* Static string naming a status. */
const char* kve_status_str(kve_status status);

/* Library version (major * 10000 + minor * 100 + patch). */
int32_t kve_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVEVICT_H */
