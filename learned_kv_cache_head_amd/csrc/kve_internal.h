// Internal launch interface between the C-ABI layer (kvevict.hip) and the
// kernels. Not installed; the public interface is include/kvevict.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kve {

// ---------------------------------------------------------------------------
// Device helpers shared by the kernels.
// ---------------------------------------------------------------------------

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16lo(uint32_t w) {
  return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf16hi(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}

// Orderable 32-bit key of a float32 score: unsigned comparison of keys
// equals numeric comparison of scores; -0.0 maps to the key of +0.0.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Static priority under temporal decay (KVpop Eq. 20), ranked in float32
// (Appendix F): the product position * log(gamma) is rounded to float32,
// then the difference. Contraction is off here: hipcc fuses a * b + c into
// one multiply-add by default, which rounds once and can reorder keys that
// the two roundings make equal or adjacent.
__device__ __forceinline__ float decayed_priority(float s, int pos, float lg) {
#pragma clang fp contract(off)
  const float prod = (float)pos * lg;
  return s - prod;
}

// The noisy key of the stochastic rule: -key + noise, one float32 add.
__device__ __forceinline__ float noisy_key(float key, float noise) {
#pragma clang fp contract(off)
  return -key + noise;
}

// ---------------------------------------------------------------------------
// Launch descriptors.
// ---------------------------------------------------------------------------

constexpr int kMaxSplit = 256;  // split-K pieces per slice, at most

struct AttnLaunch {
  const void* k;        // cache base [batch][H][cap][D]
  const void* v;
  const void* q;        // [batch][H*G][D]
  float* out;           // [batch][H*G][D]
  float* lse;           // [batch][H*G] or null
  float* partial;       // [batch][H*G][nsplit][D+2] (acc[D], m, l); nsplit > 1
  int batch, H, G, D, cap, len;
  int nsplit, rows_per_split;
  int is_bf16;
  // Optional fused append of the newest token into slot new_slot.
  int new_slot;         // -1: none
  int new_pos;
  const void* k_new;    // [batch][H][D]
  const void* v_new;
  void* k_store;        // cache base pointers for the append (same as k, v)
  void* v_store;
  int32_t* pos;         // [batch][H][cap]
  // Optional fused copy of the new token's hidden state (hidden-state
  // scorers): hidden_new [batch][hidden_bytes] -> row hidden_row of
  // hidden_buf [batch][hidden_rows][hidden_bytes]. Null: none.
  const void* hidden_new;
  void* hidden_buf;
  int hidden_bytes, hidden_rows, hidden_row;
};

// Every launcher validates its launch configuration on the host first and
// returns hipErrorInvalidValue if the kernel cannot run it. With check_only
// it stops there and launches nothing: kve_step checks every launch of a
// step this way before it enqueues the first one.
hipError_t launch_attention(const AttnLaunch& a, hipStream_t s,
                            bool check_only = false);

hipError_t launch_append(void* k, void* v, int32_t* pos, int batch, int H,
                         int D, int cap, int elem_bytes, int slot,
                         int position, const void* k_new, const void* v_new,
                         const void* hidden_new, void* hidden_buf,
                         int hidden_dim, int hidden_rows, int hidden_row,
                         hipStream_t s, bool check_only = false);

hipError_t launch_select(const float* score, const int32_t* pos,
                         const float* log_gamma, const float* gumbel, int H,
                         int slices, int cap, int len, int n_keep, int S,
                         int W, int32_t* keep, hipStream_t s,
                         bool check_only = false);

hipError_t launch_compact(void* k, void* v, float* score, int32_t* pos,
                          int slices, int cap, int row_bytes, int len,
                          const int32_t* keep, int n_keep, hipStream_t s,
                          bool check_only = false);

// Select followed by compaction, as one launch when the slice is short
// enough for the register-resident select (the kept list stays on chip),
// else launch_select then launch_compact. Same results as the two calls.
hipError_t launch_select_compact(void* k, void* v, float* score, int32_t* pos,
                                 const float* log_gamma, const float* gumbel,
                                 int H, int slices, int cap, int row_bytes,
                                 int len, int n_keep, int S, int W,
                                 int32_t* keep, hipStream_t s,
                                 bool check_only = false);

// The evicting step of a bf16 MLP-scored cache in one launch (optionally
// with the new token's append): scoring of the pending rows [pend0, len),
// select and compaction to n_keep, the moved rows read once. Same results
// as launch_append + launch_score_mlp + launch_select_compact. Only shapes
// for which evict_mlp_fits holds: slices of up to 4096 entries, at most 128
// pending rows, and pend0 <= n_keep (every row that moves is pending).
struct EvictMlpLaunchArgs {
  void* k;
  void* v;
  float* score;
  int32_t* pos;
  const void* w1;
  const float* b1;
  const float* w2;
  const float* b2;
  int act;
  const float* log_gamma;
  const float* gumbel;
  int slices, H, D, hidden, cap, len, n_keep, S, W, pend0;
  int32_t* keep;
  const void* k_new;     // null: the new row is already in slot len - 1
  const void* v_new;
  int new_pos;
};
bool evict_mlp_fits(int D, int hidden, int len, int n_keep, int pend0);
hipError_t launch_evict_mlp(const EvictMlpLaunchArgs& e, hipStream_t s,
                            bool check_only = false);

struct MlpLaunch {
  const void* k;         // cache base
  const void* v;
  float* score;          // [batch][H][cap]
  const void* w1;        // [H][hidden][in_dim]
  const float* b1;       // [H][hidden] or null
  const float* w2;       // [H][hidden]
  const float* b2;       // [H] or null
  int batch, H, D, cap, hidden, act, is_bf16;
  int slot_begin, slot_end;
  int cus;               // compute units of the device (workgroup sizing)
};
hipError_t launch_score_mlp(const MlpLaunch& m, hipStream_t s,
                            bool check_only = false);

struct GateLaunch {
  const void* hidden;    // bf16 [batch][rows_stride][in_dim]
  long long batch_stride;  // elements between batches of `hidden`
  float* score;          // [batch][H][cap]
  const void* w;         // bf16 [H][in_dim]
  const float* b;        // [H] or null
  int batch, H, cap, in_dim;
  int slot_begin, slot_end;
};
hipError_t launch_score_gate(const GateLaunch& g, hipStream_t s,
                             bool check_only = false);

struct SinkGateLaunch {
  const void* hidden;      // bf16 [batch][rows_stride][in_dim]
  long long batch_stride;  // elements between batches of `hidden`
  float* score;            // [batch][H][cap]
  const void* w;           // bf16 [H*16 + H*G*16][in_dim]: W_k, then W_q
  const float* norm;       // [32] (g_k, g_q) or null
  const float* sinks;      // [n_sink][16]
  const float* b;          // [H*G] or null
  int batch, H, G, cap, in_dim, n_sink;
  int slot_begin, slot_end;
};
hipError_t launch_score_sink_gate(const SinkGateLaunch& g, hipStream_t s,
                                  bool check_only = false);

struct MlstmLaunch {
  const void* k;         // cache base (bf16)
  const void* v;
  const int32_t* pos;    // [batch][H][cap]
  float* score;          // [batch][H][cap]
  float* state;          // [batch][H][mlstm_state_floats(D)]
  const void* w;         // bf16 [H][3P+2][2D]: W_q, W_k, W_v rows, w_i, w_f
  const float* b;        // [H][2] (b_i, b_f) or null
  const float* a;        // [H][P] read-out weights
  const float* b2;       // [H] or null
  int batch, H, D, cap;
  int slot_begin, slot_end;
  int delay;             // read-out delay W
};
hipError_t launch_score_mlstm(const MlstmLaunch& m, hipStream_t s,
                              bool check_only = false);

// Prefill selection and masked prefill attention.
constexpr int kMaxPrefillLen = 262144;  // the cutoff bitmap lives in LDS
size_t prefill_ws_bytes(long long slices, int n);
hipError_t launch_prefill_select(const float* score, const float* lg, int H,
                                 int slices, int cap, int n, int S, int W,
                                 int k, void* ws, int32_t* rank, int32_t* tau,
                                 hipStream_t s);
struct PrefillAttnLaunch {
  const void* k;         // cache base (bf16), slot = position
  const void* v;
  const int32_t* rank;   // [batch][H][n]
  const int32_t* tau;    // [batch][H][n]
  const void* q;         // bf16 [batch][H*G][n][D]
  float* out;            // [batch][H*G][n][D]
  float* lse;            // [batch][H*G][n] or null
  int batch, H, G, D, cap, n, S, W;
  int gsub, nsub;        // query heads per workgroup, head subsets per KV head
  int g0;                // first query head (of G) the launch covers
  int32_t* list;         // [batch*H][query blocks][kmax] long-range keys
  int32_t* count;        // [batch*H][query blocks]
  uint32_t* vmax;        // [batch*H][query blocks] largest |v|, bf16 bits
  uint16_t* v16;         // [batch*H][n][D] V in float16
  int kmax;              // max(k, 1)
};
size_t prefill_attn_ws_bytes(long long slices, int n, int kmax, int D);
// Carves list, count, vmax and v16 out of ws (prefill_attn_ws_bytes bytes).
hipError_t launch_prefill_attn(PrefillAttnLaunch a, void* ws, hipStream_t s);
size_t mlstm_state_floats(int D);  // 0 for an unsupported head_dim

}  // namespace kve
