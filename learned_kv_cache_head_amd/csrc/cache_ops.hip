// Cache maintenance kernels: append, select (radix select of the eviction
// cut) and in-place compaction by hole filling.
//
// Retention rule (KVpop section 3, Eq. 1 and 4; Appendix C.1, Eq. 26):
// positions below S are sink tokens and the W most recent positions the
// protected window; the other entries are the eligible long-range
// candidates, of which the top ones by score are kept. Periodic eviction (ForesightKV summary,
// "Methodology in plain English"; Fast KVzip Appendix A.5) cuts a slice of
// len entries back to n_keep = B entries. Ranking uses float32 scores
// (KVpop Appendix F) with the older entry (lower position) evicted first
// among equal scores.
#include "kve_internal.h"
#include "mlp_tile.h"

namespace kve {
namespace {

// ---------------------------------------------------------------------------
// Append: one new token per (batch, KV head) slice.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void append_kernel(
    char* k, char* v, int32_t* pos, int H, int row_bytes, int cap, int slot,
    int position, const char* k_new, const char* v_new, int batch,
    const char* hidden_new, char* hidden_buf, int hidden_bytes,
    int hidden_rows, int hidden_row) {
  const int blk = blockIdx.x;
  const int slices = batch * H;
  if (blk < slices) {
    const size_t dst = ((size_t)blk * cap + slot) * row_bytes;
    const size_t src = (size_t)blk * row_bytes;
    for (int i = threadIdx.x; i < row_bytes / 16; i += 64) {
      ((u32x4*)(k + dst))[i] = ((const u32x4*)(k_new + src))[i];
      ((u32x4*)(v + dst))[i] = ((const u32x4*)(v_new + src))[i];
    }
    if (threadIdx.x == 0) pos[(size_t)blk * cap + slot] = position;
  } else {
    // Hidden state of the new token into the pending-token buffer.
    const int b = blk - slices;
    const size_t dst = ((size_t)b * hidden_rows + hidden_row) * hidden_bytes;
    const size_t src = (size_t)b * hidden_bytes;
    for (int i = threadIdx.x; i < hidden_bytes / 16; i += 64)
      ((u32x4*)(hidden_buf + dst))[i] = ((const u32x4*)(hidden_new + src))[i];
  }
}

// ---------------------------------------------------------------------------
// Select: one workgroup per slice.
//
// Candidates are the entries of the eligible set E(P) = {S <= pos <= P - W}
// with P the newest position present (KVpop Eq. 4); all other entries (sink
// tokens, recent window) are kept. Among the candidates, the r = len -
// n_keep with the smallest (key, position) are evicted; the key is the score
// or, with temporal decay, the static priority (KVpop Appendix B.3).
//  1. block max of the positions -> P;
//  2. four 8-bit MSB radix passes over the orderable 32-bit score keys of
//     the candidates -> the r-th smallest key thr, the number `need` of
//     entries with key thr to evict and the number of candidates with it;
//  3. if some but not all candidates with key thr are evicted, four radix
//     passes over their positions -> the need-th smallest such position;
//  4. an ordered pass writes the kept slots ascending (block-wide scan).
// Every output write is bounded by n_keep, so positions that break the
// contract (duplicates, missing sinks or window) cannot write out of bounds.
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / 64;
// Every pass over a slice's entries runs in sweeps of kSelV entries per
// thread (entry c = base + v * kSelThreads + tid): the index is clamped to
// len - 1, so all loads of a sweep are in bounds and unconditional and are in
// flight together, and entries past len are masked afterwards. A pass over
// 131072 entries is 16 sweeps instead of 256 dependent load round trips.
constexpr int kSelV = 16;
constexpr int kSelSweep = kSelThreads * kSelV;
// Slices of up to kSelCacheMax entries (when few enough slices run that one
// workgroup per CU fills the chip) keep every entry's ranking key in LDS,
// with kSelNoCand marking entries that are not candidates: the radix passes
// and the ordered pass then read LDS, and only the newest-position pass and
// the pass that fills the keys read HBM. kSelNoCand is the key of a NaN
// score, outside the contract.
constexpr int kSelCacheMax = 40000;  // 160,000 bytes of LDS
constexpr uint32_t kSelNoCand = 0xffffffffu;

__device__ __forceinline__ uint32_t lane_prefix(uint64_t mask) {
  // Number of set bits of `mask` in lanes below this one.
  uint32_t lo = __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u);
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), lo);
}

// One radix pass, after hist holds the pass's 256-bin histogram: the bin in
// which the cumulative count reaches `remaining` (sh[0]), the count below
// it (sh[1]) and its own count (sh[2]). Threads 0..255 (4 waves) scan.
__device__ __forceinline__ void radix_find_bin(const uint32_t* hist,
                                               uint32_t* wsum, uint32_t* sh,
                                               uint32_t remaining) {
  const int tid = threadIdx.x;
  uint32_t v = 0, incl = 0;
  if (tid < 256) {
    v = hist[tid];
    incl = v;
    const int lane = tid & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    if (lane == 63) wsum[tid >> 6] = incl;
  }
  __syncthreads();
  if (tid < 256) {
    for (int w = 0; w < (tid >> 6); ++w) incl += wsum[w];
    if (incl >= remaining && incl - v < remaining) {
      sh[0] = (uint32_t)tid;
      sh[1] = incl - v;
      sh[2] = v;
    }
  }
  __syncthreads();
}

// Radix select over 32-bit keys: the value of the `rank`-th smallest key
// (1-based) among the entries i < len with take(i), and how many of those
// keys equal it must still be taken (`rank` minus the number of smaller
// keys). `count_eq` receives how many such entries have exactly that key.
// take and key_of must be safe to call on any index below len.
template <typename KeyFn, typename TakeFn>
__device__ void radix_select(int len, uint32_t rank, KeyFn key_of,
                             TakeFn take, uint32_t* hist, uint32_t* wsum,
                             uint32_t* sh, uint32_t* key_out,
                             uint32_t* need_out, uint32_t* count_eq_out) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, mask = 0, remaining = rank, count_eq = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
    if (tid == 0) {
      sh[0] = 255u;   // defaults: last bin, nothing below (never read if
      sh[1] = 0u;     // rank <= number of entries, which the caller ensures)
      sh[2] = 0u;
    }
    __syncthreads();
    // Each thread counts a run of its entries that fall in one bin locally
    // and adds the run with one atomic when the bin changes. Scores packed
    // into a few bins (a gate's sigmoid outputs share their top key bits)
    // would otherwise send every lane of a wave to the same LDS address for
    // every entry; spread scores cost one compare more per entry.
    uint32_t run_bin = 0, run_cnt = 0;
    for (int base = 0; base < len; base += kSelSweep) {
      bool t[kSelV];
      uint32_t k[kSelV];
#pragma unroll
      for (int v = 0; v < kSelV; ++v) {
        const int c = base + v * kSelThreads + tid;
        const int cc = min(c, len - 1);
        t[v] = (c < len) & take(cc);
        k[v] = key_of(cc);
      }
#pragma unroll
      for (int v = 0; v < kSelV; ++v) {
        if (t[v] && (k[v] & mask) == prefix) {
          const uint32_t bin = (k[v] >> shift) & 255u;
          if (bin != run_bin) {
            if (run_cnt) atomicAdd(&hist[run_bin], run_cnt);
            run_bin = bin;
            run_cnt = 0;
          }
          ++run_cnt;
        }
      }
    }
    if (run_cnt) atomicAdd(&hist[run_bin], run_cnt);
    __syncthreads();
    radix_find_bin(hist, wsum, sh, remaining);
    const uint32_t digit = sh[0];
    prefix |= digit << shift;
    mask |= 255u << shift;
    remaining -= sh[1];
    count_eq = sh[2];
    __syncthreads();
  }
  *key_out = prefix;
  *need_out = remaining;
  *count_eq_out = count_eq;
}

template <bool CACHE>
__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const float* score, const int32_t* pos, const float* log_gamma,
    const float* gumbel, int H, int cap, int len, int n_keep, int S, int W,
    int32_t* keep) {
  const size_t slice = blockIdx.x;
  const float* sc = score + slice * (size_t)cap;
  const int32_t* ps = pos + slice * (size_t)cap;
  const float* gs = gumbel ? gumbel + slice * (size_t)cap : nullptr;
  int32_t* out = keep + slice * (size_t)n_keep;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  if (n_keep >= len) {  // nothing to evict: identity
    for (int i = tid; i < len; i += kSelThreads) out[i] = i;
    return;
  }
  const uint32_t r = (uint32_t)(len - n_keep);  // entries to evict

  __shared__ uint32_t hist[256];
  __shared__ uint32_t wsum[kSelWaves];
  __shared__ uint32_t sh[4];
  __shared__ int32_t sh_max[kSelWaves];
  __shared__ uint32_t kc[CACHE ? kSelCacheMax : 1];  // keys (CACHE)

  // 1. Newest position present.
  int32_t mx = INT32_MIN;
  for (int base = 0; base < len; base += kSelSweep) {
#pragma unroll
    for (int v = 0; v < kSelV; ++v)
      mx = max(mx, ps[min(base + v * kSelThreads + tid, len - 1)]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = max(mx, __shfl_xor(mx, off));
  if (lane == 0) sh_max[wave] = mx;
  __syncthreads();
  int32_t newest = sh_max[0];
#pragma unroll
  for (int w = 1; w < kSelWaves; ++w) newest = max(newest, sh_max[w]);
  const long long last_eligible = (long long)newest - W;
  auto is_cand = [&](int c) {
    const int32_t p = ps[c];
    return (p >= S) & ((long long)p <= last_eligible);
  };
  // Ranking key: the score, or under temporal decay the static priority
  // score - position * log(gamma) (KVpop Eq. 20), each operation rounded to
  // float32 separately (no fused multiply-add).
  const float lg = log_gamma ? log_gamma[slice % H] : 0.f;
  const bool decay = log_gamma != nullptr;
  auto fkey = [&](int c) {
    float r = sc[c];
    if (decay) r = decayed_priority(r, ps[c], lg);
    return r;
  };
  auto skey = [&](int c) { return score_key(fkey(c)); };
  auto pkey = [&](int c) { return (uint32_t)ps[c]; };

  // The `count` entries with take() that come first in (key, position)
  // order: cut key `thr`, and among entries with key thr those at positions
  // <= `pthr` (all of them unless the cut falls inside a tie).
  auto cut = [&](uint32_t count, auto key_of, auto take, uint32_t* thr_out,
                 uint32_t* pthr_out) {
    uint32_t thr, need, count_eq;
    radix_select(len, count, key_of, take, hist, wsum, sh, &thr, &need,
                 &count_eq);
    uint32_t pthr = 0xffffffffu;
    if (need < count_eq) {
      auto tied = [&](int c) { return take(c) & (key_of(c) == thr); };
      uint32_t pneed, pcount;
      radix_select(len, need, pkey, tied, hist, wsum, sh, &pthr, &pneed,
                   &pcount);
    }
    *thr_out = thr;
    *pthr_out = pthr;
  };
  // Non-short-circuit forms, so the loads of both operands are always made.
  auto before = [&](uint32_t k, int c, uint32_t thr, uint32_t pthr) {
    return (k < thr) | ((k == thr) & ((uint32_t)ps[c] <= pthr));
  };

  // 2-3. Deterministic: evict the r lowest candidates.
  uint32_t thr, pthr;
  // Stochastic (ForesightKV): the pool is the 2r lowest candidates; evict
  // the r pool entries with the largest float32 sum -key + noise, i.e. the
  // smallest descending key, equal sums the lower position first.
  uint32_t gthr = 0, gpthr = 0;
  auto dkey = [&](int c) { return ~score_key(noisy_key(fkey(c), gs[c])); };
  if (!gs) {
    if constexpr (CACHE) {
      for (int base = 0; base < len; base += kSelSweep) {
        uint32_t kv[kSelV];
#pragma unroll
        for (int v = 0; v < kSelV; ++v) {
          const int cc = min(base + v * kSelThreads + tid, len - 1);
          const uint32_t k = skey(cc);  // loaded whether or not a candidate
          kv[v] = is_cand(cc) ? k : kSelNoCand;
        }
#pragma unroll
        for (int v = 0; v < kSelV; ++v) {
          const int c = base + v * kSelThreads + tid;
          if (c < len) kc[c] = kv[v];
        }
      }
      __syncthreads();
      auto ckey = [&](int c) { return kc[c]; };
      auto ccand = [&](int c) { return kc[c] != kSelNoCand; };
      cut(r, ckey, ccand, &thr, &pthr);
    } else {
      cut(r, skey, is_cand, &thr, &pthr);
    }
  } else {
    __shared__ uint32_t ncand_sh;
    if (tid == 0) ncand_sh = 0;
    __syncthreads();
    uint32_t nc = 0;
    for (int base = 0; base < len; base += kSelSweep) {
#pragma unroll
      for (int v = 0; v < kSelV; ++v) {
        const int c = base + v * kSelThreads + tid;
        nc += ((c < len) & is_cand(min(c, len - 1))) ? 1u : 0u;
      }
    }
    atomicAdd(&ncand_sh, nc);
    __syncthreads();
    const uint32_t pool = min(2u * r, ncand_sh);
    cut(pool, skey, is_cand, &thr, &pthr);
    auto in_pool = [&](int c) {
      return is_cand(c) & before(skey(c), c, thr, pthr);
    };
    cut(r, dkey, in_pool, &gthr, &gpthr);
  }
  auto evicted = [&](int c) {
    if constexpr (CACHE) {
      if (!gs) {
        // Positions are read only when the cut falls inside a tie.
        const uint32_t k = kc[c];
        return (k != kSelNoCand) &
               ((k < thr) | ((k == thr) & (pthr == 0xffffffffu ||
                                            (uint32_t)ps[c] <= pthr)));
      }
    }
    const bool low = is_cand(c) & before(skey(c), c, thr, pthr);
    return gs ? (low & before(dkey(c), c, gthr, gpthr)) : low;
  };

  // 4. Kept slots, ascending. A sweep holds kSelV slabs of kSelThreads
  // consecutive slots (slab v, slot base + v * kSelThreads + tid): one
  // ballot count per wave and slab, one barrier, then every kept entry's
  // rank is the kept count of the earlier slabs, of the earlier waves of its
  // slab and of the lower lanes of its wave.
  __shared__ uint32_t cnt_sh[kSelV][kSelWaves];
  uint32_t carry = 0;
  for (int base = 0; base < len; base += kSelSweep) {
    uint64_t m[kSelV];
#pragma unroll
    for (int v = 0; v < kSelV; ++v) {
      const int c = base + v * kSelThreads + tid;
      const bool kept = (c < len) & !evicted(min(c, len - 1));
      m[v] = __builtin_amdgcn_ballot_w64(kept);
      if (lane == 0) cnt_sh[v][wave] = (uint32_t)__builtin_popcountll(m[v]);
    }
    __syncthreads();
    uint32_t before_slab = carry;
#pragma unroll
    for (int v = 0; v < kSelV; ++v) {
      uint32_t in_slab = 0, slab_total = 0;
#pragma unroll
      for (int w = 0; w < kSelWaves; ++w) {
        const uint32_t cw = cnt_sh[v][w];
        in_slab += (w < wave) ? cw : 0u;
        slab_total += cw;
      }
      const int c = base + v * kSelThreads + tid;
      const uint32_t idx = before_slab + in_slab + lane_prefix(m[v]);
      if (((m[v] >> lane) & 1ull) && idx < (uint32_t)n_keep) out[idx] = c;
      before_slab += slab_total;
    }
    carry = before_slab;
    __syncthreads();  // cnt_sh is rewritten by the next sweep
  }
}

// ---------------------------------------------------------------------------
// Select for slices of up to kSelSmallMax entries, every entry held in
// registers: thread tid owns slots v * kSelThreads + tid (v < R, the fewest
// of 3, 5 or 8 slots per thread that hold the slice). The
// score, position (and noise) of each entry are loaded once, and the radix
// passes and the ordered pass read registers only. Same rule, ties and
// outputs as select_kernel.
//
// With FUSE the kernel also compacts the slice in place (the placement rule
// of the compaction kernels: the j-th hole below n_keep receives the j-th
// kept entry at or above n_keep). The ordered pass knows the rank of every
// hole (its slot minus the kept slots before it) and of every mover (its
// kept index), so both lists go to LDS and the rows move right after it:
// the kept list never makes a round trip through memory. All score and
// position reads happen before the ordered pass, and the moves read only
// slots at or above n_keep and write only slots below it.
// ---------------------------------------------------------------------------
constexpr int kSelMaxR = 8;                          // slots per thread
constexpr int kSelSmallMax = kSelThreads * kSelMaxR;  // 4096 entries
constexpr int kFuseMaxMoves = kSelSmallMax / 2;       // holes <= min(n_keep, r)

// radix_select over the R register entries of every thread. Each pass takes
// two barriers: the histogram is double-buffered (the next pass's buffer is
// cleared while this one fills) and one wave scans the 256 bins.
template <int R>
__device__ void radix_select_regs(uint32_t rank, const uint32_t (&key)[R],
                                  const bool (&take)[R],
                                  uint32_t (*hist)[256], uint32_t (*sh)[4],
                                  uint32_t* key_out, uint32_t* need_out,
                                  uint32_t* count_eq_out) {
  const int tid = threadIdx.x;
  for (int i = tid; i < 256; i += kSelThreads) hist[0][i] = 0;
  __syncthreads();
  uint32_t prefix = 0, mask = 0, remaining = rank, count_eq = 0;
  int cur = 0;
  for (int shift = 24; shift >= 0; shift -= 8, cur ^= 1) {
#pragma unroll
    for (int v = 0; v < R; ++v)
      if (take[v] && (key[v] & mask) == prefix)
        atomicAdd(&hist[cur][(key[v] >> shift) & 255u], 1u);
    // the other buffer was last read before the previous pass's second
    // barrier
    for (int i = tid; i < 256; i += kSelThreads) hist[cur ^ 1][i] = 0;
    __syncthreads();
    if (tid < 64) {
      // lane l holds bins 4l..4l+3; an inclusive scan over the lanes
      const int l = tid;
      uint32_t c[4], t = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = hist[cur][4 * l + j];
        t += c[j];
      }
      uint32_t incl = t;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_up(incl, off);
        if (l >= off) incl += o;
      }
      if (l == 0) {  // default: the last bin (rank beyond the entries)
        sh[cur][0] = 255u;
        sh[cur][1] = 0u;
        sh[cur][2] = 0u;
      }
      uint32_t run = incl - t;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t below = run;
        run += c[j];
        if (run >= remaining && below < remaining) {
          sh[cur][0] = (uint32_t)(4 * l + j);
          sh[cur][1] = below;
          sh[cur][2] = c[j];
        }
      }
    }
    __syncthreads();
    prefix |= sh[cur][0] << shift;
    mask |= 255u << shift;
    remaining -= sh[cur][1];
    count_eq = sh[cur][2];
  }
  *key_out = prefix;
  *need_out = remaining;
  *count_eq_out = count_eq;
}

// LDS of the register-resident select.
template <int R>
struct SelRegsLds {
  uint32_t hist[2][256];
  uint32_t sh[2][4];
  int32_t sh_max[kSelWaves];
  uint32_t ncand;
  uint32_t nholes;
  uint32_t cnt[R][kSelWaves];
};

// Loads the R entries of this thread (slot v * kSelThreads + tid):
// position, score and noise; clamped indices keep every load in bounds and
// all of them in flight together, entries past len are masked by valid.
template <int R>
__device__ __forceinline__ void select_load_regs(
    const float* sc, const int32_t* ps, const float* gs, int len,
    int32_t (&p)[R], float (&s)[R], float (&g)[R],
    bool (&valid)[R]) {
#pragma unroll
  for (int v = 0; v < R; ++v) {
    const int c = v * kSelThreads + (int)threadIdx.x;
    const int cc = min(c, len - 1);
    valid[v] = c < len;
    p[v] = ps[cc];
    s[v] = sc[cc];
    g[v] = gs ? gs[cc] : 0.f;
  }
}

// The select rule on the register entries (select_kernel's rule): which
// entries are evicted when r of them must go. lg is the KV head's log decay
// (decay: the ranking key is the static priority), g the noise (gumbel: the
// stochastic rule). L.nholes is cleared here for the ordered pass.
template <int R>
__device__ void select_rule_regs(SelRegsLds<R>& L, const int32_t (&p)[R],
                                 const float (&s)[R],
                                 const float (&g)[R],
                                 const bool (&valid)[R], bool decay,
                                 float lg, bool gumbel, int S, int W,
                                 uint32_t r, bool (&evicted)[R]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // Newest position present (clamped copies repeat a present entry).
  int32_t mx = p[0];
#pragma unroll
  for (int v = 1; v < R; ++v) mx = max(mx, p[v]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = max(mx, __shfl_xor(mx, off));
  if (lane == 0) L.sh_max[wave] = mx;
  if (tid == 0) {
    L.ncand = 0;
    L.nholes = 0;
  }
  __syncthreads();
  int32_t newest = L.sh_max[0];
#pragma unroll
  for (int w = 1; w < kSelWaves; ++w) newest = max(newest, L.sh_max[w]);
  const long long last_eligible = (long long)newest - W;
  bool cand[R];
  uint32_t key[R], pk[R];
  float fk[R];
#pragma unroll
  for (int v = 0; v < R; ++v) {
    cand[v] = valid[v] & (p[v] >= S) & ((long long)p[v] <= last_eligible);
    // static priority under decay: two separately rounded operations
    fk[v] = decay ? decayed_priority(s[v], p[v], lg) : s[v];
    key[v] = score_key(fk[v]);
    pk[v] = (uint32_t)p[v];
  }
  // The `count` first entries with take[] in (key, position) order: cut key
  // thr and, among entries with key thr, those at positions <= pthr.
  auto cut = [&](uint32_t count, const uint32_t (&kk)[R],
                 const bool (&take)[R], uint32_t* thr_out,
                 uint32_t* pthr_out) {
    uint32_t thr, need, count_eq;
    radix_select_regs<R>(count, kk, take, L.hist, L.sh, &thr, &need,
                         &count_eq);
    uint32_t pthr = 0xffffffffu;
    if (need < count_eq) {
      bool tied[R];
#pragma unroll
      for (int v = 0; v < R; ++v) tied[v] = take[v] & (kk[v] == thr);
      uint32_t pneed, pcount;
      radix_select_regs<R>(need, pk, tied, L.hist, L.sh, &pthr, &pneed,
                           &pcount);
    }
    *thr_out = thr;
    *pthr_out = pthr;
  };
  auto before = [&](uint32_t k, int v, uint32_t thr, uint32_t pthr) {
    return (k < thr) | ((k == thr) & (pk[v] <= pthr));
  };
  uint32_t thr, pthr;
  if (!gumbel) {
    cut(r, key, cand, &thr, &pthr);
#pragma unroll
    for (int v = 0; v < R; ++v)
      evicted[v] = cand[v] & before(key[v], v, thr, pthr);
    return;
  }
  // ForesightKV: pool = the 2r lowest candidates; evict the r pool entries
  // with the smallest descending key of -key + noise.
  uint32_t nc = 0;
#pragma unroll
  for (int v = 0; v < R; ++v) nc += cand[v] ? 1u : 0u;
  atomicAdd(&L.ncand, nc);
  __syncthreads();
  const uint32_t pool = min(2u * r, L.ncand);
  cut(pool, key, cand, &thr, &pthr);
  bool in_pool[R];
  uint32_t dk[R];
#pragma unroll
  for (int v = 0; v < R; ++v) {
    in_pool[v] = cand[v] & before(key[v], v, thr, pthr);
    dk[v] = ~score_key(noisy_key(fk[v], g[v]));
  }
  uint32_t gthr, gpthr;
  cut(r, dk, in_pool, &gthr, &gpthr);
#pragma unroll
  for (int v = 0; v < R; ++v)
    evicted[v] = in_pool[v] & before(dk[v], v, gthr, gpthr);
}

// Ordered pass: kept slots, ascending, into out[0, n_keep). Slab v holds
// slots v * kSelThreads + tid: one ballot count per wave and slab, one
// barrier; a slot's kept rank is the kept count of the earlier slabs,
// earlier waves and lower lanes. on_slot(c, kept, idx) sees every valid
// slot with idx the number of kept slots before it.
template <int R, typename OnSlot>
__device__ __forceinline__ void select_ordered_regs(
    SelRegsLds<R>& L, const bool (&valid)[R], const bool (&evicted)[R],
    int n_keep, int32_t* out, OnSlot on_slot) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  uint64_t m[R];
#pragma unroll
  for (int v = 0; v < R; ++v) {
    const bool kept = valid[v] & !evicted[v];
    m[v] = __builtin_amdgcn_ballot_w64(kept);
    if (lane == 0) L.cnt[v][wave] = (uint32_t)__builtin_popcountll(m[v]);
  }
  __syncthreads();
  uint32_t before_slab = 0;
#pragma unroll
  for (int v = 0; v < R; ++v) {
    uint32_t in_slab = 0, slab_total = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
      const uint32_t cw = L.cnt[v][w];
      in_slab += (w < wave) ? cw : 0u;
      slab_total += cw;
    }
    const int c = v * kSelThreads + tid;
    const uint32_t idx = before_slab + in_slab + lane_prefix(m[v]);
    const bool kept = (m[v] >> lane) & 1ull;
    if (kept && idx < (uint32_t)n_keep) out[idx] = c;
    if (valid[v]) on_slot(c, kept, idx);
    before_slab += slab_total;
  }
}

template <bool FUSE, int R>
__global__ __launch_bounds__(kSelThreads) void select_small_kernel(
    float* score, int32_t* pos, const float* log_gamma, const float* gumbel,
    int H, int cap, int len, int n_keep, int S, int W, int32_t* keep,
    char* kc_, char* vc_, int row_bytes) {
  const size_t slice = blockIdx.x;
  float* sc = score + slice * (size_t)cap;
  int32_t* ps = pos + slice * (size_t)cap;
  const float* gs = gumbel ? gumbel + slice * (size_t)cap : nullptr;
  int32_t* out = keep + slice * (size_t)n_keep;
  const int tid = threadIdx.x;

  if (n_keep >= len) {  // nothing to evict: identity, nothing moves
    for (int i = tid; i < len; i += kSelThreads) out[i] = i;
    return;
  }
  const uint32_t r = (uint32_t)(len - n_keep);
  __shared__ SelRegsLds<R> L;
  __shared__ int32_t holes_sh[FUSE ? kFuseMaxMoves : 1];
  __shared__ int32_t movers_sh[FUSE ? kFuseMaxMoves : 1];

  int32_t p[R];
  float s[R], g[R];
  bool valid[R], evicted[R];
  select_load_regs(sc, ps, gs, len, p, s, g, valid);
  const float lg = log_gamma ? log_gamma[slice % H] : 0.f;
  select_rule_regs(L, p, s, g, valid, log_gamma != nullptr, lg, gs != nullptr,
                   S, W, r, evicted);

  const int M = min(n_keep, (int)r);  // moves, at most
  if (FUSE) {
    for (int i = tid; i < M; i += kSelThreads) {
      holes_sh[i] = -1;
      movers_sh[i] = -1;
    }
  }
  // idx counts the kept slots before c. A hole below n_keep has hole rank
  // c - idx; a kept slot at or above n_keep has kept rank idx, and the kept
  // ranks of the movers are the last ones below n_keep.
  select_ordered_regs(L, valid, evicted, n_keep, out,
                      [&](int c, bool kept, uint32_t idx) {
    if (!FUSE) return;
    if (!kept && c < n_keep) {
      const int j = c - (int)idx;
      if (j < M) holes_sh[j] = c;
      atomicAdd(&L.nholes, 1u);
    } else if (kept && c >= n_keep && idx < (uint32_t)n_keep) {
      const int j = (int)idx - (n_keep - M);
      if (j >= 0) movers_sh[j] = c;
    }
  });
  if (!FUSE) return;
  __syncthreads();

  // Moves: hole j <- mover M - nh + j (the movers' kept ranks run from
  // n_keep - nh to n_keep - 1). A slice that breaks the contract (repeated
  // positions) can leave an entry unset: its row is skipped, never written.
  const int nh = min((int)L.nholes, M);
  const int cpr = row_bytes >> 4;  // 16-byte chunks per K (or V) row
  const int items = nh * 2 * cpr;  // K and V chunks of every moved row
  const size_t base = slice * (size_t)cap;
  constexpr int RB = 8;            // chunks in flight per thread
  for (int i0 = tid; i0 < items; i0 += RB * kSelThreads) {
    u32x4 buf[RB];
    int dst[RB];
    size_t doff[RB];
    bool isv[RB];
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const int it = i0 + u * kSelThreads;
      dst[u] = -1;
      if (it < items) {
        const int j = it / (2 * cpr);
        const int q = it % (2 * cpr);
        const int d = holes_sh[j];
        const int src = movers_sh[M - nh + j];
        if (d >= 0 && d < n_keep && src >= n_keep && src < cap) {
          isv[u] = q >= cpr;
          const size_t qo = (size_t)(q % cpr) * 16;
          const char* from = (isv[u] ? vc_ : kc_) +
                             (base + src) * (size_t)row_bytes + qo;
          buf[u] = *(const u32x4*)from;
          dst[u] = d;
          doff[u] = (base + d) * (size_t)row_bytes + qo;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < RB; ++u)
      if (dst[u] >= 0) *(u32x4*)((isv[u] ? vc_ : kc_) + doff[u]) = buf[u];
  }
  for (int j = tid; j < nh; j += kSelThreads) {
    const int d = holes_sh[j];
    const int src = movers_sh[M - nh + j];
    if (d >= 0 && d < n_keep && src >= n_keep && src < cap) {
      sc[d] = sc[src];
      ps[d] = ps[src];
    }
  }
}

// ---------------------------------------------------------------------------
// The evicting step of a bf16 MLP-scored slice in one launch: score the
// pending rows, select, compact. The pending rows (the slots the last
// scoring left unscored, L of them at a periodic eviction) are the newest
// entries; when they start at or above n_keep they include every kept entry
// at or above n_keep, i.e. every row compaction moves. Each wave loads its
// 16-row tiles of them once, in the MFMA operand layout (a lane holds
// 16-byte chunks of one row), scores them with the scorer's own tile
// arithmetic (the same bits as the scorer kernel), and after the select
// stores the same registers into the holes: the moved rows are read from
// memory once instead of three times (scorer, compaction read) and the kept
// list never leaves the chip. The step's new token can be appended here as
// well (its lanes read it from k_new / v_new and store it to its slot).
// Results equal kve_append + kve_score + kve_select_evict + kve_compact.
// ---------------------------------------------------------------------------
struct EvictMlpLaunch {
  void* k;
  void* v;
  float* score;
  int32_t* pos;
  const void* w1;        // bf16 [H][hidden][2D]
  const float* b1;       // [H][hidden] or null
  const float* w2;       // [H][hidden]
  const float* b2;       // [H] or null
  int act;
  const float* log_gamma;
  const float* gumbel;
  int H, cap, len, n_keep, S, W;
  int pend0;             // pending rows: slots [pend0, len)
  int32_t* keep;
  // The step's new token, appended here at slot len - 1 (its K, V row and
  // position) instead of by a launch of its own; k_new null: already there.
  const void* k_new;     // [batch][H][D]
  const void* v_new;
  int new_pos;
};

// Three workgroups per CU (6 waves per SIMD, 80 VGPRs) run all 768 slices
// of a batch-96 layer in one round. That bound holds without scratch for the
// 3-slot form up to 64 hidden units at d = 128 and 96 at d = 64; wider
// hidden layers take 4 waves per SIMD (128 VGPRs), and 128 hidden units at
// d = 128 and the 8-slot form no bound (the compiler's choice spills nothing).
constexpr int evict_waves(int D, int NB, int R) {
  if (R > 3 || (D == 128 && NB >= 8)) return 1;
  return ((D == 128 && NB <= 4) || (D == 64 && NB <= 6)) ? 6 : 4;
}

template <int D, int NB, int TPW, int R>
__global__ __launch_bounds__(kSelThreads)
__attribute__((amdgpu_waves_per_eu(evict_waves(D, NB, R))))
void evict_mlp_kernel(
    EvictMlpLaunch a) {
  constexpr int HID = NB * 16;
  constexpr int IN = 2 * D;
  constexpr int KSTEPS = IN / 32;
  constexpr int KHALF = D / 32;
  constexpr int LSTR = IN + 8;      // bf16 per staged W1 row
  constexpr int PMAX = kSelWaves * TPW * 16;
  __shared__ uint16_t w1s[HID * LSTR];
  __shared__ float nsc[PMAX];       // scores of the pending rows
  __shared__ int32_t krank[PMAX];   // kept rank of a kept pending row >= n_keep
  __shared__ int32_t holes_sh[PMAX];
  __shared__ SelRegsLds<R> L;

  const size_t slice = blockIdx.x;
  const int h = (int)(slice % a.H);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const size_t base = slice * (size_t)a.cap;
  const int P = a.len - a.pend0;    // pending rows, 1..PMAX
  uint16_t* kc = (uint16_t*)a.k + base * D;
  uint16_t* vc = (uint16_t*)a.v + base * D;
  float* sc = a.score + base;
  int32_t* ps = a.pos + base;
  const int kq = (lane >> 4) * 8;

  // Pending rows, tile t of this wave: rows (t * kSelWaves + wave) * 16 +
  // lane % 16 of the pending range (clamped: computed, never stored). The
  // new token's row comes from k_new / v_new when it is appended here.
  const int last = a.len - 1;
  const bool app = a.k_new != nullptr;
  const uint16_t* kn = app ? (const uint16_t*)a.k_new + slice * D : nullptr;
  const uint16_t* vn = app ? (const uint16_t*)a.v_new + slice * D : nullptr;
  bf16x8_t rows[TPW][KSTEPS];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    int ri = (t * kSelWaves + wave) * 16 + (lane & 15);
    ri = ri < P ? ri : P - 1;
    const size_t slot = (size_t)(a.pend0 + ri);
    const bool nw = app && (int)slot == last;
    mlp_load_row<D>(rows[t], nw ? kn : kc + slot * D, nw ? vn : vc + slot * D,
                    kq);
  }
  mlp_stage_w1<HID, IN>(w1s, LSTR, (const uint16_t*)a.w1 + (size_t)h * HID * IN,
                        kSelThreads);
  for (int i = tid; i < PMAX; i += kSelThreads) {
    krank[i] = -1;
    holes_sh[i] = -1;
  }
  float bias[NB], w2v[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = nb * 16 + (lane & 15);
    bias[nb] = a.b1 ? a.b1[(size_t)h * HID + n] : 0.f;
    w2v[nb] = a.w2[(size_t)h * HID + n];
  }
  const float b2 = a.b2 ? a.b2[h] : 0.f;
  __syncthreads();

  // Scores of the pending rows, to the cache and to LDS.
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    float o[4];
    mlp_tile_scores<D, NB>(rows[t], w1s, LSTR, bias, w2v, b2, a.act, o);
    if ((lane & 15) == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ri = (t * kSelWaves + wave) * 16 + 4 * (lane >> 4) + i;
        if (ri < P) {
          nsc[ri] = o[i];
          sc[a.pend0 + ri] = o[i];
        }
      }
    }
  }
  // The select's registers are loaded only now: live across the MFMA tiles
  // they pushed the 6-waves-per-SIMD form past its 80 VGPRs into scratch.
  // Their loads are in flight during the barrier; the pending slots' scores
  // come from LDS below, so the stores above need not be visible to them.
  int32_t p[R];
  float s[R], g[R];
  bool valid[R], evicted[R];
  select_load_regs(sc, ps, a.gumbel ? a.gumbel + base : nullptr, a.len, p, s,
                   g, valid);
  if (app) {
#pragma unroll
    for (int v = 0; v < R; ++v)
      if (v * kSelThreads + tid == last) p[v] = a.new_pos;
  }
  __syncthreads();
#pragma unroll
  for (int v = 0; v < R; ++v) {
    const int c = v * kSelThreads + tid;
    if (valid[v] && c >= a.pend0) s[v] = nsc[c - a.pend0];
  }

  const uint32_t r = (uint32_t)(a.len - a.n_keep);
  const float lg = a.log_gamma ? a.log_gamma[h] : 0.f;
  select_rule_regs(L, p, s, g, valid, a.log_gamma != nullptr, lg,
                   a.gumbel != nullptr, a.S, a.W, r, evicted);
  int32_t* out = a.keep + slice * (size_t)a.n_keep;
  const int n_keep = a.n_keep;
  select_ordered_regs(L, valid, evicted, n_keep, out,
                      [&](int c, bool kept, uint32_t idx) {
    if (!kept && c < n_keep) {
      const int j = c - (int)idx;  // hole rank
      if (j < PMAX) holes_sh[j] = c;
      atomicAdd(&L.nholes, 1u);
    } else if (kept && c >= n_keep && idx < (uint32_t)n_keep) {
      krank[c - a.pend0] = (int)idx;  // c >= n_keep >= pend0
    }
  });
  __syncthreads();

  // Moves from registers: pending row ri with kept rank idx >= n_keep - nh
  // is mover idx - (n_keep - nh) and fills that hole (the holes and the
  // movers each rank 0..nh-1 in slot order). The appended row is also
  // stored to its own slot, as the append would have left it.
  const int nh = (int)L.nholes;
  auto store_row = [&](const bf16x8_t (&row)[KSTEPS], int d) {
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      uint16_t* to = ks < KHALF ? kc + (size_t)d * D + ks * 32 + kq
                                : vc + (size_t)d * D + (ks - KHALF) * 32 + kq;
      *(u32x4*)to = __builtin_bit_cast(u32x4, row[ks]);
    }
  };
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int ri = (t * kSelWaves + wave) * 16 + (lane & 15);
    const int kr = ri < P ? krank[ri] : -1;
    const int j = kr - (n_keep - nh);
    const int d = (kr >= 0 && j >= 0 && j < nh && j < PMAX) ? holes_sh[j] : -1;
    const bool nw = app && ri < P && a.pend0 + ri == last;
    const int32_t src_pos = nw ? a.new_pos : (ri < P ? ps[a.pend0 + ri] : 0);
    if (d >= 0 && d < n_keep) {
      store_row(rows[t], d);
      if ((lane >> 4) == 0) {
        sc[d] = nsc[ri];
        ps[d] = src_pos;
      }
    }
    if (nw) {
      store_row(rows[t], last);
      if ((lane >> 4) == 0) ps[last] = a.new_pos;
    }
  }
}

// ---------------------------------------------------------------------------
// Compact in place by filling holes (KVpop Appendix C: the decode cache
// holds only retained entries): keep[0..n_keep) lists the kept slots
// ascending. Kept entries below n_keep stay where they are; the j-th slot
// below n_keep that was not kept (a hole, ascending) receives the j-th kept
// entry at or above n_keep (ascending). Sources lie at or above n_keep and
// destinations below it, so no copy can overwrite an unread source, and all
// copies run in parallel.
//
// With i0 kept slots below n_keep, the number of holes before keep[i]
// (i < i0) is c(i) = keep[i] - i, non-decreasing, and c(i0) = n_keep - i0 =
// the number of holes. Hole j lies in the gap before the first i with
// c(i) > j, at slot j + i.
//
// Grid: (slice, group of kCompRows moved rows); 8 threads per row copy its
// K and V bytes with 16-byte accesses.
// ---------------------------------------------------------------------------
constexpr int kCompThreads = 256;
constexpr int kCompRows = kCompThreads / 8;  // rows per workgroup

__global__ __launch_bounds__(kCompThreads) void compact_kernel(
    char* k, char* v, float* score, int32_t* pos, int cap, int row_bytes,
    const int32_t* keep, int n_keep) {
  const size_t slice = blockIdx.x;
  const int32_t* kp = keep + slice * (size_t)n_keep;
  const int tid = threadIdx.x;
  __shared__ int sh_i0;
  __shared__ int dst_sh[kCompRows], src_sh[kCompRows];
  if (tid == 0) {
    int lo = 0, hi = n_keep;  // first i with keep[i] >= n_keep
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (kp[mid] < n_keep) lo = mid + 1; else hi = mid;
    }
    sh_i0 = lo;
  }
  __syncthreads();
  const int i0 = sh_i0;
  const int holes = n_keep - i0;
  const int j0 = blockIdx.y * kCompRows;
  if (j0 >= holes) return;  // uniform: no barrier below for this group
  if (tid < kCompRows) {
    const int j = j0 + tid;
    int d = -1, src = -1;
    if (j < holes) {
      int lo = 0, hi = i0;  // first i in [0, i0] with c(i) > j
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (kp[mid] - mid > j) hi = mid; else lo = mid + 1;
      }
      d = j + lo;
      src = kp[i0 + j];
    }
    dst_sh[tid] = d;
    src_sh[tid] = src;
  }
  __syncthreads();
  const int row = tid >> 3;
  const int sub = tid & 7;
  const int d = dst_sh[row];
  const int src = src_sh[row];
  if (d < 0) return;
  const size_t base = slice * (size_t)cap;
  const size_t drow = (base + d) * (size_t)row_bytes;
  const size_t srow = (base + src) * (size_t)row_bytes;
  for (int c = sub * 16; c < row_bytes; c += 128) {
    *(u32x4*)(k + drow + c) = *(const u32x4*)(k + srow + c);
    *(u32x4*)(v + drow + c) = *(const u32x4*)(v + srow + c);
  }
  if (sub == 0) {
    score[base + d] = score[base + src];
    pos[base + d] = pos[base + src];
  }
}

// Slices with n_keep <= kCompSmallKeep: a workgroup handles holes
// [blockIdx.y * hpw, +hpw) of one slice. The kept list goes to LDS with
// coalesced loads, the kept slots below n_keep become a bitmap, and the
// holes are the bitmap's zero bits in ascending order (word popcounts and
// one prefix scan), so no thread runs a dependent search through global
// memory. The same placement rule as compact_kernel: the j-th hole below
// n_keep receives keep[i0 + j].
constexpr int kCompSmallKeep = 4096;
constexpr int kCompSmallWords = kCompSmallKeep / 32;

__global__ __launch_bounds__(kCompThreads) void compact_small_kernel(
    char* k, char* v, float* score, int32_t* pos, int cap, int row_bytes,
    const int32_t* keep, int n_keep, int hpw) {
  const size_t slice = blockIdx.x;
  const int32_t* kp = keep + slice * (size_t)n_keep;
  const int tid = threadIdx.x;
  __shared__ int32_t ks[kCompSmallKeep];        // kept slots, then sources
  __shared__ uint32_t bits[kCompSmallWords];    // kept slots below n_keep
  __shared__ uint32_t zpre[kCompSmallWords];    // holes before each word
  __shared__ int32_t dst[kCompSmallKeep];       // hole j_begin + i -> slot
  __shared__ int i0_sh;
  for (int w = tid; w < kCompSmallWords; w += kCompThreads) bits[w] = 0u;
  if (tid == 0) i0_sh = n_keep;
  __syncthreads();
  // Kept list into LDS; i0 = first index whose slot is >= n_keep (the list
  // ascends); kept slots below n_keep set their bits.
  for (int i = tid; i < n_keep; i += kCompThreads) {
    const int32_t sl = kp[i];
    ks[i] = sl;
    if (sl < n_keep) {
      atomicOr(&bits[sl >> 5], 1u << (sl & 31));
    } else if (i == 0 || kp[i - 1] < n_keep) {
      i0_sh = i;  // the one index where the list crosses n_keep
    }
  }
  __syncthreads();
  const int i0 = i0_sh;
  const int j_begin = blockIdx.y * hpw;
  const int j_end = min(n_keep - i0, j_begin + hpw);  // holes: n_keep - i0
  if (j_begin >= j_end) return;  // uniform
  const int nwords = (n_keep + 31) >> 5;
  // Exclusive prefix of the words' zero counts (bits past n_keep excluded),
  // by the first wave.
  if (tid < 64) {
    uint32_t carry = 0;
    for (int w0 = 0; w0 < nwords; w0 += 64) {
      const int w = w0 + tid;
      uint32_t z = 0;
      if (w < nwords) {
        const int valid = min(32, n_keep - (w << 5));
        const uint32_t vmask = valid == 32 ? 0xffffffffu : ((1u << valid) - 1u);
        z = (uint32_t)__builtin_popcount(~bits[w] & vmask);
      }
      uint32_t incl = z;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_up(incl, off);
        if (tid >= off) incl += o;
      }
      if (w < nwords) zpre[w] = carry + incl - z;
      carry += __shfl(incl, 63);
    }
  }
  __syncthreads();
  // Hole j: the word holding zero number j (binary search over zpre in
  // LDS), then that zero bit within the word.
  for (int j = j_begin + tid; j < j_end; j += kCompThreads) {
    int lo = 0, hi = nwords - 1;  // last word with zpre <= j
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int)zpre[mid] <= j) lo = mid; else hi = mid - 1;
    }
    uint32_t zeros = ~bits[lo];
    for (int r = j - (int)zpre[lo]; r > 0; --r) zeros &= zeros - 1u;
    // A kept list that breaks the contract (not ascending, repeated slots)
    // can leave no such zero: the hole is then skipped, never written.
    dst[j - j_begin] = zeros ? (lo << 5) + __builtin_ctz(zeros) : -1;
  }
  __syncthreads();
  // Copies: 8 lanes per row, 16-byte accesses, RB rows per thread loaded
  // before any of them is stored (sources lie at or above
  // n_keep and destinations below it, so no load reads a row stored here).
  constexpr int RB = 4;                  // rows in flight per thread
  constexpr int NC = 4;                  // 128-byte chunks per row, at most
  const int nc = row_bytes >> 7;         // 1..4
  const int sub = tid & 7;
  const size_t base = slice * (size_t)cap;
  for (int j0 = j_begin + (tid >> 3); j0 < j_end;
       j0 += RB * (kCompThreads / 8)) {
    u32x4 kb[RB][NC], vb[RB][NC];
    float sv[RB];
    int32_t pv[RB];
    int dr[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int j = j0 + r * (kCompThreads / 8);
      int d = -1, src = 0;
      if (j < j_end) {
        d = dst[j - j_begin];
        src = ks[i0 + j];
        if (src < n_keep || src >= cap) d = -1;
      }
      dr[r] = d;
      if (d >= 0) {
        const size_t srow = (base + src) * (size_t)row_bytes + sub * 16;
#pragma unroll
        for (int c = 0; c < NC; ++c)
          if (c < nc) {
            kb[r][c] = *(const u32x4*)(k + srow + c * 128);
            vb[r][c] = *(const u32x4*)(v + srow + c * 128);
          }
        sv[r] = score[base + src];
        pv[r] = pos[base + src];
      }
    }
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int d = dr[r];
      if (d < 0) continue;
      const size_t drow = (base + d) * (size_t)row_bytes + sub * 16;
#pragma unroll
      for (int c = 0; c < NC; ++c)
        if (c < nc) {
          *(u32x4*)(k + drow + c * 128) = kb[r][c];
          *(u32x4*)(v + drow + c * 128) = vb[r][c];
        }
      if (sub == 0) {
        score[base + d] = sv[r];
        pos[base + d] = pv[r];
      }
    }
  }
}

}  // namespace

hipError_t launch_append(void* k, void* v, int32_t* pos, int batch, int H,
                         int D, int cap, int elem_bytes, int slot,
                         int position, const void* k_new, const void* v_new,
                         const void* hidden_new, void* hidden_buf,
                         int hidden_dim, int hidden_rows, int hidden_row,
                         hipStream_t s, bool check_only) {
  const int slices = batch * H;
  const int extra = hidden_new ? batch : 0;
  if (check_only) return hipSuccess;
  hipLaunchKernelGGL(append_kernel, dim3(slices + extra), dim3(64), 0, s,
                     (char*)k, (char*)v, pos, H, D * elem_bytes, cap, slot,
                     position, (const char*)k_new, (const char*)v_new, batch,
                     (const char*)hidden_new, (char*)hidden_buf,
                     hidden_dim * 2, hidden_rows, hidden_row);
  return hipGetLastError();
}

hipError_t launch_select(const float* score, const int32_t* pos,
                         const float* log_gamma, const float* gumbel, int H,
                         int slices, int cap, int len, int n_keep, int S,
                         int W, int32_t* keep, hipStream_t s,
                         bool check_only) {
  // The key cache takes all of a CU's LDS: used when few slices run.
  const bool cache = !gumbel && len > 2048 && len <= kSelCacheMax &&
                     slices <= 256;
  if (check_only) return hipSuccess;
  if (len <= kSelSmallMax) {
    float* sc = const_cast<float*>(score);
    int32_t* ps = const_cast<int32_t*>(pos);
#define KVE_SEL(RR)                                                          \
    hipLaunchKernelGGL((select_small_kernel<false, RR>), dim3(slices),       \
                       dim3(kSelThreads), 0, s, sc, ps, log_gamma, gumbel, H, \
                       cap, len, n_keep, S, W, keep, nullptr, nullptr, 0)
    if (len <= 3 * kSelThreads) KVE_SEL(3);
    else if (len <= 5 * kSelThreads) KVE_SEL(5);
    else KVE_SEL(kSelMaxR);
#undef KVE_SEL
    return hipGetLastError();
  }
  if (cache)
    hipLaunchKernelGGL(select_kernel<true>, dim3(slices), dim3(kSelThreads), 0,
                       s, score, pos, log_gamma, gumbel, H, cap, len, n_keep,
                       S, W, keep);
  else
    hipLaunchKernelGGL(select_kernel<false>, dim3(slices), dim3(kSelThreads),
                       0, s, score, pos, log_gamma, gumbel, H, cap, len,
                       n_keep, S, W, keep);
  return hipGetLastError();
}

hipError_t launch_compact(void* k, void* v, float* score, int32_t* pos,
                          int slices, int cap, int row_bytes, int len,
                          const int32_t* keep, int n_keep, hipStream_t s,
                          bool check_only) {
  if (row_bytes % 128 != 0) return hipErrorInvalidValue;
  // Moved rows per slice: at most the slots at or above n_keep, and at most
  // the holes below it.
  const int max_moves = n_keep < len - n_keep ? n_keep : len - n_keep;
  if (max_moves <= 0) return hipSuccess;
  if (n_keep <= kCompSmallKeep) {
    // About 1024 workgroups in all, at least 32 holes each.
    int groups = (1024 + slices - 1) / slices;
    const int by_rows = (max_moves + 31) / 32;
    if (groups > by_rows) groups = by_rows;
    if (groups < 1) groups = 1;
    const int hpw = (max_moves + groups - 1) / groups;
    if (check_only) return hipSuccess;
    hipLaunchKernelGGL(compact_small_kernel, dim3(slices, groups),
                       dim3(kCompThreads), 0, s, (char*)k, (char*)v, score, pos,
                       cap, row_bytes, keep, n_keep, hpw);
    return hipGetLastError();
  }
  const int groups = (max_moves + kCompRows - 1) / kCompRows;
  if (groups > 65535) return hipErrorInvalidValue;
  if (check_only) return hipSuccess;
  hipLaunchKernelGGL(compact_kernel, dim3(slices, groups), dim3(kCompThreads),
                     0, s, (char*)k, (char*)v, score, pos, cap, row_bytes,
                     keep, n_keep);
  return hipGetLastError();
}

bool evict_mlp_fits(int D, int hidden, int len, int n_keep, int pend0) {
  return (D == 64 || D == 128) && hidden >= 16 && hidden <= 128 &&
         hidden % 16 == 0 && len <= kSelSmallMax && n_keep < len &&
         pend0 <= n_keep && len - pend0 >= 1 &&
         len - pend0 <= kSelWaves * 16;  // one 16-row tile per wave
}

hipError_t launch_evict_mlp(const EvictMlpLaunchArgs& e, hipStream_t s,
                            bool check_only) {
  if (!evict_mlp_fits(e.D, e.hidden, e.len, e.n_keep, e.pend0))
    return hipErrorInvalidValue;
  if (check_only) return hipSuccess;
  EvictMlpLaunch a{};
  a.k = e.k;
  a.v = e.v;
  a.score = e.score;
  a.pos = e.pos;
  a.w1 = e.w1;
  a.b1 = e.b1;
  a.w2 = e.w2;
  a.b2 = e.b2;
  a.act = e.act;
  a.log_gamma = e.log_gamma;
  a.gumbel = e.gumbel;
  a.H = e.H;
  a.cap = e.cap;
  a.len = e.len;
  a.n_keep = e.n_keep;
  a.S = e.S;
  a.W = e.W;
  a.pend0 = e.pend0;
  a.keep = e.keep;
  a.k_new = e.k_new;
  a.v_new = e.v_new;
  a.new_pos = e.new_pos;
  const dim3 grid((unsigned)e.slices), block(kSelThreads);
  const bool r3 = e.len <= 3 * kSelThreads;  // register slots per thread
#define KVE_EVICT(DD, NBB)                                                  \
  if (e.D == DD && e.hidden == NBB * 16) {                                  \
    if (r3)                                                                 \
      hipLaunchKernelGGL((evict_mlp_kernel<DD, NBB, 1, 3>), grid, block, 0, \
                         s, a);                                             \
    else                                                                    \
      hipLaunchKernelGGL((evict_mlp_kernel<DD, NBB, 1, kSelMaxR>), grid,    \
                         block, 0, s, a);                                   \
    return hipGetLastError();                                               \
  }
  KVE_EVICT(128, 1) KVE_EVICT(128, 2) KVE_EVICT(128, 3) KVE_EVICT(128, 4)
  KVE_EVICT(128, 5) KVE_EVICT(128, 6) KVE_EVICT(128, 7) KVE_EVICT(128, 8)
  KVE_EVICT(64, 1) KVE_EVICT(64, 2) KVE_EVICT(64, 3) KVE_EVICT(64, 4)
  KVE_EVICT(64, 5) KVE_EVICT(64, 6) KVE_EVICT(64, 7) KVE_EVICT(64, 8)
#undef KVE_EVICT
  return hipErrorInvalidValue;
}

hipError_t launch_select_compact(void* k, void* v, float* score, int32_t* pos,
                                 const float* log_gamma, const float* gumbel,
                                 int H, int slices, int cap, int row_bytes,
                                 int len, int n_keep, int S, int W,
                                 int32_t* keep, hipStream_t s,
                                 bool check_only) {
  const int moves = n_keep < len - n_keep ? n_keep : len - n_keep;
  const bool fused = len <= kSelSmallMax && moves <= kFuseMaxMoves &&
                     row_bytes % 16 == 0;
  if (!fused) {
    hipError_t e = launch_select(score, pos, log_gamma, gumbel, H, slices, cap,
                                 len, n_keep, S, W, keep, s, check_only);
    if (e != hipSuccess) return e;
    return launch_compact(k, v, score, pos, slices, cap, row_bytes, len, keep,
                          n_keep, s, check_only);
  }
  if (check_only) return hipSuccess;
#define KVE_SEL(RR)                                                          \
  hipLaunchKernelGGL((select_small_kernel<true, RR>), dim3(slices),          \
                     dim3(kSelThreads), 0, s, score, pos, log_gamma, gumbel,  \
                     H, cap, len, n_keep, S, W, keep, (char*)k, (char*)v,     \
                     row_bytes)
  if (len <= 3 * kSelThreads) KVE_SEL(3);
  else if (len <= 5 * kSelThreads) KVE_SEL(5);
  else KVE_SEL(kSelMaxR);
#undef KVE_SEL
  return hipGetLastError();
}

}  // namespace kve
