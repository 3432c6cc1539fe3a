// Cache maintenance kernels: append, select (radix select of the eviction
// cut) and in-place order-preserving compaction.
//
// Retention rule (KVpop section 3, Eq. 1 and 4; Appendix C.1, Eq. 26):
// slots [0, S) are sink tokens and [len - W, len) the protected recent
// window; the other slots are the eligible long-range candidates, of which
// the top ones by score are kept. Periodic eviction (ForesightKV summary,
// "Methodology in plain English"; Fast KVzip Appendix A.5) cuts a slice of
// len entries back to n_keep = B entries. Ranking uses float32 scores
// (KVpop Appendix F) with the older entry evicted first among equal scores.
#include "kve_internal.h"

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
// Among the m = len - S - W candidates, evict the r = len - n_keep with the
// smallest (score, slot) keys. A four-pass 8-bit MSB radix select finds the
// r-th smallest 32-bit score key thr and the number need of entries equal
// to thr that fall below the cut; a final ordered pass evicts every key
// < thr and the first `need` keys == thr in slot order (older first), and
// writes the survivors' slots in ascending order with a block-wide scan.
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / 64;

__device__ __forceinline__ uint32_t lane_prefix(uint64_t mask) {
  // Number of set bits of `mask` in lanes below this one.
  uint32_t lo = __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u);
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), lo);
}

// Exclusive block-wide prefix count of `flag` (slot order = thread order);
// returns the prefix and writes the block total to *total.
__device__ __forceinline__ uint32_t block_excl_count(bool flag, uint32_t* sh,
                                                     uint32_t* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint64_t mask = __builtin_amdgcn_ballot_w64(flag);
  const uint32_t in_wave = lane_prefix(mask);
  if (lane == 0) sh[wave] = (uint32_t)__builtin_popcountll(mask);
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const uint32_t c = sh[w];
    before += (w < wave) ? c : 0u;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return before + in_wave;
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const float* score, int cap, int len, int n_keep, int S, int W,
    int32_t* keep) {
  const size_t slice = blockIdx.x;
  const float* sc = score + slice * (size_t)cap;
  int32_t* out = keep + slice * (size_t)n_keep;
  const int tid = threadIdx.x;

  if (n_keep >= len) {  // nothing to evict: identity
    for (int i = tid; i < len; i += kSelThreads) out[i] = i;
    return;
  }
  const int m = len - S - W;      // candidates, slots [S, len - W)
  const int r = len - n_keep;     // entries to evict, 1 <= r <= m
  for (int i = tid; i < S; i += kSelThreads) out[i] = i;
  for (int j = tid; j < W; j += kSelThreads) out[n_keep - W + j] = len - W + j;

  __shared__ uint32_t hist[256];
  __shared__ uint32_t wsum[kSelWaves];
  __shared__ uint32_t sh_digit, sh_below;
  uint32_t prefix = 0, mask = 0;
  uint32_t remaining = (uint32_t)r;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    for (int c = tid; c < m; c += kSelThreads) {
      const uint32_t key = score_key(sc[S + c]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    // Inclusive scan of the 256 bins by threads 0..255 (4 waves).
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
        sh_digit = (uint32_t)tid;
        sh_below = incl - v;
      }
    }
    __syncthreads();
    prefix |= sh_digit << shift;
    mask |= 255u << shift;
    remaining -= sh_below;
    __syncthreads();
  }
  const uint32_t thr = prefix;     // key of the r-th smallest candidate
  const uint32_t need = remaining; // keys == thr to evict (oldest first)

  __shared__ uint32_t scan_sh[kSelWaves];
  uint32_t carry_eq = 0, carry_keep = 0;
  for (int base = 0; base < m; base += kSelThreads) {
    const int c = base + tid;
    const bool valid = c < m;
    const uint32_t key = valid ? score_key(sc[S + c]) : 0u;
    const bool is_eq = valid && key == thr;
    const bool is_lt = valid && key < thr;
    uint32_t tot_eq, tot_keep;
    const uint32_t eq_rank = carry_eq + block_excl_count(is_eq, scan_sh, &tot_eq);
    const bool kept = valid && !is_lt && !(is_eq && eq_rank < need);
    const uint32_t kidx =
        carry_keep + block_excl_count(kept, scan_sh, &tot_keep);
    if (kept) out[S + kidx] = S + c;
    carry_eq += tot_eq;
    carry_keep += tot_keep;
  }
}

// ---------------------------------------------------------------------------
// Compact in place, order-preserving: new slot i = old slot keep[i].
//
// Grid: (slice, part); each part owns one 128-byte column block of the K or
// V rows (part 0 also moves score and pos). keep is strictly ascending, so
// keep[i] >= i and the destination of output i never lies after its source.
// Outputs are processed in ascending chunks; every chunk reads all of its
// sources before any of its writes (barrier in between), and later chunks'
// sources lie beyond this chunk's destinations, so no unread source is ever
// overwritten. Slots before the first hole (keep[i] == i) are skipped.
// ---------------------------------------------------------------------------
constexpr int kCompThreads = 256;
constexpr int kCompRowsPerLoad = kCompThreads / 8;  // 8 lanes x 16 B per row
constexpr int kCompLoads = 4;
constexpr int kCompChunk = kCompRowsPerLoad * kCompLoads;  // 128 rows

__global__ __launch_bounds__(kCompThreads) void compact_kernel(
    char* k, char* v, float* score, int32_t* pos, int cap, int row_bytes,
    const int32_t* keep, int n_keep) {
  const size_t slice = blockIdx.x;
  const int parts_per_tensor = row_bytes / 128;
  const int part = blockIdx.y;
  const int tensor = part / parts_per_tensor;
  const int col = part % parts_per_tensor;
  char* base = (tensor == 0 ? k : v) + slice * (size_t)cap * row_bytes + col * 128;
  const bool meta = (part == 0);
  float* sc = score + slice * (size_t)cap;
  int32_t* ps = pos + slice * (size_t)cap;
  const int32_t* kp = keep + slice * (size_t)n_keep;
  const int tid = threadIdx.x;

  // First index that moves: keep[i] == i holds exactly for i < first.
  __shared__ int sh_first;
  if (tid == 0) {
    int lo = 0, hi = n_keep;  // invariant: keep[i] == i for i < lo
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (kp[mid] == mid) lo = mid + 1; else hi = mid;
    }
    sh_first = lo;
  }
  __syncthreads();
  const int first = sh_first;

  const int r_in = tid >> 3;        // row within a load
  const int c16 = (tid & 7) * 16;   // byte offset within the 128-byte block
  for (int c0 = first; c0 < n_keep; c0 += kCompChunk) {
    u32x4 val[kCompLoads];
    float sv = 0.f;
    int32_t pv = 0;
#pragma unroll
    for (int j = 0; j < kCompLoads; ++j) {
      const int i = c0 + j * kCompRowsPerLoad + r_in;
      if (i < n_keep) {
        const int src = kp[i];
        val[j] = *(const u32x4*)(base + (size_t)src * row_bytes + c16);
      }
    }
    const int im = c0 + tid;
    if (meta && tid < kCompChunk && im < n_keep) {
      const int src = kp[im];
      sv = sc[src];
      pv = ps[src];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kCompLoads; ++j) {
      const int i = c0 + j * kCompRowsPerLoad + r_in;
      if (i < n_keep) *(u32x4*)(base + (size_t)i * row_bytes + c16) = val[j];
    }
    if (meta && tid < kCompChunk && im < n_keep) {
      sc[im] = sv;
      ps[im] = pv;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_append(void* k, void* v, int32_t* pos, int batch, int H,
                         int D, int cap, int elem_bytes, int slot,
                         int position, const void* k_new, const void* v_new,
                         const void* hidden_new, void* hidden_buf,
                         int hidden_dim, int hidden_rows, int hidden_row,
                         hipStream_t s) {
  const int slices = batch * H;
  const int extra = hidden_new ? batch : 0;
  hipLaunchKernelGGL(append_kernel, dim3(slices + extra), dim3(64), 0, s,
                     (char*)k, (char*)v, pos, H, D * elem_bytes, cap, slot,
                     position, (const char*)k_new, (const char*)v_new, batch,
                     (const char*)hidden_new, (char*)hidden_buf,
                     hidden_dim * 2, hidden_rows, hidden_row);
  return hipGetLastError();
}

hipError_t launch_select(const float* score, int slices, int cap, int len,
                         int n_keep, int S, int W, int32_t* keep,
                         hipStream_t s) {
  hipLaunchKernelGGL(select_kernel, dim3(slices), dim3(kSelThreads), 0, s,
                     score, cap, len, n_keep, S, W, keep);
  return hipGetLastError();
}

hipError_t launch_compact(void* k, void* v, float* score, int32_t* pos,
                          int slices, int cap, int row_bytes,
                          const int32_t* keep, int n_keep, hipStream_t s) {
  if (row_bytes % 128 != 0) return hipErrorInvalidValue;
  const int parts = 2 * (row_bytes / 128);
  hipLaunchKernelGGL(compact_kernel, dim3(slices, parts), dim3(kCompThreads),
                     0, s, (char*)k, (char*)v, score, pos, cap, row_bytes,
                     keep, n_keep);
  return hipGetLastError();
}

}  // namespace kve
