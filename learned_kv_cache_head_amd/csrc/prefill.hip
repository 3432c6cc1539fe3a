// Prefill side of the fixed-budget policy (KVpop section 3.2 "Running top-k
// sparse attention", Appendix C.1-C.2, Eq. 26):
//
//  * ranks: rank(t) of every prompt token under its static priority (the
//    score, or score - t log(gamma) with decay, float32), rank 0 best; equal
//    keys rank the newer token first (the reverse of the eviction order);
//  * cutoffs: tau_q, the rank of the k-th best token of the eligible set
//    E(q) = {S <= t <= q - W}, for every query position q;
//  * masked prefill attention: each query q attends to the sinks, its
//    recent window and the eligible tokens with rank(t) <= tau_q.
//
// Ranks: each workgroup sorts a chunk of 4096 (key, position) pairs in LDS
// (bitonic sort, descending); a token's rank is then the number of larger
// pairs, summed over the chunks by binary search.
//
// Cutoffs: ranks are distinct, so an LDS bitmap over rank values holds the
// eligible set E(q). One workgroup per (slice, 64-query block): it sets the
// bits of E(q0) for the block's first query q0 in parallel and finds
// tau_{q0}, the k-th set bit, from word popcounts and a block scan. One wave
// then walks the block's other 63 queries in order: as q grows by one, one
// token enters E(q) and tau_q can only move to a better (smaller) rank.
// While |E| < k, tau = n; when the k-th token enters, tau is the largest
// inserted rank; afterwards a new token better than tau moves tau to the
// next smaller set rank (the predecessor in the bitmap, found 64 words at a
// time with a ballot). (The pages use a Fenwick tree with binary lifting;
// the monotone cutoff makes a bitmap predecessor search enough, and the
// parallel rebuild per block replaces a chain of n sequential steps by one
// of 64.)
//
// Attention: a flash-attention forward on MFMA (float32 accumulation) with
// the Eq. 26 predicate applied to each logit. A workgroup owns 64 query
// positions of one KV head and 2 of its query heads (two waves per SIMD
// fit; an odd last head goes to a second launch, one head per workgroup);
// the 4 waves take 16 positions each. Each 64-key block of K and
// V is staged in LDS, row-major, and shared by all of them; the V^T operand
// comes from LDS transpose reads. The kernel computes S^T = K Q^T
// (v_mfma_f32_16x16x32_bf16), so a lane's accumulators hold 8 keys of one
// query column: those are exactly the operand of P^T that O^T = V^T P^T
// needs, and the online-softmax state is one value per lane and head.
// O^T = V^T P^T runs in float16 (v_mfma_f32_16x16x32_f16 on a float16 copy
// of V, each weight rounded to 11 significant bits) for slices whose V fits
// float16, else in bf16 with each weight as two parts (its rounding and the
// remainder, about 17 bits), two MFMAs into one float32 accumulator. The
// key-list kernel writes the float16 copy of its query block's V rows and
// records their largest |v| for that choice. Workgroups are ordered so that
// each XCD takes whole slices, which share key rows in its L2.
#include "kve_internal.h"

namespace kve {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// Two floats to packed float16 (round to nearest even), a in the low half:
// one v_cvt_pk_f16_f32.
__device__ __forceinline__ uint32_t pack2h(float a, float b) {
  return __builtin_bit_cast(uint32_t,
                            __builtin_convertvector(f32x2_t{a, b}, f16x2_t));
}
// Two packed bf16 to packed float16 (exact for magnitudes in [2^-17, 65280]).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  return pack2h(bf16lo(w), bf16hi(w));
}

constexpr int kSortChunk = 4096;   // pairs sorted per workgroup
constexpr int kQBlock = 64;        // query positions per attention workgroup
constexpr int kSortThreads = 512;

// Orderable 32-bit key of a token's static priority (KVpop Eq. 20),
// rounded like the select kernel: the product, then the difference.
__device__ __forceinline__ uint32_t priority_key(float s, int pos,
                                                 const float* lg, int h) {
  if (lg) s = decayed_priority(s, pos, lg[h]);
  return score_key(s);
}

// ---------------------------------------------------------------------------
// Chunk sort: pairs v = key << 32 | position, descending, padded with 0.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kSortThreads) void rank_sort_kernel(
    const float* score, const float* lg, int H, int cap, int n, int npad,
    uint64_t* sorted) {
  __shared__ uint64_t v[kSortChunk];
  const int slice = blockIdx.y;
  const int c0 = blockIdx.x * kSortChunk;
  const float* sc = score + (size_t)slice * cap;
  for (int i = threadIdx.x; i < kSortChunk; i += kSortThreads) {
    const int t = c0 + i;
    v[i] = t < n ? ((uint64_t)priority_key(sc[t], t, lg, slice % H) << 32) |
                       (uint32_t)t
                 : 0ull;
  }
  __syncthreads();
  for (int size = 2; size <= kSortChunk; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < kSortChunk / 2; i += kSortThreads) {
        // pair (a, a + stride) inside blocks of 2 * stride
        const int a = (i / stride) * 2 * stride + (i % stride);
        const int b = a + stride;
        // descending overall: blocks whose bit `size` is clear sort down
        const bool desc = (a & size) == 0;
        const uint64_t x = v[a], y = v[b];
        if ((x < y) == desc) {
          v[a] = y;
          v[b] = x;
        }
      }
      __syncthreads();
    }
  }
  uint64_t* out = sorted + (size_t)slice * npad + c0;
  for (int i = threadIdx.x; i < kSortChunk; i += kSortThreads) out[i] = v[i];
}

// rank(t) = number of pairs larger than token t's, over all chunks.
__global__ __launch_bounds__(256) void rank_count_kernel(
    const float* score, const float* lg, int H, int cap, int n, int npad,
    const uint64_t* sorted, int32_t* rank) {
  const int slice = blockIdx.y;
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= n) return;
  const uint64_t v =
      ((uint64_t)priority_key(score[(size_t)slice * cap + t], t, lg, slice % H)
       << 32) | (uint32_t)t;
  const uint64_t* base = sorted + (size_t)slice * npad;
  int r = 0;
  for (int c0 = 0; c0 < npad; c0 += kSortChunk) {
    // first index in the descending chunk whose pair is <= v
    int lo = 0, hi = kSortChunk;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (base[c0 + mid] > v) lo = mid + 1;
      else hi = mid;
    }
    r += lo;
  }
  rank[(size_t)slice * n + t] = r;
}

// ---------------------------------------------------------------------------
// Running cutoffs, one workgroup per (slice, 64-query block). tau_q is the
// k-th smallest rank in E(q) = {S <= t <= q - W}; ranks are distinct
// (0..n-1), so a bitmap over rank values holds E. For its first query q0
// the workgroup sets the bits of E(q0) (positions S..q0 - W, in parallel)
// and finds the k-th set bit by a block scan of word popcounts; then one
// wave inserts t = q - W for the block's other queries in order: while
// |E| < k, tau = n (all kept) and the largest rank so far is tracked; at
// |E| = k the cut is that largest rank; after that, an entering rank below
// the cut moves the cut to the largest set rank below it (a predecessor
// search over the bitmap words, 64 words per wave ballot).
// Dynamic LDS: ceil(n / 32) words.
// ---------------------------------------------------------------------------
constexpr int kCutThreads = 256;

__global__ __launch_bounds__(kCutThreads) void cutoff_kernel(
    const int32_t* rank, int n, int S, int W, int k, int32_t* tau) {
  extern __shared__ uint32_t bm[];
  __shared__ uint32_t wpart[kCutThreads / 64];
  __shared__ int sh_cut, sh_maxr;
  const int qb = blockIdx.x;
  const int slice = blockIdx.y;
  const int q0 = qb * kQBlock;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int32_t* rk = rank + (size_t)slice * n;
  int32_t* out = tau + (size_t)slice * n;
  const int m = min(kQBlock, n - q0);
  if (k == 0) {  // no long-range budget: every tau is -1
    if (tid < m) out[q0 + tid] = -1;
    return;
  }
  const int words = (n + 31) >> 5;
  for (int w = tid; w < words; w += kCutThreads) bm[w] = 0u;
  if (tid == 0) {
    sh_cut = n;
    sh_maxr = -1;
  }
  __syncthreads();
  // E(q0): positions S .. q0 - W.
  const int lim = q0 - W;
  int lmax = -1;
  for (int t = S + tid; t <= lim; t += kCutThreads) {
    const int r = rk[t];
    atomicOr(&bm[r >> 5], 1u << (r & 31));
    lmax = max(lmax, r);
  }
  const int count0 = max(0, lim - S + 1);
  // Largest rank of E(q0) (the cut once |E| reaches k).
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) lmax = max(lmax, __shfl_xor(lmax, off));
  if (lane == 0) atomicMax(&sh_maxr, lmax);
  __syncthreads();
  if (count0 >= k) {
    // k-th set bit: thread i counts its run of words, block exclusive scan.
    const int per = (words + kCutThreads - 1) / kCutThreads;
    const int wb = tid * per, we = min(words, wb + per);
    uint32_t c = 0;
    for (int w = wb; w < we; ++w) c += __popc(bm[w]);
    uint32_t incl = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    if (lane == 63) wpart[wave] = incl;
    __syncthreads();
    uint32_t before = incl - c;
    for (int w = 0; w < wave; ++w) before += wpart[w];
    const uint32_t kk = (uint32_t)k;
    if (before < kk && before + c >= kk) {
      uint32_t need = kk - before;  // the need-th set bit of this run
      for (int w = wb; w < we; ++w) {
        uint32_t word = bm[w];
        const uint32_t pc = __popc(word);
        if (need > pc) {
          need -= pc;
          continue;
        }
        for (uint32_t j = 1; j < need; ++j) word &= word - 1u;  // drop lowest
        sh_cut = w * 32 + __ffs(word) - 1;
        break;
      }
    }
  }
  __syncthreads();
  if (wave != 0) return;
  // One wave: the block's queries in order; lane i keeps tau of q0 + i.
  int count = count0;
  int cut = sh_cut;
  int maxr = sh_maxr;
  const int ql = q0 + lane;
  const int tl = ql - W;
  const int rl = (lane > 0 && ql < n && tl >= S) ? rk[tl] : -1;  // entering rank
  int mine = 0;
  for (int i = 0; i < m; ++i) {
    const int r = __builtin_amdgcn_readlane(rl, i);
    if (r >= 0) {
      if (lane == 0) bm[r >> 5] |= 1u << (r & 31);
      ++count;
      maxr = max(maxr, r);
      if (count == k) {
        cut = maxr;
      } else if (count > k && r < cut) {
        // largest set rank below cut (r itself at worst)
        int w0 = (cut - 1) >> 5;
        const uint32_t below = (cut & 31) ? ((1u << (cut & 31)) - 1u) : ~0u;
        int found = -1;
        while (found < 0) {
          const int w = w0 - lane;
          uint32_t word = 0u;
          if (w >= 0) {
            word = bm[w];
            if (w == (cut >> 5)) word &= below;
          }
          const uint64_t nz = __ballot(word != 0u);
          if (nz) {
            const int l = __ffsll((unsigned long long)nz) - 1;  // highest word
            const uint32_t wv = __shfl(word, l);
            found = (w0 - l) * 32 + 31 - __clz(wv);
          } else {
            w0 -= 64;
          }
        }
        cut = found;
      }
    }
    const int t = count >= k ? cut : n;
    mine = lane == i ? t : mine;
  }
  if (lane < m) out[q0 + lane] = mine;
}

// ---------------------------------------------------------------------------
// Long-range key lists: for the query block starting at q0, the eligible
// tokens t in [S, q0 - W] with rank(t) <= tau_q0, in position order. The
// cutoff only tightens as q grows, so these hold every long-range key any
// query of the block keeps (at most k of them: the top-k of E(q0)).
// ---------------------------------------------------------------------------
// The same workgroup records the largest |v| of the block's V rows (the bf16
// bit pattern without its sign), from which the attention chooses the
// arithmetic of its P.V products for the whole slice, and writes the rows in
// float16 to v16 [slice][n][D], which the attention reads when the slice
// fits float16 (rows of other slices are left unread).
__global__ __launch_bounds__(256) void keylist_kernel(const int32_t* rank,
                                                      const int32_t* tau, int n,
                                                      int S, int W, int kmax,
                                                      int32_t* list,
                                                      int32_t* count,
                                                      const uint16_t* v, int D,
                                                      int cap, uint32_t* vmax,
                                                      uint16_t* v16) {
  __shared__ int wsum[4];
  __shared__ uint32_t wmax[4];
  const int qb = blockIdx.x;
  const int slice = blockIdx.y;
  const int nqb = gridDim.x;
  const int q0 = qb * kQBlock;
  {
    const int chunks = min(kQBlock, n - q0) * D / 8;  // 16-byte chunks
    const u32x4* vr = (const u32x4*)(v + ((size_t)slice * cap + q0) * D);
    u32x4* vw = (u32x4*)(v16 + ((size_t)slice * n + q0) * D);
    // At most 64 rows of 128 values: 4 chunks per thread, loaded together.
    u32x4 w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = threadIdx.x + 256 * j;
      if (i < chunks) w[j] = vr[i];
    }
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = threadIdx.x + 256 * j;
      if (i >= chunks) break;
      vw[i] = u32x4{bf16x2_to_f16x2(w[j].x), bf16x2_to_f16x2(w[j].y),
                    bf16x2_to_f16x2(w[j].z), bf16x2_to_f16x2(w[j].w)};
      const uint32_t a = w[j].x & 0x7fff7fffu, b = w[j].y & 0x7fff7fffu;
      const uint32_t c = w[j].z & 0x7fff7fffu, d = w[j].w & 0x7fff7fffu;
      m = max(m, max(max(a >> 16, a & 0xffffu), max(b >> 16, b & 0xffffu)));
      m = max(m, max(max(c >> 16, c & 0xffffu), max(d >> 16, d & 0xffffu)));
    }
    for (int off = 32; off > 0; off >>= 1)
      m = max(m, (uint32_t)__shfl_xor((int)m, off));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0)
      vmax[(size_t)slice * nqb + qb] =
          max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  }
  const int32_t* rk = rank + (size_t)slice * n;
  const int t0 = tau[(size_t)slice * n + q0];
  int32_t* out = list + ((size_t)slice * nqb + qb) * kmax;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lim = q0 - W;  // last eligible position at q0
  int base = 0;
  // 1024 positions per pass, 4 consecutive ones per thread; kept positions
  // are written in order at their exclusive-scan offsets.
  for (int c = S; c <= lim; c += 1024) {
    const int tb = c + 4 * threadIdx.x;
    bool f[4];
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = tb + j;
      f[j] = t <= lim && rk[t] <= t0;
      cnt += f[j] ? 1 : 0;
    }
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int at = base + incl - cnt;
    for (int w = 0; w < wave; ++w) at += wsum[w];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (f[j]) {
        if (at < kmax) out[at] = tb + j;
        ++at;
      }
    }
    base += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
  if (threadIdx.x == 0) count[(size_t)slice * nqb + qb] = min(base, kmax);
}

// ---------------------------------------------------------------------------
// Masked prefill attention.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bf16x8_t load8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *(const u32x4*)p);
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// Two floats to packed bf16 (round to nearest even), a in the low half:
// one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return __builtin_bit_cast(uint32_t,
                            __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// The value lane l ^ 32 (l ^ 16) of the wave holds. permlane32_swap
// exchanges the upper half of its first operand with the lower half of its
// second, so lane l finds its partner in the second result below lane 32
// and in the first from lane 32 on (rows of 16 lanes likewise for
// permlane16_swap, which exchanges odd rows of the first operand with even
// rows of the second).
__device__ __forceinline__ float lane_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                                  __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}
__device__ __forceinline__ float lane_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x),
                                                  __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
}
template <bool B> struct Flag { static constexpr bool value = B; };

constexpr int kQB = kQBlock;
constexpr int kKB = 64;   // keys per block (measured faster than 32)
constexpr float kLazy = 8.f;  // log2 headroom of the softmax reference
constexpr int kWin = 1024;    // key positions held in LDS ahead of the loads

template <int D, int GS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_attn_kernel(PrefillAttnLaunch p) {
  constexpr int KS = D / 32;      // contraction steps of S^T
  constexpr int DT = D / 16;      // 16-row tiles of O^T
  constexpr int KT = kKB / 16;    // 16-key tiles per block
  constexpr int KSTR = D + 8;     // bf16 per staged K row
  // bf16 per staged V row: a row stride of 8 words (mod 32 banks) keeps the
  // 16 lanes of a transpose read (4 rows x 4 column chunks) on distinct banks
  constexpr int VSTR = D + 16;
  __shared__ __align__(16) uint16_t ks[2][kKB * KSTR];
  __shared__ __align__(16) uint16_t vs[2][kKB * VSTR];
  __shared__ __align__(16) int rks[2][kKB];   // rank of each staged key
  __shared__ __align__(16) int tps[2][kKB];   // its position (INT_MAX: padding)
  __shared__ int kpos[kWin];    // positions of key indices [wbase, wbase + kWin)

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nqb = (p.n + kQB - 1) / kQB;
  // Workgroup L runs on XCD L % 8. Each XCD takes a contiguous range of the
  // grid in (query block, head subset, slice) order, so the workgroups of a
  // slice, which gather the same key rows, share one L2.
  const uint32_t nwg = gridDim.x * gridDim.y * gridDim.z;
  const uint32_t L = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const uint32_t xq = nwg / 8, xr = nwg % 8, xcd = L % 8;
  const uint32_t T =
      (xcd < xr ? xcd * (xq + 1) : xr * (xq + 1) + (xcd - xr) * xq) + L / 8;
  const int tx = T % gridDim.x;
  const int ty = (T / gridDim.x) % gridDim.y;
  const int qb = nqb - 1 - tx;  // heavy (late) query blocks first
  const int h = ty / p.nsub;
  const int sub = ty % p.nsub;
  const int b = T / (gridDim.x * gridDim.y);
  const int q0 = qb * kQB;
  const size_t slice = (size_t)b * p.H + h;
  const uint16_t* kc = (const uint16_t*)p.k + slice * p.cap * D;
  const uint16_t* vc = (const uint16_t*)p.v + slice * p.cap * D;  // or v16
  const int32_t* rk = p.rank + slice * p.n;
  const int hq = p.H * p.G;

  // This lane's query column: position qpos, heads sub*GS + gi.
  const int qpos = q0 + wave * 16 + (lane & 15);
  const int qc = min(qpos, p.n - 1);
  const int tau = p.tau[slice * p.n + qc];
  const int g8 = (lane >> 4) * 8;
  bf16x8_t qf[GS][KS];
#pragma unroll
  for (int gi = 0; gi < GS; ++gi) {
    const int g = min(p.g0 + sub * GS + gi, p.G - 1);
    const uint16_t* qr =
        (const uint16_t*)p.q + (((size_t)b * hq + h * p.G + g) * p.n + qc) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[gi][s] = load8(qr + s * 32 + g8);
  }

  f32x4_t o[DT][GS];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int gi = 0; gi < GS; ++gi) o[dt][gi] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mrun[GS], lrun[GS];
#pragma unroll
  for (int gi = 0; gi < GS; ++gi) {
    mrun[gi] = -__builtin_inff();
    lrun[gi] = 0.f;
  }
  const float qscale = 1.4426950408889634f / sqrtf((float)D);  // log2(e)/sqrt(d)

  // Keys of this workgroup in position order: the sinks, the long-range
  // list of this query block, then the span of its recent windows. Every
  // other key is masked for all of its queries.
  const int last_q = min(q0 + kQB, p.n) - 1;
  const int nS = min(p.S, last_q + 1);
  const int qbi = q0 / kQB;
  const int nL = p.count[slice * nqb + qbi];
  const int32_t* lst = p.list + (slice * nqb + qbi) * p.kmax;
  const int w0 = max(p.S, q0 - p.W + 1);
  const int nWin = max(0, last_q - w0 + 1);
  const int nkeys = nS + nL + nWin;
  auto key_pos = [&](int j) {
    return j < nS ? j : (j < nS + nL ? lst[j - nS] : w0 + (j - nS - nL));
  };

  // Staging: a 64-key block is 64 rows of D bf16 (D/8 chunks of 16 B per
  // row) of K and of V; each of the 256 threads moves D/32 chunks of each.
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  u32x4 kreg[kKB * CPR / 256], vreg[kKB * CPR / 256];
  int rreg = 0, treg = 0;
  const int nkb = (nkeys + kKB - 1) / kKB;
  // The K/V loads take their row positions from LDS, so they never wait on
  // the key-list loads (a wait on those would drain every load in flight).
  int wbase = 0;
  auto refill = [&](int j0) {
    wbase = j0;
    for (int i = threadIdx.x; i < kWin; i += 256) {
      const int j = j0 + i;
      kpos[i] = j < nkeys ? key_pos(j) : 0x7fffffff;
    }
  };
  auto fetch = [&](int kb) {
#pragma unroll
    for (int c = 0; c < kKB * CPR / 256; ++c) {
      const int idx = threadIdx.x + c * 256;
      const int row = idx / CPR;
      const int ch = idx % CPR;
      const int t0 = kpos[kb * kKB + row - wbase];
      const int t = t0 == 0x7fffffff ? 0 : t0;  // padding reads row 0
      // 32-bit byte offset from the slice base (a slice holds at most
      // 262144 rows of 256 B), so the loads use a scalar base address
      const uint32_t off = (uint32_t)(t * D + ch * 8) * 2u;
      kreg[c] = *(const u32x4*)((const char*)kc + off);
      vreg[c] = *(const u32x4*)((const char*)vc + off);
    }
    if (threadIdx.x < kKB) {
      treg = kpos[kb * kKB + threadIdx.x - wbase];
      rreg = treg == 0x7fffffff ? 0x7fffffff : rk[treg];
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int c = 0; c < kKB * CPR / 256; ++c) {
      const int idx = threadIdx.x + c * 256;
      const int row = idx / CPR;
      const int ch = idx % CPR;
      *(u32x4*)(&ks[buf][row * KSTR + ch * 8]) = kreg[c];
      *(u32x4*)(&vs[buf][row * VSTR + ch * 8]) = vreg[c];
    }
    if (threadIdx.x < kKB) {
      rks[buf][threadIdx.x] = rreg;
      tps[buf][threadIdx.x] = treg;
    }
  };

  // The P.V products of the slice. When its largest |v| lies in [2^-6,
  // 65280], every V element converts to float16 exactly (magnitudes of at
  // least 2^-17) or within 2^-25 absolute (below): the rows come from the
  // key-list kernel's float16 copy, and each weight enters one float16 MFMA,
  // rounded to 11 significant bits (weights are at most 2^kLazy, far inside
  // float16's range). Otherwise (larger or tiny values, NaN, inf) V is read
  // from the cache in bf16 and each weight enters as two bf16 parts. The
  // choice is uniform per slice, from the maxima the key-list kernel
  // recorded per query block.
  uint32_t vm = 0;
  for (int i = lane; i < nqb; i += 64) vm = max(vm, p.vmax[slice * nqb + i]);
  for (int off = 32; off > 0; off >>= 1)
    vm = max(vm, (uint32_t)__shfl_xor((int)vm, off));
  vm = __builtin_amdgcn_readfirstlane(vm);
  const bool fp16 = vm >= 0x3c80u && vm <= 0x477fu;  // bf16 2^-6 and 65280
  if (fp16) vc = p.v16 + slice * p.n * D;

  auto run = [&](auto f16) {
  constexpr bool F16 = decltype(f16)::value;
  refill(0);
  __syncthreads();
  fetch(0);
  stage(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nkb) {
      if ((kb + 2) * kKB > wbase + kWin) {  // uniform; last read of kpos
        refill((kb + 1) * kKB);             // was before the last barrier
        __syncthreads();
      }
      fetch(kb + 1);
    }
    {
      // S^T = K Q^T: KT 16-key tiles x GS query tiles.
      f32x4_t s[KT][GS];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int gi = 0; gi < GS; ++gi) s[kt][gi] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < KS; ++st) {
          const bf16x8_t A = __builtin_bit_cast(
              bf16x8_t, *(const u32x4*)(&ks[buf][(kt * 16 + (lane & 15)) * KSTR +
                                                  st * 32 + g8]));
#pragma unroll
          for (int gi = 0; gi < GS; ++gi)
            s[kt][gi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, qf[gi][st],
                                                                s[kt][gi], 0, 0, 0);
        }
      }
      // Eq. 26 predicate for this lane's keys and its query position.
      // Blocks made only of long-range list keys (t <= q0 - W for every
      // query of the workgroup, never sinks) need only the rank test.
      // (Evaluated without short-circuits: every operand is loaded, so no
      // branches split the block.)
      const int j0 = kb * kKB;
      const bool list_only = j0 >= nS && j0 + kKB <= nS + nL;  // uniform
      bool keep[KT][4];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const int kr = kt * 16 + 4 * (lane >> 4);
        const int4 r4 = *(const int4*)&rks[buf][kr];
        const int rv[4] = {r4.x, r4.y, r4.z, r4.w};
        if (list_only) {
#pragma unroll
          for (int i = 0; i < 4; ++i) keep[kt][i] = rv[i] <= tau;
        } else {
          const int4 t4 = *(const int4*)&tps[buf][kr];
          const int tv[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i)
            keep[kt][i] = (tv[i] <= qpos) &
                          ((tv[i] < p.S) | (tv[i] > qpos - p.W) | (rv[i] <= tau));
        }
      }
      // Online softmax per query column, then O^T += V^T P^T, 32 keys per
      // contraction step: half hh holds key tiles 2hh and 2hh+1. Each weight
      // goes to the MFMA as one float16 (pk), or as two bf16 parts, its
      // rounding and the remainder (pk, pl), whose sum carries a relative
      // error of at most 2^-17.
      uint32_t pk[GS][KT / 2][4], pl[GS][KT / 2][4];
#pragma unroll
      for (int gi = 0; gi < GS; ++gi) {
        // Raw logits (the scale is positive, so the maximum commutes with
        // it); the scale folds into the exponent's FMA below.
        float x[KT * 4];
        float mx = -__builtin_inff();
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = keep[kt][i] ? s[kt][gi][i] : -__builtin_inff();
            x[kt * 4 + i] = v;
            mx = fmaxf(mx, v);
          }
        mx = fmaxf(mx, lane_xor16(mx));
        mx = fmaxf(mx, lane_xor32(mx));
        mx *= qscale;
        // Lazy rescaling: the reference maximum moves only when a logit
        // passes it by more than 2^kLazy (or on the first kept key), so
        // weights stay below 2^kLazy and the accumulators are rarely scaled.
        const bool move = mx > mrun[gi] + kLazy;
        const float mnew = move ? mx : mrun[gi];
        const float alpha = move ? __builtin_amdgcn_exp2f(mrun[gi] - mnew) : 1.f;
        const float mref = mnew == -__builtin_inff() ? 0.f : mnew;
        // bf16 path: p enters as hi = bf16(p) and lo = bf16(p - hi); p - hi
        // is exact in float32 and at most 2^-9 p, so hi + lo is within
        // 2^-17 p. The normaliser, and so lse, sums the float32 values.
        float ps = 0.f;
#pragma unroll
        for (int j = 0; j < KT * 4; j += 2) {
          const float e0 = __builtin_amdgcn_exp2f(fmaf(x[j], qscale, -mref));
          const float e1 = __builtin_amdgcn_exp2f(fmaf(x[j + 1], qscale, -mref));
          if constexpr (F16) {
            pk[gi][j >> 3][(j >> 1) & 3] = pack2h(e0, e1);
          } else {
            const uint32_t hi = pack2(e0, e1);
            pk[gi][j >> 3][(j >> 1) & 3] = hi;
            pl[gi][j >> 3][(j >> 1) & 3] = pack2(e0 - bf16lo(hi), e1 - bf16hi(hi));
          }
          ps += e0 + e1;
        }
        lrun[gi] = lrun[gi] * alpha + ps;
        mrun[gi] = mnew;
        if (__ballot(move)) {  // some column's reference moved
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) o[dt][gi] *= alpha;
        }
      }
      // V^T operand by LDS transpose reads (ds_read_b64_tr_b16): in each
      // 16-lane group, lane 4j + s points at the 4 columns 4s.. of key row
      // j, and lane m receives column m of the 4 rows. Lane l thus gets
      // V[keys pi(l/16, 0..3)][dt * 16 + l % 16], the A rows of O^T.
      const int trow = 4 * (lane >> 4) + ((lane & 15) >> 2);
      const int tcol = 4 * (lane & 3);
#pragma unroll
      for (int hh = 0; hh < KT / 2; ++hh) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const uint16_t* v0 = &vs[buf][(hh * 32 + trow) * VSTR + dt * 16 + tcol];
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)v0);
          const i16x4 hi =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v0 + 16 * VSTR));
          const u32x4 a = u32x4{__builtin_bit_cast(u32x2, lo).x, __builtin_bit_cast(u32x2, lo).y,
                                __builtin_bit_cast(u32x2, hi).x, __builtin_bit_cast(u32x2, hi).y};
          if constexpr (F16) {
#pragma unroll
            for (int gi = 0; gi < GS; ++gi) {
              const u32x4 bw{pk[gi][hh][0], pk[gi][hh][1], pk[gi][hh][2], pk[gi][hh][3]};
              o[dt][gi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                  __builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, bw),
                  o[dt][gi], 0, 0, 0);
            }
          } else {
            const bf16x8_t A = __builtin_bit_cast(bf16x8_t, a);
#pragma unroll
            for (int gi = 0; gi < GS; ++gi) {
              const bf16x8_t B = __builtin_bit_cast(
                  bf16x8_t,
                  u32x4{pk[gi][hh][0], pk[gi][hh][1], pk[gi][hh][2], pk[gi][hh][3]});
              o[dt][gi] =
                  __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, o[dt][gi], 0, 0, 0);
            }
#pragma unroll
            for (int gi = 0; gi < GS; ++gi) {
              const bf16x8_t B = __builtin_bit_cast(
                  bf16x8_t,
                  u32x4{pl[gi][hh][0], pl[gi][hh][1], pl[gi][hh][2], pl[gi][hh][3]});
              o[dt][gi] =
                  __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, o[dt][gi], 0, 0, 0);
            }
          }
        }
      }
    }
    // The other buffer was last read before the previous barrier.
    if (kb + 1 < nkb) stage(buf ^ 1);
    __syncthreads();
  }
  };
  if (fp16)
    run(Flag<true>{});
  else
    run(Flag<false>{});

  // Epilogue: normalise and store this lane's column (4 rows per d tile).
#pragma unroll
  for (int gi = 0; gi < GS; ++gi) {
    const int g = p.g0 + sub * GS + gi;
    float l = lrun[gi];
    l += lane_xor16(l);
    l += lane_xor32(l);
    if (g >= p.G || qpos >= p.n) continue;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* orow = p.out + (((size_t)b * hq + h * p.G + g) * p.n + qpos) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const f32x4_t v = o[dt][gi] * inv;
      *(float4*)(orow + dt * 16 + 4 * (lane >> 4)) = float4{v[0], v[1], v[2], v[3]};
    }
    if (p.lse && (lane >> 4) == 0)
      p.lse[((size_t)b * hq + h * p.G + g) * p.n + qpos] =
          l > 0.f ? 0.6931471805599453f * (mrun[gi] + log2f(l)) : -__builtin_inff();
  }
}

}  // namespace

size_t prefill_ws_bytes(long long slices, int n) {
  const long long npad = (n + kSortChunk - 1) / kSortChunk * kSortChunk;
  return (size_t)(slices * npad) * sizeof(uint64_t);
}

hipError_t launch_prefill_select(const float* score, const float* lg, int H,
                                 int slices, int cap, int n, int S, int W,
                                 int k, void* ws, int32_t* rank, int32_t* tau,
                                 hipStream_t s) {
  const int npad = (n + kSortChunk - 1) / kSortChunk * kSortChunk;
  uint64_t* sorted = (uint64_t*)ws;
  hipLaunchKernelGGL(rank_sort_kernel, dim3(npad / kSortChunk, slices),
                     dim3(kSortThreads), 0, s, score, lg, H, cap, n, npad, sorted);
  hipLaunchKernelGGL(rank_count_kernel, dim3((n + 255) / 256, slices), dim3(256),
                     0, s, score, lg, H, cap, n, npad, (const uint64_t*)sorted,
                     rank);
  const int nqb = (n + kQBlock - 1) / kQBlock;
  const size_t bm_bytes = (size_t)((n + 31) / 32) * sizeof(uint32_t);
  hipLaunchKernelGGL(cutoff_kernel, dim3(nqb, slices), dim3(kCutThreads),
                     bm_bytes, s, (const int32_t*)rank, n, S, W, k, tau);
  return hipGetLastError();
}

// Workspace: the key lists, then one count and one V maximum per (slice,
// query block), each part rounded up to 256 bytes, then the float16 copy of
// V (n rows of D per slice).
size_t prefill_attn_ws_bytes(long long slices, int n, int kmax, int D) {
  const long long nqb = (n + kQB - 1) / kQB;
  const size_t lists = (size_t)(slices * nqb) * kmax * sizeof(int32_t);
  const size_t blocks = (size_t)(slices * nqb) * sizeof(int32_t);
  return (lists + 255) / 256 * 256 + (2 * blocks + 255) / 256 * 256 +
         (size_t)slices * n * D * sizeof(uint16_t);
}

hipError_t launch_prefill_attn(PrefillAttnLaunch a, void* ws, hipStream_t s) {
  const int nqb = (a.n + kQB - 1) / kQB;
  const size_t blocks = (size_t)a.batch * a.H * nqb;
  const size_t lists = (blocks * a.kmax * sizeof(int32_t) + 255) / 256 * 256;
  a.list = (int32_t*)ws;
  a.count = (int32_t*)((char*)ws + lists);
  a.vmax = (uint32_t*)(a.count + blocks);
  a.v16 = (uint16_t*)((char*)ws + lists + (2 * blocks * sizeof(int32_t) + 255) / 256 * 256);
  hipLaunchKernelGGL(keylist_kernel, dim3(nqb, a.batch * a.H), dim3(256), 0, s,
                     a.rank, a.tau, a.n, a.S, a.W, a.kmax, a.list, a.count,
                     (const uint16_t*)a.v, a.D, a.cap, a.vmax, a.v16);
  if (a.D != 128 && a.D != 64) return hipErrorInvalidValue;
  // Query heads in pairs (two per workgroup), and an odd last head in a
  // launch of its own with one head per workgroup, so that no workgroup
  // computes a head twice.
  auto launch = [&](int gs, int nsub, int g0) {
    PrefillAttnLaunch b = a;
    b.gsub = gs;
    b.nsub = nsub;
    b.g0 = g0;
    const dim3 grid(nqb, b.H * nsub, b.batch);
    if (b.D == 128 && gs == 2)
      hipLaunchKernelGGL((prefill_attn_kernel<128, 2>), grid, dim3(256), 0, s, b);
    else if (b.D == 128)
      hipLaunchKernelGGL((prefill_attn_kernel<128, 1>), grid, dim3(256), 0, s, b);
    else if (gs == 2)
      hipLaunchKernelGGL((prefill_attn_kernel<64, 2>), grid, dim3(256), 0, s, b);
    else
      hipLaunchKernelGGL((prefill_attn_kernel<64, 1>), grid, dim3(256), 0, s, b);
  };
  if (a.G / 2 > 0) launch(2, a.G / 2, 0);
  if (a.G % 2) launch(1, 1, a.G - 1);
  return hipGetLastError();
}

}  // namespace kve
