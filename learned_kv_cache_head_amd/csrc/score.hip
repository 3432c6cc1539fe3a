// Scorers: per-KV-head importance score of each pending cache slot.
//
//  * MLP over [k; v] (KVpop section 3.3 "Stateless scorers", Appendix
//    E.1-E.2, Eq. 35-36): score = w2 . act(W1 [k; v] + b1) + b2, key first.
//    For bf16 caches the first layer is a dense contraction
//    (rows x 2d) x (2d x hidden) and runs on MFMA (v_mfma_f32_16x16x32_bf16,
//    float32 accumulation) with W1 staged in LDS; the hidden activations
//    stay in float32 for the second layer. Float32 caches use a float32 VALU
//    kernel.
//  * Gate on hidden states (Fast KVzip section 3.1, g_l: R^D -> [0,1]^H):
//    score = sigmoid(w_h . x + b_h), all H heads of a token at once as a
//    (rows x D) x (D x H) MFMA contraction with H padded to 16.
//
// MFMA operand layout used here (16x16x32 bf16): lane l supplies row
// (l % 16) of A and column (l % 16) of B, each with 8 consecutive
// contraction indices starting at 8 * (l / 16); the accumulator holds
// C[4 * (l / 16) + i][l % 16], i = 0..3. A and B always use the same
// contraction order, so only the row/column mapping matters.
#include "kve_internal.h"
#include "mlp_tile.h"

namespace kve {
namespace {

__device__ __forceinline__ bf16x8_t load8(const uint16_t* p) {
  return load_bf16x8(p);
}

__device__ __forceinline__ float activate(float a, int act) {
  return mlp_activate(a, act);
}

// ---------------------------------------------------------------------------
// MLP scorer on MFMA (bf16 K/V and W1). A workgroup scores kMlpWaves * TILES
// * 16 rows of one KV head, flattened over (batch, slot); the head's W1 is
// staged once in LDS (rows padded by 16 bytes against bank conflicts) and
// every wave loops over TILES tiles of 16 rows, loading the next tile's
// [k; v] operands before the MFMAs of the current one. Eight tiles per wave
// halve the W1 staging per row for prompts; the buffered rows of a decode
// eviction (L per slice) take fewer tiles so that every CU gets workgroups.
// ---------------------------------------------------------------------------
constexpr int kMlpWaves = 4;
constexpr int kMlpMaxTiles = 8;  // tiles per wave for long row counts

template <int D, int NB, int TILES>
__global__ __launch_bounds__(256) void mlp_mfma_kernel(MlpLaunch p) {
  constexpr int kMlpRowsPerWG = kMlpWaves * TILES * 16;
  constexpr int HID = NB * 16;
  constexpr int IN = 2 * D;
  constexpr int KSTEPS = IN / 32;   // 32-wide contraction steps
  constexpr int LSTR = IN + 8;      // bf16 per staged W1 row
  __shared__ uint16_t w1s[HID * LSTR];
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rows = p.slot_end - p.slot_begin;  // rows per slice
  const long long total = (long long)p.batch * rows;
  const long long wg_row0 = (long long)blockIdx.x * kMlpRowsPerWG;

  mlp_stage_w1<HID, IN>(w1s, LSTR,
                         (const uint16_t*)p.w1 + (size_t)h * HID * IN, 256);
  const int ncol = lane & 15;       // MFMA column = hidden unit within block
  const int kq = (lane >> 4) * 8;   // this lane's 8 contraction indices
  float bias[NB], w2v[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = nb * 16 + ncol;
    bias[nb] = p.b1 ? p.b1[(size_t)h * HID + n] : 0.f;
    w2v[nb] = p.w2[(size_t)h * HID + n];
  }
  const float b2 = p.b2 ? p.b2[h] : 0.f;
  __syncthreads();

  // Tile t of this wave covers rows wg_row0 + (t * kMlpWaves + wave) * 16 ..
  // +15. Rows past the end are clamped (computed, never written), so every
  // load below is unconditional and in bounds.
  auto tile_row0 = [&](int t) {
    return wg_row0 + (long long)(t * kMlpWaves + wave) * 16;
  };
  auto load_tile = [&](bf16x8_t (&a)[KSTEPS], int t) {
    long long rid = tile_row0(t) + (lane & 15);
    if (rid >= total) rid = total - 1;
    const int b = (int)(rid / rows);
    const int slot = p.slot_begin + (int)(rid - (long long)b * rows);
    const size_t slice = (size_t)b * p.H + h;
    const uint16_t* krow = (const uint16_t*)p.k + (slice * p.cap + slot) * D;
    const uint16_t* vrow = (const uint16_t*)p.v + (slice * p.cap + slot) * D;
    mlp_load_row<D>(a, krow, vrow, kq);
  };
  auto compute_tile = [&](const bf16x8_t (&a)[KSTEPS], int t) {
    float sc4[4];
    mlp_tile_scores<D, NB>(a, w1s, LSTR, bias, w2v, b2, p.act, sc4);
    if (ncol == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const long long rid = tile_row0(t) + 4 * (lane >> 4) + i;
        if (rid < total) {
          const int b = (int)(rid / rows);
          const int slot = p.slot_begin + (int)(rid - (long long)b * rows);
          p.score[((size_t)b * p.H + h) * p.cap + slot] = sc4[i];
        }
      }
    }
  };

  bf16x8_t a0[KSTEPS], a1[KSTEPS];
  load_tile(a0, 0);
  if constexpr (TILES == 1) {
    compute_tile(a0, 0);
  } else {
#pragma unroll
    for (int t = 0; t < TILES; t += 2) {
      load_tile(a1, t + 1);
      compute_tile(a0, t);
      if (t + 2 < TILES) load_tile(a0, t + 2);
      compute_tile(a1, t + 1);
    }
  }
}

// ---------------------------------------------------------------------------
// MLP scorer on the float32 VALU (float32 caches, or shapes the MFMA kernel
// does not take). One thread per row; the row's [k; v] features in LDS;
// weights are read with workgroup-uniform addresses.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(64) void mlp_valu_kernel(MlpLaunch p) {
  extern __shared__ float xs[];  // [64][IN + 1]
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int t = threadIdx.x;
  const int D = p.D;
  const int IN = 2 * D;
  const int rows = p.slot_end - p.slot_begin;
  const int row = blockIdx.x * 64 + t;
  const bool ok = row < rows;
  const int slot = p.slot_begin + (ok ? row : rows - 1);
  const size_t slice = (size_t)b * p.H + h;
  float* x = xs + t * (IN + 1);
  for (int i = 0; i < D; ++i) {
    const size_t off = (slice * p.cap + slot) * D + i;
    if constexpr (BF16) {
      x[i] = __uint_as_float((uint32_t)((const uint16_t*)p.k)[off] << 16);
      x[D + i] = __uint_as_float((uint32_t)((const uint16_t*)p.v)[off] << 16);
    } else {
      x[i] = ((const float*)p.k)[off];
      x[D + i] = ((const float*)p.v)[off];
    }
  }
  float s = p.b2 ? p.b2[h] : 0.f;
  for (int j = 0; j < p.hidden; ++j) {
    const size_t wo = ((size_t)h * p.hidden + j) * IN;
    float a = p.b1 ? p.b1[(size_t)h * p.hidden + j] : 0.f;
    for (int i = 0; i < IN; ++i) {
      float w;
      if constexpr (BF16) {
        w = __uint_as_float((uint32_t)((const uint16_t*)p.w1)[wo + i] << 16);
      } else {
        w = ((const float*)p.w1)[wo + i];
      }
      a = fmaf(w, x[i], a);
    }
    s = fmaf(activate(a, p.act), p.w2[(size_t)h * p.hidden + j], s);
  }
  if (ok) p.score[slice * p.cap + slot] = s;
}

// ---------------------------------------------------------------------------
// Gate scorer on MFMA (Fast KVzip section 3.1: a linear map of the token's
// hidden state per KV head, then a sigmoid). The contraction is
// (tokens x D) x (D x H), H <= 16 padded to the 16 columns of
// v_mfma_f32_16x16x32_bf16. One wave = kGateRG groups of 16 tokens x all H
// heads: each 16-byte weight load feeds kGateRG MFMAs, so the weight reads
// (from L2) are a quarter of the hidden-state stream, and a k step keeps
// kGateRG hidden-state loads per lane in flight, kGateUnroll steps ahead.
// ---------------------------------------------------------------------------
constexpr int kGateRG = 4;                       // 16-token groups per wave
constexpr int kGateRowsPerWG = 4 * 16 * kGateRG;  // 4 waves

__global__ __launch_bounds__(256) void gate_mfma_kernel(GateLaunch g) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rows = g.slot_end - g.slot_begin;
  const int r0 = blockIdx.x * kGateRowsPerWG + wave * 16 * kGateRG;
  if (r0 >= rows) return;
  const uint16_t* x[kGateRG];
#pragma unroll
  for (int gi = 0; gi < kGateRG; ++gi) {
    const int rrow = r0 + gi * 16 + (lane & 15);
    const int rc = rrow < rows ? rrow : rows - 1;  // clamp: in bounds
    x[gi] = (const uint16_t*)g.hidden + (size_t)b * g.batch_stride +
            (size_t)rc * g.in_dim;
  }
  const int n = lane & 15;
  const bool has_w = n < g.H;
  const uint16_t* w = (const uint16_t*)g.w + (size_t)(has_w ? n : 0) * g.in_dim;
  // Lanes of columns n >= H load weight row 0 (in bounds, no branch): an
  // MFMA output column depends only on its own B column, and those columns
  // are never stored.
  const int kq = (lane >> 4) * 8;
  f32x4_t acc[kGateRG];
#pragma unroll
  for (int gi = 0; gi < kGateRG; ++gi) acc[gi] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto step = [&](const u32x4& wb, const u32x4& xa, int gi) {
    acc[gi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
        __builtin_bit_cast(bf16x8_t, xa), __builtin_bit_cast(bf16x8_t, wb),
        acc[gi], 0, 0, 0);
  };
  auto wload = [&](int kidx) { return *(const u32x4*)(w + kidx); };
  // k blocks of kGateKU steps: every load of a block is issued before its
  // MFMAs.
  constexpr int kGateKU = 4;
  const int ksteps = g.in_dim / 32;
  int ks = 0;
  for (; ks + kGateKU <= ksteps; ks += kGateKU) {
    u32x4 wb[kGateKU], xa[kGateKU][kGateRG];
#pragma unroll
    for (int u = 0; u < kGateKU; ++u) {
      const int kidx = (ks + u) * 32 + kq;
      wb[u] = wload(kidx);
#pragma unroll
      for (int gi = 0; gi < kGateRG; ++gi)
        xa[u][gi] = *(const u32x4*)(x[gi] + kidx);
    }
    // Keep the scheduler from interleaving the block's loads with its MFMAs
    // (it would reuse the registers and leave few loads in flight).
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kGateKU; ++u)
#pragma unroll
      for (int gi = 0; gi < kGateRG; ++gi) step(wb[u], xa[u][gi], gi);
  }
  for (; ks < ksteps; ++ks) {
    const int kidx = ks * 32 + kq;
    const u32x4 wb = wload(kidx);
#pragma unroll
    for (int gi = 0; gi < kGateRG; ++gi)
      step(wb, *(const u32x4*)(x[gi] + kidx), gi);
  }
  if (has_w) {
    const float bias = g.b ? g.b[n] : 0.f;
    float* out = g.score + ((size_t)b * g.H + n) * g.cap + g.slot_begin;
#pragma unroll
    for (int gi = 0; gi < kGateRG; ++gi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = r0 + gi * 16 + 4 * (lane >> 4) + i;
        if (row < rows) out[row] = 1.f / (1.f + __expf(-(acc[gi][i] + bias)));
      }
  }
}

// Few rows (the L pending tokens of a decode eviction): one workgroup of
// kGateSmallWaves waves per 16 tokens, each wave taking a slice of the D
// contraction; the partial sums meet in LDS before the sigmoid. A single wave
// walking the whole contraction would chain D / 128 dependent load blocks,
// and one workgroup for all the tokens would be held to one CU's bandwidth.
constexpr int kGateSmallWaves = 16;
constexpr int kGateSmallMaxRows = 64;  // row counts served by this kernel

// With `stride` 8 only every 8th workgroup id works: workgroups are handed
// to the 8 XCDs round-robin, so the working ones share one XCD and its L2,
// and the weights they all read come from memory once (used when so few
// workgroups run that one XCD's CUs hold them all).
__global__ __launch_bounds__(64 * kGateSmallWaves) void gate_mfma_small_kernel(
    GateLaunch g, int stride) {
  constexpr int RG = 1;  // 16-token groups per workgroup
  __shared__ f32x4_t red[kGateSmallWaves][RG][64];
  if (blockIdx.x % stride) return;  // uniform: before any barrier
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rows = g.slot_end - g.slot_begin;
  const int r0 = (blockIdx.x / stride) * 16 * RG;
  const uint16_t* x[RG];
#pragma unroll
  for (int gi = 0; gi < RG; ++gi) {
    const int rrow = r0 + gi * 16 + (lane & 15);
    const int rc = rrow < rows ? rrow : rows - 1;  // clamp: in bounds
    x[gi] = (const uint16_t*)g.hidden + (size_t)b * g.batch_stride +
            (size_t)rc * g.in_dim;
  }
  const int n = lane & 15;
  const uint16_t* w =
      (const uint16_t*)g.w + (size_t)(n < g.H ? n : 0) * g.in_dim;
  const int kq = (lane >> 4) * 8;
  const int ksteps = g.in_dim / 32;
  const int per = (ksteps + kGateSmallWaves - 1) / kGateSmallWaves;
  const int k0 = wave * per;
  const int k1 = min(ksteps, k0 + per);
  f32x4_t acc[RG];
#pragma unroll
  for (int gi = 0; gi < RG; ++gi) acc[gi] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto step = [&](const u32x4& wb, const u32x4& xa, int gi) {
    acc[gi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
        __builtin_bit_cast(bf16x8_t, xa), __builtin_bit_cast(bf16x8_t, wb),
        acc[gi], 0, 0, 0);
  };
  // Blocks of four steps, every load of a block ahead of its MFMAs.
  constexpr int KU = 4;
  int ks = k0;
  for (; ks + KU <= k1; ks += KU) {
    u32x4 wb[KU], xa[KU][RG];
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int kidx = (ks + u) * 32 + kq;
      wb[u] = *(const u32x4*)(w + kidx);
#pragma unroll
      for (int gj = 0; gj < RG; ++gj)
        xa[u][gj] = *(const u32x4*)(x[gj] + kidx);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < KU; ++u)
#pragma unroll
      for (int gj = 0; gj < RG; ++gj) step(wb[u], xa[u][gj], gj);
  }
  for (; ks < k1; ++ks) {
    const int kidx = ks * 32 + kq;
    const u32x4 wb = *(const u32x4*)(w + kidx);
#pragma unroll
    for (int gj = 0; gj < RG; ++gj)
      step(wb, *(const u32x4*)(x[gj] + kidx), gj);
  }
#pragma unroll
  for (int gi = 0; gi < RG; ++gi) red[wave][gi][lane] = acc[gi];
  __syncthreads();
  // Thread t < 256 * RG: group t / 256, lane (t / 4) % 64, element t % 4.
  if (tid >= 256 * RG) return;
  const int gi = tid >> 8;
  const int ol = (tid >> 2) & 63;
  const int i = tid & 3;
  float sum = 0.f;
#pragma unroll
  for (int wv = 0; wv < kGateSmallWaves; ++wv) sum += red[wv][gi][ol][i];
  const int col = ol & 15;
  const int row = r0 + gi * 16 + 4 * (ol >> 4) + i;
  if (col < g.H && row < rows) {
    const float bias = g.b ? g.b[col] : 0.f;
    g.score[((size_t)b * g.H + col) * g.cap + g.slot_begin + row] =
        1.f / (1.f + __expf(-(sum + bias)));
  }
}

// ---------------------------------------------------------------------------
// Low-rank sink-attention gate (Fast KVzip section 3.4) over hidden states.
//
// The projections P = W x for the rows of W_k (16 per KV head) and W_q (16
// per query head) are one GEMM. A workgroup of 8 waves computes 256 tokens x
// 2 HPW KV heads: waves (wr, wc) own tokens 64 wr .. 64 wr + 63 and the
// NTW = HPW (1 + G) 16-row weight tiles of head column wc. The operands move
// from global memory straight into LDS (global_load_lds_dwordx4: lane l's 16
// bytes land at base + 16 l), one 1 KB block per 16-row x 32-k MFMA
// fragment, so the fragment reads are linear and conflict-free. Chunks of
// 32 k go through a 3-stage ring: chunk ch + 2 is requested while chunk ch
// is multiplied (a fourth stage, all 160 KB of LDS, measured no faster). Workgroup ids are mapped so that the head groups of a token
// block run back to back on one XCD and share its hidden states in L2.
//
// The MFMA takes W as A and x as B, so a lane ends with 4 features (rows
// 4 (l / 16) + v) of token l % 16: per-token sums over the 16 features are
// 4 in-lane terms plus two cross-lane steps (lanes l ^ 16, l ^ 32). The 16
// sink logits of a query are a 16 x 16 x 16 fp32 MFMA with the raw q tile as
// B, so lane l gets sinks 4 (l / 16) + i of its token.
// ---------------------------------------------------------------------------
constexpr int kSgTok = 256;       // tokens per workgroup
constexpr int kSgStages = 3;
constexpr float kSgEps = 1e-6f;   // RMS normalisation epsilon

template <int G>
struct SgCfg {
  static constexpr int HPW = 12 / (1 + G);    // heads per wave column
  static constexpr int NTW = HPW * (1 + G);   // weight tiles per wave
  static constexpr int NB = 16 + 2 * NTW;     // 1 KB blocks per chunk
  static constexpr int LPW = (NB + 7) / 8;    // blocks each wave loads
  static constexpr int NBP = 8 * LPW;         // padded: every wave loads LPW
};

__device__ __forceinline__ float xsum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}
__device__ __forceinline__ float xmax(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}

template <int G>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void sink_gate_kernel(SinkGateLaunch g, int nb, int ncg) {
  using C = SgCfg<G>;
  constexpr int NTW = C::NTW, LPW = C::LPW;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kSgStages][C::NBP * 1024];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave & 3;   // token quarter
  const int wc = wave >> 2;  // head column
  const int c = lane & 15;
  const int kq = (lane >> 4) * 8;

  // Block id -> (token block, head group); see the comment above.
  const int id = blockIdx.x;
  const int grp = 8 * ncg;
  const int base = id - id % grp;
  const int rr = id - base;
  const int total = nb * g.batch * ncg;
  int blk, cg;
  if (base + grp <= total) {
    blk = base / ncg + rr % 8;
    cg = rr / 8;
  } else {
    blk = base / ncg + rr / ncg;
    cg = rr % ncg;
  }
  const int b = blk / nb;
  const int tok0 = (blk - b * nb) * kSgTok;
  const int rows = g.slot_end - g.slot_begin;
  const int h0 = cg * 2 * C::HPW;  // first head of the workgroup

  // Source of each block this wave loads (chunk 0). Blocks 0..15: token
  // tiles; 16..NB-1: weight tiles of head columns 0 and 1; past NB: padding
  // (a copy of block 16's source into an unread slot).
  const uint16_t* xb = (const uint16_t*)g.hidden + (size_t)b * g.batch_stride;
  const uint16_t* src[LPW];
#pragma unroll
  for (int s = 0; s < LPW; ++s) {
    const int bi = wave * LPW + s;
    if (bi < 16) {
      const int r = min(tok0 + bi * 16 + c, rows - 1);
      src[s] = xb + (size_t)r * g.in_dim + kq;
    } else {
      const int q = bi < C::NB ? bi - 16 : 0;
      const int col = q / NTW, j = q % NTW;
      const int h = min(h0 + col * C::HPW + j / (1 + G), g.H - 1);
      const int jj = j % (1 + G);
      const size_t grow = jj == 0 ? (size_t)h * 16 + c
                                  : (size_t)g.H * 16 + (size_t)(h * G + jj - 1) * 16 + c;
      src[s] = (const uint16_t*)g.w + grow * g.in_dim + kq;
    }
  }
  const int nch = g.in_dim / 32;
  auto issue = [&](int ch, int stage) {
#pragma unroll
    for (int s = 0; s < LPW; ++s)
      __builtin_amdgcn_global_load_lds(
          (const void*)(src[s] + ch * 32),
          (__attribute__((address_space(3))) void*)&lds[stage][(wave * LPW + s) * 1024],
          16, 0, 0);
  };

  f32x4_t acc[NTW][4];
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[j][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Chunks past the last one re-request the last chunk into a stage nobody
  // reads, so every wave always has LPW loads per chunk in flight and the
  // wait count below is exact.
  constexpr int AHEAD = kSgStages - 1;        // chunks in flight
  constexpr int NWAIT = (AHEAD - 1) * LPW;     // loads allowed to fly on
#pragma unroll
  for (int i = 0; i < AHEAD; ++i) issue(min(i, nch - 1), i);
  int st = 0;
  for (int ch = 0; ch < nch; ++ch) {
    // Own loads of chunk ch done (later chunks' may still fly), then
    // everyone's: the block is complete and the stage read at ch - 1 free.
    // (A bare s_barrier: a fence here would wait for every load.)
    __builtin_amdgcn_s_waitcnt((NWAIT & 15) | ((NWAIT >> 4) << 14) | (7 << 4) | (15 << 8));
    __builtin_amdgcn_s_barrier();
    const int st2 = st == 0 ? kSgStages - 1 : st - 1;  // (ch + AHEAD) % stages
    issue(min(ch + AHEAD, nch - 1), st2);
    const uint8_t* sb = &lds[st][lane * 16];
    bf16x8_t xa[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      xa[t] = __builtin_bit_cast(bf16x8_t, *(const u32x4*)(sb + (wr * 4 + t) * 1024));
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const bf16x8_t wf = __builtin_bit_cast(
          bf16x8_t, *(const u32x4*)(sb + (16 + wc * NTW + j) * 1024));
#pragma unroll
      for (int t = 0; t < 4; ++t)
        acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, xa[t], acc[j][t], 0, 0, 0);
    }
    // Fragment reads run two weight tiles ahead of the MFMAs.
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      if (j + 2 < NTW) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    st = st == kSgStages - 1 ? 0 : st + 1;
  }
  // No load may still be writing this workgroup's LDS when it exits.
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));

  // Epilogue. Lane l: features f_v = 4 (l / 16) + v of token l % 16.
  const int f0 = (lane >> 4) * 4;
  float gk[4], gq[4], sp[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    gk[v] = g.norm ? g.norm[f0 + v] : 1.f;
    gq[v] = g.norm ? g.norm[16 + f0 + v] : 1.f;
    // A operand of the sink MFMA v: row c (sink), k = l / 16 (feature f_v).
    sp[v] = c < g.n_sink ? gq[v] * g.sinks[c * 16 + f0 + v] : 0.f;
  }
  bool sink_ok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) sink_ok[i] = f0 + i < g.n_sink;
#pragma unroll
  for (int hp = 0; hp < C::HPW; ++hp) {
    const int hv = h0 + wc * C::HPW + hp;
    const bool live = hv < g.H;
    const int h = min(hv, g.H - 1);
    float bj[G];
#pragma unroll
    for (int j = 0; j < G; ++j) bj[j] = g.b ? g.b[h * G + j] : 0.f;
    float* out = g.score + ((size_t)b * g.H + h) * g.cap + g.slot_begin;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const f32x4_t kt = acc[hp * (1 + G)][t];
      const float ik = rsqrtf(xsum(kt[0] * kt[0] + kt[1] * kt[1] + kt[2] * kt[2] +
                                   kt[3] * kt[3]) * (1.f / 16.f) + kSgEps);
      float kg[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) kg[v] = gq[v] * gk[v] * kt[v] * ik;
      float best = 0.f;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const f32x4_t qt = acc[hp * (1 + G) + 1 + j][t];
        const float iq = rsqrtf(xsum(qt[0] * qt[0] + qt[1] * qt[1] + qt[2] * qt[2] +
                                     qt[3] * qt[3]) * (1.f / 16.f) + kSgEps);
        const float a = xsum(qt[0] * kg[0] + qt[1] * kg[1] + qt[2] * kg[2] +
                             qt[3] * kg[3]) * iq * 0.25f;
        f32x4_t cs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int v = 0; v < 4; ++v)
          cs = __builtin_amdgcn_mfma_f32_16x16x4f32(sp[v], qt[v], cs, 0, 0, 0);
        float cl[4], m = a;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          cl[i] = sink_ok[i] ? cs[i] * iq * 0.25f : -__builtin_inff();
          m = fmaxf(m, cl[i]);
        }
        m = xmax(m);
        const float e = xsum(__expf(cl[0] - m) + __expf(cl[1] - m) + __expf(cl[2] - m) +
                             __expf(cl[3] - m));
        const float ea = __expf(a - m);
        best = fmaxf(best, ea / (ea + e + bj[j] * __expf(-m)));
      }
      const int r = tok0 + wr * 64 + t * 16 + c;
      if (live && lane < 16 && r < rows) out[r] = best;
    }
  }
}

}  // namespace

hipError_t launch_score_mlp(const MlpLaunch& m, hipStream_t s,
                            bool check_only) {
  const int rows = m.slot_end - m.slot_begin;
  if (rows <= 0) return hipSuccess;
  const dim3 grid((rows + 63) / 64, m.H, m.batch);
  const bool mfma_ok = m.is_bf16 && (m.hidden % 16 == 0) && m.hidden <= 128 &&
                       (m.D == 64 || m.D == 128);
  if (mfma_ok) {
    const long long total = (long long)m.batch * rows;
    // Tiles per wave: the most that still give every CU two workgroups.
    const long long want = 2LL * (m.cus > 0 ? m.cus : 256);
    int tiles = kMlpMaxTiles;
    while (tiles > 1 &&
           (total + kMlpWaves * tiles * 16 - 1) / (kMlpWaves * tiles * 16) *
                   m.H < want)
      tiles = tiles == kMlpMaxTiles ? 2 : 1;
    const long long rpw = kMlpWaves * tiles * 16;
    const long long wgs = (total + rpw - 1) / rpw;
    if (wgs > 0x7fffffffLL) return hipErrorInvalidValue;
    const dim3 mgrid((unsigned)wgs, m.H);
#define KVE_MLP(DD, NBB)                                                     \
  if (m.D == DD && m.hidden == NBB * 16) {                                   \
    if (check_only) return hipSuccess;                                       \
    if (tiles == kMlpMaxTiles)                                               \
      hipLaunchKernelGGL((mlp_mfma_kernel<DD, NBB, kMlpMaxTiles>), mgrid,    \
                         dim3(256), 0, s, m);                                \
    else if (tiles == 2)                                                     \
      hipLaunchKernelGGL((mlp_mfma_kernel<DD, NBB, 2>), mgrid, dim3(256), 0, \
                         s, m);                                              \
    else                                                                     \
      hipLaunchKernelGGL((mlp_mfma_kernel<DD, NBB, 1>), mgrid, dim3(256), 0, \
                         s, m);                                              \
    return hipGetLastError();                                                \
  }
    KVE_MLP(128, 1) KVE_MLP(128, 2) KVE_MLP(128, 3) KVE_MLP(128, 4)
    KVE_MLP(128, 5) KVE_MLP(128, 6) KVE_MLP(128, 7) KVE_MLP(128, 8)
    KVE_MLP(64, 1) KVE_MLP(64, 2) KVE_MLP(64, 3) KVE_MLP(64, 4)
    KVE_MLP(64, 5) KVE_MLP(64, 6) KVE_MLP(64, 7) KVE_MLP(64, 8)
#undef KVE_MLP
  }
  const size_t lds = (size_t)64 * (2 * m.D + 1) * sizeof(float);
  if (check_only) return hipSuccess;
  if (m.is_bf16) {
    hipLaunchKernelGGL((mlp_valu_kernel<true>), grid, dim3(64), lds, s, m);
  } else {
    hipLaunchKernelGGL((mlp_valu_kernel<false>), grid, dim3(64), lds, s, m);
  }
  return hipGetLastError();
}

hipError_t launch_score_sink_gate(const SinkGateLaunch& g, hipStream_t s,
                                  bool check_only) {
  const int rows = g.slot_end - g.slot_begin;
  if (rows <= 0) return hipSuccess;
  const int nb = (rows + kSgTok - 1) / kSgTok;
  switch (g.G) {
#define KVE_SG(GG)                                                           \
    case GG: {                                                               \
      const int ncg = (g.H + 2 * SgCfg<GG>::HPW - 1) / (2 * SgCfg<GG>::HPW); \
      const long long wgs = (long long)nb * g.batch * ncg;                   \
      if (wgs > 0x7fffffffLL) return hipErrorInvalidValue;                   \
      if (check_only) return hipSuccess;                                     \
      hipLaunchKernelGGL((sink_gate_kernel<GG>), dim3((unsigned)wgs),        \
                         dim3(512), 0, s, g, nb, ncg);                       \
      break;                                                                 \
    }
    KVE_SG(1) KVE_SG(2) KVE_SG(3) KVE_SG(4) KVE_SG(5) KVE_SG(6) KVE_SG(7) KVE_SG(8)
#undef KVE_SG
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_score_gate(const GateLaunch& g, hipStream_t s,
                             bool check_only) {
  const int rows = g.slot_end - g.slot_begin;
  if (rows <= 0) return hipSuccess;
  if (check_only) return hipSuccess;
  if (rows <= kGateSmallMaxRows) {
    const int nblk = (rows + 15) / 16;
    // One XCD (32 CUs) holds them all: group them there (see the kernel).
    const int stride = (long long)nblk * g.batch <= 32 ? 8 : 1;
    hipLaunchKernelGGL(gate_mfma_small_kernel, dim3(nblk * stride, g.batch),
                       dim3(64 * kGateSmallWaves), 0, s, g, stride);
    return hipGetLastError();
  }
  const dim3 grid((rows + kGateRowsPerWG - 1) / kGateRowsPerWG, g.batch);
  hipLaunchKernelGGL(gate_mfma_kernel, grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace kve
