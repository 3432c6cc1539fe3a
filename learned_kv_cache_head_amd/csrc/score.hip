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

namespace kve {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t load8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *(const u32x4*)p);
}

__device__ __forceinline__ float activate(float a, int act) {
  if (act == 0) return fmaxf(a, 0.f);
  return a / (1.f + __expf(-a));  // SiLU
}

// ---------------------------------------------------------------------------
// MLP scorer on MFMA (bf16 K/V and W1). A workgroup scores kMlpRowsPerWG
// rows of one KV head, flattened over (batch, slot); the head's W1 is staged
// once in LDS (rows padded by 16 bytes against bank conflicts) and every
// wave loops over kMlpTiles tiles of 16 rows, loading the next tile's [k; v]
// operands before the MFMAs of the current one.
// ---------------------------------------------------------------------------
constexpr int kMlpWaves = 4;
constexpr int kMlpTiles = 4;                       // tiles per wave
constexpr int kMlpRowsPerWG = kMlpWaves * kMlpTiles * 16;

template <int D, int NB>
__global__ __launch_bounds__(256) void mlp_mfma_kernel(MlpLaunch p) {
  constexpr int HID = NB * 16;
  constexpr int IN = 2 * D;
  constexpr int KSTEPS = IN / 32;   // 32-wide contraction steps
  constexpr int KHALF = D / 32;     // steps taken from the key
  constexpr int LSTR = IN + 8;      // bf16 per staged W1 row
  __shared__ uint16_t w1s[HID * LSTR];
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rows = p.slot_end - p.slot_begin;  // rows per slice
  const long long total = (long long)p.batch * rows;
  const long long wg_row0 = (long long)blockIdx.x * kMlpRowsPerWG;

  const uint16_t* w1 = (const uint16_t*)p.w1 + (size_t)h * HID * IN;
  for (int c = tid; c < HID * IN / 8; c += 256) {
    const int n = c / (IN / 8);
    const int k8 = c % (IN / 8);
    *(u32x4*)(w1s + n * LSTR + k8 * 8) =
        *(const u32x4*)(w1 + (size_t)n * IN + k8 * 8);
  }
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
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      a[ks] = ks < KHALF ? load8(krow + ks * 32 + kq)
                         : load8(vrow + (ks - KHALF) * 32 + kq);
  };
  auto compute_tile = [&](const bf16x8_t (&a)[KSTEPS], int t) {
    f32x4_t acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const bf16x8_t B = __builtin_bit_cast(
            bf16x8_t, *(const u32x4*)(w1s + (nb * 16 + ncol) * LSTR +
                                       ks * 32 + kq));
        acc[nb] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], B, acc[nb], 0, 0, 0);
      }
    }
    // Row 4 * (lane >> 4) + i of the tile: second layer over the 16 hidden
    // units of this lane's columns, then summed over the 16 columns.
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        part[i] += activate(acc[nb][i] + bias[nb], p.act) * w2v[nb];
#pragma unroll
    for (int off = 1; off < 16; off <<= 1)
#pragma unroll
      for (int i = 0; i < 4; ++i) part[i] += __shfl_xor(part[i], off);
    if (ncol == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const long long rid = tile_row0(t) + 4 * (lane >> 4) + i;
        if (rid < total) {
          const int b = (int)(rid / rows);
          const int slot = p.slot_begin + (int)(rid - (long long)b * rows);
          p.score[((size_t)b * p.H + h) * p.cap + slot] = part[i] + b2;
        }
      }
    }
  };

  bf16x8_t a0[KSTEPS], a1[KSTEPS];
  load_tile(a0, 0);
#pragma unroll
  for (int t = 0; t < kMlpTiles; t += 2) {
    load_tile(a1, t + 1);
    compute_tile(a0, t);
    if (t + 2 < kMlpTiles) load_tile(a0, t + 2);
    compute_tile(a1, t + 1);
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
// Gate scorer on MFMA: one wave = 16 tokens x all H heads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gate_mfma_kernel(GateLaunch g) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rows = g.slot_end - g.slot_begin;
  const int r0 = blockIdx.x * 64 + wave * 16;
  if (r0 >= rows) return;
  const int rrow = r0 + (lane & 15);
  const int rc = rrow < rows ? rrow : rows - 1;
  const uint16_t* x =
      (const uint16_t*)g.hidden + (size_t)b * g.batch_stride + (size_t)rc * g.in_dim;
  const int n = lane & 15;
  const bool has_w = n < g.H;
  const uint16_t* w = (const uint16_t*)g.w + (size_t)(has_w ? n : 0) * g.in_dim;
  const int kq = (lane >> 4) * 8;
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const bf16x8_t zero = __builtin_bit_cast(bf16x8_t, u32x4{0u, 0u, 0u, 0u});
  const int ksteps = g.in_dim / 32;
#pragma unroll 8
  for (int ks = 0; ks < ksteps; ++ks) {
    const int kidx = ks * 32 + kq;
    const bf16x8_t A = load8(x + kidx);
    const bf16x8_t B = has_w ? load8(w + kidx) : zero;
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc, 0, 0, 0);
  }
  if (has_w) {
    const float bias = g.b ? g.b[n] : 0.f;
    float* out = g.score + ((size_t)b * g.H + n) * g.cap + g.slot_begin;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = r0 + 4 * (lane >> 4) + i;
      if (row < rows) out[row] = 1.f / (1.f + __expf(-(acc[i] + bias)));
    }
  }
}

// ---------------------------------------------------------------------------
// Low-rank sink-attention gate (Fast KVzip section 3.4): one wave scores 64
// tokens of one KV head. The projections k = W_k x (D' = 16 outputs) and
// q_j = W_q[j] x (G x 16) of the hidden states run on MFMA, four 16-token
// tiles per wave so each weight fragment serves 64 tokens. In the
// accumulator layout a token's 16 features sit in one 16-lane row, so the
// RMS normalisations and dot products are DPP row sums; the S sink logits
// of a query come from a reduce-scatter over the row (lane c ends with
// sink c's logit).
// ---------------------------------------------------------------------------
constexpr int kSgTiles = 4;        // 16-token tiles per wave
constexpr float kSgEps = 1e-6f;    // RMS normalisation epsilon

template <int CTRL>
__device__ __forceinline__ float dppf(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                         0xF, 0xF, false));
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dppf<0xB1>(x);
  x += dppf<0x4E>(x);
  x += dppf<0x141>(x);
  return x + dppf<0x140>(x);
}
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dppf<0xB1>(x));
  x = fmaxf(x, dppf<0x4E>(x));
  x = fmaxf(x, dppf<0x141>(x));
  return fmaxf(x, dppf<0x140>(x));
}
// p[r] in every lane c of a 16-lane row -> sum over the row of p[c], in
// lane c. The partners c^8, c^7 (row_half_mirror), c^2, c^1 flip bits 3, 2,
// 1, 0 in turn; each step keeps the half of the vector that the lane's bit
// selects and adds the partner's copy of it.
__device__ __forceinline__ float reduce_scatter16(const float (&p)[16], int c) {
  float a8[8], a4[4], a2[2];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const bool up = c & 8;
    const float keep = up ? p[8 + j] : p[j];
    const float send = up ? p[j] : p[8 + j];
    a8[j] = keep + dppf<0x128>(send);      // row_ror:8 = lane c^8
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool up = c & 4;
    const float keep = up ? a8[4 + j] : a8[j];
    const float send = up ? a8[j] : a8[4 + j];
    a4[j] = keep + dppf<0x141>(send);      // row_half_mirror = lane c^7
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const bool up = c & 2;
    const float keep = up ? a4[2 + j] : a4[j];
    const float send = up ? a4[j] : a4[2 + j];
    a2[j] = keep + dppf<0x4E>(send);       // lane c^2
  }
  const bool up = c & 1;
  const float keep = up ? a2[1] : a2[0];
  const float send = up ? a2[0] : a2[1];
  return keep + dppf<0xB1>(send);          // lane c^1
}

// One workgroup: 256 tokens (64 per wave, four 16-token tiles) x HP KV
// heads, i.e. NT = HP (1 + G) 16-column tiles of the projection [k_h; q_j].
// The weight rows of those tiles are staged through LDS in 64-wide k chunks
// (double-buffered, shared by the four waves); each wave reads its own token
// rows straight from global memory one chunk ahead. Workgroup ids are
// mapped so that the head groups of one token block run back to back on the
// same XCD and share its hidden states in that XCD's L2.
constexpr int kSgRowsWG = 256;
constexpr int kSgKC = 64;                    // k chunk
constexpr int kSgRowB = kSgKC * 2 + 16;      // LDS bytes per weight row
// Heads per workgroup for group size G: about 6 column tiles (96
// accumulators a lane), so that two workgroups fit on a CU.
constexpr int sg_heads(int G) { return G >= 5 ? 1 : 6 / (1 + G); }

template <int G, int HP, int WPE = (HP * (1 + G) <= 7 ? 2 : 1)>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void sink_gate_kernel(SinkGateLaunch g, int nb, int ncg) {
  constexpr int NT = HP * (1 + G);
  constexpr int NROWS = NT * 16;
  constexpr int SEGS = NROWS * (kSgKC / 8);  // 16-byte pieces per chunk
  constexpr int SPT = (SEGS + 255) / 256;
  // Rows past NROWS take the stores of the pieces past SEGS (never read),
  // so every thread stores unconditionally.
  constexpr int LROWS = SPT * 256 / (kSgKC / 8);
  __shared__ __attribute__((aligned(16))) uint8_t wl[2][LROWS * kSgRowB];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c = lane & 15;
  const int kq = (lane >> 4) * 8;

  // Block id -> (token block, head group). Within each run of 8 * ncg ids,
  // the ncg head groups of a token block share id % 8 (the XCD).
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
  const int tb = blk - b * nb;
  const int rows = g.slot_end - g.slot_begin;
  const int r0 = tb * kSgRowsWG + wave * 64;

  const uint16_t* xb = (const uint16_t*)g.hidden + (size_t)b * g.batch_stride;
  const uint16_t* xr[kSgTiles];
#pragma unroll
  for (int t = 0; t < kSgTiles; ++t) {
    const int r = min(r0 + t * 16 + c, rows - 1);
    xr[t] = xb + (size_t)r * g.in_dim + kq;
  }
  // Weight pieces this thread stages: LDS row R <- global row of tile R/16.
  const uint16_t* wsrc[SPT];
  int wdst[SPT];
#pragma unroll
  for (int s = 0; s < SPT; ++s) {
    const int seg = min(tid + s * 256, SEGS - 1);
    const int R = seg / (kSgKC / 8);
    const int part = seg % (kSgKC / 8);
    const int Rs = (tid + s * 256) / (kSgKC / 8);  // LDS row of the store
    const int tile = R / 16;
    const int hp = tile / (1 + G);
    const int j = tile % (1 + G);
    const int h = min(cg * HP + hp, g.H - 1);
    const size_t grow = j == 0 ? (size_t)h * 16 + (R & 15)
                               : (size_t)g.H * 16 + (size_t)(h * G + j - 1) * 16 + (R & 15);
    wsrc[s] = (const uint16_t*)g.w + grow * g.in_dim + part * 8;
    wdst[s] = Rs * kSgRowB + part * 16;
  }
  const int nch = (g.in_dim + kSgKC - 1) / kSgKC;
  // A chunk is 64 wide except possibly the last (in_dim % 64 == 32).
  auto full = [&](int ch) { return ch * kSgKC + kSgKC <= g.in_dim; };
  u32x4 wreg[SPT];
  // In a half chunk (in_dim % 64 == 32) the upper 32 columns of the staged
  // weights are zero, so the second k step adds nothing.
  auto load_w = [&](int ch) {
    const int back = full(ch) ? 0 : 32;
#pragma unroll
    for (int s = 0; s < SPT; ++s) {
      const int part = (wdst[s] % kSgRowB) / 16;
      wreg[s] = *(const u32x4*)(wsrc[s] + ch * kSgKC - (part < 4 ? 0 : back));
    }
  };
  auto store_w = [&](int ch, int buf) {
    const bool f = full(ch);
#pragma unroll
    for (int s = 0; s < SPT; ++s) {
      const int part = (wdst[s] % kSgRowB) / 16;
      const u32x4 v = (f || part < 4) ? wreg[s] : u32x4{0u, 0u, 0u, 0u};
      *(u32x4*)(&wl[buf][wdst[s]]) = v;
    }
  };
  bf16x8_t A[2][kSgTiles], An[2][kSgTiles];
  auto load_a = [&](bf16x8_t (&a)[2][kSgTiles], int ch) {
    // In a half chunk the second half repeats the first (in bounds, unused).
    const int hi = full(ch) ? 32 : 0;
#pragma unroll
    for (int t = 0; t < kSgTiles; ++t) {
      a[0][t] = load8(xr[t] + ch * kSgKC);
      a[1][t] = load8(xr[t] + ch * kSgKC + hi);
    }
  };

  f32x4_t acc[kSgTiles][NT];
#pragma unroll
  for (int t = 0; t < kSgTiles; ++t)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[t][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // The first chunk's token rows are requested before its weights, so that
  // the weight store's wait leaves no load in flight when the loop starts.
  load_a(A, 0);
  load_w(0);
  store_w(0, 0);
  __syncthreads();
  for (int ch = 0; ch < nch; ++ch) {
    // Request the next chunk; the last chunk requests itself again (in
    // bounds, unused), so the loads carry no branch and the wait counts
    // stay exact.
    const int nx = min(ch + 1, nch - 1);
    load_w(nx);
    load_a(An, nx);
    // Weight fragments of the second k step are read from LDS while the
    // first step's MFMAs run.
    const uint8_t* wb = wl[ch & 1] + c * kSgRowB + kq * 2;
    bf16x8_t B0[NT], B1[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j)
      B0[j] = __builtin_bit_cast(bf16x8_t, *(const u32x4*)(wb + j * 16 * kSgRowB));
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      B1[j] = __builtin_bit_cast(bf16x8_t, *(const u32x4*)(wb + j * 16 * kSgRowB + 64));
#pragma unroll
      for (int t = 0; t < kSgTiles; ++t)
        acc[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[0][t], B0[j], acc[t][j],
                                                            0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int t = 0; t < kSgTiles; ++t)
        acc[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[1][t], B1[j], acc[t][j],
                                                            0, 0, 0);
    // Into the buffer no wave reads in this chunk (after the last chunk, a
    // copy nobody reads).
    store_w(nx, (ch + 1) & 1);
    // Order: next chunk's global loads, first-step weight reads, first-step
    // MFMAs interleaved with the second step's reads, second-step MFMAs,
    // weight stores.
    __builtin_amdgcn_sched_group_barrier(0x020, SPT + 2 * kSgTiles, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, NT, 0);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, kSgTiles, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kSgTiles * NT, 0);
    __builtin_amdgcn_sched_group_barrier(0x200, SPT, 0);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int t = 0; t < kSgTiles; ++t) A[ks][t] = An[ks][t];
  }

  // Epilogue: lane c holds feature c of 4 tokens per tile.
  const float gk = g.norm ? g.norm[c] : 1.f;
  const float gq = g.norm ? g.norm[16 + c] : 1.f;
  float ks16[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) ks16[r] = r < g.n_sink ? g.sinks[r * 16 + c] : 0.f;
  const float inv_sqrt = 0.25f;  // 1 / sqrt(16)
#pragma unroll
  for (int hp = 0; hp < HP; ++hp) {
    const int h = min(cg * HP + hp, g.H - 1);
    const bool live = cg * HP + hp < g.H;
    float bj[G];
#pragma unroll
    for (int j = 0; j < G; ++j) bj[j] = g.b ? g.b[h * G + j] : 0.f;
    float* out = g.score + ((size_t)b * g.H + h) * g.cap + g.slot_begin;
    // One token (row i of tile t) at a time; the accumulator values are
    // copied out first so that no register array is indexed dynamically.
    auto token = [&](const f32x4_t (&tile)[1 + G], int t, int i) {
      float kc = tile[0][0], qv[G];
      if (i == 1) kc = tile[0][1];
      if (i == 2) kc = tile[0][2];
      if (i == 3) kc = tile[0][3];
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const f32x4_t v = tile[1 + j];
        qv[j] = i == 0 ? v[0] : i == 1 ? v[1] : i == 2 ? v[2] : v[3];
      }
      const float kn = gk * kc * rsqrtf(row_sum16(kc * kc) * (1.f / 16.f) + kSgEps);
      float best = 0.f;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float qc = qv[j];
        const float qn = gq * qc * rsqrtf(row_sum16(qc * qc) * (1.f / 16.f) + kSgEps);
        const float a = row_sum16(qn * kn) * inv_sqrt;
        float pr[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) pr[r] = qn * ks16[r];
        float cs = reduce_scatter16(pr, c) * inv_sqrt;  // sink c's logit
        cs = c < g.n_sink ? cs : -__builtin_inff();
        const float m = fmaxf(a, row_max16(cs));
        const float ssum = row_sum16(__expf(cs - m));
        const float ea = __expf(a - m);
        best = fmaxf(best, ea / (ea + ssum + bj[j] * __expf(-m)));
      }
      const int r = r0 + t * 16 + 4 * (lane >> 4) + i;
      if (live && c == 0 && r < rows) out[r] = best;
    };
#pragma unroll
    for (int t = 0; t < kSgTiles; ++t) {
      f32x4_t ht[1 + G];
#pragma unroll
      for (int j = 0; j <= G; ++j) ht[j] = acc[t][hp * (1 + G) + j];
      for (int i = 0; i < 4; ++i) token(ht, t, i);
    }
  }
}

}  // namespace

hipError_t launch_score_mlp(const MlpLaunch& m, hipStream_t s) {
  const int rows = m.slot_end - m.slot_begin;
  if (rows <= 0) return hipSuccess;
  const dim3 grid((rows + 63) / 64, m.H, m.batch);
  const bool mfma_ok = m.is_bf16 && (m.hidden % 16 == 0) && m.hidden <= 128 &&
                       (m.D == 64 || m.D == 128);
  if (mfma_ok) {
    const long long total = (long long)m.batch * rows;
    const long long wgs = (total + kMlpRowsPerWG - 1) / kMlpRowsPerWG;
    if (wgs > 0x7fffffffLL) return hipErrorInvalidValue;
    const dim3 mgrid((unsigned)wgs, m.H);
#define KVE_MLP(DD, NBB)                                                     \
  if (m.D == DD && m.hidden == NBB * 16) {                                   \
    hipLaunchKernelGGL((mlp_mfma_kernel<DD, NBB>), mgrid, dim3(256), 0, s, m); \
    return hipGetLastError();                                                \
  }
    KVE_MLP(128, 1) KVE_MLP(128, 2) KVE_MLP(128, 3) KVE_MLP(128, 4)
    KVE_MLP(128, 5) KVE_MLP(128, 6) KVE_MLP(128, 7) KVE_MLP(128, 8)
    KVE_MLP(64, 1) KVE_MLP(64, 2) KVE_MLP(64, 3) KVE_MLP(64, 4)
    KVE_MLP(64, 5) KVE_MLP(64, 6) KVE_MLP(64, 7) KVE_MLP(64, 8)
#undef KVE_MLP
  }
  const size_t lds = (size_t)64 * (2 * m.D + 1) * sizeof(float);
  if (m.is_bf16) {
    hipLaunchKernelGGL((mlp_valu_kernel<true>), grid, dim3(64), lds, s, m);
  } else {
    hipLaunchKernelGGL((mlp_valu_kernel<false>), grid, dim3(64), lds, s, m);
  }
  return hipGetLastError();
}

hipError_t launch_score_sink_gate(const SinkGateLaunch& g, hipStream_t s) {
  const int rows = g.slot_end - g.slot_begin;
  if (rows <= 0) return hipSuccess;
  const int nb = (rows + kSgRowsWG - 1) / kSgRowsWG;
  const int hp = sg_heads(g.G);
  const int ncg = (g.H + hp - 1) / hp;
  const long long wgs = (long long)nb * g.batch * ncg;
  if (wgs > 0x7fffffffLL) return hipErrorInvalidValue;
  switch (g.G) {
#define KVE_SG(GG)                                                           \
    case GG:                                                                 \
      hipLaunchKernelGGL((sink_gate_kernel<GG, sg_heads(GG)>),               \
                         dim3((unsigned)wgs), dim3(256), 0, s, g, nb, ncg);  \
      break;
    KVE_SG(1) KVE_SG(2) KVE_SG(3) KVE_SG(4) KVE_SG(5) KVE_SG(6) KVE_SG(7) KVE_SG(8)
#undef KVE_SG
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_score_gate(const GateLaunch& g, hipStream_t s) {
  const int rows = g.slot_end - g.slot_begin;
  if (rows <= 0) return hipSuccess;
  const dim3 grid((rows + 63) / 64, g.batch);
  hipLaunchKernelGGL(gate_mfma_kernel, grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace kve
