// Stateful mLSTM scorer with delayed readout (KVpop section 3.3 "Stateful
// scorers", Appendix A and E.3-E.4, Eq. 10-11 and 37-42).
//
// Per (batch, KV head) slice and token x_t = [k_t; v_t] (key first):
//   q~_t = phi(W_q x_t), k~_t = phi(W_k x_t), v~_t = W_v x_t     (Eq. 37)
//   phi(y) = [softmax(y); softmax(-y)]              (Hedgehog, Appendix A)
//   i_t = exp(w_i . x_t + b_i), f_t = sigmoid(w_f . x_t + b_f)   (Eq. 40)
//   C_t = f_t C_{t-1} + i_t k~_t v~_t^T, z_t = f_t z_{t-1} + i_t k~_t
// After absorbing the token at position q, the token at position u = q - W
// is scored from the state that has seen q (Eq. 41-42, without the optional
// norm):  h = (q~_u^T C_q) / (q~_u^T z_q),  score = a . SiLU(h) + b.
//
// One workgroup owns one slice for the whole call, so the state lives in
// registers between tokens and crosses HBM once per call (read at the
// start, written at the end). Work goes in chunks of kChunk tokens:
//  1. the projections of the chunk's absorbed tokens (W_k, W_v, gates) and
//     of the tokens they read out (W_q) run on MFMA
//     (v_mfma_f32_16x16x32_bf16, float32 accumulation) against the head's
//     weights, staged once in LDS;
//  2. Hedgehog features in float32, in LDS;
//  3. a sequential scan over the chunk: the rank-1 update of C and z and
//     the readout of the delayed token, all float32.
//
// Numerics: the stored state is (Cs, zs, m) with C = exp(m) Cs and
// z = exp(m) zs. The forget gate only moves m (m += log f); a new token adds
// exp(log i - m) k~ v~^T to Cs. When that exponent would exceed kRescale the
// state is renormalised to m = log i. The readout ratio does not depend on
// the common scale, so h needs no rescaling. This is the stabilised mLSTM
// recurrence in a lazy form: the same values up to float32 rounding.
//
// Register layout of the state: wave w owns CPW = P/4 columns of C; lane l
// holds column w*CPW + l/G for the RPG rows of row group l%G (G = 64/CPW
// groups), so a column's read-out sums over an aligned group of G lanes.
// Every wave keeps the whole normaliser z, ZPL rows per lane.
#include "kve_internal.h"

namespace kve {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kChunk = 32;        // tokens per chunk (two 16-row MFMA tiles)
constexpr float kRescale = 30.f;  // renormalise when exponents pass m + this
constexpr float kSpread = 40.f;   // chunks whose gate exponents spread wider
                                  // renormalise token by token

__device__ __forceinline__ bf16x8_t load8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *(const u32x4*)p);
}

// Lane exchanges within 16-lane rows (DPP): quad_perm [1,0,3,2] = 0xB1,
// [2,3,0,1] = 0x4E, row_half_mirror = 0x141, row_mirror = 0x140.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                         0xF, 0xF, false));
}
__device__ __forceinline__ float lane_of(float x, int l) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}
// Sum over the aligned group of N = 4, 8 or 16 lanes, in every lane of it.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  if constexpr (N >= 8) x += dpp<0x141>(x);
  if constexpr (N >= 16) x += dpp<0x140>(x);
  return x;
}
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  return fmaxf(x, dpp<0x140>(x));
}
__device__ __forceinline__ float row_min16(float x) {
  x = fminf(x, dpp<0xB1>(x));
  x = fminf(x, dpp<0x4E>(x));
  x = fminf(x, dpp<0x141>(x));
  return fminf(x, dpp<0x140>(x));
}
// Sum over the wave, as a wave-uniform value: row sums, then the four rows.
__device__ __forceinline__ float wave_total(float x) {
  x = group_sum<16>(x);
  return (lane_of(x, 0) + lane_of(x, 16)) + (lane_of(x, 32) + lane_of(x, 48));
}
__device__ __forceinline__ float wave_max(float x) {
  x = row_max16(x);
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float wave_min(float x) {
  x = row_min16(x);
  x = fminf(x, __shfl_xor(x, 16));
  return fminf(x, __shfl_xor(x, 32));
}

template <int D>
struct MlstmGeo {
  static constexpr int P = D / 2;          // projection width
  static constexpr int F = D;              // Hedgehog feature width 2P
  static constexpr int IN = 2 * D;         // [k; v]
  static constexpr int NOUT = 3 * P + 2;   // W_q, W_k, W_v rows, w_i, w_f
  static constexpr int LSTR = IN + 8;      // bf16 per staged weight row
  static constexpr int KSTEPS = IN / 32;
  static constexpr int KHALF = D / 32;
  static constexpr int PT = P / 16;        // 16-column tiles per projection
  static constexpr int CPW = P / 4;        // state columns per wave
  static constexpr int G = 64 / CPW;       // row groups per wave
  static constexpr int RPG = F / G;        // state rows per lane
  static constexpr int ZPL = F / 64;       // normaliser rows per lane
  static constexpr int STRIDE = F * P + F + 64;  // floats of state per slice
};

template <int D>
// One workgroup per CU (the LDS holds the head weights): let the compiler use
// the registers of one wave per SIMD to keep loads in flight.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mlstm_kernel(MlstmLaunch p) {
  using Geo = MlstmGeo<D>;
  constexpr int P = Geo::P, F = Geo::F, IN = Geo::IN, LSTR = Geo::LSTR;
  constexpr int KSTEPS = Geo::KSTEPS, KHALF = Geo::KHALF, PT = Geo::PT;
  constexpr int CPW = Geo::CPW, RPG = Geo::RPG, ZPL = Geo::ZPL;
  constexpr int NOUT = Geo::NOUT;

  __shared__ uint16_t ws[NOUT * LSTR];             // W_q; W_k; W_v; w_i; w_f
  __shared__ __align__(16) float kf[kChunk][F];    // k~ of absorbed tokens
  __shared__ __align__(16) float qf[kChunk][F];    // q~ of read-out tokens
  __shared__ float vf[kChunk][P];                  // v~ of absorbed tokens
  __shared__ float gi[kChunk], gf[kChunk];         // gate preactivations
  __shared__ float part[kChunk][P + 1];            // a_j SiLU(h_j) per token
  __shared__ int tab_slot[kChunk], tab_pos[kChunk];  // position lookup
  __shared__ int rslot[2][kChunk];                 // read-out slot per token

  const int slice = blockIdx.x;
  const int h = slice % p.H;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const size_t sbase = (size_t)slice * p.cap;
  const uint16_t* kc = (const uint16_t*)p.k + sbase * D;
  const uint16_t* vc = (const uint16_t*)p.v + sbase * D;
  const int32_t* pos = p.pos + sbase;
  float* st = p.state + (size_t)slice * Geo::STRIDE;

  // Stage the head's weights.
  const uint16_t* w = (const uint16_t*)p.w + (size_t)h * NOUT * IN;
  for (int c = tid; c < NOUT * IN / 8; c += 256) {
    const int n = c / (IN / 8);
    const int k8 = c % (IN / 8);
    *(u32x4*)(ws + n * LSTR + k8 * 8) = *(const u32x4*)(w + (size_t)n * IN + k8 * 8);
  }
  const float bi = p.b ? p.b[2 * h] : 0.f;
  const float bfg = p.b ? p.b[2 * h + 1] : 0.f;
  const float b2 = p.b2 ? p.b2[h] : 0.f;
  if (tid < kChunk) tab_pos[tid] = -1;
  __syncthreads();  // before the first lookup writes tab_pos

  // Scan-phase lane coordinates and the state.
  constexpr int G = Geo::G;
  const int jj = lane / G;
  const int grp = lane % G;
  const int col = wave * CPW + jj;
  const float acol = p.a[(size_t)h * P + col];
  float c[RPG];
#pragma unroll
  for (int r = 0; r < RPG; ++r) c[r] = st[r * 256 + tid];
  float z[ZPL];
#pragma unroll
  for (int e = 0; e < ZPL; ++e) z[e] = st[RPG * 256 + lane * ZPL + e];
  float m = st[RPG * 256 + F];
  int n = __float_as_int(st[RPG * 256 + F + 1]);

  const int rows = p.slot_end - p.slot_begin;
  const int A0 = pos[p.slot_begin];  // position of the first absorbed token
  const int n0 = n;                  // tokens absorbed before this call

  // MFMA roles: waves 0-1 project the chunk's absorbed tokens (16 each),
  // waves 2-3 the tokens those read out.
  const int rtile = wave & 1;
  const bool absorb = wave < 2;
  const int kq = (lane >> 4) * 8;
  const int ncol = lane & 15;

  // Read-outs of the chunk at c0 whose token precedes this call sit below
  // slot_begin: record their slots by position.
  auto lookup = [&](int c0) {
    const int nt = min(kChunk, rows - c0);
    const int u0 = A0 + c0 - p.delay;
    if (u0 < A0 && n0 + c0 + nt - 1 >= p.delay) {
      for (int s = tid; s < p.slot_begin; s += 256) {
        const int ps = pos[s];
        const int d = ps - u0;
        if (d >= 0 && d < kChunk) {
          tab_slot[d] = s;
          tab_pos[d] = ps;
        }
      }
    }
  };
  // Issue this lane's MFMA operand loads for the chunk at c0; the read-out
  // waves also record the slot each token reads out (-1: none).
  auto load_a = [&](bf16x8_t (&a)[KSTEPS], int c0, int buf) {
    const int nt = min(kChunk, rows - c0);
    const int t = rtile * 16 + (lane & 15);
    int slot;
    if (absorb) {
      slot = p.slot_begin + c0 + min(t, nt - 1);
    } else {
      slot = -1;
      if (t < nt && n0 + c0 + t >= p.delay) {
        const int u = A0 + c0 - p.delay + t;
        if (u >= A0) slot = p.slot_begin + (u - A0);
        else if (tab_pos[t] == u) slot = tab_slot[t];
      }
      if (lane < 16) rslot[buf][t] = slot;
      if (slot < 0) slot = p.slot_begin;  // in bounds; result unused
    }
    const uint16_t* krow = kc + (size_t)slot * D;
    const uint16_t* vrow = vc + (size_t)slot * D;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      a[ks] = ks < KHALF ? load8(krow + ks * 32 + kq)
                         : load8(vrow + (ks - KHALF) * 32 + kq);
  };
  // Output columns wrow0 .. wrow0+15 (weight rows) for the 16 tokens.
  auto tile = [&](const bf16x8_t (&a)[KSTEPS], int wrow0) {
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const bf16x8_t B = __builtin_bit_cast(
          bf16x8_t, *(const u32x4*)(ws + (wrow0 + ncol) * LSTR + ks * 32 + kq));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], B, acc, 0, 0, 0);
    }
    return acc;
  };
  // Hedgehog features of the 4 tokens this lane holds (rows r0..r0+3 of
  // the P projected columns: 16 per tile, spread over a 16-lane row) into
  // dst[token][0..2P).
  auto hedgehog = [&](const f32x4_t (&y)[PT], float (*dst)[F], int r0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mx = y[0][i], mn = y[0][i];
#pragma unroll
      for (int ct = 1; ct < PT; ++ct) {
        mx = fmaxf(mx, y[ct][i]);
        mn = fminf(mn, y[ct][i]);
      }
      mx = row_max16(mx);
      mn = row_min16(mn);
      float e1[PT], e2[PT], s1 = 0.f, s2 = 0.f;
#pragma unroll
      for (int ct = 0; ct < PT; ++ct) {
        e1[ct] = __expf(y[ct][i] - mx);
        e2[ct] = __expf(mn - y[ct][i]);
        s1 += e1[ct];
        s2 += e2[ct];
      }
      const float i1 = 1.f / group_sum<16>(s1);
      const float i2 = 1.f / group_sum<16>(s2);
#pragma unroll
      for (int ct = 0; ct < PT; ++ct) {
        dst[r0 + i][ct * 16 + ncol] = e1[ct] * i1;
        dst[r0 + i][P + ct * 16 + ncol] = e2[ct] * i2;
      }
    }
  };

  bf16x8_t a[KSTEPS];
  lookup(0);
  __syncthreads();
  load_a(a, 0, 0);

  for (int ci = 0, c0 = 0; c0 < rows; ++ci, c0 += kChunk) {
    const int nt = min(kChunk, rows - c0);
    const int cb = ci & 1;
    const bool more = c0 + kChunk < rows;

    // --- 1. projections on MFMA and Hedgehog features -----------------------
    {
      const int r0 = rtile * 16 + 4 * (lane >> 4);  // tokens r0 .. r0+3
      if (absorb) {
        f32x4_t yk[PT];
#pragma unroll
        for (int ct = 0; ct < PT; ++ct) {
          yk[ct] = tile(a, P + ct * 16);
          const f32x4_t yv = tile(a, 2 * P + ct * 16);
#pragma unroll
          for (int i = 0; i < 4; ++i) vf[r0 + i][ct * 16 + ncol] = yv[i];
        }
        hedgehog(yk, kf, r0);
        // Rows 3P and 3P+1 (w_i, w_f) are columns 14 and 15 of the tile
        // that starts at row 3P - 14; its other 14 columns repeat W_v rows.
        const f32x4_t yg = tile(a, 3 * P - 14);
        if (ncol >= 14) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (ncol == 14) gi[r0 + i] = yg[i] + bi;
            else gf[r0 + i] = yg[i] + bfg;
          }
        }
      } else {
        f32x4_t yq[PT];
#pragma unroll
        for (int ct = 0; ct < PT; ++ct) yq[ct] = tile(a, ct * 16);
        hedgehog(yq, qf, r0);
      }
    }
    if (more) lookup(c0 + kChunk);
    __syncthreads();
    // --- 2. the next chunk's operands stay in flight during the scan --------
    if (more) load_a(a, c0 + kChunk, cb ^ 1);

    // --- 3. gate weights of the chunk (every wave; lane = token) ------------
    // With L_t = sum_{j<=t} log f_j over the chunk, the true state after
    // token t is exp(mref + L_t) Cs_t, and token t enters Cs with weight
    // exp(x_t - mref), x_t = log i_t - L_t.
    const int tl = lane & 31;
    const bool tv = tl < nt;
    const float li = tv ? gi[tl] : 0.f;
    const float af = tv ? gf[tl] : 0.f;
    const float lf = tv ? -(fmaxf(-af, 0.f) + log1pf(__expf(-fabsf(af)))) : 0.f;
    float L = lf;
#pragma unroll
    for (int off = 1; off < kChunk; off <<= 1) {
      const float y = __shfl_up(L, off, kChunk);
      if (tl >= off) L += y;
    }
    const float x = tv ? li - L : -__builtin_inff();
    const float xm = wave_max(x);
    const float xn = wave_min(tv ? x : __builtin_inff());

    // --- 4. sequential scan: update, then read out (read-outs of tokens
    // that have none are computed and dropped) ------------------------------
    // Token t's features as this lane needs them: k~ and q~ of its RPG
    // state rows, k~ and q~ of its ZPL normaliser rows, v~ of its column.
    struct Feat {
      float4 k[RPG / 4], q[RPG / 4];
      float kz[ZPL], qz[ZPL];
      float v;
    };
    const float4* kf4 = reinterpret_cast<const float4*>(&kf[0][0]);
    const float4* qf4 = reinterpret_cast<const float4*>(&qf[0][0]);
    auto fetch = [&](int t, Feat& f) {
      const int base = (t * F + grp * RPG) / 4;
#pragma unroll
      for (int r = 0; r < RPG / 4; ++r) {
        f.k[r] = kf4[base + r];
        f.q[r] = qf4[base + r];
      }
#pragma unroll
      for (int q = 0; q < ZPL; ++q) {
        f.kz[q] = kf[t][lane * ZPL + q];
        f.qz[q] = qf[t][lane * ZPL + q];
      }
      f.v = vf[t][col];
    };
    // Absorb token t with weight wgt, then the read-out's column numerator
    // (summed over the row groups) and this lane's normaliser part.
    auto absorb_read = [&](const Feat& f, float wgt, float& num, float& den) {
      const float wv = wgt * f.v;
#pragma unroll
      for (int r = 0; r < RPG / 4; ++r) {
        c[4 * r] = fmaf(f.k[r].x, wv, c[4 * r]);
        c[4 * r + 1] = fmaf(f.k[r].y, wv, c[4 * r + 1]);
        c[4 * r + 2] = fmaf(f.k[r].z, wv, c[4 * r + 2]);
        c[4 * r + 3] = fmaf(f.k[r].w, wv, c[4 * r + 3]);
      }
      den = 0.f;
#pragma unroll
      for (int q = 0; q < ZPL; ++q) {
        z[q] = fmaf(wgt, f.kz[q], z[q]);
        den = fmaf(f.qz[q], z[q], den);
      }
      float n4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < RPG / 4; ++r) {
        n4[0] = fmaf(f.q[r].x, c[4 * r], n4[0]);
        n4[1] = fmaf(f.q[r].y, c[4 * r + 1], n4[1]);
        n4[2] = fmaf(f.q[r].z, c[4 * r + 2], n4[2]);
        n4[3] = fmaf(f.q[r].w, c[4 * r + 3], n4[3]);
      }
      num = group_sum<G>((n4[0] + n4[1]) + (n4[2] + n4[3]));
    };
    // The read-out's term a_j SiLU(num_j / den) of this lane's column j,
    // stored once per column for the sum over columns after the chunk.
    auto score_term = [&](int t, float num, float den) {
      const float hv = num * __builtin_amdgcn_rcpf(wave_total(den));
      const float sc = acol * hv * __builtin_amdgcn_rcpf(1.f + __expf(-hv));
      if (grp == 0) part[t][col] = sc;
    };
    auto rescale = [&](float r) {
#pragma unroll
      for (int q = 0; q < RPG; ++q) c[q] *= r;
#pragma unroll
      for (int q = 0; q < ZPL; ++q) z[q] *= r;
    };

    float mref;
    if (xm - xn <= kSpread) {
      // One reference for the chunk: new weights lie in
      // [exp(-kSpread - kRescale), exp(kRescale)].
      if (n == 0) {
        mref = xm;  // the state is empty (zero)
      } else if (xm > m + kRescale) {
        mref = xm;
        rescale(__expf(m - xm));
      } else {
        mref = m;
      }
      const float wg = tv ? __expf(x - mref) : 0.f;  // 0: no token
      const int ntu = (nt + 3) & ~3;
      // Groups of 4 tokens: the updates run in order, token t+1's features
      // loading during token t; the 4 read-out tails (normaliser sum,
      // SiLU, score sum) are independent and overlap.
      Feat fb[2];
      fetch(0, fb[0]);
      for (int t0 = 0; t0 < ntu; t0 += 4) {
        float nm[4], dn[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          fetch(min(t0 + k + 1, kChunk - 1), fb[(k + 1) & 1]);
          absorb_read(fb[k & 1], lane_of(wg, t0 + k), nm[k], dn[k]);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) score_term(t0 + k, nm[k], dn[k]);
      }
    } else {
      // Steep gates: move the reference token by token when a weight would
      // pass exp(kRescale).
      mref = n == 0 ? lane_of(x, 0) : m;
      for (int t = 0; t < nt; ++t) {
        const float xt = lane_of(x, t);
        if (xt > mref + kRescale) {
          rescale(__expf(mref - xt));
          mref = xt;
        }
        Feat f;
        fetch(t, f);
        float nm, dn;
        absorb_read(f, __expf(xt - mref), nm, dn);
        score_term(t, nm, dn);
      }
    }
    m = mref + lane_of(L, nt - 1);
    n += nt;
    __syncthreads();
    if (tid < nt) {
      const int slot = rslot[cb][tid];
      if (slot >= 0) {
        // sum over the P columns in four interleaved partial sums
        float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < P; j += 4) {
          s4[0] += part[tid][j];
          s4[1] += part[tid][j + 1];
          s4[2] += part[tid][j + 2];
          s4[3] += part[tid][j + 3];
        }
        p.score[sbase + slot] = ((s4[0] + s4[1]) + (s4[2] + s4[3])) + b2;
      }
    }
    // The next chunk writes the features and part only after its first
    // barrier, and rslot[cb] only in its step 2.
  }

#pragma unroll
  for (int r = 0; r < RPG; ++r) st[r * 256 + tid] = c[r];
  if (wave == 0) {
#pragma unroll
    for (int e = 0; e < ZPL; ++e) st[RPG * 256 + lane * ZPL + e] = z[e];
  }
  if (tid == 0) {
    st[RPG * 256 + F] = m;
    st[RPG * 256 + F + 1] = __int_as_float(n);
  }
}

}  // namespace

size_t mlstm_state_floats(int D) {
  if (D == 128) return MlstmGeo<128>::STRIDE;
  if (D == 64) return MlstmGeo<64>::STRIDE;
  return 0;
}

hipError_t launch_score_mlstm(const MlstmLaunch& m, hipStream_t s,
                              bool check_only) {
  if (m.slot_end <= m.slot_begin) return hipSuccess;
  const dim3 grid((unsigned)(m.batch * m.H));
  if (m.D != 128 && m.D != 64) return hipErrorInvalidValue;
  if (check_only) return hipSuccess;
  if (m.D == 128) {
    hipLaunchKernelGGL((mlstm_kernel<128>), grid, dim3(256), 0, s, m);
  } else if (m.D == 64) {
    hipLaunchKernelGGL((mlstm_kernel<64>), grid, dim3(256), 0, s, m);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kve
