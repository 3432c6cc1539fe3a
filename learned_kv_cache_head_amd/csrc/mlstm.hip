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
// holds column w*CPW + l%CPW for the RPG rows of row group l/CPW. Every wave
// keeps the whole normaliser z, ZPL rows per lane.
#include "kve_internal.h"

namespace kve {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kChunk = 32;        // tokens per chunk (two 16-row MFMA tiles)
constexpr float kRescale = 30.f;  // renormalise when log i - m exceeds this

__device__ __forceinline__ bf16x8_t load8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *(const u32x4*)p);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ float wave_min(float x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x = fminf(x, __shfl_xor(x, off));
  return x;
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
__global__ __launch_bounds__(256) void mlstm_kernel(MlstmLaunch p) {
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
  __shared__ float part[kChunk][4];                // per-wave score parts
  __shared__ int tab[kChunk];                      // read-out slots

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

  // Scan-phase lane coordinates and the state.
  const int jj = lane % CPW;
  const int grp = lane / CPW;
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
  __syncthreads();

  for (int c0 = 0; c0 < rows; c0 += kChunk) {
    const int nt = min(kChunk, rows - c0);
    // Read-out rows whose token precedes this call live below slot_begin;
    // find them by position.
    const int u0 = A0 + c0 - p.delay;  // position read out by chunk token 0
    const bool need_lookup = (n0 + c0 + nt - 1 >= p.delay) && u0 < A0;
    if (tid < kChunk) tab[tid] = -1;
    __syncthreads();
    if (need_lookup) {
      for (int s = tid; s < p.slot_begin; s += 256) {
        const int d = pos[s] - u0;
        if (d >= 0 && d < kChunk) tab[d] = s;
      }
    }
    __syncthreads();
    // Chunk token t: absorbed slot, read-out slot (-1: no read-out).
    auto absorb_slot = [&](int t) { return p.slot_begin + c0 + min(t, nt - 1); };
    auto readout_slot = [&](int t) {
      if (t >= nt || n0 + c0 + t < p.delay) return -1;
      const int u = u0 + t;
      return u >= A0 ? p.slot_begin + (u - A0) : tab[t];
    };

    // --- 1. projections on MFMA -------------------------------------------
    {
      const int rtile = wave & 1;          // 16-row tile of the chunk
      const bool absorb = wave < 2;
      const int t = rtile * 16 + (lane & 15);
      int slot = absorb ? absorb_slot(t) : readout_slot(t);
      if (slot < 0) slot = absorb_slot(0);  // in bounds; result unused
      const uint16_t* krow = kc + (size_t)slot * D;
      const uint16_t* vrow = vc + (size_t)slot * D;
      const int kq = (lane >> 4) * 8;
      bf16x8_t a[KSTEPS];
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
        a[ks] = ks < KHALF ? load8(krow + ks * 32 + kq)
                           : load8(vrow + (ks - KHALF) * 32 + kq);
      const int ncol = lane & 15;
      // Output columns wrow0 .. wrow0+15 (weight rows) for the 16 tokens.
      auto tile = [&](int wrow0) {
        f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          const bf16x8_t B = __builtin_bit_cast(
              bf16x8_t, *(const u32x4*)(ws + (wrow0 + ncol) * LSTR + ks * 32 + kq));
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], B, acc, 0, 0, 0);
        }
        return acc;
      };
      const int r0 = rtile * 16 + 4 * (lane >> 4);  // rows r0 .. r0+3
      if (absorb) {
#pragma unroll
        for (int ct = 0; ct < PT; ++ct) {
          const f32x4_t yk = tile(P + ct * 16);
          const f32x4_t yv = tile(2 * P + ct * 16);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            kf[r0 + i][ct * 16 + ncol] = yk[i];
            vf[r0 + i][ct * 16 + ncol] = yv[i];
          }
        }
        // Rows 3P and 3P+1 (w_i, w_f) are columns 14 and 15 of the tile
        // that starts at row 3P - 14; its other 14 columns repeat W_v rows.
        const f32x4_t yg = tile(3 * P - 14);
        if (ncol >= 14) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (ncol == 14) gi[r0 + i] = yg[i] + bi;
            else gf[r0 + i] = yg[i] + bfg;
          }
        }
      } else {
#pragma unroll
        for (int ct = 0; ct < PT; ++ct) {
          const f32x4_t yq = tile(ct * 16);
#pragma unroll
          for (int i = 0; i < 4; ++i) qf[r0 + i][ct * 16 + ncol] = yq[i];
        }
      }
    }
    __syncthreads();

    // --- 2. Hedgehog features: [softmax(y); softmax(-y)] ------------------
    for (int item = wave; item < 2 * kChunk; item += 4) {
      float* row = item < kChunk ? kf[item] : qf[item - kChunk];
      const bool live = lane < P;
      const float y = live ? row[lane] : 0.f;
      const float mx = wave_max(live ? y : -__builtin_inff());
      const float mn = wave_min(live ? y : __builtin_inff());
      const float e1 = live ? __expf(y - mx) : 0.f;
      const float e2 = live ? __expf(mn - y) : 0.f;
      const float s1 = wave_sum(e1);
      const float s2 = wave_sum(e2);
      if (live) {
        row[lane] = e1 / s1;
        row[P + lane] = e2 / s2;
      }
    }
    __syncthreads();

    // --- 3. sequential scan --------------------------------------------------
    for (int t = 0; t < nt; ++t) {
      const float li = gi[t];
      const float af = gf[t];
      // log sigmoid(af) = -softplus(-af)
      const float lf = -(fmaxf(-af, 0.f) + log1pf(__expf(-fabsf(af))));
      float e;
      if (n == 0) {
        m = li;
        e = 0.f;
      } else {
        m += lf;
        e = li - m;
        if (e > kRescale) {
          const float s = __expf(-e);
#pragma unroll
          for (int r = 0; r < RPG; ++r) c[r] *= s;
#pragma unroll
          for (int q = 0; q < ZPL; ++q) z[q] *= s;
          m = li;
          e = 0.f;
        }
      }
      const float wgt = __expf(e);
      const float wv = wgt * vf[t][col];
      const float* kr = kf[t] + grp * RPG;
#pragma unroll
      for (int r = 0; r < RPG; r += 4) {
        const float4 k4 = *(const float4*)(kr + r);
        c[r] = fmaf(k4.x, wv, c[r]);
        c[r + 1] = fmaf(k4.y, wv, c[r + 1]);
        c[r + 2] = fmaf(k4.z, wv, c[r + 2]);
        c[r + 3] = fmaf(k4.w, wv, c[r + 3]);
      }
#pragma unroll
      for (int q = 0; q < ZPL; ++q) z[q] = fmaf(wgt, kf[t][lane * ZPL + q], z[q]);
      const int idx = n0 + c0 + t;  // index of this token in the state
      ++n;
      const bool readout = idx >= p.delay && (u0 + t >= A0 || tab[t] >= 0);
      if (readout) {
        const float* qr = qf[t] + grp * RPG;
        float n4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < RPG; r += 4) {
          const float4 q4 = *(const float4*)(qr + r);
          n4[0] = fmaf(q4.x, c[r], n4[0]);
          n4[1] = fmaf(q4.y, c[r + 1], n4[1]);
          n4[2] = fmaf(q4.z, c[r + 2], n4[2]);
          n4[3] = fmaf(q4.w, c[r + 3], n4[3]);
        }
        float num = (n4[0] + n4[1]) + (n4[2] + n4[3]);
#pragma unroll
        for (int off = CPW; off < 64; off <<= 1) num += __shfl_xor(num, off);
        float den = 0.f;
#pragma unroll
        for (int q = 0; q < ZPL; ++q) den = fmaf(qf[t][lane * ZPL + q], z[q], den);
        den = wave_sum(den);
        const float hv = num / den;
        float sc = acol * (hv / (1.f + __expf(-hv)));
#pragma unroll
        for (int off = 1; off < CPW; off <<= 1) sc += __shfl_xor(sc, off);
        if (lane == 0) part[t][wave] = sc;
      }
    }
    __syncthreads();
    if (tid < nt) {
      const int slot = readout_slot(tid);
      if (slot >= 0)
        p.score[sbase + slot] =
            ((part[tid][0] + part[tid][1]) + (part[tid][2] + part[tid][3])) + b2;
    }
    // The next chunk rewrites tab, the features and part only after its
    // first barrier.
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

hipError_t launch_score_mlstm(const MlstmLaunch& m, hipStream_t s) {
  if (m.slot_end <= m.slot_begin) return hipSuccess;
  const dim3 grid((unsigned)(m.batch * m.H));
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
