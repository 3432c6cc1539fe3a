// Split-K flash-decode GQA attention over the compact retained cache.
//
// For every batch b, KV head h and query head j = h*G + g (contiguous GQA
// groups: the G query heads of a group share one KV head, KVpop section
// 3.1), decode attention over the len retained rows of the slice (KVpop
// Appendix C: decoding attends directly over the compact cache; Appendix
// D.1, Eq. 27-29: logits <q, k>/sqrt(d_k), log-sum-exp normaliser):
//     out_j = sum_t softmax_t(<q_j, k_t>/sqrt(d)) v_t,  lse_j = log sum_t exp(.)
//
// Decode attention streams every retained K/V row once per step and is
// bound by HBM bandwidth (KV-Kaizen section 1: each decoded token reads the
// whole cache, so decoding is limited by memory bandwidth). At 4 flop/byte
// (G = 4) the q.k and p.v products fit the float32 VALU with room to spare,
// so the design is about keeping enough bytes in flight:
//  * one workgroup = 4 waves = one (split, KV head, batch) triple; each lane
//    owns one 16-byte chunk of a row (16 lanes per bf16 d = 128 row), so one
//    load instruction reads 4 whole 256-byte rows per wave, and every loaded
//    K/V element is used by all G query heads of the group from registers;
//  * software pipelining: each wave holds two stages of 16 rows in
//    registers and issues the loads of the next stage before it computes on
//    the current one;
//  * K/V rows are read with non-temporal loads: each row is used once per
//    launch, and the streaming hint keeps it from being allocated in the
//    caches (measured ~12% faster than plain loads on the batch-96 layer);
//  * q.k partial products with v_dot2_f32_bf16 on the raw bf16 pairs
//    (float32 FMAs for float32 caches), summed over the lanes of a row with
//    DPP (quad_perm, row_half_mirror, row_mirror);
//  * online softmax in base 2, accumulator rescale skipped (wave-uniform)
//    when no running maximum moved; p.v in float32;
//  * no split (direct output) whenever the slices alone fill the chip; else
//    per-workgroup partials (m, l, acc) merged by a separate combine kernel.
//    The split workgroups never synchronise with each other: a device-scope
//    fence on this chip writes back and invalidates the L2 of the issuing
//    XCD, which costs far more than the second launch.
#include <float.h>

#include <type_traits>

#include "kve_internal.h"

namespace kve {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                         0xF, 0xF, false));
}

// Sum over the LPR consecutive lanes that hold one row (LPR a power of 2).
template <int LPR>
__device__ __forceinline__ float sum_row_lanes(float x) {
  if constexpr (LPR >= 2) x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (LPR >= 4) x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (LPR >= 8) x += dpp_mov<0x141>(x);  // row_half_mirror
  if constexpr (LPR >= 16) x += dpp_mov<0x140>(x); // row_mirror
  if constexpr (LPR >= 32) x += __shfl_xor(x, 16);
  if constexpr (LPR >= 64) x += __shfl_xor(x, 32);
  return x;
}

// Value of lane J of this lane's quad.
template <int J>
__device__ __forceinline__ float quad_bcast(float x) {
  return dpp_mov<J * 0x55>(x);
}

// Sums of four per-lane values (one per head of a quad of query heads) over
// the 16 lanes of a row, reduce-scattered: quad lane j = lane & 3 of every
// quad ends up with the full sum of one head (see quad_lane_of_head).
// Two exchange steps inside the quad halve the values each time; two rotations
// by 4 and 8 lanes inside the row add the four quads.
__device__ __forceinline__ float reduce_scatter4(float t0, float t1, float t2,
                                                 float t3, bool odd, bool hi) {
  float a0 = odd ? t2 : t0, b0 = odd ? t0 : t2;
  float a1 = odd ? t3 : t1, b1 = odd ? t1 : t3;
  a0 += dpp_mov<0xB1>(b0);  // partner lane ^ 1
  a1 += dpp_mov<0xB1>(b1);
  float c = hi ? a1 : a0;
  const float d = hi ? a0 : a1;
  c += dpp_mov<0x4E>(d);    // partner lane ^ 2
  c += dpp_mov<0x124>(c);   // row_ror:4
  c += dpp_mov<0x128>(c);   // row_ror:8
  return c;
}
// Quad lane j owns head ((j & 1) << 1) | (j >> 1) after reduce_scatter4; the
// map is its own inverse, so head h sits in quad lane ((h & 1) << 1) | (h >> 1).
constexpr int quad_lane_of_head(int h) { return ((h & 1) << 1) | (h >> 1); }

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

__device__ __forceinline__ bool wave_any(bool p) {
  return __builtin_amdgcn_ballot_w64(p) != 0ull;
}

// Geometry of one kernel instantiation.
template <bool BF16, int D>
struct Geo {
  static constexpr int kEB = BF16 ? 2 : 4;        // bytes per element
  static constexpr int kRowB = D * kEB;           // bytes per row
  static constexpr int kLPR = kRowB / 16;         // lanes per row
  static constexpr int kEPL = 16 / kEB;           // elements per lane
  static constexpr int kRPL = 64 / kLPR;          // rows per wave load
  static constexpr int kU = (BF16 ? 16 : 8) / kRPL;  // loads per lane per stage
  static constexpr int kWaveRows = kRPL * kU;     // rows per wave per stage
  static constexpr int kStageRows = kWaves * kWaveRows;
  static_assert(kLPR >= 1 && kLPR <= 64 && kU >= 1, "unsupported row size");
};

template <int U>
struct Stage {
  u32x4 k[U];
  u32x4 v[U];
};

template <bool BF16, int D, int G>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnLaunch a) {
  using Gm = Geo<BF16, D>;
  constexpr int LPR = Gm::kLPR, EPL = Gm::kEPL, RPL = Gm::kRPL, U = Gm::kU;
  constexpr int ROWB = Gm::kRowB;

  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rslot = lane / LPR;  // which of the RPL rows of a load
  const int sub = lane % LPR;    // which 16-byte chunk of the row
  const int Hq = a.H * G;
  const size_t slice = (size_t)b * a.H + h;
  const int r_begin = split * a.rows_per_split;
  const int r_end = min(a.len, r_begin + a.rows_per_split);

  const char* kbase = (const char*)a.k + slice * (size_t)a.cap * ROWB;
  const char* vbase = (const char*)a.v + slice * (size_t)a.cap * ROWB;
  const int new_slot = a.new_slot;
  const char* knew = nullptr;
  const char* vnew = nullptr;
  // Fused append: the workgroup whose rows contain the new slot stores the
  // new row into the cache (and, for hidden-state scorers, the workgroup of
  // KV head 0 copies the token's hidden state into the pending-token buffer
  // of its batch row). No thread of this launch reads that slot from the
  // cache: the row is read straight from k_new / v_new below. The row is
  // loaded here and stored after the output, so its memory latency overlaps
  // the stream instead of delaying it; the hidden state (kilobytes, too many
  // registers to hold through the stream) is copied after the output.
  constexpr int NV = ROWB / 16;
  const bool appends = new_slot >= 0 && new_slot >= r_begin && new_slot < r_end;
  u32x4 app = {0u, 0u, 0u, 0u};
  if (new_slot >= 0) {
    knew = (const char*)a.k_new + slice * ROWB;
    vnew = (const char*)a.v_new + slice * ROWB;
    if (appends) {
      if (tid < NV) {
        app = ((const u32x4*)knew)[tid];
      } else if (tid < 2 * NV) {
        app = ((const u32x4*)vnew)[tid - NV];
      }
    }
  }

  // This lane's chunk of every query head of the group (same element order
  // as the K chunk it loads). Logits are taken in base 2. Float32 q rows are
  // scaled here; bf16 sums are scaled afterwards (rscale: the factor still
  // to apply to a raw q.k sum).
  const float qscale = kLog2e * rsqrtf((float)D);
  const float rscale = BF16 ? qscale : 1.f;
  u32x4 qv[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const char* qrow =
        (const char*)a.q + ((size_t)b * Hq + (size_t)h * G + g) * ROWB;
    qv[g] = *(const u32x4*)(qrow + sub * 16);
    if constexpr (!BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        qv[g][i] = __float_as_uint(__uint_as_float(qv[g][i]) * qscale);
    }
  }

  // Reduce-scatter path: 16 lanes per row and whole quads of query heads.
  // Each lane then owns one head of every quad for the softmax bookkeeping.
  constexpr bool RS = (LPR == 16) && (G % 4 == 0);
  constexpr int NQ = RS ? G / 4 : 1;   // quads of query heads
  constexpr int NS = RS ? NQ : G;      // softmax states per lane
  const bool odd = (lane & 1) != 0;
  const bool hi = (lane & 2) != 0;

  // Running maximum (raw q.k in the reduce-scatter path, base-2 scaled logit
  // otherwise), normaliser and accumulators.
  float m[NS], l[NS], acc[G][EPL];
#pragma unroll
  for (int c = 0; c < NS; ++c) {
    m[c] = -FLT_MAX;
    l[c] = 0.f;
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;

  const int nrows = r_end - r_begin;
  const int n_stages = (nrows + Gm::kStageRows - 1) / Gm::kStageRows;
  const int row0 = r_begin + wave * Gm::kWaveRows + rslot;

  using Full = std::integral_constant<bool, false>;
  using Masked = std::integral_constant<bool, true>;

  // Loads of one stage. The appended row (if any) is the last row of the
  // slice, so it can only fall in the last stage of the last split: only
  // that stage (MASK) clamps rows to r_end and reads the new row from k_new /
  // v_new; full stages address the slice with 32-bit offsets.
  const uint32_t lane_off =
      (uint32_t)(wave * Gm::kWaveRows + rslot) * ROWB + (uint32_t)sub * 16;
  auto load = [&](Stage<U>& st, int s, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (MASK) {
        const int row = row0 + s * Gm::kStageRows + u * RPL;
        const int rc = row < r_end ? row : r_end - 1;  // clamp: in bounds
        const char* kr = (rc == new_slot) ? knew : kbase + (size_t)rc * ROWB;
        const char* vr = (rc == new_slot) ? vnew : vbase + (size_t)rc * ROWB;
        st.k[u] = __builtin_nontemporal_load((const u32x4*)(kr + sub * 16));
        st.v[u] = __builtin_nontemporal_load((const u32x4*)(vr + sub * 16));
      } else {
        const uint32_t off = (uint32_t)(r_begin + s * Gm::kStageRows + u * RPL) *
                                 ROWB + lane_off;
        st.k[u] = __builtin_nontemporal_load((const u32x4*)(kbase + off));
        st.v[u] = __builtin_nontemporal_load((const u32x4*)(vbase + off));
      }
    }
  };

  // This lane's partial q.k of row u for head g (its 16-byte chunk).
  auto partial_dot = [&](const Stage<U>& st, int u, int g) {
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // Copy the vector elements to scalars before the bit casts: a bit
      // cast applied directly to an ext_vector element lvalue reads
      // element 0 with this compiler.
      const uint32_t kw = st.k[u][i];
      const uint32_t qw = qv[g][i];
      if constexpr (BF16) {
        t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qw),
                                            __builtin_bit_cast(bf16x2_t, kw),
                                            t, false);
      } else {
        t = fmaf(__uint_as_float(qw), __uint_as_float(kw), t);
      }
    }
    return t;
  };

  auto v_floats = [&](const Stage<U>& st, int u, float (&vf)[EPL]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = st.v[u][i];
      if constexpr (BF16) {
        vf[2 * i] = __uint_as_float(w << 16);
        vf[2 * i + 1] = __uint_as_float(w & 0xffff0000u);
      } else {
        vf[i] = __uint_as_float(w);
      }
    }
  };

  // One stage of rows. MASK: some rows of the stage may lie past r_end (only
  // the last stage of a workgroup).
  auto compute = [&](const Stage<U>& st, int s, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      ok[u] = !MASK || (row0 + s * Gm::kStageRows + u * RPL < r_end);
    if constexpr (RS) {
      // Scores of the owned heads, q.k as summed (the factor rscale > 0
      // still owed to them is applied inside the exponentials).
      float sc[U][NQ];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
          const float t = reduce_scatter4(
              partial_dot(st, u, 4 * c), partial_dot(st, u, 4 * c + 1),
              partial_dot(st, u, 4 * c + 2), partial_dot(st, u, 4 * c + 3),
              odd, hi);
          sc[u][c] = ok[u] ? t : -INFINITY;
        }
      float p[U][NQ], alpha[NQ];
      bool moved = false;
#pragma unroll
      for (int c = 0; c < NQ; ++c) {
        float mx = m[c];
#pragma unroll
        for (int u = 0; u < U; ++u) mx = fmaxf(mx, sc[u][c]);
        moved |= (mx != m[c]);
        alpha[c] = fast_exp2((m[c] - mx) * rscale);
        const float nmx = -mx * rscale;
        float lsum = l[c] * alpha[c];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          p[u][c] = fast_exp2(fmaf(sc[u][c], rscale, nmx));
          lsum += p[u][c];
        }
        l[c] = lsum;
        m[c] = mx;
      }
      if (wave_any(moved)) {
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
          const float al[4] = {quad_bcast<quad_lane_of_head(0)>(alpha[c]),
                               quad_bcast<quad_lane_of_head(1)>(alpha[c]),
                               quad_bcast<quad_lane_of_head(2)>(alpha[c]),
                               quad_bcast<quad_lane_of_head(3)>(alpha[c])};
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[4 * c + j][e] *= al[j];
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float vf[EPL];
        v_floats(st, u, vf);
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
          const float pb[4] = {quad_bcast<quad_lane_of_head(0)>(p[u][c]),
                               quad_bcast<quad_lane_of_head(1)>(p[u][c]),
                               quad_bcast<quad_lane_of_head(2)>(p[u][c]),
                               quad_bcast<quad_lane_of_head(3)>(p[u][c])};
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < EPL; ++e)
              acc[4 * c + j][e] = fmaf(pb[j], vf[e], acc[4 * c + j][e]);
        }
      }
    } else {
      // Every lane keeps all G heads: full row sums by DPP.
      float sc[U][G];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float t = sum_row_lanes<LPR>(partial_dot(st, u, g));
          t *= rscale;
          sc[u][g] = ok[u] ? t : -INFINITY;
        }
      float p[U][G], alpha[G];
      bool moved = false;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float mx = m[g];
#pragma unroll
        for (int u = 0; u < U; ++u) mx = fmaxf(mx, sc[u][g]);
        alpha[g] = fast_exp2(m[g] - mx);
        moved |= (mx != m[g]);
        m[g] = mx;
        float lsum = l[g] * alpha[g];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          p[u][g] = fast_exp2(sc[u][g] - mx);
          lsum += p[u][g];
        }
        l[g] = lsum;
      }
      if (wave_any(moved)) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha[g];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float vf[EPL];
        v_floats(st, u, vf);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int e = 0; e < EPL; ++e)
            acc[g][e] = fmaf(p[u][g], vf[e], acc[g][e]);
      }
    }
  };

  // Two register stages. The loads inside the loop are unconditional, so
  // every path into the loop header has the same loads outstanding and the
  // compiler waits only for the stage about to be used. Only the last stage
  // can hold rows past r_end.
  Stage<U> sa, sb;
  if (n_stages == 1) {
    load(sa, 0, Masked{});
    compute(sa, 0, Masked{});
  } else {
    load(sa, 0, Full{});
    int s = 0;
    for (; s + 2 < n_stages; s += 2) {
      load(sb, s + 1, Full{});
      compute(sa, s, Full{});
      if (s + 2 == n_stages - 1) {
        load(sa, s + 2, Masked{});
      } else {
        load(sa, s + 2, Full{});
      }
      compute(sb, s + 1, Full{});
    }
    if (s + 1 < n_stages) {
      load(sb, s + 1, Masked{});
      compute(sa, s, Full{});
      compute(sb, s + 1, Masked{});
    } else {
      compute(sa, s, Masked{});
    }
  }

  // Per-head (scaled maximum, normaliser) in every lane.
  float mh[G], lh[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if constexpr (RS) {
      float mv, lv;
      switch (g & 3) {
        case 0: mv = quad_bcast<quad_lane_of_head(0)>(m[g >> 2]);
                lv = quad_bcast<quad_lane_of_head(0)>(l[g >> 2]); break;
        case 1: mv = quad_bcast<quad_lane_of_head(1)>(m[g >> 2]);
                lv = quad_bcast<quad_lane_of_head(1)>(l[g >> 2]); break;
        case 2: mv = quad_bcast<quad_lane_of_head(2)>(m[g >> 2]);
                lv = quad_bcast<quad_lane_of_head(2)>(l[g >> 2]); break;
        default: mv = quad_bcast<quad_lane_of_head(3)>(m[g >> 2]);
                 lv = quad_bcast<quad_lane_of_head(3)>(l[g >> 2]); break;
      }
      mh[g] = mv * rscale;
      lh[g] = lv;
    } else {
      mh[g] = m[g];
      lh[g] = l[g];
    }
  }

  // Merge the 4 * RPL partial states of the workgroup (one per wave and row
  // slot; each holds every head and, across its LPR lanes, every dim)
  // through LDS: per head, the weight of each partial first, then one
  // weighted sum per output element.
  constexpr int NP = kWaves * RPL;
  __shared__ float red[NP][G][D];
  __shared__ float ml[NP][G][2];
  __shared__ float wts[G][NP];
  __shared__ float tot[G][2];
  const int pidx = wave * RPL + rslot;
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) red[pidx][g][sub * EPL + e] = acc[g][e];
    if (sub == 0) {
      ml[pidx][g][0] = mh[g];
      ml[pidx][g][1] = lh[g];
    }
  }
  __syncthreads();
  for (int g = wave; g < G; g += kWaves) {
    // One wave per head: lane i < NP takes partial i.
    const int i = lane;
    const float mi = i < NP ? ml[i][g][0] : -FLT_MAX;
    float M = mi;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float w = i < NP ? fast_exp2(mi - M) : 0.f;
    float L = i < NP ? ml[i][g][1] * w : 0.f;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off);
    if (i < NP) wts[g][i] = w;
    if (i == 0) {
      tot[g][0] = M;
      tot[g][1] = L;
    }
  }
  __syncthreads();

  const int nsplit = a.nsplit;
  for (int item = tid; item < G * D; item += kThreads) {
    const int g = item / D;
    const int d = item % D;
    float O = 0.f;
#pragma unroll
    for (int q = 0; q < NP; ++q) O = fmaf(red[q][g][d], wts[g][q], O);
    const float M = tot[g][0], L = tot[g][1];
    const size_t hq = (size_t)b * Hq + (size_t)h * G + g;
    if (nsplit == 1) {
      a.out[hq * D + d] = O / L;
      if (d == 0 && a.lse) a.lse[hq] = (M + log2f(L)) * kLn2;
    } else {
      float* part = a.partial + (hq * nsplit + split) * (D + 2);
      part[d] = O;
      if (d == 0) {
        part[D] = M;
        part[D + 1] = L;
      }
    }
  }

  // Stores of the fused append (payload loaded at the start).
  if (appends) {
    char* ks = (char*)a.k_store + (slice * (size_t)a.cap + new_slot) * ROWB;
    char* vs = (char*)a.v_store + (slice * (size_t)a.cap + new_slot) * ROWB;
    if (tid < NV) {
      ((u32x4*)ks)[tid] = app;
    } else if (tid < 2 * NV) {
      ((u32x4*)vs)[tid - NV] = app;
    } else if (tid == 2 * NV) {
      a.pos[slice * (size_t)a.cap + new_slot] = a.new_pos;
    }
    if (a.hidden_new && h == 0) {
      // Four chunks per thread in flight before their stores.
      constexpr int kHidRegs = 4;
      const int n = a.hidden_bytes / 16;
      const u32x4* hs =
          (const u32x4*)((const char*)a.hidden_new + (size_t)b * a.hidden_bytes);
      u32x4* hd = (u32x4*)((char*)a.hidden_buf +
                           ((size_t)b * a.hidden_rows + a.hidden_row) *
                               a.hidden_bytes);
      for (int i0 = tid; i0 < n; i0 += kHidRegs * kThreads) {
        u32x4 t[kHidRegs];
#pragma unroll
        for (int r = 0; r < kHidRegs; ++r) {
          const int i = i0 + r * kThreads;
          if (i < n) t[r] = hs[i];
        }
#pragma unroll
        for (int r = 0; r < kHidRegs; ++r) {
          const int i = i0 + r * kThreads;
          if (i < n) hd[i] = t[r];
        }
      }
    }
  }
}

// Merge of the split partials: one workgroup per query head, one thread per
// head-dim element; each thread folds the splits in order with the online
// softmax rule (the loads of a batch of splits are independent, so they are
// all in flight at once).
template <int D>
__global__ __launch_bounds__(D) void combine_kernel(AttnLaunch a) {
  const size_t hq = (size_t)blockIdx.y * a.H * a.G + blockIdx.x;
  const int nsplit = a.nsplit;
  const float* part = a.partial + hq * nsplit * (D + 2);
  const int d = threadIdx.x;
  float M = -FLT_MAX, L = 0.f, O = 0.f;
#pragma unroll 16
  for (int s = 0; s < nsplit; ++s) {
    const float* p = part + (size_t)s * (D + 2);
    const float ms = p[D], ls = p[D + 1], os = p[d];
    const float mx = fmaxf(M, ms);
    const float c0 = fast_exp2(M - mx);
    const float c1 = fast_exp2(ms - mx);
    L = L * c0 + ls * c1;
    O = O * c0 + os * c1;
    M = mx;
  }
  a.out[hq * D + d] = O / L;
  if (d == 0 && a.lse) a.lse[hq] = (M + log2f(L)) * kLn2;
}

template <bool BF16, int D, int G>
hipError_t launch_one(const AttnLaunch& a, hipStream_t s, bool check_only) {
  if (check_only) return hipSuccess;
  hipLaunchKernelGGL((attn_kernel<BF16, D, G>), dim3(a.nsplit, a.H, a.batch),
                     dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  hipLaunchKernelGGL((combine_kernel<D>), dim3(a.H * G, a.batch), dim3(D), 0,
                     s, a);
  return hipGetLastError();
}

template <bool BF16, int D>
hipError_t launch_g(const AttnLaunch& a, hipStream_t s, bool check_only) {
  switch (a.G) {
    case 1: return launch_one<BF16, D, 1>(a, s, check_only);
    case 2: return launch_one<BF16, D, 2>(a, s, check_only);
    case 3: return launch_one<BF16, D, 3>(a, s, check_only);
    case 4: return launch_one<BF16, D, 4>(a, s, check_only);
    case 5: return launch_one<BF16, D, 5>(a, s, check_only);
    case 6: return launch_one<BF16, D, 6>(a, s, check_only);
    case 7: return launch_one<BF16, D, 7>(a, s, check_only);
    case 8: return launch_one<BF16, D, 8>(a, s, check_only);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attention(const AttnLaunch& a, hipStream_t s,
                            bool check_only) {
  if (a.nsplit < 1 || a.nsplit > kMaxSplit) return hipErrorInvalidValue;
  if (a.is_bf16) {
    if (a.D == 128) return launch_g<true, 128>(a, s, check_only);
    if (a.D == 64) return launch_g<true, 64>(a, s, check_only);
  } else {
    if (a.D == 128) return launch_g<false, 128>(a, s, check_only);
    if (a.D == 64) return launch_g<false, 64>(a, s, check_only);
  }
  return hipErrorInvalidValue;
}

}  // namespace kve
