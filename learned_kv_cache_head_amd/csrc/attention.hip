// Split-K flash-decode GQA attention over the compact retained cache.
//
// Computes, for every batch b, KV head h and query head j = h*G + g
// (contiguous GQA groups, KVpop section 3.1), the decode attention over the
// len retained rows of the slice (KVpop Appendix C: decoding attends
// directly over the compact cache; Appendix D.1, Eq. 27-29: logits
// <q, k>/sqrt(d_k), log-sum-exp normaliser):
//     out_j = sum_t softmax_t(<q_j, k_t>/sqrt(d)) v_t,   lse_j = log sum_t exp(.)
//
// Decode attention streams every retained K/V row once per step and is
// bound by HBM bandwidth (KV-Kaizen section 1: every decoded token reads
// the whole cache). Design for gfx950:
//  * one workgroup = 4 waves = one (split, KV head, batch) triple; the slice's
//    rows are split over enough workgroups (split-K) to put several
//    workgroups on each of the 256 CUs;
//  * 8 lanes own one 256-byte row (lane i reads 16-byte chunks i and i+8, so
//    every load instruction covers whole 128-byte lines), a wave covers 8
//    rows per load, and every loaded K/V row is used by all G query heads of
//    the group before it is dropped;
//  * q.k partial dot products use v_dot2_f32_bf16 on the raw bf16 pairs
//    (float32 FMAs for float32 caches) and are summed over the 8 lanes with
//    three DPP steps (quad_perm and row_half_mirror);
//  * online softmax in base 2 with a wave-uniform skip of the accumulator
//    rescale when no running maximum moved; P.V in float32;
//  * the per-workgroup partials (m, l, acc) of a slice are merged by the
//    last workgroup to finish (device-scope atomic ticket, self-resetting),
//    so a decode step of one layer is a single launch; a separate combine
//    kernel is kept for comparison.
#include <float.h>

#include "kve_internal.h"

namespace kve {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kLPR = 8;                                 // lanes per row
constexpr int kRowsPerPass = kWaves * (64 / kLPR);      // 32 rows
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <bool BF16>
struct Elem {
  static constexpr int kBytes = BF16 ? 2 : 4;
  static constexpr int kPerChunk = 16 / kBytes;  // elements per 16-byte chunk
};

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                         0xF, 0xF, false));
}

// Sum over the 8 lanes of an aligned lane octet (lane bits 0..2).
__device__ __forceinline__ float sum_octet(float x) {
  x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]: partner lane ^ 1
  x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]: partner lane ^ 2
  x += dpp_mov<0x141>(x);  // row_half_mirror: lane i <-> 7 - i in the octet
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

__device__ __forceinline__ uint32_t wave_any(bool p) {
  return __builtin_amdgcn_ballot_w64(p) != 0ull;
}

// Element e of a lane's register slice sits at head-dim index
// (sub + 8*c) * kPerChunk + j, with c = e / kPerChunk, j = e % kPerChunk.
template <int PER_CHUNK>
__device__ __forceinline__ int dim_of(int sub, int e) {
  return (sub + kLPR * (e / PER_CHUNK)) * PER_CHUNK + (e % PER_CHUNK);
}

template <bool BF16, int D, int G>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnLaunch a) {
  using E = Elem<BF16>;
  constexpr int CE = E::kPerChunk;
  constexpr int NCH = D / CE;        // 16-byte chunks per row
  constexpr int CPL = NCH / kLPR;    // chunks per lane
  constexpr int EPL = CPL * CE;      // elements per lane
  constexpr int ROWB = D * E::kBytes;
  constexpr int U = 2;               // rows per lane octet per iteration
  static_assert(CPL >= 1, "row must span at least one chunk per lane");

  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = lane >> 3;
  const int sub = lane & 7;
  const int H = a.H;
  const int Hq = H * G;
  const size_t slice = (size_t)b * H + h;
  const int r_begin = split * a.rows_per_split;
  const int r_end = min(a.len, r_begin + a.rows_per_split);

  const char* kbase = (const char*)a.k + slice * (size_t)a.cap * ROWB;
  const char* vbase = (const char*)a.v + slice * (size_t)a.cap * ROWB;
  const char* knew = nullptr;
  const char* vnew = nullptr;
  const int new_slot = a.new_slot;
  if (new_slot >= 0) {
    knew = (const char*)a.k_new + slice * ROWB;
    vnew = (const char*)a.v_new + slice * ROWB;
    // Fused append: the workgroup whose rows contain the new slot stores the
    // new row into the cache (no thread of this launch reads it back from
    // there: the row is read straight from k_new / v_new below).
    if (new_slot >= r_begin && new_slot < r_end) {
      constexpr int NV = ROWB / 16;
      char* ks = (char*)a.k_store + (slice * (size_t)a.cap + new_slot) * ROWB;
      char* vs = (char*)a.v_store + (slice * (size_t)a.cap + new_slot) * ROWB;
      if (tid < NV) {
        ((u32x4*)ks)[tid] = ((const u32x4*)knew)[tid];
      } else if (tid < 2 * NV) {
        ((u32x4*)vs)[tid - NV] = ((const u32x4*)vnew)[tid - NV];
      } else if (tid == 2 * NV) {
        a.pos[slice * (size_t)a.cap + new_slot] = a.new_pos;
      }
    }
  }

  // Query registers, same element order as the K chunks a lane loads.
  const float qscale = kLog2e * rsqrtf((float)D);
  uint32_t qw[G][BF16 ? EPL / 2 : 1];
  float qf[G][BF16 ? 1 : EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const char* qrow =
        (const char*)a.q + ((size_t)b * Hq + (size_t)h * G + g) * ROWB;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const u32x4 w = *(const u32x4*)(qrow + (sub + kLPR * c) * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (BF16) {
          qw[g][c * 4 + i] = w[i];
        } else {
          qf[g][c * 4 + i] = __uint_as_float(w[i]) * qscale;
        }
      }
    }
  }

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -FLT_MAX;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
  }

  const int nrows = r_end - r_begin;
  const int n_iter = (nrows + kRowsPerPass * U - 1) / (kRowsPerPass * U);
  const int my0 = r_begin + wave * (64 / kLPR) + grp;

  for (int it = 0; it < n_iter; ++it) {
    u32x4 kc[U][CPL], vc[U][CPL];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = my0 + (it * U + u) * kRowsPerPass;
      ok[u] = row < r_end;
      const int rc = ok[u] ? row : r_end - 1;  // clamp: always in bounds
      const char* kr = (rc == new_slot) ? knew : kbase + (size_t)rc * ROWB;
      const char* vr = (rc == new_slot) ? vnew : vbase + (size_t)rc * ROWB;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        kc[u][c] = *(const u32x4*)(kr + (sub + kLPR * c) * 16);
        vc[u][c] = *(const u32x4*)(vr + (sub + kLPR * c) * 16);
      }
    }

    float s[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float t = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if constexpr (BF16) {
              // Copy the vector element to a scalar before the bit cast:
              // a bit cast applied directly to an ext_vector element lvalue
              // reads element 0 with this compiler.
              const uint32_t kw = kc[u][c][i];
              const uint32_t qv = qw[g][c * 4 + i];
              t = __builtin_amdgcn_fdot2_f32_bf16(
                  __builtin_bit_cast(bf16x2_t, qv),
                  __builtin_bit_cast(bf16x2_t, kw), t, false);
            } else {
              t = fmaf(qf[g][c * 4 + i], __uint_as_float(kc[u][c][i]), t);
            }
          }
        }
        t = sum_octet(t);
        if constexpr (BF16) t *= qscale;
        s[u][g] = ok[u] ? t : -INFINITY;
      }
    }

    float p[U][G];
    bool moved = false;
    float alpha[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = m[g];
#pragma unroll
      for (int u = 0; u < U; ++u) mx = fmaxf(mx, s[u][g]);
      alpha[g] = fast_exp2(m[g] - mx);
      moved |= (mx != m[g]);
      m[g] = mx;
      float lsum = l[g] * alpha[g];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        p[u][g] = fast_exp2(s[u][g] - mx);
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
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (BF16) {
            vf[c * 8 + 2 * i] = bf16lo(vc[u][c][i]);
            vf[c * 8 + 2 * i + 1] = bf16hi(vc[u][c][i]);
          } else {
            vf[c * 4 + i] = __uint_as_float(vc[u][c][i]);
          }
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(p[u][g], vf[e], acc[g][e]);
    }
  }

  // Merge the 8 lane octets of the wave (they hold the same head-dim slice
  // for different rows): butterfly over lane bits 3..5.
#pragma unroll
  for (int off = 8; off < 64; off <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mo = __shfl_xor(m[g], off);
      const float lo = __shfl_xor(l[g], off);
      const float mx = fmaxf(m[g], mo);
      const float a0 = fast_exp2(m[g] - mx);
      const float a1 = fast_exp2(mo - mx);
      l[g] = l[g] * a0 + lo * a1;
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        acc[g][e] = acc[g][e] * a0 + __shfl_xor(acc[g][e], off) * a1;
      m[g] = mx;
    }
  }

  // Merge the waves through LDS; the result is this workgroup's partial.
  __shared__ float red[kWaves][G][D + 2];
  if (grp == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) red[wave][g][dim_of<CE>(sub, e)] = acc[g][e];
      if (sub == 0) {
        red[wave][g][D] = m[g];
        red[wave][g][D + 1] = l[g];
      }
    }
  }
  __syncthreads();

  const int nsplit = a.nsplit;
  for (int item = tid; item < G * D; item += kThreads) {
    const int g = item / D;
    const int d = item % D;
    float M = red[0][g][D];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, red[w][g][D]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = fast_exp2(red[w][g][D] - M);
      L += red[w][g][D + 1] * wt;
      O += red[w][g][d] * wt;
    }
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
  if (nsplit == 1 || !a.fused_combine) return;

  // Last-arriving workgroup of the slice merges the nsplit partials.
  __shared__ int last;
  __threadfence();  // make this workgroup's partial visible device-wide
  __syncthreads();
  if (tid == 0) {
    const unsigned ticket = atomicAdd(&a.counters[slice], 1u);
    last = (ticket == (unsigned)(nsplit - 1));
  }
  __syncthreads();
  if (!last) return;
  __threadfence();  // acquire the other workgroups' partials

  __shared__ float wts[G][256];
  __shared__ float Ms[G], Ls[G];
  for (int g = 0; g < G; ++g) {
    const size_t hq = (size_t)b * Hq + (size_t)h * G + g;
    const float* part = a.partial + hq * nsplit * (D + 2);
    if (tid < 64) {
      float mx = -FLT_MAX;
      for (int s = tid; s < nsplit; s += 64) mx = fmaxf(mx, part[s * (D + 2) + D]);
      for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      float lsum = 0.f;
      for (int s = tid; s < nsplit; s += 64) {
        const float wt = fast_exp2(part[s * (D + 2) + D] - mx);
        wts[g][s] = wt;
        lsum += part[s * (D + 2) + D + 1] * wt;
      }
      for (int off = 32; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off);
      if (tid == 0) {
        Ms[g] = mx;
        Ls[g] = lsum;
      }
    }
  }
  __syncthreads();
  for (int item = tid; item < G * D; item += kThreads) {
    const int g = item / D;
    const int d = item % D;
    const size_t hq = (size_t)b * Hq + (size_t)h * G + g;
    const float* part = a.partial + hq * nsplit * (D + 2);
    float O = 0.f;
    for (int s = 0; s < nsplit; ++s) O += part[s * (D + 2) + d] * wts[g][s];
    a.out[hq * D + d] = O / Ls[g];
    if (d == 0 && a.lse) a.lse[hq] = (Ms[g] + log2f(Ls[g])) * kLn2;
  }
  if (tid == 0) atomicExch(&a.counters[slice], 0u);
}

// Separate merge of the split partials (one workgroup per query head).
template <int D>
__global__ __launch_bounds__(128) void combine_kernel(AttnLaunch a) {
  const int hq_local = blockIdx.x;  // 0 .. H*G-1
  const int b = blockIdx.y;
  const int Hq = a.H * a.G;
  const size_t hq = (size_t)b * Hq + hq_local;
  const int nsplit = a.nsplit;
  const float* part = a.partial + hq * nsplit * (D + 2);
  __shared__ float wts[256];
  __shared__ float ML[2];
  const int tid = threadIdx.x;
  if (tid < 64) {
    float mx = -FLT_MAX;
    for (int s = tid; s < nsplit; s += 64) mx = fmaxf(mx, part[s * (D + 2) + D]);
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    float lsum = 0.f;
    for (int s = tid; s < nsplit; s += 64) {
      const float wt = fast_exp2(part[s * (D + 2) + D] - mx);
      wts[s] = wt;
      lsum += part[s * (D + 2) + D + 1] * wt;
    }
    for (int off = 32; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off);
    if (tid == 0) {
      ML[0] = mx;
      ML[1] = lsum;
    }
  }
  __syncthreads();
  for (int d = tid; d < D; d += 128) {
    float O = 0.f;
    for (int s = 0; s < nsplit; ++s) O += part[s * (D + 2) + d] * wts[s];
    a.out[hq * D + d] = O / ML[1];
    if (d == 0 && a.lse) a.lse[hq] = (ML[0] + log2f(ML[1])) * kLn2;
  }
}

template <bool BF16, int D>
hipError_t launch_g(const AttnLaunch& a, hipStream_t s) {
  dim3 grid(a.nsplit, a.H, a.batch);
  switch (a.G) {
#define KVE_CASE(GG)                                                      \
  case GG:                                                                \
    hipLaunchKernelGGL((attn_kernel<BF16, D, GG>), grid, dim3(kThreads), 0, \
                       s, a);                                             \
    break;
    KVE_CASE(1) KVE_CASE(2) KVE_CASE(3) KVE_CASE(4)
    KVE_CASE(5) KVE_CASE(6) KVE_CASE(7) KVE_CASE(8)
#undef KVE_CASE
    default:
      return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.nsplit > 1 && !a.fused_combine) {
    hipLaunchKernelGGL((combine_kernel<D>), dim3(a.H * a.G, a.batch),
                       dim3(128), 0, s, a);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

hipError_t launch_attention(const AttnLaunch& a, hipStream_t s) {
  if (a.nsplit < 1 || a.nsplit > 256) return hipErrorInvalidValue;
  if (a.is_bf16) {
    if (a.D == 128) return launch_g<true, 128>(a, s);
    if (a.D == 64) return launch_g<true, 64>(a, s);
  } else {
    if (a.D == 128) return launch_g<false, 128>(a, s);
    if (a.D == 64) return launch_g<false, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace kve
