// Router: top-k selection, mixing weights, load statistics, and its backward.
//
// The Ultimate MoE Training Handbook, §3.1 Router scoring (Gating function, Output
// scale, Precision: the z-loss) and §3.3 Load balancing (Aux loss, Scope: the
// sequence-wise loss, Loss-free bias: the bias update); the MaxVio statistic of §3.2.
//
// One wavefront per token.  Lane l holds experts e = l + 64*i (i < EPL) in registers, so
// a token's whole score row never leaves registers: k rounds of (local best, 6-step
// butterfly arg-max) pick the experts, the lower index winning ties.  Per-block expert
// histograms and probability sums are written as partials and summed in block order by
// a second kernel: no floating-point atomics, so results are bit-reproducible.
#include <float.h>
#include <limits.h>

#include <type_traits>

#include "moe_internal.h"

namespace moe {

namespace {

// 64 tokens per block: a block's expert histogram is also the permute's chunk histogram,
// so this must equal the permute chunk.
constexpr int kRouterTokensPerBlock = 64;
// Waves per block, by keys per lane: a wave's top-k is a chain of dependent cross-lane
// steps, so more waves per SIMD hide more of it; the count is the most whose registers
// still fit without spilling (16 waves: 128 VGPRs each; 12: 168; 8: 256).
template <int EPL>
constexpr int router_waves() { return EPL <= 4 ? 16 : (EPL == 8 ? 12 : 8); }

// KT: the key type.  Softmax keys are the fp32 logits themselves, so they are compared as
// floats (the same order as in fp64, and one exchange per step instead of two); the
// elementwise scores are fp64.
template <typename KT>
struct Best {
  KT key;
  int e;
  float l;
};

__device__ __forceinline__ bool better(double ka, int ea, double kb, int eb) {
  return ka > kb || (ka == kb && ea < eb);
}
__device__ __forceinline__ bool better(float ka, int ea, float kb, int eb) {
  return ka > kb || (ka == kb && ea < eb);
}
template <typename KT>
__device__ __forceinline__ KT lowest_key() { return sizeof(KT) == 8 ? static_cast<KT>(-DBL_MAX) : static_cast<KT>(-FLT_MAX); }

// fp64 score of one logit for the elementwise gating functions (selection keys and
// weights): sigmoid, or sqrt(softplus) with softplus(l) = max(l, 0) + log(1 + e^-|l|).
__device__ __forceinline__ double score_f64(int score, float lf) {
  const double l = static_cast<double>(lf);
  if (score == MOE_SIGMOID) return 1.0 / (1.0 + exp(-l));
  return sqrt(fmax(l, 0.0) + log1p(exp(-fabs(l))));
}
// fp32 versions for the statistics and the backward.
__device__ __forceinline__ float softplus_f(float l) { return fmaxf(l, 0.0f) + log1pf(__expf(-fabsf(l))); }
__device__ __forceinline__ float score_f32(int score, float l) {
  return score == MOE_SIGMOID ? sigmoid_f(l) : sqrtf(softplus_f(l));
}
// ds/dl: s (1 - s) for sigmoid, sigma(l) / (2 s) for sqrt(softplus).
__device__ __forceinline__ float score_deriv_f32(int score, float l) {
  if (score == MOE_SIGMOID) {
    const float s = sigmoid_f(l);
    return s * (1.0f - s);
  }
  return sigmoid_f(l) / (2.0f * sqrtf(softplus_f(l)));
}

// Per token (one wave): keys, top-k, weights; per block: expert histogram, sums of the
// aux probabilities q (full softmax, or the scores normalised over all E), and the sum of
// logsumexp^2 for the z-loss.  pnorm[t] = (m, 1/Z) so that q_te = exp(l_te - m) / Z
// (softmax) or s(l_te) / Z (normalised scores) can be recomputed by the sequence pass.
template <int EPL, typename KT>
__global__ __launch_bounds__(64 * router_waves<EPL>()) void router_topk_kernel(const float* __restrict__ logits,
                                                          const float* __restrict__ expert_bias,
                                                          int T, int E, int k, int score, int pre_softmax,
                                                          float scaling, int ngroups, int gtopk,
                                                          int32_t* __restrict__ idx, float* __restrict__ w,
                                                          int32_t* __restrict__ cnt_part,
                                                          float* __restrict__ prob_part,
                                                          float* __restrict__ z_part,
                                                          float2* __restrict__ pnorm) {
  extern __shared__ int smem_i[];
  int* hist = smem_i;                                          // [E]
  constexpr int NW = router_waves<EPL>();
  float* red = reinterpret_cast<float*>(smem_i + E);           // [NW][E]
  __shared__ float red_z[NW];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();

  float acc[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) acc[i] = 0.0f;
  float zacc = 0.0f;  // wave-uniform

  const int t0 = blockIdx.x * kRouterTokensPerBlock;
  for (int s = wave; s < kRouterTokensPerBlock; s += NW) {
    const int t = t0 + s;
    if (t >= T) break;
    const float* row = logits + static_cast<int64_t>(t) * E;
    float l[EPL];
    KT key[EPL];
    uint32_t taken = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      if (e < E) {
        l[i] = row[e];
        if (score == MOE_SOFTMAX) {
          key[i] = static_cast<KT>(l[i]);
        } else {
          // s(l) (+ bias) in fp64 from the fp32 values
          const double sc = score_f64(score, l[i]);
          key[i] = static_cast<KT>(expert_bias ? sc + static_cast<double>(expert_bias[e]) : sc);
        }
      } else {
        l[i] = 0.0f;
        key[i] = lowest_key<KT>();
        taken |= 1u << i;
      }
    }
    if (ngroups > 0) {
      // group-limited routing: a group's score is the sum of its m = k / gtopk best keys,
      // added from the largest down; lane g holds group g's score
      const int n = E / ngroups, m = k / gtopk;
      double gsc = -DBL_MAX;
      for (int g = 0; g < ngroups; ++g) {
        uint32_t used = 0;
        double sum = 0.0;
        for (int r = 0; r < m; ++r) {
          double bk = -DBL_MAX;
          int be = INT_MAX;
#pragma unroll
          for (int i = 0; i < EPL; ++i) {
            const int e = lane + 64 * i;
            if (e < E && e / n == g && !(used & (1u << i)) && better(static_cast<double>(key[i]), e, bk, be)) {
              bk = key[i];
              be = e;
            }
          }
#pragma unroll
          for (int o = 32; o >= 1; o >>= 1) {
            const double ok = __shfl_xor(bk, o, 64);
            const int oe = __shfl_xor(be, o, 64);
            if (better(ok, oe, bk, be)) {
              bk = ok;
              be = oe;
            }
          }
          if ((be & 63) == lane) used |= 1u << (be >> 6);
          sum += bk;
        }
        if (lane == g) gsc = sum;
      }
      // keep the gtopk best groups, ties to the lower group index
      uint64_t kept = 0;
      for (int r = 0; r < gtopk; ++r) {
        const bool live = lane < ngroups && !((kept >> lane) & 1ull);
        double bk = live ? gsc : -DBL_MAX;
        int be = live ? lane : INT_MAX;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
          const double ok = __shfl_xor(bk, o, 64);
          const int oe = __shfl_xor(be, o, 64);
          if (better(ok, oe, bk, be)) {
            bk = ok;
            be = oe;
          }
        }
        kept |= 1ull << be;
      }
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        if (e < E && !((kept >> (e / n)) & 1ull)) taken |= 1u << i;
      }
    }
    int my_e = -1;
    float my_l = 0.0f;
    float top_l = 0.0f;
    for (int j = 0; j < k; ++j) {
      Best<KT> b{lowest_key<KT>(), INT_MAX, 0.0f};
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        if (!(taken & (1u << i)) && better(key[i], lane + 64 * i, b.key, b.e)) {
          b.key = key[i];
          b.e = lane + 64 * i;
        }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        KT ok = __shfl_xor(b.key, o, 64);
        int oe = __shfl_xor(b.e, o, 64);
        if (better(ok, oe, b.key, b.e)) {
          b.key = ok;
          b.e = oe;
        }
      }
      // the winner (the same on every lane) is lane b.e % 64's key b.e / 64: its logit
      // comes from that lane once, rather than riding along every exchange above
      float wl = 0.0f;
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if ((b.e >> 6) == i) wl = l[i];
      b.l = __shfl(wl, b.e & 63, 64);
      if ((b.e & 63) == lane) taken |= 1u << (b.e >> 6);
      if (lane == j) {
        my_e = b.e;
        my_l = b.l;
      }
      if (j == 0) top_l = b.l;
    }
    // aux probabilities over all E (and, for softmax, the full-softmax normaliser that the
    // pre-softmax weights use); for softmax top_l is the row maximum
    float q[EPL];
    float m = 0.0f, inv;
    if (score == MOE_SOFTMAX) {
      m = top_l;
      float part = 0.0f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        q[i] = (lane + 64 * i < E) ? expf(l[i] - m) : 0.0f;
        part += q[i];
      }
      const float z = wave_sum(part);
      inv = 1.0f / z;
      if (z_part) zacc += (m + logf(z)) * (m + logf(z));
    } else {
      float part = 0.0f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        q[i] = (lane + 64 * i < E) ? score_f32(score, l[i]) : 0.0f;
        part += q[i];
      }
      inv = 1.0f / (wave_sum(part) + 1e-20f);
      if (z_part) {
        float mx = -FLT_MAX;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          if (lane + 64 * i < E) mx = fmaxf(mx, l[i]);
        mx = wave_max(mx);
        float pe = 0.0f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) pe += (lane + 64 * i < E) ? expf(l[i] - mx) : 0.0f;
        const float lse = mx + logf(wave_sum(pe));
        zacc += lse * lse;
      }
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) acc[i] += q[i] * inv;
    if (pnorm && lane == 0) pnorm[t] = make_float2(m, inv);
    // mixing weights: lane j < k owns slot j
    float wv;
    if (score == MOE_SOFTMAX && pre_softmax) {
      wv = lane < k ? expf(my_l - top_l) * inv : 0.0f;
    } else if (score == MOE_SOFTMAX) {
      float ex = lane < k ? expf(my_l - top_l) : 0.0f;
      float z = wave_sum(ex);
      wv = ex / z;
    } else {
      double sg = lane < k ? score_f64(score, my_l) : 0.0;
      double z = wave_sum(sg);
      wv = static_cast<float>(k > 1 ? sg / (z + 1e-20) : sg);
    }
    if (lane < k) {
      idx[static_cast<int64_t>(t) * k + lane] = my_e;
      w[static_cast<int64_t>(t) * k + lane] = wv * scaling;
      atomicAdd(&hist[my_e], 1);   // integer: order-independent
    }
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) red[wave * E + e] = acc[i];
  }
  if (lane == 0) red_z[wave] = zacc;
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    cnt_part[static_cast<int64_t>(blockIdx.x) * E + e] = hist[e];
    float s = 0.0f;
#pragma unroll
    for (int v = 0; v < NW; ++v) s += red[v * E + e];
    prob_part[static_cast<int64_t>(blockIdx.x) * E + e] = s;
  }
  if (z_part && threadIdx.x == 0) {
    float s = 0.0f;
#pragma unroll
    for (int v = 0; v < NW; ++v) s += red_z[v];
    z_part[blockIdx.x] = s;
  }
}

// Per-sequence statistics for the sequence-wise loss.  Block (c, b): positions
// [64 c, 64 c + 64) of sequence b (tokens t = s * B + b).  Writes that chunk's expert
// histogram and its sums of q_te, recomputed from the logits and pnorm exactly as the
// router computed them.
__global__ __launch_bounds__(256) void seq_stats_kernel(const float* __restrict__ logits,
                                                        const float2* __restrict__ pnorm,
                                                        const int32_t* __restrict__ idx, int E, int k, int S,
                                                        int B, int score, int32_t* __restrict__ cnt_part,
                                                        float* __restrict__ prob_part) {
  extern __shared__ int hist_s[];  // [E]
  const int c = blockIdx.x, b = blockIdx.y, nsc = gridDim.x;
  const int s0 = c * 64, s1 = min(S, s0 + 64);
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist_s[e] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < (s1 - s0) * k; i += blockDim.x) {
    const int64_t t = static_cast<int64_t>(s0 + i / k) * B + b;
    atomicAdd(&hist_s[idx[t * k + i % k]], 1);  // integer: order-independent
  }
  __syncthreads();
  const int64_t out = (static_cast<int64_t>(b) * nsc + c) * E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    float acc = 0.0f;
    // unrolled so that several rows' loads are in flight; the sum keeps its order
#pragma unroll 8
    for (int s = s0; s < s1; ++s) {
      const int64_t t = static_cast<int64_t>(s) * B + b;
      const float l = logits[t * E + e];
      const float2 pn = pnorm[t];
      acc += (score == MOE_SOFTMAX ? expf(l - pn.x) : score_f32(score, l)) * pn.y;
    }
    cnt_part[out + e] = hist_s[e];
    prob_part[out + e] = acc;
  }
}

// seq_counts[b, e] and the sequence-wise loss coeff * E / (k S^2 B) * sum_be counts * P
// (P the sum of q over the sequence), chunk partials summed in chunk order, the products
// in a fixed tree.
__global__ __launch_bounds__(1024) void seq_finalize_kernel(const int32_t* __restrict__ cnt_part,
                                                            const float* __restrict__ prob_part, int nsc, int B,
                                                            int E, int k, int S, float coeff,
                                                            int32_t* __restrict__ seq_counts,
                                                            float* __restrict__ stats) {
  __shared__ double s_dot[1024];
  double dot = 0.0;
  for (int pair = threadIdx.x; pair < B * E; pair += blockDim.x) {
    const int b = pair / E, e = pair - b * E;
    int cnt = 0;
    float P = 0.0f;
    // the chunks in order, 8 of each part's loads in flight before they are added
    const int64_t i0 = static_cast<int64_t>(b) * nsc * E + e;
    int c = 0;
    for (; c + 8 <= nsc; c += 8) {
      int cv[8];
      float pv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        cv[u] = cnt_part[i0 + static_cast<int64_t>(c + u) * E];
        pv[u] = prob_part[i0 + static_cast<int64_t>(c + u) * E];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        cnt += cv[u];
        P += pv[u];
      }
    }
    for (; c < nsc; ++c) {
      cnt += cnt_part[i0 + static_cast<int64_t>(c) * E];
      P += prob_part[i0 + static_cast<int64_t>(c) * E];
    }
    seq_counts[pair] = cnt;
    dot += static_cast<double>(P) * cnt;
  }
  s_dot[threadIdx.x] = dot;
  __syncthreads();
  for (int h = blockDim.x / 2; h > 0; h >>= 1) {
    if (threadIdx.x < h) s_dot[threadIdx.x] += s_dot[threadIdx.x + h];
    __syncthreads();
  }
  if (stats && threadIdx.x == 0) {
    const double Sd = static_cast<double>(S);
    stats[5] = static_cast<float>(s_dot[0] * coeff * E / (static_cast<double>(k) * Sd * Sd * B));
  }
}

// One step of the loss-free bias: exact integer directions, then fp32 steps (one block).
__global__ __launch_bounds__(1024) void bias_update_kernel(const int32_t* __restrict__ counts, int E, float rate,
                                                           int centered, float* __restrict__ bias) {
  __shared__ long long s_tot[1024];
  __shared__ int s_dir[1024];
  long long tot = 0;
  for (int e = threadIdx.x; e < E; e += blockDim.x) tot += counts[e];
  s_tot[threadIdx.x] = tot;
  __syncthreads();
  for (int h = blockDim.x / 2; h > 0; h >>= 1) {
    if (threadIdx.x < h) s_tot[threadIdx.x] += s_tot[threadIdx.x + h];
    __syncthreads();
  }
  const long long total = s_tot[0];
  int dsum = 0;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const long long v = total - static_cast<long long>(counts[e]) * E;
    dsum += (v > 0) - (v < 0);
  }
  s_dir[threadIdx.x] = dsum;
  __syncthreads();
  for (int h = blockDim.x / 2; h > 0; h >>= 1) {
    if (threadIdx.x < h) s_dir[threadIdx.x] += s_dir[threadIdx.x + h];
    __syncthreads();
  }
  const float m = centered ? __fdiv_rn(__fmul_rn(rate, static_cast<float>(s_dir[0])), static_cast<float>(E)) : 0.0f;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const long long v = total - static_cast<long long>(counts[e]) * E;
    float step = __fmul_rn(static_cast<float>((v > 0) - (v < 0)), rate);
    if (centered) step = __fsub_rn(step, m);
    bias[e] = __fadd_rn(bias[e], step);
  }
}

// Column sums of the per-block partials in a fixed order: 1024 threads = 64 experts x 16
// interleaved block subsets, each subset summed in block order, then the 16 subset sums
// added by a fixed pairwise tree.
__global__ __launch_bounds__(1024) void router_finalize_kernel(const int32_t* __restrict__ cnt_part,
                                                               const float* __restrict__ prob_part, int nblk,
                                                               int E, int32_t* __restrict__ counts,
                                                               float* __restrict__ prob_sum) {
  constexpr int R = 16;
  __shared__ int sc[R][64];
  __shared__ float sp[R][64];
  const int c = threadIdx.x & 63, r = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + c;
  int ci = 0;
  float pf = 0.0f;
  if (e < E) {
    for (int b = r; b < nblk; b += R) {
      ci += cnt_part[static_cast<int64_t>(b) * E + e];
      if (prob_part) pf += prob_part[static_cast<int64_t>(b) * E + e];
    }
  }
  sc[r][c] = ci;
  sp[r][c] = pf;
  __syncthreads();
  for (int h = R / 2; h > 0; h >>= 1) {
    if (r < h) {
      sc[r][c] += sc[r + h][c];
      sp[r][c] += sp[r + h][c];
    }
    __syncthreads();
  }
  if (r == 0 && e < E) {
    counts[e] = sc[0][c];
    if (prob_part && prob_sum) prob_sum[e] = sp[0][c];
  }
}

// aux = coeff * E / (k T^2) * sum_e prob_sum[e] * counts[e]  (= coeff * E * sum f_e P_e);
// MaxVio = (max count - mean) / mean; empty experts; max count.  One block, fixed tree.
// z = z_coeff / T * sum of the block partials of logsumexp^2 (NULL: no z-loss); the
// sequence-wise slot is written by seq_finalize_kernel, or zeroed here when that loss is
// off.
__global__ __launch_bounds__(1024) void router_stats_kernel(const int32_t* __restrict__ counts,
                                                            const float* __restrict__ prob_sum, int E, int T,
                                                            int k, float coeff, const float* __restrict__ z_part,
                                                            int nblk, float z_coeff, int seq_on,
                                                            float* __restrict__ stats) {
  __shared__ double s_dot[1024];
  __shared__ double s_z[1024];
  __shared__ int s_max[1024];
  __shared__ int s_empty[1024];
  double dot = 0.0, zs = 0.0;
  int mx = 0, empty = 0;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int c = counts[e];
    dot += static_cast<double>(prob_sum[e]) * c;
    mx = max(mx, c);
    empty += (c == 0);
  }
  if (z_part)
    for (int b = threadIdx.x; b < nblk; b += blockDim.x) zs += z_part[b];
  s_dot[threadIdx.x] = dot;
  s_z[threadIdx.x] = zs;
  s_max[threadIdx.x] = mx;
  s_empty[threadIdx.x] = empty;
  __syncthreads();
  for (int h = blockDim.x / 2; h > 0; h >>= 1) {
    if (threadIdx.x < h) {
      s_dot[threadIdx.x] += s_dot[threadIdx.x + h];
      s_z[threadIdx.x] += s_z[threadIdx.x + h];
      s_max[threadIdx.x] = max(s_max[threadIdx.x], s_max[threadIdx.x + h]);
      s_empty[threadIdx.x] += s_empty[threadIdx.x + h];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double Td = static_cast<double>(T);
    const double mean = Td * k / E;
    stats[0] = static_cast<float>(s_dot[0] * coeff * E / (k * Td * Td));
    stats[1] = static_cast<float>((s_max[0] - mean) / mean);
    stats[2] = static_cast<float>(s_empty[0]);
    stats[3] = static_cast<float>(s_max[0]);
    stats[4] = z_part ? static_cast<float>(z_coeff * s_z[0] / Td) : 0.0f;
    if (!seq_on) stats[5] = 0.0f;
  }
}

// ======================================================================= row-group router
// The router of layers without group-limited routing.  A token is handled by a group of
// LPT lanes (16, 32 or 64): lane g of a group holds the experts e = i * LPT + g, i < KPL,
// so a token's logits are read with coalesced loads and its keys stay in registers.  Each
// lane keeps its three best keys in order (key descending, then index ascending); a
// token's k winners come from k rounds of a group arg-max over the lanes' first entries --
// DPP moves inside a 16-lane row and the gfx950 permlane swaps across rows, no LDS -- after
// which the winning lane drops its first entry, and rescans its keys in the rare round
// where all three are used.  Slot j's winner is kept by lane j of the group (LPT >= k).
namespace rg {

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) { return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false); }
template <int CTRL>
__device__ __forceinline__ float dpp_v(float v) { return __int_as_float(dpp_i<CTRL>(__float_as_int(v))); }
template <int CTRL>
__device__ __forceinline__ double dpp_v(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = dpp_i<CTRL>(static_cast<int>(b));
  const int hi = dpp_i<CTRL>(static_cast<int>(b >> 32));
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
}
// A permlane swap of v with itself: every lane gets its own value in one half of the pair
// and its partner's (W = 16 or 32 lanes away) in the other.
template <int W>
__device__ __forceinline__ void swap_i(int v, int& a, int& b) {
  if constexpr (W == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    a = static_cast<int>(r[0]);
    b = static_cast<int>(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    a = static_cast<int>(r[0]);
    b = static_cast<int>(r[1]);
  }
}
template <int W>
__device__ __forceinline__ void swap_v(float v, float& a, float& b) {
  int ia, ib;
  swap_i<W>(__float_as_int(v), ia, ib);
  a = __int_as_float(ia);
  b = __int_as_float(ib);
}
template <int W>
__device__ __forceinline__ void swap_v(double v, double& a, double& b) {
  const long long x = __double_as_longlong(v);
  int la, lb, ha, hb;
  swap_i<W>(static_cast<int>(x), la, lb);
  swap_i<W>(static_cast<int>(x >> 32), ha, hb);
  a = __longlong_as_double((static_cast<long long>(ha) << 32) | static_cast<unsigned int>(la));
  b = __longlong_as_double((static_cast<long long>(hb) << 32) | static_cast<unsigned int>(lb));
}

// DPP controls: lane ^ 1 and lane ^ 2 (quad permutes), the other quad of each 8 lanes
// (half-row mirror), the other 8 lanes of each 16 (row mirror).  After each step both lanes
// of a pair hold the same value, so the mirrors pair whole reduced blocks.
constexpr int kXor1 = 0xB1, kXor2 = 0x4E, kHalfMirror = 0x141, kMirror = 0x140;

template <int CTRL, typename KT>
__device__ __forceinline__ void argmax_step(KT& k, int& e) {
  const KT ok = dpp_v<CTRL>(k);
  const int oe = dpp_i<CTRL>(e);
  if (better(ok, oe, k, e)) {
    k = ok;
    e = oe;
  }
}
template <int W, typename KT>
__device__ __forceinline__ void argmax_swap(KT& k, int& e) {
  KT ka, kb;
  int ea, eb;
  swap_v<W>(k, ka, kb);
  swap_i<W>(e, ea, eb);
  const bool b_wins = better(kb, eb, ka, ea);
  k = b_wins ? kb : ka;
  e = b_wins ? eb : ea;
}
// (key, index) arg-max over the LPT lanes of each group, the lower index winning ties; the
// result is on every lane of the group.
template <int LPT, typename KT>
__device__ __forceinline__ void group_argmax(KT& k, int& e) {
  argmax_step<kXor1>(k, e);
  argmax_step<kXor2>(k, e);
  argmax_step<kHalfMirror>(k, e);
  argmax_step<kMirror>(k, e);
  if constexpr (LPT >= 32) argmax_swap<16>(k, e);
  if constexpr (LPT == 64) argmax_swap<32>(k, e);
}
// Sum over the LPT lanes of each group (fixed order, the same bits on every lane).
template <int LPT, typename V>
__device__ __forceinline__ V group_sum(V v) {
  v += dpp_v<kXor1>(v);
  v += dpp_v<kXor2>(v);
  v += dpp_v<kHalfMirror>(v);
  v += dpp_v<kMirror>(v);
  V a, b;
  if constexpr (LPT >= 32) {
    swap_v<16>(v, a, b);
    v = a + b;
  }
  if constexpr (LPT == 64) {
    swap_v<32>(v, a, b);
    v = a + b;
  }
  return v;
}
template <int LPT>
__device__ __forceinline__ float group_max(float v) {
  v = fmaxf(v, dpp_v<kXor1>(v));
  v = fmaxf(v, dpp_v<kXor2>(v));
  v = fmaxf(v, dpp_v<kHalfMirror>(v));
  v = fmaxf(v, dpp_v<kMirror>(v));
  float a, b;
  if constexpr (LPT >= 32) {
    swap_v<16>(v, a, b);
    v = fmaxf(a, b);
  }
  if constexpr (LPT == 64) {
    swap_v<32>(v, a, b);
    v = fmaxf(a, b);
  }
  return v;
}
// Sum over the 64 / LPT groups of a wave, lane by lane (lane g of every group gets the sum
// of lane g of all groups).
template <int LPT>
__device__ __forceinline__ float across_groups_sum(float v) {
  float a, b;
  if constexpr (LPT == 16) {
    swap_v<16>(v, a, b);
    v = a + b;
  }
  if constexpr (LPT <= 32) {
    swap_v<32>(v, a, b);
    v = a + b;
  }
  return v;
}

// A lane's three best (key, expert) pairs in order.  insert() takes keys in ascending expert
// order, so a key equal to one already held ranks after it.
template <typename KT>
struct Top3 {
  KT k0, k1, k2;
  int e0, e1, e2;
  __device__ __forceinline__ void clear() {
    k0 = k1 = k2 = lowest_key<KT>();
    e0 = e1 = e2 = INT_MAX;
  }
  __device__ __forceinline__ void insert(KT kv, int ev) {
    const bool c0 = kv > k0, c1 = kv > k1, c2 = kv > k2;
    if (c2) {
      k2 = c1 ? k1 : kv;
      e2 = c1 ? e1 : ev;
    }
    if (c1) {
      k1 = c0 ? k0 : kv;
      e1 = c0 ? e0 : ev;
    }
    if (c0) {
      k0 = kv;
      e0 = ev;
    }
  }
  __device__ __forceinline__ void pop() {
    k0 = k1;
    e0 = e1;
    k1 = k2;
    e1 = e2;
    k2 = lowest_key<KT>();
    e2 = INT_MAX;
  }
};

}  // namespace rg

struct RouterRowArgs {
  const float* logits;
  const float* expert_bias;
  int T, E, k, score, pre_softmax;
  float scaling;
  int32_t* idx;
  float* w;
  int32_t* cnt_part;   // [nblk, E]
  float* prob_part;    // [nblk, E], NULL: the aux probabilities are not summed
  float* z_part;       // [nblk], NULL: no z-loss
  float2* pnorm;       // [T], NULL: no sequence-wise pass
  int32_t* done;       // the finaliser's block counter, reset here
};

namespace rg {

// k rounds of the group arg-max over the lanes' Top3 lists built from key[] (keys of the
// experts i * LPT + g, lowest_key for experts the token does not have).  Lane j of the
// group gets slot j's winner (my_e, my_key); every lane gets the first (top) and the last
// (kth) winner.
template <int LPT, int KPL, typename KT>
__device__ __forceinline__ void select_topk(const KT (&key)[KPL], int g, int E, int k, bool live, int& my_e,
                                            KT& my_key, KT& top_key, KT& kth_key, int& kth_e) {
  // keys the token does not have are lowest_key, which insert() never takes
  Top3<KT> top;
  top.clear();
#pragma unroll
  for (int i = 0; i < KPL; ++i) top.insert(key[i], i * LPT + g);
  my_e = 0;
  my_key = lowest_key<KT>();
  for (int j = 0; j < k; ++j) {
    KT bk = top.k0;
    int be = top.e0;
    group_argmax<LPT>(bk, be);
    if (j == 0) top_key = bk;
    kth_key = bk;
    kth_e = be;
    if (g == j) {
      my_e = be;
      my_key = bk;
    }
    if (top.e0 == be) {
      const KT lk = top.k0;
      const int le = top.e0;
      top.pop();
      if (top.e0 == INT_MAX && j + 1 < k) {
        // all three used: the next three of this lane's keys after the last one taken
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
          const int e = i * LPT + g;
          if (better(lk, le, key[i], e)) top.insert(key[i], e);
        }
      }
    }
  }
}

// DPP moves between neighbouring lanes of a 16-lane row: lane i gets lane i + 1's value
// (row_shl:1) or lane i - 1's (row_shr:1).
constexpr int kFromNext = 0x101, kFromPrev = 0x111;

}  // namespace rg


// KEYS: 0 = the fp32 logits (softmax); 1 = fp64 keys s(l) (+ bias); 2 = sigmoid keys chosen
// on fp32 approximations and confirmed in fp64: the fp32 key of an expert is within
// half of sig_band of its fp64 key, so when no expert outside the fp32 top-k lies within
// sig_band of the k-th fp32 key, the fp32 top-k is the fp64 top-k as a set; the slots are
// then put in fp64 order (a neighbour sort wherever two fp32 keys lie that close), and a
// wave with any token not so separated routes all its tokens on fp64 keys instead.
__device__ __forceinline__ float sig_band(float kth) { return 2.0f * (0x1p-19f + 0x1p-22f * fabsf(kth)); }
__device__ __forceinline__ float sigmoid32(float l) { return __builtin_amdgcn_rcpf(1.0f + __expf(-l)); }

// 64 tokens per block (the permute's chunk, whose histograms it reuses), NW waves; each
// wave routes 64 / LPT tokens per pass.
template <int LPT, int KPL, int NW, int KEYS, bool FULL>
__global__ __launch_bounds__(64 * NW) void router_rows_kernel(const RouterRowArgs a) {
  extern __shared__ int smem_r[];
  const int E = a.E, k = a.k;
  constexpr int TPW = 64 / LPT;
  // LDS: hist [E] | (KEYS 2: each token's logits [NW * TPW][E]) | (KEYS 1, 2: the selection
  // biases [E]) | red [NW][E] (prob sums only)
  int* hist = smem_r;
  float* stage = reinterpret_cast<float*>(smem_r + E);
  float* bias_s = stage + (KEYS == 2 ? NW * TPW * E : 0);
  float* red = bias_s + (KEYS != 0 ? E : 0);
  __shared__ float red_z[NW];
  constexpr int PASSES = kRouterTokensPerBlock / (NW * TPW);
  static_assert(PASSES * NW * TPW == kRouterTokensPerBlock, "a block routes 64 tokens");
  static_assert(KEYS != 2 || LPT == 16, "the fp32-first sigmoid keys sort slots inside one 16-lane row");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane % LPT, grp = lane / LPT;
  // FULL: E == KPL * LPT, so every lane's every key is an expert (no bounds checks)
  const auto inr = [&](int i) { return FULL || i * LPT + g < E; };
  const auto col = [&](int i) { return FULL ? i * LPT + g : min(i * LPT + g, E - 1); };
  const bool softmax = KEYS == 0;
  const bool want_p = a.prob_part != nullptr;
  // the full-E normaliser: aux probabilities, pre-softmax weights, the sequence pass
  const bool want_norm = want_p || a.pnorm != nullptr || (softmax && (a.pre_softmax || a.z_part));
  const auto token = [&](int pass) { return blockIdx.x * kRouterTokensPerBlock + (pass * NW + wave) * TPW + grp; };
  const auto row_of_pass = [&](int pass) {
    const int t = token(pass);
    return a.logits + static_cast<int64_t>(t < a.T ? t : 0) * E;
  };
  // one pass per wave: its logits loads are issued before the LDS set-up and its barrier,
  // so that their latency overlaps the expert biases' loads
  float l0[PASSES == 1 ? KPL : 1];
  if constexpr (PASSES == 1) {
    const float* row = row_of_pass(0);
#pragma unroll
    for (int i = 0; i < KPL; ++i) l0[i] = row[col(i)];
  }
  if (blockIdx.x == 0 && threadIdx.x == 0 && a.done) *a.done = 0;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    hist[e] = 0;
    if (KEYS != 0) bias_s[e] = a.expert_bias ? a.expert_bias[e] : 0.0f;
  }
  __syncthreads();

  float acc[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) acc[i] = 0.0f;
  float zacc = 0.0f;
#pragma unroll 1
  for (int pass = 0; pass < PASSES; ++pass) {
    const int t = token(pass);
    const bool live = t < a.T;
    const float* row = row_of_pass(pass);
    // every load of the token's logits (and biases) is issued before any is used: the
    // addresses are clamped into the row instead of being guarded by branches
    float l[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) l[i] = PASSES == 1 ? l0[i] : row[col(i)];
    float* my_stage = stage + static_cast<int64_t>(wave * TPW + grp) * E;
    if constexpr (KEYS == 2) {
      // the token's logits stay in LDS for the slots' scores below
#pragma unroll
      for (int i = 0; i < KPL; ++i)
        if (inr(i)) my_stage[i * LPT + g] = l[i];
    }
#pragma unroll
    for (int i = 0; i < KPL; ++i)
      if (!(live && inr(i))) l[i] = 0.0f;
    // winners: my_e for lane j < k of the group (slot j); for softmax, top_l is the top-1 logit
    int my_e = 0;
    float my_l = 0.0f, top_l = 0.0f;
    double my_k64 = 0.0, my_s64 = 0.0;   // mode 1, and mode 2's fp64 paths
    bool have_s64 = false;
    if constexpr (KEYS == 1) {
      double key[KPL];
#pragma unroll
      for (int i = 0; i < KPL; ++i)
        key[i] = (live && inr(i))
                     ? score_f64(a.score, l[i]) + static_cast<double>(bias_s[col(i)])
                     : lowest_key<double>();
      double tk, kk;
      int ke;
      rg::select_topk<LPT, KPL, double>(key, g, E, k, live, my_e, my_k64, tk, kk, ke);
      my_e = (g < k && live) ? my_e : 0;
    } else {
      float key[KPL];
#pragma unroll
      for (int i = 0; i < KPL; ++i) {
        const int e = i * LPT + g;
        const float kv = KEYS == 0 ? l[i] : sigmoid32(l[i]) + bias_s[col(i)];
        key[i] = (live && inr(i)) ? kv : lowest_key<float>();
      }
      float my_key, top_key, kth_key;
      int kth_e;
      rg::select_topk<LPT, KPL, float>(key, g, E, k, live, my_e, my_key, top_key, kth_key, kth_e);
      my_e = (g < k && live) ? my_e : 0;
      if constexpr (KEYS == 0) {
        my_l = my_key;
        top_l = top_key;
      } else {
        const float band = sig_band(kth_key);
        bool far = true;   // no unselected expert within the band of the k-th key
#pragma unroll
        for (int i = 0; i < KPL; ++i)
          if (live && better(kth_key, kth_e, key[i], i * LPT + g) && key[i] >= kth_key - band) far = false;
        if (__ballot(!far) != 0) {
          // some token of this wave has an unselected expert that close: fp64 keys for all
          double k64[KPL];
#pragma unroll
          for (int i = 0; i < KPL; ++i)
            k64[i] = (live && inr(i))
                         ? score_f64(MOE_SIGMOID, my_stage[col(i)]) +
                               static_cast<double>(bias_s[col(i)])
                         : lowest_key<double>();
          double tk, kk;
          int ke;
          rg::select_topk<LPT, KPL, double>(k64, g, E, k, live, my_e, my_k64, tk, kk, ke);
          my_e = (g < k && live) ? my_e : 0;
        } else {
          // slots in fp64 order: a neighbour (odd-even) sort where two fp32 keys lie within
          // the band of each other
          const float next_key = __int_as_float(rg::dpp_i<rg::kFromNext>(__float_as_int(my_key)));
          const bool near = g + 1 < k && live && my_key - next_key <= sig_band(my_key);
          if (__ballot(near) != 0) {
            const bool slot = g < k && live;
            my_s64 = slot ? score_f64(MOE_SIGMOID, my_stage[my_e]) : 0.0;
            my_k64 = slot ? my_s64 + static_cast<double>(bias_s[my_e]) : lowest_key<double>();
            have_s64 = true;
            for (int ph = 0; ph < k; ++ph) {
              // both neighbours' values on every lane first: a DPP move reads its source
              // lane only while that lane is active, so none may sit in a divergent branch
              const double kn = rg::dpp_v<rg::kFromNext>(my_k64), kp = rg::dpp_v<rg::kFromPrev>(my_k64);
              const double sn = rg::dpp_v<rg::kFromNext>(my_s64), sp = rg::dpp_v<rg::kFromPrev>(my_s64);
              const int en = rg::dpp_i<rg::kFromNext>(my_e), ep = rg::dpp_i<rg::kFromPrev>(my_e);
              const bool lower = (g & 1) == (ph & 1);
              const double nk = lower ? kn : kp;
              const double ns = lower ? sn : sp;
              const int ne = lower ? en : ep;
              const int partner = lower ? g + 1 : g - 1;
              if (g < k && partner >= 0 && partner < k) {
                const bool pb = better(nk, ne, my_k64, my_e);
                if (lower == pb) {
                  my_k64 = nk;
                  my_s64 = ns;
                  my_e = ne;
                }
              }
            }
          }
        }
      }
    }
    // the full-E normaliser (softmax: exp(l - max), the max being the top-1 logit; other
    // scores: s(l)), and the z-loss's logsumexp of the logits
    float q[KPL];
    float m = 0.0f, inv = 0.0f, lse = 0.0f;
    if (want_norm || a.z_part) {
      if (softmax) {
        m = top_l;
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
          q[i] = (live && inr(i)) ? expf(l[i] - m) : 0.0f;
          part += q[i];
        }
        const float z = rg::group_sum<LPT>(part);
        inv = 1.0f / z;
        lse = m + logf(z);
      } else {
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
          if (KEYS == 2) l[i] = (live && inr(i)) ? my_stage[col(i)] : 0.0f;
          q[i] = (live && inr(i)) ? score_f32(a.score, l[i]) : 0.0f;
          part += q[i];
        }
        inv = 1.0f / (rg::group_sum<LPT>(part) + 1e-20f);
        if (a.z_part) {
          float mx = -FLT_MAX;
#pragma unroll
          for (int i = 0; i < KPL; ++i)
            if (inr(i)) mx = fmaxf(mx, l[i]);
          mx = rg::group_max<LPT>(mx);
          float pe = 0.0f;
#pragma unroll
          for (int i = 0; i < KPL; ++i) pe += (live && inr(i)) ? expf(l[i] - mx) : 0.0f;
          lse = mx + logf(rg::group_sum<LPT>(pe));
        }
      }
      if (want_p && live) {
#pragma unroll
        for (int i = 0; i < KPL; ++i) acc[i] += q[i] * inv;
      }
      if (a.z_part && live && g == 0) zacc += lse * lse;
      if (a.pnorm && live && g == 0) a.pnorm[t] = make_float2(m, inv);
    }
    // mixing weights: lane j < k of the group owns slot j
    const bool slot = g < k && live;
    float wv;
    if constexpr (KEYS == 0) {
      if (a.pre_softmax) {
        wv = slot ? expf(my_l - top_l) * inv : 0.0f;
      } else {
        const float ex = slot ? expf(my_l - top_l) : 0.0f;
        wv = ex / rg::group_sum<LPT>(ex);
      }
    } else if constexpr (KEYS == 1) {
      const double sg = slot ? score_f64(a.score, row[slot ? my_e : 0]) : 0.0;
      const double z = rg::group_sum<LPT>(sg);
      wv = static_cast<float>(k > 1 ? sg / (z + 1e-20) : sg);
    } else {
      // sigmoid scores of the selected experts, renormalised over them (fp32)
      const float sg = slot ? (have_s64 ? static_cast<float>(my_s64) : sigmoid32(my_stage[my_e])) : 0.0f;
      const float z = rg::group_sum<LPT>(sg);
      wv = k > 1 ? sg / (z + 1e-20f) : sg;
    }
    if (slot) {
      a.idx[static_cast<int64_t>(t) * k + g] = my_e;
      a.w[static_cast<int64_t>(t) * k + g] = wv * a.scaling;
      atomicAdd(&hist[my_e], 1);   // integer: order-independent
    }
  }
  if (want_p) {
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const float v = rg::across_groups_sum<LPT>(acc[i]);
      const int e = i * LPT + g;
      if (grp == 0 && e < E) red[wave * E + e] = v;
    }
  }
  if (a.z_part) {
    const float zw = rg::group_sum<64>(zacc);
    if (lane == 0) red_z[wave] = zw;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    a.cnt_part[static_cast<int64_t>(blockIdx.x) * E + e] = hist[e];
    if (want_p) {
      float sum = 0.0f;
#pragma unroll
      for (int v = 0; v < NW; ++v) sum += red[v * E + e];
      a.prob_part[static_cast<int64_t>(blockIdx.x) * E + e] = sum;
    }
  }
  if (a.z_part && threadIdx.x == 0) {
    float sum = 0.0f;
#pragma unroll
    for (int v = 0; v < NW; ++v) sum += red_z[v];
    a.z_part[blockIdx.x] = sum;
  }
}

// Column sums of the router's block partials and then, in the last block to finish, the
// statistics (aux, MaxVio, empty experts, max count, z-loss).  Block x sums the 32 experts
// [32 x, 32 x + 32): thread (r, c) adds the partials of blocks b = r, r + 32, ... of expert
// c in that order, 16 loads in flight, then the 32 subset sums are added by a fixed tree.
// The last block (a counter that router_rows_kernel zeroed, this kernel running after it
// on the stream) reduces the finished sums in a fixed order: no float atomics.
__device__ __forceinline__ int coherent_load(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_load(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kFinCols = 32;

// Block reduction of the per-thread statistics parts of a 1024-thread block (fixed butterfly
// per wave, then the 16 wave results in order by thread 0), and the statistics written by
// thread 0: aux, MaxVio, empty experts, max count, z-loss (and a zero sequence-wise loss
// when that loss is off).
__device__ void router_block_stats(double dot, double zs, int mx, int empty, int E, int T, int k, float coeff,
                                   bool has_z, float z_coeff, int seq_on, float* __restrict__ stats) {
  __shared__ double s_dot[16], s_z[16];
  __shared__ int s_max[16], s_empty[16];
  dot = wave_sum(dot);
  zs = wave_sum(zs);
  for (int o = 32; o >= 1; o >>= 1) {
    mx = max(mx, __shfl_xor(mx, o, 64));
    empty += __shfl_xor(empty, o, 64);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    s_dot[w] = dot;
    s_z[w] = zs;
    s_max[w] = mx;
    s_empty[w] = empty;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double d = 0.0, z = 0.0;
    int m = 0, em = 0;
    for (int i = 0; i < static_cast<int>(blockDim.x >> 6); ++i) {
      d += s_dot[i];
      z += s_z[i];
      m = max(m, s_max[i]);
      em += s_empty[i];
    }
    const double Td = static_cast<double>(T);
    const double mean = Td * k / E;
    stats[0] = static_cast<float>(d * coeff * E / (k * Td * Td));
    stats[1] = static_cast<float>((m - mean) / mean);
    stats[2] = static_cast<float>(em);
    stats[3] = static_cast<float>(m);
    stats[4] = has_z ? static_cast<float>(z_coeff * z / Td) : 0.0f;
    if (!seq_on) stats[5] = 0.0f;
  }
}

__global__ __launch_bounds__(1024) void router_finalize_stats_kernel(
    const int32_t* __restrict__ cnt_part, const float* __restrict__ prob_part, int nblk, int E, int T, int k,
    float coeff, const float* __restrict__ z_part, float z_coeff, int seq_on, int32_t* __restrict__ counts,
    float* __restrict__ prob_sum, float* __restrict__ stats, int32_t* __restrict__ done) {
  constexpr int R = 1024 / kFinCols, U = 16;
  __shared__ int sc[R][kFinCols];
  __shared__ float sp[R][kFinCols];
  __shared__ int s_last;
  const int c = threadIdx.x % kFinCols, r = threadIdx.x / kFinCols;
  const int e = blockIdx.x * kFinCols + c;
  int ci = 0;
  float pf = 0.0f;
  if (e < E) {
    for (int b0 = r; b0 < nblk; b0 += R * U) {
      int v[U];
      float pv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int b = b0 + u * R;
        v[u] = b < nblk ? cnt_part[static_cast<int64_t>(b) * E + e] : 0;
        pv[u] = (prob_part && b < nblk) ? prob_part[static_cast<int64_t>(b) * E + e] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        ci += v[u];
        pf += pv[u];
      }
    }
  }
  sc[r][c] = ci;
  sp[r][c] = pf;
  __syncthreads();
  for (int h = R / 2; h > 0; h >>= 1) {
    if (r < h) {
      sc[r][c] += sc[r + h][c];
      sp[r][c] += sp[r + h][c];
    }
    __syncthreads();
  }
  if (r == 0 && e < E) {
    counts[e] = sc[0][c];
    if (prob_part) prob_sum[e] = sp[0][c];
  }
  if (!stats) return;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_last = atomicAdd(done, 1) == static_cast<int>(gridDim.x) - 1;
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  double dot = 0.0, zs = 0.0;
  int mx = 0, empty = 0;
  for (int x = threadIdx.x; x < E; x += blockDim.x) {
    const int cnt = coherent_load(counts + x);
    if (prob_part) dot += static_cast<double>(coherent_load(prob_sum + x)) * cnt;
    mx = max(mx, cnt);
    empty += (cnt == 0);
  }
  if (z_part)
    for (int b = threadIdx.x; b < nblk; b += blockDim.x) zs += z_part[b];
  router_block_stats(dot, zs, mx, empty, E, T, k, coeff, z_part != nullptr, z_coeff, seq_on, stats);
}

// Small partials (up to kFinOneBlockBytes): one block sums the columns and computes the
// statistics itself, so no block waits for another (no counter, no device-wide fence).
// VEC experts per thread (4: 16-byte loads).  Thread (r, c) adds rows b = r, r + R, ... of
// column group c in that order, 8 loads in flight; expert e's R row sums are then added in
// the order r = 0, 1, ..., R - 1.  The caller guarantees E % VEC == 0 and E / VEC <= 1024.
constexpr size_t kFinOneBlockBytes = 512 * 1024;

template <int VEC>
__global__ __launch_bounds__(1024) void router_finalize_one_block_kernel(
    const int32_t* __restrict__ cnt_part, const float* __restrict__ prob_part, int nblk, int E, int T, int k,
    float coeff, const float* __restrict__ z_part, float z_coeff, int seq_on, int32_t* __restrict__ counts,
    float* __restrict__ prob_sum, float* __restrict__ stats) {
  extern __shared__ int smem_f[];
  constexpr int U = 8;
  const int ncol = E / VEC, R = 1024 / ncol;
  int* sc = smem_f;                                          // [R][E]
  float* sp = reinterpret_cast<float*>(smem_f + R * E);      // [R][E], with prob_part
  const int c = threadIdx.x % ncol, r = threadIdx.x / ncol;
  if (r < R) {
    int ci[VEC];
    float pf[VEC];
#pragma unroll
    for (int q = 0; q < VEC; ++q) {
      ci[q] = 0;
      pf[q] = 0.0f;
    }
    for (int b0 = r; b0 < nblk; b0 += R * U) {
      int v[U][VEC];
      float pv[U][VEC];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int b = b0 + u * R;
        const int64_t o = static_cast<int64_t>(b < nblk ? b : 0) * E + c * VEC;
        if constexpr (VEC == 4) {
          const int4 iv = *reinterpret_cast<const int4*>(cnt_part + o);
          const float4 fv = prob_part ? *reinterpret_cast<const float4*>(prob_part + o) : make_float4(0, 0, 0, 0);
          v[u][0] = iv.x; v[u][1] = iv.y; v[u][2] = iv.z; v[u][3] = iv.w;
          pv[u][0] = fv.x; pv[u][1] = fv.y; pv[u][2] = fv.z; pv[u][3] = fv.w;
        } else {
          v[u][0] = cnt_part[o];
          pv[u][0] = prob_part ? prob_part[o] : 0.0f;
        }
        if (b >= nblk) {
#pragma unroll
          for (int q = 0; q < VEC; ++q) {
            v[u][q] = 0;
            pv[u][q] = 0.0f;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int q = 0; q < VEC; ++q) {
          ci[q] += v[u][q];
          pf[q] += pv[u][q];
        }
    }
#pragma unroll
    for (int q = 0; q < VEC; ++q) {
      sc[r * E + c * VEC + q] = ci[q];
      if (prob_part) sp[r * E + c * VEC + q] = pf[q];
    }
  }
  __syncthreads();
  double dot = 0.0, zs = 0.0;
  int mx = 0, empty = 0;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int cnt = 0;
    float p = 0.0f;
    for (int rr = 0; rr < R; ++rr) {
      cnt += sc[rr * E + e];
      if (prob_part) p += sp[rr * E + e];
    }
    counts[e] = cnt;
    if (prob_part) {
      prob_sum[e] = p;
      dot += static_cast<double>(p) * cnt;
    }
    mx = max(mx, cnt);
    empty += (cnt == 0);
  }
  if (!stats) return;
  if (z_part)
    for (int b = threadIdx.x; b < nblk; b += blockDim.x) zs += z_part[b];
  router_block_stats(dot, zs, mx, empty, E, T, k, coeff, z_part != nullptr, z_coeff, seq_on, stats);
}

// Router backward, one wave per token (see moe_router_bwd in moe.h for the formulas).
struct RouterBwdArgs {
  const float* logits;
  const int32_t* idx;
  const float* w;
  const float* dw;
  const int32_t* counts;
  const int32_t* seq_counts;
  int T, E, k, score, pre_softmax, S, B;
  float scaling, g_aux, g_seq, z_scale, daux;  // g_aux = coeff E / (k T^2), g_seq = coeff E / (k S^2 B),
                                                // z_scale = daux z_coeff 2 / T
  float* dlogits;
};

template <int EPL>
__global__ __launch_bounds__(256) void router_bwd_kernel(const RouterBwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int E = a.E, k = a.k, score = a.score;
  const float* row = a.logits + static_cast<int64_t>(t) * E;
  float val[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) val[i] = 0.0f;

  int my_e = 0;
  float my_w = 0.0f, my_dw = 0.0f;
  if (lane < k) {
    my_e = a.idx[static_cast<int64_t>(t) * k + lane];
    my_w = a.w[static_cast<int64_t>(t) * k + lane];
    my_dw = a.dw[static_cast<int64_t>(t) * k + lane];
  }
  const bool pre = score == MOE_SOFTMAX && a.pre_softmax;
  const bool with_aux = a.counts != nullptr;      // host passes NULL when the term is off
  const bool with_seq = a.seq_counts != nullptr;
  const bool with_z = a.z_scale != 0.0f;
  if (with_aux || with_seq || pre || with_z) {
    float l[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) l[i] = (lane + 64 * i < E) ? row[lane + 64 * i] : 0.0f;
    // softmax of the logits: the aux probabilities of a softmax router, and the z-loss
    float ex[EPL];
    float m = -FLT_MAX, zs = 1.0f;
    if (score == MOE_SOFTMAX || with_z) {
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane + 64 * i < E) m = fmaxf(m, l[i]);
      m = wave_max(m);
      float part = 0.0f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        ex[i] = (lane + 64 * i < E) ? expf(l[i] - m) : 0.0f;
        part += ex[i];
      }
      zs = wave_sum(part);
    }
    // G: the upstream gradient of the aux probabilities q_t
    float G[EPL];
    const int b = with_seq ? t % a.B : 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      float g = 0.0f;
      if (e < E) {
        if (with_aux) g += a.daux * a.g_aux * static_cast<float>(a.counts[e]);
        if (with_seq) g += a.daux * a.g_seq * static_cast<float>(a.seq_counts[static_cast<int64_t>(b) * E + e]);
      }
      G[i] = g;
    }
    if (pre) {
      // w_j = c p_{e_j}: upstream gradient c dw_j at the selected experts
      for (int j = 0; j < k; ++j) {
        const int ej = __shfl(my_e, j, 64);
        const float gj = a.scaling * __shfl(my_dw, j, 64);
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          if (ej == lane + 64 * i) G[i] += gj;
      }
    }
    if (with_aux || with_seq || pre) {
      if (score == MOE_SOFTMAX) {
        const float inv = 1.0f / zs;
        float gq = 0.0f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) gq += G[i] * ex[i] * inv;
        gq = wave_sum(gq);
#pragma unroll
        for (int i = 0; i < EPL; ++i) val[i] += ex[i] * inv * (G[i] - gq);
      } else {
        float sc[EPL];
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
          sc[i] = (lane + 64 * i < E) ? score_f32(score, l[i]) : 0.0f;
          part += sc[i];
        }
        const float inv = 1.0f / (wave_sum(part) + 1e-20f);
        float gq = 0.0f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) gq += G[i] * sc[i] * inv;
        gq = wave_sum(gq);
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          if (lane + 64 * i < E) val[i] += score_deriv_f32(score, l[i]) * (G[i] - gq) * inv;
      }
    }
    if (with_z) {
      const float lse = m + logf(zs);
      const float f = a.z_scale * lse / zs;
#pragma unroll
      for (int i = 0; i < EPL; ++i) val[i] += f * ex[i];
    }
  }

  if (!pre) {
    float dl;
    if (score == MOE_SOFTMAX) {
      const float wdw = wave_sum(lane < k ? my_w * my_dw : 0.0f);
      dl = my_w * my_dw - (my_w / a.scaling) * wdw;
    } else {
      const float lsel = lane < k ? row[my_e] : 0.0f;
      const float s = lane < k ? score_f32(score, lsel) : 0.0f;
      const float sd = lane < k ? score_deriv_f32(score, lsel) : 0.0f;
      if (k > 1) {
        const float z = wave_sum(s) + 1e-20f;
        const float dws = wave_sum(my_dw * s);
        const float ds = (a.scaling / z) * (my_dw - dws / z);
        dl = ds * sd;
      } else {
        dl = a.scaling * my_dw * sd;
      }
    }
    for (int j = 0; j < k; ++j) {
      const int ej = __shfl(my_e, j, 64);
      const float dj = __shfl(dl, j, 64);
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (ej == lane + 64 * i) val[i] += dj;
    }
  }
  float* out = a.dlogits + static_cast<int64_t>(t) * E;
#pragma unroll
  for (int i = 0; i < EPL; ++i)
    if (lane + 64 * i < E) out[lane + 64 * i] = val[i];
}


}  // namespace

int router_epl(int E) {
  int epl = 1;
  while (epl * 64 < E) epl *= 2;
  return epl;
}

int64_t router_num_blocks(int T) { return ceil_div(T, kRouterTokensPerBlock); }

namespace {

template <int EPL, typename KT>
moe_status_t launch_topk_kt(const moe_config_t& c, int nblk, const float* logits, const float* expert_bias,
                            int32_t* idx, float* w, const RouterWs& rw, float* zp, float2* pn, hipStream_t s) {
  const size_t shm = static_cast<size_t>(c.E) * sizeof(int) + static_cast<size_t>(router_waves<EPL>()) * c.E * sizeof(float);
  if (shm > 65536 &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(router_topk_kernel<EPL, KT>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(shm)) != hipSuccess)
    return fail(MOE_ERR_HIP, "router: cannot raise the LDS limit to %zu bytes", shm);
  router_topk_kernel<EPL, KT><<<nblk, 64 * router_waves<EPL>(), shm, s>>>(
      logits, expert_bias, c.T, c.E, c.k, c.score, c.pre_softmax, c.routed_scaling, c.num_groups, c.group_topk, idx,
      w, rw.cnt_part, rw.prob_part, zp, pn);
  return MOE_OK;
}

// softmax keys are the fp32 logits: compared as floats (above 1024 experts the fp64
// instance, which spills less, serves them too); the elementwise scores in fp64
template <int EPL>
moe_status_t launch_topk(const moe_config_t& c, int nblk, const float* logits, const float* expert_bias,
                         int32_t* idx, float* w, const RouterWs& rw, float* zp, float2* pn, hipStream_t s) {
  return c.score == MOE_SOFTMAX && EPL <= 16
             ? launch_topk_kt<EPL, float>(c, nblk, logits, expert_bias, idx, w, rw, zp, pn, s)
                                : launch_topk_kt<EPL, double>(c, nblk, logits, expert_bias, idx, w, rw, zp, pn, s);
}

}  // namespace

namespace {

template <int LPT, int KPL, int NW, int KEYS>
moe_status_t launch_rows_inst(const moe_config_t& c, const RouterRowArgs& a, int nblk, hipStream_t s) {
  const size_t shm = static_cast<size_t>(c.E) * sizeof(int) +
                     (KEYS == 2 ? static_cast<size_t>(NW * (64 / LPT)) * c.E * 4 : 0) + (KEYS != 0 ? c.E * 4 : 0) +
                     (a.prob_part ? static_cast<size_t>(NW) * c.E * 4 : 0);
  // the instance without bounds checks serves E == LPT * KPL, except for 32 fp64 keys per
  // lane, where the compiler spills more without them
  constexpr bool kFullOk = !(KEYS == 1 && KPL == 32);
  const bool full = kFullOk && c.E == LPT * KPL;
  const void* fn = full ? reinterpret_cast<const void*>(router_rows_kernel<LPT, KPL, NW, KEYS, kFullOk>)
                        : reinterpret_cast<const void*>(router_rows_kernel<LPT, KPL, NW, KEYS, false>);
  if (shm > 65536 &&
      hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(shm)) != hipSuccess)
    return fail(MOE_ERR_HIP, "router: cannot raise the LDS limit to %zu bytes", shm);
  if (full)
    router_rows_kernel<LPT, KPL, NW, KEYS, kFullOk><<<nblk, 64 * NW, shm, s>>>(a);
  else
    router_rows_kernel<LPT, KPL, NW, KEYS, false><<<nblk, 64 * NW, shm, s>>>(a);
  return MOE_OK;
}

// lanes per token: 16 while k <= 16 and E <= 512 (up to 32 keys per lane), else 32 (k > 16,
// E <= 512) or 64 (a group's lane j keeps slot j, so LPT >= k).  Blocks whose lanes hold
// more than 16 keys, or whose groups span rows, run 8 waves so that each may use up to 256
// registers without spilling.
template <int KEYS>
moe_status_t launch_rows(const moe_config_t& c, const RouterRowArgs& a, int nblk, hipStream_t s) {
  if (c.k <= 16 && c.E <= 512) {
    if (c.E <= 16) return launch_rows_inst<16, 1, 16, KEYS>(c, a, nblk, s);
    if (c.E <= 32) return launch_rows_inst<16, 2, 16, KEYS>(c, a, nblk, s);
    if (c.E <= 64) return launch_rows_inst<16, 4, 16, KEYS>(c, a, nblk, s);
    if (c.E <= 128) return launch_rows_inst<16, 8, 16, KEYS>(c, a, nblk, s);
    if (c.E <= 256) return launch_rows_inst<16, 16, 16, KEYS>(c, a, nblk, s);
    if constexpr (KEYS != 2) return launch_rows_inst<16, 32, 8, KEYS>(c, a, nblk, s);
  }
  if constexpr (KEYS == 2) {
    return fail(MOE_ERR_UNSUPPORTED, "router: fp32-first sigmoid keys need k <= 16 and E <= 256");
  } else {
    if (c.E <= 512) return launch_rows_inst<32, 16, 8, KEYS>(c, a, nblk, s);
    if (c.E <= 1024) return launch_rows_inst<64, 16, 8, KEYS>(c, a, nblk, s);
    return launch_rows_inst<64, 32, 8, KEYS>(c, a, nblk, s);
  }
}

}  // namespace

moe_status_t launch_router_topk(const moe_config_t& c, const float* logits, const float* expert_bias,
                                int32_t* idx, float* w, int32_t* counts, float* prob_sum, float* prob_scratch,
                                float* stats, int32_t* seq_counts, const RouterWs& rw, hipStream_t s) {
  const int nblk = static_cast<int>(router_num_blocks(c.T));
  if (nblk != permute_num_chunks(c.T)) return fail(MOE_ERR_UNSUPPORTED, "router blocks differ from permute chunks");
  const bool seq_on = c.seq_aux_coeff != 0.0f;
  float* zp = c.z_coeff != 0.0f ? rw.z_part : nullptr;
  float2* pn = seq_on ? reinterpret_cast<float2*>(rw.pnorm) : nullptr;
  if (c.num_groups == 0) {
    // the row-group kernel; the aux probabilities are summed only when asked for or when
    // the aux loss needs them
    const bool want_p = prob_sum != nullptr || c.aux_coeff != 0.0f;
    float* ps = prob_sum ? prob_sum : (want_p ? prob_scratch : nullptr);
    RouterRowArgs a{};
    a.logits = logits; a.expert_bias = expert_bias;
    a.T = c.T; a.E = c.E; a.k = c.k; a.score = c.score; a.pre_softmax = c.pre_softmax; a.scaling = c.routed_scaling;
    a.idx = idx; a.w = w;
    a.cnt_part = rw.cnt_part; a.prob_part = want_p ? rw.prob_part : nullptr; a.z_part = zp; a.pnorm = pn;
    a.done = rw.done;
    // sigmoid keys are chosen on fp32 approximations and confirmed in fp64 when 16 lanes
    // route a token; other scores compare fp64 keys
    const bool sig16 = c.score == MOE_SIGMOID && c.k <= 16 && c.E <= 256;
    MOE_TRY_INTERNAL(c.score == MOE_SOFTMAX ? launch_rows<0>(c, a, nblk, s)
                     : sig16                ? launch_rows<2>(c, a, nblk, s)
                                            : launch_rows<1>(c, a, nblk, s));
    const size_t part_bytes = static_cast<size_t>(nblk) * c.E * 4 * (a.prob_part ? 2 : 1);
    const bool al16 = ((reinterpret_cast<uintptr_t>(rw.cnt_part) | reinterpret_cast<uintptr_t>(a.prob_part)) & 15u) == 0;
    const int vec = (c.E % 4 == 0 && al16) ? 4 : 1;
    if (part_bytes <= kFinOneBlockBytes && c.E / vec <= 1024) {
      const size_t shm = static_cast<size_t>(1024 / (c.E / vec)) * c.E * 4 * (a.prob_part ? 2 : 1);
      if (vec == 4)
        router_finalize_one_block_kernel<4><<<1, 1024, shm, s>>>(rw.cnt_part, a.prob_part, nblk, c.E, c.T, c.k,
                                                                 c.aux_coeff, zp, c.z_coeff, seq_on ? 1 : 0, counts,
                                                                 ps, stats);
      else
        router_finalize_one_block_kernel<1><<<1, 1024, shm, s>>>(rw.cnt_part, a.prob_part, nblk, c.E, c.T, c.k,
                                                                 c.aux_coeff, zp, c.z_coeff, seq_on ? 1 : 0, counts,
                                                                 ps, stats);
    } else {
      router_finalize_stats_kernel<<<static_cast<int>(ceil_div(c.E, kFinCols)), 1024, 0, s>>>(
          rw.cnt_part, a.prob_part, nblk, c.E, c.T, c.k, c.aux_coeff, zp, c.z_coeff, seq_on ? 1 : 0, counts, ps,
          stats, rw.done);
    }
  } else {
    // group-limited routing: one wave per token
    float* ps = prob_sum ? prob_sum : prob_scratch;
    const int epl = router_epl(c.E);
    moe_status_t st = MOE_OK;
    switch (epl) {
      case 1: st = launch_topk<1>(c, nblk, logits, expert_bias, idx, w, rw, zp, pn, s); break;
      case 2: st = launch_topk<2>(c, nblk, logits, expert_bias, idx, w, rw, zp, pn, s); break;
      case 4: st = launch_topk<4>(c, nblk, logits, expert_bias, idx, w, rw, zp, pn, s); break;
      case 8: st = launch_topk<8>(c, nblk, logits, expert_bias, idx, w, rw, zp, pn, s); break;
      case 16: st = launch_topk<16>(c, nblk, logits, expert_bias, idx, w, rw, zp, pn, s); break;
      case 32: st = launch_topk<32>(c, nblk, logits, expert_bias, idx, w, rw, zp, pn, s); break;
      default:
        return fail(MOE_ERR_UNSUPPORTED, "router: E=%d too large", c.E);
    }
    MOE_TRY_INTERNAL(st);
    router_finalize_kernel<<<static_cast<int>(ceil_div(c.E, 64)), 1024, 0, s>>>(rw.cnt_part, rw.prob_part, nblk,
                                                                              c.E, counts, ps);
    if (stats)
      router_stats_kernel<<<1, 1024, 0, s>>>(counts, ps, c.E, c.T, c.k, c.aux_coeff, zp, nblk, c.z_coeff,
                                             seq_on ? 1 : 0, stats);
  }
  if (seq_on) {
    const int S = c.seq_len, B = c.T / c.seq_len, nsc = static_cast<int>(ceil_div(S, 64));
    const size_t shm_s = static_cast<size_t>(c.E) * sizeof(int);
    seq_stats_kernel<<<dim3(nsc, B), 256, shm_s, s>>>(logits, pn, idx, c.E, c.k, S, B, c.score, rw.seq_cnt_part,
                                                     rw.seq_prob_part);
    seq_finalize_kernel<<<1, 1024, 0, s>>>(rw.seq_cnt_part, rw.seq_prob_part, nsc, B, c.E, c.k, S, c.seq_aux_coeff,
                                           seq_counts, stats);
  }
  return check_launch("router_topk");
}

size_t router_seq_part_elems(const moe_config_t& c) {
  if (c.seq_aux_coeff == 0.0f || c.seq_len < 1) return 0;
  return static_cast<size_t>(c.T / c.seq_len) * static_cast<size_t>(ceil_div(c.seq_len, 64)) * c.E;
}

moe_status_t launch_bias_update(const int32_t* counts, int E, float rate, int centered, float* bias, hipStream_t s) {
  bias_update_kernel<<<1, 1024, 0, s>>>(counts, E, rate, centered, bias);
  return check_launch("expert_bias_update");
}

moe_status_t launch_router_bwd(const moe_config_t& c, const float* logits, const int32_t* idx, const float* w,
                               const float* dw, const int32_t* counts, const int32_t* seq_counts, float daux,
                               float* dlogits, hipStream_t s) {
  const int grid = static_cast<int>(ceil_div(c.T, 4));
  RouterBwdArgs a{};
  a.logits = logits; a.idx = idx; a.w = w; a.dw = dw;
  const bool aux = c.aux_coeff != 0.0f && daux != 0.0f;
  const bool seq = c.seq_aux_coeff != 0.0f && daux != 0.0f;
  a.counts = aux ? counts : nullptr;
  a.seq_counts = seq ? seq_counts : nullptr;
  a.T = c.T; a.E = c.E; a.k = c.k; a.score = c.score; a.pre_softmax = c.pre_softmax;
  a.S = seq ? c.seq_len : 1;
  a.B = seq ? c.T / c.seq_len : 1;
  a.scaling = c.routed_scaling;
  const double Td = c.T;
  a.g_aux = static_cast<float>(static_cast<double>(c.aux_coeff) * c.E / (c.k * Td * Td));
  const double Sd = a.S;
  a.g_seq = static_cast<float>(static_cast<double>(c.seq_aux_coeff) * c.E / (c.k * Sd * Sd * a.B));
  a.z_scale = static_cast<float>(static_cast<double>(daux) * c.z_coeff * 2.0 / Td);
  a.daux = daux;
  a.dlogits = dlogits;
#define MOE_RBWD_CASE(N)                                         \
  case N:                                                        \
    router_bwd_kernel<N><<<grid, 256, 0, s>>>(a);                \
    break;
  switch (router_epl(c.E)) {
    MOE_RBWD_CASE(1)
    MOE_RBWD_CASE(2)
    MOE_RBWD_CASE(4)
    MOE_RBWD_CASE(8)
    MOE_RBWD_CASE(16)
    MOE_RBWD_CASE(32)
    default:
      return fail(MOE_ERR_UNSUPPORTED, "router bwd: E=%d too large", c.E);
  }
#undef MOE_RBWD_CASE
  return check_launch("router_bwd");
}


}  // namespace moe
