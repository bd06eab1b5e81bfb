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
    for (int c = 0; c < nsc; ++c) {
      const int64_t i = (static_cast<int64_t>(b) * nsc + c) * E + e;
      cnt += cnt_part[i];
      P += prob_part[i];
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

moe_status_t launch_router_topk(const moe_config_t& c, const float* logits, const float* expert_bias,
                                int32_t* idx, float* w, int32_t* counts, float* prob_sum, float* stats,
                                int32_t* seq_counts, const RouterWs& rw, hipStream_t s) {
  const int nblk = static_cast<int>(router_num_blocks(c.T));
  if (nblk != permute_num_chunks(c.T)) return fail(MOE_ERR_UNSUPPORTED, "router blocks differ from permute chunks");
  const int epl = router_epl(c.E);
  const bool seq_on = c.seq_aux_coeff != 0.0f;
  float* zp = c.z_coeff != 0.0f ? rw.z_part : nullptr;
  float2* pn = seq_on ? reinterpret_cast<float2*>(rw.pnorm) : nullptr;
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
  router_finalize_kernel<<<static_cast<int>(ceil_div(c.E, 64)), 1024, 0, s>>>(rw.cnt_part, rw.prob_part, nblk, c.E,
                                                                            counts, prob_sum);
  if (stats)
    router_stats_kernel<<<1, 1024, 0, s>>>(counts, prob_sum, c.E, c.T, c.k, c.aux_coeff, zp, nblk, c.z_coeff,
                                           seq_on ? 1 : 0, stats);
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
