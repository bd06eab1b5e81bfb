// Router: top-k selection, mixing weights, load statistics, and its backward.
//
// The Ultimate MoE Training Handbook, §3.1 Router scoring (Gating function, Output
// scale, Precision) and §3.3 Load balancing (Aux loss); the MaxVio statistic of §3.2.
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

constexpr int kRouterWaves = 8;
// 64 tokens per block (8 per wave): a block's expert histogram is also the permute's
// chunk histogram, so this must equal the permute chunk.
constexpr int kRouterTokensPerBlock = 64;

struct Best {
  double key;
  int e;
  float l;
};

__device__ __forceinline__ bool better(double ka, int ea, double kb, int eb) {
  return ka > kb || (ka == kb && ea < eb);
}

template <int EPL>
__global__ __launch_bounds__(64 * kRouterWaves) void router_topk_kernel(const float* __restrict__ logits,
                                                          const float* __restrict__ expert_bias,
                                                          int T, int E, int k, int score, float scaling,
                                                          int32_t* __restrict__ idx, float* __restrict__ w,
                                                          int32_t* __restrict__ cnt_part,
                                                          float* __restrict__ prob_part) {
  extern __shared__ int smem_i[];
  int* hist = smem_i;                                          // [E]
  float* red = reinterpret_cast<float*>(smem_i + E);           // [kRouterWaves][E]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();

  float acc[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) acc[i] = 0.0f;

  const int t0 = blockIdx.x * kRouterTokensPerBlock;
  for (int s = wave; s < kRouterTokensPerBlock; s += kRouterWaves) {
    const int t = t0 + s;
    if (t >= T) break;
    const float* row = logits + static_cast<int64_t>(t) * E;
    float l[EPL];
    double key[EPL];
    uint32_t taken = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      if (e < E) {
        l[i] = row[e];
        if (score == MOE_SOFTMAX) {
          key[i] = static_cast<double>(l[i]);
        } else {
          // sigma(l) (+ bias) in fp64 from the fp32 values
          double sg = 1.0 / (1.0 + exp(-static_cast<double>(l[i])));
          key[i] = expert_bias ? sg + static_cast<double>(expert_bias[e]) : sg;
        }
      } else {
        l[i] = 0.0f;
        key[i] = -DBL_MAX;
        taken |= 1u << i;
      }
    }
    int my_e = -1;
    float my_l = 0.0f;
    float top_l = 0.0f;
    for (int j = 0; j < k; ++j) {
      Best b{-DBL_MAX, INT_MAX, 0.0f};
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        if (!(taken & (1u << i)) && better(key[i], lane + 64 * i, b.key, b.e)) {
          b.key = key[i];
          b.e = lane + 64 * i;
          b.l = l[i];
        }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        double ok = __shfl_xor(b.key, o, 64);
        int oe = __shfl_xor(b.e, o, 64);
        float ol = __shfl_xor(b.l, o, 64);
        if (better(ok, oe, b.key, b.e)) {
          b.key = ok;
          b.e = oe;
          b.l = ol;
        }
      }
      if ((b.e & 63) == lane) taken |= 1u << (b.e >> 6);
      if (lane == j) {
        my_e = b.e;
        my_l = b.l;
      }
      if (j == 0) top_l = b.l;
    }
    // mixing weights: lane j < k owns slot j
    float wv;
    if (score == MOE_SOFTMAX) {
      float ex = lane < k ? expf(my_l - top_l) : 0.0f;
      float z = wave_sum(ex);
      wv = ex / z;
    } else {
      double sg = lane < k ? 1.0 / (1.0 + exp(-static_cast<double>(my_l))) : 0.0;
      double z = wave_sum(sg);
      wv = static_cast<float>(k > 1 ? sg / (z + 1e-20) : sg);
    }
    if (lane < k) {
      idx[static_cast<int64_t>(t) * k + lane] = my_e;
      w[static_cast<int64_t>(t) * k + lane] = wv * scaling;
      atomicAdd(&hist[my_e], 1);   // integer: order-independent
    }
    if (score == MOE_SOFTMAX) {
      // full softmax over all E for the aux statistic; top_l is the row maximum
      float ex[EPL];
      float part = 0.0f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        ex[i] = (lane + 64 * i < E) ? expf(l[i] - top_l) : 0.0f;
        part += ex[i];
      }
      const float z = wave_sum(part);
      const float inv = 1.0f / z;
#pragma unroll
      for (int i = 0; i < EPL; ++i) acc[i] += ex[i] * inv;
    }
  }
  if (score == MOE_SOFTMAX) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      if (e < E) red[wave * E + e] = acc[i];
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    cnt_part[static_cast<int64_t>(blockIdx.x) * E + e] = hist[e];
    if (score == MOE_SOFTMAX) {
      float s = 0.0f;
#pragma unroll
      for (int v = 0; v < kRouterWaves; ++v) s += red[v * E + e];
      prob_part[static_cast<int64_t>(blockIdx.x) * E + e] = s;
    }
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
__global__ __launch_bounds__(1024) void router_stats_kernel(const int32_t* __restrict__ counts,
                                                            const float* __restrict__ prob_sum, int E, int T,
                                                            int k, float coeff, float* __restrict__ stats) {
  __shared__ double s_dot[1024];
  __shared__ int s_max[1024];
  __shared__ int s_empty[1024];
  double dot = 0.0;
  int mx = 0, empty = 0;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int c = counts[e];
    if (prob_sum) dot += static_cast<double>(prob_sum[e]) * c;
    mx = max(mx, c);
    empty += (c == 0);
  }
  s_dot[threadIdx.x] = dot;
  s_max[threadIdx.x] = mx;
  s_empty[threadIdx.x] = empty;
  __syncthreads();
  for (int h = blockDim.x / 2; h > 0; h >>= 1) {
    if (threadIdx.x < h) {
      s_dot[threadIdx.x] += s_dot[threadIdx.x + h];
      s_max[threadIdx.x] = max(s_max[threadIdx.x], s_max[threadIdx.x + h]);
      s_empty[threadIdx.x] += s_empty[threadIdx.x + h];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double Td = static_cast<double>(T);
    const double mean = Td * k / E;
    stats[0] = prob_sum ? static_cast<float>(s_dot[0] * coeff * E / (k * Td * Td)) : 0.0f;
    stats[1] = static_cast<float>((s_max[0] - mean) / mean);
    stats[2] = static_cast<float>(s_empty[0]);
    stats[3] = static_cast<float>(s_max[0]);
  }
}

// Router backward, one wave per token (see moe_router_bwd in moe.h for the formulas).
template <int EPL>
__global__ __launch_bounds__(256) void router_bwd_kernel(const float* __restrict__ logits,
                                                         const int32_t* __restrict__ idx,
                                                         const float* __restrict__ w,
                                                         const float* __restrict__ dw,
                                                         const int32_t* __restrict__ counts, int T, int E,
                                                         int k, int score, float scaling, float aux_coeff,
                                                         float daux, float* __restrict__ dlogits) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + static_cast<int64_t>(t) * E;
  float val[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) val[i] = 0.0f;

  const bool with_aux = score == MOE_SOFTMAX && aux_coeff != 0.0f && daux != 0.0f;
  if (with_aux) {
    float l[EPL], p[EPL];
    float m = -FLT_MAX;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      l[i] = (lane + 64 * i < E) ? row[lane + 64 * i] : -FLT_MAX;
      m = fmaxf(m, l[i]);
    }
    m = wave_max(m);
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      p[i] = (lane + 64 * i < E) ? expf(l[i] - m) : 0.0f;
      part += p[i];
    }
    const float inv = 1.0f / wave_sum(part);
    // g_e = coeff * E * counts[e] / (T k T)
    const float gs = aux_coeff * static_cast<float>(E) / (static_cast<float>(T) * k * static_cast<float>(T));
    float g[EPL];
    float pg = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      p[i] *= inv;
      g[i] = (lane + 64 * i < E) ? gs * static_cast<float>(counts[lane + 64 * i]) : 0.0f;
      pg += p[i] * g[i];
    }
    pg = wave_sum(pg);
#pragma unroll
    for (int i = 0; i < EPL; ++i) val[i] = daux * p[i] * (g[i] - pg);
  }

  int my_e = 0;
  float my_w = 0.0f, my_dw = 0.0f;
  if (lane < k) {
    my_e = idx[static_cast<int64_t>(t) * k + lane];
    my_w = w[static_cast<int64_t>(t) * k + lane];
    my_dw = dw[static_cast<int64_t>(t) * k + lane];
  }
  float dl;
  if (score == MOE_SOFTMAX) {
    const float wdw = wave_sum(lane < k ? my_w * my_dw : 0.0f);
    dl = my_w * my_dw - (my_w / scaling) * wdw;
  } else {
    const float s = lane < k ? sigmoid_f(row[my_e]) : 0.0f;
    if (k > 1) {
      const float z = wave_sum(s) + 1e-20f;
      const float dws = wave_sum(my_dw * s);
      const float ds = (scaling / z) * (my_dw - dws / z);
      dl = ds * s * (1.0f - s);
    } else {
      dl = scaling * my_dw * s * (1.0f - s);
    }
  }
  for (int j = 0; j < k; ++j) {
    const int ej = __shfl(my_e, j, 64);
    const float dj = __shfl(dl, j, 64);
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (ej == lane + 64 * i) val[i] += dj;
  }
  float* out = dlogits + static_cast<int64_t>(t) * E;
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

moe_status_t launch_router_topk(const moe_config_t& c, const float* logits, const float* expert_bias,
                                int32_t* idx, float* w, int32_t* counts, float* prob_sum, float* stats,
                                int32_t* cnt_part, float* prob_part, hipStream_t s) {
  const int nblk = static_cast<int>(router_num_blocks(c.T));
  if (nblk != permute_num_chunks(c.T)) return fail(MOE_ERR_UNSUPPORTED, "router blocks differ from permute chunks");
  const size_t shm = static_cast<size_t>(c.E) * sizeof(int) + static_cast<size_t>(kRouterWaves) * c.E * sizeof(float);
  const int epl = router_epl(c.E);
  float* pp = c.score == MOE_SOFTMAX ? prob_part : nullptr;
#define MOE_ROUTER_CASE(N)                                                                              \
  case N:                                                                                               \
    if (shm > 65536 &&                                                                                  \
        hipFuncSetAttribute(reinterpret_cast<const void*>(router_topk_kernel<N>),                       \
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(shm)) != hipSuccess) \
      return fail(MOE_ERR_HIP, "router: cannot raise the LDS limit to %zu bytes", shm);                 \
    router_topk_kernel<N><<<nblk, 64 * kRouterWaves, shm, s>>>(logits, expert_bias, c.T, c.E, c.k, c.score,          \
                                                 c.routed_scaling, idx, w, cnt_part, pp);               \
    break;
  switch (epl) {
    MOE_ROUTER_CASE(1)
    MOE_ROUTER_CASE(2)
    MOE_ROUTER_CASE(4)
    MOE_ROUTER_CASE(8)
    MOE_ROUTER_CASE(16)
    MOE_ROUTER_CASE(32)
    default:
      return fail(MOE_ERR_UNSUPPORTED, "router: E=%d too large", c.E);
  }
#undef MOE_ROUTER_CASE
  router_finalize_kernel<<<static_cast<int>(ceil_div(c.E, 64)), 1024, 0, s>>>(cnt_part, pp, nblk, c.E, counts,
                                                                            c.score == MOE_SOFTMAX ? prob_sum : nullptr);
  if (stats) {
    // for softmax, prob_sum is never NULL here (the C-ABI layer supplies workspace)
    router_stats_kernel<<<1, 1024, 0, s>>>(counts, c.score == MOE_SOFTMAX ? prob_sum : nullptr, c.E, c.T, c.k,
                                           c.aux_coeff, stats);
  }
  return check_launch("router_topk");
}

moe_status_t launch_router_bwd(const moe_config_t& c, const float* logits, const int32_t* idx, const float* w,
                               const float* dw, const int32_t* counts, float daux, float* dlogits, hipStream_t s) {
  const int grid = static_cast<int>(ceil_div(c.T, 4));
#define MOE_RBWD_CASE(N)                                                                                  \
  case N:                                                                                                 \
    router_bwd_kernel<N><<<grid, 256, 0, s>>>(logits, idx, w, dw, counts, c.T, c.E, c.k, c.score,        \
                                              c.routed_scaling, c.aux_coeff, daux, dlogits);              \
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
