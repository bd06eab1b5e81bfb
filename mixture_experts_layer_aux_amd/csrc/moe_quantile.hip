// Quantile balancing: The Ultimate MoE Training Handbook, §3.3 Load balancing, Quantile.
//
// The selection bias is solved for per micro-batch instead of stepped.  Routing: each
// token keeps the k + 1 largest keys scores - beta (fp32, ties to the lower expert index);
// the first k are its experts and the (k+1)-th key is its alpha.  Solve: each expert's new
// bias is the (T k / E + 1)-th largest of scores[:, e] - alpha over the tokens.
//
// The per-expert selection is a radix select over the fp32 bit patterns, made order
// preserving (sign bit flipped for non-negative values, all bits flipped for negative
// ones): four passes of 8 bits from the top.  Each pass histograms, per expert, the values
// whose already-decided high bits match, then one wave per expert finds, by a suffix scan
// over its 256 bins, the bin that holds the wanted rank counted from the top.  Blocks of 64 experts x 256 tokens
// read whole 256-byte row pieces of scores; their LDS histograms are merged into the
// global one with integer atomics (order-independent, so the result is reproducible).
#include <float.h>
#include <limits.h>

#include "moe_internal.h"

namespace moe {

namespace {

__device__ __forceinline__ uint32_t orderable(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_orderable(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// One wave per token, 4 tokens per block.
template <int EPL>
__global__ __launch_bounds__(256) void quantile_topk_kernel(const float* __restrict__ scores,
                                                            const float* __restrict__ beta, int T, int E, int k,
                                                            int32_t* __restrict__ idx, float* __restrict__ alpha) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = scores + static_cast<int64_t>(t) * E;
  float key[EPL];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      key[i] = row[e] - beta[e];
    } else {
      key[i] = -FLT_MAX;
      taken |= 1u << i;
    }
  }
  int my_e = 0;
  float kth = 0.0f;
  for (int j = 0; j <= k; ++j) {
    float bk = -FLT_MAX;
    int be = INT_MAX;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      if (!(taken & (1u << i)) && (key[i] > bk || (key[i] == bk && e < be))) {
        bk = key[i];
        be = e;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ok = __shfl_xor(bk, o, 64);
      const int oe = __shfl_xor(be, o, 64);
      if (ok > bk || (ok == bk && oe < be)) {
        bk = ok;
        be = oe;
      }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == j) my_e = be;
    if (j == k) kth = bk;
  }
  if (lane < k) idx[static_cast<int64_t>(t) * k + lane] = my_e;
  if (lane == 0) alpha[t] = kth;
}

// hist = 0, prefix = 0, rank = target + 1 (the wanted rank from the top, 1-based).
__global__ __launch_bounds__(256) void quantile_init_kernel(int E, int rank0, int32_t* __restrict__ hist,
                                                            uint32_t* __restrict__ prefix,
                                                            int32_t* __restrict__ rank) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < E * 256) hist[i] = 0;
  if (i < E) {
    prefix[i] = 0u;
    rank[i] = rank0;
  }
}

constexpr int kQExperts = 64;   // experts per histogram block (one per lane)
constexpr int kQTokens = 256;   // tokens per histogram block
constexpr int kQPad = 257;      // LDS row stride: equal digits of 64 experts fall in distinct banks

__global__ __launch_bounds__(256) void quantile_hist_kernel(const float* __restrict__ scores,
                                                            const float* __restrict__ alpha, int T, int E,
                                                            int shift, const uint32_t* __restrict__ prefix,
                                                            int32_t* __restrict__ hist) {
  __shared__ int h[kQExperts * kQPad];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e0 = blockIdx.x * kQExperts, t0 = blockIdx.y * kQTokens;
  for (int i = threadIdx.x; i < kQExperts * kQPad; i += 256) h[i] = 0;
  __syncthreads();
  const int e = e0 + lane;
  if (e < E) {
    const uint32_t mask = shift == 24 ? 0u : (0xFFFFFFFFu << (shift + 8));
    const uint32_t pre = prefix[e] & mask;
    const int t1 = min(T, t0 + kQTokens);
    // eight rows' loads in flight before their histogram updates (the integer counts do
    // not depend on the order)
    constexpr int U = 8;
    int t = t0 + wave;
    for (; t + 4 * (U - 1) < t1; t += 4 * U) {
      uint32_t u[U];
#pragma unroll
      for (int j = 0; j < U; ++j) u[j] = orderable(scores[static_cast<int64_t>(t + 4 * j) * E + e] - alpha[t + 4 * j]);
#pragma unroll
      for (int j = 0; j < U; ++j)
        if ((u[j] & mask) == pre) atomicAdd(&h[lane * kQPad + ((u[j] >> shift) & 255u)], 1);
    }
    for (; t < t1; t += 4) {
      const uint32_t u = orderable(scores[static_cast<int64_t>(t) * E + e] - alpha[t]);
      if ((u & mask) == pre) atomicAdd(&h[lane * kQPad + ((u >> shift) & 255u)], 1);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kQExperts * 256; i += 256) {
    const int le = i >> 8, d = i & 255;
    const int c = h[le * kQPad + d];
    if (c && e0 + le < E) atomicAdd(&hist[static_cast<int64_t>(e0 + le) * 256 + d], c);
  }
}

// One wave per expert: each lane holds 4 consecutive bins (lane 63 the top ones); a
// suffix scan across the lanes finds the lane whose bins hold the wanted rank, counted
// from the top, and that lane walks its 4 bins.  The histogram is cleared for the next
// pass; the last pass writes the selected value.
__global__ __launch_bounds__(256) void quantile_pick_kernel(int E, int shift, int32_t* __restrict__ hist,
                                                            uint32_t* __restrict__ prefix,
                                                            int32_t* __restrict__ rank,
                                                            float* __restrict__ beta_local) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  int4* he = reinterpret_cast<int4*>(hist + static_cast<int64_t>(e) * 256);
  const int4 c = he[lane];
  he[lane] = make_int4(0, 0, 0, 0);
  const int r = rank[e];
  const int own = c.x + c.y + c.z + c.w;
  // inclusive suffix sum over lanes lane..63
  int suf = own;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_down(suf, o, 64);
    if (lane + o < 64) suf += v;
  }
  const int above = suf - own;   // count in the bins of the higher lanes
  // the lane with above < r <= suf holds the rank (exactly one lane)
  if (above < r && r <= suf) {
    int cum = above, bin = 4 * lane;
    const int cs[4] = {c.x, c.y, c.z, c.w};
    for (int j = 3; j >= 0; --j) {
      if (cum + cs[j] >= r) {
        bin = 4 * lane + j;
        break;
      }
      cum += cs[j];
    }
    const uint32_t p = prefix[e] | (static_cast<uint32_t>(bin) << shift);
    prefix[e] = p;
    rank[e] = r - cum;
    if (shift == 0) beta_local[e] = from_orderable(p);
  }
}

// beta = ema beta + (1 - ema) beta_local, then the mean over the experts is taken out
// (sum in a fixed tree, in fp64).
__global__ __launch_bounds__(1024) void quantile_update_kernel(const float* __restrict__ local, int E, float ema,
                                                               float* __restrict__ beta) {
  __shared__ double s[1024];
  double acc = 0.0;
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    acc += static_cast<double>(ema * beta[e] + (1.0f - ema) * local[e]);
  s[threadIdx.x] = acc;
  __syncthreads();
  for (int h = blockDim.x / 2; h > 0; h >>= 1) {
    if (threadIdx.x < h) s[threadIdx.x] += s[threadIdx.x + h];
    __syncthreads();
  }
  const float mean = static_cast<float>(s[0] / E);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) beta[e] = (ema * beta[e] + (1.0f - ema) * local[e]) - mean;
}

}  // namespace

size_t quantile_ws_bytes(int E) { return static_cast<size_t>(E) * (256 * 4 + 4 + 4); }

moe_status_t launch_router_quantile(const moe_config_t& c, const float* scores, const float* beta, int32_t* idx,
                                    float* alpha, float* beta_local, void* ws, hipStream_t s) {
  const int grid = static_cast<int>(ceil_div(c.T, 4));
#define MOE_Q_CASE(N)                                                                                   \
  case N:                                                                                               \
    quantile_topk_kernel<N><<<grid, 256, 0, s>>>(scores, beta, c.T, c.E, c.k, idx, alpha);              \
    break;
  switch (router_epl(c.E)) {
    MOE_Q_CASE(1)
    MOE_Q_CASE(2)
    MOE_Q_CASE(4)
    MOE_Q_CASE(8)
    MOE_Q_CASE(16)
    MOE_Q_CASE(32)
    default:
      return fail(MOE_ERR_UNSUPPORTED, "quantile router: E=%d too large", c.E);
  }
#undef MOE_Q_CASE
  if (!beta_local) return check_launch("router_quantile");
  int32_t* hist = static_cast<int32_t*>(ws);
  uint32_t* prefix = reinterpret_cast<uint32_t*>(hist + static_cast<int64_t>(c.E) * 256);
  int32_t* rank = reinterpret_cast<int32_t*>(prefix + c.E);
  const int target = static_cast<int>(static_cast<int64_t>(c.T) * c.k / c.E);
  quantile_init_kernel<<<static_cast<int>(ceil_div(static_cast<int64_t>(c.E) * 256, 256)), 256, 0, s>>>(
      c.E, target + 1, hist, prefix, rank);
  const dim3 hgrid(static_cast<unsigned>(ceil_div(c.E, kQExperts)), static_cast<unsigned>(ceil_div(c.T, kQTokens)));
  for (int shift = 24; shift >= 0; shift -= 8) {
    quantile_hist_kernel<<<hgrid, 256, 0, s>>>(scores, alpha, c.T, c.E, shift, prefix, hist);
    quantile_pick_kernel<<<static_cast<int>(ceil_div(c.E, 4)), 256, 0, s>>>(c.E, shift, hist, prefix, rank,
                                                                            beta_local);
  }
  return check_launch("router_quantile");
}

moe_status_t launch_quantile_update(const float* beta_local, int E, float ema, float* beta, hipStream_t s) {
  quantile_update_kernel<<<1, 1024, 0, s>>>(beta_local, E, ema, beta);
  return check_launch("quantile_bias_update");
}

}  // namespace moe
