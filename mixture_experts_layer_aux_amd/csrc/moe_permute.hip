// Dropless permutation, weighted combine, and their backward passes.
//
// LeCompute, "MoE training: cluster, routing, load balancing", section "Read the
// timeline before blaming the network" (tokens grouped by expert before the expert
// matmuls and restored to their order afterwards) and section "An expert transforms
// numbers inside the model" (the weighted sum of the selected outputs); The Ultimate
// MoE Training Handbook, §3.4 Shared experts (shared output added at weight 1).
//
// Permutation, deterministic and atomic-free in its order:
//   1. per 64-token chunk, an expert histogram (LDS integer adds);
//   2. per expert, an exclusive scan of the chunk histograms in chunk order, and an
//      exclusive scan of the expert totals -> offsets;
//   3. per chunk, each token's rank inside its expert from a 64-bit LDS lane mask
//      (popcount of the lanes below it), so rows inside an expert follow token order;
//   4. a token-major copy: each token's row is read once and written to its k rows.
// All data movement kernels are one wavefront per token moving 16-byte units.
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kChunk = 64;  // tokens per histogram chunk (one wave)

__global__ __launch_bounds__(64) void chunk_hist_kernel(const int32_t* __restrict__ idx, int T, int E, int k,
                                                        int32_t* __restrict__ blk_hist) {
  extern __shared__ int hist[];
  for (int e = threadIdx.x; e < E; e += 64) hist[e] = 0;
  __syncthreads();
  const int t = blockIdx.x * kChunk + threadIdx.x;
  if (t < T)
    for (int j = 0; j < k; ++j) atomicAdd(&hist[idx[static_cast<int64_t>(t) * k + j]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 64) blk_hist[static_cast<int64_t>(blockIdx.x) * E + e] = hist[e];
}

// Per expert column: blk_base[b][e] = sum_{b' < b} blk_hist[b'][e]; counts[e] = total.
// 256 threads = 64 experts x 4 contiguous quarters of the chunks.
__global__ __launch_bounds__(256) void chunk_scan_kernel(const int32_t* __restrict__ blk_hist, int nblk, int E,
                                                         int32_t* __restrict__ blk_base,
                                                         int32_t* __restrict__ counts) {
  __shared__ int part[4][64];
  const int c = threadIdx.x & 63, r = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + c;
  const int q = (nblk + 3) / 4;
  const int b0 = r * q, b1 = min(nblk, b0 + q);
  int s = 0;
  if (e < E)
    for (int b = b0; b < b1; ++b) s += blk_hist[static_cast<int64_t>(b) * E + e];
  part[r][c] = s;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < r; ++i) base += part[i][c];
  if (e < E) {
    for (int b = b0; b < b1; ++b) {
      const int v = blk_hist[static_cast<int64_t>(b) * E + e];
      blk_base[static_cast<int64_t>(b) * E + e] = base;
      base += v;
    }
    if (r == 3) counts[e] = base;
  }
}

// offsets = exclusive prefix of counts (one block, E <= 2048).
__global__ __launch_bounds__(1024) void offsets_kernel(const int32_t* __restrict__ counts, int E,
                                                       int32_t* __restrict__ offsets) {
  __shared__ int s[2048];
  for (int e = threadIdx.x; e < 2048; e += 1024) s[e] = e < E ? counts[e] : 0;
  __syncthreads();
  // Hillis-Steele inclusive scan over 2048 entries, two per thread
  for (int off = 1; off < 2048; off <<= 1) {
    int a0 = 0, a1 = 0;
    const int i0 = threadIdx.x, i1 = threadIdx.x + 1024;
    if (i0 >= off) a0 = s[i0 - off];
    if (i1 >= off) a1 = s[i1 - off];
    __syncthreads();
    s[i0] += a0;
    s[i1] += a1;
    __syncthreads();
  }
  for (int e = threadIdx.x; e <= E; e += 1024) offsets[e] = e == 0 ? 0 : s[e - 1];
}

__global__ __launch_bounds__(64) void permute_index_kernel(const int32_t* __restrict__ idx, int T, int E, int k,
                                                           const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ blk_base,
                                                           int32_t* __restrict__ row_of,
                                                           int32_t* __restrict__ token_of) {
  extern __shared__ unsigned long long mask[];
  const int lane = threadIdx.x;
  const int t = blockIdx.x * kChunk + lane;
  const bool ok = t < T;
  for (int j = 0; j < k && ok; ++j) mask[idx[static_cast<int64_t>(t) * k + j]] = 0ull;
  __syncthreads();
  for (int j = 0; j < k && ok; ++j) atomicOr(&mask[idx[static_cast<int64_t>(t) * k + j]], 1ull << lane);
  __syncthreads();
  if (!ok) return;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int j = 0; j < k; ++j) {
    const int e = idx[static_cast<int64_t>(t) * k + j];
    const int r = offsets[e] + blk_base[static_cast<int64_t>(blockIdx.x) * E + e] + __popcll(mask[e] & below);
    row_of[static_cast<int64_t>(t) * k + j] = r;
    token_of[r] = t;
  }
}

// x_perm[row_of[t, j]] = x[t]; one wave per token, 16-byte units.
__global__ __launch_bounds__(256) void permute_copy_kernel(const uint4* __restrict__ x, int T, int units, int k,
                                                           const int32_t* __restrict__ row_of,
                                                           uint4* __restrict__ x_perm) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int my_r = lane < k ? row_of[static_cast<int64_t>(t) * k + lane] : 0;
  const uint4* src = x + static_cast<int64_t>(t) * units;
  for (int u = lane; u < units; u += 64) {
    const uint4 v = src[u];
    for (int j = 0; j < k; ++j) {
      const int r = __shfl(my_r, j, 64);
      x_perm[static_cast<int64_t>(r) * units + u] = v;
    }
  }
}

// 16-byte unit <-> fp32 lanes for the two storage types.
template <typename T> struct Unit;
template <> struct Unit<uint16_t> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void to_f32(const uint4& v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  __device__ __forceinline__ static uint4 from_f32(const float* f) {
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                      pack_bf16x2(f[6], f[7]));
  }
};
template <> struct Unit<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void to_f32(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
  __device__ __forceinline__ static uint4 from_f32(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
  }
};

// y[t] = sum_j w[t,j] * Y[row_of[t,j]] (+ add_act[t]) (+ add_f32[t]); w NULL means 1.
// Also the unpermute-reduce of the backward (w NULL, two addends).
template <typename T>
__global__ __launch_bounds__(256) void gather_sum_kernel(const uint4* __restrict__ Y, int Tn, int units, int k,
                                                         const int32_t* __restrict__ row_of,
                                                         const float* __restrict__ w,
                                                         const uint4* __restrict__ add_act,
                                                         const float4* __restrict__ add_f32,
                                                         uint4* __restrict__ out) {
  constexpr int N = Unit<T>::N;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int my_r = lane < k ? row_of[static_cast<int64_t>(t) * k + lane] : 0;
  const float my_w = (lane < k && w) ? w[static_cast<int64_t>(t) * k + lane] : 1.0f;
  for (int u = lane; u < units; u += 64) {
    float acc[N];
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = 0.0f;
    for (int j = 0; j < k; ++j) {
      const int r = __shfl(my_r, j, 64);
      const float wj = __shfl(my_w, j, 64);
      float f[N];
      Unit<T>::to_f32(Y[static_cast<int64_t>(r) * units + u], f);
#pragma unroll
      for (int i = 0; i < N; ++i) acc[i] += wj * f[i];
    }
    if (add_act) {
      float f[N];
      Unit<T>::to_f32(add_act[static_cast<int64_t>(t) * units + u], f);
#pragma unroll
      for (int i = 0; i < N; ++i) acc[i] += f[i];
    }
    if (add_f32) {
      const float4* p = add_f32 + (static_cast<int64_t>(t) * units + u) * (N / 4);
#pragma unroll
      for (int q = 0; q < N / 4; ++q) {
        const float4 v = p[q];
        acc[4 * q] += v.x;
        acc[4 * q + 1] += v.y;
        acc[4 * q + 2] += v.z;
        acc[4 * q + 3] += v.w;
      }
    }
    out[static_cast<int64_t>(t) * units + u] = Unit<T>::from_f32(acc);
  }
}

// dY_perm[row_of[t,j]] = w[t,j] * dy[t];  dw[t,j] = <dy[t], Y_perm[row_of[t,j]]>.
template <typename T>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const uint4* __restrict__ dy,
                                                          const uint4* __restrict__ Y, int Tn, int units,
                                                          int k, const int32_t* __restrict__ row_of,
                                                          const float* __restrict__ w,
                                                          uint4* __restrict__ dY, float* __restrict__ dw) {
  constexpr int N = Unit<T>::N;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int my_r = lane < k ? row_of[static_cast<int64_t>(t) * k + lane] : 0;
  const float my_w = lane < k ? w[static_cast<int64_t>(t) * k + lane] : 0.0f;
  const uint4* dyt = dy + static_cast<int64_t>(t) * units;
  float my_dw = 0.0f;
  for (int j = 0; j < k; ++j) {
    const int r = __shfl(my_r, j, 64);
    const float wj = __shfl(my_w, j, 64);
    float part = 0.0f;
    for (int u = lane; u < units; u += 64) {
      float g[N], y[N];
      Unit<T>::to_f32(dyt[u], g);
      Unit<T>::to_f32(Y[static_cast<int64_t>(r) * units + u], y);
#pragma unroll
      for (int i = 0; i < N; ++i) {
        part += g[i] * y[i];
        g[i] *= wj;
      }
      dY[static_cast<int64_t>(r) * units + u] = Unit<T>::from_f32(g);
    }
    part = wave_sum(part);
    if (lane == j) my_dw = part;
  }
  if (lane < k) dw[static_cast<int64_t>(t) * k + lane] = my_dw;
}

}  // namespace

int64_t permute_num_chunks(int T) { return ceil_div(T, kChunk); }

moe_status_t launch_permute(const moe_config_t& c, const void* x, const int32_t* idx, int32_t* offsets,
                            int32_t* row_of, int32_t* token_of, void* x_perm, int32_t* blk_hist,
                            int32_t* blk_base, int32_t* counts_ws, bool hist_ready, hipStream_t s) {
  const int nblk = static_cast<int>(permute_num_chunks(c.T));
  if (!hist_ready)
    chunk_hist_kernel<<<nblk, 64, c.E * sizeof(int), s>>>(idx, c.T, c.E, c.k, blk_hist);
  chunk_scan_kernel<<<static_cast<int>(ceil_div(c.E, 64)), 256, 0, s>>>(blk_hist, nblk, c.E, blk_base, counts_ws);
  offsets_kernel<<<1, 1024, 0, s>>>(counts_ws, c.E, offsets);
  permute_index_kernel<<<nblk, 64, c.E * sizeof(unsigned long long), s>>>(idx, c.T, c.E, c.k, offsets, blk_base,
                                                                          row_of, token_of);
  const int units = static_cast<int>(static_cast<int64_t>(c.d) * act_bytes(c) / 16);
  permute_copy_kernel<<<static_cast<int>(ceil_div(c.T, 4)), 256, 0, s>>>(
      static_cast<const uint4*>(x), c.T, units, c.k, row_of, static_cast<uint4*>(x_perm));
  return check_launch("permute");
}

moe_status_t launch_gather_sum(const moe_config_t& c, const void* Y, const int32_t* row_of, const float* w,
                               const void* add_act, const float* add_f32, void* out, hipStream_t s) {
  const int units = static_cast<int>(static_cast<int64_t>(c.d) * act_bytes(c) / 16);
  const int grid = static_cast<int>(ceil_div(c.T, 4));
  if (c.act_dtype == MOE_BF16)
    gather_sum_kernel<uint16_t><<<grid, 256, 0, s>>>(static_cast<const uint4*>(Y), c.T, units, c.k, row_of, w,
                                                     static_cast<const uint4*>(add_act),
                                                     reinterpret_cast<const float4*>(add_f32),
                                                     static_cast<uint4*>(out));
  else
    gather_sum_kernel<float><<<grid, 256, 0, s>>>(static_cast<const uint4*>(Y), c.T, units, c.k, row_of, w,
                                                  static_cast<const uint4*>(add_act),
                                                  reinterpret_cast<const float4*>(add_f32),
                                                  static_cast<uint4*>(out));
  return check_launch("gather_sum");
}

moe_status_t launch_combine_bwd(const moe_config_t& c, const void* dy, const void* Y, const int32_t* row_of,
                                const float* w, void* dY, float* dw, hipStream_t s) {
  const int units = static_cast<int>(static_cast<int64_t>(c.d) * act_bytes(c) / 16);
  const int grid = static_cast<int>(ceil_div(c.T, 4));
  if (c.act_dtype == MOE_BF16)
    combine_bwd_kernel<uint16_t><<<grid, 256, 0, s>>>(static_cast<const uint4*>(dy), static_cast<const uint4*>(Y),
                                                      c.T, units, c.k, row_of, w, static_cast<uint4*>(dY), dw);
  else
    combine_bwd_kernel<float><<<grid, 256, 0, s>>>(static_cast<const uint4*>(dy), static_cast<const uint4*>(Y),
                                                   c.T, units, c.k, row_of, w, static_cast<uint4*>(dY), dw);
  return check_launch("combine_bwd");
}

}  // namespace moe
