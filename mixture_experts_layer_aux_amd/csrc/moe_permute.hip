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

// Expert id of a slot, clamped into [0, E): ids outside it break the caller's contract,
// and clamping keeps every access that the id addresses inside its buffer.
__device__ __forceinline__ int expert_of(const int32_t* __restrict__ idx, int64_t i, int E) {
  return min(max(idx[i], 0), E - 1);
}

__global__ __launch_bounds__(64) void chunk_hist_kernel(const int32_t* __restrict__ idx, int T, int E, int k,
                                                        int32_t* __restrict__ blk_hist) {
  extern __shared__ int hist[];
  for (int e = threadIdx.x; e < E; e += 64) hist[e] = 0;
  __syncthreads();
  const int t = blockIdx.x * kChunk + threadIdx.x;
  if (t < T)
    for (int j = 0; j < k; ++j) atomicAdd(&hist[expert_of(idx, static_cast<int64_t>(t) * k + j, E)], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 64) blk_hist[static_cast<int64_t>(blockIdx.x) * E + e] = hist[e];
}

// Per expert column: blk_base[b][e] = sum_{b' < b} blk_hist[b'][e]; counts[e] = total.
// 256 threads = 16 experts x 16 contiguous parts of the chunks, so that each thread walks
// few chunks (their loads unrolled and in flight together) and the grid spans E / 16
// blocks.
constexpr int kScanParts = 16, kScanCols = 256 / kScanParts;
__global__ __launch_bounds__(256) void chunk_scan_kernel(const int32_t* __restrict__ blk_hist, int nblk, int E,
                                                         int32_t* __restrict__ blk_base,
                                                         int32_t* __restrict__ counts) {
  __shared__ int part[kScanParts][kScanCols];
  const int c = threadIdx.x % kScanCols, r = threadIdx.x / kScanCols;
  const int e = blockIdx.x * kScanCols + c;
  const int q = (nblk + kScanParts - 1) / kScanParts;
  const int b0 = min(nblk, r * q), b1 = min(nblk, b0 + q);
  int s = 0;
  if (e < E) {
#pragma unroll 8
    for (int b = b0; b < b1; ++b) s += blk_hist[static_cast<int64_t>(b) * E + e];
  }
  part[r][c] = s;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < r; ++i) base += part[i][c];
  if (e < E) {
#pragma unroll 8
    for (int b = b0; b < b1; ++b) {
      const int v = blk_hist[static_cast<int64_t>(b) * E + e];
      blk_base[static_cast<int64_t>(b) * E + e] = base;
      base += v;
    }
    if (r == kScanParts - 1) counts[e] = base;
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
  for (int j = 0; j < k && ok; ++j) mask[expert_of(idx, static_cast<int64_t>(t) * k + j, E)] = 0ull;
  __syncthreads();
  for (int j = 0; j < k && ok; ++j) atomicOr(&mask[expert_of(idx, static_cast<int64_t>(t) * k + j, E)], 1ull << lane);
  __syncthreads();
  if (!ok) return;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int j = 0; j < k; ++j) {
    const int e = expert_of(idx, static_cast<int64_t>(t) * k + j, E);
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
  typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
  const u32x4_nt* src = reinterpret_cast<const u32x4_nt*>(x) + static_cast<int64_t>(t) * units;
  u32x4_nt* dst = reinterpret_cast<u32x4_nt*>(x_perm);
  for (int u = lane; u < units; u += 64) {
    const u32x4_nt v = src[u];
    for (int j = 0; j < k; ++j) {
      const int r = __shfl(my_r, j, 64);
      __builtin_nontemporal_store(v, dst + static_cast<int64_t>(r) * units + u);   // written once
    }
  }
}

// Groups of 8 consecutive elements <-> fp32, for the two storage types.
// Row strips: a row of d values is walked in blocks of up to 512 values (64 lanes x 8);
// in a block of nb lanes, lane l holds the 4-value chunks c0 = 128 m + l and c1 = c0 + nb,
// so each access instruction of the wave covers one contiguous run of the row (whole cache
// lines) rather than every other 16 bytes of it.
// NT: a stream touched once (each expert-output row in the combine, dy, the written
// gradients), loaded and stored with the non-temporal hint so it does not displace reused
// data (the gate weight, rows still to be gathered) from the caches.
typedef float f32x4_nt __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_nt __attribute__((ext_vector_type(2)));
template <bool NT, typename V>
__device__ __forceinline__ V ld(const V* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT, typename V>
__device__ __forceinline__ void st(V* p, V v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}
template <typename T> struct R8;
template <> struct R8<float> {
  template <bool NT = false>
  __device__ __forceinline__ static void load(const void* base, int64_t row, int c0, int c1, float* f) {
    const f32x4_nt* p = reinterpret_cast<const f32x4_nt*>(static_cast<const float*>(base) + row);
    const f32x4_nt a = ld<NT>(p + c0), b = ld<NT>(p + c1);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
  template <bool NT = false>
  __device__ __forceinline__ static void store(void* base, int64_t row, int c0, int c1, const float* f) {
    f32x4_nt* p = reinterpret_cast<f32x4_nt*>(static_cast<float*>(base) + row);
    st<NT>(p + c0, f32x4_nt{f[0], f[1], f[2], f[3]});
    st<NT>(p + c1, f32x4_nt{f[4], f[5], f[6], f[7]});
  }
};
template <> struct R8<uint16_t> {
  template <bool NT = false>
  __device__ __forceinline__ static void load(const void* base, int64_t row, int c0, int c1, float* f) {
    const u32x2_nt* p = reinterpret_cast<const u32x2_nt*>(static_cast<const uint16_t*>(base) + row);
    const u32x2_nt a = ld<NT>(p + c0), b = ld<NT>(p + c1);
    const uint32_t w[4] = {a.x, a.y, b.x, b.y};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  template <bool NT = false>
  __device__ __forceinline__ static void store(void* base, int64_t row, int c0, int c1, const float* f) {
    u32x2_nt* p = reinterpret_cast<u32x2_nt*>(static_cast<uint16_t*>(base) + row);
    st<NT>(p + c0, u32x2_nt{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3])});
    st<NT>(p + c1, u32x2_nt{pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])});
  }
};

// out[t] = sum_j w[t,j] * Y[row_of[t,j]] (+ a1_scale[t] * add1[t]) (+ add2[t])
//          (+ r1_coef[t] * r1_vec), fp32 accumulation in slot order then addend order; w
// NULL means 1, a1_scale NULL means 1.  The combine (Y fp32 expert outputs, add1 the
// shared expert's output, a1_scale its sigmoid gate) and the unpermute-reduce of the
// backward (Y the per-row input gradients, add1 the shared expert's, add2 the router's,
// r1 the shared gate's input gradient dl_t Wsg) share it.
template <typename TY, typename TA1, typename TO>
__global__ __launch_bounds__(256) void gather_sum_kernel(const void* __restrict__ Y, int Tn, int groups, int k,
                                                         const int32_t* __restrict__ row_of,
                                                         const float* __restrict__ w,
                                                         const void* __restrict__ add1,
                                                         const float* __restrict__ a1_scale,
                                                         const float* __restrict__ add2,
                                                         const float* __restrict__ r1_coef,
                                                         const float* __restrict__ r1_vec, void* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int my_r = lane < k ? row_of[static_cast<int64_t>(t) * k + lane] : 0;
  const float my_w = (lane < k && w) ? w[static_cast<int64_t>(t) * k + lane] : 1.0f;
  const int d = groups * 8;
  // every lane stays in the loop (the row shuffles read lanes of the whole wave); lanes
  // past the end of a short last block only skip their memory accesses
  for (int m = 0; 64 * m < groups; ++m) {
    const int nb = min(64, groups - 64 * m);
    const bool on = lane < nb;
    const int c0 = 128 * m + lane, c1 = c0 + nb;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    const int64_t gi = static_cast<int64_t>(t) * d;
    // the addends are loaded first, so that their latency overlaps the gathered rows'
    // (they are still added after the slots)
    float fa1[8] = {}, fa2[8] = {};
    if (on && add1) R8<TA1>::template load<true>(add1, gi, c0, c1, fa1);
    if (on && add2) R8<float>::load<true>(add2, gi, c0, c1, fa2);
    // slots eight, then four at a time: the rows are loaded before any is added, so each
    // lane has that many loads in flight; the sum still runs in slot order
    int j = 0;
    for (; j + 8 <= k; j += 8) {
      float f[8][8] = {}, wj[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int r = __shfl(my_r, j + q, 64);
        wj[q] = __shfl(my_w, j + q, 64);
        if (on) R8<TY>::template load<true>(Y, static_cast<int64_t>(r) * d, c0, c1, f[q]);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += wj[q] * f[q][i];
    }
    for (; j + 4 <= k; j += 4) {
      float f[4][8] = {}, wj[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = __shfl(my_r, j + q, 64);
        wj[q] = __shfl(my_w, j + q, 64);
        if (on) R8<TY>::template load<true>(Y, static_cast<int64_t>(r) * d, c0, c1, f[q]);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += wj[q] * f[q][i];
    }
    for (; j < k; ++j) {
      const int r = __shfl(my_r, j, 64);
      const float wj = __shfl(my_w, j, 64);
      float f[8] = {};
      if (on) R8<TY>::template load<true>(Y, static_cast<int64_t>(r) * d, c0, c1, f);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += wj * f[i];
    }
    if (!on) continue;
    if (add1) {
      if (a1_scale) {
        const float sc = a1_scale[t];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += sc * fa1[i];
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += fa1[i];
      }
    }
    if (add2) {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += fa2[i];
    }
    if (r1_coef) {
      float v[8];
      R8<float>::load(r1_vec, 0, c0, c1, v);
      const float cf = r1_coef[t];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += cf * v[i];
    }
    R8<TO>::template store<true>(out, gi, c0, c1, acc);
  }
}

// dY_perm[row_of[t,j]] = w[t,j] * dy[t]  (activation dtype);
// dw[t,j] = <dy[t], Y_perm[row_of[t,j]]>  (fp32: per lane over its columns in order, then
// a fixed butterfly across the wave);  dY_s[t] = dy[t] in the activation dtype (optional),
// times gs[t] for a gated shared expert, and then dl_s[t] = gs (1 - gs) <dy[t], Y_s[t]>,
// the gradient of the gate's logit.
// One wave per token, one pass over the columns: dy is loaded once per column group and the
// k rows four at a time; KMAX >= k partial sums live in registers.
template <typename TACT, int KMAX>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const float* __restrict__ dy,
                                                          const float* __restrict__ Y, int Tn, int groups,
                                                          int k, const int32_t* __restrict__ row_of,
                                                          const float* __restrict__ w, void* __restrict__ dY,
                                                          float* __restrict__ dw, void* __restrict__ dY_s,
                                                          const float* __restrict__ gs,
                                                          const float* __restrict__ Ys,
                                                          float* __restrict__ dl_s) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const float gs_t = gs ? gs[t] : 1.0f;
  float part_s = 0.0f;
  const int my_r = lane < k ? row_of[static_cast<int64_t>(t) * k + lane] : 0;
  const float my_w = lane < k ? w[static_cast<int64_t>(t) * k + lane] : 0.0f;
  const int d = groups * 8;
  const int64_t t0 = static_cast<int64_t>(t) * d;
  float part[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) part[j] = 0.0f;
  for (int m = 0; 64 * m < groups; ++m) {
    const int nb = min(64, groups - 64 * m);
    const bool on = lane < nb;  // all lanes stay for the shuffles; off lanes add zeros
    const int c0 = 128 * m + lane, c1 = c0 + nb;
    float g[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) g[i] = 0.0f;
    if (on) R8<float>::load<true>(dy, t0, c0, c1, g);
    if (on && dY_s) {
      if (gs) {
        float gg[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) gg[i] = gs_t * g[i];
        R8<TACT>::template store<true>(dY_s, t0, c0, c1, gg);
      } else {
        R8<TACT>::template store<true>(dY_s, t0, c0, c1, g);
      }
    }
    if (Ys) {
      float ys[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) ys[i] = 0.0f;
      if (on) R8<float>::load<true>(Ys, t0, c0, c1, ys);
#pragma unroll
      for (int i = 0; i < 8; ++i) part_s += g[i] * ys[i];
    }
#pragma unroll
    for (int j0 = 0; j0 < KMAX; j0 += 4) {
      if (j0 < k) {
        float y[4][8];
        int r[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          r[q] = __shfl(my_r, j0 + q, 64);
#pragma unroll
          for (int i = 0; i < 8; ++i) y[q][i] = 0.0f;
          if (on && j0 + q < k) R8<float>::load<true>(Y, static_cast<int64_t>(r[q]) * d, c0, c1, y[q]);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (j0 + q < k) {
            const float wj = __shfl(my_w, j0 + q, 64);
            float gw[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              part[j0 + q] += g[i] * y[q][i];
              gw[i] = g[i] * wj;
            }
            if (on && dY) R8<TACT>::template store<true>(dY, static_cast<int64_t>(r[q]) * d, c0, c1, gw);
          }
        }
      }
    }
  }
  float my_dw = 0.0f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k) {
      const float v = wave_sum(part[j]);
      if (lane == j) my_dw = v;
    }
  }
  if (lane < k) dw[static_cast<int64_t>(t) * k + lane] = my_dw;
  if (dl_s) {
    const float v = wave_sum(part_s);
    if (lane == 0) dl_s[t] = gs_t * (1.0f - gs_t) * v;
  }
}

// The shared expert's sigmoid gate (The Ultimate MoE Training Handbook, §3.4 Shared
// experts): gs[t] = sigma(<x[t], Wsg>), one wave per token, fp32 dot in a fixed order.
template <typename TX>
__global__ __launch_bounds__(256) void shared_gate_kernel(const void* __restrict__ x, const float* __restrict__ Wsg,
                                                          int Tn, int groups, float* __restrict__ gs) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int64_t t0 = static_cast<int64_t>(t) * groups * 8;
  float acc = 0.0f;
  for (int m = 0; 64 * m < groups; ++m) {
    const int nb = min(64, groups - 64 * m);
    if (lane < nb) {
      const int c0 = 128 * m + lane, c1 = c0 + nb;
      float f[8], v[8];
      R8<TX>::load(x, t0, c0, c1, f);
      R8<float>::load(Wsg, 0, c0, c1, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc += f[i] * v[i];
    }
  }
  acc = wave_sum(acc);
  if (lane == 0) gs[t] = 1.0f / (1.0f + expf(-acc));
}

// dWsg = sum_t dl_s[t] x[t]: per chunk of 256 tokens and column, partial sums in token
// order; then the chunks summed in order.
constexpr int kGateChunk = 256;
template <typename TX>
__global__ __launch_bounds__(256) void shared_gate_wgrad_part_kernel(const void* __restrict__ x,
                                                                     const float* __restrict__ dl, int Tn, int d,
                                                                     float* __restrict__ part) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= d) return;
  const int t0 = blockIdx.y * kGateChunk, t1 = min(Tn, t0 + kGateChunk);
  float acc = 0.0f;
  for (int t = t0; t < t1; ++t) acc += dl[t] * Elem<TX>::load(static_cast<const TX*>(x), static_cast<int64_t>(t) * d + c);
  part[static_cast<int64_t>(blockIdx.y) * d + c] = acc;
}
__global__ __launch_bounds__(256) void shared_gate_wgrad_final_kernel(const float* __restrict__ part, int nchunk,
                                                                      int d, float* __restrict__ dWsg, int beta) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= d) return;
  float acc = 0.0f;
  for (int q = 0; q < nchunk; ++q) acc += part[static_cast<int64_t>(q) * d + c];
  dWsg[c] = beta ? dWsg[c] + acc : acc;
}

}  // namespace

int64_t permute_num_chunks(int T) { return ceil_div(T, kChunk); }

moe_status_t launch_permute(const moe_config_t& c, const void* x, const int32_t* idx, int32_t* offsets,
                            int32_t* row_of, int32_t* token_of, void* x_perm, int32_t* blk_hist,
                            int32_t* blk_base, int32_t* counts_ws, bool hist_ready, hipStream_t s,
                            int elem_bytes) {
  const int nblk = static_cast<int>(permute_num_chunks(c.T));
  if (!hist_ready)
    chunk_hist_kernel<<<nblk, 64, c.E * sizeof(int), s>>>(idx, c.T, c.E, c.k, blk_hist);
  chunk_scan_kernel<<<static_cast<int>(ceil_div(c.E, kScanCols)), 256, 0, s>>>(blk_hist, nblk, c.E, blk_base, counts_ws);
  offsets_kernel<<<1, 1024, 0, s>>>(counts_ws, c.E, offsets);
  permute_index_kernel<<<nblk, 64, c.E * sizeof(unsigned long long), s>>>(idx, c.T, c.E, c.k, offsets, blk_base,
                                                                          row_of, token_of);
  if (x_perm) {   // NULL: the grouped GEMMs read the token rows of x through token_of instead
    const int units = static_cast<int>(static_cast<int64_t>(c.d) * (elem_bytes ? elem_bytes : act_bytes(c)) / 16);
    permute_copy_kernel<<<static_cast<int>(ceil_div(c.T, 4)), 256, 0, s>>>(
        static_cast<const uint4*>(x), c.T, units, c.k, row_of, static_cast<uint4*>(x_perm));
  }
  return check_launch("permute");
}

moe_status_t launch_combine(const moe_config_t& c, const float* Y, const int32_t* row_of, const float* w,
                            const float* Y_s, const float* gs, float* y, hipStream_t s) {
  const int groups = c.d / 8;
  gather_sum_kernel<float, float, float><<<static_cast<int>(ceil_div(c.T, 4)), 256, 0, s>>>(
      Y, c.T, groups, c.k, row_of, w, Y_s, gs, nullptr, nullptr, nullptr, y);
  return check_launch("combine");
}

moe_status_t launch_unpermute_reduce(const moe_config_t& c, const float* dX, const int32_t* row_of,
                                     const float* dx_s, const float* dx_r, const float* dl_s, const float* Wsg,
                                     float* dx, hipStream_t s) {
  const int groups = c.d / 8;
  const int grid = static_cast<int>(ceil_div(c.T, 4));
  gather_sum_kernel<float, float, float><<<grid, 256, 0, s>>>(dX, c.T, groups, c.k, row_of, nullptr, dx_s, nullptr,
                                                              dx_r, dl_s, dl_s ? Wsg : nullptr, dx);
  return check_launch("unpermute_reduce");
}

size_t shared_gate_part_bytes(const moe_config_t& c) {
  return c.shared_gate ? static_cast<size_t>(ceil_div(c.T, kGateChunk)) * c.d * 4 : 0;
}

moe_status_t launch_shared_gate(const moe_config_t& c, const void* x, const float* Wsg, float* gs, hipStream_t s) {
  const int grid = static_cast<int>(ceil_div(c.T, 4));
  if (c.act_dtype == MOE_BF16)
    shared_gate_kernel<uint16_t><<<grid, 256, 0, s>>>(x, Wsg, c.T, c.d / 8, gs);
  else
    shared_gate_kernel<float><<<grid, 256, 0, s>>>(x, Wsg, c.T, c.d / 8, gs);
  return check_launch("shared_gate");
}

moe_status_t launch_shared_gate_bwd(const moe_config_t& c, const void* x, const float* dl_s, float* dWsg,
                                    float* part, hipStream_t s, int beta) {
  const int nchunk = static_cast<int>(ceil_div(c.T, kGateChunk));
  const dim3 grid(static_cast<unsigned>(ceil_div(c.d, 256)), static_cast<unsigned>(nchunk));
  if (c.act_dtype == MOE_BF16)
    shared_gate_wgrad_part_kernel<uint16_t><<<grid, 256, 0, s>>>(x, dl_s, c.T, c.d, part);
  else
    shared_gate_wgrad_part_kernel<float><<<grid, 256, 0, s>>>(x, dl_s, c.T, c.d, part);
  shared_gate_wgrad_final_kernel<<<static_cast<int>(ceil_div(c.d, 256)), 256, 0, s>>>(part, nchunk, c.d, dWsg, beta);
  return check_launch("shared_gate_bwd");
}

moe_status_t launch_combine_bwd(const moe_config_t& c, const float* dy, const float* Y, const int32_t* row_of,
                                const float* w, void* dY, float* dw, void* dY_s, const float* gs, const float* Ys,
                                float* dl_s, hipStream_t s) {
  const int groups = c.d / 8;
  const int grid = static_cast<int>(ceil_div(c.T, 4));
  const bool bf = c.act_dtype == MOE_BF16;
#define MOE_CB(KM)                                                                                        \
  if (c.k <= KM) {                                                                                        \
    if (bf) combine_bwd_kernel<uint16_t, KM><<<grid, 256, 0, s>>>(dy, Y, c.T, groups, c.k, row_of, w, dY, dw, dY_s, \
                                                                  gs, Ys, dl_s);                            \
    else combine_bwd_kernel<float, KM><<<grid, 256, 0, s>>>(dy, Y, c.T, groups, c.k, row_of, w, dY, dw, dY_s,    \
                                                            gs, Ys, dl_s);                                  \
    return check_launch("combine_bwd");                                                                   \
  }
  MOE_CB(8)
  MOE_CB(16)
  MOE_CB(32)
#undef MOE_CB
  return fail(MOE_ERR_UNSUPPORTED, "combine_bwd: k above 32");
}

}  // namespace moe
