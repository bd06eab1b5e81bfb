// fp32-accumulating FMA GEMM (grouped or not) and the elementwise SwiGLU kernels of the
// fp32 path.  Used for the fp32 router GEMMs (logits = x Wg^T, dWg = dlogits^T x,
// dx_r = dlogits Wg) and for every expert GEMM when activations are fp32.
//
// C(m, n) = sum_k A(m, k) B(k, n), with A stored [M][K] (K_MAJOR) or [K][M] (MN_MAJOR)
// and B stored [N][K] (K_MAJOR) or [K][N] (MN_MAJOR).  64x64 tiles, 16-deep K steps,
// 256 threads each owning a 4x4 strided block of the tile.
#include <type_traits>

#include "moe_internal.h"

namespace moe {

namespace {

constexpr int TM = 64, TN = 64, TK = 16;

template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

template <typename TA, typename TB, int AMAJ, int BMAJ, int RAG, int EPI>
__global__ __launch_bounds__(256) void gemm_fma_kernel(GemmDesc g) {
  __shared__ float As[TK][TM + 1];
  __shared__ float Bs[TK][TN + 1];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int grp = blockIdx.z;
  int m_begin = 0, m_end = g.M, k_begin = 0, k_end = g.K;
  if (RAG == RAGGED_M) {
    m_begin = g.offsets ? g.offsets[grp] : 0;
    m_end = g.offsets ? g.offsets[grp + 1] : g.range_end;
  } else {
    k_begin = g.offsets ? g.offsets[grp] : 0;
    k_end = g.offsets ? g.offsets[grp + 1] : g.range_end;
  }
  const int m0 = m_begin + blockIdx.y * TM;
  const int n0 = blockIdx.x * TN;
  if (m0 >= m_end) return;
  const TA* A = static_cast<const TA*>(g.A);
  const TB* B = static_cast<const TB*>(g.B) + (RAG == RAGGED_M ? grp * g.b_gstride : 0);
  float acc[4][4] = {};
  for (int k0 = k_begin; k0 < k_end; k0 += TK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + 256 * i;
      int mm, kk;
      if (AMAJ == K_MAJOR) { mm = id / TK; kk = id % TK; } else { kk = id / TM; mm = id % TM; }
      const int m = m0 + mm, k = k0 + kk;
      float v = 0.0f;
      if (m < m_end && k < k_end) v = AMAJ == K_MAJOR ? ld(A, (int64_t)m * g.lda + k) : ld(A, (int64_t)k * g.lda + m);
      As[kk][mm] = v;
      int nn;
      if (BMAJ == K_MAJOR) { nn = id / TK; kk = id % TK; } else { kk = id / TN; nn = id % TN; }
      const int n = n0 + nn, k2 = k0 + kk;
      float u = 0.0f;
      if (n < g.N && k2 < k_end) u = BMAJ == K_MAJOR ? ld(B, (int64_t)n * g.ldb + k2) : ld(B, (int64_t)k2 * g.ldb + n);
      Bs[kk][nn] = u;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* C = static_cast<float*>(g.C) + (RAG == RAGGED_K ? grp * g.c_gstride : 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty + 16 * i;
    if (m >= m_end) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx + 16 * j;
      if (n >= g.N) continue;
      float v = acc[i][j];
      if (EPI == EPI_STORE_BIAS) v += g.bias[n];
      if (g.beta) v += C[(int64_t)m * g.ldc + n];
      C[(int64_t)m * g.ldc + n] = v;
    }
  }
}

__global__ void swiglu_fwd_kernel(Glu glu, const float* __restrict__ H, float* __restrict__ Act, int64_t rows,
                                  int F) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= rows * F) return;
  const int64_t r = i / F;
  const int c = (int)(i % F);
  const float gt = H[r * 2 * F + c], up = H[r * 2 * F + F + c];
  Act[i] = glu.kind == 0 ? gt / (1.0f + expf(-gt)) * up : glu_f(glu, gt, up);
}

__global__ void swiglu_bwd_kernel(Glu glu, const float* __restrict__ H, const float* __restrict__ dAct,
                                  float* __restrict__ dH, int64_t rows, int F) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= rows * F) return;
  const int64_t r = i / F;
  const int c = (int)(i % F);
  const float gt = H[r * 2 * F + c], up = H[r * 2 * F + F + c];
  const float da = dAct[i];
  if (glu.kind != 0) {
    float dg, du;
    glu_grad_f(glu, gt, up, da, dg, du);
    dH[r * 2 * F + c] = dg;
    dH[r * 2 * F + F + c] = du;
    return;
  }
  const float s = 1.0f / (1.0f + expf(-gt));
  dH[r * 2 * F + c] = da * up * s * (1.0f + gt * (1.0f - s));
  dH[r * 2 * F + F + c] = da * gt * s;
}

template <typename TA, typename TB, int AMAJ, int BMAJ, int RAG, int EPI>
void launch_one(const GemmDesc& g, hipStream_t s) {
  dim3 grid;
  grid.x = (unsigned)ceil_div(g.N, TN);
  if (RAG == RAGGED_M) {
    grid.y = (unsigned)ceil_div(g.offsets ? g.rows_upper : g.range_end, TM);
    grid.z = g.offsets ? g.G : 1;
  } else {
    grid.y = (unsigned)ceil_div(g.M, TM);
    grid.z = g.offsets ? g.G : 1;
  }
  gemm_fma_kernel<TA, TB, AMAJ, BMAJ, RAG, EPI><<<grid, 256, 0, s>>>(g);
}

}  // namespace

moe_status_t launch_gemm_fma(const GemmDesc& g, hipStream_t s) {
  if (g.c_type != MOE_F32) return fail(MOE_ERR_UNSUPPORTED, "fma gemm: output must be fp32");
  const bool a16 = g.a_type == MOE_BF16, b16 = g.b_type == MOE_BF16;
  const int key = (a16 << 6) | (b16 << 5) | (g.a_major << 4) | (g.b_major << 3) | (g.ragged << 2) | g.epi;
#define MOE_FMA(TA, TB, AM, BM, RG, EP)                                                            \
  case (((std::is_same<TA, uint16_t>::value) << 6) | ((std::is_same<TB, uint16_t>::value) << 5) | \
        (AM << 4) | (BM << 3) | (RG << 2) | EP):                                                   \
    launch_one<TA, TB, AM, BM, RG, EP>(g, s);                                                      \
    break;
  switch (key) {
    // router logits: x (fp32 or bf16) [T][d] times Wg [E][d]
    MOE_FMA(float, float, K_MAJOR, K_MAJOR, RAGGED_M, EPI_STORE)
    MOE_FMA(float, float, K_MAJOR, K_MAJOR, RAGGED_M, EPI_STORE_BIAS)
    MOE_FMA(uint16_t, float, K_MAJOR, K_MAJOR, RAGGED_M, EPI_STORE)
    MOE_FMA(uint16_t, float, K_MAJOR, K_MAJOR, RAGGED_M, EPI_STORE_BIAS)
    // dWg = dlogits^T x
    MOE_FMA(float, float, MN_MAJOR, MN_MAJOR, RAGGED_K, EPI_STORE)
    MOE_FMA(float, uint16_t, MN_MAJOR, MN_MAJOR, RAGGED_K, EPI_STORE)
    // dx_r = dlogits Wg ; fp32 expert dgrad
    MOE_FMA(float, float, K_MAJOR, MN_MAJOR, RAGGED_M, EPI_STORE)
    default:
      return fail(MOE_ERR_UNSUPPORTED, "fma gemm: unsupported operand combination (key %d)", key);
  }
#undef MOE_FMA
  return check_launch("gemm_fma");
}

moe_status_t launch_swiglu_fwd_elementwise(Glu glu, const float* H, float* Act, int64_t rows, int F, hipStream_t s) {
  const int64_t n = rows * F;
  if (n > 0) swiglu_fwd_kernel<<<(unsigned)ceil_div(n, 256), 256, 0, s>>>(glu, H, Act, rows, F);
  return check_launch("swiglu_fwd");
}

moe_status_t launch_swiglu_bwd_elementwise(Glu glu, const float* H, const float* dAct, float* dH, int64_t rows, int F,
                                           hipStream_t s) {
  const int64_t n = rows * F;
  if (n > 0) swiglu_bwd_kernel<<<(unsigned)ceil_div(n, 256), 256, 0, s>>>(glu, H, dAct, dH, rows, F);
  return check_launch("swiglu_bwd");
}

}  // namespace moe
