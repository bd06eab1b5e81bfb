// The router's linear layer in fp32 on the bf16 matrix cores.
//
// The Ultimate MoE Training Handbook, §3.1 Precision: the router GEMM runs in fp32.  With
// bf16 activations x is exact in bf16, and every fp32 value v splits exactly enough into
// three bf16 parts, hi = bf16(v), mid = bf16(v - hi), lo = bf16(v - hi - mid) (24 significant
// bits in all, the differences exact in fp32).  So
//   logits = x Wg^T            = x hi^T + x mid^T + x lo^T            (each product exact)
//   dWg    = dlogits^T x       = hi^T x + mid^T x + lo^T x
//   dx_r   = dlogits Wg        ~ a1 b1 + a1 b2 + a2 b1 + a1 b3 + a2 b2 + a3 b1
// (a = dlogits, b = Wg parts; the dropped terms are below 2^-24 of the product) run as
// bf16 GEMMs with fp32 accumulation: the parts of the fp32 operand are stacked along the
// output (the three partial results then summed in a fixed order) or, for dx_r, along the
// reduction.  The GEMMs are the grouped bf16 MFMA kernel with a single group.
#include "moe_internal.h"

namespace moe {

namespace {

// out[r * row_stride + q * slot_stride + c] = part[pat[q]] of src[r][c], q < nslot.
__global__ __launch_bounds__(256) void split_parts_kernel(const float* __restrict__ src, int64_t rows, int cols,
                                                          uint16_t* __restrict__ out, int64_t row_stride,
                                                          int64_t slot_stride, int nslot, uint32_t pat) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= rows * cols) return;
  const int64_t r = i / cols;
  const int c = static_cast<int>(i - r * cols);
  const float v = src[i];
  uint16_t p[3];
  p[0] = f32_to_bf16(v);
  const float r1 = v - bf16_to_f32(p[0]);
  p[1] = f32_to_bf16(r1);
  p[2] = f32_to_bf16(r1 - bf16_to_f32(p[1]));
  uint16_t* o = out + r * row_stride + c;
  for (int q = 0; q < nslot; ++q) o[q * slot_stride] = p[(pat >> (2 * q)) & 3u];
}

// out[r][c] = (in[r][c] + in[r][c + stride]) + in[r][c + 2 stride] (+ bias[c]), added into
// out when beta
__global__ __launch_bounds__(256) void sum_parts_kernel(const float* __restrict__ in, int64_t rows, int cols,
                                                        int64_t in_ld, int64_t stride, float* __restrict__ out,
                                                        int64_t out_ld, const float* __restrict__ bias, int beta) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= rows * cols) return;
  const int64_t r = i / cols;
  const int c = static_cast<int>(i - r * cols);
  const float* p = in + r * in_ld + c;
  float v = (p[0] + p[stride]) + p[2 * stride];
  if (bias) v += bias[c];
  if (beta) v = out[r * out_ld + c] + v;
  out[r * out_ld + c] = v;
}

// Column sums in a fixed order: partial sums over 64-row chunks (rows in order), then per
// column 16 interleaved runs of chunks (run g: chunks g, g + 16, ..., in order), then the
// 16 run sums in run order.  Each thread keeps 16 loads in flight, so neither pass waits on
// one load at a time.
constexpr int kColChunk = 64, kColRuns = 16, kColUnroll = 16;
__global__ __launch_bounds__(256) void colsum_part_kernel(const float* __restrict__ X, int rows, int cols,
                                                          float* __restrict__ part) {
  const int col = blockIdx.x * 256 + threadIdx.x;
  if (col >= cols) return;
  const int r0 = blockIdx.y * kColChunk, r1 = min(rows, r0 + kColChunk);
  float s = 0.0f;
  int r = r0;
  for (; r + kColUnroll <= r1; r += kColUnroll) {
    float v[kColUnroll];
#pragma unroll
    for (int u = 0; u < kColUnroll; ++u) v[u] = X[static_cast<int64_t>(r + u) * cols + col];
#pragma unroll
    for (int u = 0; u < kColUnroll; ++u) s += v[u];
  }
  for (; r < r1; ++r) s += X[static_cast<int64_t>(r) * cols + col];
  part[static_cast<int64_t>(blockIdx.y) * cols + col] = s;
}
// block: 64 columns x kColRuns runs (1024 threads)
__global__ __launch_bounds__(1024) void colsum_final_kernel(const float* __restrict__ part, int nchunk, int cols,
                                                            float* __restrict__ out, int beta) {
  __shared__ float srun[kColRuns][64];
  const int c = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int col = blockIdx.x * 64 + c;
  float s = 0.0f;
  if (col < cols) {
    int q = g;
    for (; q + (kColUnroll - 1) * kColRuns < nchunk; q += kColUnroll * kColRuns) {
      float v[kColUnroll];
#pragma unroll
      for (int u = 0; u < kColUnroll; ++u) v[u] = part[static_cast<int64_t>(q + u * kColRuns) * cols + col];
#pragma unroll
      for (int u = 0; u < kColUnroll; ++u) s += v[u];
    }
    for (; q < nchunk; q += kColRuns) s += part[static_cast<int64_t>(q) * cols + col];
  }
  srun[g][c] = s;
  __syncthreads();
  if (g == 0 && col < cols) {
    float t = 0.0f;
#pragma unroll
    for (int h = 0; h < kColRuns; ++h) t += srun[h][c];
    out[col] = beta ? out[col] + t : t;
  }
}

// slot patterns (2 bits per slot: part index 0 = hi, 1 = mid, 2 = lo)
constexpr uint32_t kPat3 = 0u | (1u << 2) | (2u << 4);                                          // hi mid lo
constexpr uint32_t kPatA6 = 0u | (0u << 2) | (1u << 4) | (0u << 6) | (1u << 8) | (2u << 10);  // a1 a1 a2 a1 a2 a3
constexpr uint32_t kPatB6 = 0u | (1u << 2) | (0u << 4) | (2u << 6) | (1u << 8) | (0u << 10);  // b1 b2 b1 b3 b2 b1

moe_status_t split(const float* src, int64_t rows, int cols, uint16_t* out, int64_t row_stride, int64_t slot_stride,
                   int nslot, uint32_t pat, hipStream_t s) {
  const int64_t n = rows * cols;
  if (n == 0) return MOE_OK;
  split_parts_kernel<<<ceil_div(n, 256), 256, 0, s>>>(src, rows, cols, out, row_stride, slot_stride, nslot, pat);
  return check_launch("gate split");
}

moe_status_t sum3(const float* in, int64_t rows, int cols, int64_t in_ld, int64_t stride, float* out, int64_t out_ld,
                  const float* bias, hipStream_t s, int beta = 0) {
  const int64_t n = rows * cols;
  if (n == 0) return MOE_OK;
  sum_parts_kernel<<<ceil_div(n, 256), 256, 0, s>>>(in, rows, cols, in_ld, stride, out, out_ld, bias, beta);
  return check_launch("gate sum");
}

}  // namespace

bool gate_on_mfma(const moe_config_t& c) { return c.act_dtype == MOE_BF16 && c.E % 16 == 0; }

size_t gate_fwd_ws_bytes(const moe_config_t& c) {
  if (!gate_on_mfma(c)) return 0;
  return static_cast<size_t>(3) * c.E * c.d * 2 + 256 + static_cast<size_t>(c.T) * 3 * c.E * 4;
}

size_t gate_bwd_ws_bytes(const moe_config_t& c) {
  const size_t T = c.T, E = c.E, d = c.d;
  size_t b = ceil_div(c.T, kColChunk) * E * 4 + 256;
  if (gate_on_mfma(c)) {
    b += T * 3 * E * 2 + 256 + T * 6 * E * 2 + 256 + 6 * E * d * 2 + 256 + 3 * E * d * 4 + 256;
    b += wgrad_split_bytes(3 * c.E, c.d, c.T) + 256;   // split-K partials of dWg
  }
  return b;
}

static char* carve(char*& p, size_t n) {
  char* q = p;
  p += (n + 255) / 256 * 256;
  return q;
}

moe_status_t launch_gate_fwd_mfma(const moe_config_t& c, const void* x, const float* Wg, const float* bg,
                                  float* logits, void* ws, hipStream_t s) {
  char* p = static_cast<char*>(ws);
  uint16_t* Wg3 = reinterpret_cast<uint16_t*>(carve(p, static_cast<size_t>(3) * c.E * c.d * 2));
  float* C3 = reinterpret_cast<float*>(carve(p, static_cast<size_t>(c.T) * 3 * c.E * 4));
  MOE_TRY_INTERNAL(split(Wg, c.E, c.d, Wg3, c.d, static_cast<int64_t>(c.E) * c.d, 3, kPat3, s));
  GemmDesc g{};
  g.a_major = K_MAJOR; g.b_major = K_MAJOR; g.ragged = RAGGED_M; g.epi = EPI_STORE;
  g.a_type = g.b_type = MOE_BF16; g.c_type = MOE_F32;
  g.N = 3 * c.E; g.K = c.d;
  g.A = x; g.lda = c.d; g.B = Wg3; g.ldb = c.d; g.C = C3; g.ldc = 3 * c.E;
  g.range_end = c.T; g.G = 1;
  MOE_TRY_INTERNAL(launch_gemm_mfma(g, nullptr, s));
  return sum3(C3, c.T, c.E, 3 * c.E, c.E, logits, c.E, bg, s);
}

moe_status_t launch_colsum_ws(const float* X, int rows, int cols, float* out, float* part, hipStream_t s, int beta) {
  const int nchunk = static_cast<int>(ceil_div(rows, kColChunk));
  if (nchunk == 0) return MOE_OK;
  if (nchunk > 65535) return fail(MOE_ERR_UNSUPPORTED, "column sums: at most 65535 x 64 rows");
  colsum_part_kernel<<<dim3(static_cast<unsigned>(ceil_div(cols, 256)), nchunk), 256, 0, s>>>(X, rows, cols, part);
  colsum_final_kernel<<<static_cast<unsigned>(ceil_div(cols, 64)), 1024, 0, s>>>(part, nchunk, cols, out, beta);
  return check_launch("colsum");
}

moe_status_t launch_gate_bwd_mfma(const moe_config_t& c, const void* x, const float* Wg, const float* dlogits,
                                  float* dWg, float* dbg, float* dx_r, void* ws, hipStream_t s, int beta) {
  const int64_t T = c.T, E = c.E, d = c.d;
  char* p = static_cast<char*>(ws);
  float* part = reinterpret_cast<float*>(carve(p, ceil_div(c.T, kColChunk) * E * 4));
  uint16_t* D3 = reinterpret_cast<uint16_t*>(carve(p, T * 3 * E * 2));
  uint16_t* A6 = reinterpret_cast<uint16_t*>(carve(p, T * 6 * E * 2));
  uint16_t* B6 = reinterpret_cast<uint16_t*>(carve(p, 6 * E * d * 2));
  float* C3 = reinterpret_cast<float*>(carve(p, 3 * E * d * 4));
  // dWg = dlogits^T x: the three parts of dlogits side by side in each row.  Its [3E, d]
  // output has few tiles (48 at E = 512, d = 2048) for a reduction over all T tokens, so
  // the tokens are split into chunks whose fp32 partials are summed in chunk order first.
  const WgradSplit sp = wgrad_split(3 * c.E, c.d, c.T);
  float* P = reinterpret_cast<float*>(carve(p, wgrad_split_bytes(3 * c.E, c.d, c.T)));
  MOE_TRY_INTERNAL(split(dlogits, T, c.E, D3, 3 * E, E, 3, kPat3, s));
  GemmDesc gw{};
  gw.a_major = MN_MAJOR; gw.b_major = MN_MAJOR; gw.ragged = RAGGED_K; gw.epi = EPI_STORE;
  gw.a_type = gw.b_type = MOE_BF16; gw.c_type = MOE_F32;
  gw.M = 3 * c.E; gw.N = c.d;
  gw.A = D3; gw.lda = 3 * E; gw.B = x; gw.ldb = d; gw.C = C3; gw.ldc = d;
  gw.range_end = c.T; gw.G = 1;
  if (sp.chunks > 1) {
    gw.C = P; gw.c_gstride = 3 * E * d; gw.G = sp.chunks; gw.kchunk = sp.kchunk;
    MOE_TRY_INTERNAL(launch_gemm_mfma(gw, nullptr, s));
    MOE_TRY_INTERNAL(launch_splitk_reduce(P, sp.chunks, 3 * E * d, C3, MOE_F32, 0, s));
  } else {
    MOE_TRY_INTERNAL(launch_gemm_mfma(gw, nullptr, s));
  }
  MOE_TRY_INTERNAL(sum3(C3, E, c.d, d, E * d, dWg, d, nullptr, s, beta));
  if (dbg) MOE_TRY_INTERNAL(launch_colsum_ws(dlogits, c.T, c.E, dbg, part, s, beta));
  if (dx_r) {
    // dx_r = dlogits Wg: six part products stacked along the reduction
    MOE_TRY_INTERNAL(split(dlogits, T, c.E, A6, 6 * E, E, 6, kPatA6, s));
    MOE_TRY_INTERNAL(split(Wg, E, c.d, B6, d, E * d, 6, kPatB6, s));
    GemmDesc gx{};
    gx.a_major = K_MAJOR; gx.b_major = MN_MAJOR; gx.ragged = RAGGED_M; gx.epi = EPI_STORE;
    gx.a_type = gx.b_type = MOE_BF16; gx.c_type = MOE_F32;
    gx.N = c.d; gx.K = 6 * c.E;
    gx.A = A6; gx.lda = 6 * E; gx.B = B6; gx.ldb = d; gx.C = dx_r; gx.ldc = d;
    gx.range_end = c.T; gx.G = 1;
    MOE_TRY_INTERNAL(launch_gemm_mfma(gx, nullptr, s));
  }
  return MOE_OK;
}

}  // namespace moe
