// bf16 grouped GEMM on gfx950 matrix cores, fp32 accumulation.
//
// The expert FFNs of The Ultimate MoE Training Handbook, §3.4 (fc1 of width 2F split
// into gate and up halves, SwiGLU, fc2 back to d), run as one grouped GEMM per
// projection: each expert owns a ragged block of rows (forward, data gradient) or a
// ragged block of the reduction dimension (weight gradient).
//
// Design (per workgroup: 256 threads = 4 waves in a 2x2 grid):
//   * 256 x 256 output tile, 64-deep K steps, each wave a 128 x 128 sub-tile held as
//     4 x 4 accumulators of v_mfma_f32_32x32x16_bf16 (16 fp32 per lane each);
//   * both operands staged in LDS as [256 rows][64 k] bf16 with an XOR swizzle of the
//     16-byte chunk index ((r ^ (r >> 3)) & 7) so that fragment reads (32 consecutive
//     rows, one chunk) and transposing writes (rows 8 apart) spread over all banks;
//   * double-buffered LDS (2 x 64 KB): the next K step is fetched into registers while
//     the current one is multiplied, then written to the other buffer; one barrier per
//     step;
//   * operands stored K-contiguous are copied in 16-byte chunks; operands stored
//     row-contiguous (the weights in the data-gradient GEMMs, both operands of the
//     weight-gradient GEMMs) are read as 8 x 8 bf16 blocks and transposed in registers;
//   * a device-built tile list (per-expert prefix of row tiles) so the host never
//     reads the expert counts; empty experts get no tiles (forward) or exact-zero
//     gradients (weight gradient, zero-length reduction);
//   * row-ragged launches map workgroup h to tile (h mod 8) * ceil(tiles / 8) + h / 8:
//     workgroups are dealt round-robin to the 8 XCDs, so each XCD walks a contiguous
//     run of tiles (expert, column tile, row tile) and the tiles sharing a weight tile
//     or an activation tile run together on one L2;
//   * fused epilogues: SwiGLU (forward: H in fp32 and Act in bf16 from the same
//     accumulators, the gate and up rows of W13 interleaved per 32-row block of the B
//     tile) and the SwiGLU backward (reads the saved fp32 H, writes dH in bf16).
#include "moe_internal.h"

namespace moe {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, BK = 64, NTHR = 256;
constexpr int TILE = 256 * 64;  // bf16 elements of one operand tile

struct MfmaArgs {
  const uint16_t* A;
  int64_t lda;
  const uint16_t* B;
  int64_t ldb, b_gstride;
  void* C;
  int64_t ldc, c_gstride;
  uint16_t* C2;
  int64_t ldc2;
  const float* H;
  int64_t ldh;
  const int32_t* offsets;
  const int32_t* tile_prefix;
  int G, M, N, K, F, range_end, nN, nM;
};

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int r, int kc) { return r * 64 + ((kc ^ swz(r)) << 3); }

// 8 x 8 transpose of bf16: in[kk] holds columns 0..7 of row kk; out[cc] holds rows 0..7
// of column cc.
__device__ __forceinline__ void transpose8x8(const u32x4_t (&in)[8], u32x4_t (&out)[8]) {
#pragma unroll
  for (int cc = 0; cc < 8; ++cc) {
#pragma unroll
    for (int pq = 0; pq < 4; ++pq) {
      const uint32_t a = in[2 * pq][cc >> 1], b = in[2 * pq + 1][cc >> 1];
      out[cc][pq] = (cc & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
    }
  }
}

// Tiles of a row-ragged launch: group g has ceil(rows_g / 256) row tiles.
__global__ __launch_bounds__(1024) void tile_prefix_kernel(const int32_t* __restrict__ offsets, int G,
                                                           int32_t* __restrict__ prefix) {
  __shared__ int s[2048];
  for (int g = threadIdx.x; g < 2048; g += 1024)
    s[g] = g < G ? (offsets[g + 1] - offsets[g] + BM - 1) / BM : 0;
  __syncthreads();
  for (int off = 1; off < 2048; off <<= 1) {
    const int i0 = threadIdx.x, i1 = threadIdx.x + 1024;
    const int a0 = i0 >= off ? s[i0 - off] : 0;
    const int a1 = i1 >= off ? s[i1 - off] : 0;
    __syncthreads();
    s[i0] += a0;
    s[i1] += a1;
    __syncthreads();
  }
  for (int g = threadIdx.x; g <= G; g += 1024) prefix[g] = g == 0 ? 0 : s[g - 1];
}

template <int AMAJ, int BMAJ, int RAG, int EPI, bool OUT_F32>
__global__ __launch_bounds__(NTHR, 1) void gemm_mfma_kernel(const MfmaArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[4 * TILE];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ------------------------------------------------------------ tile of this workgroup
  int grp, mt, nt;
  int row_begin, row_end;  // RAGGED_M: rows of A/C;  RAGGED_K: rows [0, M) of C
  int k_begin, k_end;
  if (RAG == RAGGED_M) {
    const int h = blockIdx.x;
    const int total_m = p.offsets ? p.tile_prefix[p.G] : (p.range_end + BM - 1) / BM;
    const int total = total_m * p.nN;
    const int chunk = (total + 7) >> 3;
    const int q = h >> 3;
    const int L = (h & 7) * chunk + q;
    if (q >= chunk || L >= total) return;
    int g = 0;
    if (p.offsets) {
      int lo = 0, hi = p.G - 1;  // largest g with prefix[g] * nN <= L
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (p.tile_prefix[mid] * p.nN <= L) lo = mid; else hi = mid - 1;
      }
      g = lo;
    }
    const int base = p.offsets ? p.tile_prefix[g] : 0;
    const int mtiles = p.offsets ? p.tile_prefix[g + 1] - base : total_m;
    const int local = L - base * p.nN;
    nt = local / mtiles;
    mt = local - nt * mtiles;
    grp = g;
    const int gb = p.offsets ? p.offsets[g] : 0;
    row_begin = gb + mt * BM;
    row_end = p.offsets ? p.offsets[g + 1] : p.range_end;
    k_begin = 0;
    k_end = p.K;
  } else {
    const int L = blockIdx.x;
    const int per = p.nM * p.nN;
    if (L >= p.G * per) return;
    grp = L / per;
    const int local = L - grp * per;
    mt = local / p.nN;
    nt = local - mt * p.nN;
    row_begin = mt * BM;
    row_end = p.M;
    k_begin = p.offsets ? p.offsets[grp] : 0;
    k_end = p.offsets ? p.offsets[grp + 1] : p.range_end;
  }
  const int n0 = nt * BN;
  const uint16_t* Bg = p.B + (RAG == RAGGED_M ? static_cast<int64_t>(grp) * p.b_gstride : 0);

  // ------------------------------------------------------------ global -> registers
  u32x4_t ra[8], rb[8];
  auto load_a = [&](int k0) {
    if (AMAJ == K_MAJOR) {
      const int kc = tid & 7;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int r = (tid >> 3) + 32 * q;
        const int grow = min(row_begin + r, row_end - 1);
        ra[q] = *reinterpret_cast<const u32x4_t*>(p.A + static_cast<int64_t>(grow) * p.lda + k0 + kc * 8);
      }
    } else {
      const int cb = tid & 31, kb = tid >> 5;
      const int col = min(row_begin + cb * 8, p.M - 8);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int kr = k0 + kb * 8 + kk;
        if (kr < k_end)
          ra[kk] = *reinterpret_cast<const u32x4_t*>(p.A + static_cast<int64_t>(kr) * p.lda + col);
        else
          ra[kk] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };
  auto load_b = [&](int k0) {
    if (BMAJ == K_MAJOR) {
      const int kc = tid & 7;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        int n;
        if (EPI == EPI_SWIGLU_FWD)
          n = ((q & 1) ? p.F : 0) + nt * 128 + (q >> 1) * 32 + (tid >> 3);
        else
          n = min(n0 + (tid >> 3) + 32 * q, p.N - 1);
        rb[q] = *reinterpret_cast<const u32x4_t*>(Bg + static_cast<int64_t>(n) * p.ldb + k0 + kc * 8);
      }
    } else {
      const int cb = tid & 31, kb = tid >> 5;
      const int col = min(n0 + cb * 8, p.N - 8);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int kr = k0 + kb * 8 + kk;
        if (kr < k_end)
          rb[kk] = *reinterpret_cast<const u32x4_t*>(Bg + static_cast<int64_t>(kr) * p.ldb + col);
        else
          rb[kk] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };
  // ------------------------------------------------------------ registers -> LDS
  auto store_tile = [&](uint16_t* dst, const u32x4_t (&rg)[8], int major) {
    if (major == K_MAJOR) {
      const int kc = tid & 7;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int r = (tid >> 3) + 32 * q;
        *reinterpret_cast<u32x4_t*>(dst + lds_off(r, kc)) = rg[q];
      }
    } else {
      const int cb = tid & 31, kb = tid >> 5;
      u32x4_t t[8];
      transpose8x8(rg, t);
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) *reinterpret_cast<u32x4_t*>(dst + lds_off(cb * 8 + cc, kb)) = t[cc];
    }
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int nk = k_end > k_begin ? (k_end - k_begin + BK - 1) / BK : 0;
  if (nk > 0) {
    load_a(k_begin);
    load_b(k_begin);
    store_tile(lds, ra, AMAJ);
    store_tile(lds + TILE, rb, BMAJ);
  }
  __syncthreads();
  for (int it = 0; it < nk; ++it) {
    const int cur = it & 1;
    if (it + 1 < nk) {
      load_a(k_begin + (it + 1) * BK);
      load_b(k_begin + (it + 1) * BK);
    }
    const uint16_t* As = lds + cur * 2 * TILE;
    const uint16_t* Bs = As + TILE;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8_t a[4], b[4];
      const int kc = ks * 2 + (lane >> 5);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(As + lds_off(wm * 128 + i * 32 + (lane & 31), kc));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const bf16x8_t*>(Bs + lds_off(wn * 128 + j * 32 + (lane & 31), kc));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (it + 1 < nk) {
      uint16_t* nxt = lds + (cur ^ 1) * 2 * TILE;
      store_tile(nxt, ra, AMAJ);
      store_tile(nxt + TILE, rb, BMAJ);
    }
    __syncthreads();
  }

  // ------------------------------------------------------------ epilogue
  // acc[i][j][e] is row wm*128 + i*32 + 8*(e/4) + 4*(lane/32) + e%4, column
  // wn*128 + j*32 + lane%32 of the tile.
  const int64_t cg = RAG == RAGGED_K ? static_cast<int64_t>(grp) * p.c_gstride : 0;
  uint16_t* C = static_cast<uint16_t*>(p.C) + cg;
  float* Cf = static_cast<float*>(p.C) + cg;
  const int rbase = row_begin + wm * 128 + 4 * (lane >> 5);
  if (EPI == EPI_SWIGLU_FWD) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int col = nt * 128 + wn * 64 + q * 32 + (lane & 31);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = rbase + i * 32 + 8 * (e >> 2) + (e & 3);
          if (row < row_end) {
            const float gt = acc[i][2 * q][e], up = acc[i][2 * q + 1][e];
            Cf[static_cast<int64_t>(row) * p.ldc + col] = gt;
            Cf[static_cast<int64_t>(row) * p.ldc + p.F + col] = up;
            p.C2[static_cast<int64_t>(row) * p.ldc2 + col] = f32_to_bf16(silu_f(gt) * up);
          }
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + wn * 128 + j * 32 + (lane & 31);
        if (col >= p.N) continue;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = rbase + i * 32 + 8 * (e >> 2) + (e & 3);
          if (row >= row_end) continue;
          const float v = acc[i][j][e];
          if (EPI == EPI_SWIGLU_BWD) {
            const int64_t hr = static_cast<int64_t>(row) * p.ldh;
            const float gt = p.H[hr + col], up = p.H[hr + p.F + col];
            const float sg = sigmoid_f(gt);
            C[static_cast<int64_t>(row) * p.ldc + col] = f32_to_bf16(v * up * sg * (1.0f + gt * (1.0f - sg)));
            C[static_cast<int64_t>(row) * p.ldc + p.F + col] = f32_to_bf16(v * gt * sg);
          } else if (OUT_F32) {
            Cf[static_cast<int64_t>(row) * p.ldc + col] = v;
          } else {
            C[static_cast<int64_t>(row) * p.ldc + col] = f32_to_bf16(v);
          }
        }
      }
  }
}

template <int AMAJ, int BMAJ, int RAG, int EPI, bool OUT_F32>
void launch_kernel(const MfmaArgs& a, int64_t grid, hipStream_t s) {
  gemm_mfma_kernel<AMAJ, BMAJ, RAG, EPI, OUT_F32><<<static_cast<unsigned>(grid), NTHR, 0, s>>>(a);
}

}  // namespace

size_t mfma_schedule_bytes(int G) { return static_cast<size_t>(G + 1) * sizeof(int32_t); }

moe_status_t launch_gemm_mfma(const GemmDesc& g, int32_t* sched, hipStream_t s) {
  if (g.a_type != MOE_BF16 || g.b_type != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "mfma gemm: bf16 operands only");
  const bool out_f32 = g.c_type == MOE_F32;

  MfmaArgs a{};
  a.A = static_cast<const uint16_t*>(g.A);
  a.lda = g.lda;
  a.B = static_cast<const uint16_t*>(g.B);
  a.ldb = g.ldb;
  a.b_gstride = g.b_gstride;
  a.C = g.C;
  a.ldc = g.ldc;
  a.c_gstride = g.c_gstride;
  a.C2 = static_cast<uint16_t*>(g.C2);
  a.ldc2 = g.ldc2;
  a.H = static_cast<const float*>(g.Hin);
  a.ldh = g.ldh;
  a.offsets = g.offsets;
  a.tile_prefix = sched;
  a.G = g.G;
  a.M = g.M;
  a.N = g.N;
  a.K = g.K;
  a.F = g.F;
  a.range_end = g.range_end;
  int64_t grid;
  if (g.ragged == RAGGED_M) {
    a.nN = static_cast<int>(g.epi == EPI_SWIGLU_FWD ? ceil_div(g.N, 256) : ceil_div(g.N, BN));
    int64_t upper;
    if (g.offsets) {
      tile_prefix_kernel<<<1, 1024, 0, s>>>(g.offsets, g.G, sched);
      upper = (ceil_div(g.rows_upper, BM) + g.G) * a.nN;
    } else {
      upper = ceil_div(g.range_end, BM) * a.nN;
    }
    grid = ceil_div(upper, 8) * 8;
  } else {
    a.nM = static_cast<int>(ceil_div(g.M, BM));
    a.nN = static_cast<int>(ceil_div(g.N, BN));
    grid = static_cast<int64_t>(g.offsets ? g.G : 1) * a.nM * a.nN;
  }
  if (grid == 0) return MOE_OK;
#define MOE_MF(AM, BMJ, RG, EP, OF)                                                              \
  if (g.a_major == AM && g.b_major == BMJ && g.ragged == RG && g.epi == EP && out_f32 == OF) { \
    launch_kernel<AM, BMJ, RG, EP, OF>(a, grid, s);                                              \
    return check_launch("gemm_mfma");                                                            \
  }
  MOE_MF(K_MAJOR, K_MAJOR, RAGGED_M, EPI_SWIGLU_FWD, true)    // fc1 + SwiGLU -> H (fp32), Act (bf16)
  MOE_MF(K_MAJOR, K_MAJOR, RAGGED_M, EPI_STORE, true)         // fc2 -> Y (fp32)
  MOE_MF(K_MAJOR, MN_MAJOR, RAGGED_M, EPI_SWIGLU_BWD, false)  // fc2 data gradient + SwiGLU backward -> dH (bf16)
  MOE_MF(K_MAJOR, MN_MAJOR, RAGGED_M, EPI_STORE, true)        // fc1 data gradient -> dX (fp32)
  MOE_MF(MN_MAJOR, MN_MAJOR, RAGGED_K, EPI_STORE, true)       // weight gradients (fp32)
#undef MOE_MF
  return fail(MOE_ERR_UNSUPPORTED, "mfma gemm: unsupported operand combination");
}

}  // namespace moe
