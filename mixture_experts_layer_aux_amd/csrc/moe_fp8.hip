// fp8 (e4m3) experts: the block quantiser, the permute of e4m3 rows and their scales, and
// the grouped SwiGLU GEMM on the gfx950 fp8 matrix cores.
//
// Recipe (a reading: The Ultimate MoE Training Handbook leaves low-precision expert GEMMs
// open, §3.1 Precision asks only for an fp32 router): OCP e4m3 codes, one fp32 scale per
// block = amax / 448 in fp32 (1 for an all-zero block), code = nearest e4m3 value to the
// fp32 quotient v / scale, ties to the even code, saturated to 448.  Weights use 128 x 128
// blocks, activations 1 x 128 (per token per 128 columns).
//
// GEMM design (per workgroup: 512 threads = 8 waves):
//   * two tile shapes of the same area: 256 x 128 (waves 4 x 2) and 128 x 256 (waves
//     2 x 4), each wave 64 x 64 as 2 x 2 accumulators of v_mfma_f32_32x32x64_f8f6f4
//     (e4m3 x e4m3, fp32 out).  Launches whose experts average fewer than 512 rows take
//     128-row tiles: a 256-row tile of an expert with a few hundred rows is mostly
//     padding.  The 128 x 256 fc1 tile holds 128 Act columns of each row, one whole
//     quantisation block, so its epilogue writes the e4m3 codes and the block scale
//     itself (no fp32 Act round trip through HBM);
//   * one stage = one 128-wide K block = one scale block: both operands (128 bytes per row)
//     and the row scales of the A operand go from HBM into LDS by buffer_load ... lds,
//     through a ring of 3 stages (147 / 146 KB);
//   * per K block, each accumulator pair is formed from zero by two MFMAs and added to the
//     fp32 accumulator times (row scale x weight-block scale): the block scales of both
//     operands apply exactly once per block;
//   * operand rows are stored 128 bytes wide with the 16-byte chunk index XORed by
//     (r ^ (r >> 3)) & 7, and read with ds_read_b128 (lane l: row l % 32, bytes
//     32 (l / 32) .. +31 of each 64-wide half);
//   * the B fragment goes first, so each lane owns one output row and four consecutive
//     columns per register quad (vector epilogue stores);
//   * fc1's B tile interleaves 32 gate rows and 32 up rows, so the SwiGLU epilogue finds a
//     gate value and its up value in the same lane; it writes H (fp32, optional) and Act
//     (fp32 for the per-row quantiser, or, with 128-row tiles, e4m3 codes and scales).
#include "moe_internal.h"

namespace moe {

namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr float kE4M3Max = 448.0f;

// fp32 -> e4m3 code by the rule above.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 31) << 7;
  const float a = fabsf(x);
  uint32_t mag;
  if (!(a < kE4M3Max)) {
    mag = 0x7E;                                              // 448, and saturation
  } else if (a < 0.015625f) {                                // below 2^-6: subnormal codes
    mag = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));  // steps of 2^-9, ties to even
  } else {
    // keep 3 mantissa bits, round the 20 dropped bits to nearest even; the exponent
    // rebias (127 -> 7) is a subtraction on the combined exponent|mantissa field
    const uint32_t u = __float_as_uint(a);
    const uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);
    mag = min((r >> 20) - (120u << 3), 0x7Eu);
  }
  return sign | mag;
}

__device__ __forceinline__ float block_scale(float amax) {
  return amax > 0.0f ? __fdiv_rn(amax, kE4M3Max) : 1.0f;
}

template <typename T> __device__ __forceinline__ void load8(const T* p, float* f);
template <> __device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float* f) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
template <> __device__ __forceinline__ void load8<float>(const float* p, float* f) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

__device__ __forceinline__ uint2 encode8(const float* f, float scale) {
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) lo |= e4m3_code(__fdiv_rn(f[i], scale)) << (8 * i);
#pragma unroll
  for (int i = 0; i < 4; ++i) hi |= e4m3_code(__fdiv_rn(f[4 + i], scale)) << (8 * i);
  return make_uint2(lo, hi);
}

// Blocks of 1 x 128: 16 lanes per block, 8 values per lane; a 256-thread workgroup covers
// 16 blocks.  nblk = rows * cols / 128.
template <typename T>
__global__ __launch_bounds__(256) void quant_rows_kernel(const T* __restrict__ src, int64_t nblk,
                                                         uint8_t* __restrict__ q, float* __restrict__ scale) {
  const int64_t blk = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  const bool live = blk < nblk;
  float f[8];
  float amax = 0.0f;
  if (live) {
    load8<T>(src + blk * 128 + sub * 8, f);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  if (!live) return;
  const float s = block_scale(amax);
  *reinterpret_cast<uint2*>(q + blk * 128 + sub * 8) = encode8(f, s);
  if (sub == 0) scale[blk] = s;
}

// Blocks of 128 x 128: one 256-thread workgroup per block; thread t owns columns
// 8 (t % 16) .. +7 of rows t / 16 + 16 i.
template <typename T>
__global__ __launch_bounds__(256) void quant_tiles_kernel(const T* __restrict__ src, int cols, int nbc,
                                                          uint8_t* __restrict__ q, float* __restrict__ scale) {
  __shared__ float red[4];
  const int br = blockIdx.x / nbc, bc = blockIdx.x - br * nbc;
  const int c0 = bc * 128 + (threadIdx.x & 15) * 8;
  const int r0 = br * 128 + (threadIdx.x >> 4);
  float f[8][8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    load8<T>(src + static_cast<int64_t>(r0 + 16 * i) * cols + c0, f[i]);
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(f[i][e]));
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = block_scale(amax);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<uint2*>(q + static_cast<int64_t>(r0 + 16 * i) * cols + c0) = encode8(f[i], s);
  if (threadIdx.x == 0) scale[blockIdx.x] = s;
}

// x_perm_scale[row] = x_scale[token_of[row]], nb floats per row.
__global__ __launch_bounds__(256) void gather_scales_kernel(const float* __restrict__ xs, const int32_t* __restrict__ token_of,
                                                            int64_t A, int nb, float* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= A * nb) return;
  const int64_t r = i / nb;
  const int b = static_cast<int>(i - r * nb);
  out[i] = xs[static_cast<int64_t>(token_of[r]) * nb + b];
}

// ------------------------------------------------------------------ grouped fp8 GEMM

constexpr int BKB = 128, STAGES = 3;     // BKB: K bytes (= values) per stage
constexpr int NWAVES = 8, NTHR = 512;
constexpr int NI = 2, NJ = 2;            // 32 x 32 blocks per wave (64 x 64)
constexpr int TILE_AREA = 256 * 128;     // BM x BN of both tile shapes
// Tile shape of a launch: BM rows (256 or 128) by BN = TILE_AREA / BM columns.
template <int BM> struct Fp8Tile {
  static constexpr int BN = TILE_AREA / BM;
  static constexpr int WAVES_M = BM / 64, WAVES_N = BN / 64;
  static constexpr int A_BYTES = BM * BKB, B_BYTES = BN * BKB;   // 32 + 16 KB or 16 + 32 KB
  static constexpr int S_BYTES = BM * 4;                        // A row scales of one stage
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES + S_BYTES;
  static constexpr int A_DMA = A_BYTES / 1024 / NWAVES;          // one-KB loads per wave
  static constexpr int B_DMA = B_BYTES / 1024 / NWAVES;
  static constexpr int S_WAVES = BM / 64;                        // waves that carry the row scales
  static_assert(WAVES_M * WAVES_N == NWAVES, "8 waves of 64 x 64");
};
constexpr int kRsrcFlags = 0x00020000;
enum { FP8_SWIGLU = 0, FP8_STORE = 1 };

struct Fp8Args {
  const uint8_t* A;       // [rows, K] codes
  const float* A_scale;   // [rows, K/128]
  const uint8_t* B;       // [G, N, K] codes
  const float* B_scale;   // [G, N/128, K/128]
  float* C;               // STORE: [rows, N]; SWIGLU: Act fp32 [rows, F] (unless Cq)
  float* H;               // SWIGLU: [rows, 2F] or NULL
  uint8_t* Cq;            // SWIGLU with 128-row tiles: Act e4m3 codes [rows, F] (C unused)
  float* Cq_scale;        //   and their scales [rows, F/128]
  const int32_t* offsets;
  const int32_t* tile_prefix;   // prefix [G + 1], then the owner of each row tile [tile_cap]
  int tile_cap;
  int G, N, K, F, nN;
  Glu glu;                // SWIGLU: the gated activation
  const int32_t* gather;  // GATHER: row r of A (and of A_scale) is row gather[r] of the given ones
  int gather_rows;        // rows of the gathered A
  int gather_len;         // entries of gather
};
// Byte offset past the end of a gathered operand (bounded below 2^31 at launch).
constexpr int kOob = 0x7FFFFFF0;

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kRsrcFlags);
}

// Waits until at most n (a multiple of 1 up to 8, rounded down) of this wave's vector
// memory operations are outstanding.
__device__ __forceinline__ void wait_vm_upto8(int n) {
  // s_waitcnt simm16: vmcnt in bits 3:0 (and 15:14), expcnt 7 in 6:4, lgkmcnt 15 in 11:8
  switch (n >= 8 ? 8 : (n < 0 ? 0 : n)) {
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
  }
  asm volatile("" ::: "memory");
}
// Waits until this wave's LDS reads have returned.
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt 0; vmcnt (63) and expcnt (7) at their maxima
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// A barrier after LDS writes that other waves read next: s_barrier does not wait for this
// wave's own LDS operations to complete.
__device__ __forceinline__ void lds_barrier() {
  wait_lgkm0();
  block_barrier();
}

// The tile schedule: prefix[g] = row tiles of the experts before g (G + 1 entries), then
// owner[m] = the expert of row tile m (cap entries; a count past cap is the caller's
// broken offsets, and the writes stop there).
__global__ __launch_bounds__(1024) void fp8_tile_prefix_kernel(const int32_t* __restrict__ offsets, int G, int bm,
                                                               int cap, int32_t* __restrict__ prefix) {
  __shared__ int s[4096];
  for (int g = threadIdx.x; g < 4096; g += 1024)
    s[g] = g < G ? max(0, (offsets[g + 1] - offsets[g] + bm - 1) / bm) : 0;
  __syncthreads();
  for (int off = 1; off < 4096; off <<= 1) {
    int a[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = threadIdx.x + 1024 * u;
      a[u] = i >= off ? s[i - off] : 0;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) s[threadIdx.x + 1024 * u] += a[u];
    __syncthreads();
  }
  for (int g = threadIdx.x; g <= G; g += 1024) prefix[g] = g == 0 ? 0 : s[g - 1];
  int32_t* owner = prefix + G + 1;
  for (int g = threadIdx.x; g < G; g += 1024)
    for (int m = g ? s[g - 1] : 0; m < s[g] && m < cap; ++m) owner[m] = g;
}

constexpr int kMaxKB = 128;  // K <= 16384

// GATHER: the grouped rows of A and their scales are read from their token rows (the
// permuted copy is never made).
template <int EPI, bool GATHER, int BM>
__device__ __forceinline__ void fp8_gemm_body(const Fp8Args& p) {
  using Tl = Fp8Tile<BM>;
  constexpr int BN = Tl::BN, WAVES_N = Tl::WAVES_N, A_BYTES = Tl::A_BYTES, B_BYTES = Tl::B_BYTES;
  constexpr int STAGE_BYTES = Tl::STAGE_BYTES, A_DMA = Tl::A_DMA, B_DMA = Tl::B_DMA, S_WAVES = Tl::S_WAVES;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[STAGES * STAGE_BYTES];
  // the tile's weight-block scales per K block: every wave's fragment j lies in one
  // 128-row block of the weights, which depends on the wave's column slot wn
  __shared__ float s_bs[WAVES_N][NJ][kMaxKB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  // tile: workgroup h runs on XCD h % 8; each XCD walks a contiguous run of
  // (expert, column tile, row tile)
  const int h = blockIdx.x;
  const int total = min(p.tile_prefix[p.G], p.tile_cap) * p.nN;
  const int chunk = (total + 7) >> 3;
  const int qh = h >> 3;
  const int L = (h & 7) * chunk + qh;
  if (qh >= chunk || L >= total) return;
  // expert g owns tiles [prefix[g] nN, prefix[g+1] nN), so tile L's row-tile index L / nN
  // lies in its range: one lookup in the owner table
  const int g = min(max(p.tile_prefix[p.G + 1 + L / p.nN], 0), p.G - 1);
  const int base = p.tile_prefix[g];
  const int mtiles = p.tile_prefix[g + 1] - base;
  const int local = L - base * p.nN;
  const int nt = local / mtiles, mt = local - nt * mtiles;
  const int row_begin = p.offsets[g] + mt * BM, row_end = p.offsets[g + 1];
  const int a_rows = min(BM, row_end - row_begin);
  const int KB = p.K / 128;
  const uint8_t* Bg = p.B + static_cast<int64_t>(g) * p.N * p.K;
  const float* Bsg = p.B_scale + static_cast<int64_t>(g) * (p.N / 128) * KB;

  // B-tile row r -> weight row: fc1 interleaves 32 gate rows and 32 up rows (BN / 2 Act
  // columns per tile)
  auto brow = [&](int r) -> int {
    return EPI == FP8_SWIGLU ? (((r >> 5) & 1) ? p.F : 0) + nt * (BN / 2) + (r >> 6) * 32 + (r & 31) : nt * BN + r;
  };
  // The weight-block scales of this tile per K block (every wave's fragment j lies in one
  // 128-row block of the weights), staged in LDS once.  Their loads go out first, so that
  // their latency overlaps the offsets' set-up and the first stages' DMA; they reach LDS
  // with the wait for stage 0.
  constexpr int NBS = (WAVES_N * NJ * kMaxKB + NTHR - 1) / NTHR;   // per thread, at most
  float bsv[NBS];
#pragma unroll
  for (int u = 0; u < NBS; ++u) {
    const int t = tid + u * NTHR;
    bsv[u] = 0.0f;
    if (t < WAVES_N * NJ * KB) {
      const int wj = t / KB, kb = t - wj * KB;
      const int w = wj / NJ, j = wj - w * NJ;
      bsv[u] = Bsg[(brow(w * 64 + j * 32) / 128) * KB + kb];
    }
  }
  // per-lane DMA offsets (bytes from the stage's base)
  int voffA[A_DMA], voffB[B_DMA];
#pragma unroll
  for (int q = 0; q < A_DMA; ++q) {
    const int r = (wave * A_DMA + q) * 8 + (lane >> 3);
    if constexpr (GATHER) {
      const int src = r < a_rows && row_begin + r < p.gather_len ? p.gather[row_begin + r] : -1;
      voffA[q] = src >= 0 ? src * p.K + (((lane & 7) ^ swz(r)) << 4) : kOob;
    } else {
      voffA[q] = r * p.K + (((lane & 7) ^ swz(r)) << 4);
    }
  }
#pragma unroll
  for (int q = 0; q < B_DMA; ++q) {
    const int r = (wave * B_DMA + q) * 8 + (lane >> 3);
    voffB[q] = brow(r) * p.K + (((lane & 7) ^ swz(r)) << 4);
  }
  int voffS = (wave * 64 + lane) * KB * 4;  // waves 0 .. S_WAVES-1 carry the BM row scales
  if constexpr (GATHER) {
    const int r = wave * 64 + lane;
    const int src = (wave < S_WAVES && r < a_rows && row_begin + r < p.gather_len) ? p.gather[row_begin + r] : -1;
    voffS = src >= 0 ? src * KB * 4 : kOob;
  }
  const int ndma = A_DMA + B_DMA + (wave < S_WAVES ? 1 : 0);

  auto issue = [&](int st) {
    uint8_t* dst = lds + (st % STAGES) * STAGE_BYTES;
    const int k0 = st * BKB;
    const __amdgpu_buffer_rsrc_t ra =
        GATHER ? make_rsrc(p.A + k0, p.gather_rows * p.K - k0)
               : make_rsrc(p.A + static_cast<int64_t>(row_begin) * p.K + k0, (a_rows - 1) * p.K + BKB);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bg + k0, (p.N - 1) * p.K + BKB);
#pragma unroll
    for (int q = 0; q < A_DMA; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)(dst + (wave * A_DMA + q) * 1024), 16, voffA[q], 0, 0, 0);
#pragma unroll
    for (int q = 0; q < B_DMA; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_t*)(dst + A_BYTES + (wave * B_DMA + q) * 1024), 16,
                                               voffB[q], 0, 0, 0);
    if (wave < S_WAVES) {
      const __amdgpu_buffer_rsrc_t rs =
          GATHER ? make_rsrc(p.A_scale + st, (p.gather_rows * KB - st) * 4)
                 : make_rsrc(p.A_scale + static_cast<int64_t>(row_begin) * KB + st, ((a_rows - 1) * KB + 1) * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(dst + A_BYTES + B_BYTES + wave * 256), 4, voffS, 0, 0,
                                               0);
    }
  };
  // fragment of a 32-row block at r0, 64-wide half hh: row r0 + lane % 32, bytes
  // 64 hh + 32 (lane / 32) .. +31
  auto frag = [&](const uint8_t* t, int r0, int hh) -> i32x8_t {
    const int r = r0 + (lane & 31);
    const int c = hh * 4 + 2 * (lane >> 5);
    const uint4 v0 = *reinterpret_cast<const uint4*>(t + r * BKB + ((c ^ swz(r)) << 4));
    const uint4 v1 = *reinterpret_cast<const uint4*>(t + r * BKB + (((c + 1) ^ swz(r)) << 4));
    const i32x8_t v = {static_cast<int>(v0.x), static_cast<int>(v0.y), static_cast<int>(v0.z), static_cast<int>(v0.w),
                       static_cast<int>(v1.x), static_cast<int>(v1.y), static_cast<int>(v1.z), static_cast<int>(v1.w)};
    return v;
  };

  f32x16_t acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Main loop, two wave groups in alternation (waves 0-3 and 4-7; wave w and w+4 share a
  // SIMD): every stage is a memory phase (read the stage's fragments and scales into
  // registers, issue this wave's DMA part of stage it+D, wait for its part of stage it+1)
  // and a compute phase (matrix and scale instructions from registers only), each ended
  // by a workgroup barrier.  The second group runs one phase behind the first, so on every
  // SIMD one wave computes while the other reads and issues.  Slot reuse: stage it+D
  // overwrites the slot of stage it-1, which both groups finished reading one barrier
  // earlier.
  constexpr int D = STAGES - 1;
  const bool late = wave >= 4;
  const int nk = KB;
#pragma unroll
  for (int st = 0; st < D; ++st)
    if (st < nk) issue(st);
#pragma unroll
  for (int u = 0; u < NBS; ++u) {
    const int t = tid + u * NTHR;
    if (t < WAVES_N * NJ * KB) {
      const int wj = t / KB, kb = t - wj * KB;
      s_bs[wj / NJ][wj % NJ][kb] = bsv[u];
    }
  }
  wait_vm_upto8(max(0, min(D, nk) - 1) * ndma);   // own part of stage 0 landed
  wait_lgkm0();                                   // the scales written
  block_barrier();
  if (late) block_barrier();
  for (int it = 0; it < nk; ++it) {
    const uint8_t* As = lds + (it % STAGES) * STAGE_BYTES;
    const uint8_t* Bs = As + A_BYTES;
    const float* Ss = reinterpret_cast<const float*>(As + A_BYTES + B_BYTES);
    i32x8_t fa[NI][2], fb[NJ][2];
    float sa[NI], sb[NJ];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      fa[i][0] = frag(As, wm * 64 + i * 32, 0);
      fa[i][1] = frag(As, wm * 64 + i * 32, 1);
      sa[i] = Ss[wm * 64 + i * 32 + (lane & 31)];
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      fb[j][0] = frag(Bs, wn * 64 + j * 32, 0);
      fb[j][1] = frag(Bs, wn * 64 + j * 32, 1);
      sb[j] = s_bs[wn][j][it];
    }
    // the stage's reads go out before the next DMA is issued: the compiler would
    // otherwise wait for that DMA before any LDS read that follows it
    __builtin_amdgcn_sched_barrier(0);
    if (it + D < nk) issue(it + D);
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkm0();  // fragments and scales in registers before the slot may be refilled
    wait_vm_upto8(max(0, min(it + D, nk - 1) - (it + 1)) * ndma);  // own part of stage it+1 landed
    __builtin_amdgcn_sched_barrier(0);
    block_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        f32x16_t t = {};
        t = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j][0], fa[i][0], t, 0, 0, 0, 0, 0, 0);
        t = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j][1], fa[i][1], t, 0, 0, 0, 0, 0, 0);
        const float f = sa[i] * sb[j];
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = fmaf(t[e], f, acc[i][j][e]);
      }
    __builtin_amdgcn_sched_barrier(0);
    block_barrier();
    __builtin_amdgcn_sched_barrier(0);
  }
  if (!late) block_barrier();

  // epilogue: acc[i][j][4q + c] is row wm*64 + i*32 + lane%32, column
  // wn*64 + j*32 + 8q + 4(lane/32) + c of the B tile.  The BM x BN fp32 tile goes through
  // LDS (row-major, 16-byte chunk c of row r at r * (BN / 4) + (c ^ (r & 31))), so that the
  // global writes run along whole rows instead of 16-byte pieces of 32 rows.  The fp32
  // outputs go out as non-temporal stores (written once, larger than the L2s).
  constexpr int RC = BN / 4;   // 16-byte chunks per tile row
  float4* L4 = reinterpret_cast<float4*>(lds);
  static_assert(STAGES * STAGE_BYTES >= BM * BN * 4, "epilogue staging needs the tile in LDS");
  block_barrier();  // every wave is done with the last stage (and its DMA, waited above)
  const int cb = 4 * (lane >> 5);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int r = wm * 64 + i * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = (wn * 64 + j * 32 + 8 * q + cb) >> 2;
        L4[r * RC + (c ^ (r & 31))] =
            make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
      }
  }
  lds_barrier();
  constexpr int RPW = BM / NWAVES;   // tile rows per wave in the write-out
  if (EPI == FP8_SWIGLU) {
    // B-tile column blocks of 32 alternate gate and up.  LPR = BN / 8 lanes per row, lane
    // l the output columns 4l .. 4l+3 of the tile's BN / 2 (from nt * BN / 2), 64 / LPR
    // rows per step
    constexpr int LPR = BN / 8, RPS = 64 / LPR;
    const int l = lane % LPR;
    const int cgate = (l >> 3) * 16 + (l & 7), col = nt * (BN / 2) + 4 * l;
#pragma unroll 2
    for (int rr = 0; rr < RPW / RPS; ++rr) {
      const int r = wave * RPW + rr * RPS + lane / LPR;
      const int row = row_begin + r;
      const bool live = row < row_end;
      const float4 gt = L4[r * RC + (cgate ^ (r & 31))], up = L4[r * RC + ((cgate + 8) ^ (r & 31))];
      float4 act;
      act.x = glu_f(p.glu, gt.x, up.x); act.y = glu_f(p.glu, gt.y, up.y);
      act.z = glu_f(p.glu, gt.z, up.z); act.w = glu_f(p.glu, gt.w, up.w);
      if (live && p.H) {
        float* hrow = p.H + static_cast<int64_t>(row) * 2 * p.F;
        store_nt(reinterpret_cast<float4*>(hrow + col), gt);
        store_nt(reinterpret_cast<float4*>(hrow + p.F + col), up);
      }
      if constexpr (BN / 2 == 128) {
        if (p.Cq) {
          // the row's 128 Act columns of this tile are one quantisation block, held by
          // the 32 lanes of this half-wave: the block amax, its scale and the codes by
          // the rule of the standalone quantiser (quant_rows_kernel)
          float amax = fmaxf(fmaxf(fabsf(act.x), fabsf(act.y)), fmaxf(fabsf(act.z), fabsf(act.w)));
#pragma unroll
          for (int m = 1; m < 32; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
          const float sc = block_scale(amax);
          if (live) {
            const uint32_t code = e4m3_code(__fdiv_rn(act.x, sc)) | (e4m3_code(__fdiv_rn(act.y, sc)) << 8) |
                                  (e4m3_code(__fdiv_rn(act.z, sc)) << 16) | (e4m3_code(__fdiv_rn(act.w, sc)) << 24);
            *reinterpret_cast<uint32_t*>(p.Cq + static_cast<int64_t>(row) * p.F + col) = code;
            if (l == 0) p.Cq_scale[static_cast<int64_t>(row) * (p.F / 128) + nt] = sc;
          }
          continue;
        }
      }
      if (live) store_nt(reinterpret_cast<float4*>(p.C + static_cast<int64_t>(row) * p.F + col), act);
    }
  } else {
    // 64 / RC rows per step, RC lanes per row, lane l the columns 4l .. 4l+3 of nt*BN ..
    constexpr int RPS = 64 / RC;
    const int l = lane % RC, col = nt * BN + 4 * l;
#pragma unroll 4
    for (int rr = 0; rr < RPW / RPS; ++rr) {
      const int r = wave * RPW + rr * RPS + lane / RC;
      const int row = row_begin + r;
      if (row >= row_end) continue;
      store_nt(reinterpret_cast<float4*>(p.C + static_cast<int64_t>(row) * p.N + col), L4[r * RC + (l ^ (r & 31))]);
    }
  }
}


// One plain kernel per launched variant around the device-function body (the host pass
// emitted no launch stubs for the body as a kernel template).
#define MOE_FP8_KERNEL(NAME, EP, GT, BMV) \
  __global__ __launch_bounds__(NTHR, 1) void NAME(const Fp8Args p) { fp8_gemm_body<EP, GT, BMV>(p); }
MOE_FP8_KERNEL(fp8_gemm_swiglu_gather_256, FP8_SWIGLU, true, 256)
MOE_FP8_KERNEL(fp8_gemm_swiglu_256, FP8_SWIGLU, false, 256)
MOE_FP8_KERNEL(fp8_gemm_store_256, FP8_STORE, false, 256)
MOE_FP8_KERNEL(fp8_gemm_swiglu_gather_128, FP8_SWIGLU, true, 128)
MOE_FP8_KERNEL(fp8_gemm_swiglu_128, FP8_SWIGLU, false, 128)
MOE_FP8_KERNEL(fp8_gemm_store_128, FP8_STORE, false, 128)
#undef MOE_FP8_KERNEL

}  // namespace

moe_status_t launch_quantize_fp8(int src_dtype, const void* src, int64_t rows, int cols, int block_rows, uint8_t* q,
                                 float* scale, hipStream_t s) {
  if (block_rows == 1) {
    const int64_t nblk = rows * (cols / 128);
    const int64_t grid = ceil_div(nblk, 16);
    if (src_dtype == MOE_BF16)
      quant_rows_kernel<uint16_t><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(src), nblk, q, scale);
    else
      quant_rows_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float*>(src), nblk, q, scale);
  } else {
    const int nbc = cols / 128;
    const int64_t grid = (rows / 128) * nbc;
    if (src_dtype == MOE_BF16)
      quant_tiles_kernel<uint16_t><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(src), cols, nbc, q, scale);
    else
      quant_tiles_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float*>(src), cols, nbc, q, scale);
  }
  return check_launch("quantize_fp8");
}

moe_status_t launch_gather_scales(const float* xs, const int32_t* token_of, int64_t A, int nb, float* out,
                                  hipStream_t s) {
  if (A == 0) return MOE_OK;
  gather_scales_kernel<<<ceil_div(A * nb, 256), 256, 0, s>>>(xs, token_of, A, nb, out);
  return check_launch("gather_scales");
}

namespace {
int64_t fp8_tile_cap(int E, int64_t rows) { return ceil_div(rows, int64_t{128}) + E; }
}
size_t fp8_schedule_bytes(int E, int64_t rows) { return static_cast<size_t>(E + 1 + fp8_tile_cap(E, rows)) * 4; }

// fc1 (+ SwiGLU -> H, Act fp32) when act32 != NULL and C is NULL, else fc2 -> C.
int fp8_tile_rows(int64_t rows_upper, int G, int N, int F, bool swiglu) {
  // 128-row tiles when the experts average fewer than 512 rows and the 256-wide column
  // tile divides the output (fc1: F / 128 Act columns blocks; fc2: N)
  const bool narrow_ok = swiglu ? F % 128 == 0 : N % 256 == 0;
  return rows_upper < int64_t{512} * G && narrow_ok ? 128 : 256;
}

moe_status_t launch_gemm_fp8(bool swiglu, const uint8_t* A, const float* A_scale, const uint8_t* B,
                             const float* B_scale, float* C, float* H, const int32_t* offsets, int G, int64_t rows_upper,
                             int N, int K, int F, int32_t* sched, hipStream_t s, Glu glu, const int32_t* gather,
                             int gather_rows, int bm, uint8_t* act_q, float* act_scale) {
  if (G > 4096) return fail(MOE_ERR_UNSUPPORTED, "fp8 gemm: more than 4096 experts");
  if (K > 128 * kMaxKB || K % 128 || N % 128) return fail(MOE_ERR_UNSUPPORTED, "fp8 gemm: K must be a multiple of 128 up to 16384");
  if (static_cast<int64_t>(N) * K >= (int64_t{1} << 31) || rows_upper * K >= (int64_t{1} << 31))
    return fail(MOE_ERR_UNSUPPORTED, "fp8 gemm: operand above 2 GB");
  if (bm != 128 && bm != 256) return fail(MOE_ERR_INVALID_ARG, "fp8 gemm: tile rows must be 128 or 256");
  const int bn = TILE_AREA / bm;
  if (swiglu ? F % (bn / 2) : N % bn) return fail(MOE_ERR_UNSUPPORTED, "fp8 gemm: output not a multiple of the tile");
  if (act_q && !(swiglu && bm == 128)) return fail(MOE_ERR_INVALID_ARG, "fp8 gemm: fused Act codes need fc1 with 128-row tiles");
  Fp8Args a{};
  a.A = A; a.A_scale = A_scale; a.B = B; a.B_scale = B_scale; a.C = C; a.H = H;
  a.Cq = act_q; a.Cq_scale = act_scale;
  a.offsets = offsets; a.tile_prefix = sched; a.G = G; a.N = N; a.K = K; a.F = F; a.glu = glu;
  a.nN = swiglu ? F / (bn / 2) : N / bn;
  if (gather) {
    if (!swiglu) return fail(MOE_ERR_UNSUPPORTED, "fp8 gemm: the row gather is for fc1");
    if (static_cast<int64_t>(gather_rows) * K > kOob - 4096)
      return fail(MOE_ERR_UNSUPPORTED, "fp8 gemm: gathered operand above 2 GB");
    a.gather = gather;
    a.gather_rows = gather_rows;
    a.gather_len = static_cast<int>(rows_upper);
  }
  a.tile_cap = static_cast<int>(ceil_div(rows_upper, int64_t{bm}) + G);
  fp8_tile_prefix_kernel<<<1, 1024, 0, s>>>(offsets, G, bm, a.tile_cap, sched);
  const int64_t upper = (ceil_div(rows_upper, bm) + G) * a.nN;
  const int64_t grid = ceil_div(upper, 8) * 8;
  if (grid == 0) return MOE_OK;
#define MOE_FP8(NAME, SW, GT, BMV)                                   \
  if (SW == swiglu && GT == (gather != nullptr) && bm == BMV) {       \
    NAME<<<static_cast<unsigned>(grid), NTHR, 0, s>>>(a);            \
    return check_launch("gemm_fp8");                                  \
  }
  MOE_FP8(fp8_gemm_swiglu_gather_256, true, true, 256)
  MOE_FP8(fp8_gemm_swiglu_256, true, false, 256)
  MOE_FP8(fp8_gemm_store_256, false, false, 256)
  MOE_FP8(fp8_gemm_swiglu_gather_128, true, true, 128)
  MOE_FP8(fp8_gemm_swiglu_128, true, false, 128)
  MOE_FP8(fp8_gemm_store_128, false, false, 128)
#undef MOE_FP8
  return fail(MOE_ERR_UNSUPPORTED, "fp8 gemm: unsupported variant");
}

}  // namespace moe
