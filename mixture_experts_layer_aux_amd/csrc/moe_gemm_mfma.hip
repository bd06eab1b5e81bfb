// bf16 grouped GEMM on gfx950 matrix cores, fp32 accumulation.
//
// The expert FFNs of The Ultimate MoE Training Handbook, §3.4 (fc1 of width 2F split
// into gate and up halves, SwiGLU, fc2 back to d), run as one grouped GEMM per
// projection: each expert owns a ragged block of rows (forward, data gradient) or a
// ragged block of the reduction dimension (weight gradient).
//
// Design (per workgroup: 512 threads = 8 waves in a 2 x 4 grid):
//   * 256 x 256 output tile, each wave a 128 x 64 sub-tile held as 4 x 2 accumulators of
//     v_mfma_f32_32x32x16_bf16 (128 fp32 per lane);
//   * operands go from HBM straight into LDS (buffer_load ... lds, 16 bytes per lane), 32
//     K values per stage, through a ring of 4 stages (128 KB): three stages are in flight
//     while one is read, and no VGPRs stage the data;
//   * ping-pong: waves 0-3 and 4-7 (wave w and w+4 share a SIMD) alternate a memory phase
//     (the stage's fragments into registers, this wave's DMA part of a later stage, waits)
//     and a compute phase (MFMAs only), one workgroup barrier apart and one phase out of
//     step, so the matrix core of every SIMD is fed while the other wave is stalled on LDS
//     or on issuing DMA;
//   * buffer descriptors bound every load: rows past the end of a ragged reduction (weight
//     gradient) and past the end of an operand read as zeros, so no tail handling exists
//     in the loop;
//   * operands contiguous in K are stored [rows][32 k] with the 16-byte chunk index XORed
//     by (r >> 2) & 3, and read with ds_read_b128; operands contiguous in rows (the
//     weights of the data gradients, both operands of the weight gradients) are stored
//     as loaded, [32 k][256 rows] with the chunk index XORed by 4 * (k & 3), and
//     read with the gfx950 transposing ds_read_b64_tr_b16 (a 16-lane group reads 4 k-rows
//     of 16 columns and gets back, per lane, one column's 4 k values), so no operand is
//     ever transposed through registers;
//   * the MFMA takes the B fragment first, so the accumulator comes out transposed and
//     each lane owns four consecutive output columns of one row;
//   * the epilogue stages the tile through LDS in two passes of 128 rows and then works on
//     whole tile rows, so its global loads and stores are contiguous runs of a row (a 1 KB
//     row of fp32 per store instruction) rather than 16 bytes of each of 32 rows; a bf16
//     weight gradient that overwrites is rounded first and staged in one pass.  The
//     outputs go out as non-temporal stores, so they do not evict operand lines from L2;
//   * a one-group weight gradient can be split over its reduction rows (kchunk): each
//     chunk is a group writing fp32 partials, summed in chunk order by splitk_reduce_kernel;
//   * in an expert's last row tile, the 32-row accumulator blocks past its end skip their
//     fragment reads and MFMAs (a wave-uniform branch around a second copy of the loop);
//   * a device-built tile list (per-expert prefix of row tiles) so the host never reads
//     the expert counts; empty experts get no tiles (forward) or exact-zero gradients
//     (weight gradient, zero-length reduction);
//   * workgroups are dealt round-robin to the 8 XCDs, so workgroup h runs on XCD h mod 8.
//     Row-ragged launches map h to tile (h mod 8) * ceil(tiles / 8) + h / 8, so each XCD
//     walks a contiguous run of tiles (expert, column tile, row tile) and tiles sharing a
//     weight or activation tile run together on one L2; reduction-ragged launches give
//     each XCD one eighth of every expert's tiles, walked in bands of 4 row tiles;
//   * fused epilogues: SwiGLU (forward: H in fp32 and Act in bf16 from the same
//     accumulators, the gate and up rows of W13 interleaved per 32-row block of the B
//     tile) and the SwiGLU backward (reads the saved fp32 H, writes dH in bf16).
#include <algorithm>
#include <type_traits>

#include "moe_internal.h"

namespace moe {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int BM = 256, BN = 256, BK = 32, STAGES = 4;
// Main-loop schedule: wave groups alternating memory and compute phases (see the loop).
constexpr bool PING_PONG = true;
// Waves of a workgroup: WAVES_M x WAVES_N, each owning a (BM / WAVES_M) x (BN / WAVES_N)
// sub-tile as (BM / WAVES_M / 32) x (BN / WAVES_N / 32) accumulators of 32 x 32.
constexpr int WAVES_M = 2, WAVES_N = 4, NWAVES = WAVES_M * WAVES_N, NTHR = 64 * NWAVES;
constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N, NI = WTM / 32, NJ = WTN / 32;
constexpr int KCH = BK / 8;                         // 16-byte chunks per K-contiguous row
constexpr int DMA_PER_WAVE = (BK / 2) / NWAVES;     // one-KB blocks per operand per stage per wave
constexpr int NDMA = 2 * DMA_PER_WAVE;               // LDS-DMA instructions per wave per stage
constexpr int TILE = 256 * BK;          // bf16 elements of one operand tile of one stage
constexpr int STAGE_ELEMS = 2 * TILE;   // A then B
constexpr int BLOCK_ELEMS = 512;        // one wave-wide 16-byte-per-lane LDS DMA = 1 KB
// 4th descriptor dword of a raw (untyped, 32-bit element) buffer on gfx9.
constexpr int kRsrcFlags = 0x00020000;

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
  const int32_t* tile_prefix;   // prefix [G + 1], then the owner of each row tile [tile_cap]
  int tile_cap;
  int G, M, N, K, F, range_end, nN, nM;
  int b_rows_bytes;  // K-major B: bytes of one group's weight matrix (bounds the DMA)
  Glu glu;           // SwiGLU epilogues: the gated activation
  int beta;          // EPI_STORE: 1 = add into C
  int kchunk;        // RAGGED_K without offsets: reduction rows per group (0: one group)
  const int32_t* gather;  // GA: source row of each grouped row (see the kernel)
  int gather_rows;        // rows of the gathered operand
  int gather_len;         // entries of gather (bounds the index loads)
  const int32_t* skip;    // reduction-ragged: groups left to the skew split path, or NULL
};

// K-contiguous layout: element (r, k) of a stage tile at r * BK + ((k/8) ^ swk(r)) * 8 + k%8
// (XORs that measured conflict-free for 32 consecutive rows read at one 16-byte chunk).
__device__ __forceinline__ int swk(int r) { return KCH == 8 ? ((r ^ (r >> 3)) & 7) : ((r >> 2) & 3); }
// Row-contiguous layout: element (k, c) at k * 256 + ((c/8) ^ swm(k)) * 8 + c%8; the 4 k-rows
// a 16-lane transposing read touches land 4 chunks apart, so two such groups (32 lanes)
// cover 16 distinct chunks.
__device__ __forceinline__ int swm(int k) { return (k & 3) << 2; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kRsrcFlags);
}

// Waits until at most n of this wave's buffer loads are outstanding (n rounded down to a
// multiple of 4, at most 24).
__device__ __forceinline__ void wait_vm(int n) {
  // s_waitcnt simm16: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14, expcnt (7) in
  // bits 6:4 and lgkmcnt (15) in bits 11:8 left at their maxima
  if (n >= 24) __builtin_amdgcn_s_waitcnt(0x4F78);
  else if (n >= 16) __builtin_amdgcn_s_waitcnt(0x4F70);
  else if (n >= 12) __builtin_amdgcn_s_waitcnt(0x0F7C);
  else if (n >= 8) __builtin_amdgcn_s_waitcnt(0x0F78);
  else if (n >= 4) __builtin_amdgcn_s_waitcnt(0x0F74);
  else __builtin_amdgcn_s_waitcnt(0x0F70);
  asm volatile("" ::: "memory");
}
// Transposing LDS read of 4 bf16 (ds_read_b64_tr_b16).  The restrict parameter gives the
// read alias-scope information; without it the compiler cannot tell the read apart from
// the LDS-DMA writes still in flight and waits for all of them (vmcnt 0) before every
// such read, which drains the DMA pipeline once per stage.  The kernels order their LDS
// reads after the DMA explicitly (each wave waits for its own loads, then a barrier).
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
__device__ __attribute__((always_inline)) inline i16x4_t lds_read_tr(lds_i16x4_t* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
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

// Tiles of a row-ragged launch: group g has ceil(rows_g / 256) row tiles.
// prefix [G + 1] of the row tiles, then owner[m] = the group of row tile m (cap entries;
// a count past cap is the caller's broken offsets, and the writes stop there).  G <= 2048:
// thread i holds groups 2i and 2i + 1; a wave-level scan, then the 16 wave totals; each
// owner entry is found by a binary search of the inclusive prefix.
__global__ __launch_bounds__(1024) void tile_prefix_kernel(const int32_t* __restrict__ offsets, int G, int cap,
                                                           int32_t* __restrict__ prefix) {
  __shared__ int s[2048];   // inclusive prefix of the row tiles
  __shared__ int wtot[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g0 = 2 * tid, g1 = g0 + 1;
  const int c0 = g0 < G ? max(0, (offsets[g0 + 1] - offsets[g0] + BM - 1) / BM) : 0;
  const int c1 = g1 < G ? max(0, (offsets[g1 + 1] - offsets[g1] + BM - 1) / BM) : 0;
  int v = c0 + c1;
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  if (lane == 63) wtot[w] = v;
  __syncthreads();
  for (int i = 0; i < w; ++i) v += wtot[i];
  s[g1] = v;
  s[g0] = v - c1;
  __syncthreads();
  for (int g = tid; g <= G; g += 1024) prefix[g] = g == 0 ? 0 : s[g - 1];
  int32_t* owner = prefix + G + 1;
  const int lim = G > 0 ? min(s[G - 1], cap) : 0;
  for (int m = tid; m < lim; m += 1024) {
    int lo = 0, hi = G - 1;   // the first group whose inclusive prefix exceeds m
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s[mid] > m) hi = mid;
      else lo = mid + 1;
    }
    owner[m] = lo;
  }
}

// Byte offset past the end of every gathered operand (bounded below 2^31 at launch): a
// DMA lane given it reads zeros.
constexpr int kOob = 0x7FFFFFF0;

// GA: 0 = operands as given; 1 = K-contiguous A of a row-ragged launch read through a row
// gather (grouped row r of the tile from row gather[r] of A: the fc1 forward on the token
// rows).  The fc1 weight gradient over the token rows runs on moe_wgrad.hip.
template <int AMAJ, int BMAJ, int RAG, int EPI, bool OUT_F32, int GA>
__global__ __launch_bounds__(NTHR, 1) void gemm_mfma_kernel(const MfmaArgs p) {
  static_assert(GA == 0 || (GA == 1 && AMAJ == K_MAJOR && RAG == RAGGED_M), "unsupported gather");
  __shared__ __attribute__((aligned(1024))) uint16_t lds[STAGES * STAGE_ELEMS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  // ------------------------------------------------------------ tile of this workgroup
  int grp, mt, nt;
  int row_begin, row_end;  // RAGGED_M: rows of A/C;  RAGGED_K: rows [0, M) of C
  int k_begin, k_end;
  if (RAG == RAGGED_M) {
    const int h = blockIdx.x;
    const int total_m = p.offsets ? min(p.tile_prefix[p.G], p.tile_cap) : (p.range_end + BM - 1) / BM;
    const int total = total_m * p.nN;
    const int chunk = (total + 7) >> 3;
    const int q = h >> 3;
    const int L = (h & 7) * chunk + q;
    if (q >= chunk || L >= total) return;
    // group g owns tiles [prefix[g] nN, prefix[g+1] nN), so the row-tile index L / nN of
    // tile L lies in its range: one lookup in the owner table
    const int g = p.offsets ? min(max(p.tile_prefix[p.G + 1 + L / p.nN], 0), p.G - 1) : 0;
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
    // Reduction-ragged (weight gradient): a tile's work grows with its expert's rows, so
    // every expert's tiles are split into 8 equal runs, one per XCD.  The runs follow a
    // blocked order: bands of WG_BAND row tiles, walked column by column with the row tile
    // fastest, so the ~32 tiles one XCD holds at a time span WG_BAND slices of A and about
    // 8 of B (instead of 1-2 of A and every slice of B), and L2 serves the rest.
    constexpr int WG_BAND = 4;
    const int per = p.nM * p.nN;
    const int run = (per + 7) >> 3;
    const int h = blockIdx.x;
    const int q = h >> 3;
    grp = q / run;
    const int local = (h & 7) * run + (q - grp * run);
    if (grp >= p.G || local >= per) return;
    if (p.skip && p.skip[grp]) return;
    const int band = local / (WG_BAND * p.nN);
    const int rem = local - band * WG_BAND * p.nN;
    const int bh = min(WG_BAND, p.nM - band * WG_BAND);
    nt = rem / bh;
    mt = band * WG_BAND + (rem - nt * bh);
    row_begin = mt * BM;
    row_end = p.M;
    if (p.offsets) {
      k_begin = p.offsets[grp];
      k_end = p.offsets[grp + 1];
    } else {   // split-K chunks of one group (kchunk 0: the whole range)
      k_begin = grp * p.kchunk;
      k_end = p.kchunk ? min(p.range_end, k_begin + p.kchunk) : p.range_end;
    }
  }
  const int n0 = nt * BN;
  const uint16_t* Bg = p.B + (RAG == RAGGED_M ? static_cast<int64_t>(grp) * p.b_gstride : 0);
  const int a_rows = min(BM, row_end - row_begin);  // K-major A rows that exist (RAGGED_M)

  // ------------------------------------------------------------ HBM -> LDS (DMA)
  // Each wave moves 4 one-KB blocks of A and 4 of B per stage.  voff*: per-lane byte
  // offsets of those blocks relative to the stage's base (constant over the K loop).
  int voffA[DMA_PER_WAVE], voffB[DMA_PER_WAVE];
#pragma unroll
  for (int q = 0; q < DMA_PER_WAVE; ++q) {
    const int blk = wave * DMA_PER_WAVE + q;
    if (AMAJ == K_MAJOR) {
      const int r = blk * (64 / KCH) + lane / KCH;
      const int c = (lane % KCH) ^ swk(r);
      if constexpr (GA == 1) {
        const int src = r < a_rows && row_begin + r < p.gather_len ? p.gather[row_begin + r] : -1;
        voffA[q] = src >= 0 ? src * static_cast<int>(p.lda) * 2 + c * 16 : kOob;
      } else {
        voffA[q] = r * static_cast<int>(p.lda) * 2 + c * 16;
      }
    } else {
      const int kr = blk * 2 + (lane >> 5);
      const int c = (lane & 31) ^ swm(kr);
      voffA[q] = kr * static_cast<int>(p.lda) * 2 + (row_begin + c * 8) * 2;
    }
    if (BMAJ == K_MAJOR) {
      const int r = blk * (64 / KCH) + lane / KCH;
      const int c = (lane % KCH) ^ swk(r);
      int n;
      if (EPI == EPI_SWIGLU_FWD)  // B-tile block j of 32 rows: gate rows if j is even, up rows if odd
        n = (((r >> 5) & 1) ? p.F : 0) + nt * 128 + (r >> 6) * 32 + (r & 31);
      else
        n = n0 + r;
      voffB[q] = n * static_cast<int>(p.ldb) * 2 + c * 16;
    } else {
      const int kr = blk * 2 + (lane >> 5);
      const int c = (lane & 31) ^ swm(kr);
      voffB[q] = kr * static_cast<int>(p.ldb) * 2 + (n0 + c * 8) * 2;
    }
  }
  auto stage_rsrc = [&](int st, __amdgpu_buffer_rsrc_t& ra, __amdgpu_buffer_rsrc_t& rb) {
    const int k0 = k_begin + st * BK;
    if (GA == 1)
      ra = make_rsrc(p.A + k0, p.gather_rows * static_cast<int>(p.lda) * 2 - k0 * 2);
    else if (AMAJ == K_MAJOR)
      ra = make_rsrc(p.A + static_cast<int64_t>(row_begin) * p.lda + k0,
                     (a_rows - 1) * static_cast<int>(p.lda) * 2 + BK * 2);
    else
      ra = make_rsrc(p.A + static_cast<int64_t>(k0) * p.lda, min(BK, k_end - k0) * static_cast<int>(p.lda) * 2);
    if (BMAJ == K_MAJOR)
      rb = make_rsrc(Bg + k0, p.b_rows_bytes - k0 * 2);
    else
      rb = make_rsrc(Bg + static_cast<int64_t>(k0) * p.ldb, min(BK, k_end - k0) * static_cast<int>(p.ldb) * 2);
  };
  // Stage st, DMA instruction q of this wave: q < DMA_PER_WAVE moves a block of A, the
  // rest blocks of B.
  auto issue_one = [&](int st, int q, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb) {
    uint16_t* dst = lds + (st % STAGES) * STAGE_ELEMS;
    if (q < DMA_PER_WAVE)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)(dst + (wave * DMA_PER_WAVE + q) * BLOCK_ELEMS), 16,
                                               voffA[q], 0, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb, (lds_void_t*)(dst + TILE + (wave * DMA_PER_WAVE + q - DMA_PER_WAVE) * BLOCK_ELEMS), 16,
          voffB[q - DMA_PER_WAVE], 0, 0, 0);
  };
  auto issue_stage = [&](int st) {
    __amdgpu_buffer_rsrc_t ra, rb;
    stage_rsrc(st, ra, rb);
#pragma unroll
    for (int q = 0; q < NDMA; ++q) issue_one(st, q, ra, rb);
  };

  // ------------------------------------------------------------ LDS -> fragments
  // Fragment of a 32-row block at row offset rb0 for substep ks (16 k): lane l gets rows
  // rb0 + l%32, k = 16 ks + 8 (l/32) + 0..7.
  auto frag = [&](const uint16_t* t, int major, int rb0, int ks) -> bf16x8_t {
    if (major == K_MAJOR) {
      const int r = rb0 + (lane & 31);
      const int c = (ks * 2 + (lane >> 5)) ^ swk(r);
      return *reinterpret_cast<const bf16x8_t*>(t + r * BK + c * 8);
    } else {
      const int j = lane & 15, g = lane >> 4;
      const int col = rb0 + 16 * (g & 1) + 4 * (j & 3);
      i16x4_t h[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int kr = ks * 16 + 8 * (g >> 1) + 4 * hh + (j >> 2);
        const uint16_t* a = t + kr * 256 + (((col >> 3) ^ swm(kr)) << 3) + (col & 7);
        h[hh] = lds_read_tr((lds_i16x4_t*)a);
      }
      const i16x4_t lo = h[0], hi = h[1];
      typedef short i16x8_t __attribute__((ext_vector_type(8)));
      const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      return __builtin_bit_cast(bf16x8_t, v);
    }
  };

  f32x16_t acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int nk = k_end > k_begin ? (k_end - k_begin + BK - 1) / BK : 0;
  if (RAG == RAGGED_K && EPI == EPI_STORE && nk == 0) {
    // A group without rows: its gradient tile is exact zeros, written straight out with
    // 16-byte stores along whole tile rows (no accumulators, no LDS staging, no barrier);
    // accumulating into C leaves it as it is.
    if (p.beta) return;
    constexpr int EB = OUT_F32 ? 4 : 2;    // bytes per output element
    constexpr int TPR = BN * EB / 16;      // threads per tile row
    constexpr int RPI = NTHR / TPR;        // tile rows per pass of the workgroup
    const int col = n0 + (tid % TPR) * (16 / EB);
    if (col < p.N) {
      char* base = static_cast<char*>(p.C) + static_cast<int64_t>(grp) * p.c_gstride * EB;
      for (int r = tid / TPR; r < BM && row_begin + r < row_end; r += RPI)
        store_nt(reinterpret_cast<uint4*>(base + (static_cast<int64_t>(row_begin + r) * p.ldc + col) * EB),
                 make_uint4(0u, 0u, 0u, 0u));
    }
    return;
  }
  if constexpr (PING_PONG) {
    // Two wave groups, waves 0-3 (rows 0-127 of the tile) and 4-7 (rows 128-255); wave w
    // and w+4 share a SIMD.  Every stage is a memory phase (read the stage's fragments
    // from LDS into registers, issue this wave's DMA part of stage it+D, wait for its part
    // of stage it+1) and a compute phase (MFMAs from registers only), each ended by a
    // workgroup barrier.  The second group runs one phase behind the first, so on every
    // SIMD one wave issues MFMAs while the other is in its memory phase, and a wave stalled
    // on a DMA issue no longer idles the matrix core.  Slot reuse: stage it+D overwrites
    // the slot of stage it-1, which both groups finished reading one barrier earlier.
    constexpr int D = STAGES - 1;
    const bool late = wm == 1;
    // This wave's 32-row accumulator blocks that hold rows of the group.  In a group's last
    // row tile the blocks past its end are padding that the epilogue never stores: their
    // fragment reads and MFMAs are skipped (the loads still run, every wave takes its part
    // of each stage's DMA).  Wave-uniform, so the skip is a scalar branch.
    const int vi = __builtin_amdgcn_readfirstlane(min(NI, max(0, (row_end - row_begin - wm * WTM + 31) / 32)));
#pragma unroll
    for (int st = 0; st < D; ++st)
      if (st < nk) issue_stage(st);
    wait_vm(max(0, min(D, nk) - 1) * NDMA);
    block_barrier();
    if (late) block_barrier();
    // FULL: every block of the wave is live (all but the last row tile of a group); the
    // partial copy of the loop differs only by the per-block guards.
    auto main_loop = [&](auto full) {
      constexpr bool FULL = decltype(full)::value;
      for (int it = 0; it < nk; ++it) {
        const uint16_t* As = lds + (it % STAGES) * STAGE_ELEMS;
        const uint16_t* Bs = As + TILE;
        bf16x8_t fa[BK / 16][NI], fb[BK / 16][NJ];
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
#pragma unroll
          for (int i = 0; i < NI; ++i)
            if (FULL || i < vi) fa[ks][i] = frag(As, AMAJ, wm * WTM + i * 32, ks);
#pragma unroll
          for (int j = 0; j < NJ; ++j) fb[ks][j] = frag(Bs, BMAJ, wn * WTN + j * 32, ks);
        }
        if (it + D < nk) issue_stage(it + D);
        wait_lgkm0();  // fragments in registers before the slot may be refilled
        wait_vm(max(0, min(it + D, nk - 1) - (it + 1)) * NDMA);  // own part of stage it+1 landed
        __builtin_amdgcn_sched_barrier(0);
        block_barrier();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks)
#pragma unroll
          for (int i = 0; i < NI; ++i)
            if (FULL || i < vi) {
#pragma unroll
              for (int j = 0; j < NJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks][j], fa[ks][i], acc[i][j], 0, 0, 0);
            }
        __builtin_amdgcn_sched_barrier(0);
        block_barrier();
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (vi == NI)
      main_loop(std::true_type{});
    else
      main_loop(std::false_type{});
    if (!late) block_barrier();
  } else {
    // prologue: stages 0 .. STAGES-2 in flight
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
      if (st < nk) issue_stage(st);
    for (int it = 0; it < nk; ++it) {
      // stage `it` has landed once at most (stages issued after it) * NDMA loads of this
      // wave are pending
      const int ahead = min(STAGES - 2, nk - 1 - it);
      wait_vm(ahead * NDMA);
      block_barrier();  // every wave's part of stage `it` is in LDS; stage it-1 is consumed
      if (it + STAGES - 1 < nk) issue_stage(it + STAGES - 1);  // into the slot stage it-1 freed
      const uint16_t* As = lds + (it % STAGES) * STAGE_ELEMS;
      const uint16_t* Bs = As + TILE;
      // Fragments are double-buffered over the 16-wide substeps: the reads of substep ks+1
      // are in flight while the MFMAs of substep ks run.
      bf16x8_t fa[2][NI], fb[2][NJ];
      auto load_frags = [&](int ks, bf16x8_t* a, bf16x8_t* b) {
#pragma unroll
        for (int i = 0; i < NI; ++i) a[i] = frag(As, AMAJ, wm * WTM + i * 32, ks);
#pragma unroll
        for (int j = 0; j < NJ; ++j) b[j] = frag(Bs, BMAJ, wn * WTN + j * 32, ks);
      };
      load_frags(0, fa[0], fb[0]);
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        if (ks + 1 < BK / 16) load_frags(ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
        // keep the scheduler from sinking these reads below the MFMAs (it would, to save
        // registers, and expose the LDS latency before every MFMA pair)
        __builtin_amdgcn_sched_barrier(0);
        // B fragment first: the accumulator comes out transposed (see the epilogue)
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks & 1][j], fa[ks & 1][i], acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // ------------------------------------------------------------ epilogue
  // acc[i][j][4q + c] is row wm*WTM + i*32 + lane%32 and column
  // wn*WTN + j*32 + 8q + 4*(lane/32) + c of the tile (c = 0..3: consecutive columns).
  // The tile goes through LDS in two passes of 128 rows (pass h takes accumulator rows
  // i = 2h, 2h+1 of every wave; 128 KB, the whole of LDS), row-major with the 16-byte chunk
  // c of pass row lr at lr * 64 + (c ^ (lr & 63)).  Each wave then works on whole tile rows,
  // so every global access of the epilogue is a contiguous run of a row (a 1 KB row of fp32
  // per instruction for the plain store) instead of 16-byte pieces of 32 rows.
  const int64_t cg = RAG == RAGGED_K ? static_cast<int64_t>(grp) * p.c_gstride : 0;
  uint16_t* C = static_cast<uint16_t*>(p.C) + cg;
  float* Cf = static_cast<float*>(p.C) + cg;
  const int cbase = 4 * (lane >> 5);
  float4* L4 = reinterpret_cast<float4*>(lds);
  static_assert(STAGES * STAGE_ELEMS * 2 >= 128 * BN * 4, "epilogue staging needs 128 KB of LDS");
  auto pass_row = [&](int lr, int h) { return row_begin + (lr >> 6) * WTM + h * 64 + (lr & 63); };
  auto chunk = [&](int lr, int c) -> const float4& { return L4[lr * 64 + (c ^ (lr & 63))]; };
  if (RAG == RAGGED_K && EPI == EPI_STORE && !OUT_F32) {
    if (!p.beta) {
      // bf16 weight gradient, overwritten: rounded in registers, so the whole 256 x 256
      // tile fits the LDS in one pass (8-byte unit u of tile row r at r * 64 + (u ^ (r & 63)),
      // four consecutive columns), then stored a 512-byte row per wave instruction.
      uint2* U2 = reinterpret_cast<uint2*>(lds);
      block_barrier();  // the main loop is done with the LDS
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int lr = wm * WTM + i * 32 + (lane & 31);
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int u = (wn * WTN + j * 32 + 8 * q + cbase) >> 2;
            U2[lr * 64 + (u ^ (lr & 63))] = make_uint2(pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                                                       pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]));
          }
      }
      lds_barrier();
      const int col = n0 + 4 * lane;
#pragma unroll 4
      for (int rr = 0; rr < BM / NWAVES; ++rr) {
        const int lr = wave * (BM / NWAVES) + rr;
        const int row = row_begin + lr;
        if (row >= row_end || col >= p.N) continue;
        store_nt(reinterpret_cast<uint2*>(C + static_cast<int64_t>(row) * p.ldc + col), U2[lr * 64 + (lane ^ (lr & 63))]);
      }
      return;
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    block_barrier();  // the previous use of LDS (main loop, or the previous pass) is over
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int i = 2 * h + ii;
      const int lr = wm * 64 + ii * 32 + (lane & 31);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = (wn * WTN + j * 32 + 8 * q + cbase) >> 2;
          L4[lr * 64 + (c ^ (lr & 63))] =
              make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        }
    }
    lds_barrier();
    if (EPI == EPI_SWIGLU_FWD) {
      // tile column blocks of 32 alternate gate and up (block 2b gate, 2b + 1 up, for
      // output columns nt*128 + 32b ..); two rows per step, 32 lanes per row, lane l the
      // output columns 4l .. 4l+3 of its row
      const int l = lane & 31;
      const int cgate = (l >> 3) * 16 + (l & 7), col = nt * 128 + 4 * l;
#pragma unroll 2
      for (int rr = 0; rr < 8; ++rr) {
        const int lr = wave * 16 + 2 * rr + (lane >> 5);
        const int row = pass_row(lr, h);
        if (row < row_end) {
          const float4 gt = chunk(lr, cgate), up = chunk(lr, cgate + 8);
          float* hrow = Cf + static_cast<int64_t>(row) * p.ldc;
          store_nt(reinterpret_cast<float4*>(hrow + col), gt);
          store_nt(reinterpret_cast<float4*>(hrow + p.F + col), up);
          uint2 av;
          av.x = pack_bf16x2(glu_f(p.glu, gt.x, up.x), glu_f(p.glu, gt.y, up.y));
          av.y = pack_bf16x2(glu_f(p.glu, gt.z, up.z), glu_f(p.glu, gt.w, up.w));
          store_nt(reinterpret_cast<uint2*>(p.C2 + static_cast<int64_t>(row) * p.ldc2 + col), av);
        }
      }
    } else {
      // one row per step, lane l the tile columns 4l .. 4l+3
      const int col = n0 + 4 * lane;
#pragma unroll 4
      for (int rr = 0; rr < 16; ++rr) {
        const int lr = wave * 16 + rr;
        const int row = pass_row(lr, h);
        if (row >= row_end || col >= p.N) continue;
        const float4 v = chunk(lr, lane);
        if (EPI == EPI_SWIGLU_BWD) {
          // dAct -> dH: gate and up halves from the saved fp32 H
          const float* hrow = p.H + static_cast<int64_t>(row) * p.ldh;
          const float4 gt = *reinterpret_cast<const float4*>(hrow + col);
          const float4 up = *reinterpret_cast<const float4*>(hrow + p.F + col);
          const float g[4] = {gt.x, gt.y, gt.z, gt.w}, u[4] = {up.x, up.y, up.z, up.w};
          const float dv[4] = {v.x, v.y, v.z, v.w};
          float dg[4], du[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) glu_grad_f(p.glu, g[c], u[c], dv[c], dg[c], du[c]);
          uint16_t* drow = C + static_cast<int64_t>(row) * p.ldc;
          store_nt(reinterpret_cast<uint2*>(drow + col), make_uint2(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3])));
          store_nt(reinterpret_cast<uint2*>(drow + p.F + col), make_uint2(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3])));
        } else if (OUT_F32) {
          float4* dst = reinterpret_cast<float4*>(Cf + static_cast<int64_t>(row) * p.ldc + col);
          if (p.beta) {
            const float4 o = *dst;
            *dst = make_float4(o.x + v.x, o.y + v.y, o.z + v.z, o.w + v.w);
          } else {
            store_nt(dst, v);
          }
        } else {
          uint2* dst = reinterpret_cast<uint2*>(C + static_cast<int64_t>(row) * p.ldc + col);
          float4 w = v;
          if (p.beta) {   // one rounding of old + fp32 accumulator
            const uint2 o = *dst;
            w.x += __uint_as_float(o.x << 16);
            w.y += __uint_as_float(o.x & 0xFFFF0000u);
            w.z += __uint_as_float(o.y << 16);
            w.w += __uint_as_float(o.y & 0xFFFF0000u);
          }
          store_nt(dst, make_uint2(pack_bf16x2(w.x, w.y), pack_bf16x2(w.z, w.w)));
        }
      }
    }
  }
}


// out[i] = sum over s of part[s][i], s in order (+ out[i] when beta), four elements a lane
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int splits, int64_t elems,
                                                            void* __restrict__ out, int out_bf16, int beta) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= elems) return;
  float4 v = *reinterpret_cast<const float4*>(part + i);
  for (int q = 1; q < splits; ++q) {
    const float4 u = *reinterpret_cast<const float4*>(part + q * elems + i);
    v = make_float4(v.x + u.x, v.y + u.y, v.z + u.z, v.w + u.w);
  }
  if (out_bf16) {
    uint2* dst = reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + i);
    if (beta) {   // one rounding of old + the fp32 sum
      const uint2 o = *dst;
      v.x += __uint_as_float(o.x << 16);
      v.y += __uint_as_float(o.x & 0xFFFF0000u);
      v.z += __uint_as_float(o.y << 16);
      v.w += __uint_as_float(o.y & 0xFFFF0000u);
    }
    *dst = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
  } else {
    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(out) + i);
    if (beta) {
      const float4 o = *dst;
      v = make_float4(o.x + v.x, o.y + v.y, o.z + v.z, o.w + v.w);
    }
    *dst = v;
  }
}

template <int AMAJ, int BMAJ, int RAG, int EPI, bool OUT_F32, int GA>
void launch_kernel(const MfmaArgs& a, int64_t grid, hipStream_t s) {
  gemm_mfma_kernel<AMAJ, BMAJ, RAG, EPI, OUT_F32, GA><<<static_cast<unsigned>(grid), NTHR, 0, s>>>(a);
}

}  // namespace

size_t mfma_schedule_bytes(int G, int64_t rows) {
  return static_cast<size_t>(G + 1 + ceil_div(rows, int64_t{BM}) + G) * sizeof(int32_t);
}

// A one-group weight gradient whose output has fewer than 128 tiles (a shared expert's
// narrow projections: 32 or 16 tiles on a chip of 256 CUs) is split over its reduction
// rows into up to 8 chunks of at least 256 rows, so that about 256 workgroups run.
WgradSplit wgrad_split(int M, int N, int64_t rows) {
  const int64_t tiles = ceil_div(static_cast<int64_t>(M), BM) * ceil_div(static_cast<int64_t>(N), BN);
  const int64_t want = std::min<int64_t>({8, 256 / std::max<int64_t>(tiles, 1), rows / 256});
  if (tiles >= 128 || want < 2) return WgradSplit{1, static_cast<int>(rows)};
  const int64_t chunk = ceil_div(ceil_div(rows, want), 64) * 64;
  return WgradSplit{static_cast<int>(ceil_div(rows, chunk)), static_cast<int>(chunk)};
}

size_t wgrad_split_bytes(int M, int N, int64_t rows) {
  const WgradSplit sp = wgrad_split(M, N, rows);
  return sp.chunks > 1 ? static_cast<size_t>(sp.chunks) * M * N * sizeof(float) : 0;
}

moe_status_t launch_splitk_reduce(const float* part, int splits, int64_t elems, void* out, int out_dtype, int beta,
                                  hipStream_t s) {
  if (elems % 4) return fail(MOE_ERR_UNSUPPORTED, "split-K reduce: elements must be a multiple of 4");
  if (elems > 0)
    splitk_reduce_kernel<<<static_cast<unsigned>(ceil_div(elems / 4, 256)), 256, 0, s>>>(
        part, splits, elems, out, out_dtype == MOE_BF16, beta);
  return check_launch("splitk_reduce");
}

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
  a.glu = g.glu;
  a.beta = g.beta;
  a.kchunk = g.kchunk;
  a.skip = g.ragged == RAGGED_K ? g.skip : nullptr;
  int ga = 0;
  if (g.gather) {
    // the row gather is for the K-contiguous A of a row-ragged launch (the fc1 forward);
    // a gathered weight gradient runs on moe_wgrad.hip
    if (g.ragged != RAGGED_M || g.a_major != K_MAJOR)
      return fail(MOE_ERR_UNSUPPORTED, "mfma gemm: only a row-ragged launch's K-contiguous A can be gathered");
    ga = 1;
    if (static_cast<int64_t>(g.gather_rows) * g.lda * 2 > kOob - 4096)
      return fail(MOE_ERR_UNSUPPORTED, "mfma gemm: gathered operand above 2 GB");
    a.gather = g.gather;
    a.gather_rows = g.gather_rows;
    a.gather_len = static_cast<int>(g.rows_upper ? g.rows_upper : g.range_end);
  }
  if (g.b_major == K_MAJOR) {
    const int64_t bytes = static_cast<int64_t>(g.epi == EPI_SWIGLU_FWD ? 2 * g.F : g.N) * g.ldb * 2;
    if (bytes >= (int64_t{1} << 31)) return fail(MOE_ERR_UNSUPPORTED, "mfma gemm: weight matrix above 2 GB");
    a.b_rows_bytes = static_cast<int>(bytes);
  }
  int64_t grid;
  if (g.ragged == RAGGED_M) {
    a.nN = static_cast<int>(g.epi == EPI_SWIGLU_FWD ? ceil_div(g.N, 256) : ceil_div(g.N, BN));
    int64_t upper;
    if (g.offsets) {
      if (g.G > 2048) return fail(MOE_ERR_UNSUPPORTED, "mfma gemm: more than 2048 row-ragged groups");
      a.tile_cap = static_cast<int>(ceil_div(g.rows_upper, int64_t{BM}) + g.G);
      tile_prefix_kernel<<<1, 1024, 0, s>>>(g.offsets, g.G, a.tile_cap, sched);
      upper = (ceil_div(g.rows_upper, BM) + g.G) * a.nN;
    } else {
      upper = ceil_div(g.range_end, BM) * a.nN;
    }
    grid = ceil_div(upper, 8) * 8;
  } else {
    a.nM = static_cast<int>(ceil_div(g.M, BM));
    a.nN = static_cast<int>(ceil_div(g.N, BN));
    // groups: the offsets' groups, or the split-K chunks of one group
    grid = 8 * static_cast<int64_t>(g.offsets || g.kchunk ? g.G : 1) * ceil_div(static_cast<int64_t>(a.nM) * a.nN, 8);
  }
  if (grid == 0) return MOE_OK;
#define MOE_MF(AM, BMJ, RG, EP, OF, GA)                                                                    \
  if (g.a_major == AM && g.b_major == BMJ && g.ragged == RG && g.epi == EP && out_f32 == OF && ga == GA) { \
    launch_kernel<AM, BMJ, RG, EP, OF, GA>(a, grid, s);                                                    \
    return check_launch("gemm_mfma");                                                                      \
  }
  MOE_MF(K_MAJOR, K_MAJOR, RAGGED_M, EPI_SWIGLU_FWD, true, 0)    // fc1 + SwiGLU -> H (fp32), Act (bf16)
  MOE_MF(K_MAJOR, K_MAJOR, RAGGED_M, EPI_SWIGLU_FWD, true, 1)    // the same on the token rows of x
  MOE_MF(K_MAJOR, K_MAJOR, RAGGED_M, EPI_STORE, true, 0)         // fc2 -> Y (fp32)
  MOE_MF(K_MAJOR, MN_MAJOR, RAGGED_M, EPI_SWIGLU_BWD, false, 0)  // fc2 data gradient + SwiGLU backward -> dH (bf16)
  MOE_MF(K_MAJOR, MN_MAJOR, RAGGED_M, EPI_STORE, true, 0)        // fc1 data gradient -> dX (fp32)
  MOE_MF(MN_MAJOR, MN_MAJOR, RAGGED_K, EPI_STORE, true, 0)       // weight gradients (fp32)
  MOE_MF(MN_MAJOR, MN_MAJOR, RAGGED_K, EPI_STORE, false, 0)      // weight gradients (bf16, rounded once from fp32)
#undef MOE_MF
  return fail(MOE_ERR_UNSUPPORTED, "mfma gemm: unsupported operand combination");
}

}  // namespace moe
