// Weight gradients of the grouped experts: two workgroups per CU, the memory work of each
// wave interleaved with its MFMAs.
//
// The Ultimate MoE Training Handbook, §3.4 (the expert FFN): for each expert the
// gradients of its two projections, dW[g] = dY_g^T X_g over the expert's ragged block of
// reduction rows (its tokens).  Every non-empty expert owns a full grid of output tiles,
// and an expert's reduction is short (a few hundred rows), so a tile spends about as long
// on its prologue (the first stages' load latency) and its epilogue (the tile's store,
// bound by HBM writes) as on its reduction.  The 8-wave 256 x 256 kernel of
// moe_gemm_mfma.hip holds a CU alone (128 KB of LDS), so nothing hides those.  This kernel
// runs 256 x 128 tiles with 4 waves and 72 KB of LDS, so two workgroups share a CU and
// one's prologue and epilogue overlap the other's reduction.
//
// Design (per workgroup: 256 threads = 4 waves in a 2 x 2 grid, one wave per SIMD):
//   * each wave a 128 x 64 sub-tile as 4 x 2 accumulators of v_mfma_f32_32x32x16_bf16;
//   * both operands are contiguous along the output (dY [rows][M], X [rows][N]) and go
//     from HBM into LDS by buffer_load ... lds, 32 reduction rows per stage, through a
//     ring of 3 stages: A as [32][256] (2 k-rows per 1 KB load), B as [32][128] (4 k-rows
//     per load), the 16-byte chunk index XORed by 4 (k & 3), read with the transposing
//     ds_read_b64_tr_b16 (these 8-byte reads run at 128 B/clk per CU, half the rate of
//     16-byte reads, so the LDS carries a large share of the stage);
//   * a stage is two 16-deep substeps of 8 MFMAs.  After each MFMA the wave issues its
//     share of the next substep's fragment reads (in the order the next MFMAs need them)
//     and, in the second substep, one load of the stage three ahead, so the wave's own
//     memory work runs between its MFMAs; the other workgroup's wave on the SIMD fills in
//     while one waits;
//   * one barrier per stage, taken once stage st+1 has landed and this wave's reads of
//     stage st have returned; after it the slot of stage st takes stage st + 3;
//   * every slot is loaded on that fixed schedule, past the group's end too (empty
//     descriptors, zeros), so the loop has no branches and its wait counts are
//     constants; the last stage is peeled off the loop;
//   * X read through a row gather (x_rows): the indices of stage st + 3 travel into LDS
//     with stage st (a 4-byte-per-lane load into an 8-slot ring);
//   * descriptor-bounded loads: rows past the group's end and indices past the source
//     read zeros, so the ragged tail needs no code;
//   * the epilogue stages the tile through the LDS (bf16 overwritten: one pass of the
//     rounded tile, 64 KB; otherwise two passes of 128 fp32 rows, 64 KB each) and stores
//     whole tile rows, non-temporal (the gradient, and the zeros of a group without rows,
//     are written once and would only evict operand lines from L2); the bf16 overwrite,
//     bf16 accumulate and fp32 outputs are separate
//     kernels (a run-time branch between the epilogues makes the register allocator spill
//     the accumulators).
#include <algorithm>
#include <type_traits>

#include "moe_internal.h"

namespace moe {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int BM = 256, BN = 128, BK = 32, STAGES = 3, NTHR = 256;
constexpr int WTM = 128, WTN = 64, NI = WTM / 32, NJ = WTN / 32;
constexpr int A_ELEMS = BK * BM, B_ELEMS = BK * BN, STAGE_ELEMS = A_ELEMS + B_ELEMS;  // bf16 elements
constexpr int A_DMA = A_ELEMS / 512 / 4, B_DMA = B_ELEMS / 512 / 4;  // 1 KB loads per wave: 4 and 2
constexpr int NDMA = A_DMA + B_DMA;
constexpr int LPR_B = BN / 8;                         // 16-byte chunks (lanes) per B row
constexpr int MPS = NI * NJ, RPS = 2 * (NI + NJ);     // MFMAs and fragment reads per substep
constexpr int TOK_SLOTS = 8;
constexpr int kRsrcFlags = 0x00020000;
constexpr int kOob = 0x7FFFFFF0;   // an offset past every gathered operand's descriptor

struct WgArgs {
  const uint16_t* A;   // dY [rows][M], row stride lda
  int64_t lda;
  const uint16_t* B;   // X [rows or gather_rows][N], row stride ldb
  int64_t ldb;
  void* C;             // dW [G][M][N], row stride ldc, group stride c_gstride (elements)
  int64_t ldc, c_gstride;
  const int32_t* offsets;   // [G + 1] or NULL (one group over [0, range_end))
  const int32_t* gather;    // NULL, or the source row of each reduction row
  int gather_rows, gather_len;
  int G, M, N, range_end, nM, nN;
  int band;            // row tiles per band of an XCD's run of a group's tiles (wgrad_band)
  int beta;            // 1: add into C
  const int32_t* skip;    // skew plan: groups left to the split path, or NULL
  const int32_t* pairs;   // skew plan: [2 G] row range of each group (instead of offsets), or NULL
  const int32_t* gcount;  // skew plan: groups that exist, or NULL
};

__device__ __forceinline__ int swm(int k) { return (k & 3) << 2; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kRsrcFlags);
}
// Transposing LDS read; the restrict parameter gives the call alias-scope information, so
// the compiler does not wait for the LDS-DMA loads in flight before it (the waits below
// order the reads after the DMA).
__device__ __attribute__((always_inline)) inline i16x4_t lds_read_tr(lds_i16x4_t* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
}
// Waits until at most N (0..63) of this wave's vector memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm_c() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
  asm volatile("" ::: "memory");
}
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

// OUT: 0 bf16 overwritten, 1 bf16 accumulated, 2 fp32 (accumulated when p.beta).
template <int OUT, bool GATHER>
__device__ __forceinline__ void wgrad_body(const WgArgs& p) {
  constexpr bool OUT_F32 = OUT == 2;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[STAGES * STAGE_ELEMS + (GATHER ? TOK_SLOTS * 64 * 2 : 0)];
  int32_t(*tok_lds)[64] = reinterpret_cast<int32_t(*)[64]>(lds + STAGES * STAGE_ELEMS);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // ---------------------------------------------------------------- tile
  // each group's tiles in 8 runs, one per XCD, bands of p.band row tiles walked column by
  // column
  const int WG_BAND = p.band;
  const int per = p.nM * p.nN;
  const int run = (per + 7) >> 3;
  const int h = blockIdx.x;
  const int q8 = h >> 3;
  const int grp = q8 / run;
  const int local = (h & 7) * run + (q8 - grp * run);
  if (grp >= p.G || local >= per) return;
  if ((p.gcount && grp >= *p.gcount) || (p.skip && p.skip[grp])) return;
  const int band = local / (WG_BAND * p.nN);
  const int rem = local - band * WG_BAND * p.nN;
  const int bh = min(WG_BAND, p.nM - band * WG_BAND);
  const int nt = rem / bh;
  const int mt = band * WG_BAND + (rem - nt * bh);
  const int row_begin = mt * BM, n0 = nt * BN;
  const int k_begin = p.pairs ? p.pairs[2 * grp] : (p.offsets ? p.offsets[grp] : 0);
  const int k_end = p.pairs ? p.pairs[2 * grp + 1] : (p.offsets ? p.offsets[grp + 1] : p.range_end);
  const int nk = k_end > k_begin ? (k_end - k_begin + BK - 1) / BK : 0;
  const int64_t cg = static_cast<int64_t>(grp) * p.c_gstride;

  if (nk == 0) {
    // a group without rows: exact zeros when overwriting, untouched when accumulating
    if (OUT == 1 || p.beta) return;
    constexpr int EB = OUT_F32 ? 4 : 2;
    constexpr int TPR = BN * EB / 16;
    constexpr int RPI = NTHR / TPR;
    const int col = n0 + (tid % TPR) * (16 / EB);
    if (col < p.N) {
      char* base = static_cast<char*>(p.C) + cg * EB;
      for (int r = tid / TPR; r < BM && row_begin + r < p.M; r += RPI)
        store_nt(reinterpret_cast<uint4*>(base + (static_cast<int64_t>(row_begin + r) * p.ldc + col) * EB),
                 make_uint4(0u, 0u, 0u, 0u));
    }
    return;
  }

  // ---------------------------------------------------------------- HBM -> LDS (DMA)
  // A block b (1 KB) = k-rows 2b, 2b+1 of the stage, 256 columns (lane: row 2b + lane/32,
  // chunk lane%32); B block b = k-rows 4b .. 4b+3, 128 columns (lane: row 4b + lane/16,
  // chunk lane%16).  LDS position q of a row holds chunk q ^ swm(k).
  auto krA = [&](int q) { return (wave * A_DMA + q) * 2 + (lane >> 5); };
  auto krB = [&](int q) { return (wave * B_DMA + q) * (64 / LPR_B) + lane / LPR_B; };
  int voffA[A_DMA], colB[B_DMA];
#pragma unroll
  for (int q = 0; q < A_DMA; ++q) {
    const int kr = krA(q);
    voffA[q] = kr * static_cast<int>(p.lda) * 2 + (row_begin + (((lane & 31) ^ swm(kr)) * 8)) * 2;
  }
#pragma unroll
  for (int q = 0; q < B_DMA; ++q) colB[q] = (n0 + (((lane % LPR_B) ^ swm(krB(q))) * 8)) * 2;
  // a stage past the group's end gets an empty descriptor (its loads write zeros)
  auto stage_A_rsrc = [&](int st) {
    const int k0 = min(k_begin + st * BK, k_end);
    return make_rsrc(p.A + static_cast<int64_t>(k0) * p.lda, min(BK, k_end - k0) * static_cast<int>(p.lda) * 2);
  };
  auto stage_B_rsrc = [&](int st) {
    if constexpr (GATHER) return make_rsrc(p.B, p.gather_rows * static_cast<int>(p.ldb) * 2);
    const int k0 = min(k_begin + st * BK, k_end);
    return make_rsrc(p.B + static_cast<int64_t>(k0) * p.ldb, min(BK, k_end - k0) * static_cast<int>(p.ldb) * 2);
  };
  // B byte offsets: consecutive rows, or the gathered source rows (src), a row past the
  // group's end or a negative index going past the descriptor
  auto voffB_of = [&](int st, int q, int src) {
    const int kr = krB(q);
    if constexpr (GATHER)
      return (k_begin + st * BK + kr < k_end && src >= 0) ? src * static_cast<int>(p.ldb) * 2 + colB[q] : kOob;
    else
      return kr * static_cast<int>(p.ldb) * 2 + colB[q];
  };
  constexpr int GL = NDMA + (GATHER ? 1 : 0);   // loads per stage and wave
  // load q of stage st (q < A_DMA: A; then B; q = NDMA: the indices of stage st + STAGES)
  auto issue_one = [&](int st, int q, const int (&src)[B_DMA]) __attribute__((always_inline)) {
    uint16_t* dst = lds + (st % STAGES) * STAGE_ELEMS;
    if (q < A_DMA) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(stage_A_rsrc(st), (lds_void_t*)(dst + (wave * A_DMA + q) * 512), 16,
                                               voffA[q], 0, 0, 0);
    } else if (q < NDMA) {
      const int qb = q - A_DMA;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(stage_B_rsrc(st), (lds_void_t*)(dst + A_ELEMS + (wave * B_DMA + qb) * 512),
                                               16, voffB_of(st, qb, src[qb]), 0, 0, 0);
    } else if (GATHER) {
      const int tst = st + STAGES;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(p.gather, p.gather_len * 4),
                                               (lds_void_t*)(&tok_lds[tst % TOK_SLOTS][0]), 4,
                                               (k_begin + tst * BK + lane) * 4, 0, 0, 0);
    }
  };

  // ---------------------------------------------------------------- LDS -> fragments
  // fragment read r of a substep, two transposing reads per 32 x 16 fragment (hh = r & 1),
  // fragments in the order the next substep's MFMAs first need them: A0, B0 .. B(NJ-1),
  // A1 .. A(NI-1) (half[buf][f]: f < NI the A blocks, NI + j the B blocks)
  i16x4_t half[2][NI + NJ][2];
  auto read_one = [&](auto bufc, int st, int ks, int r) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    const int fr = r >> 1, hh = r & 1;
    const bool is_a = fr == 0 || fr > NJ;
    const int blk = fr == 0 ? 0 : (is_a ? fr - NJ : fr - 1);
    const int f = is_a ? blk : NI + blk;
    const int W = is_a ? BM : BN;
    const uint16_t* t = lds + (st % STAGES) * STAGE_ELEMS + (is_a ? 0 : A_ELEMS);
    const int rb0 = (is_a ? wm * WTM : wn * WTN) + blk * 32;
    const int j = lane & 15, g = lane >> 4;
    const int col = rb0 + 16 * (g & 1) + 4 * (j & 3);
    const int kr = ks * 16 + 8 * (g >> 1) + 4 * hh + (j >> 2);
    half[buf][f][hh] = lds_read_tr((lds_i16x4_t*)(t + kr * W + (((col >> 3) ^ swm(kr)) << 3) + (col & 7)));
  };
  auto frag = [&](int buf, int f) __attribute__((always_inline)) -> bf16x8_t {
    const i16x4_t lo = half[buf][f][0], hi = half[buf][f][1];
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16_t acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // ---------------------------------------------------------------- main loop
  {
    int src0[STAGES][B_DMA];
#pragma unroll
    for (int st = 0; st < STAGES; ++st)
#pragma unroll
      for (int q = 0; q < B_DMA; ++q) {
        const int row = k_begin + st * BK + krB(q);
        src0[st][q] = GATHER && row < k_end && row < p.gather_len ? p.gather[row] : -1;
      }
#pragma unroll
    for (int st = 0; st < STAGES; ++st)
#pragma unroll
      for (int q = 0; q < GL; ++q) issue_one(st, q, src0[st]);
  }
  wait_vm_c<(STAGES - 1) * GL>();   // stage 0 landed
  block_barrier();
#pragma unroll
  for (int r = 0; r < RPS; ++r) read_one(std::integral_constant<int, 0>{}, 0, 0, r);

  // one substep: MPS MFMAs on fragment buffer cur; after MFMA r, its share of the next
  // substep's fragment reads (into 1 - cur) and, when loading, load r of stage ld_st
  auto substep = [&](auto curc, auto rdc, auto ldc, int rd_st, int rd_ks, int ld_st, const int (&src)[B_DMA])
                     __attribute__((always_inline)) {
    constexpr int cur = decltype(curc)::value;
    constexpr bool rd = decltype(rdc)::value, ld = decltype(ldc)::value;
#pragma unroll
    for (int r = 0; r < MPS; ++r) {
      const int i = r / NJ, jj = r % NJ;
      acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag(cur, NI + jj), frag(cur, i), acc[i][jj], 0, 0, 0);
      if constexpr (rd) {
#pragma unroll
        for (int q = r * RPS / MPS; q < (r + 1) * RPS / MPS; ++q) read_one(std::integral_constant<int, 1 - cur>{}, rd_st, rd_ks, q);
      }
      if constexpr (ld)
        if (r < GL) issue_one(ld_st, r, src);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (ld)
#pragma unroll
      for (int q = MPS; q < GL; ++q) issue_one(ld_st, q, src);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using T = std::true_type;
  using F = std::false_type;
  const int no_src[B_DMA] = {};
  for (int it = 0; it < nk - 1; ++it) {
    // (it, 0) in buffer 0; read (it, 1)
    substep(I0{}, T{}, F{}, it, 1, 0, no_src);
    // stage it+1 landed (the later ones may be in flight) and this wave's reads of stage it
    // returned; after the barrier every wave is done with stage it, whose slot takes stage
    // it + STAGES
    wait_lgkm0();
    wait_vm_c<(STAGES - 2) * GL>();
    block_barrier();
    int src[B_DMA];
#pragma unroll
    for (int q = 0; q < B_DMA; ++q) src[q] = GATHER ? tok_lds[(it + STAGES) % TOK_SLOTS][krB(q)] : 0;
    substep(I1{}, T{}, T{}, it + 1, 0, it + STAGES, src);
  }
  substep(I0{}, T{}, F{}, nk - 1, 1, 0, no_src);
  substep(I1{}, F{}, F{}, 0, 0, 0, no_src);
  wait_vm_c<0>();   // the loads past the group's end write the LDS too

  // ---------------------------------------------------------------- epilogue
  // acc[i][j][4u + c] is tile row wm*128 + i*32 + lane%32, column wn*64 + j*32 + 8u +
  // 4 (lane/32) + c
  const int cbase = 4 * (lane >> 5);
  if constexpr (OUT == 0) {
    // bf16, overwritten: the rounded tile in LDS in one pass (8-byte unit u of row r at
    // r * 32 + (u ^ (r % 32))), then two whole rows per store instruction
    constexpr int UPR = BN / 4;
    uint2* U2 = reinterpret_cast<uint2*>(lds);
    block_barrier();  // every wave is done with the last stage
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = wm * WTM + i * 32 + (lane & 31);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c = (wn * WTN + j * 32 + 8 * u + cbase) >> 2;
          U2[r * UPR + (c ^ (r & (UPR - 1)))] = make_uint2(pack_bf16x2(acc[i][j][4 * u], acc[i][j][4 * u + 1]),
                                                           pack_bf16x2(acc[i][j][4 * u + 2], acc[i][j][4 * u + 3]));
        }
    }
    lds_barrier();
    uint16_t* C = static_cast<uint16_t*>(p.C) + cg;
    constexpr int RPI = 64 / UPR;                 // rows per store instruction
    constexpr int NST = BM / 4 / RPI, CH = 16;    // store instructions per wave
    const int l = lane % UPR, col = n0 + 4 * l;
#pragma unroll
    for (int s0 = 0; s0 < NST; s0 += CH) {
      uint2 v[CH];
#pragma unroll
      for (int q = 0; q < CH; ++q) {
        const int r = wave * (BM / 4) + (s0 + q) * RPI + lane / UPR;
        v[q] = U2[r * UPR + (l ^ (r & (UPR - 1)))];
      }
#pragma unroll
      for (int q = 0; q < CH; ++q) {
        const int row = row_begin + wave * (BM / 4) + (s0 + q) * RPI + lane / UPR;
        if (row < p.M && col < p.N) store_nt(reinterpret_cast<uint2*>(C + static_cast<int64_t>(row) * p.ldc + col), v[q]);
      }
    }
    return;
  }
  // fp32 out, or accumulating: two passes of 128 tile rows (16-byte chunk c of pass row lr
  // at lr * FPR + (c ^ (lr % FPR))); pass hp holds the accumulator blocks i = 2hp, 2hp+1 of
  // every wave: pass row lr is tile row (lr / 64) * 128 + 64 hp + lr % 64
  constexpr int FPR = BN / 4;
  float4* L4 = reinterpret_cast<float4*>(lds);
  static_assert(STAGES * STAGE_ELEMS * 2 >= 128 * BN * 4, "an epilogue pass needs 64 KB of LDS");
  auto pass = [&](auto hc) {
    constexpr int hp = decltype(hc)::value;
    block_barrier();
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int i = 2 * hp + ii;
      const int lr = wm * 64 + ii * 32 + (lane & 31);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c = (wn * WTN + j * 32 + 8 * u + cbase) >> 2;
          L4[lr * FPR + (c ^ (lr & (FPR - 1)))] =
              make_float4(acc[i][j][4 * u], acc[i][j][4 * u + 1], acc[i][j][4 * u + 2], acc[i][j][4 * u + 3]);
        }
    }
    lds_barrier();
    constexpr int RPI = 64 / FPR;
    const int l = lane % FPR, col = n0 + 4 * l;
#pragma unroll 4
    for (int q = 0; q < 32 / RPI; ++q) {
      const int lr = wave * 32 + q * RPI + lane / FPR;
      const int row = row_begin + (lr >> 6) * WTM + hp * 64 + (lr & 63);
      if (row >= p.M || col >= p.N) continue;
      const float4 v = L4[lr * FPR + (l ^ (lr & (FPR - 1)))];
      if constexpr (OUT_F32) {
        float4* dst = reinterpret_cast<float4*>(static_cast<float*>(p.C) + cg + static_cast<int64_t>(row) * p.ldc + col);
        if (p.beta) {
          const float4 o = *dst;
          *dst = make_float4(o.x + v.x, o.y + v.y, o.z + v.z, o.w + v.w);
        } else {
          store_nt(dst, v);
        }
      } else {
        uint2* dst = reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.C) + cg + static_cast<int64_t>(row) * p.ldc + col);
        float4 w = v;
        const uint2 o = *dst;
        w.x += __uint_as_float(o.x << 16);
        w.y += __uint_as_float(o.x & 0xFFFF0000u);
        w.z += __uint_as_float(o.y << 16);
        w.w += __uint_as_float(o.y & 0xFFFF0000u);
        store_nt(dst, make_uint2(pack_bf16x2(w.x, w.y), pack_bf16x2(w.z, w.w)));
      }
    }
  };
  pass(std::integral_constant<int, 0>{});
  pass(std::integral_constant<int, 1>{});
}

// one plain kernel per output and row source (kernel templates whose bodies hold lambdas
// lose their host launch stubs)
__global__ __launch_bounds__(NTHR, 2) void wgrad_bf16(const WgArgs p) { wgrad_body<0, false>(p); }
__global__ __launch_bounds__(NTHR, 2) void wgrad_bf16_gather(const WgArgs p) { wgrad_body<0, true>(p); }
__global__ __launch_bounds__(NTHR, 2) void wgrad_bf16_acc(const WgArgs p) { wgrad_body<1, false>(p); }
__global__ __launch_bounds__(NTHR, 2) void wgrad_bf16_acc_gather(const WgArgs p) { wgrad_body<1, true>(p); }
__global__ __launch_bounds__(NTHR, 2) void wgrad_f32(const WgArgs p) { wgrad_body<2, false>(p); }
__global__ __launch_bounds__(NTHR, 2) void wgrad_f32_gather(const WgArgs p) { wgrad_body<2, true>(p); }

}  // namespace

// ---------------------------------------------------------------- skew splitting
// A group's weight-gradient tiles each reduce over all of the group's rows.  When one group
// holds a large share of the rows (a long-tailed routing), its few tiles run for the whole
// launch on a few CUs while the others idle.  The plan cuts every group with more rows
// than the chunk into row chunks; the main launch skips those groups, one fp32 launch
// computes a partial per chunk, and the partials are summed in chunk order.
namespace {

// One block, thread i holding groups 4i .. 4i + 3 (G <= 4096): per group its chunk count
// (0 when not split) and split flag, their prefix sums by wave shuffles and the 16 wave
// totals, then the tables.
__global__ __launch_bounds__(1024) void skew_plan_kernel(const int32_t* __restrict__ offsets, int G, int chunk,
                                                         int max_vg, int max_split, int32_t* __restrict__ plan) {
  __shared__ int wn[16], wf[16];
  int32_t* skip = plan;
  int32_t* gcount = plan + G;
  int32_t* nsplit = plan + G + 1;
  int32_t* pairs = plan + G + 2;
  int32_t* split_e = pairs + 2 * max_vg;
  int32_t* split_first = split_e + max_split;
  int32_t* split_n = split_first + max_split;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int n[4], tn = 0, tf = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = 4 * tid + u;
    n[u] = 0;
    if (e < G) {
      const int r = offsets[e + 1] - offsets[e];
      n[u] = r > chunk ? (r + chunk - 1) / chunk : 0;
      skip[e] = n[u] > 0;
    }
    tn += n[u];
    tf += n[u] > 0;
  }
  int in = tn, inf = tf;   // inclusive prefixes at the thread's last group
  for (int o = 1; o < 64; o <<= 1) {
    const int a = __shfl_up(in, o, 64), b = __shfl_up(inf, o, 64);
    if (lane >= o) {
      in += a;
      inf += b;
    }
  }
  if (lane == 63) {
    wn[w] = in;
    wf[w] = inf;
  }
  __syncthreads();
  for (int i = 0; i < w; ++i) {
    in += wn[i];
    inf += wf[i];
  }
  int vb = in - tn, j = inf - tf;   // first chunk and split index of the thread's first group
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = 4 * tid + u;
    if (n[u] > 0) {
      if (j < max_split) {
        split_e[j] = e;
        split_first[j] = vb;
        split_n[j] = n[u];
      }
      const int lo = offsets[e], hi = offsets[e + 1];
      for (int c = 0; c < n[u] && vb + c < max_vg; ++c) {
        pairs[2 * (vb + c)] = lo + c * chunk;
        pairs[2 * (vb + c) + 1] = min(lo + (c + 1) * chunk, hi);
      }
      ++j;
    }
    vb += n[u];
  }
  if (tid == 1023) {   // its inclusive prefixes cover all 4096 slots
    *gcount = min(in, max_vg);
    *nsplit = min(inf, max_split);
  }
}

// dW[e] = the split group's partials summed in chunk order (+ dW when beta), four
// elements a thread; blockIdx.y = split group j (those past *nsplit do nothing).
__global__ __launch_bounds__(256) void skew_reduce_kernel(const float* __restrict__ part, int64_t elems,
                                                          const int32_t* __restrict__ nsplit,
                                                          const int32_t* __restrict__ split_e,
                                                          const int32_t* __restrict__ split_first,
                                                          const int32_t* __restrict__ split_n, int max_vg,
                                                          void* __restrict__ dW, int64_t c_gstride, int out_bf16,
                                                          int beta) {
  const int j = blockIdx.y;
  if (j >= *nsplit) return;
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= elems) return;
  // (the clamp keeps every read inside the partials even for offsets that break their
  // contract; for valid offsets the plan's capacity always holds every chunk)
  const int e = split_e[j], first = split_first[j], n = min(split_n[j], max_vg - first);
  if (n < 1) return;
  float4 v = *reinterpret_cast<const float4*>(part + static_cast<int64_t>(first) * elems + i);
  for (int c = 1; c < n; ++c) {
    const float4 u = *reinterpret_cast<const float4*>(part + static_cast<int64_t>(first + c) * elems + i);
    v = make_float4(v.x + u.x, v.y + u.y, v.z + u.z, v.w + u.w);
  }
  const int64_t o = static_cast<int64_t>(e) * c_gstride + i;
  if (out_bf16) {
    uint2* dst = reinterpret_cast<uint2*>(static_cast<uint16_t*>(dW) + o);
    if (beta) {   // one rounding of old + the fp32 sum
      const uint2 old = *dst;
      v.x += __uint_as_float(old.x << 16);
      v.y += __uint_as_float(old.x & 0xFFFF0000u);
      v.z += __uint_as_float(old.y << 16);
      v.w += __uint_as_float(old.y & 0xFFFF0000u);
    }
    store_nt(dst, make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)));
  } else {
    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(dW) + o);
    if (beta) {
      const float4 old = *dst;
      v = make_float4(old.x + v.x, old.y + v.y, old.z + v.z, old.w + v.w);
    }
    store_nt(dst, v);
  }
}

}  // namespace

#ifndef MOE_SKEW_PARTS
#define MOE_SKEW_PARTS 2
#endif
SkewPlan skew_plan(int G, int64_t rows, int64_t max_group_rows, int M, int N, int tiles, int slots) {
  SkewPlan sp{};
  if (G < 1 || G > 4096 || rows <= 0 || tiles <= 0 || slots <= 0) return sp;
  // a balanced launch gives each slot rows * tiles / slots rows of work; a chunk is half
  // of that (at least 1024 rows), so no tile is longer than half a slot's share (a quarter
  // or an eighth left the fp32 partials and their sum costing more than the balance won)
  int64_t chunk = std::max<int64_t>(1024, ceil_div(ceil_div(rows * tiles, slots), MOE_SKEW_PARTS));
  chunk = ceil_div(chunk, 256) * 256;
  if (chunk >= max_group_rows || chunk >= rows || chunk >= (int64_t{1} << 30)) return sp;
  sp.chunk = static_cast<int>(chunk);
  sp.max_split = static_cast<int>(rows / chunk);                       // each split group has > chunk rows
  sp.max_vg = static_cast<int>(ceil_div(rows, chunk)) + sp.max_split;  // sum of ceil(r / chunk) over them
  sp.plan_bytes = static_cast<size_t>(G + 2 + 2 * sp.max_vg + 3 * sp.max_split) * 4;
  sp.partial_bytes = static_cast<size_t>(sp.max_vg) * M * N * 4;
  return sp;
}

SkewTables skew_tables(const int32_t* plan, int G, const SkewPlan& sp) {
  SkewTables t;
  t.skip = plan;
  t.gcount = plan + G;
  t.nsplit = plan + G + 1;
  t.pairs = plan + G + 2;
  t.split_e = t.pairs + 2 * sp.max_vg;
  t.split_first = t.split_e + sp.max_split;
  t.split_n = t.split_first + sp.max_split;
  return t;
}

moe_status_t launch_skew_plan(const int32_t* offsets, int G, const SkewPlan& sp, int32_t* plan, hipStream_t s) {
  if (G < 1 || G > 4096) return fail(MOE_ERR_UNSUPPORTED, "skew plan: 1 to 4096 groups");
  skew_plan_kernel<<<1, 1024, 0, s>>>(offsets, G, sp.chunk, sp.max_vg, sp.max_split, plan);
  return check_launch("skew_plan");
}

moe_status_t launch_skew_reduce(const float* part, const SkewTables& t, const SkewPlan& sp, int64_t elems,
                                void* dW, int64_t c_gstride, int out_dtype, int beta, hipStream_t s) {
  if (elems % 4 || c_gstride % 4) return fail(MOE_ERR_UNSUPPORTED, "skew reduce: sizes must be multiples of 4");
  if (sp.max_split < 1 || elems == 0) return MOE_OK;
  const dim3 grid(static_cast<unsigned>(ceil_div(elems / 4, 256)), static_cast<unsigned>(sp.max_split));
  skew_reduce_kernel<<<grid, 256, 0, s>>>(part, elems, t.nsplit, t.split_e, t.split_first, t.split_n, sp.max_vg, dW,
                                          c_gstride, out_dtype == MOE_BF16, beta);
  return check_launch("skew_reduce");
}

bool wgrad2_supported(const GemmDesc& g) {
  return g.ragged == RAGGED_K && g.epi == EPI_STORE && g.a_major == MN_MAJOR && g.b_major == MN_MAJOR &&
         g.a_type == MOE_BF16 && g.b_type == MOE_BF16 && g.kchunk == 0 && g.M % 8 == 0 && g.N % 8 == 0 &&
         g.lda % 8 == 0 && g.ldb % 8 == 0 && g.ldc % 8 == 0 && g.c_gstride % 8 == 0;
}

// Band height of the tile walk.  An XCD runs an eighth of a group's tiles, band after
// band, each band's row tiles column by column, so in a run of r tiles it reads the dY
// columns of about b row tiles and the X columns of r / b column tiles.  b minimises that
// footprint, b BM + ceil(r / b) BN operand columns, over 1, 2 and 4 up to nM (the smaller
// b on a tie).  The 112-tile runs of the DeepSeek-V3-shaped fc1 gradient would take b = 8,
// which was slower there (9.19 against 9.06 ms) though its footprint is smaller.
static int wgrad_band(int nM, int nN) {
#ifdef MOE_WG_BAND_FIXED
  return std::min(MOE_WG_BAND_FIXED, nM);
#endif
  const int64_t run = ceil_div(static_cast<int64_t>(nM) * nN, 8);
  int best = 1;
  int64_t best_cols = INT64_MAX;
  for (int b = 1; b <= nM && b <= 4; b *= 2) {
    const int64_t cols = static_cast<int64_t>(b) * BM + ceil_div(run, b) * BN;
    if (cols < best_cols) {
      best_cols = cols;
      best = b;
    }
  }
  return best;
}

moe_status_t launch_wgrad2(const GemmDesc& g, hipStream_t s) {
  if (!wgrad2_supported(g)) return fail(MOE_ERR_UNSUPPORTED, "wgrad: unsupported operand combination");
  const int groups = g.offsets || g.pairs ? g.G : 1;
  if (groups < 1) return MOE_OK;
  WgArgs a{};
  a.A = static_cast<const uint16_t*>(g.A);
  a.lda = g.lda;
  a.B = static_cast<const uint16_t*>(g.B);
  a.ldb = g.ldb;
  a.C = g.C;
  a.ldc = g.ldc;
  a.c_gstride = g.c_gstride;
  a.offsets = g.offsets;
  a.G = groups;
  a.M = g.M;
  a.N = g.N;
  a.range_end = g.range_end;
  a.beta = g.beta;
  a.skip = g.skip;
  a.pairs = g.pairs;
  a.gcount = g.gcount;
  a.nM = static_cast<int>(ceil_div(g.M, BM));
  a.nN = static_cast<int>(ceil_div(g.N, BN));
  if (a.nM <= 0 || a.nN <= 0) return MOE_OK;
  a.band = wgrad_band(a.nM, a.nN);
  if (g.gather) {
    if (static_cast<int64_t>(g.gather_rows) * g.ldb * 2 > kOob - 4096)
      return fail(MOE_ERR_UNSUPPORTED, "wgrad: gathered operand above 2 GB");
    a.gather = g.gather;
    a.gather_rows = g.gather_rows;
    a.gather_len = g.range_end;
  }
  const int64_t grid = 8 * static_cast<int64_t>(groups) * ceil_div(static_cast<int64_t>(a.nM) * a.nN, 8);
  if (grid == 0) return MOE_OK;
  const unsigned nb = static_cast<unsigned>(grid);
  const bool gt = g.gather != nullptr;
  if (g.c_type == MOE_F32) {
    if (gt) wgrad_f32_gather<<<nb, NTHR, 0, s>>>(a);
    else wgrad_f32<<<nb, NTHR, 0, s>>>(a);
  } else if (g.beta) {
    if (gt) wgrad_bf16_acc_gather<<<nb, NTHR, 0, s>>>(a);
    else wgrad_bf16_acc<<<nb, NTHR, 0, s>>>(a);
  } else {
    if (gt) wgrad_bf16_gather<<<nb, NTHR, 0, s>>>(a);
    else wgrad_bf16<<<nb, NTHR, 0, s>>>(a);
  }
  return check_launch("wgrad");
}

}  // namespace moe
