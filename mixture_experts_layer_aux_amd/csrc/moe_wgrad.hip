// Weight gradients of the grouped experts with two workgroups per CU.
//
// The Ultimate MoE Training Handbook, §3.4 (the expert FFN): for each expert the
// gradients of its two projections, dW[g] = dY_g^T X_g over the expert's ragged block of
// reduction rows (its tokens).  Every non-empty expert owns a full grid of output tiles,
// and an expert's reduction is short (a few hundred rows, often fewer), so a tile spends
// about as long on its prologue (the first stages' load latency) and its epilogue (the
// tile's store) as on its reduction.  The 8-wave 256 x 256 kernel of moe_gemm_mfma.hip
// holds a CU alone (128 KB of LDS), so nothing hides those.  This kernel runs 256 x 128
// tiles with 4 waves and 72 KB of LDS, so two workgroups share a CU and one's prologue
// and epilogue overlap the other's reduction.
//
// Design (per workgroup: 256 threads = 4 waves in a 2 x 2 grid, one wave per SIMD):
//   * each wave a 128 x 64 sub-tile as 4 x 2 accumulators of v_mfma_f32_32x32x16_bf16;
//   * both operands are contiguous along the output (dY [rows][M], X [rows][N]) and go
//     from HBM into LDS by buffer_load ... lds, 32 reduction rows per stage, through a
//     ring of 3 stages: A as [32][256] (2 k-rows per 1 KB load), B as [32][128] (4 k-rows
//     per load), the 16-byte chunk index XORed by 4 (k & 3), read with the transposing
//     ds_read_b64_tr_b16;
//   * one barrier per stage: wait for this wave's part of stage it, barrier, issue stage
//     it+2 into the slot of stage it-1, read stage it's fragments (the second 16-deep
//     half while the first half's MFMAs run), MFMAs.  The other workgroup on the CU fills
//     the matrix cores while a wave waits;
//   * X read through a row gather (x_rows): the indices of stage s + 2 travel into LDS
//     with stage s (a 4-byte-per-lane load into a 4-slot ring), so they have landed when
//     stage s + 2 is issued;
//   * descriptor-bounded loads: rows past the group's end and indices past the source
//     read zeros, so the ragged tail needs no code;
//   * the epilogue stages the tile through the LDS (bf16 overwritten: one pass of the
//     rounded tile, 64 KB; otherwise two passes of 128 fp32 rows, 64 KB each) and stores
//     whole tile rows.
#include "moe_internal.h"

namespace moe {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int BM = 256, BN = 128, BK = 32, STAGES = 3, NTHR = 256;
constexpr int WAVES_N = 2, WTM = 128, WTN = 64, NI = WTM / 32, NJ = WTN / 32;
constexpr int A_ELEMS = BK * BM, B_ELEMS = BK * BN, STAGE_ELEMS = A_ELEMS + B_ELEMS;  // bf16 elements
constexpr int A_DMA = A_ELEMS / 512 / 4, B_DMA = B_ELEMS / 512 / 4;  // 1 KB loads per wave: 4 and 2
constexpr int NDMA = A_DMA + B_DMA;
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
  int beta;            // 1: add into C
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
template <int N>
__device__ __forceinline__ void wait_vm_const() {
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
  asm volatile("" ::: "memory");
}
// Waits until at most n (0..15) of this wave's vector memory operations are outstanding.
__device__ __forceinline__ void wait_vm(int n) {
  switch (n < 0 ? 0 : n) {
    case 0: wait_vm_const<0>(); break;
    case 1: wait_vm_const<1>(); break;
    case 2: wait_vm_const<2>(); break;
    case 3: wait_vm_const<3>(); break;
    case 4: wait_vm_const<4>(); break;
    case 5: wait_vm_const<5>(); break;
    case 6: wait_vm_const<6>(); break;
    case 7: wait_vm_const<7>(); break;
    case 8: wait_vm_const<8>(); break;
    case 9: wait_vm_const<9>(); break;
    case 10: wait_vm_const<10>(); break;
    case 11: wait_vm_const<11>(); break;
    case 12: wait_vm_const<12>(); break;
    case 13: wait_vm_const<13>(); break;
    case 14: wait_vm_const<14>(); break;
    default: wait_vm_const<15>(); break;
  }
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

template <bool OUT_F32, bool GATHER>
__device__ __forceinline__ void wgrad_body(const WgArgs& p) {
  // stage slots, then (GATHER) the ring of 4 slots of 64 gather indices
  __shared__ __attribute__((aligned(1024))) uint16_t lds[STAGES * STAGE_ELEMS + (GATHER ? 4 * 64 * 2 : 0)];
  int32_t(*tok_lds)[64] = reinterpret_cast<int32_t(*)[64]>(lds + STAGES * STAGE_ELEMS);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  // ---------------------------------------------------------------- tile
  // every group's nM x nN tiles are split into 8 equal runs, one per XCD (workgroup h runs
  // on XCD h % 8), each walked in bands of 4 row tiles, column by column
  constexpr int WG_BAND = 4;
  const int per = p.nM * p.nN;
  const int run = (per + 7) >> 3;
  const int h = blockIdx.x;
  const int q8 = h >> 3;
  const int grp = q8 / run;
  const int local = (h & 7) * run + (q8 - grp * run);
  if (grp >= p.G || local >= per) return;
  const int band = local / (WG_BAND * p.nN);
  const int rem = local - band * WG_BAND * p.nN;
  const int bh = min(WG_BAND, p.nM - band * WG_BAND);
  const int nt = rem / bh;
  const int mt = band * WG_BAND + (rem - nt * bh);
  const int row_begin = mt * BM;   // rows of dW (the M columns of dY)
  const int n0 = nt * BN;          // columns of dW
  const int k_begin = p.offsets ? p.offsets[grp] : 0;
  const int k_end = p.offsets ? p.offsets[grp + 1] : p.range_end;
  const int nk = k_end > k_begin ? (k_end - k_begin + BK - 1) / BK : 0;
  const int64_t cg = static_cast<int64_t>(grp) * p.c_gstride;

  if (nk == 0) {
    // a group without rows: exact zeros when overwriting, untouched when accumulating
    if (p.beta) return;
    constexpr int EB = OUT_F32 ? 4 : 2;
    constexpr int TPR = BN * EB / 16;   // threads per tile row (16 bytes each)
    constexpr int RPI = NTHR / TPR;
    const int col = n0 + (tid % TPR) * (16 / EB);
    if (col < p.N) {
      char* base = static_cast<char*>(p.C) + cg * EB;
      for (int r = tid / TPR; r < BM && row_begin + r < p.M; r += RPI)
        *reinterpret_cast<uint4*>(base + (static_cast<int64_t>(row_begin + r) * p.ldc + col) * EB) =
            make_uint4(0u, 0u, 0u, 0u);
    }
    return;
  }

  // ---------------------------------------------------------------- HBM -> LDS (DMA)
  // A: block b (1 KB) = k-rows 2b, 2b+1 of the stage, 256 columns (lane: row 2b + lane/32,
  // chunk lane%32); B: block b = k-rows 4b .. 4b+3, 128 columns (lane: row 4b + lane/16,
  // chunk lane%16).  LDS position p of a row holds chunk p ^ swm(k).
  int voffA[A_DMA], colB[B_DMA];
#pragma unroll
  for (int q = 0; q < A_DMA; ++q) {
    const int kr = (wave * A_DMA + q) * 2 + (lane >> 5);
    const int c = (lane & 31) ^ swm(kr);
    voffA[q] = kr * static_cast<int>(p.lda) * 2 + (row_begin + c * 8) * 2;
  }
  auto krB = [&](int q) { return (wave * B_DMA + q) * 4 + (lane >> 4); };
#pragma unroll
  for (int q = 0; q < B_DMA; ++q) colB[q] = (n0 + (((lane & 15) ^ swm(krB(q))) * 8)) * 2;

  auto stage_A_rsrc = [&](int st) {
    const int k0 = k_begin + st * BK;
    return make_rsrc(p.A + static_cast<int64_t>(k0) * p.lda, min(BK, k_end - k0) * static_cast<int>(p.lda) * 2);
  };
  // B byte offsets of stage st: consecutive rows, or the gathered source rows (src), a
  // row past the group's end or a negative index going past the descriptor
  auto voffB_of = [&](int st, int q, int src) {
    const int kr = krB(q);
    if constexpr (GATHER)
      return (k_begin + st * BK + kr < k_end && src >= 0) ? src * static_cast<int>(p.ldb) * 2 + colB[q] : kOob;
    else
      return kr * static_cast<int>(p.ldb) * 2 + colB[q];
  };
  auto stage_B_rsrc = [&](int st) {
    if constexpr (GATHER) return make_rsrc(p.B, p.gather_rows * static_cast<int>(p.ldb) * 2);
    const int k0 = k_begin + st * BK;
    return make_rsrc(p.B + static_cast<int64_t>(k0) * p.ldb, min(BK, k_end - k0) * static_cast<int>(p.ldb) * 2);
  };
  constexpr int D = STAGES - 1;
  // GATHER: the indices of stage st go into tok_lds[st & 3] (64 loaded, BK used)
  auto issue_tok = [&](int st) {
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.gather, p.gather_len * 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rg, (lds_void_t*)(&tok_lds[st & 3][0]), 4,
                                             (k_begin + st * BK + lane) * 4, 0, 0, 0);
  };
  // stage st (and, GATHER, the indices of stage st + D first) into slot st % STAGES
  auto issue_stage = [&](int st, const int (&src)[B_DMA]) {
    if constexpr (GATHER)
      if (st + D < nk) issue_tok(st + D);
    uint16_t* dst = lds + (st % STAGES) * STAGE_ELEMS;
    const __amdgpu_buffer_rsrc_t ra = stage_A_rsrc(st), rb = stage_B_rsrc(st);
#pragma unroll
    for (int q = 0; q < A_DMA; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)(dst + (wave * A_DMA + q) * 512), 16, voffA[q], 0, 0, 0);
#pragma unroll
    for (int q = 0; q < B_DMA; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_t*)(dst + A_ELEMS + (wave * B_DMA + q) * 512), 16,
                                               voffB_of(st, q, src[q]), 0, 0, 0);
  };
  // loads of one stage's group (its indices ride with it)
  auto group_loads = [&](int st) { return NDMA + ((GATHER && st + D < nk) ? 1 : 0); };

  // ---------------------------------------------------------------- LDS -> fragments
  // 32-row block at rb0 of a [32][W] tile, substep ks: lane l gets column rb0 + 16 (g & 1)
  // + 4 (j & 3) .. (g = l / 16, j = l % 16) at k = 16 ks + 8 (g / 2) + 4 hh + j / 4
  auto frag = [&](const uint16_t* t, int W, int rb0, int ks) -> bf16x8_t {
    const int j = lane & 15, g = lane >> 4;
    const int col = rb0 + 16 * (g & 1) + 4 * (j & 3);
    i16x4_t v[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int kr = ks * 16 + 8 * (g >> 1) + 4 * hh + (j >> 2);
      v[hh] = lds_read_tr((lds_i16x4_t*)(t + kr * W + (((col >> 3) ^ swm(kr)) << 3) + (col & 7)));
    }
    const i16x8_t w = {v[0][0], v[0][1], v[0][2], v[0][3], v[1][0], v[1][1], v[1][2], v[1][3]};
    return __builtin_bit_cast(bf16x8_t, w);
  };

  f32x16_t acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // ---------------------------------------------------------------- main loop
  // prologue: stages 0 .. D-1 (their gather indices straight from memory)
  {
    int src0[D][B_DMA];
#pragma unroll
    for (int st = 0; st < D; ++st)
#pragma unroll
      for (int q = 0; q < B_DMA; ++q) {
        const int row = k_begin + st * BK + krB(q);
        src0[st][q] = GATHER && row < k_end && row < p.gather_len ? p.gather[row] : -1;
      }
#pragma unroll
    for (int st = 0; st < D; ++st)
      if (st < nk) issue_stage(st, src0[st]);
  }
  for (int it = 0; it < nk; ++it) {
    // this wave's part of stage it landed: the loads after it are stage it+1's group
    wait_vm(it + 1 < nk ? group_loads(it + 1) : 0);
    block_barrier();  // every part of stage it is in LDS; every wave is done with stage it-1
    const uint16_t* As = lds + (it % STAGES) * STAGE_ELEMS;
    const uint16_t* Bs = As + A_ELEMS;
    bf16x8_t fa[2][NI], fb[2][NJ];
    auto load_frags = [&](int ks, int buf) {
#pragma unroll
      for (int i = 0; i < NI; ++i) fa[buf][i] = frag(As, BM, wm * WTM + i * 32, ks);
#pragma unroll
      for (int j = 0; j < NJ; ++j) fb[buf][j] = frag(Bs, BN, wn * WTN + j * 32, ks);
    };
    load_frags(0, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (it + D < nk) {
      // into the slot of stage it-1; its indices landed with stage it
      int src[B_DMA];
#pragma unroll
      for (int q = 0; q < B_DMA; ++q) src[q] = GATHER ? tok_lds[(it + D) & 3][krB(q)] : 0;
      issue_stage(it + D, src);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      if (ks + 1 < BK / 16) load_frags(ks + 1, (ks + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks & 1][j], fa[ks & 1][i], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---------------------------------------------------------------- epilogue
  // acc[i][j][4u + c] is tile row wm*WTM + i*32 + lane%32, column wn*WTN + j*32 + 8u +
  // 4 (lane/32) + c
  const int cbase = 4 * (lane >> 5);
  if (!OUT_F32 && !p.beta) {
    // bf16, overwritten: rounded in registers, the whole 256 x 128 tile in LDS in one pass
    // (8-byte unit u of row r at r * 32 + (u ^ (r & 31))), then two rows per store
    // instruction (32 lanes x 8 bytes each)
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
          U2[r * 32 + (c ^ (r & 31))] = make_uint2(pack_bf16x2(acc[i][j][4 * u], acc[i][j][4 * u + 1]),
                                                   pack_bf16x2(acc[i][j][4 * u + 2], acc[i][j][4 * u + 3]));
        }
    }
    lds_barrier();
    uint16_t* C = static_cast<uint16_t*>(p.C) + cg;
    const int l = lane & 31, col = n0 + 4 * l;
    // every LDS read first (one latency), then the stores
    constexpr int RR = BM / 4 / 2;
    uint2 v[RR];
#pragma unroll
    for (int rr = 0; rr < RR; ++rr) {
      const int r = wave * (BM / 4) + rr * 2 + (lane >> 5);
      v[rr] = U2[r * 32 + (l ^ (r & 31))];
    }
#pragma unroll
    for (int rr = 0; rr < RR; ++rr) {
      const int row = row_begin + wave * (BM / 4) + rr * 2 + (lane >> 5);
      if (row < p.M && col < p.N) *reinterpret_cast<uint2*>(C + static_cast<int64_t>(row) * p.ldc + col) = v[rr];
    }
    return;
  }
  // fp32 out, or accumulating: two passes of 128 tile rows (16-byte chunk c of pass row lr
  // at lr * 32 + (c ^ (lr & 31))); pass h holds the accumulator blocks i = 2h, 2h+1 of
  // every wave: pass row lr is tile row (lr / 64) * WTM + 64 h + lr % 64
  float4* L4 = reinterpret_cast<float4*>(lds);
  static_assert(STAGES * STAGE_ELEMS * 2 >= 128 * BN * 4, "an epilogue pass needs 64 KB of LDS");
#pragma unroll
  for (int hp = 0; hp < 2; ++hp) {
    block_barrier();  // the previous use of the LDS (main loop or the previous pass) is over
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int i = 2 * hp + ii;
      const int lr = wm * 64 + ii * 32 + (lane & 31);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c = (wn * WTN + j * 32 + 8 * u + cbase) >> 2;
          L4[lr * 32 + (c ^ (lr & 31))] =
              make_float4(acc[i][j][4 * u], acc[i][j][4 * u + 1], acc[i][j][4 * u + 2], acc[i][j][4 * u + 3]);
        }
    }
    lds_barrier();
    const int l = lane & 31, col = n0 + 4 * l;
    constexpr int RR = 128 / 4 / 2;
    float4 vv[RR];
#pragma unroll
    for (int rr = 0; rr < RR; ++rr) {
      const int lr = wave * 32 + rr * 2 + (lane >> 5);
      vv[rr] = L4[lr * 32 + (l ^ (lr & 31))];
    }
#pragma unroll
    for (int rr = 0; rr < RR; ++rr) {
      const int lr = wave * 32 + rr * 2 + (lane >> 5);
      const int row = row_begin + (lr >> 6) * WTM + hp * 64 + (lr & 63);
      if (row >= p.M || col >= p.N) continue;
      const float4 v = vv[rr];
      if constexpr (OUT_F32) {
        float4* dst = reinterpret_cast<float4*>(static_cast<float*>(p.C) + cg + static_cast<int64_t>(row) * p.ldc + col);
        if (p.beta) {
          const float4 o = *dst;
          *dst = make_float4(o.x + v.x, o.y + v.y, o.z + v.z, o.w + v.w);
        } else {
          *dst = v;
        }
      } else {
        uint2* dst = reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.C) + cg + static_cast<int64_t>(row) * p.ldc + col);
        float4 w = v;
        const uint2 o = *dst;   // accumulating (the overwriting bf16 case returned above)
        w.x += __uint_as_float(o.x << 16);
        w.y += __uint_as_float(o.x & 0xFFFF0000u);
        w.z += __uint_as_float(o.y << 16);
        w.w += __uint_as_float(o.y & 0xFFFF0000u);
        *dst = make_uint2(pack_bf16x2(w.x, w.y), pack_bf16x2(w.z, w.w));
      }
    }
  }
}

// one plain kernel per output type and row source (kernel templates whose bodies hold
// lambdas lose their host launch stubs)
__global__ __launch_bounds__(NTHR, 2) void wgrad_bf16(const WgArgs p) { wgrad_body<false, false>(p); }
__global__ __launch_bounds__(NTHR, 2) void wgrad_bf16_gather(const WgArgs p) { wgrad_body<false, true>(p); }
__global__ __launch_bounds__(NTHR, 2) void wgrad_f32(const WgArgs p) { wgrad_body<true, false>(p); }
__global__ __launch_bounds__(NTHR, 2) void wgrad_f32_gather(const WgArgs p) { wgrad_body<true, true>(p); }

}  // namespace

bool wgrad2_supported(const GemmDesc& g) {
  return g.ragged == RAGGED_K && g.epi == EPI_STORE && g.a_major == MN_MAJOR && g.b_major == MN_MAJOR &&
         g.a_type == MOE_BF16 && g.b_type == MOE_BF16 && g.kchunk == 0 && g.M % 8 == 0 && g.N % 8 == 0 &&
         g.lda % 8 == 0 && g.ldb % 8 == 0 && g.ldc % 8 == 0 && g.c_gstride % 8 == 0;
}

moe_status_t launch_wgrad2(const GemmDesc& g, hipStream_t s) {
  if (!wgrad2_supported(g)) return fail(MOE_ERR_UNSUPPORTED, "wgrad: unsupported operand combination");
  const int groups = g.offsets ? g.G : 1;
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
  a.nM = static_cast<int>(ceil_div(g.M, BM));
  a.nN = static_cast<int>(ceil_div(g.N, BN));
  if (g.gather) {
    if (static_cast<int64_t>(g.gather_rows) * g.ldb * 2 > kOob - 4096)
      return fail(MOE_ERR_UNSUPPORTED, "wgrad: gathered operand above 2 GB");
    a.gather = g.gather;
    a.gather_rows = g.gather_rows;
    a.gather_len = g.range_end;
  }
  const int64_t grid = 8 * static_cast<int64_t>(groups) * ceil_div(static_cast<int64_t>(a.nM) * a.nN, 8);
  if (grid == 0) return MOE_OK;
  const bool f32 = g.c_type == MOE_F32;
  const unsigned nb = static_cast<unsigned>(grid);
  if (f32 && g.gather) wgrad_f32_gather<<<nb, NTHR, 0, s>>>(a);
  else if (f32) wgrad_f32<<<nb, NTHR, 0, s>>>(a);
  else if (g.gather) wgrad_bf16_gather<<<nb, NTHR, 0, s>>>(a);
  else wgrad_bf16<<<nb, NTHR, 0, s>>>(a);
  return check_launch("wgrad");
}

}  // namespace moe
