// Internal launcher interface between the C-ABI layer and the kernel translation units.
#pragma once

#include "moe_common.h"

namespace moe {

inline int act_bytes(const moe_config_t& c) { return c.act_dtype == MOE_BF16 ? 2 : 4; }

// ---------------------------------------------------------------- router
int router_epl(int E);
int64_t router_num_blocks(int T);  // == permute_num_chunks(T): both use 64-token chunks
// Router scratch, carved from the caller's workspace.
struct RouterWs {
  int32_t* cnt_part;       // [nblk, E] block histograms (== the permute's chunk histograms)
  float* prob_part;        // [nblk, E] block sums of the aux probabilities
  float* z_part;           // [nblk]    block sums of logsumexp^2
  float* pnorm;            // [T, 2]    per-token (m, 1/Z) of the aux probabilities
  int32_t* seq_cnt_part;   // [B, ceil(S/64), E]
  float* seq_prob_part;    // [B, ceil(S/64), E]
  int32_t* done;           // one counter: blocks of the router's finaliser that are done
};
// elements of each per-sequence partial (0 when the sequence-wise loss is off)
size_t router_seq_part_elems(const moe_config_t& c);
moe_status_t launch_router_topk(const moe_config_t& c, const float* logits, const float* expert_bias,
                                int32_t* idx, float* w, int32_t* counts, float* prob_sum, float* prob_scratch,
                                float* stats, int32_t* seq_counts, const RouterWs& rw, hipStream_t s);
moe_status_t launch_router_bwd(const moe_config_t& c, const float* logits, const int32_t* idx, const float* w,
                               const float* dw, const int32_t* counts, const int32_t* seq_counts, float daux,
                               float* dlogits, hipStream_t s);
moe_status_t launch_bias_update(const int32_t* counts, int E, float rate, int centered, float* bias, hipStream_t s);
// quantile balancing (moe_quantile.hip); ws: quantile_ws_bytes(E) bytes
size_t quantile_ws_bytes(int E);
moe_status_t launch_router_quantile(const moe_config_t& c, const float* scores, const float* beta, int32_t* idx,
                                    float* alpha, float* beta_local, void* ws, hipStream_t s);
moe_status_t launch_quantile_update(const float* beta_local, int E, float ema, float* beta, hipStream_t s);

// ---------------------------------------------------------------- permute / combine
int64_t permute_num_chunks(int T);
// elem_bytes: bytes per element of x (0: the activation dtype's; 1 for e4m3 rows)
moe_status_t launch_permute(const moe_config_t& c, const void* x, const int32_t* idx, int32_t* offsets,
                            int32_t* row_of, int32_t* token_of, void* x_perm, int32_t* blk_hist,
                            int32_t* blk_base, int32_t* counts_ws, bool hist_ready, hipStream_t s,
                            int elem_bytes = 0);
// y = sum_j w Y_perm[row] + gs Y_s  (all fp32; gs NULL means 1)
moe_status_t launch_combine(const moe_config_t& c, const float* Y, const int32_t* row_of, const float* w,
                            const float* Y_s, const float* gs, float* y, hipStream_t s);
// dx = sum_j dX_perm[row] + dx_s + dx_r + dl_s Wsg  (all fp32; NULL terms skipped)
moe_status_t launch_unpermute_reduce(const moe_config_t& c, const float* dX, const int32_t* row_of,
                                     const float* dx_s, const float* dx_r, const float* dl_s, const float* Wsg,
                                     float* dx, hipStream_t s);
moe_status_t launch_combine_bwd(const moe_config_t& c, const float* dy, const float* Y, const int32_t* row_of,
                                const float* w, void* dY, float* dw, void* dY_s, const float* gs, const float* Ys,
                                float* dl_s, hipStream_t s);
// the shared expert's sigmoid gate: gs = sigma(x Wsg); dWsg = x^T dl_s (part: scratch)
size_t shared_gate_part_bytes(const moe_config_t& c);
moe_status_t launch_shared_gate(const moe_config_t& c, const void* x, const float* Wsg, float* gs, hipStream_t s);
moe_status_t launch_shared_gate_bwd(const moe_config_t& c, const void* x, const float* dl_s, float* dWsg,
                                    float* part, hipStream_t s, int beta = 0);

#define MOE_TRY_INTERNAL(x)      \
  do {                           \
    const moe_status_t _st = (x); \
    if (_st != MOE_OK) return _st; \
  } while (0)

// ---------------------------------------------------------------- router GEMMs (fp32)
// On the bf16 matrix cores through exact bf16 splits of the fp32 operand when the
// activations are bf16 and E % 16 == 0; the fp32 FMA GEMM otherwise.
bool gate_on_mfma(const moe_config_t& c);
size_t gate_fwd_ws_bytes(const moe_config_t& c);
size_t gate_bwd_ws_bytes(const moe_config_t& c);
moe_status_t launch_gate_fwd_mfma(const moe_config_t& c, const void* x, const float* Wg, const float* bg,
                                  float* logits, void* ws, hipStream_t s);
moe_status_t launch_gate_bwd_mfma(const moe_config_t& c, const void* x, const float* Wg, const float* dlogits,
                                  float* dWg, float* dbg, float* dx_r, void* ws, hipStream_t s, int beta = 0);
// column sums in a fixed order; part: ceil(rows / 256) * cols floats of scratch
moe_status_t launch_colsum_ws(const float* X, int rows, int cols, float* out, float* part, hipStream_t s,
                              int beta = 0);

// ---------------------------------------------------------------- fp8 experts
moe_status_t launch_quantize_fp8(int src_dtype, const void* src, int64_t rows, int cols, int block_rows, uint8_t* q,
                                 float* scale, hipStream_t s);
moe_status_t launch_gather_scales(const float* xs, const int32_t* token_of, int64_t A, int nb, float* out,
                                  hipStream_t s);
size_t fp8_schedule_bytes(int E, int64_t rows);   // rows: the upper bound of the grouped rows
// swiglu: fc1 of width N = 2F, Act (fp32) -> C [rows, F], H (optional); else C [rows, N].
// bm: tile rows, 256 (256 x 128 tiles) or 128 (128 x 256); fp8_tile_rows picks it.  With
// bm 128, fc1 can write Act as e4m3 codes act_q [rows, F] and scales act_scale [rows, F/128]
// (the rule of launch_quantize_fp8 with block_rows 1) in place of C.
int fp8_tile_rows(int64_t rows_upper, int G, int N, int F, bool swiglu);
moe_status_t launch_gemm_fp8(bool swiglu, const uint8_t* A, const float* A_scale, const uint8_t* B,
                             const float* B_scale, float* C, float* H, const int32_t* offsets, int G, int64_t rows_upper,
                             int N, int K, int F, int32_t* sched, hipStream_t s, Glu glu, const int32_t* gather,
                             int gather_rows, int bm, uint8_t* act_q = nullptr, float* act_scale = nullptr);

// ---------------------------------------------------------------- GEMMs
// Storage of an operand: K_MAJOR = [rows][K] (K contiguous), MN_MAJOR = [K][rows].
enum Major { K_MAJOR = 0, MN_MAJOR = 1 };
// Grouping: RAGGED_M = group g owns rows [off[g], off[g+1]) of A and C, and B + g*b_gstride;
//           RAGGED_K = group g owns K rows [off[g], off[g+1]) of A and B, and C + g*c_gstride.
// offsets == nullptr means one group spanning [0, range_end).
enum Ragged { RAGGED_M = 0, RAGGED_K = 1 };
enum Epi { EPI_STORE = 0, EPI_SWIGLU_FWD = 1, EPI_SWIGLU_BWD = 2, EPI_STORE_BIAS = 3 };

struct GemmDesc {
  int a_major, b_major, ragged, epi;
  int a_type, b_type, c_type;  // moe_dtype_t
  int M, N, K;                  // the non-ragged extents (M or K per group when ragged)
  const void* A;
  int64_t lda, a_gstride;
  const void* B;
  int64_t ldb, b_gstride;
  void* C;
  int64_t ldc, c_gstride;
  void* C2;                     // EPI_SWIGLU_FWD: Act out [rows][F]
  int64_t ldc2;
  const void* Hin;              // EPI_SWIGLU_BWD: saved H [rows][2F], fp32
  int64_t ldh;
  const float* bias;            // EPI_STORE_BIAS: [N]
  int F;                        // SwiGLU: offset of the up half (columns of H / rows of W13)
  Glu glu;                      // SwiGLU epilogues: the gated activation (zero: plain SwiGLU)
  int beta;                     // EPI_STORE: 1 = add into C (accumulate), 0 = overwrite
  int kchunk;                   // RAGGED_K without offsets: group g owns reduction rows
                                // [g kchunk, min(range_end, (g + 1) kchunk)) (0: one group)
  const int32_t* offsets;
  int G;
  int range_end;
  int64_t rows_upper;           // ragged M: upper bound of sum of rows (for grid sizing)
  // Row gather of the permuted activation (the grouped rows are read from their token rows
  // instead of a permuted copy): ragged M with a K-contiguous A reads row r of A from row
  // gather[r] of A; ragged K with a row-contiguous B reads reduction row k of B from row
  // gather[k] of B.  gather_rows: rows of the gathered operand (bounds every gathered read).
  const int32_t* gather;
  int gather_rows;
  // Skew splitting of reduction-ragged weight gradients (device tables of a split plan):
  // skip[g] != 0: group g is left alone (its chunks are reduced elsewhere); pairs: group g
  // reduces rows [pairs[2g], pairs[2g + 1]) instead of the offsets' range; gcount: the
  // number of groups that exist (groups g >= *gcount do nothing).
  const int32_t* skip;
  const int32_t* pairs;
  const int32_t* gcount;
};

// fp32-accumulating FMA GEMM for fp32 (and mixed fp32/bf16) operands; SwiGLU epilogues are
// separate elementwise kernels on this path.
moe_status_t launch_gemm_fma(const GemmDesc& g, hipStream_t s);
moe_status_t launch_swiglu_fwd_elementwise(Glu glu, const float* H, float* Act, int64_t rows, int F, hipStream_t s);
moe_status_t launch_swiglu_bwd_elementwise(Glu glu, const float* H, const float* dAct, float* dH, int64_t rows, int F,
                                           hipStream_t s);

// bf16 MFMA grouped GEMM (gfx950 v_mfma_f32_32x32x16_bf16), fused epilogues.
size_t mfma_schedule_bytes(int G, int64_t rows);  // rows: the upper bound of the grouped rows
moe_status_t launch_gemm_mfma(const GemmDesc& g, int32_t* sched_ws, hipStream_t s);
// Reduction-ragged bf16 weight gradients (both operands row-contiguous, no split-K) on
// 256 x 128 tiles of 4 waves, two workgroups per CU (moe_wgrad.hip).
bool wgrad2_supported(const GemmDesc& g);
moe_status_t launch_wgrad2(const GemmDesc& g, hipStream_t s);
// Split-K of a one-group weight gradient dW [M, N] over `rows` reduction rows: the row
// chunk (a multiple of 64) and the number of chunks, 1 when the output alone has enough
// tiles to fill the chip (then kchunk = rows).  Partials: chunks * M * N fp32.
struct WgradSplit { int chunks; int kchunk; };
// Skew splitting of a grouped weight gradient dW[g] [M, N] (g < G) over ragged reduction
// rows (`rows` in all, at most `max_group_rows` in one group), `tiles` output tiles per
// group on a kernel that holds `slots` tiles at once.  A group with more rows than `chunk`
// is cut into row chunks of `chunk` rows; each chunk is an fp32 partial of its own, and
// the partials are summed in chunk order.  chunk 0: no group can exceed the balance point,
// nothing is split.
struct SkewPlan {
  int chunk;      // rows per chunk (0: no split)
  int max_vg;     // capacity: chunks of all split groups together
  int max_split;  // capacity: split groups
  size_t plan_bytes, partial_bytes;
};
SkewPlan skew_plan(int G, int64_t rows, int64_t max_group_rows, int M, int N, int tiles, int slots);
// Builds the plan's device tables (one block): skip [G], gcount, nsplit, pairs [2 max_vg],
// split_e / split_first / split_n [max_split] in `plan` (plan_bytes).
moe_status_t launch_skew_plan(const int32_t* offsets, int G, const SkewPlan& sp, int32_t* plan, hipStream_t s);
// Device table views of a plan buffer.
struct SkewTables {
  const int32_t *skip, *gcount, *nsplit, *pairs, *split_e, *split_first, *split_n;
};
SkewTables skew_tables(const int32_t* plan, int G, const SkewPlan& sp);
// dW[split_e[j]] = sum_{c < split_n[j]} part[split_first[j] + c] (+ dW when beta), in
// the weight-gradient dtype (bf16: rounded once), for j < *nsplit.
moe_status_t launch_skew_reduce(const float* part, const SkewTables& t, const SkewPlan& sp, int64_t elems,
                                void* dW, int64_t c_gstride, int out_dtype, int beta, hipStream_t s);
WgradSplit wgrad_split(int M, int N, int64_t rows);
size_t wgrad_split_bytes(int M, int N, int64_t rows);
// out = sum of the `splits` fp32 partials [splits, elems] in order (+ out when beta), in the
// weight-gradient dtype (bf16: rounded once).
moe_status_t launch_splitk_reduce(const float* part, int splits, int64_t elems, void* out, int out_dtype, int beta,
                                  hipStream_t s);

}  // namespace moe
