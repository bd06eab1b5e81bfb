// The C ABI of libmoe: argument checks, workspace layout and the order of launches.
// Every entry point validates all of its arguments on the host before it enqueues
// anything, allocates nothing, and never synchronises the host.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>

#include "moe_internal.h"

namespace moe {

namespace {
thread_local char g_err[512] = "";
}

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

moe_status_t fail(moe_status_t s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

moe_status_t check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Workspace carving, shared by moe_workspace_size and the calls.
struct FwdWs {
  int32_t* cnt_part;   // [nchunk, E] router chunk histograms == permute chunk histograms
  float* prob_part;    // [nchunk, E]
  float* z_part;       // [nchunk]
  int32_t* done;       // the router finaliser's block counter
  float* pnorm;        // [T, 2] (sequence-wise loss only)
  int32_t* seq_cnt_part;  // router_seq_part_elems
  float* seq_prob_part;   // router_seq_part_elems
  void* quantile;      // quantile_ws_bytes(E): histograms and radix-select state
  int32_t* blk_base;   // [nchunk, E]
  int32_t* counts;     // [E]
  float* prob_sum;     // [E]
  int32_t* sched;      // tile schedule of the grouped GEMMs: [E + 1] prefix + owner table
  uint8_t* xq;         // fp8 experts: [T, d] e4m3 codes of x
  float* xs;           // fp8 experts: [T, d/128] their scales
  float* act32;        // fp8 experts: [A, F] fp32 SwiGLU output before quantisation
  void* gate;          // router GEMM scratch (gate_fwd_ws_bytes)
  size_t bytes;
};

FwdWs carve_fwd(const moe_config_t& c, void* base) {
  char* p = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t n) {
    char* q = p ? p + off : nullptr;
    off += align_up(n);
    return q;
  };
  const size_t nch = static_cast<size_t>(permute_num_chunks(c.T));
  FwdWs w;
  w.cnt_part = reinterpret_cast<int32_t*>(take(nch * c.E * 4));
  w.prob_part = reinterpret_cast<float*>(take(nch * c.E * 4));
  w.z_part = reinterpret_cast<float*>(take(nch * 4));
  w.done = reinterpret_cast<int32_t*>(take(4));
  const size_t nseq = router_seq_part_elems(c);
  w.pnorm = nseq ? reinterpret_cast<float*>(take(static_cast<size_t>(c.T) * 8)) : nullptr;
  w.seq_cnt_part = nseq ? reinterpret_cast<int32_t*>(take(nseq * 4)) : nullptr;
  w.seq_prob_part = nseq ? reinterpret_cast<float*>(take(nseq * 4)) : nullptr;
  w.quantile = take(quantile_ws_bytes(c.E));
  w.blk_base = reinterpret_cast<int32_t*>(take(nch * c.E * 4));
  w.counts = reinterpret_cast<int32_t*>(take(static_cast<size_t>(c.E) * 4));
  w.prob_sum = reinterpret_cast<float*>(take(static_cast<size_t>(c.E) * 4));
  const int64_t rows = static_cast<int64_t>(c.T) * c.k;
  w.sched = reinterpret_cast<int32_t*>(take(std::max(mfma_schedule_bytes(c.E, rows), fp8_schedule_bytes(c.E, rows))));
  w.xq = nullptr;
  w.xs = w.act32 = nullptr;
  if (c.w_dtype == MOE_FP8_E4M3) {
    const size_t T = c.T, A = T * c.k;
    w.xq = reinterpret_cast<uint8_t*>(take(T * c.d));
    w.xs = reinterpret_cast<float*>(take(T * (c.d / 128) * 4));
    w.act32 = reinterpret_cast<float*>(take(A * c.F * 4));
  }
  w.gate = take(gate_fwd_ws_bytes(c));
  w.bytes = off;
  return w;
}

struct BwdWs {
  void* dY;        // [A, d] act: dY_perm
  float* dX;       // [A, d] fp32: dX_perm (its own buffer, so the fc2 weight gradient can still
                   // read dY_perm while the fc1 data gradient writes dX_perm)
  void* dH;        // [A, 2F] act
  float* dw;       // [T, k]
  float* dlogits;  // [T, E]
  float* dx_r;     // [T, d]
  void* dH_s;      // [T, 2Fs] act
  void* dx_s;      // [T, d] fp32
  void* dY_s;      // [T, d] act: the shared expert's upstream gradient
  float* dl_s;     // [T]: the shared gate's logit gradient
  float* sg_part;  // shared_gate_part_bytes: partial sums of its weight gradient
  float* dact;     // fp32 path: [max(A, T), max(F, Fs)]
  float* wsplit;   // bf16 shared expert: split-K partials of its weight gradients (or NULL)
  int32_t* sched;  // tile schedule of the grouped GEMMs: [E + 1] prefix + owner table
  void* gate;      // router GEMM scratch (gate_bwd_ws_bytes)
  void* skew;      // skew split of the routed weight gradients: plan tables + fp32 partials
  size_t skew_bytes;
  size_t bytes;
};

// Workspace of the skew split of a routed weight gradient dW [M, N] (bf16 layers): the
// plan's tables and its fp32 partials, 0 when no expert can reach the split point.  The
// plan does not depend on which weight-gradient kernel runs: that kernel's tiles and
// slots change by the same factor.
size_t routed_skew_bytes(const moe_config_t& c, int M, int N) {
  const int64_t A = static_cast<int64_t>(c.T) * c.k;
  const int tiles = static_cast<int>(ceil_div(M, 256) * ceil_div(N, 256));
  const SkewPlan sp = skew_plan(c.E, A, c.T, M, N, tiles, 256);
  return sp.chunk ? align_up(sp.plan_bytes) + sp.partial_bytes : 0;
}
size_t skew_ws_bytes(const moe_config_t& c) {
  if (c.act_dtype != MOE_BF16) return 0;
  return std::max(routed_skew_bytes(c, c.d, c.F), routed_skew_bytes(c, 2 * c.F, c.d));
}

BwdWs carve_bwd(const moe_config_t& c, void* base) {
  char* p = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t n) {
    char* q = p ? p + off : nullptr;
    off += align_up(n);
    return q;
  };
  const size_t A = static_cast<size_t>(c.T) * c.k, T = static_cast<size_t>(c.T), eb = act_bytes(c);
  BwdWs w;
  w.dY = take(A * c.d * eb);
  w.dX = reinterpret_cast<float*>(take(A * c.d * 4));
  w.dH = take(A * 2 * c.F * eb);
  w.dw = reinterpret_cast<float*>(take(A * 4));
  w.dlogits = reinterpret_cast<float*>(take(T * c.E * 4));
  w.dx_r = reinterpret_cast<float*>(take(T * c.d * 4));
  w.dH_s = c.Fs ? take(T * 2 * c.Fs * eb) : nullptr;
  w.dx_s = c.Fs ? take(T * c.d * 4) : nullptr;
  w.dY_s = c.Fs ? take(T * c.d * eb) : nullptr;
  w.dl_s = c.shared_gate ? reinterpret_cast<float*>(take(T * 4)) : nullptr;
  w.sg_part = c.shared_gate ? reinterpret_cast<float*>(take(shared_gate_part_bytes(c))) : nullptr;
  w.dact = c.act_dtype == MOE_F32 ? reinterpret_cast<float*>(take(std::max(A, T) * std::max(c.F, c.Fs) * 4)) : nullptr;
  const size_t split = c.Fs && c.act_dtype == MOE_BF16
                           ? std::max(wgrad_split_bytes(c.d, c.Fs, c.T), wgrad_split_bytes(2 * c.Fs, c.d, c.T))
                           : 0;
  w.wsplit = split ? reinterpret_cast<float*>(take(split)) : nullptr;
  w.sched = reinterpret_cast<int32_t*>(take(mfma_schedule_bytes(c.E, A)));
  w.gate = take(gate_bwd_ws_bytes(c));
  w.skew_bytes = skew_ws_bytes(c);
  w.skew = w.skew_bytes ? take(w.skew_bytes) : nullptr;
  w.bytes = off;
  return w;
}

RouterWs router_ws(const FwdWs& f) {
  RouterWs r;
  r.cnt_part = f.cnt_part;
  r.prob_part = f.prob_part;
  r.z_part = f.z_part;
  r.done = f.done;
  r.pnorm = f.pnorm;
  r.seq_cnt_part = f.seq_cnt_part;
  r.seq_prob_part = f.seq_prob_part;
  return r;
}

// The router's own scratch (its block partials and, for the sequence-wise loss, the
// per-token normalisers and per-sequence partials) plus a prob_sum buffer for callers that
// pass none: the layout of moe_router_topk_noalloc's static scratch.
struct RouterScratch {
  RouterWs rw;
  float* prob_sum;  // [E]
  size_t bytes;
};

RouterScratch carve_router(const moe_config_t& c, void* base) {
  char* p = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t n) {
    char* q = p ? p + off : nullptr;
    off += align_up(n);
    return q;
  };
  const size_t nblk = static_cast<size_t>(router_num_blocks(c.T));
  RouterScratch r{};
  r.rw.cnt_part = reinterpret_cast<int32_t*>(take(nblk * c.E * 4));
  r.rw.prob_part = reinterpret_cast<float*>(take(nblk * c.E * 4));
  r.rw.z_part = reinterpret_cast<float*>(take(nblk * 4));
  r.rw.done = reinterpret_cast<int32_t*>(take(4));
  const size_t nseq = router_seq_part_elems(c);
  r.rw.pnorm = nseq ? reinterpret_cast<float*>(take(static_cast<size_t>(c.T) * 8)) : nullptr;
  r.rw.seq_cnt_part = nseq ? reinterpret_cast<int32_t*>(take(nseq * 4)) : nullptr;
  r.rw.seq_prob_part = nseq ? reinterpret_cast<float*>(take(nseq * 4)) : nullptr;
  r.prob_sum = reinterpret_cast<float*>(take(static_cast<size_t>(c.E) * 4));
  r.bytes = off;
  return r;
}

moe_status_t validate(const moe_config_t* c) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "config is NULL");
  if (c->T < 1 || c->d < 1 || c->E < 1 || c->k < 1 || c->F < 1 || c->Fs < 0)
    return fail(MOE_ERR_INVALID_ARG, "sizes must be positive (T=%d d=%d E=%d k=%d F=%d Fs=%d)", c->T, c->d, c->E,
                c->k, c->F, c->Fs);
  if (c->k > c->E) return fail(MOE_ERR_INVALID_ARG, "k=%d exceeds E=%d", c->k, c->E);
  if (c->k > 32) return fail(MOE_ERR_UNSUPPORTED, "k=%d exceeds 32", c->k);
  if (c->E > 2048) return fail(MOE_ERR_UNSUPPORTED, "E=%d exceeds 2048", c->E);
  if (static_cast<int64_t>(c->T) * c->k >= (int64_t{1} << 31)) return fail(MOE_ERR_INVALID_ARG, "T*k >= 2^31");
  if (c->score != MOE_SOFTMAX && c->score != MOE_SIGMOID && c->score != MOE_SQRTSOFTPLUS)
    return fail(MOE_ERR_INVALID_ARG, "unknown score function");
  if (c->pre_softmax != 0 && c->pre_softmax != 1) return fail(MOE_ERR_INVALID_ARG, "pre_softmax must be 0 or 1");
  if (c->pre_softmax && c->score != MOE_SOFTMAX)
    return fail(MOE_ERR_UNSUPPORTED, "pre-softmax top-k is a softmax setting");
  if (c->score == MOE_SOFTMAX && c->k == 1 && !c->pre_softmax)
    return fail(MOE_ERR_UNSUPPORTED, "softmax over one selected logit has no gradient; top-1 needs pre-softmax");
  if (!(c->aux_coeff >= 0.0f && c->aux_coeff < INFINITY) || !(c->z_coeff >= 0.0f && c->z_coeff < INFINITY) ||
      !(c->seq_aux_coeff >= 0.0f && c->seq_aux_coeff < INFINITY))
    return fail(MOE_ERR_INVALID_ARG, "loss coefficients must be finite and >= 0");
  if (c->shared_gate != 0 && c->shared_gate != 1) return fail(MOE_ERR_INVALID_ARG, "shared_gate must be 0 or 1");
  if (c->shared_gate && c->Fs == 0) return fail(MOE_ERR_INVALID_ARG, "shared_gate needs a shared expert (Fs > 0)");
  if (c->num_groups != 0) {
    if (c->num_groups < 1 || c->num_groups > 64 || c->E % c->num_groups)
      return fail(MOE_ERR_INVALID_ARG, "num_groups=%d must be in [1, 64] and divide E=%d", c->num_groups, c->E);
    const int n = c->E / c->num_groups;
    if (c->group_topk < 1 || c->group_topk > c->num_groups || c->group_topk > c->k || c->k / c->group_topk > n ||
        c->group_topk * n < c->k)
      return fail(MOE_ERR_INVALID_ARG, "group_topk=%d does not fit k=%d in groups of %d experts", c->group_topk, c->k,
                  n);
  } else if (c->group_topk != 0) {
    return fail(MOE_ERR_INVALID_ARG, "group_topk without num_groups");
  }
  if (c->glu_kind != MOE_GLU_SWIGLU && c->glu_kind != MOE_GLU_CLAMP && c->glu_kind != MOE_GLU_SITU)
    return fail(MOE_ERR_INVALID_ARG, "unknown gated activation");
  if (c->glu_kind != MOE_GLU_SWIGLU && !(c->glu_c > 0.0f && c->glu_c < INFINITY))
    return fail(MOE_ERR_INVALID_ARG, "the activation bound glu_c must be finite and > 0");
  if (c->glu_kind == MOE_GLU_SITU && !(c->glu_c_linear >= 0.0f && c->glu_c_linear < INFINITY))
    return fail(MOE_ERR_INVALID_ARG, "glu_c_linear must be finite and >= 0");
  if (c->seq_aux_coeff != 0.0f && (c->seq_len < 1 || c->T % c->seq_len))
    return fail(MOE_ERR_INVALID_ARG, "seq_len=%d must be >= 1 and divide T=%d", c->seq_len, c->T);
  if (c->seq_aux_coeff != 0.0f && c->T / c->seq_len > 65535)
    return fail(MOE_ERR_UNSUPPORTED, "more than 65535 sequences (T / seq_len) for the sequence-wise loss");
  if (!(c->routed_scaling > 0.0f)) return fail(MOE_ERR_INVALID_ARG, "routed_scaling must be > 0");
  if (c->act_dtype != MOE_F32 && c->act_dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "unknown act dtype");
  if (c->wgrad_dtype != MOE_F32 && c->wgrad_dtype != MOE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "unknown weight-gradient dtype");
  if (c->wgrad_dtype == MOE_BF16 && c->act_dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "bf16 weight gradients need bf16 activations");
  if (c->w_dtype != 0 && c->w_dtype != MOE_FP8_E4M3) return fail(MOE_ERR_INVALID_ARG, "unknown weight dtype");
  if (c->w_dtype == MOE_FP8_E4M3) {
    if (c->act_dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "fp8 experts need bf16 activations");
    if (c->Fs) return fail(MOE_ERR_UNSUPPORTED, "fp8 experts: a shared expert is not provided");
    if (c->d % 128 || c->F % 128) return fail(MOE_ERR_UNSUPPORTED, "fp8 experts need d and F multiples of 128");
  }
  if (c->d % 64 || c->F % 64 || c->Fs % 64)
    return fail(MOE_ERR_UNSUPPORTED, "d, F and Fs must be multiples of 64 (d=%d F=%d Fs=%d)", c->d, c->F, c->Fs);
  if (c->act_dtype == MOE_BF16 && (c->F % 128 || c->Fs % 128))
    return fail(MOE_ERR_UNSUPPORTED, "bf16 path needs F and Fs multiples of 128");
  return MOE_OK;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define MOE_TRY(x)                  \
  do {                              \
    const moe_status_t _s = (x);    \
    if (_s != MOE_OK) return _s;    \
  } while (0)
#define MOE_NEED(p)                                                               \
  do {                                                                            \
    if (!(p)) return fail(MOE_ERR_INVALID_ARG, "%s: %s is NULL", __func__, #p);   \
  } while (0)
#define MOE_NEED16(p)                                                                          \
  do {                                                                                         \
    if (!(p)) return fail(MOE_ERR_INVALID_ARG, "%s: %s is NULL", __func__, #p);                \
    if (!aligned16(p)) return fail(MOE_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", __func__, #p); \
  } while (0)

moe_status_t need_ws(size_t have, size_t need, const char* fn) {
  if (have < need) return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, have, need);
  return MOE_OK;
}

hipStream_t S(void* s) { return static_cast<hipStream_t>(s); }

// Events of one moe_layer_bwd call that overlaps its expert weight gradients on a second,
// caller-owned stream: created by the call, recorded and waited on, and destroyed before it
// returns (a destroyed event's pending waits still complete), so no HIP object outlives the
// call.
struct CallEvents {
  hipEvent_t dy = nullptr, dh = nullptr, join = nullptr;
  ~CallEvents() {
    for (hipEvent_t e : {dy, dh, join})
      if (e) (void)hipEventDestroy(e);
  }
  moe_status_t create() {
    for (hipEvent_t* e : {&dy, &dh, &join})
      if (hipEventCreateWithFlags(e, hipEventDisableTiming) != hipSuccess) {
        *e = nullptr;
        return fail(MOE_ERR_HIP, "moe_layer_bwd: hipEventCreateWithFlags failed");
      }
    return MOE_OK;
  }
};

// Makes `waiter` wait for the work queued on `from` so far (no-op on one stream).
moe_status_t fork(hipStream_t from, hipEvent_t ev, hipStream_t waiter) {
  if (from == waiter) return MOE_OK;
  if (hipEventRecord(ev, from) != hipSuccess || hipStreamWaitEvent(waiter, ev, 0) != hipSuccess)
    return fail(MOE_ERR_HIP, "stream fork/join failed");
  return MOE_OK;
}

// The routed fc1 operand: the grouped rows x_perm, or (token_of given, x_perm NULL) the
// token rows of x read through token_of, bf16 only.
moe_status_t check_rows_source(const moe_config_t& c, const void* x_perm, const int32_t* token_of, const void* x) {
  if (!token_of) {
    MOE_NEED16(x_perm);
    return MOE_OK;
  }
  if (x_perm) return fail(MOE_ERR_INVALID_ARG, "give x_perm or token_of, not both");
  if (c.act_dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "the token_of row gather needs bf16 activations");
  MOE_NEED16(x);
  return MOE_OK;
}

// ----------------------------------------------------------------- launch sequences
moe_status_t run_gate(const moe_config_t& c, const void* x, const float* Wg, const float* bg, float* logits,
                      void* gate_ws, hipStream_t s) {
  if (gate_on_mfma(c)) return launch_gate_fwd_mfma(c, x, Wg, bg, logits, gate_ws, s);
  GemmDesc g{};
  g.a_major = K_MAJOR; g.b_major = K_MAJOR; g.ragged = RAGGED_M; g.epi = bg ? EPI_STORE_BIAS : EPI_STORE;
  g.a_type = c.act_dtype; g.b_type = MOE_F32; g.c_type = MOE_F32;
  g.N = c.E; g.K = c.d;
  g.A = x; g.lda = c.d; g.B = Wg; g.ldb = c.d; g.C = logits; g.ldc = c.E; g.bias = bg;
  g.range_end = c.T;
  return launch_gemm_fma(g, s);
}

// x_perm NULL: the routed fc1 reads the token rows of x through token_of (bf16 only).
moe_status_t run_experts_fwd(const moe_config_t& c, const void* x_perm, const int32_t* token_of,
                             const int32_t* offsets, const void* W13, const void* W2, const void* x, const void* W13s,
                             const void* W2s, void* H, void* Act, void* Y_perm, void* H_s, void* Act_s, void* Y_s,
                             int32_t* sched, hipStream_t s) {
  const int64_t A = static_cast<int64_t>(c.T) * c.k;
  for (int shared = 0; shared < (c.Fs ? 2 : 1); ++shared) {
    const int F = shared ? c.Fs : c.F;
    const void* X = shared ? x : x_perm;
    void* h = shared ? H_s : H;
    void* act = shared ? Act_s : Act;
    GemmDesc g1{};
    g1.a_major = K_MAJOR; g1.b_major = K_MAJOR; g1.ragged = RAGGED_M;
    g1.a_type = g1.b_type = c.act_dtype;
    g1.c_type = MOE_F32;  // H is kept in fp32 for the SwiGLU backward
    g1.N = 2 * F; g1.K = c.d; g1.F = F;
    g1.A = X; g1.lda = c.d;
    g1.B = shared ? W13s : W13; g1.ldb = c.d; g1.b_gstride = shared ? 0 : int64_t{2} * F * c.d;
    g1.C = h; g1.ldc = 2 * F; g1.C2 = act; g1.ldc2 = F;
    g1.offsets = shared ? nullptr : offsets; g1.G = shared ? 1 : c.E; g1.range_end = c.T; g1.rows_upper = A;
    g1.glu = glu_of(c);
    if (!shared && !x_perm) {
      g1.A = x;
      g1.gather = token_of;
      g1.gather_rows = c.T;
    }
    GemmDesc g2 = g1;
    g2.gather = nullptr;
    g2.c_type = MOE_F32;  // expert outputs are kept in fp32 for the combine
    g2.N = c.d; g2.K = F; g2.A = act; g2.lda = F;
    g2.B = shared ? W2s : W2; g2.ldb = F; g2.b_gstride = shared ? 0 : int64_t{1} * c.d * F;
    g2.C = shared ? Y_s : Y_perm; g2.ldc = c.d; g2.C2 = nullptr; g2.epi = EPI_STORE;
    if (c.act_dtype == MOE_BF16) {
      g1.epi = EPI_SWIGLU_FWD;
      MOE_TRY(launch_gemm_mfma(g1, sched, s));
      MOE_TRY(launch_gemm_mfma(g2, sched, s));
    } else {
      g1.epi = EPI_STORE;
      MOE_TRY(launch_gemm_fma(g1, s));
      MOE_TRY(launch_swiglu_fwd_elementwise(glu_of(c), static_cast<const float*>(h), static_cast<float*>(act),
                                            shared ? c.T : A,
                                            F, s));
      MOE_TRY(launch_gemm_fma(g2, s));
    }
  }
  return MOE_OK;
}

// dW[g] = dY_g^T X_g over the rows of each group (reduction-ragged); fp32 accumulation,
// output in the weight-gradient dtype.  A one-group bf16 call with split_ws (at least
// wgrad_split_bytes(N, K, rows)) is split over its rows when its output has too few tiles:
// fp32 partials per row chunk, then their sum in chunk order.
// x_rows (bf16 only): reduction row r of X is row x_rows[r] of X, which has x_src_rows rows.
// skew (with off, bf16): workspace of the skew split (routed_skew_bytes); a group with more
// rows than the plan's chunk is left to a second, fp32 launch over its row chunks, whose
// partials are then summed in chunk order.  max_group_rows bounds any group's rows.
moe_status_t run_wgrad(int act_dtype, int wgrad_dtype, const int32_t* off, int G, int64_t rows, const void* dY, int N,
                       const void* X, int K, void* dW, hipStream_t s, int beta, float* split_ws = nullptr,
                       const int32_t* x_rows = nullptr, int x_src_rows = 0, void* skew = nullptr,
                       size_t skew_bytes = 0, int64_t max_group_rows = 0) {
  GemmDesc w{};
  w.a_major = MN_MAJOR; w.b_major = MN_MAJOR; w.ragged = RAGGED_K; w.epi = EPI_STORE;
  w.a_type = w.b_type = act_dtype;
  w.c_type = wgrad_dtype;
  w.M = N; w.N = K;
  w.A = dY; w.lda = N; w.B = X; w.ldb = K;
  w.C = dW; w.ldc = K; w.c_gstride = int64_t{1} * N * K;
  w.offsets = off; w.G = G; w.range_end = static_cast<int>(rows);
  w.beta = beta;
  if (x_rows) {
    if (act_dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "gathered weight gradients need bf16 activations");
    w.gather = x_rows;
    w.gather_rows = x_src_rows;
  }
  const bool two_wg = act_dtype == MOE_BF16 && off && (x_rows || (K >= 1024 && wgrad2_supported(w)));
  if (act_dtype == MOE_BF16 && off && skew) {
    const int tiles = static_cast<int>(ceil_div(N, 256) * ceil_div(K, 256));
    const SkewPlan sp = skew_plan(G, rows, max_group_rows, N, K, tiles, 256);
    GemmDesc pc = w;
    pc.c_type = MOE_F32;
    pc.beta = 0;
    if (sp.chunk && align_up(sp.plan_bytes) + sp.partial_bytes <= skew_bytes && wgrad2_supported(pc)) {
      int32_t* plan = static_cast<int32_t*>(skew);
      float* part = reinterpret_cast<float*>(static_cast<char*>(skew) + align_up(sp.plan_bytes));
      MOE_TRY(launch_skew_plan(off, G, sp, plan, s));
      const SkewTables t = skew_tables(plan, G, sp);
      w.skip = t.skip;   // the split groups are left to the chunks below
      MOE_TRY(two_wg ? launch_wgrad2(w, s) : launch_gemm_mfma(w, nullptr, s));
      pc.pairs = t.pairs;
      pc.gcount = t.gcount;
      pc.G = sp.max_vg;
      pc.C = part;
      pc.ldc = K;
      pc.c_gstride = int64_t{1} * N * K;
      MOE_TRY(launch_wgrad2(pc, s));
      return launch_skew_reduce(part, t, sp, int64_t{1} * N * K, dW, w.c_gstride, wgrad_dtype, beta, s);
    }
  }
  if (x_rows) return launch_wgrad2(w, s);   // (fails with MOE_ERR_UNSUPPORTED on dimensions not multiples of 8)
  // per-expert gradients: many short reductions, each tile's fixed cost hidden by a second
  // workgroup on the CU.  Gradients with fewer than 1024 columns (fc2's at F = 512) are
  // faster on the 256 x 256 tiles, which read dY half as often.
  if (two_wg) return launch_wgrad2(w, s);
  if (act_dtype == MOE_BF16 && !off && split_ws) {
    const WgradSplit sp = wgrad_split(N, K, rows);
    if (sp.chunks > 1) {
      w.c_type = MOE_F32; w.C = split_ws; w.G = sp.chunks; w.kchunk = sp.kchunk; w.beta = 0;
      MOE_TRY(launch_gemm_mfma(w, nullptr, s));
      return launch_splitk_reduce(split_ws, sp.chunks, int64_t{1} * N * K, dW, wgrad_dtype, beta, s);
    }
  }
  return act_dtype == MOE_BF16 ? launch_gemm_mfma(w, nullptr, s) : launch_gemm_fma(w, s);
}

// fp8 experts: fc1 (+ SwiGLU -> act32, H), Act quantised per row per 128, fc2 -> Y_perm.
// token_of (or NULL): x_perm and xps are the token rows [T, ...], read through token_of.
moe_status_t run_experts_fp8(const moe_config_t& c, const uint8_t* x_perm, const float* xps, const int32_t* offsets,
                             const uint8_t* W13, const float* W13_scale, const uint8_t* W2, const float* W2_scale,
                             float* H, uint8_t* Act, float* Act_scale, float* Y_perm, float* act32, int32_t* sched,
                             hipStream_t s, const int32_t* token_of = nullptr) {
  const int64_t A = static_cast<int64_t>(c.T) * c.k;
  // one tile shape for both GEMMs (they share the tile schedule); with 128-row tiles the
  // fc1 epilogue quantises Act itself
  const bool narrow = fp8_tile_rows(A, c.E, 2 * c.F, c.F, true) == 128 && fp8_tile_rows(A, c.E, c.d, c.F, false) == 128;
  const int bm = narrow ? 128 : 256;
  const bool fused = bm == 128;
  MOE_TRY(launch_gemm_fp8(true, x_perm, xps, W13, W13_scale, fused ? nullptr : act32, H, offsets, c.E, A, 2 * c.F,
                          c.d, c.F, sched, s, glu_of(c), token_of, c.T, bm, fused ? Act : nullptr,
                          fused ? Act_scale : nullptr));
  if (!fused) MOE_TRY(launch_quantize_fp8(MOE_F32, act32, A, c.F, 1, Act, Act_scale, s));
  return launch_gemm_fp8(false, Act, Act_scale, W2, W2_scale, Y_perm, nullptr, offsets, c.E, A, c.d, c.F, c.F, sched,
                         s, Glu{0, 0.0f, 0.0f}, nullptr, 0, bm);
}

moe_status_t run_experts_bwd(const moe_config_t& c, const void* x_perm, const int32_t* offsets, const void* W13,
                             const void* W2, const void* H, const void* Act, const void* dY_perm, void* dH,
                             void* dX_perm, void* dW13, void* dW2, const void* x, const void* W13s, const void* W2s,
                             const void* H_s, const void* Act_s, const void* dY_s, void* dH_s, void* dx_s,
                             void* dW13s, void* dW2s, int32_t* sched, float* dact, float* wsplit, void* skew,
                             size_t skew_bytes, hipStream_t s, hipStream_t s2 = nullptr, hipEvent_t ev_dh = nullptr,
                             int beta = 0, const int32_t* token_of = nullptr) {
  // x_perm NULL: the routed fc1 weight gradient reads the token rows of x through token_of
  // s2 (when given, with dY_perm and dX_perm distinct) runs the weight gradients; its
  // caller has made it wait for dY_perm and joins it back.
  if (!s2) s2 = s;
  const int64_t A = static_cast<int64_t>(c.T) * c.k;
  for (int shared = 0; shared < (c.Fs ? 2 : 1); ++shared) {
    const int F = shared ? c.Fs : c.F;
    const int32_t* off = shared ? nullptr : offsets;
    const int G = shared ? 1 : c.E;
    const int64_t rows = shared ? c.T : A;
    const void* X = shared ? x : x_perm;
    const void* h = shared ? H_s : H;
    const void* act = shared ? Act_s : Act;
    const void* dY = shared ? dY_s : dY_perm;
    void* dh = shared ? dH_s : dH;
    void* dX = shared ? dx_s : dX_perm;
    const void* w13 = shared ? W13s : W13;
    const void* w2 = shared ? W2s : W2;
    void* dw13 = shared ? dW13s : dW13;
    void* dw2 = shared ? dW2s : dW2;
    const int et = c.act_dtype;
    // (1) fc2 data gradient: dAct = dY W2 (+ SwiGLU backward -> dH)
    GemmDesc d2{};
    d2.a_major = K_MAJOR; d2.b_major = MN_MAJOR; d2.ragged = RAGGED_M;
    d2.a_type = d2.b_type = d2.c_type = et;
    d2.N = F; d2.K = c.d; d2.F = F;
    d2.A = dY; d2.lda = c.d;
    d2.B = w2; d2.ldb = F; d2.b_gstride = shared ? 0 : int64_t{1} * c.d * F;
    d2.Hin = h; d2.ldh = 2 * F; d2.glu = glu_of(c);
    d2.offsets = off; d2.G = G; d2.range_end = c.T; d2.rows_upper = A;
    // (3) fc1 data gradient: dX = dH W13
    GemmDesc d1{};
    d1.a_major = K_MAJOR; d1.b_major = MN_MAJOR; d1.ragged = RAGGED_M; d1.epi = EPI_STORE;
    d1.a_type = d1.b_type = et;
    d1.c_type = MOE_F32;  // per-row input gradients in fp32 for the unpermute-reduce
    d1.N = c.d; d1.K = 2 * F;
    d1.A = dh; d1.lda = 2 * F;
    d1.B = w13; d1.ldb = c.d; d1.b_gstride = shared ? 0 : int64_t{2} * F * c.d;
    d1.C = dX; d1.ldc = c.d;
    d1.offsets = off; d1.G = G; d1.range_end = c.T; d1.rows_upper = A;
    if (et == MOE_BF16) {
      d2.epi = EPI_SWIGLU_BWD;
      d2.C = dh; d2.ldc = 2 * F;
      MOE_TRY(launch_gemm_mfma(d2, sched, s));
    } else {
      d2.epi = EPI_STORE;
      d2.C = dact; d2.ldc = F;
      MOE_TRY(launch_gemm_fma(d2, s));
      MOE_TRY(launch_swiglu_bwd_elementwise(glu_of(c), static_cast<const float*>(h), dact, static_cast<float*>(dh),
                                            rows, F, s));
    }
    // (2) fc2 weight gradient dW2 = dY^T Act, queued before dX may overwrite an aliased dY
    float* sw = shared ? wsplit : nullptr;   // both shared weight gradients run on s2, one after the other
    void* sk = shared ? nullptr : skew;   // the routed experts' (the two run on s2, one after the other)
    if (dw2) MOE_TRY(run_wgrad(et, c.wgrad_dtype, off, G, rows, dY, c.d, act, F, dw2, s2, beta, sw, nullptr, 0, sk,
                               skew_bytes, c.T));
    MOE_TRY(fork(s, ev_dh, s2));  // dH ready for the fc1 weight gradient
    MOE_TRY(et == MOE_BF16 ? launch_gemm_mfma(d1, sched, s) : launch_gemm_fma(d1, s));
    // (4) fc1 weight gradient dW13 = dH^T X
    const bool gathered = !shared && !x_perm;
    if (dw13)
      MOE_TRY(run_wgrad(et, c.wgrad_dtype, off, G, rows, dh, 2 * F, gathered ? x : X, c.d, dw13, s2, beta, sw,
                        gathered ? token_of : nullptr, c.T, sk, skew_bytes, c.T));
  }
  return MOE_OK;
}

moe_status_t run_gate_bwd(const moe_config_t& c, const void* x, const float* Wg, const float* dlogits, float* dWg,
                          float* dbg, float* dx_r, void* gate_ws, hipStream_t s, int beta = 0) {
  if (gate_on_mfma(c)) return launch_gate_bwd_mfma(c, x, Wg, dlogits, dWg, dbg, dx_r, gate_ws, s, beta);
  GemmDesc gw{};
  gw.a_major = MN_MAJOR; gw.b_major = MN_MAJOR; gw.ragged = RAGGED_K; gw.epi = EPI_STORE;
  gw.a_type = MOE_F32; gw.b_type = c.act_dtype; gw.c_type = MOE_F32;
  gw.M = c.E; gw.N = c.d;
  gw.A = dlogits; gw.lda = c.E; gw.B = x; gw.ldb = c.d; gw.C = dWg; gw.ldc = c.d;
  gw.range_end = c.T;
  gw.beta = beta;
  MOE_TRY(launch_gemm_fma(gw, s));
  if (dbg) MOE_TRY(launch_colsum_ws(dlogits, c.T, c.E, dbg, static_cast<float*>(gate_ws), s, beta));
  if (dx_r) {
    GemmDesc gx{};
    gx.a_major = K_MAJOR; gx.b_major = MN_MAJOR; gx.ragged = RAGGED_M; gx.epi = EPI_STORE;
    gx.a_type = MOE_F32; gx.b_type = MOE_F32; gx.c_type = MOE_F32;
    gx.N = c.d; gx.K = c.E;
    gx.A = dlogits; gx.lda = c.E; gx.B = Wg; gx.ldb = c.d; gx.C = dx_r; gx.ldc = c.d;
    gx.range_end = c.T;
    MOE_TRY(launch_gemm_fma(gx, s));
  }
  return MOE_OK;
}

// ------------------------------------------------- scratch of the allocation-free router call
// moe_router_topk_noalloc keeps its scratch in this file-scope device array instead of a
// workspace.  Each GPU the library runs on holds its own copy until the process ends.  In
// host code `scratch` names a host-side stand-in, not device memory: the device address is
// taken once per device with hipGetSymbolAddress and only that address is used.
constexpr size_t kNoallocScratchBytes = size_t{8} << 20;
__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

moe_status_t scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_HIP, "moe_router_topk_noalloc: no current device (or device id >= %d)", kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MOE_ERR_HIP, "moe_router_topk_noalloc: hipGetSymbolAddress failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_string(moe_status_t st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

const char* moe_last_error(void) { return g_err; }

moe_status_t moe_validate(const moe_config_t* cfg) {
  const moe_status_t st = validate(cfg);
  if (st == MOE_OK) g_err[0] = '\0';
  return st;
}

moe_status_t moe_workspace_size(const moe_config_t* cfg, size_t* fwd_bytes, size_t* bwd_bytes) {
  MOE_TRY(validate(cfg));
  if (fwd_bytes) *fwd_bytes = carve_fwd(*cfg, nullptr).bytes;
  if (bwd_bytes) *bwd_bytes = carve_bwd(*cfg, nullptr).bytes;
  return MOE_OK;
}

moe_status_t moe_gate_logits(const moe_config_t* cfg, const void* x, const float* Wg, const float* bg,
                             float* logits, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(validate(cfg));
  MOE_NEED(x); MOE_NEED(Wg); MOE_NEED(logits); MOE_NEED(ws);
  const FwdWs fw = carve_fwd(*cfg, ws);
  MOE_TRY(need_ws(ws_bytes, fw.bytes, __func__));
  return run_gate(*cfg, x, Wg, bg, logits, fw.gate, S(stream));
}

moe_status_t moe_router_topk(const moe_config_t* cfg, const float* logits, const float* expert_bias, int32_t* idx,
                             float* w, int32_t* counts, float* prob_sum, float* stats, int32_t* seq_counts, void* ws,
                             size_t ws_bytes, void* stream) {
  MOE_TRY(validate(cfg));
  MOE_NEED(logits); MOE_NEED(idx); MOE_NEED(w); MOE_NEED(counts); MOE_NEED(ws);
  if (cfg->seq_aux_coeff != 0.0f) MOE_NEED(seq_counts);
  if (expert_bias && cfg->score == MOE_SOFTMAX)
    return fail(MOE_ERR_UNSUPPORTED, "the expert bias is provided for sigmoid and sqrt(softplus) scores only");
  const FwdWs fw = carve_fwd(*cfg, ws);
  MOE_TRY(need_ws(ws_bytes, fw.bytes, __func__));
  return launch_router_topk(*cfg, logits, expert_bias, idx, w, counts, prob_sum, fw.prob_sum, stats, seq_counts,
                            router_ws(fw), S(stream));
}

moe_status_t moe_router_topk_noalloc(const moe_config_t* cfg, const float* logits, const float* expert_bias,
                                     int32_t* idx, float* w, int32_t* counts, float* prob_sum, float* stats,
                                     int32_t* seq_counts, void* stream) {
  MOE_TRY(validate(cfg));
  MOE_NEED(logits); MOE_NEED(idx); MOE_NEED(w); MOE_NEED(counts);
  if (cfg->seq_aux_coeff != 0.0f) MOE_NEED(seq_counts);
  if (expert_bias && cfg->score == MOE_SOFTMAX)
    return fail(MOE_ERR_UNSUPPORTED, "the expert bias is provided for sigmoid and sqrt(softplus) scores only");
  const size_t need = carve_router(*cfg, nullptr).bytes;
  if (need > kNoallocScratchBytes)
    return fail(MOE_ERR_WORKSPACE, "%s: this configuration needs %zu bytes of scratch, more than the %zu of the static "
                "scratch (use moe_router_topk with a workspace)", __func__, need, kNoallocScratchBytes);
  void* base = nullptr;
  MOE_TRY(scratch_address(&base));
  const RouterScratch rs = carve_router(*cfg, base);
  return launch_router_topk(*cfg, logits, expert_bias, idx, w, counts, prob_sum, rs.prob_sum, stats, seq_counts,
                            rs.rw, S(stream));
}

moe_status_t moe_expert_bias_update(const moe_config_t* cfg, const int32_t* counts, float rate, int32_t centered,
                                    float* expert_bias, void* stream) {
  MOE_TRY(validate(cfg));
  MOE_NEED(counts); MOE_NEED(expert_bias);
  if (!(rate > -INFINITY && rate < INFINITY)) return fail(MOE_ERR_INVALID_ARG, "rate must be finite");
  return launch_bias_update(counts, cfg->E, rate, centered ? 1 : 0, expert_bias, S(stream));
}

moe_status_t moe_router_quantile(const moe_config_t* cfg, const float* scores, const float* beta, int32_t* idx,
                                 float* alpha, float* beta_local, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(validate(cfg));
  MOE_NEED(scores); MOE_NEED(beta); MOE_NEED(idx); MOE_NEED(alpha); MOE_NEED(ws);
  if (cfg->k >= cfg->E) return fail(MOE_ERR_INVALID_ARG, "quantile routing needs k < E (k=%d E=%d)", cfg->k, cfg->E);
  if (cfg->num_groups) return fail(MOE_ERR_UNSUPPORTED, "quantile balancing does not take group-limited routing");
  if (beta_local && (static_cast<int64_t>(cfg->T) * cfg->k) % cfg->E)
    return fail(MOE_ERR_INVALID_ARG, "quantile balancing needs T*k (%lld) to be a multiple of E=%d",
                static_cast<long long>(cfg->T) * cfg->k, cfg->E);
  const FwdWs fw = carve_fwd(*cfg, ws);
  MOE_TRY(need_ws(ws_bytes, fw.bytes, __func__));
  return launch_router_quantile(*cfg, scores, beta, idx, alpha, beta_local, fw.quantile, S(stream));
}

moe_status_t moe_quantile_bias_update(const moe_config_t* cfg, const float* beta_local, float ema, float* beta,
                                      void* stream) {
  MOE_TRY(validate(cfg));
  MOE_NEED(beta_local); MOE_NEED(beta);
  if (!(ema >= 0.0f && ema <= 1.0f)) return fail(MOE_ERR_INVALID_ARG, "ema must be in [0, 1]");
  return launch_quantile_update(beta_local, cfg->E, ema, beta, S(stream));
}

moe_status_t moe_permute(const moe_config_t* cfg, const void* x, const int32_t* idx, int32_t* offsets,
                         int32_t* row_of, int32_t* token_of, void* x_perm, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(validate(cfg));
  MOE_NEED(idx); MOE_NEED(offsets); MOE_NEED(row_of); MOE_NEED(token_of); MOE_NEED(ws);
  if (x_perm) { MOE_NEED16(x); MOE_NEED16(x_perm); }   // NULL x_perm: the grouping only
  const FwdWs fw = carve_fwd(*cfg, ws);
  MOE_TRY(need_ws(ws_bytes, fw.bytes, __func__));
  return launch_permute(*cfg, x, idx, offsets, row_of, token_of, x_perm, fw.cnt_part, fw.blk_base, fw.counts,
                        false, S(stream));
}

moe_status_t moe_grouped_gemm_swiglu(const moe_config_t* cfg, const void* x_perm, const int32_t* token_of,
                                     const int32_t* offsets, const void* W13, const void* W2, const void* x,
                                     const void* W13s, const void* W2s, void* H, void* Act, void* Y_perm, void* H_s,
                                     void* Act_s, void* Y_s, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(validate(cfg));
  MOE_TRY(check_rows_source(*cfg, x_perm, token_of, x));
  MOE_NEED(offsets); MOE_NEED16(W13); MOE_NEED16(W2); MOE_NEED16(H); MOE_NEED16(Act);
  MOE_NEED16(Y_perm); MOE_NEED(ws);
  if (cfg->Fs) {
    MOE_NEED16(x); MOE_NEED16(W13s); MOE_NEED16(W2s); MOE_NEED16(H_s); MOE_NEED16(Act_s); MOE_NEED16(Y_s);
  }
  const FwdWs fw = carve_fwd(*cfg, ws);
  MOE_TRY(need_ws(ws_bytes, fw.bytes, __func__));
  return run_experts_fwd(*cfg, x_perm, token_of, offsets, W13, W2, x, W13s, W2s, H, Act, Y_perm, H_s, Act_s, Y_s,
                         fw.sched, S(stream));
}

moe_status_t moe_unpermute_combine(const moe_config_t* cfg, const float* Y_perm, const int32_t* row_of,
                                   const float* w, const float* Y_s, const float* gs, float* y, void* stream) {
  MOE_TRY(validate(cfg));
  MOE_NEED16(Y_perm); MOE_NEED(row_of); MOE_NEED(w); MOE_NEED16(y);
  if (Y_s && !aligned16(Y_s)) return fail(MOE_ERR_INVALID_ARG, "Y_s is not 16-byte aligned");
  if (gs && !Y_s) return fail(MOE_ERR_INVALID_ARG, "gs without Y_s");
  return launch_combine(*cfg, static_cast<const float*>(Y_perm), row_of, w, static_cast<const float*>(Y_s), gs,
                        static_cast<float*>(y), S(stream));
}

moe_status_t moe_shared_gate(const moe_config_t* cfg, const void* x, const float* Wsg, float* gs, void* stream) {
  MOE_TRY(validate(cfg));
  MOE_NEED16(x); MOE_NEED16(Wsg); MOE_NEED(gs);
  return launch_shared_gate(*cfg, x, Wsg, gs, S(stream));
}

moe_status_t moe_shared_gate_bwd(const moe_config_t* cfg, const void* x, const float* dl_s, float* dWsg, void* ws,
                                 size_t ws_bytes, void* stream) {
  MOE_TRY(validate(cfg));
  MOE_NEED(x); MOE_NEED(dl_s); MOE_NEED(dWsg); MOE_NEED(ws);
  if (!cfg->shared_gate) return fail(MOE_ERR_INVALID_ARG, "moe_shared_gate_bwd needs shared_gate = 1");
  const BwdWs bw = carve_bwd(*cfg, ws);
  MOE_TRY(need_ws(ws_bytes, bw.bytes, __func__));
  return launch_shared_gate_bwd(*cfg, x, dl_s, dWsg, bw.sg_part, S(stream));
}

moe_status_t moe_layer_fwd(const moe_config_t* cfg, const moe_weights_t* W, const void* x, const moe_saved_t* sv,
                           float* y, float* stats, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(validate(cfg));
  MOE_NEED(W); MOE_NEED(sv); MOE_NEED16(x); MOE_NEED16(y); MOE_NEED(ws);
  MOE_NEED(W->Wg); MOE_NEED16(W->W13); MOE_NEED16(W->W2);
  MOE_NEED(sv->logits); MOE_NEED(sv->idx); MOE_NEED(sv->w); MOE_NEED(sv->counts); MOE_NEED(sv->offsets);
  MOE_NEED(sv->row_of); MOE_NEED(sv->token_of); MOE_NEED16(sv->Act);
  MOE_NEED16(sv->Y_perm);
  // saved->x_perm NULL: the grouped fc1 reads the token rows of x through token_of
  const bool gathered = sv->x_perm == nullptr;
  if (gathered && cfg->act_dtype != MOE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "saved->x_perm is needed with fp32 activations (the row gather is bf16 only)");
  if (!gathered) MOE_NEED16(sv->x_perm);
  const bool fp8 = cfg->w_dtype == MOE_FP8_E4M3;
  if (fp8) {
    MOE_NEED(W->W13_scale); MOE_NEED(W->W2_scale); MOE_NEED(sv->Act_scale);
    if (!gathered) MOE_NEED(sv->x_perm_scale);
    if (sv->H && !aligned16(sv->H)) return fail(MOE_ERR_INVALID_ARG, "H is not 16-byte aligned");
  } else {
    MOE_NEED16(sv->H);
  }
  if (cfg->Fs) {
    MOE_NEED16(W->W13s); MOE_NEED16(W->W2s); MOE_NEED16(sv->H_s); MOE_NEED16(sv->Act_s); MOE_NEED16(sv->Y_s);
  }
  if (W->expert_bias && cfg->score == MOE_SOFTMAX)
    return fail(MOE_ERR_UNSUPPORTED, "the expert bias is provided for sigmoid and sqrt(softplus) scores only");
  if (cfg->seq_aux_coeff != 0.0f) MOE_NEED(sv->seq_counts);
  if (cfg->shared_gate) { MOE_NEED16(W->Wsg); MOE_NEED(sv->gs); }
  const FwdWs fw = carve_fwd(*cfg, ws);
  MOE_TRY(need_ws(ws_bytes, fw.bytes, __func__));
  const moe_config_t& c = *cfg;
  hipStream_t s = S(stream);
  MOE_TRY(run_gate(c, x, W->Wg, W->bg, sv->logits, fw.gate, s));
  if (c.shared_gate) MOE_TRY(launch_shared_gate(c, x, W->Wsg, sv->gs, s));
  MOE_TRY(launch_router_topk(c, sv->logits, W->expert_bias, sv->idx, sv->w, sv->counts, nullptr, fw.prob_sum, stats,
                             sv->seq_counts, router_ws(fw), s));
  if (fp8) {
    // x is quantised per token per 128 before the permute, so the permute moves e4m3 rows
    const int64_t A = static_cast<int64_t>(c.T) * c.k;
    MOE_TRY(launch_quantize_fp8(MOE_BF16, x, c.T, c.d, 1, fw.xq, fw.xs, s));
    MOE_TRY(launch_permute(c, fw.xq, sv->idx, sv->offsets, sv->row_of, sv->token_of, sv->x_perm, fw.cnt_part,
                           fw.blk_base, fw.counts, true, s, 1));
    if (!gathered) MOE_TRY(launch_gather_scales(fw.xs, sv->token_of, A, c.d / 128, sv->x_perm_scale, s));
    MOE_TRY(run_experts_fp8(c, gathered ? fw.xq : static_cast<const uint8_t*>(sv->x_perm),
                            gathered ? fw.xs : sv->x_perm_scale, sv->offsets,
                            static_cast<const uint8_t*>(W->W13), W->W13_scale, static_cast<const uint8_t*>(W->W2),
                            W->W2_scale, static_cast<float*>(sv->H), static_cast<uint8_t*>(sv->Act), sv->Act_scale,
                            static_cast<float*>(sv->Y_perm), fw.act32, fw.sched, s,
                            gathered ? sv->token_of : nullptr));
    return launch_combine(c, static_cast<const float*>(sv->Y_perm), sv->row_of, sv->w, nullptr, nullptr,
                          static_cast<float*>(y), s);
  }
  MOE_TRY(launch_permute(c, x, sv->idx, sv->offsets, sv->row_of, sv->token_of, sv->x_perm, fw.cnt_part, fw.blk_base,
                         fw.counts, true, s));
  MOE_TRY(run_experts_fwd(c, sv->x_perm, sv->token_of, sv->offsets, W->W13, W->W2, x, W->W13s, W->W2s, sv->H,
                          sv->Act, sv->Y_perm, sv->H_s, sv->Act_s, sv->Y_s, fw.sched, s));
  return launch_combine(c, static_cast<const float*>(sv->Y_perm), sv->row_of, sv->w,
                        c.Fs ? static_cast<const float*>(sv->Y_s) : nullptr, c.shared_gate ? sv->gs : nullptr,
                        static_cast<float*>(y), s);
}

moe_status_t moe_unpermute_combine_bwd(const moe_config_t* cfg, const float* dy, const float* Y_perm,
                                       const int32_t* row_of, const float* w, void* dY_perm, float* dw,
                                       void* dY_s, const float* gs, const float* Y_s, float* dl_s, void* stream) {
  MOE_TRY(validate(cfg));
  MOE_NEED16(dy); MOE_NEED16(Y_perm); MOE_NEED(row_of); MOE_NEED(w); MOE_NEED(dw);
  if (dY_perm && !aligned16(dY_perm)) return fail(MOE_ERR_INVALID_ARG, "dY_perm is not 16-byte aligned");
  if (dY_s && !aligned16(dY_s)) return fail(MOE_ERR_INVALID_ARG, "dY_s is not 16-byte aligned");
  if ((gs != nullptr) != (dl_s != nullptr) || (gs != nullptr) != (Y_s != nullptr))
    return fail(MOE_ERR_INVALID_ARG, "the shared gate needs gs, Y_s and dl_s together");
  if (Y_s && !aligned16(Y_s)) return fail(MOE_ERR_INVALID_ARG, "Y_s is not 16-byte aligned");
  return launch_combine_bwd(*cfg, dy, Y_perm, row_of, w, dY_perm, dw, dY_s, gs, Y_s, dl_s, S(stream));
}

moe_status_t moe_grouped_gemm_swiglu_bwd(const moe_config_t* cfg, const void* x_perm, const int32_t* token_of,
                                         const int32_t* offsets, const void* W13, const void* W2, const void* H,
                                         const void* Act, const void* dY_perm, void* dH, void* dX_perm, void* dW13,
                                         void* dW2, const void* x, const void* W13s, const void* W2s,
                                         const void* H_s, const void* Act_s, const void* dY_s, void* dH_s,
                                         void* dx_s, void* dW13s, void* dW2s, void* ws, size_t ws_bytes,
                                         void* stream) {
  MOE_TRY(validate(cfg));
  MOE_NEED(offsets); MOE_NEED16(W13); MOE_NEED16(W2); MOE_NEED16(H); MOE_NEED16(Act);
  MOE_NEED16(dY_perm); MOE_NEED16(dH); MOE_NEED16(dX_perm); MOE_NEED(ws);
  const bool wgrad = dW13 || dW2;
  if (wgrad) MOE_TRY(check_rows_source(*cfg, x_perm, token_of, x));
  if (wgrad) { MOE_NEED16(dW13); MOE_NEED16(dW2); }
  if (cfg->Fs) {
    MOE_NEED16(x); MOE_NEED16(W13s); MOE_NEED16(W2s); MOE_NEED16(H_s); MOE_NEED16(Act_s); MOE_NEED16(dY_s);
    MOE_NEED16(dH_s); MOE_NEED16(dx_s);
    if (wgrad) { MOE_NEED16(dW13s); MOE_NEED16(dW2s); }
    else if (dW13s || dW2s) return fail(MOE_ERR_INVALID_ARG, "shared weight gradients given without routed ones");
  }
  const BwdWs bw = carve_bwd(*cfg, ws);
  MOE_TRY(need_ws(ws_bytes, bw.bytes, __func__));
  return run_experts_bwd(*cfg, x_perm, offsets, W13, W2, H, Act, dY_perm, dH, dX_perm, dW13, dW2, x, W13s, W2s, H_s,
                         Act_s, dY_s, dH_s, dx_s, dW13s, dW2s, bw.sched, bw.dact, bw.wsplit, bw.skew, bw.skew_bytes,
                         S(stream), nullptr, nullptr, 0, token_of);
}

moe_status_t moe_grouped_wgrad(const moe_config_t* cfg, const int32_t* offsets, int32_t groups, int64_t rows,
                               const void* dY, int32_t N, const void* X, int32_t K, const int32_t* x_rows,
                               int32_t x_src_rows, void* dW, int32_t accumulate, void* ws, size_t ws_bytes,
                               void* stream) {
  MOE_TRY(validate(cfg));
  MOE_NEED16(dY); MOE_NEED16(X); MOE_NEED16(dW);
  if (groups < 1 || groups > 4096) return fail(MOE_ERR_INVALID_ARG, "groups must be in [1, 4096]");
  if (!offsets && groups != 1) return fail(MOE_ERR_INVALID_ARG, "without offsets there is exactly one group");
  if (rows < 0 || rows >= (int64_t{1} << 31)) return fail(MOE_ERR_INVALID_ARG, "rows must be in [0, 2^31)");
  if (N < 64 || K < 64 || N % 64 || K % 64) return fail(MOE_ERR_INVALID_ARG, "N and K must be positive multiples of 64");
  if (static_cast<int64_t>(N) * K * 4 >= (int64_t{1} << 40)) return fail(MOE_ERR_INVALID_ARG, "dW group too large");
  if (accumulate != 0 && accumulate != 1) return fail(MOE_ERR_INVALID_ARG, "accumulate must be 0 or 1");
  if (x_rows) {
    if (cfg->act_dtype != MOE_BF16)
      return fail(MOE_ERR_UNSUPPORTED, "x_rows (the row gather of X) needs bf16 activations");
    if (x_src_rows < 1) return fail(MOE_ERR_INVALID_ARG, "x_src_rows must be >= 1 with x_rows");
    const bool skew = ws && offsets && aligned16(ws);
    return run_wgrad(cfg->act_dtype, cfg->wgrad_dtype, offsets, groups, rows, dY, N, X, K, dW, S(stream), accumulate,
                     nullptr, x_rows, x_src_rows, skew ? ws : nullptr, skew ? ws_bytes : 0, std::min<int64_t>(rows, cfg->T));
  }
  float* split = nullptr;
  if (ws && !offsets && cfg->act_dtype == MOE_BF16) {
    const size_t need = wgrad_split_bytes(N, K, rows);
    if (need) {
      MOE_TRY(need_ws(ws_bytes, need, __func__));
      if (!aligned16(ws)) return fail(MOE_ERR_INVALID_ARG, "ws is not 16-byte aligned");
      split = static_cast<float*>(ws);
    }
  }
  // with offsets: the skew split of the layer backward when ws holds its plan.  A group is
  // an expert's rows, at most T of them, so the split is enabled exactly when the layer's
  // is (chunk below T and below rows), and gives the layer's bits
  const bool skew = ws && offsets && aligned16(ws);
  return run_wgrad(cfg->act_dtype, cfg->wgrad_dtype, offsets, groups, rows, dY, N, X, K, dW, S(stream), accumulate,
                   split, nullptr, 0, skew ? ws : nullptr, skew ? ws_bytes : 0, std::min<int64_t>(rows, cfg->T));
}

moe_status_t moe_quantize_fp8(int32_t src_dtype, const void* src, int64_t rows, int32_t cols, int32_t block_rows,
                              uint8_t* q, float* scale, void* stream) {
  MOE_NEED16(src); MOE_NEED16(q); MOE_NEED(scale);
  if (src_dtype != MOE_BF16 && src_dtype != MOE_F32) return fail(MOE_ERR_INVALID_ARG, "src dtype must be bf16 or fp32");
  if (block_rows != 1 && block_rows != 128) return fail(MOE_ERR_INVALID_ARG, "block_rows must be 1 or 128");
  if (rows < 1 || cols < 128 || cols % 128) return fail(MOE_ERR_INVALID_ARG, "rows >= 1 and cols a multiple of 128");
  if (rows % block_rows) return fail(MOE_ERR_INVALID_ARG, "rows must be a multiple of block_rows");
  if (rows * cols >= (int64_t{1} << 40)) return fail(MOE_ERR_INVALID_ARG, "matrix too large");
  return launch_quantize_fp8(src_dtype, src, rows, cols, block_rows, q, scale, S(stream));
}

moe_status_t moe_permute_fp8(const moe_config_t* cfg, const uint8_t* x_q, const float* x_scale, const int32_t* idx,
                             int32_t* offsets, int32_t* row_of, int32_t* token_of, uint8_t* x_perm,
                             float* x_perm_scale, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(validate(cfg));
  if (cfg->w_dtype != MOE_FP8_E4M3) return fail(MOE_ERR_INVALID_ARG, "moe_permute_fp8 needs w_dtype fp8");
  MOE_NEED(idx); MOE_NEED(offsets); MOE_NEED(row_of); MOE_NEED(token_of); MOE_NEED(ws);
  if ((x_perm != nullptr) != (x_perm_scale != nullptr))
    return fail(MOE_ERR_INVALID_ARG, "x_perm and x_perm_scale go together (both NULL: the grouping only)");
  if (x_perm) { MOE_NEED16(x_q); MOE_NEED(x_scale); MOE_NEED16(x_perm); }
  const FwdWs fw = carve_fwd(*cfg, ws);
  MOE_TRY(need_ws(ws_bytes, fw.bytes, __func__));
  hipStream_t s = S(stream);
  MOE_TRY(launch_permute(*cfg, x_q, idx, offsets, row_of, token_of, x_perm, fw.cnt_part, fw.blk_base, fw.counts,
                         false, s, 1));
  if (!x_perm) return MOE_OK;
  return launch_gather_scales(x_scale, token_of, static_cast<int64_t>(cfg->T) * cfg->k, cfg->d / 128, x_perm_scale,
                              s);
}

moe_status_t moe_grouped_gemm_swiglu_fp8(const moe_config_t* cfg, const uint8_t* x_perm, const float* x_perm_scale,
                                         const int32_t* token_of, const int32_t* offsets, const uint8_t* W13,
                                         const float* W13_scale,
                                         const uint8_t* W2, const float* W2_scale, float* H, uint8_t* Act,
                                         float* Act_scale, float* Y_perm, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(validate(cfg));
  if (cfg->w_dtype != MOE_FP8_E4M3) return fail(MOE_ERR_INVALID_ARG, "moe_grouped_gemm_swiglu_fp8 needs w_dtype fp8");
  MOE_NEED16(x_perm); MOE_NEED(x_perm_scale); MOE_NEED(offsets); MOE_NEED16(W13); MOE_NEED(W13_scale);
  MOE_NEED16(W2); MOE_NEED(W2_scale); MOE_NEED16(Act); MOE_NEED(Act_scale); MOE_NEED16(Y_perm); MOE_NEED(ws);
  if (H && !aligned16(H)) return fail(MOE_ERR_INVALID_ARG, "H is not 16-byte aligned");
  const FwdWs fw = carve_fwd(*cfg, ws);
  MOE_TRY(need_ws(ws_bytes, fw.bytes, __func__));
  return run_experts_fp8(*cfg, x_perm, x_perm_scale, offsets, W13, W13_scale, W2, W2_scale, H, Act, Act_scale, Y_perm,
                         fw.act32, fw.sched, S(stream), token_of);
}

moe_status_t moe_permute_bwd(const moe_config_t* cfg, const float* dX_perm, const int32_t* row_of, const float* dx_s,
                             const float* dx_r, const float* dl_s, const float* Wsg, float* dx, void* stream) {
  MOE_TRY(validate(cfg));
  MOE_NEED16(dX_perm); MOE_NEED(row_of); MOE_NEED16(dx);
  if (dx_s && !aligned16(dx_s)) return fail(MOE_ERR_INVALID_ARG, "dx_s is not 16-byte aligned");
  if (dx_r && !aligned16(dx_r)) return fail(MOE_ERR_INVALID_ARG, "dx_r is not 16-byte aligned");
  if ((dl_s != nullptr) != (Wsg != nullptr)) return fail(MOE_ERR_INVALID_ARG, "dl_s and Wsg go together");
  if (Wsg && !aligned16(Wsg)) return fail(MOE_ERR_INVALID_ARG, "Wsg is not 16-byte aligned");
  return launch_unpermute_reduce(*cfg, dX_perm, row_of, dx_s, dx_r, dl_s, Wsg, dx, S(stream));
}

moe_status_t moe_router_bwd(const moe_config_t* cfg, const float* logits, const int32_t* idx, const float* w,
                            const float* dw, const int32_t* counts, const int32_t* seq_counts, float daux,
                            float* dlogits, void* stream) {
  MOE_TRY(validate(cfg));
  MOE_NEED(logits); MOE_NEED(idx); MOE_NEED(w); MOE_NEED(dw); MOE_NEED(dlogits);
  if (!(daux > -INFINITY && daux < INFINITY)) return fail(MOE_ERR_INVALID_ARG, "daux must be finite");
  if (cfg->aux_coeff != 0.0f && daux != 0.0f) MOE_NEED(counts);
  if (cfg->seq_aux_coeff != 0.0f && daux != 0.0f) MOE_NEED(seq_counts);
  return launch_router_bwd(*cfg, logits, idx, w, dw, counts, seq_counts, daux, dlogits, S(stream));
}

moe_status_t moe_gate_logits_bwd(const moe_config_t* cfg, const void* x, const float* Wg, const float* dlogits,
                                 float* dWg, float* dbg, float* dx_r, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(validate(cfg));
  MOE_NEED(x); MOE_NEED(Wg); MOE_NEED(dlogits); MOE_NEED(dWg); MOE_NEED(ws);
  const BwdWs bw = carve_bwd(*cfg, ws);
  MOE_TRY(need_ws(ws_bytes, bw.bytes, __func__));
  return run_gate_bwd(*cfg, x, Wg, dlogits, dWg, dbg, dx_r, bw.gate, S(stream));
}

moe_status_t moe_layer_bwd(const moe_config_t* cfg, const moe_weights_t* W, const moe_saved_t* sv, const void* x,
                           const float* dy, float daux, float* dx, const moe_grads_t* gr, void* ws, size_t ws_bytes,
                           void* stream, void* wgrad_stream) {
  MOE_TRY(validate(cfg));
  MOE_NEED(W); MOE_NEED(sv); MOE_NEED(gr); MOE_NEED16(x); MOE_NEED16(dy); MOE_NEED16(dx); MOE_NEED(ws);
  MOE_NEED(W->Wg); MOE_NEED16(W->W13); MOE_NEED16(W->W2);
  MOE_NEED(sv->logits); MOE_NEED(sv->idx); MOE_NEED(sv->w); MOE_NEED(sv->counts); MOE_NEED(sv->offsets);
  MOE_NEED(sv->row_of); MOE_NEED16(sv->Y_perm); MOE_NEED(gr->dWg);
  if (!(daux > -INFINITY && daux < INFINITY)) return fail(MOE_ERR_INVALID_ARG, "daux must be finite");
  if (cfg->seq_aux_coeff != 0.0f && daux != 0.0f) MOE_NEED(sv->seq_counts);
  if (gr->accumulate != 0 && gr->accumulate != 1) return fail(MOE_ERR_INVALID_ARG, "accumulate must be 0 or 1");
  const int beta = gr->accumulate;
  if (cfg->w_dtype == MOE_FP8_E4M3) {
    // frozen e4m3 experts: the backward runs through the mixing weights only
    if (gr->dW13 || gr->dW2 || gr->dW13s || gr->dW2s)
      return fail(MOE_ERR_INVALID_ARG, "fp8 experts are frozen: expert weight gradients must be NULL");
    const BwdWs bw = carve_bwd(*cfg, ws);
    MOE_TRY(need_ws(ws_bytes, bw.bytes, __func__));
    const moe_config_t& c = *cfg;
    hipStream_t s = S(stream);
    MOE_TRY(launch_combine_bwd(c, dy, static_cast<const float*>(sv->Y_perm), sv->row_of, sv->w, nullptr, bw.dw,
                               nullptr, nullptr, nullptr, nullptr, s));
    MOE_TRY(launch_router_bwd(c, sv->logits, sv->idx, sv->w, bw.dw, sv->counts, sv->seq_counts, daux, bw.dlogits, s));
    return run_gate_bwd(c, x, W->Wg, bw.dlogits, gr->dWg, gr->dbg, dx, bw.gate, s, beta);
  }
  if (sv->x_perm) {
    MOE_NEED16(sv->x_perm);
  } else {   // the fc1 weight gradient reads the token rows of x through token_of
    if (cfg->act_dtype != MOE_BF16)
      return fail(MOE_ERR_INVALID_ARG, "saved->x_perm is needed with fp32 activations (the row gather is bf16 only)");
    MOE_NEED(sv->token_of);
  }
  MOE_NEED16(sv->H); MOE_NEED16(sv->Act); MOE_NEED16(gr->dW13); MOE_NEED16(gr->dW2);
  if (cfg->Fs) {
    MOE_NEED16(W->W13s); MOE_NEED16(W->W2s); MOE_NEED16(sv->H_s); MOE_NEED16(sv->Act_s);
    MOE_NEED16(gr->dW13s); MOE_NEED16(gr->dW2s);
  }
  if (cfg->shared_gate) { MOE_NEED16(W->Wsg); MOE_NEED16(sv->gs); MOE_NEED16(sv->Y_s); MOE_NEED(gr->dWsg); }
  const BwdWs bw = carve_bwd(*cfg, ws);
  MOE_TRY(need_ws(ws_bytes, bw.bytes, __func__));
  const moe_config_t& c = *cfg;
  hipStream_t s = S(stream);
  // the shared expert's upstream gradient is dy itself in the activation dtype (an fp32
  // layer reads dy in place), or gs dy behind its gate
  const bool dy_in_place = c.act_dtype == MOE_F32 && !c.shared_gate;
  void* dY_s = c.Fs ? (dy_in_place ? const_cast<float*>(dy) : bw.dY_s) : nullptr;
  MOE_TRY(launch_combine_bwd(c, dy, static_cast<const float*>(sv->Y_perm), sv->row_of, sv->w, bw.dY, bw.dw,
                             dy_in_place ? nullptr : dY_s, c.shared_gate ? sv->gs : nullptr,
                             c.shared_gate ? static_cast<const float*>(sv->Y_s) : nullptr, bw.dl_s, s));
  // the expert weight gradients go to wgrad_stream when the caller gives a second stream:
  // it waits for dY_perm (and the shared expert's dY) here and for dH inside run_experts_bwd
  hipStream_t s2 = wgrad_stream ? S(wgrad_stream) : s;
  CallEvents ev;
  if (s2 != s) MOE_TRY(ev.create());
  MOE_TRY(fork(s, ev.dy, s2));
  MOE_TRY(run_experts_bwd(c, sv->x_perm, sv->offsets, W->W13, W->W2, sv->H, sv->Act, bw.dY, bw.dH, bw.dX, gr->dW13,
                          gr->dW2, x, W->W13s, W->W2s, sv->H_s, sv->Act_s, dY_s, bw.dH_s, bw.dx_s, gr->dW13s,
                          gr->dW2s, bw.sched, bw.dact, bw.wsplit, bw.skew, bw.skew_bytes, s, s2, ev.dh, beta,
                          sv->token_of));
  MOE_TRY(launch_router_bwd(c, sv->logits, sv->idx, sv->w, bw.dw, sv->counts, sv->seq_counts, daux, bw.dlogits, s));
  MOE_TRY(run_gate_bwd(c, x, W->Wg, bw.dlogits, gr->dWg, gr->dbg, bw.dx_r, bw.gate, s, beta));
  if (c.shared_gate) MOE_TRY(launch_shared_gate_bwd(c, x, bw.dl_s, gr->dWsg, bw.sg_part, s, beta));
  MOE_TRY(launch_unpermute_reduce(c, bw.dX, sv->row_of, c.Fs ? static_cast<const float*>(bw.dx_s) : nullptr,
                                  bw.dx_r, c.shared_gate ? bw.dl_s : nullptr, c.shared_gate ? W->Wsg : nullptr, dx,
                                  s));
  return fork(s2, ev.join, s);  // the caller's stream sees the weight gradients too
}

}  // extern "C"
