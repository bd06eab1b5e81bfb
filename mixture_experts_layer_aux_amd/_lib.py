"""ctypes binding of libmoe (include/moe.h): argument marshalling only.

Each function takes torch tensors (device memory owned by the caller), checks their
dtype, size and contiguity, and passes raw device pointers plus the current HIP stream
to the C entry point of the same name.  All arithmetic runs in the HIP kernels; if
libmoe.so is missing every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
MOE_SOFTMAX, MOE_SIGMOID, MOE_SQRTSOFTPLUS = 0, 1, 2
_SCORES = {"softmax": MOE_SOFTMAX, "sigmoid": MOE_SIGMOID, "sqrtsoftplus": MOE_SQRTSOFTPLUS}
# stats[]: aux, MaxVio, empty experts, max count, z-loss, sequence-wise aux loss
MOE_NSTATS = 6
MOE_GLU_SWIGLU, MOE_GLU_CLAMP, MOE_GLU_SITU = 0, 1, 2
_GLUS = {"swiglu": MOE_GLU_SWIGLU, "clamp": MOE_GLU_CLAMP, "situ": MOE_GLU_SITU}

EXPORTED = (
    "moe_status_string", "moe_last_error", "moe_validate", "moe_workspace_size", "moe_gate_logits",
    "moe_router_topk", "moe_permute", "moe_grouped_gemm_swiglu", "moe_unpermute_combine", "moe_layer_fwd",
    "moe_unpermute_combine_bwd", "moe_grouped_gemm_swiglu_bwd", "moe_grouped_wgrad", "moe_permute_bwd", "moe_router_bwd",
    "moe_quantize_fp8", "moe_permute_fp8", "moe_grouped_gemm_swiglu_fp8",
    "moe_gate_logits_bwd", "moe_layer_bwd", "moe_expert_bias_update", "moe_router_quantile",
    "moe_quantile_bias_update", "moe_shared_gate", "moe_shared_gate_bwd", "moe_router_topk_noalloc",
)


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libmoe status {status}: {msg}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("F", ctypes.c_int32), ("Fs", ctypes.c_int32), ("score", ctypes.c_int32),
                ("pre_softmax", ctypes.c_int32), ("routed_scaling", ctypes.c_float), ("aux_coeff", ctypes.c_float),
                ("act_dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32), ("z_coeff", ctypes.c_float),
                ("seq_aux_coeff", ctypes.c_float), ("seq_len", ctypes.c_int32), ("wgrad_dtype", ctypes.c_int32),
                ("glu_kind", ctypes.c_int32), ("glu_c", ctypes.c_float), ("glu_c_linear", ctypes.c_float),
                ("num_groups", ctypes.c_int32), ("group_topk", ctypes.c_int32), ("shared_gate", ctypes.c_int32)]


_P = ctypes.c_void_p


class Weights(ctypes.Structure):
    _fields_ = [("Wg", _P), ("bg", _P), ("expert_bias", _P), ("W13", _P), ("W2", _P), ("W13s", _P), ("W2s", _P),
                ("W13_scale", _P), ("W2_scale", _P), ("Wsg", _P)]


class Saved(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("logits", "idx", "w", "counts", "offsets", "row_of", "token_of", "x_perm", "H",
                                  "Act", "Y_perm", "H_s", "Act_s", "Y_s", "x_perm_scale", "Act_scale",
                                  "seq_counts", "gs")]


class Grads(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("dWg", "dbg", "dW13", "dW2", "dW13s", "dW2s", "dWsg")] + [
        ("accumulate", ctypes.c_int32)]


_lib = None


def load() -> ctypes.CDLL:
    """Loads libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m mixture_experts_layer_aux_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        lib.moe_status_string.restype = ctypes.c_char_p
        lib.moe_status_string.argtypes = [ctypes.c_int]
        lib.moe_last_error.restype = ctypes.c_char_p
        lib.moe_last_error.argtypes = []
        for name in EXPORTED[2:]:
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
    return _lib


def _check(status: int) -> None:
    if status != MOE_OK:
        lib = load()
        raise MoeError(status, f"{lib.moe_status_string(status).decode()}: {lib.moe_last_error().decode()}")


def make_config(T, d, E, k, F, Fs=0, score="softmax", scaling=1.0, aux_coeff=0.0, act="bf16", wq="",
                pre_softmax=False, z_coeff=0.0, seq_aux_coeff=0.0, seq_len=0, wgrad=None,
                glu="swiglu", glu_c=0.0, glu_c_linear=0.0, num_groups=0, group_topk=0, shared_gate=False) -> Config:
    """wq: "" (expert weights in the activation dtype) or "fp8" (e4m3 codes + block scales).
    wgrad: dtype of the expert weight gradients, "bf16" or "f32"; None = the activation dtype.
    glu: the experts' gated activation, "swiglu", "clamp" (limit glu_c) or "situ" (gate cap
    glu_c, up cap glu_c_linear, 0 = none)."""
    wgrad = act if wgrad is None else wgrad
    return Config(T=T, d=d, E=E, k=k, F=F, Fs=Fs, score=_SCORES[score], pre_softmax=int(bool(pre_softmax)),
                  routed_scaling=scaling, aux_coeff=aux_coeff, act_dtype=MOE_BF16 if act == "bf16" else MOE_F32,
                  w_dtype=MOE_FP8_E4M3 if wq == "fp8" else 0, z_coeff=z_coeff, seq_aux_coeff=seq_aux_coeff,
                  seq_len=seq_len, wgrad_dtype=MOE_BF16 if wgrad == "bf16" else MOE_F32, glu_kind=_GLUS[glu],
                  glu_c=glu_c, glu_c_linear=glu_c_linear, num_groups=num_groups, group_topk=group_topk,
                  shared_gate=int(bool(shared_gate)))


def config_from_shape(s, **extra) -> Config:
    kw = dict(pre_softmax=getattr(s, "pre_softmax", False), z_coeff=getattr(s, "z_coeff", 0.0),
              seq_aux_coeff=getattr(s, "seq_aux_coeff", 0.0), seq_len=getattr(s, "seq_len", 0),
              glu=getattr(s, "glu", "swiglu"), glu_c=getattr(s, "glu_c", 0.0),
              glu_c_linear=getattr(s, "glu_c_linear", 0.0), num_groups=getattr(s, "num_groups", 0),
              group_topk=getattr(s, "group_topk", 0), shared_gate=getattr(s, "shared_gate", False))
    kw.update(extra)
    return make_config(s.T, s.d, s.E, s.k, s.F, s.Fs, s.score, s.scaling, s.aux_coeff, s.act, getattr(s, "wq", ""),
                       **kw)


def num_sequences(cfg: Config) -> int:
    """B of the sequence-wise loss (0 when it is off)."""
    return cfg.T // cfg.seq_len if cfg.seq_aux_coeff != 0.0 and cfg.seq_len > 0 else 0


def is_fp8(cfg: Config) -> bool:
    return cfg.w_dtype == MOE_FP8_E4M3


def act_dtype(cfg: Config) -> torch.dtype:
    return torch.bfloat16 if cfg.act_dtype == MOE_BF16 else torch.float32


def wgrad_dtype(cfg: Config) -> torch.dtype:
    """torch dtype of the expert weight gradients."""
    return torch.bfloat16 if cfg.wgrad_dtype == MOE_BF16 else torch.float32


def validate(cfg: Config) -> None:
    _check(load().moe_validate(ctypes.byref(cfg)))


def workspace_size(cfg: Config) -> Tuple[int, int]:
    f, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(load().moe_workspace_size(ctypes.byref(cfg), ctypes.byref(f), ctypes.byref(b)))
    return f.value, b.value


# ----------------------------------------------------------------- marshalling helpers

def _ptr(t: Optional[torch.Tensor], dtype=None, numel=None, name="tensor") -> Optional[int]:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return t.data_ptr()


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ws(ws: torch.Tensor) -> Tuple[int, int]:
    return _ptr(ws, torch.uint8, name="ws"), ws.numel()


# ----------------------------------------------------------------- entry points

def gate_logits(cfg, x, Wg, bg, logits, ws, stream=None):
    ad = act_dtype(cfg)
    wp, wn = _ws(ws)
    _check(load().moe_gate_logits(ctypes.byref(cfg), _P(_ptr(x, ad, cfg.T * cfg.d, "x")),
                                  _P(_ptr(Wg, torch.float32, cfg.E * cfg.d, "Wg")),
                                  _P(_ptr(bg, torch.float32, cfg.E, "bg")),
                                  _P(_ptr(logits, torch.float32, cfg.T * cfg.E, "logits")), _P(wp), ctypes.c_size_t(wn),
                                  _P(_stream(stream))))


def router_topk(cfg, logits, expert_bias, idx, w, counts, prob_sum, stats, ws, stream=None, seq_counts=None):
    wp, wn = _ws(ws)
    TK = cfg.T * cfg.k
    nsc = num_sequences(cfg) * cfg.E
    _check(load().moe_router_topk(ctypes.byref(cfg), _P(_ptr(logits, torch.float32, cfg.T * cfg.E, "logits")),
                                  _P(_ptr(expert_bias, torch.float32, cfg.E, "expert_bias")),
                                  _P(_ptr(idx, torch.int32, TK, "idx")), _P(_ptr(w, torch.float32, TK, "w")),
                                  _P(_ptr(counts, torch.int32, cfg.E, "counts")),
                                  _P(_ptr(prob_sum, torch.float32, cfg.E, "prob_sum")),
                                  _P(_ptr(stats, torch.float32, MOE_NSTATS, "stats")),
                                  _P(_ptr(seq_counts, torch.int32, nsc, "seq_counts")), _P(wp), ctypes.c_size_t(wn),
                                  _P(_stream(stream))))


def router_topk_noalloc(cfg, logits, expert_bias, idx, w, counts, prob_sum, stats, stream=None, seq_counts=None):
    """moe_router_topk with the library's static scratch instead of a workspace."""
    TK = cfg.T * cfg.k
    nsc = num_sequences(cfg) * cfg.E
    _check(load().moe_router_topk_noalloc(ctypes.byref(cfg), _P(_ptr(logits, torch.float32, cfg.T * cfg.E, "logits")),
                                          _P(_ptr(expert_bias, torch.float32, cfg.E, "expert_bias")),
                                          _P(_ptr(idx, torch.int32, TK, "idx")), _P(_ptr(w, torch.float32, TK, "w")),
                                          _P(_ptr(counts, torch.int32, cfg.E, "counts")),
                                          _P(_ptr(prob_sum, torch.float32, cfg.E, "prob_sum")),
                                          _P(_ptr(stats, torch.float32, MOE_NSTATS, "stats")),
                                          _P(_ptr(seq_counts, torch.int32, nsc, "seq_counts")), _P(_stream(stream))))


def expert_bias_update(cfg, counts, rate, centered, expert_bias, stream=None):
    _check(load().moe_expert_bias_update(ctypes.byref(cfg), _P(_ptr(counts, torch.int32, cfg.E, "counts")),
                                         ctypes.c_float(rate), ctypes.c_int32(int(bool(centered))),
                                         _P(_ptr(expert_bias, torch.float32, cfg.E, "expert_bias")),
                                         _P(_stream(stream))))


def router_quantile(cfg, scores, beta, idx, alpha, beta_local, ws, stream=None):
    """Quantile balancing of one micro-batch: idx, alpha and (unless beta_local is None) the
    solved bias."""
    wp, wn = _ws(ws)
    T, E, k = cfg.T, cfg.E, cfg.k
    _check(load().moe_router_quantile(ctypes.byref(cfg), _P(_ptr(scores, torch.float32, T * E, "scores")),
                                      _P(_ptr(beta, torch.float32, E, "beta")), _P(_ptr(idx, torch.int32, T * k, "idx")),
                                      _P(_ptr(alpha, torch.float32, T, "alpha")),
                                      _P(_ptr(beta_local, torch.float32, E, "beta_local")), _P(wp),
                                      ctypes.c_size_t(wn), _P(_stream(stream))))


def quantile_bias_update(cfg, beta_local, ema, beta, stream=None):
    _check(load().moe_quantile_bias_update(ctypes.byref(cfg), _P(_ptr(beta_local, torch.float32, cfg.E, "beta_local")),
                                           ctypes.c_float(ema), _P(_ptr(beta, torch.float32, cfg.E, "beta")),
                                           _P(_stream(stream))))


def permute(cfg, x, idx, offsets, row_of, token_of, x_perm, ws, stream=None):
    """The grouping (offsets, row_of, token_of) and, when x_perm is given, the grouped copy
    of x; x_perm None: the grouping only (x may be None too)."""
    ad, TK = act_dtype(cfg), cfg.T * cfg.k
    wp, wn = _ws(ws)
    _check(load().moe_permute(ctypes.byref(cfg), _P(_ptr(x, ad, cfg.T * cfg.d, "x")),
                              _P(_ptr(idx, torch.int32, TK, "idx")), _P(_ptr(offsets, torch.int32, cfg.E + 1, "offsets")),
                              _P(_ptr(row_of, torch.int32, TK, "row_of")), _P(_ptr(token_of, torch.int32, TK, "token_of")),
                              _P(_ptr(x_perm, ad, TK * cfg.d, "x_perm")), _P(wp), ctypes.c_size_t(wn),
                              _P(_stream(stream))))


def grouped_gemm_swiglu(cfg, x_perm, offsets, W13, W2, x, W13s, W2s, H, Act, Y_perm, H_s, Act_s, Y_s, ws,
                        stream=None, token_of=None):
    """token_of given (x_perm None): the routed fc1 reads row token_of[r] of x."""
    ad, A, T, d, E, F, Fs = act_dtype(cfg), cfg.T * cfg.k, cfg.T, cfg.d, cfg.E, cfg.F, cfg.Fs
    wp, wn = _ws(ws)
    _check(load().moe_grouped_gemm_swiglu(
        ctypes.byref(cfg), _P(_ptr(x_perm, ad, A * d, "x_perm")), _P(_ptr(token_of, torch.int32, A, "token_of")),
        _P(_ptr(offsets, torch.int32, E + 1, "offsets")),
        _P(_ptr(W13, ad, E * 2 * F * d, "W13")), _P(_ptr(W2, ad, E * d * F, "W2")),
        _P(_ptr(x, ad, T * d, "x")), _P(_ptr(W13s, ad, 2 * Fs * d, "W13s")), _P(_ptr(W2s, ad, d * Fs, "W2s")),
        _P(_ptr(H, torch.float32, A * 2 * F, "H")), _P(_ptr(Act, ad, A * F, "Act")),
        _P(_ptr(Y_perm, torch.float32, A * d, "Y_perm")),
        _P(_ptr(H_s, torch.float32, T * 2 * Fs, "H_s")), _P(_ptr(Act_s, ad, T * Fs, "Act_s")),
        _P(_ptr(Y_s, torch.float32, T * d, "Y_s")),
        _P(wp), ctypes.c_size_t(wn), _P(_stream(stream))))


def unpermute_combine(cfg, Y_perm, row_of, w, Y_s, y, stream=None, gs=None):
    A, f32 = cfg.T * cfg.k, torch.float32
    _check(load().moe_unpermute_combine(ctypes.byref(cfg), _P(_ptr(Y_perm, f32, A * cfg.d, "Y_perm")),
                                        _P(_ptr(row_of, torch.int32, A, "row_of")), _P(_ptr(w, f32, A, "w")),
                                        _P(_ptr(Y_s, f32, cfg.T * cfg.d, "Y_s")), _P(_ptr(gs, f32, cfg.T, "gs")),
                                        _P(_ptr(y, f32, cfg.T * cfg.d, "y")), _P(_stream(stream))))


def shared_gate(cfg, x, Wsg, gs, stream=None):
    """gs = sigmoid(x Wsg): the shared expert's gate."""
    _check(load().moe_shared_gate(ctypes.byref(cfg), _P(_ptr(x, act_dtype(cfg), cfg.T * cfg.d, "x")),
                                  _P(_ptr(Wsg, torch.float32, cfg.d, "Wsg")), _P(_ptr(gs, torch.float32, cfg.T, "gs")),
                                  _P(_stream(stream))))


def shared_gate_bwd(cfg, x, dl_s, dWsg, ws, stream=None):
    wp, wn = _ws(ws)
    _check(load().moe_shared_gate_bwd(ctypes.byref(cfg), _P(_ptr(x, act_dtype(cfg), cfg.T * cfg.d, "x")),
                                      _P(_ptr(dl_s, torch.float32, cfg.T, "dl_s")),
                                      _P(_ptr(dWsg, torch.float32, cfg.d, "dWsg")), _P(wp), ctypes.c_size_t(wn),
                                      _P(_stream(stream))))


def unpermute_combine_bwd(cfg, dy, Y_perm, row_of, w, dY_perm, dw, dY_s=None, stream=None, gs=None, Y_s=None,
                          dl_s=None):
    ad, A, f32 = act_dtype(cfg), cfg.T * cfg.k, torch.float32
    _check(load().moe_unpermute_combine_bwd(ctypes.byref(cfg), _P(_ptr(dy, f32, cfg.T * cfg.d, "dy")),
                                            _P(_ptr(Y_perm, f32, A * cfg.d, "Y_perm")),
                                            _P(_ptr(row_of, torch.int32, A, "row_of")),
                                            _P(_ptr(w, f32, A, "w")),
                                            _P(_ptr(dY_perm, ad, A * cfg.d, "dY_perm")),
                                            _P(_ptr(dw, f32, A, "dw")), _P(_ptr(dY_s, ad, cfg.T * cfg.d, "dY_s")),
                                            _P(_ptr(gs, f32, cfg.T, "gs")), _P(_ptr(Y_s, f32, cfg.T * cfg.d, "Y_s")),
                                            _P(_ptr(dl_s, f32, cfg.T, "dl_s")), _P(_stream(stream))))


def grouped_gemm_swiglu_bwd(cfg, x_perm, offsets, W13, W2, H, Act, dY_perm, dH, dX_perm, dW13, dW2, x, W13s, W2s,
                            H_s, Act_s, dY_s, dH_s, dx_s, dW13s, dW2s, ws, stream=None, token_of=None):
    """token_of given (x_perm None): the routed dW13 reads row token_of[r] of x."""
    ad, A, T, d, E, F, Fs = act_dtype(cfg), cfg.T * cfg.k, cfg.T, cfg.d, cfg.E, cfg.F, cfg.Fs
    wp, wn = _ws(ws)
    _check(load().moe_grouped_gemm_swiglu_bwd(
        ctypes.byref(cfg), _P(_ptr(x_perm, ad, A * d, "x_perm")), _P(_ptr(token_of, torch.int32, A, "token_of")),
        _P(_ptr(offsets, torch.int32, E + 1, "offsets")),
        _P(_ptr(W13, ad, E * 2 * F * d, "W13")), _P(_ptr(W2, ad, E * d * F, "W2")),
        _P(_ptr(H, torch.float32, A * 2 * F, "H")),
        _P(_ptr(Act, ad, A * F, "Act")), _P(_ptr(dY_perm, ad, A * d, "dY_perm")), _P(_ptr(dH, ad, A * 2 * F, "dH")),
        _P(_ptr(dX_perm, torch.float32, A * d, "dX_perm")), _P(_ptr(dW13, wgrad_dtype(cfg), E * 2 * F * d, "dW13")),
        _P(_ptr(dW2, wgrad_dtype(cfg), E * d * F, "dW2")), _P(_ptr(x, ad, T * d, "x")),
        _P(_ptr(W13s, ad, 2 * Fs * d, "W13s")),
        _P(_ptr(W2s, ad, d * Fs, "W2s")), _P(_ptr(H_s, torch.float32, T * 2 * Fs, "H_s")),
        _P(_ptr(Act_s, ad, T * Fs, "Act_s")),
        _P(_ptr(dY_s, ad, T * d, "dY_s")), _P(_ptr(dH_s, ad, T * 2 * Fs, "dH_s")), _P(_ptr(dx_s, torch.float32, T * d, "dx_s")),
        _P(_ptr(dW13s, wgrad_dtype(cfg), 2 * Fs * d, "dW13s")), _P(_ptr(dW2s, wgrad_dtype(cfg), d * Fs, "dW2s")),
        _P(wp),
        ctypes.c_size_t(wn),
        _P(_stream(stream))))


def grouped_wgrad(cfg, offsets, groups, rows, dY, N, X, K, dW, stream=None, accumulate=False, ws=None, x_rows=None):
    """dW[g] = dY_g^T X_g per group of rows (offsets None: one group of `rows` rows);
    accumulate: dW[g] += dY_g^T X_g; ws: scratch that lets a one-group call split its rows;
    x_rows [rows] int32: reduction row r of X is row x_rows[r] of X (X then has any number
    of rows)."""
    wp, wn = _ws(ws) if ws is not None else (None, 0)
    ad = act_dtype(cfg)
    if offsets is not None and offsets.numel() != groups + 1:
        raise ValueError(f"offsets: expected {groups + 1} entries, got {offsets.numel()}")
    x_src = X.numel() // K if x_rows is not None else 0
    _check(load().moe_grouped_wgrad(
        ctypes.byref(cfg), _P(_ptr(offsets, torch.int32, groups + 1, "offsets")), ctypes.c_int32(groups),
        ctypes.c_int64(rows), _P(_ptr(dY, ad, rows * N, "dY")), ctypes.c_int32(N),
        _P(_ptr(X, ad, (x_src if x_rows is not None else rows) * K, "X")), ctypes.c_int32(K),
        _P(_ptr(x_rows, torch.int32, rows, "x_rows")), ctypes.c_int32(x_src),
        _P(_ptr(dW, wgrad_dtype(cfg), groups * N * K, "dW")), ctypes.c_int32(int(accumulate)),
        _P(wp), ctypes.c_size_t(wn), _P(_stream(stream))))


def quantize_fp8(src, block_rows, q, scale, stream=None):
    """e4m3 codes q [rows, cols] and fp32 scales [rows / block_rows, cols / 128] of src
    (bf16 or fp32, [rows, cols] contiguous)."""
    if src.dim() != 2:
        raise ValueError("src must be 2-D")
    rows, cols = src.shape
    sd = MOE_BF16 if src.dtype == torch.bfloat16 else MOE_F32
    _check(load().moe_quantize_fp8(
        ctypes.c_int32(sd), _P(_ptr(src, src.dtype, rows * cols, "src")), ctypes.c_int64(rows), ctypes.c_int32(cols),
        ctypes.c_int32(block_rows), _P(_ptr(q, torch.uint8, rows * cols, "q")),
        _P(_ptr(scale, torch.float32, (rows // max(block_rows, 1)) * (cols // 128), "scale")), _P(_stream(stream))))


def permute_fp8(cfg, x_q, x_scale, idx, offsets, row_of, token_of, x_perm, x_perm_scale, ws, stream=None):
    """x_perm and x_perm_scale None: the grouping only."""
    A, T, d, E = cfg.T * cfg.k, cfg.T, cfg.d, cfg.E
    wp, wn = _ws(ws)
    _check(load().moe_permute_fp8(
        ctypes.byref(cfg), _P(_ptr(x_q, torch.uint8, T * d, "x_q")), _P(_ptr(x_scale, torch.float32, T * (d // 128), "x_scale")),
        _P(_ptr(idx, torch.int32, A, "idx")), _P(_ptr(offsets, torch.int32, E + 1, "offsets")),
        _P(_ptr(row_of, torch.int32, A, "row_of")), _P(_ptr(token_of, torch.int32, A, "token_of")),
        _P(_ptr(x_perm, torch.uint8, A * d, "x_perm")), _P(_ptr(x_perm_scale, torch.float32, A * (d // 128), "x_perm_scale")),
        _P(wp), ctypes.c_size_t(wn), _P(_stream(stream))))


def grouped_gemm_swiglu_fp8(cfg, x_perm, x_perm_scale, offsets, W13, W13_scale, W2, W2_scale, H, Act, Act_scale,
                            Y_perm, ws, stream=None, token_of=None):
    """token_of given: x_perm, x_perm_scale are the token rows x_q [T, d], x_scale [T, d/128],
    read through token_of."""
    A, d, E, F = cfg.T * cfg.k, cfg.d, cfg.E, cfg.F
    R = cfg.T if token_of is not None else A
    wp, wn = _ws(ws)
    u8, f32 = torch.uint8, torch.float32
    _check(load().moe_grouped_gemm_swiglu_fp8(
        ctypes.byref(cfg), _P(_ptr(x_perm, u8, R * d, "x_perm")), _P(_ptr(x_perm_scale, f32, R * (d // 128), "x_perm_scale")),
        _P(_ptr(token_of, torch.int32, A, "token_of")), _P(_ptr(offsets, torch.int32, E + 1, "offsets")), _P(_ptr(W13, u8, E * 2 * F * d, "W13")),
        _P(_ptr(W13_scale, f32, E * (2 * F // 128) * (d // 128), "W13_scale")), _P(_ptr(W2, u8, E * d * F, "W2")),
        _P(_ptr(W2_scale, f32, E * (d // 128) * (F // 128), "W2_scale")), _P(_ptr(H, f32, A * 2 * F, "H")),
        _P(_ptr(Act, u8, A * F, "Act")), _P(_ptr(Act_scale, f32, A * (F // 128), "Act_scale")),
        _P(_ptr(Y_perm, f32, A * d, "Y_perm")), _P(wp), ctypes.c_size_t(wn), _P(_stream(stream))))


def permute_bwd(cfg, dX_perm, row_of, dx_s, dx_r, dx, stream=None, dl_s=None, Wsg=None):
    ad, A = act_dtype(cfg), cfg.T * cfg.k
    _check(load().moe_permute_bwd(ctypes.byref(cfg), _P(_ptr(dX_perm, torch.float32, A * cfg.d, "dX_perm")),
                                  _P(_ptr(row_of, torch.int32, A, "row_of")),
                                  _P(_ptr(dx_s, torch.float32, cfg.T * cfg.d, "dx_s")),
                                  _P(_ptr(dx_r, torch.float32, cfg.T * cfg.d, "dx_r")),
                                  _P(_ptr(dl_s, torch.float32, cfg.T, "dl_s")), _P(_ptr(Wsg, torch.float32, cfg.d, "Wsg")),
                                  _P(_ptr(dx, torch.float32, cfg.T * cfg.d, "dx")), _P(_stream(stream))))


def router_bwd(cfg, logits, idx, w, dw, counts, daux, dlogits, stream=None, seq_counts=None):
    A = cfg.T * cfg.k
    _check(load().moe_router_bwd(ctypes.byref(cfg), _P(_ptr(logits, torch.float32, cfg.T * cfg.E, "logits")),
                                 _P(_ptr(idx, torch.int32, A, "idx")), _P(_ptr(w, torch.float32, A, "w")),
                                 _P(_ptr(dw, torch.float32, A, "dw")), _P(_ptr(counts, torch.int32, cfg.E, "counts")),
                                 _P(_ptr(seq_counts, torch.int32, num_sequences(cfg) * cfg.E, "seq_counts")),
                                 ctypes.c_float(daux), _P(_ptr(dlogits, torch.float32, cfg.T * cfg.E, "dlogits")),
                                 _P(_stream(stream))))


def gate_logits_bwd(cfg, x, Wg, dlogits, dWg, dbg, dx_r, ws, stream=None):
    ad = act_dtype(cfg)
    wp, wn = _ws(ws)
    _check(load().moe_gate_logits_bwd(ctypes.byref(cfg), _P(_ptr(x, ad, cfg.T * cfg.d, "x")),
                                      _P(_ptr(Wg, torch.float32, cfg.E * cfg.d, "Wg")),
                                      _P(_ptr(dlogits, torch.float32, cfg.T * cfg.E, "dlogits")),
                                      _P(_ptr(dWg, torch.float32, cfg.E * cfg.d, "dWg")),
                                      _P(_ptr(dbg, torch.float32, cfg.E, "dbg")),
                                      _P(_ptr(dx_r, torch.float32, cfg.T * cfg.d, "dx_r")), _P(wp),
                                      ctypes.c_size_t(wn), _P(_stream(stream))))


def _weights_struct(cfg, W: Dict[str, torch.Tensor]) -> Weights:
    ad, d, E, F, Fs = act_dtype(cfg), cfg.d, cfg.E, cfg.F, cfg.Fs
    wd = torch.uint8 if is_fp8(cfg) else ad
    return Weights(Wg=_ptr(W["Wg"], torch.float32, E * d, "Wg"), bg=_ptr(W.get("bg"), torch.float32, E, "bg"),
                   expert_bias=_ptr(W.get("expert_bias"), torch.float32, E, "expert_bias"),
                   W13=_ptr(W["W13"], wd, E * 2 * F * d, "W13"), W2=_ptr(W["W2"], wd, E * d * F, "W2"),
                   W13s=_ptr(W.get("W13s"), ad, 2 * Fs * d, "W13s"), W2s=_ptr(W.get("W2s"), ad, d * Fs, "W2s"),
                   W13_scale=_ptr(W.get("W13_scale"), torch.float32, E * (2 * F // 128) * (d // 128), "W13_scale"),
                   W2_scale=_ptr(W.get("W2_scale"), torch.float32, E * (d // 128) * (F // 128), "W2_scale"),
                   Wsg=_ptr(W.get("Wsg"), torch.float32, d, "Wsg"))


def _saved_struct(cfg, S: Dict[str, torch.Tensor]) -> Saved:
    ad, T, d, E, F, Fs, A = act_dtype(cfg), cfg.T, cfg.d, cfg.E, cfg.F, cfg.Fs, cfg.T * cfg.k
    qd = torch.uint8 if is_fp8(cfg) else ad
    spec = dict(logits=(torch.float32, T * E), idx=(torch.int32, A), w=(torch.float32, A), counts=(torch.int32, E),
                offsets=(torch.int32, E + 1), row_of=(torch.int32, A), token_of=(torch.int32, A),
                x_perm=(qd, A * d), H=(torch.float32, A * 2 * F), Act=(qd, A * F), Y_perm=(torch.float32, A * d),
                H_s=(torch.float32, T * 2 * Fs), Act_s=(ad, T * Fs), Y_s=(torch.float32, T * d),
                x_perm_scale=(torch.float32, A * (d // 128)), Act_scale=(torch.float32, A * (F // 128)),
                seq_counts=(torch.int32, num_sequences(cfg) * E), gs=(torch.float32, T))
    return Saved(**{n: _ptr(S.get(n), dt, ne, n) for n, (dt, ne) in spec.items()})


def layer_fwd(cfg, W, x, S, y, stats, ws, stream=None):
    wp, wn = _ws(ws)
    ad = act_dtype(cfg)
    ws_ = _weights_struct(cfg, W)
    ss = _saved_struct(cfg, S)
    _check(load().moe_layer_fwd(ctypes.byref(cfg), ctypes.byref(ws_), _P(_ptr(x, ad, cfg.T * cfg.d, "x")),
                                ctypes.byref(ss), _P(_ptr(y, torch.float32, cfg.T * cfg.d, "y")),
                                _P(_ptr(stats, torch.float32, MOE_NSTATS, "stats")), _P(wp), ctypes.c_size_t(wn),
                                _P(_stream(stream))))


def layer_bwd(cfg, W, S, x, dy, daux, dx, G, ws, stream=None, accumulate=False, wgrad_stream=None):
    """The layer's backward; accumulate: add the weight gradients into G's buffers;
    wgrad_stream: a second torch stream for the expert weight gradients (None: one stream)."""
    wp, wn = _ws(ws)
    ad, d, E, F, Fs = act_dtype(cfg), cfg.d, cfg.E, cfg.F, cfg.Fs
    ws_ = _weights_struct(cfg, W)
    ss = _saved_struct(cfg, S)
    f32 = torch.float32
    wd = wgrad_dtype(cfg)
    gs = Grads(dWg=_ptr(G["dWg"], f32, E * d, "dWg"), dbg=_ptr(G.get("dbg"), f32, E, "dbg"),
               dW13=_ptr(G.get("dW13"), wd, E * 2 * F * d, "dW13"), dW2=_ptr(G.get("dW2"), wd, E * d * F, "dW2"),
               dW13s=_ptr(G.get("dW13s"), wd, 2 * Fs * d, "dW13s"), dW2s=_ptr(G.get("dW2s"), wd, d * Fs, "dW2s"),
               dWsg=_ptr(G.get("dWsg"), f32, d, "dWsg"), accumulate=int(accumulate))
    _check(load().moe_layer_bwd(ctypes.byref(cfg), ctypes.byref(ws_), ctypes.byref(ss),
                                _P(_ptr(x, ad, cfg.T * d, "x")), _P(_ptr(dy, f32, cfg.T * d, "dy")),
                                ctypes.c_float(daux), _P(_ptr(dx, f32, cfg.T * d, "dx")), ctypes.byref(gs), _P(wp),
                                ctypes.c_size_t(wn), _P(_stream(stream)),
                                _P(wgrad_stream.cuda_stream if wgrad_stream is not None else None)))


# ----------------------------------------------------------------- buffer helpers

def alloc_saved(cfg: Config, device="cuda", x_perm=None) -> Dict[str, torch.Tensor]:
    """Buffers of moe_saved_t.  x_perm: keep the grouped copy of x (default: only with fp32
    activations; bf16 layers read the token rows of x through token_of instead)."""
    ad, T, d, E, F, Fs, A = act_dtype(cfg), cfg.T, cfg.d, cfg.E, cfg.F, cfg.Fs, cfg.T * cfg.k
    e = lambda *s, dt=ad: torch.empty(*s, dtype=dt, device=device)  # noqa: E731
    qd = torch.uint8 if is_fp8(cfg) else ad
    if x_perm is None:
        x_perm = ad != torch.bfloat16
    S = dict(logits=e(T, E, dt=torch.float32), idx=e(T, cfg.k, dt=torch.int32), w=e(T, cfg.k, dt=torch.float32),
             counts=e(E, dt=torch.int32), offsets=e(E + 1, dt=torch.int32), row_of=e(T, cfg.k, dt=torch.int32),
             token_of=e(A, dt=torch.int32), H=e(A, 2 * F, dt=torch.float32),
             Act=e(A, F, dt=qd), Y_perm=e(A, d, dt=torch.float32))
    if x_perm:
        S["x_perm"] = e(A, d, dt=qd)
    if is_fp8(cfg):
        S["Act_scale"] = e(A, F // 128, dt=torch.float32)
        if x_perm:
            S["x_perm_scale"] = e(A, d // 128, dt=torch.float32)
    if Fs:
        S.update(H_s=e(T, 2 * Fs, dt=torch.float32), Act_s=e(T, Fs), Y_s=e(T, d, dt=torch.float32))
    if num_sequences(cfg):
        S["seq_counts"] = e(num_sequences(cfg), E, dt=torch.int32)
    if cfg.shared_gate:
        S["gs"] = e(T, dt=torch.float32)
    return S


def alloc_grads(cfg: Config, device="cuda", with_dbg=False) -> Dict[str, torch.Tensor]:
    d, E, F, Fs, f32, wd = cfg.d, cfg.E, cfg.F, cfg.Fs, torch.float32, wgrad_dtype(cfg)
    G = dict(dWg=torch.empty(E, d, dtype=f32, device=device))
    if not is_fp8(cfg):   # fp8 experts are frozen: no expert weight gradients
        G.update(dW13=torch.empty(E, 2 * F, d, dtype=wd, device=device),
                 dW2=torch.empty(E, d, F, dtype=wd, device=device))
    if with_dbg:
        G["dbg"] = torch.empty(E, dtype=f32, device=device)
    if Fs:
        G.update(dW13s=torch.empty(2 * Fs, d, dtype=wd, device=device), dW2s=torch.empty(d, Fs, dtype=wd, device=device))
    if cfg.shared_gate:
        G["dWsg"] = torch.empty(d, dtype=f32, device=device)
    return G


def alloc_workspace(cfg: Config, device="cuda") -> torch.Tensor:
    f, b = workspace_size(cfg)
    return torch.empty(max(f, b), dtype=torch.uint8, device=device)
