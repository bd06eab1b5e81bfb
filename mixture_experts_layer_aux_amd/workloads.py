"""Seeded synthetic inputs for the MoE layer: shapes, value distributions, load shapes.

This module only draws numbers and casts them to the storage dtypes; it holds none of
the layer's arithmetic (no routing, no GEMM, no quantiser rule beyond the cast of
inputs).  Both the fp64 oracle (via the tests) and the HIP path consume the bytes it
returns, so the two sides are always fed identical inputs.

Recipe (one independent PCG64 stream per tensor chunk, so any tensor or any single
expert's weights can be regenerated alone and generation can run on many threads
with a result that does not depend on the thread count):

  stream(seed, tensor_id, chunk) = Generator(PCG64(SeedSequence(seed, spawn_key=(tensor_id, chunk))))

  x      [T, d]     ~ N(0, 1)                                  (row chunks of 256 rows)
  Wg     [E, d]     ~ N(0, std_w) fp32 (router weight kept fp32; The Ultimate MoE
                                        Training Handbook, §3.4 Count and size, the
                                        fp32 gate parameter)
  W13[e] [2F, d]    ~ N(0, std_w) (gate rows, then up rows), one stream per expert
  W2[e]  [d, F]     ~ N(0, std_w), one stream per expert
  W13s   [2Fs, d], W2s [d, Fs]   shared expert, same law
  dy     [T, d]     ~ N(0, 1)   upstream gradient
  std_w  = 1/sqrt(fan_in) for the tiny fp32 layer, 0.02 for every other layer.

Selection biases (all fp32):
  * expert_bias[e] ~ N(0, 0.1)  (sigmoid router; bias enters selection only)
  * zipf:  bg[e] = -1.1 * ln(r_e), r = a seeded permutation of 1..E (a Zipf(1.1) prior
    on the softmax scores, giving a long-tailed load with empty experts)
  * skew:  bg[e] = -30 for a seeded 5% of experts (they go empty), +beta for one
    seeded hot expert, 0 elsewhere.

Casts: fp32 masters are rounded to bfloat16 with round-to-nearest-even; the bf16
arrays are returned as uint16 bit patterns.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace
from typing import Dict, Optional

import numpy as np

# tensor ids of the independent streams
_TID_X, _TID_WG, _TID_BIAS, _TID_W13, _TID_W2, _TID_W13S, _TID_W2S, _TID_DY, _TID_LOGITS, _TID_AUX, _TID_WSG = range(11)
_ROW_CHUNK = 256


@dataclass(frozen=True)
class LayerShape:
    name: str
    T: int
    d: int
    E: int
    k: int
    F: int
    Fs: int = 0                 # shared-expert width, 0 = no shared expert
    score: str = "softmax"      # "softmax" (top-k on logits, softmax over the k) | "sigmoid"
    act: str = "bf16"           # activation / expert-weight storage dtype: "f32" | "bf16"
    aux_coeff: float = 0.0
    scaling: float = 1.0        # routed scaling factor
    init: str = "std002"        # "fan_in" | "std002"
    bias: str = "none"          # "none" | "expert_bias" | "zipf" | "skew"
    skew_beta: float = 0.0      # hot-expert logit bias for bias == "skew"
    wq: str = ""                # "fp8": expert weights are given as fp32 masters, to be
                                # quantised to e4m3 in 128 x 128 blocks by each side
    pre_softmax: bool = False   # softmax only: top-k of the full softmax, no renormalisation
    z_coeff: float = 0.0        # router z-loss coefficient
    seq_aux_coeff: float = 0.0  # sequence-wise balance loss coefficient
    seq_len: int = 0            # S of that loss (tokens ordered [S, B])
    glu: str = "swiglu"         # the experts' gated activation: "swiglu" | "clamp" | "situ"
    glu_c: float = 0.0          # clamp: the limit; situ: the gate cap
    glu_c_linear: float = 0.0   # situ: the up cap (0 = none)
    num_groups: int = 0         # group-limited routing: expert groups (0 = off)
    group_topk: int = 0         # groups kept per token
    shared_gate: bool = False   # a sigmoid gate on the shared expert (gate weight Wsg [d], fp32)

    @property
    def A(self) -> int:
        return self.T * self.k


# The five layers.  Their numbers follow the workloads the pages name:
#  - the first MoE of The Ultimate MoE Training Handbook, §2.5 (d=2048, 64 experts,
#    top-8, expert ffn 1024, aux loss) for the small bf16 layer;
#  - the shapes the summary page lists (DeepSeek-V3 1 shared + 256 routed top-8,
#    Qwen3-Next 512 experts, Kimi K3 16-of-896) for the three large layers.
LAYERS: Dict[int, LayerShape] = {
    1: LayerShape("tiny-fp32", T=128, d=64, E=8, k=2, F=128, Fs=0, score="softmax",
                  act="f32", aux_coeff=1.0, init="fan_in"),
    2: LayerShape("small-bf16", T=8192, d=2048, E=64, k=8, F=1024, Fs=0, score="softmax",
                  act="bf16", aux_coeff=1e-2),
    3: LayerShape("deepseek-v3-shaped-bf16", T=16384, d=7168, E=256, k=8, F=2048, Fs=2048,
                  score="sigmoid", act="bf16", aux_coeff=0.0, bias="expert_bias"),
    4: LayerShape("qwen3-next-shaped-bf16", T=32768, d=2048, E=512, k=10, F=512, Fs=512,
                  score="softmax", act="bf16", aux_coeff=0.0, bias="zipf"),
    5: LayerShape("skewed-896x16-fp8", T=16384, d=4096, E=896, k=16, F=512, Fs=0,
                  score="softmax", act="bf16", aux_coeff=0.0, bias="skew", skew_beta=1.46, wq="fp8"),
}

# Reduced layers with the same router, bias law and dtype as the full ones, at sizes the
# fp64 oracle finishes in seconds while still spanning several GEMM tiles (256 x 256
# output tiles, 64-deep K steps) and a ragged tail in every expert.
SMALL: Dict[int, LayerShape] = {
    1: LAYERS[1],
    2: replace(LAYERS[2], name="small-bf16-reduced", T=1024, d=512, E=16, k=4, F=384),
    3: replace(LAYERS[3], name="deepseek-v3-shaped-reduced", T=1024, d=768, E=32, k=8,
               F=256, Fs=384),
    4: replace(LAYERS[4], name="qwen3-next-shaped-reduced", T=2048, d=512, E=64, k=10,
               F=128, Fs=256),
    5: replace(LAYERS[5], name="skewed-reduced-bf16", T=1024, d=512, E=112, k=16, F=128, wq=""),
}
# The skewed layer with its e4m3 experts, at the reduced size.
SMALL_FP8 = replace(LAYERS[5], name="skewed-reduced-fp8", T=1024, d=512, E=112, k=16, F=128)


def _stream(seed: int, tid: int, chunk: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tid, chunk))))


def _threads(threads: Optional[int]) -> int:
    if threads:
        return threads
    return max(1, min(16, os.cpu_count() or 1))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _cast(a32: np.ndarray, act: str) -> np.ndarray:
    if act == "f32":
        return a32.astype(np.float32, copy=False)
    if act == "bf16":
        return f32_to_bf16_bits(a32)
    raise ValueError(act)


def _normal_rows(seed: int, tid: int, rows: int, cols: int, std: float, act: str,
                 pool: ThreadPoolExecutor) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.float32 if act == "f32" else np.uint16)

    def work(c: int) -> None:
        r0, r1 = c * _ROW_CHUNK, min(rows, (c + 1) * _ROW_CHUNK)
        g = _stream(seed, tid, c)
        v = g.standard_normal((r1 - r0, cols), dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        out[r0:r1] = _cast(v, act)

    list(pool.map(work, range((rows + _ROW_CHUNK - 1) // _ROW_CHUNK)))
    return out


def _expert_stack(seed: int, tid: int, E: int, rows: int, cols: int, std: float, act: str,
                  pool: ThreadPoolExecutor, experts=None) -> np.ndarray:
    ids = range(E) if experts is None else list(experts)
    out = np.empty((len(ids), rows, cols), dtype=np.float32 if act == "f32" else np.uint16)

    def work(i_e):
        i, e = i_e
        v = _stream(seed, tid, e).standard_normal((rows, cols), dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        out[i] = _cast(v, act)

    list(pool.map(work, enumerate(ids)))
    return out


def weight_std(shape: LayerShape, fan_in: int) -> float:
    return float(1.0 / np.sqrt(fan_in)) if shape.init == "fan_in" else 0.02


def selection_bias(shape: LayerShape, seed: int):
    """Returns (bg, expert_bias): the additive logit bias and the selection-only bias."""
    E = shape.E
    if shape.bias == "none":
        return None, None
    g = _stream(seed, _TID_BIAS)
    if shape.bias == "expert_bias":
        return None, (g.standard_normal(E, dtype=np.float32) * np.float32(0.1)).astype(np.float32)
    if shape.bias == "zipf":
        r = g.permutation(E) + 1
        return (-1.1 * np.log(r.astype(np.float64))).astype(np.float32), None
    if shape.bias == "skew":
        perm = g.permutation(E)
        n_dead = max(1, int(round(0.05 * E)))
        bg = np.zeros(E, dtype=np.float32)
        bg[perm[:n_dead]] = -30.0
        bg[perm[n_dead]] = np.float32(shape.skew_beta)
        return bg, None
    raise ValueError(shape.bias)


def make_inputs(shape: LayerShape, seed: int, with_dy: bool = True, threads: Optional[int] = None,
                with_experts: bool = True) -> Dict[str, np.ndarray]:
    """All inputs of one layer call, as numpy arrays in their storage dtypes."""
    T, d, E, F, Fs, act = shape.T, shape.d, shape.E, shape.F, shape.Fs, shape.act
    with ThreadPoolExecutor(_threads(threads)) as pool:
        out: Dict[str, np.ndarray] = {}
        out["x"] = _normal_rows(seed, _TID_X, T, d, 1.0, act, pool)
        out["Wg"] = _normal_rows(seed, _TID_WG, E, d, weight_std(shape, d), "f32", pool)
        bg, eb = selection_bias(shape, seed)
        out["bg"], out["expert_bias"] = bg, eb
        if with_experts:
            wact = "f32" if shape.wq == "fp8" else act     # fp8 experts: fp32 masters
            out["W13"] = _expert_stack(seed, _TID_W13, E, 2 * F, d, weight_std(shape, d), wact, pool)
            out["W2"] = _expert_stack(seed, _TID_W2, E, d, F, weight_std(shape, F), wact, pool)
            if Fs:
                out["W13s"] = _normal_rows(seed, _TID_W13S, 2 * Fs, d, weight_std(shape, d), act, pool)
                out["W2s"] = _normal_rows(seed, _TID_W2S, d, Fs, weight_std(shape, Fs), act, pool)
                out["Wsg"] = (_normal_rows(seed, _TID_WSG, 1, d, weight_std(shape, d), "f32", pool)[0]
                              if shape.shared_gate else None)
            else:
                out["W13s"] = out["W2s"] = out["Wsg"] = None
        if with_dy:
            out["dy"] = _normal_rows(seed, _TID_DY, T, d, 1.0, act, pool)
    return out


def expert_weights(shape: LayerShape, seed: int, experts, threads: Optional[int] = None):
    """Regenerates the routed weights of only the listed experts (same bytes as make_inputs)."""
    d, F = shape.d, shape.F
    with ThreadPoolExecutor(_threads(threads)) as pool:
        wact = "f32" if shape.wq == "fp8" else shape.act
        W13 = _expert_stack(seed, _TID_W13, shape.E, 2 * F, d, weight_std(shape, d), wact, pool, experts)
        W2 = _expert_stack(seed, _TID_W2, shape.E, d, F, weight_std(shape, F), wact, pool, experts)
    return W13, W2


def random_logits(T: int, E: int, seed: int, std: float = 1.0) -> np.ndarray:
    """Plain N(0, std) fp32 logits, for feeding the router alone."""
    return (_stream(seed, _TID_LOGITS).standard_normal((T, E), dtype=np.float32) * np.float32(std))


def random_rows(T: int, n: int, seed: int, tid_offset: int = 0, act: str = "f32") -> np.ndarray:
    """Plain N(0,1) rows in the given storage dtype (generic operand for single-step tests)."""
    v = _stream(seed, _TID_AUX, tid_offset).standard_normal((T, n), dtype=np.float32)
    return _cast(v, act)


def to_f32(a: Optional[np.ndarray], act: str) -> Optional[np.ndarray]:
    """Storage bytes -> fp32 values (exact)."""
    if a is None:
        return None
    if act == "bf16" and a.dtype == np.uint16:
        return bf16_bits_to_f32(a)
    return a.astype(np.float32, copy=False)


class ExpertView:
    """Per-expert fp32 view of a stacked expert-weight array, converted on access
    (lets a CPU consumer walk a large bf16 stack one expert at a time)."""

    def __init__(self, stack: np.ndarray, act: str):
        self.stack, self.act = stack, act

    def __len__(self) -> int:
        return self.stack.shape[0]

    def __getitem__(self, e: int) -> np.ndarray:
        return to_f32(self.stack[e], self.act)
