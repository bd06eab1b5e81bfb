"""Parity of the experts' activation variants (The Ultimate MoE Training Handbook, §3.4
Activation): the hard-clamped SwiGLU and SiTU-GLU, in the grouped GEMM epilogues (bf16
matrix cores), the fp32 elementwise kernels and the e4m3 experts' forward, against the
fp64 oracle at each path's usual bar.

The clamp's derivative jumps at its bound, so an element of H within the fp32 accumulation
error of the bound could take the other branch on the two sides (both correct).  H does not
depend on the activation, so these tests place the bound in the middle of the widest gap
among the oracle's gate values and |up| values in a range, and check that the gap leaves a
margin far above that error.
"""
from dataclasses import replace

import numpy as np
import pytest

from helpers import O, W, oracle_inputs, spec_of
from test_gpu_layer import _check_layer
from test_gpu_pieces import check_grouped_experts

pytestmark = pytest.mark.gpu


def _oracle_H(shape, seed):
    """The oracle's H of the routed rows and of the shared expert (independent of the
    activation)."""
    inp = W.make_inputs(shape, seed=seed)
    o = oracle_inputs(inp, shape)
    f = O.layer_forward(o["x"], o["Wg"], o["W13"], o["W2"], spec_of(shape), bg=o["bg"],
                        expert_bias=o["expert_bias"], W13s=o["W13s"], W2s=o["W2s"])
    out = [(f["H"], shape.F)]
    if f["shared"] is not None:
        out.append((f["shared"]["H"], shape.Fs))
    return out


def _bound_in_widest_gap(Hs, lo, hi, need):
    v = np.sort(np.concatenate([np.concatenate([H[:, :F].ravel(), np.abs(H[:, F:]).ravel()]) for H, F in Hs]))
    v = v[(v > lo) & (v < hi)]
    gaps = np.diff(v)
    i = int(np.argmax(gaps))
    c = np.float32((v[i] + v[i + 1]) / 2)
    margin = min(abs(float(c) - v[i]), abs(v[i + 1] - float(c)))
    assert margin > need, f"widest gap leaves a margin of {margin:.2e} only"
    frac = np.mean(np.concatenate([np.concatenate([H[:, :F].ravel(), np.abs(H[:, F:]).ravel()]) for H, F in Hs]) > c)
    assert frac > 0.05, "the bound clamps too few values to test it"
    return float(c)


def test_grouped_experts_clamp_bf16():
    base = W.SMALL[3]
    c = _bound_in_widest_gap(_oracle_H(base, 3), 0.3, 0.8, need=4e-6)
    print(f"clamp bound {c:.7f}", flush=True)
    check_grouped_experts(replace(base, glu="clamp", glu_c=c), 3)


@pytest.mark.parametrize("cl", [1.2, 0.0])
def test_grouped_experts_situ_bf16(cl):
    check_grouped_experts(replace(W.SMALL[3], glu="situ", glu_c=0.7, glu_c_linear=cl), 3)


def test_layer_clamp_fp32():
    base = W.LAYERS[1]
    c = _bound_in_widest_gap(_oracle_H(base, 5), 0.5, 1.0, need=2e-6)
    print(f"clamp bound {c:.7f}", flush=True)
    _check_layer(replace(base, glu="clamp", glu_c=c), seed=5)


def test_layer_situ_bf16_and_fp32():
    _check_layer(replace(W.SMALL[2], glu="situ", glu_c=0.6, glu_c_linear=0.9), seed=2)
    _check_layer(replace(W.LAYERS[1], glu="situ", glu_c=1.5, glu_c_linear=0.0), seed=1)
