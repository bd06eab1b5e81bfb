"""Pins of the fp64 oracle against things other than itself.

Each test pins one oracle function to a value the pages print (fixtures under
tests/golden/), a closed form, brute force, an independent library routine, or central
finite differences, chosen so that a dropped term, a wrong sign or index, or a
transposed operand anywhere in the oracle fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import expit

from oracle import moe_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _ffn_torch(x, W13, W2):
    """Dense bias-free SwiGLU FFN via torch's own silu and linear, in float64."""
    x, W13, W2 = (torch.as_tensor(np.asarray(a, dtype=np.float64)) for a in (x, W13, W2))
    F = W13.shape[0] // 2
    h = torch.nn.functional.linear(x, W13)
    return (torch.nn.functional.silu(h[:, :F]) * h[:, F:]) @ W2.T


def _rand_layer(rng, T, d, E, k, F, Fs=0, score="softmax", scaling=1.0, aux=0.0, bias=None, **extra):
    x = rng.standard_normal((T, d))
    Wg = rng.standard_normal((E, d)) / np.sqrt(d)
    W13 = rng.standard_normal((E, 2 * F, d)) / np.sqrt(d)
    W2 = rng.standard_normal((E, d, F)) / np.sqrt(F)
    W13s = rng.standard_normal((2 * Fs, d)) / np.sqrt(d) if Fs else None
    W2s = rng.standard_normal((d, Fs)) / np.sqrt(Fs) if Fs else None
    bg = rng.standard_normal(E) * 0.3 if bias == "bg" else None
    eb = rng.standard_normal(E) * 0.1 if bias == "expert_bias" else None
    dy = rng.standard_normal((T, d))
    spec = O.LayerSpec(E=E, k=k, score=score, scaling=scaling, aux_coeff=aux, **extra)
    Wsg = rng.standard_normal(d) / np.sqrt(d) if spec.shared_gate else None
    return dict(x=x, Wg=Wg, W13=W13, W2=W2, W13s=W13s, W2s=W2s, bg=bg, expert_bias=eb, dy=dy, Wsg=Wsg), spec


# ------------------------------------------------------------------ worked examples

def test_worked_mixture_075_025():
    g = gold("worked_mixture.json")
    wa, wb = g["weights"]
    # a softmax over the two selected logits gives (0.75, 0.25) iff l_A - l_B = ln 3
    logits = np.array([[math.log(3.0), 0.0]])
    idx = O.topk(O.selection_keys(logits, "softmax"), 2)
    assert idx.tolist() == [[0, 1]]
    w = O.mixing_weights(logits, idx, "softmax")
    assert abs(w[0, 0] - wa) < 1e-15 and abs(w[0, 1] - wb) < 1e-15
    # whole layer: y = 0.75 * A(x) + 0.25 * B(x), coordinate by coordinate
    rng = np.random.default_rng(0)
    d, F = 2, 4
    x = np.array([[1.0, 0.0]])
    Wg = np.array([[math.log(3.0), 0.0], [0.0, 0.0]])
    W13 = rng.standard_normal((2, 2 * F, d))
    W2 = rng.standard_normal((2, d, F))
    out = O.layer_forward(x, Wg, W13, W2, O.LayerSpec(E=2, k=2))
    A = _ffn_torch(x, W13[0], W2[0]).numpy()
    B = _ffn_torch(x, W13[1], W2[1]).numpy()
    np.testing.assert_allclose(out["y"], wa * A + wb * B, rtol=1e-13, atol=1e-13)


def test_four_gpu_scenario_counts_maxvio_buffer():
    g = gold("four_gpu_loads.json")
    T, k, E = g["tokens"], g["top_k"], g["experts"]
    labels = np.repeat(np.arange(E), g["loads"])          # 8192 expert labels
    assert labels.size == g["assignments"]
    idx = np.stack([labels[:T], labels[T:]], axis=1)       # token t gets labels t and t+T
    assert np.all(idx[:, 0] != idx[:, 1])
    counts = O.expert_counts(idx, E)
    assert counts.tolist() == g["loads"]
    assert counts.sum() == T * k == g["assignments"]
    assert O.max_violation(counts) == g["maxvio"]
    assert counts.mean() == g["even_load_per_expert"]
    perm = O.permutation(idx, E)
    assert perm.token_of.size == g["assignments"]
    assert O.permuted_buffer_bytes(T, k, g["values_per_vector"], g["bytes_per_value"]) == g["permuted_input_bytes"]
    assert g["permuted_input_bytes"] == 32 * 2 ** 20


def test_first_moe_shapes_and_extremes():
    g = gold("first_moe.json")
    d, F = g["d_model"], g["expert_ffn"]
    assert O.expert_param_count(d, F) == g["params_per_expert"]
    assert 8 * O.expert_param_count(d, F) == g["params_eight_experts"] == 3 * d * g["dense_ffn_width"]
    # busiest expert receives every token: MaxVio = E/k - 1 = 7 at 64 experts, top-8
    E, k, T = g["num_experts"], g["top_k"], 4096
    idx = np.zeros((T, k), dtype=np.int64)
    idx[:, 0] = 0
    rest = np.arange(T * (k - 1)) % (E - 1) + 1
    idx[:, 1:] = rest.reshape(T, k - 1)
    idx[:, 1:] = (np.arange(T)[:, None] * (k - 1) + np.arange(k - 1)[None, :]) % (E - 1) + 1
    assert all(len(set(r)) == k for r in idx.tolist())
    assert O.max_violation(O.expert_counts(idx, E)) == g["most_biased_maxvio"]


def test_single_expert_lb_loss_is_one_and_router_gets_no_gradient():
    g = gold("first_moe.json")
    rng = np.random.default_rng(1)
    L, spec = _rand_layer(rng, T=32, d=8, E=1, k=1, F=6, aux=1e-3)
    f = O.layer_forward(L["x"], L["Wg"], L["W13"], L["W2"], spec)
    assert f["route"]["aux"] / spec.aux_coeff == pytest.approx(g["one_expert_load_balancing_loss"], abs=1e-15)
    b = O.layer_backward(f, L["x"], L["Wg"], L["W13"], L["W2"], L["dy"], spec)
    assert np.all(b["dlogits"] == 0.0) and np.all(b["dWg"] == 0.0)
    # and the one-expert layer is the dense FFN (independent torch implementation)
    np.testing.assert_allclose(f["y"], _ffn_torch(L["x"], L["W13"][0], L["W2"][0]).numpy(), rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------------- router

def test_topk_matches_brute_force_with_ties():
    rng = np.random.default_rng(2)
    for trial in range(300):
        E = int(rng.integers(2, 8))
        k = int(rng.integers(1, E + 1))
        levels = int(rng.integers(1, 4)) if trial % 2 else 1000
        keys = rng.integers(0, levels, size=(1, E)).astype(np.float64) + (0 if levels < 1000 else rng.random((1, E)))
        got = O.topk(keys, k)[0].tolist()
        assert got == O.brute_force_topk(keys[0], k), (keys, k)


def test_constructed_ties_go_to_lower_index():
    keys = np.array([[0.5, 1.0, 1.0, 0.2, 1.0]])
    assert O.topk(keys, 2).tolist() == [[1, 2]]
    assert O.topk(keys, 4).tolist() == [[1, 2, 4, 0]]
    assert O.topk(np.zeros((1, 6)), 3).tolist() == [[0, 1, 2]]


def test_weights_sum_to_one_or_scaling():
    rng = np.random.default_rng(3)
    l = rng.standard_normal((64, 16)) * 2
    for score in ("softmax", "sigmoid"):
        for c in (1.0, 2.5):
            idx = O.topk(O.selection_keys(l, score), 4)
            w = O.mixing_weights(l, idx, score, c)
            np.testing.assert_allclose(w.sum(1), c, rtol=1e-14)
            assert np.all(w > 0)


def test_softmax_weights_equal_renormalised_full_softmax():
    rng = np.random.default_rng(4)
    l = rng.standard_normal((32, 12))
    idx = O.topk(l, 3)
    p = torch.softmax(torch.as_tensor(l), dim=1).numpy()     # library softmax over all E
    pS = np.take_along_axis(p, idx, axis=1)
    np.testing.assert_allclose(O.mixing_weights(l, idx, "softmax"), pS / pS.sum(1, keepdims=True), rtol=1e-13)


def test_sigmoid_matches_library_and_bias_selects_only():
    rng = np.random.default_rng(5)
    l = rng.standard_normal((256, 16)) * 2
    np.testing.assert_allclose(O.sigmoid(l), expit(l), rtol=1e-15)
    bias = rng.standard_normal(16) * 0.3
    idx_b = O.topk(O.selection_keys(l, "sigmoid", bias), 4)
    idx_0 = O.topk(O.selection_keys(l, "sigmoid"), 4)
    assert np.any(idx_b != idx_0)                 # the bias does change the selection ...
    w = O.mixing_weights(l, idx_b, "sigmoid")
    s = expit(np.take_along_axis(l, idx_b, axis=1))
    np.testing.assert_allclose(w, s / s.sum(1, keepdims=True), rtol=1e-14)  # ... but not the weights
    # k = 1 sigmoid: the raw score, no renormalisation
    idx1 = O.topk(O.selection_keys(l, "sigmoid"), 1)
    np.testing.assert_allclose(O.mixing_weights(l, idx1, "sigmoid"), expit(np.take_along_axis(l, idx1, 1)), rtol=1e-15)


def test_shift_invariance():
    rng = np.random.default_rng(6)
    l = rng.standard_normal((128, 16))
    idx = O.topk(l, 4)
    assert np.array_equal(O.topk(l + 3.25, 4), idx)
    np.testing.assert_allclose(O.mixing_weights(l + 3.25, idx, "softmax"), O.mixing_weights(l, idx, "softmax"), rtol=1e-13)
    bias = rng.standard_normal(16) * 0.1
    assert np.array_equal(O.topk(O.selection_keys(l, "sigmoid", bias + 0.5), 4),
                          O.topk(O.selection_keys(l, "sigmoid", bias), 4))


def test_top1_post_softmax_weight_one_and_no_router_gradient():
    rng = np.random.default_rng(7)
    L, spec = _rand_layer(rng, T=24, d=6, E=4, k=1, F=4)
    f = O.layer_forward(L["x"], L["Wg"], L["W13"], L["W2"], spec)
    assert np.all(f["route"]["w"] == 1.0)
    b = O.layer_backward(f, L["x"], L["Wg"], L["W13"], L["W2"], L["dy"], spec)
    assert np.all(b["dlogits"] == 0.0)
    assert np.any(b["dw"] != 0.0)


def test_aux_loss_closed_forms():
    rng = np.random.default_rng(8)
    T, E, k = 200, 8, 2
    # flat router probabilities: aux / coeff = 1 whatever the load
    for _ in range(5):
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
        counts = O.expert_counts(idx, E)
        assert O.aux_loss(counts, np.full((T, E), 1.0 / E), k, 1.0) == pytest.approx(1.0, abs=1e-14)
    # a one-hot router that sends every token's whole probability to expert 0, which
    # is also in every token's top-k: f_0 = 1/k, P_0 = 1 -> aux / coeff = E / k
    idx = np.stack([np.r_[0, rng.permutation(np.arange(1, E))[:k - 1]] for _ in range(T)])
    p = np.zeros((T, E)); p[:, 0] = 1.0
    assert O.aux_loss(O.expert_counts(idx, E), p, k, 1.0) == pytest.approx(E / k, rel=1e-15)
    # counts always sum to T * k
    l = rng.standard_normal((T, E))
    assert O.expert_counts(O.topk(l, k), E).sum() == T * k


def test_aux_loss_matches_printed_code_form():
    # the handbook's code form: sum(probs.sum(0) * tokens_per_expert) * E * coeff / (k * T * T)
    rng = np.random.default_rng(9)
    T, E, k, c = 97, 10, 3, 0.013
    l = rng.standard_normal((T, E))
    idx = O.topk(l, k)
    probs = torch.softmax(torch.as_tensor(l), dim=1)
    tpe = torch.bincount(torch.as_tensor(idx).flatten(), minlength=E).double()
    code = float(torch.sum(probs.sum(0) * tpe) * (E * c / (k * T * T)))
    assert O.aux_loss(O.expert_counts(idx, E), O.softmax_full(l), k, c) == pytest.approx(code, rel=1e-13)


# ------------------------------------------------------------------- permutation

def test_permutation_is_valid_and_matches_counting_sort():
    rng = np.random.default_rng(10)
    for T, E, k in [(1, 1, 1), (7, 3, 2), (50, 9, 4), (300, 32, 8), (64, 64, 64)]:
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
        p = O.permutation(idx, E)
        # independent construction: a pure-Python counting sort
        buckets = [[] for _ in range(E)]
        for t in range(T):
            for j in range(k):
                buckets[idx[t, j]].append((t, j))
        flat = [tj for b in buckets for tj in b]
        assert [t for t, _ in flat] == p.token_of.tolist()
        for r, (t, j) in enumerate(flat):
            assert p.row_of[t, j] == r
        assert p.offsets[0] == 0 and p.offsets[-1] == T * k
        assert np.all(np.diff(p.offsets) >= 0)
        assert np.array_equal(p.token_of[p.row_of], np.repeat(np.arange(T)[:, None], k, 1))


# ------------------------------------------------------------------------- experts

def test_swiglu_matches_torch_and_silu_matches_library():
    rng = np.random.default_rng(11)
    X = rng.standard_normal((9, 6)); W13 = rng.standard_normal((10, 6)); W2 = rng.standard_normal((6, 5))
    H, Act, Y = O.swiglu_forward(X, W13, W2)
    np.testing.assert_allclose(Y, _ffn_torch(X, W13, W2).numpy(), rtol=1e-12, atol=1e-12)
    g = rng.standard_normal(1000) * 5
    np.testing.assert_allclose(O.silu(g), g * expit(g), rtol=1e-14, atol=1e-300)


def test_identical_experts_make_routing_irrelevant():
    rng = np.random.default_rng(12)
    L, spec = _rand_layer(rng, T=40, d=8, E=6, k=3, F=5, Fs=4, score="sigmoid", scaling=2.5)
    W13 = np.repeat(L["W13"][:1], 6, 0); W2 = np.repeat(L["W2"][:1], 6, 0)
    f = O.layer_forward(L["x"], L["Wg"], W13, W2, spec, W13s=L["W13s"], W2s=L["W2s"])
    ref = 2.5 * _ffn_torch(L["x"], W13[0], W2[0]).numpy() + _ffn_torch(L["x"], L["W13s"], L["W2s"]).numpy()
    np.testing.assert_allclose(f["y"], ref, rtol=1e-12, atol=1e-12)


def test_layer_against_independent_token_loop():
    """The vectorised layer equals a per-token loop over torch's dense FFNs."""
    rng = np.random.default_rng(13)
    L, spec = _rand_layer(rng, T=30, d=8, E=5, k=2, F=6, Fs=3, score="softmax", bias="bg")
    f = O.layer_forward(L["x"], L["Wg"], L["W13"], L["W2"], spec, bg=L["bg"], W13s=L["W13s"], W2s=L["W2s"])
    logits = torch.as_tensor(L["x"]) @ torch.as_tensor(L["Wg"]).T + torch.as_tensor(L["bg"])
    for t in range(30):
        vals, ids = torch.topk(logits[t], 2)
        w = torch.softmax(vals, 0)
        y = _ffn_torch(L["x"][t:t + 1], L["W13s"], L["W2s"])[0]
        for j in range(2):
            e = int(ids[j])
            y = y + w[j] * _ffn_torch(L["x"][t:t + 1], L["W13"][e], L["W2"][e])[0]
        np.testing.assert_allclose(f["y"][t], y.numpy(), rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------------ backward

@pytest.mark.parametrize("case", [
    dict(score="softmax", k=2, aux=0.7, Fs=0, scaling=1.0, bias="bg"),
    dict(score="softmax", k=3, aux=0.0, Fs=4, scaling=2.5, bias=None),
    dict(score="sigmoid", k=2, aux=0.0, Fs=4, scaling=1.0, bias="expert_bias"),
    dict(score="sigmoid", k=1, aux=0.0, Fs=0, scaling=1.3, bias=None),
    # the balancing losses and router variants
    dict(score="softmax", k=1, aux=0.4, Fs=0, scaling=1.0, bias="bg", extra=dict(pre_softmax=True, z_coeff=0.05)),
    dict(score="softmax", k=2, aux=0.0, Fs=0, scaling=2.5, bias=None,
         extra=dict(pre_softmax=True, seq_aux_coeff=0.3, seq_len=4)),
    dict(score="softmax", k=2, aux=0.2, Fs=0, scaling=1.0, bias=None,
         extra=dict(z_coeff=0.02, seq_aux_coeff=0.5, seq_len=8)),
    dict(score="sigmoid", k=2, aux=0.3, Fs=4, scaling=1.0, bias="expert_bias",
         extra=dict(z_coeff=0.01, seq_aux_coeff=0.4, seq_len=4)),
    dict(score="sqrtsoftplus", k=2, aux=0.0, Fs=0, scaling=1.7, bias="expert_bias",
         extra=dict(seq_aux_coeff=0.6, seq_len=16)),
    dict(score="sqrtsoftplus", k=1, aux=0.5, Fs=0, scaling=1.0, bias=None, extra=dict(z_coeff=0.03)),
    # the clamped SwiGLU and SiTU-GLU experts
    dict(score="softmax", k=2, aux=0.0, Fs=4, scaling=1.0, bias=None, extra=dict(glu=O.GLU("clamp", 0.35))),
    dict(score="sigmoid", k=2, aux=0.0, Fs=4, scaling=1.0, bias=None, extra=dict(glu=O.GLU("situ", 0.6, 0.5))),
    dict(score="softmax", k=3, aux=0.1, Fs=0, scaling=1.0, bias=None, extra=dict(glu=O.GLU("situ", 0.8, 0.0))),
    # the sigmoid gate on the shared expert
    dict(score="softmax", k=2, aux=0.0, Fs=4, scaling=1.0, bias="bg", extra=dict(shared_gate=True)),
    dict(score="sigmoid", k=2, aux=0.0, Fs=4, scaling=2.5, bias=None,
         extra=dict(shared_gate=True, glu=O.GLU("clamp", 0.4))),
])
def test_backward_matches_central_differences(case):
    rng = np.random.default_rng(14)
    L, spec = _rand_layer(rng, T=16, d=8, E=4, k=case["k"], F=8, Fs=case["Fs"], score=case["score"],
                          scaling=case["scaling"], aux=case["aux"], bias=case["bias"], **case.get("extra", {}))
    keys = O.selection_keys(O.gate_logits(L["x"], L["Wg"], L["bg"]), spec.score, L["expert_bias"])
    assert O.margins(keys, spec.k).min() > 1e-4           # far from a routing flip
    kw = dict(bg=L["bg"], expert_bias=L["expert_bias"], W13s=L["W13s"], W2s=L["W2s"], Wsg=L["Wsg"])
    f = O.layer_forward(L["x"], L["Wg"], L["W13"], L["W2"], spec, **kw)
    b = O.layer_backward(f, L["x"], L["Wg"], L["W13"], L["W2"], L["dy"], spec,
                         W13s=L["W13s"], W2s=L["W2s"], daux=1.0, Wsg=L["Wsg"])
    names = [("x", "dx"), ("Wg", "dWg"), ("W13", "dW13"), ("W2", "dW2")]
    if L["bg"] is not None:
        names.append(("bg", "dbg"))
    if case["Fs"]:
        names += [("W13s", "dW13s"), ("W2s", "dW2s")]
    if spec.shared_gate:
        names.append(("Wsg", "dWsg"))
    h = 1e-6
    for pname, gname in names:
        P = L[pname]
        flat = P.reshape(-1)
        picks = rng.choice(flat.size, size=min(flat.size, 40), replace=False)
        for i in picks:
            old = flat[i]
            flat[i] = old + h
            lp = O.layer_loss(L["x"], L["Wg"], L["W13"], L["W2"], L["dy"], spec, **kw)
            flat[i] = old - h
            lm = O.layer_loss(L["x"], L["Wg"], L["W13"], L["W2"], L["dy"], spec, **kw)
            flat[i] = old
            fd = (lp - lm) / (2 * h)
            an = b[gname].reshape(-1)[i]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (pname, i, fd, an)


# ------------------------------------------------------------------ fp8 (e4m3) quantiser

def _torch_e4m3(v):
    """torch's own float32 -> float8_e4m3fn cast (round to nearest even, no saturation)."""
    return torch.as_tensor(np.asarray(v, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_table_and_rounding_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    finite = codes[(codes & 0x7F) != 0x7F]
    ref = torch.as_tensor(finite).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(O.e4m3_decode(finite), ref)
    assert O.E4M3_MAX == ref.max() == 448.0
    # every finite code round-trips
    assert np.array_equal(O.e4m3_encode(O.e4m3_decode(finite)), finite)
    # random values inside the range, plus every midpoint between neighbouring codes
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.standard_normal(20000) * 30, rng.standard_normal(2000) * 1e-3,
                        (O._E4M3[1:] + O._E4M3[:-1]) / 2, -(O._E4M3[1:] + O._E4M3[:-1]) / 2]).astype(np.float32)
    v = v[np.abs(v) <= 448]
    assert np.array_equal(O.e4m3_encode(v), _torch_e4m3(v))


def test_e4m3_saturation_and_signed_zero():
    assert list(O.e4m3_encode(np.array([448, 449, 464, 1e6, -500], dtype=np.float32))) == [0x7E] * 4 + [0xFE]
    assert list(O.e4m3_encode(np.array([0.0, -0.0, -1e-30, 2.0 ** -10], dtype=np.float32))) == [0x00, 0x80, 0x80, 0x00]


def test_block_quantiser_scale_rule_and_bounds():
    rng = np.random.default_rng(3)
    v = (rng.standard_normal((256, 384)) * rng.uniform(0.01, 5, size=(256, 1))).astype(np.float32)
    v[:128, 128:256] = 0.0                       # an all-zero 128 x 128 block
    for br in (1, 128):
        q, s = O.quantize_blocks(v, br)
        assert q.shape == v.shape and s.shape == (256 // br, 3) and s.dtype == np.float32
        blocks = np.abs(v).reshape(256 // br, br, 3, 128).max(axis=(1, 3))
        assert np.array_equal(s, np.where(blocks > 0, blocks.astype(np.float32) / np.float32(448), 1).astype(np.float32))
        # the quantised values are torch's rounding of v / scale
        full = np.repeat(np.repeat(s, br, axis=0), 128, axis=1)
        assert np.array_equal(q, _torch_e4m3(np.minimum(np.abs(v / full), 448) * np.sign(v / full)) |
                              np.where(np.signbit(v), 0x80, 0).astype(np.uint8))
        # each block's largest magnitude lands on +-448
        deq = O.dequantize_blocks(q, s, br)
        nz = blocks > 0
        big = np.abs(O.e4m3_decode(q)).reshape(256 // br, br, 3, 128).max(axis=(1, 3))
        assert np.all(big[nz] == 448.0) and np.all(big[~nz] == 0.0)
        # error within half a step: 2^-4 relative for normal codes, 2^-10 scale for subnormal ones
        bound = np.maximum(2.0 ** -4 * np.abs(v), 2.0 ** -10 * full)
        assert np.all(np.abs(deq - v) <= bound)
        # idempotent on codes
        q2, _ = O.quantize_blocks(deq.astype(np.float32), br)
        assert np.array_equal(q2, q)


def test_fp8_layer_equals_exact_layer_up_to_act_rounding():
    """With x and the weights exactly on the e4m3 grids, the fp8 layer differs from the
    exact layer only by the per-token rounding of Act, which is bounded element by element."""
    rng = np.random.default_rng(11)
    T, d, E, k, F = 24, 256, 4, 2, 128
    spec = O.LayerSpec(E=E, k=k, score="softmax")
    # x: e4m3 codes times a per-row power of two, with a 448 in every 128-block so scale = 2^j
    codes = rng.integers(0, 0x7E, size=(T, d)).astype(np.uint8) | (rng.integers(0, 2, size=(T, d)) * 0x80).astype(np.uint8)
    codes[:, ::128] = 0x7E
    x = O.e4m3_decode(codes) * (2.0 ** rng.integers(-12, -6, size=(T, 1)))
    W13m = rng.standard_normal((E, 2 * F, d)).astype(np.float32) * 0.05
    W2m = rng.standard_normal((E, d, F)).astype(np.float32) * 0.05
    q13 = [O.quantize_blocks(W13m[e], 128) for e in range(E)]
    q2 = [O.quantize_blocks(W2m[e], 128) for e in range(E)]
    W13q, W13s = np.stack([a for a, _ in q13]), np.stack([b for _, b in q13])
    W2q, W2s = np.stack([a for a, _ in q2]), np.stack([b for _, b in q2])
    Wg = rng.standard_normal((E, d)) / 16
    f8 = O.layer_forward_fp8(x, Wg, W13q, W13s, W2q, W2s, spec)
    # x survives quantisation exactly
    assert np.array_equal(O.dequantize_blocks(f8["x_q"], f8["x_scale"], 1), x)
    W13d = np.stack([O.dequantize_blocks(W13q[e], W13s[e], 128) for e in range(E)])
    W2d = np.stack([O.dequantize_blocks(W2q[e], W2s[e], 128) for e in range(E)])
    ex = O.layer_forward(x, Wg, W13d, W2d, spec)
    assert np.array_equal(f8["route"]["idx"], ex["route"]["idx"])
    assert np.allclose(f8["H"], ex["H"], rtol=1e-12, atol=0)
    # |dAct| <= half a step of the Act grid of its row
    full = np.repeat(f8["Act_scale"].astype(np.float64), 128, axis=1)
    dact_bound = np.maximum(2.0 ** -4 * np.abs(f8["Act"]), 2.0 ** -10 * full)
    deq = O.dequantize_blocks(f8["Act_q"], f8["Act_scale"], 1)
    assert np.all(np.abs(deq - f8["Act"]) <= dact_bound)
    # propagate the bound through fc2 and the combine
    perm, r = f8["perm"], f8["route"]
    yb = np.zeros((T * k, d))
    for e in range(E):
        a, b = perm.offsets[e], perm.offsets[e + 1]
        yb[a:b] = dact_bound[a:b] @ np.abs(W2d[e]).T
    bound = np.einsum("tk,tkd->td", np.abs(r["w"]), yb[perm.row_of])
    diff = np.abs(f8["y"] - ex["y"])
    assert np.all(diff <= bound * (1 + 1e-9) + 1e-15)
    assert diff.max() > 0          # the Act rounding did happen


# ------------------------------------------------- router variants and balancing losses

def test_z_loss_closed_form_and_library_logsumexp():
    from scipy.special import logsumexp
    rng = np.random.default_rng(21)
    T, E, c = 50, 16, 1e-3
    # equal logits: lse = v + ln E for every token
    v = 1.7
    assert O.z_loss(np.full((T, E), v), c) == pytest.approx(c * (v + math.log(E)) ** 2, rel=1e-14)
    l = rng.standard_normal((T, E)) * 3 + 40.0       # large shared offset: no overflow
    assert O.z_loss(l, c) == pytest.approx(c * np.mean(logsumexp(l, axis=1) ** 2), rel=1e-13)
    # a shared shift u moves every lse by u
    u = -2.5
    np.testing.assert_allclose(O.logsumexp_rows(l + u), O.logsumexp_rows(l) + u, rtol=1e-14)


def test_seq_aux_loss_reduces_to_aux_and_matches_printed_code_form():
    rng = np.random.default_rng(22)
    E, k, S, B, c = 12, 3, 20, 5, 0.01
    T = S * B
    l = rng.standard_normal((T, E))
    idx = O.topk(l, k)
    p = O.softmax_full(l)
    # one sequence: the micro-batch loss
    assert O.seq_aux_loss(idx, p, k, T, c) == pytest.approx(O.aux_loss(O.expert_counts(idx, E), p, k, c), rel=1e-14)
    # flat probabilities: coeff, whatever the load
    assert O.seq_aux_loss(idx, np.full((T, E), 1.0 / E), k, S, c) == pytest.approx(c, rel=1e-14)
    # the printed code form: reshape [S*B, E] -> [S, B*E], per-(sequence, expert) counts,
    # the Switch formula with S tokens, divided by B
    probs = torch.as_tensor(p).reshape(S, B * E)
    rmap = torch.zeros(T, E, dtype=torch.float64)
    rmap.scatter_(1, torch.as_tensor(idx), 1.0)
    tpe = rmap.reshape(S, B * E).sum(0)
    code = float(torch.sum(probs.sum(0) * tpe) * (E * c / (k * S * S))) / B
    assert O.seq_aux_loss(idx, p, k, S, c) == pytest.approx(code, rel=1e-13)
    # a per-sequence loop that gathers sequence b's tokens b, b + B, b + 2B, ...
    loop = np.mean([O.aux_loss(O.expert_counts(idx[b::B], E), p[b::B], k, c) for b in range(B)])
    assert O.seq_aux_loss(idx, p, k, S, c) == pytest.approx(loop, rel=1e-13)
    cnt = O.sequence_counts(idx, E, S)
    assert cnt.shape == (B, E) and np.all(cnt.sum(axis=1) == S * k)


def test_pre_softmax_weights_are_full_probabilities():
    rng = np.random.default_rng(23)
    T, E = 40, 10
    l = rng.standard_normal((T, E)) * 2
    probs = torch.softmax(torch.as_tensor(l), dim=1)
    for k in (1, 3, E):
        tv, ti = torch.topk(probs, k, dim=1)              # library top-k on the probabilities
        idx = O.topk(O.selection_keys(l, "softmax"), k)
        assert np.array_equal(idx, ti.numpy())
        w = O.mixing_weights(l, idx, "softmax", 1.0, pre_softmax=True)
        np.testing.assert_allclose(w, tv.numpy(), rtol=1e-14)
        if k < E:
            assert np.all(w.sum(axis=1) < 1.0)            # no renormalisation
        else:
            np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-14)
    # top-1 with pre-softmax: the weight is the top probability and the router gets a
    # gradient (post-softmax top-1 gives weight 1 and none)
    spec = O.LayerSpec(E=E, k=1, pre_softmax=True)
    idx = O.topk(l, 1)
    w = O.mixing_weights(l, idx, "softmax", 1.0, pre_softmax=True)
    dl = O.router_backward(l, idx, w, np.ones((T, 1)), spec)
    assert np.abs(dl).max() > 1e-3
    # d w_top / d l for dw = 1: p_top (1 - p_top) at the top expert, -p_top p_e elsewhere
    pt = probs.numpy()
    ref = -pt * pt[np.arange(T), idx[:, 0]][:, None]
    ref[np.arange(T), idx[:, 0]] = pt[np.arange(T), idx[:, 0]] * (1 - pt[np.arange(T), idx[:, 0]])
    np.testing.assert_allclose(dl, ref, rtol=1e-12, atol=1e-15)


def test_sqrt_softplus_scores():
    rng = np.random.default_rng(24)
    l = rng.standard_normal((30, 9)) * 4
    ref = torch.nn.functional.softplus(torch.as_tensor(l)).sqrt().numpy()
    np.testing.assert_allclose(O.score_values(l, "sqrtsoftplus"), ref, rtol=1e-14)
    assert O.score_values(np.array([0.0]), "sqrtsoftplus")[0] == pytest.approx(math.sqrt(math.log(2.0)), rel=1e-15)
    # no overflow far out: softplus(l) -> l
    assert O.score_values(np.array([800.0]), "sqrtsoftplus")[0] == pytest.approx(math.sqrt(800.0), rel=1e-15)
    # the three gating functions rank experts alike
    for k in (1, 4):
        a = O.topk(O.selection_keys(l, "softmax"), k)
        assert np.array_equal(a, O.topk(O.selection_keys(l, "sigmoid"), k))
        assert np.array_equal(a, O.topk(O.selection_keys(l, "sqrtsoftplus"), k))
    # for positive logits the ratio of two weights tends to sqrt of the ratio of the logits
    L1, L2 = 3.0, 1.2
    for a, tol in ((10.0, 1e-2), (1000.0, 1e-4)):
        lg = np.array([[a * L1, a * L2, -50.0]])
        w = O.mixing_weights(lg, np.array([[0, 1]]), "sqrtsoftplus")
        assert w[0, 0] / w[0, 1] == pytest.approx(math.sqrt(L1 / L2), rel=tol)
    # derivative against the library's autograd
    t = torch.as_tensor(l, dtype=torch.float64).requires_grad_(True)
    torch.nn.functional.softplus(t).sqrt().sum().backward()
    np.testing.assert_allclose(O.score_derivative(l, "sqrtsoftplus"), t.grad.numpy(), rtol=1e-13)


def test_normalised_aux_probabilities_for_sigmoid_scores():
    rng = np.random.default_rng(25)
    l = rng.standard_normal((20, 7))
    for score in ("sigmoid", "sqrtsoftplus"):
        q = O.aux_probs(l, score)
        np.testing.assert_allclose(q.sum(axis=1), 1.0, rtol=1e-14)
        s = expit(l) if score == "sigmoid" else np.sqrt(np.log1p(np.exp(l)))
        np.testing.assert_allclose(q, s / s.sum(axis=1, keepdims=True), rtol=1e-13)


def test_expert_bias_update_printed_rule_and_properties():
    rng = np.random.default_rng(26)
    E, T, k, rate = 16, 256, 4, 1e-3
    # a few hot experts and many just under the mean load
    counts = np.full(E, T * k // E - 3, dtype=np.int64)
    counts[:3] += (T * k - counts.sum()) // 3
    counts[0] += T * k - counts.sum()
    assert counts.sum() == T * k
    bias = (rng.standard_normal(E) * 0.1).astype(np.float32)
    new = O.expert_bias_update(bias, counts, rate)
    # the printed form, in torch: direction = sign(total - count * E), bias += direction * rate
    tc = torch.as_tensor(counts)
    direction = torch.sign(tc.sum(-1, keepdim=True) - tc * E)
    code = torch.as_tensor(bias) + direction.to(torch.float32) * rate
    assert np.array_equal(new, code.numpy())
    over, under = counts * E > T * k, counts * E < T * k
    assert np.all(new[over] < bias[over]) and np.all(new[under] > bias[under])
    # an expert exactly at the mean keeps its bias; the integer comparison is exact where
    # the mean total / E is not an integer
    c2 = np.array([3, 2, 2], dtype=np.int64)            # mean 7/3
    b2 = O.expert_bias_update(np.zeros(3, np.float32), c2, 0.5)
    assert list(b2) == [-0.5, 0.5, 0.5]
    c3 = np.array([4, 4, 4, 4], dtype=np.int64)
    assert np.array_equal(O.expert_bias_update(bias[:4], c3, rate), bias[:4])
    # most steps point up here: the sign update lifts the mean bias; the centered update
    # keeps it (to fp32 rounding), and both route alike (a shared shift keeps the top-k)
    cen = O.expert_bias_update(bias, counts, rate, centered=True)
    assert new.mean() - bias.mean() > 0.5 * rate
    assert abs(float(cen.astype(np.float64).sum() - bias.astype(np.float64).sum())) < E * 1e-7
    s = O.sigmoid(rng.standard_normal((T, E)))
    assert np.array_equal(O.topk(s + new.astype(np.float64), k), O.topk(s + (cen + (new - cen).mean()).astype(np.float64), k)) or \
        np.allclose(new - cen, (new - cen).mean(), atol=1e-9)


def test_expert_bias_update_balances_a_fixed_batch():
    # the loop of the loss-free bias on one batch: repeated sign steps bring MaxVio down
    rng = np.random.default_rng(27)
    T, E, k = 512, 16, 2
    l = rng.standard_normal((T, E)) + np.linspace(-1.5, 1.5, E)[None, :]
    s = O.sigmoid(l)
    bias = np.zeros(E, np.float32)
    first = None
    for step in range(400):
        counts = O.expert_counts(O.topk(s + bias.astype(np.float64), k), E)
        mv = O.max_violation(counts)
        first = mv if first is None else first
        bias = O.expert_bias_update(bias, counts, 2e-3)
    assert first > 1.0 and mv < 0.25 * first


# ------------------------------------------------------------------- quantile balancing

def test_quantile_route_matches_printed_code_form():
    # the printed form in torch fp32: (scores - beta).topk(k + 1, dim=1); alpha = its last
    # value; (scores - alpha).topk(T k / E + 1, dim=0).values[-1]; continuous scores, so no
    # ties leave the order open
    rng = np.random.default_rng(31)
    T, E, k = 96, 12, 3
    scores = rng.random((T, E)).astype(np.float32)
    beta = (rng.standard_normal(E) * 0.05).astype(np.float32)
    ts, tb = torch.as_tensor(scores), torch.as_tensor(beta)
    top = (ts - tb).topk(k + 1, dim=1)
    alpha = top.values[:, -1:]
    bl = (ts - alpha).topk(T * k // E + 1, dim=0).values[-1]
    idx, a, b = O.quantile_route(scores, beta, k)
    assert np.array_equal(idx, top.indices[:, :-1].numpy())
    assert np.array_equal(a, alpha[:, 0].numpy())
    assert np.array_equal(b, bl.numpy())


def test_quantile_bias_is_the_target_share_quantile():
    # the solved bias is the score that only the expert's target share of tokens beats: it
    # is the (target + 1)-th largest of scores - alpha, so at most target = T k / E values
    # lie above it and at least target + 1 at or above it (every token's (k+1)-th expert
    # gives exactly 0, so ties at 0 are part of the method)
    rng = np.random.default_rng(32)
    T, E, k = 400, 16, 2
    target = T * k // E
    scores = rng.random((T, E)).astype(np.float32) ** 3
    idx, alpha, bl = O.quantile_route(scores, np.zeros(E, np.float32), k)
    v = (scores - alpha[:, None]).astype(np.float32)
    above, at_or_above = (v > bl[None, :]).sum(axis=0), (v >= bl[None, :]).sum(axis=0)
    assert np.all(above <= target) and np.all(at_or_above >= target + 1)
    assert np.any(above == target)
    # brute force on one column: sort it, count down target places
    col = sorted(v[:, 5].tolist(), reverse=True)
    assert bl[5] == col[target]
    # ties in the keys go to the lower expert index, as in the router
    tie = np.zeros((1, 4), np.float32)
    assert list(O.quantile_route(tie, np.zeros(4, np.float32), 2, update=False)[0][0]) == [0, 1]
    with pytest.raises(ValueError):
        O.quantile_route(scores[:7], np.zeros(E, np.float32), k)     # 7 * 2 is not a multiple of 16


def test_quantile_balancing_evens_a_fixed_batch_and_update_is_centered():
    # routing one skewed batch repeatedly with its own solved bias (no smoothing) brings the
    # load close to even within a few steps; the update keeps the mean bias at zero
    rng = np.random.default_rng(33)
    T, E, k = 1024, 16, 2
    logits = rng.standard_normal((T, E)) + np.linspace(-2.0, 2.0, E)[None, :]
    scores = O.softmax_full(logits).astype(np.float32)
    beta = np.zeros(E, np.float32)
    mv = []
    for _ in range(6):
        idx, _, bl = O.quantile_route(scores, beta, k)
        mv.append(O.max_violation(O.expert_counts(idx, E)))
        beta = O.quantile_bias_update(beta, bl, 0.0).astype(np.float32)
    assert mv[0] > 2.0 and mv[-1] < 0.1 * mv[0]
    nb = O.quantile_bias_update(rng.standard_normal(E), rng.standard_normal(E), 0.9)
    assert abs(nb.mean()) < 1e-15
    # ema = 1 keeps the old bias (centred), ema = 0 takes the new solution (centred)
    b0, b1 = rng.standard_normal(E), rng.standard_normal(E)
    np.testing.assert_allclose(O.quantile_bias_update(b0, b1, 1.0), b0 - b0.mean(), atol=1e-15)
    np.testing.assert_allclose(O.quantile_bias_update(b0, b1, 0.0), b1 - b1.mean(), atol=1e-15)


# ------------------------------------------------------------------ activation variants

def _glu_torch(H, glu):
    """The printed forms, in torch: glu() with the clamp (gate from above, up on both sides),
    and situ_glu() with tanh_soft_clamp."""
    H = torch.as_tensor(H, dtype=torch.float64).requires_grad_(True)
    g, u = torch.chunk(H, 2, dim=-1)
    if glu.kind == "clamp":
        out = torch.nn.functional.silu(g.clamp(min=None, max=glu.c)) * u.clamp(min=-glu.c, max=glu.c)
    elif glu.kind == "situ":
        tsc = lambda x, sc: sc * torch.tanh(x / sc)  # noqa: E731
        ul = tsc(u, glu.c_linear) if glu.c_linear > 0 else u
        out = tsc(g, glu.c) * torch.sigmoid(g) * ul
    else:
        out = torch.nn.functional.silu(g) * u
    return H, out


@pytest.mark.parametrize("glu", [O.GLU("clamp", 0.7), O.GLU("clamp", 10.0), O.GLU("situ", 4.0, 25.0),
                                 O.GLU("situ", 0.5, 0.0), O.SWIGLU])
def test_glu_variants_match_printed_forms_and_autograd(glu):
    rng = np.random.default_rng(51)
    H = rng.standard_normal((40, 24)) * 3.0
    H[0, 0], H[0, 12] = glu.c + 0.25, -(glu.c + 0.25)      # clamped on both halves
    Ht, out = _glu_torch(H, glu)
    np.testing.assert_allclose(O.glu_forward(H, glu), out.detach().numpy(), rtol=1e-13, atol=1e-14)
    dAct = rng.standard_normal((40, 12))
    out.backward(torch.as_tensor(dAct))
    np.testing.assert_allclose(O.glu_backward(H, dAct, glu), Ht.grad.numpy(), rtol=1e-12, atol=1e-14)


def test_glu_variants_reduce_to_swiglu():
    rng = np.random.default_rng(52)
    H = rng.standard_normal((30, 16))
    plain = O.glu_forward(H)
    np.testing.assert_allclose(O.glu_forward(H, O.GLU("clamp", 1e6)), plain, rtol=1e-15)
    # s tanh(x / s) -> x as s grows, so SiTU-GLU -> silu(gate) * up
    np.testing.assert_allclose(O.glu_forward(H, O.GLU("situ", 1e5, 0.0)), plain, rtol=1e-8, atol=1e-12)
    # a clamped unit passes no gradient to its input
    Hc = np.array([[5.0, -1.0, 0.3, 7.0]])
    dH = O.glu_backward(Hc, np.ones((1, 2)), O.GLU("clamp", 2.0))
    assert dH[0, 0] == 0.0 and dH[0, 3] == 0.0 and dH[0, 1] != 0.0 and dH[0, 2] != 0.0


# ------------------------------------------------------------------ group-limited routing

def test_group_limited_topk_reductions_and_brute_force():
    from itertools import combinations
    rng = np.random.default_rng(61)
    T, E, k, G = 60, 16, 4, 4
    keys = rng.standard_normal((T, E))
    # keeping every group is plain top-k
    idx, kept, _ = O.group_limited_topk(keys, k, G, G)
    assert np.array_equal(idx, O.topk(keys, k))
    for gk in (1, 2, 3):
        idx, kept, gm = O.group_limited_topk(keys, k, G, gk)
        n, m = E // G, k // gk
        for t in range(T):
            # brute force: every subset of gk groups, scored by the sum of each group's m
            # best keys; the kept subset has the largest total (unique for random keys)
            score = [sum(sorted(keys[t, g * n:(g + 1) * n], reverse=True)[:m]) for g in range(G)]
            best = max(combinations(range(G), gk), key=lambda S: sum(score[g] for g in S))
            assert sorted(kept[t].tolist()) == sorted(best)
            # every selected expert lies in a kept group, and they are the k best there
            assert set((idx[t] // n).tolist()) <= set(kept[t].tolist())
            pool = [e for g in kept[t] for e in range(g * n, (g + 1) * n)]
            assert sorted(idx[t].tolist()) == sorted(sorted(pool, key=lambda e: -keys[t, e])[:k])
            assert gm[t] > 0 if gk < G else gm[t] == np.inf
    # a token whose plain top-4 spans three groups keeps two: the constraint binds
    row = np.array([[9, 0, 0, 0, 8, 7, 0, 0, 6, 0, 0, 0, 0, 0, 0, 0]], dtype=float)
    idx, kept, _ = O.group_limited_topk(row, 4, 4, 2)
    assert sorted(kept[0].tolist()) == [0, 1] and sorted(idx[0].tolist()) == [0, 1, 4, 5]
    assert sorted(O.topk(row, 4)[0].tolist()) == [0, 4, 5, 8]


def test_group_limited_route_margin_covers_the_group_decision():
    rng = np.random.default_rng(62)
    logits = rng.standard_normal((50, 16))
    spec = O.LayerSpec(E=16, k=4, score="sigmoid", num_groups=4, group_topk=2)
    r = O.route(logits, spec)
    _, _, gm = O.group_limited_topk(r["keys"], 4, 4, 2)
    assert np.all(r["margin"] <= gm)


def test_shared_gate_printed_form_and_limits():
    # the printed forward: output * sigmoid(linear(hidden, gate_weight)), in torch
    rng = np.random.default_rng(71)
    L, spec = _rand_layer(rng, T=20, d=8, E=4, k=2, F=8, Fs=6, shared_gate=True)
    f = O.layer_forward(L["x"], L["Wg"], L["W13"], L["W2"], spec, W13s=L["W13s"], W2s=L["W2s"], Wsg=L["Wsg"])
    xs = torch.as_tensor(L["x"])
    shared = _ffn_torch(L["x"], L["W13s"], L["W2s"]) * torch.sigmoid(torch.nn.functional.linear(
        xs, torch.as_tensor(L["Wsg"])[None, :]))
    plain = O.layer_forward(L["x"], L["Wg"], L["W13"], L["W2"], O.LayerSpec(E=4, k=2), W13s=L["W13s"], W2s=L["W2s"])
    np.testing.assert_allclose(f["y"], plain["y"] - plain["shared"]["Y"] + shared.numpy(), rtol=1e-12, atol=1e-12)
    # a zero gate weight halves the shared output
    z = O.layer_forward(L["x"], L["Wg"], L["W13"], L["W2"], spec, W13s=L["W13s"], W2s=L["W2s"], Wsg=np.zeros(8))
    np.testing.assert_allclose(z["y"], plain["y"] - 0.5 * plain["shared"]["Y"], rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ routing margins

def _brute_margin(row, k):
    """Pure Python: the smallest selected key minus the largest unselected key, the
    selected set taken from the brute-force top-k (inf when every expert is selected)."""
    sel = set(O.brute_force_topk(row, k))
    if len(sel) == len(row):
        return math.inf
    return min(float(row[e]) for e in sel) - max(float(row[e]) for e in range(len(row)) if e not in sel)


def test_margins_match_brute_force_and_distance_to_a_flip():
    rng = np.random.default_rng(81)
    T, E = 30, 7
    keys = rng.standard_normal((T, E))
    for k in range(1, E + 1):
        m = O.margins(keys, k)
        assert m.shape == (T,)
        for t in range(T):
            assert m[t] == _brute_margin(keys[t], k)
    assert np.all(O.margins(keys, E) == np.inf)
    # an exact tie at the k-th place has margin 0; a tie inside the selection does not matter
    row = np.array([[3.0, 1.0, 2.0, 1.0, 0.5]])
    assert O.margins(row, 3)[0] == 0.0
    assert O.margins(row, 2)[0] == 1.0
    assert O.margins(row, 4)[0] == 0.5
    # the margin is the distance to a flip: moving the k-th key down and the (k+1)-th up by
    # just under half of it keeps the selected set, by just over half of it changes the set
    k = 3
    m = O.margins(keys, k)
    for t in range(T):
        order = np.argsort(-keys[t], kind="stable")
        s_last, u_first = order[k - 1], order[k]
        for frac, same in ((0.49, True), (0.51, False)):
            p = keys[t].copy()
            p[s_last] -= frac * m[t]
            p[u_first] += frac * m[t]
            moved = set(O.topk(p[None, :], k)[0].tolist()) != set(order[:k].tolist())
            assert moved != same, (t, frac)


def test_group_limited_route_margin_matches_brute_force():
    """The margin of a group-limited token is the nearer of its two decisions: the gap between
    the last kept and the first dropped group score, and the key gap inside the kept groups."""
    from itertools import combinations
    rng = np.random.default_rng(82)
    T, E, G, gk, k = 40, 16, 4, 2, 4
    n, mpick = E // G, k // gk
    logits = rng.standard_normal((T, E))
    spec = O.LayerSpec(E=E, k=k, score="sigmoid", num_groups=G, group_topk=gk)
    r = O.route(logits, spec)
    for t in range(T):
        row = [float(v) for v in r["keys"][t]]
        # group scores added from the largest key down, as the oracle states
        score = []
        for g in range(G):
            acc = 0.0
            for v in sorted(row[g * n:(g + 1) * n], reverse=True)[:mpick]:
                acc += v
            score.append(acc)
        kept = max(combinations(range(G), gk), key=lambda S: sum(score[g] for g in S))
        ranked = sorted(score, reverse=True)
        gmargin = ranked[gk - 1] - ranked[gk]
        pool = [e for g in sorted(kept) for e in range(g * n, (g + 1) * n)]
        inner = sorted((row[e] for e in pool), reverse=True)
        kmargin = inner[k - 1] - inner[k]
        assert r["margin"][t] == min(gmargin, kmargin), t
        assert r["margin"][t] > 0


# ------------------------------------------------------------------ router-path backward

_RP_CASES = [
    dict(score="softmax", k=2, aux=0.7, bias="bg"),
    dict(score="sigmoid", k=3, aux=0.0, bias="expert_bias", extra=dict(scaling=2.5)),
    dict(score="softmax", k=2, aux=0.2, bias=None, extra=dict(z_coeff=0.05, seq_aux_coeff=0.3, seq_len=4)),
    dict(score="softmax", k=1, aux=0.4, bias="bg", extra=dict(pre_softmax=True)),
    dict(score="sqrtsoftplus", k=2, aux=0.3, bias="expert_bias"),
]


def _router_path_loss(x_router, x_expert, Wg, bg, eb, Yfull, dy, spec):
    """L = sum(dy * y) + aux + z + seq_aux where the router sees x_router and every expert
    output is frozen at Yfull [T, E, d] (computed from x_expert)."""
    logits = O.gate_logits(x_router, Wg, bg)
    r = O.route(logits, spec, eb)
    T = x_expert.shape[0]
    y = np.zeros_like(x_expert)
    for t in range(T):
        for j in range(spec.k):
            y[t] += r["w"][t, j] * Yfull[t, r["idx"][t, j]]
    return float(np.sum(dy * y) + r["aux"] + r["z"] + r["seq_aux"])


@pytest.mark.parametrize("case", _RP_CASES)
def test_router_path_backward_equals_layer_backward_and_differences(case):
    rng = np.random.default_rng(83)
    extra = dict(case.get("extra", {}))
    scaling = extra.pop("scaling", 1.0)
    L, spec = _rand_layer(rng, T=16, d=8, E=5, k=case["k"], F=6, score=case["score"], scaling=scaling,
                          aux=case["aux"], bias=case["bias"], **extra)
    keys = O.selection_keys(O.gate_logits(L["x"], L["Wg"], L["bg"]), spec.score, L["expert_bias"])
    assert O.margins(keys, spec.k).min() > 1e-4
    f = O.layer_forward(L["x"], L["Wg"], L["W13"], L["W2"], spec, bg=L["bg"], expert_bias=L["expert_bias"])
    b = O.layer_backward(f, L["x"], L["Wg"], L["W13"], L["W2"], L["dy"], spec, daux=1.0)
    rp = O.router_path_backward(f, L["x"], L["Wg"], L["dy"], spec, daux=1.0)
    for name in ("dw", "dlogits", "dWg", "dbg", "dx_router"):
        np.testing.assert_allclose(rp[name], b[name], rtol=1e-12, atol=1e-14, err_msg=name)
    # central differences with the experts frozen: every token's output under every expert
    Yfull = np.stack([np.stack([O.swiglu_forward(L["x"][t:t + 1], L["W13"][e], L["W2"][e])[2][0]
                                for e in range(spec.E)]) for t in range(16)])
    args = lambda xr, Wg, bg: _router_path_loss(xr, L["x"], Wg, bg, L["expert_bias"], Yfull, L["dy"], spec)  # noqa: E731
    h = 1e-6
    params = [("x", "dx_router"), ("Wg", "dWg")] + ([("bg", "dbg")] if L["bg"] is not None else [])
    for pname, gname in params:
        P = (L["x"] if pname == "x" else L[pname]).copy()
        flat = P.reshape(-1)
        for i in rng.choice(flat.size, size=min(flat.size, 30), replace=False):
            old = flat[i]
            vals = []
            for step in (h, -h):
                flat[i] = old + step
                xr = P if pname == "x" else L["x"]
                Wg = P if pname == "Wg" else L["Wg"]
                bg = P if pname == "bg" else L["bg"]
                vals.append(args(xr, Wg, bg))
            flat[i] = old
            fd = (vals[0] - vals[1]) / (2 * h)
            an = rp[gname].reshape(-1)[i]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (pname, i, fd, an)


def test_router_path_backward_of_the_fp8_layer_matches_differences():
    """The e4m3 layer's experts do not depend on Wg or bg, so the loss's derivatives in those
    are the router-path gradients the oracle returns for it."""
    rng = np.random.default_rng(84)
    T, d, E, k, F = 6, 128, 4, 2, 128
    spec = O.LayerSpec(E=E, k=k, score="softmax", aux_coeff=0.5)
    x = rng.standard_normal((T, d))
    Wg = rng.standard_normal((E, d)) / np.sqrt(d)
    bg = rng.standard_normal(E) * 0.3
    dy = rng.standard_normal((T, d))
    q13 = [O.quantize_blocks(rng.standard_normal((2 * F, d)).astype(np.float32) * 0.05, 128) for _ in range(E)]
    q2 = [O.quantize_blocks(rng.standard_normal((d, F)).astype(np.float32) * 0.05, 128) for _ in range(E)]
    W13q, W13s = np.stack([a for a, _ in q13]), np.stack([b for _, b in q13])
    W2q, W2s = np.stack([a for a, _ in q2]), np.stack([b for _, b in q2])
    assert O.margins(O.gate_logits(x, Wg, bg), k).min() > 1e-4

    def loss(Wg_, bg_):
        f = O.layer_forward_fp8(x, Wg_, W13q, W13s, W2q, W2s, spec, bg=bg_)
        return float(np.sum(dy * f["y"]) + f["route"]["aux"])

    f = O.layer_forward_fp8(x, Wg, W13q, W13s, W2q, W2s, spec, bg=bg)
    rp = O.router_path_backward(f, x, Wg, dy, spec, daux=1.0)
    h = 1e-6
    for P, gname, pick in ((Wg, "dWg", 30), (bg, "dbg", E)):
        flat = P.reshape(-1)
        for i in rng.choice(flat.size, size=pick, replace=False):
            old = flat[i]
            flat[i] = old + h
            lp = loss(Wg, bg)
            flat[i] = old - h
            lm = loss(Wg, bg)
            flat[i] = old
            fd = (lp - lm) / (2 * h)
            an = rp[gname].reshape(-1)[i]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (gname, i, fd, an)
    # dx_router is dlogits through the router's weight
    np.testing.assert_allclose(rp["dx_router"], rp["dlogits"] @ Wg, rtol=1e-12, atol=1e-14)
