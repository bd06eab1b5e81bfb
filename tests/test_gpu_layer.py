"""End-to-end parity of moe_layer_fwd / moe_layer_bwd against the fp64 oracle.

The oracle routes with its own fp64 logits.  Outputs that depend only on a token's own
routing (y, dx, dw) are compared on the tokens whose top-k margin exceeds 1e-3 in key
space; expert weight gradients are compared on every expert whose token set is the same
on both sides (a token can only move between experts when its margin is below the fp32
logit error, which is checked too); the router weight gradient, a sum over all tokens,
is compared when no token moved.
"""
from dataclasses import replace

import numpy as np
import pytest

from helpers import (MARGIN, O, W, check_layer_grads, dev, oracle_inputs, rel_err, routing_moved, spec_of, to_dev, to_np,
                     tol, torch_mod)

pytestmark = pytest.mark.gpu


def _run_layer(shape, inp, wgrad_stream=None, copy=None, **cfg_extra):
    torch = torch_mod()
    from mixture_experts_layer_aux_amd import _lib as L
    cfg = L.config_from_shape(shape, **cfg_extra)
    d = dev()
    Wt = dict(Wg=to_dev(inp["Wg"]), bg=to_dev(inp["bg"]), expert_bias=to_dev(inp["expert_bias"]),
              W13=to_dev(inp["W13"]), W2=to_dev(inp["W2"]), W13s=to_dev(inp["W13s"]), W2s=to_dev(inp["W2s"]),
              Wsg=to_dev(inp.get("Wsg")))
    x = to_dev(inp["x"])
    dy = to_dev(W.to_f32(inp["dy"], shape.act).copy())     # upstream gradient, fp32
    S = L.alloc_saved(cfg, d, x_perm=copy)     # default: bf16 layers keep no grouped copy of x
    G = L.alloc_grads(cfg, d, with_dbg=inp["bg"] is not None)
    ws = L.alloc_workspace(cfg, d)
    y = torch.empty(shape.T, shape.d, dtype=torch.float32, device=d)
    dx = torch.empty(shape.T, shape.d, dtype=torch.float32, device=d)
    stats = torch.empty(L.MOE_NSTATS, dtype=torch.float32, device=d)
    L.layer_fwd(cfg, Wt, x, S, y, stats, ws)
    L.layer_bwd(cfg, Wt, S, x, dy, 1.0, dx, G, ws, wgrad_stream=wgrad_stream)
    if wgrad_stream is not None:      # copies queued on the caller's stream right after the call
        G = {k: v.clone() for k, v in G.items()}
    torch.cuda.synchronize()
    return dict(y=y, dx=dx, stats=stats, **{f"S_{k}": v for k, v in S.items()}, **G)


def _check_layer(shape, seed, **cfg_extra):
    inp = W.make_inputs(shape, seed=seed)
    got = _run_layer(shape, inp, **cfg_extra)
    o = oracle_inputs(inp, shape)
    spec = spec_of(shape)
    f = O.layer_forward(o["x"], o["Wg"], o["W13"], o["W2"], spec, bg=o["bg"], expert_bias=o["expert_bias"],
                        W13s=o["W13s"], W2s=o["W2s"], Wsg=o["Wsg"])
    b = O.layer_backward(f, o["x"], o["Wg"], o["W13"], o["W2"], o["dy"], spec, W13s=o["W13s"], W2s=o["W2s"],
                         daux=1.0, Wsg=o["Wsg"])
    r = f["route"]
    tl = tol(shape)
    safe = r["margin"] > MARGIN
    idx_gpu = to_np(got["S_idx"])
    moved = routing_moved(idx_gpu, r)     # a token may only be routed differently at a near-tie
    assert rel_err(to_np(got["S_logits"]), f["logits"]) < 1e-5
    assert rel_err(to_np(got["y"]), f["y"], safe) < tl, "y"
    assert rel_err(to_np(got["dx"]), b["dx"], safe) < tl, "dx"
    st = to_np(got["stats"])
    if shape.score == "softmax" and shape.aux_coeff:
        assert st[0] == pytest.approx(r["aux"], rel=1e-4)
    if not moved.any():
        assert np.array_equal(to_np(got["S_counts"]), r["counts"])
        assert st[1] == pytest.approx(r["maxvio"], rel=1e-6)
    same = np.ones(shape.E, dtype=bool)
    for t in np.where(moved)[0]:
        same[idx_gpu[t]] = False
        same[r["idx"][t]] = False
    assert same.sum() >= shape.E - 2 * shape.k * moved.sum()
    # every weight gradient element by element (the router's when no token moved)
    grads = {n: to_np(got[n]) for n in ("dW13", "dW2", "dW13s", "dW2s", "dWg", "dbg", "dWsg") if n in got}
    check_layer_grads(grads, f, b, o, spec, shape, ids=np.where(same)[0], router=not moved.any())
    if getattr(shape, "shared_gate", False):
        gs_err = np.abs(to_np(got["S_gs"]) - f["shared"]["gs"]).max()
        assert gs_err < 1e-5 if shape.act == "bf16" else gs_err < 1e-6, f"gs: {gs_err:.2e}"
    return got


@pytest.mark.parametrize("cid", sorted(W.SMALL))
def test_layer_small(cid):
    _check_layer(W.SMALL[cid], seed=cid)


def test_layer_determinism():
    """Two runs on the same inputs give bit-identical outputs and gradients."""
    torch = torch_mod()
    shape = W.SMALL[3]
    inp = W.make_inputs(shape, seed=3)
    a = _run_layer(shape, inp)
    b = _run_layer(shape, inp)
    for k in a:
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("cid", [3, 4])
def test_layer_two_streams(cid):
    """The expert weight gradients on a second stream of the caller give the same bits as on
    one stream, and the caller's stream sees them when the call returns."""
    torch = torch_mod()
    shape = W.SMALL[cid]
    inp = W.make_inputs(shape, seed=cid)
    one = _run_layer(shape, inp)
    side = torch.cuda.Stream()
    two = _run_layer(shape, inp, wgrad_stream=side)
    for k in one:
        assert torch.equal(one[k], two[k]), k


_GATHER_CASES = {
    "small2": (W.SMALL[2], {}),
    "small3": (W.SMALL[3], {}),
    "small4": (W.SMALL[4], {}),
    "small5": (W.SMALL[5], {}),
    "ragged_t257": (replace(W.SMALL[3], T=257), {}),
    "empty_experts": (replace(W.SMALL[3], T=3, k=2, E=32), {}),
    "fp32_wgrad": (W.SMALL[3], {"wgrad": "f32"}),
}


@pytest.mark.parametrize("case", list(_GATHER_CASES))
def test_layer_token_rows_match_the_grouped_copy(case):
    """saved->x_perm NULL (the fc1 and its weight gradient read the token rows of x through
    token_of) gives the same bits as the layer with the grouped copy of x."""
    torch = torch_mod()
    shape, extra = _GATHER_CASES[case]
    inp = W.make_inputs(shape, seed=21)
    a = _run_layer(shape, inp, copy=True, **extra)
    b = _run_layer(shape, inp, copy=False, **extra)
    assert "S_x_perm" in a and "S_x_perm" not in b
    for k in b:
        assert torch.equal(a[k], b[k]), k


def test_layer_fp32_weight_gradients():
    """The fp32 weight-gradient option of a bf16 layer (the default is bf16)."""
    got = _check_layer(W.SMALL[3], seed=3, wgrad="f32")
    assert got["dW13"].dtype == torch_mod().float32


@pytest.mark.parametrize("variant", ["scaling", "no_shared_sigmoid", "k_equals_E", "one_row_experts", "ragged_split"])
def test_layer_edge_cases(variant):
    base = W.SMALL[3]
    if variant == "scaling":
        shape = replace(W.SMALL[2], scaling=2.5, T=300)
    elif variant == "no_shared_sigmoid":
        shape = replace(base, Fs=0, T=257)
    elif variant == "k_equals_E":
        shape = replace(W.SMALL[2], E=4, k=4, T=130, aux_coeff=0.1)
    elif variant == "ragged_split":
        # the shared expert's weight gradients and the gate's split over the tokens with
        # a short last chunk (384, 384 and 232 tokens)
        shape = replace(base, T=1000)
    else:  # tiny T: every expert gets at most a handful of rows, many get none
        shape = replace(base, T=3, k=2, E=32)
    _check_layer(shape, seed=11)
