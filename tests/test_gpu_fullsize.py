"""Parity at the full layer sizes, on outputs the oracle can compute one at a time.

The whole layer runs on the GPU at its real T, d, E, k and F through moe_layer_fwd and
moe_layer_bwd (the kernels and launch shapes the benchmark times).  The oracle then
recomputes, independently and in fp64:
  * the logits and routing of every token (indices bit-exact wherever the top-k margin
    exceeds 1e-5), the expert counts and the load statistics;
  * y_t and dx_t of a seeded sample of tokens whose margin exceeds 1e-3, each from the
    token alone (the aux-loss part of dlogits, which needs every token's counts, comes
    from the oracle's router backward over all tokens);
  * the weight gradients of the expert with the fewest rows, from exactly its rows, and
    the exact zeros of an expert with none.
"""
import numpy as np
import pytest

from helpers import (MARGIN, O, W, check_grad, dev, f64, rel_err, routing_moved, spec_of, to_dev, to_np, tol,
                     torch_mod)

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

N_TOKENS = 6


def _run_full(shape, inp):
    torch = torch_mod()
    from mixture_experts_layer_aux_amd import _lib as L
    cfg = L.config_from_shape(shape)
    d = dev()
    Wt = dict(Wg=to_dev(inp["Wg"]), bg=to_dev(inp["bg"]), expert_bias=to_dev(inp["expert_bias"]),
              W13=to_dev(inp["W13"]), W2=to_dev(inp["W2"]), W13s=to_dev(inp["W13s"]), W2s=to_dev(inp["W2s"]))
    x = to_dev(inp["x"])
    dy = to_dev(W.to_f32(inp["dy"], shape.act).copy())
    S = L.alloc_saved(cfg, d)
    G = L.alloc_grads(cfg, d)
    ws = L.alloc_workspace(cfg, d)
    y = torch.empty(shape.T, shape.d, dtype=torch.float32, device=d)
    dx = torch.empty(shape.T, shape.d, dtype=torch.float32, device=d)
    stats = torch.empty(L.MOE_NSTATS, dtype=torch.float32, device=d)
    L.layer_fwd(cfg, Wt, x, S, y, stats, ws)
    torch.cuda.synchronize()
    fwd_state = {n: S[n].clone() for n in ("idx", "w", "counts", "logits")}
    L.layer_bwd(cfg, Wt, S, x, dy, 1.0, dx, G, ws)
    torch.cuda.synchronize()
    for n, t in fwd_state.items():       # the backward reads the saved routing, never writes it
        assert torch.equal(S[n], t), f"saved {n} changed during the backward"
    out = dict(idx=to_np(S["idx"]), counts=to_np(S["counts"]), logits=to_np(S["logits"]), y=to_np(y),
               dx=to_np(dx), stats=to_np(stats), dW13=G["dW13"], dW2=G["dW2"])
    del Wt, S, ws, x, dy
    return out


@pytest.mark.parametrize("cid", [2, 3, 4])
def test_full_size_layer_on_sampled_outputs(cid):
    torch = torch_mod()
    shape = W.CONFIGS[cid]
    spec = spec_of(shape)
    inp = W.make_inputs(shape, seed=cid)
    print(f"full-size layer {shape.name}: T={shape.T} d={shape.d} E={shape.E} k={shape.k} F={shape.F}", flush=True)
    got = _run_full(shape, inp)
    x64 = f64(inp["x"], shape.act)
    logits = O.gate_logits(x64, inp["Wg"], inp["bg"])
    assert rel_err(got["logits"], logits) < 1e-5, "logits"
    r = O.route(logits, spec, inp["expert_bias"])
    idx_gpu = got["idx"]
    moved = routing_moved(idx_gpu, r)
    if not moved.any():
        assert np.array_equal(got["counts"], r["counts"])
        assert got["stats"][1] == pytest.approx(r["maxvio"], rel=1e-6)
        if shape.score == "softmax" and shape.aux_coeff:
            assert got["stats"][0] == pytest.approx(r["aux"], rel=1e-4)
    # a seeded sample of tokens, recomputed one by one
    rng = np.random.default_rng(1000 + cid)
    cand = np.where(r["margin"] > MARGIN)[0]
    toks = np.sort(rng.choice(cand, size=N_TOKENS, replace=False))
    W13v, W2v = W.ExpertView(inp["W13"], shape.act), W.ExpertView(inp["W2"], shape.act)
    W13s, W2s = f64(inp["W13s"], shape.act), f64(inp["W2s"], shape.act)
    dy64 = f64(inp["dy"], shape.act)
    # aux-loss part of dlogits (zero mixing-weight gradient isolates it), all tokens
    dl_aux = O.router_backward(logits, r["idx"], r["w"], np.zeros_like(r["w"]), spec, counts=r["counts"], daux=1.0)
    y_ref, dx_ref = [], []
    for t in toks:
        f = O.layer_forward(x64[t:t + 1], inp["Wg"], W13v, W2v, spec, bg=inp["bg"], expert_bias=inp["expert_bias"],
                            W13s=W13s, W2s=W2s)
        assert np.array_equal(np.sort(f["route"]["idx"][0]), np.sort(r["idx"][t]))
        b = O.layer_backward(f, x64[t:t + 1], inp["Wg"], W13v, W2v, dy64[t:t + 1], spec, W13s=W13s, W2s=W2s,
                             daux=0.0, sparse_expert_grads=True)
        y_ref.append(f["y"][0])
        dx_ref.append(b["dx"][0] + dl_aux[t] @ inp["Wg"].astype(np.float64))
    err = rel_err(got["y"][toks], np.stack(y_ref))
    assert err < tol(shape), f"y (sampled tokens): {err:.3e}"
    err = rel_err(got["dx"][toks], np.stack(dx_ref))
    assert err < tol(shape), f"dx (sampled tokens): {err:.3e}"
    # weight gradients of the smallest non-empty expert, from exactly its rows
    counts = r["counts"]
    live = np.where(counts > 0)[0]
    e = int(live[np.argmin(counts[live])])
    if not np.any(idx_gpu[moved] == e) and not np.any(r["idx"][moved] == e):
        rows_t, rows_j = np.where(r["idx"] == e)
        Xe = x64[rows_t]
        dYe = r["w"][rows_t, rows_j][:, None] * dy64[rows_t]
        H, _, _ = O.swiglu_forward(Xe, W13v[e], W2v[e])
        g = O.swiglu_backward(Xe, W13v[e], W2v[e], H, dYe)
        check_grad(f"dW13[{e}] ({counts[e]} rows)", got["dW13"][e].double().cpu().numpy(), g["dW13"], shape)
        check_grad(f"dW2[{e}] ({counts[e]} rows)", got["dW2"][e].double().cpu().numpy(), g["dW2"], shape)
    for e0 in np.where(counts == 0)[0][:4]:
        if not np.any(idx_gpu[moved] == e0):
            assert not torch.any(got["dW13"][e0]) and not torch.any(got["dW2"][e0]), f"expert {e0} has no rows"
