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
    shape = W.LAYERS[cid]
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


class _LazyQuantised:
    """Per-expert e4m3 codes and scales of a stacked fp32 master, made by the oracle's
    quantiser on first access (a full-size stack is too large to quantise whole on the host)."""

    def __init__(self, master):
        self.master, self.cache = master, {}
        E, R, C = master.shape
        self.q, self.s = _View(self, 0, (E, R, C)), _View(self, 1, (E, R // 128, C // 128))

    def get(self, e):
        if e not in self.cache:
            self.cache[e] = O.quantize_blocks(self.master[e], 128)
        return self.cache[e]


class _View:
    def __init__(self, owner, which, shape):
        self.owner, self.which, self.shape = owner, which, shape

    def __getitem__(self, e):
        return self.owner.get(int(e))[self.which]


def test_full_size_fp8_layer_on_sampled_tokens():
    """The e4m3 skewed layer at full size: GPU weight quantisation and the permuted e4m3 rows
    bit-exact for the sampled tokens' experts, y and the router-path dx within the flip
    bound of the reduced fp8 test, routing of every token against the oracle's."""
    from test_gpu_fp8 import _check_within, _flip_bound
    torch = torch_mod()
    from mixture_experts_layer_aux_amd import _lib as L
    shape = W.LAYERS[5]
    T, d, E, k, F = shape.T, shape.d, shape.E, shape.k, shape.F
    spec = spec_of(shape)
    cfg = L.config_from_shape(shape)
    inp = W.make_inputs(shape, seed=5)
    print(f"full-size fp8 layer {shape.name}: T={T} d={d} E={E} k={k} F={F}", flush=True)
    dv = dev()
    q13 = torch.empty(E, 2 * F, d, dtype=torch.uint8, device=dv)
    s13 = torch.empty(E * 2 * F // 128, d // 128, dtype=torch.float32, device=dv)
    q2 = torch.empty(E, d, F, dtype=torch.uint8, device=dv)
    s2 = torch.empty(E * d // 128, F // 128, dtype=torch.float32, device=dv)
    m = to_dev(inp["W13"])
    L.quantize_fp8(m.view(E * 2 * F, d), 128, q13.view(E * 2 * F, d), s13)
    del m
    m = to_dev(inp["W2"])
    L.quantize_fp8(m.view(E * d, F), 128, q2.view(E * d, F), s2)
    del m
    Wt = dict(Wg=to_dev(inp["Wg"]), bg=to_dev(inp["bg"]), W13=q13, W13_scale=s13.view(-1), W2=q2,
              W2_scale=s2.view(-1))
    x = to_dev(inp["x"])
    dy = to_dev(W.to_f32(inp["dy"], shape.act).copy())
    S = L.alloc_saved(cfg, dv)
    G = L.alloc_grads(cfg, dv, with_dbg=True)
    ws = L.alloc_workspace(cfg, dv)
    y = torch.empty(T, d, dtype=torch.float32, device=dv)
    dx = torch.empty(T, d, dtype=torch.float32, device=dv)
    stats = torch.empty(L.MOE_NSTATS, dtype=torch.float32, device=dv)
    L.layer_fwd(cfg, Wt, x, S, y, stats, ws)
    L.layer_bwd(cfg, Wt, S, x, dy, 1.0, dx, G, ws)
    torch.cuda.synchronize()
    x64 = f64(inp["x"], shape.act)
    logits = O.gate_logits(x64, inp["Wg"], inp["bg"])
    assert rel_err(to_np(S["logits"]), logits) < 1e-5, "logits"
    r = O.route(logits, spec, inp["expert_bias"])
    moved = routing_moved(to_np(S["idx"]), r)
    if not moved.any():
        assert np.array_equal(to_np(S["counts"]), r["counts"])
    rng = np.random.default_rng(1005)
    toks = np.sort(rng.choice(np.where(r["margin"] > MARGIN)[0], size=4, replace=False))
    lw13, lw2 = _LazyQuantised(inp["W13"]), _LazyQuantised(inp["W2"])
    row_of = to_np(S["row_of"])
    idx_gpu = to_np(S["idx"])
    dy64 = f64(inp["dy"], shape.act)
    for t in toks:
        f = O.layer_forward_fp8(x64[t:t + 1], inp["Wg"], lw13.q, lw13.s, lw2.q, lw2.s, spec, bg=inp["bg"])
        assert np.array_equal(np.sort(f["route"]["idx"][0]), np.sort(r["idx"][t]))
        # the GPU's e4m3 weights of this token's experts and its permuted e4m3 rows
        for e in r["idx"][t]:
            oq, os_ = lw13.get(int(e))
            assert np.array_equal(q13[e].cpu().numpy(), oq), f"W13 codes of expert {e}"
            assert np.array_equal(s13.view(E, 2 * F // 128, d // 128)[e].cpu().numpy(), os_), f"W13 scales of {e}"
            oq, os_ = lw2.get(int(e))
            assert np.array_equal(q2[e].cpu().numpy(), oq), f"W2 codes of expert {e}"
            assert np.array_equal(s2.view(E, d // 128, F // 128)[e].cpu().numpy(), os_), f"W2 scales of {e}"
        for j in range(k):
            rw = int(row_of[t, j])
            assert np.array_equal(S["x_perm"][rw].cpu().numpy(), f["x_q"][0]), "permuted e4m3 row"
            assert np.array_equal(S["x_perm_scale"][rw].cpu().numpy(), f["x_scale"][0]), "permuted row scales"
        # y_t within the legitimate Act-rounding flips (the GPU's slot order may differ)
        rf = f["route"]
        bY = _flip_bound(f, lw2.q, lw2.s, spec)
        ybound = np.einsum("tk,tkd->td", np.abs(rf["w"]), bY[f["perm"].row_of])
        _check_within(to_np(y[t:t + 1]), f["y"], ybound, 2e-3, f"y[{t}]")
        # router-path dx_t (aux off): the bound through dw, the selected softmax and Wg
        b = O.router_path_backward(f, x64[t:t + 1], inp["Wg"], dy64[t:t + 1], spec)
        bdw = np.einsum("td,tkd->tk", np.abs(dy64[t:t + 1]), bY[f["perm"].row_of])
        w = np.abs(rf["w"])
        bdl = w * bdw + w * np.sum(w * bdw, axis=1, keepdims=True)
        bdx = np.einsum("tk,tkd->td", bdl, np.abs(inp["Wg"].astype(np.float64))[rf["idx"]])
        _check_within(to_np(dx[t:t + 1]), b["dx_router"], bdx, 2e-2, f"dx[{t}] (router path)")
        assert np.array_equal(np.sort(idx_gpu[t]), np.sort(rf["idx"][0]))
