"""Parity at the full layer sizes, on outputs the oracle can compute one at a time.

The whole layer runs on the GPU at its real T, d, E, k and F through moe_layer_fwd and
moe_layer_bwd (the kernels and launch shapes the benchmark times).  The oracle then
recomputes, independently and in fp64:
  * the logits and routing of every token (indices bit-exact wherever the top-k margin
    exceeds 1e-5), the expert counts and the load statistics;
  * y_t and dx_t of a seeded sample of 64 tokens whose margin exceeds 1e-3, from those
    tokens alone (the aux-loss part of dlogits, which needs every token's counts, comes
    from the oracle's router backward over all tokens);
  * the weight gradients of the expert with the most rows and of the one with the fewest,
    on a seeded 256-column slice, element by element, from exactly the rows the GPU gave
    them (its routing, pinned: it equals the oracle's wherever a token is not at a
    near-tie, which is asserted), and the exact zeros of experts with none.
"""
import numpy as np
import pytest

from helpers import (MARGIN, O, W, check_wgrad, dev, f64, grad_sig2, rel_err, routing_moved, spec_of, to_dev, to_np,
                     tol, torch_mod)

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

N_TOKENS = 64
SLICE = 256


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
    f = O.layer_forward(x64[toks], inp["Wg"], W13v, W2v, spec, bg=inp["bg"], expert_bias=inp["expert_bias"],
                        W13s=W13s, W2s=W2s)
    assert np.array_equal(np.sort(f["route"]["idx"], axis=1), np.sort(r["idx"][toks], axis=1))
    b = O.layer_backward(f, x64[toks], inp["Wg"], W13v, W2v, dy64[toks], spec, W13s=W13s, W2s=W2s, daux=0.0,
                         sparse_expert_grads=True)
    err = rel_err(got["y"][toks], f["y"])
    assert err < tol(shape), f"y (sampled tokens): {err:.3e}"
    err = rel_err(got["dx"][toks], b["dx"] + dl_aux[toks] @ inp["Wg"].astype(np.float64))
    assert err < tol(shape), f"dx (sampled tokens): {err:.3e}"
    # weight gradients of the largest and the smallest expert, on a column slice, from the
    # rows the GPU routed to them (ascending token order is the GPU's row order)
    counts_gpu = got["counts"]
    live = np.where(counts_gpu > 0)[0]
    w_gpu = O.mixing_weights(logits, idx_gpu, spec.score, spec.scaling, spec.pre_softmax)
    for e in (int(live[np.argmax(counts_gpu[live])]), int(live[np.argmin(counts_gpu[live])])):
        rows_t, rows_j = np.where(idx_gpu == e)
        assert len(rows_t) == counts_gpu[e]
        Xe = x64[rows_t]
        dYe = w_gpu[rows_t, rows_j][:, None] * dy64[rows_t]
        W13e, W2e = W13v[e].astype(np.float64), W2v[e].astype(np.float64)
        H = Xe @ W13e.T
        Act = O.glu_forward(H, spec.glu)
        dH = O.glu_backward(H, dYe @ W2e, spec.glu)
        c13 = int(rng.integers(0, shape.d // SLICE)) * SLICE
        c2 = int(rng.integers(0, shape.F // SLICE)) * SLICE
        print(f"  expert {e}: {len(rows_t)} rows, dW13 columns {c13}.., dW2 columns {c2}..", flush=True)
        g13 = got["dW13"][e][:, c13:c13 + SLICE].double().cpu().numpy()
        g2 = got["dW2"][e][:, c2:c2 + SLICE].double().cpu().numpy()
        check_wgrad(f"dW13[{e}][:, {c13}:]", g13, dH, Xe[:, c13:c13 + SLICE], 1, 0, grad_sig2(H, dYe, W2e, spec.glu))
        check_wgrad(f"dW2[{e}][:, {c2}:]", g2, dYe, Act[:, c2:c2 + SLICE], 1, 1)
    for e0 in np.where(counts_gpu == 0)[0][:4]:
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
    """The e4m3 skewed layer at full size: GPU weight quantisation and the token's e4m3 rows
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
    # the layer keeps no grouped copy: its fc1 reads the token rows' e4m3 codes, which the
    # same quantiser call reproduces here
    assert "x_perm" not in S
    xq = torch.empty(T, d, dtype=torch.uint8, device=dv)
    xs = torch.empty(T, d // 128, dtype=torch.float32, device=dv)
    L.quantize_fp8(x, 1, xq, xs)
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
    idx_gpu = to_np(S["idx"])
    dy64 = f64(inp["dy"], shape.act)
    for t in toks:
        f = O.layer_forward_fp8(x64[t:t + 1], inp["Wg"], lw13.q, lw13.s, lw2.q, lw2.s, spec, bg=inp["bg"])
        assert np.array_equal(np.sort(f["route"]["idx"][0]), np.sort(r["idx"][t]))
        # the GPU's e4m3 weights of this token's experts and its e4m3 row
        for e in r["idx"][t]:
            oq, os_ = lw13.get(int(e))
            assert np.array_equal(q13[e].cpu().numpy(), oq), f"W13 codes of expert {e}"
            assert np.array_equal(s13.view(E, 2 * F // 128, d // 128)[e].cpu().numpy(), os_), f"W13 scales of {e}"
            oq, os_ = lw2.get(int(e))
            assert np.array_equal(q2[e].cpu().numpy(), oq), f"W2 codes of expert {e}"
            assert np.array_equal(s2.view(E, d // 128, F // 128)[e].cpu().numpy(), os_), f"W2 scales of {e}"
        assert np.array_equal(xq[t].cpu().numpy(), f["x_q"][0]), "e4m3 row"
        assert np.array_equal(xs[t].cpu().numpy(), f["x_scale"][0]), "row scales"
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
