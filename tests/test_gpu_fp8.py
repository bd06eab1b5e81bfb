"""Parity of the e4m3 expert path (the skewed 896-expert layer, reduced) with the fp64 oracle.

The quantiser and the permute of e4m3 rows are integer/byte work and must match the
oracle bit for bit.  The GEMMs accumulate products of e4m3 codes on the matrix cores
(not an exactly rounded fp32 sum), so H is compared at a 1e-3 max-abs/rms bar; the per-row
quantisation of Act then decides codes from slightly different values on the two sides,
so a code may differ by one step where the oracle's value sits next to a rounding
midpoint, and nowhere else.  Both roundings are correct results; with 128 values per
scale block one such flip of a large Act element moves an output by several percent of
its RMS, so Y and y are checked element-wise against the oracle's values widened by
exactly the flips that are legitimate (one code step at every Act element the oracle
places within the GEMM error of a midpoint, through |W2| and the mixing weights), plus
2e-3 of the RMS.  The router-path input gradient gets the same treatment (the bound
carried through dw = <dy, Y>, the selected softmax and Wg) with the 2e-2 bar on tokens
with top-k margin > 1e-3; the router weight gradients carry it further through |x|, with the
fp32 rounding of the router backward added (the only part left of dl where a weight saturates).
"""
from dataclasses import replace

import numpy as np
import pytest

from helpers import MARGIN, O, W, dev, f64, rel_err, routing_moved, spec_of, to_dev, to_np, torch_mod

pytestmark = pytest.mark.gpu

SHAPE = W.SMALL_FP8
TOL_H = 1e-3


def _lib():
    from mixture_experts_layer_aux_amd import _lib as L
    L.load()
    return L


def _quantise_gpu(L, src, block_rows):
    torch = torch_mod()
    rows, cols = src.shape
    q = torch.empty(rows, cols, dtype=torch.uint8, device=dev())
    s = torch.empty(rows // block_rows, cols // 128, dtype=torch.float32, device=dev())
    L.quantize_fp8(src, block_rows, q, s)
    return q, s


def _expert_weights(L, inp, shape):
    """e4m3 weights from the fp32 masters on both sides; the two must agree bit for bit."""
    E, F, d = shape.E, shape.F, shape.d
    q13, s13 = _quantise_gpu(L, to_dev(inp["W13"].reshape(E * 2 * F, d)), 128)
    q2, s2 = _quantise_gpu(L, to_dev(inp["W2"].reshape(E * d, F)), 128)
    o13 = [O.quantize_blocks(inp["W13"][e], 128) for e in range(E)]
    o2 = [O.quantize_blocks(inp["W2"][e], 128) for e in range(E)]
    oq13, os13 = np.stack([a for a, _ in o13]), np.stack([b for _, b in o13])
    oq2, os2 = np.stack([a for a, _ in o2]), np.stack([b for _, b in o2])
    assert np.array_equal(q13.cpu().numpy().reshape(oq13.shape), oq13)
    assert np.array_equal(s13.cpu().numpy().reshape(os13.shape), os13)
    assert np.array_equal(q2.cpu().numpy().reshape(oq2.shape), oq2)
    assert np.array_equal(s2.cpu().numpy().reshape(os2.shape), os2)
    gpu = dict(W13=q13.view(E, 2 * F, d), W13_scale=s13.reshape(-1), W2=q2.view(E, d, F), W2_scale=s2.reshape(-1))
    return gpu, dict(W13q=oq13, W13s=os13, W2q=oq2, W2s=os2)


@pytest.mark.parametrize("block_rows", [1, 128])
@pytest.mark.parametrize("src", ["bf16", "f32"])
def test_quantiser_bit_exact(block_rows, src):
    torch = torch_mod()
    L = _lib()
    rng = np.random.default_rng(5 + block_rows)
    v = (rng.standard_normal((256, 640)) * np.exp(rng.uniform(-12, 6, size=(256, 1)))).astype(np.float32)
    v[:128, 128:256] = 0.0                                  # an all-zero block
    v[128:, 256:384] *= 1e-3                                # values far into the subnormal codes
    v[3, 5] = -0.0
    if src == "bf16":
        bits = W.f32_to_bf16_bits(v)
        v = W.bf16_bits_to_f32(bits)
        dv = to_dev(bits)
    else:
        dv = to_dev(v)
    q, s = _quantise_gpu(L, dv, block_rows)
    torch.cuda.synchronize()
    oq, os_ = O.quantize_blocks(v, block_rows)
    assert np.array_equal(s.cpu().numpy(), os_)
    assert np.array_equal(q.cpu().numpy(), oq)


def test_fp8_permute_bit_exact():
    torch = torch_mod()
    L = _lib()
    shape = SHAPE
    cfg = L.config_from_shape(shape)
    inp = W.make_inputs(shape, seed=5, with_dy=False, with_experts=False)
    T, k, E, d, A = shape.T, shape.k, shape.E, shape.d, shape.A
    logits = O.gate_logits(f64(inp["x"], shape.act), inp["Wg"], inp["bg"])
    idx = O.route(logits, spec_of(shape), inp["expert_bias"])["idx"]
    xq, xs = _quantise_gpu(L, to_dev(inp["x"]), 1)
    e = lambda *s_, dt=torch.int32: torch.empty(*s_, dtype=dt, device=dev())  # noqa: E731
    offsets, row_of, token_of = e(E + 1), e(T, k), e(A)
    x_perm, x_perm_scale = e(A, d, dt=torch.uint8), e(A, d // 128, dt=torch.float32)
    ws = L.alloc_workspace(cfg, dev())
    L.permute_fp8(cfg, xq, xs, to_dev(idx.astype(np.int32)), offsets, row_of, token_of, x_perm, x_perm_scale, ws)
    torch.cuda.synchronize()
    p = O.permutation(idx, E)
    oq, os_ = O.quantize_blocks(W.to_f32(inp["x"], shape.act), 1)
    assert np.array_equal(to_np(offsets), p.offsets)
    assert np.array_equal(to_np(row_of), p.row_of)
    assert np.array_equal(x_perm.cpu().numpy(), oq[p.token_of])
    assert np.array_equal(x_perm_scale.cpu().numpy(), os_[p.token_of])


def _check_act_codes(got_q, got_s, act32, ref_q, ref_s):
    """Where a code differs from the oracle's, the GPU's value must still be a rounding of
    a value within the GEMM's accumulation error of the oracle's Act: its distance to the
    oracle's exact Act is at most half a code step plus 1e-3 of the row's RMS."""
    got_s = np.asarray(got_s, dtype=np.float64)
    assert np.all(np.abs(got_s / ref_s - 1.0) <= 1e-4), "Act scales"
    diff = got_q != ref_q
    if diff.any():
        act = act32.astype(np.float64)
        s_full = np.repeat(got_s, 128, axis=1)
        deq = O.e4m3_decode(got_q) * s_full
        half_step = np.maximum(2.0 ** -4 * np.abs(act), 2.0 ** -10 * s_full)
        rms = np.sqrt(np.mean(act ** 2, axis=1, keepdims=True)) * np.ones_like(act)
        bound = half_step + 1e-3 * rms
        worst = np.max(np.abs(deq[diff] - act[diff]) / bound[diff])
        assert worst <= 1.0, f"an Act code differs beyond rounding of a nearby value ({worst:.2f} of the bound)"
    assert diff.mean() < 0.01, f"{diff.mean():.4f} of the Act codes differ"


def _flip_bound(f, W2q, W2s, spec, rel_rms=1e-3):
    """How far Y_perm may legitimately move when the GPU rounds an Act element to the other
    neighbour of a midpoint: for every oracle Act element within rel_rms of its row's RMS
    of a rounding midpoint, one code step times |W2|, summed over the row; per routed row
    and output column."""
    act = f["Act"].astype(np.float32).astype(np.float64)
    s_full = np.repeat(f["Act_scale"].astype(np.float64), 128, axis=1)
    mag = np.abs(f["Act_q"]).astype(np.int64) & 0x7F
    tab = np.append(O._E4M3, O._E4M3[-1])                      # no code above 0x7E
    v = O._E4M3[mag] * s_full
    up = tab[np.minimum(mag + 1, 127)] * s_full
    dn = O._E4M3[np.maximum(mag - 1, 0)] * s_full
    rms = np.sqrt(np.mean(act ** 2, axis=1, keepdims=True))
    a = np.abs(act)
    near_up = np.abs(a - (v + up) / 2) <= rel_rms * rms
    near_dn = np.abs(a - (v + dn) / 2) <= rel_rms * rms
    step = np.where(near_up, up - v, 0.0) + np.where(near_dn, v - dn, 0.0)
    # a sign flip around zero moves the value by at most the smallest step twice
    step = np.where(a <= rel_rms * rms, np.maximum(step, 2 * O._E4M3[1] * s_full), step)
    perm = f["perm"]
    bound = np.zeros((act.shape[0], W2q.shape[1]))
    for e in range(spec.E):
        lo, hi = perm.offsets[e], perm.offsets[e + 1]
        if hi > lo:
            bound[lo:hi] = step[lo:hi] @ np.abs(O.dequantize_blocks(W2q[e], W2s[e], 128)).T
    return bound


def _check_within(got, ref, bound, eps, name, mask=None):
    """|got - ref| <= bound + eps * rms(ref) element-wise (rows in mask)."""
    got, ref = np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    if mask is not None:
        got, ref, bound = got[mask], ref[mask], bound[mask]
    assert ref.size, f"{name}: no element to compare"
    rms = np.sqrt(np.mean(ref ** 2))
    excess = np.abs(got - ref) - bound
    worst = float(np.max(excess) / rms)
    assert worst <= eps, f"{name}: exceeds the flip bound by {worst:.3e} of the RMS"


def test_fp8_grouped_experts_forward():
    torch = torch_mod()
    L = _lib()
    shape = SHAPE
    cfg = L.config_from_shape(shape)
    inp = W.make_inputs(shape, seed=5, with_dy=False)
    T, k, E, d, F, A = shape.T, shape.k, shape.E, shape.d, shape.F, shape.A
    wg, wo = _expert_weights(L, inp, shape)
    # routing and x quantisation of the oracle; the GPU's own quantiser gives the same bytes
    spec = spec_of(shape)
    f = O.layer_forward_fp8(f64(inp["x"], shape.act), inp["Wg"], wo["W13q"], wo["W13s"], wo["W2q"], wo["W2s"], spec,
                            bg=inp["bg"])
    p = f["perm"]
    xq, xs = _quantise_gpu(L, to_dev(inp["x"]), 1)
    tok = torch.from_numpy(p.token_of.astype(np.int64)).to(dev())
    x_perm, x_perm_scale = xq[tok].contiguous(), xs[tok].contiguous()
    off = to_dev(p.offsets.astype(np.int32))
    e32 = lambda *s_: torch.empty(*s_, dtype=torch.float32, device=dev())  # noqa: E731
    H, Y = e32(A, 2 * F), e32(A, d)
    Act = torch.empty(A, F, dtype=torch.uint8, device=dev())
    Act_scale = e32(A, F // 128)
    ws = L.alloc_workspace(cfg, dev())
    L.grouped_gemm_swiglu_fp8(cfg, x_perm, x_perm_scale, off, wg["W13"], wg["W13_scale"], wg["W2"], wg["W2_scale"],
                              H, Act, Act_scale, Y, ws)
    torch.cuda.synchronize()
    err = rel_err(to_np(H), f["H"])
    assert err < TOL_H, f"H: {err:.3e}"
    _check_act_codes(Act.cpu().numpy(), Act_scale.cpu().numpy(), f["Act"].astype(np.float32), f["Act_q"],
                     f["Act_scale"])
    # Y: the oracle's, moved at most by the legitimate Act code flips, plus the GEMM's own error
    bound = _flip_bound(f, wo["W2q"], wo["W2s"], spec)
    _check_within(to_np(Y), f["Y_perm"], bound, 2e-3, "Y")
    # H may be skipped
    Y2 = e32(A, d)
    L.grouped_gemm_swiglu_fp8(cfg, x_perm, x_perm_scale, off, wg["W13"], wg["W13_scale"], wg["W2"], wg["W2_scale"],
                              None, Act, Act_scale, Y2, ws)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2)
    # the token rows' codes and scales read through token_of: the same bits
    gH, gY = e32(A, 2 * F), e32(A, d)
    gAct, gAct_scale = torch.empty_like(Act), e32(A, F // 128)
    L.grouped_gemm_swiglu_fp8(cfg, xq, xs, off, wg["W13"], wg["W13_scale"], wg["W2"], wg["W2_scale"], gH, gAct,
                              gAct_scale, gY, ws, token_of=to_dev(p.token_of.astype(np.int32)))
    torch.cuda.synchronize()
    for name, a, b in (("H", H, gH), ("Act", Act, gAct), ("Act_scale", Act_scale, gAct_scale), ("Y", Y, gY)):
        assert torch.equal(a, b), f"{name}: token_of gather differs from the grouped copy"


def test_fp8_layer_forward_and_router_backward():
    _check_fp8_layer(SHAPE, seed=5)


# Degenerate shapes of the e4m3 layer: one token (16 one-row experts, the rest empty), a
# token count that leaves a ragged last permute chunk, and a hot expert that every token
# selects (its logit bias pushed to +40: one full 256-row tile, near-zero weights elsewhere).
# (seed 13 gives the single token a top-k margin of 0.033, so its outputs are compared)
FP8_EDGE = {
    "one_token": (replace(SHAPE, name="fp8-one-token", T=1), 13),
    "ragged_chunk": (replace(SHAPE, name="fp8-ragged", T=200), 11),
    "one_hot_expert": (replace(SHAPE, name="fp8-one-hot", T=256, skew_beta=40.0), 11),
    # SiTU-GLU in the fp8 fc1 epilogue (The Ultimate MoE Training Handbook, §3.4 Activation)
    "situ_glu": (replace(SHAPE, name="fp8-situ", T=300, glu="situ", glu_c=0.3, glu_c_linear=0.5), 11),
    # 512 rows per expert on average: the GEMMs take 256 x 128 tiles and the standalone
    # Act quantiser (the other cases take 128 x 256 tiles with Act quantised in fc1)
    "few_experts": (replace(SHAPE, name="fp8-few-experts", E=32, T=1024), 11),
}


@pytest.mark.parametrize("case", list(FP8_EDGE))
def test_fp8_layer_edge_cases(case):
    shape, seed = FP8_EDGE[case]
    _check_fp8_layer(shape, seed)


def test_fp8_layer_with_the_grouped_copy():
    _check_fp8_layer(replace(SHAPE, T=300), seed=7, copy=True)


@pytest.mark.parametrize("case", ["reduced", "one_token", "ragged_chunk"])
def test_fp8_layer_token_rows_match_the_grouped_copy(case):
    """The e4m3 layer without saved->x_perm (its fc1 reads the token rows' codes through
    token_of) gives the same bits as with the grouped copy."""
    torch = torch_mod()
    L = _lib()
    shape, seed = (SHAPE, 5) if case == "reduced" else FP8_EDGE[case]
    cfg = L.config_from_shape(shape)
    inp = W.make_inputs(shape, seed=seed)
    wg, _ = _expert_weights(L, inp, shape)
    Wt = dict(Wg=to_dev(inp["Wg"]), bg=to_dev(inp["bg"]), **wg)
    x = to_dev(inp["x"])
    dy = to_dev(W.to_f32(inp["dy"], shape.act).copy())
    out = []
    for copy in (True, False):
        S = L.alloc_saved(cfg, dev(), x_perm=copy)
        G = L.alloc_grads(cfg, dev(), with_dbg=True)
        ws = L.alloc_workspace(cfg, dev())
        y = torch.empty(shape.T, shape.d, dtype=torch.float32, device=dev())
        dx = torch.empty_like(y)
        stats = torch.empty(L.MOE_NSTATS, dtype=torch.float32, device=dev())
        L.layer_fwd(cfg, Wt, x, S, y, stats, ws)
        L.layer_bwd(cfg, Wt, S, x, dy, 1.0, dx, G, ws)
        torch.cuda.synchronize()
        out.append(dict(y=y, dx=dx, stats=stats, **{f"S_{k}": v for k, v in S.items()}, **G))
    a, b = out
    assert "S_x_perm" in a and "S_x_perm" not in b
    for k in b:
        assert torch.equal(a[k], b[k]), k


def _check_fp8_layer(shape, seed, copy=None):
    torch = torch_mod()
    L = _lib()
    cfg = L.config_from_shape(shape)
    inp = W.make_inputs(shape, seed=seed)
    T, d, E = shape.T, shape.d, shape.E
    wg, wo = _expert_weights(L, inp, shape)
    Wt = dict(Wg=to_dev(inp["Wg"]), bg=to_dev(inp["bg"]), **wg)
    x = to_dev(inp["x"])
    dy = to_dev(W.to_f32(inp["dy"], shape.act).copy())
    S = L.alloc_saved(cfg, dev(), x_perm=copy)
    G = L.alloc_grads(cfg, dev(), with_dbg=True)
    assert "dW13" not in G
    ws = L.alloc_workspace(cfg, dev())
    y = torch.empty(T, d, dtype=torch.float32, device=dev())
    dx = torch.empty(T, d, dtype=torch.float32, device=dev())
    stats = torch.empty(L.MOE_NSTATS, dtype=torch.float32, device=dev())
    L.layer_fwd(cfg, Wt, x, S, y, stats, ws)
    L.layer_bwd(cfg, Wt, S, x, dy, 1.0, dx, G, ws)
    torch.cuda.synchronize()
    spec = spec_of(shape)
    xo = f64(inp["x"], shape.act)
    f = O.layer_forward_fp8(xo, inp["Wg"], wo["W13q"], wo["W13s"], wo["W2q"], wo["W2s"], spec, bg=inp["bg"])
    b = O.router_path_backward(f, xo, inp["Wg"], f64(inp["dy"], shape.act), spec)
    r = f["route"]
    safe = r["margin"] > MARGIN
    moved = routing_moved(to_np(S["idx"]), r)
    # the e4m3 rows are the oracle's bytes (the saved grouped copy, or the token rows the
    # layer quantises in its workspace, which the same quantiser call reproduces)
    tok = f["perm"].token_of
    if "x_perm" in S:
        assert np.array_equal(S["x_perm"].cpu().numpy(), f["x_q"][tok])
        assert np.array_equal(S["x_perm_scale"].cpu().numpy(), f["x_scale"][tok])
    else:
        xq, xs = _quantise_gpu(L, x, 1)
        assert np.array_equal(xq.cpu().numpy(), f["x_q"]) and np.array_equal(xs.cpu().numpy(), f["x_scale"])
        assert np.array_equal(to_np(S["token_of"]), tok)
    # y: the combine of the per-row bound (routing equal on the compared tokens)
    ybound = np.einsum("tk,tkd->td", np.abs(r["w"]), _flip_bound(f, wo["W2q"], wo["W2s"], spec)[f["perm"].row_of])
    _check_within(to_np(y), f["y"], ybound, 2e-3, "y", safe)
    # dx of the router path: the Y bound through dw = <dy, Y>, the softmax over the selected
    # logits (dl_S = w dw - w <w, dw>) and dl Wg
    bY = _flip_bound(f, wo["W2q"], wo["W2s"], spec)
    dyo = np.abs(f64(inp["dy"], shape.act))
    bdw = np.einsum("td,tkd->tk", dyo, bY[f["perm"].row_of])
    w = np.abs(r["w"])
    bdl = w * bdw + w * np.sum(w * bdw, axis=1, keepdims=True)
    bdx = np.einsum("tk,tkd->td", bdl, np.abs(inp["Wg"].astype(np.float64))[r["idx"]])
    _check_within(to_np(dx), b["dx_router"], bdx, 2e-2, "dx (router path)", safe)
    if not moved.any():
        # dWg = dl^T x and dbg = column sums of dl, element-wise: the dl bound above, with the
        # fp32 error of the dot products dw = <dy, Y> (d terms) added to the flip bound, plus
        # the fp32 rounding of dl = w dw - w <w, dw>.  When one weight saturates at 1 (the hot
        # expert), dl is a difference of nearly equal terms and these rounding terms are all
        # that is left of it, so a relative bar would compare rounding noise.
        eps32 = 2.0 ** -23
        Yrows = np.abs(f["Y_perm"])[f["perm"].row_of]
        bdw_all = bdw + d * eps32 * np.einsum("td,tkd->tk", dyo, Yrows)
        wdw = np.abs(r["w"] * b["dw"])
        bdl_all = (w * bdw_all + w * np.sum(w * bdw_all, axis=1, keepdims=True)
                   + (shape.k + 2) * eps32 * (wdw + w * np.sum(wdw, axis=1, keepdims=True)))
        bl = np.zeros((T, E))
        np.put_along_axis(bl, r["idx"], bdl_all, axis=1)
        _check_within(to_np(G["dWg"]), b["dWg"], bl.T @ np.abs(xo), 2e-2, "dWg")
        _check_within(to_np(G["dbg"]), b["dbg"], bl.sum(axis=0), 2e-2, "dbg")
