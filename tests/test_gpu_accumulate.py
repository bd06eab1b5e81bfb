"""Gradient accumulation into the caller's buffers (moe_grads_t.accumulate and the
accumulate argument of moe_grouped_wgrad).

Accumulating adds the gradient of one call to what the buffer holds, for summing the
gradients of several micro-batches.  The fp32 sum of one call is formed exactly as when
overwriting, so the result is fixed bit for bit by the overwriting call, whose parity with
the fp64 oracle the layer and piece tests establish:
  * an fp32 gradient becomes fp32(old + G), G the overwriting call's output;
  * a bf16 gradient becomes bf16_rne(old + G32), G32 the fp32-output weight gradient
    (the same accumulator, which the bf16 output rounds once);
  * an expert without rows keeps its old gradient.
The input gradient dx is overwritten as always.  The first call of each test is also held
to the oracle here.
"""
from dataclasses import replace

import numpy as np
import pytest

from helpers import O, W, check_layer_grads, dev, oracle_inputs, spec_of, to_dev, to_np, torch_mod

pytestmark = pytest.mark.gpu

_WEIGHT_GRADS = ("dW13", "dW2", "dW13s", "dW2s")


def _prior(G, seed):
    """Random values of each gradient's dtype to accumulate onto."""
    torch = torch_mod()
    gen = torch.Generator(device="cpu").manual_seed(seed)
    return {k: (torch.randn(v.shape, generator=gen) * 1e-2).to(v.dtype).to(v.device) for k, v in G.items()}


def _expected(prior, G32):
    """fp32(old + G32), rounded once to the prior's dtype."""
    return (prior.float() + G32).to(prior.dtype)


_LAYER_CASES = {
    # bf16 experts with bf16 weight gradients, ~5% empty experts, gate bias, shared expert behind its gate
    "skewed-bf16-shared-gate": (replace(W.SMALL[5], Fs=128, shared_gate=True), {}),
    # bf16 experts with fp32 weight gradients, router GEMMs on the matrix cores
    "small-bf16-wgrad-f32": (W.SMALL[2], {"wgrad": "f32"}),
    # fp32 activations: every GEMM on the FMA path
    "tiny-fp32": (W.LAYERS[1], {}),
}


@pytest.mark.parametrize("name", list(_LAYER_CASES))
def test_layer_bwd_accumulate(name):
    torch = torch_mod()
    from mixture_experts_layer_aux_amd import _lib as L
    shape, extra = _LAYER_CASES[name]
    print(f"layer accumulate {name}", flush=True)
    inp = W.make_inputs(shape, seed=11)
    cfg = L.config_from_shape(shape, **extra)
    cfg32 = L.config_from_shape(shape, **{**extra, "wgrad": "f32"})   # same layer, fp32 weight gradients
    d = dev()
    Wt = dict(Wg=to_dev(inp["Wg"]), bg=to_dev(inp["bg"]), expert_bias=to_dev(inp["expert_bias"]),
              W13=to_dev(inp["W13"]), W2=to_dev(inp["W2"]), W13s=to_dev(inp["W13s"]), W2s=to_dev(inp["W2s"]),
              Wsg=to_dev(inp.get("Wsg")))
    x = to_dev(inp["x"])
    dy = to_dev(W.to_f32(inp["dy"], shape.act).copy())
    S = L.alloc_saved(cfg, d)
    ws = L.alloc_workspace(cfg, d)
    y = torch.empty(shape.T, shape.d, dtype=torch.float32, device=d)
    stats = torch.empty(L.MOE_NSTATS, dtype=torch.float32, device=d)
    L.layer_fwd(cfg, Wt, x, S, y, stats, ws)
    with_dbg = inp["bg"] is not None
    # the overwriting backward, with fp32 weight gradients
    G32 = L.alloc_grads(cfg32, d, with_dbg=with_dbg)
    dx0 = torch.empty(shape.T, shape.d, dtype=torch.float32, device=d)
    L.layer_bwd(cfg32, Wt, S, x, dy, 1.0, dx0, G32, ws)
    # accumulate twice onto a prior, in the layer's own weight-gradient dtype
    G = L.alloc_grads(cfg, d, with_dbg=with_dbg)
    prior = _prior(G, seed=5)
    for k in G:
        G[k].copy_(prior[k])
    dx = torch.full((shape.T, shape.d), float("nan"), dtype=torch.float32, device=d)
    L.layer_bwd(cfg, Wt, S, x, dy, 1.0, dx, G, ws, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(dx, dx0), "dx is overwritten whatever the flag"
    once = {k: v.clone() for k, v in G.items()}
    L.layer_bwd(cfg, Wt, S, x, dy, 1.0, dx, G, ws, accumulate=True)
    torch.cuda.synchronize()
    counts = to_np(S["counts"])
    if name.startswith("skewed"):
        assert (counts == 0).any(), "the skewed layer should leave some experts empty"
    assert set(G) >= {"dWg", "dW13", "dW2"}
    for k in G:
        want1 = _expected(prior[k], G32[k])
        assert torch.equal(once[k], want1), f"{k}: first accumulation"
        assert torch.equal(G[k], _expected(once[k], G32[k])), f"{k}: second accumulation"
    for k in ("dW13", "dW2"):
        for e in np.where(counts == 0)[0]:
            assert torch.equal(G[k][e], prior[k][e]), f"{k}[{e}]: an expert without rows keeps its gradient"
    # the overwriting call against the oracle
    o = oracle_inputs(inp, shape)
    spec = spec_of(shape)
    f = O.layer_forward(o["x"], o["Wg"], o["W13"], o["W2"], spec, bg=o["bg"], expert_bias=o["expert_bias"],
                        W13s=o["W13s"], W2s=o["W2s"], Wsg=o["Wsg"])
    if np.array_equal(f["route"]["idx"], to_np(S["idx"])):
        b = O.layer_backward(f, o["x"], o["Wg"], o["W13"], o["W2"], o["dy"], spec, W13s=o["W13s"], W2s=o["W2s"],
                             daux=1.0, Wsg=o["Wsg"])
        check_layer_grads({k: to_np(v) for k, v in G32.items()}, f, b, o, spec, shape)
    else:
        print("routing differs from the oracle's at a near-tie: oracle check left to the layer tests", flush=True)


@pytest.mark.parametrize("wgrad,K", [("bf16", 320), ("f32", 320), ("bf16", 1024), ("f32", 1024)])
def test_grouped_wgrad_accumulate(wgrad, K):
    """The grouped weight gradient on ragged groups, some empty, three calls on one buffer:
    overwrite, then accumulate twice.  K = 1024 columns take the two-workgroup kernel
    (narrower gradients the 8-wave GEMM); there the same calls with X read through a row
    gather (x_rows) must give the same bits."""
    torch = torch_mod()
    from mixture_experts_layer_aux_amd import _lib as L
    print(f"grouped wgrad accumulate {wgrad} K={K}", flush=True)
    shape = W.SMALL[2]
    cfg = L.config_from_shape(shape, wgrad=wgrad)
    cfg32 = L.config_from_shape(shape, wgrad="f32")
    rng = np.random.default_rng(7)
    sizes = np.array([300, 0, 257, 1, 0, 64, 511, 0], dtype=np.int64)
    G, N = len(sizes), 192
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    rows = int(off[-1])
    dY = rng.standard_normal((rows, N)).astype(np.float32)
    X = rng.standard_normal((rows, K)).astype(np.float32)
    bits = lambda a: torch.from_numpy(W.f32_to_bf16_bits(a).view(np.int16)).view(torch.bfloat16)  # noqa: E731
    dY_d, X_d = bits(dY).to(dev()), bits(X).to(dev())
    off_d = torch.from_numpy(off).to(dev())
    wd = L.wgrad_dtype(cfg)
    ref32 = torch.empty(G, N, K, dtype=torch.float32, device=dev())
    L.grouped_wgrad(cfg32, off_d, G, rows, dY_d, N, X_d, K, ref32)
    dW = torch.full((G, N, K), 7.0, dtype=wd, device=dev())
    L.grouped_wgrad(cfg, off_d, G, rows, dY_d, N, X_d, K, dW)
    torch.cuda.synchronize()
    assert torch.equal(dW, ref32.to(wd)), "overwrite"
    prior = _prior({"dW": dW}, seed=9)["dW"]
    dW.copy_(prior)
    L.grouped_wgrad(cfg, off_d, G, rows, dY_d, N, X_d, K, dW, accumulate=True)
    torch.cuda.synchronize()
    once = dW.clone()
    L.grouped_wgrad(cfg, off_d, G, rows, dY_d, N, X_d, K, dW, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(once, _expected(prior, ref32)), "first accumulation"
    assert torch.equal(dW, _expected(once, ref32)), "second accumulation"
    for g in np.where(sizes == 0)[0]:
        assert torch.equal(dW[g], prior[g]), f"group {g} without rows keeps its gradient"
    if K >= 1024:
        # X's rows scattered over a larger source, read back through x_rows
        src_rows = rows + 37
        perm = rng.permutation(src_rows)[:rows].astype(np.int32)
        Xsrc = torch.zeros(src_rows, K, dtype=X_d.dtype, device=dev())
        Xsrc[torch.from_numpy(perm).long().to(dev())] = X_d
        x_rows = torch.from_numpy(perm).to(dev())
        gW = torch.full((G, N, K), 7.0, dtype=wd, device=dev())
        L.grouped_wgrad(cfg, off_d, G, rows, dY_d, N, Xsrc, K, gW, x_rows=x_rows)
        torch.cuda.synchronize()
        assert torch.equal(gW, ref32.to(wd)), "overwrite through x_rows"
        gW.copy_(prior)
        L.grouped_wgrad(cfg, off_d, G, rows, dY_d, N, Xsrc, K, gW, x_rows=x_rows, accumulate=True)
        torch.cuda.synchronize()
        assert torch.equal(gW, once), "accumulation through x_rows"
    # the fp32 sums against fp64 dY_g^T X_g of the bf16 operands
    dY64 = W.bf16_bits_to_f32(W.f32_to_bf16_bits(dY)).astype(np.float64)
    X64 = W.bf16_bits_to_f32(W.f32_to_bf16_bits(X)).astype(np.float64)
    got = to_np(ref32)
    for g in range(G):
        ref = dY64[off[g]:off[g + 1]].T @ X64[off[g]:off[g + 1]]
        err = np.abs(got[g] - ref).max() / max(1.0, np.sqrt(max(sizes[g], 1)))
        assert err < 1e-4, f"group {g}: {err:.2e}"


def test_grouped_wgrad_split_k():
    """A one-group weight gradient with too few output tiles is split over its rows when a
    workspace is given: 1000 rows in three chunks of 384, 384 and 232.  The split sum is
    held to fp64, and to the unsplit call within fp32 rounding.  The bf16 output is the
    split fp32 sum rounded once, and accumulating adds to it in fp32 first, bit for bit.
    A workspace smaller than the partials is refused."""
    torch = torch_mod()
    from mixture_experts_layer_aux_amd import _lib as L
    print("grouped wgrad split-K", flush=True)
    shape = W.SMALL[2]
    c16, c32 = L.config_from_shape(shape, wgrad="bf16"), L.config_from_shape(shape, wgrad="f32")
    rng = np.random.default_rng(21)
    rows, N, K = 1000, 192, 320
    dY = rng.standard_normal((rows, N)).astype(np.float32)
    X = rng.standard_normal((rows, K)).astype(np.float32)
    bits = lambda a: torch.from_numpy(W.f32_to_bf16_bits(a).view(np.int16)).view(torch.bfloat16)  # noqa: E731
    dY_d, X_d = bits(dY).to(dev()), bits(X).to(dev())
    ws = torch.empty(3 * N * K * 4, dtype=torch.uint8, device=dev())
    whole = torch.empty(N, K, dtype=torch.float32, device=dev())
    L.grouped_wgrad(c32, None, 1, rows, dY_d, N, X_d, K, whole)
    split32 = torch.empty(N, K, dtype=torch.float32, device=dev())
    L.grouped_wgrad(c32, None, 1, rows, dY_d, N, X_d, K, split32, ws=ws)
    split16 = torch.empty(N, K, dtype=torch.bfloat16, device=dev())
    L.grouped_wgrad(c16, None, 1, rows, dY_d, N, X_d, K, split16, ws=ws)
    prior = _prior({"dW": split16}, seed=4)["dW"]
    acc16 = prior.clone()
    L.grouped_wgrad(c16, None, 1, rows, dY_d, N, X_d, K, acc16, ws=ws, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(split16, split32.to(torch.bfloat16)), "bf16 split output is the fp32 split sum rounded once"
    assert torch.equal(acc16, _expected(prior, split32)), "split accumulation"
    ref = (W.bf16_bits_to_f32(W.f32_to_bf16_bits(dY)).astype(np.float64).T
           @ W.bf16_bits_to_f32(W.f32_to_bf16_bits(X)).astype(np.float64))
    for got in (split32, whole):
        err = np.abs(to_np(got) - ref).max() / np.sqrt(rows)
        assert err < 1e-4, f"against fp64: {err:.2e}"
    small = torch.empty(3 * N * K * 4 - 16, dtype=torch.uint8, device=dev())
    with pytest.raises(L.MoeError, match="workspace"):
        L.grouped_wgrad(c32, None, 1, rows, dY_d, N, X_d, K, split32, ws=small)


@pytest.mark.parametrize("K", [320, 1024])
def test_grouped_wgrad_skew_split(K):
    """Groups with more rows than the skew plan's chunk (1024 rows here) are cut into row
    chunks when ws is given: 3000 rows in three chunks, 1025 and 2049 with a one-row last
    chunk, 1024 left whole.  The unsplit groups give the bits of the call without ws, the
    split ones the fp64 sum within fp32 rounding; the bf16 output is the fp32 split sum
    rounded once, accumulation adds to it in fp32 first, groups without rows keep their
    gradient, the row gather of X (K = 1024) gives the same bits, and a workspace too small
    for the plan gives the unsplit call's bits."""
    torch = torch_mod()
    from mixture_experts_layer_aux_amd import _lib as L
    print(f"grouped wgrad skew split K={K}", flush=True)
    shape = replace(W.SMALL[2], T=8192)   # groups of up to T rows: the split is enabled
    c16, c32 = L.config_from_shape(shape, wgrad="bf16"), L.config_from_shape(shape, wgrad="f32")
    rng = np.random.default_rng(33)
    sizes = np.array([3000, 0, 37, 1025, 1024, 0, 1, 2049, 512], dtype=np.int64)
    G, N = len(sizes), 192
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    rows = int(off[-1])
    dY = rng.standard_normal((rows, N)).astype(np.float32)
    X = rng.standard_normal((rows, K)).astype(np.float32)
    bits = lambda a: torch.from_numpy(W.f32_to_bf16_bits(a).view(np.int16)).view(torch.bfloat16)  # noqa: E731
    dY_d, X_d = bits(dY).to(dev()), bits(X).to(dev())
    off_d = torch.from_numpy(off).to(dev())
    ws = torch.empty(20 * N * K * 4 + (1 << 16), dtype=torch.uint8, device=dev())
    e32 = lambda: torch.full((G, N, K), 7.0, dtype=torch.float32, device=dev())  # noqa: E731
    e16 = lambda: torch.full((G, N, K), 7.0, dtype=torch.bfloat16, device=dev())  # noqa: E731
    whole, split32, split16 = e32(), e32(), e16()
    L.grouped_wgrad(c32, off_d, G, rows, dY_d, N, X_d, K, whole)
    L.grouped_wgrad(c32, off_d, G, rows, dY_d, N, X_d, K, split32, ws=ws)
    L.grouped_wgrad(c16, off_d, G, rows, dY_d, N, X_d, K, split16, ws=ws)
    prior16 = _prior({"dW": split16}, seed=5)["dW"]
    prior32 = _prior({"dW": split32}, seed=6)["dW"]
    acc16, acc32 = prior16.clone(), prior32.clone()
    L.grouped_wgrad(c16, off_d, G, rows, dY_d, N, X_d, K, acc16, ws=ws, accumulate=True)
    L.grouped_wgrad(c32, off_d, G, rows, dY_d, N, X_d, K, acc32, ws=ws, accumulate=True)
    tiny = torch.empty(4096, dtype=torch.uint8, device=dev())
    small32 = e32()
    L.grouped_wgrad(c32, off_d, G, rows, dY_d, N, X_d, K, small32, ws=tiny)
    torch.cuda.synchronize()
    assert torch.equal(small32, whole), "a workspace too small for the plan: no split"
    assert torch.equal(split16, split32.to(torch.bfloat16)), "bf16 split output is the fp32 split sum rounded once"
    assert torch.equal(acc16, _expected(prior16, split32)), "bf16 split accumulation"
    assert torch.equal(acc32, _expected(prior32, split32)), "fp32 split accumulation"
    for g in np.where(sizes == 0)[0]:
        assert torch.equal(acc16[g], prior16[g]) and torch.equal(acc32[g], prior32[g]), f"empty group {g}"
    for g in np.where(sizes <= 1024)[0]:
        assert torch.equal(split32[g], whole[g]), f"group {g} ({sizes[g]} rows) is not split"
    dY64 = W.bf16_bits_to_f32(W.f32_to_bf16_bits(dY)).astype(np.float64)
    X64 = W.bf16_bits_to_f32(W.f32_to_bf16_bits(X)).astype(np.float64)
    got_s, got_w = to_np(split32), to_np(whole)
    for g in range(G):
        ref = dY64[off[g]:off[g + 1]].T @ X64[off[g]:off[g + 1]]
        for name, got in (("split", got_s), ("whole", got_w)):
            err = np.abs(got[g] - ref).max() / max(1.0, np.sqrt(max(sizes[g], 1)))
            assert err < 1e-4, f"{name} group {g}: {err:.2e}"
    assert not torch.equal(split32[0], whole[0]), "the 3000-row group was not split"
    if K >= 1024:
        src_rows = rows + 37
        perm = rng.permutation(src_rows)[:rows].astype(np.int32)
        Xsrc = torch.zeros(src_rows, K, dtype=X_d.dtype, device=dev())
        Xsrc[torch.from_numpy(perm).long().to(dev())] = X_d
        x_rows = torch.from_numpy(perm).to(dev())
        g16 = e16()
        L.grouped_wgrad(c16, off_d, G, rows, dY_d, N, Xsrc, K, g16, ws=ws, x_rows=x_rows)
        torch.cuda.synchronize()
        assert torch.equal(g16, split16), "split through x_rows"
