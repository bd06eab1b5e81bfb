"""The allocation-free router call (moe_router_topk_noalloc) against moe_router_topk.

Both run the same kernels; the allocation-free call takes its scratch from the library's
static device array instead of a workspace.  Two calls in a row, the second on a smaller
input (whose scratch layout differs and which must not see the first call's partials),
each compared bit for bit with the workspace call on the same logits: indices, weights,
counts, probability sums and every statistic.
"""
from dataclasses import replace

import numpy as np
import pytest

from helpers import O, W, dev, f64, spec_of, to_dev, to_np, torch_mod

pytestmark = pytest.mark.gpu


def _outputs(L, cfg, logits, bias, noalloc, ws=None):
    torch = torch_mod()
    T, E, k = cfg.T, cfg.E, cfg.k
    out = dict(idx=torch.full((T, k), -1, dtype=torch.int32, device=dev()),
               w=torch.full((T, k), float("nan"), dtype=torch.float32, device=dev()),
               counts=torch.full((E,), -1, dtype=torch.int32, device=dev()),
               prob_sum=torch.full((E,), float("nan"), dtype=torch.float32, device=dev()),
               stats=torch.full((L.MOE_NSTATS,), float("nan"), dtype=torch.float32, device=dev()))
    B = L.num_sequences(cfg)
    if B:
        out["seq_counts"] = torch.full((B, E), -1, dtype=torch.int32, device=dev())
    args = (cfg, logits, bias, out["idx"], out["w"], out["counts"], out["prob_sum"], out["stats"])
    if noalloc:
        L.router_topk_noalloc(*args, seq_counts=out.get("seq_counts"))
    else:
        L.router_topk(*args, ws, seq_counts=out.get("seq_counts"))
    return out


def test_router_topk_noalloc_matches_the_workspace_call():
    torch = torch_mod()
    from mixture_experts_layer_aux_amd import _lib as L
    big = W.LAYERS[3]                                    # 16384 tokens, 256 experts, sigmoid + selection bias
    small = replace(W.SMALL[2], T=1000, aux_coeff=0.01, z_coeff=1e-3, seq_aux_coeff=1e-4, seq_len=250)
    for shape, seed in ((big, 3), (small, 2)):
        print(f"noalloc router: {shape.name} T={shape.T} E={shape.E} k={shape.k}", flush=True)
        inp = W.make_inputs(shape, seed=seed, with_dy=False, with_experts=False)
        logits = to_dev(O.gate_logits(f64(inp["x"], shape.act), inp["Wg"], inp["bg"]).astype(np.float32))
        bias = to_dev(inp["expert_bias"])
        cfg = L.config_from_shape(shape)
        ws = L.alloc_workspace(cfg, dev())
        want = _outputs(L, cfg, logits, bias, noalloc=False, ws=ws)
        got = _outputs(L, cfg, logits, bias, noalloc=True)
        torch.cuda.synchronize()
        for n in want:
            assert torch.equal(got[n], want[n]), f"{shape.name}: {n} differs from moe_router_topk"
        # and the routing is the oracle's (up to near-ties, as for the workspace call)
        r = O.route(to_np(logits), spec_of(shape), None if inp["expert_bias"] is None
                    else inp["expert_bias"].astype(np.float64))
        assert np.array_equal(to_np(got["idx"]), r["idx"])
        assert np.array_equal(to_np(got["counts"]), r["counts"])
