"""fp64 CPU oracle of one Mixture-of-Experts layer, forward and backward.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import this module.  It shares no code with the HIP library and imports
nothing from it: it is plain numpy in float64, one dense matmul per expert, written
from the definitions on the pages so that it can be checked by eye.

Sources (cited by page title and section):
  [HB]  "The Ultimate MoE Training Handbook" (Hugging Face), chapters 2-3.
  [LC]  LeCompute, "MoE training: cluster, routing, load balancing".

Notation: T tokens, d model width, E routed experts, k experts per token, F expert
FFN width, Fs shared-expert width; A = T*k routed rows.

Every function has a pin in tests/test_oracle_pins.py that checks it against
something other than itself (worked numbers printed on the pages, closed forms,
brute force, finite differences, an independent dense FFN).

Readings where the pages leave a step open (the same list is kept with the design notes):
  * top-k ties go to the lowest expert index; slots are ordered by key descending,
    then index ascending.
  * sigmoid selection keys sigma(l) + bias are evaluated in float64 from the fp32
    logits and fp32 bias.
  * the aux loss uses the full softmax over all E experts as the router probability,
    and counts carry no gradient.
  * the shared expert is ungated and added at weight 1.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np

f64 = np.float64


def _d(a):
    return None if a is None else np.asarray(a, dtype=f64)


# ----------------------------------------------------------------------------- router

def gate_logits(x, Wg, bg=None):
    """Router logits l = x W_g^T (+ b_g), in float64.

    [HB] §3.1 Router scoring, Precision: the router's linear layer runs in the router
    dtype (fp32 or fp64) on a [E, d] weight, optionally with an additive bias.
    """
    l = _d(x) @ _d(Wg).T
    if bg is not None:
        l = l + _d(bg)[None, :]
    return l


def sigmoid(z):
    z = _d(z)
    return 1.0 / (1.0 + np.exp(-z))


def selection_keys(logits, score: str, expert_bias=None):
    """The values top-k ranks.

    [HB] §3.1 Router scoring, Gating function: the softmax router (renormalised,
    the default) takes top-k on the raw logits and applies softmax to the k selected;
    the sigmoid router takes top-k on sigma(l), or on sigma(l) + expert_bias when the
    loss-free bias is on ([HB] §3.3 Load balancing, Loss-free bias: the bias changes
    only which experts are selected).
    """
    l = _d(logits)
    if score == "softmax":
        if expert_bias is not None:
            raise ValueError("the expert bias is only defined for sigmoid scores")
        return l
    if score == "sigmoid":
        s = sigmoid(l)
        return s if expert_bias is None else s + _d(expert_bias)[None, :]
    raise ValueError(score)


def topk(keys, k: int):
    """Indices of the k largest keys per row, key descending, ties to the lower index.

    [HB] §3.1 Router scoring, Precision: PyTorch leaves the order of tied experts
    unspecified; here the lower expert index wins.  Stable sort of -key realises that.
    """
    keys = _d(keys)
    order = np.argsort(-keys, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def margins(keys, k: int):
    """key_k - key_{k+1} per token (inf when k == E): how far a token is from a flip."""
    keys = _d(keys)
    if k >= keys.shape[1]:
        return np.full(keys.shape[0], np.inf)
    s = -np.sort(-keys, axis=1)
    return s[:, k - 1] - s[:, k]


def mixing_weights(logits, idx, score: str, scaling: float = 1.0):
    """Mixing weights of the selected experts, shape [T, k].

    [HB] §3.1 Router scoring, Gating function and Output scale:
      softmax: softmax over the k selected logits (equal to the full softmax
               renormalised over the top-k);
      sigmoid: sigma(l_S) / (sum sigma(l_S) + 1e-20) for k > 1, sigma(l_S) for k == 1;
      then the routed scaling factor multiplies the result.
    """
    l = _d(logits)
    lS = np.take_along_axis(l, idx, axis=1)
    k = idx.shape[1]
    if score == "softmax":
        z = np.exp(lS - lS.max(axis=1, keepdims=True))
        w = z / z.sum(axis=1, keepdims=True)
    elif score == "sigmoid":
        s = sigmoid(lS)
        w = s / (s.sum(axis=1, keepdims=True) + 1e-20) if k > 1 else s
    else:
        raise ValueError(score)
    return w * scaling


def softmax_full(logits):
    l = _d(logits)
    z = np.exp(l - l.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def expert_counts(idx, E: int):
    """Tokens per expert: how many (token, slot) pairs chose each expert."""
    return np.bincount(np.asarray(idx).ravel(), minlength=E).astype(np.int64)


def aux_loss(counts, probs, k: int, coeff: float):
    """Switch load-balancing loss at micro-batch scope.

    [HB] §3.3 Load balancing, Aux loss: coeff * E * sum_e f_e * P_e, with f_e the
    expert's share of the T*k assignments and P_e its mean router probability over the
    T tokens.  probs is [T, E] (the full softmax; see the readings above).
    """
    probs = _d(probs)
    T, E = probs.shape
    f = np.asarray(counts, dtype=f64) / (T * k)
    P = probs.mean(axis=0)
    return coeff * E * float(np.sum(f * P))


def max_violation(counts):
    """MaxVio = (busiest expert's load - mean load) / mean load.

    [HB] §3.2 Routing strategy, Who selects, and [LC] "Why add a load-balancing
    objective?" (the definition from the auxiliary-loss-free study).
    """
    c = np.asarray(counts, dtype=f64)
    m = c.mean()
    return float((c.max() - m) / m)


# ------------------------------------------------------------------------ permutation

@dataclass
class Permutation:
    offsets: np.ndarray   # [E+1]  first row of each expert's group
    row_of: np.ndarray    # [T, k] permuted row of (token, slot)
    token_of: np.ndarray  # [A]    token of each permuted row


def permutation(idx, E: int) -> Permutation:
    """Group the T*k (token, slot) copies by expert: expert ascending, token ascending.

    [LC] "Read the timeline before blaming the network": tokens are grouped by expert
    before the expert matmuls and put back in their original order afterwards
    (dropless: every copy is kept).  Each token picks an expert at most once, so
    sorting the copies by (expert, token) defines the order uniquely.
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    t = np.repeat(np.arange(T), k)
    j = np.tile(np.arange(k), T)
    e = idx.ravel()
    order = np.lexsort((t, e))          # primary key e, then t
    row_of = np.empty(T * k, dtype=np.int64)
    row_of[order] = np.arange(T * k)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(np.bincount(e, minlength=E))
    return Permutation(offsets=offsets, row_of=row_of.reshape(T, k), token_of=t[order])


# --------------------------------------------------------------------------- experts

def silu(g):
    g = _d(g)
    return g / (1.0 + np.exp(-g))


def swiglu_forward(X, W13, W2):
    """One bias-free SwiGLU expert on rows X.

    [HB] §3.4 Experts, Count and size (fc1 is twice the expert width for a gated
    linear unit; fc2 maps the width back to d) and Activation (the GLU splits fc1's
    output in two halves, gate first, and multiplies silu(gate) by the up half).
    Returns H = X W13^T [n, 2F], Act = silu(H_gate) * H_up [n, F], Y = Act W2^T [n, d].
    """
    H = _d(X) @ _d(W13).T
    F = H.shape[1] // 2
    Act = silu(H[:, :F]) * H[:, F:]
    Y = Act @ _d(W2).T
    return H, Act, Y


def swiglu_backward(X, W13, W2, H, dY):
    """Backward of swiglu_forward by the chain rule (derived, not printed on the pages).

    dAct = dY W2; with s = sigma(g): silu'(g) = s (1 + g (1 - s));
    dH_gate = dAct * up * silu'(g), dH_up = dAct * silu(g);
    dX = dH W13, dW13 = dH^T X, dW2 = dY^T Act.
    """
    X, W13, W2, H, dY = map(_d, (X, W13, W2, H, dY))
    F = H.shape[1] // 2
    g, u = H[:, :F], H[:, F:]
    s = sigmoid(g)
    act = g * s * u
    dAct = dY @ W2
    dH = np.concatenate([dAct * u * s * (1.0 + g * (1.0 - s)), dAct * g * s], axis=1)
    return dict(dX=dH @ W13, dW13=dH.T @ X, dW2=dY.T @ act, dH=dH, dAct=dAct)


# ------------------------------------------------------------------------ full layer

@dataclass
class LayerSpec:
    E: int
    k: int
    score: str = "softmax"
    scaling: float = 1.0
    aux_coeff: float = 0.0


def route(logits, spec: LayerSpec, expert_bias=None) -> Dict[str, np.ndarray]:
    """Router: keys -> top-k -> weights -> counts and load statistics."""
    keys = selection_keys(logits, spec.score, expert_bias)
    idx = topk(keys, spec.k)
    w = mixing_weights(logits, idx, spec.score, spec.scaling)
    counts = expert_counts(idx, spec.E)
    out = dict(keys=keys, idx=idx, w=w, counts=counts, margin=margins(keys, spec.k),
               maxvio=max_violation(counts))
    if spec.score == "softmax":
        p = softmax_full(logits)
        out["prob_sum"] = p.sum(axis=0)
        out["aux"] = aux_loss(counts, p, spec.k, spec.aux_coeff)
    else:
        out["prob_sum"] = None
        out["aux"] = 0.0
    return out


def layer_forward(x, Wg, W13, W2, spec: LayerSpec, bg=None, expert_bias=None,
                  W13s=None, W2s=None, idx=None) -> Dict[str, object]:
    """The whole layer forward.

    y_t = sum_j w_tj * Expert_{idx_tj}(x_t) + Shared(x_t)
    ([LC] "An expert transforms numbers inside the model": the weighted sum of the
    selected experts' outputs, coordinate by coordinate; [HB] §3.4 Shared experts:
    without a gate the shared output is added at weight 1).
    `idx` may be given to evaluate the layer at a fixed routing.  W13 and W2 only need
    per-expert indexing (W13[e] -> [2F, d]), so a lazily converted stack works.
    """
    x = _d(x)
    T, d = x.shape
    logits = gate_logits(x, Wg, bg)
    r = route(logits, spec, expert_bias)
    if idx is not None:
        r["idx"] = np.asarray(idx, dtype=np.int64)
        r["w"] = mixing_weights(logits, r["idx"], spec.score, spec.scaling)
        r["counts"] = expert_counts(r["idx"], spec.E)
    perm = permutation(r["idx"], spec.E)
    A = T * spec.k
    xp = x[perm.token_of]
    F2 = 2 * np.shape(W2[int(r["idx"].ravel()[0])])[1]
    H = np.zeros((A, F2))
    Act = np.zeros((A, F2 // 2))
    Yp = np.zeros((A, d))
    for e in range(spec.E):
        a, b = perm.offsets[e], perm.offsets[e + 1]
        if b > a:
            H[a:b], Act[a:b], Yp[a:b] = swiglu_forward(xp[a:b], W13[e], W2[e])
    y = np.einsum("tk,tkd->td", r["w"], Yp[perm.row_of])
    shared = None
    if W13s is not None:
        Hs, Acts, Ys = swiglu_forward(x, W13s, W2s)
        y = y + Ys
        shared = dict(H=Hs, Act=Acts, Y=Ys)
    return dict(logits=logits, route=r, perm=perm, x_perm=xp, H=H, Act=Act, Y_perm=Yp,
                shared=shared, y=y)


def router_backward(logits, idx, w, dw, spec: LayerSpec, counts=None, daux: float = 1.0):
    """d(loss)/d(logits) from the mixing-weight gradient dw [T, k] and the aux loss.

    Softmax over the selected set S with weights w = c * p (c the scaling factor):
      dl_S = w * dw - (w / c) * <w, dw>, zero off S.
    Sigmoid renormalised (k > 1), z = sum sigma(l_S) + 1e-20, w = c * s / z:
      ds = (c / z) * (dw - <dw, s> / z),  dl_S = ds * s * (1 - s).
    Aux: with g_e = coeff * E * f_e / T (counts held constant),
      dl_t += daux * p_t * (g - <g, p_t>), p_t the full softmax.
    """
    l = _d(logits)
    T, E = l.shape
    k = idx.shape[1]
    c = spec.scaling
    dw = _d(dw)
    w = _d(w)
    dl = np.zeros_like(l)
    if spec.score == "softmax":
        dlS = w * dw - (w / c) * np.sum(w * dw, axis=1, keepdims=True)
    else:
        s = sigmoid(np.take_along_axis(l, idx, axis=1))
        if k > 1:
            z = s.sum(axis=1, keepdims=True) + 1e-20
            ds = (c / z) * (dw - np.sum(dw * s, axis=1, keepdims=True) / z)
        else:
            ds = c * dw
        dlS = ds * s * (1.0 - s)
    np.put_along_axis(dl, idx, dlS, axis=1)
    if spec.score == "softmax" and spec.aux_coeff != 0.0 and daux != 0.0:
        p = softmax_full(l)
        f = np.asarray(counts, dtype=f64) / (T * k)
        g = spec.aux_coeff * E * f / T
        dl += daux * p * (g[None, :] - (p @ g)[:, None])
    return dl


def layer_backward(fwd: Dict[str, object], x, Wg, W13, W2, dy, spec: LayerSpec,
                   W13s=None, W2s=None, daux: float = 1.0, sparse_expert_grads: bool = False
                   ) -> Dict[str, np.ndarray]:
    """Gradients of L = sum(dy * y) + daux * aux with respect to every input.

    With sparse_expert_grads the expert weight gradients come back as {e: array} for the
    experts that received rows (the others are zero), instead of full [E, ...] stacks.

    The expert path gets its gradient through the weighted sum ([LC] "How the router
    learns without an expert-selection answer key": the signal reaches the router only
    through the mixing weights of the selected outputs; selection itself has none).
    """
    x, dy = _d(x), _d(dy)
    T, d = x.shape
    r, perm = fwd["route"], fwd["perm"]
    idx, w = r["idx"], r["w"]
    Yp = fwd["Y_perm"]
    # combine backward
    rows = perm.row_of
    dw = np.einsum("td,tkd->tk", dy, Yp[rows])
    dYp = np.zeros_like(Yp)
    dYp[rows.ravel()] = (w[:, :, None] * dy[:, None, :]).reshape(-1, d)
    xp = fwd["x_perm"]
    dXp = np.zeros_like(xp)
    if sparse_expert_grads:
        dW13, dW2 = {}, {}
    else:
        dW13 = np.zeros((spec.E,) + np.shape(W13[0]))
        dW2 = np.zeros((spec.E,) + np.shape(W2[0]))
    dH = np.zeros_like(fwd["H"])
    for e in range(spec.E):
        a, b = perm.offsets[e], perm.offsets[e + 1]
        if b > a:
            g = swiglu_backward(xp[a:b], W13[e], W2[e], fwd["H"][a:b], dYp[a:b])
            dXp[a:b], dW13[e], dW2[e], dH[a:b] = g["dX"], g["dW13"], g["dW2"], g["dH"]
    dx = dXp[rows].sum(axis=1)
    out = dict(dw=dw, dY_perm=dYp, dX_perm=dXp, dH=dH, dW13=dW13, dW2=dW2)
    if W13s is not None:
        gs = swiglu_backward(x, W13s, W2s, fwd["shared"]["H"], dy)
        dx = dx + gs["dX"]
        out.update(dW13s=gs["dW13"], dW2s=gs["dW2"], dH_s=gs["dH"])
    dlogits = router_backward(fwd["logits"], idx, w, dw, spec, counts=r["counts"], daux=daux)
    out["dlogits"] = dlogits
    out["dWg"] = dlogits.T @ x
    out["dbg"] = dlogits.sum(axis=0)
    out["dx_router"] = dlogits @ _d(Wg)
    out["dx"] = dx + out["dx_router"]
    return out


def layer_loss(x, Wg, W13, W2, dy, spec: LayerSpec, bg=None, expert_bias=None,
               W13s=None, W2s=None, daux: float = 1.0) -> float:
    """L = sum(dy * y) + daux * aux, the scalar whose gradient layer_backward returns."""
    f = layer_forward(x, Wg, W13, W2, spec, bg=bg, expert_bias=expert_bias, W13s=W13s, W2s=W2s)
    return float(np.sum(_d(dy) * f["y"]) + daux * f["route"]["aux"])


def expert_param_count(d: int, F: int) -> int:
    """Parameters of one bias-free SwiGLU expert: fc1 [2F, d] plus fc2 [d, F]."""
    return 2 * F * d + d * F


def permuted_buffer_bytes(T: int, k: int, d: int, elem_bytes: int) -> int:
    """Bytes of the grouped copy of the input: one row of d values per (token, slot)."""
    return T * k * d * elem_bytes


def brute_force_topk(keys_row, k: int):
    """All C(E, k) subsets: the one with the largest exact key sum, lowest indices on ties,
    listed by key descending then index ascending.  Pure Python, tiny E only."""
    from fractions import Fraction
    from itertools import combinations
    E = len(keys_row)
    kv = [Fraction(float(v)) for v in keys_row]
    best, best_sum = None, None
    for S in combinations(range(E), k):
        s = sum(kv[i] for i in S)
        if best_sum is None or s > best_sum or (s == best_sum and S < best):
            best, best_sum = S, s
    return sorted(best, key=lambda i: (-kv[i], i))


def num_choices(n: int, r: int) -> int:
    return math.comb(n, r)
