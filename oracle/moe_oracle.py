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
  * the aux loss uses the full softmax over all E experts as the router probability
    (sigmoid and sqrt(softplus): the scores normalised over all E), and counts carry
    no gradient; the sequence-wise loss reads tokens in [S, B] order.
  * pre-softmax top-k ranks the logits (the same order as the probabilities).
  * the shared expert is ungated and added at weight 1.
  * fp8 experts: OCP e4m3 codes with one fp32 scale (amax / 448) per 128 x 128 weight
    block and per token per 128 activation columns; quotient and rounding in fp32.
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


def softplus(z):
    """log(1 + e^z), evaluated as max(z, 0) + log(1 + e^-|z|) so that it never overflows."""
    z = _d(z)
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def score_values(logits, score: str):
    """Per-expert scores of the two elementwise gating functions.

    [HB] §3.1 Router scoring, Gating function: sigmoid s = 1 / (1 + e^-l), or the
    square root of softplus, s = sqrt(log(1 + e^l)).  Both are increasing in l.
    """
    if score == "sigmoid":
        return sigmoid(logits)
    if score == "sqrtsoftplus":
        return np.sqrt(softplus(logits))
    raise ValueError(score)


def score_derivative(logits, score: str):
    """ds/dl of score_values: s (1 - s) for sigmoid; sigma(l) / (2 sqrt(softplus(l))) for
    sqrt(softplus) (softplus' = sigma).  Derived by the chain rule."""
    l = _d(logits)
    if score == "sigmoid":
        s = sigmoid(l)
        return s * (1.0 - s)
    if score == "sqrtsoftplus":
        return sigmoid(l) / (2.0 * np.sqrt(softplus(l)))
    raise ValueError(score)


def selection_keys(logits, score: str, expert_bias=None):
    """The values top-k ranks.

    [HB] §3.1 Router scoring, Gating function: the softmax router (renormalised,
    the default) takes top-k on the raw logits and applies softmax to the k selected;
    the sigmoid and sqrt(softplus) routers take top-k on their scores s(l), or on
    s(l) + expert_bias when the loss-free bias is on ([HB] §3.3 Load balancing,
    Loss-free bias: the bias changes only which experts are selected; the bias is
    refused with softmax).  Pre-softmax top-k ranks the full softmax, which is
    increasing in the logit, so it ranks the logits too (the logits are used, so that
    two logits fp32 would round to one probability still rank apart).
    """
    l = _d(logits)
    if score == "softmax":
        if expert_bias is not None:
            raise ValueError("the expert bias is only defined for sigmoid and sqrt(softplus) scores")
        return l
    s = score_values(l, score)
    return s if expert_bias is None else s + _d(expert_bias)[None, :]


def topk(keys, k: int):
    """Indices of the k largest keys per row, key descending, ties to the lower index.

    [HB] §3.1 Router scoring, Precision: PyTorch leaves the order of tied experts
    unspecified; here the lower expert index wins.  Stable sort of -key realises that.
    """
    keys = _d(keys)
    order = np.argsort(-keys, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def group_scores(keys, num_groups: int, m: int):
    """Per token and group of E / num_groups consecutive experts: the sum of the group's m
    largest keys, added from the largest down (one rounding order on both sides)."""
    keys = _d(keys)
    T, E = keys.shape
    g = -np.sort(-keys.reshape(T, num_groups, E // num_groups), axis=2)
    out = np.zeros((T, num_groups))
    for j in range(m):
        out = out + g[:, :, j]
    return out


def group_limited_topk(keys, k: int, num_groups: int, group_topk: int):
    """Group-limited top-k ([HB] §3.1 Gating function: group-limited routing picks groups by
    summing their best scores).  The experts form num_groups groups of consecutive indices;
    a group's score is the sum of its best k / group_topk keys (the reading taken: enough
    picks per kept group to fill k); the group_topk best groups are kept (ties to the lower
    group index); top-k runs over the experts of the kept groups.
    Returns (idx [T, k], the kept groups [T, group_topk], the group-score margin [T])."""
    keys = _d(keys)
    T, E = keys.shape
    n = E // num_groups
    gs = group_scores(keys, num_groups, k // group_topk)
    order = np.argsort(-gs, axis=1, kind="stable")
    kept = order[:, :group_topk]
    gsorted = np.take_along_axis(gs, order, axis=1)
    gmargin = (gsorted[:, group_topk - 1] - gsorted[:, group_topk] if group_topk < num_groups
               else np.full(T, np.inf))
    allowed = np.zeros((T, num_groups), dtype=bool)
    np.put_along_axis(allowed, kept, True, axis=1)
    masked = np.where(np.repeat(allowed, n, axis=1), keys, -np.inf)
    return topk(masked, k), kept, gmargin


def margins(keys, k: int):
    """key_k - key_{k+1} per token (inf when k == E): how far a token is from a flip."""
    keys = _d(keys)
    if k >= keys.shape[1]:
        return np.full(keys.shape[0], np.inf)
    s = -np.sort(-keys, axis=1)
    return s[:, k - 1] - s[:, k]


def mixing_weights(logits, idx, score: str, scaling: float = 1.0, pre_softmax: bool = False):
    """Mixing weights of the selected experts, shape [T, k].

    [HB] §3.1 Router scoring, Gating function and Output scale:
      softmax: softmax over the k selected logits (equal to the full softmax
               renormalised over the top-k);
      softmax with pre-softmax: the full softmax over all E, read at the selected
               experts, not renormalised (the flag turns renormalisation off);
      sigmoid / sqrt(softplus): s(l_S) / (sum s(l_S) + 1e-20) for k > 1, s(l_S) for k == 1;
      then the routed scaling factor multiplies the result.
    """
    l = _d(logits)
    lS = np.take_along_axis(l, idx, axis=1)
    k = idx.shape[1]
    if score == "softmax" and pre_softmax:
        w = np.take_along_axis(softmax_full(l), idx, axis=1)
    elif score == "softmax":
        z = np.exp(lS - lS.max(axis=1, keepdims=True))
        w = z / z.sum(axis=1, keepdims=True)
    elif score in ("sigmoid", "sqrtsoftplus"):
        s = score_values(lS, score)
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


def aux_probs(logits, score: str):
    """The router probabilities the balancing losses average, [T, E].

    softmax: the full softmax over all E experts.  sigmoid / sqrt(softplus): the scores
    normalised over all E experts, s / (sum_e s + 1e-20), so that each row sums to 1 and
    P_e is a mean probability as the aux loss of [HB] §3.3 asks (the pages name "mean
    router probability" but do not print how the scores for the loss are formed; this is
    the reading taken).
    """
    if score == "softmax":
        return softmax_full(logits)
    s = score_values(logits, score)
    return s / (s.sum(axis=1, keepdims=True) + 1e-20)


def logsumexp_rows(logits):
    """lse_t = log sum_e exp(l_te), with the row maximum taken out first."""
    l = _d(logits)
    m = l.max(axis=1)
    return m + np.log(np.exp(l - m[:, None]).sum(axis=1))


def z_loss(logits, coeff: float):
    """Router z-loss: coeff * mean over tokens of (logsumexp of the token's logits)^2.

    [HB] §3.1 Router scoring, Precision: a penalty on the logits' logsumexp, squared and
    averaged over the tokens, times the coefficient (ST-MoE's 1e-3 is the value named).
    """
    return coeff * float(np.mean(logsumexp_rows(logits) ** 2))


def sequence_of_token(T: int, seq_len: int):
    """Sequence index of every token.  Tokens are ordered [S, B] (position-major, the
    layout the printed sequence-wise loss reshapes from [S*B, E] to [S, B*E]): token
    t = s * B + b is position s of sequence b, B = T / S."""
    if seq_len < 1 or T % seq_len:
        raise ValueError("seq_len must divide T")
    B = T // seq_len
    return np.arange(T) % B


def sequence_counts(idx, E: int, seq_len: int):
    """counts[b, e]: how many (token, slot) pairs of sequence b chose expert e."""
    idx = np.asarray(idx)
    T, k = idx.shape
    B = T // seq_len
    seq = sequence_of_token(T, seq_len)
    out = np.zeros((B, E), dtype=np.int64)
    np.add.at(out, (np.repeat(seq, k), idx.ravel()), 1)
    return out


def seq_aux_loss(idx, probs, k: int, seq_len: int, coeff: float):
    """Sequence-wise balance loss: the micro-batch aux loss applied to each sequence on
    its own, then averaged over the B sequences.

    [HB] §3.3 Load balancing, Scope: seq_aux_loss balances per sequence (DeepSeek-V3 keeps
    one at a coefficient of 1e-4 beside the loss-free bias).  For sequence b with S
    tokens: coeff * E * sum_e f_be P_be, f_be = counts[b, e] / (k S), P_be the mean of
    its tokens' probabilities for e; the result is the mean over b.
    """
    probs = _d(probs)
    T, E = probs.shape
    B = T // seq_len
    seq = sequence_of_token(T, seq_len)
    cnt = sequence_counts(idx, E, seq_len)
    total = 0.0
    for b in range(B):
        f = cnt[b] / (k * seq_len)
        P = probs[seq == b].mean(axis=0)
        total += coeff * E * float(np.sum(f * P))
    return total / B


def expert_bias_update(expert_bias, counts, rate: float, centered: bool = False):
    """One step of the loss-free balancing bias, in fp32 (the bias is kept in fp32).

    [HB] §3.3 Load balancing, Loss-free bias: every step each expert's bias moves by the
    fixed update rate, up when the expert got fewer than the mean load and down when it
    got more; the comparison with the mean is made on integers, count * E against the
    total count, so it is exact: direction = sign(total - count * E).  The centered
    variant subtracts the mean of the steps (Moonlight, Trinity Mini), so the mean bias
    does not drift.  Each fp32 operation below is one rounding, in this order:
      step_e = direction_e * rate                       (exact: direction is -1, 0 or 1)
      centered: m = (rate * sum_e direction_e) / E,  step_e = step_e - m
      bias_e = bias_e + step_e
    """
    c = np.asarray(counts, dtype=np.int64)
    E = c.shape[0]
    total = int(c.sum())
    direction = np.sign(total - c * E).astype(np.int64)
    b = np.asarray(expert_bias, dtype=np.float32)
    r = np.float32(rate)
    step = direction.astype(np.float32) * r
    if centered:
        m = np.float32(np.float32(r * np.float32(direction.sum())) / np.float32(E))
        step = (step - m).astype(np.float32)
    return (b + step).astype(np.float32)


def quantile_route(scores, beta, k: int, update: bool = True):
    """Quantile balancing, one micro-batch ([HB] §3.3 Load balancing, Quantile).

    The bias is solved for instead of stepped: each expert ranks the tokens by their score
    for it and reads off the score that only its target share of tokens beats.  With the
    router in fp32 (the precision the pages ask for), every value below is one fp32
    rounding, so the selections are exactly reproducible:
      keys = scores - beta; per token the k + 1 largest keys, key descending, ties to the
        lower expert index: the first k are the selected experts, and the (k+1)-th key is
        the token's alpha;
      with update (T k a multiple of E): target = T k / E tokens per expert, and expert e's
        solved bias is the (target + 1)-th largest of scores[:, e] - alpha over the tokens.
    scores [T, E], beta [E].  Returns idx [T, k], alpha [T] fp32, beta_local [E] fp32 (None
    without update).
    """
    s = np.asarray(scores, dtype=np.float32)
    b = np.asarray(beta, dtype=np.float32)
    T, E = s.shape
    if k + 1 > E:
        raise ValueError("quantile routing needs k < E")
    keys = (s - b[None, :]).astype(np.float32)
    order = np.argsort(-keys, axis=1, kind="stable")[:, :k + 1]
    idx = order[:, :k].astype(np.int64)
    alpha = keys[np.arange(T), order[:, k]]
    if not update:
        return idx, alpha, None
    if (T * k) % E:
        raise ValueError("quantile balancing needs T * k to be a multiple of E")
    target = T * k // E
    v = (s - alpha[:, None]).astype(np.float32)
    beta_local = -np.sort(-v, axis=0)[target, :]
    return idx, alpha, beta_local.astype(np.float32)


def quantile_bias_update(beta, beta_local_avg, ema: float):
    """The step update of the quantile bias ([HB] §3.3 Quantile): an exponential moving
    average that keeps `ema` of the previous bias and mixes in the rest of the new solution
    (the solutions of the step's micro-batches, averaged by the caller), then the mean over
    the experts is taken out.  float64."""
    new = ema * _d(beta) + (1.0 - ema) * _d(beta_local_avg)
    return new - new.mean()


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


@dataclass(frozen=True)
class GLU:
    """The gated activation between an expert's projections ([HB] §3.4 Activation).

    kind "swiglu": silu(gate) * up;
    kind "clamp":  the hard clamp: gate clamped from above at c, up clamped to [-c, c],
                   then silu(gate) * up;
    kind "situ":   SiTU-GLU: s tanh(gate / s) sigma(gate) * up', with up' = s_l tanh(up / s_l)
                   when s_l > 0, else up (c is s, c_linear is s_l).
    """
    kind: str = "swiglu"
    c: float = 0.0
    c_linear: float = 0.0


SWIGLU = GLU()


def glu_forward(H, glu: GLU = SWIGLU):
    """Act from H = [gate | up] (gate half first)."""
    H = _d(H)
    F = H.shape[1] // 2
    g, u = H[:, :F], H[:, F:]
    if glu.kind == "swiglu":
        return silu(g) * u
    if glu.kind == "clamp":
        return silu(np.minimum(g, glu.c)) * np.clip(u, -glu.c, glu.c)
    if glu.kind == "situ":
        a = glu.c * np.tanh(g / glu.c) * sigmoid(g)
        ul = glu.c_linear * np.tanh(u / glu.c_linear) if glu.c_linear > 0 else u
        return a * ul
    raise ValueError(glu.kind)


def glu_backward(H, dAct, glu: GLU = SWIGLU):
    """dH = [dgate | dup] by the chain rule (derived; the pages print the forward only).

    silu'(g) = sigma(g) (1 + g (1 - sigma(g)));  a clamp passes the gradient where its
    input lies inside the closed interval and none outside;  d/dx [s tanh(x/s) sigma(x)] =
    (1 - tanh^2(x/s)) sigma(x) + s tanh(x/s) sigma(x) (1 - sigma(x));
    d/dx [s_l tanh(x/s_l)] = 1 - tanh^2(x/s_l).
    """
    H, dAct = _d(H), _d(dAct)
    F = H.shape[1] // 2
    g, u = H[:, :F], H[:, F:]
    if glu.kind in ("swiglu", "clamp"):
        gc, uc = (g, u) if glu.kind == "swiglu" else (np.minimum(g, glu.c), np.clip(u, -glu.c, glu.c))
        s = sigmoid(gc)
        dg = dAct * uc * s * (1.0 + gc * (1.0 - s))
        du = dAct * gc * s
        if glu.kind == "clamp":
            dg = np.where(g <= glu.c, dg, 0.0)
            du = np.where(np.abs(u) <= glu.c, du, 0.0)
        return np.concatenate([dg, du], axis=1)
    if glu.kind == "situ":
        sc = glu.c
        th, s = np.tanh(g / sc), sigmoid(g)
        a = sc * th * s
        da = (1.0 - th * th) * s + sc * th * s * (1.0 - s)
        if glu.c_linear > 0:
            tl = np.tanh(u / glu.c_linear)
            ul, dul = glu.c_linear * tl, 1.0 - tl * tl
        else:
            ul, dul = u, np.ones_like(u)
        return np.concatenate([dAct * ul * da, dAct * a * dul], axis=1)
    raise ValueError(glu.kind)


def swiglu_forward(X, W13, W2, glu: GLU = SWIGLU):
    """One bias-free gated expert on rows X.

    [HB] §3.4 Experts, Count and size (fc1 is twice the expert width for a gated
    linear unit; fc2 maps the width back to d) and Activation (the GLU splits fc1's
    output in two halves, gate first, and multiplies silu(gate) by the up half; the clamp
    and SiTU-GLU variants bound it).
    Returns H = X W13^T [n, 2F], Act = glu(H) [n, F], Y = Act W2^T [n, d].
    """
    H = _d(X) @ _d(W13).T
    Act = glu_forward(H, glu)
    Y = Act @ _d(W2).T
    return H, Act, Y


def swiglu_backward(X, W13, W2, H, dY, glu: GLU = SWIGLU):
    """Backward of swiglu_forward by the chain rule (derived, not printed on the pages).

    dAct = dY W2; dH = glu_backward(H, dAct) (for plain SwiGLU, with s = sigma(g):
    dH_gate = dAct * up * s (1 + g (1 - s)), dH_up = dAct * silu(g));
    dX = dH W13, dW13 = dH^T X, dW2 = dY^T Act.
    """
    X, W13, W2, H, dY = map(_d, (X, W13, W2, H, dY))
    act = glu_forward(H, glu)
    dAct = dY @ W2
    dH = glu_backward(H, dAct, glu)
    return dict(dX=dH @ W13, dW13=dH.T @ X, dW2=dY.T @ act, dH=dH, dAct=dAct)


# ------------------------------------------------------------------------ full layer

@dataclass
class LayerSpec:
    E: int
    k: int
    score: str = "softmax"          # "softmax" | "sigmoid" | "sqrtsoftplus"
    scaling: float = 1.0
    aux_coeff: float = 0.0
    pre_softmax: bool = False       # softmax only: weights from the full softmax, no renormalisation
    z_coeff: float = 0.0            # router z-loss coefficient
    seq_aux_coeff: float = 0.0      # sequence-wise balance loss coefficient
    seq_len: int = 0                # S of that loss (tokens ordered [S, B])
    glu: GLU = SWIGLU               # the experts' gated activation
    num_groups: int = 0             # group-limited routing: groups of experts (0 = off)
    group_topk: int = 0             # groups kept per token
    shared_gate: bool = False       # a sigmoid gate on the shared expert's output


def route(logits, spec: LayerSpec, expert_bias=None) -> Dict[str, np.ndarray]:
    """Router: keys -> top-k -> weights -> counts and load statistics and losses.

    The balancing losses (aux, z, sequence-wise) are all reported; a zero coefficient
    gives a zero loss.
    """
    keys = selection_keys(logits, spec.score, expert_bias)
    if spec.num_groups:
        idx, _, gmargin = group_limited_topk(keys, spec.k, spec.num_groups, spec.group_topk)
        # the keys a token can still pick from, and the nearer of its two decisions
        allowed = np.zeros(keys.shape, dtype=bool)
        n = spec.E // spec.num_groups
        for j in range(spec.k):
            g = idx[:, j] // n
            for q in range(n):
                allowed[np.arange(keys.shape[0]), g * n + q] = True
        margin = np.minimum(margins(np.where(allowed, keys, -np.inf), spec.k), gmargin)
    else:
        idx = topk(keys, spec.k)
        margin = margins(keys, spec.k)
    w = mixing_weights(logits, idx, spec.score, spec.scaling, spec.pre_softmax)
    counts = expert_counts(idx, spec.E)
    out = dict(keys=keys, idx=idx, w=w, counts=counts, margin=margin, maxvio=max_violation(counts))
    p = aux_probs(logits, spec.score)
    out["prob_sum"] = p.sum(axis=0)
    out["aux"] = aux_loss(counts, p, spec.k, spec.aux_coeff)
    out["z"] = z_loss(logits, spec.z_coeff)
    if spec.seq_len:
        out["seq_counts"] = sequence_counts(idx, spec.E, spec.seq_len)
        out["seq_aux"] = seq_aux_loss(idx, p, spec.k, spec.seq_len, spec.seq_aux_coeff)
    else:
        out["seq_counts"] = None
        out["seq_aux"] = 0.0
    return out


def layer_forward(x, Wg, W13, W2, spec: LayerSpec, bg=None, expert_bias=None,
                  W13s=None, W2s=None, idx=None, Wsg=None) -> Dict[str, object]:
    """The whole layer forward.

    y_t = sum_j w_tj * Expert_{idx_tj}(x_t) + gs_t * Shared(x_t)
    ([LC] "An expert transforms numbers inside the model": the weighted sum of the
    selected experts' outputs, coordinate by coordinate; [HB] §3.4 Shared experts:
    without a gate the shared output is added at weight 1, gs_t = 1; with the sigmoid gate,
    gs_t = sigma(x_t . Wsg), Wsg [d]).
    `idx` may be given to evaluate the layer at a fixed routing.  W13 and W2 only need
    per-expert indexing (W13[e] -> [2F, d]), so a lazily converted stack works.
    """
    x = _d(x)
    T, d = x.shape
    logits = gate_logits(x, Wg, bg)
    r = route(logits, spec, expert_bias)
    if idx is not None:
        r["idx"] = np.asarray(idx, dtype=np.int64)
        r["w"] = mixing_weights(logits, r["idx"], spec.score, spec.scaling, spec.pre_softmax)
        r["counts"] = expert_counts(r["idx"], spec.E)
        if spec.seq_len:
            r["seq_counts"] = sequence_counts(r["idx"], spec.E, spec.seq_len)
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
            H[a:b], Act[a:b], Yp[a:b] = swiglu_forward(xp[a:b], W13[e], W2[e], spec.glu)
    y = np.einsum("tk,tkd->td", r["w"], Yp[perm.row_of])
    shared = None
    if W13s is not None:
        Hs, Acts, Ys = swiglu_forward(x, W13s, W2s, spec.glu)
        gs = sigmoid(x @ _d(Wsg)) if spec.shared_gate else np.ones(T)
        y = y + gs[:, None] * Ys
        shared = dict(H=Hs, Act=Acts, Y=Ys, gs=gs)
    return dict(logits=logits, route=r, perm=perm, x_perm=xp, H=H, Act=Act, Y_perm=Yp,
                shared=shared, y=y)


def router_backward(logits, idx, w, dw, spec: LayerSpec, counts=None, daux: float = 1.0, seq_counts=None):
    """d(loss)/d(logits) from the mixing-weight gradient dw [T, k] and the balancing losses.

    Selected set S, scaling factor c:
      softmax (renormalised), w = c * softmax(l_S):  dl_S = w * dw - (w / c) * <w, dw>;
      softmax with pre-softmax, w = c * p_S, p the full softmax: through the full softmax
        with the upstream gradient c * dw at the selected experts (below);
      sigmoid / sqrt(softplus) renormalised (k > 1), z = sum s(l_S) + 1e-20, w = c * s / z:
        ds = (c / z) * (dw - <dw, s> / z),  dl_S = ds * s'(l_S);  k == 1: ds = c * dw.
    Balancing losses, counts held constant, q_t the aux probabilities of the token:
      aux:      g_e = coeff * E * counts_e / (k T^2);
      seq aux:  g_e = coeff * E * seq_counts[b(t), e] / (k S^2 B);
      through q: softmax q: dl_t += q_t * (G - <G, q_t>);  normalised scores
        q = s / Z (Z = sum_e s + 1e-20): dl_t += s'(l_t) * (G - <G, q_t>) / Z,
      G = daux * (the g above) (+ c * dw scattered to S for pre-softmax);
      z-loss:   dl_t += daux * z_coeff * (2 / T) * lse_t * softmax(l_t).
    """
    l = _d(logits)
    T, E = l.shape
    k = idx.shape[1]
    c = spec.scaling
    dw = _d(dw)
    w = _d(w)
    dl = np.zeros_like(l)
    G = np.zeros_like(l)
    if spec.score == "softmax" and spec.pre_softmax:
        np.put_along_axis(G, idx, c * dw, axis=1)
    elif spec.score == "softmax":
        dlS = w * dw - (w / c) * np.sum(w * dw, axis=1, keepdims=True)
        np.put_along_axis(dl, idx, dlS, axis=1)
    else:
        lS = np.take_along_axis(l, idx, axis=1)
        s = score_values(lS, spec.score)
        if k > 1:
            z = s.sum(axis=1, keepdims=True) + 1e-20
            ds = (c / z) * (dw - np.sum(dw * s, axis=1, keepdims=True) / z)
        else:
            ds = c * dw
        np.put_along_axis(dl, idx, ds * score_derivative(lS, spec.score), axis=1)
    if daux != 0.0 and spec.aux_coeff != 0.0:
        G += daux * spec.aux_coeff * E * np.asarray(counts, dtype=f64)[None, :] / (k * T * T)
    if daux != 0.0 and spec.seq_aux_coeff != 0.0:
        S = spec.seq_len
        B = T // S
        sc = np.asarray(seq_counts, dtype=f64)
        G += daux * spec.seq_aux_coeff * E * sc[sequence_of_token(T, S)] / (k * S * S * B)
    if np.any(G):
        q = aux_probs(l, spec.score)
        Gq = np.sum(G * q, axis=1, keepdims=True)
        if spec.score == "softmax":
            dl += q * (G - Gq)
        else:
            Z = score_values(l, spec.score).sum(axis=1, keepdims=True) + 1e-20
            dl += score_derivative(l, spec.score) * (G - Gq) / Z
    if daux != 0.0 and spec.z_coeff != 0.0:
        dl += daux * spec.z_coeff * (2.0 / T) * logsumexp_rows(l)[:, None] * softmax_full(l)
    return dl


def layer_backward(fwd: Dict[str, object], x, Wg, W13, W2, dy, spec: LayerSpec,
                   W13s=None, W2s=None, daux: float = 1.0, sparse_expert_grads: bool = False,
                   Wsg=None) -> Dict[str, np.ndarray]:
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
            g = swiglu_backward(xp[a:b], W13[e], W2[e], fwd["H"][a:b], dYp[a:b], spec.glu)
            dXp[a:b], dW13[e], dW2[e], dH[a:b] = g["dX"], g["dW13"], g["dW2"], g["dH"]
    dx = dXp[rows].sum(axis=1)
    out = dict(dw=dw, dY_perm=dYp, dX_perm=dXp, dH=dH, dW13=dW13, dW2=dW2)
    if W13s is not None:
        sh = fwd["shared"]
        # the gate: dY_s = gs dy;  d gs_t = <dy_t, Y_s[t]>, through sigma: gs (1 - gs)
        gsh = swiglu_backward(x, W13s, W2s, sh["H"], sh["gs"][:, None] * dy, spec.glu)
        dx = dx + gsh["dX"]
        out.update(dW13s=gsh["dW13"], dW2s=gsh["dW2"], dH_s=gsh["dH"])
        if spec.shared_gate:
            dl = sh["gs"] * (1.0 - sh["gs"]) * np.sum(dy * sh["Y"], axis=1)
            out.update(dl_s=dl, dWsg=dl @ x)
            dx = dx + dl[:, None] * _d(Wsg)[None, :]
    dlogits = router_backward(fwd["logits"], idx, w, dw, spec, counts=r["counts"], daux=daux,
                              seq_counts=r.get("seq_counts"))
    out["dlogits"] = dlogits
    out["dWg"] = dlogits.T @ x
    out["dbg"] = dlogits.sum(axis=0)
    out["dx_router"] = dlogits @ _d(Wg)
    out["dx"] = dx + out["dx_router"]
    return out


def layer_loss(x, Wg, W13, W2, dy, spec: LayerSpec, bg=None, expert_bias=None,
               W13s=None, W2s=None, daux: float = 1.0, Wsg=None) -> float:
    """L = sum(dy * y) + daux * (aux + z + seq_aux), the scalar whose gradient
    layer_backward returns."""
    f = layer_forward(x, Wg, W13, W2, spec, bg=bg, expert_bias=expert_bias, W13s=W13s, W2s=W2s, Wsg=Wsg)
    r = f["route"]
    return float(np.sum(_d(dy) * f["y"]) + daux * (r["aux"] + r["z"] + r["seq_aux"]))


# ------------------------------------------------------------------------ fp8 experts
#
# The pages give no low-precision recipe for the expert GEMMs ([HB] §3.1 Precision only
# asks for an fp32 router).  The reading taken for the fp8 layer:
#   * format: OCP e4m3 (E4M3FN): sign, 4 exponent bits with bias 7, 3 mantissa bits;
#     the largest finite magnitude is 448 (exponent 15, mantissa 6), there is no infinity;
#   * one fp32 scale per block (128 x 128 for expert weights, 1 x 128 per token for
#     activations): scale = amax / 448 evaluated in fp32, or 1 for an all-zero block;
#   * code = the e4m3 value nearest to v / scale (the quotient in fp32), ties to the even
#     code, magnitudes above 448 saturated to 448; the sign bit is the sign of v;
#   * value = decode(code) * scale.
# Both decisions that produce integers (the quotient and its rounding) are taken in fp32,
# the precision of the kernel, so that both sides pick the same codes.

E4M3_MAX = 448.0


def e4m3_magnitudes() -> np.ndarray:
    """The 127 non-negative finite e4m3 values, indexed by their codes 0x00..0x7E."""
    out = np.zeros(127)
    for c in range(127):
        e, m = c >> 3, c & 7
        out[c] = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_E4M3 = e4m3_magnitudes()


def e4m3_decode(codes) -> np.ndarray:
    """uint8 codes (never 0x7F or 0xFF) -> float64 values."""
    c = np.asarray(codes).astype(np.int64)
    mag = _E4M3[c & 0x7F]
    return np.where(c & 0x80, -mag, mag)


def e4m3_encode(v) -> np.ndarray:
    """Values (exactly representable in fp32) -> e4m3 codes, by the rule above."""
    v = np.asarray(v, dtype=np.float32).astype(f64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.clip(np.searchsorted(_E4M3, a, side="left"), 0, 126)
    lo = np.maximum(hi - 1, 0)
    d_hi = _E4M3[hi] - a
    d_lo = a - _E4M3[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == 0.0, 0, code)
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def quantize_blocks(v, block_rows: int, block_cols: int = 128):
    """v [R, C] -> (codes uint8 [R, C], scales float32 [R / block_rows, C / block_cols]).

    One scale per block of block_rows x block_cols, by the rule above.
    """
    v = np.asarray(v, dtype=np.float32)
    R, C = v.shape
    assert R % block_rows == 0 and C % block_cols == 0
    blocks = np.abs(v).reshape(R // block_rows, block_rows, C // block_cols, block_cols)
    amax = blocks.max(axis=(1, 3)).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    full = np.repeat(np.repeat(scale, block_rows, axis=0), block_cols, axis=1)
    return e4m3_encode(v / full), scale


def dequantize_blocks(codes, scales, block_rows: int, block_cols: int = 128) -> np.ndarray:
    """decode(code) * scale in float64."""
    full = np.repeat(np.repeat(_d(scales), block_rows, axis=0), block_cols, axis=1)
    return e4m3_decode(codes) * full


def layer_forward_fp8(x, Wg, W13q, W13_scale, W2q, W2_scale, spec: "LayerSpec", bg=None,
                      expert_bias=None) -> Dict[str, object]:
    """The layer forward with e4m3 expert weights and activations.

    Routing as in layer_forward (fp32-exact logits of the given x).  The expert GEMMs take
    x quantised per token per 128 columns, the weights given as codes and 128 x 128
    block scales, and the SwiGLU output quantised per token per 128 columns after a cast
    to fp32; every product and sum after dequantisation is exact (float64).
    """
    x = _d(x)
    T, d = x.shape
    logits = gate_logits(x, Wg, bg)
    r = route(logits, spec, expert_bias)
    perm = permutation(r["idx"], spec.E)
    xq, xs = quantize_blocks(x.astype(np.float32), 1)
    xd = dequantize_blocks(xq, xs, 1)
    xp = xd[perm.token_of]
    F = np.shape(W2q[int(r["idx"].ravel()[0])])[1]
    A = T * spec.k
    H = np.zeros((A, 2 * F))
    Act = np.zeros((A, F))
    Actq = np.zeros((A, F), dtype=np.uint8)
    Acts = np.ones((A, F // 128), dtype=np.float32)
    Yp = np.zeros((A, d))
    for e in range(spec.E):
        a, b = perm.offsets[e], perm.offsets[e + 1]
        if b == a:
            continue
        w13 = dequantize_blocks(W13q[e], W13_scale[e], 128)
        w2 = dequantize_blocks(W2q[e], W2_scale[e], 128)
        H[a:b] = xp[a:b] @ w13.T
        Act[a:b] = glu_forward(H[a:b], spec.glu)
        Actq[a:b], Acts[a:b] = quantize_blocks(Act[a:b].astype(np.float32), 1)
        Yp[a:b] = dequantize_blocks(Actq[a:b], Acts[a:b], 1) @ w2.T
    y = np.einsum("tk,tkd->td", r["w"], Yp[perm.row_of])
    return dict(logits=logits, route=r, perm=perm, x_q=xq, x_scale=xs, H=H, Act=Act, Act_q=Actq,
                Act_scale=Acts, Y_perm=Yp, y=y)


def router_path_backward(fwd: Dict[str, object], x, Wg, dy, spec: "LayerSpec", daux: float = 1.0):
    """The backward through the mixing weights only (combine -> router -> gate GEMM), as
    for a layer whose expert weights are frozen: dw, dlogits, dWg, dbg and the input
    gradient of the router path.  Same formulas as layer_backward."""
    x, dy = _d(x), _d(dy)
    r, perm = fwd["route"], fwd["perm"]
    dw = np.einsum("td,tkd->tk", dy, fwd["Y_perm"][perm.row_of])
    dl = router_backward(fwd["logits"], r["idx"], r["w"], dw, spec, counts=r["counts"], daux=daux,
                         seq_counts=r.get("seq_counts"))
    return dict(dw=dw, dlogits=dl, dWg=dl.T @ x, dbg=dl.sum(axis=0), dx_router=dl @ _d(Wg))


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
