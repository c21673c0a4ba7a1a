"""Token sampling and the speculative accept / resample rule.

The pages state that speculative decoding is lossless and that EasySpec keeps
the base model's output distribution (abstract; rebuttal reply on the 7%
accuracy drop); they cite Leviathan et al., "Fast Inference from Transformers
via Speculative Decoding" and Chen et al., "Accelerating Large Language Model
Decoding with Speculative Sampling" for the rule.  Written out (standard
speculative sampling):
  for j = 1..k: accept draft d_j with probability min(1, p_j(d_j) / q_j(d_j));
  at the first rejection emit y ~ norm(max(0, p_j - q_j)) and stop;
  if all k are accepted emit a bonus y ~ p_{k+1}.
With temperature T > 0, p_j = softmax(z^base_j / T), q_j = softmax(z^draft_j / T).
Greedy (T = 0): accept iff d_j = argmax p_j; y = argmax p_j at the first
mismatch, else argmax p_{k+1}.  Ties go to the lowest index.

Sampling primitive (build's reading): Gumbel-max, y = argmax_v (s_v + G_v)
with G_v = -log(-log u_v) and u_v from the Philox stream of the decision; for a
categorical with log-weights s this samples exactly softmax(s).  The accept
test draws one uniform u and accepts iff u * q(d) < p(d).
"""
from __future__ import annotations

import numpy as np

from . import philox


def argmax_first(x) -> int:
    return int(np.argmax(x))   # numpy returns the first maximal index


def top2_gap(x) -> float:
    x = np.asarray(x, dtype=np.float64)
    if x.size < 2:
        return np.inf
    i = int(np.argmax(x))
    rest = np.delete(x, i)
    return float(x[i] - rest.max())


def gumbel(u):
    return -np.log(-np.log(u))


def softmax(z):
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - z.max())
    return e / e.sum()


def sample_from_logits(z, inv_temp: float, seed: int, b: int, pos: int, purpose: int):
    """Sample the token for position `pos` from logits z.  Returns (token, margin)."""
    z = np.asarray(z, dtype=np.float64)
    if inv_temp == 0.0:
        return argmax_first(z), top2_gap(z)
    s = z * inv_temp + gumbel(philox.stream_uniforms(seed, b, pos, purpose, z.size))
    return argmax_first(s), top2_gap(s)


def draw_residual(zp, zq, inv_temp: float, seed: int, b: int, pos: int):
    """y ~ norm(max(0, p - q)) for the decision at `pos` (T > 0).
    Falls back to p when no entry has p > q.  Returns (y, margin)."""
    p = softmax(np.asarray(zp, dtype=np.float64) * inv_temp)
    q = softmax(np.asarray(zq, dtype=np.float64) * inv_temp)
    diff = p - q
    g = gumbel(philox.stream_uniforms(seed, b, pos, philox.TARGET, p.size))
    if np.any(diff > 0):
        with np.errstate(divide="ignore"):
            s = np.where(diff > 0, np.log(np.where(diff > 0, diff, 1.0)), -np.inf) + g
    else:
        s = np.log(p) + g
    return argmax_first(s), top2_gap(s[np.isfinite(s)])


def draw_bonus(zp, inv_temp: float, seed: int, b: int, pos: int):
    """y ~ p = softmax(zp / T) (argmax of zp when T = 0).  Returns (y, margin)."""
    return sample_from_logits(zp, inv_temp, seed, b, pos, philox.TARGET)


def draw_y(p_logits, q_logits, a: int, t: int, inv_temp: float, seed: int, b: int):
    """The emitted token of a round whose accepted prefix has length a."""
    k = len(q_logits)
    if inv_temp == 0.0 or a >= k:
        return draw_bonus(p_logits[a], inv_temp, seed, b, t + a + 1)
    return draw_residual(p_logits[a], q_logits[a], inv_temp, seed, b, t + a + 1)


def accept_resample(p_logits, q_logits, drafts, t: int, inv_temp: float, seed: int, b: int):
    """One accept / resample decision for one sequence.

    p_logits [k+1][V] (base), q_logits [k][V] (draft), drafts [k]; the round's
    pending token sits at position t, so d_j is at position t + j.
    Returns (a, y, info); info['margins'] lists (kind, j, margin) for every
    decision taken: the accept test margin is |u - p/q|, the argmax and Gumbel
    margins are the top-2 gaps of the maximised scores.
    """
    p_logits = np.asarray(p_logits, dtype=np.float64)
    q_logits = np.asarray(q_logits, dtype=np.float64)
    k = len(drafts)
    margins = []
    a = k
    for j in range(1, k + 1):
        d = int(drafts[j - 1])
        if inv_temp == 0.0:
            zp = p_logits[j - 1]
            margins.append(("argmax", j, top2_gap(zp)))
            ok = d == argmax_first(zp)
        else:
            p = softmax(p_logits[j - 1] * inv_temp)
            q = softmax(q_logits[j - 1] * inv_temp)
            u = float(philox.stream_uniform0(seed, b, t + j, philox.ACCEPT))
            ratio = p[d] / q[d] if q[d] > 0 else np.inf
            margins.append(("accept", j, abs(u - ratio)))
            ok = u * q[d] < p[d]
        if not ok:
            a = j - 1
            break
    y, mg = draw_y(p_logits, q_logits, a, t, inv_temp, seed, b)
    margins.append(("y", a + 1, mg))
    return a, y, {"margins": margins}


def accept_law(p, q):
    """Exact output law of one accept/resample step with a draft d ~ q:
    P(y) = q(y) min(1, p(y)/q(y)) + (1 - sum_v min(p_v, q_v)) r(y),
    r = max(0, p - q) / sum(max(0, p - q))."""
    p = np.asarray(p, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    acc = np.minimum(p, q)
    resid = np.maximum(p - q, 0.0)
    rej = 1.0 - acc.sum()
    r = resid / resid.sum() if resid.sum() > 0 else p
    return acc + rej * r


def accept_resample_batch(p, q, seed, b, t, inv_temp_unused=None):
    """Vectorised k = 1 accept/resample over many independent sequences for the
    statistical tests: p, q are [V] probability vectors (the step's base and
    draft distributions); sequence b draws its draft from q with the DRAFT
    stream at position t+1, then runs the rule above.  Returns y [nb]."""
    b = np.asarray(b)
    V = p.size
    logq, logp = np.log(q), np.log(p)
    ud = philox.stream_uniforms(seed, b, t + 1, philox.DRAFT, V)
    d = np.argmax(logq[None, :] + gumbel(ud), axis=1)
    ua = philox.stream_uniform0(seed, b, t + 1, philox.ACCEPT)
    accepted = ua * q[d] < p[d]
    ur = philox.stream_uniforms(seed, b, t + 1, philox.TARGET, V)
    diff = p - q
    with np.errstate(divide="ignore"):
        ls = np.where(diff > 0, np.log(np.where(diff > 0, diff, 1.0)), -np.inf)
    y_res = np.argmax(ls[None, :] + gumbel(ur), axis=1)
    return np.where(accepted, d, y_res)
