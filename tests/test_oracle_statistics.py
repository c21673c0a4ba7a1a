"""Statistical pins: the accept / resample rule and the whole round loop keep
the base distribution (EasySpec abstract: the original distributions of the
base model are preserved), checked by closed form and by chi-square tests on
seeded trials."""
import numpy as np
import pytest
from scipy import stats

from oracle import model as oracle_model
from oracle import philox, sampling
from oracle.decode import spec_generate
from oracle.model import KVCache, OracleModel, forward
from oracle.plan import default_group_plan
from oracle.sampling import accept_law, accept_resample, accept_resample_batch, sample_from_logits, softmax
from helpers import tiny_pair
from synth import make_weights, tiny_shape

P_MIN = 1e-4      # reject the null below this p-value


def _pq(V, seed, alpha=0.7):
    rng = np.random.default_rng(seed)
    p = rng.dirichlet(np.full(V, alpha)) + 1e-3
    q = rng.dirichlet(np.full(V, alpha)) + 1e-3
    return p / p.sum(), q / q.sum()


def _chi2_p(counts, probs):
    exp = probs * counts.sum()
    return stats.chisquare(counts, exp).pvalue


@pytest.mark.parametrize("V", [2, 4, 16, 256])
def test_one_step_law_is_exactly_p(V):
    for s in range(5):
        p, q = _pq(V, 100 + s)
        np.testing.assert_allclose(accept_law(p, q), p, rtol=0, atol=1e-12)
    # equal distributions: everything accepted, no residual mass
    np.testing.assert_allclose(accept_law(p, p), p, atol=1e-15)


def _first_token(p, q, seed, b, t=10):
    zq = np.log(q)
    d, _ = sample_from_logits(zq, 1.0, seed, b, t + 1, philox.DRAFT)
    a, y, _ = accept_resample(np.stack([np.log(p), np.log(p)]), zq[None], [d], t, 1.0, seed, b)
    return d if a == 1 else y


@pytest.mark.parametrize("V,n", [(4, 8000), (16, 8000)])
def test_accept_resample_chi2(V, n):
    p, q = _pq(V, 7 + V)
    ys = np.array([_first_token(p, q, 1234, b) for b in range(n)])
    assert _chi2_p(np.bincount(ys, minlength=V), p) > P_MIN


def test_batched_rule_equals_per_sequence_rule():
    p, q = _pq(8, 3)
    yb = accept_resample_batch(p, q, 77, np.arange(1500), 10)
    ys = np.array([_first_token(p, q, 77, b) for b in range(1500)])
    np.testing.assert_array_equal(yb, ys)


@pytest.mark.parametrize("V,n", [(4, 1_000_000), (16, 200_000), (256, 20_000)])
def test_accept_resample_chi2_large(V, n):
    p, q = _pq(V, 31 + V)
    counts = np.zeros(V, dtype=np.int64)
    for lo in range(0, n, 50_000):
        y = accept_resample_batch(p, q, 555, np.arange(lo, min(n, lo + 50_000)), 3)
        counts += np.bincount(y, minlength=V)
    assert _chi2_p(counts, p) > P_MIN


def test_chi2_detects_a_planted_mistake(monkeypatch):
    """Power check: resampling from p instead of the residual max(0, p - q)
    (a plausible mistake) must fail the same test."""
    V, n = 4, 8000
    p, q = _pq(V, 7 + V)

    def wrong(zp, zq, inv_temp, seed, b, pos):
        return sample_from_logits(zp, inv_temp, seed, b, pos, philox.TARGET)
    monkeypatch.setattr(sampling, "draw_residual", wrong)
    ys = np.array([_first_token(p, q, 1234, b) for b in range(n)])
    assert _chi2_p(np.bincount(ys, minlength=V), p) < P_MIN


@pytest.mark.parametrize("inv_temp", [1.0, 1.0 / 0.7])
def test_gumbel_sampler_chi2(inv_temp):
    rng = np.random.default_rng(5)
    z = rng.normal(size=10)
    n = 20000
    ys = np.array([sample_from_logits(z, inv_temp, 9, b, 4, philox.DRAFT)[0] for b in range(n)])
    assert _chi2_p(np.bincount(ys, minlength=10), softmax(z * inv_temp)) > P_MIN


def test_greedy_sampler_is_first_argmax():
    z = np.array([0.5, 2.0, -1.0, 2.0])
    assert sample_from_logits(z, 0.0, 1, 0, 0, philox.DRAFT)[0] == 1


def test_round_loop_preserves_base_joint_law():
    """The first two emitted tokens of speculative decoding with a
    layer-parallel draft follow the base model's autoregressive joint law
    p(x1) p(x2 | x1).  Exercises drafting, verify indexing, acceptance,
    residual and bonus draws and the calibration seam."""
    V = 5
    ds, dw, bs, bw = tiny_pair(V=V, base_layers=3, draft_noise=0.35, d=16, hq=2, hkv=1, hd=8, ffn=32)
    d, b = OracleModel.from_torch(ds, dw), OracleModel.from_torch(bs, bw)
    prompt = [1, 3, 0]
    # exact base law
    c = KVCache(bs, 1, 16)
    z1 = forward(b, c, 0, prompt, range(3), logits="last")
    p1 = softmax(z1)
    joint = np.zeros((V, V))
    for x1 in range(V):
        c2 = KVCache(bs, 1, 16)
        z2 = forward(b, c2, 0, prompt + [x1], range(4), logits="last")
        joint[x1] = p1[x1] * softmax(z2)
    sets = [[0], [1, 2]]      # a real layer-parallel set (default grouping of 3 layers: singletons)
    n = 2500
    counts = np.zeros((V, V), dtype=np.int64)
    acc = 0
    for s in range(n):
        toks, rounds = spec_generate(d, b, prompt, 2, sets, 2, 1.0, 1000 + s)
        counts[toks[0], toks[1]] += 1
        acc += rounds[0]["a"]
    assert 0.2 * n < acc < 1.8 * n          # both accept and reject paths are exercised
    assert _chi2_p(counts.ravel(), joint.ravel()) > P_MIN


def _expected_overlap(V, sd_p, sd_q, n, seed):
    """E[sum_v min(p_v, q_v)] for p = softmax(z_p), q = softmax(z_q) with
    independent logit vectors of i.i.d. N(0, sd^2) entries (Monte Carlo)."""
    rng = np.random.default_rng(seed)
    tot = 0.0
    for _ in range(n // 2000):
        zp = rng.normal(size=(2000, V)) * sd_p
        zq = rng.normal(size=(2000, V)) * sd_q
        p = np.exp(zp - zp.max(1, keepdims=True))
        q = np.exp(zq - zq.max(1, keepdims=True))
        tot += np.minimum(p / p.sum(1, keepdims=True), q / q.sum(1, keepdims=True)).sum()
    return tot / n


def _observed_acceptance(inv_temp, sw, V, dq, dp, k, n_pairs=6, new_tokens=120):
    """Per-draft acceptance of the round loop on independent random-init
    pairs: accepted drafts / tested drafts (a round tests min(a + 1, k))."""
    acc = tested = 0
    for s in range(n_pairs):
        ds = tiny_shape(4, dq, 4, 2, 8, 64, V)
        bs = tiny_shape(3, dp, 4, 2, 16, 128, V)
        d = OracleModel.from_torch(ds, make_weights(ds, 50 + 2 * s, std=sw))
        b = OracleModel.from_torch(bs, make_weights(bs, 51 + 2 * s, std=sw))
        prompt = np.random.default_rng(s).integers(0, V, size=8).tolist()
        _, rounds = spec_generate(d, b, prompt, k, default_group_plan(4, 2), new_tokens, inv_temp, 900 + s)
        for r in rounds:
            acc += r["a"]
            tested += min(r["a"] + 1, len(r["drafts"]))
    return acc / tested, tested


def _check_random_init_acceptance(T):
    V, sw, k, dq, dp = 256, 0.15, 4, 32, 64
    # unit gains: the final RMSNorm leaves a hidden state of squared norm d,
    # so with an independent N(0, sw^2) lm head the logits are i.i.d.
    # N(0, sw^2 d) given the state, independently for draft and base
    alpha = _expected_overlap(V, sw * np.sqrt(dp) / T, sw * np.sqrt(dq) / T, 40_000, 1)
    obs, n = _observed_acceptance(1.0 / T, sw, V, dq, dp, k)
    return alpha, obs, n


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_random_init_acceptance_matches_closed_form(T):
    """Acceptance on random-init pairs is fixed by the weights' law: a draft
    d ~ q is accepted with probability sum_v min(p_v, q_v) (the accept rule
    the pages cite), whose expectation over i.i.d. Gaussian logits is
    computable.  The layer-parallel draft changes q's hidden state, not its
    law, so the same value holds for any plan."""
    alpha, obs, n = _check_random_init_acceptance(T)
    se = np.sqrt(alpha * (1 - alpha) / n)
    assert abs(obs - alpha) < 4 * se + 0.02, (alpha, obs, n)


def test_random_init_acceptance_detects_a_planted_mistake(monkeypatch):
    """Power check: a head that skips the final RMSNorm (logit scale no
    longer sw * sqrt(d)) must fail the same comparison."""
    monkeypatch.setattr(oracle_model, "final_logits", lambda m, h: oracle_model.linear(h, m.w["lm_head"]))
    alpha, obs, n = _check_random_init_acceptance(1.0)
    se = np.sqrt(alpha * (1 - alpha) / n)
    assert abs(obs - alpha) > 4 * se + 0.02, (alpha, obs, n)


# a 4-layer draft plan with a real layer-parallel set (the default grouping of
# 4 layers in sets of 2 has only singletons: layers 1 and 2 fall in different
# aligned pairs)
FUZZY4 = [[0], [1, 2], [3]]


def _round_law(d, b, prompt, k, sets, inv_t, separate):
    """Exact law of the tokens one round emits, E = (d_1..d_a, y), over every
    draft path: spec_generate runs the round with the drafts forced through its
    hook and returns the draft and base distributions it computed for that
    path; the accept rule composes them (accept d_j with probability
    min(1, p_j(d_j) / q_j(d_j)), at the first rejection y ~ max(0, p_j - q_j)
    normalised, after k acceptances y ~ p_{k+1})."""
    import itertools
    V = b.shape.vocab
    law = {}
    for path in itertools.product(range(V), repeat=k):
        hook = lambda kind, key, value, margin: path[key[1] - 1] if kind == "draft" else value
        _, rounds = spec_generate(d, b, prompt, k, sets, 1, inv_t, 5, hook=hook, separate=separate)
        q = [softmax(z * inv_t) for z in rounds[0]["q_logits"]]
        p = [softmax(z * inv_t) for z in rounds[0]["p_logits"]]
        w = np.prod([q[j][path[j]] for j in range(k)])          # probability of drafting this path
        for a in range(k + 1):
            acc = np.prod([min(1.0, p[j][path[j]] / q[j][path[j]]) for j in range(a)])
            if a < k:
                stop = 1.0 - min(1.0, p[a][path[a]] / q[a][path[a]])
                res = np.maximum(p[a] - q[a], 0.0)
                ylaw = res / res.sum() if res.sum() > 0 else p[a]
            else:
                stop, ylaw = 1.0, p[k]
            for y in range(V):
                e = tuple(path[:a]) + (y,)
                law[e] = law.get(e, 0.0) + w * acc * stop * ylaw[y]
    return law


@pytest.mark.parametrize("separate", [False, True])
@pytest.mark.parametrize("inv_t", [1.0, 1.0 / 0.7])
def test_round_law_exact_enumeration(separate, inv_t):
    """Losslessness of one round, exactly: the first k + 1 tokens, with the
    round's emitted tokens completed by the base's own law where the round
    stops early, follow the base model's autoregressive joint law (float64,
    every draft path enumerated).  The rule is lossless for any draft
    distribution, so this pins the round itself: which draft and base
    distributions meet in each decision, at which positions, across the
    prompt seam and both readings of the calibration pass."""
    import itertools
    V, k = 4, 3
    ds, dw, bs, bw = tiny_pair(V=V, draft_layers=4, base_layers=3, d=16, hq=2, hkv=1, hd=8, ffn=32)
    d, b = OracleModel.from_torch(ds, dw), OracleModel.from_torch(bs, bw)
    prompt = [1, 3, 0, 2]
    law = _round_law(d, b, prompt, k, FUZZY4, inv_t, separate)
    assert abs(sum(law.values()) - 1.0) < 1e-12

    cond = {}      # base law of the next token after prompt + prefix, by separate precise forwards

    def base_next(prefix):
        if prefix not in cond:
            seq = prompt + list(prefix)
            z = forward(b, KVCache(bs, 1, 16), 0, seq, range(len(seq)), logits="last")
            cond[prefix] = softmax(z * inv_t)
        return cond[prefix]

    worst = 0.0
    for s in itertools.product(range(V), repeat=k + 1):
        target = np.prod([base_next(s[:i])[s[i]] for i in range(k + 1)])
        got = 0.0
        for i in range(1, k + 2):
            pe = law.get(s[:i], 0.0)
            if pe:
                got += pe * np.prod([base_next(s[:j])[s[j]] for j in range(i, k + 1)])
        worst = max(worst, abs(got - target))
    assert worst < 1e-12, worst


def test_round_law_detects_a_planted_mistake(monkeypatch):
    """Power check: a verify pass that places the drafts one position late
    (an off-by-one in the round's positions) breaks the exact equality."""
    import itertools
    import oracle.decode as odec
    real = odec.forward

    def shifted(m, kv, bb, toks, pos, logits="all"):
        if logits == "all" and m is base_model[0]:
            pos = [p + 1 for p in pos]
        return real(m, kv, bb, toks, pos, logits=logits)
    base_model = [None]
    monkeypatch.setattr(odec, "forward", shifted)
    V, k = 4, 2
    ds, dw, bs, bw = tiny_pair(V=V, draft_layers=4, base_layers=3, d=16, hq=2, hkv=1, hd=8, ffn=32)
    d, b = OracleModel.from_torch(ds, dw), OracleModel.from_torch(bs, bw)
    base_model[0] = b
    prompt = [1, 3, 0, 2]
    law = _round_law(d, b, prompt, k, FUZZY4, 1.0, False)
    worst = 0.0
    for s in itertools.product(range(V), repeat=k + 1):
        pn = []
        for i in range(k + 1):
            seq = prompt + list(s[:i])
            pn.append(softmax(forward(b, KVCache(bs, 1, 16), 0, seq, range(len(seq)), logits="last")))
        target = np.prod([pn[i][s[i]] for i in range(k + 1)])
        got = sum(law.get(s[:i], 0.0) * np.prod([pn[j][s[j]] for j in range(i, k + 1)]) for i in range(1, k + 2))
        worst = max(worst, abs(got - target))
    assert worst > 1e-6, worst
