"""Statistical pins: the accept / resample rule and the whole round loop keep
the base distribution (EasySpec abstract: the original distributions of the
base model are preserved), checked by closed form and by chi-square tests on
seeded trials."""
import numpy as np
import pytest
from scipy import stats

from oracle import philox, sampling
from oracle.decode import spec_generate
from oracle.model import KVCache, OracleModel, forward
from oracle.plan import default_group_plan
from oracle.sampling import accept_law, accept_resample, accept_resample_batch, sample_from_logits, softmax
from helpers import tiny_pair

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
    sets = default_group_plan(3, 2)
    n = 2500
    counts = np.zeros((V, V), dtype=np.int64)
    acc = 0
    for s in range(n):
        toks, rounds = spec_generate(d, b, prompt, 2, sets, 2, 1.0, 1000 + s)
        counts[toks[0], toks[1]] += 1
        acc += rounds[0]["a"]
    assert 0.2 * n < acc < 1.8 * n          # both accept and reject paths are exercised
    assert _chi2_p(counts.ravel(), joint.ravel()) > P_MIN
