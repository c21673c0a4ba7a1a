"""Pins of the two oracle branches that serve the ablation and the diagnostic:
the loop without KV calibration, and the attention-input trace behind the
cosine-similarity diagnostic.

No-calibration ablation (rebuttal, reply on bonus calibration: without
calibration the fuzzy errors accumulate; the ablation keeps them): after the
acceptance, the accepted drafts keep the entries their fuzzy steps wrote and
only the emitted token y runs precisely, at the position after the accepted
drafts.  Cosine trace (rebuttal, reply on Table 3: similarity of the hidden
state a set feeds its attentions to the one a sequential pass would feed):
for every layer of a set, the set input h0 and the running state the layer
would read if its set ran in order.

Both are checked against states that a separate computation fixes (a
sequential forward of a truncated model, a fresh sequential prefill), and a
planted mistake in each branch must fail the same check.
"""
import numpy as np
import pytest

import oracle.decode as odec
import oracle.model as omod
from oracle.decode import spec_generate
from oracle.model import KVCache, OracleModel, forward, forward_hidden, fuzzy_step_hidden
from synth import make_weights, tiny_shape
from helpers import tiny_pair

CAP = 64
PROMPT = [3, 1, 4, 1, 5, 9]
SETS5 = [[0], [1, 2, 3], [4]]          # a real layer-parallel set


def _pair(draft_layers=5):
    ds, dw, bs, bw = tiny_pair(V=32, draft_layers=draft_layers, draft_noise=None)
    return OracleModel.from_torch(ds, dw), OracleModel.from_torch(bs, bw)


def _prefill(m, toks, cap=CAP):
    c = KVCache(m.shape, 1, cap)
    forward(m, c, 0, toks, range(len(toks)), logits=None)
    return c


def _run_with_snapshots(d, b, sets, calibrate, k=3, new=14, inv_temp=1.0, seed=5):
    """Run the loop and snapshot the draft KV (a) right after each round's
    verification (hook 'y': drafting done, calibration not yet) and (b) at
    the start of the next round (hook 'draft' of its first slot)."""
    dkv, bkv = KVCache(d.shape, 1, CAP), KVCache(b.shape, 1, CAP)
    after_verify, next_start = {}, {}

    def hook(kind, key, value, margin):
        if kind == "y":
            after_verify[key[0]] = (dkv.k.copy(), dkv.v.copy())
        elif kind == "draft" and key[1] == 1:
            next_start[key[0]] = (dkv.k.copy(), dkv.v.copy())
        return value

    toks, rounds = spec_generate(d, b, PROMPT, k, sets, new, inv_temp, seed, caches=(dkv, bkv), capacity=CAP,
                                 calibrate=calibrate, hook=hook)
    return toks, rounds, after_verify, next_start, dkv


def _check_no_calibration_round_invariants(d, b, sets, k=3):
    """For every round r that is followed by another: the entries of the
    accepted drafts that a fuzzy step fed (t+1 .. t+min(a, k-1)) are the ones
    those steps wrote (unchanged since the verification); the remaining
    emitted tokens (y, and d_k when all k were accepted) have the entries of a
    precise forward over the cache as it stood; every other position is
    untouched."""
    toks, rounds, av, ns, _ = _run_with_snapshots(d, b, sets, calibrate=False, k=k)
    assert len(rounds) >= 3
    n_fuzzy = n_full = 0
    for r, rd in enumerate(rounds[:-1]):
        t, a, y = rd["t"], rd["a"], rd["y"]
        emitted = rd["drafts"][:a] + [y]
        j0 = min(a, k - 1)
        k_av, v_av = av[r]
        k_ns, v_ns = ns[r + 1]
        np.testing.assert_array_equal(k_ns[:, :, :, t + 1:t + 1 + j0], k_av[:, :, :, t + 1:t + 1 + j0])
        np.testing.assert_array_equal(v_ns[:, :, :, t + 1:t + 1 + j0], v_av[:, :, :, t + 1:t + 1 + j0])
        n_fuzzy += j0
        n_full += a == k
        ref = KVCache.__new__(KVCache)
        ref.k, ref.v, ref.capacity = k_av.copy(), v_av.copy(), CAP
        forward(d, ref, 0, emitted[j0:], range(t + 1 + j0, t + a + 2), logits=None)
        np.testing.assert_array_equal(k_ns[:, :, :, t + 1 + j0:t + a + 2], ref.k[:, :, :, t + 1 + j0:t + a + 2])
        np.testing.assert_array_equal(v_ns[:, :, :, t + 1 + j0:t + a + 2], ref.v[:, :, :, t + 1 + j0:t + a + 2])
        keep = np.ones(CAP, bool)
        keep[t + 1:t + a + 2] = False
        np.testing.assert_array_equal(k_ns[:, :, :, keep], k_av[:, :, :, keep])
        np.testing.assert_array_equal(v_ns[:, :, :, keep], v_av[:, :, :, keep])
    return n_fuzzy, n_full


@pytest.mark.parametrize("draft_noise", [None, 0.02])
def test_no_calibration_keeps_fuzzy_entries_and_runs_the_rest_precisely(draft_noise):
    ds, dw, bs, bw = tiny_pair(V=32, draft_layers=5 if draft_noise is None else 3, draft_noise=draft_noise)
    d, b = OracleModel.from_torch(ds, dw), OracleModel.from_torch(bs, bw)
    sets = SETS5 if draft_noise is None else [[0, 1], [2]]
    n_fuzzy, n_full = _check_no_calibration_round_invariants(d, b, sets)
    assert n_fuzzy > 0   # accepted drafts kept their fuzzy entries
    if draft_noise is not None:
        assert n_full > 0   # rounds with every draft accepted (d_k has no fuzzy entry)


def test_no_calibration_leaves_fuzzy_entries_that_calibration_replaces():
    """With a real set, the kept entries are not the precise ones (which the
    calibrated loop restores): the ablation really differs."""
    d, b = _pair()
    toks, rounds, _, _, dkv = _run_with_snapshots(d, b, SETS5, calibrate=False)
    seq = PROMPT + toks
    a_tot = sum(r["a"] for r in rounds[:-1])
    assert a_tot > 0
    last = rounds[-1]["t"]          # every position < last is committed
    ref = _prefill(d, seq[:last])
    assert not np.allclose(dkv.k[:, :, :, :last], ref.k[:, :, :, :last], rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("inv_temp", [0.0, 1.0])
def test_no_calibration_with_singleton_plan_is_the_precise_loop(inv_temp):
    """Without layer-parallel sets every fuzzy entry is already precise, so
    skipping calibration changes nothing: the tokens equal the calibrated
    loop's and the draft KV of every committed position equals a fresh
    sequential prefill of the committed tokens (this fixes both the position
    and the token the branch runs)."""
    d, b = _pair()
    singles = [[l] for l in range(5)]
    t1, r1, _, _, dkv = _run_with_snapshots(d, b, singles, calibrate=False, inv_temp=inv_temp)
    t2, _, _, _, _ = _run_with_snapshots(d, b, singles, calibrate=True, inv_temp=inv_temp)
    assert t1 == t2
    seq = PROMPT + t1
    last = r1[-1]["t"] + 1          # positions up to the last pending token
    ref = _prefill(d, seq[:last])
    np.testing.assert_allclose(dkv.k[:, :, :, :last], ref.k[:, :, :, :last], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dkv.v[:, :, :, :last], ref.v[:, :, :, :last], rtol=1e-12, atol=1e-14)


def _shift_single_token_forward(monkeypatch):
    """Planted mistake: the precise forward of the no-calibration branch (the
    only forward of at most two tokens with last-row logits when the prompt
    is longer) runs one position early."""
    real = odec.forward

    def shifted(m, kv, bb, toks, pos, logits="all"):
        pos = list(pos)
        if len(toks) <= 2 and logits == "last":
            pos = [p - 1 for p in pos]
        return real(m, kv, bb, toks, pos, logits=logits)
    monkeypatch.setattr(odec, "forward", shifted)


def test_no_calibration_pins_detect_a_wrong_position(monkeypatch):
    _shift_single_token_forward(monkeypatch)
    d, b = _pair()
    with pytest.raises(AssertionError):
        _check_no_calibration_round_invariants(d, b, SETS5)
    singles = [[l] for l in range(5)]
    t1, r1, _, _, dkv = _run_with_snapshots(d, b, singles, calibrate=False)
    seq = PROMPT + t1
    last = r1[-1]["t"] + 1
    ref = _prefill(d, seq[:last])
    assert not np.allclose(dkv.k[:, :, :, :last], ref.k[:, :, :, :last], rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------ cosine trace
def _truncated(m: OracleModel, n: int) -> OracleModel:
    """The first n layers of m as a model of its own (same weights)."""
    w = dict(m.w)
    for key in ("attn_norm", "wqkv", "bqkv", "wo", "ffn_norm", "w_gate_up", "w_down"):
        if w.get(key) is not None:
            w[key] = w[key][:n]
    return OracleModel(m.shape.replace(n_layers=n), w, m.bf16)


def _precise_state(m, n, toks, pos, tok):
    """Hidden state after the first n layers of a precise forward of `tok` at
    `pos` over a sequential prefill of toks (n = 0: the embedding)."""
    if n == 0:
        return m.w["embed"][tok][None].copy()
    mt = _truncated(m, n)
    c = _prefill(mt, toks)
    return forward_hidden(mt, c, 0, [tok], [pos])


def _trace(m, toks, tok, sets, step=fuzzy_step_hidden):
    c = _prefill(m, toks)
    tr = []
    step(m, c, 0, tok, len(toks), sets, trace=tr)
    return {l: (h0, h) for (l, h0, h) in tr}


def _check_trace(m, sets, toks=(5, 9, 1, 3), tok=17, dead_first=False, step=fuzzy_step_hidden):
    """Every member of a set records the same set input, and the first member
    records it as its running state too.  Up to the first layer-parallel set
    (all earlier sets singletons): set input h0 = precise state before the
    set's first layer, and the traced
    state of the second member = precise state after the first member (the
    first member's attention reads h0 in both runs).  With the first member
    dead (W_o, W_down zero) the third member's traced state = precise state
    after the second member."""
    toks = list(toks)
    tr = _trace(m, toks, tok, sets, step)
    precise_so_far = True      # every set before this one was a singleton
    for s in sets:
        l0 = s[0]
        for l in s:
            np.testing.assert_array_equal(tr[l][0], tr[l0][0])
        np.testing.assert_array_equal(tr[l0][1], tr[l0][0])
        if not precise_so_far:
            continue
        precise_so_far = len(s) == 1
        h0 = _precise_state(m, l0, toks, len(toks), tok)
        np.testing.assert_allclose(tr[l0][0], h0, rtol=1e-12, atol=1e-12)
        if len(s) >= 2:
            np.testing.assert_allclose(tr[s[1]][1], _precise_state(m, l0 + 1, toks, len(toks), tok),
                                       rtol=1e-12, atol=1e-12)
        if dead_first and len(s) >= 3:
            np.testing.assert_allclose(tr[s[2]][1], _precise_state(m, l0 + 2, toks, len(toks), tok),
                                       rtol=1e-12, atol=1e-12)


def _model(L=6, zero=None):
    sh = tiny_shape(L, 32, 4, 2, 8, 64, 40)
    return OracleModel.from_torch(sh, make_weights(sh, 31, gain_std=0.1, std=0.08, zero_mask=zero))


@pytest.mark.parametrize("sets", [[[0], [1, 2], [3, 4], [5]], [[0], [1, 2, 3, 4], [5]],
                                  [[0], [1], [2], [3, 4], [5]]])
def test_cosine_trace_matches_precise_states(sets):
    _check_trace(_model(), sets)


def test_cosine_trace_third_member_with_dead_first_member():
    m = _model(zero={"wo": [1], "w_down": [1]})
    _check_trace(m, [[0], [1, 2, 3, 4], [5]], dead_first=True)


def test_cosine_trace_singleton_plan_has_unit_cosine():
    m = _model()
    tr = _trace(m, [5, 9, 1, 3], 17, [[l] for l in range(6)])
    for l, (h0, h) in tr.items():
        np.testing.assert_array_equal(h0, h)
        assert abs(float(h0[0] @ h[0]) / float(np.linalg.norm(h0) * np.linalg.norm(h)) - 1.0) < 1e-14


def test_cosine_trace_pins_detect_a_post_add_trace(monkeypatch):
    """Planted mistake: the traced running state already contains the
    member's own attention output (recorded after h += a_i)."""
    last_a = {}
    real_attn = omod.attn_part

    def attn(m, cache, l, b, h_in, positions):
        a = real_attn(m, cache, l, b, h_in, positions)
        last_a[l] = a
        return a
    monkeypatch.setattr(omod, "attn_part", attn)

    class PostAdd(list):
        def __init__(self, target):
            super().__init__()
            self.target = target

        def append(self, item):
            l, h0, h = item
            self.target.append((l, h0, h + last_a[l]))

    def mutant(m, c, b, tok, pos, sets, trace=None):
        return fuzzy_step_hidden(m, c, b, tok, pos, sets, trace=PostAdd(trace))

    with pytest.raises(AssertionError):
        _check_trace(_model(), [[0], [1, 2], [3, 4], [5]], step=mutant)
