"""GPU parity of the forward entry points (draft group step, calibration,
verify) against the oracle on the same seeded weights and tokens."""
import numpy as np
import pytest
import torch

from oracle import philox
from oracle.model import KVCache, OracleModel, forward, fuzzy_step, MLP_PARALLEL, MLP_SEQUENTIAL
from oracle.plan import default_group_plan, offsets_to_sets, plan_offsets
from oracle.sampling import sample_from_logits
from synth import make_weights, tiny_shape
from synth.configs import BF16, F32
from gpu_common import MARGIN, TOL_BF16, TOL_F32, exclusion, i32, rel_linf, say, to_dev, ws

pytestmark = pytest.mark.gpu

SHAPES = {
    # name: (shape, tolerance)
    "c1-draft-f32": (tiny_shape(2, 64, 4, 4, 16, 256, 256), TOL_F32),
    "gqa-bias-f32": (tiny_shape(4, 128, 8, 2, 16, 320, 512, qkv_bias=True), TOL_F32),
    "gqa-bf16": (tiny_shape(5, 256, 8, 2, 32, 512, 1024, dtype=BF16, rope_theta=5e5), TOL_BF16),
    "hd64-bias-bf16": (tiny_shape(4, 256, 4, 1, 64, 384, 2048, dtype=BF16, qkv_bias=True, rms_eps=1e-6,
                                  rope_theta=1e6), TOL_BF16),
    "hd128-bf16": (tiny_shape(3, 512, 8, 2, 128, 1024, 1000, dtype=BF16), TOL_BF16),
}


def _setup(name, B, P, cap=96, seed=5):
    shape, tol = SHAPES[name]
    w = make_weights(shape, seed, gain_std=0.1, std=0.05)
    om = OracleModel.from_torch(shape, w)
    from layer_speculative_decoding_amd import api
    gm = api.SpecModel(shape, to_dev(w))
    gkv = api.KVCache(shape, B, cap)
    okv = KVCache(shape, B, cap)
    rng = np.random.default_rng(seed + 17)
    prompts = rng.integers(0, shape.vocab, size=(B, P)).astype(np.int32)
    return shape, tol, om, gm, gkv, okv, prompts


def _kv_rel(gkv, okv, upto):
    k = gkv.k.float().cpu().numpy()[:, :, :, :upto]
    v = gkv.v.float().cpu().numpy()[:, :, :, :upto]
    return rel_linf(k, okv.k[:, :, :, :upto]), rel_linf(v, okv.v[:, :, :, :upto])


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("inv_temp", [0.0, 1.0])
def test_calibrate_prefill_matches_oracle(name, inv_temp):
    from layer_speculative_decoding_amd import api
    B, P = 2, 37
    shape, tol, om, gm, gkv, okv, prompts = _setup(name, B, P)
    say(f"calibrate prefill {name} B={B} P={P} invT={inv_temp}")
    w = ws(api.spec_workspace_bytes(gm, B, P, 1))
    logits = torch.zeros(B, shape.vocab, device="cuda")
    tok = torch.zeros(B, dtype=torch.int32, device="cuda")
    api.spec_calibrate_kv(gm, gkv, B, i32(prompts), i32([0] * B), None, P, P - 1, inv_temp, 99, logits,
                          shape.vocab, tok, 1, w)
    torch.cuda.synchronize()
    zg, tg = logits.cpu().numpy(), tok.cpu().numpy()
    for b in range(B):
        zo = forward(om, okv, b, prompts[b], range(P), logits="last")
        err = rel_linf(zg[b], zo)
        say(f"  b={b} logits rel {err:.2e}")
        assert err < tol
        t_or, mg = sample_from_logits(zo, inv_temp, 99, b, P, philox.DRAFT)
        if mg >= exclusion(zg[b], zo, inv_temp):
            assert tg[b] == t_or
    ek, ev = _kv_rel(gkv, okv, P)
    say(f"  kv rel {ek:.2e} {ev:.2e}")
    assert ek < tol and ev < tol


@pytest.mark.parametrize("name", ["c1-draft-f32", "gqa-bias-f32", "gqa-bf16", "hd64-bias-bf16", "hd128-bf16"])
def test_calibrate_ragged_matches_oracle(name):
    """n_tokens differ per sequence (accepted-prefix lengths); rows past
    n_tokens must not touch the cache."""
    from layer_speculative_decoding_amd import api
    B, P, M = 3, 20, 6
    shape, tol, om, gm, gkv, okv, prompts = _setup(name, B, P + M)
    say(f"calibrate ragged {name}")
    w = ws(api.spec_workspace_bytes(gm, B, P + M, 1))
    tok = torch.zeros(B, dtype=torch.int32, device="cuda")
    api.spec_calibrate_kv(gm, gkv, B, i32(prompts[:, :P]), i32([0] * B), None, P, P - 1, 0.0, 1, None, 0, tok, 1,
                          w)
    for b in range(B):
        forward(om, okv, b, prompts[b, :P], range(P), logits=None)
    ntok = np.array([1, 4, 6], dtype=np.int32)
    start = np.array([P, P, P], dtype=np.int32)
    logits = torch.zeros(B, shape.vocab, device="cuda")
    before = gkv.k.float().cpu().numpy().copy()
    api.spec_calibrate_kv(gm, gkv, B, i32(prompts[:, P:]), i32(start), i32(ntok), M, P + M - 1, 1.0, 7, logits,
                          shape.vocab, tok, 1, w)
    torch.cuda.synchronize()
    zg, tg = logits.cpu().numpy(), tok.cpu().numpy()
    after = gkv.k.float().cpu().numpy()
    for b in range(B):
        zo = forward(om, okv, b, prompts[b, P:P + ntok[b]], range(P, P + ntok[b]), logits="last")
        err = rel_linf(zg[b], zo)
        say(f"  b={b} n={ntok[b]} logits rel {err:.2e}")
        assert err < tol
        t_or, mg = sample_from_logits(zo, 1.0, 7, b, P + ntok[b], philox.DRAFT)
        if mg >= exclusion(zg[b], zo, 1.0):
            assert tg[b] == t_or
        # positions beyond n_tokens untouched
        np.testing.assert_array_equal(after[:, b, :, P + ntok[b]:], before[:, b, :, P + ntok[b]:])
    ek, _ = _kv_rel(gkv, okv, P + 1)
    assert ek < tol


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("m", [1, 5, 9, 28])
def test_verify_matches_oracle(name, m):
    from layer_speculative_decoding_amd import api
    B, P = 2, 30
    shape, tol, om, gm, gkv, okv, prompts = _setup(name, B, P + m, cap=P + m + 4)
    say(f"verify {name} m={m}")
    w = ws(api.spec_workspace_bytes(gm, B, max(P, m), 1))
    api.spec_verify_forward(gm, gkv, B, i32(prompts[:, :P]), i32([0, 0]), P, P - 1, None, w)
    for b in range(B):
        forward(om, okv, b, prompts[b, :P], range(P), logits=None)
    vt = prompts[:, P:P + m].copy()
    logits = torch.zeros(B, m, shape.vocab, device="cuda")
    st = np.array([P, P - 2], dtype=np.int32)       # sequence 1 overwrites two positions
    api.spec_verify_forward(gm, gkv, B, i32(vt), i32(st), m, int(st.max()) + m - 1, logits, w)
    torch.cuda.synchronize()
    zg = logits.cpu().numpy()
    for b in range(B):
        zo = forward(om, okv, b, vt[b], range(st[b], st[b] + m), logits="all")
        err = rel_linf(zg[b], zo)
        say(f"  b={b} logits rel {err:.2e}")
        assert err < tol
        srt = np.sort(zo, axis=1)
        ok = (srt[:, -1] - srt[:, -2]) >= exclusion(zg[b], zo, 0.0)
        np.testing.assert_array_equal(np.argmax(zg[b], 1)[ok], np.argmax(zo, 1)[ok])



@pytest.mark.parametrize("name", ["hd64-bias-bf16", "hd128-bf16"])
def test_verify_split_keys_ragged_batch(name):
    """Verify rows of three sequences at a context long enough for several
    key splits, with ragged start positions.  For hd64-bias-bf16 the
    attention launch has twelve (kv head, sequence, split) groups of two
    query blocks, so its workgroup renumbering covers eight groups and leaves
    a tail of four in plain order; hd128-bf16 has 24 groups (no tail)."""
    from layer_speculative_decoding_amd import api
    B, P, m = 3, 190, 6
    shape, tol, om, gm, gkv, okv, prompts = _setup(name, B, P + m, cap=P + m + 4)
    say(f"verify split keys {name} B={B} P={P} m={m}")
    w = ws(api.spec_workspace_bytes(gm, B, max(P, m), 1))
    api.spec_verify_forward(gm, gkv, B, i32(prompts[:, :P]), i32([0] * B), P, P - 1, None, w)
    for b in range(B):
        forward(om, okv, b, prompts[b, :P], range(P), logits=None)
    vt = prompts[:, P:P + m].copy()
    logits = torch.zeros(B, m, shape.vocab, device="cuda")
    st = np.array([P, P - 3, P - 7], dtype=np.int32)
    api.spec_verify_forward(gm, gkv, B, i32(vt), i32(st), m, int(st.max()) + m - 1, logits, w)
    torch.cuda.synchronize()
    zg = logits.cpu().numpy()
    for b in range(B):
        zo = forward(om, okv, b, vt[b], range(st[b], st[b] + m), logits="all")
        err = rel_linf(zg[b], zo)
        say(f"  b={b} start {st[b]} logits rel {err:.2e}")
        assert err < tol
        srt = np.sort(zo, axis=1)
        ok = (srt[:, -1] - srt[:, -2]) >= exclusion(zg[b], zo, 0.0)
        np.testing.assert_array_equal(np.argmax(zg[b], 1)[ok], np.argmax(zo, 1)[ok])


PLANS = {
    "c1-draft-f32": [[[0], [1]], [[0, 1]]],
    "gqa-bias-f32": [[[0], [1, 2], [3]], [[0, 1, 2, 3]]],
    "gqa-bf16": [default_group_plan(5, 2), default_group_plan(5, 4), [[l] for l in range(5)]],
    "hd64-bias-bf16": [default_group_plan(4, 3)],
    "hd128-bf16": [[[0], [1, 2]]],
}


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("mlp", [MLP_SEQUENTIAL, MLP_PARALLEL])
@pytest.mark.parametrize("inv_temp", [0.0, 1.0])
def test_draft_group_step_matches_oracle(name, mlp, inv_temp):
    from layer_speculative_decoding_amd import api
    B, P = 3, 23
    shape, tol, om, gm, gkv, okv, prompts = _setup(name, B, P + 4)
    for sets in PLANS[name]:
        offs = plan_offsets(sets)
        G = max(len(s) for s in sets)
        say(f"draft step {name} plan={offs} mlp={mlp} invT={inv_temp}")
        gkv.k.zero_(); gkv.v.zero_()
        okv = KVCache(shape, B, gkv.capacity)
        w = ws(max(api.spec_workspace_bytes(gm, B, P, 1), api.spec_workspace_bytes(gm, B, 1, G)))
        tok = torch.zeros(B, dtype=torch.int32, device="cuda")
        lens = np.array([P, P - 5, P - 11], dtype=np.int32)
        for b in range(B):
            forward(om, okv, b, prompts[b, :lens[b]], range(lens[b]), logits=None)
        # batched ragged prefill through calibrate (n_tokens per sequence)
        api.spec_calibrate_kv(gm, gkv, B, i32(prompts[:, :P]), i32([0] * B), i32(lens), P, P - 1, 0.0, 0, None,
                              0, tok, 1, w)
        cur = prompts[:, P].copy()
        pos = lens.copy()
        for step in range(3):
            logits = torch.zeros(B, shape.vocab, device="cuda")
            out = torch.zeros(B, dtype=torch.int32, device="cuda")
            api.spec_draft_group_step(gm, gkv, offs, mlp, B, i32(cur), 1, i32(pos), int(pos.max()), inv_temp, 31,
                                      logits, shape.vocab, out, 1, w)
            torch.cuda.synchronize()
            zg, tg = logits.cpu().numpy(), out.cpu().numpy()
            nxt = np.zeros(B, dtype=np.int32)
            for b in range(B):
                zo = fuzzy_step(om, okv, b, int(cur[b]), int(pos[b]), sets, mlp)
                err = rel_linf(zg[b], zo)
                assert err < tol, (step, b, err)
                t_or, mg = sample_from_logits(zo, inv_temp, 31, b, int(pos[b]) + 1, philox.DRAFT)
                if mg >= exclusion(zg[b], zo, inv_temp):
                    assert tg[b] == t_or, (step, b)
                nxt[b] = tg[b]
            say(f"  step {step}: logits rel (last row) {err:.2e}")
            cur, pos = nxt, pos + 1
        ek, ev = _kv_rel(gkv, okv, int(pos.max()))
        assert ek < tol and ev < tol



@pytest.mark.parametrize("name", ["gqa-bf16", "hd64-bias-bf16", "hd128-bf16"])
@pytest.mark.parametrize("tile", [None, "64 3", "128 1"])
def test_prompt_prefill_matches_oracle(name, tile, monkeypatch):
    """Prompt-length row counts (several 128-row activation tiles and a ragged
    last tile) through the tiled matrix-core products: base-style verify
    prefill with every row's logits, and draft-style calibration prefill with
    ragged prompt lengths.  `tile` forces the tile width and the number of K
    slices (3 slices over 4..16 K steps: ragged last slice)."""
    from layer_speculative_decoding_amd import api
    if tile is not None:
        monkeypatch.setenv("SPEC_TILE", tile)
    B, P = 2, 150
    shape, tol, om, gm, gkv, okv, prompts = _setup(name, B, P, cap=P + 8)
    say(f"prompt prefill {name} B={B} P={P} tile={tile}")
    w = ws(api.spec_workspace_bytes(gm, B, P, 1))
    logits = torch.zeros(B, P, shape.vocab, device="cuda")
    api.spec_verify_forward(gm, gkv, B, i32(prompts), i32([0, 0]), P, P - 1, logits, w)
    torch.cuda.synchronize()
    zg = logits.cpu().numpy()
    for b in range(B):
        zo = forward(om, okv, b, prompts[b], range(P), logits="all")
        err = rel_linf(zg[b], zo)
        say(f"  verify b={b} logits rel {err:.2e}")
        assert err < tol
    ek, ev = _kv_rel(gkv, okv, P)
    say(f"  kv rel {ek:.2e} {ev:.2e}")
    assert ek < tol and ev < tol

    # calibration prefill, ragged: sequence 1 covers P - 41 tokens
    gkv.k.zero_(); gkv.v.zero_()
    okv = KVCache(shape, B, gkv.capacity)
    lens = np.array([P, P - 41], dtype=np.int32)
    last = torch.zeros(B, shape.vocab, device="cuda")
    tok = torch.zeros(B, dtype=torch.int32, device="cuda")
    api.spec_calibrate_kv(gm, gkv, B, i32(prompts), i32([0, 0]), i32(lens), P, P - 1, 1.0, 5, last, shape.vocab,
                          tok, 1, w)
    torch.cuda.synchronize()
    zg, tg = last.cpu().numpy(), tok.cpu().numpy()
    for b in range(B):
        zo = forward(om, okv, b, prompts[b, :lens[b]], range(lens[b]), logits="last")
        err = rel_linf(zg[b], zo)
        say(f"  calibrate b={b} n={lens[b]} logits rel {err:.2e}")
        assert err < tol
        t_or, mg = sample_from_logits(zo, 1.0, 5, b, int(lens[b]), philox.DRAFT)
        if mg >= exclusion(zg[b], zo, 1.0):
            assert tg[b] == t_or
    k = gkv.k.float().cpu().numpy()
    assert not np.any(k[:, 1, :, lens[1]:])      # rows past n_tokens leave the cache alone
    ek, ev = _kv_rel(gkv, okv, int(lens[0]))
    assert ek < tol and ev < tol


@pytest.mark.parametrize("hq,hkv,hd,tight", [(4, 4, 64, False), (8, 4, 128, False), (14, 2, 64, False),
                                             (16, 2, 128, False), (16, 1, 64, False), (8, 4, 128, True),
                                             (14, 2, 64, True)])
def test_prompt_attention_group_sizes(hq, hkv, hd, tight):
    """Prompt-length prefills through the flash-style prompt attention (one
    workgroup per 16 * (8 / G) rows of one kv head, two 16-row blocks per
    wave; G = 16 falls back to the decode kernel) at q heads per kv head
    G = 1, 2, 7, 8, 16, ragged last row tile, a ragged second sequence;
    tight: the KV capacity equals the prompt length (the last row's keys end
    at the cache's last slot)."""
    from layer_speculative_decoding_amd import api
    shape = tiny_shape(2, hq * hd // 2, hq, hkv, hd, 256, 512, dtype=BF16)
    w = make_weights(shape, 11, gain_std=0.1, std=0.05)
    om = OracleModel.from_torch(shape, w)
    gm = api.SpecModel(shape, to_dev(w))
    B, P = 2, 83
    cap = P if tight else P + 4
    gkv = api.KVCache(shape, B, cap)
    okv = KVCache(shape, B, cap)
    prompts = np.random.default_rng(3).integers(0, shape.vocab, size=(B, P)).astype(np.int32)
    say(f"prompt attention hq={hq} hkv={hkv} hd={hd} B={B} P={P} capacity={cap}")
    wsb = ws(api.spec_workspace_bytes(gm, B, P, 1))
    lens = np.array([P, P - 30], dtype=np.int32)
    last = torch.zeros(B, shape.vocab, device="cuda")
    tok = torch.zeros(B, dtype=torch.int32, device="cuda")
    api.spec_calibrate_kv(gm, gkv, B, i32(prompts), i32([0, 0]), i32(lens), P, P - 1, 0.0, 5, last, shape.vocab,
                          tok, 1, wsb)
    torch.cuda.synchronize()
    zg = last.cpu().numpy()
    for b in range(B):
        zo = forward(om, okv, b, prompts[b, :lens[b]], range(lens[b]), logits="last")
        err = rel_linf(zg[b], zo)
        say(f"  b={b} n={lens[b]} logits rel {err:.2e}")
        assert err < TOL_BF16
    ek, ev = _kv_rel(gkv, okv, int(lens[1]))
    assert ek < TOL_BF16 and ev < TOL_BF16


@pytest.mark.parametrize("name", list(SHAPES))
def test_attention_input_cosine_matches_oracle(name):
    """The cosine diagnostic of the fuzzy inputs against the oracle's trace of
    the same layer-parallel step (sequential MLPs): per layer, cos(h0, h_l)."""
    from layer_speculative_decoding_amd import api
    from oracle.model import fuzzy_step_hidden
    B, P = 2, 19
    shape, tol, om, gm, gkv, okv, prompts = _setup(name, B, P + 2)
    L = shape.n_layers
    for sets in PLANS[name]:
        offs = plan_offsets(sets)
        G = max(len(s) for s in sets)
        say(f"cosine {name} plan={offs}")
        gkv.k.zero_(); gkv.v.zero_()
        okv = KVCache(shape, B, gkv.capacity)
        w = ws(max(api.spec_workspace_bytes(gm, B, P, 1), api.spec_workspace_bytes(gm, B, 1, G)))
        tok = torch.zeros(B, dtype=torch.int32, device="cuda")
        api.spec_calibrate_kv(gm, gkv, B, i32(prompts[:, :P]), i32([0] * B), None, P, P - 1, 0.0, 0, None, 0, tok,
                              1, w)
        for b in range(B):
            forward(om, okv, b, prompts[b, :P], range(P), logits=None)
        cur = prompts[:, P].copy()
        pos = np.full(B, P, dtype=np.int32)
        cos = torch.full((B, L + 3), -7.0, device="cuda")
        api.spec_draft_attention_cosine(gm, gkv, offs, B, i32(cur), 1, i32(pos), int(pos.max()), cos, L + 3, w)
        torch.cuda.synchronize()
        cg = cos.cpu().numpy()
        assert np.all(cg[:, L:] == -7.0)                 # nothing past n_layers
        for b in range(B):
            tr = []
            fuzzy_step_hidden(om, okv, b, int(cur[b]), int(pos[b]), sets, MLP_SEQUENTIAL, trace=tr)
            co = np.zeros(L)
            for l, h0, h in tr:
                x, y = h0.reshape(-1), h.reshape(-1)
                co[l] = float(np.dot(x, y) / (np.linalg.norm(x) * np.linalg.norm(y)))
            err = float(np.max(np.abs(cg[b, :L] - co)))
            say(f"  b={b} cos {np.round(co, 4).tolist()} max |gpu - oracle| {err:.1e}")
            assert err < (1e-5 if tol == TOL_F32 else 1e-2)
            for s in sets:                              # the first member reads exactly h0
                assert abs(cg[b, s[0]] - 1.0) < 1e-5


@pytest.mark.parametrize("name", ["gqa-bias-f32", "hd64-bias-bf16", "hd128-bf16"])
def test_kv_filled_to_capacity(name):
    """Every forward entry point at the last KV slot: a verify whose rows of
    sequence 0 end at position capacity - 1 (several key splits, the last
    one ragged: the capacity, 301, is no multiple of a key block or chunk),
    a layer-parallel draft step at that position, and a ragged calibration
    ending there.  The oracle takes the same calls, so the whole KV cache is
    compared at the end."""
    from layer_speculative_decoding_amd import api
    B, m, cap = 2, 6, 301
    P = cap - m
    shape, tol, om, gm, gkv, okv, prompts = _setup(name, B, cap + 1, cap=cap)
    sets = PLANS[name][0]
    offs = plan_offsets(sets)
    G = max(len(s) for s in sets)
    say(f"capacity edge {name} cap={cap} plan={offs}")
    w = ws(max(api.spec_workspace_bytes(gm, B, P, 1), api.spec_workspace_bytes(gm, B, 1, G)))

    api.spec_verify_forward(gm, gkv, B, i32(prompts[:, :P]), i32([0] * B), P, P - 1, None, w)
    for b in range(B):
        forward(om, okv, b, prompts[b, :P], range(P), logits=None)

    # verify: rows P .. cap - 1 (sequence 0) and P - 2 .. cap - 3 (sequence 1)
    vt = prompts[:, P:P + m].copy()
    st = np.array([P, P - 2], dtype=np.int32)
    logits = torch.zeros(B, m, shape.vocab, device="cuda")
    api.spec_verify_forward(gm, gkv, B, i32(vt), i32(st), m, cap - 1, logits, w)
    torch.cuda.synchronize()
    zg = logits.cpu().numpy()
    for b in range(B):
        zo = forward(om, okv, b, vt[b], range(st[b], st[b] + m), logits="all")
        err = rel_linf(zg[b], zo)
        say(f"  verify b={b} start {st[b]} logits rel {err:.2e}")
        assert err < tol

    # draft step writing fuzzy K/V at the last slot of both sequences
    cur = prompts[:, cap].copy()
    pos = np.array([cap - 1, cap - 1], dtype=np.int32)
    dl = torch.zeros(B, shape.vocab, device="cuda")
    out = torch.zeros(B, dtype=torch.int32, device="cuda")
    api.spec_draft_group_step(gm, gkv, offs, MLP_SEQUENTIAL, B, i32(cur), 1, i32(pos), cap - 1, 1.0, 77,
                              dl, shape.vocab, out, 1, w)
    torch.cuda.synchronize()
    zg, tg = dl.cpu().numpy(), out.cpu().numpy()
    for b in range(B):
        zo = fuzzy_step(om, okv, b, int(cur[b]), int(pos[b]), sets, MLP_SEQUENTIAL)
        err = rel_linf(zg[b], zo)
        say(f"  draft step b={b} logits rel {err:.2e}")
        assert err < tol
        t_or, mg = sample_from_logits(zo, 1.0, 77, b, int(pos[b]) + 1, philox.DRAFT)
        if mg >= exclusion(zg[b], zo, 1.0):
            assert tg[b] == t_or

    # ragged calibration: sequence 0 rewrites the last m slots, sequence 1
    # m - 2 slots ending two before the last
    ct = prompts[:, P - 1:P - 1 + m].copy()
    cs = np.array([cap - m, cap - m - 2], dtype=np.int32)
    cn = np.array([m, m - 2], dtype=np.int32)
    ll = torch.zeros(B, shape.vocab, device="cuda")
    tok = torch.zeros(B, dtype=torch.int32, device="cuda")
    api.spec_calibrate_kv(gm, gkv, B, i32(ct), i32(cs), i32(cn), m, cap - 1, 0.0, 0, ll, shape.vocab, tok, 1, w)
    torch.cuda.synchronize()
    zg = ll.cpu().numpy()
    for b in range(B):
        zo = forward(om, okv, b, ct[b, :cn[b]], range(cs[b], cs[b] + cn[b]), logits="last")
        err = rel_linf(zg[b], zo)
        say(f"  calibrate b={b} rows {cs[b]}..{cs[b] + cn[b] - 1} last logits rel {err:.2e}")
        assert err < tol
    ek, ev = _kv_rel(gkv, okv, cap)
    say(f"  KV rel over all {cap} slots: k {ek:.2e} v {ev:.2e}")
    assert ek < tol and ev < tol
