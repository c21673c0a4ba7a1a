"""GPU parity at the workloads' full per-layer shapes, in the launch
configurations the benchmark times.

The KV cache of the context is an input of every entry point, so instead of
an (expensive) oracle prefill both sides start from the same seeded random KV
contents (bf16 values read by the GPU, the same values given to the oracle),
with the context length of the workload.  Weights are the seeded random-init
weights of the workload, generated on the GPU and copied to the host for the
oracle.  The 70B-shaped base is truncated to its first layers (every layer
has the same shape and launch configuration) so that the oracle's float32
copy fits in host memory.
"""
import gc

import numpy as np
import pytest
import torch

from oracle import philox
from oracle.model import (MLP_PARALLEL, MLP_SEQUENTIAL, KVCache, OracleModel, attention, embed, final_logits,
                          forward, fuzzy_step, linear, mlp_part, rmsnorm, rope)
from oracle.plan import default_group_plan, plan_offsets
from oracle.sampling import accept_resample, sample_from_logits
from synth import get_config, make_weights
from gpu_common import TOL_BF16, exclusion, i32, rel_linf, say, ws

pytestmark = pytest.mark.gpu


def _random_kv(gkv, ctx, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    for t in (gkv.k, gkv.v):
        t[:, :, :, :ctx].copy_(torch.randn(t[:, :, :, :ctx].shape, generator=g, device="cuda").to(t.dtype))


def _oracle_kv(shape, gkv):
    okv = KVCache.__new__(KVCache)
    okv.k = gkv.k.float().cpu().numpy().astype(np.float32)
    okv.v = gkv.v.float().cpu().numpy().astype(np.float32)
    okv.capacity = gkv.capacity
    return okv


def _copy_kv(okv):
    c = KVCache.__new__(KVCache)
    c.k, c.v, c.capacity = okv.k.copy(), okv.v.copy(), okv.capacity
    return c


def _setup(shape, seed, batch, ctx, extra, layers=None):
    from layer_speculative_decoding_amd import api
    sh = shape if layers is None else shape.replace(n_layers=layers)
    w = make_weights(sh, seed, device="cuda")
    torch.cuda.synchronize()
    gm = api.SpecModel(sh, w)
    gkv = api.KVCache(sh, batch, ctx + extra + 2)
    _random_kv(gkv, ctx, seed + 5)
    om = OracleModel.from_torch(sh, w, np.float32)
    okv = _oracle_kv(sh, gkv)
    return sh, w, gm, gkv, om, okv


CASES = [
    # (config, which model, context, batch, layers of the model to keep)
    ("llama-1b-8b", "draft", 512, 1, None),
    ("llama-1b-8b", "base", 512, 1, None),
    ("llama-1b-8b-n4", "draft", 2048, 1, None),
    ("llama-1b-8b-n4", "base", 2048, 1, None),
    ("qwen-0.5b-7b", "draft", 1024, 1, None),
    ("qwen-0.5b-7b", "base", 1024, 1, None),
    ("llama-8b-70b", "draft", 8192, 4, None),
    ("llama-8b-70b", "base", 8192, 4, 4),
]


@pytest.mark.parametrize("cfg_name,which,ctx,batch,layers", CASES)
def test_fullsize_forward_entry_points(cfg_name, which, ctx, batch, layers):
    """One draft group step (draft models) or one k+1-token verify (base
    models) plus one ragged calibration, against the oracle."""
    from layer_speculative_decoding_amd import api
    cfg = get_config(cfg_name)
    shape = cfg.draft if which == "draft" else cfg.base
    seed = cfg.seed_draft if which == "draft" else cfg.seed_base
    k = cfg.k
    say(f"fullsize {cfg_name} {which} ctx={ctx} B={batch} layers={layers or shape.n_layers}")
    sh, w, gm, gkv, om, okv = _setup(shape, seed, batch, ctx, k + 1, layers)
    rng = np.random.default_rng(seed)
    V = sh.vocab
    inv_t = float(np.float32(1.0 / cfg.temperatures[-1])) if cfg.temperatures[-1] > 0 else 1.0
    pos = ctx - 1 - np.arange(batch, dtype=np.int32) * 3       # ragged positions
    if which == "draft":
        sets = default_group_plan(sh.n_layers, cfg.group_size)
        offs = plan_offsets(sets)
        G = max(len(s) for s in sets)
        wsb = ws(max(api.spec_workspace_bytes(gm, batch, 1, G), api.spec_workspace_bytes(gm, batch, k + 1, 1)))
        tok = rng.integers(0, V, size=batch).astype(np.int32)
        logits = torch.zeros(batch, V, device="cuda")
        out = torch.zeros(batch, dtype=torch.int32, device="cuda")
        # both MLP readings at the same positions (each step writes the fuzzy
        # K/V there before its attention reads them)
        for mlp in (MLP_SEQUENTIAL, MLP_PARALLEL):
            api.spec_draft_group_step(gm, gkv, offs, mlp, batch, i32(tok), 1, i32(pos), int(pos.max()), inv_t, 77,
                                      logits, V, out, 1, wsb)
            torch.cuda.synchronize()
            zg, tg = logits.cpu().numpy(), out.cpu().numpy()
            for b in range(batch):
                zo = fuzzy_step(om, okv, b, int(tok[b]), int(pos[b]), sets, mlp)
                err = rel_linf(zg[b], zo)
                say(f"  draft step ({'parallel' if mlp else 'sequential'} MLPs) b={b} logits rel {err:.2e}")
                assert err < TOL_BF16
                t_or, mg = sample_from_logits(zo, inv_t, 77, b, int(pos[b]) + 1, philox.DRAFT)
                if mg >= exclusion(zg[b], zo, inv_t):
                    assert tg[b] == t_or
        # ragged calibration over the same positions (rewrites the fuzzy entries)
        ntok = np.array([min(k + 1, 1 + (b * 2) % (k + 1)) for b in range(batch)], dtype=np.int32)
        toks = rng.integers(0, V, size=(batch, k + 1)).astype(np.int32)
        last = torch.zeros(batch, V, device="cuda")
        api.spec_calibrate_kv(gm, gkv, batch, i32(toks), i32(pos), i32(ntok), k + 1, int((pos + ntok - 1).max()),
                              inv_t, 78, last, V, out, 1, wsb)
        torch.cuda.synchronize()
        zg, tg = last.cpu().numpy(), out.cpu().numpy()
        for b in range(batch):
            zo = forward(om, okv, b, toks[b, :ntok[b]], range(pos[b], pos[b] + ntok[b]), logits="last")
            err = rel_linf(zg[b], zo)
            say(f"  calibrate b={b} n={ntok[b]} logits rel {err:.2e}")
            assert err < TOL_BF16
            t_or, mg = sample_from_logits(zo, inv_t, 78, b, int(pos[b] + ntok[b]), philox.DRAFT)
            if mg >= exclusion(zg[b], zo, inv_t):
                assert tg[b] == t_or
    else:
        m = k + 1
        wsb = ws(api.spec_workspace_bytes(gm, batch, m, 1))
        toks = rng.integers(0, V, size=(batch, m)).astype(np.int32)
        logits = torch.zeros(batch, m, V, device="cuda")
        api.spec_verify_forward(gm, gkv, batch, i32(toks), i32(pos), m, int(pos.max()) + m - 1, logits, wsb)
        torch.cuda.synchronize()
        zg = logits.cpu().numpy()
        for b in range(batch):
            if b == 0:
                # the plain float32 statement on the same bf16 weights and the
                # same context (no bf16 rounding of the new K/V either)
                plain = OracleModel(sh, om.w, False)
                zp = forward(plain, _copy_kv(okv), b, toks[b], range(pos[b], pos[b] + m), logits="all")
                ep = rel_linf(zg[b], zp)
                say(f"  verify b=0 logits rel to the plain float32 oracle {ep:.2e}")
                assert ep < TOL_BF16
            zo = forward(om, okv, b, toks[b], range(pos[b], pos[b] + m), logits="all")   # writes the KV too
            err = rel_linf(zg[b], zo)
            say(f"  verify b={b} logits rel {err:.2e}")
            assert err < TOL_BF16
            srt = np.sort(zo, axis=1)
            ok = (srt[:, -1] - srt[:, -2]) >= exclusion(zg[b], zo, 0.0)
            np.testing.assert_array_equal(np.argmax(zg[b], 1)[ok], np.argmax(zo, 1)[ok])
        # the KV the verify wrote
        kg = gkv.k.float().cpu().numpy()
        for b in range(batch):
            e = rel_linf(kg[:, b, :, pos[b]:pos[b] + m], okv.k[:, b, :, pos[b]:pos[b] + m])
            e0 = rel_linf(kg[0, b, :, pos[b]:pos[b] + m], okv.k[0, b, :, pos[b]:pos[b] + m])
            say(f"  verify KV b={b}: layer 0 rel {e0:.2e}, all layers rel {e:.2e}")
            assert e0 < 1e-2 and e < TOL_BF16, (e0, e)
    del gm, w, om, okv, gkv
    gc.collect()
    torch.cuda.empty_cache()


PREFILL_CASES = [
    # (config, which model, prompt rows per sequence, batch, layers of the model to keep)
    ("llama-1b-8b", "draft", 512, 1, None),
    ("llama-1b-8b", "base", 511, 1, None),
    ("llama-1b-8b-n4", "draft", 2048, 1, None),
    ("llama-1b-8b-n4", "base", 2047, 1, None),
    ("qwen-0.5b-7b", "draft", 1024, 1, None),
    ("qwen-0.5b-7b", "base", 1023, 1, None),
    ("llama-8b-70b", "base", 256, 4, 2),
]


@pytest.mark.parametrize("cfg_name,which,P,batch,layers", PREFILL_CASES)
def test_fullsize_prompt_prefill(cfg_name, which, P, batch, layers):
    """The prompt prefill at the workload's shapes, through the tiled
    matrix-core products the benchmark's prefill runs: the draft's
    calibration over the whole prompt (last-row logits and the sampled d_1)
    and the base's prefill (here with every row's logits), each with the KV
    it writes, against the oracle."""
    from layer_speculative_decoding_amd import api
    cfg = get_config(cfg_name)
    shape = cfg.draft if which == "draft" else cfg.base
    seed = cfg.seed_draft if which == "draft" else cfg.seed_base
    say(f"fullsize prefill {cfg_name} {which} P={P} B={batch} layers={layers or shape.n_layers}")
    sh, w, gm, gkv, om, okv = _setup(shape, seed, batch, 0, P, layers)
    rng = np.random.default_rng(seed + 3)
    V = sh.vocab
    toks = rng.integers(0, V, size=(batch, P)).astype(np.int32)
    wsb = ws(api.spec_workspace_bytes(gm, batch, P, 1))
    zero = i32([0] * batch)
    if which == "draft":
        inv_t = float(np.float32(1.0 / cfg.temperatures[-1])) if cfg.temperatures[-1] > 0 else 1.0
        last = torch.zeros(batch, V, device="cuda")
        out = torch.zeros(batch, dtype=torch.int32, device="cuda")
        api.spec_calibrate_kv(gm, gkv, batch, i32(toks), zero, None, P, P - 1, inv_t, 79, last, V, out, 1, wsb)
        torch.cuda.synchronize()
        zg, tg = last.cpu().numpy(), out.cpu().numpy()
        for b in range(batch):
            if b == 0:
                zp = forward(OracleModel(sh, om.w, False), _copy_kv(okv), b, toks[b], range(P), logits="last")
                say(f"  calibrate prefill b=0 logits rel to the plain float32 oracle {rel_linf(zg[b], zp):.2e}")
            zo = forward(om, okv, b, toks[b], range(P), logits="last")      # writes the KV too
            err = rel_linf(zg[b], zo)
            say(f"  calibrate prefill b={b} logits rel {err:.2e}")
            assert err < TOL_BF16
            t_or, mg = sample_from_logits(zo, inv_t, 79, b, P, philox.DRAFT)
            if mg >= exclusion(zg[b], zo, inv_t):
                assert tg[b] == t_or
    else:
        logits = torch.zeros(batch, P, V, device="cuda")
        api.spec_verify_forward(gm, gkv, batch, i32(toks), zero, P, P - 1, logits, wsb)
        torch.cuda.synchronize()
        zg = logits.cpu().numpy()
        del logits
        for b in range(batch):
            zo = forward(om, okv, b, toks[b], range(P), logits="all")       # writes the KV too
            err = rel_linf(zg[b], zo)
            say(f"  base prefill b={b} logits rel {err:.2e}")
            assert err < TOL_BF16
            srt = np.sort(zo, axis=1)
            ok = (srt[:, -1] - srt[:, -2]) >= exclusion(zg[b], zo, 0.0)
            np.testing.assert_array_equal(np.argmax(zg[b], 1)[ok], np.argmax(zo, 1)[ok])
    kg, vg = gkv.k.float().cpu().numpy(), gkv.v.float().cpu().numpy()
    for b in range(batch):
        e0 = rel_linf(kg[0, b, :, :P], okv.k[0, b, :, :P])
        ek = rel_linf(kg[:, b, :, :P], okv.k[:, b, :, :P])
        ev = rel_linf(vg[:, b, :, :P], okv.v[:, b, :, :P])
        say(f"  prefill KV b={b}: layer 0 K rel {e0:.2e}, all layers K {ek:.2e} V {ev:.2e}")
        assert e0 < 1e-2 and ek < TOL_BF16 and ev < TOL_BF16, (e0, ek, ev)
    del gm, w, om, okv, gkv
    gc.collect()
    torch.cuda.empty_cache()


def layer0_kv(om, toks_b):
    """Layer 0's keys and values [hkv][P][hd] for every prompt row (positions
    0 .. P-1) and its QKV rows, as the oracle's forward writes them."""
    sh = om.shape
    hq, hkv, hd, P = sh.n_q_heads, sh.n_kv_heads, sh.head_dim, len(toks_b)
    h0 = embed(om, toks_b)
    qkv = linear(rmsnorm(h0, om.w["attn_norm"][0], sh.rms_eps), om.w["wqkv"][0])
    K0 = om.rnd(rope(qkv[:, hq * hd:(hq + hkv) * hd].reshape(P, hkv, hd), range(P), sh.rope_theta)).transpose(1, 0, 2)
    V0 = om.rnd(qkv[:, (hq + hkv) * hd:].reshape(P, hkv, hd)).transpose(1, 0, 2)
    return h0, qkv, K0, V0


def layer0_output(om, h0, qkv, K0, V0, rows):
    """Layer 0's output at prompt rows `rows` (causal attention over the rows
    before each), given layer0_kv's results."""
    sh = om.shape
    hq, hkv, hd, n = sh.n_q_heads, sh.n_kv_heads, sh.head_dim, len(rows)
    q = rope(qkv[rows, :hq * hd].reshape(n, hq, hd), rows, sh.rope_theta)
    o = attention(q, K0, V0, rows, hkv).reshape(n, hq * hd)
    h1 = h0[rows] + linear(o, om.w["wo"][0])
    return h1 + mlp_part(om, 0, h1)


def layer1_kv_at(om, h2, rows):
    """Layer 1's keys and values [hkv][n][hd] at prompt rows `rows` from layer
    0's output h2 there."""
    sh = om.shape
    hq, hkv, hd, n = sh.n_q_heads, sh.n_kv_heads, sh.head_dim, len(rows)
    qkv1 = linear(rmsnorm(h2, om.w["attn_norm"][1], sh.rms_eps), om.w["wqkv"][1])
    K1 = om.rnd(rope(qkv1[:, hq * hd:(hq + hkv) * hd].reshape(n, hkv, hd), rows, sh.rope_theta)).transpose(1, 0, 2)
    V1 = om.rnd(qkv1[:, (hq + hkv) * hd:].reshape(n, hkv, hd)).transpose(1, 0, 2)
    return K1, V1


def test_fullsize_70b_prefill_sampled_rows():
    """The 70B-shaped base prefill in the launch configuration the benchmark
    times: four sequences of 8191 prompt rows in one call, so 32764 activation
    rows through the tiled products (their largest grids and the XCD-grouped
    tile order) and the prompt attention over the whole 8191-row prefix, here
    on the first two base layers.  Layer 0's keys and values depend on one
    product only, so the oracle forms them for every row and compares them
    all; for sampled rows it continues through layer 0's attention, O and MLP
    (on the oracle's own layer-0 cache) and compares the keys and values layer
    1 wrote there, which depend on every product of the prefill."""
    from layer_speculative_decoding_amd import api
    cfg = get_config("llama-8b-70b")
    sh = cfg.base.replace(n_layers=2)
    B, P = cfg.batch, cfg.prompt_len - 1
    say(f"fullsize prefill llama-8b-70b base, sampled rows: B={B} x P={P} rows in one call, 2 of "
        f"{cfg.base.n_layers} layers")
    w = make_weights(sh, cfg.seed_base, device="cuda")
    torch.cuda.synchronize()
    gm = api.SpecModel(sh, w)
    gkv = api.KVCache(sh, B, P + 2)
    rng = np.random.default_rng(cfg.seed_base + 11)
    toks = rng.integers(0, sh.vocab, size=(B, P)).astype(np.int32)
    wsb = ws(api.spec_workspace_bytes(gm, B, P, 1))
    api.spec_verify_forward(gm, gkv, B, i32(toks), i32([0] * B), P, P - 1, None, wsb)
    torch.cuda.synchronize()
    del wsb
    kg, vg = gkv.k.float().cpu().numpy(), gkv.v.float().cpu().numpy()    # [L][B][hkv][cap][hd]
    om = OracleModel.from_torch(sh, w, np.float32)
    del gm, gkv, w
    gc.collect()
    torch.cuda.empty_cache()
    say("  GPU prefill done, oracle weights ready")
    # block and tile edges of the prompt kernel and the tiled products, the
    # last rows, and a few others
    rows = sorted({0, 1, 15, 16, 31, 32, 127, 128, 1023, 2047, 2048, 4095, 4096, 6143, P - 2, P - 1}
                  | {int(r) for r in rng.integers(0, P, 8)})
    n = len(rows)
    for b in range(B):
        h0, qkv, K0, V0 = layer0_kv(om, toks[b])
        e0k = rel_linf(kg[0, b, :, :P], K0)
        e0v = rel_linf(vg[0, b, :, :P], V0)
        h2 = layer0_output(om, h0, qkv, K0, V0, rows)
        del qkv
        K1, V1 = layer1_kv_at(om, h2, rows)
        e1k = rel_linf(kg[1, b][:, rows], K1)
        e1v = rel_linf(vg[1, b][:, rows], V1)
        say(f"  b={b}: layer 0 K/V (all {P} rows) rel {e0k:.2e} / {e0v:.2e}; layer 1 K/V at {n} sampled rows "
            f"rel {e1k:.2e} / {e1v:.2e}")
        assert e0k < 1e-2 and e0v < 1e-2, (e0k, e0v)
        assert e1k < TOL_BF16 and e1v < TOL_BF16, (e1k, e1v)
    del om
    gc.collect()


def test_fullsize_70b_draft_calibration_prefill():
    """The 8B-shaped draft's calibration over the four 8192-token prompts in
    one call (32768 rows, the benchmark's draft prefill), on the draft's
    first layer: every row's keys and values against the oracle, then the
    last row of each sequence through the oracle's attention over the whole
    prompt, MLP, final norm and head, against the GPU's last-row logits (the
    gathered-row head) and its sampled d_1."""
    from layer_speculative_decoding_amd import api
    cfg = get_config("llama-8b-70b")
    sh = cfg.draft.replace(n_layers=1)
    B, P = cfg.batch, cfg.prompt_len
    inv_t = float(np.float32(1.0 / cfg.temperatures[-1])) if cfg.temperatures[-1] > 0 else 1.0
    say(f"fullsize calibration prefill llama-8b-70b draft: B={B} x P={P} rows in one call, 1 of "
        f"{cfg.draft.n_layers} layers, T={cfg.temperatures[-1]}")
    w = make_weights(sh, cfg.seed_draft, device="cuda")
    torch.cuda.synchronize()
    gm = api.SpecModel(sh, w)
    gkv = api.KVCache(sh, B, P + 2)
    rng = np.random.default_rng(cfg.seed_draft + 13)
    toks = rng.integers(0, sh.vocab, size=(B, P)).astype(np.int32)
    wsb = ws(api.spec_workspace_bytes(gm, B, P, 1))
    last = torch.zeros(B, sh.vocab, device="cuda")
    out = torch.zeros(B, dtype=torch.int32, device="cuda")
    api.spec_calibrate_kv(gm, gkv, B, i32(toks), i32([0] * B), None, P, P - 1, inv_t, 79, last, sh.vocab, out, 1,
                          wsb)
    torch.cuda.synchronize()
    del wsb
    kg, vg = gkv.k.float().cpu().numpy(), gkv.v.float().cpu().numpy()
    zg, tg = last.cpu().numpy(), out.cpu().numpy()
    om = OracleModel.from_torch(sh, w, np.float32)
    del gm, gkv, w, last, out
    gc.collect()
    torch.cuda.empty_cache()
    for b in range(B):
        h0, qkv, K0, V0 = layer0_kv(om, toks[b])
        ek = rel_linf(kg[0, b, :, :P], K0)
        ev = rel_linf(vg[0, b, :, :P], V0)
        zo = final_logits(om, layer0_output(om, h0, qkv, K0, V0, [P - 1]))[0]
        err = rel_linf(zg[b], zo)
        t_or, mg = sample_from_logits(zo, inv_t, 79, b, P, philox.DRAFT)
        decided = mg >= exclusion(zg[b], zo, inv_t)
        say(f"  b={b}: K/V (all {P} rows) rel {ek:.2e} / {ev:.2e}; last-row logits rel {err:.2e}; d_1 GPU "
            f"{tg[b]} oracle {t_or} (margin {mg:.2e}{'' if decided else ', excluded'})")
        assert ek < 1e-2 and ev < 1e-2, (ek, ev)
        assert err < TOL_BF16
        if decided:
            assert tg[b] == t_or
    del om
    gc.collect()


@pytest.mark.parametrize("cfg_name", ["llama-1b-8b", "llama-1b-8b-n4", "qwen-0.5b-7b", "llama-8b-70b"])
def test_fullsize_accept_resample(cfg_name):
    """accept / resample at the workload's vocabulary, batch and k, on logits
    whose draft and base rows are close (so both branches occur)."""
    from layer_speculative_decoding_amd import api
    cfg = get_config(cfg_name)
    B, k, V = cfg.batch, cfg.k, cfg.draft.vocab
    B = max(B, 4)
    say(f"fullsize accept {cfg_name} B={B} k={k} V={V}")
    rng = np.random.default_rng(cfg.index)
    for T in (0.0,) + tuple(t for t in cfg.temperatures if t > 0) + (1.0,):
        invt = 0.0 if T == 0 else float(np.float32(1.0 / T))
        zp = (rng.normal(size=(B, k + 1, V)) * 1.3).astype(np.float32)
        zq = (zp[:, :k] + 0.4 * rng.normal(size=(B, k, V))).astype(np.float32)
        d = np.argmax(zq, -1).astype(np.int32)
        t = np.full(B, 700, dtype=np.int32)
        vt = np.concatenate([np.zeros((B, 1), np.int32), d], 1)
        n_acc = torch.zeros(B, dtype=torch.int32, device="cuda")
        nxt = torch.zeros(B, dtype=torch.int32, device="cuda")
        w = ws(api.spec_accept_workspace_bytes(B, k, V))
        VT = i32(vt)
        api.spec_accept_resample(B, k, V, torch.tensor(zp, device="cuda"), torch.tensor(zq, device="cuda"),
                                 VT[:, 1:], k + 1, i32(t), invt, 99, n_acc, nxt, 1, None, w)
        a_g, y_g = n_acc.cpu().numpy(), nxt.cpu().numpy()
        for b in range(B):
            a, y, info = accept_resample(zp[b].astype(np.float64), zq[b].astype(np.float64), list(d[b]), 700,
                                         invt, 99, b)
            if min(mg for _, _, mg in info["margins"]) < 1e-3:
                continue
            assert (a_g[b], y_g[b]) == (a, y), (T, b)
