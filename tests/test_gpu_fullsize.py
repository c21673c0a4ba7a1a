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
import copy
import gc

import numpy as np
import pytest
import torch

import oracle.model as omod
from oracle import philox
from oracle.model import KVCache, OracleModel, forward, fuzzy_step
from oracle.plan import default_group_plan, plan_offsets
from oracle.sampling import accept_resample, sample_from_logits
from synth import get_config, make_weights
from gpu_common import TOL_BF16, exclusion, i32, rel_linf, say, ws

pytestmark = pytest.mark.gpu


def _random_kv(gkv, ctx, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    for t in (gkv.k, gkv.v):
        t[:, :, :, :ctx].copy_(torch.randn(t[:, :, :, :ctx].shape, generator=g, device="cuda").to(t.dtype))


def _sensitive(fn, okv):
    """Run fn(okv_copy) cleanly and with float32-level relative noise (6e-8)
    injected at the normalisation outputs; returns (clean, noisy).

    On the bf16 path the operands of every product are rounded to bf16, so a
    perturbation of float32 size flips some roundings; through a deep
    random-init stack those flips grow.  The GPU computes in float32 with its
    own accumulation order, so its distance from the oracle is of the same
    size as this self-perturbation."""
    clean = fn(copy.deepcopy(okv))
    orig = omod.rmsnorm

    def noisy(x, g, eps):
        y = orig(x, g, eps)
        return y * (1.0 + np.random.default_rng(1).normal(size=y.shape) * 6e-8)
    omod.rmsnorm = noisy
    try:
        pert = fn(copy.deepcopy(okv))
    finally:
        omod.rmsnorm = orig
    return clean, pert


def _tol(clean, pert):
    return max(TOL_BF16, 2.0 * rel_linf(pert, clean))


def _oracle_kv(shape, gkv):
    okv = KVCache.__new__(KVCache)
    okv.k = gkv.k.float().cpu().numpy().astype(np.float32)
    okv.v = gkv.v.float().cpu().numpy().astype(np.float32)
    okv.capacity = gkv.capacity
    return okv


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
    ("llama-1b-8b-n4", "base", 2048, 1, 8),
    ("qwen-0.5b-7b", "draft", 1024, 1, None),
    ("qwen-0.5b-7b", "base", 1024, 1, None),
    ("llama-8b-70b", "draft", 8192, 4, 8),
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
        api.spec_draft_group_step(gm, gkv, offs, 0, batch, i32(tok), 1, i32(pos), int(pos.max()), inv_t, 77,
                                  logits, V, out, 1, wsb)
        torch.cuda.synchronize()
        zg, tg = logits.cpu().numpy(), out.cpu().numpy()
        for b in range(batch):
            zo, zn = _sensitive(lambda kv: fuzzy_step(om, kv, b, int(tok[b]), int(pos[b]), sets), okv)
            fuzzy_step(om, okv, b, int(tok[b]), int(pos[b]), sets)       # advance the oracle's cache
            err, tol = rel_linf(zg[b], zo), _tol(zo, zn)
            say(f"  draft step b={b} logits rel {err:.2e} (oracle self-sensitivity {rel_linf(zn, zo):.2e})")
            assert err < tol
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
            fn = lambda kv: forward(om, kv, b, toks[b, :ntok[b]], range(pos[b], pos[b] + ntok[b]), logits="last")
            zo, zn = _sensitive(fn, okv)
            err, tol = rel_linf(zg[b], zo), _tol(zo, zn)
            say(f"  calibrate b={b} n={ntok[b]} logits rel {err:.2e} (self-sensitivity {rel_linf(zn, zo):.2e})")
            assert err < tol
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
        tols = []
        for b in range(batch):
            zo, zn = _sensitive(lambda kv: forward(om, kv, b, toks[b], range(pos[b], pos[b] + m), logits="all"), okv)
            forward(om, okv, b, toks[b], range(pos[b], pos[b] + m), logits=None)   # the KV it writes
            err, tol = rel_linf(zg[b], zo), _tol(zo, zn)
            tols.append(tol)
            say(f"  verify b={b} logits rel {err:.2e} (self-sensitivity {rel_linf(zn, zo):.2e})")
            assert err < tol
            srt = np.sort(zo, axis=1)
            ok = (srt[:, -1] - srt[:, -2]) >= exclusion(zg[b], zo, 0.0)
            np.testing.assert_array_equal(np.argmax(zg[b], 1)[ok], np.argmax(zo, 1)[ok])
        # the KV the verify wrote
        kg = gkv.k.float().cpu().numpy()
        for b in range(batch):
            e = rel_linf(kg[:, b, :, pos[b]:pos[b] + m], okv.k[:, b, :, pos[b]:pos[b] + m])
            e0 = rel_linf(kg[0, b, :, pos[b]:pos[b] + m], okv.k[0, b, :, pos[b]:pos[b] + m])
            say(f"  verify KV b={b}: layer 0 rel {e0:.2e}, all layers rel {e:.2e}")
            assert e0 < 1e-2 and e < tols[b], (e0, e)
    del gm, w, om, okv, gkv
    gc.collect()
    torch.cuda.empty_cache()


PREFILL_CASES = [
    # (config, which model, prompt rows per sequence, batch, layers of the model to keep)
    ("llama-1b-8b", "draft", 512, 1, None),
    ("llama-1b-8b", "base", 511, 1, None),
    ("llama-1b-8b-n4", "draft", 2048, 1, 4),
    ("llama-1b-8b-n4", "base", 2047, 1, 2),
    ("qwen-0.5b-7b", "draft", 1024, 1, None),
    ("qwen-0.5b-7b", "base", 1023, 1, 8),
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
    tols = []
    if which == "draft":
        inv_t = float(np.float32(1.0 / cfg.temperatures[-1])) if cfg.temperatures[-1] > 0 else 1.0
        last = torch.zeros(batch, V, device="cuda")
        out = torch.zeros(batch, dtype=torch.int32, device="cuda")
        api.spec_calibrate_kv(gm, gkv, batch, i32(toks), zero, None, P, P - 1, inv_t, 79, last, V, out, 1, wsb)
        torch.cuda.synchronize()
        zg, tg = last.cpu().numpy(), out.cpu().numpy()
        for b in range(batch):
            fn = lambda kv: forward(om, kv, b, toks[b], range(P), logits="last")
            zo, zn = _sensitive(fn, okv)
            forward(om, okv, b, toks[b], range(P), logits=None)       # the KV it writes
            err, tol = rel_linf(zg[b], zo), _tol(zo, zn)
            tols.append(tol)
            say(f"  calibrate prefill b={b} logits rel {err:.2e} (self-sensitivity {rel_linf(zn, zo):.2e})")
            assert err < tol
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
            fn = lambda kv: forward(om, kv, b, toks[b], range(P), logits="all")
            zo, zn = _sensitive(fn, okv)
            forward(om, okv, b, toks[b], range(P), logits=None)
            err, tol = rel_linf(zg[b], zo), _tol(zo, zn)
            tols.append(tol)
            say(f"  base prefill b={b} logits rel {err:.2e} (self-sensitivity {rel_linf(zn, zo):.2e})")
            assert err < tol
            srt = np.sort(zo, axis=1)
            ok = (srt[:, -1] - srt[:, -2]) >= exclusion(zg[b], zo, 0.0)
            np.testing.assert_array_equal(np.argmax(zg[b], 1)[ok], np.argmax(zo, 1)[ok])
    kg, vg = gkv.k.float().cpu().numpy(), gkv.v.float().cpu().numpy()
    for b in range(batch):
        e0 = rel_linf(kg[0, b, :, :P], okv.k[0, b, :, :P])
        ek = rel_linf(kg[:, b, :, :P], okv.k[:, b, :, :P])
        ev = rel_linf(vg[:, b, :, :P], okv.v[:, b, :, :P])
        say(f"  prefill KV b={b}: layer 0 K rel {e0:.2e}, all layers K {ek:.2e} V {ev:.2e}")
        assert e0 < 1e-2 and ek < tols[b] and ev < tols[b], (e0, ek, ev)
    del gm, w, om, okv, gkv
    gc.collect()
    torch.cuda.empty_cache()


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
