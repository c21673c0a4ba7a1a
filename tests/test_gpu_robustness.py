"""Run-level properties of the GPU path: bit-determinism, no reads of stale
workspace contents, and resumption from the committed tokens.

Every reduction in the kernels has a fixed order and none uses float atomics,
so two runs on the same inputs are bit-identical.  No call may depend on what
an earlier call left in the shared workspace, so filling it with NaN before
every call changes nothing.  The state of a round is a function of the
committed tokens (rebuttal, reply on the fuzzy KV cache: fuzzy entries never
outlive a round, the calibration replaces them) and the uniforms are keyed by
the position of the decided token, so a run stopped after R rounds and
restarted from its committed tokens continues exactly as the uninterrupted
run."""
import numpy as np
import pytest
import torch

from oracle.plan import plan_offsets
from synth import make_prompts, make_weights, tiny_shape
from synth.configs import BF16
from gpu_common import say, to_dev

pytestmark = pytest.mark.gpu

SETS = [[0], [1, 2], [3]]


def _pair(dtype, seed=5, noise=0.006):
    sh = tiny_shape(4, 128, 8, 2, 16, 384, 512, dtype=dtype, qkv_bias=True)
    bw = make_weights(sh, seed, gain_std=0.1, std=0.05)
    g = torch.Generator().manual_seed(seed + 1)
    dw = {k: (None if v is None else (v.float() + noise * torch.randn(v.shape, generator=g)).to(v.dtype))
          for k, v in bw.items()}
    return sh, to_dev(dw), to_dev(bw)


def _decoder(sh, dw, bw, B, P, k, new, inv_temp, seed=31):
    from layer_speculative_decoding_amd.runtime import SpecDecoder
    dec = SpecDecoder(sh, dw, sh, bw, B, P + new + k + 2, k, plan_offsets(SETS), P, inv_temp, seed)
    dec.record = True
    return dec


def _run(sh, dw, bw, prompts, k, new, inv_temp):
    dec = _decoder(sh, dw, bw, prompts.shape[0], prompts.shape[1], k, new, inv_temp)
    out = dec.generate(prompts, new)
    torch.cuda.synchronize()
    return dec, out


@pytest.mark.parametrize("dtype", [0, BF16])
def test_two_runs_are_bit_identical(dtype):
    sh, dw, bw = _pair(dtype)
    B, P, k, new = 3, 12, 4, 20
    prompts = make_prompts(sh.vocab, P, B, lambda b: 401 + b)
    say(f"determinism dtype={dtype}")
    d1, o1 = _run(sh, dw, bw, prompts, k, new, 1.0)
    d2, o2 = _run(sh, dw, bw, prompts, k, new, 1.0)
    assert o1 == o2
    assert len(d1.records) == len(d2.records)
    for r1, r2 in zip(d1.records, d2.records):
        np.testing.assert_array_equal(r1.tokens, r2.tokens)
        np.testing.assert_array_equal(r1.n_acc, r2.n_acc)
        assert r1.q_logits.tobytes() == r2.q_logits.tobytes()
        assert r1.p_logits.tobytes() == r2.p_logits.tobytes()
    for c1, c2 in ((d1.dkv, d2.dkv), (d1.bkv, d2.bkv)):
        assert torch.equal(c1.k.view(torch.int16 if dtype else torch.int32), c2.k.view(torch.int16 if dtype else torch.int32))
        assert torch.equal(c1.v.view(torch.int16 if dtype else torch.int32), c2.v.view(torch.int16 if dtype else torch.int32))
    say(f"  {len(d1.records)} rounds bit-identical; accepted {sum(int(a) for r in d1.records for a in r.n_acc)}")


@pytest.mark.parametrize("dtype", [0, BF16])
def test_nan_poisoned_workspace_changes_nothing(dtype, monkeypatch):
    """Fill the shared workspace with NaN bit patterns before every call of
    the library: the run must equal a clean run bit for bit."""
    from layer_speculative_decoding_amd import api, runtime
    sh, dw, bw = _pair(dtype)
    B, P, k, new = 2, 10, 4, 16
    prompts = make_prompts(sh.vocab, P, B, lambda b: 411 + b)
    say(f"NaN-poisoned workspace dtype={dtype}")
    d1, o1 = _run(sh, dw, bw, prompts, k, new, 1.0)
    calls = {"n": 0}

    def poisoned(fn):
        def wrap(*a, **kw):
            ws = kw.get("workspace")
            if ws is None:
                ws = next(x for x in reversed(a) if isinstance(x, torch.Tensor) and x.dtype == torch.uint8)
            ws.fill_(0xFF)
            calls["n"] += 1
            return fn(*a, **kw)
        return wrap
    for name in ("spec_draft_group_step", "spec_calibrate_kv", "spec_verify_forward", "spec_accept_resample"):
        monkeypatch.setattr(runtime.api, name, poisoned(getattr(api, name)))
    d2, o2 = _run(sh, dw, bw, prompts, k, new, 1.0)
    assert calls["n"] > 4 * len(d2.records)
    assert o1 == o2
    for r1, r2 in zip(d1.records, d2.records):
        assert r1.q_logits.tobytes() == r2.q_logits.tobytes()
        assert r1.p_logits.tobytes() == r2.p_logits.tobytes()
    say(f"  {calls['n']} poisoned calls, {len(d2.records)} rounds bit-identical")


@pytest.mark.parametrize("dtype,inv_temp", [(0, 1.0), (0, 0.0), (BF16, 1.0)])
def test_resume_from_committed_tokens(dtype, inv_temp):
    """Stop after R rounds, start a new decoder on prompt + the tokens those
    rounds committed, and generate the rest: the tokens equal the
    uninterrupted run's.  (Resuming at a round boundary: a truncated round
    would move the later rounds' boundaries.  One sequence: the Philox key
    holds the sequence index.)"""
    sh, dw, bw = _pair(dtype)
    P, k, new = 10, 4, 24
    prompts = make_prompts(sh.vocab, P, 1, lambda b: 421 + b)
    say(f"resume dtype={dtype} invT={inv_temp}")
    d1, full = _run(sh, dw, bw, prompts, k, new, inv_temp)
    for R in (1, 3):
        done = sum(int(r.n_acc[0]) + 1 for r in d1.records[:R])
        assert done < new
        p2 = np.array([list(prompts[0]) + full[0][:done]], dtype=np.int32)
        dec = _decoder(sh, dw, bw, 1, p2.shape[1], k, new - done, inv_temp)
        rest = dec.generate(p2, new - done)[0]
        assert full[0][:done] + rest == full[0], (R, done)
        say(f"  resumed after {R} round(s) at {done} committed tokens: identical continuation")
