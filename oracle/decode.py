"""The speculative round loop and vanilla decoding, for one sequence.

Round structure (EasySpec abstract and rebuttal reply on the fuzzy KV cache):
the draft proposes k tokens with layer-parallel (fuzzy) steps, the base model
verifies them in one forward pass, the acceptance decisions come back, and the
draft KV cache is calibrated in a single precise forward pass so that fuzzy
entries live for one speculation phase only.

Readings adopted where the pages are silent:
  * prompt seam: the base prefills prompt[0:P-1]; the last prompt token is
    the first pending token x_t (t = P-1); the draft calibrates all P tokens;
  * calibration is merged with the forward of the emitted token: one precise
    draft pass over [d_1..d_a, y] at positions t+1..t+a+1, whose last position
    gives q_1 and d_1 of the next round, so a round has k-1 fuzzy steps;
  * exactly `new_tokens` tokens are produced; the last round is truncated.

separate=True is the other reading of what calibration covers (an ablation):
the draft prefills prompt[0:P-1] like the base, every round drafts all k
tokens with fuzzy steps starting from the pending token x_t, and after the
acceptance a separate precise pass rewrites the draft KV of the tokens that
were drafted fuzzily and committed, [x_t, d_1..d_a] at positions t..t+a; the
emitted token y is the next round's pending token.

A `hook(kind, key, value, margin)` may replace any decision (kinds 'draft',
'accept', 'y'); lock-step parity tests use it to adopt the GPU's choice where
the oracle's decision margin is below the exclusion threshold.
"""
from __future__ import annotations

from typing import Callable, List, Optional

import numpy as np

from . import philox
from .model import KVCache, OracleModel, forward, fuzzy_step, MLP_SEQUENTIAL
from .sampling import accept_resample, draw_y, sample_from_logits


def _id_hook(kind, key, value, margin):
    return value


def spec_generate(draft: OracleModel, base: OracleModel, prompt, k: int, sets,
                  new_tokens: int, inv_temp: float, seed: int, b: int = 0,
                  capacity: Optional[int] = None, mlp_mode: int = MLP_SEQUENTIAL,
                  calibrate: bool = True, hook: Optional[Callable] = None,
                  ftype=np.float64, caches=None, separate: bool = False):
    """Speculative decoding of one sequence.  Returns (tokens, rounds) where
    rounds is a list of dicts (t, drafts, a, y, q_logits, p_logits)."""
    hook = hook or _id_hook
    prompt = [int(x) for x in prompt]
    P = len(prompt)
    cap = capacity or (P + new_tokens + k + 2)
    if caches is None:
        dkv = KVCache(draft.shape, b + 1, cap, ftype)
        bkv = KVCache(base.shape, b + 1, cap, ftype)
    else:
        dkv, bkv = caches
    if P > 1:
        forward(base, bkv, b, prompt[:-1], range(P - 1), logits=None)
    if separate:
        if P > 1:
            forward(draft, dkv, b, prompt[:-1], range(P - 1), logits=None)
        zq = None
    else:
        zq = forward(draft, dkv, b, prompt, range(P), logits="last")
    t = P - 1
    seq = list(prompt)
    rounds = []
    r = 0
    while len(seq) - P < new_tokens:
        drafts: List[int] = []
        xt = seq[-1]
        if separate:
            zq = fuzzy_step(draft, dkv, b, xt, t, sets, mlp_mode)
        qlog = [zq]
        d, mg = sample_from_logits(zq, inv_temp, seed, b, t + 1, philox.DRAFT)
        drafts.append(hook("draft", (r, 1), d, mg))
        for j in range(1, k):
            z = fuzzy_step(draft, dkv, b, drafts[-1], t + j, sets, mlp_mode)
            qlog.append(z)
            d, mg = sample_from_logits(z, inv_temp, seed, b, t + j + 1, philox.DRAFT)
            drafts.append(hook("draft", (r, j + 1), d, mg))
        plog = forward(base, bkv, b, [xt] + drafts, range(t, t + k + 1), logits="all")
        a_or, y, info = accept_resample(plog, np.stack(qlog), drafts, t, inv_temp, seed, b)
        acc_m = [m for (kind, _, m) in info["margins"] if kind in ("accept", "argmax")]
        a = hook("accept", (r,), a_or, min(acc_m) if acc_m else np.inf)
        mg = info["margins"][-1][2]
        if a != a_or:
            y, mg = draw_y(plog, np.stack(qlog), a, t, inv_temp, seed, b)
        y = hook("y", (r,), y, mg)
        emitted = drafts[:a] + [y]
        rounds.append({"t": t, "drafts": list(drafts), "a": a, "y": y,
                       "q_logits": np.stack(qlog), "p_logits": plog})
        room = new_tokens - (len(seq) - P)
        seq += emitted[:room]
        if len(seq) - P >= new_tokens:
            break
        if separate:
            forward(draft, dkv, b, [xt] + drafts[:a], range(t, t + a + 1), logits=None)
        elif calibrate:
            zq = forward(draft, dkv, b, emitted, range(t + 1, t + a + 2), logits="last")
        else:
            # ablation: accepted drafts keep the fuzzy entries their steps
            # wrote; the tokens that have no draft entry yet run precisely:
            # y, and d_k too when every draft was accepted (no fuzzy step
            # feeds the last draft)
            j0 = min(a, k - 1)
            zq = forward(draft, dkv, b, emitted[j0:], range(t + 1 + j0, t + a + 2), logits="last")
        t = t + a + 1
        r += 1
    return seq[P:], rounds


def vanilla_generate(base: OracleModel, prompt, new_tokens: int, inv_temp: float, seed: int,
                     b: int = 0, capacity: Optional[int] = None, ftype=np.float64, hook=None):
    """Plain autoregressive decoding of the base model with the same streams
    the bonus draw uses (TARGET purpose at the position being decided)."""
    hook = hook or _id_hook
    prompt = [int(x) for x in prompt]
    P = len(prompt)
    cap = capacity or (P + new_tokens + 2)
    bkv = KVCache(base.shape, b + 1, cap, ftype)
    if P > 1:
        forward(base, bkv, b, prompt[:-1], range(P - 1), logits=None)
    seq = list(prompt)
    t = P - 1
    while len(seq) - P < new_tokens:
        z = forward(base, bkv, b, [seq[-1]], [t], logits="all")[0]
        y, mg = sample_from_logits(z, inv_temp, seed, b, t + 1, philox.TARGET)
        seq.append(hook("y", (t,), y, mg))
        t += 1
    return seq[P:]
