"""Lock-step comparison of a GPU speculative run with the oracle.

The GPU run records every round (pending position, [x_t, d_1..d_k], accept
count, emitted token, and the round's draft / base logits).  The oracle then
replays the rounds, always continuing with the GPU's decision so that both
stay on one trajectory, and logs its own decision and margin.

Every decision is then taken a third time: by the oracle's sampling code on
the GPU's own logits (same Philox words), which is the decision the GPU's
logits imply.
  * The GPU's decision must equal it (the sampling / accept kernels decide
    exactly as the rule says on the logits they were given), except where
    that implied decision is itself within TIE of a tie (float32 scores on
    the GPU against float64 here).
  * Where the oracle's logits give the same decision as the GPU's logits, the
    GPU must have taken it: 'checked'.
  * Where the two sets of logits give different decisions, the logit
    difference (held to the stated tolerance) flips a near tie: 'flipped'.
    Only these, and decisions within MARGIN (1e-3) of a tie or threshold on
    the oracle's side ('excluded'), are not compared with the oracle.
"""
import numpy as np

from oracle import philox
from oracle.decode import spec_generate
from oracle.sampling import accept_resample, draw_y, sample_from_logits
from gpu_common import MARGIN

TIE = 1e-4


def _implied(kind, key, rec, b, k, inv_temp, seed):
    """The decision the GPU's logits of round rec imply, and its margin."""
    t = int(rec.t[b])
    zq = rec.q_logits[b].astype(np.float64)
    zp = rec.p_logits[b].astype(np.float64)
    if kind == "draft":
        j = key[1]
        return sample_from_logits(zq[j - 1], inv_temp, seed, b, t + j, philox.DRAFT)
    if kind == "accept":
        a, _, info = accept_resample(zp, zq, [int(x) for x in rec.tokens[b, 1:k + 1]], t, inv_temp, seed, b)
        m = [mg for (kd, _, mg) in info["margins"] if kd in ("accept", "argmax")]
        return a, (min(m) if m else np.inf)
    return draw_y(zp, zq, int(rec.n_acc[b]), t, inv_temp, seed, b)


def lockstep(dec, om_draft, om_base, prompts, k, sets, new_tokens, inv_temp, seed, mlp_mode, tol, calibrate=True,
             separate=False):
    B = prompts.shape[0]
    dec.record = True
    dec.records = []
    gpu_out = dec.generate(prompts, new_tokens)
    recs = dec.records
    stats = {"checked": 0, "excluded": 0, "flipped": 0, "err": 0.0, "rounds": len(recs)}
    for b in range(B):
        log = []

        def hook(kind, key, value, margin, b=b):
            rec = recs[key[0]]
            if kind == "draft":
                g = int(rec.tokens[b, key[1]])
            elif kind == "accept":
                g = int(rec.n_acc[b])
            else:
                g = int(rec.y[b])
            log.append((kind, key, value, margin, g))
            return g

        toks, rounds = spec_generate(om_draft, om_base, prompts[b], k, sets, new_tokens, inv_temp, seed, b=b,
                                     capacity=dec.cap, mlp_mode=mlp_mode, calibrate=calibrate, hook=hook,
                                     separate=separate)
        assert toks == gpu_out[b], (b, toks[:20], gpu_out[b][:20])
        for r, rd in enumerate(rounds):
            rec = recs[r]
            assert rec.t[b] == rd["t"]
            zq, zp = rec.q_logits[b], rec.p_logits[b]
            r1 = float(np.max(np.abs(zq - rd["q_logits"]))) / float(np.max(np.abs(rd["q_logits"])))
            r2 = float(np.max(np.abs(zp - rd["p_logits"]))) / float(np.max(np.abs(rd["p_logits"])))
            stats["err"] = max(stats["err"], r1, r2)
            assert r1 < tol and r2 < tol, (b, r, r1, r2)
        for kind, key, value, margin, g in log:
            imp, mg = _implied(kind, key, recs[key[0]], b, k, inv_temp, seed)
            if mg >= TIE:
                assert g == imp, ("GPU decision differs from the one its logits imply", b, kind, key, g, imp, mg)
            if margin < MARGIN or mg < TIE:
                stats["excluded"] += 1
            elif value == imp:
                assert g == value, (b, kind, key, g, value, margin)
                stats["checked"] += 1
            else:
                stats["flipped"] += 1
    return stats
