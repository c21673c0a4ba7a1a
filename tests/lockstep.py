"""Lock-step comparison of a GPU speculative run with the oracle.

The GPU run records every round (pending position, [x_t, d_1..d_k], accept
count, emitted token, and the round's draft / base logits).  The oracle then
replays the rounds, always continuing with the GPU's decision so that both
stay on one trajectory, and logs its own decision and margin.  Afterwards
every decision whose oracle margin exceeds the exclusion bound must equal the
GPU's.  The bound follows from the measured logit error dz of that round and
sequence (scores are z / T plus identical Gumbel noise):
  draft / greedy / bonus arg-max:   2 * s * dz      (s = 1/T, or 1 greedy)
  accept test |u - p/q|, residual:  8 * s * dz      (p/q and log(p - q) move
                                                     by at most ~4 s dz)
never below MARGIN.  The stats separate the excluded decisions into those
below MARGIN (the fixed rule: within 1e-3 of a tie or threshold) and those in
the band between MARGIN and the error-derived bound ('band'), and count how
many excluded decisions the GPU took differently ('flipped')."""
import numpy as np

from oracle.decode import spec_generate
from gpu_common import MARGIN


def lockstep(dec, om_draft, om_base, prompts, k, sets, new_tokens, inv_temp, seed, mlp_mode, tol, calibrate=True,
             separate=False):
    B = prompts.shape[0]
    dec.record = True
    dec.records = []
    gpu_out = dec.generate(prompts, new_tokens)
    recs = dec.records
    s = 1.0 if inv_temp == 0.0 else inv_temp
    stats = {"checked": 0, "excluded": 0, "band": 0, "flipped": 0, "err": 0.0, "rounds": len(recs)}
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
        dz = []
        for r, rd in enumerate(rounds):
            rec = recs[r]
            assert rec.t[b] == rd["t"]
            zq, zp = rec.q_logits[b], rec.p_logits[b]
            e1 = float(np.max(np.abs(zq - rd["q_logits"])))
            e2 = float(np.max(np.abs(zp - rd["p_logits"])))
            r1 = e1 / float(np.max(np.abs(rd["q_logits"])))
            r2 = e2 / float(np.max(np.abs(rd["p_logits"])))
            stats["err"] = max(stats["err"], r1, r2)
            assert r1 < tol and r2 < tol, (b, r, r1, r2)
            dz.append(max(e1, e2))
        for kind, key, value, margin, g in log:
            c = 2.0 if (kind == "draft" or inv_temp == 0.0) else 8.0
            thr = max(MARGIN, c * s * dz[key[0]] + 1e-5)
            if margin >= thr:
                assert g == value, (b, kind, key, g, value, margin, thr)
                stats["checked"] += 1
            else:
                stats["excluded"] += 1
                stats["band"] += margin >= MARGIN
                stats["flipped"] += g != value
    return stats
