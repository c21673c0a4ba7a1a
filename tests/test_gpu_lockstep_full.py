"""Whole decode loop in lock step with the oracle at the four large
workloads' per-layer shapes: vocabulary (128256 / 152064), width, heads, set
size N and draft length k of each workload, several rounds at greedy and at
the workload's sampling temperature, and the 70B-shaped pair at batch 4 with
ragged accept counts and lanes that finish (and freeze) before the others.

Depth is truncated (every layer of a model has the same shape and launch
configuration, and the draft keeps a full layer-parallel set of its N) and
the prompts are shorter than the workloads' (the full-context entry points
are covered by the single-call tests at the workloads' contexts), so that the
oracle's float32 copy and its per-round cost fit the test budget.  Each round
the oracle recomputes from the GPU's committed history (EasySpec abstract:
draft, verify, calibrate; rebuttal reply on the fuzzy KV cache: the round's
state is a function of the committed tokens) and every decision outside the
exclusion bound must match."""
import gc
import time

import numpy as np
import pytest
import torch

from oracle.model import MLP_SEQUENTIAL, OracleModel
from oracle.plan import default_group_plan, plan_offsets
from synth import get_config, make_prompts, make_weights
from gpu_common import TOL_BF16, say
from lockstep import lockstep

pytestmark = pytest.mark.gpu

# (workload, draft layers kept, base layers kept, prompt length, new tokens,
#  temperatures)
CASES = [
    ("llama-1b-8b", 16, 8, 128, 16, (0.0, 1.0)),
    ("llama-1b-8b-n4", 16, 8, 128, 20, (0.0, 1.0)),
    ("qwen-0.5b-7b", 24, 7, 128, 16, (0.0, 0.7)),
    ("llama-8b-70b", 9, 4, 64, 12, (0.0, 1.0)),
]


@pytest.mark.parametrize("cfg_name,dl,bl,P,new,temps", CASES)
def test_lockstep_at_workload_shapes(cfg_name, dl, bl, P, new, temps):
    from layer_speculative_decoding_amd.runtime import SpecDecoder
    cfg = get_config(cfg_name)
    ds = cfg.draft.replace(n_layers=dl)
    bs = cfg.base.replace(n_layers=bl)
    B, k = cfg.batch, cfg.k
    sets = default_group_plan(dl, cfg.group_size)
    assert max(len(s) for s in sets) == cfg.group_size       # a full layer-parallel set
    say(f"lockstep {cfg_name}: draft {dl}/{cfg.draft.n_layers} layers, base {bl}/{cfg.base.n_layers}, "
        f"V {ds.vocab}, k {k}, N {cfg.group_size}, B {B}, P {P}, {new} tokens")
    t0 = time.time()
    dw = make_weights(ds, cfg.seed_draft, device="cuda")
    bw = make_weights(bs, cfg.seed_base, device="cuda")
    torch.cuda.synchronize()
    od = OracleModel.from_torch(ds, dw, np.float32)
    ob = OracleModel.from_torch(bs, bw, np.float32)
    prompts = make_prompts(ds.vocab, P, B, cfg.prompt_seed)
    say(f"  weights ready in {time.time() - t0:.1f}s")
    for T in temps:
        t1 = time.time()
        dec = SpecDecoder(ds, dw, bs, bw, B, P + new + k + 2, k, plan_offsets(sets), P, 0.0 if T == 0 else 1.0 / T,
                          cfg.sample_seed)
        st = lockstep(dec, od, ob, prompts, k, sets, new, dec.inv_temp, cfg.sample_seed, MLP_SEQUENTIAL, TOL_BF16)
        acc = [int(a) for r in dec.records for a in r.n_acc]
        finished_early = 0
        if B > 1:
            # rounds in which some lane was already frozen
            done = np.zeros(B, int)
            for r in dec.records:
                finished_early += int((done >= new).any() and (done < new).any())
                done += np.minimum(r.n_acc + 1, new - done)
        say(f"  T={T}: rounds {st['rounds']}, checked {st['checked']}, flipped by the logit difference "
            f"{st['flipped']}, excluded {st['excluded']}, max logit rel err {st['err']:.2e}, "
            f"accept counts {acc[:24]}{' ...' if len(acc) > 24 else ''}, rounds with frozen lanes "
            f"{finished_early}, {time.time() - t1:.1f}s")
        assert st["rounds"] >= 8
        assert st["excluded"] + st["flipped"] <= 2 + st["checked"] // 25
        if B > 1 and T > 0:
            assert len(set(acc)) > 1            # ragged accept counts
        del dec
    del dw, bw, od, ob
    gc.collect()
    torch.cuda.empty_cache()
