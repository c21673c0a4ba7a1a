"""The draft step that allocates nothing (its workspace is the library's
per-GPU scratch array) against the ordinary draft step with a caller
workspace: two calls in a row, the second with a smaller batch, through the
C ABI; logits, sampled tokens and the KV cache must be bit-identical (the
same kernels on the same inputs)."""
import numpy as np
import pytest
import torch

from oracle.plan import default_group_plan, plan_offsets
from synth import get_config, make_weights
from gpu_common import i32, say, ws

pytestmark = pytest.mark.gpu


def _same(a, b):
    return a.view(torch.int16).equal(b.view(torch.int16)) if a.dtype == torch.bfloat16 else torch.equal(a, b)


@pytest.mark.parametrize("layers", [4, None])
def test_noalloc_draft_step_matches_workspace_draft_step(layers):
    from layer_speculative_decoding_amd import api
    cfg = get_config("llama-1b-8b")
    sh = cfg.draft if layers is None else cfg.draft.replace(n_layers=layers)
    say(f"no-alloc draft step: {sh.n_layers}-layer 1B-shaped draft")
    w = make_weights(sh, cfg.seed_draft, device="cuda")
    gm = api.SpecModel(sh, w)
    B, ctx, V = 3, 300, sh.vocab
    offs = plan_offsets(default_group_plan(sh.n_layers, cfg.group_size))
    kv_a = api.KVCache(sh, B, ctx + 8)
    g = torch.Generator(device="cuda").manual_seed(5)
    for t in (kv_a.k, kv_a.v):
        t.copy_(torch.randn(t.shape, generator=g, device="cuda").to(t.dtype))
    kv_b = api.KVCache(sh, B, ctx + 8)
    kv_b.k.copy_(kv_a.k)
    kv_b.v.copy_(kv_a.v)
    G = max(offs[i + 1] - offs[i] for i in range(len(offs) - 1))
    wsb = ws(api.spec_workspace_bytes(gm, B, 1, G))
    rng = np.random.default_rng(3)
    for call, batch in enumerate((3, 1)):
        tok = i32(rng.integers(0, V, size=batch))
        pos = i32(ctx - 1 - 7 * np.arange(batch) - call)
        outs = []
        for kv, noalloc in ((kv_a, False), (kv_b, True)):
            logits = torch.full((batch, V), float("nan"), device="cuda")
            out = torch.full((batch,), -1, dtype=torch.int32, device="cuda")
            args = (gm, kv, offs, 0, batch, tok, 1, pos, int(pos.max()), 1.0, 77, logits, V, out, 1)
            if noalloc:
                api.spec_draft_group_step_noalloc(*args)
            else:
                api.spec_draft_group_step(*args, wsb)
            torch.cuda.synchronize()
            outs.append((logits, out))
        (la, oa), (lb, ob) = outs
        assert torch.equal(oa, ob)
        assert la.view(torch.int32).equal(lb.view(torch.int32))
        assert not torch.isnan(la).any()
        assert _same(kv_a.k, kv_b.k) and _same(kv_a.v, kv_b.v)
        say(f"  call {call + 1} (batch {batch}): tokens {ob.tolist()} identical, logits and KV bit-identical")
