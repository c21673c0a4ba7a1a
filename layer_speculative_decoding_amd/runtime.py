"""Round loop of layer-parallel speculative decoding on one GPU.

Per round (EasySpec abstract and rebuttal reply on the fuzzy KV cache): k-1
layer-parallel draft steps, one k+1-token base verification, the
accept / resample decision, and one precise draft pass that calibrates the
draft KV over the emitted tokens and yields the next round's first draft.
All arithmetic runs in libspec's HIP kernels; this module only owns buffers,
uploads the round's positions and reads back the accept counts.

Readings where the pages are silent (shared with the CPU statement of the
method): the base prefills prompt[0:P-1] and the last prompt token is the
first pending token; calibration is merged with the emitted token's forward,
so a round has k-1 fuzzy steps; generation stops at exactly `new_tokens`.
"""
from __future__ import annotations

import time
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

from . import api
from ._lib import SPEC_MLP_SEQUENTIAL
from .trace import rng


@dataclass
class RoundRecord:
    t: List[int]
    tokens: np.ndarray          # [B][k+1]: x_t, d_1..d_k
    n_acc: np.ndarray           # [B]
    y: np.ndarray               # [B]
    q_logits: Optional[np.ndarray] = None   # [B][k][V]
    p_logits: Optional[np.ndarray] = None   # [B][k+1][V]


class SpecDecoder:
    def __init__(self, draft_shape, draft_w, base_shape, base_w, batch: int, capacity: int, k: int,
                 plan_offsets, prompt_len: int, inv_temp: float, seed: int,
                 mlp_mode: int = SPEC_MLP_SEQUENTIAL, device="cuda", calibrate: bool = True,
                 separate: bool = False):
        if k < 1:
            raise ValueError("k must be >= 1")
        self.dev = torch.device(device)
        self.draft = api.SpecModel(draft_shape, draft_w)
        self.base = api.SpecModel(base_shape, base_w)
        api.spec_check_pair(self.draft, self.base)
        self.B, self.k, self.V = batch, k, draft_shape.vocab
        self.cap = capacity
        self.plan = list(plan_offsets)
        self.G = max(self.plan[i + 1] - self.plan[i] for i in range(len(self.plan) - 1))
        self.mlp_mode = mlp_mode
        # calibrate=False is the ablation without KV calibration: the fuzzy
        # entries of accepted drafts stay, and only the emitted tokens that
        # have no draft entry yet run precisely (y, and d_k when every draft
        # was accepted, since no fuzzy step feeds the last draft); that pass
        # also yields the next d_1
        self.calibrate = calibrate
        # separate=True is the other reading of the calibration (ablation):
        # all k drafts come from fuzzy steps starting at the pending token,
        # and after the acceptance a precise pass rewrites the draft KV of
        # [x_t, d_1..d_a] at t..t+a; the emitted token is the next pending one
        self.separate = separate
        if separate and not calibrate:
            raise ValueError("separate calibration needs calibrate=True")
        self.inv_temp = float(np.float32(inv_temp))
        self.seed = int(seed)
        self.dkv = api.KVCache(draft_shape, batch, capacity, device)
        self.bkv = api.KVCache(base_shape, batch, capacity, device)
        P = prompt_len
        d_ws = max(api.spec_workspace_bytes(self.draft, batch, max(P, k + 1), 1),
                   api.spec_workspace_bytes(self.draft, batch, 1, self.G))
        b_ws = api.spec_workspace_bytes(self.base, batch, max(P - 1, k + 1), 1)
        a_ws = api.spec_accept_workspace_bytes(batch, k, self.V)
        self.ws = torch.empty(max(d_ws, b_ws, a_ws), dtype=torch.uint8, device=self.dev)
        i32 = dict(dtype=torch.int32, device=self.dev)
        self.vtok = torch.zeros(batch, k + 1, **i32)           # x_t, d_1..d_k
        self.q_logits = torch.zeros(batch, k, self.V, dtype=torch.float32, device=self.dev)
        self.p_logits = torch.zeros(batch, k + 1, self.V, dtype=torch.float32, device=self.dev)
        self.n_acc = torch.zeros(batch, **i32)
        self.commit = torch.zeros(batch, k + 1, **i32)
        self.xt = torch.zeros(batch, **i32)                    # pending token of the round
        self.caltok = torch.zeros(batch, k + 1, **i32)         # [x_t, d_1..d_k] (separate calibration)
        self.nocal_host = torch.zeros(batch, k + 1, dtype=torch.int32).pin_memory()
        self.dummy_tok = torch.zeros(batch, **i32)
        # per-round integer table: [0:k] positions t+j for j = 0..k-1 ([B] each),
        # [k] calibration start t+1, [k+1] calibration count a+1
        self.tab = torch.zeros(k + 2, batch, **i32)
        self.tab_host = torch.zeros(k + 2, batch, dtype=torch.int32).pin_memory()
        self.back_host = torch.zeros(batch, 2 * (k + 1) + 1, dtype=torch.int32).pin_memory()
        self.t = [0] * batch
        self.out: List[List[int]] = [[] for _ in range(batch)]
        self.records: List[RoundRecord] = []
        self.record = False

    # ---------------------------------------------------------------- prefill
    def prefill(self, prompts: np.ndarray):
        with rng("prefill"):
            self._prefill(prompts)

    def _prefill(self, prompts: np.ndarray):
        B, P = prompts.shape
        assert B == self.B and P >= 1
        toks = torch.from_numpy(np.ascontiguousarray(prompts, dtype=np.int32)).to(self.dev)
        zero = torch.zeros(B, dtype=torch.int32, device=self.dev)
        if P > 1:
            pre = toks[:, :P - 1].contiguous()
            api.spec_verify_forward(self.base, self.bkv, B, pre, zero, P - 1, P - 2, None, self.ws)
        if self.separate:
            # the last prompt token is drafted from with a fuzzy step
            if P > 1:
                api.spec_calibrate_kv(self.draft, self.dkv, B, toks[:, :P - 1].contiguous(), zero, None, P - 1,
                                      P - 2, self.inv_temp, self.seed, None, 0, self.dummy_tok, 1, self.ws)
        else:
            api.spec_calibrate_kv(self.draft, self.dkv, B, toks, zero, None, P, P - 1, self.inv_temp, self.seed,
                                  self.q_logits[:, 0], self.k * self.V, self.vtok[:, 1], self.k + 1, self.ws)
        self.vtok[:, 0].copy_(toks[:, P - 1])
        self.t = [P - 1] * B
        self.out = [[] for _ in range(B)]

    # ------------------------------------------------------------------ round
    def _upload_positions(self):
        th = self.tab_host
        for b in range(self.B):
            for j in range(self.k):
                th[j, b] = self.t[b] + j
        self.tab[:self.k].copy_(th[:self.k], non_blocking=True)

    def draft_phase(self):
        k, B = self.k, self.B
        for j in range(0 if self.separate else 1, k):
            api.spec_draft_group_step(
                self.draft, self.dkv, self.plan, self.mlp_mode, B, self.vtok[:, j], k + 1, self.tab[j],
                max(self.t) + j, self.inv_temp, self.seed, self.q_logits[:, j], k * self.V,
                self.vtok[:, j + 1], k + 1, self.ws)

    def verify_phase(self):
        k, B = self.k, self.B
        api.spec_verify_forward(self.base, self.bkv, B, self.vtok, self.tab[0], k + 1, max(self.t) + k,
                                self.p_logits, self.ws)

    def accept_phase(self):
        k, B = self.k, self.B
        api.spec_accept_resample(B, k, self.V, self.p_logits, self.q_logits, self.vtok[:, 1:], k + 1,
                                 self.tab[0], self.inv_temp, self.seed, self.n_acc, self.vtok[:, 0], k + 1,
                                 self.commit, self.ws)

    def step(self, new_tokens: int, marks=None) -> bool:
        with rng("round"):
            return self._step(new_tokens, marks)

    def _step(self, new_tokens: int, marks=None) -> bool:
        """One round; returns True while some sequence still needs tokens.

        marks: optional list of 5 timing events recorded on the stream at the
        round's phase boundaries (start, after drafting, after verify, after
        accept, after calibration)."""
        k, B = self.k, self.B
        self._upload_positions()
        if marks:
            marks[0].record()
        with rng("draft"):
            self.draft_phase()
        if marks:
            marks[1].record()
        with rng("verify"):
            self.verify_phase()
        if marks:
            marks[2].record()
        if self.separate:
            self.xt.copy_(self.vtok[:, 0])
        if self.record:
            tok_before = self.vtok.to("cpu").numpy().copy()
            ql = self.q_logits.cpu().numpy().copy()
            pl = self.p_logits.cpu().numpy().copy()
        with rng("accept"):
            self.accept_phase()
        if marks:
            marks[3].record()
        bh = self.back_host
        bh[:, 0].copy_(self.n_acc, non_blocking=True)
        bh[:, 1:k + 2].copy_(self.commit, non_blocking=True)
        torch.cuda.current_stream().synchronize()
        a = bh[:, 0].numpy().copy()
        com = bh[:, 1:k + 2].numpy().copy()
        if self.record:
            self.records.append(RoundRecord(list(self.t), tok_before, a.copy(),
                                            np.array([com[b, a[b]] for b in range(B)]), ql, pl))
        more = False
        th = self.tab_host
        for b in range(B):
            room = new_tokens - len(self.out[b])
            th[k, b] = self.t[b] + 1
            th[k + 1, b] = 0
            if room <= 0:
                # finished sequence: its lane keeps running with the batch,
                # frozen at its position (no calibration rows), so it never
                # outgrows the cache
                continue
            emitted = [int(x) for x in com[b, :a[b] + 1]]
            self.out[b].extend(emitted[:room])
            if len(self.out[b]) >= new_tokens:
                continue
            th[k + 1, b] = a[b] + 1
            if self.separate:
                th[k, b] = self.t[b]       # [x_t, d_1..d_a] at t..t+a
            self.t[b] += int(a[b]) + 1
            if not self.calibrate:
                # accepted drafts d_1..d_j0 keep their fuzzy entries
                j0 = min(int(a[b]), k - 1)
                th[k, b] = self.t[b] - int(a[b]) + j0
                th[k + 1, b] = int(a[b]) + 1 - j0
                for i, x in enumerate(emitted[j0:]):
                    self.nocal_host[b, i] = x
            more = True
        if not more:
            if marks:
                marks[4].record()
            return False
        self.tab[k:].copy_(th[k:], non_blocking=True)
        # the calibration covers exactly the emitted tokens: its row bound is
        # the longest a + 1 of the round (token rows keep their k + 1 stride)
        rows = max(1, max(int(th[k + 1, b]) for b in range(B)))
        if not self.calibrate:
            self.caltok.copy_(self.nocal_host, non_blocking=True)
        with rng("calibrate"):
            self._calibrate(th, rows, k, B)
        if marks:
            marks[4].record()
        return True

    def _calibrate(self, th, rows, k, B):
        if self.separate:
            self.caltok[:, 0].copy_(self.xt)
            self.caltok[:, 1:].copy_(self.vtok[:, 1:])
            api.spec_calibrate_kv(self.draft, self.dkv, B, self.caltok, self.tab[k], self.tab[k + 1], rows,
                                  max(self.t), self.inv_temp, self.seed, None, 0, self.dummy_tok, 1, self.ws,
                                  tokens_stride=k + 1)
        else:
            toks = self.commit if self.calibrate else self.caltok
            api.spec_calibrate_kv(self.draft, self.dkv, B, toks, self.tab[k], self.tab[k + 1], rows,
                                  max(self.t), self.inv_temp, self.seed, self.q_logits[:, 0], k * self.V,
                                  self.vtok[:, 1], k + 1, self.ws, tokens_stride=k + 1)

    def generate(self, prompts: np.ndarray, new_tokens: int) -> List[List[int]]:
        self.prefill(prompts)
        while self.step(new_tokens):
            pass
        return [o[:new_tokens] for o in self.out]


class VanillaDecoder:
    """Plain autoregressive decoding of the base on the same kernels: verify
    with m = 1 and accept / resample with k = 0 (a sampling step from p_1)."""

    def __init__(self, base_shape, base_w, batch: int, capacity: int, prompt_len: int, inv_temp: float,
                 seed: int, device="cuda"):
        self.dev = torch.device(device)
        self.base = api.SpecModel(base_shape, base_w)
        self.B, self.V = batch, base_shape.vocab
        self.inv_temp = float(np.float32(inv_temp))
        self.seed = int(seed)
        self.bkv = api.KVCache(base_shape, batch, capacity, device)
        ws = max(api.spec_workspace_bytes(self.base, batch, max(prompt_len - 1, 1), 1),
                 api.spec_accept_workspace_bytes(batch, 0, self.V))
        self.ws = torch.empty(ws, dtype=torch.uint8, device=self.dev)
        i32 = dict(dtype=torch.int32, device=self.dev)
        self.tok = torch.zeros(batch, 1, **i32)
        self.pos = torch.zeros(batch, **i32)
        self.logits = torch.zeros(batch, 1, self.V, dtype=torch.float32, device=self.dev)
        self.n_acc = torch.zeros(batch, **i32)
        self.hist = None

    def generate(self, prompts: np.ndarray, new_tokens: int) -> List[List[int]]:
        B, P = prompts.shape
        toks = torch.from_numpy(np.ascontiguousarray(prompts, dtype=np.int32)).to(self.dev)
        zero = torch.zeros(B, dtype=torch.int32, device=self.dev)
        if P > 1:
            api.spec_verify_forward(self.base, self.bkv, B, toks[:, :P - 1].contiguous(), zero, P - 1, P - 2,
                                    None, self.ws)
        self.tok[:, 0].copy_(toks[:, P - 1])
        self.pos.fill_(P - 1)
        hist = torch.zeros(B, new_tokens, dtype=torch.int32, device=self.dev)
        torch.cuda.current_stream().synchronize()
        t0 = time.perf_counter()
        for i in range(new_tokens):
            t = P - 1 + i
            api.spec_verify_forward(self.base, self.bkv, B, self.tok, self.pos, 1, t, self.logits, self.ws)
            api.spec_accept_resample(B, 0, self.V, self.logits, None, None, 1, self.pos, self.inv_temp,
                                     self.seed, self.n_acc, hist[:, i], new_tokens, None, self.ws)
            self.tok[:, 0].copy_(hist[:, i])
            self.pos.add_(1)
        out = hist.cpu().numpy().tolist()
        self.decode_s = time.perf_counter() - t0
        return out
