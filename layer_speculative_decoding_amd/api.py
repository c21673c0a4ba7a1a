"""Python entry points with the C ABI's names (argument marshalling only).

Tensors must live on the GPU; pointers and the current torch stream are handed
to libspec, which does all of the computation in its HIP kernels.
"""
from __future__ import annotations

import ctypes as C
from typing import Optional, Sequence

import torch

from ._lib import KV, ModelDesc, Weights, SpecError, check, load, SPEC_BF16, SPEC_F32

_WKEYS = ("embed", "attn_norm", "wqkv", "bqkv", "wo", "ffn_norm", "w_gate_up", "w_down", "final_norm", "lm_head")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


class SpecModel:
    """A libspec model handle over caller-owned device weight arenas."""

    def __init__(self, shape, weights: dict):
        lib = load()
        self.shape = shape
        self.weights = weights          # keeps the device memory alive
        dt = SPEC_BF16 if shape.dtype == 1 else SPEC_F32
        want = torch.bfloat16 if dt == SPEC_BF16 else torch.float32
        for k in ("embed", "wqkv", "wo", "w_gate_up", "w_down", "lm_head"):
            t = weights[k]
            if t.dtype != want or not t.is_contiguous() or not t.is_cuda:
                raise ValueError(f"weight {k} must be a contiguous {want} GPU tensor")
        self.desc = ModelDesc(shape.n_layers, shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                              shape.d_ffn, shape.vocab, int(shape.qkv_bias), dt, shape.rms_eps, shape.rope_theta)
        self.w = Weights(*[_ptr(weights.get(k)) for k in _WKEYS])
        h = C.c_void_p()
        check(lib.spec_model_create(C.byref(self.desc), C.byref(self.w), C.byref(h)))
        self.handle = h

    def __del__(self):
        h = getattr(self, "handle", None)
        if h:
            try:
                load().spec_model_destroy(h)
            except Exception:   # interpreter shutdown
                pass
            self.handle = None


class KVCache:
    """K and V arenas [L][B][hkv][capacity][hd] in the model dtype."""

    def __init__(self, shape, batch: int, capacity: int, device="cuda"):
        dt = torch.bfloat16 if shape.dtype == 1 else torch.float32
        dims = (shape.n_layers, batch, shape.n_kv_heads, capacity, shape.head_dim)
        self.k = torch.zeros(dims, dtype=dt, device=device)
        self.v = torch.zeros(dims, dtype=dt, device=device)
        self.capacity, self.batch = capacity, batch
        self.c = KV(self.k.data_ptr(), self.v.data_ptr(), capacity, batch)


def spec_check_pair(draft: SpecModel, base: SpecModel):
    check(load().spec_check_pair(draft.handle, base.handle))


def spec_default_group_plan(n_layers: int, group_size: int) -> list:
    buf = (C.c_int32 * (n_layers + 2))()
    n = C.c_int()
    check(load().spec_default_group_plan(n_layers, group_size, buf, n_layers + 2, C.byref(n)))
    return [int(buf[i]) for i in range(n.value + 1)]


def spec_workspace_bytes(model: SpecModel, batch: int, max_m: int, max_group: int = 1) -> int:
    return int(load().spec_workspace_bytes(model.handle, batch, max_m, max_group))


def spec_accept_workspace_bytes(batch: int, k: int, vocab: int) -> int:
    return int(load().spec_accept_workspace_bytes(batch, k, vocab))


def _plan_array(offsets: Sequence[int]):
    return (C.c_int32 * len(offsets))(*[int(x) for x in offsets])


def spec_draft_group_step(model: SpecModel, kv: KVCache, plan_offsets, flags: int, batch: int,
                          tokens: torch.Tensor, tokens_stride: int, positions: torch.Tensor, max_pos: int,
                          inv_temperature: float, seed: int, logits_out: Optional[torch.Tensor],
                          logits_stride: int, token_out: torch.Tensor, token_out_stride: int,
                          workspace: torch.Tensor, stream=None):
    plan = _plan_array(plan_offsets)
    check(load().spec_draft_group_step(
        model.handle, C.byref(kv.c), plan, len(plan_offsets) - 1, flags, batch, _ptr(tokens), tokens_stride,
        _ptr(positions), max_pos, C.c_float(inv_temperature), C.c_uint64(seed), _ptr(logits_out),
        logits_stride, _ptr(token_out), token_out_stride, _ptr(workspace), workspace.numel(), _stream(stream)))


def spec_draft_group_step_noalloc(model: SpecModel, kv: KVCache, plan_offsets, flags: int, batch: int,
                                  tokens: torch.Tensor, tokens_stride: int, positions: torch.Tensor, max_pos: int,
                                  inv_temperature: float, seed: int, logits_out: Optional[torch.Tensor],
                                  logits_stride: int, token_out: torch.Tensor, token_out_stride: int, stream=None):
    """spec_draft_group_step without a workspace argument: the library's
    per-GPU scratch array serves instead (nothing is allocated)."""
    plan = _plan_array(plan_offsets)
    check(load().spec_draft_group_step_noalloc(
        model.handle, C.byref(kv.c), plan, len(plan_offsets) - 1, flags, batch, _ptr(tokens), tokens_stride,
        _ptr(positions), max_pos, C.c_float(inv_temperature), C.c_uint64(seed), _ptr(logits_out),
        logits_stride, _ptr(token_out), token_out_stride, _stream(stream)))


def spec_draft_attention_cosine(model: SpecModel, kv: KVCache, plan_offsets, batch: int, tokens: torch.Tensor,
                                tokens_stride: int, positions: torch.Tensor, max_pos: int, cos_out: torch.Tensor,
                                cos_stride: int, workspace: torch.Tensor, stream=None):
    plan = _plan_array(plan_offsets)
    check(load().spec_draft_attention_cosine(
        model.handle, C.byref(kv.c), plan, len(plan_offsets) - 1, batch, _ptr(tokens), tokens_stride,
        _ptr(positions), max_pos, _ptr(cos_out), cos_stride, _ptr(workspace), workspace.numel(), _stream(stream)))


def spec_calibrate_kv(model: SpecModel, kv: KVCache, batch: int, tokens: torch.Tensor, start_pos: torch.Tensor,
                      n_tokens: Optional[torch.Tensor], max_m: int, max_pos: int, inv_temperature: float,
                      seed: int, last_logits_out: Optional[torch.Tensor], logits_stride: int,
                      token_out: torch.Tensor, token_out_stride: int, workspace: torch.Tensor, stream=None,
                      tokens_stride: Optional[int] = None):
    """tokens_stride: elements between sequences' token rows (default max_m)."""
    check(load().spec_calibrate_kv(
        model.handle, C.byref(kv.c), batch, _ptr(tokens), max_m if tokens_stride is None else tokens_stride,
        _ptr(start_pos), _ptr(n_tokens), max_m, max_pos,
        C.c_float(inv_temperature), C.c_uint64(seed), _ptr(last_logits_out), logits_stride, _ptr(token_out),
        token_out_stride, _ptr(workspace), workspace.numel(), _stream(stream)))


def spec_verify_forward(model: SpecModel, kv: KVCache, batch: int, tokens: torch.Tensor, start_pos: torch.Tensor,
                        m: int, max_pos: int, logits_out: Optional[torch.Tensor], workspace: torch.Tensor,
                        stream=None):
    check(load().spec_verify_forward(
        model.handle, C.byref(kv.c), batch, _ptr(tokens), _ptr(start_pos), m, max_pos, _ptr(logits_out),
        _ptr(workspace), workspace.numel(), _stream(stream)))


def spec_accept_resample(batch: int, k: int, vocab: int, p_logits: torch.Tensor, q_logits: Optional[torch.Tensor],
                         draft_tokens: Optional[torch.Tensor], draft_stride: int, round_pos: torch.Tensor,
                         inv_temperature: float, seed: int, n_accepted_out: torch.Tensor,
                         next_token_out: torch.Tensor, next_token_stride: int,
                         commit_out: Optional[torch.Tensor], workspace: torch.Tensor, stream=None,
                         draft_offset: int = 0):
    """draft_offset: element offset into draft_tokens (e.g. 1 to skip x_t in
    a [B][k+1] verify-token buffer)."""
    dptr = None if draft_tokens is None else _ptr(draft_tokens) + 4 * draft_offset
    check(load().spec_accept_resample(
        batch, k, vocab, _ptr(p_logits), _ptr(q_logits), dptr, draft_stride, _ptr(round_pos),
        C.c_float(inv_temperature), C.c_uint64(seed), _ptr(n_accepted_out), _ptr(next_token_out),
        next_token_stride, _ptr(commit_out), _ptr(workspace), workspace.numel(), _stream(stream)))


def spec_profile_enable(on: bool):
    check(load().spec_profile_enable(1 if on else 0))


def spec_profile_reset():
    load().spec_profile_reset()


def spec_profile_collect() -> dict:
    """{kernel instance: (launches, total_ms, total_bytes, total_flops)} of
    the launches recorded while profiling was enabled (synchronises their
    events)."""
    lib = load()
    n = lib.spec_profile_collect()
    out = {}
    buf = C.create_string_buffer(256)
    for i in range(n):
        la, ms, by, fl = C.c_int64(), C.c_double(), C.c_double(), C.c_double()
        check(lib.spec_profile_entry(i, buf, 256, C.byref(la), C.byref(ms), C.byref(by), C.byref(fl)))
        out[buf.value.decode()] = (la.value, ms.value, by.value, fl.value)
    return out
