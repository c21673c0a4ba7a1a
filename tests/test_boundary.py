"""C-ABI boundary checks that need no GPU: the library loads, exports every
symbol include/spec.h declares, and rejects bad arguments on the host before
launching anything."""
import ctypes as C
import os
import re

import pytest

import layer_speculative_decoding_amd as L
from layer_speculative_decoding_amd import _lib
from layer_speculative_decoding_amd import api
from oracle.plan import default_group_plan, plan_offsets

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "spec.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert _declared() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = L.load()
    for name in _declared():
        assert hasattr(lib, name), name
    assert lib.spec_version().decode().endswith("gfx950")


@pytest.mark.parametrize("L_,N", [(2, 2), (16, 2), (16, 4), (24, 3), (28, 3), (32, 4), (80, 4), (5, 1), (1, 2), (7, 9)])
def test_c_plan_matches_oracle_plan(L_, N):
    assert api.spec_default_group_plan(L_, N) == plan_offsets(default_group_plan(L_, N))


def _desc(**kw):
    base = dict(n_layers=2, d_model=64, n_q_heads=4, n_kv_heads=2, head_dim=16, d_ffn=128, vocab=256,
                has_qkv_bias=0, dtype=0, rms_eps=1e-5, rope_theta=1e4)
    base.update(kw)
    return _lib.ModelDesc(**base)


def _fake_weights(bias=False):
    # host-side validation only looks at NULL-ness; nothing is dereferenced
    w = _lib.Weights(*([0x1000] * 10))
    if not bias:
        w.bqkv = None
    return w


def _create(desc, w):
    h = C.c_void_p()
    st = L.load().spec_model_create(C.byref(desc), C.byref(w), C.byref(h))
    return st, h


def test_model_create_and_validation():
    lib = L.load()
    st, h = _create(_desc(), _fake_weights())
    assert st == 0 and h
    assert lib.spec_workspace_bytes(h, 1, 8, 2) > 0
    assert lib.spec_workspace_bytes(h, 0, 8, 2) == 0
    lib.spec_model_destroy(h)
    for bad, code in [(dict(head_dim=48), -8), (dict(n_q_heads=3, n_kv_heads=2), -2), (dict(dtype=5), -1),
                      (dict(d_model=68), -2), (dict(vocab=255), -2), (dict(has_qkv_bias=1), -1),
                      (dict(rms_eps=0.0), -1), (dict(n_layers=0), -2)]:
        st, _ = _create(_desc(**bad), _fake_weights())
        assert st == code, (bad, st)
        assert lib.spec_last_error()
    w = _fake_weights()
    w.lm_head = None
    assert _create(_desc(), w)[0] == -1


def test_vocab_mismatch_rejected():
    lib = L.load()
    _, a = _create(_desc(vocab=256), _fake_weights())
    _, b = _create(_desc(vocab=258), _fake_weights())
    assert lib.spec_check_pair(a, b) == -3
    assert b"258" in lib.spec_last_error()
    assert lib.spec_check_pair(a, a) == 0


def _kv(cap=64, batch=1):
    return _lib.KV(0x2000, 0x3000, cap, batch)


def _draft_call(h, kv, offs, **kw):
    args = dict(flags=0, batch=1, tokens=0x4000, tstride=1, positions=0x5000, max_pos=3, invt=0.0,
                logits=0x6000, lstride=256, tok_out=0x7000, ostride=1, ws=0x8000, wsb=1 << 40)
    args.update(kw)
    plan = (C.c_int32 * len(offs))(*offs)
    return L.load().spec_draft_group_step(h, C.byref(kv), plan, len(offs) - 1, args["flags"], args["batch"],
                                          args["tokens"], args["tstride"], args["positions"], args["max_pos"],
                                          args["invt"], 0, args["logits"], args["lstride"], args["tok_out"],
                                          args["ostride"], args["ws"], args["wsb"], None)


def test_draft_step_host_validation():
    _, h = _create(_desc(n_layers=4), _fake_weights())
    kv = _kv()
    assert _draft_call(h, kv, [0, 2, 3]) == -4               # does not cover layer 3
    assert _draft_call(h, kv, [0, 2, 2, 4]) == -4            # empty stage
    assert _draft_call(h, kv, [0, 3, 1, 4]) == -4            # out of order
    assert _draft_call(h, kv, [0, 1, 3, 4], max_pos=64) == -5
    assert _draft_call(h, kv, [0, 1, 3, 4], max_pos=-1) == -5
    assert _draft_call(h, kv, [0, 1, 3, 4], wsb=16) == -6
    assert _draft_call(h, kv, [0, 1, 3, 4], ws=None) == -6
    assert _draft_call(h, kv, [0, 1, 3, 4], flags=7) == -1
    assert _draft_call(h, kv, [0, 1, 3, 4], batch=2) == -2   # kv holds one sequence
    assert _draft_call(h, kv, [0, 1, 3, 4], invt=-1.0) == -1
    assert _draft_call(h, kv, [0, 1, 3, 4], tokens=None) == -1
    assert _draft_call(h, kv, [0, 1, 3, 4], lstride=100) == -1


def test_verify_calibrate_accept_host_validation():
    lib = L.load()
    _, h = _create(_desc(), _fake_weights())
    kv = _kv(cap=16)
    big = 1 << 40
    assert lib.spec_verify_forward(h, C.byref(kv), 1, 0x10, 0x20, 5, 16, 0x30, 0x40, big, None) == -5
    assert lib.spec_verify_forward(h, C.byref(kv), 1, 0x10, 0x20, 0, 3, 0x30, 0x40, big, None) == -1
    assert lib.spec_verify_forward(h, C.byref(kv), 1, None, 0x20, 2, 3, 0x30, 0x40, big, None) == -1
    assert lib.spec_verify_forward(h, C.byref(kv), 1, 0x10, 0x20, 2, 3, 0x30, 0x40, 8, None) == -6
    assert lib.spec_calibrate_kv(h, C.byref(kv), 1, 0x10, 4, 0x20, None, 4, 16, 0.0, 0, None, 0, 0x50, 1, 0x40, big,
                                 None) == -5
    assert lib.spec_calibrate_kv(h, C.byref(kv), 1, 0x10, 1, 0x20, None, 0, 3, 0.0, 0, None, 0, 0x50, 1, 0x40, big,
                                 None) == -1
    assert lib.spec_calibrate_kv(h, C.byref(kv), 1, 0x10, 2, 0x20, None, 2, 3, 0.0, 0, None, 0, None, 1, 0x40, big,
                                 None) == -1
    assert lib.spec_calibrate_kv(h, C.byref(kv), 1, 0x10, 2, 0x20, None, 2, 3, 0.0, 0, 0x60, 100, 0x50, 1, 0x40, big,
                                 None) == -1
    # token rows closer together than max_m
    assert lib.spec_calibrate_kv(h, C.byref(kv), 1, 0x10, 1, 0x20, None, 2, 3, 0.0, 0, None, 0, 0x50, 1, 0x40, big,
                                 None) == -1
    acc = lib.spec_accept_resample
    assert lib.spec_accept_workspace_bytes(1, 4, 256) > 0
    assert acc(1, 65, 256, 0x10, 0x20, 0x30, 65, 0x40, 1.0, 0, 0x50, 0x60, 1, None, 0x70, big, None) == -8
    assert acc(1, 4, 256, 0x10, None, 0x30, 5, 0x40, 1.0, 0, 0x50, 0x60, 1, None, 0x70, big, None) == -1
    assert acc(1, 4, 256, 0x10, 0x20, 0x30, 3, 0x40, 1.0, 0, 0x50, 0x60, 1, None, 0x70, big, None) == -1
    assert acc(1, 4, 256, 0x10, 0x20, 0x30, 5, 0x40, 1.0, 0, 0x50, 0x60, 1, None, 0x70, 4, None) == -6
    assert acc(0, 4, 256, 0x10, 0x20, 0x30, 5, 0x40, 1.0, 0, 0x50, 0x60, 1, None, 0x70, big, None) == -2
    assert acc(1, 4, 256, 0x10, 0x20, 0x30, 5, 0x40, -2.0, 0, 0x50, 0x60, 1, None, 0x70, big, None) == -1


def test_status_strings():
    lib = L.load()
    for code in _lib.STATUS:
        assert lib.spec_status_string(code)


def test_noalloc_draft_step_rejects_before_touching_the_gpu():
    """The entry point that allocates nothing rejects plans and shapes whose
    workspace would not fit its scratch array, on the host, before any HIP
    call (there is no GPU here)."""
    lib = L.load()
    big = _desc(n_layers=10, d_model=8192, n_q_heads=64, n_kv_heads=8, head_dim=128, d_ffn=28672, vocab=1024,
                dtype=1)
    _, h = _create(big, _fake_weights())
    kv = _kv(cap=64, batch=8)
    plan = [0, 1, 9, 10]                            # one set of 8 layers
    need = lib.spec_workspace_bytes(h, 8, 1, 8)
    assert need > _lib.SPEC_SCRATCH_BYTES
    arr = (C.c_int32 * len(plan))(*plan)
    st = lib.spec_draft_group_step_noalloc(h, C.byref(kv), arr, 3, 0, 8, 0x4000, 1, 0x5000, 3, 0.0, 0, None, 0,
                                           0x7000, 1, None)
    assert st == -6
    assert b"scratch" in lib.spec_last_error()
    bad = (C.c_int32 * 3)(0, 2, 9)                  # does not cover the last layer
    assert lib.spec_draft_group_step_noalloc(h, C.byref(kv), bad, 2, 0, 8, 0x4000, 1, 0x5000, 3, 0.0, 0, None, 0,
                                             0x7000, 1, None) == -4
