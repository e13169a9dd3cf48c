"""C ABI checks that need no GPU: the library loads, exports every entry point
that include/dflash.h declares, and rejects bad arguments before any HIP call."""
import ctypes as C
import math
import os
import re

import numpy as np
import pytest

from block_diffusion_drafter_target_amd import binding as bd
from block_diffusion_drafter_target_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "dflash.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_[a-z_]+)\s*\(", src)))


def test_header_declares_the_step_calls():
    names = declared_functions()
    for n in ("dflash_fuse_ctx", "dflash_inject_kv", "dflash_draft_block", "dflash_verify_accept"):
        assert n in names
    assert set(names) == set(bd.EXPORTED)


def test_loaded_library_is_the_selected_build():
    lib = bd.load()
    assert os.path.realpath(lib._name) == os.path.realpath(bd.LIB_PATH)
    if os.environ.get("DFLASH_LIB"):  # the sanitized build: its runtime is in the process
        assert hasattr(C.CDLL(None), "__asan_init")


def test_library_exports_every_declared_symbol():
    lib = bd.load()
    for n in declared_functions():
        assert hasattr(lib, n), n


def _cfg(**kw):
    c = synth.CONFIGS["c2"]
    d = dict(hidden=c.hidden, n_layers=c.n_layers, n_q_heads=c.n_q_heads, n_kv_heads=c.n_kv_heads,
             head_dim=c.head_dim, intermediate=c.intermediate, vocab=c.vocab, n_tap=c.n_tap,
             block=c.block, mask_id=c.mask_id, rope_theta=c.rope_theta, rms_eps=c.rms_eps)
    d.update(kw)
    return bd.dflash_config(**d)


def _fake_weights(n_layers):
    # non-null dummy addresses: create never dereferences them
    layers = (bd.dflash_layer_weights * n_layers)()
    for l in range(n_layers):
        for f in ("g_in", "w_qkv", "g_q", "g_k", "w_o", "g_post", "w_gate", "w_up", "w_down"):
            setattr(layers[l], f, 0x1000)
    w = bd.dflash_weights(embed=0x1000, lm_head=0x1000, w_fc=0x1000, g_fc=0x1000, g_final=0x1000,
                          layers=layers, rope=0x1000, rope_max_pos=4096)
    return w, layers


def _create(cfg, w):
    h = C.c_void_p()
    rc = bd.load().dflash_model_create(C.byref(cfg), C.byref(w), C.byref(h))
    return rc, h.value


def test_model_create_validation():
    w, keep = _fake_weights(5)
    rc, h = _create(_cfg(), w)
    assert rc == bd.DFLASH_OK and h
    bd.dflash_model_destroy(h)
    bad = {
        "head_dim": (96, bd.DFLASH_ERR_UNSUPPORTED),
        "block": (17, bd.DFLASH_ERR_UNSUPPORTED),
        "n_kv_heads": (7, bd.DFLASH_ERR_SHAPE),
        "hidden": (4000, bd.DFLASH_ERR_UNSUPPORTED),
        "mask_id": (151936, bd.DFLASH_ERR_SHAPE),
        "vocab": (151937, bd.DFLASH_ERR_UNSUPPORTED),
        "n_layers": (17, bd.DFLASH_ERR_UNSUPPORTED),
        "rms_eps": (0.0, bd.DFLASH_ERR_SHAPE),
    }
    for field, (val, code) in bad.items():
        rc, h = _create(_cfg(**{field: val}), w)
        assert rc == code, field
        assert not h
    w.w_fc = None
    assert _create(_cfg(), w)[0] == bd.DFLASH_ERR_NULL
    w, keep = _fake_weights(5)
    keep[3].w_down = None
    assert _create(_cfg(), w)[0] == bd.DFLASH_ERR_NULL


def test_calls_reject_bad_arguments_without_a_gpu():
    lib = bd.load()
    w, keep = _fake_weights(5)
    rc, h = _create(_cfg(), w)
    assert rc == 0
    try:
        ws_need = bd.dflash_workspace_bytes(h, 1, 2048, 16)
        assert ws_need > 0
        assert bd.dflash_workspace_bytes(h, 8, 2048, 16) > ws_need
        kv = bd.dflash_kv(k=0x1000, v=0x1000, batch=1, max_ctx=2048, ctx_len=0x1000, status=0x1000)
        # workspace too small
        assert lib.dflash_draft_block(h, C.byref(kv), 0x1000, 0x1000, None, None, 0x1000,
                                      ws_need - 1, None) == bd.DFLASH_ERR_WORKSPACE
        # null pointers
        assert lib.dflash_draft_block(h, C.byref(kv), None, 0x1000, None, None, 0x1000,
                                      ws_need, None) == bd.DFLASH_ERR_NULL
        assert lib.dflash_draft_block(None, C.byref(kv), 0x1000, 0x1000, None, None, 0x1000,
                                      ws_need, None) == bd.DFLASH_ERR_NULL
        # cache smaller than one block, batch out of range
        small = bd.dflash_kv(k=0x1000, v=0x1000, batch=1, max_ctx=8, ctx_len=0x1000, status=0x1000)
        assert lib.dflash_draft_block(h, C.byref(small), 0x1000, 0x1000, None, None, 0x1000,
                                      ws_need, None) == bd.DFLASH_ERR_SHAPE
        big = bd.dflash_kv(k=0x1000, v=0x1000, batch=5000, max_ctx=2048, ctx_len=0x1000, status=0x1000)
        assert lib.dflash_draft_block(h, C.byref(big), 0x1000, 0x1000, None, None, 0x1000,
                                      1 << 40, None) == bd.DFLASH_ERR_SHAPE
        # fuse: zero rows is a no-op, negative rows a shape error, tiny workspace rejected
        assert lib.dflash_fuse_ctx(h, None, 0, None, None, 0, None) == bd.DFLASH_OK
        assert lib.dflash_fuse_ctx(h, 0x1000, -1, 0x1000, 0x1000, 1 << 30, None) == bd.DFLASH_ERR_SHAPE
        assert lib.dflash_fuse_ctx(h, 0x1000, 16, 0x1000, 0x1000, 16, None) == bd.DFLASH_ERR_WORKSPACE
        # inject: nothing to commit is a no-op; missing count pointer rejected
        assert lib.dflash_inject_kv(h, 0x1000, 16, 0x1000, 0x1000, 0, C.byref(kv), 0x1000, 1 << 30,
                                    None) == bd.DFLASH_OK
        assert lib.dflash_inject_kv(h, 0x1000, 16, 0x1000, None, 16, C.byref(kv), 0x1000, 1 << 30,
                                    None) == bd.DFLASH_ERR_NULL
        assert lib.dflash_inject_kv(h, 0x1000, 16, 0x1000, 0x1000, 16, C.byref(kv), 0x1000, 16,
                                    None) == bd.DFLASH_ERR_WORKSPACE
        # context rows beyond 32-bit element offsets (2^31 / 4096 rows)
        assert lib.dflash_inject_kv(h, 0x1000, (1 << 31) // 4096 + 1, 0x1000, 0x1000, 16, C.byref(kv), 0x1000,
                                    1 << 30, None) == bd.DFLASH_ERR_UNSUPPORTED
        # verify: negative stop count, stop ids missing
        args = [0x1000] * 2
        outs = [0x1000] * 7
        assert lib.dflash_verify_accept(h, C.byref(kv), *args, None, -1, None, *outs, None) == bd.DFLASH_ERR_SHAPE
        assert lib.dflash_verify_accept(h, C.byref(kv), *args, None, 2, None, *outs, None) == bd.DFLASH_ERR_NULL
        assert lib.dflash_verify_accept(h, C.byref(kv), None, 0x1000, None, 0, None, *outs,
                                        None) == bd.DFLASH_ERR_NULL
    finally:
        bd.dflash_model_destroy(h)


def _create_target(cfg, w, taps):
    h = C.c_void_p()
    arr = (C.c_int32 * len(taps))(*taps)
    rc = bd.load().dflash_target_create(C.byref(cfg), C.byref(w), arr, C.byref(h))
    return rc, h.value


def test_target_create_and_calls_without_a_gpu():
    lib = bd.load()
    # a 36-layer Qwen3-8B-shaped target tapping 5 layers, passes of up to 16 tokens;
    # the drafter's fusion weights are not needed
    w, keep = _fake_weights(36)
    w.w_fc = None
    w.g_fc = None
    taps = [1, 9, 17, 25, 33]
    rc, h = _create_target(_cfg(n_layers=36), w, taps)
    assert rc == bd.DFLASH_OK and h
    try:
        need16 = bd.dflash_workspace_bytes(h, 1, 2048, 0)
        assert need16 > 0
        kv = bd.dflash_kv(k=0x1000, v=0x1000, batch=1, max_ctx=2048, ctx_len=0x1000, status=0x1000)
        f = lib.dflash_target_forward
        assert f(h, C.byref(kv), 0x1000, 0, 0x1000, None, None, 0x1000, need16, None) == bd.DFLASH_ERR_SHAPE
        assert f(h, C.byref(kv), 0x1000, 17, 0x1000, None, None, 0x1000, need16, None) == bd.DFLASH_ERR_SHAPE
        assert f(h, C.byref(kv), None, 4, 0x1000, None, None, 0x1000, need16, None) == bd.DFLASH_ERR_NULL
        assert f(h, C.byref(kv), 0x1000, 16, 0x1000, None, None, 0x1000, 64, None) == bd.DFLASH_ERR_WORKSPACE
        # the drafter entry points refuse a target model
        assert lib.dflash_draft_block(h, C.byref(kv), 0x1000, 0x1000, None, None, 0x1000, need16,
                                      None) == bd.DFLASH_ERR_UNSUPPORTED
        assert lib.dflash_fuse_ctx(h, 0x1000, 16, 0x1000, 0x1000, 1 << 30, None) == bd.DFLASH_ERR_UNSUPPORTED
        assert lib.dflash_verify_accept(h, C.byref(kv), 0x1000, 0x1000, None, 0, None,
                                        *([0x1000] * 7), None) == bd.DFLASH_ERR_UNSUPPORTED
        # commit: nothing to commit is a no-op, missing count rejected
        assert lib.dflash_kv_commit(h, C.byref(kv), None, None, 0, None) == bd.DFLASH_OK
        assert lib.dflash_kv_commit(h, C.byref(kv), 0x1000, None, 4, None) == bd.DFLASH_ERR_NULL
        assert lib.dflash_kv_commit(h, C.byref(kv), 0x1000, 0x1000, -1, None) == bd.DFLASH_ERR_SHAPE
    finally:
        bd.dflash_model_destroy(h)
    # a drafter cannot be asked for a target pass
    wd, keepd = _fake_weights(5)
    rc, hd = _create(_cfg(), wd)
    assert rc == 0
    try:
        kv = bd.dflash_kv(k=0x1000, v=0x1000, batch=1, max_ctx=2048, ctx_len=0x1000, status=0x1000)
        assert lib.dflash_target_forward(hd, C.byref(kv), 0x1000, 4, 0x1000, None, None, 0x1000, 1 << 30,
                                         None) == bd.DFLASH_ERR_UNSUPPORTED
    finally:
        bd.dflash_model_destroy(hd)
    # tap layers must be increasing and inside the stack; passes of at most 64 tokens
    for t, code in (([1, 9, 9, 25, 33], bd.DFLASH_ERR_SHAPE), ([1, 9, 17, 25, 36], bd.DFLASH_ERR_SHAPE),
                    ([-1, 9, 17, 25, 33], bd.DFLASH_ERR_SHAPE)):
        assert _create_target(_cfg(n_layers=36), w, t)[0] == code
    assert _create_target(_cfg(n_layers=36, block=65), w, taps)[0] == bd.DFLASH_ERR_UNSUPPORTED
    assert _create_target(_cfg(n_layers=257), _fake_weights(257)[0], taps)[0] == bd.DFLASH_ERR_UNSUPPORTED


def test_rope_table_values():
    max_pos, D, theta = 300, 64, 1e6
    out = np.empty(max_pos * D // 2 * 2, np.float32)
    bd.dflash_rope_table(out.ctypes.data_as(C.c_void_p), max_pos, D, theta)
    out = out.reshape(max_pos, D // 2, 2)
    for p in (0, 1, 17, 299):
        for i in (0, 1, 5, 31):
            ang = p * theta ** (-2.0 * i / D)
            assert out[p, i, 0] == np.float32(math.cos(ang))
            assert out[p, i, 1] == np.float32(math.sin(ang))
    assert bd.load().dflash_rope_table(None, 4, 64, 1e6) == bd.DFLASH_ERR_NULL
    assert bd.load().dflash_rope_table(out.ctypes.data_as(C.c_void_p), 4, 63, 1e6) == bd.DFLASH_ERR_SHAPE


def test_profile_controls_without_a_gpu():
    # enabling, pausing, resuming and reading record nothing without a launch
    bd.dflash_profile_enable(["lm_head"])
    bd.dflash_profile_pause(True)
    bd.dflash_profile_pause(False)
    assert bd.dflash_profile_read("lm_head") == (0.0, 0)
    bd.dflash_profile_enable([])
    assert bd.load().dflash_profile_read(99, bd.C.byref(bd.C.c_double()), bd.C.byref(bd.C.c_int32())) == bd.DFLASH_ERR_SHAPE


def test_status_strings():
    assert bd.status_string(0) == "ok"
    assert "workspace" in bd.status_string(bd.DFLASH_ERR_WORKSPACE)


def test_sampling_entry_points_check_arguments_without_a_gpu():
    """Argument checks of the sampling-mode entry points run on the host and
    return before any HIP call."""
    lib = bd.load()
    w, keep = _fake_weights(5)
    rc, h = _create(_cfg(), w)
    assert rc == bd.DFLASH_OK
    try:
        kv = bd.dflash_kv(k=0x1000, v=0x1000, batch=2, max_ctx=2048, ctx_len=0x1000, status=0x1000)
        ws = bd.dflash_workspace_bytes(h, 2, 2048, 32)
        P = 0x1000
        ds = lib.dflash_draft_block_sample
        assert ds(h, C.byref(kv), P, P, None, 1.0, 7, 1, None, P, ws, None) == bd.DFLASH_ERR_NULL  # logits
        for t in (0.0, -1.0, float("nan"), float("inf")):
            assert ds(h, C.byref(kv), P, P, P, t, 7, 1, None, P, ws, None) == bd.DFLASH_ERR_SHAPE
        assert ds(h, C.byref(kv), P, P, P, 1.0, 7, 1, None, P, 16, None) == bd.DFLASH_ERR_WORKSPACE
        vs = lib.dflash_verify_sample
        args = [P, P, P, 1.0, 7, 1, None, None, 0, None] + [P] * 7 + [P, ws, None]
        bad = list(args)
        bad[1] = None  # draft logits
        assert vs(h, C.byref(kv), *bad) == bd.DFLASH_ERR_NULL
        bad = list(args)
        bad[3] = 0.0
        assert vs(h, C.byref(kv), *bad) == bd.DFLASH_ERR_SHAPE
        bad = list(args)
        bad[8] = -1  # n_stop
        assert vs(h, C.byref(kv), *bad) == bd.DFLASH_ERR_SHAPE
        bad = list(args)
        bad[8] = 2  # stop ids missing
        assert vs(h, C.byref(kv), *bad) == bd.DFLASH_ERR_NULL
        bad = list(args)
        bad[-2] = 64
        assert vs(h, C.byref(kv), *bad) == bd.DFLASH_ERR_WORKSPACE
        sl = lib.dflash_sample_logits
        assert sl(h, P, 0, 1.0, 7, 0, 0, P, P, ws, None) == bd.DFLASH_OK  # nothing to sample
        assert sl(h, P, -1, 1.0, 7, 0, 0, P, P, ws, None) == bd.DFLASH_ERR_SHAPE
        assert sl(h, None, 3, 1.0, 7, 0, 0, P, P, ws, None) == bd.DFLASH_ERR_NULL
        assert sl(h, P, 3, 0.0, 7, 0, 0, P, P, ws, None) == bd.DFLASH_ERR_SHAPE
        assert sl(h, P, 3, 1.0, 7, 0, 0, P, P, 8, None) == bd.DFLASH_ERR_WORKSPACE
    finally:
        bd.dflash_model_destroy(h)


def test_noalloc_draft_block_checks_without_a_gpu():
    """The allocation-free draft block runs the draft block's checks and
    rejects a pass whose workspace exceeds its static array, all before any
    HIP call."""
    src = open(os.path.join(ROOT, "include", "dflash.h")).read()
    m = re.search(r"#define DFLASH_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == bd.NOALLOC_SCRATCH_BYTES
    lib = bd.load()
    w, keep = _fake_weights(5)
    rc, h = _create(_cfg(), w)
    assert rc == 0
    try:
        # Qwen3-8B-shaped drafter at batch 32 with 4096-key contexts: ~118 MiB
        kv = bd.dflash_kv(k=0x1000, v=0x1000, batch=32, max_ctx=4096 + 64, ctx_len=0x1000, status=0x1000)
        assert bd.dflash_workspace_bytes(h, 32, 4096 + 64, 1) > bd.NOALLOC_SCRATCH_BYTES
        assert lib.dflash_draft_block_noalloc(h, C.byref(kv), 0x1000, 0x1000, None, None,
                                              None) == bd.DFLASH_ERR_WORKSPACE
        one = bd.dflash_kv(k=0x1000, v=0x1000, batch=1, max_ctx=2048, ctx_len=0x1000, status=0x1000)
        assert bd.dflash_workspace_bytes(h, 1, 2048, 1) < bd.NOALLOC_SCRATCH_BYTES
        assert lib.dflash_draft_block_noalloc(h, C.byref(one), None, 0x1000, None, None,
                                              None) == bd.DFLASH_ERR_NULL
        assert lib.dflash_draft_block_noalloc(h, C.byref(one), 0x1000, None, None, None,
                                              None) == bd.DFLASH_ERR_NULL
        assert lib.dflash_draft_block_noalloc(None, C.byref(one), 0x1000, 0x1000, None, None,
                                              None) == bd.DFLASH_ERR_NULL
        small = bd.dflash_kv(k=0x1000, v=0x1000, batch=1, max_ctx=8, ctx_len=0x1000, status=0x1000)
        assert lib.dflash_draft_block_noalloc(h, C.byref(small), 0x1000, 0x1000, None, None,
                                              None) == bd.DFLASH_ERR_SHAPE
    finally:
        bd.dflash_model_destroy(h)


def test_loop_entry_points_check_arguments_without_a_gpu():
    lib = bd.load()
    w, keep = _fake_weights(5)
    rc, h = _create(_cfg(), w)
    assert rc == 0
    try:
        kv = bd.dflash_kv(k=0x1000, v=0x1000, batch=2, max_ctx=2048, ctx_len=0x1000, status=0x1000)
        p = 0x1000
        assert lib.dflash_loop_tokens(h, C.byref(kv), None, p, p, None) == bd.DFLASH_ERR_NULL
        assert lib.dflash_loop_tokens(h, C.byref(kv), p, p, None, None) == bd.DFLASH_ERR_NULL
        bad = bd.dflash_kv(k=0x1000, v=0x1000, batch=0, max_ctx=2048, ctx_len=0x1000, status=0x1000)
        assert lib.dflash_loop_tokens(h, C.byref(bad), p, p, p, None) == bd.DFLASH_ERR_SHAPE
        # out row stride below the token budget; negative budget; missing cursor
        assert lib.dflash_loop_advance(h, C.byref(kv), p, p, p, p, p, 10, 11, p, p, p, None,
                                       None) == bd.DFLASH_ERR_SHAPE
        assert lib.dflash_loop_advance(h, C.byref(kv), p, p, p, p, p, 10, -1, p, p, p, None,
                                       None) == bd.DFLASH_ERR_SHAPE
        assert lib.dflash_loop_advance(h, C.byref(kv), p, p, p, p, p, 10, 10, None, p, p, None,
                                       None) == bd.DFLASH_ERR_NULL
        # ingest rows: sequence out of range, negative start or count, past the cache, null outputs
        assert lib.dflash_ingest_rows(h, C.byref(kv), 2, 0, 4, p, p, None) == bd.DFLASH_ERR_SHAPE
        assert lib.dflash_ingest_rows(h, C.byref(kv), -1, 0, 4, p, p, None) == bd.DFLASH_ERR_SHAPE
        assert lib.dflash_ingest_rows(h, C.byref(kv), 0, -1, 4, p, p, None) == bd.DFLASH_ERR_SHAPE
        assert lib.dflash_ingest_rows(h, C.byref(kv), 0, 0, -4, p, p, None) == bd.DFLASH_ERR_SHAPE
        assert lib.dflash_ingest_rows(h, C.byref(kv), 1, 2040, 9, p, p, None) == bd.DFLASH_ERR_SHAPE
        assert lib.dflash_ingest_rows(h, C.byref(kv), 0, 0, 4, None, p, None) == bd.DFLASH_ERR_NULL
        assert lib.dflash_ingest_rows(h, C.byref(kv), 0, 0, 4, p, None, None) == bd.DFLASH_ERR_NULL
    finally:
        bd.dflash_model_destroy(h)
