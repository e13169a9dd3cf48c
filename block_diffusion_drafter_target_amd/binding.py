"""ctypes binding of libdflash.so: the C ABI's structs and entry points.

Argument marshalling only. Device buffers are torch tensors (their data
pointers are passed through); every step of the draft step runs in the HIP
kernels of the library. Loading fails loudly when the library is missing.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# DFLASH_LIB selects another build of the library (the sanitized one of the
# CPU tests); by default the in-tree libdflash.so
LIB_PATH = os.environ.get("DFLASH_LIB") or os.path.join(HERE, "libdflash.so")

DFLASH_OK = 0
DFLASH_ERR_NULL = -1
DFLASH_ERR_SHAPE = -2
DFLASH_ERR_UNSUPPORTED = -3
DFLASH_ERR_WORKSPACE = -4
DFLASH_ERR_CAPACITY = -5
DFLASH_ERR_HIP = -6

EXPORTED = ("dflash_model_create", "dflash_model_destroy", "dflash_rope_table",
            "dflash_workspace_bytes", "dflash_fuse_ctx", "dflash_inject_kv",
            "dflash_draft_block", "dflash_verify_accept", "dflash_status_string",
            "dflash_profile_enable", "dflash_profile_read", "dflash_pack_matrix",
            "dflash_target_create", "dflash_target_forward", "dflash_kv_commit",
            "dflash_draft_block_sample", "dflash_verify_sample", "dflash_sample_logits",
            "dflash_draft_block_noalloc", "dflash_loop_tokens", "dflash_loop_advance",
            "dflash_ingest_rows", "dflash_profile_pause")

# bytes of the static device workspace behind dflash_draft_block_noalloc
NOALLOC_SCRATCH_BYTES = 64 << 20

PHASES = {"lm_head": 0, "attention": 1, "qkv": 2, "o": 3, "gate_up": 4, "down": 5, "fuse": 6,
          "inject": 7, "verify": 8, "merge": 9}


class dflash_config(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_layers", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("intermediate", C.c_int32),
                ("vocab", C.c_int32), ("n_tap", C.c_int32), ("block", C.c_int32),
                ("mask_id", C.c_int32), ("rope_theta", C.c_float), ("rms_eps", C.c_float)]


class dflash_layer_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("g_in", "w_qkv", "g_q", "g_k", "w_o", "g_post",
                                          "w_gate", "w_up", "w_down")]


class dflash_weights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("lm_head", C.c_void_p), ("w_fc", C.c_void_p),
                ("g_fc", C.c_void_p), ("g_final", C.c_void_p),
                ("layers", C.POINTER(dflash_layer_weights)), ("rope", C.c_void_p),
                ("rope_max_pos", C.c_int32)]


class dflash_kv(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("batch", C.c_int32),
                ("max_ctx", C.c_int32), ("ctx_len", C.c_void_p), ("status", C.c_void_p)]


class DFlashError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {status_string(code)} ({code})")
        self.code = code


_lib = None


def load() -> C.CDLL:
    """Load the built library (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: run `python -m block_diffusion_drafter_target_amd.build`")
    lib = C.CDLL(LIB_PATH)
    vp, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
    lib.dflash_model_create.argtypes = [C.POINTER(dflash_config), C.POINTER(dflash_weights), C.POINTER(vp)]
    lib.dflash_model_destroy.argtypes = [vp]
    lib.dflash_model_destroy.restype = None
    lib.dflash_rope_table.argtypes = [vp, i32, i32, C.c_float]
    lib.dflash_workspace_bytes.argtypes = [vp, i32, i32, i32]
    lib.dflash_workspace_bytes.restype = sz
    lib.dflash_fuse_ctx.argtypes = [vp, vp, i32, vp, vp, sz, vp]
    lib.dflash_inject_kv.argtypes = [vp, vp, i32, vp, vp, i32, C.POINTER(dflash_kv), vp, sz, vp]
    lib.dflash_draft_block.argtypes = [vp, C.POINTER(dflash_kv), vp, vp, vp, vp, vp, sz, vp]
    lib.dflash_draft_block_noalloc.argtypes = [vp, C.POINTER(dflash_kv), vp, vp, vp, vp, vp]
    lib.dflash_loop_tokens.argtypes = [vp, C.POINTER(dflash_kv), vp, vp, vp, vp]
    lib.dflash_ingest_rows.argtypes = [vp, C.POINTER(dflash_kv), i32, i32, i32, vp, vp, vp]
    lib.dflash_loop_advance.argtypes = [vp, C.POINTER(dflash_kv), vp, vp, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp]
    lib.dflash_target_create.argtypes = [C.POINTER(dflash_config), C.POINTER(dflash_weights), vp, C.POINTER(vp)]
    lib.dflash_target_forward.argtypes = [vp, C.POINTER(dflash_kv), vp, i32, vp, vp, vp, vp, sz, vp]
    lib.dflash_kv_commit.argtypes = [vp, C.POINTER(dflash_kv), vp, vp, i32, vp]
    lib.dflash_verify_accept.argtypes = [vp, C.POINTER(dflash_kv), vp, vp, vp, i32, vp, vp, vp, vp,
                                         vp, vp, vp, vp, vp]
    u64, f32 = C.c_uint64, C.c_float
    lib.dflash_draft_block_sample.argtypes = [vp, C.POINTER(dflash_kv), vp, vp, vp, f32, u64, i32, vp, vp, sz, vp]
    lib.dflash_verify_sample.argtypes = [vp, C.POINTER(dflash_kv), vp, vp, vp, f32, u64, i32, vp, vp, i32, vp, vp,
                                         vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.dflash_sample_logits.argtypes = [vp, vp, i32, f32, u64, i32, i32, vp, vp, sz, vp]
    lib.dflash_pack_matrix.argtypes = [vp, vp, i32, i32, vp]
    lib.dflash_pack_matrix.restype = i32
    lib.dflash_profile_enable.argtypes = [C.c_uint32]
    lib.dflash_profile_enable.restype = i32
    lib.dflash_profile_read.argtypes = [i32, C.POINTER(C.c_double), C.POINTER(C.c_int32)]
    lib.dflash_profile_read.restype = i32
    lib.dflash_profile_pause.argtypes = [i32]
    lib.dflash_profile_pause.restype = i32
    lib.dflash_status_string.argtypes = [i32]
    lib.dflash_status_string.restype = C.c_char_p
    for fn in ("dflash_model_create", "dflash_rope_table", "dflash_fuse_ctx", "dflash_inject_kv",
               "dflash_draft_block", "dflash_verify_accept", "dflash_target_create",
               "dflash_target_forward", "dflash_kv_commit", "dflash_draft_block_sample",
               "dflash_verify_sample", "dflash_sample_logits", "dflash_draft_block_noalloc",
               "dflash_loop_tokens", "dflash_loop_advance", "dflash_ingest_rows"):
        getattr(lib, fn).restype = i32
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().dflash_status_string(int(code)).decode()


def _check(fn: str, code: int) -> int:
    if code != DFLASH_OK:
        raise DFlashError(fn, code)
    return code


def ptr(t) -> int | None:
    """Data pointer of a tensor (or None)."""
    if t is None:
        return None
    return t.data_ptr()


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI; raise DFlashError on a nonzero status)
# ---------------------------------------------------------------------------

def dflash_model_create(cfg: dflash_config, w: dflash_weights) -> int:
    h = C.c_void_p()
    _check("dflash_model_create", load().dflash_model_create(C.byref(cfg), C.byref(w), C.byref(h)))
    return h.value


def dflash_target_create(cfg: dflash_config, w: dflash_weights, tap_layers) -> int:
    taps = (C.c_int32 * len(tap_layers))(*[int(t) for t in tap_layers])
    h = C.c_void_p()
    _check("dflash_target_create", load().dflash_target_create(C.byref(cfg), C.byref(w), taps, C.byref(h)))
    return h.value


def dflash_model_destroy(model: int) -> None:
    load().dflash_model_destroy(model)


def dflash_rope_table(out_host, max_pos: int, head_dim: int, theta: float) -> None:
    _check("dflash_rope_table", load().dflash_rope_table(out_host, max_pos, head_dim, theta))


def dflash_workspace_bytes(model: int, max_batch: int, max_ctx: int, max_rows: int) -> int:
    return int(load().dflash_workspace_bytes(model, max_batch, max_ctx, max_rows))


def dflash_fuse_ctx(model, taps, n_rows, ctx, ws, ws_bytes, stream) -> None:
    _check("dflash_fuse_ctx", load().dflash_fuse_ctx(model, taps, n_rows, ctx, ws, ws_bytes, stream))


def dflash_inject_kv(model, ctx, n_ctx_rows, commit_rows, n_commit, max_commit, kv, ws, ws_bytes,
                     stream) -> None:
    _check("dflash_inject_kv", load().dflash_inject_kv(model, ctx, n_ctx_rows, commit_rows, n_commit,
                                                       max_commit, C.byref(kv), ws, ws_bytes, stream))


def dflash_draft_block(model, kv, anchor, draft, dbg_logits, dbg_hidden, ws, ws_bytes, stream) -> None:
    _check("dflash_draft_block", load().dflash_draft_block(model, C.byref(kv), anchor, draft, dbg_logits,
                                                           dbg_hidden, ws, ws_bytes, stream))


def dflash_draft_block_noalloc(model, kv, anchor, draft, dbg_logits, dbg_hidden, stream) -> None:
    _check("dflash_draft_block_noalloc", load().dflash_draft_block_noalloc(model, C.byref(kv), anchor, draft,
                                                                           dbg_logits, dbg_hidden, stream))


def dflash_ingest_rows(model, kv, seq: int, start: int, n: int, commit_rows, n_commit, stream) -> None:
    _check("dflash_ingest_rows", load().dflash_ingest_rows(model, C.byref(kv), seq, start, n, commit_rows, n_commit,
                                                           stream))


def dflash_loop_tokens(model, kv, anchor, draft, tokens, stream) -> None:
    _check("dflash_loop_tokens", load().dflash_loop_tokens(model, C.byref(kv), anchor, draft, tokens, stream))


def dflash_loop_advance(model, kv, anchor_out, emitted, n_emit, done, out, ld_out: int, max_new: int, cursor,
                        alive, anchor, step_dev, stream) -> None:
    _check("dflash_loop_advance", load().dflash_loop_advance(model, C.byref(kv), anchor_out, emitted, n_emit, done,
                                                             out, ld_out, max_new, cursor, alive, anchor, step_dev,
                                                             stream))


def dflash_target_forward(model, kv, tokens, n, argmax, taps, dbg_logits, ws, ws_bytes, stream) -> None:
    _check("dflash_target_forward", load().dflash_target_forward(model, C.byref(kv), tokens, n, argmax, taps,
                                                                 dbg_logits, ws, ws_bytes, stream))


def dflash_kv_commit(model, kv, commit_rows, n_commit, max_commit, stream) -> None:
    _check("dflash_kv_commit", load().dflash_kv_commit(model, C.byref(kv), commit_rows, n_commit, max_commit,
                                                       stream))


def dflash_verify_accept(model, kv, draft, target_argmax, stop_ids, n_stop, budget, accept_len,
                         anchor_out, emitted, n_emit, done, commit_rows, n_commit, stream) -> None:
    _check("dflash_verify_accept", load().dflash_verify_accept(
        model, C.byref(kv), draft, target_argmax, stop_ids, n_stop, budget, accept_len, anchor_out,
        emitted, n_emit, done, commit_rows, n_commit, stream))


def dflash_draft_block_sample(model, kv, anchor, draft, logits, temperature: float, seed: int, step: int,
                              step_dev, ws, ws_bytes, stream) -> None:
    _check("dflash_draft_block_sample", load().dflash_draft_block_sample(
        model, C.byref(kv), anchor, draft, logits, temperature, seed, step, step_dev, ws, ws_bytes, stream))


def dflash_verify_sample(model, kv, draft, draft_logits, target_logits, temperature: float, seed: int, step: int,
                         step_dev, stop_ids, n_stop, budget, accept_len, anchor_out, emitted, n_emit, done,
                         commit_rows, n_commit, ws, ws_bytes, stream) -> None:
    _check("dflash_verify_sample", load().dflash_verify_sample(
        model, C.byref(kv), draft, draft_logits, target_logits, temperature, seed, step, step_dev, stop_ids,
        n_stop, budget, accept_len, anchor_out, emitted, n_emit, done, commit_rows, n_commit, ws, ws_bytes,
        stream))


def dflash_sample_logits(model, logits, rows: int, temperature: float, seed: int, step: int, row0: int, tokens,
                         ws, ws_bytes, stream) -> None:
    _check("dflash_sample_logits", load().dflash_sample_logits(model, logits, rows, temperature, seed, step, row0,
                                                               tokens, ws, ws_bytes, stream))


def dflash_pack_matrix(src, dst, rows: int, cols: int, stream) -> None:
    _check("dflash_pack_matrix", load().dflash_pack_matrix(src, dst, rows, cols, stream))


def dflash_profile_enable(phases=()) -> None:
    """Time the named phases (an empty list switches timing off)."""
    mask = 0
    for p in phases:
        mask |= 1 << (PHASES[p] if isinstance(p, str) else int(p))
    _check("dflash_profile_enable", load().dflash_profile_enable(mask))


def dflash_profile_pause(paused: bool) -> None:
    """Stop (True) or resume (False) recording phase events; records and mask are kept."""
    _check("dflash_profile_pause", load().dflash_profile_pause(1 if paused else 0))


def dflash_profile_read(phase) -> tuple[float, int]:
    """(summed ms, launches) of one phase (name or id) since profiling was enabled."""
    pid = PHASES[phase] if isinstance(phase, str) else int(phase)
    t, n = C.c_double(), C.c_int32()
    _check("dflash_profile_read", load().dflash_profile_read(pid, C.byref(t), C.byref(n)))
    return t.value, n.value
