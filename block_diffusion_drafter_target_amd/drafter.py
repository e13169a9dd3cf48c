"""Device-resident drafter over the C ABI, and the greedy speculative loop.

``Drafter`` owns torch device buffers (weights, draft KV cache, workspace,
per-step outputs) and a model handle; each method marshals pointers to one
C entry point. ``DeviceTarget`` does the same for a target model (causal
passes that emit taps and argmax). ``spec_generate`` drives the greedy loop for one sequence with a
caller-supplied target, following the pages' ``spec_generate`` call shape
(input ids, a token budget, temperature 0, a target, stop ids) [P4
"Ejecutando DFlash"].

Pages: [P4] DFlash news article, 7minutos.es, 2026-06-26.
"""
from __future__ import annotations

import ctypes as C
from typing import Protocol, Sequence

import numpy as np

from . import binding as bd
from .synth import DraftConfig, f32_to_bf16


def _torch():
    import torch
    return torch


# matrices the weight-streaming GEMM reads, stored in the packed fragment layout
PACKED = ("lm_head", "w_fc", "w_qkv", "w_o", "w_gate", "w_up", "w_down")


def is_packed(name: str) -> bool:
    return name.split(".")[-1] in PACKED


def pack_matrix(t, stream=None):
    """Device bf16 row-major [rows, cols] -> new tensor in the packed layout."""
    out = _torch().empty_like(t)
    bd.dflash_pack_matrix(t.data_ptr(), out.data_ptr(), t.shape[0], t.shape[1],
                          _torch().cuda.current_stream().cuda_stream if stream is None else stream)
    return out


def to_device_bf16(a: np.ndarray, device):
    """bf16 bits (uint16) or fp32 on the bf16 grid -> torch bf16 tensor on device."""
    torch = _torch()
    if a.dtype != np.uint16:
        a = f32_to_bf16(a)
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return t.to(device)


class Drafter:
    """A drafter, its draft KV cache for ``batch`` sequences of up to ``max_ctx``
    slots, and the workspace for fuse/inject calls of up to ``max_rows`` rows."""

    def __init__(self, cfg: DraftConfig, weights: dict, batch: int, max_ctx: int,
                 max_rows: int | None = None, device="cuda", rope_max: int | None = None):
        torch = _torch()
        bd.load()
        self.cfg = cfg
        self.device = torch.device(device)
        self.batch = batch
        self.max_ctx = max_ctx
        B = cfg.block
        self.max_rows = max_rows if max_rows is not None else batch * B
        self.rope_max = rope_max or max_ctx
        # weights (device bf16, GEMM matrices packed); the tensors are kept so the
        # pointers stay valid
        self.w = {}
        for name, arr in weights.items():
            t = arr if hasattr(arr, "data_ptr") else to_device_bf16(np.asarray(arr), self.device)
            self.w[name] = pack_matrix(t) if is_packed(name) else t
            del t
        rope = np.empty(self.rope_max * (cfg.head_dim // 2) * 2, np.float32)
        bd.dflash_rope_table(rope.ctypes.data_as(C.c_void_p), self.rope_max, cfg.head_dim, cfg.rope_theta)
        self.rope = torch.from_numpy(rope).to(self.device)
        c = bd.dflash_config(hidden=cfg.hidden, n_layers=cfg.n_layers, n_q_heads=cfg.n_q_heads,
                             n_kv_heads=cfg.n_kv_heads, head_dim=cfg.head_dim,
                             intermediate=cfg.intermediate, vocab=cfg.vocab, n_tap=cfg.n_tap,
                             block=B, mask_id=cfg.mask_id, rope_theta=cfg.rope_theta,
                             rms_eps=cfg.rms_eps)
        layers = (bd.dflash_layer_weights * cfg.n_layers)()
        for l in range(cfg.n_layers):
            for f in ("g_in", "w_qkv", "g_q", "g_k", "w_o", "g_post", "w_gate", "w_up", "w_down"):
                setattr(layers[l], f, self.w[f"layers.{l}.{f}"].data_ptr())
        wst = bd.dflash_weights(embed=self.w["embed"].data_ptr(), lm_head=self.w["lm_head"].data_ptr(),
                                w_fc=self.w["w_fc"].data_ptr(), g_fc=self.w["g_fc"].data_ptr(),
                                g_final=self.w["g_final"].data_ptr(), layers=layers,
                                rope=self.rope.data_ptr(), rope_max_pos=self.rope_max)
        self._c_cfg, self._c_layers, self._c_w = c, layers, wst
        self.model = bd.dflash_model_create(c, wst)
        # the library's own destroy call, kept here so that __del__ needs no
        # module globals (they may already be gone at interpreter exit)
        self._destroy = bd.load().dflash_model_destroy
        # draft KV cache
        NL, Hkv, D = cfg.n_layers, cfg.n_kv_heads, cfg.head_dim
        dev = self.device
        self.k = torch.zeros((NL, batch, Hkv, max_ctx, D), dtype=torch.bfloat16, device=dev)
        self.v = torch.zeros((NL, batch, Hkv, max_ctx, D), dtype=torch.bfloat16, device=dev)
        self.ctx_len = torch.zeros(batch, dtype=torch.int32, device=dev)
        self.status = torch.zeros(batch, dtype=torch.int32, device=dev)
        self.kv = bd.dflash_kv(k=self.k.data_ptr(), v=self.v.data_ptr(), batch=batch, max_ctx=max_ctx,
                               ctx_len=self.ctx_len.data_ptr(), status=self.status.data_ptr())
        self.ws_bytes = bd.dflash_workspace_bytes(self.model, batch, max_ctx, self.max_rows)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        # per-step buffers
        i32 = dict(dtype=torch.int32, device=dev)
        self.anchor = torch.zeros(batch, **i32)
        self.draft = torch.zeros((batch, B - 1), **i32)
        self.accept_len = torch.zeros(batch, **i32)
        self.anchor_out = torch.zeros(batch, **i32)
        self.emitted = torch.zeros((batch, B), **i32)
        self.n_emit = torch.zeros(batch, **i32)
        self.done = torch.zeros(batch, **i32)
        self.commit_rows = torch.zeros((batch * B, 3), **i32)
        self.n_commit = torch.zeros(1, **i32)
        self.ctx = torch.zeros((self.max_rows, cfg.hidden), dtype=torch.bfloat16, device=dev)

    def __del__(self):
        m, destroy = getattr(self, "model", None), getattr(self, "_destroy", None)
        if m and destroy is not None:
            destroy(m)
            self.model = None

    @staticmethod
    def stream():
        return _torch().cuda.current_stream().cuda_stream

    # -- entry points --------------------------------------------------------
    def fuse_ctx(self, taps, n_rows: int | None = None, ctx=None):
        n = taps.shape[0] if n_rows is None else n_rows
        out = self.ctx if ctx is None else ctx
        bd.dflash_fuse_ctx(self.model, bd.ptr(taps), n, bd.ptr(out), bd.ptr(self.ws), self.ws_bytes,
                           self.stream())
        return out

    def inject_kv(self, ctx, n_ctx_rows: int, commit_rows, n_commit, max_commit: int):
        bd.dflash_inject_kv(self.model, bd.ptr(ctx), n_ctx_rows, bd.ptr(commit_rows), bd.ptr(n_commit),
                            max_commit, self.kv, bd.ptr(self.ws), self.ws_bytes, self.stream())

    def draft_block(self, anchor=None, dbg_logits=None, dbg_hidden=None):
        a = self.anchor if anchor is None else anchor
        bd.dflash_draft_block(self.model, self.kv, bd.ptr(a), bd.ptr(self.draft), bd.ptr(dbg_logits),
                              bd.ptr(dbg_hidden), bd.ptr(self.ws), self.ws_bytes, self.stream())
        return self.draft

    def draft_block_noalloc(self, anchor=None, dbg_logits=None, dbg_hidden=None):
        """The draft block on the library's static workspace (no workspace
        argument; for callers that cannot allocate)."""
        a = self.anchor if anchor is None else anchor
        bd.dflash_draft_block_noalloc(self.model, self.kv, bd.ptr(a), bd.ptr(self.draft), bd.ptr(dbg_logits),
                                      bd.ptr(dbg_hidden), self.stream())
        return self.draft

    def draft_block_sample(self, temperature: float, seed: int, step: int, anchor=None, step_dev=None):
        """Sampling-mode draft block: tokens sampled from the drafter's own
        distributions (Gumbel-max, Philox draws of (seed, step)); the raw logits
        stay in self.draft_logits [batch*(B-1), V] for the verify."""
        a = self.anchor if anchor is None else anchor
        self._ensure_draft_logits()
        bd.dflash_draft_block_sample(self.model, self.kv, bd.ptr(a), bd.ptr(self.draft), bd.ptr(self.draft_logits),
                                     float(temperature), int(seed), int(step), bd.ptr(step_dev), bd.ptr(self.ws),
                                     self.ws_bytes, self.stream())
        return self.draft

    def _ensure_draft_logits(self):
        if getattr(self, "draft_logits", None) is None:
            torch = _torch()
            self.draft_logits = torch.empty((self.batch * (self.cfg.block - 1), self.cfg.vocab),
                                            dtype=torch.float32, device=self.device)
        return self.draft_logits

    def verify_sample(self, target_logits, temperature: float, seed: int, step: int, stop_ids=None, budget=None,
                      draft=None, draft_logits=None, step_dev=None):
        """Speculative-sampling verification against the target's logits
        [batch*B, V] (fp32) of the block rows; same outputs as verify_accept."""
        d = self.draft if draft is None else draft
        zd = self.draft_logits if draft_logits is None else draft_logits
        n_stop = 0 if stop_ids is None else int(stop_ids.numel())
        bd.dflash_verify_sample(self.model, self.kv, bd.ptr(d), bd.ptr(zd), bd.ptr(target_logits),
                                float(temperature), int(seed), int(step), bd.ptr(step_dev), bd.ptr(stop_ids), n_stop,
                                bd.ptr(budget),
                                bd.ptr(self.accept_len), bd.ptr(self.anchor_out), bd.ptr(self.emitted),
                                bd.ptr(self.n_emit), bd.ptr(self.done), bd.ptr(self.commit_rows),
                                bd.ptr(self.n_commit), bd.ptr(self.ws), self.ws_bytes, self.stream())

    def sample_logits(self, logits, temperature: float, seed: int, step: int, row0: int = 0, out=None):
        """Gumbel-max samples of softmax(logits / T) per row (fp32 [rows, V])."""
        torch = _torch()
        rows = logits.shape[0]
        out = torch.empty(rows, dtype=torch.int32, device=self.device) if out is None else out
        bd.dflash_sample_logits(self.model, bd.ptr(logits), rows, float(temperature), int(seed), int(step),
                                int(row0), bd.ptr(out), bd.ptr(self.ws), self.ws_bytes, self.stream())
        return out

    def loop_tokens(self, tokens, anchor=None, draft=None):
        """tokens [batch, B] = [anchor, draft] (the target's input of a loop step)."""
        a = self.anchor if anchor is None else anchor
        d = self.draft if draft is None else draft
        bd.dflash_loop_tokens(self.model, self.kv, bd.ptr(a), bd.ptr(d), bd.ptr(tokens), self.stream())
        return tokens

    def loop_advance(self, out, max_new: int, cursor, alive, step_dev=None):
        """End of a loop step: the emitted tokens of running sequences appended
        to out [batch, ld] at cursor, cursor/alive/anchor advanced, step_dev
        incremented (sampling mode)."""
        bd.dflash_loop_advance(self.model, self.kv, bd.ptr(self.anchor_out), bd.ptr(self.emitted),
                               bd.ptr(self.n_emit), bd.ptr(self.done), bd.ptr(out), out.shape[1], max_new,
                               bd.ptr(cursor), bd.ptr(alive), bd.ptr(self.anchor), bd.ptr(step_dev),
                               self.stream())

    def verify_accept(self, target_argmax, stop_ids=None, budget=None, draft=None):
        d = self.draft if draft is None else draft
        n_stop = 0 if stop_ids is None else int(stop_ids.numel())
        bd.dflash_verify_accept(self.model, self.kv, bd.ptr(d), bd.ptr(target_argmax), bd.ptr(stop_ids),
                                n_stop, bd.ptr(budget), bd.ptr(self.accept_len), bd.ptr(self.anchor_out),
                                bd.ptr(self.emitted), bd.ptr(self.n_emit), bd.ptr(self.done),
                                bd.ptr(self.commit_rows), bd.ptr(self.n_commit), self.stream())

    # -- helpers -------------------------------------------------------------
    def ingest(self, b: int, taps, start: int = 0):
        """Fuse and inject context rows of sequence b at positions start.. ."""
        torch = _torch()
        n = taps.shape[0]
        ctx = torch.empty((n, self.cfg.hidden), dtype=torch.bfloat16, device=self.device)
        if n > self.max_rows:
            raise ValueError("ingest rows exceed max_rows of the workspace")
        self.fuse_ctx(taps, n, ctx)
        # commit rows (src, seq, pos) written by the library on the device: no
        # host round trip between the calls
        rows = torch.empty((max(n, 1), 3), dtype=torch.int32, device=self.device)
        cnt = torch.empty((1,), dtype=torch.int32, device=self.device)
        bd.dflash_ingest_rows(self.model, self.kv, int(b), int(start), n, bd.ptr(rows), bd.ptr(cnt), self.stream())
        self.inject_kv(ctx, n, rows, cnt, n)


class DeviceTarget:
    """A target model on the device: ``n_layers`` decoder layers of the
    drafter's layer shape sharing its embedding and LM head, its own KV cache,
    and the layers in ``tap_layers`` tapped. ``pass_tokens`` runs the causal
    pass over up to ``max_n`` new tokens per sequence (K/V written
    speculatively) and ``commit`` keeps verified rows; ``forward``/``truncate``
    /``reset`` are the loop's target protocol for one sequence."""

    def __init__(self, cfg: DraftConfig, weights: dict, n_layers: int, tap_layers: Sequence[int],
                 batch: int = 1, max_ctx: int = 4096, max_n: int = 16, device="cuda", rope_max: int | None = None):
        torch = _torch()
        bd.load()
        self.cfg = cfg
        self.device = torch.device(device)
        self.batch, self.max_ctx, self.max_n = batch, max_ctx, max_n
        self.n_layers, self.tap_layers = n_layers, tuple(int(t) for t in tap_layers)
        self.rope_max = rope_max or max_ctx
        self.w = {}
        for name, arr in weights.items():
            if name.startswith("layers.") and int(name.split(".")[1]) >= n_layers:
                continue
            if name in ("w_fc", "g_fc"):
                continue
            t = arr if hasattr(arr, "data_ptr") else to_device_bf16(np.asarray(arr), self.device)
            self.w[name] = pack_matrix(t) if is_packed(name) else t
            del t
        rope = np.empty(self.rope_max * (cfg.head_dim // 2) * 2, np.float32)
        bd.dflash_rope_table(rope.ctypes.data_as(C.c_void_p), self.rope_max, cfg.head_dim, cfg.rope_theta)
        self.rope = torch.from_numpy(rope).to(self.device)
        c = bd.dflash_config(hidden=cfg.hidden, n_layers=n_layers, n_q_heads=cfg.n_q_heads,
                             n_kv_heads=cfg.n_kv_heads, head_dim=cfg.head_dim,
                             intermediate=cfg.intermediate, vocab=cfg.vocab, n_tap=len(self.tap_layers),
                             block=max_n, mask_id=cfg.mask_id, rope_theta=cfg.rope_theta,
                             rms_eps=cfg.rms_eps)
        layers = (bd.dflash_layer_weights * n_layers)()
        for l in range(n_layers):
            for f in ("g_in", "w_qkv", "g_q", "g_k", "w_o", "g_post", "w_gate", "w_up", "w_down"):
                setattr(layers[l], f, self.w[f"layers.{l}.{f}"].data_ptr())
        wst = bd.dflash_weights(embed=self.w["embed"].data_ptr(), lm_head=self.w["lm_head"].data_ptr(),
                                w_fc=None, g_fc=None, g_final=self.w["g_final"].data_ptr(), layers=layers,
                                rope=self.rope.data_ptr(), rope_max_pos=self.rope_max)
        self._c_cfg, self._c_layers, self._c_w = c, layers, wst
        self.model = bd.dflash_target_create(c, wst, self.tap_layers)
        self._destroy = bd.load().dflash_model_destroy
        Hkv, D = cfg.n_kv_heads, cfg.head_dim
        self.k = torch.zeros((n_layers, batch, Hkv, max_ctx, D), dtype=torch.bfloat16, device=self.device)
        self.v = torch.zeros((n_layers, batch, Hkv, max_ctx, D), dtype=torch.bfloat16, device=self.device)
        self.ctx_len = torch.zeros(batch, dtype=torch.int32, device=self.device)
        self.status = torch.zeros(batch, dtype=torch.int32, device=self.device)
        self.kv = bd.dflash_kv(k=self.k.data_ptr(), v=self.v.data_ptr(), batch=batch, max_ctx=max_ctx,
                               ctx_len=self.ctx_len.data_ptr(), status=self.status.data_ptr())
        self.ws_bytes = bd.dflash_workspace_bytes(self.model, batch, max_ctx, 0)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        self.argmax = torch.zeros(batch * max_n, dtype=torch.int32, device=self.device)
        self.taps = torch.zeros((batch * max_n, len(self.tap_layers) * cfg.hidden), dtype=torch.bfloat16,
                                device=self.device)

    def __del__(self):
        m, destroy = getattr(self, "model", None), getattr(self, "_destroy", None)
        if m and destroy is not None:
            destroy(m)
            self.model = None

    # -- entry points --------------------------------------------------------
    def pass_tokens(self, tokens, dbg_logits=None):
        """tokens: device int32 [batch, n] (contiguous); returns (argmax [batch, n],
        taps [batch*n, n_tap*H]) as views of the target's output buffers."""
        n = tokens.shape[1]
        if tokens.dtype != _torch().int32 or not tokens.is_contiguous() or tokens.shape[0] != self.batch:
            raise ValueError("tokens must be a contiguous int32 [batch, n] device tensor")
        bd.dflash_target_forward(self.model, self.kv, bd.ptr(tokens), n, bd.ptr(self.argmax), bd.ptr(self.taps),
                                 bd.ptr(dbg_logits), bd.ptr(self.ws), self.ws_bytes, Drafter.stream())
        return self.argmax[:self.batch * n].view(self.batch, n), self.taps[:self.batch * n]

    def commit(self, commit_rows, n_commit, max_commit: int):
        bd.dflash_kv_commit(self.model, self.kv, bd.ptr(commit_rows), bd.ptr(n_commit), max_commit,
                            Drafter.stream())

    # -- loop protocol (batch 1) ---------------------------------------------
    # The host-driven loop knows the committed length; a pass's rows are kept
    # with dflash_kv_commit, and a truncation (rollback) writes the length the
    # loop decided.
    def reset(self) -> None:
        self._len = 0
        self.ctx_len.zero_()
        self.status.zero_()

    def forward(self, tokens: Sequence[int], logits: bool = False):
        """Append tokens (in passes of up to max_n, each committed); returns
        (argmax as numpy [n], taps as a device bf16 tensor [n, n_tap*H]), and
        with logits=True also the fp32 logits of the last pass's rows (device
        [rows, V])."""
        torch = _torch()
        if self.batch != 1:
            raise ValueError("the loop protocol drives one sequence")
        toks = torch.tensor(list(tokens), dtype=torch.int32, device=self.device)
        outs, taps = [], []
        z = None
        L = getattr(self, "_len", 0)
        for i in range(0, len(toks), self.max_n):
            part = toks[i:i + self.max_n][None, :]
            n = part.shape[1]
            if logits:
                z = torch.empty((n, self.cfg.vocab), dtype=torch.float32, device=self.device)
            a, t = self.pass_tokens(part, dbg_logits=z)
            outs.append(a[0].clone())
            taps.append(t.clone())
            rows = torch.tensor([[j, 0, L + j] for j in range(n)], dtype=torch.int32, device=self.device)
            self.commit(rows, torch.tensor([n], dtype=torch.int32, device=self.device), n)
            L += n
        self._len = L
        if logits:
            return torch.cat(outs).cpu().numpy(), torch.cat(taps), z
        return torch.cat(outs).cpu().numpy(), torch.cat(taps)

    def truncate(self, length: int) -> None:
        torch = _torch()
        self._len = int(length)
        self.ctx_len.copy_(torch.tensor([self._len], dtype=torch.int32))


class Target(Protocol):
    """What the loop needs from the target model (batch 1)."""

    def reset(self) -> None: ...

    def forward(self, tokens: Sequence[int]):
        """Append tokens; return (greedy argmax per row, taps [n, n_tap*H] as an
        array or a device bf16 tensor)."""

    def truncate(self, length: int) -> None: ...


def _taps_dev(taps, dev):
    """Taps as a device bf16 tensor (a device target's are already there)."""
    return taps if hasattr(taps, "data_ptr") else to_device_bf16(np.asarray(taps, np.float32), dev)


def spec_generate(drafter: Drafter, target: Target, prompt: Sequence[int], max_new_tokens: int,
                  stop_token_ids: Sequence[int] = (), temperature: float = 0.0, seed: int = 0):
    """Speculative decoding of one sequence with the device drafter: greedy
    at temperature 0, speculative sampling above (seed keys the draws).

    Returns (tokens, accepted lengths per step)."""
    if temperature < 0.0:
        raise ValueError("temperature must be >= 0")
    if drafter.batch != 1:
        raise ValueError("spec_generate drives one sequence")
    if temperature > 0.0:
        return _spec_sample(drafter, target, prompt, max_new_tokens, stop_token_ids, temperature, seed)
    torch = _torch()
    dev = drafter.device
    B = drafter.cfg.block
    target.reset()
    drafter.ctx_len.zero_()
    a, taps = target.forward(list(prompt))
    anchor = int(a[-1])
    out = [anchor]
    P = len(prompt)
    drafter.ingest(0, _taps_dev(taps, dev))
    stops = torch.tensor(list(stop_token_ids), dtype=torch.int32, device=dev) if stop_token_ids else None
    budget = torch.tensor([max_new_tokens - 1], dtype=torch.int32, device=dev)
    L = P
    ms = []
    stop_set = set(int(s) for s in stop_token_ids)
    while len(out) < max_new_tokens and out[-1] not in stop_set:
        drafter.anchor.fill_(anchor)
        d = drafter.draft_block().cpu().numpy()[0]
        at, taps = target.forward([anchor] + [int(t) for t in d])
        tgt = torch.from_numpy(np.asarray(at, np.int32).reshape(1, B)).to(dev)
        drafter.verify_accept(tgt, stops, budget)
        m = int(drafter.accept_len.item())
        target.truncate(L + m + 1)
        ctx = drafter.fuse_ctx(_taps_dev(taps, dev), B)
        drafter.inject_kv(ctx, B, drafter.commit_rows, drafter.n_commit, B)
        n = int(drafter.n_emit.item())
        out += [int(t) for t in drafter.emitted[0, :n].cpu().numpy()]
        ms.append(m)
        anchor = int(drafter.anchor_out.item())
        L += m + 1
        if int(drafter.done.item()):
            break
    return out[:max_new_tokens], ms


def _spec_sample(drafter: Drafter, target: "DeviceTarget", prompt, max_new_tokens: int, stop_token_ids,
                 temperature: float, seed: int, trace: list | None = None):
    """The sampling loop: the first token is sampled from the target's last
    prompt row (draws of step 0); step s >= 1 samples the block (draft
    block, draws of step s), runs the target pass with logits and verifies by
    speculative sampling (draws of step s). ``trace`` collects per step
    (draft, draft logits, target logits, accept_len, emitted) copies."""
    torch = _torch()
    dev = drafter.device
    B = drafter.cfg.block
    target.reset()
    drafter.ctx_len.zero_()
    _, taps, z = target.forward(list(prompt), logits=True)
    first = drafter.sample_logits(z[-1:].contiguous(), temperature, seed, 0)
    anchor = int(first.item())
    out = [anchor]
    drafter.ingest(0, _taps_dev(taps, dev))
    stops = torch.tensor(list(stop_token_ids), dtype=torch.int32, device=dev) if stop_token_ids else None
    budget = torch.tensor([max_new_tokens - 1], dtype=torch.int32, device=dev)
    L = len(prompt)
    ms = []
    stop_set = set(int(s) for s in stop_token_ids)
    step = 0
    zt = torch.empty((B, drafter.cfg.vocab), dtype=torch.float32, device=dev)
    while len(out) < max_new_tokens and out[-1] not in stop_set:
        step += 1
        drafter.anchor.fill_(anchor)
        drafter.draft_block_sample(temperature, seed, step)
        toks = torch.cat([drafter.anchor[:, None], drafter.draft], dim=1).contiguous()
        _, taps_b = target.pass_tokens(toks, dbg_logits=zt)
        taps_b = taps_b.clone()
        drafter.verify_sample(zt, temperature, seed, step, stops, budget)
        m = int(drafter.accept_len.item())
        target.commit(drafter.commit_rows, drafter.n_commit, B)
        ctx = drafter.fuse_ctx(taps_b, B)
        drafter.inject_kv(ctx, B, drafter.commit_rows, drafter.n_commit, B)
        n = int(drafter.n_emit.item())
        em = [int(t) for t in drafter.emitted[0, :n].cpu().numpy()]
        if trace is not None:
            trace.append({"draft": drafter.draft.cpu().numpy().copy(),
                          "draft_logits": drafter.draft_logits.cpu().numpy().copy(),
                          "target_logits": zt.cpu().numpy().copy(), "accept_len": m, "emitted": em,
                          "step": step})
        out += em
        ms.append(m)
        anchor = int(drafter.anchor_out.item())
        L += m + 1
        if int(drafter.done.item()):
            break
    return out[:max_new_tokens], ms


# ---------------------------------------------------------------------------
# the whole loop on the device
# ---------------------------------------------------------------------------

class _LoopState:
    """Device buffers of spec_generate_device (fixed shapes, so a step can be
    captured in a graph). In sampling mode (temperature > 0) the step counter
    keying the draws lives on the device too, so every replay of a captured
    step draws afresh."""

    def __init__(self, torch, batch, B, max_new, dev, stops, temperature=0.0, seed=0, vocab=0):
        i32 = dict(dtype=torch.int32, device=dev)
        self.tokens = torch.zeros((batch, B), **i32)       # target input [anchor, d_1..d_{B-1}]
        self.out = torch.full((batch, max(1, max_new)), -1, **i32)
        self.cursor = torch.zeros(batch, **i32)
        self.alive = torch.ones(batch, **i32)
        self.budget = torch.zeros(batch, **i32)
        self.stops = stops
        self.max_new = max_new
        self.temperature, self.seed = float(temperature), int(seed)
        if self.temperature > 0.0:
            self.step = torch.ones(1, **i32)  # step 0 drew the first token after the prompt
            self.zt = torch.empty((batch * B, vocab), dtype=torch.float32, device=dev)


def _prefill_device(drafter: Drafter, target: DeviceTarget, prompts, st: _LoopState):
    """Target passes over the prompts (passes of up to max_n tokens, ragged
    prompts committed row by row), the drafter's fuse + inject of the same
    rows, and the first anchor: the target's token after each prompt, greedy
    or, in sampling mode, drawn from the target's distribution after the
    prompt with the draws of step 0 (RNG row = sequence index)."""
    torch = _torch()
    dev, batch = target.device, target.batch
    P = max(len(p) for p in prompts)
    anchor = np.zeros(batch, np.int32)
    sampling = st.temperature > 0.0
    for i0 in range(0, P, target.max_n):
        n = min(target.max_n, P - i0)
        toks = np.zeros((batch, n), np.int32)
        rows = []
        for b, p in enumerate(prompts):
            for j in range(n):
                if i0 + j < len(p):
                    toks[b, j] = p[i0 + j]
                    rows.append((b * n + j, b, i0 + j))
        z = torch.empty((batch * n, drafter.cfg.vocab), dtype=torch.float32, device=dev) if sampling else None
        a, taps = target.pass_tokens(torch.from_numpy(toks).to(dev), dbg_logits=z)
        crow = torch.zeros((batch * n, 3), dtype=torch.int32, device=dev)
        if rows:
            crow[:len(rows)] = torch.tensor(rows, dtype=torch.int32, device=dev)
        cnt = torch.tensor([len(rows)], dtype=torch.int32, device=dev)
        target.commit(crow, cnt, batch * n)
        drafter.fuse_ctx(taps, batch * n, drafter.ctx)
        drafter.inject_kv(drafter.ctx, batch * n, crow, cnt, batch * n)
        a = a.cpu().numpy()
        for b, p in enumerate(prompts):
            if i0 <= len(p) - 1 < i0 + n:
                if sampling:
                    r = b * n + len(p) - 1 - i0
                    tok = drafter.sample_logits(z[r:r + 1], st.temperature, st.seed, 0, row0=b)
                    anchor[b] = int(tok.item())
                else:
                    anchor[b] = a[b, len(p) - 1 - i0]
    drafter.anchor.copy_(torch.from_numpy(anchor))
    return anchor


def device_step(drafter: Drafter, target: DeviceTarget, st: _LoopState) -> None:
    """One speculative step with no host synchronisation, every part a library
    call: draft, the target's input row, target pass over [anchor, draft],
    verify, commit in both caches, fuse and inject of the accepted rows' taps,
    and the advance (emitted tokens of sequences still running appended to the
    output, cursors, running flags, next anchors). In sampling mode the block
    is sampled, the target pass keeps its logits, the verify is speculative
    sampling, and the advance also moves the device step counter."""
    B = drafter.cfg.block
    batch = drafter.batch
    sampling = st.temperature > 0.0
    if sampling:
        drafter.draft_block_sample(st.temperature, st.seed, 0, anchor=drafter.anchor, step_dev=st.step)
    else:
        drafter.draft_block(anchor=drafter.anchor)
    drafter.loop_tokens(st.tokens)
    a, taps = target.pass_tokens(st.tokens, dbg_logits=st.zt if sampling else None)
    if sampling:
        drafter.verify_sample(st.zt, st.temperature, st.seed, 0, st.stops, st.budget, step_dev=st.step)
    else:
        drafter.verify_accept(a, st.stops, st.budget)
    target.commit(drafter.commit_rows, drafter.n_commit, batch * B)
    drafter.fuse_ctx(taps, batch * B, drafter.ctx)
    drafter.inject_kv(drafter.ctx, batch * B, drafter.commit_rows, drafter.n_commit, batch * B)
    drafter.loop_advance(st.out, st.max_new, st.cursor, st.alive, step_dev=st.step if sampling else None)


def spec_generate_device(drafter: Drafter, target: DeviceTarget, prompts, max_new_tokens: int,
                         stop_token_ids: Sequence[int] = (), steps_per_sync: int = 8, graph: bool = True,
                         temperature: float = 0.0, seed: int = 0):
    """Speculative decoding of a batch with the drafter and the target on the
    device, greedy at temperature 0 and speculative sampling above (seed keys
    the draws; step s of the loop draws with step s, as spec_generate does for
    one sequence): steps run without host synchronisation (``steps_per_sync``
    of them captured in one graph when ``graph``), stop ids and the token
    budget are applied on the device, and the host only checks between groups
    of steps whether every sequence has finished. Returns the tokens of each
    sequence (as spec_generate does for one)."""
    torch = _torch()
    if drafter.batch != target.batch or len(prompts) != drafter.batch:
        raise ValueError("one prompt per sequence of the drafter and the target")
    if target.max_n < drafter.cfg.block:
        raise ValueError("the target's passes must hold a whole block")
    if not temperature >= 0.0:
        raise ValueError("temperature must be >= 0")
    dev = drafter.device
    B = drafter.cfg.block
    stops = torch.tensor(list(stop_token_ids), dtype=torch.int32, device=dev) if stop_token_ids else None
    st = _LoopState(torch, drafter.batch, B, max_new_tokens, dev, stops, temperature, seed, drafter.cfg.vocab)
    if st.temperature > 0.0:
        drafter._ensure_draft_logits()  # allocated before any capture: a graph must not own it
    target.reset()
    drafter.ctx_len.zero_()
    drafter.status.zero_()
    anchor = _prefill_device(drafter, target, [list(p) for p in prompts], st)
    st.out[:, 0] = torch.from_numpy(anchor).to(dev)
    st.cursor.fill_(1)
    stop_set = set(int(x) for x in stop_token_ids)
    st.alive.copy_(torch.tensor([0 if int(a) in stop_set or max_new_tokens <= 1 else 1 for a in anchor],
                                dtype=torch.int32))
    st.budget.fill_(max_new_tokens - 1)
    g = None
    if graph:
        # capture records the steps without running them; every replay then
        # advances the state in place
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for _ in range(steps_per_sync):
                    device_step(drafter, target, st)
        torch.cuda.current_stream().wait_stream(s)
    for _ in range(0, max_new_tokens + steps_per_sync, steps_per_sync):
        if g is not None:
            g.replay()
        else:
            for _ in range(steps_per_sync):
                device_step(drafter, target, st)
        if int(st.alive.max()) == 0 or int(st.cursor.min()) >= max_new_tokens:
            break
    out = st.out.cpu().numpy()
    cur = st.cursor.cpu().numpy()
    return [list(int(t) for t in out[b, :min(int(cur[b]), max_new_tokens)]) for b in range(drafter.batch)]
