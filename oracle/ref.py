"""Plain fp64 numpy oracle of one DFlash-style draft step — TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use this module. It shares no code with the HIP library.

Every input arrives as whatever float array the caller has (bf16 values widened
exactly, or fp32) and is upcast to fp64; no intermediate is ever rounded.
Matrix products use numpy's ``@`` as a library primitive; nothing is blocked,
fused or reordered beyond the definitions written out below.

Sources. The method is described only in prose on four web pages:
  [P1] "DFlash: slik kan spekulativ dekoding gi opptil 6x raskere AI-inferens"
       (jansverre.net/?p=12023)
  [P2] DFlash news article on news.bpdata.com (no title in the extracted
       text; address slug "dflash-block-diffuzios-spekulativ-dekodolassal-akar-15")
  [P3] "DFlash Crea Blocchi Interi di Token Contemporaneamente, Aumentando Fino
       a 15x la Velocità su NVIDIA Blackwell" (theaistack.guide)
  [P4] DFlash news article on 7minutos.es, 2026-06-26 (no title in the
       extracted text; address slug "la-decodificacion-especulativa-de-dflash-
       elabora-bloques-de-tokens-completos-en-paralelo-...")
The pages give the steps (fuse taps from several target layers into one
feature; put that feature into the K/V projections of every draft layer, where
it stays in the draft KV cache; denoise a masked block in one pass; the target
verifies and the longest valid prefix is kept) but no equations. Where they are
silent, the plain readings used here are:
  * block row 0 holds the anchor (the target's newest greedy token, which has no
    tap yet); rows 1..B-1 hold the mask id; row j predicts the token at its own
    position (no shift), so B-1 tokens are drafted;
  * fusion = concat of taps in increasing layer order -> linear (no bias) ->
    RMSNorm;
  * injection uses the layer's own W_k, W_v, k-norm gain and RoPE, at the
    context row's position; the layer's input RMSNorm applies to block rows
    only;
  * layers are Qwen3-shaped: RMSNorm, q/k per-head RMSNorm, rotate-half RoPE
    (pairs i, i+D/2, angle p*theta^(-2i/D)), GQA attention with scale 1/sqrt(D)
    and no mask inside the block (full context), SwiGLU MLP, no biases;
  * greedy argmax takes the lowest index on ties.
"""
from __future__ import annotations

import dataclasses
from typing import Sequence

import numpy as np

__all__ = [
    "OracleConfig", "rms_norm", "rope", "silu", "attention", "argmax_rows",
    "decoder_layer", "fuse_ctx", "inject_kv", "new_cache", "draft_block",
    "verify_accept", "TinyTarget", "greedy_generate", "spec_generate",
    "rel_err",
]


@dataclasses.dataclass(frozen=True)
class OracleConfig:
    hidden: int
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    n_tap: int
    block: int
    rope_theta: float
    rms_eps: float

    @property
    def mask_id(self) -> int:
        return self.vocab - 1

    @classmethod
    def from_any(cls, c) -> "OracleConfig":
        return cls(**{f.name: getattr(c, f.name) for f in dataclasses.fields(cls)})


def f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# primitives
# ---------------------------------------------------------------------------

def rms_norm(x, g, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis."""
    x = f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * f64(g)


def rope(x, pos, theta: float) -> np.ndarray:
    """Rotate-half rotary embedding.

    x: [n, heads, D]; pos: [n]. Pair (x_i, x_{i+D/2}) for i < D/2 is rotated
    counter-clockwise by the angle pos * theta^(-2i/D).
    """
    x = f64(x)
    D = x.shape[-1]
    half = D // 2
    freq = float(theta) ** (-2.0 * np.arange(half, dtype=np.float64) / D)
    ang = f64(pos)[:, None, None] * freq[None, None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def silu(z) -> np.ndarray:
    z = f64(z)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def attention(q, k, v, allowed=None) -> np.ndarray:
    """Grouped-query softmax attention.

    q: [nq, Hq, D]; k, v: [nk, Hkv, D]; query head h reads kv head h // (Hq/Hkv).
    allowed: optional bool [nq, nk]; None means every query sees every key
    (the draft block's non-causal attention over context + block).
    """
    q, k, v = f64(q), f64(k), f64(v)
    nq, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.empty((nq, Hq, v.shape[2]), dtype=np.float64)
    for h in range(Hq):
        g = h // G
        s = (q[:, h, :] @ k[:, g, :].T) / np.sqrt(D)
        if allowed is not None:
            s = np.where(allowed, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, g, :]
    return out


def argmax_rows(z) -> np.ndarray:
    """Row-wise argmax; the lowest index wins ties (numpy's rule)."""
    return np.argmax(f64(z), axis=-1).astype(np.int64)


def rel_err(got, ref) -> float:
    """max |got - ref| / max |ref| over the whole tensor."""
    got, ref = f64(got), f64(ref)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(got - ref)) if ref.size else 0.0
    return float(num / den) if den > 0 else float(num)


# ---------------------------------------------------------------------------
# one decoder layer (drafter and tiny target share the definition)
# ---------------------------------------------------------------------------

def _lw(W, l: int, name: str):
    return W[f"layers.{l}.{name}"]


def project_kv(cfg: OracleConfig, W, l: int, u, pos):
    """k (normed, rotated) and v of layer l for input rows u at positions pos."""
    Hq, Hkv, D = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    wqkv = f64(_lw(W, l, "w_qkv"))
    wk = wqkv[Hq * D:(Hq + Hkv) * D]
    wv = wqkv[(Hq + Hkv) * D:(Hq + 2 * Hkv) * D]
    n = u.shape[0]
    k = (u @ wk.T).reshape(n, Hkv, D)
    v = (u @ wv.T).reshape(n, Hkv, D)
    k = rope(rms_norm(k, _lw(W, l, "g_k"), cfg.rms_eps), pos, cfg.rope_theta)
    return k, v


def decoder_layer(cfg: OracleConfig, W, l: int, x, pos, k_ctx, v_ctx, allowed=None):
    """x -> x' for rows x [n, H] at positions pos [n].

    Keys and values are [k_ctx; k_rows] and [v_ctx; v_rows]; ``allowed`` masks
    (query row, key) pairs in that order (None = no mask). Returns (x', k_rows,
    v_rows) where k_rows/v_rows are this layer's own (normed, rotated) K/V.
    [P3 "Come funziona il drafting a blocchi"; the Qwen3 layer shape is a
    reading, the pages give no layer equations]
    """
    Hq, Hkv, D = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    x = f64(x)
    n = x.shape[0]
    u = rms_norm(x, _lw(W, l, "g_in"), cfg.rms_eps)
    wqkv = f64(_lw(W, l, "w_qkv"))
    q = (u @ wqkv[:Hq * D].T).reshape(n, Hq, D)
    q = rope(rms_norm(q, _lw(W, l, "g_q"), cfg.rms_eps), pos, cfg.rope_theta)
    k, v = project_kv(cfg, W, l, u, pos)
    K = np.concatenate([f64(k_ctx).reshape(-1, Hkv, D), k], axis=0)
    V = np.concatenate([f64(v_ctx).reshape(-1, Hkv, D), v], axis=0)
    o = attention(q, K, V, allowed).reshape(n, Hq * D)
    x = x + o @ f64(_lw(W, l, "w_o")).T
    w = rms_norm(x, _lw(W, l, "g_post"), cfg.rms_eps)
    s = silu(w @ f64(_lw(W, l, "w_gate")).T) * (w @ f64(_lw(W, l, "w_up")).T)
    x = x + s @ f64(_lw(W, l, "w_down")).T
    return x, k, v


# ---------------------------------------------------------------------------
# draft side: fuse, inject, draft block
# ---------------------------------------------------------------------------

def fuse_ctx(cfg: OracleConfig, W, taps) -> np.ndarray:
    """Context feature c_r = RMSNorm(W_fc [h_r^(s1); ...; h_r^(sn)]; g_fc).

    taps: [n_rows, n_tap*H], layer-major within a row. The pages state that
    hidden states of several target layers are merged into one compact
    context feature that conditions the drafter. [P3 "L'idea chiave: Il target
    sa meglio"; P4 "La idea de que 'el objetivo sabe más'"; P2 "Hogyan működik
    a DFlash spekulatív dekódolás?"]
    """
    return rms_norm(f64(taps) @ f64(W["w_fc"]).T, W["g_fc"], cfg.rms_eps)


def new_cache(cfg: OracleConfig, batch: int, max_ctx: int, fill=0.0):
    """Draft KV cache: K, V each [NL, batch, max_ctx, Hkv, D] fp64."""
    shape = (cfg.n_layers, batch, max_ctx, cfg.n_kv_heads, cfg.head_dim)
    return {"k": np.full(shape, fill), "v": np.full(shape, fill)}


def inject_kv(cfg: OracleConfig, W, ctx, rows: Sequence[tuple[int, int, int]], cache) -> None:
    """Write K/V of context rows into every draft layer's cache.

    For every layer l and commit row (src, seq, pos):
      K^l[seq, pos] = RoPE(RMSNorm_head(W_k^l c_src; g_k^l), pos)
      V^l[seq, pos] = W_v^l c_src
    The feature enters the key and value projections of every draft layer and
    the projections stay in the draft KV cache across drafting iterations.
    [P3 "L'idea chiave: Il target sa meglio"; P4 "La idea de que 'el objetivo
    sabe más'"; P1 "Hva gjør DFlash annerledes enn vanlig spekulativ
    dekoding?"]
    """
    if len(rows) == 0:
        return
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    c = f64(ctx)[rows[:, 0]]
    for l in range(cfg.n_layers):
        k, v = project_kv(cfg, W, l, c, rows[:, 2])
        cache["k"][l, rows[:, 1], rows[:, 2]] = k
        cache["v"][l, rows[:, 1], rows[:, 2]] = v


def draft_block(cfg: OracleConfig, W, cache, ctx_len, anchor):
    """One single-pass denoising of the masked block for every sequence.

    Block rows j = 0..B-1 sit at positions L_b + j; row 0 holds the anchor and
    rows 1..B-1 the mask id. Each layer attends, with no mask, over its cached
    context K/V [0, L_b) followed by the block's own K/V. The draft for row j is
    the argmax of its logits, j = 1..B-1. [P1 "Hva gjør DFlash annerledes enn
    vanlig spekulativ dekoding?"; P3 "Come funziona il drafting a blocchi";
    P2 "Hogyan működik a DFlash spekulatív dekódolás?"]

    Returns dict with
      draft  [batch, B-1] int64
      logits [batch, B-1, V]
      hidden [batch, NL+1, B, H]  residual stream after embed and each layer
      final  [batch, B, H]        RMSNorm_final of the last residual
      block_k, block_v [batch, NL, B, Hkv, D]
    """
    B, H, NL = cfg.block, cfg.hidden, cfg.n_layers
    E = W["embed"]
    out = {"draft": [], "logits": [], "hidden": [], "final": [], "block_k": [], "block_v": []}
    for b in range(len(anchor)):
        L = int(ctx_len[b])
        toks = np.array([int(anchor[b])] + [cfg.mask_id] * (B - 1), dtype=np.int64)
        pos = L + np.arange(B)
        x = f64(E[toks])
        hs, bk, bv = [x], [], []
        for l in range(NL):
            x, k, v = decoder_layer(cfg, W, l, x, pos, cache["k"][l, b, :L], cache["v"][l, b, :L])
            hs.append(x)
            bk.append(k)
            bv.append(v)
        fin = rms_norm(x, W["g_final"], cfg.rms_eps)
        z = fin[1:] @ f64(W["lm_head"]).T
        out["draft"].append(argmax_rows(z))
        out["logits"].append(z)
        out["hidden"].append(np.stack(hs))
        out["final"].append(fin)
        out["block_k"].append(np.stack(bk))
        out["block_v"].append(np.stack(bv))
    return {k: np.stack(v) for k, v in out.items()}


# ---------------------------------------------------------------------------
# verification
# ---------------------------------------------------------------------------

def verify_accept(draft, target, ctx_len, stop_ids=(), budget=None):
    """Greedy acceptance of the longest valid prefix.

    draft [batch, B-1] holds d_1..d_{B-1}; target [batch, B] holds the target's
    argmax a_0..a_{B-1} on [anchor, d_1..d_{B-1}]. m_b is the largest k <= B-1
    with d_j = a_{j-1} for every j <= k. The emitted tokens are a_0..a_m (equal
    to d_1..d_m then a_m), cut after the first stop id and to the remaining
    budget. Rows 0..m of the block become context (commit); every slot from
    L_b + m + 1 on is dead (rollback). [P2 introduction: the target checks the
    proposals in parallel and keeps the longest valid prefix; P3 introduction;
    P4 "Ejecutando DFlash" for stop tokens and the token budget]

    Returns dict: accept_len, anchor_out, emitted [batch, B] (-1 padded),
    n_emit, done, commit_rows [n, 3] (src = b*B + i, seq, pos), new_ctx_len,
    budget (updated copy or None).
    """
    draft = np.asarray(draft, dtype=np.int64)
    target = np.asarray(target, dtype=np.int64)
    batch, B = target.shape
    stops = set(int(s) for s in stop_ids)
    res = {"accept_len": np.zeros(batch, np.int64), "anchor_out": np.zeros(batch, np.int64),
           "emitted": np.full((batch, B), -1, np.int64), "n_emit": np.zeros(batch, np.int64),
           "done": np.zeros(batch, np.int64), "new_ctx_len": np.zeros(batch, np.int64)}
    new_budget = None if budget is None else np.array(budget, dtype=np.int64)
    commit = []
    for b in range(batch):
        m = 0
        while m < B - 1 and draft[b, m] == target[b, m]:
            m += 1
        toks = [int(t) for t in target[b, :m + 1]]
        done = False
        for i, t in enumerate(toks):
            if t in stops:
                toks = toks[:i + 1]
                done = True
                break
        if new_budget is not None:
            left = max(0, int(new_budget[b]))
            if len(toks) >= left:
                toks = toks[:left]
                done = True
            new_budget[b] = left - len(toks)
        res["accept_len"][b] = m
        res["anchor_out"][b] = target[b, m]
        res["emitted"][b, :len(toks)] = toks
        res["n_emit"][b] = len(toks)
        res["done"][b] = int(done)
        L = int(ctx_len[b])
        res["new_ctx_len"][b] = L + m + 1
        commit += [(b * B + i, b, L + i) for i in range(m + 1)]
    res["commit_rows"] = np.asarray(commit, dtype=np.int64).reshape(-1, 3)
    res["budget"] = new_budget
    return res


# ---------------------------------------------------------------------------
# tiny causal target and the two decoding loops (CPU-checkable instance)
# ---------------------------------------------------------------------------

class TinyTarget:
    """A small causal decoder (same layer shape, no injection) with a KV cache.

    It stands in for the autoregressive target: it supplies the hidden states of
    the tapped layers and the greedy argmax that verification needs.
    """

    def __init__(self, cfg: OracleConfig, W, n_layers: int, tap_layers: Sequence[int]):
        self.cfg = dataclasses.replace(cfg, n_layers=n_layers)
        self.W = W
        self.tap_layers = tuple(tap_layers)
        self.reset()

    def reset(self):
        c = self.cfg
        self.k = [np.zeros((0, c.n_kv_heads, c.head_dim)) for _ in range(c.n_layers)]
        self.v = [np.zeros((0, c.n_kv_heads, c.head_dim)) for _ in range(c.n_layers)]

    @property
    def length(self) -> int:
        return self.k[0].shape[0]

    def forward(self, tokens):
        """Append tokens at positions length..; returns (logits [n, V], taps [n, n_tap*H])."""
        c = self.cfg
        tokens = np.asarray(tokens, dtype=np.int64)
        n, L = len(tokens), self.length
        pos = L + np.arange(n)
        allowed = np.arange(L + n)[None, :] <= pos[:, None]
        x = f64(self.W["embed"][tokens])
        taps = []
        for l in range(c.n_layers):
            x, k, v = decoder_layer(c, self.W, l, x, pos, self.k[l], self.v[l], allowed)
            self.k[l] = np.concatenate([self.k[l], k])
            self.v[l] = np.concatenate([self.v[l], v])
            if l in self.tap_layers:
                taps.append(x)
        z = rms_norm(x, self.W["g_final"], c.rms_eps) @ f64(self.W["lm_head"]).T
        return z, np.concatenate(taps, axis=1)

    def truncate(self, length: int) -> None:
        for l in range(self.cfg.n_layers):
            self.k[l] = self.k[l][:length]
            self.v[l] = self.v[l][:length]


def greedy_generate(target: TinyTarget, prompt, n_new: int, stop_ids=()):
    """Plain autoregressive greedy decoding: the losslessness reference."""
    target.reset()
    z, _ = target.forward(prompt)
    out = [int(argmax_rows(z[-1:])[0])]
    stops = set(int(s) for s in stop_ids)
    while len(out) < n_new and out[-1] not in stops:
        z, _ = target.forward([out[-1]])
        out.append(int(argmax_rows(z)[0]))
    return out


def spec_generate(cfg: OracleConfig, target: TinyTarget, prompt, n_new: int, W=None,
                  propose=None, stop_ids=(), max_ctx: int | None = None):
    """Greedy speculative decoding with a block drafter and KV-injected context.

    W: drafter weights; the context rows are fused and injected with them into
    the draft cache. ``propose(anchor, L, cache) -> d_1..d_{B-1}`` replaces the
    drafter's own :func:`draft_block` (stub drafters for the loop tests).

    Loop (batch 1): prefill; anchor = greedy token; fuse+inject the prompt rows
    at 0..P-1. Then repeat: draft, the target verifies [anchor, d_1..d_{B-1}]
    at positions L..L+B-1, its cache keeps rows L..L+m, the taps of rows 0..m
    are fused and injected at L..L+m, a_0..a_m are emitted, anchor = a_m and
    L += m+1. [P2 introduction; P4 "Ejecutando DFlash" (the spec_generate call
    with a target, a token budget, temperature 0 and stop ids)]

    Returns (tokens, info) with info = {"m": [m per step], "cache", "ctx_len"}.
    """
    B = cfg.block
    P = len(prompt)
    max_ctx = max_ctx or (P + n_new + 2 * B)
    cache = new_cache(cfg, 1, max_ctx)
    if propose is None:
        def propose(a, L, c):
            return draft_block(cfg, W, c, [L], [a])["draft"][0]
    target.reset()
    z, taps = target.forward(prompt)
    anchor = int(argmax_rows(z[-1:])[0])
    out = [anchor]
    stops = set(int(s) for s in stop_ids)
    budget = np.array([n_new - 1], np.int64)
    if W is not None:
        inject_kv(cfg, W, fuse_ctx(cfg, W, taps), [(r, 0, r) for r in range(P)], cache)
    L = P
    ms = []
    while len(out) < n_new and out[-1] not in stops:
        d = np.asarray(propose(anchor, L, cache), dtype=np.int64).reshape(1, B - 1)
        zt, taps = target.forward([anchor] + [int(t) for t in d[0]])
        a = argmax_rows(zt).reshape(1, B)
        r = verify_accept(d, a, [L], stop_ids, budget)
        m = int(r["accept_len"][0])
        budget = r["budget"]
        target.truncate(L + m + 1)
        if W is not None:
            inject_kv(cfg, W, fuse_ctx(cfg, W, taps[:m + 1]),
                      [(i, 0, L + i) for i in range(m + 1)], cache)
        out += [int(t) for t in r["emitted"][0, :r["n_emit"][0]]]
        ms.append(m)
        anchor = int(r["anchor_out"][0])
        L += m + 1
        if r["done"][0]:
            break
    return out[:n_new], {"m": ms, "cache": cache, "ctx_len": L}
