"""Seeded synthetic inputs for the draft step: shapes, weights, taps, lengths.

This module holds no arithmetic of the method itself. It draws random numbers,
rounds them to bf16 and lays them out; both the fp64 oracle (through the tests)
and the HIP path consume what it produces.

Generator: numpy PCG64. A 2-D tensor is cut into row blocks of about 2**20
elements; block ``i`` of tensor ``tid`` draws from
``Generator(PCG64(SeedSequence([seed, tid, i])))``. Blocks are therefore
independent, can be drawn on several threads, and a single block can be
regenerated alone (the full-size parity tests use this to rebuild only the
weight rows they sample).

Values are drawn in fp32 and rounded to bf16 round-to-nearest-even. bf16 data
is carried as ``np.uint16`` bit patterns; :func:`bf16_to_f32` widens them.

Seeds (one per role): 0 drafter weights, 1 taps, 2 context lengths,
3 anchors, 4 synthetic target tokens and acceptance draws, 5 tiny-target
weights, 6 prompts.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

SEED_WEIGHTS = 0
SEED_TAPS = 1
SEED_CTX = 2
SEED_ANCHOR = 3
SEED_TARGET = 4
SEED_TARGET_WEIGHTS = 5
SEED_PROMPT = 6

WEIGHT_STD = 0.02


@dataclasses.dataclass(frozen=True)
class DraftConfig:
    """Shape of a drafter (and of the tiny target for the CPU-checkable case)."""

    name: str
    hidden: int
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    n_tap: int
    block: int
    rope_theta: float = 1.0e6
    rms_eps: float = 1.0e-6
    # workload
    batch: int = 1
    ctx_len: int | tuple[int, int] = 1024  # fixed length, or (lo, hi) uniform
    # target model paired with the drafter (tiny case: the CPU-checkable
    # target; Qwen3-8B shape: the device target of the verify pass)
    target_layers: int = 0
    tap_layers: tuple[int, ...] = ()
    n_new: int = 0
    weights_fp32: bool = False

    @property
    def mask_id(self) -> int:
        return self.vocab - 1

    @property
    def q_width(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_width(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def qkv_width(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def tap_width(self) -> int:
        return self.n_tap * self.hidden

    def with_(self, **kw) -> "DraftConfig":
        return dataclasses.replace(self, **kw)


# The five workloads. c1 is small enough for the oracle to run whole.
CONFIGS: dict[str, DraftConfig] = {
    "c1": DraftConfig(
        name="tiny-4L-target-2L-drafter", hidden=256, n_layers=2, n_q_heads=4,
        n_kv_heads=4, head_dim=64, intermediate=768, vocab=1024, n_tap=3,
        block=8, batch=1, ctx_len=64, target_layers=4, tap_layers=(1, 2, 3),
        n_new=64, weights_fp32=True),
    "c2": DraftConfig(
        name="qwen3-8b-shaped-5L", hidden=4096, n_layers=5, n_q_heads=32,
        n_kv_heads=8, head_dim=128, intermediate=12288, vocab=151936, n_tap=5,
        block=16, batch=1, ctx_len=1024, target_layers=36, tap_layers=(1, 9, 17, 25, 33)),
    "c3": DraftConfig(
        name="qwen3-8b-shaped-5L", hidden=4096, n_layers=5, n_q_heads=32,
        n_kv_heads=8, head_dim=128, intermediate=12288, vocab=151936, n_tap=5,
        block=16, batch=32, ctx_len=(512, 4096), target_layers=36, tap_layers=(1, 9, 17, 25, 33)),
    "c4": DraftConfig(
        name="qwen3-8b-shaped-5L", hidden=4096, n_layers=5, n_q_heads=32,
        n_kv_heads=8, head_dim=128, intermediate=12288, vocab=151936, n_tap=5,
        block=16, batch=8, ctx_len=8192, target_layers=36, tap_layers=(1, 9, 17, 25, 33)),
    "c5": DraftConfig(
        name="gpt-oss-120b-shaped-8L", hidden=2880, n_layers=8, n_q_heads=64,
        n_kv_heads=8, head_dim=64, intermediate=2880, vocab=201088, n_tap=5,
        block=16, batch=4, ctx_len=32768),
}


# --------------------------------------------------------------------------
# bf16 bit handling (storage format only)
# --------------------------------------------------------------------------

def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to fp32 exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_to_f32(b).astype(np.float64)


# --------------------------------------------------------------------------
# block-seeded normal tensors
# --------------------------------------------------------------------------

_BLOCK_ELEMS = 1 << 20


def rows_per_block(cols: int) -> int:
    return max(1, _BLOCK_ELEMS // max(1, cols))


def _block(seed: int, tid: int, i: int, rows: int, cols: int, std: float) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, i])))
    a = g.standard_normal((rows, cols), dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_tensor(seed: int, tid: int, rows: int, cols: int, std: float,
                  fp32: bool = False, row_range: tuple[int, int] | None = None) -> np.ndarray:
    """A [rows, cols] N(0, std^2) tensor, bf16 bits (uint16) or fp32 on the bf16 grid.

    ``row_range=(r0, r1)`` returns only rows r0..r1-1, bit-identical to the same
    rows of the full tensor.
    """
    r0, r1 = (0, rows) if row_range is None else row_range
    rpb = rows_per_block(cols)
    b0, b1 = r0 // rpb, (r1 + rpb - 1) // rpb
    out = np.empty((r1 - r0, cols), dtype=np.float32 if fp32 else np.uint16)

    def work(i):
        lo, hi = i * rpb, min(rows, (i + 1) * rpb)
        blk = f32_to_bf16(_block(seed, tid, i, hi - lo, cols, std))
        a, b = max(lo, r0), min(hi, r1)
        piece = blk[a - lo:b - lo]
        out[a - r0:b - r0] = bf16_to_f32(piece) if fp32 else piece

    idx = list(range(b0, b1))
    if len(idx) <= 2:
        for i in idx:
            work(i)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, idx))
    return out


# --------------------------------------------------------------------------
# weights
# --------------------------------------------------------------------------

def weight_shapes(cfg: DraftConfig) -> list[tuple[str, int, int]]:
    """Every random drafter matrix in its fixed order: (name, rows, cols).

    Layout conventions (all row-major, [out, in]):
      embed, lm_head   [V, H]      shared with the target
      w_fc             [H, n_tap*H] columns layer-major (tap 0 first)
      layer.w_qkv      [(Hq+2Hkv)*D, H] rows: q heads, then k heads, then v heads
      layer.w_o        [H, Hq*D]
      layer.w_gate     [I, H]
      layer.w_up       [I, H]
      layer.w_down     [H, I]
    """
    H, V = cfg.hidden, cfg.vocab
    out = [("embed", V, H), ("lm_head", V, H), ("w_fc", H, cfg.tap_width)]
    for l in range(cfg.n_layers):
        out += [
            (f"layers.{l}.w_qkv", cfg.qkv_width, H),
            (f"layers.{l}.w_o", H, cfg.q_width),
            (f"layers.{l}.w_gate", cfg.intermediate, H),
            (f"layers.{l}.w_up", cfg.intermediate, H),
            (f"layers.{l}.w_down", H, cfg.intermediate),
        ]
    return out


def gain_shapes(cfg: DraftConfig) -> list[tuple[str, int]]:
    H, D = cfg.hidden, cfg.head_dim
    out = [("g_fc", H), ("g_final", H)]
    for l in range(cfg.n_layers):
        out += [(f"layers.{l}.g_in", H), (f"layers.{l}.g_q", D),
                (f"layers.{l}.g_k", D), (f"layers.{l}.g_post", H)]
    return out


# random norm gains (opt-in): 1 + GAIN_STD * N(0, 1), every gain vector drawn
# from its own stream so that each differs from 1 and from every other gain
GAIN_STD = 0.3
_GAIN_TID0 = 1 << 16  # tensor ids of gain streams (clear of the matrices' ids)


def _gain(n: int, fp32: bool, seed: int | None, tid: int) -> np.ndarray:
    if seed is None:
        a = np.ones(n, np.float32)
    else:
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _GAIN_TID0 + tid])))
        a = (1.0 + GAIN_STD * g.standard_normal(n)).astype(np.float32)
    b = f32_to_bf16(a)
    return bf16_to_f32(b) if fp32 else b


def make_weights(cfg: DraftConfig, seed: int = SEED_WEIGHTS, only: set[str] | None = None,
                 gains: str = "ones") -> dict[str, np.ndarray]:
    """Drafter weights: matrices N(0, 0.02^2); norm gains 1.0, or with
    ``gains="random"`` 1 + 0.3 N(0, 1) on the bf16 grid, each gain vector from
    its own seeded stream.

    bf16 bits (uint16) unless ``cfg.weights_fp32`` (then fp32 values that lie on
    the bf16 grid, so the oracle and a bf16 device path read identical numbers).
    """
    if gains not in ("ones", "random"):
        raise ValueError("gains must be 'ones' or 'random'")
    w: dict[str, np.ndarray] = {}
    for tid, (name, r, c) in enumerate(weight_shapes(cfg)):
        if only is not None and name not in only:
            continue
        w[name] = normal_tensor(seed, tid, r, c, WEIGHT_STD, fp32=cfg.weights_fp32)
    gseed = seed if gains == "random" else None
    for tid, (name, n) in enumerate(gain_shapes(cfg)):
        if only is not None and name not in only:
            continue
        w[name] = _gain(n, cfg.weights_fp32, gseed, tid)
    return w


def weight_rows(cfg: DraftConfig, name: str, r0: int, r1: int, seed: int = SEED_WEIGHTS) -> np.ndarray:
    """Rows r0..r1-1 of one drafter matrix, identical to ``make_weights``'s."""
    for tid, (n, r, c) in enumerate(weight_shapes(cfg)):
        if n == name:
            return normal_tensor(seed, tid, r, c, WEIGHT_STD, fp32=cfg.weights_fp32, row_range=(r0, r1))
    raise KeyError(name)


def target_weight_shapes(cfg: DraftConfig) -> list[tuple[str, int, int]]:
    """Target: same layer shapes as the drafter, ``cfg.target_layers`` deep.

    Its embedding and LM head are the drafter's (shared)."""
    H = cfg.hidden
    out = []
    for l in range(cfg.target_layers):
        out += [
            (f"layers.{l}.w_qkv", cfg.qkv_width, H),
            (f"layers.{l}.w_o", H, cfg.q_width),
            (f"layers.{l}.w_gate", cfg.intermediate, H),
            (f"layers.{l}.w_up", cfg.intermediate, H),
            (f"layers.{l}.w_down", H, cfg.intermediate),
        ]
    return out


def make_target_weights(cfg: DraftConfig, drafter: dict[str, np.ndarray],
                        seed: int = SEED_TARGET_WEIGHTS, gains: str = "ones") -> dict[str, np.ndarray]:
    """Target weights (embedding and LM head shared with the drafter); gains as
    in :func:`make_weights`."""
    if gains not in ("ones", "random"):
        raise ValueError("gains must be 'ones' or 'random'")
    w: dict[str, np.ndarray] = {"embed": drafter["embed"], "lm_head": drafter["lm_head"]}
    for tid, (name, r, c) in enumerate(target_weight_shapes(cfg)):
        w[name] = normal_tensor(seed, tid, r, c, WEIGHT_STD, fp32=cfg.weights_fp32)
    gseed = seed if gains == "random" else None
    names = [("g_final", cfg.hidden)]
    for l in range(cfg.target_layers):
        names += [(f"layers.{l}.g_in", cfg.hidden), (f"layers.{l}.g_post", cfg.hidden),
                  (f"layers.{l}.g_q", cfg.head_dim), (f"layers.{l}.g_k", cfg.head_dim)]
    for tid, (name, n) in enumerate(names):
        w[name] = _gain(n, cfg.weights_fp32, gseed, tid)
    return w


# --------------------------------------------------------------------------
# activations and workload draws
# --------------------------------------------------------------------------

def make_taps(cfg: DraftConfig, n_rows: int, seed: int = SEED_TAPS, tid: int = 0,
              row_range: tuple[int, int] | None = None) -> np.ndarray:
    """Target hidden-state taps [n_rows, n_tap*H], N(0, 1), bf16 bits."""
    return normal_tensor(seed, tid, n_rows, cfg.tap_width, 1.0, row_range=row_range)


def make_ctx_lens(cfg: DraftConfig, seed: int = SEED_CTX) -> np.ndarray:
    """Committed context length per sequence (int32)."""
    if isinstance(cfg.ctx_len, tuple):
        lo, hi = cfg.ctx_len
        g = np.random.Generator(np.random.PCG64(seed))
        return g.integers(lo, hi + 1, size=cfg.batch).astype(np.int32)
    return np.full(cfg.batch, cfg.ctx_len, np.int32)


def make_anchors(cfg: DraftConfig, seed: int = SEED_ANCHOR, step: int = 0) -> np.ndarray:
    """Anchor tokens uniform over [0, V-2] (V-1 is the mask id)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, step])))
    return g.integers(0, cfg.vocab - 1, size=cfg.batch).astype(np.int32)


def make_prompt(cfg: DraftConfig, length: int, seed: int = SEED_PROMPT) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seed))
    return g.integers(0, cfg.vocab - 1, size=length).astype(np.int64)


def geometric_accept(batch: int, block: int, p: float = 0.8, seed: int = SEED_TARGET,
                     step: int = 0) -> np.ndarray:
    """Accepted-prefix lengths m with P(m >= k) = p**k, truncated at block-1."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, step])))
    m = np.zeros(batch, np.int32)
    alive = np.ones(batch, bool)
    for _ in range(block - 1):
        alive &= g.random(batch) < p
        m += alive
    return m


def synth_target_tokens(draft: np.ndarray, m: np.ndarray, vocab: int,
                        seed: int = SEED_TARGET, step: int = 0) -> np.ndarray:
    """Target argmax rows [batch, B] whose matched prefix with ``draft`` is ``m``.

    draft is [batch, B-1]. a[j] = draft[j] for j < m; a[m] = (draft[m]+1) mod (V-1)
    when m < B-1 (a guaranteed mismatch that avoids the mask id); the rest are
    uniform draws over [0, V-2].
    """
    batch, bm1 = draft.shape
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, step, 1])))
    a = g.integers(0, vocab - 1, size=(batch, bm1 + 1)).astype(np.int32)
    for b in range(batch):
        k = int(m[b])
        a[b, :k] = draft[b, :k]
        if k < bm1:
            a[b, k] = (int(draft[b, k]) + 1) % (vocab - 1)
    return a
