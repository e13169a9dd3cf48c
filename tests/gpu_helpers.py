"""Shared pieces of the GPU parity tests: seeded cases, oracle conversion,
tolerance checks. The oracle side always receives the exact bf16 (or fp32)
values that the device path receives, widened to fp64."""
from __future__ import annotations

import sys

import numpy as np

from block_diffusion_drafter_target_amd import synth
from oracle import ref

# max |gpu - ref| / max |ref| for bf16 hidden states and logits
TOL = 2e-2


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def as_f64(a: np.ndarray) -> np.ndarray:
    return synth.bf16_to_f64(a) if a.dtype == np.uint16 else np.asarray(a, np.float64)


def oracle_weights(W: dict) -> dict:
    return {k: as_f64(v) for k, v in W.items()}


def to_np_bf16(t) -> np.ndarray:
    """torch bf16 tensor -> fp64 numpy (exact)."""
    import torch
    u = t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)
    return synth.bf16_to_f64(u)


def check_rel(got, want, tol=TOL, what="", axis=None, rows=False):
    """max|got - want| / max|want| <= tol over the whole tensor, and, so that
    an error confined to small-magnitude parts cannot hide under the largest
    values, also over every slice along ``axis`` (e.g. each kv head of a cache
    [n, Hkv, D]) and, with ``rows``, over every row (last axis: one row of
    logits or of a hidden state). The slices are held to the stated 2e-2
    (TOL) even where the whole tensor takes a tighter tolerance (stage
    replays): a slice normalised by its own smaller maximum carries a larger
    relative rounding error. Returns the largest of these errors."""
    stol = max(tol, TOL)
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    e = ref.rel_err(got, want)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    assert e <= tol, f"{what}: rel err {e:.3e} > {tol}"
    if axis is not None:
        for i in range(got.shape[axis]):
            ei = ref.rel_err(np.take(got, i, axis=axis), np.take(want, i, axis=axis))
            assert ei <= stol, f"{what}: slice {i} of axis {axis}: rel err {ei:.3e} > {stol}"
            e = max(e, ei)
    if rows and got.size:
        g2, w2 = got.reshape(-1, got.shape[-1]), want.reshape(-1, want.shape[-1])
        for i in range(len(g2)):
            ei = ref.rel_err(g2[i], w2[i])
            assert ei <= stol, f"{what}: row {i}: rel err {ei:.3e} > {stol}"
            e = max(e, ei)
    return e


BF16_U = 2.0 ** -8  # unit roundoff of bf16 (8 significant bits, round to nearest even)


def e2e_band(ref_logits, tol=TOL):
    """Tie band for tokens compared end to end: both logits of a pair may be
    off by the stated logits tolerance, tol * max|ref| over the tensor."""
    return 2.0 * tol * float(np.max(np.abs(ref_logits)))


def replay_band(fin, w_lm, roundings=1, sigmas=6.0):
    """Tie band for an LM head replayed in fp64 from the device's own final
    hidden state. The device rounds the normalised row to bf16 before the
    product (``roundings`` = 2 when the replay starts from a bf16 copy of the
    hidden state, which adds one more rounding per element); every element then
    carries an independent relative error of at most u = 2^-8, spread uniformly
    (standard deviation u / sqrt(3)). The gap z_a - z_b = sum_k fin_k (W_ak -
    W_bk) then has a standard deviation sqrt(roundings) u / sqrt(3) *
    ||fin * (W_a - W_b)||_2; the band is ``sigmas`` of those, plus 1e-5 of the
    two logits for the fp32 accumulation (K 2^-24 relative at K <= 8192).
    Returns band(row, a, b)."""
    fin = np.asarray(fin, np.float64)

    def band(i, a, b):
        d = fin[i] * (w_lm[a] - w_lm[b])
        sd = np.sqrt(roundings) * BF16_U / np.sqrt(3.0) * float(np.sqrt(np.sum(d * d)))
        acc = 1e-5 * (abs(float(fin[i] @ w_lm[a])) + abs(float(fin[i] @ w_lm[b])) + 1.0)
        return sigmas * sd + acc
    return band


def check_tokens(gpu_tok, gpu_logits, ref_logits, band, what="", max_band=None):
    """Tokens: the device argmax equals the argmax of its own fp32 logits (same
    precision, bit exact). Against the fp64 reference a different token is
    allowed only where the reference's own gap between its top token and the
    device's token is at most ``band`` (a number, or band(row, ref_token,
    gpu_token) from :func:`replay_band`), an a priori bound that does not
    depend on the device's output. The rows at risk are those whose reference
    top-2 gap lies inside the band (found from the reference alone); at most
    ``max_band`` rows may be decided differently, by default half of the rows
    at risk (at least one). Returns (rows decided differently, rows at risk)."""
    gpu_tok = np.asarray(gpu_tok).reshape(-1)
    gl = np.asarray(gpu_logits, np.float64).reshape(len(gpu_tok), -1)
    rl = np.asarray(ref_logits, np.float64).reshape(len(gpu_tok), -1)
    assert np.array_equal(gpu_tok, np.argmax(gl, axis=1)), f"{what}: token is not the argmax of its logits"
    rt = np.argmax(rl, axis=1)
    lim_of = (lambda i, a, b: band(i, a, b)) if callable(band) else (lambda i, a, b: float(band))
    second = np.argsort(rl, axis=1)[:, -2]
    at_risk = sum(1 for i in range(len(rt)) if rl[i, rt[i]] - rl[i, second[i]] <= lim_of(i, rt[i], second[i]))
    cap = max(1, (at_risk + 1) // 2) if max_band is None else max_band
    n = 0
    for i in np.nonzero(gpu_tok != rt)[0]:
        gap = rl[i, rt[i]] - rl[i, gpu_tok[i]]
        lim = lim_of(i, rt[i], gpu_tok[i])
        assert gap <= lim, f"{what}: row {i} token {gpu_tok[i]} vs {rt[i]}, gap {gap:.3e} > band {lim:.3e}"
        n += 1
    assert n <= cap, f"{what}: {n} rows decided differently, {at_risk} rows at risk (cap {cap})"
    return n, at_risk


# small shapes that exercise every kernel branch (see the parity tests)
SHAPES = {
    # GQA G=4, D=128, B=16, 80 block rows (two GEMM row chunks), ragged and
    # empty contexts, vocab not a multiple of 64
    "gqa-d128": synth.DraftConfig(name="gqa-d128", hidden=512, n_layers=2, n_q_heads=8, n_kv_heads=2,
                                  head_dim=128, intermediate=1024, vocab=4144, n_tap=3, block=16,
                                  batch=5, ctx_len=0),
    # G=8, D=64 (two query tiles per wave), k = 320 and 1600 (partial k blocks)
    "g8-d64": synth.DraftConfig(name="g8-d64", hidden=320, n_layers=3, n_q_heads=16, n_kv_heads=2,
                                head_dim=64, intermediate=640, vocab=1008, n_tap=5, block=16,
                                batch=2, ctx_len=0),
    # block 12 (three query tiles, one idle wave), MHA-free G=4
    "b12": synth.DraftConfig(name="b12", hidden=256, n_layers=2, n_q_heads=8, n_kv_heads=2,
                             head_dim=64, intermediate=512, vocab=512, n_tap=2, block=12,
                             batch=3, ctx_len=0),

    # 9 sequences x 16 rows = 144 block rows: the LDS-tiled GEMM with two row
    # tiles (the second ragged), LM head over 135 rows
    "tiled-b9": synth.DraftConfig(name="tiled-b9", hidden=384, n_layers=2, n_q_heads=12, n_kv_heads=4,
                                  head_dim=64, intermediate=640, vocab=1040, n_tap=2, block=16,
                                  batch=9, ctx_len=0),
    # wide MLP (I = 8192): single-pass SwiGLU in the tiled kernel at batch 10
    # (160 rows, two row tiles) and in the streaming kernel at batch 2
    "mlp-wide": synth.DraftConfig(name="mlp-wide", hidden=256, n_layers=1, n_q_heads=4, n_kv_heads=2,
                                  head_dim=64, intermediate=8192, vocab=1024, n_tap=2, block=16,
                                  batch=10, ctx_len=0),
    # one sequence (16 rows): the single-pass SwiGLU on the streaming kernel
    # with four weight groups per workgroup (32 output columns, 256 workgroups)
    "mlp-wide-b1": synth.DraftConfig(name="mlp-wide-b1", hidden=256, n_layers=1, n_q_heads=4, n_kv_heads=2,
                                     head_dim=64, intermediate=8192, vocab=1024, n_tap=2, block=16,
                                     batch=1, ctx_len=0),
    "mlp-wide-b2": synth.DraftConfig(name="mlp-wide-b2", hidden=256, n_layers=1, n_q_heads=4, n_kv_heads=2,
                                     head_dim=64, intermediate=8192, vocab=1024, n_tap=2, block=16,
                                     batch=2, ctx_len=0),
    # 19 sequences x 16 rows = 304 block rows: every layer GEMM on the
    # large-tile kernel (qkv and o on two 256-row tiles, the second ragged;
    # down and fuse split-K over three 128-row tiles, the last ragged;
    # single-pass SwiGLU), the LM head over 285 rows with a vocabulary that ends
    # inside a 256-column tile; ingests of up to 300 rows take it too
    "big-b19": synth.DraftConfig(name="big-b19", hidden=256, n_layers=2, n_q_heads=4, n_kv_heads=2,
                                 head_dim=64, intermediate=768, vocab=1040, n_tap=2, block=16,
                                 batch=19, ctx_len=0),
    # block 8 over 40 sequences = 320 block rows on the large-tile kernel:
    # qkv, o and down split-K over three 128-row tiles (the last ragged),
    # the SwiGLU on 256 x 192 tiles (1536 = 16 x 96 output columns), the
    # LM head over 280 rows (a 24-row second tile)
    "big-b8x40": synth.DraftConfig(name="big-b8x40", hidden=512, n_layers=2, n_q_heads=8, n_kv_heads=2,
                                   head_dim=64, intermediate=1536, vocab=1040, n_tap=2, block=8,
                                   batch=40, ctx_len=0),
    # K % 128 == 64 on the tiled kernels: hidden 320 (QKV, o's input width
    # 256 aside, and the LM head on the LDS-tiled kernel over 80 rows, the
    # last 128-k slab half used) and I = 8256 (gate/up on the deep-prefetch
    # kernel with 129 workgroups, down on it with K = 8256: both end in a half
    # slab)
    "ws-tail": synth.DraftConfig(name="ws-tail", hidden=320, n_layers=1, n_q_heads=4, n_kv_heads=2,
                                 head_dim=64, intermediate=8256, vocab=1040, n_tap=2, block=16,
                                 batch=5, ctx_len=0),
    # rows wider than 4096 (hidden 5120): the embedding and row-norm kernels
    # with four float4 columns per thread (three used, the fourth clamped)
    "wide-h5120": synth.DraftConfig(name="wide-h5120", hidden=5120, n_layers=1, n_q_heads=8, n_kv_heads=2,
                                    head_dim=64, intermediate=512, vocab=1040, n_tap=2, block=16,
                                    batch=2, ctx_len=0),
    # long contexts: chunks of many 64-key attention slices, G = 8, D = 64
    "long-d64": synth.DraftConfig(name="long-d64", hidden=512, n_layers=1, n_q_heads=64, n_kv_heads=8,
                                  head_dim=64, intermediate=512, vocab=1024, n_tap=2, block=16,
                                  batch=4, ctx_len=0),
    # long contexts, G = 4, D = 128
    "long-d128": synth.DraftConfig(name="long-d128", hidden=512, n_layers=1, n_q_heads=16, n_kv_heads=4,
                                   head_dim=128, intermediate=512, vocab=1024, n_tap=2, block=16,
                                   batch=4, ctx_len=0),
    # one long sequence among many short ones, one kv head: the attention
    # chunk length is set by the 64-chunks-per-sequence bound (the batch's
    # average alone would cut the long sequence into 94 chunks), so it gets
    # 47 chunks over two merge load rounds
    "ragged-1long": synth.DraftConfig(name="ragged-1long", hidden=256, n_layers=1, n_q_heads=4, n_kv_heads=1,
                                      head_dim=64, intermediate=512, vocab=1024, n_tap=2, block=16,
                                      batch=24, ctx_len=0),
}

CTX = {"gqa-d128": [1, 300, 777, 0, 64], "g8-d64": [500, 33], "b12": [129, 0, 64],
       "tiled-b9": [17, 260, 0, 64, 1, 333, 90, 128, 2],
       "long-d64": [8900, 8500, 8193, 100], "long-d128": [16900, 16000, 9000, 3],
       "mlp-wide": [40, 0, 17, 300, 64, 1, 129, 90, 33, 7], "mlp-wide-b2": [70, 250], "mlp-wide-b1": [130], "wide-h5120": [77, 0],
       "big-b19": [0, 1, 17, 64, 129, 260, 300, 33, 90, 5, 200, 150, 75, 12, 280, 45, 100, 3, 64],
       "big-b8x40": [(37 * i) % 211 for i in range(40)], "ws-tail": [0, 33, 100, 64, 7],
       "ragged-1long": [6000, 0, 1, 5, 17, 3, 64, 2, 0, 9, 33, 1, 7, 0, 12, 4, 65, 1, 2, 8, 0, 3, 1, 6]}
