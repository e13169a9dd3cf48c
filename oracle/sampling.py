"""Sampling-mode (temperature > 0) verification, plain fp64 — TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use this module. It shares no code with the HIP library.

The pages quote DFlash's speed-up under sampling next to the greedy one and
show the user call with a ``temperature`` argument [P4 "Ejecutando DFlash";
P2 results], but give no acceptance rule for it. The plain reading is the
standard speculative-sampling rule, which keeps the emitted tokens distributed
exactly as the target's own sampling would:

  * the drafter samples each block token d_j from its own distribution at that
    position, q_j = softmax(z^d_j / T) (here by the Gumbel-max trick: the argmax
    of z^d_j / T + g with g_v = -log(-log u_v), u_v uniform on (0, 1));
  * with p_i = softmax(z^t_i / T) the target's distribution after row i of
    [anchor, d_1 .. d_{B-1}], draft token d_j is accepted when
    u_j <= p_{j-1}(d_j) / q_j(d_j), walking j = 1, 2, ... until the first
    rejection;
  * at the first rejection (position j) the next token is sampled from the
    normalised residual max(0, p_{j-1} - q_j); when all B-1 drafts pass, a bonus
    token is sampled from p_{B-1};
  * the accepted drafts and the new token are emitted; rows 0..m of the block
    are committed exactly as in greedy verification.

Random numbers. Every uniform is drawn from Philox4x32-10, the counter-based
generator of Salmon, Moraes, Dror and Shaw ("Parallel random numbers: as easy as
1, 2, 3", SC'11), written here from its published definition: 10 rounds of two
32x32->64-bit multiplications (by 0xD2511F53 and 0xCD9E8D57) with a Weyl key
schedule (0x9E3779B9, 0xBB67AE85). A draw is addressed by
(seed, tag, step, row, v): key = (seed mod 2^32, seed div 2^32), counter =
(v div 4, row, step, tag), output word v mod 4; the uniform is
((word >> 9) + 0.5) / 2^23 (24 significant bits: exactly representable in
float32, in [2^-24, 1 - 2^-24]). Tags:
  0  draft token sampling, row = LM row b*(B-1) + j-1, v = vocab index;
  1  acceptance uniform of draft j of sequence b, row = b*B + j, v = 0;
  2  residual or bonus sample of sequence b, row = b, v = vocab index.
"""
from __future__ import annotations

import numpy as np

from .ref import verify_accept

__all__ = ["philox4x32", "philox4x32_np", "uniforms", "gumbel", "sample_rows", "row_logsumexp",
           "verify_sample", "TAG_DRAFT", "TAG_ACCEPT", "TAG_RESIDUAL"]

TAG_DRAFT, TAG_ACCEPT, TAG_RESIDUAL = 0, 1, 2

_M0, _M1 = 0xD2511F53, 0xCD9E8D57
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
_MASK = 0xFFFFFFFF


def philox4x32(counter, key, rounds: int = 10):
    """Philox4x32 on one counter (4 words) and key (2 words), plain Python ints."""
    c0, c1, c2, c3 = (int(x) & _MASK for x in counter)
    k0, k1 = (int(x) & _MASK for x in key)
    for r in range(rounds):
        if r:
            k0 = (k0 + _W0) & _MASK
            k1 = (k1 + _W1) & _MASK
        p0 = _M0 * c0
        p1 = _M1 * c2
        hi0, lo0 = p0 >> 32, p0 & _MASK
        hi1, lo1 = p1 >> 32, p1 & _MASK
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def philox4x32_np(c0, c1, c2, c3, k0: int, k1: int, rounds: int = 10):
    """Philox4x32 over arrays of counters (the same definition, numpy uint64 words)."""
    c = [np.asarray(x, dtype=np.uint64) & np.uint64(_MASK) for x in np.broadcast_arrays(c0, c1, c2, c3)]
    k0, k1 = int(k0) & _MASK, int(k1) & _MASK
    for r in range(rounds):
        if r:
            k0 = (k0 + _W0) & _MASK
            k1 = (k1 + _W1) & _MASK
        p0 = np.uint64(_M0) * c[0]  # < 2^64: exact in uint64
        p1 = np.uint64(_M1) * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(_MASK)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(_MASK)
        c = [hi1 ^ c[1] ^ np.uint64(k0), lo1, hi0 ^ c[3] ^ np.uint64(k1), lo0]
    return c


def uniforms(seed: int, tag: int, step: int, row, v) -> np.ndarray:
    """Uniforms on (0, 1) for the draws (seed, tag, step, row, v) (row, v broadcast)."""
    row, v = np.broadcast_arrays(np.asarray(row, dtype=np.int64), np.asarray(v, dtype=np.int64))
    words = philox4x32_np(v >> 2, row, np.full(row.shape, step, np.int64), np.full(row.shape, tag, np.int64),
                          seed & _MASK, (seed >> 32) & _MASK)
    w = np.choose(v & 3, [words[0], words[1], words[2], words[3]])
    return ((w >> np.uint64(9)).astype(np.float64) + 0.5) / 8388608.0


def gumbel(u) -> np.ndarray:
    """Standard Gumbel variates from uniforms: -log(-log u)."""
    return -np.log(-np.log(np.asarray(u, dtype=np.float64)))


def row_logsumexp(z) -> np.ndarray:
    """log sum_v exp(z_v) per row, in fp64 (shifted by the row max)."""
    z = np.asarray(z, dtype=np.float64)
    mx = z.max(axis=-1, keepdims=True)
    return (mx + np.log(np.exp(z - mx).sum(axis=-1, keepdims=True)))[..., 0]


def sample_rows(logits, temperature: float, seed: int, step: int, rows, tag: int = TAG_DRAFT):
    """Gumbel-max samples of softmax(logits / T) per row; rows = RNG row ids.

    Returns (tokens, margin): margin is the gap between the best and the second
    best perturbed score (a sample within rounding of a tie can go either way).
    """
    z = np.asarray(logits, dtype=np.float64)
    n, V = z.shape
    rows = np.asarray(rows, dtype=np.int64).reshape(n, 1)
    s = z / temperature + gumbel(uniforms(seed, tag, step, rows, np.arange(V)[None, :]))
    tok = np.argmax(s, axis=1)
    part = np.sort(s, axis=1)
    return tok.astype(np.int64), part[:, -1] - part[:, -2]


def verify_sample(draft, draft_logits, target_logits, temperature: float, seed: int, step: int, ctx_len,
                  stop_ids=(), budget=None):
    """Speculative-sampling verification of one block per sequence.

    draft [batch, B-1]: d_1..d_{B-1}; draft_logits [batch, B-1, V]: the
    drafter's logits of rows 1..B-1 (q_j = softmax(. / T)); target_logits
    [batch, B, V]: the target's logits after rows 0..B-1 of [anchor, d_1..]
    (p_i = softmax(. / T)). The new token of each sequence is written into a
    target-token row a (a_{j-1} = d_j for the accepted drafts, a_m = the new
    token) and the greedy rule of :func:`verify_accept` on (draft, a) then
    yields exactly the sampled outcome (a rejected draft never equals the
    residual sample: the residual is zero at it). Returns verify_accept's dict
    plus "target_tokens" (a), "accept_margin" [batch, B-1] (log u - log(p/q)
    of every tested draft, nan where untested) and "sample_margin" [batch].
    """
    draft = np.asarray(draft, dtype=np.int64)
    zd = np.asarray(draft_logits, dtype=np.float64) / temperature
    zt = np.asarray(target_logits, dtype=np.float64) / temperature
    batch, B, V = zt.shape
    lse_d = row_logsumexp(zd)
    lse_t = row_logsumexp(zt)
    a = np.zeros((batch, B), np.int64)
    acc_margin = np.full((batch, B - 1), np.nan)
    smp_margin = np.zeros(batch)
    for b in range(batch):
        m = 0
        rejected = False
        for j in range(1, B):
            d = int(draft[b, j - 1])
            log_ratio = (zt[b, j - 1, d] - lse_t[b, j - 1]) - (zd[b, j - 1, d] - lse_d[b, j - 1])
            u = uniforms(seed, TAG_ACCEPT, step, b * B + j, 0)
            acc_margin[b, j - 1] = np.log(u) - log_ratio
            if np.log(u) <= log_ratio:
                a[b, j - 1] = d
                m = j
            else:
                rejected = True
                break
        g = gumbel(uniforms(seed, TAG_RESIDUAL, step, b, np.arange(V)))
        if rejected:
            # residual max(0, p_{m} - q_{m+1}); its log where positive
            p = np.exp(zt[b, m] - lse_t[b, m])
            q = np.exp(zd[b, m] - lse_d[b, m])
            r = p - q
            with np.errstate(divide="ignore"):
                s = np.where(r > 0, np.log(np.where(r > 0, r, 1.0)), -np.inf) + g
        else:
            s = zt[b, B - 1] - lse_t[b, B - 1] + g
        a[b, m] = int(np.argmax(s))
        part = np.sort(s)
        smp_margin[b] = part[-1] - part[-2]
    res = verify_accept(draft, a, ctx_len, stop_ids, budget)
    res["target_tokens"] = a
    res["accept_margin"] = acc_margin
    res["sample_margin"] = smp_margin
    return res
