"""Pins of the oracle's sampling-mode verification (oracle/sampling.py).

* Philox4x32-10 against the known-answer vectors published with the generator
  (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3",
  SC'11, and its Random123 distribution's known-answer file), and the array
  version against the scalar one;
* the uniforms it yields pass a Kolmogorov-Smirnov test;
* Gumbel-max sampling reproduces softmax(z / T) (chi-square);
* speculative sampling keeps the target's distribution: one block position
  (chi-square against p) with the acceptance rate sum_v min(p_v, q_v) of the
  rule, and two tokens through two loop steps with a Markov target (chi-square
  against the exact joint p(x1 | a) p(x2 | x1)): an index or sign slip anywhere
  in the rule breaks one of these;
* as T -> 0 the rule becomes greedy verification (bit exact).
"""
import numpy as np
import pytest
from scipy import stats

from oracle import ref
from oracle import sampling as S

# (counter, key, output) known answers of philox4x32 with 10 rounds
KAT = [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,want", KAT)
def test_philox_known_answers(ctr, key, want):
    assert S.philox4x32(ctr, key) == want
    got = S.philox4x32_np(*[np.array([c]) for c in ctr], *key)
    assert tuple(int(w[0]) for w in got) == want


def test_philox_array_matches_scalar():
    g = np.random.default_rng(5)
    ctr = g.integers(0, 2**32, size=(64, 4), dtype=np.uint64)
    key = (0x12345678, 0x9ABCDEF0)
    arr = S.philox4x32_np(ctr[:, 0], ctr[:, 1], ctr[:, 2], ctr[:, 3], *key)
    for i in range(64):
        assert tuple(int(a[i]) for a in arr) == S.philox4x32(tuple(int(c) for c in ctr[i]), key)


def test_uniforms_are_uniform():
    u = S.uniforms(2024, S.TAG_DRAFT, 3, np.arange(200)[:, None], np.arange(500)[None, :]).ravel()
    assert u.min() > 0.0 and u.max() < 1.0
    assert np.all(u == u.astype(np.float32))  # exactly representable in float32
    assert stats.kstest(u, "uniform").pvalue > 1e-3
    # different tags, steps and rows give different streams
    a = S.uniforms(7, 0, 0, 0, np.arange(64))
    for other in (S.uniforms(7, 1, 0, 0, np.arange(64)), S.uniforms(7, 0, 1, 0, np.arange(64)),
                  S.uniforms(7, 0, 0, 1, np.arange(64)), S.uniforms(8, 0, 0, 0, np.arange(64))):
        assert not np.array_equal(a, other)


def _chi2_pvalue(counts, probs):
    counts = np.asarray(counts, dtype=np.float64)
    exp = np.asarray(probs) * counts.sum()
    keep = exp > 5
    return stats.chisquare(counts[keep], exp[keep] * counts[keep].sum() / exp[keep].sum()).pvalue


def _softmax(z):
    e = np.exp(z - z.max())
    return e / e.sum()


def test_gumbel_max_samples_the_softmax():
    V, n, T = 8, 40000, 0.7
    z = np.random.default_rng(1).normal(0, 1.5, V)
    tok, _ = S.sample_rows(np.broadcast_to(z, (n, V)), T, seed=11, step=0, rows=np.arange(n))
    assert _chi2_pvalue(np.bincount(tok, minlength=V), _softmax(z / T)) > 1e-4


def test_one_position_keeps_the_target_distribution():
    """B = 2: the emitted token is distributed as p, and the draft is accepted
    with probability sum_v min(p_v, q_v)."""
    V, n, T = 6, 40000, 1.0
    g = np.random.default_rng(2)
    zq, zp = g.normal(0, 1.2, V), g.normal(0, 1.2, V)
    p, q = _softmax(zp / T), _softmax(zq / T)
    d, _ = S.sample_rows(np.broadcast_to(zq, (n, V)), T, seed=3, step=0, rows=np.arange(n))
    assert _chi2_pvalue(np.bincount(d, minlength=V), q) > 1e-4
    r = S.verify_sample(d.reshape(n, 1), np.broadcast_to(zq, (n, 1, V)), np.broadcast_to(zp, (n, 2, V)), T,
                        seed=3, step=0, ctx_len=np.zeros(n, np.int64))
    first = r["emitted"][:, 0]
    assert _chi2_pvalue(np.bincount(first, minlength=V), p) > 1e-4
    rate = np.minimum(p, q).sum()
    acc = r["accept_len"].mean()
    assert abs(acc - rate) < 4 * np.sqrt(rate * (1 - rate) / n)
    # the accepted ones emitted their draft; the others a token != the draft
    m = r["accept_len"]
    assert np.all(first[m == 1] == d[m == 1]) and np.all(first[m == 0] != d[m == 0])
    assert np.all(r["n_emit"] == m + 1)


def test_two_tokens_through_two_steps_keep_the_markov_joint():
    """A Markov target (the next-token logits depend on the current token) and a
    block drafter with fixed per-position distributions: the first two emitted
    tokens are distributed as p(x1 | a) p(x2 | x1), over one or two steps."""
    V, n, T, B = 4, 30000, 0.9, 3
    g = np.random.default_rng(4)
    trans = g.normal(0, 1.3, (V, V))  # logits of the next token given the current one
    zq = g.normal(0, 1.0, (B - 1, V))  # drafter logits of rows 1, 2
    a0 = 2
    joint = np.outer(_softmax(trans[a0] / T), np.ones(V)) * np.stack([_softmax(trans[x] / T) for x in range(V)])

    def step(anchor, s):
        d = np.stack([S.sample_rows(np.broadcast_to(zq[j], (n, V)), T, seed=9, step=s,
                                    rows=np.arange(n) * (B - 1) + j)[0] for j in range(B - 1)], axis=1)
        toks = np.concatenate([anchor[:, None], d], axis=1)
        zt = trans[toks]  # [n, B, V]
        r = S.verify_sample(d, np.broadcast_to(zq, (n, B - 1, V)), zt, T, seed=9, step=s,
                            ctx_len=np.zeros(n, np.int64))
        return r

    r1 = step(np.full(n, a0), 0)
    x1 = r1["emitted"][:, 0]
    x2 = np.where(r1["n_emit"] >= 2, r1["emitted"][:, 1], -1)
    need = x2 < 0
    r2 = step(r1["anchor_out"], 1)  # only read where the first step emitted one token
    x2[need] = r2["emitted"][need, 0]
    assert np.all(r1["anchor_out"][need] == x1[need])
    counts = np.bincount(x1 * V + x2, minlength=V * V)
    assert _chi2_pvalue(counts, joint.ravel()) > 1e-4


def test_zero_temperature_limit_is_greedy():
    """With logit gaps >= 0.05 and T = 1e-4, every softmax is one-hot in fp64:
    sampling verification equals greedy verification, stop ids and budgets
    included."""
    g = np.random.default_rng(6)
    V, B, batch = 7, 5, 200
    base = np.arange(V) * 0.05

    def rand_logits(shape):
        return np.stack([g.permutation(base) for _ in range(int(np.prod(shape)))]).reshape(*shape, V)

    zd = rand_logits((batch, B - 1))
    zt = rand_logits((batch, B))
    # drafts: the drafter's own (one-hot) samples, its greedy tokens
    draft = np.argmax(zd, axis=-1)
    # targets that agree with the drafts for a while
    for b in range(batch):
        k = g.integers(0, B)
        for j in range(1, k + 1):
            zt[b, j - 1, draft[b, j - 1]] = 1.0
    budget = g.integers(1, 2 * B, batch)
    r = S.verify_sample(draft, zd, zt, 1e-4, seed=5, step=2, ctx_len=np.full(batch, 10), stop_ids=[3],
                        budget=budget)
    greedy = ref.verify_accept(draft, np.argmax(zt, axis=-1), np.full(batch, 10), stop_ids=[3], budget=budget)
    for k in ("accept_len", "anchor_out", "emitted", "n_emit", "done", "new_ctx_len", "commit_rows", "budget"):
        assert np.array_equal(r[k], greedy[k]), k
