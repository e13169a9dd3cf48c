"""Sampling mode on the device (dflash_sample_logits, dflash_draft_block_sample,
dflash_verify_sample) against the oracle's speculative sampling
(oracle/sampling.py), with the same Philox draws on both sides.

The oracle takes the device's own fp32 logits (widened to fp64) as input, so a
sampled token or an acceptance can differ only where the fp32 and fp64
evaluations of the same decision straddle a tie: a Gumbel-max sample whose two
best perturbed scores lie within the fp32 error of each other, or an
acceptance whose log u lies within it of log(p/q). Such cases are counted and
allowed; everything else is compared bit exactly (tokens, acceptance lengths,
emitted tokens, commit rows, budgets).
"""
import numpy as np
import pytest

import gpu_helpers as gh
from block_diffusion_drafter_target_amd import DeviceTarget, Drafter, spec_generate_device, synth
from block_diffusion_drafter_target_amd.drafter import _spec_sample
from oracle import ref
from oracle import sampling as S

pytestmark = pytest.mark.gpu

SEED = 0x1234ABCD5678


def _torch():
    import torch
    return torch


def _drafter(vocab=None, batch=1, max_ctx=256):
    cfg = synth.CONFIGS["c1"]
    if vocab:
        cfg = cfg.with_(vocab=vocab)
    W = synth.make_weights(cfg)
    return cfg, W, Drafter(cfg, W, batch=batch, max_ctx=max_ctx, max_rows=max(64, batch * cfg.block))


def _score_tol(z, T):
    """fp32 error bound of a perturbed score z / T + g (rounding of the scaling,
    of the two logs of the Gumbel transform and of the comparison)."""
    return 1e-4 + 2e-6 * float(np.max(np.abs(z))) / T


def _check_samples(dev_tok, z, T, step, rows, what):
    """Device Gumbel-max samples against the oracle's on the same logits."""
    z = np.asarray(z, np.float64)
    want, margin = S.sample_rows(z, T, SEED, step, rows)
    tol = _score_tol(z, T)
    band = 0
    g = S.gumbel(S.uniforms(SEED, S.TAG_DRAFT, step, np.asarray(rows)[:, None], np.arange(z.shape[1])[None, :]))
    for i in np.nonzero(np.asarray(dev_tok) != want)[0]:
        s = z[i] / T + g[i]
        gap = s[want[i]] - s[dev_tok[i]]
        assert gap <= tol, f"{what}: row {i} sampled {dev_tok[i]}, oracle {want[i]}, score gap {gap:.3e} > {tol:.1e}"
        band += 1
    return band


@pytest.mark.parametrize("vocab,rows,T", [(1024, 7, 1.0), (20000, 5, 0.6), (151936, 3, 1.4)])
def test_sample_logits_parity(gpu_lib, vocab, rows, T):
    torch = _torch()
    cfg, W, dr = _drafter(vocab)
    z = np.random.default_rng(vocab).normal(0, 2.0, (rows, vocab)).astype(np.float32)
    zt = torch.from_numpy(z).cuda()
    for step in (0, 3):
        tok = dr.sample_logits(zt, T, SEED, step, row0=11).cpu().numpy()
        band = _check_samples(tok, z, T, step, 11 + np.arange(rows), f"V={vocab} step {step}")
        gh.log(f"[sample_logits] V {vocab} step {step}: {rows} rows, {band} in the tie band")


def _verify_case(vocab, B, batch, T, accept_bias, stops, budget_lo, seed_case):
    """Synthetic logits: draft rows N(0, 1.5); target rows either independent
    (low acceptance) or the draft row plus small noise (p close to q: long
    accepted prefixes, some blocks fully accepted and given a bonus token)."""
    g = np.random.default_rng(seed_case)
    zd = g.normal(0, 1.5, (batch, B - 1, vocab)).astype(np.float32)
    zt = g.normal(0, 1.5, (batch, B, vocab)).astype(np.float32)
    for b in range(batch):
        if accept_bias[b]:
            zt[b, :B - 1] = zd[b] + g.normal(0, 0.05, (B - 1, vocab)).astype(np.float32)
    draft = np.stack([S.sample_rows(zd[b], T, seed_case, 99, b * (B - 1) + np.arange(B - 1))[0]
                      for b in range(batch)]).astype(np.int32)
    budget = g.integers(budget_lo, 2 * B, batch).astype(np.int32)
    return zd, zt, draft, budget


@pytest.mark.parametrize("vocab,B,batch,T", [(1024, 8, 6, 1.0), (20000, 16, 4, 0.7), (151936, 16, 3, 1.3)])
def test_verify_sample_parity(gpu_lib, vocab, B, batch, T):
    torch = _torch()
    cfg = synth.CONFIGS["c1"].with_(vocab=vocab, block=B)
    W = synth.make_weights(cfg)
    dr = Drafter(cfg, W, batch=batch, max_ctx=256, max_rows=batch * B)
    ctx = np.arange(batch) * 7 + 20
    dr.ctx_len.copy_(torch.tensor(ctx, dtype=torch.int32))
    accept_bias = [b % 2 == 1 for b in range(batch)]
    zd, zt, draft, budget = _verify_case(vocab, B, batch, T, accept_bias, None, 3, 1000 + vocab)
    stop = int(draft[1, 2]) if batch > 1 else None  # a stop id that some emitted row contains
    stops = [stop] if stop is not None else []
    step = 5
    d_dev = torch.from_numpy(draft).cuda()
    zd_dev = torch.from_numpy(zd.reshape(batch * (B - 1), vocab)).cuda()
    zt_dev = torch.from_numpy(zt.reshape(batch * B, vocab)).cuda()
    bud = torch.from_numpy(budget.copy()).cuda()
    stop_dev = torch.tensor(stops, dtype=torch.int32, device="cuda") if stops else None
    dr.verify_sample(zt_dev, T, SEED, step, stop_dev, bud, draft=d_dev, draft_logits=zd_dev)
    torch.cuda.synchronize()
    r = S.verify_sample(draft, zd, zt, T, SEED, step, ctx, stop_ids=stops, budget=budget)
    m_dev = dr.accept_len.cpu().numpy()
    # residual scores log(p - q) lose accuracy where p and q nearly cancel
    tol = max(1e-3, _score_tol(np.concatenate([zd.ravel(), zt.ravel()]), T))
    band = 0
    for b in range(batch):
        am = r["accept_margin"][b]
        tested = am[~np.isnan(am)]
        if np.any(np.abs(tested) < 1e-4) or r["sample_margin"][b] < tol:
            band += 1  # a decision within rounding of its threshold: not compared
            continue
        assert m_dev[b] == r["accept_len"][b], f"seq {b}: accept_len {m_dev[b]} vs {r['accept_len'][b]}"
        assert int(dr.anchor_out[b]) == r["anchor_out"][b], f"seq {b}: new token"
        n = int(r["n_emit"][b])
        assert int(dr.n_emit[b]) == n
        assert dr.emitted[b, :n].cpu().numpy().tolist() == r["emitted"][b, :n].tolist()
        assert int(dr.done[b]) == r["done"][b]
        assert int(bud[b]) == r["budget"][b]
    if band == 0:
        nc = int(dr.n_commit.item())
        assert np.array_equal(dr.commit_rows[:nc].cpu().numpy(), r["commit_rows"])
    gh.log(f"[verify_sample] V {vocab} B {B} batch {batch}: accept {m_dev.tolist()} "
           f"(oracle {r['accept_len'].tolist()}), {band} sequences in the tie band")
    assert band <= max(1, batch // 3)
    # the accepted prefixes really vary: low and high acceptance both occur
    assert m_dev.min() < B - 1


def test_draft_block_sample_parity(gpu_lib):
    """The sampled draft block's logits match the oracle's draft block, and its
    tokens are the Gumbel-max samples of those logits; a greedy block after it
    still returns the argmax."""
    torch = _torch()
    cfg, W, dr = _drafter(batch=2)
    WO = gh.oracle_weights(W)
    ocfg = ref.OracleConfig.from_any(cfg)
    L, B, V = cfg.ctx_len, cfg.block, cfg.vocab
    cache = ref.new_cache(ocfg, 2, 256)
    for b in range(2):
        taps = synth.make_taps(cfg, L - 5 * b, tid=b)
        dr.ingest(b, torch.from_numpy(taps.view(np.int16)).view(torch.bfloat16).cuda())
        ref.inject_kv(ocfg, WO, ref.fuse_ctx(ocfg, WO, synth.bf16_to_f64(taps)),
                      [(r, b, r) for r in range(L - 5 * b)], cache)
    anchor = np.array([5, 17], np.int32)
    dr.anchor.copy_(torch.from_numpy(anchor))
    T, step = 0.8, 7
    dr.draft_block_sample(T, SEED, step)
    torch.cuda.synchronize()
    z = dr.draft_logits.cpu().numpy()
    tok = dr.draft.cpu().numpy().reshape(-1)
    want = ref.draft_block(ocfg, WO, cache, [L, L - 5], anchor)
    gh.check_rel(z, want["logits"].reshape(2 * (B - 1), V), what="sampled block logits", rows=True)
    band = _check_samples(tok, z, T, step, np.arange(2 * (B - 1)), "draft samples")
    assert not np.array_equal(tok, np.argmax(z, axis=1))  # a sample, not the argmax
    dr.draft_block()
    torch.cuda.synchronize()
    assert np.array_equal(dr.draft.cpu().numpy().reshape(-1), np.argmax(z, axis=1))
    gh.log(f"[draft_block_sample] {band} rows in the tie band")


def test_sampling_loop_step_by_step(gpu_lib):
    """The sampling loop with drafter and target on the device: every step's
    drafts are the Gumbel-max samples of its draft logits and every verify
    outcome is the oracle's speculative-sampling outcome on that step's
    logits; the loop is deterministic in its seed."""
    cfg = synth.CONFIGS["c1"]
    W = synth.make_weights(cfg)
    TW = synth.make_target_weights(cfg, W)
    prompt = list(synth.make_prompt(cfg, 40))
    B = cfg.block
    max_ctx = 40 + cfg.n_new + 2 * B + 8
    tgt = DeviceTarget(cfg, TW, cfg.target_layers, cfg.tap_layers, max_ctx=max_ctx, max_n=B)
    dr = Drafter(cfg, W, batch=1, max_ctx=max_ctx, max_rows=64)
    T = 0.9
    trace = []
    out, ms = _spec_sample(dr, tgt, prompt, cfg.n_new, (), T, SEED, trace=trace)
    assert len(out) == cfg.n_new and all(0 <= t < cfg.vocab for t in out)
    band = 0
    L = 40
    for s in trace:
        zd = s["draft_logits"]
        band += _check_samples(s["draft"].reshape(-1), zd, T, s["step"], np.arange(B - 1), f"step {s['step']}")
        r = S.verify_sample(s["draft"], zd.reshape(1, B - 1, -1), s["target_logits"].reshape(1, B, -1), T, SEED,
                            s["step"], [L])
        am = r["accept_margin"][0]
        if np.any(np.abs(am[~np.isnan(am)]) < 1e-4) or r["sample_margin"][0] < 1e-3:
            band += 1
        else:
            assert s["accept_len"] == r["accept_len"][0], f"step {s['step']}"
            n = len(s["emitted"])  # the token budget may cut the last step short
            assert s["emitted"] == r["emitted"][0, :n].tolist() and n <= r["n_emit"][0]
            assert n == r["n_emit"][0] or s is trace[-1]
        L += s["accept_len"] + 1
    gh.log(f"[sampling loop] {len(trace)} steps, mean accepted {np.mean(ms):.2f}, {band} tie-band decisions")
    again, _ = _spec_sample(dr, tgt, prompt, cfg.n_new, (), T, SEED)
    assert again == out
    other, _ = _spec_sample(dr, tgt, prompt, cfg.n_new, (), T, SEED + 1)
    assert other != out


def test_device_loop_sampling_matches_host_loop(gpu_lib):
    """Sampling in the loop with no per-step host synchronisation (steps
    captured in a graph, with the draws' step counter advanced on the device,
    and run eagerly): one sequence emits exactly what the host-driven sampling
    loop emits; in a batch of two, the first sequence (whose RNG rows are
    those of a batch of one) emits the same again, and graph and eager runs
    agree. A replayed graph that froze the step would repeat its draws and
    diverge from the host loop."""
    import torch
    cfg = synth.CONFIGS["c1"]
    W = synth.make_weights(cfg)
    TW = synth.make_target_weights(cfg, W)
    prompts = [list(synth.make_prompt(cfg, 64)), list(synth.make_prompt(cfg, 37, seed=11))]
    n_new, S, T = cfg.n_new, 4, 0.9
    max_ctx = 64 + n_new + (S + 2) * cfg.block + 16
    tgt1 = DeviceTarget(cfg, TW, cfg.target_layers, cfg.tap_layers, max_ctx=max_ctx, max_n=16)
    dr1 = Drafter(cfg, W, batch=1, max_ctx=max_ctx, max_rows=64)
    host, ms = _spec_sample(dr1, tgt1, prompts[0], n_new, (), T, SEED)
    assert len(ms) > S  # more steps than one graph holds: replays must draw afresh
    for graph in (True, False):
        one = spec_generate_device(dr1, tgt1, prompts[:1], n_new, steps_per_sync=S, graph=graph,
                                   temperature=T, seed=SEED)
        assert one[0] == host, f"batch 1, graph={graph}"
    del tgt1, dr1
    tgt = DeviceTarget(cfg, TW, cfg.target_layers, cfg.tap_layers, batch=2, max_ctx=max_ctx, max_n=16)
    dr = Drafter(cfg, W, batch=2, max_ctx=max_ctx, max_rows=2 * 16)
    outs = [spec_generate_device(dr, tgt, prompts, n_new, steps_per_sync=S, graph=graph, temperature=T, seed=SEED)
            for graph in (True, False)]
    assert outs[0] == outs[1]
    assert outs[0][0] == host
    assert len(outs[0][1]) == n_new and all(0 <= t < cfg.vocab for t in outs[0][1])
    torch.cuda.synchronize()
    gh.log(f"[device sampling loop] {len(ms)} host steps, mean accepted {np.mean(ms):.2f}")
