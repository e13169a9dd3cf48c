"""Full-size parity at the block-size sweep workload: the Qwen3-8B-shaped
5-layer drafter (H 4096, 32/8 heads of 128, I 12288, V 151936, 5 taps),
batch 8, context 8192 per sequence, block 8, 12 and 16.

The context is ingested once (65,536 rows) by the block-16 drafter; the cache
does not depend on the block size, so the block-8 and block-12 drafters start
from a copy of it. The fp64 oracle cannot redo the whole ingest at this size,
so every check is sampled or replayed stage by stage from the device's state:
  * fuse and inject of sampled context rows of two sequences, in every layer;
  * for every block size, every layer of two sequences from the device's own
    layer input and cache (fp64 attention over all 8192 + B keys), the block's
    K/V appended at slots [8192, 8192 + B);
  * for every block size, the full LM head of those sequences' rows in fp64
    (logits and tokens), and one verify step of all eight sequences on
    synthetic targets (accept lengths, emitted tokens and commit rows bit
    exact, ctx_len left alone).
Every drafter runs the attention split of bench.py's launch (the chunk count
per sequence and kv head depends on the batch and the kv heads only here).
"""
import numpy as np
import pytest

import gpu_helpers as gh
from block_diffusion_drafter_target_amd import Drafter, synth
from oracle import ref

pytestmark = pytest.mark.gpu

BLOCKS = (8, 12, 16)
ROWS = (0, 1, 4099, 8191)  # sampled context rows
SEQS = (0, 7)              # sequences replayed in fp64
L = 8192


def _bf16_dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _cache(dr, l, b, lo, hi):
    """Device K and V of layer l, sequence b, slots [lo, hi) as [n, Hkv, D] fp64."""
    k = gh.to_np_bf16(dr.k[l, b, :, lo:hi]).transpose(1, 0, 2)
    v = gh.to_np_bf16(dr.v[l, b, :, lo:hi]).transpose(1, 0, 2)
    return k, v


@pytest.fixture(scope="module")
def c4(gpu_lib):
    import torch
    cfg16 = synth.CONFIGS["c4"]
    assert cfg16.block == 16 and cfg16.ctx_len == L
    gh.log("[fullsize c4] generating weights")
    W = synth.make_weights(cfg16)
    max_ctx = L + 2 * max(BLOCKS) + 64
    drs = {16: Drafter(cfg16, W, batch=cfg16.batch, max_ctx=max_ctx, max_rows=L)}
    taps_rows = {}
    for b in range(cfg16.batch):
        gh.log(f"[fullsize c4] ingest sequence {b} ({L} rows)")
        t = synth.make_taps(cfg16, L, tid=b)
        drs[16].ingest(b, _bf16_dev(torch, t))
        if b in SEQS:
            taps_rows[b] = t[list(ROWS)].copy()
        del t
    torch.cuda.synchronize()
    assert drs[16].ctx_len.cpu().tolist() == [L] * cfg16.batch
    for B in BLOCKS:
        if B == 16:
            continue
        dr = Drafter(cfg16.with_(block=B), W, batch=cfg16.batch, max_ctx=max_ctx, max_rows=cfg16.batch * B)
        dr.k.copy_(drs[16].k)
        dr.v.copy_(drs[16].v)
        dr.ctx_len.copy_(drs[16].ctx_len)
        drs[B] = dr
    torch.cuda.synchronize()
    outs = {}
    for B in BLOCKS:
        dr, cfg = drs[B], drs[B].cfg
        gh.log(f"[fullsize c4] draft_block, block {B}")
        dr.anchor.copy_(torch.from_numpy(synth.make_anchors(cfg)))
        logits = torch.empty((cfg.batch * (B - 1), cfg.vocab), dtype=torch.float32, device="cuda")
        hidden = torch.empty((cfg.n_layers + 1, cfg.batch * B, cfg.hidden), dtype=torch.float32, device="cuda")
        dr.draft_block(dbg_logits=logits, dbg_hidden=hidden)
        torch.cuda.synchronize()
        assert dr.status.cpu().tolist() == [0] * cfg.batch
        assert dr.ctx_len.cpu().tolist() == [L] * cfg.batch  # drafting never commits
        outs[B] = {"draft": dr.draft.cpu().numpy().copy(), "logits": logits.cpu().numpy().astype(np.float64),
                   "hidden": hidden.cpu().numpy().astype(np.float64)}
    return cfg16, W, drs, taps_rows, outs


def test_c4_fuse_and_inject_sampled(c4):
    import torch
    cfg, W, drs, taps_rows, outs = c4
    ocfg = ref.OracleConfig.from_any(cfg)
    dr = drs[16]
    WF = {"w_fc": synth.bf16_to_f64(W["w_fc"]), "g_fc": synth.bf16_to_f64(W["g_fc"])}
    rows = np.array(ROWS)
    for b in SEQS:
        gh.log(f"[fullsize c4] fuse/inject rows {ROWS} of sequence {b}")
        ctx = torch.empty((len(ROWS), cfg.hidden), dtype=torch.bfloat16, device="cuda")
        dr.fuse_ctx(_bf16_dev(torch, taps_rows[b]), len(ROWS), ctx)
        torch.cuda.synchronize()
        got = gh.to_np_bf16(ctx)
        gh.check_rel(got, ref.fuse_ctx(ocfg, WF, synth.bf16_to_f64(taps_rows[b])), what=f"fuse seq {b}", rows=True)
        for l in range(cfg.n_layers):
            LW = {k: synth.bf16_to_f64(v) for k, v in W.items() if k.startswith(f"layers.{l}.")}
            k, v = ref.project_kv(ocfg, LW, l, got, rows)
            kd, vd = _cache(dr, l, b, 0, L)
            gh.check_rel(kd[rows], k, what=f"K seq {b} layer {l}", axis=1)
            gh.check_rel(vd[rows], v, what=f"V seq {b} layer {l}", axis=1)


def test_c4_layers_stage_replay(c4):
    cfg, W, drs, taps_rows, outs = c4
    for l in range(cfg.n_layers):
        LW = {k: synth.bf16_to_f64(v) for k, v in W.items() if k.startswith(f"layers.{l}.")}
        for B in BLOCKS:
            ocfg = ref.OracleConfig.from_any(drs[B].cfg)
            hid = outs[B]["hidden"]
            for b in SEQS:
                gh.log(f"[fullsize c4] block {B}: replay layer {l} sequence {b}")
                kc, vc = _cache(drs[B], l, b, 0, L)
                x = hid[l, b * B:(b + 1) * B]
                want, kb, vb = ref.decoder_layer(ocfg, LW, l, x, L + np.arange(B), kc, vc)
                e = gh.check_rel(hid[l + 1, b * B:(b + 1) * B], want, tol=1e-2, what=f"B{B} layer {l} seq {b}", rows=True)
                kbd, vbd = _cache(drs[B], l, b, L, L + B)
                gh.check_rel(kbd, kb, what=f"B{B} block K layer {l} seq {b}", axis=1)
                gh.check_rel(vbd, vb, what=f"B{B} block V layer {l} seq {b}", axis=1)
                gh.log(f"    rel err {e:.2e}")


def test_c4_lm_head_and_tokens(c4):
    cfg, W, drs, taps_rows, outs = c4
    gh.log("[fullsize c4] LM head (full vocabulary, fp64)")
    lm = synth.bf16_to_f64(W["lm_head"])
    gf = synth.bf16_to_f64(W["g_final"])
    for B in BLOCKS:
        o = outs[B]
        z_all = o["logits"].reshape(cfg.batch, B - 1, cfg.vocab)
        for b in SEQS:
            fin = ref.rms_norm(o["hidden"][cfg.n_layers, b * B + 1:(b + 1) * B], gf, cfg.rms_eps)
            z = fin @ lm.T
            e = gh.check_rel(z_all[b], z, tol=1e-2, what=f"B{B} logits seq {b}", rows=True)
            band = gh.check_tokens(o["draft"][b], z_all[b], z, gh.replay_band(fin, lm), what=f"B{B} draft tokens seq {b}")
            gh.log(f"    block {B} seq {b}: rel err {e:.2e}, tie-band rows {band}/{B - 1}")


def test_c4_verify_and_commit(c4):
    import torch
    cfg, W, drs, taps_rows, outs = c4
    for B in BLOCKS:
        dr = drs[B]
        draft = outs[B]["draft"]
        gh.log(f"[fullsize c4] block {B}: verify / commit")
        m = synth.geometric_accept(cfg.batch, B, 0.8, step=B)
        tgt = synth.synth_target_tokens(draft, m, cfg.vocab, step=B)
        dr.verify_accept(torch.from_numpy(tgt).cuda())
        torch.cuda.synchronize()
        r = ref.verify_accept(draft, tgt, [L] * cfg.batch)
        assert dr.accept_len.cpu().numpy().tolist() == r["accept_len"].tolist() == m.tolist()
        assert np.array_equal(dr.emitted.cpu().numpy(), r["emitted"])
        n = int(dr.n_commit.item())
        assert np.array_equal(dr.commit_rows.cpu().numpy()[:n], r["commit_rows"])
        assert dr.ctx_len.cpu().tolist() == [L] * cfg.batch  # verify never advances ctx_len
