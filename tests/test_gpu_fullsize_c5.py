"""Full-size parity at the gpt-oss-120b-shaped workload: the 8-layer drafter
(H 2880, 64/8 heads of 64, I 2880, V 201088, 5 taps), batch 4, block 16,
context 32768 per sequence, then a few draft / verify / commit steps.

The fp64 oracle cannot redo every context row at this size (the K/V
projection of the 131,072 context rows alone is about 390 GFLOP per layer),
so each check is sampled or replayed stage by stage from the device's state:
  * fuse and inject of sampled context rows of every sequence, in every layer;
  * every layer of two sequences from the device's own layer input and cache
    (attention over all 32,784 keys in fp64);
  * the full LM head of all 60 rows in fp64 (logits and tokens);
  * three steps of verify (bit exact against the oracle), commit (ctx_len and
    the committed K/V slots from the device's fused rows) and rollback (the
    next block's first layer replayed over [0, ctx_len) only, so a rejected
    slot that leaked into the attention would show).
"""
import numpy as np
import pytest

import gpu_helpers as gh
from block_diffusion_drafter_target_amd import Drafter, synth
from oracle import ref

pytestmark = pytest.mark.gpu

STEPS = 3
ROWS = (0, 1, 20011, 32767)  # sampled context rows of every sequence
REPLAY_SEQS = (0, 3)


def _bf16_dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _layer_w(W, l):
    return {k: synth.bf16_to_f64(v) for k, v in W.items() if k.startswith(f"layers.{l}.")}


def _cache(dr, l, b, lo, hi):
    """Device K and V of layer l, sequence b, slots [lo, hi) as [n, Hkv, D] fp64."""
    k = gh.to_np_bf16(dr.k[l, b, :, lo:hi]).transpose(1, 0, 2)
    v = gh.to_np_bf16(dr.v[l, b, :, lo:hi]).transpose(1, 0, 2)
    return k, v


def _draft(torch, dr, cfg, anchor=None):
    B, batch = cfg.block, cfg.batch
    logits = torch.empty((batch * (B - 1), cfg.vocab), dtype=torch.float32, device="cuda")
    hidden = torch.empty((cfg.n_layers + 1, batch * B, cfg.hidden), dtype=torch.float32, device="cuda")
    dr.draft_block(anchor=anchor, dbg_logits=logits, dbg_hidden=hidden)
    torch.cuda.synchronize()
    return {"draft": dr.draft.cpu().numpy().copy(), "logits": logits.cpu().numpy().astype(np.float64),
            "hidden": hidden.cpu().numpy().astype(np.float64)}


@pytest.fixture(scope="module")
def c5(gpu_lib):
    import torch
    cfg = synth.CONFIGS["c5"]
    lens = synth.make_ctx_lens(cfg)
    L, B, batch = int(lens.max()), cfg.block, cfg.batch
    assert max(ROWS) < int(lens.min())
    gh.log("[fullsize c5] generating weights")
    W = synth.make_weights(cfg)
    dr = Drafter(cfg, W, batch=batch, max_ctx=L + (STEPS + 2) * B + 64, max_rows=L)
    taps_rows = []
    for b in range(batch):
        gh.log(f"[fullsize c5] ingest sequence {b} ({int(lens[b])} rows)")
        t = synth.make_taps(cfg, int(lens[b]), tid=b)
        dr.ingest(b, _bf16_dev(torch, t))
        taps_rows.append(t[list(ROWS)].copy())
        del t
    torch.cuda.synchronize()
    assert dr.ctx_len.cpu().tolist() == lens.tolist()
    anchor = synth.make_anchors(cfg)
    dr.anchor.copy_(torch.from_numpy(anchor))
    gh.log("[fullsize c5] draft_block")
    out = _draft(torch, dr, cfg)
    assert dr.status.cpu().tolist() == [0] * batch
    return cfg, W, dr, lens, taps_rows, out


def test_c5_fuse_and_inject_sampled(c5):
    import torch
    cfg, W, dr, lens, taps_rows, out = c5
    ocfg = ref.OracleConfig.from_any(cfg)
    WF = {"w_fc": synth.bf16_to_f64(W["w_fc"]), "g_fc": synth.bf16_to_f64(W["g_fc"])}
    rows = np.array(ROWS)
    for b in range(cfg.batch):
        ctx = torch.empty((len(ROWS), cfg.hidden), dtype=torch.bfloat16, device="cuda")
        dr.fuse_ctx(_bf16_dev(torch, taps_rows[b]), len(ROWS), ctx)
        torch.cuda.synchronize()
        got = gh.to_np_bf16(ctx)
        gh.check_rel(got, ref.fuse_ctx(ocfg, WF, synth.bf16_to_f64(taps_rows[b])), what=f"fuse seq {b}", rows=True)
        for l in range(cfg.n_layers):
            k, v = ref.project_kv(ocfg, _layer_w(W, l), l, got, rows)
            kd = gh.to_np_bf16(dr.k[l, b][:, rows]).transpose(1, 0, 2)
            vd = gh.to_np_bf16(dr.v[l, b][:, rows]).transpose(1, 0, 2)
            gh.check_rel(kd, k, what=f"K seq {b} layer {l}", axis=1)
            gh.check_rel(vd, v, what=f"V seq {b} layer {l}", axis=1)


def test_c5_layers_stage_replay(c5):
    cfg, W, dr, lens, taps_rows, out = c5
    ocfg = ref.OracleConfig.from_any(cfg)
    B = cfg.block
    for l in range(cfg.n_layers):
        LW = _layer_w(W, l)
        for b in REPLAY_SEQS:
            L = int(lens[b])
            gh.log(f"[fullsize c5] replay layer {l} sequence {b}")
            kc, vc = _cache(dr, l, b, 0, L)
            x = out["hidden"][l, b * B:(b + 1) * B]
            want, kb, vb = ref.decoder_layer(ocfg, LW, l, x, L + np.arange(B), kc, vc)
            e = gh.check_rel(out["hidden"][l + 1, b * B:(b + 1) * B], want, tol=1e-2,
                             what=f"layer {l} seq {b}", rows=True)
            kbd, vbd = _cache(dr, l, b, L, L + B)
            gh.check_rel(kbd, kb, what=f"block K layer {l} seq {b}", axis=1)
            gh.check_rel(vbd, vb, what=f"block V layer {l} seq {b}", axis=1)
            gh.log(f"    rel err {e:.2e}")


def test_c5_lm_head_and_tokens(c5):
    cfg, W, dr, lens, taps_rows, out = c5
    B, NL = cfg.block, cfg.n_layers
    gh.log("[fullsize c5] LM head (all 60 rows, full vocabulary, fp64)")
    rows = [b * B + j for b in range(cfg.batch) for j in range(1, B)]
    fin = ref.rms_norm(out["hidden"][NL][rows], synth.bf16_to_f64(W["g_final"]), cfg.rms_eps)
    lm = synth.bf16_to_f64(W["lm_head"])
    z = fin @ lm.T
    e = gh.check_rel(out["logits"], z, tol=1e-2, what="logits", rows=True)
    band = gh.check_tokens(out["draft"].reshape(-1), out["logits"], z, gh.replay_band(fin, lm), what="draft tokens")
    gh.log(f"    rel err {e:.2e}, tie-band rows {band}/{len(rows)}")


def test_c5_verify_commit_rollback(c5):
    import torch
    cfg, W, dr, lens, taps_rows, out = c5
    ocfg = ref.OracleConfig.from_any(cfg)
    B, batch, NL = cfg.block, cfg.batch, cfg.n_layers
    WF = {"w_fc": synth.bf16_to_f64(W["w_fc"]), "g_fc": synth.bf16_to_f64(W["g_fc"])}
    W0, WL = _layer_w(W, 0), _layer_w(W, NL - 1)
    taps_step = synth.make_taps(cfg, batch * B, tid=999)
    ctx_len = lens.astype(np.int64).copy()
    draft = out["draft"]
    for step in range(STEPS):
        gh.log(f"[fullsize c5] step {step}: verify, commit, next block")
        m = synth.geometric_accept(batch, B, 0.8, step=step)
        tgt = synth.synth_target_tokens(draft, m, cfg.vocab, step=step)
        dr.verify_accept(torch.from_numpy(tgt).cuda())
        torch.cuda.synchronize()
        r = ref.verify_accept(draft, tgt, ctx_len.tolist())
        assert dr.accept_len.cpu().numpy().tolist() == r["accept_len"].tolist() == m.tolist()
        assert dr.anchor_out.cpu().numpy().tolist() == r["anchor_out"].tolist()
        assert np.array_equal(dr.emitted.cpu().numpy(), r["emitted"])
        assert dr.n_emit.cpu().numpy().tolist() == r["n_emit"].tolist()
        n = int(dr.n_commit.item())
        rows = dr.commit_rows.cpu().numpy()[:n]
        assert np.array_equal(rows, r["commit_rows"])
        # commit: fuse the block rows' taps, inject the accepted rows
        dr.fuse_ctx(_bf16_dev(torch, taps_step), batch * B, dr.ctx)
        dr.inject_kv(dr.ctx, batch * B, dr.commit_rows, dr.n_commit, batch * B)
        torch.cuda.synchronize()
        ctx_len = ctx_len + m + 1
        assert dr.ctx_len.cpu().numpy().tolist() == ctx_len.tolist()
        assert dr.status.cpu().tolist() == [0] * batch
        ctx = gh.to_np_bf16(dr.ctx[:batch * B])
        gh.check_rel(ctx, ref.fuse_ctx(ocfg, WF, synth.bf16_to_f64(taps_step)), what=f"step {step} fuse", rows=True)
        for l, LW in ((0, W0), (NL - 1, WL)):
            for b in range(batch):
                sel = rows[rows[:, 1] == b]
                k, v = ref.project_kv(ocfg, LW, l, ctx[sel[:, 0]], sel[:, 2])
                kd, vd = _cache(dr, l, b, int(sel[0, 2]), int(sel[-1, 2]) + 1)
                gh.check_rel(kd, k, what=f"step {step} committed K layer {l} seq {b}", axis=1)
                gh.check_rel(vd, v, what=f"step {step} committed V layer {l} seq {b}", axis=1)
        # next block from the new anchors; layer 0 of sequence 0 replayed over
        # [0, ctx_len) only: slots of the rejected block rows must not be read
        nxt = _draft(torch, dr, cfg, anchor=dr.anchor_out)
        L0 = int(ctx_len[0])
        kc, vc = _cache(dr, 0, 0, 0, L0)
        want, _, _ = ref.decoder_layer(ocfg, W0, 0, nxt["hidden"][0, :B], L0 + np.arange(B), kc, vc)
        gh.check_rel(nxt["hidden"][1, :B], want, tol=1e-2, what=f"step {step} next block layer 0", rows=True)
        draft = nxt["draft"]
