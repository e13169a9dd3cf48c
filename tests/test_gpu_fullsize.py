"""Full-size parity at the benchmarked workload: the Qwen3-8B-shaped 5-layer
drafter (H 4096, 32/8 heads of 128, I 12288, V 151936, 5 taps), batch 1,
block 16, context 1024, in the launch configuration bench.py times (same
cache capacity, hence the same attention split).

Checked against the fp64 oracle: sampled fuse rows; K/V cache rows of every
layer (stage replay from the device's context feature); every layer's output
from the device's own input and cache (stage replay); the full LM head from the
device's final hidden state (logits and tokens); an end-to-end oracle draft
from the same taps; verify on synthetic targets.
"""
import numpy as np
import pytest

import gpu_helpers as gh
from block_diffusion_drafter_target_amd import Drafter, synth
from oracle import ref

pytestmark = pytest.mark.gpu

# bench.py defaults: 1 bootstrap + 20 warmup + 200 timed + 20 breakdown steps
BENCH_STEPS = 1 + 20 + 200 + 20


def _bf16_dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


@pytest.fixture(scope="module")
def c2(gpu_lib):
    import torch
    cfg = synth.CONFIGS["c2"]
    L, B = cfg.ctx_len, cfg.block
    gh.log("[fullsize c2] generating weights")
    W = synth.make_weights(cfg)
    max_ctx = L + (BENCH_STEPS + 2) * B + 64
    dr = Drafter(cfg, W, batch=1, max_ctx=max_ctx, max_rows=L)
    taps = synth.make_taps(cfg, L, tid=0)
    gh.log("[fullsize c2] ingest + draft_block")
    dr.ingest(0, _bf16_dev(torch, taps))
    anchor = synth.make_anchors(cfg)
    dr.anchor.copy_(torch.from_numpy(anchor))
    logits = torch.empty((B - 1, cfg.vocab), dtype=torch.float32, device="cuda")
    hidden = torch.empty((cfg.n_layers + 1, B, cfg.hidden), dtype=torch.float32, device="cuda")
    dr.draft_block(dbg_logits=logits, dbg_hidden=hidden)
    torch.cuda.synchronize()
    out = {"draft": dr.draft.cpu().numpy()[0], "logits": logits.cpu().numpy().astype(np.float64),
           "hidden": hidden.cpu().numpy().astype(np.float64)}
    assert dr.status.cpu().tolist() == [0]
    return cfg, W, dr, taps, anchor, out


def _layer_w(W, l):
    keys = [k for k in W if k.startswith(f"layers.{l}.")]
    return {k: synth.bf16_to_f64(W[k]) for k in keys}


def test_fullsize_fuse_and_inject(c2):
    import torch
    cfg, W, dr, taps, anchor, out = c2
    ocfg = ref.OracleConfig.from_any(cfg)
    rows = [0, 1, 517, cfg.ctx_len - 1]
    gh.log("[fullsize c2] fuse rows %s" % rows)
    ctx = torch.empty((len(rows), cfg.hidden), dtype=torch.bfloat16, device="cuda")
    dr.fuse_ctx(_bf16_dev(torch, taps[rows]), len(rows), ctx)
    torch.cuda.synchronize()
    got = gh.to_np_bf16(ctx)
    WF = {"w_fc": synth.bf16_to_f64(W["w_fc"]), "g_fc": synth.bf16_to_f64(W["g_fc"])}
    want = ref.fuse_ctx(ocfg, WF, synth.bf16_to_f64(taps[rows]))
    gh.check_rel(got, want, what="fuse rows", rows=True)
    # injected K/V of those positions in every layer, from the device's ctx
    for l in range(cfg.n_layers):
        LW = _layer_w(W, l)
        k, v = ref.project_kv(ocfg, LW, l, got, np.array(rows))
        kd = gh.to_np_bf16(dr.k[l, 0][:, rows]).transpose(1, 0, 2)
        vd = gh.to_np_bf16(dr.v[l, 0][:, rows]).transpose(1, 0, 2)
        gh.check_rel(kd, k, what=f"K layer {l}", axis=1)
        gh.check_rel(vd, v, what=f"V layer {l}", axis=1)


def test_fullsize_layers_stage_replay(c2):
    cfg, W, dr, taps, anchor, out = c2
    ocfg = ref.OracleConfig.from_any(cfg)
    L, B = cfg.ctx_len, cfg.block
    pos = L + np.arange(B)
    for l in range(cfg.n_layers):
        gh.log(f"[fullsize c2] replay layer {l}")
        LW = _layer_w(W, l)
        kc = gh.to_np_bf16(dr.k[l, 0, :, :L]).transpose(1, 0, 2)
        vc = gh.to_np_bf16(dr.v[l, 0, :, :L]).transpose(1, 0, 2)
        want, kb, vb = ref.decoder_layer(ocfg, LW, l, out["hidden"][l], pos, kc, vc)
        e = gh.check_rel(out["hidden"][l + 1], want, tol=1e-2, what=f"layer {l}", rows=True)
        gh.log(f"    rel err {e:.2e}")
        kbl = gh.to_np_bf16(dr.k[l, 0, :, L:L + B]).transpose(1, 0, 2)
        gh.check_rel(kbl, kb, what=f"block K layer {l}", axis=1)


def test_fullsize_lm_head_and_tokens(c2):
    cfg, W, dr, taps, anchor, out = c2
    gh.log("[fullsize c2] LM head (full vocabulary, fp64)")
    fin = ref.rms_norm(out["hidden"][cfg.n_layers][1:], synth.bf16_to_f64(W["g_final"]), cfg.rms_eps)
    lm = synth.bf16_to_f64(W["lm_head"])
    z = fin @ lm.T
    e = gh.check_rel(out["logits"], z, tol=1e-2, what="logits", rows=True)
    band = gh.check_tokens(out["draft"], out["logits"], z, gh.replay_band(fin, lm), what="draft tokens")
    gh.log(f"    rel err {e:.2e}, tie-band rows {band}/{len(out['draft'])}")


def test_fullsize_end_to_end(c2):
    cfg, W, dr, taps, anchor, out = c2
    gh.log("[fullsize c2] end-to-end oracle draft (fp64)")
    ocfg = ref.OracleConfig.from_any(cfg)
    WO = gh.oracle_weights(W)
    cache = ref.new_cache(ocfg, 1, cfg.ctx_len)
    ref.inject_kv(ocfg, WO, ref.fuse_ctx(ocfg, WO, synth.bf16_to_f64(taps)),
                  [(r, 0, r) for r in range(cfg.ctx_len)], cache)
    r = ref.draft_block(ocfg, WO, cache, [cfg.ctx_len], anchor)
    for l in range(cfg.n_layers + 1):
        gh.check_rel(out["hidden"][l], r["hidden"][0, l], what=f"hidden {l}", rows=True)
    e = gh.check_rel(out["logits"], r["logits"][0], what="logits", rows=True)
    band = gh.check_tokens(out["draft"], out["logits"], r["logits"][0], gh.e2e_band(r["logits"][0]), what="tokens")
    gh.log(f"    logits rel err {e:.2e}, tie-band rows {band}")


def test_fullsize_verify(c2):
    import torch
    cfg, W, dr, taps, anchor, out = c2
    B = cfg.block
    for step in range(8):
        m = synth.geometric_accept(1, B, 0.8, step=step)
        tgt = synth.synth_target_tokens(out["draft"][None], m, cfg.vocab, step=step)
        dr.verify_accept(torch.from_numpy(tgt).cuda())
        torch.cuda.synchronize()
        r = ref.verify_accept(out["draft"][None], tgt, [cfg.ctx_len])
        assert int(dr.accept_len.item()) == int(r["accept_len"][0]) == int(m[0])
        n = int(dr.n_commit.item())
        assert np.array_equal(dr.commit_rows.cpu().numpy()[:n], r["commit_rows"])
        assert np.array_equal(dr.emitted.cpu().numpy(), r["emitted"])


def test_fullsize_random_gains_layer(gpu_lib):
    """One layer of the benchmarked shape with random norm gains (g_fc, g_in,
    g_q, g_k, g_post, g_final each its own draw): fused rows, injected K/V, the
    layer replayed from the device's input and cache, and the full LM head."""
    import torch
    cfg = synth.CONFIGS["c2"].with_(n_layers=1)
    L, B = cfg.ctx_len, cfg.block
    ocfg = ref.OracleConfig.from_any(cfg)
    gh.log("[fullsize c2, random gains] one layer, context 1024")
    W = synth.make_weights(cfg, gains="random")
    dr = Drafter(cfg, W, batch=1, max_ctx=L + 2 * B, max_rows=L)
    taps = synth.make_taps(cfg, L, tid=0)
    dr.ingest(0, _bf16_dev(torch, taps))
    dr.anchor.copy_(torch.from_numpy(synth.make_anchors(cfg)))
    logits = torch.empty((B - 1, cfg.vocab), dtype=torch.float32, device="cuda")
    hidden = torch.empty((2, B, cfg.hidden), dtype=torch.float32, device="cuda")
    dr.draft_block(dbg_logits=logits, dbg_hidden=hidden)
    rows = [0, 333, L - 1]
    ctx = torch.empty((len(rows), cfg.hidden), dtype=torch.bfloat16, device="cuda")
    dr.fuse_ctx(_bf16_dev(torch, taps[rows]), len(rows), ctx)
    torch.cuda.synchronize()
    assert dr.status.cpu().tolist() == [0]
    LW = _layer_w(W, 0)
    WF = {"w_fc": synth.bf16_to_f64(W["w_fc"]), "g_fc": synth.bf16_to_f64(W["g_fc"])}
    got = gh.to_np_bf16(ctx)
    gh.check_rel(got, ref.fuse_ctx(ocfg, WF, synth.bf16_to_f64(taps[rows])), what="fuse rows", rows=True)
    k, v = ref.project_kv(ocfg, LW, 0, got, np.array(rows))
    gh.check_rel(gh.to_np_bf16(dr.k[0, 0][:, rows]).transpose(1, 0, 2), k, what="K rows", axis=1)
    gh.check_rel(gh.to_np_bf16(dr.v[0, 0][:, rows]).transpose(1, 0, 2), v, what="V rows", axis=1)
    hid = hidden.cpu().numpy().astype(np.float64)
    # the embedding row is the embedding itself (the input norm's gain acts inside the layer)
    E = synth.bf16_to_f64(W["embed"])
    toks = [int(dr.anchor.item())] + [cfg.mask_id] * (B - 1)
    assert np.array_equal(hid[0], E[toks])
    kc = gh.to_np_bf16(dr.k[0, 0, :, :L]).transpose(1, 0, 2)
    vc = gh.to_np_bf16(dr.v[0, 0, :, :L]).transpose(1, 0, 2)
    want, kb, vb = ref.decoder_layer(ocfg, LW, 0, hid[0], L + np.arange(B), kc, vc)
    e = gh.check_rel(hid[1], want, tol=1e-2, what="layer 0", rows=True)
    gh.check_rel(gh.to_np_bf16(dr.k[0, 0, :, L:L + B]).transpose(1, 0, 2), kb, what="block K", axis=1)
    gh.check_rel(gh.to_np_bf16(dr.v[0, 0, :, L:L + B]).transpose(1, 0, 2), vb, what="block V", axis=1)
    fin = ref.rms_norm(hid[1][1:], synth.bf16_to_f64(W["g_final"]), cfg.rms_eps)
    lm = synth.bf16_to_f64(W["lm_head"])
    z = fin @ lm.T
    el = gh.check_rel(logits.cpu().numpy(), z, tol=1e-2, what="logits", rows=True)
    band = gh.check_tokens(dr.draft.cpu().numpy()[0], logits.cpu().numpy(), z, gh.replay_band(fin, lm),
                           what="tokens")
    gh.log(f"    layer rel err {e:.2e}, logits {el:.2e}, tie-band rows {band}")
