"""Full-size parity at the ragged batched workload: the Qwen3-8B-shaped 5-layer
drafter, batch 32, block 16, context lengths uniform in 512..4096 per
sequence (seeded), then two draft / verify / commit steps.

At 512 block rows every GEMM runs on the large-tile kernel: two 256-row tiles
share each weight tile (direct global-to-LDS loads, the XCD-grouped tile
order), o and down with 8-way split-K, the LM head on 480 rows (the second row
tile ragged), and the attention chunks follow the batch's longest sequence.
The checks are sampled or replayed stage by stage from the device's state:
  * every layer of sequences 0 and 31 (block rows in the first and last row
    tile) from the device's own input and cache, with their block K/V;
  * the full LM head in fp64 for the rows of three sequences, one of them
    straddling the boundary of two row tiles (logits and tokens);
  * fuse and inject of sampled context rows of three sequences;
  * two steps of verify for all 32 sequences (bit exact) and commit
    (ctx_len), then the first layer of the next block of sequence 31
    replayed over [0, ctx_len).
"""
import numpy as np
import pytest

import gpu_helpers as gh
from block_diffusion_drafter_target_amd import Drafter, synth
from oracle import ref

pytestmark = pytest.mark.gpu

STEPS = 2
REPLAY_SEQS = (0, 31)
LM_SEQS = (0, 17, 31)  # sequence 17's LM rows are 255..269: rows 255 and 256 sit in different tiles
FUSE_SEQS = (0, 15, 31)


def _bf16_dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _layer_w(W, l):
    return {k: synth.bf16_to_f64(v) for k, v in W.items() if k.startswith(f"layers.{l}.")}


def _cache(dr, l, b, lo, hi):
    k = gh.to_np_bf16(dr.k[l, b, :, lo:hi]).transpose(1, 0, 2)
    v = gh.to_np_bf16(dr.v[l, b, :, lo:hi]).transpose(1, 0, 2)
    return k, v


def _draft(torch, dr, cfg, anchor=None):
    B, batch = cfg.block, cfg.batch
    logits = torch.empty((batch * (B - 1), cfg.vocab), dtype=torch.float32, device="cuda")
    hidden = torch.empty((cfg.n_layers + 1, batch * B, cfg.hidden), dtype=torch.float32, device="cuda")
    dr.draft_block(anchor=anchor, dbg_logits=logits, dbg_hidden=hidden)
    torch.cuda.synchronize()
    return {"draft": dr.draft.cpu().numpy().copy(), "logits": logits.cpu().numpy(),
            "hidden": hidden.cpu().numpy()}


@pytest.fixture(scope="module")
def c3(gpu_lib):
    import torch
    cfg = synth.CONFIGS["c3"]
    lens = synth.make_ctx_lens(cfg)
    B, batch = cfg.block, cfg.batch
    gh.log(f"[fullsize c3] contexts {int(lens.min())}..{int(lens.max())}, total {int(lens.sum())}")
    W = synth.make_weights(cfg)
    dr = Drafter(cfg, W, batch=batch, max_ctx=int(lens.max()) + (STEPS + 2) * B + 64, max_rows=int(lens.max()))
    rows = {}
    for b in range(batch):
        t = synth.make_taps(cfg, int(lens[b]), tid=b)
        dr.ingest(b, _bf16_dev(torch, t))
        if b in FUSE_SEQS:
            pick = np.array([0, int(lens[b]) // 2, int(lens[b]) - 1])
            rows[b] = (pick, t[pick].copy())
        del t
    torch.cuda.synchronize()
    assert dr.ctx_len.cpu().tolist() == lens.tolist()
    dr.anchor.copy_(torch.from_numpy(synth.make_anchors(cfg)))
    gh.log("[fullsize c3] draft_block")
    out = _draft(torch, dr, cfg)
    assert dr.status.cpu().tolist() == [0] * batch
    return cfg, W, dr, lens, rows, out


def test_c3_layers_stage_replay(c3):
    cfg, W, dr, lens, rows, out = c3
    ocfg = ref.OracleConfig.from_any(cfg)
    B = cfg.block
    for l in range(cfg.n_layers):
        LW = _layer_w(W, l)
        for b in REPLAY_SEQS:
            L = int(lens[b])
            kc, vc = _cache(dr, l, b, 0, L)
            x = out["hidden"][l, b * B:(b + 1) * B].astype(np.float64)
            want, kb, vb = ref.decoder_layer(ocfg, LW, l, x, L + np.arange(B), kc, vc)
            e = gh.check_rel(out["hidden"][l + 1, b * B:(b + 1) * B], want, tol=1e-2, what=f"layer {l} seq {b}", rows=True)
            kbd, vbd = _cache(dr, l, b, L, L + B)
            gh.check_rel(kbd, kb, what=f"block K layer {l} seq {b}", axis=1)
            gh.check_rel(vbd, vb, what=f"block V layer {l} seq {b}", axis=1)
            gh.log(f"[fullsize c3] layer {l} seq {b} (context {L}): rel err {e:.2e}")


def test_c3_lm_head_and_tokens(c3):
    cfg, W, dr, lens, rows, out = c3
    B, NL = cfg.block, cfg.n_layers
    lm = synth.bf16_to_f64(W["lm_head"])
    g = synth.bf16_to_f64(W["g_final"])
    for b in LM_SEQS:
        hid = out["hidden"][NL, b * B + 1:(b + 1) * B].astype(np.float64)
        fin = ref.rms_norm(hid, g, cfg.rms_eps)
        z = fin @ lm.T
        got = out["logits"][b * (B - 1):(b + 1) * (B - 1)].astype(np.float64)
        e = gh.check_rel(got, z, tol=1e-2, what=f"logits seq {b}", rows=True)
        band = gh.check_tokens(out["draft"][b], got, z, gh.replay_band(fin, lm), what=f"tokens seq {b}")
        gh.log(f"[fullsize c3] LM head seq {b}: rel err {e:.2e}, tie-band rows {band}")


def test_c3_fuse_and_inject_sampled(c3):
    import torch
    cfg, W, dr, lens, rows, out = c3
    ocfg = ref.OracleConfig.from_any(cfg)
    WF = {"w_fc": synth.bf16_to_f64(W["w_fc"]), "g_fc": synth.bf16_to_f64(W["g_fc"])}
    for b, (pick, taps) in rows.items():
        ctx = torch.empty((len(pick), cfg.hidden), dtype=torch.bfloat16, device="cuda")
        dr.fuse_ctx(_bf16_dev(torch, taps), len(pick), ctx)
        torch.cuda.synchronize()
        got = gh.to_np_bf16(ctx)
        gh.check_rel(got, ref.fuse_ctx(ocfg, WF, synth.bf16_to_f64(taps)), what=f"fuse seq {b}", rows=True)
        for l in range(cfg.n_layers):
            k, v = ref.project_kv(ocfg, _layer_w(W, l), l, got, pick)
            kd = gh.to_np_bf16(dr.k[l, b][:, pick]).transpose(1, 0, 2)
            vd = gh.to_np_bf16(dr.v[l, b][:, pick]).transpose(1, 0, 2)
            gh.check_rel(kd, k, what=f"K seq {b} layer {l}", axis=1)
            gh.check_rel(vd, v, what=f"V seq {b} layer {l}", axis=1)


def test_c3_verify_commit(c3):
    import torch
    cfg, W, dr, lens, rows, out = c3
    ocfg = ref.OracleConfig.from_any(cfg)
    B, batch = cfg.block, cfg.batch
    W0 = _layer_w(W, 0)
    taps_step = _bf16_dev(torch, synth.make_taps(cfg, batch * B, tid=999))
    ctx_len = lens.astype(np.int64).copy()
    draft = out["draft"]
    for step in range(STEPS):
        m = synth.geometric_accept(batch, B, 0.8, step=step)
        tgt = synth.synth_target_tokens(draft, m, cfg.vocab, step=step)
        dr.verify_accept(torch.from_numpy(tgt).cuda())
        torch.cuda.synchronize()
        r = ref.verify_accept(draft, tgt, ctx_len.tolist())
        assert dr.accept_len.cpu().numpy().tolist() == r["accept_len"].tolist() == m.tolist()
        assert np.array_equal(dr.emitted.cpu().numpy(), r["emitted"])
        n = int(dr.n_commit.item())
        assert np.array_equal(dr.commit_rows.cpu().numpy()[:n], r["commit_rows"])
        dr.fuse_ctx(taps_step, batch * B, dr.ctx)
        dr.inject_kv(dr.ctx, batch * B, dr.commit_rows, dr.n_commit, batch * B)
        torch.cuda.synchronize()
        ctx_len = ctx_len + m + 1
        assert dr.ctx_len.cpu().numpy().tolist() == ctx_len.tolist()
        nxt = _draft(torch, dr, cfg, anchor=dr.anchor_out)
        b = batch - 1
        L = int(ctx_len[b])
        kc, vc = _cache(dr, 0, b, 0, L)
        x = nxt["hidden"][0, b * B:(b + 1) * B].astype(np.float64)
        want, _, _ = ref.decoder_layer(ocfg, W0, 0, x, L + np.arange(B), kc, vc)
        gh.check_rel(nxt["hidden"][1, b * B:(b + 1) * B], want, tol=1e-2, what=f"step {step} next block seq {b}", rows=True)
        gh.log(f"[fullsize c3] step {step}: accept {m.tolist()[:8]}...")
        draft = nxt["draft"]
