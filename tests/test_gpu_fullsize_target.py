"""Target verify pass at the benchmarked layer shape: a 3-layer target of the
Qwen3-8B-shaped layer (H 4096, 32/8 heads of 128, I 12288, V 151936), every
layer tapped, batch 2 with ragged contexts of 1024 and 700 tokens (prefilled on
the device in passes of 16), then one causal pass of 16 tokens per sequence.

Checked against the fp64 oracle, stage by stage from the device's state: every
layer of the pass replayed from the previous layer's tap (the embedding for the
first) and the device's cache of that layer, with the causal mask inside the
block (row j sees keys < L + j + 1) over all L + 16 keys; the block's K/V
written at slots [L, L + 16); the full LM head from the last tap (logits and
argmax, tokens up to the tie band); context slots left as committed.
"""
import numpy as np
import pytest

import gpu_helpers as gh
from block_diffusion_drafter_target_amd import DeviceTarget, synth
from oracle import ref

pytestmark = pytest.mark.gpu

LENS = (1024, 700)
N = 16
LAYERS = 3


@pytest.fixture(scope="module")
def target(gpu_lib):
    import torch
    cfg = synth.CONFIGS["c2"].with_(batch=len(LENS), target_layers=LAYERS, tap_layers=tuple(range(LAYERS)))
    gh.log("[fullsize target] generating weights")
    W = synth.make_weights(cfg, only={"embed", "lm_head"})
    TW = synth.make_target_weights(cfg, W)
    batch = len(LENS)
    tgt = DeviceTarget(cfg, TW, LAYERS, cfg.tap_layers, batch=batch, max_ctx=max(LENS) + 2 * N + 64, max_n=N)
    lens = torch.tensor(LENS, dtype=torch.int32, device="cuda")
    gh.log("[fullsize target] prefill in passes of 16")
    for i0 in range(0, max(LENS), N):
        toks = np.stack([synth.make_prompt(cfg, N, seed=1000 + 7 * b + i0) for b in range(batch)]).astype(np.int32)
        tgt.pass_tokens(torch.from_numpy(toks).cuda())
        tgt.ctx_len.copy_(torch.minimum(tgt.ctx_len + N, lens))
    torch.cuda.synchronize()
    assert tgt.ctx_len.cpu().tolist() == list(LENS)
    k_before = [tgt.k[:, b, :, :L].clone() for b, L in enumerate(LENS)]
    toks = np.stack([synth.make_prompt(cfg, N, seed=5000 + b) for b in range(batch)]).astype(np.int32)
    gh.log("[fullsize target] causal pass of 16 tokens")
    z = torch.empty((batch * N, cfg.vocab), dtype=torch.float32, device="cuda")
    a, t = tgt.pass_tokens(torch.from_numpy(toks).cuda(), dbg_logits=z)
    torch.cuda.synchronize()
    assert tgt.status.cpu().tolist() == [0] * batch
    assert tgt.ctx_len.cpu().tolist() == list(LENS)  # a pass writes speculatively, commits nothing
    for b, L in enumerate(LENS):
        assert bool(torch.equal(tgt.k[:, b, :, :L], k_before[b])), "committed context slots changed"
    out = {"toks": toks, "argmax": a.cpu().numpy().copy(), "taps": gh.to_np_bf16(t).reshape(batch, N, LAYERS, -1),
           "logits": z.cpu().numpy().astype(np.float64).reshape(batch, N, cfg.vocab)}
    return cfg, W, TW, tgt, out


def test_target_layers_stage_replay(target):
    cfg, W, TW, tgt, out = target
    ocfg = ref.OracleConfig.from_any(cfg)
    for l in range(LAYERS):
        LW = {k: synth.bf16_to_f64(v) for k, v in TW.items() if k.startswith(f"layers.{l}.")}
        for b, L in enumerate(LENS):
            gh.log(f"[fullsize target] replay layer {l} sequence {b}")
            x = (synth.bf16_to_f64(TW["embed"][out["toks"][b]]) if l == 0 else out["taps"][b, :, l - 1])
            pos = L + np.arange(N)
            allowed = np.arange(L + N)[None, :] <= pos[:, None]
            kc = gh.to_np_bf16(tgt.k[l, b, :, :L]).transpose(1, 0, 2)
            vc = gh.to_np_bf16(tgt.v[l, b, :, :L]).transpose(1, 0, 2)
            want, kb, vb = ref.decoder_layer(ocfg, LW, l, x, pos, kc, vc, allowed=allowed)
            e = gh.check_rel(out["taps"][b, :, l], want, what=f"layer {l} seq {b}", rows=True)
            kd = gh.to_np_bf16(tgt.k[l, b, :, L:L + N]).transpose(1, 0, 2)
            vd = gh.to_np_bf16(tgt.v[l, b, :, L:L + N]).transpose(1, 0, 2)
            gh.check_rel(kd, kb, what=f"block K layer {l} seq {b}", axis=1)
            gh.check_rel(vd, vb, what=f"block V layer {l} seq {b}", axis=1)
            gh.log(f"    rel err {e:.2e}")


def test_target_lm_head_and_argmax(target):
    cfg, W, TW, tgt, out = target
    gh.log("[fullsize target] LM head (full vocabulary, fp64)")
    lm = synth.bf16_to_f64(TW["lm_head"])
    gf = synth.bf16_to_f64(TW["g_final"])
    for b in range(len(LENS)):
        # replayed from the bf16 tap of the last layer (one more rounding per element)
        fin = ref.rms_norm(out["taps"][b, :, LAYERS - 1], gf, cfg.rms_eps)
        z = fin @ lm.T
        e = gh.check_rel(out["logits"][b], z, what=f"logits seq {b}", rows=True)
        assert np.array_equal(out["argmax"][b], np.argmax(out["logits"][b], axis=1))
        band = gh.check_tokens(out["argmax"][b], out["logits"][b], z, gh.replay_band(fin, lm, roundings=2),
                               what=f"argmax seq {b}")
        gh.log(f"    seq {b}: rel err {e:.2e}, tie-band rows {band}/{N}")
