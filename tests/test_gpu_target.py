"""Target-side verify pass on the device (dflash_target_forward / dflash_kv_commit)
against the oracle's causal target, and the whole greedy loop with both models
on the device."""
import numpy as np
import pytest

import gpu_helpers as gh
from block_diffusion_drafter_target_amd import DeviceTarget, Drafter, spec_generate, spec_generate_device, synth
from oracle import ref

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _tiny(batch=1, max_ctx=256, max_n=16, gains="ones"):
    cfg = synth.CONFIGS["c1"]
    W = synth.make_weights(cfg, gains=gains)
    TW = synth.make_target_weights(cfg, W, gains=gains)
    dev = DeviceTarget(cfg, TW, cfg.target_layers, cfg.tap_layers, batch=batch, max_ctx=max_ctx, max_n=max_n)
    ocfg = ref.OracleConfig.from_any(cfg)
    return cfg, W, TW, dev, ocfg


def _oracle_target(cfg, ocfg, TW):
    return ref.TinyTarget(ocfg, gh.oracle_weights(TW), cfg.target_layers, cfg.tap_layers)


def assert_oracle_greedy(cfg, TW, prompt, got, stop_ids=(), what=""):
    """``got`` must be the fp64 oracle's plain greedy decoding of ``prompt``
    [P2 introduction; P3 introduction: the output is lossless]. A first
    difference is allowed only at a position where the oracle's own top-2 gap,
    after the common prefix, lies inside the tie band of the logits tolerance
    (2 * 2e-2 * max|z|); past it the two decodings continue from different
    tokens and are not compared. Returns the length of the common prefix."""
    ocfg = ref.OracleConfig.from_any(cfg)
    tgt = _oracle_target(cfg, ocfg, TW)
    want = ref.greedy_generate(tgt, prompt, len(got), stop_ids)
    same = next((i for i, (x, y) in enumerate(zip(got, want)) if x != y), min(len(got), len(want)))
    if same == len(got) == len(want):
        return same
    assert same < len(got) and same < len(want), f"{what}: lengths {len(got)} vs {len(want)}"
    tgt.reset()
    z, _ = tgt.forward(list(prompt) + list(got[:same]))
    z = z[-1]
    gap = z[want[same]] - z[got[same]]
    band = gh.e2e_band(z)
    assert gap <= band, f"{what}: token {same} is {got[same]}, oracle {want[same]}, gap {gap:.3e} > {band:.3e}"
    gh.log(f"    {what}: first difference from the oracle at token {same} (oracle gap {gap:.2e}, band {band:.2e})")
    return same


@pytest.mark.parametrize("gains", ["ones", "random"])
def test_target_pass_parity(gpu_lib, gains):
    """A 40-token prompt in passes of 16, 16 and 8 tokens (each causal over the
    cached context) against one oracle pass over all 40: logits, tokens, taps,
    and the K/V written to the cache; with unit and with random norm gains."""
    torch = _torch()
    cfg, W, TW, dev, ocfg = _tiny(gains=gains)
    prompt = synth.make_prompt(cfg, 40)
    gh.log(f"[target] prefill 40 tokens in passes of 16/16/8, gains {gains}")
    logits, toks, taps = [], [], []
    for i0 in range(0, 40, 16):
        part = torch.tensor(prompt[i0:i0 + 16], dtype=torch.int32, device="cuda")[None, :]
        z = torch.empty((part.shape[1], cfg.vocab), dtype=torch.float32, device="cuda")
        a, t = dev.pass_tokens(part, dbg_logits=z)
        torch.cuda.synchronize()
        logits.append(z.cpu().numpy())
        toks.append(a[0].cpu().numpy().copy())
        taps.append(gh.to_np_bf16(t))
        dev.ctx_len += part.shape[1]
    assert dev.status.cpu().tolist() == [0]
    z, tp, tk = np.concatenate(logits), np.concatenate(taps), np.concatenate(toks)
    tgt = _oracle_target(cfg, ocfg, TW)
    zr, tr = tgt.forward(prompt)
    e = gh.check_rel(z, zr, what="target logits", rows=True)
    gh.check_tokens(tk, z, zr, gh.e2e_band(zr), what="target argmax")
    gh.check_rel(tp, tr, what="target taps", rows=True)
    for l in range(cfg.target_layers):
        k = gh.to_np_bf16(dev.k[l, 0, :, :40]).transpose(1, 0, 2)
        v = gh.to_np_bf16(dev.v[l, 0, :, :40]).transpose(1, 0, 2)
        gh.check_rel(k, tgt.k[l], what=f"target K layer {l}", axis=1)
        gh.check_rel(v, tgt.v[l], what=f"target V layer {l}", axis=1)
    gh.log(f"    logits rel err {e:.2e}")


def test_target_ragged_batch_and_commit(gpu_lib):
    """Three sequences share a first pass of 16 tokens; verify-style commit
    rows keep 16, 5 and 12 of them, so a second 8-token pass runs over ragged
    contexts (the uncommitted slots are overwritten and never read)."""
    torch = _torch()
    cfg, W, TW, dev, ocfg = _tiny(batch=3)
    keep = [16, 5, 12]
    t1 = np.stack([synth.make_prompt(cfg, 16, seed=100 + b) for b in range(3)]).astype(np.int32)
    t2 = np.stack([synth.make_prompt(cfg, 8, seed=200 + b) for b in range(3)]).astype(np.int32)
    dev.pass_tokens(torch.from_numpy(t1).cuda())
    rows = np.array([(b * 16 + i, b, i) for b in range(3) for i in range(keep[b])], np.int32)
    max_commit = 48
    crow = torch.zeros((max_commit, 3), dtype=torch.int32, device="cuda")
    crow[:len(rows)] = torch.from_numpy(rows).cuda()
    ncom = torch.tensor([len(rows)], dtype=torch.int32, device="cuda")
    dev.commit(crow, ncom, max_commit)
    torch.cuda.synchronize()
    assert dev.ctx_len.cpu().tolist() == keep
    z = torch.empty((3 * 8, cfg.vocab), dtype=torch.float32, device="cuda")
    a, taps = dev.pass_tokens(torch.from_numpy(t2).cuda(), dbg_logits=z)
    torch.cuda.synchronize()
    z = z.cpu().numpy().reshape(3, 8, -1)
    a = a.cpu().numpy()
    tp = gh.to_np_bf16(taps).reshape(3, 8, -1)
    for b in range(3):
        tgt = _oracle_target(cfg, ocfg, TW)
        tgt.forward(t1[b, :keep[b]])
        zr, tr = tgt.forward(t2[b])
        gh.check_rel(z[b], zr, what=f"seq {b} logits", rows=True)
        gh.check_tokens(a[b], z[b], zr, gh.e2e_band(zr), what=f"seq {b} argmax")
        gh.check_rel(tp[b], tr, what=f"seq {b} taps", rows=True)


def test_target_capacity_and_commit_edges(gpu_lib):
    torch = _torch()
    cfg, W, TW, dev, ocfg = _tiny(batch=2, max_ctx=40)
    dev.ctx_len.copy_(torch.tensor([20, 30], dtype=torch.int32))
    toks = torch.from_numpy(np.stack([synth.make_prompt(cfg, 12, seed=7)] * 2).astype(np.int32)).cuda()
    a, _ = dev.pass_tokens(toks)
    torch.cuda.synchronize()
    assert dev.status.cpu().tolist() == [0, -5]  # 30 + 12 > 40
    assert a[1].cpu().tolist() == [-1] * 12
    assert all(0 <= t < cfg.vocab for t in a[0].cpu().tolist())
    # commit rows with an invalid sequence, a position past the cache and a
    # count above max_commit: only the valid rows within max_commit count
    rows = torch.tensor([[0, 0, 25], [1, 5, 3], [2, 0, 40], [3, 0, 31], [4, 1, 35]], dtype=torch.int32,
                        device="cuda")
    n = torch.tensor([99], dtype=torch.int32, device="cuda")
    dev.commit(rows, n, 4)
    torch.cuda.synchronize()
    assert dev.ctx_len.cpu().tolist() == [32, 30]


def test_loop_lossless_with_device_target(gpu_lib):
    """Greedy speculative decoding with the drafter and the target both on the
    device emits exactly what greedy decoding with the same device target
    does (a row's arithmetic does not depend on the rows beside it)."""
    cfg = synth.CONFIGS["c1"]
    W = synth.make_weights(cfg)
    TW = synth.make_target_weights(cfg, W)
    prompt = synth.make_prompt(cfg, cfg.ctx_len)
    max_ctx = cfg.ctx_len + cfg.n_new + 2 * cfg.block
    tgt = DeviceTarget(cfg, TW, cfg.target_layers, cfg.tap_layers, max_ctx=max_ctx, max_n=16)
    tgt.reset()
    a, _ = tgt.forward(prompt)
    greedy = [int(a[-1])]
    while len(greedy) < cfg.n_new:
        a, _ = tgt.forward([greedy[-1]])
        greedy.append(int(a[0]))
    dr = Drafter(cfg, W, batch=1, max_ctx=max_ctx, max_rows=cfg.ctx_len)
    out, ms = spec_generate(dr, tgt, prompt, cfg.n_new)
    gh.log(f"[target loop] steps {len(ms)}, mean accepted {np.mean(ms):.2f}")
    assert out == greedy
    same = assert_oracle_greedy(cfg, TW, prompt, greedy, what="device greedy")
    gh.log(f"    device greedy equals the fp64 oracle's greedy decoding for {same}/{len(greedy)} tokens")


def test_device_loop_matches_host_loop(gpu_lib):
    """The loop with no per-step host synchronisation (steps captured in a
    graph, and run eagerly), over a batch of two prompts of different lengths
    with a stop id, emits per sequence exactly what the host-driven loop does
    for that prompt alone."""
    cfg = synth.CONFIGS["c1"]
    W = synth.make_weights(cfg)
    TW = synth.make_target_weights(cfg, W)
    prompts = [list(synth.make_prompt(cfg, 64)), list(synth.make_prompt(cfg, 37, seed=11))]
    n_new, S = cfg.n_new, 4
    max_ctx = 64 + n_new + (S + 2) * cfg.block + 16
    ref_out = []
    for p in prompts:
        tgt1 = DeviceTarget(cfg, TW, cfg.target_layers, cfg.tap_layers, max_ctx=max_ctx, max_n=16)
        dr1 = Drafter(cfg, W, batch=1, max_ctx=max_ctx, max_rows=64)
        ref_out.append(spec_generate(dr1, tgt1, p, n_new)[0])
        del tgt1, dr1
    tgt = DeviceTarget(cfg, TW, cfg.target_layers, cfg.tap_layers, batch=2, max_ctx=max_ctx, max_n=16)
    dr = Drafter(cfg, W, batch=2, max_ctx=max_ctx, max_rows=2 * 16)
    for graph in (True, False):
        out = spec_generate_device(dr, tgt, prompts, n_new, steps_per_sync=S, graph=graph)
        assert out == ref_out, f"graph={graph}"
    for b, p in enumerate(prompts):
        assert_oracle_greedy(cfg, TW, p, out[b], what=f"device loop seq {b}")
    # a stop id (the 21st token of the first sequence) ends that sequence there
    stop = ref_out[0][20]
    want = []
    for r in ref_out:
        cut = r.index(stop) + 1 if stop in r else len(r)
        want.append(r[:cut])
    out = spec_generate_device(dr, tgt, prompts, n_new, stop_token_ids=[stop], steps_per_sync=S, graph=True)
    assert out == want
    for b, p in enumerate(prompts):
        assert_oracle_greedy(cfg, TW, p, out[b], stop_ids=[stop], what=f"device loop with a stop id, seq {b}")
    gh.log(f"[device loop] lengths {[len(o) for o in out]}")


def test_device_loop_random_gains_against_oracle(gpu_lib):
    """The on-device loop (graph-replayed) with random norm gains in the
    drafter and the target, three prompts of different lengths, against the
    fp64 oracle's plain greedy decoding of each prompt."""
    cfg = synth.CONFIGS["c1"]
    W = synth.make_weights(cfg, gains="random")
    TW = synth.make_target_weights(cfg, W, gains="random")
    prompts = [list(synth.make_prompt(cfg, n, seed=30 + n)) for n in (64, 20, 45)]
    n_new, S = 40, 3
    max_ctx = 64 + n_new + (S + 2) * cfg.block + 16
    tgt = DeviceTarget(cfg, TW, cfg.target_layers, cfg.tap_layers, batch=3, max_ctx=max_ctx, max_n=16)
    dr = Drafter(cfg, W, batch=3, max_ctx=max_ctx, max_rows=3 * 16)
    out = spec_generate_device(dr, tgt, prompts, n_new, steps_per_sync=S, graph=True)
    assert [len(o) for o in out] == [n_new] * 3
    for b, p in enumerate(prompts):
        assert_oracle_greedy(cfg, TW, p, out[b], what=f"random gains seq {b}")
