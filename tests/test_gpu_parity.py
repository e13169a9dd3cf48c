"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Every case prints its name before touching the GPU. Tolerances: bf16 hidden
states, caches and logits within max|d|/max|ref| <= 2e-2; tokens bit-exact up
to the tie band (see gpu_helpers.check_tokens); verify, acceptance, commit rows
and ctx_len bit-exact.
"""
import numpy as np
import pytest

import gpu_helpers as gh
from block_diffusion_drafter_target_amd import Drafter, spec_generate, synth
from oracle import ref

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def make_case(cfg, ctx_lens, extra_ctx=48, gains="ones"):
    torch = _torch()
    W = synth.make_weights(cfg, gains=gains)
    WO = gh.oracle_weights(W)
    ocfg = ref.OracleConfig.from_any(cfg)
    batch = len(ctx_lens)
    max_ctx = max(ctx_lens) + cfg.block + extra_ctx
    dr = Drafter(cfg, W, batch=batch, max_ctx=max_ctx, max_rows=max(max(ctx_lens), batch * cfg.block, 1))
    cache = ref.new_cache(ocfg, batch, max_ctx)
    taps = []
    for b, L in enumerate(ctx_lens):
        t = synth.make_taps(cfg, L, tid=b) if L else np.zeros((0, cfg.tap_width), np.uint16)
        taps.append(t)
        if L:
            dr.ingest(b, torch.from_numpy(t.view(np.int16)).view(torch.bfloat16).to("cuda"))
            ref.inject_kv(ocfg, WO, ref.fuse_ctx(ocfg, WO, synth.bf16_to_f64(t)),
                          [(r, b, r) for r in range(L)], cache)
    torch.cuda.synchronize()
    return W, WO, ocfg, dr, cache, taps


def gpu_cache(dr, l, b, L):
    """Layer l, sequence b, slots [0, L) of the device cache as [L, Hkv, D] fp64."""
    k = gh.to_np_bf16(dr.k[l, b, :, :L]).transpose(1, 0, 2)
    v = gh.to_np_bf16(dr.v[l, b, :, :L]).transpose(1, 0, 2)
    return k, v


def test_pack_matrix_layout(gpu_lib):
    """The packed fragment layout, element by element (bit exact)."""
    torch = _torch()
    from block_diffusion_drafter_target_amd.drafter import pack_matrix
    gh.log("[pack] 48 x 96 and 160 x 4096")
    for rows, cols in ((48, 96), (160, 4096)):
        w = np.random.default_rng(rows).integers(0, 1 << 16, size=(rows, cols), dtype=np.uint16)
        t = torch.from_numpy(w.view(np.int16)).cuda()
        got = pack_matrix(t.view(torch.bfloat16)).view(torch.int16).cpu().numpy().view(np.uint16)
        # [rg][kc][g][r][e] = W[16 rg + r][32 kc + 8 g + e]
        want = w.reshape(rows // 16, 16, cols // 32, 4, 8).transpose(0, 2, 3, 1, 4).reshape(rows, cols)
        assert np.array_equal(got.reshape(rows, cols), want)


def test_ingest_rows_and_offset_ingest(gpu_lib):
    """The commit rows of a context ingest (bit exact, also for n = 0), and an
    ingest of one sequence in two parts, the second at an offset: the cache
    slots of both parts against the oracle's injection at those positions,
    the other sequences untouched."""
    torch = _torch()
    from block_diffusion_drafter_target_amd import binding as bd
    cfg = gh.SHAPES["b12"]
    gh.log("[ingest rows] b12, sequence 1: 7 rows at 0, then 20 at 7")
    W = synth.make_weights(cfg, gains="random")
    WO = gh.oracle_weights(W)
    ocfg = ref.OracleConfig.from_any(cfg)
    dr = Drafter(cfg, W, batch=3, max_ctx=64, max_rows=32)
    rows = torch.full((9, 3), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    bd.dflash_ingest_rows(dr.model, dr.kv, 2, 5, 9, bd.ptr(rows), bd.ptr(cnt), dr.stream())
    torch.cuda.synchronize()
    want = np.stack([np.arange(9), np.full(9, 2), 5 + np.arange(9)], axis=1)
    assert np.array_equal(rows.cpu().numpy(), want) and int(cnt.item()) == 9
    bd.dflash_ingest_rows(dr.model, dr.kv, 0, 64, 0, bd.ptr(rows), bd.ptr(cnt), dr.stream())
    torch.cuda.synchronize()
    assert int(cnt.item()) == 0 and np.array_equal(rows.cpu().numpy(), want)
    t0, t1 = synth.make_taps(cfg, 7, tid=0), synth.make_taps(cfg, 20, tid=1)
    dev = lambda t: torch.from_numpy(t.view(np.int16)).view(torch.bfloat16).to("cuda")
    dr.ingest(1, dev(t0), start=0)
    dr.ingest(1, dev(t1), start=7)
    torch.cuda.synchronize()
    cache = ref.new_cache(ocfg, 3, 64)
    ref.inject_kv(ocfg, WO, ref.fuse_ctx(ocfg, WO, synth.bf16_to_f64(t0)), [(r, 1, r) for r in range(7)], cache)
    ref.inject_kv(ocfg, WO, ref.fuse_ctx(ocfg, WO, synth.bf16_to_f64(t1)), [(r, 1, 7 + r) for r in range(20)], cache)
    assert dr.ctx_len.cpu().tolist() == [0, 27, 0]
    for l in range(cfg.n_layers):
        k, v = gpu_cache(dr, l, 1, 27)
        gh.check_rel(k, cache["k"][l, 1, :27], what=f"K layer {l}", axis=1)
        gh.check_rel(v, cache["v"][l, 1, :27], what=f"V layer {l}", axis=1)
        for b in (0, 2):
            assert not dr.k[l, b].abs().sum().item() and not dr.v[l, b].abs().sum().item()


# every shape with unit gains, and the shapes below again with random gains
# (each gain vector its own draw, so a swapped, unused or misindexed gain
# changes the compared values)
GAIN_SHAPES = ["gqa-d128", "g8-d64", "tiled-b9", "big-b19", "big-b8x40", "mlp-wide-b2", "b12", "ws-tail", "mlp-wide-b1", "wide-h5120"]
CASES = [(s, "ones") for s in sorted(gh.SHAPES)] + [(s, "random") for s in GAIN_SHAPES]
CASE_IDS = [f"{s}-{g}" for s, g in CASES]


@pytest.mark.parametrize("shape,gains", CASES, ids=CASE_IDS)
def test_fuse_ctx_parity(gpu_lib, shape, gains):
    torch = _torch()
    cfg = gh.SHAPES[shape]
    gh.log(f"[fuse] {shape} gains {gains}")
    W = synth.make_weights(cfg, only={"w_fc", "g_fc"}, gains=gains)
    full = synth.make_weights(cfg, gains=gains)
    WO = gh.oracle_weights(W)
    ocfg = ref.OracleConfig.from_any(cfg)
    n = 300  # tiled GEMM: three row tiles, the last ragged
    taps = synth.make_taps(cfg, n, tid=7)
    dr = Drafter(cfg, full, batch=1, max_ctx=64, max_rows=n)
    ctx = dr.fuse_ctx(torch.from_numpy(taps.view(np.int16)).view(torch.bfloat16).cuda(), n,
                      torch.empty((n, cfg.hidden), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    got = gh.to_np_bf16(ctx)
    want = ref.fuse_ctx(ocfg, WO, synth.bf16_to_f64(taps))
    e = gh.check_rel(got, want, what="fuse", rows=True)
    gh.log(f"    rel err {e:.2e}")


@pytest.mark.parametrize("shape,gains", CASES, ids=CASE_IDS)
def test_inject_kv_parity(gpu_lib, shape, gains):
    torch = _torch()
    cfg = gh.SHAPES[shape]
    gh.log(f"[inject] {shape} gains {gains}")
    lens = gh.CTX[shape]
    W, WO, ocfg, dr, cache, taps = make_case(cfg, lens, gains=gains)
    assert dr.ctx_len.cpu().tolist() == lens
    assert dr.status.cpu().tolist() == [0] * len(lens)
    for b, L in enumerate(lens):
        if not L:
            continue
        # stage replay: the oracle injects the device's own bf16 context feature
        ctx = dr.fuse_ctx(torch.from_numpy(taps[b].view(np.int16)).view(torch.bfloat16).cuda(), L,
                          torch.empty((L, cfg.hidden), dtype=torch.bfloat16, device="cuda"))
        ctx64 = gh.to_np_bf16(ctx)
        rc = ref.new_cache(ocfg, 1, L)
        ref.inject_kv(ocfg, WO, ctx64, [(r, 0, r) for r in range(L)], rc)
        for l in range(cfg.n_layers):
            k, v = gpu_cache(dr, l, b, L)
            gh.check_rel(k, rc["k"][l, 0, :L], what=f"K replay l{l} b{b}", axis=1)
            gh.check_rel(v, rc["v"][l, 0, :L], what=f"V replay l{l} b{b}", axis=1)
            # end to end from the taps
            gh.check_rel(k, cache["k"][l, b, :L], what=f"K l{l} b{b}", axis=1)
            gh.check_rel(v, cache["v"][l, b, :L], what=f"V l{l} b{b}", axis=1)
    # slots past the committed context were never written
    for b, L in enumerate(lens):
        assert float(dr.k[:, b, :, L:].abs().max()) == 0.0


@pytest.mark.parametrize("shape,gains", CASES, ids=CASE_IDS)
def test_draft_block_parity(gpu_lib, shape, gains):
    torch = _torch()
    cfg = gh.SHAPES[shape]
    gh.log(f"[draft_block] {shape} gains {gains}")
    lens = gh.CTX[shape]
    W, WO, ocfg, dr, cache, taps = make_case(cfg, lens, gains=gains)
    batch, B, H, NL, V = len(lens), cfg.block, cfg.hidden, cfg.n_layers, cfg.vocab
    anchor = synth.make_anchors(cfg.with_(batch=batch))
    dr.anchor.copy_(torch.from_numpy(anchor))
    dbg_logits = torch.empty((batch * (B - 1), V), dtype=torch.float32, device="cuda")
    dbg_hidden = torch.empty((NL + 1, batch * B, H), dtype=torch.float32, device="cuda")
    dr.draft_block(dbg_logits=dbg_logits, dbg_hidden=dbg_hidden)
    torch.cuda.synchronize()
    draft = dr.draft.cpu().numpy()
    logits = dbg_logits.cpu().numpy().astype(np.float64).reshape(batch, B - 1, V)
    hidden = dbg_hidden.cpu().numpy().astype(np.float64).reshape(NL + 1, batch, B, H)
    assert dr.status.cpu().tolist() == [0] * batch
    assert dr.ctx_len.cpu().tolist() == lens  # drafting never commits

    # end to end against the oracle from the same inputs
    r = ref.draft_block(ocfg, WO, cache, lens, anchor)
    for l in range(NL + 1):
        gh.check_rel(hidden[l], r["hidden"][:, l], what=f"hidden after layer {l}", rows=True)
    gh.check_rel(logits, r["logits"], what="logits", rows=True)
    band = gh.check_tokens(draft, logits, r["logits"], gh.e2e_band(r["logits"]), what="draft tokens")
    gh.log(f"    tie-band rows (end to end): {band}/{draft.size}")

    # stage replay: every layer from the device's own input and cached context
    for b, L in enumerate(lens):
        pos = L + np.arange(B)
        for l in range(NL):
            kc, vc = gpu_cache(dr, l, b, L)
            want, kb, vb = ref.decoder_layer(ocfg, WO, l, hidden[l, b], pos, kc, vc)
            gh.check_rel(hidden[l + 1, b], want, tol=1e-2, what=f"replay layer {l} seq {b}", rows=True)
            # the block's own K/V were appended at slots L..L+B-1
            kbl, vbl = gpu_cache(dr, l, b, L + B)
            gh.check_rel(kbl[L:], kb, what=f"block K l{l} b{b}", axis=1)
            gh.check_rel(vbl[L:], vb, what=f"block V l{l} b{b}", axis=1)
        fin = ref.rms_norm(hidden[NL, b], WO["g_final"], cfg.rms_eps)
        z = fin[1:] @ WO["lm_head"].T
        gh.check_rel(logits[b], z, tol=1e-2, what=f"replay lm head seq {b}", rows=True)
        gh.check_tokens(draft[b], logits[b], z, gh.replay_band(fin[1:], WO["lm_head"]), what=f"replay tokens seq {b}")


def test_draft_block_capacity_status(gpu_lib):
    torch = _torch()
    cfg = gh.SHAPES["b12"]
    gh.log("[draft_block] capacity")
    lens = [40, 0, 20]
    W, WO, ocfg, dr, cache, taps = make_case(cfg, lens, extra_ctx=0)
    assert dr.max_ctx == 40 + cfg.block  # sequence 0 fills the cache exactly
    dr.ctx_len[2] = dr.max_ctx - cfg.block + 1  # sequence 2 would overflow by one slot
    dr.anchor.copy_(torch.tensor([1, 2, 3], dtype=torch.int32))
    lg = torch.empty((3 * (cfg.block - 1), cfg.vocab), dtype=torch.float32, device="cuda")
    dr.draft_block(dbg_logits=lg)
    torch.cuda.synchronize()
    assert dr.status.cpu().tolist() == [0, 0, -5]
    d = dr.draft.cpu().numpy()
    assert (d[2] == -1).all()
    r = ref.draft_block(ocfg, WO, cache, lens[:2], [1, 2])
    logits = lg.cpu().numpy().astype(np.float64).reshape(3, cfg.block - 1, cfg.vocab)
    gh.check_rel(logits[:2], r["logits"], what="logits beside a failed sequence", rows=True)
    gh.check_tokens(d[:2], logits[:2], r["logits"], gh.e2e_band(r["logits"]), what="tokens beside a failed sequence")


@pytest.mark.parametrize("B", [2, 3, 5])
def test_small_blocks_draft_and_verify(gpu_lib, B):
    """Blocks of 2 (one drafted token), 3 and 5: G*B = 8, 12 and 20 query rows
    per kv head (padded query tiles), LM heads of 1, 2 and 4 rows per sequence;
    the draft block end to end against the oracle, then verify bit exact."""
    torch = _torch()
    cfg = synth.DraftConfig(name=f"small-b{B}", hidden=256, n_layers=2, n_q_heads=8, n_kv_heads=2, head_dim=64,
                            intermediate=512, vocab=640, n_tap=2, block=B, batch=3, ctx_len=0)
    gh.log(f"[draft_block] block {B}")
    lens = [0, 70, 5]
    W, WO, ocfg, dr, cache, taps = make_case(cfg, lens)
    anchor = synth.make_anchors(cfg)
    dr.anchor.copy_(torch.from_numpy(anchor))
    V = cfg.vocab
    lg = torch.empty((cfg.batch * (B - 1), V), dtype=torch.float32, device="cuda")
    dr.draft_block(dbg_logits=lg)
    torch.cuda.synchronize()
    assert dr.status.cpu().tolist() == [0] * cfg.batch
    d = dr.draft.cpu().numpy()
    logits = lg.cpu().numpy().astype(np.float64).reshape(cfg.batch, B - 1, V)
    r = ref.draft_block(ocfg, WO, cache, lens, anchor)
    gh.check_rel(logits, r["logits"], what=f"logits, block {B}", rows=True)
    gh.check_tokens(d, logits, r["logits"], gh.e2e_band(r["logits"]), what=f"tokens, block {B}")
    for step in range(4):
        m = synth.geometric_accept(cfg.batch, B, 0.8, step=step)
        tgt = synth.synth_target_tokens(d, m, V, step=step)
        dr.verify_accept(torch.from_numpy(tgt).cuda())
        torch.cuda.synchronize()
        rv = ref.verify_accept(d, tgt, lens)
        assert dr.accept_len.cpu().numpy().tolist() == rv["accept_len"].tolist() == m.tolist()
        assert np.array_equal(dr.emitted.cpu().numpy(), rv["emitted"])
        assert np.array_equal(dr.n_emit.cpu().numpy(), rv["n_emit"])
        assert np.array_equal(dr.anchor_out.cpu().numpy(), rv["anchor_out"])
        n = int(dr.n_commit.item())
        assert np.array_equal(dr.commit_rows.cpu().numpy()[:n], rv["commit_rows"])


def test_draft_block_batch_over_64(gpu_lib):
    """70 sequences: the attention chunk split walks two groups of 64 sequences
    (chunk counts and first slots carried from the first group to the second),
    ragged and empty contexts, and a last sequence past its cache capacity
    (no chunks, draft -1, the others unaffected); 560 block rows take the
    large-tile GEMMs."""
    torch = _torch()
    cfg = synth.DraftConfig(name="batch70", hidden=256, n_layers=1, n_q_heads=4, n_kv_heads=2, head_dim=64,
                            intermediate=512, vocab=512, n_tap=2, block=8, batch=70, ctx_len=0)
    gh.log("[draft_block] batch of 70")
    g = np.random.Generator(np.random.PCG64(70))
    lens = [int(x) for x in g.integers(0, 301, size=cfg.batch)]
    lens[3] = lens[64] = 0
    lens[65] = 300
    W, WO, ocfg, dr, cache, taps = make_case(cfg, lens)
    bad = cfg.batch - 1
    dr.ctx_len[bad] = dr.max_ctx - cfg.block + 1  # one slot past the cache
    anchor = synth.make_anchors(cfg)
    dr.anchor.copy_(torch.from_numpy(anchor))
    B, V = cfg.block, cfg.vocab
    lg = torch.empty((cfg.batch * (B - 1), V), dtype=torch.float32, device="cuda")
    dr.draft_block(dbg_logits=lg)
    torch.cuda.synchronize()
    assert dr.status.cpu().tolist() == [0] * bad + [-5]
    d = dr.draft.cpu().numpy()
    assert (d[bad] == -1).all()
    r = ref.draft_block(ocfg, WO, cache, lens[:bad], anchor[:bad])
    logits = lg.cpu().numpy().astype(np.float64).reshape(cfg.batch, B - 1, V)
    gh.check_rel(logits[:bad], r["logits"], what="logits of 69 sequences", rows=True)
    band = gh.check_tokens(d[:bad], logits[:bad], r["logits"], gh.e2e_band(r["logits"]), what="tokens of 69 sequences")
    gh.log(f"    tie-band rows {band}/{d[:bad].size}")


def test_dead_slots_do_not_leak(gpu_lib):
    """Rollback by construction: NaN in every slot >= ctx_len changes nothing."""
    torch = _torch()
    cfg = gh.SHAPES["gqa-d128"]
    gh.log("[draft_block] NaN-poisoned dead slots")
    lens = gh.CTX["gqa-d128"]
    W, WO, ocfg, dr, cache, taps = make_case(cfg, lens)
    dr.anchor.copy_(torch.from_numpy(synth.make_anchors(cfg)))
    lg0 = torch.empty((len(lens) * (cfg.block - 1), cfg.vocab), dtype=torch.float32, device="cuda")
    dr.draft_block(dbg_logits=lg0)
    d0 = dr.draft.clone()
    for b, L in enumerate(lens):
        dr.k[:, b, :, L:] = float("nan")
        dr.v[:, b, :, L:] = float("nan")
    lg1 = torch.empty_like(lg0)
    dr.draft_block(dbg_logits=lg1)
    torch.cuda.synchronize()
    assert torch.isfinite(lg1).all()
    assert torch.equal(lg0, lg1)
    assert torch.equal(d0, dr.draft)


def test_verify_accept_parity(gpu_lib):
    torch = _torch()
    gh.log("[verify] random batch")
    cfg = gh.SHAPES["gqa-d128"].with_(batch=37)
    W = synth.make_weights(cfg)
    B = cfg.block
    g = np.random.default_rng(5)
    for trial in range(6):
        batch = [1, 2, 37, 300, 7, 64][trial]
        dr = Drafter(cfg, W, batch=batch, max_ctx=256, max_rows=batch * B)
        alphabet = [2, 3, 50, 1000, 2, 4][trial]
        draft = g.integers(0, alphabet, size=(batch, B - 1)).astype(np.int32)
        m = synth.geometric_accept(batch, B, 0.7, step=trial)
        target = synth.synth_target_tokens(draft, m, cfg.vocab, step=trial) % alphabet
        target = target.astype(np.int32)
        ctx = g.integers(0, 200, size=batch).astype(np.int32)
        stops = [1] if trial % 2 else []
        budget = g.integers(0, 20, size=batch).astype(np.int32) if trial >= 2 else None
        dr.ctx_len.copy_(torch.from_numpy(ctx))
        tdev = torch.from_numpy(target).cuda()
        ddev = torch.from_numpy(draft).cuda()
        sdev = torch.tensor(stops, dtype=torch.int32, device="cuda") if stops else None
        bdev = torch.from_numpy(budget).cuda() if budget is not None else None
        dr.verify_accept(tdev, sdev, bdev, draft=ddev)
        torch.cuda.synchronize()
        r = ref.verify_accept(draft, target, ctx, stops, budget)
        assert dr.accept_len.cpu().numpy().tolist() == r["accept_len"].tolist()
        assert dr.anchor_out.cpu().numpy().tolist() == r["anchor_out"].tolist()
        assert dr.n_emit.cpu().numpy().tolist() == r["n_emit"].tolist()
        assert dr.done.cpu().numpy().tolist() == r["done"].tolist()
        assert np.array_equal(dr.emitted.cpu().numpy(), r["emitted"])
        n = int(dr.n_commit.item())
        assert n == len(r["commit_rows"])
        assert np.array_equal(dr.commit_rows.cpu().numpy()[:n], r["commit_rows"])
        if budget is not None:
            assert bdev.cpu().numpy().tolist() == r["budget"].tolist()
        assert dr.ctx_len.cpu().numpy().tolist() == ctx.tolist()  # verify never commits


class OracleTarget:
    """The oracle's tiny causal target behind the loop's target interface."""

    def __init__(self, t):
        self.t = t

    def reset(self):
        self.t.reset()

    def forward(self, tokens):
        z, taps = self.t.forward(tokens)
        return ref.argmax_rows(z), taps

    def truncate(self, n):
        self.t.truncate(n)


def test_tiny_loop_lossless_with_device_drafter(gpu_lib):
    torch = _torch()
    gh.log("[loop] tiny target, device drafter")
    cfg = synth.CONFIGS["c1"]
    W = synth.make_weights(cfg)
    TW = synth.make_target_weights(cfg, W)
    ocfg = ref.OracleConfig.from_any(cfg)
    prompt = synth.make_prompt(cfg, cfg.ctx_len)
    tgt = ref.TinyTarget(ocfg, TW, cfg.target_layers, cfg.tap_layers)
    greedy = ref.greedy_generate(tgt, prompt, cfg.n_new)
    dr = Drafter(cfg, W, batch=1, max_ctx=cfg.ctx_len + cfg.n_new + 2 * cfg.block, max_rows=cfg.ctx_len)
    out, ms = spec_generate(dr, OracleTarget(tgt), prompt, cfg.n_new)
    assert out == greedy
    gh.log(f"    steps {len(ms)}, mean accepted {np.mean(ms):.2f}")
    # the device cache holds the committed context: compare with the oracle's
    # own fuse + inject of a full prefill of the committed tokens
    L = int(dr.ctx_len.item())
    assert L == len(prompt) + sum(m + 1 for m in ms)
    WO = gh.oracle_weights(W)
    tgt.reset()
    seq = list(prompt) + list(greedy[:L - len(prompt)]) if L - len(prompt) <= len(greedy) else None
    if seq is not None:
        _, taps = tgt.forward(seq)
        fresh = ref.new_cache(ocfg, 1, L)
        ref.inject_kv(ocfg, WO, ref.fuse_ctx(ocfg, WO, taps), [(r, 0, r) for r in range(L)], fresh)
        for l in range(cfg.n_layers):
            k, v = gpu_cache(dr, l, 0, L)
            gh.check_rel(k, fresh["k"][l, 0], what=f"loop cache K l{l}", axis=1)
            gh.check_rel(v, fresh["v"][l, 0], what=f"loop cache V l{l}", axis=1)
    # stop token ends the loop right after it
    stop = greedy[20]
    out2, _ = spec_generate(dr, OracleTarget(tgt), prompt, cfg.n_new, stop_token_ids=[stop])
    assert out2 == greedy[:greedy.index(stop) + 1]


def test_run_twice_is_bit_identical(gpu_lib):
    torch = _torch()
    cfg = gh.SHAPES["g8-d64"]
    gh.log("[determinism] g8-d64")
    W, WO, ocfg, dr, cache, taps = make_case(cfg, gh.CTX["g8-d64"])
    dr.anchor.copy_(torch.tensor([5, 6], dtype=torch.int32))
    outs = []
    for _ in range(2):
        lg = torch.empty((2 * (cfg.block - 1), cfg.vocab), dtype=torch.float32, device="cuda")
        dr.draft_block(dbg_logits=lg)
        torch.cuda.synchronize()
        outs.append((dr.draft.cpu().numpy().copy(), lg.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("shape", ["long-d64", "long-d128"])
def test_attention_reference_moves_mid_chunk(gpu_lib, shape):
    """Keys whose scores jump far above the running softmax reference in the
    middle of an attention chunk: a few cached keys of every layer are scaled by
    16 (exact in bf16), so their base-2 scores exceed the reference taken from
    the chunk's earlier slices by much more than 8. The lazy reference then
    moves mid-chunk, and in the two-buffer D = 64 loop the next slice's scores,
    already computed against the old reference, are shifted too. Every layer
    is replayed in fp64 from the device's own input and (modified) cache."""
    torch = _torch()
    cfg = gh.SHAPES[shape]
    lens = gh.CTX[shape]
    gh.log(f"[attention reference moves] {shape}")
    W, WO, ocfg, dr, cache, taps = make_case(cfg, lens)
    batch, B, H, NL = len(lens), cfg.block, cfg.hidden, cfg.n_layers
    for b, L in enumerate(lens):
        slots = sorted({min(L - 1, L * k // 7 + 37) for k in range(1, 7)}) if L > 1 else []
        for s in slots:
            dr.k[:, b, :, s] *= 16
    anchor = synth.make_anchors(cfg.with_(batch=batch))
    dr.anchor.copy_(torch.from_numpy(anchor))
    dbg_hidden = torch.empty((NL + 1, batch * B, H), dtype=torch.float32, device="cuda")
    dr.draft_block(dbg_hidden=dbg_hidden)
    torch.cuda.synchronize()
    assert dr.status.cpu().tolist() == [0] * batch
    hidden = dbg_hidden.cpu().numpy().astype(np.float64).reshape(NL + 1, batch, B, H)
    for b, L in enumerate(lens):
        pos = L + np.arange(B)
        for l in range(NL):
            kc, vc = gpu_cache(dr, l, b, L)
            want, _, _ = ref.decoder_layer(ocfg, WO, l, hidden[l, b], pos, kc, vc)
            e = gh.check_rel(hidden[l + 1, b], want, tol=1e-2, what=f"replay layer {l} seq {b}", rows=True)
            gh.log(f"    layer {l} seq {b} (context {L}): rel err {e:.2e}")
