"""The allocation-free draft block (dflash_draft_block_noalloc, workspace in
the library's static device array) against dflash_draft_block with a caller
workspace: bit-identical drafts, logits, hidden states and block K/V, over
calls in a row whose inputs shrink, so that contents a larger call left in
the shared array are there for the smaller one to trip over."""
import numpy as np
import pytest

import gpu_helpers as gh
from block_diffusion_drafter_target_amd import Drafter, synth

pytestmark = pytest.mark.gpu


def _case(cfg, lens, gains):
    import torch
    W = synth.make_weights(cfg, gains=gains)
    batch = len(lens)
    max_ctx = max(lens) + 2 * cfg.block
    dr = Drafter(cfg, W, batch=batch, max_ctx=max_ctx, max_rows=max(max(lens), 1))
    for b, L in enumerate(lens):
        if L:
            t = synth.make_taps(cfg, L, tid=b)
            dr.ingest(b, torch.from_numpy(t.view(np.int16)).view(torch.bfloat16).to("cuda"))
    dr.anchor.copy_(torch.from_numpy(synth.make_anchors(cfg.with_(batch=batch))))
    return dr


def _run(dr, noalloc):
    import torch
    cfg, batch = dr.cfg, dr.batch
    B, NL = cfg.block, cfg.n_layers
    lg = torch.full((batch * (B - 1), cfg.vocab), float("nan"), dtype=torch.float32, device="cuda")
    hd = torch.full((NL + 1, batch * B, cfg.hidden), float("nan"), dtype=torch.float32, device="cuda")
    dr.draft.fill_(-7)
    L = dr.ctx_len.cpu().numpy()
    for b in range(batch):  # the pass must write every block slot again
        dr.k[:, b, :, L[b]:L[b] + B] = float("nan")
        dr.v[:, b, :, L[b]:L[b] + B] = float("nan")
    if noalloc:
        dr.draft_block_noalloc(dbg_logits=lg, dbg_hidden=hd)
    else:
        dr.draft_block(dbg_logits=lg, dbg_hidden=hd)
    torch.cuda.synchronize()
    kb = [dr.k[:, b, :, L[b]:L[b] + B].clone() for b in range(batch)]
    vb = [dr.v[:, b, :, L[b]:L[b] + B].clone() for b in range(batch)]
    return dr.draft.clone(), lg, hd, kb, vb, dr.status.clone()


def _same(a, b, what):
    import torch
    assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                       b.view(torch.int32) if b.dtype == torch.float32 else b), what


def test_noalloc_matches_draft_block(gpu_lib):
    """Three drafters, largest workspace first: the benchmarked layer shape
    (one layer, context 1024), 19 sequences of a small model (large-tile
    GEMMs) and 3 sequences at block 12; for each, the caller-workspace draft
    block, then the allocation-free one, then the allocation-free one again."""
    from block_diffusion_drafter_target_amd import binding as bd
    cases = [("c2-1layer", synth.CONFIGS["c2"].with_(n_layers=1), [1024], "ones"),
             ("big-b19", gh.SHAPES["big-b19"], gh.CTX["big-b19"], "random"),
             ("b12", gh.SHAPES["b12"], gh.CTX["b12"], "ones")]
    prev = None
    for name, cfg, lens, gains in cases:
        gh.log(f"[noalloc] {name}: batch {len(lens)}, contexts {lens[:4]}...")
        dr = _case(cfg, lens, gains)
        need = bd.dflash_workspace_bytes(dr.model, dr.batch, dr.max_ctx, 1)
        assert need <= bd.NOALLOC_SCRATCH_BYTES
        if prev is not None:
            assert need < prev, "each call's input is smaller than the one before"
        prev = need
        want = _run(dr, noalloc=False)
        for rep in range(2):
            got = _run(dr, noalloc=True)
            assert (got[5].cpu().numpy() == 0).all()
            _same(got[0], want[0], f"{name} drafts (call {rep})")
            _same(got[1], want[1], f"{name} logits (call {rep})")
            _same(got[2], want[2], f"{name} hidden states (call {rep})")
            for b in range(dr.batch):
                _same(got[3][b], want[3][b], f"{name} block K seq {b}")
                _same(got[4][b], want[4][b], f"{name} block V seq {b}")
        assert int(want[0].min()) >= 0
        del dr
