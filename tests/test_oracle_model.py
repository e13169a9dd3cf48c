"""Pins of the oracle's layer, target, fuse and inject against a library model.

The oracle's decoder layer is checked against ``transformers``' Qwen3 decoder
layer run in float64 on the CPU: a library implementation of the same layer
shape (RMSNorm, q/k norm, rotate-half RoPE, GQA, SwiGLU). Its RMSNorm and
softmax internally run in float32, hence the 1e-5 tolerances. Weights and gains
are random here (gains != 1) so that a dropped gain or a swapped projection
fails.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import ref

transformers = pytest.importorskip("transformers")
from transformers import Qwen3Config, Qwen3ForCausalLM  # noqa: E402
from transformers.cache_utils import DynamicCache  # noqa: E402
from transformers.models.qwen3.modeling_qwen3 import apply_rotary_pos_emb  # noqa: E402

TOL = 2e-5


def small_cfg(**kw):
    base = dict(hidden=64, n_layers=3, n_q_heads=8, n_kv_heads=2, head_dim=16,
                intermediate=96, vocab=97, n_tap=3, block=6, rope_theta=1e4, rms_eps=1e-6)
    base.update(kw)
    return ref.OracleConfig(**base)


def rand_weights(cfg, n_layers, seed=0, gains_random=True):
    g = np.random.default_rng(seed)
    H, D, I, V = cfg.hidden, cfg.head_dim, cfg.intermediate, cfg.vocab
    qkv = (cfg.n_q_heads + 2 * cfg.n_kv_heads) * D

    def m(r, c, s=0.1):
        return g.standard_normal((r, c)) * s

    def gain(n):
        return 1.0 + 0.3 * g.standard_normal(n) if gains_random else np.ones(n)
    W = {"embed": m(V, H, 1.0), "lm_head": m(V, H), "w_fc": m(H, cfg.n_tap * H),
         "g_fc": gain(H), "g_final": gain(H)}
    for l in range(n_layers):
        W[f"layers.{l}.w_qkv"] = m(qkv, H)
        W[f"layers.{l}.w_o"] = m(H, cfg.n_q_heads * D)
        W[f"layers.{l}.w_gate"] = m(I, H)
        W[f"layers.{l}.w_up"] = m(I, H)
        W[f"layers.{l}.w_down"] = m(H, I)
        for n, k in (("g_in", H), ("g_post", H), ("g_q", D), ("g_k", D)):
            W[f"layers.{l}.{n}"] = gain(k)
    return W


def hf_model(cfg, W, n_layers):
    c = Qwen3Config(vocab_size=cfg.vocab, hidden_size=cfg.hidden, intermediate_size=cfg.intermediate,
                    num_hidden_layers=n_layers, num_attention_heads=cfg.n_q_heads,
                    num_key_value_heads=cfg.n_kv_heads, head_dim=cfg.head_dim,
                    rms_norm_eps=cfg.rms_eps, rope_theta=cfg.rope_theta,
                    tie_word_embeddings=False, max_position_embeddings=4096,
                    attention_bias=False)
    c._attn_implementation = "sdpa"
    model = Qwen3ForCausalLM(c).to(torch.float64).eval()
    Hq, Hkv, D = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))  # noqa: E731
    with torch.no_grad():
        model.model.embed_tokens.weight.copy_(t(W["embed"]))
        model.lm_head.weight.copy_(t(W["lm_head"]))
        model.model.norm.weight.copy_(t(W["g_final"]))
        for l in range(n_layers):
            L = model.model.layers[l]
            qkv = W[f"layers.{l}.w_qkv"]
            L.self_attn.q_proj.weight.copy_(t(qkv[:Hq * D]))
            L.self_attn.k_proj.weight.copy_(t(qkv[Hq * D:(Hq + Hkv) * D]))
            L.self_attn.v_proj.weight.copy_(t(qkv[(Hq + Hkv) * D:]))
            L.self_attn.o_proj.weight.copy_(t(W[f"layers.{l}.w_o"]))
            L.self_attn.q_norm.weight.copy_(t(W[f"layers.{l}.g_q"]))
            L.self_attn.k_norm.weight.copy_(t(W[f"layers.{l}.g_k"]))
            L.mlp.gate_proj.weight.copy_(t(W[f"layers.{l}.w_gate"]))
            L.mlp.up_proj.weight.copy_(t(W[f"layers.{l}.w_up"]))
            L.mlp.down_proj.weight.copy_(t(W[f"layers.{l}.w_down"]))
            L.input_layernorm.weight.copy_(t(W[f"layers.{l}.g_in"]))
            L.post_attention_layernorm.weight.copy_(t(W[f"layers.{l}.g_post"]))
    return model


def test_target_prefill_matches_library_model():
    cfg = small_cfg()
    W = rand_weights(cfg, 4)
    model = hf_model(cfg, W, 4)
    toks = np.random.default_rng(3).integers(0, cfg.vocab, size=23)
    tgt = ref.TinyTarget(cfg, W, 4, (1, 2))
    z, taps = tgt.forward(toks)
    with torch.no_grad():
        out = model(torch.from_numpy(toks)[None], output_hidden_states=True)
    zr = out.logits[0].numpy()
    assert ref.rel_err(z, zr) < TOL
    hs = out.hidden_states  # embeddings, then the output of each layer
    assert ref.rel_err(taps[:, :cfg.hidden], hs[2][0].numpy()) < TOL
    assert ref.rel_err(taps[:, cfg.hidden:], hs[3][0].numpy()) < TOL
    # incremental forward after a truncation equals the prefill
    tgt.reset()
    tgt.forward(toks[:10])
    tgt.forward(toks[10:15])
    tgt.truncate(12)
    z2, _ = tgt.forward(toks[12:])
    assert ref.rel_err(z2, z[12:]) < 1e-10


def test_greedy_matches_library_generate():
    cfg = small_cfg(vocab=61)
    W = rand_weights(cfg, 4, seed=5)
    model = hf_model(cfg, W, 4)
    prompt = np.random.default_rng(4).integers(0, cfg.vocab, size=9)
    tgt = ref.TinyTarget(cfg, W, 4, (1,))
    mine = ref.greedy_generate(tgt, prompt, 20)
    with torch.no_grad():
        gen = model.generate(torch.from_numpy(prompt)[None], max_new_tokens=20, do_sample=False,
                             eos_token_id=None, pad_token_id=0, min_new_tokens=20)
    assert mine == gen[0, len(prompt):].tolist()


def _hf_ctx_kv(layer, cfg, rot, ctx, pos):
    """Context K/V produced with the library layer's own modules."""
    att = layer.self_attn
    D, Hkv = cfg.head_dim, cfg.n_kv_heads
    c = torch.from_numpy(ctx)[None]
    k = att.k_norm(att.k_proj(c).view(1, -1, Hkv, D)).transpose(1, 2)
    v = att.v_proj(c).view(1, -1, Hkv, D).transpose(1, 2)
    cos, sin = rot(c, torch.from_numpy(pos)[None])
    _, k = apply_rotary_pos_emb(k, k, cos, sin)
    return k, v


@pytest.mark.parametrize("L", [0, 1, 29])
def test_draft_layer_with_injected_context_matches_library(L):
    cfg = small_cfg()
    W = rand_weights(cfg, 1, seed=7)
    model = hf_model(cfg, W, 1)
    layer = model.model.layers[0]
    rot = model.model.rotary_emb
    g = np.random.default_rng(11)
    ctx = g.standard_normal((L, cfg.hidden))
    x = g.standard_normal((cfg.block, cfg.hidden))
    cpos = np.arange(L)
    bpos = L + np.arange(cfg.block)
    # oracle: inject then run the layer with no mask
    k_ctx, v_ctx = ref.project_kv(cfg, W, 0, ctx, cpos)
    got, _, _ = ref.decoder_layer(cfg, W, 0, x, bpos, k_ctx, v_ctx)
    with torch.no_grad():
        cache = DynamicCache()
        if L:
            kh, vh = _hf_ctx_kv(layer, cfg, rot, ctx, cpos)
            assert ref.rel_err(kh[0].transpose(0, 1).numpy(), k_ctx) < TOL
            assert ref.rel_err(vh[0].transpose(0, 1).numpy(), v_ctx) < 1e-12
            cache.update(kh, vh, 0)
        xt = torch.from_numpy(x)[None]
        pe = rot(xt, torch.from_numpy(bpos)[None])
        mask = torch.zeros(1, 1, cfg.block, L + cfg.block, dtype=torch.float64)
        want = layer(xt, attention_mask=mask, position_ids=torch.from_numpy(bpos)[None],
                     past_key_values=cache, use_cache=True, position_embeddings=pe)
        want = want[0] if isinstance(want, tuple) else want
    assert ref.rel_err(got, want[0].numpy()) < TOL


def test_fuse_matches_torch():
    cfg = small_cfg()
    W = rand_weights(cfg, 1)
    taps = np.random.default_rng(2).standard_normal((7, cfg.n_tap * cfg.hidden))
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))  # noqa: E731
    want = F.rms_norm(F.linear(t(taps), t(W["w_fc"])), (cfg.hidden,), t(W["g_fc"]), cfg.rms_eps)
    assert np.max(np.abs(ref.fuse_ctx(cfg, W, taps) - want.numpy())) < 1e-12


def test_inject_writes_every_layer_at_commit_positions():
    cfg = small_cfg()
    W = rand_weights(cfg, 3)
    ctx = np.random.default_rng(8).standard_normal((5, cfg.hidden))
    cache = ref.new_cache(cfg, 2, 20, fill=np.nan)
    rows = [(0, 1, 3), (4, 0, 0), (2, 1, 19)]
    ref.inject_kv(cfg, W, ctx, rows, cache)
    for l in range(cfg.n_layers):
        for src, b, p in rows:
            k, v = ref.project_kv(cfg, W, l, ctx[src:src + 1], np.array([p]))
            assert np.allclose(cache["k"][l, b, p], k[0], rtol=0, atol=1e-12)
            assert np.allclose(cache["v"][l, b, p], v[0], rtol=0, atol=1e-12)
    written = sum(1 for _ in rows) * cfg.n_layers * cfg.n_kv_heads * cfg.head_dim
    assert np.sum(~np.isnan(cache["k"])) == written


# ---------------------------------------------------------------- whole draft block

def _hf_block(model, cfg, ctx, L, ids, pos, causal=False):
    """The library model run over one block: context K/V made by each library
    layer's own k/v projections, k-norm and rotary embedding from the context
    feature rows ``ctx`` (at positions 0..L-1), then a forward over ``ids`` at
    ``pos``. Returns (logits [n, V], hidden states (embeddings, then each
    layer's output), the final norm's input, the final norm's output)."""
    n = len(ids)
    rot = model.model.rotary_emb
    seen = {}
    hook = model.model.norm.register_forward_hook(
        lambda m, a, o: seen.update(pre=a[0].clone(), post=o.clone()))
    try:
        with torch.no_grad():
            cache = DynamicCache()
            if L:
                for l, layer in enumerate(model.model.layers):
                    kh, vh = _hf_ctx_kv(layer, cfg, rot, ctx, np.arange(L))
                    cache.update(kh.contiguous(), vh.contiguous(), l)
            allowed = np.ones((n, L + n), bool)
            if causal:
                allowed = np.arange(L + n)[None, :] <= np.asarray(pos)[:, None]
            mask = torch.from_numpy(np.where(allowed, 0.0, -np.inf))[None, None]
            out = model(input_ids=torch.tensor([list(ids)]), position_ids=torch.tensor([list(pos)]),
                        past_key_values=cache if L else None, attention_mask=mask, use_cache=True,
                        output_hidden_states=True)
    finally:
        hook.remove()
    hs = [h[0].numpy() for h in out.hidden_states]
    return out.logits[0].numpy(), hs, seen["pre"][0].numpy(), seen["post"][0].numpy()


@pytest.mark.parametrize("L", [0, 1, 29])
def test_draft_block_matches_library_model(L):
    """ref.draft_block's assembly against the library model run over the block.

    The reading pinned here: row 0 holds the anchor and rows 1..B-1 the mask id,
    the rows sit at positions L..L+B-1 after a context injected at 0..L-1 with
    each layer's own k/v projections, attention inside the block is unmasked,
    the drafter's own final norm precedes the shared LM head, and rows 1..B-1
    (no shift) give the B-1 drafted tokens. [P1 "Hva gjør DFlash annerledes
    enn vanlig spekulativ dekoding?"; P3 "Come funziona il drafting a
    blocchi"; P3 "L'idea chiave: Il target sa meglio"]"""
    cfg = small_cfg(block=16)
    NL, B = cfg.n_layers, cfg.block
    W = rand_weights(cfg, NL, seed=21)
    model = hf_model(cfg, W, NL)
    g = np.random.default_rng(100 + L)
    ctx = g.standard_normal((L, cfg.hidden))
    anchor = int(g.integers(0, cfg.vocab - 1))
    cache = ref.new_cache(cfg, 1, L + B + 3, fill=np.nan)
    ref.inject_kv(cfg, W, ctx, [(r, 0, r) for r in range(L)], cache)
    r = ref.draft_block(cfg, W, cache, [L], [anchor])

    ids = [anchor] + [cfg.mask_id] * (B - 1)
    pos = L + np.arange(B)
    z, hs, pre, post = _hf_block(model, cfg, ctx, L, ids, pos)
    for l in range(NL):
        assert ref.rel_err(r["hidden"][0, l], hs[l]) < TOL, f"hidden after layer {l}"
    assert ref.rel_err(r["hidden"][0, NL], pre) < TOL
    assert ref.rel_err(r["final"][0], post) < TOL
    assert ref.rel_err(r["logits"][0], z[1:]) < TOL
    zs = np.sort(z[1:], axis=1)
    assert np.all(zs[:, -1] - zs[:, -2] > 1e-3), "a near tie would make the token check meaningless"
    assert np.array_equal(r["draft"][0], np.argmax(z[1:], axis=1))

    # Each plausible slip in the assembly moves the result far outside the
    # tolerance, so an oracle that made it would fail the checks above.
    # (With no context every position shift is a global shift, which rotary
    # embeddings cannot see: the position slip is only checked for L >= 1.)
    far = 100 * TOL
    if L:
        z_pos = _hf_block(model, cfg, ctx, L, ids, pos + 1)
        assert ref.rel_err(z_pos[0][1:], z[1:]) > far, "block positions L+1+j"
    z_mask = _hf_block(model, cfg, ctx, L, [cfg.mask_id] * B, pos)
    assert ref.rel_err(z_mask[0][1:], z[1:]) > far, "row 0 holding the mask"
    assert ref.rel_err(z[:-1], z[1:]) > far, "LM rows shifted by one"
    z_nonorm = pre @ W["lm_head"].T
    assert ref.rel_err(z_nonorm[1:], z[1:]) > far, "final norm dropped"
    z_causal = _hf_block(model, cfg, ctx, L, ids, pos, causal=True)
    assert ref.rel_err(z_causal[0][1:], z[1:]) > far, "causal mask inside the block"
