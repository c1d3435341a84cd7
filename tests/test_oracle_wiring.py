"""Pins of the oracle's layer wiring and storage points.

The TensorFold page (#1851, "What this changes", item 1) describes the drafter layer
as a plain qwen3 body with eleven tensors and two residual adds; the Exactness list
keeps activations in bf16 with fp32 sums. These pins check, against torch's library
routines and a second implementation written apart from the oracle
(tests/textbook_round.py), that

  * the input norm feeds attention and the post-attention norm feeds the MLP;
  * residual add 1 lands on the layer input and residual add 2 on add 1's result;
  * every tensor the round stores is representable in the activation dtype, so no
    storage rounding is skipped;
  * whole rounds of several streams agree with the second implementation: stored
    tensors bit for bit, logits to float64 rounding.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import textbook_round as TB
from oracle import dflash_oracle as O
from test_oracle_pins import cfg_small, ctx_small, weights_small

STORED = ("a", "q", "k", "v", "o", "x_attn", "b", "m", "x_out")


def t(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


def rms(x, g, eps):
    return F.rms_norm(x, (x.shape[-1],), t(g), eps=eps)


def cfg3(**over):
    c = dict(n_layers=3, layer_window=[4, 0, 7], n_q_heads=6, n_kv_heads=2, head_dim=8, block_size=5)
    c.update(over)
    return cfg_small(**c)


def rounded_weights(cfg, seed=0):
    """Small weights rounded to the storage dtype, as a bound drafter would hold them."""
    W = weights_small(cfg, seed=seed)
    dt = "f64" if cfg.dtype == "f64" else cfg.dtype
    return {k: O.round_to(v, dt) for k, v in W.items()}


def stream_inputs(cfg, seeds):
    rng = np.random.default_rng(seeds)
    streams = []
    for s, (C, R, anchor) in enumerate([(9, 3, 4), (14, 6, 11), (6, 6, 0)]):
        k, v = ctx_small(cfg, C, seed=40 + s)
        k = [O.round_to(x, cfg.dtype) for x in k]
        v = [O.round_to(x, cfg.dtype) for x in v]
        taps = [O.round_to(rng.normal(0, 1, (R, cfg.hidden)), cfg.dtype) for _ in range(cfg.n_taps)]
        streams.append(dict(taps=taps, C=C, k_ctx=k, v_ctx=v, anchor=anchor))
    return streams


# ---------------------------------------------------------------- second implementation

@pytest.mark.parametrize("dtype", ["f64", "f32", "bf16"])
@pytest.mark.parametrize("make_cfg", [cfg_small, cfg3], ids=["2_layers", "3_layers"])
def test_whole_rounds_agree_with_the_second_implementation(dtype, make_cfg):
    cfg = make_cfg(dtype=dtype)
    W = rounded_weights(cfg)
    streams = stream_inputs(cfg, 7)
    orc = O.run_round(cfg, W, streams)
    tb = TB.Textbook(cfg, W)
    for s, st in enumerate(streams):
        f, ks, vs, logits, toks = tb.round(st["taps"], st["C"], st["k_ctx"], st["v_ctx"], st["anchor"])
        R = f.shape[0]
        exact = (lambda a, b: np.testing.assert_array_equal(a, b)) if dtype != "f64" else \
            (lambda a, b: np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12))
        exact(orc[s]["fused"], f.numpy())
        for l in range(cfg.n_layers):
            exact(orc[s]["kv"][l][0], ks[l][st["C"] - R:].numpy())
            exact(orc[s]["kv"][l][1], vs[l][st["C"] - R:].numpy())
        np.testing.assert_allclose(orc[s]["logits"], logits.numpy(), rtol=1e-11, atol=1e-11)
        np.testing.assert_array_equal(orc[s]["tokens"], toks.numpy())


def test_verify_agrees_with_the_second_implementation():
    rng = np.random.default_rng(21)
    for B in (2, 3, 8, 16):
        d = rng.integers(0, 3, (400, B - 1))
        tg = rng.integers(0, 3, (400, B))
        acc, bon, com = O.verify_greedy(d, tg)
        for i in range(400):
            a, b = TB.verify(d[i], tg[i])
            assert (acc[i], bon[i]) == (a, b)
            assert list(com[i]) == list(d[i][:a]) + [b] + [-1] * (B - 1 - a)


def test_second_implementation_rounding_is_single_rounding():
    # the round-to-odd route agrees with the correctly rounded value on cases where
    # a plain cast through fp32 would round twice
    x = torch.tensor([1.0 + 2.0 ** -8 + 2.0 ** -30, -(1.0 + 2.0 ** -8 + 2.0 ** -30), 1.0 + 2.0 ** -8,
                      1.0 + 3 * 2.0 ** -8, 3.0e38, 0.0], dtype=torch.float64)
    got = TB.round_storage(x, "bf16").tolist()
    assert got == [1.0 + 2.0 ** -7, -(1.0 + 2.0 ** -7), 1.0, 1.0 + 2.0 ** -6, float(torch.tensor(3.0e38).to(
        torch.bfloat16).double()), 0.0]
    rng = np.random.default_rng(5)
    v = rng.normal(0, 1, 100000) * np.exp2(rng.integers(-30, 30, 100000))
    np.testing.assert_array_equal(TB.round_storage(t(v), "bf16").numpy(), O.round_bf16(v))


# ---------------------------------------------------------------- storage points

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_every_stored_tensor_is_representable(dtype):
    cfg = cfg3(dtype=dtype)
    W = rounded_weights(cfg)
    st = stream_inputs(cfg, 8)[1]
    fused = O.fuse_taps(cfg, st["taps"], W)
    kv = O.inject_kv(cfg, fused, np.arange(st["C"] - fused.shape[0], st["C"]), W)
    tr = {}
    O.draft_stream(cfg, W, st["k_ctx"], st["v_ctx"], st["C"], st["anchor"], trace=tr)
    named = [("fused", fused), ("z", tr["z"])] + [(f"K{l}", kv[l][0]) for l in range(cfg.n_layers)] + \
            [(f"V{l}", kv[l][1]) for l in range(cfg.n_layers)]
    for l, lay in enumerate(tr["layers"]):
        named += [(f"layer {l} {n}", lay[n]) for n in STORED]
    for name, x in named:
        x = np.asarray(x, dtype=np.float64)
        np.testing.assert_array_equal(TB.round_storage(t(x), dtype).numpy(), x, err_msg=name)
        # and each is a genuinely rounded tensor, not one that happens to be exact
        assert np.mean(np.abs(x) > 0) > 0.5, name


# ---------------------------------------------------------------- wiring, step by step

@pytest.mark.parametrize("dtype", ["f64", "bf16"])
def test_layer_steps_chain_as_the_pages_describe(dtype):
    """Each stored tensor of a layer, recomputed with library routines from the stored
    tensors it depends on: the input norm's gain on a, the post norm's on b, add 1 on
    the layer input, add 2 on add 1's sum, SiLU on the gate branch only."""
    cfg = cfg3(dtype=dtype)
    W = rounded_weights(cfg)
    st = stream_inputs(cfg, 9)[0]
    tr = {}
    O.draft_stream(cfg, W, st["k_ctx"], st["v_ctx"], st["C"], st["anchor"], trace=tr)
    R = lambda x: TB.round_storage(x, dtype).numpy()
    eps = cfg.rms_eps
    X = t(tr["x0"])
    for l, lay in enumerate(tr["layers"]):
        p = f"layers.{l}."
        eq = (lambda a, b, n: np.testing.assert_array_equal(a, b, err_msg=f"layer {l} {n}")) if dtype != "f64" else \
            (lambda a, b, n: np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13, err_msg=f"layer {l} {n}"))
        eq(lay["a"], R(rms(X, W[p + "in_norm"], eps)), "a")
        eq(lay["x_attn"], R(X + F.linear(t(lay["o"]), t(W[p + "wo"]))), "x_attn")
        X1 = t(lay["x_attn"])
        eq(lay["b"], R(rms(X1, W[p + "post_norm"], eps)), "b")
        b = t(lay["b"])
        eq(lay["m"], R(F.silu(F.linear(b, t(W[p + "w_gate"]))) * F.linear(b, t(W[p + "w_up"]))), "m")
        eq(lay["x_out"], R(X1 + F.linear(t(lay["m"]), t(W[p + "w_down"]))), "x_out")
        X = t(lay["x_out"])
    eq(tr["z"], R(rms(X[1:], W["norm"], eps)), "z")


def _attention_only_logits(cfg, W, k_ctx, v_ctx, C, anchor):
    """Closed form of the round when every w_gate is zero: SiLU(0) = 0 makes the MLP
    product zero, so each layer is X + wo . attn(RMSNorm(X) * in_norm) alone."""
    tb = TB.Textbook(cfg, W)
    B = cfg.block_size
    X = t(W["embed"][[anchor] + [cfg.mask_token_id] * (B - 1)])
    pos = torch.arange(C, C + B)
    d, nq, nkv = cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads
    for l in range(cfg.n_layers):
        p = f"layers.{l}."
        a = rms(X, W[p + "in_norm"], cfg.rms_eps)
        q = TB.rotary(rms(F.linear(a, t(W[p + "wq"])).view(B, nq, d), W[p + "q_norm"], cfg.rms_eps), pos,
                      cfg.rope_theta)
        k = TB.rotary(rms(F.linear(a, t(W[p + "wk"])).view(B, nkv, d), W[p + "k_norm"], cfg.rms_eps), pos,
                      cfg.rope_theta)
        v = F.linear(a, t(W[p + "wv"])).view(B, nkv, d)
        w = cfg.layer_window[l]
        lo = max(0, C - w) if w > 0 else 0
        kk = torch.cat([t(k_ctx[l][lo:C]), k]).transpose(0, 1)
        vv = torch.cat([t(v_ctx[l][lo:C]), v]).transpose(0, 1)
        o = F.scaled_dot_product_attention(q.transpose(0, 1), kk, vv, enable_gqa=True).transpose(0, 1)
        X = X + F.linear(o.reshape(B, nq * d), t(W[p + "wo"]))
    z = rms(X[1:], W["norm"], cfg.rms_eps)
    del tb
    return F.linear(z, t(W["lm_head"])).numpy()


def test_zero_gate_leaves_attention_and_residual_add_one():
    cfg = cfg3(dtype="f64")
    W = weights_small(cfg, seed=3)
    for l in range(cfg.n_layers):
        W[f"layers.{l}.w_gate"] = np.zeros_like(W[f"layers.{l}.w_gate"])
    k, v = ctx_small(cfg, 11)
    tr = {}
    logits, _ = O.draft_stream(cfg, W, k, v, 11, 6, trace=tr)
    for lay in tr["layers"]:
        assert not np.any(lay["m"]), "SiLU(0) * up must be exactly zero"
        np.testing.assert_array_equal(lay["x_out"], lay["x_attn"])
    np.testing.assert_allclose(logits, _attention_only_logits(cfg, W, k, v, 11, 6), rtol=1e-11, atol=1e-11)


def test_zero_output_projection_leaves_the_mlp_on_the_layer_input():
    """wo = 0: add 1 returns the layer input, and add 2 is X + w_down . SwiGLU(RMSNorm(X) * post_norm)."""
    cfg = cfg3(dtype="f64")
    W = weights_small(cfg, seed=4)
    for l in range(cfg.n_layers):
        W[f"layers.{l}.wo"] = np.zeros_like(W[f"layers.{l}.wo"])
    k, v = ctx_small(cfg, 11)
    logits, _ = O.draft_stream(cfg, W, k, v, 11, 2)
    B = cfg.block_size
    X = t(W["embed"][[2] + [cfg.mask_token_id] * (B - 1)])
    for l in range(cfg.n_layers):
        p = f"layers.{l}."
        b = rms(X, W[p + "post_norm"], cfg.rms_eps)
        X = X + F.linear(F.silu(F.linear(b, t(W[p + "w_gate"]))) * F.linear(b, t(W[p + "w_up"])), t(W[p + "w_down"]))
    ref = F.linear(rms(X[1:], W["norm"], cfg.rms_eps), t(W["lm_head"])).numpy()
    np.testing.assert_allclose(logits, ref, rtol=1e-11, atol=1e-11)


# ---------------------------------------------------------------- context built from taps

@pytest.mark.parametrize("dtype", ["f64", "f32", "bf16"])
def test_context_from_taps_agrees_with_the_second_implementation(dtype):
    # The existing context built the way a round builds its rows (fuse, then inject at
    # positions 0..n-1), against the textbook fuse and K/V of the second implementation.
    cfg = cfg_small(dtype=dtype)
    W = rounded_weights(cfg)
    rng = np.random.default_rng(71)
    n = 11
    taps = [O.round_to(rng.normal(0, 1, (n, cfg.hidden)), dtype) for _ in range(cfg.n_taps)]
    k_ctx, v_ctx = O.context_from_taps(cfg, taps, W)
    tb = TB.Textbook(cfg, W)
    f = tb.fuse(taps)
    for l in range(cfg.n_layers):
        k, v = tb.context_kv(f, torch.arange(n), l)
        if dtype == "f64":
            np.testing.assert_allclose(k_ctx[l], k.numpy(), rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(v_ctx[l], v.numpy(), rtol=1e-12, atol=1e-12)
        else:
            np.testing.assert_array_equal(k_ctx[l], k.numpy())
            np.testing.assert_array_equal(v_ctx[l], v.numpy())
    e_k, e_v = O.context_from_taps(cfg, [t[:0] for t in taps], W)
    assert all(x.shape == (0, cfg.n_kv_heads, cfg.head_dim) for x in e_k + e_v)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_round_over_a_context_from_taps_does_not_depend_on_where_the_round_starts(dtype):
    # The same n + R tap rows, split as n context rows and R round rows or as n + R - 2
    # and 2: each row lands at its own position either way, so the round's cache and
    # its logits are the same bits (a context row placed one position off would move them).
    cfg = cfg_small(dtype=dtype)
    W = rounded_weights(cfg)
    rng = np.random.default_rng(72)
    n, R = 9, 4
    taps = [O.round_to(rng.normal(0, 1, (n + R, cfg.hidden)), dtype) for _ in range(cfg.n_taps)]
    a = O.run_round(cfg, W, [dict(taps=[t[n:] for t in taps], C=n + R, ctx_taps=[t[:n] for t in taps], anchor=5)])
    b = O.run_round(cfg, W, [dict(taps=[t[n + R - 2:] for t in taps], C=n + R, ctx_taps=[t[:n + R - 2] for t in taps],
                                  anchor=5)])
    np.testing.assert_array_equal(a[0]["logits"], b[0]["logits"])
    np.testing.assert_array_equal(a[0]["tokens"], b[0]["tokens"])
    for l in range(cfg.n_layers):
        np.testing.assert_array_equal(a[0]["kv"][l][0][R - 2:], b[0]["kv"][l][0])
