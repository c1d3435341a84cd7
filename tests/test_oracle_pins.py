"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these re-types the oracle's own formulas: each check is a closed form,
an invariant, a special case that reduces to a library or textbook routine,
a brute-force enumeration, or a figure printed on the pages (tests/golden).
"""
import itertools
import json
import math
import os
from types import SimpleNamespace

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import dflash_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def cfg_small(**over):
    c = dict(dtype="f64", hidden=32, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=8,
             intermediate=48, vocab=64, block_size=6, mask_token_id=63,
             layer_window=[5, 0], rope_theta=1.0e4, rms_eps=1e-6, n_taps=3)
    c.update(over)
    return SimpleNamespace(**c)


def weights_small(cfg, seed=0, gain_noise=0.1):
    rng = np.random.default_rng(seed)
    h, d, I = cfg.hidden, cfg.head_dim, cfg.intermediate
    W = {"embed": rng.normal(0, 1, (cfg.vocab, h)), "lm_head": rng.normal(0, 0.2, (cfg.vocab, h)),
         "fc": rng.normal(0, 0.2, (h, cfg.n_taps * h)),
         "hidden_norm": 1 + rng.normal(0, gain_noise, h), "norm": 1 + rng.normal(0, gain_noise, h)}
    for l in range(cfg.n_layers):
        p = f"layers.{l}."
        W[p + "in_norm"] = 1 + rng.normal(0, gain_noise, h)
        W[p + "post_norm"] = 1 + rng.normal(0, gain_noise, h)
        W[p + "wq"] = rng.normal(0, 0.3, (cfg.n_q_heads * d, h))
        W[p + "wk"] = rng.normal(0, 0.3, (cfg.n_kv_heads * d, h))
        W[p + "wv"] = rng.normal(0, 0.3, (cfg.n_kv_heads * d, h))
        W[p + "wo"] = rng.normal(0, 0.2, (h, cfg.n_q_heads * d))
        W[p + "q_norm"] = 1 + rng.normal(0, gain_noise, d)
        W[p + "k_norm"] = 1 + rng.normal(0, gain_noise, d)
        W[p + "w_gate"] = rng.normal(0, 0.2, (I, h))
        W[p + "w_up"] = rng.normal(0, 0.2, (I, h))
        W[p + "w_down"] = rng.normal(0, 0.2, (h, I))
    return W


def ctx_small(cfg, C, seed=1):
    rng = np.random.default_rng(seed)
    k = [rng.normal(0, 1, (C, cfg.n_kv_heads, cfg.head_dim)) for _ in range(cfg.n_layers)]
    v = [rng.normal(0, 1, (C, cfg.n_kv_heads, cfg.head_dim)) for _ in range(cfg.n_layers)]
    return k, v


# ---------------------------------------------------------------- bf16 rounding

def test_round_bf16_matches_torch_rne_on_fp32_values():
    rng = np.random.default_rng(3)
    x32 = (rng.normal(0, 1, 400000) * np.exp2(rng.integers(-140, 120, 400000))).astype(np.float32)
    x32 = np.concatenate([x32, np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38], np.float32)])
    ours = O.round_bf16(x32.astype(np.float64))
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_round_bf16_special_cases():
    r = lambda v: float(O.round_bf16(np.array([v]))[0])
    assert r(1.0 + 2.0 ** -8) == 1.0                       # tie -> even (k=128)
    assert r(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6        # tie -> even (k=130)
    assert r(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7  # one rounding, no fp32 stage
    assert r(-(1.0 + 2.0 ** -8 + 2.0 ** -30)) == -(1.0 + 2.0 ** -7)
    assert r(2.0 ** -134) == 0.0                            # subnormal tie -> even (0)
    assert r(3 * 2.0 ** -134) == 2.0 ** -132                # subnormal tie -> even
    assert r(2.0 ** 128) == math.inf
    assert r((2.0 - 2.0 ** -7) * 2.0 ** 127) == (2.0 - 2.0 ** -7) * 2.0 ** 127
    bits = O.bf16_bits(np.array([1.0, -2.0, 0.5]))
    assert list(bits) == [0x3F80, 0xC000, 0x3F00]
    np.testing.assert_array_equal(O.bf16_bits_to_f64(bits), [1.0, -2.0, 0.5])


# ---------------------------------------------------------------- building blocks

def test_rms_norm_matches_library_and_closed_form():
    rng = np.random.default_rng(4)
    x = rng.normal(0, 3, (5, 7, 64))
    g = rng.normal(1, 0.3, 64)
    ref = F.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(O.rms_norm(x, g, 1e-6), ref, rtol=1e-13, atol=1e-13)
    c = np.full(16, 2.5)
    np.testing.assert_allclose(O.rms_norm(c, np.ones(16), 0.0), np.ones(16), rtol=1e-15)
    y = O.rms_norm(x, np.ones(64), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, -1)), 1.0, rtol=1e-13)


def test_rope_closed_forms_and_invariants():
    rng = np.random.default_rng(5)
    d, theta = 16, 1.0e6
    x = rng.normal(0, 1, (9, d))
    pos = np.arange(9) * 37.0
    y = O.rope(x, pos, theta)
    # complex-multiplication form: z_i = x_i + i x_{i+d/2} turns by pos * theta^(-2i/d)
    z = (x[:, :d // 2] + 1j * x[:, d // 2:]) * np.exp(1j * pos[:, None] * theta ** (-2.0 * np.arange(d // 2) / d))
    np.testing.assert_allclose(y, np.concatenate([z.real, z.imag], -1), rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(O.rope(x, np.zeros(9), theta), x)           # p = 0 is the identity
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    # d = 2: a plane rotation by pos radians
    v = np.array([[1.0, 0.0]])
    np.testing.assert_allclose(O.rope(v, np.array([0.7]), theta), [[math.cos(0.7), math.sin(0.7)]], rtol=1e-15)
    # scores depend only on the position difference
    q, k = rng.normal(0, 1, d), rng.normal(0, 1, d)
    s1 = O.rope(q, np.array(100.0), theta) @ O.rope(k, np.array(40.0), theta)
    s2 = O.rope(q, np.array(1100.0), theta) @ O.rope(k, np.array(1040.0), theta)
    assert abs(s1 - s2) < 1e-12


def test_silu_and_softmax_match_library():
    x = np.linspace(-20, 20, 1001)
    np.testing.assert_allclose(O.silu(x), F.silu(torch.from_numpy(x)).numpy(), rtol=1e-14, atol=1e-300)
    s = np.random.default_rng(6).normal(0, 5, (4, 33))
    np.testing.assert_allclose(O.softmax(s), torch.softmax(torch.from_numpy(s), -1).numpy(), rtol=1e-14)


# ---------------------------------------------------------------- attention

def test_block_attention_matches_library_sdpa_with_gqa():
    rng = np.random.default_rng(7)
    B, N, nq, nkv, d = 6, 23, 8, 2, 16
    q = rng.normal(0, 1, (B, nq, d))
    k = rng.normal(0, 1, (N, nkv, d))
    v = rng.normal(0, 1, (N, nkv, d))
    o = O.block_attention(q, k, v, nkv)
    g = nq // nkv
    kk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(g, 0)   # [nq, N, d]
    vv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(g, 0)
    ref = F.scaled_dot_product_attention(torch.from_numpy(q).permute(1, 0, 2), kk, vv, is_causal=False)
    np.testing.assert_allclose(o, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_block_attention_special_cases():
    rng = np.random.default_rng(8)
    B, nq, nkv, d = 4, 4, 2, 8
    q = rng.normal(0, 1, (B, nq, d))
    one_k, one_v = rng.normal(0, 1, (1, nkv, d)), rng.normal(0, 1, (1, nkv, d))
    o = O.block_attention(q, one_k, one_v, nkv)
    for h in range(nq):
        np.testing.assert_allclose(o[:, h], np.broadcast_to(one_v[0, h // 2], (B, d)), rtol=1e-15)
    # identical keys -> uniform weights -> the mean of the values
    k = np.broadcast_to(one_k, (9, nkv, d)).copy()
    v = rng.normal(0, 1, (9, nkv, d))
    o = O.block_attention(q, k, v, nkv)
    for h in range(nq):
        np.testing.assert_allclose(o[:, h], np.broadcast_to(v[:, h // 2].mean(0), (B, d)), rtol=1e-12, atol=1e-14)
    # non-causal: the key order does not matter
    k = rng.normal(0, 1, (9, nkv, d))
    perm = rng.permutation(9)
    np.testing.assert_allclose(O.block_attention(q, k, v, nkv), O.block_attention(q, k[perm], v[perm], nkv),
                               rtol=1e-12, atol=1e-14)
    # GQA with duplicated kv heads equals the same heads read as full multi-head attention
    kd, vd = np.repeat(k, nq // nkv, axis=1), np.repeat(v, nq // nkv, axis=1)
    np.testing.assert_allclose(O.block_attention(q, k, v, nkv), O.block_attention(q, kd, vd, nq),
                               rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- fuse

def test_fuse_identity_fc_is_textbook_rmsnorm_of_each_tap():
    cfg = cfg_small()
    h, n = cfg.hidden, cfg.n_taps
    rng = np.random.default_rng(9)
    taps = [rng.normal(0, 1, (5, h)) for _ in range(n)]
    W = weights_small(cfg)
    for i in range(n):
        fc = np.zeros((h, n * h))
        fc[:, i * h:(i + 1) * h] = np.eye(h)       # selects tap plane i
        W["fc"] = fc
        ref = F.rms_norm(torch.from_numpy(taps[i]), (h,), torch.from_numpy(W["hidden_norm"]), eps=cfg.rms_eps)
        np.testing.assert_allclose(O.fuse_taps(cfg, taps, W), ref.numpy(), rtol=1e-13, atol=1e-13)


def test_fuse_is_linear_in_taps_then_scale_free():
    cfg = cfg_small(rms_eps=0.0)
    rng = np.random.default_rng(10)
    W = weights_small(cfg)
    taps = [rng.normal(0, 1, (4, cfg.hidden)) for _ in range(cfg.n_taps)]
    a = O.fuse_taps(cfg, taps, W)
    b = O.fuse_taps(cfg, [3.0 * t for t in taps], W)
    np.testing.assert_allclose(a, b, rtol=1e-12)
    # the fc output is the sum of per-tap products: one tap's contribution scales alone
    W2 = dict(W)
    fc = W["fc"].copy()
    fc[:, cfg.hidden:] = 0.0
    W2["fc"] = fc
    c = O.fuse_taps(cfg, [taps[0], 100 * taps[1], -7 * taps[2]], W2)
    np.testing.assert_allclose(c, O.fuse_taps(cfg, [taps[0], 0 * taps[1], 0 * taps[2]], W2), rtol=1e-12)


def test_storage_closed_forms_from_the_pages():
    g = json.load(open(os.path.join(GOLDEN, "storage_sizes.json")))
    fr = g["fused_row"]
    assert O.fused_row_bytes(fr["hidden"]) == fr["fused_bytes"] == 8 * 1024
    assert O.raw_tap_row_bytes(fr["n_taps"], fr["hidden"]) == fr["raw_bytes"] == 64 * 1024
    t = g["tap_row_fusing"]
    assert O.tap_row_bytes(t["n_taps"], t["hidden"], True) == t["rows_of_hidden"] * t["hidden"] * t["elem_bytes"]
    assert O.tap_row_bytes(5, 5120, False) == g["tap_row_raw"]["n_planes"] * 5120 * 2


# ---------------------------------------------------------------- inject

def test_inject_projection_orientation_and_no_input_norm():
    cfg = cfg_small()
    W = weights_small(cfg)
    h, d = cfg.hidden, cfg.head_dim
    rng = np.random.default_rng(11)
    f = rng.normal(0, 1, (3, h))
    wv = np.zeros((cfg.n_kv_heads * d, h))
    wv[:d, :d] = np.eye(d)                 # kv head 0 of V copies the first d features
    wv[d:2 * d, h - d:] = 2 * np.eye(d)    # kv head 1 copies twice the last d features
    W["layers.0.wv"] = wv
    kv = O.inject_kv(cfg, f, np.arange(3), W)
    np.testing.assert_allclose(kv[0][1][:, 0], f[:, :d], rtol=1e-15)
    np.testing.assert_allclose(kv[0][1][:, 1], 2 * f[:, h - d:], rtol=1e-15)
    # V is linear in the fused row (no input norm): scaling f scales V
    kv3 = O.inject_kv(cfg, 3 * f, np.arange(3), W)
    np.testing.assert_allclose(kv3[1][1], 3 * kv[1][1], rtol=1e-12)
    # K at position 0 is the textbook RMSNorm of each head of wk . f (RoPE is the identity there)
    kv0 = O.inject_kv(cfg, f, np.zeros(3), W)
    k_raw = torch.from_numpy(f @ W["layers.1.wk"].T).reshape(3, cfg.n_kv_heads, d)
    ref = F.rms_norm(k_raw, (d,), torch.from_numpy(W["layers.1.k_norm"]), eps=cfg.rms_eps).numpy()
    np.testing.assert_allclose(kv0[1][0], ref, rtol=1e-13, atol=1e-13)


def test_inject_in_chunks_equals_one_shot():
    cfg = cfg_small()
    W = weights_small(cfg)
    f = np.random.default_rng(12).normal(0, 1, (7, cfg.hidden))
    pos = np.arange(10, 17)
    one = O.inject_kv(cfg, f, pos, W)
    a, b = O.inject_kv(cfg, f[:3], pos[:3], W), O.inject_kv(cfg, f[3:], pos[3:], W)
    for l in range(cfg.n_layers):
        for i in range(2):
            np.testing.assert_array_equal(one[l][i], np.concatenate([a[l][i], b[l][i]]))


# ---------------------------------------------------------------- draft block

class Recorder(dict):
    """A weights dict that records which tensor names are read."""

    def __init__(self, *a, **k):
        super().__init__(*a, **k)
        self.seen = set()

    def __getitem__(self, key):
        self.seen.add(key)
        return super().__getitem__(key)


def test_draft_reads_eleven_tensors_a_layer_plus_three():
    g = json.load(open(os.path.join(GOLDEN, "storage_sizes.json")))
    cfg = cfg_small(n_layers=g["tensor_names"]["layers"])
    cfg.layer_window = [0] * cfg.n_layers
    W = Recorder(weights_small(cfg))
    k, v = ctx_small(cfg, 10)
    taps = [np.ones((1, cfg.hidden))] * cfg.n_taps
    O.fuse_taps(cfg, taps, W)
    O.draft_stream(cfg, W, k, v, 10, 3)
    drafter = W.seen - {"embed", "lm_head"}
    per_layer = {n.split(".")[-1] for n in drafter if n.startswith("layers.")}
    assert len(per_layer) == g["tensor_names"]["per_layer"]
    assert len(drafter) == g["tensor_names"]["total"] == 11 * cfg.n_layers + 3


def test_block_has_anchor_plus_fifteen_mask_rows():
    g = json.load(open(os.path.join(GOLDEN, "storage_sizes.json")))["block"]
    cfg = cfg_small(block_size=g["block_size"])
    W = weights_small(cfg)
    k, v = ctx_small(cfg, 12)
    tr = {}
    logits, toks = O.draft_stream(cfg, W, k, v, 12, 5, trace=tr)
    assert logits.shape == (g["mask_rows"], cfg.vocab) and toks.shape == (15,)
    np.testing.assert_array_equal(tr["x0"][0], W["embed"][5])
    for j in range(1, 16):
        np.testing.assert_array_equal(tr["x0"][j], W["embed"][cfg.mask_token_id])


def test_zero_output_projections_make_every_layer_the_identity():
    """With wo = w_down = 0 both residual adds add nothing: a closed form for the logits."""
    for dtype in ("f64", "f32", "bf16"):
        cfg = cfg_small(dtype=dtype)
        W = weights_small(cfg)
        for l in range(cfg.n_layers):
            W[f"layers.{l}.wo"] = np.zeros_like(W[f"layers.{l}.wo"])
            W[f"layers.{l}.w_down"] = np.zeros_like(W[f"layers.{l}.w_down"])
        W["embed"] = O.round_to(W["embed"], dtype)
        k, v = ctx_small(cfg, 9)
        logits, toks = O.draft_stream(cfg, W, k, v, 9, 4)
        e = W["embed"][cfg.mask_token_id]
        z = O.round_to(e / np.sqrt(np.mean(e * e) + cfg.rms_eps) * W["norm"], dtype)
        expect = W["lm_head"] @ z
        for j in range(cfg.block_size - 1):
            np.testing.assert_allclose(logits[j], expect, rtol=1e-12, atol=1e-12)
        assert np.all(toks == np.argmax(expect))


def test_each_residual_branch_can_be_silenced_alone():
    cfg = cfg_small()
    W = weights_small(cfg)
    k, v = ctx_small(cfg, 9)
    # w_down = 0: gate/up no longer matter
    W0 = dict(W)
    for l in range(cfg.n_layers):
        W0[f"layers.{l}.w_down"] = np.zeros_like(W[f"layers.{l}.w_down"])
    W1 = dict(W0)
    for l in range(cfg.n_layers):
        W1[f"layers.{l}.w_gate"] = W0[f"layers.{l}.w_gate"] * -3.0
    np.testing.assert_array_equal(O.draft_stream(cfg, W0, k, v, 9, 4)[0], O.draft_stream(cfg, W1, k, v, 9, 4)[0])
    # wo = 0: the context no longer matters
    W2 = dict(W)
    for l in range(cfg.n_layers):
        W2[f"layers.{l}.wo"] = np.zeros_like(W[f"layers.{l}.wo"])
    k2, v2 = ctx_small(cfg, 9, seed=99)
    np.testing.assert_array_equal(O.draft_stream(cfg, W2, k, v, 9, 4)[0], O.draft_stream(cfg, W2, k2, v2, 9, 4)[0])
    # but both branches do contribute when present
    assert not np.array_equal(O.draft_stream(cfg, W, k, v, 9, 4)[0], O.draft_stream(cfg, W0, k, v, 9, 4)[0])
    assert not np.array_equal(O.draft_stream(cfg, W, k, v, 9, 4)[0], O.draft_stream(cfg, W2, k, v, 9, 4)[0])


def test_block_is_non_causal():
    """Row 0 (the anchor) sees the mask rows after it: changing the mask token moves it."""
    cfg = cfg_small()
    W = weights_small(cfg)
    k, v = ctx_small(cfg, 9)
    t1, t2 = {}, {}
    O.draft_stream(cfg, W, k, v, 9, 4, trace=t1)
    cfg2 = cfg_small(mask_token_id=17)
    O.draft_stream(cfg2, W, k, v, 9, 4, trace=t2)
    assert np.max(np.abs(t1["layers"][0]["o"][0] - t2["layers"][0]["o"][0])) > 1e-6
    np.testing.assert_array_equal(t1["x0"][0], t2["x0"][0])


def test_sliding_layer_reach_by_perturbation():
    """A sliding layer reads only its own window of the context; the full layer reads all of it."""
    cfg = cfg_small(layer_window=[5, 0])
    W = weights_small(cfg)
    C = 12
    k, v = ctx_small(cfg, C)
    base = O.draft_stream(cfg, W, k, v, C, 4)[0]
    kp = [x.copy() for x in k]
    vp = [x.copy() for x in v]
    kp[0][:C - 5] += 5.0
    vp[0][:C - 5] -= 3.0       # layer 0 (sliding 5): rows before C-5 are out of reach
    np.testing.assert_array_equal(O.draft_stream(cfg, W, kp, vp, C, 4)[0], base)
    kp[0][C - 5] += 1.0        # the oldest row inside the window is read
    assert not np.array_equal(O.draft_stream(cfg, W, kp, vp, C, 4)[0], base)
    kq = [x.copy() for x in k]
    kq[1][0] += 1.0            # layer 1 (full) reads position 0
    assert not np.array_equal(O.draft_stream(cfg, W, kq, v, C, 4)[0], base)
    # a window covering the whole context is the full layer, bit for bit
    cfg_w = cfg_small(layer_window=[C, 0])
    cfg_f = cfg_small(layer_window=[0, 0])
    np.testing.assert_array_equal(O.draft_stream(cfg_w, W, k, v, C, 4)[0], O.draft_stream(cfg_f, W, k, v, C, 4)[0])


def test_round_is_invariant_to_a_global_position_shift():
    """Shifting every position (context and block) by D leaves the logits unchanged (f64 mode)."""
    cfg = cfg_small(layer_window=[7, 7])
    W = weights_small(cfg)
    rng = np.random.default_rng(13)
    R, D = 7, 11
    taps = [rng.normal(0, 1, (R, cfg.hidden)) for _ in range(cfg.n_taps)]
    f = O.fuse_taps(cfg, taps, W)
    kv_a = O.inject_kv(cfg, f, np.arange(R), W)
    kv_b = O.inject_kv(cfg, f, np.arange(D, D + R), W)
    pad = np.full((D, cfg.n_kv_heads, cfg.head_dim), 1e3)   # out of every window
    la = O.draft_stream(cfg, W, [x[0] for x in kv_a], [x[1] for x in kv_a], R, 2)[0]
    lb = O.draft_stream(cfg, W, [np.concatenate([pad, x[0]]) for x in kv_b],
                        [np.concatenate([pad, x[1]]) for x in kv_b], R + D, 2)[0]
    np.testing.assert_allclose(la, lb, rtol=1e-9, atol=1e-9)


def test_streams_are_independent():
    cfg = cfg_small()
    W = weights_small(cfg)
    rng = np.random.default_rng(14)
    streams = []
    for s in range(3):
        R = 2 + s
        C = 8 + 3 * s
        k, v = ctx_small(cfg, C, seed=20 + s)
        streams.append(dict(taps=[rng.normal(0, 1, (R, cfg.hidden)) for _ in range(cfg.n_taps)],
                            C=C, k_ctx=k, v_ctx=v, anchor=s + 1))
    together = O.run_round(cfg, W, streams)
    for s in range(3):
        solo = O.run_round(cfg, W, [streams[s]])[0]
        np.testing.assert_array_equal(together[s]["logits"], solo["logits"])


# ---------------------------------------------------------------- argmax and verify

def test_argmax_lowest_index_by_brute_force():
    rng = np.random.default_rng(15)
    x = rng.integers(0, 4, (500, 37)).astype(np.float64)    # many ties
    got = O.argmax_lowest(x)
    for r in range(x.shape[0]):
        best = 0
        for i in range(1, x.shape[1]):
            if x[r, i] > x[r, best]:
                best = i
        assert got[r] == best
    t1, t2 = O.top2(np.array([[1.0, 5.0, 5.0, 2.0]]))
    assert t1[0] == 5.0 and t2[0] == 5.0


def _verify_by_definition(d, t):
    """a = max{k in 0..B-1 : d_j = t_{j-1} for every 1 <= j <= k}."""
    Bm1 = len(d)
    a = max(k for k in range(Bm1 + 1) if all(d[j - 1] == t[j - 1] for j in range(1, k + 1)))
    return a, t[a]


@pytest.mark.parametrize("B", [2, 3, 4, 5])
def test_verify_exhaustive_against_definition(B):
    V = 3
    drafts = list(itertools.product(range(V), repeat=B - 1))
    targets = list(itertools.product(range(V), repeat=B))
    D = np.array([d for d in drafts for _ in targets])
    T = np.array([t for _ in drafts for t in targets])
    acc, bonus, com = O.verify_greedy(D, T)
    for i in range(len(D)):
        a, b = _verify_by_definition(list(D[i]), list(T[i]))
        assert acc[i] == a and bonus[i] == b
        assert list(com[i][:a]) == list(D[i][:a]) and com[i][a] == b and all(com[i][a + 1:] == -1)


def test_verify_golden_cases():
    g = json.load(open(os.path.join(GOLDEN, "verify_greedy_cases.json")))
    for c in g["cases"]:
        acc, bonus, com = O.verify_greedy(np.array([c["draft"]]), np.array([c["target"]]))
        assert acc[0] == c["accept"], c["name"]
        assert bonus[0] == c["bonus"], c["name"]
        assert list(com[0]) == c["committed"], c["name"]


# ---------------------------------------------------------------- the tiny preset end to end

def test_tiny_preset_round_runs_and_is_finite():
    import workloads as wl
    p = wl.preset("tiny_f32")
    W = {k: v.numpy() for k, v in wl.make_weights(p).items()}
    C = 128
    taps = [t.numpy() for t in wl.make_taps(p, 8)]
    k = [wl.make_context_kv(p, l, 0, C, "k").numpy() for l in range(p.n_layers)]
    v = [wl.make_context_kv(p, l, 0, C, "v").numpy() for l in range(p.n_layers)]
    out = O.run_round(p, W, [dict(taps=taps, C=C, k_ctx=k, v_ctx=v, anchor=int(wl.make_anchor(p)[0]))])[0]
    assert out["fused"].shape == (8, 256) and np.all(np.isfinite(out["logits"]))
    assert out["tokens"].shape == (7,)
    # gains ~ 1 + N(0, 0.02): logits have a usable spread (reading of the weight recipe)
    assert 0.05 < np.std(out["logits"]) < 5


def test_swiglu_is_linear_in_the_up_projection_only():
    """SiLU gates the w_gate branch: scaling w_up scales the MLP output, scaling w_gate does not."""
    cfg = cfg_small(n_layers=1, layer_window=[0])
    W = weights_small(cfg)
    k, v = ctx_small(cfg, 9)
    t1, t2, t3 = {}, {}, {}
    O.draft_stream(cfg, W, k, v, 9, 4, trace=t1)
    W2 = dict(W)
    W2["layers.0.w_up"] = 3.0 * W["layers.0.w_up"]
    O.draft_stream(cfg, W2, k, v, 9, 4, trace=t2)
    np.testing.assert_allclose(t2["layers"][0]["m"], 3.0 * t1["layers"][0]["m"], rtol=1e-12, atol=1e-14)
    W3 = dict(W)
    W3["layers.0.w_gate"] = 3.0 * W["layers.0.w_gate"]
    O.draft_stream(cfg, W3, k, v, 9, 4, trace=t3)
    assert np.max(np.abs(t3["layers"][0]["m"] - 3.0 * t1["layers"][0]["m"])) > 1e-3


def test_block_rows_continue_the_context_positions():
    """Block and context share one position axis: the anchor sits at position C.

    The anchor row's key at a layer equals the key that injection gives the
    same (normed) input row at position C; mask row j likewise sits at C + j.
    """
    cfg = cfg_small()
    W = weights_small(cfg)
    C = 9
    k, v = ctx_small(cfg, C)
    tr = {}
    O.draft_stream(cfg, W, k, v, C, 4, trace=tr)
    for l in range(cfg.n_layers):
        a = tr["layers"][l]["a"]
        kv = O.inject_kv(cfg, a, C + np.arange(cfg.block_size), W)
        np.testing.assert_allclose(tr["layers"][l]["k"], kv[l][0], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(tr["layers"][l]["v"], kv[l][1], rtol=1e-12, atol=1e-12)
