"""A second, independent float64 implementation of the DFlash draft round, in torch.

Test infrastructure: it exists only to check the oracle (oracle/dflash_oracle.py)
against something other than itself. It shares no code with the oracle or with the
HIP library and is written as a textbook model would be: torch's own RMSNorm,
linear, SiLU and grouped-query scaled-dot-product attention, rotary embedding in its
complex-multiplication form, and bf16 rounding through fp32 rounded to odd (a
double-rounding-free route from float64; Boldo and Melquiond, "When double rounding
is odd", 2005) instead of the oracle's frexp/rint grid.

What the round computes (the pages on DFlash, by title and section):
  * fuse: fc over the tap planes side by side, then the hidden_norm RMSNorm
    (TensorFold #1851, "What this changes", items 3-4);
  * inject: per layer, k = RoPE(k_norm(wk f)) and v = wv f of each fused row, with no
    input norm (item 4; DFlash explainer section 3, "KV injection");
  * draft: a plain qwen3 layer stack over the anchor and B-1 mask rows, non-causal,
    with two residual adds a layer; a sliding layer sees the last W context rows
    plus the block, a full layer all of them (item 1 and 4; explainer section 3);
    final norm, shared LM head, top-1 per mask row (explainer section 5);
  * verify: the longest prefix of drafts equal to the target's argmax, and the
    target's token after it (explainer section 4, "Greedy decoding").
The storage points (where a stored tensor is rounded to the activation dtype) are
the fused row, the context K/V, each normalised layer input, the block's q/k/v, the
attention output, the two residual sums, the SwiGLU product and the final-normed
mask rows. Logits are not rounded.
"""
import math

import torch
import torch.nn.functional as F

DT = torch.float64


def round_storage(x, dtype):
    """Round float64 values to the storage dtype ("f64": unchanged)."""
    if dtype == "f64":
        return x
    if dtype == "f32":
        return x.to(torch.float32).to(DT)
    assert dtype == "bf16", dtype
    f = x.to(torch.float32)                      # nearest fp32
    back = f.to(DT)
    inexact = back != x
    bits = f.view(torch.int32)
    # round to odd: step the fp32 value back toward zero when the cast went past x,
    # then set the last bit of every inexact result
    bits = bits - (inexact & (back.abs() > x.abs())).to(torch.int32)
    bits = bits | inexact.to(torch.int32)
    return bits.view(torch.float32).to(torch.bfloat16).to(DT)


def t64(a):
    """numpy / torch storage (float values) -> float64 tensor."""
    return torch.as_tensor(a).to(DT) if torch.is_tensor(a) else torch.from_numpy(a).to(DT)


def rotary(x, pos, theta):
    """Rotary embedding, complex form: element i of the first half and element i of
    the second half form one complex number, turned by the angle pos * theta^(-2i/d).
    x [..., n, d] with pos broadcasting over [...] (one position per row)."""
    d = x.shape[-1]
    half = d // 2
    freq = torch.pow(torch.tensor(float(theta), dtype=DT), -torch.arange(0, d, 2, dtype=DT) / d)
    ang = pos.to(DT)[..., None, None] * freq                    # [..., 1, half]
    z = torch.complex(x[..., :half], x[..., half:]) * torch.polar(torch.ones_like(ang), ang)
    return torch.cat([z.real, z.imag], dim=-1)


class Textbook:
    """The round for one config (SimpleNamespace or preset) and a float64 weight dict."""

    def __init__(self, cfg, W):
        self.c = cfg
        self.W = {k: t64(v) for k, v in W.items()}
        self.dt = cfg.dtype

    def R(self, x):
        return round_storage(x, self.dt)

    def norm(self, x, g):
        return F.rms_norm(x, (x.shape[-1],), g, eps=float(self.c.rms_eps))

    def fuse(self, taps):
        x = torch.cat([t64(t) for t in taps], dim=-1)
        return self.R(self.norm(F.linear(x, self.W["fc"]), self.W["hidden_norm"]))

    def context_kv(self, f, pos, layer):
        c, W, p = self.c, self.W, f"layers.{layer}."
        rows = f.shape[0]
        k = self.norm(F.linear(f, W[p + "wk"]).view(rows, c.n_kv_heads, c.head_dim), W[p + "k_norm"])
        k = rotary(k, pos, c.rope_theta)
        v = F.linear(f, W[p + "wv"]).view(rows, c.n_kv_heads, c.head_dim)
        return self.R(k), self.R(v)

    def layer(self, l, X, k_ctx, v_ctx, C):
        c, W, p = self.c, self.W, f"layers.{l}."
        B = X.shape[0]
        pos = torch.arange(C, C + B)
        a = self.R(self.norm(X, W[p + "in_norm"]))
        q = self.norm(F.linear(a, W[p + "wq"]).view(B, c.n_q_heads, c.head_dim), W[p + "q_norm"])
        k = self.norm(F.linear(a, W[p + "wk"]).view(B, c.n_kv_heads, c.head_dim), W[p + "k_norm"])
        v = F.linear(a, W[p + "wv"]).view(B, c.n_kv_heads, c.head_dim)
        q, k, v = self.R(rotary(q, pos, c.rope_theta)), self.R(rotary(k, pos, c.rope_theta)), self.R(v)
        w = c.layer_window[l]
        lo = max(0, C - w) if w > 0 else 0
        keys = torch.cat([k_ctx[lo:C], k], dim=0).transpose(0, 1)       # [n_kv, N, d]
        vals = torch.cat([v_ctx[lo:C], v], dim=0).transpose(0, 1)
        o = F.scaled_dot_product_attention(q.transpose(0, 1), keys, vals, is_causal=False, enable_gqa=True,
                                           scale=1.0 / math.sqrt(c.head_dim))
        o = self.R(o.transpose(0, 1).reshape(B, c.n_q_heads * c.head_dim))
        X = self.R(X + F.linear(o, W[p + "wo"]))                          # residual add 1
        b = self.R(self.norm(X, W[p + "post_norm"]))
        m = self.R(F.silu(F.linear(b, W[p + "w_gate"])) * F.linear(b, W[p + "w_up"]))
        return self.R(X + F.linear(m, W[p + "w_down"]))                  # residual add 2

    def draft(self, k_ctx, v_ctx, C, anchor):
        """k_ctx/v_ctx: per layer float64 [>= C, n_kv, d]. Returns (logits [B-1, V], tokens)."""
        c, W = self.c, self.W
        ids = torch.tensor([int(anchor)] + [c.mask_token_id] * (c.block_size - 1))
        X = W["embed"][ids]
        for l in range(c.n_layers):
            X = self.layer(l, X, k_ctx[l], v_ctx[l], C)
        z = self.R(self.norm(X[1:], W["norm"]))
        logits = F.linear(z, W["lm_head"])
        return logits, torch.argmax(logits, dim=-1)      # first maximum on a tie

    def round(self, taps, C, k_old, v_old, anchor):
        """Fuse and inject the R new rows at C-R..C-1 over the existing rows, then draft."""
        f = self.fuse(taps)
        R = f.shape[0]
        ks, vs = [], []
        for l in range(self.c.n_layers):
            k, v = self.context_kv(f, torch.arange(C - R, C), l)
            ks.append(torch.cat([t64(k_old[l])[:C - R], k]))
            vs.append(torch.cat([t64(v_old[l])[:C - R], v]))
        logits, toks = self.draft(ks, vs, C, anchor)
        return f, ks, vs, logits, toks


def verify(draft, target):
    """Greedy acceptance of one stream: matches of d_j against t_{j-1}, counted up to
    the first mismatch; the token after them is the target's."""
    d = torch.as_tensor(draft)
    t = torch.as_tensor(target)
    a = int(torch.cumprod((d == t[:-1]).to(torch.int64), 0).sum())
    return a, int(t[a])
