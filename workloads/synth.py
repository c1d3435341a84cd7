"""Seeded synthetic inputs for the draft round.

Every tensor is drawn from its own torch.Generator, seeded from the preset's
seed and the tensor's index, so any tensor can be regenerated on its own.
Distributions: weight matrices 0.02 * N(0, 1); RMSNorm gains 1 + 0.02 * N(0, 1);
tap planes (the round's and the context's) and pre-written context K/V N(0, 1);
all cast to the preset's dtype (bf16 by round-to-nearest-even, or fp32). Nothing
here computes any part of the round: drafted tokens enter make_target_rows only
as given values.
"""
import numpy as np
import torch

LAYER_TENSORS = ["in_norm", "wq", "wk", "wv", "wo", "q_norm", "k_norm",
                 "post_norm", "w_gate", "w_up", "w_down"]
GLOBAL_TENSORS = ["fc", "hidden_norm", "norm"]
SHARED_TENSORS = ["embed", "lm_head"]   # taken from the target, frozen


def _torch_dtype(p):
    return torch.float32 if p.dtype == "f32" else torch.bfloat16


def tensor_names(p, include_shared=True):
    names = (list(SHARED_TENSORS) if include_shared else []) + list(GLOBAL_TENSORS)
    for l in range(p.n_layers):
        names += [f"layers.{l}.{t}" for t in LAYER_TENSORS]
    return names


def tensor_shape(p, name):
    h, d, I = p.hidden, p.head_dim, p.intermediate
    nq, nkv = p.n_q_heads * d, p.n_kv_heads * d
    if name in ("embed", "lm_head"):
        return (p.vocab, h)
    if name == "fc":
        return (h, p.n_taps * h)
    if name in ("hidden_norm", "norm"):
        return (h,)
    t = name.split(".")[-1]
    return {"in_norm": (h,), "post_norm": (h,), "wq": (nq, h), "wk": (nkv, h),
            "wv": (nkv, h), "wo": (h, nq), "q_norm": (d,), "k_norm": (d,),
            "w_gate": (I, h), "w_up": (I, h), "w_down": (h, I)}[t]


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFFFFFFFFFFFFFF)
    return g


def _randn(shape, device, seed, dtype, scale=1.0, offset=0.0):
    g = _gen(device, seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if scale != 1.0:
        x.mul_(scale)
    if offset != 0.0:
        x.add_(offset)
    return x.to(dtype)


def make_weights(p, device="cpu", seed=None, names=None):
    """All drafter tensors (plus the shared embed / lm_head) as a name -> tensor dict."""
    seed = p.seed if seed is None else seed
    dt = _torch_dtype(p)
    out = {}
    for i, name in enumerate(tensor_names(p)):
        if names is not None and name not in names:
            continue
        shape = tensor_shape(p, name)
        s = seed * 100003 + i * 7919 + 17
        if len(shape) == 1:   # RMSNorm gain
            out[name] = _randn(shape, device, s, dt, scale=0.02, offset=1.0)
        else:
            out[name] = _randn(shape, device, s, dt, scale=0.02)
    return out


def make_taps(p, n_rows, device="cpu", seed=None):
    """n_taps tap planes, each [n_rows, hidden], N(0, 1), in ascending tap order."""
    seed = (p.seed if seed is None else seed) * 31 + 5
    return [_randn((n_rows, p.hidden), device, seed * 1009 + t, _torch_dtype(p))
            for t in range(p.n_taps)]


def make_context_taps(p, stream, n_rows, device="cpu", seed=None):
    """Tap planes of stream `stream`'s existing context rows (positions 0..n_rows-1),
    n_taps planes [n_rows, hidden], N(0, 1), drawn apart from the round's own taps."""
    seed = (p.seed if seed is None else seed) * 37 + 11
    return [_randn((n_rows, p.hidden), device, (seed * 1009 + stream) * 131 + t, _torch_dtype(p))
            for t in range(p.n_taps)]


def make_context_kv(p, layer, stream, n_pos, kind, device="cpu", seed=None, start=0):
    """Pre-written context K or V rows [n_pos, n_kv, head_dim], N(0, 1).

    Rows are drawn per 1024-position block so that any position range can be
    regenerated on its own; `start` must be a multiple of 1024.
    """
    assert kind in ("k", "v") and start % 1024 == 0
    seed = (p.seed if seed is None else seed) * 7 + 3
    dt = _torch_dtype(p)
    blocks = []
    pos = start
    end = start + n_pos
    while pos < end:
        blk = pos // 1024
        s = ((seed * 1000003 + layer) * 131 + stream) * 2 + (kind == "v")
        x = _randn((1024, p.n_kv_heads, p.head_dim), device, s * 65537 + blk, dt)
        lo = pos - blk * 1024
        hi = min(1024, end - blk * 1024)
        blocks.append(x[lo:hi])
        pos = blk * 1024 + hi
    if not blocks:
        return torch.empty((0, p.n_kv_heads, p.head_dim), dtype=dt, device=device)
    return torch.cat(blocks, 0)


def ctx_lens(p, seed=None):
    """Context length of each stream (tokens the draft block sees)."""
    seed = (p.seed if seed is None else seed) * 13 + 1
    spec = p.ctx_spec
    if isinstance(spec, int):
        return [spec] * p.n_streams
    if isinstance(spec, (list, tuple)) and spec and spec[0] == "uniform":
        rng = np.random.default_rng(seed)
        return [int(x) for x in rng.integers(spec[1], spec[2] + 1, size=p.n_streams)]
    return [int(x) for x in spec]


def draw_accept_lengths(p, seed=None):
    """Per-stream prefix length L for a synthetic target row.

    ("uniform",): L ~ U{0..B}; ("geometric", q): L ~ Geom on {0,1,...} with
    success probability q, clamped to B-1; ("full",): L = B-1.
    """
    seed = (p.seed if seed is None else seed) * 17 + 9
    rng = np.random.default_rng(seed)
    B = p.block_size
    kind = p.accept_spec[0]
    if kind == "uniform":
        return [int(x) for x in rng.integers(0, B + 1, size=p.n_streams)]
    if kind == "geometric":
        q = p.accept_spec[1]
        return [int(min(B - 1, x - 1)) for x in rng.geometric(q, size=p.n_streams)]
    return [B - 1] * p.n_streams


def round_rows(p, seed=None):
    """Rows fused and injected in a round per stream: prior acceptance + 1."""
    return [min(a, p.block_size - 1) + 1 for a in draw_accept_lengths(p, (p.seed if seed is None else seed) + 77)]


def make_page_table(p, ctx, extra_tokens=0, permute=True, seed=None):
    """Page table [S, pages_per_stream] int32 and the pool size in pages.

    Each stream gets ceil((max ctx + extra) / page_size) pages; the pool is the
    sum, assigned by a seeded permutation (or in order).
    """
    seed = (p.seed if seed is None else seed) * 19 + 4
    ps = p.page_size
    span = max(ctx) + extra_tokens
    pages_per_stream = (span + ps - 1) // ps
    pool = pages_per_stream * len(ctx)
    ids = np.arange(pool, dtype=np.int64)
    if permute:
        ids = np.random.default_rng(seed).permutation(pool)
    table = ids.reshape(len(ctx), pages_per_stream).astype(np.int32)
    return table, pool


def make_anchor(p, seed=None):
    """Anchor token per stream, uniform over [0, vocab - 2] (the mask id is vocab - 1)."""
    seed = (p.seed if seed is None else seed) * 23 + 2
    rng = np.random.default_rng(seed)
    return rng.integers(0, p.vocab - 1, size=p.n_streams).astype(np.int32)


def make_target_rows(draft, prefix_len, vocab, seed):
    """Synthetic target argmax rows [S, B] agreeing with `draft` on a given prefix.

    For stream s with prefix length L: t[j-1] = d_j for j <= min(L, B-1); when
    L < B-1 the entry t[L] is forced to differ from d_{L+1}; all other entries
    are seeded uniform tokens.
    """
    draft = np.asarray(draft, dtype=np.int64)
    S, Bm1 = draft.shape
    rng = np.random.default_rng(seed)
    t = rng.integers(0, vocab, size=(S, Bm1 + 1)).astype(np.int64)
    for s in range(S):
        L = int(prefix_len[s])
        k = min(L, Bm1)
        t[s, :k] = draft[s, :k]
        if k < Bm1 and t[s, k] == draft[s, k]:
            t[s, k] = (draft[s, k] + 1 + rng.integers(0, vocab - 1)) % vocab
    return t.astype(np.int32)
