"""CPU oracle of the DFlash block-diffusion draft round. TEST INFRASTRUCTURE ONLY.

Only the test suite, the package entry's smoke check and the benchmark's CPU
baseline leg may import this module. The product path (the HIP library and
its Python binding) never imports, calls or links anything here, and this
module imports nothing from the product path.

What it computes (sources are the four pages on DFlash):
  * fuse:   fc over the concatenated tap planes, then the hidden_norm RMSNorm,
            one fused context row per token (TensorFold pull request #1851,
            "What this changes", items 3 and 4; DFlash explainer, section 3,
            "Target knows best").
  * inject: the fused rows projected to k and v only, written into every draft
            layer's cache (TensorFold #1851, item 4; explainer section 3,
            "KV injection into every layer").
  * draft:  one non-causal forward of a qwen3 body over an anchor plus B-1 mask
            rows: eleven tensors a layer, two residual adds a layer, final norm;
            sliding layers see only their own window of the context, the full
            layer sees all of it (TensorFold #1851, items 1 and 4; explainer
            section 3, "Block diffusion parallel drafting"); then the shared
            LM head and an independent top-1 at every mask row (explainer
            section 5, "Candidate path selector", which states that the
            original DFlash picks top-1 at each position independently).
  * verify: greedy acceptance of the longest prefix equal to the target's
            argmax, plus the target's token at the first mismatch (explainer
            section 4, "Greedy decoding"; "Port the DFlash2 protocol, not its
            checkpoint", "What is portable" and "Golden replay before
            training").
  * sampling: inverse-CDF draws from tempered softmax rows, and speculative-
            sampling acceptance with the residual max(p_target - p_draft, 0)
            (explainer section 4, "Sampling decoding").
  * selector: DFlash2's candidate path over the top-k tokens of each drafted
            position, with rank-r pair scores and a min-p stop (explainer section 5;
            TensorFold #1851 item 1; Strata #3457, "Problem and result").
  * 4-bit weights: affine quantization in groups of 64 along each weight row,
            and the dequantized weights used exactly (explainer section 8; TensorFold
            #1851, "Exactness", Precision).

Numerics: every product and reduction is float64. Values are rounded to the
activation dtype (bf16 by round-to-nearest-even straight from float64, or
fp32) only at the points the round stores a tensor:
  R1 fused row, R2 context K/V, R3 normed layer input, R4 q/k/v of the block,
  R5 attention output, R6 residual after attention, R7 SwiGLU product,
  R8 residual after the MLP, R9 final-normed mask rows.
Logits stay float64. This follows the TensorFold page's "Exactness" list
(bf16 activations with fp32 sums) and the Strata page's "Validation" list
(a native drafter checked against an f64 host reference).

Readings taken where the pages are silent:
  taps concatenated in ascending tap-id order; fc then hidden_norm; RMSNorm is
  x / sqrt(mean(x^2) + eps) * g; no biases; the eleven layer tensors are
  in_norm, wq, wk, wv, wo, q_norm, k_norm, post_norm, w_gate, w_up, w_down;
  context K/V use the layer's own wk/wv (+ k_norm, RoPE) on the fused row with
  no input norm; context rows sit at positions 0..C-1, the anchor at C and mask
  row j at C+j; rotate-half RoPE over the whole head; a sliding layer with
  window W sees context rows [max(0, C-W), C) plus all B block rows; q head h
  reads kv head h // (n_q / n_kv); scale 1/sqrt(head_dim); mask row j predicts
  the token at position C+j; argmax ties go to the lowest index; sampling
  accepts d when u * p_draft(d) < p_target(d), draws by inverse CDF over token
  ids in ascending order with one uniform per draw, and falls back to the
  target's distribution when the residual has no mass; a 4-bit group's bias is its
  smallest weight and its scale (max - min) / 15 rounded once to bf16, codes round to
  nearest even, and the LM head and fc are quantized with the layers (the embedding is
  not).
"""
import math

import numpy as np

# --------------------------------------------------------------------------
# Storage formats


def bf16_bits_to_f64(u):
    """Decode bf16 bit patterns (uint16) to float64 values, exactly."""
    u = np.asarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def as_f64(a):
    """Tensor storage (uint16 bf16 bits, float32, or float64) -> float64."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64, copy=False)


_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_bf16(x):
    """Round float64 values to the nearest bf16 value, ties to even.

    bf16 keeps 8 significant bits: a finite value with frexp exponent e lies on
    the grid k * 2**(e-8); the grid never gets finer than the subnormal step
    2**-133. Rounding happens once, straight from float64.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.maximum(e - 8, -133)
    y = np.ldexp(np.rint(np.ldexp(x, -q)), q)
    y = np.where(np.abs(y) > _BF16_MAX, np.copysign(np.inf, x), y)
    return np.where(np.isfinite(x), y, x)


def round_f32(x):
    """Round float64 values to the nearest fp32 value (IEEE cast, ties to even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_to(x, dtype):
    """Round to the activation dtype: "bf16", "f32", or "f64" (no rounding; pins only)."""
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return round_f32(x)
    assert dtype == "f64", dtype
    return np.asarray(x, dtype=np.float64)


def bf16_bits(x):
    """bf16 bit patterns of float64 values that are already bf16-representable."""
    return (np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


# --------------------------------------------------------------------------
# Building blocks


def rms_norm(x, g, eps):
    """x / sqrt(mean(x^2) + eps) * g over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def rope(x, pos, theta):
    """Rotate-half rotary embedding over the last axis (length d).

    Pair (i, i + d/2) turns by the angle pos * theta**(-2i/d).
    `pos` has the shape of x without its last axis, or broadcasts to it.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    inv_freq = float(theta) ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(x):
    return x / (1.0 + np.exp(-x))


def softmax(s):
    s = s - np.max(s, axis=-1, keepdims=True)
    e = np.exp(s)
    return e / np.sum(e, axis=-1, keepdims=True)


def linear(x, w):
    """x [.., K] times w [N, K] transposed -> [.., N] (w in storage format)."""
    return np.asarray(x, dtype=np.float64) @ as_f64(w).T


# --------------------------------------------------------------------------
# Step 1: tap fusion (fc, then hidden_norm)


def fuse_taps(cfg, taps, W):
    """Fused context rows [R, hidden], rounded (R1).

    taps: list of n_taps planes [R, hidden] in ascending tap-id order.
    """
    x = np.concatenate([as_f64(t) for t in taps], axis=-1)        # [R, n*h]
    y = linear(x, W["fc"])                                        # [R, h]
    return round_to(rms_norm(y, as_f64(W["hidden_norm"]), cfg.rms_eps), cfg.dtype)


# --------------------------------------------------------------------------
# Step 2: context K/V injection (k and v only)


def inject_kv(cfg, fused, pos, W):
    """Per layer (K, V), each [R, n_kv, head_dim], rounded (R2).

    K = RoPE_pos(k_norm(wk . f)) per kv head; V = wv . f. The fused row enters
    without the layer's input norm.
    """
    f = as_f64(fused)
    R = f.shape[0]
    nkv, d = cfg.n_kv_heads, cfg.head_dim
    pos = np.asarray(pos, dtype=np.float64)
    out = []
    for l in range(cfg.n_layers):
        pre = f"layers.{l}."
        k = linear(f, W[pre + "wk"]).reshape(R, nkv, d)
        k = rms_norm(k, as_f64(W[pre + "k_norm"]), cfg.rms_eps)
        k = rope(k, pos[:, None], cfg.rope_theta)
        v = linear(f, W[pre + "wv"]).reshape(R, nkv, d)
        out.append((round_to(k, cfg.dtype), round_to(v, cfg.dtype)))
    return out


# --------------------------------------------------------------------------
# Step 3: the non-causal block forward


def block_attention(q, keys, values, n_kv):
    """Non-causal attention of every block query over the same key set.

    q [B, n_q, d]; keys/values [N, n_kv, d]. q head h reads kv head h // g.
    """
    B, nq, d = q.shape
    g = nq // n_kv
    o = np.empty_like(q)
    scale = 1.0 / math.sqrt(d)
    for h in range(nq):
        kvh = h // g
        s = (q[:, h, :] @ keys[:, kvh, :].T) * scale                 # [B, N]
        o[:, h, :] = softmax(s) @ values[:, kvh, :]
    return o


def context_reach(C, window):
    """Context positions [lo, C) a layer attends: all for window 0, else the last W."""
    return (0 if window == 0 else max(0, C - window)), C


def draft_layer(cfg, l, X, W, k_ctx, v_ctx, C, trace=None, given=None):
    """One qwen3 layer over the block rows X [B, h] (two residual adds).

    `given` (parity tests only): stored tensors of another implementation of this
    layer (any of a, q, k, v, o, x_attn, b, m; q [B, n_q, d], k and v [B, n_kv, d],
    the others [B, width]). A step whose input is given reads it instead of this
    function's own previous step, so every step is computed on exactly the inputs the
    other implementation used; the trace still records this function's own results.
    """
    pre = f"layers.{l}."
    dt, eps = cfg.dtype, cfg.rms_eps
    B = X.shape[0]
    nq, nkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    pos = C + np.arange(B)
    g = {} if given is None else given
    use = lambda name, own: as_f64(g[name]) if name in g else own

    a = round_to(rms_norm(X, as_f64(W[pre + "in_norm"]), eps), dt)                    # R3
    a_in = use("a", a)
    q = rms_norm(linear(a_in, W[pre + "wq"]).reshape(B, nq, d), as_f64(W[pre + "q_norm"]), eps)
    k = rms_norm(linear(a_in, W[pre + "wk"]).reshape(B, nkv, d), as_f64(W[pre + "k_norm"]), eps)
    v = linear(a_in, W[pre + "wv"]).reshape(B, nkv, d)
    q = round_to(rope(q, pos[:, None], cfg.rope_theta), dt)                           # R4
    k = round_to(rope(k, pos[:, None], cfg.rope_theta), dt)
    v = round_to(v, dt)

    lo, hi = context_reach(C, cfg.layer_window[l])
    keys = np.concatenate([as_f64(k_ctx[lo:hi]), use("k", k)], axis=0)
    vals = np.concatenate([as_f64(v_ctx[lo:hi]), use("v", v)], axis=0)
    o = round_to(block_attention(use("q", q), keys, vals, nkv).reshape(B, nq * d), dt)  # R5

    X1 = round_to(X + linear(use("o", o), W[pre + "wo"]), dt)                         # R6: add #1
    X1_in = use("x_attn", X1)
    b = round_to(rms_norm(X1_in, as_f64(W[pre + "post_norm"]), eps), dt)              # R3
    b_in = use("b", b)
    m = round_to(silu(linear(b_in, W[pre + "w_gate"])) * linear(b_in, W[pre + "w_up"]), dt)  # R7
    X2 = round_to(X1_in + linear(use("m", m), W[pre + "w_down"]), dt)                 # R8: add #2
    if trace is not None:
        trace.setdefault("layers", []).append(
            dict(a=a, q=q, k=k, v=v, o=o, x_attn=X1, b=b, m=m, x_out=X2, reach=(lo, hi)))
    return X2


def lm_head_logits(z, lm_head, chunk=16384):
    """Logits z . lm_head^T in float64, computed over vocab chunks."""
    V = lm_head.shape[0]
    out = np.empty((z.shape[0], V), dtype=np.float64)
    for c0 in range(0, V, chunk):
        c1 = min(V, c0 + chunk)
        out[:, c0:c1] = z @ as_f64(lm_head[c0:c1]).T
    return out


def argmax_lowest(logits):
    """Index of the maximum of each row; on a tie the lowest index wins."""
    logits = np.asarray(logits)
    assert np.all(np.isfinite(logits)), "oracle expects finite logits"
    return np.argmax(logits, axis=-1).astype(np.int64)   # numpy returns the first maximum


def draft_stream(cfg, W, k_ctx, v_ctx, C, anchor, trace=None):
    """Draft one block for one stream.

    k_ctx/v_ctx: per layer, context rows [>= C, n_kv, d] (positions 0..C-1).
    Returns (logits [B-1, V] float64, tokens [B-1]).
    """
    B = cfg.block_size
    toks = np.full(B, cfg.mask_token_id, dtype=np.int64)
    toks[0] = int(anchor)
    X = as_f64(W["embed"][toks])                                                       # [B, h]
    if trace is not None:
        trace["x0"] = X
    for l in range(cfg.n_layers):
        X = draft_layer(cfg, l, X, W, k_ctx[l], v_ctx[l], C, trace)
    z = round_to(rms_norm(X[1:], as_f64(W["norm"]), cfg.rms_eps), cfg.dtype)         # R9
    logits = lm_head_logits(z, W["lm_head"])
    if trace is not None:
        trace["z"] = z
    return logits, argmax_lowest(logits)


def top2(logits):
    """Largest and second-largest value of each row (float64)."""
    srt = np.sort(logits, axis=-1)
    return srt[..., -1], srt[..., -2]


# --------------------------------------------------------------------------
# Step 4: greedy verify


def verify_greedy(draft, target):
    """Greedy acceptance per stream.

    draft [S, B-1] holds d_1..d_{B-1}; target [S, B] holds t_0..t_{B-1}, the
    target's argmax after the anchor and after each drafted token. The
    accepted length a is the number of leading j with d_j = t_{j-1}; the bonus
    token is t_a; committed = d_1..d_a, t_a, padded with -1 to length B.
    """
    draft = np.asarray(draft, dtype=np.int64)
    target = np.asarray(target, dtype=np.int64)
    S, Bm1 = draft.shape
    accept = np.zeros(S, dtype=np.int64)
    bonus = np.zeros(S, dtype=np.int64)
    committed = np.full((S, Bm1 + 1), -1, dtype=np.int64)
    for s in range(S):
        a = 0
        while a < Bm1 and draft[s, a] == target[s, a]:
            a += 1
        accept[s] = a
        bonus[s] = target[s, a]
        committed[s, :a] = draft[s, :a]
        committed[s, a] = target[s, a]
    return accept, bonus, committed


# --------------------------------------------------------------------------
# Sampling (DFlash explainer, section 4, "Sampling decoding"): the standard
# speculative-sampling rule the page names, with its residual distribution.


def tempered_probs(logits, T):
    """softmax(logits / T) over the last axis, float64 (T > 0)."""
    return softmax(np.asarray(logits, dtype=np.float64) / float(T))


def sample_index(p, u):
    """Inverse-CDF draw from the weights p (not necessarily normalised) with one
    uniform u in [0, 1): the smallest k with p_0 + ... + p_k > u * sum(p). A
    zero weight is never drawn."""
    p = np.asarray(p, dtype=np.float64)
    c = np.cumsum(p)
    k = int(np.searchsorted(c, u * c[-1], side="right"))
    if k >= len(p):                      # u * sum landed on the total: the last nonzero weight
        k = int(np.flatnonzero(p > 0)[-1])
    return k


def verify_sampling(draft, draft_logits, target_logits, T, u_accept, u_sample):
    """Speculative-sampling acceptance per stream.

    draft [S, B-1]: d_1..d_{B-1}, drawn from the draft's tempered distributions
    p_j = softmax(draft_logits[s, j-1] / T); target_logits [S, B]: row i gives the
    target's distribution q_i = softmax(target_logits[s, i] / T) for the token
    after the anchor and d_1..d_i. Walking j = 1, 2, ..., d_j is accepted when
    u_accept[s, j-1] * p_j(d_j) < q_{j-1}(d_j) (probability min(1, q/p)). At the
    first rejection j the next token is drawn with u_sample[s] from the residual
    max(q_{j-1} - p_j, 0) (renormalised; q_{j-1} itself if that residual has no
    mass); when every d_j is accepted it is drawn from q_{B-1}. Returns the
    accepted length a, that token, and committed = d_1..d_a, token (-1 padded),
    as in verify_greedy.
    """
    draft = np.asarray(draft, dtype=np.int64)
    S, Bm1 = draft.shape
    accept = np.zeros(S, dtype=np.int64)
    token = np.zeros(S, dtype=np.int64)
    committed = np.full((S, Bm1 + 1), -1, dtype=np.int64)
    for s in range(S):
        a = 0
        nxt = None
        while a < Bm1:
            p = tempered_probs(draft_logits[s, a], T)
            q = tempered_probs(target_logits[s, a], T)
            d = draft[s, a]
            if u_accept[s, a] * p[d] < q[d]:
                a += 1
                continue
            r = np.maximum(q - p, 0.0)
            nxt = sample_index(r if r.sum() > 0 else q, u_sample[s])
            break
        if nxt is None:
            nxt = sample_index(tempered_probs(target_logits[s, Bm1], T), u_sample[s])
        accept[s] = a
        token[s] = nxt
        committed[s, :a] = draft[s, :a]
        committed[s, a] = nxt
    return accept, token, committed


# --------------------------------------------------------------------------
# DFlash2 candidate path selector (DFlash explainer, section 5, "Candidate path
# selector": top-k candidates at each position, a lightweight score of adjacent
# candidate pairs, one consistent path; the DFlash2 config's selector_top_k 16 and
# selector_rank 256; TensorFold #1851 item 1: with rank 0 the edge term is zero and
# the path comes from each position's marginals; Strata #3457, "Problem and result":
# --spec-min-p stops a draft where the selector's confidence falls below it).


def top_k_ordered(logits, k):
    """The k largest logits of a row, largest first, ties to the lowest index."""
    order = np.lexsort((np.arange(logits.shape[-1]), -np.asarray(logits, dtype=np.float64)))
    return order[:k]


def log_softmax(logits):
    x = np.asarray(logits, dtype=np.float64)
    m = np.max(x)
    return x - m - np.log(np.sum(np.exp(x - m)))


def select_path(logits, code_u, code_w, k, min_p):
    """One stream's path over its B-1 drafted positions.

    logits [B-1, V]; code_u, code_w [V, r] token codebooks (r may be 0). Position j
    keeps its top-k tokens c with node score log softmax(logits_j)(c); adjacent
    candidates (a at j, b at j+1) add the edge score <code_u[a], code_w[b]>. The path
    maximises the sum of node and edge scores (a tie goes to the earlier candidate,
    i.e. the larger logit, at the latest position first). The draft stops before the
    first position whose chosen token's probability is below min_p. Returns the tokens
    (-1 past the stop) and the draft length.
    """
    Bm1 = logits.shape[0]
    cand = [top_k_ordered(logits[j], k) for j in range(Bm1)]
    node = [log_softmax(logits[j])[cand[j]] for j in range(Bm1)]
    U = as_f64(code_u) if code_u is not None else None
    Wc = as_f64(code_w) if code_w is not None else None

    def edge(j):          # [k, k]: candidates of j against those of j + 1
        if U is None or U.shape[1] == 0:
            return np.zeros((k, k))
        return U[cand[j]] @ Wc[cand[j + 1]].T

    best = node[0].copy()
    back = []
    for j in range(1, Bm1):
        tot = best[:, None] + edge(j - 1)                  # [from, to]
        arg = np.argmax(tot, axis=0)                       # first maximum: the earlier candidate
        back.append(arg)
        best = tot[arg, np.arange(k)] + node[j]
    path = [int(np.argmax(best))]
    for arg in reversed(back):
        path.append(int(arg[path[-1]]))
    path.reverse()
    toks = np.array([cand[j][path[j]] for j in range(Bm1)], dtype=np.int64)
    probs = np.array([np.exp(node[j][path[j]]) for j in range(Bm1)])
    length = Bm1
    for j in range(Bm1):
        if probs[j] < min_p:
            length = j
            break
    toks[length:] = -1
    return toks, length


# --------------------------------------------------------------------------
# Storage closed forms (the prompt-memory planner and the fused ring)


def fused_row_bytes(hidden, elem_bytes=2):
    """One fused context row: a single hidden-wide plane."""
    return hidden * elem_bytes


def raw_tap_row_bytes(n_taps, hidden, elem_bytes=2):
    """One token's raw tap planes."""
    return n_taps * hidden * elem_bytes


def tap_row_bytes(n_taps, hidden, fusing, elem_bytes=2):
    """Planner price of a prompt row's taps.

    A fusing (v1) drafter holds its tap planes, their row-major copy, fc's
    output row and the fused row: (2n + 2) rows of hidden. A non-fusing
    drafter holds only its raw planes.
    """
    if fusing:
        return (2 * n_taps + 2) * hidden * elem_bytes
    return n_taps * hidden * elem_bytes


# --------------------------------------------------------------------------
# 4-bit drafter weights (DFlash explainer, section 8: the drafter's layers are
# quantized at load with 4 bits in groups of 64; TensorFold #1851, "Exactness",
# Precision: the drafter's 4-bit copies, with bf16 activations and fp32 sums)

QUANT_GROUP = 64
QUANT_BITS = 4


def quantized_names(cfg):
    """The weights a 4-bit drafter reads quantized: every GEMM weight (fc, the LM head,
    each layer's q/k/v/o and MLP projections); the embedding (a row gather) and the
    norm gains stay as they are."""
    names = ["fc", "lm_head"]
    for l in range(cfg.n_layers):
        names += [f"layers.{l}.{t}" for t in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")]
    return names


def quantize_affine(w, group=QUANT_GROUP, bits=QUANT_BITS):
    """Affine group quantization of a weight matrix [N, K] along K.

    For each run of `group` consecutive weights of a row: bias = the smallest weight,
    scale = (largest - smallest) / (2^bits - 1) rounded once to bf16, and each code =
    (w - bias) / scale rounded to the nearest integer (ties to even) and clamped to
    [0, 2^bits - 1], all in float64. A group whose weights are all equal (or whose
    scale rounds to zero) gets scale 0 and codes 0. Returns codes uint8 [N, K] and
    scale, bias float64 [N, K / group] (bf16 values).
    """
    w = as_f64(w)
    N, K = w.shape
    assert K % group == 0, (K, group)
    g = w.reshape(N, K // group, group)
    lo, hi = g.min(axis=-1), g.max(axis=-1)
    levels = (1 << bits) - 1
    scale = round_bf16((hi - lo) / levels)
    safe = np.where(scale > 0, scale, 1.0)[..., None]
    q = np.where(scale[..., None] > 0, np.rint((g - lo[..., None]) / safe), 0.0)
    q = np.clip(q, 0, levels).astype(np.uint8)
    return q.reshape(N, K), scale, lo


def dequantize_affine(q, scale, bias, group=QUANT_GROUP):
    """The weight each code stands for, bias + scale * code, in float64 (exact)."""
    N, K = q.shape
    g = q.reshape(N, K // group, group).astype(np.float64)
    return (bias[..., None] + scale[..., None] * g).reshape(N, K)


def quantized_weights(cfg, W):
    """W with every quantized weight replaced by its dequantized float64 values."""
    out = dict(W)
    for name in quantized_names(cfg):
        out[name] = dequantize_affine(*quantize_affine(W[name]))
    return out


# --------------------------------------------------------------------------
# A whole round for several streams (reference driver for the tests)


def context_from_taps(cfg, ctx_taps, W):
    """A stream's existing context built the way a round builds its new rows (steps 1
    and 2 above): the tap planes of its n context rows fused, then injected at
    positions 0..n-1. Returns per-layer lists k_ctx, v_ctx of [n, n_kv, head_dim]."""
    n = ctx_taps[0].shape[0]
    if n == 0:
        e = np.zeros((0, cfg.n_kv_heads, cfg.head_dim))
        return [e] * cfg.n_layers, [e] * cfg.n_layers
    kv = inject_kv(cfg, fuse_taps(cfg, ctx_taps, W), np.arange(n), W)
    return [k for k, _ in kv], [v for _, v in kv]


def run_round(cfg, W, streams, target_rows=None):
    """One round over several independent streams.

    streams: list of dicts with keys taps (list of [R, h] planes), C (context
    length the block sees after this round's injection), anchor, and the rows
    for positions 0..C-R-1 already in the cache: either k_ctx/v_ctx (per layer)
    or ctx_taps (their tap planes, built here by context_from_taps).
    The R new rows are fused and injected at positions C-R..C-1.
    Returns per-stream dicts with fused, kv (new rows), logits, tokens, and
    (when target_rows is given) accept, bonus, committed.
    """
    out = []
    for s, st in enumerate(streams):
        if "k_ctx" not in st:
            k_ctx, v_ctx = context_from_taps(cfg, st["ctx_taps"], W)
            st = dict(st, k_ctx=k_ctx, v_ctx=v_ctx)
        fused = fuse_taps(cfg, st["taps"], W)
        R = fused.shape[0]
        C = st["C"]
        pos = np.arange(C - R, C)
        kv = inject_kv(cfg, fused, pos, W)
        k_full = [np.concatenate([as_f64(st["k_ctx"][l][:C - R]), kv[l][0]], 0) for l in range(cfg.n_layers)]
        v_full = [np.concatenate([as_f64(st["v_ctx"][l][:C - R]), kv[l][1]], 0) for l in range(cfg.n_layers)]
        logits, toks = draft_stream(cfg, W, k_full, v_full, C, st["anchor"])
        out.append(dict(fused=fused, kv=kv, logits=logits, tokens=toks))
    if target_rows is not None:
        draft = np.stack([o["tokens"] for o in out])
        acc, bon, com = verify_greedy(draft, target_rows)
        for s, o in enumerate(out):
            o.update(accept=int(acc[s]), bonus=int(bon[s]), committed=com[s])
    return out
