"""Planted mistakes in the oracle: each must fail at least one pin.

Every case below edits one plausible mistake into a copy of the oracle's source (a
dropped term or rounding, a swapped operand, a wrong sign, index or reach), loads the
copy as a module of its own, and runs the CPU pins against it. A mistake that no pin
notices would mean that part of the oracle is unpinned. The real oracle is never
modified; the pins run against the copy by replacing the module each pin file uses.
"""
import os
import types

import pytest

import test_oracle_pins as P
import test_oracle_quant as PQ
import test_oracle_selector as PSel
import test_oracle_sampling as PS
import test_oracle_wiring as PW

ORACLE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "dflash_oracle.py")

# (name, text in the oracle, replacement); a case may plant several edits at once
MUTATIONS = [
    # layer wiring (TensorFold #1851 item 1: plain qwen3 body, two residual adds)
    ("in_norm and post_norm gains trade places",
     ['rms_norm(X, as_f64(W[pre + "in_norm"]), eps)', 'rms_norm(X1_in, as_f64(W[pre + "post_norm"]), eps)'],
     ['rms_norm(X, as_f64(W[pre + "post_norm"]), eps)', 'rms_norm(X1_in, as_f64(W[pre + "in_norm"]), eps)']),
    ("norm gains swapped: post_norm before attention",
     'rms_norm(X, as_f64(W[pre + "in_norm"]), eps)', 'rms_norm(X, as_f64(W[pre + "post_norm"]), eps)'),
    ("norm gains swapped: in_norm before the MLP",
     'rms_norm(X1_in, as_f64(W[pre + "post_norm"]), eps)', 'rms_norm(X1_in, as_f64(W[pre + "in_norm"]), eps)'),
    ("add 2 onto the layer input, dropping add 1 from the stream",
     'X2 = round_to(X1_in + linear(use("m", m), W[pre + "w_down"]), dt)',
     'X2 = round_to(X + linear(use("m", m), W[pre + "w_down"]), dt)'),
    ("add 1 dropped", 'X1 = round_to(X + linear(use("o", o), W[pre + "wo"]), dt)',
     'X1 = round_to(linear(use("o", o), W[pre + "wo"]), dt)'),
    ("add 2 dropped", 'X2 = round_to(X1_in + linear(use("m", m), W[pre + "w_down"]), dt)',
     'X2 = round_to(linear(use("m", m), W[pre + "w_down"]), dt)'),
    ("MLP normalises the layer input instead of add 1's sum",
     'b = round_to(rms_norm(X1_in,', 'b = round_to(rms_norm(X,'),
    ("SiLU on the up branch", 'silu(linear(b_in, W[pre + "w_gate"])) * linear(b_in, W[pre + "w_up"])',
     'linear(b_in, W[pre + "w_gate"]) * silu(linear(b_in, W[pre + "w_up"]))'),
    ("q normalised with k_norm's gain", 'as_f64(W[pre + "q_norm"]), eps)', 'as_f64(W[pre + "k_norm"]), eps)'),
    ("block values taken from wk", 'v = linear(a_in, W[pre + "wv"]).reshape(B, nkv, d)',
     'v = linear(a_in, W[pre + "wk"]).reshape(B, nkv, d)'),
    # storage points R1..R9
    ("R1 fused row not rounded", 'return round_to(rms_norm(y, as_f64(W["hidden_norm"]), cfg.rms_eps), cfg.dtype)',
     'return rms_norm(y, as_f64(W["hidden_norm"]), cfg.rms_eps)'),
    ("R2 context K not rounded", "out.append((round_to(k, cfg.dtype), round_to(v, cfg.dtype)))",
     "out.append((k, round_to(v, cfg.dtype)))"),
    ("R3 layer input not rounded", 'a = round_to(rms_norm(X, as_f64(W[pre + "in_norm"]), eps), dt)',
     'a = rms_norm(X, as_f64(W[pre + "in_norm"]), eps)'),
    ("R4 block v not rounded", "v = round_to(v, dt)", "v = v"),
    ("R5 attention output not rounded",
     'o = round_to(block_attention(use("q", q), keys, vals, nkv).reshape(B, nq * d), dt)',
     'o = block_attention(use("q", q), keys, vals, nkv).reshape(B, nq * d)'),
    ("R6 add 1 not rounded", 'X1 = round_to(X + linear(use("o", o), W[pre + "wo"]), dt)',
     'X1 = X + linear(use("o", o), W[pre + "wo"])'),
    ("R7 SwiGLU product not rounded",
     'm = round_to(silu(linear(b_in, W[pre + "w_gate"])) * linear(b_in, W[pre + "w_up"]), dt)',
     'm = silu(linear(b_in, W[pre + "w_gate"])) * linear(b_in, W[pre + "w_up"])'),
    ("R8 add 2 not rounded", 'X2 = round_to(X1_in + linear(use("m", m), W[pre + "w_down"]), dt)',
     'X2 = X1_in + linear(use("m", m), W[pre + "w_down"])'),
    ("R9 final-normed rows not rounded", 'z = round_to(rms_norm(X[1:], as_f64(W["norm"]), cfg.rms_eps), cfg.dtype)',
     'z = rms_norm(X[1:], as_f64(W["norm"]), cfg.rms_eps)'),
    ("bf16 rounding through an fp32 stage", "y = np.ldexp(np.rint(np.ldexp(x, -q)), q)",
     "y = np.ldexp(np.rint(np.ldexp(x.astype(np.float32).astype(np.float64), -q)), q)"),
    # fuse and inject (items 3-4; explainer section 3)
    ("taps concatenated in reverse order", "x = np.concatenate([as_f64(t) for t in taps], axis=-1)",
     "x = np.concatenate([as_f64(t) for t in taps[::-1]], axis=-1)"),
    ("hidden_norm before fc", 'y = linear(x, W["fc"])', 'y = linear(x / np.sqrt(np.mean(x * x, -1, keepdims=True)), W["fc"])'),
    ("inject applies the layer's input norm", "f = as_f64(fused)\n    R = f.shape[0]",
     "f = as_f64(fused)\n    R = f.shape[0]\n    f = rms_norm(f, as_f64(W['layers.0.in_norm']), cfg.rms_eps)"),
    ("inject skips k_norm", 'k = rms_norm(k, as_f64(W[pre + "k_norm"]), cfg.rms_eps)\n        k = rope',
     "k = k\n        k = rope"),
    # RoPE, attention, reach, positions
    ("RoPE turned the other way", "return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)",
     "return np.concatenate([x1 * c + x2 * s, x2 * c - x1 * s], axis=-1)"),
    ("RoPE frequencies over d/2", "inv_freq = float(theta) ** (-2.0 * np.arange(half, dtype=np.float64) / d)",
     "inv_freq = float(theta) ** (-2.0 * np.arange(half, dtype=np.float64) / half)"),
    ("GQA heads interleaved", "kvh = h // g", "kvh = h % n_kv"),
    ("attention scale 1/d", "scale = 1.0 / math.sqrt(d)", "scale = 1.0 / d"),
    ("sliding reach one row short", "return (0 if window == 0 else max(0, C - window)), C",
     "return (0 if window == 0 else max(0, C - window + 1)), C"),
    ("block rows one position early", "pos = C + np.arange(B)", "pos = C - 1 + np.arange(B)"),
    ("block keys left out",
     'keys = np.concatenate([as_f64(k_ctx[lo:hi]), use("k", k)], axis=0)\n    vals = np.concatenate([as_f64(v_ctx[lo:hi]), use("v", v)], axis=0)',
     "keys = as_f64(k_ctx[lo:hi]) if hi > lo else k\n    vals = as_f64(v_ctx[lo:hi]) if hi > lo else v"),
    # head and verify (explainer sections 4-5)
    ("logits from the rows before the masks", 'z = round_to(rms_norm(X[1:],', 'z = round_to(rms_norm(X[:-1],'),
    ("argmax takes the last maximum", "return np.argmax(logits, axis=-1).astype(np.int64)",
     "return (logits.shape[-1] - 1 - np.argmax(logits[..., ::-1], axis=-1)).astype(np.int64)"),
    ("verify compares d_j with t_j", "while a < Bm1 and draft[s, a] == target[s, a]:",
     "while a < Bm1 and draft[s, a] == target[s, a + 1]:"),
    ("bonus is the target's next token", "bonus[s] = target[s, a]", "bonus[s] = target[s, min(a + 1, Bm1)]"),
    # sampling (explainer section 4, "Sampling decoding")
    ("acceptance ratio inverted", "if u_accept[s, a] * p[d] < q[d]:", "if u_accept[s, a] * q[d] < p[d]:"),
    ("residual p - q", "r = np.maximum(q - p, 0.0)", "r = np.maximum(p - q, 0.0)"),
    ("no residual", "nxt = sample_index(r if r.sum() > 0 else q, u_sample[s])", "nxt = sample_index(q, u_sample[s])"),
    ("bonus from the target's first row", "nxt = sample_index(tempered_probs(target_logits[s, Bm1], T), u_sample[s])",
     "nxt = sample_index(tempered_probs(target_logits[s, 0], T), u_sample[s])"),
    # 4-bit weights (explainer section 8)
    ("4-bit scale over 16 levels", "scale = round_bf16((hi - lo) / levels)", "scale = round_bf16((hi - lo) / (levels + 1))"),
    ("4-bit bias is the group maximum", "return q.reshape(N, K), scale, lo", "return q.reshape(N, K), scale, hi"),
    ("4-bit codes truncated", "q = np.where(scale[..., None] > 0, np.rint((g - lo[..., None]) / safe), 0.0)",
     "q = np.where(scale[..., None] > 0, np.floor((g - lo[..., None]) / safe), 0.0)"),
    ("4-bit scale kept in float64", "scale = round_bf16((hi - lo) / levels)", "scale = (hi - lo) / levels"),
    ("4-bit dequantization drops the bias", "return (bias[..., None] + scale[..., None] * g).reshape(N, K)",
     "return (scale[..., None] * g).reshape(N, K)"),
    ("4-bit groups of 32", "QUANT_GROUP = 64", "QUANT_GROUP = 32"),
    # the DFlash2 candidate path selector (explainer section 5)
    ("selector pair score transposed", "return U[cand[j]] @ Wc[cand[j + 1]].T", "return Wc[cand[j]] @ U[cand[j + 1]].T"),
    ("selector candidates tie to the highest id",
     "order = np.lexsort((np.arange(logits.shape[-1]), -np.asarray(logits, dtype=np.float64)))",
     "order = np.lexsort((-np.arange(logits.shape[-1]), -np.asarray(logits, dtype=np.float64)))"),
    ("selector stops at or below min-p", "        if probs[j] < min_p:", "        if probs[j] <= min_p + 0.06:"),
    ("selector ignores the node scores", "        best = tot[arg, np.arange(k)] + node[j]", "        best = tot[arg, np.arange(k)]"),
    ("context from taps placed one position later", "fuse_taps(cfg, ctx_taps, W), np.arange(n), W)",
     "fuse_taps(cfg, ctx_taps, W), np.arange(1, n + 1), W)"),
    ("context from taps injected without fusing (first plane as the row)",
     "kv = inject_kv(cfg, fuse_taps(cfg, ctx_taps, W), np.arange(n), W)",
     "kv = inject_kv(cfg, as_f64(ctx_taps[0]), np.arange(n), W)"),
    ("storage sizes: planner counts one copy", "return (2 * n_taps + 2) * hidden * elem_bytes",
     "return (n_taps + 2) * hidden * elem_bytes"),
]


def load_mutant(old, new):
    src = open(ORACLE).read()
    olds, news = ([old], [new]) if isinstance(old, str) else (old, new)
    for o, n in zip(olds, news):
        assert src.count(o) == 1, f"the planted text must occur exactly once: {o!r}"
        src = src.replace(o, n)
    mod = types.ModuleType("dflash_oracle_mutant")
    mod.__file__ = ORACLE
    exec(compile(src, ORACLE + " (mutant)", "exec"), mod.__dict__)
    return mod


def pin_calls():
    """Every CPU pin of the oracle, with its parameters."""
    calls = []
    for mod in (P, PW, PS, PQ, PSel):
        for name in sorted(dir(mod)):
            fn = getattr(mod, name)
            if not name.startswith("test_") or not callable(fn):
                continue
            params = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
            if not params:
                calls.append((mod, name, {}))
                continue
            combos = [{}]
            for m in params:
                names = [n.strip() for n in m.args[0].split(",")] if isinstance(m.args[0], str) else list(m.args[0])
                nxt = []
                for c in combos:
                    for v in m.args[1]:
                        vals = v if len(names) > 1 else (v,)
                        nxt.append(dict(c, **dict(zip(names, vals))))
                combos = nxt
            calls += [(mod, name, c) for c in combos]
    return calls


def test_pins_pass_on_the_real_oracle_through_this_harness():
    # the harness itself: with the real oracle every pin it runs passes
    failed = [f"{m.__name__}.{n}{kw}" for m, n, kw in pin_calls() if not _passes(m, n, kw, None)]
    assert not failed, failed


def _passes(mod, name, kw, mutant):
    saved = mod.O
    if mutant is not None:
        mod.O = mutant
    try:
        getattr(mod, name)(**kw)
        return True
    except Exception:
        return False
    finally:
        mod.O = saved


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(name, old, new):
    mutant = load_mutant(old, new)
    for mod, fn, kw in pin_calls():
        if not _passes(mod, fn, kw, mutant):
            return                       # caught
    pytest.fail(f"no pin fails with the planted mistake: {name}")
