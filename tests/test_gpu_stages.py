"""Stage-by-stage parity at full size: every step of the GPU's draft checked on exactly
the inputs it read.

The library's stage trace copies every tensor a draft stores (each layer's input
stream, a, q, block k and v, o, the stream after residual add 1, b, m; the last
stream and the final-normed mask rows). For every stream and layer the oracle then
computes each step from the GPU's own stored inputs (draft_layer with `given`), and
the step's result is compared with what the GPU stored:

  * no element may differ by more than 1 bf16 ulp plus 2^-16 of its row's RMS (the
    same bar as the fused rows and K/V: fp32 sums carry an absolute error of order
    sqrt(K) 2^-24 times the row scale, which elements near zero cannot absorb in one
    ulp of their own);
  * at most 1e-3 of a step's elements may differ at all (a one-ulp rounding flip):
    fp32 sums place a value on the other side of a bf16 rounding boundary only when it
    lies within their error of it, while a wrong operand, index or missing term moves
    most elements;
  * the logits of the GPU's own final-normed rows: within 1e-4 of the float64 product
    (fp32 sums over hidden terms), and the drafted token equal to the float64 argmax
    wherever its top-2 gap exceeds 1e-4.

Streams: all of them, at the 9B ctx-4096, 9B 32k-span, DFlash2-shaped 16-stream and
long-context 4-stream workloads (through the C-ABI, the launch configuration the
benchmark times).
"""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import dflash_oracle as O
from workloads.round_case import RoundCase, to_np

pytestmark = pytest.mark.gpu

FLIP_CEILING = 1e-3
LOGIT_BAR = 1e-4
STEPS = ("a", "q", "k", "v", "o", "x_attn", "b", "m", "x_out")


def log(msg):
    print(msg, flush=True)


def ulp_bf16(x):
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.exp2(e - 7), 2.0 ** -133)


class Window:
    """Cache rows [lo, C) of one stream and layer, indexed by absolute position."""

    def __init__(self, rows, lo):
        self.rows, self.lo = rows, lo

    def __getitem__(self, sl):
        assert sl.start >= self.lo, (sl, self.lo)
        return self.rows[sl.start - self.lo:sl.stop - self.lo]


def read_trace(case, buf):
    p, S, B = case.p, case.p.n_streams, case.p.block_size
    M, Mm, H, I = S * B, S * (B - 1), p.hidden, p.intermediate
    nq, nkv, d = p.n_q_heads * p.head_dim, p.n_kv_heads, p.head_dim
    es = 4 if p.dtype == "f32" else 2
    flat = O.as_f64(to_np(buf.view(torch.float32 if es == 4 else torch.bfloat16)))
    sizes = [("x_in", (M, H)), ("a", (M, H)), ("q", (M, nq)), ("kblk", (S, nkv, 32, d)), ("vblk", (S, nkv, d, 32)),
             ("o", (M, nq)), ("x_attn", (M, H)), ("b", (M, H)), ("m", (M, I))]
    off = 0
    layers = []
    for _ in range(p.n_layers):
        rec = {}
        for name, shp in sizes:
            n = int(np.prod(shp))
            rec[name] = flat[off:off + n].reshape(shp)
            off += n
        layers.append(rec)
    x_last = flat[off:off + M * H].reshape(M, H)
    off += M * H
    z = flat[off:off + Mm * H].reshape(Mm, H)
    assert off + Mm * H == flat.size
    return layers, x_last, z


def compare_step(gpu, orc, what, stats, dtype):
    g, o = np.asarray(gpu, np.float64), np.asarray(orc, np.float64)
    assert g.shape == o.shape, (what, g.shape, o.shape)
    diff = np.abs(g - o)
    if dtype == "bf16":
        rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True))
        bad = int(np.sum(diff > ulp_bf16(o) + 2.0 ** -16 * rms))
        off = int(np.sum(diff > 0))
    else:   # fp32 storage: the fp32 bar of the fused rows, no flip count
        bad = int(np.sum(diff > 2e-5 * np.abs(o) + 2e-6))
        off = 0
    st = stats.setdefault(what, [0, 0, 0])
    st[0] += off
    st[1] += bad
    st[2] += g.size


def run_stages(preset, streams=None, q4=False):
    p = wl.preset(preset)
    case = RoundCase(p, q4=q4)
    S, B = p.n_streams, p.block_size
    buf = torch.zeros(case.dr.trace_bytes(S), dtype=torch.uint8, device="cuda")
    case.dr.set_trace(buf)
    case.run_gpu()
    case.dr.set_trace(None)
    torch.cuda.synchronize()
    layers, x_last, z_gpu = read_trace(case, buf)
    logits_gpu = case.logits.cpu().numpy().astype(np.float64)
    toks_gpu = case.draft.cpu().numpy()
    W = case.weights_np()
    if q4:       # the oracle's steps on the dequantized 4-bit weights
        W = O.quantized_weights(p, {k: O.as_f64(v) for k, v in W.items()})
    d, nq, nkv = p.head_dim, p.n_q_heads, p.n_kv_heads
    stats = {}
    worst_logit = 0.0
    streams = range(S) if streams is None else streams
    log(f"[stages] {p.name}: streams {list(streams)}, ctx {case.ctx}")
    for l in range(p.n_layers):
        Wl = dict(W)
        for t in wl.LAYER_TENSORS:                 # float64 once per layer
            Wl[f"layers.{l}.{t}"] = O.as_f64(W[f"layers.{l}.{t}"])
        for s in streams:
            C = case.ctx[s]
            lo, _ = O.context_reach(C, p.layer_window[l])
            kc, vc = case.kv.read_rows(l, s, lo, C - lo)
            kwin, vwin = Window(O.as_f64(to_np(kc)), lo), Window(O.as_f64(to_np(vc)), lo)
            rows = slice(s * B, (s + 1) * B)
            L = layers[l]
            given = dict(a=L["a"][rows], q=L["q"][rows].reshape(B, nq, d),
                         k=L["kblk"][s, :, :B, :].transpose(1, 0, 2),
                         v=L["vblk"][s, :, :, :B].transpose(2, 0, 1),
                         o=L["o"][rows], x_attn=L["x_attn"][rows], b=L["b"][rows], m=L["m"][rows])
            tr = {}
            O.draft_layer(p, l, L["x_in"][rows], Wl, kwin, vwin, C, trace=tr, given=given)
            own = tr["layers"][0]
            for name in ("a", "q", "k", "v", "o", "x_attn", "b", "m"):
                compare_step(given[name], own[name], name, stats, p.dtype)
            nxt = layers[l + 1]["x_in"][rows] if l + 1 < p.n_layers else x_last[rows]
            sel = slice(0, B) if l + 1 < p.n_layers else slice(1, B)   # the last add updates mask rows only
            compare_step(nxt[sel], own["x_out"][sel], "x_out", stats, p.dtype)
        del Wl
    lm = O.as_f64(W["lm_head"])
    for s in streams:
        rows = slice(s * B + 1, (s + 1) * B)
        zs = z_gpu[s * (B - 1):(s + 1) * (B - 1)]
        z_own = O.round_to(O.rms_norm(x_last[rows], O.as_f64(W["norm"]), p.rms_eps), p.dtype)
        compare_step(zs, z_own, "z", stats, p.dtype)
        ref = zs @ lm.T
        dl = float(np.max(np.abs(ref - logits_gpu[s])))
        worst_logit = max(worst_logit, dl)
        srt = np.sort(ref, axis=-1)
        sure = (srt[:, -1] - srt[:, -2]) > LOGIT_BAR
        assert np.array_equal(toks_gpu[s][sure], O.argmax_lowest(ref)[sure]), f"stream {s}: tokens"
    problems = []
    for name in STEPS + ("z",):
        off, bad, n = stats[name]
        log(f"[stages] {p.name} {name:7s}: {n:10d} elements, {off:7d} differ ({off / n:.2e}), {bad} past the bar")
        if bad:
            problems.append(f"{name}: {bad} elements past 1 ulp + 2^-16 rms")
        if off > FLIP_CEILING * n:
            problems.append(f"{name}: {off / n:.2e} of elements differ (ceiling {FLIP_CEILING:g})")
    log(f"[stages] {p.name} logits from the GPU's z: max-abs {worst_logit:.3g} (bar {LOGIT_BAR:g})")
    if worst_logit > LOGIT_BAR:
        problems.append(f"logits {worst_logit:.3g} > {LOGIT_BAR:g}")
    assert not problems, "; ".join(problems)


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_stages_tiny_f32():
    run_stages("tiny_f32")


@pytest.mark.parametrize("preset", ["9b_ctx4k", "9b_ctx32k", "dflash2_x16", "9b_long_x4"])
def test_every_step_on_identical_inputs(preset):
    run_stages(preset)
