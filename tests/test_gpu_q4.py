"""4-bit drafter weights on the GPU (DFlash explainer, section 8; TensorFold #1851,
"Exactness", Precision), through the C-ABI.

  * the codes, scales and biases the library's quantizer writes are the oracle's
    quantizer's bit for bit (integer and bf16 decisions, taken in float64 on both sides),
    read back from the documented 4-bit packing;
  * rounds drafted with the 4-bit weights against the oracle run on the dequantized
    weights, with the bars of the bf16 rounds; and every step at the 9B shapes on
    identical inputs within 1 ulp (the stage test's bar);
  * calls the 4-bit path does not take (more than 32 rows) are refused.
"""
import numpy as np
import pytest
import torch

import block_diffusion_drafter_dflash_amd as D
import test_gpu_parity as GP
import test_gpu_stages as GS
import workloads as wl
from oracle import dflash_oracle as O
from workloads.presets import small_variant
from workloads.round_case import RoundCase, to_np

pytestmark = pytest.mark.gpu

GROUP, CHUNK = 64, 1024 + 128


def decode_q4(buf, N, K):
    """Codes [N, K], scale and bias [N, K / 64] (float64) of one matrix in the 4-bit
    packing: tile t, chunk c at (t * K/64 + c) * 1152 bytes; lane (lr, lg) holds 16 bytes
    at 16 (16 lg + lr): row lr then row 16 + lr, 8 bytes each, codes k = 16 lg .. +15,
    two a byte, low nibble first; then (scale, bias) bf16 pairs of rows lr, 16 + lr at
    1024 + 8 lr."""
    tiles, chunks = (N + 31) // 32, K // GROUP
    b = np.asarray(buf[:tiles * chunks * CHUNK], dtype=np.uint8).reshape(tiles, chunks, CHUNK)
    sb = np.ascontiguousarray(b[:, :, 1024:]).reshape(tiles, chunks, 16, 2, 4).view(np.uint16)   # [.., lr, nt, scale|bias]
    lanes = b[:, :, :1024].reshape(tiles, chunks, 4, 16, 2, 8)            # [tile, chunk, lg, lr, nt, byte]
    lo, hi = lanes & 0xF, lanes >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(tiles, chunks, 4, 16, 2, 16)  # code k = 16 lg + j
    # -> [tile, nt, lr, chunk, lg, j] = row 16 nt + lr, k = 64 chunk + 16 lg + j
    codes = nib.transpose(0, 4, 3, 1, 2, 5).reshape(tiles * 32, K)
    scale = O.bf16_bits_to_f64(sb[..., 0].transpose(0, 3, 2, 1).reshape(tiles * 32, chunks))
    bias = O.bf16_bits_to_f64(sb[..., 1].transpose(0, 3, 2, 1).reshape(tiles * 32, chunks))
    return codes[:N], scale[:N], bias[:N], codes[N:], scale[N:]


MID_Q4 = small_variant(GP.MID, name="mid_q4", vocab=1000, n_streams=2, ctx_spec=[300, 1030], seed=2301)


def test_quantized_codes_equal_the_oracle_quantizer():
    case = RoundCase(MID_Q4, q4=True)
    p = case.p
    buf = to_np(case.dr._packed)
    W = case.weights_np()
    h, nq, nkv, I = p.hidden, p.n_q_heads * p.head_dim, p.n_kv_heads * p.head_dim, p.intermediate
    off = 0

    def take(N, K):
        nonlocal off
        n = (N + 31) // 32 * (K // GROUP) * CHUNK
        seg = buf[off:off + n]
        off += (n + 255) // 256 * 256
        return decode_q4(seg, N, K)

    def check(name, got, w):
        q, s, b = O.quantize_affine(w)
        gq, gs, gb, pad_q, pad_s = got
        assert np.array_equal(gq, q), f"{name}: codes"
        assert np.array_equal(gs, s), f"{name}: scales"
        assert np.array_equal(gb, b), f"{name}: biases"
        assert not pad_q.any() and not pad_s.any(), f"{name}: padding rows"

    check("fc", take(h, p.n_taps * h), W["fc"])
    check("lm_head", take(p.vocab, h), W["lm_head"])          # 1000 rows: a ragged last tile
    for l in range(p.n_layers):
        L = f"layers.{l}."
        check(f"{L}qkv", take(nq + 2 * nkv, h), np.concatenate([W[L + "wq"], W[L + "wk"], W[L + "wv"]]))
        check(f"{L}wo", take(h, nq), W[L + "wo"])
        gu = take(2 * I, h)
        # tile t: gate rows 16 t .. 16 t + 15, then the matching up rows
        order = np.concatenate([np.r_[16 * t:16 * t + 16, I + 16 * t:I + 16 * t + 16] for t in range(I // 16)])
        check(f"{L}gate_up", gu, np.concatenate([W[L + "w_gate"], W[L + "w_up"]])[order])
        check(f"{L}w_down", take(h, I), W[L + "w_down"])


def run_q4_round(case, streams, conditioning=False):
    case.run_gpu()
    Wq = O.quantized_weights(case.p, {k: O.as_f64(v) for k, v in case.weights_np().items()})
    orc = O.run_round(case.p, Wq, case.oracle_streams(streams))
    tol = None
    if conditioning:
        import conditioning as CD
        base = [o["logits"] for o in orc]
        pert = CD.with_flips(lambda: O.run_round(case.p, Wq, case.oracle_streams(streams)), CD.RATE, 12345)
        mx, _ = CD.movement(base, [o["logits"] for o in pert])
        tol = max(2e-2, CD.FACTOR * mx)
    return GP.compare_round(case, streams, orc, tol)


def test_q4_round_parity_mid_two_streams():
    # 32 block rows (the skinny GEMMs), ragged LM head, sliding and full layers
    run_q4_round(RoundCase(MID_Q4, q4=True), [0, 1])


def test_q4_round_parity_9b_ctx4k():
    run_q4_round(RoundCase(wl.preset("9b_ctx4k"), q4=True), [0], conditioning=True)


def test_q4_every_step_on_identical_inputs_9b_ctx4k():
    GS.run_stages("9b_ctx4k", q4=True)


def test_q4_refuses_the_tiled_batch_sizes():
    case = RoundCase(GP.MID, q4=True)           # 4 streams x 16 = 64 block rows
    with pytest.raises(D.DFlashError) as e:
        case.draft_block()
    assert e.value.code == -7 and "4-bit" in str(e.value)
    one = small_variant(GP.MID, n_streams=1, ctx_spec=[300])
    prompt = RoundCase(one, ctx=[300], rows=[40], q4=True)      # a 40-row fuse and inject
    for call in (prompt.fuse, prompt.inject):
        with pytest.raises(D.DFlashError) as e:
            call()
        assert e.value.code == -7 and "4-bit" in str(e.value)
    small = RoundCase(one, ctx=[300], rows=[32], q4=True)       # 32 rows and 16 block rows: taken
    small.run_gpu()
    assert torch.isfinite(small.logits).all()
