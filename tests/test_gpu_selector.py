"""The DFlash2 candidate path selector on the GPU against the oracle's, on identical
fp32 logits, through the C-ABI (DFlash explainer, section 5; TensorFold #1851 item 1;
Strata #3457, --spec-min-p).

Bars: draft lengths and tokens equal to the oracle's; where a path differs, both
sides' paths must score the same within 1e-9 (float64 sums in another order can only
split an exact tie). Rank 0 gives the round's own drafts.
"""
import numpy as np
import pytest
import torch

import block_diffusion_drafter_dflash_amd as D
import workloads as wl
from oracle import dflash_oracle as O
from workloads.presets import small_variant
from workloads.round_case import RoundCase, to_np

pytestmark = pytest.mark.gpu


def path_score(logits, U, W, toks, k):
    """Node plus pair scores of a token path (the oracle's terms, float64)."""
    sc = 0.0
    for j, t in enumerate(toks):
        sc += O.log_softmax(logits[j])[t]
        assert t in O.top_k_ordered(logits[j], k)
        if j + 1 < len(toks) and U is not None:
            sc += U[t] @ W[toks[j + 1]]
    return sc


def test_rank_zero_gives_the_rounds_drafts():
    case = RoundCase(wl.preset("9b_ctx4k"))
    case.run_gpu()
    B = case.p.block_size
    out = torch.full((1, B - 1), -7, dtype=torch.int32, device="cuda")
    lens = torch.zeros(1, dtype=torch.int32, device="cuda")
    case.dr.dflash_select_path(case.logits, None, None, 16, 0.0, out, lens, case.ws)
    torch.cuda.synchronize()
    assert torch.equal(out, case.draft) and lens.item() == B - 1


@pytest.mark.parametrize("S,V,rank,k,min_p", [(3, 151936, 256, 16, 0.0), (4, 151936, 256, 16, 0.3),
                                              (2, 1000, 8, 5, 0.0), (5, 3000, 32, 16, 0.45)])
def test_selector_parity(S, V, rank, k, min_p):
    p = small_variant(wl.preset("tiny_f32"), dtype="bf16", vocab=V, block_size=16, n_streams=S)
    dr = D.Drafter(D.config_from_preset(p, max_streams=S))
    ws = dr.new_workspace(16, S, 128)
    g = torch.Generator(device="cuda").manual_seed(100 * S + rank)
    logits = torch.randn((S, 15, V), generator=g, device="cuda") * 1.3
    # peaked rows: a random token a random height above the rest, so min-p stops vary
    tok = torch.randint(0, V, (S, 15), generator=g, device="cuda")
    # around the level where the peak holds half the mass (a row's partition sum is
    # about V e^0.85), so min-p stops land at different positions
    peak = np.log(V) + 0.85 - 1.0 + torch.rand((S, 15), generator=g, device="cuda") * 6.0
    logits.scatter_add_(2, tok[..., None], peak[..., None])
    U = (torch.randn((V, rank), generator=g, device="cuda") * 0.3).to(torch.bfloat16)
    W = (torch.randn((V, rank), generator=g, device="cuda") * 0.3).to(torch.bfloat16)
    out = torch.full((S, 15), -7, dtype=torch.int32, device="cuda")
    lens = torch.zeros(S, dtype=torch.int32, device="cuda")
    dr.dflash_select_path(logits, U, W, k, min_p, out, lens, ws)
    torch.cuda.synchronize()
    L = logits.cpu().numpy().astype(np.float64)
    Un, Wn = O.as_f64(to_np(U)), O.as_f64(to_np(W))
    got, glen = out.cpu().numpy(), lens.cpu().numpy()
    mp = float(np.float32(min_p))
    for s in range(S):
        toks, n = O.select_path(L[s], Un, Wn, k, mp)
        assert glen[s] == n, (s, glen[s], n)
        if not np.array_equal(got[s], toks):
            a = path_score(L[s], Un, Wn, got[s][:n], k)
            b = path_score(L[s], Un, Wn, toks[:n], k)
            assert abs(a - b) <= 1e-9, (s, a, b)
        print(f"[selector] V={V} rank={rank} k={k} min_p={min_p} stream {s}: length {n}", flush=True)


def test_selector_refuses_bad_arguments():
    p = small_variant(wl.preset("tiny_f32"), n_streams=1)
    dr = D.Drafter(D.config_from_preset(p))
    ws = dr.new_workspace(8, 1, 128)
    logits = torch.zeros((1, 7, p.vocab), device="cuda")
    out = torch.zeros((1, 7), dtype=torch.int32, device="cuda")
    lens = torch.zeros(1, dtype=torch.int32, device="cuda")
    for bad_k in (0, 17):
        with pytest.raises(D.DFlashError):
            dr.dflash_select_path(logits, None, None, bad_k, 0.0, out, lens, ws)
    with pytest.raises(D.DFlashError):
        dr.dflash_select_path(logits, None, None, 4, float("nan"), out, lens, ws)
