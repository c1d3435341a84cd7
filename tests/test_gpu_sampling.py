"""GPU parity of the sampling calls (dflash_sample_rows, dflash_verify_sampling)
against the oracle's tempered draws and speculative-sampling verify, through the C-ABI.

Floating point decides integers here (which id a uniform lands on, whether a draft
token is accepted). The GPU forms probabilities from fp32 exponentials summed in
float64, the oracle in float64, so the two can differ only where a uniform lies
within a few 1e-7 (relative) of a decision boundary. The bar: every decision equals
the oracle's unless the oracle's own margin is below 1e-5 of the quantities compared;
there the GPU's outcome must still be a valid one (its id's oracle CDF interval
contains the uniform within that margin). Counts of such near-boundary cases are
printed; with seeded uniforms they are expected to be zero.
"""
import numpy as np
import pytest
import torch

import block_diffusion_drafter_dflash_amd as D
import workloads as wl
from oracle import dflash_oracle as O
from workloads.presets import small_variant

pytestmark = pytest.mark.gpu
EPS = 1e-5


def log(msg):
    print(msg, flush=True)


def drafter(vocab, block=16, max_streams=16):
    p = small_variant(wl.preset("9b_ctx4k"), name=f"sampling_v{vocab}", vocab=vocab, block_size=block)
    return D.Drafter(D.config_from_preset(p, max_streams=max_streams)), p


def check_draw(tok, probs, u, what):
    """tok must be the oracle's draw, or (near a boundary) a valid one."""
    k = O.sample_index(probs, u)
    if tok == k:
        return 0
    c = np.cumsum(probs) / probs.sum()
    lo = c[tok - 1] if tok > 0 else 0.0
    assert 0 <= tok < len(probs) and probs[tok] > 0, f"{what}: id {tok} invalid"
    assert lo - EPS <= u < c[tok] + EPS, f"{what}: id {tok} (oracle {k}) does not own u={u}"
    return 1


@pytest.mark.parametrize("vocab,T", [(151936, 1.0), (151936, 0.25), (1000, 3.0), (1000, 0.05)])
def test_sample_rows_parity(vocab, T):
    dr, _ = drafter(vocab)
    rows = 37
    ws = dr.new_workspace(rows, 1, 64)
    g = torch.Generator(device="cuda").manual_seed(vocab + int(T * 100))
    logits = torch.randn((rows, vocab), generator=g, device="cuda", dtype=torch.float32) * 3.0
    logits[5, ::3] = float("-inf")          # a row with masked ids
    u = torch.rand(rows, generator=g, device="cuda")
    u[0], u[1] = 0.0, 1.0 - 2.0 ** -24
    tok = torch.zeros(rows, dtype=torch.int32, device="cuda")
    prob = torch.zeros(rows, dtype=torch.float32, device="cuda")
    log(f"[sample_rows] V={vocab} T={T} rows={rows}")
    dr.dflash_sample_rows(logits, T, u, tok, ws, prob_out=prob)
    torch.cuda.synchronize()
    L, U, K, P = logits.cpu().numpy().astype(np.float64), u.cpu().numpy(), tok.cpu().numpy(), prob.cpu().numpy()
    near = 0
    for r in range(rows):
        q = O.tempered_probs(L[r], T)
        near += check_draw(int(K[r]), q, float(U[r]), f"row {r}")
        assert abs(P[r] - q[K[r]]) <= 1e-5 * q[K[r]] + 1e-12, (r, P[r], q[K[r]])
    assert all(K[5] % 3 != 0 for _ in [0]), "a masked id was drawn"
    log(f"  near-boundary draws: {near}")
    # deterministic
    tok2 = torch.zeros_like(tok)
    dr.dflash_sample_rows(logits, T, u, tok2, ws)
    torch.cuda.synchronize()
    assert torch.equal(tok, tok2)


def run_verify(dr, draft, dlog, tlog, T, ua, us, ws, ctx=None):
    S = draft.shape[0]
    B = tlog.shape[1]
    acc = torch.zeros(S, dtype=torch.int32, device="cuda")
    tok = torch.zeros(S, dtype=torch.int32, device="cuda")
    com = torch.full((S, B), 7, dtype=torch.int32, device="cuda")
    dr.dflash_verify_sampling(draft, dlog, tlog, T, ua, us, acc, tok, com, ws, ctx_len_inout=ctx)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), tok.cpu().numpy(), com.cpu().numpy()


def check_verify(draft, dlog, tlog, T, ua, us, acc, tok, com):
    """Stream by stream against the oracle; near-boundary decisions checked for validity."""
    S, Bm1 = draft.shape
    oa, ot, oc = O.verify_sampling(draft, dlog, tlog, T, ua, us)
    near = 0
    for s in range(S):
        if acc[s] != oa[s]:
            # the first differing decision must sit on the oracle's boundary
            j = min(acc[s], oa[s])
            p = O.tempered_probs(dlog[s, j], T)[draft[s, j]]
            q = O.tempered_probs(tlog[s, j], T)[draft[s, j]]
            assert abs(ua[s, j] * p - q) <= EPS * max(q, ua[s, j] * p), (s, acc[s], oa[s])
            near += 1
            continue
        a = int(acc[s])
        if a < Bm1:
            r = np.maximum(O.tempered_probs(tlog[s, a], T) - O.tempered_probs(dlog[s, a], T), 0.0)
            w = r if r.sum() > 0 else O.tempered_probs(tlog[s, a], T)
        else:
            w = O.tempered_probs(tlog[s, Bm1], T)
        near += check_draw(int(tok[s]), w, float(us[s]), f"stream {s}")
        assert list(com[s]) == list(draft[s, :a]) + [int(tok[s])] + [-1] * (Bm1 - a), s
    return near


@pytest.mark.parametrize("vocab,S,T", [(151936, 16, 1.0), (1000, 9, 0.7)])
def test_verify_sampling_parity(vocab, S, T):
    B = 16
    dr, _ = drafter(vocab, block=B)
    ws = dr.new_workspace(1, S, 64)
    g = torch.Generator(device="cuda").manual_seed(7 * vocab + S)
    tlog = torch.randn((S, B, vocab), generator=g, device="cuda") * 2.0
    # draft logits near the target's, so acceptance runs are long and rejections occur
    dlog = (tlog[:, :B - 1] + 0.6 * torch.randn((S, B - 1, vocab), generator=g, device="cuda")).contiguous()
    u_draw = torch.rand((S * (B - 1),), generator=g, device="cuda")
    draft = torch.zeros(S * (B - 1), dtype=torch.int32, device="cuda")
    dr.dflash_sample_rows(dlog.view(S * (B - 1), vocab), T, u_draw, draft, ws)
    draft = draft.view(S, B - 1)
    ua = torch.rand((S, B - 1), generator=g, device="cuda")
    us = torch.rand(S, generator=g, device="cuda")
    ctx = torch.full((S,), 100, dtype=torch.int32, device="cuda")
    log(f"[verify_sampling] V={vocab} S={S} T={T}")
    acc, tok, com = run_verify(dr, draft, dlog, tlog, T, ua, us, ws, ctx)
    D_, DL, TL = draft.cpu().numpy(), dlog.cpu().numpy().astype(np.float64), tlog.cpu().numpy().astype(np.float64)
    UA, US = ua.cpu().numpy().astype(np.float64), us.cpu().numpy().astype(np.float64)
    near = check_verify(D_, DL, TL, T, UA, US, acc, tok, com)
    log(f"  accepted lengths {list(acc)}; near-boundary decisions: {near}")
    assert np.array_equal(ctx.cpu().numpy(), 100 + acc + 1)
    assert 0 < acc.mean() < B - 1, "the case should mix acceptances and rejections"
    acc2, tok2, com2 = run_verify(dr, draft, dlog, tlog, T, ua, us, ws)
    assert np.array_equal(acc, acc2) and np.array_equal(tok, tok2) and np.array_equal(com, com2)


def test_verify_sampling_edge_cases():
    B, V, S, T = 8, 1000, 4, 1.0
    dr, _ = drafter(V, block=B)
    ws = dr.new_workspace(1, S, 64)
    g = torch.Generator(device="cuda").manual_seed(11)
    tlog = torch.randn((S, B, V), generator=g, device="cuda")
    ua = torch.rand((S, B - 1), generator=g, device="cuda")
    us = torch.rand(S, generator=g, device="cuda")
    draft = torch.randint(0, V, (S, B - 1), generator=g, device="cuda", dtype=torch.int32)
    # identical distributions: everything is accepted, the token comes from q_{B-1}
    dlog = tlog[:, :B - 1].contiguous()
    acc, tok, com = run_verify(dr, draft, dlog, tlog, T, ua, us, ws)
    assert np.all(acc == B - 1)
    check_verify(draft.cpu().numpy(), dlog.cpu().numpy().astype(np.float64), tlog.cpu().numpy().astype(np.float64),
                 T, ua.cpu().numpy().astype(np.float64), us.cpu().numpy().astype(np.float64), acc, tok, com)
    # an id outside the vocabulary is rejected where it stands
    bad = draft.clone()
    bad[1, 3] = V + 5
    bad[2, 0] = -1
    acc, tok, com = run_verify(dr, bad, dlog, tlog, T, ua, us, ws)
    assert acc[1] == 3 and acc[2] == 0 and acc[0] == B - 1
    # the target excludes the drafted id: rejection, and the draw avoids it
    t2 = tlog.clone()
    for s in range(S):
        t2[s, 0, int(draft[s, 0])] = float("-inf")
    acc, tok, com = run_verify(dr, draft, dlog, t2, T, ua, us, ws)
    assert np.all(acc == 0) and all(int(tok[s]) != int(draft[s, 0]) for s in range(S))


def test_sampling_calls_refuse_bad_arguments():
    dr, _ = drafter(1000, block=8)
    ws = dr.new_workspace(1, 2, 64)
    x = torch.zeros((2, 1000), device="cuda")
    u = torch.zeros(2, device="cuda")
    t = torch.zeros(2, dtype=torch.int32, device="cuda")
    for T in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(D.DFlashError):
            dr.dflash_sample_rows(x, T, u, t, ws)
    narrow = torch.zeros((2, 500), device="cuda")
    with pytest.raises(D.DFlashError):
        dr.dflash_sample_rows(narrow, 1.0, u, t, ws)    # row stride below the vocabulary
    big, _ = drafter(262144 + 256, block=8)        # past the kernels' vocabulary bound (host refusal)
    wide = torch.zeros((2, 262144 + 256), device="cuda")
    with pytest.raises(D.DFlashError):
        big.dflash_sample_rows(wide, 1.0, u, t, ws)
