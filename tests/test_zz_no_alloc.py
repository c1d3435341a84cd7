"""The draft entry point that allocates nothing (dflash_draft_block_noalloc), against
dflash_draft_block on the same inputs, through the C-ABI.

Two calls in a row, the second with a smaller input (fewer streams, a shorter
context), each bit for bit equal to the workspace entry point's result (the same
kernels on the same inputs); and a draft too large for the device array refused
before anything is enqueued.
"""
import ctypes
from types import SimpleNamespace

import pytest
import torch

import block_diffusion_drafter_dflash_amd as D
import workloads as wl
from workloads.presets import small_variant
from workloads.round_case import RoundCase

pytestmark = pytest.mark.gpu

MID = small_variant(wl.preset("9b_ctx32k"), name="noalloc_bf16", hidden=384, n_layers=3, n_q_heads=6,
                    n_kv_heads=2, head_dim=128, intermediate=640, vocab=1000, n_taps=3,
                    tap_layer_ids=[0, 4, 11], target_n_layers=12, layer_window=[100, 0, 37],
                    n_streams=4, ctx_spec=[300, 77, 1030, 0], accept_spec=("uniform",), seed=2101)


def sub_kv(case, streams):
    kv = SimpleNamespace(struct=D.KV())
    for l in range(case.p.n_layers):
        kv.struct.k_pool[l] = case.kv.k[l].data_ptr()
        kv.struct.v_pool[l] = case.kv.v[l].data_ptr()
    kv.pt = case.kv.page_table[streams].contiguous()
    kv.struct.page_table = kv.pt.data_ptr()
    kv.struct.pages_per_stream = case.kv.pages_per_stream
    return kv


def both_ways(case, streams, max_ctx):
    kv = sub_kv(case, streams)
    anchor = case.anchor[streams].contiguous()
    ctx = case.ctx_len[streams].contiguous()
    S, B, V = len(streams), case.p.block_size, case.p.vocab
    out = []
    for noalloc in (False, True):
        logits = torch.full((S, B - 1, V), float("nan"), device="cuda")
        top2 = torch.full((S, B - 1, 2), float("nan"), device="cuda")
        draft = torch.full((S, B - 1), -7, dtype=torch.int32, device="cuda")
        if noalloc:
            case.dr.dflash_draft_block_noalloc(anchor, ctx, max_ctx, kv, draft, logits_out=logits, top2_out=top2)
        else:
            case.dr.dflash_draft_block(anchor, ctx, max_ctx, kv, draft, case.ws, logits_out=logits, top2_out=top2)
        torch.cuda.synchronize()
        out.append((logits, top2, draft))
    (la, ta, da), (lb, tb, db) = out
    assert torch.equal(la.view(torch.int32), lb.view(torch.int32))
    assert torch.equal(ta.view(torch.int32), tb.view(torch.int32))
    assert torch.equal(da, db)
    assert not torch.isnan(lb).any()


def test_noalloc_draft_matches_the_workspace_draft_twice_then_smaller():
    case = RoundCase(MID)
    case.fuse()
    case.inject()
    torch.cuda.synchronize()
    print(f"[noalloc] {MID.name}: 4 streams, ctx {case.ctx}", flush=True)
    both_ways(case, [0, 1, 2, 3], case.max_ctx)       # 64 block rows (tiled class)
    print("[noalloc] second call: 1 stream, ctx 77", flush=True)
    both_ways(case, [1], 77)                          # 16 rows, a shorter context


def test_noalloc_draft_with_a_k_split_gate_up_tail():
    # 2 * 17408 gate/up rows: the tiled kernel's last 16 column tiles go through K ranges
    # whose partials also live in the device array (96 block rows, then 16).
    p = small_variant(MID, name="noalloc_tail_bf16", intermediate=17408, n_streams=6,
                      ctx_spec=[300, 77, 1030, 0, 513, 64], seed=2103)
    case = RoundCase(p)
    case.fuse()
    case.inject()
    torch.cuda.synchronize()
    assert case.dr.workspace_bytes(0, 6, case.max_ctx) <= 32 << 20
    print(f"[noalloc] {p.name}: 6 streams, ctx {case.ctx}", flush=True)
    both_ways(case, list(range(6)), case.max_ctx)
    print("[noalloc] second call: 1 stream, ctx 300", flush=True)
    both_ways(case, [0], 300)


def test_noalloc_refuses_a_draft_past_its_array():
    case = RoundCase(small_variant(MID, n_streams=1, ctx_spec=[64]))
    S = 1
    big = 1 << 21                                     # a context whose attention partials exceed 32 MiB
    assert case.dr.workspace_bytes(0, S, big) > 32 << 20
    kv = SimpleNamespace(struct=D.KV())
    for l in range(case.p.n_layers):
        kv.struct.k_pool[l] = case.kv.k[l].data_ptr()
        kv.struct.v_pool[l] = case.kv.v[l].data_ptr()
    kv.struct.page_table = case.kv.page_table.data_ptr()
    kv.struct.pages_per_stream = big // 16            # nothing is read: the call is refused on the host
    lib = D.library()
    rc = lib.dflash_draft_block_noalloc(case.dr.h, S, ctypes.c_void_p(case.anchor.data_ptr()),
                                        ctypes.c_void_p(case.ctx_len.data_ptr()), big, ctypes.byref(kv.struct),
                                        ctypes.c_void_p(case.draft.data_ptr()), None, None, None)
    assert rc == -4 and "scratch" in case.dr.last_error()
