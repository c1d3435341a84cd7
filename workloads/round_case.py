"""Set up one draft round on synthetic inputs, run it through the HIP library, and
(for the tests) gather the same input bytes for the CPU oracle. Used by the GPU
parity tests, smoke() and the benchmark; not imported by the oracle, nor by
workloads/__init__.

The existing context of each stream (positions 0 .. C-R-1) is built, for presets with
context_from_taps, from seeded tap planes through the library's own fuse + inject
(the oracle fuses and injects the same planes itself), and otherwise written straight
into the paged caches as seeded N(0, 1) rows. The round then fuses and injects its
own R rows at positions C-R .. C-1, drafts at C .. C+B-1, and verifies against a
synthetic target row.
"""
import numpy as np
import torch

import block_diffusion_drafter_dflash_amd as D
import workloads as wl


def to_np(t):
    """Tensor -> numpy in storage format (bf16 -> uint16 bits, fp32 -> float32)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class RoundCase:
    def __init__(self, p, ctx=None, rows=None, device="cuda", permute_pages=True, seed=None, weights=None, q4=False):
        self.p = p
        self.device = device
        seed = p.seed if seed is None else seed
        self.seed = seed
        S, B = p.n_streams, p.block_size
        self.ctx = list(ctx) if ctx is not None else wl.ctx_lens(p, seed)
        self.rows = list(rows) if rows is not None else wl.round_rows(p, seed)
        self.rows = [min(r, c) for r, c in zip(self.rows, self.ctx)]
        self.dtype = torch.float32 if p.dtype == "f32" else torch.bfloat16
        self.W = weights if weights is not None else wl.make_weights(p, device=device, seed=seed)
        R = sum(self.rows)
        self.R = R
        self.taps = wl.make_taps(p, R, device=device, seed=seed)
        rs, rp = [], []
        for s in range(S):
            rs += [s] * self.rows[s]
            rp += list(range(self.ctx[s] - self.rows[s], self.ctx[s]))
        self.row_stream = torch.tensor(rs, dtype=torch.int32, device=device)
        self.row_pos = torch.tensor(rp, dtype=torch.int32, device=device)
        self.anchor = torch.from_numpy(wl.make_anchor(p, seed)).to(device)
        self.ctx_len = torch.tensor(self.ctx, dtype=torch.int32, device=device)
        self.max_ctx = max(self.ctx)
        table, pool = wl.make_page_table(p, self.ctx, extra_tokens=0, permute=permute_pages, seed=seed)
        self.page_table = torch.from_numpy(table)
        self.pool_pages = pool
        self.cfg = D.config_from_preset(p, max_streams=S, pool_pages=pool)
        self.kv = D.PagedKV(self.cfg, self.page_table, pool, self.dtype, device=device)
        # Pre-existing context rows: built from seeded tap planes through the library's
        # own fuse + inject (presets with context_from_taps; the 4-bit drafter runs
        # calls of at most 32 rows, so its cases take the written rows), or seeded
        # K/V rows written straight into the cache.
        self.ctx_from_taps = bool(p.context_from_taps) and not q4
        if not self.ctx_from_taps:
            for l in range(p.n_layers):
                for s in range(S):
                    n = self.ctx[s] - self.rows[s]
                    if n > 0:
                        k = wl.make_context_kv(p, l, s, n, "k", device=device, seed=seed)
                        v = wl.make_context_kv(p, l, s, n, "v", device=device, seed=seed)
                        self.kv.write_rows(l, s, 0, k, v)
        self.dr = D.Drafter(self.cfg)
        self.dr.dflash_bind_weights(self.W)
        self.q4 = q4
        if q4:
            self.dr.new_q4_weights(device=device)        # the drafter's 4-bit copies
        else:
            self.dr.new_packed_weights(device=device)
        if self.ctx_from_taps:
            self._prefill_context()
        self.ws = self.dr.new_workspace(max(R, 1), S, self.max_ctx, device=device)
        self.fused = torch.zeros((max(R, 1), p.hidden), dtype=self.dtype, device=device)
        self.draft = torch.zeros((S, B - 1), dtype=torch.int32, device=device)
        self.logits = torch.zeros((S, B - 1, p.vocab), dtype=torch.float32, device=device)
        self.top2 = torch.zeros((S, B - 1, 2), dtype=torch.float32, device=device)
        self.accept = torch.zeros(S, dtype=torch.int32, device=device)
        self.bonus = torch.zeros(S, dtype=torch.int32, device=device)
        self.committed = torch.zeros((S, B), dtype=torch.int32, device=device)
        self.target = None

    # ---------------------------------------------------------------- GPU path
    def _prefill_context(self):
        """Stream s's context rows 0..C_s-R_s-1: its seeded context tap planes fused
        (dflash_fuse_taps) and injected at those positions (dflash_inject_kv), one call
        each per stream."""
        p, dev = self.p, self.device
        ns = [c - r for c, r in zip(self.ctx, self.rows)]
        nmax = max(ns + [0])
        if nmax == 0:
            return
        ws = self.dr.new_workspace(nmax, p.n_streams, self.max_ctx, device=dev)
        fused = torch.empty((nmax, p.hidden), dtype=self.dtype, device=dev)
        for s, n in enumerate(ns):
            if n <= 0:
                continue
            taps = wl.make_context_taps(p, s, n, device=dev, seed=self.seed)
            self.dr.dflash_fuse_taps(taps, fused, ws, n_rows=n)
            rs = torch.full((n,), s, dtype=torch.int32, device=dev)
            rp = torch.arange(n, dtype=torch.int32, device=dev)
            self.dr.dflash_inject_kv(fused, rs, rp, self.kv, ws, n_rows=n)
            del taps
        torch.cuda.synchronize()
        del ws, fused

    def fuse(self):
        self.dr.dflash_fuse_taps(self.taps, self.fused, self.ws, n_rows=self.R)

    def inject(self):
        self.dr.dflash_inject_kv(self.fused, self.row_stream, self.row_pos, self.kv, self.ws, n_rows=self.R)

    def draft_block(self, logits=True, top2=True, ctx_len=None):
        self.dr.dflash_draft_block(self.anchor, self.ctx_len if ctx_len is None else ctx_len, self.max_ctx,
                                   self.kv, self.draft, self.ws, logits_out=self.logits if logits else None,
                                   top2_out=self.top2 if top2 else None)

    def verify(self, ctx_inout=None):
        self.dr.dflash_verify_greedy(self.draft, self.target, self.accept, self.bonus, self.committed,
                                     ctx_len_inout=ctx_inout)

    def run_gpu(self):
        self.fuse()
        self.inject()
        self.draft_block()
        torch.cuda.synchronize()

    def set_target_from(self, tokens, seed_offset=0):
        L = wl.draw_accept_lengths(self.p, self.seed + seed_offset)
        t = wl.make_target_rows(np.asarray(tokens), L, self.p.vocab, self.seed + 991 + seed_offset)
        self.target = torch.from_numpy(t).to(self.device)
        return t

    # ---------------------------------------------------------------- oracle inputs
    def weights_np(self):
        if not hasattr(self, "_wnp"):
            self._wnp = {k: to_np(v) for k, v in self.W.items()}
        return self._wnp

    def oracle_streams(self, streams):
        """Oracle stream dicts for the chosen streams: taps, C, anchor, and the existing
        context as given K/V rows (k_ctx, v_ctx) or, when it was built from taps, as
        those tap planes (ctx_taps) for the oracle to fuse and inject itself."""
        p = self.p
        out = []
        off = np.cumsum([0] + self.rows)
        taps = [to_np(t) for t in self.taps]
        anchor = self.anchor.cpu().numpy()
        for s in streams:
            n = self.ctx[s] - self.rows[s]
            if self.ctx_from_taps:
                ctx_taps = [to_np(t) for t in wl.make_context_taps(p, s, max(n, 0), device=self.device, seed=self.seed)]
                out.append(dict(taps=[t[off[s]:off[s + 1]] for t in taps], C=self.ctx[s], ctx_taps=ctx_taps,
                                anchor=int(anchor[s])))
                continue
            kc, vc = [], []
            for l in range(p.n_layers):
                if n > 0:
                    kc.append(to_np(wl.make_context_kv(p, l, s, n, "k", device=self.device, seed=self.seed)))
                    vc.append(to_np(wl.make_context_kv(p, l, s, n, "v", device=self.device, seed=self.seed)))
                else:
                    e = np.zeros((0, p.n_kv_heads, p.head_dim), dtype=taps[0].dtype)
                    kc.append(e)
                    vc.append(e)
            out.append(dict(taps=[t[off[s]:off[s + 1]] for t in taps], C=self.ctx[s], k_ctx=kc, v_ctx=vc,
                            anchor=int(anchor[s])))
        return out
