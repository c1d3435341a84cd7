"""Python binding of libdflash.so, the MI355X (gfx950) DFlash draft-round library.

Argument marshalling only: every step of the round runs in the library's HIP
kernels. PyTorch tensors supply device memory and the current stream. If the
library is not built this module raises on use; there is no fallback path.

The four calls of a round keep the C-ABI's names:
    dflash_fuse_taps, dflash_inject_kv, dflash_draft_block, dflash_verify_greedy
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lib", "libdflash.so")

MAX_LAYERS = 64
MAX_TAPS = 8

DFLASH_F32, DFLASH_BF16 = 0, 1
STATUS = {0: "OK", -1: "ERR_ARG", -2: "ERR_CONFIG", -3: "ERR_SHAPE", -4: "ERR_CAPACITY",
          -5: "ERR_STATE", -6: "ERR_DEVICE", -7: "ERR_UNIMPLEMENTED"}


class DFlashError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code
        self.status = STATUS.get(code, str(code))


class Config(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_layers", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("intermediate", ctypes.c_int32), ("vocab", ctypes.c_int32), ("n_taps", ctypes.c_int32),
                ("tap_layer_ids", ctypes.c_int32 * MAX_TAPS), ("target_n_layers", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("mask_token_id", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("layer_window", ctypes.c_int32 * MAX_LAYERS), ("rope_theta", ctypes.c_float),
                ("rms_eps", ctypes.c_float), ("max_streams", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("pool_pages", ctypes.c_int32)]


_VP = ctypes.c_void_p
_LAYER_FIELDS = ["in_norm", "wq", "wk", "wv", "wo", "q_norm", "k_norm", "post_norm", "w_gate", "w_up", "w_down"]


class Weights(ctypes.Structure):
    _fields_ = [(n, _VP) for n in ("embed", "lm_head", "fc", "hidden_norm", "norm")] + \
               [(n, _VP * MAX_LAYERS) for n in _LAYER_FIELDS]


class KV(ctypes.Structure):
    _fields_ = [("k_pool", _VP * MAX_LAYERS), ("v_pool", _VP * MAX_LAYERS), ("page_table", _VP),
                ("pages_per_stream", ctypes.c_int32)]


_lib = None


def library():
    """Load libdflash.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m block_diffusion_drafter_dflash_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "dflash_config_init": (None, [ctypes.POINTER(Config)]),
        "dflash_create": (i32, [ctypes.POINTER(Config), ctypes.POINTER(_VP)]),
        "dflash_tensor_count": (i32, [ctypes.POINTER(Config)]),
        "dflash_bind_weights": (i32, [_VP, ctypes.POINTER(Weights), ctypes.POINTER(i64)]),
        "dflash_packed_weight_bytes": (sz, [_VP]),
        "dflash_pack_weights": (i32, [_VP, _VP, sz, _VP]),
        "dflash_q4_weight_bytes": (sz, [_VP]),
        "dflash_pack_weights_q4": (i32, [_VP, _VP, sz, _VP]),
        "dflash_fused_row_bytes": (i64, [ctypes.POINTER(Config)]),
        "dflash_tap_row_bytes": (i64, [ctypes.POINTER(Config), i32]),
        "dflash_workspace_bytes": (sz, [_VP, i32, i32, i32]),
        "dflash_workspace_init": (i32, [_VP, _VP, sz, _VP]),
        "dflash_fuse_taps": (i32, [_VP, ctypes.POINTER(_VP), i64, i32, _VP, _VP, sz, _VP]),
        "dflash_inject_kv": (i32, [_VP, _VP, i32, _VP, _VP, ctypes.POINTER(KV), _VP, sz, _VP]),
        "dflash_inject_kv_layers": (i32, [_VP, _VP, i32, _VP, _VP, ctypes.POINTER(KV), ctypes.c_uint64, _VP, sz,
                                          _VP]),
        "dflash_layers_reading": (ctypes.c_uint64, [_VP, i32, i32]),
        "dflash_draft_block": (i32, [_VP, i32, _VP, _VP, i32, ctypes.POINTER(KV), _VP, _VP, _VP, _VP, sz, _VP]),
        "dflash_draft_block_noalloc": (i32, [_VP, i32, _VP, _VP, i32, ctypes.POINTER(KV), _VP, _VP, _VP, _VP]),
        "dflash_verify_greedy": (i32, [_VP, i32, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
        "dflash_sample_rows": (i32, [_VP, i32, _VP, i64, ctypes.c_float, _VP, _VP, _VP, _VP, sz, _VP]),
        "dflash_verify_sampling": (i32, [_VP, i32, _VP, _VP, _VP, i64, ctypes.c_float, _VP, _VP, _VP, _VP, _VP,
                                         _VP, _VP, sz, _VP]),
        "dflash_select_path": (i32, [_VP, i32, _VP, i64, _VP, _VP, i32, i32, ctypes.c_float, _VP, _VP, _VP, sz, _VP]),
        "dflash_trace_bytes": (sz, [_VP, i32]),
        "dflash_set_trace": (i32, [_VP, _VP, sz]),
        "dflash_set_profiling": (i32, [_VP, i32]),
        "dflash_profile_read": (i32, [_VP, ctypes.c_char_p, sz]),
        "dflash_last_error": (ctypes.c_char_p, [_VP]),
        "dflash_destroy": (None, [_VP]),
        "dflash_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


EXPORTED = ["dflash_config_init", "dflash_create", "dflash_tensor_count", "dflash_bind_weights",
            "dflash_packed_weight_bytes", "dflash_pack_weights", "dflash_q4_weight_bytes", "dflash_pack_weights_q4",
            "dflash_fused_row_bytes", "dflash_tap_row_bytes", "dflash_workspace_bytes", "dflash_workspace_init",
            "dflash_fuse_taps", "dflash_inject_kv", "dflash_inject_kv_layers", "dflash_layers_reading",
            "dflash_draft_block", "dflash_draft_block_noalloc", "dflash_verify_greedy",
            "dflash_sample_rows", "dflash_verify_sampling", "dflash_select_path",
            "dflash_trace_bytes", "dflash_set_trace", "dflash_set_profiling", "dflash_profile_read", "dflash_last_error", "dflash_destroy", "dflash_version"]


def make_config(hidden, n_layers, n_q_heads, n_kv_heads, head_dim, intermediate, vocab, tap_layer_ids,
                target_n_layers, block_size, mask_token_id, layer_window, dtype="bf16", rope_theta=1.0e6,
                rms_eps=1.0e-6, max_streams=1, pool_pages=1, page_size=16, causal=0):
    c = Config()
    library().dflash_config_init(ctypes.byref(c))
    c.dtype = DFLASH_F32 if dtype == "f32" else DFLASH_BF16
    c.hidden, c.n_layers, c.n_q_heads, c.n_kv_heads = hidden, n_layers, n_q_heads, n_kv_heads
    c.head_dim, c.intermediate, c.vocab = head_dim, intermediate, vocab
    c.n_taps = len(tap_layer_ids)
    for i, t in enumerate(tap_layer_ids[:MAX_TAPS]):
        c.tap_layer_ids[i] = t
    c.target_n_layers = target_n_layers
    c.block_size, c.mask_token_id, c.causal = block_size, mask_token_id, causal
    for i, wdw in enumerate(layer_window[:MAX_LAYERS]):
        c.layer_window[i] = wdw
    c.rope_theta, c.rms_eps = rope_theta, rms_eps
    c.max_streams, c.page_size, c.pool_pages = max_streams, page_size, pool_pages
    return c


def config_from_preset(p, max_streams=None, pool_pages=1):
    return make_config(p.hidden, p.n_layers, p.n_q_heads, p.n_kv_heads, p.head_dim, p.intermediate, p.vocab,
                       list(p.tap_layer_ids), p.target_n_layers, p.block_size, p.mask_token_id,
                       list(p.layer_window), dtype=p.dtype, rope_theta=p.rope_theta, rms_eps=p.rms_eps,
                       max_streams=max_streams or p.n_streams, pool_pages=pool_pages, page_size=p.page_size)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def tensor_order(n_layers):
    names = ["embed", "lm_head", "fc", "hidden_norm", "norm"]
    for l in range(n_layers):
        names += [f"layers.{l}.{t}" for t in _LAYER_FIELDS]
    return names


class Drafter:
    """A handle of the draft-round library with bound weights (all device memory caller-owned)."""

    def __init__(self, config: Config):
        self.lib = library()
        self.cfg = config
        h = ctypes.c_void_p()
        rc = self.lib.dflash_create(ctypes.byref(config), ctypes.byref(h))
        if rc != 0:
            raise DFlashError(rc, self.lib.dflash_last_error(None).decode())
        self.h = h
        self._keep = []

    def __del__(self):
        try:
            if getattr(self, "h", None):
                self.lib.dflash_destroy(self.h)
                self.h = None
        except Exception:
            pass

    def _check(self, rc):
        if rc != 0:
            raise DFlashError(rc, self.lib.dflash_last_error(self.h).decode())

    def last_error(self):
        return self.lib.dflash_last_error(self.h).decode()

    def dflash_select_path(self, logits, code_u, code_w, top_k, min_p, draft_out, draft_len, ws, n_streams=None,
                           stream=None):
        """DFlash2 path selector over logits [S, B-1, V] (fp32); code_u / code_w bf16 [V, r] or None."""
        n_streams = logits.shape[0] if n_streams is None else n_streams
        rank = 0 if code_u is None else int(code_u.shape[1])
        self._check(self.lib.dflash_select_path(self.h, n_streams, _ptr(logits), logits.stride(1), _ptr(code_u),
                                                _ptr(code_w), rank, int(top_k), float(min_p), _ptr(draft_out),
                                                _ptr(draft_len), _ptr(ws), ws.numel(), _stream(stream)))

    # -- instrumentation
    def trace_bytes(self, n_streams):
        return int(self.lib.dflash_trace_bytes(self.h, n_streams))

    def set_trace(self, buf):
        """Copy every stored tensor of each dflash_draft_block into `buf` (a device
        tensor of at least trace_bytes(n_streams) bytes); None turns it off."""
        self._check(self.lib.dflash_set_trace(self.h, _ptr(buf), 0 if buf is None else buf.numel() * buf.element_size()))

    def set_profiling(self, enable=True):
        self._check(self.lib.dflash_set_profiling(self.h, 1 if enable else 0))

    def profile_read(self):
        """{kernel name: (launches, total ms)} since the last read."""
        buf = ctypes.create_string_buffer(1 << 16)
        n = self.lib.dflash_profile_read(self.h, buf, len(buf))
        if n < 0:
            self._check(n)
        out = {}
        for line in buf.value.decode().splitlines():
            name, cnt, ms = line.split()
            out[name] = (int(cnt), float(ms))
        return out

    # -- weights
    def dflash_bind_weights(self, tensors: dict):
        """Bind a name -> tensor dict (names as in tensor_order); shapes are checked by the library."""
        w = Weights()
        shapes = []
        for name in tensor_order(self.cfg.n_layers):
            t = tensors.get(name)
            p = None if t is None else t.data_ptr()
            if name.startswith("layers."):
                _, l, field = name.split(".")
                getattr(w, field)[int(l)] = p
            else:
                setattr(w, name, p)
            if t is None:
                shapes += [0, 0]
            elif t.dim() == 1:
                shapes += [t.shape[0], 1]
            else:
                shapes += [t.shape[0], t.shape[1]]
        arr = (ctypes.c_int64 * len(shapes))(*shapes)
        self._check(self.lib.dflash_bind_weights(self.h, ctypes.byref(w), arr))
        self._keep = [tensors]

    def packed_weight_bytes(self):
        return int(self.lib.dflash_packed_weight_bytes(self.h))

    def dflash_pack_weights(self, buf, stream=None):
        self._check(self.lib.dflash_pack_weights(self.h, _ptr(buf), buf.numel() * buf.element_size(), _stream(stream)))
        self._packed = buf            # the library reads it from now on: keep it alive

    def new_packed_weights(self, device="cuda"):
        """Allocate the packed-weight buffer and pack the bound weights into it."""
        buf = torch.empty(self.packed_weight_bytes(), dtype=torch.uint8, device=device)
        self.dflash_pack_weights(buf)
        return buf

    def q4_weight_bytes(self):
        return int(self.lib.dflash_q4_weight_bytes(self.h))

    def dflash_pack_weights_q4(self, buf, stream=None):
        self._check(self.lib.dflash_pack_weights_q4(self.h, _ptr(buf), buf.numel() * buf.element_size(),
                                                    _stream(stream)))
        self._packed = buf

    def new_q4_weights(self, device="cuda"):
        """Allocate the 4-bit weight buffer and quantize the bound weights into it."""
        buf = torch.empty(self.q4_weight_bytes(), dtype=torch.uint8, device=device)
        self.dflash_pack_weights_q4(buf)
        return buf

    # -- workspace
    def workspace_bytes(self, max_rows, n_streams, max_ctx):
        return int(self.lib.dflash_workspace_bytes(self.h, max_rows, n_streams, max_ctx))

    def new_workspace(self, max_rows, n_streams, max_ctx, device="cuda"):
        n = self.workspace_bytes(max_rows, n_streams, max_ctx)
        if n == 0:
            raise DFlashError(-4, "workspace size request out of range")
        ws = torch.empty(n, dtype=torch.uint8, device=device)
        self._check(self.lib.dflash_workspace_init(self.h, _ptr(ws), n, _stream()))
        return ws

    # -- the round
    def dflash_fuse_taps(self, taps, fused_out, ws, n_rows=None, stream=None):
        n_rows = taps[0].shape[0] if n_rows is None else n_rows
        stride = taps[0].stride(0)
        arr = (ctypes.c_void_p * len(taps))(*[t.data_ptr() for t in taps])
        self._check(self.lib.dflash_fuse_taps(self.h, arr, stride, n_rows, _ptr(fused_out), _ptr(ws),
                                              ws.numel(), _stream(stream)))

    def dflash_inject_kv(self, fused, row_stream, row_pos, kv, ws, n_rows=None, stream=None):
        n_rows = fused.shape[0] if n_rows is None else n_rows
        self._check(self.lib.dflash_inject_kv(self.h, _ptr(fused), n_rows, _ptr(row_stream), _ptr(row_pos),
                                              ctypes.byref(kv.struct), _ptr(ws), ws.numel(), _stream(stream)))

    def dflash_inject_kv_layers(self, fused, row_stream, row_pos, kv, layer_mask, ws, n_rows=None, stream=None):
        n_rows = fused.shape[0] if n_rows is None else n_rows
        self._check(self.lib.dflash_inject_kv_layers(self.h, _ptr(fused), n_rows, _ptr(row_stream), _ptr(row_pos),
                                                     ctypes.byref(kv.struct), ctypes.c_uint64(layer_mask), _ptr(ws),
                                                     ws.numel(), _stream(stream)))

    def dflash_layers_reading(self, pos, ctx_len):
        """Bit mask of the layers that read context position `pos` at context length `ctx_len`."""
        return int(self.lib.dflash_layers_reading(self.h, int(pos), int(ctx_len)))

    def dflash_draft_block(self, anchor, ctx_len, max_ctx_len, kv, draft_out, ws, logits_out=None, top2_out=None,
                           n_streams=None, stream=None):
        n_streams = anchor.shape[0] if n_streams is None else n_streams
        self._check(self.lib.dflash_draft_block(self.h, n_streams, _ptr(anchor), _ptr(ctx_len), int(max_ctx_len),
                                                ctypes.byref(kv.struct), _ptr(draft_out), _ptr(logits_out),
                                                _ptr(top2_out), _ptr(ws), ws.numel(), _stream(stream)))

    def dflash_draft_block_noalloc(self, anchor, ctx_len, max_ctx_len, kv, draft_out, logits_out=None, top2_out=None,
                                   n_streams=None, stream=None):
        n_streams = anchor.shape[0] if n_streams is None else n_streams
        self._check(self.lib.dflash_draft_block_noalloc(self.h, n_streams, _ptr(anchor), _ptr(ctx_len),
                                                        int(max_ctx_len), ctypes.byref(kv.struct), _ptr(draft_out),
                                                        _ptr(logits_out), _ptr(top2_out), _stream(stream)))

    def dflash_verify_greedy(self, draft, target, accept_len, bonus, committed, ctx_len_inout=None,
                             n_streams=None, stream=None):
        n_streams = draft.shape[0] if n_streams is None else n_streams
        self._check(self.lib.dflash_verify_greedy(self.h, n_streams, _ptr(draft), _ptr(target), _ptr(accept_len),
                                                  _ptr(bonus), _ptr(committed), _ptr(ctx_len_inout),
                                                  _stream(stream)))

    def dflash_sample_rows(self, logits, temperature, u, token_out, ws, prob_out=None, n_rows=None, stream=None):
        n_rows = logits.shape[0] if n_rows is None else n_rows
        self._check(self.lib.dflash_sample_rows(self.h, n_rows, _ptr(logits), logits.stride(0), float(temperature),
                                                _ptr(u), _ptr(token_out), _ptr(prob_out), _ptr(ws), ws.numel(),
                                                _stream(stream)))

    def dflash_verify_sampling(self, draft, draft_logits, target_logits, temperature, u_accept, u_sample,
                               accept_len, token, committed, ws, ctx_len_inout=None, n_streams=None, stream=None):
        n_streams = draft.shape[0] if n_streams is None else n_streams
        self._check(self.lib.dflash_verify_sampling(self.h, n_streams, _ptr(draft), _ptr(draft_logits),
                                                    _ptr(target_logits), draft_logits.stride(-2),
                                                    float(temperature), _ptr(u_accept), _ptr(u_sample),
                                                    _ptr(accept_len), _ptr(token), _ptr(committed),
                                                    _ptr(ctx_len_inout), _ptr(ws), ws.numel(), _stream(stream)))


class PagedKV:
    """Caller-owned paged draft caches and their page table.

    Per layer a K pool [pool_pages, n_kv, 16, d] (a page holds 16 key rows) and a V pool
    [pool_pages, n_kv, d, 16] (a page holds the same 16 positions' values transposed).
    """

    def __init__(self, cfg: Config, page_table: torch.Tensor, pool_pages: int, dtype, device="cuda"):
        kshape = (pool_pages, cfg.n_kv_heads, cfg.page_size, cfg.head_dim)
        vshape = (pool_pages, cfg.n_kv_heads, cfg.head_dim, cfg.page_size)
        self.k = [torch.zeros(kshape, dtype=dtype, device=device) for _ in range(cfg.n_layers)]
        self.v = [torch.zeros(vshape, dtype=dtype, device=device) for _ in range(cfg.n_layers)]
        self.page_table = page_table.to(device=device, dtype=torch.int32).contiguous()
        self.pages_per_stream = self.page_table.shape[1]
        self.page_size = cfg.page_size
        s = KV()
        for l in range(cfg.n_layers):
            s.k_pool[l] = self.k[l].data_ptr()
            s.v_pool[l] = self.v[l].data_ptr()
        s.page_table = self.page_table.data_ptr()
        s.pages_per_stream = self.pages_per_stream
        self.struct = s

    def _slots(self, stream, start, n):
        pos = torch.arange(start, start + n, device=self.page_table.device)
        pages = self.page_table[stream, (pos // self.page_size).long()].long()
        return pages, (pos % self.page_size).long()

    def write_rows(self, layer, stream, start, k_rows, v_rows):
        """Write context rows [n, n_kv, d] for positions start.. of a stream (host-side setup of inputs)."""
        pages, slots = self._slots(stream, start, k_rows.shape[0])
        self.k[layer][pages, :, slots, :] = k_rows.to(self.k[layer].dtype)
        self.v[layer][pages, :, :, slots] = v_rows.to(self.v[layer].dtype)

    def read_rows(self, layer, stream, start, n):
        """K and V rows [n, n_kv, d] of positions start.. of a stream."""
        pages, slots = self._slots(stream, start, n)
        return self.k[layer][pages, :, slots, :], self.v[layer][pages, :, :, slots]
