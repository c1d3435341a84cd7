"""Host-side tests of the C-ABI boundary: no GPU needed, no compute call is made.

Refusals are checked to happen on the host before any enqueue (TensorFold pull
request #1851, item 1: taps past the target or repeated, a causal draft;
"Port the DFlash2 protocol, not its checkpoint": no partial loads).
"""
import ctypes
import os
import re

import pytest

import block_diffusion_drafter_dflash_amd as D
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_[a-z_0-9]+)\s*\(", src)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = D.library()
    names = declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(D.EXPORTED)
    assert lib.dflash_version().decode().startswith("dflash")


def cfg_of(name="9b_ctx4k", **over):
    p = wl.preset(name)
    c = D.config_from_preset(p, pool_pages=1024)
    for k, v in over.items():
        if k in ("tap_layer_ids", "layer_window"):
            arr = getattr(c, k)
            for i, x in enumerate(v):
                arr[i] = x
        else:
            setattr(c, k, v)
    return c


def create(c):
    lib = D.library()
    h = ctypes.c_void_p()
    rc = lib.dflash_create(ctypes.byref(c), ctypes.byref(h))
    return rc, h, lib.dflash_last_error(None).decode()


@pytest.mark.parametrize("name", ["tiny_f32", "9b_ctx4k", "9b_ctx32k", "dflash2_x16", "9b_long_x4"])
def test_presets_are_accepted(name):
    rc, h, msg = create(cfg_of(name))
    assert rc == 0, msg
    D.library().dflash_destroy(h)


@pytest.mark.parametrize("over,needle", [
    (dict(causal=1), "causal"),
    (dict(tap_layer_ids=[1, 5, 9, 13, 17, 21, 25, 32]), "past the target"),
    (dict(tap_layer_ids=[1, 5, 5, 13, 17, 21, 25, 29]), "repeated"),
    (dict(tap_layer_ids=[1, 9, 5, 13, 17, 21, 25, 29]), "ascending"),
    (dict(n_taps=0), "n_taps"),
    (dict(n_taps=9), "n_taps"),
    (dict(block_size=1), "block_size"),
    (dict(n_kv_heads=6), "multiple"),
    (dict(head_dim=96), "head_dim"),
    (dict(hidden=4000), "hidden"),
    (dict(hidden=16384 + 128), "exceeds"),
    (dict(mask_token_id=151936), "mask_token_id"),
    (dict(layer_window=[0, 0, -1]), "window"),
    (dict(page_size=32), "page_size"),
    (dict(pool_pages=1 << 28), "2^31"),
    (dict(dtype=7), "dtype"),
    (dict(max_streams=0), "max_streams"),
])
def test_config_refusals(over, needle):
    rc, h, msg = create(cfg_of(**over))
    assert rc == -2 and not h.value
    assert needle in msg


def test_tensor_count_and_storage_closed_forms():
    lib = D.library()
    assert lib.dflash_tensor_count(ctypes.byref(cfg_of("9b_ctx4k"))) == 69
    assert lib.dflash_tensor_count(ctypes.byref(cfg_of("tiny_f32"))) == 25
    assert lib.dflash_tensor_count(ctypes.byref(cfg_of("dflash2_x16"))) == 58
    c = cfg_of("9b_ctx4k")
    assert lib.dflash_fused_row_bytes(ctypes.byref(c)) == 8 * 1024
    assert lib.dflash_tap_row_bytes(ctypes.byref(c), 1) == 18 * 4096 * 2
    assert lib.dflash_tap_row_bytes(ctypes.byref(c), 0) == 8 * 4096 * 2 == 64 * 1024
    c2 = cfg_of("dflash2_x16")
    assert lib.dflash_tap_row_bytes(ctypes.byref(c2), 0) == 5 * 5120 * 2


def fake_tensors(p, bad=None, misalign=None):
    """Shape-only stand-ins with aligned fake addresses (bind never dereferences them)."""
    class T:
        def __init__(self, shape, addr):
            self.shape = shape
            self._a = addr

        def dim(self):
            return len(self.shape)

        def data_ptr(self):
            return self._a

    out = {}
    addr = 1 << 20
    for name in D.tensor_order(p.n_layers):
        shape = wl.tensor_shape(p, name)
        if name == bad:
            shape = tuple(x + 1 for x in shape)
        out[name] = T(shape, addr + (8 if name == misalign else 0))
        addr += 1 << 12
    return out


def test_bind_checks_every_tensor_and_refuses_as_a_whole():
    p = wl.preset("tiny_f32")
    dr = D.Drafter(cfg_of("tiny_f32"))
    with pytest.raises(D.DFlashError) as e:
        dr.dflash_bind_weights(fake_tensors(p, bad="layers.1.w_down"))
    assert e.value.status == "ERR_SHAPE" and "layers.1.w_down" in str(e.value)
    with pytest.raises(D.DFlashError) as e:
        dr.dflash_bind_weights(fake_tensors(p, misalign="layers.0.wq"))
    assert e.value.status == "ERR_ARG"
    t = fake_tensors(p)
    del t["layers.0.k_norm"]
    with pytest.raises(D.DFlashError) as e:
        dr.dflash_bind_weights(t)
    assert "k_norm" in str(e.value)
    # nothing was bound: the round calls still refuse with ERR_STATE
    lib = D.library()
    rc = lib.dflash_fuse_taps(dr.h, None, 256, 4, None, None, 0, None)
    assert rc == -5
    dr.dflash_bind_weights(fake_tensors(p))       # a whole, valid set binds


def test_round_calls_refuse_on_the_host_before_any_enqueue():
    p = wl.preset("tiny_f32")
    dr = D.Drafter(cfg_of("tiny_f32"))
    dr.dflash_bind_weights(fake_tensors(p))
    lib = D.library()
    fake = ctypes.c_void_p(1 << 24)
    # workspace never initialised -> ERR_STATE (checked before any launch)
    planes = (ctypes.c_void_p * 3)(1 << 24, 1 << 25, 1 << 26)
    rc = lib.dflash_fuse_taps(dr.h, planes, 256, 4, fake, fake, 1 << 20, None)
    assert rc == -5 and "initialised" in dr.last_error()
    # bad stride (below hidden, not a multiple of 8, past 2^27), zero rows is a no-op
    assert lib.dflash_fuse_taps(dr.h, planes, 100, 4, fake, fake, 1 << 20, None) == -1
    assert lib.dflash_fuse_taps(dr.h, planes, 260, 4, fake, fake, 1 << 20, None) == -1
    assert lib.dflash_fuse_taps(dr.h, planes, (1 << 27) + 8, 4, fake, fake, 1 << 20, None) == -1
    assert "2^27" in dr.last_error()
    assert lib.dflash_fuse_taps(dr.h, planes, 256, 0, fake, fake, 1 << 20, None) == 0
    # a request past the cache span is refused
    kv = D.KV()
    for l in range(p.n_layers):
        kv.k_pool[l] = 1 << 24
        kv.v_pool[l] = 1 << 25
    kv.page_table = 1 << 26
    kv.pages_per_stream = 8            # 128 tokens
    rc = lib.dflash_draft_block(dr.h, 1, fake, fake, 129, ctypes.byref(kv), fake, None, None, fake, 1 << 20, None)
    assert rc == -4 and "span" in dr.last_error()
    rc = lib.dflash_draft_block(dr.h, 2, fake, fake, 64, ctypes.byref(kv), fake, None, None, fake, 1 << 20, None)
    assert rc == -4 and "n_streams" in dr.last_error()
    # a layer mask naming a layer past n_layers; an empty mask is a no-op
    rc = lib.dflash_inject_kv_layers(dr.h, fake, 4, fake, fake, ctypes.byref(kv), 1 << p.n_layers, fake, 1 << 20, None)
    assert rc == -1 and "layer_mask" in dr.last_error()
    assert lib.dflash_inject_kv_layers(dr.h, fake, 4, fake, fake, ctypes.byref(kv), 0, fake, 1 << 20, None) == 0
    kv.k_pool[1] = 0
    rc = lib.dflash_inject_kv(dr.h, fake, 4, fake, fake, ctypes.byref(kv), fake, 1 << 20, None)
    assert rc == -1 and "pool" in dr.last_error()
    rc = lib.dflash_inject_kv_layers(dr.h, fake, 4, fake, fake, ctypes.byref(kv), 0b10, fake, 1 << 20, None)
    assert rc == -1 and "pool" in dr.last_error()
    assert lib.dflash_verify_greedy(dr.h, 0, fake, fake, fake, fake, fake, None, None) == -1


def test_workspace_registration_enqueues_nothing_and_bounds_later_calls():
    # dflash_workspace_init only records the buffer (no kernel: it works without a GPU);
    # a call given more bytes than were registered is refused before any launch, and
    # registering the buffer again with more bytes is accepted.
    p = wl.preset("tiny_f32")
    dr = D.Drafter(cfg_of("tiny_f32"))
    dr.dflash_bind_weights(fake_tensors(p))
    lib = D.library()
    fake = ctypes.c_void_p(1 << 24)
    assert lib.dflash_workspace_init(dr.h, fake, 1 << 20, None) == 0
    planes = (ctypes.c_void_p * 3)(1 << 24, 1 << 25, 1 << 26)
    rc = lib.dflash_fuse_taps(dr.h, planes, 256, 4, fake, fake, 1 << 21, None)
    assert rc == -5 and "initialised" in dr.last_error()
    assert lib.dflash_workspace_init(dr.h, fake, 1 << 21, None) == 0
    assert lib.dflash_workspace_init(dr.h, fake, 0, None) == -4
    assert lib.dflash_workspace_init(dr.h, None, 1 << 20, None) == -1
    assert lib.dflash_workspace_init(dr.h, ctypes.c_void_p((1 << 24) + 8), 1 << 20, None) == -1


def test_workspace_sizes_grow_with_the_request():
    dr = D.Drafter(cfg_of("9b_long_x4"))
    a = dr.workspace_bytes(16, 1, 4096)
    b = dr.workspace_bytes(64, 4, 131072)
    assert 0 < a < b
    assert dr.workspace_bytes(16, 5, 4096) == 0      # more streams than max_streams
    assert dr.workspace_bytes(-1, 1, 4096) == 0


def test_layers_reading_follows_each_layers_reach():
    # A layer reads position pos at context C when pos lies in its reach, as the oracle
    # defines it ([max(0, C - W), C), all of [0, C) for a full layer).
    from oracle import dflash_oracle as O
    p = wl.preset("9b_long_x4")            # five sliding layers (W = 4096) and one full
    dr = D.Drafter(cfg_of("9b_long_x4"))
    for C in (0, 1, 100, 4096, 4097, 32768):
        for pos in sorted({-1, 0, 1, C - 4097, C - 4096, C - 4095, C - 1, C, C + 5}):
            want = 0
            for l in range(p.n_layers):
                lo, hi = O.context_reach(C, p.layer_window[l])
                if lo <= pos < hi:
                    want |= 1 << l
            assert dr.dflash_layers_reading(pos, C) == want, (pos, C)
    # a prompt row older than every window is read by the full layer alone
    assert dr.dflash_layers_reading(0, 32768) == 1 << 5
    assert D.library().dflash_layers_reading(None, 0, 10) == 0


def test_prompt_scale_calls_need_a_bounded_workspace():
    # fuse and inject run calls of more than 8192 rows as passes of at most 8192 rows,
    # so the workspace for a 65536-row prompt is the one for 8192 rows; calls of up to
    # 32 rows (float64 partials) are covered by any larger request too
    dr = D.Drafter(cfg_of("9b_ctx4k"))
    a = dr.workspace_bytes(8192, 1, 4096)
    assert dr.workspace_bytes(65536, 1, 4096) == a
    assert dr.workspace_bytes(40, 1, 4096) >= dr.workspace_bytes(32, 1, 4096)
    assert dr.workspace_bytes(2048, 1, 4096) < a


def test_packed_weight_bytes_closed_form():
    # every GEMM weight once, its output columns padded to tiles of 32 rows: fc, LM head,
    # and per layer [wq | wk | wv], wo, [w_gate | w_up], w_down (each 256-byte aligned)
    def tile32(n):
        return (n + 31) // 32 * 32

    def align(b):
        return (b + 255) // 256 * 256

    for name in ("9b_ctx4k", "dflash2_x16", "tiny_f32"):
        p = wl.preset(name)
        es = 4 if p.dtype == "f32" else 2
        h, nq, nkv, I = p.hidden, p.n_q_heads * p.head_dim, p.n_kv_heads * p.head_dim, p.intermediate
        want = align(tile32(h) * p.n_taps * h * es) + align(tile32(p.vocab) * h * es)
        want += p.n_layers * (align(tile32(nq + 2 * nkv) * h * es) + align(tile32(h) * nq * es) +
                              align(tile32(2 * I) * h * es) + align(tile32(h) * I * es))
        assert D.Drafter(cfg_of(name)).packed_weight_bytes() == want, name
    dr = D.Drafter(cfg_of("tiny_f32"))
    assert D.library().dflash_pack_weights(dr.h, None, 0, None) == -5      # nothing bound yet
