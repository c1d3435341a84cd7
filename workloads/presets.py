"""The five workload presets of the draft round (shapes only).

T1 tiny fp32 parity case; T2 9B-shaped single stream at 4K context; T3 the same
drafter over a 32K served span with sliding layers; T4 a DFlash2-shaped
16-stream lane round; T5 a long-context 4-stream round.
"""
from dataclasses import dataclass, field
from typing import List, Optional


@dataclass
class Preset:
    name: str
    dtype: str                 # "f32" or "bf16": weights, activations and caches
    hidden: int
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    n_taps: int
    tap_layer_ids: List[int]
    target_n_layers: int
    block_size: int
    layer_window: List[int]    # 0 = full attention, W > 0 = sliding window W
    n_streams: int
    ctx_spec: object           # int, list of ints, or ("uniform", lo, hi)
    accept_spec: object        # ("uniform",) | ("geometric", p) | ("full",)
    seed: int
    rope_theta: float = 1.0e6
    rms_eps: float = 1.0e-6
    page_size: int = 16
    mask_token_id: Optional[int] = None
    note: str = ""
    # True: the streams' existing context is built as a round builds its new rows,
    # seeded tap planes fused and injected (each side with its own fuse + inject);
    # False: seeded N(0, 1) K/V rows written straight into the cache.
    context_from_taps: bool = False

    def __post_init__(self):
        if self.mask_token_id is None:
            self.mask_token_id = self.vocab - 1

    @property
    def group(self):
        return self.n_q_heads // self.n_kv_heads

    def n_tensors(self):
        """Named drafter tensors: eleven a layer plus fc, hidden_norm, norm."""
        return 11 * self.n_layers + 3


PRESETS = {
    "tiny_f32": Preset(
        name="tiny_f32", dtype="f32", hidden=256, n_layers=2, n_q_heads=4,
        n_kv_heads=2, head_dim=64, intermediate=768, vocab=2048, n_taps=3,
        tap_layer_ids=[2, 5, 7], target_n_layers=8, block_size=8,
        layer_window=[32, 0], n_streams=1, ctx_spec=128,
        accept_spec=("uniform",), seed=1001, context_from_taps=True,
        note="tiny fp32 round: hidden 256, 2 layers (sliding 32, full), block 8, ctx 128, vocab 2048"),
    "9b_ctx4k": Preset(
        name="9b_ctx4k", dtype="bf16", hidden=4096, n_layers=6, n_q_heads=32,
        n_kv_heads=8, head_dim=128, intermediate=12288, vocab=151936, n_taps=8,
        tap_layer_ids=[1, 5, 9, 13, 17, 21, 25, 29], target_n_layers=32,
        block_size=16, layer_window=[0] * 6, n_streams=1, ctx_spec=4096,
        accept_spec=("full",), seed=1002, context_from_taps=True,
        note="9B-shaped v1 drafter, 8 taps, block 16, ctx 4096, all layers full"),
    "9b_ctx32k": Preset(
        name="9b_ctx32k", dtype="bf16", hidden=4096, n_layers=6, n_q_heads=32,
        n_kv_heads=8, head_dim=128, intermediate=12288, vocab=151936, n_taps=8,
        tap_layer_ids=[1, 5, 9, 13, 17, 21, 25, 29], target_n_layers=32,
        block_size=16, layer_window=[4096] * 5 + [0], n_streams=1,
        ctx_spec=32768, accept_spec=("full",), seed=1003,
        note="9B-shaped drafter over a 32K span: 5 sliding (4096) + 1 full layer"),
    "dflash2_x16": Preset(
        name="dflash2_x16", dtype="bf16", hidden=5120, n_layers=5, n_q_heads=40,
        n_kv_heads=8, head_dim=128, intermediate=17408, vocab=151936, n_taps=5,
        tap_layer_ids=[5, 19, 33, 47, 61], target_n_layers=64, block_size=16,
        layer_window=[0] * 5, n_streams=16, ctx_spec=("uniform", 1024, 8192),
        accept_spec=("uniform",), seed=1004,
        note="DFlash2-shaped lane round: hidden 5120, 5 raw taps, 16 streams, ctx U{1024..8192}"),
    "9b_long_x4": Preset(
        name="9b_long_x4", dtype="bf16", hidden=4096, n_layers=6, n_q_heads=32,
        n_kv_heads=8, head_dim=128, intermediate=12288, vocab=151936, n_taps=8,
        tap_layer_ids=[1, 5, 9, 13, 17, 21, 25, 29], target_n_layers=32,
        block_size=16, layer_window=[4096] * 5 + [0], n_streams=4,
        ctx_spec=[131072, 65536, 32768, 16384], accept_spec=("geometric", 1.0 / 7.0),
        seed=1005,
        note="long-context 4-stream round: ctx 131072/65536/32768/16384, 5 sliding + 1 full"),
}

# Short aliases by position in the preset list (T1..T5).
_ORDER = ["tiny_f32", "9b_ctx4k", "9b_ctx32k", "dflash2_x16", "9b_long_x4"]


def preset(name_or_index):
    if isinstance(name_or_index, int):
        return PRESETS[_ORDER[name_or_index]]
    return PRESETS[name_or_index]


def small_variant(base: Preset, **over) -> Preset:
    """A copy of a preset with some fields replaced (used for scaled-down cases)."""
    d = dict(base.__dict__)
    d.update(over)
    if "vocab" in over and "mask_token_id" not in over:
        d["mask_token_id"] = over["vocab"] - 1
    return Preset(**d)
