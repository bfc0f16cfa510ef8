"""The five synthetic workloads the sparse-decode path is exercised on.

Shapes follow the models the SparseEngine pages evaluate on (a GQA model with
32 query / 4 KV heads of width 128 over 48 layers, and an MLA model whose
keys are a 512-wide latent plus a 64-wide rope part), at the long contexts
those pages stress (16K to 128K tokens).  Sizes are stated here once and every
test, the bench and the smoke check read them from this table.
"""
from dataclasses import dataclass, field, replace
from typing import Tuple


@dataclass(frozen=True)
class WorkloadConfig:
    cfg_id: int
    name: str
    dtype: str                 # "f32" or "bf16": element type of q, K, V and page metadata
    batch: int
    n_q_heads: int
    n_kv_heads: int
    d_k: int
    d_v: int
    context: int               # tokens in the cache when decoding starts
    page_size: int = 16
    top_pages: int = 0         # Quest: pages kept per KV head
    snap_window: int = 0       # SnapKV observation window (last prompt tokens)
    snap_pool: int = 0         # SnapKV max-pool kernel width
    snap_budget: int = 0       # SnapKV tokens kept per KV head (window included)
    h2o_heavy: int = 0         # H2O heavy-hitter slots
    h2o_recent: int = 0        # H2O recent window
    omni_layers: int = 0       # OmniKV layer sweep depth
    omni_filters: Tuple[int, ...] = ()
    omni_top_k: int = 0
    decode_steps: int = 1
    latent: bool = False       # MLA: V is the first d_v columns of K
    scale: float = 0.0         # softmax scale; 0 means 1/sqrt(d_k)
    planted_pages: int = 0     # Quest workload: pages whose keys lean towards the query direction
    planted_region_pages: int = 0
    snap_peaks: int = 0        # SnapKV workload: planted key positions (a ladder of vote levels)
    snap_peak_spacing: int = 0
    snap_peak_levels: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def units(self) -> int:
        return self.batch * self.n_kv_heads

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale > 0 else 1.0 / float(self.d_k) ** 0.5

    def with_(self, **kw) -> "WorkloadConfig":
        return replace(self, **kw)


CONFIGS = {
    # Tiny fp32 case: everything runs on a CPU in seconds.
    0: WorkloadConfig(
        cfg_id=0, name="tiny_f32", dtype="f32", batch=2, n_q_heads=4, n_kv_heads=1,
        d_k=64, d_v=64, context=512, page_size=16, top_pages=8,
        snap_window=16, snap_pool=7, snap_budget=128, decode_steps=5),
    # Quest decode at 32K: 16 x (32q/4kv, d128), pages of 16, top-128 pages.
    1: WorkloadConfig(
        cfg_id=1, name="quest_32k", dtype="bf16", batch=16, n_q_heads=32, n_kv_heads=4,
        d_k=128, d_v=128, context=32768, page_size=16, top_pages=128, decode_steps=64,
        planted_pages=8, planted_region_pages=2048),
    # SnapKV prefill-end eviction of a 128K prompt to 8192 tokens, then decode.
    2: WorkloadConfig(
        cfg_id=2, name="snapkv_128k", dtype="bf16", batch=8, n_q_heads=32, n_kv_heads=4,
        d_k=128, d_v=128, context=131072, snap_window=32, snap_pool=7, snap_budget=8192,
        decode_steps=128, snap_peaks=1280, snap_peak_spacing=100, snap_peak_levels=40),
    # H2O (1024 heavy + 256 recent) and OmniKV (48 layers, filters 2/8/16, top-2048) at 16K.
    3: WorkloadConfig(
        cfg_id=3, name="h2o_omnikv_16k", dtype="bf16", batch=64, n_q_heads=32, n_kv_heads=4,
        d_k=128, d_v=128, context=16384, h2o_heavy=1024, h2o_recent=256,
        omni_layers=48, omni_filters=(2, 8, 16), omni_top_k=2048, decode_steps=128,
        extra={"omni_steps": 64}),
    # MLA latent cache at 128K: 32 heads share one 576-wide latent row per token.
    4: WorkloadConfig(
        cfg_id=4, name="mla_128k", dtype="bf16", batch=32, n_q_heads=32, n_kv_heads=1,
        d_k=576, d_v=512, context=131072, page_size=64, top_pages=64, decode_steps=64,
        latent=True, scale=1.0 / 192.0 ** 0.5),
}


def get_config(cfg_id: int, **overrides) -> WorkloadConfig:
    cfg = CONFIGS[cfg_id]
    return cfg.with_(**overrides) if overrides else cfg
