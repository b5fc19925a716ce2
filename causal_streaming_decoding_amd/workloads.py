"""The synthetic workloads the window step is tested and measured on.

Each workload is named by what it is. The shapes follow the backbones the WeDLM
pages name (Qwen2.5-7B and Qwen3-8B attention shapes; sai.science review,
"Summary"), with a paged KV cache of 16-token pages (mlsanity.com page,
"Builds on": PagedAttention). The pages publish no benchmark inputs; these are
synthetic stand-ins with the sizes and value distributions listed here.
"""

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str              # "f32" or "bf16": storage type of every tensor on the path
    n_layers: int
    B: int
    Hq: int
    Hkv: int
    D: int
    theta: float
    W: int
    V: int
    lam: float
    tau: float
    prefix: tuple           # ("fixed", L), ("uniform", lo, hi) inclusive, or ("list", (L_0, ..))
    fill: tuple             # ("count", n) | ("frac", lo, hi) one draw | ("frac_per_seq", lo, hi) | ("none",)
    spike: tuple            # ("slots", n, mag) | ("all_uniform", lo, hi) | ("prob", p, lo, hi) | ("none",)
    steps: int = 1          # window steps of one run (the streaming loop runs many)
    page_size: int = 16
    logit_sigma: float = 2.0
    seed: int = 0
    min_fill: int = 1
    mask_id: int = -1
    notes: str = field(default="", compare=False)

    @property
    def g(self):
        return self.Hq // self.Hkv


TINY_FP32 = Workload(
    name="tiny_fp32_L40_W8", dtype="f32", n_layers=1, B=1, Hq=2, Hkv=1, D=64, theta=1e4, W=8,
    V=512, lam=0.1, tau=1.0, prefix=("fixed", 40), fill=("count", 3), spike=("slots", 4, 8.0),
    notes="one sequence, 2 query heads on 1 kv head, 3 of 8 slots filled, +8 spike in half the slots")

QWEN3_8B_BS1 = Workload(
    name="qwen3_8b_bs1_L2048_W16", dtype="bf16", n_layers=1, B=1, Hq=32, Hkv=8, D=128, theta=1e6,
    W=16, V=151936, lam=0.1, tau=1.0, prefix=("fixed", 2048), fill=("frac", 0.25, 0.75),
    spike=("all_uniform", 6.0, 12.0),
    notes="one layer, one sequence, 25-75% of the window filled, a +6..+12 spike per slot")

QWEN25_7B_RAGGED = Workload(
    name="qwen25_7b_bs16_ragged_W32", dtype="bf16", n_layers=1, B=16, Hq=28, Hkv=4, D=128,
    theta=1e6, W=32, V=152064, lam=0.05, tau=0.8, prefix=("uniform", 512, 4096),
    fill=("frac_per_seq", 0.0, 1.0), spike=("all_uniform", 0.0, 12.0),
    notes="ragged prefixes 512..4096 with scattered pages, GQA group of 7")

QWEN3_8B_LONG = Workload(
    name="qwen3_8b_bs4_L32768_W16", dtype="bf16", n_layers=1, B=4, Hq=32, Hkv=8, D=128, theta=1e6,
    W=16, V=151936, lam=0.1, tau=1.0, prefix=("fixed", 32768), fill=("count", 8), spike=("none",),
    notes="long context, KV-read bound, half the window filled, no spikes")

QWEN3_8B_STREAM = Workload(
    name="qwen3_8b_36L_bs16_L1024_W16_stream256", dtype="bf16", n_layers=36, B=16, Hq=32, Hkv=8,
    D=128, theta=1e6, W=16, V=151936, lam=0.1, tau=1.0, prefix=("fixed", 1024), fill=("none",),
    spike=("prob", 0.7, 6.0, 12.0), steps=256,
    notes="36 independent layers' caches, 256 streaming steps from an all-mask window")

ALL = [TINY_FP32, QWEN3_8B_BS1, QWEN25_7B_RAGGED, QWEN3_8B_LONG, QWEN3_8B_STREAM]
BY_NAME = {w.name: w for w in ALL}
