"""Named synthetic KV-cache workloads.

The pages give no workload of their own (the abstract of *Beyond Compression
Ratio: High-Throughput KV Compression for Disaggregated LLM Serving* speaks
only of "evaluated workloads"), so these presets stand in for KV caches of
well-known model shapes.  Values are synthetic: Gaussian with a few
outlier channels in K -- the kind of distribution a randomized Hadamard
transform is meant to flatten before quantization.
"""

from dataclasses import dataclass, replace
import math


@dataclass(frozen=True)
class Preset:
    name: str
    layers: int
    kv_heads: int
    head_dim: int
    dtype: str                 # "bf16" or "fp16"
    bits_k: int
    bits_v: int
    group: int
    tokens: int = 0            # contiguous layout only
    k_sigma: float = 1.0       # standard deviation of K
    v_sigma: float = 1.0       # standard deviation of V
    k_outlier_channels: int = 0
    outlier_scale: float = 20.0
    spike_prob: float = 0.0    # Bernoulli spikes on K and V
    spike_scale: float = 50.0
    seed: int = 0              # sign seed of the transform
    paged: bool = False
    num_requests: int = 0
    len_min: int = 0
    len_max: int = 0
    block_size: int = 16
    spare_blocks: float = 0.05  # unused pool blocks, as a fraction of used ones

    def with_(self, **kw) -> "Preset":
        return replace(self, **kw)

    @property
    def elements(self) -> int:
        if self.paged:
            raise ValueError("element count of a paged preset depends on the lengths")
        return self.layers * 2 * self.tokens * self.kv_heads * self.head_dim

    @property
    def shape(self):
        return (self.layers, 2, self.tokens, self.kv_heads, self.head_dim)


PRESETS = {
    # 1 layer, K and V, 256 tokens, 2 heads, head_dim 64, fp16 N(0,1),
    # 2 fixed K outlier channels x20, seed 0, 4-bit, group 64.
    "tiny": Preset("tiny", layers=1, kv_heads=2, head_dim=64, dtype="fp16",
                   bits_k=4, bits_v=4, group=64, tokens=256,
                   k_outlier_channels=2),
    # Llama-3-8B-shaped: 32 x {K,V} x 4096 x 8 x 128 bf16 (512 MiB);
    # K N(0,1) with 4 outlier channels per layer x20, V N(0, 0.5) (variance).
    "llama3_8b_4k": Preset("llama3_8b_4k", layers=32, kv_heads=8, head_dim=128,
                           dtype="bf16", bits_k=4, bits_v=4, group=128, tokens=4096,
                           k_outlier_channels=4, v_sigma=math.sqrt(0.5)),
    # same shape at 32768 tokens (4 GiB), 2-bit, group 32.
    "llama3_8b_32k": Preset("llama3_8b_32k", layers=32, kv_heads=8, head_dim=128,
                            dtype="bf16", bits_k=2, bits_v=2, group=32, tokens=32768,
                            k_outlier_channels=4, v_sigma=math.sqrt(0.5)),
    # Llama-3-70B-shaped: 80 x {K,V} x 16384 x 8 x 128 bf16 (5 GiB), N(0,1),
    # 4 K outlier channels x20, 0.1% spikes x50 on K and V; 4-bit, group 128.
    "llama3_70b_16k": Preset("llama3_70b_16k", layers=80, kv_heads=8, head_dim=128,
                             dtype="bf16", bits_k=4, bits_v=4, group=128, tokens=16384,
                             k_outlier_channels=4, spike_prob=1e-3),
    # Paged Qwen-7B-shaped: 28 layers, 4 heads, head_dim 128, bf16, 64 requests
    # of U[512, 8192] tokens in 16-token blocks; K 2-bit, V 4-bit, group 64.
    "qwen7b_paged": Preset("qwen7b_paged", layers=28, kv_heads=4, head_dim=128,
                           dtype="bf16", bits_k=2, bits_v=4, group=64,
                           k_outlier_channels=4, v_sigma=math.sqrt(0.5),
                           paged=True, num_requests=64, len_min=512, len_max=8192),
}

ORDER = ["tiny", "llama3_8b_4k", "llama3_8b_32k", "llama3_70b_16k", "qwen7b_paged"]


def preset(name_or_index) -> Preset:
    """A preset by name or by 1-based position in ``ORDER``."""
    if isinstance(name_or_index, int):
        return PRESETS[ORDER[name_or_index - 1]]
    return PRESETS[name_or_index]
