"""Seeded synthetic workloads for the Ulysses 4D relayout.

This module only names geometries and draws random inputs.  It holds none
of the relayout's arithmetic: the GPU library and the CPU oracle each
compute the result from these inputs on their own.

Geometries follow the shapes the pages talk about: the video-DiT attention
operand of the fast-ulysses pages (Wan 720p, bf16: 75,600 tokens, 40 heads,
head dim 128, split over 8 ranks), and the FastVideo GB200 geometry
(250,000 tokens, 56 heads, head dim 128, sequence parallelism of four, a
1 GiB window per rank, one batch plane at a time).  Synthetic N(0, 1)
tensors stand in for real activations; the relayout moves bytes and does
not depend on their values.
"""
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

try:  # torch supplies device memory and the seeded device generator
    import torch
except ImportError:  # pragma: no cover - the oracle tests run without torch
    torch = None


DTYPES = ("bf16", "fp16", "fp32", "fp8_e4m3", "fp8_e5m2", "int8", "uint8")
ELEM_BYTES = {"bf16": 2, "fp16": 2, "fp32": 4, "fp8_e4m3": 1, "fp8_e5m2": 1,
              "int8": 1, "uint8": 1}


def torch_dtype(name):
    return {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32,
            "fp8_e4m3": torch.float8_e4m3fn, "fp8_e5m2": torch.float8_e5m2,
            "int8": torch.int8, "uint8": torch.uint8}[name]


def even_splits(total: int, world: int) -> List[int]:
    if total % world:
        raise ValueError(f"{total} does not split evenly over {world} ranks")
    return [total // world] * world


def seeded_partition(seed: int, total: int, world: int) -> List[int]:
    """A random partition of `total` into `world` parts, each >= 1.

    W-1 distinct cut points drawn from [1, total) with numpy's default
    generator, sorted; the parts are the gaps between them.
    """
    rng = np.random.default_rng(seed)
    cuts = np.sort(rng.choice(np.arange(1, total), world - 1, replace=False))
    parts = np.diff(np.concatenate([[0], cuts, [total]]))
    return [int(v) for v in parts]


@dataclass
class Workload:
    name: str
    world: int
    b: int
    d: int
    seq_splits: List[int]
    head_splits: List[int]
    dtypes: List[str] = field(default_factory=lambda: ["bf16"])
    seed: int = 0
    window_cap_bytes: int = 0
    fused: bool = False
    planes_note: Optional[str] = None

    @property
    def s_global(self):
        return sum(self.seq_splits)

    @property
    def n_global(self):
        return sum(self.head_splits)

    def shard_shape(self, mode: int, rank: int, is_dst: bool):
        """(b, S_r, n_global, d) on the sequence-sharded side, else
        (b, s_global, H_r, d).  Mode 0 goes sequence -> head sharded."""
        seq_side = (not is_dst) if mode == 0 else is_dst
        if seq_side:
            return (self.b, self.seq_splits[rank], self.n_global, self.d)
        return (self.b, self.s_global, self.head_splits[rank], self.d)


def workloads():
    """The five named workloads, smallest first."""
    return {
        "w2_tiny": Workload(
            "w2_tiny: W=2, b=1, s=2x16, n=8, d=128, bf16, mode 0 then 1",
            world=2, b=1, d=128, seq_splits=[16, 16], head_splits=[4, 4], seed=1),
        "w8_wan720p": Workload(
            "w8_wan720p: W=8, b=1, s=75,600 (9,450/rank), n=40 (5/rank), d=128, bf16",
            world=8, b=1, d=128, seq_splits=even_splits(75600, 8),
            head_splits=even_splits(40, 8), seed=2),
        "w7_uneven": Workload(
            "w7_uneven: W=7, b=2, s=75,597 seeded partition, n=40 as 6,6,6,6,6,5,5, d=128",
            world=7, b=2, d=128, seq_splits=seeded_partition(3, 75597, 7),
            head_splits=[6, 6, 6, 6, 6, 5, 5], dtypes=["bf16", "fp32", "fp8_e4m3", "int8"],
            seed=3),
        "w4_qkv_chunked": Workload(
            "w4_qkv_chunked: W=4, 3 planes (Q,K,V) as batch, s=250,000 (62,500/rank), "
            "n=56 (14/rank), d=128, bf16, 1 GiB window cap",
            world=4, b=3, d=128, seq_splits=even_splits(250000, 4),
            head_splits=even_splits(56, 4), seed=4, window_cap_bytes=1 << 30),
        "w8_fused_qknorm_rope": Workload(
            "w8_fused_qknorm_rope: W=8, q,k,v each b=1, s=75,600, n=40, d=128, bf16; "
            "RMSNorm eps=1e-6, RoPE theta=1e4",
            world=8, b=1, d=128, seq_splits=even_splits(75600, 8),
            head_splits=even_splits(40, 8), seed=5, fused=True),
    }


# ---------------------------------------------------------------------------
# Random tensors
# ---------------------------------------------------------------------------

def _generator(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def random_tensor(shape, dtype_name, gen, device):
    """bf16/fp16/fp32: N(0, 1) drawn in fp32 and converted by torch.
    fp8 and the integer types: uniform random bytes, every bit pattern
    (NaN encodings included for fp8)."""
    if dtype_name in ("bf16", "fp16", "fp32"):
        x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        return x.to(torch_dtype(dtype_name))
    raw = torch.randint(0, 256, shape, generator=gen, device=device, dtype=torch.uint8)
    return raw.view(torch_dtype(dtype_name))


def make_shards(wl: Workload, mode: int, dtype_name: str, seed: int, device="cpu"):
    """The W source shards of `mode`, each its own contiguous allocation."""
    gen = _generator(seed, device)
    return [random_tensor(wl.shard_shape(mode, r, False), dtype_name, gen, device)
            for r in range(wl.world)]


def make_gamma(d: int, seed: int, device="cpu"):
    """RMSNorm gain ~ U(0.5, 1.5), fp32, one value per element of d."""
    gen = _generator(seed, device)
    return torch.rand(d, generator=gen, device=device, dtype=torch.float32) + 0.5


def index_coded_shards(wl: Workload, mode: int):
    """int32 shards whose every element holds a distinct code of its own
    source coordinates (rank, bi, s, h, e), for brute-force checks."""
    out = []
    for r in range(wl.world):
        shape = wl.shard_shape(mode, r, False)
        n = int(np.prod(shape))
        if n >= (1 << 27) or r >= 16:
            raise ValueError("index coding holds shards below 2^27 elements and 16 ranks")
        out.append((np.arange(n, dtype=np.int64) + (r << 27)).astype(np.int32).reshape(shape))
    return out
