"""Seeded input recipes (torch CPU generator, float32 draws, RNE cast).

Every tensor is drawn with torch.Generator('cpu').manual_seed(seed) and
torch.randn/torch.rand in float32, in the order stated per recipe, combined in
float32 and then cast to the storage dtype with torch's round-to-nearest-even.
The shapes are the ones the prime-rl NS microbenchmark table lists (square
4096² and 8192², the 4096×14336 MLP weight, the 128×1536×2048 and
32×7168×2048 expert stacks) plus a one-rank expert shard (16 of 128 experts,
the local-update shape in the prime-rl "Summary", item 2) and a small 256×512
case.  The pages do not state their input distributions; the recipes below are
the readings used here.
"""

from dataclasses import dataclass
import math

import torch


def gaussian(shape, seed, dtype=torch.float32, scale=1.0):
    """iid N(0, 1) * scale in float32 from a fresh seeded CPU generator, cast to dtype."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    if scale != 1.0:
        x = x * scale
    return x.to(dtype)


@dataclass(frozen=True)
class Workload:
    name: str
    shape: tuple
    dtype: torch.dtype
    seed: int
    recipe: str

    @property
    def batch(self):
        return math.prod(self.shape[:-2]) if len(self.shape) > 2 else 1

    @property
    def rows(self):
        return self.shape[-2]

    @property
    def cols(self):
        return self.shape[-1]


WORKLOADS = {
    w.name: w
    for w in [
        Workload("iid_256x512", (256, 512), torch.float32, 0,
                 "Z iid N(0,1), float32 (the bf16 run casts this tensor)"),
        Workload("lowrank64_4096x4096", (4096, 4096), torch.bfloat16, 1,
                 "U[4096,64], V[4096,64], Z[4096,4096] iid N(0,1) drawn in that "
                 "order; X = U Vᵀ + 0.1 Z in float32, cast to bf16"),
        Workload("mlp_4096x14336", (4096, 14336), torch.bfloat16, 2,
                 "Z[4096,14336], U[4096,32], V[14336,32] iid N(0,1) in that "
                 "order; X = Z + U Vᵀ in float32, cast to bf16"),
        Workload("mlp_14336x4096", (14336, 4096), torch.bfloat16, 2,
                 "the transpose (made contiguous) of mlp_4096x14336"),
        Workload("experts16_1536x2048", (16, 1536, 2048), torch.bfloat16, 3,
                 "16 scales s_i = exp(U(ln 1e-3, ln 1)) drawn first, then "
                 "Z[16,1536,2048] iid N(0,1); X_i = s_i Z_i, cast to bf16"),
        Workload("experts128_1536x2048", (128, 1536, 2048), torch.bfloat16, 4,
                 "seed-4 generator, first draw: Z[128,1536,2048] iid N(0,1)"),
        Workload("experts32_7168x2048", (32, 7168, 2048), torch.bfloat16, 4,
                 "seed-4 generator, second draw: Z[32,7168,2048] iid N(0,1)"),
        Workload("square_8192x8192", (8192, 8192), torch.bfloat16, 4,
                 "seed-4 generator, third draw: Z[8192,8192] iid N(0,1)"),
        Workload("experts128_2048x768", (128, 2048, 768), torch.bfloat16, 5,
                 "seed 5: Z[128,2048,768] iid N(0,1) (the pages' sixth microbenchmark "
                 "shape; tall, Gram 768 x 768)"),
    ]
}


def workload_names():
    return list(WORKLOADS)


_seed4_cache = {}


def _seed4_stack(which):
    # The three seed-4 tensors come from ONE generator, drawn in a fixed order,
    # so a later one needs the earlier draws to have happened.
    if which not in _seed4_cache:
        g = torch.Generator("cpu").manual_seed(4)
        order = ["experts128_1536x2048", "experts32_7168x2048", "square_8192x8192"]
        for name in order:
            t = torch.randn(*WORKLOADS[name].shape, generator=g, dtype=torch.float32)
            if name == which:
                _seed4_cache.clear()
                _seed4_cache[which] = t.to(torch.bfloat16)
                break
            del t
    return _seed4_cache[which]


def make_workload(name):
    """Return the CPU tensor of the named workload (its storage dtype)."""
    w = WORKLOADS[name]
    if name == "iid_256x512":
        return gaussian(w.shape, w.seed, torch.float32)
    if name == "lowrank64_4096x4096":
        g = torch.Generator("cpu").manual_seed(w.seed)
        u = torch.randn(4096, 64, generator=g)
        v = torch.randn(4096, 64, generator=g)
        z = torch.randn(4096, 4096, generator=g)
        return (u @ v.T + 0.1 * z).to(torch.bfloat16)
    if name in ("mlp_4096x14336", "mlp_14336x4096"):
        g = torch.Generator("cpu").manual_seed(w.seed)
        z = torch.randn(4096, 14336, generator=g)
        u = torch.randn(4096, 32, generator=g)
        v = torch.randn(14336, 32, generator=g)
        x = (z + u @ v.T).to(torch.bfloat16)
        return x if name == "mlp_4096x14336" else x.T.contiguous()
    if name == "experts16_1536x2048":
        g = torch.Generator("cpu").manual_seed(w.seed)
        lo, hi = math.log(1e-3), math.log(1.0)
        s = torch.exp(lo + (hi - lo) * torch.rand(16, generator=g))
        z = torch.randn(16, 1536, 2048, generator=g)
        return (z * s.view(16, 1, 1)).to(torch.bfloat16)
    if name in ("experts128_1536x2048", "experts32_7168x2048", "square_8192x8192"):
        return _seed4_stack(name)
    if name == "experts128_2048x768":
        return gaussian(w.shape, w.seed, torch.bfloat16)
    raise KeyError(name)


# Sets of stacks for the grouped call (several leaf shapes in one call).  The
# first two use the NS table's sizes: all six of its shapes, and the 4096 and
# 14336 sizes arranged as one decoder block's matrices (four 4096 x 4096,
# one 4096 x 14336, two 14336 x 4096).  The leaf sets are synthetic small
# leaves, where one launch per stage and stack leaves the GPU underfilled.
# Stack i of a set is iid N(0, 1), seed 1000 + 32 k + i (k: the set's index),
# bf16.
GROUPED_SETS = {
    "ns_table_shapes": [(1, 4096, 4096), (1, 8192, 8192), (1, 4096, 14336), (128, 1536, 2048),
                        (128, 2048, 768), (32, 7168, 2048)],
    "block_4096_14336": [(4, 4096, 4096), (1, 4096, 14336), (2, 14336, 4096)],
    "leaves_768_3072": [(48, 768, 768), (12, 768, 3072), (12, 3072, 768)],
    "leaves_1024_4096": [(4, 1024, 1024), (1, 1024, 4096), (1, 4096, 1024)],
    "leaves_24_small": [(1, 512 + 64 * (i % 4), 512 + 128 * (i % 3)) for i in range(24)],
}


def make_grouped_set(name, dtype=torch.bfloat16):
    """CPU tensors of the named set of stacks."""
    k = list(GROUPED_SETS).index(name)
    return [gaussian(s, 1000 + 32 * k + i, dtype) for i, s in enumerate(GROUPED_SETS[name])]

