"""Seeded synthetic BRA workloads (shapes and input generators).

This module only draws inputs; it holds none of the attention arithmetic,
and both the HIP path's tests and the CPU oracle consume what it draws.

The shapes follow the BiFormer pages: stage maps of a 224x224 image at
S = 7 with top-k [1, 4, 16] (explainer "BiFormer Reshapes Visual Attention
with 'Bi-Level Routing'", Part 4.3 "Model Scaling Specifications" and Part
6.3 table; 64 attended tokens per query at every stage), and a dense
prediction map at S = 8 (Part 4.3: S = 8 for segmentation). Head dim 32.
No dataset or trained activation is used; the region-clustered workload
stands in for spatially coherent features.

Draw recipe (reproducibility only; parity never depends on it):
``torch.Generator('cpu').manual_seed(seed)``, ``torch.randn`` float32 of
shape [B, H, W, C] for Q, then K, then V. The clustered workload draws, in
order, region means of Q [B, S*S, C], token noise of Q [B, H, W, C], the same
two for K, then V; each token of Q (K) is its region's mean plus 0.5 times
its noise. bf16 workloads are cast (round to nearest even) after composing.

Local-context filters (``make_lce_params``): a generator seeded with
``seed + 1000`` draws the [C, 5, 5] depthwise weights as ``randn / 5`` (so a
filter applied to unit-variance values gives roughly unit variance) and the
[C] bias as ``randn / 10``, both cast to the workload's dtype. No trained
filter is used.

Output gradients for the backward pass (``make_grad_output``): a generator
seeded with ``seed + 2000`` draws ``randn`` [B, H, W, C], cast to the dtype.

Projection inputs (``make_projection``): a generator seeded with
``seed + 3000`` draws the block input X as ``randn`` [B, H, W, C], the
[3C, C] weight as ``randn / sqrt(C)`` (unit-variance outputs) and the [3C]
bias as ``randn / 10``, all cast to the dtype.
"""

from __future__ import annotations

from dataclasses import dataclass, asdict

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    W: int
    C: int
    heads: int
    S: int
    topk: int
    dtype: str  # "f32" or "bf16"
    seed: int
    content: str = "iid"  # "iid" or "clustered"

    @property
    def R(self) -> int:
        return self.S * self.S

    @property
    def n(self) -> int:
        return (self.H // self.S) * (self.W // self.S)

    @property
    def d(self) -> int:
        return self.C // self.heads

    @property
    def kv(self) -> int:
        return self.topk * self.n

    @property
    def tokens(self) -> int:
        return self.B * self.H * self.W

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def asdict(self) -> dict:
        return asdict(self)


WORKLOADS = [
    Workload("tiny-b1-16x16-c32-h1-s4-k2-f32", 1, 16, 16, 32, 1, 4, 2, "f32", 0),
    Workload("stage1-b64-56x56-c64-h2-s7-k1-bf16", 64, 56, 56, 64, 2, 7, 1, "bf16", 1),
    Workload("stage2-b64-28x28-c128-h4-s7-k4-bf16", 64, 28, 28, 128, 4, 7, 4, "bf16", 2),
    Workload("stage3-b64-14x14-c256-h8-s7-k16-bf16", 64, 14, 14, 256, 8, 7, 16, "bf16", 3),
    Workload("dense-b2-128x128-c64-h2-s8-k4-bf16-clustered", 2, 128, 128, 64, 2, 8, 4, "bf16", 4, "clustered"),
]

# Detection-shaped maps at S = 16 (explainer Part 4.3: S = 16 for object
# detection; paper summary Appendix C: larger S for dense prediction): 256
# regions per image, the routing over 256 candidates. Measured beside the
# five workloads above; not part of them.
DETECTION = [
    Workload("det-b2-128x128-c64-h2-s16-k4-bf16", 2, 128, 128, 64, 2, 16, 4, "bf16", 5),
    Workload("det-b2-64x64-c64-h2-s16-k8-bf16-clustered", 2, 64, 64, 64, 2, 16, 8, "bf16", 6, "clustered"),
]

BY_NAME = {w.name: w for w in WORKLOADS + DETECTION}

# The headline workload: stage-1 shape, 56x56 map, S = 7.
HEADLINE = WORKLOADS[1]


def custom(B, H, W, C, heads, S, topk, dtype="bf16", seed=0, content="iid", name=None) -> Workload:
    """An ad-hoc workload (tests of ragged and edge shapes)."""
    name = name or f"custom-b{B}-{H}x{W}-c{C}-h{heads}-s{S}-k{topk}-{dtype}-{content}-seed{seed}"
    return Workload(name, B, H, W, C, heads, S, topk, dtype, seed, content)


def _expand_regions(means: torch.Tensor, H: int, W: int, S: int) -> torch.Tensor:
    """[B, S*S, C] region means -> [B, H, W, C] with each token set to its
    region's mean (regions row-major over the S x S grid)."""
    B, R, C = means.shape
    g = means.reshape(B, S, S, C)
    g = g.repeat_interleave(H // S, dim=1).repeat_interleave(W // S, dim=2)
    return g


def make_inputs(w: Workload):
    """Draw (Q, K, V) on the CPU in the workload's dtype, [B, H, W, C]."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(w.seed))
    shape = (w.B, w.H, w.W, w.C)
    if w.content == "iid":
        q = torch.randn(shape, generator=gen, dtype=torch.float32)
        k = torch.randn(shape, generator=gen, dtype=torch.float32)
        v = torch.randn(shape, generator=gen, dtype=torch.float32)
    elif w.content == "clustered":
        mq = torch.randn((w.B, w.R, w.C), generator=gen, dtype=torch.float32)
        nq = torch.randn(shape, generator=gen, dtype=torch.float32)
        mk = torch.randn((w.B, w.R, w.C), generator=gen, dtype=torch.float32)
        nk = torch.randn(shape, generator=gen, dtype=torch.float32)
        v = torch.randn(shape, generator=gen, dtype=torch.float32)
        q = _expand_regions(mq, w.H, w.W, w.S) + 0.5 * nq
        k = _expand_regions(mk, w.H, w.W, w.S) + 0.5 * nk
    else:
        raise ValueError(f"unknown content kind {w.content!r}")
    dt = w.torch_dtype
    return q.to(dt).contiguous(), k.to(dt).contiguous(), v.to(dt).contiguous()


def make_lce_params(w: Workload):
    """Draw (weight [C, 5, 5], bias [C]) of the local-context depthwise
    filter on the CPU in the workload's dtype."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(w.seed) + 1000)
    weight = torch.randn((w.C, 5, 5), generator=gen, dtype=torch.float32) / 5.0
    bias = torch.randn((w.C,), generator=gen, dtype=torch.float32) / 10.0
    dt = w.torch_dtype
    return weight.to(dt).contiguous(), bias.to(dt).contiguous()


def make_grad_output(w: Workload):
    """Draw dL/dO [B, H, W, C] on the CPU in the workload's dtype."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(w.seed) + 2000)
    g = torch.randn((w.B, w.H, w.W, w.C), generator=gen, dtype=torch.float32)
    return g.to(w.torch_dtype).contiguous()


def make_projection(w: Workload):
    """Draw (X [B, H, W, C], Wqkv [3C, C], bqkv [3C]) on the CPU in the
    workload's dtype."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(w.seed) + 3000)
    x = torch.randn((w.B, w.H, w.W, w.C), generator=gen, dtype=torch.float32)
    wq = torch.randn((3 * w.C, w.C), generator=gen, dtype=torch.float32) / float(w.C) ** 0.5
    bq = torch.randn((3 * w.C,), generator=gen, dtype=torch.float32) / 10.0
    dt = w.torch_dtype
    return x.to(dt).contiguous(), wq.to(dt).contiguous(), bq.to(dt).contiguous()


def to_f64(t: torch.Tensor):
    """Exact upcast of a CPU/GPU tensor (fp32 or bf16) to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()
