"""Seeded synthetic inputs for the forward and decode workloads.

Random numbers only: this module holds none of the attention arithmetic.  It
serves the tests, the benchmark and the smoke check alike.  Draw order is
fixed: every q head, then every k head, then every v head, each as an
[N, dim] float32 standard-normal draw from one generator seeded with `seed`,
then transformed (ReLU for q and k where the workload says so, then a scale)
and rounded to the storage dtype (round-to-nearest-even by torch).
Decode steps draw q, k, v for step 0, then step 1, and so on.  Upstream
gradients for the backward pass are N(0,1) draws of their own generator.
"""
import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    dv: int
    block: int
    dtype: torch.dtype
    relu_qk: bool     # q, k = ReLU(N(0,1)) * scale; otherwise N(0,1) * scale
    scale_v: bool     # v scaled like q and k (the fp32 case) or left N(0,1)
    steps: int = 0    # decode steps after an N-token prefix


# The five workloads of the method: sizes follow the pages' 128 query heads
# over 32 KV heads and 1M-token context, head size 128, 64-token blocks.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 1, 1, 256, 64, 64, 64, torch.float32, False, True),
    "mha_4k": Workload("mha_4k", 2, 8, 8, 4096, 128, 128, 64, torch.bfloat16, True, False),
    "gqa_64k": Workload("gqa_64k", 1, 128, 32, 65536, 128, 128, 64, torch.bfloat16, True, False),
    "gqa_1m": Workload("gqa_1m", 1, 128, 32, 1048576, 128, 128, 64, torch.bfloat16, True, False),
    "decode_256": Workload("decode_256", 256, 128, 32, 8192, 128, 128, 64, torch.bfloat16, True, False, 1000),
    # the same 1M-token GQA shape at head size 64, and a 1M-token MHA shape at
    # 64 (not on the pages: a second head size of the matrix-core kernels, and
    # one query head per KV head)
    "gqa_1m_d64": Workload("gqa_1m_d64", 1, 128, 32, 1048576, 64, 64, 64, torch.bfloat16, True, False),
    "mha_1m_d64": Workload("mha_1m_d64", 1, 32, 32, 1048576, 64, 64, 64, torch.bfloat16, True, False),
}


def _fill(dst, gen, relu, scale):
    """Fill dst [B, H, N, dim] head by head from gen (float32 draw on dst's device)."""
    B, H, N, dim = dst.shape
    for b in range(B):
        for h in range(H):
            x = torch.randn((N, dim), generator=gen, device=dst.device, dtype=torch.float32)
            if relu:
                x.clamp_(min=0.0)
            if scale != 1.0:
                x.mul_(scale)
            dst[b, h].copy_(x)
            del x


def make_qkv(w, device, seed=0, N=None, B=None):
    """q [B,Hq,N,d], k [B,Hkv,N,d], v [B,Hkv,N,dv] for workload w (N, B overridable)."""
    N = w.N if N is None else N
    B = w.B if B is None else B
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    sq = 1.0 / math.sqrt(w.d)
    q = torch.empty((B, w.Hq, N, w.d), dtype=w.dtype, device=device)
    k = torch.empty((B, w.Hkv, N, w.d), dtype=w.dtype, device=device)
    v = torch.empty((B, w.Hkv, N, w.dv), dtype=w.dtype, device=device)
    _fill(q, gen, w.relu_qk, sq)
    _fill(k, gen, w.relu_qk, sq)
    _fill(v, gen, False, sq if w.scale_v else 1.0)
    return q, k, v


def make_decode_steps(w, device, seed=1, steps=None, B=None):
    """Per-step decode inputs: q [T,B,Hq,d], k [T,B,Hkv,d], v [T,B,Hkv,dv]."""
    T = w.steps if steps is None else steps
    B = w.B if B is None else B
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    sq = 1.0 / math.sqrt(w.d)
    q = torch.empty((T, B, w.Hq, w.d), dtype=w.dtype, device=device)
    k = torch.empty((T, B, w.Hkv, w.d), dtype=w.dtype, device=device)
    v = torch.empty((T, B, w.Hkv, w.dv), dtype=w.dtype, device=device)
    for t in range(T):
        for dst, relu, sc in ((q[t], w.relu_qk, sq), (k[t], w.relu_qk, sq), (v[t], False, 1.0)):
            x = torch.randn(dst.shape, generator=gen, device=device, dtype=torch.float32)
            if relu:
                x.clamp_(min=0.0)
            if sc != 1.0:
                x.mul_(sc)
            dst.copy_(x)
    return q, k, v


def make_grad(shape, device, seed=3, dtype=torch.bfloat16, chunk_rows=1 << 20):
    """An upstream gradient dL/do of `shape` [B, H, N, dv]: N(0,1) draws head
    by head (rows in chunks of chunk_rows), rounded to dtype."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = torch.empty(shape, dtype=dtype, device=device)
    B, H, N, dv = shape
    for b in range(B):
        for h in range(H):
            for a in range(0, N, chunk_rows):
                e = min(a + chunk_rows, N)
                out[b, h, a:e].copy_(torch.randn((e - a, dv), generator=gen, device=device, dtype=torch.float32))
    return out


def random_state(shape, device, seed=2, scale=1.0):
    """A float32 initial state drawn N(0,1) * scale (for resume and decode tests)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * scale
