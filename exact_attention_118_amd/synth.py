"""Seeded synthetic inputs for the attention workloads (no attention arithmetic here).

Shared by the tests, the benchmark and the CPU oracle checks: both sides of a
parity test receive the very same tensors from here.

Recipe: a ``torch.Generator`` on the target device seeded with ``seed``; draw
order Q, K, V, dO; each an i.i.d. standard normal float32 tensor of shape
[B, H, Nq or Nk, d]; Q and K are multiplied by ``qk_mult`` before the cast to
the compute dtype (round-to-nearest-even for bf16).  Draws on a GPU use that
device's generator, so their values differ from CPU draws with the same seed;
each is reproducible on its own.
"""

from __future__ import annotations

from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    dtype: torch.dtype
    qk_mult: float = 1.0
    backward: bool = True

    @property
    def scale(self) -> float:
        return 1.0 / float(self.d) ** 0.5

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # tiny fp32 forward: B=1, H=2, N=128, d=64, non-causal
    "tiny_fp32": Workload("tiny_fp32", 1, 2, 128, 128, 64, False, torch.float32, backward=False),
    # forward+backward, bf16, B=4, H=16, N=1024, d=64, causal
    "b4h16n1024d64_causal": Workload("b4h16n1024d64_causal", 4, 16, 1024, 1024, 64, True, torch.bfloat16),
    # forward+backward, bf16, B=2, H=16, N=4096, d=128, causal and non-causal
    "b2h16n4096d128_causal": Workload("b2h16n4096d128_causal", 2, 16, 4096, 4096, 128, True, torch.bfloat16),
    "b2h16n4096d128": Workload("b2h16n4096d128", 2, 16, 4096, 4096, 128, False, torch.bfloat16),
    # the same causal shape with fp16 inputs
    "b2h16n4096d128_causal_fp16": Workload("b2h16n4096d128_causal_fp16", 2, 16, 4096, 4096, 128, True,
                                           torch.float16),
    # long sequence, bf16, B=1, H=32, N=8192, d=128, causal, Q and K scaled by 3
    "b1h32n8192d128_causal": Workload("b1h32n8192d128_causal", 1, 32, 8192, 8192, 128, True,
                                      torch.bfloat16, qk_mult=3.0),
    # decode-shaped forward: B=16, H=32, one query against 16384 keys, d=128
    "decode_b16h32k16384d128": Workload("decode_b16h32k16384d128", 16, 32, 1, 16384, 128, False,
                                        torch.bfloat16, backward=False),
}


def make_inputs(w: Workload, seed: int = 0, device="cpu", with_grad_out: bool | None = None):
    """Return dict with Q, K, V (and dO when the workload has a backward pass)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    if with_grad_out is None:
        with_grad_out = w.backward

    def draw(n):
        return torch.randn((w.B, w.H, n, w.d), generator=g, device=device, dtype=torch.float32)

    Q = draw(w.Nq)
    K = draw(w.Nk)
    V = draw(w.Nk)
    out = {}
    if w.qk_mult != 1.0:
        Q.mul_(w.qk_mult)
        K.mul_(w.qk_mult)
    out["Q"] = Q.to(w.dtype).contiguous()
    del Q
    out["K"] = K.to(w.dtype).contiguous()
    del K
    out["V"] = V.to(w.dtype).contiguous()
    del V
    if with_grad_out:
        out["dO"] = draw(w.Nq).to(w.dtype).contiguous()
    return out


def make_bias(B: int, H: int, Nq: int, Nk: int, dtype, seed: int = 0, device="cpu",
              per_batch: bool = True, per_head: bool = True, row_stride: int | None = None,
              drop: float = 0.0, pad_value: float = float("nan")):
    """Seeded additive bias, returned as a view of shape [B or 1, H or 1, Nq, Nk].

    Recipe: a ``torch.Generator`` on ``device`` seeded with ``seed``; an i.i.d.
    standard normal float32 tensor of shape [B', H', Nq, row_stride] (B' = B if
    ``per_batch`` else 1, H' likewise; row_stride defaults to Nk); then, when
    ``drop`` > 0, a second uniform draw of the same shape sets each entry with
    u < drop to -inf, except key 0 of every row, so that every row keeps a
    finite entry; the columns past Nk are set to ``pad_value`` (NaN by
    default: they are not part of the problem); cast to ``dtype``.  A
    dimension of size 1 is meant to broadcast.
    """
    sq = Nk if row_stride is None else row_stride
    if sq < Nk:
        raise ValueError("row_stride must be >= Nk")
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    shape = (B if per_batch else 1, H if per_head else 1, Nq, sq)
    b = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if drop > 0.0:
        u = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
        u[..., 0] = 1.0
        b[u < drop] = float("-inf")
    b[..., Nk:] = pad_value
    return b.to(dtype)[..., :Nk]
