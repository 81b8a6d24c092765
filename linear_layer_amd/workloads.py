"""Seeded synthetic inputs for the GEMM / fully-connected workloads.

This module only draws numbers; it holds none of the product's arithmetic.
Both the GPU path (through the tests and the bench) and the CPU oracle are fed
the very same host arrays made here.

Recipe: a ``torch.Generator('cpu')`` seeded with ``100*config + tensor``
(tensor: A 0, B 1, C_in 2, bias 3), uniform values from ``2*rand - 1`` in
fp32 (so [-1, 1)), the fully-connected operands scaled by 1/64 = 1/sqrt(4096)
(exact in binary), the bias from ``0.2*rand - 0.1``, and fp16 / bf16 operands
rounded from the fp32 draw to nearest-even. Integer-valued variants draw from
``randint`` and are converted to float exactly.

The first five workloads are those of the GEMM pages' measurements: square FP32
products (page "GPU架构下的矩阵乘法深入优化" measures 4096 cubed, page
"GEMM 优化详解" 1024 cubed), the fully-connected layer of page
"GEMM 优化详解" section "Level 6: Kernel Fusion" at a ragged batch, and the
FP16-input / FP32-accumulate product of the tensor-core section of page
"GPU架构下的矩阵乘法深入优化" (section 6). The sixth is the same 16-bit
product with bfloat16 inputs (page "GEMM 优化详解", "进一步优化方向": the
matrix units take FP16 or BF16); the seventh and eighth give B (W) N-by-K, the
[out][in] weight layout and the B^T of Q*K^T (page "GEMM 优化详解", table
"为什么 GEMM 重要"). B (W) of the transposed forms is drawn in its N-by-K shape.
The ninth runs C1's 256-cubed product 256 times as one strided batch (page
"GEMM 优化详解", section "矩阵大小选择策略": small matrices are batched); its
operands are drawn as (batch, rows, cols) tensors. The tenth and eleventh are
one GPU's share of the 4096-cubed product and of the fully-connected layer
split eight ways; the twelfth a 16-bit product of 144 256-square tiles. The
thirteenth and fourteenth are the fully-connected layer with one and four
rows of X: by the intensity formula of page "GEMM 优化详解" (table
"计算复杂度分析"), 2MNK / (MK + KN + MN) / 4, they do about M/2 FLOP per byte,
far below the ridge, so HBM bounds them and the bench rates them in GB/s.
The fifteenth is the one-row decode step with 16-bit operands and B given
N-by-K, HBM-bound too.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    index: int          # 1-based workload number, also the seed base
    name: str
    kind: str           # "gemm_f32", "gemm_f16f32", "gemm_bf16f32", "linear" (and _nt forms:
                        # B given N-by-K)
    M: int
    N: int
    K: int
    alpha: float = 1.0
    beta: float = 0.0
    act: int = 1        # linear only: 0 none, 1 ReLU
    scale: float = 1.0  # operand scale (linear: 1/64)
    batch: int = 1      # strided batch of independent products (batched kinds)
    bound: str = "mfma"  # the roofline that bounds it: "mfma", or "hbm" for a few rows of A
    extra: dict = field(default_factory=dict)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K * self.batch

    @property
    def hbm_bytes(self) -> int:
        """Compulsory HBM bytes of one call: A, B and the bias read once, C
        read (beta != 0) and written once."""
        esize = 2 if self.kind in HALF_KINDS else 4
        rw_c = 2 if self.beta != 0.0 else 1
        bias = 4 * self.N if self.kind in ("linear", "linear_nt") else 0
        return self.batch * (esize * (self.M * self.K + self.K * self.N) + 4 * rw_c * self.M * self.N) + bias


WORKLOADS = {
    "gemm_f32_256": Workload(1, "gemm_f32_256", "gemm_f32", 256, 256, 256),
    "gemm_f32_1024_ab": Workload(2, "gemm_f32_1024_ab", "gemm_f32", 1024, 1024, 1024, alpha=1.5, beta=0.5),
    "gemm_f32_4096": Workload(3, "gemm_f32_4096", "gemm_f32", 4096, 4096, 4096),
    "linear_relu_2047x4096x11008": Workload(4, "linear_relu_2047x4096x11008", "linear", 2047, 11008, 4096,
                                            act=1, scale=1.0 / 64.0),
    "gemm_f16f32_8192": Workload(5, "gemm_f16f32_8192", "gemm_f16f32", 8192, 8192, 8192),
    # the bfloat16 variant of the 16-bit product (same shape, inputs rounded to bf16)
    "gemm_bf16f32_8192": Workload(6, "gemm_bf16f32_8192", "gemm_bf16f32", 8192, 8192, 8192),
    # transposed-B forms: the same fully-connected layer with its weight stored
    # [out][in] (N-by-K), and the 16-bit product with B given N-by-K
    "linear_relu_nt_2047x4096x11008": Workload(7, "linear_relu_nt_2047x4096x11008", "linear_nt",
                                               2047, 11008, 4096, act=1, scale=1.0 / 64.0),
    "gemm_f16f32_nt_8192": Workload(8, "gemm_f16f32_nt_8192", "gemm_f16f32_nt", 8192, 8192, 8192),
    # many small products in one batched call: 256 independent 256^3 FP32 GEMMs
    "gemm_f32_batched_256x256x256_b256": Workload(9, "gemm_f32_batched_256x256x256_b256",
                                                  "gemm_f32_batched", 256, 256, 256, batch=256),
    # one GPU's share when the 4096^3 product is split 8 ways along M, and when
    # the fully-connected layer is split 8 ways along N (its output features)
    "gemm_f32_512x4096x4096": Workload(10, "gemm_f32_512x4096x4096", "gemm_f32", 512, 4096, 4096),
    "linear_relu_2047x1376x4096": Workload(11, "linear_relu_2047x1376x4096", "linear", 2047, 1376, 4096,
                                           act=1, scale=1.0 / 64.0),
    # a 16-bit product whose 256x256 tiles (144) would leave CUs idle; it runs
    # on 192x192 tiles, one per CU
    "gemm_f16f32_3072": Workload(12, "gemm_f16f32_3072", "gemm_f16f32", 3072, 3072, 3072),
    # the fully-connected layer's weight with a handful of input rows (one
    # token's decode through the [out][in] weight, four rows through the
    # [in][out] one): bound by reading the weight from HBM, not by the MFMAs
    "linear_relu_nt_1x4096x11008": Workload(13, "linear_relu_nt_1x4096x11008", "linear_nt", 1, 11008, 4096,
                                            act=1, scale=1.0 / 64.0, bound="hbm"),
    "linear_relu_4x4096x11008": Workload(14, "linear_relu_4x4096x11008", "linear", 4, 11008, 4096,
                                         act=1, scale=1.0 / 64.0, bound="hbm"),
    # the same decode step with 16-bit inputs: one row of A (K = 4096) against
    # B given 11008 x 4096 [out][in]
    "gemm_f16f32_nt_1x4096x11008": Workload(15, "gemm_f16f32_nt_1x4096x11008", "gemm_f16f32_nt", 1, 11008, 4096,
                                            bound="hbm"),
}

HALF_KINDS = ("gemm_f16f32", "gemm_bf16f32", "gemm_f16f32_nt")
BATCHED_KINDS = ("gemm_f32_batched",)
B_TRANSPOSED_KINDS = ("linear_nt", "gemm_f16f32_nt")


def generator(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def uniform(shape, seed: int, scale: float = 1.0) -> torch.Tensor:
    """fp32 values in [-scale, scale) drawn as scale*(2*rand - 1)."""
    x = torch.rand(shape, generator=generator(seed), dtype=torch.float32) * 2.0 - 1.0
    if scale != 1.0:
        x = x * scale
    return x


def bias_uniform(n: int, seed: int) -> torch.Tensor:
    """fp32 bias in [-0.1, 0.1) drawn as 0.2*rand - 0.1."""
    return torch.rand((n,), generator=generator(seed), dtype=torch.float32) * 0.2 - 0.1


def integers(shape, seed: int, lo: int, hi: int, dtype=torch.float32) -> torch.Tensor:
    """Integer values in [lo, hi] (inclusive) as an exact float tensor."""
    return torch.randint(lo, hi + 1, shape, generator=generator(seed), dtype=torch.int64).to(dtype)


def to_half(x: torch.Tensor) -> torch.Tensor:
    """Round fp32 to binary16, nearest-even."""
    return x.to(torch.float16)


def to_bf16(x: torch.Tensor) -> torch.Tensor:
    """Round fp32 to bfloat16, nearest-even."""
    return x.to(torch.bfloat16)


def half_bits(x: torch.Tensor):
    """The 16-bit patterns of a float16 or bfloat16 tensor as a uint16 numpy array."""
    return x.contiguous().view(torch.int16).numpy().view("uint16")


def make_inputs(w: Workload, integer: bool = False, M: int | None = None,
                N: int | None = None, K: int | None = None, batch: int | None = None) -> dict:
    """Host (CPU) input tensors for workload ``w``; sizes may be overridden.

    Returns a dict with A, B (and C for beta != 0, bias for linear). For fp16
    and bf16 workloads A and B are float16 / bfloat16 tensors; for batched
    workloads every tensor gains a leading batch axis. ``integer=True`` gives
    the integer-valued variant whose exact result every summation order
    reaches: fp32 entries in [-2, 2], C_in and bias in [-4, 4], fp16 entries in
    [-8, 8].
    """
    M = w.M if M is None else M
    N = w.N if N is None else N
    K = w.K if K is None else K
    lead = ((w.batch if batch is None else batch),) if w.kind in BATCHED_KINDS else ()
    s = 100 * w.index
    out = {}
    ashape = lead + (M, K)
    bshape = lead + ((N, K) if w.kind in B_TRANSPOSED_KINDS else (K, N))
    cshape = lead + (M, N)
    linear = w.kind in ("linear", "linear_nt")
    if integer:
        lim = 8 if w.kind in HALF_KINDS else 2
        out["A"] = integers(ashape, s + 0, -lim, lim)
        out["B"] = integers(bshape, s + 1, -lim, lim)
        if w.beta != 0.0:
            out["C"] = integers(cshape, s + 2, -4, 4)
        if linear:
            out["bias"] = integers((N,), s + 3, -4, 4)
    else:
        out["A"] = uniform(ashape, s + 0, w.scale)
        out["B"] = uniform(bshape, s + 1, w.scale)
        if w.beta != 0.0:
            out["C"] = uniform(cshape, s + 2)
        if linear:
            out["bias"] = bias_uniform(N, s + 3)
    if w.kind in ("gemm_f16f32", "gemm_f16f32_nt"):
        out["A"] = to_half(out["A"])
        out["B"] = to_half(out["B"])
    if w.kind == "gemm_bf16f32":
        out["A"] = to_bf16(out["A"])
        out["B"] = to_bf16(out["B"])
    return out
