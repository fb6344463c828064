"""Work accounting for the attention forward pass: counted FLOPs, algorithmic
bytes and the MI355X peaks they are compared against.

FLOP convention: the forward pass is two matrix products per head, S = Q K^T
and O = P V, each of cost 2*M*N*K for an M x K by K x N product ("TCA 51%,
MFU 不足 8%", section "GEMM").  Per head that is 2 * (2 * N * N * d), so
4 * B * H * N^2 * d in all, halved under the causal mask (the masked half of
the score matrix is not counted).  The same article measures attention
throughput this way (section "MFU 总比TCA 低一些"), and the B300 blog's
harness lines ("Flash Attention CUDA Kernel 优化 ... G4", V14 to V20) agree
with it; tests/test_accounting.py checks both against the printed numbers.

Algorithmic bytes: the fused pass must read Q, K and V once and write O and
the row log-sum-exp once; the N x N score matrix never reaches HBM.  The
backward likewise reads its inputs once and writes its gradients once.
"""
from __future__ import annotations

# MI355X published dense peaks (no structured sparsity).
PEAK_TFLOPS = {"fp16": 2516.6, "bf16": 2516.6, "fp8": 5033.2}
PEAK_HBM_GBPS = 8000.0
ELEMENT_BYTES = {"fp16": 2, "bf16": 2, "fp8": 1}
OUT_BYTES = 2          # O is stored as fp16 for every input type
LSE_BYTES = 4          # float32 per query row


def counted_flops(B: int, H: int, N: int, d: int, causal: bool) -> float:
    """4*B*H*N^2*d, halved for the causal mask."""
    f = 4.0 * B * H * N * N * d
    return f / 2.0 if causal else f


def algorithmic_bytes(B: int, H: int, N: int, d: int, dtype: str) -> int:
    """Q, K, V read once + O (fp16) and LSE (fp32) written once."""
    e = ELEMENT_BYTES[dtype]
    return B * H * N * d * (3 * e + OUT_BYTES) + B * H * N * LSE_BYTES


def algorithmic_bytes_bwd(B: int, H: int, N: int, d: int, dtype: str) -> int:
    """Backward at the library's boundary: Q, K, V, O and dO (input type) and
    LSE (fp32) read once; dQ, dK, dV (fp32) and delta = rowsum(dO * O)
    (fp32) written once."""
    e = ELEMENT_BYTES[dtype]
    return B * H * N * d * (5 * e + 3 * 4) + B * H * N * (LSE_BYTES + 4)


def tflops(flops: float, seconds: float) -> float:
    return flops / seconds / 1e12


def gib_per_s(nbytes: float, seconds: float) -> float:
    """Binary gigabytes per second (the unit of the blog harness's bandwidth line)."""
    return nbytes / seconds / 2.0 ** 30


def frac_of_peak(achieved_tflops: float, dtype: str) -> float:
    return achieved_tflops / PEAK_TFLOPS[dtype]
