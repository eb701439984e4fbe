"""Seeded synthetic inputs for W4A16 layers: the one module that both the HIP path's
tests/benchmark and the CPU oracle draw their inputs from.

It holds none of the method's arithmetic: it draws random 32-bit words and random
floats and rounds the floats to the 16-bit activation dtype. It never packs,
unpacks, dequantises or multiplies.

Why drawing whole int32 words is the same as drawing codes and packing them:
every 32-bit pattern is a valid AWQ word, and drawing the word uniformly over all
2^32 patterns makes its eight 4-bit codes independent and each uniform on 0..15,
whatever slot order the packing uses. So qweight / qzeros drawn this way are
exactly "uniform int4 codes and zero points, AWQ-packed as int32".

The workloads are Llama-style layer shapes (the vllm-omni commit "cpu_int4:
repack weights in n-blocks ..." lists gate_up 13312x2048, down 2048x6656,
q_k_v 3072x2048 and a tied 131072x2048 embedding / LM head). No checkpoint is
available, so weights are random: codes and zeros uniform on 0..15, scales
uniform on [0.005, 0.02), activations N(0, 1).

Draw order for one weight set, from numpy Generator(PCG64(seed)):
  1. qweight  uint32 [K, N/8]    uniform on [0, 2^32)
  2. qzeros   uint32 [K/G, N/8]  uniform on [0, 2^32)
  3. scales   float64 [K/G, N]   uniform on [0.005, 0.02), cast to float32, then
                                 rounded to the dtype (round to nearest even)
then, from the same generator, one activation matrix per M in the order listed:
  4. x        float32 [M, K]     standard normal, rounded to the dtype (RNE)
16-bit values are returned as uint16 bit patterns.
"""

from dataclasses import dataclass, field

import numpy as np

FP16 = "fp16"
BF16 = "bf16"


def f32_to_bf16_bits(a):
    """float32 -> bf16 bit patterns, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def f32_to_half_bits(a, dtype):
    if dtype == BF16:
        return f32_to_bf16_bits(a)
    if dtype == FP16:
        return np.asarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)
    raise ValueError(dtype)


@dataclass
class Workload:
    name: str
    seed: int
    K: int
    N: int
    dtype: str
    Ms: tuple
    group_size: int = 128
    description: str = ""


# The five workloads (the fourth split in two layer shapes).
WORKLOADS = {
    "small_fp16": Workload("small_fp16", 101, 512, 512, FP16, (4,),
                           description="W4A16 GEMM M=4 K=512 N=512, fp16"),
    "gate_up_decode": Workload("gate_up_decode", 201, 2048, 13312, BF16, (1,),
                               description="decode GEMV M=1 over the gate_up shape K=2048 N=13312"),
    "down_proj": Workload("down_proj", 301, 6656, 2048, BF16, (1, 8, 16),
                          description="down-projection K=6656 N=2048 at M=1, 8, 16"),
    "qkv_prefill": Workload("qkv_prefill", 401, 2048, 3072, BF16, (512,),
                            description="prefill GEMM M=512 over the qkv shape K=2048 N=3072"),
    "gate_up_prefill": Workload("gate_up_prefill", 402, 2048, 13312, BF16, (512,),
                                description="prefill GEMM M=512 over the gate_up shape K=2048 N=13312"),
    "lm_head": Workload("lm_head", 501, 2048, 131072, BF16, (1, 512),
                        description="tied embedding / LM head K=2048 N=131072 at M=1 and M=512"),
}


@dataclass
class WeightSet:
    K: int
    N: int
    group_size: int
    dtype: str
    qweight: np.ndarray      # int32 [K, N/8]
    qzeros: np.ndarray       # int32 [K/G, N/8]
    scale_bits: np.ndarray   # uint16 [K/G, N]
    x_bits: dict = field(default_factory=dict)   # M -> uint16 [M, K]


def draw_weights(rng, K, N, group_size, dtype):
    G = K if group_size == -1 else group_size
    qweight = rng.integers(0, 2**32, size=(K, N // 8), dtype=np.uint32).view(np.int32)
    qzeros = rng.integers(0, 2**32, size=(K // G, N // 8), dtype=np.uint32).view(np.int32)
    scales = rng.uniform(0.005, 0.02, size=(K // G, N)).astype(np.float32)
    return WeightSet(K, N, group_size, dtype, qweight, qzeros, f32_to_half_bits(scales, dtype))


def draw_activations(rng, M, K, dtype):
    return f32_to_half_bits(rng.standard_normal((M, K), dtype=np.float32), dtype)


def make(workload, Ms=None):
    """Weights and activations of a named workload, in the documented draw order.
    Ms (a subset of the workload's M values) only skips storing the others; the
    draws are the same."""
    wl = WORKLOADS[workload] if isinstance(workload, str) else workload
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    ws = draw_weights(rng, wl.K, wl.N, wl.group_size, wl.dtype)
    for M in wl.Ms:
        xb = draw_activations(rng, M, wl.K, wl.dtype)
        if Ms is None or M in Ms:
            ws.x_bits[M] = xb
    return ws


def make_custom(seed, M, K, N, dtype=BF16, group_size=128):
    """A weight set plus one activation matrix for an arbitrary shape, same recipe."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ws = draw_weights(rng, K, N, group_size, dtype)
    ws.x_bits[M] = draw_activations(rng, M, K, dtype)
    return ws


def draw_token_ids(seed, T, N):
    """Token ids for an embedding lookup: T ids uniform on [0, N), int32, from their
    own generator Generator(PCG64(seed)) (prompt tokens of a vocabulary of N)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(0, N, size=T, dtype=np.int64).astype(np.int32)


@dataclass
class GptqWeightSet:
    K: int
    N: int
    group_size: int
    dtype: str
    qweight: np.ndarray      # int32 [K/8, N]   (codes packed along K)
    qzeros: np.ndarray       # int32 [K/G, N/8] (zero points packed along N)
    scale_bits: np.ndarray   # uint16 [K/G, N]


def draw_gptq_weights(seed, K, N, dtype=BF16, group_size=128):
    """A GPTQ-standard weight set, same recipe as draw_weights: whole int32 words
    uniform over all 2^32 patterns (so every code and zero point is uniform on 0..15
    whatever the order inside the word), then scales uniform on [0.005, 0.02)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    G = K if group_size == -1 else group_size
    qweight = rng.integers(0, 2**32, size=(K // 8, N), dtype=np.uint32).view(np.int32)
    qzeros = rng.integers(0, 2**32, size=(K // G, N // 8), dtype=np.uint32).view(np.int32)
    scales = rng.uniform(0.005, 0.02, size=(K // G, N)).astype(np.float32)
    return GptqWeightSet(K, N, group_size, dtype, qweight, qzeros, f32_to_half_bits(scales, dtype))
