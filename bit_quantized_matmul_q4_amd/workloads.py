"""Seeded synthetic inputs for the 4-bit matmul path.

This module only draws random numbers and knows the workload shapes; it holds
none of the quantization or matmul arithmetic.  The tests, the smoke check and
the benchmark draw inputs here and hand the very same arrays to both the HIP
library and the CPU oracle.

Recipe (one ``torch.Generator`` per workload, seeded explicitly):
  * weights  W = 0.02 * N(0, 1)   fp32 [N][K]  (drawn first)
  * activations x = N(0, 1)       fp32 [M][K]  (drawn second, same generator)
  * outliers: a mask ``rand(M, K) < 0.01`` (drawn third) scales x by 20.

The shapes follow a ~4B dense decoder (hidden 2560, FFN 9216, vocab 151936)
for decode and a ~9B-shaped FFN (4096 <-> 12288) for prefill; the pages
measure on Qwen3.5-4B Q4_K_M decode (vllm.cpp issue 5, "Goal") and on a
Qwen3.5 9B HFQ4 prefill (hipfire MMQ note, benchmark table).  No checkpoint is
used: random weights of those shapes stand in for them.
"""
import torch

GROUP = 256
BLOCK = 32

# Decode projection set of a ~4B dense transformer, M = 1: (name, K, N).
# The seed of the k-th projection is k, in this order.
DECODE_PROJECTIONS = [
    ("q", 2560, 4096),
    ("k", 2560, 1024),
    ("v", 2560, 1024),
    ("o", 4096, 2560),
    ("gate", 2560, 9216),
    ("up", 2560, 9216),
    ("down", 9216, 2560),
    ("lm_head", 2560, 151936),
]
DECODE_LAYERS = 36  # projection layers streamed per decoded token (lm_head once)

SINGLE_GEMV = dict(M=1, N=4096, K=4096, seed=0)
TINY_M = dict(Ms=(1, 2, 4, 8, 16), N=151936, K=4096, seed=0)
MMQ_512 = dict(M=512, K=2560, N=9216, seed=0, outliers=False)
MMQ_2048 = [
    dict(name="gate_up", M=2048, K=4096, N=12288, seed=0, outliers=True),
    dict(name="down", M=2048, K=12288, N=4096, seed=1, outliers=True),
]


def generator(seed, device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def draw_weights(gen, N, K, device="cpu"):
    """W ~ 0.02 * N(0, 1), fp32 [N][K]."""
    w = torch.randn((N, K), generator=gen, dtype=torch.float32, device=device)
    return w.mul_(0.02)


def draw_activations(gen, M, K, outliers=False, device="cpu"):
    """x ~ N(0, 1), fp32 [M][K]; with outliers, 1 % of entries (i.i.d.) times 20."""
    x = torch.randn((M, K), generator=gen, dtype=torch.float32, device=device)
    if outliers:
        mask = torch.rand((M, K), generator=gen, device=device) < 0.01
        x = torch.where(mask, x * 20.0, x)
    return x


def gemv_case(seed, M, N, K, device="cpu"):
    """(W, x) for one GEMV workload, W drawn before x from one generator."""
    g = generator(seed, device)
    W = draw_weights(g, N, K, device)
    x = draw_activations(g, M, K, False, device)
    return W, x


def mmq_case(seed, M, N, K, outliers=False, device="cpu"):
    """(W, x) for one prefill workload, W drawn before x from one generator."""
    g = generator(seed, device)
    W = draw_weights(g, N, K, device)
    x = draw_activations(g, M, K, outliers, device)
    return W, x


def small_case(seed, M, N, K, outliers=False):
    """Small CPU case for parity tests: same recipe, any shape."""
    return mmq_case(seed, M, N, K, outliers, "cpu")
