"""Seeded synthetic inputs, shared by the tests, the benchmark and the smoke
check.

This module holds no arithmetic of the method: it only draws numbers and
stores them in the representation the library takes (bf16 bit patterns as
uint16, or float32).  Both the HIP path and the CPU oracle are fed from here.

Recipe (shapes and distributions of the workloads the pages describe for an
8B-class model: hidden 4096, MLP 14336, vocabulary 151936):
  * numpy ``default_rng([seed, stream])`` (PCG64), one stream per tensor:
    X=0, A/W=1, B=2, gamma=3, logits=4;
  * ``N(mean, std)`` draws are taken in fp64, scaled, rounded to float32
    (numpy, round to nearest even), then to bf16 by rounding the float32 bit
    pattern to nearest even;
  * draws fill the array in C order, so the first rows of a tall draw equal
    a shorter draw with the same seed: batches are prefixes of one tensor.
"""
import numpy as np

STREAM_X = 0
STREAM_W = 1
STREAM_B = 2
STREAM_GAMMA = 3
STREAM_LOGITS = 4
STREAM_BASE = 5
STREAM_BIAS = 6
STREAM_Q = 7
STREAM_K = 8
STREAM_V = 9


def rng(seed, stream):
    return np.random.default_rng([int(seed), int(stream)])


def f32_bits_to_bf16_bits(f):
    """float32 array -> bf16 bit patterns, nearest even on the bit pattern
    (inputs here are finite)."""
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b):
    """bf16 bit patterns -> float32 values (a bit shift; exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def normal_f32(shape, mean, std, seed, stream):
    g = rng(seed, stream)
    return (g.standard_normal(shape) * std + mean).astype(np.float32)


def normal_bf16(shape, mean, std, seed, stream):
    return f32_bits_to_bf16_bits(normal_f32(shape, mean, std, seed, stream))


def integer_f32(shape, lo, hi, seed, stream):
    """Integer values in [lo, hi]; exact in bf16 when |v| <= 256."""
    g = rng(seed, stream)
    return g.integers(lo, hi + 1, size=shape).astype(np.float32)


def integer_bf16(shape, lo, hi, seed, stream):
    return f32_bits_to_bf16_bits(integer_f32(shape, lo, hi, seed, stream))


# --- the workloads, one function each -------------------------------------

def lora_inputs(M, K, r, seed=0):
    """LoRA shrink/expand: X[M,K] ~ N(0,1), A[K,r] ~ N(0,0.02),
    B[r,K] ~ N(0,0.02), bf16 bits (K is the hidden size)."""
    X = normal_bf16((M, K), 0.0, 1.0, seed, STREAM_X)
    A = normal_bf16((K, r), 0.0, 0.02, seed, STREAM_W)
    B = normal_bf16((r, K), 0.0, 0.02, seed, STREAM_B)
    return X, A, B


def dense_inputs(M, K, N, seed=0):
    """Dense projection: X[M,K] ~ N(0,1), W[K,N] ~ N(0,0.02), bf16 bits."""
    X = normal_bf16((M, K), 0.0, 1.0, seed, STREAM_X)
    W = normal_bf16((K, N), 0.0, 0.02, seed, STREAM_W)
    return X, W


def rmsnorm_inputs(B, H, seed=0):
    """RMSNorm: x[B,H] ~ N(0,1), gamma[H] ~ N(1,0.1), bf16 bits."""
    x = normal_bf16((B, H), 0.0, 1.0, seed, STREAM_X)
    g = normal_bf16((H,), 1.0, 0.1, seed, STREAM_GAMMA)
    return x, g


def logits_inputs(B, V, seed=0):
    """log_softmax / mean: logits[B,V] ~ N(0,3), float32."""
    return normal_f32((B, V), 0.0, 3.0, seed, STREAM_LOGITS)


def lora_layer_inputs(M, K, N, r, seed=0):
    """A LoRA-adapted linear layer: X[M,K] ~ N(0,1), base W[K,N], A[K,r] and
    B[r,N] ~ N(0,0.02), bf16 bits."""
    X = normal_bf16((M, K), 0.0, 1.0, seed, STREAM_X)
    W = normal_bf16((K, N), 0.0, 0.02, seed, STREAM_BASE)
    A = normal_bf16((K, r), 0.0, 0.02, seed, STREAM_W)
    B = normal_bf16((r, N), 0.0, 0.02, seed, STREAM_B)
    return X, W, A, B


def bias_inputs(N, seed=0):
    """An fp32 bias row of N values ~ N(0,1)."""
    return normal_f32((N,), 0.0, 1.0, seed, STREAM_BIAS)


def attention_inputs(B, Hq, Hkv, L, D, seed=0):
    """Decode attention: q[B,Hq,D], k and v [B,Hkv,L,D] ~ N(0,1), bf16 bits."""
    q = normal_bf16((B, Hq, D), 0.0, 1.0, seed, STREAM_Q)
    k = normal_bf16((B, Hkv, L, D), 0.0, 1.0, seed, STREAM_K)
    v = normal_bf16((B, Hkv, L, D), 0.0, 1.0, seed, STREAM_V)
    return q, k, v
