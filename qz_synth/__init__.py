"""Seeded synthetic inputs for the layer quantizer: calibration activations X and
pretrained weights W_hat.

This module is shared by the CPU oracle, the GPU tests and the benchmark, and it
holds none of the quantizer's arithmetic: it only draws random numbers and casts
them to the storage types (bf16 bit patterns or fp32).

Distributions (stand-ins for the calibration set of 128 sequences x 2048 tokens
that the GPTQ tutorial page uses in its evidence section, and for the 8B/32B-like
layer widths named in the ADMM-Q summary's experiments):

* X = T + Z A, T iid Student-t with 4 degrees of freedom, Z ~ N(0,1) [n x r],
  A ~ N(0, 1/r) [r x d_i] (r = 64, a correlated low-rank part); then a fraction p
  of the channels, chosen without replacement, is multiplied by an outlier factor f.
  Cast to bf16 by round-to-nearest-even of the fp32 bits.
* W_hat ~ N(0, sigma_w^2), cast to bf16 (or kept fp32 for the tiny layer).
* The tiny layer: X [512 x 128] fp32 N(0,1) with two channels x20, W_hat fp32
  N(0, 0.02^2) [64 x 128].

Student-t(4) is drawn as z / sqrt((e1 + e2) / 2) with z ~ N(0,1), e1, e2 ~ Exp(1):
chi-square with 4 degrees of freedom is 2 (e1 + e2), so this is exact for nu = 4.

Streams: numpy.random.default_rng([seed, stream]); stream 0 is metadata (A and the
outlier channels), stream 1 + c is token chunk c (CHUNK tokens each), stream
10**6 is W_hat.  The torch variants draw the token chunks with a seeded
torch.Generator on the target device instead (for full-size inputs that the host
would take minutes to draw); the metadata still comes from numpy stream 0.
"""
from __future__ import annotations

import numpy as np

CHUNK = 2048
RANK = 64
W_STREAM = 10 ** 6


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    out = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _meta(seed: int, d_i: int, p_out: float, rank: int = RANK):
    rng = np.random.default_rng([seed, 0])
    A = rng.standard_normal((rank, d_i)) / np.sqrt(rank)
    k = int(round(p_out * d_i))
    ch = np.sort(rng.choice(d_i, size=k, replace=False)) if k > 0 else np.zeros(0, np.int64)
    return A.astype(np.float32), ch


def outlier_channels(seed: int, d_i: int, p_out: float) -> np.ndarray:
    return _meta(seed, d_i, p_out)[1]


def calib_chunk_f32(seed: int, c: int, d_i: int, p_out: float, f_out: float,
                    tokens: int = CHUNK) -> np.ndarray:
    """Token chunk c of the heavy-tailed + low-rank + outlier calibration set (fp32)."""
    A, ch = _meta(seed, d_i, p_out)
    rng = np.random.default_rng([seed, 1 + c])
    z = rng.standard_normal((tokens, d_i), dtype=np.float32)
    e = rng.standard_exponential((2, tokens, d_i), dtype=np.float32)
    t = z / np.sqrt((e[0] + e[1]) * np.float32(0.5))
    lr = rng.standard_normal((tokens, A.shape[0]), dtype=np.float32) @ A
    x = t + lr
    if ch.size:
        x[:, ch] *= np.float32(f_out)
    return x


def calib_bf16(seed: int, n: int, d_i: int, p_out: float = 0.01, f_out: float = 30.0) -> np.ndarray:
    """X [n x d_i] as bf16 bit patterns (uint16), drawn chunk by chunk on the host."""
    out = np.empty((n, d_i), dtype=np.uint16)
    for c, a in enumerate(range(0, n, CHUNK)):
        b = min(a + CHUNK, n)
        out[a:b] = f32_to_bf16_bits(calib_chunk_f32(seed, c, d_i, p_out, f_out, b - a))
    return out


def weights_bf16(seed: int, d_o: int, d_i: int, sigma_w: float = 0.015) -> np.ndarray:
    """W_hat [d_o x d_i] ~ N(0, sigma_w^2) as bf16 bit patterns."""
    rng = np.random.default_rng([seed, W_STREAM])
    w = rng.standard_normal((d_o, d_i), dtype=np.float32) * np.float32(sigma_w)
    return f32_to_bf16_bits(w)


def tiny_layer(seed: int = 1, n: int = 512, d_i: int = 128, d_o: int = 64,
               n_out: int = 2, f_out: float = 20.0, sigma_w: float = 0.02):
    """The tiny fp32 layer: X [n x d_i] N(0,1) with n_out channels x f_out,
    W_hat [d_o x d_i] N(0, sigma_w^2). Returns (X, W_hat, outlier channel ids)."""
    rng = np.random.default_rng([seed, 0])
    ch = np.sort(rng.choice(d_i, size=n_out, replace=False))
    X = np.random.default_rng([seed, 1]).standard_normal((n, d_i), dtype=np.float32)
    X[:, ch] *= np.float32(f_out)
    W = np.random.default_rng([seed, W_STREAM]).standard_normal((d_o, d_i), dtype=np.float32)
    W *= np.float32(sigma_w)
    return X, W, ch


# ---------------------------------------------------------------- device-side draws
def calib_bf16_torch(seed: int, n: int, d_i: int, p_out: float = 0.01, f_out: float = 30.0,
                     device="cuda"):
    """X [n x d_i] torch.bfloat16 on `device`, same recipe as calib_bf16 but the
    token draws come from a seeded torch.Generator on the device."""
    import torch
    A, ch = _meta(seed, d_i, p_out)
    A_t = torch.from_numpy(A).to(device)
    ch_t = torch.from_numpy(ch.astype(np.int64)).to(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 1000003 + 17)
    out = torch.empty((n, d_i), dtype=torch.bfloat16, device=device)
    step = 8 * CHUNK
    for a in range(0, n, step):
        b = min(a + step, n)
        m = b - a
        z = torch.randn((m, d_i), generator=gen, device=device, dtype=torch.float32)
        e1 = torch.empty((m, d_i), device=device, dtype=torch.float32).exponential_(generator=gen)
        e2 = torch.empty((m, d_i), device=device, dtype=torch.float32).exponential_(generator=gen)
        x = z / torch.sqrt((e1 + e2) * 0.5)
        del z, e1, e2
        x += torch.randn((m, A.shape[0]), generator=gen, device=device) @ A_t
        if ch.size:
            x[:, ch_t] *= f_out
        out[a:b] = x.to(torch.bfloat16)   # round-to-nearest-even
        del x
    return out


def weights_bf16_torch(seed: int, d_o: int, d_i: int, sigma_w: float = 0.015, device="cuda"):
    """W_hat [d_o x d_i] torch.bfloat16 on `device` from the same numpy stream as
    weights_bf16 (bit-identical to it)."""
    import torch
    return torch.from_numpy(weights_bf16(seed, d_o, d_i, sigma_w).view(np.int16)).view(
        torch.bfloat16).to(device)


# ---------------------------------------------------------------- workload table
# The five layer workloads: (name, d_i, d_o, bits, group, gptq_block, admm params)
WORKLOADS = {
    "tiny_128x64_w4": dict(d_i=128, d_o=64, n=512, bits=4, group=128, B=32,
                            iters=20, rho0=0.1, gamma=1.3, refresh=1, damp=0.01),
    "attn_4096x4096_w3g128": dict(d_i=4096, d_o=4096, n=262144, bits=3, group=128, B=128,
                                   iters=100, rho0=0.05, gamma=1.05, refresh=1, damp=0.01,
                                   p_out=0.01, f_out=30.0, seed=2),
    "up_4096x12288_w3g128": dict(d_i=4096, d_o=12288, n=262144, bits=3, group=128, B=128,
                                  iters=100, rho0=0.05, gamma=1.05, refresh=1, damp=0.01,
                                  p_out=0.01, f_out=30.0, seed=4),
    "mlp_up_4096x12288_w2g128": dict(d_i=4096, d_o=12288, n=262144, bits=2, group=128, B=128,
                                      iters=150, rho0=0.05, gamma=1.05, refresh=1, damp=0.01,
                                      p_out=0.01, f_out=30.0, seed=3),
    "mlp_down_12288x4096_w2g128": dict(d_i=12288, d_o=4096, n=262144, bits=2, group=128, B=128,
                                        iters=150, rho0=0.05, gamma=1.05, refresh=1, damp=0.01,
                                        p_out=0.01, f_out=30.0, seed=3),
    "32b_down_25600x5120_w3g128": dict(d_i=25600, d_o=5120, n=262144, bits=3, group=128, B=128,
                                        iters=200, rho0=0.05, gamma=1.05, refresh=10, damp=0.01,
                                        p_out=0.005, f_out=50.0, seed=5),
    "32b_up_5120x25600_w3g128": dict(d_i=5120, d_o=25600, n=262144, bits=3, group=128, B=128,
                                      iters=200, rho0=0.05, gamma=1.05, refresh=10, damp=0.01,
                                      p_out=0.005, f_out=50.0, seed=5),
}


# ---------------------------------------------------------------- decoder block
# One 8B-like decoder block quantized sub-layer by sub-layer: (name, input, d_i, d_o,
# weight seed).  Inputs (the block's input hidden states are the calibration tokens,
# 128 sequences of seq_len tokens): x_qkv = RMSNorm of the hidden states; x_attn = the
# causal attention output of each sequence; x_mlp = RMSNorm of the hidden states plus
# o_proj's output; x_down = silu(gate) * up.  q/k/v share x_qkv's Hessian and gate/up
# share x_mlp's.  Only sizes and seeds live here; tests/block_driver.py evaluates it.
BLOCK_8B = dict(
    n=262144, seq_len=2048, d_model=4096, d_ff=12288, kv_heads=8, head_dim=128, q_heads=32,
    calib_seed=6, p_out=0.01, f_out=30.0, damp=0.01, group=128, B=128,
    iters=100, rho0=0.05, gamma=1.05, refresh=1,
    sublayers=[("q_proj", "x_qkv", 4096, 4096, 11), ("k_proj", "x_qkv", 4096, 1024, 12),
               ("v_proj", "x_qkv", 4096, 1024, 13), ("o_proj", "x_attn", 4096, 4096, 14),
               ("gate_proj", "x_mlp", 4096, 12288, 15), ("up_proj", "x_mlp", 4096, 12288, 16),
               ("down_proj", "x_down", 12288, 4096, 17)],
)
