"""Seeded synthetic inputs for the quantizers and the GEMM.

This module only draws random numbers (NumPy PCG64, float32 draws, in a
fixed order) and casts them to bfloat16 with round-to-nearest-even; it holds
none of the quantization arithmetic.  The tests, the benchmark and the CPU
oracle all take their inputs from here.

Workloads (shapes and distributions of the quantizer's use cases):
  gaussian   N(0,1) fp32 tensor -- the format-comparison distribution.
  gradient   N(0,1) with 5 % of entries replaced by N(0, 10^2) outliers,
             bf16 -- a gradient with outliers inside the 16-blocks (the
             contaminated-block case of the palettes blog).
  weight     Student-t(nu=4) rows times per-row lognormal(0, 0.5) magnitudes,
             bf16 -- weight channels of differing scale (IF4 Figure 3 case).
  wgrad      dY = 1e-3 N(0,1) with 1 % of entries scaled by 10, X = N(0,1),
             both bf16 -- one linear layer's weight-gradient GEMM operands.
  mlp_step   X N(0,1), W 0.02 N(0,1), dY 1e-3 N(0,1), all bf16 -- one MLP
             up-projection training step.
Sign vectors for the 128-point rotation are drawn from the same generator
after the data.
"""
import numpy as np

__all__ = ["gaussian", "gradient", "weight", "wgrad", "mlp_step", "signs_from_rng",
           "mc_signs", "to_bf16_f32", "GRADIENT_SHAPE", "WEIGHT_SHAPE", "WGRAD_SHAPE",
           "MLP_SHAPES"]

GRADIENT_SHAPE = (4096, 4096)
WEIGHT_SHAPE = (8192, 8192)
WGRAD_SHAPE = (16384, 4096)
MLP_SHAPES = {"X": (32768, 4096), "W": (11008, 4096), "dY": (32768, 11008)}


def to_bf16_f32(a):
    """Round an fp32 array to bfloat16 (nearest, ties to even) and return the
    result as fp32 (exact).  NaN handling is irrelevant for these inputs."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).reshape(a.shape)


def signs_from_rng(rng):
    """128 flags in {0, 1}; 1 negates that coordinate before the transform."""
    return rng.integers(0, 2, 128).astype(np.uint8)


def mc_signs(trial):
    """Independent sign vector for Monte-Carlo trial t of the gradient case."""
    return signs_from_rng(np.random.default_rng([1, int(trial)]))


def gaussian(rows=256, cols=256, seed=0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((rows, cols), dtype=np.float32)


def gradient(rows=4096, cols=4096, seed=1, frac=0.05, outlier_sigma=10.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    mask = rng.random((rows, cols), dtype=np.float32) < frac
    x[mask] = outlier_sigma * rng.standard_normal(int(mask.sum()), dtype=np.float32)
    signs = signs_from_rng(rng)
    return to_bf16_f32(x), signs


def weight(rows=8192, cols=8192, seed=2, nu=4.0):
    rng = np.random.default_rng(seed)
    t = rng.standard_t(nu, (rows, cols)).astype(np.float32)
    mag = rng.lognormal(0.0, 0.5, (rows, 1)).astype(np.float32)
    return to_bf16_f32(t * mag)


def wgrad(tokens=16384, dim=4096, seed=3, frac=0.01):
    rng = np.random.default_rng(seed)
    dy = np.float32(1e-3) * rng.standard_normal((tokens, dim), dtype=np.float32)
    mask = rng.random((tokens, dim), dtype=np.float32) < frac
    dy[mask] *= np.float32(10.0)
    x = rng.standard_normal((tokens, dim), dtype=np.float32)
    signs = signs_from_rng(rng)
    return to_bf16_f32(dy), to_bf16_f32(x), signs


def mlp_step(tokens=32768, d_in=4096, d_out=11008, seed=4):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((tokens, d_in), dtype=np.float32)
    w = np.float32(0.02) * rng.standard_normal((d_out, d_in), dtype=np.float32)
    dy = np.float32(1e-3) * rng.standard_normal((tokens, d_out), dtype=np.float32)
    signs = signs_from_rng(rng)
    return to_bf16_f32(x), to_bf16_f32(w), to_bf16_f32(dy), signs
