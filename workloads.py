"""Seeded synthetic bf16 inputs for the block-scaled cast workloads.

This module only draws random numbers and rounds them to bf16 (torch's CPU
float32 -> bfloat16 conversion, round to nearest even).  It holds none of the
quantisation arithmetic, and both the CPU oracle's tests and the GPU path's
tests/bench take their inputs from here.

The pages benchmark the cast kernels on model-shaped random tensors (the
"Full per-workload numbers" table of the TransformerEngine LDS/STS PR; the
16384 x 16384, block 32 run of the torchao "Multiply with inverse scale" PR);
these recipes stand in for those tensors.  Every array is returned as uint16
bf16 bit patterns, row-major.

Recipes (seed per workload; numpy PCG64, drawn in float32 unless stated):
  special_256x512   N(0,1) bulk with four 32x32 diagonal tiles, each a whole
                    block in both directions: all +0; 0.5*N(0,1) clipped to
                    |x| <= 7.9 with +-8 on the tile diagonal (block amax = 2^3
                    exactly); 1e-30 * N(0,1); random sign * U(2.9e38, 3.0e38).
  loguniform_rows   z * 10^u_m, z ~ N(0,1), u_m ~ U(-3, 3) drawn once per row.
  normal            sigma * N(0,1).
  student_t_rows    Student-t (nu = 3, drawn in float64) with round(1% of M)
                    distinct rows chosen by the generator and multiplied by 100.
"""
import numpy as np
import torch

CHUNK_ROWS = 1024


def bf16_bits(f32) -> np.ndarray:
    """Round float32 values to bf16 (RNE) and return the uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def special_256x512(seed: int = 1, M: int = 256, K: int = 512) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K), dtype=np.float32)
    t = 32
    x[0:t, 0:t] = 0.0
    a = np.clip(0.5 * rng.standard_normal((t, t), dtype=np.float32), -7.9, 7.9)
    sgn = np.where(np.arange(t) % 2 == 0, 8.0, -8.0).astype(np.float32)
    a[np.arange(t), np.arange(t)] = sgn
    x[t:2 * t, t:2 * t] = a
    x[2 * t:3 * t, 2 * t:3 * t] = 1e-30 * rng.standard_normal((t, t), dtype=np.float32)
    mag = rng.uniform(2.9e38, 3.0e38, size=(t, t)).astype(np.float32)
    sign = np.where(rng.random((t, t)) < 0.5, -1.0, 1.0).astype(np.float32)
    x[3 * t:4 * t, 3 * t:4 * t] = mag * sign
    return bf16_bits(x)


def loguniform_rows(M: int, K: int, seed: int = 2) -> np.ndarray:
    rng = np.random.default_rng(seed)
    u = rng.uniform(-3.0, 3.0, size=M)
    scale = np.power(10.0, u).astype(np.float32)
    out = np.empty((M, K), np.uint16)
    for r0 in range(0, M, CHUNK_ROWS):
        r1 = min(M, r0 + CHUNK_ROWS)
        z = rng.standard_normal((r1 - r0, K), dtype=np.float32)
        z *= scale[r0:r1, None]
        out[r0:r1] = bf16_bits(z)
    return out


def normal(M: int, K: int, seed: int, sigma: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    out = np.empty((M, K), np.uint16)
    s = np.float32(sigma)
    for r0 in range(0, M, CHUNK_ROWS):
        r1 = min(M, r0 + CHUNK_ROWS)
        z = rng.standard_normal((r1 - r0, K), dtype=np.float32)
        if sigma != 1.0:
            z *= s
        out[r0:r1] = bf16_bits(z)
    return out


def student_t_rows(M: int, K: int, seed: int = 5, nu: float = 3.0,
                   frac: float = 0.01, factor: float = 100.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    n_big = int(round(frac * M))
    big = np.zeros(M, bool)
    big[rng.choice(M, size=n_big, replace=False)] = True
    out = np.empty((M, K), np.uint16)
    for r0 in range(0, M, CHUNK_ROWS):
        r1 = min(M, r0 + CHUNK_ROWS)
        z = rng.standard_t(nu, size=(r1 - r0, K)).astype(np.float32)
        z[big[r0:r1]] *= np.float32(factor)
        out[r0:r1] = bf16_bits(z)
    return out


# The five workloads at their full sizes (and the metric run, which reuses the
# 16384^2 log-uniform tensor with both directions in one pass).
FULL = {
    "c1_special": dict(shape=(256, 512)),
    "c2_dim1_16384": dict(shape=(16384, 16384)),
    "c3_gelu_dbias_8192": dict(shape=(8192, 8192)),
    "c4_gated_8192": dict(shape=(8192, 8192)),
    "c5_nvfp4_16384": dict(shape=(16384, 16384)),
}


def moe_group_rows(total: int, groups: int, seed: int, step: int = 16) -> list:
    """Uneven per-expert row counts (multiples of `step`) summing to `total`:
    expert shares drawn from a symmetric Dirichlet(1) (seeded), rounded down to
    the step, the remainder given to the largest expert.  Sizes only; no
    quantisation arithmetic."""
    rng = np.random.default_rng(seed)
    share = rng.dirichlet(np.ones(groups))
    rows = [int(r) // step * step for r in share * total]
    rows[int(np.argmax(rows))] += total - sum(rows)
    return rows


def make(name: str, M: int = None, K: int = None):
    """Inputs of a workload, optionally at a reduced shape with the same recipe."""
    if name == "c1_special":
        return special_256x512(1, M or 256, K or 512)
    if name == "c2_dim1_16384":
        return loguniform_rows(M or 16384, K or 16384, seed=2)
    if name == "c3_gelu_dbias_8192":
        M, K = M or 8192, K or 8192
        return normal(M, K, seed=3, sigma=float(np.sqrt(2.0))), normal(M, K, seed=33)
    if name == "c4_gated_8192":
        return normal(M or 8192, K or 8192, seed=4)
    if name == "c5_nvfp4_16384":
        return student_t_rows(M or 16384, K or 16384, seed=5)
    if name == "f1_dsilu_dbias_8192":
        # the backward of the fused cast: forward input ~N(0, 2), grad ~N(0, 1)
        M, K = M or 8192, K or 8192
        return normal(M, K, seed=6, sigma=float(np.sqrt(2.0))), normal(M, K, seed=66)
    if name == "f1_dgated_8192":
        # gated backward: grad [M][N] ~N(0, 1) and the forward input
        # [gate | linear] [M][2N] ~N(0, 1); here K names N
        M, N = M or 8192, K or 4096
        return normal(M, N, seed=7), normal(M, 2 * N, seed=77)
    if name == "f4_grouped_moe":
        # 8 experts' tokens stacked along rows, N(0, 1); the row counts come
        # from moe_group_rows(M, 8, seed=8)
        return normal(M or 16384, K or 7168, seed=88)
    raise KeyError(name)
