"""Seeded synthetic inputs shaped like the pages' workloads.

This module only draws random data. It holds none of the quantisation
arithmetic, and both the HIP path's tests and the CPU oracle consume the
same host bytes it returns.

Workloads (page titles, then the table or passage that fixes the shape):

* dim0 per-token-group shapes (256, 4096), (4096, 4096), (65536, 4096) with
  4-16 groups: "[moe training] use smaller block sizes for per group scaling
  kernels to improve perf", old and new autotuner tables.
* dim1 per-group rowwise shape (16640, 8192) with 1, 16 and 64 groups:
  "[moe fp8 training] test and bench new faster method for per group rowwise
  scaling", Benchmarks table.
* MX dim0 cast on a (16, 8192, 5120) token batch: "[mxfp8 moe training] fix
  mxfp8 a2a bench script; set mxfp8 a2a scaling type to RCEIL", results table.
* Value scale 0.02 and token-group alignment 16: the test source quoted in the
  torch.compile failure report of the block-size page (init_std, group
  alignment setter).

Recipe: numpy ``default_rng(seed)`` (PCG64); standard normals drawn in fp32,
times sigma, rounded to bf16 with round-to-nearest-even; outliers at exactly
``round(0.001 * numel)`` distinct positions, each +-magnitude with a random
sign; uniform group sizes are 16 x the gaps between G-1 sorted uniform
integers in [0, extent/16] (empty groups allowed); Dirichlet sizes are
``dirichlet([alpha] * G) * extent/16`` rounded, with the residual put on the
largest group.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np

ALIGN = 16


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def randn_bf16(rng: np.random.Generator, shape, sigma: float,
               outlier_frac: float = 0.0, outlier_mag: float = 0.0,
               chunk: int = 1 << 26) -> np.ndarray:
    """bf16 bits of sigma * N(0, 1) with optional +-outlier_mag outliers."""
    numel = int(np.prod(shape))
    out = np.empty(numel, dtype=np.uint16)
    for lo in range(0, numel, chunk):
        hi = min(numel, lo + chunk)
        v = rng.standard_normal(hi - lo, dtype=np.float32)
        v *= np.float32(sigma)
        out[lo:hi] = f32_to_bf16_bits(v)
    if outlier_frac > 0.0 and numel > 0:
        n_out = int(round(outlier_frac * numel))
        if n_out > 0:
            pos = rng.choice(numel, size=n_out, replace=False)
            sign = rng.integers(0, 2, size=n_out)
            mags = np.where(sign == 1, -outlier_mag, outlier_mag).astype(np.float32)
            out[pos] = f32_to_bf16_bits(mags)
    return out.reshape(shape)


def uniform_group_offsets(rng: np.random.Generator, extent: int, G: int,
                          align: int = ALIGN) -> np.ndarray:
    """int32 end offsets of G groups with random multiple-of-align sizes."""
    if extent % align != 0:
        raise ValueError("extent must be a multiple of the alignment")
    units = extent // align
    cuts = np.sort(rng.integers(0, units + 1, size=G - 1))
    ends = np.concatenate([cuts, [units]]) * align
    return ends.astype(np.int32)


def dirichlet_group_offsets(rng: np.random.Generator, extent: int, G: int,
                            alpha: float = 0.5, align: int = ALIGN) -> np.ndarray:
    units = extent // align
    p = rng.dirichlet([alpha] * G)
    sizes = np.rint(p * units).astype(np.int64)
    sizes[int(np.argmax(sizes))] += units - int(sizes.sum())
    return (np.cumsum(sizes) * align).astype(np.int32)


def sizes_from_offsets(offsets: np.ndarray) -> np.ndarray:
    off = np.asarray(offsets, dtype=np.int64)
    return np.diff(np.concatenate([[0], off]))


@dataclasses.dataclass
class Workload:
    name: str
    kind: str                  # "dim0" | "dim1" | "mx"
    x: np.ndarray              # uint16 bf16 bits, (M, K) row-major
    offsets: Optional[np.ndarray]
    pow2: bool = False
    modes: tuple = ()
    note: str = ""

    @property
    def shape(self):
        return self.x.shape

    def sha256(self) -> str:
        h = hashlib.sha256(self.x.tobytes())
        if self.offsets is not None:
            h.update(self.offsets.tobytes())
        return h.hexdigest()

    def algorithmic_bytes(self) -> int:
        """Minimum bytes the method moves: read x once, write q once, write
        the scales (and read the offsets)."""
        M, K = self.x.shape
        if self.kind == "mx":
            return M * K * 2 + M * K + M * (K // 32)
        G = len(self.offsets)
        n_scales = G * K if self.kind == "dim0" else M * G
        return M * K * 2 + M * K + n_scales * 4 + G * 4


def c1_dim0_small(seed: int = 1) -> Workload:
    """(256, 4096) bf16, randn*0.02 + 0.1% outliers at +-8, G=4."""
    rng = np.random.default_rng(seed)
    x = randn_bf16(rng, (256, 4096), 0.02, 0.001, 8.0)
    off = uniform_group_offsets(rng, 256, 4)
    return Workload("dim0 (256,4096) G=4", "dim0", x, off)


def c2_dim0_pow2(seed: int = 2) -> Workload:
    """(4096, 4096), G=16, one empty group, one all-zero group, pow2 scales."""
    rng = np.random.default_rng(seed)
    x = randn_bf16(rng, (4096, 4096), 0.02, 0.001, 8.0)
    off = uniform_group_offsets(rng, 4096, 16)
    sizes = sizes_from_offsets(off)
    # force one empty group: merge group 3 into group 4
    if sizes[3] != 0:
        sizes[4] += sizes[3]
        sizes[3] = 0
    off = np.cumsum(sizes).astype(np.int32)
    # zero all rows of the first non-empty group after the empty one
    nz = [g for g in range(16) if sizes[g] > 0 and g > 3]
    gz = nz[0]
    r0 = int(off[gz - 1]) if gz > 0 else 0
    x[r0:int(off[gz])] = 0
    return Workload("dim0 (4096,4096) G=16 pow2", "dim0", x, off, pow2=True,
                    note="group 3 empty, group %d all zero" % gz)


def c3_dim0_large(seed: int = 3) -> Workload:
    """(65536, 4096) randn*1.0, G=8 with Dirichlet(0.5) sizes."""
    rng = np.random.default_rng(seed)
    x = randn_bf16(rng, (65536, 4096), 1.0)
    off = dirichlet_group_offsets(rng, 65536, 8, 0.5)
    return Workload("dim0 (65536,4096) G=8 dirichlet", "dim0", x, off)


def token_major_gradient(seed: int = 4) -> np.ndarray:
    """T (16640, 8192) bf16 randn*0.02, the token-major gradient."""
    rng = np.random.default_rng(seed)
    return randn_bf16(rng, (16640, 8192), 0.02)


def target_offsets(G: int) -> np.ndarray:
    """Uniform multiple-of-16 group sizes summing to 16640 (seed 40 + G)."""
    return uniform_group_offsets(np.random.default_rng(40 + G), 16640, G)


def c4_dim1(G: int, T: Optional[np.ndarray] = None) -> Workload:
    """(8192, 16640) = T transposed, made contiguous; groups along dim1."""
    if T is None:
        T = token_major_gradient()
    return Workload("dim1 (8192,16640) G=%d" % G, "dim1",
                    np.ascontiguousarray(T.T), target_offsets(G))


def c6_dim0_target(G: int = 64, T: Optional[np.ndarray] = None) -> Workload:
    """T (16640, 8192) itself, groups along dim0 (the target's dim0 half)."""
    if T is None:
        T = token_major_gradient()
    return Workload("dim0 (16640,8192) G=%d" % G, "dim0", T, target_offsets(G))


def c5_mx(seed: int = 5, M: int = 131072, K: int = 5120) -> Workload:
    """(131072, 5120) randn*1.0 + 0.1% outliers at +-100; block-32 MX cast."""
    rng = np.random.default_rng(seed)
    x = randn_bf16(rng, (M, K), 1.0, 0.001, 100.0)
    return Workload("mx dim0 (%d,%d)" % (M, K), "mx", x, None, modes=(0, 1))
