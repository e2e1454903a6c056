"""Seeded synthetic inputs for pixel-aligned projection conditioning.

This module draws inputs only: token coordinates, feature maps, weights, bias
and per-image FOVs. It holds none of the method's arithmetic (no projection, no
sampling, no camera solve), so the GPU path and the CPU oracle can both take
their inputs from it without sharing any computation.

The pages publish no input images, features or weights, so every workload is
synthetic with the pages' shapes: a dense 16^3 grid for the sparse-structure
stage, 1024 DINOv3 channels, 2048 channels where the NAF-upsampled half is
concatenated, a 1536-wide model, surface shells at about 1.4 % occupancy of a
64^3 grid, and a texture stage of about 1e5 tokens with a null (CFG) branch of
the same size.

Sparse tokens follow one recipe ("ellipsoid shell"), per batch item b:
  semi-axes a = R * U(0.35, 0.48)^3 around the centre R/2; directions u drawn
  as normalised N(0, I3) vectors, in batches; voxel = clip(floor(centre + a*u),
  0, R-1); first-seen unique voxels are kept until the item has its target
  count; the item's voxels are sorted lexicographically by (x, y, z) and
  prefixed with b. Random streams are numpy default_rng seeded with
  [seed, b] (coords) or [seed, b, chunk] (maps, drawn in chunks of rows).
"""
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

__all__ = ["Workload", "WORKLOADS", "EXTRA_WORKLOADS", "workload", "shell_coords",
           "feature_map", "feature_maps", "weight", "bias", "fovs", "bf16_bits", "bits_to_f32"]


@dataclass(frozen=True)
class Workload:
    """One synthetic workload. dtype is the map / weight / output type."""
    name: str
    resolution: int
    batch: int
    dense: bool
    tokens_per_item: int          # sparse target per item (dense: R^3)
    height: int
    width: int
    channels: int
    out_dim: int
    dtype: str                    # "f32" or "bf16"
    map_dist: Tuple[str, float, float]   # ("normal", mean, std) / ("uniform", lo, hi)
    bias: str                     # "none", "zeros" or "normal"
    fov: Tuple[str, float, float]  # ("fixed", deg, 0) or ("uniform", lo, hi)
    distance: Optional[float]     # None = closed-form distance for the FOV
    null_rows: bool               # CFG null branch of the same size as the tokens
    seeds: dict = field(default_factory=dict)
    # second map (height, width, channels), concatenated after the first;
    # `channels` is then map 0's and the weight is [out_dim, channels + C1]
    map1: Optional[Tuple[int, int, int]] = None
    points: str = "cell_centres"  # or "grid_nodes"
    # cascade: coords are drawn on a grid of this resolution and must be
    # requantized onto `resolution` nodes before projection
    coords_resolution: Optional[int] = None

    @property
    def n_tokens(self):
        if self.dense:
            return self.batch * self.resolution ** 3
        return self.batch * self.tokens_per_item

    @property
    def n_null(self):
        return self.n_tokens if self.null_rows else 0

    @property
    def k_total(self):
        return self.channels + (self.map1[2] if self.map1 else 0)


WORKLOADS = [
    Workload("dense16_f32_c1024_d1024", 16, 1, True, 16 ** 3, 32, 32, 1024, 1024,
             "f32", ("normal", 0.0, 1.0), "zeros", ("fixed", 40.0, 0.0), 2.0, False,
             dict(map=0, weight=100, bias=101)),
    Workload("dense32_f32_c1024_d1536_border", 32, 1, True, 32 ** 3, 64, 64, 1024, 1536,
             "f32", ("uniform", -3.0, 3.0), "none", ("fixed", 25.0, 0.0), 1.6, False,
             dict(map=200, weight=201)),
    Workload("shell64x2_bf16_c2048_d1536", 64, 2, False, 3500, 128, 128, 2048, 1536,
             "bf16", ("normal", 0.0, 1.0), "none", ("fixed", 40.0, 0.0), None, False,
             dict(coords=1, map=300, weight=301)),
    Workload("shell256x2_bf16_c2048_d1536_bias", 256, 2, False, 100000, 256, 256, 2048, 1536,
             "bf16", ("normal", 0.0, 1.0), "normal", ("uniform", 30.0, 50.0), None, False,
             dict(coords=400, fov=401, map=402, weight=403, bias=404)),
    Workload("shell1024_cfg_bf16_c2048_d1536", 1024, 1, False, 100000, 512, 512, 2048, 1536,
             "bf16", ("normal", 0.0, 1.0), "none", ("fixed", 40.0, 0.0), None, True,
             dict(coords=500, map=501, weight=502)),
]

# Workloads of the adjacent parts:
#  - the cascade: a res-512 shell's coords requantized onto the 64-node
#    high-resolution projection grid (64 cells of 16 res-1024 voxels), then
#    projected as grid nodes; one 2048-channel map as in the texture stage;
#  - two maps: the texture stage's tokens sampled on the DINOv3 map of a
#    1024-pixel image (64 x 64 patches, 1024 channels) and on its upsampled
#    version (512 x 512, 1024 channels), concatenated into 2048 proj channels.
EXTRA_WORKLOADS = [
    Workload("cascade512_grid64_nodes_bf16_c2048_d1536", 64, 1, False, 100000, 512, 512, 2048,
             1536, "bf16", ("normal", 0.0, 1.0), "none", ("fixed", 40.0, 0.0), None, False,
             dict(coords=600, map=601, weight=602), points="grid_nodes",
             coords_resolution=512),
    Workload("shell1024_cfg_twomap_bf16_c1024x2_d1536", 1024, 1, False, 100000, 64, 64, 1024,
             1536, "bf16", ("normal", 0.0, 1.0), "none", ("fixed", 40.0, 0.0), None, True,
             dict(coords=500, map=701, map1=702, weight=703), map1=(512, 512, 1024)),
]


def workload(name_or_index):
    if isinstance(name_or_index, int):
        return WORKLOADS[name_or_index]
    for w in WORKLOADS + EXTRA_WORKLOADS:
        if w.name == name_or_index:
            return w
    raise KeyError(name_or_index)


# ---------------------------------------------------------------- bf16 bits
def bf16_bits(x):
    """float32 -> bf16 bit patterns (uint16), round to nearest even. Inputs
    here are finite draws, so no NaN handling is needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bits_to_f32(bits):
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


# ------------------------------------------------------------------ tokens
def shell_coords(resolution, batch, per_item, seed):
    """int32 [batch*per_item, 4] (b, x, y, z), ellipsoid-shell recipe."""
    R = int(resolution)
    out = []
    for b in range(batch):
        rng = np.random.default_rng([seed, b])
        a = R * rng.uniform(0.35, 0.48, size=3)
        centre = R / 2.0
        seen = {}
        draws = 0
        step = max(4096, per_item)
        while len(seen) < per_item:
            if draws > 400 * per_item:
                raise RuntimeError("shell too small for %d tokens at R=%d" % (per_item, R))
            u = rng.standard_normal((step, 3))
            u /= np.linalg.norm(u, axis=1, keepdims=True)
            v = np.clip(np.floor(centre + a * u), 0, R - 1).astype(np.int64)
            keys = (v[:, 0] * R + v[:, 1]) * R + v[:, 2]
            for k in keys.tolist():
                if k not in seen:
                    seen[k] = None
                    if len(seen) == per_item:
                        break
            draws += step
        keys = np.sort(np.fromiter(seen.keys(), dtype=np.int64, count=per_item))
        xyz = np.stack([keys // (R * R), (keys // R) % R, keys % R], axis=1)
        c = np.empty((per_item, 4), np.int32)
        c[:, 0] = b
        c[:, 1:] = xyz
        out.append(c)
    return np.concatenate(out, axis=0)


def coords(w: Workload):
    """Token coords for a workload (None for the dense grid). For a cascade
    workload these are on the coords_resolution grid (before requantization)."""
    if w.dense:
        return None
    return shell_coords(w.coords_resolution or w.resolution, w.batch, w.tokens_per_item,
                        w.seeds["coords"])


# ------------------------------------------------------------------ tensors
def _draw(rng, dist, shape):
    kind, p, q = dist
    if kind == "normal":
        return (rng.standard_normal(shape, dtype=np.float32) * np.float32(q)
                + np.float32(p))
    if kind == "uniform":
        return rng.uniform(p, q, size=shape).astype(np.float32)
    raise ValueError(kind)


def feature_map(w: Workload, rows_per_chunk=64, which=0):
    """Channels-last [B, H, W, C] map (map `which` of the workload): float32,
    or uint16 bf16 bits."""
    if which == 0:
        B, H, W, C = w.batch, w.height, w.width, w.channels
        seed = w.seeds["map"]
    else:
        (H, W, C), B = w.map1, w.batch
        seed = w.seeds["map1"]
    dt = np.uint16 if w.dtype == "bf16" else np.float32
    out = np.empty((B, H, W, C), dt)

    def chunk(job):
        b, ci = job
        y0 = ci * rows_per_chunk
        y1 = min(H, y0 + rows_per_chunk)
        rng = np.random.default_rng([seed, b, ci])
        x = _draw(rng, w.map_dist, (y1 - y0, W, C))
        out[b, y0:y1] = bf16_bits(x) if w.dtype == "bf16" else x

    jobs = [(b, ci) for b in range(B) for ci in range((H + rows_per_chunk - 1) // rows_per_chunk)]
    with ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(chunk, jobs))
    return out


def feature_maps(w: Workload):
    """The workload's maps as a list (one or two)."""
    return [feature_map(w)] + ([feature_map(w, which=1)] if w.map1 else [])


def weight(w: Workload):
    """proj_linear weight [D, K] ~ N(0, 0.02) (K = summed map channels):
    float32 or bf16 bits."""
    rng = np.random.default_rng([w.seeds["weight"]])
    x = _draw(rng, ("normal", 0.0, 0.02), (w.out_dim, w.k_total))
    return bf16_bits(x) if w.dtype == "bf16" else x


def bias(w: Workload):
    """proj_linear bias [D] or None."""
    if w.bias == "none":
        return None
    if w.bias == "zeros":
        x = np.zeros(w.out_dim, np.float32)
    else:
        rng = np.random.default_rng([w.seeds["bias"]])
        x = _draw(rng, ("normal", 0.0, 0.02), (w.out_dim,))
    return bf16_bits(x) if w.dtype == "bf16" else x


def fovs(w: Workload):
    """Per-item FOV in degrees (list of floats)."""
    kind, p, q = w.fov
    if kind == "fixed":
        return [float(p)] * w.batch
    rng = np.random.default_rng([w.seeds["fov"]])
    return [float(v) for v in rng.uniform(p, q, size=w.batch)]


def random_coords(resolution, batch, n, seed, spill=0):
    """Uniform random cells, for edge-case tests; `spill` widens the range
    past [0, R) on every axis (points outside the unit cube)."""
    rng = np.random.default_rng([seed])
    c = np.empty((n, 4), np.int32)
    c[:, 0] = rng.integers(0, batch, size=n)
    c[:, 1:] = rng.integers(-spill, resolution + spill, size=(n, 3))
    return c
