"""Seeded synthetic inputs shaped like visual-autoregressive workloads.

This module only draws random numbers and lays them out; it contains none of
the attention arithmetic.  Both the GPU library's tests/benchmark and the CPU
oracle consume exactly these bytes.  It imports nothing from the rest of the
package, so importing it never loads the native library.

Workloads (scale schedules of square grids, CFG batch of 2 = cond + uncond
as in "ARVAR ...", Key Design 1):

* ``tiny_fp32``   grids 1,2,3,4 (30 tokens), B=1, H=2, D=32, float32.
* ``var256``      grids 1,2,3,4,5,6,8,10,13,16 (680 tokens), B=2, H=16, D=64, bf16.
* ``var512``      grids 1,2,3,4,6,9,13,18,24,32 (2240 tokens), B=2, H=30, D=64,
                  bf16, sink offset on the first 3 scales.
* ``var1024``     grids 1,2,4,6,8,12,16,20,24,32,40,48,64 (10521 tokens), B=2,
                  H=16, D=128, bf16, sink offset on the first 7 scales.
* ``var1024_sparse``  the same tensors, plus the tile-mask parameters (64x64
                  tiles, 7 sink scales, window radius 2 from scale 7 on) and a
                  seeded 40 % subset of the last step's 4096 query positions
                  scattered over a 48x48 base.

Recipe: ``rng = numpy.random.default_rng(seed)``; draw Q, then K, then V as
float32 N(0, 1) of shape [B, H, L, D]; if the workload has sink scales, draw
u ~ N(0, I_D), normalise it, and add 3u to K on the sink tokens and to Q on all
tokens (an attention-sink-like bias shared by Q and K); finally round to the
workload dtype (bf16 round-to-nearest-even via torch).
"""

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    grids: tuple            # square side of every scale, in order
    batch: int
    heads: int
    head_dim: int
    dtype: str              # "f32" or "bf16"
    sink_offset_scales: int = 0
    # block-sparse / pruned parameters (only for the sparse workload)
    tile: int = 64
    sink_scales: int = 7
    local_from_scale: int = 7
    radius: int = 2
    prune_keep: float = 0.0
    base_grid: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def h(self):
        return list(self.grids)

    @property
    def w(self):
        return list(self.grids)

    @property
    def tokens(self):
        return sum(g * g for g in self.grids)

    @property
    def num_scales(self):
        return len(self.grids)


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", (1, 2, 3, 4), 1, 2, 32, "f32"),
    "var256": Workload("var256", (1, 2, 3, 4, 5, 6, 8, 10, 13, 16), 2, 16, 64, "bf16"),
    "var512": Workload("var512", (1, 2, 3, 4, 6, 9, 13, 18, 24, 32), 2, 30, 64, "bf16",
                       sink_offset_scales=3),
    "var1024": Workload("var1024", (1, 2, 4, 6, 8, 12, 16, 20, 24, 32, 40, 48, 64), 2, 16, 128,
                        "bf16", sink_offset_scales=7),
    "var1024_sparse": Workload("var1024_sparse", (1, 2, 4, 6, 8, 12, 16, 20, 24, 32, 40, 48, 64),
                               2, 16, 128, "bf16", sink_offset_scales=7, tile=64, sink_scales=7,
                               local_from_scale=7, radius=2, prune_keep=0.4, base_grid=48),
}


def custom_workload(grids, batch, heads, head_dim, dtype="bf16", sink_offset_scales=0, name="custom"):
    return Workload(name, tuple(int(g) for g in grids), int(batch), int(heads), int(head_dim),
                    dtype, sink_offset_scales=int(sink_offset_scales))


def make_qkv_f32(wl, seed, grids_hw=None):
    """Float32 numpy Q, K, V [B, H, L, D] following the recipe in the module docstring.

    ``grids_hw`` may give explicit (h, w) pairs for non-square schedules.
    """
    if grids_hw is None:
        sizes = [g * g for g in wl.grids]
    else:
        sizes = [int(a) * int(b) for a, b in grids_hw]
    L = sum(sizes)
    shape = (wl.batch, wl.heads, L, wl.head_dim)
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if wl.sink_offset_scales > 0:
        u = rng.standard_normal(wl.head_dim)
        u = (3.0 * u / np.linalg.norm(u)).astype(np.float32)
        n_sink = sum(sizes[: wl.sink_offset_scales])
        k[:, :, :n_sink, :] += u
        q += u
    return q, k, v


def make_qkv(wl, seed, device="cpu", grids_hw=None):
    """torch tensors of the workload dtype (bf16 rounded RNE, or float32)."""
    import torch

    q, k, v = make_qkv_f32(wl, seed, grids_hw)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    out = []
    for a in (q, k, v):
        t = torch.from_numpy(a)
        out.append(t.to(dt).to(device) if device != "cpu" else t.to(dt))
    return tuple(out)


def pruned_index(n_positions, keep_fraction, seed):
    """Seeded subset of floor(keep_fraction * n) distinct positions, ascending, int32."""
    n_sel = int(np.floor(keep_fraction * n_positions))
    rng = np.random.default_rng(seed + 1)
    idx = rng.choice(n_positions, n_sel, replace=False)
    return np.sort(idx).astype(np.int32)


def random_index(n_positions, n_sel, seed, ascending=True):
    rng = np.random.default_rng(seed + 7)
    idx = rng.choice(n_positions, n_sel, replace=False).astype(np.int32)
    return np.sort(idx) if ascending else idx


def normal_tensor(shape, seed, dtype="f32"):
    """Seeded N(0,1) float32 numpy array (e.g. a stand-in scatter base)."""
    rng = np.random.default_rng(seed + 11)
    return rng.standard_normal(shape, dtype=np.float32)
