"""Seeded synthetic inputs for the Mesh-Attention tile workloads.

This module is shared by the tests, the benchmark and the smoke check.  It
holds workload shapes and random-number generation only: no attention, no
merge, no block classification and no mesh geometry.  Which partitions a
tile holds is decided by the caller (the library's block list on the product
side, the oracle's on the checking side); this module just draws and
concatenates them.

Every (tensor, partition) pair has its own random stream, so two sibling
tiles that hold the same partition see identical values.  "do" is the
gradient of the attention output for the backward (shaped like q).
"""

from dataclasses import dataclass

import numpy as np

TENSORS = ("q", "k", "v", "do", "lse", "delta")


@dataclass(frozen=True)
class Workload:
    """Shape and distribution of one synthetic tile workload."""
    name: str
    dtype: str              # "bf16" or "f32"
    part_len: int           # tokens per sequence partition
    mesh_rows: int
    mesh_cols: int
    tile_row: int
    tile_col: int
    causal: bool
    kv_rotate: bool
    heads_q: int
    heads_kv: int
    head_dim: int
    std: tuple = (1.0, 1.0, 1.0)  # standard deviation of q, k, v (do: 1)
    seed: int = 0
    merge: str = "siblings"  # "siblings" or "per_kv_part"
    numpy_whole_sequence: bool = False  # draw Q, K, V of the whole sequence with numpy

    @property
    def n_parts(self):
        return self.mesh_rows * self.mesh_cols

    @property
    def seq_len(self):
        return self.n_parts * self.part_len


# The five workloads: sequence length, mesh, tile position, heads, dtype and
# value distributions.  The tile position is the middle of the mesh for the
# square meshes (the tile then holds full, diagonal and skipped blocks).
WORKLOADS = {
    1: Workload("f32 non-causal S=2048 d=64, 2x2 mesh, tile (0,0)", "f32", 512, 2, 2, 0, 0,
                False, False, 1, 1, 64, numpy_whole_sequence=True),
    2: Workload("bf16 non-causal MHA 8 heads d=128, 4x4 mesh, L=8192, tile (2,2)", "bf16",
                8192, 4, 4, 2, 2, False, False, 8, 8, 128),
    3: Workload("bf16 causal GQA 32/8 d=128, 4x4 mesh rotated, L=8192, tile (2,2)", "bf16",
                8192, 4, 4, 2, 2, True, True, 32, 8, 128),
    4: Workload("bf16 causal GQA 32/8 d=128, 1M tokens, 8x8 mesh rotated, L=16384, tile (4,4)",
                "bf16", 16384, 8, 8, 4, 4, True, True, 32, 8, 128),
    5: Workload("bf16 causal GQA 64/8 d=128, 1M tokens, 16x4 mesh rotated, L=16384, tile (8,2), "
                "K ~ N(0,4)", "bf16", 16384, 16, 4, 8, 2, True, True, 64, 8, 128,
                std=(1.0, 2.0, 1.0), merge="per_kv_part"),
}


def stream_seed(seed, tensor, part):
    """Seed of the random stream of one (tensor, partition) pair."""
    return (int(seed) * 1_000_003 + TENSORS.index(tensor) * 65_537 + int(part) * 7 + 12_345) % (2**63)


def _std(w, tensor):
    i = TENSORS.index(tensor)
    return float(w.std[i]) if i < len(w.std) else 1.0


def _heads(w, tensor):
    return w.heads_q if tensor in ("q", "do") else w.heads_kv


def _numpy_sequence(w):
    """Whole-sequence draw for the fp32 workload: numpy default_rng(seed)
    produces Q, K, V (then dO) in that order as float64 standard normals, cast
    to fp32."""
    rng = np.random.default_rng(w.seed)
    out = {}
    for t in ("q", "k", "v", "do"):
        x = rng.standard_normal((w.seq_len, _heads(w, t), w.head_dim))
        out[t] = (x * _std(w, t)).astype(np.float32)
    return out


_NUMPY_CACHE = {}


def partition(w, tensor, part, device="cpu"):
    """One partition [part_len, heads, head_dim] of ``tensor`` as a torch tensor."""
    import torch
    if not 0 <= part < w.n_parts:
        raise ValueError("partition id outside the sequence")
    heads = _heads(w, tensor)
    if w.numpy_whole_sequence:
        key = (w, tensor)
        if key not in _NUMPY_CACHE:
            _NUMPY_CACHE.update({(w, t): a for t, a in _numpy_sequence(w).items()})
        a = _NUMPY_CACHE[key][part * w.part_len:(part + 1) * w.part_len]
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(stream_seed(w.seed, tensor, part))
    x = torch.randn((w.part_len, heads, w.head_dim), generator=gen, device=device,
                    dtype=torch.float32)
    if _std(w, tensor) != 1.0:
        x.mul_(_std(w, tensor))
    return x.to(torch_dtype(w.dtype))


def gather(w, tensor, parts, device="cpu"):
    """Concatenate partitions ``parts`` (slot order) into [len*part_len, heads, d]."""
    import torch
    return torch.cat([partition(w, tensor, p, device) for p in parts], dim=0).contiguous()


def row_terms(w, parts, device="cpu"):
    """Synthetic per-row lse and D for the backward, float32 [len*part_len, H_q]:
    lse uniform in [10, 14) (the size of ln(sum exp) over tens of thousands of
    keys with unit-variance scores) and D standard normal.  Used where the
    backward is checked as a function of given lse and D."""
    import torch
    out = []
    for name in ("lse", "delta"):
        parts_out = []
        for part in parts:
            gen = torch.Generator(device=device)
            gen.manual_seed(stream_seed(w.seed, name, part))
            shape = (w.part_len, w.heads_q)
            if name == "lse":
                x = 10.0 + 4.0 * torch.rand(shape, generator=gen, device=device, dtype=torch.float32)
            else:
                x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
            parts_out.append(x)
        out.append(torch.cat(parts_out, dim=0).contiguous())
    return out[0], out[1]


def torch_dtype(name):
    import torch
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def small(dtype="bf16", part_len=64, mesh_rows=2, mesh_cols=2, tile_row=0, tile_col=0,
          causal=True, kv_rotate=True, heads_q=4, heads_kv=2, head_dim=128, seed=0,
          std=None):
    """A small workload for parity tests (oracle-sized)."""
    return Workload(f"small {dtype} L={part_len} {mesh_rows}x{mesh_cols} ({tile_row},{tile_col}) "
                    f"causal={int(causal)} rot={int(kv_rotate)} H={heads_q}/{heads_kv} d={head_dim}",
                    dtype, part_len, mesh_rows, mesh_cols, tile_row, tile_col, causal, kv_rotate,
                    heads_q, heads_kv, head_dim,
                    std=tuple(std or (1.0, 1.0, 1.0)), seed=seed)


def sample_rows(n_tokens, heads_q, heads_kv, part_len, n_sample=1024, seed=1):
    """Seeded (token, head) rows to check on large tiles, plus forced edge rows:
    tokens 0, 1, L/2 and L-1 of every Q slot, each with query heads 0, G-1, G
    and H_q-1 (G = heads_q / heads_kv)."""
    rng = np.random.default_rng(seed)
    tok = rng.integers(0, n_tokens, size=n_sample)
    head = rng.integers(0, heads_q, size=n_sample)
    rows = set(zip(tok.tolist(), head.tolist()))
    group = heads_q // heads_kv
    edge_heads = sorted({0, group - 1, min(group, heads_q - 1), heads_q - 1})
    for s in range(n_tokens // part_len):
        for u in sorted({0, 1 % part_len, part_len // 2, part_len - 1}):
            for h in edge_heads:
                rows.add((s * part_len + u, h))
    return np.array(sorted(rows), dtype=np.int64)
