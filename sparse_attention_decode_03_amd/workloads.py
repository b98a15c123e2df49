"""Seeded synthetic workloads for the DSA decode path.

This module only draws inputs. It holds none of the method's arithmetic: it
does not score, select or attend, and both the HIP path and the CPU oracle
read the very bytes it produces. Number-format encoding (fp32 -> bf16 and
fp32 -> OCP E4M3 with saturation) goes through torch's CPU casts, which are
round-to-nearest-even.

Layouts (all little-endian, C-contiguous):
  seq_lens      [R]                 int32, R = num_seqs * rows_per_seq, rows
                                    sequence-major (r = s * K + j)
  q_idx         [R, Hi, D]          bf16 codes (uint16)
  w             [R, Hi]             float32, already carrying Hi^-0.5
  k_normed      [S, k_capacity, D]  bf16 codes; rows at or past the longest
                                    row of a sequence hold the bf16 NaN 0x7FC0
                                    (nothing may read them)
  q             [R, H, 512]         bf16 codes (latent-absorbed query)
  kv_cache      [num_pages, ps, 512] OCP E4M3 bytes; slots past a sequence's
                                    last token hold the NaN code 0x7F
  block_tables  [S, max_blocks]     int32 physical page ids, -1 past the last
                                    page a sequence needs; the physical pages
                                    of all sequences are one random permutation
Scalars: top_k, page_size, kv_scale, sm_scale.

Draw order from numpy's PCG64(seed): ragged lengths, page permutation,
q_idx, w, q, then per sequence the keys and the latent rows.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

BF16_NAN = 0x7FC0
E4M3_NAN = 0x7F
E4M3_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    num_seqs: int
    rows_per_seq: int
    num_heads: int
    index_heads: int
    index_dim: int
    top_k: int
    page_size: int
    seed: int
    # lengths: "fixed" -> every row at `context`; "ragged" -> per sequence
    # uniform integer in [lo, hi]; "verify" -> row j of a sequence at base + j + 1
    lengths: str = "fixed"
    context: int = 0
    lo: int = 0
    hi: int = 0
    base: int = 0
    key_dist: str = "normal"  # or "student_t3"
    latent_dim: int = 512
    kv_scale: float = 0.5
    sm_scale: float = 1.0 / math.sqrt(512.0)

    @property
    def num_rows(self) -> int:
        return self.num_seqs * self.rows_per_seq


# The five workloads of the benchmark, in order (seeds 0..4), and the
# row-group shape: 16 consecutive query rows of a sequence selected in one
# pass, as the pages' prefill does it (layer.rs, the prefill row-group
# selector, 16 rows of a 9,000-token prefill), here for 8 sequences.
WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 1, 1, 8, 4, 64, 64, 16, seed=0, context=256),
    "single": Workload("single", 1, 1, 64, 32, 128, 2048, 64, seed=1, context=8192),
    "batched": Workload("batched", 32, 1, 64, 32, 128, 2048, 64, seed=2,
                        lengths="ragged", lo=1024, hi=32768),
    "kverify": Workload("kverify", 16, 4, 64, 32, 128, 2048, 64, seed=3,
                        lengths="verify", base=16384),
    "long": Workload("long", 8, 1, 64, 32, 128, 2048, 64, seed=4, context=131072,
                     key_dist="student_t3"),
    "rowgroup": Workload("rowgroup", 8, 16, 64, 32, 128, 2048, 64, seed=5,
                         lengths="verify", base=9000),
}


def f32_to_bf16_codes(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32_to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """Round to nearest even, saturating at +-448 (clamp first: torch's cast
    turns overflow into NaN)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.clamp_(-E4M3_MAX, E4M3_MAX)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def row_lengths(wl: Workload, rng: np.random.Generator) -> np.ndarray:
    S, K = wl.num_seqs, wl.rows_per_seq
    if wl.lengths == "fixed":
        per_seq = np.full(S, wl.context, dtype=np.int64)
        lens = np.repeat(per_seq, K)
    elif wl.lengths == "ragged":
        per_seq = rng.integers(wl.lo, wl.hi, size=S, endpoint=True)
        lens = np.repeat(per_seq, K)
    elif wl.lengths == "verify":
        lens = np.tile(np.arange(K, dtype=np.int64) + wl.base + 1, S)
    else:
        raise ValueError(f"unknown length law {wl.lengths!r}")
    return lens.astype(np.int32)


def make_inputs(wl: Workload, seed: Optional[int] = None) -> dict:
    """Draw every input of one decode step for workload `wl`."""
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    S, K, R = wl.num_seqs, wl.rows_per_seq, wl.num_rows
    H, Hi, D, Dl, ps = wl.num_heads, wl.index_heads, wl.index_dim, wl.latent_dim, wl.page_size

    seq_lens = row_lengths(wl, rng)
    seq_max = seq_lens.reshape(S, K).max(axis=1)
    k_capacity = int(seq_max.max()) if S else 0
    max_len = k_capacity
    pages_per_seq = (seq_max + ps - 1) // ps
    num_pages = int(pages_per_seq.sum())
    max_blocks = int(pages_per_seq.max()) if S else 0

    perm = rng.permutation(num_pages).astype(np.int32)
    block_tables = np.full((S, max(max_blocks, 1)), -1, dtype=np.int32)
    off = 0
    for s in range(S):
        n = int(pages_per_seq[s])
        block_tables[s, :n] = perm[off:off + n]
        off += n

    q_idx = f32_to_bf16_codes(rng.standard_normal((R, Hi, D), dtype=np.float32))
    w = (rng.random((R, Hi), dtype=np.float32) * np.float32(Hi ** -0.5)).astype(np.float32)
    q = f32_to_bf16_codes(rng.standard_normal((R, H, Dl), dtype=np.float32))

    k_normed = np.full((S, k_capacity, D), BF16_NAN, dtype=np.uint16)
    kv_cache = np.full((num_pages, ps, Dl), E4M3_NAN, dtype=np.uint8)
    inv_scale = np.float32(1.0 / wl.kv_scale)
    for s in range(S):
        L = int(seq_max[s])
        if wl.key_dist == "normal":
            keys = rng.standard_normal((L, D), dtype=np.float32)
        elif wl.key_dist == "student_t3":
            keys = rng.standard_t(3, size=(L, D)).astype(np.float32)
        else:
            raise ValueError(f"unknown key law {wl.key_dist!r}")
        k_normed[s, :L] = f32_to_bf16_codes(keys)
        del keys
        lat = f32_to_e4m3_codes(rng.standard_normal((L, Dl), dtype=np.float32) * inv_scale)
        pages = block_tables[s, :int(pages_per_seq[s])]
        full = L // ps
        if full:
            kv_cache[pages[:full]] = lat[:full * ps].reshape(full, ps, Dl)
        if L % ps:
            kv_cache[pages[full], :L % ps] = lat[full * ps:]
        del lat

    return dict(
        workload=wl,
        seq_lens=seq_lens,
        q_idx=q_idx,
        w=w,
        k_normed=k_normed,
        q=q,
        kv_cache=kv_cache,
        block_tables=block_tables,
        num_seqs=S,
        rows_per_seq=K,
        num_heads=H,
        latent_dim=Dl,
        index_heads=Hi,
        index_dim=D,
        top_k=wl.top_k,
        page_size=ps,
        max_len=max_len,
        k_capacity=k_capacity,
        max_blocks=block_tables.shape[1],
        num_pages=num_pages,
        kv_scale=float(wl.kv_scale),
        sm_scale=float(wl.sm_scale),
    )


def custom(name: str = "custom", **kw) -> Workload:
    """A workload with the shape of `single` unless overridden."""
    base = dataclasses.asdict(WORKLOADS["single"])
    base.update(name=name)
    base.update(kw)
    return Workload(**base)

