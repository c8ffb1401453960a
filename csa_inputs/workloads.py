"""Seeded synthetic workloads: the five shard configurations and small variants.

Every array is drawn from ``numpy.random.default_rng(seed)`` as float32
standard normals (uniform for the indexer weights), in a fixed draw order:
queries (local rows in physical order), keys (the full gathered stream),
values, then the extras of the configuration.  bf16 workloads round each draw
to bfloat16 by round-to-nearest-even and keep the exact bf16 values in float32
arrays, so that the GPU path (which converts them to bf16 without loss) and
the fp64 oracle (which widens them without loss) read identical numbers.

The five named workloads:

* ``dense_f32``   - 512 tokens, 2 heads, D=64, fp32; contiguous shard of 128
  queries at offset 256 (cp 4, rank 2); blocks of 64 and top-8, which admits
  every permitted block, so the result is dense causal attention.
* ``moba_mha_8k`` - 8192 tokens, 16 heads, D=128, bf16; last 2048 queries
  (cp 4, rank 3); blocks of 512, top-3 past blocks plus the own block.
* ``moba_gqa_zigzag_32k`` - 32768 tokens, 32 query / 8 kv heads, D=128, bf16;
  zigzag cp 4, rank 1 (chunks 1 and 6 of 8); blocks of 1024, top-4 plus own;
  13 of the 256 (kv head, block) pairs get +2 on every key component.
* ``dsa_mla_16k`` - absorbed-MLA shape: 128 query heads share one latent key
  head of width 576 (512 latent + 64 rope); the value is the first 512
  columns of the key; 16384 tokens, 4096 queries at offset 8192; indexer with
  64 heads of width 128 and weights U(0,1); top-2048 tokens.
* ``moba_thd_64k`` - 65536 packed tokens from sequences with lengths drawn
  uniformly from [1024, 16384] until they cover the stream (last one trimmed),
  zigzag over the packed stream for cp 4, rank 0; 32 query / 4 kv heads,
  D=128; blocks of 512, top-4 plus own.
"""

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

from .layout import (
    contiguous_positions,
    zigzag_positions,
    seq_ids_for_positions,
    cu_from_lengths,
)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); float32 result."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    return rounded.astype(np.uint32).view(np.float32).reshape(x.shape)


@dataclass
class Workload:
    name: str
    dtype: str  # "f32" or "bf16": the element type of q, k, v (and iq, ik)
    mode: str  # "block" (MoBA gating) or "token" (DSA indexer)
    q: np.ndarray  # [n_q, hq, dqk]
    k: np.ndarray  # [n_kv, hkv, dqk]
    v: Optional[np.ndarray]  # [n_kv, hkv, dv]; None when the value aliases k[..., :dv]
    dv: int
    q_pos: np.ndarray  # [n_q] int32 global (packed) position of each local row
    q_seq: np.ndarray  # [n_q] int32 sequence id of each local row
    cu_seqlens: np.ndarray  # [n_seq + 1] int32
    topk: int
    scale: float
    block_size: int = 0  # block mode only
    iq: Optional[np.ndarray] = None  # token mode: [n_q, hi, di]
    ik: Optional[np.ndarray] = None  # token mode: [n_kv, di]
    w: Optional[np.ndarray] = None  # token mode: [n_q, hi] float32
    info: dict = field(default_factory=dict)

    @property
    def n_q(self):
        return self.q.shape[0]

    @property
    def n_kv(self):
        return self.k.shape[0]

    @property
    def hq(self):
        return self.q.shape[1]

    @property
    def hkv(self):
        return self.k.shape[1]

    @property
    def dqk(self):
        return self.q.shape[2]

    @property
    def value(self) -> np.ndarray:
        """The value tensor (a view of k when aliased)."""
        return self.v if self.v is not None else self.k[..., : self.dv]

    @property
    def v_alias(self) -> bool:
        return self.v is None


def _normal(rng, shape, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return bf16_round(x) if dtype == "bf16" else x


def _uniform(rng, shape):
    return rng.random(size=shape, dtype=np.float32)


def _block_workload(name, seed, dtype, lengths, positions, hq, hkv, d, block, topk,
                    q_rows_full=None, key_bias=None):
    rng = np.random.default_rng(seed)
    cu = cu_from_lengths(lengths)
    n_kv = int(cu[-1])
    if q_rows_full is not None:
        # draw every row of the stream, then keep the shard's rows
        q = _normal(rng, (q_rows_full, hq, d), dtype)[positions]
    else:
        q = _normal(rng, (len(positions), hq, d), dtype)
    k_raw = rng.standard_normal(size=(n_kv, hkv, d), dtype=np.float32)
    v = _normal(rng, (n_kv, hkv, d), dtype)
    info = {}
    if key_bias is not None:
        n_pairs, amount = key_bias
        n_blocks = n_kv // block
        chosen = rng.choice(n_blocks * hkv, size=n_pairs, replace=False)
        for p in chosen:
            b, g = divmod(int(p), hkv)
            k_raw[b * block:(b + 1) * block, g, :] += amount
        info["biased_pairs"] = sorted((int(p) // hkv, int(p) % hkv) for p in chosen)
    k = bf16_round(k_raw) if dtype == "bf16" else k_raw
    q_seq = seq_ids_for_positions(positions, cu)
    return Workload(name=name, dtype=dtype, mode="block", q=np.ascontiguousarray(q), k=k,
                    v=v, dv=d, q_pos=np.asarray(positions, np.int32), q_seq=q_seq,
                    cu_seqlens=cu, topk=topk, scale=1.0 / np.sqrt(d), block_size=block,
                    info=info)


def _dense_f32():
    pos = contiguous_positions(512, 4, 2)
    return _block_workload("dense_f32", 1, "f32", [512], pos, 2, 2, 64, 64, 8,
                           q_rows_full=512)


def _moba_mha_8k():
    pos = contiguous_positions(8192, 4, 3)
    return _block_workload("moba_mha_8k", 2, "bf16", [8192], pos, 16, 16, 128, 512, 3)


def _moba_gqa_zigzag_32k():
    pos = zigzag_positions(32768, 4, 1)
    n_pairs = int(round(0.05 * (32768 // 1024) * 8))
    return _block_workload("moba_gqa_zigzag_32k", 3, "bf16", [32768], pos, 32, 8, 128,
                           1024, 4, key_bias=(n_pairs, 2.0))


def _thd_lengths(rng, total, lo, hi):
    lengths = []
    while sum(lengths) < total:
        lengths.append(int(rng.integers(lo, hi + 1)))
    lengths[-1] -= sum(lengths) - total
    return lengths


def _moba_thd_64k():
    rng = np.random.default_rng(5)
    total, hq, hkv, d = 65536, 32, 4, 128
    pos = zigzag_positions(total, 4, 0)
    q = _normal(rng, (len(pos), hq, d), "bf16")
    k = _normal(rng, (total, hkv, d), "bf16")
    v = _normal(rng, (total, hkv, d), "bf16")
    lengths = _thd_lengths(rng, total, 1024, 16384)
    cu = cu_from_lengths(lengths)
    return Workload(name="moba_thd_64k", dtype="bf16", mode="block", q=q, k=k, v=v, dv=d,
                    q_pos=pos, q_seq=seq_ids_for_positions(pos, cu), cu_seqlens=cu,
                    topk=4, scale=1.0 / np.sqrt(d), block_size=512,
                    info={"lengths": lengths})


def _token_workload(name, seed, dtype, lengths, positions, hq, dqk, dv, hi, di, topk):
    rng = np.random.default_rng(seed)
    cu = cu_from_lengths(lengths)
    n_kv = int(cu[-1])
    q = _normal(rng, (len(positions), hq, dqk), dtype)
    k = _normal(rng, (n_kv, 1, dqk), dtype)
    iq = _normal(rng, (len(positions), hi, di), dtype)
    ik = _normal(rng, (n_kv, di), dtype)
    w = _uniform(rng, (len(positions), hi))
    return Workload(name=name, dtype=dtype, mode="token", q=q, k=k, v=None, dv=dv,
                    q_pos=np.asarray(positions, np.int32),
                    q_seq=seq_ids_for_positions(positions, cu), cu_seqlens=cu, topk=topk,
                    scale=1.0 / np.sqrt(dqk), iq=iq, ik=ik, w=w)


def _dsa_mla_16k():
    pos = np.arange(8192, 8192 + 4096, dtype=np.int32)
    return _token_workload("dsa_mla_16k", 4, "bf16", [16384], pos, 128, 576, 512, 64, 128,
                           2048)


_BUILDERS = {
    "dense_f32": _dense_f32,
    "moba_mha_8k": _moba_mha_8k,
    "moba_gqa_zigzag_32k": _moba_gqa_zigzag_32k,
    "dsa_mla_16k": _dsa_mla_16k,
    "moba_thd_64k": _moba_thd_64k,
}
WORKLOAD_NAMES = list(_BUILDERS)


def make_workload(name_or_index) -> Workload:
    """Build a named workload; an int 1..5 selects by position in ``WORKLOAD_NAMES``."""
    if isinstance(name_or_index, int):
        name_or_index = WORKLOAD_NAMES[name_or_index - 1]
    return _BUILDERS[name_or_index]()


def tiny_block_workload(seed=0, lengths=(40, 24), layout="contiguous", cp=2, rank=1,
                        positions=None, hq=4, hkv=2, d=8, block=8, topk=2, dtype="f32",
                        key_bias=None):
    """Small block-mode workload over a packed stream of ``lengths``."""
    total = int(sum(lengths))
    if positions is None:
        if layout == "contiguous":
            positions = contiguous_positions(total, cp, rank)
        elif layout == "zigzag":
            positions = zigzag_positions(total, cp, rank)
        elif layout == "all":
            positions = np.arange(total, dtype=np.int32)
        else:
            raise ValueError(layout)
    return _block_workload(f"tiny_block_{seed}", seed, dtype, list(lengths),
                           np.asarray(positions, np.int32), hq, hkv, d, block, topk,
                           key_bias=key_bias)


def tiny_token_workload(seed=0, lengths=(48, 16), positions=None, hq=4, dqk=12, dv=8,
                        hi=3, di=8, topk=5, dtype="f32"):
    """Small token-mode workload (one latent key head, value = first dv key columns)."""
    total = int(sum(lengths))
    if positions is None:
        positions = np.arange(total, dtype=np.int32)
    return _token_workload(f"tiny_token_{seed}", seed, dtype, list(lengths),
                           np.asarray(positions, np.int32), hq, dqk, dv, hi, di, topk)


def up_projection_inputs(n_q, hq, dl, dv, seed=11):
    """Inputs of the absorbed-MLA value up-projection, as exact bf16 values in float32.

    o [n_q, hq, dl]: stands in for the latent attention output, a convex
    combination of latent value rows drawn N(0, 1), so N(0, 1) entries scaled by
    1/2; w [hq, dv, dl]: each head's up-projection (linear-layer layout, rows =
    output channels), N(0, 1/dl) as at initialisation.
    """
    rng = np.random.default_rng(seed)
    o = bf16_round(0.5 * rng.standard_normal(size=(n_q, hq, dl), dtype=np.float32))
    w = bf16_round(rng.standard_normal(size=(hq, dv, dl), dtype=np.float32) / np.float32(np.sqrt(dl)))
    return o, w
