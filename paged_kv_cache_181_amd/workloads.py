"""Seeded synthetic inputs for paged-KV decode (shared by tests and bench).

Holds only random draws, their 16-bit encodings and the harness bookkeeping
(block tables, slot lists, accept counts).  It performs none of the attention
or quantization arithmetic and imports neither the HIP binding nor the oracle.

Workloads follow the shapes the pages describe: single-user long-context
decode ("The KV Cache", arithmetic and layout paragraphs), batched decode with
rows that advance at different rates ("How MTPLX Manages Memory with KV Caching
Strategies", RaggedBatchKVCache), speculative verify with rollback (mlxcel
"KV Cache", Speculative Rewind) and K8/V4 storage ("The KV Cache", K/V
asymmetry).  Random draws use ``numpy.random.Generator(PCG64(seed))`` in a
fixed order: lengths, table permutation, K, V, query, new K/V, accept counts.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BLOCK_SIZE = 16


def rng_for(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bits(x: np.ndarray, fmt: str) -> np.ndarray:
    """Round float32 draws to fp16 or bf16 (nearest-even) and return the bits."""
    x = np.asarray(x, dtype=np.float32)
    if fmt == "f16":
        return x.astype(np.float16).view(np.uint16)
    if fmt == "bf16":
        u = x.view(np.uint32)
        # nearest-even: add 0x7FFF plus the lowest kept bit, then truncate
        # (finite inputs only: the sum cannot wrap)
        t = u >> np.uint32(16)
        t &= np.uint32(1)
        t += np.uint32(0x7FFF)
        t += u
        t >>= np.uint32(16)
        return t.astype(np.uint16)
    raise ValueError(fmt)


def normal_bits(rng: np.random.Generator, shape, fmt: str) -> np.ndarray:
    """~N(0,1) float32 draws stored as fp16/bf16 bits."""
    return f32_to_bits(rng.standard_normal(size=shape, dtype=np.float32), fmt)


@dataclass
class PagedCase:
    """One decode step's inputs: pool, tables, lengths, query and new tokens."""
    name: str
    batch: int
    q_len: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    fmt: str                          # storage of K/V as drawn: "f16" or "bf16"
    num_blocks: int
    context_lens: np.ndarray          # int32 [B]; includes this step's q_len tokens
    block_tables: np.ndarray          # int32 [B, max_blocks]; unused entries = -1
    key_cache: np.ndarray             # uint16 [NB, 16, Hkv, D]
    value_cache: np.ndarray           # uint16 [NB, 16, Hkv, D]
    query: np.ndarray                 # uint16 [B, Q, Hq, D]
    new_key: np.ndarray               # uint16 [T, Hkv, D]
    new_value: np.ndarray             # uint16 [T, Hkv, D]
    slot_mapping: np.ndarray          # int64 [T]
    scale: float
    block_size: int = BLOCK_SIZE
    accepted: Optional[np.ndarray] = None     # int32 [B] (verify workloads)
    extra: dict = field(default_factory=dict)

    @property
    def gqa_factor(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_blocks(self) -> int:
        return self.block_tables.shape[1]


def slot_of(block_tables: np.ndarray, b: int, pos: int, block_size: int = BLOCK_SIZE) -> int:
    """Harness bookkeeping: the cache slot assigned to position ``pos`` of row ``b``."""
    return int(block_tables[b, pos // block_size]) * block_size + pos % block_size


def build_tables(rng, blocks_needed, num_blocks, max_blocks=None):
    """Disjoint random block picks from a pool: a seeded permutation of the
    pool is cut into consecutive chunks of ``blocks_needed[b]`` entries."""
    blocks_needed = np.asarray(blocks_needed, dtype=np.int64)
    total = int(blocks_needed.sum())
    if total > num_blocks:
        raise ValueError("pool too small")
    perm = rng.permutation(num_blocks).astype(np.int32)
    mb = int(max_blocks if max_blocks is not None else max(1, blocks_needed.max()))
    tables = np.full((len(blocks_needed), mb), -1, dtype=np.int32)
    start = 0
    for b, n in enumerate(blocks_needed.tolist()):
        tables[b, :n] = perm[start:start + n]
        start += n
    return tables


def fill_pool(rng, tables, blocks_needed, num_blocks, num_kv_heads, head_dim, fmt):
    """K and V pools with ~N(0,1) values in every referenced block (all 16 rows,
    so rows past a sequence's length hold ordinary values); other blocks are 0.
    K is drawn for all referenced blocks (in table order), then V."""
    shape = (num_blocks, BLOCK_SIZE, num_kv_heads, head_dim)
    used = np.concatenate([tables[b, :n] for b, n in enumerate(blocks_needed)]) \
        if len(blocks_needed) else np.zeros(0, np.int32)
    kc = np.zeros(shape, dtype=np.uint16)
    vc = np.zeros(shape, dtype=np.uint16)
    chunk = 2048
    for pool in (kc, vc):
        for s in range(0, len(used), chunk):
            ids = used[s:s + chunk]
            pool[ids] = normal_bits(rng, (len(ids),) + shape[1:], fmt)
    return kc, vc


@dataclass
class Layout:
    """Lengths, block tables and this step's slots, without any K/V values."""
    context_lens: np.ndarray
    block_tables: np.ndarray
    num_blocks: int
    slot_mapping: np.ndarray
    blocks_needed: np.ndarray


def make_layout(rng, *, batch: int, q_len: int, lengths, num_blocks: Optional[int] = None,
                spare_blocks: int = 0, extra_positions: int = 0) -> Layout:
    """Draw the lengths (if a callable) and the table permutation.  Tables
    cover ``length + extra_positions`` positions per row so that a follow-up
    write (after a verify step) always has a block."""
    lengths_arr = np.asarray(lengths(rng) if callable(lengths) else lengths, dtype=np.int64)
    if lengths_arr.shape != (batch,):
        raise ValueError("lengths must have one entry per row")
    need = (lengths_arr + extra_positions + BLOCK_SIZE - 1) // BLOCK_SIZE
    nb = int(num_blocks if num_blocks is not None else need.sum() + spare_blocks)
    tables = build_tables(rng, need, nb)
    # this step's tokens: positions L-q_len .. L-1 of every row
    slots = [slot_of(tables, b, int(lengths_arr[b]) - q_len + i)
             if int(lengths_arr[b]) - q_len + i >= 0 else -1
             for b in range(batch) for i in range(q_len)]
    return Layout(lengths_arr.astype(np.int32), tables, nb, np.asarray(slots, dtype=np.int64), need)


def make_case(name: str, seed: int, *, batch: int, q_len: int, num_q_heads: int,
              num_kv_heads: int, head_dim: int, fmt: str, lengths,
              num_blocks: Optional[int] = None, spare_blocks: int = 0,
              extra_positions: int = 0, accept: bool = False) -> PagedCase:
    """General builder.  ``lengths`` is an int array, or a callable
    ``rng -> int array``."""
    rng = rng_for(seed)
    lay = make_layout(rng, batch=batch, q_len=q_len, lengths=lengths, num_blocks=num_blocks,
                      spare_blocks=spare_blocks, extra_positions=extra_positions)
    kc, vc = fill_pool(rng, lay.block_tables, lay.blocks_needed, lay.num_blocks, num_kv_heads,
                       head_dim, fmt)
    query = normal_bits(rng, (batch, q_len, num_q_heads, head_dim), fmt)
    t = len(lay.slot_mapping)
    new_key = normal_bits(rng, (t, num_kv_heads, head_dim), fmt)
    new_value = normal_bits(rng, (t, num_kv_heads, head_dim), fmt)
    accepted = rng.integers(0, q_len + 1, size=batch).astype(np.int32) if accept else None
    return PagedCase(
        name=name, batch=batch, q_len=q_len, num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, fmt=fmt, num_blocks=lay.num_blocks,
        context_lens=lay.context_lens, block_tables=lay.block_tables,
        key_cache=kc, value_cache=vc, query=query, new_key=new_key, new_value=new_value,
        slot_mapping=lay.slot_mapping,
        scale=float(np.float32(1.0 / np.sqrt(head_dim))), accepted=accepted)


# ---------------------------------------------------------------------------
# The five workloads.  Defaults are the full sizes; the size arguments give
# small variants of the same structure for fast parity runs.
# ---------------------------------------------------------------------------

def tiny(seed: int = 1) -> PagedCase:
    """1 sequence, 8/2 heads, D 64, fp16, 256 tokens = 16 blocks picked by a
    seeded permutation of a 64-block pool, plus one new-token write."""
    return make_case("tiny", seed, batch=1, q_len=1, num_q_heads=8, num_kv_heads=2,
                     head_dim=64, fmt="f16", lengths=[256], num_blocks=64)


def llama8b_batch(seed: int = 2, batch: int = 32, lo: int = 512, hi: int = 4096,
                  num_blocks: int = 16384) -> PagedCase:
    """Llama-3-8B-shaped layer: 32/8 heads, D 128, bf16, lengths uniform in
    [lo, hi], disjoint random picks from a shared 16384-block pool."""
    return make_case("llama8b_batch", seed, batch=batch, q_len=1, num_q_heads=32,
                     num_kv_heads=8, head_dim=128, fmt="bf16",
                     lengths=lambda r: r.integers(lo, hi + 1, size=batch),
                     num_blocks=num_blocks)


def long32k(seed: int = 3, length: int = 32768) -> PagedCase:
    """Single-user 32K decode layer: 32/8 heads, D 128, fp16, 2048 blocks in a
    randomly permuted pool of exactly 2048 blocks."""
    nb = (length + BLOCK_SIZE - 1) // BLOCK_SIZE
    return make_case("long32k", seed, batch=1, q_len=1, num_q_heads=32, num_kv_heads=8,
                     head_dim=128, fmt="f16", lengths=[length], num_blocks=nb)


def spec_verify(seed: int = 4, batch: int = 64, lo: int = 256, hi: int = 16384,
                q_len: int = 4, spare_blocks: int = 64) -> PagedCase:
    """Ragged speculative verify: q_len 4 drafts per row, 32/8 heads, D 128,
    bf16, lengths log-uniform in [lo, hi] (drafts included), accept counts
    uniform in {0..q_len}; tables leave room for the next step's write."""
    def lengths(r):
        return np.round(np.exp(r.uniform(np.log(lo), np.log(hi), size=batch))).astype(np.int64)
    return make_case("spec_verify", seed, batch=batch, q_len=q_len, num_q_heads=32,
                     num_kv_heads=8, head_dim=128, fmt="bf16", lengths=lengths,
                     spare_blocks=spare_blocks, extra_positions=1, accept=True)


def k8v4(seed: int = 5, batch: int = 16, length: int = 8192) -> PagedCase:
    """K8/V4 decode: 32/8 heads, D 128, fp16 K/V draws (quantized by the write
    path), context 8192, pool of exactly the needed blocks, permuted."""
    nb = batch * ((length + BLOCK_SIZE - 1) // BLOCK_SIZE)
    return make_case("k8v4", seed, batch=batch, q_len=1, num_q_heads=32, num_kv_heads=8,
                     head_dim=128, fmt="f16", lengths=[length] * batch, num_blocks=nb)


def shared_prefix_layout(rng, groups: int, group_size: int, prefix_len: int, suffix_lo: int,
                         suffix_hi: int):
    """Lengths and tables of a shared-prefix batch (draws: suffix lengths, then
    the pool permutation).  Returns (lens int64 [B], tables int32 [B, mb],
    num_blocks, used block ids, group_members [groups, group_size],
    prefix_blocks [groups])."""
    if prefix_len % BLOCK_SIZE:
        raise ValueError("the shared prefix is whole blocks")
    batch = groups * group_size
    suffix = rng.integers(suffix_lo, suffix_hi + 1, size=batch).astype(np.int64)
    lens = prefix_len + suffix
    pre_blocks = prefix_len // BLOCK_SIZE
    own = (suffix + BLOCK_SIZE - 1) // BLOCK_SIZE
    nb = groups * pre_blocks + int(own.sum()) + 8
    perm = rng.permutation(nb).astype(np.int32)
    mb = int(pre_blocks + own.max())
    tables = np.full((batch, mb), -1, dtype=np.int32)
    pos = 0
    group_blocks = []
    for _ in range(groups):
        group_blocks.append(perm[pos:pos + pre_blocks])
        pos += pre_blocks
    for b in range(batch):
        tables[b, :pre_blocks] = group_blocks[b // group_size]
        tables[b, pre_blocks:pre_blocks + own[b]] = perm[pos:pos + own[b]]
        pos += int(own[b])
    used = np.concatenate(group_blocks + [tables[b, pre_blocks:pre_blocks + own[b]]
                                          for b in range(batch)])
    members = np.arange(batch, dtype=np.int32).reshape(groups, group_size)
    return lens, tables, nb, used, members, np.full(groups, pre_blocks, dtype=np.int32)


def shared_prefix(seed: int = 6, groups: int = 8, group_size: int = 4, prefix_len: int = 4096,
                  suffix_lo: int = 64, suffix_hi: int = 1024, num_q_heads: int = 32,
                  num_kv_heads: int = 8, head_dim: int = 128, fmt: str = "bf16",
                  q_len: int = 1) -> PagedCase:
    """Batches whose sequences share a whole-block prefix in groups (a common
    system prompt): ``groups`` groups of ``group_size`` sequences; the members
    of a group point their first ``prefix_len / 16`` table entries at the same
    physical blocks, then each has its own suffix of uniform length in
    [suffix_lo, suffix_hi] (this step's tokens included).  Draw order:
    suffix lengths, pool permutation, K, V, query, new K, new V.
    ``extra`` holds ``group_members`` int32 [groups, group_size] and
    ``prefix_blocks`` int32 [groups]."""
    rng = rng_for(seed)
    lens, tables, nb, used, members, pre = shared_prefix_layout(rng, groups, group_size,
                                                                prefix_len, suffix_lo, suffix_hi)
    batch = groups * group_size
    shape = (nb, BLOCK_SIZE, num_kv_heads, head_dim)
    kc = np.zeros(shape, dtype=np.uint16)
    vc = np.zeros(shape, dtype=np.uint16)
    for pool in (kc, vc):
        for st in range(0, len(used), 2048):
            ids = used[st:st + 2048]
            pool[ids] = normal_bits(rng, (len(ids),) + shape[1:], fmt)
    query = normal_bits(rng, (batch, q_len, num_q_heads, head_dim), fmt)
    slots = np.asarray([slot_of(tables, b, int(lens[b]) - q_len + i)
                        for b in range(batch) for i in range(q_len)], dtype=np.int64)
    new_key = normal_bits(rng, (batch * q_len, num_kv_heads, head_dim), fmt)
    new_value = normal_bits(rng, (batch * q_len, num_kv_heads, head_dim), fmt)
    return PagedCase(
        name="shared_prefix", batch=batch, q_len=q_len, num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, fmt=fmt, num_blocks=nb,
        context_lens=lens.astype(np.int32), block_tables=tables, key_cache=kc, value_cache=vc,
        query=query, new_key=new_key, new_value=new_value, slot_mapping=slots,
        scale=float(np.float32(1.0 / np.sqrt(head_dim))),
        extra={"group_members": members, "prefix_blocks": pre})


def layout_of(name: str, seed: int) -> tuple:
    """(Layout, batch, q_len, Hq, Hkv, D, fmt) of a named workload, drawing only
    the lengths and tables (same draws as the full builder up to that point)."""
    rng = rng_for(seed)
    if name == "tiny":
        return make_layout(rng, batch=1, q_len=1, lengths=[256], num_blocks=64), 1, 1, 8, 2, 64, "f16"
    if name == "llama8b_batch":
        return (make_layout(rng, batch=32, q_len=1, lengths=lambda r: r.integers(512, 4097, size=32),
                            num_blocks=16384), 32, 1, 32, 8, 128, "bf16")
    if name == "long32k":
        return make_layout(rng, batch=1, q_len=1, lengths=[32768], num_blocks=2048), 1, 1, 32, 8, 128, "f16"
    if name == "spec_verify":
        def lengths(r):
            return np.round(np.exp(r.uniform(np.log(256), np.log(16384), size=64))).astype(np.int64)
        return (make_layout(rng, batch=64, q_len=4, lengths=lengths, spare_blocks=64,
                            extra_positions=1), 64, 4, 32, 8, 128, "bf16")
    if name == "k8v4":
        return (make_layout(rng, batch=16, q_len=1, lengths=[8192] * 16, num_blocks=8192),
                16, 1, 32, 8, 128, "f16")
    raise KeyError(name)


WORKLOADS = {
    "tiny": tiny,
    "llama8b_batch": llama8b_batch,
    "long32k": long32k,
    "spec_verify": spec_verify,
    "k8v4": k8v4,
    "shared_prefix": shared_prefix,
}


def next_step_slots(case: PagedCase, new_lens: np.ndarray) -> np.ndarray:
    """After a verify commit, the slot of each row's next token (position
    ``new_lens[b]``), using the room the tables were built with."""
    return np.asarray([slot_of(case.block_tables, b, int(new_lens[b]))
                       for b in range(case.batch)], dtype=np.int64)


def poison_unused(case: PagedCase, nan_bits: int = 0x7FC1) -> None:
    """Fill every cache row at or past each sequence's length, and every block
    no table references, with a NaN pattern (0x7FC1 is a NaN in fp16 and in
    bf16); point unused table entries at an
    out-of-range block id.  Used to show such data is never read."""
    nb = case.num_blocks
    referenced = np.zeros(nb, dtype=bool)
    for b in range(case.batch):
        L = int(case.context_lens[b])
        nblk = (L + BLOCK_SIZE - 1) // BLOCK_SIZE
        ids = case.block_tables[b, :nblk]
        referenced[ids] = True
        if L % BLOCK_SIZE:
            last = ids[-1]
            case.key_cache[last, L % BLOCK_SIZE:] = nan_bits
            case.value_cache[last, L % BLOCK_SIZE:] = nan_bits
        case.block_tables[b, nblk:] = nb + 7
    case.key_cache[~referenced] = nan_bits
    case.value_cache[~referenced] = nan_bits
