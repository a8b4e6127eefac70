"""Plain CPU oracle for paged-KV decode: test infrastructure only.

This module is the checker, not the product.  Only the test suite, the smoke
check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import
it.  It shares no code with the HIP library: it never loads it, never touches a
GPU, and re-derives every step from the definitions on the pages.

Numerics: attention is evaluated in float64 on values decoded from the stored
fp16/bf16 bit patterns.  The K8/V4 quantizer works in float32, the precision in
which the GPU write kernel takes the same integer decisions (see
``quantize_k8`` / ``quantize_v4``).

Sources (page title, then the part of it used):

* "How the Paged KV Cache Works in MTPLX", Physical Layout and Memory
  Organization: caches are 4-D ``[num_blocks, block_size, num_kv_heads,
  head_dim]`` with 16 tokens per block.
* "The KV Cache" (metalworking), layout paragraph: paged layouts are
  fixed-size blocks plus an indirection table (our int32 block table).
* "The KV Cache", arithmetic paragraph: one K and one V vector per KV head per
  token per layer; query head ``h`` reads KV head ``h // gqa_factor``.
* "How MTPLX Manages Memory Using Request-Sized Paged KV Cache", Request-Sized
  Offset Tracking: the write advances the offset, then attention reads the
  cache up to that offset (so ``context_lens`` counts this step's tokens).
* mlxcel "KV Cache", Matrix-Absorbed MLA Decode and Speculative Rewind: a
  multi-token verify block attends behind the cache; rejected tokens are
  removed by rewinding the logical length.
* "How MTPLX Manages Memory with KV Caching Strategies", VllmMetalPagedKVCache
  and Quantization-Aware Allocation: quantized caches keep scale/zero side
  tensors and are written through a symmetric quantizer.
* "The KV Cache", the K/V asymmetry paragraph: int8 K, 4-bit V.

Readings where the pages are silent are listed next to each function.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
against something other than itself (brute force through independent code
paths, closed forms, invariants, hand-built quantizer vectors, K8/V4 side
arrays checked slot by slot against the input rows, the length clamp against
attention at the table's capacity), and a planted mistake in each of these
parts fails a pin.
"""

from __future__ import annotations

import numpy as np

BLOCK_SIZE = 16
FMT_F16 = "f16"
FMT_BF16 = "bf16"
FMT_K8V4 = "k8v4"

K8_QMAX = 127          # symmetric int8 range used for K: codes in [-127, 127]
V4_QMAX = 15           # unsigned 4-bit codes for V: [0, 15]
V4_GROUP = 32          # V elements sharing one (scale, zero) pair


# ---------------------------------------------------------------------------
# Storage decoding (the oracle's own; raw caches are uint16 bit patterns)
# ---------------------------------------------------------------------------

def decode(bits: np.ndarray, fmt: str) -> np.ndarray:
    """Stored 16-bit patterns -> float64 values (exact for both formats)."""
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError("storage must be uint16 bit patterns")
    if fmt == FMT_F16:
        return bits.view(np.float16).astype(np.float64)
    if fmt == FMT_BF16:
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown 16-bit format {fmt!r}")


# ---------------------------------------------------------------------------
# Step 1: the slot scatter (reshape_and_cache)
# ---------------------------------------------------------------------------

def kv_cache_write(key, value, key_cache, value_cache, slot_mapping, block_size=BLOCK_SIZE):
    """Return copies of the caches with token ``t`` written at ``slot_mapping[t]``.

    "How the Paged KV Cache Works in MTPLX", Physical Layout: the cache is
    ``[num_blocks, block_size, num_kv_heads, head_dim]``; slot ``s`` is block
    ``s // block_size``, row ``s % block_size``.  "The KV Cache" names the
    scatter kernel (reshape_and_cache) that performs this write.

    Reading (pages silent): a negative slot, or one past the pool, means "no
    write" for that token; duplicate slots are not allowed.
    """
    key = np.asarray(key)
    value = np.asarray(value)
    kc = np.array(key_cache, copy=True)
    vc = np.array(value_cache, copy=True)
    num_blocks = kc.shape[0]
    seen = set()
    for t, s in enumerate(np.asarray(slot_mapping).tolist()):
        if s < 0 or s >= num_blocks * block_size:
            continue
        if s in seen:
            raise ValueError(f"slot {s} written twice")
        seen.add(s)
        blk, off = divmod(s, block_size)
        kc[blk, off] = key[t]
        vc[blk, off] = value[t]
    return kc, vc


# ---------------------------------------------------------------------------
# Step 2: block-table resolution
# ---------------------------------------------------------------------------

def effective_length(context_len: int, max_blocks: int, block_size=BLOCK_SIZE) -> int:
    """Reading: a length is clamped to [0, max_blocks * block_size]."""
    return int(min(max(int(context_len), 0), max_blocks * block_size))


def resolve_positions(block_table_row, length, num_blocks, block_size=BLOCK_SIZE):
    """Logical positions 0..length-1 -> (valid, physical block, row in block).

    "The KV Cache", layout paragraph: fixed-size blocks plus an indirection
    table.  Position ``j`` lives in table entry ``j // block_size`` at row
    ``j % block_size``.  Reading (pages silent): an entry outside
    ``[0, num_blocks)`` marks its 16 positions as absent; they take no part in
    the softmax.
    """
    j = np.arange(length)
    blk = np.asarray(block_table_row, dtype=np.int64)[j // block_size]
    off = j % block_size
    valid = (blk >= 0) & (blk < num_blocks)
    return valid, np.where(valid, blk, 0), off


# ---------------------------------------------------------------------------
# Step 3: attention (plain masked softmax, fp64)
# ---------------------------------------------------------------------------

def visible_count(length: int, q_len: int, i: int) -> int:
    """Number of positions query row ``i`` of a ``q_len`` block may see.

    Reading: the cache length already includes the ``q_len`` new tokens
    (write first, then attend), and row ``i`` sits at position
    ``length - q_len + i`` with causal masking inside the block, so it sees
    positions ``0 .. length - q_len + i``.  For ``q_len == 1`` this is the
    whole cache.
    """
    return length - q_len + i + 1


def window_start(length: int, q_len: int, i: int, window: int) -> int:
    """First position query row ``i`` may see under a sliding window.

    "How MTPLX Manages Memory Using Request-Sized Paged KV Cache",
    Sliding-Window Memory Control: attention is trimmed to the most recent
    ``window`` cached tokens, older ones are masked (their blocks stay
    allocated); mlxcel "KV Cache", RotatingKVCache.  Reading for a block of
    ``q_len`` rows: row ``i`` at position ``p = length - q_len + i`` sees its
    own ``window`` most recent positions ``p - window + 1 .. p`` (so each
    verify row still equals a single-token decode).  ``window <= 0`` means no
    window.
    """
    if window <= 0:
        return 0
    return max(visible_count(length, q_len, i) - window, 0)


def attend_rows(q, keys, vals, valid, scale, q_len, window=0):
    """Masked softmax attention for one (sequence, KV head).

    q: float64 ``[q_len, G, D]`` (the G query heads sharing this KV head);
    keys/vals: float64 ``[n_pos, D]``; valid: bool ``[n_pos]``.
    Returns float64 ``[q_len, G, D]``.  Rows that see no valid position
    return zeros (reading: pages silent).  Row ``i`` sees positions
    ``window_start .. visible_count - 1``.
    """
    ql, g, d = q.shape
    out = np.zeros((ql, g, d), dtype=np.float64)
    n_pos = keys.shape[0]
    for i in range(ql):
        n = min(visible_count(n_pos, q_len, i), n_pos)
        lo = window_start(n_pos, q_len, i, window)
        if n <= lo:
            continue
        mask = valid[lo:n]
        if not mask.any():
            continue
        kv = keys[lo:n][mask]
        vv = vals[lo:n][mask]
        s = float(scale) * (q[i] @ kv.T)              # [G, n_visible]
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        out[i] = (p @ vv) / p.sum(axis=1, keepdims=True)
    return out


def paged_attention(query, key_cache, value_cache, block_tables, context_lens,
                    scale, gqa_factor, fmt, q_fmt=None, block_size=BLOCK_SIZE, window=0):
    """Paged-attention decode, evaluated as the plain definition.

    query: uint16 bits ``[B, Q, Hq, D]``; caches: uint16 bits
    ``[NB, block_size, Hkv, D]``; block_tables int32 ``[B, max_blocks]``;
    context_lens int32 ``[B]``.  Returns float64 ``[B, Q, Hq, D]``.

    Query head ``h`` reads KV head ``h // gqa_factor`` ("The KV Cache",
    arithmetic paragraph: the stride trick ``kv_head_idx = tid.y /
    gqa_factor``).  The softmax scale is the float32 value the kernel receives,
    widened to float64.  ``window`` > 0 restricts each row to its most recent
    positions (``window_start``).
    """
    q_fmt = q_fmt or fmt
    qv = decode(query, q_fmt)

    def rows(blk, off):
        return decode(key_cache[blk, off], fmt), decode(value_cache[blk, off], fmt)

    return _attend(qv, rows, key_cache.shape[0], key_cache.shape[2], block_tables,
                   context_lens, scale, gqa_factor, block_size, window)


def _attend(qv, read_rows, num_blocks, hkv, block_tables, context_lens, scale,
            gqa_factor, block_size, window=0):
    """Shared driver: resolve each sequence, decode only its rows, attend."""
    b_count, q_len, hq, d = qv.shape
    if hq != hkv * gqa_factor:
        raise ValueError("num_q_heads must equal num_kv_heads * gqa_factor")
    scale64 = float(np.float32(scale))
    bt = np.asarray(block_tables)
    out = np.zeros((b_count, q_len, hq, d), dtype=np.float64)
    for b in range(b_count):
        length = effective_length(int(context_lens[b]), bt.shape[1], block_size)
        valid, blk, off = resolve_positions(bt[b], length, num_blocks, block_size)
        keys, vals = read_rows(blk, off)               # float64 [length, Hkv, D]
        for g in range(hkv):
            heads = slice(g * gqa_factor, (g + 1) * gqa_factor)
            out[b, :, heads, :] = attend_rows(qv[b, :, heads, :], keys[:, g, :], vals[:, g, :],
                                              valid, scale64, q_len, window)
    return out


# ---------------------------------------------------------------------------
# Sparse-V (approximate): the error bound its skip rule guarantees
# ---------------------------------------------------------------------------

def sparse_v_error_bound(query, key_cache, value_cache, block_tables, context_lens, scale,
                         gqa_factor, fmt, threshold, block_size=BLOCK_SIZE):
    """Elementwise bound on |sparse-V output - exact output|.

    "The KV Cache" (metalworking), arithmetic paragraph: a sparse-V decode
    path at 32K deletes KV-cache traffic; the rule for what it skips is not
    stated.  Reading: the V row of position j is read only when some query
    row of its KV head has weight ``w_ij >= threshold * w_i,max`` with
    respect to that row's running maximum; skipped positions still count in
    the softmax denominator.  Since a running maximum never exceeds the final
    one, every skipped position has ``w_ij / max_j w_ij < threshold`` in the
    exact weights, so for each output element

        |o_sparse - o_exact| <= sum_{j : w_ij < threshold * max w_i} w_ij |v_jd| / sum_j w_ij.

    Returns float64 ``[B, Q, Hq, D]`` of that right-hand side (0 when
    ``threshold`` is 0).
    """
    qv = decode(query, fmt)
    b_count, q_len, hq, d = qv.shape
    hkv = key_cache.shape[2]
    bt = np.asarray(block_tables)
    out = np.zeros((b_count, q_len, hq, d), dtype=np.float64)
    scale64 = float(np.float32(scale))
    for b in range(b_count):
        length = effective_length(int(context_lens[b]), bt.shape[1], block_size)
        valid, blk, off = resolve_positions(bt[b], length, key_cache.shape[0], block_size)
        keys = decode(key_cache[blk, off], fmt)
        vals = decode(value_cache[blk, off], fmt)
        for h in range(hq):
            g = h // gqa_factor
            for i in range(q_len):
                n = min(visible_count(length, q_len, i), length)
                if n <= 0:
                    continue
                mask = valid[:n]
                if not mask.any():
                    continue
                s = scale64 * (keys[:n][mask][:, g, :] @ qv[b, i, h])
                w = np.exp(s - s.max())
                small = w < threshold
                out[b, i, h] = (w[small][:, None] * np.abs(vals[:n][mask][small][:, g, :])).sum(0) \
                    / w.sum()
    return out


# ---------------------------------------------------------------------------
# gather_kv_cache: paged -> contiguous (the inverse of the slot scatter)
# ---------------------------------------------------------------------------

def gather_kv_cache(key_cache, value_cache, block_tables, cu_seq_lens, total_tokens,
                    block_size=BLOCK_SIZE):
    """Copy every sequence's cached rows out of the pages into packed arrays.

    "The KV Cache" (metalworking), layout paragraph, names a gather_kv_cache
    kernel beside reshape_and_cache; reading (its arguments are not given):
    it is the inverse of the slot scatter, laying each sequence's positions
    ``0 .. L_b - 1`` out contiguously for dense consumers.  Sequence ``b``
    fills output rows ``cu_seq_lens[b] .. cu_seq_lens[b+1] - 1`` (so
    ``L_b = cu_seq_lens[b+1] - cu_seq_lens[b]``); position ``j`` comes from
    block ``block_tables[b][j // block_size]``, row ``j % block_size``.
    Readings: a length is clamped to ``[0, max_blocks * block_size]`` like
    every length; a position whose table entry names no pool block gives a
    zero row; output rows outside ``[0, total_tokens)`` are not written; rows
    no sequence covers stay zero.  Returns ``(keys, values)``, each
    ``[total_tokens, Hkv, D]`` of the caches' element type.
    """
    bt = np.asarray(block_tables)
    cu = np.asarray(cu_seq_lens, dtype=np.int64)
    nb = key_cache.shape[0]
    out_k = np.zeros((total_tokens,) + key_cache.shape[2:], dtype=key_cache.dtype)
    out_v = np.zeros((total_tokens,) + value_cache.shape[2:], dtype=value_cache.dtype)
    for b in range(len(cu) - 1):
        length = effective_length(int(cu[b + 1] - cu[b]), bt.shape[1], block_size)
        for j in range(length):
            row = int(cu[b]) + j
            if not 0 <= row < total_tokens:
                continue
            blk = int(bt[b, j // block_size])
            if 0 <= blk < nb:
                out_k[row] = key_cache[blk, j % block_size]
                out_v[row] = value_cache[blk, j % block_size]
    return out_k, out_v


# ---------------------------------------------------------------------------
# The decode step as one call: write the new rows where the tables put them,
# then attend
# ---------------------------------------------------------------------------

def append_slots(block_tables, context_lens, q_len, num_blocks, block_size=BLOCK_SIZE):
    """Cache slot of each new token, from the block tables.

    Token ``i`` of sequence ``b`` is the one at position ``L_b - q_len + i``
    (the length counts this step's tokens: "How MTPLX Manages Memory Using
    Request-Sized Paged KV Cache", Request-Sized Offset Tracking), which lives
    in table entry ``pos // block_size`` at row ``pos % block_size`` ("The KV
    Cache", layout paragraph).  Returns int64 ``[B * q_len]`` in ``[b][i]``
    order, -1 where the position is negative or its table entry names no pool
    block (reading: such a token is neither stored nor attended).  ``L_b`` is
    first clamped like every length (``effective_length``).
    """
    bt = np.asarray(block_tables)
    out = np.full(len(context_lens) * q_len, -1, dtype=np.int64)
    for b in range(len(context_lens)):
        length = effective_length(int(context_lens[b]), bt.shape[1], block_size)
        for i in range(q_len):
            pos = length - q_len + i
            if pos < 0:
                continue
            blk = int(bt[b, pos // block_size])
            if 0 <= blk < num_blocks:
                out[b * q_len + i] = blk * block_size + pos % block_size
    return out


def decode_append(query, new_key, new_value, key_cache, value_cache, block_tables,
                  context_lens, scale, gqa_factor, fmt, block_size=BLOCK_SIZE):
    """One decode step: store the new rows at their table slots, then attend
    over the updated caches (mlxcel "KV Cache", Attention Dispatch and In-Place
    Decode Writes: the new row goes into the cache in place during decode).

    Returns ``(out float64 [B, Q, Hq, D], key_cache', value_cache')``.
    """
    q_len = np.asarray(query).shape[1]
    slots = append_slots(block_tables, context_lens, q_len, key_cache.shape[0], block_size)
    kc, vc = kv_cache_write(new_key, new_value, key_cache, value_cache, slots, block_size)
    out = paged_attention(query, kc, vc, block_tables, context_lens, scale, gqa_factor, fmt,
                          block_size=block_size)
    return out, kc, vc


# ---------------------------------------------------------------------------
# Split-KV partition + log-sum-exp merge (used by the tests to show that the
# partitioned form reaches the plain result)
# ---------------------------------------------------------------------------

def attend_rows_partitioned(q, keys, vals, valid, scale, q_len, partition_size):
    """Same result as ``attend_rows`` via partitions of ``partition_size``
    logical positions merged by their log-sum-exp.

    "The KV Cache" names split-KV decode kernels for single-user decode; the
    merge is the usual one: with per-partition max ``m_p``, weight sum ``l_p``
    and normalised output ``o_p``, the result is
    ``sum_p e^(m_p - M) l_p o_p / sum_p e^(m_p - M) l_p`` with ``M = max m_p``.
    """
    ql, g, d = q.shape
    n_pos = keys.shape[0]
    out = np.zeros((ql, g, d), dtype=np.float64)
    for i in range(ql):
        n = min(visible_count(n_pos, q_len, i), n_pos)
        parts = []
        for start in range(0, max(n, 0), partition_size):
            stop = min(start + partition_size, n)
            mask = valid[start:stop]
            if not mask.any():
                continue
            s = scale * (q[i] @ keys[start:stop][mask].T)
            m_p = s.max(axis=1)
            p = np.exp(s - m_p[:, None])
            l_p = p.sum(axis=1)
            o_p = (p @ vals[start:stop][mask]) / l_p[:, None]
            parts.append((m_p, l_p, o_p))
        if not parts:
            continue
        big_m = np.max(np.stack([m for m, _, _ in parts]), axis=0)
        num = np.zeros((g, d))
        den = np.zeros(g)
        for m_p, l_p, o_p in parts:
            w = np.exp(m_p - big_m) * l_p
            num += w[:, None] * o_p
            den += w
        out[i] = num / den[:, None]
    return out


# ---------------------------------------------------------------------------
# K8/V4 quantization (float32 decisions) and dequantization (float64)
# ---------------------------------------------------------------------------

def _as_f32_values(bits, fmt):
    return decode(bits, fmt).astype(np.float32)   # exact: f16/bf16 fit in f32


def quantize_k8(k32: np.ndarray):
    """Symmetric int8 quantization of K, one fp16 scale per row (last axis).

    "How MTPLX Manages Memory with KV Caching Strategies" names a symmetric
    quantizer on the write path; "The KV Cache" fixes K at 8 bits.  Reading of
    the steps, all in float32: ``amax = max |k|``; ``s = fp16(amax / 127)``
    (correctly rounded divide, round-to-nearest-even to fp16); if ``s == 0``
    every code is 0, else ``c = clamp(rint(k / s), -127, 127)`` with ties to
    even.  Returns (int8 codes, float16 scales).
    """
    k32 = np.asarray(k32, dtype=np.float32)
    amax = np.max(np.abs(k32), axis=-1)
    s16 = (amax / np.float32(K8_QMAX)).astype(np.float32).astype(np.float16)
    s32 = s16.astype(np.float32)
    safe = np.where(s32 == 0, np.float32(1), s32)
    with np.errstate(invalid="ignore", over="ignore"):
        c = np.rint(k32 / safe[..., None])
    c = np.clip(c, -K8_QMAX, K8_QMAX)
    c = np.where((s32 == 0)[..., None], 0, c)
    return c.astype(np.int8), s16


def quantize_v4(v32: np.ndarray):
    """Asymmetric 4-bit quantization of V per group of 32 along the last axis.

    "The KV Cache" (K/V asymmetry) fixes V at low precision; "How MTPLX
    Manages Memory with KV Caching Strategies" keeps scale and zero tensors
    next to the cache.  Reading of the steps, all in float32 per group:
    ``mn, mx`` = group min/max; ``s = fp16((mx - mn) / 15)``; ``z = fp16(mn)``;
    if ``s == 0`` codes are 0, else ``c = clamp(rint((v - z) / s), 0, 15)``.
    Returns (uint8 codes unpacked ``[..., D]``, fp16 scales, fp16 zeros),
    scales/zeros shaped ``[..., D // 32]``.
    """
    v32 = np.asarray(v32, dtype=np.float32)
    d = v32.shape[-1]
    if d % V4_GROUP:
        raise ValueError("head_dim must be a multiple of 32")
    grp = v32.reshape(v32.shape[:-1] + (d // V4_GROUP, V4_GROUP))
    mn = grp.min(axis=-1)
    mx = grp.max(axis=-1)
    s16 = ((mx - mn) / np.float32(V4_QMAX)).astype(np.float32).astype(np.float16)
    z16 = mn.astype(np.float16)
    s32 = s16.astype(np.float32)
    z32 = z16.astype(np.float32)
    safe = np.where(s32 == 0, np.float32(1), s32)
    with np.errstate(invalid="ignore", over="ignore"):
        c = np.rint((grp - z32[..., None]) / safe[..., None])
    c = np.clip(c, 0, V4_QMAX)
    c = np.where((s32 == 0)[..., None], 0, c)
    return c.reshape(v32.shape).astype(np.uint8), s16, z16


def pack_v4(codes: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte: element ``2i`` in bits 0-3, ``2i+1`` in bits 4-7."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << np.uint8(4))).astype(np.uint8)


def unpack_v4(packed: np.ndarray) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & np.uint8(0x0F)
    out[..., 1::2] = packed >> np.uint8(4)
    return out


def dequant_k8(codes, scales) -> np.ndarray:
    """``k = c * s`` in float64 (exact)."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(scales, dtype=np.float64)[..., None]


def dequant_v4(packed, scales, zeros) -> np.ndarray:
    """``v = c * s + z`` per group of 32, in float64 (exact)."""
    c = unpack_v4(packed).astype(np.float64)
    d = c.shape[-1]
    grp = c.reshape(c.shape[:-1] + (d // V4_GROUP, V4_GROUP))
    v = grp * np.asarray(scales, dtype=np.float64)[..., None] + \
        np.asarray(zeros, dtype=np.float64)[..., None]
    return v.reshape(c.shape)


def kv_cache_write_k8v4(key, value, in_fmt, k_cache, k_scale, v_cache, v_scale, v_zero,
                        slot_mapping, block_size=BLOCK_SIZE):
    """Quantize-on-write into the K8/V4 cache arrays; returns updated copies.

    Layout reading: side tensors are indexed exactly like the cache ("How
    MTPLX Manages Memory Using Request-Sized Paged KV Cache",
    Quantization-Aware Memory Layout: the same offsets and block indices
    apply): k_cache int8 ``[NB, BS, Hkv, D]``, k_scale fp16 ``[NB, BS, Hkv]``,
    v_cache uint8 ``[NB, BS, Hkv, D/2]``, v_scale / v_zero fp16
    ``[NB, BS, Hkv, D/32]``.
    """
    kq, ks = quantize_k8(_as_f32_values(key, in_fmt))
    vq, vs, vz = quantize_v4(_as_f32_values(value, in_fmt))
    vp = pack_v4(vq)
    arrs = [np.array(a, copy=True) for a in (k_cache, k_scale, v_cache, v_scale, v_zero)]
    num_blocks = arrs[0].shape[0]
    seen = set()
    for t, s in enumerate(np.asarray(slot_mapping).tolist()):
        if s < 0 or s >= num_blocks * block_size:
            continue
        if s in seen:
            raise ValueError(f"slot {s} written twice")
        seen.add(s)
        blk, off = divmod(s, block_size)
        arrs[0][blk, off] = kq[t]
        arrs[1][blk, off] = ks[t]
        arrs[2][blk, off] = vp[t]
        arrs[3][blk, off] = vs[t]
        arrs[4][blk, off] = vz[t]
    return tuple(arrs)


def paged_attention_k8v4(query, q_fmt, k_cache, k_scale, v_cache, v_scale, v_zero,
                         block_tables, context_lens, scale, gqa_factor, block_size=BLOCK_SIZE):
    """Paged decode over K8/V4 storage: dequantize the stored codes exactly in
    float64, then the same plain attention as ``paged_attention``."""
    qv = decode(query, q_fmt)

    def rows(blk, off):
        return (dequant_k8(k_cache[blk, off], k_scale[blk, off]),
                dequant_v4(v_cache[blk, off], v_scale[blk, off], v_zero[blk, off]))

    return _attend(qv, rows, k_cache.shape[0], k_cache.shape[2], block_tables,
                   context_lens, scale, gqa_factor, block_size)


# ---------------------------------------------------------------------------
# Cache size closed form and the speculative-verify commit
# ---------------------------------------------------------------------------

def kv_cache_bytes_per_token(num_layers, num_kv_heads, head_dim, fmt) -> int:
    """Bytes of cache one token occupies over all layers.

    "The KV Cache", arithmetic paragraph: per token and layer, one K and one V
    vector per KV head (fp16: ~128 KB per token for 32 layers and 1024-wide
    KV).  For K8/V4 the same count holds with 1-byte K plus one fp16 scale per
    KV head, and 4-bit V plus an fp16 scale and zero per 32 elements.
    """
    if fmt in (FMT_F16, FMT_BF16):
        return 2 * num_layers * num_kv_heads * head_dim * 2
    if fmt == FMT_K8V4:
        per_head = head_dim + 2 + head_dim // 2 + 2 * 2 * (head_dim // V4_GROUP)
        return num_layers * num_kv_heads * per_head
    raise ValueError(fmt)


def spec_commit(context_lens, q_len, accepted):
    """Lengths after a verify step accepts ``accepted[b]`` of ``q_len`` drafts.

    mlxcel "KV Cache", Speculative Rewind: rejected tokens are removed by
    rewinding the logical offset; the bytes stay and are overwritten later.
    """
    L = np.asarray(context_lens, dtype=np.int64)
    a = np.asarray(accepted, dtype=np.int64)
    if np.any(a < 0) or np.any(a > q_len):
        raise ValueError("accepted counts must lie in [0, q_len]")
    return (L - q_len + a).astype(np.int32)
