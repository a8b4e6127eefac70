"""Seeded random shapes through the split-KV calls, each against the oracle.

Every case draws its own batch size (up to 89 sequences, so past one 64-lane
chunk of lengths), q_len (1..4), GQA factor (G * q_len <= 16), KV head count
(1, 2, 3, 4 or 8: the balanced split's all-heads, head-pair and one-head
workgroups), head_dim, 16-bit format and lengths (zeros and lengths shorter
than q_len included).  Each case runs the balanced split (partition_size 0),
its append form (caches bit-exact after the call) and a fixed partition size
drawn from 16..1024, so the launcher's grid-dependent choices (head pairs,
quads, eights, the merge's two forms, the balanced run count) meet shapes no
hand-written case picked.  The cascade cases draw groups, group sizes, shared
prefixes and suffixes, and clear member slots at random (sequences outside
every group, and groups whose first slot is empty, which are ignored).  The
K8/V4 cases run the quantize-on-write append form, direct and split (the code
arrays bit-exact after the call), and the window cases the windowed decode,
direct and split, and the windowed append form, with windows from 1 to twice
the longest sequence.  fp32 output within 2e-4 of the fp64 oracle throughout.
"""

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_181_amd import workloads as W

from gpu_util import DevCase, dev_to_bits, max_err, oracle_decode, run_decode
from test_gpu_parity import (k8v4_append_expected, run_append, run_cascade, run_k8v4_append,
                             run_window, run_window_append, small)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_181_amd as lib
    return lib


def _case(seed):
    r = np.random.default_rng(9000 + seed)
    q_len = int(r.choice([1, 1, 2, 3, 4]))
    hkv = int(r.choice([1, 2, 3, 4, 8]))
    gs = [g for g in (1, 2, 4, 8, 16) if g * q_len <= 16 and g * hkv <= 32]
    g = int(r.choice(gs))
    batch = int(r.integers(1, 90))
    hi = int(r.choice([40, 300, 1500]))
    lengths = r.integers(0, hi + 1, size=batch)
    lengths[r.random(batch) < 0.1] = 0                       # empty sequences among the others
    lengths[r.random(batch) < 0.1] = int(r.integers(0, q_len + 1))   # shorter than q_len
    head_dim = int(r.choice([64, 128]))
    fmt = str(r.choice(["f16", "bf16"]))
    psize = int(r.choice([16, 32, 64, 256, 512, 1024]))
    case = small(9000 + seed, batch=batch, q_len=q_len, num_q_heads=g * hkv, num_kv_heads=hkv,
                 head_dim=head_dim, fmt=fmt, lengths=[int(x) for x in lengths])
    return case, psize


@pytest.mark.parametrize("seed", range(48))
def test_random_shapes(P, seed):
    case, psize = _case(seed)
    print(f"[random] seed {seed}: B {case.batch} Q {case.q_len} Hq {case.num_q_heads} "
          f"Hkv {case.num_kv_heads} D {case.head_dim} {case.fmt} max L "
          f"{int(case.context_lens.max())} partition {psize}", flush=True)
    ref = oracle_decode(case)
    dc = DevCase(case)
    for part in (0, psize):
        out = run_decode(P, dc, split=True, partition_size=part)
        err = max_err(out, ref)
        assert err <= 2e-4, f"seed {seed} partition {part}: fp32-out max abs err {err}"
    aref, kc, vc = oracle.decode_append(case.query, case.new_key, case.new_value, case.key_cache,
                                        case.value_cache, case.block_tables, case.context_lens,
                                        case.scale, case.gqa_factor, case.fmt)
    out, k, v = run_append(P, dc, split=True, psize=0)
    assert np.array_equal(dev_to_bits(k), kc), f"seed {seed}: key cache differs"
    assert np.array_equal(dev_to_bits(v), vc), f"seed {seed}: value cache differs"
    err = max_err(out, aref)
    assert err <= 2e-4, f"seed {seed} balanced append: fp32-out max abs err {err}"


@pytest.mark.parametrize("seed", range(16))
def test_random_cascades(P, seed):
    r = np.random.default_rng(9500 + seed)
    q_len = int(r.choice([1, 1, 2]))
    hkv = int(r.choice([1, 2, 4]))
    g = int(r.choice([1, 2, 4]))
    group_size = int(r.integers(1, 16 // (g * q_len) + 1))
    groups = int(r.integers(1, 13))
    case = W.shared_prefix(seed=9500 + seed, groups=groups, group_size=group_size,
                           prefix_len=16 * int(r.integers(1, 21)),
                           suffix_lo=1, suffix_hi=int(r.choice([20, 200])),
                           num_q_heads=g * hkv, num_kv_heads=hkv,
                           head_dim=int(r.choice([64, 128])), fmt=str(r.choice(["f16", "bf16"])),
                           q_len=q_len)
    members = case.extra["group_members"].copy()
    members[r.random(members.shape) < 0.15] = -1             # empty slots, outsiders
    psize = int(r.choice([16, 64, 512]))
    print(f"[random cascade] seed {seed}: {groups} groups of {group_size}, G {g} Q {q_len} "
          f"Hkv {hkv}, partition {psize}", flush=True)
    ref = oracle_decode(case)
    out = run_cascade(P, DevCase(case), members, case.extra["prefix_blocks"], psize=psize)
    err = max_err(out, ref)
    assert err <= 2e-4, f"cascade seed {seed}: fp32-out max abs err {err}"


@pytest.mark.parametrize("seed", range(24))
def test_random_k8v4(P, seed):
    case, psize = _case(100 + seed)
    print(f"[random k8v4] seed {seed}: B {case.batch} Q {case.q_len} Hq {case.num_q_heads} "
          f"Hkv {case.num_kv_heads} D {case.head_dim} {case.fmt} max L "
          f"{int(case.context_lens.max())} partition {psize}", flush=True)
    before, after, ref = k8v4_append_expected(case)
    for split in (False, True):
        out, arrays = run_k8v4_append(P, case, before, split=split, psize=psize)
        for got, want in zip(arrays, after):
            assert np.array_equal(got, want), f"k8v4 seed {seed} split {split}: arrays differ"
        err = max_err(out, ref)
        assert err <= 2e-4, f"k8v4 seed {seed} split {split}: fp32-out max abs err {err}"


@pytest.mark.parametrize("seed", range(16))
def test_random_windows(P, seed):
    case, psize = _case(200 + seed)
    r = np.random.default_rng(9700 + seed)
    window = int(r.integers(1, 2 * max(int(case.context_lens.max()), 1) + 1))
    print(f"[random window] seed {seed}: B {case.batch} Q {case.q_len} Hq {case.num_q_heads} "
          f"Hkv {case.num_kv_heads} max L {int(case.context_lens.max())} window {window} "
          f"partition {psize}", flush=True)
    ref = oracle.paged_attention(case.query, case.key_cache, case.value_cache, case.block_tables,
                                 case.context_lens, case.scale, case.gqa_factor, case.fmt,
                                 window=window)
    dc = DevCase(case)
    for split in (False, True):
        out = run_window(P, dc, window, split=split, psize=psize)
        err = max_err(out, ref)
        assert err <= 2e-4, f"window seed {seed} split {split}: fp32-out max abs err {err}"
    slots = oracle.append_slots(case.block_tables, case.context_lens, case.q_len, case.num_blocks)
    kc, vc = oracle.kv_cache_write(case.new_key, case.new_value, case.key_cache, case.value_cache,
                                   slots)
    aref = oracle.paged_attention(case.query, kc, vc, case.block_tables, case.context_lens,
                                  case.scale, case.gqa_factor, case.fmt, window=window)
    out, k, v = run_window_append(P, dc, window, split=True, psize=psize)
    assert np.array_equal(dev_to_bits(k), kc), f"window seed {seed}: key cache differs"
    assert np.array_equal(dev_to_bits(v), vc), f"window seed {seed}: value cache differs"
    err = max_err(out, aref)
    assert err <= 2e-4, f"window seed {seed} append: fp32-out max abs err {err}"
