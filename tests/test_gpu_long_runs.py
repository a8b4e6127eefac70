"""GPU parity for wavefront runs longer than one block-table chunk, and for the
K8/V4 tiles with fewer than four query rows.

Each wavefront of the partition kernel walks a contiguous run of its
partition's blocks and reads the run's table entries 64 at a time (one per
lane), a chunk ahead.  The cases here give waves runs of more than 64 blocks in
every workgroup form: one KV head per workgroup (the 32K sequence in the
direct form and at 12288- and 16384-token partitions), head pairs and head
quads (batches sized so that the one-head grid needs two, or more than three and up to four,
workgroups per CU of a 256-CU device), in the decode, append, window and
windowed-append calls, each against the oracle.  The spec-verify commit runs
at the workload's full size, the K8/V4 column-group tiles run with
G * q_len of 1, 2 and 3 (copy columns past the real rows), and the merge of
the partials runs in both of its forms (whole rows, 32-dim slices).
"""

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_181_amd import workloads as W

from gpu_util import TOL, DevCase, bits_to_dev, dev_to_bits, max_err, run_decode
from test_gpu_parity import (k8v4_append_expected, oracle_k8v4_pool, run_append, run_k8v4_append,
                             run_window, run_window_append, assert_k8v4_arrays_equal, small)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_181_amd as lib
    return lib


def _uniform(lo, hi, n):
    return lambda r: r.integers(lo, hi + 1, size=n)      # noqa: E731


# name -> (builder, partition size or 0 for the direct form, window); the
# comments give the form the launcher picks and the blocks per wave
LONG = {
    # one head per workgroup, 8 waves x 256 blocks (four chunks)
    "long32k_direct": (lambda: W.long32k(), 0, 30000),
    # one head, 16 workgroups, 8 waves x 128 blocks
    "long32k_p16384": (lambda: W.long32k(), 16384, 20000),
    # one head, partitions of 768 blocks: 96 per wave, the last partition 64
    "long32k_p12288": (lambda: W.long32k(), 12288, 30000),
    # 3 partitions x 8 heads x 12 sequences = 288 one-head workgroups: head
    # pairs, 4 waves per head x 128 blocks
    "pairs_p8192": (lambda: small(140, batch=12, q_len=2, num_q_heads=16, num_kv_heads=8,
                                  head_dim=64, lengths=_uniform(16400, 24576, 12)), 8192, 17000),
    # direct form, 40 x 8 = 320 workgroups: head pairs, 66..94 blocks per wave
    "pairs_direct": (lambda: small(141, batch=40, q_len=1, num_q_heads=32, num_kv_heads=8,
                                   head_dim=64, fmt="bf16", lengths=_uniform(4200, 6000, 40)),
                     0, 4300),
    # 3 x 8 x 40 = 960 workgroups: head quads, 2 waves per head x 80 blocks
    "quads_p2560": (lambda: small(142, batch=40, q_len=1, num_q_heads=32, num_kv_heads=8,
                                  head_dim=64, fmt="bf16", lengths=_uniform(5200, 6000, 40)),
                    2560, 5150),
    # direct form, 100 x 8 = 800 workgroups: head quads, 65..81 blocks per wave
    "quads_direct": (lambda: small(143, batch=100, q_len=2, num_q_heads=16, num_kv_heads=8,
                                   head_dim=64, lengths=_uniform(2080, 2600, 100)), 0, 2090),
}


def _reference(case, kind, window):
    """The oracle's result for one call kind: "decode", "append" (store the
    new rows at their table slots, then attend), "window", "window_append"."""
    kc, vc = case.key_cache, case.value_cache
    if kind in ("append", "window_append"):
        slots = oracle.append_slots(case.block_tables, case.context_lens, case.q_len,
                                    case.num_blocks)
        kc, vc = oracle.kv_cache_write(case.new_key, case.new_value, kc, vc, slots)
    w = window if kind.startswith("window") else 0
    ref = oracle.paged_attention(case.query, kc, vc, case.block_tables, case.context_lens,
                                 case.scale, case.gqa_factor, case.fmt, window=w)
    return ref, kc, vc


@pytest.mark.parametrize("name", list(LONG))
def test_long_runs(P, name):
    """Decode, append, window and windowed append of one case, each against
    the oracle (fp32 output within 2e-4; caches after an append bit-exact)."""
    builder, psize, window = LONG[name]
    case = builder()
    dc = DevCase(case)
    split = psize > 0
    for kind in ("decode", "append", "window", "window_append"):
        print(f"[long runs] {name} {kind} partition {psize} window {window}", flush=True)
        ref, kc, vc = _reference(case, kind, window)
        if kind == "decode":
            out = run_decode(P, dc, split=split, partition_size=psize or 512)
        elif kind == "append":
            out, k, v = run_append(P, dc, split=split, psize=psize or 512)
        elif kind == "window":
            out = run_window(P, dc, window, split=split, psize=psize or 512)
        else:
            out, k, v = run_window_append(P, dc, window, split=split, psize=psize or 512)
        if kind.endswith("append"):
            assert np.array_equal(dev_to_bits(k), kc), f"{name} {kind}: key cache differs"
            assert np.array_equal(dev_to_bits(v), vc), f"{name} {kind}: value cache differs"
            del k, v
        err = max_err(out, ref)
        assert err <= 2e-4, f"{name} {kind}: fp32-out max abs err {err}"
        del ref, kc, vc


def test_spec_verify_commit_then_next_write_full_size(P):
    """The ragged verify batch at full size (64 rows, lengths up to 16384):
    write the 4 drafts, attend at the bench's partition size, commit the
    accepted prefixes by rewinding the lengths, write the next token of every
    row (it lands on the first rejected slot or past the drafts) and attend
    again over exactly the committed history."""
    case = W.spec_verify()
    dc = DevCase(case)
    P.kv_cache_write(dc.new_k, dc.new_v, dc.k, dc.v, dc.slots)
    out = run_decode(P, dc, split=True, partition_size=1024, out_dtype=torch.bfloat16)
    kc, vc = oracle.kv_cache_write(case.new_key, case.new_value, case.key_cache,
                                   case.value_cache, case.slot_mapping)
    assert np.array_equal(dev_to_bits(dc.k), kc) and np.array_equal(dev_to_bits(dc.v), vc)
    ref = oracle.paged_attention(case.query, kc, vc, case.block_tables, case.context_lens,
                                 case.scale, case.gqa_factor, "bf16")
    assert max_err(out, ref) <= TOL
    new_lens = oracle.spec_commit(case.context_lens, 4, case.accepted)
    nxt = W.next_step_slots(case, new_lens)
    rng = np.random.default_rng(78)
    nk = W.normal_bits(rng, (case.batch, 8, 128), "bf16")
    nv = W.normal_bits(rng, (case.batch, 8, 128), "bf16")
    P.kv_cache_write(bits_to_dev(nk, "bf16"), bits_to_dev(nv, "bf16"), dc.k, dc.v,
                     torch.from_numpy(nxt).cuda())
    kc, vc = oracle.kv_cache_write(nk, nv, kc, vc, nxt)
    assert np.array_equal(dev_to_bits(dc.k), kc) and np.array_equal(dev_to_bits(dc.v), vc)
    lens2 = (new_lens + 1).astype(np.int32)
    q1 = W.normal_bits(rng, (case.batch, 1, 32, 128), "bf16")
    out2 = run_decode(P, dc, split=True, partition_size=1024, q=bits_to_dev(q1, "bf16"),
                      cl=torch.from_numpy(lens2).cuda())
    ref2 = oracle.paged_attention(q1, kc, vc, case.block_tables, lens2, case.scale, 4, "bf16")
    assert max_err(out2, ref2) <= TOL


# ------------------------------------------------------------------ K8/V4 with G * q_len < 4

K8_FEW_ROWS = {
    "g1_d128": lambda: small(150, batch=4, num_q_heads=8, num_kv_heads=8, head_dim=128,
                             lengths=[1, 37, 300, 513]),
    "g2_d64": lambda: small(151, batch=4, num_q_heads=8, num_kv_heads=4, head_dim=64,
                            lengths=[16, 33, 200, 700]),
    "g2_d128_bf16": lambda: small(152, batch=3, num_q_heads=16, num_kv_heads=8, head_dim=128,
                                  fmt="bf16", lengths=[90, 260, 1100]),
    "g3_d64": lambda: small(153, batch=3, num_q_heads=6, num_kv_heads=2, head_dim=64,
                            lengths=[5, 140, 529]),
    "g1_q3_d64": lambda: small(154, batch=4, q_len=3, num_q_heads=4, num_kv_heads=4, head_dim=64,
                               lengths=[3, 17, 130, 600]),
    "g1_q3_d128": lambda: small(155, batch=3, q_len=3, num_q_heads=8, num_kv_heads=8,
                                head_dim=128, lengths=[2, 48, 777]),
}
_k8 = {}


def k8_few(name):
    if name not in _k8:
        case = K8_FEW_ROWS[name]()
        arrs = oracle_k8v4_pool(case)[0]
        ref = oracle.paged_attention_k8v4(case.query, case.fmt, *arrs, case.block_tables,
                                          case.context_lens, case.scale, case.gqa_factor)
        _k8[name] = (case, arrs, ref, k8v4_append_expected(case))
    return _k8[name]


@pytest.mark.parametrize("name", list(K8_FEW_ROWS))
@pytest.mark.parametrize("split,psize", [(False, 0), (True, 512), (True, 32)])
def test_k8v4_few_query_rows(P, name, split, psize):
    case, arrs, ref, _ = k8_few(name)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()      # noqa: E731
    q = bits_to_dev(case.query, case.fmt)
    args = (*[dev(a) for a in arrs], dev(case.block_tables), dev(case.context_lens), case.scale,
            case.gqa_factor)
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    if split:
        mcl = int(case.context_lens.max())
        n = P.splitkv_workspace_size(*q.shape[:3], q.shape[3], mcl, psize)
        ws = torch.full((n // 4 + 4,), float("nan"), dtype=torch.float32, device="cuda")
        P.paged_attention_decode_splitkv_k8v4(out, q, *args, mcl, psize, ws)
    else:
        P.paged_attention_decode_k8v4(out, q, *args)
    torch.cuda.synchronize()
    err = max_err(out, ref)
    assert err <= 2e-4, f"{name}: fp32-out max abs err {err}"


@pytest.mark.parametrize("name", list(K8_FEW_ROWS))
@pytest.mark.parametrize("split,psize", [(False, 0), (True, 512), (True, 32)])
def test_k8v4_few_query_rows_append(P, name, split, psize):
    case, _, _, (before, after, ref) = k8_few(name)
    out, arrs = run_k8v4_append(P, case, before, split=split, psize=psize or 512)
    assert_k8v4_arrays_equal(arrs, after)
    err = max_err(out, ref)
    assert err <= 2e-4, f"{name}: fp32-out max abs err {err}"


# ------------------------------------------------------------------ K8/V4 head groups
#
# With eight KV heads and at least one workgroup of eight heads per CU
# (partitions x sequences >= 256 here), the K8/V4 kernel runs one wavefront per
# head, each over its whole partition, eight heads per workgroup.

K8_HEAD_GROUPS = {
    # 10 partitions of 32 tokens x 40 sequences = 400 head-group workgroups
    "hg_b40_p32": (lambda: small(160, batch=40, num_q_heads=32, num_kv_heads=8, head_dim=128,
                                 lengths=lambda r: r.integers(200, 320, size=40)), 32),
    "hg_g1_d64_p16": (lambda: small(161, batch=48, num_q_heads=8, num_kv_heads=8, head_dim=64,
                                    fmt="bf16", lengths=lambda r: r.integers(1, 150, size=48)), 16),
    "hg_q2_g2_p64": (lambda: small(162, batch=36, q_len=2, num_q_heads=16, num_kv_heads=8,
                                   head_dim=128, lengths=lambda r: r.integers(2, 600, size=36)), 64),
    # the K8/V4 batch at partition 512: 16 x 16 = 256 workgroups
    "k8v4_p512": (lambda: W.k8v4(), 512),
}
_hg = {}


def hg_case(name):
    if name not in _hg:
        _hg.clear()
        case = K8_HEAD_GROUPS[name][0]()
        arrs = oracle_k8v4_pool(case)[0]
        ref = oracle.paged_attention_k8v4(case.query, case.fmt, *arrs, case.block_tables,
                                          case.context_lens, case.scale, case.gqa_factor)
        _hg[name] = (case, arrs, ref, k8v4_append_expected(case))
    return _hg[name]


@pytest.mark.parametrize("name", list(K8_HEAD_GROUPS))
def test_k8v4_head_groups(P, name):
    case, arrs, ref, (before, after, aref) = hg_case(name)
    psize = K8_HEAD_GROUPS[name][1]
    print(f"[k8v4 head groups] {name} partition {psize}", flush=True)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()      # noqa: E731
    q = bits_to_dev(case.query, case.fmt)
    mcl = int(case.context_lens.max())
    n = P.splitkv_workspace_size(*q.shape[:3], q.shape[3], mcl, psize)
    ws = torch.full((n // 4 + 4,), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    P.paged_attention_decode_splitkv_k8v4(out, q, *[dev(a) for a in arrs], dev(case.block_tables),
                                          dev(case.context_lens), case.scale, case.gqa_factor,
                                          mcl, psize, ws)
    torch.cuda.synchronize()
    err = max_err(out, ref)
    assert err <= 2e-4, f"{name}: fp32-out max abs err {err}"
    out2, got = run_k8v4_append(P, case, before, split=True, psize=psize)
    assert_k8v4_arrays_equal(got, after)
    err = max_err(out2, aref)
    assert err <= 2e-4, f"{name} append: fp32-out max abs err {err}"


# ------------------------------------------------------------------ 16-bit eight-head groups
#
# When the one-head grid needs more than seven and at most eight workgroups per
# CU (of 256) and the KV heads divide by eight, the 16-bit kernel runs eight heads per workgroup,
# one wavefront per head over its whole partition.

EIGHTS = {
    # 32K at 128-token partitions: 256 x 8 = 2048 one-head workgroups
    "long32k_p128": (lambda: W.long32k(), 128, 2000),
    # 10 partitions of 32 tokens x 8 heads x 24 sequences = 1920 (the
    # longest sequence, 319 or 300 tokens, sets the 10 partitions)
    "eights_b24_p32": (lambda: small(163, batch=24, q_len=1, num_q_heads=32, num_kv_heads=8,
                                     head_dim=128, fmt="bf16",
                                     lengths=lambda r: np.concatenate(
                                         [[319], r.integers(200, 320, size=23)])), 32, 100),
    "eights_q2_d64_p32": (lambda: small(164, batch=24, q_len=2, num_q_heads=16, num_kv_heads=8,
                                        head_dim=64, lengths=lambda r: np.concatenate(
                                            [[300], r.integers(2, 300, size=23)])),
                          32, 40),
}


@pytest.mark.parametrize("name", list(EIGHTS))
def test_eight_head_groups(P, name):
    builder, psize, window = EIGHTS[name]
    case = builder()
    dc = DevCase(case)
    for kind in ("decode", "append", "window_append"):
        print(f"[eights] {name} {kind} partition {psize}", flush=True)
        ref, kc, vc = _reference(case, kind, window)
        if kind == "decode":
            out = run_decode(P, dc, split=True, partition_size=psize)
        elif kind == "append":
            out, k, v = run_append(P, dc, split=True, psize=psize)
        else:
            out, k, v = run_window_append(P, dc, window, split=True, psize=psize)
        if kind != "decode":
            assert np.array_equal(dev_to_bits(k), kc) and np.array_equal(dev_to_bits(v), vc)
        err = max_err(out, ref)
        assert err <= 2e-4, f"{name} {kind}: fp32-out max abs err {err}"


# The merge of the split partials: with few output rows (at most two per
# compute unit) each row is taken by D / 32 workgroups of 32 dims, else by one
# workgroup that loops over rounds of loads when the partitions are many.
MERGES = {
    # 188 partitions, 8 rows, head_dim 64: two 32-dim slices per row
    "slices_d64": lambda: small(165, batch=1, q_len=1, num_q_heads=8, num_kv_heads=2,
                                head_dim=64, lengths=[6000]),
    # 244 partitions (not a multiple of the 32 groups), 8 rows, head_dim 128,
    # the shorter sequence's tail partitions empty: four slices per row
    "slices_d128_ragged": lambda: small(166, batch=2, q_len=1, num_q_heads=4, num_kv_heads=1,
                                        head_dim=128, fmt="bf16", lengths=[3000, 7777]),
    # 125 partitions, 640 rows: whole rows, two rounds of loads
    "rows_two_rounds": lambda: small(167, batch=20, q_len=2, num_q_heads=16, num_kv_heads=4,
                                     head_dim=128, lengths=_uniform(3500, 4000, 20)),
}


@pytest.mark.parametrize("name", list(MERGES))
def test_merge_forms(P, name):
    """32-token partitions, decode and append against the oracle."""
    case = MERGES[name]()
    dc = DevCase(case)
    for kind in ("decode", "append"):
        print(f"[merge forms] {name} {kind}", flush=True)
        ref, kc, vc = _reference(case, kind, 0)
        if kind == "decode":
            out = run_decode(P, dc, split=True, partition_size=32)
        else:
            out, k, v = run_append(P, dc, split=True, psize=32)
            assert np.array_equal(dev_to_bits(k), kc), f"{name}: key cache differs"
            assert np.array_equal(dev_to_bits(v), vc), f"{name}: value cache differs"
        err = max_err(out, ref)
        assert err <= 2e-4, f"{name} {kind}: fp32-out max abs err {err}"
