"""GPU parity of the balanced split-KV decode (partition_size 0).

With partition_size 0 the split-KV calls cut the batch's blocks, laid end to
end per KV head, into equal runs, one per wavefront, and merge one partial per
(run, sequence) piece.  Same contract and result as any partition size: these
tests compare it with the oracle (fp32 output within 2e-4, 16-bit output the
fp32 result rounded once), with the caches after the append form bit-exact,
and with the fixed-partition split; plus batches of more than 64 sequences,
empty sequences among non-empty ones, NaN poison past the lengths, run-to-run
determinism and HIP graph replay.
"""

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_181_amd import workloads as W

from gpu_util import TOL, DevCase, dev_to_bits, max_err, run_decode
from test_gpu_parity import APPEND_CASES, CASES, get_append_case, get_case, run_append, small

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_181_amd as lib
    return lib


EXTRA = {
    # 150 sequences (three chunks of 64 lengths), many shorter than a run
    "many_short": lambda: small(170, batch=150, q_len=1, num_q_heads=16, num_kv_heads=4,
                                head_dim=64, lengths=lambda r: r.integers(1, 200, size=150)),
    # empty sequences between others, q_len 2 (rows that see nothing too)
    "empties_q2": lambda: small(171, batch=9, q_len=2, num_q_heads=8, num_kv_heads=2,
                                head_dim=128, fmt="bf16",
                                lengths=[0, 700, 0, 0, 1, 33, 0, 2100, 0]),
    # one sequence over every run, G 1, odd KV head count (one head per workgroup)
    "single_g1_hkv3": lambda: small(172, batch=1, q_len=1, num_q_heads=3, num_kv_heads=3,
                                    head_dim=128, lengths=[5000]),
    # the ragged verify batch's shape at a quarter of its size (16-row tiles)
    "verify_b16": lambda: W.spec_verify(batch=16),
    # G*q_len 6 at head_dim 128 and 10 at 64, one sequence over many runs
    "slices_gq6_d128": lambda: small(174, batch=7, q_len=2, num_q_heads=6, num_kv_heads=2,
                                     head_dim=128, fmt="bf16",
                                     lengths=[9000, 40, 300, 2, 1200, 0, 650]),
    "slices_gq10_d64": lambda: small(175, batch=5, q_len=2, num_q_heads=10, num_kv_heads=2,
                                     head_dim=64, lengths=[7000, 3, 500, 64, 2222]),
}
_extra = {}


def extra_case(name):
    if name not in _extra:
        case = EXTRA[name]()
        _extra[name] = (case, oracle.paged_attention(
            case.query, case.key_cache, case.value_cache, case.block_tables, case.context_lens,
            case.scale, case.gqa_factor, case.fmt))
    return _extra[name]


def balanced(P, dc, out_dtype=torch.float32, q=None, fill=float("nan")):
    c = dc.case
    q = dc.q if q is None else q
    out = torch.full(q.shape, float("nan"), dtype=out_dtype, device="cuda")
    B, Q, Hq, D = q.shape
    mcl = int(dc.cl.max().item())
    n = P.splitkv_workspace_size(B, Q, Hq, D, mcl, 0)
    ws = torch.full((n // 4 + 4,), fill, dtype=torch.float32, device="cuda")
    P.paged_attention_decode_splitkv(out, q, dc.k, dc.v, dc.bt, dc.cl, c.scale, c.gqa_factor,
                                     mcl, 0, ws)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", list(CASES) + list(EXTRA))
def test_balanced_matches_oracle(P, name):
    case, ref = extra_case(name) if name in EXTRA else get_case(name)
    print(f"[balanced] {name}", flush=True)
    dc = DevCase(case)
    out32 = balanced(P, dc)
    err = max_err(out32, ref)
    assert err <= 2e-4, f"{name}: fp32-out max abs err {err}"
    out16 = balanced(P, dc, out_dtype=dc.q.dtype)
    assert torch.equal(out16, out32.to(dc.q.dtype))
    assert max_err(out16, ref) <= TOL or int(case.context_lens.min()) < 256


@pytest.mark.parametrize("name", list(APPEND_CASES))
def test_balanced_append_matches_write_then_attend(P, name):
    case, (ref, kc, vc) = get_append_case(name)
    print(f"[balanced append] {name}", flush=True)
    dc = DevCase(case)
    out, k, v = run_append(P, dc, split=True, psize=0)
    assert np.array_equal(dev_to_bits(k), kc), "key cache after the append differs"
    assert np.array_equal(dev_to_bits(v), vc), "value cache after the append differs"
    err = max_err(out, ref)
    assert err <= 2e-4, f"{name}: fp32-out max abs err {err}"


def test_balanced_agrees_with_fixed_partitions(P):
    case, _ = get_case("llama8b_batch")
    dc = DevCase(case)
    a = balanced(P, dc)
    b = run_decode(P, dc, split=True, partition_size=512)
    assert (a - b).abs().max().item() <= 1e-5


def test_balanced_nan_poison_is_never_read(P):
    case = small(173, batch=6, q_len=2, num_q_heads=8, num_kv_heads=2, head_dim=64,
                 lengths=[3, 17, 40, 129, 300, 1])
    ref = oracle.paged_attention(case.query, case.key_cache, case.value_cache, case.block_tables,
                                 case.context_lens, case.scale, case.gqa_factor, case.fmt)
    W.poison_unused(case)
    out = balanced(P, DevCase(case))
    assert max_err(out, ref) <= 2e-4


def test_balanced_is_deterministic_and_graph_replays_match(P):
    case, _ = get_case("spec_verify")
    dc = DevCase(case)
    first = balanced(P, dc)
    for _ in range(3):
        assert torch.equal(balanced(P, dc), first)
    B, Q, Hq, D = dc.q.shape
    mcl = int(dc.cl.max().item())
    ws = torch.zeros(P.splitkv_workspace_size(B, Q, Hq, D, mcl, 0) // 4 + 4, device="cuda")
    out = torch.zeros(dc.q.shape, dtype=torch.float32, device="cuda")

    def step():
        P.paged_attention_decode_splitkv(out, dc.q, dc.k, dc.v, dc.bt, dc.cl, case.scale,
                                         case.gqa_factor, mcl, 0, ws)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, first), f"replay {rep}"
        run_decode(P, dc, split=False)              # eager work between replays


def test_balanced_no_alloc(P):
    case, ref = get_case("llama8b_batch")
    dc = DevCase(case)
    out = torch.full(dc.q.shape, float("nan"), dtype=torch.float32, device="cuda")
    P.paged_attention_decode_splitkv_noalloc(out, dc.q, dc.k, dc.v, dc.bt, dc.cl, case.scale,
                                             case.gqa_factor, int(case.context_lens.max()), 0)
    torch.cuda.synchronize()
    assert torch.equal(out, balanced(P, dc))
    assert max_err(out, ref) <= 2e-4
