"""The read probes (include/pagedkv_probe.h) read exactly the bytes they are
timed on.

Each probe folds every 32-bit word it loads into one XOR per wavefront and
stores it to `sink`.  A word loaded an even number of times cancels, so the
fold of a wave equals the XOR of the words it reads an odd number of times:
for the streaming read, its share of the slice; for the paged reads, the K
and V rows of its KV head in its run of blocks (the K8/V4 scale loads are
issued by the four lanes of a token alike and cancel).  The expected folds
are computed here with numpy from the same buffers.
"""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def probe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_181_amd import probe as pr
    return pr


def _xor(a):
    return int(np.bitwise_xor.reduce(np.ascontiguousarray(a).view(np.uint32).ravel()))


def _sink_words(sink, n):
    return sink[:n].cpu().view(torch.int32).numpy().view(np.uint32)


@pytest.mark.parametrize("wgs,waves,depth", [(4, 4, 1), (8, 8, 2), (2, 16, 4), (6, 8, 8)])
def test_stream_read_folds_its_slice(probe, wgs, waves, depth):
    g = torch.Generator().manual_seed(wgs * 100 + waves + depth)
    half = wgs // 2
    nbytes = half * waves * depth * 1024 * 3                 # three rounds per workgroup
    b0 = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g)
    b1 = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g)
    sink = torch.zeros(wgs * waves + 8, dtype=torch.float32, device="cuda")
    probe.stream_read(b0.cuda(), b1.cuda(), wgs, waves, depth, sink)
    got = _sink_words(sink, wgs * waves)
    slice_words = nbytes // half // 4
    for i in range(wgs):
        src = (b0 if i < half else b1).numpy().view(np.uint32)
        sl = src[(i % half) * slice_words:(i % half + 1) * slice_words]
        for w in range(waves):
            # wave w: chunks w*depth .. +depth-1 of every round of waves*depth KiB
            chunks = sl.reshape(-1, waves, depth, 256)[:, w]
            assert got[i * waves + w] == _xor(chunks), (i, w)


@pytest.mark.parametrize("hp,waves,part,depth", [(2, 8, 32, 2), (1, 8, 32, 3), (8, 8, 8, 4),
                                                 (4, 16, 16, 1)])
def test_paged_read_folds_its_heads_rows(probe, hp, waves, part, depth):
    g = torch.Generator().manual_seed(hp * 1000 + waves * 10 + depth)
    nb, hkv, d, table = 96, 8, 128, 64
    k = torch.randint(-2**15, 2**15 - 1, (nb, 16, hkv, d), dtype=torch.int16, generator=g)
    v = torch.randint(-2**15, 2**15 - 1, (nb, 16, hkv, d), dtype=torch.int16, generator=g)
    bt = torch.randperm(nb, generator=g)[:table].to(torch.int32)
    bt[5] = -1                                                # entries outside the pool: not read
    bt[17] = nb + 3
    grid_x, grid_y = table // part, hkv // hp
    sink = torch.zeros(grid_x * grid_y * waves + 8, dtype=torch.float32, device="cuda")
    probe.paged_read(k.cuda().view(torch.float16), v.cuda().view(torch.float16), bt.cuda(), hp,
                     waves, part, depth, 0, sink)
    got = _sink_words(sink, grid_x * grid_y * waves)
    kn, vn, btn = k.numpy(), v.numpy(), bt.numpy()
    nwh, per = waves // hp, part // (waves // hp)
    for y in range(grid_y):
        for x in range(grid_x):
            for w in range(waves):
                head = y * hp + w // nwh
                blocks = [b for b in btn[x * part + (w % nwh) * per:x * part + (w % nwh + 1) * per]
                          if 0 <= b < nb]
                want = _xor(kn[blocks, :, head]) ^ _xor(vn[blocks, :, head]) if blocks else 0
                assert got[(y * grid_x + x) * waves + w] == want, (x, y, w)


@pytest.mark.parametrize("part,depth", [(32, 2), (8, 1), (16, 3), (64, 4)])
def test_k8v4_read_folds_its_heads_rows(probe, part, depth):
    g = torch.Generator().manual_seed(part * 10 + depth)
    nb, hkv, d, table = 160, 8, 128, 128
    kc = torch.randint(-128, 127, (nb, 16, hkv, d), dtype=torch.int8, generator=g)
    vc = torch.randint(0, 255, (nb, 16, hkv, d // 2), dtype=torch.uint8, generator=g)
    ks = torch.randint(-2**15, 2**15 - 1, (nb, 16, hkv), dtype=torch.int16, generator=g)
    vs = torch.randint(-2**15, 2**15 - 1, (nb, 16, hkv, d // 32), dtype=torch.int16, generator=g)
    vz = torch.randint(-2**15, 2**15 - 1, (nb, 16, hkv, d // 32), dtype=torch.int16, generator=g)
    bt = torch.randperm(nb, generator=g)[:table].to(torch.int32)
    bt[3] = -7
    bt[40] = nb
    sink = torch.zeros(table // part * 8 + 8, dtype=torch.float32, device="cuda")
    probe.k8v4_read(kc.cuda(), ks.cuda().view(torch.float16), vc.cuda(),
                    vs.cuda().view(torch.float16), vz.cuda().view(torch.float16), bt.cuda(), part,
                    depth, 0, sink)
    got = _sink_words(sink, table // part * 8)
    kn, vn, btn = kc.numpy(), vc.numpy(), bt.numpy()
    for x in range(table // part):
        blocks = [b for b in btn[x * part:(x + 1) * part] if 0 <= b < nb]
        for head in range(hkv):
            want = _xor(kn[blocks, :, head]) ^ _xor(vn[blocks, :, head]) if blocks else 0
            assert got[x * 8 + head] == want, (x, head)
