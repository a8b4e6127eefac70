"""ctypes binding of libpagedkv_probe.so (include/pagedkv_probe.h): read-only
measurement probes used by ``bench.py --ceiling``.  Argument marshalling only."""

from __future__ import annotations

import ctypes
import os

from ._binding import PagedKVError, _ptr, _stream

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpagedkv_probe.so")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m paged_kv_cache_181_amd.build`")
    import torch  # noqa: F401  (one HIP runtime in the process, as for the main library)
    return ctypes.CDLL(LIB_PATH)


lib = _load()
_p, _i, _i64, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = {
    "pkv_probe_last_error": ([], ctypes.c_char_p),
    "pkv_probe_stream_read": ([_p, _p, _sz, _i, _i, _i, _p, _sz, _p], _i),
    "pkv_probe_paged_read": ([_p, _p, _p, _i, _i64, _i, _i, _i, _i, _i, _i, _i, _p, _sz, _p], _i),
    "pkv_probe_k8v4_read": ([_p, _p, _p, _p, _p, _p, _i, _i64, _i, _i, _i, _i, _i, _p, _sz, _p],
                            _i),
}
for _name, (_args, _res) in SIGNATURES.items():
    getattr(lib, _name).argtypes = _args
    getattr(lib, _name).restype = _res


def _check(rc):
    if rc != 0:
        raise PagedKVError(rc, lib.pkv_probe_last_error().decode())


def stream_read(buf0, buf1, workgroups, waves, depth, sink):
    """Plain streaming read of two equal device buffers (see pagedkv_probe.h)."""
    nbytes = buf0.numel() * buf0.element_size()
    if buf1.numel() * buf1.element_size() != nbytes:
        raise ValueError("the two buffers must have the same size")
    _check(lib.pkv_probe_stream_read(_ptr(buf0), _ptr(buf1), nbytes, workgroups, waves, depth,
                                     _ptr(sink), sink.numel(), _stream(buf0.device)))


def paged_read(k_cache, v_cache, block_table, heads_per_wg, waves, part_blocks, depth, lds_bytes,
               sink):
    """Paged read of one sequence's blocks with the partition kernel's lane
    addressing (see pagedkv_probe.h)."""
    nb, bs, hkv, d = k_cache.shape
    _check(lib.pkv_probe_paged_read(_ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                    block_table.numel(), nb, hkv, d, heads_per_wg, waves,
                                    part_blocks, depth, lds_bytes, _ptr(sink), sink.numel(),
                                    _stream(k_cache.device)))


def k8v4_read(k_codes, k_scale, v_codes, v_scale, v_zero, block_table, part_blocks, depth,
              lds_bytes, sink):
    """Paged read of a K8/V4 cache's blocks with the head-group form's lane
    addressing (see pagedkv_probe.h)."""
    nb, bs, hkv, d = k_codes.shape
    _check(lib.pkv_probe_k8v4_read(_ptr(k_codes), _ptr(v_codes), _ptr(k_scale), _ptr(v_scale),
                                   _ptr(v_zero), _ptr(block_table), block_table.numel(), nb, hkv,
                                   d, part_blocks, depth, lds_bytes, _ptr(sink), sink.numel(),
                                   _stream(k_codes.device)))
