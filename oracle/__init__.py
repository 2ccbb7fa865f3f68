"""fp64 CPU oracle for paged-KV decode attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it and
shares no code with it; the two meet only through the seeded inputs of
``workloads``.

The arithmetic lives in ``pkv_oracle.c`` (plain C loops in fp64).  This module
compiles that file with gcc into ``liboracle.so`` and wraps its three calls:

* :func:`append` -- bit copy of each entry's new K/V row into its last page
  ("Adding a Model", vox-serve docs, section 1: ``set_kv_cache``).
* :func:`decode` -- softmax(sm_scale * q K^T) V per (entry, query head) over
  the entry's page list, natural-log LSE, optional split into fixed page runs
  merged by log-sum-exp ("Adding a Model", section 1: ``run``; "Supported
  Models", LTX-2.5 notes, for merging partial attentions).
* :func:`decode_rows` -- the same for a chosen list of rows.
* :func:`qk_norm_rope_append` -- per-head RMSNorm of q and k, rotary
  embedding at each entry's position, and the KV write of the rotated k and
  the v rows ("Supported Models", M* docs, Qwen3-Omni and Qwen3-TTS notes:
  q/k norm, RoPE and KV write as one fused step).
* :func:`qk_norm_mrope_append` -- the same with multimodal RoPE: a (t, h, w)
  position per entry, each rotary pair following one named component (the
  Qwen3-Omni Thinker's q/k norm + multimodal RoPE + KV write, same notes).
* :func:`bf16_round` -- fp64 to bf16, round to nearest even.
* :func:`append_rows` / :func:`prefill` -- several new rows per entry: their
  append at the entry's last positions, and the causal attention of each row
  over the tokens up to its own position (paged prefill and mixed steps).

Every function here is pinned by ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pkv_oracle.c")
# PKV_ORACLE_LIB: another build of pkv_oracle.c to load instead (the
# sanitizer test runs every pin against an AddressSanitizer build)
_LIB_PATH = os.environ.get("PKV_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the C oracle with gcc (-O2, no hand SIMD) into a shared library."""
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load(path: str = _LIB_PATH):
    """Load (building first if absent) and return the ctypes handle."""
    global _lib
    if _lib is not None and path == _LIB_PATH:
        return _lib
    if not os.path.exists(path) or (
            path == _LIB_PATH and not os.environ.get("PKV_ORACLE_LIB")
            and os.path.getmtime(path) < os.path.getmtime(_SRC)):
        build(out=path)
    lib = ctypes.CDLL(path)
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_append.argtypes = [p] + [i64] * 6 + [p, p, p, p, p, i64]
    lib.oracle_append.restype = ctypes.c_int
    lib.oracle_decode.argtypes = ([p] + [i64] * 6 + [p, i64, p, p, p, i64,
                                  ctypes.c_double, i64, p, p])
    lib.oracle_decode.restype = ctypes.c_int
    lib.oracle_decode_rows.argtypes = ([p] + [i64] * 6 + [p, i64, p, p, p, i64,
                                       ctypes.c_double, i64, p, p, i64, p, p])
    lib.oracle_decode_rows.restype = ctypes.c_int
    d64 = ctypes.c_double
    lib.oracle_qk_norm_rope_append.argtypes = ([p] + [i64] * 6 + [p, i64, p, p, p, p, d64,
                                               d64, p, p, p, p, i64, p, p])
    lib.oracle_qk_norm_rope_append.restype = ctypes.c_int
    lib.oracle_qk_norm_mrope_append.argtypes = ([p] + [i64] * 6 + [p, i64, p, p, p, p, d64,
                                                d64, p, p, p, p, p, i64, p, p])
    lib.oracle_qk_norm_mrope_append.restype = ctypes.c_int
    lib.oracle_append_rows.argtypes = [p] + [i64] * 6 + [p, p, p, p, p, p, i64]
    lib.oracle_append_rows.restype = ctypes.c_int
    lib.oracle_prefill.argtypes = [p] + [i64] * 6 + [p, i64, p, p, p, p, i64, d64, p, p]
    lib.oracle_prefill.restype = ctypes.c_int
    lib.oracle_bf16_round.argtypes = [d64]
    lib.oracle_bf16_round.restype = ctypes.c_uint16
    if path == _LIB_PATH:
        _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check_cache(cache: np.ndarray):
    if cache.dtype != np.uint16 or cache.ndim != 6 or not cache.flags.c_contiguous:
        raise ValueError("cache must be C-contiguous uint16 (bf16 bits) "
                         "[layers, pages, 2, page_size, kv_heads, head_dim]")
    if cache.shape[2] != 2:
        raise ValueError("cache axis 2 must hold K and V")


def _tables(indptr, indices, last_len):
    return (np.ascontiguousarray(indptr, dtype=np.int32),
            np.ascontiguousarray(indices, dtype=np.int32),
            np.ascontiguousarray(last_len, dtype=np.int32))


def append(cache, layer, k_new, v_new, indptr, indices, last_len, lib=None):
    """In-place bit copy of k_new/v_new [batch, Hkv, D] (uint16) into ``cache``."""
    lib = lib or load()
    _check_cache(cache)
    nl, npg, _, ps, hkv, d = cache.shape
    indptr, indices, last_len = _tables(indptr, indices, last_len)
    k_new = np.ascontiguousarray(k_new, dtype=np.uint16)
    v_new = np.ascontiguousarray(v_new, dtype=np.uint16)
    batch = len(last_len)
    if k_new.shape != (batch, hkv, d) or v_new.shape != (batch, hkv, d):
        raise ValueError("k_new/v_new must be [batch, Hkv, D]")
    rc = lib.oracle_append(_ptr(cache), nl, npg, ps, hkv, d, layer, _ptr(k_new),
                           _ptr(v_new), _ptr(indptr), _ptr(indices), _ptr(last_len),
                           batch)
    if rc:
        raise ValueError(f"oracle_append rejected the page table (code {rc})")


def decode(cache, layer, q, indptr, indices, last_len, sm_scale, chunk_pages=0,
           lib=None):
    """Return (out fp64 [batch, Hq, D], lse fp64 [batch, Hq]) for every row."""
    lib = lib or load()
    _check_cache(cache)
    nl, npg, _, ps, hkv, d = cache.shape
    indptr, indices, last_len = _tables(indptr, indices, last_len)
    q = np.ascontiguousarray(q, dtype=np.uint16)
    batch, hq, dq = q.shape
    if dq != d or batch != len(last_len):
        raise ValueError("q must be [batch, Hq, D]")
    out = np.zeros((batch, hq, d), dtype=np.float64)
    lse = np.zeros((batch, hq), dtype=np.float64)
    rc = lib.oracle_decode(_ptr(cache), nl, npg, ps, hkv, d, layer, _ptr(q), hq,
                           _ptr(indptr), _ptr(indices), _ptr(last_len), batch,
                           float(sm_scale), int(chunk_pages), _ptr(out), _ptr(lse))
    if rc:
        raise ValueError(f"oracle_decode failed (code {rc})")
    return out, lse


def decode_rows(cache, layer, q, indptr, indices, last_len, sm_scale, rows_b,
                rows_hq, chunk_pages=0, lib=None):
    """Return (out fp64 [n, D], lse fp64 [n]) for rows (rows_b[i], rows_hq[i])."""
    lib = lib or load()
    _check_cache(cache)
    nl, npg, _, ps, hkv, d = cache.shape
    indptr, indices, last_len = _tables(indptr, indices, last_len)
    q = np.ascontiguousarray(q, dtype=np.uint16)
    batch, hq, _ = q.shape
    rows_b = np.ascontiguousarray(rows_b, dtype=np.int64)
    rows_hq = np.ascontiguousarray(rows_hq, dtype=np.int64)
    n = len(rows_b)
    out = np.zeros((n, d), dtype=np.float64)
    lse = np.zeros((n,), dtype=np.float64)
    rc = lib.oracle_decode_rows(_ptr(cache), nl, npg, ps, hkv, d, layer, _ptr(q), hq,
                                _ptr(indptr), _ptr(indices), _ptr(last_len), batch,
                                float(sm_scale), int(chunk_pages), _ptr(rows_b),
                                _ptr(rows_hq), n, _ptr(out), _ptr(lse))
    if rc:
        raise ValueError(f"oracle_decode_rows failed (code {rc})")
    return out, lse


def qk_norm_rope_append(cache, layer, q, k_new, v_new, q_norm_w, k_norm_w, eps, theta,
                        positions, indptr, indices, last_len, lib=None):
    """Return (q_out fp64 [batch, Hq, D], k_out fp64 [batch, Hkv, D]); write
    bf16(k_out) and v_new into each entry's append slot of ``cache``."""
    lib = lib or load()
    _check_cache(cache)
    nl, npg, _, ps, hkv, d = cache.shape
    indptr, indices, last_len = _tables(indptr, indices, last_len)
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k_new = np.ascontiguousarray(k_new, dtype=np.uint16)
    v_new = np.ascontiguousarray(v_new, dtype=np.uint16)
    q_norm_w = np.ascontiguousarray(q_norm_w, dtype=np.uint16)
    k_norm_w = np.ascontiguousarray(k_norm_w, dtype=np.uint16)
    positions = np.ascontiguousarray(positions, dtype=np.int32)
    batch, hq, dq = q.shape
    if (dq != d or batch != len(last_len) or k_new.shape != (batch, hkv, d)
            or v_new.shape != (batch, hkv, d) or q_norm_w.shape != (d,)
            or k_norm_w.shape != (d,) or positions.shape != (batch,)):
        raise ValueError("shapes: q [batch, Hq, D], k_new/v_new [batch, Hkv, D], "
                         "weights [D], positions [batch]")
    q_out = np.zeros((batch, hq, d), dtype=np.float64)
    k_out = np.zeros((batch, hkv, d), dtype=np.float64)
    rc = lib.oracle_qk_norm_rope_append(
        _ptr(cache), nl, npg, ps, hkv, d, layer, _ptr(q), hq, _ptr(k_new), _ptr(v_new),
        _ptr(q_norm_w), _ptr(k_norm_w), float(eps), float(theta), _ptr(positions),
        _ptr(indptr), _ptr(indices), _ptr(last_len), batch, _ptr(q_out), _ptr(k_out))
    if rc:
        raise ValueError(f"oracle_qk_norm_rope_append failed (code {rc})")
    return q_out, k_out


def bf16_round(x, lib=None) -> np.ndarray:
    """fp64 values rounded to bf16 bits (nearest, ties to even), one by one."""
    lib = lib or load()
    flat = np.asarray(x, dtype=np.float64).ravel()
    out = np.array([lib.oracle_bf16_round(float(v)) for v in flat], dtype=np.uint16)
    return out.reshape(np.shape(x))


def qk_norm_mrope_append(cache, layer, q, k_new, v_new, q_norm_w, k_norm_w, eps, theta,
                         positions, pair_axis, indptr, indices, last_len, lib=None):
    """Multimodal RoPE: positions [batch, 3] (t, h, w), pair_axis [D/2] (each 0,
    1 or 2); returns (q_out, k_out) fp64 and writes the cache as
    :func:`qk_norm_rope_append` does."""
    lib = lib or load()
    _check_cache(cache)
    nl, npg, _, ps, hkv, d = cache.shape
    indptr, indices, last_len = _tables(indptr, indices, last_len)
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k_new = np.ascontiguousarray(k_new, dtype=np.uint16)
    v_new = np.ascontiguousarray(v_new, dtype=np.uint16)
    q_norm_w = np.ascontiguousarray(q_norm_w, dtype=np.uint16)
    k_norm_w = np.ascontiguousarray(k_norm_w, dtype=np.uint16)
    positions = np.ascontiguousarray(positions, dtype=np.int32)
    pair_axis = np.ascontiguousarray(pair_axis, dtype=np.uint8)
    batch, hq, dq = q.shape
    if (dq != d or batch != len(last_len) or k_new.shape != (batch, hkv, d)
            or v_new.shape != (batch, hkv, d) or q_norm_w.shape != (d,)
            or k_norm_w.shape != (d,) or positions.shape != (batch, 3)
            or pair_axis.shape != (d // 2,)):
        raise ValueError("shapes: q [batch, Hq, D], k_new/v_new [batch, Hkv, D], "
                         "weights [D], positions [batch, 3], pair_axis [D/2]")
    q_out = np.zeros((batch, hq, d), dtype=np.float64)
    k_out = np.zeros((batch, hkv, d), dtype=np.float64)
    rc = lib.oracle_qk_norm_mrope_append(
        _ptr(cache), nl, npg, ps, hkv, d, layer, _ptr(q), hq, _ptr(k_new), _ptr(v_new),
        _ptr(q_norm_w), _ptr(k_norm_w), float(eps), float(theta), _ptr(positions),
        _ptr(pair_axis), _ptr(indptr), _ptr(indices), _ptr(last_len), batch, _ptr(q_out),
        _ptr(k_out))
    if rc:
        raise ValueError(f"oracle_qk_norm_mrope_append failed (code {rc})")
    return q_out, k_out


def append_rows(cache, layer, k_new, v_new, qo_indptr, indptr, indices, last_len,
                lib=None):
    """In-place bit copy of each entry's new rows k_new/v_new [rows, Hkv, D]
    into its last positions."""
    lib = lib or load()
    _check_cache(cache)
    nl, npg, _, ps, hkv, d = cache.shape
    indptr, indices, last_len = _tables(indptr, indices, last_len)
    qo_indptr = np.ascontiguousarray(qo_indptr, dtype=np.int32)
    k_new = np.ascontiguousarray(k_new, dtype=np.uint16)
    v_new = np.ascontiguousarray(v_new, dtype=np.uint16)
    rows = int(qo_indptr[-1])
    if k_new.shape != (rows, hkv, d) or v_new.shape != (rows, hkv, d):
        raise ValueError("k_new/v_new must be [rows, Hkv, D]")
    rc = lib.oracle_append_rows(_ptr(cache), nl, npg, ps, hkv, d, layer, _ptr(k_new),
                                _ptr(v_new), _ptr(qo_indptr), _ptr(indptr), _ptr(indices),
                                _ptr(last_len), len(last_len))
    if rc:
        raise ValueError(f"oracle_append_rows rejected the tables (code {rc})")


def prefill(cache, layer, q, qo_indptr, indptr, indices, last_len, sm_scale, lib=None):
    """Return (out fp64 [rows, Hq, D], lse fp64 [rows, Hq]): causal attention
    of each new row over its entry's tokens up to its own position."""
    lib = lib or load()
    _check_cache(cache)
    nl, npg, _, ps, hkv, d = cache.shape
    indptr, indices, last_len = _tables(indptr, indices, last_len)
    qo_indptr = np.ascontiguousarray(qo_indptr, dtype=np.int32)
    q = np.ascontiguousarray(q, dtype=np.uint16)
    rows, hq, dq = q.shape
    if dq != d or rows != int(qo_indptr[-1]) or len(qo_indptr) != len(last_len) + 1:
        raise ValueError("q must be [rows, Hq, D] with rows = qo_indptr[-1]")
    out = np.zeros((rows, hq, d), dtype=np.float64)
    lse = np.zeros((rows, hq), dtype=np.float64)
    rc = lib.oracle_prefill(_ptr(cache), nl, npg, ps, hkv, d, layer, _ptr(q), hq,
                            _ptr(qo_indptr), _ptr(indptr), _ptr(indices), _ptr(last_len),
                            len(last_len), float(sm_scale), _ptr(out), _ptr(lse))
    if rc:
        raise ValueError(f"oracle_prefill failed (code {rc})")
    return out, lse
