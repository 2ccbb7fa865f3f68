"""The C ABI loads and validates host arguments without a GPU (CPU only).

Only calls that must fail validation (or are no-ops) are made here: nothing
reaches the HIP runtime.
"""
import ctypes
import subprocess

import numpy as np
import pytest

import paged_kv_decode_pkv_amd as pkv
from paged_kv_decode_pkv_amd import CacheDesc, lib

FAKE = ctypes.c_void_p(0x100000)      # never dereferenced: validation fails first
NULL = ctypes.c_void_p(0)
DESC = CacheDesc(2, 64, 16, 2, 64)


def test_every_declared_symbol_is_exported():
    names = pkv.declared_functions()
    assert set(names) == {"pkv_append", "pkv_qk_norm_rope_append", "pkv_prefill",
                          "pkv_qk_norm_mrope_append",
                          "pkv_decode_workspace_size",
                          "pkv_append_decode", "pkv_decode", "pkv_plan", "pkv_run",
                          "pkv_run_qk_norm_rope", "pkv_decode_static",
                          "pkv_plan_mixed", "pkv_mixed_run", "pkv_run_qk_norm_mrope",
                          "pkv_validate_page_table", "pkv_status_string",
                          "pkv_last_hip_error"}
    for n in names:
        assert hasattr(lib, n), n
    dyn = subprocess.run(["nm", "-D", "--defined-only", pkv.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in dyn.splitlines() if " T " in line}
    assert set(names) <= exported


def test_status_strings():
    for code, name in pkv.STATUS.items():
        assert pkv.status_string(code).startswith(name)
    assert pkv.status_string(12345) == "unknown pkv status"


def test_workspace_size():
    d = CacheDesc(36, 8192, 16, 8, 128)
    # fixed runs of 16 pages over entries of at most 16 pages: one run each;
    # the plan holds 8 x (1 + 32) records per block row of 8 entries
    ws = pkv.workspace_size(d, 32, 64, 16, 16)
    assert ws >= 64 * (1 + 32) * 16 and ws % 256 == 0
    # fixed runs of 32 pages over 2048-page entries: 64 runs of partials
    # (fp16 outputs and an fp32 {lse, scale} pair per row)
    ws = pkv.workspace_size(d, 32, 8, 2048, 32)
    rows = 8 * 64 * 32
    assert ws >= rows * 128 * 2 + rows * 8 + 8 * 4096 * 16 and ws % 256 == 0
    # balanced: a record per tile of batch x max_pages pages, partial slots for
    # every workgroup plus every entry, counters and entry descriptors
    wb = pkv.workspace_size(d, 32, 64, 256, 0)
    assert wb >= 64 * 256 * 2 * 16 + 64 * 32 * (128 * 2 + 8) + 64 * 8 * 4 + 64 * 16
    assert pkv.workspace_size(d, 32, 0, 256, 0) == 0
    assert pkv.workspace_size(d, 30, 64, 256, 0) > 0        # sizes only
    assert pkv.workspace_size(CacheDesc(36, 8192, 12, 8, 128), 32, 64, 256, 0) == 0
    # pages of fewer than 8 tokens are one tile each
    assert (pkv.workspace_size(CacheDesc(1, 64, 2, 8, 128), 32, 64, 256, 16)
            > pkv.workspace_size(CacheDesc(1, 64, 2, 8, 128), 32, 64, 128, 16))


def _decode(desc=DESC, layer=0, q=FAKE, hq=4, batch=3, scale=0.125, out=FAKE, lse=NULL,
            maxp=4, chunk=0, ws=NULL, wsb=0, tables=(FAKE, FAKE, FAKE)):
    return lib.pkv_decode(FAKE, desc, layer, q, hq, *tables, batch, scale, out, lse, maxp,
                          chunk, ws, wsb, NULL)


def _append(desc=DESC, layer=0, batch=3, k=FAKE, v=FAKE, tables=(FAKE, FAKE, FAKE),
            cache=FAKE):
    return lib.pkv_append(cache, desc, layer, k, v, *tables, batch, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(layer=2), -2), (dict(layer=-1), -2), (dict(batch=-1), -2),
    (dict(desc=CacheDesc(2, 64, 12, 2, 64)), -3), (dict(desc=CacheDesc(2, 64, 0, 2, 64)), -2),
    (dict(desc=CacheDesc(2, 64, 512, 2, 64)), -3), (dict(desc=CacheDesc(0, 64, 16, 2, 64)), -2),
    (dict(desc=CacheDesc(2, 64, 16, 2, 60)), -3),
    (dict(k=NULL), -1), (dict(tables=(FAKE, NULL, FAKE)), -1), (dict(cache=NULL), -1),
    (dict(k=ctypes.c_void_p(0x100008)), -6),
])
def test_append_validation(kw, code):
    assert _append(**kw) == code


def test_append_batch_zero_is_noop():
    assert _append(batch=0, k=NULL, v=NULL, cache=NULL) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(layer=5), -2), (dict(batch=-2), -2), (dict(hq=3), -2), (dict(hq=0), -2),
    (dict(scale=float("nan")), -2), (dict(scale=float("inf")), -2), (dict(maxp=0), -2),
    (dict(chunk=-1), -2), (dict(chunk=65537), -3), (dict(hq=18), -3),
    (dict(desc=CacheDesc(2, 64, 16, 17, 64), hq=17), -3),
    (dict(desc=CacheDesc(2, 64, 16, 2, 96)), -3), (dict(desc=CacheDesc(2, 64, 6, 2, 64)), -3),
    (dict(q=NULL), -1), (dict(out=NULL), -1), (dict(tables=(FAKE, FAKE, NULL)), -1),
    (dict(maxp=40, chunk=16), -4),
    (dict(maxp=40, chunk=16, ws=FAKE, wsb=16), -4),
    (dict(out=ctypes.c_void_p(0x100004)), -6),
])
def test_decode_validation(kw, code):
    assert _decode(**kw) == code


def test_decode_batch_zero_is_noop():
    assert _decode(batch=0, q=NULL, out=NULL, tables=(NULL, NULL, NULL)) == 0


def _norm_rope(desc=DESC, layer=0, q=FAKE, hq=4, k=FAKE, v=FAKE, qw=FAKE, kw=FAKE, eps=1e-6,
               theta=1e6, pos=FAKE, batch=3, q_out=FAKE, cache=FAKE,
               tables=(FAKE, FAKE, FAKE)):
    return lib.pkv_qk_norm_rope_append(cache, desc, layer, q, hq, k, v, qw, kw, eps, theta,
                                       pos, *tables, batch, q_out, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(layer=2), -2), (dict(batch=-1), -2), (dict(hq=0), -2),
    (dict(eps=-1.0), -2), (dict(eps=float("nan")), -2), (dict(theta=0.0), -2),
    (dict(theta=float("inf")), -2), (dict(desc=CacheDesc(2, 64, 16, 2, 32)), -3),
    (dict(desc=CacheDesc(2, 64, 12, 2, 64)), -3),
    (dict(q=NULL), -1), (dict(kw=NULL), -1), (dict(pos=NULL), -1), (dict(q_out=NULL), -1),
    (dict(tables=(FAKE, FAKE, NULL)), -1), (dict(cache=NULL), -1),
    (dict(qw=ctypes.c_void_p(0x100008)), -6), (dict(q_out=ctypes.c_void_p(0x100004)), -6),
    # head counts whose 32-bit sum would overflow are rejected before any sum
    (dict(hq=0x7fffffff), -2), (dict(hq=65536), -2),
    (dict(desc=CacheDesc(2, 64, 16, 70000, 64)), -2),
])
def test_norm_rope_validation(kw, code):
    assert _norm_rope(**kw) == code


def test_norm_rope_batch_zero_is_noop():
    assert _norm_rope(batch=0, q=NULL, k=NULL, v=NULL, qw=NULL, kw=NULL, pos=NULL,
                      q_out=NULL, cache=NULL, tables=(NULL, NULL, NULL)) == 0


def _prefill(desc=CacheDesc(2, 64, 16, 2, 128), layer=0, q=FAKE, hq=4, qo=FAKE, k=FAKE,
             v=FAKE, batch=3, maxr=8, scale=0.1, out=FAKE, tables=(FAKE, FAKE, FAKE)):
    return lib.pkv_prefill(FAKE, desc, layer, q, hq, qo, k, v, *tables, batch, maxr, scale,
                           out, NULL, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(layer=2), -2), (dict(batch=-1), -2), (dict(hq=3), -2), (dict(maxr=0), -2),
    (dict(scale=float("nan")), -2), (dict(desc=CacheDesc(2, 64, 16, 2, 32)), -3),
    (dict(batch=70000), -3), (dict(q=NULL), -1), (dict(qo=NULL), -1), (dict(out=NULL), -1),
    (dict(k=NULL), -1), (dict(tables=(FAKE, NULL, FAKE)), -1),
    (dict(out=ctypes.c_void_p(0x100004)), -6), (dict(hq=0x7fffffff), -2),
])
def test_prefill_validation(kw, code):
    assert _prefill(**kw) == code


def test_prefill_batch_zero_is_noop():
    assert _prefill(batch=0, q=NULL, qo=NULL, k=NULL, v=NULL, out=NULL,
                    tables=(NULL, NULL, NULL)) == 0


def _append_decode(k=FAKE, v=FAKE, layer=0, batch=3, chunk=0, hq=4, out=FAKE):
    return lib.pkv_append_decode(FAKE, DESC, layer, k, v, FAKE, hq, FAKE, FAKE, FAKE, batch,
                                 0.125, out, NULL, 4, chunk, NULL, 0, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(k=NULL), -1), (dict(v=NULL), -1), (dict(layer=9), -2), (dict(hq=3), -2),
    (dict(out=NULL), -1), (dict(k=ctypes.c_void_p(0x100002)), -6),
    (dict(), -4),                                  # balanced needs a workspace
])
def test_append_decode_validation(kw, code):
    assert _append_decode(**kw) == code


def test_append_decode_batch_zero_is_noop():
    assert _append_decode(batch=0, k=NULL, v=NULL, out=NULL) == 0


def _plan(desc=DESC, hq=4, batch=3, maxp=4, chunk=0, ws=NULL, wsb=0,
          tables=(FAKE, FAKE, FAKE)):
    return lib.pkv_plan(desc, hq, *tables, batch, maxp, chunk, ws, wsb, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), -2), (dict(hq=3), -2), (dict(maxp=0), -2), (dict(chunk=-1), -2),
    (dict(chunk=65537), -3), (dict(desc=CacheDesc(2, 64, 16, 2, 96)), -3),
    (dict(tables=(FAKE, NULL, FAKE)), -1), (dict(), -4), (dict(chunk=2), -4),
    (dict(ws=FAKE, wsb=16), -4),
    (dict(ws=ctypes.c_void_p(0x100010), wsb=1 << 30), -6),
])
def test_plan_validation(kw, code):
    assert _plan(**kw) == code


def _run(k=NULL, v=NULL, layer=0, batch=3, hq=4, q=FAKE, out=FAKE, chunk=0, ws=NULL,
         wsb=0, scale=0.125):
    return lib.pkv_run(FAKE, DESC, layer, k, v, q, hq, batch, scale, out, NULL, 4, chunk,
                       ws, wsb, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(layer=2), -2), (dict(hq=3), -2), (dict(scale=float("nan")), -2),
    (dict(q=NULL), -1), (dict(out=NULL), -1), (dict(k=FAKE), -1), (dict(v=FAKE), -1),
    (dict(out=ctypes.c_void_p(0x100004)), -6),
    (dict(k=FAKE, v=ctypes.c_void_p(0x100002)), -6),
    (dict(), -4), (dict(chunk=1, ws=FAKE, wsb=64), -4),
])
def test_run_validation(kw, code):
    assert _run(**kw) == code


def test_plan_and_run_batch_zero_are_noops():
    assert _plan(batch=0, tables=(NULL, NULL, NULL)) == 0
    assert _run(batch=0, q=NULL, out=NULL) == 0


def _plan_mixed(hq=4, qo=FAKE, batch=3, rows=5, maxp=4, chunk=0, ws=NULL, wsb=0,
                tables=(FAKE, FAKE, FAKE)):
    return lib.pkv_plan_mixed(DESC, hq, qo, *tables, batch, rows, maxp, chunk, ws, wsb, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), -2), (dict(rows=-1), -2), (dict(hq=3), -2), (dict(maxp=0), -2),
    (dict(batch=70000), -3), (dict(rows=9000), -3), (dict(qo=NULL), -1),
    (dict(tables=(FAKE, NULL, FAKE)), -1), (dict(), -4),
])
def test_plan_mixed_validation(kw, code):
    assert _plan_mixed(**kw) == code


def _mixed_run(layer=0, q=FAKE, hq=4, qo=FAKE, k=FAKE, v=FAKE, batch=3, rows=5, maxr=4,
               scale=0.125, out=FAKE, chunk=0, ws=NULL, wsb=0):
    return lib.pkv_mixed_run(FAKE, DESC, layer, q, hq, qo, k, v, FAKE, FAKE, FAKE, batch,
                             rows, maxr, scale, out, NULL, 4, chunk, ws, wsb, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(layer=2), -2), (dict(rows=-1), -2), (dict(hq=3), -2), (dict(maxr=0), -2),
    (dict(scale=float("inf")), -2), (dict(qo=NULL), -1), (dict(q=NULL), -1),
    (dict(k=NULL), -1), (dict(out=ctypes.c_void_p(0x100004)), -6),
    (dict(), -4),                                  # the decode rows need their plan
])
def test_mixed_run_validation(kw, code):
    assert _mixed_run(**kw) == code


def test_mixed_batch_zero_is_noop():
    assert _plan_mixed(batch=0, rows=0, qo=NULL, tables=(NULL, NULL, NULL)) == 0
    assert _mixed_run(batch=0, rows=0, q=NULL, qo=NULL, k=NULL, v=NULL, out=NULL) == 0


def test_validate_page_table():
    indptr = np.array([0, 2, 3, 4])
    indices = np.array([5, 7, 0, 9])
    last = np.array([3, 1, 16])
    assert pkv.validate_page_table(indptr, indices, last, 16, 16, 4) == (0, -1)
    bad = [
        (np.array([1, 2, 3, 4]), indices, last, -1),          # indptr[0] != 0
        (np.array([0, 2, 2, 4]), indices, last, 1),           # empty entry
        (indptr, indices, np.array([3, 2, 16]), 1),           # padding with 2 rows
        (indptr, np.array([5, 0, 0, 9]), last, 0),            # page 0 in a real entry
        (indptr, np.array([5, 7, 0, 16]), last, 2),           # id out of range
        (indptr, indices, np.array([0, 1, 16]), 0),           # last_len 0
        (indptr, indices, np.array([3, 1, 17]), 2),           # last_len > page_size
        (indptr, np.array([5, 7, 0, 7]), last, 2),            # two appends into page 7
    ]
    for ip, ix, ll, entry in bad:
        assert pkv.validate_page_table(ip, ix, ll, 16, 16, 4) == (-7, entry)
    assert pkv.validate_page_table(indptr, indices, last, 16, 16, 1) == (-7, 0)


def test_single_hip_runtime_shared_with_torch():
    # torch's streams and allocations are only meaningful to torch's own HIP
    # runtime instance; libpkv must resolve to that same instance.
    import os
    import torch
    rts = pkv._hip_runtimes()
    assert len(rts) == 1
    assert os.path.dirname(next(iter(rts))) == os.path.realpath(
        os.path.join(os.path.dirname(torch.__file__), "lib"))


DESC128 = CacheDesc(2, 64, 16, 2, 128)


def _run_nr(desc=DESC128, layer=0, k=FAKE, v=FAKE, q=FAKE, hq=8, batch=3, qw=FAKE, kw=FAKE,
            eps=1e-6, theta=1e6, pos=FAKE, scale=0.125, out=FAKE, chunk=0, ws=NULL, wsb=0):
    return lib.pkv_run_qk_norm_rope(FAKE, desc, layer, k, v, q, hq, batch, qw, kw, eps, theta,
                                    pos, scale, out, NULL, 4, chunk, ws, wsb, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(layer=2), -2), (dict(hq=3), -2), (dict(scale=float("nan")), -2),
    (dict(eps=-1.0), -2), (dict(eps=float("inf")), -2), (dict(theta=0.0), -2),
    (dict(theta=float("nan")), -2),
    (dict(desc=CacheDesc(2, 64, 16, 2, 64)), -3),      # head_dim 128 only
    (dict(hq=10), -3),                                  # groups up to 4
    (dict(k=NULL), -1), (dict(v=NULL), -1), (dict(qw=NULL), -1), (dict(kw=NULL), -1),
    (dict(pos=NULL), -1), (dict(q=NULL), -1), (dict(out=NULL), -1),
    (dict(kw=ctypes.c_void_p(0x100008)), -6), (dict(out=ctypes.c_void_p(0x100004)), -6),
    (dict(), -4), (dict(chunk=1, ws=FAKE, wsb=64), -4),
])
def test_run_norm_rope_validation(kw, code):
    assert _run_nr(**kw) == code


def test_run_norm_rope_batch_zero_is_noop():
    assert _run_nr(batch=0, k=NULL, v=NULL, q=NULL, qw=NULL, kw=NULL, pos=NULL,
                   out=NULL) == 0


AXIS = (ctypes.c_uint8 * 32)(*([0] * 11 + [1] * 11 + [2] * 10))
AXIS64 = (ctypes.c_uint8 * 64)(*([0] * 24 + [1] * 20 + [2] * 20))


def _run_nmr(axis=AXIS64, desc=DESC128, batch=3, hq=8, pos=FAKE, theta=1e6, k=FAKE):
    return lib.pkv_run_qk_norm_mrope(FAKE, desc, 0, k, FAKE, FAKE, hq, batch, FAKE, FAKE, 1e-6,
                                     theta, pos, axis, 0.125, FAKE, NULL, 4, 0, NULL, 0, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(axis=None), -1), (dict(axis=(ctypes.c_uint8 * 64)(*([0] * 63 + [3]))), -2),
    (dict(theta=-1.0), -2), (dict(hq=10), -3), (dict(desc=CacheDesc(2, 64, 16, 2, 64)), -3),
    (dict(pos=NULL), -1), (dict(k=NULL), -1), (dict(), -4),
])
def test_run_norm_mrope_validation(kw, code):
    assert _run_nmr(**kw) == code


def test_run_norm_mrope_batch_zero_is_noop():
    assert _run_nmr(batch=0, pos=NULL, k=NULL) == 0


def _norm_mrope(axis=AXIS, desc=DESC, batch=3, q=FAKE, pos=FAKE, eps=1e-6):
    return lib.pkv_qk_norm_mrope_append(FAKE, desc, 0, q, 4, FAKE, FAKE, FAKE, FAKE, eps, 1e6,
                                        pos, axis, FAKE, FAKE, FAKE, batch, FAKE, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(axis=None), -1), (dict(axis=(ctypes.c_uint8 * 32)(*([0] * 31 + [3]))), -2),
    (dict(eps=-1.0), -2), (dict(desc=CacheDesc(2, 64, 16, 2, 32)), -3),
    (dict(q=NULL), -1), (dict(pos=NULL), -1),
])
def test_norm_mrope_validation(kw, code):
    assert _norm_mrope(**kw) == code


def test_norm_mrope_batch_zero_is_noop():
    assert _norm_mrope(batch=0) == 0


def test_decode_static_rejects_what_its_array_cannot_hold():
    # 16 MiB of device memory behind pkv_decode_static: a call needing more is
    # refused before anything reaches the device (no GPU here), argument
    # errors as for pkv_decode, batch 0 a no-op
    d = CacheDesc(1, 1 << 20, 16, 8, 128)
    assert pkv.workspace_size(d, 32, 4096, 4096, 0) > 16 << 20
    assert lib.pkv_decode_static(FAKE, d, 0, FAKE, 32, FAKE, FAKE, FAKE, 4096, 0.1, FAKE,
                                 NULL, 4096, 0, NULL) == -4
    assert lib.pkv_decode_static(FAKE, d, 1, FAKE, 32, FAKE, FAKE, FAKE, 4, 0.1, FAKE, NULL,
                                 16, 0, NULL) == -2
    assert lib.pkv_decode_static(FAKE, d, 0, FAKE, 30, FAKE, FAKE, FAKE, 4, 0.1, FAKE, NULL,
                                 16, 0, NULL) == -2
    assert lib.pkv_decode_static(NULL, d, 0, NULL, 32, NULL, NULL, NULL, 0, 0.1, NULL, NULL,
                                 16, 0, NULL) == 0
