"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path
through the C ABI, and compare with the fp64 oracle on the same inputs."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
import paged_kv_decode_pkv_amd as pkv
import workloads
from workloads import bf16_to_f32

DEV = "cuda:0"
# Tolerances on bf16 outputs and fp32 LSE (over active rows).
OUT_MAX_ABS = 1e-2
OUT_MEAN_ABS = 1e-3
LSE_MAX_ABS = 1e-3


def to_dev_u16(a: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bits (host) -> bf16 tensor on the GPU, same bits."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(
        torch.bfloat16)


def to_host_u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def table_to_dev(table: workloads.PageTable):
    return tuple(torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(DEV)
                 for x in (table.indptr, table.indices, table.last_len))


def gpu_step(cache_dev, layer, ld_dev, tables_dev, table, sm_scale, chunk=0,
             max_pages=None, append=True):
    """One append + decode of ``layer`` through the C ABI; returns (out, lse)."""
    q, kn, vn = ld_dev
    if append:
        pkv.append(cache_dev, layer, kn, vn, *tables_dev)
    mp = table.max_pages_per_req if max_pages is None else max_pages
    return pkv.decode(cache_dev, layer, q, *tables_dev, sm_scale, max_pages_per_req=mp,
                      kv_chunk_pages=chunk)


def compare(out_gpu, lse_gpu, out_ref, lse_ref, rows=None, what=""):
    """Check bf16 GPU rows against fp64 oracle rows; return the error stats."""
    og = bf16_to_f32(to_host_u16(out_gpu)).astype(np.float64)
    lg = lse_gpu.detach().cpu().numpy().astype(np.float64)
    if rows is not None:
        og, lg = og[rows], lg[rows]
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg)), f"{what}: non-finite"
    err = np.abs(og - out_ref)
    lerr = np.abs(lg - lse_ref)
    stats = {"out_max": float(err.max()), "out_mean": float(err.mean()),
             "lse_max": float(lerr.max())}
    assert stats["out_max"] <= OUT_MAX_ABS, f"{what}: {stats}"
    assert stats["out_mean"] <= OUT_MEAN_ABS, f"{what}: {stats}"
    assert stats["lse_max"] <= LSE_MAX_ABS, f"{what}: {stats}"
    return stats


def host_layer_case(spec, table, layer, stale="random", unused="zero"):
    """Host data of one layer, plus its device copies."""
    ld = workloads.layer_data(spec, table, layer, stale=stale, unused=unused)
    return ld, (to_dev_u16(ld.q), to_dev_u16(ld.k_new), to_dev_u16(ld.v_new))


def oracle_rows_from_device(cache_dev_layer, ld_host, table, entries, heads, sm_scale,
                            chunk=0):
    """Oracle rows for (entries x heads) of a layer whose cache lives on the GPU.

    ``cache_dev_layer`` must still hold the PRE-append pages (device tensor
    [NP, 2, PS, Hkv, D]); only the listed entries' pages are copied to host,
    into a compact cache whose page ids are renumbered (the result does not
    depend on physical page ids).  ``ld_host`` holds host q/k_new/v_new.
    """
    entries = list(entries)
    pages = [table.indices[table.indptr[b]:table.indptr[b + 1]] for b in entries]
    flat = np.concatenate(pages).astype(np.int64)
    host_pages = to_host_u16(cache_dev_layer[torch.from_numpy(flat).to(DEV)])
    mini = np.zeros((1, 1 + len(flat)) + host_pages.shape[1:], dtype=np.uint16)
    mini[0, 1:] = host_pages
    indptr = np.zeros(len(entries) + 1, dtype=np.int32)
    indptr[1:] = np.cumsum([len(p) for p in pages])
    indices = np.arange(1, 1 + len(flat), dtype=np.int32)
    last = np.asarray(table.last_len)[entries].astype(np.int32)
    oracle.append(mini, 0, ld_host.k_new[entries], ld_host.v_new[entries], indptr,
                  indices, last)
    rb = np.repeat(np.arange(len(entries)), len(heads))
    rh = np.tile(np.asarray(heads), len(entries))
    out, lse = oracle.decode_rows(mini, 0, ld_host.q[entries], indptr, indices, last,
                                  sm_scale, rb, rh, chunk_pages=chunk)
    return out, lse, (np.asarray(entries)[rb], rh)


def oracle_threads() -> int:
    """Host threads the oracle may use in a test: every CPU of the process's
    affinity set, at most 16 (the oracle releases the GIL)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_all_rows_from_device(cache_dev_layer, ld_host, table, sm_scale):
    """Oracle rows for EVERY active entry and EVERY query head of a layer whose
    cache lives on the GPU (pre-append pages, as for oracle_rows_from_device).

    The active entries' pages are copied to the host once; the oracle appends
    the new rows there and then computes the rows on a pool of host threads,
    each taking its own share of the (entry, head) rows.  Returns (out fp64
    [A, Hq, D], lse fp64 [A, Hq], active entry ids)."""
    entries = np.flatnonzero(table.active)
    pages = [table.indices[table.indptr[b]:table.indptr[b + 1]] for b in entries]
    flat = np.concatenate(pages).astype(np.int64)
    host_pages = to_host_u16(cache_dev_layer[torch.from_numpy(flat).to(DEV)])
    mini = np.zeros((1, 1 + len(flat)) + host_pages.shape[1:], dtype=np.uint16)
    mini[0, 1:] = host_pages
    del host_pages
    indptr = np.zeros(len(entries) + 1, dtype=np.int32)
    indptr[1:] = np.cumsum([len(p) for p in pages])
    indices = np.arange(1, 1 + len(flat), dtype=np.int32)
    last = np.asarray(table.last_len)[entries].astype(np.int32)
    q = np.ascontiguousarray(ld_host.q[entries])
    oracle.append(mini, 0, ld_host.k_new[entries], ld_host.v_new[entries], indptr,
                  indices, last)
    hq = q.shape[1]
    rb = np.repeat(np.arange(len(entries)), hq)
    rh = np.tile(np.arange(hq), len(entries))
    # interleaved shares: long and short entries spread over the threads
    nt = oracle_threads()
    shares = [np.arange(i, len(rb), nt) for i in range(nt)]

    def job(idx):
        return oracle.decode_rows(mini, 0, q, indptr, indices, last, sm_scale, rb[idx],
                                  rh[idx])

    out = np.zeros((len(rb), q.shape[2]))
    lse = np.zeros(len(rb))
    with ThreadPoolExecutor(max_workers=nt) as ex:
        for idx, (o, l) in zip(shares, ex.map(job, shares)):
            out[idx], lse[idx] = o, l
    return out.reshape(len(entries), hq, -1), lse.reshape(len(entries), hq), entries
