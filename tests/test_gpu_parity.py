"""Parity of the HIP path (through the C ABI) with the fp64 oracle on the GPU.

Bars: pkv_append bit-exact; pkv_decode out within max |err| 1e-2 and mean
|err| 1e-3 (bf16 output against fp64), lse within 1e-3, over active rows.
Inputs are the seeded workloads of ``workloads`` (host numpy for the small
configurations, torch's seeded GPU generator for the multi-gigabyte ones).
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_pkv_amd as pkv
import workloads
from golden_cases import build_case, load_cases
from gpu_util import (DEV, compare, gpu_step, host_layer_case, oracle_all_rows_from_device,
                      oracle_rows_from_device, table_to_dev, to_dev_u16, to_host_u16)
from workloads import CONFIGS, bf16_to_f32, make_table, table_from_lengths

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def _full_cache(spec_or_shape, table, layer_data_list):
    """Device cache [L, NP, 2, PS, Hkv, D] from per-layer host slabs."""
    slabs = np.stack([ld.cache for ld in layer_data_list])
    return to_dev_u16(slabs)


def _oracle_full(cache_host, layer, ld, table, scale, chunk=0):
    oracle.append(cache_host, layer, ld.k_new, ld.v_new, table.indptr, table.indices,
                  table.last_len)
    return oracle.decode(cache_host, layer, ld.q, table.indptr, table.indices,
                         table.last_len, scale, chunk)


# ---------------------------------------------------------------- golden cases
@pytest.mark.parametrize("chunk", [0, 1])
def test_golden_cases(chunk):
    for case in load_cases():
        g = build_case(case)
        cache = to_dev_u16(g["cache"])
        tables = tuple(torch.from_numpy(x).to(DEV)
                       for x in (g["indptr"], g["indices"], g["last_len"]))
        q = to_dev_u16(g["q"])
        maxp = int(np.diff(g["indptr"]).max())
        out, lse = pkv.decode(cache, 0, q, *tables, g["sm_scale"], max_pages_per_req=maxp,
                              kv_chunk_pages=chunk)
        m = g["checked"]
        compare(out, lse, g["out"][m], g["lse"][m], rows=m, what=case["name"])


# ------------------------------------------------------------ random shapes
SHAPES = [
    # hq, hkv, d, page_size, lengths, active
    (1, 1, 64, 16, [1, 17, 200], None),
    (2, 2, 128, 16, [5, 64, 300, 16], [1, 1, 0, 1]),
    (3, 1, 128, 8, [100, 1, 33], None),
    (4, 2, 64, 1, [9, 40, 3], None),
    (5, 1, 64, 2, [77, 2], None),
    (6, 3, 128, 4, [51, 18, 1, 250], [1, 1, 0, 1]),
    (7, 1, 64, 32, [500, 31, 32, 33], None),
    (8, 2, 128, 128, [129, 700, 1], None),
    (14, 2, 64, 16, [256, 255, 1, 97], [1, 0, 1, 1]),
    (32, 8, 128, 16, [1024, 4096, 64, 3], None),
]


@pytest.mark.parametrize("idx", range(len(SHAPES)))
@pytest.mark.parametrize("chunk", [0, 1, 3, 64])
def test_random_shapes(idx, chunk):
    hq, hkv, d, ps, lengths, active = SHAPES[idx]
    rng = np.random.default_rng(1000 + idx)
    act = np.ones(len(lengths), bool) if active is None else np.asarray(active, bool)
    table = table_from_lengths(lengths, act, ps, None, rng)
    lds = [workloads.draw_layer(rng, table, hq, hkv, d, 1.0, stale="nan", unused="nan")
           for _ in range(2)]
    cache_host = np.stack([ld.cache for ld in lds])
    cache = to_dev_u16(cache_host)
    tables = table_to_dev(table)
    scale = 1.0 / math.sqrt(d)
    for layer in (1, 0):
        ld = lds[layer]
        dev = (to_dev_u16(ld.q), to_dev_u16(ld.k_new), to_dev_u16(ld.v_new))
        out, lse = gpu_step(cache, layer, dev, tables, table, scale, chunk=chunk)
        ro, rl = _oracle_full(cache_host, layer, ld, table, scale)
        compare(out, lse, ro[act], rl[act], rows=act, what=f"shape {idx} layer {layer}")


# ------------------------------------------------------------------- append
@pytest.mark.parametrize("idx", range(len(SHAPES)))
def test_append_bit_exact(idx):
    hq, hkv, d, ps, lengths, active = SHAPES[idx]
    rng = np.random.default_rng(2000 + idx)
    act = np.ones(len(lengths), bool) if active is None else np.asarray(active, bool)
    table = table_from_lengths(lengths, act, ps, None, rng)
    lds = [workloads.draw_layer(rng, table, hq, hkv, d, 1.0) for _ in range(3)]
    cache_host = np.stack([ld.cache for ld in lds])
    cache = to_dev_u16(cache_host)
    tables = table_to_dev(table)
    for layer in (2, 0):
        ld = lds[layer]
        pkv.append(cache, layer, to_dev_u16(ld.k_new), to_dev_u16(ld.v_new), *tables)
        oracle.append(cache_host, layer, ld.k_new, ld.v_new, table.indptr, table.indices,
                      table.last_len)
        got = to_host_u16(cache)
        pad = np.flatnonzero(~act)
        if len(pad):   # padding entries race on page 0 slot 0: element by element,
            # one or another of their rows wins
            for kv, rows in ((0, ld.k_new), (1, ld.v_new)):
                assert np.all(np.any(got[layer, 0, kv, 0][None] == rows[pad], axis=0))
            got[layer, 0] = cache_host[layer, 0]
        np.testing.assert_array_equal(got, cache_host, err_msg=f"shape {idx} layer {layer}")


@pytest.mark.parametrize("cfg", [1, 2])
def test_append_bit_exact_configs(cfg):
    spec = CONFIGS[cfg]
    table = make_table(spec)
    ld, dev = host_layer_case(spec, table, 0)
    cache_host = ld.cache[None].copy()
    cache = to_dev_u16(cache_host)
    tables = table_to_dev(table)
    pkv.append(cache, 0, dev[1], dev[2], *tables)
    oracle.append(cache_host, 0, ld.k_new, ld.v_new, table.indptr, table.indices,
                  table.last_len)
    got = to_host_u16(cache)
    got[0, 0] = cache_host[0, 0]
    np.testing.assert_array_equal(got, cache_host)


# ------------------------------------------------------------- configs 1, 2
@pytest.mark.parametrize("cfg", [1, 2])
@pytest.mark.parametrize("chunk", [0, 1, 4, 16, 64])
def test_decode_config(cfg, chunk):
    spec = CONFIGS[cfg]
    table = make_table(spec)
    ld, dev = host_layer_case(spec, table, 0, stale="nan")
    cache_host = ld.cache[None].copy()
    cache = to_dev_u16(cache_host)
    out, lse = gpu_step(cache, 0, dev, table_to_dev(table), table, spec.sm_scale, chunk)
    ro, rl = _oracle_full(cache_host, 0, ld, table, spec.sm_scale)
    act = table.active
    compare(out, lse, ro[act], rl[act], rows=act, what=f"cfg{cfg} chunk{chunk}")


# ------------------------------------------------------ device-drawn configs
def _device_case(spec, batch=None, layers=(0,), extra_layers=0):
    """Cache on the GPU drawn with the device generator; host copies of q/k/v."""
    table = make_table(spec, batch)
    nl = max(layers) + 1 + extra_layers
    cache = torch.zeros((nl, table.num_pages, 2, spec.page_size, spec.num_kv_heads,
                         spec.head_dim), dtype=torch.bfloat16, device=DEV)
    per_layer = {}
    for layer in layers:
        q, kn, vn = workloads.draw_layer_device(
            cache[layer], table, [1000 * spec.cfg + layer, table.batch],
            spec.num_qo_heads, spec.sigma, workloads.k_offsets(spec),
            real_head_dim=spec.real_head_dim)
        per_layer[layer] = (q, kn, vn)
    return table, cache, per_layer


class _HostRows:
    def __init__(self, q, kn, vn):
        self.q, self.k_new, self.v_new = to_host_u16(q), to_host_u16(kn), to_host_u16(vn)


def _sampled_check(spec, table, cache, layer, dev, entries, heads, chunk=0, what=""):
    """Run append+decode of one layer; compare sampled rows with the oracle."""
    host_rows = _HostRows(*dev)
    ro, rl, (rb, rh) = oracle_rows_from_device(cache[layer], host_rows, table, entries,
                                               heads, spec.sm_scale)
    out, lse = gpu_step(cache, layer, dev, table_to_dev(table), table, spec.sm_scale,
                        chunk)
    og = out[torch.from_numpy(rb).to(DEV), torch.from_numpy(rh).to(DEV)]
    lg = lse[torch.from_numpy(rb).to(DEV), torch.from_numpy(rh).to(DEV)]
    return compare(og, lg, ro, rl, what=what)


@pytest.mark.parametrize("chunk", [32, 64, 0])
def test_decode_config5_long_context(chunk):
    spec = CONFIGS[5]
    table, cache, per_layer = _device_case(spec)
    _sampled_check(spec, table, cache, 0, per_layer[0], range(spec.batch),
                   [0, 3, 4, 17, 31], chunk=chunk, what=f"cfg5 chunk{chunk}")


@pytest.mark.parametrize("chunk", [0, 4])
def test_decode_config6_cfg_pairs_zero_padded_heads(chunk):
    """CFG talker-like layer: each session's conditional and unconditional
    streams ride one plan as two entries; 128-token pages from a pool of 1025
    with sink page 0; heads of 72 values zero-padded to 128, scale 1/sqrt(72).
    Zero-padding is exact: the padded output columns are exactly zero, and the
    first 72 match the oracle run on the unpadded 72-value heads."""
    spec = CONFIGS[6]
    real = spec.real_head_dim
    table, cache, per_layer = _device_case(spec)
    q, kn, vn = per_layer[0]
    entries = list(range(0, 12))          # six sessions, both streams
    heads = [0, 5, 11, 15]
    # the unpadded oracle case: the entries' pages sliced to 72 values
    pages = [table.indices[table.indptr[b]:table.indptr[b + 1]] for b in entries]
    flat = np.concatenate(pages).astype(np.int64)
    host_pages = to_host_u16(cache[0][torch.from_numpy(flat).to(DEV)])
    assert not host_pages[..., real:].any()
    mini = np.zeros((1, 1 + len(flat)) + host_pages.shape[1:-1] + (real,), dtype=np.uint16)
    mini[0, 1:] = host_pages[..., :real]
    indptr = np.zeros(len(entries) + 1, dtype=np.int32)
    indptr[1:] = np.cumsum([len(p) for p in pages])
    indices = np.arange(1, 1 + len(flat), dtype=np.int32)
    last = table.last_len[entries].astype(np.int32)
    qh, kh, vh = (to_host_u16(t)[entries][..., :real] for t in (q, kn, vn))
    oracle.append(mini, 0, kh, vh, indptr, indices, last)
    rb = np.repeat(np.arange(len(entries)), len(heads))
    rh = np.tile(np.asarray(heads), len(entries))
    ro, rl = oracle.decode_rows(mini, 0, qh, indptr, indices, last, spec.sm_scale, rb, rh)
    out, lse = gpu_step(cache, 0, per_layer[0], table_to_dev(table), table, spec.sm_scale,
                        chunk)
    eb = torch.from_numpy(np.asarray(entries)[rb]).to(DEV)
    eh = torch.from_numpy(rh).to(DEV)
    assert not to_host_u16(out[..., real:]).any(), "padded output columns are not zero"
    compare(out[eb, eh][..., :real], lse[eb, eh], ro, rl, what=f"cfg6 chunk {chunk}")


def _full_check(spec, table, cache, layer, dev, chunk=0, what="", fused=False):
    """Append + decode of one layer in the benchmark's launch shape; EVERY
    active entry x EVERY query head compared with the oracle, element by
    element, at the decode bars."""
    host_rows = _HostRows(*dev)
    ro, rl, ent = oracle_all_rows_from_device(cache[layer], host_rows, table, spec.sm_scale)
    tables = table_to_dev(table)
    if fused:
        q, kn, vn = dev
        out, lse = pkv.append_decode(cache, layer, kn, vn, q, *tables, spec.sm_scale,
                                     max_pages_per_req=table.max_pages_per_req,
                                     kv_chunk_pages=chunk)
    else:
        out, lse = gpu_step(cache, layer, dev, tables, table, spec.sm_scale, chunk)
    sel = torch.from_numpy(ent).to(DEV)
    stats = compare(out[sel], lse[sel], ro, rl, what=what)
    print(f"{what}: {len(ent)} entries x {ro.shape[1]} heads: {stats}", flush=True)
    return stats


@pytest.mark.parametrize("chunk", [0, 32, 64])
def test_decode_config5_all_rows(chunk):
    """Long-context layer (batch 8, 16k-32k tokens, per-head K offsets): every
    query head of every entry, for the balanced split and 32- and 64-page
    runs (16-64 runs merged per entry)."""
    spec = CONFIGS[5]
    table, cache, per_layer = _device_case(spec)
    _full_check(spec, table, cache, 0, per_layer[0], chunk=chunk, what=f"cfg5 chunk{chunk}")


def test_decode_config3_all_rows():
    """Qwen3-4B-like step in the benchmark's launch shape (balanced split,
    fused append + decode): layers 0, 17 and 35, every query head of all 64
    entries."""
    spec = CONFIGS[3]
    table, cache, per_layer = _device_case(spec, layers=(0, 17, 35))
    for layer in (0, 17, 35):
        _full_check(spec, table, cache, layer, per_layer[layer], fused=True,
                    what=f"cfg3 layer {layer}")


@pytest.mark.parametrize("chunk", [0, 16])
def test_decode_config4_all_rows(chunk):
    """Qwen3-0.6B-like layers at batch 256 (26 padding entries): layers 0 and
    27, every query head of every active entry."""
    spec = CONFIGS[4]
    table, cache, per_layer = _device_case(spec, 256, layers=(0, 27))
    for layer in (0, 27):
        _full_check(spec, table, cache, layer, per_layer[layer], chunk=chunk,
                    what=f"cfg4 B=256 layer {layer} chunk {chunk}")


def _pick_entries(table, n):
    act = np.flatnonzero(table.active)
    order = act[np.argsort(table.lengths[act])]
    picks = {int(order[0]), int(order[-1]), int(order[len(order) // 2])}
    rng = np.random.default_rng(7)
    picks |= set(int(x) for x in rng.choice(act, size=min(n, len(act)), replace=False))
    return sorted(picks)


def test_decode_config3_all_layers_sampled():
    """Qwen3-4B-like step: 36 layers, batch 64, in the benchmark's launch shape
    (default chunking, one append + decode per layer); sampled rows of three
    layers are checked against the oracle."""
    spec = CONFIGS[3]
    table = make_table(spec)
    check = {0, 17, 35}
    cache = torch.zeros((spec.num_layers, table.num_pages, 2, 16, 8, 128),
                        dtype=torch.bfloat16, device=DEV)
    tables = table_to_dev(table)
    entries = _pick_entries(table, 5)
    for layer in range(spec.num_layers):
        dev = workloads.draw_layer_device(cache[layer], table, [3000 + layer, 64], 32,
                                          1.0, None)
        if layer in check:
            _sampled_check(spec, table, cache, layer, dev, entries, [0, 9, 22, 31],
                           what=f"cfg3 layer {layer}")
        else:
            gpu_step(cache, layer, dev, tables, table, spec.sm_scale)
    torch.cuda.synchronize()


@pytest.mark.parametrize("batch", workloads.CFG4_SWEEP)
def test_decode_config4_sweep_sampled(batch):
    spec = CONFIGS[4]
    table, cache, per_layer = _device_case(spec, batch, layers=(0, 27))
    entries = _pick_entries(table, 4)
    for layer in (0, 27):
        _sampled_check(spec, table, cache, layer, per_layer[layer], entries, [0, 7, 15],
                       what=f"cfg4 B={batch} layer {layer}")


# ------------------------------------------------------------ invariances
@pytest.mark.parametrize("chunk", [1, 16])
def test_batch_invariance_bit_exact(chunk):
    """With fixed runs, an entry's rows are bit-identical alone, in
    sub-batches and in the full batch (cfg-4 shapes): the split depends only
    on the entry's own length."""
    spec = CONFIGS[4]
    table, cache, per_layer = _device_case(spec, 256)
    q, kn, vn = per_layer[0]
    tables = table_to_dev(table)
    pkv.append(cache, 0, kn, vn, *tables)
    full_out, full_lse = pkv.decode(cache, 0, q, *tables, spec.sm_scale,
                                    max_pages_per_req=table.max_pages_per_req,
                                    kv_chunk_pages=chunk)
    rng = np.random.default_rng(3)
    act = np.flatnonzero(table.active)
    for size in (1, 2, 4, 16, 64):
        sel = rng.choice(act, size=size, replace=False)
        n = np.diff(table.indptr)[sel]
        ip = np.zeros(size + 1, np.int32)
        ip[1:] = np.cumsum(n)
        ix = np.concatenate([table.indices[table.indptr[b]:table.indptr[b + 1]] for b in sel])
        sub = tuple(torch.from_numpy(x.astype(np.int32)).to(DEV)
                    for x in (ip, ix, table.last_len[sel]))
        o, l_ = pkv.decode(cache, 0, q[torch.from_numpy(sel).to(DEV)].contiguous(), *sub,
                           spec.sm_scale, max_pages_per_req=int(n.max()) + 7,
                           kv_chunk_pages=chunk)
        sel_t = torch.from_numpy(sel).to(DEV)
        assert torch.equal(o.view(torch.int16), full_out[sel_t].view(torch.int16))
        assert torch.equal(l_, full_lse[sel_t])


def test_page_relabel_bit_exact():
    spec = CONFIGS[2]
    table = make_table(spec)
    ld, dev = host_layer_case(spec, table, 0)
    cache_host = ld.cache[None].copy()
    cache = to_dev_u16(cache_host)
    out0, lse0 = gpu_step(cache, 0, dev, table_to_dev(table), table, spec.sm_scale)
    perm = np.concatenate([[0], 1 + np.random.default_rng(5).permutation(
        table.num_pages - 1)])
    moved = np.empty_like(cache_host)
    moved[:, perm] = cache_host
    t2 = workloads.PageTable(table.lengths, table.active, table.indptr,
                             perm[table.indices].astype(np.int32), table.last_len,
                             table.num_pages, table.page_size)
    out1, lse1 = gpu_step(to_dev_u16(moved), 0, dev, table_to_dev(t2), t2, spec.sm_scale)
    act = torch.from_numpy(np.flatnonzero(table.active)).to(DEV)
    assert torch.equal(out0[act].view(torch.int16), out1[act].view(torch.int16))
    assert torch.equal(lse0[act], lse1[act])


def test_padding_isolation():
    """Append touches only the entries' target slots and page 0; adding
    padding entries leaves the active rows bit-identical."""
    spec = CONFIGS[2]
    table = make_table(spec)
    ld, dev = host_layer_case(spec, table, 0)
    cache = to_dev_u16(ld.cache[None].copy())
    before = to_host_u16(cache)
    tables = table_to_dev(table)
    pkv.append(cache, 0, dev[1], dev[2], *tables)
    after = to_host_u16(cache)
    changed = np.argwhere(np.any(before != after, axis=(2, 4, 5)))   # (layer, page, slot)
    allowed = {(0, 0, 0)}
    for b in range(table.batch):
        allowed.add((0, int(table.indices[table.indptr[b + 1] - 1]),
                     int(table.last_len[b]) - 1))
    assert {tuple(map(int, x)) for x in changed} <= allowed
    out0, lse0 = pkv.decode(cache, 0, dev[0], *tables, spec.sm_scale,
                            max_pages_per_req=table.max_pages_per_req, kv_chunk_pages=8)
    # the same active entries without any padding entry (fixed runs, so the
    # rows may not depend on the rest of the batch)
    act = np.flatnonzero(table.active)
    n = np.diff(table.indptr)[act]
    ip = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    ix = np.concatenate([table.indices[table.indptr[b]:table.indptr[b + 1]] for b in act])
    sub = tuple(torch.from_numpy(x.astype(np.int32)).to(DEV)
                for x in (ip, ix, table.last_len[act]))
    act_t = torch.from_numpy(act).to(DEV)
    o1, l1 = pkv.decode(cache, 0, dev[0][act_t].contiguous(), *sub, spec.sm_scale,
                        max_pages_per_req=table.max_pages_per_req, kv_chunk_pages=8)
    assert torch.equal(o1.view(torch.int16), out0[act_t].view(torch.int16))
    assert torch.equal(l1, lse0[act_t])


# ------------------------------------------------------------ closed forms
def test_closed_forms():
    spec = CONFIGS[2]
    table = make_table(spec)
    ld, dev = host_layer_case(spec, table, 0)
    act = table.active
    tables = table_to_dev(table)
    # V = 1 everywhere: every convex combination is exactly 1.
    cache_host = ld.cache[None].copy()
    cache_host[:, :, 1] = 0x3F80
    out, _ = gpu_step(to_dev_u16(cache_host), 0,
                      (dev[0], dev[1], torch.ones_like(dev[2])), tables, table,
                      spec.sm_scale)
    assert torch.all(out[torch.from_numpy(np.flatnonzero(act)).to(DEV)] == 1.0)
    # q = 0: lse = ln L and out = mean of V.
    q0 = torch.zeros_like(dev[0])
    cache = to_dev_u16(ld.cache[None].copy())
    _, lse = gpu_step(cache, 0, (q0, dev[1], dev[2]), tables, table, spec.sm_scale)
    want = np.log(table.lengths[act].astype(np.float64))[:, None]
    got = lse.cpu().numpy()[act]
    assert np.max(np.abs(got - want)) < 1e-3
    # L = 1 for every entry: out is v_new of its KV head, bit for bit.
    t1 = table_from_lengths([1] * 8, np.ones(8, bool), 16, 64, np.random.default_rng(1))
    l1 = workloads.draw_layer(np.random.default_rng(2), t1, 24, 8, 128, stale="nan",
                              unused="nan")
    d1 = (to_dev_u16(l1.q), to_dev_u16(l1.k_new), to_dev_u16(l1.v_new))
    out, lse = gpu_step(to_dev_u16(l1.cache[None].copy()), 0, d1, table_to_dev(t1), t1,
                        0.1)
    want = np.repeat(l1.v_new, 3, axis=1)
    np.testing.assert_array_equal(to_host_u16(out), want)


# ------------------------------------------------------------ fused append
@pytest.mark.parametrize("idx", range(len(SHAPES)))
@pytest.mark.parametrize("chunk", [0, 2])
def test_append_decode_fused(idx, chunk):
    """pkv_append_decode leaves the cache bit-identical to pkv_append and gives
    the rows of pkv_decode on it (bit-identical: same split, same values)."""
    hq, hkv, d, ps, lengths, active = SHAPES[idx]
    rng = np.random.default_rng(3000 + idx)
    act = np.ones(len(lengths), bool) if active is None else np.asarray(active, bool)
    table = table_from_lengths(lengths, act, ps, None, rng)
    lds = [workloads.draw_layer(rng, table, hq, hkv, d, 1.0, stale="nan", unused="nan")
           for _ in range(2)]
    cache_host = np.stack([ld.cache for ld in lds])
    fused_cache = to_dev_u16(cache_host)
    sep_cache = to_dev_u16(cache_host)
    tables = table_to_dev(table)
    scale = 1.0 / math.sqrt(d)
    layer = 1
    ld = lds[layer]
    q, kn, vn = to_dev_u16(ld.q), to_dev_u16(ld.k_new), to_dev_u16(ld.v_new)
    mp = table.max_pages_per_req
    fo, fl = pkv.append_decode(fused_cache, layer, kn, vn, q, *tables, scale,
                               max_pages_per_req=mp, kv_chunk_pages=chunk)
    pkv.append(sep_cache, layer, kn, vn, *tables)
    so, sl = pkv.decode(sep_cache, layer, q, *tables, scale, max_pages_per_req=mp,
                        kv_chunk_pages=chunk)
    ro, rl = _oracle_full(cache_host, layer, ld, table, scale)
    got = to_host_u16(fused_cache)
    if (~act).any():
        cands = [ld.k_new[b] for b in np.flatnonzero(~act)]
        assert any(np.array_equal(got[layer, 0, 0, 0], c) for c in cands)
        got[layer, 0] = cache_host[layer, 0]
    np.testing.assert_array_equal(got, cache_host)
    act_t = torch.from_numpy(np.flatnonzero(act)).to(DEV)
    assert torch.equal(fo[act_t].view(torch.int16), so[act_t].view(torch.int16))
    assert torch.equal(fl[act_t], sl[act_t])
    compare(fo, fl, ro[act], rl[act], rows=act, what=f"fused shape {idx}")


def test_append_decode_config3_layers():
    spec = CONFIGS[3]
    table = make_table(spec)
    cache = torch.zeros((3, table.num_pages, 2, 16, 8, 128), dtype=torch.bfloat16,
                        device=DEV)
    tables = table_to_dev(table)
    entries = _pick_entries(table, 5)
    for layer in range(3):
        dev = workloads.draw_layer_device(cache[layer], table, [3000 + layer, 64], 32, 1.0,
                                          None)
        host_rows = _HostRows(*dev)
        ro, rl, (rb, rh) = oracle_rows_from_device(cache[layer], host_rows, table, entries,
                                                   [0, 5, 31], spec.sm_scale)
        out, lse = pkv.append_decode(cache, layer, dev[1], dev[2], dev[0], *tables,
                                     spec.sm_scale, max_pages_per_req=table.max_pages_per_req)
        og = out[torch.from_numpy(rb).to(DEV), torch.from_numpy(rh).to(DEV)]
        lg = lse[torch.from_numpy(rb).to(DEV), torch.from_numpy(rh).to(DEV)]
        compare(og, lg, ro, rl, what=f"fused cfg3 layer {layer}")


@pytest.mark.parametrize("chunk", [4, 0])
def test_entries_over_the_page_bound_get_nan_rows(chunk):
    """An entry listing more pages than max_pages_per_req gets NaN rows (a
    visible broken precondition, in both split modes); the other rows stay
    correct."""
    spec = CONFIGS[2]
    table = make_table(spec)
    ld, dev = host_layer_case(spec, table, 0)
    cache_host = ld.cache[None].copy()
    cache = to_dev_u16(cache_host)
    tables = table_to_dev(table)
    n = np.diff(table.indptr)
    bound = int(np.sort(n)[-3])          # the two longest entries exceed it
    pkv.append(cache, 0, dev[1], dev[2], *tables)
    out, lse = pkv.decode(cache, 0, dev[0], *tables, spec.sm_scale,
                          max_pages_per_req=bound, kv_chunk_pages=chunk)
    over = n > bound
    assert over.any() and (table.active & ~over).any()
    lse_h = lse.cpu().numpy()
    assert np.all(np.isnan(lse_h[over]))
    assert np.all(np.isnan(bf16_to_f32(to_host_u16(out))[over]))
    ro, rl = _oracle_full(cache_host, 0, ld, table, spec.sm_scale)
    ok = table.active & ~over
    compare(out, lse, ro[ok], rl[ok], rows=ok, what="rows under the bound")


def test_run_on_a_mismatched_plan_gives_nan_rows_and_no_cache_writes():
    """pkv_run compares the plan's signature with its own arguments before it
    uses the plan: on a workspace holding no plan (zeroed, or filled with a
    byte pattern) or a plan made for other arguments it writes NaN rows and
    leaves every cache byte as it was, fused append included; a matching plan
    then gives the oracle's rows."""
    spec = CONFIGS[2]
    table = make_table(spec)
    ld, dev = host_layer_case(spec, table, 0)
    cache_host = ld.cache[None].copy()
    cache = to_dev_u16(cache_host)
    tables = table_to_dev(table)
    mp = table.max_pages_per_req
    hq, b = spec.num_qo_heads, table.batch
    desc = pkv.cache_desc(cache)
    need = max(pkv.workspace_size(desc, hq, b, mp, c) for c in (0, 4))
    need = max(need, pkv.workspace_size(desc, hq, b, 2 * mp, 0))

    def expect_nan_untouched(ws, chunk, maxp, what):
        plan = pkv.DecodePlan(ws, b, hq, maxp, chunk)
        out, lse = pkv.run(cache, 0, dev[0], plan, spec.sm_scale, k_new=dev[1], v_new=dev[2])
        torch.cuda.synchronize()
        assert np.all(np.isnan(lse.cpu().numpy())), what
        assert np.all(np.isnan(bf16_to_f32(to_host_u16(out)))), what
        np.testing.assert_array_equal(to_host_u16(cache), cache_host, err_msg=what)

    expect_nan_untouched(torch.zeros(need, dtype=torch.uint8, device=DEV), 0, mp,
                         "zeroed workspace")
    expect_nan_untouched(torch.full((need,), 0xA5, dtype=torch.uint8, device=DEV), 0, mp,
                         "byte-pattern workspace")
    # plans made for other arguments, each in a workspace of its own (a
    # workspace still holding an earlier plan for these very arguments is a
    # valid plan for them: the page table is the caller's to keep unchanged)
    def other_plan(*plan_args):
        ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
        pkv.plan(cache, hq, *plan_args, workspace=ws)
        return ws

    expect_nan_untouched(other_plan(*tables, mp, 0), 4, mp,
                         "planned balanced, run as 4-page runs")
    expect_nan_untouched(other_plan(*tables, mp, 4), 0, mp,
                         "planned as 4-page runs, run balanced")
    expect_nan_untouched(other_plan(*tables, mp, 0), 0, 2 * mp,
                         "planned for another page bound")
    half = (tables[0][: b // 2 + 1], tables[1], tables[2][: b // 2])
    expect_nan_untouched(other_plan(*half, mp, 0), 0, mp, "planned for half the batch")
    # the matching plan: the oracle's rows and appends
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    plan = pkv.plan(cache, hq, *tables, mp, 0, workspace=ws)
    out, lse = pkv.run(cache, 0, dev[0], plan, spec.sm_scale, k_new=dev[1], v_new=dev[2])
    ro, rl = _oracle_full(cache_host, 0, ld, table, spec.sm_scale)
    act = table.active
    compare(out, lse, ro[act], rl[act], rows=act, what="matching plan")
    got = to_host_u16(cache)
    got[0, 0] = cache_host[0, 0]
    np.testing.assert_array_equal(got, cache_host)


# ------------------------------------------------------------ plan once, run per layer
@pytest.mark.parametrize("idx", [1, 3, 9])
@pytest.mark.parametrize("chunk", [0, 2])
def test_plan_once_run_every_layer(idx, chunk):
    """One pkv_plan serves pkv_run on every layer, decode-only and fused: each
    layer's rows are bit-identical to a standalone pkv_decode /
    pkv_append_decode on the same inputs, and within tolerance of the oracle;
    the cache after the fused runs equals the oracle's appends."""
    hq, hkv, d, ps, lengths, active = SHAPES[idx]
    rng = np.random.default_rng(5000 + idx)
    act = np.ones(len(lengths), bool) if active is None else np.asarray(active, bool)
    table = table_from_lengths(lengths, act, ps, None, rng)
    nl = 3
    lds = [workloads.draw_layer(rng, table, hq, hkv, d, 1.0, stale="nan", unused="nan")
           for _ in range(nl)]
    cache_host = np.stack([ld.cache for ld in lds])
    cache_a = to_dev_u16(cache_host)
    cache_b = to_dev_u16(cache_host)
    tables = table_to_dev(table)
    scale = 1.0 / math.sqrt(d)
    mp = table.max_pages_per_req
    plan = pkv.plan(cache_a, hq, *tables, mp, chunk)
    for rep in range(2):
        for layer in (2, 0, 1):
            ld = lds[layer]
            q, kn, vn = to_dev_u16(ld.q), to_dev_u16(ld.k_new), to_dev_u16(ld.v_new)
            if rep == 0:
                out, lse = pkv.run(cache_a, layer, q, plan, scale, k_new=kn, v_new=vn)
                out2, lse2 = pkv.append_decode(cache_b, layer, kn, vn, q, *tables, scale,
                                               max_pages_per_req=mp, kv_chunk_pages=chunk)
                ro, rl = _oracle_full(cache_host, layer, ld, table, scale)
            else:
                out, lse = pkv.run(cache_a, layer, q, plan, scale)
                out2, lse2 = pkv.decode(cache_b, layer, q, *tables, scale,
                                        max_pages_per_req=mp, kv_chunk_pages=chunk)
                ro, rl = oracle.decode(cache_host, layer, ld.q, table.indptr,
                                       table.indices, table.last_len, scale)
            assert torch.equal(out[act].view(torch.int16), out2[act].view(torch.int16))
            assert torch.equal(lse[act], lse2[act])
            compare(out, lse, ro[act], rl[act], rows=act,
                    what=f"shape {idx} layer {layer} rep {rep}")
    got = to_host_u16(cache_a)
    want = cache_host.copy()
    pages = np.unique(table.indices[table.indices > 0])
    np.testing.assert_array_equal(got[:, pages], want[:, pages])


# ------------------------------------------------------------ workspace reuse
def test_shared_workspace_across_calls():
    """One workspace serves a sequence of balanced and fixed calls of
    different shapes: whatever an earlier call left in it, every call's rows
    equal those of a call given a fresh workspace (bit for bit) and the
    oracle's."""
    cases = []
    for idx in (9, 5, 7):
        hq, hkv, d, ps, lengths, active = SHAPES[idx]
        rng = np.random.default_rng(4000 + idx)
        act = np.ones(len(lengths), bool) if active is None else np.asarray(active, bool)
        table = table_from_lengths(lengths, act, ps, None, rng)
        ld = workloads.draw_layer(rng, table, hq, hkv, d, 1.0)
        cases.append((idx, table, ld, act))
    need = 0
    for idx, table, ld, act in cases:
        hq, hkv, d, ps = SHAPES[idx][:4]
        desc = pkv.CacheDesc(1, table.num_pages, ps, hkv, d)
        for chunk in (0, 1):
            need = max(need, pkv.workspace_size(desc, hq, table.batch,
                                                table.max_pages_per_req, chunk))
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device=DEV)
    for rep in range(2):
        for idx, table, ld, act in cases:
            hq, hkv, d, ps = SHAPES[idx][:4]
            cache = to_dev_u16(ld.cache[None])
            tables = table_to_dev(table)
            q = to_dev_u16(ld.q)
            scale = 1.0 / math.sqrt(d)
            for chunk in (0, 1):
                kw = dict(max_pages_per_req=table.max_pages_per_req, kv_chunk_pages=chunk)
                out, lse = pkv.decode(cache, 0, q, *tables, scale, workspace=ws, **kw)
                out2, lse2 = pkv.decode(cache, 0, q, *tables, scale, **kw)
                assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
                assert torch.equal(lse, lse2)
                ro = oracle.decode(ld.cache[None], 0, ld.q, table.indptr, table.indices,
                                   table.last_len, scale)
                compare(out, lse, ro[0][act], ro[1][act], rows=act,
                        what=f"shape {idx} chunk {chunk} rep {rep}")


@pytest.mark.parametrize("chunk", [0, 1])
def test_batch_above_balanced_limit(chunk):
    """4200 entries (above the 4096 the balanced schedule holds, so the
    default falls back to fixed runs of 16 pages) x 16 KV heads, pages of one
    token, 1 to 24 tokens each; with runs of one 8-token tile most entries
    are split in 2 or 3 and merged."""
    rng = np.random.default_rng(4242)
    batch, hq, hkv, d, ps = 4200, 16, 16, 64, 1
    lengths = rng.integers(1, 25, size=batch)
    act = np.ones(batch, bool)
    table = table_from_lengths(lengths.tolist(), act, ps, None, rng)
    ld = workloads.draw_layer(rng, table, hq, hkv, d, 1.0)
    cache = to_dev_u16(ld.cache[None])
    tables = table_to_dev(table)
    scale = 1.0 / math.sqrt(d)
    out, lse = pkv.decode(cache, 0, to_dev_u16(ld.q), *tables, scale,
                          max_pages_per_req=table.max_pages_per_req, kv_chunk_pages=chunk)
    ro, rl = oracle.decode(ld.cache[None], 0, ld.q, table.indptr, table.indices,
                           table.last_len, scale)
    compare(out, lse, ro, rl, what=f"batch 4200 x 16 heads, chunk {chunk}")
