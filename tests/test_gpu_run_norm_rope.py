"""Parity of the decode with the q/k RMSNorm, rotary embedding and append
folded in (pkv_run_qk_norm_rope) with the fp64 oracle (GPU, through the C ABI).

The oracle runs its q/k norm + rotary + KV write step and then decodes its own
bf16-rounded q over its own cache.  Bars: the K slots of active entries within
half a bf16 step of the fp64 rotation plus 2e-6 times the row's RMS (as for
the standalone norm/rotary step), the V slots and every other byte of the
cache bit for bit, the outputs within the decode bars (max |err| 1e-2, mean
1e-3, lse 1e-3).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_pkv_amd as pkv
import workloads
from gpu_util import DEV, compare, table_to_dev, to_dev_u16, to_host_u16
from workloads import bf16_bits, bf16_to_f32, draw_layer, table_from_lengths

pytestmark = pytest.mark.gpu

D = 128
HALF_STEP = 2.0 ** -8     # half a bf16 step, relative to the value
ROW_FLOOR = 2e-6          # times the row's RMS


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def _check_k(got_bits, want, what):
    got = bf16_to_f32(got_bits).astype(np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    rms = np.sqrt(np.mean(want * want, axis=-1, keepdims=True))
    err = np.abs(got - want)
    bad = err > HALF_STEP * np.abs(want) + ROW_FLOOR * rms
    assert not bad.any(), f"{what}: {int(bad.sum())} elements out of bound"
    same = np.mean(got_bits == oracle.bf16_round(want))
    assert same >= 0.97, f"{what}: only {same:.3f} of elements equal the rounded fp64 value"


def _case(seed, batch, hq, hkv, ps, lo, hi, npad=0, pos_max=None, layers=2):
    rng = np.random.default_rng(seed)
    lengths = rng.integers(lo, hi + 1, size=batch)
    active = np.ones(batch, bool)
    if npad:
        active[rng.choice(batch, size=npad, replace=False)] = False
    table = table_from_lengths(lengths, active, ps, None, rng)
    lds = [draw_layer(rng, table, hq, hkv, D, 1.0) for _ in range(layers)]
    cache = np.stack([ld.cache for ld in lds])
    qw = bf16_bits(rng.uniform(0.5, 1.5, size=D).astype(np.float32))
    kw = bf16_bits(rng.uniform(0.5, 1.5, size=D).astype(np.float32))
    if pos_max is None:
        positions = (table.lengths - 1).astype(np.int32)
        positions[~table.active] = 0
    else:
        positions = rng.integers(0, pos_max + 1, size=batch).astype(np.int32)
    return table, cache, lds, qw, kw, positions


def _gpu_run(table, cache, ld, qw, kw, positions, hq, theta, eps, chunk, layer, maxp=None,
             pair_axis=None):
    cache_dev = to_dev_u16(cache)
    tabs = table_to_dev(table)
    maxp = table.max_pages_per_req if maxp is None else maxp
    p = pkv.plan(cache_dev, hq, *tabs, maxp, kv_chunk_pages=chunk)
    out, lse = pkv.run_qk_norm_rope(cache_dev, layer, to_dev_u16(ld.q), p, 1.0 / np.sqrt(D),
                                    to_dev_u16(ld.k_new), to_dev_u16(ld.v_new),
                                    to_dev_u16(qw), to_dev_u16(kw),
                                    torch.from_numpy(positions).to(DEV), eps=eps,
                                    rope_theta=theta, pair_axis=pair_axis)
    torch.cuda.synchronize()
    return cache_dev, out, lse


def _oracle(table, cache, ld, qw, kw, positions, theta, eps, layer, pair_axis=None):
    host = cache.copy()
    if pair_axis is None:
        q_ref, k_ref = oracle.qk_norm_rope_append(host, layer, ld.q, ld.k_new, ld.v_new, qw, kw,
                                                  eps, theta, positions, table.indptr,
                                                  table.indices, table.last_len)
    else:
        q_ref, k_ref = oracle.qk_norm_mrope_append(host, layer, ld.q, ld.k_new, ld.v_new, qw,
                                                   kw, eps, theta, positions, pair_axis,
                                                   table.indptr, table.indices, table.last_len)
    return host, q_ref, k_ref


def _check_cache(table, got_cache, host, k_ref, v_new, layer, what, rows=None):
    act = table.active if rows is None else rows
    pages = table.indices[table.indptr[1:] - 1].astype(np.int64)
    slots = (table.last_len - 1).astype(np.int64)
    _check_k(got_cache[layer, pages[act], 0, slots[act]], k_ref[act], f"{what} k")
    mask = np.ones(got_cache.shape, bool)
    mask[layer, pages[act], 0, slots[act]] = False
    if (~table.active).any():
        # padding entries all write page 0 slot 0 and race there: each V
        # element holds the value of one or another of their rows
        mask[layer, 0, :, 0] = False
        v_pad = got_cache[layer, 0, 1, 0]
        pad = ~table.active
        assert np.all(np.any(v_pad[None] == v_new[pad], axis=0)), \
            f"{what}: padding slot holds values of no padding entry"
    np.testing.assert_array_equal(got_cache[mask], host[mask], err_msg=f"{what} cache")


SHAPES = [
    # seed, batch, hq, hkv, ps, lo, hi, npad, pos_max, chunk
    (1, 6, 32, 8, 16, 1, 700, 1, None, 0),        # G 4, balanced, a padding entry
    (2, 5, 16, 8, 16, 1, 300, 0, 100000, 2),      # G 2, fixed runs, far positions
    (3, 7, 24, 8, 1, 1, 60, 0, None, 0),          # G 3, one-token pages
    (4, 3, 8, 8, 128, 100, 2000, 0, None, 0),     # G 1, 128-token pages, long entries
    (5, 1, 4, 1, 16, 1, 1, 0, 0, 0),              # one token, position 0
    (6, 40, 32, 8, 16, 1, 3000, 3, None, 0),      # many split entries
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"s{s[0]}" for s in SHAPES])
def test_run_norm_rope_matches_oracle(shape):
    seed, batch, hq, hkv, ps, lo, hi, npad, pos_max, chunk = shape
    print(f"run_qk_norm_rope shape {shape}", flush=True)
    theta, eps = (1e4, 1e-5) if seed == 2 else (1e6, 1e-6)
    table, cache, lds, qw, kw, positions = _case(seed, batch, hq, hkv, ps, lo, hi, npad,
                                                 pos_max)
    ld = lds[1]
    cache_dev, out, lse = _gpu_run(table, cache, ld, qw, kw, positions, hq, theta, eps, chunk,
                                   layer=1)
    host, q_ref, k_ref = _oracle(table, cache, ld, qw, kw, positions, theta, eps, layer=1)
    _check_cache(table, to_host_u16(cache_dev), host, k_ref, ld.v_new, 1, f"shape {seed}")
    act = np.flatnonzero(table.active)
    rb, rh = np.repeat(act, hq), np.tile(np.arange(hq), len(act))
    o_ref, l_ref = oracle.decode_rows(host, 1, oracle.bf16_round(q_ref), table.indptr,
                                      table.indices, table.last_len, 1.0 / np.sqrt(D), rb, rh)
    ib, ih = torch.from_numpy(rb).to(DEV), torch.from_numpy(rh).to(DEV)
    compare(out[ib, ih], lse[ib, ih], o_ref, l_ref, what=f"shape {seed}")


def test_run_norm_rope_matches_two_launch_path():
    # the same layer through pkv_qk_norm_rope_append + pkv_run: outputs within
    # the decode bars of each other, K slots within one bf16 step
    table, cache, lds, qw, kw, positions = _case(21, 12, 32, 8, 16, 1, 900, npad=1)
    ld = lds[0]
    cache_dev, out, lse = _gpu_run(table, cache, ld, qw, kw, positions, 32, 1e6, 1e-6, 0,
                                   layer=0)
    cache2 = to_dev_u16(cache)
    tabs = table_to_dev(table)
    qo = pkv.qk_norm_rope_append(cache2, 0, to_dev_u16(ld.q), to_dev_u16(ld.k_new),
                                 to_dev_u16(ld.v_new), to_dev_u16(qw), to_dev_u16(kw),
                                 torch.from_numpy(positions).to(DEV), *tabs)
    p = pkv.plan(cache2, 32, *tabs, table.max_pages_per_req)
    out2, lse2 = pkv.run(cache2, 0, qo, p, 1.0 / np.sqrt(D))
    torch.cuda.synchronize()
    act = torch.from_numpy(table.active).to(DEV)
    o1 = out[act].float()
    o2 = out2[act].float()
    assert float((o1 - o2).abs().max()) <= 1e-2
    assert float((lse[act] - lse2[act]).abs().max()) <= 1e-3
    g1, g2 = to_host_u16(cache_dev), to_host_u16(cache2)
    pages = table.indices[table.indptr[1:] - 1][table.active]
    slots = (table.last_len - 1)[table.active]
    k1 = bf16_to_f32(g1[0, pages, 0, slots]).astype(np.float64)
    k2 = bf16_to_f32(g2[0, pages, 0, slots]).astype(np.float64)
    assert np.all(np.abs(k1 - k2) <= 2.0 ** -7 * np.maximum(np.abs(k1), np.abs(k2)))
    np.testing.assert_array_equal(g1[0, pages, 1, slots], g2[0, pages, 1, slots])


@pytest.mark.parametrize("chunk", [4, 0])
def test_run_norm_rope_over_the_page_bound(chunk):
    # entries over max_pages_per_req get NaN rows and still their transformed
    # k row and their v row in the cache; the other rows stay correct
    table, cache, lds, qw, kw, positions = _case(31, 10, 32, 8, 16, 1, 600)
    n = np.diff(table.indptr)
    bound = int(np.sort(n)[-3])
    ld = lds[1]
    cache_dev, out, lse = _gpu_run(table, cache, ld, qw, kw, positions, 32, 1e6, 1e-6, chunk,
                                   layer=1, maxp=bound)
    host, q_ref, k_ref = _oracle(table, cache, ld, qw, kw, positions, 1e6, 1e-6, layer=1)
    _check_cache(table, to_host_u16(cache_dev), host, k_ref, ld.v_new, 1, "over the bound")
    over = n > bound
    assert over.any() and (~over).any()
    lse_h = lse.cpu().numpy()
    assert np.all(np.isnan(lse_h[over]))
    assert np.all(np.isnan(bf16_to_f32(to_host_u16(out))[over]))
    ok = np.flatnonzero(~over)
    rb, rh = np.repeat(ok, 32), np.tile(np.arange(32), len(ok))
    o_ref, l_ref = oracle.decode_rows(host, 1, oracle.bf16_round(q_ref), table.indptr,
                                      table.indices, table.last_len, 1.0 / np.sqrt(D), rb, rh)
    ib, ih = torch.from_numpy(rb).to(DEV), torch.from_numpy(rh).to(DEV)
    compare(out[ib, ih], lse[ib, ih], o_ref, l_ref, what="under the bound")


def test_run_norm_rope_qwen3_4b_batch64():
    # the benchmarked shape: Qwen3-4B-like heads (32/8, D 128, 16-token pages)
    # at batch 64 with the workload's lengths, sampled rows of every entry
    spec = workloads.CONFIGS[3]
    assert (spec.num_qo_heads, spec.num_kv_heads, spec.head_dim) == (32, 8, 128)
    table = workloads.make_table(spec)
    rng = np.random.default_rng(4001)
    ld = draw_layer(rng, table, 32, 8, 128, spec.sigma)
    cache = ld.cache[None]
    qw = bf16_bits(rng.uniform(0.5, 1.5, size=D).astype(np.float32))
    kw = bf16_bits(rng.uniform(0.5, 1.5, size=D).astype(np.float32))
    positions = (table.lengths - 1).astype(np.int32)
    cache_dev, out, lse = _gpu_run(table, cache, ld, qw, kw, positions, 32, 1e6, 1e-6, 0,
                                   layer=0)
    host, q_ref, k_ref = _oracle(table, cache, ld, qw, kw, positions, 1e6, 1e-6, layer=0)
    _check_cache(table, to_host_u16(cache_dev), host, k_ref, ld.v_new, 0, "qwen3-4b")
    act = np.flatnonzero(table.active)
    sel = rng.choice(32, size=4, replace=False)
    rb, rh = np.repeat(act, len(sel)), np.tile(sel, len(act))
    o_ref, l_ref = oracle.decode_rows(host, 0, oracle.bf16_round(q_ref), table.indptr,
                                      table.indices, table.last_len, spec.sm_scale, rb, rh)
    ib, ih = torch.from_numpy(rb).to(DEV), torch.from_numpy(rh).to(DEV)
    compare(out[ib, ih], lse[ib, ih], o_ref, l_ref, what="qwen3-4b fused norm/rotary")


# Multimodal RoPE folded into the decode (pkv_run_qk_norm_mrope): the
# Qwen3-Omni Thinker's contiguous 24:20:20 sections of the 64 pairs, an
# interleaved map and a random one, against the oracle's multimodal step.
MAPS = {
    "sections": np.array([0] * 24 + [1] * 20 + [2] * 20, np.uint8),
    "interleaved": np.arange(64, dtype=np.uint8) % 3,
    "random": np.random.default_rng(77).integers(0, 3, size=64).astype(np.uint8),
}
MSHAPES = [
    # seed, batch, hq, hkv, ps, lo, hi, npad, chunk
    (41, 9, 32, 8, 16, 1, 900, 1, 0),      # G 4, balanced, a padding entry
    (42, 6, 16, 8, 16, 1, 400, 0, 2),      # G 2, fixed runs
    (43, 30, 32, 8, 16, 1, 3000, 2, 0),    # many split entries
]


def _positions3(rng, table, spread):
    """(t, h, w) per entry: t the last position, h and w up to `spread` apart."""
    t = (table.lengths - 1).astype(np.int64)
    h = t - rng.integers(0, spread + 1, size=len(t))
    w = t - rng.integers(0, spread + 1, size=len(t))
    pos = np.stack([t, np.maximum(h, 0), np.maximum(w, 0)], axis=1).astype(np.int32)
    pos[~table.active] = 0
    return pos


@pytest.mark.parametrize("name", list(MAPS))
@pytest.mark.parametrize("shape", MSHAPES, ids=[f"s{s[0]}" for s in MSHAPES])
def test_run_norm_mrope_matches_oracle(shape, name):
    seed, batch, hq, hkv, ps, lo, hi, npad, chunk = shape
    axis = MAPS[name]
    print(f"run_qk_norm_mrope shape {shape} map {name}", flush=True)
    table, cache, lds, qw, kw, _ = _case(seed, batch, hq, hkv, ps, lo, hi, npad)
    positions = _positions3(np.random.default_rng(seed + 1000), table, 500)
    ld = lds[1]
    cache_dev, out, lse = _gpu_run(table, cache, ld, qw, kw, positions, hq, 1e6, 1e-6, chunk,
                                   layer=1, pair_axis=axis)
    host, q_ref, k_ref = _oracle(table, cache, ld, qw, kw, positions, 1e6, 1e-6, layer=1,
                                 pair_axis=axis)
    _check_cache(table, to_host_u16(cache_dev), host, k_ref, ld.v_new, 1, f"mrope {seed}")
    act = np.flatnonzero(table.active)
    rb, rh = np.repeat(act, hq), np.tile(np.arange(hq), len(act))
    o_ref, l_ref = oracle.decode_rows(host, 1, oracle.bf16_round(q_ref), table.indptr,
                                      table.indices, table.last_len, 1.0 / np.sqrt(D), rb, rh)
    ib, ih = torch.from_numpy(rb).to(DEV), torch.from_numpy(rh).to(DEV)
    compare(out[ib, ih], lse[ib, ih], o_ref, l_ref, what=f"mrope {seed} {name}")


def test_run_norm_mrope_equal_components_is_plain_rope():
    # t = h = w: the multimodal kernel gives the plain folded kernel's bits
    table, cache, lds, qw, kw, positions = _case(44, 12, 32, 8, 16, 1, 1200, npad=1)
    ld = lds[0]
    pos3 = np.repeat(positions[:, None], 3, axis=1)
    c1, o1, l1 = _gpu_run(table, cache, ld, qw, kw, positions, 32, 1e6, 1e-6, 0, layer=0)
    c2, o2, l2 = _gpu_run(table, cache, ld, qw, kw, pos3, 32, 1e6, 1e-6, 0, layer=0,
                          pair_axis=MAPS["random"])
    np.testing.assert_array_equal(to_host_u16(c1), to_host_u16(c2))
    np.testing.assert_array_equal(to_host_u16(o1), to_host_u16(o2))
    assert torch.equal(l1, l2)
