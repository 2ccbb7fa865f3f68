"""Parity of the fused q/k RMSNorm + rotary embedding + KV write with the fp64
oracle (GPU, through the C ABI).

Bar: every rotated q and k element within half a bf16 step of the fp64 value
(the kernel computes in fp32 and rounds once, so it lands on the correctly
rounded bf16 value or, next to a midpoint, on its neighbour), plus a floor of
2e-6 times the row's RMS for the fp32 rounding of the rotation's two products;
the V slot bit for bit; every other byte of the cache untouched.  Then the
decode of the written cache against the oracle's decode (the decode bars).
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

HALF_STEP = 2.0 ** -8     # half a bf16 step, relative to the value
ROW_FLOOR = 2e-6          # times the row's RMS


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def _check_rows(got_bits, want, what):
    """got_bits: bf16 bits [..., D]; want: fp64 [..., D]."""
    got = bf16_to_f32(got_bits).astype(np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    rms = np.sqrt(np.mean(want * want, axis=-1, keepdims=True))
    tol = HALF_STEP * np.abs(want) + ROW_FLOOR * rms
    err = np.abs(got - want)
    bad = err > tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements out of bound, worst "
                           f"err {err[bad].max():.3g} at |want| {np.abs(want[bad]).max():.3g}")
    same = np.mean(got_bits == oracle.bf16_round(want))
    assert same >= 0.97, f"{what}: only {same:.3f} of elements equal the rounded fp64 value"
    return float(err.max())


def _case(seed, batch, hq, hkv, d, ps, lo, hi, theta, eps, npad=0, pos_max=None):
    rng = np.random.default_rng(seed)
    lengths = rng.integers(lo, hi + 1, size=batch)
    active = np.ones(batch, bool)
    if npad:
        active[rng.choice(batch, size=npad, replace=False)] = False
    table = table_from_lengths(lengths, active, ps, None, rng)
    layers = [draw_layer(rng, table, hq, hkv, d, 1.0) for _ in range(2)]
    cache = np.stack([ld.cache for ld in layers])
    ld = layers[1]
    qw = bf16_bits(rng.uniform(0.5, 1.5, size=d).astype(np.float32))
    kw = bf16_bits(rng.uniform(0.5, 1.5, size=d).astype(np.float32))
    if pos_max is None:
        positions = (table.lengths - 1).astype(np.int32)
        positions[~table.active] = 0
    else:
        positions = rng.integers(0, pos_max + 1, size=batch).astype(np.int32)
    return table, cache, ld, qw, kw, positions


def _run(table, cache, ld, qw, kw, positions, theta, eps, in_place=False, layer=1):
    cache_dev = to_dev_u16(cache)
    tabs = table_to_dev(table)
    q = to_dev_u16(ld.q)
    q_out = q if in_place else None
    out = pkv.qk_norm_rope_append(cache_dev, layer, q, to_dev_u16(ld.k_new),
                                  to_dev_u16(ld.v_new), to_dev_u16(qw), to_dev_u16(kw),
                                  torch.from_numpy(positions).to(DEV), *tabs, eps=eps,
                                  rope_theta=theta, q_out=q_out)
    torch.cuda.synchronize()
    host = cache.copy()
    q_ref, k_ref = oracle.qk_norm_rope_append(host, layer, ld.q, ld.k_new, ld.v_new, qw, kw,
                                              eps, theta, positions, table.indptr,
                                              table.indices, table.last_len)
    return cache_dev, to_host_u16(out), host, q_ref, k_ref


def _slots(table):
    """(page, slot) the append fills, per entry."""
    pages = table.indices[table.indptr[1:] - 1]
    return pages.astype(np.int64), (table.last_len - 1).astype(np.int64)


def _check_all(table, cache_dev, q_got, host, q_ref, k_ref, v_new, what, layer=1):
    act = table.active
    _check_rows(q_got[act], q_ref[act], f"{what} q")
    got_cache = to_host_u16(cache_dev)
    pages, slots = _slots(table)
    # K slots of active entries against the fp64 rotation; V slots and all
    # else bit for bit (padding entries share page 0 slot 0: any one of their
    # rows may remain, so that slot is compared to the candidates)
    k_got = got_cache[layer, pages[act], 0, slots[act]]
    _check_rows(k_got, k_ref[act], f"{what} k")
    mask = np.ones(got_cache.shape, bool)
    mask[layer, pages[act], 0, slots[act]] = False
    if (~act).any():
        # padding entries all write page 0 slot 0 and race there: each V
        # element holds the value of one or another of their rows (the K row
        # next to it is not compared)
        mask[layer, 0, :, 0] = False
        v_pad = got_cache[layer, 0, 1, 0]
        assert np.all(np.any(v_pad[None] == v_new[~act], axis=0)), \
            f"{what}: padding slot holds values of no padding entry"
    np.testing.assert_array_equal(got_cache[mask], host[mask], err_msg=f"{what} cache")


SHAPES = [
    # seed, batch, hq, hkv, d, ps, lo, hi, theta, eps, npad, pos_max
    (1, 4, 14, 2, 64, 16, 1, 256, 1e6, 1e-6, 1, None),
    (2, 7, 8, 8, 128, 16, 1, 300, 1e4, 1e-6, 0, 100000),
    (3, 5, 32, 8, 128, 16, 1, 64, 1e6, 1e-6, 0, 40000),
    (4, 3, 16, 2, 64, 4, 2, 40, 5e5, 1e-5, 0, 7),
    (5, 9, 12, 4, 128, 8, 1, 90, 1e6, 1e-6, 2, None),
    (6, 1, 1, 1, 128, 1, 1, 3, 1e6, 0.0, 0, 0),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"s{s[0]}" for s in SHAPES])
def test_norm_rope_matches_oracle(shape):
    seed, batch, hq, hkv, d, ps, lo, hi, theta, eps, npad, pos_max = shape
    print(f"norm_rope shape {shape}", flush=True)
    table, cache, ld, qw, kw, positions = _case(seed, batch, hq, hkv, d, ps, lo, hi, theta,
                                                eps, npad, pos_max)
    cache_dev, q_got, host, q_ref, k_ref = _run(table, cache, ld, qw, kw, positions, theta,
                                                eps)
    _check_all(table, cache_dev, q_got, host, q_ref, k_ref, ld.v_new, f"shape {seed}")


def test_norm_rope_in_place():
    table, cache, ld, qw, kw, positions = _case(7, 6, 16, 4, 128, 16, 1, 200, 1e6, 1e-6)
    cache_dev, q_got, host, q_ref, k_ref = _run(table, cache, ld, qw, kw, positions, 1e6,
                                                1e-6, in_place=True)
    _check_all(table, cache_dev, q_got, host, q_ref, k_ref, ld.v_new, "in place")


def test_norm_rope_then_decode_config3_shape():
    # Qwen3-4B-like heads (32/8, D 128) at batch 64 with log-uniform lengths:
    # the fused step, then the decode (no append) of the same layer, against
    # the oracle's step and decode on its own bf16-rounded q and cache.
    spec = workloads.CONFIGS[3]
    rng = np.random.default_rng(3001)
    lengths = np.clip(np.rint(np.exp(rng.uniform(np.log(64), np.log(4096), size=64))),
                      64, 4096).astype(np.int64)
    table = table_from_lengths(lengths, np.ones(64, bool), 16, None, rng)
    ld = draw_layer(rng, table, 32, 8, 128, 1.0)
    cache = ld.cache[None]
    qw = bf16_bits(rng.uniform(0.5, 1.5, size=128).astype(np.float32))
    kw = bf16_bits(rng.uniform(0.5, 1.5, size=128).astype(np.float32))
    positions = (table.lengths - 1).astype(np.int32)
    cache_dev, q_got, host, q_ref, k_ref = _run(table, cache, ld, qw, kw, positions, 1e6,
                                                1e-6, layer=0)
    _check_all(table, cache_dev, q_got, host, q_ref, k_ref, ld.v_new, "qwen3-4b shape",
               layer=0)
    tabs = table_to_dev(table)
    q_dev = to_dev_u16(q_got)
    out, lse = pkv.decode(cache_dev, 0, q_dev, *tabs, spec.sm_scale,
                          max_pages_per_req=table.max_pages_per_req)
    torch.cuda.synchronize()
    rows = np.arange(64)
    sel = rng.choice(32, size=4, replace=False)
    rb, rh = np.repeat(rows, len(sel)), np.tile(sel, 64)
    q_bits = oracle.bf16_round(q_ref)
    o_ref, l_ref = oracle.decode_rows(host, 0, q_bits, table.indptr, table.indices,
                                      table.last_len, spec.sm_scale, rb, rh)
    og = out[torch.from_numpy(rb).to(DEV), torch.from_numpy(rh).to(DEV)]
    lg = lse[torch.from_numpy(rb).to(DEV), torch.from_numpy(rh).to(DEV)]
    compare(og, lg, o_ref, l_ref, what="decode after norm_rope")


# ---- multimodal RoPE: a (t, h, w) position per entry, a component per pair

def _axis(kind, d, rng):
    h = d // 2
    if kind == "sections":        # contiguous t / h / w bands, 24 : 20 : 20
        t, hh = h * 24 // 64, h * 20 // 64
        return np.array([0] * t + [1] * hh + [2] * (h - t - hh), np.uint8)
    if kind == "interleaved":
        return (np.arange(h) % 3).astype(np.uint8)
    return rng.integers(0, 3, size=h).astype(np.uint8)


MR_SHAPES = [
    # seed, batch, hq, hkv, d, ps, lo, hi, axes, pos_max, npad
    (31, 5, 16, 4, 128, 16, 1, 200, "sections", 40000, 1),
    (32, 6, 14, 2, 64, 8, 1, 90, "interleaved", 100000, 0),
    (33, 3, 8, 8, 128, 1, 1, 40, "random", 7, 0),
]


@pytest.mark.parametrize("shape", MR_SHAPES, ids=[f"m{s[0]}" for s in MR_SHAPES])
def test_norm_mrope_matches_oracle(shape):
    seed, batch, hq, hkv, d, ps, lo, hi, kind, pos_max, npad = shape
    print(f"norm_mrope shape {shape}", flush=True)
    table, cache, ld, qw, kw, _ = _case(seed, batch, hq, hkv, d, ps, lo, hi, 1e6, 1e-6, npad)
    rng = np.random.default_rng(seed + 100)
    pos3 = rng.integers(0, pos_max + 1, size=(batch, 3)).astype(np.int32)
    axis = _axis(kind, d, rng)
    cache_dev = to_dev_u16(cache)
    tabs = table_to_dev(table)
    q_out = pkv.qk_norm_mrope_append(cache_dev, 1, to_dev_u16(ld.q), to_dev_u16(ld.k_new),
                                     to_dev_u16(ld.v_new), to_dev_u16(qw), to_dev_u16(kw),
                                     torch.from_numpy(pos3).to(DEV), axis, *tabs)
    torch.cuda.synchronize()
    host = cache.copy()
    q_ref, k_ref = oracle.qk_norm_mrope_append(host, 1, ld.q, ld.k_new, ld.v_new, qw, kw,
                                               1e-6, 1e6, pos3, axis, table.indptr,
                                               table.indices, table.last_len)
    _check_all(table, cache_dev, to_host_u16(q_out), host, q_ref, k_ref, ld.v_new,
               f"mrope {seed}")


def test_norm_mrope_equal_components_is_plain_rope():
    # t = h = w: the same angles as the plain kernel, so the same bits
    table, cache, ld, qw, kw, positions = _case(34, 7, 32, 8, 128, 16, 1, 500, 1e6, 1e-6)
    tabs = table_to_dev(table)
    pos3 = np.repeat(positions[:, None], 3, axis=1).astype(np.int32)
    axis = _axis("random", 128, np.random.default_rng(5))
    c1, c2 = to_dev_u16(cache), to_dev_u16(cache)
    args = (to_dev_u16(ld.q), to_dev_u16(ld.k_new), to_dev_u16(ld.v_new), to_dev_u16(qw),
            to_dev_u16(kw))
    q1 = pkv.qk_norm_rope_append(c1, 1, *args, torch.from_numpy(positions).to(DEV), *tabs)
    q2 = pkv.qk_norm_mrope_append(c2, 1, *args, torch.from_numpy(pos3).to(DEV), axis, *tabs)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2)
    assert torch.equal(c1, c2)
