"""Pins of the fp64 oracle to things other than itself (CPU only).

Each ``pin_*`` function takes a loaded oracle library and raises
AssertionError when the library disagrees with what the mathematics or the
serving pages fix:

* hand-derived closed forms (``tests/golden/closed_form_cases.json``);
* brute force: each entry's pages gathered into contiguous K/V and handed to
  torch's fp64 ``scaled_dot_product_attention`` (its own GQA grouping) and
  ``logsumexp``;
* special cases with textbook answers (one token, zero query, constant V,
  one-hot V, equal keys, huge scores against scipy's softmax);
* invariants (shift of keys, page relabelling, split runs vs unsplit);
* the append's bit copy, checked through a contiguous view of the pages and a
  byte diff of the whole cache;
* for the fused q/k RMSNorm + rotary embedding + KV write: hand-derived bf16
  roundings, the RMSNorm of a constant head in closed form, rotations of unit
  vectors worked by hand, the relative-position and length invariants of the
  rotation, and its KV write checked against the pinned append.

``tests/test_oracle_mutants.py`` re-runs all of them on deliberately broken
copies of the oracle and requires each copy to fail at least one.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
import workloads
from golden_cases import build_case, load_cases
from workloads import bf16_bits, bf16_to_f32, draw_layer, table_from_lengths

NUM_LAYERS, LAYER = 3, 1   # decode a middle layer so the layer index matters


def _case(seed, hq, hkv, d, ps, lengths, active=None, sigma=1.0, stale="random",
          num_pages=None):
    """Random 3-layer cache plus one layer's q/k_new/v_new (pre-append)."""
    rng = np.random.default_rng(seed)
    active = np.ones(len(lengths), bool) if active is None else np.asarray(active)
    table = table_from_lengths(lengths, active, ps, num_pages, rng)
    layers = [draw_layer(rng, table, hq, hkv, d, sigma, stale=stale)
              for _ in range(NUM_LAYERS)]
    cache = np.stack([ld.cache for ld in layers])
    ld = layers[LAYER]
    return table, cache, ld.q, ld.k_new, ld.v_new


def _dense(cache, layer, q, table, sm_scale):
    """Brute force: contiguous K/V per entry, torch SDPA (fp64, enable_gqa)."""
    b, hq, d = q.shape
    hkv = cache.shape[4]
    out = np.zeros((b, hq, d))
    lse = np.zeros((b, hq))
    for i in range(b):
        pages = table.indices[table.indptr[i]:table.indptr[i + 1]]
        n = len(pages)
        length = (n - 1) * table.page_size + int(table.last_len[i])
        kk = bf16_to_f32(cache[layer, pages, 0]).reshape(n * table.page_size, hkv, d)
        vv = bf16_to_f32(cache[layer, pages, 1]).reshape(n * table.page_size, hkv, d)
        kt = torch.from_numpy(kk[:length].astype(np.float64)).permute(1, 0, 2)[None]
        vt = torch.from_numpy(vv[:length].astype(np.float64)).permute(1, 0, 2)[None]
        qt = torch.from_numpy(bf16_to_f32(q[i]).astype(np.float64))[None, :, None, :]
        o = F.scaled_dot_product_attention(qt, kt, vt, scale=sm_scale, enable_gqa=True)
        out[i] = o[0, :, 0, :].numpy()
        krep = kt.repeat_interleave(hq // hkv, dim=1)
        s = torch.matmul(qt, krep.transpose(-1, -2).contiguous()) * sm_scale
        lse[i] = torch.logsumexp(s, dim=-1)[0, :, 0].numpy()
    return out, lse


def _decode(lib, cache, q, table, sm_scale, layer=LAYER, chunk=0):
    return oracle.decode(cache, layer, q, table.indptr, table.indices, table.last_len,
                         sm_scale, chunk, lib=lib)


def _append(lib, cache, k_new, v_new, table, layer=LAYER):
    oracle.append(cache, layer, k_new, v_new, table.indptr, table.indices,
                  table.last_len, lib=lib)


RANDOM_SHAPES = [
    # (hq, hkv, d, page_size, lengths, active)
    (1, 1, 4, 1, [1, 5, 9], None),
    (2, 1, 8, 2, [3, 1, 8, 13], [1, 1, 0, 1]),
    (6, 2, 8, 3, [7, 19, 2], None),
    (7, 1, 64, 16, [40, 1, 17], [1, 0, 1]),
    (14, 2, 64, 16, [33, 16, 5, 64], [1, 1, 0, 1]),
    (4, 4, 8, 2, [11, 6], None),
]


def pin_golden(lib):
    for case in load_cases():
        g = build_case(case)
        cache = g["cache"]
        table = workloads.PageTable(np.zeros(0), np.ones(len(g["last_len"]), bool),
                                    g["indptr"], g["indices"], g["last_len"],
                                    cache.shape[1], cache.shape[3])
        for chunk in (0, 1):
            out, lse = _decode(lib, cache, g["q"], table, g["sm_scale"], layer=0,
                               chunk=chunk)
            m = g["checked"]
            np.testing.assert_allclose(out[m], g["out"][m], rtol=0, atol=1e-12,
                                       err_msg=f"{case['name']} out (chunk={chunk})")
            np.testing.assert_allclose(lse[m], g["lse"][m], rtol=1e-13, atol=1e-12,
                                       err_msg=f"{case['name']} lse (chunk={chunk})")


def pin_dense_sdpa(lib):
    for seed, (hq, hkv, d, ps, lengths, active) in enumerate(RANDOM_SHAPES):
        table, cache, q, kn, vn = _case(100 + seed, hq, hkv, d, ps, lengths, active)
        _append(lib, cache, kn, vn, table)
        scale = 1.0 / math.sqrt(d)
        out, lse = _decode(lib, cache, q, table, scale)
        ref_out, ref_lse = _dense(cache, LAYER, q, table, scale)
        np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-12,
                                   err_msg=f"shape #{seed} out")
        np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12,
                                   err_msg=f"shape #{seed} lse")


def pin_single_token(lib):
    # L = 1: the only weight is 1, so out = v_0 exactly and lse = s_0.
    table, cache, q, kn, vn = _case(7, 6, 2, 64, 16, [1, 1, 1])
    _append(lib, cache, kn, vn, table)
    scale = 0.125
    out, lse = _decode(lib, cache, q, table, scale)
    v = bf16_to_f32(vn).astype(np.float64)
    k = bf16_to_f32(kn).astype(np.float64)
    qf = bf16_to_f32(q).astype(np.float64)
    for hq in range(6):
        np.testing.assert_array_equal(out[:, hq], v[:, hq // 3])
        s0 = np.array([np.dot(qf[b, hq], k[b, hq // 3]) for b in range(3)]) * scale
        np.testing.assert_allclose(lse[:, hq], s0, rtol=1e-14, atol=1e-13)


def pin_zero_query(lib):
    # q = 0: every score is 0, so lse = ln L and out = mean of the L value rows.
    lengths = [1, 7, 33, 18]
    table, cache, q, kn, vn = _case(8, 4, 2, 8, 16, lengths)
    q[:] = 0
    _append(lib, cache, kn, vn, table)
    out, lse = _decode(lib, cache, q, table, 0.3)
    np.testing.assert_allclose(lse, np.log(np.array(lengths, float))[:, None]
                               * np.ones((1, 4)), rtol=0, atol=1e-13)
    for b, length in enumerate(lengths):
        pages = table.indices[table.indptr[b]:table.indptr[b + 1]]
        vv = bf16_to_f32(cache[LAYER, pages, 1]).reshape(-1, 2, 8)[:length]
        mean = vv.astype(np.float64).mean(axis=0)          # [Hkv, D]
        np.testing.assert_allclose(out[b], np.repeat(mean, 2, axis=0), atol=1e-13)


def pin_constant_values(lib):
    # Every V row equal to c: any convex combination returns c.
    table, cache, q, kn, vn = _case(9, 3, 1, 8, 2, [5, 12, 1])
    c = bf16_bits(np.linspace(-2, 2, 8, dtype=np.float32))
    cache[:, :, 1] = c
    vn[:] = c
    _append(lib, cache, kn, vn, table)
    out, _ = _decode(lib, cache, q, table, 0.7)
    np.testing.assert_allclose(out, np.broadcast_to(bf16_to_f32(c), out.shape),
                               rtol=0, atol=1e-14)


def pin_one_hot_values_are_softmax(lib):
    # V_t = e_t (L <= D): out[t] is weight t, which must equal scipy's softmax
    # of the scores, and the weights must sum to 1.
    d, lengths = 64, [20, 64, 3]
    table, cache, q, kn, vn = _case(10, 2, 1, d, 16, lengths)
    _append(lib, cache, kn, vn, table)
    for b, length in enumerate(lengths):
        pages = table.indices[table.indptr[b]:table.indptr[b + 1]]
        for t in range(length):
            cache[LAYER, pages[t // 16], 1, t % 16, 0] = 0
            cache[LAYER, pages[t // 16], 1, t % 16, 0, t] = bf16_bits(np.float32([1]))[0]
    scale = 0.125
    out, lse = _decode(lib, cache, q, table, scale)
    for b, length in enumerate(lengths):
        pages = table.indices[table.indptr[b]:table.indptr[b + 1]]
        kk = bf16_to_f32(cache[LAYER, pages, 0]).reshape(-1, 1, d)[:length, 0]
        for hq in range(2):
            s = kk.astype(np.float64) @ bf16_to_f32(q[b, hq]).astype(np.float64) * scale
            np.testing.assert_allclose(out[b, hq, :length], scipy.special.softmax(s),
                                       rtol=1e-12, atol=1e-15)
            np.testing.assert_allclose(out[b, hq, length:], 0, atol=0)
            assert abs(out[b, hq].sum() - 1.0) < 1e-12
            np.testing.assert_allclose(lse[b, hq], scipy.special.logsumexp(s),
                                       rtol=1e-14, atol=1e-13)


def pin_huge_scores(lib):
    # Scores near 1e3 overflow exp() unless the maximum is subtracted first;
    # scipy's softmax/logsumexp give the exact answer.
    table, cache, q, kn, vn = _case(11, 1, 1, 8, 4, [9])
    pages = table.indices[table.indptr[0]:table.indptr[1]]
    q[:] = 0
    q[0, 0, 0] = bf16_bits(np.float32([1.0]))[0]
    keys = 8192.0 + 64.0 * np.array([0, 3, 1, 4, 1, 5, 2, 6, 5], dtype=np.float32)
    for t, kv in enumerate(keys):
        cache[LAYER, pages[t // 4], 0, t % 4, 0, :] = 0
        cache[LAYER, pages[t // 4], 0, t % 4, 0, 0] = bf16_bits(np.float32([kv]))[0]
    kn[:] = cache[LAYER, pages[2], 0, 0]
    _append(lib, cache, kn, vn, table)
    scale = math.log(2.0) / 8.0
    out, lse = _decode(lib, cache, q, table, scale)
    s = keys.astype(np.float64) * scale
    w = scipy.special.softmax(s)
    vv = bf16_to_f32(cache[LAYER, pages, 1]).reshape(-1, 1, 8)[:9, 0].astype(np.float64)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    np.testing.assert_allclose(out[0, 0], w @ vv, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], scipy.special.logsumexp(s), rtol=1e-14)


def pin_key_shift(lib):
    # Adding c to every key of a head shifts each score row by sm_scale * q.c:
    # out is unchanged and lse moves by that amount.  Small integers keep the
    # shifted keys exact in bf16.
    rng = np.random.default_rng(12)
    table, cache, q, kn, vn = _case(12, 4, 2, 8, 2, [6, 11])
    cache[:, :, 0] = bf16_bits(rng.integers(-4, 5, cache[:, :, 0].shape).astype(np.float32))
    kn[:] = bf16_bits(rng.integers(-4, 5, kn.shape).astype(np.float32))
    q[:] = bf16_bits(rng.integers(-3, 4, q.shape).astype(np.float32))
    _append(lib, cache, kn, vn, table)
    scale = 0.25
    out0, lse0 = _decode(lib, cache, q, table, scale)
    shift = rng.integers(-8, 9, (2, 8)).astype(np.float32)          # [Hkv, D]
    shifted = cache.copy()
    shifted[:, :, 0] = bf16_bits(bf16_to_f32(cache[:, :, 0]) + shift)
    out1, lse1 = _decode(lib, shifted, q, table, scale)
    qf = bf16_to_f32(q).astype(np.float64)
    delta = np.einsum("bhd,hd->bh", qf, np.repeat(shift, 2, axis=0).astype(np.float64))
    np.testing.assert_allclose(out1, out0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse1, lse0 + scale * delta, rtol=0, atol=1e-12)


def pin_split_matches_unsplit(lib):
    table, cache, q, kn, vn = _case(13, 6, 2, 8, 4, [1, 9, 30, 57, 64], [1, 1, 0, 1, 1])
    _append(lib, cache, kn, vn, table)
    out0, lse0 = _decode(lib, cache, q, table, 0.4)
    active = table.active
    for chunk in (1, 2, 3, 5, 16, 100):
        out1, lse1 = _decode(lib, cache, q, table, 0.4, chunk=chunk)
        np.testing.assert_allclose(out1[active], out0[active], rtol=0, atol=1e-12,
                                   err_msg=f"chunk={chunk}")
        np.testing.assert_allclose(lse1[active], lse0[active], rtol=0, atol=1e-12,
                                   err_msg=f"chunk={chunk}")


def pin_page_relabel(lib):
    # Moving every page to another physical slot (same logical content) leaves
    # the result bit-identical.
    table, cache, q, kn, vn = _case(14, 4, 2, 8, 4, [13, 2, 21])
    _append(lib, cache, kn, vn, table)
    out0, lse0 = _decode(lib, cache, q, table, 0.35)
    npg = cache.shape[1]
    perm = np.concatenate([[0], 1 + np.random.default_rng(15).permutation(npg - 1)])
    moved = np.empty_like(cache)
    moved[:, perm] = cache
    t2 = workloads.PageTable(table.lengths, table.active, table.indptr,
                             perm[table.indices].astype(np.int32), table.last_len,
                             table.num_pages, table.page_size)
    out1, lse1 = _decode(lib, moved, q, t2, 0.35)
    np.testing.assert_array_equal(out1, out0)
    np.testing.assert_array_equal(lse1, lse0)


def pin_append_is_last_token(lib):
    # After the append, the new rows are token L-1 of each entry's contiguous
    # K/V, and every other byte of the cache is unchanged except the
    # entries' target slots (page 0 for padding).
    for seed, (hq, hkv, d, ps, lengths, active) in enumerate(RANDOM_SHAPES):
        table, cache, q, kn, vn = _case(200 + seed, hq, hkv, d, ps, lengths, active)
        before = cache.copy()
        _append(lib, cache, kn, vn, table)
        expect = before.copy()
        for b in range(table.batch):
            pages = table.indices[table.indptr[b]:table.indptr[b + 1]]
            n = len(pages)
            length = (n - 1) * ps + int(table.last_len[b])
            kk = cache[LAYER, pages, 0].reshape(n * ps, hkv, d)
            vv = cache[LAYER, pages, 1].reshape(n * ps, hkv, d)
            if table.active[b]:
                np.testing.assert_array_equal(kk[length - 1], kn[b])
                np.testing.assert_array_equal(vv[length - 1], vn[b])
                # the rows before it are the pre-append history
                kb = before[LAYER, pages, 0].reshape(n * ps, hkv, d)
                np.testing.assert_array_equal(kk[:length - 1], kb[:length - 1])
            view_k = expect[LAYER, :, 0].reshape(-1, hkv, d)
            view_v = expect[LAYER, :, 1].reshape(-1, hkv, d)
            row = pages[(length - 1) // ps] * ps + (length - 1) % ps
            view_k[row] = kn[b]
            view_v[row] = vn[b]
            expect[LAYER, :, 0] = view_k.reshape(expect[LAYER, :, 0].shape)
            expect[LAYER, :, 1] = view_v.reshape(expect[LAYER, :, 1].shape)
        # padding entries all write page 0 slot 0; any of them may land last
        pad = ~table.active
        if pad.any():
            candidates = [kn[b] for b in np.flatnonzero(pad)]
            assert any(np.array_equal(cache[LAYER, 0, 0, 0], c) for c in candidates)
            expect[LAYER, 0, :, 0] = cache[LAYER, 0, :, 0]
        np.testing.assert_array_equal(cache, expect, err_msg=f"shape #{seed}")


def pin_append_then_single_token_decode(lib):
    # Append into fresh one-row entries, then decode: out must be v_new, bit
    # for bit once widened, on every layer's own slab.
    table, cache, q, kn, vn = _case(16, 4, 4, 8, 8, [1, 1, 1, 1, 1])
    cache[:] = workloads.BF16_NAN
    for layer in range(NUM_LAYERS):
        _append(lib, cache, kn, vn, table, layer=layer)
        out, _ = _decode(lib, cache, q, table, 1.0, layer=layer)
        np.testing.assert_array_equal(out, bf16_to_f32(vn).astype(np.float64))


# ---- fused q/k RMSNorm + rotary embedding + KV write

def _bf16(x):
    return bf16_bits(np.asarray(x, dtype=np.float32))


def _norm_rope(lib, q, k, v, qw, kw, eps, theta, positions, lengths, ps=4, hkv=None,
               cache=None, seed=0):
    """One layer of a 2-layer cache; returns (q_out, k_out, cache before, cache after)."""
    rng = np.random.default_rng(seed)
    b, hq, d = q.shape
    hkv = k.shape[1]
    table = table_from_lengths(np.asarray(lengths), np.ones(b, bool), ps, None, rng)
    if cache is None:
        cache = bf16_bits(rng.normal(size=(2, table.num_pages, 2, ps, hkv, d)))
    before = cache.copy()
    q_out, k_out = oracle.qk_norm_rope_append(cache, 1, q, k, v, qw, kw, eps, theta,
                                              positions, table.indptr, table.indices,
                                              table.last_len, lib=lib)
    return q_out, k_out, before, cache, table


def pin_bf16_round(lib):
    # Hand-derived roundings: 1 + 2^-8 is halfway between bf16 1.0 and the next
    # value (1 + 2^-7): ties go to the even one; a hair above (below) the
    # midpoint rounds up (down) even though fp32 alone would land on the
    # midpoint; negative values mirror.
    cases = [(1.0, 0x3F80), (3.0, 0x4040), (-2.5, 0xC020),
             (1 + 2.0 ** -8, 0x3F80), (1 + 3 * 2.0 ** -8, 0x3F82),
             (1 + 2.0 ** -8 + 2.0 ** -40, 0x3F81), (1 + 2.0 ** -8 - 2.0 ** -40, 0x3F80),
             (-(1 + 2.0 ** -8 + 2.0 ** -40), 0xBF81), (1 + 2.0 ** -9, 0x3F80),
             (1 + 2.0 ** -7 - 2.0 ** -12, 0x3F81), (0.0, 0x0000)]
    for x, bits in cases:
        got = int(lib.oracle_bf16_round(float(x)))
        assert got == bits, f"bf16({x!r}) = {got:#06x}, want {bits:#06x}"


def pin_rms_norm_closed_form(lib):
    # A head of D equal values c normalises to c / sqrt(c^2 + eps) per element
    # (times the weight); at position 0 the rotation is the identity.
    d, eps = 8, 1e-6
    rng = np.random.default_rng(20)
    cs = bf16_to_f32(_bf16([1e-3, -1e-3, 0.75, -40.0, 3e-4])).astype(np.float64)
    q = np.repeat(_bf16(cs)[None, :, None], d, axis=2)              # [1, 5, D]
    qw = _bf16(rng.uniform(0.5, 2.0, size=d))
    kw = _bf16(rng.uniform(0.5, 2.0, size=d))
    k = q[:, :1]
    q_out, k_out, _, _, _ = _norm_rope(lib, q, k, k, qw, kw, eps, 1e6, [0], [3])
    w_q = bf16_to_f32(qw).astype(np.float64)
    w_k = bf16_to_f32(kw).astype(np.float64)
    want = (cs / np.sqrt(cs * cs + eps))[:, None] * w_q[None, :]
    np.testing.assert_allclose(q_out[0], want, rtol=1e-14, atol=0)
    np.testing.assert_allclose(k_out[0, 0], cs[0] / math.sqrt(cs[0] ** 2 + eps) * w_k,
                               rtol=1e-14, atol=0)


def pin_rope_worked_example(lib):
    # D = 4, eps = 0, unit weights: the unit vector e_j normalises to 2 e_j;
    # then element i pairs with i + 2 and turns by pos * theta^(-i/2).
    d = 4
    q = _bf16(np.eye(d))[None]                                         # [1, 4, 4]
    ones = _bf16(np.ones(d))
    for pos, theta in [(1, 10000.0), (3, 100.0), (-2, 10000.0)]:
        q_out, _, _, _, _ = _norm_rope(lib, q, q[:, :1], q[:, :1], ones, ones, 0.0,
                                       theta, [pos], [2])
        a0, a1 = pos * 1.0, pos * theta ** -0.5
        want = 2 * np.array([[math.cos(a0), 0, math.sin(a0), 0],
                             [0, math.cos(a1), 0, math.sin(a1)],
                             [-math.sin(a0), 0, math.cos(a0), 0],
                             [0, -math.sin(a1), 0, math.cos(a1)]])
        np.testing.assert_allclose(q_out[0], want, rtol=0, atol=1e-14,
                                   err_msg=f"pos {pos} theta {theta}")


def pin_rope_relative_position(lib):
    # <rope(q, m), rope(k, n)> depends on m - n only, and the rotation keeps
    # each pair's length.
    rng = np.random.default_rng(21)
    d, eps, theta = 128, 1e-6, 1e6
    qrow = _bf16(rng.normal(size=(1, 1, d)))
    krow = _bf16(rng.normal(size=(1, 1, d)))
    w = _bf16(rng.uniform(0.5, 1.5, size=d))
    q = np.concatenate([qrow, qrow])
    k = np.concatenate([krow, krow])
    dots = []
    for m, n in [(5000, 1234), (3766, 0), (40000, 36234)]:
        q_out, k_out, _, _, _ = _norm_rope(lib, q, k, k, w, w, eps, theta, [m, n], [3, 7])
        dots.append(float(q_out[0, 0] @ k_out[1, 0]))
        for row, src in [(q_out[0, 0], qrow[0, 0]), (k_out[1, 0], krow[0, 0])]:
            x = bf16_to_f32(src).astype(np.float64)
            y = x / math.sqrt(np.mean(x * x) + eps) * bf16_to_f32(w)
            np.testing.assert_allclose(row[:d // 2] ** 2 + row[d // 2:] ** 2,
                                       y[:d // 2] ** 2 + y[d // 2:] ** 2, rtol=1e-12)
    np.testing.assert_allclose(dots[1:], dots[0], rtol=1e-10)


def pin_norm_rope_write_is_append(lib):
    # The KV write lands where the pinned append puts rows: bf16(k_out) in the
    # K slot, v bit for bit in the V slot, nothing else touched.  The k path
    # is the q path with the k weight.
    rng = np.random.default_rng(22)
    b, hq, hkv, d = 3, 4, 2, 16
    q = _bf16(rng.normal(size=(b, hq, d)))
    k = _bf16(rng.normal(size=(b, hkv, d)))
    v = _bf16(rng.normal(size=(b, hkv, d)))
    qw = _bf16(rng.uniform(0.5, 1.5, size=d))
    kw = _bf16(rng.uniform(0.5, 1.5, size=d))
    pos = [7, 0, 123]
    q_out, k_out, before, after, table = _norm_rope(lib, q, k, v, qw, kw, 1e-6, 1e4, pos,
                                                    [5, 9, 13])
    expect = before.copy()
    oracle.append(expect, 1, oracle.bf16_round(k_out, lib=lib), v, table.indptr,
                  table.indices, table.last_len, lib=lib)
    np.testing.assert_array_equal(after, expect)
    q2, _, _, _, _ = _norm_rope(lib, k, k, v, kw, kw, 1e-6, 1e4, pos, [5, 9, 13])
    np.testing.assert_array_equal(q2, k_out)


def _norm_mrope(lib, q, k, v, qw, kw, eps, theta, positions, axis, lengths, ps=4, seed=0):
    rng = np.random.default_rng(seed)
    b, hq, d = q.shape
    hkv = k.shape[1]
    table = table_from_lengths(np.asarray(lengths), np.ones(b, bool), ps, None, rng)
    cache = bf16_bits(rng.normal(size=(2, table.num_pages, 2, ps, hkv, d)))
    before = cache.copy()
    q_out, k_out = oracle.qk_norm_mrope_append(cache, 1, q, k, v, qw, kw, eps, theta,
                                               np.asarray(positions, np.int32),
                                               np.asarray(axis, np.uint8), table.indptr,
                                               table.indices, table.last_len, lib=lib)
    return q_out, k_out, before, cache, table


def pin_mrope_worked_example(lib):
    # D = 8, eps = 0, unit weights, base 16: the rates 16^(-2i/8) are 1, 1/2,
    # 1/4, 1/8, and e_j normalises to sqrt(8) e_j.  Pair i (elements i, i + 4)
    # turns by the component of (t, h, w) its axis names.
    d = 8
    q = _bf16(np.eye(d))[None]                                         # [1, 8, 8]
    ones = _bf16(np.ones(d))
    for pos, axis in [((3, -2, 5), (0, 1, 2, 0)), ((7, 1, 0), (0, 0, 1, 2)),
                      ((0, 4, 9), (2, 2, 1, 1))]:
        q_out, _, _, _, _ = _norm_mrope(lib, q, q[:, :1], q[:, :1], ones, ones, 0.0, 16.0,
                                        [pos], axis, [2])
        want = np.zeros((d, d))
        for i in range(4):
            a = pos[axis[i]] * 2.0 ** -i
            c, s = math.cos(a), math.sin(a)
            want[i, i], want[i, i + 4] = c, s               # row e_i
            want[i + 4, i], want[i + 4, i + 4] = -s, c      # row e_{i+4}
        np.testing.assert_allclose(q_out[0], math.sqrt(8) * want, rtol=0, atol=1e-14,
                                   err_msg=f"positions {pos} axes {axis}")


def pin_mrope_equal_components_is_rope(lib):
    # with t = h = w the multimodal rotation is the plain one, for any axes
    rng = np.random.default_rng(23)
    b, hq, hkv, d = 3, 4, 2, 64
    q = _bf16(rng.normal(size=(b, hq, d)))
    k = _bf16(rng.normal(size=(b, hkv, d)))
    v = _bf16(rng.normal(size=(b, hkv, d)))
    qw = _bf16(rng.uniform(0.5, 1.5, size=d))
    kw = _bf16(rng.uniform(0.5, 1.5, size=d))
    pos = [11, 0, 4000]
    axis = rng.integers(0, 3, size=d // 2)
    q1, k1, _, c1, _ = _norm_rope(lib, q, k, v, qw, kw, 1e-6, 1e6, pos, [5, 9, 13])
    q3, k3, _, c3, _ = _norm_mrope(lib, q, k, v, qw, kw, 1e-6, 1e6,
                                   [[p, p, p] for p in pos], axis, [5, 9, 13])
    np.testing.assert_array_equal(q3, q1)
    np.testing.assert_array_equal(k3, k1)
    np.testing.assert_array_equal(c3, c1)


def pin_mrope_components_act_on_their_pairs(lib):
    # moving one component changes exactly the pairs that follow it
    rng = np.random.default_rng(24)
    d = 32
    q = _bf16(rng.normal(size=(1, 2, d)))
    k = _bf16(rng.normal(size=(1, 1, d)))
    w = _bf16(rng.uniform(0.5, 1.5, size=d))
    axis = np.array([0] * 6 + [1] * 5 + [2] * 5)
    base, _, _, _, _ = _norm_mrope(lib, q, k, k, w, w, 1e-6, 1e4, [[9, 4, 2]], axis, [3])
    for comp in range(3):
        pos = [9, 4, 2]
        pos[comp] += 3
        moved, _, _, _, _ = _norm_mrope(lib, q, k, k, w, w, 1e-6, 1e4, [pos], axis, [3])
        pairs = np.concatenate([axis, axis]) == comp       # element i and i + D/2
        np.testing.assert_array_equal(moved[..., ~pairs], base[..., ~pairs])
        assert np.all(np.abs(moved[..., pairs] - base[..., pairs]).max(axis=-1) > 1e-3)


# ---- several new rows per entry: append at the last positions, causal attention

def _rows_case(seed, hq, hkv, d, ps, lengths, nrows):
    rng = np.random.default_rng(seed)
    table = table_from_lengths(np.asarray(lengths), np.ones(len(lengths), bool), ps, None,
                               rng)
    cache = bf16_bits(rng.normal(size=(NUM_LAYERS, table.num_pages, 2, ps, hkv, d)))
    qo = np.concatenate([[0], np.cumsum(nrows)]).astype(np.int32)
    rows = int(qo[-1])
    q = bf16_bits(rng.normal(size=(rows, hq, d)))
    kn = bf16_bits(rng.normal(size=(rows, hkv, d)))
    vn = bf16_bits(rng.normal(size=(rows, hkv, d)))
    return table, cache, qo, q, kn, vn


def _gather(cache, layer, table, b, kv):
    """Contiguous [L, Hkv, D] K (kv 0) or V (kv 1) rows of entry b, in token order."""
    pages = table.indices[table.indptr[b]:table.indptr[b + 1]]
    rows = cache[layer, pages, kv].reshape(-1, cache.shape[4], cache.shape[5])
    return rows[:int(table.lengths[b])]


def pin_append_rows_positions(lib):
    # Entry b's new rows land at token positions L - n .. L - 1 of its page
    # list (read back through a contiguous gather); nothing else changes.
    table, cache, qo, q, kn, vn = _rows_case(30, 4, 2, 8, 4, [9, 5, 12, 3], [4, 1, 0, 3])
    before = cache.copy()
    oracle.append_rows(cache, LAYER, kn, vn, qo, table.indptr, table.indices,
                       table.last_len, lib=lib)
    expect = before.copy()
    for b in range(table.batch):
        n, L = int(qo[b + 1] - qo[b]), int(table.lengths[b])
        pages = table.indices[table.indptr[b]:table.indptr[b + 1]]
        for j in range(n):
            t = L - n + j
            expect[LAYER, pages[t // 4], 0, t % 4] = kn[qo[b] + j]
            expect[LAYER, pages[t // 4], 1, t % 4] = vn[qo[b] + j]
        np.testing.assert_array_equal(_gather(cache, LAYER, table, b, 0)[L - n:],
                                      kn[qo[b]:qo[b + 1]])
    np.testing.assert_array_equal(cache, expect)


def pin_prefill_causal_sdpa(lib):
    # Brute force: each entry's K/V gathered contiguous, torch's fp64
    # scaled_dot_product_attention with a bottom-right causal mask (row j
    # sees tokens 0 .. L - n + j) and its own GQA grouping; lse by logsumexp.
    for seed, (hq, hkv, d, ps, lengths, nrows) in enumerate([
            (4, 2, 8, 4, [9, 5, 12, 7], [4, 1, 12, 2]),
            (6, 3, 16, 8, [20, 1, 33], [20, 1, 5]),
            (8, 8, 8, 1, [3, 6], [2, 6])]):
        table, cache, qo, q, kn, vn = _rows_case(31 + seed, hq, hkv, d, ps, lengths, nrows)
        oracle.append_rows(cache, LAYER, kn, vn, qo, table.indptr, table.indices,
                           table.last_len, lib=lib)
        scale = 0.37
        out, lse = oracle.prefill(cache, LAYER, q, qo, table.indptr, table.indices,
                                  table.last_len, scale, lib=lib)
        for b in range(table.batch):
            n, L = int(qo[b + 1] - qo[b]), int(table.lengths[b])
            if n == 0:
                continue
            K = torch.from_numpy(bf16_to_f32(_gather(cache, LAYER, table, b, 0))).double()
            V = torch.from_numpy(bf16_to_f32(_gather(cache, LAYER, table, b, 1))).double()
            Q = torch.from_numpy(bf16_to_f32(q[qo[b]:qo[b + 1]])).double()
            qh, kh, vh = Q.permute(1, 0, 2), K.permute(1, 0, 2), V.permute(1, 0, 2)
            pos = torch.arange(n)[:, None] + (L - n)
            mask = torch.arange(L)[None, :] <= pos                      # [n, L]
            o = F.scaled_dot_product_attention(qh[None], kh[None], vh[None],
                                               attn_mask=mask[None, None], scale=scale,
                                               enable_gqa=True)[0]
            grp = hq // hkv
            s_ = torch.einsum("hnd,hld->hnl", qh, kh.repeat_interleave(grp, 0)) * scale
            s_ = s_.masked_fill(~mask[None], float("-inf"))
            ls = torch.logsumexp(s_, dim=-1)                            # [hq, n]
            np.testing.assert_allclose(out[qo[b]:qo[b + 1]], o.permute(1, 0, 2).numpy(),
                                       rtol=0, atol=1e-12, err_msg=f"case {seed} entry {b}")
            np.testing.assert_allclose(lse[qo[b]:qo[b + 1]], ls.T.numpy(), rtol=0,
                                       atol=1e-12)


def pin_prefill_one_row_is_decode(lib):
    # One new row per entry is a decode step: same cache after the append,
    # same rows as the (separately pinned) decode.
    table, cache, qo, q, kn, vn = _rows_case(35, 6, 2, 8, 4, [9, 5, 12, 1], [1, 1, 1, 1])
    c2 = cache.copy()
    oracle.append_rows(cache, LAYER, kn, vn, qo, table.indptr, table.indices,
                       table.last_len, lib=lib)
    _append(lib, c2, kn, vn, table)
    np.testing.assert_array_equal(cache, c2)
    out, lse = oracle.prefill(cache, LAYER, q, qo, table.indptr, table.indices,
                              table.last_len, 0.5, lib=lib)
    o2, l2 = _decode(lib, cache, q, table, 0.5)
    np.testing.assert_array_equal(out, o2)
    np.testing.assert_array_equal(lse, l2)


PINS = [pin_golden, pin_dense_sdpa, pin_single_token, pin_zero_query,
        pin_constant_values, pin_one_hot_values_are_softmax, pin_huge_scores,
        pin_key_shift, pin_split_matches_unsplit, pin_page_relabel,
        pin_append_is_last_token, pin_append_then_single_token_decode,
        pin_bf16_round, pin_rms_norm_closed_form, pin_rope_worked_example,
        pin_rope_relative_position, pin_norm_rope_write_is_append,
        pin_mrope_worked_example, pin_mrope_equal_components_is_rope,
        pin_mrope_components_act_on_their_pairs,
        pin_append_rows_positions, pin_prefill_causal_sdpa, pin_prefill_one_row_is_decode]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle.load())


def test_decode_rows_matches_decode():
    lib = oracle.load()
    table, cache, q, kn, vn = _case(17, 6, 3, 8, 4, [5, 14, 22])
    _append(lib, cache, kn, vn, table)
    out, lse = _decode(lib, cache, q, table, 0.3, chunk=2)
    rb = np.array([2, 0, 1, 2])
    rh = np.array([5, 0, 3, 1])
    o2, l2 = oracle.decode_rows(cache, LAYER, q, table.indptr, table.indices,
                                table.last_len, 0.3, rb, rh, chunk_pages=2, lib=lib)
    np.testing.assert_array_equal(o2, out[rb, rh])
    np.testing.assert_array_equal(l2, lse[rb, rh])


def test_oracle_rejects_bad_tables():
    lib = oracle.load()
    table, cache, q, kn, vn = _case(18, 2, 1, 8, 4, [5, 6])
    bad = table.last_len.copy()
    bad[1] = 5            # > page_size
    with pytest.raises(ValueError):
        oracle.decode(cache, LAYER, q, table.indptr, table.indices, bad, 1.0, lib=lib)
    with pytest.raises(ValueError):
        oracle.append(cache, LAYER, kn, vn, table.indptr, table.indices, bad, lib=lib)
    with pytest.raises(ValueError):
        oracle.decode(cache, NUM_LAYERS, q, table.indptr, table.indices,
                      table.last_len, 1.0, lib=lib)
