"""Parity of the paged prefill / mixed step (several new rows per entry) with
the fp64 oracle (GPU, through the C ABI).

Bars: the multi-row append bit for bit (the whole cache compared).  Each
output element within half a bf16 step of the fp64 value plus 1e-3 (the
kernel rounds its fp32 result to bf16 once; a row that attends a few tokens
returns values of single V rows, up to about 4.5 at unit variance, whose
rounding alone passes the decode's absolute 1e-2), mean |err| within 2^-8 of
the mean |output| plus 1e-4, lse within 1e-3.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_pkv_amd as pkv
from bench import prefill_parity
from gpu_util import DEV, compare, table_to_dev, to_dev_u16, to_host_u16
from workloads import bf16_bits, bf16_to_f32, table_from_lengths

pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def check_rows(out, lse, ref_out, ref_lse, what):
    got = bf16_to_f32(to_host_u16(out)).astype(np.float64)
    lg = lse.detach().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(lg)), f"{what}: non-finite"
    err = np.abs(got - ref_out)
    steps = err / np.maximum(2.0 ** -7 * np.abs(ref_out), 1e-30)   # in bf16 steps
    # the bars bench.py reports for its mixed step (the mean scales with the
    # outputs' size, as rounding errors do)
    stats = prefill_parity(got, ref_out, lg, ref_lse)
    stats["worst_in_bf16_steps"] = float(steps[err > 1e-3].max(initial=0.0))
    assert stats["pass"], f"{what}: {stats}"
    return stats


def _case(seed, hq, hkv, ps, lengths, nrows, sigma=1.0, d=D):
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths)
    table = table_from_lengths(lengths, np.ones(len(lengths), bool), ps, None, rng)
    cache = bf16_bits((rng.standard_normal((2, table.num_pages, 2, ps, hkv, d),
                                           dtype=np.float32) * sigma))
    qo = np.concatenate([[0], np.cumsum(nrows)]).astype(np.int32)
    rows = int(qo[-1])
    q = bf16_bits(rng.standard_normal((rows, hq, d), dtype=np.float32) * sigma)
    kn = bf16_bits(rng.standard_normal((rows, hkv, d), dtype=np.float32) * sigma)
    vn = bf16_bits(rng.standard_normal((rows, hkv, d), dtype=np.float32) * sigma)
    return table, cache, qo, q, kn, vn


def _run(table, cache, qo, q, kn, vn, scale, append=True, layer=1, maxr=None):
    cache_dev = to_dev_u16(cache)
    tabs = table_to_dev(table)
    qo_dev = torch.from_numpy(qo).to(DEV)
    if maxr is None:
        maxr = int(np.max(np.diff(qo))) if len(qo) > 1 else 1
    out, lse = pkv.prefill(cache_dev, layer, to_dev_u16(q), qo_dev, *tabs, scale,
                           max(maxr, 1), k_new=to_dev_u16(kn) if append else None,
                           v_new=to_dev_u16(vn) if append else None)
    torch.cuda.synchronize()
    host = cache.copy()
    if append:
        oracle.append_rows(host, layer, kn, vn, qo, table.indptr, table.indices,
                           table.last_len)
    ro, rl = oracle.prefill(host, layer, q, qo, table.indptr, table.indices,
                            table.last_len, scale)
    return cache_dev, out, lse, host, ro, rl


CASES = [
    # seed, hq, hkv, ps, lengths, rows per entry
    (1, 32, 8, 16, [300, 40, 17, 1, 64, 129], [300, 1, 5, 1, 16, 0]),     # mixed step
    (2, 8, 8, 16, [50, 33], [50, 33]),                                      # pure prefill, G 1
    (3, 16, 8, 1, [20, 9, 31], [7, 1, 31]),                                 # one-token pages
    (4, 16, 2, 128, [700, 129, 1000], [45, 2, 1]),                          # G 8, 128-token pages
    (5, 24, 8, 16, [17, 16, 15, 33], [17, 1, 15, 32]),                      # G 3, ragged tiles
    (6, 32, 8, 16, [1, 1, 1, 1, 1], [1, 1, 1, 1, 1]),                       # one token each
    # column tiles of 128 (row, head) pairs, taken in pairs (k, T-1-k) by two
    # chains of waves that split the longer tile's tokens and merge
    (7, 16, 4, 16, [512, 200], [512, 150]),                                 # T 16 and 5
    (8, 4, 4, 16, [400, 390], [300, 129]),                                  # G 1: T 3 (middle
                                                                            # tile halved), 2
    (9, 64, 8, 16, [2100, 40], [100, 40]),                                  # G 8, long prefix
    (10, 8, 2, 1, [2500, 70], [96, 70]),                                    # one-token pages,
                                                                            # 80 pages a walk
    (11, 32, 8, 64, [1100, 5, 333], [700, 5, 1]),                           # 64-token pages
]


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("case", CASES, ids=[f"c{c[0]}" for c in CASES])
def test_prefill_matches_oracle(case, d):
    seed, hq, hkv, ps, lengths, nrows = case
    print(f"prefill case {case} head_dim {d}", flush=True)
    table, cache, qo, q, kn, vn = _case(seed, hq, hkv, ps, lengths, nrows, d=d)
    scale = 1.0 / np.sqrt(d)
    cache_dev, out, lse, host, ro, rl = _run(table, cache, qo, q, kn, vn, scale)
    np.testing.assert_array_equal(to_host_u16(cache_dev), host, err_msg="append")
    if qo[-1]:
        check_rows(out, lse, ro, rl, what=f"prefill case {seed}")


def test_prefill_rows_already_in_cache():
    # no k_new / v_new: the rows were appended before (here by the oracle)
    table, cache, qo, q, kn, vn = _case(11, 32, 8, 16, [90, 260, 3], [12, 64, 3])
    oracle.append_rows(cache, 1, kn, vn, qo, table.indptr, table.indices, table.last_len)
    cache_dev, out, lse, host, ro, rl = _run(table, cache, qo, q, kn, vn, 0.09, append=False)
    np.testing.assert_array_equal(to_host_u16(cache_dev), cache)
    check_rows(out, lse, ro, rl, what="no append")


def test_prefill_decode_rows_match_decode():
    # one row per entry is a decode step: the prefill path and the decode path
    # agree within the decode bars on the same cache
    table, cache, qo, q, kn, vn = _case(12, 32, 8, 16, [500, 77, 1024, 9], [1, 1, 1, 1])
    scale = 1.0 / np.sqrt(D)
    cache_dev, out, lse, host, ro, rl = _run(table, cache, qo, q, kn, vn, scale)
    tabs = table_to_dev(table)
    o2, l2 = pkv.decode(cache_dev, 1, to_dev_u16(q), *tabs, scale,
                        max_pages_per_req=table.max_pages_per_req)
    torch.cuda.synchronize()
    compare(out, lse, ro, rl, what="prefill path")
    compare(o2, l2, ro, rl, what="decode path")


def test_prefill_large_scores():
    # sigma 4: scores spread over hundreds of log2 units; the running maximum
    # and the split weights keep every row finite and on the oracle
    table, cache, qo, q, kn, vn = _case(13, 16, 4, 16, [200, 48], [80, 48], sigma=4.0)
    cache_dev, out, lse, host, ro, rl = _run(table, cache, qo, q, kn, vn, 1.0 / np.sqrt(D))
    check_rows(out, lse, ro, rl, what="large scores")


def test_prefill_negative_and_zero_scale():
    # a negative scale flips every score (folded into q as a sign flip); a
    # zero scale weighs every visible token alike
    for scale in (-0.07, 0.0):
        table, cache, qo, q, kn, vn = _case(14, 16, 4, 16, [260, 37], [200, 30])
        cache_dev, out, lse, host, ro, rl = _run(table, cache, qo, q, kn, vn, scale)
        check_rows(out, lse, ro, rl, what=f"scale {scale}")


def test_prefill_rows_past_max_rows():
    # rows past max_q_rows are neither appended nor computed: the cache holds
    # the appended rows of the first 130 rows of each entry and the old
    # values at the positions of the others
    maxr = 130
    table, cache, qo, q, kn, vn = _case(15, 16, 4, 16, [300, 90], [260, 90])
    cache_dev, out, lse, full, ro, rl = _run(table, cache, qo, q, kn, vn, 0.1, maxr=maxr)
    keep = np.concatenate([np.arange(0, maxr), np.arange(260, 350)])
    got_out = bf16_to_f32(to_host_u16(out)).astype(np.float64)[keep]
    got_lse = lse.detach().cpu().numpy().astype(np.float64)[keep]
    stats = prefill_parity(got_out, ro[keep], got_lse, rl[keep])
    assert stats["pass"], stats
    want = cache.copy()
    lengths = np.array([300, 90])
    for e, n in enumerate([260, 90]):
        for j in range(min(n, maxr)):
            pos = lengths[e] - n + j
            page = table.indices[table.indptr[e] + pos // 16]
            want[1, page, :, pos % 16] = full[1, page, :, pos % 16]
    np.testing.assert_array_equal(to_host_u16(cache_dev), want)


# One-call mixed step (pkv_plan_mixed + pkv_mixed_run): decode rows (entries
# with one new row) through the decode's balanced or fixed-run schedule, so a
# long decode row is split over workgroups and merged; prompts through the
# prefill.  Decode rows are held to the decode bars, prompt rows to the
# prefill bars above, the cache bit for bit.
MIXED = [
    # seed, hq, hkv, ps, lengths, rows per entry, fixed run pages (0 balanced)
    (21, 32, 8, 16, [9000, 600, 33, 64, 1, 40], [1, 512, 1, 64, 1, 0], 0),
    (22, 32, 8, 16, [9000, 600, 33, 64, 1, 40], [1, 512, 1, 64, 1, 0], 16),
    (23, 16, 2, 128, [20000, 300, 129, 5000], [1, 200, 1, 1], 0),         # G 8
    (24, 8, 8, 1, [3000, 50, 7], [1, 50, 1], 0),                          # G 1, 1-token pages
    (25, 24, 8, 16, [4000, 3000, 2000, 100], [1, 1, 1, 100], 32),         # G 3, fixed
]


def _mixed(table, cache, qo, q, kn, vn, scale, chunk, append=True, layer=1):
    cache_dev = to_dev_u16(cache)
    tabs = table_to_dev(table)
    qo_dev = torch.from_numpy(qo).to(DEV)
    rows = int(qo[-1])
    maxr = int(np.max(np.diff(qo)))
    pl = pkv.plan_mixed(cache_dev, q.shape[1], qo_dev, *tabs, rows, table.max_pages_per_req,
                        chunk)
    out, lse = pkv.mixed_run(cache_dev, layer, to_dev_u16(q), *tabs, pl, scale, max(maxr, 1),
                             k_new=to_dev_u16(kn) if append else None,
                             v_new=to_dev_u16(vn) if append else None)
    torch.cuda.synchronize()
    return cache_dev, out, lse


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("case", MIXED, ids=[f"m{c[0]}" for c in MIXED])
def test_mixed_step_matches_oracle(case, d):
    seed, hq, hkv, ps, lengths, nrows, chunk = case
    print(f"mixed case {case} head_dim {d}", flush=True)
    table, cache, qo, q, kn, vn = _case(seed, hq, hkv, ps, lengths, nrows, d=d)
    scale = 1.0 / np.sqrt(d)
    cache_dev, out, lse = _mixed(table, cache, qo, q, kn, vn, scale, chunk)
    host = cache.copy()
    oracle.append_rows(host, 1, kn, vn, qo, table.indptr, table.indices, table.last_len)
    ro, rl = oracle.prefill(host, 1, q, qo, table.indptr, table.indices, table.last_len, scale)
    np.testing.assert_array_equal(to_host_u16(cache_dev), host, err_msg="append")
    n = np.diff(qo)
    single = qo[:-1][n == 1]
    multi = np.concatenate([np.arange(qo[e], qo[e + 1]) for e in range(len(n)) if n[e] > 1])
    compare(out, lse, ro[single], rl[single], rows=single, what="decode rows")
    idx = torch.from_numpy(multi).to(DEV)
    check_rows(out[idx], lse[idx], ro[multi], rl[multi], what="prompt rows")


def test_mixed_step_of_decode_rows_is_the_decode():
    # every entry one new row: the mixed plan is the decode's plan and the
    # results match pkv_plan + pkv_run bit for bit
    table, cache, qo, q, kn, vn = _case(26, 32, 8, 16, [7000, 12, 900, 1, 300], [1] * 5)
    scale = 1.0 / np.sqrt(D)
    for chunk in (0, 16):
        cache_dev, out, lse = _mixed(table, cache, qo, q, kn, vn, scale, chunk)
        c2 = to_dev_u16(cache)
        tabs = table_to_dev(table)
        pl = pkv.plan(c2, 32, *tabs, table.max_pages_per_req, chunk)
        o2, l2 = pkv.run(c2, 1, to_dev_u16(q), pl, scale, k_new=to_dev_u16(kn),
                         v_new=to_dev_u16(vn))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_host_u16(cache_dev), to_host_u16(c2))
        np.testing.assert_array_equal(to_host_u16(out), to_host_u16(o2))
        assert torch.equal(lse, l2)


def test_mixed_step_of_prompts_is_the_prefill():
    # no entry with one new row: the decode half has no tiles and the results
    # match pkv_prefill bit for bit
    table, cache, qo, q, kn, vn = _case(27, 16, 4, 16, [300, 45, 64], [200, 45, 2])
    scale = 0.1
    cache_dev, out, lse = _mixed(table, cache, qo, q, kn, vn, scale, 0)
    c2, o2, l2, host, ro, rl = _run(table, cache, qo, q, kn, vn, scale)
    np.testing.assert_array_equal(to_host_u16(cache_dev), to_host_u16(c2))
    np.testing.assert_array_equal(to_host_u16(out), to_host_u16(o2))
    assert torch.equal(lse, l2)
