"""The seeded generators draw what the workload recipes say (CPU only)."""
import numpy as np
import pytest

import workloads
from workloads import CONFIGS, CFG4_SWEEP, bf16_bits, bf16_to_f32, make_table


def _check_table(t, spec_ps):
    assert t.indptr[0] == 0 and np.all(np.diff(t.indptr) >= 1)
    assert np.all((t.last_len >= 1) & (t.last_len <= spec_ps))
    n = np.diff(t.indptr)
    np.testing.assert_array_equal((n - 1) * spec_ps + t.last_len, t.lengths)
    real = np.concatenate([t.indices[t.indptr[b]:t.indptr[b + 1]]
                           for b in range(t.batch) if t.active[b]])
    assert np.all(real >= 1) and np.all(real < t.num_pages)
    assert len(np.unique(real)) == len(real), "a page is shared by two entries"
    for b in np.flatnonzero(~t.active):
        assert n[b] == 1 and t.indices[t.indptr[b]] == 0 and t.last_len[b] == 1


@pytest.mark.parametrize("cfg", sorted(CONFIGS))
def test_config_tables(cfg):
    spec = CONFIGS[cfg]
    t = make_table(spec)
    _check_table(t, spec.page_size)
    assert t.batch == spec.batch
    act = t.lengths[t.active]
    assert act.min() >= spec.length_lo and act.max() <= spec.length_hi
    npad = {1: 1, 2: 4, 3: 0, 4: 26, 5: 0, 6: 0}[cfg]
    assert int((~t.active).sum()) == npad
    if spec.num_pages is not None:
        assert t.num_pages == spec.num_pages
    else:   # twice the next power of two at or above (real pages + page 0)
        used = int(np.diff(t.indptr)[t.active].sum())
        p2 = 1
        while p2 < used + 1:
            p2 *= 2
        assert t.num_pages == 2 * p2
    # same seed, same bytes
    t2 = make_table(spec)
    np.testing.assert_array_equal(t.indices, t2.indices)
    np.testing.assert_array_equal(t.lengths, t2.lengths)


def test_cfg6_pairs_and_padded_heads():
    # a session's conditional and unconditional streams have equal lengths;
    # the pool has the sink page plus 1024 pages; drawn heads carry 72 values
    spec = CONFIGS[6]
    t = make_table(spec)
    np.testing.assert_array_equal(t.lengths[0::2], t.lengths[1::2])
    assert t.num_pages == 1025 and t.max_pages_per_req <= 16
    assert abs(spec.sm_scale - 1 / np.sqrt(72)) < 1e-15
    small = workloads.table_from_lengths(t.lengths[:4], np.ones(4, bool), 128, 64,
                                         np.random.default_rng(0))
    ld = workloads.draw_layer(np.random.default_rng(1), small, 16, 16, 128,
                              real_head_dim=72)
    for a in (ld.q, ld.k_new, ld.v_new, ld.cache):
        assert not a[..., 72:].any()
        assert a[..., :72].any()


def test_cfg4_sweep_padding():
    spec = CONFIGS[4]
    pads = [int((~make_table(spec, b).active).sum()) for b in CFG4_SWEEP]
    assert pads == [0, 0, 0, 1, 2, 3, 6, 13, 26]
    for b in CFG4_SWEEP:
        _check_table(make_table(spec, b), 16)


def test_layer_data_deterministic_and_shaped():
    spec = CONFIGS[1]
    t = make_table(spec)
    a = workloads.layer_data(spec, t, 0)
    b = workloads.layer_data(spec, t, 0)
    c = workloads.layer_data(spec, t, 1)
    for x, y in ((a.cache, b.cache), (a.q, b.q), (a.k_new, b.k_new)):
        np.testing.assert_array_equal(x, y)
    assert not np.array_equal(a.q, c.q)
    assert a.cache.shape == (128, 2, 16, 2, 64) and a.q.shape == (4, 14, 64)
    assert a.k_new.shape == a.v_new.shape == (4, 2, 64)
    vals = bf16_to_f32(a.q).astype(np.float64)
    assert abs(vals.std() - 1.0) < 0.05


def test_stale_nan_only_after_history():
    spec = CONFIGS[1]
    t = make_table(spec)
    ld = workloads.layer_data(spec, t, 0, stale="nan", unused="nan")
    for b in np.flatnonzero(t.active):
        pages = t.indices[t.indptr[b]:t.indptr[b + 1]]
        rows = ld.cache[pages].transpose(1, 0, 2, 3, 4).reshape(2, -1, 2, 64)
        hist = int(t.lengths[b]) - 1
        assert not np.any(rows[:, :hist] == workloads.BF16_NAN)
        assert np.all(rows[:, hist:] == workloads.BF16_NAN)


def test_k_offsets_cfg5():
    off = workloads.k_offsets(CONFIGS[5])
    assert off.shape == (8, 128)
    assert 1.6 < off.std() < 2.4
    assert workloads.k_offsets(CONFIGS[3]) is None


def test_bf16_rounding_ties_to_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 1.0 + 2**-9], np.float32)
    got = bf16_to_f32(bf16_bits(x))
    np.testing.assert_array_equal(got, np.array([1.0, 1.0, 1.0 + 2**-6, -2.5, 1.0],
                                                np.float32))


def test_algorithmic_bytes_formula():
    spec = CONFIGS[2]
    t = make_table(spec)
    by = workloads.algorithmic_bytes(t, 24, 8, 128)
    assert by["kv"] == int(t.lengths[t.active].sum()) * 4096
    assert by["total"] > by["decode"] > by["kv"]
