"""pkv_decode_static (the entry point that allocates nothing: the plan and
partial rows live in the library's own device array) against pkv_decode, the
entry point it varies, on the GPU through the C ABI: two calls in a row, the
second with a smaller input, each bit-identical to pkv_decode on the same
inputs and within the decode bars of the fp64 oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_pkv_amd as pkv
import workloads
from gpu_util import DEV, compare, table_to_dev, to_dev_u16
from workloads import CONFIGS, make_table, table_from_lengths

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def _layer(spec, table, seed):
    rng = np.random.default_rng(seed)
    ld = workloads.draw_layer(rng, table, spec.num_qo_heads, spec.num_kv_heads,
                              spec.head_dim, spec.sigma)
    return ld


def _check(spec, table, ld, chunk, what):
    cache = to_dev_u16(ld.cache[None])
    tabs = table_to_dev(table)
    q = to_dev_u16(ld.q)
    mp = table.max_pages_per_req
    print(f"{what}: batch {table.batch}, chunk {chunk}", flush=True)
    out_s, lse_s = pkv.decode_static(cache, 0, q, *tabs, spec.sm_scale,
                                     max_pages_per_req=mp, kv_chunk_pages=chunk)
    out_w, lse_w = pkv.decode(cache, 0, q, *tabs, spec.sm_scale, max_pages_per_req=mp,
                              kv_chunk_pages=chunk)
    torch.cuda.synchronize()
    act = torch.from_numpy(table.active).to(DEV)
    assert torch.equal(out_s[act].view(torch.int16), out_w[act].view(torch.int16)), what
    assert torch.equal(lse_s[act], lse_w[act]), what
    ro, rl = oracle.decode(ld.cache[None], 0, ld.q, table.indptr, table.indices,
                           table.last_len, spec.sm_scale)
    compare(out_s, lse_s, ro[table.active], rl[table.active], rows=table.active, what=what)


@pytest.mark.parametrize("chunk", [0, 4])
def test_decode_static_matches_decode_twice_second_smaller(chunk):
    # a Llama-3.2-3B-like layer (batch 32), then a smaller input on the same
    # array: the Qwen2-0.5B-like batch of 4 (one padding entry, head_dim 64)
    spec = CONFIGS[2]
    table = make_table(spec)
    _check(spec, table, _layer(spec, table, 71), chunk, "first call, batch 32")
    spec1 = CONFIGS[1]
    table1 = make_table(spec1)
    _check(spec1, table1, _layer(spec1, table1, 72), chunk, "second call, batch 4")


def test_decode_static_long_entries_then_short():
    # many long entries (many split runs and merges), then three short ones
    spec = CONFIGS[2]
    rng = np.random.default_rng(73)
    big = table_from_lengths([3000, 2500, 4000, 1800, 3600, 2900], np.ones(6, bool), 16,
                             None, rng)
    _check(spec, big, _layer(spec, big, 74), 0, "long entries")
    small = table_from_lengths([5, 17, 40], np.ones(3, bool), 16, None, rng)
    _check(spec, small, _layer(spec, small, 75), 0, "short entries")
