"""A whole decode step captured as one HIP graph replays bit for bit like the
eager calls (GPU).

The step is the one the benchmark captures: one ``pkv_plan``, then per layer
the fused append + decode ``pkv_run``, the fused q/k norm + rotary + KV write
followed by a decode-only ``pkv_run``, or the one ``pkv_run_qk_norm_rope``
that does all of it.  The graph is replayed several
times with eager work in between (the cache and the outputs are reset by
ordinary copies and fills), and every replay must reproduce the eager outputs,
LSEs and cache exactly; the eager step itself is checked against the oracle
on sampled rows.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_pkv_amd as pkv
from gpu_util import DEV, compare, table_to_dev, to_dev_u16, to_host_u16
from workloads import bf16_bits, draw_layer, table_from_lengths

pytestmark = pytest.mark.gpu

LAYERS, HQ, HKV, D, PS = 4, 32, 8, 128, 16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def _inputs(seed, batch=24, npad=3):
    rng = np.random.default_rng(seed)
    lengths = rng.integers(1, 700, size=batch)
    active = np.ones(batch, bool)
    active[rng.choice(batch, size=npad, replace=False)] = False
    table = table_from_lengths(lengths, active, PS, None, rng)
    lds = [draw_layer(rng, table, HQ, HKV, D, 1.0) for _ in range(LAYERS)]
    cache = np.stack([ld.cache for ld in lds])
    qw = bf16_bits(rng.uniform(0.5, 1.5, size=(LAYERS, D)).astype(np.float32))
    kw = bf16_bits(rng.uniform(0.5, 1.5, size=(LAYERS, D)).astype(np.float32))
    return table, lds, cache, qw, kw


@pytest.mark.parametrize("mode", ["fused_append", "norm_rope", "run_norm_rope"])
def test_graph_replays_match_eager(mode):
    print(f"graph mode {mode}", flush=True)
    table, lds, cache_host, qw_h, kw_h = _inputs({"fused_append": 41, "norm_rope": 42,
                                                  "run_norm_rope": 43}[mode])
    batch, scale = table.batch, 1.0 / np.sqrt(D)
    maxp = table.max_pages_per_req
    tabs = table_to_dev(table)
    cache0 = to_dev_u16(cache_host)
    Q = [to_dev_u16(ld.q) for ld in lds]
    KN = [to_dev_u16(ld.k_new) for ld in lds]
    VN = [to_dev_u16(ld.v_new) for ld in lds]
    QW, KW = to_dev_u16(qw_h), to_dev_u16(kw_h)
    pos_h = (table.lengths - 1).astype(np.int32)
    pos = torch.from_numpy(pos_h).to(DEV)
    ws = torch.empty(max(pkv.workspace_size(pkv.cache_desc(cache0), HQ, batch, maxp, 0), 256),
                     dtype=torch.uint8, device=DEV)

    def buffers():
        return (torch.empty((LAYERS, batch, HQ, D), dtype=torch.bfloat16, device=DEV),
                torch.empty((LAYERS, batch, HQ), dtype=torch.float32, device=DEV),
                torch.empty((LAYERS, batch, HQ, D), dtype=torch.bfloat16, device=DEV))

    def step(cache, out, lse, qo):
        p = pkv.plan(cache, HQ, *tabs, maxp, workspace=ws)
        for layer in range(LAYERS):
            if mode == "fused_append":
                pkv.run(cache, layer, Q[layer], p, scale, k_new=KN[layer], v_new=VN[layer],
                        out=out[layer], lse=lse[layer])
            elif mode == "run_norm_rope":
                pkv.run_qk_norm_rope(cache, layer, Q[layer], p, scale, KN[layer], VN[layer],
                                     QW[layer], KW[layer], pos, out=out[layer], lse=lse[layer])
            else:
                pkv.qk_norm_rope_append(cache, layer, Q[layer], KN[layer], VN[layer],
                                        QW[layer], KW[layer], pos, *tabs, q_out=qo[layer])
                pkv.run(cache, layer, qo[layer], p, scale, out=out[layer], lse=lse[layer])

    cache_e = cache0.clone()
    out_e, lse_e, qo_e = buffers()
    step(cache_e, out_e, lse_e, qo_e)
    torch.cuda.synchronize()

    cache_g = cache0.clone()
    out_g, lse_g, qo_g = buffers()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(cache_g, out_g, lse_g, qo_g)
    act = torch.from_numpy(table.active).to(DEV)
    for rep in range(3):
        cache_g.copy_(cache0)
        out_g.fill_(0)
        lse_g.fill_(float("nan"))
        qo_g.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g[:, act], out_e[:, act]), f"replay {rep}: out differs"
        assert torch.equal(lse_g[:, act], lse_e[:, act]), f"replay {rep}: lse differs"
        # padding entries all write page 0 slot 0 and race there: each element
        # of that slot holds the value of one or another of their rows
        keep = torch.ones(cache_g.shape[:4], dtype=torch.bool, device=DEV)
        keep[:, 0, :, 0] = False
        assert torch.equal(cache_g[keep], cache_e[keep]), f"replay {rep}: cache differs"
        pad = np.flatnonzero(~table.active)
        for layer in range(LAYERS):
            halves = [(1, lds[layer].v_new)]
            if mode == "fused_append":
                halves.append((0, lds[layer].k_new))
            for kv, rows in halves:
                got = to_host_u16(cache_g[layer, 0, kv, 0])
                assert np.all(np.any(got[None] == rows[pad], axis=0)), \
                    f"replay {rep}: padding slot of layer {layer} holds foreign values"

    # the eager step against the oracle, on sampled rows of every layer
    host = cache_host.copy()
    rng = np.random.default_rng(7)
    rb = np.flatnonzero(table.active)[rng.integers(0, int(table.active.sum()), size=12)]
    rh = rng.integers(0, HQ, size=12)
    for layer in range(LAYERS):
        ld = lds[layer]
        if mode == "fused_append":
            oracle.append(host, layer, ld.k_new, ld.v_new, table.indptr, table.indices,
                          table.last_len)
            q_rows = ld.q
        else:
            q_ref, _ = oracle.qk_norm_rope_append(host, layer, ld.q, ld.k_new, ld.v_new,
                                                  qw_h[layer], kw_h[layer], 1e-6, 1e6, pos_h,
                                                  table.indptr, table.indices,
                                                  table.last_len)
            q_rows = oracle.bf16_round(q_ref)
        o_ref, l_ref = oracle.decode_rows(host, layer, q_rows, table.indptr, table.indices,
                                          table.last_len, scale, rb, rh)
        ib, ih = torch.from_numpy(rb).to(DEV), torch.from_numpy(rh).to(DEV)
        compare(out_e[layer][ib, ih], lse_e[layer][ib, ih], o_ref, l_ref,
                what=f"{mode} layer {layer}")
