"""Loader for ``tests/golden/closed_form_cases.json`` (hand-derived decode cases)."""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

from workloads import bf16_bits

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "closed_form_cases.json")


def load_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def _scale(s):
    if s == "ln2":
        return math.log(2.0)
    if s == "ln2/8":
        return math.log(2.0) / 8.0
    return float(s)


def build_case(case: dict) -> dict:
    """Arrays of one golden case: a one-layer cache holding every token."""
    hq, hkv, d = case["num_qo_heads"], case["num_kv_heads"], case["head_dim"]
    ps, npg = case["page_size"], case["num_pages"]
    pages, lengths = case["pages"], case["lengths"]
    b = len(lengths)
    cache = np.zeros((1, npg, 2, ps, hkv, d), dtype=np.uint16)
    q = np.zeros((b, hq, d), dtype=np.uint16)
    for e, h, dim, val in case["q"]:
        q[e, h, dim] = bf16_bits(np.float32([val]))[0]
    for kv, key in ((0, "k"), (1, "v")):
        for e, t, h, dim, val in case[key]:
            page = pages[e][t // ps]
            cache[0, page, kv, t % ps, h, dim] = bf16_bits(np.float32([val]))[0]
    indptr = np.zeros(b + 1, dtype=np.int32)
    indptr[1:] = np.cumsum([len(p) for p in pages])
    indices = np.array([p for ps_ in pages for p in ps_], dtype=np.int32)
    last_len = np.array([lengths[i] - (len(pages[i]) - 1) * ps for i in range(b)],
                        dtype=np.int32)
    out = np.zeros((b, hq, d), dtype=np.float64)
    for e, h, dim, frac in case["out"]:
        out[e, h, dim] = float(Fraction(frac))
    lse = np.full((b, hq), np.nan)
    for e, h, a, n in case["lse"]:
        lse[e, h] = a * math.log(2.0) + math.log(n)
    checked = np.ones(b, dtype=bool)
    checked[case["ignore"]] = False
    return {"cache": cache, "q": q, "indptr": indptr, "indices": indices,
            "last_len": last_len, "sm_scale": _scale(case["sm_scale"]),
            "out": out, "lse": lse, "checked": checked}
