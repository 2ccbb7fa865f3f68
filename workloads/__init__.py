"""Seeded synthetic decode batches for paged-KV attention.

This module only draws inputs: request lengths, padding positions, page
tables, bf16 cache contents, queries and the new K/V rows.  It holds none of
the attention arithmetic, and both the GPU library's tests and the fp64 oracle
read the same arrays from it.

Conventions it draws to (readings of the serving pages, stated once here):

* Cache layout [num_layers, num_pages, 2, page_size, num_kv_heads, head_dim],
  K at index 0 and V at index 1 of the third axis ("Adding a Model",
  vox-serve docs, section 1 "The model code").
* CSR page table per entry: ``indptr[B+1]``, ``indices[indptr[B]]``,
  ``last_len[B]`` in [1, page_size], counted after this step's new row.
* Padding entries (active == 0) list scratch page 0 with one row
  ("Adding a Model", "How a program runs": unused entries point at KV page 0).
  Real pages are a random permutation of [1, num_pages), dealt out in entry
  order, so page 0 is never a real page (the pools on "Supported Models"
  reserve one sink page the same way).
* Before a layer's append, each active entry's pages hold L - 1 prior rows;
  slot L - 1 of the last page (the row the append fills) and the slots after
  it hold stale data from an earlier tenant: random values by default, or NaN
  when ``stale="nan"`` to prove nothing reads them.
* ``N(0, s)`` means standard deviation s; values are drawn in fp32 and rounded
  to bf16 with round-to-nearest-even, so every consumer sees identical bits.

Seeds: tables come from the stream ``[1000 * cfg + 999, B]``, layer data from
``[1000 * cfg + layer, B]``, and per-head K offsets from ``[1000 * cfg + 998]``
(numpy PCG64 via ``default_rng``).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BF16_NAN = np.uint16(0x7FC0)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest, ties to even); return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    u = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to fp32 values."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def _next_pow2(n: int) -> int:
    return 1 << max(0, (int(n) - 1).bit_length())


@dataclass(frozen=True)
class ConfigSpec:
    """Shape and distribution of one synthetic decode workload."""
    cfg: int
    name: str
    num_layers: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    batch: int
    num_padding: int | None        # None: round(0.1 * batch)
    length_dist: str               # "uniform" | "loguniform"
    length_lo: int
    length_hi: int
    sigma: float
    num_pages: int | None          # None: 2 * next_pow2(1 + pages used)
    k_offset_sigma: float = 0.0    # per-KV-head K offset (long-context stress)
    chunk_pages: tuple = ()        # split sizes its parity tests exercise
    description: str = ""
    real_head_dim: int = 0         # > 0: q/k/v carry this many values, zero-padded
    paired: bool = False           # entries come in pairs of equal length

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.real_head_dim or self.head_dim)

    @property
    def group(self) -> int:
        return self.num_qo_heads // self.num_kv_heads

    def padding_for(self, batch: int) -> int:
        if self.num_padding is not None and batch == self.batch:
            return self.num_padding
        return int(round(0.1 * batch)) if self.num_padding is None else 0


CONFIGS = {
    1: ConfigSpec(1, "qwen2_0.5b_like_b4", 1, 14, 2, 64, 16, 4, 1, "uniform", 1, 256,
                  1.0, 128,
                  description="single layer, batch 4 with one padding entry, "
                              "Qwen2-0.5B-like GQA 14/2, head_dim 64"),
    2: ConfigSpec(2, "llama3.2_3b_like_b32", 1, 24, 8, 128, 16, 32, 4, "uniform", 128,
                  2048, 1.0, 8192,
                  description="Llama-3.2-3B-like layer, 24/8 heads, batch 32 "
                              "(4 padding), lengths U[128, 2048]"),
    3: ConfigSpec(3, "qwen3_4b_like_b64_36l", 36, 32, 8, 128, 16, 64, 0, "loguniform",
                  64, 4096, 1.0, None,
                  description="Qwen3-4B-like decode step over 36 layers, 32/8 heads, "
                              "batch 64, lengths log-uniform [64, 4096]"),
    4: ConfigSpec(4, "qwen3_0.6b_like_b256_28l", 28, 16, 8, 128, 16, 256, None,
                  "uniform", 16, 512, 0.5, None,
                  description="Qwen3-0.6B-like, 28 layers, 16/8 heads, batch 256 with "
                              "10% padding, lengths U[16, 512], N(0, 0.5); batch "
                              "sweep 1..256"),
    5: ConfigSpec(5, "qwen3_4b_like_long_b8", 1, 32, 8, 128, 16, 8, 0, "uniform", 16384,
                  32768, 1.0, None, k_offset_sigma=2.0, chunk_pages=(32, 64),
                  description="long-context Qwen3-4B-like layer, batch 8, lengths "
                              "U[16384, 32768], per-head K offsets N(0, 2)"),
    6: ConfigSpec(6, "talker_cfg_pairs_ps128_d72", 1, 16, 16, 128, 128, 64, 0, "uniform",
                  38, 2000, 1.0, 1025, real_head_dim=72, paired=True,
                  description="CFG talker-like layer: 32 sessions x (conditional, "
                              "unconditional) streams of equal length U[38, 2000], 16/16 "
                              "heads of 72 values zero-padded to 128, 128-token pages, "
                              "pool of 1025 pages with sink page 0"),
}

CFG4_SWEEP = (1, 2, 4, 8, 16, 32, 64, 128, 256)


@dataclass
class PageTable:
    """CSR page table of one decode batch (int32 arrays ready for a kernel)."""
    lengths: np.ndarray        # int64 [B]: tokens per entry after the append
    active: np.ndarray         # bool  [B]
    indptr: np.ndarray         # int32 [B+1]
    indices: np.ndarray        # int32 [indptr[-1]]
    last_len: np.ndarray       # int32 [B]
    num_pages: int
    page_size: int
    extra: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return len(self.last_len)

    @property
    def max_pages_per_req(self) -> int:
        return int(np.max(np.diff(self.indptr))) if self.batch else 0


def table_from_lengths(lengths, active, page_size: int, num_pages: int | None,
                       rng: np.random.Generator) -> PageTable:
    """Deal random real pages (from [1, num_pages)) to entries of given lengths.

    Padding entries (active False) get page 0 and one row.
    """
    lengths = np.asarray(lengths, dtype=np.int64).copy()
    active = np.asarray(active, dtype=bool)
    lengths[~active] = 1
    if np.any(lengths < 1):
        raise ValueError("every entry needs at least one token")
    npages = (lengths + page_size - 1) // page_size
    used = int(npages[active].sum())
    if num_pages is None:
        num_pages = 2 * _next_pow2(1 + used)
    if used > num_pages - 1:
        raise ValueError(f"pool of {num_pages} pages cannot hold {used} real pages")
    perm = rng.permutation(np.arange(1, num_pages, dtype=np.int32))
    indptr = np.zeros(len(lengths) + 1, dtype=np.int32)
    indptr[1:] = np.cumsum(npages)
    indices = np.zeros(int(indptr[-1]), dtype=np.int32)
    off = 0
    for b in range(len(lengths)):
        n = int(npages[b])
        if active[b]:
            indices[indptr[b]:indptr[b + 1]] = perm[off:off + n]
            off += n
        else:
            indices[indptr[b]:indptr[b + 1]] = 0
    last_len = (lengths - (npages - 1) * page_size).astype(np.int32)
    return PageTable(lengths, active, indptr, indices, last_len, int(num_pages),
                     page_size)


def make_table(spec: ConfigSpec, batch: int | None = None) -> PageTable:
    """Lengths, padding positions and page permutation of a config (seeded)."""
    batch = spec.batch if batch is None else batch
    rng = np.random.default_rng([1000 * spec.cfg + 999, batch])
    n = (batch + 1) // 2 if spec.paired else batch
    if spec.length_dist == "uniform":
        lengths = rng.integers(spec.length_lo, spec.length_hi + 1, size=n)
    elif spec.length_dist == "loguniform":
        u = rng.uniform(math.log(spec.length_lo), math.log(spec.length_hi), size=n)
        lengths = np.clip(np.rint(np.exp(u)), spec.length_lo, spec.length_hi)
    else:
        raise ValueError(spec.length_dist)
    if spec.paired:   # a session's two streams advance together
        lengths = np.repeat(lengths, 2)[:batch]
    active = np.ones(batch, dtype=bool)
    npad = spec.padding_for(batch)
    if npad:
        active[rng.choice(batch, size=npad, replace=False)] = False
    return table_from_lengths(lengths, active, spec.page_size, spec.num_pages, rng)


def k_offsets(spec: ConfigSpec) -> np.ndarray | None:
    """Per-KV-head K offset vectors [Hkv, D] (fp32), or None."""
    if not spec.k_offset_sigma:
        return None
    rng = np.random.default_rng([1000 * spec.cfg + 998])
    return (rng.standard_normal((spec.num_kv_heads, spec.head_dim), dtype=np.float32)
            * np.float32(spec.k_offset_sigma))


@dataclass
class LayerData:
    """One layer's inputs: the pre-append cache slab and this step's rows."""
    cache: np.ndarray   # uint16 [num_pages, 2, page_size, Hkv, D]
    q: np.ndarray       # uint16 [B, Hq, D]
    k_new: np.ndarray   # uint16 [B, Hkv, D]
    v_new: np.ndarray   # uint16 [B, Hkv, D]


def draw_layer(rng: np.random.Generator, table: PageTable, num_qo_heads: int,
               num_kv_heads: int, head_dim: int, sigma: float = 1.0,
               k_offset: np.ndarray | None = None, stale: str = "random",
               unused: str = "zero", real_head_dim: int = 0) -> LayerData:
    """Draw one layer of a batch described by ``table``.

    Draw order: q, k_new, v_new, then the active entries' pages in table order.
    With ``real_head_dim`` > 0 the values past it in every row (q, k_new,
    v_new, the drawn pages) are zero: heads of that size zero-padded.
    """
    b, ps = table.batch, table.page_size
    sig = np.float32(sigma)

    def normal(shape):
        return rng.standard_normal(shape, dtype=np.float32) * sig

    q = bf16_bits(normal((b, num_qo_heads, head_dim)))
    kn = normal((b, num_kv_heads, head_dim))
    if k_offset is not None:
        kn += k_offset[None]
    k_new = bf16_bits(kn)
    v_new = bf16_bits(normal((b, num_kv_heads, head_dim)))

    shape = (table.num_pages, 2, ps, num_kv_heads, head_dim)
    if unused == "zero":
        cache = np.zeros(shape, dtype=np.uint16)
    elif unused == "nan":
        cache = np.full(shape, BF16_NAN, dtype=np.uint16)
    else:
        raise ValueError(unused)
    pages = np.concatenate([table.indices[table.indptr[i]:table.indptr[i + 1]]
                            for i in range(b) if table.active[i]] or
                           [np.zeros(0, np.int32)])
    if len(pages):
        vals = normal((len(pages), 2, ps, num_kv_heads, head_dim))
        if k_offset is not None:
            vals[:, 0] += k_offset[None, None]
        cache[pages] = bf16_bits(vals)
    if stale == "nan":
        for i in range(b):
            if not table.active[i]:
                continue
            last = table.indices[table.indptr[i + 1] - 1]
            cache[last, :, table.last_len[i] - 1:] = BF16_NAN
    elif stale != "random":
        raise ValueError(stale)
    if real_head_dim:
        for a in (q, k_new, v_new):
            a[..., real_head_dim:] = 0
        if len(pages):
            cache[pages, ..., real_head_dim:] = 0
    return LayerData(cache, q, k_new, v_new)


def layer_data(spec: ConfigSpec, table: PageTable, layer: int, **kw) -> LayerData:
    """Seeded data of ``layer`` for config ``spec`` and its page table."""
    rng = np.random.default_rng([1000 * spec.cfg + layer, table.batch])
    return draw_layer(rng, table, spec.num_qo_heads, spec.num_kv_heads, spec.head_dim,
                      spec.sigma, k_offsets(spec), real_head_dim=spec.real_head_dim, **kw)


def active_pages(table: PageTable) -> np.ndarray:
    """Real pages of the active entries, in table order."""
    parts = [table.indices[table.indptr[i]:table.indptr[i + 1]]
             for i in range(table.batch) if table.active[i]]
    return np.concatenate(parts) if parts else np.zeros(0, np.int32)


def draw_layer_device(cache_layer, table: PageTable, seed, num_qo_heads: int,
                      sigma: float = 1.0, k_offset: np.ndarray | None = None,
                      real_head_dim: int = 0):
    """Fill one layer of a device cache and return device (q, k_new, v_new).

    The big configurations hold gigabytes of K/V, so their bulk values are
    drawn on the GPU with torch's seeded generator instead of numpy.  Same
    recipe as :func:`draw_layer`: N(0, sigma) in fp32, rounded to bf16 (torch
    rounds to nearest even), optional per-KV-head K offset, real pages of the
    active entries filled, other pages left as they are.  ``cache_layer`` is a
    bf16 tensor [num_pages, 2, page_size, Hkv, D]; ``seed`` is an int or a
    list of ints (folded into one 63-bit seed).  ``real_head_dim`` > 0 zeroes
    the values past it, as in :func:`draw_layer`.
    """
    import torch
    dev = cache_layer.device
    _, _, ps, hkv, d = cache_layer.shape
    if isinstance(seed, (list, tuple)):
        seed = int(np.random.SeedSequence(list(seed)).generate_state(1, np.uint64)[0]
                   >> np.uint64(1))
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed))
    b = table.batch

    def normal(shape):
        return torch.randn(shape, generator=gen, device=dev,
                           dtype=torch.float32) * float(sigma)

    off = None if k_offset is None else torch.from_numpy(k_offset).to(dev)
    q = normal((b, num_qo_heads, d)).to(torch.bfloat16)
    kn = normal((b, hkv, d))
    if off is not None:
        kn += off[None]
    k_new = kn.to(torch.bfloat16)
    v_new = normal((b, hkv, d)).to(torch.bfloat16)
    pages = active_pages(table)
    step = max(1, (1 << 27) // (2 * ps * hkv * d))     # ~512 MB of fp32 at a time
    for s in range(0, len(pages), step):
        idx = torch.from_numpy(pages[s:s + step].astype(np.int64)).to(dev)
        vals = normal((len(idx), 2, ps, hkv, d))
        if off is not None:
            vals[:, 0] += off[None, None]
        if real_head_dim:
            vals[..., real_head_dim:] = 0
        cache_layer[idx] = vals.to(torch.bfloat16)
    if real_head_dim:
        for t in (q, k_new, v_new):
            t[..., real_head_dim:] = 0
    return q, k_new, v_new


def algorithmic_bytes(table: PageTable, num_qo_heads: int, num_kv_heads: int,
                      head_dim: int) -> dict:
    """Bytes one layer's append + decode must move (bf16 K/V/q/out, fp32 lse).

    Streamed K/V rows of active entries, q in, out and lse out, the page table,
    and the append's read of the new rows plus its write into the cache.
    """
    b = table.batch
    kv = int(table.lengths[table.active].sum()) * 2 * num_kv_heads * head_dim * 2
    q = b * num_qo_heads * head_dim * 2
    out = b * num_qo_heads * head_dim * 2
    lse = b * num_qo_heads * 4
    ptab = 4 * (b + 1) + 4 * int(table.indptr[-1]) + 4 * b
    app = 2 * (2 * b * num_kv_heads * head_dim * 2)
    # the fused q/k norm + rotary + KV write: q in and out, k and v in and into
    # the cache, the two norm weights, positions and each entry's last-page
    # lookup (two indptr words, one page id, one last-page length)
    norm_rope = 2 * q + app + 2 * head_dim * 2 + 4 * b + 16 * b
    return {"kv": kv, "q": q, "out": out, "lse": lse, "ptab": ptab, "append": app,
            "decode": kv + q + out + lse + ptab, "total": kv + q + out + lse + ptab + app,
            "norm_rope": norm_rope,
            # the decode with the append and the norm/rotary folded in: the
            # fused append's bytes plus the two norm weights and the positions
            "fused_norm_rope": kv + q + out + lse + ptab + app + 2 * head_dim * 2 + 4 * b}
