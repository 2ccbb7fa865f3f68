"""Python binding of libpkv: paged-KV append and decode attention on MI355X.

Argument marshalling only.  Every step of the path runs in the gfx950 kernels
behind the C ABI of ``include/pkv.h``; this module checks tensor dtypes,
devices and shapes, allocates outputs or workspace with torch when the caller
does not pass them, and hands raw device pointers and the current HIP stream
to the library.  There is no fallback: importing this package fails if
``libpkv.so`` has not been built (``python paged_kv_decode_pkv_amd/build.py``).

The calls follow the per-layer API on the vox-serve "Adding a Model" page
(section 1): :func:`append` is ``set_kv_cache(kv_cache, k, v)`` and
:func:`decode` is ``run(q, kv_cache)``, with the step's page table passed in
CSR form (``page_indptr``, ``page_indices``, ``last_page_len``).  A step that
decodes many layers on one page table calls :func:`plan` once and
:func:`run` per layer.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "pkv.h")

PKV_OK = 0
STATUS = {0: "PKV_OK", -1: "PKV_ERR_NULL_PTR", -2: "PKV_ERR_BAD_SHAPE",
          -3: "PKV_ERR_UNSUPPORTED", -4: "PKV_ERR_WORKSPACE", -5: "PKV_ERR_HIP",
          -6: "PKV_ERR_ALIGNMENT", -7: "PKV_ERR_BAD_TABLE"}


class CacheDesc(ctypes.Structure):
    """Mirror of pkv_cache_desc_t."""
    _fields_ = [("num_layers", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32)]


class PkvError(RuntimeError):
    """A libpkv call returned a negative status."""

    def __init__(self, code: int, what: str):
        self.code = code
        extra = ""
        if code == -5:
            self.hip_error = int(lib.pkv_last_hip_error())
            extra = f", hipError_t {self.hip_error}"
        super().__init__(f"{what}: {status_string(code)} ({code}{extra})")


def _hip_runtimes() -> set[str]:
    """Distinct HIP runtime files mapped into this process (Linux)."""
    found = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                path = line.split()[-1]
                if "libamdhip64.so" in os.path.basename(path):
                    found.add(os.path.realpath(path))
    except OSError:
        pass
    return found


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python paged_kv_decode_pkv_amd/build.py` (no fallback path exists)")
    # torch owns the device memory and the streams handed to the library, so
    # libpkv must bind to torch's HIP runtime: importing torch first makes the
    # dynamic loader resolve libpkv's libamdhip64.so.7 to the one torch loaded.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    runtimes = _hip_runtimes()
    if len(runtimes) > 1:
        raise ImportError(
            "two HIP runtimes are loaded in this process "
            f"({sorted(runtimes)}); import torch before anything that loads "
            "another libamdhip64")
    p, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.pkv_append.argtypes = [p, CacheDesc, i32, p, p, p, p, p, i32, p]
    lib.pkv_append.restype = ctypes.c_int
    f32 = ctypes.c_float
    lib.pkv_qk_norm_rope_append.argtypes = [p, CacheDesc, i32, p, i32, p, p, p, p, f32, f32,
                                            p, p, p, p, i32, p, p]
    lib.pkv_qk_norm_rope_append.restype = ctypes.c_int
    lib.pkv_qk_norm_mrope_append.argtypes = [p, CacheDesc, i32, p, i32, p, p, p, p, f32, f32,
                                             p, p, p, p, p, i32, p, p]
    lib.pkv_qk_norm_mrope_append.restype = ctypes.c_int
    lib.pkv_prefill.argtypes = [p, CacheDesc, i32, p, i32, p, p, p, p, p, p, i32, i32, f32,
                                p, p, p]
    lib.pkv_prefill.restype = ctypes.c_int
    lib.pkv_decode_workspace_size.argtypes = [CacheDesc, i32, i32, i32, i32]
    lib.pkv_decode_workspace_size.restype = sz
    lib.pkv_decode.argtypes = [p, CacheDesc, i32, p, i32, p, p, p, i32, ctypes.c_float,
                               p, p, i32, i32, p, sz, p]
    lib.pkv_decode.restype = ctypes.c_int
    lib.pkv_decode_static.argtypes = [p, CacheDesc, i32, p, i32, p, p, p, i32,
                                      ctypes.c_float, p, p, i32, i32, p]
    lib.pkv_decode_static.restype = ctypes.c_int
    lib.pkv_append_decode.argtypes = [p, CacheDesc, i32, p, p, p, i32, p, p, p, i32,
                                      ctypes.c_float, p, p, i32, i32, p, sz, p]
    lib.pkv_append_decode.restype = ctypes.c_int
    lib.pkv_plan.argtypes = [CacheDesc, i32, p, p, p, i32, i32, i32, p, sz, p]
    lib.pkv_plan.restype = ctypes.c_int
    lib.pkv_run.argtypes = [p, CacheDesc, i32, p, p, p, i32, i32, ctypes.c_float, p, p,
                            i32, i32, p, sz, p]
    lib.pkv_run.restype = ctypes.c_int
    lib.pkv_run_qk_norm_rope.argtypes = [p, CacheDesc, i32, p, p, p, i32, i32, p, p, f32, f32,
                                         p, f32, p, p, i32, i32, p, sz, p]
    lib.pkv_run_qk_norm_rope.restype = ctypes.c_int
    lib.pkv_run_qk_norm_mrope.argtypes = [p, CacheDesc, i32, p, p, p, i32, i32, p, p, f32, f32,
                                          p, p, f32, p, p, i32, i32, p, sz, p]
    lib.pkv_run_qk_norm_mrope.restype = ctypes.c_int
    lib.pkv_plan_mixed.argtypes = [CacheDesc, i32, p, p, p, p, i32, i32, i32, i32, p, sz, p]
    lib.pkv_plan_mixed.restype = ctypes.c_int
    lib.pkv_mixed_run.argtypes = [p, CacheDesc, i32, p, i32, p, p, p, p, p, p, i32, i32, i32,
                                  f32, p, p, i32, i32, p, sz, p]
    lib.pkv_mixed_run.restype = ctypes.c_int
    lib.pkv_validate_page_table.argtypes = [p, p, p, i32, i32, i32, i32,
                                            ctypes.POINTER(i32)]
    lib.pkv_validate_page_table.restype = ctypes.c_int
    lib.pkv_last_hip_error.argtypes = []
    lib.pkv_last_hip_error.restype = ctypes.c_int
    lib.pkv_status_string.argtypes = [ctypes.c_int]
    lib.pkv_status_string.restype = ctypes.c_char_p
    return lib


lib = _load()


def declared_functions(header: str = HEADER) -> list[str]:
    """Names of the functions ``include/pkv.h`` declares."""
    text = re.sub(r"/\*.*?\*/", "", open(header).read(), flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*(pkv_[a-z_0-9]+)\s*\(",
                      text, flags=re.M)


def status_string(code: int) -> str:
    return lib.pkv_status_string(int(code)).decode()


def workspace_size(desc: CacheDesc, num_qo_heads: int, batch: int,
                   max_pages_per_req: int, kv_chunk_pages: int = 0) -> int:
    """Bytes of workspace pkv_decode / pkv_append_decode need (0: none)."""
    return int(lib.pkv_decode_workspace_size(desc, num_qo_heads, batch, max_pages_per_req,
                                             kv_chunk_pages))


def cache_desc(kv_cache) -> CacheDesc:
    shape = tuple(kv_cache.shape)
    if len(shape) != 6 or shape[2] != 2:
        raise ValueError("kv_cache must be [num_layers, num_pages, 2, page_size, "
                         f"num_kv_heads, head_dim], got {shape}")
    nl, npg, _, ps, hkv, d = shape
    return CacheDesc(nl, npg, ps, hkv, d)


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream")
                           else int(stream))


def _dev_ptr(t, name, dtype=None, device=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live in GPU memory")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return ctypes.c_void_p(t.data_ptr())


def _tables(kv_cache, page_indptr, page_indices, last_page_len):
    import torch
    dev = kv_cache.device
    return (_dev_ptr(page_indptr, "page_indptr", torch.int32, dev),
            _dev_ptr(page_indices, "page_indices", torch.int32, dev),
            _dev_ptr(last_page_len, "last_page_len", torch.int32, dev))


def append(kv_cache, layer: int, k_new, v_new, page_indptr, page_indices, last_page_len,
           stream=None) -> None:
    """Write k_new / v_new [batch, Hkv, D] (bf16) into each entry's last page slot."""
    import torch
    desc = cache_desc(kv_cache)
    batch = int(last_page_len.shape[0])
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if tuple(t.shape) != (batch, desc.num_kv_heads, desc.head_dim):
            raise ValueError(f"{name} must be [batch, Hkv, D], got {tuple(t.shape)}")
    dev = kv_cache.device
    rc = lib.pkv_append(_dev_ptr(kv_cache, "kv_cache", torch.bfloat16), desc, int(layer),
                        _dev_ptr(k_new, "k_new", torch.bfloat16, dev),
                        _dev_ptr(v_new, "v_new", torch.bfloat16, dev),
                        *_tables(kv_cache, page_indptr, page_indices, last_page_len),
                        batch, _stream(stream))
    if rc != PKV_OK:
        raise PkvError(rc, "pkv_append")


def qk_norm_rope_append(kv_cache, layer: int, q, k_new, v_new, q_norm_weight,
                        k_norm_weight, positions, page_indptr, page_indices, last_page_len,
                        eps: float = 1e-6, rope_theta: float = 1e6, q_out=None,
                        stream=None):
    """Fused per-head RMSNorm of q and k, rotary embedding at ``positions`` and
    the KV write of the rotated k and of v; returns q_out [batch, Hq, D] (bf16,
    allocated when not given; may be ``q`` itself)."""
    import torch
    desc = cache_desc(kv_cache)
    batch = int(last_page_len.shape[0])
    d = desc.head_dim
    if q.dim() != 3 or q.shape[0] != batch or q.shape[2] != d:
        raise ValueError(f"q must be [batch, Hq, {d}], got {tuple(q.shape)}")
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if tuple(t.shape) != (batch, desc.num_kv_heads, d):
            raise ValueError(f"{name} must be [batch, Hkv, D], got {tuple(t.shape)}")
    for name, t in (("q_norm_weight", q_norm_weight), ("k_norm_weight", k_norm_weight)):
        if tuple(t.shape) != (d,):
            raise ValueError(f"{name} must be [{d}], got {tuple(t.shape)}")
    if tuple(positions.shape) != (batch,):
        raise ValueError(f"positions must be [batch], got {tuple(positions.shape)}")
    if q_out is None:
        q_out = torch.empty_like(q)
    dev = kv_cache.device
    rc = lib.pkv_qk_norm_rope_append(
        _dev_ptr(kv_cache, "kv_cache", torch.bfloat16), desc, int(layer),
        _dev_ptr(q, "q", torch.bfloat16, dev), int(q.shape[1]),
        _dev_ptr(k_new, "k_new", torch.bfloat16, dev),
        _dev_ptr(v_new, "v_new", torch.bfloat16, dev),
        _dev_ptr(q_norm_weight, "q_norm_weight", torch.bfloat16, dev),
        _dev_ptr(k_norm_weight, "k_norm_weight", torch.bfloat16, dev),
        float(eps), float(rope_theta), _dev_ptr(positions, "positions", torch.int32, dev),
        *_tables(kv_cache, page_indptr, page_indices, last_page_len), batch,
        _dev_ptr(q_out, "q_out", torch.bfloat16, dev), _stream(stream))
    if rc != PKV_OK:
        raise PkvError(rc, "pkv_qk_norm_rope_append")
    return q_out


def qk_norm_mrope_append(kv_cache, layer: int, q, k_new, v_new, q_norm_weight,
                         k_norm_weight, positions, pair_axis, page_indptr, page_indices,
                         last_page_len, eps: float = 1e-6, rope_theta: float = 1e6,
                         q_out=None, stream=None):
    """:func:`qk_norm_rope_append` with multimodal RoPE: positions [batch, 3]
    int32 on the device, pair_axis a host sequence of head_dim/2 values in
    {0, 1, 2} (the position component each rotary pair follows)."""
    import torch
    desc = cache_desc(kv_cache)
    batch = int(last_page_len.shape[0])
    d = desc.head_dim
    if q.dim() != 3 or q.shape[0] != batch or q.shape[2] != d:
        raise ValueError(f"q must be [batch, Hq, {d}], got {tuple(q.shape)}")
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if tuple(t.shape) != (batch, desc.num_kv_heads, d):
            raise ValueError(f"{name} must be [batch, Hkv, D], got {tuple(t.shape)}")
    for name, t in (("q_norm_weight", q_norm_weight), ("k_norm_weight", k_norm_weight)):
        if tuple(t.shape) != (d,):
            raise ValueError(f"{name} must be [{d}], got {tuple(t.shape)}")
    if tuple(positions.shape) != (batch, 3) or not positions.is_contiguous():
        raise ValueError(f"positions must be contiguous [batch, 3], got {tuple(positions.shape)}")
    axis = np.ascontiguousarray(pair_axis, dtype=np.uint8)
    if axis.shape != (d // 2,):
        raise ValueError(f"pair_axis must hold {d // 2} values")
    if q_out is None:
        q_out = torch.empty_like(q)
    dev = kv_cache.device
    rc = lib.pkv_qk_norm_mrope_append(
        _dev_ptr(kv_cache, "kv_cache", torch.bfloat16), desc, int(layer),
        _dev_ptr(q, "q", torch.bfloat16, dev), int(q.shape[1]),
        _dev_ptr(k_new, "k_new", torch.bfloat16, dev),
        _dev_ptr(v_new, "v_new", torch.bfloat16, dev),
        _dev_ptr(q_norm_weight, "q_norm_weight", torch.bfloat16, dev),
        _dev_ptr(k_norm_weight, "k_norm_weight", torch.bfloat16, dev),
        float(eps), float(rope_theta), _dev_ptr(positions, "positions", torch.int32, dev),
        axis.ctypes.data_as(ctypes.c_void_p),
        *_tables(kv_cache, page_indptr, page_indices, last_page_len), batch,
        _dev_ptr(q_out, "q_out", torch.bfloat16, dev), _stream(stream))
    if rc != PKV_OK:
        raise PkvError(rc, "pkv_qk_norm_mrope_append")
    return q_out


def prefill(kv_cache, layer: int, q, qo_indptr, page_indptr, page_indices, last_page_len,
            sm_scale: float, max_q_rows: int, k_new=None, v_new=None, out=None, lse=None,
            with_lse: bool = True, stream=None):
    """Several new rows per entry (qo_indptr): optional append of k_new/v_new
    [rows, Hkv, D] at each entry's last positions, then the causal attention
    of every row; returns (out [rows, Hq, D] bf16, lse [rows, Hq] fp32 or None)."""
    import torch
    desc = cache_desc(kv_cache)
    batch = int(last_page_len.shape[0])
    if q.dim() != 3 or q.shape[2] != desc.head_dim:
        raise ValueError(f"q must be [rows, Hq, {desc.head_dim}], got {tuple(q.shape)}")
    rows, hq = int(q.shape[0]), int(q.shape[1])
    if tuple(qo_indptr.shape) != (batch + 1,):
        raise ValueError("qo_indptr must be [batch + 1]")
    append = k_new is not None or v_new is not None
    if append:
        for name, t in (("k_new", k_new), ("v_new", v_new)):
            if t is None or tuple(t.shape) != (rows, desc.num_kv_heads, desc.head_dim):
                raise ValueError(f"{name} must be [rows, Hkv, D]")
    dev = kv_cache.device
    if out is None:
        out = torch.empty_like(q)
    if lse is None and with_lse:
        lse = torch.empty((rows, hq), dtype=torch.float32, device=dev)
    null = ctypes.c_void_p(0)
    rc = lib.pkv_prefill(_dev_ptr(kv_cache, "kv_cache", torch.bfloat16), desc, int(layer),
                         _dev_ptr(q, "q", torch.bfloat16, dev), hq,
                         _dev_ptr(qo_indptr, "qo_indptr", torch.int32, dev),
                         _dev_ptr(k_new, "k_new", torch.bfloat16, dev) if append else null,
                         _dev_ptr(v_new, "v_new", torch.bfloat16, dev) if append else null,
                         *_tables(kv_cache, page_indptr, page_indices, last_page_len), batch,
                         int(max_q_rows), float(sm_scale),
                         _dev_ptr(out, "out", torch.bfloat16, dev),
                         null if lse is None else _dev_ptr(lse, "lse", torch.float32, dev),
                         _stream(stream))
    if rc != PKV_OK:
        raise PkvError(rc, "pkv_prefill")
    return out, lse


def _decode_outputs(kv_cache, q, out, lse, with_lse, workspace, max_pages_per_req,
                    kv_chunk_pages):
    import torch
    desc = cache_desc(kv_cache)
    if q.dim() != 3 or q.shape[2] != desc.head_dim:
        raise ValueError(f"q must be [batch, Hq, {desc.head_dim}], got {tuple(q.shape)}")
    batch, hq = int(q.shape[0]), int(q.shape[1])
    dev = kv_cache.device
    if out is None:
        out = torch.empty((batch, hq, desc.head_dim), dtype=torch.bfloat16, device=dev)
    if lse is None and with_lse:
        lse = torch.empty((batch, hq), dtype=torch.float32, device=dev)
    if tuple(out.shape) != (batch, hq, desc.head_dim):
        raise ValueError("out must match q")
    if lse is not None and tuple(lse.shape) != (batch, hq):
        raise ValueError("lse must be [batch, Hq]")
    need = workspace_size(desc, hq, batch, max_pages_per_req, kv_chunk_pages)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr = ctypes.c_void_p(0) if workspace is None else _dev_ptr(workspace, "workspace",
                                                                   device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lse_ptr = ctypes.c_void_p(0) if lse is None else _dev_ptr(lse, "lse", torch.float32,
                                                              dev)
    return desc, batch, hq, out, lse, lse_ptr, ws_ptr, ws_bytes


def decode(kv_cache, layer: int, q, page_indptr, page_indices, last_page_len,
           sm_scale: float, max_pages_per_req: int, kv_chunk_pages: int = 0, out=None,
           lse=None, with_lse: bool = True, workspace=None, stream=None):
    """Attention of one query row per entry over its pages; returns (out, lse).

    ``q`` is bf16 [batch, Hq, D]; ``out`` (bf16, same shape) and ``lse`` (fp32
    [batch, Hq], natural log) are allocated when not given; ``lse`` is None
    when ``with_lse`` is False and none is passed.  ``max_pages_per_req`` is
    the host-side bound on any entry's page count.  ``kv_chunk_pages`` 0 shares
    the batch's tokens evenly over the GPU; > 0 cuts each entry into runs of
    that many pages, which makes every row independent of the rest of the
    batch, bit for bit.
    """
    import torch
    desc, batch, hq, out, lse, lse_ptr, ws_ptr, ws_bytes = _decode_outputs(
        kv_cache, q, out, lse, with_lse, workspace, max_pages_per_req, kv_chunk_pages)
    dev = kv_cache.device
    rc = lib.pkv_decode(_dev_ptr(kv_cache, "kv_cache", torch.bfloat16), desc, int(layer),
                        _dev_ptr(q, "q", torch.bfloat16, dev), hq,
                        *_tables(kv_cache, page_indptr, page_indices, last_page_len),
                        batch, float(sm_scale),
                        _dev_ptr(out, "out", torch.bfloat16, dev), lse_ptr,
                        int(max_pages_per_req), int(kv_chunk_pages), ws_ptr, ws_bytes,
                        _stream(stream))
    if rc != PKV_OK:
        raise PkvError(rc, "pkv_decode")
    return out, lse


def decode_static(kv_cache, layer: int, q, page_indptr, page_indices, last_page_len,
                  sm_scale: float, max_pages_per_req: int, kv_chunk_pages: int = 0,
                  out=None, lse=None, with_lse: bool = True, stream=None):
    """:func:`decode` through pkv_decode_static: no workspace, the plan and
    partial rows in the library's own 16 MiB device array (callers that
    cannot allocate; ``out`` and ``lse`` must then be passed in)."""
    import torch
    desc = cache_desc(kv_cache)
    if q.dim() != 3 or q.shape[2] != desc.head_dim:
        raise ValueError(f"q must be [batch, Hq, {desc.head_dim}], got {tuple(q.shape)}")
    batch, hq = int(q.shape[0]), int(q.shape[1])
    dev = kv_cache.device
    if out is None:
        out = torch.empty((batch, hq, desc.head_dim), dtype=torch.bfloat16, device=dev)
    if lse is None and with_lse:
        lse = torch.empty((batch, hq), dtype=torch.float32, device=dev)
    lse_ptr = ctypes.c_void_p(0) if lse is None else _dev_ptr(lse, "lse", torch.float32, dev)
    rc = lib.pkv_decode_static(_dev_ptr(kv_cache, "kv_cache", torch.bfloat16), desc,
                               int(layer), _dev_ptr(q, "q", torch.bfloat16, dev), hq,
                               *_tables(kv_cache, page_indptr, page_indices, last_page_len),
                               batch, float(sm_scale),
                               _dev_ptr(out, "out", torch.bfloat16, dev), lse_ptr,
                               int(max_pages_per_req), int(kv_chunk_pages), _stream(stream))
    if rc != PKV_OK:
        raise PkvError(rc, "pkv_decode_static")
    return out, lse


def append_decode(kv_cache, layer: int, k_new, v_new, q, page_indptr, page_indices,
                  last_page_len, sm_scale: float, max_pages_per_req: int,
                  kv_chunk_pages: int = 0, out=None, lse=None, with_lse: bool = True,
                  workspace=None, stream=None):
    """:func:`append` then :func:`decode` of one layer in a single pass."""
    import torch
    desc, batch, hq, out, lse, lse_ptr, ws_ptr, ws_bytes = _decode_outputs(
        kv_cache, q, out, lse, with_lse, workspace, max_pages_per_req, kv_chunk_pages)
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if tuple(t.shape) != (batch, desc.num_kv_heads, desc.head_dim):
            raise ValueError(f"{name} must be [batch, Hkv, D], got {tuple(t.shape)}")
    dev = kv_cache.device
    rc = lib.pkv_append_decode(_dev_ptr(kv_cache, "kv_cache", torch.bfloat16), desc,
                               int(layer), _dev_ptr(k_new, "k_new", torch.bfloat16, dev),
                               _dev_ptr(v_new, "v_new", torch.bfloat16, dev),
                               _dev_ptr(q, "q", torch.bfloat16, dev), hq,
                               *_tables(kv_cache, page_indptr, page_indices, last_page_len),
                               batch, float(sm_scale),
                               _dev_ptr(out, "out", torch.bfloat16, dev), lse_ptr,
                               int(max_pages_per_req), int(kv_chunk_pages), ws_ptr,
                               ws_bytes, _stream(stream))
    if rc != PKV_OK:
        raise PkvError(rc, "pkv_append_decode")
    return out, lse


class DecodePlan:
    """A step's decode schedule (pkv_plan) in its workspace, with the shape
    arguments every :func:`run` on it repeats."""

    def __init__(self, workspace, batch, num_qo_heads, max_pages_per_req, kv_chunk_pages):
        self.workspace = workspace
        self.batch = batch
        self.num_qo_heads = num_qo_heads
        self.max_pages_per_req = max_pages_per_req
        self.kv_chunk_pages = kv_chunk_pages


def plan(kv_cache, num_qo_heads: int, page_indptr, page_indices, last_page_len,
         max_pages_per_req: int, kv_chunk_pages: int = 0, workspace=None,
         stream=None) -> DecodePlan:
    """Walk the step's page table once (pkv_plan); returns the plan for :func:`run`."""
    import torch
    desc = cache_desc(kv_cache)
    batch = int(last_page_len.shape[0])
    dev = kv_cache.device
    need = workspace_size(desc, num_qo_heads, batch, max_pages_per_req, kv_chunk_pages)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    rc = lib.pkv_plan(desc, int(num_qo_heads),
                      *_tables(kv_cache, page_indptr, page_indices, last_page_len), batch,
                      int(max_pages_per_req), int(kv_chunk_pages),
                      _dev_ptr(workspace, "workspace", device=dev),
                      workspace.numel() * workspace.element_size(), _stream(stream))
    if rc != PKV_OK:
        raise PkvError(rc, "pkv_plan")
    return DecodePlan(workspace, batch, int(num_qo_heads), int(max_pages_per_req),
                      int(kv_chunk_pages))


def run(kv_cache, layer: int, q, plan_: DecodePlan, sm_scale: float, k_new=None,
        v_new=None, out=None, lse=None, with_lse: bool = True, stream=None):
    """Decode one layer on a plan (pkv_run); with k_new / v_new also the append."""
    import torch
    desc = cache_desc(kv_cache)
    if q.dim() != 3 or q.shape[0] != plan_.batch or q.shape[1] != plan_.num_qo_heads:
        raise ValueError("q must be [batch, Hq, D] of the plan")
    batch, hq = plan_.batch, plan_.num_qo_heads
    dev = kv_cache.device
    if out is None:
        out = torch.empty((batch, hq, desc.head_dim), dtype=torch.bfloat16, device=dev)
    if lse is None and with_lse:
        lse = torch.empty((batch, hq), dtype=torch.float32, device=dev)
    fused = k_new is not None or v_new is not None
    if fused:
        for name, t in (("k_new", k_new), ("v_new", v_new)):
            if t is None or tuple(t.shape) != (batch, desc.num_kv_heads, desc.head_dim):
                raise ValueError(f"{name} must be [batch, Hkv, D]")
    null = ctypes.c_void_p(0)
    ws = plan_.workspace
    rc = lib.pkv_run(_dev_ptr(kv_cache, "kv_cache", torch.bfloat16), desc, int(layer),
                     _dev_ptr(k_new, "k_new", torch.bfloat16, dev) if fused else null,
                     _dev_ptr(v_new, "v_new", torch.bfloat16, dev) if fused else null,
                     _dev_ptr(q, "q", torch.bfloat16, dev), hq, batch, float(sm_scale),
                     _dev_ptr(out, "out", torch.bfloat16, dev),
                     null if lse is None else _dev_ptr(lse, "lse", torch.float32, dev),
                     plan_.max_pages_per_req, plan_.kv_chunk_pages,
                     _dev_ptr(ws, "workspace", device=dev), ws.numel() * ws.element_size(),
                     _stream(stream))
    if rc != PKV_OK:
        raise PkvError(rc, "pkv_run")
    return out, lse


class MixedPlan(DecodePlan):
    """A mixed step's decode schedule (pkv_plan_mixed): the decode rows of a
    batch that also carries prompts, planned under their row indices."""

    def __init__(self, workspace, batch, total_rows, num_qo_heads, max_pages_per_req,
                 kv_chunk_pages, qo_indptr):
        super().__init__(workspace, total_rows, num_qo_heads, max_pages_per_req,
                         kv_chunk_pages)
        self.entries = batch
        self.qo_indptr = qo_indptr


def plan_mixed(kv_cache, num_qo_heads: int, qo_indptr, page_indptr, page_indices,
               last_page_len, total_rows: int, max_pages_per_req: int,
               kv_chunk_pages: int = 0, workspace=None, stream=None) -> MixedPlan:
    """Plan the decode rows of a mixed step (pkv_plan_mixed): entries with one
    new row; total_rows = qo_indptr[-1].  Returns the plan for
    :func:`mixed_run`."""
    import torch
    desc = cache_desc(kv_cache)
    batch = int(last_page_len.shape[0])
    if tuple(qo_indptr.shape) != (batch + 1,):
        raise ValueError("qo_indptr must be [batch + 1]")
    dev = kv_cache.device
    need = workspace_size(desc, num_qo_heads, int(total_rows), max_pages_per_req,
                          kv_chunk_pages)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    rc = lib.pkv_plan_mixed(desc, int(num_qo_heads),
                            _dev_ptr(qo_indptr, "qo_indptr", torch.int32, dev),
                            *_tables(kv_cache, page_indptr, page_indices, last_page_len),
                            batch, int(total_rows), int(max_pages_per_req),
                            int(kv_chunk_pages), _dev_ptr(workspace, "workspace", device=dev),
                            workspace.numel() * workspace.element_size(), _stream(stream))
    if rc != PKV_OK:
        raise PkvError(rc, "pkv_plan_mixed")
    return MixedPlan(workspace, batch, int(total_rows), int(num_qo_heads),
                     int(max_pages_per_req), int(kv_chunk_pages), qo_indptr)


def mixed_run(kv_cache, layer: int, q, page_indptr, page_indices, last_page_len,
              plan_: MixedPlan, sm_scale: float, max_q_rows: int, k_new=None, v_new=None,
              out=None, lse=None, with_lse: bool = True, stream=None):
    """One layer of a mixed step in one call (pkv_mixed_run): decode rows on
    the plan, prompts through the prefill; returns (out, lse) like
    :func:`prefill`."""
    import torch
    desc = cache_desc(kv_cache)
    rows, hq = plan_.batch, plan_.num_qo_heads
    if q.dim() != 3 or q.shape[0] != rows or q.shape[1] != hq:
        raise ValueError("q must be [total_rows, Hq, D] of the plan")
    append = k_new is not None or v_new is not None
    if append:
        for name, t in (("k_new", k_new), ("v_new", v_new)):
            if t is None or tuple(t.shape) != (rows, desc.num_kv_heads, desc.head_dim):
                raise ValueError(f"{name} must be [total_rows, Hkv, D]")
    dev = kv_cache.device
    if out is None:
        out = torch.empty_like(q)
    if lse is None and with_lse:
        lse = torch.empty((rows, hq), dtype=torch.float32, device=dev)
    null = ctypes.c_void_p(0)
    ws = plan_.workspace
    rc = lib.pkv_mixed_run(_dev_ptr(kv_cache, "kv_cache", torch.bfloat16), desc, int(layer),
                           _dev_ptr(q, "q", torch.bfloat16, dev), hq,
                           _dev_ptr(plan_.qo_indptr, "qo_indptr", torch.int32, dev),
                           _dev_ptr(k_new, "k_new", torch.bfloat16, dev) if append else null,
                           _dev_ptr(v_new, "v_new", torch.bfloat16, dev) if append else null,
                           *_tables(kv_cache, page_indptr, page_indices, last_page_len),
                           plan_.entries, rows, int(max_q_rows), float(sm_scale),
                           _dev_ptr(out, "out", torch.bfloat16, dev),
                           null if lse is None else _dev_ptr(lse, "lse", torch.float32, dev),
                           plan_.max_pages_per_req, plan_.kv_chunk_pages,
                           _dev_ptr(ws, "workspace", device=dev), ws.numel() * ws.element_size(),
                           _stream(stream))
    if rc != PKV_OK:
        raise PkvError(rc, "pkv_mixed_run")
    return out, lse


def run_qk_norm_rope(kv_cache, layer: int, q, plan_: DecodePlan, sm_scale: float, k_new,
                     v_new, q_norm_weight, k_norm_weight, positions, eps: float = 1e-6,
                     rope_theta: float = 1e6, out=None, lse=None, with_lse: bool = True,
                     stream=None, pair_axis=None):
    """Decode one layer on a plan with the append and the q/k RMSNorm + rotary
    embedding folded in (pkv_run_qk_norm_rope): q, k_new are the raw
    projections; returns (out, lse).  With pair_axis (a host sequence of
    head_dim/2 values in {0, 1, 2}) the rotary embedding is multimodal
    (pkv_run_qk_norm_mrope) and positions is [batch, 3] (t, h, w)."""
    import torch
    desc = cache_desc(kv_cache)
    batch, hq, d = plan_.batch, plan_.num_qo_heads, desc.head_dim
    if q.dim() != 3 or q.shape[0] != batch or q.shape[1] != hq:
        raise ValueError("q must be [batch, Hq, D] of the plan")
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if t is None or tuple(t.shape) != (batch, desc.num_kv_heads, d):
            raise ValueError(f"{name} must be [batch, Hkv, D]")
    for name, t in (("q_norm_weight", q_norm_weight), ("k_norm_weight", k_norm_weight)):
        if tuple(t.shape) != (d,):
            raise ValueError(f"{name} must be [{d}], got {tuple(t.shape)}")
    multimodal = pair_axis is not None
    if multimodal:
        axis = np.ascontiguousarray(pair_axis, dtype=np.uint8)
        if axis.shape != (d // 2,):
            raise ValueError(f"pair_axis must hold {d // 2} values")
        if tuple(positions.shape) != (batch, 3):
            raise ValueError(f"positions must be [batch, 3], got {tuple(positions.shape)}")
    elif tuple(positions.shape) != (batch,):
        raise ValueError(f"positions must be [batch], got {tuple(positions.shape)}")
    dev = kv_cache.device
    if out is None:
        out = torch.empty((batch, hq, d), dtype=torch.bfloat16, device=dev)
    if lse is None and with_lse:
        lse = torch.empty((batch, hq), dtype=torch.float32, device=dev)
    null = ctypes.c_void_p(0)
    ws = plan_.workspace
    head = (_dev_ptr(kv_cache, "kv_cache", torch.bfloat16), desc, int(layer),
            _dev_ptr(k_new, "k_new", torch.bfloat16, dev),
            _dev_ptr(v_new, "v_new", torch.bfloat16, dev),
            _dev_ptr(q, "q", torch.bfloat16, dev), hq, batch,
            _dev_ptr(q_norm_weight, "q_norm_weight", torch.bfloat16, dev),
            _dev_ptr(k_norm_weight, "k_norm_weight", torch.bfloat16, dev),
            float(eps), float(rope_theta), _dev_ptr(positions, "positions", torch.int32, dev))
    tail = (float(sm_scale), _dev_ptr(out, "out", torch.bfloat16, dev),
            null if lse is None else _dev_ptr(lse, "lse", torch.float32, dev),
            plan_.max_pages_per_req, plan_.kv_chunk_pages,
            _dev_ptr(ws, "workspace", device=dev), ws.numel() * ws.element_size(),
            _stream(stream))
    if multimodal:
        name = "pkv_run_qk_norm_mrope"
        rc = lib.pkv_run_qk_norm_mrope(*head, axis.ctypes.data_as(ctypes.c_void_p), *tail)
    else:
        name = "pkv_run_qk_norm_rope"
        rc = lib.pkv_run_qk_norm_rope(*head, *tail)
    if rc != PKV_OK:
        raise PkvError(rc, name)
    return out, lse


def validate_page_table(page_indptr, page_indices, last_page_len, num_pages: int,
                        page_size: int, max_pages_per_req: int = 0):
    """Check HOST copies of a page table; returns (status, first bad entry)."""
    ip = np.ascontiguousarray(page_indptr, dtype=np.int32)
    ix = np.ascontiguousarray(page_indices, dtype=np.int32)
    ll = np.ascontiguousarray(last_page_len, dtype=np.int32)
    bad = ctypes.c_int32(-1)
    rc = lib.pkv_validate_page_table(ip.ctypes.data_as(ctypes.c_void_p),
                                     ix.ctypes.data_as(ctypes.c_void_p),
                                     ll.ctypes.data_as(ctypes.c_void_p), len(ll),
                                     int(num_pages), int(page_size),
                                     int(max_pages_per_req), ctypes.byref(bad))
    return int(rc), int(bad.value)
