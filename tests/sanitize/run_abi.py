"""Test infrastructure, run in a child process by tests/test_sanitizers.py:
drive the C ABI's host code, built under AddressSanitizer and
UndefinedBehaviorSanitizer with tests/sanitize/host_stub.cpp in place of the
kernel launches, through every validation case of tests/test_abi.py and
through successful calls of every entry point on fake device pointers (the
stand-ins never dereference them).

    python tests/sanitize/run_abi.py LIB
"""
import ctypes
import os
import sys
import types

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))


def load_binding(lib_path):
    """The package's binding with its library path pointed at `lib_path`."""
    pkg = os.path.join(ROOT, "paged_kv_decode_pkv_amd", "__init__.py")
    src = open(pkg).read()
    old = 'LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")'
    assert old in src
    src = src.replace(old, f"LIB_PATH = {os.path.abspath(lib_path)!r}")
    mod = types.ModuleType("paged_kv_decode_pkv_amd")
    mod.__file__ = pkg
    mod.__path__ = [os.path.dirname(pkg)]
    exec(compile(src, pkg, "exec"), mod.__dict__)
    sys.modules["paged_kv_decode_pkv_amd"] = mod
    return mod


def full_calls(pkv):
    """Every entry point with valid arguments: each must return PKV_OK."""
    lib, CacheDesc = pkv.lib, pkv.CacheDesc
    f = lambda a: ctypes.c_void_p(a)   # noqa: E731
    dev = f(0x100000)
    ws = f(0x200000)
    null = f(0)
    shapes = [(CacheDesc(36, 8192, 16, 8, 128), 32, 64, 219),
              (CacheDesc(1, 128, 16, 2, 64), 14, 4, 16),
              (CacheDesc(28, 8192, 16, 8, 128), 16, 256, 32),
              (CacheDesc(1, 32768, 16, 8, 128), 32, 8, 2048),
              (CacheDesc(1, 1025, 128, 16, 128), 16, 64, 16),
              (CacheDesc(2, 64, 1, 16, 64), 16, 4200, 24)]
    n = 0
    for desc, hq, batch, maxp in shapes:
        for chunk in (0, 1, 16, 64):
            wsb = pkv.workspace_size(desc, hq, batch, maxp, chunk)
            assert wsb > 0
            rc = lib.pkv_decode(dev, desc, 0, dev, hq, dev, dev, dev, batch, 0.1, dev, dev,
                                maxp, chunk, ws, wsb, null)
            assert rc == 0, (desc.head_dim, hq, batch, chunk, rc)
            rc = lib.pkv_append_decode(dev, desc, 0, dev, dev, dev, hq, dev, dev, dev, batch,
                                       0.1, dev, null, maxp, chunk, ws, wsb, null)
            assert rc == 0
            assert lib.pkv_plan(desc, hq, dev, dev, dev, batch, maxp, chunk, ws, wsb,
                                null) == 0
            assert lib.pkv_run(dev, desc, 0, null, null, dev, hq, batch, 0.1, dev, dev,
                               maxp, chunk, ws, wsb, null) == 0
            # one byte short of the workspace is refused
            assert lib.pkv_run(dev, desc, 0, null, null, dev, hq, batch, 0.1, dev, dev,
                               maxp, chunk, ws, wsb - 1, null) == -4
            if wsb <= 16 << 20:
                assert lib.pkv_decode_static(dev, desc, 0, dev, hq, dev, dev, dev, batch, 0.1,
                                             dev, dev, maxp, chunk, null) == 0
            n += 5
        assert lib.pkv_append(dev, desc, 0, dev, dev, dev, dev, dev, batch, null) == 0
        assert lib.pkv_qk_norm_rope_append(dev, desc, 0, dev, hq, dev, dev, dev, dev, 1e-6,
                                           1e6, dev, dev, dev, dev, batch, dev, null) == 0
        axis = (ctypes.c_uint8 * (desc.head_dim // 2))(*([0, 1, 2] * 64)[:desc.head_dim // 2])
        assert lib.pkv_qk_norm_mrope_append(dev, desc, 0, dev, hq, dev, dev, dev, dev, 1e-6,
                                            1e6, dev, axis, dev, dev, dev, batch, dev,
                                            null) == 0
        if desc.head_dim == 128 and hq // desc.num_kv_heads <= 4:
            wsb = pkv.workspace_size(desc, hq, batch, maxp, 0)
            assert lib.pkv_run_qk_norm_rope(dev, desc, 0, dev, dev, dev, hq, batch, dev, dev,
                                            1e-6, 1e6, dev, 0.1, dev, dev, maxp, 0, ws, wsb,
                                            null) == 0
        if desc.head_dim == 128 and batch <= 65535:
            assert lib.pkv_prefill(dev, desc, 0, dev, hq, dev, dev, dev, dev, dev, dev, batch,
                                   8, 0.1, dev, dev, null) == 0
        n += 4
    return n


def main():
    pkv = load_binding(sys.argv[1])
    import pytest
    rc = pytest.main([os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-p",
                      "no:cacheprovider", "-k", "not hip_runtime"])
    if rc != 0:
        return int(rc)
    print(f"full host paths: {full_calls(pkv)} calls returned as expected", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
