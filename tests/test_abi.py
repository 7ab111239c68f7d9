"""The C-ABI library loads, exports every symbol include/ap.h declares, and
rejects invalid arguments before it touches the device (CPU only)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_symbols():
    src = open(os.path.join(ROOT, "include", "ap.h")).read()
    return sorted(set(re.findall(r"\b(ap_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    from rank_compressed_kv_ap_amd import binding
    syms = _header_symbols()
    assert "ap_compress" in syms and "ap_decode_attn" in syms and "ap_free" in syms
    missing = [s for s in syms if not hasattr(binding.lib, s)]
    assert not missing, missing
    assert set(syms) == set(binding.EXPORTED)


def test_struct_layouts_match_header(tmp_path):
    """Every field offset and struct size of the binding's ctypes mirrors equals what a
    C compiler computes from include/ap.h."""
    import subprocess
    from rank_compressed_kv_ap_amd import binding
    structs = {"ap_compress_params": binding.CompressParams, "ap_decode_params": binding.DecodeParams}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "ap.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'  printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    inc = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include")
    subprocess.run(["gcc", "-I", inc, str(src), "-o", str(exe)], check=True)
    got = dict(l.rsplit(" ", 1) for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                        check=True).stdout.splitlines())
    for cname, py in structs.items():
        assert int(got[f"{cname} size"]) == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert int(got[f"{cname} {f}"]) == getattr(py, f).offset, (cname, f)


def _compress_status(**kw):
    from rank_compressed_kv_ap_amd import binding as b
    base = dict(batch=2, n_tokens=64, n_kv_heads=2, n_q_heads=4, head_dim=32, rank=16,
                oversample=16, power_iters=2, storage=b.AP_BF16, reserved=0, seed=0, omega=None)
    base.update(kw)
    p = b.CompressParams(**base)
    out = ctypes.c_void_p(1)
    st = b.lib.ap_compress(None, None, ctypes.byref(p), None, ctypes.byref(out))
    return st, out.value


@pytest.mark.parametrize("kw,status", [
    (dict(storage=7), 3),
    (dict(reserved=1), 2),
    (dict(batch=-1), 2),
    (dict(n_tokens=0), 2),
    (dict(n_q_heads=3), 2),
    (dict(rank=0), 2),
    (dict(rank=65), 2),
    (dict(head_dim=0), 2),
    (dict(n_tokens=40000, rank=16), 4),
    (dict(rank=144, n_tokens=256, head_dim=128), 4),
    (dict(n_q_heads=128, n_kv_heads=2), 4),
    (dict(power_iters=-1), 2),
])
def test_compress_validation_errors(kw, status):
    st, out = _compress_status(**kw)
    assert st == status
    assert out is None


def test_null_arguments():
    from rank_compressed_kv_ap_amd import binding as b
    out = ctypes.c_void_p(1)
    assert b.lib.ap_compress(None, None, None, None, ctypes.byref(out)) == b.AP_ERR_NULL_ARG
    p = b.CompressParams(2, 64, 2, 4, 32, 16, 16, 2, b.AP_BF16, 0, 0, None)
    assert b.lib.ap_compress(ctypes.c_void_p(16), None, ctypes.byref(p), None,
                             ctypes.byref(out)) == b.AP_ERR_NULL_ARG
    assert out.value is None
    dp = b.DecodeParams(4, 8, 0.1, 0, None, None, None, 0)
    assert b.lib.ap_decode_attn(None, None, None, ctypes.byref(dp), None) == b.AP_ERR_NULL_ARG
    b.lib.ap_free(None)
    assert b.lib.ap_status_string(b.AP_ERR_UNSUPPORTED) == b"unsupported"
    assert b"n_kv_heads" in b.lib.ap_last_error() or b.lib.ap_last_error() != b""


def test_compress_rejects_large_probe_count_before_touching_memory():
    # ell = min(r + p, N, W) = 160 > 144: refused during validation, so the (never
    # dereferenced) fake device pointers are safe on a machine without a GPU
    from rank_compressed_kv_ap_amd import binding as b
    p = b.CompressParams(1, 512, 4, 4, 64, 128, 32, 2, b.AP_BF16, 0, 0, None)
    out = ctypes.c_void_p(1)
    st = b.lib.ap_compress(ctypes.c_void_p(256), ctypes.c_void_p(512), ctypes.byref(p), None,
                           ctypes.byref(out))
    assert st == b.AP_ERR_UNSUPPORTED and out.value is None
    assert b"144" in b.lib.ap_last_error()


def test_compress_rejects_batch_beyond_the_grid_limit():
    # 2 * batch matrices index one grid dimension (at most 65535): batch 32768 is refused
    # during validation, before any device memory is touched (CPU only)
    from rank_compressed_kv_ap_amd import binding as b
    p = b.CompressParams(32768, 64, 1, 1, 64, 8, 4, 1, b.AP_BF16, 0, 0, None)
    out = ctypes.c_void_p(1)
    st = b.lib.ap_compress(None, None, ctypes.byref(p), None, ctypes.byref(out))
    assert st == b.AP_ERR_UNSUPPORTED and out.value is None
    assert b"32767" in b.lib.ap_last_error()


def test_decode_rejects_text_pointers_without_text_tokens():
    # text_k / text_v are NULL iff n_text == 0; checked before the cache is looked at, so
    # a NULL cache handle is safe here (CPU only)
    from rank_compressed_kv_ap_amd import binding as b
    for tk, tv in ((ctypes.c_void_p(64), None), (None, ctypes.c_void_p(64)),
                   (ctypes.c_void_p(64), ctypes.c_void_p(128))):
        dp = b.DecodeParams(4, 8, 0.1, 0, tk, tv, None, 0)
        assert b.lib.ap_decode_attn(None, None, None, ctypes.byref(dp), None) == b.AP_ERR_BAD_SHAPE
        assert b"n_text" in b.lib.ap_last_error()
    dp = b.DecodeParams(4, 8, 0.1, 0, None, None, None, 0)
    assert b.lib.ap_decode_attn(None, None, None, ctypes.byref(dp), None) == b.AP_ERR_NULL_ARG


def test_read_bandwidth_rejects_bad_arguments_before_any_launch():
    # every check runs before a device call, so bogus (never dereferenced) pointers are safe
    from rank_compressed_kv_ap_amd import binding as b
    ms = ctypes.c_float()
    assert b.lib.ap_read_bandwidth(None, 1024, 1, None, ctypes.byref(ms)) == b.AP_ERR_NULL_ARG
    assert b.lib.ap_read_bandwidth(ctypes.c_void_p(256), 1024, 1, None, None) == b.AP_ERR_NULL_ARG
    for ptr, nbytes, passes in ((256, 1000, 1), (256, 0, 1), (8, 1024, 1), (256, 1024, 0), (256, 1024, 1001)):
        assert b.lib.ap_read_bandwidth(ctypes.c_void_p(ptr), nbytes, passes, None,
                                       ctypes.byref(ms)) == b.AP_ERR_BAD_SHAPE, (ptr, nbytes, passes)
    assert b"16-byte" in b.lib.ap_last_error()
