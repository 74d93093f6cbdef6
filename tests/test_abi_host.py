"""Host-side checks of the C ABI (CPU only, no kernel launches).

The library must load, export every function include/rsq.h declares, and
reject bad arguments with the documented status before enqueuing anything.
Every call here fails validation, so no GPU is touched.
"""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rsq.h")


def _lib():
    import rotation_bit_post_amd as rsq
    return rsq


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rsq_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_four_path_entry_points():
    names = _declared_functions()
    for fn in ("rsq_subspace_correct", "rsq_quant_act", "rsq_qgemm", "rsq_layer_fused"):
        assert fn in names


def test_library_exports_every_declared_function():
    rsq = _lib()
    declared = _declared_functions()
    for name in declared:
        assert hasattr(rsq.LIB, name), name
    assert set(declared) == set(rsq.EXPORTS)


def test_status_strings_and_queries():
    rsq = _lib()
    assert rsq.LIB.rsq_status_str(0) == b"RSQ_OK"
    assert rsq.LIB.rsq_status_str(2) == b"RSQ_ERR_UNSUPPORTED"
    assert rsq.LIB.rsq_status_str(99) == b"RSQ_UNKNOWN_STATUS"
    assert rsq.rsq_version() >= 100
    assert rsq.rsq_packed_row_bytes(4096, 4) == 2048
    assert rsq.rsq_packed_row_bytes(4096, 3) == 1536
    assert rsq.rsq_packed_row_bytes(11008, 3) == 4128
    assert rsq.rsq_packed_row_bytes(33, 4) == 0 and rsq.rsq_packed_row_bytes(64, 5) == 0
    assert rsq.rsq_site_bytes(4096, 32) == 4096 * 32 * 8
    assert rsq.rsq_site_bytes(256, 8) == 256 * 32 * 8        # r padded to 32
    assert rsq.rsq_site_bytes(4096, 65) == 0


FAKE = 1 << 20  # a 16-byte aligned non-null address; never dereferenced because validation fails first


def _call(fn, *args):
    rsq = _lib()
    st = getattr(rsq.LIB, fn)(*args)
    return st, rsq.LIB.rsq_last_error().decode()


@pytest.mark.parametrize("args,status,needle", [
    ((FAKE, FAKE, 1, 4, 100, 4096, FAKE, 32, None), 1, "multiple of 32"),      # d
    ((FAKE, FAKE, 1, 4, 4096, 4096, FAKE, 0, None), 1, "r = 0"),               # r
    ((FAKE, FAKE, 1, 4, 4096, 4096, FAKE, 96, None), 2, "exceeds the supported"),
    ((FAKE, FAKE, 2, 4, 4096, 4096, FAKE, 32, None), 1, "h_dtype"),
    ((FAKE, FAKE, 1, -1, 4096, 4096, FAKE, 32, None), 1, "negative"),
    ((FAKE, FAKE, 1, 4, 4096, 4000, FAKE, 32, None), 1, "ld_h"),
    ((FAKE, FAKE, 1, 4, 4096, 4100, FAKE, 32, None), 1, "multiple of 16"),
    ((None, FAKE, 1, 4, 4096, 4096, FAKE, 32, None), 1, "null pointer"),
    ((FAKE + 8, FAKE + 8, 1, 4, 4096, 4096, FAKE, 32, None), 1, "aligned"),
    ((FAKE, FAKE + 64, 1, 4, 4096, 4096, FAKE, 32, None), 1, "overlap"),
    ((FAKE, FAKE, 1, 4, 32 * 9 * 8, 32 * 9 * 8, FAKE, 32, None), 2, "waves"),  # d/32 = 72: no even split
])
def test_subspace_correct_validation(args, status, needle):
    st, msg = _call("rsq_subspace_correct", *args)
    assert st == status and needle in msg, (st, msg)


@pytest.mark.parametrize("args,status,needle", [
    ((FAKE, 1, 4, 4096, 4096, 0, None, 1e-5, 5, FAKE, FAKE, None), 1, "bits"),
    ((FAKE, 1, 4, 4016, 4016, 0, None, 1e-5, 4, FAKE, FAKE, None), 1, "multiple of 32"),
    ((FAKE, 1, 4, 65536, 65536, 0, None, 1e-5, 4, FAKE, FAKE, None), 2, "32768"),
    ((FAKE, 1, 4, 4096, 4096, 4, None, 1e-5, 4, FAKE, FAKE, None), 1, "flags"),
    ((FAKE, 1, 4, 4096, 4096, 1, None, -1.0, 4, FAKE, FAKE, None), 1, "eps"),
    ((FAKE, 1, 4, 4096, 4096, 0, None, 1e-5, 4, None, FAKE, None), 1, "null pointer"),
    ((None, 1, 4, 4096, 4096, 0, None, 1e-5, 4, FAKE, FAKE, None), 1, "x must be"),
    ((FAKE, 1, 4, 4096, 4096, 1, FAKE + 8, 1e-5, 4, FAKE, FAKE, None), 1, "norm_w"),
])
def test_quant_act_validation(args, status, needle):
    st, msg = _call("rsq_quant_act", *args)
    assert st == status and needle in msg, (st, msg)


@pytest.mark.parametrize("args,status,needle", [
    ((FAKE, FAKE, 8, FAKE, FAKE, 100, 4096, 4, FAKE, 1, 100, None, None, 0, None), 1, "n_out"),
    ((FAKE, FAKE, 8, FAKE, FAKE, 128, 4016, 4, FAKE, 1, 128, None, None, 0, None), 1, "multiple of 32"),
    ((FAKE, FAKE, 8, FAKE, FAKE, 128, 4096, 2, FAKE, 1, 128, None, None, 0, None), 1, "bits"),
    ((FAKE, FAKE, 8, FAKE, FAKE, 128, 4096, 4, FAKE, 1, 64, None, None, 0, None), 1, "ld_y"),
    ((FAKE, FAKE, 8, FAKE, FAKE, 128, 131072, 4, FAKE, 1, 128, None, None, 0, None), 2, "65536"),
    ((FAKE, FAKE, 8, None, FAKE, 128, 4096, 4, FAKE, 1, 128, None, None, 0, None), 1, "null pointer"),
    ((FAKE, FAKE, 8, FAKE, FAKE, 128, 4096, 4, FAKE, 1, 128, FAKE + 4, None, 0, None), 1, "acc_out"),
])
def test_qgemm_validation(args, status, needle):
    st, msg = _call("rsq_qgemm", *args)
    assert st == status and needle in msg, (st, msg)


def test_qgemm_residual_validation():
    # (a, sa, n, w, sw, n_out, k, bits, residual, ld_r, y, y_dtype, ld_y, stream)
    # (a, sa, n, w, sw, n_out, k, bits, residual, ld_r, y, y_dtype, ld_y, workspace, workspace_bytes, stream)
    st, msg = _call("rsq_qgemm_residual", FAKE, FAKE, 4, FAKE, FAKE, 128, 256, 4, None, 128, FAKE, 1, 128, None, 0, None)
    assert st == 1 and "null" in msg
    st, msg = _call("rsq_qgemm_residual", FAKE, FAKE, 4, FAKE, FAKE, 128, 256, 4, FAKE, 64, FAKE + 4096, 1, 128, None, 0,
                    None)
    assert st == 1 and "ld_r" in msg
    st, msg = _call("rsq_qgemm_residual", FAKE, FAKE, 4, FAKE, FAKE, 128, 256, 4, FAKE, 128, FAKE + 64, 1, 128, None, 0,
                    None)
    assert st == 1 and "overlap" in msg
    st, msg = _call("rsq_qgemm_residual", FAKE, FAKE, 4, FAKE, FAKE, 128, 256, 4, FAKE, 160, FAKE, 1, 128, None, 0, None)
    assert st == 1 and "in place" in msg
    assert _call("rsq_qgemm_residual", None, None, 0, None, None, 128, 256, 4, None, 128, None, 1, 128, None, 0,
                 None)[0] == 0


def test_empty_batches_are_accepted_without_pointers():
    # n = 0 enqueues nothing, so it needs neither data pointers nor a device
    assert _call("rsq_subspace_correct", None, None, 1, 0, 4096, 4096, None, 32, None)[0] == 0
    assert _call("rsq_quant_act", None, 1, 0, 4096, 4096, 0, None, 1e-5, 4, None, None, None)[0] == 0
    assert _call("rsq_qgemm", None, None, 0, None, None, 128, 4096, 4, None, 1, 128, None, None, 0, None)[0] == 0
    assert _call("rsq_correct_quant", None, None, 1, 0, 4096, None, 32, None, C.c_float(1e-5), 4, None, None, None, 0,
                 None)[0] == 0


def test_layer_fused_and_site_prepare_validation():
    st, msg = _call("rsq_layer_fused", FAKE, FAKE, 1, 4, 4096, FAKE, 32, None, C.c_float(1e-5), 4, FAKE, FAKE,
                    FAKE, FAKE, 100, FAKE, 1, None, 0, None)
    assert st == 1 and "n_out" in msg
    st, msg = _call("rsq_layer_fused", FAKE, FAKE, 1, 4, 4096, FAKE, 32, FAKE + 4, C.c_float(1e-5), 4, FAKE, FAKE,
                    FAKE, FAKE, 128, FAKE, 1, None, 0, None)
    assert st == 1 and "norm_w" in msg
    st, msg = _call("rsq_site_prepare", FAKE, FAKE, 4096, 128, FAKE, None)
    assert st == 2 and "exceeds" in msg
    st, msg = _call("rsq_site_prepare", None, FAKE, 4096, 32, FAKE, None)
    assert st == 1 and "null" in msg


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "rsq_binding_copy", os.path.join(ROOT, "rotation_bit_post_amd", "_binding.py"))
    mod = importlib.util.module_from_spec(spec)
    monkeypatch.setattr(os.path, "exists", lambda p: False if p.endswith("librsq.so") else os.path.isfile(p))
    with pytest.raises(ImportError, match="no fallback"):
        spec.loader.exec_module(mod)
