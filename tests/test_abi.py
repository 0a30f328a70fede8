"""The C ABI library loads, exports every entry point include/tbe.h declares,
and rejects bad arguments on the host before touching a GPU."""
import ctypes
import os
import re

import pytest

import table_embedding_bag_amd as tbe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "tbe.h")).read()
    return sorted(set(re.findall(r"^\s*(?:tbe_status|void|const char\*|int32_t)\s+(tbe_\w+)\(", src, re.M)))


def test_header_and_binding_agree():
    assert _declared() == sorted(tbe.EXPORTED_SYMBOLS)


def test_header_constants_match_the_binding():
    """Every TBE_FLAG_* / TBE_OPTION_* value the header defines is the binding's constant of
    the same name (a mismatch would pass the wrong option or flag through the ABI)."""
    src = open(os.path.join(ROOT, "include", "tbe.h")).read()
    found = re.findall(r"\bTBE_((?:FLAG|OPTION)_\w+)\s*=\s*(\d+)u?", src)
    assert found
    for name, value in found:
        assert getattr(tbe, name) == int(value), name


def test_static_scratch_size_matches_the_binding():
    src = open(os.path.join(ROOT, "include", "tbe.h")).read()
    m = re.search(r"#define TBE_STATIC_SCRATCH_BYTES \((\d+)u << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == tbe.STATIC_SCRATCH_BYTES


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(tbe.library_path())
    for name in _declared():
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings():
    assert tbe.tbe_abi_version() == 2
    for s in range(8):
        assert tbe.tbe_status_string(s)
    assert tbe.tbe_status_string(0) == "ok"


def _cfg(rows, dims, dtype=0, pooling=0, opt=0, flags=0):
    T = len(rows)
    r = (ctypes.c_int64 * T)(*rows)
    d = (ctypes.c_int32 * T)(*dims)
    return tbe._Config(T, r, d, dtype, pooling, opt, flags), (r, d)


@pytest.mark.parametrize("case", ["null_weights", "no_tables", "zero_rows", "dim_too_big", "bad_dtype",
                                  "bad_pooling", "bad_optimizer", "adagrad_without_state",
                                  "unknown_flag", "lowest_unknown_flag", "conflicting_flags",
                                  "misaligned_weights"])
def test_create_rejects_bad_configs_on_host(case):
    lib = tbe.load()
    rows, dims, kw, w, st = [10, 20], [8, 8], {}, 4096, None
    if case == "no_tables":
        rows, dims = [], []
    elif case == "zero_rows":
        rows = [10, 0]
    elif case == "dim_too_big":
        dims = [8, 4096]
    elif case == "bad_dtype":
        kw["dtype"] = 7
    elif case == "bad_pooling":
        kw["pooling"] = 3
    elif case == "bad_optimizer":
        kw["opt"] = 9
    elif case == "adagrad_without_state":
        kw["opt"] = 1
    elif case == "unknown_flag":
        kw["flags"] = 256
    elif case == "lowest_unknown_flag":
        kw["flags"] = tbe.FLAG_COUNT_BACKWARD << 1
    elif case == "conflicting_flags":
        kw["flags"] = 6
    elif case == "misaligned_weights":
        w = 4096 + 4
    if case == "null_weights":
        w = None
    cfg, keep = _cfg(rows, dims, **kw)
    out = ctypes.c_void_p(123)
    rc = lib.tbe_create(ctypes.byref(cfg), w, st, ctypes.byref(out))
    assert rc == 1 and out.value is None


@pytest.mark.parametrize("dtype,rows,dims", [(0, [10, 20], [16, 16]),     # fp32 storage
                                             (2, [10, 2000], [16, 16]),   # a table over 1024 rows
                                             (1, [10, 20], [16, 24]),     # a dim not in 16-column tiles
                                             (2, [10, 20], [16, 512])])   # a dim over 256
def test_forced_histogram_on_an_ineligible_table_is_unsupported(dtype, rows, dims):
    """The count-matrix forward only takes small fp16/bf16 tables; forcing it on any other
    table fails at create, before any device call."""
    lib = tbe.load()
    cfg, keep = _cfg(rows, dims, dtype=dtype, flags=tbe.FLAG_FORCE_HISTOGRAM)
    out = ctypes.c_void_p(123)
    assert lib.tbe_create(ctypes.byref(cfg), 4096, None, ctypes.byref(out)) == 2
    assert out.value is None


def test_null_handle_calls_are_rejected():
    lib = tbe.load()
    n = ctypes.c_size_t(0)
    assert lib.tbe_backward_workspace_size(None, 4, 10, ctypes.byref(n)) == 1
    assert lib.tbe_forward(None, 4, None, None, 1, 0, None, None, None) == 1
    assert lib.tbe_set_option(None, 1, 5) == 1
    assert lib.tbe_forward_group(None, 4, None, None, 1, 0, None, None, None, 0, None) == 1
    assert lib.tbe_backward_update_grouped(None, 4, None, None, 1, 0, None, None, 0.1, 0.0, None,
                                           0, None, None) == 1
    assert lib.tbe_psw_grad(None, 4, None, None, 1, 0, None, None, None) == 1
    assert lib.tbe_check_device_status(None, None) == 1
    assert lib.tbe_backward_update_no_alloc(None, 4, None, None, 1, 0, None, None, 0.1, 0.0,
                                            None, None) == 1
    assert lib.tbe_forward_scratch_size(None, ctypes.byref(n)) == 1
    assert lib.tbe_set_forward_scratch(None, None, 0) == 1
    lib.tbe_destroy(None)


@pytest.mark.parametrize("rows,dims", [([10, 2000], [16, 16]),   # a table over 1024 rows
                                       ([10, 20], [16, 24]),     # a dim not in 16-column tiles
                                       ([10, 20], [16, 512])])   # a dim over 256
def test_count_backward_on_an_ineligible_table_is_unsupported(rows, dims):
    """The count-matrix backward takes only handles whose every table is small; otherwise
    tbe_create fails before any device call."""
    lib = tbe.load()
    cfg, keep = _cfg(rows, dims, dtype=0, flags=tbe.FLAG_COUNT_BACKWARD)
    out = ctypes.c_void_p(123)
    assert lib.tbe_create(ctypes.byref(cfg), 4096, None, ctypes.byref(out)) == 2
    assert out.value is None
