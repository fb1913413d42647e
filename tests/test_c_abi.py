"""The C ABI used from C: tests/c_abi_check.c is compiled against
include/vsa.h with gcc, linked to libvsa.so and run (host-only calls).  Its
struct layouts must match the ctypes binding, and its sizing answers must
match the same queries made through the binding."""
import ctypes
import os
import subprocess

import pytest

from block_sparse_attention_centroids_amd import _lib

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.fixture(scope="module")
def c_output(tmp_path_factory):
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libvsa.so is not built")
    exe = str(tmp_path_factory.mktemp("cabi") / "c_abi_check")
    libdir = os.path.dirname(_lib.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "c_abi_check.c"), "-L", libdir, "-lvsa", "-Wl,-rpath," + libdir, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    out = {}
    for line in r.stdout.splitlines():
        key, *vals = line.split()
        out[key] = vals
    return out


def test_struct_layouts_match_binding(c_output):
    assert int(c_output["sizeof_shape"][0]) == ctypes.sizeof(_lib.VsaShape)
    assert int(c_output["sizeof_index"][0]) == ctypes.sizeof(_lib.VsaIndex)
    assert int(c_output["offsetof_index_row_ptr"][0]) == _lib.VsaIndex.row_ptr.offset
    assert int(c_output["offsetof_index_capacity"][0]) == _lib.VsaIndex.capacity.offset
    assert int(c_output["offsetof_index_equal_heads"][0]) == _lib.VsaIndex.equal_heads.offset
    assert int(c_output["sizeof_select"][0]) == ctypes.sizeof(_lib.VsaSelect)
    assert int(c_output["offsetof_select_value"][0]) == _lib.VsaSelect.value.offset
    assert int(c_output["offsetof_select_estimator"][0]) == _lib.VsaSelect.estimator.offset
    assert int(c_output["sizeof_head_option"][0]) == ctypes.sizeof(_lib.VsaHeadOption)


def test_sizing_matches_binding(c_output):
    import block_sparse_attention_centroids_amd as vsa
    shape = _lib.VsaShape(1, 12, 128, 21, 30, 52, 4, 4, 8, _lib.VSA_BF16)
    st, rl, cap, pws, aws = c_output["query"]
    assert st == "0" and (int(rl), int(cap), int(pws), int(aws)) == vsa.query(shape, 0.2)
    st, rl, cap, pws = c_output["query_select"]
    assert st == "0" and (int(rl), int(cap), int(pws)) == vsa.query_select(shape, "topp", 0.25, -1, 2, None, "dsa")
    st, rl, cap, pws = c_output["query_mixed"]
    kinds = ["dynamic", "static", "dense"]
    opts = [{"kind": kinds[h % 3], "value": 0.2, "window_t": (h % 4) - 1} for h in range(12)]
    assert st == "0" and (int(rl), int(cap), int(pws)) == vsa.query_mixed(shape, opts)
    assert c_output["scheme_workspace"][0] == "0" and int(c_output["scheme_workspace"][1]) > 0
    assert c_output["bad_density"] == [str(_lib.VSA_ERR_INVALID_ARG)]
    lib = _lib.load()
    cands = (ctypes.c_int32 * 6)(4, 4, 8, 1, 8, 16)
    ws, offs = ctypes.c_size_t(), (ctypes.c_size_t * 4)()
    assert lib.vsa_scheme_means_workspace(ctypes.byref(shape), cands, 2, ctypes.byref(ws), offs) == 0
    assert c_output["scheme_means_workspace"] == ["0", str(ws.value)] + [str(o) for o in offs]
    assert int(c_output["noalloc_max_ws"][0]) == _lib.VSA_PLAN_NOALLOC_MAX_WS
    assert [int(x) for x in c_output["calib_limits"]] == [_lib.VSA_CALIB_POOL_BYTES, _lib.VSA_CALIB_MAX_WORKGROUPS,
                                                           _lib.VSA_CALIB_MAX_ITERS]
    bad = str(_lib.VSA_ERR_INVALID_ARG)
    for key in ("plan_heads_no_list", "plan_heads_repeated", "attn_heads_null", "plan_noalloc_null", "calib_null"):
        assert c_output[key] == [bad], key
    assert " ".join(c_output["status_str"]) == "index capacity too small"
