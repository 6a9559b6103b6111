"""The C ABI from plain C: tests/abi_c_check.c, compiled as pedantic C99
against include/mla.h and linked with libmla.so, calls the host-only entry
points; its results must equal the Python binding's (same library)."""

import os
import subprocess

import pytest

import mla_latent_kv_lat_amd as mla
from mla_latent_kv_lat_amd import binding
from tests._cprog import program


@pytest.fixture(scope="module")
def c_output(tmp_path_factory):
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("library not built")
    exe = program("abi_c_check", str(tmp_path_factory.mktemp("abi_c")))
    if exe is None:
        pytest.skip("no C compiler")
    out = subprocess.run([exe], check=True, capture_output=True, text=True, timeout=60).stdout
    return [line.split() for line in out.splitlines()]


def _get(lines, key):
    return [ln[1:] for ln in lines if ln[0] == key]


def test_status_strings_match(c_output):
    rows = _get(c_output, "status")
    assert len(rows) == 6
    for code, *text in rows:
        got = " ".join(text)
        assert got == binding._lib.mla_status_string(int(code)).decode()
        assert got.split(":")[0] == binding.STATUS[int(code)]


def test_split_plan_matches_binding(c_output):
    assert _get(c_output, "split_plan_status") == [["0"]]
    fu, lu, ft = mla.mla_split_plan([100, 0, 1000, 64], 7)
    rows = _get(c_output, "plan")
    assert [[int(x) for x in r] for r in rows] == [[b, int(fu[b]), int(lu[b]), int(ft[b])]
                                                   for b in range(4)]
    assert _get(c_output, "split_plan_zero_splits") == [["1"]]  # MLA_ERR_INVALID_ARG


def test_workspace_bytes_match_binding(c_output):
    assert _get(c_output, "workspace_status") == [["0"]]
    d = mla.dims(64, 1, 128, 128, 64, 512, 128, mla.BF16, mla.BF16)
    ob, lb = mla.mla_workspace_bytes(d, 256)
    assert _get(c_output, "workspace") == [[str(ob), str(lb)]]
    assert _get(c_output, "workspace_bad_dims") == [["1"]]
