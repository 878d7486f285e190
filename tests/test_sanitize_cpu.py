"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

g++ builds the tile scheduler (``mla_sched.cpp``) and the entry points'
argument validation (``mla_api.cpp``) with ``-fsanitize=address,undefined``
and no recovery, linked with ``tests/sanitize/san_driver.cpp`` and stub kernel
launchers that abort if reached.  No GPU and no HIP runtime are involved: the
scheduler is host code, and every decode call the driver makes is one that
validation rejects.

* The scheduler writes into a heap array of exactly the capacity
  ``mla_metadata_capacity`` promises, for hypothesis-generated and edge-case
  lengths, and its output must equal the reference scheduler's bit for bit.
* Every rejection case returns its error code without reaching a launcher.

Any sanitizer report aborts the driver, which fails the test.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle.schedule import ref_schedule

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_paged_kv_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "sanitize")
FLAGS = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all"]
INCLUDES = ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{ROOT}/include", f"-I{CSRC}"]
ENV = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:halt_on_error=1:detect_leaks=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"):
        pytest.skip("g++ or the HIP headers are missing")
    out = tmp_path_factory.mktemp("san")
    objs = []
    for src in (os.path.join(CSRC, "mla_sched.cpp"), os.path.join(CSRC, "mla_api.cpp"),
                os.path.join(HERE, "launch_stubs.cpp"), os.path.join(HERE, "san_driver.cpp")):
        obj = str(out / (os.path.basename(src) + ".o"))
        subprocess.run([gxx, *FLAGS, *INCLUDES, "-c", src, "-o", obj], check=True)
        objs.append(obj)
    exe = str(out / "san_driver")
    subprocess.run([gxx, "-fsanitize=address,undefined", *objs, "-o", exe], check=True)
    return exe


def run(driver, text: str) -> list[str]:
    r = subprocess.run([driver], input=text, capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0 and "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, \
        r.stderr[-4000:]
    return r.stdout.splitlines()


def check_schedules(driver, cases):
    text = "".join(f"S {P} {rows} {len(lens)} {' '.join(map(str, lens))}\n" for lens, P, rows in cases)
    lines = run(driver, text)
    assert len(lines) == len(cases)
    for (lens, P, rows), line in zip(cases, lines):
        vals = [int(v) for v in line.split()]
        rc, n = vals[0], vals[1]
        assert rc == 0, (lens, P, rows, rc)
        np.testing.assert_array_equal(np.array(vals[2:2 + n], dtype=np.int32),
                                      ref_schedule(lens, P, rows), err_msg=str((lens, P, rows)))


CASE = st.tuples(st.lists(st.integers(0, 20000), min_size=0, max_size=40), st.integers(1, 1100),
                 st.integers(1, 256))


@settings(max_examples=5, deadline=None)
@given(cases=st.lists(CASE, min_size=40, max_size=40))
def test_scheduler_under_sanitizers_matches_reference(driver, cases):
    check_schedules(driver, cases)


def test_scheduler_edge_cases_under_sanitizers(driver):
    rng = np.random.default_rng(5)
    cases = [
        ([], 1, 16), ([], 1024, 128), ([0], 1, 1), ([0] * 7, 300, 64), ([1], 1024, 256),
        ([1 << 24], 1024, 128), ([1 << 24, 1, 0], 7, 16), ([64] * 4096, 1024, 64),
        (rng.integers(0, 4097, 4096).tolist(), 256, 128), ([131072] * 8 + [5] * 8, 251, 64),
        ([4096] * 128, 128, 256), (rng.integers(0, 100, 300).tolist(), 1, 33),
    ]
    check_schedules(driver, cases)


EXPECTED = {
    "paged_h_kv": -2, "paged_page": -2, "paged_d_qk": -2, "paged_dv_gt_dqk": -1,
    "paged_misaligned": -1, "paged_no_workspace": -1, "paged_small_workspace": -3,
    "paged_batch": -1, "paged_s_q": -1, "paged_h_q": -1, "paged_causal": -1, "paged_scale": -1,
    "paged_null_table": -1, "paged_bt_stride": -1, "paged_nblk": -1, "paged_negative_batch": -1,
    "paged_bad_header": -1, "paged_bad_slots": -1, "paged_null_info": -1, "paged_fp8_d512": -2,
    "paged_f16_h_kv": -2, "splitkv_paged_batch": -1, "sparse_null_indices": -1,
    "sparse_topk": -1, "sparse_batch": -1, "sparse_h_q": -1, "sparse_dv": -2,
    "sparse_small_workspace": -3, "sparse_nblk": -1, "prefill_s_kv": -1, "prefill_topk": -1,
    "combine_null_meta": -1, "combine_small_workspace": -3,
}


def test_validation_under_sanitizers(driver):
    got = dict(line.split() for line in run(driver, "R\n"))
    assert "setup_failed" not in got
    for name, code in EXPECTED.items():
        assert int(got[name]) == code, name
    for c in (0, 1, -1, -2, -3, -4, -99):
        assert got[f"strerror_{c}"] == "1"
