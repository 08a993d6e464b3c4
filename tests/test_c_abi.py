"""The library used from plain C (tests/c_abi/consumer.c): the header and the
shared library are all a C caller needs.  The host test runs the program's
host-only calls (version, workspace sizes, argument checks) on any machine;
the GPU test runs one W4A4 layer step (route prep -> INT4 GEMM -> combine)
from C on the 64-token workload and compares what it wrote with the oracle."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CDIR = os.path.join(ROOT, "tests", "c_abi")
EXE = os.path.join(CDIR, "moeq_consumer")


def consumer():
    """The built program; built here only when it is missing."""
    if not os.path.exists(EXE):
        import quantized_moe_grouped_route_amd as mq
        if not os.path.exists(mq.LIB_PATH):
            from quantized_moe_grouped_route_amd import build as b
            b.build()
        subprocess.run(["make", "-C", CDIR], check=True, capture_output=True)
    return EXE


def test_c_consumer_host_calls():
    r = subprocess.run([consumer(), "host"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    got = {}
    for ln in r.stdout.splitlines():
        key, _, val = ln.partition(" ")
        got[key if key != "ws" else "ws " + " ".join(val.split()[:3])] = val.split()[-1] if key == "ws" else val
    assert got["abi"] == "3"
    import ctypes as C
    import quantized_moe_grouped_route_amd as mq
    L = C.CDLL(mq.LIB_PATH)
    L.moe_route_prep_workspace_bytes.restype = C.c_size_t
    L.moe_route_prep_workspace_bytes.argtypes = [C.c_int64, C.c_int32, C.c_int32]
    for T, k, E in ((64, 2, 4), (8192, 2, 8), (4096, 8, 256)):
        assert int(got[f"ws {T} {k} {E}"]) == L.moe_route_prep_workspace_bytes(T, k, E)
    # MOEQ_EINVAL = 1, MOEQ_EALIGN = 2
    assert got["route_null"] == "1" and got["route_e0"] == "1"
    assert got["int4_n48"] == "2" and got["int4_decode_k384"] == "2"
    assert got["int4_k131072"] == "1"
    assert got["combine_n12"] == "2"
    assert "multiple of 8" in got["last_error"]
    # T = 2^62 with topk = 4: rejected (MOEQ_EINVAL) without forming T*topk
    assert got["ws_huge"] == "0"
    for key in ("route_huge", "noalloc_huge", "combine_huge", "sum_pairs_huge"):
        assert got[key] == "1", key
    # MOEQ_EUNSUPPORTED = 3
    assert got["fp8_n64"] == "2" and got["nvfp4_x_f32"] == "3" and got["quant_k40"] == "2"
    assert got["repack_overlap"] == "1" and got["cast_overlap"] == "1"


def test_c_consumer_host_calls_under_sanitizers():
    """The library's host layer (argument checks, size arithmetic, error
    text) rebuilt by g++ under AddressSanitizer and UndefinedBehaviorSanitizer
    (tests/c_abi/Makefile, target sanitize) runs the host calls with no
    report and prints exactly what the ordinary build prints."""
    import shutil
    import quantized_moe_grouped_route_amd as mq
    kobj = os.path.join(os.path.dirname(mq.LIB_PATH), "_build", "route.hip.o")
    if not (shutil.which("gcc") and shutil.which("g++") and os.path.exists(kobj)):
        pytest.skip("needs gcc/g++ and the kernel objects of a library build")
    r = subprocess.run(["make", "-B", "-s", "-C", CDIR, "sanitize"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="halt_on_error=1:detect_leaks=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    san = subprocess.run([os.path.join(CDIR, "moeq_consumer_san"), "host"], capture_output=True, text=True,
                         timeout=60, env=env)
    assert san.returncode == 0, san.stderr
    assert "runtime error" not in san.stderr and "Sanitizer" not in san.stderr, san.stderr
    plain = subprocess.run([consumer(), "host"], capture_output=True, text=True, timeout=60)
    assert plain.returncode == 0, plain.stderr
    assert san.stdout == plain.stdout


@pytest.mark.gpu
def test_c_consumer_layer_step_matches_oracle(tmp_path):
    d = synth.workload(0)
    T, k, E = d["T"], d["k"], d["E"]
    N, K = d["w"].shape[1], 2 * d["w"].shape[2]
    (tmp_path / "meta.txt").write_text(f"{T} {k} {E} {N} {K}\n")
    for name, arr, dt in (("topk_ids", d["topk_ids"], np.int32), ("a", d["a"], np.uint8),
                          ("a_scale", d["a_scale"], np.float32), ("w", d["w"], np.uint8),
                          ("w_scale", d["w_scale"], np.float32), ("topk_weights", d["topk_weights"], np.float32)):
        np.ascontiguousarray(arr, dt).tofile(tmp_path / f"{name}.bin")
    print(f"C consumer: T={T} topk={k} E={E} N={N} K={K}", flush=True)
    r = subprocess.run([consumer(), "gpu", str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    ref = oracle.int4_layer(d, y_dtype="f32")
    rd = lambda n, dt: np.fromfile(tmp_path / f"{n}.bin", dt)
    assert np.array_equal(rd("offsets", np.int32), ref["offsets"])
    assert np.array_equal(rd("sorted", np.int32), ref["sorted_pair_ids"])
    assert np.array_equal(rd("p2s", np.int32), ref["pair_to_sorted"])
    assert rd("n_invalid", np.int32)[0] == ref["n_invalid"]
    n = int(ref["offsets"][-1])
    y = rd("y", np.float32).reshape(T * k, N).astype(np.float64)
    # sa * sw * acc in fp32: two roundings of an exact integer product
    assert np.all(np.abs(y[:n] - ref["y"]) <= 3e-7 * np.abs(ref["y"]))
    out = rd("out", np.float32).reshape(T, N).astype(np.float64)
    norm = np.linalg.norm(ref["out"], axis=1)
    assert np.all(np.abs(out - ref["out"]).max(axis=1) <= 2e-3 * norm)
