"""The library's host C++ (packer, blob check, status strings) built with
AddressSanitizer and UndefinedBehaviorSanitizer (g++, CPU only) and driven
by tests/sanitize_driver.cpp: packs seeded layers (every width, ragged dout,
edge values) whose bytes must equal the oracle packer's, then checks
corrupted blobs and bad arguments.  Any sanitizer report fails the test."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import synth
from oracle import fmt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "spectral_expert_gemv_amd", "csrc")
FLAGS = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-pthread"]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    cxx = shutil.which("g++")
    if not cxx:
        pytest.skip("g++ not found")
    out = str(tmp_path_factory.mktemp("asan") / "sanitize_driver")
    cmd = [cxx] + FLAGS + ["-I", os.path.join(ROOT, "include"), "-I", CSRC,
                           os.path.join(CSRC, "pack.cpp"), os.path.join(CSRC, "common.cpp"),
                           os.path.join(ROOT, "tests", "sanitize_driver.cpp"), "-o", out]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    return out


def _edge_layer(E=3, r=64, dout=100, seed=11):
    rng = np.random.default_rng(seed)
    p = rng.standard_normal((E, r, dout)).astype(np.float32)
    p /= np.linalg.norm(p, axis=2, keepdims=True)
    bits = rng.choice([0, 1, 2, 3, 4, 6, 8, 16], size=(E, r)).astype(np.uint8)
    bits[1] = 0                                   # an expert with no stored column
    p[0, 0] = 0.25                                # constant column
    p[0, 1] = 0.0                                 # zero column
    p[0, 2, ::2] = 60000.0                        # the largest accepted magnitude
    p[0, 3] = np.float32(1e-42)                   # subnormal float32
    p[0, 4, :] = -0.0                             # signed zeros
    bits[0, :5] = [1, 4, 16, 8, 2]
    a = rng.lognormal(0, 0.5, (E, r)).astype(np.float32)
    a[0, 5] = 0.0
    return p, a, bits


def _cases():
    L = synth.make_layer(synth.LAYERS["tiny"])
    yield "tiny_gate", L.p["gate"], L.a["gate"], L.bits["gate"]
    yield "edge", *_edge_layer()
    rng = np.random.default_rng(5)
    p = rng.standard_normal((1, 1, 1)).astype(np.float32)
    yield "one", p / np.abs(p), np.ones((1, 1), np.float32), np.full((1, 1), 3, np.uint8)


@pytest.mark.parametrize("name", ["tiny_gate", "edge", "one"])
def test_packer_under_sanitizers(driver, tmp_path, name):
    case = {c[0]: c[1:] for c in _cases()}[name]
    p, a, bits = case
    E, r, dout = p.shape
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(fin, "wb") as f:
        f.write(np.ascontiguousarray(p, np.float32).tobytes())
        f.write(np.ascontiguousarray(a, np.float32).tobytes())
        f.write(np.ascontiguousarray(bits, np.uint8).tobytes())
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r_ = subprocess.run([driver, str(E), str(dout), str(r), str(fin), str(fout)],
                        stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env,
                        timeout=300)
    assert r_.returncode == 0, r_.stdout
    assert "Sanitizer" not in r_.stdout and "runtime error" not in r_.stdout, r_.stdout
    got = fout.read_bytes()
    assert got == fmt.pack(p, a, bits)
