"""The oracle (oracle/qmv_oracle.c) and the library's host-side rules
(block_quant_weight_amd/csrc/qmv_host.cpp) under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

- The oracle is rebuilt with the sanitizers and the oracle's own pin tests
  (tests/test_oracle*.py but the mutants) run against that build in a child
  process with the ASan runtime preloaded; any out-of-bounds access or
  undefined behaviour aborts the child.
- The host rules are built with the sanitizers into a small driver
  (tests/san_host_driver.cpp) that runs a battery of cases: sizes and class
  rules are compared with the oracle's, buffer checks run on exact-size heap
  buffers (a read past the caller's byte count is caught), and the row
  exponents of seeded scale arrays (with inf, NaN and subnormal patterns)
  are compared with a numpy computation of the same rule."""
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "block_quant_weight_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g", "-O1"]


def asan_runtime():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def builds(tmp_path_factory):
    if shutil.which("gcc") is None or shutil.which("g++") is None or asan_runtime() is None:
        pytest.skip("no gcc sanitizer runtime")
    d = tmp_path_factory.mktemp("san")
    lib = str(d / "libqmv_oracle_san.so")
    subprocess.check_call(["gcc", *SAN, "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                           "-fPIC", "-shared", "-o", lib, os.path.join(ROOT, "oracle", "qmv_oracle.c"),
                           "-lm"])
    drv = str(d / "san_host_driver")
    subprocess.check_call(["g++", *SAN, "-std=c++17", "-I", os.path.join(ROOT, "include"),
                           "-I", CSRC, "-o", drv, os.path.join(HERE, "san_host_driver.cpp"),
                           os.path.join(CSRC, "qmv_host.cpp")])
    return lib, drv


def san_env():
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:allocator_may_return_null=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


def test_oracle_pins_under_sanitizers(builds):
    lib, _ = builds
    env = san_env()
    env["LD_PRELOAD"] = asan_runtime()
    env["QMV_ORACLE_LIB"] = lib
    # (the mutant tests load their own unsanitized copies of the oracle)
    files = sorted(os.path.join(HERE, f) for f in os.listdir(HERE)
                   if f.startswith("test_oracle") and f.endswith(".py") and "mutant" not in f)
    p = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider", *files],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1500)
    tail = (p.stdout + p.stderr)[-4000:]
    assert p.returncode == 0, tail
    assert "passed" in p.stdout and "ERROR: AddressSanitizer" not in p.stderr, tail


def drive(drv, lines):
    p = subprocess.run([drv], input="\n".join(lines) + "\n", env=san_env(),
                       capture_output=True, text=True, timeout=600)
    assert p.returncode == 0, p.stderr[-4000:]
    out = p.stdout.strip().split("\n")
    assert len(out) == len(lines)
    return out


STATUS = {0: "ok", -1: "arg", -2: "format", -3: "shape"}
SHAPES = [(1, 32), (3, 32), (5, 96), (4096, 4096), (248320, 1024), (7, 4064),
          (16777216, 32), (1, 16777216), (0, 32), (1, 0), (1, 48), (16777217, 32),
          (32, 16777248), (4294967295, 32)]


def test_host_sizes_and_class_rule(builds):
    _, drv = builds
    lines, want = [], []
    for wt in (0, 1, 2, 3):
        for sf in (0, 1, 2):
            for R, C in SHAPES:
                R32, C32 = min(R, 2 ** 32 - 1), min(C, 2 ** 32 - 1)
                lines.append(f"span {wt} {sf} {R32} {C32}")
                st, s = O.span(wt, sf, R32, C32)
                want.append((st, s))
        for R, C in SHAPES:
            lines.append(f"gspan {wt} {min(R, 2 ** 32 - 1)} {C}")
            want.append(("g",) + O.gguf_span(wt, min(R, 2 ** 32 - 1), C))
    for fw in (0, 1, 2, 3):
        for mask in (0, 8, 64, 8 | 64, 0xFF, 0xFFFFFFFF):
            for bit in (0, 1, 2, 4, 8, 16, 32, 64, 128, 3, 1 << 31):
                for shared in (0, 1, 2):
                    lines.append(f"class {fw} {mask} {bit} {shared}")
                    want.append(("c",) + O.class_wtype(fw, mask, bit, shared))
    out = drive(drv, lines)
    for line, got, w in zip(lines, out, want):
        f = got.split()
        if w[0] == "g":
            assert STATUS[int(f[0])] == w[1], line
            if w[1] == "ok":
                assert int(f[1]) == w[2], line
        elif w[0] == "c":
            assert STATUS[int(f[0])] == w[1], line
            if w[1] == "ok":
                assert int(f[1]) == w[2], line
        else:
            st, s = w
            assert STATUS[int(f[0])] == st, line
            if st == "ok":
                assert [int(v) for v in f[1:]] == [s["q_bytes"], s["d_offset"], s["d_bytes"],
                                                   s["min_span"]], line


def test_host_buffer_checks_read_only_the_given_bytes(builds):
    _, drv = builds
    lines, want = [], []
    for wt, sf, R, C in [(1, 0, 3, 64), (1, 1, 5, 96), (2, 1, 7, 32), (2, 0, 2, 4096), (1, 1, 1, 32)]:
        st, s = O.span(wt, sf, R, C)
        for n in (0, 1, s["min_span"] - 1, s["min_span"], s["min_span"] + 5):
            for plant in (-1, 0, s["q_bytes"] - 1, s["q_bytes"], n - 1):
                lines.append(f"check {wt} {sf} {R} {C} {n} {plant}")
                img = np.zeros(max(n, 1), dtype=np.uint8)
                if 0 <= plant < n:
                    img[plant] = 0x80
                want.append(O.check_image(wt, sf, R, C, img, n))
        ok, gb = O.gguf_span(wt, R, C)
        for n in (0, gb - 1, gb, gb + 3):
            for plant in (-1, 2, gb - 1, n - 1):
                lines.append(f"gcheck {wt} {R} {C} {n} {plant}")
                a = np.zeros(max(n, 1), dtype=np.uint8)
                if 0 <= plant < n:
                    a[plant] = 0x80
                want.append(O.check_gguf(wt, R, C, a, n))
    out = drive(drv, lines)
    for line, got, w in zip(lines, out, want):
        assert STATUS[int(got)] == w, (line, got, w)


def row_exponents(wt, sf, R, C, gguf, seed):
    """numpy: the exponent of the largest finite scale magnitude per row and
    over the matrix (0 if none), from the same splitmix64 bytes."""
    st, s = O.span(wt, 1 if gguf else sf, R, C)
    n = O.gguf_span(wt, R, C)[1] if gguf else s["min_span"]
    mask = (1 << 64) - 1
    state, out = seed, bytearray()
    while len(out) < n:
        state = (state + 0x9E3779B97F4A7C15) & mask
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & mask
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & mask
        out.append((z ^ (z >> 31)) & 0xFF)
    buf = np.frombuffer(bytes(out[:n]), dtype=np.uint8)
    nblk = C // 32
    if gguf:
        stride = 34 if wt == 1 else 18
        starts = np.arange(R * nblk) * stride
        d = (buf[starts].astype(np.uint16) | (buf[starts + 1].astype(np.uint16) << 8)).view(np.float16)
    else:
        raw = buf[s["d_offset"]:s["d_offset"] + s["d_bytes"]].copy()
        d = raw.view(np.float16 if sf else np.float32)
    a = np.abs(d.astype(np.float64)).reshape(R, nblk)
    a[~np.isfinite(a)] = 0.0

    def ex(m):
        return 0 if m == 0 else int(np.frexp(m)[1])
    return ex(a.max()), [ex(v) for v in a.max(axis=1)]


def test_host_row_exponents(builds):
    _, drv = builds
    cases = [(2, 1, 5, 64, 0, 11), (1, 0, 7, 96, 0, 12), (1, 1, 3, 4096, 0, 13),
             (2, 1, 9, 256, 1, 14), (1, 1, 4, 128, 1, 15), (2, 0, 2, 32, 0, 16)]
    out = drive(drv, [f"exps {wt} {sf} {R} {C} {g} {seed}" for wt, sf, R, C, g, seed in cases])
    for (wt, sf, R, C, g, seed), got in zip(cases, out):
        f = [int(v) for v in got.split()]
        m, rows = row_exponents(wt, sf, R, C, g, seed)
        assert f[0] == m and f[1:] == rows, (wt, sf, R, C, g)


def test_host_status_text(builds):
    _, drv = builds
    out = drive(drv, [f"status {k}" for k in (0, -1, -2, -3, -4, -5, 7)])
    assert all(o.strip() for o in out)
