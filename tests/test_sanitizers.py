"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only, no GPU).

* The fp64 oracle (oracle/gdr2_oracle.c) is rebuilt with gcc -fsanitize=address,undefined
  and run in a child process on small ragged shapes (T not a multiple of anything, T = 1,
  d_k != d_v, with and without initial state); its outputs must equal the plain build's
  bit for bit, and any sanitizer report aborts the child.
* The HIP library is rebuilt with its host code sanitized (hipcc -Xarch_host
  -fsanitize=...; device code unchanged) and tests/test_abi.py, which drives every entry
  point's argument checking, workspace sizing and error strings, runs against it in a
  child process with the sanitizer runtime preloaded.

Both children run with halt_on_error, so a single report fails the test.
"""
import glob
import os
import shutil
import subprocess
import sys
import textwrap

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_gdr2_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}

SHAPES = [  # B, T, H, DK, DV, with h0
    (1, 1, 1, 4, 4, False),
    (2, 37, 3, 8, 12, True),
    (1, 70, 2, 16, 8, True),
]


def _gcc_runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _inputs(B, T, H, DK, DV, with_h0, seed):
    rng = np.random.default_rng(seed)
    x = {"q": rng.standard_normal((B, T, H, DK)), "k": rng.standard_normal((B, T, H, DK)) / np.sqrt(DK),
         "v": rng.standard_normal((B, T, H, DV)), "g": -rng.uniform(0.0, 1.0, (B, T, H, DK)),
         "b": rng.uniform(0.0, 1.0, (B, T, H, DK)), "w": rng.uniform(0.0, 1.0, (B, T, H, DV)),
         "do": rng.standard_normal((B, T, H, DV))}
    x["h0"] = rng.standard_normal((B, H, DK, DV)) if with_h0 else None
    return x


CHILD = textwrap.dedent("""
    import ctypes, sys
    import numpy as np
    sys.path.insert(0, sys.argv[1])
    ctypes.CDLL(None).__asan_init  # the sanitizer runtime is in the process
    import oracle
    d = np.load(sys.argv[2])
    for i in range(int(d["n"])):
        x = {k: d["%d_%s" % (i, k)] for k in ("q", "k", "v", "g", "b", "w", "do")}
        h0 = d["%d_h0" % i] if ("%d_h0" % i) in d else None
        o, ht = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["b"], x["w"], h0)
        gr = oracle.bwd(x["q"], x["k"], x["v"], x["g"], x["b"], x["w"], h0, x["do"], ht)
        out = {"o": o, "ht": ht}
        out.update(gr)
        for k, v in out.items():
            if not np.array_equal(v, d["%d_ref_%s" % (i, k)]):
                raise SystemExit("sanitized oracle differs: shape %d, %s" % (i, k))
    print("sanitized oracle ok")
""")


def test_oracle_under_asan_ubsan(tmp_path):
    import oracle
    asan = _gcc_runtime("libasan.so")
    if asan is None or shutil.which("gcc") is None:
        pytest.skip("gcc's sanitizer runtime is not installed")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
                    "-shared", "-std=c11", "-o", lib, os.path.join(ROOT, "oracle", "gdr2_oracle.c"), "-lm"],
                   check=True)
    data = {"n": np.array(len(SHAPES))}
    for i, (B, T, H, DK, DV, with_h0) in enumerate(SHAPES):
        x = _inputs(B, T, H, DK, DV, with_h0, seed=100 + i)
        o, ht = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["b"], x["w"], x["h0"])
        gr = oracle.bwd(x["q"], x["k"], x["v"], x["g"], x["b"], x["w"], x["h0"], x["do"], ht)
        ref = {"o": o, "ht": ht}
        ref.update(gr)
        for k, v in x.items():
            if v is not None:
                data["%d_%s" % (i, k)] = v
        for k, v in ref.items():
            data["%d_ref_%s" % (i, k)] = v
    npz = str(tmp_path / "cases.npz")
    np.savez(npz, **data)
    env = dict(os.environ, LD_PRELOAD=asan, GDR2_ORACLE_LIB=lib, OMP_NUM_THREADS="2", **SAN_ENV)
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT, npz], env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "sanitized oracle ok" in r.stdout


def test_abi_under_asan_ubsan(tmp_path):
    rts = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not os.path.exists(HIPCC) or not rts:
        pytest.skip("hipcc or its sanitizer runtime is not installed")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Wno-unused-function",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    from gated_delta_rule_gdr2_amd.build import SOURCES
    procs, objs = [], []
    for src in SOURCES:
        obj = str(tmp_path / (src + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([HIPCC] + flags + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    for p, src in zip(procs, SOURCES):
        _, err = p.communicate(timeout=900)
        assert p.returncode == 0, "hipcc failed for %s:\n%s" % (src, err[-3000:])
    lib = str(tmp_path / "libgdr2_san.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", lib] + objs, check=True,
                   capture_output=True)
    env = dict(os.environ, LD_PRELOAD=sorted(rts)[-1], GDR2_LIB=lib, **SAN_ENV)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-x",
                        "-p", "no:cacheprovider"], env=env, capture_output=True, text=True, timeout=900, cwd=ROOT)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout
