"""The CPU code under AddressSanitizer and UndefinedBehaviorSanitizer.

Three libraries are rebuilt with both sanitizers into a temporary folder:
  - the oracle (oracle.c) and the host generator (synth.c), with gcc;
  - libmoe with the host code of api.hip instrumented (argument checks,
    workspace layout, the expert tier's repin policy), compiled for the host
    alone (api.hip holds no kernels) and linked with the ordinary objects of
    the kernel files, with clang's runtime.
Each test runs existing CPU test files in a child process that loads the
instrumented library (ORACLE_LIB / SYNTH_HOST_LIB / MOE_LIB) with the matching
sanitizer runtime preloaded; a report of either sanitizer aborts the child.
The child first checks that the instrumented libraries are the ones mapped.
A planted heap overflow and a planted signed overflow, each in a scratch C
file built the same way, show that the runtimes are live."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
GCC_SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined"]


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-4000:])
    return r


def gcc_runtime():
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()


def clang_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.fixture(scope="module")
def san(tmp_path_factory):
    d = tmp_path_factory.mktemp("san")
    out = {}
    run(["gcc", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math", "-ffp-contract=off", *GCC_SAN,
         os.path.join(ROOT, "oracle", "oracle.c"), "-o", str(d / "liboracle.so"), "-lm"])
    run(["gcc", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math", *GCC_SAN,
         os.path.join(ROOT, "synth", "synth.c"), "-o", str(d / "libsynth.so"), "-lm"])
    out["oracle"], out["synth"] = str(d / "liboracle.so"), str(d / "libsynth.so")
    out["dir"] = d
    return out


def child_env(preload, **libs):
    env = dict(os.environ)
    env.update(libs)
    env["LD_PRELOAD"] = preload
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["PYTHONDONTWRITEBYTECODE"] = "1"
    return env


MAPPED = """
import sys
sys.path.insert(0, %r)
want = sys.argv[1:]
for mod in ("oracle", "synth", "moe"):
    if mod == "oracle":
        import oracle; oracle.lib()
    elif mod == "synth":
        import synth; synth.key(0, 0)
    else:
        import os
        if os.environ.get("MOE_LIB"):
            from quantized_moe_noaux_amd import moe
maps = open("/proc/self/maps").read()
missing = [w for w in want if w not in maps]
assert not missing, ("not mapped", missing)
print("mapped:", want)
""" % ROOT


def run_tests(env, files, want):
    run([sys.executable, "-c", MAPPED, *want], env=env, cwd=ROOT)
    r = run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu", *files],
            env=env, cwd=ROOT)
    assert "passed" in r.stdout and "runtime error" not in r.stderr + r.stdout


def test_oracle_and_generator_under_sanitizers(san):
    env = child_env(gcc_runtime(), ORACLE_LIB=san["oracle"], SYNTH_HOST_LIB=san["synth"])
    run_tests(env, ["tests/test_oracle_pins.py", "tests/test_oracle_accept.py", "tests/test_synth.py",
                    "tests/test_equivalence.py"], [san["oracle"], san["synth"]])


def test_library_host_code_under_sanitizers(san):
    rt = clang_runtime()
    if rt is None:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    import importlib.util
    spec = importlib.util.spec_from_file_location("_moe_build", os.path.join(ROOT, "quantized_moe_noaux_amd",
                                                                            "_build.py"))
    build_mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(build_mod)
    objd = os.path.join(ROOT, "quantized_moe_noaux_amd", "_obj")
    # every source but api.hip, as the ordinary build compiled it
    kernels = [os.path.join(objd, f.replace(".hip", ".o")) for f in build_mod.SOURCES if f != "api.hip"]
    if not all(os.path.exists(o) for o in kernels):
        build_mod.build()
    d = san["dir"]
    api = str(d / "api_host.o")
    run([HIPCC, "--offload-arch=gfx950", "--cuda-host-only", "-std=c++17", "-fPIC", "-fno-gpu-rdc",
         "-O1", "-g", "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address,undefined",
         "-Xarch_host", "-fno-sanitize-recover=undefined",
         "-c", os.path.join(ROOT, "quantized_moe_noaux_amd", "csrc", "api.hip"), "-o", api])
    lib = str(d / "libmoe.so")
    run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan", "-Xarch_host",
         "-fsanitize=address,undefined", api, *kernels, "-o", lib])
    run_tests(child_env(rt, MOE_LIB=lib), ["tests/test_abi.py", "tests/test_tier_plan.py"], [lib])


PLANTED = r"""
#include <stdlib.h>
#include <limits.h>
int heap_overflow(int n) { int *a = malloc(sizeof(int) * n); int v = a[n]; free(a); return v; }
int signed_overflow(int x) { return x + INT_MAX; }
"""


@pytest.mark.parametrize("fn,report", [("heap_overflow", "heap-buffer-overflow"),
                                       ("signed_overflow", "signed integer overflow")])
def test_runtimes_catch_planted_errors(san, fn, report):
    d = san["dir"]
    src, so = d / "planted.c", d / "libplanted.so"
    if not so.exists():
        src.write_text(PLANTED)
        run(["gcc", "-std=c99", "-fPIC", "-shared", *GCC_SAN, str(src), "-o", str(so)])
    code = "import ctypes; print(ctypes.CDLL(%r).%s(4))" % (str(so), fn)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       env=child_env(gcc_runtime()))
    assert r.returncode != 0 and report in r.stderr, r.stderr[-2000:]
