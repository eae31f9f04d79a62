"""The host side of the library (block manager, copy-on-write and rollback,
prefix cache, host-tier bookkeeping) under AddressSanitizer and
UndefinedBehaviorSanitizer.

The host sources are built with g++ -fsanitize=address,undefined into a
separate host-only library (its device entry points all fail with
KV_ERR_UNSUPPORTED), and the CPU tests of the C ABI -- random programs with
out-of-memory rollback, fenced release, prefix-cache insert/evict programs and
swap bookkeeping -- run against it in a child process with the ASan runtime
preloaded.  Any invalid access, use after free, double free or undefined
behaviour in that code aborts the child and fails this test.  Refcount and
free-list bookkeeping is where such errors hide ([BT] §08 copy-on-write
reference counts, §13 debugging checklist).
"""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

CSRC = os.path.join(ROOT, "pagedattention_decode_amd", "csrc")
HOST_TESTS = ["tests/test_allocator_abi.py", "tests/test_prefix_cache.py", "tests/test_swap_abi.py"]


def build_host_sanitized():
    """pool.cpp and prefix_cache.cpp (every host-only source of the library) plus
    san_stubs.cpp, built by g++ with ASan and UBSan into _build/; no device code."""
    out_dir = os.path.join(ROOT, "_build")
    os.makedirs(out_dir, exist_ok=True)
    lib = os.path.join(out_dir, "libpagedkv_host_asan.so")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    srcs = [os.path.join(CSRC, s) for s in ("pool.cpp", "prefix_cache.cpp", "san_stubs.cpp")]
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", f"-I{rocm}/include", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           *srcs, f"-L{rocm}/lib", "-lamdhip64", f"-Wl,-rpath,{rocm}/lib", "-o", lib + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    os.replace(lib + ".tmp", lib)
    return lib


def sanitizer_env(lib):
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()
    assert os.path.isabs(asan) and os.path.exists(asan), "the ASan runtime of g++ is missing"
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": asan,
        # the interpreter itself is not instrumented and keeps its objects until exit
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
        "PAGEDKV_LIBRARY": lib,
    })
    return env


def test_host_code_under_address_and_undefined_sanitizers():
    lib = build_host_sanitized()
    env = sanitizer_env(lib)
    # the child really runs instrumented: the ASan runtime is mapped and the
    # binding loads the sanitized library, which carries ASan's instrumentation
    probe = ("import ctypes, sys; sys.path.insert(0, '.');"
             "from pagedattention_decode_amd import binding as B;"
             "h = B.lib(); maps = open('/proc/self/maps').read();"
             "assert 'libasan' in maps and B.lib_path() == sys.argv[1];"
             "assert 'libpagedkv_host_asan' in maps;"
             "ctypes.CDLL(None).__asan_report_load1;"
             "print('sanitized library loaded')")
    r = subprocess.run([sys.executable, "-c", probe, lib], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and "sanitized library loaded" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *HOST_TESTS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = r.stdout[-3000:] + r.stderr[-6000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
    assert " passed" in r.stdout, tail
