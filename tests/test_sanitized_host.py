"""The library's host code (mask builders, schedules, split unit lists,
transposes, argument checks) built with AddressSanitizer and
UndefinedBehaviorSanitizer and driven by a seeded random-CSR exerciser
(tests/c_abi/mask_fuzz.cpp, results compared with brute-force dense
matrices) and by the plain C caller (tests/c_abi/host_calls.c).  Host code
only: the .hip kernels are left out of this link (tests/c_abi/
host_only_launchers.cpp stands in for their launchers, which a host without
a device never reaches)."""

import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_jvp_causal_attn_amd", "csrc")
CABI = os.path.join(ROOT, "tests", "c_abi")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    gxx, gcc = shutil.which("g++"), shutil.which("gcc")
    if gxx is None or gcc is None or not os.path.exists(os.path.join(ROCM, "include", "hip")):
        pytest.skip("needs g++, gcc and the HIP headers")
    out = tmp_path_factory.mktemp("san")
    inc = ["-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), "-I",
           os.path.join(ROOT, "include"), "-I", CSRC]
    units = [(gxx, os.path.join(CSRC, "attn_jvp_mask.cpp"), ["-std=c++17"] + inc),
             (gxx, os.path.join(CSRC, "attn_jvp_api.cpp"), ["-std=c++17"] + inc),
             (gxx, os.path.join(CABI, "host_only_launchers.cpp"), ["-std=c++17"] + inc),
             (gxx, os.path.join(CABI, "mask_fuzz.cpp"), ["-std=c++17", "-Wall"] + inc),
             (gcc, os.path.join(CABI, "host_calls.c"),
              ["-std=c99", "-I", os.path.join(ROOT, "include")])]

    def compile_unit(u):
        cc, src, flags = u
        obj = str(out / (os.path.basename(src) + ".o"))
        r = subprocess.run([cc] + flags + SAN + ["-c", src, "-o", obj], capture_output=True,
                           text=True)
        assert r.returncode == 0, r.stderr
        return obj

    with cf.ThreadPoolExecutor(len(units)) as ex:
        objs = list(ex.map(compile_unit, units))
    lib = objs[:3]
    link = ["-L", os.path.join(ROCM, "lib"), "-lamdhip64",
            "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    exes = {}
    for name, main in (("mask_fuzz", objs[3]), ("host_calls", objs[4])):
        exe = str(out / name)
        r = subprocess.run([gxx] + SAN + lib + [main, "-o", exe] + link, capture_output=True,
                           text=True)
        assert r.returncode == 0, r.stderr
        exes[name] = exe
    return exes


@pytest.mark.parametrize("seed", [1, 20240607])
def test_random_csr_masks_under_sanitizers(sanitized, seed):
    r = subprocess.run([sanitized["mask_fuzz"], "2000", str(seed)], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


def test_plain_c_caller_under_sanitizers(sanitized):
    r = subprocess.run([sanitized["host_calls"]], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
