"""Host sanitizer build of the C-ABI layer (no GPU).

The boundary's own code -- argument validation, workspace size queries, the
host-side group size and tile classes -- is compiled with AddressSanitizer
and UndefinedBehaviorSanitizer on the host side (the kernel launchers are
replaced by stand-ins that abort if reached) and driven through every
rejection path and the extreme sizes by tests/host_sanitize/abi_validation.cpp.
Any out-of-bounds access, signed overflow, bad shift, invalid enum load or
other undefined behaviour in those paths fails the test."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rope_context_extension_jl_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

pytestmark = pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC),
                                reason="hipcc not available")


def _stubs(path):
    """Definitions for every launcher declared in jl_internal.hpp: each aborts."""
    text = open(os.path.join(CSRC, "jl_internal.hpp")).read()
    decls = re.findall(r"hipError_t\s+(launch_\w+)\(([^;]*?)\);", text, flags=re.S)
    assert len(decls) >= 10, "launcher declarations not found"
    lines = ["#include <cstdio>", "#include <cstdlib>", '#include "jl_internal.hpp"',
             "namespace jl {"]
    for name, params in decls:
        lines.append(f'hipError_t {name}({params}) {{ std::fprintf(stderr, "{name} reached\\n"); '
                     "std::abort(); }")
    lines.append("}  // namespace jl")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def test_abi_validation_is_clean_under_asan_and_ubsan(tmp_path):
    stubs = str(tmp_path / "stubs.cpp")
    exe = str(tmp_path / "abi_validation")
    _stubs(stubs)
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           os.path.join(CSRC, "api.cpp"), stubs,
           "-x", "c++", os.path.join(ROOT, "tests", "host_sanitize", "abi_validation.cpp"),
           "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ)
    # the HIP runtime's own allocations are not the code under test; a library
    # the environment preloads may precede the sanitizer runtime
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = run.stdout + run.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert "runtime error" not in out, out[-4000:]
    assert run.returncode == 0, out[-4000:]
    assert "abi_validation: 0 failure(s)" in out, out[-4000:]
