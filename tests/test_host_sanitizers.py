"""CPU: the library's host code - descriptor checks, the capacity rule,
trim, the launch planning of both attention kernels and of the copies, mask
extents - built with AddressSanitizer and UndefinedBehaviorSanitizer (host
code only) and driven with extreme shapes and strides, with no GPU visible
(HIP_VISIBLE_DEVICES empty: a call that passes every check fails at its
launch and nothing runs on a device)
(``tests/sanitize/rbq_host_sanitize.cpp``).  A sanitizer report aborts the
driver; the test needs its exit status 0."""
import concurrent.futures
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rotated_bit_quantized_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"  # the same compiler family as hipcc (one ASan runtime)
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout[-4000:] + r.stderr[-4000:]
    return r


@pytest.mark.skipif(not os.path.exists(CLANGXX) or not os.path.exists(HIPCC),
                    reason="needs ROCm's clang++ and hipcc")
def test_host_code_under_asan_and_ubsan(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", "/opt/rocm/include"]
    objs = []
    host_src = os.path.join(CSRC, "rbq_host.cpp")
    o = str(tmp_path / "rbq_host.o")
    _run([CLANGXX, "-std=c++17", "-O1", "-g", "-ffp-contract=off", *SAN, *inc, "-c", host_src,
          "-o", o])
    objs.append(o)
    # the HIP sources with each sanitizer flag for the host pass only (the
    # device code is built as usual; the driver runs with no visible GPU);
    # the four compiles side by side
    host_san = [x for f in SAN for x in ("-Xarch_host", f)]
    srcs = ("rbq_append.hip", "rbq_attn_mfma.hip", "rbq_attn_prefill.hip", "rbq_attn_tile.hip")
    cmds = [[HIPCC, "--offload-arch=gfx950", "-std=c++17", "-O1", "-g",
             *host_san, *inc, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-c",
             os.path.join(CSRC, src), "-o", str(tmp_path / (src + ".o"))] for src in srcs]
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as pool:
        list(pool.map(_run, cmds))
    objs += [str(tmp_path / (src + ".o")) for src in srcs]
    drv = os.path.join(ROOT, "tests", "sanitize", "rbq_host_sanitize.cpp")
    exe = str(tmp_path / "rbq_host_sanitize")
    _run([CLANGXX, "-std=c++17", "-O1", "-g", *SAN, *inc, drv, *objs, "-o", exe,
          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-6000:]
    assert "ok" in r.stdout
