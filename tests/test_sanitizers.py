"""The host side of the library (argument checks, workspace plan, pass
scheduler, stream state) under the address and undefined-behaviour
sanitizers: tests/sanitize/dry_run_main.cpp walks every workload's launch
schedule in dry-run mode, linked with wvd_api.cpp built with
-fsanitize=address,undefined on its host code (device code is not
instrumented; no GPU is used)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "video_diffusion_vae_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _objects_of_kernels():
    """The kernel objects of the ordinary build (compiled here if absent)."""
    from video_diffusion_vae_amd.csrc import build as b
    objs = [os.path.join(b.BUILD_DIR, n) for n in ("wvd_conv.o", "wvd_aux.o")]
    srcs = [os.path.join(CSRC, n) for n in ("wvd_conv.hip", "wvd_aux.hip")]
    if not all(os.path.exists(o) and os.path.getmtime(o) >= os.path.getmtime(s) for o, s in zip(objs, srcs)):
        b.build()
    return objs


@pytest.mark.skipif(not os.path.exists(HIPCC) or shutil.which("g++") is None, reason="needs hipcc")
def test_host_code_is_clean_under_asan_and_ubsan():
    os.makedirs(OUT, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    common = ["-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    api_o = os.path.join(OUT, "wvd_api_san.o")
    main_o = os.path.join(OUT, "dry_run_main.o")
    exe = os.path.join(OUT, "dry_run_san")
    steps = [
        [HIPCC] + common + san + ["-x", "hip", "-c", os.path.join(CSRC, "wvd_api.cpp"), "-o", api_o],
        [HIPCC] + common + san + ["-c", os.path.join(ROOT, "tests", "sanitize", "dry_run_main.cpp"), "-o", main_o],
        [HIPCC, "--offload-arch=gfx950"] + san + [main_o, api_o] + _objects_of_kernels() + ["-o", exe],
    ]
    for cmd in steps:
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        assert r.returncode == 0, "\n".join(l for l in r.stdout.splitlines() if "packed-fp32" not in l)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env, timeout=600)
    print(r.stdout[-4000:])
    assert r.returncode == 0, r.stdout[-4000:]
    assert "clean" in r.stdout
