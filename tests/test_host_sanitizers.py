"""The library's host-side planning code (csrc/plan.cpp: workspace layouts,
argument checks, position ids; csrc/tile_map.hpp: the GEMM tile map) built
with the host compiler under AddressSanitizer and UndefinedBehaviorSanitizer,
without HIP, and driven by tests/host_checks/plan_check.cpp through every
error path and up to the largest sizes the checks accept. Its workspace
sizes must equal those of the built library."""
import os
import shutil
import subprocess

import pytest

from diffusion_transformer_fwd_amd import dit, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "diffusion_transformer_fwd_amd", "csrc")

# the configurations plan_check.cpp uses, by index
CONFIGS = [
    synth.FLUX2_KLEIN,
    synth.DitConfig(hidden=256, heads=2, head_dim=128, mlp_hidden=768, txt_channels=256),
    synth.DitConfig(hidden=4096, heads=32, head_dim=128, mlp_hidden=16384, time_channels=4096),
]


@pytest.fixture(scope="module")
def plan_check(tmp_path_factory):
    cxx = shutil.which("g++")
    if not cxx:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("san") / "plan_check")
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-Wall", "-Wextra", "-Werror",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, "plan.cpp"),
           os.path.join(ROOT, "tests", "host_checks", "plan_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    return r


def test_plan_check_clean_under_sanitizers(plan_check):
    r = plan_check
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "plan_check: ok" in r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr


def test_sanitized_layouts_equal_the_library(plan_check):
    kinds = {dit.WS_DUAL, dit.WS_SINGLE, dit.WS_STEP, dit.WS_MOD, dit.WS_DENOISE}
    n = 0
    for line in plan_check.stdout.splitlines():
        if not line.startswith("layout "):
            continue
        ci, kind, B, S, total = (int(v) for v in line.split()[1:])
        assert kind in kinds
        assert dit.workspace_bytes(CONFIGS[ci], kind, B, S) == total, line
        n += 1
    assert n > 300


def test_sanitized_decoder_layouts_equal_the_library(plan_check):
    import dataclasses
    cfgs = [synth.VAE_KLEIN,
            dataclasses.replace(synth.VAE_KLEIN, block_channels=(32, 64, 64, 128), layers=2),
            dataclasses.replace(synth.VAE_KLEIN, block_channels=(256, 512, 1024, 2048), layers=4)]
    n = 0
    for line in plan_check.stdout.splitlines():
        if not line.startswith("vae_layout "):
            continue
        ci, B, hp, wp, total = (int(v) for v in line.split()[1:])
        assert dit.vae_workspace_bytes(cfgs[ci], B, hp, wp) == total, line
        n += 1
    assert n == 3 * 4 * 7
