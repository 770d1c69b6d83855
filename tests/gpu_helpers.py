"""Shared helpers for the GPU parity tests (inputs, comparisons, logging)."""
import sys
import time

import numpy as np

from diffusion_transformer_fwd_amd import dit, synth

# Tolerance of the bf16 path against the fp64 oracle: max-abs 2e-2 and
# relative L2 1e-2 on the compared tensor (x after a block, v after a step).
MAX_ABS = 2e-2
REL_L2 = 1e-2


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def stats(got: np.ndarray, want: np.ndarray):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    d = got - want
    return float(np.abs(d).max()), float(np.linalg.norm(d) / max(np.linalg.norm(want), 1e-30))


def assert_close(got, want, max_abs=MAX_ABS, rel_l2=REL_L2, what=""):
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    ma, rl = stats(got, want)
    log(f"{what}: max_abs {ma:.3e} rel_l2 {rl:.3e}")
    assert ma <= max_abs and rl <= rel_l2, f"{what}: max_abs {ma:.3e} rel_l2 {rl:.3e}"
    return ma, rl


def to_np(t) -> np.ndarray:
    return t.detach().float().cpu().numpy()
