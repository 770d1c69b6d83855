"""Write the oracle's expected outputs for the full-size step workloads.

Calls only ``oracle/`` (and the seeded input generator). The full step mixes
every row through attention in every block, so a sampled output cannot be
computed on its own; the oracle runs the whole step once here (float64, tens
of minutes on a few cores) and stores the velocity:

* the whole tensor v [B, n_img, C_in] (rounded to float32, far below the
  comparison tolerance) for the single-sample workloads — the 1024x1024 step,
  the step with one reference, the 848x624 step with three references and
  the 512x512 step with one reference — so every output element is compared;
* every 32nd image-token row (plus the last) for the 1920x1088 batch-4 step,
  whose whole tensor would be 17 MB; there the whole-tensor check is the sum
  of squares per batch row.

Usage: python tests/golden/make_golden.py [step_1024px_s4608 ...]
Output: tests/golden/<workload>.npz with rows (int64), v ([B, len(rows), C]),
        and the oracle's full-tensor sum of squares and max-abs per batch row.
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import dit_oracle as O  # noqa: E402
from diffusion_transformer_fwd_amd import synth  # noqa: E402

# workload -> row stride of the stored velocity (1 = whole tensor, stored fp32)
WORKLOADS = {
    synth.W_STEP_1024.name: (synth.W_STEP_1024, 1),
    synth.W_STEP_1024_REF.name: (synth.W_STEP_1024_REF, 1),
    synth.W_STEP_1920x1088_B4.name: (synth.W_STEP_1920x1088_B4, 32),
    synth.W_STEP_848x624_3REF.name: (synth.W_STEP_848x624_3REF, 1),
    synth.W_STEP_512_REF.name: (synth.W_STEP_512_REF, 1),
}


def sample_rows(n_img: int, stride: int) -> np.ndarray:
    rows = list(range(0, n_img, stride))
    if rows[-1] != n_img - 1:
        rows.append(n_img - 1)
    return np.asarray(rows, dtype=np.int64)


def run(name: str) -> None:
    wl, stride = WORKLOADS[name]
    cfg = synth.FLUX2_KLEIN
    weights = synth.ModelWeights(cfg, 0, cache=False)
    ins = [synth.step_inputs(cfg, wl, batch_row=b) for b in range(wl.batch)]
    txt = np.stack([i["txt"] for i in ins])
    lat = np.stack([i["latents"] for i in ins])
    pos = O.position_ids(wl.n_txt, wl.img_grid, wl.ref_grids)
    sigma = np.full(wl.batch, wl.sigma)
    t0 = time.time()

    def tick(kind, i, x):
        print(f"  {name}: {kind} {i} done at {time.time() - t0:.0f}s", flush=True)

    v = O.step(cfg, weights, txt, lat, sigma, wl.n_img, pos, on_block=tick)
    rows = sample_rows(wl.n_img, stride)
    vs = v[:, rows]
    if stride == 1:
        vs = vs.astype(np.float32)
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), f"{name}.npz")
    np.savez(out, rows=rows, v=vs, sumsq=(v * v).sum(axis=(1, 2)),
             maxabs=np.abs(v).max(axis=(1, 2)), seconds=time.time() - t0)
    print(f"wrote {out} in {time.time() - t0:.0f}s", flush=True)


if __name__ == "__main__":
    for n in (sys.argv[1:] or list(WORKLOADS)):
        run(n)
