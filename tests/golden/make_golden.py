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

The 4-step sampling loop at 1024x1024 (the pages' four steps; schedule 1,
0.75, 0.5, 0.25, 0 from the workload's noise latent, no reference) stores the
whole latent after the last Euler update (fp32, [1, 4096, 128]).

The latent decoder's workloads (oracle/vae_oracle.py, float64, one batch
row at a time) store the image [B, H, W, 3]: whole (fp32) for the 1024x1024
decode, every 16th pixel row (plus the last) of each batch row for the
1920x1088 batch-4 decode (the whole tensor would be 100 MB), with the
full-image sum of squares per batch row.

Usage: python tests/golden/make_golden.py [step_1024px_s4608 ...]
Output: tests/golden/<workload>.npz with rows (int64), v ([B, len(rows), C]),
        z ([B, n_img, C], the loop) or image ([B, len(rows), W, 3]), and the
        oracle's full-tensor sum of squares and max-abs per batch row.
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import dit_oracle as O  # noqa: E402
from oracle import vae_oracle as V  # noqa: E402
from diffusion_transformer_fwd_amd import synth  # noqa: E402

# workload -> row stride of the stored velocity (1 = whole tensor, stored fp32)
WORKLOADS = {
    synth.W_STEP_1024.name: (synth.W_STEP_1024, 1),
    synth.W_STEP_1024_REF.name: (synth.W_STEP_1024_REF, 1),
    synth.W_STEP_1920x1088_B4.name: (synth.W_STEP_1920x1088_B4, 32),
    synth.W_STEP_848x624_3REF.name: (synth.W_STEP_848x624_3REF, 1),
    synth.W_STEP_512_REF.name: (synth.W_STEP_512_REF, 1),
}

# sampling-loop workload -> (step workload whose inputs it starts from, schedule)
DENOISE_WORKLOADS = {
    "denoise4_1024px_s4608": (synth.W_STEP_1024, [1.0, 0.75, 0.5, 0.25, 0.0]),
}

# decoder workload -> pixel-row stride of the stored image
VAE_WORKLOADS = {
    synth.V_DECODE_1024.name: (synth.V_DECODE_1024, 1),
    synth.V_DECODE_1920x1088_B4.name: (synth.V_DECODE_1920x1088_B4, 16),
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


def run_denoise(name: str) -> None:
    wl, sched = DENOISE_WORKLOADS[name]
    cfg = synth.FLUX2_KLEIN
    weights = synth.ModelWeights(cfg, 0, cache=False)
    ins = synth.step_inputs(cfg, wl, batch_row=0)
    txt = ins["txt"][None]
    z0 = ins["latents"][None, :wl.n_img]
    pos = O.position_ids(wl.n_txt, wl.img_grid, wl.ref_grids)
    sigmas = np.asarray([sched], dtype=np.float64)
    t0 = time.time()
    done = [0]

    def velocity(z, sig):
        v = O.step(cfg, weights, txt, z, sig, wl.n_img, pos)
        done[0] += 1
        print(f"  {name}: step {done[0]} done at {time.time() - t0:.0f}s", flush=True)
        return v

    z = O.denoise(velocity, z0, sigmas)
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), f"{name}.npz")
    np.savez(out, z=z.astype(np.float32), sigmas=sigmas, sumsq=(z * z).sum(axis=(1, 2)),
             maxabs=np.abs(z).max(axis=(1, 2)), seconds=time.time() - t0)
    print(f"wrote {out} in {time.time() - t0:.0f}s", flush=True)


def run_vae(name: str) -> None:
    wl, stride = VAE_WORKLOADS[name]
    vcfg = synth.VAE_KLEIN
    w = synth.vae_weights(vcfg, 0)
    hp, wp = wl.grid
    rows = sample_rows(16 * hp, stride)
    t0 = time.time()
    imgs, sumsq, maxabs = [], [], []
    for b in range(wl.batch):
        z = synth.vae_latents(vcfg, b, hp, wp)[None]
        img = V.decode(vcfg, w, z, hp, wp)[0]
        imgs.append(img[rows].astype(np.float32))
        sumsq.append(float((img * img).sum()))
        maxabs.append(float(np.abs(img).max()))
        print(f"  {name}: batch row {b} done at {time.time() - t0:.0f}s", flush=True)
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), f"{name}.npz")
    np.savez(out, rows=rows, image=np.stack(imgs), sumsq=np.asarray(sumsq),
             maxabs=np.asarray(maxabs), seconds=time.time() - t0)
    print(f"wrote {out} in {time.time() - t0:.0f}s", flush=True)


if __name__ == "__main__":
    for n in (sys.argv[1:] or list(WORKLOADS) + list(DENOISE_WORKLOADS) + list(VAE_WORKLOADS)):
        if n in VAE_WORKLOADS:
            run_vae(n)
        elif n in DENOISE_WORKLOADS:
            run_denoise(n)
        else:
            run(n)
