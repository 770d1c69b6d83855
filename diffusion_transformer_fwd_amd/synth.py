"""Seeded synthetic inputs for the DiT denoise step.

This module only draws random numbers and names tensor shapes. It holds none
of the step's arithmetic, so both the CPU oracle's tests and the GPU harness
can take their inputs from it without sharing any of the method.

Scheme:
  * every tensor has a name; its stream is NumPy PCG64 seeded with
    (seed, crc32(name)), so a tensor never depends on which others were drawn;
  * matrices are N(0, 1/fan_in) with fan_in = the contraction length K of an
    [N, K] weight; activations are N(0, 1); QK-norm gains are 1 + 0.1 N(0, 1);
  * every value is drawn in fp32 and then rounded to the nearest bf16 value
    (ties to even), so a bf16 kernel and an fp64 oracle consume identical
    numbers.

The model follows the FLUX.2 [klein] layout the pages describe (model card
"flux2-klein-p100a", sections "Caveats" and "Things that are easy to get
wrong"; PYTHON.md "Modules": 5 dual-stream + 20 single-stream blocks).
"""
from __future__ import annotations

import dataclasses
import zlib
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

PRENORM_RMS = 0
PRENORM_LAYER = 1


@dataclasses.dataclass(frozen=True)
class DitConfig:
    hidden: int = 3072          # D
    heads: int = 24             # H
    head_dim: int = 128         # d
    mlp_hidden: int = 9216      # F = 3 D (SwiGLU inner width)
    n_dual: int = 5
    n_single: int = 20
    in_channels: int = 128      # 2x2-patchified latent channels
    txt_channels: int = 7680    # three text-encoder layers of 2560, concatenated
    axes_dim: Tuple[int, int, int, int] = (32, 32, 32, 32)
    theta: float = 2000.0
    eps: float = 1e-6
    prenorm: int = PRENORM_RMS
    time_channels: int = 256    # sinusoidal timestep features

    @property
    def mod_rows(self) -> int:
        """Rows of the per-step modulation buffer: 6 + 6 + 3 + 2 vectors of D."""
        return 17


FLUX2_KLEIN = DitConfig()
# Small dual-block configuration: hidden 256 = 2 heads x 128.
TINY_256 = DitConfig(hidden=256, heads=2, head_dim=128, mlp_hidden=768,
                     n_dual=1, n_single=0, in_channels=128, txt_channels=256)


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 value, ties to even.

    Returns float32 holding bf16-representable values. Inputs are finite.
    """
    a = np.array(a, dtype=np.float32, copy=True, order="C")
    u = a.view(np.uint32)
    # finite inputs: u + 0x8000 never wraps (max finite magnitude is 0x7F7FFFFF)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u &= np.uint32(0xFFFF0000)
    return a


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """The upper 16 bits of bf16-representable float32 values, as uint16."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _rng(seed: int, name: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([int(seed), zlib.crc32(name.encode())]))


def normal(seed: int, name: str, shape: Sequence[int], std: float = 1.0,
           mean: float = 0.0) -> np.ndarray:
    """bf16-rounded N(mean, std^2) draws, float32 storage."""
    x = _rng(seed, name).standard_normal(tuple(shape), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return bf16_round(x)


def matrix(seed: int, name: str, n: int, k: int) -> np.ndarray:
    """[n, k] weight in nn.Linear layout, N(0, 1/k)."""
    return normal(seed, name, (n, k), std=1.0 / np.sqrt(k))


def gain(seed: int, name: str, d: int) -> np.ndarray:
    """QK-norm gain: 1 + 0.1 N(0, 1), bf16-rounded."""
    return normal(seed, name, (d,), std=0.1, mean=1.0)


# ---------------------------------------------------------------- weights

def dual_weights(cfg: DitConfig, seed: int, idx: int) -> Dict[str, np.ndarray]:
    """One dual-stream block. Stream 0 = text, stream 1 = image.

    qkv: [3D, D] (q rows, then k rows, then v rows; head j = rows 128j..)
    out: [D, D]; mlp_in: [2F, D] (gate rows, then up rows); mlp_out: [D, F].
    """
    D, F, d = cfg.hidden, cfg.mlp_hidden, cfg.head_dim
    w: Dict[str, np.ndarray] = {}
    for s, tag in ((0, "txt"), (1, "img")):
        p = f"dual.{idx}.{tag}."
        w[f"qkv{s}"] = matrix(seed, p + "qkv", 3 * D, D)
        w[f"out{s}"] = matrix(seed, p + "out", D, D)
        w[f"mlp_in{s}"] = matrix(seed, p + "mlp_in", 2 * F, D)
        w[f"mlp_out{s}"] = matrix(seed, p + "mlp_out", D, F)
        w[f"q_gain{s}"] = gain(seed, p + "q_gain", d)
        w[f"k_gain{s}"] = gain(seed, p + "k_gain", d)
    return w


def single_weights(cfg: DitConfig, seed: int, idx: int) -> Dict[str, np.ndarray]:
    """One single-stream block.

    w_in: [3D + 2F, D] = [Wq; Wk; Wv; W_gate; W_up]; w_out: [D, D + F]
    (columns 0..D-1 take the attention output, D.. the SwiGLU activation).
    """
    D, F, d = cfg.hidden, cfg.mlp_hidden, cfg.head_dim
    p = f"single.{idx}."
    return {
        "w_in": matrix(seed, p + "w_in", 3 * D + 2 * F, D),
        "w_out": matrix(seed, p + "w_out", D, D + F),
        "q_gain": gain(seed, p + "q_gain", d),
        "k_gain": gain(seed, p + "k_gain", d),
    }


def global_weights(cfg: DitConfig, seed: int) -> Dict[str, np.ndarray]:
    """Time MLP, the four modulation projections, embeds and the output head."""
    D = cfg.hidden
    return {
        "t_in": matrix(seed, "time.in", D, cfg.time_channels),
        "t_out": matrix(seed, "time.out", D, D),
        "mod_dual_img": matrix(seed, "mod.dual_img", 6 * D, D),
        "mod_dual_txt": matrix(seed, "mod.dual_txt", 6 * D, D),
        "mod_single": matrix(seed, "mod.single", 3 * D, D),
        "mod_final": matrix(seed, "mod.final", 2 * D, D),
        "x_embed": matrix(seed, "embed.x", D, cfg.in_channels),
        "ctx_embed": matrix(seed, "embed.ctx", D, cfg.txt_channels),
        "proj_out": matrix(seed, "proj_out", cfg.in_channels, D),
    }


class ModelWeights:
    """Lazily drawn full-model weights (a 4B-parameter model is ~15 GB as
    float32, so blocks are drawn on demand and may be dropped after use)."""

    def __init__(self, cfg: DitConfig, seed: int = 0, cache: bool = False):
        self.cfg, self.seed, self.cache = cfg, seed, cache
        self._glob: Optional[Dict[str, np.ndarray]] = None
        self._blocks: Dict[Tuple[str, int], Dict[str, np.ndarray]] = {}

    @property
    def glob(self) -> Dict[str, np.ndarray]:
        if self._glob is None:
            self._glob = global_weights(self.cfg, self.seed)
        return self._glob

    def dual(self, i: int) -> Dict[str, np.ndarray]:
        key = ("dual", i)
        if key in self._blocks:
            return self._blocks[key]
        w = dual_weights(self.cfg, self.seed, i)
        if self.cache:
            self._blocks[key] = w
        return w

    def single(self, i: int) -> Dict[str, np.ndarray]:
        key = ("single", i)
        if key in self._blocks:
            return self._blocks[key]
        w = single_weights(self.cfg, self.seed, i)
        if self.cache:
            self._blocks[key] = w
        return w


# ---------------------------------------------------------------- inputs

def text_embedding(cfg: DitConfig, seed: int, n_txt: int) -> np.ndarray:
    """Prompt embedding [n_txt, C_txt] standing in for the text encoder output."""
    return normal(seed, "input.txt", (n_txt, cfg.txt_channels))


def latents(cfg: DitConfig, seed: int, n_tok: int, name: str = "input.latents") -> np.ndarray:
    """2x2-patchified latent tokens [n_tok, C_in]."""
    return normal(seed, name, (n_tok, cfg.in_channels))


def residual(cfg: DitConfig, seed: int, rows: int, name: str = "input.x") -> np.ndarray:
    """Residual-stream activations [rows, D] for block-level tests."""
    return normal(seed, name, (rows, cfg.hidden))


def patch_grid(width_px: int, height_px: int) -> Tuple[int, int]:
    """(Hp, Wp) patch rows/cols: /8 VAE factor, then 2x2 patches."""
    return height_px // 16, width_px // 16


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape of one step: batch, text rows, image grid and reference grids."""
    name: str
    batch: int
    n_txt: int
    img_grid: Tuple[int, int]                       # (Hp, Wp)
    ref_grids: Tuple[Tuple[int, int], ...] = ()
    sigma: float = 0.75

    @property
    def n_img(self) -> int:
        return self.img_grid[0] * self.img_grid[1]

    @property
    def n_ref(self) -> int:
        return sum(h * w for h, w in self.ref_grids)

    @property
    def seq(self) -> int:
        return self.n_txt + self.n_img + self.n_ref


# Configurations of the measured workloads.
W_DUAL_TINY = Workload("dual_block_d256_s96", 1, 32, (8, 8), (), 0.5)
W_SINGLE_1024 = Workload("single_block_1024px_s4608", 1, 512, (64, 64), (), 0.75)
W_STEP_1024 = Workload("step_1024px_s4608", 1, 512, (64, 64), (), 0.75)
W_STEP_1024_REF = Workload("step_1024px_1ref_s8704", 1, 512, (64, 64), ((64, 64),), 0.75)
W_STEP_1920x1088_B4 = Workload("step_1920x1088_b4_s8672", 4, 512, (68, 120), (), 0.75)
# non-square output (848x624 -> 39 x 53 patches, no tile-aligned size) with
# three references at their own aspect (1024x1024, 1184x880, 512x768 px)
W_STEP_848x624_3REF = Workload("step_848x624_3ref_s12281", 1, 512, (39, 53),
                               ((64, 64), (55, 74), (48, 32)), 0.75)
# the smallest listed size with a reference: 512x512 output, one 512x512 reference
W_STEP_512_REF = Workload("step_512px_1ref_s2560", 1, 512, (32, 32), ((32, 32),), 0.75)
# the longest sequence: 1920x1088 output with three 1024x1024 references
W_SINGLE_MAX = Workload("single_block_1920x1088_3ref_s20960", 1, 512, (68, 120),
                        ((64, 64), (64, 64), (64, 64)), 0.75)


def step_inputs(cfg: DitConfig, wl: Workload, batch_row: int = 0,
                input_seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Per-sample inputs: text embedding and image (+reference) latents.

    Batch row b uses input seed b unless `input_seed` is given.
    """
    s = batch_row if input_seed is None else input_seed
    lat = [latents(cfg, s, wl.n_img, "input.latents")]
    for i, (h, w) in enumerate(wl.ref_grids):
        lat.append(latents(cfg, s, h * w, f"input.ref{i}"))
    return {
        "txt": text_embedding(cfg, s, wl.n_txt),
        "latents": np.concatenate(lat, axis=0),
    }


# ---------------------------------------------------------------- VAE decoder

@dataclasses.dataclass(frozen=True)
class VaeConfig:
    """Shape of the latent decoder (a reading; the pages give none: they say
    only that the decoder runs on the card, has GroupNorm layers and takes
    non-square images, "flux2-klein-p100a", What this port adds).

    block_channels lists the encoder-order widths; the decoder's up levels
    run them in reverse (512, 512, 256, 128 for the default), each with
    `layers` ResNet blocks and, except the last, a 2x upsample.
    """
    z_channels: int = 32
    block_channels: Tuple[int, ...] = (128, 256, 512, 512)
    layers: int = 3
    groups: int = 32
    eps: float = 1e-6
    out_channels: int = 3

    @property
    def top(self) -> int:
        return self.block_channels[-1]

    @property
    def level_channels(self) -> Tuple[int, ...]:
        return tuple(reversed(self.block_channels))

    def resnet_channels(self):
        """[(name, c_in, c_out)] of every ResNet block in execution order."""
        out = [("mid.res0.", self.top, self.top), ("mid.res1.", self.top, self.top)]
        c = self.top
        for lv, co in enumerate(self.level_channels):
            for r in range(self.layers):
                out.append((f"up{lv}.res{r}.", c, co))
                c = co
        return out


VAE_KLEIN = VaeConfig()
# Small decoder for element-wise tests: both identity and 1x1 shortcuts,
# 1, 2 and 4 channels per group.
VAE_TINY = VaeConfig(block_channels=(32, 64, 64, 128), layers=2)


def _conv_w(seed: int, name: str, c_out: int, k: int, c_in: int) -> np.ndarray:
    """[c_out, k, k, c_in] conv weight, N(0, 1 / (k k c_in))."""
    return normal(seed, name, (c_out, k, k, c_in), std=1.0 / np.sqrt(k * k * c_in))


def _bias(seed: int, name: str, n: int) -> np.ndarray:
    return normal(seed, name, (n,), std=0.02)


def vae_weights(vcfg: VaeConfig, seed: int = 0) -> Dict[str, np.ndarray]:
    """Decoder weights by dotted name (float32 storage of bf16 values).

    Conv weights are [C_out, kh, kw, C_in]; GroupNorm gains are
    1 + 0.1 N(0, 1), GroupNorm shifts 0.1 N(0, 1), biases N(0, 0.02^2); the
    latent affine acts on the 4 z_channels token channels.
    """
    z, top = vcfg.z_channels, vcfg.top
    w: Dict[str, np.ndarray] = {
        "lat_scale": normal(seed, "vae.lat_scale", (4 * z,), std=0.1, mean=1.0),
        "lat_shift": normal(seed, "vae.lat_shift", (4 * z,), std=0.1),
        "conv_in.w": _conv_w(seed, "vae.conv_in.w", top, 3, z),
        "conv_in.b": _bias(seed, "vae.conv_in.b", top),
    }

    def gn(p: str, c: int):
        w[p + "g"] = normal(seed, "vae." + p + "g", (c,), std=0.1, mean=1.0)
        w[p + "b"] = normal(seed, "vae." + p + "b", (c,), std=0.1)

    def conv(p: str, co: int, k: int, ci: int):
        w[p + "w"] = _conv_w(seed, "vae." + p + "w", co, k, ci)
        w[p + "b"] = _bias(seed, "vae." + p + "b", co)

    for p, ci, co in vcfg.resnet_channels():
        gn(p + "gn1.", ci)
        conv(p + "conv1.", co, 3, ci)
        gn(p + "gn2.", co)
        conv(p + "conv2.", co, 3, co)
        if ci != co:
            conv(p + "short.", co, 1, ci)
    gn("mid.attn.gn.", top)
    for t in "qkvo":
        conv(f"mid.attn.{t}.", top, 1, top)
    for lv, co in enumerate(vcfg.level_channels[:-1]):
        conv(f"up{lv}.upconv.", co, 3, co)
    c0 = vcfg.level_channels[-1]
    gn("norm_out.", c0)
    conv("conv_out.", vcfg.out_channels, 3, c0)
    return w


def vae_latents(vcfg: VaeConfig, seed: int, hp: int, wp: int) -> np.ndarray:
    """Image tokens [hp * wp, 4 z] as the sampler leaves them, N(0, 1)."""
    return normal(seed, "vae.input.z", (hp * wp, 4 * vcfg.z_channels))


@dataclasses.dataclass(frozen=True)
class VaeWorkload:
    """One decode: batch and token grid (hp, wp); the image is 16 hp x 16 wp."""
    name: str
    batch: int
    grid: Tuple[int, int]


V_DECODE_1024 = VaeWorkload("vae_decode_1024px", 1, (64, 64))
V_DECODE_1920x1088_B4 = VaeWorkload("vae_decode_1920x1088_b4", 4, (68, 120))
