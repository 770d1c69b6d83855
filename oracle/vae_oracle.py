"""Plain CPU oracle for the latent decoder (VAE decode) that turns the
sampler's image tokens into pixels.

TEST INFRASTRUCTURE ONLY. This module is the checker for the HIP decoder:
only the test suite, the smoke check and the bench's CPU-baseline leg may
import it. The product path never calls it and shares no code with it.

What the pages fix: the decoder runs on the card after the last step, as
``decode(latents)`` ("tt_flux2_klein - Python reference", Lower-level entry
points), it is tt-metal's tt_dit VAE with a GroupNorm grid fix and
non-square slicing ("flux2-klein-p100a", What this port adds), so it has
GroupNorm layers and takes non-square images; the image post-processing
stays on the host (card header). Everything else is a reading, stated at
each function: the convolutional KL-autoencoder decoder of the
latent-diffusion family (conv_in; mid ResNet / attention / ResNet; up levels
of ResNet blocks with nearest 2x upsampling and a 3x3 conv; GroupNorm, SiLU,
conv_out), with a per-channel affine on the tokens and the 2x2 unpatchify in
front of it.

Everything is float64 NumPy (``dtype`` selectable) with ``matmul`` as the
only library primitive. Convolutions are written as their definition, a sum
over kernel taps of shifted inputs times the tap's weight matrix, in bands
of output rows to bound memory. Layouts: activations [B, H, W, C]
(channels last), conv weights [C_out, kh, kw, C_in].
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np


def unpatchify(z: np.ndarray, hp: int, wp: int, z_ch: int) -> np.ndarray:
    """Tokens [B, hp*wp, 4 z_ch] -> latent image [B, 2 hp, 2 wp, z_ch].

    Reading: token (r, c) (row-major over the patch grid) holds latent pixels
    (2r + i, 2c + j), channel k at token channel 4k + 2i + j.
    """
    B = z.shape[0]
    x = z.reshape(B, hp, wp, z_ch, 2, 2)          # [B, r, c, k, i, j]
    x = x.transpose(0, 1, 4, 2, 5, 3)             # [B, r, i, c, j, k]
    return x.reshape(B, 2 * hp, 2 * wp, z_ch)


def conv2d(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray],
           band: int = 64) -> np.ndarray:
    """Cross-correlation, stride 1, zero padding (k - 1) / 2, plus bias.

    out[n, y, x, o] = b[o] + sum_{ky, kx, c} xpad[n, y + ky, x + kx, c]
    w[o, ky, kx, c] with xpad the input padded by (k - 1) / 2 zeros on each
    side. x: [B, H, W, C]; w: [O, k, k, C] with odd k.
    """
    B, H, W, C = x.shape
    O, kh, kw, Ci = w.shape
    assert Ci == C and kh == kw and kh % 2 == 1
    p = kh // 2
    xp = np.pad(x, ((0, 0), (p, p), (p, p), (0, 0)))
    out = np.empty((B, H, W, O), dtype=np.result_type(x, w))
    for y0 in range(0, H, band):
        y1 = min(H, y0 + band)
        acc = np.zeros((B, y1 - y0, W, O), dtype=out.dtype)
        for ky in range(kh):
            for kx in range(kw):
                acc += xp[:, y0 + ky:y1 + ky, kx:kx + W, :] @ w[:, ky, kx, :].T
        if b is not None:
            acc += b
        out[:, y0:y1] = acc
    return out


def group_norm(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray, groups: int,
               eps: float) -> np.ndarray:
    """GroupNorm over [B, H, W, C]: channels split into `groups` runs of
    consecutive channels; each (sample, group) is normalized by its mean and
    biased variance over H * W * C / groups values, eps inside the root; then
    per-channel gamma, beta (reading V4)."""
    B, H, W, C = x.shape
    xr = x.reshape(B, H * W, groups, C // groups)
    mu = xr.mean(axis=(1, 3), keepdims=True)
    d = xr - mu
    var = (d * d).mean(axis=(1, 3), keepdims=True)
    y = (d / np.sqrt(var + eps)).reshape(B, H, W, C)
    return y * gamma + beta


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def upsample2x(x: np.ndarray) -> np.ndarray:
    """Nearest-neighbour 2x: out[y, x] = in[y // 2, x // 2]."""
    return np.repeat(np.repeat(x, 2, axis=1), 2, axis=2)


def resnet(x: np.ndarray, w: Dict[str, np.ndarray], p: str, groups: int,
           eps: float) -> np.ndarray:
    """Reading V2: h = conv(SiLU(GN1(x))); h = conv(SiLU(GN2(h)));
    out = x + h, or conv1x1(x) + h when the channel count changes."""
    h = conv2d(silu(group_norm(x, w[p + "gn1.g"], w[p + "gn1.b"], groups, eps)),
               w[p + "conv1.w"], w[p + "conv1.b"])
    h = conv2d(silu(group_norm(h, w[p + "gn2.g"], w[p + "gn2.b"], groups, eps)),
               w[p + "conv2.w"], w[p + "conv2.b"])
    s = x if (p + "short.w") not in w else conv2d(x, w[p + "short.w"], w[p + "short.b"])
    return s + h


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, chunk: int = 2048) -> np.ndarray:
    """softmax(q k^T / sqrt(C)) v for one sample; q, k, v: [N, C]."""
    C = q.shape[-1]
    out = np.empty_like(v, dtype=np.result_type(q, v))
    kt = k.T
    for s0 in range(0, q.shape[0], chunk):
        s = (q[s0:s0 + chunk] @ kt) / math.sqrt(C)
        s = s - s.max(axis=-1, keepdims=True)
        e = np.exp(s)
        out[s0:s0 + chunk] = (e / e.sum(axis=-1, keepdims=True)) @ v
    return out


def attention_block(x: np.ndarray, w: Dict[str, np.ndarray], p: str, groups: int,
                    eps: float) -> np.ndarray:
    """Reading V3: GN (no SiLU), q/k/v 1x1 convs with bias, one head of width
    C over all H * W positions of each sample, 1x1 output conv, residual."""
    B, H, W, C = x.shape
    t = group_norm(x, w[p + "gn.g"], w[p + "gn.b"], groups, eps)
    q = conv2d(t, w[p + "q.w"], w[p + "q.b"]).reshape(B, H * W, C)
    k = conv2d(t, w[p + "k.w"], w[p + "k.b"]).reshape(B, H * W, C)
    v = conv2d(t, w[p + "v.w"], w[p + "v.b"]).reshape(B, H * W, C)
    o = np.stack([attention(q[b], k[b], v[b]) for b in range(B)]).reshape(B, H, W, C)
    return x + conv2d(o, w[p + "o.w"], w[p + "o.b"])


def decode(vcfg, w: Dict[str, np.ndarray], z: np.ndarray, hp: int, wp: int,
           dtype=np.float64) -> np.ndarray:
    """Image [B, 16 hp, 16 wp, out_channels] from tokens z [B, hp*wp, 4 z_ch].

    Reading V6: u = z * scale + shift per token channel, then unpatchify.
    Reading V1: conv_in; mid ResNet, attention, ResNet; for each up level
    (channels reversed(block_channels)) `layers` ResNet blocks, then, except
    after the last level, upsample2x and a 3x3 conv; GroupNorm, SiLU,
    conv_out. Output unclamped (reading V7).
    """
    g, eps = vcfg.groups, vcfg.eps
    w = {k: np.asarray(v, dtype=dtype) for k, v in w.items()}
    z = np.asarray(z, dtype=dtype)
    u = z * w["lat_scale"] + w["lat_shift"]
    x = unpatchify(u, hp, wp, vcfg.z_channels)
    x = conv2d(x, w["conv_in.w"], w["conv_in.b"])
    x = resnet(x, w, "mid.res0.", g, eps)
    x = attention_block(x, w, "mid.attn.", g, eps)
    x = resnet(x, w, "mid.res1.", g, eps)
    n_lv = len(vcfg.level_channels)
    for lv in range(n_lv):
        for r in range(vcfg.layers):
            x = resnet(x, w, f"up{lv}.res{r}.", g, eps)
        if lv + 1 < n_lv:
            x = conv2d(upsample2x(x), w[f"up{lv}.upconv.w"], w[f"up{lv}.upconv.b"])
    x = silu(group_norm(x, w["norm_out.g"], w["norm_out.b"], g, eps))
    return conv2d(x, w["conv_out.w"], w["conv_out.b"])


def decode_flops(vcfg, B: int, hp: int, wp: int) -> float:
    """Multiply-adds x 2 of every convolution and of attention's two products."""
    H, W = 2 * hp, 2 * wp
    top = vcfg.top
    f = 2.0 * H * W * top * 9 * vcfg.z_channels
    res_list = vcfg.resnet_channels()
    h, wd = H, W
    # mid
    for _, ci, co in res_list[:2]:
        f += 2.0 * h * wd * co * 9 * (ci + co)
    n = h * wd
    f += 2.0 * n * top * top * 4 + 4.0 * n * n * top
    idx = 2
    for lv, co in enumerate(vcfg.level_channels):
        for r in range(vcfg.layers):
            _, ci, co2 = res_list[idx]
            idx += 1
            f += 2.0 * h * wd * co2 * 9 * (ci + co2)
            if ci != co2:
                f += 2.0 * h * wd * co2 * ci
        if lv + 1 < len(vcfg.level_channels):
            h, wd = 2 * h, 2 * wd
            f += 2.0 * h * wd * co * 9 * co
    f += 2.0 * h * wd * vcfg.out_channels * 9 * vcfg.level_channels[-1]
    return B * f
