"""Plain CPU oracle for one FLUX.2-[klein]-style DiT denoise step.

TEST INFRASTRUCTURE ONLY. This module is the checker for the HIP path: only
the test suite, the smoke check and the bench's CPU-baseline leg may import
it. The product path never calls it and shares no code with it.

It computes, in float64 by default (``dtype=np.float32`` is allowed for a
cross-check), exactly what the method defines, one step at a time, with NumPy
matmuls as the only library primitive. Nothing is fused, blocked or reordered
beyond chunking attention over query rows to bound memory.

Sources (the pages this follows):
  [card]   "flux2-klein-p100a" model card: header (scheduler on the host,
           DiT on the card), the Tasks/Size/Steps/References table, and
           "Caveats" (all 512 padded text rows, no mask; layers 9/18/27
           concatenated to [512, 7680]; one modulation result per step for
           all blocks).
  [py]     "tt_flux2_klein - Python reference": "Lower-level entry points"
           (encode -> [512, 7680]), "Modules" (host.py: token ids, RoPE;
           tt_dit.py: 5 dual-stream + 20 single-stream blocks) and "Things
           that are easy to get wrong" (global modulation; unmasked text rows;
           RoPE 32 dims per axis, theta 2000, adjacent pairs; reference image
           i at t = 10 + 10 i).
  [mstar]  "FLUX.2 [klein] 4B/9B + Z-Image-Turbo on a shared DiT scaffold":
           "What does this PR do?" (batch rows independent bit for bit).

Where the pages leave a step open, the reading taken is stated at the
function (hidden 3072 = 24 x 128, MLP ratio 3 with SwiGLU, QK-RMSNorm,
dual = separate text/image weights with joint attention, single = fused
QKV+MLP, 2x2 patchified latents, no biases, AdaLN (1 + scale) / shift / gate,
RMS pre-norm by default with LayerNorm as an option, eps 1e-6, sinusoidal
timestep features of sigma x 1000 with cosines first).

Layouts: a sample's token sequence is text rows [0, n_txt), then image rows
(row-major over the patch grid), then reference rows; B samples are stacked
as x[B, S, D].
"""
from __future__ import annotations

import math
from typing import Callable, Dict, Optional, Sequence, Tuple

import numpy as np

PRENORM_RMS = 0
PRENORM_LAYER = 1


# ------------------------------------------------------------ position ids

def position_ids(n_txt: int, img_grid: Tuple[int, int],
                 ref_grids: Sequence[Tuple[int, int]] = ()) -> np.ndarray:
    """Token ids (t, h, w, l) for one sample, int64 [S, 4].

    [py] "Modules" puts token ids in the host maths; "Things that are easy to
    get wrong" fixes reference image i at t = 10 + 10 i. Reading: i counts
    from 0; text row l gets (0, 0, 0, l); image patch (r, c) of the row-major
    grid gets (0, r, c, 0); reference i patch (r, c) gets (10 + 10 i, r, c, 0).
    """
    rows = []
    for l in range(n_txt):
        rows.append((0, 0, 0, l))
    hp, wp = img_grid
    for r in range(hp):
        for c in range(wp):
            rows.append((0, r, c, 0))
    for i, (rh, rw) in enumerate(ref_grids):
        t = 10 + 10 * i
        for r in range(rh):
            for c in range(rw):
                rows.append((t, r, c, 0))
    return np.asarray(rows, dtype=np.int64).reshape(-1, 4)


# ------------------------------------------------------------ RoPE

def rope_angles(pos: np.ndarray, axes_dim: Sequence[int] = (32, 32, 32, 32),
                theta: float = 2000.0) -> np.ndarray:
    """Rotation angle of every adjacent pair, float64 [S, sum(axes_dim)/2].

    [py] "Things that are easy to get wrong": 32 dims per axis, theta 2000,
    adjacent pairs. Axis a owns head dims [32a, 32a + 32); its pair j
    (dims 32a + 2j, 32a + 2j + 1) turns by pos_a * theta^(-2j / 32).
    """
    pos = np.asarray(pos, dtype=np.float64)
    cols = []
    for a, dim in enumerate(axes_dim):
        j = np.arange(dim // 2, dtype=np.float64)
        omega = theta ** (-2.0 * j / dim)
        cols.append(pos[:, a:a + 1] * omega[None, :])
    return np.concatenate(cols, axis=1)


def rope_tables(pos: np.ndarray, axes_dim: Sequence[int] = (32, 32, 32, 32),
                theta: float = 2000.0) -> Tuple[np.ndarray, np.ndarray]:
    """cos and sin of every pair angle, float64 [S, 64] for head_dim 128."""
    phi = rope_angles(pos, axes_dim, theta)
    return np.cos(phi), np.sin(phi)


def apply_rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate each adjacent pair (x[2m], x[2m+1]) of the last axis.

    x: [..., S, 128]; cos, sin: [S, 64].
    y[2m] = x[2m] cos - x[2m+1] sin; y[2m+1] = x[2m] sin + x[2m+1] cos.
    """
    xe = x[..., 0::2]
    xo = x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = xe * cos - xo * sin
    y[..., 1::2] = xe * sin + xo * cos
    return y


# ------------------------------------------------------------ elementwise

def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def timestep_features(sigma: np.ndarray, channels: int = 256,
                      dtype=np.float64) -> np.ndarray:
    """Sinusoidal features of tau = 1000 sigma, [B, channels].

    Reading (the pages only say each of the 4 steps is one DiT call at a
    sigma from the host schedule): half = channels / 2 frequencies
    f_k = exp(-ln(1e4) k / half); features [cos(tau f_k) | sin(tau f_k)].
    Evaluated in float64.
    """
    sigma = np.asarray(sigma, dtype=np.float64).reshape(-1)
    half = channels // 2
    k = np.arange(half, dtype=np.float64)
    f = np.exp(-math.log(10000.0) * k / half)
    ang = (1000.0 * sigma)[:, None] * f[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(dtype)


def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """x @ w.T for a weight in [out, in] layout (no bias anywhere)."""
    return x @ w.T


def prenorm(x: np.ndarray, kind: int = PRENORM_RMS, eps: float = 1e-6) -> np.ndarray:
    """Affine-free pre-norm over the last axis.

    RMS (the default reading; the pages name no norm kind for the AdaLN
    pre-norm): x / sqrt(mean(x^2) + eps). LAYER: (x - mean) / sqrt(var + eps).
    """
    if kind == PRENORM_LAYER:
        mu = x.mean(axis=-1, keepdims=True)
        xc = x - mu
        var = (xc * xc).mean(axis=-1, keepdims=True)
        return xc / np.sqrt(var + eps)
    ms = (x * x).mean(axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps)


def modulate(x: np.ndarray, shift: np.ndarray, scale: np.ndarray,
             kind: int = PRENORM_RMS, eps: float = 1e-6) -> np.ndarray:
    """AdaLN: N(x) * (1 + scale) + shift, shift/scale broadcast over rows."""
    return prenorm(x, kind, eps) * (1.0 + scale) + shift


def qk_rmsnorm(x: np.ndarray, g: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """Per-head RMSNorm with a learned gain: x / sqrt(mean(x^2) + eps) * g."""
    ms = (x * x).mean(axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


# ------------------------------------------------------------ attention

def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
              chunk: int = 1024) -> np.ndarray:
    """softmax(q k^T / sqrt(d)) v per (batch, head); no mask.

    q, k, v: [B, H, S, d]. [card] "Caveats" and [py] "Things that are easy to
    get wrong": all text rows, padded ones included, take part unmasked.
    """
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d)
    out = np.empty_like(q)
    S = q.shape[2]
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            kt = k[b, h].T
            for s0 in range(0, S, chunk):
                s = (q[b, h, s0:s0 + chunk] @ kt) * scale
                s = s - s.max(axis=-1, keepdims=True)
                p = np.exp(s)
                p /= p.sum(axis=-1, keepdims=True)
                out[b, h, s0:s0 + chunk] = p @ v[b, h]
    return out


def _heads(x: np.ndarray, heads: int) -> np.ndarray:
    """[B, S, H*d] -> [B, H, S, d]."""
    B, S, HD = x.shape
    return x.reshape(B, S, heads, HD // heads).transpose(0, 2, 1, 3)


def _merge(x: np.ndarray) -> np.ndarray:
    """[B, H, S, d] -> [B, S, H*d]."""
    B, H, S, d = x.shape
    return x.transpose(0, 2, 1, 3).reshape(B, S, H * d)


def _qkv_attention(qkv: np.ndarray, heads: int, q_gain, k_gain, cos, sin, eps):
    """Split [B, S, 3D] into q/k/v heads, QK-RMSNorm then RoPE, attend.

    Reading: the q/k RMS norms come before the rotation (RoPE acts on the
    normalized vectors).
    Returns the attention output merged back to [B, S, D].
    """
    D = qkv.shape[-1] // 3
    q = _heads(qkv[..., :D], heads)
    k = _heads(qkv[..., D:2 * D], heads)
    v = _heads(qkv[..., 2 * D:], heads)
    q = apply_rope(qk_rmsnorm(q, q_gain, eps), cos, sin)
    k = apply_rope(qk_rmsnorm(k, k_gain, eps), cos, sin)
    return _merge(attention(q, k, v))


def swiglu(u: np.ndarray) -> np.ndarray:
    """SiLU(first half) * second half of the last axis."""
    F = u.shape[-1] // 2
    return silu(u[..., :F]) * u[..., F:]


# ------------------------------------------------------------ modulation

def modulation(gw: Dict[str, np.ndarray], sigma: np.ndarray, channels: int = 256,
               dtype=np.float64) -> Dict[str, np.ndarray]:
    """Per-step AdaLN parameters, computed once and shared by every block.

    [card] "Caveats" and [py] "Things that are easy to get wrong": one set of
    AdaLN vectors per step, which every block reuses (no block computes its
    own). Reading: temb = W_out SiLU(W_in e(sigma)),
    m = SiLU(temb), then four projections of m:
      dual_img [B, 6, D] and dual_txt [B, 6, D]: shift1, scale1, gate1,
        shift2, scale2, gate2 (attention branch, then MLP branch);
      single [B, 3, D]: shift, scale, gate;   final [B, 2, D]: shift, scale.
    """
    e = timestep_features(sigma, channels, dtype)
    f = lambda n: gw[n].astype(dtype)
    temb = linear(silu(linear(e, f("t_in"))), f("t_out"))
    m = silu(temb)
    B = m.shape[0]
    D = temb.shape[-1]
    return {
        "dual_img": linear(m, f("mod_dual_img")).reshape(B, 6, D),
        "dual_txt": linear(m, f("mod_dual_txt")).reshape(B, 6, D),
        "single": linear(m, f("mod_single")).reshape(B, 3, D),
        "final": linear(m, f("mod_final")).reshape(B, 2, D),
    }


# ------------------------------------------------------------ blocks

def dual_block(x: np.ndarray, n_txt: int, w: Dict[str, np.ndarray],
               mod_txt: np.ndarray, mod_img: np.ndarray, cos: np.ndarray,
               sin: np.ndarray, heads: int, eps: float = 1e-6,
               prenorm_kind: int = PRENORM_RMS, dtype=np.float64) -> np.ndarray:
    """One dual-stream block; returns the updated residual x [B, S, D].

    [py] "Modules": tt_dit.py runs 5 dual-stream blocks first. The text
    stream is rows [0, n_txt) and uses stream-0 weights and mod_txt; the
    image stream (image and reference rows) uses stream-1 weights and
    mod_img. The two streams attend jointly over the whole sequence, text
    first. mod_*: [B, 6, D].
    """
    x = np.asarray(x, dtype=dtype)
    f = lambda n: w[n].astype(dtype)
    rows = (slice(0, n_txt), slice(n_txt, x.shape[1]))
    mods = (np.asarray(mod_txt, dtype), np.asarray(mod_img, dtype))

    # attention branch: per-stream norm + QKV, joint attention, per-stream out
    qkv = []
    for s in (0, 1):
        md = mods[s]
        h = modulate(x[:, rows[s]], md[:, None, 0], md[:, None, 1], prenorm_kind, eps)
        qkv.append(linear(h, f(f"qkv{s}")))
    D = x.shape[-1]
    qkv_all = np.concatenate(qkv, axis=1)
    # QK-norm gains differ per stream: normalise and rotate each stream's rows
    q_parts, k_parts = [], []
    for s in (0, 1):
        t = qkv[s]
        q = qk_rmsnorm(_heads(t[..., :D], heads), f(f"q_gain{s}"), eps)
        k = qk_rmsnorm(_heads(t[..., D:2 * D], heads), f(f"k_gain{s}"), eps)
        q_parts.append(q)
        k_parts.append(k)
    q = apply_rope(np.concatenate(q_parts, axis=2), cos, sin)
    k = apply_rope(np.concatenate(k_parts, axis=2), cos, sin)
    v = _heads(qkv_all[..., 2 * D:], heads)
    o = _merge(attention(q, k, v))

    out = x.copy()
    for s in (0, 1):
        md = mods[s]
        out[:, rows[s]] += md[:, None, 2] * linear(o[:, rows[s]], f(f"out{s}"))
    # MLP branch
    for s in (0, 1):
        md = mods[s]
        h2 = modulate(out[:, rows[s]], md[:, None, 3], md[:, None, 4], prenorm_kind, eps)
        a = swiglu(linear(h2, f(f"mlp_in{s}")))
        out[:, rows[s]] += md[:, None, 5] * linear(a, f(f"mlp_out{s}"))
    return out


def single_block(x: np.ndarray, w: Dict[str, np.ndarray], mod: np.ndarray,
                 cos: np.ndarray, sin: np.ndarray, heads: int, eps: float = 1e-6,
                 prenorm_kind: int = PRENORM_RMS, dtype=np.float64) -> np.ndarray:
    """One single-stream block; returns the updated residual x [B, S, D].

    [py] "Modules": 20 single-stream blocks follow the dual ones. One fused
    input projection gives q, k, v and the SwiGLU pre-activations; attention
    and MLP run in parallel from the same normed input and one fused output
    projection of [attention | activation] is added under one gate.
    mod: [B, 3, D] = shift, scale, gate.
    """
    x = np.asarray(x, dtype=dtype)
    mod = np.asarray(mod, dtype)
    D = x.shape[-1]
    w_in = w["w_in"].astype(dtype)
    h = modulate(x, mod[:, None, 0], mod[:, None, 1], prenorm_kind, eps)
    u = linear(h, w_in)
    o = _qkv_attention(u[..., :3 * D], heads, w["q_gain"].astype(dtype),
                       w["k_gain"].astype(dtype), cos, sin, eps)
    a = swiglu(u[..., 3 * D:])
    y = linear(np.concatenate([o, a], axis=-1), w["w_out"].astype(dtype))
    return x + mod[:, None, 2] * y


def single_block_rows(x: np.ndarray, w: Dict[str, np.ndarray], mod: np.ndarray,
                      cos: np.ndarray, sin: np.ndarray, heads: int, rows: np.ndarray,
                      eps: float = 1e-6, prenorm_kind: int = PRENORM_RMS,
                      dtype=np.float64) -> np.ndarray:
    """single_block's output at the token rows `rows` only, [B, len(rows), D].

    The same definition restricted to the queries asked for: keys and values
    come from every row (attention sees the whole sequence), while q, the
    SwiGLU branch and the output projection are formed for the listed rows.
    This is what lets a long sequence be checked row by row.
    """
    x = np.asarray(x, dtype=dtype)
    mod = np.asarray(mod, dtype)
    rows = np.asarray(rows)
    D = x.shape[-1]
    w_in = w["w_in"].astype(dtype)
    h = modulate(x, mod[:, None, 0], mod[:, None, 1], prenorm_kind, eps)
    kv = linear(h, w_in[D:3 * D])
    u = linear(h[:, rows], w_in)
    q = apply_rope(qk_rmsnorm(_heads(u[..., :D], heads), w["q_gain"].astype(dtype), eps),
                   cos[rows], sin[rows])
    k = apply_rope(qk_rmsnorm(_heads(kv[..., :D], heads), w["k_gain"].astype(dtype), eps),
                   cos, sin)
    o = _merge(attention(q, k, _heads(kv[..., D:], heads)))
    a = swiglu(u[..., 3 * D:])
    y = linear(np.concatenate([o, a], axis=-1), w["w_out"].astype(dtype))
    return x[:, rows] + mod[:, None, 2] * y


# ------------------------------------------------------------ step

def embed(gw: Dict[str, np.ndarray], txt: np.ndarray, lat: np.ndarray,
          dtype=np.float64) -> np.ndarray:
    """x = [txt W_ctx^T ; latents W_x^T] per sample, [B, S, D].

    [card] "Caveats" / [py] "Lower-level entry points": the prompt embedding
    is [512, 7680]; reading: one bias-free linear to the hidden size. Image
    and reference latents share the x-embedding.
    """
    xt = linear(np.asarray(txt, dtype), gw["ctx_embed"].astype(dtype))
    xi = linear(np.asarray(lat, dtype), gw["x_embed"].astype(dtype))
    return np.concatenate([xt, xi], axis=1)


def final_layer(gw: Dict[str, np.ndarray], x: np.ndarray, n_txt: int, n_img: int,
                mod_final: np.ndarray, eps: float = 1e-6,
                prenorm_kind: int = PRENORM_RMS, dtype=np.float64) -> np.ndarray:
    """Velocity for the image rows only: (N(x) (1 + scale) + shift) W_o^T.

    Text and reference rows are dropped. Returns [B, n_img, C_in].
    """
    md = np.asarray(mod_final, dtype)
    xi = np.asarray(x, dtype)[:, n_txt:n_txt + n_img]
    h = modulate(xi, md[:, None, 0], md[:, None, 1], prenorm_kind, eps)
    return linear(h, gw["proj_out"].astype(dtype))


def step(cfg, weights, txt: np.ndarray, lat: np.ndarray, sigma: np.ndarray,
         n_img: int, pos: np.ndarray, dtype=np.float64,
         on_block: Optional[Callable[[str, int, np.ndarray], None]] = None) -> np.ndarray:
    """One denoise step: global modulation, embeds, 5 dual + 20 single blocks,
    final layer. Returns the velocity [B, n_img, C_in].

    [card] Tasks table: each of the 4 steps is one DiT call (no CFG).
    [py] "Modules": 5 dual-stream then 20 single-stream blocks.
    The one modulation result is handed to every block.

    cfg: any object with hidden, heads, n_dual, n_single, axes_dim, theta,
    eps, prenorm, time_channels. weights: .glob, .dual(i), .single(i).
    txt [B, n_txt, C_txt]; lat [B, n_img + n_ref, C_in]; sigma [B];
    pos [S, 4] shared by the batch.
    """
    gw = weights.glob
    n_txt = txt.shape[1]
    mod = modulation(gw, sigma, cfg.time_channels, dtype)
    cos, sin = rope_tables(pos, cfg.axes_dim, cfg.theta)
    cos, sin = cos.astype(dtype), sin.astype(dtype)
    x = embed(gw, txt, lat, dtype)
    for i in range(cfg.n_dual):
        x = dual_block(x, n_txt, weights.dual(i), mod["dual_txt"], mod["dual_img"],
                       cos, sin, cfg.heads, cfg.eps, cfg.prenorm, dtype)
        if on_block is not None:
            on_block("dual", i, x)
    for i in range(cfg.n_single):
        x = single_block(x, weights.single(i), mod["single"], cos, sin, cfg.heads,
                         cfg.eps, cfg.prenorm, dtype)
        if on_block is not None:
            on_block("single", i, x)
    return final_layer(gw, x, n_txt, n_img, mod["final"], cfg.eps, cfg.prenorm, dtype)


def euler(z: np.ndarray, v: np.ndarray, sigma: float, sigma_next: float) -> np.ndarray:
    """Host flow-matching update between steps: z + (sigma_next - sigma) v.

    [card] header: the scheduler stays on the host.
    """
    return z + (sigma_next - sigma) * v


def denoise(velocity: Callable[[np.ndarray, np.ndarray], np.ndarray], z: np.ndarray,
            sigmas: np.ndarray) -> np.ndarray:
    """The sampling loop: for i = 0 .. n-1, v = velocity(z, sigma[:, i]) and
    z <- euler(z, v, sigma[:, i], sigma[:, i + 1]), per batch row.

    [card] Tasks table: 4 steps, one DiT call each (no CFG); header: the
    scheduler runs on the host, so the schedule sigmas [B, n + 1] is given.
    z [B, ...]; returns the latent after the last update.
    """
    sigmas = np.asarray(sigmas, dtype=np.float64)
    z = np.array(z, dtype=np.float64)
    for i in range(sigmas.shape[1] - 1):
        v = velocity(z, sigmas[:, i])
        shape = (-1,) + (1,) * (z.ndim - 1)
        z = euler(z, v, sigmas[:, i].reshape(shape), sigmas[:, i + 1].reshape(shape))
    return z


def denoise_dit(cfg, weights, txt: np.ndarray, z: np.ndarray, ref: Optional[np.ndarray],
                sigmas: np.ndarray, pos: np.ndarray, dtype=np.float64) -> np.ndarray:
    """The sampling loop with the DiT step as the velocity: each step sees the
    image latents z [B, n_img, C_in] followed by the fixed reference tokens
    ref [B, n_ref, C_in] (or None)."""
    n_img = z.shape[1]

    def velocity(zc, sig):
        lat = zc if ref is None else np.concatenate([zc, ref], axis=1)
        return step(cfg, weights, txt, lat, sig, n_img, pos, dtype)

    return denoise(velocity, z, sigmas)
