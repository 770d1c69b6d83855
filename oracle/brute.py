"""Brute-force float64 re-derivation of the DiT step for tiny shapes.

TEST INFRASTRUCTURE ONLY (checker code; never used by the product path).

Written independently of ``dit_oracle``: plain Python loops over tokens,
heads and pairs, Python floats (IEEE double), the ``math`` module, no NumPy
arithmetic. RoPE is done as a complex multiplication, norms and softmax as
explicit sums. It exists to pin the vectorised oracle: any index, transpose,
sign or ordering slip in either one shows up as a mismatch on tiny inputs.

Each function takes nested lists (or arrays, converted with .tolist()) and
follows the same readings of the pages as the oracle (see its header):
"flux2-klein-p100a" card "Caveats" and "tt_flux2_klein - Python reference"
"Things that are easy to get wrong" (global modulation, unmasked text rows,
RoPE 32 dims per axis / theta 2000 / adjacent pairs, reference t = 10 + 10 i).
"""
from __future__ import annotations

import cmath
import math
from typing import Dict, List, Sequence


def _l(a):
    return a.tolist() if hasattr(a, "tolist") else a


def dot(a: Sequence[float], b: Sequence[float]) -> float:
    s = 0.0
    for i in range(len(a)):
        s += a[i] * b[i]
    return s


def matvec(w: List[List[float]], x: Sequence[float]) -> List[float]:
    """w in [out][in] layout."""
    return [dot(row, x) for row in w]


def silu(v: float) -> float:
    return v / (1.0 + math.exp(-v))


def rms_normalize(x: Sequence[float], eps: float) -> List[float]:
    n = len(x)
    ss = 0.0
    for v in x:
        ss += v * v
    r = 1.0 / math.sqrt(ss / n + eps)
    return [v * r for v in x]


def layer_normalize(x: Sequence[float], eps: float) -> List[float]:
    n = len(x)
    mu = sum(x) / n
    var = 0.0
    for v in x:
        var += (v - mu) * (v - mu)
    r = 1.0 / math.sqrt(var / n + eps)
    return [(v - mu) * r for v in x]


def adaln(x, shift, scale, eps, layer=False) -> List[float]:
    n = layer_normalize(x, eps) if layer else rms_normalize(x, eps)
    return [n[i] * (1.0 + scale[i]) + shift[i] for i in range(len(n))]


def rotate(vec: Sequence[float], pos: Sequence[int], axes_dim=(32, 32, 32, 32),
           theta: float = 2000.0) -> List[float]:
    """Adjacent-pair rotation of a head vector, as complex multiplication."""
    out = list(vec)
    base = 0
    for a, dim in enumerate(axes_dim):
        for j in range(dim // 2):
            ang = pos[a] * math.pow(theta, -(2.0 * j) / dim)
            z = complex(vec[base + 2 * j], vec[base + 2 * j + 1]) * cmath.exp(1j * ang)
            out[base + 2 * j] = z.real
            out[base + 2 * j + 1] = z.imag
        base += dim
    return out


def attention_rows(q: List[List[float]], k: List[List[float]],
                   v: List[List[float]]) -> List[List[float]]:
    """One head: q, k, v as [S][d] lists; softmax(q k / sqrt d) v."""
    d = len(q[0])
    out = []
    for qi in q:
        logits = [dot(qi, kj) / math.sqrt(d) for kj in k]
        m = max(logits)
        e = [math.exp(t - m) for t in logits]
        z = sum(e)
        row = [0.0] * d
        for j, ej in enumerate(e):
            pj = ej / z
            for c in range(d):
                row[c] += pj * v[j][c]
        out.append(row)
    return out


def timestep_features(sigma: float, channels: int = 256) -> List[float]:
    half = channels // 2
    tau = 1000.0 * sigma
    freqs = [math.exp(-math.log(10000.0) * k / half) for k in range(half)]
    return [math.cos(tau * f) for f in freqs] + [math.sin(tau * f) for f in freqs]


def modulation(gw: Dict, sigma: float, channels: int = 256) -> Dict[str, List[List[float]]]:
    e = timestep_features(sigma, channels)
    h = [silu(t) for t in matvec(_l(gw["t_in"]), e)]
    temb = matvec(_l(gw["t_out"]), h)
    m = [silu(t) for t in temb]
    D = len(m)
    res = {}
    for name, key, n in (("dual_img", "mod_dual_img", 6), ("dual_txt", "mod_dual_txt", 6),
                         ("single", "mod_single", 3), ("final", "mod_final", 2)):
        flat = matvec(_l(gw[key]), m)
        res[name] = [flat[i * D:(i + 1) * D] for i in range(n)]
    return res


def _qk(vec, gain, pos, eps, axes_dim, theta):
    n = rms_normalize(vec, eps)
    return rotate([n[i] * gain[i] for i in range(len(n))], pos, axes_dim, theta)


def _attend_all(qs, ks, vs, heads, d):
    """qs/ks/vs: per token lists of length heads*d; returns per-token outputs."""
    S = len(qs)
    out = [[0.0] * (heads * d) for _ in range(S)]
    for h in range(heads):
        sl = slice(h * d, (h + 1) * d)
        oh = attention_rows([t[sl] for t in qs], [t[sl] for t in ks], [t[sl] for t in vs])
        for t in range(S):
            out[t][sl] = oh[t]
    return out


def dual_block(x, n_txt: int, w: Dict, mod_txt, mod_img, pos, heads: int,
               eps: float = 1e-6, layer: bool = False, axes_dim=(32, 32, 32, 32),
               theta: float = 2000.0) -> List[List[float]]:
    """One sample: x [S][D]; mod_* [6][D]; pos [S][4]."""
    x = _l(x)
    pos = _l(pos)
    S, D = len(x), len(x[0])
    d = D // heads
    W = {k: _l(v) for k, v in w.items()}
    mods = (_l(mod_txt), _l(mod_img))
    st = [0 if t < n_txt else 1 for t in range(S)]
    qs, ks, vs = [], [], []
    for t in range(S):
        s, md = st[t], mods[st[t]]
        h = adaln(x[t], md[0], md[1], eps, layer)
        u = matvec(W[f"qkv{s}"], h)
        q, k, v = u[:D], u[D:2 * D], u[2 * D:]
        qr, kr = [], []
        for hh in range(heads):
            sl = slice(hh * d, (hh + 1) * d)
            qr += _qk(q[sl], W[f"q_gain{s}"], pos[t], eps, axes_dim, theta)
            kr += _qk(k[sl], W[f"k_gain{s}"], pos[t], eps, axes_dim, theta)
        qs.append(qr)
        ks.append(kr)
        vs.append(v)
    o = _attend_all(qs, ks, vs, heads, d)
    x1 = []
    for t in range(S):
        s, md = st[t], mods[st[t]]
        y = matvec(W[f"out{s}"], o[t])
        x1.append([x[t][i] + md[2][i] * y[i] for i in range(D)])
    x2 = []
    for t in range(S):
        s, md = st[t], mods[st[t]]
        h2 = adaln(x1[t], md[3], md[4], eps, layer)
        u = matvec(W[f"mlp_in{s}"], h2)
        F = len(u) // 2
        a = [silu(u[i]) * u[F + i] for i in range(F)]
        y = matvec(W[f"mlp_out{s}"], a)
        x2.append([x1[t][i] + md[5][i] * y[i] for i in range(D)])
    return x2


def single_block(x, w: Dict, mod, pos, heads: int, eps: float = 1e-6,
                 layer: bool = False, axes_dim=(32, 32, 32, 32),
                 theta: float = 2000.0) -> List[List[float]]:
    """One sample: x [S][D]; mod [3][D]."""
    x = _l(x)
    pos = _l(pos)
    mod = _l(mod)
    S, D = len(x), len(x[0])
    d = D // heads
    w_in, w_out = _l(w["w_in"]), _l(w["w_out"])
    qg, kg = _l(w["q_gain"]), _l(w["k_gain"])
    qs, ks, vs, acts = [], [], [], []
    for t in range(S):
        h = adaln(x[t], mod[0], mod[1], eps, layer)
        u = matvec(w_in, h)
        q, k, v, m = u[:D], u[D:2 * D], u[2 * D:3 * D], u[3 * D:]
        F = len(m) // 2
        acts.append([silu(m[i]) * m[F + i] for i in range(F)])
        qr, kr = [], []
        for hh in range(heads):
            sl = slice(hh * d, (hh + 1) * d)
            qr += _qk(q[sl], qg, pos[t], eps, axes_dim, theta)
            kr += _qk(k[sl], kg, pos[t], eps, axes_dim, theta)
        qs.append(qr)
        ks.append(kr)
        vs.append(v)
    o = _attend_all(qs, ks, vs, heads, d)
    out = []
    for t in range(S):
        y = matvec(w_out, o[t] + acts[t])
        out.append([x[t][i] + mod[2][i] * y[i] for i in range(D)])
    return out


def step(cfg, weights, txt, lat, sigma: float, n_img: int, pos) -> List[List[float]]:
    """One sample's full step; returns v [n_img][C_in]."""
    gw = weights.glob
    eps, layer = cfg.eps, cfg.prenorm == 1
    mod = modulation(gw, sigma, cfg.time_channels)
    txt, lat = _l(txt), _l(lat)
    x = [matvec(_l(gw["ctx_embed"]), r) for r in txt] + [matvec(_l(gw["x_embed"]), r) for r in lat]
    n_txt = len(txt)
    for i in range(cfg.n_dual):
        x = dual_block(x, n_txt, weights.dual(i), mod["dual_txt"], mod["dual_img"], pos,
                       cfg.heads, eps, layer, cfg.axes_dim, cfg.theta)
    for i in range(cfg.n_single):
        x = single_block(x, weights.single(i), mod["single"], pos, cfg.heads, eps, layer,
                         cfg.axes_dim, cfg.theta)
    fm = mod["final"]
    wo = _l(gw["proj_out"])
    return [matvec(wo, adaln(x[t], fm[0], fm[1], eps, layer)) for t in range(n_txt, n_txt + n_img)]


# ------------------------------------------------------------ latent decoder
# Loop versions of the decoder's primitives for one sample, images as nested
# [H][W][C] lists, conv weights as [O][k][k][C] (the readings of the
# decoder's header in vae_oracle: cross-correlation with zero padding,
# GroupNorm over consecutive channel runs, nearest 2x upsampling, 2x2
# patches with token channel 4k + 2i + j).

def conv_image(x, w, b=None):
    x, w = _l(x), _l(w)
    H, W, C = len(x), len(x[0]), len(x[0][0])
    O, k = len(w), len(w[0])
    p = k // 2
    out = [[[0.0] * O for _ in range(W)] for _ in range(H)]
    for y in range(H):
        for xx in range(W):
            for o in range(O):
                s = 0.0 if b is None else float(_l(b)[o])
                for ky in range(k):
                    yy = y + ky - p
                    if yy < 0 or yy >= H:
                        continue
                    for kx in range(k):
                        xs = xx + kx - p
                        if xs < 0 or xs >= W:
                            continue
                        px, wk = x[yy][xs], w[o][ky][kx]
                        for c in range(C):
                            s += px[c] * wk[c]
                out[y][xx][o] = s
    return out


def group_norm_image(x, gamma, beta, groups: int, eps: float):
    x, gamma, beta = _l(x), _l(gamma), _l(beta)
    H, W, C = len(x), len(x[0]), len(x[0][0])
    cg = C // groups
    out = [[[0.0] * C for _ in range(W)] for _ in range(H)]
    for g in range(groups):
        vals = [x[y][xx][c] for y in range(H) for xx in range(W)
                for c in range(g * cg, (g + 1) * cg)]
        n = len(vals)
        mu = sum(vals) / n
        var = sum((v - mu) * (v - mu) for v in vals) / n
        r = 1.0 / math.sqrt(var + eps)
        for y in range(H):
            for xx in range(W):
                for c in range(g * cg, (g + 1) * cg):
                    out[y][xx][c] = (x[y][xx][c] - mu) * r * gamma[c] + beta[c]
    return out


def map_image(f, x):
    return [[[f(v) for v in px] for px in row] for row in _l(x)]


def add_images(a, b):
    return [[[u + v for u, v in zip(pa, pb)] for pa, pb in zip(ra, rb)]
            for ra, rb in zip(_l(a), _l(b))]


def upsample_image(x):
    x = _l(x)
    H, W = len(x), len(x[0])
    return [[list(x[y // 2][xx // 2]) for xx in range(2 * W)] for y in range(2 * H)]


def patchify_image(img):
    """[2hp][2wp][Z] -> tokens [hp * wp][4 Z], token (r, c) row-major,
    channel 4k + 2i + j = pixel (2r + i, 2c + j) channel k."""
    img = _l(img)
    hp, wp, Z = len(img) // 2, len(img[0]) // 2, len(img[0][0])
    toks = []
    for r in range(hp):
        for c in range(wp):
            t = [0.0] * (4 * Z)
            for k in range(Z):
                for i in range(2):
                    for j in range(2):
                        t[4 * k + 2 * i + j] = img[2 * r + i][2 * c + j][k]
            toks.append(t)
    return toks


def resnet_image(x, w, p: str, groups: int, eps: float):
    h = conv_image(map_image(silu, group_norm_image(x, w[p + "gn1.g"], w[p + "gn1.b"],
                                                    groups, eps)),
                   w[p + "conv1.w"], w[p + "conv1.b"])
    h = conv_image(map_image(silu, group_norm_image(h, w[p + "gn2.g"], w[p + "gn2.b"],
                                                    groups, eps)),
                   w[p + "conv2.w"], w[p + "conv2.b"])
    s = x if (p + "short.w") not in w else conv_image(x, w[p + "short.w"], w[p + "short.b"])
    return add_images(s, h)


def attention_block_image(x, w, p: str, groups: int, eps: float):
    x = _l(x)
    H, W = len(x), len(x[0])
    t = group_norm_image(x, w[p + "gn.g"], w[p + "gn.b"], groups, eps)
    flat = lambda im: [px for row in im for px in row]
    q = flat(conv_image(t, w[p + "q.w"], w[p + "q.b"]))
    k = flat(conv_image(t, w[p + "k.w"], w[p + "k.b"]))
    v = flat(conv_image(t, w[p + "v.w"], w[p + "v.b"]))
    o = attention_rows(q, k, v)
    o_img = [[o[y * W + xx] for xx in range(W)] for y in range(H)]
    return add_images(x, conv_image(o_img, w[p + "o.w"], w[p + "o.b"]))
