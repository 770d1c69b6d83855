"""GPU parity of the latent decoder: the HIP path (through the C ABI) against
the fp64 CPU oracle (oracle/vae_oracle.py) on the same seeded inputs.

Tolerances:
  * one convolution, one GroupNorm (bf16 output): |err| <= 2^-8 |ref| + 1e-3
    (one rounding of the fp32 result to bf16, whose unit roundoff is 2^-8,
    plus fp32 accumulation, about 1e-6 here, with room for the fp32 result
    itself to sit next to a rounding boundary); fp32 output:
    |err| <= 1e-5 |ref| + 1e-4;
  * the whole decoder: rel-L2 <= 2.5e-2 and max-abs <= 0.15 rms(ref). Every
    stored activation is rounded to bf16 (the oracle rounds nothing); that
    rounding alone, simulated in float64 on these decoders, gives rel-L2
    1.0-1.2e-2 and max-abs 0.054-0.075 rms(ref); the bounds are twice that.
"""
import contextlib
import os

import numpy as np
import pytest

from diffusion_transformer_fwd_amd import dit, synth
from oracle import vae_oracle as V
from gpu_helpers import log, to_np

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

DEC_REL_L2 = 2.5e-2
DEC_MAX_OVER_RMS = 0.15


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    dit.lib()


@contextlib.contextmanager
def attn_rows(n):
    old = os.environ.get("DIT_VAE_ATTN_ROWS")
    os.environ["DIT_VAE_ATTN_ROWS"] = str(n)
    try:
        yield
    finally:
        if old is None:
            del os.environ["DIT_VAE_ATTN_ROWS"]
        else:
            os.environ["DIT_VAE_ATTN_ROWS"] = old


def check_bf16_result(got, ref, what):
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-3
    worst = float((err / bound).max())
    log(f"{what}: max_abs {err.max():.3e}, worst err/bound {worst:.3f}")
    assert worst <= 1.0, f"{what}: err/bound {worst:.3f}"


# ---------------------------------------------------------------- one convolution

# (name, B, H, W, c_in, ksize, up, c_out, c_short, resid, out_f32)
CONV_CASES = [
    ("conv_in_c32", 1, 16, 24, 32, 3, 0, 512, 0, False, False),
    ("ragged_n40_b2_resid", 2, 10, 14, 64, 3, 0, 40, 0, True, False),
    ("upsample_c128", 1, 12, 20, 128, 3, 1, 128, 0, False, False),
    ("shortcut_512_to_256", 1, 16, 16, 256, 3, 0, 256, 512, False, False),
    ("conv_out_n3_f32_b2", 2, 18, 26, 128, 3, 0, 3, 0, False, True),
    ("one_by_one_resid", 1, 8, 40, 512, 1, 0, 512, 0, True, False),
    ("n128_tall", 1, 40, 36, 256, 3, 0, 128, 0, False, False),
    ("wide_512_b2_resid", 2, 20, 70, 512, 3, 0, 512, 0, True, False),
    ("upsample_512_ragged", 1, 18, 46, 512, 3, 1, 256, 0, False, False),
]


@pytest.mark.parametrize("case", CONV_CASES, ids=[c[0] for c in CONV_CASES])
def test_conv_against_oracle(case):
    name, B, H, W, ci, k, up, co, cs, use_res, f32 = case
    log(f"conv {name}")
    Hi, Wi = (H // 2, W // 2) if up else (H, W)
    x = np.stack([synth.normal(b, "t.conv.x", (Hi, Wi, ci)) for b in range(B)])
    w = synth._conv_w(0, "t.conv.w", co, k, ci)
    bias = synth.normal(0, "t.conv.b", (co,), std=0.1)
    ref_in = V.upsample2x(x.astype(np.float64)) if up else x.astype(np.float64)
    ref = V.conv2d(ref_in, w.astype(np.float64), bias.astype(np.float64))
    kw = {}
    if cs:
        xs = np.stack([synth.normal(b, "t.conv.xs", (H, W, cs)) for b in range(B)])
        ws = synth._conv_w(0, "t.conv.ws", co, 1, cs)
        bs = synth.normal(0, "t.conv.bs", (co,), std=0.1)
        ref = ref + V.conv2d(xs.astype(np.float64), ws.astype(np.float64), bs.astype(np.float64))
        kw = dict(xs=dit.to_bf16_device(xs), c_short=cs, short_w=dit.to_bf16_device(ws),
                  short_b=dit.to_f32_device(bs))
    if use_res:
        res = np.stack([synth.normal(b, "t.conv.res", (H, W, co)) for b in range(B)])
        ref = ref + res
        kw["resid"] = dit.to_bf16_device(res)
    xd = dit.to_bf16_device(x)
    wd = dit.to_bf16_device(w)
    bd = dit.to_f32_device(bias)
    out = dit.vae_conv(xd, ci, k, up, wd, bd, B, H, W, co, out_f32=f32, **kw)
    torch.cuda.synchronize()
    got = to_np(out).astype(np.float64)
    if f32:
        err = np.abs(got - ref)
        worst = float((err / (1e-5 * np.abs(ref) + 1e-4)).max())
        log(f"{name}: max_abs {err.max():.3e}, worst err/bound {worst:.3f}")
        assert worst <= 1.0
    else:
        check_bf16_result(got, ref, name)
    if B > 1:
        # each batch row alone gives the same bits
        for b in range(B):
            one = dit.vae_conv(xd[b:b + 1], ci, k, up, wd, bd, 1, H, W, co, out_f32=f32,
                               **{kk: (v[b:b + 1] if kk in ("xs", "resid") else v)
                                  for kk, v in kw.items()})
            torch.cuda.synchronize()
            assert torch.equal(one[0], out[b]), f"{name}: batch row {b} differs alone"


@contextlib.contextmanager
def conv_tile(c):
    old = os.environ.get("DIT_CONV_TILE")
    os.environ["DIT_CONV_TILE"] = str(c)
    try:
        yield
    finally:
        if old is None:
            del os.environ["DIT_CONV_TILE"]
        else:
            os.environ["DIT_CONV_TILE"] = old


# tile shapes of the conv launcher: 0-3 implicit GEMM (256x256, 512x128,
# 256x128, 512x32), 4-5 halo (8x32 pixels x 256 or 128 channels)
TILE_SHAPES = range(6)


@pytest.mark.parametrize("case", [("c128_up", 2, 12, 40, 128, 1, 192, 0), ("c256_ragged", 1, 13, 37, 256, 0, 72, 0),
                                  ("c64", 1, 9, 70, 64, 0, 128, 0),
                                  ("c256_short128_b2", 2, 11, 45, 256, 0, 256, 128),
                                  ("c128_short64_ragged", 1, 9, 35, 128, 0, 40, 64)], ids=lambda c: c[0])
def test_conv_tile_shapes_bitwise(case):
    """Every tile shape (both kernels) gives the same bits for one conv: the
    same k-steps in the same order, whatever the tiling, the 1x1 shortcut's
    slices after the 3x3 slices. (A conv with a shortcut has no halo shape:
    asking for one falls back to the planned implicit tile.)"""
    name, B, H, W, ci, up, co, cs = case
    Hi, Wi = (H // 2, W // 2) if up else (H, W)
    x = dit.to_bf16_device(np.stack([synth.normal(b, "t.tile.x", (Hi, Wi, ci)) for b in range(B)]))
    w = dit.to_bf16_device(synth._conv_w(0, "t.tile.w", co, 3, ci))
    bias = dit.to_f32_device(synth.normal(0, "t.tile.b", (co,), std=0.1))
    kw = {}
    if cs:
        kw = dict(xs=dit.to_bf16_device(np.stack([synth.normal(b, "t.tile.xs", (H, W, cs)) for b in range(B)])),
                  c_short=cs, short_w=dit.to_bf16_device(synth._conv_w(0, "t.tile.ws", co, 1, cs)),
                  short_b=dit.to_f32_device(synth.normal(0, "t.tile.bs", (co,), std=0.1)))
    outs = []
    for c in TILE_SHAPES:
        with conv_tile(c):
            outs.append(dit.vae_conv(x, ci, 3, up, w, bias, B, H, W, co, **kw))
    torch.cuda.synchronize()
    for c in TILE_SHAPES[1:]:
        assert torch.equal(outs[0], outs[c]), f"{name}: tile shape {c} differs from shape 0"
    log(f"{name}: {len(TILE_SHAPES)} tile shapes bitwise equal")


# ---------------------------------------------------------------- GroupNorm

# (B, HW, C, groups, silu, offset)
GN_CASES = [(1, 4096, 128, 32, True, 0.0), (2, 333, 512, 32, False, 0.0),
            (1, 77, 64, 32, True, 0.0), (3, 1000, 32, 8, True, 6.0), (1, 20000, 256, 32, True, 0.0)]


@pytest.mark.parametrize("case", GN_CASES, ids=[f"b{c[0]}_hw{c[1]}_c{c[2]}_g{c[3]}" for c in GN_CASES])
def test_group_norm_against_oracle(case):
    B, HW, Cc, G, act, off = case
    log(f"group norm {case}")
    x = np.stack([synth.normal(b, "t.gn.x", (HW, Cc), std=2.0, mean=off) for b in range(B)])
    g = synth.normal(0, "t.gn.g", (Cc,), std=0.1, mean=1.0)
    be = synth.normal(0, "t.gn.b", (Cc,), std=0.1)
    ref = V.group_norm(x.astype(np.float64)[:, None], g.astype(np.float64),
                       be.astype(np.float64), G, 1e-6)[:, 0]
    if act:
        ref = V.silu(ref)
    y = dit.vae_group_norm(dit.to_bf16_device(x), dit.to_f32_device(g), dit.to_f32_device(be),
                           B, HW, Cc, G, 1e-6, act)
    torch.cuda.synchronize()
    check_bf16_result(to_np(y), ref, f"group norm {case}")


# ---------------------------------------------------------------- the decoder

_WEIGHTS = {}


def vae_weights(vcfg):
    if vcfg not in _WEIGHTS:
        host = synth.vae_weights(vcfg, 0)
        _WEIGHTS[vcfg] = (host, dit.VaeWeights(vcfg, host))
    return _WEIGHTS[vcfg]


def check_decode(got, ref, what):
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    d = got - ref
    rms = float(np.sqrt((ref ** 2).mean()))
    ma = float(np.abs(d).max())
    rl = float(np.linalg.norm(d) / np.linalg.norm(ref))
    log(f"{what}: max_abs {ma:.3e} ({ma / rms:.3f} rms) rel_l2 {rl:.3e}")
    assert rl <= DEC_REL_L2 and ma <= DEC_MAX_OVER_RMS * rms, what


def decode_both(vcfg, B, hp, wp):
    host, dev = vae_weights(vcfg)
    z = np.stack([synth.vae_latents(vcfg, b, hp, wp) for b in range(B)])
    ref = V.decode(vcfg, host, z, hp, wp)
    img = dit.vae_decode(vcfg, dev, dit.to_f32_device(z), hp, wp)
    torch.cuda.synchronize()
    return z, ref, img


# (config name, B, hp, wp)
DECODE_CASES = [("tiny", 1, 3, 5), ("tiny", 2, 4, 3), ("tiny", 1, 1, 1), ("klein", 1, 2, 3),
                ("klein", 1, 8, 8), ("klein", 2, 3, 5)]
CFGS = {"tiny": synth.VAE_TINY, "klein": synth.VAE_KLEIN}


@pytest.mark.parametrize("case", DECODE_CASES, ids=[f"{c[0]}_b{c[1]}_{c[2]}x{c[3]}" for c in DECODE_CASES])
def test_decode_against_oracle(case):
    name, B, hp, wp = case
    log(f"decode {case}")
    vcfg = CFGS[name]
    z, ref, img = decode_both(vcfg, B, hp, wp)
    assert tuple(img.shape) == (B, 16 * hp, 16 * wp, 3)
    check_decode(to_np(img), ref, f"decode {case}")


def test_decode_batch_rows_bitwise_independent():
    vcfg = synth.VAE_KLEIN
    _, dev = vae_weights(vcfg)
    hp, wp = 4, 6
    z = np.stack([synth.vae_latents(vcfg, b, hp, wp) for b in range(3)])
    zd = dit.to_f32_device(z)
    both = dit.vae_decode(vcfg, dev, zd, hp, wp)
    for b in range(3):
        one = dit.vae_decode(vcfg, dev, zd[b:b + 1].contiguous(), hp, wp)
        torch.cuda.synchronize()
        assert torch.equal(one[0], both[b]), f"batch row {b} differs when decoded alone"


def test_decode_tile_plan_and_folded_group_norm_bitwise():
    """The decode with every conv on the implicit GEMM's 256 x 256 tiles and
    every GroupNorm written out by its own pass equals the planned decode
    (halo convs with the GroupNorm folded into their input), bit for bit."""
    vcfg = synth.VAE_KLEIN
    _, dev = vae_weights(vcfg)
    hp, wp = 5, 7
    z = dit.to_f32_device(np.stack([synth.vae_latents(vcfg, b, hp, wp) for b in range(2)]))
    planned = dit.vae_decode(vcfg, dev, z, hp, wp)
    with conv_tile(0):
        plain = dit.vae_decode(vcfg, dev, z, hp, wp)
    # every 3x3 conv without a shortcut on one halo shape, GroupNorm folded
    forced = []
    for c in (4, 5):
        with conv_tile(c):
            forced.append(dit.vae_decode(vcfg, dev, z, hp, wp))
    torch.cuda.synchronize()
    assert torch.equal(planned, plain), "tile plan / folded GroupNorm changed the decode"
    for c, img in zip((4, 5), forced):
        assert torch.equal(img, plain), f"halo shape {c} with folded GroupNorm changed the decode"


def test_decode_chunked_attention_matches_whole():
    # 16 x 16 tokens = 32 x 32 latent pixels = 1024 queries, run as four
    # chunks of 256 rows
    vcfg = synth.VAE_TINY
    host, dev = vae_weights(vcfg)
    hp, wp = 16, 16
    z = synth.vae_latents(vcfg, 0, hp, wp)[None]
    zd = dit.to_f32_device(z)
    whole = dit.vae_decode(vcfg, dev, zd, hp, wp)
    with attn_rows(256):
        chunked = dit.vae_decode(vcfg, dev, zd, hp, wp)
    torch.cuda.synchronize()
    assert torch.equal(whole, chunked), "query chunking changed the result"
    ref = V.decode(vcfg, host, z, hp, wp)
    check_decode(to_np(chunked), ref, "decode tiny 16x16 chunked")


# ---------------------------------------------------------------- full size

def _golden(name):
    path = os.path.join(GOLDEN, f"{name}.npz")
    if not os.path.exists(path):
        pytest.fail(f"{path} missing: run tests/golden/make_golden.py {name}")
    return np.load(path)


@pytest.mark.parametrize("wl", [synth.V_DECODE_1024, synth.V_DECODE_1920x1088_B4],
                         ids=lambda w: w.name)
def test_decode_full_size_against_golden(wl):
    """The decodes the bench times, against the oracle's stored images:
    every pixel at 1024x1024; at 1920x1088 batch 4 every 16th pixel row of
    each batch row, plus each row's whole-image sum of squares
    (| |g|^2 - |r|^2 | <= (2 + e) e |r|^2 for rel-L2 e)."""
    g = _golden(wl.name)
    vcfg = synth.VAE_KLEIN
    _, dev = vae_weights(vcfg)
    hp, wp = wl.grid
    log(f"full-size decode {wl.name}")
    z = np.stack([synth.vae_latents(vcfg, b, hp, wp) for b in range(wl.batch)])
    img = dit.vae_decode(vcfg, dev, dit.to_f32_device(z), hp, wp)
    torch.cuda.synchronize()
    rows = g["rows"]
    got = to_np(img[:, torch.from_numpy(rows).cuda()]).astype(np.float64)
    ref = g["image"].astype(np.float64)
    assert got.shape == ref.shape
    what = f"{wl.name} ({'every pixel' if len(rows) == 16 * hp else f'{len(rows)} rows'})"
    check_decode(got, ref, what)
    ss = (img.double() ** 2).sum(dim=(1, 2, 3)).cpu().numpy()
    e = DEC_REL_L2
    rel = np.abs(ss - g["sumsq"]) / g["sumsq"]
    log(f"{wl.name}: sum of squares rel diff {rel.max():.3e}")
    assert np.all(rel <= (2 + e) * e)
