"""Pins for the decoder oracle (oracle/vae_oracle.py): checks against the
mathematics of each primitive and against special cases of the composition,
never against the oracle's own formulas retyped.

  * loop versions of every primitive (oracle/brute.py) on tiny tensors;
  * closed forms: a unit impulse fixes the convolution's orientation, a
    1x1 kernel is a matrix product, GroupNorm output has zero mean and
    var / (var + eps) variance per group, one channel per group is instance
    norm and one group is layer norm, a constant group maps to beta, equal
    keys average the values;
  * the composition: with the second conv of every ResNet and attention's
    output conv zeroed, each block is the identity; with identity upsample
    convs as well, the whole decoder reduces to
    conv_out(SiLU(GN(up(up(up(conv_in(u))))))), computed with the loop
    primitives;
  * planted mistakes that one of the pins must catch: slips put into the
    oracle module itself (a dropped bias, a flipped kernel, eps outside the
    root, unbiased or per-row GroupNorm statistics, SiLU as a sigmoid, an
    upsample off by one row, a sliced shortcut, SiLU before the norm, a
    1 / C score scale, softmax over queries, a channel-major patch order).
The layer list itself is a reading with nothing on the pages to check it
against.
"""
import math

import numpy as np
import pytest

from oracle import brute
from oracle import vae_oracle as V
from diffusion_transformer_fwd_amd import synth

RNG = np.random.default_rng(1234)


def _img(h, w, c):
    return RNG.standard_normal((1, h, w, c))


def test_conv_matches_loops_3x3_and_1x1():
    x = _img(4, 5, 3)
    for k in (3, 1):
        w = RNG.standard_normal((2, k, k, 3))
        b = RNG.standard_normal(2)
        got = V.conv2d(x, w, b, band=3)
        ref = np.array(brute.conv_image(x[0], w, b))
        np.testing.assert_allclose(got[0], ref, rtol=0, atol=1e-12)


def test_conv_impulse_fixes_orientation():
    # cross-correlation: an impulse at (y0, x0) channel c puts w[o, ky, kx, c]
    # at output (y0 + 1 - ky, x0 + 1 - kx)
    H, W, C = 5, 6, 2
    w = RNG.standard_normal((3, 3, 3, C))
    y0, x0, c = 2, 3, 1
    x = np.zeros((1, H, W, C))
    x[0, y0, x0, c] = 1.0
    out = V.conv2d(x, w, None)
    for ky in range(3):
        for kx in range(3):
            np.testing.assert_array_equal(out[0, y0 + 1 - ky, x0 + 1 - kx], w[:, ky, kx, c])
    # nothing else is touched
    mask = np.ones((H, W), bool)
    mask[y0 - 1:y0 + 2, x0 - 1:x0 + 2] = False
    assert np.all(out[0][mask] == 0.0)


def test_conv_border_is_zero_padded():
    # an all-ones image and all-ones kernel count the in-bounds taps
    x = np.ones((1, 4, 5, 1))
    w = np.ones((1, 3, 3, 1))
    out = V.conv2d(x, w, None)[0, :, :, 0]
    rows = np.array([2, 3, 3, 2])[:, None]
    cols = np.array([2, 3, 3, 3, 2])[None, :]
    np.testing.assert_array_equal(out, rows * cols)


def test_conv_1x1_is_matrix_product():
    x = _img(3, 4, 5)
    w = RNG.standard_normal((7, 1, 1, 5))
    b = RNG.standard_normal(7)
    got = V.conv2d(x, w, b)
    ref = np.einsum("bhwc,oc->bhwo", x, w[:, 0, 0, :]) + b
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("groups", [1, 2, 4, 8])
def test_group_norm_matches_loops(groups):
    x = _img(3, 4, 8) * 3 + 1.5
    g = RNG.standard_normal(8)
    b = RNG.standard_normal(8)
    got = V.group_norm(x, g, b, groups, 1e-6)
    ref = np.array(brute.group_norm_image(x[0], g, b, groups, 1e-6))
    np.testing.assert_allclose(got[0], ref, rtol=0, atol=1e-12)


def test_group_norm_closed_forms():
    B, H, W, C, G, eps = 2, 5, 3, 12, 4, 1e-6
    x = RNG.standard_normal((B, H, W, C)) * 2.0 + 7.0
    y = V.group_norm(x, np.ones(C), np.zeros(C), G, eps)
    for b in range(B):
        for g in range(G):
            xs = x[b, :, :, 3 * g:3 * g + 3]
            ys = y[b, :, :, 3 * g:3 * g + 3]
            var = xs.var()
            assert abs(ys.mean()) < 1e-12
            assert abs(ys.var() - var / (var + eps)) < 1e-12
    # one channel per group: each channel normalized over H * W on its own
    y1 = V.group_norm(x, np.ones(C), np.zeros(C), C, eps)
    for c in range(C):
        xc = x[0, :, :, c]
        np.testing.assert_allclose(y1[0, :, :, c], (xc - xc.mean()) / math.sqrt(xc.var() + eps),
                                   atol=1e-12)
    # one group: the whole sample normalized together
    yl = V.group_norm(x, np.ones(C), np.zeros(C), 1, eps)
    np.testing.assert_allclose(yl[1], (x[1] - x[1].mean()) / math.sqrt(x[1].var() + eps),
                               atol=1e-12)
    # a constant group maps to beta
    xc = x.copy()
    xc[:, :, :, 0:3] = 4.25
    beta = RNG.standard_normal(C)
    yc = V.group_norm(xc, RNG.standard_normal(C), beta, G, eps)
    np.testing.assert_allclose(yc[:, :, :, 0:3], np.broadcast_to(beta[0:3], yc[:, :, :, 0:3].shape),
                               atol=1e-12)


def test_upsample_index_map():
    x = _img(3, 4, 2)
    u = V.upsample2x(x)
    assert u.shape == (1, 6, 8, 2)
    np.testing.assert_array_equal(u[0], np.array(brute.upsample_image(x[0])))
    for y in range(6):
        for xx in range(8):
            np.testing.assert_array_equal(u[0, y, xx], x[0, y // 2, xx // 2])


def test_unpatchify_inverts_loop_patchify():
    img = RNG.standard_normal((6, 10, 3))
    toks = np.array(brute.patchify_image(img))[None]
    np.testing.assert_array_equal(V.unpatchify(toks, 3, 5, 3)[0], img)


def test_attention_matches_loops_and_closed_forms():
    q, k, v = (RNG.standard_normal((7, 4)) for _ in range(3))
    np.testing.assert_allclose(V.attention(q, k, v, chunk=3),
                               np.array(brute.attention_rows(q, k, v)), atol=1e-12)
    # equal keys: uniform weights, every output is the mean of the values
    ke = np.tile(RNG.standard_normal(4), (7, 1))
    np.testing.assert_allclose(V.attention(q, ke, v), np.tile(v.mean(0), (7, 1)), atol=1e-12)
    # permuting keys with their values changes nothing
    p = RNG.permutation(7)
    np.testing.assert_allclose(V.attention(q, k[p], v[p]), V.attention(q, k, v), atol=1e-12)


def _tiny_weights(vcfg, seed=0):
    return {k: v.astype(np.float64) for k, v in synth.vae_weights(vcfg, seed).items()}


def test_resnet_and_attention_blocks_match_loops():
    vcfg = synth.VaeConfig(z_channels=4, block_channels=(4, 8, 8, 8), layers=1, groups=4)
    w = _tiny_weights(vcfg)
    x = _img(3, 4, 8)
    # identity shortcut (8 -> 8) and 1x1 shortcut (8 -> 4)
    for p, ci in (("mid.res0.", 8), ("up3.res0.", 8)):
        got = V.resnet(x, w, p, 4, 1e-6)
        ref = np.array(brute.resnet_image(x[0], w, p, 4, 1e-6))
        np.testing.assert_allclose(got[0], ref, rtol=0, atol=1e-11)
    got = V.attention_block(x, w, "mid.attn.", 4, 1e-6)
    ref = np.array(brute.attention_block_image(x[0], w, "mid.attn.", 4, 1e-6))
    np.testing.assert_allclose(got[0], ref, rtol=0, atol=1e-11)


def _reduced(vcfg, w):
    """Zero every ResNet's second conv and attention's output conv, and make
    every upsample conv a center-tap identity."""
    w = dict(w)
    for p, _, _ in vcfg.resnet_channels():
        w[p + "conv2.w"] = np.zeros_like(w[p + "conv2.w"])
        w[p + "conv2.b"] = np.zeros_like(w[p + "conv2.b"])
    w["mid.attn.o.w"] = np.zeros_like(w["mid.attn.o.w"])
    w["mid.attn.o.b"] = np.zeros_like(w["mid.attn.o.b"])
    for lv in range(len(vcfg.level_channels) - 1):
        c = vcfg.level_channels[lv]
        e = np.zeros((c, 3, 3, c))
        e[np.arange(c), 1, 1, np.arange(c)] = 1.0
        w[f"up{lv}.upconv.w"] = e
        w[f"up{lv}.upconv.b"] = np.zeros(c)
    return w


def test_decoder_reduces_to_conv_in_upsample_conv_out():
    vcfg = synth.VaeConfig(z_channels=4, block_channels=(8, 8, 8, 8), layers=2, groups=4)
    w = _reduced(vcfg, _tiny_weights(vcfg))
    hp, wp = 1, 2
    z = RNG.standard_normal((1, hp * wp, 16))
    got = V.decode(vcfg, w, z, hp, wp)
    assert got.shape == (1, 16 * hp, 16 * wp, 3)
    # the same path from loop primitives, with the affine and patch order
    # taken token by token
    u = [[z[0, t, c] * w["lat_scale"][c] + w["lat_shift"][c] for c in range(16)]
         for t in range(hp * wp)]
    lat = [[[0.0] * 4 for _ in range(2 * wp)] for _ in range(2 * hp)]
    for r in range(hp):
        for c in range(wp):
            for k in range(4):
                for i in range(2):
                    for j in range(2):
                        lat[2 * r + i][2 * c + j][k] = u[r * wp + c][4 * k + 2 * i + j]
    x = brute.conv_image(lat, w["conv_in.w"], w["conv_in.b"])
    for _ in range(3):
        x = brute.upsample_image(x)
    x = brute.map_image(brute.silu, brute.group_norm_image(x, w["norm_out.g"], w["norm_out.b"],
                                                           4, 1e-6))
    ref = np.array(brute.conv_image(x, w["conv_out.w"], w["conv_out.b"]))
    np.testing.assert_allclose(got[0], ref, rtol=0, atol=1e-11)


def test_zeroed_branches_are_identities():
    vcfg = synth.VaeConfig(z_channels=4, block_channels=(8, 8, 8, 8), layers=1, groups=4)
    w = _reduced(vcfg, _tiny_weights(vcfg))
    x = _img(3, 5, 8)
    np.testing.assert_array_equal(V.resnet(x, w, "mid.res0.", 4, 1e-6), x)
    np.testing.assert_array_equal(V.attention_block(x, w, "mid.attn.", 4, 1e-6), x)


def test_decode_batch_rows_independent_and_fp32_close():
    vcfg = synth.VaeConfig(z_channels=4, block_channels=(8, 8, 16, 16), layers=1, groups=4)
    w = synth.vae_weights(vcfg, 0)
    z = np.stack([synth.vae_latents(vcfg, s, 2, 3) for s in (0, 1)])
    both = V.decode(vcfg, w, z, 2, 3)
    for b in range(2):
        one = V.decode(vcfg, w, z[b:b + 1], 2, 3)
        np.testing.assert_allclose(both[b], one[0], rtol=0, atol=1e-12)
    f32 = V.decode(vcfg, w, z, 2, 3, dtype=np.float32)
    rel = np.linalg.norm(f32 - both) / np.linalg.norm(both)
    assert rel < 1e-5


def test_decode_flops_counts_every_contraction():
    # count 2 * MACs from the layer list of a tiny decoder by hand
    vcfg = synth.VaeConfig(z_channels=4, block_channels=(8, 16, 16, 32), layers=1, groups=4)
    hp, wp = 2, 3
    H, W = 4, 6
    f = 2 * H * W * 32 * 9 * 4                        # conv_in
    f += 2 * 2 * H * W * 32 * 9 * 64                   # mid ResNets, two 3x3 convs each
    n = H * W
    f += 2 * n * 32 * 32 * 4 + 4 * n * n * 32          # q, k, v, o and the two products
    f += 2 * H * W * 32 * 9 * 64                       # up0 ResNet 32 -> 32
    f += 2 * (2 * H) * (2 * W) * 32 * 9 * 32           # up0 upsample conv
    f += 2 * (2 * H) * (2 * W) * (16 * 9 * 32 + 16 * 9 * 16 + 16 * 32)  # up1 32 -> 16
    f += 2 * (4 * H) * (4 * W) * 16 * 9 * 16           # up1 upsample conv
    f += 2 * (4 * H) * (4 * W) * 16 * 9 * 32           # up2 ResNet 16 -> 16
    f += 2 * (8 * H) * (8 * W) * 16 * 9 * 16           # up2 upsample conv
    f += 2 * (8 * H) * (8 * W) * (8 * 9 * 16 + 8 * 9 * 8 + 8 * 16)  # up3 16 -> 8
    f += 2 * (8 * H) * (8 * W) * 3 * 9 * 8             # conv_out
    assert V.decode_flops(vcfg, 1, hp, wp) == f
    assert V.decode_flops(vcfg, 3, hp, wp) == 3 * f


# ---------------------------------------------------------------- planted mistakes

def test_planted_flipped_kernel_is_caught():
    def conv_flipped(x, w, b, band=64):
        return V.conv2d(x, w[:, ::-1, ::-1, :], b, band)
    H, W, C = 5, 6, 2
    w = RNG.standard_normal((3, 3, 3, C))
    x = np.zeros((1, H, W, C))
    x[0, 2, 3, 1] = 1.0
    out = conv_flipped(x, w, None)
    assert not np.array_equal(out[0, 3, 4], w[:, 0, 0, 1])


def test_planted_patch_order_is_caught():
    img = RNG.standard_normal((4, 6, 3))
    toks = np.array(brute.patchify_image(img))[None]

    def unpatchify_swapped(z, hp, wp, zc):
        x = z.reshape(1, hp, wp, zc, 2, 2).transpose(0, 1, 5, 2, 4, 3)
        return x.reshape(1, 2 * hp, 2 * wp, zc)
    assert not np.array_equal(unpatchify_swapped(toks, 2, 3, 3)[0], img)


def test_planted_per_channel_norm_is_caught():
    x = _img(3, 4, 8)
    g, b = np.ones(8), np.zeros(8)
    wrong = V.group_norm(x, g, b, 8, 1e-6)   # stats per channel instead of per group of 2
    ref = np.array(brute.group_norm_image(x[0], g, b, 4, 1e-6))
    assert np.abs(wrong[0] - ref).max() > 1e-3


# Planted mistakes in the oracle module itself: each mutant below is a
# plausible slip in one oracle function, patched into the module; at least one
# of the listed pins (which compare against loops and closed forms, not the
# oracle's own formulas) must then fail.
_conv2d, _group_norm, _silu, _upsample2x = V.conv2d, V.group_norm, V.silu, V.upsample2x
_resnet, _attention, _unpatchify = V.resnet, V.attention, V.unpatchify


def _gn_eps_outside_root(x, gamma, beta, groups, eps):
    B, H, W, C = x.shape
    xr = x.reshape(B, H * W, groups, C // groups)
    d = xr - xr.mean(axis=(1, 3), keepdims=True)
    sd = np.sqrt((d * d).mean(axis=(1, 3), keepdims=True))
    return (d / (sd + eps)).reshape(B, H, W, C) * gamma + beta


def _gn_unbiased(x, gamma, beta, groups, eps):
    B, H, W, C = x.shape
    xr = x.reshape(B, H * W, groups, C // groups)
    d = xr - xr.mean(axis=(1, 3), keepdims=True)
    n = H * W * (C // groups)
    var = (d * d).sum(axis=(1, 3), keepdims=True) / (n - 1)
    return (d / np.sqrt(var + eps)).reshape(B, H, W, C) * gamma + beta


def _gn_stats_over_width_only(x, gamma, beta, groups, eps):
    # statistics per (sample, row, group) instead of per (sample, group)
    B, H, W, C = x.shape
    xr = x.reshape(B, H, W, groups, C // groups)
    d = xr - xr.mean(axis=(2, 4), keepdims=True)
    var = (d * d).mean(axis=(2, 4), keepdims=True)
    return (d / np.sqrt(var + eps)).reshape(B, H, W, C) * gamma + beta


def _resnet_no_shortcut_conv(x, w, p, groups, eps):
    h = _conv2d(_silu(_group_norm(x, w[p + "gn1.g"], w[p + "gn1.b"], groups, eps)),
                w[p + "conv1.w"], w[p + "conv1.b"])
    h = _conv2d(_silu(_group_norm(h, w[p + "gn2.g"], w[p + "gn2.b"], groups, eps)),
                w[p + "conv2.w"], w[p + "conv2.b"])
    if (p + "short.w") in w:
        return h + x[..., :h.shape[-1]]
    return x + h


def _resnet_silu_before_norm(x, w, p, groups, eps):
    h = _conv2d(_group_norm(_silu(x), w[p + "gn1.g"], w[p + "gn1.b"], groups, eps),
                w[p + "conv1.w"], w[p + "conv1.b"])
    h = _conv2d(_silu(_group_norm(h, w[p + "gn2.g"], w[p + "gn2.b"], groups, eps)),
                w[p + "conv2.w"], w[p + "conv2.b"])
    s = x if (p + "short.w") not in w else _conv2d(x, w[p + "short.w"], w[p + "short.b"])
    return s + h


def _attention_scale_by_c(q, k, v, chunk=2048):
    return _attention(q * math.sqrt(q.shape[-1]) / q.shape[-1], k, v, chunk)


def _attention_softmax_over_queries(q, k, v, chunk=2048):
    s = (q @ k.T) / math.sqrt(q.shape[-1])
    e = np.exp(s - s.max(axis=0, keepdims=True))
    return (e / e.sum(axis=0, keepdims=True)) @ v


def _unpatchify_channel_major(z, hp, wp, z_ch):
    B = z.shape[0]
    x = z.reshape(B, hp, wp, 2, 2, z_ch).transpose(0, 1, 3, 2, 4, 5)
    return x.reshape(B, 2 * hp, 2 * wp, z_ch)


_MUTANTS = {
    "conv_without_bias": ("conv2d", lambda x, w, b, band=64: _conv2d(x, w, None, band),
                          [test_conv_matches_loops_3x3_and_1x1, test_conv_1x1_is_matrix_product]),
    "conv_true_convolution": ("conv2d",
                              lambda x, w, b, band=64: _conv2d(x, w[:, ::-1, ::-1, :], b, band),
                              [test_conv_impulse_fixes_orientation]),
    "gn_eps_outside_root": ("group_norm", _gn_eps_outside_root,
                            [test_group_norm_closed_forms]),
    "gn_unbiased_variance": ("group_norm", _gn_unbiased, [test_group_norm_closed_forms]),
    "gn_stats_per_row": ("group_norm", _gn_stats_over_width_only,
                         [lambda: test_group_norm_matches_loops(2), test_group_norm_closed_forms]),
    "silu_as_sigmoid": ("silu", lambda x: 1.0 / (1.0 + np.exp(-x)),
                        [test_resnet_and_attention_blocks_match_loops]),
    "upsample_offset_by_one": ("upsample2x",
                               lambda x: np.concatenate([_upsample2x(x)[:, 1:], _upsample2x(x)[:, -1:]], 1),
                               [test_upsample_index_map]),
    "resnet_shortcut_sliced": ("resnet", _resnet_no_shortcut_conv,
                               [test_resnet_and_attention_blocks_match_loops]),
    "resnet_silu_before_norm": ("resnet", _resnet_silu_before_norm,
                                [test_resnet_and_attention_blocks_match_loops]),
    "attention_scaled_by_c": ("attention", _attention_scale_by_c,
                              [test_resnet_and_attention_blocks_match_loops]),
    "attention_softmax_over_queries": ("attention", _attention_softmax_over_queries,
                                       [test_attention_matches_loops_and_closed_forms]),
    "unpatchify_channel_major": ("unpatchify", _unpatchify_channel_major,
                                 [test_unpatchify_inverts_loop_patchify,
                                  test_decoder_reduces_to_conv_in_upsample_conv_out]),
}


@pytest.mark.parametrize("name", sorted(_MUTANTS))
def test_planted_decoder_mistake_is_caught(name, monkeypatch):
    attr, mutant, pins = _MUTANTS[name]
    monkeypatch.setattr(V, attr, mutant)
    caught = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin caught the planted mistake {name}"
