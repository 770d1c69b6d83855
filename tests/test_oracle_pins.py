"""Pins for the CPU oracle: checks against what the pages and the mathematics
fix, never against the oracle's own formulas retyped.

Kinds of pin used here:
  * facts the pages state (tests/golden/page_facts.txt, position-id fixture);
  * closed forms and special cases (pos 0, sigma 0, zero gate, zeroed branch);
  * invariants (rotation norm, relative-position invariance, softmax rows,
    key permutation, scale/shift invariance of the norms, batch independence);
  * an independent brute-force float64 re-derivation on tiny inputs
    (oracle/brute.py: loops, complex-number RoPE, explicit softmax);
  * planted mistakes: a plausible slip put into a copy of the oracle (the
    Euler step, head split, attention scale) or patched into the module in
    place of one page rule (position ids, RoPE ladder, timestep features,
    pre-norm, modulation, QK-norm, SwiGLU) must be caught by one of the pins
    above.
"""
import math
import os

import numpy as np
import pytest

from oracle import brute
from oracle import dit_oracle as O
from diffusion_transformer_fwd_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _facts():
    out = {}
    with open(os.path.join(GOLDEN, "page_facts.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = (s.strip() for s in line.split("=", 1))
                out[k] = v
    return out


FACTS = _facts()


def tiny_cfg(**kw):
    base = dict(hidden=256, heads=2, head_dim=128, mlp_hidden=768, n_dual=1, n_single=1,
                in_channels=8, txt_channels=16, time_channels=256)
    base.update(kw)
    return synth.DitConfig(**base)


# ---------------------------------------------------------------- page facts

def test_config_matches_page_facts():
    cfg = synth.FLUX2_KLEIN
    assert cfg.n_dual == int(FACTS["dual_blocks"])
    assert cfg.n_single == int(FACTS["single_blocks"])
    assert cfg.txt_channels == int(FACTS["text_channels"])
    assert len(FACTS["text_layers"].split(",")) * 2560 == cfg.txt_channels
    assert all(a == int(FACTS["rope_dims_per_axis"]) for a in cfg.axes_dim)
    assert sum(cfg.axes_dim) == cfg.head_dim
    assert cfg.theta == float(FACTS["rope_theta"])
    assert synth.W_STEP_1024.n_txt == int(FACTS["text_rows"])


def test_workload_sizes_within_page_limits():
    lo, hi, g = (int(FACTS[k]) for k in ("size_min_px", "size_max_px", "size_grid_px"))
    for w, h in ((1024, 1024), (1920, 1088)):
        assert lo <= w <= hi and lo <= h <= hi and w % g == 0 and h % g == 0
        assert w * h <= int(FACTS["max_pixels"])
    assert synth.patch_grid(1024, 1024) == (64, 64)
    assert synth.patch_grid(1920, 1088) == (68, 120)
    assert synth.W_STEP_1920x1088_B4.seq == 512 + 8160
    assert len(synth.W_STEP_1024_REF.ref_grids) <= int(FACTS["max_refs"])


def test_position_ids_reference_rule():
    base, stride = int(FACTS["ref_t_base"]), int(FACTS["ref_t_stride"])
    grids = [(2, 3), (1, 4), (3, 1)]
    pos = O.position_ids(5, (4, 4), grids)
    assert pos.shape == (5 + 16 + 6 + 4 + 3, 4)
    start = 5 + 16
    for i, (h, w) in enumerate(grids):
        blk = pos[start:start + h * w]
        assert np.all(blk[:, 0] == base + stride * i)
        assert np.array_equal(blk[:, 1], np.repeat(np.arange(h), w))
        assert np.array_equal(blk[:, 2], np.tile(np.arange(w), h))
        assert np.all(blk[:, 3] == 0)
        start += h * w
    # text rows and the image grid never use the t axis
    assert np.all(pos[:21, 0] == 0)


def test_position_ids_fixture():
    want = np.loadtxt(os.path.join(GOLDEN, "position_ids_1ref_2x2.txt"), dtype=np.int64)
    got = O.position_ids(3, (2, 2), [(1, 2), (1, 2)])
    assert np.array_equal(got, want)


def test_position_ids_match_brute_token_count():
    for wl in (synth.W_DUAL_TINY, synth.W_STEP_1024, synth.W_STEP_1024_REF,
               synth.W_STEP_1920x1088_B4):
        pos = O.position_ids(wl.n_txt, wl.img_grid, wl.ref_grids)
        assert pos.shape[0] == wl.seq


# ---------------------------------------------------------------- RoPE

def test_rope_identity_at_position_zero():
    cos, sin = O.rope_tables(np.zeros((3, 4), np.int64))
    assert np.array_equal(cos, np.ones((3, 64)))
    assert np.array_equal(sin, np.zeros((3, 64)))


def test_rope_frequency_ladder():
    # Per axis: 16 pairs, first frequency 1 rad per position, each next pair
    # slower by theta^(-2/32), so the last is theta^(-30/32).
    theta = float(FACTS["rope_theta"])
    phi = O.rope_angles(np.array([[1, 1, 1, 1]]), theta=theta)[0]
    for a in range(4):
        ax = phi[16 * a:16 * a + 16]
        assert ax[0] == 1.0
        r = ax[1:] / ax[:-1]
        assert np.allclose(r, theta ** (-1.0 / 16), rtol=1e-14)
        assert math.isclose(ax[-1], theta ** (-30.0 / 32), rel_tol=1e-14)


def test_rope_preserves_pair_norms_and_matches_complex_product():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 128))
    pos = rng.integers(0, 200, size=(7, 4))
    cos, sin = O.rope_tables(pos)
    y = O.apply_rope(x, cos, sin)
    n0 = x[:, 0::2] ** 2 + x[:, 1::2] ** 2
    n1 = y[:, 0::2] ** 2 + y[:, 1::2] ** 2
    assert np.allclose(n0, n1, rtol=1e-12)
    for t in range(7):
        want = brute.rotate(x[t].tolist(), pos[t].tolist())
        assert np.allclose(y[t], want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("axis", [0, 1, 2, 3])
def test_rope_relative_position_invariance(axis):
    # Shifting every token's position on one axis by the same amount leaves
    # all q.k logits unchanged; only position differences matter.
    rng = np.random.default_rng(2 + axis)
    q = rng.standard_normal((9, 128))
    k = rng.standard_normal((9, 128))
    pos = rng.integers(0, 64, size=(9, 4))
    pos2 = pos.copy()
    pos2[:, axis] += 37
    c1, s1 = O.rope_tables(pos)
    c2, s2 = O.rope_tables(pos2)
    l1 = O.apply_rope(q, c1, s1) @ O.apply_rope(k, c1, s1).T
    l2 = O.apply_rope(q, c2, s2) @ O.apply_rope(k, c2, s2).T
    assert np.allclose(l1, l2, rtol=0, atol=1e-10)


def test_rope_pairs_are_adjacent():
    # Only dims 0 and 1 are non-zero: a t-axis rotation must keep all the
    # energy in dims (0, 1); a split-half pairing would move it to dim 64.
    x = np.zeros((1, 128))
    x[0, 0] = 1.0
    cos, sin = O.rope_tables(np.array([[3, 0, 0, 0]]))
    y = O.apply_rope(x, cos, sin)
    assert math.isclose(y[0, 0], math.cos(3.0), abs_tol=1e-15)
    assert math.isclose(y[0, 1], math.sin(3.0), abs_tol=1e-15)
    assert np.all(y[0, 2:] == 0)


# ---------------------------------------------------------------- timestep

def test_timestep_features_closed_forms():
    e = O.timestep_features(np.array([0.0, 0.5]))
    assert np.array_equal(e[0], np.r_[np.ones(128), np.zeros(128)])
    assert np.allclose(e[:, :128] ** 2 + e[:, 128:] ** 2, 1.0, atol=1e-15)
    assert math.isclose(e[1, 0], math.cos(500.0), abs_tol=1e-15)
    assert math.isclose(e[1, 128], math.sin(500.0), abs_tol=1e-15)
    # lowest frequency: 1e4^(-127/128)
    assert math.isclose(e[1, 127], math.cos(500.0 * 1e4 ** (-127 / 128)), abs_tol=1e-15)
    b = brute.timestep_features(0.5)
    assert np.allclose(e[1], b, atol=1e-15)


# ---------------------------------------------------------------- norms

def test_rms_norm_identities():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 3072)) * 3.0
    n = O.prenorm(x, O.PRENORM_RMS, 0.0)
    assert np.allclose((n * n).mean(-1), 1.0, rtol=1e-12)
    assert np.allclose(O.prenorm(7.5 * x, O.PRENORM_RMS, 0.0), n, rtol=1e-12)
    ne = O.prenorm(x, O.PRENORM_RMS, 1e-6)
    assert np.allclose(ne, [brute.rms_normalize(r, 1e-6) for r in x.tolist()], rtol=1e-12)


def test_layer_norm_identities():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 512)) * 2.0 + 0.7
    n = O.prenorm(x, O.PRENORM_LAYER, 0.0)
    assert np.allclose(n.mean(-1), 0.0, atol=1e-12)
    assert np.allclose((n * n).mean(-1), 1.0, rtol=1e-12)
    assert np.allclose(O.prenorm(x + 11.0, O.PRENORM_LAYER, 0.0), n, atol=1e-10)
    ne = O.prenorm(x, O.PRENORM_LAYER, 1e-6)
    assert np.allclose(ne, [brute.layer_normalize(r, 1e-6) for r in x.tolist()], rtol=1e-12)


def test_modulate_zero_scale_is_plain_norm_and_minus_one_zeroes():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 256))
    z = np.zeros(256)
    assert np.array_equal(O.modulate(x, z, z), O.prenorm(x))
    assert np.array_equal(O.modulate(x, z, -np.ones(256)), np.zeros_like(x))
    sh = rng.standard_normal(256)
    assert np.allclose(O.modulate(x, sh, -np.ones(256)), np.broadcast_to(sh, x.shape))


# ---------------------------------------------------------------- attention

def test_attention_brute_force():
    rng = np.random.default_rng(6)
    q, k, v = (rng.standard_normal((1, 2, 11, 128)) for _ in range(3))
    o = O.attention(q, k, v, chunk=4)
    for h in range(2):
        want = brute.attention_rows(q[0, h].tolist(), k[0, h].tolist(), v[0, h].tolist())
        assert np.allclose(o[0, h], want, rtol=0, atol=1e-12)


def test_attention_invariants():
    rng = np.random.default_rng(7)
    q, k, v = (rng.standard_normal((2, 3, 13, 128)) * 2 for _ in range(3))
    o = O.attention(q, k, v)
    # key/value permutation invariance (no mask, no positions inside)
    perm = rng.permutation(13)
    assert np.allclose(O.attention(q, k[:, :, perm], v[:, :, perm]), o, atol=1e-12)
    # constant values: rows of the softmax sum to one
    c = np.broadcast_to(rng.standard_normal(128), v.shape).copy()
    assert np.allclose(O.attention(q, k, c), c, atol=1e-12)
    # single key returns its value
    o1 = O.attention(q, k[:, :, :1], v[:, :, :1])
    assert np.allclose(o1, np.broadcast_to(v[:, :, :1], o1.shape), atol=1e-12)
    # one dominant key
    k2 = k.copy()
    k2[:, :, 5] = q[:, :, 0] * 100.0
    o2 = O.attention(q[:, :, :1], k2, v)
    assert np.allclose(o2[:, :, 0], v[:, :, 5], atol=1e-9)


def test_swiglu_closed_form():
    u = np.array([[0.0, 1.0, 5.0, 7.0, -3.0, 2.0]])
    a = O.swiglu(u)
    want = [0.0, 1.0 / (1 + math.exp(-1.0)) * (-3.0), 5.0 / (1 + math.exp(-5.0)) * 2.0]
    assert np.allclose(a[0], want, rtol=1e-15)


# ---------------------------------------------------------------- blocks

def _block_setup(cfg, n_txt=3, grid=(2, 3), refs=(), seed=0):
    pos = O.position_ids(n_txt, grid, refs)
    S = pos.shape[0]
    x = synth.residual(cfg, seed, S)[None].astype(np.float64)
    cos, sin = O.rope_tables(pos, cfg.axes_dim, cfg.theta)
    gw = synth.global_weights(cfg, seed)
    mod = O.modulation(gw, np.array([0.5]), cfg.time_channels)
    return pos, x, cos, sin, gw, mod


@pytest.mark.parametrize("layer", [False, True])
def test_dual_block_matches_brute_force(layer):
    cfg = tiny_cfg(prenorm=int(layer))
    pos, x, cos, sin, gw, mod = _block_setup(cfg)
    w = synth.dual_weights(cfg, 0, 0)
    got = O.dual_block(x, 3, w, mod["dual_txt"], mod["dual_img"], cos, sin, cfg.heads,
                       cfg.eps, cfg.prenorm)
    want = brute.dual_block(x[0], 3, w, mod["dual_txt"][0], mod["dual_img"][0], pos,
                            cfg.heads, cfg.eps, layer)
    assert np.allclose(got[0], want, rtol=0, atol=1e-11)


@pytest.mark.parametrize("layer", [False, True])
def test_single_block_matches_brute_force(layer):
    cfg = tiny_cfg(prenorm=int(layer))
    pos, x, cos, sin, gw, mod = _block_setup(cfg, refs=[(1, 2)])
    w = synth.single_weights(cfg, 0, 0)
    got = O.single_block(x, w, mod["single"], cos, sin, cfg.heads, cfg.eps, cfg.prenorm)
    want = brute.single_block(x[0], w, mod["single"][0], pos, cfg.heads, cfg.eps, layer)
    assert np.allclose(got[0], want, rtol=0, atol=1e-11)


def test_modulation_matches_brute_force():
    cfg = tiny_cfg()
    gw = synth.global_weights(cfg, 0)
    m = O.modulation(gw, np.array([0.75, 0.25]), cfg.time_channels)
    for b, s in enumerate((0.75, 0.25)):
        want = brute.modulation(gw, s, cfg.time_channels)
        for k in ("dual_img", "dual_txt", "single", "final"):
            assert np.allclose(m[k][b], want[k], rtol=0, atol=1e-13)


def test_step_matches_brute_force():
    cfg = tiny_cfg()
    wl = synth.Workload("t", 1, 3, (2, 2), ((1, 2),), 0.75)
    pos = O.position_ids(wl.n_txt, wl.img_grid, wl.ref_grids)
    weights = synth.ModelWeights(cfg, 0, cache=True)
    inp = synth.step_inputs(cfg, wl)
    v = O.step(cfg, weights, inp["txt"][None], inp["latents"][None], np.array([0.75]),
               wl.n_img, pos)
    want = brute.step(cfg, weights, inp["txt"], inp["latents"], 0.75, wl.n_img, pos)
    assert v.shape == (1, 4, cfg.in_channels)
    assert np.allclose(v[0], want, rtol=0, atol=1e-11)


def test_zero_gate_leaves_residual_unchanged():
    cfg = tiny_cfg()
    pos, x, cos, sin, gw, mod = _block_setup(cfg)
    md = mod["dual_img"].copy()
    md[:, 2] = 0.0
    md[:, 5] = 0.0
    mt = mod["dual_txt"].copy()
    mt[:, 2] = 0.0
    mt[:, 5] = 0.0
    y = O.dual_block(x, 3, synth.dual_weights(cfg, 0, 0), mt, md, cos, sin, cfg.heads)
    assert np.array_equal(y, x)
    ms = mod["single"].copy()
    ms[:, 2] = 0.0
    y = O.single_block(x, synth.single_weights(cfg, 0, 0), ms, cos, sin, cfg.heads)
    assert np.array_equal(y, x)


def test_zeroed_branch_input_leaves_residual_unchanged():
    # scale = -1, shift = 0 -> normed input 0 -> q = k = v = 0 and SwiGLU 0.
    cfg = tiny_cfg()
    pos, x, cos, sin, gw, mod = _block_setup(cfg)
    md = mod["dual_img"].copy()
    mt = mod["dual_txt"].copy()
    for m in (md, mt):
        m[:, 0] = 0.0
        m[:, 1] = -1.0
        m[:, 3] = 0.0
        m[:, 4] = -1.0
    y = O.dual_block(x, 3, synth.dual_weights(cfg, 0, 0), mt, md, cos, sin, cfg.heads)
    assert np.array_equal(y, x)
    ms = mod["single"].copy()
    ms[:, 0] = 0.0
    ms[:, 1] = -1.0
    y = O.single_block(x, synth.single_weights(cfg, 0, 0), ms, cos, sin, cfg.heads)
    assert np.array_equal(y, x)


def test_dual_block_split_point_irrelevant_when_streams_identical():
    # Same weights and mods for both streams: the joint sequence is then one
    # stream, so the result cannot depend on where text ends.
    cfg = tiny_cfg()
    pos, x, cos, sin, gw, mod = _block_setup(cfg, n_txt=4, grid=(2, 2))
    w = synth.dual_weights(cfg, 0, 0)
    for k in ("qkv", "out", "mlp_in", "mlp_out", "q_gain", "k_gain"):
        w[f"{k}0"] = w[f"{k}1"]
    m = mod["dual_img"]
    ys = [O.dual_block(x, n, w, m, m, cos, sin, cfg.heads) for n in (0, 1, 4, 8)]
    for y in ys[1:]:
        assert np.allclose(y, ys[0], rtol=0, atol=1e-12)


def test_batch_rows_independent():
    cfg = tiny_cfg()
    pos = O.position_ids(3, (2, 3))
    S = pos.shape[0]
    cos, sin = O.rope_tables(pos)
    xa = synth.residual(cfg, 0, S)[None].astype(np.float64)
    xb = synth.residual(cfg, 1, S)[None].astype(np.float64)
    gw = synth.global_weights(cfg, 0)
    mod = O.modulation(gw, np.array([0.75, 0.3]))
    w = synth.single_weights(cfg, 0, 0)
    both = O.single_block(np.concatenate([xa, xb]), w, mod["single"], cos, sin, cfg.heads)
    ya = O.single_block(xa, w, mod["single"][:1], cos, sin, cfg.heads)
    yb = O.single_block(xb, w, mod["single"][1:], cos, sin, cfg.heads)
    assert np.allclose(both[0], ya[0], rtol=0, atol=1e-13)
    assert np.allclose(both[1], yb[0], rtol=0, atol=1e-13)


def test_step_uses_one_global_modulation():
    # The step equals its blocks composed by hand with the single modulation
    # result computed from sigma: one set of AdaLN vectors per step, shared by
    # every block ("tt_flux2_klein - Python reference", Things that are easy
    # to get wrong).
    cfg = tiny_cfg(n_dual=2, n_single=2)
    wl = synth.Workload("t", 1, 3, (2, 2), (), 0.6)
    pos = O.position_ids(wl.n_txt, wl.img_grid)
    weights = synth.ModelWeights(cfg, 0, cache=True)
    inp = synth.step_inputs(cfg, wl)
    txt, lat = inp["txt"][None], inp["latents"][None]
    sig = np.array([0.6])
    v = O.step(cfg, weights, txt, lat, sig, wl.n_img, pos)
    mod = O.modulation(weights.glob, sig)
    cos, sin = O.rope_tables(pos)
    x = O.embed(weights.glob, txt, lat)
    for i in range(2):
        x = O.dual_block(x, 3, weights.dual(i), mod["dual_txt"], mod["dual_img"], cos, sin, 2)
    for i in range(2):
        x = O.single_block(x, weights.single(i), mod["single"], cos, sin, 2)
    assert np.array_equal(v, O.final_layer(weights.glob, x, 3, 4, mod["final"]))


def test_fp32_oracle_close_to_fp64_at_dual_block_d256():
    cfg = synth.TINY_256
    wl = synth.W_DUAL_TINY
    pos = O.position_ids(wl.n_txt, wl.img_grid)
    x = synth.residual(cfg, 0, wl.seq)[None]
    gw = synth.global_weights(cfg, 0)
    w = synth.dual_weights(cfg, 0, 0)
    outs = []
    for dt in (np.float64, np.float32):
        mod = O.modulation(gw, np.array([0.5]), dtype=dt)
        cos, sin = O.rope_tables(pos)
        outs.append(O.dual_block(x, wl.n_txt, w, mod["dual_txt"], mod["dual_img"],
                                 cos.astype(dt), sin.astype(dt), cfg.heads, dtype=dt))
    a, b = outs
    assert b.dtype == np.float32
    assert np.linalg.norm(b - a) / np.linalg.norm(a) <= 1e-5


def test_euler_update():
    z = np.array([1.0, -2.0])
    v = np.array([0.5, 4.0])
    assert np.array_equal(O.euler(z, v, 1.0, 0.75), np.array([0.875, -3.0]))


def test_single_block_rows_equals_full_block():
    """The row-restricted block (used where the whole block is too long for the
    oracle) gives the full block's rows, including the first and last."""
    cfg = synth.DitConfig(hidden=256, heads=2, head_dim=128, mlp_hidden=768)
    pos = O.position_ids(16, (5, 7), ((3, 2),))
    S = pos.shape[0]
    x = np.stack([synth.residual(cfg, b, S) for b in range(2)])
    w = synth.single_weights(cfg, 0, 0)
    mod = O.modulation(synth.global_weights(cfg, 0), np.array([0.75, 0.3]))["single"]
    cos, sin = O.rope_tables(pos)
    full = O.single_block(x, w, mod, cos, sin, cfg.heads)
    rows = np.array([0, 3, 15, 16, 40, S - 1])
    got = O.single_block_rows(x, w, mod, cos, sin, cfg.heads, rows)
    np.testing.assert_allclose(got, full[:, rows], rtol=0, atol=1e-12)


def test_denoise_linear_field_closed_form():
    """v = a z is a linear ODE; each Euler step multiplies z by
    1 + a (sigma_{i+1} - sigma_i), so n steps give the product of those
    factors (per batch row, with its own schedule)."""
    rng = np.random.default_rng(3)
    z0 = rng.standard_normal((2, 5, 4))
    sig = np.array([[1.0, 0.75, 0.5, 0.25, 0.0], [0.9, 0.6, 0.35, 0.1, 0.0]])
    a = -1.7
    got = O.denoise(lambda z, s: a * z, z0, sig)
    fac = np.prod(1.0 + a * np.diff(sig, axis=1), axis=1)
    np.testing.assert_allclose(got, z0 * fac[:, None, None], rtol=1e-14, atol=0)


def test_denoise_straight_path_is_exact():
    """On the straight path z(sigma) = (1 - sigma) x0 + sigma n the velocity
    n - x0 is constant, so Euler lands on x0 at sigma = 0 for any schedule
    (the rectified-flow property the update is built on)."""
    rng = np.random.default_rng(4)
    x0, n = rng.standard_normal((2, 1, 3, 8))
    sig = np.array([[1.0, 0.8, 0.3, 0.05, 0.0]])
    seen = []

    def vel(z, s):
        seen.append(s.copy())
        np.testing.assert_allclose(z, (1 - s[0]) * x0 + s[0] * n, atol=1e-12)
        return n - x0

    got = O.denoise(vel, (1 - sig[0, 0]) * x0 + sig[0, 0] * n, sig)
    np.testing.assert_allclose(got, x0, atol=1e-12)
    assert [float(x[0]) for x in seen] == [1.0, 0.8, 0.3, 0.05]


def test_denoise_dit_keeps_references_fixed():
    """The DiT loop passes the reference tokens unchanged to every step and
    updates only the image latents: with one step it is one step plus Euler."""
    cfg = synth.DitConfig(hidden=256, heads=2, head_dim=128, mlp_hidden=768, n_dual=1,
                          n_single=1, in_channels=128, txt_channels=256)
    mw = synth.ModelWeights(cfg, 0, cache=True)
    wl = synth.Workload("s", 1, 8, (2, 3), ((2, 2),), 0.75)
    ins = synth.step_inputs(cfg, wl)
    pos = O.position_ids(wl.n_txt, wl.img_grid, wl.ref_grids)
    z = ins["latents"][None, :wl.n_img]
    ref = ins["latents"][None, wl.n_img:]
    got = O.denoise_dit(cfg, mw, ins["txt"][None], z, ref, np.array([[0.75, 0.4]]), pos)
    v = O.step(cfg, mw, ins["txt"][None], ins["latents"][None], np.array([0.75]), wl.n_img, pos)
    np.testing.assert_allclose(got, z + (0.4 - 0.75) * v, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- planted mistakes

def _mutants():
    """Plausible slips, each as a replacement for one oracle function."""
    orig_rope, orig_heads, orig_attn = O.apply_rope, O._heads, O.attention

    def rope_sign(x, c, s):
        return orig_rope(x, c, -s)

    def rope_half_split(x, c, s):
        h = x.shape[-1] // 2
        y = np.empty_like(x)
        y[..., :h] = x[..., :h] * c - x[..., h:] * s
        y[..., h:] = x[..., :h] * s + x[..., h:] * c
        return y

    def heads_wrong(x, heads):
        B, S, HD = x.shape
        return x.reshape(B, S, HD // heads, heads).transpose(0, 3, 1, 2)

    def attn_no_scale(q, k, v, chunk=1024):
        return orig_attn(q * math.sqrt(q.shape[-1]), k, v, chunk)

    def linear_t(x, w):
        return x @ w.T if w.shape[0] != w.shape[1] else x @ w

    return {
        "apply_rope": rope_sign,
        "apply_rope_half": rope_half_split,
        "_heads": heads_wrong,
        "attention": attn_no_scale,
        "linear": linear_t,
    }


@pytest.mark.parametrize("name", list(_mutants()))
def test_planted_mistake_is_caught(name, monkeypatch):
    cfg = tiny_cfg()
    pos, x, cos, sin, gw, mod = _block_setup(cfg)
    w = synth.dual_weights(cfg, 0, 0)
    want = brute.dual_block(x[0], 3, w, mod["dual_txt"][0], mod["dual_img"][0], pos,
                            cfg.heads, cfg.eps)
    attr = "apply_rope" if name.startswith("apply_rope") else name
    monkeypatch.setattr(O, attr, _mutants()[name])
    got = O.dual_block(x, 3, w, mod["dual_txt"], mod["dual_img"], cos, sin, cfg.heads)
    assert not np.allclose(got[0], want, rtol=0, atol=1e-6)


def test_planted_euler_mistakes_are_caught(monkeypatch):
    """Slips in the update are caught by the straight-path pin: Euler then
    no longer lands on x0."""
    rng = np.random.default_rng(5)
    x0, n = rng.standard_normal((2, 1, 4, 8))
    sig = np.array([[1.0, 0.6, 0.2, 0.0]])
    z0 = (1 - sig[0, 0]) * x0 + sig[0, 0] * n
    for bad in (lambda z, v, s, s1: z - (s1 - s) * v,   # sign of the step
                lambda z, v, s, s1: z + s1 * v,         # sigma instead of its change
                lambda z, v, s, s1: v + (s1 - s) * z):  # latent and velocity swapped
        monkeypatch.setattr(O, "euler", bad)
        got = O.denoise(lambda z, s: n - x0, z0, sig)
        assert not np.allclose(got, x0, atol=1e-6)


# Slips in the page-fixed rules (position ids, RoPE, timestep features, the
# AdaLN modulation, SwiGLU), patched into the oracle module: each must fail at
# least one of the listed pins, which check the pages' examples, closed forms
# and loop versions rather than the oracle's own formulas.
_O_pos, _O_angles, _O_feat = O.position_ids, O.rope_angles, O.timestep_features
_O_prenorm, _O_mod = O.prenorm, O.modulation


def _pos_ref_from_zero(n_txt, img_grid, ref_grids=()):
    p = _O_pos(n_txt, img_grid, ref_grids)
    p[:, 0] = np.where(p[:, 0] > 0, p[:, 0] - 10, p[:, 0])   # t = 10 i
    return p


def _pos_rows_cols_swapped(n_txt, img_grid, ref_grids=()):
    p = _O_pos(n_txt, img_grid, ref_grids)
    return p[:, [0, 2, 1, 3]]


def _rope_exponent_without_two(pos, axes_dim=(32, 32, 32, 32), theta=2000.0):
    pos = np.asarray(pos, dtype=np.float64)
    cols = [pos[:, a:a + 1] * theta ** (-np.arange(d // 2) / d)[None, :]
            for a, d in enumerate(axes_dim)]
    return np.concatenate(cols, axis=1)


def _modulation_chunks_swapped(gw, sigma, channels=256, dtype=np.float64):
    m = _O_mod(gw, sigma, channels, dtype)
    m["dual_img"] = m["dual_img"][:, [1, 0, 2, 4, 3, 5]]        # scale and shift swapped
    return m


_PAGE_MUTANTS = {
    "ref_t_from_zero": ("position_ids", _pos_ref_from_zero,
                        [test_position_ids_reference_rule, test_position_ids_fixture]),
    "grid_rows_cols_swapped": ("position_ids", _pos_rows_cols_swapped,
                               [test_position_ids_reference_rule, test_position_ids_fixture]),
    "rope_theta_10000": ("rope_angles",
                         lambda pos, axes_dim=(32, 32, 32, 32), theta=2000.0:
                         _O_angles(pos, axes_dim, 10000.0),
                         [test_rope_frequency_ladder,
                          test_rope_preserves_pair_norms_and_matches_complex_product]),
    "rope_exponent_without_two": ("rope_angles", _rope_exponent_without_two,
                                  [test_rope_frequency_ladder,
                                   test_rope_preserves_pair_norms_and_matches_complex_product]),
    "features_sin_first": ("timestep_features",
                           lambda sigma, channels=256, dtype=np.float64:
                           _O_feat(sigma, channels, dtype)[:, ::-1],
                           [test_timestep_features_closed_forms]),
    "rms_eps_outside_root": ("prenorm",
                             lambda x, kind=O.PRENORM_RMS, eps=1e-6:
                             _O_prenorm(x, kind, 0.0) if kind == O.PRENORM_LAYER else
                             x / (np.sqrt((x * x).mean(axis=-1, keepdims=True)) + eps),
                             [test_rms_norm_identities]),
    "modulate_without_one": ("modulate",
                             lambda x, shift, scale, kind=O.PRENORM_RMS, eps=1e-6:
                             _O_prenorm(x, kind, eps) * scale + shift,
                             [test_modulate_zero_scale_is_plain_norm_and_minus_one_zeroes]),
    "modulation_chunks_swapped": ("modulation", _modulation_chunks_swapped,
                                  [test_modulation_matches_brute_force]),
    "qk_norm_over_all_heads": ("qk_rmsnorm",
                               lambda x, g, eps=1e-6:
                               x / np.sqrt((x * x).mean(axis=(-3, -1), keepdims=True) + eps) * g,
                               [lambda: test_dual_block_matches_brute_force(False),
                                lambda: test_single_block_matches_brute_force(False)]),
    "swiglu_halves_swapped": ("swiglu", lambda u: O.silu(u[..., u.shape[-1] // 2:]) *
                              u[..., :u.shape[-1] // 2],
                              [test_swiglu_closed_form]),
}


@pytest.mark.parametrize("name", sorted(_PAGE_MUTANTS))
def test_planted_page_rule_mistake_is_caught(name, monkeypatch):
    attr, mutant, pins = _PAGE_MUTANTS[name]
    monkeypatch.setattr(O, attr, mutant)
    caught = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin caught the planted mistake {name}"
