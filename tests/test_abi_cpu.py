"""CPU-side checks of libdit.so: it loads without a GPU, exports every entry
point declared in include/dit.h, and its host-only logic (position ids,
configuration checks, workspace sizing, argument validation that must fail
before any launch) behaves as documented. No kernel is launched here.
"""
import ctypes as C
import os
import re

import numpy as np
import pytest

from diffusion_transformer_fwd_amd import dit, synth
from oracle import dit_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(dit.library_path()):
        from diffusion_transformer_fwd_amd import build
        build.build()
    return dit.lib()


def header_functions(name):
    txt = open(os.path.join(ROOT, "include", name)).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(dit_[a-z_0-9]+)\s*\(", txt)))


def test_exports_every_declared_function(L):
    names = header_functions("dit.h")
    assert len(names) == 15, names
    assert sorted(dit.EXPORTS) == names
    vae = header_functions("dit_vae.h")
    assert len(vae) == 7, vae
    assert sorted(dit.VAE_EXPORTS) == vae
    headers = sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))
    assert headers == ["dit.h", "dit_vae.h"], headers
    for n in names + vae:
        assert hasattr(L, n), f"{n} not exported"


def test_profile_end_without_begin(L):
    arr = (dit.KernelStats * dit.K_COUNT)()
    assert L.dit_profile_end(arr) == dit.DIT_E_VALUE
    assert L.dit_profile_end(None) == dit.DIT_E_NULL
    assert L.dit_profile_begin() == dit.DIT_OK
    assert L.dit_profile_end(arr) == dit.DIT_OK  # nothing recorded
    assert all(a.launches == 0 for a in arr)


def test_status_strings(L):
    for s in range(-6, 1):
        assert L.dit_status_string(s)
    assert L.dit_status_string(-99) == b"unknown status"


# ---------------------------------------------------------------- config checks

def _cfg(**kw):
    return dit.config(synth.DitConfig(**kw)) if kw else dit.config(synth.FLUX2_KLEIN)


@pytest.mark.parametrize("kw,status", [
    ({}, dit.DIT_OK),
    (dict(hidden=256, heads=2, mlp_hidden=768), dit.DIT_OK),
    (dict(head_dim=64, hidden=24 * 64), dit.DIT_E_UNSUPPORTED),
    (dict(hidden=3000), dit.DIT_E_SHAPE),
    (dict(axes_dim=(32, 32, 32, 30)), dit.DIT_E_SHAPE),
    (dict(axes_dim=(32, 32, 32, 31)), dit.DIT_E_SHAPE),
    (dict(axes_dim=(16, 48, 32, 32)), dit.DIT_OK),
    (dict(prenorm=5), dit.DIT_E_VALUE),
    (dict(theta=float("nan")), dit.DIT_E_VALUE),
    (dict(eps=-1.0), dit.DIT_E_VALUE),
    (dict(txt_channels=100), dit.DIT_E_UNSUPPORTED),
    (dict(mlp_hidden=100), dit.DIT_E_UNSUPPORTED),
])
def test_config_check(L, kw, status):
    c = _cfg(**kw)
    assert L.dit_config_check(C.byref(c)) == status
    if status != dit.DIT_OK:
        assert dit.last_error()


def test_config_check_null(L):
    assert L.dit_config_check(None) == dit.DIT_E_NULL


# ---------------------------------------------------------------- position ids

@pytest.mark.parametrize("n_txt,grid,refs", [
    (512, (64, 64), []),
    (512, (64, 64), [(64, 64)]),
    (512, (68, 120), []),
    (32, (8, 8), []),
    (3, (2, 5), [(1, 2), (3, 1), (2, 2)]),
    (0, (1, 1), []),
    (7, (0, 0), [(2, 3)]),
])
def test_position_ids_match_oracle(L, n_txt, grid, refs):
    got = dit.position_ids(n_txt, grid, refs)
    want = O.position_ids(n_txt, grid, refs)
    assert got.dtype == np.int32
    assert np.array_equal(got, want)


def test_position_ids_errors(L):
    out = np.zeros((100, 4), np.int32)
    rh = (C.c_int32 * 4)(1, 1, 1, 1)
    rw = (C.c_int32 * 4)(1, 1, 1, 1)
    f = L.dit_position_ids
    assert f(4, 2, 2, 4, C.cast(rh, C.c_void_p), C.cast(rw, C.c_void_p), out.ctypes.data, 100) == dit.DIT_E_SHAPE
    assert f(4, 2, 2, 0, None, None, out.ctypes.data, 7) == dit.DIT_E_SHAPE  # 8 rows > cap 7
    assert f(-1, 2, 2, 0, None, None, out.ctypes.data, 100) == dit.DIT_E_SHAPE
    assert f(4, 2, 2, 1, None, None, out.ctypes.data, 100) == dit.DIT_E_NULL
    assert f(4, 2, 2, 0, None, None, out.ctypes.data, 8) == 8


# ---------------------------------------------------------------- workspace sizing

def test_workspace_bytes(L):
    cfg = synth.FLUX2_KLEIN
    for kind in (dit.WS_DUAL, dit.WS_SINGLE, dit.WS_STEP, dit.WS_DENOISE):
        a = dit.workspace_bytes(cfg, kind, 1, 4608)
        b = dit.workspace_bytes(cfg, kind, 1, 8704)
        c = dit.workspace_bytes(cfg, kind, 4, 8672)
        assert 0 < a < b < c
        assert a % 256 == 0
    # the step workspace holds the fp32 residual, the modulation buffer and a block's
    step = dit.workspace_bytes(cfg, dit.WS_STEP, 1, 4608)
    assert step >= 4608 * 3072 * 4 + 17 * 3072 * 4 + dit.workspace_bytes(cfg, dit.WS_SINGLE, 1, 4608)
    assert dit.workspace_bytes(cfg, dit.WS_MOD, 4, 0) > 0
    # the sampling loop adds its bf16 latent operand and fp32 velocity to a step's
    assert dit.workspace_bytes(cfg, dit.WS_DENOISE, 1, 4608) >= step + 4608 * 128 * 6
    c = dit.config(cfg)
    assert L.dit_workspace_bytes(C.byref(c), dit.WS_STEP, 0, 10) == 0
    assert L.dit_workspace_bytes(C.byref(c), dit.WS_STEP, 65, 10) == 0
    assert L.dit_workspace_bytes(C.byref(c), 9, 1, 10) == 0


# ---------------------------------------------------------------- validation before launch
# Fake (non-null, aligned) device addresses: every call below must be rejected
# by a check that runs before the first HIP call.
FAKE = 1 << 20


def _fake_model(cfg):
    n_d, n_s = max(cfg.n_dual, 1), max(cfg.n_single, 1)
    duals = (dit.DualWeightsC * n_d)()
    for d in duals:
        for i in range(2):
            d.qkv[i] = d.out[i] = d.mlp_in[i] = d.mlp_out[i] = d.q_gain[i] = d.k_gain[i] = FAKE
    singles = (dit.SingleWeightsC * n_s)()
    for s in singles:
        s.w_in = s.w_out = s.q_gain = s.k_gain = FAKE
    m = dit.ModelWeightsC()
    for k in ("t_in", "t_out", "mod_dual_img", "mod_dual_txt", "mod_single", "mod_final",
              "x_embed", "ctx_embed", "proj_out"):
        setattr(m, k, FAKE)
    m.dual = C.cast(duals, C.POINTER(dit.DualWeightsC))
    m.single = C.cast(singles, C.POINTER(dit.SingleWeightsC))
    return m, duals, singles


def _step(L, cfg, m, sig, B=1, n_txt=512, n_img=4096, n_ref=0, ws=FAKE, ws_bytes=1 << 40,
          txt=FAKE, lat=FAKE, v=FAKE, cos=FAKE):
    c = dit.config(cfg)
    sig = np.ascontiguousarray(sig, np.float32)
    return L.dit_step_forward(C.byref(c), C.byref(m) if m is not None else None, txt, lat,
                              sig.ctypes.data, B, n_txt, n_img, n_ref, cos, FAKE, v, ws,
                              ws_bytes, None)


def test_step_validation_errors(L):
    cfg = synth.FLUX2_KLEIN
    m, _d, _s = _fake_model(cfg)
    nan = [float("nan")]
    assert _step(L, cfg, None, [0.5]) == dit.DIT_E_NULL
    assert _step(L, cfg, m, nan) == dit.DIT_E_VALUE
    assert _step(L, cfg, m, [0.5], B=0) == dit.DIT_E_SHAPE
    assert _step(L, cfg, m, [0.5] * 65, B=65) == dit.DIT_E_SHAPE
    assert _step(L, cfg, m, [0.5], n_img=0) == dit.DIT_E_SHAPE
    assert _step(L, cfg, m, [0.5], lat=0) == dit.DIT_E_NULL
    assert _step(L, cfg, m, [0.5], v=FAKE + 4) == dit.DIT_E_SHAPE  # misaligned
    assert _step(L, cfg, m, [0.5], ws_bytes=1024) == dit.DIT_E_WORKSPACE
    assert _step(L, cfg, m, [0.5], ws=FAKE + 16) == dit.DIT_E_WORKSPACE
    assert _step(L, cfg, m, [0.5], ws=0) == dit.DIT_E_NULL
    # one operand beyond 4 GiB of 32-bit buffer offsets
    assert _step(L, cfg, m, [0.5] * 64, B=64, n_img=8160 * 3) == dit.DIT_E_UNSUPPORTED
    bad = synth.DitConfig(head_dim=64, hidden=24 * 64)
    assert _step(L, bad, m, [0.5]) == dit.DIT_E_UNSUPPORTED
    m.dual[3].mlp_out[1] = 0
    assert _step(L, cfg, m, [0.5]) == dit.DIT_E_NULL
    assert "mlp_out" in dit.last_error()


def _denoise(L, cfg, m, sig, n_steps, B=1, n_txt=512, n_img=4096, n_ref=0, z=FAKE, ref=FAKE,
             ws_bytes=1 << 40, in_channels=None):
    c = dit.config(cfg)
    sig = np.ascontiguousarray(sig, np.float32)
    return L.dit_denoise_forward(C.byref(c), C.byref(m), FAKE, z, ref, sig.ctypes.data, n_steps,
                                 B, n_txt, n_img, n_ref, FAKE, FAKE, FAKE, ws_bytes, None)


def test_denoise_validation_errors(L):
    cfg = synth.FLUX2_KLEIN
    m, _d, _s = _fake_model(cfg)
    sig = [1.0, 0.75, 0.5, 0.25, 0.0]
    assert _denoise(L, cfg, m, sig, 0) == dit.DIT_E_SHAPE
    assert _denoise(L, cfg, m, sig * 20, 65) == dit.DIT_E_SHAPE
    assert _denoise(L, cfg, m, [1.0, float("inf"), 0.5, 0.25, 0.0], 4) == dit.DIT_E_VALUE
    # the second batch row's schedule is read too
    assert _denoise(L, cfg, m, sig + [1.0, 0.5, float("nan"), 0.2, 0.0], 4, B=2) == dit.DIT_E_VALUE
    assert _denoise(L, cfg, m, sig, 4, z=0) == dit.DIT_E_NULL
    assert _denoise(L, cfg, m, sig, 4, n_ref=4096, ref=0) == dit.DIT_E_NULL
    assert _denoise(L, cfg, m, sig, 4, ws_bytes=1 << 20) == dit.DIT_E_WORKSPACE
    assert _denoise(L, synth.DitConfig(in_channels=130), m, sig, 4) == dit.DIT_E_UNSUPPORTED


def test_block_validation_errors(L):
    cfg = synth.FLUX2_KLEIN
    c = dit.config(cfg)
    _m, duals, singles = _fake_model(cfg)
    f = L.dit_dual_block_forward
    args = dict(x=FAKE, B=1, S=4608, n_txt=512, mt=FAKE, mi=FAKE, mbs=17 * 3072, ws=FAKE,
                wsb=1 << 40)

    def dual(**kw):
        a = dict(args, **kw)
        return f(C.byref(c), C.byref(duals[0]), a["x"], a["B"], a["S"], a["n_txt"], a["mt"],
                 a["mi"], a["mbs"], FAKE, FAKE, a["ws"], a["wsb"], None)

    assert dual(n_txt=4609) == dit.DIT_E_SHAPE
    assert dual(n_txt=-1) == dit.DIT_E_SHAPE
    assert dual(S=0) == dit.DIT_E_SHAPE
    assert dual(x=0) == dit.DIT_E_NULL
    assert dual(mt=0) == dit.DIT_E_NULL
    assert dual(mbs=3) == dit.DIT_E_SHAPE
    assert dual(wsb=100) == dit.DIT_E_WORKSPACE
    g = L.dit_single_block_forward
    assert g(C.byref(c), None, FAKE, 1, 4608, FAKE, 0, FAKE, FAKE, FAKE, 1 << 40, None) == dit.DIT_E_NULL
    assert g(C.byref(c), C.byref(singles[0]), FAKE, 1, 4608, FAKE, 0, FAKE, FAKE, FAKE, 64,
             None) == dit.DIT_E_WORKSPACE
    r = L.dit_rope_tables_build
    assert r(C.byref(c), None, 10, FAKE, FAKE, None) == dit.DIT_E_NULL
    assert r(C.byref(c), FAKE, -1, FAKE, FAKE, None) == dit.DIT_E_SHAPE
    assert r(C.byref(c), FAKE, 0, FAKE, FAKE, None) == dit.DIT_OK  # nothing to do


def test_modulation_noalloc_validation_errors(L):
    # every rejection happens before the scratch lookup and the first launch
    cfg = synth.FLUX2_KLEIN
    c = dit.config(cfg)
    m, _d, _s = _fake_model(cfg)
    f = L.dit_modulation_forward_noalloc

    def call(sig, B, mod=FAKE, model=m):
        s = np.ascontiguousarray(sig, np.float32)
        return f(C.byref(c), C.byref(model) if model is not None else None, s.ctypes.data, B,
                 mod, None)

    assert call([0.5], 0) == dit.DIT_E_SHAPE
    assert call([0.5] * 65, 65) == dit.DIT_E_SHAPE
    assert call([float("nan")], 1) == dit.DIT_E_VALUE
    assert call([0.5], 1, mod=0) == dit.DIT_E_NULL
    assert call([0.5], 1, mod=FAKE + 4) == dit.DIT_E_SHAPE
    assert call([0.5], 1, model=None) == dit.DIT_E_NULL
    m.t_in = 0
    assert call([0.5], 1) == dit.DIT_E_NULL
    assert "t_in" in dit.last_error()
    assert f(C.byref(c), C.byref(m), None, 1, FAKE, None) == dit.DIT_E_NULL


# ---------------------------------------------------------------- latent decoder

def _vcfg(**kw):
    import dataclasses
    return dit.vae_config(dataclasses.replace(synth.VAE_KLEIN, **kw))


def test_vae_config_default_and_check(L):
    c = dit.VaeConfigC()
    L.dit_vae_config_default(C.byref(c))
    assert (c.z_channels, list(c.block_channels), c.layers, c.groups) == (32, [128, 256, 512, 512], 3, 32)
    assert abs(c.eps - 1e-6) < 1e-12
    assert L.dit_vae_config_check(C.byref(c)) == dit.DIT_OK
    assert L.dit_vae_config_check(None) == dit.DIT_E_NULL
    for kw, st in ((dict(z_channels=12), dit.DIT_E_UNSUPPORTED),
                   (dict(block_channels=(128, 256, 384, 512)), dit.DIT_E_UNSUPPORTED),
                   (dict(block_channels=(16, 256, 512, 512)), dit.DIT_E_UNSUPPORTED),
                   (dict(groups=24), dit.DIT_E_UNSUPPORTED),
                   (dict(layers=0), dit.DIT_E_UNSUPPORTED),
                   (dict(layers=5), dit.DIT_E_UNSUPPORTED),
                   (dict(eps=0.0), dit.DIT_E_VALUE)):
        c = _vcfg(**kw)
        assert L.dit_vae_config_check(C.byref(c)) == st, kw


def test_vae_workspace_bytes(L):
    c = dit.vae_config(synth.VAE_KLEIN)
    n1 = L.dit_vae_workspace_bytes(C.byref(c), 1, 64, 64)
    # four activation buffers of the widest tensor (1024 x 1024 x 256 bf16),
    # the fp32 scores of all 16384 queries and their bf16 probabilities
    assert n1 >= 3 * 512 * 2 ** 20 + 256 * 2 ** 20 + 1.5 * 2 ** 30
    assert L.dit_vae_workspace_bytes(C.byref(c), 2, 64, 64) > n1
    assert L.dit_vae_workspace_bytes(C.byref(c), 0, 64, 64) == 0
    assert L.dit_vae_workspace_bytes(C.byref(c), 1, 0, 64) == 0
    assert L.dit_vae_workspace_bytes(C.byref(c), 1, 64, 3000) == 0
    # 1920 x 1088: 32640 latent pixels, all queries at once: 4.3 GB of fp32
    # scores and 2.1 GB of bf16 probabilities on top of the activations
    n = L.dit_vae_workspace_bytes(C.byref(c), 4, 68, 120)
    assert 6.3e9 < n < 24 * 2 ** 30


def test_vae_decode_validation_errors(L):
    c = dit.vae_config(synth.VAE_TINY)
    w = dit.VaeWeightsC()
    fake = 1 << 20  # never dereferenced: validation fails first
    st = L.dit_vae_decode_forward(C.byref(c), C.byref(w), fake, 1, 2, 2, fake, fake, 1 << 30, None)
    assert st == dit.DIT_E_NULL and "weight" in dit.last_error()
    st = L.dit_vae_decode_forward(C.byref(c), None, fake, 1, 2, 2, fake, fake, 1 << 30, None)
    assert st == dit.DIT_E_NULL
    # every weight present: shape, alignment and workspace errors
    ptrs = iter(range(1 << 20, 1 << 40, 1 << 12))
    vcfg = synth.VAE_TINY
    for f, _ in dit.VaeWeightsC._fields_:
        v = getattr(w, f)
        if isinstance(v, int) or v is None:
            setattr(w, f, next(ptrs))
    for arr in (w.attn_w, w.attn_b, w.upconv_w, w.upconv_b):
        for i in range(len(arr)):
            arr[i] = next(ptrs)

    def fill(r, ci, co):
        for f, _ in dit.VaeResnetC._fields_:
            if f.startswith("short") and ci == co:
                setattr(r, f, None)
            else:
                setattr(r, f, next(ptrs))
    for name, ci, co in vcfg.resnet_channels():
        if name.startswith("mid"):
            fill(w.mid[int(name[7])], ci, co)
        else:
            fill(w.up[int(name[2])][int(name[7])], ci, co)
    need = L.dit_vae_workspace_bytes(C.byref(c), 1, 2, 2)
    # (never a call whose arguments are all valid: it would launch kernels)
    st = L.dit_vae_decode_forward(C.byref(c), C.byref(w), fake, 0, 2, 2, fake, fake, need, None)
    assert st == dit.DIT_E_SHAPE
    st = L.dit_vae_decode_forward(C.byref(c), C.byref(w), fake, 1, 2, 2, fake, fake, need - 1, None)
    assert st == dit.DIT_E_WORKSPACE
    st = L.dit_vae_decode_forward(C.byref(c), C.byref(w), fake + 4, 1, 2, 2, fake, fake, need, None)
    assert st == dit.DIT_E_SHAPE and "aligned" in dit.last_error()
    # a shortcut where the width is kept, and a missing one where it changes
    w.mid[0].short_w = next(ptrs)
    st = L.dit_vae_decode_forward(C.byref(c), C.byref(w), fake, 1, 2, 2, fake, fake, need, None)
    assert st == dit.DIT_E_NULL and "shortcut" in dit.last_error()
    w.mid[0].short_w = None
    w.up[1][0].short_w = None
    st = L.dit_vae_decode_forward(C.byref(c), C.byref(w), fake, 1, 2, 2, fake, fake, need, None)
    assert st == dit.DIT_E_NULL


def test_vae_conv_and_group_norm_validation_errors(L):
    fake = 1 << 20
    conv = L.dit_vae_conv_forward
    ok = dict(xin=fake, c_in=64, ksize=3, up=0, w=fake, bias=fake, xs=None, c_short=0,
              short_w=None, short_b=None, resid=None, B=1, H=8, W=8, c_out=64, out=fake,
              out_f32=0, stream=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return conv(*a.values())
    assert call(xin=None) == dit.DIT_E_NULL
    assert call(c_in=12) == dit.DIT_E_SHAPE
    assert call(ksize=5) == dit.DIT_E_SHAPE
    assert call(up=1, H=7) == dit.DIT_E_SHAPE
    assert call(xs=fake) == dit.DIT_E_NULL
    assert call(B=0) == dit.DIT_E_SHAPE
    assert call(H=1) == dit.DIT_E_SHAPE
    assert call(out=fake + 8) == dit.DIT_E_SHAPE
    gn = L.dit_vae_group_norm_forward
    need = L.dit_vae_group_norm_ws_bytes(1, 100, 64, 32)
    assert need > 0
    assert gn(fake, fake + 4096, fake, fake, 1, 100, 48, 16, 1e-6, 1, fake, need, None) == dit.DIT_E_UNSUPPORTED
    assert gn(fake, fake + 4096, fake, fake, 1, 100, 64, 24, 1e-6, 1, fake, need, None) == dit.DIT_E_UNSUPPORTED
    assert gn(fake, fake, fake, fake, 1, 100, 64, 32, 1e-6, 1, fake, need, None) == dit.DIT_E_VALUE
    assert gn(fake, fake + 4096, fake, fake, 1, 100, 64, 32, 0.0, 1, fake, need, None) == dit.DIT_E_VALUE
    assert gn(fake, fake + 4096, fake, fake, 1, 100, 64, 32, 1e-6, 1, fake, need - 1, None) == dit.DIT_E_WORKSPACE


def test_linear_validation_errors(L):
    fake = 1 << 20
    f = L.dit_linear_forward
    y = fake + (1 << 24)
    assert f(None, fake, y, 256, 256, 128, None) == dit.DIT_E_NULL
    assert f(fake, fake, None, 256, 256, 128, None) == dit.DIT_E_NULL
    assert f(fake + 8, fake, y, 256, 256, 128, None) == dit.DIT_E_SHAPE   # unaligned a
    assert f(fake, fake, y, -1, 256, 128, None) == dit.DIT_E_SHAPE
    assert f(fake, fake, y, 256, 254, 128, None) == dit.DIT_E_SHAPE       # N % 4
    assert f(fake, fake, y, 256, 256, 96, None) == dit.DIT_E_SHAPE        # K % 64
    assert f(fake, fake, y, 256, 0, 128, None) == dit.DIT_E_SHAPE
    assert f(fake, fake, y, 1 << 22, 256, 1024, None) == dit.DIT_E_UNSUPPORTED  # 8 GiB of a
    assert f(fake, fake, fake + 4096, 256, 256, 128, None) == dit.DIT_E_VALUE   # y inside a
    assert f(fake, fake, y, 0, 256, 128, None) == dit.DIT_OK              # nothing to launch
    assert f(None, None, None, 0, 256, 128, None) == dit.DIT_OK
    assert f(None, None, None, 0, 254, 128, None) == dit.DIT_E_SHAPE
