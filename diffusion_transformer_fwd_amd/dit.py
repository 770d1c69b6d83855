"""ctypes binding of libdit.so (the C ABI declared in include/dit.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libdit.so. torch supplies device memory and the current stream.
The library is loaded on first use; if it is missing, calls raise.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from . import synth

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdit.so")
_lib: Optional[C.CDLL] = None

DIT_OK, DIT_E_NULL, DIT_E_SHAPE, DIT_E_UNSUPPORTED, DIT_E_WORKSPACE, DIT_E_HIP, DIT_E_VALUE = (
    0, -1, -2, -3, -4, -5, -6)
WS_DUAL, WS_SINGLE, WS_STEP, WS_MOD, WS_DENOISE = 0, 1, 2, 3, 4
MOD_DUAL_IMG, MOD_DUAL_TXT, MOD_SINGLE, MOD_FINAL, MOD_ROWS = 0, 6, 12, 15, 17
MAX_BATCH = 64
EXPORTS = ("dit_position_ids", "dit_workspace_bytes", "dit_status_string", "dit_last_error",
           "dit_config_check", "dit_rope_tables_build", "dit_modulation_forward",
           "dit_dual_block_forward", "dit_single_block_forward", "dit_step_forward",
           "dit_denoise_forward", "dit_profile_begin", "dit_profile_end",
           "dit_modulation_forward_noalloc", "dit_linear_forward")
# the latent decoder (include/dit_vae.h)
VAE_EXPORTS = ("dit_vae_config_check", "dit_vae_config_default", "dit_vae_workspace_bytes",
               "dit_vae_decode_forward", "dit_vae_conv_forward", "dit_vae_group_norm_ws_bytes",
               "dit_vae_group_norm_forward")
(K_GEMM, K_ATTENTION, K_MODNORM, K_QKV_PAD, K_GEMV, K_ROPE_TABLES, K_TIME, K_SPLIT_SUM, K_LATENT,
 K_ATTN_GEMM, K_CONV, K_GROUPNORM, K_SOFTMAX, K_LATENT_IMAGE, K_CONV_HALO, K_COUNT) = range(16)
KERNEL_NAMES = ("gemm", "attention", "modnorm", "qkv_pad", "gemv", "rope_tables", "time_features",
                "split_sum", "latent", "attn_gemm", "conv", "group_norm", "softmax",
                "latent_image", "conv_halo")
VAE_MAX_LAYERS = 4
MAX_STEPS = 64


class DitError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"dit status {status}: {msg}")
        self.status = status


class Config(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("heads", C.c_int32), ("head_dim", C.c_int32),
                ("mlp_hidden", C.c_int32), ("n_dual", C.c_int32), ("n_single", C.c_int32),
                ("in_channels", C.c_int32), ("txt_channels", C.c_int32),
                ("time_channels", C.c_int32), ("axes_dim", C.c_int32 * 4),
                ("prenorm", C.c_int32), ("theta", C.c_float), ("eps", C.c_float)]


class DualWeightsC(C.Structure):
    _fields_ = [("qkv", C.c_void_p * 2), ("out", C.c_void_p * 2), ("mlp_in", C.c_void_p * 2),
                ("mlp_out", C.c_void_p * 2), ("q_gain", C.c_void_p * 2),
                ("k_gain", C.c_void_p * 2)]


class SingleWeightsC(C.Structure):
    _fields_ = [("w_in", C.c_void_p), ("w_out", C.c_void_p), ("q_gain", C.c_void_p),
                ("k_gain", C.c_void_p)]


class KernelStats(C.Structure):
    _fields_ = [("kind", C.c_int32), ("launches", C.c_int32), ("total_ms", C.c_double),
                ("flops", C.c_double), ("bytes", C.c_double)]


class ModelWeightsC(C.Structure):
    _fields_ = [("t_in", C.c_void_p), ("t_out", C.c_void_p), ("mod_dual_img", C.c_void_p),
                ("mod_dual_txt", C.c_void_p), ("mod_single", C.c_void_p),
                ("mod_final", C.c_void_p), ("x_embed", C.c_void_p), ("ctx_embed", C.c_void_p),
                ("proj_out", C.c_void_p), ("dual", C.POINTER(DualWeightsC)),
                ("single", C.POINTER(SingleWeightsC))]


class VaeConfigC(C.Structure):
    _fields_ = [("z_channels", C.c_int32), ("block_channels", C.c_int32 * 4),
                ("layers", C.c_int32), ("groups", C.c_int32), ("eps", C.c_float)]


class VaeResnetC(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("gn1_gamma", "gn1_beta", "conv1_w", "conv1_b",
                                          "gn2_gamma", "gn2_beta", "conv2_w", "conv2_b",
                                          "short_w", "short_b")]


class VaeWeightsC(C.Structure):
    _fields_ = [("lat_scale", C.c_void_p), ("lat_shift", C.c_void_p),
                ("conv_in_w", C.c_void_p), ("conv_in_b", C.c_void_p),
                ("mid", VaeResnetC * 2), ("attn_gn_gamma", C.c_void_p),
                ("attn_gn_beta", C.c_void_p), ("attn_w", C.c_void_p * 4),
                ("attn_b", C.c_void_p * 4), ("up", (VaeResnetC * VAE_MAX_LAYERS) * 4),
                ("upconv_w", C.c_void_p * 3), ("upconv_b", C.c_void_p * 3),
                ("norm_out_gamma", C.c_void_p), ("norm_out_beta", C.c_void_p),
                ("conv_out_w", C.c_void_p), ("conv_out_b", C.c_void_p)]


def library_path() -> str:
    return _LIB_PATH


def lib() -> C.CDLL:
    """Load libdit.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m diffusion_transformer_fwd_amd.build`")
    L = C.CDLL(_LIB_PATH)
    vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    pc = C.POINTER(Config)
    L.dit_position_ids.restype = i64
    L.dit_position_ids.argtypes = [i64, i32, i32, i32, vp, vp, vp, i64]
    L.dit_workspace_bytes.restype = sz
    L.dit_workspace_bytes.argtypes = [pc, i32, i32, i64]
    L.dit_status_string.restype = C.c_char_p
    L.dit_status_string.argtypes = [C.c_int]
    L.dit_last_error.restype = C.c_char_p
    L.dit_last_error.argtypes = []
    L.dit_config_check.restype = C.c_int
    L.dit_config_check.argtypes = [pc]
    L.dit_rope_tables_build.restype = C.c_int
    L.dit_rope_tables_build.argtypes = [pc, vp, i64, vp, vp, vp]
    L.dit_modulation_forward.restype = C.c_int
    L.dit_modulation_forward.argtypes = [pc, C.POINTER(ModelWeightsC), vp, i32, vp, vp, sz, vp]
    L.dit_modulation_forward_noalloc.restype = C.c_int
    L.dit_modulation_forward_noalloc.argtypes = [pc, C.POINTER(ModelWeightsC), vp, i32, vp, vp]
    L.dit_dual_block_forward.restype = C.c_int
    L.dit_dual_block_forward.argtypes = [pc, C.POINTER(DualWeightsC), vp, i32, i64, i64, vp, vp,
                                         i64, vp, vp, vp, sz, vp]
    L.dit_single_block_forward.restype = C.c_int
    L.dit_single_block_forward.argtypes = [pc, C.POINTER(SingleWeightsC), vp, i32, i64, vp, i64,
                                           vp, vp, vp, sz, vp]
    L.dit_step_forward.restype = C.c_int
    L.dit_step_forward.argtypes = [pc, C.POINTER(ModelWeightsC), vp, vp, vp, i32, i64, i64, i64,
                                   vp, vp, vp, vp, sz, vp]
    L.dit_denoise_forward.restype = C.c_int
    L.dit_denoise_forward.argtypes = [pc, C.POINTER(ModelWeightsC), vp, vp, vp, vp, i32, i32, i64,
                                      i64, i64, vp, vp, vp, sz, vp]
    L.dit_profile_begin.restype = C.c_int
    L.dit_linear_forward.restype = C.c_int
    L.dit_linear_forward.argtypes = [vp, vp, vp, i64, i32, i32, vp]
    L.dit_profile_begin.argtypes = []
    L.dit_profile_end.restype = C.c_int
    L.dit_profile_end.argtypes = [C.POINTER(KernelStats)]
    pv = C.POINTER(VaeConfigC)
    L.dit_vae_config_check.restype = C.c_int
    L.dit_vae_config_check.argtypes = [pv]
    L.dit_vae_config_default.restype = None
    L.dit_vae_config_default.argtypes = [pv]
    L.dit_vae_workspace_bytes.restype = sz
    L.dit_vae_workspace_bytes.argtypes = [pv, i32, i32, i32]
    L.dit_vae_decode_forward.restype = C.c_int
    L.dit_vae_decode_forward.argtypes = [pv, C.POINTER(VaeWeightsC), vp, i32, i32, i32, vp, vp,
                                         sz, vp]
    L.dit_vae_conv_forward.restype = C.c_int
    L.dit_vae_conv_forward.argtypes = [vp, i32, i32, i32, vp, vp, vp, i32, vp, vp, vp, i32, i32,
                                       i32, i32, vp, i32, vp]
    L.dit_vae_group_norm_ws_bytes.restype = sz
    L.dit_vae_group_norm_ws_bytes.argtypes = [i32, i64, i32, i32]
    L.dit_vae_group_norm_forward.restype = C.c_int
    L.dit_vae_group_norm_forward.argtypes = [vp, vp, vp, vp, i32, i64, i32, i32, C.c_float, i32,
                                             vp, sz, vp]
    _lib = L
    return L


def last_error() -> str:
    return lib().dit_last_error().decode()


def _check(status: int) -> None:
    if status != DIT_OK:
        raise DitError(status, last_error())


def config(cfg: synth.DitConfig) -> Config:
    c = Config()
    c.hidden, c.heads, c.head_dim = cfg.hidden, cfg.heads, cfg.head_dim
    c.mlp_hidden, c.n_dual, c.n_single = cfg.mlp_hidden, cfg.n_dual, cfg.n_single
    c.in_channels, c.txt_channels, c.time_channels = (cfg.in_channels, cfg.txt_channels,
                                                      cfg.time_channels)
    for i in range(4):
        c.axes_dim[i] = cfg.axes_dim[i]
    c.prenorm, c.theta, c.eps = cfg.prenorm, cfg.theta, cfg.eps
    return c


# ---------------------------------------------------------------- host helpers

def position_ids(n_txt: int, img_grid: Tuple[int, int],
                 ref_grids: Sequence[Tuple[int, int]] = ()) -> np.ndarray:
    """int32 [S, 4] token ids from the library's host routine."""
    hp, wp = img_grid
    cap = n_txt + hp * wp + sum(h * w for h, w in ref_grids)
    out = np.zeros((max(cap, 1), 4), np.int32)
    rh = (C.c_int32 * 3)(*[g[0] for g in ref_grids])
    rw = (C.c_int32 * 3)(*[g[1] for g in ref_grids])
    s = lib().dit_position_ids(n_txt, hp, wp, len(ref_grids), C.cast(rh, C.c_void_p),
                               C.cast(rw, C.c_void_p), out.ctypes.data, cap)
    if s < 0:
        raise DitError(int(s), last_error())
    return out[:s]


def workspace_bytes(cfg: synth.DitConfig, kind: int, B: int, S: int) -> int:
    c = config(cfg)
    n = lib().dit_workspace_bytes(C.byref(c), kind, B, S)
    if n == 0:
        raise DitError(DIT_E_SHAPE, last_error())
    return int(n)


def profile_begin() -> None:
    _check(lib().dit_profile_begin())


def profile_end() -> Dict[str, Dict[str, float]]:
    """Per-kernel-family totals of the launches since profile_begin()."""
    arr = (KernelStats * K_COUNT)()
    _check(lib().dit_profile_end(arr))
    return {KERNEL_NAMES[k.kind]: {"launches": k.launches, "total_ms": k.total_ms,
                                   "flops": k.flops, "bytes": k.bytes} for k in arr}


# ---------------------------------------------------------------- device side

def _torch():
    import torch
    return torch


def _stream() -> int:
    return _torch().cuda.current_stream().cuda_stream


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def to_bf16_device(a: np.ndarray, device="cuda"):
    """Upload bf16-representable float32 values as torch.bfloat16 (exact)."""
    torch = _torch()
    bits = synth.bf16_bits(a)
    return torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)


def to_f32_device(a: np.ndarray, device="cuda"):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


class Workspace:
    """A grow-only device workspace (torch-allocated, 256-byte aligned)."""

    def __init__(self):
        self.buf = None

    def get(self, nbytes: int):
        torch = _torch()
        if self.buf is None or self.buf.numel() < nbytes + 256:
            self.buf = torch.empty(nbytes + 256, dtype=torch.uint8, device="cuda")
        p = self.buf.data_ptr()
        off = (-p) % 256
        return p + off, self.buf.numel() - off


class DualWeights:
    def __init__(self, w: Dict[str, np.ndarray]):
        self.t = {k: (to_f32_device(v) if "gain" in k else to_bf16_device(v)) for k, v in w.items()}
        s = DualWeightsC()
        for i in range(2):
            s.qkv[i] = _ptr(self.t[f"qkv{i}"])
            s.out[i] = _ptr(self.t[f"out{i}"])
            s.mlp_in[i] = _ptr(self.t[f"mlp_in{i}"])
            s.mlp_out[i] = _ptr(self.t[f"mlp_out{i}"])
            s.q_gain[i] = _ptr(self.t[f"q_gain{i}"])
            s.k_gain[i] = _ptr(self.t[f"k_gain{i}"])
        self.c = s


class SingleWeights:
    def __init__(self, w: Dict[str, np.ndarray]):
        self.t = {k: (to_f32_device(v) if "gain" in k else to_bf16_device(v)) for k, v in w.items()}
        s = SingleWeightsC()
        s.w_in, s.w_out = _ptr(self.t["w_in"]), _ptr(self.t["w_out"])
        s.q_gain, s.k_gain = _ptr(self.t["q_gain"]), _ptr(self.t["k_gain"])
        self.c = s


class ModelWeights:
    """Device copy of a synth.ModelWeights (bf16 matrices, fp32 gains)."""

    def __init__(self, mw: synth.ModelWeights, workers: int = 8):
        import concurrent.futures as cf
        cfg = mw.cfg
        self.cfg = cfg
        self.glob = {k: to_bf16_device(v) for k, v in mw.glob.items()}
        # blocks are drawn on host threads (independent streams per tensor)
        with cf.ThreadPoolExecutor(max_workers=workers) as ex:
            self.dual: List[DualWeights] = list(
                ex.map(lambda i: DualWeights(mw.dual(i)), range(cfg.n_dual)))
            self.single: List[SingleWeights] = list(
                ex.map(lambda i: SingleWeights(mw.single(i)), range(cfg.n_single)))
        self._dual_arr = (DualWeightsC * max(1, cfg.n_dual))(*[d.c for d in self.dual])
        self._single_arr = (SingleWeightsC * max(1, cfg.n_single))(*[s.c for s in self.single])
        m = ModelWeightsC()
        for k in ("t_in", "t_out", "mod_dual_img", "mod_dual_txt", "mod_single", "mod_final",
                  "x_embed", "ctx_embed", "proj_out"):
            setattr(m, k, _ptr(self.glob[k]))
        m.dual = C.cast(self._dual_arr, C.POINTER(DualWeightsC))
        m.single = C.cast(self._single_arr, C.POINTER(SingleWeightsC))
        self.c = m


def rope_tables(cfg: synth.DitConfig, pos: np.ndarray):
    """cos, sin fp32 [S, head_dim/2] on the device from int32 positions [S, 4]."""
    torch = _torch()
    pos_d = torch.from_numpy(np.ascontiguousarray(pos, dtype=np.int32)).cuda()
    S = pos.shape[0]
    cos = torch.empty((S, cfg.head_dim // 2), dtype=torch.float32, device="cuda")
    sin = torch.empty_like(cos)
    c = config(cfg)
    _check(lib().dit_rope_tables_build(C.byref(c), pos_d.data_ptr(), S, cos.data_ptr(),
                                       sin.data_ptr(), _stream()))
    torch.cuda.current_stream().synchronize()
    return cos, sin


def modulation(cfg: synth.DitConfig, w: ModelWeights, sigma: Sequence[float],
               ws: Optional[Workspace] = None):
    """mod fp32 [B, 17, D] on the device."""
    torch = _torch()
    B = len(sigma)
    mod = torch.empty((B, MOD_ROWS, cfg.hidden), dtype=torch.float32, device="cuda")
    sig = np.ascontiguousarray(sigma, dtype=np.float32)
    ws = ws or Workspace()
    p, n = ws.get(workspace_bytes(cfg, WS_MOD, B, 0))
    c = config(cfg)
    _check(lib().dit_modulation_forward(C.byref(c), C.byref(w.c), sig.ctypes.data, B,
                                        mod.data_ptr(), p, n, _stream()))
    return mod


def modulation_noalloc(cfg: synth.DitConfig, w: ModelWeights, sigma: Sequence[float], out=None):
    """mod fp32 [B, 17, D] through the entry point that takes no workspace
    (its scratch is the library's fixed device array); out may be given."""
    torch = _torch()
    B = len(sigma)
    if out is None:
        out = torch.empty((B, MOD_ROWS, cfg.hidden), dtype=torch.float32, device="cuda")
    sig = np.ascontiguousarray(sigma, dtype=np.float32)
    c = config(cfg)
    _check(lib().dit_modulation_forward_noalloc(C.byref(c), C.byref(w.c), sig.ctypes.data, B,
                                                out.data_ptr(), _stream()))
    return out


def dual_block(cfg: synth.DitConfig, w: DualWeights, x, n_txt: int, mod, cos, sin,
               ws: Optional[Workspace] = None) -> None:
    """In place on x (fp32 [B, S, D]); mod fp32 [B, 17, D] (the step buffer)."""
    B, S, D = x.shape
    ws = ws or Workspace()
    p, n = ws.get(workspace_bytes(cfg, WS_DUAL, B, S))
    c = config(cfg)
    mp = mod.data_ptr()
    _check(lib().dit_dual_block_forward(
        C.byref(c), C.byref(w.c), x.data_ptr(), B, S, n_txt, mp + 4 * MOD_DUAL_TXT * D,
        mp + 4 * MOD_DUAL_IMG * D, MOD_ROWS * D, cos.data_ptr(), sin.data_ptr(), p, n, _stream()))


def single_block(cfg: synth.DitConfig, w: SingleWeights, x, mod, cos, sin,
                 ws: Optional[Workspace] = None) -> None:
    B, S, D = x.shape
    ws = ws or Workspace()
    p, n = ws.get(workspace_bytes(cfg, WS_SINGLE, B, S))
    c = config(cfg)
    _check(lib().dit_single_block_forward(
        C.byref(c), C.byref(w.c), x.data_ptr(), B, S, mod.data_ptr() + 4 * MOD_SINGLE * D,
        MOD_ROWS * D, cos.data_ptr(), sin.data_ptr(), p, n, _stream()))


def step(cfg: synth.DitConfig, w: ModelWeights, txt, latents, sigma: Sequence[float],
         n_img: int, cos, sin, ws: Optional[Workspace] = None, out=None):
    """One denoise step; txt bf16 [B, n_txt, C_txt], latents bf16 [B, n_img+n_ref, C_in].

    Returns v fp32 [B, n_img, C_in]."""
    torch = _torch()
    B, n_txt = txt.shape[0], txt.shape[1]
    n_ref = latents.shape[1] - n_img
    S = n_txt + n_img + n_ref
    if out is None:
        out = torch.empty((B, n_img, cfg.in_channels), dtype=torch.float32, device="cuda")
    sig = np.ascontiguousarray(sigma, dtype=np.float32)
    ws = ws or Workspace()
    p, n = ws.get(workspace_bytes(cfg, WS_STEP, B, S))
    c = config(cfg)
    _check(lib().dit_step_forward(
        C.byref(c), C.byref(w.c), txt.data_ptr(), latents.data_ptr(), sig.ctypes.data, B, n_txt,
        n_img, n_ref, cos.data_ptr(), sin.data_ptr(), out.data_ptr(), p, n, _stream()))
    return out


def denoise(cfg: synth.DitConfig, w: ModelWeights, txt, z, ref, sigmas, cos, sin,
            ws: Optional[Workspace] = None):
    """The sampling loop, in place on z (fp32 [B, n_img, C_in]).

    txt bf16 [B, n_txt, C_txt]; ref bf16 [B, n_ref, C_in] or None; sigmas
    [B, n_steps + 1] (host values). Returns z."""
    B, n_img = z.shape[0], z.shape[1]
    n_txt = txt.shape[1]
    n_ref = 0 if ref is None else ref.shape[1]
    sig = np.ascontiguousarray(np.broadcast_to(np.asarray(sigmas, dtype=np.float32),
                                               (B, np.shape(sigmas)[-1])))
    n_steps = sig.shape[1] - 1
    S = n_txt + n_img + n_ref
    ws = ws or Workspace()
    p, n = ws.get(workspace_bytes(cfg, WS_DENOISE, B, S))
    c = config(cfg)
    _check(lib().dit_denoise_forward(
        C.byref(c), C.byref(w.c), txt.data_ptr(), z.data_ptr(), _ptr(ref), sig.ctypes.data,
        n_steps, B, n_txt, n_img, n_ref, cos.data_ptr(), sin.data_ptr(), p, n, _stream()))
    return z


def linear(a, w, out=None):
    """y = a w^T in fp32 for bf16 device tensors a [M, K] and w [N, K]."""
    torch = _torch()
    M, K = a.shape
    N = w.shape[0]
    out = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=a.device)
    _check(lib().dit_linear_forward(a.data_ptr(), w.data_ptr(), out.data_ptr(), M, N, K,
                                    _stream()))
    return out


# ---------------------------------------------------------------- latent decoder

def vae_config(vcfg: synth.VaeConfig) -> VaeConfigC:
    c = VaeConfigC()
    c.z_channels = vcfg.z_channels
    for i in range(4):
        c.block_channels[i] = vcfg.block_channels[i]
    c.layers, c.groups, c.eps = vcfg.layers, vcfg.groups, vcfg.eps
    return c


def vae_config_check(vcfg: synth.VaeConfig) -> None:
    c = vae_config(vcfg)
    _check(lib().dit_vae_config_check(C.byref(c)))


def vae_workspace_bytes(vcfg: synth.VaeConfig, B: int, hp: int, wp: int) -> int:
    c = vae_config(vcfg)
    n = lib().dit_vae_workspace_bytes(C.byref(c), B, hp, wp)
    if n == 0:
        raise DitError(DIT_E_SHAPE, last_error())
    return int(n)


class VaeWeights:
    """Device copy of synth.vae_weights: conv weights bf16 in their
    [C_out, kh, kw, C_in] order, everything else fp32."""

    def __init__(self, vcfg: synth.VaeConfig, w: Dict[str, np.ndarray]):
        self.t = {k: (to_bf16_device(v) if k.endswith(".w") else to_f32_device(v))
                  for k, v in w.items()}
        t = self.t
        g = lambda k: _ptr(t.get(k))
        s = VaeWeightsC()
        s.lat_scale, s.lat_shift = g("lat_scale"), g("lat_shift")
        s.conv_in_w, s.conv_in_b = g("conv_in.w"), g("conv_in.b")

        def res(dst, p):
            for f, k in (("gn1_gamma", "gn1.g"), ("gn1_beta", "gn1.b"), ("conv1_w", "conv1.w"),
                         ("conv1_b", "conv1.b"), ("gn2_gamma", "gn2.g"), ("gn2_beta", "gn2.b"),
                         ("conv2_w", "conv2.w"), ("conv2_b", "conv2.b"), ("short_w", "short.w"),
                         ("short_b", "short.b")):
                setattr(dst, f, g(p + k))
        res(s.mid[0], "mid.res0.")
        res(s.mid[1], "mid.res1.")
        s.attn_gn_gamma, s.attn_gn_beta = g("mid.attn.gn.g"), g("mid.attn.gn.b")
        for i, n in enumerate("qkvo"):
            s.attn_w[i] = g(f"mid.attn.{n}.w")
            s.attn_b[i] = g(f"mid.attn.{n}.b")
        for lv in range(4):
            for r in range(vcfg.layers):
                res(s.up[lv][r], f"up{lv}.res{r}.")
        for lv in range(3):
            s.upconv_w[lv] = g(f"up{lv}.upconv.w")
            s.upconv_b[lv] = g(f"up{lv}.upconv.b")
        s.norm_out_gamma, s.norm_out_beta = g("norm_out.g"), g("norm_out.b")
        s.conv_out_w, s.conv_out_b = g("conv_out.w"), g("conv_out.b")
        self.c = s


def vae_decode(vcfg: synth.VaeConfig, w: VaeWeights, z, hp: int, wp: int,
               ws: Optional[Workspace] = None, out=None):
    """Image fp32 [B, 16 hp, 16 wp, 3] from tokens z fp32 [B, hp * wp, 4 Z]."""
    torch = _torch()
    B = z.shape[0]
    if out is None:
        out = torch.empty((B, 16 * hp, 16 * wp, 3), dtype=torch.float32, device="cuda")
    ws = ws or Workspace()
    p, n = ws.get(vae_workspace_bytes(vcfg, B, hp, wp))
    c = vae_config(vcfg)
    _check(lib().dit_vae_decode_forward(C.byref(c), C.byref(w.c), z.data_ptr(), B, hp, wp,
                                        out.data_ptr(), p, n, _stream()))
    return out


def vae_conv(xin, c_in: int, ksize: int, up: int, w, bias, B: int, H: int, W: int, c_out: int,
             xs=None, c_short: int = 0, short_w=None, short_b=None, resid=None,
             out_f32: bool = False, out=None):
    """One decoder convolution (dit_vae_conv_forward); tensors on the device,
    activations channels-last bf16, weights bf16 [c_out, k, k, c_in]."""
    torch = _torch()
    if out is None:
        out = torch.empty((B, H, W, c_out), dtype=torch.float32 if out_f32 else torch.bfloat16,
                          device="cuda")
    _check(lib().dit_vae_conv_forward(
        _ptr(xin), c_in, ksize, up, _ptr(w), _ptr(bias), _ptr(xs), c_short, _ptr(short_w),
        _ptr(short_b), _ptr(resid), B, H, W, c_out, out.data_ptr(), 1 if out_f32 else 0,
        _stream()))
    return out


def vae_group_norm(x, gamma, beta, B: int, HW: int, Cc: int, groups: int, eps: float,
                   silu: bool, ws: Optional[Workspace] = None, out=None):
    """y = act(GroupNorm(x)) (dit_vae_group_norm_forward), bf16 [B, HW, C]."""
    torch = _torch()
    if out is None:
        out = torch.empty((B, HW, Cc), dtype=torch.bfloat16, device="cuda")
    n = lib().dit_vae_group_norm_ws_bytes(B, HW, Cc, groups)
    if n == 0:
        raise DitError(DIT_E_SHAPE, last_error())
    ws = ws or Workspace()
    p, cap = ws.get(int(n))
    _check(lib().dit_vae_group_norm_forward(x.data_ptr(), out.data_ptr(), gamma.data_ptr(),
                                            beta.data_ptr(), B, HW, Cc, groups, eps,
                                            1 if silu else 0, p, cap, _stream()))
    return out
