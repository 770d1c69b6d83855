// Host-side planning and argument checks of libdit.so (see plan.hpp).
#include "plan.hpp"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

namespace dit {
namespace host {

namespace {
thread_local std::string g_last_error;

}  // namespace

const char* last_error_message() { return g_last_error.c_str(); }

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}


size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }


// ---------------------------------------------------------------- layouts

// kind: 0 = dual, 1 = single
BlockLayout block_layout(const dit_config& c, int kind, int64_t B, int64_t S) {
  BlockLayout L;
  const int64_t D = c.hidden, F = c.mlp_hidden;
  L.R = B * S;
  L.S_pad = round_up(S, 256);  // attention reads whole 256-query blocks
  L.u_cols = kind == 0 ? F : 0;  // dual: the SwiGLU activation (q, k, v go straight to L.q/k/vt)
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.h = take((size_t)L.R * D * 2);
  if (L.u_cols) L.u = take((size_t)L.R * L.u_cols * 2);
  if (kind == 1) L.d6 = take((size_t)L.R * (D + F) * 2);
  else L.o = take((size_t)L.R * D * 2);
  const size_t qk = (size_t)B * c.heads * L.S_pad * c.head_dim * 2;
  L.q = take(qk);
  L.k = take(qk);
  L.vt = take(qk);
  L.total = off;
  return L;
}


ModLayout mod_layout(const dit_config& c, int64_t B) {
  ModLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.e = take((size_t)B * c.time_channels * 4);
  L.t1 = take((size_t)B * c.hidden * 4);
  L.m = take((size_t)B * c.hidden * 4);
  L.total = off;
  return L;
}


StepLayout step_layout(const dit_config& c, int64_t B, int64_t S) {
  StepLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.x = take((size_t)B * S * c.hidden * 4);
  L.mod = take((size_t)B * DIT_MOD_ROWS * c.hidden * 4);
  L.modws = take(mod_layout(c, B).total);
  const size_t blk = std::max(block_layout(c, 0, B, S).total, block_layout(c, 1, B, S).total);
  L.block = take(blk);
  L.total = off;
  return L;
}

// The sampling loop: the step's workspace, then its latent operand
// lat bf16 [B, S, C] and velocity v fp32 [B, S, C] (sized for S rows, so the
// workspace query needs no split of S into image and reference tokens).
// Steps whose modulation vectors one pass over the modulation weights
// computes in the sampling loop (the GEMV takes four rows per pass, so at
// B = 1 the pages' four steps cost one pass instead of four).


DenoiseLayout denoise_layout(const dit_config& c, int64_t B, int64_t S) {
  DenoiseLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.step = take(step_layout(c, B, S).total);
  L.lat = take((size_t)B * S * c.in_channels * 2);
  L.v = take((size_t)B * S * c.in_channels * 4);
  L.mods = take((size_t)kModSteps * B * DIT_MOD_ROWS * c.hidden * 4);
  L.modws = take(mod_layout(c, (int64_t)kModSteps * B).total);
  L.txt = take((size_t)B * S * c.hidden * 4);  // embedded text rows (n_txt <= S)
  L.total = off;
  return L;
}

// K split of a GEMM whose tiles alone would leave most CUs idle for the whole
// launch: the final projection (N = 128, one column of tiles) and the text
// embedding (K = 7680 on 2 B row tiles). With so few tiles a launch is bound
// by the latency of each tile's own K loop, so the chunks are short (about
// 384 to 1152 of K). The chunk count depends on N and K only, never on M,
// and the chunks are summed in a fixed order, so a batch row's result does
// not depend on the rest of the batch.
int split_k_chunks(int64_t N, int64_t K) {
  if (N <= 256) return (int)std::max<int64_t>(1, std::min<int64_t>(8, K / 384));
  return (int)std::max<int64_t>(1, std::min<int64_t>(7, K / 1024));
}

// ---------------------------------------------------------------- validation

int check_config(const dit_config* c) {
  if (!c) return fail(DIT_E_NULL, "config is NULL");
  if (c->head_dim != 128)
    return fail(DIT_E_UNSUPPORTED, "head_dim %d: only 128 is supported", c->head_dim);
  if (c->heads < 1 || c->heads > 256)
    return fail(DIT_E_SHAPE, "heads %d out of range [1, 256]", c->heads);
  if (c->hidden != c->heads * c->head_dim)
    return fail(DIT_E_SHAPE, "hidden %d != heads %d x head_dim %d", c->hidden, c->heads,
                c->head_dim);
  if (c->hidden % 64 || c->hidden > 4096)
    return fail(DIT_E_UNSUPPORTED, "hidden %d must be a multiple of 64 and <= 4096", c->hidden);
  if (c->mlp_hidden < 64 || c->mlp_hidden % 64)
    return fail(DIT_E_UNSUPPORTED, "mlp_hidden %d must be a positive multiple of 64",
                c->mlp_hidden);
  if (c->n_dual < 0 || c->n_single < 0 || c->n_dual > 1024 || c->n_single > 1024)
    return fail(DIT_E_SHAPE, "block counts %d/%d out of range", c->n_dual, c->n_single);
  if (c->in_channels < 64 || c->in_channels % 64)
    return fail(DIT_E_UNSUPPORTED, "in_channels %d must be a positive multiple of 64",
                c->in_channels);
  if (c->txt_channels < 64 || c->txt_channels % 64)
    return fail(DIT_E_UNSUPPORTED, "txt_channels %d must be a positive multiple of 64",
                c->txt_channels);
  if (c->time_channels < 2 || c->time_channels % 8 || c->time_channels > 4096)
    return fail(DIT_E_UNSUPPORTED, "time_channels %d must be even, a multiple of 8, <= 4096",
                c->time_channels);
  int sum = 0;
  for (int a = 0; a < 4; ++a) {
    if (c->axes_dim[a] < 0 || c->axes_dim[a] % 2)
      return fail(DIT_E_SHAPE, "axes_dim[%d] = %d must be even and >= 0", a, c->axes_dim[a]);
    sum += c->axes_dim[a];
  }
  if (sum != c->head_dim)
    return fail(DIT_E_SHAPE, "sum of axes_dim %d != head_dim %d", sum, c->head_dim);
  if (c->prenorm != DIT_PRENORM_RMS && c->prenorm != DIT_PRENORM_LAYER)
    return fail(DIT_E_VALUE, "prenorm %d is neither RMS (0) nor LAYER (1)", c->prenorm);
  if (!std::isfinite(c->theta) || c->theta <= 1.0f)
    return fail(DIT_E_VALUE, "theta %g must be finite and > 1", (double)c->theta);
  if (!std::isfinite(c->eps) || c->eps < 0.0f)
    return fail(DIT_E_VALUE, "eps %g must be finite and >= 0", (double)c->eps);
  return DIT_OK;
}

int check_batch_seq(int32_t B, int64_t S) {
  if (B < 1 || B > DIT_MAX_BATCH) return fail(DIT_E_SHAPE, "B %d out of range [1, %d]", B, DIT_MAX_BATCH);
  if (S < 1 || S > (1 << 20)) return fail(DIT_E_SHAPE, "S %lld out of range [1, 2^20]", (long long)S);
  return DIT_OK;
}

int check_ws(const void* ws, size_t have, size_t need) {
  if (need > 0 && !ws) return fail(DIT_E_NULL, "workspace is NULL (%zu bytes needed)", need);
  if (have < need) return fail(DIT_E_WORKSPACE, "workspace %zu bytes < %zu needed", have, need);
  if (!aligned(ws, kAlign)) return fail(DIT_E_WORKSPACE, "workspace not 256-byte aligned");
  return DIT_OK;
}

int check_ptr(const void* p, const char* what, size_t align) {
  if (!p) return fail(DIT_E_NULL, "%s is NULL", what);
  if (!aligned(p, align)) return fail(DIT_E_SHAPE, "%s is not %zu-byte aligned", what, align);
  return DIT_OK;
}

// Every GEMM operand must stay addressable with 32-bit byte offsets.
int check_operand_sizes(const dit_config& c, int64_t rows) {
  const uint64_t D = c.hidden, F = c.mlp_hidden;
  const uint64_t widest = std::max<uint64_t>({3 * D, D + F, F, (uint64_t)c.txt_channels});
  if ((uint64_t)rows * widest * 2 > kMaxBufferBytes)
    return fail(DIT_E_UNSUPPORTED, "%lld rows x %llu columns exceeds 4 GiB per operand",
                (long long)rows, (unsigned long long)widest);
  if ((3 * D + 2 * F) * D * 2 > kMaxBufferBytes || D * (D + F) * 2 > kMaxBufferBytes)
    return fail(DIT_E_UNSUPPORTED, "weights exceed 4 GiB per matrix");
  return DIT_OK;
}

int check_dual_weights(const dit_dual_weights* w) {
  if (!w) return fail(DIT_E_NULL, "dual weights are NULL");
  for (int s = 0; s < 2; ++s) {
    DIT_CHECK(check_ptr(w->qkv[s], "dual qkv"));
    DIT_CHECK(check_ptr(w->out[s], "dual out"));
    DIT_CHECK(check_ptr(w->mlp_in[s], "dual mlp_in"));
    DIT_CHECK(check_ptr(w->mlp_out[s], "dual mlp_out"));
    DIT_CHECK(check_ptr(w->q_gain[s], "dual q_gain"));
    DIT_CHECK(check_ptr(w->k_gain[s], "dual k_gain"));
  }
  return DIT_OK;
}

int check_single_weights(const dit_single_weights* w) {
  if (!w) return fail(DIT_E_NULL, "single weights are NULL");
  DIT_CHECK(check_ptr(w->w_in, "single w_in"));
  DIT_CHECK(check_ptr(w->w_out, "single w_out"));
  DIT_CHECK(check_ptr(w->q_gain, "single q_gain"));
  DIT_CHECK(check_ptr(w->k_gain, "single k_gain"));
  return DIT_OK;
}

int check_model_weights(const dit_config& c, const dit_model_weights* w, bool blocks) {
  if (!w) return fail(DIT_E_NULL, "model weights are NULL");
  DIT_CHECK(check_ptr(w->t_in, "t_in"));
  DIT_CHECK(check_ptr(w->t_out, "t_out"));
  DIT_CHECK(check_ptr(w->mod_dual_img, "mod_dual_img"));
  DIT_CHECK(check_ptr(w->mod_dual_txt, "mod_dual_txt"));
  DIT_CHECK(check_ptr(w->mod_single, "mod_single"));
  DIT_CHECK(check_ptr(w->mod_final, "mod_final"));
  if (!blocks) return DIT_OK;
  DIT_CHECK(check_ptr(w->x_embed, "x_embed"));
  DIT_CHECK(check_ptr(w->ctx_embed, "ctx_embed"));
  DIT_CHECK(check_ptr(w->proj_out, "proj_out"));
  if (c.n_dual > 0 && !w->dual) return fail(DIT_E_NULL, "dual block array is NULL");
  if (c.n_single > 0 && !w->single) return fail(DIT_E_NULL, "single block array is NULL");
  for (int i = 0; i < c.n_dual; ++i) DIT_CHECK(check_dual_weights(&w->dual[i]));
  for (int i = 0; i < c.n_single; ++i) DIT_CHECK(check_single_weights(&w->single[i]));
  return DIT_OK;
}

int check_sigmas(const float* sigma, int32_t B) {
  if (!sigma) return fail(DIT_E_NULL, "sigma_host is NULL");
  for (int b = 0; b < B; ++b)
    if (!std::isfinite(sigma[b]))
      return fail(DIT_E_VALUE, "sigma[%d] is not finite", b);
  return DIT_OK;
}

int check_block_common(const dit_config* cfg, float* x, int32_t B, int64_t S,
                       int64_t mod_batch_stride, const float* cos_t, const float* sin_t) {
  DIT_CHECK(check_config(cfg));
  DIT_CHECK(check_batch_seq(B, S));
  DIT_CHECK(check_ptr(x, "x"));
  DIT_CHECK(check_ptr(cos_t, "cos"));
  DIT_CHECK(check_ptr(sin_t, "sin"));
  if (mod_batch_stride < 0 || mod_batch_stride % 4)
    return fail(DIT_E_SHAPE, "mod_batch_stride %lld must be >= 0 and a multiple of 4",
                (long long)mod_batch_stride);
  DIT_CHECK(check_operand_sizes(*cfg, (int64_t)B * S));
  return DIT_OK;
}

// Checks shared by the step and the sampling loop (everything but the
// latent, sigma, output and workspace arguments).
int check_step_args(const dit_config* cfg, const dit_model_weights* w, const void* txt,
                    int32_t B, int64_t n_txt, int64_t n_img, int64_t n_ref,
                    const float* cos_dev, const float* sin_dev) {
  DIT_CHECK(check_config(cfg));
  if (n_txt < 0 || n_img < 1 || n_ref < 0)
    return fail(DIT_E_SHAPE, "token counts n_txt %lld, n_img %lld, n_ref %lld invalid",
                (long long)n_txt, (long long)n_img, (long long)n_ref);
  const int64_t S = n_txt + n_img + n_ref;
  DIT_CHECK(check_batch_seq(B, S));
  DIT_CHECK(check_operand_sizes(*cfg, (int64_t)B * S));
  DIT_CHECK(check_model_weights(*cfg, w, true));
  if (n_txt > 0) DIT_CHECK(check_ptr(txt, "txt"));
  DIT_CHECK(check_ptr(cos_dev, "cos"));
  DIT_CHECK(check_ptr(sin_dev, "sin"));
  return DIT_OK;
}

int validate_rope(const dit_config* cfg, const int32_t* pos_dev, int64_t S, const float* cos_dev,
                  const float* sin_dev) {
  DIT_CHECK(check_config(cfg));
  if (S < 0 || S > (1 << 20)) return fail(DIT_E_SHAPE, "S %lld out of range", (long long)S);
  if (S == 0) return DIT_OK;
  DIT_CHECK(check_ptr(pos_dev, "pos", 4));
  DIT_CHECK(check_ptr(cos_dev, "cos"));
  DIT_CHECK(check_ptr(sin_dev, "sin"));
  return DIT_OK;
}

int validate_modulation(const dit_config* cfg, const dit_model_weights* w,
                        const float* sigma_host, int32_t B, const float* mod_dev, const void* ws,
                        size_t ws_bytes, bool noalloc) {
  DIT_CHECK(check_config(cfg));
  if (B < 1 || B > DIT_MAX_BATCH) return fail(DIT_E_SHAPE, "B %d out of range", B);
  DIT_CHECK(check_model_weights(*cfg, w, false));
  DIT_CHECK(check_sigmas(sigma_host, B));
  DIT_CHECK(check_ptr(mod_dev, "mod"));
  if (!noalloc) return check_ws(ws, ws_bytes, mod_layout(*cfg, B).total);
  const size_t need = mod_layout(*cfg, B).total;
  if (need > (size_t)DIT_NOALLOC_SCRATCH_BYTES)
    return fail(DIT_E_UNSUPPORTED, "modulation scratch of %zu bytes exceeds the fixed %zu", need,
                (size_t)DIT_NOALLOC_SCRATCH_BYTES);
  return DIT_OK;
}

int validate_dual(const dit_config* cfg, const dit_dual_weights* w, float* x, int32_t B,
                  int64_t S, int64_t n_txt, const float* mod_txt, const float* mod_img,
                  int64_t mod_batch_stride, const float* cos_dev, const float* sin_dev,
                  const void* ws, size_t ws_bytes) {
  DIT_CHECK(check_block_common(cfg, x, B, S, mod_batch_stride, cos_dev, sin_dev));
  if (n_txt < 0 || n_txt > S)
    return fail(DIT_E_SHAPE, "n_txt %lld out of range [0, S=%lld]", (long long)n_txt,
                (long long)S);
  DIT_CHECK(check_dual_weights(w));
  DIT_CHECK(check_ptr(mod_txt, "mod_txt"));
  DIT_CHECK(check_ptr(mod_img, "mod_img"));
  return check_ws(ws, ws_bytes, block_layout(*cfg, 0, B, S).total);
}

int validate_single(const dit_config* cfg, const dit_single_weights* w, float* x, int32_t B,
                    int64_t S, const float* mod, int64_t mod_batch_stride, const float* cos_dev,
                    const float* sin_dev, const void* ws, size_t ws_bytes) {
  DIT_CHECK(check_block_common(cfg, x, B, S, mod_batch_stride, cos_dev, sin_dev));
  DIT_CHECK(check_single_weights(w));
  DIT_CHECK(check_ptr(mod, "mod"));
  return check_ws(ws, ws_bytes, block_layout(*cfg, 1, B, S).total);
}

int validate_step(const dit_config* cfg, const dit_model_weights* w, const void* txt,
                  const void* latents, const float* sigma_host, int32_t B, int64_t n_txt,
                  int64_t n_img, int64_t n_ref, const float* cos_dev, const float* sin_dev,
                  const float* v_out, const void* ws, size_t ws_bytes) {
  DIT_CHECK(check_step_args(cfg, w, txt, B, n_txt, n_img, n_ref, cos_dev, sin_dev));
  DIT_CHECK(check_ptr(latents, "latents"));
  DIT_CHECK(check_sigmas(sigma_host, B));
  DIT_CHECK(check_ptr(v_out, "v_out"));
  return check_ws(ws, ws_bytes, step_layout(*cfg, B, n_txt + n_img + n_ref).total);
}

int validate_denoise(const dit_config* cfg, const dit_model_weights* w, const void* txt,
                     const float* z, const void* ref, const float* sigmas_host, int32_t n_steps,
                     int32_t B, int64_t n_txt, int64_t n_img, int64_t n_ref,
                     const float* cos_dev, const float* sin_dev, const void* ws,
                     size_t ws_bytes) {
  DIT_CHECK(check_step_args(cfg, w, txt, B, n_txt, n_img, n_ref, cos_dev, sin_dev));
  if (n_steps < 1 || n_steps > DIT_MAX_STEPS)
    return fail(DIT_E_SHAPE, "n_steps %d out of range [1, %d]", n_steps, (int)DIT_MAX_STEPS);
  DIT_CHECK(check_ptr(z, "z"));
  if (n_ref > 0) DIT_CHECK(check_ptr(ref, "ref", 8));
  if (!sigmas_host) return fail(DIT_E_NULL, "sigmas is NULL");
  for (int64_t i = 0; i < (int64_t)B * (n_steps + 1); ++i)
    if (!std::isfinite(sigmas_host[i]))
      return fail(DIT_E_VALUE, "sigmas[%lld] is not finite", (long long)i);
  return check_ws(ws, ws_bytes, denoise_layout(*cfg, B, n_txt + n_img + n_ref).total);
}


// ---------------------------------------------------------------- decoder

namespace {
bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
constexpr int64_t kMaxSampleBytes = 0x7FFFFFFFll;  // conv offsets and the zero-read marker
}  // namespace

void gn_blocks(int64_t HW, int C, int* ppb, int* nblk) {
  const int64_t ppi = 256 / (C / 8);
  int64_t p = 65536 / C;  // about 128 KiB of bf16 per block
  if (p < ppi) p = ppi;
  p = p / ppi * ppi;
  *ppb = (int)p;
  *nblk = (int)((HW + p - 1) / p);
}

int check_vae_config(const dit_vae_config* c) {
  if (!c) return fail(DIT_E_NULL, "decoder config is NULL");
  if (c->z_channels < 8 || c->z_channels > 256 || c->z_channels % 8)
    return fail(DIT_E_UNSUPPORTED, "z_channels %d: a multiple of 8 in [8, 256]", c->z_channels);
  if (c->groups < 1 || c->groups > 1024)
    return fail(DIT_E_UNSUPPORTED, "groups %d out of [1, 1024]", c->groups);
  for (int i = 0; i < 4; ++i) {
    const int w = c->block_channels[i];
    if (!pow2(w) || w < 32 || w > 2048 || w % c->groups)
      return fail(DIT_E_UNSUPPORTED,
                  "block_channels[%d] = %d: a power of two in [32, 2048] divisible by groups %d",
                  i, w, c->groups);
  }
  if (c->layers < 1 || c->layers > DIT_VAE_MAX_LAYERS)
    return fail(DIT_E_UNSUPPORTED, "layers %d out of [1, %d]", c->layers, DIT_VAE_MAX_LAYERS);
  if (!(c->eps > 0.f) || !std::isfinite(c->eps))
    return fail(DIT_E_VALUE, "eps must be positive and finite");
  return DIT_OK;
}

int vae_level_channels(const dit_vae_config& c, int l) { return c.block_channels[3 - l]; }

int vae_resnet_in(const dit_vae_config& c, int l, int r) {
  if (r > 0) return vae_level_channels(c, l);
  return l == 0 ? c.block_channels[3] : vae_level_channels(c, l - 1);
}

VaeLayout vae_layout(const dit_vae_config& c, int64_t B, int64_t hp, int64_t wp) {
  VaeLayout L;
  const int64_t H0 = 2 * hp, W0 = 2 * wp, top = c.block_channels[3];
  L.n0 = H0 * W0;
  auto gn = [&](int64_t pix, int C) {
    int ppb, nblk;
    gn_blocks(pix, C, &ppb, &nblk);
    L.gn_nblk = std::max<int64_t>(L.gn_nblk, nblk);
  };
  L.act = L.n0 * top;
  L.act_h = L.n0 * top;
  gn(L.n0, (int)top);
  int cmax = (int)top;
  for (int l = 0; l < 4; ++l) {
    const int64_t pix = (H0 << l) * (W0 << l);
    const int co = vae_level_channels(c, l);
    cmax = std::max(cmax, co);
    for (int r = 0; r < c.layers; ++r) {
      const int ci = vae_resnet_in(c, l, r);
      L.act = std::max<int64_t>(L.act, pix * std::max(ci, co));
      L.act_h = std::max<int64_t>(L.act_h, pix * co);
      gn(pix, ci);
      gn(pix, co);
    }
  }
  L.ld = round_up(L.n0, 8);
  L.mq = L.n0;
  // query rows per chunk: all of them while the bf16 probabilities (the
  // product's A operand, read with 32-bit buffer offsets) stay under 2^31
  // bytes (every size up to 32768 latent pixels, e.g. 1920x1088); fewer
  // rows mean fewer tiles for the P V product, which has only C columns
  if (L.n0 * L.ld * 2 > kMaxSampleBytes)
    L.mq = std::max<int64_t>(256, kMaxSampleBytes / (L.ld * 2) / 256 * 256);
  // DIT_VAE_ATTN_ROWS (tests): a smaller positive multiple of 256 query rows
  // per chunk, so that small images exercise the chunked path
  if (const char* e = std::getenv("DIT_VAE_ATTN_ROWS")) {
    const long long v = std::atoll(e);
    if (v > 0 && v % 256 == 0 && v < L.mq) L.mq = v;
  }
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.p = take((size_t)(B * L.act * 2));
  L.q = take((size_t)(B * L.act * 2));
  L.t = take((size_t)(B * L.act * 2));
  L.h = take((size_t)(B * L.act_h * 2));
  L.lat = take((size_t)(B * L.n0 * c.z_channels * 2));
  L.part = take((size_t)(B * L.gn_nblk * c.groups * 2 * 4));
  L.ab = take((size_t)(B * cmax * 2 * 4));
  L.s = take((size_t)(L.mq * L.ld * 4));
  L.pm = take((size_t)(L.mq * L.ld * 2));
  L.vt = take((size_t)(B * top * L.ld * 2));
  L.total = off;
  return L;
}

namespace {
int check_resnet(const dit_vae_resnet& r, int ci, int co, const char* where) {
  const void* need[] = {r.gn1_gamma, r.gn1_beta, r.conv1_w, r.conv1_b,
                        r.gn2_gamma, r.gn2_beta, r.conv2_w, r.conv2_b};
  for (const void* p : need) DIT_CHECK(check_ptr(p, where));
  if (ci != co) {
    DIT_CHECK(check_ptr(r.short_w, where));
    DIT_CHECK(check_ptr(r.short_b, where));
  } else if (r.short_w || r.short_b) {
    return fail(DIT_E_NULL, "%s: a shortcut is given but the block keeps %d channels", where, ci);
  }
  return DIT_OK;
}
}  // namespace

int validate_vae_decode(const dit_vae_config* cfg, const dit_vae_weights* w, const float* z,
                        int32_t B, int32_t hp, int32_t wp, const float* image, const void* ws,
                        size_t ws_bytes) {
  DIT_CHECK(check_vae_config(cfg));
  if (!w) return fail(DIT_E_NULL, "decoder weights are NULL");
  const void* need[] = {w->lat_scale, w->lat_shift, w->conv_in_w, w->conv_in_b,
                        w->attn_gn_gamma, w->attn_gn_beta, w->norm_out_gamma,
                        w->norm_out_beta, w->conv_out_w, w->conv_out_b};
  for (const void* p : need) DIT_CHECK(check_ptr(p, "decoder weight"));
  for (int i = 0; i < 4; ++i) {
    DIT_CHECK(check_ptr(w->attn_w[i], "attention weight"));
    DIT_CHECK(check_ptr(w->attn_b[i], "attention bias"));
  }
  const int top = cfg->block_channels[3];
  DIT_CHECK(check_resnet(w->mid[0], top, top, "mid ResNet 0"));
  DIT_CHECK(check_resnet(w->mid[1], top, top, "mid ResNet 1"));
  char where[64];
  for (int l = 0; l < 4; ++l) {
    for (int r = 0; r < cfg->layers; ++r) {
      snprintf(where, sizeof where, "level %d ResNet %d", l, r);
      DIT_CHECK(check_resnet(w->up[l][r], vae_resnet_in(*cfg, l, r), vae_level_channels(*cfg, l),
                             where));
    }
    if (l < 3) {
      DIT_CHECK(check_ptr(w->upconv_w[l], "upsample conv weight"));
      DIT_CHECK(check_ptr(w->upconv_b[l], "upsample conv bias"));
    }
  }
  DIT_CHECK(check_ptr(z, "z"));
  DIT_CHECK(check_ptr(image, "image"));
  if (B < 1 || B > DIT_MAX_BATCH)
    return fail(DIT_E_SHAPE, "B %d out of [1, %d]", B, DIT_MAX_BATCH);
  if (hp < 1 || wp < 1 || 16ll * hp > 32766 || 16ll * wp > 32767)
    return fail(DIT_E_SHAPE, "token grid %d x %d out of range", hp, wp);
  const VaeLayout L = vae_layout(*cfg, B, hp, wp);
  if (L.act * 2 > kMaxSampleBytes || L.mq * L.ld * 2 > kMaxSampleBytes ||
      (int64_t)top * L.ld * 2 > kMaxSampleBytes)
    return fail(DIT_E_UNSUPPORTED, "a %d x %d token grid needs activations over 2 GiB per sample",
                hp, wp);
  return check_ws(ws, ws_bytes, L.total);
}

int validate_vae_conv(const void* xin, int32_t c_in, int32_t ksize, int32_t up, const void* w,
                      const float* bias, const void* xs, int32_t c_short, const void* short_w,
                      const float* short_b, const void* resid, int32_t B, int32_t H, int32_t W,
                      int32_t c_out, const void* out) {
  DIT_CHECK(check_ptr(xin, "xin"));
  DIT_CHECK(check_ptr(w, "w"));
  DIT_CHECK(check_ptr(out, "out"));
  if (bias) DIT_CHECK(check_ptr(bias, "bias"));
  if (resid) DIT_CHECK(check_ptr(resid, "resid"));
  if ((xs != nullptr) != (short_w != nullptr))
    return fail(DIT_E_NULL, "xs and short_w go together");
  if (xs) {
    DIT_CHECK(check_ptr(xs, "xs"));
    DIT_CHECK(check_ptr(short_w, "short_w"));
    if (short_b) DIT_CHECK(check_ptr(short_b, "short_b"));
    if (c_short < 8 || c_short % 8) return fail(DIT_E_SHAPE, "c_short %d: a multiple of 8", c_short);
  }
  if (c_in < 8 || c_in % 8) return fail(DIT_E_SHAPE, "c_in %d: a multiple of 8", c_in);
  if (ksize != 1 && ksize != 3) return fail(DIT_E_SHAPE, "ksize %d: 1 or 3", ksize);
  if (up != 0 && up != 1) return fail(DIT_E_VALUE, "up must be 0 or 1");
  if (B < 1 || B > DIT_MAX_BATCH) return fail(DIT_E_SHAPE, "B %d out of [1, %d]", B, DIT_MAX_BATCH);
  if (H < 2 || W < 1 || H > 32766 || W > 32767 || c_out < 1 || c_out > 4096)
    return fail(DIT_E_SHAPE, "grid %d x %d, c_out %d out of range", H, W, c_out);
  if (up && (H % 2 || W % 2)) return fail(DIT_E_SHAPE, "an upsampled conv needs an even grid");
  const int64_t pix = (int64_t)H * W;
  const int64_t taps = (int64_t)ksize * ksize;
  if ((up ? pix / 4 : pix) * c_in * 2 > kMaxSampleBytes || pix * c_out * 4 > kMaxSampleBytes ||
      pix * c_short * 2 > kMaxSampleBytes ||
      ((int64_t)c_out + 256) * taps * c_in * 2 > kMaxSampleBytes ||
      ((int64_t)c_out + 256) * c_short * 2 > kMaxSampleBytes)
    return fail(DIT_E_UNSUPPORTED, "a sample or a weight exceeds 2 GiB");
  return DIT_OK;
}

int validate_linear(const void* a, const void* w, const float* y, int64_t M, int32_t N,
                    int32_t K) {
  if (M < 0 || M > INT32_MAX) return fail(DIT_E_SHAPE, "M %lld out of [0, 2^31)", (long long)M);
  if (N < 4 || N % 4) return fail(DIT_E_SHAPE, "N %d: a positive multiple of 4", N);
  if (K < 64 || K % 64) return fail(DIT_E_SHAPE, "K %d: a positive multiple of 64", K);
  if ((uint64_t)M * K * 2 > kMaxBufferBytes || (uint64_t)N * K * 2 > kMaxBufferBytes)
    return fail(DIT_E_UNSUPPORTED, "an operand exceeds 32-bit byte offsets");
  if (M == 0) return DIT_OK;  // nothing to read or write
  DIT_CHECK(check_ptr(a, "a"));
  DIT_CHECK(check_ptr(w, "w"));
  DIT_CHECK(check_ptr(y, "y"));
  const uintptr_t y0 = reinterpret_cast<uintptr_t>(y), y1 = y0 + (uint64_t)M * N * 4;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), a1 = a0 + (uint64_t)M * K * 2;
  const uintptr_t w0 = reinterpret_cast<uintptr_t>(w), w1 = w0 + (uint64_t)N * K * 2;
  if ((y0 < a1 && a0 < y1) || (y0 < w1 && w0 < y1))
    return fail(DIT_E_VALUE, "y overlaps a or w");
  return DIT_OK;
}

size_t vae_group_norm_ws(int64_t B, int64_t HW, int C, int groups) {
  int ppb, nblk;
  gn_blocks(HW, C, &ppb, &nblk);
  return align_up((size_t)(B * nblk * groups * 2 * 4)) + align_up((size_t)(B * C * 2 * 4));
}

int validate_vae_group_norm(const void* x, const void* y, const float* gamma, const float* beta,
                            int32_t B, int64_t HW, int32_t C, int32_t groups, float eps,
                            const void* ws, size_t ws_bytes) {
  DIT_CHECK(check_ptr(x, "x"));
  DIT_CHECK(check_ptr(y, "y"));
  DIT_CHECK(check_ptr(gamma, "gamma"));
  DIT_CHECK(check_ptr(beta, "beta"));
  if (x == y) return fail(DIT_E_VALUE, "x and y may not alias");
  if (B < 1 || B > DIT_MAX_BATCH) return fail(DIT_E_SHAPE, "B %d out of [1, %d]", B, DIT_MAX_BATCH);
  if (HW < 1 || HW > (1ll << 30)) return fail(DIT_E_SHAPE, "HW %lld out of range", (long long)HW);
  if (!pow2(C) || C < 8 || C > 2048)
    return fail(DIT_E_UNSUPPORTED, "C %d: a power of two in [8, 2048]", C);
  if (groups < 1 || groups > 1024 || C % groups)
    return fail(DIT_E_UNSUPPORTED, "groups %d must divide C %d (at most 1024)", groups, C);
  if (!(eps > 0.f) || !std::isfinite(eps)) return fail(DIT_E_VALUE, "eps must be positive and finite");
  return check_ws(ws, ws_bytes, vae_group_norm_ws(B, HW, C, groups));
}

}  // namespace host
}  // namespace dit

// ======================================================================= ABI
// (host-only entry points)

using namespace dit::host;

extern "C" {

const char* dit_status_string(int status) {
  switch (status) {
    case DIT_OK: return "ok";
    case DIT_E_NULL: return "null pointer";
    case DIT_E_SHAPE: return "inconsistent or out-of-range sizes";
    case DIT_E_UNSUPPORTED: return "unsupported configuration";
    case DIT_E_WORKSPACE: return "workspace too small or misaligned";
    case DIT_E_HIP: return "HIP runtime error";
    case DIT_E_VALUE: return "invalid scalar value";
    default: return "unknown status";
  }
}

const char* dit_last_error(void) { return dit::host::last_error_message(); }

int dit_config_check(const dit_config* cfg) { return check_config(cfg); }

int64_t dit_position_ids(int64_t n_txt, int32_t hp, int32_t wp, int32_t n_ref,
                         const int32_t* ref_hp, const int32_t* ref_wp, int32_t* out,
                         int64_t cap_rows) {
  if (n_txt < 0 || hp < 0 || wp < 0)
    return fail(DIT_E_SHAPE, "negative size (n_txt %lld, grid %d x %d)", (long long)n_txt, hp, wp);
  if (n_ref < 0 || n_ref > 3) return fail(DIT_E_SHAPE, "n_ref %d out of range [0, 3]", n_ref);
  if (n_ref > 0 && (!ref_hp || !ref_wp)) return fail(DIT_E_NULL, "reference grids are NULL");
  int64_t S = n_txt + (int64_t)hp * wp;
  for (int i = 0; i < n_ref; ++i) {
    if (ref_hp[i] < 0 || ref_wp[i] < 0)
      return fail(DIT_E_SHAPE, "reference %d grid %d x %d is negative", i, ref_hp[i], ref_wp[i]);
    S += (int64_t)ref_hp[i] * ref_wp[i];
  }
  if (S > cap_rows) return fail(DIT_E_SHAPE, "%lld rows exceed capacity %lld", (long long)S,
                                (long long)cap_rows);
  if (S > 0 && !out) return fail(DIT_E_NULL, "out is NULL");
  int64_t r = 0;
  auto put = [&](int t, int h, int w, int l) {
    out[4 * r + 0] = t;
    out[4 * r + 1] = h;
    out[4 * r + 2] = w;
    out[4 * r + 3] = l;
    ++r;
  };
  for (int64_t l = 0; l < n_txt; ++l) put(0, 0, 0, (int)l);
  for (int i = 0; i < hp; ++i)
    for (int j = 0; j < wp; ++j) put(0, i, j, 0);
  for (int k = 0; k < n_ref; ++k)
    for (int i = 0; i < ref_hp[k]; ++i)
      for (int j = 0; j < ref_wp[k]; ++j) put(10 + 10 * k, i, j, 0);
  return S;
}

size_t dit_workspace_bytes(const dit_config* cfg, int32_t kind, int32_t B, int64_t S) {
  if (check_config(cfg) != DIT_OK) return 0;
  if (kind == DIT_WS_MOD) {
    if (B < 1 || B > DIT_MAX_BATCH) {
      fail(DIT_E_SHAPE, "B %d out of range", B);
      return 0;
    }
    return mod_layout(*cfg, B).total;
  }
  if (check_batch_seq(B, S) != DIT_OK) return 0;
  switch (kind) {
    case DIT_WS_DUAL: return block_layout(*cfg, 0, B, S).total;
    case DIT_WS_SINGLE: return block_layout(*cfg, 1, B, S).total;
    case DIT_WS_STEP: return step_layout(*cfg, B, S).total;
    case DIT_WS_DENOISE: return denoise_layout(*cfg, B, S).total;
    default: fail(DIT_E_VALUE, "unknown workspace kind %d", kind); return 0;
  }
}


int dit_vae_config_check(const dit_vae_config* cfg) { return check_vae_config(cfg); }

void dit_vae_config_default(dit_vae_config* cfg) {
  if (!cfg) return;
  cfg->z_channels = 32;
  cfg->block_channels[0] = 128;
  cfg->block_channels[1] = 256;
  cfg->block_channels[2] = 512;
  cfg->block_channels[3] = 512;
  cfg->layers = 3;
  cfg->groups = 32;
  cfg->eps = 1e-6f;
}

size_t dit_vae_workspace_bytes(const dit_vae_config* cfg, int32_t B, int32_t hp, int32_t wp) {
  if (check_vae_config(cfg) != DIT_OK) return 0;
  if (B < 1 || B > DIT_MAX_BATCH || hp < 1 || wp < 1 || 16ll * hp > 32766 || 16ll * wp > 32767) {
    fail(DIT_E_SHAPE, "B %d, token grid %d x %d out of range", B, hp, wp);
    return 0;
  }
  return vae_layout(*cfg, B, hp, wp).total;
}

size_t dit_vae_group_norm_ws_bytes(int32_t B, int64_t HW, int32_t C, int32_t groups) {
  if (B < 1 || HW < 1 || C < 8 || C % 8 || C > 2048 || groups < 1 || C % groups) {
    fail(DIT_E_SHAPE, "B %d, HW %lld, C %d, groups %d out of range", B, (long long)HW, C, groups);
    return 0;
  }
  return vae_group_norm_ws(B, HW, C, groups);
}

}  // extern "C"
