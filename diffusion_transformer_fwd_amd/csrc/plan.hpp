// Host-side planning and argument checks of libdit.so: workspace layouts,
// validation of every entry point's arguments (all of it runs before the
// first launch, so an error leaves device memory untouched), the thread-local
// error message, and the host-only entry points (position ids, workspace
// sizes, status strings). Plain C++ with no HIP dependency, so it also builds
// with a host compiler and its sanitizers.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/dit.h"
#include "../../include/dit_vae.h"

#define DIT_CHECK(status)                                                         \
  do {                                                                            \
    const int s_ = (status);                                                      \
    if (s_ != DIT_OK) return s_;                                                  \
  } while (0)

namespace dit {
namespace host {

constexpr size_t kAlign = 256;
constexpr uint64_t kMaxBufferBytes = 0xFFFFFFFFull;  // 32-bit buffer offsets

// Records a printf-style message as the thread's last error; returns status.
int fail(int status, const char* fmt, ...);
// The calling thread's last message.
const char* last_error_message();

size_t align_up(size_t v);
int64_t round_up(int64_t v, int64_t m);
bool aligned(const void* p, size_t a);

// Workspace regions (byte offsets, each 256-byte aligned) of one block call,
// kind 0 = dual, 1 = single.
struct BlockLayout {
  int64_t R = 0, S_pad = 0;
  int64_t u_cols = 0;
  size_t h = 0, u = 0, d6 = 0, o = 0, q = 0, k = 0, vt = 0, total = 0;
};
BlockLayout block_layout(const dit_config& c, int kind, int64_t B, int64_t S);

// The modulation's intermediate vectors.
struct ModLayout {
  size_t e = 0, t1 = 0, m = 0, total = 0;
};
ModLayout mod_layout(const dit_config& c, int64_t B);

// One step: residual, modulation result, the modulation's and a block's
// workspace.
struct StepLayout {
  size_t x = 0, mod = 0, modws = 0, block = 0, total = 0;
};
StepLayout step_layout(const dit_config& c, int64_t B, int64_t S);

// Steps whose modulation vectors one pass over the modulation weights
// computes in the sampling loop.
constexpr int kModSteps = 4;

// The sampling loop: a step's workspace, the latent operand and velocity, the
// modulation of kModSteps steps and the embedded text rows.
struct DenoiseLayout {
  size_t step = 0, lat = 0, v = 0, mods = 0, modws = 0, txt = 0, total = 0;
};
DenoiseLayout denoise_layout(const dit_config& c, int64_t B, int64_t S);

// K chunks of a GEMM that runs K-split (depends on N and K only).
int split_k_chunks(int64_t N, int64_t K);

// Checks shared by the entry points.
int check_config(const dit_config* c);
int check_batch_seq(int32_t B, int64_t S);
int check_ws(const void* ws, size_t have, size_t need);
int check_ptr(const void* p, const char* what, size_t align = 16);
int check_operand_sizes(const dit_config& c, int64_t rows);
int check_dual_weights(const dit_dual_weights* w);
int check_single_weights(const dit_single_weights* w);
int check_model_weights(const dit_config& c, const dit_model_weights* w, bool blocks);
int check_sigmas(const float* sigma, int32_t B);
int check_block_common(const dit_config* cfg, float* x, int32_t B, int64_t S,
                       int64_t mod_batch_stride, const float* cos_t, const float* sin_t);
int check_step_args(const dit_config* cfg, const dit_model_weights* w, const void* txt,
                    int32_t B, int64_t n_txt, int64_t n_img, int64_t n_ref,
                    const float* cos_dev, const float* sin_dev);

// All argument checks of each device entry point, in the order the entry
// point runs them; DIT_OK means the call may launch. ws_bytes / ws of the
// no-allocation modulation are ignored there (noalloc = true checks the
// fixed scratch capacity instead).
int validate_rope(const dit_config* cfg, const int32_t* pos_dev, int64_t S, const float* cos_dev,
                  const float* sin_dev);
int validate_modulation(const dit_config* cfg, const dit_model_weights* w,
                        const float* sigma_host, int32_t B, const float* mod_dev, const void* ws,
                        size_t ws_bytes, bool noalloc);
int validate_dual(const dit_config* cfg, const dit_dual_weights* w, float* x, int32_t B,
                  int64_t S, int64_t n_txt, const float* mod_txt, const float* mod_img,
                  int64_t mod_batch_stride, const float* cos_dev, const float* sin_dev,
                  const void* ws, size_t ws_bytes);
int validate_single(const dit_config* cfg, const dit_single_weights* w, float* x, int32_t B,
                    int64_t S, const float* mod, int64_t mod_batch_stride, const float* cos_dev,
                    const float* sin_dev, const void* ws, size_t ws_bytes);
int validate_step(const dit_config* cfg, const dit_model_weights* w, const void* txt,
                  const void* latents, const float* sigma_host, int32_t B, int64_t n_txt,
                  int64_t n_img, int64_t n_ref, const float* cos_dev, const float* sin_dev,
                  const float* v_out, const void* ws, size_t ws_bytes);
int validate_linear(const void* a, const void* w, const float* y, int64_t M, int32_t N,
                    int32_t K);
int validate_denoise(const dit_config* cfg, const dit_model_weights* w, const void* txt,
                     const float* z, const void* ref, const float* sigmas_host, int32_t n_steps,
                     int32_t B, int64_t n_txt, int64_t n_img, int64_t n_ref,
                     const float* cos_dev, const float* sin_dev, const void* ws,
                     size_t ws_bytes);

// ---------------------------------------------------------------- decoder
// GroupNorm statistics blocks: pixels per block (a multiple of the pixels
// one pass of 256 threads covers, 256 / (C / 8)) and block count.
void gn_blocks(int64_t HW, int C, int* ppb, int* nblk);

// Decoder workspace: activation buffers p, q (stream), t (normalized), h
// (first conv of a ResNet), the unpatchified latent, GroupNorm partials and
// per-channel scale / shift, and the attention's scores (fp32) and
// probabilities (bf16) for mq query rows at a time, and v^T (bf16 [B][C][ld]).
struct VaeLayout {
  int64_t n0 = 0, ld = 0, mq = 0;     // attention: pixels, padded row, query rows per chunk
  int64_t act = 0, act_h = 0;        // elements per sample of p / q / t and of h
  int64_t gn_nblk = 0;               // largest GroupNorm block count
  size_t p = 0, q = 0, t = 0, h = 0, lat = 0, part = 0, ab = 0, s = 0, pm = 0, vt = 0,
         total = 0;
};
VaeLayout vae_layout(const dit_vae_config& c, int64_t B, int64_t hp, int64_t wp);
int check_vae_config(const dit_vae_config* c);
// channel width of decoder level l (0 = deepest) and the input width of
// ResNet r of level l
int vae_level_channels(const dit_vae_config& c, int l);
int vae_resnet_in(const dit_vae_config& c, int l, int r);
int validate_vae_decode(const dit_vae_config* cfg, const dit_vae_weights* w, const float* z,
                        int32_t B, int32_t hp, int32_t wp, const float* image, const void* ws,
                        size_t ws_bytes);
int validate_vae_conv(const void* xin, int32_t c_in, int32_t ksize, int32_t up, const void* w,
                      const float* bias, const void* xs, int32_t c_short, const void* short_w,
                      const float* short_b, const void* resid, int32_t B, int32_t H, int32_t W,
                      int32_t c_out, const void* out);
size_t vae_group_norm_ws(int64_t B, int64_t HW, int C, int groups);
int validate_vae_group_norm(const void* x, const void* y, const float* gamma, const float* beta,
                            int32_t B, int64_t HW, int32_t C, int32_t groups, float eps,
                            const void* ws, size_t ws_bytes);

}  // namespace host
}  // namespace dit
