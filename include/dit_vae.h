/* C ABI of the latent decoder in libdit.so: image tokens -> pixels on the
 * GPU, after the last denoise step.
 *
 * What the pages fix: the decoder runs on the card as decode(latents)
 * ("tt_flux2_klein - Python reference", Lower-level entry points; its time
 * is the vae_decode_s field of Timing), it is tt-metal's tt_dit VAE with a
 * GroupNorm grid fix and non-square slicing ("flux2-klein-p100a", What this
 * port adds: so it has GroupNorm layers and takes non-square images), and
 * the image post-processing stays on the host (the card's header). The
 * layer list below is a reading (the pages give no architecture): the
 * convolutional KL-autoencoder decoder of the latent-diffusion family.
 *
 *   u      = z * lat_scale + lat_shift           per token channel (4 Z)
 *   x      = unpatchify(u)   token (r, c), channel 4k + 2i + j ->
 *                            pixel (2r + i, 2c + j), channel k (k < Z)
 *   x      = conv_in(x)                           3x3, Z -> C_top
 *   x      = res(x); x = attn(x); x = res(x)      mid, C_top channels
 *   for level l = 0..3 (channels block_channels[3 - l]):
 *     x = res(x) (layers times; the first changes the channel count)
 *     if l < 3: x = upconv_l(upsample2x(x))      nearest 2x, then 3x3
 *   image  = conv_out(SiLU(GN_out(x)))            3x3 -> 3 channels
 *   res(x) = s(x) + conv2(SiLU(GN2(conv1(SiLU(GN1(x))))))
 *            s = identity, or a 1x1 conv when the channel count changes
 *   attn(x)= x + o(softmax(q k^T / sqrt(C)) v),  q, k, v, o 1x1 convs of
 *            GN(x) (one head of width C over all pixels of a sample)
 * Convolutions are cross-correlations, stride 1, zero padding 1 for 3x3,
 * each with a bias. GroupNorm: `groups` runs of consecutive channels, mean
 * and biased variance over a sample's pixels and the group's channels, eps
 * inside the root, per-channel gamma, beta.
 *
 * Numerics: bf16 weights and stored activations, fp32 accumulation, fp32
 * GroupNorm statistics (combined in double) and softmax; every launch's
 * result for a batch row is independent of the other rows, bit for bit.
 *
 * Layouts: activations channels-last; conv weights bf16 [C_out][kh][kw][C_in]
 * (K index (ky kw + kx) C_in + c contiguous per output channel); biases,
 * GroupNorm gamma / beta and the latent affine fp32. All pointers are device
 * pointers, 16-byte aligned; the library never frees or keeps them. */
#ifndef DIT_VAE_H
#define DIT_VAE_H

#include "dit.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dit_vae_config {
  int32_t z_channels;         /* Z: 32 (the 128 token channels are 2x2 x Z) */
  int32_t block_channels[4];  /* encoder order: 128, 256, 512, 512 */
  int32_t layers;             /* ResNet blocks per up level: 3 */
  int32_t groups;             /* GroupNorm groups: 32 */
  float eps;                  /* GroupNorm eps: 1e-6 */
} dit_vae_config;

enum { DIT_VAE_MAX_LAYERS = 4, DIT_VAE_OUT_CHANNELS = 3 };

/* One ResNet block (c_in -> c_out). short_w / short_b: the 1x1 shortcut
 * [c_out][1][1][c_in], present exactly when c_in != c_out (NULL otherwise). */
typedef struct dit_vae_resnet {
  const float* gn1_gamma;  /* [c_in] */
  const float* gn1_beta;
  const void* conv1_w;     /* bf16 [c_out][3][3][c_in] */
  const float* conv1_b;    /* [c_out] */
  const float* gn2_gamma;  /* [c_out] */
  const float* gn2_beta;
  const void* conv2_w;     /* bf16 [c_out][3][3][c_out] */
  const float* conv2_b;
  const void* short_w;
  const float* short_b;
} dit_vae_resnet;

typedef struct dit_vae_weights {
  const float* lat_scale;        /* [4 Z] */
  const float* lat_shift;        /* [4 Z] */
  const void* conv_in_w;         /* bf16 [C_top][3][3][Z] */
  const float* conv_in_b;
  dit_vae_resnet mid[2];
  const float* attn_gn_gamma;    /* [C_top] */
  const float* attn_gn_beta;
  const void* attn_w[4];         /* q, k, v, o: bf16 [C_top][1][1][C_top] */
  const float* attn_b[4];
  dit_vae_resnet up[4][DIT_VAE_MAX_LAYERS];  /* [level][block], blocks < layers */
  const void* upconv_w[3];       /* level l < 3: bf16 [C_l][3][3][C_l] */
  const float* upconv_b[3];
  const float* norm_out_gamma;   /* [block_channels[0]] */
  const float* norm_out_beta;
  const void* conv_out_w;        /* bf16 [3][3][3][block_channels[0]] */
  const float* conv_out_b;       /* [3] */
} dit_vae_weights;

/* Validates a decoder configuration (DIT_OK, or DIT_E_NULL / DIT_E_SHAPE /
 * DIT_E_UNSUPPORTED / DIT_E_VALUE with dit_last_error set): 8 <= z_channels <= 256, z_channels % 8 == 0; every
 * block width a power of two in [32, 2048] and a multiple of `groups`;
 * 1 <= groups <= 1024; 1 <= layers <= DIT_VAE_MAX_LAYERS; eps > 0 and
 * finite. */
int dit_vae_config_check(const dit_vae_config* cfg);

/* Reading defaults: z 32, widths 128/256/512/512, 3 layers, 32 groups,
 * eps 1e-6. */
void dit_vae_config_default(dit_vae_config* cfg);

/* Bytes of device workspace dit_vae_decode_forward needs for B samples of
 * an hp x wp token grid (image 16 hp x 16 wp pixels); 0 on invalid
 * arguments, with dit_last_error set. */
size_t dit_vae_workspace_bytes(const dit_vae_config* cfg, int32_t B, int32_t hp, int32_t wp);

/* The decoder (layer list above) for B samples.
 *   z:     dev fp32 [B][hp * wp][4 Z], the sampler's image tokens (the
 *          denoise loop's z), row-major over the token grid;
 *   image: dev fp32 [B][16 hp][16 wp][3], written (unclamped);
 *   ws:    dit_vae_workspace_bytes(cfg, B, hp, wp) bytes, 256-byte aligned.
 * 1 <= B <= DIT_MAX_BATCH; hp, wp >= 1 with every stored activation of one
 * sample under 2^31 bytes (images up to about 2048 x 2000 at the default
 * widths). Work is enqueued on `stream`; the call returns without waiting.
 * Errors: DIT_E_NULL (a required pointer, a weight or a missing / extra
 * shortcut), DIT_E_SHAPE (sizes, 16-byte alignment), DIT_E_UNSUPPORTED /
 * DIT_E_VALUE (configuration), DIT_E_WORKSPACE, all before any launch
 * (device memory untouched); DIT_E_HIP from a launch. */
int dit_vae_decode_forward(const dit_vae_config* cfg, const dit_vae_weights* w, const float* z,
                           int32_t B, int32_t hp, int32_t wp, float* image, void* ws,
                           size_t ws_bytes, dit_stream_t stream);

/* Building block of the decoder, exported for tests of its layers: one
 * convolution (bias and residual fused) over B samples of an H x W grid.
 *   out[b, y, x, n] = bias[n] + short_b[n] + resid[b, y, x, n]
 *                     + sum_{ky, kx, c} xin[b, y + ky - 1, x + kx - 1, c] w[n, ky, kx, c]
 *                     + sum_c xs[b, y, x, c] short_w[n, 0, 0, c]
 *   ksize 3 (zero padding 1) or 1; up = 1: xin is at (H / 2, W / 2) and is
 *   read through a nearest 2x upsample (H, W even); xs / short_w / short_b
 *   (a 1x1 second source, c_short channels at the output grid) and resid
 *   (bf16 [B][H][W][c_out]) may be NULL; out bf16 [B][H][W][c_out], or fp32
 *   when out_f32. c_in, c_short multiples of 8. No workspace. */
int dit_vae_conv_forward(const void* xin, int32_t c_in, int32_t ksize, int32_t up,
                         const void* w, const float* bias, const void* xs, int32_t c_short,
                         const void* short_w, const float* short_b, const void* resid,
                         int32_t B, int32_t H, int32_t W, int32_t c_out, void* out,
                         int32_t out_f32, dit_stream_t stream);

/* Building block: y = act(GroupNorm(x)), act = SiLU when silu != 0,
 * x, y bf16 [B][HW][C] (may not alias), gamma / beta fp32 [C].
 * ws: dit_vae_group_norm_ws_bytes(B, HW, C, groups) bytes. */
size_t dit_vae_group_norm_ws_bytes(int32_t B, int64_t HW, int32_t C, int32_t groups);
int dit_vae_group_norm_forward(const void* x, void* y, const float* gamma, const float* beta,
                               int32_t B, int64_t HW, int32_t C, int32_t groups, float eps,
                               int32_t silu, void* ws, size_t ws_bytes, dit_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DIT_VAE_H */
