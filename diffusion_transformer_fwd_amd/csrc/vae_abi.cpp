// C ABI of the latent decoder (include/dit_vae.h): the launch sequence of a
// decode and the exported building blocks. Argument checks and the
// workspace layout live in plan.cpp; every check runs before the first
// launch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <utility>

#include "../../include/dit_vae.h"
#include "kernels.hpp"
#include "plan.hpp"
#include "profile.hpp"

namespace {

using namespace dit::host;
using dit::bf16_t;
using dit::prof::timed;

#define VAE_TRY(expr)                                                             \
  do {                                                                            \
    const hipError_t e_ = (expr);                                                 \
    if (e_ != hipSuccess)                                                         \
      return fail(DIT_E_HIP, "%s: %s", #expr, hipGetErrorString(e_));             \
  } while (0)

const bf16_t* bf(const void* p) { return static_cast<const bf16_t*>(p); }

// A channels-last source on an image grid of pix_in pixels per sample,
// weights [N][taps][C].
dit::ConvSource image_src(const void* x, int C, int64_t pix_in, const void* w, int taps, int N,
                          int up) {
  dit::ConvSource s{};
  s.x = bf(x);
  s.w = bf(w);
  s.x_bs = pix_in * C;
  s.w_bs = 0;
  s.x_bytes = (uint32_t)(pix_in * C * 2);
  s.w_bytes = (uint32_t)((int64_t)N * taps * C * 2);
  s.lda = C;
  s.ldw = taps * C;
  s.C = C;
  s.taps = taps;
  s.up = up;
  return s;
}

struct Conv {
  dit::ConvArgs a{};
  double flops = 0.0, bytes = 0.0;
};

int run_conv(Conv& c, hipStream_t st) {
  const int kind = dit::conv_uses_halo(c.a) ? DIT_K_CONV_HALO : DIT_K_CONV;
  VAE_TRY(timed(kind, c.flops, c.bytes, st, [&] { return dit::conv_launch(c.a, st); }));
  return DIT_OK;
}

// out[B][H][W][N] = conv(x) (+ 1x1 conv of xs) + bias (+ bias2) (+ resid).
Conv image_conv(const void* x, int C, int taps, int up, const void* w, const float* bias,
                const void* xs, int Cs, const void* ws, const float* bias2, const void* resid,
                int B, int H, int W, int N, void* out, int out_f32) {
  Conv c;
  dit::ConvArgs& a = c.a;
  const int64_t pix = (int64_t)H * W, pix_in = up ? pix / 4 : pix;
  a.src[0] = image_src(x, C, pix_in, w, taps, N, up);
  a.nsrc = 1;
  if (xs) {
    a.src[1] = image_src(xs, Cs, pix, ws, 1, N, 0);
    a.nsrc = 2;
  }
  a.out = out;
  a.bias = bias;
  a.bias2 = bias2;
  a.resid = bf(resid);
  a.out_bs = pix * N;
  a.resid_bs = pix * N;
  a.B = B;
  a.H = H;
  a.W = W;
  a.N = N;
  a.ldo = N;
  a.ldr = N;
  a.out_f32 = out_f32;
  const double K = (double)taps * C + (xs ? Cs : 0);
  c.flops = 2.0 * B * pix * N * K;
  c.bytes = (double)B * (pix_in * C * 2.0 + (xs ? pix * Cs * 2.0 : 0.0) +
                         pix * N * (out_f32 ? 4.0 : 2.0) + (resid ? pix * N * 2.0 : 0.0)) +
            N * K * 2.0;
  return c;
}

int conv_image(const void* x, int C, int taps, int up, const void* w, const float* bias,
               const void* xs, int Cs, const void* ws, const float* bias2, const void* resid,
               int B, int H, int W, int N, void* out, int out_f32, hipStream_t st) {
  Conv c = image_conv(x, C, taps, up, w, bias, xs, Cs, ws, bias2, resid, B, H, W, N, out, out_f32);
  return run_conv(c, st);
}

// out[b][m][n] = sum_{k < K} A[b][m][k] W[b][n][k] (+ bias[n], or bias[m]
// with bias_rows) for m < M, n < N: the 1 x M grid of the conv kernel. W
// rows at or past w_rows read as zero.
int gemm_rows(const void* A, int64_t lda, int64_t a_bs, int64_t M, const void* Wt, int64_t ldw,
              int64_t w_bs, int64_t w_rows, int64_t N, int64_t K, int B, void* out, int64_t ldo,
              int64_t out_bs, int out_f32, const float* bias, int bias_rows, hipStream_t st) {
  Conv c;
  dit::ConvArgs& a = c.a;
  dit::ConvSource& s = a.src[0];
  s.x = bf(A);
  s.w = bf(Wt);
  s.x_bs = a_bs;
  s.w_bs = w_bs;
  s.x_bytes = (uint32_t)(M * lda * 2);
  s.w_bytes = (uint32_t)(w_rows * ldw * 2);
  s.lda = (int32_t)lda;
  s.ldw = (int32_t)ldw;
  s.C = (int32_t)K;
  s.taps = 1;
  s.up = 0;
  a.nsrc = 1;
  a.out = out;
  a.bias = bias;
  a.bias_rows = bias_rows;
  a.out_bs = out_bs;
  a.B = B;
  a.H = 1;
  a.W = (int32_t)M;
  a.N = (int32_t)N;
  a.ldo = (int32_t)ldo;
  a.ldr = (int32_t)ldo;
  a.out_f32 = out_f32;
  c.flops = 2.0 * B * M * N * K;
  c.bytes = (double)B * (M * K * 2.0 + (w_bs ? N * K * 2.0 : 0.0) +
                         M * N * (out_f32 ? 4.0 : 2.0)) +
            (w_bs ? 0.0 : N * K * 2.0);
  return run_conv(c, st);
}

// y = act(GroupNorm(x)); with y == nullptr only the statistics and the
// per-channel scale / shift (ab) are computed, for a conv that folds them in.
int group_norm(const void* x, void* y, const float* gamma, const float* beta, int B, int64_t HW,
               int C, int G, float eps, int silu, float* part, float* ab, hipStream_t st) {
  dit::GroupNormArgs a{};
  a.x = bf(x);
  a.y = static_cast<bf16_t*>(y);
  a.part = part;
  a.ab = ab;
  a.gamma = gamma;
  a.beta = beta;
  a.x_bs = HW * C;
  a.y_bs = HW * C;
  a.B = B;
  a.HW = (int32_t)HW;
  a.C = C;
  a.G = G;
  a.silu = silu;
  a.apply = y != nullptr;
  a.eps = eps;
  gn_blocks(HW, C, &a.ppb, &a.nblk);
  // statistics read x once, the normalization reads it again and writes y
  const double bytes = (double)B * HW * C * 2.0 * (a.apply ? 3.0 : 1.0);
  VAE_TRY(timed(DIT_K_GROUPNORM, 0.0, bytes, st, [&] { return dit::group_norm_launch(a, st); }));
  return DIT_OK;
}

int decode(const dit_vae_config& c, const dit_vae_weights& w, const float* z, int B, int hp,
           int wp, float* image, void* ws, hipStream_t st) {
  const VaeLayout L = vae_layout(c, B, hp, wp);
  char* const base = static_cast<char*>(ws);
  void* P = base + L.p;  // the block stream
  void* Q = base + L.q;  // the other stream buffer
  void* const T = base + L.t;
  void* const Hh = base + L.h;
  void* const lat = base + L.lat;
  float* const part = reinterpret_cast<float*>(base + L.part);
  float* const ab = reinterpret_cast<float*>(base + L.ab);
  float* const S = reinterpret_cast<float*>(base + L.s);
  bf16_t* const Pm = reinterpret_cast<bf16_t*>(base + L.pm);
  bf16_t* const Vt = reinterpret_cast<bf16_t*>(base + L.vt);
  const int G = c.groups, Z = c.z_channels, top = c.block_channels[3];
  const float eps = c.eps;
  int H = 2 * hp, W = 2 * wp;

  dit::LatentImageArgs la{z, w.lat_scale, w.lat_shift, static_cast<bf16_t*>(lat), B, hp, wp, Z};
  const double lat_bytes = (double)B * hp * wp * 4 * Z * (4.0 + 2.0);
  VAE_TRY(timed(DIT_K_LATENT_IMAGE, 0.0, lat_bytes, st,
                [&] { return dit::latent_image_launch(la, st); }));
  DIT_CHECK(conv_image(lat, Z, 9, 0, w.conv_in_w, w.conv_in_b, nullptr, 0, nullptr, nullptr,
                       nullptr, B, H, W, top, P, 0, st));

  // conv c over SiLU(GN(x)) (c's source 0 is x): on the halo kernel the
  // normalization is folded into the conv's input, otherwise it is written
  // to T first; both give the same bits
  auto norm_conv = [&](Conv& c, const void* x, int C, const float* gamma, const float* beta,
                       int64_t pix) -> int {
    c.a.src[0].x = bf(x);
    c.a.gn_ab = ab;
    c.a.gn_silu = 1;
    if (dit::conv_uses_halo(c.a)) {
      DIT_CHECK(group_norm(x, nullptr, gamma, beta, B, pix, C, G, eps, 1, part, ab, st));
      return run_conv(c, st);
    }
    c.a.src[0].x = bf(T);
    c.a.gn_ab = nullptr;
    DIT_CHECK(group_norm(x, T, gamma, beta, B, pix, C, G, eps, 1, part, ab, st));
    return run_conv(c, st);
  };

  // x (in P) <- s(x) + conv2(SiLU(GN2(conv1(SiLU(GN1(x))))))
  auto resnet = [&](const dit_vae_resnet& r, int ci, int co) -> int {
    const int64_t pix = (int64_t)H * W;
    Conv c1 = image_conv(P, ci, 9, 0, r.conv1_w, r.conv1_b, nullptr, 0, nullptr, nullptr, nullptr,
                         B, H, W, co, Hh, 0);
    DIT_CHECK(norm_conv(c1, P, ci, r.gn1_gamma, r.gn1_beta, pix));
    if (ci == co) {  // identity shortcut: added in the epilogue, in place
      Conv c2 = image_conv(Hh, co, 9, 0, r.conv2_w, r.conv2_b, nullptr, 0, nullptr, nullptr, P, B,
                           H, W, co, P, 0);
      return norm_conv(c2, Hh, co, r.gn2_gamma, r.gn2_beta, pix);
    }
    // 1x1 shortcut: a second K range of the same launch
    Conv c2 = image_conv(Hh, co, 9, 0, r.conv2_w, r.conv2_b, P, ci, r.short_w, r.short_b, nullptr,
                         B, H, W, co, Q, 0);
    DIT_CHECK(norm_conv(c2, Hh, co, r.gn2_gamma, r.gn2_beta, pix));
    std::swap(P, Q);
    return DIT_OK;
  };

  // x (in P) <- x + o(softmax(q k^T / sqrt(C)) v), q, k, v, o 1x1 convs of GN(x)
  auto attention = [&]() -> int {
    const int C = top;
    const int64_t n0 = (int64_t)H * W, ld = L.ld;
    DIT_CHECK(group_norm(P, T, w.attn_gn_gamma, w.attn_gn_beta, B, n0, C, G, eps, 0, part, ab,
                         st));
    DIT_CHECK(conv_image(T, C, 1, 0, w.attn_w[0], w.attn_b[0], nullptr, 0, nullptr, nullptr,
                         nullptr, B, H, W, C, Hh, 0, st));  // q
    DIT_CHECK(conv_image(T, C, 1, 0, w.attn_w[1], w.attn_b[1], nullptr, 0, nullptr, nullptr,
                         nullptr, B, H, W, C, Q, 0, st));   // k
    // v^T[b][c][j] = sum_i W_v[c][i] t[b][j][i] + b_v[c] for j < ld; columns
    // j >= n0 hold b_v (finite) and meet zero probabilities
    DIT_CHECK(gemm_rows(w.attn_w[2], C, 0, C, T, C, n0 * C, n0, ld, C, B, Vt, ld, (int64_t)C * ld,
                        0, w.attn_b[2], 1, st));
    const float scale = 1.0f / std::sqrt((float)C);
    for (int b = 0; b < B; ++b) {
      for (int64_t r0 = 0; r0 < n0; r0 += L.mq) {
        const int64_t mq = std::min<int64_t>(L.mq, n0 - r0);
        const bf16_t* q = bf(Hh) + ((int64_t)b * n0 + r0) * C;
        const bf16_t* k = bf(Q) + (int64_t)b * n0 * C;
        DIT_CHECK(gemm_rows(q, C, 0, mq, k, C, 0, n0, n0, C, 1, S, ld, 0, 1, nullptr, 0, st));
        dit::SoftmaxArgs sa{S, Pm, ld, ld, (int32_t)mq, (int32_t)n0, scale};
        VAE_TRY(timed(DIT_K_SOFTMAX, 0.0, (double)mq * n0 * 6.0, st,
                      [&] { return dit::softmax_rows_launch(sa, st); }));
        bf16_t* o = static_cast<bf16_t*>(T) + ((int64_t)b * n0 + r0) * C;
        DIT_CHECK(gemm_rows(Pm, ld, 0, mq, Vt + (int64_t)b * C * ld, ld, 0, C, C, ld, 1, o, C, 0,
                            0, nullptr, 0, st));
      }
    }
    return conv_image(T, C, 1, 0, w.attn_w[3], w.attn_b[3], nullptr, 0, nullptr, nullptr, P, B,
                      H, W, C, P, 0, st);
  };

  DIT_CHECK(resnet(w.mid[0], top, top));
  DIT_CHECK(attention());
  DIT_CHECK(resnet(w.mid[1], top, top));
  for (int l = 0; l < 4; ++l) {
    const int co = vae_level_channels(c, l);
    for (int r = 0; r < c.layers; ++r) DIT_CHECK(resnet(w.up[l][r], vae_resnet_in(c, l, r), co));
    if (l < 3) {  // nearest 2x, read through the conv's address map
      H *= 2;
      W *= 2;
      DIT_CHECK(conv_image(P, co, 9, 1, w.upconv_w[l], w.upconv_b[l], nullptr, 0, nullptr,
                           nullptr, nullptr, B, H, W, co, Q, 0, st));
      std::swap(P, Q);
    }
  }
  const int c0 = vae_level_channels(c, 3);
  Conv co = image_conv(P, c0, 9, 0, w.conv_out_w, w.conv_out_b, nullptr, 0, nullptr, nullptr,
                       nullptr, B, H, W, DIT_VAE_OUT_CHANNELS, image, 1);
  return norm_conv(co, P, c0, w.norm_out_gamma, w.norm_out_beta, (int64_t)H * W);
}

}  // namespace

extern "C" {

int dit_vae_decode_forward(const dit_vae_config* cfg, const dit_vae_weights* w, const float* z,
                           int32_t B, int32_t hp, int32_t wp, float* image, void* ws,
                           size_t ws_bytes, dit_stream_t stream) {
  DIT_CHECK(validate_vae_decode(cfg, w, z, B, hp, wp, image, ws, ws_bytes));
  return decode(*cfg, *w, z, B, hp, wp, image, ws, stream);
}

int dit_vae_conv_forward(const void* xin, int32_t c_in, int32_t ksize, int32_t up, const void* w,
                         const float* bias, const void* xs, int32_t c_short, const void* short_w,
                         const float* short_b, const void* resid, int32_t B, int32_t H, int32_t W,
                         int32_t c_out, void* out, int32_t out_f32, dit_stream_t stream) {
  DIT_CHECK(validate_vae_conv(xin, c_in, ksize, up, w, bias, xs, c_short, short_w, short_b, resid,
                              B, H, W, c_out, out));
  return conv_image(xin, c_in, ksize * ksize, up, w, bias, xs, c_short, short_w, short_b, resid,
                    B, H, W, c_out, out, out_f32 ? 1 : 0, stream);
}

int dit_vae_group_norm_forward(const void* x, void* y, const float* gamma, const float* beta,
                               int32_t B, int64_t HW, int32_t C, int32_t groups, float eps,
                               int32_t silu, void* ws, size_t ws_bytes, dit_stream_t stream) {
  DIT_CHECK(validate_vae_group_norm(x, y, gamma, beta, B, HW, C, groups, eps, ws, ws_bytes));
  int ppb, nblk;
  gn_blocks(HW, C, &ppb, &nblk);
  float* part = static_cast<float*>(ws);
  float* ab = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                       align_up((size_t)B * nblk * groups * 2 * 4));
  return group_norm(x, y, gamma, beta, B, HW, C, groups, eps, silu ? 1 : 0, part, ab, stream);
}

}  // extern "C"
