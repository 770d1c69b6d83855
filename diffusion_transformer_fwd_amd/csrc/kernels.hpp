// Host-side launch interface of the gfx950 kernels (internal to libdit.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

typedef uint16_t bf16_t;

// ------------------------------------------------------------------ GEMM
// C = A W^T with A [M, K] bf16 (row stride lda) and W [N', K] bf16 (row
// stride ldw), fp32 accumulation on MFMA, and one of four epilogues.
// Output row r of a problem is written to row
//   (r / seg_len) * seg_stride + seg_off + (r % seg_len)
// of C, which lets one launch scatter stream-major rows back to the token
// order of x[B, S, D] without copies.
enum Epilogue : int32_t {
  EPI_BF16 = 0,    // C bf16 [., ldc]:  C[row, n] = acc
  EPI_SWIGLU = 1,  // C bf16: C[row, n] = SiLU(acc_gate) * acc_up; W rows
                   //   [0, N) are gate rows and [N, 2N) are up rows
  EPI_RESID = 2,   // C fp32: C[row, n] += gate[b * gate_bstride + n] * acc,
                   //   b = r / seg_len
  EPI_F32 = 3,     // C fp32: C[row, n] = acc
  EPI_QKV = 4      // QK-RMSNorm + RoPE into the attention operands (C unused):
                   //   N = 3D columns q | k | v, head h = columns 128h..128h+127
                   //   of each third; row r is token s = seg_off + r % seg_len
                   //   of batch row b = r / seg_len. q, k: per head vector
                   //   x / sqrt(mean(x^2) + eps) * gain, rotated by the token's
                   //   (cos, sin) per adjacent pair, q also times q_scale,
                   //   stored bf16 at [b, h, s, :]; v stored bf16 at v^T[b, h, :, s]
};

struct GemmProblem {
  const bf16_t* A;
  const bf16_t* W;
  void* C;
  const float* gate;
  int64_t lda, ldw, ldc, gate_bstride, seg_stride;
  int32_t M, N, K, epi;
  int32_t seg_len, seg_off;
  // set by gemm_launch: tile height 128 fm rows (fm = 2 or 3), tile counts,
  // and the problem's first tile in launch order
  int32_t tiles_m, tiles_n, tile_begin, fm;
};

constexpr int kMaxGemmProblems = 8;

// Operands of the EPI_QKV epilogue, shared by the problems of a launch; the
// QK gains are per problem (text and image streams differ).
struct QkvEpilogue {
  bf16_t* q;             // [B, H, S_pad, 128]
  bf16_t* k;             // [B, H, S_pad, 128]
  bf16_t* vt;            // [B, H, 128, S_pad]
  const float* cos_t;    // [S, 64]
  const float* sin_t;
  const float* q_gain[kMaxGemmProblems];  // [128] each
  const float* k_gain[kMaxGemmProblems];
  int64_t S_pad;
  int32_t H, D;
  float eps, q_scale;    // q_scale = log2(e) / sqrt(head_dim)
};

struct GemmBatch {
  GemmProblem p[kMaxGemmProblems];
  int32_t count;
  int32_t total_tiles;
  QkvEpilogue qkv;
};

// Requirements checked by the caller: K % 64 == 0, N % 32 == 0 (EPI_QKV: N = 3D,
// D % 128 == 0),
// lda/ldw % 8 == 0, 16-byte aligned A and W; ldc % 4 == 0.
constexpr int kGemmBN = 256, kGemmBK = 64;

// The problems of one launch are all of the fp32 family (EPI_F32 /
// EPI_RESID) or all of the bf16 family (the others).
// Picks the tile shapes (rows per problem, width per launch), fills
// fm/tiles_m/tiles_n/tile_begin/total_tiles and launches. May reorder the
// problems of its copy of the batch (with their QK gains); the caller's
// batch keeps its order.
hipError_t gemm_launch(GemmBatch& batch, hipStream_t stream);

// ------------------------------------------------------------------ norms
// h[out_base + r] = N(x[row(r)]) * (1 + scale[b]) + shift[b] (bf16), for up
// to two row segments; row(r) = b * S + seg_off + r % seg_len, b = r / seg_len.
struct NormSegment {
  const float* shift;  // + b * mod_bstride
  const float* scale;
  int64_t out_base;    // first output row
  int32_t seg_off, seg_len;
};
struct NormArgs {
  const float* x;
  bf16_t* h;
  int64_t S, mod_bstride;
  int32_t D, B, kind, nseg;
  float eps;
  NormSegment seg[2];
};
hipError_t modnorm_launch(const NormArgs& a, hipStream_t stream);

// ------------------------------------------------------------------ padding
// Zeroes rows s in [S, S_pad) of q and k [B, H, S_pad, 128] and columns
// [S, S_pad) of v^T [B, H, 128, S_pad]: the attention kernel reads whole
// 64-key tiles, and a padded V column must be finite (its probability is 0).
struct QkvPadArgs {
  bf16_t* q;
  bf16_t* k;
  bf16_t* vt;
  int64_t S, S_pad;
  int32_t B, H;
};
hipError_t qkv_pad_launch(const QkvPadArgs& a, hipStream_t stream);

// ------------------------------------------------------------------ split-K sum
// c[row(r), n] += p[0][r, n], then += p[1][r, n], ... (np partials in that
// order, np <= 7), row(r) = (r / seg_len) * seg_stride + seg_off + r % seg_len: the
// end of a GEMM whose K range ran as np + 1 chunk problems of one launch,
// chunk 0 writing c and chunk k + 1 writing p[k] [rows, ldp]. cols % 4 == 0.
struct SplitSumArgs {
  float* c;
  const float* p[7];
  int64_t ldc, ldp, seg_stride;
  int32_t rows, cols, np, seg_len, seg_off;
};
hipError_t split_sum_launch(const SplitSumArgs& a, hipStream_t stream);

// ------------------------------------------------------------------ attention
// O = softmax(q k^T / sqrt(128)) v for every (b, h), no mask, over S keys.
// q (pre-scaled by log2(e) / sqrt(128)), k [B, H, S_pad, 128], vt [B, H, 128,
// S_pad] (zero beyond S). The output row of token (b, s) is
//   stream_major ? (s < n_txt ? b*n_txt + s : B*n_txt + b*(S-n_txt) + s-n_txt)
//                : b*S + s,
// written at o + row * ldo + h * 128.
struct AttnArgs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* vt;
  bf16_t* o;
  int64_t S, S_pad, ldo, n_txt;
  int32_t B, H, stream_major;
};
hipError_t attention_launch(const AttnArgs& a, hipStream_t stream);

// Attention fused with a bf16-family GEMM batch that does not depend on it
// (one launch: the attention's work-groups first, then the GEMM tiles, which
// fill the CUs of the attention's last round). An empty batch is a plain
// attention launch.
hipError_t attn_gemm_launch(const AttnArgs& a, GemmBatch& batch, hipStream_t stream);

// For a GEMM launch of {first, rows [0, m) of rest} followed by a fused
// launch of {attention a, rows [m, rest.M) of rest}: the m (a multiple of
// row_step, or rest.M) that minimises the modelled time of the two launches.
int64_t fused_split_rows(const GemmProblem& first, const GemmProblem& rest, int64_t row_step,
                         const AttnArgs& a);

// ------------------------------------------------------------------ small ops
// RoPE tables from int32 positions [S, 4]: omega[a][j] given in double.
struct RopeArgs {
  const int32_t* pos;
  float* cos_t;
  float* sin_t;
  int64_t S;
  int32_t pairs;          // head_dim / 2
  int32_t axis_of[64];    // pair -> axis
  double omega[64];       // pair -> frequency
};
hipError_t rope_tables_launch(const RopeArgs& a, hipStream_t stream);

// Sinusoidal timestep features e[B, C] (fp32) from per-row sigma.
struct TimeArgs {
  float* e;
  int32_t B, C;
  float sigma[64];
};
hipError_t time_features_launch(const TimeArgs& a, hipStream_t stream);

// y[b, out_off_s + n] = act_out(sum_k W_s[n, k] act_in(x[b, k])), fp32 out,
// for up to four weight segments sharing one input x [B, K] (fp32).
enum Act : int32_t { ACT_NONE = 0, ACT_SILU = 1 };
struct GemvSegment {
  const bf16_t* W;   // [rows, K]
  int64_t out_off;   // first output column in y
  int32_t rows, row_begin;  // row_begin: first global row of this segment
};
struct GemvArgs {
  const float* x;    // [B, K]
  float* y;          // [B, ldy]
  int64_t ldy;
  int32_t B, K, act_in, act_out, nseg, total_rows;
  GemvSegment seg[4];
};
hipError_t gemv_launch(const GemvArgs& a, hipStream_t stream);

// ------------------------------------------------------------------ sampler loop
// Latent state of the on-device sampling loop: z fp32 [B, n_img, C] (image
// tokens), the step's bf16 operand lat [B, n_img + n_ref, C] (image rows, then
// the reference rows copied from ref [B, n_ref, C]), and the step's velocity
// v fp32 [B, n_img, C]. C % 4 == 0.
//   latent_pack: lat[b, r] = bf16(z[b, r]) for r < n_img, ref rows copied.
//   euler:       z[b, r] += dsig[b] * v[b, r]; lat[b, r] = bf16(z[b, r]).
struct LatentArgs {
  float* z;
  const float* v;
  const bf16_t* ref;
  bf16_t* lat;
  int64_t n_img, n_ref;
  int32_t B, C;
  float dsig[64];
};
hipError_t latent_pack_launch(const LatentArgs& a, hipStream_t stream);

// dst[b * dst_bstride + r, :] = src[b * src_bstride + r, :] for rows r < n of
// each of B batch rows (fp32, D % 4 == 0): the embedded text rows kept
// across the steps of the sampling loop.
struct RowsCopyArgs {
  const float* src;
  float* dst;
  int64_t n, src_bstride, dst_bstride;  // strides in rows
  int32_t B, D;
};
hipError_t rows_copy_launch(const RowsCopyArgs& a, hipStream_t stream);
hipError_t euler_launch(const LatentArgs& a, hipStream_t stream);

// ------------------------------------------------------------------ latent decoder
// Implicit-GEMM convolution, channels last: out[b, m, n] for output pixel m
// of an H x W grid (row-major) and channel n,
//   sum over sources s, K index k < taps_s C_s (k = tap C_s + c) of
//   A_s[b, pixel(m, tap), c] W_s[b][n, k]
// plus bias, a second bias and a bf16 residual, stored bf16 or fp32. A 3x3
// tap (dy, dx) = (tap / 3 - 1, tap % 3 - 1) reads pixel (y + dy, x + dx),
// zero outside the grid; with `up` the source grid is (H / 2, W / 2) and
// the pixel read is ((y + dy) / 2, (x + dx) / 2) (nearest 2x upsampling
// before the conv). A plain GEMM is the 1 x M grid with taps = 1.
struct ConvSource {
  const bf16_t* x;      // [B][pixels][lda] (sample stride x_bs elements)
  const bf16_t* w;      // [N][ldw] (sample stride w_bs; 0 = shared weights)
  int64_t x_bs, w_bs;
  uint32_t x_bytes, w_bytes;  // bytes of one sample's A / of W (< 2^31)
  int32_t lda, ldw, C, taps, up;
  int32_t slices;       // ceil(taps C / 64), set by conv_launch
  float inv_c;          // 1 / C, set by conv_launch
};
struct ConvArgs {
  ConvSource src[2];
  void* out;            // [B][M][ldo], bf16 or fp32
  const float* bias;    // [N] (or [M] with bias_rows), may be null
  const float* bias2;   // [N], may be null
  const bf16_t* resid;  // [B][M][ldr] bf16, may be null; may alias out
  int64_t out_bs, resid_bs;
  // GroupNorm folded into the input of the halo kernel (source 0 only):
  // when gn_ab is set, source 0 is read as act(x a_c + s_c) rounded to bf16
  // (act = SiLU when gn_silu), zero padding kept zero; gn_ab [B][C][2]
  // holds (a_c, s_c) per sample and channel. Only the halo kernel takes it.
  const float* gn_ab;
  int32_t gn_silu;
  int32_t nsrc, B, H, W, N, ldo, ldr, out_f32, bias_rows;
  int32_t vec;          // 16-byte epilogue stores allowed (set by conv_launch)
  int32_t tiles_m, tiles_n, tiles_x, cfg;  // set by conv_launch
};
// Checks the shapes the kernel assumes (returns hipErrorInvalidValue on a
// violation), picks the tile shape and launches.
hipError_t conv_launch(ConvArgs& a, hipStream_t stream);
// Whether conv_launch will run a's convolution on the halo-tiled kernel.
bool conv_uses_halo(const ConvArgs& a);

// GroupNorm (+ optional SiLU), channels last, per sample over H * W pixels:
// statistics from per-block partial sums around a per-group shift (the
// group's first value), combined in double in a fixed order; then
// y = act(x * a_c + s_c) with a_c = gamma_c rstd, s_c = beta_c - mean a_c.
struct GroupNormArgs {
  const bf16_t* x;
  bf16_t* y;
  float* part;          // [B][nblk][G][2] partial sums (workspace)
  float* ab;            // [B][C][2] per-channel scale / shift (workspace)
  const float* gamma;
  const float* beta;
  int64_t x_bs, y_bs;   // sample strides (elements)
  int32_t B, HW, C, G, ppb, nblk, silu;
  int32_t apply;        // 0: statistics and scale / shift only (y unused)
  float eps;
};
// ppb / nblk: pixels per statistics block (a multiple of 256 / (C / 8)) and
// the block count per sample, ppb nblk >= HW.
hipError_t group_norm_launch(const GroupNormArgs& a, hipStream_t stream);

// Row softmax: p[r, j] = bf16(exp(c s[r, j] - max) / sum), c = scale,
// j < n (n % 4 == 0), rows of s fp32 (stride lds), p bf16 (stride ldp).
struct SoftmaxArgs {
  const float* s;
  bf16_t* p;
  int64_t lds, ldp;
  int32_t rows, n;
  float scale;
};
hipError_t softmax_rows_launch(const SoftmaxArgs& a, hipStream_t stream);

// Latent tokens z fp32 [B][hp * wp][4 Z] -> image x bf16 [B][2hp][2wp][Z]:
// u = z * scale[c] + shift[c] per token channel c = 4k + 2i + j, written to
// pixel (2r + i, 2c + j) channel k of token (r, c).
struct LatentImageArgs {
  const float* z;
  const float* scale;
  const float* shift;
  bf16_t* x;
  int32_t B, hp, wp, Z;
};
hipError_t latent_image_launch(const LatentImageArgs& a, hipStream_t stream);

}  // namespace dit
