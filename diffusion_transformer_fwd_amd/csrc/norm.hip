// Bandwidth-bound kernels of the step on gfx950:
//   * modnorm: AdaLN pre-norm of the fp32 residual into a bf16 GEMM operand
//   * split_sum: the fixed-order sum of a K-split GEMM's partial results
//   * qkv_pad: zeros of the padded attention operand rows (QK-RMSNorm and
//     RoPE themselves run in the QKV GEMM's epilogue)
//   * rope_tables: cos/sin of every pair angle from integer positions
//   * time_features + gemv: the global modulation vectors from sigma
//   * latent_pack + euler: the latent state of the sampling loop between
//     steps (flow-matching Euler update, bf16 operand of the next step);
//     rows_copy: the embedded text rows the loop keeps across steps
//
// The maths each one follows is stated at its kernel; the pages it comes
// from are "flux2-klein-p100a" (Caveats: one modulation result per step for
// every block) and "tt_flux2_klein - Python reference" (Things that are easy
// to get wrong: RoPE of 32 dims per axis, theta 2000, adjacent pairs).
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace dit {
namespace {

// ------------------------------------------------------------------ modnorm
// One wavefront per output row, the row held in registers (VPL float4 per
// lane, D <= 256 * VPL): one read of x, one write of h, coalesced 16-byte /
// 8-byte accesses. h = N(x) * (1 + scale[b]) + shift[b] in bf16, with
// N = RMS: x / sqrt(mean(x^2) + eps), or LAYER: (x - mean) / sqrt(var + eps).
template <int VPL>
__global__ __launch_bounds__(256) void modnorm_kernel(const NormArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  // segment lookup: seg[1] (if any) starts after seg[0]'s output rows
  const int si = (a.nseg > 1 && row >= a.seg[1].out_base) ? 1 : 0;
  const NormSegment& sg = si ? a.seg[1] : a.seg[0];
  const int64_t r = row - sg.out_base;
  if (r < 0 || r >= (int64_t)a.B * sg.seg_len) return;
  const int b = (int)(r / sg.seg_len);
  const int64_t xrow = (int64_t)b * a.S + sg.seg_off + (r - (int64_t)b * sg.seg_len);
  const int D = a.D, D4 = D >> 2;
  const f32x4* xr = reinterpret_cast<const f32x4*>(a.x + xrow * D);
  f32x4 v[VPL];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int c = i * 64 + lane;
    v[i] = c < D4 ? xr[c] : f32x4{0.f, 0.f, 0.f, 0.f};
    s += v[i][0] + v[i][1] + v[i][2] + v[i][3];
  }
  float mean = 0.f;
  if (a.kind == 1) mean = wave_sum(s) / D;
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int c = i * 64 + lane;
    if (c < D4) {
      const f32x4 d = v[i] - mean;
      ss += d[0] * d[0] + d[1] * d[1] + d[2] * d[2] + d[3] * d[3];
    }
  }
  const float rstd = rsqrtf(wave_sum(ss) / D + a.eps);
  const f32x4* sh = reinterpret_cast<const f32x4*>(sg.shift + (int64_t)b * a.mod_bstride);
  const f32x4* sc = reinterpret_cast<const f32x4*>(sg.scale + (int64_t)b * a.mod_bstride);
  u32x2* out = reinterpret_cast<u32x2*>(a.h + row * D);
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int c = i * 64 + lane;
    if (c < D4) {
      const f32x4 y = (v[i] - mean) * rstd * (1.f + sc[c]) + sh[c];
      out[c] = pack_bf16x4(y);
    }
  }
}

// One workgroup (4 waves) per R consecutive output rows, VPT float4 per
// thread per row (D <= 1024 VPT). When the R rows belong to one segment and
// one batch row (every workgroup but those at a segment's or batch row's
// edge) the shift and scale vectors are read once for all R rows, and all
// loads are issued before the first reduction; otherwise the rows are done
// one at a time. The sums go through LDS, R at a time; each row's arithmetic
// and summation order are the same either way. Same arithmetic as
// modnorm_kernel, with the reductions in another order.
template <int VPT, int R>
__device__ __forceinline__ void modnorm_rows(const NormArgs& a, const int64_t (&xrow)[R],
                                             const int64_t (&orow)[R], const float* shift,
                                             const float* scale, float (*part)[4]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int D = a.D, D4 = D >> 2;
  const f32x4* sh = reinterpret_cast<const f32x4*>(shift);
  const f32x4* sc = reinterpret_cast<const f32x4*>(scale);
  f32x4 v[R][VPT], vs[VPT], vh[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int c = i * 256 + tid;
    const bool ok = c < D4;
#pragma unroll
    for (int k = 0; k < R; ++k)
      v[k][i] = ok ? reinterpret_cast<const f32x4*>(a.x + xrow[k] * D)[c] : f32x4{0.f, 0.f, 0.f, 0.f};
    vh[i] = ok ? sh[c] : f32x4{0.f, 0.f, 0.f, 0.f};
    vs[i] = ok ? sc[c] : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // R block sums at once: per wave, then the four waves' partials in a fixed order
  auto block_sums = [&](float (&t)[R]) {
#pragma unroll
    for (int k = 0; k < R; ++k) t[k] = wave_sum(t[k]);
    if (lane == 0) {
#pragma unroll
      for (int k = 0; k < R; ++k) part[k][wave] = t[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < R; ++k) t[k] = (part[k][0] + part[k][1]) + (part[k][2] + part[k][3]);
    __syncthreads();  // part is reused by the next sums
  };
  float mean[R], ss[R];
#pragma unroll
  for (int k = 0; k < R; ++k) mean[k] = 0.f;
  if (a.kind == 1) {
#pragma unroll
    for (int k = 0; k < R; ++k) {
      float s1 = 0.f;
#pragma unroll
      for (int i = 0; i < VPT; ++i) s1 += v[k][i][0] + v[k][i][1] + v[k][i][2] + v[k][i][3];
      mean[k] = s1;
    }
    block_sums(mean);
#pragma unroll
    for (int k = 0; k < R; ++k) mean[k] = mean[k] / D;
  }
#pragma unroll
  for (int k = 0; k < R; ++k) {
    ss[k] = 0.f;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      if (i * 256 + tid < D4) {
        const f32x4 d = v[k][i] - mean[k];
        ss[k] += d[0] * d[0] + d[1] * d[1] + d[2] * d[2] + d[3] * d[3];
      }
    }
  }
  block_sums(ss);
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const float rstd = rsqrtf(ss[k] / D + a.eps);
    u32x2* out = reinterpret_cast<u32x2*>(a.h + orow[k] * D);
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = i * 256 + tid;
      if (c < D4) out[c] = pack_bf16x4((v[k][i] - mean[k]) * rstd * (1.f + vs[i]) + vh[i]);
    }
  }
}

template <int VPT, int R>
__global__ __launch_bounds__(256) void modnorm_row_kernel(const NormArgs a, int64_t rows) {
  __shared__ float part[R][4];
  // segment, batch row and x row of each of the workgroup's output rows
  int si[R], bb[R];
  int64_t xrow[R], orow[R];
  bool ok[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int64_t row = (int64_t)blockIdx.x * R + k;
    orow[k] = row;
    si[k] = (a.nseg > 1 && row >= a.seg[1].out_base) ? 1 : 0;
    const NormSegment& sg = si[k] ? a.seg[1] : a.seg[0];
    const int64_t r = row - sg.out_base;
    ok[k] = row < rows && r >= 0 && r < (int64_t)a.B * sg.seg_len;
    bb[k] = ok[k] ? (int)(r / sg.seg_len) : 0;
    xrow[k] = ok[k] ? (int64_t)bb[k] * a.S + sg.seg_off + (r - (int64_t)bb[k] * sg.seg_len) : 0;
  }
  bool same = ok[0];
#pragma unroll
  for (int k = 1; k < R; ++k) same = same && ok[k] && si[k] == si[0] && bb[k] == bb[0];
  if (same) {  // uniform per workgroup
    const NormSegment& sg = si[0] ? a.seg[1] : a.seg[0];
    modnorm_rows<VPT, R>(a, xrow, orow, sg.shift + (int64_t)bb[0] * a.mod_bstride,
                         sg.scale + (int64_t)bb[0] * a.mod_bstride, part);
    return;
  }
#pragma unroll
  for (int k = 0; k < R; ++k) {
    if (!ok[k]) continue;  // uniform per workgroup
    const NormSegment& sg = si[k] ? a.seg[1] : a.seg[0];
    const int64_t x1[1] = {xrow[k]}, o1[1] = {orow[k]};
    modnorm_rows<VPT, 1>(a, x1, o1, sg.shift + (int64_t)bb[k] * a.mod_bstride,
                         sg.scale + (int64_t)bb[k] * a.mod_bstride, part);
  }
}

// ------------------------------------------------------------------ qkv padding
// Grid (B * H), 256 threads: zero q, k rows [S, S_pad) (128 bf16 each) and
// v^T columns [S, S_pad) of its 128 rows, with 2-byte stores (the pad is at
// most 255 tokens).
__global__ __launch_bounds__(256) void qkv_pad_kernel(const QkvPadArgs a) {
  const int64_t bh = blockIdx.x;
  const int64_t pad = a.S_pad - a.S;
  bf16_t* q = a.q + (bh * a.S_pad + a.S) * 128;
  bf16_t* k = a.k + (bh * a.S_pad + a.S) * 128;
  for (int64_t i = threadIdx.x; i < pad * 128; i += blockDim.x) {
    q[i] = 0;
    k[i] = 0;
  }
  bf16_t* vt = a.vt + bh * 128 * a.S_pad + a.S;
  for (int64_t i = threadIdx.x; i < pad * 128; i += blockDim.x) vt[(i / pad) * a.S_pad + i % pad] = 0;
}

// ------------------------------------------------------------------ split-K sum
// One thread per 4 columns of a row: c += p[0] + ... in a fixed order.
__global__ __launch_bounds__(256) void split_sum_kernel(const SplitSumArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int c4 = a.cols >> 2;
  if (i >= (int64_t)a.rows * c4) return;
  const int r = (int)(i / c4), q = (int)(i - (int64_t)r * c4);
  const int b = r / a.seg_len;
  const int64_t row = (int64_t)b * a.seg_stride + a.seg_off + (r - b * a.seg_len);
  f32x4* c = reinterpret_cast<f32x4*>(a.c + row * a.ldc) + q;
  f32x4 v = *c;
  for (int k = 0; k < a.np; ++k)
    v += *(reinterpret_cast<const f32x4*>(a.p[k] + (int64_t)r * a.ldp) + q);
  *c = v;
}

// ------------------------------------------------------------------ rope tables
// cos/sin[s, j] of pos[s, axis(j)] * omega[j], angle and cos/sin in double.
__global__ __launch_bounds__(256) void rope_tables_kernel(const RopeArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= a.S * a.pairs) return;
  const int64_t s = i / a.pairs;
  const int j = (int)(i - s * a.pairs);
  const double phi = (double)a.pos[s * 4 + a.axis_of[j]] * a.omega[j];
  double sv, cv;
  sincos(phi, &sv, &cv);
  a.cos_t[i] = (float)cv;
  a.sin_t[i] = (float)sv;
}

// ------------------------------------------------------------------ time features
// e[b] = [cos(tau f_k) | sin(tau f_k)], tau = 1000 sigma_b,
// f_k = exp(-ln(1e4) k / half); evaluated in double.
__global__ __launch_bounds__(256) void time_features_kernel(const TimeArgs a) {
  const int b = blockIdx.x;
  const int half = a.C / 2;
  const double tau = 1000.0 * (double)a.sigma[b];
  for (int k = threadIdx.x; k < half; k += 256) {
    const double f = exp(-log(10000.0) * (double)k / (double)half);
    double sv, cv;
    sincos(tau * f, &sv, &cv);
    a.e[(int64_t)b * a.C + k] = (float)cv;
    a.e[(int64_t)b * a.C + half + k] = (float)sv;
  }
}

// ------------------------------------------------------------------ gemv
// y[b, out_off + n] = act_out(sum_k W[n, k] act_in(x[b, k])) for B <= 4
// batch rows per launch. Workgroup = NW waves, one weight row per wave per
// iteration; the B input rows are staged in LDS (fp32, after act_in; B * K
// floats of dynamic LDS) and the weight row is streamed once with 16-byte
// loads: the kernel reads each weight byte exactly once. One input row
// leaves room for many 4-wave workgroups per CU; with four rows (48 KiB at
// K = 3072) only three would fit, so those launches share one LDS copy
// among 16 waves. An element's arithmetic does not depend on NW.
constexpr int kGemvMaxB = 4;
constexpr int kGemvMaxK = 4096;
template <int NW>
__global__ __launch_bounds__(64 * NW) void gemv_kernel(const GemvArgs a) {
  // x as [B][2][K / 8][4]: element k = 8 c + e of row b at ((2 b + e / 4) K/8 + c) 4 + e % 4,
  // so the lanes of a wave, which take consecutive chunks c, read consecutive
  // 16-byte words (a plain [B][K] layout has them 32 bytes apart, which
  // conflicts on the LDS banks)
  extern __shared__ __attribute__((aligned(16))) float xs_dyn[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K8 = a.K >> 3;
  for (int i = tid; i < a.B * a.K; i += 64 * NW) {
    const int b = i / a.K, k = i - b * a.K;
    const float v = a.x[(int64_t)b * a.K + k];
    const int c = k >> 3, e = k & 7;
    xs_dyn[((2 * b + (e >> 2)) * K8 + c) * 4 + (e & 3)] = a.act_in == ACT_SILU ? silu_f(v) : v;
  }
  __syncthreads();
  for (int row = blockIdx.x * NW + wave; row < a.total_rows; row += gridDim.x * NW) {
    int si = 0;
#pragma unroll
    for (int i = 1; i < 4; ++i)
      if (i < a.nseg && row >= a.seg[i].row_begin) si = i;
    const GemvSegment& sg = a.seg[si];
    const int n = row - sg.row_begin;
    const u32x4* w = reinterpret_cast<const u32x4*>(sg.W + (int64_t)n * a.K);
    float acc[kGemvMaxB] = {0.f, 0.f, 0.f, 0.f};
    // all of the lane's chunks of the row (K <= 4096: at most 8) in flight at once
    u32x4 raw[kGemvMaxK / 512];
#pragma unroll
    for (int t = 0; t < kGemvMaxK / 512; ++t) {
      const int c = lane + 64 * t;
      if (c < K8) raw[t] = w[c];
    }
#pragma unroll
    for (int t = 0; t < kGemvMaxK / 512; ++t) {
      const int c = lane + 64 * t;
      if (c >= K8) break;
      float wv[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        wv[2 * e] = bf16_to_f32(raw[t][e] & 0xFFFFu);
        wv[2 * e + 1] = bf16_to_f32(raw[t][e] >> 16);
      }
#pragma unroll
      for (int b = 0; b < kGemvMaxB; ++b) {
        if (b < a.B) {
          const f32x4 x0 = *reinterpret_cast<const f32x4*>(&xs_dyn[((2 * b) * K8 + c) * 4]);
          const f32x4 x1 = *reinterpret_cast<const f32x4*>(&xs_dyn[((2 * b + 1) * K8 + c) * 4]);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[b] += wv[e] * x0[e];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[b] += wv[4 + e] * x1[e];
        }
      }
    }
#pragma unroll
    for (int b = 0; b < kGemvMaxB; ++b) {
      if (b < a.B) {
        float v = wave_sum(acc[b]);
        if (lane == 0) {
          if (a.act_out == ACT_SILU) v = silu_f(v);
          a.y[(int64_t)b * a.ldy + sg.out_off + n] = v;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ sampler loop
// One thread per 4 channels of a latent row; 16-byte fp32 loads and 8-byte
// bf16 stores, rows of a batch sample contiguous.
__global__ __launch_bounds__(256) void latent_pack_kernel(const LatentArgs a) {
  const int c4 = a.C >> 2;
  const int64_t rows = a.n_img + a.n_ref;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.B * rows * c4) return;
  const int64_t br = i / c4;
  const int q = (int)(i - br * c4);
  const int64_t b = br / rows, r = br - b * rows;
  u32x2* out = reinterpret_cast<u32x2*>(a.lat + br * a.C) + q;
  if (r < a.n_img) {
    *out = pack_bf16x4(*(reinterpret_cast<const f32x4*>(a.z + (b * a.n_img + r) * a.C) + q));
  } else {
    *out = *(reinterpret_cast<const u32x2*>(a.ref + (b * a.n_ref + (r - a.n_img)) * a.C) + q);
  }
}

// z += dsig[b] * v (one fp32 fma per element), and the bf16 copy of the new
// z into the image rows of the next step's operand.
__global__ __launch_bounds__(256) void euler_kernel(const LatentArgs a) {
  const int c4 = a.C >> 2;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.B * a.n_img * c4) return;
  const int64_t br = i / c4;
  const int q = (int)(i - br * c4);
  const int64_t b = br / a.n_img, r = br - b * a.n_img;
  f32x4* zp = reinterpret_cast<f32x4*>(a.z + br * a.C) + q;
  const f32x4 v = *(reinterpret_cast<const f32x4*>(a.v + br * a.C) + q);
  const float d = a.dsig[b];
  f32x4 z = *zp;
#pragma unroll
  for (int e = 0; e < 4; ++e) z[e] = fmaf(d, v[e], z[e]);
  *zp = z;
  *(reinterpret_cast<u32x2*>(a.lat + (b * (a.n_img + a.n_ref) + r) * a.C) + q) = pack_bf16x4(z);
}

// One thread per 4 columns of a row.
__global__ __launch_bounds__(256) void rows_copy_kernel(const RowsCopyArgs a) {
  const int c4 = a.D >> 2;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.B * a.n * c4) return;
  const int64_t br = i / c4;
  const int q = (int)(i - br * c4);
  const int64_t b = br / a.n, r = br - b * a.n;
  *(reinterpret_cast<f32x4*>(a.dst + (b * a.dst_bstride + r) * a.D) + q) =
      *(reinterpret_cast<const f32x4*>(a.src + (b * a.src_bstride + r) * a.D) + q);
}

}  // namespace

hipError_t modnorm_launch(const NormArgs& a, hipStream_t stream) {
  int64_t rows = 0;
  for (int i = 0; i < a.nseg; ++i)
    rows = max(rows, a.seg[i].out_base + (int64_t)a.B * a.seg[i].seg_len);
  if (rows == 0) return hipSuccess;
  const int vpt = (a.D / 4 + 255) / 256;
  if (vpt >= 2 && vpt <= 4) {  // wide rows: one workgroup per 3 rows
    constexpr int R = 3;
    const dim3 rgrid((unsigned)((rows + R - 1) / R));
    if (vpt == 2) hipLaunchKernelGGL((modnorm_row_kernel<2, R>), rgrid, dim3(256), 0, stream, a, rows);
    else if (vpt == 3) hipLaunchKernelGGL((modnorm_row_kernel<3, R>), rgrid, dim3(256), 0, stream, a, rows);
    else hipLaunchKernelGGL((modnorm_row_kernel<4, R>), rgrid, dim3(256), 0, stream, a, rows);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((rows + 3) / 4));
  const int vpl = (a.D / 4 + 63) / 64;
  if (vpl <= 1) hipLaunchKernelGGL(modnorm_kernel<1>, grid, dim3(256), 0, stream, a);
  else if (vpl <= 2) hipLaunchKernelGGL(modnorm_kernel<2>, grid, dim3(256), 0, stream, a);
  else if (vpl <= 4) hipLaunchKernelGGL(modnorm_kernel<4>, grid, dim3(256), 0, stream, a);
  else if (vpl <= 8) hipLaunchKernelGGL(modnorm_kernel<8>, grid, dim3(256), 0, stream, a);
  else if (vpl <= 12) hipLaunchKernelGGL(modnorm_kernel<12>, grid, dim3(256), 0, stream, a);
  else if (vpl <= 16) hipLaunchKernelGGL(modnorm_kernel<16>, grid, dim3(256), 0, stream, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t qkv_pad_launch(const QkvPadArgs& a, hipStream_t stream) {
  if (a.S_pad <= a.S || a.B == 0) return hipSuccess;
  hipLaunchKernelGGL(qkv_pad_kernel, dim3((unsigned)((int64_t)a.B * a.H)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t split_sum_launch(const SplitSumArgs& a, hipStream_t stream) {
  if (a.np < 1 || a.np > 7 || (a.cols & 3) || a.seg_len < 1) return hipErrorInvalidValue;
  const int64_t n = (int64_t)a.rows * (a.cols >> 2);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(split_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t rope_tables_launch(const RopeArgs& a, hipStream_t stream) {
  const int64_t n = a.S * a.pairs;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_tables_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t time_features_launch(const TimeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(time_features_kernel, dim3((unsigned)a.B), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t gemv_launch(const GemvArgs& a, hipStream_t stream) {
  if (a.B > kGemvMaxB || a.K > kGemvMaxK || (a.K & 7)) return hipErrorInvalidValue;
  // 1024 workgroups (4 per CU): every workgroup first copies x into LDS, so
  // more of them cost more than their extra loads in flight bring (the
  // three modulation GEMVs: 84 us at 1024, 87-90 at 2048, 104 at 512, 122
  // at one row per wave)
  const size_t lds = (size_t)a.B * a.K * sizeof(float);
  if (a.B == 1) {
    const int blocks = min(1024, (a.total_rows + 3) / 4);
    hipLaunchKernelGGL(gemv_kernel<4>, dim3((unsigned)blocks), dim3(256), lds, stream, a);
  } else {
    // 16-wave workgroups, two per CU
    const int blocks = min(512, (a.total_rows + 15) / 16);
    hipLaunchKernelGGL(gemv_kernel<16>, dim3((unsigned)blocks), dim3(1024), lds, stream, a);
  }
  return hipGetLastError();
}

hipError_t latent_pack_launch(const LatentArgs& a, hipStream_t stream) {
  if ((a.C & 3) || a.B < 0 || a.B > 64) return hipErrorInvalidValue;
  const int64_t n = (int64_t)a.B * (a.n_img + a.n_ref) * (a.C >> 2);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(latent_pack_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t euler_launch(const LatentArgs& a, hipStream_t stream) {
  if ((a.C & 3) || a.B < 0 || a.B > 64) return hipErrorInvalidValue;
  const int64_t n = (int64_t)a.B * a.n_img * (a.C >> 2);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(euler_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t rows_copy_launch(const RowsCopyArgs& a, hipStream_t stream) {
  if ((a.D & 3) || a.B < 0 || a.n < 0) return hipErrorInvalidValue;
  const int64_t n = (int64_t)a.B * a.n * (a.D >> 2);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(rows_copy_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dit
