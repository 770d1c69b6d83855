// Latent decoder kernels on gfx950 (the decoder that runs on the card after
// the last step, "tt_flux2_klein - Python reference", Lower-level entry
// points: decode; it has GroupNorm layers and takes non-square images,
// "flux2-klein-p100a", What this port adds). The layer list is a reading,
// stated in dit_vae.h.
//
// Convolution as an implicit GEMM on MFMA (one workgroup = 8 waves, one
// output tile of BM pixels by BN channels):
//  * Activations are channels-last bf16, so for a fixed kernel tap a pixel's
//    64-channel K slice is one 128-byte run. Slices go from L2 straight into
//    LDS with buffer loads that write LDS (as in the DiT GEMM): every loader
//    lane computes, per slice, the source pixel of each of its rows for its
//    16-byte chunk's tap, and a pixel outside the grid (zero padding), a K
//    index past the end, or a row past the tile's last pixel reads through
//    an offset beyond the buffer's range, which returns zeros. The upsample
//    before a conv is the same address map at half resolution, so the
//    upsampled tensor never exists.
//  * A ResNet's 1x1 shortcut is a second K range of the same tile (its own
//    source and weights), so the block output is one launch.
//  * Only waves 4-7 issue loads; all eight run MFMAs (v_mfma_f32_32x32x16_bf16,
//    wave tile 64 x 32 FN), two LDS stages, one barrier per slice; in the
//    main loop the loader waves run at a raised wave priority.
//  * Epilogue: fp32 accumulators staged through LDS in two passes; bias(es)
//    and the residual are added in fp32, then one rounding to bf16 (or an
//    fp32 store), 16 bytes per lane where the row allows.
//  * Tiles are walked channel-tile fastest and dealt to the XCDs in
//    contiguous ranges, so an XCD's L2 holds a band of image rows and their
//    halo.
// The k order of every output element depends only on the layer (its taps
// and channels), not on the tile shape or position, so batch rows are
// bitwise independent.
#include <algorithm>
#include <cmath>
#include <cstdlib>

#include "common.hpp"
#include "kernels.hpp"

namespace dit {
namespace {

// SiLU of the decoder's GroupNorm: v / (1 + e^-v) with the hardware
// reciprocal (1 ulp) instead of an IEEE divide; the normalize kernel and the
// halo conv's folded normalization both use it, so they agree bit for bit.
__device__ __forceinline__ float gn_silu(float v) {
  return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v));
}

constexpr int CBK = 64;            // K slice
constexpr int CNT = 512;           // 8 waves
constexpr int ROW_U = CBK / 8;     // 16-byte units per LDS row
constexpr uint32_t OOB = 0x80000000u;  // beyond every buffer's range (< 2^31 bytes)

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Epilogue of a conv tile: the lane holds tile rows wm*64 + 32 i + fr (i <
// 2) and channels wn*32FN + 32 j + 8q + 4fg + 0..3 of its accumulators. Pass
// p stages block i = p of every wave as fp32 [WM*32][BN] in LDS (16-byte
// chunk c of row r at c ^ (r & SWM)); the caller's LDS must be free (the
// main loop's last fragment reads came before its last barrier). pix(t) is
// the output pixel of tile row t, or -1 for none. Bias(es) and the residual
// are added in fp32 and the sum is rounded once (bf16) or stored fp32.
template <int WM, int FN, class PixOf>
__device__ __forceinline__ void conv_epilogue(const ConvArgs& a, f32x16 (&acc)[2][FN], char* T,
                                              int b, int n0, int wm, int wn, int fr, int fg,
                                              PixOf pix) {
  constexpr int WN = 8 / WM;
  constexpr int FM = 2;
  constexpr int BN = 32 * FN * WN;
  const int tid = threadIdx.x;
  constexpr int SROW = BN * 4;
  constexpr int SWM = (BN / 4 < 32 ? BN / 4 : 32) - 1;
  constexpr int UPR = BN / 8;  // 8-channel units per stage row
#pragma unroll
  for (int pass = 0; pass < FM; ++pass) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = wm * 32 + fr;
        const int c = (wn * 32 * FN + j * 32 + 8 * q + 4 * fg) >> 2;
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[pass][j][4 * q + e];
        *reinterpret_cast<f32x4*>(T + r * SROW + ((c ^ (r & SWM)) << 4)) = v;
      }
    __syncthreads();
    for (int u = tid; u < WM * 32 * UPR; u += CNT) {
      const int r = u / UPR, cu = u - r * UPR;
      const int m = pix((r >> 5) * 64 + 32 * pass + (r & 31));
      const int col = n0 + 8 * cu;
      if (m < 0 || col >= a.N) continue;
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(T + r * SROW + (((2 * cu) ^ (r & SWM)) << 4));
      const f32x4 v1 =
          *reinterpret_cast<const f32x4*>(T + r * SROW + (((2 * cu + 1) ^ (r & SWM)) << 4));
      float o[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      const int nv = a.N - col < 8 ? a.N - col : 8;
      const bool full = nv == 8 && a.vec;
      if (a.bias) {
        if (a.bias_rows) {
          const float bb = a.bias[m];
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] += bb;
        } else if (full) {
          const f32x4 b0 = *reinterpret_cast<const f32x4*>(a.bias + col);
          const f32x4 b1 = *reinterpret_cast<const f32x4*>(a.bias + col + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[e] += b0[e];
            o[4 + e] += b1[e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e < nv) o[e] += a.bias[col + e];
        }
      }
      if (a.bias2) {
        if (full) {
          const f32x4 b0 = *reinterpret_cast<const f32x4*>(a.bias2 + col);
          const f32x4 b1 = *reinterpret_cast<const f32x4*>(a.bias2 + col + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[e] += b0[e];
            o[4 + e] += b1[e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e < nv) o[e] += a.bias2[col + e];
        }
      }
      if (a.resid) {
        const bf16_t* rp = a.resid + (int64_t)b * a.resid_bs + (int64_t)m * a.ldr + col;
        if (full) {
          const u32x4 rv = *reinterpret_cast<const u32x4*>(rp);
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] += bf16_to_f32((rv[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e < nv) o[e] += bf16_to_f32(rp[e]);
        }
      }
      if (a.out_f32) {
        float* op = static_cast<float*>(a.out) + (int64_t)b * a.out_bs + (int64_t)m * a.ldo + col;
        if (full) {
          *reinterpret_cast<f32x4*>(op) = f32x4{o[0], o[1], o[2], o[3]};
          *reinterpret_cast<f32x4*>(op + 4) = f32x4{o[4], o[5], o[6], o[7]};
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e < nv) op[e] = o[e];
        }
      } else {
        bf16_t* op = static_cast<bf16_t*>(a.out) + (int64_t)b * a.out_bs + (int64_t)m * a.ldo + col;
        const f32x8 ov = {o[0], o[1], o[2], o[3], o[4], o[5], o[6], o[7]};
        const bf16x8 pv = pack_bf16x8(ov);
        if (full) {
          *reinterpret_cast<bf16x8*>(op) = pv;
        } else {
          const u32x4 pw = __builtin_bit_cast(u32x4, pv);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e < nv) op[e] = (bf16_t)((pw[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
        }
      }
    }
    __syncthreads();  // the next pass overwrites the stage
  }
}

// WM waves along the pixels (4 or 8), 8 / WM along the channels; wave tile
// 64 x 32 FN.
template <int WM, int FN>
__global__ __launch_bounds__(CNT, 1) void conv_kernel(const ConvArgs a) {
  constexpr int WN = 8 / WM;
  constexpr int FM = 2;
  constexpr int BM = 64 * WM, BN = 32 * FN * WN;
  constexpr int A_PER = BM / 128;           // 32-row A blocks per loader wave
  constexpr int W_BLK = BN / 32;            // 32-row W blocks in the tile
  constexpr int W_PER = (W_BLK + 3) / 4;    // W blocks per loader wave (at most)
  constexpr int STAGE_U = (BM + BN) * ROW_U;
  __shared__ u32x4 lds[2 * STAGE_U];
  static_assert(WM * 32 * BN * 4 <= 2 * STAGE_U * 16, "epilogue stage fits");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int per_b = a.tiles_m * a.tiles_n;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int b = L / per_b;
  const int rem = L - b * per_b;
  const int tm = rem / a.tiles_n, tn = rem - tm * a.tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  const int H = a.H, W = a.W, M = H * W;

  // ---- loaders: waves 4-7. Lane (lr, lp) of an 8-row group writes physical
  // chunk lp of row lr, i.e. logical chunk lp ^ swz(row) = lp ^ lr ^ (i & 1)
  // for the group's index i within its 32-row block.
  const int lr = (lane >> 3), lp = lane & 7;
  const bool loader = wave >= 4;
  const int lw = wave - 4;
  // Each A row of this lane: on an image grid the pixel (y, x) packed as
  // y << 16 | x (y = 0x7FFF past the last pixel, which fails every bounds
  // check); on a 1 x M grid (a plain GEMM, gemm_rows) the row index itself
  // (0xFFFFFFFF past the end).
  const bool gemm_rows = H == 1;
  uint32_t yx[A_PER * 4];
#pragma unroll
  for (int h = 0; h < A_PER; ++h)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + 32 * (lw + 4 * h) + 8 * i + lr;
      uint32_t v;
      if (gemm_rows) {
        v = m < M ? (uint32_t)m : 0xFFFFFFFFu;
      } else {
        v = 0x7FFFu << 16;
        if (m < M) {
          const int y = m / W;
          v = ((uint32_t)y << 16) | (uint32_t)(m - y * W);
        }
      }
      yx[h * 4 + i] = v;
    }
  __amdgpu_buffer_rsrc_t ar[2], wr[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const ConvSource& S = a.src[s < a.nsrc ? s : 0];
    ar[s] = make_rsrc(S.x + (int64_t)b * S.x_bs, S.x_bytes);
    wr[s] = make_rsrc(S.w + (int64_t)b * S.w_bs, S.w_bytes);
  }
  const int slices0 = a.src[0].slices;
  const int nk = slices0 + (a.nsrc > 1 ? a.src[1].slices : 0);

  auto dma = [&](int kt, int stage) {
    if (!loader) return;
    const int s = kt >= slices0 ? 1 : 0;
    const ConvSource& S = a.src[s];
    const int j = kt - (s ? slices0 : 0);
    const int C = S.C, lda = S.lda, taps = S.taps, up = S.up;
    const int kend = taps * C;
    // K order: a 3x3 conv over whole 64-channel slices runs slices outer and
    // taps inner (slice j = 9 cs + tap), the order of the halo kernel, so
    // either kernel gives the same bits; other sources run k = tap C + c in
    // order, 64 at a time.
    const bool cs_outer = taps == 9 && C % CBK == 0;
    const int cs_u = cs_outer ? j / 9 : 0, tap_u = cs_outer ? j - 9 * cs_u : 0;
    // per chunk parity: tap offsets, channel, and whether k is in range
    int dy[2], dx[2], ci[2];
    bool kok[2];
    int kk[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int cl = lp ^ lr ^ par;
      int tap, c, k;
      if (cs_outer) {
        tap = tap_u;
        c = cs_u * CBK + cl * 8;
        k = tap * C + c;
        kok[par] = true;
      } else {
        k = j * CBK + cl * 8;
        kok[par] = k < kend;
        tap = taps != 1 ? (int)(((float)k + 0.5f) * S.inv_c) : 0;
        c = k - tap * C;
      }
      kk[par] = k;
      ci[par] = c;
      const int ty = (tap * 11) >> 5;  // tap / 3 for tap < 9
      dy[par] = taps == 1 ? 0 : ty - 1;
      dx[par] = taps == 1 ? 0 : tap - 3 * ty - 1;
    }
    u32x4* const sa = lds + stage * STAGE_U;
    u32x4* const sw = lds + stage * STAGE_U + BM * ROW_U;
    const __amdgpu_buffer_rsrc_t A = s ? ar[1] : ar[0];
    const __amdgpu_buffer_rsrc_t Wr = s ? wr[1] : wr[0];
    const int Wi = up ? (W >> 1) : W;
#pragma unroll
    for (int h = 0; h < A_PER; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int par = i & 1;
        const uint32_t v = yx[h * 4 + i];
        uint32_t off;
        if (gemm_rows) {
          off = (kok[par] && v < (uint32_t)M) ? (v * (uint32_t)lda + (uint32_t)ci[par]) * 2u : OOB;
        } else {
          const int y = (int)(v >> 16), x = (int)(v & 0xFFFFu);
          const int yy = y + dy[par], xx = x + dx[par];
          const bool ok = kok[par] && (unsigned)yy < (unsigned)H && (unsigned)xx < (unsigned)W;
          const int py = up ? (yy >> 1) : yy, px = up ? (xx >> 1) : xx;
          off = ok ? (uint32_t)((py * Wi + px) * lda + ci[par]) * 2u : OOB;
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            A, (lds_ptr_t)(sa + (32 * (lw + 4 * h) + 8 * i) * ROW_U), 16, off, 0, 0, 0);
      }
#pragma unroll
    for (int h = 0; h < W_PER; ++h) {
      const int wb = lw + 4 * h;
      if (wb >= W_BLK) break;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int par = i & 1;
        const int n = n0 + 32 * wb + 8 * i + lr;
        const uint32_t off =
            kok[par] ? (uint32_t)(n * S.ldw + kk[par]) * 2u : OOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            Wr, (lds_ptr_t)(sw + (32 * wb + 8 * i) * ROW_U), 16, off, 0, 0, 0);
      }
    }
  };

  // ---- MFMA fragments (both operands double-buffered across k-steps)
  const int fr = lane & 31, fg = lane >> 5;
  const int wm = WM == 8 ? wave : (wave & 3), wn = WM == 8 ? 0 : (wave >> 2);
  const int a_rd = (wm * 64 + fr) * ROW_U;
  const int w_rd = BM * ROW_U + (wn * 32 * FN + fr) * ROW_U;
  const int sfr = swz(fr);
  bf16x8 af[2][FM], wf[2][FN];
  auto fload = [&](int stage, int s, int buf) {
    const u32x4* st = lds + stage * STAGE_U;
    const int ch = (2 * s + fg) ^ sfr;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      af[buf][i] = __builtin_bit_cast(bf16x8, st[a_rd + i * 32 * ROW_U + ch]);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      wf[buf][j] = __builtin_bit_cast(bf16x8, st[w_rd + j * 32 * ROW_U + ch]);
  };
  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};
  auto mfmas = [&](int buf) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[buf][j], af[buf][i], acc[i][j], 0, 0, 0);
  };

  dma(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (nk > 1) dma(1, 1);
  // loader waves at a raised wave priority in the main loop (as in the DiT
  // GEMM: a loader's reads, loads and MFMAs go first when both waves of a
  // SIMD are ready)
  if (loader) __builtin_amdgcn_s_setprio(1);
  fload(0, 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
#pragma unroll
    for (int s = 0; s < CBK / 16 - 1; ++s) {
      fload(cur, s + 1, (s + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
      mfmas(s & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // every wave is done with stage cur and slice kt + 1 has landed
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();
    if (kt + 2 < nk) dma(kt + 2, cur);
    if (kt + 1 < nk) fload(cur ^ 1, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    mfmas((CBK / 16 - 1) & 1);
    __builtin_amdgcn_sched_barrier(0);
  }

  __builtin_amdgcn_s_setprio(0);
  conv_epilogue<WM, FN>(a, acc, reinterpret_cast<char*>(lds), b, n0, wm, wn, fr, fg,
                        [&](int t) { return m0 + t < M ? m0 + t : -1; });
}

// ------------------------------------------------------------------ halo conv
// 3x3 convolution with the input halo of the tile resident in LDS: the
// implicit GEMM above reloads a pixel's K slice once per tap; here an output
// tile of 8 image rows x 32 columns loads its (8 + 2) x (32 + 2) input
// pixels once per 64-channel slice and the 9 taps read shifted fragments of
// it, so per channel slice the L2 -> LDS stream is the halo (44 KiB) plus
// the 9 taps' weights (BN x 128 bytes each) instead of 9 x (256 + BN) rows.
//  * K order: channel slices outer, taps inner (tap = 3 (dy + 1) + dx + 1),
//    16-wide k-steps, the same for every tile: batch rows stay bitwise
//    independent.
//  * Steps (slice, tap): a tap's weights go to one of two W buffers, a
//    slice's halo to one of two halo buffers, each loaded one step ahead
//    (the halo at the step before the slice's first tap); one barrier per
//    step. Out-of-image halo pixels (zero padding) read through an offset
//    past the buffer's range. With `up`, the halo pixel (Y, X) of the output
//    grid reads source pixel (Y / 2, X / 2).
//  * Waves: 4 along the rows (two image rows = two 32-pixel MFMA blocks
//    each) x 2 along the channels (32 FN each); BN = 64 FN.
constexpr int HT_ROWS = 8, HT_COLS = 32;
constexpr int HALO_W = HT_COLS + 2;
constexpr int HALO_PIX = (HT_ROWS + 2) * HALO_W;       // 340
constexpr int HALO_GROUPS = (HALO_PIX + 7) / 8;        // 8-pixel load groups: 43
constexpr int HALO_U = HALO_GROUPS * 8 * ROW_U;        // LDS units per halo buffer
constexpr int AB_U = 64;                               // GroupNorm scale / shift of a slice

template <int FN>
__global__ __launch_bounds__(CNT, 1) void conv3_halo_kernel(const ConvArgs a) {
  constexpr int WM = 4, FM = 2;
  constexpr int BN = 64 * FN;
  constexpr int W_U = BN * ROW_U;
  constexpr int HG_PER = (HALO_GROUPS + 3) / 4;  // halo groups per loader wave (at most)
  constexpr int WG_PER = BN / 8 / 4;             // weight-row groups per loader wave
  // halo 0 | halo 1 | W 0 | W 1 | GroupNorm (a, s) 0 | 1
  __shared__ u32x4 lds[2 * HALO_U + 2 * W_U + 2 * AB_U];
  constexpr int AB0 = 2 * HALO_U + 2 * W_U;
  static_assert(WM * 32 * BN * 4 <= (2 * HALO_U + 2 * W_U) * 16, "epilogue stage fits");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int per_b = a.tiles_m * a.tiles_n;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int b = L / per_b;
  const int rem = L - b * per_b;
  const int tm = rem / a.tiles_n, tn = rem - tm * a.tiles_n;
  const int ty = tm / a.tiles_x, tx = tm - ty * a.tiles_x;
  const int y0 = ty * HT_ROWS, x0 = tx * HT_COLS, n0 = tn * BN;
  const int H = a.H, W = a.W;
  const ConvSource& S = a.src[0];
  const int C = S.C, lda = S.lda, up = S.up;
  const int Wi = up ? (W >> 1) : W;
  const int nsteps = (C / CBK) * 9;
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(S.x + (int64_t)b * S.x_bs, S.x_bytes);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(S.w + (int64_t)b * S.w_bs, S.w_bytes);

  // ---- loaders (waves 4-7). Lane (lr, lp) of an 8-row load group g writes
  // physical chunk lp of row 8g + lr (a halo pixel or a weight row), whose
  // swizzle is swz(8g + lr) = lr ^ (g & 1): it fetches logical chunk
  // lp ^ lr ^ (g & 1).
  const int lr = lane >> 3, lp = lane & 7;
  const bool loader = wave >= 4;
  const int lw = wave - 4;
  const uint32_t cofs[2] = {(uint32_t)((lp ^ lr) * 16), (uint32_t)((lp ^ lr ^ 1) * 16)};
  uint32_t hoff[HG_PER];  // byte offset of channel 0 of the lane's halo pixels, or OOB
#pragma unroll
  for (int i = 0; i < HG_PER; ++i) {
    const int g = lw + 4 * i;
    const int p = 8 * g + lr;
    const int hy = p / HALO_W, hx = p - hy * HALO_W;
    const int Y = y0 - 1 + hy, X = x0 - 1 + hx;
    const bool ok = g < HALO_GROUPS && p < HALO_PIX && (unsigned)Y < (unsigned)H &&
                    (unsigned)X < (unsigned)W;
    const int sy = up ? (Y >> 1) : Y, sx = up ? (X >> 1) : X;
    hoff[i] = ok ? (uint32_t)((sy * Wi + sx) * lda) * 2u : OOB;
  }
  uint32_t woff[WG_PER];  // byte offset of the lane's weight rows, or OOB
#pragma unroll
  for (int i = 0; i < WG_PER; ++i) {
    const int n = n0 + 8 * (lw + 4 * i) + lr;
    woff[i] = n < a.N ? (uint32_t)(n * S.ldw) * 2u : OOB;
  }
  auto load_halo = [&](int cs, int buf) {
    if (!loader) return;
    u32x4* const dst = lds + buf * HALO_U;
#pragma unroll
    for (int i = 0; i < HG_PER; ++i) {
      const int g = lw + 4 * i;
      if (g >= HALO_GROUPS) break;
      const uint32_t off = hoff[i] == OOB ? OOB : hoff[i] + (uint32_t)(cs * CBK * 2) + cofs[g & 1];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (lds_ptr_t)(dst + 8 * g * ROW_U), 16, off, 0,
                                               0, 0);
    }
  };
  // GroupNorm folded into the input: the slice's 64 (a_c, s_c) pairs go to
  // LDS with the halo (one load instruction, lanes 32-63 read zeros), and
  // the landed halo is transformed in place once, before its first tap.
  const bool gn = a.gn_ab != nullptr;
  const __amdgpu_buffer_rsrc_t abr =
      make_rsrc(gn ? a.gn_ab + (int64_t)b * C * 2 : a.gn_ab, gn ? (uint32_t)(C * 2 * 4) : 0u);
  auto load_ab = [&](int cs, int buf) {
    if (!gn || wave != 4) return;
    const uint32_t off = lane < 32 ? (uint32_t)((cs * CBK * 2 + lane * 4) * 4) : OOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(abr, (lds_ptr_t)(lds + AB0 + buf * AB_U), 16, off, 0,
                                             0, 0);
  };
  // act(x a_c + s_c) of the in-image halo pixels of buffer buf, in place
  // (the formula of the normalize kernel, so either path gives the same
  // bits); out-of-image pixels stay zero. Part `part` of XF_PARTS: 16-byte
  // chunks [part XF_CH, (part + 1) XF_CH), one per thread.
  constexpr int XF_PARTS = 8;
  constexpr int XF_CH = (HALO_PIX * 8 + XF_PARTS - 1) / XF_PARTS;  // 340 chunks
  static_assert(XF_CH <= CNT, "one chunk per thread and part");
  auto transform = [&](int buf, int part) {
    u32x4* const hb = lds + buf * HALO_U;
    const float* const abl = reinterpret_cast<const float*>(lds + AB0 + buf * AB_U);
    {
      if (tid >= XF_CH) return;
      const int u = part * XF_CH + tid;
      const int p = u >> 3;
      if (p >= HALO_PIX) return;
      const int hy = p / HALO_W, hx = p - hy * HALO_W;
      const int Y = y0 - 1 + hy, X = x0 - 1 + hx;
      if ((unsigned)Y >= (unsigned)H || (unsigned)X >= (unsigned)W) return;
      const int lc = (u & 7) ^ swz(p);
      const u32x4 v = hb[u];
      const f32x4 q0 = *reinterpret_cast<const f32x4*>(abl + lc * 16);
      const f32x4 q1 = *reinterpret_cast<const f32x4*>(abl + lc * 16 + 4);
      const f32x4 q2 = *reinterpret_cast<const f32x4*>(abl + lc * 16 + 8);
      const f32x4 q3 = *reinterpret_cast<const f32x4*>(abl + lc * 16 + 12);
      const float sc[8] = {q0[0], q0[2], q1[0], q1[2], q2[0], q2[2], q3[0], q3[2]};
      const float sf[8] = {q0[1], q0[3], q1[1], q1[3], q2[1], q2[3], q3[1], q3[3]};
      f32x8 r;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float t =
            fmaf(bf16_to_f32((v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu), sc[e], sf[e]);
        r[e] = a.gn_silu ? gn_silu(t) : t;
      }
      hb[u] = __builtin_bit_cast(u32x4, pack_bf16x8(r));
    }
  };
  auto load_w = [&](int cs, int tap, int buf) {
    if (!loader) return;
    u32x4* const dst = lds + 2 * HALO_U + buf * W_U;
    const uint32_t kb = (uint32_t)((tap * C + cs * CBK) * 2);
#pragma unroll
    for (int i = 0; i < WG_PER; ++i) {
      const int g = lw + 4 * i;
      const uint32_t off = woff[i] == OOB ? OOB : woff[i] + kb + cofs[g & 1];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t)(dst + 8 * g * ROW_U), 16, off, 0,
                                               0, 0);
    }
  };

  // ---- fragments: block i of wave wm is image row 2 wm + i of the tile;
  // for tap (dy, dx) its 32 pixels are halo pixels (2 wm + i + 1 + dy) *
  // HALO_W + fr + 1 + dx
  const int fr = lane & 31, fg = lane >> 5;
  const int wm = wave & 3, wn = wave >> 2;
  const int w_rd = (wn * 32 * FN + fr) * ROW_U;
  const int sfr = swz(fr);
  bf16x8 af[2][FM], wf[2][FN];
  auto fload = [&](int cs, int tap, int step, int s, int buf) {
    const int ty3 = (tap * 11) >> 5;
    const int dy = ty3 - 1, dx = tap - 3 * ty3 - 1;
    const u32x4* hb = lds + (cs & 1) * HALO_U;
    const u32x4* wb = lds + 2 * HALO_U + (step & 1) * W_U;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int p = (2 * wm + i + 1 + dy) * HALO_W + fr + 1 + dx;
      af[buf][i] = __builtin_bit_cast(bf16x8, hb[p * ROW_U + ((2 * s + fg) ^ swz(p))]);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j)
      wf[buf][j] = __builtin_bit_cast(bf16x8, wb[w_rd + j * 32 * ROW_U + ((2 * s + fg) ^ sfr)]);
  };
  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};
  auto mfmas = [&](int buf) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[buf][j], af[buf][i], acc[i][j], 0, 0, 0);
  };

  // Schedule: the weights of step j are loaded during step j - 1; the halo
  // (and GroupNorm pairs) of slice c + 1 during step 9c, the slice's first
  // tap, and with GroupNorm folded in, transformed one eighth at a time
  // during its taps 1-8, between their MFMAs. Every step ends with all
  // loads landed and one barrier.
  const int CS = C / CBK;
  load_halo(0, 0);
  load_ab(0, 0);
  load_w(0, 0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (nsteps > 1) load_w(0, 1, 1);
  if (CS > 1) {
    load_halo(1, 1);
    load_ab(1, 1);
  }
  if (gn) {
#pragma unroll 1
    for (int part = 0; part < XF_PARTS; ++part) transform(0, part);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __syncthreads();
  }
  // loader waves at a raised wave priority in the main loop (same box: 335
  // -> 324 us per launch at 1024^2, decode 13.5 -> 13.2 ms)
  if (loader) __builtin_amdgcn_s_setprio(1);
  fload(0, 0, 0, 0, 0);
  int cs = 0, tap = 0;  // of the current step
  for (int step = 0; step < nsteps; ++step) {
    const bool xform = gn && tap >= 1 && cs + 1 < CS;
#pragma unroll
    for (int s = 0; s < CBK / 16 - 1; ++s) {
      fload(cs, tap, step, s + 1, (s + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
      mfmas(s & 1);
      __builtin_amdgcn_sched_barrier(0);
      if (s == 0 && xform) {
        transform((cs + 1) & 1, tap - 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // every wave is done with this step's buffers; the next step's landed
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();
    int cs1 = cs, tap1 = tap + 1;
    if (tap1 == 9) {
      tap1 = 0;
      ++cs1;
    }
    if (step + 2 < nsteps) {
      int cs2 = cs1, tap2 = tap1 + 1;
      if (tap2 == 9) {
        tap2 = 0;
        ++cs2;
      }
      load_w(cs2, tap2, step & 1);
    }
    // the next step starts slice cs1: the halo of slice cs1 + 1 goes into
    // the buffer slice cs1 - 1 used
    if (tap1 == 0 && cs1 + 1 < CS) {
      load_halo(cs1 + 1, (cs1 + 1) & 1);
      load_ab(cs1 + 1, (cs1 + 1) & 1);
    }
    if (step + 1 < nsteps) fload(cs1, tap1, step + 1, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    mfmas((CBK / 16 - 1) & 1);
    __builtin_amdgcn_sched_barrier(0);
    cs = cs1;
    tap = tap1;
  }

  __builtin_amdgcn_s_setprio(0);
  conv_epilogue<WM, FN>(a, acc, reinterpret_cast<char*>(lds), b, n0, wm, wn, fr, fg,
                        [&](int t) {
                          const int y = y0 + (t >> 5), x = x0 + (t & 31);
                          return (y < H && x < W) ? y * W + x : -1;
                        });
}

// ------------------------------------------------------------------ GroupNorm
constexpr int GN_NT = 256;

// Partial sums of d = x - shift_g and d^2 per (sample, block, group); block
// blockIdx.x covers pixels [blk ppb, blk ppb + ppb) of sample blockIdx.y.
// Thread: 8 consecutive channels (chunk tid % (C / 8)) of every
// (256 / (C / 8))-th pixel; sums per channel, then over the block's pixel
// lanes and over the group's channels in a fixed order.
__global__ __launch_bounds__(GN_NT) void gn_stats_kernel(const GroupNormArgs g) {
  __shared__ float red[GN_NT * 8 * 2];
  const int tid = threadIdx.x;
  const int b = blockIdx.y, blk = blockIdx.x;
  const int C = g.C, cpt = C >> 3, ppi = GN_NT / cpt;
  const int cu = tid % cpt, pl = tid / cpt;
  const int cg = C / g.G;
  const bf16_t* x = g.x + (int64_t)b * g.x_bs;
  float sh[8], s1[8], s2[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = 8 * cu + e;
    sh[e] = bf16_to_f32(x[(c / cg) * cg]);
    s1[e] = 0.f;
    s2[e] = 0.f;
  }
  const int p0 = blk * g.ppb;
  const int p1 = min(p0 + g.ppb, g.HW);
  for (int p = p0 + pl; p < p1; p += ppi) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(x + (int64_t)p * C + 8 * cu);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float d = bf16_to_f32((v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu) - sh[e];
      s1[e] += d;
      s2[e] += d * d;
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    red[(pl * C + 8 * cu + e) * 2] = s1[e];
    red[(pl * C + 8 * cu + e) * 2 + 1] = s2[e];
  }
  __syncthreads();
  // per channel, over the pixel lanes in order (C <= 2048: up to 8 channels
  // per thread); results kept in registers, then written over red[0 .. 2C)
  float c1[8], c2[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int c = tid + t * GN_NT;
    c1[t] = 0.f;
    c2[t] = 0.f;
    if (c < C) {
      for (int q = 0; q < ppi; ++q) {
        c1[t] += red[(q * C + c) * 2];
        c2[t] += red[(q * C + c) * 2 + 1];
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int c = tid + t * GN_NT;
    if (c < C) {
      red[2 * c] = c1[t];
      red[2 * c + 1] = c2[t];
    }
  }
  __syncthreads();
  for (int gg = tid; gg < g.G; gg += GN_NT) {
    float a1 = 0.f, a2 = 0.f;
    for (int c = gg * cg; c < (gg + 1) * cg; ++c) {
      a1 += red[2 * c];
      a2 += red[2 * c + 1];
    }
    float* out = g.part + (((int64_t)b * g.nblk + blk) * g.G + gg) * 2;
    out[0] = a1;
    out[1] = a2;
  }
}

// One workgroup per (group, sample): thread t adds the partials of blocks
// t, t + 256, ... in order, in double; a fixed shuffle tree and the four
// waves in order give the totals; then the group's per-channel scale and
// shift.
__global__ __launch_bounds__(GN_NT) void gn_finalize_kernel(const GroupNormArgs g) {
  __shared__ double red[2][GN_NT / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gg = blockIdx.x, b = blockIdx.y;
  const int cg = g.C / g.G;
  double a1 = 0.0, a2 = 0.0;
  for (int k = tid; k < g.nblk; k += GN_NT) {
    const float* p = g.part + (((int64_t)b * g.nblk + k) * g.G + gg) * 2;
    a1 += (double)p[0];
    a2 += (double)p[1];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    a1 += __shfl_xor(a1, o, 64);
    a2 += __shfl_xor(a2, o, 64);
  }
  if (lane == 0) {
    red[0][wave] = a1;
    red[1][wave] = a2;
  }
  __syncthreads();
  double s1 = 0.0, s2 = 0.0;
#pragma unroll
  for (int w = 0; w < GN_NT / 64; ++w) {
    s1 += red[0][w];
    s2 += red[1][w];
  }
  const bf16_t* x = g.x + (int64_t)b * g.x_bs;
  const double n = (double)g.HW * (double)cg;
  const double md = s1 / n;
  double var = s2 / n - md * md;
  if (var < 0.0) var = 0.0;
  const double mean = (double)bf16_to_f32(x[gg * cg]) + md;
  const double rstd = 1.0 / sqrt(var + (double)g.eps);
  for (int c = gg * cg + tid; c < (gg + 1) * cg; c += GN_NT) {
    const double sc = (double)g.gamma[c] * rstd;
    g.ab[((int64_t)b * g.C + c) * 2] = (float)sc;
    g.ab[((int64_t)b * g.C + c) * 2 + 1] = (float)((double)g.beta[c] - mean * sc);
  }
}

// y = act(x a_c + s_c), 8 channels per thread and step. Grid (., B): a
// thread keeps one 8-channel chunk (the grid stride is a multiple of C / 8)
// and its scale / shift in registers, and has four steps' loads in flight.
__global__ __launch_bounds__(GN_NT) void gn_apply_kernel(const GroupNormArgs g) {
  constexpr int U = 4;
  const int b = blockIdx.y;
  const int cpt = g.C >> 3;
  const int64_t units = (int64_t)g.HW * cpt;
  const int64_t stride = (int64_t)gridDim.x * GN_NT;
  int64_t u = (int64_t)blockIdx.x * GN_NT + threadIdx.x;
  const int cu = (int)(u % cpt);
  const float* ab = g.ab + ((int64_t)b * g.C + 8 * cu) * 2;
  float sc[8], sf[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(ab + 4 * q);
    sc[2 * q] = v[0];
    sf[2 * q] = v[1];
    sc[2 * q + 1] = v[2];
    sf[2 * q + 1] = v[3];
  }
  const bf16_t* x = g.x + (int64_t)b * g.x_bs;
  bf16_t* y = g.y + (int64_t)b * g.y_bs;
  for (; u < units; u += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int64_t ui = u + i * stride;
      if (ui < units) v[i] = *reinterpret_cast<const u32x4*>(x + ui * 8);
    }
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int64_t ui = u + i * stride;
      if (ui >= units) break;
      f32x8 r;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float t =
            fmaf(bf16_to_f32((v[i][e >> 1] >> (16 * (e & 1))) & 0xFFFFu), sc[e], sf[e]);
        r[e] = g.silu ? gn_silu(t) : t;
      }
      *reinterpret_cast<bf16x8*>(y + ui * 8) = pack_bf16x8(r);
    }
  }
}

// ------------------------------------------------------------------ softmax
__global__ __launch_bounds__(256) void softmax_rows_kernel(const SoftmaxArgs a) {
  __shared__ float wm_[4], wl_[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const float* s = a.s + row * a.lds;
  const float c = a.scale * 1.4426950408889634f;  // log2(e)
  float m = -INFINITY, l = 0.f;
  for (int i = 4 * tid; i < a.n; i += 1024) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(s + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float t = v[e] * c;
      if (t > m) {
        l = l * exp2f(m - t) + 1.f;
        m = t;
      } else {
        l += exp2f(t - m);
      }
    }
  }
  // combine (m, l) over the block
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), l2 = __shfl_xor(l, o, 64);
    const float mm = fmaxf(m, m2);
    l = (m == -INFINITY ? 0.f : l * exp2f(m - mm)) + (m2 == -INFINITY ? 0.f : l2 * exp2f(m2 - mm));
    m = mm;
  }
  if (lane == 0) {
    wm_[wave] = m;
    wl_[wave] = l;
  }
  __syncthreads();
  float M = wm_[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) M = fmaxf(M, wm_[w]);
  float Lsum = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) Lsum += wl_[w] * exp2f(wm_[w] - M);
  const float inv = 1.f / Lsum;
  bf16_t* p = a.p + row * a.ldp;
  for (int i = 4 * tid; i < a.n; i += 1024) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(s + i);
    f32x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = exp2f(v[e] * c - M) * inv;
    *reinterpret_cast<u32x2*>(p + i) = pack_bf16x4(y);
  }
  // padding columns [n, ldp) read as exact zeros by a product over ldp keys
  for (int64_t i = a.n + tid; i < a.ldp; i += 256) p[i] = 0;
}

// ------------------------------------------------------------------ latent image
__global__ __launch_bounds__(256) void latent_image_kernel(const LatentImageArgs a) {
  const int H = 2 * a.hp, W = 2 * a.wp, Z = a.Z;
  const int64_t total = (int64_t)a.B * H * W * Z;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * 256) {
    const int k = (int)(t % Z);
    const int64_t px = t / Z;
    const int X = (int)(px % W);
    const int64_t by = px / W;
    const int Y = (int)(by % H);
    const int b = (int)(by / H);
    const int64_t tok = (int64_t)b * a.hp * a.wp + (int64_t)(Y >> 1) * a.wp + (X >> 1);
    const int ch = 4 * k + 2 * (Y & 1) + (X & 1);
    const float u = fmaf(a.z[tok * 4 * Z + ch], a.scale[ch], a.shift[ch]);
    const f32x4 uv = {u, 0.f, 0.f, 0.f};
    a.x[t] = (bf16_t)(pack_bf16x4(uv)[0] & 0xFFFFu);
  }
}

// ------------------------------------------------------------------ host side
// Tile shapes: 0-3 the implicit GEMM (rows x channels), 4-5 the halo conv
// (8 x 32 pixels x channels; single-source 3x3 convs with 64-channel slices).
struct TileCfg {
  int bm, bn;
  bool halo;
  double eff;  // relative MFMA efficiency of the shape
};
// The implicit GEMM's loop is paced by the L2 -> LDS stream of (rows +
// columns) x 128 bytes per K slice, so its efficiency follows
// rows x columns / (rows + columns): 1, 0.85, 0.7, 0.25 of the 256 x 256
// tile; the halo shapes are MFMA-bound (measured 1.3 and 1.2).
constexpr TileCfg kCfgs[] = {{256, 256, false, 1.0}, {512, 128, false, 0.85},
                             {256, 128, false, 0.7}, {512, 32, false, 0.25},
                             {256, 256, true, 1.3},  {256, 128, true, 1.2}};
constexpr int kNumCfgs = 6;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool halo_ok(const ConvArgs& a) {
  return a.nsrc == 1 && a.src[0].taps == 9 && a.src[0].C % CBK == 0 && a.H > 1;
}

// Tile count of shape c for the launch.
int64_t cfg_tiles(const ConvArgs& a, int c) {
  const TileCfg& t = kCfgs[c];
  if (t.halo)
    return (int64_t)a.B * ceil_div(a.H, HT_ROWS) * ceil_div(a.W, HT_COLS) * ceil_div(a.N, t.bn);
  return (int64_t)a.B * ceil_div((int64_t)a.H * a.W, t.bm) * ceil_div(a.N, t.bn);
}

// Tile shape: the modelled time is the rounds of tiles over 256 CUs (at
// least one; a partial last round counts by its fraction, since its tiles
// run faster with fewer neighbours) times a tile's MFMA work divided by the
// shape's relative efficiency (measured on the decoder's layers: the halo
// shapes reach 1.1-1.2 PFLOP/s at 256 and 512 channels). The choice
// never changes a result: every shape of both kernels adds an output
// element's terms in the same k-steps in the same order (for 3x3 convs over
// 64-channel slices: slices outer, taps inner).
int pick_cfg(const ConvArgs& a) {
  if (a.N <= 32) return 3;  // narrow outputs (conv_out): wider tiles only waste columns
  const bool halo = halo_ok(a);
  int best = 0;
  double best_t = 1e300;
  for (int c = 0; c < kNumCfgs; ++c) {
    const TileCfg& t = kCfgs[c];
    if (t.halo && !halo) continue;
    const double rounds = std::max(1.0, (double)cfg_tiles(a, c) / 256.0);
    const double time = rounds * t.bm * t.bn / t.eff;
    if (time < best_t * 0.999) {
      best_t = time;
      best = c;
    }
  }
  return best;
}

// DIT_CONV_TILE (tests): force tile shape c when it applies to the launch.
int forced_cfg(const ConvArgs& a) {
  const char* e = std::getenv("DIT_CONV_TILE");
  if (!e || !*e) return -1;
  const int c = std::atoi(e);
  if (c < 0 || c >= kNumCfgs || (kCfgs[c].halo && !halo_ok(a))) return -1;
  return c;
}

}  // namespace

bool conv_uses_halo(const ConvArgs& a) {
  if (a.N <= 0 || a.nsrc < 1) return false;
  const int f = forced_cfg(a);
  return kCfgs[f >= 0 ? f : pick_cfg(a)].halo;
}

hipError_t conv_launch(ConvArgs& a, hipStream_t stream) {
  const int64_t M = (int64_t)a.H * a.W;
  if (a.B <= 0 || M <= 0 || a.N <= 0) return hipSuccess;
  // image grids: y and x fit the packed 16-bit fields; 1 x M grids: plain rows
  if (a.nsrc < 1 || a.nsrc > 2 || M > (1 << 30) || (a.H > 1 && (a.H > 32766 || a.W > 32767)))
    return hipErrorInvalidValue;
  for (int s = 0; s < a.nsrc; ++s) {
    ConvSource& S = a.src[s];
    if (!S.x || !S.w || S.C <= 0 || S.C % 8 || S.lda % 8 || S.ldw % 8 ||
        (S.taps != 1 && S.taps != 9) || (S.up && (a.H % 2 || a.W % 2)) ||
        (a.H == 1 && (S.taps != 1 || S.up)) ||
        S.x_bytes >= OOB || S.w_bytes >= OOB || S.lda < S.C || S.ldw < S.taps * S.C)
      return hipErrorInvalidValue;
    // offsets of every row (pixel or weight row) stay below 2^31
    const int64_t pix = S.up ? M / 4 : M;
    if ((int64_t)pix * S.lda * 2 > (int64_t)S.x_bytes ||
        ((int64_t)a.N + 256) * S.ldw * 2 >= (int64_t)OOB)
      return hipErrorInvalidValue;
    S.slices = (int)ceil_div((int64_t)S.taps * S.C, CBK);
    S.inv_c = 1.0f / (float)S.C;
  }
  if (!a.out || (a.resid && a.ldr < a.N) || a.ldo < a.N) return hipErrorInvalidValue;
  if (a.nsrc < 2) a.src[1] = a.src[0];
  a.vec = (a.ldo % 8 == 0) && (reinterpret_cast<uintptr_t>(a.out) % 16 == 0) &&
          (a.out_bs % 8 == 0) &&
          (!a.resid || (a.ldr % 8 == 0 && reinterpret_cast<uintptr_t>(a.resid) % 16 == 0 &&
                        a.resid_bs % 8 == 0)) &&
          (!a.bias || a.bias_rows || reinterpret_cast<uintptr_t>(a.bias) % 16 == 0) &&
          (!a.bias2 || reinterpret_cast<uintptr_t>(a.bias2) % 16 == 0);
  const int c = forced_cfg(a) >= 0 ? forced_cfg(a) : pick_cfg(a);
  const TileCfg& t = kCfgs[c];
  if (a.gn_ab && !t.halo) return hipErrorInvalidValue;  // only the halo kernel folds GroupNorm
  a.cfg = c;
  if (t.halo) {
    a.tiles_x = (int)ceil_div(a.W, HT_COLS);
    a.tiles_m = (int)ceil_div(a.H, HT_ROWS) * a.tiles_x;
  } else {
    a.tiles_x = 0;
    a.tiles_m = (int)ceil_div(M, t.bm);
  }
  a.tiles_n = (int)ceil_div(a.N, t.bn);
  const int64_t n_wg = (int64_t)a.B * a.tiles_m * a.tiles_n;
  if (n_wg > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)n_wg);
  switch (c) {
    case 0: hipLaunchKernelGGL((conv_kernel<4, 4>), grid, dim3(CNT), 0, stream, a); break;
    case 1: hipLaunchKernelGGL((conv_kernel<8, 4>), grid, dim3(CNT), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((conv_kernel<4, 2>), grid, dim3(CNT), 0, stream, a); break;
    case 3: hipLaunchKernelGGL((conv_kernel<8, 1>), grid, dim3(CNT), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((conv3_halo_kernel<4>), grid, dim3(CNT), 0, stream, a); break;
    default: hipLaunchKernelGGL((conv3_halo_kernel<2>), grid, dim3(CNT), 0, stream, a); break;
  }
  return hipGetLastError();
}

hipError_t group_norm_launch(const GroupNormArgs& g, hipStream_t stream) {
  if (g.B <= 0 || g.HW <= 0) return hipSuccess;
  const int cpt = g.C / 8;
  if (g.C % 8 || g.C > 2048 || GN_NT % cpt || g.G <= 0 || g.C % g.G || g.G > 1024 ||
      g.ppb % (GN_NT / cpt) || (int64_t)g.nblk * g.ppb < g.HW)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(gn_stats_kernel, dim3((unsigned)g.nblk, (unsigned)g.B), dim3(GN_NT), 0,
                     stream, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gn_finalize_kernel, dim3((unsigned)g.G, (unsigned)g.B), dim3(GN_NT), 0,
                     stream, g);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!g.apply) return hipSuccess;
  const int64_t units = (int64_t)g.HW * cpt;
  const int64_t blocks = std::max<int64_t>(
      1, std::min<int64_t>(ceil_div(units, GN_NT * 4), std::max<int64_t>(1, 4096 / g.B)));
  hipLaunchKernelGGL(gn_apply_kernel, dim3((unsigned)blocks, (unsigned)g.B), dim3(GN_NT), 0,
                     stream, g);
  return hipGetLastError();
}

hipError_t softmax_rows_launch(const SoftmaxArgs& a, hipStream_t stream) {
  if (a.rows <= 0 || a.n <= 0) return hipSuccess;
  if (a.n % 4 || a.lds % 4 || a.ldp % 4 || a.lds < a.n || a.ldp < a.n)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(softmax_rows_kernel, dim3((unsigned)a.rows), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t latent_image_launch(const LatentImageArgs& a, hipStream_t stream) {
  const int64_t total = (int64_t)a.B * 4 * a.hp * a.wp * a.Z;
  if (total <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>(ceil_div(total, 256), 4096);
  hipLaunchKernelGGL(latent_image_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dit
