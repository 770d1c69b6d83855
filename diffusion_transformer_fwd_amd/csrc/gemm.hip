// bf16 GEMM on gfx950 MFMA with fused epilogues: C = A W^T.
//
// This carries every dense contraction of the step: the QKV / output / MLP
// projections of the dual-stream blocks, the fused input (QKV + SwiGLU) and
// output projections of the single-stream blocks, the two embeddings and
// the final projection ("tt_flux2_klein - Python reference", Modules: the
// DiT's 5 dual + 20 single blocks; the block maths is stated in dit.h).
//
// Design (one workgroup = 4 waves = 256 threads, one 256 x 256 output tile):
//  * A [M, K] and W [N, K] are both K-contiguous, so one 64-wide K slice of
//    each tile is a set of 128-byte row segments: every thread fetches 16
//    bytes per row segment (coalesced), and the slice is stored to LDS with
//    its 16-byte chunks XOR-swizzled by row so that MFMA fragment reads are
//    free of bank conflicts. Two LDS stages (128 KiB of the CU's 160 KiB):
//    the next slice is fetched into registers while the current one feeds
//    the MFMAs, then written to the other stage; one barrier per slice.
//  * Each wave owns a 128 x 128 sub-tile as 4 x 4 blocks of
//    v_mfma_f32_32x32x16_bf16 (fp32 accumulators, 256 per lane). The weight
//    fragment is the MFMA's first operand and the activation fragment the
//    second, so each lane ends up holding one output row and runs of four
//    consecutive output columns: epilogue stores are 8-byte (bf16) or
//    16-byte (fp32) vectors.
//  * Epilogues: bf16 store; SwiGLU (each wave's column half is gate rows and
//    the other half the matching up rows, so SiLU(g) * u is lane-local);
//    gated residual x += gate[b] * acc on the fp32 residual; fp32 store.
//    Output rows go through a (segment length, stride, offset) map, so
//    stream-major operands scatter back into x[B, S, D] in place.
//  * Up to four independent problems share one launch (text + image
//    streams, or the single block's QKV part + SwiGLU part), so the small
//    512-row text problem fills gaps instead of taking its own launch.
//  * Tile order: launch index -> XCD-contiguous logical index -> groups of
//    8 row tiles walked column by column, so co-resident tiles on one XCD
//    share A and W panels in its L2.
//  * The accumulation order of an output element depends only on K, never
//    on M or the tile position, so a batch row's results are bitwise the
//    same whatever else is in the batch.
#include "common.hpp"
#include "kernels.hpp"

namespace dit {
namespace {

constexpr int BM = kGemmBM, BN = kGemmBN, BK = kGemmBK;
constexpr int NT = 256;
constexpr int WTM = 128, WTN = 128;
constexpr int FM = WTM / 32, FN = WTN / 32;
constexpr int ROW_U = BK / 8;                 // 16-byte units per LDS row
constexpr int CH_A = BM * ROW_U / NT;         // chunks per thread per slice
constexpr int CH_W = BN * ROW_U / NT;
constexpr int STAGE_U = (BM + BN) * ROW_U;    // 16-byte units per stage

static_assert(CH_A == 8 && CH_W == 8, "loader assumes 8 chunks per thread");

// Chunk swizzle by row: distinct for 8 consecutive rows and for the 8 rows of
// either parity among 16 consecutive rows.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ void tile_coords(int local, int tiles_m, int tiles_n,
                                            int& tm, int& tn) {
  constexpr int GROUP = 8;
  const int per_group = GROUP * tiles_n;
  const int grp = local / per_group;
  const int first = grp * GROUP;
  const int gsize = min(tiles_m - first, GROUP);
  const int in = local - grp * per_group;
  tm = first + in % gsize;
  tn = in / gsize;
}

__device__ __forceinline__ void store4(const GemmProblem& P, int epi, int64_t out_row,
                                       int col, int b, f32x4 v) {
  if (epi == EPI_BF16 || epi == EPI_SWIGLU) {
    bf16_t* c = static_cast<bf16_t*>(P.C) + out_row * P.ldc + col;
    *reinterpret_cast<u32x2*>(c) = pack_bf16x4(v);
  } else if (epi == EPI_F32) {
    float* c = static_cast<float*>(P.C) + out_row * P.ldc + col;
    *reinterpret_cast<f32x4*>(c) = v;
  } else {
    float* c = static_cast<float*>(P.C) + out_row * P.ldc + col;
    const f32x4 g = *reinterpret_cast<const f32x4*>(P.gate + (int64_t)b * P.gate_bstride + col);
    f32x4 x = *reinterpret_cast<f32x4*>(c);
    x += g * v;
    *reinterpret_cast<f32x4*>(c) = x;
  }
}

__global__ __launch_bounds__(NT, 1) void gemm_bf16_kernel(const GemmBatch args) {
  __shared__ u32x4 lds[2 * STAGE_U];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  int pi = 0;
#pragma unroll
  for (int i = 1; i < kMaxGemmProblems; ++i)
    if (i < args.count && L >= args.p[i].tile_begin) pi = i;
  pi = __builtin_amdgcn_readfirstlane(pi);
  // Constant-index copies keep every field in scalar registers.
  GemmProblem P;
  if (pi == 0) P = args.p[0];
  else if (pi == 1) P = args.p[1];
  else if (pi == 2) P = args.p[2];
  else P = args.p[3];
  const int M = P.M, N = P.N, K = P.K, epi = P.epi;
  int tm, tn;
  tile_coords(L - P.tile_begin, P.tiles_m, P.tiles_n, tm, tn);
  const int m0 = tm * BM;

  // ---- global -> LDS loader: thread owns chunk ckc of rows crow + 32 i.
  // Buffer loads: rows past the end of A or W read as zero (tail tiles).
  const int crow = tid >> 3, ckc = tid & 7;
  const int w_rows = epi == EPI_SWIGLU ? 2 * N : N;
  const uint32_t a_bytes = clamp_u32((int64_t)M * P.lda * 2);
  const uint32_t w_bytes = clamp_u32((int64_t)w_rows * P.ldw * 2);
  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(P.A, a_bytes);
  const __amdgpu_buffer_rsrc_t w_rsrc = make_rsrc(P.W, w_bytes);
  const uint32_t a_voff = (uint32_t)(((int64_t)(m0 + crow) * P.lda + ckc * 8) * 2);
  const uint32_t a_step = (uint32_t)(32 * P.lda * 2);
  uint32_t w_voff, w_step[CH_W];
  if (epi == EPI_SWIGLU) {
    // tile column j = crow + 32 i: wave column half wn = i / 4; i % 4 < 2 are
    // gate rows, the rest the matching up rows (N further down)
    w_voff = (uint32_t)(((int64_t)(tn * (BN / 2) + crow) * P.ldw + ckc * 8) * 2);
#pragma unroll
    for (int i = 0; i < CH_W; ++i)
      w_step[i] = (uint32_t)(((i / 4) * (WTN / 2) + 32 * (i % 2) + ((i % 4) >= 2 ? N : 0)) *
                             P.ldw * 2);
  } else {
    w_voff = (uint32_t)(((int64_t)(tn * BN + crow) * P.ldw + ckc * 8) * 2);
#pragma unroll
    for (int i = 0; i < CH_W; ++i) w_step[i] = (uint32_t)(i * 32 * P.ldw * 2);
  }
  const int st_off = crow * ROW_U + (ckc ^ swz(crow));

  // ---- MFMA fragment readers
  const int fr = lane & 31, fg = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;
  const int a_rd = (wm * WTM + fr) * ROW_U;
  const int w_rd = BM * ROW_U + (wn * WTN + fr) * ROW_U;
  const int sfr = swz(fr);

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

  u32x4 ra[CH_A], rw[CH_W];
  const int nk = K / BK;

#pragma unroll
  for (int i = 0; i < CH_A; ++i)
    ra[i] = __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, a_voff + i * a_step, 0, 0);
#pragma unroll
  for (int i = 0; i < CH_W; ++i)
    rw[i] = __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, w_voff + w_step[i], 0, 0);
#pragma unroll
  for (int i = 0; i < CH_A; ++i) lds[st_off + i * 32 * ROW_U] = ra[i];
#pragma unroll
  for (int i = 0; i < CH_W; ++i) lds[BM * ROW_U + st_off + i * 32 * ROW_U] = rw[i];
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const uint32_t ko = (uint32_t)(kt + 1) * (BK * 2);
#pragma unroll
      for (int i = 0; i < CH_A; ++i)
        ra[i] = __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, a_voff + i * a_step + ko, 0, 0);
#pragma unroll
      for (int i = 0; i < CH_W; ++i)
        rw[i] = __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, w_voff + w_step[i] + ko, 0, 0);
    }
    const u32x4* st = lds + cur * STAGE_U;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int ch = (2 * s + fg) ^ sfr;
      bf16x8 af[FM], wf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = __builtin_bit_cast(bf16x8, st[a_rd + i * 32 * ROW_U + ch]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        wf[j] = __builtin_bit_cast(bf16x8, st[w_rd + j * 32 * ROW_U + ch]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j], af[i], acc[i][j], 0, 0, 0);
    }
    if (more) {
      u32x4* dst = lds + (cur ^ 1) * STAGE_U;
#pragma unroll
      for (int i = 0; i < CH_A; ++i) dst[st_off + i * 32 * ROW_U] = ra[i];
#pragma unroll
      for (int i = 0; i < CH_W; ++i) dst[BM * ROW_U + st_off + i * 32 * ROW_U] = rw[i];
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds row m0 + wm*128 + i*32 + fr, columns
  //      (block j) j*32 + 8*q + 4*fg + 0..3 for q = 0..3
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int r = m0 + wm * WTM + i * 32 + fr;
    if (r >= M) continue;
    const int b = r / P.seg_len;
    const int64_t out_row = (int64_t)b * P.seg_stride + P.seg_off + (r - b * P.seg_len);
    if (epi == EPI_SWIGLU) {
#pragma unroll
      for (int j = 0; j < FN / 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = tn * (BN / 2) + wn * (WTN / 2) + j * 32 + 8 * q + 4 * fg;
          if (col >= N) continue;
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            v[e] = silu_f(acc[i][j][4 * q + e]) * acc[i][j + FN / 2][4 * q + e];
          store4(P, EPI_SWIGLU, out_row, col, b, v);
        }
    } else {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = tn * BN + wn * WTN + j * 32 + 8 * q + 4 * fg;
          if (col >= N) continue;
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
          store4(P, epi, out_row, col, b, v);
        }
    }
  }
}

}  // namespace

hipError_t gemm_launch(GemmBatch& batch, hipStream_t stream) {
  int total = 0;
  for (int i = 0; i < batch.count; ++i) {
    GemmProblem& p = batch.p[i];
    const int cols = p.epi == EPI_SWIGLU ? BN / 2 : BN;
    p.tiles_m = (p.M + BM - 1) / BM;
    p.tiles_n = (p.N + cols - 1) / cols;
    p.tile_begin = total;
    total += p.tiles_m * p.tiles_n;
  }
  for (int i = batch.count; i < kMaxGemmProblems; ++i) batch.p[i] = GemmProblem{};
  batch.total_tiles = total;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(gemm_bf16_kernel, dim3(total), dim3(NT), 0, stream, batch);
  return hipGetLastError();
}

}  // namespace dit
