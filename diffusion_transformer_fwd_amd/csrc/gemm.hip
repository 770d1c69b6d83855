// bf16 GEMM on gfx950 MFMA with fused epilogues: C = A W^T.
//
// This carries every dense contraction of the step: the QKV / output / MLP
// projections of the dual-stream blocks, the fused input (QKV + SwiGLU) and
// output projections of the single-stream blocks, the two embeddings and
// the final projection ("tt_flux2_klein - Python reference", Modules: the
// DiT's 5 dual + 20 single blocks; the block maths is stated in dit.h).
//
// Design (one workgroup = 8 waves = 512 threads, one 256 x 256 output tile):
//  * A [M, K] and W [N, K] are both K-contiguous, so one 64-wide K slice of
//    each tile is a set of 128-byte row segments. Slices go from HBM/L2
//    straight into LDS with buffer loads that write LDS (no register
//    staging, no LDS store instructions), their 16-byte chunks XOR-swizzled
//    by row so that MFMA fragment reads are free of bank conflicts. Two LDS
//    stages (128 KiB of the CU's 160 KiB), one barrier per slice; fragments
//    for the next 16-wide k-step are read while the current one's MFMAs run.
//    A CU pulls about 36 bytes per clock from L2 into LDS this way, close to
//    the 32 B/clk a 256 x 256 tile consumes at the full MFMA rate, so the
//    loads must overlap the math: the tile runs 8 waves (two per SIMD) and
//    only the upper four issue loads, while the lower four keep issuing
//    MFMAs.
//  * Each wave owns a 64 x 128 sub-tile (4 x 2 waves) as 2 x 4 blocks of
//    v_mfma_f32_32x32x16_bf16 (fp32 accumulators, 128 per lane). The weight
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
constexpr int NT = 512;                       // 8 waves, two per SIMD
constexpr int WTM = 64, WTN = 128;            // wave tile: 4 x 2 waves
constexpr int FM = WTM / 32, FN = WTN / 32;
constexpr int ROW_U = BK / 8;                 // 16-byte units per LDS row
constexpr int STAGE_U = (BM + BN) * ROW_U;    // 16-byte units per stage

static_assert(NT == 512 && BM == 256 && BN == 256, "loader assumes 8 waves x 32 rows");

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

typedef __attribute__((address_space(3))) void* lds_ptr_t;

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

  // ---- global -> LDS: buffer loads that write LDS directly (no register
  // staging). Waves 4-7 issue every load of a slice: wave w fills tile rows
  // 32 w' .. 32 w' + 31 of A and of W for w' = w and w' = w - 4, four
  // instructions of 8 rows each per block of 32 rows. Waves 0-3 issue none,
  // so their MFMAs never queue behind a load issue that waits for room in the
  // CU's vector-memory queue, and each SIMD (one wave of either half) keeps
  // its matrix core busy. A lane writes physical chunk lane % 8 of its row,
  // so it fetches logical chunk (lane % 8) ^ swz(row). Rows past the end of
  // A or W read as zero.
  const int w_rows = epi == EPI_SWIGLU ? 2 * N : N;
  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(P.A, clamp_u32((int64_t)M * P.lda * 2));
  const __amdgpu_buffer_rsrc_t w_rsrc = make_rsrc(P.W, clamp_u32((int64_t)w_rows * P.ldw * 2));
  const int lr = lane >> 3, lp = lane & 7;
  const bool loader = wave >= 4;
  uint32_t a_off[2][2], w_off[2][2];  // [row block h: w' = wave - 4 h][row parity]
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int wb = wave - 4 * h;  // row block 32 wb .. 32 wb + 31
      const int c = lp ^ (lr ^ par);
      a_off[h][par] = (uint32_t)(((int64_t)(m0 + 32 * wb + lr) * P.lda + c * 8) * 2);
      // SwiGLU: tile row j = 32 wb + r belongs to wave column group j / 128 =
      // wb / 4; rows with (wb % 4) < 2 are gate rows, the others the matching
      // up rows (N further down), so each wave's 128 output columns hold gate
      // and up values of the same 64 activations
      int64_t wrow;
      if (epi == EPI_SWIGLU)
        wrow = tn * (BN / 2) + (wb >> 2) * 64 + 32 * (wb & 1) + lr + (((wb & 3) >= 2) ? N : 0);
      else
        wrow = (int64_t)tn * BN + 32 * wb + lr;
      w_off[h][par] = (uint32_t)((wrow * P.ldw + c * 8) * 2);
    }
  const uint32_t a_istep = (uint32_t)(8 * P.lda * 2), w_istep = (uint32_t)(8 * P.ldw * 2);
  auto dma = [&](int kt, int stage) {
    if (!loader) return;
    const uint32_t ko = (uint32_t)kt * (BK * 2);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4* base = lds + stage * STAGE_U + (wave - 4 * h) * 32 * ROW_U;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_ptr_t)(base + i * 64), 16,
                                                 a_off[h][i & 1] + i * a_istep + ko, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(w_rsrc, (lds_ptr_t)(base + BM * ROW_U + i * 64),
                                                 16, w_off[h][i & 1] + i * w_istep + ko, 0, 0, 0);
    }
  };

  // ---- MFMA fragments, double-buffered across k-steps
  const int fr = lane & 31, fg = lane >> 5;
  const int wm = wave & 3, wn = wave >> 2;
  const int a_rd = (wm * WTM + fr) * ROW_U;
  const int w_rd = BM * ROW_U + (wn * WTN + fr) * ROW_U;
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
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[buf][j], af[buf][i], acc[i][j],
                                                            0, 0, 0);
  };

  // Two LDS stages. Slice kt + 2 is fetched while kt + 1 is in flight and kt
  // is consumed; one barrier per slice, placed before the slice's last
  // k-step so that k-step's MFMAs (operands already in registers) cover the
  // first fragment reads of the next slice. Scheduling barriers keep each
  // k-step's fragment reads ahead of the previous k-step's MFMAs.
  const int nk = K / BK;
  dma(0, 0);
  if (nk > 1) {
    dma(1, 1);
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");  // a loader's 16 loads of slice 1 may fly
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();
  fload(0, 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
#pragma unroll
    for (int s = 0; s < BK / 16 - 1; ++s) {
      fload(cur, s + 1, (s + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
      mfmas(s & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // everyone is done with this stage and slice kt + 1 has landed
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();
    if (kt + 2 < nk) dma(kt + 2, cur);
    if (kt + 1 < nk) fload(cur ^ 1, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    mfmas((BK / 16 - 1) & 1);
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- epilogue: lane holds row m0 + wm*64 + i*32 + fr, columns
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
