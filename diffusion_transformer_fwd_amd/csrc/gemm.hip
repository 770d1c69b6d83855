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
//    gated residual x += gate[b] * acc on the fp32 residual; fp32 store; and
//    QK-RMSNorm + RoPE straight into the attention operands (a wave's 128
//    columns are one head), so the fused projection never round-trips HBM.
//    Output rows go through a (segment length, stride, offset) map, so
//    stream-major operands scatter back into x[B, S, D] in place.
//  * Up to eight independent problems share one launch (text + image
//    streams, the single block's QKV part + SwiGLU part, or the K chunks of
//    a split contraction), so the small 512-row text problem fills gaps
//    instead of taking its own launch.
//  * Launches without the SwiGLU / QKV epilogues may use 256 x 224 tiles
//    when that takes fewer rounds of tiles over the CUs (the N = 3072
//    projections at 4608 rows: 252 tiles in one round instead of 216 full
//    ones leaving 40 CUs idle).
//  * Tile order: launch index -> XCD-contiguous logical index -> groups of
//    7 row tiles walked column by column, so co-resident tiles on one XCD
//    share A and W panels in its L2.
//  * The accumulation order of an output element depends only on K, never
//    on M, the tile width or the tile position, so a batch row's results
//    are bitwise the same whatever else is in the batch.
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

// Tile order of a problem: groups of GROUP row tiles, row tile fastest, so the
// 32 tiles an XCD runs at once span about 7 row tiles x 4-5 column tiles of
// A and W panels in its L2. 7 measured best of 4..12 (0.5 % per step against
// 8 on two boxes, 6 and 5 in between).
__device__ __forceinline__ void tile_coords(int local, int tiles_m, int tiles_n,
                                            int& tm, int& tn) {
  constexpr int GROUP = 7;
  const int per_group = GROUP * tiles_n;
  const int grp = local / per_group;
  const int first = grp * GROUP;
  const int gsize = min(tiles_m - first, GROUP);
  const int in = local - grp * per_group;
  tm = first + in % gsize;
  tn = in / gsize;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <int V>
struct count_t {
  static constexpr int value = V;
};

// BNT: output columns per tile, 256 or 224 (BF16 / F32 / RESID epilogues
// only). At 224 the N = 1 waves run three 32-column blocks instead of four
// and W tile rows 224..255 are never loaded; per output element nothing
// changes (same MFMA, same k order), so the width may be picked per launch.
// EPI_QKV for one wave tile (64 rows x 128 columns = one head of q, k or v):
// a row's 128 accumulators sit in lanes l and l ^ 32 (64 each), so the RMS
// is lane-local plus one cross-half exchange; each lane's runs of 4 columns
// hold two whole rotation pairs.
template <int BNT>
__global__ __launch_bounds__(NT, 1) void gemm_bf16_kernel(const GemmBatch args) {
  // two K-slice stages, then (EPI_QKV) 1 / rms of each tile row per wave column
  __shared__ u32x4 lds[2 * STAGE_U + 2 * BM * 4 / 16];
  float (*const row_scale)[BM] = reinterpret_cast<float (*)[BM]>(lds + 2 * STAGE_U);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  int pi = 0;
#pragma unroll
  for (int i = 1; i < kMaxGemmProblems; ++i)
    if (i < args.count && L >= args.p[i].tile_begin) pi = i;
  pi = __builtin_amdgcn_readfirstlane(pi);
  // Constant-index copies keep every field in scalar registers.
  GemmProblem P;
  switch (pi) {
    case 0: P = args.p[0]; break;
    case 1: P = args.p[1]; break;
    case 2: P = args.p[2]; break;
    case 3: P = args.p[3]; break;
    case 4: P = args.p[4]; break;
    case 5: P = args.p[5]; break;
    case 6: P = args.p[6]; break;
    default: P = args.p[7]; break;
  }
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
        wrow = (int64_t)tn * BNT + 32 * wb + lr;
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
      if (BNT == 224 && wave - 4 * h == 7) continue;  // W rows 224..255: not in the tile
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
  // FNA (a compile-time count): the wave's active 32-column blocks
  auto fload = [&](auto fna, int stage, int s, int buf) {
    constexpr int FNA = decltype(fna)::value;
    const u32x4* st = lds + stage * STAGE_U;
    const int ch = (2 * s + fg) ^ sfr;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      af[buf][i] = __builtin_bit_cast(bf16x8, st[a_rd + i * 32 * ROW_U + ch]);
#pragma unroll
    for (int j = 0; j < FNA; ++j)
      wf[buf][j] = __builtin_bit_cast(bf16x8, st[w_rd + j * 32 * ROW_U + ch]);
  };
  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};
  auto mfmas = [&](auto fna, int buf) {
    constexpr int FNA = decltype(fna)::value;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FNA; ++j)
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
    // a loader's loads of slice 1 may fly (16, or 12 for the wave that skips W rows 224..255)
    if (BNT == 224 && wave == 7) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();
  auto main_loop = [&](auto fna) {
    fload(fna, 0, 0, 0);
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
#pragma unroll
      for (int s = 0; s < BK / 16 - 1; ++s) {
        fload(fna, cur, s + 1, (s + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(fna, s & 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      // everyone is done with this stage and slice kt + 1 has landed
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
      __syncthreads();
      if (kt + 2 < nk) dma(kt + 2, cur);
      if (kt + 1 < nk) fload(fna, cur ^ 1, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      mfmas(fna, (BK / 16 - 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if (BNT == 224 && wn == 1) main_loop(count_t<FN - 1>{});
  else main_loop(count_t<FN>{});

  // ---- epilogue. Lane holds row wm*64 + i*32 + fr of the tile, columns
  // (block j) wn*128 + j*32 + 8*q + 4*fg + 0..3 for q = 0..3. Results are
  // staged in LDS (free now: every fragment read of the loop happened before
  // its last barrier) and leave in whole rows, 16 bytes per lane: stores
  // straight from the MFMA layout would be 16-byte pieces of 32 rows per
  // instruction. Every wave reaches every barrier below.
  char* const T = reinterpret_cast<char*>(lds);
  // bf16 stage [256][256]: 16-byte chunk c of row r at c ^ (r & 31)
  auto stage_bf16 = [&](int r, int col, f32x4 v) {
    *reinterpret_cast<u32x2*>(T + r * 512 + (((col >> 3) ^ (r & 31)) << 4) + ((col & 4) << 1)) =
        pack_bf16x4(v);
  };
  auto out_row_of = [&](int gr, int& b) -> int64_t {
    b = gr / P.seg_len;
    return (int64_t)b * P.seg_stride + P.seg_off + (gr - b * P.seg_len);
  };

  if (epi == EPI_F32 || epi == EPI_RESID) {
    // fp32 stage [128][256] per pass (rows 128 p ..), 16-byte chunk c of row r at c ^ (r & 31)
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      if ((wm >> 1) == pass) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int r = (wm & 1) * WTM + i * 32 + fr;
              const int c = (wn * WTN + j * 32 + 8 * q + 4 * fg) >> 2;
              f32x4 v;
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
              *reinterpret_cast<f32x4*>(T + r * 1024 + ((c ^ (r & 31)) << 4)) = v;
            }
      }
      __syncthreads();
      // 16-byte unit u = it * NT + tid: row u / 64 = 8 it + wave, chunk
      // u % 64 = lane. The residual and gate reads of 8 rows are issued
      // together before any store (a store could alias a later read, so the
      // compiler would not move reads above it), one memory latency per 8 rows.
      const int c = lane, col = tn * BNT + c * 4;
      const bool col_ok = c * 4 < BNT && col < N;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float* dst[8];
        f32x4 x[8], g[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int r = 8 * (8 * half + k) + wave;
          const int gr = m0 + pass * 128 + r;
          dst[k] = nullptr;
          if (col_ok && gr < M) {
            int b;
            dst[k] = static_cast<float*>(P.C) + out_row_of(gr, b) * P.ldc + col;
            if (epi == EPI_RESID) {
              g[k] = *reinterpret_cast<const f32x4*>(P.gate + (int64_t)b * P.gate_bstride + col);
              x[k] = *reinterpret_cast<const f32x4*>(dst[k]);
            }
          }
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int r = 8 * (8 * half + k) + wave;
          if (dst[k] == nullptr) continue;
          const f32x4 v = *reinterpret_cast<const f32x4*>(T + r * 1024 + ((c ^ (r & 31)) << 4));
          *reinterpret_cast<f32x4*>(dst[k]) = epi == EPI_RESID ? x[k] + g[k] * v : v;
        }
      }
      __syncthreads();
    }
    return;
  }

  // bf16 results: phase A, values into the stage
  if (epi == EPI_SWIGLU) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN / 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            v[e] = silu_f(acc[i][j][4 * q + e]) * acc[i][j + FN / 2][4 * q + e];
          stage_bf16(wm * WTM + i * 32 + fr, wn * (WTN / 2) + j * 32 + 8 * q + 4 * fg, v);
        }
  } else if (epi == EPI_QKV && tn * BN + wn * WTN < N && (tn * BN + wn * WTN) / args.qkv.D < 2) {
    // q or k head (the wave's 128 columns): the row's 1 / rms (times q_scale
    // for q) from the fp32 accumulators, kept per row in LDS; a row's 128
    // values sit in lanes l and l ^ 32, so the sum of squares needs one
    // cross-half exchange. The values are staged raw; gain and rotation are
    // applied on the way out, where 16 lanes share a token row.
    const QkvEpilogue& E = args.qkv;
    const float sc = (tn * BN + wn * WTN) / E.D == 0 ? E.q_scale : 1.f;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) ss += acc[i][j][e] * acc[i][j][e];
      ss = half_sum(ss);
      if (fg == 0) row_scale[wn][wm * WTM + i * 32 + fr] = rsqrtf(ss * (1.f / 128.f) + E.eps) * sc;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
          stage_bf16(wm * WTM + i * 32 + fr, wn * WTN + j * 32 + 8 * q + 4 * fg, v);
        }
    }
  } else {
    // plain bf16 (also the v heads of EPI_QKV)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
          stage_bf16(wm * WTM + i * 32 + fr, wn * WTN + j * 32 + 8 * q + 4 * fg, v);
        }
  }
  __syncthreads();

  // phase B: whole rows out, 16 bytes per lane
  if (epi != EPI_QKV) {
    const int ncol = epi == EPI_SWIGLU ? BN / 2 : BNT;  // output columns of the tile
    const int upr = ncol / 8;                          // 16-byte units per row
#pragma unroll 4
    for (int it = 0; it < 256 * (BN / 8) / NT; ++it) {
      const int u = it * NT + tid;
      if (u >= 256 * upr) break;
      const int r = u / upr, c = u - r * upr;
      const int gr = m0 + r, col = tn * ncol + c * 8;
      if (gr >= M || col >= N) continue;
      int b;
      *reinterpret_cast<u32x4*>(static_cast<bf16_t*>(P.C) + out_row_of(gr, b) * P.ldc + col) =
          *reinterpret_cast<const u32x4*>(T + r * 512 + ((c ^ (r & 31)) << 4));
    }
    return;
  }
  // EPI_QKV: per 128-column head of the tile: q / k rows to [b, h, s, :]
  // (16 lanes per token), v gathered 8 tokens per dim to v^T[b, h, d, s..s+7]
  const QkvEpilogue& E = args.qkv;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int col0 = tn * BN + hh * 128;
    if (col0 >= N) break;
    const int part = col0 / E.D;
    const int h = (col0 - part * E.D) >> 7;
    if (part < 2) {
      // 16 lanes per token row, 8 columns (4 rotation pairs) per lane
      bf16_t* base = part == 0 ? E.q : E.k;
      const float* gain = part == 0 ? E.q_gain[pi] : E.k_gain[pi];
      const int cl = (tid & 15) * 8;  // column within the head
      const f32x4 g0 = *reinterpret_cast<const f32x4*>(gain + cl);
      const f32x4 g1 = *reinterpret_cast<const f32x4*>(gain + cl + 4);
#pragma unroll 4
      for (int it = 0; it < 256 * 16 / NT; ++it) {
        const int u = it * NT + tid;
        const int r = u >> 4, c = hh * 16 + (u & 15);
        const int gr = m0 + r;
        if (gr >= M) continue;
        const int b = gr / P.seg_len;
        const int s = P.seg_off + (gr - b * P.seg_len);
        const u32x4 raw = *reinterpret_cast<const u32x4*>(T + r * 512 + ((c ^ (r & 31)) << 4));
        const float rsc = row_scale[hh][r];
        const f32x4 co = *reinterpret_cast<const f32x4*>(E.cos_t + (int64_t)s * 64 + (cl >> 1));
        const f32x4 si = *reinterpret_cast<const f32x4*>(E.sin_t + (int64_t)s * 64 + (cl >> 1));
        f32x8 y;
#pragma unroll
        for (int pr = 0; pr < 4; ++pr) {
          const float gx0 = pr < 2 ? g0[2 * pr] : g1[2 * pr - 4];
          const float gx1 = pr < 2 ? g0[2 * pr + 1] : g1[2 * pr - 3];
          const float x0 = bf16_to_f32(raw[pr] & 0xFFFFu) * rsc * gx0;
          const float x1 = bf16_to_f32(raw[pr] >> 16) * rsc * gx1;
          y[2 * pr] = x0 * co[pr] - x1 * si[pr];
          y[2 * pr + 1] = x0 * si[pr] + x1 * co[pr];
        }
        *reinterpret_cast<bf16x8*>(base + (((int64_t)b * E.H + h) * E.S_pad + s) * 128 + cl) =
            pack_bf16x8(y);
      }
    } else {
#pragma unroll 2
      for (int it = 0; it < 128 * 32 / NT; ++it) {
        const int u = it * NT + tid;
        const int d = u & 127, tg = u >> 7;  // dim, group of 8 tokens
        const int colb = ((hh * 128 + d) >> 3), wb = (d & 7) << 1;
        uint16_t tok[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = tg * 8 + e;
          tok[e] = *reinterpret_cast<const uint16_t*>(T + r * 512 + ((colb ^ (r & 31)) << 4) + wb);
        }
        const int r0 = m0 + tg * 8;
        if (r0 >= M) continue;
        const int b0 = r0 / P.seg_len;
        const int s0 = P.seg_off + (r0 - b0 * P.seg_len);
        if (r0 + 7 < M && (r0 + 7) / P.seg_len == b0 && (s0 & 7) == 0) {
          u32x4 pk;
#pragma unroll
          for (int e = 0; e < 4; ++e) pk[e] = (uint32_t)tok[2 * e] | ((uint32_t)tok[2 * e + 1] << 16);
          *reinterpret_cast<u32x4*>(E.vt + (((int64_t)b0 * E.H + h) * 128 + d) * E.S_pad + s0) = pk;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int gr = r0 + e;
            if (gr >= M) break;
            const int b = gr / P.seg_len;
            const int s = P.seg_off + (gr - b * P.seg_len);
            E.vt[(((int64_t)b * E.H + h) * 128 + d) * E.S_pad + s] = tok[e];
          }
        }
      }
    }
  }
}

// Compute units of the current device (cached per device).
int device_cus() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Tile counts of every problem for tile width bnt; returns the total.
int64_t assign_tiles(GemmBatch& batch, int bnt) {
  int64_t total = 0;
  for (int i = 0; i < batch.count; ++i) {
    GemmProblem& p = batch.p[i];
    const int cols = p.epi == EPI_SWIGLU ? BN / 2 : bnt;
    p.tiles_m = (p.M + BM - 1) / BM;
    p.tiles_n = (p.N + cols - 1) / cols;
    p.tile_begin = (int32_t)total;
    total += (int64_t)p.tiles_m * p.tiles_n;
  }
  return total;
}

}  // namespace

hipError_t gemm_launch(GemmBatch& batch, hipStream_t stream) {
  for (int i = batch.count; i < kMaxGemmProblems; ++i) batch.p[i] = GemmProblem{};
  // Tile width: 224 instead of 256 when every epilogue allows it and the
  // launch then takes fewer rounds x per-tile time. A 224-wide tile does 7/8
  // of the MFMA work but loads 15/16 of the bytes, and the loads bound it,
  // so its time counts as 15/16. E.g. N = 3072 at M = 4608: 216 tiles of 256
  // leave 40 of 256 CUs idle for the whole launch, 252 tiles of 224 finish
  // in one shorter round; N = 27648 keeps 256 (8 rounds against 9 x 15/16).
  bool narrow_ok = true;
  for (int i = 0; i < batch.count; ++i)
    if (batch.p[i].epi == EPI_SWIGLU || batch.p[i].epi == EPI_QKV) narrow_ok = false;
  int bnt = BN;
  if (narrow_ok) {
    const int64_t cus = device_cus();
    const int64_t r256 = (assign_tiles(batch, 256) + cus - 1) / cus;
    const int64_t r224 = (assign_tiles(batch, 224) + cus - 1) / cus;
    if (r224 * 15 < r256 * 16) bnt = 224;
  }
  const int64_t total = assign_tiles(batch, bnt);
  if (total > INT32_MAX) return hipErrorInvalidValue;
  batch.total_tiles = (int32_t)total;
  if (total == 0) return hipSuccess;
  if (bnt == 224)
    hipLaunchKernelGGL(gemm_bf16_kernel<224>, dim3((unsigned)total), dim3(NT), 0, stream, batch);
  else
    hipLaunchKernelGGL(gemm_bf16_kernel<256>, dim3((unsigned)total), dim3(NT), 0, stream, batch);
  return hipGetLastError();
}

}  // namespace dit
