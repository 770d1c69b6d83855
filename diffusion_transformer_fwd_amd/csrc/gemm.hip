// bf16 GEMM on gfx950 MFMA with fused epilogues: C = A W^T.
//
// This carries every dense contraction of the step: the QKV / output / MLP
// projections of the dual-stream blocks, the fused input (QKV + SwiGLU) and
// output projections of the single-stream blocks, the two embeddings and
// the final projection ("tt_flux2_klein - Python reference", Modules: the
// DiT's 5 dual + 20 single blocks; the block maths is stated in dit.h).
//
// Design (one workgroup = 8 waves = 512 threads, one output tile of 256 or
// 384 rows by 256 columns):
//  * A [M, K] and W [N, K] are both K-contiguous, so one 64-wide K slice of
//    each tile is a set of 128-byte row segments. Slices go from HBM/L2
//    straight into LDS with buffer loads that write LDS (no register
//    staging, no LDS store instructions), their 16-byte chunks XOR-swizzled
//    by row so that MFMA fragment reads are free of bank conflicts. Two LDS
//    stages, one barrier per slice; fragments are read ahead of the MFMAs
//    that use them (two k-steps ahead, one read after each MFMA, in 256-row
//    full-width tiles; one k-step ahead elsewhere).
//  * What paces a slice is the stream of slice bytes from L2 into the CU
//    (about 23 bytes per clock under full MFMA load), not the matrix cores:
//    a 256 x 256 tile needs 32 B/clk to keep them busy. A 384-row tile does
//    1.5x the MFMA work of a 256-row one for 1.25x the bytes (80 KiB per
//    slice; the two stages fill the 160 KiB LDS), so launches use 384-row
//    tiles wherever the rounds of tiles over the CUs allow it.
//  * Loads overlap the math: the tile runs 8 waves (two per SIMD) and only
//    the upper four issue loads, while the lower four keep issuing MFMAs
//    (a wave that issues loads stalls while the CU's load queue is full).
//    In the main loop the loader waves run at a raised wave priority.
//  * Each wave owns a (32 FM) x 128 sub-tile (4 x 2 waves, FM = 2 or 3) as
//    FM x 4 blocks of v_mfma_f32_32x32x16_bf16 (fp32 accumulators, 16 FM
//    per lane per block column). The weight fragment is the MFMA's first
//    operand and the activation fragment the second, so each lane ends up
//    holding one output row and runs of four consecutive output columns.
//  * Epilogues: bf16 store; SwiGLU (each wave's column half is gate rows and
//    the other half the matching up rows, so SiLU(g) * u is lane-local);
//    gated residual x += gate[b] * acc on the fp32 residual; fp32 store; and
//    QK-RMSNorm + RoPE straight into the attention operands (a wave's 128
//    columns are one head), so the fused projection never round-trips HBM.
//    Results are staged through LDS in passes of whole rows and leave 16
//    bytes per lane. Output rows go through a (segment length, stride,
//    offset) map, so stream-major operands scatter back into x[B, S, D].
//  * Up to eight independent problems share one launch (text + image
//    streams, the single block's QKV part + SwiGLU part, or the K chunks of
//    a split contraction); each problem has its own tile height.
//  * Launches without the SwiGLU / QKV epilogues may use 224-wide tiles
//    when that takes fewer rounds of tiles over the CUs (the N = 3072
//    projections at 4608 rows: 252 tiles in one round instead of 216 full
//    ones leaving 40 CUs idle).
//  * Tile order: every problem's tiles are dealt to the 8 XCDs in
//    contiguous ranges (tile_map.hpp), so each XCD runs the same mix of
//    tile sizes, larger first, and co-resident tiles on one XCD share A and
//    W panels in its L2; inside a problem, groups of 7 row tiles are walked
//    column by column.
//  * The accumulation order of an output element depends only on K, never
//    on M, the tile shape or the tile position (every tile runs the same
//    MFMA over the same 16-wide k-steps in order), so a batch row's results
//    are bitwise the same whatever else is in the batch.
#include <algorithm>
#include <cstdlib>
#include <map>
#include <mutex>
#include <tuple>
#include <vector>

#include "common.hpp"
#include "kernels.hpp"
#include "tile_map.hpp"
#include "attention_unit.hpp"

namespace dit {
namespace {

constexpr int BN = kGemmBN, BK = kGemmBK;
constexpr int NT = 512;                       // 8 waves, two per SIMD
constexpr int WTN = 128, FN = WTN / 32;       // wave tile columns; 4 x 2 waves
constexpr int ROW_U = BK / 8;                 // 16-byte units per LDS row
constexpr int MAX_BM = 384;
constexpr int LDS_U = 2 * (MAX_BM + BN) * ROW_U;     // two stages of the tallest tile
constexpr int RS_BYTE = LDS_U * 16 - 2 * MAX_BM * 4; // epilogue row scales, [2][BM]

static_assert(NT == 512 && BN == 256 && BK == 64, "loader assumes 8 waves x 32 rows");
static_assert(LDS_U * 16 == 160 * 1024, "two 384-row stages fill the LDS");

// Chunk swizzle by row: distinct for 8 consecutive rows and for the 8 rows of
// either parity among 16 consecutive rows.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// Tile order of a problem: groups of GROUP row tiles, row tile fastest, so the
// tiles an XCD runs at once span a few row tiles x a few column tiles of A and
// W panels in its L2. 7 measured best of 4..12 (0.5 % per step against 8 on
// two boxes, 6 and 5 in between).
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

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// One output tile of problem P (index pi of the launch): BM = 128 FM rows,
// BNT columns (256, or 224 for the BF16 / F32 / RESID epilogues only: the
// N = 1 waves then run three 32-column blocks instead of four and W tile
// rows 224..255 are never loaded; per output element nothing changes).
// EPI_QKV for one wave tile (32 FM rows x 128 columns = one head of q, k or
// v): a row's 128 accumulators sit in lanes l and l ^ 32 (64 each), so the
// RMS is lane-local plus one cross-half exchange; each lane's runs of 4
// columns hold two whole rotation pairs.
// FAM: the epilogue family of a launch, FAM_F32 (EPI_F32 / EPI_RESID) or
// FAM_BF16 (EPI_BF16 / EPI_SWIGLU / EPI_QKV): one kernel per family. EK: the
// epilogue code a tile instantiation carries (EK_F32, EK_QKV, or EK_BF16 for
// EPI_BF16 / EPI_SWIGLU); each has its own copy of the main loop, which keeps
// every instantiation's registers within the budget at 384 rows.
enum { FAM_BF16 = 0, FAM_F32 = 1 };
enum { EK_BF16 = 0, EK_QKV = 1, EK_F32 = 2 };

template <int BNT, int FM, int EK>
__device__ __forceinline__ void gemm_tile(const GemmBatch& args, const GemmProblem& P, int pi,
                                          int local, u32x4* lds) {
  constexpr int BM = 128 * FM, WTM = 32 * FM;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int M = P.M, N = P.N, K = P.K, epi = P.epi;
  int tm, tn;
  tile_coords(local, P.tiles_m, P.tiles_n, tm, tn);
  const int m0 = tm * BM;

  // ---- global -> LDS: buffer loads that write LDS directly (no register
  // staging). Waves 4-7 issue every load of a slice: loader lw = wave - 4
  // fills the 32-row blocks lw + 4 h of A (h < FM) and of W (h < 2), four
  // instructions of 8 rows each per block. Waves 0-3 issue none, so their
  // MFMAs never queue behind a load issue that waits for room in the CU's
  // vector-memory queue, and each SIMD (one wave of either half) keeps its
  // matrix core busy. A lane writes physical chunk lane % 8 of its row, so
  // it fetches logical chunk (lane % 8) ^ swz(row). Rows past the end of A
  // or W read as zero.
  const int w_rows = epi == EPI_SWIGLU ? 2 * N : N;
  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(P.A, clamp_u32((int64_t)M * P.lda * 2));
  const __amdgpu_buffer_rsrc_t w_rsrc = make_rsrc(P.W, clamp_u32((int64_t)w_rows * P.ldw * 2));
  const int lr = lane >> 3, lp = lane & 7;
  const bool loader = wave >= 4;
  const int lw = wave - 4;
  // lane part of a load's byte offset (row lr of an 8-row group, logical
  // chunk (lane % 8) ^ swz(row) of the row, which depends on the row's
  // parity); everything else is wave-uniform and goes to the scalar offset
  uint32_t a_lane[2], w_lane[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int c = lp ^ (lr ^ par);
    a_lane[par] = (uint32_t)((lr * P.lda + c * 8) * 2);
    w_lane[par] = (uint32_t)((lr * P.ldw + c * 8) * 2);
  }
  // first row of W tile block wb (32 rows): SwiGLU tile row j = 32 wb + r
  // belongs to wave column group j / 128 = wb / 4; rows with (wb % 4) < 2 are
  // gate rows, the others the matching up rows (N further down), so each
  // wave's 128 output columns hold gate and up values of the same 64
  // activations
  auto w_row0 = [&](int wb) -> int64_t {
    if (epi == EPI_SWIGLU)
      return (int64_t)tn * (BN / 2) + (wb >> 2) * 64 + 32 * (wb & 1) + (((wb & 3) >= 2) ? N : 0);
    return (int64_t)tn * BNT + 32 * wb;
  };
  const uint32_t a_row_b = (uint32_t)(P.lda * 2), w_row_b = (uint32_t)(P.ldw * 2);
  auto dma = [&](int kt, int stage) {
    if (!loader) return;
    const uint32_t ko = (uint32_t)kt * (BK * 2);
    u32x4* const sa = lds + stage * (BM * ROW_U);
    u32x4* const sw = lds + 2 * BM * ROW_U + stage * (BN * ROW_U);
    // The whole byte offset goes in the vector offset, which the buffer's
    // range check covers (rows past the operand read as zero); its
    // wave-uniform part is a running sum, 8 rows per instruction.
#pragma unroll
    for (int h = 0; h < FM; ++h) {
      const int row = 32 * (lw + 4 * h);  // first tile row of the block
      uint32_t so = __builtin_amdgcn_readfirstlane((uint32_t)(m0 + row) * a_row_b + ko);
#pragma unroll
      for (int i = 0; i < 4; ++i, so += 8 * a_row_b)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_ptr_t)(sa + (row + 8 * i) * ROW_U),
                                                 16, a_lane[i & 1] + so, 0, 0, 0);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int wb = lw + 4 * h;
      if (BNT == 224 && wb == 7) continue;  // W rows 224..255: not in the tile
      uint32_t so = __builtin_amdgcn_readfirstlane((uint32_t)w_row0(wb) * w_row_b + ko);
#pragma unroll
      for (int i = 0; i < 4; ++i, so += 8 * w_row_b)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(w_rsrc,
                                                 (lds_ptr_t)(sw + (32 * wb + 8 * i) * ROW_U), 16,
                                                 w_lane[i & 1] + so, 0, 0, 0);
    }
  };

  // ---- MFMA fragments. 256-row tiles double-buffer both operands across
  // k-steps (at full width the main loop keeps four buffers instead, below);
  // 384-row tiles (192 accumulators per lane) double-buffer A only and
  // refetch each W fragment right after its last MFMA of the k-step.
  constexpr int WB = FM == 2 ? 2 : 1;  // W fragment buffers
  const int fr = lane & 31, fg = lane >> 5;
  const int wm = wave & 3, wn = wave >> 2;
  // LDS: A stage 0 | A stage 1 | W stage 0 | W stage 1 (rows of 8 units),
  // so one base per operand and k-step reaches either stage and every row
  // block through the read's immediate offset
  const int a_rd = (wm * WTM + fr) * ROW_U;
  const int w_rd = 2 * BM * ROW_U + (wn * WTN + fr) * ROW_U;
  const int sfr = swz(fr);
  bf16x8 af[2][FM], wf[WB][FN];
  // FNA (a compile-time count): the wave's active 32-column blocks
  auto fload = [&](auto fna, int stage, int s, int buf) {
    constexpr int FNA = decltype(fna)::value;
    const u32x4* sa = lds + stage * (BM * ROW_U);
    const u32x4* sw = lds + stage * (BN * ROW_U);
    const int ch = (2 * s + fg) ^ sfr;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      af[buf][i] = __builtin_bit_cast(bf16x8, sa[a_rd + i * 32 * ROW_U + ch]);
#pragma unroll
    for (int j = 0; j < FNA; ++j)
      wf[buf % WB][j] = __builtin_bit_cast(bf16x8, sw[w_rd + j * 32 * ROW_U + ch]);
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
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[buf % WB][j], af[buf][i],
                                                            acc[i][j], 0, 0, 0);
  };
  // 384-row tiles: k-step with fragments A in af[buf], W in wf[0]; with
  // `more`, the next k-step's fragments (k-step s of `stage`) are read
  // meanwhile: A into af[buf ^ 1] first, then each W fragment right after
  // the last MFMA that reads its register.
  auto kstep_rolling = [&](auto fna, int buf, bool more, int stage, int s) {
    constexpr int FNA = decltype(fna)::value;
    const u32x4* sa = lds + stage * (BM * ROW_U);
    const u32x4* sw = lds + stage * (BN * ROW_U);
    const int ch = (2 * s + fg) ^ sfr;
    if (more) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[buf ^ 1][i] = __builtin_bit_cast(bf16x8, sa[a_rd + i * 32 * ROW_U + ch]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < FNA; ++j) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[0][j], af[buf][i], acc[i][j],
                                                            0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (more) wf[0][j] = __builtin_bit_cast(bf16x8, sw[w_rd + j * 32 * ROW_U + ch]);
      __builtin_amdgcn_sched_barrier(0);
    }
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
    // a loader's loads of slice 1 may fly: 4 FM + 8 instructions, 4 fewer for
    // the wave that skips W rows 224..255
    if (BNT == 224 && wave == 7) wait_vmcnt<4 * FM + 4>();
    else wait_vmcnt<4 * FM + 8>();
  } else {
    wait_vmcnt<0>();
  }
  __syncthreads();
  auto main_loop = [&](auto fna) {
    if constexpr (FM == 2 && BNT == BN) {
      // 256-row tiles at full width (the only shape whose registers allow
      // it without spills): fragments two k-steps ahead in four buffers, one
      // per k-step of a slice, each k-step's six reads issued one after each
      // of its first MFMAs, so a read has a k-step and a half of MFMAs
      // before its use even when all eight waves read at once. The slice
      // barrier sits before k-step 2: k-step 2 and 3's fragments were read
      // (and waited for) before it, so after it slice kt's stage takes the
      // loads of slice kt + 2. Same MFMAs in the same k order as below.
      constexpr int FNA = decltype(fna)::value;
      bf16x8 af4[4][FM], wf4[4][FNA];
      auto read_all = [&](int stage, int s, int buf) {
        const u32x4* sa = lds + stage * (BM * ROW_U);
        const u32x4* sw = lds + stage * (BN * ROW_U);
        const int ch = (2 * s + fg) ^ sfr;
#pragma unroll
        for (int i = 0; i < FM; ++i)
          af4[buf][i] = __builtin_bit_cast(bf16x8, sa[a_rd + i * 32 * ROW_U + ch]);
#pragma unroll
        for (int j = 0; j < FNA; ++j)
          wf4[buf][j] = __builtin_bit_cast(bf16x8, sw[w_rd + j * 32 * ROW_U + ch]);
      };
      // the MFMAs on buffer buf; with RD, k-step s of `stage` read into
      // buffer rb, one fragment after each MFMA
      auto kstep = [&](int buf, auto rdc, int stage, int s, int rb) {
        constexpr bool RD = decltype(rdc)::value;
        const u32x4* sa = lds + stage * (BM * ROW_U);
        const u32x4* sw = lds + stage * (BN * ROW_U);
        const int ch = (2 * s + fg) ^ sfr;
#pragma unroll
        for (int t = 0; t < FM * FNA; ++t) {
          const int i = t / FNA, j = t % FNA;
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf4[buf][j], af4[buf][i],
                                                              acc[i][j], 0, 0, 0);
          if constexpr (RD) {
            if (t < FM)
              af4[rb][t] = __builtin_bit_cast(bf16x8, sa[a_rd + t * 32 * ROW_U + ch]);
            else if (t < FM + FNA)
              wf4[rb][t - FM] = __builtin_bit_cast(bf16x8, sw[w_rd + (t - FM) * 32 * ROW_U + ch]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      using T = std::true_type;
      // MORE: a slice kt + 1 exists
      auto slice = [&](int kt, auto morec) {
        constexpr bool MORE = decltype(morec)::value;
        const int cur = kt & 1;
        kstep(0, T{}, cur, 2, 2);
        kstep(1, T{}, cur, 3, 3);
        // every read of this stage is done and slice kt + 1 has landed
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __syncthreads();
        if (MORE && kt + 2 < nk) dma(kt + 2, cur);
        kstep(2, morec, cur ^ 1, 0, 0);
        kstep(3, morec, cur ^ 1, 1, 1);
      };
      read_all(0, 0, 0);
      read_all(0, 1, 1);
      int kt = 0;
      for (; kt + 1 < nk; ++kt) slice(kt, T{});
      slice(kt, std::false_type{});
      return;
    }
    fload(fna, 0, 0, 0);
    if (FM == 3) {
      for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
#pragma unroll
        for (int s = 0; s < BK / 16 - 1; ++s) kstep_rolling(fna, s & 1, true, cur, s + 1);
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __syncthreads();
        if (kt + 2 < nk) dma(kt + 2, cur);
        kstep_rolling(fna, (BK / 16 - 1) & 1, kt + 1 < nk, cur ^ 1, 0);
      }
      return;
    }
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
  // The loader waves issue at a higher priority than the compute-only wave
  // sharing their SIMD, so a loader's fragment reads, slice loads and MFMAs
  // go first when both waves are ready (same box: 29.89 -> 29.59 ms per
  // 1024^2 step; raising it only around the slice loads, or for the other
  // waves, gained nothing). Back to the default for the epilogue.
  if (loader) __builtin_amdgcn_s_setprio(1);
  if (BNT == 224 && wn == 1) main_loop(count_t<FN - 1>{});
  else main_loop(count_t<FN>{});
  __builtin_amdgcn_s_setprio(0);

  // ---- epilogue. Lane holds rows wm*WTM + i*32 + fr of the tile (i < FM),
  // columns (block j) wn*128 + j*32 + 8*q + 4*fg + 0..3 for q = 0..3. Results
  // are staged in LDS (free now: every fragment read of the loop happened
  // before its last barrier) in passes of whole rows and leave 16 bytes per
  // lane: stores straight from the MFMA layout would be 16-byte pieces of 32
  // rows per instruction. Every wave reaches every barrier below.
  char* const T = reinterpret_cast<char*>(lds);
  // The problem's output fields, read once: through the reference into the
  // kernel arguments they would be read again after every store (a store
  // could alias them), one scalar-load round trip per 16 bytes written.
  const int seg_len = P.seg_len, seg_off = P.seg_off;
  const int64_t seg_stride = P.seg_stride, ldc = P.ldc;
  void* const Cp = P.C;
  // A tile's rows lie in one segment unless a segment is shorter than the
  // tile; then output row and batch row come without a division.
  const int b_first = m0 / seg_len, b_last = (min(M, m0 + BM) - 1) / seg_len;
  const bool one_seg = b_first == b_last;
  auto batch_of = [&](int gr) -> int { return one_seg ? b_first : gr / seg_len; };
  // bf16 stage [rows][256]: 16-byte chunk c of row r at c ^ (r & 31)
  auto out_row_of = [&](int gr, int& b) -> int64_t {
    b = batch_of(gr);
    return (int64_t)b * seg_stride + seg_off + (gr - b * seg_len);
  };

  if (EK == EK_F32) {
    // fp32 stage [128][256] per pass: pass p holds accumulator block i = p
    // of every wave (stage row r is tile row (r / 32) WTM + 32 p + r % 32),
    // so each pass frees its registers; 16-byte chunk c of row r at c ^ (r & 31).
    // A wave writes 16 rows of a pass: row r = 8 k + wave for k < 16, one
    // 16-byte unit per lane (chunk = lane). The rows' output offsets are
    // wave-uniform.
    int m0p = m0;
    asm volatile("" : "+s"(m0p));
    const int c = lane, col = tn * BNT + c * 4;
    const bool col_ok = c * 4 < BNT && col < N;
    const float* const gate = P.gate;
    const int64_t gate_bs = P.gate_bstride;
    const bool resid = epi == EPI_RESID;
    float* const Cf = static_cast<float*>(Cp);
    // inside one batch segment a lane's gate is one vector for the whole tile
    // (read once at 256 rows; at 384 rows, with its batch of 8 rows, like a
    // tile across batch segments)
    const bool gate_once = FM == 2 && one_seg;
    f32x4 g1 = {};
    if (resid && gate_once && col_ok) g1 = *reinterpret_cast<const f32x4*>(gate + (int64_t)b_first * gate_bs + col);
    // The residual reads of RB rows per wave are in flight together. At 256
    // rows (registers allow 16) a pass's reads are issued before its
    // accumulators are staged, so their latency hides behind the staging and
    // its barrier (and, in the first pass, behind the last MFMAs' results
    // arriving): one memory latency per pass. At 384 rows they go in batches
    // of 8 after the barrier.
    constexpr int RB = FM == 2 ? 16 : 8;
    auto stage = [&](int pass) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = wm * 32 + fr;
          const int cc = (wn * WTN + j * 32 + 8 * q + 4 * fg) >> 2;
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[pass][j][4 * q + e];
          *reinterpret_cast<f32x4*>(T + r * 1024 + ((cc ^ (r & 31)) << 4)) = v;
        }
    };
#pragma unroll
    for (int pass = 0; pass < FM; ++pass) {
      f32x4 x[RB];
      // row k of batch bt is stage row 8 (RB bt + k) + wave
      auto reads = [&](int bt) {
#pragma unroll
        for (int k = 0; k < RB; ++k) {
          const int r = 8 * (RB * bt + k) + wave;
          const int gr = m0p + (r >> 5) * WTM + 32 * pass + (r & 31);
          if (resid && col_ok && gr < M) {
            int b;
            x[k] = *reinterpret_cast<const f32x4*>(Cf + out_row_of(gr, b) * ldc + col);
          }
        }
      };
      if (FM == 2) reads(0);
      __builtin_amdgcn_sched_barrier(0);
      stage(pass);
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      // the row offsets again, from a copy of m0 the compiler cannot see
      // through (kept from the reads they would hold 32 scalar registers)
      int m0q = m0;
      asm volatile("" : "+s"(m0q));
#pragma unroll
      for (int bt = 0; bt < 16 / RB; ++bt) {
        if (FM != 2) reads(bt);
#pragma unroll
        for (int h = 0; h < RB / 8; ++h) {
          // a tile across batch segments reads each row's gate, 8 rows at a time
          f32x4 g[8];
          if (resid && !gate_once) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              const int r = 8 * (RB * bt + 8 * h + k) + wave;
              const int gr = m0q + (r >> 5) * WTM + 32 * pass + (r & 31);
              g[k] = g1;
              if (col_ok && gr < M)
                g[k] = *reinterpret_cast<const f32x4*>(gate + (int64_t)batch_of(gr) * gate_bs + col);
            }
          }
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const int r = 8 * (RB * bt + 8 * h + k) + wave;
            const int gr = m0q + (r >> 5) * WTM + 32 * pass + (r & 31);
            if (!col_ok || gr >= M) continue;
            int b;
            const f32x4 v = *reinterpret_cast<const f32x4*>(T + r * 1024 + ((c ^ (r & 31)) << 4));
            float* const d = Cf + out_row_of(gr, b) * ldc + col;
            *reinterpret_cast<f32x4*>(d) = resid ? x[8 * h + k] + (gate_once ? g1 : g[k]) * v : v;
          }
        }
      }
      __syncthreads();
    }
    return;
  }

  if (EK == EK_QKV) {
    // fp32 stage [128][256] per pass, laid out like the fp32 family's: pass p
    // holds accumulator block i = p of every wave, so q and k are rounded to
    // bf16 once, after the norm, gain and rotation. A row's 1 / rms (times
    // q_scale for q) comes from the fp32 accumulators first and is kept per
    // row in LDS (outside every pass's stage); a row's 128 values of a head
    // sit in lanes l and l ^ 32, so the sum of squares needs one cross-half
    // exchange.
    // the shared operands, read once (see above)
    bf16_t* const eq = args.qkv.q;
    bf16_t* const ek = args.qkv.k;
    bf16_t* const evt = args.qkv.vt;
    const float* const cos_t = args.qkv.cos_t;
    const float* const sin_t = args.qkv.sin_t;
    const float* const q_gain = args.qkv.q_gain[pi];
    const float* const k_gain = args.qkv.k_gain[pi];
    const int64_t S_pad = args.qkv.S_pad;
    const int EH = args.qkv.H, ED = args.qkv.D;
    const float eps = args.qkv.eps, q_scale = args.qkv.q_scale;
    float* const row_scale = reinterpret_cast<float*>(T + RS_BYTE);  // [2][BM]
    const int wcol0 = tn * BN + wn * WTN;  // first projection column of the wave
    if (wcol0 < N && wcol0 / ED < 2) {
      const float sc = wcol0 / ED == 0 ? q_scale : 1.f;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) ss += acc[i][j][e] * acc[i][j][e];
        ss = half_sum(ss);
        if (fg == 0)
          row_scale[wn * BM + wm * WTM + i * 32 + fr] = rsqrtf(ss * (1.f / 128.f) + eps) * sc;
      }
    }
#pragma unroll
    for (int pass = 0; pass < FM; ++pass) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = wm * 32 + fr;
          const int c = (wn * WTN + j * 32 + 8 * q + 4 * fg) >> 2;
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[pass][j][4 * q + e];
          *reinterpret_cast<f32x4*>(T + r * 1024 + ((c ^ (r & 31)) << 4)) = v;
        }
      __syncthreads();
      // stage row r is tile row (r / 32) WTM + 32 pass + r % 32
      auto tile_row = [&](int r) { return (r >> 5) * WTM + 32 * pass + (r & 31); };
      auto stage_f32 = [&](int r, int col) -> const float* {  // tile column col of stage row r
        return reinterpret_cast<const float*>(T + r * 1024 + ((((col >> 2) ^ (r & 31))) << 4)) +
               (col & 3);
      };
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int col0 = tn * BN + hh * 128;
        if (col0 >= N) break;
        const int part = col0 / ED;
        const int h = (col0 - part * ED) >> 7;
        if (part < 2) {
          // q / k rows to [b, h, s, :]: 16 lanes per token row, 8 columns (4
          // rotation pairs) per lane
          bf16_t* base = part == 0 ? eq : ek;
          const float* gain = part == 0 ? q_gain : k_gain;
          const int cl = (tid & 15) * 8;  // column within the head
          const f32x4 g0 = *reinterpret_cast<const f32x4*>(gain + cl);
          const f32x4 g1 = *reinterpret_cast<const f32x4*>(gain + cl + 4);
#pragma unroll 2
          for (int it = 0; it < 128 * 16 / NT; ++it) {
            const int r = (it * NT + tid) >> 4;
            const int tr = tile_row(r);
            const int gr = m0 + tr;
            if (gr >= M) continue;
            const int b = batch_of(gr);
            const int s = seg_off + (gr - b * seg_len);
            const f32x4 v0 = *reinterpret_cast<const f32x4*>(stage_f32(r, hh * 128 + cl));
            const f32x4 v1 = *reinterpret_cast<const f32x4*>(stage_f32(r, hh * 128 + cl + 4));
            const float rsc = row_scale[hh * BM + tr];
            const f32x4 co = *reinterpret_cast<const f32x4*>(cos_t + (int64_t)s * 64 + (cl >> 1));
            const f32x4 si = *reinterpret_cast<const f32x4*>(sin_t + (int64_t)s * 64 + (cl >> 1));
            f32x8 y;
#pragma unroll
            for (int pr = 0; pr < 4; ++pr) {
              const float gx0 = pr < 2 ? g0[2 * pr] : g1[2 * pr - 4];
              const float gx1 = pr < 2 ? g0[2 * pr + 1] : g1[2 * pr - 3];
              const float a0 = pr < 2 ? v0[2 * pr] : v1[2 * pr - 4];
              const float a1 = pr < 2 ? v0[2 * pr + 1] : v1[2 * pr - 3];
              const float x0 = a0 * rsc * gx0;
              const float x1 = a1 * rsc * gx1;
              y[2 * pr] = x0 * co[pr] - x1 * si[pr];
              y[2 * pr + 1] = x0 * si[pr] + x1 * co[pr];
            }
            *reinterpret_cast<bf16x8*>(base + (((int64_t)b * EH + h) * S_pad + s) * 128 + cl) =
                pack_bf16x8(y);
          }
        } else {
          // v to v^T[b, h, d, s..s+7]: 8 tokens per dim and lane
#pragma unroll 2
          for (int it = 0; it < 128 * 16 / NT; ++it) {
            const int u = it * NT + tid;
            const int d = u & 127, tg = u >> 7;  // dim, group of 8 stage rows
            f32x8 tv;
#pragma unroll
            for (int e = 0; e < 8; ++e) tv[e] = *stage_f32(tg * 8 + e, hh * 128 + d);
            const bf16x8 tb = pack_bf16x8(tv);
            const int r0 = m0 + tile_row(tg * 8);  // 8 stage rows = 8 tile rows
            if (r0 >= M) continue;
            const int b0 = batch_of(r0);
            const int s0 = seg_off + (r0 - b0 * seg_len);
            if (r0 + 7 < M && batch_of(r0 + 7) == b0 && (s0 & 7) == 0) {
              *reinterpret_cast<bf16x8*>(evt + (((int64_t)b0 * EH + h) * 128 + d) * S_pad + s0) = tb;
            } else {
              const u32x4 tw = __builtin_bit_cast(u32x4, tb);
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const int gr = r0 + e;
                if (gr >= M) break;
                const int b = batch_of(gr);
                const int s = seg_off + (gr - b * seg_len);
                evt[(((int64_t)b * EH + h) * 128 + d) * S_pad + s] =
                    (bf16_t)((tw[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
              }
            }
          }
        }
      }
      if (pass + 1 < FM) __syncthreads();  // the next pass overwrites the stage
    }
    return;
  }

  // bf16 results (SwiGLU, plain bf16) in passes of up to two accumulator
  // blocks of every wave (the whole tile at 256 rows; blocks {0, 1} then {2}
  // at 384 rows: a 384 x 256 bf16 stage would not fit the LDS). In pass p
  // with nb blocks, stage row r is tile row
  // (r / (32 nb)) WTM + 32 (2 p + (r / 32) % nb) + r % 32.
  constexpr int NPASS = (FM + 1) / 2;
  // every result as bf16, packed 4 per register pair: half the registers of
  // the accumulators, which the later passes would otherwise hold through
  // the earlier passes' stores (SwiGLU: the gate and up halves combine
  // first, so columns j < FN / 2 carry the products)
  u32x2 pk[FM][FN][4];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4 v;
        if (epi == EPI_SWIGLU) {
          if (j >= FN / 2) continue;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            v[e] = silu_f(acc[i][j][4 * q + e]) * acc[i][j + FN / 2][4 * q + e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
        }
        pk[i][j][q] = pack_bf16x4(v);
      }
#pragma unroll
  for (int pass = 0; pass < NPASS; ++pass) {
    constexpr int BPP = 2;
    const int nb = min(FM - BPP * pass, BPP);  // blocks in this pass
    const int prow = 32 * nb * 4;              // stage rows of this pass
    // tile row of stage row r
    auto tile_row = [&](int r) {
      return (r / (32 * nb)) * WTM + 32 * (BPP * pass + (r >> 5) % nb) + (r & 31);
    };
    // phase A: this pass's blocks into the stage
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (i / BPP != pass) continue;
      const int r = wm * 32 * nb + (i - BPP * pass) * 32 + fr;
      // SwiGLU: 64 output columns per wave; plain bf16: 128
      const int nj = epi == EPI_SWIGLU ? FN / 2 : FN;
      const int cw = epi == EPI_SWIGLU ? WTN / 2 : WTN;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if (j >= nj) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = wn * cw + j * 32 + 8 * q + 4 * fg;
          *reinterpret_cast<u32x2*>(T + r * 512 + (((col >> 3) ^ (r & 31)) << 4) +
                                    ((col & 4) << 1)) = pk[i][j][q];
        }
      }
    }
    __syncthreads();

    // phase B: whole rows out, 16 bytes per lane; unit u = it NT + tid is
    // row u / upr, chunk u % upr, stepped without a division
    const int ncol = epi == EPI_SWIGLU ? BN / 2 : BNT;  // output columns of the tile
    const int upr = ncol / 8;                          // 16-byte units per row
    // (prow upr is a multiple of NT for every tile shape: no partial step);
    // the LDS reads of four units go out before their four stores
    const int r_step = NT / upr, c_step = NT - r_step * upr;
    const int n_it = prow * upr / NT;
    int r = tid / upr, c = tid - (tid / upr) * upr;
    for (int it0 = 0; it0 < n_it; it0 += 4) {
      u32x4 v[4];
      bf16_t* dst[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        dst[k] = nullptr;
        if (it0 + k < n_it) {
          const int gr = m0 + tile_row(r), col = tn * ncol + c * 8;
          v[k] = *reinterpret_cast<const u32x4*>(T + r * 512 + ((c ^ (r & 31)) << 4));
          if (gr < M && col < N) {
            int b;
            dst[k] = static_cast<bf16_t*>(Cp) + out_row_of(gr, b) * ldc + col;
          }
          r += r_step;
          c += c_step;
          if (c >= upr) {
            c -= upr;
            ++r;
          }
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (dst[k] != nullptr) *reinterpret_cast<u32x4*>(dst[k]) = v[k];
    }
    if (pass + 1 < NPASS) __syncthreads();  // the next pass overwrites the stage
  }
}

// GEMM tile of launch index `block` of batch args.
template <int BNT, int FAM>
__device__ __forceinline__ void gemm_block(const GemmBatch& args, int block, u32x4* lds) {
  int pi = 0, local = 0;
  const auto tiles_of = [&](int i) { return args.p[i].tiles_m * args.p[i].tiles_n; };
  if (!tile_of_block<kMaxGemmProblems>(tiles_of, args.count, block, &pi, &local))
    return;  // not reached: the grid has exactly one workgroup per tile
  pi = __builtin_amdgcn_readfirstlane(pi);
  local = __builtin_amdgcn_readfirstlane(local);
  // fields are read from the kernel arguments (scalar loads) as needed
  const GemmProblem& P = args.p[pi];
  if (FAM == FAM_F32) {
    if (P.fm == 3) gemm_tile<BNT, 3, EK_F32>(args, P, pi, local, lds);
    else gemm_tile<BNT, 2, EK_F32>(args, P, pi, local, lds);
  } else if (P.epi == EPI_QKV) {
    if (P.fm == 3) gemm_tile<BNT, 3, EK_QKV>(args, P, pi, local, lds);
    else gemm_tile<BNT, 2, EK_QKV>(args, P, pi, local, lds);
  } else {
    if (P.fm == 3) gemm_tile<BNT, 3, EK_BF16>(args, P, pi, local, lds);
    else gemm_tile<BNT, 2, EK_BF16>(args, P, pi, local, lds);
  }
}

template <int BNT, int FAM>
__global__ __launch_bounds__(NT, 1) void gemm_bf16_kernel(const GemmBatch args) {
  __shared__ u32x4 lds[LDS_U];
  gemm_block<BNT, FAM>(args, (int)blockIdx.x, lds);
}

// Fused launch: the attention units (blocks [0, n_attn), dealt to the XCDs
// like the attention kernel's) and then the tiles of a bf16-family GEMM batch
// that does not depend on them. The hardware hands out workgroups in launch
// order, so the GEMM tiles start as attention units finish and fill the CUs
// that the attention's last round would leave idle. Both parts run 8 waves
// with two per SIMD; the attention uses the first 128 KiB of the LDS.
struct AttnGemmArgs {
  AttnArgs attn;
  GemmBatch gemm;
  int32_t n_attn;
};

__global__ __launch_bounds__(NT, 1) void attn_gemm_kernel(const AttnGemmArgs args) {
  __shared__ u32x4 lds[LDS_U];
  static_assert(att::NT == NT && att::LDS_BYTES <= LDS_U * 16, "one workgroup shape");
  const int blk = (int)blockIdx.x;
  if (blk < args.n_attn) {
    att::attention_unit(args.attn, xcd_remap(blk, args.n_attn), reinterpret_cast<char*>(lds));
    return;
  }
  gemm_block<BN, FAM_BF16>(args.gemm, blk - args.n_attn, lds);
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

// ---- launch plan: tile width of the launch and, per problem, the tile
// height of its rows (a problem whose rows form one segment may have its
// first rows in 384-row tiles and the rest in 256-row tiles: two parts).
// A tile's time per K slice is modelled from what a loader wave does in it:
// its load instructions (4 FM + 8) and its own MFMAs (FM x 4 k-steps x its
// active column blocks), weighted 4 : 3. Fitted to kernel traces at 4608
// rows (a 384-row tile takes 1.40x a 256-row one: 116 vs 83 us at K = 3072).
// The launch time is modelled as one XCD's share of every part (a part's
// tiles are dealt evenly to the 8 XCDs), in launch order, placed greedily on
// that XCD's CUs, which reproduces the traced launch times of the step
// within 3 %; plans are cached per launch shape.
struct Part {
  int prob;   // problem of the batch
  int row0;   // its first row
  int rows;
  int fm;     // tile height 128 fm
};

struct Plan {
  int bnt;
  int nparts;
  Part part[kMaxGemmProblems];  // launch order
};

int64_t tile_cost(int fm, int bnt, int64_t K) {
  const int loads = 4 * fm + 8, mfmas = fm * (bnt == 224 ? 3 : 4) * 4;
  return (int64_t)(4 * loads + 3 * mfmas) * (K / BK);
}

// Model time of an attention unit over S keys, in tile_cost units: a unit
// takes about 1.55 us per 64-key tile at S = 4608 next to 83 us for a
// 256-row GEMM tile at K = 3072 (7680 units).
int64_t attn_unit_cost(int64_t S) { return 143 * ((S + 63) / 64); }

// Work ahead of the GEMM tiles in a fused launch (none for a plain one).
struct Prefix {
  int64_t units = 0;  // attention units of the launch
  int64_t cost = 0;   // model cost of one
};

int64_t model_time(const GemmBatch& b, const Plan& pl, int cus_per_xcd, const Prefix& pre) {
  std::vector<int64_t> cu((size_t)std::max(cus_per_xcd, 1), 0);
  auto place = [&](int64_t n, int64_t c) {
    for (int64_t t = 0; t < n; ++t) {
      auto it = std::min_element(cu.begin(), cu.end());
      *it += c;
    }
  };
  place((pre.units + 7) / 8, pre.cost);
  for (int k = 0; k < pl.nparts; ++k) {
    const Part& pt = pl.part[k];
    const GemmProblem& p = b.p[pt.prob];
    const int cols = p.epi == EPI_SWIGLU ? BN / 2 : pl.bnt;
    const int64_t n = (int64_t)((pt.rows + 128 * pt.fm - 1) / (128 * pt.fm)) *
                      ((p.N + cols - 1) / cols);
    place((n + 7) / 8, tile_cost(pt.fm, pl.bnt, p.K));
  }
  return *std::max_element(cu.begin(), cu.end());
}

// DIT_GEMM_TILE_ROWS=256 or 384 forces one tile height on every problem
// (tests compare the two bit for bit; timing runs compare them with the
// model's choice). Any other value, or none, leaves the choice to the model.
int forced_rows() {
  const char* e = std::getenv("DIT_GEMM_TILE_ROWS");
  if (!e) return 0;
  const int v = std::atoi(e);
  return v == 256 || v == 384 ? v : 0;
}

// DIT_GEMM_SPLIT_ROWS=a (a positive multiple of 384) forces the split of
// every launch's largest one-segment problem with more than a rows at row a
// (tests compare it bit for bit with the other tilings); 0 when unset.
int forced_split() {
  const char* e = std::getenv("DIT_GEMM_SPLIT_ROWS");
  if (!e) return 0;
  const int v = std::atoi(e);
  return v > 0 && v % 384 == 0 ? v : 0;
}

// Parts in launch order: taller tiles first (stable), so each XCD ends on
// its short tiles.
void order_parts(Plan& pl) {
  std::stable_sort(pl.part, pl.part + pl.nparts,
                   [](const Part& x, const Part& y) { return x.fm > y.fm; });
}

Plan make_plan(const GemmBatch& b, int cus, int forced, const Prefix& pre, int64_t* time) {
  bool narrow_ok = true;
  for (int i = 0; i < b.count; ++i)
    if (b.p[i].epi == EPI_SWIGLU || b.p[i].epi == EPI_QKV) narrow_ok = false;
  // candidates: 384-row tiles for any subset of the (at most three) largest
  // problems with at least 384 rows, everything else 256 rows; and the
  // largest problem whose rows form one segment split into a 384-row part
  // (a multiple of 384 rows) and a 256-row part
  int big[3], nbig = 0, split = -1;
  if (!forced) {
    std::vector<std::pair<int64_t, int>> sz;
    for (int i = 0; i < b.count; ++i)
      if (b.p[i].M >= 384) sz.push_back({-(int64_t)b.p[i].M * b.p[i].N * b.p[i].K, i});
    std::sort(sz.begin(), sz.end());
    for (size_t j = 0; j < sz.size() && nbig < 3; ++j) big[nbig++] = sz[j].second;
    for (size_t j = 0; j < sz.size() && split < 0; ++j)
      if (b.p[sz[j].second].seg_len >= b.p[sz[j].second].M && b.p[sz[j].second].M > 384)
        split = sz[j].second;
    if (b.count >= kMaxGemmProblems) split = -1;  // no slot for a second part
  }
  const int fsplit = forced ? 0 : forced_split();
  if (fsplit > 0 && split >= 0 && b.p[split].M > fsplit) {
    // the forced split, every other problem in 256-row tiles
    Plan ps{};
    ps.bnt = BN;
    for (int i = 0; i < b.count; ++i) {
      if (i != split) {
        ps.part[ps.nparts++] = Part{i, 0, b.p[i].M, 2};
      } else {
        ps.part[ps.nparts++] = Part{i, 0, fsplit, 3};
        ps.part[ps.nparts++] = Part{i, fsplit, b.p[i].M - fsplit, 2};
      }
    }
    order_parts(ps);
    if (time) *time = model_time(b, ps, std::max(1, cus / 8), pre);
    return ps;
  }
  Plan best{};
  int64_t best_t = -1;
  const int cpx = std::max(1, cus / 8);
  auto consider = [&](const Plan& pl) {
    const int64_t t = model_time(b, pl, cpx, pre);
    if (best_t < 0 || t < best_t) {
      best_t = t;
      best = pl;
    }
  };
  for (int bnt : {256, 224}) {
    if (bnt == 224 && !narrow_ok) continue;
    for (int mask = 0; mask < (1 << nbig); ++mask) {
      int fm[kMaxGemmProblems];
      for (int i = 0; i < kMaxGemmProblems; ++i) fm[i] = forced == 384 ? 3 : 2;
      for (int j = 0; j < nbig; ++j)
        if (mask >> j & 1) fm[big[j]] = 3;
      Plan pl{};
      pl.bnt = bnt;
      pl.nparts = b.count;
      for (int i = 0; i < b.count; ++i) pl.part[i] = Part{i, 0, b.p[i].M, fm[i]};
      order_parts(pl);
      consider(pl);
      if (split < 0) continue;
      const int M = b.p[split].M;
      for (int a = 384; a < M; a += 384) {
        Plan ps{};
        ps.bnt = bnt;
        ps.nparts = 0;
        for (int i = 0; i < b.count; ++i) {
          if (i != split) {
            ps.part[ps.nparts++] = Part{i, 0, b.p[i].M, fm[i]};
          } else {
            ps.part[ps.nparts++] = Part{i, 0, a, 3};
            ps.part[ps.nparts++] = Part{i, a, M - a, 2};
          }
        }
        order_parts(ps);
        consider(ps);
      }
    }
  }
  if (time) *time = best_t;
  return best;
}

using PlanKey = std::tuple<int, int, int64_t, int, std::vector<int64_t>>;

Plan cached_plan(const GemmBatch& b, int cus, const Prefix& pre = Prefix{}) {
  const int forced = forced_rows();
  const int fsplit = forced_split();
  static std::mutex mu;
  static std::map<PlanKey, Plan> cache;
  std::vector<int64_t> shape;
  for (int i = 0; i < b.count; ++i) {
    const GemmProblem& p = b.p[i];
    shape.insert(shape.end(), {(int64_t)p.M, (int64_t)p.N, (int64_t)p.K, (int64_t)p.epi});
  }
  shape.insert(shape.end(), {pre.units, pre.cost});
  PlanKey key{cus, forced, fsplit, b.count, shape};
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  const Plan pl = make_plan(b, cus, forced, pre, nullptr);
  if (cache.size() < 4096) cache.emplace(key, pl);
  return pl;
}

}  // namespace

namespace {

bool is_f32_epi(int epi) { return epi == EPI_F32 || epi == EPI_RESID; }

// Applies plan pl to a copy of batch: one problem per part, in launch
// order, with its tile height and counts. A part that starts at row r0 of
// its (one-segment) problem reads A from row r0 and writes output rows (and
// QKV tokens) from seg_off + r0.
// Returns the tile count (< 0 if it does not fit the grid).
int64_t prepare(const GemmBatch& batch, const Plan& pl, GemmBatch& b) {
  b = batch;
  b.count = pl.nparts;
  for (int k = 0; k < pl.nparts; ++k) {
    const Part& pt = pl.part[k];
    GemmProblem p = batch.p[pt.prob];
    if (pt.row0 != 0 || pt.rows != p.M) {
      p.A += (int64_t)pt.row0 * p.lda;
      p.seg_off += pt.row0;
      p.M = pt.rows;
    }
    b.p[k] = p;
    b.qkv.q_gain[k] = batch.qkv.q_gain[pt.prob];
    b.qkv.k_gain[k] = batch.qkv.k_gain[pt.prob];
  }
  int64_t total = 0;
  for (int k = 0; k < b.count; ++k) {
    GemmProblem& p = b.p[k];
    p.fm = pl.part[k].fm;
    const int cols = p.epi == EPI_SWIGLU ? BN / 2 : pl.bnt;
    p.tiles_m = (p.M + 128 * p.fm - 1) / (128 * p.fm);
    p.tiles_n = (p.N + cols - 1) / cols;
    p.tile_begin = (int32_t)std::min<int64_t>(total, INT32_MAX);
    total += (int64_t)p.tiles_m * p.tiles_n;
  }
  if (total > INT32_MAX) return -1;
  b.total_tiles = (int32_t)total;
  return total;
}

bool valid_batch(GemmBatch& batch) {
  for (int i = batch.count; i < kMaxGemmProblems; ++i) batch.p[i] = GemmProblem{};
  if (batch.count < 1 || batch.count > kMaxGemmProblems) return false;
  // one epilogue family per launch
  for (int i = 1; i < batch.count; ++i)
    if (is_f32_epi(batch.p[i].epi) != is_f32_epi(batch.p[0].epi)) return false;
  return true;
}

}  // namespace

hipError_t gemm_launch(GemmBatch& batch, hipStream_t stream) {
  if (!valid_batch(batch)) return hipErrorInvalidValue;
  const bool f32 = is_f32_epi(batch.p[0].epi);
  const Plan pl = cached_plan(batch, device_cus());
  GemmBatch b;
  const int64_t total = prepare(batch, pl, b);
  if (total < 0) return hipErrorInvalidValue;
  batch.total_tiles = b.total_tiles;
  if (total == 0) return hipSuccess;
  const dim3 grid((unsigned)total);
  if (f32)
    hipLaunchKernelGGL((pl.bnt == 224 ? gemm_bf16_kernel<224, FAM_F32> : gemm_bf16_kernel<256, FAM_F32>),
                       grid, dim3(NT), 0, stream, b);
  else if (pl.bnt == 224)
    hipLaunchKernelGGL((gemm_bf16_kernel<224, FAM_BF16>), grid, dim3(NT), 0, stream, b);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<256, FAM_BF16>), grid, dim3(NT), 0, stream, b);
  return hipGetLastError();
}

hipError_t attn_gemm_launch(const AttnArgs& a, GemmBatch& batch, hipStream_t stream) {
  if (batch.count == 0) return attention_launch(a, stream);
  if (!valid_batch(batch) || is_f32_epi(batch.p[0].epi)) return hipErrorInvalidValue;
  Prefix pre;
  pre.units = att::attention_units(a);
  pre.cost = attn_unit_cost(a.S);
  const Plan pl0 = cached_plan(batch, device_cus(), pre);
  Plan pl = pl0;
  pl.bnt = BN;  // the fused kernel runs full-width tiles only
  AttnGemmArgs args{};
  args.attn = a;
  args.n_attn = (int32_t)pre.units;
  const int64_t total = prepare(batch, pl, args.gemm);
  if (total < 0 || pre.units + total > INT32_MAX) return hipErrorInvalidValue;
  batch.total_tiles = args.gemm.total_tiles;
  hipLaunchKernelGGL(attn_gemm_kernel, dim3((unsigned)(pre.units + total)), dim3(NT), 0, stream,
                     args);
  return hipGetLastError();
}

int64_t fused_split_rows(const GemmProblem& first, const GemmProblem& rest, int64_t row_step,
                         const AttnArgs& a) {
  // DIT_FUSED_SPLIT_ROWS=m forces the split at min(m, rows) (tests compare
  // splits bit for bit; timing runs compare them with the model's choice)
  if (const char* e = std::getenv("DIT_FUSED_SPLIT_ROWS")) {
    const long long v = std::atoll(e);
    if (v >= 0) return std::min<int64_t>((int64_t)v, rest.M);
  }
  static std::mutex mu;
  static std::map<std::vector<int64_t>, int64_t> cache;
  const int cus = device_cus(), forced = forced_rows();
  const std::vector<int64_t> key{cus, forced, forced_split(), row_step, first.M, first.N, first.K, first.epi,
                                 rest.M, rest.N, rest.K, rest.epi, a.S, a.B, a.H};
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  Prefix pre;
  pre.units = att::attention_units(a);
  pre.cost = attn_unit_cost(a.S);
  const int64_t R = rest.M;
  int64_t best_rows = 0, best_t = -1;
  for (int64_t m1 = 0; m1 <= R; m1 = (m1 + row_step > R && m1 < R) ? R : m1 + row_step) {
    GemmBatch b1{}, b2{};
    b1.p[b1.count++] = first;
    if (m1 > 0) {
      b1.p[b1.count] = rest;
      b1.p[b1.count++].M = (int32_t)m1;
    }
    if (m1 < R) {
      b2.p[b2.count] = rest;
      b2.p[b2.count++].M = (int32_t)(R - m1);
    }
    int64_t t1 = 0, t2 = 0;
    make_plan(b1, cus, forced, Prefix{}, &t1);
    if (b2.count) make_plan(b2, cus, forced, pre, &t2);
    else {
      Plan none{};
      none.bnt = BN;
      t2 = model_time(b2, none, std::max(1, cus / 8), pre);
    }
    if (best_t < 0 || t1 + t2 < best_t) {
      best_t = t1 + t2;
      best_rows = m1;
    }
    if (m1 == R) break;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (cache.size() < 4096) cache.emplace(key, best_rows);
  return best_rows;
}

}  // namespace dit
