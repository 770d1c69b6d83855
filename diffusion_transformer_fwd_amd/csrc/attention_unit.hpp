// Joint attention work unit for gfx950, shared by the attention kernel and
// the fused attention + GEMM kernel (see attention.hip for the design).
#pragma once

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace dit {
namespace att {

constexpr int NT = 512;    // 8 waves
constexpr int QB = 256;    // queries per workgroup (32 per wave)
constexpr int KT = 64;     // keys per tile
constexpr int NSTAGE = 4;  // LDS stages
constexpr int KU = 16;     // 16-byte units per K row (128 bf16)
constexpr int VU = 8;      // 16-byte units per V^T row (64 keys)
constexpr int K_BYTES = KT * KU * 16;    // 16 KiB per K stage
constexpr int V_BYTES = 128 * VU * 16;   // 16 KiB per V^T stage
constexpr int V_BASE = NSTAGE * K_BYTES; // V^T stages follow the K stages
constexpr float kSumGuard = 18446744073709551616.f;  // 2^64

typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int LDS_BYTES = V_BASE + NSTAGE * V_BYTES;  // 128 KiB

// K tile swizzle: a bit permutation of the key's low 4 bits chosen so that
// the 8 (and 16) keys read together by one fragment load hit distinct banks.
__device__ __forceinline__ int kswz(int key) {
  return (key & 3) | (((key >> 3) & 1) << 2) | (((key >> 2) & 1) << 3);
}
// V^T tile swizzle (rows of 128 bytes).
__device__ __forceinline__ int vswz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// Key (within a 32-key block) at score-accumulator row r: chosen so that a
// lane's accumulator entries i = 8 s + e (s = 0, 1) are keys 16 s + 8 g + e.
__device__ __forceinline__ int key_of_row(int r) {
  const int j = r >> 3, gp = (r >> 2) & 1, t = r & 3;
  return 16 * (j >> 1) + 8 * gp + 4 * (j & 1) + t;
}

template <int STG>
using stage_t = std::integral_constant<int, STG>;

// Workgroup barrier without __syncthreads()' release fence, which would also
// wait for the tile loads still in flight. LDS reads before it have all been
// consumed by MFMAs (so they completed), and a tile's loads are waited for by
// the wave that issued them before the barrier that publishes the tile.
__device__ __forceinline__ void wg_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// One unit of work: query block qb of (batch b, head h) for logical index
// L = (b * H + h) * n_qb + qb, with the K / V^T tiles staged at lb (LDS of
// LDS_BYTES, starting at LDS offset 0). Every wave of the workgroup calls it.
__device__ __forceinline__ void attention_unit(const AttnArgs& a, int L, char* const lb) {

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool leader = wave < 4;  // waves 0-3 lead; 4-7 lag half an iteration
  // XCD-contiguous work order: consecutive query blocks of one (b, h) run on
  // the same XCD, so that head's K and V^T stay in that XCD's L2.
  const int n_qb = (int)((a.S + QB - 1) / QB);
  const int qb = L % n_qb, bhi = L / n_qb;
  const int h = bhi % a.H, b = bhi / a.H;
  const int64_t bh = (int64_t)b * a.H + h;
  const int64_t q0 = (int64_t)qb * QB + wave * 32;
  const int qi = lane & 31, g = lane >> 5;

  // Q fragments (second MFMA operand): query q0 + qi, dims 16 ks + 8 g + 0..7
  bf16x8 qf[8];
  {
    const u32x4* qp = reinterpret_cast<const u32x4*>(a.q + (bh * a.S_pad + q0 + qi) * 128);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, qp[2 * ks + g]);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // K / V^T tiles go straight from memory into LDS (buffer loads that write
  // LDS at M0 + 16 * lane). With lw = wave % 4, a tile's K rows 16 lw ..
  // 16 lw + 15 (four instructions of 4 rows x 16 chunks) come from wave lw + 4
  // and its V^T rows 32 lw .. 32 lw + 31 (four of 8 rows x 8 chunks) from
  // wave lw, except tiles 0 and 1, which waves 0-3 fetch whole; each lane
  // fetches the logical chunk whose swizzled position is its own.
  const __amdgpu_buffer_rsrc_t k_rsrc =
      make_rsrc(a.k + bh * a.S_pad * 128, clamp_u32(a.S_pad * 128 * 2));
  const __amdgpu_buffer_rsrc_t v_rsrc =
      make_rsrc(a.vt + bh * 128 * a.S_pad, clamp_u32(a.S_pad * 128 * 2));
  const int lw = wave & 3;
  uint32_t k_off[4], v_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int krow = 16 * lw + 4 * i + (lane >> 4);
    k_off[i] = (uint32_t)((krow * 128 + (((lane & 15) ^ kswz(krow)) * 8)) * 2);
    const int vrow = 32 * lw + 8 * i + (lane >> 3);
    v_off[i] = (uint32_t)((vrow * a.S_pad + (((lane & 7) ^ vswz(vrow)) * 8)) * 2);
  }
  // instruction j (0..7) of this wave's share of tile t: K rows for j < 4,
  // V^T rows for j >= 4
  auto dma_part = [&](int t, auto stage, int j) {
    constexpr int STG = decltype(stage)::value;
    if (j < 4)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          k_rsrc, (lds_ptr_t)(lb + STG * K_BYTES + (16 * lw + 4 * j) * KU * 16), 16,
          k_off[j] + (uint32_t)t * KT * 128 * 2, 0, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          v_rsrc, (lds_ptr_t)(lb + V_BASE + STG * V_BYTES + (32 * lw + 8 * (j - 4)) * VU * 16),
          16, v_off[j - 4] + (uint32_t)t * KT * 2, 0, 0, 0);
  };

  // fragment read addresses (bytes, stage 0): K row key_of_row(qi) (+32 rows
  // for the second key block), chunk 2 ks + g; V^T row qi (+32 per dim block),
  // chunk 2 s + g; both through their swizzles.
  uint32_t k_rd[8], v_rd[4];
  {
    const int krow = key_of_row(qi), ksw = kswz(krow), vsw = vswz(qi);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) k_rd[ks] = (uint32_t)((krow * KU + ((2 * ks + g) ^ ksw)) * 16);
#pragma unroll
    for (int s = 0; s < 4; ++s)
      v_rd[s] = (uint32_t)(V_BASE + (qi * VU + ((2 * s + g) ^ vsw)) * 16);
  }

  // ninth k-step of the score product: every key row carries a 1 and the
  // query column carries -m at k = 0 (lanes g = 0), zeros elsewhere
  bf16x8 kaug = {}, qaug = {};
  kaug[0] = (__bf16)(g == 0 ? 1.0f : 0.0f);
  float m = 0.f;  // running max (log2 units), exact in bf16; set by the first tile

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  f32x16 sacc[2];
  bf16x8 pf[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pf[i] = bf16x8{};
  float l = 0.f;
  // V^T stage NSTAGE - 1 is read (times P = 0) before any tile lands there
  {
    u32x4* vz = reinterpret_cast<u32x4*>(lb + V_BASE + (NSTAGE - 1) * V_BYTES);
    for (int i = tid; i < V_BYTES / 16; i += NT) vz[i] = u32x4{};
  }
  const int n_tiles = (int)((a.S + KT - 1) / KT);

  // Matrix phase of iteration t: S^T - m of tile t (2 + 16 MFMAs into sacc)
  // and O^T += V^T P^T of tile t - 1 (16 MFMAs into o), alternating, with
  // the fragments read from LDS PF operations ahead; no loads are issued
  // here (a load instruction can hold its wave back, and this phase sets the
  // pace of the workgroup). Every iteration runs both
  // products (one code path keeps the register allocation tight): at t = 0
  // the PV product reads a zeroed V^T stage with P = 0, and the scores
  // computed at t = n_tiles are never used.
  auto matrix_phase = [&](int t, auto stage) {
    constexpr int STG = decltype(stage)::value;
    constexpr int PSTG = (STG + NSTAGE - 1) % NSTAGE;
    constexpr int N = 32, PF = 4;
    // op i: even -> score block (ks, kb) = (i / 4, (i / 2) % 2);
    //        odd  -> PV block (s, db) = (i / 8, (i / 2) % 4)
    auto frag = [&](int i) -> u32x4 {
      const int j = i >> 1;
      const uint32_t addr = (i & 1) == 0
          ? k_rd[j >> 1] + STG * K_BYTES + (j & 1) * 32 * KU * 16
          : v_rd[j >> 2] + PSTG * V_BYTES + (j & 3) * 32 * VU * 16;
      return *reinterpret_cast<const u32x4*>(lb + addr);
    };
    u32x4 buf[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) buf[i] = frag(i);
    sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kaug, qaug, f32x16{}, 0, 0, 0);
    sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kaug, qaug, f32x16{}, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const bf16x8 x = __builtin_bit_cast(bf16x8, buf[i % PF]);
      if (i + PF < N) buf[i % PF] = frag(i + PF);
      const int j = i >> 1;
      if ((i & 1) == 0)
        sacc[j & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, qf[j >> 1], sacc[j & 1], 0, 0, 0);
      else
        o[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, pf[j >> 2], o[j & 3], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);  // keep the read-ahead distance
    }
  };

  // probabilities exp2(sacc - shift) of this lane's 32 scores as bf16 MFMA
  // operands, their sum added to l
  auto probabilities = [&](float shift) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      f32x8 p;
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(sacc[s >> 1][8 * (s & 1) + e] - shift);
      pf[s] = pack_bf16x8(p);
#pragma unroll
      for (int e = 0; e < 8; ++e) l += p[e];
    }
  };

  // softmax phase of iteration t (t < n_tiles)
  auto softmax_phase = [&](int t) {
    if (t + 1 == n_tiles && (a.S % KT)) {
      // keys [0, valid) exist; entry i of block kb is key kb*32 + 16(i/8) + 8g + i%8
      const int lim = (int)(a.S - (int64_t)t * KT) - 8 * g;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kb * 32 + 16 * (i >> 3) + (i & 7) >= lim) sacc[kb][i] = -INFINITY;
    }
    const float l_prev = l;
    probabilities(0.f);
    if (t == 0 || __ballot(!(l <= kSumGuard)) != 0) {
      // (re)set the offset: m_new = max(m, bf16(m + tile max)); the first
      // tile sets it outright. O and l scale by 2^(m - m_new).
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sacc[kb][i]);
      tmax = half_max(tmax);
      float m_new = (float)(__bf16)(m + tmax);
      if (t > 0) m_new = fmaxf(m_new, m);
      const float shift = m_new - m;
      const float alpha = t == 0 ? 0.f : __builtin_amdgcn_exp2f(-shift);
      l = l_prev * alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] *= alpha;
      probabilities(shift);
      m = m_new;
      qaug[0] = (__bf16)(g == 0 ? -m : 0.f);
    }
    // materialise the results here, ahead of the load wait that follows
#pragma unroll
    for (int s = 0; s < 4; ++s) asm volatile("" : "+v"(pf[s]));
    asm volatile("" : "+v"(l));
  };

  // one iteration: matrix phase, barrier, softmax phase, barrier. Returns
  // true after the drain iteration t == n_tiles.
  auto iteration = [&](int t, auto stage) -> bool {
    matrix_phase(t, stage);
    wg_barrier();
    if (t < n_tiles) {
      // The softmax phase has slack against the other half's matrix phase,
      // so it carries the tile loads. Waves 0-3 request the V^T rows of tile
      // t + 2 (stage (t + 2) % 4: its last V^T reads, the PV of tile t - 2,
      // ended two phases ago), waves 4-7 the K rows of tile t + 3 (stage
      // (t + 3) % 4: its last K reads, the scores of tile t - 1, ended in the
      // previous phase).
      constexpr int STG = decltype(stage)::value;
      if (leader) {
        if (t + 2 < n_tiles) {
#pragma unroll
          for (int j = 4; j < 8; ++j) dma_part(t + 2, stage_t<(STG + 2) % NSTAGE>{}, j);
        }
      } else if (t + 3 < n_tiles) {
#pragma unroll
        for (int j = 0; j < 4; ++j) dma_part(t + 3, stage_t<(STG + 3) % NSTAGE>{}, j);
      }
      softmax_phase(t);
      // this wave's older loads have landed (the four just issued may fly):
      // V^T of tile t + 1 (waves 0-3, needed from phase 2t + 4 on) or K of
      // tile t + 2 (waves 4-7, needed from phase 2t + 4 on); the barrier
      // below publishes them
      __builtin_amdgcn_sched_barrier(0);
      if (t + (leader ? 2 : 3) < n_tiles) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    wg_barrier();
    return t == n_tiles;
  };

  if (leader) {
#pragma unroll
    for (int j = 0; j < 8; ++j) dma_part(0, stage_t<0>{}, j);
    if (n_tiles > 1) {
#pragma unroll
      for (int j = 0; j < 8; ++j) dma_part(1, stage_t<1>{}, j);
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
  }
  __syncthreads();  // tiles 0 (and 1) requested, tile 0 landed, zero stage written
  if (!leader) {
    // K rows of tile 2 (their first reader is phase 4), then lag by one phase
    if (n_tiles > 2) {
#pragma unroll
      for (int j = 0; j < 4; ++j) dma_part(2, stage_t<2>{}, j);
    }
    wg_barrier();
  }
  for (int t = 0;; t += NSTAGE) {
    if (iteration(t, stage_t<0>{})) break;
    if (iteration(t + 1, stage_t<1>{})) break;
    if (iteration(t + 2, stage_t<2>{})) break;
    if (iteration(t + 3, stage_t<3>{})) break;
  }
  if (leader) wg_barrier();  // match the lagging waves' barrier count

  // normalise and store: lane holds query q0 + qi, dims db*32 + 8 j + 4 g + 0..3
  l = half_sum(l);
  const int64_t q = q0 + qi;
  if (q >= a.S) return;
  const float inv = 1.f / l;
  int64_t row;
  if (!a.stream_major) row = (int64_t)b * a.S + q;
  else if (q < a.n_txt) row = (int64_t)b * a.n_txt + q;
  else row = (int64_t)a.B * a.n_txt + (int64_t)b * (a.S - a.n_txt) + (q - a.n_txt);
  bf16_t* out = a.o + row * a.ldo + h * 128;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = o[db][4 * j + e] * inv;
      *reinterpret_cast<u32x2*>(out + db * 32 + 8 * j + 4 * g) = pack_bf16x4(v);
    }
}


// Workgroups (query blocks) of one attention launch.
inline int64_t attention_units(const AttnArgs& a) {
  return ((a.S + QB - 1) / QB) * a.H * a.B;
}

}  // namespace att
}  // namespace dit
