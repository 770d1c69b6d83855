// Joint attention on gfx950: O = softmax(Q K^T / sqrt(128)) V per (batch,
// head), no mask, over all S tokens of the sequence (text rows, padded ones
// included, then image and reference rows). "flux2-klein-p100a", Caveats,
// and "tt_flux2_klein - Python reference", Things that are easy to get
// wrong: all 512 text rows take part with no mask.
//
// Flash-style, one pass over K/V with an online softmax:
//  * Workgroup = 8 waves = 256 queries (32 per wave, two waves per SIMD so
//    one wave's softmax overlaps the other's MFMAs); the wave's Q block
//    lives in registers for the whole pass.
//  * K/V advance in tiles of 64 keys that buffer loads write straight into
//    LDS (K as [key][128], V as V^T [128][key], both 16-byte-chunk swizzled),
//    three stages deep so two tiles are in flight while one is consumed.
//  * Workgroups walk (batch, head, query block) XCD-contiguously, so a
//    head's K and V^T are shared through one XCD's L2.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: each lane then holds 32 scores of ONE query,
//    so the running max / sum are lane-local (one cross-lane exchange per
//    tile for the max, one at the end for the sum).
//  * The K rows feeding the score MFMA are permuted so that the score
//    registers of a lane are, 8 at a time, exactly the operand layout of the
//    next product, O^T = V^T P^T: probabilities go from accumulator to MFMA
//    operand by a bf16 conversion, with no shuffles or LDS round trip.
//  * exp2 with log2(e)/sqrt(d) folded into one scale; the running max is
//    only raised (and O, l rescaled) when a tile's max exceeds it by more
//    than 8 (a factor 256), which keeps every probability <= 256 in fp32
//    and bf16 and skips most rescales. The result is the same softmax; only
//    the rounding differs.
//  * Keys past S in the last tile are masked to -inf (the padded V rows are
//    zero); queries past S are computed but not stored.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace dit {
namespace {

constexpr int NT = 512;    // 8 waves
constexpr int QB = 256;    // queries per workgroup (32 per wave)
constexpr int KT = 64;     // keys per tile
constexpr int NSTAGE = 3;  // LDS stages (tiles in flight)
constexpr int KU = 16;     // 16-byte units per K row (128 bf16)
constexpr int VU = 8;      // 16-byte units per V^T row (64 keys)
constexpr int K_UNITS = KT * KU;   // 1024
constexpr int V_UNITS = 128 * VU;  // 1024
constexpr int STAGE_U = K_UNITS + V_UNITS;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

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

__global__ __launch_bounds__(NT, 1) void attention_kernel(const AttnArgs a) {
  __shared__ u32x4 lds[NSTAGE * STAGE_U];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // XCD-contiguous work order: consecutive query blocks of one (b, h) run on
  // the same XCD, so that head's K and V^T stay in that XCD's L2.
  const int n_qb = (int)((a.S + QB - 1) / QB);
  const int L = xcd_remap(blockIdx.x, gridDim.x);
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
  // LDS at M0 + 16 * lane). Wave w fills K rows 8 w .. 8 w + 7 (two
  // instructions of 4 rows x 16 chunks) and V^T rows 16 w .. 16 w + 15 (two
  // of 8 rows x 8 chunks); each lane fetches the logical chunk whose
  // swizzled position is its own.
  const __amdgpu_buffer_rsrc_t k_rsrc =
      make_rsrc(a.k + bh * a.S_pad * 128, clamp_u32(a.S_pad * 128 * 2));
  const __amdgpu_buffer_rsrc_t v_rsrc =
      make_rsrc(a.vt + bh * 128 * a.S_pad, clamp_u32(a.S_pad * 128 * 2));
  uint32_t k_off[2], v_off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int krow = 8 * wave + 4 * i + (lane >> 4);
    k_off[i] = (uint32_t)((krow * 128 + (((lane & 15) ^ kswz(krow)) * 8)) * 2);
    const int vrow = 16 * wave + 8 * i + (lane >> 3);
    v_off[i] = (uint32_t)((vrow * a.S_pad + (((lane & 7) ^ vswz(vrow)) * 8)) * 2);
  }
  auto dma = [&](int t, int stage) {
    u32x4* st = lds + stage * STAGE_U;
    const uint32_t kk = (uint32_t)t * KT * 128 * 2, vk = (uint32_t)t * KT * 2;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(k_rsrc, (lds_ptr_t)(st + (8 * wave + 4 * i) * KU),
                                               16, k_off[i] + kk, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          v_rsrc, (lds_ptr_t)(st + K_UNITS + (16 * wave + 8 * i) * VU), 16, v_off[i] + vk, 0, 0, 0);
  };

  // fragment read offsets
  int k_rd[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) k_rd[kb] = (kb * 32 + key_of_row(qi)) * KU;
  const int kswz0 = kswz(key_of_row(qi));  // same for kb = 0, 1 (low 4 bits)
  const int v_rd = K_UNITS + qi * VU;      // + db * 32 rows
  const int vsw = vswz(qi);

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  float m = -INFINITY, l = 0.f;

  const int n_tiles = (int)((a.S + KT - 1) / KT);
  dma(0, 0);
  if (n_tiles > 1) dma(1, 1);

  // One 64-key tile: scores, online softmax, PV. MASKED (only the last tile
  // of a ragged sequence) sets scores of keys >= S to -inf.
  auto tile = [&](int t, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    // tile t landed (this wave's loads), then everyone's: the barrier also
    // retires all reads of tile t - 1, whose stage receives tile t + 2
    if (t + 1 < n_tiles) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t + 2 < n_tiles) dma(t + 2, (t + 2) % NSTAGE);
    const u32x4* st = lds + (t % NSTAGE) * STAGE_U;

    // S^T block: 64 keys x 32 queries as two 32x32 accumulators
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int ch = (2 * ks + g) ^ kswz0;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = __builtin_bit_cast(bf16x8, st[k_rd[kb] + ch]);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sacc[kb], 0, 0, 0);
      }
    }

    if (MASKED) {
      const int valid = (int)(a.S - (int64_t)t * KT);  // keys [0, valid) exist
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb * 32 + 16 * (i >> 3) + 8 * g + (i & 7);
          if (key >= valid) sacc[kb][i] = -INFINITY;
        }
    }
    // raw-score max of this lane's query over the tile (the scale is > 0)
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sacc[kb][i]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64)) * a.scale_log2;
    if (__ballot(tmax > m + 8.f) != 0) {
      const float mn = fmaxf(m, tmax);
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] *= alpha;
      m = mn;
    }

    // probabilities exp2(s * scale - m) -> bf16 operands of O^T += V^T P^T
    bf16x8 pf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      f32x8 p;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pv =
            __builtin_amdgcn_exp2f(fmaf(sacc[s >> 1][8 * (s & 1) + e], a.scale_log2, -m));
        p[e] = pv;
        l += pv;
      }
      pf[s] = pack_bf16x8(p);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int ch = (2 * s + g) ^ vsw;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8 vf = __builtin_bit_cast(bf16x8, st[v_rd + db * 32 * VU + ch]);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[s], o[db], 0, 0, 0);
      }
    }
  };
  for (int t = 0; t + 1 < n_tiles; ++t) tile(t, std::false_type{});
  if (a.S % KT) tile(n_tiles - 1, std::true_type{});
  else tile(n_tiles - 1, std::false_type{});

  // normalise and store: lane holds query q0 + qi, dims db*32 + 8 j + 4 g + 0..3
  l += __shfl_xor(l, 32, 64);
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

}  // namespace

hipError_t attention_launch(const AttnArgs& a, hipStream_t stream) {
  if (a.S == 0 || a.B == 0) return hipSuccess;
  const int64_t n_wg = ((a.S + QB - 1) / QB) * a.H * a.B;
  const dim3 grid((unsigned)n_wg);
  hipLaunchKernelGGL(attention_kernel, grid, dim3(NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dit
