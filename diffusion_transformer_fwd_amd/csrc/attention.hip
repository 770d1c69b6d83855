// Joint attention on gfx950: O = softmax(Q K^T / sqrt(128)) V per (batch,
// head), no mask, over all S tokens of the sequence (text rows, padded ones
// included, then image and reference rows). "flux2-klein-p100a", Caveats,
// and "tt_flux2_klein - Python reference", Things that are easy to get
// wrong: all 512 text rows take part with no mask.
//
// Flash-style, one pass over K/V with an online softmax:
//  * Workgroup = 4 waves = 128 queries (32 per wave); the wave's Q block
//    lives in registers for the whole pass.
//  * K/V advance in tiles of 64 keys, double-buffered in LDS (K as
//    [key][128], V as V^T [128][key], both 16-byte-chunk swizzled).
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
#include "common.hpp"
#include "kernels.hpp"

namespace dit {
namespace {

constexpr int NT = 256;
constexpr int QB = 128;   // queries per workgroup
constexpr int KT = 64;    // keys per tile
constexpr int KU = 16;    // 16-byte units per K row (128 bf16)
constexpr int VU = 8;     // 16-byte units per V^T row (64 keys)
constexpr int K_UNITS = KT * KU;   // 1024
constexpr int V_UNITS = 128 * VU;  // 1024
constexpr int STAGE_U = K_UNITS + V_UNITS;

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

__global__ __launch_bounds__(NT, 2) void attention_kernel(const AttnArgs a) {
  __shared__ u32x4 lds[2 * STAGE_U];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t bh = (int64_t)b * a.H + h;
  const int64_t q0 = (int64_t)blockIdx.x * QB + wave * 32;
  const int qi = lane & 31, g = lane >> 5;

  // Q fragments (second MFMA operand): query q0 + qi, dims 16 ks + 8 g + 0..7
  bf16x8 qf[8];
  {
    const u32x4* qp = reinterpret_cast<const u32x4*>(a.q + (bh * a.S_pad + q0 + qi) * 128);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, qp[2 * ks + g]);
  }

  // loaders: K rows tid/16 + 16 i (unit tid%16); V^T rows tid/8 + 32 i (unit tid%8)
  const int kr = tid >> 4, kc = tid & 15;
  const int vr = tid >> 3, vc = tid & 7;
  const u32x4* kg = reinterpret_cast<const u32x4*>(a.k + (bh * a.S_pad + kr) * 128) + kc;
  const u32x4* vg = reinterpret_cast<const u32x4*>(a.vt + (bh * 128 + vr) * a.S_pad) + vc;
  const int k_st = kr * KU + (kc ^ kswz(kr));
  const int v_st = K_UNITS + vr * VU + (vc ^ vswz(vr));
  const int64_t k_rowstep = 16 * 128 / 8;          // units between K rows kr and kr+16
  const int64_t v_rowstep = 32 * a.S_pad / 8;      // units between V^T rows vr and vr+32

  u32x4 rk[4], rv[4];
  auto gload = [&](int64_t kv0) {
    const int64_t ko = kv0 * 128 / 8, vo = kv0 / 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) rk[i] = kg[ko + i * k_rowstep];
#pragma unroll
    for (int i = 0; i < 4; ++i) rv[i] = vg[vo + i * v_rowstep];
  };
  auto lstore = [&](int stage) {
    u32x4* st = lds + stage * STAGE_U;
#pragma unroll
    for (int i = 0; i < 4; ++i) st[k_st + i * 16 * KU] = rk[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) st[v_st + i * 32 * VU] = rv[i];
  };

  // fragment read offsets
  int k_rd[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = kb * 32 + key_of_row(qi);
    k_rd[kb] = key * KU;
  }
  const int kswz0 = kswz(key_of_row(qi));  // same for kb = 0, 1 (low 4 bits)
  const int v_rd = K_UNITS + qi * VU;      // + db * 32 rows
  const int vsw = vswz(qi);

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  float m = -INFINITY, l = 0.f;

  const int n_tiles = (int)((a.S + KT - 1) / KT);
  gload(0);
  lstore(0);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int cur = t & 1;
    const bool more = t + 1 < n_tiles;
    if (more) gload((int64_t)(t + 1) * KT);
    const u32x4* st = lds + cur * STAGE_U;

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

    // scale to log2 units, mask keys past S, tile max for this lane's query
    const int64_t kv0 = (int64_t)t * KT;
    float tmax = -INFINITY;
    const bool tail = kv0 + KT > a.S;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float v = sacc[kb][i] * a.scale_log2;
        if (tail) {
          const int key = kb * 32 + 16 * (i >> 3) + 8 * g + (i & 7);
          if (kv0 + key >= a.S) v = -INFINITY;
        }
        sacc[kb][i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    if (__ballot(tmax > m + 8.f) != 0) {
      const float mn = fmaxf(m, tmax);
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] *= alpha;
      m = mn;
    }

    // probabilities -> bf16 operands of O^T += V^T P^T
    bf16x8 pf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      f32x8 p;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pv = __builtin_amdgcn_exp2f(sacc[s >> 1][8 * (s & 1) + e] - m);
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

    if (more) lstore(cur ^ 1);
    __syncthreads();
  }

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
  const dim3 grid((unsigned)((a.S + QB - 1) / QB), (unsigned)a.H, (unsigned)a.B);
  hipLaunchKernelGGL(attention_kernel, grid, dim3(NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dit
