// Joint attention on gfx950: O = softmax(Q K^T / sqrt(128)) V per (batch,
// head), no mask, over all S tokens of the sequence (text rows, padded ones
// included, then image and reference rows). "flux2-klein-p100a", Caveats,
// and "tt_flux2_klein - Python reference", Things that are easy to get
// wrong: all 512 text rows take part with no mask.
//
// Flash-style, one pass over K/V with an online softmax:
//  * Q arrives pre-scaled by log2(e) / sqrt(head_dim) (the QK-norm/RoPE
//    kernel applies it before rounding to bf16), so a score in log2 units is
//    a plain dot product and the probability is exp2(score - m).
//  * Workgroup = 8 waves = 256 queries (32 per wave); a wave's Q block lives
//    in registers for the whole pass.
//  * K/V advance in tiles of 64 keys that buffer loads write straight into
//    LDS (K as [key][128], V as V^T [128][key], both 16-byte-chunk swizzled),
//    four stages deep.
//  * Ping-pong: waves 0-3 and waves 4-7 (one of each on every SIMD) run the
//    same loop half an iteration apart. An iteration is a matrix phase
//    (scores of tile t and the P V product of tile t - 1: 34 MFMAs) and a
//    softmax phase (exp2 and bf16 packing of tile t: vector ALU only), each
//    closed by a workgroup barrier, so one wave's MFMAs run under its
//    partner's softmax.
//  * The tile loads ride in the softmax phases, which have slack against the
//    partner's matrix phase (a load instruction can hold its wave back, and
//    the matrix phase sets the pace): waves 0-3 request the V^T rows of tile
//    t + 2, waves 4-7 the K rows of tile t + 3 (tiles 0 and 1 come whole
//    from waves 0-3 before the loop, the K rows of tile 2 from waves 4-7).
//    Each wave waits for its own older loads at the end of its softmax phase
//    and the barrier after it publishes them; a load only overwrites a stage
//    whose last reads ended before an earlier barrier.
//  * Workgroups walk (batch, head, query block) XCD-contiguously, so a
//    head's K and V^T are shared through one XCD's L2.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: each lane then holds 32 scores of ONE query,
//    so the softmax bookkeeping is lane-local.
//  * The K rows feeding the score MFMA are permuted so that the score
//    registers of a lane are, 8 at a time, exactly the operand layout of the
//    next product, O^T = V^T P^T: probabilities go from accumulator to MFMA
//    operand by a bf16 conversion, with no shuffles or LDS round trip.
//  * The running max m (per query, kept exactly representable in bf16) is
//    subtracted by the score MFMA itself: a ninth k-step multiplies a key
//    column of ones by a query row of -m, so the accumulator ends as
//    score - m and each probability costs one exp2. m is set from the first
//    tile and raised only when the row sum passes 2^64 (a guard far below
//    fp32 / bf16 overflow): softmax is invariant to the offset, so no
//    per-tile max is needed. The row sum l adds the fp32 probabilities with
//    plain adds: the bf16 dot2 instruction would share the matrix pipeline
//    with the partner wave's MFMAs and stall behind them.
//  * Keys past S in the last tile are masked to -inf (the padded V rows are
//    zero); queries past S are computed but not stored.
#include "attention_unit.hpp"

namespace dit {
namespace {

__global__ __launch_bounds__(att::NT, 1) void attention_kernel(const AttnArgs a) {
  __shared__ u32x4 lds[att::LDS_BYTES / 16];
  // XCD-contiguous work order: consecutive query blocks of one (b, h) run on
  // the same XCD, so that head's K and V^T stay in that XCD's L2.
  att::attention_unit(a, xcd_remap(blockIdx.x, gridDim.x), reinterpret_cast<char*>(lds));
}

}  // namespace

hipError_t attention_launch(const AttnArgs& a, hipStream_t stream) {
  if (a.S == 0 || a.B == 0) return hipSuccess;
  const int64_t n_wg = att::attention_units(a);
  const dim3 grid((unsigned)n_wg);
  hipLaunchKernelGGL(attention_kernel, grid, dim3(att::NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dit
