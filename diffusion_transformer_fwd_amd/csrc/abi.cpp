// C ABI of libdit.so: the device entry points and the launch sequence of the
// DiT step (the entry points and their maths are documented in
// include/dit.h). Argument checks and workspace layouts live in plan.cpp
// (host C++ without HIP); every check runs before the first launch, so an
// error return leaves device memory untouched.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dit.h"
#include "kernels.hpp"
#include "plan.hpp"
#include "profile.hpp"

namespace dit {
namespace prof {
Profiler& state() {
  static Profiler p;
  return p;
}
}  // namespace prof
}  // namespace dit

namespace {

using namespace dit::host;

#define DIT_TRY(expr)                                                             \
  do {                                                                            \
    const hipError_t e_ = (expr);                                                 \
    if (e_ != hipSuccess)                                                         \
      return fail(DIT_E_HIP, "%s: %s", #expr, hipGetErrorString(e_));             \
  } while (0)

// ---------------------------------------------------------------- profiling
using dit::prof::timed;

// ---------------------------------------------------------------- layouts

// ---------------------------------------------------------------- fixed scratch
// Scratch of dit_modulation_forward_noalloc: the modulation's intermediate
// vectors (features e, hidden t1, SiLU input m; mod_layout) for up to
// DIT_MAX_BATCH rows at the largest time_channels and hidden that
// check_config accepts (4096 each), plus the alignment slack of its three
// regions. Every GPU the library runs on holds one copy until the process
// ends. In host code `scratch` names a host-side stand-in: kernels get the
// device address from scratch_address(), never the array's name.
constexpr size_t kScratchBytes = (size_t)DIT_MAX_BATCH * (4096 + 2 * 4096) * 4 + 3 * kAlign;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
static_assert(kScratchBytes == DIT_NOALLOC_SCRATCH_BYTES, "dit.h states the scratch size");

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
int scratch_address(void** out) {
  int dev = -1;
  DIT_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(DIT_E_UNSUPPORTED, "device %d: at most %d devices are supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    DIT_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(DIT_E_HIP, "hipGetSymbolAddress returned NULL for the scratch array");
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return DIT_OK;
}

// ---------------------------------------------------------------- validation

// ---------------------------------------------------------------- launches

using dit::bf16_t;

const bf16_t* bf(const void* p) { return static_cast<const bf16_t*>(p); }
bf16_t* bf(void* p) { return static_cast<bf16_t*>(p); }
char* at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

dit::GemmProblem problem(const void* A, int64_t lda, const void* W, int64_t ldw, int M, int N,
                         int K, int epi, void* C, int64_t ldc) {
  dit::GemmProblem p{};
  p.A = bf(A);
  p.W = bf(W);
  p.C = C;
  p.lda = lda;
  p.ldw = ldw;
  p.ldc = ldc;
  p.M = M;
  p.N = N;
  p.K = K;
  p.epi = epi;
  p.seg_len = std::max(M, 1);
  p.seg_stride = 0;
  p.seg_off = 0;
  return p;
}

void set_rows(dit::GemmProblem& p, int seg_len, int64_t seg_stride, int seg_off) {
  p.seg_len = std::max(seg_len, 1);
  p.seg_stride = seg_stride;
  p.seg_off = seg_off;
}

void gemm_work(const dit::GemmBatch& g, double& flops, double& bytes);

int run_gemm(dit::GemmBatch& g, hipStream_t st) {
  double flops, bytes;
  gemm_work(g, flops, bytes);
  DIT_TRY(timed(DIT_K_GEMM, flops, bytes, st, [&] { return dit::gemm_launch(g, st); }));
  return DIT_OK;
}

// Appends p's K chunks (multiples of 64, at most G) to g: chunk 0 writes p's
// output through p's row map, chunk j >= 1 writes fp32 partial j - 1 at
// part + (j - 1) M N ([M, N], identity rows). Returns the number of chunks.
int add_split_problems(dit::GemmBatch& g, const dit::GemmProblem& p, int G, float* part) {
  const int64_t kc = round_up((p.K + G - 1) / G, 64);
  int n = 0;
  for (int64_t k0 = 0; k0 < p.K; k0 += kc, ++n) {
    dit::GemmProblem q = p;
    q.A = p.A + k0;
    q.W = p.W + k0;
    q.K = (int)std::min<int64_t>(kc, p.K - k0);
    if (n > 0) {
      q.C = part + (size_t)(n - 1) * p.M * p.N;
      q.ldc = p.N;
      q.seg_len = std::max(p.M, 1);
      q.seg_stride = 0;
      q.seg_off = 0;
    }
    g.p[g.count++] = q;
  }
  return n;
}

int run_split_sum(const dit::SplitSumArgs& a, hipStream_t st) {
  const double bytes = (double)a.rows * a.cols * 4.0 * (2.0 + a.np);
  DIT_TRY(timed(DIT_K_SPLIT_SUM, (double)a.rows * a.cols * a.np, bytes, st,
                [&] { return dit::split_sum_launch(a, st); }));
  return DIT_OK;
}

// Runs batch g in which p (an EPI_F32 problem) is split into K chunks when
// split_k_chunks allows it, its partials fit in part_bytes at part, and g
// has room; otherwise p runs whole. p goes last into g.
int run_gemm_split_f32(dit::GemmBatch& g, const dit::GemmProblem& p, float* part,
                       size_t part_bytes, hipStream_t st) {
  if (g.count >= dit::kMaxGemmProblems) return fail(DIT_E_SHAPE, "GEMM batch full");
  int G = std::min(split_k_chunks(p.N, p.K), dit::kMaxGemmProblems - g.count);
  // partials that fit in part_bytes (a multiple of the batch size, like M,
  // so the count does not depend on B either)
  const size_t one = (size_t)std::max(p.M, 1) * p.N * 4;
  G = (int)std::min<size_t>((size_t)G, 1 + part_bytes / one);
  const int64_t kc = round_up((p.K + G - 1) / std::max(G, 1), 64);
  G = (int)((p.K + kc - 1) / kc);
  if (G < 2 || p.epi != dit::EPI_F32 || (p.N & 3) || (p.ldc & 3)) {
    g.p[g.count++] = p;
    return run_gemm(g, st);
  }
  const int n = add_split_problems(g, p, G, part);
  DIT_CHECK(run_gemm(g, st));
  dit::SplitSumArgs ss{};
  ss.c = static_cast<float*>(p.C);
  for (int j = 0; j + 1 < n; ++j) ss.p[j] = part + (size_t)j * p.M * p.N;
  ss.ldc = p.ldc;
  ss.ldp = p.N;
  ss.seg_stride = p.seg_stride;
  ss.rows = p.M;
  ss.cols = p.N;
  ss.np = n - 1;
  ss.seg_len = p.seg_len;
  ss.seg_off = p.seg_off;
  return run_split_sum(ss, st);
}

int run_norm(const dit::NormArgs& na, hipStream_t st) {
  double rows = 0;
  for (int i = 0; i < na.nseg; ++i) rows += (double)na.B * na.seg[i].seg_len;
  DIT_TRY(timed(DIT_K_MODNORM, 0.0, rows * na.D * 6.0, st,
                [&] { return dit::modnorm_launch(na, st); }));
  return DIT_OK;
}

int run_qkv_pad(const dit::QkvPadArgs& pa, hipStream_t st) {
  if (pa.S_pad <= pa.S) return DIT_OK;
  const double bytes = (double)pa.B * pa.H * (pa.S_pad - pa.S) * 128.0 * 2.0 * 3.0;
  DIT_TRY(timed(DIT_K_QKV_PAD, 0.0, bytes, st, [&] { return dit::qkv_pad_launch(pa, st); }));
  return DIT_OK;
}

// QKV projection with QK-RMSNorm + RoPE in the epilogue, then the zeros of the
// padded rows. problems[] already hold A, W, rows and the token map.
int run_qkv(const dit_config& c, const BlockLayout& L, void* ws, dit::GemmBatch& g,
            const float* const* q_gain, const float* const* k_gain, const float* cos_t,
            const float* sin_t, int32_t B, int64_t S, hipStream_t st) {
  dit::QkvEpilogue& E = g.qkv;
  E.q = bf(at(ws, L.q));
  E.k = bf(at(ws, L.k));
  E.vt = bf(at(ws, L.vt));
  E.cos_t = cos_t;
  E.sin_t = sin_t;
  for (int i = 0; i < g.count; ++i) {
    E.q_gain[i] = q_gain[i];
    E.k_gain[i] = k_gain[i];
  }
  E.S_pad = L.S_pad;
  E.H = c.heads;
  E.D = c.hidden;
  E.eps = c.eps;
  E.q_scale = (float)(1.4426950408889634 / std::sqrt((double)c.head_dim));
  DIT_CHECK(run_gemm(g, st));
  dit::QkvPadArgs pa{E.q, E.k, E.vt, S, L.S_pad, B, c.heads};
  return run_qkv_pad(pa, st);
}

double attention_flops(const dit::AttnArgs& aa) {
  return 4.0 * aa.B * aa.H * (double)aa.S * aa.S * 128.0;
}
double attention_bytes(const dit::AttnArgs& aa) {
  return (double)aa.B * aa.H * aa.S * 128.0 * 2.0 * 4.0;
}

int run_attention(const dit::AttnArgs& aa, hipStream_t st) {
  DIT_TRY(timed(DIT_K_ATTENTION, attention_flops(aa), attention_bytes(aa), st,
                [&] { return dit::attention_launch(aa, st); }));
  return DIT_OK;
}

// GEMM problems' algorithmic FLOPs and bytes (each operand read once, each
// result written once; a gated residual is read and written).
void gemm_work(const dit::GemmBatch& g, double& flops, double& bytes) {
  flops = bytes = 0;
  for (int i = 0; i < g.count; ++i) {
    const dit::GemmProblem& p = g.p[i];
    const double n_w = p.epi == dit::EPI_SWIGLU ? 2.0 * p.N : (double)p.N;
    flops += 2.0 * p.M * n_w * p.K;
    const double out = p.epi == dit::EPI_RESID ? 8.0 : (p.epi == dit::EPI_F32 ? 4.0 : 2.0);
    bytes += 2.0 * p.M * p.K + 2.0 * n_w * p.K + out * p.M * p.N;
  }
}

// Attention fused with the GEMM batch g (bf16 family, independent of it).
int run_attention_gemm(const dit::AttnArgs& aa, dit::GemmBatch& g, hipStream_t st) {
  if (g.count == 0) return run_attention(aa, st);
  double flops, bytes;
  gemm_work(g, flops, bytes);
  DIT_TRY(timed(DIT_K_ATTN_GEMM, flops + attention_flops(aa), bytes + attention_bytes(aa), st,
                [&] { return dit::attn_gemm_launch(aa, g, st); }));
  return DIT_OK;
}

int run_gemv(const dit::GemvArgs& g, hipStream_t st) {
  double bytes = 0;
  for (int i = 0; i < g.nseg; ++i) bytes += 2.0 * g.seg[i].rows * g.K;
  bytes += 4.0 * g.B * (g.K + g.total_rows);
  DIT_TRY(timed(DIT_K_GEMV, 2.0 * g.B * g.total_rows * g.K, bytes, st,
                [&] { return dit::gemv_launch(g, st); }));
  return DIT_OK;
}

int launch_modulation(const dit_config& c, const dit_model_weights& w, const float* sigma,
                      int32_t B, float* mod, void* ws, hipStream_t st) {
  const ModLayout L = mod_layout(c, B);
  const int64_t D = c.hidden;
  float* e = reinterpret_cast<float*>(at(ws, L.e));
  float* t1 = reinterpret_cast<float*>(at(ws, L.t1));
  float* m = reinterpret_cast<float*>(at(ws, L.m));
  for (int b0 = 0; b0 < B; b0 += 4) {
    const int nb = std::min(4, B - b0);
    dit::TimeArgs ta{};
    ta.e = e;
    ta.B = nb;
    ta.C = c.time_channels;
    for (int i = 0; i < nb; ++i) ta.sigma[i] = sigma[b0 + i];
    DIT_TRY(timed(DIT_K_TIME, 0.0, 4.0 * nb * c.time_channels, st,
                  [&] { return dit::time_features_launch(ta, st); }));
    // t1 = SiLU(W_in e)
    dit::GemvArgs g{};
    g.x = e;
    g.y = t1;
    g.ldy = D;
    g.B = nb;
    g.K = c.time_channels;
    g.act_in = dit::ACT_NONE;
    g.act_out = dit::ACT_SILU;
    g.nseg = 1;
    g.total_rows = (int)D;
    g.seg[0] = dit::GemvSegment{bf(w.t_in), 0, (int)D, 0};
    DIT_CHECK(run_gemv(g, st));
    // m = SiLU(W_out t1)
    g.x = t1;
    g.y = m;
    g.K = (int)D;
    g.seg[0] = dit::GemvSegment{bf(w.t_out), 0, (int)D, 0};
    DIT_CHECK(run_gemv(g, st));
    // mod[b] = [W_dual_img m; W_dual_txt m; W_single m; W_final m]
    g.x = m;
    g.y = mod + (int64_t)b0 * DIT_MOD_ROWS * D;
    g.ldy = DIT_MOD_ROWS * D;
    g.act_out = dit::ACT_NONE;
    g.nseg = 4;
    g.seg[0] = dit::GemvSegment{bf(w.mod_dual_img), DIT_MOD_DUAL_IMG * D, (int)(6 * D), 0};
    g.seg[1] = dit::GemvSegment{bf(w.mod_dual_txt), DIT_MOD_DUAL_TXT * D, (int)(6 * D), (int)(6 * D)};
    g.seg[2] = dit::GemvSegment{bf(w.mod_single), DIT_MOD_SINGLE * D, (int)(3 * D), (int)(12 * D)};
    g.seg[3] = dit::GemvSegment{bf(w.mod_final), DIT_MOD_FINAL * D, (int)(2 * D), (int)(15 * D)};
    g.total_rows = (int)(17 * D);
    DIT_CHECK(run_gemv(g, st));
  }
  return DIT_OK;
}

int launch_dual(const dit_config& c, const dit_dual_weights& w, float* x, int32_t B, int64_t S,
                int64_t n_txt, const float* mod_txt, const float* mod_img, int64_t mbs,
                const float* cos_t, const float* sin_t, void* ws, hipStream_t st) {
  const BlockLayout L = block_layout(c, 0, B, S);
  const int64_t D = c.hidden, F = c.mlp_hidden, n_img = S - n_txt;
  const int64_t Rt = (int64_t)B * n_txt, Ri = (int64_t)B * n_img;
  bf16_t* h = bf(at(ws, L.h));
  bf16_t* u = bf(at(ws, L.u));
  bf16_t* o = bf(at(ws, L.o));
  const float* mods[2] = {mod_txt, mod_img};
  const int64_t rows[2] = {Rt, Ri};
  const int64_t first[2] = {0, Rt};
  const int64_t segoff[2] = {0, n_txt};
  const int64_t seglen[2] = {n_txt, n_img};

  auto norm = [&](int shift_row, int scale_row) -> int {
    dit::NormArgs na{};
    na.x = x;
    na.h = h;
    na.S = S;
    na.mod_bstride = mbs;
    na.D = (int)D;
    na.B = B;
    na.kind = c.prenorm;
    na.eps = c.eps;
    na.nseg = 2;
    for (int s = 0; s < 2; ++s) {
      na.seg[s].shift = mods[s] + shift_row * D;
      na.seg[s].scale = mods[s] + scale_row * D;
      na.seg[s].out_base = first[s];
      na.seg[s].seg_off = (int)segoff[s];
      na.seg[s].seg_len = (int)seglen[s];
    }
    DIT_CHECK(run_norm(na, st));
    return DIT_OK;
  };
  // stream-major GEMM problems over h / o / act rows -> x rows (residual)
  auto resid = [&](const bf16_t* A, int64_t lda, const void* const* W, int K, int gate_row)
      -> int {
    dit::GemmBatch g{};
    g.count = 0;
    for (int s = 0; s < 2; ++s) {
      if (rows[s] == 0) continue;
      dit::GemmProblem p = problem(A + first[s] * lda, lda, W[s], K, (int)rows[s], (int)D, K,
                                   dit::EPI_RESID, x, D);
      set_rows(p, (int)seglen[s], S, (int)segoff[s]);
      p.gate = mods[s] + gate_row * D;
      p.gate_bstride = mbs;
      g.p[g.count++] = p;
    }
    return run_gemm(g, st);
  };

  // attention branch
  DIT_CHECK(norm(0, 1));
  {
    dit::GemmBatch g{};
    const float* qg[2];
    const float* kg[2];
    for (int s = 0; s < 2; ++s) {
      if (rows[s] == 0) continue;
      dit::GemmProblem p = problem(h + first[s] * D, D, w.qkv[s], D, (int)rows[s], (int)(3 * D),
                                   (int)D, dit::EPI_QKV, nullptr, 0);
      set_rows(p, (int)seglen[s], 0, (int)segoff[s]);
      qg[g.count] = w.q_gain[s];
      kg[g.count] = w.k_gain[s];
      g.p[g.count++] = p;
    }
    DIT_CHECK(run_qkv(c, L, ws, g, qg, kg, cos_t, sin_t, B, S, st));
  }
  dit::AttnArgs aa{};
  aa.q = bf(at(ws, L.q));
  aa.k = bf(at(ws, L.k));
  aa.vt = bf(at(ws, L.vt));
  aa.o = o;
  aa.S = S;
  aa.S_pad = L.S_pad;
  aa.ldo = D;
  aa.n_txt = n_txt;
  aa.B = B;
  aa.H = c.heads;
  aa.stream_major = 1;
  DIT_CHECK(run_attention(aa, st));
  DIT_CHECK(resid(o, D, w.out, (int)D, 2));

  // MLP branch
  DIT_CHECK(norm(3, 4));
  {
    dit::GemmBatch g{};
    for (int s = 0; s < 2; ++s) {
      if (rows[s] == 0) continue;
      g.p[g.count++] = problem(h + first[s] * D, D, w.mlp_in[s], D, (int)rows[s], (int)F,
                               (int)D, dit::EPI_SWIGLU, u + first[s] * F, F);
    }
    DIT_CHECK(run_gemm(g, st));
  }
  DIT_CHECK(resid(u, F, w.mlp_out, (int)F, 5));
  return DIT_OK;
}

int launch_single(const dit_config& c, const dit_single_weights& w, float* x, int32_t B,
                  int64_t S, const float* mod, int64_t mbs, const float* cos_t,
                  const float* sin_t, void* ws, hipStream_t st) {
  const BlockLayout L = block_layout(c, 1, B, S);
  const int64_t D = c.hidden, F = c.mlp_hidden, R = L.R;
  bf16_t* h = bf(at(ws, L.h));
  bf16_t* d6 = bf(at(ws, L.d6));
  const int64_t ld6 = D + F;

  dit::NormArgs na{};
  na.x = x;
  na.h = h;
  na.S = S;
  na.mod_bstride = mbs;
  na.D = (int)D;
  na.B = B;
  na.kind = c.prenorm;
  na.eps = c.eps;
  na.nseg = 1;
  na.seg[0].shift = mod;
  na.seg[0].scale = mod + D;
  na.seg[0].out_base = 0;
  na.seg[0].seg_off = 0;
  na.seg[0].seg_len = (int)S;
  DIT_CHECK(run_norm(na, st));

  // The input projection's QKV part feeds the attention; its SwiGLU part
  // does not, so its rows are split between the QKV launch and a launch
  // fused with the attention (rows [0, m1) and [m1, R)), where its tiles fill
  // the CUs the attention's last round leaves idle. The split depends on the
  // shapes only; every element's arithmetic is the same either way.
  dit::GemmProblem qkv = problem(h, D, w.w_in, D, (int)R, (int)(3 * D), (int)D, dit::EPI_QKV,
                                 nullptr, 0);
  set_rows(qkv, (int)S, 0, 0);
  const dit::GemmProblem glu = problem(h, D, bf(w.w_in) + 3 * D * D, D, (int)R, (int)F, (int)D,
                                       dit::EPI_SWIGLU, d6 + D, ld6);
  dit::AttnArgs aa{};
  aa.q = bf(at(ws, L.q));
  aa.k = bf(at(ws, L.k));
  aa.vt = bf(at(ws, L.vt));
  aa.o = d6;
  aa.S = S;
  aa.S_pad = L.S_pad;
  aa.ldo = ld6;
  aa.n_txt = 0;
  aa.B = B;
  aa.H = c.heads;
  aa.stream_major = 0;
  const int64_t m1 = dit::fused_split_rows(qkv, glu, 128, aa);
  {
    dit::GemmBatch g{};
    g.p[g.count++] = qkv;
    if (m1 > 0) {
      g.p[g.count] = glu;
      g.p[g.count++].M = (int)m1;
    }
    const float* qg[2] = {w.q_gain, nullptr};
    const float* kg[2] = {w.k_gain, nullptr};
    DIT_CHECK(run_qkv(c, L, ws, g, qg, kg, cos_t, sin_t, B, S, st));
  }
  {
    dit::GemmBatch g{};
    if (m1 < R) {
      dit::GemmProblem p = glu;
      p.A = glu.A + m1 * D;
      p.C = d6 + D + m1 * ld6;
      p.M = (int)(R - m1);
      g.p[g.count++] = p;
    }
    DIT_CHECK(run_attention_gemm(aa, g, st));
  }
  {
    dit::GemmBatch g{};
    g.count = 1;
    g.p[0] = problem(d6, ld6, w.w_out, ld6, (int)R, (int)D, (int)ld6, dit::EPI_RESID, x, D);
    set_rows(g.p[0], (int)S, S, 0);
    g.p[0].gate = mod + 2 * D;
    g.p[0].gate_bstride = mbs;
    DIT_CHECK(run_gemm(g, st));
  }
  return DIT_OK;
}

// The step after validation: enqueues modulation, embeddings, blocks and
// the final layer on st, using the step workspace at ws. With mod_pre set,
// the step's modulation vectors [B, 17, D] are taken from there instead of
// computed from sigma_host. The text rows' embedding depends on the prompt
// only: txt_save (fp32 [B, n_txt, D]) receives it, or with txt_pre it is
// copied from there instead of computed.
int launch_step(const dit_config& c, const dit_model_weights& wr, const void* txt,
                const void* latents, const float* sigma_host, int32_t B, int64_t n_txt,
                int64_t n_img, int64_t n_ref, const float* cos_dev, const float* sin_dev,
                float* v_out, void* ws, hipStream_t st, const float* mod_pre = nullptr,
                float* txt_save = nullptr, const float* txt_pre = nullptr) {
  const dit_model_weights* w = &wr;
  const int64_t S = n_txt + n_img + n_ref;
  const StepLayout L = step_layout(c, B, S);
  const int64_t D = c.hidden;
  float* x = reinterpret_cast<float*>(at(ws, L.x));
  float* mod = mod_pre ? const_cast<float*>(mod_pre) : reinterpret_cast<float*>(at(ws, L.mod));
  void* bws = at(ws, L.block);
  const int64_t mbs = DIT_MOD_ROWS * D;

  // 1. global modulation, once for the whole step
  if (!mod_pre) DIT_CHECK(launch_modulation(c, *w, sigma_host, B, mod, at(ws, L.modws), st));

  // K-split partials of the embedding and the final projection live in the
  // single block's d6 region, free before the first block and after the last
  const BlockLayout SL = block_layout(c, 1, B, S);
  float* part = reinterpret_cast<float*>(at(bws, SL.d6));
  const size_t part_bytes = (size_t)SL.R * (size_t)(D + c.mlp_hidden) * 2;

  // 2. embeddings straight into the residual rows (the text part K-split)
  {
    dit::GemmBatch g{};
    dit::GemmProblem p = problem(latents, c.in_channels, w->x_embed, c.in_channels,
                                 (int)(B * (n_img + n_ref)), (int)D, c.in_channels, dit::EPI_F32,
                                 x, D);
    set_rows(p, (int)(n_img + n_ref), S, (int)n_txt);
    g.p[g.count++] = p;
    if (n_txt > 0 && !txt_pre) {
      dit::GemmProblem t = problem(txt, c.txt_channels, w->ctx_embed, c.txt_channels,
                                   (int)(B * n_txt), (int)D, c.txt_channels, dit::EPI_F32, x, D);
      set_rows(t, (int)n_txt, S, 0);
      DIT_CHECK(run_gemm_split_f32(g, t, part, part_bytes, st));
    } else {
      DIT_CHECK(run_gemm(g, st));
    }
    if (n_txt > 0 && (txt_pre || txt_save)) {
      dit::RowsCopyArgs rc{};
      rc.src = txt_pre ? txt_pre : x;
      rc.dst = txt_pre ? x : txt_save;
      rc.n = n_txt;
      rc.src_bstride = txt_pre ? n_txt : S;
      rc.dst_bstride = txt_pre ? S : n_txt;
      rc.B = B;
      rc.D = (int)D;
      DIT_TRY(timed(DIT_K_LATENT, 0.0, 8.0 * B * n_txt * D, st,
                    [&] { return dit::rows_copy_launch(rc, st); }));
    }
  }

  // 3. blocks, all reading the one modulation buffer
  for (int i = 0; i < c.n_dual; ++i)
    DIT_CHECK(launch_dual(c, w->dual[i], x, B, S, n_txt, mod + DIT_MOD_DUAL_TXT * D,
                          mod + DIT_MOD_DUAL_IMG * D, mbs, cos_dev, sin_dev, bws, st));
  for (int i = 0; i < c.n_single; ++i)
    DIT_CHECK(launch_single(c, w->single[i], x, B, S, mod + DIT_MOD_SINGLE * D, mbs, cos_dev,
                            sin_dev, bws, st));

  // 4. final AdaLN of the image rows + projection to the latent width
  {
    const BlockLayout BL = block_layout(c, 1, B, S);
    bf16_t* h = bf(at(bws, BL.h));
    dit::NormArgs na{};
    na.x = x;
    na.h = h;
    na.S = S;
    na.mod_bstride = mbs;
    na.D = (int)D;
    na.B = B;
    na.kind = c.prenorm;
    na.eps = c.eps;
    na.nseg = 1;
    na.seg[0].shift = mod + DIT_MOD_FINAL * D;
    na.seg[0].scale = mod + (DIT_MOD_FINAL + 1) * D;
    na.seg[0].out_base = 0;
    na.seg[0].seg_off = (int)n_txt;
    na.seg[0].seg_len = (int)n_img;
    DIT_CHECK(run_norm(na, st));
    dit::GemmBatch g{};
    const dit::GemmProblem p = problem(h, D, w->proj_out, D, (int)(B * n_img), c.in_channels,
                                       (int)D, dit::EPI_F32, v_out, c.in_channels);
    DIT_CHECK(run_gemm_split_f32(g, p, part, part_bytes, st));
  }
  return DIT_OK;
}

}  // namespace

// ======================================================================= ABI

extern "C" {

int dit_rope_tables_build(const dit_config* cfg, const int32_t* pos_dev, int64_t S,
                          float* cos_dev, float* sin_dev, dit_stream_t stream) {
  DIT_CHECK(validate_rope(cfg, pos_dev, S, cos_dev, sin_dev));
  if (S == 0) return DIT_OK;
  dit::RopeArgs ra{};
  ra.pos = pos_dev;
  ra.cos_t = cos_dev;
  ra.sin_t = sin_dev;
  ra.S = S;
  ra.pairs = cfg->head_dim / 2;
  int j = 0;
  for (int a = 0; a < 4; ++a) {
    const int dim = cfg->axes_dim[a];
    for (int p = 0; p < dim / 2; ++p, ++j) {
      ra.axis_of[j] = a;
      ra.omega[j] = std::pow((double)cfg->theta, -2.0 * p / (double)dim);
    }
  }
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  DIT_TRY(timed(DIT_K_ROPE_TABLES, 0.0, (double)S * (16.0 + ra.pairs * 8.0), st,
                [&] { return dit::rope_tables_launch(ra, st); }));
  return DIT_OK;
}

int dit_modulation_forward(const dit_config* cfg, const dit_model_weights* w,
                           const float* sigma_host, int32_t B, float* mod_dev, void* ws,
                           size_t ws_bytes, dit_stream_t stream) {
  DIT_CHECK(validate_modulation(cfg, w, sigma_host, B, mod_dev, ws, ws_bytes, false));
  return launch_modulation(*cfg, *w, sigma_host, B, mod_dev, ws,
                           reinterpret_cast<hipStream_t>(stream));
}

int dit_modulation_forward_noalloc(const dit_config* cfg, const dit_model_weights* w,
                                   const float* sigma_host, int32_t B, float* mod_dev,
                                   dit_stream_t stream) {
  DIT_CHECK(validate_modulation(cfg, w, sigma_host, B, mod_dev, nullptr, 0, true));
  void* ws = nullptr;
  DIT_CHECK(scratch_address(&ws));
  return launch_modulation(*cfg, *w, sigma_host, B, mod_dev, ws,
                           reinterpret_cast<hipStream_t>(stream));
}

int dit_dual_block_forward(const dit_config* cfg, const dit_dual_weights* w, float* x,
                           int32_t B, int64_t S, int64_t n_txt, const float* mod_txt,
                           const float* mod_img, int64_t mod_batch_stride,
                           const float* cos_dev, const float* sin_dev, void* ws,
                           size_t ws_bytes, dit_stream_t stream) {
  DIT_CHECK(validate_dual(cfg, w, x, B, S, n_txt, mod_txt, mod_img, mod_batch_stride, cos_dev,
                          sin_dev, ws, ws_bytes));
  return launch_dual(*cfg, *w, x, B, S, n_txt, mod_txt, mod_img, mod_batch_stride, cos_dev,
                     sin_dev, ws, reinterpret_cast<hipStream_t>(stream));
}

int dit_single_block_forward(const dit_config* cfg, const dit_single_weights* w, float* x,
                             int32_t B, int64_t S, const float* mod, int64_t mod_batch_stride,
                             const float* cos_dev, const float* sin_dev, void* ws,
                             size_t ws_bytes, dit_stream_t stream) {
  DIT_CHECK(validate_single(cfg, w, x, B, S, mod, mod_batch_stride, cos_dev, sin_dev, ws,
                            ws_bytes));
  return launch_single(*cfg, *w, x, B, S, mod, mod_batch_stride, cos_dev, sin_dev, ws,
                       reinterpret_cast<hipStream_t>(stream));
}

int dit_step_forward(const dit_config* cfg, const dit_model_weights* w, const void* txt,
                     const void* latents, const float* sigma_host, int32_t B, int64_t n_txt,
                     int64_t n_img, int64_t n_ref, const float* cos_dev, const float* sin_dev,
                     float* v_out, void* ws, size_t ws_bytes, dit_stream_t stream) {
  DIT_CHECK(validate_step(cfg, w, txt, latents, sigma_host, B, n_txt, n_img, n_ref, cos_dev,
                          sin_dev, v_out, ws, ws_bytes));
  return launch_step(*cfg, *w, txt, latents, sigma_host, B, n_txt, n_img, n_ref, cos_dev,
                     sin_dev, v_out, ws, reinterpret_cast<hipStream_t>(stream));
}

int dit_linear_forward(const void* a, const void* w, float* y, int64_t M, int32_t N,
                       int32_t K, dit_stream_t stream) {
  DIT_CHECK(validate_linear(a, w, y, M, N, K));
  if (M == 0) return DIT_OK;
  dit::GemmBatch g{};
  g.p[g.count++] = problem(a, K, w, K, (int)M, N, K, dit::EPI_F32, y, N);
  return run_gemm(g, reinterpret_cast<hipStream_t>(stream));
}

int dit_denoise_forward(const dit_config* cfg, const dit_model_weights* w, const void* txt,
                        float* z, const void* ref, const float* sigmas_host, int32_t n_steps,
                        int32_t B, int64_t n_txt, int64_t n_img, int64_t n_ref,
                        const float* cos_dev, const float* sin_dev, void* ws, size_t ws_bytes,
                        dit_stream_t stream) {
  DIT_CHECK(validate_denoise(cfg, w, txt, z, ref, sigmas_host, n_steps, B, n_txt, n_img, n_ref,
                             cos_dev, sin_dev, ws, ws_bytes));
  const int64_t S = n_txt + n_img + n_ref;
  const DenoiseLayout L = denoise_layout(*cfg, B, S);

  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int64_t C = cfg->in_channels;
  float* v = reinterpret_cast<float*>(at(ws, L.v));
  dit::LatentArgs la{};
  la.z = z;
  la.v = v;
  la.ref = static_cast<const bf16_t*>(ref);
  la.lat = bf(at(ws, L.lat));
  la.n_img = n_img;
  la.n_ref = n_ref;
  la.B = B;
  la.C = (int32_t)C;
  DIT_TRY(timed(DIT_K_LATENT, 0.0, (double)B * (n_img * C * 6.0 + n_ref * C * 4.0), st,
                [&] { return dit::latent_pack_launch(la, st); }));
  // the modulation of up to kModSteps steps at a time: rows [step][b]
  float* mods = reinterpret_cast<float*>(at(ws, L.mods));
  const int64_t step_mod = (int64_t)B * DIT_MOD_ROWS * cfg->hidden;
  std::vector<float> sig((size_t)kModSteps * B);
  for (int i0 = 0; i0 < n_steps; i0 += kModSteps) {
    const int G = std::min(kModSteps, n_steps - i0);
    for (int j = 0; j < G; ++j)
      for (int b = 0; b < B; ++b) sig[(size_t)j * B + b] = sigmas_host[(int64_t)b * (n_steps + 1) + i0 + j];
    DIT_CHECK(launch_modulation(*cfg, *w, sig.data(), G * B, mods, at(ws, L.modws), st));
    for (int j = 0; j < G; ++j) {
      const int i = i0 + j;
      for (int b = 0; b < B; ++b)
        la.dsig[b] = sigmas_host[(int64_t)b * (n_steps + 1) + i + 1] -
                     sigmas_host[(int64_t)b * (n_steps + 1) + i];
      // the text embedding is computed by the first step and kept for the rest
      float* txt_rows = reinterpret_cast<float*>(at(ws, L.txt));
      DIT_CHECK(launch_step(*cfg, *w, txt, la.lat, nullptr, B, n_txt, n_img, n_ref, cos_dev,
                            sin_dev, v, at(ws, L.step), st, mods + j * step_mod,
                            i == 0 ? txt_rows : nullptr, i == 0 ? nullptr : txt_rows));
      DIT_TRY(timed(DIT_K_LATENT, 0.0, (double)B * n_img * C * 14.0, st,
                    [&] { return dit::euler_launch(la, st); }));
    }
  }
  return DIT_OK;
}

int dit_profile_begin(void) {
  dit::prof::Profiler& g_prof = dit::prof::state();
  std::lock_guard<std::mutex> lock(g_prof.mu);
  g_prof.recs.clear();
  g_prof.on = true;
  return DIT_OK;
}

int dit_profile_end(dit_kernel_stats* out) {
  if (!out) return fail(DIT_E_NULL, "out is NULL");
  dit::prof::Profiler& g_prof = dit::prof::state();
  std::lock_guard<std::mutex> lock(g_prof.mu);
  if (!g_prof.on) return fail(DIT_E_VALUE, "dit_profile_end without dit_profile_begin");
  g_prof.on = false;
  for (int k = 0; k < DIT_K_COUNT; ++k) out[k] = dit_kernel_stats{k, 0, 0.0, 0.0, 0.0};
  int status = DIT_OK;
  for (dit::prof::Record& r : g_prof.recs) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess && status == DIT_OK)
      status = fail(DIT_E_HIP, "profile events: %s", hipGetErrorString(e));
    dit_kernel_stats& k = out[r.kind];
    k.launches += 1;
    k.total_ms += ms;
    k.flops += r.flops;
    k.bytes += r.bytes;
    g_prof.pool.push_back(r.start);
    g_prof.pool.push_back(r.stop);
  }
  g_prof.recs.clear();
  return status;
}

}  // extern "C"
