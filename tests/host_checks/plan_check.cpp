// Host-only checks of libdit.so's planning code, meant to be built with
// AddressSanitizer and UndefinedBehaviorSanitizer and no HIP (see
// tests/test_host_sanitizers.py): every argument-check error path of the
// entry points, workspace-layout invariants up to the largest sizes the
// checks accept, position ids, the K-split rule and the GEMM tile map. Exits
// non-zero on the first failed expectation; prints one "layout" line per
// workspace query so the caller can compare them with the built library.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "plan.hpp"
#include "tile_map.hpp"

using namespace dit::host;

static int g_fail = 0;
#define EXPECT(cond)                                                             \
  do {                                                                           \
    if (!(cond)) {                                                               \
      std::printf("FAIL %s:%d: %s (last error: %s)\n", __FILE__, __LINE__, #cond, \
                  dit_last_error());                                             \
      g_fail = 1;                                                                \
    }                                                                            \
  } while (0)

static dit_config klein() {
  dit_config c{};
  c.hidden = 3072;
  c.heads = 24;
  c.head_dim = 128;
  c.mlp_hidden = 9216;
  c.n_dual = 5;
  c.n_single = 20;
  c.in_channels = 128;
  c.txt_channels = 7680;
  c.time_channels = 256;
  for (int a = 0; a < 4; ++a) c.axes_dim[a] = 32;
  c.prenorm = DIT_PRENORM_RMS;
  c.theta = 2000.f;
  c.eps = 1e-6f;
  return c;
}

// non-null, 256-byte aligned addresses that are never dereferenced
static void* fake(uintptr_t i = 0) { return reinterpret_cast<void*>((uintptr_t)(1 << 20) + 256 * i); }
static const float* ffake(uintptr_t i = 0) { return static_cast<const float*>(fake(i)); }

static void config_checks() {
  dit_config c = klein();
  EXPECT(dit_config_check(&c) == DIT_OK);
  EXPECT(dit_config_check(nullptr) == DIT_E_NULL);
  struct Case {
    void (*edit)(dit_config&);
    int status;
  } cases[] = {
      {[](dit_config& c) { c.head_dim = 64; c.hidden = 24 * 64; }, DIT_E_UNSUPPORTED},
      {[](dit_config& c) { c.hidden = 3000; }, DIT_E_SHAPE},
      {[](dit_config& c) { c.heads = 0; }, DIT_E_SHAPE},
      {[](dit_config& c) { c.heads = 40; c.hidden = 40 * 128; }, DIT_E_UNSUPPORTED},
      {[](dit_config& c) { c.mlp_hidden = 100; }, DIT_E_UNSUPPORTED},
      {[](dit_config& c) { c.n_dual = -1; }, DIT_E_SHAPE},
      {[](dit_config& c) { c.n_single = 2000; }, DIT_E_SHAPE},
      {[](dit_config& c) { c.in_channels = 32; }, DIT_E_UNSUPPORTED},
      {[](dit_config& c) { c.txt_channels = 100; }, DIT_E_UNSUPPORTED},
      {[](dit_config& c) { c.time_channels = 4100; }, DIT_E_UNSUPPORTED},
      {[](dit_config& c) { c.axes_dim[3] = 30; }, DIT_E_SHAPE},
      {[](dit_config& c) { c.axes_dim[1] = 31; }, DIT_E_SHAPE},
      {[](dit_config& c) { c.prenorm = 5; }, DIT_E_VALUE},
      {[](dit_config& c) { c.theta = NAN; }, DIT_E_VALUE},
      {[](dit_config& c) { c.theta = 1.f; }, DIT_E_VALUE},
      {[](dit_config& c) { c.eps = -1.f; }, DIT_E_VALUE},
      {[](dit_config& c) { c.eps = INFINITY; }, DIT_E_VALUE},
  };
  for (const Case& k : cases) {
    dit_config d = klein();
    k.edit(d);
    EXPECT(dit_config_check(&d) == k.status);
    EXPECT(std::strlen(dit_last_error()) > 0);
  }
  for (int s = -7; s <= 0; ++s) EXPECT(dit_status_string(s) != nullptr);
}

// every region of a layout is 256-byte aligned, in order, disjoint and
// inside the total
static void regions(const std::vector<std::pair<size_t, size_t>>& r, size_t total) {
  size_t end = 0;
  for (const auto& x : r) {
    EXPECT(x.first % kAlign == 0);
    EXPECT(x.first >= end);
    end = x.first + x.second;
  }
  EXPECT(end <= total && total % kAlign == 0 && total - end < kAlign);
}

static void layout_checks() {
  const int Bs[] = {1, 2, 3, 64};
  const int64_t Ss[] = {1, 96, 4608, 8672, 8704, 20960, 1 << 20};
  dit_config cfgs[3] = {klein(), klein(), klein()};
  cfgs[1].hidden = 256; cfgs[1].heads = 2; cfgs[1].mlp_hidden = 768; cfgs[1].txt_channels = 256;
  cfgs[2].hidden = 4096; cfgs[2].heads = 32; cfgs[2].mlp_hidden = 16384; cfgs[2].time_channels = 4096;
  for (int ci = 0; ci < 3; ++ci) {
    const dit_config& c = cfgs[ci];
    EXPECT(dit_config_check(&c) == DIT_OK);
    for (int B : Bs) {
      const ModLayout m = mod_layout(c, B);
      regions({{m.e, (size_t)B * c.time_channels * 4}, {m.t1, (size_t)B * c.hidden * 4},
               {m.m, (size_t)B * c.hidden * 4}}, m.total);
      EXPECT(m.total <= (size_t)DIT_NOALLOC_SCRATCH_BYTES);
      std::printf("layout %d %d %d 0 %zu\n", ci, DIT_WS_MOD, B, m.total);
      for (int64_t S : Ss) {
        const size_t D = c.hidden, F = c.mlp_hidden, R = (size_t)B * S;
        for (int kind = 0; kind < 2; ++kind) {
          const BlockLayout L = block_layout(c, kind, B, S);
          EXPECT(L.R == (int64_t)R && L.S_pad % 256 == 0 && L.S_pad >= S && L.S_pad - S < 256);
          const size_t qk = (size_t)B * c.heads * L.S_pad * 128 * 2;
          if (kind == 0)
            regions({{L.h, R * D * 2}, {L.u, R * F * 2}, {L.o, R * D * 2}, {L.q, qk}, {L.k, qk},
                     {L.vt, qk}}, L.total);
          else
            regions({{L.h, R * D * 2}, {L.d6, R * (D + F) * 2}, {L.q, qk}, {L.k, qk}, {L.vt, qk}},
                    L.total);
          std::printf("layout %d %d %d %lld %zu\n", ci, kind, B, (long long)S, L.total);
        }
        const StepLayout st = step_layout(c, B, S);
        const size_t blk = std::max(block_layout(c, 0, B, S).total, block_layout(c, 1, B, S).total);
        regions({{st.x, R * D * 4}, {st.mod, (size_t)B * DIT_MOD_ROWS * D * 4},
                 {st.modws, mod_layout(c, B).total}, {st.block, blk}}, st.total);
        std::printf("layout %d %d %d %lld %zu\n", ci, DIT_WS_STEP, B, (long long)S, st.total);
        const DenoiseLayout dn = denoise_layout(c, B, S);
        regions({{dn.step, st.total}, {dn.lat, R * c.in_channels * 2},
                 {dn.v, R * c.in_channels * 4},
                 {dn.mods, (size_t)kModSteps * B * DIT_MOD_ROWS * D * 4},
                 {dn.modws, mod_layout(c, (int64_t)kModSteps * B).total}, {dn.txt, R * D * 4}},
                dn.total);
        std::printf("layout %d %d %d %lld %zu\n", ci, DIT_WS_DENOISE, B, (long long)S, dn.total);
        EXPECT(dit_workspace_bytes(&c, DIT_WS_STEP, B, S) == st.total);
      }
    }
    EXPECT(dit_workspace_bytes(&c, DIT_WS_STEP, 0, 10) == 0);
    EXPECT(dit_workspace_bytes(&c, DIT_WS_STEP, 65, 10) == 0);
    EXPECT(dit_workspace_bytes(&c, DIT_WS_STEP, 1, (1 << 20) + 1) == 0);
    EXPECT(dit_workspace_bytes(&c, 9, 1, 10) == 0);
  }
}

static void operand_checks() {
  dit_config c = klein();
  // widest operand: the single block's [attention | SwiGLU] rows, D + F =
  // 12288 bf16; 4 GiB of 32-bit offsets
  const int64_t limit = (int64_t)(kMaxBufferBytes / (12288 * 2));
  EXPECT(check_operand_sizes(c, limit) == DIT_OK);
  EXPECT(check_operand_sizes(c, limit + 1) == DIT_E_UNSUPPORTED);
  EXPECT(check_operand_sizes(c, (int64_t)DIT_MAX_BATCH << 20) == DIT_E_UNSUPPORTED);
  dit_config w = klein();
  w.hidden = 4096; w.heads = 32; w.mlp_hidden = 1 << 19;  // (3D + 2F) D bf16 > 4 GiB
  EXPECT(check_operand_sizes(w, 1) == DIT_E_UNSUPPORTED);
}

static void validation_checks() {
  const dit_config c = klein();
  dit_dual_weights dw[5];
  for (auto& d : dw)
    for (int s = 0; s < 2; ++s) {
      d.qkv[s] = d.out[s] = d.mlp_in[s] = d.mlp_out[s] = fake(s + 1);
      d.q_gain[s] = d.k_gain[s] = ffake(s + 3);
    }
  dit_single_weights sw[20];
  for (auto& s : sw) {
    s.w_in = s.w_out = fake(5);
    s.q_gain = s.k_gain = ffake(6);
  }
  dit_model_weights m{};
  m.t_in = m.t_out = m.mod_dual_img = m.mod_dual_txt = m.mod_single = m.mod_final = fake(7);
  m.x_embed = m.ctx_embed = m.proj_out = fake(8);
  m.dual = dw;
  m.single = sw;
  float sig[64];
  for (int i = 0; i < 64; ++i) sig[i] = 0.5f;
  const size_t big = (size_t)1 << 40;
  // one linear layer: sizes, 32-bit operand offsets, overlap of y with a / w
  {
    const void* a = fake(0);
    const void* wl = reinterpret_cast<const void*>((uintptr_t)1 << 32);
    const float* y = reinterpret_cast<const float*>((uintptr_t)1 << 36);
    EXPECT(validate_linear(a, wl, y, 4608, 3072, 12288) == DIT_OK);
    EXPECT(validate_linear(a, wl, y, 0, 3072, 12288) == DIT_OK);
    EXPECT(validate_linear(a, wl, y, 4608, 3070, 12288) == DIT_E_SHAPE);
    EXPECT(validate_linear(a, wl, y, 4608, 3072, 12280) == DIT_E_SHAPE);
    EXPECT(validate_linear(a, wl, y, (int64_t)1 << 31, 128, 64) == DIT_E_SHAPE);
    EXPECT(validate_linear(a, wl, y, 174763, 128, 12288) == DIT_E_UNSUPPORTED);  // 4 GiB + of a
    EXPECT(validate_linear(a, wl, y, 174762, 128, 12288) == DIT_OK);
    EXPECT(validate_linear(a, wl, ffake(3), 4608, 3072, 12288) == DIT_E_VALUE);  // y inside a
    EXPECT(validate_linear(a, wl, ffake(3), 0, 3072, 12288) == DIT_OK);
    EXPECT(validate_linear(nullptr, wl, y, 1, 4, 64) == DIT_E_NULL);
    EXPECT(validate_linear(nullptr, nullptr, nullptr, 0, 4, 64) == DIT_OK);
  }
  // rope tables
  EXPECT(validate_rope(&c, static_cast<const int32_t*>(fake()), 10, ffake(), ffake()) == DIT_OK);
  EXPECT(validate_rope(&c, nullptr, 10, ffake(), ffake()) == DIT_E_NULL);
  EXPECT(validate_rope(&c, static_cast<const int32_t*>(fake()), -1, ffake(), ffake()) == DIT_E_SHAPE);
  EXPECT(validate_rope(&c, nullptr, 0, nullptr, nullptr) == DIT_OK);  // nothing to do
  // modulation, with a workspace and without
  float* mod = static_cast<float*>(fake(9));
  EXPECT(validate_modulation(&c, &m, sig, 4, mod, fake(), big, false) == DIT_OK);
  EXPECT(validate_modulation(&c, &m, sig, 4, mod, fake(), 16, false) == DIT_E_WORKSPACE);
  EXPECT(validate_modulation(&c, &m, sig, 4, mod, nullptr, 0, true) == DIT_OK);
  EXPECT(validate_modulation(&c, &m, sig, 64, mod, nullptr, 0, true) == DIT_OK);
  EXPECT(validate_modulation(&c, &m, sig, 65, mod, nullptr, 0, true) == DIT_E_SHAPE);
  EXPECT(validate_modulation(&c, &m, sig, 0, mod, nullptr, 0, true) == DIT_E_SHAPE);
  EXPECT(validate_modulation(&c, &m, nullptr, 1, mod, nullptr, 0, true) == DIT_E_NULL);
  sig[3] = NAN;
  EXPECT(validate_modulation(&c, &m, sig, 4, mod, nullptr, 0, true) == DIT_E_VALUE);
  sig[3] = 0.5f;
  EXPECT(validate_modulation(&c, &m, sig, 1, mod + 1, nullptr, 0, true) == DIT_E_SHAPE);
  // blocks
  float* x = static_cast<float*>(fake(10));
  EXPECT(validate_dual(&c, &dw[0], x, 1, 4608, 512, mod, mod, 17 * 3072, ffake(), ffake(), fake(),
                       big) == DIT_OK);
  EXPECT(validate_dual(&c, &dw[0], x, 1, 4608, 4609, mod, mod, 17 * 3072, ffake(), ffake(),
                       fake(), big) == DIT_E_SHAPE);
  EXPECT(validate_dual(&c, &dw[0], x, 1, 4608, 512, mod, mod, 3, ffake(), ffake(), fake(), big) ==
         DIT_E_SHAPE);
  EXPECT(validate_dual(&c, &dw[0], x, 1, 4608, 512, nullptr, mod, 0, ffake(), ffake(), fake(),
                       big) == DIT_E_NULL);
  EXPECT(validate_dual(&c, nullptr, x, 1, 4608, 512, mod, mod, 0, ffake(), ffake(), fake(), big) ==
         DIT_E_NULL);
  EXPECT(validate_dual(&c, &dw[0], x, 1, 4608, 512, mod, mod, 0, ffake(), ffake(),
                       static_cast<char*>(fake()) + 16, big) == DIT_E_WORKSPACE);
  EXPECT(validate_single(&c, &sw[0], x, 2, 8672, mod, 17 * 3072, ffake(), ffake(), fake(), big) ==
         DIT_OK);
  EXPECT(validate_single(&c, &sw[0], x, 2, 8672, mod, 17 * 3072, ffake(), ffake(), fake(), 64) ==
         DIT_E_WORKSPACE);
  EXPECT(validate_single(&c, &sw[0], x, 2, 0, mod, 0, ffake(), ffake(), fake(), big) == DIT_E_SHAPE);
  // step and sampling loop
  auto step = [&](int B, int64_t n_img, const void* lat, const float* v, size_t wsb) {
    return validate_step(&c, &m, fake(11), lat, sig, B, 512, n_img, 0, ffake(), ffake(), v, fake(),
                         wsb);
  };
  EXPECT(step(1, 4096, fake(12), ffake(13), big) == DIT_OK);
  EXPECT(step(0, 4096, fake(12), ffake(13), big) == DIT_E_SHAPE);
  EXPECT(step(1, 0, fake(12), ffake(13), big) == DIT_E_SHAPE);
  EXPECT(step(1, 4096, nullptr, ffake(13), big) == DIT_E_NULL);
  EXPECT(step(1, 4096, fake(12), ffake(13) + 1, big) == DIT_E_SHAPE);
  EXPECT(step(1, 4096, fake(12), ffake(13), 1024) == DIT_E_WORKSPACE);
  EXPECT(step(64, 8160 * 3, fake(12), ffake(13), big) == DIT_E_UNSUPPORTED);  // > 4 GiB operand
  dw[3].mlp_out[1] = nullptr;
  EXPECT(step(1, 4096, fake(12), ffake(13), big) == DIT_E_NULL);
  EXPECT(std::strstr(dit_last_error(), "mlp_out") != nullptr);
  dw[3].mlp_out[1] = fake(1);
  float sched[2 * 5] = {1.f, .75f, .5f, .25f, 0.f, .9f, .7f, .45f, .2f, 0.f};
  auto loop = [&](int B, int n_steps, const float* z, const void* ref, int64_t n_ref) {
    return validate_denoise(&c, &m, fake(11), z, ref, sched, n_steps, B, 512, 4096, n_ref, ffake(),
                            ffake(), fake(), big);
  };
  EXPECT(loop(2, 4, ffake(14), fake(15), 4096) == DIT_OK);
  EXPECT(loop(2, 0, ffake(14), fake(15), 4096) == DIT_E_SHAPE);
  EXPECT(loop(2, 65, ffake(14), fake(15), 4096) == DIT_E_SHAPE);
  EXPECT(loop(2, 4, nullptr, fake(15), 4096) == DIT_E_NULL);
  EXPECT(loop(2, 4, ffake(14), nullptr, 4096) == DIT_E_NULL);
  EXPECT(loop(2, 4, ffake(14), nullptr, 0) == DIT_OK);
  sched[7] = NAN;  // the second row's schedule is read too
  EXPECT(loop(2, 4, ffake(14), fake(15), 4096) == DIT_E_VALUE);
}

static void position_checks() {
  const int32_t rh[3] = {2, 3, 1}, rw[3] = {2, 1, 4};
  std::vector<int32_t> out(4 * 64);
  EXPECT(dit_position_ids(4, 2, 3, 3, rh, rw, out.data(), 64) == 4 + 6 + 4 + 3 + 4);
  // text rows, then image (0, r, c, 0), then reference i at t = 10 + 10 i
  EXPECT(out[4 * 3 + 3] == 3 && out[4 * 3 + 0] == 0);
  EXPECT(out[4 * (4 + 5) + 1] == 1 && out[4 * (4 + 5) + 2] == 2);
  EXPECT(out[4 * 10 + 0] == 10 && out[4 * 14 + 0] == 20 && out[4 * 17 + 0] == 30);
  EXPECT(out[4 * 20 + 2] == 3);  // last reference patch (0, 3)
  EXPECT(dit_position_ids(4, 2, 3, 3, rh, rw, out.data(), 20) == DIT_E_SHAPE);
  EXPECT(dit_position_ids(-1, 2, 3, 0, nullptr, nullptr, out.data(), 64) == DIT_E_SHAPE);
  EXPECT(dit_position_ids(4, 2, 3, 4, rh, rw, out.data(), 64) == DIT_E_SHAPE);
  EXPECT(dit_position_ids(4, 2, 3, 1, nullptr, rw, out.data(), 64) == DIT_E_NULL);
  EXPECT(dit_position_ids(4, 2, 3, 0, nullptr, nullptr, nullptr, 64) == DIT_E_NULL);
  EXPECT(dit_position_ids(0, 0, 0, 0, nullptr, nullptr, nullptr, 0) == 0);
}

static void split_and_tile_checks() {
  for (int64_t N = 32; N <= 1 << 15; N *= 2)
    for (int64_t K = 64; K <= 1 << 14; K += 64) {
      const int g = split_k_chunks(N, K);
      EXPECT(g >= 1 && g <= 8);
    }
  std::mt19937 rng(7);
  for (int trial = 0; trial < 20000; ++trial) {
    const int count = 1 + (int)(rng() % 8);
    int t[8];
    long total = 0;
    for (int i = 0; i < count; ++i) {
      t[i] = (rng() % 4 == 0) ? (int)(rng() % 20) : (int)(rng() % 3000);
      total += t[i];
    }
    std::vector<std::vector<char>> seen(count);
    for (int i = 0; i < count; ++i) seen[i].assign((size_t)t[i], 0);
    const auto tiles_of = [&](int i) { return t[i]; };
    for (long b = 0; b < total; ++b) {
      int p = -1, l = -1;
      const bool ok = dit::tile_of_block<8>(tiles_of, count, (int)b, &p, &l);
      EXPECT(ok && p >= 0 && p < count && l >= 0 && l < t[p]);
      if (!ok || p < 0 || p >= count || l < 0 || l >= t[p]) return;
      EXPECT(!seen[p][l]);
      seen[p][l] = 1;
    }
  }
}

// ---------------------------------------------------------------- decoder
static dit_vae_config vae_cfg(int ci) {
  dit_vae_config c{};
  dit_vae_config_default(&c);
  if (ci == 1) {  // small widths, two layers
    const int w[4] = {32, 64, 64, 128};
    for (int i = 0; i < 4; ++i) c.block_channels[i] = w[i];
    c.layers = 2;
  } else if (ci == 2) {  // the widest the check accepts, four layers
    const int w[4] = {256, 512, 1024, 2048};
    for (int i = 0; i < 4; ++i) c.block_channels[i] = w[i];
    c.layers = 4;
  }
  return c;
}

static void fill_resnet(dit_vae_resnet& r, uintptr_t& k, bool shortcut) {
  const void** f[] = {(const void**)&r.gn1_gamma, (const void**)&r.gn1_beta, &r.conv1_w,
                      (const void**)&r.conv1_b, (const void**)&r.gn2_gamma,
                      (const void**)&r.gn2_beta, &r.conv2_w, (const void**)&r.conv2_b};
  for (auto p : f) *p = fake(k++);
  r.short_w = shortcut ? fake(k++) : nullptr;
  r.short_b = shortcut ? ffake(k++) : nullptr;
}

static dit_vae_weights vae_weights(const dit_vae_config& c) {
  dit_vae_weights w{};
  uintptr_t k = 1;
  w.lat_scale = ffake(k++);
  w.lat_shift = ffake(k++);
  w.conv_in_w = fake(k++);
  w.conv_in_b = ffake(k++);
  fill_resnet(w.mid[0], k, false);
  fill_resnet(w.mid[1], k, false);
  w.attn_gn_gamma = ffake(k++);
  w.attn_gn_beta = ffake(k++);
  for (int i = 0; i < 4; ++i) {
    w.attn_w[i] = fake(k++);
    w.attn_b[i] = ffake(k++);
  }
  for (int l = 0; l < 4; ++l)
    for (int r = 0; r < c.layers; ++r)
      fill_resnet(w.up[l][r], k, vae_resnet_in(c, l, r) != vae_level_channels(c, l));
  for (int l = 0; l < 3; ++l) {
    w.upconv_w[l] = fake(k++);
    w.upconv_b[l] = ffake(k++);
  }
  w.norm_out_gamma = ffake(k++);
  w.norm_out_beta = ffake(k++);
  w.conv_out_w = fake(k++);
  w.conv_out_b = ffake(k++);
  return w;
}

static void vae_checks() {
  // configuration rules
  dit_vae_config c = vae_cfg(0);
  EXPECT(check_vae_config(&c) == DIT_OK);
  EXPECT(check_vae_config(nullptr) == DIT_E_NULL);
  c.block_channels[2] = 384;
  EXPECT(check_vae_config(&c) == DIT_E_UNSUPPORTED);
  c = vae_cfg(0);
  c.groups = 48;
  EXPECT(check_vae_config(&c) == DIT_E_UNSUPPORTED);
  c = vae_cfg(0);
  c.eps = NAN;
  EXPECT(check_vae_config(&c) == DIT_E_VALUE);
  c = vae_cfg(0);
  c.layers = 5;
  EXPECT(check_vae_config(&c) == DIT_E_UNSUPPORTED);

  // GroupNorm blocks cover the pixels exactly once
  for (int C : {8, 32, 128, 512, 2048})
    for (int64_t HW : {1ll, 77ll, 4096ll, 16384ll, 1048576ll, 8355840ll}) {
      int ppb, nblk;
      gn_blocks(HW, C, &ppb, &nblk);
      EXPECT(ppb % (256 / (C / 8)) == 0 && ppb > 0);
      EXPECT((int64_t)nblk * ppb >= HW && (int64_t)(nblk - 1) * ppb < HW);
    }

  // layouts: regions disjoint and aligned; one line per query
  const int grids[][2] = {{1, 1}, {2, 3}, {3, 5}, {32, 32}, {64, 64}, {68, 120}, {39, 53}};
  for (int ci = 0; ci < 3; ++ci) {
    const dit_vae_config vc = vae_cfg(ci);
    int cmax = 0;
    for (int i = 0; i < 4; ++i) cmax = std::max(cmax, vc.block_channels[i]);
    for (int B : {1, 2, 4, 64})
      for (const auto& g : grids) {
        const VaeLayout L = vae_layout(vc, B, g[0], g[1]);
        regions({{L.p, (size_t)(B * L.act * 2)}, {L.q, (size_t)(B * L.act * 2)},
                 {L.t, (size_t)(B * L.act * 2)}, {L.h, (size_t)(B * L.act_h * 2)},
                 {L.lat, (size_t)(B * L.n0 * vc.z_channels * 2)},
                 {L.part, (size_t)(B * L.gn_nblk * vc.groups * 2 * 4)},
                 {L.ab, (size_t)(B * cmax * 2 * 4)},
                 {L.s, (size_t)(L.mq * L.ld * 4)}, {L.pm, (size_t)(L.mq * L.ld * 2)},
                 {L.vt, (size_t)(B * vc.block_channels[3] * L.ld * 2)}},
                L.total);
        EXPECT(L.ld % 8 == 0 && L.ld >= L.n0 && L.mq >= 1 && L.mq <= L.n0);
        EXPECT(L.mq == L.n0 || L.mq % 256 == 0);
        EXPECT(L.mq * L.ld * 2 <= 0x7FFFFFFFll || L.mq == 256);
        std::printf("vae_layout %d %d %d %d %zu\n", ci, B, g[0], g[1], L.total);
      }
  }

  // decode validation: each error before any launch
  const dit_vae_config vc = vae_cfg(0);
  dit_vae_weights w = vae_weights(vc);
  const float* z = ffake(9000);
  float* img = static_cast<float*>(fake(9001));
  void* ws = fake(9002);
  const size_t need = vae_layout(vc, 1, 4, 4).total;
  EXPECT(validate_vae_decode(&vc, &w, z, 1, 4, 4, img, ws, need) == DIT_OK);
  EXPECT(validate_vae_decode(nullptr, &w, z, 1, 4, 4, img, ws, need) == DIT_E_NULL);
  EXPECT(validate_vae_decode(&vc, nullptr, z, 1, 4, 4, img, ws, need) == DIT_E_NULL);
  EXPECT(validate_vae_decode(&vc, &w, nullptr, 1, 4, 4, img, ws, need) == DIT_E_NULL);
  EXPECT(validate_vae_decode(&vc, &w, z, 0, 4, 4, img, ws, need) == DIT_E_SHAPE);
  EXPECT(validate_vae_decode(&vc, &w, z, 65, 4, 4, img, ws, need) == DIT_E_SHAPE);
  EXPECT(validate_vae_decode(&vc, &w, z, 1, 0, 4, img, ws, need) == DIT_E_SHAPE);
  EXPECT(validate_vae_decode(&vc, &w, z, 1, 4, 3000, img, ws, need) == DIT_E_SHAPE);
  EXPECT(validate_vae_decode(&vc, &w, z, 1, 200, 200, img, ws, need) == DIT_E_UNSUPPORTED);
  EXPECT(validate_vae_decode(&vc, &w, z, 1, 4, 4, img, ws, need - 1) == DIT_E_WORKSPACE);
  EXPECT(validate_vae_decode(&vc, &w, z, 1, 4, 4, img, fake(9003) , need) == DIT_OK);
  EXPECT(validate_vae_decode(&vc, &w, ffake(9000) + 1, 1, 4, 4, img, ws, need) == DIT_E_SHAPE);
  dit_vae_weights w2 = w;
  w2.up[2][1].conv2_w = nullptr;
  EXPECT(validate_vae_decode(&vc, &w2, z, 1, 4, 4, img, ws, need) == DIT_E_NULL);
  w2 = w;
  w2.up[1][0].short_w = fake(9100);  // 512 -> 512 keeps its width
  EXPECT(validate_vae_decode(&vc, &w2, z, 1, 4, 4, img, ws, need) == DIT_E_NULL);
  w2 = w;
  w2.up[2][0].short_b = nullptr;  // 512 -> 256 needs its shortcut
  EXPECT(validate_vae_decode(&vc, &w2, z, 1, 4, 4, img, ws, need) == DIT_E_NULL);
  w2 = w;
  w2.attn_b[3] = nullptr;
  EXPECT(validate_vae_decode(&vc, &w2, z, 1, 4, 4, img, ws, need) == DIT_E_NULL);

  // the building blocks
  const void* x = fake(9200);
  EXPECT(validate_vae_conv(x, 64, 3, 0, x, ffake(1), nullptr, 0, nullptr, nullptr, nullptr, 1, 8, 8,
                           64, fake(9201)) == DIT_OK);
  EXPECT(validate_vae_conv(x, 60, 3, 0, x, ffake(1), nullptr, 0, nullptr, nullptr, nullptr, 1, 8, 8,
                           64, fake(9201)) == DIT_E_SHAPE);
  EXPECT(validate_vae_conv(x, 64, 3, 1, x, ffake(1), nullptr, 0, nullptr, nullptr, nullptr, 1, 7, 8,
                           64, fake(9201)) == DIT_E_SHAPE);
  EXPECT(validate_vae_conv(x, 64, 3, 0, x, ffake(1), x, 0, x, nullptr, nullptr, 1, 8, 8, 64,
                           fake(9201)) == DIT_E_SHAPE);
  EXPECT(validate_vae_conv(x, 64, 3, 0, x, ffake(1), x, 64, nullptr, nullptr, nullptr, 1, 8, 8, 64,
                           fake(9201)) == DIT_E_NULL);
  EXPECT(validate_vae_conv(x, 512, 3, 0, x, ffake(1), nullptr, 0, nullptr, nullptr, nullptr, 1,
                           32000, 32000, 64, fake(9201)) == DIT_E_UNSUPPORTED);
  const size_t gws = vae_group_norm_ws(2, 1000, 128, 32);
  EXPECT(validate_vae_group_norm(x, fake(9300), ffake(1), ffake(2), 2, 1000, 128, 32, 1e-6f, ws,
                                 gws) == DIT_OK);
  EXPECT(validate_vae_group_norm(x, x, ffake(1), ffake(2), 2, 1000, 128, 32, 1e-6f, ws, gws) ==
         DIT_E_VALUE);
  EXPECT(validate_vae_group_norm(x, fake(9300), ffake(1), ffake(2), 2, 1000, 96, 32, 1e-6f, ws,
                                 gws) == DIT_E_UNSUPPORTED);
  EXPECT(validate_vae_group_norm(x, fake(9300), ffake(1), ffake(2), 2, 1000, 128, 32, 1e-6f, ws,
                                 gws - 1) == DIT_E_WORKSPACE);
}

int main() {
  config_checks();
  layout_checks();
  operand_checks();
  validation_checks();
  position_checks();
  split_and_tile_checks();
  vae_checks();
  std::printf(g_fail ? "plan_check: FAILED\n" : "plan_check: ok\n");
  return g_fail;
}
