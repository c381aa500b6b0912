// Host-side checks of libmoe's C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer: api.cpp compiled for the host alone, every
// kernel launcher replaced by a stub that records the call and launches
// nothing. Valid calls walk the whole launch sequence (layouts, pointer
// arithmetic, argument structs); invalid ones must be refused before any
// launch. Device pointers are fake addresses that nothing dereferences.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "../../include/moe.h"

extern int g_launches;   // stubs.cpp

static int g_fail = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__,     \
              __LINE__, #cond);                                        \
      ++g_fail;                                                        \
    }                                                                  \
  } while (0)

static void* fake(uintptr_t i) { return reinterpret_cast<void*>(0x100000 + 0x1000 * i); }

static moe_config cfg(int d, int E, int k, int S, int F, int rank = 0, int dtype = MOE_BF16,
                      int score = MOE_SOFTMAX, int capacity = 0) {
  moe_config c;
  memset(&c, 0, sizeof c);
  c.hidden = d;
  c.n_routed = E;
  c.top_k = k;
  c.n_shared = S;
  c.ffn = F;
  c.rank = rank;
  c.score = score;
  c.renorm_topk = 1;
  c.capacity = capacity;
  c.aux_coef = 0.01f;
  c.dtype = dtype;
  return c;
}

static moe_weights weights() {
  moe_weights w;
  void** p = reinterpret_cast<void**>(&w);
  for (size_t i = 0; i < sizeof w / sizeof(void*); ++i) p[i] = fake(i + 1);
  w.select_bias = nullptr;
  return w;
}

static moe_outputs outputs() {
  moe_outputs o;
  void** p = reinterpret_cast<void**>(&o);
  for (size_t i = 0; i < sizeof o / sizeof(void*); ++i) p[i] = fake(100 + i);
  return o;
}

static moe_grads grads() {
  moe_grads g;
  void** p = reinterpret_cast<void**>(&g);
  for (size_t i = 0; i < sizeof g / sizeof(void*); ++i) p[i] = fake(200 + i);
  return g;
}

// A 256-byte aligned fake workspace address of any size (never touched).
static void* ws_addr() { return fake(4096); }

static void forward_cases() {
  struct Case {
    moe_config c;
    int64_t T;
  };
  std::vector<Case> cases = {
      {cfg(1024, 24, 6, 2, 640), 4096},                                    // Quartz
      {cfg(1024, 24, 6, 2, 640), 1},                                       // decode
      {cfg(1024, 24, 6, 2, 640), 0},                                       // empty
      {cfg(1024, 32, 3, 1, 512, 0, MOE_BF16, MOE_SOFTMAX, 1920), 16384},   // Moonfrost
      {cfg(1536, 48, 4, 1, 768, 0, MOE_BF16, MOE_SIGMOID), 32768},         // Sutra
      {cfg(768, 1024, 2, 0, 512, 64), 24576},                              // Dormouse
      {cfg(768, 1024, 2, 2, 512, 64, MOE_FP8), 333},                       // fp8 factors
      {cfg(1024, 24, 6, 2, 640, 0, MOE_FP8), 4096},                        // fp8 experts
      {cfg(128, 8, 2, 1, 64, 0, MOE_F32), 64},                             // Tiny
      {cfg(128, 300, 8, 1, 64), 190},                                      // many experts
      {cfg(192, 13, 3, 3, 192), 257},                                      // odd E
  };
  for (auto& cs : cases) {
    moe_config c = cs.c;
    moe_weights w = weights();
    if (c.score == MOE_SIGMOID) w.select_bias = static_cast<const float*>(fake(77));
    moe_outputs o = outputs();
    const size_t need = moe_workspace_bytes(&c, cs.T);
    EXPECT(need > 0 || cs.T == 0);
    EXPECT(need % 256 == 0);
    const int before = g_launches;
    EXPECT(moe_layer_forward(&c, cs.T, fake(50), &w, &o, ws_addr(), need, nullptr) == MOE_OK);
    EXPECT(cs.T == 0 || g_launches > before);
    // every intermediate region lies inside the workspace
    for (int r = MOE_WS_H; r <= MOE_WS_HQ_SHARED_SCALE; ++r) {
      size_t off = 1, n = 1;
      EXPECT(moe_workspace_region(&c, cs.T, r, &off, &n) == MOE_OK);
      EXPECT(off + n <= need);
    }
    // the stage entry points on the same workspace
    EXPECT(moe_route(&c, cs.T, fake(50), &w, &o, ws_addr(), need, nullptr) == MOE_OK);
    EXPECT(moe_permute(&c, cs.T, fake(50), &o, fake(60), ws_addr(), need, nullptr) == MOE_OK);
    EXPECT(moe_grouped_ffn(&c, cs.T, MOE_GROUPS_ROUTED | MOE_GROUPS_SHARED, fake(60),
                           o.offsets, fake(50), &w, static_cast<float*>(fake(61)),
                           static_cast<float*>(fake(62)), ws_addr(), need, nullptr) == MOE_OK);
    EXPECT(moe_combine(&c, cs.T, static_cast<float*>(fake(61)), static_cast<float*>(fake(62)),
                       &o, nullptr) == MOE_OK);
    // one byte short, misaligned, missing
    const int n0 = g_launches;
    if (need > 0) {
      EXPECT(moe_layer_forward(&c, cs.T, fake(50), &w, &o, ws_addr(), need - 1, nullptr) ==
             MOE_EWORKSPACE);
      EXPECT(moe_layer_forward(&c, cs.T, fake(50), &w, &o,
                               static_cast<char*>(ws_addr()) + 8, need, nullptr) ==
             MOE_EWORKSPACE);
      EXPECT(moe_layer_forward(&c, cs.T, fake(50), &w, &o, nullptr, need, nullptr) ==
             MOE_EWORKSPACE);
    }
    EXPECT(g_launches == n0);
  }
}

static void backward_cases() {
  moe_config c = cfg(1024, 24, 6, 2, 640);
  for (int64_t T : {4096, 1, 0, 9000}) {
    moe_weights w = weights();
    moe_outputs o = outputs();
    moe_grads g = grads();
    const size_t need = moe_workspace_bytes(&c, T);
    const size_t bneed = moe_backward_workspace_bytes(&c, T);
    EXPECT(moe_layer_backward(&c, T, fake(50), &w, &o, static_cast<float*>(fake(70)), 1.0f, &g,
                              ws_addr(), need, fake(8192), bneed, nullptr) == MOE_OK);
  }
  // float32 dense experts: the fp32 FMA products, a | b recomputed
  for (int64_t T : {64, 1, 0, 3000}) {
    moe_config f = cfg(128, 8, 2, 1, 64, 0, MOE_F32);
    moe_weights w = weights();
    moe_outputs o = outputs();
    moe_grads g = grads();
    const int before = g_launches;
    EXPECT(moe_layer_backward(&f, T, fake(50), &w, &o, static_cast<float*>(fake(70)), 1.0f, &g,
                              ws_addr(), moe_workspace_bytes(&f, T), fake(8192),
                              moe_backward_workspace_bytes(&f, T), nullptr) == MOE_OK);
    EXPECT(g_launches > before);
  }
  // rank-64 experts without shared experts: the factor-gradient path
  moe_weights w = weights();
  moe_outputs o = outputs();
  moe_grads g = grads();
  for (int64_t T : {4096, 1, 0, 3000}) {
    moe_config r = cfg(768, 1024, 2, 0, 512, 64);
    const int before = g_launches;
    EXPECT(moe_layer_backward(&r, T, fake(50), &w, &o, static_cast<float*>(fake(70)), 1.0f, &g,
                              ws_addr(), moe_workspace_bytes(&r, T), fake(8192),
                              moe_backward_workspace_bytes(&r, T), nullptr) == MOE_OK);
    EXPECT(g_launches > before);
    for (int q = MOE_BWS_DY_ROUTED; q <= MOE_BWS_DAB_SHARED; ++q) {
      size_t off = 1, n = 1;
      EXPECT(moe_backward_workspace_region(&r, T, q, &off, &n) == MOE_OK);
      EXPECT(off + n <= moe_backward_workspace_bytes(&r, T));
    }
    moe_grads g2 = g;
    g2.dv_up = nullptr;
    EXPECT(moe_layer_backward(&r, T, fake(50), &w, &o, static_cast<float*>(fake(70)), 1.0f, &g2,
                              ws_addr(), moe_workspace_bytes(&r, T), fake(8192),
                              moe_backward_workspace_bytes(&r, T), nullptr) == MOE_EINVAL);
  }
  // rank-64 experts beside a shared expert (its dense backward in the same
  // call, split over tokens past 4096)
  for (int64_t T : {64, 5000}) {
    moe_config r1 = cfg(768, 1024, 2, 1, 512, 64);
    EXPECT(moe_layer_backward(&r1, T, fake(50), &w, &o, static_cast<float*>(fake(70)), 1.0f, &g,
                              ws_addr(), moe_workspace_bytes(&r1, T), fake(8192),
                              moe_backward_workspace_bytes(&r1, T), nullptr) == MOE_OK);
  }
  // rank 16: legal, no backward here
  moe_config r2 = cfg(768, 1024, 2, 0, 512, 16);
  EXPECT(moe_layer_backward(&r2, 64, fake(50), &w, &o, static_cast<float*>(fake(70)), 1.0f, &g,
                            ws_addr(), moe_workspace_bytes(&r2, 64), fake(8192),
                            moe_backward_workspace_bytes(&r2, 64), nullptr) == MOE_EUNSUPPORTED);
}

static void invalid_cases() {
  const int n0 = g_launches;
  moe_weights w = weights();
  moe_outputs o = outputs();
  // not a legal layer
  moe_config bad[] = {cfg(100, 8, 2, 1, 64), cfg(128, 8, 0, 1, 64), cfg(128, 8, 9, 1, 64),
                      cfg(128, 5000, 2, 1, 64), cfg(128, 8, 2, -1, 64)};
  for (auto& c : bad) {
    EXPECT(moe_workspace_bytes(&c, 64) == 0);
    EXPECT(moe_layer_forward(&c, 64, fake(50), &w, &o, ws_addr(), 1u << 30, nullptr) ==
           MOE_EINVAL);
  }
  // legal, not implemented here
  moe_config uns[] = {cfg(104, 8, 2, 1, 64), cfg(128, 32, 16, 1, 64), cfg(128, 8, 2, 1, 64, 40)};
  for (auto& c : uns)
    EXPECT(moe_layer_forward(&c, 64, fake(50), &w, &o, ws_addr(), 1u << 30, nullptr) ==
           MOE_EUNSUPPORTED);
  moe_config c = cfg(128, 8, 2, 1, 64);
  EXPECT(moe_layer_forward(&c, -1, fake(50), &w, &o, ws_addr(), 1u << 30, nullptr) == MOE_EINVAL);
  EXPECT(moe_layer_forward(&c, 64, nullptr, &w, &o, ws_addr(), 1u << 30, nullptr) == MOE_EINVAL);
  EXPECT(moe_layer_forward(nullptr, 64, fake(50), &w, &o, ws_addr(), 1u << 30, nullptr) ==
         MOE_EINVAL);
  moe_outputs o2 = o;
  o2.row_of_slot = nullptr;
  EXPECT(moe_layer_forward(&c, 64, fake(50), &w, &o2, ws_addr(), 1u << 30, nullptr) == MOE_EINVAL);
  size_t off, n;
  EXPECT(moe_workspace_region(&c, 64, 99, &off, &n) == MOE_EINVAL);
  EXPECT(moe_workspace_region(&c, 64, MOE_WS_H, nullptr, &n) == MOE_EINVAL);
  EXPECT(moe_bias_update(&c, 64, nullptr, static_cast<float*>(fake(5)), 0.1f, nullptr) ==
         MOE_EINVAL);
  EXPECT(moe_capacity(5, 4, 16384, 3, 32) == 1920);
  EXPECT(moe_capacity(1, 1, INT64_MAX / 4, 15, 1) == -1);
  EXPECT(moe_capacity(0, 1, 10, 2, 4) == -1);
  EXPECT(g_launches == n0);
  for (int s = 1; s >= -5; --s) EXPECT(moe_status_str(s) != nullptr);
}

int main() {
  forward_cases();
  backward_cases();
  invalid_cases();
  printf("host checks: %d launches stubbed, %d failures\n", g_launches, g_fail);
  return g_fail ? 1 : 0;
}
