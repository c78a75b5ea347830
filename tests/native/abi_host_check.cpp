// Host-side check of the C ABI's argument validation and workspace planning (include/moe.h),
// built together with the library's sources under the host sanitizers (AddressSanitizer,
// UndefinedBehaviorSanitizer) by the CPU test suite. No call here reaches a kernel launch: every
// call either plans a workspace or is rejected on the host, so no GPU is needed. Exit status 0
// and a last line "abi_host_check ok" mean every check held.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe.h"
#include "moe_internal.h"

static int failures = 0;
#define CHECK(cond, ...)              \
  do {                                \
    if (!(cond)) {                    \
      ++failures;                     \
      fprintf(stderr, "FAIL: ");      \
      fprintf(stderr, __VA_ARGS__);   \
      fprintf(stderr, "\n");          \
    }                                 \
  } while (0)

static moe_dims dims(int64_t T, int d, int E, int k, int I, int Is, int dtype) {
  moe_dims m;
  m.T = T;
  m.d = d;
  m.E = E;
  m.k = k;
  m.I = I;
  m.I_shared = Is;
  m.dtype = dtype;
  m.renormalize = 1;
  return m;
}

// fake device addresses: never dereferenced on the host, only checked for NULL and alignment
static void* at(uintptr_t a) { return (void*)a; }

int main() {
  // workspace planning over a grid of shapes, including the large layer at every few-token count
  const int64_t Ts[] = {0, 1, 2, 3, 4, 5, 6, 31, 32, 33, 63, 64, 65, 255, 256, 257, 1000, 4096, 8192, 16384};
  struct Shape { int d, E, k, I, Is; } shapes[] = {
      {8192, 512, 10, 2048, 2048}, {2048, 256, 8, 512, 512}, {256, 16, 2, 128, 128}, {264, 40, 3, 136, 72},
      {64, 1, 1, 32, 32},          {512, 1024, 16, 128, 0},  {4096, 8, 2, 256, 512}, {768, 6, 3, 512, 256}};
  for (const Shape& s : shapes)
    for (int64_t T : Ts)
      for (int dt = 0; dt <= 1; ++dt) {
        moe_dims m = dims(T, s.d, s.E, s.k, s.I, s.Is, dt);
        size_t bytes = 0;
        const moe_status st = moe_workspace_size(&m, &bytes);
        CHECK(st == MOE_OK, "workspace_size T=%lld d=%d E=%d: %s", (long long)T, s.d, s.E, moe_last_error());
        CHECK(bytes % 256 == 0, "workspace size %zu not a multiple of 256", bytes);
      }
  // few-token plans: the skinny kernels stream whole LDS stages (16 gate/up or 32 down weight
  // rows) of K splits that fit their A rows' room, and the counter banks hold a counter per
  // column block of either product (and per FP8 panel of the output) for every listed tile
  int skinny_plans = 0;
  for (const Shape& s : shapes)
    for (int64_t T : Ts) {
      moe_dims m = dims(T, s.d, s.E, s.k, s.I, s.Is, MOE_BF16);
      const moe::FfnPlan P = moe::ffn_plan(m);
      if (!P.skinny) continue;
      ++skinny_plans;
      const moe::Layout L = moe::make_layout(m);
      const int kr1 = moe::kSkinnyMat1 / 512, kr2 = moe::kSkinnyMat2 / 512;
      CHECK(P.kc1 > 0 && P.kc1 % kr1 == 0 && P.kc1 <= moe::kSkinnyMaxKC, "skinny gate/up kc %d d=%d", P.kc1, s.d);
      CHECK(P.kc2 > 0 && P.kc2 % kr2 == 0 && P.kc2 <= moe::kSkinnyMaxKC, "skinny down kc %d d=%d", P.kc2, s.d);
      CHECK(s.d % kr1 == 0 && s.I % kr2 == 0 && s.Is % kr2 == 0, "skinny K not whole stages d=%d", s.d);
      CHECK((int64_t)P.ks1 * P.kc1 >= s.d && (int64_t)(P.ks1 - 1) * P.kc1 < s.d, "gate/up splits %d x %d", P.ks1,
            P.kc1);
      CHECK(L.ffn_cnt_per_tile >= P.cb1 && L.ffn_cnt_per_tile >= P.cb2 && L.ffn_cnt_per_tile >= s.d / 128,
            "counters per tile %d (cb %d %d, d %d)", L.ffn_cnt_per_tile, P.cb1, P.cb2, s.d);
    }
  CHECK(skinny_plans >= 8, "only %d skinny plans checked", skinny_plans);
  // workspace grows with T at a fixed shape
  {
    size_t prev = 0;
    for (int64_t T : Ts) {
      moe_dims m = dims(T, 8192, 512, 10, 2048, 2048, MOE_BF16);
      size_t b = 0;
      moe_workspace_size(&m, &b);
      CHECK(b >= prev || T <= 256, "workspace shrinks from %zu to %zu at T=%lld", prev, b, (long long)T);
      prev = b;
    }
  }

  // invalid dims
  const moe_dims bad[] = {dims(-1, 64, 8, 2, 32, 32, 1),  dims(4, 12, 8, 2, 32, 32, 1), dims(4, 64, 0, 1, 32, 32, 1),
                          dims(4, 64, 8, 9, 32, 32, 1),   dims(4, 64, 8, 0, 32, 32, 1), dims(4, 64, 8, 2, 30, 32, 1),
                          dims(4, 64, 8, 2, 32, 4, 1),    dims(4, 64, 8, 2, 32, 32, 2), dims(4, 64, 1025, 2, 32, 32, 1),
                          dims(4, 64, 64, 17, 32, 32, 1), dims(INT64_MAX / 4, 64, 8, 2, 32, 32, 1),
                          dims(INT64_MAX, 64, 64, 16, 32, 32, 1), dims((1LL << 31) / 11 + 1, 64, 64, 10, 32, 32, 1)};
  for (const moe_dims& m : bad) {
    size_t b = 0;
    const moe_status st = moe_workspace_size(&m, &b);
    CHECK(st == MOE_ERR_INVALID_ARG || st == MOE_ERR_UNSUPPORTED, "bad dims accepted (status %d)", (int)st);
    CHECK(strlen(moe_last_error()) > 0, "no error text");
  }
  CHECK(moe_workspace_size(nullptr, nullptr) == MOE_ERR_INVALID_ARG, "NULL dims");
  moe_dims ok = dims(7, 64, 8, 2, 32, 32, MOE_BF16);
  CHECK(moe_workspace_size(&ok, nullptr) == MOE_ERR_INVALID_ARG, "NULL bytes");
  size_t need = 0;
  CHECK(moe_workspace_size(&ok, &need) == MOE_OK && need > 0, "workspace size");

  // every entry point rejects NULL, misaligned or short arguments before launching anything
  void* x = at(0x10000);
  void* w = at(0x20000);
  void* o = at(0x30000);
  void* ws = at(0x40000);
  float* wr = (float*)at(0x50000);
  int32_t* idx = (int32_t*)at(0x60000);
  float* tw = (float*)at(0x70000);
  hipStream_t s = nullptr;
  CHECK(moe_router_topk(&ok, nullptr, wr, nullptr, idx, tw, nullptr, ws, need, s) == MOE_ERR_INVALID_ARG, "x NULL");
  CHECK(moe_router_topk(&ok, at(0x10008), wr, nullptr, idx, tw, nullptr, ws, need, s) == MOE_ERR_INVALID_ARG,
        "x misaligned");
  CHECK(moe_router_topk(&ok, x, wr, nullptr, idx, tw, nullptr, ws, need - 256, s) == MOE_ERR_WORKSPACE, "short ws");
  CHECK(moe_router_topk(&ok, x, wr, nullptr, idx, tw, nullptr, at(0x40080), need, s) == MOE_ERR_WORKSPACE,
        "ws misaligned");
  CHECK(moe_router_topk(&ok, x, wr, nullptr, idx, tw, nullptr, nullptr, need, s) == MOE_ERR_WORKSPACE, "ws NULL");
  CHECK(moe_permute(&ok, nullptr, idx, idx, idx, ws, need, s) == MOE_ERR_INVALID_ARG, "permute NULL");
  CHECK(moe_grouped_ffn(&ok, x, idx, idx, w, w, w, nullptr, w, w, o, ws, need, s) == MOE_ERR_INVALID_ARG,
        "shared weights missing");
  CHECK(moe_combine(&ok, o, idx, nullptr, o, s) == MOE_ERR_INVALID_ARG, "combine NULL");
  CHECK(moe_combine_residual(&ok, o, idx, tw, nullptr, o, s) == MOE_ERR_INVALID_ARG, "residual NULL");
  CHECK(moe_forward(&ok, x, wr, nullptr, w, w, w, w, w, w, nullptr, nullptr, nullptr, nullptr, ws, need, s) ==
            MOE_ERR_INVALID_ARG,
        "forward out NULL");
  CHECK(moe_forward(&ok, x, wr, nullptr, w, w, w, w, w, w, o, nullptr, nullptr, nullptr, ws, 0, s) ==
            MOE_ERR_WORKSPACE,
        "forward ws 0 bytes");
  CHECK(moe_forward_block(&ok, x, w, -1.0, wr, nullptr, w, w, w, w, w, w, o, nullptr, nullptr, nullptr, ws, need,
                          s) == MOE_ERR_INVALID_ARG,
        "negative eps");
  CHECK(moe_rmsnorm(&ok, x, w, 1.0 / 0.0, o, s) == MOE_ERR_INVALID_ARG, "infinite eps");
  CHECK(moe_rmsnorm(&ok, x, nullptr, 1e-6, o, s) == MOE_ERR_INVALID_ARG, "gamma NULL");
  CHECK(moe_router_topk_stats(&ok, x, wr, nullptr, idx, tw, nullptr, nullptr, tw, ws, need, s) ==
            MOE_ERR_INVALID_ARG,
        "counts NULL");
  moe_dims f32 = dims(7, 64, 8, 2, 32, 32, MOE_F32);
  CHECK(moe_forward_fp8(&f32, x, wr, nullptr, (uint8_t*)w, (uint8_t*)w, (uint8_t*)w, tw, tw, tw, (uint8_t*)w,
                        (uint8_t*)w, (uint8_t*)w, tw, tw, tw, o, nullptr, nullptr, nullptr, ws, need,
                        s) == MOE_ERR_UNSUPPORTED,
        "fp8 with fp32 activations");
  CHECK(moe_quantize_fp8(w, MOE_BF16, 1, 30, 128, (uint8_t*)o, tw, s) == MOE_ERR_UNSUPPORTED, "fp8 K %% 32");
  CHECK(moe_quantize_fp8(w, MOE_BF16, 1, 32, 100, (uint8_t*)o, tw, s) == MOE_ERR_UNSUPPORTED, "fp8 N %% 128");
  CHECK(moe_quantize_fp8(w, 7, 1, 32, 128, (uint8_t*)o, tw, s) == MOE_ERR_INVALID_ARG, "fp8 dtype");
  CHECK(moe_quantize_fp8(w, MOE_BF16, 70000, 32, 128, (uint8_t*)o, tw, s) == MOE_ERR_INVALID_ARG, "fp8 batch");
  CHECK(moe_profile_next_forward(99, nullptr, nullptr) == MOE_ERR_INVALID_ARG, "profile kernel id");
  CHECK(moe_profile_next_forward(MOE_KERNEL_NONE, nullptr, nullptr) == MOE_OK, "profile cancel");

  // T = 0 is a no-op that needs no pointers
  moe_dims zero = dims(0, 64, 8, 2, 32, 32, MOE_BF16);
  CHECK(moe_forward(&zero, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                    nullptr, nullptr, nullptr, nullptr, 0, s) == MOE_OK,
        "T = 0 forward");
  for (int st = 0; st <= 5; ++st) CHECK(moe_status_string((moe_status)st) != nullptr, "status string %d", st);

  if (failures) {
    fprintf(stderr, "%d failure(s)\n", failures);
    return 1;
  }
  printf("abi_host_check ok\n");
  return 0;
}
