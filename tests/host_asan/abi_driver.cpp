// Host-side driver for the sanitizer build of the library (AddressSanitizer + UndefinedBehavior-
// Sanitizer on the host code; no GPU).  It calls every entry point of include/moe.h on the
// paths that return before any HIP call -- argument validation, workspace sizing and the
// capacity helper -- and checks the documented status codes.  Exit status 0 and the line
// "abi host checks: N passed" mean every check held and the sanitizers reported nothing.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "moe.h"

static int g_fail = 0, g_pass = 0;

#define CHECK(cond)                                                        \
  do {                                                                     \
    if (cond) {                                                            \
      ++g_pass;                                                            \
    } else {                                                               \
      ++g_fail;                                                            \
      std::fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);       \
    }                                                                      \
  } while (0)

static moe_shape shape(int T, int d, int de, int E, int k) {
  moe_shape s;
  std::memset(&s, 0, sizeof s);
  s.T = T; s.d = d; s.d_e = de; s.E = E; s.k = k;
  s.capacity = -1; s.renormalize = 1; s.d_e_shared = 0; s.dtype = MOE_BF16;
  s.scoring = MOE_SCORE_SOFTMAX; s.n_group = 1; s.topk_group = 1;
  s.wfmt = MOE_W_NATIVE; s.afmt = MOE_A_NATIVE;
  return s;
}

int main() {
  // status strings: every code and an unknown one
  for (int c = 0; c <= 6; ++c) CHECK(moe_status_str((moe_status)c) != nullptr);
  CHECK(std::strcmp(moe_status_str(MOE_OK), "MOE_OK") == 0);

  // capacity: floor(C T k / E) and its error paths
  int32_t cap = -7;
  CHECK(moe_capacity(8192, 1, 64, 1.25, &cap) == MOE_OK && cap == 160);
  CHECK(moe_capacity(0, 2, 8, 1.0, &cap) == MOE_OK && cap == 0);
  CHECK(moe_capacity(8, 2, 8, 1.0, nullptr) == MOE_ERR_NULL);
  CHECK(moe_capacity(-1, 2, 8, 1.0, &cap) == MOE_ERR_SHAPE);
  CHECK(moe_capacity(8, 0, 8, 1.0, &cap) == MOE_ERR_SHAPE);
  CHECK(moe_capacity(8, 2, 0, 1.0, &cap) == MOE_ERR_SHAPE);
  CHECK(moe_capacity(8, 2, 8, -1.0, &cap) == MOE_ERR_SHAPE);
  CHECK(moe_capacity(8, 2, 8, NAN, &cap) == MOE_ERR_SHAPE);
  CHECK(moe_capacity(8, 2, 8, INFINITY, &cap) == MOE_ERR_SHAPE);
  CHECK(moe_capacity(2147483647, 16, 1, 1e9, &cap) == MOE_ERR_SHAPE);

  // workspace sizes over a sweep of valid shapes: positive, and growing with T
  size_t prev = 0, bytes = 0, bbytes = 0;
  const int Ts[] = {0, 1, 15, 16, 17, 255, 4096, 65536, 262143};
  for (int T : Ts) {
    moe_shape s = shape(T, 4096, 14336, 8, 2);
    CHECK(moe_workspace_bytes(&s, &bytes) == MOE_OK && bytes > 0 && bytes >= prev);
    CHECK(moe_backward_workspace_bytes(&s, &bbytes) == MOE_OK && bbytes > 0);
    prev = bytes;
  }
  for (int E : {1, 2, 16, 17, 64, 256, 1024})
    for (int k : {1, 2, 8, 16}) {
      if (k > E) continue;
      moe_shape s = shape(1000, 256, 512, E, k);
      s.capacity = (E * 3) % 7 == 0 ? -1 : 37;
      s.d_e_shared = E % 2 ? 0 : 256;
      for (int dt : {MOE_F32, MOE_BF16}) {
        s.dtype = dt;
        CHECK(moe_workspace_bytes(&s, &bytes) == MOE_OK && bytes > 0);
        CHECK(moe_backward_workspace_bytes(&s, &bbytes) == MOE_OK && bbytes > 0);
      }
    }
  {
    moe_shape s = shape(4096, 7168, 2048, 256, 8);
    s.d_e_shared = 2048; s.scoring = MOE_SCORE_SIGMOID; s.n_group = 8; s.topk_group = 4;
    CHECK(moe_workspace_bytes(&s, &bytes) == MOE_OK);
    s.wfmt = MOE_W_MXFP4; s.afmt = MOE_A_MXFP8;
    CHECK(moe_workspace_bytes(&s, &bytes) == MOE_OK);
    CHECK(moe_backward_workspace_bytes(&s, &bbytes) == MOE_ERR_UNSUPPORTED);   // forward only
  }

  // shape validation: one violated rule at a time
  struct Case { moe_shape s; moe_status want; };
  std::vector<Case> cases;
  auto add = [&](void (*edit)(moe_shape&), moe_status want) {
    moe_shape s = shape(64, 256, 512, 8, 2);
    edit(s);
    cases.push_back({s, want});
  };
  add([](moe_shape& s) { s.T = -1; }, MOE_ERR_SHAPE);
  add([](moe_shape& s) { s.d = 0; }, MOE_ERR_SHAPE);
  add([](moe_shape& s) { s.d_e = 0; }, MOE_ERR_SHAPE);
  add([](moe_shape& s) { s.E = 0; }, MOE_ERR_SHAPE);
  add([](moe_shape& s) { s.k = 0; }, MOE_ERR_SHAPE);
  add([](moe_shape& s) { s.k = 9; }, MOE_ERR_SHAPE);
  add([](moe_shape& s) { s.d_e_shared = -128; }, MOE_ERR_SHAPE);
  add([](moe_shape& s) { s.dtype = 7; }, MOE_ERR_UNSUPPORTED);
  add([](moe_shape& s) { s.scoring = 3; }, MOE_ERR_UNSUPPORTED);
  add([](moe_shape& s) { s.n_group = 0; }, MOE_ERR_SHAPE);
  add([](moe_shape& s) { s.n_group = 3; }, MOE_ERR_SHAPE);
  add([](moe_shape& s) { s.n_group = 2; s.topk_group = 3; }, MOE_ERR_SHAPE);
  add([](moe_shape& s) { s.n_group = 4; s.topk_group = 1; s.k = 3; }, MOE_ERR_SHAPE);
  add([](moe_shape& s) { s.wfmt = 9; }, MOE_ERR_UNSUPPORTED);
  add([](moe_shape& s) { s.wfmt = MOE_W_FP8_E4M3; s.dtype = MOE_F32; }, MOE_ERR_UNSUPPORTED);
  add([](moe_shape& s) { s.afmt = 5; }, MOE_ERR_UNSUPPORTED);
  add([](moe_shape& s) { s.afmt = MOE_A_MXFP8; }, MOE_ERR_UNSUPPORTED);
  add([](moe_shape& s) { s.E = 2048; s.k = 2; }, MOE_ERR_UNSUPPORTED);
  add([](moe_shape& s) { s.E = 32; s.k = 17; }, MOE_ERR_UNSUPPORTED);
  add([](moe_shape& s) { s.d = 200; }, MOE_ERR_UNSUPPORTED);
  add([](moe_shape& s) { s.d_e = 100; }, MOE_ERR_UNSUPPORTED);
  add([](moe_shape& s) { s.d_e_shared = 64; }, MOE_ERR_UNSUPPORTED);
  add([](moe_shape& s) { s.T = 300000; s.d = 8192; }, MOE_ERR_UNSUPPORTED);   // x >= 4 GiB
  add([](moe_shape& s) { s.T = 1 << 30; s.k = 4; }, MOE_ERR_UNSUPPORTED);     // T k >= 2^31
  for (const Case& c : cases) {
    size_t b = 0;
    CHECK(moe_workspace_bytes(&c.s, &b) == c.want);
    CHECK(moe_backward_workspace_bytes(&c.s, &b) == c.want);
  }
  CHECK(moe_workspace_bytes(nullptr, &bytes) == MOE_ERR_NULL);
  {
    moe_shape s = shape(64, 256, 512, 8, 2);
    CHECK(moe_workspace_bytes(&s, nullptr) == MOE_ERR_NULL);
    CHECK(moe_backward_workspace_bytes(&s, nullptr) == MOE_ERR_NULL);
  }

  // compute entry points: rejected before any launch (bad shape, NULL pointers, small workspace).
  // The pointers below are host addresses that validation never dereferences.
  static char buf[4096];
  void* p = buf;
  float* fp = (float*)buf;
  int32_t* ip = (int32_t*)buf;
  const moe_shape good = shape(64, 256, 512, 8, 2);
  moe_shape bad = good;
  bad.k = 0;
  size_t ws_need = 0;
  CHECK(moe_workspace_bytes(&good, &ws_need) == MOE_OK && ws_need > 0);
  // moe_route
  CHECK(moe_route(&bad, p, p, nullptr, ip, fp, ip, fp, fp, fp, p, ws_need, nullptr) == MOE_ERR_SHAPE);
  CHECK(moe_route(&good, nullptr, p, nullptr, ip, fp, ip, fp, fp, fp, p, ws_need, nullptr) == MOE_ERR_NULL);
  CHECK(moe_route(&good, p, p, nullptr, ip, fp, ip, fp, fp, fp, nullptr, ws_need, nullptr) == MOE_ERR_NULL);
  CHECK(moe_route(&good, p, p, nullptr, ip, fp, ip, fp, fp, fp, p, ws_need - 1, nullptr) == MOE_ERR_WORKSPACE);
  // moe_permute
  CHECK(moe_permute(&bad, p, ip, ip, ip, ip, ip, p, p, ws_need, nullptr) == MOE_ERR_SHAPE);
  CHECK(moe_permute(&good, p, nullptr, ip, ip, ip, ip, p, p, ws_need, nullptr) == MOE_ERR_NULL);
  CHECK(moe_permute(&good, p, ip, ip, ip, ip, ip, p, p, 0, nullptr) == MOE_ERR_WORKSPACE);
  // moe_expert_ffn
  CHECK(moe_expert_ffn(&bad, p, ip, p, p, p, nullptr, fp, p, ws_need, nullptr) == MOE_ERR_SHAPE);
  CHECK(moe_expert_ffn(&good, p, ip, nullptr, p, p, nullptr, fp, p, ws_need, nullptr) == MOE_ERR_NULL);
  // moe_combine
  CHECK(moe_combine(&bad, fp, ip, fp, nullptr, fp, nullptr) == MOE_ERR_SHAPE);
  CHECK(moe_combine(&good, nullptr, ip, fp, nullptr, fp, nullptr) == MOE_ERR_NULL);
  // moe_forward and its allocation-free variant
  CHECK(moe_forward(&bad, p, p, nullptr, p, p, p, nullptr, nullptr, nullptr, nullptr, nullptr, fp, ip, fp, ip, ip,
                    fp, fp, fp, ip, ip, ip, p, ws_need, nullptr, nullptr) == MOE_ERR_SHAPE);
  CHECK(moe_forward(&good, p, p, nullptr, nullptr, p, p, nullptr, nullptr, nullptr, nullptr, nullptr, fp, ip, fp, ip,
                    ip, fp, fp, fp, ip, ip, ip, p, ws_need, nullptr, nullptr) == MOE_ERR_NULL);
  CHECK(moe_forward(&good, p, p, nullptr, p, p, p, nullptr, nullptr, nullptr, nullptr, nullptr, fp, ip, fp, ip, ip,
                    fp, fp, fp, ip, ip, ip, p, ws_need - 1, nullptr, nullptr) == MOE_ERR_WORKSPACE);
  {
    moe_shape q = good;
    q.wfmt = MOE_W_FP8_E4M3;                          // quantised weights without their scales
    CHECK(moe_forward(&q, p, p, nullptr, p, p, p, nullptr, nullptr, nullptr, nullptr, nullptr, fp, ip, fp, ip, ip,
                      fp, fp, fp, ip, ip, ip, p, ws_need * 2, nullptr, nullptr) == MOE_ERR_NULL);
    moe_shape sh = good;
    sh.d_e_shared = 256;                              // shared expert without its weights
    CHECK(moe_forward(&sh, p, p, nullptr, p, p, p, nullptr, nullptr, nullptr, nullptr, nullptr, fp, ip, fp, ip, ip,
                      fp, fp, fp, ip, ip, ip, p, ws_need * 2, nullptr, nullptr) == MOE_ERR_NULL);
  }
  CHECK(moe_forward_noalloc(&bad, p, p, nullptr, p, p, p, nullptr, nullptr, nullptr, nullptr, nullptr, fp, ip, fp, ip,
                            ip, fp, fp, fp, ip, ip, ip, nullptr, nullptr) == MOE_ERR_SHAPE);
  {
    moe_shape big = shape(65536, 4096, 14336, 8, 2);  // workspace beyond the static scratch
    CHECK(moe_forward_noalloc(&big, p, p, nullptr, p, p, p, nullptr, nullptr, nullptr, nullptr, nullptr, fp, ip, fp,
                              ip, ip, fp, fp, fp, ip, ip, ip, nullptr, nullptr) == MOE_ERR_WORKSPACE);
  }
  // moe_mxfp8_quantize
  CHECK(moe_mxfp8_quantize(-1, 64, p, (uint8_t*)p, (uint8_t*)p, nullptr) == MOE_ERR_SHAPE);
  CHECK(moe_mxfp8_quantize(4, 16, p, (uint8_t*)p, (uint8_t*)p, nullptr) == MOE_ERR_SHAPE);
  CHECK(moe_mxfp8_quantize(4, 48, p, (uint8_t*)p, (uint8_t*)p, nullptr) == MOE_ERR_SHAPE);
  CHECK(moe_mxfp8_quantize(0, 64, nullptr, nullptr, nullptr, nullptr) == MOE_OK);
  CHECK(moe_mxfp8_quantize(4, 64, nullptr, (uint8_t*)p, (uint8_t*)p, nullptr) == MOE_ERR_NULL);
  // moe_backward
  size_t bws = 0;
  CHECK(moe_backward_workspace_bytes(&good, &bws) == MOE_OK && bws > 0);
  CHECK(moe_backward(&bad, p, p, nullptr, p, p, p, nullptr, nullptr, nullptr, ip, fp, ip, ip, ip, ip, fp, 0.f, fp,
                     fp, nullptr, fp, fp, fp, nullptr, nullptr, nullptr, fp, p, bws, nullptr, nullptr) == MOE_ERR_SHAPE);
  CHECK(moe_backward(&good, p, p, nullptr, p, p, p, nullptr, nullptr, nullptr, ip, fp, ip, ip, ip, ip, nullptr, 0.f,
                     fp, fp, nullptr, fp, fp, fp, nullptr, nullptr, nullptr, fp, p, bws, nullptr, nullptr) ==
        MOE_ERR_NULL);
  CHECK(moe_backward(&good, p, p, nullptr, p, p, p, nullptr, nullptr, nullptr, ip, fp, ip, ip, ip, ip, fp, NAN, fp,
                     fp, nullptr, fp, fp, fp, nullptr, nullptr, nullptr, fp, p, bws, nullptr, nullptr) == MOE_ERR_SHAPE);
  CHECK(moe_backward(&good, p, p, nullptr, p, p, p, nullptr, nullptr, nullptr, ip, fp, ip, ip, ip, ip, fp, 0.f, fp,
                     fp, nullptr, fp, fp, fp, nullptr, nullptr, nullptr, fp, p, bws - 1, nullptr, nullptr) ==
        MOE_ERR_WORKSPACE);

  std::printf("abi host checks: %d passed, %d failed\n", g_pass, g_fail);
  return g_fail == 0 ? 0 : 1;
}
