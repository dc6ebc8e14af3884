/* Host-side paths of the C ABI, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer on the host code (tests/test_abi_sanitize.py).
 *
 * Every call here either fails argument validation or has T = 0, so the
 * library returns before any HIP call and no GPU is needed.  The calls
 * cover: status strings, packed-weight and workspace sizes over the layer
 * configurations and token counts up to the 32-bit row-offset limit (the
 * size arithmetic), each rejected configuration field, null, misaligned and
 * too-small arguments of every entry point, T = 0 and the token limit.
 * Prints "ok <checks>" and exits 0 when every status is the expected one;
 * any sanitizer report aborts the process. */
#include <stdio.h>
#include <stdint.h>
#include <string.h>

#include "k2moe.h"

static int g_checks = 0, g_fail = 0;

static void expect(int cond, const char* what) {
  ++g_checks;
  if (!cond) {
    ++g_fail;
    fprintf(stderr, "FAILED: %s (last error: %s)\n", what, moe_last_error());
  }
}

static moe_config k2(void) {
  moe_config c;
  memset(&c, 0, sizeof c);
  c.d_model = 7168;
  c.n_experts = 384;
  c.n_shared = 1;
  c.top_k = 8;
  c.d_ff = 2048;
  c.n_group = 1;
  c.topk_group = 1;
  c.norm_topk_prob = 1;
  c.fmt = MOE_FMT_BF16_FP8B128;
  c.dense = 0;
  c.routed_scaling = 2.827f;
  c.rms_eps = 1e-6f;
  return c;
}

static moe_config dense(void) {
  moe_config c = k2();
  c.n_experts = 1;
  c.n_shared = 0;
  c.top_k = 1;
  c.d_ff = 18432;
  c.dense = 1;
  c.routed_scaling = 1.0f;
  return c;
}

static moe_config tiny(void) {
  moe_config c = k2();
  c.d_model = 256;
  c.n_experts = 16;
  c.top_k = 4;
  c.d_ff = 128;
  c.fmt = MOE_FMT_F32;
  return c;
}

/* aligned, non-null stand-ins: never dereferenced (validation fails first) */
#define FAKE ((void*)(uintptr_t)0x10000)
#define FAKE_MISALIGNED ((void*)(uintptr_t)0x10002)

int main(void) {
  const moe_config cfgs[3] = {k2(), dense(), tiny()};
  /* up to the 32-bit row-offset limit of the K2 shape (T <= 66,576) */
  const int64_t tokens[] = {0, 1, 5, 64, 257, 8192, 16384, 65536};

  for (int s = 0; s <= MOE_ERR_HIP; ++s)
    expect(moe_status_str((moe_status)s) != NULL, "status");
  expect(strcmp(moe_status_str(MOE_OK), "MOE_OK") == 0, "MOE_OK string");

  /* sizes: packed weights positive; workspace non-decreasing in T */
  for (int c = 0; c < 3; ++c) {
    expect(moe_packed_weights_bytes(&cfgs[c]) > 0, "packed bytes");
    for (int e = MOE_WS_ROUTER; e <= MOE_WS_FORWARD; ++e) {
      size_t prev = 0;
      for (size_t i = 0; i < sizeof tokens / sizeof tokens[0]; ++i) {
        size_t n = 0;
        expect(moe_workspace_bytes(&cfgs[c], tokens[i], e, &n) == MOE_OK, "workspace ok");
        expect(n >= prev, "workspace monotone");
        prev = n;
      }
    }
  }
  {
    size_t n = 0;
    moe_config c = k2();
    expect(moe_workspace_bytes(&c, -1, MOE_WS_FORWARD, &n) == MOE_ERR_INVALID_ARG, "T < 0");
    expect(moe_workspace_bytes(&c, 66576, MOE_WS_FORWARD, &n) == MOE_OK, "largest K2 T");
    expect(moe_workspace_bytes(&c, 66577, MOE_WS_FORWARD, &n) == MOE_ERR_UNSUPPORTED,
           "K2 T past the row-offset limit");
    moe_config t = tiny();
    expect(moe_workspace_bytes(&t, ((int64_t)1 << 24) + 1, MOE_WS_FORWARD, &n) ==
               MOE_ERR_UNSUPPORTED,
           "T > 2^24");
    expect(moe_workspace_bytes(&c, 8, 9, &n) == MOE_ERR_INVALID_ARG, "bad entry");
    expect(moe_workspace_bytes(&c, 8, MOE_WS_FORWARD, NULL) == MOE_ERR_INVALID_ARG,
           "null size");
    expect(moe_workspace_bytes(NULL, 8, MOE_WS_FORWARD, &n) == MOE_ERR_INVALID_ARG,
           "null config");
  }

  /* each rejected configuration field */
  {
    struct { int field; int32_t value; moe_status st; } bad[] = {
        {0, 2, MOE_ERR_UNSUPPORTED},          /* n_group */
        {1, 4, MOE_ERR_UNSUPPORTED},          /* topk_group */
        {2, 7, MOE_ERR_UNSUPPORTED},          /* fmt */
        {3, 0, MOE_ERR_INVALID_ARG},          /* top_k */
        {3, 385, MOE_ERR_INVALID_ARG},        /* top_k > E */
        {4, 2, MOE_ERR_UNSUPPORTED},          /* n_shared */
        {5, 7168 + 128, MOE_ERR_UNSUPPORTED}, /* d_model % 256 */
        {6, 2048 + 64, MOE_ERR_UNSUPPORTED},  /* d_ff % 128 */
        {7, 396, MOE_ERR_UNSUPPORTED},        /* n_experts % 16 */
        {8, 1, MOE_ERR_INVALID_ARG},          /* dense with 384 experts */
    };
    for (size_t i = 0; i < sizeof bad / sizeof bad[0]; ++i) {
      moe_config c = k2();
      int32_t* f[] = {&c.n_group, &c.topk_group, &c.fmt, &c.top_k, &c.n_shared,
                      &c.d_model, &c.d_ff, &c.n_experts, &c.dense};
      *f[bad[i].field] = bad[i].value;
      size_t n = 0;
      expect(moe_workspace_bytes(&c, 8, MOE_WS_FORWARD, &n) == bad[i].st, "config field");
      expect(moe_last_error()[0] != '\0', "error text");
      expect(moe_packed_weights_bytes(&c) == 0, "packed bytes of a bad config");
    }
  }

  /* moe_forward: nulls, misalignment, small workspace, T < 0, T = 0 */
  {
    moe_config c = k2();
    size_t need = 0;
    expect(moe_workspace_bytes(&c, 64, MOE_WS_FORWARD, &need) == MOE_OK, "ws 64");
    void* p[7];
    for (int k = 0; k < 7; ++k) {
      for (int j = 0; j < 7; ++j) p[j] = FAKE;
      p[k] = NULL;
      expect(moe_forward(&c, 4, p[0], p[1], p[2], (const float*)p[3], p[4], p[5], p[6],
                         (size_t)1 << 40, NULL) == MOE_ERR_INVALID_ARG,
             "forward null");
    }
    expect(moe_forward(&c, 4, FAKE_MISALIGNED, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                       (size_t)1 << 40, NULL) == MOE_ERR_INVALID_ARG,
           "forward misaligned");
    expect(moe_forward(&c, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, NULL) ==
               MOE_ERR_WORKSPACE,
           "forward workspace");
    expect(moe_forward(&c, -1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, NULL) ==
               MOE_ERR_INVALID_ARG,
           "forward T < 0");
    expect(moe_forward(&c, 0, NULL, FAKE, FAKE, FAKE, FAKE, NULL, NULL, 0, NULL) == MOE_OK,
           "forward T = 0");
    moe_config d = dense();
    expect(moe_forward(&d, 0, NULL, FAKE, NULL, NULL, FAKE, NULL, NULL, 0, NULL) == MOE_OK,
           "dense forward T = 0 without router");
    expect(moe_forward(&c, 4, FAKE, FAKE, NULL, FAKE, FAKE, FAKE, FAKE, (size_t)1 << 40,
                       NULL) == MOE_ERR_INVALID_ARG,
           "routed forward without router");
  }

  /* the unfused entry points */
  {
    moe_config c = k2(), t = tiny();
    expect(moe_router(&t, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, FAKE, FAKE,
                      (size_t)1 << 30, NULL) == MOE_ERR_INVALID_ARG,
           "f32 router with scales");
    expect(moe_router(&c, 4, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, NULL, FAKE, FAKE, FAKE,
                      (size_t)1 << 30, NULL) == MOE_ERR_INVALID_ARG,
           "router null ids");
    expect(moe_permute(&c, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 0, NULL) == MOE_OK,
           "permute T = 0");
    expect(moe_permute(&c, 4, NULL, FAKE, FAKE, FAKE, FAKE, (size_t)1 << 30, NULL) ==
               MOE_ERR_INVALID_ARG,
           "permute null ids");
    expect(moe_grouped_swiglu(&c, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, NULL,
                              FAKE, (size_t)1 << 40, NULL) == MOE_ERR_INVALID_ARG,
           "swiglu without shared_out");
    expect(moe_grouped_swiglu(&c, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL,
                              FAKE, (size_t)1 << 40, NULL) == MOE_ERR_INVALID_ARG,
           "swiglu act_q without act_s");
    expect(moe_combine(&c, 4, NULL, FAKE, FAKE, FAKE, FAKE, FAKE, 0, NULL) ==
               MOE_ERR_INVALID_ARG,
           "combine null rows");
    moe_expert_w w[3];
    memset(w, 0, sizeof w);
    expect(moe_pack_weights(&t, w, 3, FAKE, NULL) == MOE_ERR_INVALID_ARG,
           "pack wrong expert count");
  }

  if (g_fail) {
    fprintf(stderr, "%d of %d checks failed\n", g_fail, g_checks);
    return 1;
  }
  printf("ok %d\n", g_checks);
  return 0;
}
