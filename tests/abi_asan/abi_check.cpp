// Drives every entry point of the C ABI (include/arl2.h) on the host, with the
// kernel launchers replaced by stubs (launch_stubs.cpp): each call once with
// valid arguments (it must validate and reach a launcher) and with invalid
// ones (it must return the documented status without reaching one). Built
// with g++ -fsanitize=address,undefined so that any out-of-bounds access,
// overflow or misuse inside the validation code aborts the run. Pointers are
// fake addresses 1 GiB apart: the validation code never dereferences them.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/arl2.h"

extern int g_launches;

static int g_fail = 0;
static void expect(int got, int want, const char* what, int line) {
  if (got != want) {
    fprintf(stderr, "line %d: %s returned %d, expected %d (%s)\n", line, what, got, want,
            arl2_last_error());
    ++g_fail;
  }
}
#define EXPECT(call, want) expect((int)(call), (int)(want), #call, __LINE__)

// Checks that a call validates and launches (want OK) or fails without launching.
#define LAUNCHES(call)                        \
  do {                                        \
    const int before = g_launches;            \
    EXPECT(call, ARL2_OK);                    \
    if (g_launches == before) {               \
      fprintf(stderr, "line %d: %s launched nothing\n", __LINE__, #call); \
      ++g_fail;                               \
    }                                         \
  } while (0)
#define REFUSES(call, want)                   \
  do {                                        \
    const int before = g_launches;            \
    EXPECT(call, want);                       \
    if (g_launches != before) {               \
      fprintf(stderr, "line %d: %s launched after refusing\n", __LINE__, #call); \
      ++g_fail;                               \
    }                                         \
  } while (0)

static void* P(int i) { return (void*)((uintptr_t)(i + 1) << 30); }
static float* F(int i) { return (float*)P(i); }

static void run_shape(const arl2_shape& sh, bool full_kernels) {
  const arl2_shape* s = &sh;
  void* ws = P(40);
  const size_t big = (size_t)1 << 29;
  void* q = P(0); void* k = P(1); void* v = P(2);
  void* pq = P(3); void* pk = P(4); void* pv = P(5);
  float* beta = F(6); float* alpha = F(7); float* S0 = F(8); float* S1 = F(9);
  void* o = P(10); void* oi = P(11); void* oe = P(12);
  void* M0 = P(13); void* M1 = P(14);

  LAUNCHES(arl2_feature_map(s, q, pq, o, 1, nullptr));
  REFUSES(arl2_feature_map(s, q, pq, q, 0, nullptr), ARL2_E_ALIAS);
  REFUSES(arl2_feature_map(s, q, nullptr, o, 0, nullptr), ARL2_E_NULL);
  REFUSES(arl2_feature_map(s, (char*)q + 8, pq, o, 0, nullptr), ARL2_E_LAYOUT);
  LAUNCHES(arl2_intra_attn(s, q, k, v, o, nullptr));
  REFUSES(arl2_intra_attn(s, q, k, v, v, nullptr), ARL2_E_ALIAS);
  if (full_kernels) {
    LAUNCHES(arl2_intra_attn_lse(s, q, k, v, o, F(15), nullptr));
  } else {
    REFUSES(arl2_intra_attn_lse(s, q, k, v, o, F(15), nullptr), ARL2_E_SHAPE);
  }
  LAUNCHES(arl2_inter_read(s, q, S0, oi, o, nullptr));
  LAUNCHES(arl2_inter_read(s, q, S0, o, o, nullptr));
  REFUSES(arl2_inter_read(s, q, S0, oi, S0, nullptr), ARL2_E_ALIAS);

  const size_t sc = arl2_workspace_bytes(s, ARL2_OP_STATE_COMMIT);
  LAUNCHES(arl2_state_commit(s, k, v, beta, alpha, S0, S1, ws, sc, nullptr));
  REFUSES(arl2_state_commit(s, k, v, beta, alpha, S0, S0, ws, sc, nullptr), ARL2_E_ALIAS);
  REFUSES(arl2_state_commit(s, k, v, beta, alpha, S0, (float*)ws, ws, sc, nullptr), ARL2_E_ALIAS);
  REFUSES(arl2_state_commit(s, k, v, beta, alpha, S0, (float*)k, ws, sc, nullptr), ARL2_E_ALIAS);
  if (sc > 0)
    REFUSES(arl2_state_commit(s, k, v, beta, alpha, S0, S1, ws, sc - 1, nullptr),
            ARL2_E_WORKSPACE);

  const size_t rd = arl2_workspace_bytes(s, ARL2_OP_READ);
  LAUNCHES(arl2_read(s, q, k, v, pq, S0, o, oi, oe, ws, rd, nullptr));
  LAUNCHES(arl2_read(s, q, k, v, pq, S0, o, nullptr, nullptr, ws, rd, nullptr));
  REFUSES(arl2_read(s, q, k, v, pq, S0, o, o, nullptr, ws, rd, nullptr), ARL2_E_ALIAS);
  REFUSES(arl2_read(s, q, k, v, pq, S0, o, oi, oe, ws, rd - 1, nullptr), ARL2_E_WORKSPACE);

  LAUNCHES(arl2_read_noalloc(s, q, k, v, pq, S0, o, oi, oe, nullptr));
  REFUSES(arl2_read_noalloc(s, q, k, v, pq, S0, o, o, nullptr, nullptr), ARL2_E_ALIAS);
  REFUSES(arl2_read_noalloc(s, q, k, v, pq, S0, q, nullptr, nullptr, nullptr), ARL2_E_ALIAS);
  REFUSES(arl2_read_noalloc(s, q, k, v, nullptr, S0, o, nullptr, nullptr, nullptr), ARL2_E_NULL);

  EXPECT(arl2_prepared_bytes(s) > 0, 1);
  LAUNCHES(arl2_read_prepare(s, pq, S0, M0, nullptr));
  REFUSES(arl2_read_prepare(s, pq, S0, S0, nullptr), ARL2_E_ALIAS);
  const size_t rp = arl2_workspace_bytes(s, ARL2_OP_READ_PREPARED);
  LAUNCHES(arl2_read_prepared(s, q, k, v, M0, o, oi, oe, ws, rp, nullptr));
  REFUSES(arl2_read_prepared(s, q, k, v, M0, M0, oi, oe, ws, rp, nullptr), ARL2_E_ALIAS);

  const size_t cm = arl2_workspace_bytes(s, ARL2_OP_COMMIT);
  LAUNCHES(arl2_commit(s, k, v, pk, pv, beta, alpha, S0, S1, ws, cm, nullptr));
  REFUSES(arl2_commit(s, k, v, pk, pv, beta, alpha, S0, (float*)alpha, ws, cm, nullptr),
          ARL2_E_ALIAS);
  REFUSES(arl2_commit(s, k, v, pk, pv, beta, nullptr, S0, S1, ws, cm, nullptr), ARL2_E_NULL);

  const size_t cp = arl2_workspace_bytes(s, ARL2_OP_CLEAN_PASS);
  LAUNCHES(arl2_clean_pass(s, q, k, v, pq, pk, pv, beta, alpha, S0, S1, o, oi, oe, ws, cp,
                           nullptr));
  REFUSES(arl2_clean_pass(s, q, k, v, pq, pk, pv, beta, alpha, S0, (float*)pk, o, oi, oe, ws, cp,
                          nullptr),
          ARL2_E_ALIAS);
  const size_t cpp = arl2_workspace_bytes(s, ARL2_OP_CLEAN_PASS_PREPARED);
  LAUNCHES(arl2_clean_pass_prepared(s, q, k, v, M0, pq, pk, pv, beta, alpha, S0, S1, M1, o, oi,
                                    oe, ws, cpp, nullptr));
  REFUSES(arl2_clean_pass_prepared(s, q, k, v, M0, pq, pk, pv, beta, alpha, S0, S1, M0, o, oi,
                                   oe, ws, cpp, nullptr),
          ARL2_E_ALIAS);
  REFUSES(arl2_clean_pass_prepared(s, q, k, v, M0, nullptr, pk, pv, beta, alpha, S0, S1, M1, o,
                                   oi, oe, ws, cpp, nullptr),
          ARL2_E_NULL);

  const size_t tl = arl2_workspace_bytes(s, ARL2_OP_TOKEN_LEVEL);
  const size_t ab = arl2_workspace_bytes(s, ARL2_OP_INTRA_ATTN_BACKWARD);
  const size_t rb = arl2_workspace_bytes(s, ARL2_OP_READ_BACKWARD);
  const size_t cb = arl2_workspace_bytes(s, ARL2_OP_COMMIT_BACKWARD);
  float* dphi = F(20); float* dphi2 = F(21); float* dS = F(22);
  float* db = F(23); float* da = F(24);
  void* dq = P(25); void* dk = P(26); void* dv = P(27);
  if (full_kernels) {
    LAUNCHES(arl2_token_read(s, q, k, v, pq, pk, pv, beta, S0, o, oi, oe, ws, tl, nullptr));
    LAUNCHES(arl2_token_clean_pass(s, q, k, v, pq, pk, pv, beta, alpha, S0, S1, o, oi, oe, ws,
                                   tl, nullptr));
    LAUNCHES(arl2_intra_attn_backward(s, q, k, v, oi, nullptr, oe, dq, dk, dv, 0, ws, ab,
                                      nullptr));
    LAUNCHES(arl2_read_backward(s, q, k, v, pq, S0, oi, F(15), oe, dq, dk, dv, dphi, dS, 1, ws,
                                rb, nullptr));
    LAUNCHES(arl2_commit_backward(s, k, v, pk, pv, beta, alpha, S0, S1, dk, dv, dphi, dphi2, db,
                                  da, dS, 0, ws, cb, nullptr));
    REFUSES(arl2_commit_backward(s, k, v, pk, pv, beta, alpha, S0, S1, dk, dv, dphi, dphi, db,
                                 da, dS, 0, ws, cb, nullptr),
            ARL2_E_ALIAS);
  } else {
    REFUSES(arl2_token_read(s, q, k, v, pq, pk, pv, beta, S0, o, oi, oe, ws, big, nullptr),
            ARL2_E_SHAPE);
    REFUSES(arl2_intra_attn_backward(s, q, k, v, oi, nullptr, oe, dq, dk, dv, 0, ws, big,
                                     nullptr),
            ARL2_E_SHAPE);
    REFUSES(arl2_read_backward(s, q, k, v, pq, S0, oi, nullptr, oe, dq, dk, dv, dphi, dS, 1, ws,
                               big, nullptr),
            ARL2_E_SHAPE);
    REFUSES(arl2_commit_backward(s, k, v, pk, pv, beta, alpha, S0, S1, dk, dv, dphi, dphi2, db,
                                 da, dS, 0, ws, big, nullptr),
            ARL2_E_SHAPE);
  }
  LAUNCHES(arl2_state_scan(s, 3, k, v, pk, pv, beta, alpha, S0, F(30), ws, cm, nullptr));
  REFUSES(arl2_state_scan(s, 0, k, v, pk, pv, beta, alpha, S0, F(30), ws, cm, nullptr),
          ARL2_E_SHAPE);
  LAUNCHES(arl2_fullkv_attn(s, q, k, v, sh.T, 4 * (int64_t)sh.T, o, nullptr));
  REFUSES(arl2_fullkv_attn(s, q, k, v, 5 * (int64_t)sh.T, 4 * (int64_t)sh.T, o, nullptr),
          ARL2_E_SHAPE);
}

int main() {
  const arl2_shape shapes[] = {{1, 2, 1560, 128, ARL2_BF16, 0.f},
                               {2, 3, 300, 64, ARL2_BF16, 0.f},
                               {1, 2, 77, 16, ARL2_BF16, 0.f},
                               {1, 1, 64, 16, ARL2_F32, 0.f},
                               {2, 2, 130, 128, ARL2_F32, 0.25f}};
  for (const arl2_shape& sh : shapes)
    run_shape(sh, sh.act_dtype == ARL2_F32 || sh.D == 128);

  // shape validation
  const arl2_shape bad[] = {{0, 1, 1, 128, ARL2_BF16, 0.f},  {1, 1, 1, 48, ARL2_BF16, 0.f},
                            {1, 1, 1, 128, 7, 0.f},          {1, 1, 1, 128, ARL2_F32, -1.f},
                            {4096, 64, 4096, 128, ARL2_F32, 0.f}};
  const int bad_status[] = {ARL2_E_SHAPE, ARL2_E_SHAPE, ARL2_E_DTYPE, ARL2_E_SHAPE, ARL2_E_SHAPE};
  for (int i = 0; i < 5; ++i)
    REFUSES(arl2_intra_attn(&bad[i], P(0), P(1), P(2), P(3), nullptr), bad_status[i]);
  REFUSES(arl2_intra_attn(nullptr, P(0), P(1), P(2), P(3), nullptr), ARL2_E_NULL);
  // more than the fixed scratch of the allocation-free read holds
  const arl2_shape wide = {1, 300, 64, 128, ARL2_BF16, 0.f};
  REFUSES(arl2_read_noalloc(&wide, P(0), P(1), P(2), P(3), F(4), P(5), nullptr, nullptr,
                            nullptr),
          ARL2_E_WORKSPACE);
  if (strlen(arl2_last_error()) == 0) {
    fprintf(stderr, "no detail text after a failed call\n");
    ++g_fail;
  }
  // support calls
  for (int st = 0; st <= 8; ++st)
    if (!arl2_status_string((arl2_status)st)) ++g_fail;
  EXPECT(arl2_workspace_bytes(&bad[0], ARL2_OP_READ), 0);
  EXPECT(arl2_workspace_bytes(&shapes[0], 99), 0);
  EXPECT(arl2_abi_version(), ARL2_ABI_VERSION);
  EXPECT(arl2_prepared_bytes(nullptr), 0);

  if (g_fail) {
    fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  printf("all checks passed (%d launches reached)\n", g_launches);
  return 0;
}
