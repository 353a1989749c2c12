/* Host-side validation of every svlm_* entry point, for a build of the
 * library whose host code carries AddressSanitizer and UndefinedBehaviorSanitizer.
 * Every call below has an argument the library must refuse before it touches
 * a device, so nothing is launched; the workspace queries are host-only.
 * Exit status: the number of calls whose status was not the expected one. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "svlm.h"

static int fails = 0;

static void expect(int got, int want, const char* what) {
  const char* msg = svlm_last_error();
  if (got != want) {
    fprintf(stderr, "%s: status %d, expected %d (%s)\n", what, got, want, msg);
    ++fails;
  }
  if (strlen(msg) >= 512) {
    fprintf(stderr, "%s: error text too long\n", what);
    ++fails;
  }
}

int main(void) {
  void* f = (void*)4096;          /* never dereferenced: validation fails first */
  float* ff = (float*)4096;
  int32_t* fi = (int32_t*)4096;
  char big[600];
  memset(big, 'x', sizeof big);
  big[sizeof big - 1] = 0;

  if (svlm_abi_version() != SVLM_ABI_VERSION) ++fails;
  for (int st = -2; st < 8; ++st)
    if (!svlm_status_string(st)) ++fails;

  /* workspace queries, valid and invalid sizes */
  (void)svlm_score_workspace(128, 64, 8, 25088, 25088);
  (void)svlm_score_workspace(0, 64, 8, 25088, 25088);
  (void)svlm_select_workspace(112, 141120, 1024, 1.0);
  (void)svlm_select_workspace(-1, 141120, 1024, 1.0);
  (void)svlm_decode_attn_workspace(1, 6, 64, 8, 128, 25222, 0);
  (void)svlm_decode_attn_workspace(1, 6, 64, 8, 128, 25222, 100000);
  (void)svlm_decode_attn_indexed_workspace(1, 1, 28, 4, 128, 1089, 0);
  (void)svlm_decode_attn_workspace(1 << 20, 1 << 10, 1 << 12, 1 << 6, 128, 1 << 30, 0);
  (void)svlm_uvprune_workspace(128, 8192);
  (void)svlm_verify_workspace(1, 5, 152064);
  (void)svlm_verify_workspace(1 << 20, 1 << 10, 1 << 20);
  {
    /* sizes a call refuses: the query answers 0 instead of a wrapped size */
    const int M = INT32_MAX;
    if (svlm_score_workspace(M, M, 1, 0, M) != 0) ++fails;
    if (svlm_score_workspace(16, M, M, M, M) != 0) ++fails;
    (void)svlm_score_workspace(128, M, M, M - 128, 1 << 18);
    (void)svlm_score_layers_workspace(M, 128, M, M, M - 128, 1 << 18);
    (void)svlm_score_layers_workspace(M, 128, 64, 8, M - 128, 1 << 18);
    if (svlm_select_workspace(M, M, M, 0.5) != 0) ++fails;
    if (svlm_select_workspace(M, M, 1, 1.0) != 0) ++fails;
    if (svlm_select_workspace(M, 1 << 18, 1024, 1.0) != 0) ++fails;
    if (svlm_decode_attn_workspace(M, M, M, 1, 128, M, 0) != 0) ++fails;
    if (svlm_decode_attn_workspace(M, M, M, M, 128, M, M) != 0) ++fails;
    if (svlm_decode_attn_workspace(1, 1, M, 1, 64, M, 0) != 0) ++fails;
    if (svlm_decode_attn_workspace(M, 1, 8, 1, 128, M, M) != 0) ++fails;
    if (svlm_decode_attn_indexed_workspace(M, M, M, 1, 128, M, 0) != 0) ++fails;
    if (svlm_verify_workspace(M, M, M) != 0) ++fails;
    if (svlm_verify_workspace(1 << 16, 4, 1000) != 0) ++fails;
    (void)svlm_uvprune_workspace(M, M);
    if (fails) fprintf(stderr, "a workspace query answered a refused size\n");
  }

  /* score */
  expect(svlm_score(0, 0, 0, 0, 0, 0, SVLM_BF16, 16, 212, 196, 0, 196, 4, 2, 64, 0.125f, SVLM_AGG_ALL, 1, 0, 0, 0,
                    0, 0), SVLM_E_INVALID, "score null");
  expect(svlm_score(f, 256, 64, f, 212 * 64, 64, 7, 16, 212, 196, 0, 196, 4, 2, 64, 0.125f, 2, 1, 0, ff, f, 1 << 20,
                    0), SVLM_E_UNSUPPORTED, "score dtype");
  expect(svlm_score(f, 256, 64, f, 212 * 64, 64, SVLM_BF16, 200, 212, 196, 0, 196, 4, 2, 64, 0.125f, 2, 1, 0, ff, f,
                    1 << 20, 0), SVLM_E_UNSUPPORTED, "score T");
  expect(svlm_score(f, 256, 64, f, 212 * 64, 64, SVLM_F32, 16, 212, 196, 0, 196, 4, 2, 64, -1.f, 2, 1, 0, ff, f,
                    1 << 20, 0), SVLM_E_INVALID, "score scale");
  expect(svlm_score(f, 256, 64, f, 212 * 64, 64, SVLM_F32, 16, 212, 196, 0, 196, 4, 2, 64, 0.125f, 2, 1, 0, ff, f,
                    16, 0), SVLM_E_WORKSPACE, "score workspace");

  expect(svlm_score_layers(f, 256, 64, 1 << 16, f, 212 * 64, 64, 212 * 128, 0, SVLM_BF16, 16, 212, 196, 0, 196, 4,
                           2, 64, 0.125f, 2, 1, 1, 0, ff, f, 1 << 20, 0), SVLM_E_INVALID, "score layers count");
  expect(svlm_score_layers(f, 256, 64, 1 << 16, f, 212 * 64, 64, 212 * 128, 3, SVLM_BF16, 16, 212, 196, 0, 196, 4,
                           2, 64, 0.125f, 2, 1, 1, 0, ff, f, 16, 0), SVLM_E_WORKSPACE, "score layers workspace");
  if (svlm_score_layers_workspace(-1, 16, 4, 2, 196, 196) != 0 ||
      svlm_score_layers_workspace(1, 16, 4, 2, 196, 196) != svlm_score_workspace(16, 4, 2, 196, 196)) {
    fprintf(stderr, "score layers workspace query\n");
    ++fails;
  }

  /* select */
  expect(svlm_select((const float*)f, 20, 1, 2, 2, 5, 0.5, 21, fi, fi, 0, 0, 0, 0), SVLM_E_INVALID, "select budget");
  expect(svlm_select((const float*)f, 141120, 2, 720, 14, 14, 1.0, 1024, fi, fi, 0, 0, 0, 0), SVLM_E_WORKSPACE,
         "select workspace");

  /* gather */
  expect(svlm_gather_kv(f, f, 0, 128, 10, fi, 0, 3, 8, 3, f, f, 0, 128, 1, 128, SVLM_BF16, 0), SVLM_E_INVALID,
         "gather tail");
  expect(svlm_gather_kv(f, f, 0, 66, 10, fi, 0, 3, 0, 3, f, f, 0, 64, 1, 64, SVLM_F32, 0), SVLM_E_INVALID,
         "gather stride");

  /* decode attention, all three entry points */
  expect(svlm_decode_attn(0, 0, 0, 0, 0, 0, 128, 0, 10, SVLM_BF16, 1, 1, 8, 2, 128, 0.1f, 0, 0, 0, 0, 0, 0, 0),
         SVLM_E_INVALID, "attn null");
  expect(svlm_decode_attn(f, 1024, f, f, 0, 0, 100, fi, 10, SVLM_BF16, 1, 1, 8, 2, 128, 0.1f, 0, ff, ff, 0, 0, 0, 0),
         SVLM_E_INVALID, "attn stride");
  expect(svlm_decode_attn(f, 1 << 20, f, f, 0, 128 << 20, 128, fi, 1 << 23, SVLM_BF16, 1, 1, 8, 2, 128, 0.1f, 0, ff,
                          ff, 1, 0, 0, 0), SVLM_E_UNSUPPORTED, "attn split range");
  expect(svlm_decode_attn(f, 1024, f, f, 0, 128000, 128, fi, 1000, SVLM_BF16, 1, 1, 8, 2, 128, 0.1f, 0, ff, ff, 0, 0,
                          0, 0), SVLM_E_WORKSPACE, "attn workspace");
  expect(svlm_decode_attn_indexed(f, 1024, f, f, 0, 0, 128, 100, fi, 0, 0, fi, 1, -1, 10, SVLM_BF16, 1, 1, 8, 2,
                                  128, 0.1f, 0, ff, ff, 0, 0, 0, 0), SVLM_E_INVALID, "indexed length stride");
  expect(svlm_decode_attn_indexed(f, 1024, f, f, 0, 0, 128, 100, 0, 0, 0, fi, 1, 0, 10, SVLM_BF16, 1, 1, 8, 2, 128,
                                  0.1f, 0, ff, ff, 0, 0, 0, 0), SVLM_E_INVALID, "indexed list");
  expect(svlm_decode_attn_noalloc(f, 64 * 64 * 128, f, f, 0, 128 << 20, 128, fi, 1 << 20, SVLM_BF16, 1, 64, 64, 8,
                                  128, 0.1f, 1, ff, ff, 256, 0), SVLM_E_UNSUPPORTED, "noalloc size");

  /* UV-Prune, acceptance, stream read */
  expect(svlm_uvprune_score(f, f, 256, 10, f, f, 256, 4, 250, SVLM_BF16, 1.f, 0.f, ff, f, 1 << 20, 0),
         SVLM_E_UNSUPPORTED, "uvprune d");
  expect(svlm_verify(7, 1, 1, 10, fi, ff, ff, ff, fi, fi, f, 1 << 20, 0), SVLM_E_INVALID, "verify mode");
  expect(svlm_verify(0, 1, 2, 10, fi, ff, 0, 0, fi, fi, 0, 0, 0), SVLM_E_WORKSPACE, "verify workspace");
  expect(svlm_stream_read(f, -1, 1, ff, 0), SVLM_E_INVALID, "stream bytes");
  expect(svlm_stream_read((const void*)4100, 4096, 1, ff, 0), SVLM_E_INVALID, "stream alignment");

  /* launches past the dispatch limits are refused on the host, not wrapped */
  expect(svlm_decode_attn(f, 1024, f, f, 1024, 0, 128, fi, 1000, SVLM_BF16, INT32_MAX, 1, 8, 2, 128, 0.1f, 0, ff,
                          ff, 0, f, (size_t)1 << 40, 0), SVLM_E_UNSUPPORTED, "attn grid");
  expect(svlm_decode_attn(f, 1024, f, f, 1024, 0, 128, fi, 1000, SVLM_F32, INT32_MAX, 1, 8, 2, 128, 0.1f, 0, ff,
                          ff, 0, 0, 0, 0), SVLM_E_UNSUPPORTED, "attn f32 grid");
  expect(svlm_decode_attn(f, 0, f, f, 0, 0, 128, fi, 1000, SVLM_BF16, 1, INT32_MAX, INT32_MAX, 1, 128, 0.1f, 0, ff,
                          ff, 0, 0, 0, 0), SVLM_E_UNSUPPORTED, "attn query range");
  expect(svlm_score(f, 64, 0, f, 0, 64, SVLM_F32, 16, 212, 196, 0, 196, 1 << 22, 1 << 22, 64, 0.125f, 0, 1, 0, ff,
                    f, (size_t)1 << 40, 0), SVLM_E_UNSUPPORTED, "score f32 grid");
  expect(svlm_score(f, 64, 0, f, 0, 64, SVLM_BF16, 16, 212, 196, 0, 196, 1 << 26, 1 << 26, 64, 0.125f, 2, 1, 0, ff,
                    f, (size_t)1 << 40, 0), SVLM_E_UNSUPPORTED, "score grid");
  expect(svlm_select((const float*)f, 196, 1 << 22, 1, 14, 14, 0.5, 20, fi, fi, 0, 0, 0, 0), SVLM_E_UNSUPPORTED,
         "select grid");
  expect(svlm_gather_kv(f, f, 0, 128, INT32_MAX, fi, 0, INT32_MAX, 0, 1, f, f, 0, 128, 1, 128, SVLM_BF16, 0),
         SVLM_E_UNSUPPORTED, "gather rows");
  expect(svlm_gather_kv(f, f, 0, 128, 1000, fi, 0, 1000, 0, 0, f, f, 0, 128, 1 << 16, 128, SVLM_BF16, 0),
         SVLM_E_UNSUPPORTED, "gather heads");
  expect(svlm_uvprune_score(f, f, 64, 10, f, f, 64, INT32_MAX, 64, SVLM_BF16, 1.f, 0.f, ff, f, (size_t)1 << 40, 0),
         SVLM_E_UNSUPPORTED, "uvprune grid");
  expect(svlm_verify(0, 1 << 16, 4, 1000, fi, ff, 0, 0, fi, fi, f, (size_t)1 << 40, 0), SVLM_E_UNSUPPORTED,
         "verify batch");
  expect(svlm_verify(1, 1, 1 << 16, 1000, fi, ff, ff, ff, fi, fi, f, (size_t)1 << 40, 0), SVLM_E_UNSUPPORTED,
         "verify gamma");
  expect(svlm_stream_read(f, (int64_t)1 << 40, INT32_MAX, ff, 0), SVLM_E_UNSUPPORTED, "stream grid");

  /* debug flags: only a library built with SVLM_DEBUG keeps them */
  {
    unsigned fl = 7;
    expect(svlm_debug_flags(&fl), SVLM_E_UNSUPPORTED, "debug flags");
    if (fl != 0) ++fails;
    expect(svlm_debug_flags(0), SVLM_E_INVALID, "debug flags null");
  }

  (void)big;
  if (fails) fprintf(stderr, "%d unexpected statuses\n", fails);
  return fails;
}
