// Host-only checks of the plan chooser (no HIP): built with the system C++
// compiler against plan.cpp. Exits non-zero on the first failure.
#include <stdio.h>
#include <stdlib.h>

#include <initializer_list>

#include "../plan.hpp"

#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "FAILED %s at %s:%d\n", #c, __FILE__, __LINE__); \
      exit(1);                                                     \
    }                                                              \
  } while (0)

static int cdiv(int a, int b) { return (a + b - 1) / b; }

int main() {
  vattn_plan_info in;
  // one long sequence, 8 KV heads, 256 CUs: the cap of 32 binds
  CHECK(vattn::plan_compute(1, 1, 32768, 64, 8, 128, 0, nullptr, 256, &in) == VATTN_OK);
  CHECK(in.is_decode && in.nsplit == 32 && in.grid == 256 && in.chunk_keys == 1024 && !in.direct);
  // 8 units x 32 splits = 256 workgroups fit the device at once: in-kernel merge
  CHECK(in.decode_path == VATTN_DECODE_MFMA && in.fused_combine == 1 && in.combine_grid == 0);
  CHECK(in.threads == 256);
  {
    vattn_plan_opts fu = {};
    fu.fuse_combine = 2;  // forced combine kernel
    CHECK(vattn::plan_compute(1, 1, 32768, 64, 8, 128, 0, &fu, 256, &in) == VATTN_OK);
    CHECK(in.fused_combine == 0 && in.combine_grid == 32 && in.nsplit == 32);
    fu.fuse_combine = 1;  // forced in-kernel merge
    CHECK(vattn::plan_compute(64, 1, 8192, 32, 8, 128, 0, &fu, 256, &in) == VATTN_OK);
    CHECK(in.fused_combine == 1 && in.combine_grid == 0 && in.nsplit == 8);
  }
  // continuous batching: 512 units, 16 workgroups per CU -> 8 splits; G = 4 on the MFMA path
  CHECK(vattn::plan_compute(64, 1, 8192, 32, 8, 128, 0, nullptr, 256, &in) == VATTN_OK);
  CHECK(!in.direct && in.nsplit == 8 && in.combine_grid == 64 * 16);
  CHECK(in.decode_path == VATTN_DECODE_MFMA && in.threads == 256);
  // 2048-key lists, 128 units: the work floor (16 tiles per split) gives 2 splits
  CHECK(vattn::plan_compute(16, 1, 2048, 32, 8, 128, 0, nullptr, 256, &in) == VATTN_OK);
  CHECK(in.nsplit == 2 && in.chunk_keys == 1024);
  // tiny decode (128 keys): one split, direct write
  CHECK(vattn::plan_compute(2, 1, 128, 4, 1, 64, 0, nullptr, 256, &in) == VATTN_OK);
  CHECK(in.direct && in.nsplit == 1);
  // batch * kv heads fills the device (16 workgroups per CU): direct write
  CHECK(vattn::plan_compute(512, 1, 8192, 32, 8, 128, 0, nullptr, 256, &in) == VATTN_OK);
  CHECK(in.direct && in.nsplit == 1 && in.combine_grid == 0);
  // small groups take the wave path
  CHECK(vattn::plan_compute(64, 1, 8192, 16, 8, 128, 0, nullptr, 256, &in) == VATTN_OK);
  CHECK(in.decode_path == VATTN_DECODE_WAVE);
  // prefill: G heads folded into 256 rows (D <= 128); default grid from
  // B_max and s_max_q
  CHECK(vattn::plan_compute(16, 4096, 4096, 32, 8, 128, 1, nullptr, 256, &in) == VATTN_OK);
  CHECK(!in.is_decode && in.q_tokens_per_tile == 64 && in.n_qtiles == 64);
  CHECK(in.prefill_persistent == 0 && in.grid == 8192 && in.threads == 512);
  // D = 256: 128 rows, 4 waves
  CHECK(vattn::plan_compute(16, 4096, 4096, 32, 8, 256, 1, nullptr, 256, &in) == VATTN_OK);
  CHECK(in.q_tokens_per_tile == 32 && in.n_qtiles == 128 && in.grid == 16384 && in.threads == 256);
  {
    // device-built schedule: persistent grid of one workgroup per CU over a
    // list of B_max * n_qtiles slots
    vattn_plan_opts g = {};
    g.prefill_grid = 1;
    CHECK(vattn::plan_compute(16, 4096, 4096, 32, 8, 128, 1, &g, 256, &in) == VATTN_OK);
    CHECK(in.prefill_persistent == 1 && in.grid == 256 && in.scratch_bytes == 512 + 16 * 64 * 4);
    // more query tiles than the schedule handles: stays on the s_max grid
    CHECK(vattn::plan_compute(1, 8193 * 64, 64, 4, 1, 128, 1, &g, 256, &in) == VATTN_OK);
    CHECK(in.n_qtiles == 8193 && in.prefill_persistent == 0);
  }
  // validation
  CHECK(vattn::plan_compute(1, 1, 64, 6, 4, 64, 0, nullptr, 256, &in) == VATTN_ERR_INVALID_ARG);
  CHECK(vattn::plan_compute(1, 1, 64, 8, 2, 80, 0, nullptr, 256, &in) == VATTN_ERR_UNSUPPORTED);
  CHECK(vattn::plan_compute(0, 1, 64, 8, 2, 64, 0, nullptr, 256, &in) == VATTN_ERR_INVALID_ARG);
  CHECK(vattn::plan_compute(1, 0, 64, 8, 2, 64, 0, nullptr, 256, &in) == VATTN_ERR_INVALID_ARG);
  // sweep: split-rule invariants
  const int Bs[] = {1, 3, 16, 64, 200}, Ss[] = {1, 64, 65, 1000, 32768}, Hs[] = {1, 2, 8};
  for (int B : Bs)
    for (int S : Ss)
      for (int Hkv : Hs)
        for (int G : {1, 4, 8, 20}) {
          CHECK(vattn::plan_compute(B, 1, S, Hkv * G, Hkv, 64, 0, nullptr, 256, &in) == VATTN_OK);
          const int tiles = cdiv(S, 64);
          CHECK(in.nsplit >= 1 && in.nsplit <= 32 && in.nsplit <= tiles);
          CHECK(in.nsplit <= cdiv(tiles, 16));  // at least 16 tiles of work per split
          CHECK((in.nsplit - 1) * in.chunk_keys < tiles * 64 && in.nsplit * in.chunk_keys >= S);
          CHECK(in.grid == in.n_units * in.nsplit);
          CHECK(in.direct == (in.nsplit == 1));
          if (in.n_units >= VATTN_DEFAULT_TARGET * 2 * 256) CHECK(in.direct);  // D = 64: 2x target
        }
  {
    // the pages' rule: about two workgroups per CU, no work floor
    vattn_plan_opts pg = {};
    pg.target_blocks_per_cu = VATTN_PAGES_TARGET;
    pg.min_chunk_tiles = VATTN_PAGES_MIN_CHUNK;
    // tiny decode (2 units, 2 tiles): two splits and a combine
    CHECK(vattn::plan_compute(2, 1, 128, 4, 1, 64, 0, &pg, 256, &in) == VATTN_OK);
    CHECK(in.nsplit == 2 && !in.direct && in.chunk_keys == 64 && in.combine_grid == 2 * 2);
    // long decode: the cap of 32 binds
    CHECK(vattn::plan_compute(1, 1, 32768, 64, 8, 128, 0, &pg, 256, &in) == VATTN_OK);
    CHECK(in.nsplit == 32 && in.grid == 256 && in.chunk_keys == 1024);
    // continuous batching and the edge sweep: 512 units fill the device
    CHECK(vattn::plan_compute(64, 1, 8192, 32, 8, 128, 0, &pg, 256, &in) == VATTN_OK);
    CHECK(in.direct && in.nsplit == 1 && in.combine_grid == 0 && in.grid == 512);
    CHECK(vattn::plan_compute(64, 1, 16384, 128, 8, 256, 0, &pg, 256, &in) == VATTN_OK);
    CHECK(in.direct && in.grid == 512);
    // 2048-key lists over 128 units: 4 splits of 512 keys (no floor)
    CHECK(vattn::plan_compute(16, 1, 2048, 32, 8, 128, 0, &pg, 256, &in) == VATTN_OK);
    CHECK(in.nsplit == 4 && in.chunk_keys == 512);
    for (int B : Bs)
      for (int S : Ss)
        for (int Hkv : Hs) {
          CHECK(vattn::plan_compute(B, 1, S, Hkv * 8, Hkv, 64, 0, &pg, 256, &in) == VATTN_OK);
          const int tiles = cdiv(S, 64);
          int want = cdiv(2 * 256, in.n_units);
          if (want > tiles) want = tiles;
          if (want > 32) want = 32;
          const int ch = cdiv(tiles, want);
          CHECK(in.nsplit == cdiv(tiles, ch) && in.chunk_keys == ch * 64);
          CHECK(in.direct == (in.nsplit == 1));
          if (in.n_units >= 2 * 256) CHECK(in.direct);
        }
  }
  vattn_plan_opts o = {};
  o.force_nsplit = 7;
  CHECK(vattn::plan_compute(1, 1, 64 * 40, 8, 8, 64, 0, &o, 256, &in) == VATTN_OK);
  CHECK(in.nsplit == 7 && in.chunk_keys == 6 * 64);
  printf("test_plan: ok\n");
  return 0;
}
