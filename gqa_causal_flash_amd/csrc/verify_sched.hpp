// Work split of the FP8 verifier tail (host + device).
//
// Keys are cut into 32-key tiles; the tiles are spread evenly over
// 2 * grid key streams (two per workgroup), with at least kVerifyMinTiles
// tiles per stream where the key count allows, and at most one workgroup per
// compute unit.  Each workgroup leaves one partial slot of kVerifySlotRows rows.
#pragma once

#include <stddef.h>

namespace gqa {

constexpr int kVerifyMaxRows = 48;  // 8 query rows x 6 heads
constexpr int kVerifyMaxContext = 262144;
constexpr int kVerifySlotRows = 64;
constexpr size_t kVerifySlotFloats = (size_t)kVerifySlotRows * 256 + 2 * kVerifySlotRows;
constexpr int kVerifyMaxGrid = 256;
constexpr int kVerifyMinTiles = 8;

struct VerifySched {
  int ntiles;
  int grid;
};

inline VerifySched verify_schedule(int nq, int n_kv, int hq) {
  (void)nq;
  (void)hq;
  VerifySched s;
  s.ntiles = (n_kv + 31) / 32;
  int streams = s.ntiles / kVerifyMinTiles;
  if (streams < 2) streams = 2;
  int g = (streams + 1) / 2;
  if (g > kVerifyMaxGrid) g = kVerifyMaxGrid;
  s.grid = g;
  return s;
}

inline size_t verify_workspace_bytes(const VerifySched& s) { return (size_t)s.grid * kVerifySlotFloats * 4; }

}  // namespace gqa
