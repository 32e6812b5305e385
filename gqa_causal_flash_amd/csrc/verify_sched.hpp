// Work split of the FP8 verifier tail (host + device).
//
// Keys are cut into 32-key tiles; the tiles are spread evenly over the
// workgroups (one key stream each, two per compute unit), with at least
// kVerifyMinTiles tiles per workgroup where the key count allows.  Each
// workgroup leaves one partial slot of kVerifySlotRows rows.
#pragma once

#include <stddef.h>

namespace gqa {

constexpr int kVerifyMaxRows = 48;  // 8 query rows x 6 heads
constexpr int kVerifyMaxContext = 262144;
constexpr int kVerifySlotRows = 64;
constexpr size_t kVerifySlotFloats = (size_t)kVerifySlotRows * 256 + 2 * kVerifySlotRows;
constexpr int kVerifyMaxGrid = 512;
constexpr int kVerifyMinTiles = 8;

struct VerifySched {
  int ntiles;
  int grid;
  int row_blocks;  // 32-row blocks of packed rows: 1 (q <= 5) or 2 (q = 6..8)
};

// Each workgroup has two waves per 32-row block; the two waves of a block
// take alternate tiles and combine their states in LDS before the workgroup
// writes its one partial.
inline VerifySched verify_schedule(int nq, int n_kv, int hq) {
  VerifySched s;
  s.ntiles = (n_kv + 31) / 32;
  int g = s.ntiles / kVerifyMinTiles;
  if (g < 1) g = 1;
  if (g > kVerifyMaxGrid) g = kVerifyMaxGrid;
  s.grid = g;
  s.row_blocks = nq * hq <= 32 ? 1 : 2;
  return s;
}

inline size_t verify_workspace_bytes(const VerifySched& s) { return (size_t)s.grid * kVerifySlotFloats * 4; }

// Workspace of the largest schedule (any nq <= 8, n_kv <= 262144): 33.8 MB.
constexpr size_t kVerifyScratchBytes = (size_t)kVerifyMaxGrid * kVerifySlotFloats * 4;

}  // namespace gqa
