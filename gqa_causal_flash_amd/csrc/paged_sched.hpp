// Sizes and workspace layout of the paged block-sparse prefill (host + device).
//
// Query block b = 64 query tokens = 384 packed rows (token * 6 + head), handled
// by three workgroups of 128 packed rows (4 waves x 32 rows).  Its selection
// of 4-token KV blocks is translated, checked, freed of repeats and packed by
// a prepass into the workspace:
//
//   int32 header[4]   {magic, number of query blocks, number of ids, 0}
//   int32 err[nqb]    index entries of block b dropped as invalid
//   int32 beg[nqb]    first entry of block b in `entries`
//   int32 cnt[nqb]    number of entries of block b
//   int32 nvis[nqb]   number of leading entries of block b that every row of
//                     the block sees whole (entries ascending by token, all
//                     four tokens at or before the block's first row); 0 when
//                     the entries are in the given order
//   int2  entries[n_block_ids]  {first physical cache row, first logical token};
//                                a long selection over a table too large for
//                                the prepass bitmap keeps {-1, INT32_MAX} in
//                                place for an entry that holds no live token
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace gqa {

constexpr int kBlockTokens = 4;
constexpr int kMaxPageSize = 4096;  // tokens per page; any multiple of kBlockTokens up to this
constexpr int kQBlockTokens = 64;
constexpr int kQBlockRows = kQBlockTokens * 6;  // 384 packed rows
constexpr int kPagedRowsPerWG = 128;
constexpr int kPagedWGsPerQBlock = kQBlockRows / kPagedRowsPerWG;  // 3
constexpr int kPagedMagic = 0x47514150;  // "PAQG"
constexpr int kBitmapBlocks = 262144;    // tables of up to this many blocks (1M tokens) use the bitmap prepass
constexpr int kDedupMax = 2048;          // beyond that, selections up to this many blocks are checked for repeats

// The attention kernel cuts the work, sub-tiles of 32 keys of every query
// block, into runs of equal cost, each taken by a team of three workgroups
// (one per 128-row group of the query block), 21 teams per XCD: 504
// workgroups, two per compute unit.  A query block with n sub-tiles costs
// n + kPagedSwitchUnits: starting on a query block (its Q rows, its first
// gather, writing its result) takes about as long as that many sub-tiles.  A
// team writes the query blocks it covers whole straight to O; each of the two
// at its ends that it covers only in part leaves, per row group, a partial of
// 128 rows (fp32 acc, m, l) in one of the workgroup's two slots, which a
// merge kernel combines.
constexpr int kPagedSwitchUnits = 3;
// A run boundary that would leave fewer than this many sub-tiles of a query
// block on one side moves to that block's start or end instead.
constexpr int kPagedMinPiece = 2;
constexpr int kPagedTeams = 168;  // 8 XCDs x 21 teams
constexpr int kPagedGrid = 512;   // workgroup ids: 64 per XCD, 63 of them in teams
constexpr int kPagedSlots = 2 * 3 * kPagedTeams;

constexpr size_t kPagedSlotFloats = (size_t)kPagedRowsPerWG * 256 + 2 * kPagedRowsPerWG;

struct PagedLayout {
  size_t err, beg, cnt, nvis, entries, part, total;
};

inline PagedLayout paged_layout(int nqb, int n_ids) {
  PagedLayout L;
  L.err = 16;
  L.beg = L.err + 4 * (size_t)nqb;
  L.cnt = L.beg + 4 * (size_t)nqb;
  L.nvis = L.cnt + 4 * (size_t)nqb;
  L.entries = (L.nvis + 4 * (size_t)nqb + 15) / 16 * 16;
  L.part = (L.entries + 8 * (size_t)(n_ids > 0 ? n_ids : 1) + 255) / 256 * 256;
  L.total = L.part + (size_t)kPagedSlots * kPagedSlotFloats * 4;
  return L;
}

}  // namespace gqa
