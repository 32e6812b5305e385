// Work decomposition of the dense causal prefill, shared by host and device.
//
// Packed rows: Q [nq][6][256] is read as a [nq*6][256] matrix whose row
// R = token*6 + head; all six heads of a token share the token's causal
// position q_pos0 + R/6 and the one K/V head, so a block of packed rows is one
// tall GEMM against each K/V tile (the head packing of the long-prefill page,
// Purpose).
//
// A q-block is 256 consecutive packed rows (one workgroup, eight waves of 32).
// Its key range is 0 .. pmax (the position of its last row), cut into 64-key
// tiles.  Laying the q-blocks' tiles end to end gives a line of T tiles that
// is split evenly over G workgroups (workgroup w takes tiles floor(wT/G) ..
// floor((w+1)T/G) - 1).  Where a workgroup's range cuts a q-block, each piece
// leaves an online-softmax partial (max, sum, unnormalised accumulator) that a
// second kernel merges exactly by log-sum-exp -- the block partial plus exact
// merge of the long-prefill page, with the split chosen for an even load on
// all compute units.  The piece of q-block b done by workgroup w is stored in
// partial slot w + b (unique: walking the line, every new piece starts at a
// workgroup boundary, a q-block boundary or both).
#pragma once

#include <stdint.h>

namespace gqa {

#ifndef GQA_PREFILL_ROWS
#define GQA_PREFILL_ROWS 256
#endif
constexpr int kRowsPerBlock = GQA_PREFILL_ROWS;  // packed rows per workgroup
constexpr int kWGsPerCU = 1;                     // 128 KiB of LDS per workgroup
constexpr int kTileKeys = 64;       // keys per K/V tile
constexpr int kTargetGrid = 256;    // one workgroup per MI355X compute unit
constexpr int kMinTilesPerWG = 16;

struct PrefillSched {
  int nrows;        // nq * hq
  int q_pos0;
  int nqb;          // number of q-blocks
  long long total;  // T
  int grid;         // G
  int split;        // >0: key-split mode with this many pieces per q-block (see below)
};

__host__ __device__ inline int prefill_block_tiles(int b, int nrows, int q_pos0) {
  int last = (b + 1) * kRowsPerBlock - 1;
  if (last > nrows - 1) last = nrows - 1;
  const int pmax = q_pos0 + last / 6;
  return (pmax + kTileKeys) / kTileKeys;  // ceil((pmax + 1) / 64)
}

// First tile of workgroup w's range.
__host__ __device__ inline long long prefill_range_start(int w, long long total, int grid) {
  return (long long)w * total / grid;
}

// Workgroup whose range contains tile x.
__host__ __device__ inline int prefill_owner(long long x, long long total, int grid) {
  return (int)(((x + 1) * grid - 1) / total);
}

// Key-split mode (used when split > 0): q-block b's tiles are cut into `split`
// equal key ranges, piece j = tiles floor(j n_b / split) .. floor((j+1) n_b /
// split) - 1, and workgroup u = (nqb - 1 - b) * split + j runs piece j of
// q-block b (the longest q-blocks, the last ones, go first).  With split
// dividing 8, the round-robin placement of workgroup u on XCD u % 8 puts only
// piece u % split on each XCD, so the 32 workgroups of an XCD stream the same
// K/V range at the same pace and share that XCD's L2.  Piece j of q-block b
// leaves its partial in slot b * split + j.
#ifndef GQA_PREFILL_KEYSPLIT
#define GQA_PREFILL_KEYSPLIT 1
#endif

inline PrefillSched prefill_schedule(int nq, int hq, int q_pos0) {
  PrefillSched s;
  s.nrows = nq * hq;
  s.q_pos0 = q_pos0;
  s.nqb = (s.nrows + kRowsPerBlock - 1) / kRowsPerBlock;
  long long t = 0;
  for (int b = 0; b < s.nqb; ++b) t += prefill_block_tiles(b, s.nrows, q_pos0);
  s.total = t;
  long long g = (t + kMinTilesPerWG - 1) / kMinTilesPerWG;
  if (g < s.nqb) g = s.nqb;
  if (g > kTargetGrid) g = kTargetGrid;
  if (g > t) g = t;
  s.grid = (int)g;
  s.split = 0;
  if (GQA_PREFILL_KEYSPLIT) {
    // smallest power-of-two split (<= 8) giving at least two workgroups per compute unit,
    // never more pieces than the shortest q-block has tiles
    int minnt = 1 << 30;
    for (int b = 0; b < s.nqb; ++b) {
      const int nt = prefill_block_tiles(b, s.nrows, q_pos0);
      if (nt < minnt) minnt = nt;
    }
    int sp = 1;
    while (sp < 8 && (long long)s.nqb * sp < 2LL * kTargetGrid * kWGsPerCU && sp * 2 <= minnt) sp *= 2;
    s.split = sp;
    s.grid = s.nqb * sp;
  }
  return s;
}

// Partial slot: fp32 acc [64 column quads][rows][4], then m [rows], then l [rows].
constexpr size_t kPartialFloats = (size_t)kRowsPerBlock * 256 + 2 * kRowsPerBlock;

// True when some q-block is cut between workgroups (its partials need merging).
inline bool prefill_needs_merge(const PrefillSched& s) {
  if (s.split > 0) return s.split > 1;
  long long cb = 0;
  for (int b = 0; b < s.nqb; ++b) {
    const int nt = prefill_block_tiles(b, s.nrows, s.q_pos0);
    if (prefill_owner(cb, s.total, s.grid) != prefill_owner(cb + nt - 1, s.total, s.grid)) return true;
    cb += nt;
  }
  return false;
}

inline size_t prefill_workspace_bytes(const PrefillSched& s) {
  if (!prefill_needs_merge(s)) return 0;
  if (s.split > 0) return (size_t)s.grid * kPartialFloats * sizeof(float);
  return (size_t)(s.grid + s.nqb) * kPartialFloats * sizeof(float);
}

// Varlen prefill (a batch of sequences packed end to end): the q-blocks of
// all sequences number at most cap = ceil(6 total_q / 256) + batch (each
// sequence adds at most one partial q-block), which sizes the grid before the
// sequence lengths, held in device memory, are known.  Every q-block is cut
// into `split` key ranges: the smallest power of two (<= 8) giving at least
// four workgroups per compute unit, since q-blocks of sequences of different
// lengths carry different amounts of work and finer pieces even them out.
// Workspace: header (16 B: q-blocks used, sequences skipped), cap descriptors
// of 8 int32, then cap * split partial slots when split > 1.
constexpr size_t kVarlenHeaderBytes = 16;

struct VarlenSched {
  int cap;
  int split;
};

inline VarlenSched prefill_varlen_schedule(int batch, int total_q) {
  VarlenSched s;
  s.cap = (int)((6LL * total_q + kRowsPerBlock - 1) / kRowsPerBlock) + batch;
  int sp = 1;
  while (sp < 8 && (long long)s.cap * sp < 4LL * kTargetGrid) sp *= 2;
  s.split = sp;
  return s;
}

inline size_t varlen_part_offset(const VarlenSched& s) {
  return (kVarlenHeaderBytes + (size_t)s.cap * 8 * sizeof(int) + 255) / 256 * 256;
}

inline size_t prefill_varlen_workspace_bytes(const VarlenSched& s) {
  const size_t parts = s.split > 1 ? (size_t)s.cap * s.split * kPartialFloats * sizeof(float) : 0;
  return varlen_part_offset(s) + parts;
}

}  // namespace gqa
