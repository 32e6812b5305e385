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
// tiles.  The tiles of every q-block are cut into `split` equal key ranges
// (pieces); each piece runs as one workgroup and, when split > 1, leaves an
// online-softmax partial (max, sum, unnormalised accumulator) that a second
// kernel merges exactly by log-sum-exp -- the block partial plus exact merge
// of the long-prefill page, with the split chosen for an even load on all
// compute units.  A workload too small to give every compute unit a
// workgroup that way takes q-blocks of 128 rows (four waves of 32) instead:
// twice the workgroups, each with half the matrix-core work per key tile.
#pragma once

#include <stdint.h>

namespace gqa {

constexpr int kRowsPerBlock = 256;  // packed rows per workgroup
constexpr int kRowsSmall = 128;     // packed rows per workgroup of small workloads
constexpr int kWGsPerCU = 1;        // 128 KiB of LDS per workgroup
constexpr int kTileKeys = 64;       // keys per K/V tile
constexpr int kTargetGrid = 256;    // one workgroup per MI355X compute unit

struct PrefillSched {
  int nrows;   // nq * hq
  int q_pos0;
  int rows;    // packed rows per q-block: kRowsPerBlock or kRowsSmall
  int nqb;     // number of q-blocks
  int split;   // pieces per q-block (see below)
  int grid;    // nqb * split workgroups
};

__host__ __device__ inline int prefill_block_tiles(int b, int rows, int nrows, int q_pos0) {
  int last = (b + 1) * rows - 1;
  if (last > nrows - 1) last = nrows - 1;
  const int pmax = q_pos0 + last / 6;
  return (pmax + kTileKeys) / kTileKeys;  // ceil((pmax + 1) / 64)
}

// Piece j of q-block b is tiles floor(j n_b / split) .. floor((j+1) n_b /
// split) - 1, and workgroup u = (nqb - 1 - b) * split + j runs it (the
// longest q-blocks, the last ones, go first).  With split dividing 8, the
// round-robin placement of workgroup u on XCD u % 8 puts only piece u % split
// on each XCD, so the 32 workgroups of an XCD stream the same K/V range at
// the same pace and share that XCD's L2.  Piece j of q-block b leaves its
// partial in slot b * split + j.  The split is the smallest power of two
// (<= 8) giving at least two workgroups per compute unit, and never more
// pieces than the shortest q-block has tiles.
inline PrefillSched prefill_schedule_rows(int nq, int hq, int q_pos0, int rows) {
  PrefillSched s;
  s.nrows = nq * hq;
  s.q_pos0 = q_pos0;
  s.rows = rows;
  s.nqb = (s.nrows + rows - 1) / rows;
  int minnt = 1 << 30;
  for (int b = 0; b < s.nqb; ++b) {
    const int nt = prefill_block_tiles(b, rows, s.nrows, q_pos0);
    if (nt < minnt) minnt = nt;
  }
  int sp = 1;
  while (sp < 8 && (long long)s.nqb * sp < 2LL * kTargetGrid * kWGsPerCU && sp * 2 <= minnt) sp *= 2;
  s.split = sp;
  s.grid = s.nqb * sp;
  return s;
}

// The fp16 kernel's schedule: 256-row q-blocks, or 128-row ones when the
// 256-row schedule leaves compute units without a workgroup.
inline PrefillSched prefill_schedule(int nq, int hq, int q_pos0) {
  const PrefillSched s = prefill_schedule_rows(nq, hq, q_pos0, kRowsPerBlock);
  return s.grid < kTargetGrid ? prefill_schedule_rows(nq, hq, q_pos0, kRowsSmall) : s;
}

// Partial slot of a q-block of `rows` packed rows: fp32 acc [64 column
// quads][rows][4], then m [rows], then l [rows].
__host__ __device__ constexpr size_t prefill_partial_floats(int rows) { return (size_t)rows * 256 + 2 * (size_t)rows; }
constexpr size_t kPartialFloats = prefill_partial_floats(kRowsPerBlock);

// True when the q-blocks are cut into pieces whose partials need merging.
inline bool prefill_needs_merge(const PrefillSched& s) { return s.split > 1; }

inline size_t prefill_workspace_bytes(const PrefillSched& s) {
  return prefill_needs_merge(s) ? (size_t)s.grid * prefill_partial_floats(s.rows) * sizeof(float) : 0;
}

// One workspace size serves the fp16 kernel's schedule and the E4M3 kernel's,
// which always takes 256-row q-blocks.  (The 256-row figure is the larger: a
// 128-row schedule has at most twice the q-blocks, no larger a split and
// partials of half the size.)
inline size_t prefill_any_workspace_bytes(int nq, int hq, int q_pos0) {
  const size_t a = prefill_workspace_bytes(prefill_schedule(nq, hq, q_pos0));
  const size_t b = prefill_workspace_bytes(prefill_schedule_rows(nq, hq, q_pos0, kRowsPerBlock));
  return a > b ? a : b;
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
