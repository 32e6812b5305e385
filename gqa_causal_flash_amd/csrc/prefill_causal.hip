// Dense causal GQA prefill for gfx950: fused S^T = K Q^T, online softmax and
// O^T += V^T P^T on the matrix cores, split evenly over the compute units with
// an exact log-sum-exp merge.
//
// The operation is the causal FP16 long-prefill of the long-prefill page
// ("[Kernel][SM70] Default long-prefill GQA architecture", Purpose): six query
// heads sharing one K/V head at D = 256, packed so that every K/V fragment is
// used by all six heads, with per-tile (max, sum, accumulator) states merged
// exactly.  That page's V100 design (separate QK and PV Tensor-Core GEMMs
// through a 750-MiB score workspace) is not followed: scores never leave the
// registers.
//
// Workgroup: 8 waves (two per SIMD) x 32 packed rows = 256 rows (a q-block).
// Each wave keeps its 32 rows of Q as matrix-core B fragments in registers
// (16 steps of 16 head-dim columns) and its O^T accumulator (8 tiles of 32x32
// fp32).  K/V tiles of 64 keys stream HBM -> LDS by direct-to-LDS loads into a
// double buffer (2 x 64 KiB).  Small workloads take q-blocks of 128 rows:
// four waves, one per SIMD, with the same per-wave work.  (Templates C and W
// give other row splits, 32C rows per wave and W waves; the default is C = 1,
// W = 8, or W = 4 for 128-row q-blocks.)
#include "attn_common.hpp"
#include "attn_tile.hpp"
#include "prefill_sched.hpp"
#include "launch.hpp"

#include <type_traits>

namespace gqa {

namespace {

constexpr int kTileBytes = kTileKeys * kRowBytes;  // 32 KiB per K or V tile
// Rows per wave = 32 * kPrefillC, waves per workgroup = kPrefillW (256-row
// q-blocks) or kSmallW (128-row q-blocks).
#ifndef GQA_PREFILL_C
#define GQA_PREFILL_C 1
#endif
constexpr int kPrefillC = GQA_PREFILL_C;
constexpr int kPrefillW = kRowsPerBlock / (32 * kPrefillC);
constexpr int kSmallW = kRowsSmall / (32 * kPrefillC);

struct PrefillParams {
  const _Float16* q;
  const _Float16* k;
  const _Float16* v;
  _Float16* o;
  float* part;
  int nrows;
  int qrows;    // packed rows per q-block (and per partial slot)
  int kv_live;  // keys 0 .. kv_live-1 can be visible (q_pos0 + nq)
  int q_pos0;
  int nqb;
  int grid;
  int split;  // key-split pieces per q-block
  unsigned long long* clk;  // profiling: {shader cycles, wall ticks} accumulator, or null
  float* lse;               // per packed row log-sum-exp (natural log), or null
  const int* vdesc;         // varlen: block descriptors (see prefill_varlen_prepass), else null
  uint32_t part_bytes;
  float c;     // scale * log2(e): scores are kept in log2 units
  float post;  // factor applied to O at the end (the V scale of E4M3 inputs, else 1)
};

constexpr float kLn2 = 0.69314718055994531f;

// log sum_j exp(scale q.k_j) of a row from its online-softmax state: m is the
// reference maximum and l the sum of 2^(t_j - m), both in log2 units.
__device__ __forceinline__ float row_lse(float m, float l) {
  return (l > 0.f) ? (m + __builtin_log2f(l)) * kLn2 : -INFINITY;
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Stage keys tile*64 .. tile*64+63 of K and V into LDS.  With W waves, wave w
// copies rows (64/W)w .. (64/W)(w+1)-1: 32/W copies of 1 KiB (two rows) for K
// and as many for V.  Rows past the last key read as zeros (buffer range
// check); they lie after every query position, so they are always masked.
//
// Lane l of copy i fills physical chunk l%32 of row r = (64/W)w + 2i + l/32,
// so it fetches the logical chunk that the swizzle puts there.  With
// x = r % 16 = (2i + l/32) % 16 (64/W is a multiple of 16 for W <= 4, and for
// W = 8 the wave's first row is a multiple of 8, which the V swizzle only
// needs), the byte offset from the wave's first row is
// 2i*512 + l/32*512 + 16*(l%32 ^ swz(r)): for K, swz(r) = r % 16 gives
// (kl ^ 32(i + 4*(w%2 when W=8))) + 1024i ... computed below per copy.
template <int W, int TK = kTileKeys>
__device__ __forceinline__ void issue_rows(rsrc_t rk, rsrc_t rv, uint32_t tile_byte, char* kdst, char* vdst,
                                           int wave, uint32_t kl, uint32_t vl) {
  constexpr int kRowsPerWave = TK / W;
  constexpr int kCopies = kRowsPerWave / 2;
  static_assert(kCopies >= 1 && kRowsPerWave <= 16, "2..16 rows per wave");
  const uint32_t soff = tile_byte + (uint32_t)wave * (kRowsPerWave * kRowBytes);
  // copy i covers rows r0 = kRowsPerWave*wave + 2i (+1); its index within the
  // 16-row swizzle period is j = (r0 % 16) / 2
  const int jbase = (kRowsPerWave * wave % 16) / 2;
#pragma unroll
  for (int i = 0; i < kCopies; ++i) {
    const int r0 = kRowsPerWave * wave + 2 * i;
    const uint32_t j = (uint32_t)(jbase + i);  // < 8
    load_lds_16B(rk, (GQA_LDS char*)(kdst + r0 * kRowBytes), kl ^ (32u * j), soff + 1024u * i);
    load_lds_16B(rv, (GQA_LDS char*)(vdst + r0 * kRowBytes), vl ^ (128u * (j & 3)), soff + 1024u * i);
  }
}

template <int W>
__device__ __forceinline__ void issue_tile(rsrc_t rk, rsrc_t rv, int tile, char* kdst, char* vdst, int wave,
                                           uint32_t kl, uint32_t vl) {
  issue_rows<W>(rk, rv, (uint32_t)tile * (kTileKeys * kRowBytes), kdst, vdst, wave, kl, vl);
}

// One piece of work: tiles tile_lo .. tile_hi-1 of q-block b, with W waves
// of 32*C packed rows each (32*C*W = the q-block's rows, p.qrows).
template <int C, int W>
__device__ __forceinline__ void prefill_piece(const PrefillParams& p, char* smem, int b, int tile_lo, int tile_hi,
                                              bool full, int slot) {
  constexpr int kRowsPerWave = 32 * C;
  constexpr int kRows = kRowsPerWave * W;
  static_assert(kRows == kRowsPerBlock || kRows == kRowsSmall, "a workgroup covers one q-block");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;
  const uint32_t kl = 512u * half + 16u * (uint32_t)(col ^ half);
  const uint32_t vl = 512u * half + ((16u * col) ^ (64u * half));

  const rsrc_t rq = make_rsrc(p.q, (uint32_t)p.nrows * kRowBytes);
  // keys after the last query position never take part: they read as zeros
  const rsrc_t rk = make_rsrc(p.k, (uint32_t)p.kv_live * kRowBytes);
  const rsrc_t rv = make_rsrc(p.v, (uint32_t)p.kv_live * kRowBytes);

  const int row_base = b * kRows + wave * kRowsPerWave;
  const bool wave_active = row_base < p.nrows;
  const int wrow_hi = min(row_base + kRowsPerWave - 1, p.nrows - 1);
  const int wpos_lo = p.q_pos0 + row_base / kGroup;
  const int wpos_hi = p.q_pos0 + wrow_hi / kGroup;

  int pos[C];
  h8 qf[C][16];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int row = row_base + 32 * c + col;
    pos[c] = p.q_pos0 + min(row, p.nrows - 1) / kGroup;
    const uint32_t qoff = (uint32_t)row * kRowBytes + half * 16;
#pragma unroll
    for (int s = 0; s < 16; ++s) qf[c][s] = load_16B(rq, qoff + s * 32);
  }

  f16x acc[C][8];
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[c][dt] = f16x{};
  float m[C], l[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    m[c] = -INFINITY;
    l[c] = 0.f;
  }

  // LDS: V buffers at 0 and 32 KiB, K buffers at 64 and 96 KiB (every
  // fragment offset then fits the 16-bit immediate of the LDS read).
  uint32_t bk = k_lane_base(lane);
  uint32_t bv = v_lane_base(lane);

  issue_tile<W>(rk, rv, tile_lo, smem + 2 * kTileBytes, smem, wave, kl, vl);
  wait_vmem();
  __syncthreads();

  auto step = [&](auto bufc, int tile) {
    constexpr int BUF = decltype(bufc)::value;
    if (tile + 1 < tile_hi)
      issue_tile<W>(rk, rv, tile + 1, smem + (2 + (BUF ^ 1)) * kTileBytes, smem + (BUF ^ 1) * kTileBytes, wave, kl,
                    vl);
    const GQA_LDS char* kt = (const GQA_LDS char*)smem + (2 + BUF) * kTileBytes;
    const GQA_LDS char* vt = (const GQA_LDS char*)smem + BUF * kTileBytes;

#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int k0 = tile * kTileKeys + 32 * kb;
      if (!wave_active || k0 > wpos_hi) continue;  // every key of this block is in the future
      // keep the per-lane bases opaque so derived addresses are formed here,
      // next to their use, instead of being hoisted and held in registers
      asm volatile("" : "+v"(bk), "+v"(bv));
      // mask only blocks that cross the causal diagonal of some row of the wave
      attend_32keys<C>(lds_addr(kt) + bk, vt, bv, kb, qf, acc, m, l, p.c, k0 + 31 > wpos_lo,
                       [&](int c, int vv) { return k0 + lane_key(vv, half) <= pos[c]; });
    }
    wait_vmem();
    __syncthreads();
  };

  for (int tile = tile_lo; tile < tile_hi; tile += 2) {
    step(std::integral_constant<int, 0>{}, tile);
    if (tile + 1 < tile_hi) step(std::integral_constant<int, 1>{}, tile + 1);
  }

  float lt[C];
#pragma unroll
  for (int c = 0; c < C; ++c) lt[c] = swap_halves_sum(l[c]);

  if (full) {
    const rsrc_t ro = make_rsrc(p.o, (uint32_t)p.nrows * kRowBytes);
#pragma unroll
    for (int c = 0; c < C; ++c) store_rows_f16(ro, row_base + 32 * c + col, half, acc[c], lt[c], 1.0f);
    if (p.lse != nullptr && half == 0) {
      const rsrc_t rl = make_rsrc(p.lse, (uint32_t)p.nrows * 4);
#pragma unroll
      for (int c = 0; c < C; ++c)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(row_lse(m[c], lt[c])), rl,
                                              (uint32_t)(row_base + 32 * c + col) * 4, 0, 0);
    }
  } else {
    const rsrc_t rp = make_rsrc(p.part, p.part_bytes);
    const uint32_t sbase = (uint32_t)slot * (uint32_t)(prefill_partial_floats(kRows) * 4);
#pragma unroll
    for (int c = 0; c < C; ++c)
      store_partial(rp, sbase, kRows, wave * kRowsPerWave + 32 * c + col, half, acc[c], m[c], lt[c]);
  }
}

// Runs the pieces of workgroup blockIdx.x: run(b, tile_lo, tile_hi, full, slot)
// for each (q-block, key range) the schedule gives it.
template <class Run>
__device__ __forceinline__ void prefill_workgroup(const PrefillParams& p, Run run) {
  const int w = blockIdx.x;
  // q-blocks are dispatched last first: they are the longest, so the
  // shortest pieces end the kernel
  const int b = p.nqb - 1 - w / p.split, j = w % p.split;
  const int nt = prefill_block_tiles(b, p.qrows, p.nrows, p.q_pos0);
  const int lo = (int)((long long)j * nt / p.split), hi = (int)((long long)(j + 1) * nt / p.split);
  // the split never exceeds the shortest q-block's tile count, so lo < hi
  run(b, lo, hi, p.split == 1, b * p.split + j);
}

template <int C, int W>
__global__ __launch_bounds__(64 * W, 1) void prefill_causal_fwd(PrefillParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[4 * kTileBytes];
  // profiling only: the workgroup's lifetime in shader cycles and wall ticks
  // as seen by its first wave (clock64: shader clock; wall_clock64: constant
  // rate); lane 0 adds them to the accumulator with vector atomics
  const bool stamp = p.clk != nullptr && __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 0;
  unsigned long long c0 = 0, r0 = 0;
  if (stamp) {
    c0 = clock64();
    r0 = wall_clock64();
  }
  prefill_workgroup(p, [&](int b, int lo, int hi, bool full, int slot) {
    prefill_piece<C, W>(p, smem, b, lo, hi, full, slot);
  });
  if (stamp) {
    const unsigned long long dc = clock64() - c0, dr = wall_clock64() - r0;
    if (threadIdx.x == 0) {
      atomicAdd(p.clk, dc);
      atomicAdd(p.clk + 1, dr);
    }
  }
}

// ------------------------------------------------------------ E4M3 inputs
// Causal prefill with Q, K and V given as OCP E4M3 codes and one fp32 scale
// per tensor (the long-context page's grouped E4M3 operator, "[Perf] Ship the
// qualified SM70 long-context layout...", What, with Q quantised as well so
// that S^T = K Q^T runs on the FP8 matrix cores).  Same workgroup shape,
// schedule, softmax and P V step as the fp16 kernel; what differs:
//   * Q stays as E4M3 in registers: for product step si (head-dim columns
//     64si .. 64si+63) lane (row l%32, half h) holds the 32 bytes of columns
//     64si + 32h .. +31.  K fragments carry the same columns of a key, so the
//     v_mfma_f32_32x32x64_f8f6f4 sums run over all 64 columns in either
//     operand's order (every E4M3 product is exact in fp32).
//   * K tiles stream HBM -> LDS as E4M3 (64 keys x 256 B), chunk c of row r
//     stored at c ^ (r % 16), so the two 16-byte reads of a fragment are
//     bank-conflict free.
//   * V tiles are loaded into registers one tile ahead, decoded exactly to
//     fp16 (v_cvt_scalef32_pk_f16_fp8) and written into the fp16 V layout of
//     the next buffer before the step's barrier; P V is the fp16 step.
//   * q_scale * k_scale joins the softmax scale; v_scale multiplies O at the
//     end (and the partials before they are stored).
constexpr int kRowBytes8 = kHeadDim;                 // one E4M3 row: 256 B = 16 chunks
constexpr int kTileBytes8 = kTileKeys * kRowBytes8;  // 16 KiB

typedef int v8i __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f16x mfma_fp8(v8i a, v8i b, f16x c) {
  // format 0 = E4M3 for both operands; zero scale operands select the unscaled product
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v8i cat_u4(u4 a, u4 b) {
  return v8i{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

// 16 E4M3 codes -> 16 fp16 values (exact), as two 16-byte chunks.
__device__ __forceinline__ void decode16(u4 raw, u4& lo, u4& hi) {
  h2 x[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    x[2 * w] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[w], 1.0f, false);
    x[2 * w + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[w], 1.0f, true);
  }
  lo = u4{__builtin_bit_cast(unsigned, x[0]), __builtin_bit_cast(unsigned, x[1]), __builtin_bit_cast(unsigned, x[2]),
          __builtin_bit_cast(unsigned, x[3])};
  hi = u4{__builtin_bit_cast(unsigned, x[4]), __builtin_bit_cast(unsigned, x[5]), __builtin_bit_cast(unsigned, x[6]),
          __builtin_bit_cast(unsigned, x[7])};
}

// Stage K keys tile*64 .. +63 (E4M3) into LDS: wave w copies rows 8w .. 8w+7 as
// two 1 KiB copies of four rows; lane i of copy j fills physical chunk i%16 of
// row r = 8w + 4j + i/16 with logical chunk (i%16) ^ (r%16).
__device__ __forceinline__ void issue_k8(rsrc_t rk, int tile, GQA_LDS char* kdst, int wave, int lane) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 8 * wave + 4 * j + (lane >> 4);
    const uint32_t voff = (uint32_t)r * kRowBytes8 + 16u * (uint32_t)((lane & 15) ^ (r & 15));
    load_lds_16B(rk, kdst + (8 * wave + 4 * j) * kRowBytes8, voff, (uint32_t)tile * kTileBytes8);
  }
}

// V keys tile*64 .. +63 (E4M3): thread t holds two 16-byte pieces of key
// r = t/8, pieces a and a + 8 with a = 2k for k = t%8 < 4 and 2k - 7
// otherwise (piece p = columns 16p .. 16p+15).  A piece decodes to fp16
// chunks 2p and 2p + 1; odd rows load the two 8-byte halves of a piece in
// swapped order, so register half 0 always holds chunk 2p + (r & 1).  With
// that, every 16-lane pass of each 16-byte LDS write in store_v16 (two rows
// of 8 lanes) lands on 16 distinct bank positions: the decoded tile is
// written without bank conflicts, at no vector-instruction cost.
__device__ __forceinline__ int v8_piece(int tid) {
  const int k = tid & 7;
  return k < 4 ? 2 * k : 2 * k - 7;
}
__device__ __forceinline__ void load_v8(rsrc_t rv, int tile, int tid, u4 (&raw)[2]) {
  const int r = tid >> 3;
  const uint32_t sw = 8u * (uint32_t)(r & 1);
  const uint32_t row = (uint32_t)tile * kTileBytes8 + (uint32_t)r * kRowBytes8 + 16u * (uint32_t)v8_piece(tid);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const u2 lo = __builtin_amdgcn_raw_buffer_load_b64(rv, row + 128u * i + sw, 0, 0);
    const u2 hi = __builtin_amdgcn_raw_buffer_load_b64(rv, row + 128u * i + (8u - sw), 0, 0);
    raw[i] = u4{lo[0], lo[1], hi[0], hi[1]};
  }
}

// Decoded V of thread t into the fp16 tile: piece a + 8i gives chunks
// 2(a + 8i) + (r & 1) (register half 0) and the other chunk of the pair, each
// at its swizzled place c ^ 4(r%8).
__device__ __forceinline__ void store_v16(GQA_LDS char* vdst, int tid, const u4 (&raw)[2]) {
  const int r = tid >> 3, sw = r & 1;
  const int c0 = 2 * v8_piece(tid);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    u4 d0, d1;
    decode16(raw[i], d0, d1);
    *(GQA_LDS u4*)(vdst + r * kRowBytes + 16 * v_phys_chunk(c0 + 16 * i + sw, r)) = d0;
    *(GQA_LDS u4*)(vdst + r * kRowBytes + 16 * v_phys_chunk(c0 + 16 * i + 1 - sw, r)) = d1;
  }
}

// K fragment of product step si for keys 32kb .. 32kb+31 of the E4M3 tile:
// lane (key r = l%32, half h) reads logical chunks 4si + 2h and 4si + 2h + 1 of
// row 32kb + r, at byte 8192kb + (b8 ^ 64si) and that ^ 16, where
// b8 = 256 r + 16 (2h ^ (r % 16)).
__device__ __forceinline__ uint32_t k8_lane_base(int lane) {
  const int r = lane & 31, h = lane >> 5;
  return 256u * (uint32_t)r + 16u * (uint32_t)((2 * h) ^ (r & 15));
}
__device__ __forceinline__ v8i read_k8_frag(const GQA_LDS char* kt, uint32_t bk, int kb, int si) {
  const uint32_t a = (bk ^ (64u * si)) + 8192u * kb;
  const u4 x = *(const GQA_LDS u4*)(kt + a);
  const u4 y = *(const GQA_LDS u4*)(kt + (a ^ 16u));
  return cat_u4(x, y);
}

// LDS of the E4M3 kernel: two fp16 V tiles and two E4M3 K tiles, each its own
// array so that the compiler can tell the tile being read from the one being
// loaded (it would otherwise wait for the next tile's loads before every read).
struct E4M3Lds {
  GQA_LDS char* v16[2];
  GQA_LDS char* k8[2];
};

template <int W>
__device__ __forceinline__ void prefill_piece_e4m3(const PrefillParams& p, const E4M3Lds& sm, int b, int tile_lo,
                                                   int tile_hi, bool full, int slot) {
  constexpr int kRowsPerWave = 32;
  static_assert(kRowsPerWave * W == kRowsPerBlock && W == 8, "eight waves of 32 rows");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;

  const rsrc_t rq = make_rsrc(p.q, (uint32_t)p.nrows * kRowBytes8);
  const rsrc_t rk = make_rsrc(p.k, (uint32_t)p.kv_live * kRowBytes8);
  const rsrc_t rv = make_rsrc(p.v, (uint32_t)p.kv_live * kRowBytes8);

  const int row_base = b * kRowsPerBlock + wave * kRowsPerWave;
  const bool wave_active = row_base < p.nrows;
  const int wrow_hi = min(row_base + kRowsPerWave - 1, p.nrows - 1);
  const int wpos_lo = p.q_pos0 + row_base / kGroup;
  const int wpos_hi = p.q_pos0 + wrow_hi / kGroup;

  const int row = row_base + col;
  const int pos = p.q_pos0 + min(row, p.nrows - 1) / kGroup;
  v8i qf[4];
  {
    const uint32_t qoff = (uint32_t)row * kRowBytes8 + 32u * half;
#pragma unroll
    for (int si = 0; si < 4; ++si)
      qf[si] = cat_u4(__builtin_amdgcn_raw_buffer_load_b128(rq, qoff + 64 * si, 0, 0),
                      __builtin_amdgcn_raw_buffer_load_b128(rq, qoff + 64 * si + 16, 0, 0));
  }

  f16x acc[1][8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) acc[0][dt] = f16x{};
  float m[1] = {-INFINITY}, l[1] = {0.f};

  uint32_t bk = k8_lane_base(lane);
  uint32_t bv = v_lane_base(lane);

  // first tile: K into buffer 0, V decoded into fp16 buffer 0
  {
    issue_k8(rk, tile_lo, sm.k8[0], wave, lane);
    u4 raw[2];
    load_v8(rv, tile_lo, tid, raw);
    store_v16(sm.v16[0], tid, raw);
    wait_vmem();
    __syncthreads();
  }

  auto step = [&](auto bufc, int tile) {
    constexpr int BUF = decltype(bufc)::value;
    const bool more = tile + 1 < tile_hi;
    u4 raw[2];
    if (more) {
      issue_k8(rk, tile + 1, sm.k8[BUF ^ 1], wave, lane);
      load_v8(rv, tile + 1, tid, raw);
    }
    const GQA_LDS char* kt = sm.k8[BUF];
    const GQA_LDS char* vt = sm.v16[BUF];

#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int k0 = tile * kTileKeys + 32 * kb;
      if (!wave_active || k0 > wpos_hi) continue;  // every key of this block is in the future
      asm volatile("" : "+v"(bk), "+v"(bv));
      f16x sc[1];
      sc[0] = f16x{};
      // all four fragments in flight before the products
      v8i kf[4];
#pragma unroll
      for (int si = 0; si < 4; ++si) kf[si] = read_k8_frag(kt, bk, kb, si);
#pragma unroll
      for (int si = 0; si < 4; ++si) sc[0] = mfma_fp8(kf[si], qf[si], sc[0]);
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      h8 pk[1][2];
      softmax_32keys<1>(sc, acc, m, l, p.c, k0 + 31 > wpos_lo,
                        [&](int, int vv) { return k0 + lane_key(vv, half) <= pos; }, pk);
      pv_32keys<1>(vt, bv, kb, pk, acc);  // O^T += V^T P^T
    }
    if (more) store_v16(sm.v16[BUF ^ 1], tid, raw);
    wait_vmem();
    __syncthreads();
  };

  for (int tile = tile_lo; tile < tile_hi; tile += 2) {
    step(std::integral_constant<int, 0>{}, tile);
    if (tile + 1 < tile_hi) step(std::integral_constant<int, 1>{}, tile + 1);
  }

  const float lt = swap_halves_sum(l[0]);
  if (full) {
    const rsrc_t ro = make_rsrc(p.o, (uint32_t)p.nrows * kRowBytes);
    store_rows_f16(ro, row, half, acc[0], lt, p.post);
  } else {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[0][dt] *= p.post;
    const rsrc_t rp = make_rsrc(p.part, p.part_bytes);
    store_partial(rp, (uint32_t)slot * (uint32_t)(kPartialFloats * 4), kRowsPerBlock, wave * kRowsPerWave + col, half,
                  acc[0], m[0], lt);
  }
}

__global__ __launch_bounds__(512, 1) void prefill_causal_e4m3(PrefillParams p) {
  __shared__ __attribute__((aligned(1024))) char v16a[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char v16b[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char k8a[kTileBytes8];
  __shared__ __attribute__((aligned(1024))) char k8b[kTileBytes8];
  const E4M3Lds sm = {{(GQA_LDS char*)v16a, (GQA_LDS char*)v16b}, {(GQA_LDS char*)k8a, (GQA_LDS char*)k8b}};
  // profiling only, as in prefill_causal_fwd: shader cycles and wall ticks of the workgroup
  const bool stamp = p.clk != nullptr && __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 0;
  unsigned long long c0 = 0, r0 = 0;
  if (stamp) {
    c0 = clock64();
    r0 = wall_clock64();
  }
  prefill_workgroup(p, [&](int b, int lo, int hi, bool full, int slot) {
    prefill_piece_e4m3<8>(p, sm, b, lo, hi, full, slot);
  });
  if (stamp) {
    const unsigned long long dc = clock64() - c0, dr = wall_clock64() - r0;
    if (threadIdx.x == 0) {
      atomicAdd(p.clk, dc);
      atomicAdd(p.clk + 1, dr);
    }
  }
}

// Exact merge of the partials of q-blocks that were split across workgroups:
// M = max_k m_k, O = sum_k 2^(m_k - M) acc_k / sum_k 2^(m_k - M) l_k, and
// lse = (M + log2 sum_k 2^(m_k - M) l_k) ln 2.  Thread (row rl of the slots,
// columns 32 dq .. 32 dq + 31) combines slots slot_lo .. slot_hi into output
// row `orow` of p.o (and p.lse).  Slots are taken in groups of four, then
// two, then one, with every load of a group issued before any of it is summed.
constexpr int kMergeCols = 32;                              // columns per merge thread
constexpr int kMergeThreadsPerRow = kHeadDim / kMergeCols;  // 8
constexpr int kMergeRowsPerWG = 256 / kMergeThreadsPerRow;  // 32

template <int G>
__device__ __forceinline__ void merge_group(rsrc_t rp, int rows, int w0, int rl, int dq, float M, f4 (&o)[8],
                                            float& L) {
  const uint32_t slot_bytes = (uint32_t)(prefill_partial_floats(rows) * 4);
  const uint32_t part_m = (uint32_t)(rows * kHeadDim + rl) * 4, part_l = part_m + rows * 4;
  float mw[G], lw[G];
  u4 x[G][8];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const uint32_t sb = (uint32_t)(w0 + i) * slot_bytes;
    mw[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, sb + part_m, 0, 0));
    lw[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, sb + part_l, 0, 0));
#pragma unroll
    for (int j = 0; j < 8; ++j)
      x[i][j] = __builtin_amdgcn_raw_buffer_load_b128(rp, sb + (uint32_t)(((8 * dq + j) * rows + rl) * 16), 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);  // keep every load of the group ahead of the sums
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const float aw = (mw[i] == -INFINITY) ? 0.f : fast_exp2(mw[i] - M);
    L += aw * lw[i];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] += aw * __builtin_bit_cast(f4, x[i][j]);
  }
}

__device__ __forceinline__ void merge_row(const PrefillParams& p, int slot_lo, int slot_hi, int rl, int dq, int orow) {
  const rsrc_t rp = make_rsrc(p.part, p.part_bytes);
  const int rows = p.qrows;
  const uint32_t slot_bytes = (uint32_t)(prefill_partial_floats(rows) * 4);
  const uint32_t part_m = (uint32_t)(rows * kHeadDim + rl) * 4;
  float M = -INFINITY;
  for (int w0 = slot_lo; w0 <= slot_hi; w0 += 8) {
    float mv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      mv[i] = __uint_as_float(
          __builtin_amdgcn_raw_buffer_load_b32(rp, min(w0 + i, slot_hi) * slot_bytes + part_m, 0, 0));
#pragma unroll
    for (int i = 0; i < 8; ++i) M = fmaxf(M, mv[i]);
  }
  f4 o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = f4{0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  int w0 = slot_lo;
  for (; w0 + 3 <= slot_hi; w0 += 4) merge_group<4>(rp, rows, w0, rl, dq, M, o, L);
  if (w0 + 1 <= slot_hi) {
    merge_group<2>(rp, rows, w0, rl, dq, M, o, L);
    w0 += 2;
  }
  if (w0 <= slot_hi) merge_group<1>(rp, rows, w0, rl, dq, M, o, L);
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  const rsrc_t ro = make_rsrc(p.o, (uint32_t)p.nrows * kRowBytes);
  const uint32_t obase = (uint32_t)orow * kRowBytes + 2 * kMergeCols * dq;
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const h2 a0 = cvt2(o[j][0] * inv, o[j][1] * inv), a1 = cvt2(o[j][2] * inv, o[j][3] * inv);
    const h2 b0 = cvt2(o[j + 1][0] * inv, o[j + 1][1] * inv), b1 = cvt2(o[j + 1][2] * inv, o[j + 1][3] * inv);
    const h8 xx = {a0[0], a0[1], a1[0], a1[1], b0[0], b0[1], b1[0], b1[1]};
    store_16B(ro, obase + j * 8, __builtin_bit_cast(u4, xx));
  }
  if (p.lse != nullptr && dq == 0) {
    const rsrc_t rl_ = make_rsrc(p.lse, (uint32_t)p.nrows * 4);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(row_lse(M, L)), rl_, (uint32_t)orow * 4, 0, 0);
  }
}

// Workgroup (b, part): 32 rows of q-block b; thread (row, 32 columns).
__global__ __launch_bounds__(256) void prefill_merge(PrefillParams p) {
  const int parts = p.qrows / kMergeRowsPerWG;
  const int b = blockIdx.x / parts;
  const int part = blockIdx.x % parts;
  // the pieces of q-block b are slots b*split .. b*split + split - 1 (the
  // merge runs only when split > 1)
  const int tid = threadIdx.x;
  const int rl = part * kMergeRowsPerWG + tid % kMergeRowsPerWG;
  merge_row(p, b * p.split, b * p.split + p.split - 1, rl, tid / kMergeRowsPerWG, b * p.qrows + rl);
}

// ------------------------------------------------------------------ varlen
// A batch of independent sequences packed end to end: sequence i owns query
// tokens cu_q[i] .. cu_q[i+1]-1 and keys cu_kv[i] .. cu_kv[i+1]-1, its queries
// at its last positions.  Its 6 nq_i packed rows are cut into q-blocks of 256
// rows; a one-workgroup prepass writes one descriptor per q-block (the first
// query token and key of its sequence, nq_i, nkv_i, the q-block's index in the
// sequence); descriptors past the last q-block get nq = 0.  A sequence whose
// offsets are out of order or out of range, or that has more queries than
// keys, gets no q-blocks and is counted in the header; its rows are not
// written.  Every q-block is split into `split` key ranges as in the dense
// kernel, and each (q-block, range) workgroup runs the dense 32-row-per-wave
// step on its sequence's slices.
constexpr int kVDescInts = 8;

struct VarlenPrepass {
  const int* cu_q;
  const int* cu_kv;
  int* desc;
  int* hdr;  // [0] q-blocks used, [1] sequences skipped as invalid
  int batch, total_q, total_kv, cap;
};

__global__ __launch_bounds__(256) void prefill_varlen_prepass(VarlenPrepass v) {
  __shared__ int scan[256];
  const int tid = threadIdx.x;
  const rsrc_t rq = make_rsrc(v.cu_q, (uint32_t)(v.batch + 1) * 4);
  const rsrc_t rk = make_rsrc(v.cu_kv, (uint32_t)(v.batch + 1) * 4);
  const rsrc_t rd = make_rsrc(v.desc, (uint32_t)v.cap * kVDescInts * 4);
  int base = 0, bad = 0;
  for (int s0 = 0; s0 < v.batch; s0 += 256) {
    const int i = s0 + tid;
    int cnt = 0, q0 = 0, nq = 0, k0 = 0, nkv = 0;
    if (i < v.batch) {
      q0 = (int)__builtin_amdgcn_raw_buffer_load_b32(rq, i * 4, 0, 0);
      const int q1 = (int)__builtin_amdgcn_raw_buffer_load_b32(rq, (i + 1) * 4, 0, 0);
      k0 = (int)__builtin_amdgcn_raw_buffer_load_b32(rk, i * 4, 0, 0);
      const int k1 = (int)__builtin_amdgcn_raw_buffer_load_b32(rk, (i + 1) * 4, 0, 0);
      nq = q1 - q0;
      nkv = k1 - k0;
      const bool ok = q0 >= 0 && q0 <= q1 && q1 <= v.total_q && k0 >= 0 && k0 <= k1 && k1 <= v.total_kv && nq <= nkv;
      if (ok)
        cnt = (6 * nq + kRowsPerBlock - 1) / kRowsPerBlock;
      else
        bad += 1;
    }
    // inclusive scan of the q-block counts over the 256 threads
    scan[tid] = cnt;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
      const int x = tid >= d ? scan[tid - d] : 0;
      __syncthreads();
      scan[tid] += x;
      __syncthreads();
    }
    const int first = base + scan[tid] - cnt;
    for (int j = 0; j < cnt; ++j) {
      const int e = first + j;
      if (e >= v.cap) break;
      const uint32_t off = (uint32_t)e * kVDescInts * 4;
      __builtin_amdgcn_raw_buffer_store_b32((unsigned)q0, rd, off, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32((unsigned)nq, rd, off + 4, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32((unsigned)k0, rd, off + 8, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32((unsigned)nkv, rd, off + 12, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32((unsigned)j, rd, off + 16, 0, 0);
    }
    base += scan[255];
    __syncthreads();
  }
  const int used = min(base, v.cap);
  for (int e = used + tid; e < v.cap; e += 256)
    __builtin_amdgcn_raw_buffer_store_b32(0u, rd, (uint32_t)e * kVDescInts * 4 + 4, 0, 0);  // nq = 0: unused
  scan[tid] = bad;
  __syncthreads();
  if (tid == 0) {
    int nbad = 0;
    for (int t = 0; t < 256; ++t) nbad += scan[t];
    v.hdr[0] = used;
    v.hdr[1] = nbad;
  }
}

// The dense parameters narrowed to the sequence of varlen q-block qb (false
// when the descriptor is unused).
__device__ __forceinline__ bool varlen_block(const PrefillParams& p, int qb, PrefillParams& s, int& jblk) {
  const int* d = p.vdesc + qb * kVDescInts;
  const int q0 = d[0], nq = d[1], k0 = d[2], nkv = d[3];
  jblk = d[4];
  if (nq <= 0) return false;
  s = p;
  s.q = p.q + (size_t)q0 * kGroup * kHeadDim;
  s.o = p.o + (size_t)q0 * kGroup * kHeadDim;
  s.lse = p.lse != nullptr ? p.lse + (size_t)q0 * kGroup : nullptr;
  s.k = p.k + (size_t)k0 * kHeadDim;
  s.v = p.v + (size_t)k0 * kHeadDim;
  s.nrows = nq * kGroup;
  s.q_pos0 = nkv - nq;
  s.kv_live = nkv;
  return true;
}

__global__ __launch_bounds__(512, 1) void prefill_causal_varlen(PrefillParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[4 * kTileBytes];
  const int qb = blockIdx.x / p.split, j = blockIdx.x % p.split;
  PrefillParams s;
  int jblk;
  if (!varlen_block(p, qb, s, jblk)) return;
  const int nt = prefill_block_tiles(jblk, kRowsPerBlock, s.nrows, s.q_pos0);
  const int lo = (int)((long long)j * nt / p.split), hi = (int)((long long)(j + 1) * nt / p.split);
  if (lo >= hi) {  // a short q-block has fewer tiles than pieces: leave the empty state
    const int tid = threadIdx.x, lane = tid & 63;
    f16x z[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) z[dt] = f16x{};
    store_partial(make_rsrc(p.part, p.part_bytes), (uint32_t)blockIdx.x * (uint32_t)(kPartialFloats * 4),
                  kRowsPerBlock, (tid >> 6) * 32 + (lane & 31), lane >> 5, z, -INFINITY, 0.f);
    return;
  }
  prefill_piece<1, 8>(s, smem, jblk, lo, hi, p.split == 1, blockIdx.x);
}

__global__ __launch_bounds__(256) void prefill_merge_varlen(PrefillParams p) {
  constexpr int kParts = kRowsPerBlock / kMergeRowsPerWG;
  const int qb = blockIdx.x / kParts;
  const int part = blockIdx.x % kParts;
  PrefillParams s;
  int jblk;
  if (!varlen_block(p, qb, s, jblk)) return;
  const int tid = threadIdx.x;
  const int rl = part * kMergeRowsPerWG + tid % kMergeRowsPerWG;
  const int orow = jblk * kRowsPerBlock + rl;
  if (orow >= s.nrows) return;
  merge_row(s, qb * p.split, qb * p.split + p.split - 1, rl, tid / kMergeRowsPerWG, orow);
}

}  // namespace

hipError_t launch_prefill_causal(const void* q, const void* k, const void* v, void* o, int nq, int n_kv, int q_pos0,
                                 int hq, float scale, void* workspace, hipStream_t stream) {
  const PrefillSched s = prefill_schedule(nq, hq, q_pos0);
  PrefillParams p;
  p.q = (const _Float16*)q;
  p.k = (const _Float16*)k;
  p.v = (const _Float16*)v;
  p.o = (_Float16*)o;
  p.part = (float*)workspace;
  p.nrows = s.nrows;
  p.qrows = s.rows;
  p.kv_live = q_pos0 + nq;
  (void)n_kv;
  p.q_pos0 = q_pos0;
  p.nqb = s.nqb;
  p.grid = s.grid;
  p.split = s.split;
  p.part_bytes = (uint32_t)prefill_workspace_bytes(s);
  p.c = scale * kLog2e;
  p.post = 1.0f;
  p.clk = prof_clock();
  p.lse = nullptr;
  p.vdesc = nullptr;
  hipError_t e = s.rows == kRowsSmall
                     ? launch_timed(prefill_causal_fwd<kPrefillC, kSmallW>, dim3(s.grid), dim3(64 * kSmallW), stream, p)
                     : launch_timed(prefill_causal_fwd<kPrefillC, kPrefillW>, dim3(s.grid), dim3(64 * kPrefillW),
                                    stream, p);
  if (e != hipSuccess) return e;
  if (prefill_needs_merge(s)) {
    hipLaunchKernelGGL(prefill_merge, dim3(s.nqb * (s.rows / kMergeRowsPerWG)), dim3(256), 0, stream, p);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_prefill_causal_e4m3(const void* q, float q_scale, const void* k, float k_scale, const void* v,
                                      float v_scale, void* o, int nq, int n_kv, int q_pos0, int hq, float scale,
                                      void* workspace, hipStream_t stream) {
  const PrefillSched s = prefill_schedule_rows(nq, hq, q_pos0, kRowsPerBlock);  // eight waves of 32 rows
  PrefillParams p;
  p.q = (const _Float16*)q;  // E4M3 codes, read as bytes
  p.k = (const _Float16*)k;
  p.v = (const _Float16*)v;
  p.o = (_Float16*)o;
  p.part = (float*)workspace;
  p.nrows = s.nrows;
  p.qrows = s.rows;
  p.kv_live = q_pos0 + nq;
  (void)n_kv;
  p.q_pos0 = q_pos0;
  p.nqb = s.nqb;
  p.grid = s.grid;
  p.split = s.split;
  p.part_bytes = (uint32_t)prefill_workspace_bytes(s);
  p.c = scale * q_scale * k_scale * kLog2e;
  p.post = v_scale;
  p.clk = prof_clock();
  p.lse = nullptr;
  p.vdesc = nullptr;
  hipError_t e = launch_timed(prefill_causal_e4m3, dim3(s.grid), dim3(512), stream, p);
  if (e != hipSuccess) return e;
  if (prefill_needs_merge(s)) {
    hipLaunchKernelGGL(prefill_merge, dim3(s.nqb * (s.rows / kMergeRowsPerWG)), dim3(256), 0, stream, p);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_prefill_causal_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                                        const int32_t* cu_q, const int32_t* cu_kv, int batch, int total_q,
                                        int total_kv, float scale, void* workspace, hipStream_t stream) {
  const VarlenSched vs = prefill_varlen_schedule(batch, total_q);
  char* ws = (char*)workspace;
  VarlenPrepass pre;
  pre.cu_q = cu_q;
  pre.cu_kv = cu_kv;
  pre.hdr = (int*)ws;
  pre.desc = (int*)(ws + kVarlenHeaderBytes);
  pre.batch = batch;
  pre.total_q = total_q;
  pre.total_kv = total_kv;
  pre.cap = vs.cap;
  hipLaunchKernelGGL(prefill_varlen_prepass, dim3(1), dim3(256), 0, stream, pre);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  PrefillParams p;
  p.q = (const _Float16*)q;
  p.k = (const _Float16*)k;
  p.v = (const _Float16*)v;
  p.o = (_Float16*)o;
  p.part = (float*)(ws + varlen_part_offset(vs));
  p.part_bytes = (uint32_t)((size_t)vs.cap * vs.split * kPartialFloats * 4);
  p.nrows = 0;
  p.qrows = kRowsPerBlock;
  p.kv_live = 0;
  p.q_pos0 = 0;
  p.nqb = vs.cap;
  p.grid = vs.cap * vs.split;
  p.split = vs.split;
  p.c = scale * kLog2e;
  p.post = 1.0f;
  p.clk = nullptr;
  p.lse = lse;
  p.vdesc = pre.desc;
  e = launch_timed(prefill_causal_varlen, dim3(p.grid), dim3(512), stream, p);
  if (e != hipSuccess || vs.split == 1) return e;
  hipLaunchKernelGGL(prefill_merge_varlen, dim3(vs.cap * (kRowsPerBlock / kMergeRowsPerWG)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gqa
