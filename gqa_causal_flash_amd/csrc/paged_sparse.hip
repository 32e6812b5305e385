// Paged block-sparse causal GQA prefill for gfx950.
//
// The operation of the block-sparse page ("[Kernel][SM70] Repair #378 on
// latest main", Changes): every 64-token query block attends to its own
// selection of 4-token KV blocks of a page-16 cache reached through a page
// table; selected blocks are fetched in physical-address order, positions at
// or past the live request length are clamped away, and a partial tail block
// contributes only the tokens that exist.  Causal masking applies inside the
// selection.
//
// Three kernels:
//   paged_prepass  one workgroup of 512 threads per query block: bounds-checks
//                  each block id and page, maps block x to its first physical
//                  cache row page_table[x/(P/4)]*P + 4*(x%(P/4)) for pages of P
//                  tokens (P a multiple of 4, so a 4-token block never
//                  straddles a page: 16 and 784 in the pages' geometries),
//                  drops stale, invalid and repeated blocks and packs the rest
//                  in logical order (a bitmap over the table's blocks: the
//                  blocks of a page stay together, the locality the pages ask
//                  of the fetch order).
//   paged_fwd      teams of three workgroups (one per 128-row group of a query
//                  block) over runs of equal cost: gathers 8 blocks (32 keys)
//                  per sub-tile into swizzled double-buffered LDS tiles with
//                  direct-to-LDS loads (each wave's eight copies spread over
//                  the Q K^T products of the sub-tile before), records each
//                  key's logical position,
//                  and runs the shared 32-key step with the mask "position <=
//                  query position".  The padding slots of a query block's
//                  last sub-tile are fetched at an offset past the end of the
//                  cache buffer, so they read as zeros and never bring NaN/Inf
//                  into the products; their position is INT32_MAX, so they
//                  are never visible.
//   paged_merge    combines the pieces of query blocks split between teams.
#include "attn_common.hpp"
#include "attn_tile.hpp"
#include "launch.hpp"
#include "paged_sched.hpp"

#include <type_traits>

namespace gqa {

namespace {

constexpr int kWaves = 4;
constexpr int kPrepassThreads = 512;  // threads of the prepass (one workgroup per query block)
constexpr uint32_t kNoRow = 0xFFFFFFF0u;  // buffer offset past any cache: reads zeros
constexpr int kDeadToken = 0x7FFFFFFF;    // position of a slot that holds nothing live

struct PagedParams {
  const _Float16* q;
  const _Float16* kc;
  const _Float16* vc;
  const int32_t* page_table;
  const int32_t* offsets;
  const int32_t* ids;
  _Float16* o;
  char* ws;
  int n_table, n_pages, page_size, n_ids, nq, nrows, nqb, q_pos0, live_len;
  uint32_t off_err, off_beg, off_cnt, off_nvis, off_entries, off_part;  // the workspace is below 4 GiB
  uint32_t part_bytes;
  float c;
};

// ------------------------------------------------------------------ prepass
constexpr int kHashSlots = 2 * kDedupMax;        // open-addressing table, at most half full
constexpr int kBitmapWords = kBitmapBlocks / 32;  // one bit per logical block of the table
constexpr int kPrepassWaves = kPrepassThreads / 64;

// Exclusive prefix sum of v over the workgroup, and the total.  `wave_tot`
// holds kPrepassWaves ints of LDS.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wave_tot, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kPrepassWaves; ++w) {
    const int t = wave_tot[w];
    before += w < wave ? t : 0;
    total += t;
  }
  return before + incl - v;
}

__global__ __launch_bounds__(kPrepassThreads) void paged_prepass(PagedParams p) {
  // the bitmap path uses bits + word prefixes, the hash path key + lowest index
  __shared__ int lds_a[kBitmapWords];
  __shared__ int lds_b[kBitmapWords];
  static_assert(kHashSlots <= kBitmapWords, "the hash table fits the bitmap arrays");
  __shared__ int small[kDedupMax / 64];
  __shared__ int errs;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const rsrc_t roff = make_rsrc(p.offsets, (uint32_t)(p.nqb + 1) * 4);
  const rsrc_t rids = make_rsrc(p.ids, (uint32_t)p.n_ids * 4);
  const rsrc_t rpt = make_rsrc(p.page_table, (uint32_t)p.n_table * 4);
  int* err = (int*)(p.ws + p.off_err);
  int* beg = (int*)(p.ws + p.off_beg);
  int* cnt = (int*)(p.ws + p.off_cnt);
  int* nvis = (int*)(p.ws + p.off_nvis);
  int2* ent = (int2*)(p.ws + p.off_entries);

  if (tid == 0) errs = 0;
  if (b == 0 && tid == 0) {
    int* hdr = (int*)p.ws;
    hdr[0] = kPagedMagic;
    hdr[1] = p.nqb;
    hdr[2] = p.n_ids;
    hdr[3] = 0;
  }
  const int o0 = (int)__builtin_amdgcn_raw_buffer_load_b32(roff, b * 4, 0, 0);
  const int o1 = (int)__builtin_amdgcn_raw_buffer_load_b32(roff, (b + 1) * 4, 0, 0);
  int start = min(max(o0, 0), p.n_ids);
  int end = min(max(o1, 0), p.n_ids);
  int bad_range = (o0 < 0 || o0 > p.n_ids || o1 < 0 || o1 > p.n_ids || o1 < o0) ? 1 : 0;
  if (end < start) end = start;
  const int n = end - start;
  const int blocks_per_page = p.page_size / kBlockTokens;
  const int n_blocks_table = p.n_table * blocks_per_page;

  // Entry i of this block: valid -> {physical row of its first token, first
  // token}; an id outside the table or a page outside the pool is an error; a
  // block at or past the live length holds nothing and is dropped silently.
  constexpr uint32_t kPastEnd = 0xFFFFFFF0u;  // a buffer offset that reads as 0
  auto load_id = [&](int i) {
    return (int)__builtin_amdgcn_raw_buffer_load_b32(rids, i < n ? (uint32_t)(start + i) * 4 : kPastEnd, 0, 0);
  };
  auto load_page = [&](int i, int x) {
    const bool in_table = i < n && x >= 0 && x < n_blocks_table;
    return (int)__builtin_amdgcn_raw_buffer_load_b32(rpt, in_table ? (uint32_t)(x / blocks_per_page) * 4 : kPastEnd,
                                                     0, 0);
  };
  auto translate = [&](int i, int x, int page, int& bad) -> int2 {
    if (i >= n) return int2{-1, 0};
    if (x < 0 || x >= n_blocks_table) {
      bad += 1;
      return int2{-1, 0};
    }
    const int tok0 = x * kBlockTokens;
    if (tok0 >= p.live_len) return int2{-1, 0};
    if (page < 0 || page >= p.n_pages) {
      bad += 1;
      return int2{-1, 0};
    }
    return int2{page * p.page_size + (x % blocks_per_page) * kBlockTokens, tok0};
  };
  // Selections of up to kDedupMax entries are held in registers (thread t:
  // entries t + 512 r), with the R id loads, then the R page-table loads, in
  // flight together.
  constexpr int R = kDedupMax / kPrepassThreads;
  int xs[R];
  int2 e[R];
  int bad = 0, dups = 0;
  auto load_all = [&]() {
    int pages[R];
#pragma unroll
    for (int r = 0; r < R; ++r) xs[r] = load_id(tid + kPrepassThreads * r);
#pragma unroll
    for (int r = 0; r < R; ++r) pages[r] = load_page(tid + kPrepassThreads * r, xs[r]);
#pragma unroll
    for (int r = 0; r < R; ++r) e[r] = translate(tid + kPrepassThreads * r, xs[r], pages[r], bad);
  };

  if (n_blocks_table <= kBitmapBlocks) {
    // The selection is a set of logical blocks: one bit per block of the
    // table.  A repeated id finds its bit set and is counted; the kept blocks
    // are packed in logical order (block x goes to the number of set bits
    // below x), which keeps the blocks of a page together.  Any length.
    unsigned* bits = (unsigned*)lds_a;
    int* word_before = lds_b;
    const int words = (n_blocks_table + 31) >> 5;
    for (int w = tid; w < words; w += kPrepassThreads) bits[w] = 0u;
    if (n <= kDedupMax) load_all();
    __syncthreads();  // the bitmap is clear
    auto mark = [&](int x, int2 en) {
      if (en.x < 0) return;
      const unsigned bit = 1u << (x & 31);
      if (atomicOr(&bits[x >> 5], bit) & bit) ++dups;
    };
    if (n <= kDedupMax) {
#pragma unroll
      for (int r = 0; r < R; ++r) mark(xs[r], e[r]);
    } else {
      for (int i = tid; i < n; i += kPrepassThreads) {
        const int x = load_id(i);
        mark(x, translate(i, x, load_page(i, x), bad));
      }
    }
    __syncthreads();
    // set bits before each word: thread t counts words t*wpt .. t*wpt+wpt-1
    const int wpt = (words + kPrepassThreads - 1) / kPrepassThreads;
    int c = 0;
    for (int k = 0; k < wpt; ++k) {
      const int w = tid * wpt + k;
      c += w < words ? __popc(bits[w]) : 0;
    }
    int total;
    int run = block_exclusive_scan(c, small, total);
    for (int k = 0; k < wpt; ++k) {
      const int w = tid * wpt + k;
      if (w < words) {
        word_before[w] = run;
        run += __popc(bits[w]);
      }
    }
    __syncthreads();
    // every copy of a block writes the same entry to the same place
    auto place = [&](int x, int2 en) {
      if (en.x < 0) return;
      const int at = word_before[x >> 5] + __popc(bits[x >> 5] & ((1u << (x & 31)) - 1u));
      ent[start + at] = en;
    };
    if (n <= kDedupMax) {
#pragma unroll
      for (int r = 0; r < R; ++r) place(xs[r], e[r]);
    } else {
      int bad2 = 0;  // counted in the first pass
      for (int i = tid; i < n; i += kPrepassThreads) {
        const int x = load_id(i);
        place(x, translate(i, x, load_page(i, x), bad2));
      }
    }
    if (bad + dups) atomicAdd(&errs, bad + dups);
    if (tid == 0) {
      cnt[b] = total;
      beg[b] = start;
      // blocks x < x_thr end at or before the query block's first row:
      // 4x + 3 <= q_pos0 + 64b
      const int first_pos = p.q_pos0 + b * kQBlockTokens;
      const int x_thr = min((first_pos + 1) / kBlockTokens, words * 32);
      const int wi = x_thr >> 5;
      nvis[b] = wi >= words ? total
                            : word_before[wi] + __popc(bits[wi] & ((1u << (x_thr & 31)) - 1u));
    }
  } else if (n <= kDedupMax) {
    // A table too large for the bitmap: repeats are found through an
    // open-addressing table (the copy with the lowest index stays), and the
    // kept entries are packed in the given order.
    int* hkey = lds_a;  // block id held by a slot, -1: empty
    int* hmin = lds_b;  // lowest entry index holding that id
    for (int sl = tid; sl < kHashSlots; sl += kPrepassThreads) {
      hkey[sl] = -1;
      hmin[sl] = 0x7FFFFFFF;
    }
    load_all();
    __syncthreads();  // the table is clear
    int hslot[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      hslot[r] = -1;
      if (e[r].x < 0) continue;
      uint32_t sl = ((uint32_t)xs[r] * 2654435761u) >> (32 - 12);  // Fibonacci hashing into 4096 slots
      static_assert(kHashSlots == 4096, "12-bit hash");
      for (;;) {
        const int prev = atomicCAS(&hkey[sl], -1, xs[r]);
        if (prev == -1 || prev == xs[r]) break;
        sl = (sl + 1) & (kHashSlots - 1);
      }
      atomicMin(&hmin[sl], tid + kPrepassThreads * r);
      hslot[r] = (int)sl;
    }
    __syncthreads();
    bool keep[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      keep[r] = hslot[r] >= 0 && hmin[hslot[r]] == tid + kPrepassThreads * r;
      dups += (hslot[r] >= 0 && !keep[r]) ? 1 : 0;
    }
    // stable compaction: entry i's place is the number of kept entries before
    // it; entries are numbered r-major (t + 512 r), so the count runs over the
    // (r, wave) groups in order, then over the lanes below inside the group
    unsigned long long bal[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      bal[r] = __ballot(keep[r]);
      if (lane == 0) small[r * kPrepassWaves + wave] = __popcll(bal[r]);
    }
    __syncthreads();
    int before_group[R];
    int total = 0;
    for (int gi = 0; gi < R * kPrepassWaves; ++gi) {
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (gi == r * kPrepassWaves + wave) before_group[r] = total;
      total += small[gi];
    }
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (keep[r]) ent[start + before_group[r] + __popcll(bal[r] & below)] = e[r];
    if (bad + dups) atomicAdd(&errs, bad + dups);
    if (tid == 0) {
      cnt[b] = total;
      beg[b] = start;
      nvis[b] = 0;
    }
  } else {
    // a long selection over a table too large for the bitmap: the given order,
    // with an entry that holds nothing live kept in place as {-1, INT32_MAX};
    // a repeated id is not detected
    for (int i = tid; i < n; i += kPrepassThreads) {
      const int x = load_id(i);
      const int2 t = translate(i, x, load_page(i, x), bad);
      ent[start + i] = t.x < 0 ? int2{-1, kDeadToken} : t;
    }
    if (bad) atomicAdd(&errs, bad);
    if (tid == 0) {
      cnt[b] = n;
      beg[b] = start;
      nvis[b] = 0;
    }
  }
  __syncthreads();  // errs complete
  if (tid == 0) err[b] = errs + bad_range;
}

// ------------------------------------------------------------------ attention
constexpr int kSubKeys = 32;                     // keys per sub-tile = 8 blocks
constexpr int kSubBytes = kSubKeys * kRowBytes;  // 16 KiB for K or V
// s_waitcnt vmcnt(0) (other counters untouched) as an instruction the compiler
// sees: its own wait insertion then knows that every load has landed
constexpr int kWaitVmcnt0 = 0x0F70;

// Work positions.  Query block b needs n_b = ceil(cnt[b] / 8) sub-tiles of 32
// keys for each of its three row groups.  A query block with n_b > 0 takes
// w_b = kPagedSwitchUnits + n_b consecutive positions, numbered query block by
// query block from F_b = w_0 + ... + w_(b-1): the first kPagedSwitchUnits
// stand for the cost of starting on it, then sub-tile x sits at position
// base_b + x, base_b = F_b + kPagedSwitchUnits.  The positions are cut into
// equal runs of `per`, and each run goes to a team of three workgroups, one
// per row group, which stream the same sub-tiles at the same pace: the team
// runs on one XCD, so two of the three gathers of every block come from that
// XCD's L2.  Every compute unit gets about the same work whatever the
// selection lengths.  A boundary t * per that would cut fewer than
// kPagedMinPiece sub-tiles off a query block moves to that block's start or
// end (PagedSched::bound), so small query blocks stay whole.  A run covers the
// tail of one query block, whole query blocks and the head of another: whole
// ones are written straight to O, and the (at most two) cut ones leave a
// partial of the row group in the workgroup's slots 2w (its first query block)
// and 2w + 1 (its last), with w = 3 team + g, which paged_merge combines.
__device__ __forceinline__ int paged_nsub(const int* cnt, int b) { return (cnt[b] + 7) >> 3; }
__device__ __forceinline__ int paged_weight(const int* cnt, int b) {
  const int n = paged_nsub(cnt, b);
  return n > 0 ? n + kPagedSwitchUnits : 0;
}

struct PagedRun {
  int per;    // positions per team
  int total;  // all positions
  int teams;  // teams with work
};

// The schedule as one wave sees it.  The weights of query blocks 0..63 are
// read once, one per lane, with their inclusive prefix; later query blocks
// (when there are more than 64) are read as needed, 64 per step.  Every
// result is wave-uniform.
struct PagedSched {
  const int* cnt;
  int nqb, lane;
  int w0, incl0, tot0;  // lane's weight and inclusive prefix in blocks 0..63; their sum
  PagedRun run;

  __device__ __forceinline__ PagedSched(const int* c, int n, int ln) : cnt(c), nqb(n), lane(ln) {
    w0 = lane < nqb ? paged_weight(cnt, lane) : 0;
    incl0 = w0;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl0, d);
      if (lane >= d) incl0 += y;
    }
    tot0 = __builtin_amdgcn_readlane(incl0, 63);
    int t = 0;
    for (int b0 = 64; b0 < nqb; b0 += 64) {
      const int b = b0 + lane;
      t += b < nqb ? paged_weight(cnt, b) : 0;
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) t += __shfl_xor(t, d);
    run.total = tot0 + __builtin_amdgcn_readfirstlane(t);
    // a run shorter than a query block's start cost plus the smallest piece
    // would hold little but that cost, and its team would sit idle
    run.per = max((run.total + kPagedTeams - 1) / kPagedTeams, kPagedSwitchUnits + kPagedMinPiece);
    run.teams = (run.total + run.per - 1) / run.per;
  }

  // sub-tiles of query block b
  __device__ __forceinline__ int nsub(int b) const {
    if (b < 64) {
      const int w = __builtin_amdgcn_readlane(w0, b);
      return w > 0 ? w - kPagedSwitchUnits : 0;
    }
    return __builtin_amdgcn_readfirstlane(paged_nsub(cnt, b));
  }

  // F_b: the positions of the query blocks before b
  __device__ __forceinline__ int first_of(int b) const {
    if (b < 64) return b == 0 ? 0 : __builtin_amdgcn_readlane(incl0, b - 1);
    int t = 0;
    for (int b0 = 64; b0 < b; b0 += 64) {
      const int bb = b0 + lane;
      t += bb < b ? paged_weight(cnt, bb) : 0;
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) t += __shfl_xor(t, d);
    return tot0 + __builtin_amdgcn_readfirstlane(t);
  }

  // The first query block whose positions reach past position u (u < total),
  // and its first position F_b; it always has sub-tiles.
  __device__ __forceinline__ void find(int u, int& qb, int& first) const {
    if (u < tot0) {
      const unsigned long long hit = __ballot(incl0 > u);
      const int l = __builtin_ctzll(hit);
      qb = l;
      first = l == 0 ? 0 : __builtin_amdgcn_readlane(incl0, l - 1);
      return;
    }
    int base = tot0;
    for (int b0 = 64; b0 < nqb; b0 += 64) {
      const int b = b0 + lane;
      const int n = b < nqb ? paged_weight(cnt, b) : 0;
      int incl = n;  // inclusive prefix over the 64 lanes
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d);
        if (lane >= d) incl += y;
      }
      const unsigned long long hit = __ballot(base + incl > u);
      if (hit) {
        const int l = __builtin_ctzll(hit);
        qb = b0 + l;
        first = base + (l == 0 ? 0 : __builtin_amdgcn_readlane(incl, l - 1));
        return;
      }
      base += __builtin_amdgcn_readlane(incl, 63);
    }
    qb = nqb;
    first = base;
  }

  // First position of team t's run (t <= teams; the end of the last run is total).
  __device__ __forceinline__ int bound(int t) const {
    const int u = t * run.per;
    if (u >= run.total) return run.total;
    int b, first;
    find(u, b, first);
    const int n = nsub(b);
    const int before = max(0, u - first - kPagedSwitchUnits);  // sub-tiles of b before u
    if (before < kPagedMinPiece) return first;
    if (n - before < kPagedMinPiece) return first + kPagedSwitchUnits + n;
    return u;
  }
};

// Wave w stages rows 8w .. 8w+7 of a 32-key sub-tile, i.e. entries 2w, 2w+1
// of the sub-tile; copy i covers rows 8w+2i, 8w+2i+1 = tokens 2(i%2), 2(i%2)+1
// of entry 2w + i/2.  The swizzle index of row 8w+2i+h is x = 2j + h with
// j = 4(w%2) + i, which gives the lane offsets kl ^ 32j (K) and
// vl ^ 128(j%4) (V) used by the dense kernel, shifted to the entry's
// physical row.  Lanes 0..7 also record the logical position of row 8w+l.
// The wave's two entries (2w, 2w+1 of the sub-tile) are loaded two sub-tiles
// ahead by sub_entries(), so the gather addresses do not wait on them.
struct SubEntries {
  int2 e[2];
};

// The entries are read through the scalar data cache (constant address
// space, wave-uniform addresses): they land in scalar registers and are counted
// by the scalar-memory counter, so waiting for them never waits for the
// gathers in flight, whose counter is a separate one.
typedef const __attribute__((address_space(4))) int* const_int_ptr;

__device__ __forceinline__ SubEntries sub_entries(const int2* ent, int e0, int e_end, int wave) {
  const const_int_ptr cent = (const_int_ptr)(uintptr_t)ent;
  SubEntries s;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int e = e0 + 2 * wave + k;  // wave-uniform
    if (e < e_end) {
      s.e[k] = int2{cent[2 * e], cent[2 * e + 1]};
    } else {
      s.e[k] = int2{-1, kDeadToken};
    }
  }
  return s;
}

// Copy i (0..7) of the wave's share of a sub-tile: K (i even) or V (i odd)
// rows 8w + 2c, 8w + 2c + 1 with c = i / 2.  With `more` false the copy reads
// zeros (the offset is past the cache), which keeps every copy unconditional.
__device__ __forceinline__ void paged_issue_copy(const PagedParams& p, rsrc_t rk, rsrc_t rv, const SubEntries& se,
                                                 char* kdst, char* vdst, int wave, int lane, uint32_t kl, uint32_t vl,
                                                 int i, bool more) {
  const int half = lane >> 5;
  const int c = i >> 1;
  const int2 en = se.e[c / 2];
  const int u = 2 * (c & 1) + half;
  const bool live = more && en.x >= 0 && en.y + u < p.live_len;
  const uint32_t j = (uint32_t)(4 * (wave & 1) + c);
  const uint32_t base = (uint32_t)(en.x + u) * kRowBytes - (uint32_t)(2 * c + half) * kRowBytes;
  const int r0 = 8 * wave + 2 * c;
  if ((i & 1) == 0) {
    const uint32_t vk = live ? base + (kl ^ (32u * j)) + 1024u * c : kNoRow;
    load_lds_16B(rk, (GQA_LDS char*)(kdst + r0 * kRowBytes), vk, 0);
  } else {
    const uint32_t vv = live ? base + (vl ^ (128u * (j & 3))) + 1024u * c : kNoRow;
    load_lds_16B(rv, (GQA_LDS char*)(vdst + r0 * kRowBytes), vv, 0);
  }
}

// Lanes 0..7 record the logical position of row 8w + l of the sub-tile.
__device__ __forceinline__ void paged_stage_pos(const PagedParams& p, const SubEntries& se, int* kpos, int wave,
                                                int lane) {
  if (lane < 8) {
    const int2 en = lane < 4 ? se.e[0] : se.e[1];
    const int u = lane & 3;
    const bool live = en.x >= 0 && en.y + u < p.live_len;
    kpos[8 * wave + lane] = live ? en.y + u : kDeadToken;
  }
}

__device__ __forceinline__ void paged_issue_sub(const PagedParams& p, rsrc_t rk, rsrc_t rv, const SubEntries& se,
                                                char* kdst, char* vdst, int* kpos, int wave, int lane, uint32_t kl,
                                                uint32_t vl) {
#pragma unroll
  for (int i = 0; i < 8; ++i) paged_issue_copy(p, rk, rv, se, kdst, vdst, wave, lane, kl, vl, i, true);
  paged_stage_pos(p, se, kpos, wave, lane);
}

__global__ __launch_bounds__(256, 2) void paged_fwd(PagedParams p) {
  // two slots (K at 0, V at 16 KiB of a slot's array) and two position
  // arrays, each its own array, and the loop below unrolled over the two
  // slots: every LDS access names its array at compile time, so the compiler
  // can tell that reading one slot does not touch the gather landing in the
  // other, and inserts no wait for that gather
  __shared__ __attribute__((aligned(1024))) char s0a[2 * kSubBytes];
  __shared__ __attribute__((aligned(1024))) char s1a[2 * kSubBytes];
  __shared__ __attribute__((aligned(16))) int kp0s[kSubKeys];
  __shared__ __attribute__((aligned(16))) int kp1s[kSubKeys];
  auto kslot = [&](auto sc) -> char* { return decltype(sc)::value ? s1a : s0a; };
  auto vslot = [&](auto sc) -> char* { return kslot(sc) + kSubBytes; };
  auto pslot = [&](auto sc) -> int* { return decltype(sc)::value ? kp1s : kp0s; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;
  const uint32_t kl = 512u * half + 16u * (uint32_t)(col ^ half);
  const uint32_t vl = 512u * half + ((16u * col) ^ (64u * half));
  const int* cnt = (const int*)(p.ws + p.off_cnt);
  const int* begp = (const int*)(p.ws + p.off_beg);
  const int* nvisp = (const int*)(p.ws + p.off_nvis);
  const int2* ent = (const int2*)(p.ws + p.off_entries);
  const PagedSched sched(cnt, p.nqb, lane);
  const PagedRun& run = sched.run;
  // Workgroup ids are dealt to the 8 XCDs in turn; an XCD's 64 ids hold 21
  // teams of three.  The teams with work are cut into 8 contiguous groups, one
  // per XCD, so that every XCD gets an equal share however few teams there are.
  const int per_xcd = (run.teams + 7) / 8;
  const int xi = blockIdx.x >> 3;
  if (xi >= 3 * per_xcd) return;
  const int team = (blockIdx.x & 7) * per_xcd + xi / 3;
  const int g = xi % 3;  // this workgroup's row group
  const int w = 3 * team + g;
  const int u0 = sched.bound(team);  // the team's positions u0 .. u_end-1
  const int u_end = sched.bound(team + 1);
  if (u0 >= u_end) return;
  int b, first;
  sched.find(u0, b, first);

  const rsrc_t rq = make_rsrc(p.q, (uint32_t)p.nrows * kRowBytes);
  const uint32_t cache_bytes = (uint32_t)p.n_pages * (uint32_t)p.page_size * kRowBytes;
  const rsrc_t rk = make_rsrc(p.kc, cache_bytes);
  const rsrc_t rv = make_rsrc(p.vc, cache_bytes);
  uint32_t bk = k_lane_base(lane);
  uint32_t bv = v_lane_base(lane);

  bool first_seg = true;
  while (b < p.nqb) {
    // the segment: sub-tiles s0 .. s1-1 of row group g of query block b (all
    // wave-uniform: kept in scalar registers)
    const int count = __builtin_amdgcn_readfirstlane(cnt[b]);
    const int nb = (count + 7) >> 3;
    const int base = first + kPagedSwitchUnits;  // position of sub-tile 0
    const int s0 = max(0, u0 - base);
    const int s1 = min(nb, u_end - base);
    if (s1 <= s0) break;  // the run ends before this block's first sub-tile
    const int e_beg = __builtin_amdgcn_readfirstlane(begp[b]);
    const int e_end = e_beg + count;

    const int row_local = 32 * wave + col;  // row inside the 128-row group
    const int row_base = b * kQBlockRows + g * kPagedRowsPerWG + 32 * wave;
    const int row = row_base + col;
    const int pos = p.q_pos0 + min(row, p.nrows - 1) / kGroup;
    const int wpos_lo = p.q_pos0 + min(row_base, p.nrows - 1) / kGroup;  // the wave's first row
    h8 qf[1][16];
    {
      const uint32_t qoff = (uint32_t)row * kRowBytes + half * 16;
#pragma unroll
      for (int s = 0; s < 16; ++s) qf[0][s] = load_16B(rq, qoff + s * 32);
    }
    f16x acc[1][8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[0][dt] = f16x{};
    float m[1] = {-INFINITY}, l[1] = {0.f};

    auto issue = [&](auto sc, const SubEntries& se) {
      paged_issue_sub(p, rk, rv, se, kslot(sc), vslot(sc), pslot(sc), wave, lane, kl, vl);
    };
    // Sub-tile x (i = x - s0) sits in slot i % 2, the gather of x + 1 is in
    // flight while x is computed.  The entries of x are loaded into set i % 2
    // two steps before the step that gathers with them (step x - 1), so a
    // gather never waits for its entries.
    // Sub-tiles before x_mask hold only blocks that every row of the query
    // block sees whole (the entries ascend by token), so they need no mask;
    // the rest (the blocks near the diagonal, a part-filled last sub-tile,
    // entries in the given order) take it, read from the key positions
    // staged with the tile.
    const int x_mask = max(s0, min(s1, __builtin_amdgcn_readfirstlane(nvisp[b]) / (kSubKeys / kBlockTokens)));
    SubEntries es[2];
    es[0] = sub_entries(ent, e_beg + 8 * s0, e_end, wave);
    issue(std::integral_constant<int, 0>{}, es[0]);
    es[1] = sub_entries(ent, e_beg + 8 * (s0 + 1), e_end, wave);
    es[0] = sub_entries(ent, e_beg + 8 * (s0 + 2), e_end, wave);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    lds_barrier();
    auto step = [&](auto ic, int x) {
      constexpr int I = decltype(ic)::value;  // (x - s0) % 2
      const bool mask = x >= x_mask;
      // the gather of x + 1 lands in the other slot: its positions are staged
      // here and its eight copies go out among the Q K^T products
      const bool more = x + 1 < s1;
      const SubEntries nxt = es[I ^ 1];
      if (more) paged_stage_pos(p, nxt, pslot(std::integral_constant<int, I ^ 1>{}), wave, lane);
      es[I ^ 1] = sub_entries(ent, e_beg + 8 * (x + 3), e_end, wave);  // used two steps on
      // keep the per-lane bases opaque so derived addresses are formed here,
      // next to their use, instead of being hoisted and held in registers
      asm volatile("" : "+v"(bk), "+v"(bv));
      const int* kps = pslot(std::integral_constant<int, I>{});
      auto visible = [&](int, int vv) { return kps[8 * (vv >> 2) + 4 * half + (vv & 3)] <= pos; };
      // two K fragments in flight instead of four: the registers go to the
      // schedule state, and no value of the loop is spilled
      attend_32keys_p<1, decltype(visible), 2, 2>((const GQA_LDS char*)kslot(std::integral_constant<int, I>{}), bk,
                                                  (const GQA_LDS char*)vslot(std::integral_constant<int, I>{}), bv, qf,
                                                  acc, m, l, p.c, mask, visible, [&](int i) {
                                                    paged_issue_copy(p, rk, rv, nxt,
                                                                     kslot(std::integral_constant<int, I ^ 1>{}),
                                                                     vslot(std::integral_constant<int, I ^ 1>{}), wave,
                                                                     lane, kl, vl, i, more);
                                                  });
      // the gather into the other slot has landed and every wave is done with
      // this one (a barrier without a memory fence: the wait is explicit)
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      lds_barrier();
    };
    for (int x = s0; x < s1; x += 2) {
      step(std::integral_constant<int, 0>{}, x);
      if (x + 1 < s1) step(std::integral_constant<int, 1>{}, x + 1);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

    const float lt = swap_halves_sum(l[0]);
    if (s0 == 0 && s1 == nb) {
      // rows past the last query row are dropped by the range check
      const rsrc_t ro = make_rsrc(p.o, (uint32_t)p.nrows * kRowBytes);
      store_rows_f16(ro, row, half, acc[0], lt, 1.0f);
    } else {
      const rsrc_t rp = make_rsrc(p.ws + p.off_part, p.part_bytes);
      const int slot = 2 * w + (first_seg ? 0 : 1);
      store_partial(rp, (uint32_t)slot * (uint32_t)(kPagedSlotFloats * 4), kPagedRowsPerWG, row_local, half, acc[0],
                    m[0], lt);
    }
    first_seg = false;
    if (base + s1 >= u_end) break;
    // next query block; those with nothing selected hold no positions
    first = base + nb;
    ++b;
    while (b < p.nqb && __builtin_amdgcn_readfirstlane(cnt[b]) == 0) ++b;
  }
}

// Merge of the cut row groups.  Workgroup (query block b, row group g, row
// half, column half) takes 64 rows x 128 columns; thread (row, 32 columns).
// The sub-tiles of query block b sit at positions base_b .. base_b + n_b - 1;
// the teams t_a .. t_b whose runs hold the first and the last of them cover
// it.  One team means its row groups were written whole; otherwise the
// row-group-g workgroup of team t_a contributes slot 2w + 1 if the sub-tiles
// of an earlier query block fall in its run (the last of them sits at
// F_b - 1), else slot 2w, and that of every later team slot 2w
// (w = 3 team + g).  The
// pieces are combined in one pass with a running maximum (the log-sum-exp
// merge), and the next piece's loads are in flight while one is combined.  A
// query block with nothing selected is written as zeros.
constexpr int kMergeWGsPerRowGroup = 4;  // 2 row halves x 2 column halves

__global__ __launch_bounds__(256) void paged_merge(PagedParams p) {
  const int group = blockIdx.x / kMergeWGsPerRowGroup;  // = b * 3 + g
  const int sub = blockIdx.x % kMergeWGsPerRowGroup;
  const int b = group / kPagedWGsPerQBlock, g = group % kPagedWGsPerQBlock;
  const int lane = threadIdx.x & 63;
  const int rl = (sub & 1) * 64 + lane;                      // row inside the row group
  const int c0 = (sub >> 1) * 128 + 32 * (threadIdx.x >> 6);  // first of the thread's 32 columns
  const int row = group * kPagedRowsPerWG + rl;
  const int* cnt = (const int*)(p.ws + p.off_cnt);
  // the schedule is worked out by the whole wave before any lane leaves
  const PagedSched sched(cnt, p.nqb, lane);
  const PagedRun& run = sched.run;
  const int before = sched.first_of(b);  // F_b
  const int nb = sched.nsub(b);
  // the team whose run holds position q: a boundary moves by less than
  // kPagedSwitchUnits + kPagedMinPiece, which bounds the search
  int bound_found = 0;
  auto team_of = [&](int q) {
    int t = min(run.teams - 1, (q + kPagedSwitchUnits + kPagedMinPiece) / run.per);
    int bt = sched.bound(t);
    while (t > 0 && bt > q) bt = sched.bound(--t);
    bound_found = bt;
    return t;
  };
  const int fr = before + kPagedSwitchUnits;  // position of sub-tile 0
  const int wb = nb > 0 ? team_of(fr + nb - 1) : 0;
  const int wa = nb > 0 ? team_of(fr) : 0;  // its run starts at bound_found
  const bool wa_has_earlier = bound_found < before;
  if (row >= min(p.nrows, (b + 1) * kQBlockRows)) return;
  const rsrc_t ro = make_rsrc(p.o, (uint32_t)p.nrows * kRowBytes);
  const uint32_t obase = (uint32_t)row * kRowBytes + 2 * c0;
  if (nb == 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) store_16B(ro, obase + 16 * q, u4{0u, 0u, 0u, 0u});
    return;
  }
  if (wa == wb) return;
  const rsrc_t rp = make_rsrc(p.ws + p.off_part, p.part_bytes);
  const uint32_t slot_bytes = (uint32_t)(kPagedSlotFloats * 4);
  const uint32_t m_off = (uint32_t)(kPagedRowsPerWG * kHeadDim * 4);
  auto slot_of = [&](int t) { return 2 * (3 * t + g) + (t == wa && wa_has_earlier ? 1 : 0); };
  struct Piece {
    float m, l;
    f4 x[8];
  };
  // the thread's column quads are c0/4 .. c0/4 + 7, each a run of 16-byte rows
  auto load = [&](int t, Piece& pc) {
    const uint32_t sb = (uint32_t)slot_of(t) * slot_bytes;
    pc.m = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, sb + m_off + rl * 4, 0, 0));
    pc.l = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, sb + m_off + (kPagedRowsPerWG + rl) * 4, 0, 0));
#pragma unroll
    for (int q = 0; q < 8; ++q)
      pc.x[q] = __builtin_bit_cast(
          f4, __builtin_amdgcn_raw_buffer_load_b128(rp, sb + (uint32_t)(((c0 / 4 + q) * kPagedRowsPerWG + rl) * 16), 0, 0));
  };
  float M = -INFINITY, L = 0.f;
  f4 o[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) o[q] = f4{0.f, 0.f, 0.f, 0.f};
  auto combine = [&](const Piece& pc) {
    if (pc.m == -INFINITY) return;  // nothing visible in this piece
    const float mn = fmaxf(M, pc.m);
    const float a = (M == -INFINITY) ? 0.f : fast_exp2(M - mn);
    const float e = fast_exp2(pc.m - mn);
    L = a * L + e * pc.l;
#pragma unroll
    for (int q = 0; q < 8; ++q) o[q] = a * o[q] + e * pc.x[q];
    M = mn;
  };
  Piece p0, p1;
  load(wa, p0);
  for (int t = wa; t <= wb; t += 2) {
    if (t + 1 <= wb) load(t + 1, p1);
    combine(p0);
    if (t + 1 > wb) break;
    if (t + 2 <= wb) load(t + 2, p0);
    combine(p1);
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
#pragma unroll
  for (int q = 0; q < 8; q += 2) {
    const h2 a0 = cvt2(o[q][0] * inv, o[q][1] * inv), a1 = cvt2(o[q][2] * inv, o[q][3] * inv);
    const h2 b0 = cvt2(o[q + 1][0] * inv, o[q + 1][1] * inv), b1 = cvt2(o[q + 1][2] * inv, o[q + 1][3] * inv);
    const h8 v = {a0[0], a0[1], a1[0], a1[1], b0[0], b0[1], b1[0], b1[1]};
    store_16B(ro, obase + q * 8, __builtin_bit_cast(u4, v));
  }
}

}  // namespace

hipError_t launch_paged_sparse(const void* q, const void* k_cache, const void* v_cache, const int32_t* page_table,
                               int n_table, int n_pages, int page_size, const int32_t* qblock_offsets,
                               const int32_t* kv_block_ids,
                               int n_block_ids, int nq, int q_pos0, int live_len, int hq, float scale, void* o,
                               void* workspace, hipStream_t stream) {
  PagedParams p;
  p.q = (const _Float16*)q;
  p.kc = (const _Float16*)k_cache;
  p.vc = (const _Float16*)v_cache;
  p.page_table = page_table;
  p.offsets = qblock_offsets;
  p.ids = kv_block_ids;
  p.o = (_Float16*)o;
  p.ws = (char*)workspace;
  p.n_table = n_table;
  p.n_pages = n_pages;
  p.page_size = page_size;
  p.n_ids = n_block_ids;
  p.nq = nq;
  p.nrows = nq * hq;
  p.nqb = (nq + kQBlockTokens - 1) / kQBlockTokens;
  p.q_pos0 = q_pos0;
  p.live_len = live_len;
  const PagedLayout L = paged_layout(p.nqb, n_block_ids);
  p.off_err = (uint32_t)L.err;
  p.off_beg = (uint32_t)L.beg;
  p.off_cnt = (uint32_t)L.cnt;
  p.off_nvis = (uint32_t)L.nvis;
  p.off_entries = (uint32_t)L.entries;
  p.off_part = (uint32_t)L.part;
  p.part_bytes = (uint32_t)(L.total - L.part);
  p.c = scale * kLog2e;
  hipLaunchKernelGGL(paged_prepass, dim3(p.nqb), dim3(kPrepassThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_timed(paged_fwd, dim3(kPagedGrid), dim3(64 * kWaves), stream, p);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(paged_merge, dim3(p.nqb * kPagedWGsPerQBlock * kMergeWGsPerRowGroup), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gqa
