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
// Two kernels:
//   paged_prepass  one workgroup of 512 threads per query block: bounds-checks each block id
//                  and page, maps block x to its first physical cache row
//                  page_table[x/(P/4)]*P + 4*(x%(P/4)) for pages of P tokens
//                  (P a multiple of 4, so a 4-token block never straddles a
//                  page: 16 and 784 in the pages' geometries), marks stale and invalid
//                  blocks, sorts the list by physical row and drops
//                  duplicates.
//   paged_fwd      three workgroups per query block (128 packed rows each):
//                  gathers 16 blocks (64 keys) per tile into the swizzled
//                  double-buffered LDS tiles with direct-to-LDS loads (a
//                  2 KiB contiguous block is two 1 KiB copies), records each
//                  key's logical position, and runs the shared 32-key step
//                  with the mask "position <= query position".  Slots of
//                  stale or invalid entries are fetched at an offset past the
//                  end of the cache buffer, so they read as zeros and never
//                  bring NaN/Inf into the products; their position is
//                  INT32_MAX, so they are never visible.
#include "attn_common.hpp"
#include "attn_tile.hpp"
#include "launch.hpp"
#include "paged_sched.hpp"

#include <type_traits>

namespace gqa {

namespace {

constexpr int kWaves = 4;
constexpr int kPrepassThreads = 512;  // sort lanes of the prepass (one workgroup per query block)
constexpr uint32_t kNoRow = 0xFFFFFFF0u;  // buffer offset past any cache: reads zeros

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
  size_t off_err, off_beg, off_cnt, off_entries, off_part;
  uint32_t part_bytes;
  float c;
};

// ------------------------------------------------------------------ prepass
__global__ __launch_bounds__(kPrepassThreads) void paged_prepass(PagedParams p) {
  __shared__ unsigned long long keys[kSortMax];
  __shared__ unsigned long long keys2[kSortMax];
  __shared__ int errs;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const rsrc_t roff = make_rsrc(p.offsets, (uint32_t)(p.nqb + 1) * 4);
  const rsrc_t rids = make_rsrc(p.ids, (uint32_t)p.n_ids * 4);
  const rsrc_t rpt = make_rsrc(p.page_table, (uint32_t)p.n_table * 4);
  int* err = (int*)(p.ws + p.off_err);
  int* beg = (int*)(p.ws + p.off_beg);
  int* cnt = (int*)(p.ws + p.off_cnt);
  int2* ent = (int2*)(p.ws + p.off_entries);

  if (tid == 0) errs = 0;
  if (b == 0 && tid == 0) {
    int* hdr = (int*)p.ws;
    hdr[0] = kPagedMagic;
    hdr[1] = p.nqb;
    hdr[2] = p.n_ids;
    hdr[3] = 0;
  }
  __syncthreads();
  const int o0 = (int)__builtin_amdgcn_raw_buffer_load_b32(roff, b * 4, 0, 0);
  const int o1 = (int)__builtin_amdgcn_raw_buffer_load_b32(roff, (b + 1) * 4, 0, 0);
  int start = min(max(o0, 0), p.n_ids);
  int end = min(max(o1, 0), p.n_ids);
  int bad_range = (o0 < 0 || o0 > p.n_ids || o1 < 0 || o1 > p.n_ids || o1 < o0) ? 1 : 0;
  if (end < start) end = start;
  const int n = end - start;
  const int blocks_per_page = p.page_size / kBlockTokens;
  const int n_blocks_table = p.n_table * blocks_per_page;

  // Translate entry i of this block: valid -> (physical row << 32 | token),
  // otherwise all ones (sorts last).
  auto translate = [&](int i, int& bad) -> unsigned long long {
    const int x = (int)__builtin_amdgcn_raw_buffer_load_b32(rids, (uint32_t)(start + i) * 4, 0, 0);
    if (x < 0 || x >= n_blocks_table) {
      bad = 1;
      return ~0ull;
    }
    const int tok0 = x * kBlockTokens;
    if (tok0 >= p.live_len) return ~0ull;  // stale block: not an error, just nothing live
    const int page = (int)__builtin_amdgcn_raw_buffer_load_b32(rpt, (uint32_t)(x / blocks_per_page) * 4, 0, 0);
    if (page < 0 || page >= p.n_pages) {
      bad = 1;
      return ~0ull;
    }
    const unsigned row = (unsigned)page * (unsigned)p.page_size + (unsigned)(x % blocks_per_page) * kBlockTokens;
    return ((unsigned long long)row << 32) | (unsigned)tok0;
  };

  if (n <= kSortMax) {
    int npow = 1;
    while (npow < n) npow <<= 1;
    int bad = 0;
    // Bitonic sort, ascending, with the keys in registers: thread t holds
    // elements t + 512 r (r < kSortMax / 512).  A compare-exchange at distance
    // j pairs lanes of one wave when j < 64 (register shuffle, no barrier), a
    // thread with itself when j >= 512, and otherwise goes through LDS (two
    // buffers, one barrier per such stage).
    constexpr int R = kSortMax / kPrepassThreads;
    unsigned long long kv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int i = tid + kPrepassThreads * r;
      kv[r] = (i < n) ? translate(i, bad) : ~0ull;
    }
    if (bad) atomicAdd(&errs, bad);
    const int rmax = (npow + kPrepassThreads - 1) / kPrepassThreads;  // register slots in use
    // The stages are written for a compile-time count of slots in use, so
    // that a stage issues the exchanges of all its slots before it waits.
    auto sort_slots = [&](auto rmc) {
      constexpr int RM = decltype(rmc)::value;
      int buf = 0;
      for (int k = 2; k <= npow; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
          if (j >= kPrepassThreads) {
            const int rj = j / kPrepassThreads;
#pragma unroll
            for (int r = 0; r < RM; ++r) {
              const int rp = r ^ rj;
              const int i = tid + kPrepassThreads * r;
              if (rp > r && rp < RM) {
                const bool up = (i & k) == 0;
                const unsigned long long a = kv[r], c = kv[rp];
                if ((a > c) == up) {
                  kv[r] = c;
                  kv[rp] = a;
                }
              }
            }
          } else {
            unsigned long long c[RM];
            if (j < 64) {
#pragma unroll
              for (int r = 0; r < RM; ++r) c[r] = __shfl_xor(kv[r], j);
            } else {
              unsigned long long* kb = buf ? keys2 : keys;
#pragma unroll
              for (int r = 0; r < RM; ++r) kb[tid + kPrepassThreads * r] = kv[r];
              __syncthreads();
#pragma unroll
              for (int r = 0; r < RM; ++r) c[r] = kb[(tid + kPrepassThreads * r) ^ j];
              buf ^= 1;
            }
#pragma unroll
            for (int r = 0; r < RM; ++r) {
              const int i = tid + kPrepassThreads * r;
              const unsigned long long a = kv[r];
              const bool up = (i & k) == 0;
              const bool lo = (i & j) == 0;  // the lower index of the pair keeps the smaller key when ascending
              kv[r] = (lo == up) ? (a < c[r] ? a : c[r]) : (a < c[r] ? c[r] : a);
            }
          }
        }
      }
    };
    static_assert(R == 4, "slot counts 1, 2 and 4");
    if (rmax <= 1)
      sort_slots(std::integral_constant<int, 1>{});
    else if (rmax == 2)
      sort_slots(std::integral_constant<int, 2>{});
    else
      sort_slots(std::integral_constant<int, 4>{});
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r < rmax) keys[tid + kPrepassThreads * r] = kv[r];
    __syncthreads();
    // drop duplicates (same physical row) and count the valid prefix
    int dup = 0, valid = 0;
    for (int i = tid; i < n; i += kPrepassThreads) {
      unsigned long long kv = keys[i];
      if (kv != ~0ull && i > 0 && (keys[i - 1] >> 32) == (kv >> 32)) {
        kv = ~0ull;
        dup = 1;
      }
      if (kv != ~0ull) valid = i + 1;
      ent[start + i] = (kv == ~0ull) ? int2{-1, 0x7FFFFFFF} : int2{(int)(kv >> 32), (int)(kv & 0xFFFFFFFFu)};
    }
    if (dup) atomicAdd(&errs, 1);
    __shared__ int vmax;
    if (tid == 0) vmax = 0;
    __syncthreads();
    if (valid) atomicMax(&vmax, valid);
    __syncthreads();
    if (tid == 0) {
      cnt[b] = vmax;
      beg[b] = start;
      err[b] = errs + bad_range;
    }
  } else {
    // too long to sort in LDS: keep the given order (it is only a locality choice)
    int bad = 0;
    for (int i = tid; i < n; i += kPrepassThreads) {
      const unsigned long long kv = translate(i, bad);
      ent[start + i] = (kv == ~0ull) ? int2{-1, 0x7FFFFFFF} : int2{(int)(kv >> 32), (int)(kv & 0xFFFFFFFFu)};
    }
    if (bad) atomicAdd(&errs, bad);
    __syncthreads();
    if (tid == 0) {
      cnt[b] = n;
      beg[b] = start;
      err[b] = errs + bad_range;
    }
  }
}

// ------------------------------------------------------------------ attention
constexpr int kSubKeys = 32;                     // keys per sub-tile = 8 blocks
constexpr int kSubBytes = kSubKeys * kRowBytes;  // 16 KiB for K or V
constexpr int kDeadToken = 0x7FFFFFFF;           // token of an entry that holds nothing live
// s_waitcnt vmcnt(0) (other counters untouched) as an instruction the compiler
// sees: its own wait insertion then knows that every load has landed
constexpr int kWaitVmcnt0 = 0x0F70;

// Work units.  Query block b needs n_b = ceil(cnt[b] / 8) sub-tiles of 32
// keys for each of its three row groups.  Column unit (b, x) is sub-tile x of
// query block b, numbered query block by query block; the C column units are
// cut into equal runs of `per` consecutive units, and each run goes to a team
// of three workgroups, one per row group, which stream the same sub-tiles at
// the same pace: the team runs on one XCD, so two of the three gathers of
// every block come from that XCD's L2.  Every compute unit gets the same work
// whatever the selection lengths.  A run covers the tail of one query block,
// whole query blocks and the head of another: whole ones are written straight
// to O, and the (at most two) cut ones leave a partial of the row group in the
// workgroup's slots 2w (its first query block) and 2w + 1 (its last), with
// w = 3 team + g, which paged_merge combines.
__device__ __forceinline__ int paged_nsub(const int* cnt, int b) { return (cnt[b] + 7) >> 3; }

struct PagedRun {
  int per;     // column units per team
  int total;   // all column units
  int teams;   // teams with work
};

// Sum over query blocks, computed by each wave on its own (64 query blocks per step).
__device__ __forceinline__ PagedRun paged_run(const int* cnt, int nqb, int lane) {
  int t = 0;
  for (int b0 = 0; b0 < nqb; b0 += 64) {
    const int b = b0 + lane;
    t += b < nqb ? paged_nsub(cnt, b) : 0;
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) t += __shfl_xor(t, d);
  PagedRun r;
  r.total = __builtin_amdgcn_readfirstlane(t);
  r.per = max((r.total + kPagedTeams - 1) / kPagedTeams, 2);
  r.teams = (r.total + r.per - 1) / r.per;
  return r;
}

// The query block holding column unit u and its first unit (u < total).
__device__ __forceinline__ void paged_find(const int* cnt, int nqb, int lane, int u, int& qb, int& first) {
  int base = 0;
  for (int b0 = 0; b0 < nqb; b0 += 64) {
    const int b = b0 + lane;
    const int n = b < nqb ? paged_nsub(cnt, b) : 0;
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
      first = __builtin_amdgcn_readfirstlane(base + __shfl(incl - n, l));
      return;
    }
    base = __builtin_amdgcn_readfirstlane(base + __shfl(incl, 63));
  }
  qb = nqb;
  first = base;
}

// Wave w stages rows 8w .. 8w+7 of a 32-key sub-tile, i.e. entries 2w, 2w+1
// of the sub-tile; copy i covers rows 8w+2i, 8w+2i+1 = tokens 2(i%2), 2(i%2)+1
// of entry 2w + i/2.  The swizzle index of row 8w+2i+h is x = 2j + h with
// j = 4(w%2) + i, which gives the lane offsets kl ^ 32j (K) and
// vl ^ 128(j%4) (V) used by the dense kernel, shifted to the entry's
// physical row.  Lanes 0..7 also record the logical position of row 8w+l.
// The wave's two entries (2w, 2w+1 of the sub-tile) are loaded a sub-tile
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
      s.e[k] = int2{-1, 0x7FFFFFFF};
    }
  }
  return s;
}

__device__ __forceinline__ void paged_issue_sub(const PagedParams& p, rsrc_t rk, rsrc_t rv, const SubEntries& se,
                                                char* kdst, char* vdst, int* kpos, int wave, int lane, uint32_t kl,
                                                uint32_t vl) {
  const int half = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int2 en = se.e[i / 2];
    const int u = 2 * (i & 1) + half;
    const bool live = en.x >= 0 && en.y + u < p.live_len;
    const uint32_t j = (uint32_t)(4 * (wave & 1) + i);
    const uint32_t base = (uint32_t)(en.x + u) * kRowBytes - (uint32_t)(2 * i + half) * kRowBytes;
    const uint32_t vk = live ? base + (kl ^ (32u * j)) + 1024u * i : kNoRow;
    const uint32_t vv = live ? base + (vl ^ (128u * (j & 3))) + 1024u * i : kNoRow;
    const int r0 = 8 * wave + 2 * i;
    load_lds_16B(rk, (GQA_LDS char*)(kdst + r0 * kRowBytes), vk, 0);
    load_lds_16B(rv, (GQA_LDS char*)(vdst + r0 * kRowBytes), vv, 0);
  }
  if (lane < 8) {
    const int2 en = lane < 4 ? se.e[0] : se.e[1];
    const int u = lane & 3;
    const bool live = en.x >= 0 && en.y + u < p.live_len;
    kpos[8 * wave + lane] = live ? en.y + u : 0x7FFFFFFF;
  }
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
  const int2* ent = (const int2*)(p.ws + p.off_entries);
  const PagedRun run = paged_run(cnt, p.nqb, lane);
  // Workgroup ids are dealt to the 8 XCDs in turn; an XCD's 64 ids hold 21
  // teams of three.  The teams with work are cut into 8 contiguous groups, one
  // per XCD, so that every XCD gets an equal share however few teams there are.
  const int per_xcd = (run.teams + 7) / 8;
  const int xi = blockIdx.x >> 3;
  if (xi >= 3 * per_xcd) return;
  const int team = (blockIdx.x & 7) * per_xcd + xi / 3;
  const int g = xi % 3;  // this workgroup's row group
  const int w = 3 * team + g;
  int u = team * run.per;
  const int u_end = min(run.total, u + run.per);
  if (u >= u_end) return;
  int b, first;
  paged_find(cnt, p.nqb, lane, u, b, first);

  const rsrc_t rq = make_rsrc(p.q, (uint32_t)p.nrows * kRowBytes);
  const uint32_t cache_bytes = (uint32_t)p.n_pages * (uint32_t)p.page_size * kRowBytes;
  const rsrc_t rk = make_rsrc(p.kc, cache_bytes);
  const rsrc_t rv = make_rsrc(p.vc, cache_bytes);
  uint32_t bk = k_lane_base(lane);
  uint32_t bv = v_lane_base(lane);

  bool first_seg = true;
  while (u < u_end) {
    // the segment: sub-tiles s0 .. s1-1 of row group g of query block b (all
    // wave-uniform: kept in scalar registers)
    const int count = __builtin_amdgcn_readfirstlane(cnt[b]);
    const int nb = (count + 7) >> 3;
    const int s0 = u - first;
    const int s1 = min(nb, s0 + (u_end - u));
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
    SubEntries es[2];
    es[0] = sub_entries(ent, e_beg + 8 * s0, e_end, wave);
    issue(std::integral_constant<int, 0>{}, es[0]);
    es[1] = sub_entries(ent, e_beg + 8 * (s0 + 1), e_end, wave);
    es[0] = sub_entries(ent, e_beg + 8 * (s0 + 2), e_end, wave);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    lds_barrier();
    auto step = [&](auto ic, int x) {
      constexpr int I = decltype(ic)::value;  // (x - s0) % 2
      if (x + 1 < s1) issue(std::integral_constant<int, I ^ 1>{}, es[I ^ 1]);  // lands in the other slot
      es[I ^ 1] = sub_entries(ent, e_beg + 8 * (x + 3), e_end, wave);          // used two steps on
      // keep the per-lane bases opaque so derived addresses are formed here,
      // next to their use, instead of being hoisted and held in registers
      asm volatile("" : "+v"(bk), "+v"(bv));
      const int* kps = pslot(std::integral_constant<int, I>{});
      // a sub-tile whose keys all sit at or before the wave's first row (the
      // usual case: selections lie mostly far behind the query block) needs no
      // mask; dead and stale slots carry INT32_MAX and force one.  Positions of
      // this lane's keys: 4 runs of 4 at 8q + 4h.
      int kmax = -1;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int4 v4 = *(const int4*)&kps[8 * q4 + 4 * half];
        kmax = max(kmax, max(max(v4.x, v4.y), max(v4.z, v4.w)));
      }
      const bool mask = !__all(kmax <= wpos_lo);
      auto visible = [&](int, int vv) { return kps[8 * (vv >> 2) + 4 * half + (vv & 3)] <= pos; };
      // two K fragments in flight instead of four: the registers go to the
      // schedule state, and no value of the loop is spilled
      attend_32keys_p<1, decltype(visible), 2, 2>((const GQA_LDS char*)kslot(std::integral_constant<int, I>{}), bk,
                                                  (const GQA_LDS char*)vslot(std::integral_constant<int, I>{}), bv, qf,
                                                  acc, m, l, p.c, mask, visible);
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
    u += s1 - s0;
    if (u >= u_end) break;
    // next query block; those with nothing selected hold no units
    first += nb;
    ++b;
    while (b < p.nqb && __builtin_amdgcn_readfirstlane(cnt[b]) == 0) ++b;
  }
}

// Merge of the cut row groups: workgroup (row group, half) takes 64 rows;
// thread (row, 64 columns).  Query block b holds column units first_b ..
// first_b + n_b - 1; the teams t_a = first_b / per .. t_b = (first_b + n_b - 1)
// / per cover it.  One team means its row groups were written whole;
// otherwise the row-group-g workgroup of team t_a contributes slot 2w (if b is
// its first query block) or 2w + 1, and that of every later team slot 2w
// (w = 3 team + g).  A query block with nothing selected is written as zeros.
__global__ __launch_bounds__(256) void paged_merge(PagedParams p) {
  const int group = blockIdx.x >> 1;  // = b * 3 + g
  const int b = group / kPagedWGsPerQBlock, g = group % kPagedWGsPerQBlock;
  const int rl = (blockIdx.x & 1) * 64 + (threadIdx.x & 63);
  const int dq = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int row = group * kPagedRowsPerWG + rl;
  const int* cnt = (const int*)(p.ws + p.off_cnt);
  const PagedRun run = paged_run(cnt, p.nqb, lane);
  // first column unit of query block b: the sum over the blocks before it
  int before = 0;
  for (int b0 = 0; b0 < b; b0 += 64) {
    const int bb = b0 + lane;
    before += bb < b ? paged_nsub(cnt, bb) : 0;
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) before += __shfl_xor(before, d);
  if (row >= min(p.nrows, (b + 1) * kQBlockRows)) return;
  const int nb = paged_nsub(cnt, b);
  const rsrc_t ro = make_rsrc(p.o, (uint32_t)p.nrows * kRowBytes);
  const uint32_t obase = (uint32_t)row * kRowBytes + 128 * dq;
  if (nb == 0) {
#pragma unroll
    for (int q = 0; q < 16; q += 2) store_16B(ro, obase + q * 8, u4{0u, 0u, 0u, 0u});
    return;
  }
  const int fr = before;
  const int wa = fr / run.per, wb = (fr + nb - 1) / run.per;  // teams
  if (wa == wb) return;
  const rsrc_t rp = make_rsrc(p.ws + p.off_part, p.part_bytes);
  const uint32_t slot_bytes = (uint32_t)(kPagedSlotFloats * 4);
  const uint32_t m_off = (uint32_t)(kPagedRowsPerWG * kHeadDim * 4);
  auto slot_of = [&](int t) { return 2 * (3 * t + g) + (t == wa && t * run.per != fr ? 1 : 0); };
  float M = -INFINITY;
  for (int wi = wa; wi <= wb; ++wi) {
    const uint32_t sb = (uint32_t)slot_of(wi) * slot_bytes;
    M = fmaxf(M, __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, sb + m_off + rl * 4, 0, 0)));
  }
  f4 o[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) o[q] = f4{0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  for (int wi = wa; wi <= wb; ++wi) {
    const uint32_t sb = (uint32_t)slot_of(wi) * slot_bytes;
    const float mj = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, sb + m_off + rl * 4, 0, 0));
    const float lj =
        __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, sb + m_off + (kPagedRowsPerWG + rl) * 4, 0, 0));
    const float a = (mj == -INFINITY) ? 0.f : fast_exp2(mj - M);
    L += a * lj;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const u4 x =
          __builtin_amdgcn_raw_buffer_load_b128(rp, sb + (uint32_t)(((16 * dq + q) * kPagedRowsPerWG + rl) * 16), 0, 0);
      o[q] += a * __builtin_bit_cast(f4, x);
    }
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
#pragma unroll
  for (int q = 0; q < 16; q += 2) {
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
  p.off_err = L.err;
  p.off_beg = L.beg;
  p.off_cnt = L.cnt;
  p.off_entries = L.entries;
  p.off_part = L.part;
  p.part_bytes = (uint32_t)(L.total - L.part);
  p.c = scale * kLog2e;
  hipLaunchKernelGGL(paged_prepass, dim3(p.nqb), dim3(kPrepassThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_before(stream);
  hipLaunchKernelGGL(paged_fwd, dim3(kPagedGrid), dim3(64 * kWaves), 0, stream, p);
  e = hipGetLastError();
  prof_after(stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(paged_merge, dim3(p.nqb * kPagedWGsPerQBlock * 2), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gqa
