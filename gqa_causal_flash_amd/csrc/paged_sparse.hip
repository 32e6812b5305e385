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
  int pieces;
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

__device__ __forceinline__ SubEntries sub_entries(const int2* ent, int e0, int e_end, int wave) {
  SubEntries s;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int e = e0 + 2 * wave + k;  // wave-uniform
    const int2 x = e < e_end ? ent[e] : int2{-1, 0x7FFFFFFF};
    // uniform values: kept in scalar registers
    s.e[k] = int2{__builtin_amdgcn_readfirstlane(x.x), __builtin_amdgcn_readfirstlane(x.y)};
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

// Workgroup id -> (query block, row group, piece).  Ids u with the same u % 8
// run on the same XCD, so every workgroup of one query block is given the same
// u % 8 and its gathered K/V rows are shared through that XCD's L2.
__device__ __forceinline__ bool paged_unit(int u, int nqb, int pieces, int& b, int& g, int& j) {
  const int per_block = kPagedWGsPerQBlock * pieces;
  const int x = u & 7, rest = u >> 3;
  b = (rest / per_block) * 8 + x;
  const int within = rest % per_block;
  g = within / pieces;
  j = within % pieces;
  return b < nqb;
}

__global__ __launch_bounds__(256, 2) void paged_fwd(PagedParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[4 * kSubBytes];  // V 0/16 KiB, K 32/48 KiB
  __shared__ __attribute__((aligned(16))) int kpos_s[2][kSubKeys];
  int b, g, pj;
  if (!paged_unit(blockIdx.x, p.nqb, p.pieces, b, g, pj)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;
  const uint32_t kl = 512u * half + 16u * (uint32_t)(col ^ half);
  const uint32_t vl = 512u * half + ((16u * col) ^ (64u * half));

  const int* cntp = (const int*)(p.ws + p.off_cnt);
  const int* begp = (const int*)(p.ws + p.off_beg);
  const int2* ent = (const int2*)(p.ws + p.off_entries);
  const int n = cntp[b];
  const int e_beg = begp[b];
  const int e_end = e_beg + n;
  const int n_sub = (n + 7) / 8;
  const int s_lo = (int)((long long)pj * n_sub / p.pieces);
  const int s_hi = (int)((long long)(pj + 1) * n_sub / p.pieces);

  const rsrc_t rq = make_rsrc(p.q, (uint32_t)p.nrows * kRowBytes);
  const uint32_t cache_bytes = (uint32_t)p.n_pages * (uint32_t)p.page_size * kRowBytes;
  const rsrc_t rk = make_rsrc(p.kc, cache_bytes);
  const rsrc_t rv = make_rsrc(p.vc, cache_bytes);

  const int row_local = 32 * wave + col;  // row inside the 128-row group
  const int row = b * kQBlockRows + g * kPagedRowsPerWG + row_local;
  const int pos = p.q_pos0 + min(row, p.nrows - 1) / kGroup;
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
  uint32_t bk = k_lane_base(lane);
  uint32_t bv = v_lane_base(lane);

  auto issue = [&](int x, const SubEntries& se) {
    const int buf = x & 1;
    paged_issue_sub(p, rk, rv, se, smem + (2 + buf) * kSubBytes, smem + buf * kSubBytes, kpos_s[buf], wave, lane, kl,
                    vl);
  };
  SubEntries nxt = sub_entries(ent, e_beg + 8 * s_lo, e_end, wave);
  if (s_lo < s_hi) issue(s_lo, nxt);
  nxt = sub_entries(ent, e_beg + 8 * (s_lo + 1), e_end, wave);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int x = s_lo; x < s_hi; ++x) {
    const int buf = (x - s_lo) & 1;
    if (x + 1 < s_hi) issue(x + 1, nxt);  // lands in the other slot
    nxt = sub_entries(ent, e_beg + 8 * (x + 2), e_end, wave);  // in flight during this sub-tile
    asm volatile("" : "+v"(bk), "+v"(bv));
    int kp[16];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int4 v4 = *(const int4*)&kpos_s[(x & 1)][8 * q4 + 4 * half];
      kp[4 * q4] = v4.x;
      kp[4 * q4 + 1] = v4.y;
      kp[4 * q4 + 2] = v4.z;
      kp[4 * q4 + 3] = v4.w;
    }
    (void)buf;
    attend_32keys<1>(lds_addr((const GQA_LDS char*)smem + (2 + (x & 1)) * kSubBytes) + bk,
                     (const GQA_LDS char*)smem + (x & 1) * kSubBytes, bv, 0, qf, acc, m, l, p.c, true,
                     [&](int, int vv) { return kp[vv] <= pos; });
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  const float lt = swap_halves_sum(l[0]);
  if (p.pieces == 1) {
    // rows of a short last query block that fall past the end are not written
    const int row_end = min(p.nrows, (b + 1) * kQBlockRows);
    const rsrc_t ro = make_rsrc(p.o, (uint32_t)row_end * kRowBytes);
    store_rows_f16(ro, row, half, acc[0], lt, 1.0f);
  } else {
    const rsrc_t rp = make_rsrc(p.ws + p.off_part, p.part_bytes);
    const int slot = ((b * kPagedWGsPerQBlock) + g) * p.pieces + pj;
    store_partial(rp, (uint32_t)slot * (uint32_t)(kPagedSlotFloats * 4), kPagedRowsPerWG, row_local, half, acc[0],
                  m[0], lt);
  }
}

// Merge of the pieces of each 128-row group: workgroup (group, half) takes 64
// rows; thread (row, 64 columns).
__global__ __launch_bounds__(256) void paged_merge(PagedParams p) {
  const int group = blockIdx.x >> 1;  // = b * 3 + g
  const int rl = (blockIdx.x & 1) * 64 + (threadIdx.x & 63);
  const int dq = threadIdx.x >> 6;
  const int row = group * kPagedRowsPerWG + rl;
  const int b = group / kPagedWGsPerQBlock;
  if (row >= min(p.nrows, (b + 1) * kQBlockRows)) return;
  const rsrc_t rp = make_rsrc(p.ws + p.off_part, p.part_bytes);
  const uint32_t slot_bytes = (uint32_t)(kPagedSlotFloats * 4);
  const uint32_t m_off = (uint32_t)(kPagedRowsPerWG * kHeadDim * 4);
  float M = -INFINITY;
  for (int j = 0; j < p.pieces; ++j) {
    const uint32_t sb = (uint32_t)(group * p.pieces + j) * slot_bytes;
    M = fmaxf(M, __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, sb + m_off + rl * 4, 0, 0)));
  }
  f4 o[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) o[q] = f4{0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  for (int j = 0; j < p.pieces; ++j) {
    const uint32_t sb = (uint32_t)(group * p.pieces + j) * slot_bytes;
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
  const rsrc_t ro = make_rsrc(p.o, (uint32_t)p.nrows * kRowBytes);
  const uint32_t obase = (uint32_t)row * kRowBytes + 128 * dq;
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
  p.pieces = L.pieces;
  p.c = scale * kLog2e;
  hipLaunchKernelGGL(paged_prepass, dim3(p.nqb), dim3(kPrepassThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // ids are grouped by XCD (see paged_unit): round the query blocks up to a multiple of 8
  const int units = ((p.nqb + 7) / 8) * 8 * kPagedWGsPerQBlock * p.pieces;
  prof_before(stream);
  hipLaunchKernelGGL(paged_fwd, dim3(units), dim3(64 * kWaves), 0, stream, p);
  e = hipGetLastError();
  prof_after(stream);
  if (e != hipSuccess || p.pieces == 1) return e;
  hipLaunchKernelGGL(paged_merge, dim3(p.nqb * kPagedWGsPerQBlock * 2), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gqa
