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
//   paged_prepass  one workgroup per query block: bounds-checks each block id
//                  and page, maps block x to its first physical cache row
//                  page_table[x/4]*16 + 4*(x%4) (a 4-token block never
//                  straddles a 16-token page), marks stale and invalid
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

constexpr int kTileBytes = 64 * kRowBytes;  // 32 KiB
constexpr int kWaves = 4;
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
  int n_table, n_pages, n_ids, nq, nrows, nqb, q_pos0, live_len;
  size_t off_err, off_beg, off_cnt, off_entries;
  float c;
};

// ------------------------------------------------------------------ prepass
__global__ __launch_bounds__(256) void paged_prepass(PagedParams p) {
  __shared__ unsigned long long keys[kSortMax];
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
  const int n_blocks_table = p.n_table * (kPageSize / kBlockTokens);

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
    const int page = (int)__builtin_amdgcn_raw_buffer_load_b32(rpt, (uint32_t)(x / (kPageSize / kBlockTokens)) * 4, 0, 0);
    if (page < 0 || page >= p.n_pages) {
      bad = 1;
      return ~0ull;
    }
    const unsigned row = (unsigned)page * kPageSize + (unsigned)(x % (kPageSize / kBlockTokens)) * kBlockTokens;
    return ((unsigned long long)row << 32) | (unsigned)tok0;
  };

  if (n <= kSortMax) {
    int npow = 1;
    while (npow < n) npow <<= 1;
    int bad = 0;
    for (int i = tid; i < npow; i += 256) keys[i] = (i < n) ? translate(i, bad) : ~0ull;
    if (bad) atomicAdd(&errs, bad);
    __syncthreads();
    // bitonic sort, ascending
    for (int k = 2; k <= npow; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < npow; i += 256) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const unsigned long long a = keys[i], c = keys[ixj];
            const bool up = (i & k) == 0;
            if ((a > c) == up) {
              keys[i] = c;
              keys[ixj] = a;
            }
          }
        }
        __syncthreads();
      }
    }
    // drop duplicates (same physical row) and count the valid prefix
    int dup = 0, valid = 0;
    for (int i = tid; i < n; i += 256) {
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
    for (int i = tid; i < n; i += 256) {
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
// Wave w stages rows 16w .. 16w+15 of the 64-key tile (entries 4w .. 4w+3 of
// the tile); copy i covers rows 16w+2i, 16w+2i+1 = tokens 2(i%2), 2(i%2)+1 of
// entry 4w + i/2.  Lanes 0..15 also record the logical position of row 16w+l.
__device__ __forceinline__ void paged_issue_tile(const PagedParams& p, rsrc_t rk, rsrc_t rv, const int2* ent,
                                                 int e0, int e_end, char* kdst, char* vdst, int* kpos, int wave,
                                                 int lane, uint32_t kl, uint32_t vl) {
  const int half = lane >> 5;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int e = e0 + 4 * wave + i / 2;  // wave-uniform
    int2 en = e < e_end ? ent[e] : int2{-1, 0x7FFFFFFF};
    const int u = 2 * (i & 1) + half;
    const bool live = en.x >= 0 && en.y + u < p.live_len;
    // x = row % 16 = 2i + half (wave base 16w is a multiple of 16): swizzles as in the dense kernel
    const uint32_t base = (uint32_t)(en.x + u) * kRowBytes - (uint32_t)(2 * i + half) * kRowBytes;
    const uint32_t vk = live ? base + (kl ^ (32u * i)) + 1024u * i : kNoRow;
    const uint32_t vv = live ? base + (vl ^ (128u * (i & 3))) + 1024u * i : kNoRow;
    const int r0 = 16 * wave + 2 * i;
    load_lds_16B(rk, (GQA_LDS char*)(kdst + r0 * kRowBytes), vk, 0);
    load_lds_16B(rv, (GQA_LDS char*)(vdst + r0 * kRowBytes), vv, 0);
  }
  if (lane < 16) {
    const int e = e0 + 4 * wave + lane / 4;
    const int2 en = e < e_end ? ent[e] : int2{-1, 0x7FFFFFFF};
    const int u = lane & 3;
    const bool live = en.x >= 0 && en.y + u < p.live_len;
    kpos[16 * wave + lane] = live ? en.y + u : 0x7FFFFFFF;
  }
}

__global__ __launch_bounds__(256, 1) void paged_fwd(PagedParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[4 * kTileBytes];
  __shared__ __attribute__((aligned(16))) int kpos_s[2][64];
  const int b = blockIdx.x / kPagedWGsPerQBlock;
  const int g = blockIdx.x % kPagedWGsPerQBlock;
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
  const int ntiles = (n + 15) / 16;

  const rsrc_t rq = make_rsrc(p.q, (uint32_t)p.nrows * kRowBytes);
  const uint32_t cache_bytes = (uint32_t)p.n_pages * kPageSize * kRowBytes;
  const rsrc_t rk = make_rsrc(p.kc, cache_bytes);
  const rsrc_t rv = make_rsrc(p.vc, cache_bytes);

  const int row = b * kQBlockRows + g * kPagedRowsPerWG + 32 * wave + col;
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

  if (ntiles > 0) {
    paged_issue_tile(p, rk, rv, ent, e_beg, e_end, smem + 2 * kTileBytes, smem, kpos_s[0], wave, lane, kl, vl);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  auto step = [&](auto bufc, int t) {
    constexpr int BUF = decltype(bufc)::value;
    if (t + 1 < ntiles)
      paged_issue_tile(p, rk, rv, ent, e_beg + 16 * (t + 1), e_end, smem + (2 + (BUF ^ 1)) * kTileBytes,
                       smem + (BUF ^ 1) * kTileBytes, kpos_s[BUF ^ 1], wave, lane, kl, vl);
    const GQA_LDS char* kt = (const GQA_LDS char*)smem + (2 + BUF) * kTileBytes;
    const GQA_LDS char* vt = (const GQA_LDS char*)smem + BUF * kTileBytes;
    const int keys_here = min(64, 4 * (n - 16 * t));
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (32 * kb >= keys_here) continue;
      asm volatile("" : "+v"(bk), "+v"(bv));
      // logical positions of this lane's 16 keys: runs of 4 at 32kb + 8j + 4*half
      int kp[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int4 x = *(const int4*)&kpos_s[BUF][32 * kb + 8 * j + 4 * half];
        kp[4 * j] = x.x;
        kp[4 * j + 1] = x.y;
        kp[4 * j + 2] = x.z;
        kp[4 * j + 3] = x.w;
      }
      attend_32keys<1>(lds_addr(kt) + bk, vt, bv, kb, qf, acc, m, l, p.c, true, [&](int, int vv) { return kp[vv] <= pos; });
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  for (int t = 0; t < ntiles; t += 2) {
    step(std::integral_constant<int, 0>{}, t);
    if (t + 1 < ntiles) step(std::integral_constant<int, 1>{}, t + 1);
  }

  const float lt = swap_halves_sum(l[0]);
  // rows of this workgroup that belong to the next query block (a short last
  // block) or lie past the end are not written
  const int row_end = min(p.nrows, (b + 1) * kQBlockRows);
  const rsrc_t ro = make_rsrc(p.o, (uint32_t)row_end * kRowBytes);
  store_rows_f16(ro, row, half, acc[0], lt, 1.0f);
}

}  // namespace

hipError_t launch_paged_sparse(const void* q, const void* k_cache, const void* v_cache, const int32_t* page_table,
                               int n_table, int n_pages, const int32_t* qblock_offsets, const int32_t* kv_block_ids,
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
  p.c = scale * kLog2e;
  hipLaunchKernelGGL(paged_prepass, dim3(p.nqb), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_before(stream);
  hipLaunchKernelGGL(paged_fwd, dim3(p.nqb * kPagedWGsPerQBlock), dim3(64 * kWaves), 0, stream, p);
  e = hipGetLastError();
  prof_after(stream);
  return e;
}

}  // namespace gqa
