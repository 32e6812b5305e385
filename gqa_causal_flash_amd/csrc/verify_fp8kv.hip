// FP8 (OCP E4M3) KV verifier tail for gfx950.
//
// The operation of the long-context page ("[Perf] Ship the qualified SM70
// long-context layout...", What and Changes): a speculative-decoding verifier
// step of 2..8 query rows (x 6 grouped heads) attends causally to a K/V cache
// of up to 262144 tokens stored as E4M3 bytes, with fp32 accumulation.  The
// page decodes E4M3 through a shared-memory lookup table because its GPU has
// no FP8 unit; gfx950 converts in hardware (v_cvt_scalef32_pk_f16_fp8), and
// every E4M3 value is exact in fp16, so the decoded fragments feed the same
// fp16 matrix-core step as the dense kernel.  The per-tensor K scale is folded
// into the softmax scale and the V scale into the final normalisation.
//
// The work is bound by HBM bandwidth (K + V = 512 B per key), so the key range
// is split evenly over two workgroups per compute unit.  A workgroup streams
// its keys in 32-key tiles of raw bytes through a ring of five LDS slots with
// direct HBM -> LDS loads, three tiles in flight.  It has two waves per
// 32-row block of packed query rows (one block for q = 1..5, the single-row
// tail included; two for q = 6..8): the two waves of a block take alternate
// tiles and combine their states before the workgroup writes its partial.
// The bytes are decoded to fp16 in registers, right where the matrix cores
// take them:
//   K fragments (S^T = K Q^T, A operand) by an 8-byte LDS read per lane;
//     the head-dimension order of the product is permuted so that lane half h
//     covers columns 128h .. 128h+127 (Q is loaded in the same order);
//   V^T fragments (O^T += V^T P^T, A operand) by the transposing read
//     ds_read_b64_tr_b8, which hands each lane eight consecutive keys of one
//     head-dimension column.
// Each workgroup writes one online-softmax partial; a second kernel merges the
// partials by log-sum-exp.
#include "attn_common.hpp"
#include "attn_tile.hpp"
#include "launch.hpp"
#include "verify_sched.hpp"

#include <atomic>
#include <mutex>
#include <type_traits>

namespace gqa {

namespace {

constexpr int kVTileKeys = 32;
constexpr int kFp8Row = kHeadDim;                     // bytes per E4M3 row
constexpr int kRawTile = kVTileKeys * kFp8Row;        // 8 KiB of K or V bytes
constexpr int kRing = 5;                              // LDS slots of K + V raw tiles
constexpr int kSlotBytes = 2 * kRawTile;              // 16 KiB: K at 0, V at 8 KiB

struct VerifyParams {
  const _Float16* q;
  const uint8_t* k;
  const uint8_t* v;
  _Float16* o;
  float* part;
  int nq, nrows, n_kv, ntiles, grid;
  uint32_t part_bytes;
  float c;        // scale * k_scale * log2(e)
  float v_scale;
};

// Raw tile layout in LDS: row r of a tile (256 bytes = 16 chunks of 16 B)
// keeps logical chunk c at physical chunk c ^ swz(r), with swz = r % 16 for K
// and 2 ((r % 4) + 4 ((r / 8) % 2)) for V, so that the fragment reads below
// spread over the banks (the eight V rows one transposing read takes differ
// in bits 0, 1 and 3).
__device__ __forceinline__ uint32_t k_swz(int r) { return (uint32_t)(r & 15); }
__device__ __forceinline__ uint32_t v_swz(int r) { return 2u * (uint32_t)((r & 3) | (((r >> 3) & 1) << 2)); }

typedef int v2i __attribute__((ext_vector_type(2)));

// 8 E4M3 bytes -> 8 fp16 values (exact), in byte order.
__device__ __forceinline__ h8 decode8(v2i raw) {
  const h2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)raw[0], 1.0f, false);
  const h2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)raw[0], 1.0f, true);
  const h2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)raw[1], 1.0f, false);
  const h2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)raw[1], 1.0f, true);
  return h8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// The ring slots are separate LDS arrays, and the loop is unrolled over the
// ring so that every slot index is a compile-time constant: the compiler can
// then see that the fragment reads of one slot do not touch the slots that
// loads are in flight into, and inserts no wait for those loads (it would if
// all slots lived in one array).  Completion is waited for explicitly.
struct RawRing {
  char* s[kRing];
};

// RB row blocks of 32 packed rows (RB = 1 for at most 32 rows, 2 for up to
// 64).  Wave w holds row block w % RB and takes the tiles of parity w / RB:
// the two waves of a row block compute alternate tiles, each keeping its own
// online-softmax state, and combine before the workgroup writes its partial.
// Every wave stages 16 / (2 RB) of the 16 KiB-pieces of each tile (K pieces
// first, then V).  At two workgroups per compute unit, RB = 2 puts two waves
// on every SIMD, so one wave's decode and softmax overlap the other's matrix
// products.
template <int RB>
__global__ __launch_bounds__(128 * RB, 2) void verify_fwd(VerifyParams p) {
  constexpr int kWaves = 2 * RB;
  constexpr int kLoads = 16 / kWaves;  // 1 KiB loads per tile and wave
  __shared__ __attribute__((aligned(1024))) char r0[kSlotBytes];
  __shared__ __attribute__((aligned(1024))) char r1[kSlotBytes];
  __shared__ __attribute__((aligned(1024))) char r2[kSlotBytes];
  __shared__ __attribute__((aligned(1024))) char r3[kSlotBytes];
  __shared__ __attribute__((aligned(1024))) char r4[kSlotBytes];
  static_assert(kRing == 5, "one array per slot");
  const RawRing ring = {{r0, r1, r2, r3, r4}};
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rb = wave % RB;  // row block
  const int par = wave / RB;  // tile parity
  const int half = lane >> 5;
  const int col = lane & 31;

  const int t_lo = (int)((long long)blockIdx.x * p.ntiles / p.grid);
  const int t_hi = (int)((long long)(blockIdx.x + 1) * p.ntiles / p.grid);
  const int n = t_hi - t_lo;  // >= 1

  // this wave's loads: 1 KiB pieces i = i0 .. i0 + kLoads - 1 of K (i < 8) or
  // V (i >= 8), piece i holding raw rows 4(i%8) .. 4(i%8)+3; lane l takes row
  // 4(i%8) + l/16 and physical chunk l % 16 (logical chunk (l % 16) ^ swz)
  const int i0 = wave * kLoads;
  const bool stage_v = i0 >= 8;
  const rsrc_t rkv = make_rsrc(stage_v ? (const void*)p.v : (const void*)p.k, (uint32_t)p.n_kv * kFp8Row);
  uint32_t loff[kLoads];
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const int r = 4 * ((i0 + j) & 7) + (lane >> 4);
    const uint32_t swz = stage_v ? v_swz(r) : k_swz(r);
    loff[j] = (uint32_t)r * kFp8Row + 16u * ((uint32_t)(lane & 15) ^ swz);
  }
  const uint32_t ldst = (stage_v ? kRawTile : 0) + 1024u * (uint32_t)(i0 & 7);
  const uint32_t kv_bytes = (uint32_t)p.n_kv * kFp8Row;
  auto issue = [&](char* slot, int t) {  // this wave's pieces of tile t into a slot
    GQA_LDS char* dst = (GQA_LDS char*)slot + ldst;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) load_lds_16B(rkv, dst + j * 1024, loff[j], (uint32_t)t * kRawTile);
  };

  const int row = 32 * rb + col;
  const int pos = (p.n_kv - p.nq) + min(row, p.nrows - 1) / kGroup;
  const int pos_min = p.n_kv - p.nq;  // first query position
  // Q as B fragments in the permuted column order: step s, lane half h holds
  // columns 128h + 8s .. 128h + 8s + 7 (rows past the last read as zeros)
  h8 qf[1][16];
  {
    const rsrc_t rq = make_rsrc(p.q, (uint32_t)p.nrows * kRowBytes);
    const uint32_t qoff = (uint32_t)row * kRowBytes + 256u * half;
#pragma unroll
    for (int s = 0; s < 16; ++s) qf[0][s] = load_16B(rq, qoff + 16u * s);
  }
  f16x acc[1][8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) acc[0][dt] = f16x{};
  float m[1] = {-INFINITY}, l[1] = {0.f};

  // K fragment s of lane (key r = col, half h): bytes 128h + 8s .. +7 of row r,
  // logical chunk 8h + s/2, byte 8 (s % 2)
  uint32_t kbase = (uint32_t)col * kFp8Row;
  // V^T fragment (dt, key half t): the product's key order is that of P^T as
  // it leaves the score registers: element e of lane half h is key
  // 16t + 8(e/4) + 4h + e%4.  ds_read_b64_tr_b8 gives output lane i, element e
  // byte i of the 16 bytes that source lanes 2e and 2e+1 of its 16-lane group
  // address, so source lane k of group g (half h = g/2) addresses key
  // 16t + 8(k/8) + 4h + (k/2)%4 at columns 32dt + 16(g%2) + 8(k%2), i.e.
  // logical chunk 2dt + g%2, byte 8(k%2).
  const int g = lane >> 4, sk = lane & 15;
  const int vrow0 = 8 * (sk >> 3) + 4 * (g >> 1) + ((sk >> 1) & 3);  // + 16t
  const uint32_t vswz = v_swz(vrow0);                                 // (16t keeps the swizzle)
  uint32_t vbase = (uint32_t)vrow0 * kFp8Row + 8u * (sk & 1);

  // one 32-key tile t from the raw K bytes at kt (V bytes follow)
  auto compute = [&](const GQA_LDS char* kt, int t, auto hook) {
    const GQA_LDS char* vt = kt + kRawTile;
    const int k0 = t * kVTileKeys;
    asm volatile("" : "+v"(kbase), "+v"(vbase));
    // S^T = K Q^T
    f16x s1[1];
    s1[0] = f16x{};
#pragma unroll
    for (int si = 0; si < 16; ++si) {
      const uint32_t ch = (uint32_t)(8 * half + (si >> 1)) ^ k_swz(col);
      const v2i raw = *(const GQA_LDS v2i*)(kt + kbase + 16u * ch + 8u * (si & 1));
      s1[0] = mfma(decode8(raw), qf[0][si], s1[0]);
      hook(si);
    }
    h8 pk[1][2];
    softmax_32keys<1>(s1, acc, m, l, p.c, k0 + 31 > pos_min,
                      [&](int, int vv) { return k0 + lane_key(vv, half) <= pos; }, pk);
    // O^T += V^T P^T
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const int dt = st >> 1, tt = st & 1;
      const uint32_t ch = (uint32_t)(2 * dt + (g & 1)) ^ vswz;
      const v2i raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (GQA_LDS v2i*)(vt + vbase + (uint32_t)(16 * tt) * kFp8Row + 16u * ch));
      acc[0][dt] = mfma(decode8(raw), pk[0][tt], acc[0][dt]);
    }
  };

  // Tile j of the range sits in ring slot j % kRing; step s computes tiles 2s
  // (parity 0) and 2s + 1 (parity 1).  Three tiles are issued up front; step
  // s waits for tiles 2s and 2s + 1 with tile 2s + 2 still in flight, then
  // issues tiles 2s + 3 and 2s + 4 into the slots of tiles 2s - 2 and 2s - 1,
  // which every wave finished in step s - 1.  Those copies go out spread over
  // the Q K^T products of the step's own tile, not in one burst (each copy
  // sets M0, which keeps them in issue order for the counted waits).
#pragma unroll
  for (int j = 0; j < 3; ++j)
    if (j < n) issue(ring.s[j], t_lo + j);
  // the loop is written once per parity and unrolled over the ring, so that
  // every slot a wave reads is a compile-time choice (the compiler then knows
  // the reads miss the slots being loaded)
  auto run = [&](auto parc) {
    constexpr int PAR = decltype(parc)::value;
    auto step = [&](auto sc, int st) {
      constexpr int S = decltype(sc)::value;  // st % kRing
      if (2 * st + 2 < n) {  // tile 2s + 2 may stay in flight
        if constexpr (kLoads == 8)
          asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        else
          asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      lds_barrier();
      // a tile past the range reads from a resource of no bytes: nothing is
      // fetched, and the idle slot it names fills with zeros
      const rsrc_t r3 = make_rsrc(stage_v ? (const void*)p.v : (const void*)p.k, 2 * st + 3 < n ? kv_bytes : 0u);
      const rsrc_t r4 = make_rsrc(stage_v ? (const void*)p.v : (const void*)p.k, 2 * st + 4 < n ? kv_bytes : 0u);
      GQA_LDS char* d3 = (GQA_LDS char*)ring.s[(2 * S + 3) % kRing] + ldst;
      GQA_LDS char* d4 = (GQA_LDS char*)ring.s[(2 * S + 4) % kRing] + ldst;
      const uint32_t o3 = (uint32_t)(t_lo + 2 * st + 3) * kRawTile, o4 = o3 + kRawTile;
      auto one = [&](int q) {
        if (q < kLoads)
          load_lds_16B(r3, d3 + q * 1024, loff[q], o3);
        else
          load_lds_16B(r4, d4 + (q - kLoads) * 1024, loff[q - kLoads], o4);
      };
      if (2 * st + PAR < n) {
        compute((const GQA_LDS char*)ring.s[(2 * S + PAR) % kRing], t_lo + 2 * st + PAR, [&](int si) {
          if constexpr (2 * kLoads >= 16) {
#pragma unroll
            for (int q = si * (2 * kLoads / 16); q < (si + 1) * (2 * kLoads / 16); ++q) one(q);
          } else {
            if (si % (16 / (2 * kLoads)) == 0) one(si / (16 / (2 * kLoads)));
          }
        });
      } else {
#pragma unroll
        for (int q = 0; q < 2 * kLoads; ++q) one(q);
      }
    };
    for (int st = 0; 2 * st < n; st += kRing) {
      step(std::integral_constant<int, 0>{}, st);
      if (2 * st + 2 >= n) break;
      step(std::integral_constant<int, 1>{}, st + 1);
      if (2 * st + 4 >= n) break;
      step(std::integral_constant<int, 2>{}, st + 2);
      if (2 * st + 6 >= n) break;
      step(std::integral_constant<int, 3>{}, st + 3);
      if (2 * st + 8 >= n) break;
      step(std::integral_constant<int, 4>{}, st + 4);
    }
  };
  if (par == 0)
    run(std::integral_constant<int, 0>{});
  else
    run(std::integral_constant<int, 1>{});

  // The parity-1 wave of each row block hands its state to the parity-0 wave
  // through LDS (the ring is idle now): both hold the same rows in the same
  // lanes, so the parity-0 wave combines register by register,
  // O = 2^(m1-M) O1 + 2^(m2-M) O2 and likewise l.  Accumulator j of row block
  // b sits in ring slot 2b + j / 64 at float (j % 64) * 64 + lane; m and l in
  // slot 4 at float (2b + {0, 1}) * 64 + lane.
  float lt = swap_halves_sum(l[0]);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no copy is still landing in the ring
  lds_barrier();  // every wave is done with the ring
  auto hand = [&](auto rbc, bool write) {
    constexpr int B = decltype(rbc)::value;
    auto xa = [&](int j) -> GQA_LDS float& { return ((GQA_LDS float*)ring.s[2 * B + (j >> 6)])[(j & 63) * 64 + lane]; };
    GQA_LDS float* xm = (GQA_LDS float*)ring.s[4] + 2 * B * 64 + lane;
    if (write) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) xa(16 * dt + v) = acc[0][dt][v];
      xm[0] = m[0];
      xm[64] = lt;
      return;
    }
    const float m2 = xm[0], l2 = xm[64];
    const float mm = fmaxf(m[0], m2);
    const float a1 = (m[0] == -INFINITY) ? 0.f : fast_exp2(m[0] - mm);
    const float a2 = (m2 == -INFINITY) ? 0.f : fast_exp2(m2 - mm);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[0][dt][v] = a1 * acc[0][dt][v] + a2 * xa(16 * dt + v);
    m[0] = mm;
    lt = a1 * lt + a2 * l2;
  };
  auto hand_rb = [&](bool write) {
    if (RB == 1 || rb == 0)
      hand(std::integral_constant<int, 0>{}, write);
    else
      hand(std::integral_constant<int, 1>{}, write);
  };
  if (par == 1) hand_rb(true);
  lds_barrier();
  if (par == 1) return;
  hand_rb(false);
  if (row < p.nrows) {
    // partial slot, row-major: acc[64 rows][256 columns], then m[64], l[64];
    // register 4g .. 4g+3 of tile dt holds columns 32dt + 8g + 4h .. +3
    const rsrc_t rp = make_rsrc(p.part, p.part_bytes);
    const uint32_t sb = (uint32_t)blockIdx.x * (uint32_t)(kVerifySlotFloats * 4);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f4 x = {acc[0][dt][4 * g4], acc[0][dt][4 * g4 + 1], acc[0][dt][4 * g4 + 2], acc[0][dt][4 * g4 + 3]};
        store_16B(rp, sb + (uint32_t)(row * kHeadDim + 32 * dt + 8 * g4 + 4 * half) * 4, __builtin_bit_cast(u4, x));
      }
    if (half == 0) {
      const uint32_t mo = sb + (uint32_t)(kVerifySlotRows * kHeadDim * 4);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m[0]), rp, mo + row * 4, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lt), rp, mo + (kVerifySlotRows + row) * 4, 0, 0);
    }
  }
}

// Merge of the workgroups' partials: workgroup (r, part) combines row r,
// columns 64 part .. 64 part + 63.  Thread (quad, sl) takes columns
// 64 part + 4 quad .. +3 of slots sl, sl + 32, ... (all its loads in flight
// together; the 16 quads of one slot read 256 contiguous bytes), then the
// maximum of m and the sums of 2^(m_s - M) acc_s and 2^(m_s - M) l_s are
// taken over the 32 slot lanes through LDS.
constexpr int kMergeLanes = 32;
constexpr int kMergeSlots = kVerifyMaxGrid / kMergeLanes;  // slots per thread

__global__ __launch_bounds__(16 * kMergeLanes) void verify_merge(VerifyParams p) {
  __shared__ float red[kMergeLanes][16][5];
  __shared__ float rmax[kMergeLanes];
  const int r = blockIdx.x >> 2, part = blockIdx.x & 3;
  const int tid = threadIdx.x, quad = tid & 15, sl = tid >> 4;
  const rsrc_t rp = make_rsrc(p.part, p.part_bytes);
  const uint32_t slot_bytes = (uint32_t)(kVerifySlotFloats * 4);
  const uint32_t m_off = (uint32_t)(kVerifySlotRows * kHeadDim * 4);
  const uint32_t xoff = (uint32_t)(r * kHeadDim + 64 * part + 4 * quad) * 4;
  float ms[kMergeSlots], ls[kMergeSlots];
  f4 xs[kMergeSlots];
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < kMergeSlots; ++i) {
    const int s = sl + kMergeLanes * i;
    const uint32_t sb = (uint32_t)s * slot_bytes;  // past the workspace for s >= grid: reads as zero
    const bool ok = s < p.grid;
    ms[i] = ok ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, sb + m_off + r * 4, 0, 0)) : -INFINITY;
    ls[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, sb + m_off + (kVerifySlotRows + r) * 4, 0, 0));
    xs[i] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rp, sb + xoff, 0, 0));
    M = fmaxf(M, ms[i]);
  }
  if (quad == 0) rmax[sl] = M;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kMergeLanes; ++i) M = fmaxf(M, rmax[i]);
  f4 o = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
#pragma unroll
  for (int i = 0; i < kMergeSlots; ++i) {
    const float a = (ms[i] == -INFINITY) ? 0.f : fast_exp2(ms[i] - M);
    o += a * xs[i];
    L += a * ls[i];
  }
  red[sl][quad][0] = L;
  red[sl][quad][1] = o[0];
  red[sl][quad][2] = o[1];
  red[sl][quad][3] = o[2];
  red[sl][quad][4] = o[3];
  __syncthreads();
  if (sl == 0) {
    f4 t = {0.f, 0.f, 0.f, 0.f};
    float lt = 0.f;
#pragma unroll
    for (int i = 0; i < kMergeLanes; ++i) {
      lt += red[i][quad][0];
      t[0] += red[i][quad][1];
      t[1] += red[i][quad][2];
      t[2] += red[i][quad][3];
      t[3] += red[i][quad][4];
    }
    const float inv = lt > 0.f ? p.v_scale / lt : 0.f;
    const h2 lo = cvt2(t[0] * inv, t[1] * inv), hi = cvt2(t[2] * inv, t[3] * inv);
    const rsrc_t ro = make_rsrc(p.o, (uint32_t)p.nrows * kRowBytes);
    store_8B(ro, (uint32_t)r * kRowBytes + (16 * part + quad) * 8, h4{lo[0], lo[1], hi[0], hi[1]});
  }
}

}  // namespace

hipError_t launch_verify_fp8kv(const void* q, const uint8_t* k, const uint8_t* v, float k_scale, float v_scale,
                               void* o, int nq, int n_kv, int hq, float scale, void* workspace, hipStream_t stream) {
  const VerifySched s = verify_schedule(nq, n_kv, hq);
  VerifyParams p;
  p.q = (const _Float16*)q;
  p.k = k;
  p.v = v;
  p.o = (_Float16*)o;
  p.part = (float*)workspace;
  p.nq = nq;
  p.nrows = nq * hq;
  p.n_kv = n_kv;
  p.ntiles = s.ntiles;
  p.grid = s.grid;
  p.part_bytes = (uint32_t)verify_workspace_bytes(s);
  p.c = scale * k_scale * kLog2e;
  p.v_scale = v_scale;
  hipError_t e = s.row_blocks == 1 ? launch_timed(verify_fwd<1>, dim3(s.grid), dim3(128), stream, p)
                                    : launch_timed(verify_fwd<2>, dim3(s.grid), dim3(256), stream, p);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(verify_merge, dim3(p.nrows * 4), dim3(16 * kMergeLanes), 0, stream, p);
  return hipGetLastError();
}

// Scratch of gqa_verify_fp8kv_noalloc, for callers that cannot allocate: room
// for the partial slots of the largest verifier schedule (512 slots of 64
// rows).  Every device the library runs on holds its own copy from module load
// until the process ends, and every such call on that device shares it.  The
// forward kernel writes every slot row the merge reads, so nothing in it has
// to start at zero.
static __device__ __align__(256) unsigned char scratch[kVerifyScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
}  // namespace

// Device address of the current device's copy of `scratch`, looked up once per
// device (the name itself is only a host-side stand-in for the symbol).
hipError_t verify_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace gqa
