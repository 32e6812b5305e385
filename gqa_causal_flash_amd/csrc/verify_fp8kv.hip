// FP8 (OCP E4M3) KV verifier tail for gfx950.
//
// The operation of the long-context page ("[Perf] Ship the qualified SM70
// long-context layout...", What and Changes): a speculative-decoding verifier
// step of 2..8 query rows (x 6 grouped heads) attends causally to a K/V cache
// of up to 262144 tokens stored as E4M3 bytes, with fp32 accumulation.  The
// page decodes E4M3 through a shared-memory lookup table because its GPU has
// no FP8 unit; gfx950 converts in hardware (v_cvt_scalef32_pk_f16_fp8), and
// every E4M3 value is exact in fp16, so the decoded tiles feed the same fp16
// matrix-core step as the dense kernel.  The per-tensor K scale is folded into
// the softmax scale and the V scale into the final normalisation.
//
// The work is bound by HBM bandwidth (K + V = 512 B per key), so the key range
// is split over every compute unit: each workgroup runs two independent key
// streams of two waves (one per 32-row block of the <= 48 packed query rows);
// a stream prefetches the raw bytes of its next 32-key tile into registers
// while it decodes and attends the current one.  The two streams of a
// workgroup are merged in LDS and written as one online-softmax partial; a
// second kernel merges the workgroups' partials by log-sum-exp.
#include "attn_common.hpp"
#include "attn_tile.hpp"
#include "launch.hpp"
#include "verify_sched.hpp"

namespace gqa {

namespace {

constexpr int kVTileKeys = 32;
constexpr int kVTileBytes = kVTileKeys * kRowBytes;  // fp16 tile: 16 KiB
constexpr int kFp8Row = kHeadDim;                    // bytes per E4M3 row

struct VerifyParams {
  const _Float16* q;
  const uint8_t* k;
  const uint8_t* v;
  _Float16* o;
  float* part;
  int nq, nrows, n_kv, ntiles, nstreams, grid;
  uint32_t part_bytes;
  float c;        // scale * k_scale * log2(e)
  float v_scale;
};

// Decode 16 E4M3 bytes (one 16-byte chunk: head-dim columns 16cb .. 16cb+15 of
// a row) into two fp16 chunks and store them at their swizzled LDS places.
__device__ __forceinline__ void decode_store(u4 raw, GQA_LDS char* row_base, int cb, int phys0, int phys1) {
  h8 lo, hi;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const h2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[w], 1.0f, false);
    const h2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[w], 1.0f, true);
    h8& dst = (w < 2) ? lo : hi;
    const int o = 4 * (w & 1);
    dst[o + 0] = a[0];
    dst[o + 1] = a[1];
    dst[o + 2] = b[0];
    dst[o + 3] = b[1];
  }
  (void)cb;
  *(GQA_LDS h8*)(row_base + phys0 * 16) = lo;
  *(GQA_LDS h8*)(row_base + phys1 * 16) = hi;
}

__global__ __launch_bounds__(256, 1) void verify_fwd(VerifyParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[2][2][2 * kVTileBytes];  // [stream][buf][K | V]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int stream = wave >> 1;
  const int cblk = wave & 1;  // row block 0 (rows 0..31) or 1 (rows 32..63); also K (0) / V (1) loader
  const int half = lane >> 5;
  const int col = lane & 31;

  const int sid = 2 * blockIdx.x + stream;
  const int t_lo = (int)((long long)sid * p.ntiles / p.nstreams);
  const int t_hi = (int)((long long)(sid + 1) * p.ntiles / p.nstreams);
  // the two streams may differ by one tile; every wave runs the longer count
  // of iterations so that all of them meet at the same barriers
  const int s0 = 2 * blockIdx.x;
  const int n0 = (int)((long long)(s0 + 1) * p.ntiles / p.nstreams) - (int)((long long)s0 * p.ntiles / p.nstreams);
  const int n1 = (int)((long long)(s0 + 2) * p.ntiles / p.nstreams) -
                 (int)((long long)(s0 + 1) * p.ntiles / p.nstreams);
  const int n_iter = n0 > n1 ? n0 : n1;

  const rsrc_t rq = make_rsrc(p.q, (uint32_t)p.nrows * kRowBytes);
  const rsrc_t rsrc_kv = make_rsrc(cblk == 0 ? (const void*)p.k : (const void*)p.v, (uint32_t)p.n_kv * kFp8Row);

  const int row = 32 * cblk + col;
  const bool rows_active = 32 * cblk < p.nrows;
  const int pos = (p.n_kv - p.nq) + min(row, p.nrows - 1) / kGroup;
  const int pos_min = p.n_kv - p.nq;  // first query position
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

  // this wave stages K (cblk 0) or V (cblk 1) of its stream: load j covers
  // row 4j + lane/16, byte chunk lane%16
  const int cb = lane & 15;
  u4 raw[8];
  auto load_raw = [&](int t) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      raw[j] = __builtin_amdgcn_raw_buffer_load_b128(rsrc_kv, (uint32_t)t * (kVTileKeys * kFp8Row) +
                                                                  (uint32_t)((4 * j + (lane >> 4)) * kFp8Row + 16 * cb),
                                                     0, 0);
  };
  if (t_lo < t_hi) load_raw(t_lo);

  for (int it = 0; it < n_iter; ++it) {
    const int t = t_lo + it;
    const bool live = t < t_hi;  // wave-uniform
    const int buf = it & 1;
    GQA_LDS char* kt = (GQA_LDS char*)smem[stream][buf];
    GQA_LDS char* vt = kt + kVTileBytes;
    if (live) {
      GQA_LDS char* dst = cblk == 0 ? kt : vt;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 4 * j + (lane >> 4);
        const int c0 = 2 * cb, c1 = 2 * cb + 1;
        const int p0 = cblk == 0 ? k_phys_chunk(c0, r) : v_phys_chunk(c0, r);
        const int p1 = cblk == 0 ? k_phys_chunk(c1, r) : v_phys_chunk(c1, r);
        decode_store(raw[j], dst + r * kRowBytes, cb, p0, p1);
      }
    }
    if (t + 1 < t_hi) load_raw(t + 1);
    __syncthreads();
    if (live && rows_active) {
      const int k0 = t * kVTileKeys;
      asm volatile("" : "+v"(bk), "+v"(bv));
      attend_32keys<1>(lds_addr(kt) + bk, vt, bv, 0, qf, acc, m, l, p.c, k0 + 31 > pos_min,
                       [&](int, int vv) { return k0 + lane_key(vv, half) <= pos; });
    }
  }

  // merge stream 1 into stream 0 through LDS, then write one partial per workgroup
  float lt = swap_halves_sum(l[0]);
  __syncthreads();
  float* xch = (float*)smem;  // [2 row blocks][128 floats of acc per lane group][64 lanes] + m, l
  if (stream == 1) {
    float* base = xch + cblk * (130 * 64);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) base[(dt * 16 + vv) * 64 + lane] = acc[0][dt][vv];
    base[128 * 64 + lane] = m[0];
    base[129 * 64 + lane] = lt;
  }
  __syncthreads();
  if (stream == 0 && rows_active) {
    const float* base = xch + cblk * (130 * 64);
    const float m1 = base[128 * 64 + lane];
    const float l1 = base[129 * 64 + lane];
    const float mm = fmaxf(m[0], m1);
    const float a0 = (m[0] == -INFINITY) ? 0.f : fast_exp2(m[0] - mm);
    const float a1 = (m1 == -INFINITY) ? 0.f : fast_exp2(m1 - mm);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) acc[0][dt][vv] = a0 * acc[0][dt][vv] + a1 * base[(dt * 16 + vv) * 64 + lane];
    lt = a0 * lt + a1 * l1;
    if (row < p.nrows) {
      const rsrc_t rp = make_rsrc(p.part, p.part_bytes);
      store_partial(rp, (uint32_t)blockIdx.x * (uint32_t)(kVerifySlotFloats * 4), kVerifySlotRows, row, half,
                    acc[0], mm, lt);
    }
  }
}

// Merge of the workgroups' partials: workgroup (r, part) combines row r,
// head-dim columns 64*part .. 64*part+63, over all slots.  Thread
// (quad, sl) takes columns 64*part + 4*quad .. +3 of the slots sl, sl+16, ...;
// the 16 slot lanes are then reduced through LDS.
__global__ __launch_bounds__(256) void verify_merge(VerifyParams p) {
  __shared__ float red[16][16][5];
  __shared__ float mred[16];
  const int r = blockIdx.x >> 2;
  const int part = blockIdx.x & 3;
  const int tid = threadIdx.x;
  const int quad = tid & 15;
  const int sl = tid >> 4;
  const rsrc_t rp = make_rsrc(p.part, p.part_bytes);
  const uint32_t slot_bytes = (uint32_t)(kVerifySlotFloats * 4);
  const uint32_t m_off = (uint32_t)(kVerifySlotRows * kHeadDim * 4);
  float M = -INFINITY;
  for (int s = sl; s < p.grid; s += 16)
    M = fmaxf(M, __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, s * slot_bytes + m_off + r * 4, 0, 0)));
  if (quad == 0) mred[sl] = M;
  __syncthreads();
  M = mred[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) M = fmaxf(M, mred[i]);
  f4 o = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  const uint32_t qoff = (uint32_t)(((16 * part + quad) * kVerifySlotRows + r) * 16);
#pragma unroll 4
  for (int s = sl; s < p.grid; s += 16) {
    const uint32_t sb = s * slot_bytes;
    const float ms = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, sb + m_off + r * 4, 0, 0));
    const float ls = __uint_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(rp, sb + m_off + (kVerifySlotRows + r) * 4, 0, 0));
    const u4 x = __builtin_amdgcn_raw_buffer_load_b128(rp, sb + qoff, 0, 0);
    const float a = (ms == -INFINITY) ? 0.f : fast_exp2(ms - M);
    o += a * __builtin_bit_cast(f4, x);
    L += a * ls;
  }
  red[sl][quad][0] = o[0];
  red[sl][quad][1] = o[1];
  red[sl][quad][2] = o[2];
  red[sl][quad][3] = o[3];
  red[sl][quad][4] = L;
  __syncthreads();
  if (sl == 0) {
    f4 t = {0.f, 0.f, 0.f, 0.f};
    float lt = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      t[0] += red[i][quad][0];
      t[1] += red[i][quad][1];
      t[2] += red[i][quad][2];
      t[3] += red[i][quad][3];
      lt += red[i][quad][4];
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
  p.nstreams = 2 * s.grid;
  p.grid = s.grid;
  p.part_bytes = (uint32_t)verify_workspace_bytes(s);
  p.c = scale * k_scale * kLog2e;
  p.v_scale = v_scale;
  prof_before(stream);
  hipLaunchKernelGGL(verify_fwd, dim3(s.grid), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  prof_after(stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(verify_merge, dim3(p.nrows * 4), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gqa
