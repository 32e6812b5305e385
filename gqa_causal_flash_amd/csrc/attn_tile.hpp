// One 32-key step of the fused attention loop, shared by every kernel.
//
// `kaddr` is the lane's K fragment base in the staged tile (tile address +
// k_lane_base), `vt`/`bv` the V tile and the lane's V base.
//
// For a wave holding C blocks of 32 packed query rows (Q as matrix-core B
// fragments in registers, O^T accumulators, running max m and partial sum l
// per lane) and a K/V tile staged in LDS (fp16, swizzled as described in
// attn_common.hpp), attend_32keys() folds keys 32*kb .. 32*kb+31 of the tile
// into the running online-softmax state:
//
//   S^T = K Q^T                                   (16 matrix-core steps per block)
//   t   = S * c                                   (c = scale * log2 e: log2 units)
//   if max t > m + 8 anywhere in the wave:       (lazy rescaling)
//       m' = max(m, max t);  O *= 2^(m - m');  l *= 2^(m - m')
//   P   = fp16(2^(t - m)),   l += sum P           (sum of the fp16 weights used)
//   O^T += V^T P^T
//
// Keys the caller marks invisible get t = -inf and P = 0.  m stays -inf until a
// row sees its first key; the exponent then uses 0 instead of m so no
// (-inf) - (-inf) is ever formed.  The lane's l covers only its half of the
// keys; the two halves are added when the row is finished.
#pragma once

#include "attn_common.hpp"

namespace gqa {

#ifndef GQA_KPF
#define GQA_KPF 4
#endif
#ifndef GQA_KPV
#define GQA_KPV 2
#endif

// S^T[32 keys][32C rows] = K Q^T for the 32 keys whose fragment si (head-dim
// columns 16si .. 16si+15) kfrag(si) reads.
template <int C, int KPF, class KFrag>
__device__ __forceinline__ void qk_32keys_f(KFrag kfrag, const h8 (&qf)[C][16], f16x (&s)[C]) {
#pragma unroll
  for (int c = 0; c < C; ++c) s[c] = f16x{};
  {
    // K fragments run kPF steps ahead of the matrix cores
    constexpr int kPF = KPF;
    h8 kf[kPF];
#pragma unroll
    for (int j = 0; j < kPF; ++j) kf[j] = kfrag(j);
#pragma unroll
    for (int si = 0; si < 16; ++si) {
      const h8 a = kf[si % kPF];
      if (si + kPF < 16) kf[si % kPF] = kfrag(si + kPF);
#pragma unroll
      for (int c = 0; c < C; ++c) s[c] = mfma(a, qf[c][si], s[c]);
    }
    // keep that order: kPF reads up front, then one read per matrix-core step
    __builtin_amdgcn_sched_group_barrier(0x100, kPF, 0);
#pragma unroll
    for (int si = 0; si < 16 - kPF; ++si) {
      __builtin_amdgcn_sched_group_barrier(0x008, C, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, C * kPF, 0);
  }
}

// qk_32keys_f with memory copies interleaved: hook(i), i = 0..7, issues one
// vector-memory instruction after product 2i, so that a wave's copies reach
// the vector-memory pipe spread over its products instead of in one burst.
template <int C, int KPF, class KFrag, class Hook>
__device__ __forceinline__ void qk_32keys_fh(KFrag kfrag, const h8 (&qf)[C][16], f16x (&s)[C], Hook hook) {
#pragma unroll
  for (int c = 0; c < C; ++c) s[c] = f16x{};
  constexpr int kPF = KPF;
  h8 kf[kPF];
#pragma unroll
  for (int j = 0; j < kPF; ++j) kf[j] = kfrag(j);
#pragma unroll
  for (int si = 0; si < 16; ++si) {
    const h8 a = kf[si % kPF];
    if (si + kPF < 16) kf[si % kPF] = kfrag(si + kPF);
#pragma unroll
    for (int c = 0; c < C; ++c) s[c] = mfma(a, qf[c][si], s[c]);
    if (si % 2 == 0) hook(si / 2);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, kPF, 0);
#pragma unroll
  for (int si = 0; si < 16; ++si) {
    __builtin_amdgcn_sched_group_barrier(0x008, C, 0);
    if (si + kPF < 16) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (si % 2 == 0) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
  }
}

// S^T[32 keys][32C rows] = K Q^T for keys 32kb .. 32kb+31 of the staged tile.
template <int C, int KPF = GQA_KPF>
__device__ __forceinline__ void qk_32keys(uint32_t kaddr, int kb, const h8 (&qf)[C][16], f16x (&s)[C]) {
  qk_32keys_f<C, KPF>([&](int si) { return read_k_frag(kaddr, kb, si); }, qf, s);
}

// Online-softmax update from the scores of 32 keys; returns P^T as fp16 B operands.
template <int C, class Visible>
__device__ __forceinline__ void softmax_32keys(f16x (&s)[C], f16x (&acc)[C][8], float (&m)[C], float (&l)[C],
                                               float cscale, bool mask, Visible visible, h8 (&pk)[C][2]) {
  const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
  for (int c = 0; c < C; ++c) {
    if (mask) {
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) s[c][vv] = visible(c, vv) ? s[c][vv] : -INFINITY;
    }
    float mx = s[c][0];
#pragma unroll
    for (int vv = 1; vv < 16; ++vv) mx = fmaxf(mx, s[c][vv]);
    mx = swap_halves_max(mx);
    const float tmax = mx * cscale;
    if (__any(tmax > m[c] + kRescaleTau)) {
      const float mnew = fmaxf(m[c], tmax);
      const float alpha = (mnew == -INFINITY) ? 1.0f : fast_exp2(m[c] - mnew);
      m[c] = mnew;
      l[c] *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) acc[c][dt] *= alpha;
    }
    const float msub = (m[c] == -INFINITY) ? 0.0f : m[c];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float e[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) e[u] = fast_exp2(__builtin_fmaf(s[c][8 * t + u], cscale, -msub));
      const h2 p0 = cvt2(e[0], e[1]);
      const h2 p1 = cvt2(e[2], e[3]);
      const h2 p2 = cvt2(e[4], e[5]);
      const h2 p3 = cvt2(e[6], e[7]);
      float ls = l[c];
      ls = __builtin_amdgcn_fdot2(p0, ones, ls, false);
      ls = __builtin_amdgcn_fdot2(p1, ones, ls, false);
      ls = __builtin_amdgcn_fdot2(p2, ones, ls, false);
      ls = __builtin_amdgcn_fdot2(p3, ones, ls, false);
      l[c] = ls;
      pk[c][t] = h8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    }
  }

}

// O^T[256 d][32C rows] += V^T[256 d][32 keys] P^T for keys 32kb .. 32kb+31 of the staged tile.
template <int C, int KPV = GQA_KPV>
__device__ __forceinline__ void pv_32keys(const GQA_LDS char* vt, uint32_t bv, int kb, const h8 (&pk)[C][2],
                                          f16x (&acc)[C][8]) {
  {
    // V^T fragments (two transposed reads each) run kPV steps ahead; step st
    // is head-dim tile st / 2 and key half st % 2.
    constexpr int kPV = KPV;
    h4 vlo[kPV], vhi[kPV];
#pragma unroll
    for (int j = 0; j < kPV; ++j) {
      const int dt = j >> 1, t = j & 1;
      vlo[j] = read_vt_half(vt, bv, 32 * kb + 16 * t, dt);
      vhi[j] = read_vt_half(vt, bv, 32 * kb + 16 * t + 8, dt);
    }
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const int dt = st >> 1, t = st & 1;
      const h8 a = cat_h4(vlo[st % kPV], vhi[st % kPV]);
      if (st + kPV < 16) {
        const int dn = (st + kPV) >> 1, tn = (st + kPV) & 1;
        vlo[st % kPV] = read_vt_half(vt, bv, 32 * kb + 16 * tn, dn);
        vhi[st % kPV] = read_vt_half(vt, bv, 32 * kb + 16 * tn + 8, dn);
      }
#pragma unroll
      for (int c = 0; c < C; ++c) acc[c][dt] = mfma(a, pk[c][t], acc[c][dt]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPV, 0);
#pragma unroll
    for (int st = 0; st < 16 - kPV; ++st) {
      __builtin_amdgcn_sched_group_barrier(0x008, C, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, C * kPV, 0);
  }
}

template <int C, class Visible, int KPF = GQA_KPF, int KPV = GQA_KPV>
__device__ __forceinline__ void attend_32keys(uint32_t kaddr, const GQA_LDS char* vt, uint32_t bv, int kb,
                                              const h8 (&qf)[C][16], f16x (&acc)[C][8], float (&m)[C],
                                              float (&l)[C], float cscale, bool mask, Visible visible) {
  f16x s[C];
  qk_32keys<C, KPF>(kaddr, kb, qf, s);
  h8 pk[C][2];
  softmax_32keys<C>(s, acc, m, l, cscale, mask, visible, pk);
  pv_32keys<C, KPV>(vt, bv, kb, pk, acc);
}

// attend_32keys for the first 32 keys of a K tile named by its LDS pointer `kt`
// (bk = k_lane_base of the lane): the fragment addresses keep the tile's
// identity, so the compiler can tell the tile apart from LDS that loads are
// landing in elsewhere.  hook(i), i = 0..7, issues one vector-memory copy
// among the Q K^T products (qk_32keys_fh).
template <int C, class Visible, int KPF, int KPV, class Hook>
__device__ __forceinline__ void attend_32keys_p(const GQA_LDS char* kt, uint32_t bk, const GQA_LDS char* vt, uint32_t bv,
                                                const h8 (&qf)[C][16], f16x (&acc)[C][8], float (&m)[C],
                                                float (&l)[C], float cscale, bool mask, Visible visible, Hook hook) {
  f16x s[C];
  qk_32keys_fh<C, KPF>([&](int si) { return *(const GQA_LDS h8*)(kt + (bk ^ (32u * (uint32_t)si))); }, qf, s, hook);
  h8 pk[C][2];
  softmax_32keys<C>(s, acc, m, l, cscale, mask, visible, pk);
  pv_32keys<C, KPV>(vt, bv, 0, pk, acc);
}

// Key index inside the 32-key block held by this lane's accumulator register vv.
__device__ __forceinline__ int lane_key(int vv, int half) { return 8 * (vv >> 2) + 4 * half + (vv & 3); }

// Write the finished rows of one column block as fp16, normalised by the full
// row sum lt (0 when the row saw no key).  Row `row` of the [rows][256] output
// buffer `ro`; writes past the buffer are dropped by the range check.
__device__ __forceinline__ void store_rows_f16(rsrc_t ro, int row, int half, const f16x (&acc)[8], float lt,
                                               float post_scale) {
  const float inv = lt > 0.f ? post_scale / lt : 0.f;
  const uint32_t obase = (uint32_t)row * kRowBytes + half * 8;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const h2 lo = cvt2(acc[dt][4 * g + 0] * inv, acc[dt][4 * g + 1] * inv);
      const h2 hi = cvt2(acc[dt][4 * g + 2] * inv, acc[dt][4 * g + 3] * inv);
      store_8B(ro, obase + (32 * dt + 8 * g) * 2, h4{lo[0], lo[1], hi[0], hi[1]});
    }
}

// Online-softmax partial of one column block for a later log-sum-exp merge.
// Slot layout (fp32): acc[64 column quads][rows_per_slot rows][4], then
// m[rows_per_slot], then l[rows_per_slot].  `rl` is the row inside the slot.
// The accumulator goes out written through (store_16B_through): lanes 0..31
// and 32..63 each write 512 contiguous bytes.
__device__ __forceinline__ void store_partial(rsrc_t rp, uint32_t slot_byte, int rows_per_slot, int rl, int half,
                                              const f16x (&acc)[8], float m, float lt) {
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int quad = 8 * dt + 2 * g + half;  // columns 4*quad .. 4*quad+3
      const f4 x = {acc[dt][4 * g], acc[dt][4 * g + 1], acc[dt][4 * g + 2], acc[dt][4 * g + 3]};
      store_16B_through(rp, slot_byte + (uint32_t)((quad * rows_per_slot + rl) * 16), __builtin_bit_cast(u4, x));
    }
  if (half == 0) {
    const uint32_t mo = slot_byte + (uint32_t)(rows_per_slot * kHeadDim * 4);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m), rp, mo + rl * 4, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lt), rp, mo + (rows_per_slot + rl) * 4, 0, 0);
  }
}

}  // namespace gqa
