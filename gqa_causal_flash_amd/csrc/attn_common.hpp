// Shared device-side building blocks of the gfx950 attention kernels.
//
// Matrix-core conventions (v_mfma_f32_32x32x16_f16, wave64):
//   A [32 x 16] : lane l holds A[l % 32][8 * (l / 32) + j], j = 0..7
//   B [16 x 32] : lane l holds B[8 * (l / 32) + j][l % 32]
//   C [32 x 32] : lane l, register v holds C[8 * (v / 4) + 4 * (l / 32) + v % 4][l % 32]
//
// Scores are computed transposed, S^T = K Q^T: keys run down the 32 rows of
// C and packed query rows across its 32 columns, so every lane owns one query
// row and half of its keys.  The row statistics of the online softmax are then
// per-lane values plus one exchange between the two lane halves, and P^T taken
// straight from the C registers (eight consecutive registers, converted to
// fp16) is already the B operand of the next product O^T += V^T P^T.  V^T
// comes from LDS through the transposing read ds_read_b64_tr_b16, which hands
// each lane four consecutive keys of one head-dimension column.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f16x __attribute__((ext_vector_type(16)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef short s4 __attribute__((ext_vector_type(4)));

#define GQA_LDS __attribute__((address_space(3)))
#define GQA_GLOBAL __attribute__((address_space(1)))

constexpr int kHeadDim = 256;          // D
constexpr int kGroup = 6;              // query heads per K/V head
constexpr int kRowBytes = kHeadDim * 2;  // one fp16 K or V row: 512 B = 32 chunks of 16 B
constexpr float kLog2e = 1.4426950408889634f;
// Lazy rescaling threshold (log2 units): the running reference max is only
// raised when a new score exceeds it by more than 2^8, so P stays <= 256.
constexpr float kRescaleTau = 8.0f;

// ---------------------------------------------------------------- LDS layout
// A K or V tile row (one key, 512 B) is stored with its 16-byte chunks
// permuted by an XOR of the row index so that the matrix-core operand reads
// are bank-conflict free:
//   K: chunk c of row r sits at c ^ (r % 16)      (ds_read_b128, 32 rows x 32 B)
//   V: chunk c of row r sits at c ^ 4 * (r % 8)   (ds_read_b64_tr_b16, 8 rows x 64 B)
__device__ __forceinline__ int k_phys_chunk(int c, int r) { return c ^ (r & 15); }
__device__ __forceinline__ int v_phys_chunk(int c, int r) { return c ^ ((r & 7) << 2); }

// ------------------------------------------------------------ buffer access
// All global memory is reached through buffer resources: a wave-uniform base
// and byte size in scalar registers, a 32-bit per-lane offset, and a hardware
// range check (a load past the size returns zeros and a store past it is
// dropped), so no kernel can touch memory outside the tensors it was given.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned u4 __attribute__((ext_vector_type(4)));
typedef unsigned u2 __attribute__((ext_vector_type(2)));
constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) buffer on gfx9-family parts

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// HBM -> LDS copy of 16 B per lane: byte `voff + soff` of the buffer lands in
// the lane's 16-byte chunk of the 1 KiB that the wave writes at `lds_base`.
__device__ __forceinline__ void load_lds_16B(rsrc_t r, GQA_LDS void* lds_base, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_base, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ h8 load_16B(rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}
__device__ __forceinline__ void store_16B(rsrc_t r, uint32_t voff, u4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(x, r, voff, 0, 0);
}
__device__ __forceinline__ void store_8B(rsrc_t r, uint32_t voff, h4 x) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2, x), r, voff, 0, 0);
}
// A store at system scope (cache policy sc0 sc1), written through to memory
// instead of being held dirty in the XCD's L2.  Used for split-KV partials,
// which a later kernel reads once, in runs of whole 512-byte rows of lanes:
// the tiny prefill's main kernel takes about 1 us less with them (17.0 ->
// 15.9 us), the long prefill and the paged kernel are unchanged.  Scattered
// 8-byte output stores are slower this way and keep the default policy.
constexpr int kStoreSystemScope = 17;  // sc0 (bit 0) | sc1 (bit 4)
__device__ __forceinline__ void store_16B_through(rsrc_t r, uint32_t voff, u4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(x, r, voff, 0, kStoreSystemScope);
}

// Fragment reads.  Each lane keeps two per-lane LDS byte offsets, and every
// fragment address is one of them XOR a per-step constant plus a compile-time
// offset (see the derivations below), so the loop needs one v_xor per read.
//
// K fragment (kb, s): A operand of S^T = K Q^T for key rows 32kb .. 32kb+31
// and head-dim columns 16s .. 16s+15.  Lane l reads row r = 32kb + l%32,
// logical chunk 2s + l/32, stored at chunk (2s + l/32) ^ (r % 16), i.e. at byte
//   r*512 + 16*((2s + h) ^ (l%16))  =  16384 kb + (bk ^ 32 s),
//   bk = 512 (l%32) + 16 (h ^ (l%16))            (h = l/32).
__device__ __forceinline__ uint32_t k_lane_base(int lane) {
  const int h = lane >> 5, col = lane & 31;
  return 512u * col + 16u * (uint32_t)(h ^ (col & 15));
}
// `kaddr` = LDS byte address of the tile + bk: the tile base has no bits
// below 2^14, so it commutes with the XOR and the read costs one v_xor.
__device__ __forceinline__ h8 read_k_frag(uint32_t kaddr, int kb, int s) {
  return *(const GQA_LDS h8*)(uintptr_t)((kaddr ^ (32u * s)) + 16384u * kb);
}
__device__ __forceinline__ uint32_t lds_addr(const GQA_LDS void* p) { return (uint32_t)(uintptr_t)p; }

// V^T half fragment: A operand of O^T += V^T P^T for head-dim rows
// 32dt .. 32dt+31 and keys key0 + 4h + e (e = 0..3, key0 a multiple of 8), read
// transposed from the [key][d] tile.  In each 16-lane group, source lane j
// addresses key row j/4 and columns 4(j%4) .. +3 of the group's 16 columns;
// output lane i then holds column i of those four rows.  With the V swizzle
// (chunk c of row r at c ^ 4(r%8)) the byte address is
//   key0*512 + (bv ^ 64 dt),
//   bv = 512 (4h + (l%16)/4) + 16 (2((l/16)%2) + (l%4)/2) + 8 (l%2) + 64 ((4h + (l%16)/4) % 8).
__device__ __forceinline__ uint32_t v_lane_base(int lane) {
  const int h = lane >> 5;
  const int row = 4 * h + ((lane & 15) >> 2);
  const int delta = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  return 512u * row + 16u * delta + 8u * (lane & 1) + 64u * (row & 7);
}
__device__ __forceinline__ h4 read_vt_half(const GQA_LDS char* vtile, uint32_t bv, int key0, int dt) {
  s4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GQA_LDS s4*)(vtile + key0 * kRowBytes + (bv ^ (64u * dt))));
  return __builtin_bit_cast(h4, x);
}

__device__ __forceinline__ h8 cat_h4(h4 a, h4 b) {
  return h8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// fp32 -> fp16 (round to nearest even), two at a time (v_cvt_pk_f16_f32).
__device__ __forceinline__ h2 cvt2(float a, float b) { return __builtin_convertvector(f2{a, b}, h2); }

// Value of x in the other half of the wave (lane l <-> lane l ^ 32).
__device__ __forceinline__ float swap_halves_max(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float swap_halves_sum(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Workgroup barrier for loops that keep loads into LDS in flight across it.
// __syncthreads() fences memory, and a release of LDS waits for every
// outstanding load into LDS as well; here those loads are waited for
// explicitly, as far as each step needs.  This barrier waits only for the
// wave's own LDS reads and writes (lgkmcnt), and the empty asm statements
// with a memory clobber keep the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ f16x mfma(h8 a, h8 b, f16x c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace gqa
