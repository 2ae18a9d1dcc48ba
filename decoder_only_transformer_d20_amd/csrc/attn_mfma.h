// Causal flash attention on gfx950 matrix cores, head dimension 128.
//
// Shared pieces of the forward and backward kernels.  Inputs are the
// token-major qkv rows the QKV projection writes ([B*T][3*H*128]: q | k | v,
// q and k already rotated); outputs are token-major too, so no relayout
// kernel sits between the projections and attention.
//
// Every product is a v_mfma_f32_32x32x16_bf16.  For C = A * B the lane
// holding column n (= lane & 31) of the result holds rows
// 8*(r/4) + 4*(lane/32) + (r%4) in accumulator r; the operand lanes supply
// 8 consecutive k values each, lanes 32-63 the upper 8 of every 16.  Scores
// are computed transposed (S^T = K Q^T), which puts one query row in one
// lane: the softmax statistics are per-lane scalars and the 8 consecutive
// accumulators of a 16-key group are exactly the B operand of the next
// product (P^T as B), provided the A operand (V^T, K^T, Q^T, dO^T) lists its
// 16 keys in the matching order: keys 0-3, 8-11, 4-7, 12-15 of each group
// ("slot order").  Every tile sits in LDS once, in its natural
// [rows][128 features] layout; the transposed operands are read from that
// image with gfx950's transposing LDS read (ds_read_b64_tr_b16), which
// hands each lane four consecutive rows of one feature column -- two reads
// give the eight slot-ordered keys.
#pragma once

#include "nc_internal.h"

namespace nc {
namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef const u32x4 __attribute__((address_space(1)))* gptr;

constexpr int HD = 128;               // head dimension
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

__device__ inline float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// two fp32 -> packed bf16, round to nearest even: one v_cvt_pk_bf16_f32
__device__ inline uint32_t pack2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ inline u32x4 gload(const bf16* p) { return *(gptr)p; }

// LDS image of a [64 rows][128 features] tile (256 B rows, 16 chunks of 16 B):
// chunk c of row r at slot c ^ swz(r), swz(r) = 4 (r & 3) + ((r >> 2) & 3).
// gfx950's LDS serves 256 B (64 banks) per cycle.  A natural fragment read
// takes 16 consecutive rows at one chunk: swz is a permutation over them.
// A transposing read takes, per 32 lanes, four rows r0 .. r0+3 (r0 a
// multiple of 4) at four consecutive chunks 4t .. 4t+3: swz moves row
// r0 + b to chunk group t ^ b, so the 16 slots are distinct.  A row write
// (16 lanes, one row's 16 chunks) is a permutation too.
__device__ inline uint32_t swz(int row) { return 4 * (row & 3) + ((row >> 2) & 3); }
__device__ inline uint32_t offN(int row, int chunk) { return (uint32_t)row * 256u + ((chunk ^ swz(row)) << 4); }

// Natural image of 64 rows x 128 of one head (row stride ld elements in
// global memory) by `nthr` threads starting at thread `t`: 1024 chunks.
template <int NTHR>
__device__ inline void load_nat64(const bf16* src, int64_t ld, int t, u32x4 (&reg)[1024 / NTHR]) {
#pragma unroll
  for (int i = 0; i < 1024 / NTHR; ++i) {
    const int q = t + NTHR * i;
    reg[i] = gload(src + (int64_t)(q >> 4) * ld + (q & 15) * 8);
  }
}
template <int NTHR>
__device__ inline void store_nat64(char* lds, int t, const u32x4 (&reg)[1024 / NTHR]) {
#pragma unroll
  for (int i = 0; i < 1024 / NTHR; ++i) {
    const int q = t + NTHR * i;
    *reinterpret_cast<u32x4*>(lds + offN(q >> 4, q & 15)) = reg[i];
  }
}

// Transposed fragments of a natural image: for feature block t (features
// 32t .. 32t+31) lane l receives feature 32t + (l & 31) at the 8
// slot-ordered rows 16 sp + 4 hh + {0-3, 8-11} (hh = l >> 5).  In each group
// of 16 lanes (g = l >> 4), lane j addresses row 4 hh + (j >> 2) (+8 for the
// second read) and the 4-feature piece 16 (g & 1) + 4 (j & 3) of the block;
// the read returns to lane j the four rows at feature 16 (g & 1) + j.
// Moving to sp adds 16 rows = 4096 bytes (swz is unchanged); moving to t
// adds 4 to the chunk index, which under swz (rows agree in their low 2 bits
// of the chunk term) is an xor of 64 on the byte offset.
struct TrOff {
  uint32_t lo, hi;          // byte offsets of the two reads for t = 0, sp = 0
  __device__ inline void init(int lane) {
    const int j = lane & 15, g = lane >> 4, hh = g >> 1;
    const int rlo = 4 * hh + (j >> 2), rhi = rlo + 8;
    const int c = 2 * (g & 1) + ((j & 3) >> 1);
    lo = (uint32_t)rlo * 256u + ((c ^ swz(rlo)) << 4) + 8u * (j & 1);
    hi = (uint32_t)rhi * 256u + ((c ^ swz(rhi)) << 4) + 8u * (j & 1);
  }
  __device__ inline uint32_t l(int t, int sp) const { return (lo ^ (64u * t)) + 4096u * sp; }
  __device__ inline uint32_t h(int t, int sp) const { return (hi ^ (64u * t)) + 4096u * sp; }
};
typedef short v4i16 __attribute__((ext_vector_type(4)));
__device__ inline bf16x8 frag_tr(const char* img, uint32_t lo, uint32_t hi) {
  typedef __attribute__((address_space(3))) v4i16* lptr;
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lptr)(img + lo));
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lptr)(img + hi));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef __attribute__((address_space(3))) void* lds_vptr;
typedef __attribute__((address_space(1))) void* gbl_vptr;

// Natural image of 64 rows x 128 of one head (row stride ld elements),
// copied from global memory straight into LDS by the 4 waves of a block
// (gfx950's global_load_lds_dwordx4: lane L of a wave's load writes the
// 16 bytes at LDS offset 16 L past the wave-uniform base).  Wave w's four
// 1 KB pieces hold rows 16w .. 16w+15; lane L of piece i lands in slot
// L & 15 of row 16w + 4i + L/16, so it reads the chunk that the swizzle puts
// in that slot.  Completion is waited for with vm_wait() before the barrier
// that publishes the image.
__device__ inline void dma_nat64(const bf16* src, int64_t ld, char* img, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * wave + 4 * i + (lane >> 4);
    const int chunk = (lane & 15) ^ (int)swz(row);
    __builtin_amdgcn_global_load_lds((gbl_vptr)(src + (int64_t)row * ld + chunk * 8),
                                     (lds_vptr)(img + (16 * wave + 4 * i) * 256), 16, 0, 0);
  }
}
// dma_nat64 through a buffer resource, for a block of NW waves (4 or 8):
// measured 4-5 % faster than the global-address form in the forward kernel.
// wave w copies rows (64 / NW) w .. in 1 KB pieces of 4 rows.  The per-lane
// byte offsets are computed once; a tile is selected by the scalar offset,
// so a copy is one buffer_load ... lds per piece with no per-tile address
// arithmetic.  Offsets at or past `bytes` read zeros.
template <int NW>
struct TileCopy {
  static constexpr int kPieces = 16 / NW;
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t off[kPieces];
  __device__ inline void init(const bf16* base, int64_t bytes, int64_t ld, int wave, int lane) {
    rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int row = (64 / NW) * wave + 4 * i + (lane >> 4);
      const int chunk = (lane & 15) ^ (int)swz(row);
      off[i] = (uint32_t)(((int64_t)row * ld + chunk * 8) * 2);
    }
  }
  // rows row0 .. row0 + 63 of the base (row stride ld elements) into img
  __device__ inline void copy(int row0, int64_t ld, char* img, int wave) const {
#pragma unroll
    for (int i = 0; i < kPieces; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_vptr)(img + ((64 / NW) * wave + 4 * i) * 256), 16, off[i],
                                               (int)(row0 * ld * 2), 0, 0);
  }
};
// The same for a block of NW waves copying `rows` (a multiple of 4 NW) rows:
// wave w takes rows w * rows / NW .. in 1 KB pieces of 4 rows.
template <int NW>
__device__ inline void dma_rows(const bf16* src, int64_t ld, char* img, int rows, int wave, int lane) {
  const int per = rows / NW, r0 = wave * per;
  for (int i = 0; i < per; i += 4) {
    const int row = r0 + i + (lane >> 4);
    const int chunk = (lane & 15) ^ (int)swz(row);
    __builtin_amdgcn_global_load_lds((gbl_vptr)(src + (int64_t)row * ld + chunk * 8),
                                     (lds_vptr)(img + (r0 + i) * 256), 16, 0, 0);
  }
}
__device__ inline void vm_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// every vector-memory operation but the 2 most recently issued has completed
__device__ inline void vm_wait_but2() { asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); }
// A workgroup barrier for LDS traffic only: the wave's LDS operations are
// complete, then s_barrier.  Unlike __syncthreads() it carries no release
// fence, which would wait for every global store of the wave as well.  Use
// it only where no other wave reads this wave's global stores.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// 8 consecutive fp32 accumulators -> one bf16x8 operand
__device__ inline bf16x8 pack8(const floatx16& a, int base) {
  u32x4 v;
  v[0] = pack2(a[base + 0], a[base + 1]);
  v[1] = pack2(a[base + 2], a[base + 3]);
  v[2] = pack2(a[base + 4], a[base + 5]);
  v[3] = pack2(a[base + 6], a[base + 7]);
  return as_bf16x8(v);
}

__device__ inline floatx16 mfma(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline void zero(floatx16& a) {
#pragma unroll
  for (int r = 0; r < 16; ++r) a[r] = 0.f;
}

}  // namespace attn
}  // namespace nc
