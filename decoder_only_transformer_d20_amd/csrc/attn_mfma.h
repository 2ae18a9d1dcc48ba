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
// product (P^T as B), provided the A operand (V^T, K^T, Q^T, dO^T in LDS)
// lists its 16 keys in the matching order: keys 0-3, 8-11, 4-7, 12-15 of
// each group ("slot order").  Tiles that need a transposed LDS image are
// read as 8 x 8 blocks whose 8 rows are picked in slot order and
// transposed in registers.
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

// gfx950's LDS serves 16 lanes x 16 B (64 banks, 256 B) per cycle, and a
// fragment read takes 16 consecutive rows at one chunk, so the swizzles
// give those 16 rows 16 distinct 16-byte slots modulo 256 B.
// LDS image of a [rows][128] tile (256 B rows, 16 chunks): chunk c of row r at c ^ (r & 15)
__device__ inline uint32_t off256(int row, int chunk) { return (uint32_t)row * 256u + ((uint32_t)(chunk ^ (row & 15)) << 4); }
// LDS image of a [128][64 slots] transposed tile (128 B rows, 8 chunks):
// chunk c of row r at c ^ ((r >> 1) & 7) (rows r, r+1 sit in opposite halves)
__device__ inline uint32_t off128(int row, int chunk) {
  return (uint32_t)row * 128u + ((uint32_t)(chunk ^ ((row >> 1) & 7)) << 4);
}

// key (or query) index, within a 64-row tile, of slot e of chunk cj
__device__ inline int slot_row(int cj, int e) {
  const int s = cj >> 1, h = cj & 1;
  return 16 * s + 4 * h + (e < 4 ? e : e + 4);
}

__device__ inline void transpose8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t a = in[2 * p][e >> 1], b = in[2 * p + 1][e >> 1];
      out[e][p] = (e & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
}

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
    *reinterpret_cast<u32x4*>(lds + off256(q >> 4, q & 15)) = reg[i];
  }
}

// Transposed image ([128 features][64 rows in slot order]) of 64 rows x 128:
// 128 blocks of 8 x 8; thread t < 128 takes slot chunk t & 7, features (t >> 3)*8.
__device__ inline void load_tr64(const bf16* src, int64_t ld, int t, u32x4 (&reg)[8]) {
  const int cj = t & 7, fg = t >> 3;
#pragma unroll
  for (int e = 0; e < 8; ++e) reg[e] = gload(src + (int64_t)slot_row(cj, e) * ld + fg * 8);
}
__device__ inline void store_tr64(char* lds, int t, const u32x4 (&reg)[8]) {
  const int cj = t & 7, fg = t >> 3;
  u32x4 tr[8];
  transpose8(reg, tr);
#pragma unroll
  for (int e = 0; e < 8; ++e) *reinterpret_cast<u32x4*>(lds + off128(fg * 8 + e, cj)) = tr[e];
}

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

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
