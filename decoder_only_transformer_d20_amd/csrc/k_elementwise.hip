// HBM-bound kernels of the training step: embedding gather / scatter-add,
// parameter-free RMSNorm forward / backward, the rotary cos/sin table, the
// cross-entropy combine of per-tile log-sum-exp partials, the loss and
// bits-per-byte reduction, the split-K reduction and small fills.
//
// One 64-lane wavefront owns one row wherever a row is reduced; rows are
// read with 16-byte vector loads, so a wave touches whole 128-byte lines.
#include "nc_internal.h"

namespace nc {

namespace {

constexpr int kWave = 64;

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// 16-byte vector of T
template <typename T> struct Vec;
template <> struct Vec<float> {
  static constexpr int n = 4;
  float v[4];
};
template <> struct Vec<bf16> {
  static constexpr int n = 8;
  bf16 v[8];
};

template <typename T> __device__ inline Vec<T> ld16(const T* p) {
  Vec<T> r;
  *reinterpret_cast<uint4*>(&r) = *reinterpret_cast<const uint4*>(p);
  return r;
}
template <typename T> __device__ inline void st16(T* p, const Vec<T>& r) {
  *reinterpret_cast<uint4*>(p) = *reinterpret_cast<const uint4*>(&r);
}

// ---------------------------------------------------------------------------
// embedding
// ---------------------------------------------------------------------------
// x[n, :] = E[idx[n], :]  (a bitwise copy of the row).  An id outside
// [0, V) reads nothing and gives a row of quiet NaNs, so the error shows in
// everything computed from that position instead of reading past the table.
template <typename T>
__global__ void __launch_bounds__(256) k_embed_fwd(const T* __restrict__ E, const int32_t* __restrict__ idx,
                                                   T* __restrict__ x, int64_t n, int d, int V) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n) return;
  const int id = idx[row];
  const int chunks = d * (int)sizeof(T) / 16;
  uint4* t = reinterpret_cast<uint4*>(x + row * d);
  if (id < 0 || id >= V) {
    const uint32_t q = sizeof(T) == 2 ? 0x7fc07fc0u : 0x7fc00000u;
    for (int c = lane; c < chunks; c += kWave) t[c] = make_uint4(q, q, q, q);
    return;
  }
  const uint4* s = reinterpret_cast<const uint4*>(E + (int64_t)id * d);
  for (int c = lane; c < chunks; c += kWave) t[c] = s[c];
}

// ---------------------------------------------------------------------------
// Embedding backward, deterministic: dE[v] (+)= sum of g[p] over the
// positions p with idx[p] = v, summed in increasing p.
//  1. stable LSD radix sort of (id, position) by id, 8-bit digits: per
//     pass a block histogram, one exclusive scan over (digit, block), and a
//     stable scatter (ranks within a wave from ballots over the digit bits,
//     across waves from per-wave digit counts).  Ids outside [0, V) sort as
//     V and are dropped.
//  2. the sorted rows in tiles of 32, one wave each, summed segment by
//     segment in order; a segment wholly inside a tile is written to dE,
//     one that crosses a tile boundary leaves its piece in the tile's
//     "first" (continued from the previous tile) or "last" (continuing)
//     partial row.
//  3. one wave per segment that starts in a tile and continues: its pieces,
//     added in tile order, go to dE.
// No float atomics, so the result is bitwise reproducible.
// ---------------------------------------------------------------------------
constexpr int kSortBlock = 1024;
constexpr int kEmbTile = 32;

__device__ inline int sort_key(const int32_t* kin, int64_t p, int V, bool first) {
  const int k = kin[p];
  return first ? ((k >= 0 && k < V) ? k : V) : k;
}

__global__ void __launch_bounds__(kSortBlock) k_sort_hist(const int32_t* __restrict__ kin, int64_t n, int V,
                                                          int first, int shift, int32_t* __restrict__ H, int nblk) {
  __shared__ int h[256];
  const int tid = threadIdx.x;
  if (tid < 256) h[tid] = 0;
  __syncthreads();
  const int64_t p = (int64_t)blockIdx.x * kSortBlock + tid;
  if (p < n) atomicAdd(&h[(sort_key(kin, p, V, first) >> shift) & 255], 1);
  __syncthreads();
  if (tid < 256) H[(int64_t)tid * nblk + blockIdx.x] = h[tid];
}

// in-place exclusive scan of H[0..total) by one block
__global__ void __launch_bounds__(kSortBlock) k_sort_scan(int32_t* __restrict__ H, int total) {
  __shared__ int part[kSortBlock];
  const int tid = threadIdx.x;
  const int seg = (total + kSortBlock - 1) / kSortBlock;
  const int b0 = tid * seg, b1 = min(total, b0 + seg);
  int sum = 0;
  for (int i = b0; i < b1; ++i) sum += H[i];
  part[tid] = sum;
  __syncthreads();
  for (int o = 1; o < kSortBlock; o <<= 1) {
    const int v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - sum;
  for (int i = b0; i < b1; ++i) {
    const int c = H[i];
    H[i] = run;
    run += c;
  }
}

__global__ void __launch_bounds__(kSortBlock) k_sort_scatter(const int32_t* __restrict__ kin,
                                                             const int32_t* __restrict__ vin, int64_t n, int V,
                                                             int first, int shift, const int32_t* __restrict__ off,
                                                             int nblk, int32_t* __restrict__ kout,
                                                             int32_t* __restrict__ vout) {
  constexpr int NW = kSortBlock / kWave;
  __shared__ int wcnt[NW][256];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < NW * 256; i += kSortBlock) (&wcnt[0][0])[i] = 0;
  const int64_t p = (int64_t)blockIdx.x * kSortBlock + tid;
  const bool valid = p < n;
  int key = 0, val = 0;
  if (valid) {
    key = sort_key(kin, p, V, first);
    val = first ? (int)p : vin[p];
  }
  const int dig = valid ? (key >> shift) & 255 : 256;
  // lanes of this wave with the same digit
  uint64_t m = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const bool bit = (dig >> b) & 1;
    const uint64_t bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  const int rank = __popcll(m & ((1ull << lane) - 1ull));
  __syncthreads();
  if (valid && rank == 0) wcnt[w][dig] = __popcll(m);
  __syncthreads();
  if (tid < 256) {
    int run = 0;
    for (int ww = 0; ww < NW; ++ww) {
      const int c = wcnt[ww][tid];
      wcnt[ww][tid] = run;
      run += c;
    }
  }
  __syncthreads();
  if (valid) {
    const int dst = off[(int64_t)dig * nblk + blockIdx.x] + wcnt[w][dig] + rank;
    kout[dst] = key;
    vout[dst] = val;
  }
}

template <typename T, int NCH>
struct RowAcc {
  static constexpr int VN = Vec<T>::n;
  float a[NCH][VN];
  __device__ inline void zero() {
#pragma unroll
    for (int i = 0; i < NCH; ++i)
#pragma unroll
      for (int e = 0; e < VN; ++e) a[i][e] = 0.f;
  }
  __device__ inline void add(const T* row, int lane, int chunks) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = lane + i * kWave;
      if (c < chunks) {
        const Vec<T> v = ld16(row + c * VN);
#pragma unroll
        for (int e = 0; e < VN; ++e) a[i][e] += to_f32(v.v[e]);
      }
    }
  }
  __device__ inline void add_f32(const float* row, int lane, int chunks) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = lane + i * kWave;
      if (c < chunks) {
#pragma unroll
        for (int e = 0; e < VN; e += 4) {
          const float4 v = *reinterpret_cast<const float4*>(row + c * VN + e);
          a[i][e] += v.x; a[i][e + 1] += v.y; a[i][e + 2] += v.z; a[i][e + 3] += v.w;
        }
      }
    }
  }
  // add_f32 split in two, so that several rows' loads can be in flight
  // before the (ordered) additions
  __device__ inline void load_f32(const float* row, int lane, int chunks, float (&v)[NCH][VN]) const {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = lane + i * kWave;
      if (c < chunks) {
#pragma unroll
        for (int e = 0; e < VN; e += 4) {
          const float4 q = *reinterpret_cast<const float4*>(row + c * VN + e);
          v[i][e] = q.x; v[i][e + 1] = q.y; v[i][e + 2] = q.z; v[i][e + 3] = q.w;
        }
      }
    }
  }
  __device__ inline void add_vals(const float (&v)[NCH][VN], int lane, int chunks) {
#pragma unroll
    for (int i = 0; i < NCH; ++i)
      if (lane + i * kWave < chunks) {
#pragma unroll
        for (int e = 0; e < VN; ++e) a[i][e] += v[i][e];
      }
  }
  // dst = a, or dst += a
  __device__ inline void store(float* dst, int lane, int chunks, bool add) const {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = lane + i * kWave;
      if (c < chunks) {
#pragma unroll
        for (int e = 0; e < VN; e += 4) {
          float4* q = reinterpret_cast<float4*>(dst + c * VN + e);
          float4 v = make_float4(a[i][e], a[i][e + 1], a[i][e + 2], a[i][e + 3]);
          if (add) {
            const float4 o = *q;
            v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
          }
          *q = v;
        }
      }
    }
  }
};

template <typename T, int NCH>
__global__ void __launch_bounds__(256) k_embed_tiles(const T* __restrict__ g, const int32_t* __restrict__ sid,
                                                     const int32_t* __restrict__ spos, int64_t n, int d, int V,
                                                     float* __restrict__ dE, int accumulate,
                                                     float* __restrict__ Pf, float* __restrict__ Pl) {
  const int64_t tile = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t r0 = tile * kEmbTile;
  if (r0 >= n) return;
  const int64_t r1 = r0 + kEmbTile < n ? r0 + kEmbTile : n;
  const int chunks = d / Vec<T>::n;
  RowAcc<T, NCH> acc;
  acc.zero();
  int cur = sid[r0];
  const bool from_prev = r0 > 0 && sid[r0 - 1] == cur;
  bool first = true;
  auto flush = [&](bool to_next) {
    if (cur >= V) return;                         // dropped ids
    if (first && from_prev) acc.store(Pf + tile * d, lane, chunks, false);
    else if (to_next) acc.store(Pl + tile * d, lane, chunks, false);
    else acc.store(dE + (int64_t)cur * d, lane, chunks, accumulate != 0);
  };
  for (int64_t r = r0; r < r1; ++r) {
    const int id = sid[r];
    if (id != cur) {
      flush(false);
      acc.zero();
      cur = id;
      first = false;
    }
    acc.add(g + (int64_t)spos[r] * d, lane, chunks);
  }
  flush(r1 < n && sid[r1] == cur);
}

template <typename T, int NCH>
__global__ void __launch_bounds__(256) k_embed_fix(const int32_t* __restrict__ sid, int64_t n, int d, int V,
                                                   float* __restrict__ dE, int accumulate,
                                                   const float* __restrict__ Pf, const float* __restrict__ Pl) {
  const int64_t tile = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t r0 = tile * kEmbTile;
  if (r0 >= n) return;
  const int64_t r1 = r0 + kEmbTile < n ? r0 + kEmbTile : n;
  const int id = sid[r1 - 1];
  if (r1 >= n || sid[r1] != id || id >= V) return;               // the tile's last segment ends here
  if (sid[r0] == id && r0 > 0 && sid[r0 - 1] == id) return;      // it started in an earlier tile
  const int chunks = d / Vec<T>::n;
  // The id's rows are contiguous in sid (sorted), so it continues into tile
  // u exactly when tile u starts with it.  Tile + 1 does (checked above);
  // the wave probes 64 further tile starts per step, one per lane -- the
  // continuing tiles form a prefix -- instead of one dependent load per tile.
  const int64_t ntile = (n + kEmbTile - 1) / kEmbTile;
  int64_t ulast = tile + 1;                      // last tile holding the id
  for (int64_t base = tile + 2;; base += kWave) {
    const int64_t u = base + lane;
    const bool cont = u < ntile && sid[u * kEmbTile] == id;
    const int k = __popcll(__ballot(cont));
    ulast = base - 1 + k;
    if (k < kWave) break;
  }
  // Pl[tile] + Pf[tile+1] + ... + Pf[ulast], added in that order; the loads
  // of kAhead partial rows are issued before their additions.  A Zipf-hot
  // id spans hundreds of tiles (id 0 of the d20 batch: ~280), so this one
  // wave's chain of round trips sets the kernel's time: 16 rows in flight
  // where the registers allow it.
  RowAcc<T, NCH> acc;
  acc.zero();
  acc.add_f32(Pl + tile * d, lane, chunks);
  constexpr int kAhead = NCH <= 3 ? 16 : 4;
  for (int64_t u = tile + 1; u <= ulast; u += kAhead) {
    float v[kAhead][NCH][RowAcc<T, NCH>::VN];
#pragma unroll
    for (int j = 0; j < kAhead; ++j) acc.load_f32(Pf + (u + j <= ulast ? u + j : ulast) * d, lane, chunks, v[j]);
#pragma unroll
    for (int j = 0; j < kAhead; ++j)
      if (u + j <= ulast) acc.add_vals(v[j], lane, chunks);
  }
  acc.store(dE + (int64_t)id * d, lane, chunks, accumulate != 0);
}

// ---------------------------------------------------------------------------
// RMSNorm: y = x * r, r = 1/sqrt(mean(x^2) + eps).  One wave per row; a lane
// keeps its chunks of the row in registers between the two passes.
// ---------------------------------------------------------------------------
constexpr int kMaxChunks = 8;   // d <= 64 lanes * 8 chunks * (16 B / sizeof(T))
// NCH = chunks a lane holds (a template argument, so the row stays in as
// few registers as the width needs)

template <typename T, int NCH>
__global__ void __launch_bounds__(256) k_rmsnorm_fwd(const T* __restrict__ x, T* __restrict__ y,
                                                     float* __restrict__ r, int64_t rows, int d, float eps) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  constexpr int VN = Vec<T>::n;
  const int chunks = d / VN;
  const T* xr = x + row * d;
  Vec<T> buf[NCH];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + i * kWave;
    if (c < chunks) {
      buf[i] = ld16(xr + c * VN);
#pragma unroll
      for (int e = 0; e < VN; ++e) {
        const float f = to_f32(buf[i].v[e]);
        ss += f * f;
      }
    }
  }
  ss = wave_sum(ss);
  const float rr = 1.0f / sqrtf(ss / (float)d + eps);
  T* yr = y + row * d;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + i * kWave;
    if (c < chunks) {
      Vec<T> o;
#pragma unroll
      for (int e = 0; e < VN; ++e) o.v[e] = from_f32<T>(to_f32(buf[i].v[e]) * rr);
      st16(yr + c * VN, o);
    }
  }
  if (lane == 0) r[row] = rr;
}

// dx = r * (dy - y * mean(dy * y));  dx_io = dx (accumulate = 0) or dx_io + dx.
template <typename T, int NCH>
__global__ void __launch_bounds__(256) k_rmsnorm_bwd(const T* __restrict__ y, const float* __restrict__ r,
                                                     const T* __restrict__ dy, T* __restrict__ dx_io,
                                                     int64_t rows, int d, int accumulate) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  constexpr int VN = Vec<T>::n;
  const int chunks = d / VN;
  const T* yr = y + row * d;
  const T* gr = dy + row * d;
  T* xr = dx_io + row * d;
  // every load of the row (y, dy and, when accumulating, dx) is issued
  // before the reduction
  Vec<T> yb[NCH], gb[NCH], xb[NCH];
  float dot = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + i * kWave;
    if (c < chunks) {
      yb[i] = ld16(yr + c * VN);
      gb[i] = ld16(gr + c * VN);
      if (accumulate) xb[i] = ld16(xr + c * VN);
    }
  }
  const float rr = r[row];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + i * kWave;
    if (c < chunks) {
#pragma unroll
      for (int e = 0; e < VN; ++e) dot += to_f32(yb[i].v[e]) * to_f32(gb[i].v[e]);
    }
  }
  dot = wave_sum(dot) / (float)d;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + i * kWave;
    if (c < chunks) {
      Vec<T> o = xb[i];
#pragma unroll
      for (int e = 0; e < VN; ++e) {
        float v = rr * (to_f32(gb[i].v[e]) - to_f32(yb[i].v[e]) * dot);
        if (accumulate) v += to_f32(o.v[e]);
        o.v[e] = from_f32<T>(v);
      }
      st16(xr + c * VN, o);
    }
  }
}

// ---------------------------------------------------------------------------
// rotary table: tab[t][i] = (cos, sin)(t * base^(-2i/Q)), computed in fp64
// and rounded once (angles reach T radians, far beyond fp32's safe range)
// ---------------------------------------------------------------------------
__global__ void k_rope_table(float2* tab, int t0, int T, int Q, double base) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int half = Q / 2;
  if (k >= (int64_t)T * half) return;
  const int t = (int)(k / half), i = (int)(k % half);
  const double theta = pow(base, -2.0 * (double)i / (double)Q);
  const double phi = (double)(t0 + t) * theta;
  tab[k] = make_float2((float)cos(phi), (float)sin(phi));
}

// ---------------------------------------------------------------------------
// cross-entropy: combine per-tile (max, sum exp) partials of one row into
// lse, then ce = lse - z[target] (0 for an ignored target, NaN for a target
// >= V, which has no logit)
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_ce_combine(const float2* __restrict__ part, int nblk,
                                                    const float* __restrict__ ztgt, const int32_t* __restrict__ tgt,
                                                    float* __restrict__ lse, float* __restrict__ ce, int64_t rows,
                                                    int V) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float2* p = part + row * nblk;
  float mx = -INFINITY;
  for (int b = lane; b < nblk; b += kWave) mx = fmaxf(mx, p[b].x);
  mx = wave_max(mx);
  float s = 0.f;
  for (int b = lane; b < nblk; b += kWave) s += p[b].y * expf(p[b].x - mx);
  s = wave_sum(s);
  if (lane == 0) {
    const float l = mx + logf(s);
    lse[row] = l;
    const int t = tgt[row];
    ce[row] = t < 0 ? 0.f : t < V ? l - ztgt[row] : __builtin_nanf("");
  }
}

// ---------------------------------------------------------------------------
// dz from the kept logits: z holds each logit minus the maximum of its row in
// its tile of tile_w columns (part[row][tile].x), so z + max - lse is the log
// of the softmax probability.  dz = (p - [n == tgt]) * rs; the target column
// takes p from the fp32 target logit.  A block covers 512
// 16-byte vectors of one row (bpr blocks per row).
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) k_dz_from_logits(const T* __restrict__ z, T* __restrict__ dz, int V,
                                                         int bpr, int tile_w,
                                                         const float2* __restrict__ part, int nblk,
                                                         const float* __restrict__ ztgt,
                                                         const int32_t* __restrict__ tgt,
                                                         const float* __restrict__ lse,
                                                         const float* __restrict__ rs) {
  constexpr int VN = Vec<T>::n;
  constexpr float kLog2e = 1.4426950408889634f;
  const int64_t row = blockIdx.x / bpr;
  const int cpr = V / VN;
  const int j0 = (int)(blockIdx.x % bpr) * 512 + (int)threadIdx.x;
  const float l = lse[row], sc = rs[row];
  const int t = tgt[row];
  const float pt = __builtin_amdgcn_exp2f((ztgt[row] - l) * kLog2e) - 1.f;   // used only where n = t
  const T* zr = z + row * V;
  T* dr = dz + row * V;
  Vec<T> v[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
    if (j0 + 256 * u < cpr) v[u] = ld16(zr + (int64_t)(j0 + 256 * u) * VN);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int j = j0 + 256 * u;
    if (j >= cpr) continue;
    const int n = j * VN;
    const float base = (part[row * nblk + n / tile_w].x - l) * kLog2e;
    Vec<T> o;
#pragma unroll
    for (int e = 0; e < VN; ++e) {
      float p = __builtin_amdgcn_exp2f(fmaf(to_f32(v[u].v[e]), kLog2e, base));
      if (n + e == t) p = pt;
      o.v[e] = from_f32<T>(p * sc);
    }
    st16(dr + n, o);
  }
}

// one block: number of valid targets -> 1/n (0 when none)
__global__ void __launch_bounds__(1024) k_count_valid(const int32_t* __restrict__ tgt, int64_t n, float* inv) {
  __shared__ int64_t red[1024];
  int64_t c = 0;
  for (int64_t i = threadIdx.x; i < n; i += 1024) c += tgt[i] >= 0;
  red[threadIdx.x] = c;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *inv = red[0] > 0 ? (float)(1.0 / (double)red[0]) : 0.f;
}

// per-row factor of the head's dz: 1/n_valid (times the token's weight when
// weights are given) for a valid target, 0 for an ignored one, NaN for a
// target >= V (the gradient then shows the error)
__global__ void __launch_bounds__(256) k_row_scale(const int32_t* __restrict__ tgt, const float* __restrict__ w,
                                                    const float* __restrict__ inv, int64_t n, int V,
                                                    float* __restrict__ out) {
  const float iv = *inv;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int t = tgt[i];
    out[i] = t < 0 ? 0.f : t < V ? (w ? iv * w[i] : iv) : __builtin_nanf("");
  }
}

// one block, fixed order: out = {sum w ce, sum w ce / n} over valid targets
__global__ void __launch_bounds__(1024) k_weighted_loss(const float* __restrict__ ce, const int32_t* __restrict__ tgt,
                                                        const float* __restrict__ w, int64_t n, double* out) {
  __shared__ double sce[1024];
  __shared__ int64_t sn[1024];
  double a = 0.0;
  int64_t c = 0;
  for (int64_t i = threadIdx.x; i < n; i += 1024) {
    if (tgt[i] >= 0) {
      a += (double)w[i] * (double)ce[i];
      c += 1;
    }
  }
  sce[threadIdx.x] = a;
  sn[threadIdx.x] = c;
  __syncthreads();
  for (int k = 512; k > 0; k >>= 1) {
    if ((int)threadIdx.x < k) {
      sce[threadIdx.x] += sce[threadIdx.x + k];
      sn[threadIdx.x] += sn[threadIdx.x + k];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    out[0] = sce[0];
    out[1] = sn[0] > 0 ? sce[0] / (double)sn[0] : 0.0;
  }
}

// one block, fixed order: out = {sum ce / n, sum ce / (ln2 * sum bytes), sum ce, sum bytes, n}
// (a target >= V has no byte count to read; its ce is NaN, and so are the sums)
__global__ void __launch_bounds__(1024) k_loss_bpb(const float* __restrict__ ce, const int32_t* __restrict__ tgt,
                                                   const int32_t* __restrict__ bytes, int64_t n, int V, double* out) {
  __shared__ double sce[1024];
  __shared__ int64_t sb[1024], sn[1024];
  double a = 0.0;
  int64_t b = 0, c = 0;
  for (int64_t i = threadIdx.x; i < n; i += 1024) {
    const int t = tgt[i];
    if (t >= 0) {
      a += (double)ce[i];
      if (t < V) b += bytes[t];
      c += 1;
    }
  }
  sce[threadIdx.x] = a;
  sb[threadIdx.x] = b;
  sn[threadIdx.x] = c;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      sce[threadIdx.x] += sce[threadIdx.x + w];
      sb[threadIdx.x] += sb[threadIdx.x + w];
      sn[threadIdx.x] += sn[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double s = sce[0];
    const double nb = (double)sb[0], nv = (double)sn[0];
    out[0] = nv > 0 ? s / nv : 0.0;
    out[1] = nb > 0 ? s / (0.69314718055994530942 * nb) : 0.0;
    out[2] = s;
    out[3] = nb;
    out[4] = nv;
  }
}

// out[i] = (beta ? out[i] : 0) + sum_s part[s][i], in split order
__global__ void __launch_bounds__(256) k_splitk_reduce(const float4* __restrict__ part, int splits, int64_t n4,
                                                       float4* __restrict__ out, int beta) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  // the product is summed first and then added to out, so accumulating
  // adds exactly the value a fresh call would write
  float4 a = part[i];
  for (int s = 1; s < splits; ++s) {
    const float4 p = part[s * n4 + i];
    a.x += p.x; a.y += p.y; a.z += p.z; a.w += p.w;
  }
  if (beta) {
    const float4 o = out[i];
    a.x = o.x + a.x; a.y = o.y + a.y; a.z = o.z + a.z; a.w = o.w + a.w;
  }
  out[i] = a;
}

// out[c][r] = in[r][c] for a [rows][cols] 16-bit matrix (rows, cols
// multiples of 8): 64 x 64 tiles through LDS, 16-byte reads and writes.
__global__ void __launch_bounds__(256) k_transpose16(const uint16_t* __restrict__ in, int64_t rows, int64_t cols,
                                                     uint16_t* __restrict__ out) {
  __shared__ uint16_t t[64][64 + 2];
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int q = tid + 256 * k, rr = q >> 3, ch = q & 7;      // tile row, 8-element chunk
    const int64_t r = r0 + rr, c = c0 + ch * 8;
    if (r < rows && c < cols) {
      const uint4 v = *reinterpret_cast<const uint4*>(in + r * cols + c);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        t[rr][ch * 8 + 2 * e] = (uint16_t)(w[e] & 0xffffu);
        t[rr][ch * 8 + 2 * e + 1] = (uint16_t)(w[e] >> 16);
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int q = tid + 256 * k, cc = q >> 3, ch = q & 7;      // output row (input column), chunk
    const int64_t c = c0 + cc, r = r0 + ch * 8;
    if (c < cols && r < rows) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = (uint32_t)t[ch * 8 + 2 * e][cc] | ((uint32_t)t[ch * 8 + 2 * e + 1][cc] << 16);
      *reinterpret_cast<uint4*>(out + c * rows + r) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

__global__ void k_fill_f32(float* p, int64_t n, float v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// delta[b][h][t] = sum_e dO[b,t,h,e] * O[b,t,h,e]; one wave per (token, head)
template <typename T>
__global__ void __launch_bounds__(256) k_attn_delta(const T* __restrict__ o, const T* __restrict__ dout,
                                                    float* __restrict__ delta, int B, int Tn, int H, int Q) {
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (w >= (int64_t)B * Tn * H) return;
  const int64_t tok = w / H;
  const int h = (int)(w % H);
  const int64_t base = tok * (int64_t)H * Q + (int64_t)h * Q;
  float s = 0.f;
  for (int e = lane; e < Q; e += kWave) s += to_f32(o[base + e]) * to_f32(dout[base + e]);
  s = wave_sum(s);
  if (lane == 0) {
    const int64_t b = tok / Tn, t = tok % Tn;
    delta[(b * H + h) * Tn + t] = s;
  }
}

inline unsigned nblocks(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

}  // namespace

template <typename T>
hipError_t embed_fwd(const T* E, const int32_t* idx, T* x, int64_t n, int d, int V, hipStream_t s) {
  k_embed_fwd<T><<<nblocks(n, 4), 256, 0, s>>>(E, idx, x, n, d, V);
  return hipGetLastError();
}
int64_t embed_bwd_scratch_bytes(int64_t n, int d) {
  const int64_t nblk = (n + kSortBlock - 1) / kSortBlock, ntile = (n + kEmbTile - 1) / kEmbTile;
  return 4 * n * 4 + 256 * nblk * 4 + 2 * ntile * (int64_t)d * 4 + 256;
}
template <typename T>
hipError_t embed_bwd(const T* g, const int32_t* idx, float* dE, int64_t n, int d, int V, int accumulate,
                     void* scratch, hipStream_t s) {
  constexpr int VN = Vec<T>::n;
  if (n <= 0 || d <= 0 || d % VN || d > kWave * kMaxChunks * VN || V <= 0 || n > (1LL << 31) - 1)
    return hipErrorInvalidValue;
  const int64_t nblk64 = (n + kSortBlock - 1) / kSortBlock, ntile = (n + kEmbTile - 1) / kEmbTile;
  if (256 * nblk64 > (1LL << 31) - 1) return hipErrorInvalidValue;
  const int nblk = (int)nblk64;
  int32_t* ka = (int32_t*)scratch;
  int32_t* va = ka + n;
  int32_t* kb = va + n;
  int32_t* vb = kb + n;
  int32_t* H = vb + n;
  float* Pf = (float*)(H + 256 * nblk64);
  float* Pl = Pf + ntile * d;
  // digits: enough 8-bit passes for keys 0..V (V marks dropped ids)
  int bits = 0;
  while (bits < 31 && (V >> bits) != 0) ++bits;
  const int passes = (bits + 7) / 8;
  const int32_t* kin = idx;
  const int32_t* vin = nullptr;
  for (int ps = 0; ps < passes; ++ps) {
    int32_t* ko = (ps & 1) ? kb : ka;
    int32_t* vo = (ps & 1) ? vb : va;
    k_sort_hist<<<nblk, kSortBlock, 0, s>>>(kin, n, V, ps == 0, 8 * ps, H, nblk);
    k_sort_scan<<<1, kSortBlock, 0, s>>>(H, 256 * nblk);
    k_sort_scatter<<<nblk, kSortBlock, 0, s>>>(kin, vin, n, V, ps == 0, 8 * ps, H, nblk, ko, vo);
    kin = ko;
    vin = vo;
  }
  if (!accumulate) k_fill_f32<<<nblocks((int64_t)V * d, 256), 256, 0, s>>>(dE, (int64_t)V * d, 0.f);
  const int nch = (d / VN + kWave - 1) / kWave;
  const unsigned nb = nblocks(ntile, 4);
#define NC_EMB(NCH)                                                                                        \
  do {                                                                                                     \
    k_embed_tiles<T, NCH><<<nb, 256, 0, s>>>(g, kin, vin, n, d, V, dE, accumulate, Pf, Pl);               \
    k_embed_fix<T, NCH><<<nb, 256, 0, s>>>(kin, n, d, V, dE, accumulate, Pf, Pl);                         \
  } while (0)
  switch (nch) {
    case 1: NC_EMB(1); break;
    case 2: NC_EMB(2); break;
    case 3: NC_EMB(3); break;
    case 4: NC_EMB(4); break;
    default: NC_EMB(kMaxChunks); break;
  }
#undef NC_EMB
  return hipGetLastError();
}
template <typename T>
hipError_t rmsnorm_fwd(const T* x, T* y, float* r, int64_t rows, int d, float eps, hipStream_t s) {
  if (d % Vec<T>::n != 0 || d > kWave * kMaxChunks * Vec<T>::n) return hipErrorInvalidValue;
  const int nch = (d / Vec<T>::n + kWave - 1) / kWave;
  const unsigned nb = nblocks(rows, 4);
  switch (nch) {
    case 1: k_rmsnorm_fwd<T, 1><<<nb, 256, 0, s>>>(x, y, r, rows, d, eps); break;
    case 2: k_rmsnorm_fwd<T, 2><<<nb, 256, 0, s>>>(x, y, r, rows, d, eps); break;
    case 3: k_rmsnorm_fwd<T, 3><<<nb, 256, 0, s>>>(x, y, r, rows, d, eps); break;
    case 4: k_rmsnorm_fwd<T, 4><<<nb, 256, 0, s>>>(x, y, r, rows, d, eps); break;
    default: k_rmsnorm_fwd<T, kMaxChunks><<<nb, 256, 0, s>>>(x, y, r, rows, d, eps); break;
  }
  return hipGetLastError();
}
template <typename T>
hipError_t rmsnorm_bwd(const T* y, const float* r, const T* dy, T* dx_io, int64_t rows, int d, int accumulate,
                       hipStream_t s) {
  if (d % Vec<T>::n != 0 || d > kWave * kMaxChunks * Vec<T>::n) return hipErrorInvalidValue;
  const int nch = (d / Vec<T>::n + kWave - 1) / kWave;
  const unsigned nb = nblocks(rows, 4);
  switch (nch) {
    case 1: k_rmsnorm_bwd<T, 1><<<nb, 256, 0, s>>>(y, r, dy, dx_io, rows, d, accumulate); break;
    case 2: k_rmsnorm_bwd<T, 2><<<nb, 256, 0, s>>>(y, r, dy, dx_io, rows, d, accumulate); break;
    case 3: k_rmsnorm_bwd<T, 3><<<nb, 256, 0, s>>>(y, r, dy, dx_io, rows, d, accumulate); break;
    case 4: k_rmsnorm_bwd<T, 4><<<nb, 256, 0, s>>>(y, r, dy, dx_io, rows, d, accumulate); break;
    default: k_rmsnorm_bwd<T, kMaxChunks><<<nb, 256, 0, s>>>(y, r, dy, dx_io, rows, d, accumulate); break;
  }
  return hipGetLastError();
}
template <typename T>
hipError_t attn_delta(const AttnDesc& a, hipStream_t s) {
  const int64_t w = (int64_t)a.B * a.T * a.H;
  k_attn_delta<T><<<nblocks(w, 4), 256, 0, s>>>((const T*)a.o, (const T*)a.dout, a.delta, a.B, a.T, a.H, a.Q);
  return hipGetLastError();
}

template hipError_t embed_fwd<float>(const float*, const int32_t*, float*, int64_t, int, int, hipStream_t);
template hipError_t embed_fwd<bf16>(const bf16*, const int32_t*, bf16*, int64_t, int, int, hipStream_t);
template hipError_t embed_bwd<float>(const float*, const int32_t*, float*, int64_t, int, int, int, void*, hipStream_t);
template hipError_t embed_bwd<bf16>(const bf16*, const int32_t*, float*, int64_t, int, int, int, void*, hipStream_t);
template hipError_t rmsnorm_fwd<float>(const float*, float*, float*, int64_t, int, float, hipStream_t);
template hipError_t rmsnorm_fwd<bf16>(const bf16*, bf16*, float*, int64_t, int, float, hipStream_t);
template hipError_t rmsnorm_bwd<float>(const float*, const float*, const float*, float*, int64_t, int, int, hipStream_t);
template hipError_t rmsnorm_bwd<bf16>(const bf16*, const float*, const bf16*, bf16*, int64_t, int, int, hipStream_t);
template hipError_t dz_from_logits<float>(const float*, float*, int64_t, int, int, const float2*, int, const float*,
                                          const int32_t*, const float*, const float*, hipStream_t);
template hipError_t dz_from_logits<bf16>(const bf16*, bf16*, int64_t, int, int, const float2*, int, const float*,
                                         const int32_t*, const float*, const float*, hipStream_t);
template hipError_t attn_delta<float>(const AttnDesc&, hipStream_t);
template hipError_t attn_delta<bf16>(const AttnDesc&, hipStream_t);

hipError_t rope_table(float2* tab, int T, int Q, float base, hipStream_t s) {
  return rope_table_at(tab, 0, T, Q, base, s);
}
hipError_t rope_table_at(float2* tab, int t0, int T, int Q, float base, hipStream_t s) {
  const int64_t n = (int64_t)T * (Q / 2);
  k_rope_table<<<nblocks(n, 256), 256, 0, s>>>(tab, t0, T, Q, (double)base);
  return hipGetLastError();
}
hipError_t ce_combine(const float2* part, int nblk, const float* ztgt, const int32_t* tgt, float* lse, float* ce,
                      int64_t rows, int V, hipStream_t s) {
  k_ce_combine<<<nblocks(rows, 4), 256, 0, s>>>(part, nblk, ztgt, tgt, lse, ce, rows, V);
  return hipGetLastError();
}
template <typename T>
hipError_t dz_from_logits(const T* z, T* dz, int64_t rows, int V, int tile_w, const float2* part, int nblk,
                          const float* ztgt, const int32_t* tgt, const float* lse, const float* rs, hipStream_t s) {
  constexpr int VN = Vec<T>::n;
  if (rows <= 0 || V <= 0 || V % VN || tile_w <= 0 || tile_w % VN || V % tile_w || V / tile_w != nblk)
    return hipErrorInvalidValue;
  const int bpr = (V / VN + 511) / 512;
  if (rows * bpr > INT32_MAX) return hipErrorInvalidValue;
  k_dz_from_logits<T><<<(unsigned)(rows * bpr), 256, 0, s>>>(z, dz, V, bpr, tile_w, part, nblk, ztgt, tgt, lse,
                                                              rs);
  return hipGetLastError();
}
hipError_t count_valid(const int32_t* tgt, int64_t n, float* inv, hipStream_t s) {
  k_count_valid<<<1, 1024, 0, s>>>(tgt, n, inv);
  return hipGetLastError();
}
hipError_t row_scale(const int32_t* tgt, const float* w, const float* inv_nvalid, int64_t n, int V, float* out,
                     hipStream_t s) {
  k_row_scale<<<nblocks(n, 256), 256, 0, s>>>(tgt, w, inv_nvalid, n, V, out);
  return hipGetLastError();
}
hipError_t weighted_loss(const float* ce, const int32_t* tgt, const float* w, int64_t n, double* out, hipStream_t s) {
  k_weighted_loss<<<1, 1024, 0, s>>>(ce, tgt, w, n, out);
  return hipGetLastError();
}
hipError_t loss_bpb(const float* ce, const int32_t* tgt, const int32_t* bytes, int64_t n, int V, double* out,
                    hipStream_t s) {
  k_loss_bpb<<<1, 1024, 0, s>>>(ce, tgt, bytes, n, V, out);
  return hipGetLastError();
}
hipError_t splitk_reduce(const float* part, int splits, int64_t n, float* out, int beta, hipStream_t s) {
  if (n % 4) return hipErrorInvalidValue;
  const int64_t n4 = n / 4;
  k_splitk_reduce<<<nblocks(n4, 256), 256, 0, s>>>((const float4*)part, splits, n4, (float4*)out, beta);
  return hipGetLastError();
}
hipError_t transpose_bf16(const bf16* in, int64_t rows, int64_t cols, bf16* out, hipStream_t s) {
  if (rows <= 0 || cols <= 0 || rows % 8 || cols % 8 || (rows + 63) / 64 > 65535) return hipErrorInvalidValue;
  dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows + 63) / 64));
  k_transpose16<<<grid, 256, 0, s>>>((const uint16_t*)in, rows, cols, (uint16_t*)out);
  return hipGetLastError();
}
hipError_t fill_f32(float* p, int64_t n, float v, hipStream_t s) {
  k_fill_f32<<<nblocks(n, 256), 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}
hipError_t copy_bytes(void* dst, const void* src, size_t n, hipStream_t s) {
  return hipMemcpyAsync(dst, src, n, hipMemcpyDeviceToDevice, s);
}

}  // namespace nc
