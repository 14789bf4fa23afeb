// Token reorder / inverse reorder / ASA_G mean-pool kernels (gfx950).
//
// Video-BLADE "Preprocessing": Q, K, V are gathered into curve (or cuboid)
// order before they are cut into blocks; the attention output is scattered
// back to token order afterwards.  Video-BLADE "Step 2.2 (2)": the global
// tokens are means of n consecutive reordered tokens.
//
// All three are pure data movement and HBM-bound.  Each thread moves whole
// 16-byte chunks; rows of one token are 2*d bytes contiguous on both sides,
// so every wave touches a handful of contiguous 128-256 byte segments.
#include "common.h"
#include "../launch.h"

namespace dbs {
namespace {

constexpr int kThreads = 256;

// Permutation entries are clamped to [0, N) so that a malformed permutation
// can never address outside the token buffers.
__device__ __forceinline__ int clamp_tok(int p, int N) { return p < 0 ? 0 : (p >= N ? N - 1 : p); }

// Column of token offset t inside a tiles-transposed tile: bits 2 and 3 of t
// exchanged, i.e. each group of 16 tokens is stored in the order 0-3, 8-11,
// 4-7, 12-15 (an involution).  The attention kernel relies on this order.
__device__ __forceinline__ int tile_col(int t) {
  return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1);
}

template <typename T> struct Vec8;
template <> struct Vec8<__bf16> {
  uint4 v;
  __device__ __forceinline__ void load(const __bf16* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void to_bf16(uint4& o) const { o = v; }
};
template <> struct Vec8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ __forceinline__ void to_bf16(uint4& o) const {
    o.x = pack_bf16x2(a.x, a.y);
    o.y = pack_bf16x2(a.z, a.w);
    o.z = pack_bf16x2(b.x, b.y);
    o.w = pack_bf16x2(b.z, b.w);
  }
};

// y rows layout: y[b, h, i, :] = x[b, perm[i], h, :] (i < N), zero rows after N.
// One workgroup covers 64 rows of one (b, h); D/8 threads per row.
template <typename Tin, typename Tout, int D>
__global__ __launch_bounds__(kThreads) void reorder_rows_kernel(
    const Tin* __restrict__ x, int64_t sb, int64_t sn, int64_t sh, Tout* __restrict__ y,
    const int32_t* __restrict__ perm, int perm_h_stride, int Hh, int N, int Npad) {
  constexpr int kChunks = D / 8;
  constexpr int kRowsPerPass = kThreads / kChunks;
  constexpr int kRowsPerBlock = 64;
  const int h = blockIdx.y, bi = blockIdx.z;
  const int c = threadIdx.x % kChunks;
  const int64_t ybase = ((int64_t)bi * Hh + h) * Npad;
  const int32_t* ph = perm + (int64_t)h * perm_h_stride;
#pragma unroll
  for (int pass = 0; pass < kRowsPerBlock / kRowsPerPass; ++pass) {
    const int i = blockIdx.x * kRowsPerBlock + pass * kRowsPerPass + threadIdx.x / kChunks;
    if (i >= Npad) break;
    Tout* dst = y + (ybase + i) * D + 8 * c;
    if (i < N) {
      const Tin* src = x + bi * sb + (int64_t)clamp_tok(ph[i], N) * sn + (int64_t)h * sh + 8 * c;
      if constexpr (sizeof(Tin) == sizeof(Tout)) {
        if constexpr (sizeof(Tin) == 2) {
          *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
        } else {
          reinterpret_cast<float4*>(dst)[0] = reinterpret_cast<const float4*>(src)[0];
          reinterpret_cast<float4*>(dst)[1] = reinterpret_cast<const float4*>(src)[1];
        }
      } else {
        Vec8<Tin> v;
        v.load(src);
        uint4 o;
        v.to_bf16(o);
        *reinterpret_cast<uint4*>(dst) = o;
      }
    } else {
      if constexpr (sizeof(Tout) == 2) {
        *reinterpret_cast<uint4*>(dst) = make_uint4(0, 0, 0, 0);
      } else {
        reinterpret_cast<float4*>(dst)[0] = make_float4(0, 0, 0, 0);
        reinterpret_cast<float4*>(dst)[1] = make_float4(0, 0, 0, 0);
      }
    }
  }
}

// y tiles-transposed layout: y[b, h, J, e, tile_col(t)] = x[b, perm[J*BLK + t], h, e].
// One workgroup per (tile J, h, b); thread (c, tg) gathers the 8 tokens that
// land in columns 8tg..8tg+7 for 8 channels, transposes the block in
// registers and writes 8 channel rows of 16 bytes.
template <typename Tin, int D, int BLK>
__global__ __launch_bounds__((D / 8) * (BLK / 8)) void reorder_tiles_t_kernel(
    const Tin* __restrict__ x, int64_t sb, int64_t sn, int64_t sh, __bf16* __restrict__ y,
    const int32_t* __restrict__ perm, int perm_h_stride, int Hh, int N, int nb) {
  const int J = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
  const int c = threadIdx.x % (D / 8);   // channel chunk: channels 8c..8c+7
  const int tg = threadIdx.x / (D / 8);  // token group: tokens 8tg..8tg+7 of the tile
  const int32_t* ph = perm + (int64_t)h * perm_h_stride;
  uint32_t w[8][4];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int i = J * BLK + tile_col(8 * tg + e);
    uint4 o = make_uint4(0, 0, 0, 0);
    if (i < N) {
      Vec8<Tin> v;
      v.load(x + bi * sb + (int64_t)clamp_tok(ph[i], N) * sn + (int64_t)h * sh + 8 * c);
      v.to_bf16(o);
    }
    w[e][0] = o.x; w[e][1] = o.y; w[e][2] = o.z; w[e][3] = o.w;
  }
  __bf16* tile = y + (((int64_t)bi * Hh + h) * nb + J) * (int64_t)(D * BLK);
#pragma unroll
  for (int ch = 0; ch < 8; ++ch) {
    // channel 8c+ch of tokens 8tg..8tg+7: half `ch & 1` of word ch/2 of each token
    uint32_t o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t lo = w[2 * p][ch >> 1], hi = w[2 * p + 1][ch >> 1];
      o[p] = (ch & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
    *reinterpret_cast<uint4*>(tile + (int64_t)(8 * c + ch) * BLK + 8 * tg) =
        make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// K and V of one (tile J, head h, batch b) in one workgroup of 2 * (D/8) *
// (BLK/8) threads: the first half gathers V into the tiles-transposed layout
// exactly as reorder_tiles_t_kernel does, the second half gathers the tile's
// BLK rows of K into the rows layout, 8 independent 16-byte chunks per thread
// (rows tg, tg + BLK/8, ... of the tile, channel chunk c).  Both halves share
// the permutation and run the same number of chunks, so a launch over all tiles
// is a whole number of occupancy rounds where the two separate launches were not.
// Global-token outputs of the fused K/V reorder (ASA_G, window n dividing b).
struct PoolOut {
  __bf16* k_g;   // rows [B, Hh, Ngpad, D]
  __bf16* v_g;   // tiles-transposed [B, Hh, Ngpad / b, D, b]
  int n, Ng;
};

// Eight channels 8 cc .. 8 cc + 7 of global token g: a 16-byte k_g row chunk,
// or eight entries of a v_g tile column.
template <int D, int BLK>
__device__ __forceinline__ void pool_store_t(const PoolOut& p, bool v, int64_t bh, int g, int Ngpad, int cc,
                                             const uint32_t (&o)[4]) {
  if (!v) {
    *reinterpret_cast<uint4*>(p.k_g + (bh * Ngpad + g) * D + 8 * cc) = make_uint4(o[0], o[1], o[2], o[3]);
  } else {
    uint16_t* out = reinterpret_cast<uint16_t*>(p.v_g) + bh * (int64_t)Ngpad * D;
    const int64_t base = (int64_t)(g / BLK) * D * BLK + tile_col(g % BLK);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      out[base + (int64_t)(8 * cc + 2 * q) * BLK] = (uint16_t)(o[q] & 0xffffu);
      out[base + (int64_t)(8 * cc + 2 * q + 1) * BLK] = (uint16_t)(o[q] >> 16);
    }
  }
}

template <typename Tin, int D, int BLK, bool POOL>
__global__ __launch_bounds__(2 * (D / 8) * (BLK / 8)) void reorder_kv_kernel(
    const Tin* __restrict__ k, const Tin* __restrict__ v, int64_t sb, int64_t sn, int64_t sh,
    __bf16* __restrict__ k_r, __bf16* __restrict__ v_t, const int32_t* __restrict__ perm,
    int perm_h_stride, int Hh, int N, int nb, PoolOut pool) {
  constexpr int kHalf = (D / 8) * (BLK / 8);
  const int J = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
  const int t = threadIdx.x % kHalf;
  const int c = t % (D / 8);   // channel chunk: channels 8c..8c+7
  const int tg = t / (D / 8);  // token group
  const int32_t* ph = perm + (int64_t)h * perm_h_stride;
  const int64_t bh = (int64_t)bi * Hh + h;
  uint32_t w[8][4];
  // POOL: the tile's K and V rows as bf16, token-major, for the window means
  __shared__ __attribute__((aligned(16))) __bf16 ks[POOL ? BLK : 1][POOL ? D : 8];
  __shared__ __attribute__((aligned(16))) __bf16 vs[POOL ? BLK : 1][POOL ? D : 8];
  if (threadIdx.x < kHalf) {   // wave-uniform: kHalf is a multiple of 64
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = J * BLK + tile_col(8 * tg + e);
      uint4 o = make_uint4(0, 0, 0, 0);
      if (i < N) {
        Vec8<Tin> x;
        x.load(v + bi * sb + (int64_t)clamp_tok(ph[i], N) * sn + (int64_t)h * sh + 8 * c);
        x.to_bf16(o);
      }
      w[e][0] = o.x; w[e][1] = o.y; w[e][2] = o.z; w[e][3] = o.w;
      if constexpr (POOL) {
        uint32_t* row = reinterpret_cast<uint32_t*>(&vs[tile_col(8 * tg + e)][8 * c]);
        row[0] = o.x; row[1] = o.y; row[2] = o.z; row[3] = o.w;
      }
    }
    __bf16* tile = v_t + (bh * nb + J) * (int64_t)(D * BLK);
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) {
      uint32_t o[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t lo = w[2 * p][ch >> 1], hi = w[2 * p + 1][ch >> 1];
        o[p] = (ch & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      *reinterpret_cast<uint4*>(tile + (int64_t)(8 * c + ch) * BLK + 8 * tg) =
          make_uint4(o[0], o[1], o[2], o[3]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = J * BLK + tg + e * (BLK / 8);
      uint4 o = make_uint4(0, 0, 0, 0);
      if (i < N) {
        Vec8<Tin> x;
        x.load(k + bi * sb + (int64_t)clamp_tok(ph[i], N) * sn + (int64_t)h * sh + 8 * c);
        x.to_bf16(o);
      }
      w[e][0] = o.x; w[e][1] = o.y; w[e][2] = o.z; w[e][3] = o.w;
      if constexpr (POOL) {
        uint32_t* row = reinterpret_cast<uint32_t*>(&ks[tg + e * (BLK / 8)][8 * c]);
        row[0] = o.x; row[1] = o.y; row[2] = o.z; row[3] = o.w;
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = J * BLK + tg + e * (BLK / 8);
      *reinterpret_cast<uint4*>(k_r + (bh * nb * BLK + i) * D + 8 * c) =
          make_uint4(w[e][0], w[e][1], w[e][2], w[e][3]);
    }
  }
  if constexpr (POOL) {
    // ASA_G global tokens of this tile's windows (n divides BLK): the same
    // sums as dbs_meanpool_kv, float32 in ascending token order, divided by
    // the window's valid count and rounded to bf16.  Threads of the first half
    // form k_g chunks (8 channels of one window), the second half v_g chunks.
    __syncthreads();
    const int wpt = BLK / pool.n;                 // windows per tile
    const int Ngpad = (pool.Ng + BLK - 1) / BLK * BLK;
    const bool vhalf = threadIdx.x >= kHalf;
    const int u = threadIdx.x % kHalf;
    for (int item = u; item < wpt * (D / 8); item += kHalf) {
      const int wi = item / (D / 8), cc = item % (D / 8);
      const int g = J * wpt + wi;
      float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      const int r = g < pool.Ng ? min(pool.n, N - g * pool.n) : 0;
      for (int e = 0; e < r; ++e) {
        const uint4 x = *reinterpret_cast<const uint4*>(vhalf ? &vs[wi * pool.n + e][8 * cc] : &ks[wi * pool.n + e][8 * cc]);
        const uint32_t xv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] += bf16_bits_to_f32(xv[q] & 0xffffu);
          acc[2 * q + 1] += bf16_bits_to_f32(xv[q] >> 16);
        }
      }
      const float fr = (float)(r > 0 ? r : 1);
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = r > 0 ? pack_bf16x2(acc[2 * q] / fr, acc[2 * q + 1] / fr) : 0u;
      if (g < Ngpad) pool_store_t<D, BLK>(pool, vhalf, bh, g, Ngpad, cc, o);
    }
    // rows past the last tile's windows up to Ngpad are zero
    if (J == nb - 1) {
      for (int item = u; item < (Ngpad - nb * wpt) * (D / 8); item += kHalf) {
        const int g = nb * wpt + item / (D / 8), cc = item % (D / 8);
        const uint32_t z[4] = {0u, 0u, 0u, 0u};
        pool_store_t<D, BLK>(pool, vhalf, bh, g, Ngpad, cc, z);
      }
    }
  }
}

// x[b, perm[i], h, :] = y[b, h, i, :] for i < N (y rows layout, bf16).
template <typename Tout, int D>
__global__ __launch_bounds__(kThreads) void inverse_rows_kernel(
    const __bf16* __restrict__ y, Tout* __restrict__ x, int64_t sb, int64_t sn, int64_t sh,
    const int32_t* __restrict__ perm, int perm_h_stride, int Hh, int N, int Npad) {
  constexpr int kChunks = D / 8;
  constexpr int kRowsPerPass = kThreads / kChunks;
  constexpr int kRowsPerBlock = 64;
  const int h = blockIdx.y, bi = blockIdx.z;
  const int c = threadIdx.x % kChunks;
  const int64_t ybase = ((int64_t)bi * Hh + h) * Npad;
  const int32_t* ph = perm + (int64_t)h * perm_h_stride;
#pragma unroll
  for (int pass = 0; pass < kRowsPerBlock / kRowsPerPass; ++pass) {
    const int i = blockIdx.x * kRowsPerBlock + pass * kRowsPerPass + threadIdx.x / kChunks;
    if (i >= N) break;
    const uint4 v = *reinterpret_cast<const uint4*>(y + (ybase + i) * D + 8 * c);
    Tout* dst = x + bi * sb + (int64_t)clamp_tok(ph[i], N) * sn + (int64_t)h * sh + 8 * c;
    if constexpr (sizeof(Tout) == 2) {
      *reinterpret_cast<uint4*>(dst) = v;
    } else {
      reinterpret_cast<float4*>(dst)[0] = make_float4(bf16_bits_to_f32(v.x & 0xffffu), bf16_bits_to_f32(v.x >> 16),
                                                      bf16_bits_to_f32(v.y & 0xffffu), bf16_bits_to_f32(v.y >> 16));
      reinterpret_cast<float4*>(dst)[1] = make_float4(bf16_bits_to_f32(v.z & 0xffffu), bf16_bits_to_f32(v.z >> 16),
                                                      bf16_bits_to_f32(v.w & 0xffffu), bf16_bits_to_f32(v.w >> 16));
    }
  }
}

// x[b, perm[i], h, :] = y[b, h, i, :] for i < N, float32 rows to float32 (exact copy).
template <int D>
__global__ __launch_bounds__(kThreads) void inverse_rows_f32_kernel(
    const float* __restrict__ y, float* __restrict__ x, int64_t sb, int64_t sn, int64_t sh,
    const int32_t* __restrict__ perm, int perm_h_stride, int Hh, int N, int Npad) {
  constexpr int kChunks = D / 4;
  constexpr int kRowsPerPass = kThreads / kChunks;
  constexpr int kRowsPerBlock = 64;
  const int h = blockIdx.y, bi = blockIdx.z;
  const int c = threadIdx.x % kChunks;
  const int64_t ybase = ((int64_t)bi * Hh + h) * Npad;
  const int32_t* ph = perm + (int64_t)h * perm_h_stride;
#pragma unroll
  for (int pass = 0; pass < kRowsPerBlock / kRowsPerPass; ++pass) {
    const int i = blockIdx.x * kRowsPerBlock + pass * kRowsPerPass + threadIdx.x / kChunks;
    if (i >= N) break;
    const float4 v = *reinterpret_cast<const float4*>(y + (ybase + i) * D + 4 * c);
    *reinterpret_cast<float4*>(x + bi * sb + (int64_t)clamp_tok(ph[i], N) * sn + (int64_t)h * sh + 4 * c) = v;
  }
}

// Global K tokens: k_g[b, h, g, :] = mean of rows g*n .. g*n+r-1 (rows layout).
template <int D>
__global__ __launch_bounds__(kThreads) void meanpool_k_kernel(
    const __bf16* __restrict__ k_r, __bf16* __restrict__ k_g, int Hh, int N, int Npad, int n,
    int Ng, int Ngpad) {
  constexpr int kChunks = D / 8;
  const int h = blockIdx.y, bi = blockIdx.z;
  const int g = blockIdx.x * (kThreads / kChunks) + threadIdx.x / kChunks;
  const int c = threadIdx.x % kChunks;
  if (g >= Ngpad) return;
  const int64_t bh = (int64_t)bi * Hh + h;
  uint4 o = make_uint4(0, 0, 0, 0);
  if (g < Ng) {
    const int r = min(n, N - g * n);
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int e = 0; e < r; ++e) {
      const uint4 v = *reinterpret_cast<const uint4*>(k_r + (bh * Npad + (int64_t)g * n + e) * D + 8 * c);
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += bf16_bits_to_f32(wv[q] & 0xffffu);
        acc[2 * q + 1] += bf16_bits_to_f32(wv[q] >> 16);
      }
    }
    const float fr = (float)r;
    o.x = pack_bf16x2(acc[0] / fr, acc[1] / fr);
    o.y = pack_bf16x2(acc[2] / fr, acc[3] / fr);
    o.z = pack_bf16x2(acc[4] / fr, acc[5] / fr);
    o.w = pack_bf16x2(acc[6] / fr, acc[7] / fr);
  }
  *reinterpret_cast<uint4*>(k_g + (bh * Ngpad + g) * D + 8 * c) = o;
}

// Global V tokens from the tiles-transposed V: thread per (g, channel e).
template <int D, int BLK>
__global__ __launch_bounds__(kThreads) void meanpool_v_kernel(
    const __bf16* __restrict__ v_t, __bf16* __restrict__ v_g, int Hh, int N, int nb, int n,
    int Ng, int Ngpad) {
  const int h = blockIdx.y, bi = blockIdx.z;
  const int idx = blockIdx.x * kThreads + threadIdx.x;   // over Ngpad * D, g fastest
  if (idx >= Ngpad * D) return;
  const int g = idx % Ngpad, e = idx / Ngpad;
  const int64_t bh = (int64_t)bi * Hh + h;
  float acc = 0.f;
  if (g < Ng) {
    const int r = min(n, N - g * n);
    const uint16_t* base = reinterpret_cast<const uint16_t*>(v_t) + bh * (int64_t)nb * D * BLK;
    for (int t = 0; t < r; ++t) {
      const int i = g * n + t;
      acc += bf16_bits_to_f32(base[(int64_t)(i / BLK) * D * BLK + (int64_t)e * BLK + tile_col(i % BLK)]);
    }
    acc = acc / (float)r;
  }
  const int ngt = Ngpad / BLK;
  uint16_t* out = reinterpret_cast<uint16_t*>(v_g) + bh * (int64_t)ngt * D * BLK;
  out[(int64_t)(g / BLK) * D * BLK + (int64_t)e * BLK + tile_col(g % BLK)] =
      (uint16_t)(g < Ng ? f32_to_bf16_bits(acc) : 0u);
}

template <typename Tin, typename Tout, int D>
hipError_t launch_rows(const ReorderArgs& a) {
  dim3 grid((a.Npad + 63) / 64, a.Hh, a.B);
  hipLaunchKernelGGL((reorder_rows_kernel<Tin, Tout, D>), grid, dim3(kThreads), 0, a.stream,
                     (const Tin*)a.x, a.sb, a.sn, a.sh, (Tout*)a.y, a.perm, a.perm_h_stride, a.Hh,
                     a.N, a.Npad);
  return hipGetLastError();
}

template <typename Tin, int D, int BLK>
hipError_t launch_tiles(const ReorderArgs& a) {
  dim3 grid(a.Npad / BLK, a.Hh, a.B);
  hipLaunchKernelGGL((reorder_tiles_t_kernel<Tin, D, BLK>), grid, dim3((D / 8) * (BLK / 8)), 0,
                     a.stream, (const Tin*)a.x, a.sb, a.sn, a.sh, (__bf16*)a.y, a.perm,
                     a.perm_h_stride, a.Hh, a.N, a.Npad / BLK);
  return hipGetLastError();
}

template <typename Tin, int D, int BLK>
hipError_t launch_kv(const ReorderArgs& a) {
  dim3 grid(a.Npad / BLK, a.Hh, a.B);
  PoolOut pool{(__bf16*)a.k_g, (__bf16*)a.v_g, a.n_pool, a.n_pool > 0 ? (a.N + a.n_pool - 1) / a.n_pool : 0};
  if (a.k_g != nullptr)
    hipLaunchKernelGGL((reorder_kv_kernel<Tin, D, BLK, true>), grid, dim3(2 * (D / 8) * (BLK / 8)), 0,
                       a.stream, (const Tin*)a.x, (const Tin*)a.x2, a.sb, a.sn, a.sh, (__bf16*)a.y,
                       (__bf16*)a.y2, a.perm, a.perm_h_stride, a.Hh, a.N, a.Npad / BLK, pool);
  else
    hipLaunchKernelGGL((reorder_kv_kernel<Tin, D, BLK, false>), grid, dim3(2 * (D / 8) * (BLK / 8)), 0,
                       a.stream, (const Tin*)a.x, (const Tin*)a.x2, a.sb, a.sn, a.sh, (__bf16*)a.y,
                       (__bf16*)a.y2, a.perm, a.perm_h_stride, a.Hh, a.N, a.Npad / BLK, pool);
  return hipGetLastError();
}

template <typename Tin, int D>
hipError_t dispatch_kv_b(const ReorderArgs& a) {
  return a.b == 64 ? launch_kv<Tin, D, 64>(a) : launch_kv<Tin, D, 128>(a);
}

template <typename Tin, int D>
hipError_t dispatch_tiles_b(const ReorderArgs& a) {
  return a.b == 64 ? launch_tiles<Tin, D, 64>(a) : launch_tiles<Tin, D, 128>(a);
}

template <int D>
hipError_t dispatch_reorder_d(const ReorderArgs& a) {
  const bool in_f32 = a.x_f32, out_f32 = a.y_f32;
  if (a.tiles_t) return in_f32 ? dispatch_tiles_b<float, D>(a) : dispatch_tiles_b<__bf16, D>(a);
  if (in_f32 && out_f32) return launch_rows<float, float, D>(a);
  if (in_f32) return launch_rows<float, __bf16, D>(a);
  return launch_rows<__bf16, __bf16, D>(a);
}

template <int D>
hipError_t dispatch_inverse_d(const ReorderArgs& a) {
  dim3 grid((a.Npad + 63) / 64, a.Hh, a.B);
  if (a.y_f32) {
    hipLaunchKernelGGL((inverse_rows_f32_kernel<D>), grid, dim3(kThreads), 0, a.stream,
                       (const float*)a.y, (float*)a.x_out, a.sb, a.sn, a.sh, a.perm,
                       a.perm_h_stride, a.Hh, a.N, a.Npad);
  } else if (a.x_f32) {
    hipLaunchKernelGGL((inverse_rows_kernel<float, D>), grid, dim3(kThreads), 0, a.stream,
                       (const __bf16*)a.y, (float*)a.x_out, a.sb, a.sn, a.sh, a.perm,
                       a.perm_h_stride, a.Hh, a.N, a.Npad);
  } else {
    hipLaunchKernelGGL((inverse_rows_kernel<__bf16, D>), grid, dim3(kThreads), 0, a.stream,
                       (const __bf16*)a.y, (__bf16*)a.x_out, a.sb, a.sn, a.sh, a.perm,
                       a.perm_h_stride, a.Hh, a.N, a.Npad);
  }
  return hipGetLastError();
}

template <int D, int BLK>
hipError_t launch_meanpool(const MeanpoolArgs& a) {
  const int Ngpad = (a.Ng + BLK - 1) / BLK * BLK;
  {
    dim3 grid((Ngpad + (kThreads / (D / 8)) - 1) / (kThreads / (D / 8)), a.Hh, a.B);
    hipLaunchKernelGGL((meanpool_k_kernel<D>), grid, dim3(kThreads), 0, a.stream,
                       (const __bf16*)a.k_r, (__bf16*)a.k_g, a.Hh, a.N, a.Npad, a.n, a.Ng, Ngpad);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dim3 grid((Ngpad * D + kThreads - 1) / kThreads, a.Hh, a.B);
  hipLaunchKernelGGL((meanpool_v_kernel<D, BLK>), grid, dim3(kThreads), 0, a.stream,
                     (const __bf16*)a.v_t, (__bf16*)a.v_g, a.Hh, a.N, a.Npad / BLK, a.n, a.Ng,
                     Ngpad);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reorder(const ReorderArgs& a) {
  return a.d == 64 ? dispatch_reorder_d<64>(a) : dispatch_reorder_d<128>(a);
}

hipError_t launch_reorder_kv(const ReorderArgs& a) {
  if (a.d == 64) return a.x_f32 ? dispatch_kv_b<float, 64>(a) : dispatch_kv_b<__bf16, 64>(a);
  return a.x_f32 ? dispatch_kv_b<float, 128>(a) : dispatch_kv_b<__bf16, 128>(a);
}

hipError_t launch_inverse_reorder(const ReorderArgs& a) {
  return a.d == 64 ? dispatch_inverse_d<64>(a) : dispatch_inverse_d<128>(a);
}

hipError_t launch_meanpool(const MeanpoolArgs& a) {
  if (a.d == 64) return a.b == 64 ? launch_meanpool<64, 64>(a) : launch_meanpool<64, 128>(a);
  return a.b == 64 ? launch_meanpool<128, 64>(a) : launch_meanpool<128, 128>(a);
}

}  // namespace dbs
