// Pooled block estimators and the SICS aggregation score (gfx950).
//
// Pooled estimate (SPADE notes' MEAN / DSA summaries; VEDA key design 1,
// TripPool, with the head-specific projections taken as the identity): each
// block of b reordered tokens is summarised by the mean of its valid tokens
// (MEAN) or by their mean, channel-wise maximum and minimum (TRIP, 3d
// values); S[I, J] = desc_q(I) . desc_k(J) / sqrt(d'), P[I, :] = softmax_J S.
//   pool_desc_kernel:  one workgroup per (block, head, Q or K); each thread
//                      owns eight channels of one row group (16-byte loads), in
//                      float32 from the bf16 rows (Q read in token order
//                      through the permutation).
//   pooled_scores_kernel: one workgroup per kTileI query blocks of a head; their
//                      descriptors sit in LDS and every key descriptor read
//                      from L2 serves all of them (scores into p_imp).
//   row_softmax_kernel: one wavefront per row, in place.
// SICS (SPADE notes, scheme generation): per block, || sum_i q_i / |q_i| ||^2.
//   sics_block_kernel: one pass over the block's rows, a group of D / 8
//                      threads per row (16-byte loads, eight channels per
//                      thread): the row's norm by a butterfly over the group,
//                      then the channel sums of the normalised rows, then the
//                      square.
//   sics_head_kernel:  the head's sum over its blocks in a fixed order.
#include <cmath>

#include "common.h"
#include "../launch.h"

namespace dbs {
namespace {

constexpr int kPoolThreads = 256;


// Element offset of reordered row r of (bi, hh): through the permutation
// into token-order storage (x_tok) or straight into reordered rows.
struct RowSrc {
  const void* x;
  int64_t sb, sn, sh;        // element strides of token-order storage (perm set)
  const int32_t* perm;       // nullable: x holds reordered rows [B, Hh, Npad, D]
  int perm_h_stride;
  int f32;
  __device__ __forceinline__ int64_t row_off(int bi, int hh, int r, int Hh, int Npad, int N, int D) const {
    if (perm == nullptr) return (((int64_t)bi * Hh + hh) * Npad + r) * D;
    int t = perm[(int64_t)hh * perm_h_stride + r];
    t = t < 0 ? 0 : (t >= N ? N - 1 : t);
    return bi * sb + (int64_t)t * sn + hh * sh;
  }
};

// Eight consecutive channels of one row (16 bytes of bf16, or 32 of float32
// rounded to bf16) as float32.
__device__ __forceinline__ void load8(const void* base, int64_t off, bool f32, float (&x)[8]) {
  if (f32) {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + off);
    const float4 a = p[0], c = p[1];
    const float v[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = bf16_bits_to_f32(f32_to_bf16_bits(v[e]));
  } else {
    const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + off);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(u[e] << 16);
      x[2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
    }
  }
}

// Each thread owns 8 channels of one row group (16-byte loads; D / 8 threads
// cover a row), then the row groups are combined in LDS.
template <int D>
__global__ __launch_bounds__(kPoolThreads) void pool_desc_kernel(RowSrc q, RowSrc k, PooledArgs a, float* desc) {
  constexpr int kCpr = D / 8;                     // threads per row
  constexpr int kGroups = kPoolThreads / kCpr;    // row groups
  __shared__ float red[3][kGroups][D];
  const int I = blockIdx.x, bh = blockIdx.y, which = blockIdx.z;   // 0: Q, 1: K
  const int bi = bh / a.Hh, hh = bh % a.Hh;
  const RowSrc& src = which == 0 ? q : k;
  const int c0 = (threadIdx.x % kCpr) * 8, grp = threadIdx.x / kCpr;
  const int r0 = I * a.b, n = min(a.b, a.N - r0);
  float s[8], mx[8], mn[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    s[e] = 0.f;
    mx[e] = -INFINITY;
    mn[e] = INFINITY;
  }
  for (int r = grp; r < n; r += kGroups) {
    float x[8];
    load8(src.x, src.row_off(bi, hh, r0 + r, a.Hh, a.Npad, a.N, D) + c0, src.f32, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s[e] += x[e];
      mx[e] = fmaxf(mx[e], x[e]);
      mn[e] = fminf(mn[e], x[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    red[0][grp][c0 + e] = s[e];
    red[1][grp][c0 + e] = mx[e];
    red[2][grp][c0 + e] = mn[e];
  }
  __syncthreads();
  if (threadIdx.x < D) {
    const int c = threadIdx.x;
    float ts = 0.f, tx = -INFINITY, tn = INFINITY;
    for (int g = 0; g < kGroups; ++g) {
      ts += red[0][g][c];
      tx = fmaxf(tx, red[1][g][c]);
      tn = fminf(tn, red[2][g][c]);
    }
    const int L = a.kind == 0 ? D : 3 * D;
    float* o = desc + (((int64_t)which * a.B * a.Hh + bh) * a.nb + I) * L;
    o[c] = ts / (float)n;
    if (a.kind != 0) {
      o[D + c] = tx;
      o[2 * D + c] = tn;
    }
  }
}

// kTileI query blocks per workgroup: 16 for mean descriptors (key reads
// dominate), 4 for the 3d-long TRIP descriptors (the products dominate, and
// four times as many workgroups fill the chip): 55 and 84 us on the Wan shape,
// against 103 and 117 us the other way round.
template <int L>
__global__ __launch_bounds__(kPoolThreads) void pooled_scores_kernel(const float* __restrict__ desc, PooledArgs a,
                                                                     float inv_sqrt_l) {
  constexpr int kTileI = L <= 128 ? 16 : 4;
  __shared__ float qd[kTileI][L];
  const int I0 = blockIdx.x * kTileI, bh = blockIdx.y;
  const int nI = min(kTileI, a.nb - I0);
  const float* dq = desc + ((int64_t)bh * a.nb + I0) * L;
  const float* dk = desc + ((int64_t)(a.B * a.Hh) + bh) * a.nb * L;
  for (int t = threadIdx.x; t < kTileI * L; t += kPoolThreads) qd[t / L][t % L] = t / L < nI ? dq[t] : 0.f;
  __syncthreads();
  for (int J = threadIdx.x; J < a.nb; J += kPoolThreads) {
    float acc[kTileI];
#pragma unroll
    for (int i = 0; i < kTileI; ++i) acc[i] = 0.f;
    const float4* kr = reinterpret_cast<const float4*>(dk + (int64_t)J * L);
    for (int l4 = 0; l4 < L / 4; ++l4) {
      const float4 kv = kr[l4];
#pragma unroll
      for (int i = 0; i < kTileI; ++i) {
        acc[i] = __builtin_fmaf(qd[i][4 * l4 + 0], kv.x, acc[i]);
        acc[i] = __builtin_fmaf(qd[i][4 * l4 + 1], kv.y, acc[i]);
        acc[i] = __builtin_fmaf(qd[i][4 * l4 + 2], kv.z, acc[i]);
        acc[i] = __builtin_fmaf(qd[i][4 * l4 + 3], kv.w, acc[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < kTileI; ++i)
      if (i < nI) a.p_imp[((int64_t)bh * a.nb + I0 + i) * a.nb + J] = acc[i] * inv_sqrt_l;
  }
}

// One wavefront per row of nb scores, in place: max, sum of exponentials, scale.
__global__ __launch_bounds__(256) void row_softmax_kernel(float* p, int nb, int64_t rows) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  float* r = p + row * nb;
  float m = -INFINITY;
  for (int j = lane; j < nb; j += 64) m = fmaxf(m, r[j]);
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  float s = 0.f;
  for (int j = lane; j < nb; j += 64) s += __expf(r[j] - m);
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  const float inv = 1.f / s;
  for (int j = lane; j < nb; j += 64) r[j] = __expf(r[j] - m) * inv;
}

// Candidate scoring (dbs_sics_choose): blockIdx.z = candidate * tensors + tensor
// picks the tensor (Q, then K) and the candidate's permutation; the block's
// score goes to a.sics[(z * B * Hh + bh) * nb + I].
template <int D>
__global__ __launch_bounds__(kPoolThreads) void sics_block_kernel(RowSrc q, SicsArgs a) {
  constexpr int kCpr = D / 8;                     // threads per row (8 channels, 16 bytes each)
  constexpr int kGroups = kPoolThreads / kCpr;
  __shared__ float red[kGroups][D];
  const int I = blockIdx.x, bh = blockIdx.y, z = blockIdx.z;
  const int bi = bh / a.Hh, hh = bh % a.Hh;
  const int r0 = I * a.b, n = min(a.b, a.N - r0);
  if (a.n_cand > 0) {   // candidate z / tensors, tensor z % tensors
    const int t = z % a.tensors;
    if (t == 1) q.x = a.k;
    q.perm = a.perms + (int64_t)(z / a.tensors) * a.N;
    q.perm_h_stride = 0;
  }
  float* out = a.sics + (int64_t)z * a.B * a.Hh * a.nb;
  // One pass over the rows: the kCpr threads of a row group read its 16-byte
  // chunks together, form the squared norm by a butterfly over those lanes,
  // and add the normalised chunk to their channel sums.
  const int c0 = (threadIdx.x % kCpr) * 8, grp = threadIdx.x / kCpr;
  float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int r = grp; r < n; r += kGroups) {
    float x[8];
    load8(q.x, q.row_off(bi, hh, r0 + r, a.Hh, a.Npad, a.N, D) + c0, q.f32, x);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(x[e], x[e], ss);
#pragma unroll
    for (int o = kCpr / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
    const float w = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = __builtin_fmaf(x[e], w, s[e]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[grp][c0 + e] = s[e];
  __syncthreads();
  if (threadIdx.x < 64) {
    float acc = 0.f;
    for (int cc = threadIdx.x; cc < D; cc += 64) {
      float t = 0.f;
      for (int g = 0; g < kGroups; ++g) t += red[g][cc];
      acc = __builtin_fmaf(t, t, acc);
    }
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (threadIdx.x == 0) out[(int64_t)bh * a.nb + I] = acc;
  }
}

__global__ __launch_bounds__(64) void sics_head_kernel(SicsArgs a) {
  const int bh = blockIdx.x, lane = threadIdx.x;
  float s = 0.f;
  for (int I = lane; I < a.nb; I += 64) s += a.sics[(int64_t)bh * a.nb + I];
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if (lane == 0) a.as[bh] = s;
}

// Per (batch, head): each candidate's aggregation score (the sum over the
// tensors and blocks of the block scores, lanes over blocks in a fixed order
// and a fixed butterfly), and the candidate with the largest score (the
// smallest index among equal ones).
__global__ __launch_bounds__(64) void sics_choose_kernel(SicsArgs a) {
  const int bh = blockIdx.x, lane = threadIdx.x;
  const int64_t per = (int64_t)a.B * a.Hh * a.nb;
  float best = -INFINITY;
  int arg = 0;
  for (int c = 0; c < a.n_cand; ++c) {
    float s = 0.f;
    for (int t = 0; t < a.tensors; ++t) {
      const float* blk = a.sics + (int64_t)(c * a.tensors + t) * per + (int64_t)bh * a.nb;
      for (int I = lane; I < a.nb; I += 64) s += blk[I];
    }
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    if (lane == 0) a.as[(int64_t)c * a.B * a.Hh + bh] = s;
    if (c == 0 || s > best) { best = s; arg = c; }
  }
  if (lane == 0) a.choice[bh] = arg;
}

RowSrc make_src(const TokIO& t, const void* rows) {
  RowSrc s{};
  if (t.perm != nullptr) {
    s.x = t.q; s.sb = t.qsb; s.sn = t.qsn; s.sh = t.qsh; s.perm = t.perm; s.perm_h_stride = t.perm_h_stride;
    s.f32 = t.q_f32;
  } else {
    s.x = rows;
  }
  return s;
}

}  // namespace

size_t pooled_workspace_bytes(int B, int Hh, int nb, int d) { return (size_t)2 * B * Hh * nb * 3 * d * 4; }

hipError_t launch_pooled(const PooledArgs& a) {
  const RowSrc q = make_src(a.tok, a.q_r);
  RowSrc k{};
  k.x = a.k_r;
  const int BH = a.B * a.Hh;
  float* desc = reinterpret_cast<float*>(a.workspace);
  const dim3 pg((unsigned)a.nb, (unsigned)BH, 2);
  if (a.d == 64) hipLaunchKernelGGL(pool_desc_kernel<64>, pg, dim3(kPoolThreads), 0, a.stream, q, k, a, desc);
  else hipLaunchKernelGGL(pool_desc_kernel<128>, pg, dim3(kPoolThreads), 0, a.stream, q, k, a, desc);
  const int L = (a.kind == 0 ? 1 : 3) * a.d;
  const float isl = (float)(1.0 / std::sqrt((double)L));
  const int tile = L <= 128 ? 16 : 4;
  const dim3 sg((unsigned)((a.nb + tile - 1) / tile), (unsigned)BH);
  switch (L) {
    case 64: hipLaunchKernelGGL(pooled_scores_kernel<64>, sg, dim3(kPoolThreads), 0, a.stream, desc, a, isl); break;
    case 128: hipLaunchKernelGGL(pooled_scores_kernel<128>, sg, dim3(kPoolThreads), 0, a.stream, desc, a, isl); break;
    case 192: hipLaunchKernelGGL(pooled_scores_kernel<192>, sg, dim3(kPoolThreads), 0, a.stream, desc, a, isl); break;
    default: hipLaunchKernelGGL(pooled_scores_kernel<384>, sg, dim3(kPoolThreads), 0, a.stream, desc, a, isl); break;
  }
  const int64_t rows = (int64_t)BH * a.nb;
  hipLaunchKernelGGL(row_softmax_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, a.stream, a.p_imp, a.nb,
                     rows);
  return hipGetLastError();
}

hipError_t launch_sics(const SicsArgs& a) {
  const RowSrc q = make_src(a.tok, a.q_r);
  const unsigned zs = a.n_cand > 0 ? (unsigned)(a.n_cand * a.tensors) : 1u;
  const dim3 g((unsigned)a.nb, (unsigned)(a.B * a.Hh), zs);
  if (a.d == 64) hipLaunchKernelGGL(sics_block_kernel<64>, g, dim3(kPoolThreads), 0, a.stream, q, a);
  else hipLaunchKernelGGL(sics_block_kernel<128>, g, dim3(kPoolThreads), 0, a.stream, q, a);
  if (a.n_cand > 0)
    hipLaunchKernelGGL(sics_choose_kernel, dim3((unsigned)(a.B * a.Hh)), dim3(64), 0, a.stream, a);
  else
    hipLaunchKernelGGL(sics_head_kernel, dim3((unsigned)(a.B * a.Hh)), dim3(64), 0, a.stream, a);
  return hipGetLastError();
}

}  // namespace dbs
