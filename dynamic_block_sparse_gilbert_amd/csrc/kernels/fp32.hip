// Float32 operand path (gfx950): block importance and block-sparse attention
// on float32 Q, K, V with float32 arithmetic throughout, for workloads stored
// in float32 (Video-BLADE "Step 1" and "Step 2.2" fix no precision of their
// own, so a float32 workload is computed in float32).
//
// Both kernels are plain VALU code: a float32 workload here is the small
// correctness case, and float32 matrix cores would buy little over it.
//
// estimate: one workgroup per (query block I, batch*head).  Each thread holds
//   one sampled query of a chunk of up to kQc in registers and takes one of
//   kKs slices of the keys.  For every chunk:
//   1. the softmax normaliser of each sampled query over all sampled keys
//      (each thread over its slice, online max / sum in the log2 domain, then
//      a merge of the slices), and
//   2. for every key block J (slices stride over J) the largest score of each
//      query against J's sampled keys, turned into
//      max_q exp2(sl2 * t_qJ - lse2_q) (a maximum across the chunk's lanes)
//      and folded into the row held in LDS.
//   Sampling follows the bf16 path: slot t < k_J = min(k, L_J) of block J is
//   row J*b + floor(t * L_J / k_J).
// attention: workgroups of 256 threads, each over 16 rows of a query block;
//   each row is served by 16 threads, each owning D / 16 channels of q and of
//   the output.  The kept blocks' K and V rows stream through LDS in
//   chunks of 32 keys; scores are reduced across the row's threads by lane
//   exchanges, and the online softmax rescales once per chunk.
#include "common.h"
#include "../launch.h"

namespace dbs {
namespace {

constexpr int kF32Threads = 256;
constexpr int kQc = 16;        // sampled queries per chunk (estimate)
constexpr int kKs = kF32Threads / kQc;   // key slices (estimate)
constexpr int kKc = 32;        // keys per LDS chunk (attention)
// Threads per query row (attention): 16 lanes share a row's score by lane
// exchanges, so a 128-row block spreads over eight workgroups (four for 64 rows)
// and each thread's chain per key is short.
constexpr int kF32RowThreads = 16;

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Merge two (max, sum) pairs of log2-domain partial softmax sums.
__device__ __forceinline__ void merge_ml(float& m, float& l, float m2, float l2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;
  l = (m == -INFINITY ? 0.f : l * exp2f(m - M)) + (m2 == -INFINITY ? 0.f : l2 * exp2f(m2 - M));
  m = M;
}

// Dot product of D floats with four independent partial sums.
template <int D>
__device__ __forceinline__ float dot_f32(const float* a, const float (&b)[D]) {
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
  for (int i = 0; i < D; i += 4) {
    s0 = fmaf(a[i], b[i], s0);
    s1 = fmaf(a[i + 1], b[i + 1], s1);
    s2 = fmaf(a[i + 2], b[i + 2], s2);
    s3 = fmaf(a[i + 3], b[i + 3], s3);
  }
  return (s0 + s1) + (s2 + s3);
}

template <int D>
__device__ __forceinline__ void load_row(const float* p, float (&r)[D]) {
#pragma unroll
  for (int i = 0; i < D; i += 4) {
    const float4 v = *reinterpret_cast<const float4*>(p + i);
    r[i] = v.x; r[i + 1] = v.y; r[i + 2] = v.z; r[i + 3] = v.w;
  }
}

// Dot product of a query row held in registers with a row read from memory, in
// four independent partial sums.
template <int D>
__device__ __forceinline__ float dot_row(const float (&q)[D], const float* __restrict__ p) {
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
  for (int i = 0; i < D; i += 4) {
    const float4 v = *reinterpret_cast<const float4*>(p + i);
    s0 = fmaf(q[i], v.x, s0);
    s1 = fmaf(q[i + 1], v.y, s1);
    s2 = fmaf(q[i + 2], v.z, s2);
    s3 = fmaf(q[i + 3], v.w, s3);
  }
  return (s0 + s1) + (s2 + s3);
}

template <int D>
__global__ __launch_bounds__(kF32Threads) void est_f32_kernel(const float* __restrict__ q_r,
                                                              const float* __restrict__ k_r,
                                                              float* __restrict__ p_imp, int N, int Npad, int b,
                                                              int k, int nb, float sl2) {
  extern __shared__ float pacc[];                  // [nb] the row being formed
  __shared__ float red_m[kKs][kQc], red_l[kKs][kQc];
  __shared__ float lse2[kQc];
  const int I = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x;
  // thread (qq, ks): query qq of the chunk, key slice ks; the kQc threads of one
  // slice are consecutive lanes of one wavefront
  const int qq = tid % kQc, ks = tid / kQc;
  const float* kb = k_r + (int64_t)bh * Npad * D;
  const float* qb = q_r + (int64_t)bh * Npad * D;
  const int LI = min(b, N - I * b), kI = min(k, LI);
  const int Lk = N - (nb - 1) * b, kLast = min(k, Lk);   // the last block's length and samples
  // sampled row t of key block J
  auto key_row = [&](int J, int t) {
    const int LJ = J < nb - 1 ? b : Lk, kJ = J < nb - 1 ? k : kLast;
    return kb + (int64_t)(J * b + (t * LJ) / kJ) * D;
  };
  for (int J = tid; J < nb; J += kF32Threads) pacc[J] = 0.f;

  for (int q0 = 0; q0 < kI; q0 += kQc) {
    const bool act = q0 + qq < kI;
    float q[D];
    if (act) {
      load_row<D>(qb + (int64_t)(I * b + ((q0 + qq) * LI) / kI) * D, q);
    } else {
#pragma unroll
      for (int c = 0; c < D; ++c) q[c] = 0.f;
    }
    // 1. this query's normaliser over every sampled key: slice ks takes the
    //    sampled keys r = ks, ks + kKs, ... (online max / sum, log2 domain)
    float m = -INFINITY, l = 0.f;
    for (int r = ks; r < nb * k; r += kKs) {
      const int J = r / k, t = r % k;
      if (t >= (J < nb - 1 ? k : kLast)) continue;
      const float s = dot_row<D>(q, key_row(J, t)) * sl2;
      if (s > m) {
        l = (m == -INFINITY ? 0.f : l * exp2f(m - s)) + 1.f;
        m = s;
      } else {
        l += exp2f(s - m);
      }
    }
    __syncthreads();   // the previous chunk's lse2 readers are done
    red_m[ks][qq] = m;
    red_l[ks][qq] = l;
    __syncthreads();
    if (tid < kQc) {
      float M = red_m[0][tid], L = red_l[0][tid];
      for (int w = 1; w < kKs; ++w) merge_ml(M, L, red_m[w][tid], red_l[w][tid]);
      lse2[tid] = M + log2f(L);
    }
    __syncthreads();
    // 2. per key block J (slice ks takes J = ks, ks + kKs, ...): the largest
    //    score of this query against J's samples, as exp2(sl2 * t_qJ - lse2_q),
    //    maximised over the chunk's queries and folded into the row
    const float lq = lse2[qq];
    for (int J = ks; J < nb; J += kKs) {
      const int kJ = J < nb - 1 ? k : kLast;
      float tm = -INFINITY;
      for (int t = 0; t < kJ; ++t) tm = fmaxf(tm, dot_row<D>(q, key_row(J, t)) * sl2);
      float p = act ? exp2f(tm - lq) : 0.f;
#pragma unroll
      for (int off = 1; off < kQc; off <<= 1) p = fmaxf(p, xor_shfl(p, off));
      if (qq == 0) pacc[J] = fmaxf(pacc[J], p);
    }
  }
  __syncthreads();
  float* prow = p_imp + ((int64_t)bh * nb + I) * nb;
  for (int J = tid; J < nb; J += kF32Threads) prow[J] = pacc[J];
}

template <int D, int BLK>
__global__ __launch_bounds__(kF32Threads) void attn_f32_kernel(
    const float* __restrict__ q_r, const float* __restrict__ k_r, const float* __restrict__ v_r,
    const int32_t* __restrict__ kv_count, const int32_t* __restrict__ kv_idx, const int32_t* __restrict__ order,
    float* __restrict__ o_r, float* __restrict__ lse, int N, int Npad, int nb, int rows_total, float sl2) {
  constexpr int G = kF32RowThreads;      // threads per query row
  constexpr int C = D / G;               // channels per thread
  constexpr int R = kF32Threads / G;     // query rows per workgroup
  constexpr int kSub = BLK / R;          // workgroups per query block
  __shared__ float Ks[kKc][D + 4];
  __shared__ float Vs[kKc][D + 4];
  const int tid = threadIdx.x;
  const int sub = blockIdx.x % kSub;
  int row = blockIdx.x / kSub;
  if (order != nullptr) row = clampi(order[row], 0, rows_total - 1);
  const int bh = row / nb, I = row % nb;
  const int r = tid / G, part = tid % G;
  const int qi = I * BLK + sub * R + r;
  const bool qok = qi < N;
  float q[C], o[C];
  {
    const float* qp = q_r + ((int64_t)bh * Npad + (qok ? qi : 0)) * D + part * C;
#pragma unroll
    for (int c = 0; c < C; c += 4) {
      const float4 v = qok ? *reinterpret_cast<const float4*>(qp + c) : make_float4(0.f, 0.f, 0.f, 0.f);
      q[c] = v.x; q[c + 1] = v.y; q[c + 2] = v.z; q[c + 3] = v.w;
    }
  }
#pragma unroll
  for (int c = 0; c < C; ++c) o[c] = 0.f;
  float m = -INFINITY, l = 0.f;
  const float* kb = k_r + (int64_t)bh * Npad * D;
  const float* vb = v_r + (int64_t)bh * Npad * D;
  const int cnt = clampi(kv_count[row], 0, nb);
  const int32_t* list = kv_idx + (int64_t)row * nb;
  for (int e = 0; e < cnt; ++e) {
    const int J = list[e];
    if (J < 0 || J >= nb) continue;        // uniform across the workgroup
    const int LJ = min(BLK, N - J * BLK);
    for (int c0 = 0; c0 < LJ; c0 += kKc) {
      __syncthreads();
      for (int u = tid; u < kKc * D / 4; u += kF32Threads) {
        const int kk = u / (D / 4), c = (u % (D / 4)) * 4;
        const bool ok = c0 + kk < LJ;
        const int64_t src = (int64_t)(J * BLK + c0 + kk) * D + c;
        const float4 kv = ok ? *reinterpret_cast<const float4*>(kb + src) : make_float4(0.f, 0.f, 0.f, 0.f);
        const float4 vv = ok ? *reinterpret_cast<const float4*>(vb + src) : make_float4(0.f, 0.f, 0.f, 0.f);
        *reinterpret_cast<float4*>(&Ks[kk][c]) = kv;
        *reinterpret_cast<float4*>(&Vs[kk][c]) = vv;
      }
      __syncthreads();
      float s[kKc];
      float mx = -INFINITY;
#pragma unroll
      for (int kk = 0; kk < kKc; ++kk) {
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int c = 0; c < C; c += 2) {
          a0 = fmaf(q[c], Ks[kk][part * C + c], a0);
          a1 = fmaf(q[c + 1], Ks[kk][part * C + c + 1], a1);
        }
        float p = a0 + a1;
#pragma unroll
        for (int off = 1; off < G; off <<= 1) p += xor_shfl(p, off);
        s[kk] = c0 + kk < LJ ? p * sl2 : -INFINITY;
        mx = fmaxf(mx, s[kk]);
      }
      const float m_new = fmaxf(m, mx);
      const float corr = m == -INFINITY ? 0.f : exp2f(m - m_new);
      l *= corr;
#pragma unroll
      for (int c = 0; c < C; ++c) o[c] *= corr;
#pragma unroll
      for (int kk = 0; kk < kKc; ++kk) {
        const float p = s[kk] == -INFINITY ? 0.f : exp2f(s[kk] - m_new);
        l += p;
#pragma unroll
        for (int c = 0; c < C; ++c) o[c] = fmaf(p, Vs[kk][part * C + c], o[c]);
      }
      m = m_new;
    }
  }
  if (!qok) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* op = o_r + ((int64_t)bh * Npad + qi) * D + part * C;
#pragma unroll
  for (int c = 0; c < C; c += 4)
    *reinterpret_cast<float4*>(op + c) = make_float4(o[c] * inv, o[c + 1] * inv, o[c + 2] * inv, o[c + 3] * inv);
  if (lse != nullptr && part == 0) lse[(int64_t)bh * Npad + qi] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_estimate_f32(const EstimateArgs& a) {
  dim3 grid(a.nb, a.B * a.Hh);
  const size_t lds = (size_t)a.nb * sizeof(float);
  const float sl2 = a.scale * kLog2e;
  if (a.d == 64)
    hipLaunchKernelGGL((est_f32_kernel<64>), grid, dim3(kF32Threads), lds, a.stream, (const float*)a.q_r,
                       (const float*)a.k_r, a.p_imp, a.N, a.Npad, a.b, a.k, a.nb, sl2);
  else
    hipLaunchKernelGGL((est_f32_kernel<128>), grid, dim3(kF32Threads), lds, a.stream, (const float*)a.q_r,
                       (const float*)a.k_r, a.p_imp, a.N, a.Npad, a.b, a.k, a.nb, sl2);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_f32(const AttnArgs& a) {
  const int rows = a.B * a.Hh * a.nb;
  // one workgroup per (query block, group of kF32Threads / kF32RowThreads rows)
  dim3 grid(rows * (a.b / (kF32Threads / kF32RowThreads)));
  const float sl2 = a.scale * kLog2e;
#define DBS_F32_ATTN(D, BLK)                                                                                 \
  hipLaunchKernelGGL((attn_f32_kernel<D, BLK>), grid, dim3(kF32Threads), 0, a.stream, (const float*)a.q_r,   \
                     (const float*)a.k_r, (const float*)a.v_t, a.kv_count, a.kv_idx, a.order, (float*)a.o_r, \
                     a.lse, a.N, a.Npad, a.nb, rows, sl2)
  if (a.d == 64) {
    if (a.b == 64) DBS_F32_ATTN(64, 64); else DBS_F32_ATTN(64, 128);
  } else {
    if (a.b == 64) DBS_F32_ATTN(128, 64); else DBS_F32_ATTN(128, 128);
  }
#undef DBS_F32_ATTN
  return hipGetLastError();
}

}  // namespace dbs
