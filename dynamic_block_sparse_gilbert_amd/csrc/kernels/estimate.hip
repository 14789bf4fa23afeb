// Sampled block-importance estimation (gfx950).
//
// Video-BLADE "Step 1": k tokens are sampled from every b-token block of Q and
// of K; P_approx = softmax(Q_s K_s^T * scale) over all sampled keys; P_imp is
// its max-pool over each (samples of I) x (samples of J) tile.
//
// Sampled tokens are addressed through a compact index r = J*k + t (t < k):
// slot t of block J is reordered row J*b + floor(t*L_J/k_J) when t < k_J =
// min(k, L_J), and an empty slot otherwise (only the last block can have
// empty slots).  Since softmax is monotone in the score,
//     P_imp[I, J] = exp2( max_{q in I, c in J} (x_qc - lse2_q) ),
// with x = score * scale * log2(e) and lse2_q = log2 sum_c exp2(x_qc).  Two
// passes over the sampled keys therefore suffice and nothing of size
// (sampled queries) x nb is ever stored:
//   pass 1 (stats):    online max / sum per sampled query -> lse2 (workspace);
//   pass 2 (blockmax): recompute x, subtract lse2, max-reduce each k x k
//                      group with lane butterflies, one exp2 per group.
// Both passes run S^T = K_s Q_s^T on bf16 MFMA 16x16x32 with fp32
// accumulation; a workgroup of 8 wavefronts owns 128 sampled queries (16 per
// wavefront, kept in VGPRs) and streams the sampled keys through LDS in
// chunks of 64, so every key chunk is read once per 128 queries.
#include "common.h"
#include "../launch.h"

namespace dbs {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kQPerWg = kWaves * 16;
constexpr int kChunk = 64;

struct SampleGeom {
  int N, b, k, klog2, nb, nsp, kj_last;
  // Reordered row of compact slot r, or -1 for an empty slot / r >= nsp.
  __device__ __forceinline__ int row(int r) const {
    if (r >= nsp) return -1;
    const int J = r >> klog2, t = r & (k - 1);
    const int L = min(b, N - J * b);
    const int kJ = min(k, L);
    if (t >= kJ) return -1;
    return J * b + (t * L) / kJ;
  }
  __device__ __forceinline__ bool valid(int r) const {
    if (r >= nsp) return false;
    return (r >> klog2) < nb - 1 || (r & (k - 1)) < kj_last;
  }
};

template <int D>
__device__ __forceinline__ void load_q(const __bf16* q_r, int64_t rowbase, const SampleGeom& sg,
                                       int rq, int g4, bf16x8_t (&qreg)[D / 32]) {
  const int src = sg.row(rq);
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    if (src >= 0) {
      qreg[kk] = *reinterpret_cast<const bf16x8_t*>(q_r + (rowbase + src) * D + 32 * kk + 8 * g4);
    } else {
      qreg[kk] = bf16x8_t{};
    }
  }
}

// Stage kChunk sampled key rows starting at compact index ck0 into LDS.
template <int D>
__device__ __forceinline__ void load_keys(const __bf16* k_r, int64_t rowbase, const SampleGeom& sg,
                                          int ck0, __bf16* Kc) {
  constexpr int kStride = D + 8;
#pragma unroll
  for (int c = threadIdx.x; c < kChunk * D / 8; c += kThreads) {
    const int rr = c / (D / 8), cc = c % (D / 8);
    const int src = sg.row(ck0 + rr);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (src >= 0) v = *reinterpret_cast<const uint4*>(k_r + (rowbase + src) * D + 8 * cc);
    *reinterpret_cast<uint4*>(Kc + rr * kStride + 8 * cc) = v;
  }
}

// Scores of the wave's 16 queries against the 64 staged keys:
// s[t][j] = key ck0 + 16t + 4*g4 + j, query l16.
template <int D>
__device__ __forceinline__ void score_chunk(const __bf16* Kc, int l16, int g4,
                                            const bf16x8_t (&qreg)[D / 32], f32x4_t (&s)[4]) {
  constexpr int kStride = D + 8;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    s[t] = f32x4_t{};
    const __bf16* kp = Kc + (16 * t + l16) * kStride + 8 * g4;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kp + 32 * kk);
      s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[kk], s[t], 0, 0, 0);
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void est_stats_kernel(
    const __bf16* __restrict__ q_r, const __bf16* __restrict__ k_r, float* __restrict__ lse2,
    SampleGeom sg, int Npad, float sl2) {
  __shared__ __attribute__((aligned(16))) __bf16 Kc[kChunk * (D + 8)];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int bh = blockIdx.y;
  const int64_t rowbase = (int64_t)bh * Npad;
  const int rq = blockIdx.x * kQPerWg + wave * 16 + l16;
  bf16x8_t qreg[D / 32];
  load_q<D>(q_r, rowbase, sg, rq, g4, qreg);

  float m = -INFINITY, l = 0.f;
  const int tail = (sg.nb - 1) * sg.k;   // first slot of the last block
  for (int ck0 = 0; ck0 < sg.nsp; ck0 += kChunk) {
    __syncthreads();
    load_keys<D>(k_r, rowbase, sg, ck0, Kc);
    __syncthreads();
    f32x4_t s[4];
    score_chunk<D>(Kc, l16, g4, qreg, s);
    const bool check = (ck0 + kChunk > sg.nsp) || (sg.kj_last < sg.k && ck0 + kChunk > tail);
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float x = s[t][j] * sl2;
        if (check && !sg.valid(ck0 + 16 * t + 4 * g4 + j)) x = -INFINITY;
        s[t][j] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, xor_shfl(mx, 16));
    mx = fmaxf(mx, xor_shfl(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    l *= fast_exp2(m - m_use);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int j = 0; j < 4; ++j) l += fast_exp2(s[t][j] - m_use);
    }
    m = m_new;
  }
  l += xor_shfl(l, 16);
  l += xor_shfl(l, 32);
  if (g4 == 0 && rq < sg.nsp) {
    lse2[(int64_t)bh * sg.nsp + rq] = sg.valid(rq) ? m + __log2f(l) : INFINITY;
  }
}

__global__ void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

template <int D>
__global__ __launch_bounds__(kThreads) void est_blockmax_kernel(
    const __bf16* __restrict__ q_r, const __bf16* __restrict__ k_r, const float* __restrict__ lse2,
    float* __restrict__ p_imp, SampleGeom sg, int Npad, float sl2) {
  __shared__ __attribute__((aligned(16))) __bf16 Kc[kChunk * (D + 8)];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int bh = blockIdx.y;
  const int64_t rowbase = (int64_t)bh * Npad;
  const int rq = blockIdx.x * kQPerWg + wave * 16 + l16;
  bf16x8_t qreg[D / 32];
  load_q<D>(q_r, rowbase, sg, rq, g4, qreg);
  // an empty query slot contributes -inf to its group
  const float myl = (rq < sg.nsp) ? lse2[(int64_t)bh * sg.nsp + rq] : INFINITY;
  const int k = sg.k;
  const int kr = k < 16 ? k : 16;        // group side inside one 16 x 16 tile
  const int I = rq >> sg.klog2;
  const bool qrep = (l16 & (kr - 1)) == 0;
  float* prow = p_imp + ((int64_t)bh * sg.nb + I) * sg.nb;
  const int tail = (sg.nb - 1) * sg.k;

  for (int ck0 = 0; ck0 < sg.nsp; ck0 += kChunk) {
    __syncthreads();
    load_keys<D>(k_r, rowbase, sg, ck0, Kc);
    __syncthreads();
    f32x4_t s[4];
    score_chunk<D>(Kc, l16, g4, qreg, s);
    const bool check = (ck0 + kChunk > sg.nsp) || (sg.kj_last < sg.k && ck0 + kChunk > tail);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float u[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u[j] = s[t][j] * sl2 - myl;
        if (check && !sg.valid(ck0 + 16 * t + 4 * g4 + j)) u[j] = -INFINITY;
      }
      // keys: reduce within groups of kr consecutive keys
      float v[4];
      int nv;
      if (kr >= 4) {
        v[0] = fmaxf(fmaxf(u[0], u[1]), fmaxf(u[2], u[3]));
        if (kr >= 8) v[0] = fmaxf(v[0], xor_shfl(v[0], 16));
        if (kr >= 16) v[0] = fmaxf(v[0], xor_shfl(v[0], 32));
        nv = 1;
      } else if (kr == 2) {
        v[0] = fmaxf(u[0], u[1]);
        v[1] = fmaxf(u[2], u[3]);
        nv = 2;
      } else {
        v[0] = u[0]; v[1] = u[1]; v[2] = u[2]; v[3] = u[3];
        nv = 4;
      }
      // queries: reduce within groups of kr consecutive queries (lanes)
      for (int sft = 1; sft < kr; sft <<= 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e < nv) v[e] = fmaxf(v[e], xor_shfl(v[e], sft));
      }
      const bool krep = kr >= 4 ? ((g4 & ((kr >> 2) - 1)) == 0) : true;
      if (qrep && krep && rq < sg.nsp) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (e < nv) {
            const int ck = ck0 + 16 * t + 4 * g4 + e * (4 / nv);
            if (ck < sg.nsp) {
              const int J = ck >> sg.klog2;
              const float p = fast_exp2(v[e]);
              if (k <= 16) {
                prow[J] = p;
              } else {
                atomicMax(reinterpret_cast<int*>(prow + J), __float_as_int(p));
              }
            }
          }
        }
      }
    }
  }
}

template <int D>
hipError_t launch_d(const EstimateArgs& a) {
  SampleGeom sg;
  sg.N = a.N; sg.b = a.b; sg.k = a.k; sg.nb = a.nb;
  sg.klog2 = 0;
  while ((1 << sg.klog2) < a.k) ++sg.klog2;
  sg.nsp = a.nb * a.k;
  const int Llast = a.N - (a.nb - 1) * a.b;
  sg.kj_last = a.k < Llast ? a.k : Llast;
  const float sl2 = a.scale * kLog2e;
  dim3 grid((sg.nsp + kQPerWg - 1) / kQPerWg, a.B * a.Hh);
  hipLaunchKernelGGL((est_stats_kernel<D>), grid, dim3(kThreads), 0, a.stream,
                     (const __bf16*)a.q_r, (const __bf16*)a.k_r, a.lse2, sg, a.Npad, sl2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.k > 16) {
    const int64_t n = (int64_t)a.B * a.Hh * a.nb * a.nb;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, a.stream,
                       a.p_imp, n);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((est_blockmax_kernel<D>), grid, dim3(kThreads), 0, a.stream,
                     (const __bf16*)a.q_r, (const __bf16*)a.k_r, (const float*)a.lse2, a.p_imp, sg,
                     a.Npad, sl2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_estimate(const EstimateArgs& a) {
  return a.d == 64 ? launch_d<64>(a) : launch_d<128>(a);
}

}  // namespace dbs
