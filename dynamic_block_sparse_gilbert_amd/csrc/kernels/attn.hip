// Block-sparse flash attention forward over compacted KV-block lists (gfx950).
//
// Video-BLADE "Step 2.2": the binary block mask restricts attention; every
// query block walks only its kept KV blocks (the count/index-list form the
// BSA notes call q2k_num / q2k_index).  ASA_G appends the mean-pooled global
// tokens with a +ln(r) logit bias (BLADE notes, key design 2).
//
// Work decomposition: one workgroup per (batch, head, query block of BLK
// rows); BLK/32 wavefronts, each owning 32 query rows.  Per kept KV block:
//   S^T = K Q^T      bf16 MFMA 32x32x16; Q^T stays in VGPRs, K from LDS.
//                    The accumulator layout gives every lane the scores of a
//                    single query, so the online-softmax max/sum and the
//                    rescale of the output need no cross-lane traffic except
//                    one exchange between the two wave halves.
//   P^T = exp2(S^T * scale*log2e - m)   rounded to bf16 in registers.
//   O^T += V^T P^T   bf16 MFMA 32x32x16; P^T is taken straight from the score
//                    accumulators: within each 16-key step the k index of the
//                    MFMA is mapped to keys {4g+0..3, 8+4g+0..3} (g = wave
//                    half), the same mapping for both operands.  V is stored
//                    tile-transposed (d-major) so each lane's 8 keys of one
//                    channel are two 8-byte LDS reads.
// K and V^T tiles are staged through LDS with padded rows (bank spread).
#include "common.h"
#include "../launch.h"

namespace dbs {
namespace {

template <int D, int BLK>
struct AttnCfg {
  static constexpr int kWaves = BLK / 32;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kKStride = D + 8;    // bf16 per K row in LDS (+16 bytes)
  static constexpr int kVStride = BLK + 4;  // bf16 per V^T row in LDS (+8 bytes)
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

template <int D, int BLK>
__global__ __launch_bounds__(BLK / 32 * 64) void attn_fwd_kernel(
    const __bf16* __restrict__ q_r, const __bf16* __restrict__ k_r, const __bf16* __restrict__ v_t,
    const int32_t* __restrict__ kv_count, const int32_t* __restrict__ kv_idx,
    const __bf16* __restrict__ k_g, const __bf16* __restrict__ v_g,
    __bf16* __restrict__ o_r, float* __restrict__ lse,
    int Hh, int N, int Npad, int nb, int Ng, int n_pool, float sl2, float log2n, float log2r_last,
    int total) {
  using C = AttnCfg<D, BLK>;
  __shared__ __attribute__((aligned(16))) __bf16 Ks[BLK * C::kKStride];
  __shared__ __attribute__((aligned(16))) __bf16 Vs[D * C::kVStride];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int wid = xcd_remap(blockIdx.x, total);
  const int I = wid % nb;
  const int bh = wid / nb;
  const int q0 = I * BLK + wave * 32;
  const int64_t rowbase = (int64_t)bh * Npad;

  // Q^T operand: lane (l32, g) holds Q[q0 + l32][16*kk + 8*g .. +7].
  bf16x8_t qreg[D / 16];
  {
    const __bf16* qp = q_r + (rowbase + q0 + l32) * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qreg[kk] = *reinterpret_cast<const bf16x8_t*>(qp + 16 * kk);
  }

  f32x16_t oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = f32x16_t{};
  float m = -INFINITY, l = 0.f;

  int cnt = kv_count[(int64_t)bh * nb + I];
  cnt = cnt < 0 ? 0 : (cnt > nb ? nb : cnt);
  const int32_t* idx = kv_idx + ((int64_t)bh * nb + I) * nb;
  const int Ngpad = (Ng + BLK - 1) / BLK * BLK;
  const int ntg = (k_g != nullptr) ? Ngpad / BLK : 0;

  for (int it = 0; it < cnt + ntg; ++it) {
    const bool glob = it >= cnt;
    int J;
    const __bf16* kt;
    const __bf16* vt;
    if (!glob) {
      J = idx[it];
      if (J < 0 || J >= nb) continue;  // uniform across the workgroup
      kt = k_r + (rowbase + (int64_t)J * BLK) * D;
      vt = v_t + ((int64_t)bh * nb + J) * (int64_t)(D * BLK);
    } else {
      J = it - cnt;
      kt = k_g + ((int64_t)bh * Ngpad + (int64_t)J * BLK) * D;
      vt = v_g + ((int64_t)bh * (Ngpad / BLK) + J) * (int64_t)(D * BLK);
    }

    __syncthreads();  // the previous tile is no longer read
#pragma unroll
    for (int c = threadIdx.x; c < BLK * D / 8; c += C::kThreads) {
      const int r = c / (D / 8), cc = c % (D / 8);
      const uint4 v = *reinterpret_cast<const uint4*>(kt + r * D + cc * 8);
      *reinterpret_cast<uint4*>(Ks + r * C::kKStride + cc * 8) = v;
    }
#pragma unroll
    for (int c = threadIdx.x; c < D * BLK / 8; c += C::kThreads) {
      const int r = c / (BLK / 8), cc = c % (BLK / 8);
      const uint4 v = *reinterpret_cast<const uint4*>(vt + r * BLK + cc * 8);
      uint2* dst = reinterpret_cast<uint2*>(Vs + r * C::kVStride + cc * 8);
      dst[0] = make_uint2(v.x, v.y);
      dst[1] = make_uint2(v.z, v.w);
    }
    __syncthreads();

    // ---- S^T = K Q^T ----------------------------------------------------
    f32x16_t sacc[BLK / 32];
#pragma unroll
    for (int t = 0; t < BLK / 32; ++t) {
      sacc[t] = f32x16_t{};
      const __bf16* kp = Ks + (32 * t + l32) * C::kKStride + 8 * g;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kp + 16 * kk);
        sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[kk], sacc[t], 0, 0, 0);
      }
    }

    // ---- scale, mask, bias (log2 domain) and the running max --------------
    const int key0 = J * BLK;
    float mx = -INFINITY;
    if (!glob) {
      const bool partial = key0 + BLK > N;
#pragma unroll
      for (int t = 0; t < BLK / 32; ++t) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float s = sacc[t][v] * sl2;
          if (partial) {
            const int key = key0 + 32 * t + (v >> 2) * 8 + 4 * g + (v & 3);
            if (key >= N) s = -INFINITY;
          }
          sacc[t][v] = s;
          mx = fmaxf(mx, s);
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < BLK / 32; ++t) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int gi = key0 + 32 * t + (v >> 2) * 8 + 4 * g + (v & 3);
          const float bias = gi < Ng - 1 ? log2n : (gi == Ng - 1 ? log2r_last : -INFINITY);
          const float s = sacc[t][v] * sl2 + bias;
          sacc[t][v] = s;
          mx = fmaxf(mx, s);
        }
      }
    }
    mx = fmaxf(mx, xor_shfl(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) oacc[dt] *= alpha;

    // ---- P^T = exp2(S^T - m) ------------------------------------------------
#pragma unroll
    for (int t = 0; t < BLK / 32; ++t) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = fast_exp2(sacc[t][v] - m_use);
        l += p;
        sacc[t][v] = p;
      }
    }

    // ---- O^T += V^T P^T -------------------------------------------------------
#pragma unroll
    for (int s = 0; s < BLK / 16; ++s) {
      const int t = s >> 1, i0 = 2 * (s & 1);
      uint4 pb;
      pb.x = pack_bf16x2(sacc[t][i0 * 4 + 0], sacc[t][i0 * 4 + 1]);
      pb.y = pack_bf16x2(sacc[t][i0 * 4 + 2], sacc[t][i0 * 4 + 3]);
      pb.z = pack_bf16x2(sacc[t][i0 * 4 + 4], sacc[t][i0 * 4 + 5]);
      pb.w = pack_bf16x2(sacc[t][i0 * 4 + 6], sacc[t][i0 * 4 + 7]);
      const bf16x8_t b = as_bf16x8(pb);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const __bf16* vp = Vs + (32 * dt + l32) * C::kVStride + 16 * s + 4 * g;
        const uint2 lo = *reinterpret_cast<const uint2*>(vp);
        const uint2 hi = *reinterpret_cast<const uint2*>(vp + 8);
        const bf16x8_t a = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, oacc[dt], 0, 0, 0);
      }
    }
  }

  // ---- epilogue -----------------------------------------------------------------
  const float lt = l + xor_shfl(l, 32);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const int q = q0 + l32;
  if (q < N) {
    __bf16* op = o_r + (rowbase + q) * D + 4 * g;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint2 w;
        w.x = pack_bf16x2(oacc[dt][i * 4 + 0] * inv, oacc[dt][i * 4 + 1] * inv);
        w.y = pack_bf16x2(oacc[dt][i * 4 + 2] * inv, oacc[dt][i * 4 + 3] * inv);
        *reinterpret_cast<uint2*>(op + 32 * dt + 8 * i) = w;
      }
    }
    if (lse != nullptr && g == 0) {
      lse[rowbase + q] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
    }
  }
}

template <int D, int BLK>
hipError_t launch(const AttnArgs& a) {
  const int total = a.B * a.Hh * a.nb;
  const float sl2 = a.scale * kLog2e;
  float log2n = 0.f, log2r_last = 0.f;
  if (a.k_g != nullptr) {
    log2n = std::log2((float)a.n_pool);
    log2r_last = std::log2((float)(a.N - (a.Ng - 1) * a.n_pool));
  }
  hipLaunchKernelGGL((attn_fwd_kernel<D, BLK>), dim3(total), dim3(AttnCfg<D, BLK>::kThreads), 0,
                     a.stream, (const __bf16*)a.q_r, (const __bf16*)a.k_r, (const __bf16*)a.v_t,
                     a.kv_count, a.kv_idx, (const __bf16*)a.k_g, (const __bf16*)a.v_g,
                     (__bf16*)a.o_r, a.lse, a.Hh, a.N, a.Npad, a.nb, a.Ng, a.n_pool, sl2, log2n,
                     log2r_last, total);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const AttnArgs& a) {
  if (a.d == 64) return a.b == 64 ? launch<64, 64>(a) : launch<64, 128>(a);
  return a.b == 64 ? launch<128, 64>(a) : launch<128, 128>(a);
}

}  // namespace dbs
