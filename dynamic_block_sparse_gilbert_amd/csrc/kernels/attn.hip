// Block-sparse flash attention forward over compacted KV-block lists (gfx950).
//
// Video-BLADE "Step 2.2": the binary block mask restricts attention; every
// query block walks only its kept KV blocks (the count/index-list form the
// BSA notes call q2k_num / q2k_index).  ASA_G appends the mean-pooled global
// tokens with a +ln(r) logit bias (BLADE notes, key design 2).
//
// Decomposition: one workgroup per (batch, head, query block of BLK rows);
// each wavefront owns 32 query rows (one MFMA tile), which keeps the scores of
// two stages, P, Q and O in about 180 VGPRs (two wavefronts per SIMD).  Keys
// are consumed in stages of 64 (a kept block of 128 is two stages;
// global-token tiles likewise).
//   S^T = K Q^T      bf16 MFMA 32x32x16, Q^T resident in VGPRs.  The
//                    accumulator layout gives each lane the scores of single
//                    queries, so softmax statistics stay in the lane (one
//                    exchange between the two wave halves per stage).
//   P^T = exp2(S^T * scale*log2e - m)   fp32, packed to bf16 by v_cvt_pk.
//   O^T += V^T P^T   bf16 MFMA 32x32x16; P^T comes straight from the score
//                    accumulators.  Inside each 16-key step the MFMA k index
//                    maps to keys {4g..4g+3, 8+4g..8+4g+3} (g = wave half) for
//                    both operands; V tiles store every 16 keys in the order
//                    0-3, 8-11, 4-7, 12-15, so a lane's 8 keys of one channel
//                    are one contiguous 16-byte LDS read.
// Pipelining: K and V stages are copied global -> LDS by the DMA path
// (global_load_lds_dwordx4, no VGPR staging) into double buffers, two stages
// ahead for K and one for V.  Within an iteration the MFMAs of the next
// stage's scores are issued before the softmax of the current stage, so the
// matrix core and the VALU work concurrently.  LDS tiles are XOR-swizzled in
// 16-byte units (unit ^= line & 15 within each 256-byte line); the swizzle is
// applied by choosing each lane's DMA source address.
// Online softmax with a lazy rescale: the running maximum is raised (and O, l
// rescaled) only when a stage's maximum exceeds it by more than 8 (log2
// units), so probabilities stay below 2^8 and most stages skip the rescale.
#include "common.h"
#include "../launch.h"

namespace dbs {
namespace {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

template <int D, int BLK>
struct AttnCfg {
  static constexpr int kQW = 32;                 // query rows per wavefront
  static constexpr int kWaves = BLK / kQW;       // 4 for BLK = 128, 2 for BLK = 64
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kKT = 64;                 // keys per stage
  static constexpr int kSubs = BLK / kKT;        // stages per block
  static constexpr int kUnits = kKT * D / 8;     // 16-byte units per K (or V) stage
  static constexpr int kDma = kUnits / 64;       // DMA instructions per stage
  static constexpr int kKRow = D / 8;            // units per K row
  static constexpr int kVRow = kKT / 8;          // units per V^T row
};

constexpr float kLazyThreshold = 8.0f;

// Physical 16-byte unit of logical unit u (an involution).
__device__ __forceinline__ int swz(int u) { return (u & ~15) | ((u & 15) ^ ((u >> 4) & 15)); }

__device__ __forceinline__ bf16x8_t lds_read16(const __bf16* base, int unit) {
  return *reinterpret_cast<const bf16x8_t*>(base + swz(unit) * 8);
}

__device__ __forceinline__ uint32_t cvt_pk(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  bf16x2_t p;
  p[0] = (__bf16)a;
  p[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

struct StageDesc {
  const __bf16* k;     // first K row of the stage (rows of D)
  const __bf16* v;     // row 0 of the V^T tile, offset to the stage's first key column
  int key0;            // index of the stage's first key (token, or global token)
  int kind;            // 0 full, 1 partial / invalid (mask by key index), 2 global tokens
  int limit;           // keys with index >= limit are masked (kind 1, 2)
};

template <int D, int BLK>
__global__ __launch_bounds__(BLK / 32 * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(
    const __bf16* __restrict__ q_r, const __bf16* __restrict__ k_r, const __bf16* __restrict__ v_t,
    const int32_t* __restrict__ kv_count, const int32_t* __restrict__ kv_idx,
    const __bf16* __restrict__ k_g, const __bf16* __restrict__ v_g,
    __bf16* __restrict__ o_r, float* __restrict__ lse,
    int Hh, int N, int Npad, int nb, int Ng, float sl2, float log2n, float log2r_last, int total) {
  using C = AttnCfg<D, BLK>;
  // Four distinct arrays whose roles are static in each half of the 2x-unrolled
  // pipeline, so the compiler can prove LDS reads never alias a DMA in flight
  // and does not make them wait for it.
  __shared__ __attribute__((aligned(16))) __bf16 Kb0[C::kUnits * 8];
  __shared__ __attribute__((aligned(16))) __bf16 Kb1[C::kUnits * 8];
  __shared__ __attribute__((aligned(16))) __bf16 Vb0[C::kUnits * 8];
  __shared__ __attribute__((aligned(16))) __bf16 Vb1[C::kUnits * 8];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int wid = xcd_remap(blockIdx.x, total);
  const int I = wid % nb;
  const int bh = wid / nb;
  const int q0 = I * BLK + wave * C::kQW;
  const int64_t rowbase = (int64_t)bh * Npad;

  int cnt = __builtin_amdgcn_readfirstlane(kv_count[(int64_t)bh * nb + I]);
  cnt = cnt < 0 ? 0 : (cnt > nb ? nb : cnt);
  const int32_t* idx = kv_idx + ((int64_t)bh * nb + I) * nb;
  const int Ngpad = (Ng + BLK - 1) / BLK * BLK;
  const int ntg = (k_g != nullptr) ? Ngpad / BLK : 0;
  const int U = (cnt + ntg) * C::kSubs;

  auto stage = [&](int u) -> StageDesc {
    StageDesc s;
    const int j = u / C::kSubs, h = u % C::kSubs;
    if (j < cnt) {
      int J = __builtin_amdgcn_readfirstlane(idx[j]);   // uniform: keep it scalar
      const bool ok = J >= 0 && J < nb;
      J = ok ? J : 0;
      s.key0 = J * BLK + h * C::kKT;
      s.k = k_r + (rowbase + s.key0) * D;
      s.v = v_t + ((int64_t)bh * nb + J) * (int64_t)(D * BLK) + h * C::kKT;
      s.limit = ok ? N : -1;
      s.kind = (ok && s.key0 + C::kKT <= N) ? 0 : 1;
    } else {
      const int J = j - cnt;
      s.key0 = J * BLK + h * C::kKT;
      s.k = k_g + ((int64_t)bh * Ngpad + s.key0) * D;
      s.v = v_g + ((int64_t)bh * (Ngpad / BLK) + J) * (int64_t)(D * BLK) + h * C::kKT;
      s.limit = Ng;
      s.kind = 2;
    }
    return s;
  };

  // Per-lane source offsets (elements) of the swizzled DMA: loop invariant.
  constexpr int kPer = C::kDma / C::kWaves;   // DMA instructions per wave per stage
  int koff[kPer], voff[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int n = wave + i * C::kWaves;
    const int u = swz(64 * n + lane);          // logical unit held by this lane's slot
    koff[i] = (u / C::kKRow) * D + (u % C::kKRow) * 8;
    voff[i] = (u / C::kVRow) * BLK + (u % C::kVRow) * 8;
  }

  // DMA one stage of K (kv = 0) or V^T (kv = 1) into an LDS buffer.
  auto dma = [&](const StageDesc& s, __bf16* buf, int kv) {
    const __bf16* base = kv == 0 ? s.k : s.v;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int n = wave + i * C::kWaves;
      const __bf16* src = base + (kv == 0 ? koff[i] : voff[i]);
      __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)(buf + 64 * n * 8), 16, 0, 0);
    }
  };

  // Q^T operand: lane (l32, g) holds Q[q0 + l32][16 kk + 8 g .. +7].
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

  // S^T[kt] for the stage held in K buffer kb: keys 32 kt + (v/4)*8 + 4g + v%4.
  auto scores = [&](const __bf16* kb, f32x16_t (&S)[2]) {
    S[0] = f32x16_t{};
    S[1] = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8_t a = lds_read16(kb, (32 * kt + l32) * C::kKRow + 2 * kk + g);
        S[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[kk], S[kt], 0, 0, 0);
      }
    }
  };

  // Softmax of a stage's scores, then O^T += V^T P^T from V buffer vb.
  auto consume = [&](const StageDesc& s, f32x16_t (&S)[2], const __bf16* vb) {
    float mx = -INFINITY;
    if (s.kind == 0) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, S[kt][v]);
      mx *= sl2;
    } else {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = s.key0 + 32 * kt + (v >> 2) * 8 + 4 * g + (v & 3);
          float t = S[kt][v] * sl2;
          if (s.kind == 2) t += (key < s.limit - 1) ? log2n : log2r_last;
          if (key >= s.limit) t = -INFINITY;
          S[kt][v] = t;
          mx = fmaxf(mx, t);
        }
      }
    }
    mx = fmaxf(mx, xor_shfl(mx, 32));
    const bool need = mx > m + kLazyThreshold;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float m_new = need ? mx : m;
      const float alpha = need ? fast_exp2(m - m_new) : 1.f;
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) oacc[dt] *= alpha;
    }
    const float m_use = (m == -INFINITY) ? 0.f : m;
    float ls = 0.f;
    if (s.kind == 0) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = fast_exp2(__builtin_fmaf(S[kt][v], sl2, -m_use));
          ls += p;
          S[kt][v] = p;
        }
    } else {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = fast_exp2(S[kt][v] - m_use);
          ls += p;
          S[kt][v] = p;
        }
    }
    l += ls;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int kt = st >> 1, o = (st & 1) * 8;
      uint4 w;
      w.x = cvt_pk(S[kt][o + 0], S[kt][o + 1]);
      w.y = cvt_pk(S[kt][o + 2], S[kt][o + 3]);
      w.z = cvt_pk(S[kt][o + 4], S[kt][o + 5]);
      w.w = cvt_pk(S[kt][o + 6], S[kt][o + 7]);
      const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, w);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const bf16x8_t a = lds_read16(vb, (32 * dt + l32) * C::kVRow + 2 * st + g);
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[dt], 0, 0, 0);
      }
    }
  };

  // One pipeline iteration: stage u is consumed, stage u+1's scores issued.
  // kdst / vdst receive the DMAs of stages u+2 (K) and u+1 (V); ksrc holds
  // K of stage u+1 and vsrc holds V of stage u.
  auto iterate = [&](int u, f32x16_t (&Scur)[2], f32x16_t (&Snext)[2], __bf16* kdst, __bf16* vdst,
                     const __bf16* ksrc, const __bf16* vsrc) {
    wait_dma();
    __syncthreads();
    if (u + 2 < U) dma(stage(u + 2), kdst, 0);
    if (u + 1 < U) dma(stage(u + 1), vdst, 1);
    if (u + 1 < U) scores(ksrc, Snext);
    consume(stage(u), Scur, vsrc);
  };

  if (U > 0) {
    dma(stage(0), Kb0, 0);
    dma(stage(0), Vb0, 1);
    if (U > 1) dma(stage(1), Kb1, 0);
    wait_dma();
    __syncthreads();
    f32x16_t SA[2], SB[2];
    scores(Kb0, SA);
    for (int u = 0; u < U; u += 2) {
      iterate(u, SA, SB, Kb0, Vb1, Kb1, Vb0);
      if (u + 1 < U) iterate(u + 1, SB, SA, Kb1, Vb0, Kb0, Vb1);
    }
  }

  // ---- epilogue -------------------------------------------------------------------
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
        w.x = cvt_pk(oacc[dt][i * 4 + 0] * inv, oacc[dt][i * 4 + 1] * inv);
        w.y = cvt_pk(oacc[dt][i * 4 + 2] * inv, oacc[dt][i * 4 + 3] * inv);
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
                     (__bf16*)a.o_r, a.lse, a.Hh, a.N, a.Npad, a.nb, a.Ng, sl2, log2n, log2r_last,
                     total);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const AttnArgs& a) {
  if (a.d == 64) return a.b == 64 ? launch<64, 64>(a) : launch<64, 128>(a);
  return a.b == 64 ? launch<128, 64>(a) : launch<128, 128>(a);
}

}  // namespace dbs
