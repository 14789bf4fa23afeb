// Sampled block-importance estimation (gfx950).
//
// Video-BLADE "Step 1": k tokens are sampled from every b-token block of Q and
// of K; P_approx = softmax(Q_s K_s^T * scale) over all sampled keys; P_imp is
// its max-pool over each (samples of I) x (samples of J) tile.
//
// Sampled tokens use a compact index r = J*k + t (t < k): slot t of block J is
// reordered row J*b + floor(t*L_J/k_J) when t < k_J = min(k, L_J), and an
// empty slot otherwise (only the last block can have empty slots).  Since
// softmax is monotone in the score and scale * log2(e) > 0,
//     P_imp[I, J] = exp2( max_{q in I} (sl2 * t_qJ - lse2_q) ),
//     t_qJ = max_{c in J} score_qc,  lse2_q = log2 sum_c exp2(sl2 * score_qc),
// so one pass over the sampled scores suffices if the k_J-wide maxima t_qJ
// are kept (a (sampled queries) x nb float array in the workspace; for k > 64
// a block's maximum is kept as k / 64 cell maxima, one per 64-key chunk).
// Three launches:
//   gather: copy the sampled rows of Q and K into compact row-major arrays
//           (zero rows for empty slots) in the workspace;
//   pass:   per sampled query, over a range of the sampled keys: the online
//           max / sum (one partial per key split) and the block maxima t_qJ;
//   final:  merge the partials into lse2 and form P_imp, one exp2 per
//           (query block, key block).
// The key range is split over enough workgroups (about 4096 in total) that
// the DMA latency of each key chunk is hidden by other resident workgroups.
// Both passes compute S^T = K_s Q_s^T on bf16 MFMA 16x16x32 with fp32
// accumulation.  A workgroup of 4 wavefronts owns 64 sampled queries (16 per
// wavefront, in VGPRs); the compact keys stream through double-buffered,
// XOR-swizzled LDS in chunks of 64 by the global->LDS DMA path.  Lane
// reductions use DPP row permutations and v_permlane16/32_swap (VALU, no LDS).
#include "common.h"
#include "../launch.h"

namespace dbs {
namespace {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kQPerWg = kWaves * 16;
constexpr int kChunk = 64;
constexpr int kMaxChunksPerSplit = 64;   // bound on chunks per key split

__device__ __forceinline__ int swz(int u) { return (u & ~15) | ((u & 15) ^ ((u >> 4) & 15)); }

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Lane-exchange reductions (max).  The DPP controls are row-local (16 lanes):
// quad_perm [1,0,3,2] = 0xb1, quad_perm [2,3,0,1] = 0x4e, row_half_mirror =
// 0x141, row_mirror = 0x140.  Mirrors are enough for a reduction: after the
// two quad steps every quad holds its maximum, the half-mirror pairs quad 0
// with 1 (and 2 with 3), the mirror pairs the two halves of the row.
__device__ __forceinline__ float dpp_max(float v, int ctrl) {
  const int o = (ctrl == 0xb1) ? __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xb1, 0xf, 0xf, false)
              : (ctrl == 0x4e) ? __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4e, 0xf, 0xf, false)
              : (ctrl == 0x141) ? __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xf, 0xf, false)
                                : __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xf, 0xf, false);
  return fmaxf(v, __int_as_float(o));
}
// max over lanes l and l ^ 16 / l ^ 32
__device__ __forceinline__ float max_x16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_x32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_x16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_x32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

struct SampleGeom {
  int N, b, k, klog2, nb, nsp, nsp_pad, kj_last;
  int splits, cps;   // key splits and 64-key chunks per split
  int cell_log2;     // block maxima are kept per cell of min(k, 64) compact keys
  int ncell;         // cells per sampled query: nsp >> cell_log2
  // Reordered row of compact slot r, or -1 for an empty slot / r >= nsp.
  __device__ __forceinline__ int row(int r) const {
    if (r >= nsp) return -1;
    const int J = r >> klog2, t = r & (k - 1);
    if (J < nb - 1) return J * b + t * (b >> klog2);   // full block: L = b, k_J = k
    const int L = N - J * b;
    if (t >= kj_last) return -1;
    return J * b + (t * L) / kj_last;
  }
  __device__ __forceinline__ bool valid(int r) const {
    if (r >= nsp) return false;
    return (r >> klog2) < nb - 1 || (r & (k - 1)) < kj_last;
  }
};

// Workgroup -> (bh, key split, query panel).  Logical ids run panel-fastest,
// then split, then (batch, head), and are spread so that each XCD gets a
// contiguous range: one head's sampled keys then stay in one XCD's L2.
__device__ __forceinline__ void wg_coords(const SampleGeom& sg, int& bh, int& split, int& panel) {
  const int panels = (sg.nsp + kQPerWg - 1) / kQPerWg;
  const int total = gridDim.x;
  const int id = xcd_remap(blockIdx.x, total);
  panel = id % panels;
  split = (id / panels) % sg.splits;
  bh = id / (panels * sg.splits);
}

// Compact copies of the sampled rows: qs/ks [BH][nsp_pad][D], zero rows for
// empty slots and padding.  One thread per 16-byte chunk.
template <int D>
__global__ __launch_bounds__(256) void est_gather_kernel(
    const __bf16* __restrict__ q_r, const __bf16* __restrict__ k_r, __bf16* __restrict__ qs,
    __bf16* __restrict__ ks, SampleGeom sg, int Npad) {
  const int bh = blockIdx.y;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const int r = idx / (D / 8), c = idx % (D / 8);
  if (r >= sg.nsp_pad) return;
  const int src = sg.row(r);
  uint4 vq = make_uint4(0, 0, 0, 0), vk = vq;
  if (src >= 0) {
    const int64_t off = ((int64_t)bh * Npad + src) * D + 8 * c;
    vq = *reinterpret_cast<const uint4*>(q_r + off);
    vk = *reinterpret_cast<const uint4*>(k_r + off);
  }
  const int64_t dst = ((int64_t)bh * sg.nsp_pad + r) * D + 8 * c;
  *reinterpret_cast<uint4*>(qs + dst) = vq;
  *reinterpret_cast<uint4*>(ks + dst) = vk;
}

// Empty key slots of a chunk get a score of -inf (the rare chunks that hold
// padding or the last block's empty slots; kept out of the common path).
__device__ __forceinline__ void mask_chunk(const SampleGeom& sg, int ck0, int g4, f32x4_t (&s)[4]) {
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (!sg.valid(ck0 + 16 * t + 4 * g4 + j)) s[t][j] = -INFINITY;
}

// Common streaming loop: for every chunk of 64 compact keys, S^T tiles of the
// wave's 16 queries (s[t][j]: key ck0 + 16t + 4*g4 + j, query l16) are handed
// to `body(ck0, s)`.
template <int D, typename Body>
__device__ __forceinline__ void stream_keys(const __bf16* ks_bh, int c0, int c1,
                                            const bf16x8_t (&qreg)[D / 32], Body&& body) {
  constexpr int kUnits = kChunk * D / 8;       // 16-byte units per chunk
  constexpr int kPer = kUnits / 64 / kWaves;   // DMA instructions per wave per chunk
  // Two distinct arrays with statically known roles in each half of the
  // 2x-unrolled loop: the compiler can then prove that the LDS reads of one
  // buffer do not alias the DMA in flight into the other, and does not insert
  // a wait for that DMA before the reads.
  __shared__ __attribute__((aligned(16))) __bf16 Kc0[kUnits * 8];
  __shared__ __attribute__((aligned(16))) __bf16 Kc1[kUnits * 8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  int off[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int u = swz(64 * (wave + i * kWaves) + lane);
    off[i] = (u / (D / 8)) * D + (u % (D / 8)) * 8;
  }
  auto dma = [&](int chunk, __bf16* buf) {
    const __bf16* base = ks_bh + (int64_t)chunk * kChunk * D;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int n = wave + i * kWaves;
      __builtin_amdgcn_global_load_lds((glb_void_t*)(base + off[i]), (lds_void_t*)(buf + 64 * n * 8), 16, 0, 0);
    }
  };
  auto compute = [&](int ch, const __bf16* kb) {
    f32x4_t s[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      s[t] = f32x4_t{};
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        const int u = (16 * t + l16) * (D / 8) + 4 * kk + g4;
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kb + swz(u) * 8);
        s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[kk], s[t], 0, 0, 0);
      }
    }
    body(ch * kChunk, s);
  };
  dma(c0, Kc0);
  for (int ch = c0; ch < c1; ch += 2) {
    wait_dma();
    __syncthreads();
    if (ch + 1 < c1) dma(ch + 1, Kc1);
    compute(ch, Kc0);
    if (ch + 1 < c1) {
      wait_dma();
      __syncthreads();
      if (ch + 2 < c1) dma(ch + 2, Kc0);
      compute(ch + 1, Kc1);
    }
  }
}

template <int D>
__device__ __forceinline__ void load_q(const __bf16* qs_bh, int rq, int g4, bf16x8_t (&qreg)[D / 32]) {
  const __bf16* qp = qs_bh + (int64_t)rq * D + 8 * g4;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) qreg[kk] = *reinterpret_cast<const bf16x8_t*>(qp + 32 * kk);
}

// Raw block maxima of one 16-key score tile (keys ck0 + 16t + 4*g4 + j, query
// l16): groups of kr = min(K, 16) consecutive keys, nv values per lane.
template <int K>
__device__ __forceinline__ void group_max(const f32x4_t& s, float (&v)[4]) {
  constexpr int kr = K < 16 ? K : 16;
  if constexpr (kr >= 4) {
    v[0] = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    if constexpr (kr >= 8) v[0] = max_x16(v[0]);
    if constexpr (kr >= 16) v[0] = max_x32(v[0]);
  } else if constexpr (kr == 2) {
    v[0] = fmaxf(s[0], s[1]);
    v[1] = fmaxf(s[2], s[3]);
  } else {
    v[0] = s[0]; v[1] = s[1]; v[2] = s[2]; v[3] = s[3];
  }
}

// K: the sample count k when k <= 32 (a cell is one block: a group of K keys
// inside one 16-key tile, or for K = 32 two tiles); 64 stands for every
// k >= 64 (a cell is one 64-key chunk).  A compile-time constant, so the
// reductions below are straight-line code.
template <int D, int K>
__global__ __launch_bounds__(kThreads) void est_pass_kernel(
    const __bf16* __restrict__ qs, const __bf16* __restrict__ ks, float2* __restrict__ part,
    float* __restrict__ tmax, SampleGeom sg, float sl2) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  int bh, split, panel;
  wg_coords(sg, bh, split, panel);
  const int rq = panel * kQPerWg + wave * 16 + l16;
  bf16x8_t qreg[D / 32];
  load_q<D>(qs + (int64_t)bh * sg.nsp_pad * D, rq, g4, qreg);
  float m = -INFINITY, l = 0.f;
  constexpr int kr = K < 16 ? K : 16;
  constexpr int nv = kr >= 4 ? 1 : 4 / kr;
  const bool krep = kr >= 4 ? ((g4 & ((kr >> 2) - 1)) == 0) : true;
  float* trow = tmax + ((int64_t)bh * sg.nsp + rq) * sg.ncell;
  const bool qok = rq < sg.nsp;
  const int tail = (sg.nb - 1) * sg.k;   // first slot of the last block
  const int c0 = split * sg.cps, c1 = min(sg.nsp_pad / kChunk, c0 + sg.cps);
  stream_keys<D>(ks + (int64_t)bh * sg.nsp_pad * D, c0, c1, qreg, [&](int ck0, f32x4_t (&s)[4]) {
    if ((ck0 + kChunk > sg.nsp) || (sg.kj_last < sg.k && ck0 + kChunk > tail)) mask_chunk(sg, ck0, g4, s);
    // block (cell) maxima of the raw scores
    float gv[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) group_max<K>(s[t], gv[t]);
    if constexpr (K == 32) {           // cells of two tiles: 0-1, 2-3
      gv[0][0] = fmaxf(gv[0][0], gv[1][0]);
      gv[2][0] = fmaxf(gv[2][0], gv[3][0]);
    } else if constexpr (K == 64) {    // one cell: the whole chunk
      gv[0][0] = fmaxf(fmaxf(gv[0][0], gv[1][0]), fmaxf(gv[2][0], gv[3][0]));
    }
    constexpr int tstep = K >= 64 ? 4 : (K == 32 ? 2 : 1);
    if (qok && krep) {
#pragma unroll
      for (int t = 0; t < 4; t += tstep) {
#pragma unroll
        for (int e = 0; e < nv; ++e) {
          const int ck = ck0 + 16 * t + 4 * g4 + e * kr;
          if (ck < sg.nsp) trow[ck >> sg.cell_log2] = gv[t][e];
        }
      }
    }
    // online normaliser
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) mx = fmaxf(mx, s[t][j]);
    mx = max_x32(max_x16(mx)) * sl2;
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    l *= fast_exp2(m - m_use);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int j = 0; j < 4; ++j) l += fast_exp2(__builtin_fmaf(s[t][j], sl2, -m_use));
    }
    m = m_new;
  });
  l = sum_x32(sum_x16(l));
  if (g4 == 0 && qok) part[((int64_t)bh * sg.splits + split) * sg.nsp + rq] = make_float2(m, l);
}

// log2 of the softmax normaliser of sampled query rq from its per-split partials.
__device__ __forceinline__ float merge_lse2(const float2* part_bh, const SampleGeom& sg, int rq) {
  float M = -INFINITY;
  for (int s = 0; s < sg.splits; ++s) M = fmaxf(M, part_bh[(int64_t)s * sg.nsp + rq].x);
  if (M == -INFINITY) return INFINITY;
  float L = 0.f;
  for (int s = 0; s < sg.splits; ++s) {
    const float2 p = part_bh[(int64_t)s * sg.nsp + rq];
    L += p.y * fast_exp2(p.x - M);
  }
  return M + __log2f(L);
}

// P_imp of one (batch, head, query block I) row: lse2 of the block's valid
// sampled queries from the split partials (in LDS), then for every key block
// J the maximum over those queries of sl2 * t_qJ - lse2_q, and one exp2.
// An empty query slot contributes nothing; a block without valid query slots
// (impossible: k_J >= 1) would get exp2(-inf) = 0.
constexpr int kFinalThreads = 256;
constexpr int kMaxK = 128;   // k <= b <= 128

__global__ __launch_bounds__(kFinalThreads) void est_final_kernel(const float2* __restrict__ part,
                                                                  const float* __restrict__ tmax,
                                                                  float* __restrict__ p_imp, SampleGeom sg,
                                                                  float sl2) {
  __shared__ float lse[kMaxK];
  const int I = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int kI = I < sg.nb - 1 ? sg.k : sg.kj_last;
  if (tid < sg.k) {
    const int rq = I * sg.k + tid;
    lse[tid] = tid < kI ? merge_lse2(part + (int64_t)bh * sg.splits * sg.nsp, sg, rq) : INFINITY;
  }
  __syncthreads();
  const int cpb = sg.ncell / sg.nb;   // cells per block: 1, or k / 64
  const float* t0 = tmax + ((int64_t)bh * sg.nsp + (int64_t)I * sg.k) * sg.ncell;
  float* prow = p_imp + ((int64_t)bh * sg.nb + I) * sg.nb;
  for (int J = tid; J < sg.nb; J += kFinalThreads) {
    float best = -INFINITY;
    for (int t = 0; t < kI; ++t) {
      const float* tr = t0 + (int64_t)t * sg.ncell + J * cpb;
      float v = tr[0];
      for (int c = 1; c < cpb; ++c) v = fmaxf(v, tr[c]);
      best = fmaxf(best, __builtin_fmaf(v, sl2, -lse[t]));
    }
    prow[J] = fast_exp2(best);
  }
}

// Key splits: enough workgroups in total (about 4096) to hide the latency of
// each chunk's DMA behind other resident workgroups.
void split_plan(int BH, int nsp, int& splits, int& cps) {
  const int nsp_pad = (nsp + kChunk - 1) / kChunk * kChunk;
  const int nchunks = nsp_pad / kChunk;
  const int panels = (nsp + kQPerWg - 1) / kQPerWg;
  const int64_t wgs = (int64_t)panels * BH;
  int want = (int)((4096 + wgs - 1) / wgs);
  want = want < 1 ? 1 : (want > nchunks ? nchunks : want);
  cps = (nchunks + want - 1) / want;
  if (cps > kMaxChunksPerSplit) cps = kMaxChunksPerSplit;
  splits = (nchunks + cps - 1) / cps;
}

template <int D>
hipError_t launch_d(const EstimateArgs& a) {
  SampleGeom sg;
  sg.N = a.N; sg.b = a.b; sg.k = a.k; sg.nb = a.nb;
  sg.klog2 = 0;
  while ((1 << sg.klog2) < a.k) ++sg.klog2;
  sg.nsp = a.nb * a.k;
  sg.nsp_pad = (sg.nsp + kChunk - 1) / kChunk * kChunk;
  sg.cell_log2 = sg.klog2 < 6 ? sg.klog2 : 6;
  sg.ncell = sg.nsp >> sg.cell_log2;
  const int Llast = a.N - (a.nb - 1) * a.b;
  sg.kj_last = a.k < Llast ? a.k : Llast;
  const float sl2 = a.scale * kLog2e;
  const int BH = a.B * a.Hh;
  split_plan(BH, sg.nsp, sg.splits, sg.cps);
  __bf16* qs = reinterpret_cast<__bf16*>(a.workspace);
  __bf16* ks = qs + (int64_t)BH * sg.nsp_pad * D;
  float2* part = reinterpret_cast<float2*>(ks + (int64_t)BH * sg.nsp_pad * D);
  float* tmax = reinterpret_cast<float*>(part + (int64_t)BH * sg.splits * sg.nsp);

  hipLaunchKernelGGL((est_gather_kernel<D>), dim3((sg.nsp_pad * (D / 8) + 255) / 256, BH), dim3(256), 0,
                     a.stream, (const __bf16*)a.q_r, (const __bf16*)a.k_r, qs, ks, sg, a.Npad);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)(((sg.nsp + kQPerWg - 1) / kQPerWg) * sg.splits * BH));
  switch (a.k) {
    case 1: hipLaunchKernelGGL((est_pass_kernel<D, 1>), grid, dim3(kThreads), 0, a.stream, qs, ks, part, tmax, sg, sl2); break;
    case 2: hipLaunchKernelGGL((est_pass_kernel<D, 2>), grid, dim3(kThreads), 0, a.stream, qs, ks, part, tmax, sg, sl2); break;
    case 4: hipLaunchKernelGGL((est_pass_kernel<D, 4>), grid, dim3(kThreads), 0, a.stream, qs, ks, part, tmax, sg, sl2); break;
    case 8: hipLaunchKernelGGL((est_pass_kernel<D, 8>), grid, dim3(kThreads), 0, a.stream, qs, ks, part, tmax, sg, sl2); break;
    case 16: hipLaunchKernelGGL((est_pass_kernel<D, 16>), grid, dim3(kThreads), 0, a.stream, qs, ks, part, tmax, sg, sl2); break;
    case 32: hipLaunchKernelGGL((est_pass_kernel<D, 32>), grid, dim3(kThreads), 0, a.stream, qs, ks, part, tmax, sg, sl2); break;
    default: hipLaunchKernelGGL((est_pass_kernel<D, 64>), grid, dim3(kThreads), 0, a.stream, qs, ks, part, tmax, sg, sl2); break;
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(est_final_kernel, dim3((unsigned)a.nb, (unsigned)BH), dim3(kFinalThreads), 0, a.stream,
                     (const float2*)part, (const float*)tmax, a.p_imp, sg, sl2);
  return hipGetLastError();
}

}  // namespace

size_t estimate_workspace_bytes(int B, int Hh, int nb, int k, int d) {
  const int64_t nsp = (int64_t)nb * k;
  const int64_t nsp_pad = (nsp + kChunk - 1) / kChunk * kChunk;
  const int64_t BH = (int64_t)B * Hh;
  int splits, cps;
  split_plan((int)BH, (int)nsp, splits, cps);
  int klog2 = 0;
  while ((1 << klog2) < k) ++klog2;
  const int64_t cells = nsp >> (klog2 < 6 ? klog2 : 6);
  return (size_t)(BH * nsp_pad * d * 2 * 2 + BH * splits * nsp * 8 + BH * nsp * cells * 4);
}

hipError_t launch_estimate(const EstimateArgs& a) {
  return a.d == 64 ? launch_d<64>(a) : launch_d<128>(a);
}

}  // namespace dbs
