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
// Two launches:
//   pass:   per sampled query, over a range of the sampled keys: the online
//           max / sum (one partial per key split) and the block maxima t_qJ;
//           the sampled rows of Q and K are read in place (no compact copy);
//   final:  merge the partials into lse2 and form P_imp, one exp2 per
//           (query block, key block).
// The key range is split over about 768 workgroups of 8 wavefronts (one
// and a half rounds of two per CU): longer key ranges per workgroup spread
// its fixed costs (Q loads, first copy, merge) over more chunks.
// The pass computes S^T = K_s Q_s^T on bf16 MFMA 32x32x16 with fp32
// accumulation: a workgroup of 8 wavefronts owns 256 sampled queries (32 per
// wavefront, in VGPRs), so each 64-key chunk copied to LDS feeds 256 queries;
// the sampled keys stream through double-buffered, row-padded LDS by the
// buffer form of the global -> LDS copy.
#include <type_traits>

#include "common.h"
#include "../launch.h"
#include "mask_core.h"

namespace dbs {
namespace {

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kQPerWg = kWaves * 32;
constexpr int kChunk = 64;
constexpr int kMaxChunksPerSplit = 64;   // bound on chunks per key split

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// k: slots per block, the sample count rounded up to a power of two; kf: the
// sample count (valid slots of a full block, kf <= k); kj_last: valid slots of
// the last block.  Slots t >= kf of a full block are empty, like the last
// block's slots t >= kj_last.
struct SampleGeom {
  int N, b, k, klog2, nb, nsp, nsp_pad, kj_last, kf;
  int splits, cps;   // key splits and 64-key chunks per split
  int cell_log2;     // block maxima are kept per cell of min(k, 64) compact keys
  int ncell;         // cells per sampled query: nsp >> cell_log2
  int compact;       // the pass reads K from the gathered slot rows (row r = slot r), not k_r
  // Reordered row of compact slot r, or -1 for an empty slot / r >= nsp.
  __device__ __forceinline__ int row(int r) const {
    if (r >= nsp) return -1;
    const int J = r >> klog2, t = r & (k - 1);
    if (J < nb - 1) {   // full block: L = b, k_J = kf
      if (kf == k) return J * b + t * (b >> klog2);
      return t < kf ? J * b + (t * b) / kf : -1;
    }
    const int L = N - J * b;
    if (t >= kj_last) return -1;
    return J * b + (t * L) / kj_last;
  }
  __device__ __forceinline__ bool valid(int r) const {
    if (r >= nsp) return false;
    return (r & (k - 1)) < ((r >> klog2) < nb - 1 ? kf : kj_last);
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

// Raw buffer descriptor over `bytes` bytes at `base` (gfx9 word 3: 32-bit data
// format, raw addressing).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// 16 bytes per lane from buffer offset soff + voff into LDS at lds + 16 * lane
// (the buffer form of the global -> LDS copy counts on vmcnt only).
__device__ __forceinline__ void copy16_lds(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, voff, soff, 0, 0);
}

template <int D>
struct PassCfg {
  static constexpr int kRowU = D / 8 + 1;            // 16-byte units per padded key row
  static constexpr int kStride = kRowU * 16;         // bytes per padded key row in LDS
  static constexpr int kBytes = kChunk * kStride;    // one chunk in LDS
  static constexpr int kInstr = kBytes / 1024;       // copy instructions (1 KiB) per chunk
  static constexpr int kPer = (kInstr + kWaves - 1) / kWaves;
  static_assert(kBytes % 1024 == 0, "a chunk must be whole copy instructions");
};

// Cell maxima of one chunk (keys ck0 .. ck0 + 63) of the wave's 32 queries.
// S[kt][v] holds key ck0 + 32 kt + (v / 4) * 8 + 4 g + v % 4 of query l32.
// Returns the lane's maximum over its 32 scores.  The cell maxima the lane
// must store (query rq's cells that start below nsp; the padding keys of the
// last chunk have no cell) are left in `pend` (cell index, or -1 for none)
// and stored later by CellStores::flush, so that the wave does not wait for
// those stores before the next chunk.  K as in est_pass_kernel.
template <int K>
struct CellStores {
  static constexpr int kN = K >= 32 ? 1 : 32 / K;   // stores per lane per chunk
  int idx[kN];
  float val[kN];
  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int i = 0; i < kN; ++i) idx[i] = -1;
  }
  __device__ __forceinline__ void flush(float* trow) const {
#pragma unroll
    for (int i = 0; i < kN; ++i)
      if (idx[i] >= 0) trow[idx[i]] = val[i];
  }
};

template <int K>
__device__ __forceinline__ float cell_maxima(const f32x16_t (&S)[2], int ck0, int g, int cell_log2, int nsp,
                                             CellStores<K>& pend) {
  auto mx3 = [](float a, float b, float c) { return fmaxf(fmaxf(a, b), c); };
  auto max4 = [&](const f32x16_t& t, int v0) { return fmaxf(fmaxf(t[v0], t[v0 + 1]), fmaxf(t[v0 + 2], t[v0 + 3])); };
  auto max8 = [&](const f32x16_t& t, int v0) {
    return fmaxf(mx3(t[v0], t[v0 + 1], t[v0 + 2]), mx3(t[v0 + 3], mx3(t[v0 + 4], t[v0 + 5], t[v0 + 6]), t[v0 + 7]));
  };
  // Pair exchange across the wave halves: lanes of half 0 get max(a0, a1),
  // lanes of half 1 get max(b0, b1) (x0 from half 0, x1 from half 1).
  auto swap_max = [](float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  };
  auto put = [&](int i, bool ok, int cell, float v) {
    pend.idx[i] = ok ? cell : -1;
    pend.val[i] = v;
  };
  if constexpr (K >= 64) {
    const float x = fmaxf(fmaxf(max8(S[0], 0), max8(S[0], 8)), fmaxf(max8(S[1], 0), max8(S[1], 8)));
    const float c = swap_max(x, x);
    put(0, g == 0 && ck0 < nsp, ck0 >> cell_log2, c);
    return x;
  } else if constexpr (K == 32) {
    const float x0 = fmaxf(max8(S[0], 0), max8(S[0], 8)), x1 = fmaxf(max8(S[1], 0), max8(S[1], 8));
    const float c = swap_max(x0, x1);   // half 0: tile 0, half 1: tile 1
    put(0, ck0 + 32 * g < nsp, (ck0 + 32 * g) >> 5, c);
    return fmaxf(x0, x1);
  } else if constexpr (K == 16) {
    float x = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const float lo = max8(S[kt], 0), hi = max8(S[kt], 8);
      const float c = swap_max(lo, hi);   // half 0: keys 0-15 of the tile, half 1: keys 16-31
      const int key = ck0 + 32 * kt + 16 * g;
      put(kt, key < nsp, key >> 4, c);
      x = mx3(x, lo, hi);
    }
    return x;
  } else if constexpr (K == 8) {
    float x = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const float a = max4(S[kt], 8 * p), b = max4(S[kt], 8 * p + 4);
        const float c = swap_max(a, b);   // cells of keys 16p + 0-7 (half 0) and 16p + 8-15 (half 1)
        const int key = ck0 + 32 * kt + 16 * p + 8 * g;
        put(2 * kt + p, key < nsp, key >> 3, c);
        x = mx3(x, a, b);
      }
    }
    return x;
  } else {
    // K = 1, 2, 4: every cell lies inside one lane's run of 4 keys.
    float x = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int key = ck0 + 32 * kt + 8 * a4 + 4 * g;
        const float t[4] = {S[kt][4 * a4], S[kt][4 * a4 + 1], S[kt][4 * a4 + 2], S[kt][4 * a4 + 3]};
        const int base = (4 * kt + a4) * (4 / K);
        if constexpr (K == 4) {
          const float c = fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3]));
          put(base, key < nsp, key >> 2, c);
          x = fmaxf(x, c);
        } else if constexpr (K == 2) {
          const float c0 = fmaxf(t[0], t[1]), c1 = fmaxf(t[2], t[3]);
          put(base, key < nsp, key >> 1, c0);
          put(base + 1, key + 2 < nsp, (key >> 1) + 1, c1);
          x = mx3(x, c0, c1);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) put(base + e, key + e < nsp, key + e, t[e]);
          x = mx3(x, fmaxf(t[0], t[1]), fmaxf(t[2], t[3]));
        }
      }
    }
    return x;
  }
}

// K: the sample count k when k <= 32 (a cell is one block of K keys); 64
// stands for every k >= 64 (a cell is one 64-key chunk).  A compile-time
// constant, so the reductions are straight-line code.
//
// A workgroup of 8 wavefronts owns 256 sampled queries (32 per wavefront, Q^T
// in VGPRs) and one key split: S^T = K_s Q_s^T on 32x32x16 bf16 MFMAs, with
// the sampled keys gathered straight from the reordered K rows into
// double-buffered, row-padded LDS in chunks of 64 by the buffer form of the
// global -> LDS copy.  Each lane holds whole query columns, so the online
// (max, sum) runs per lane and the two wave halves merge at the end.
//
// Sampled slot r of a full block sits at reordered row r * (b / k) (k divides
// b), so a chunk of full blocks is 64 rows at a fixed stride and its copy
// offsets are one per-lane table plus a per-chunk scalar; chunks holding the
// last block's slots or padding use the exact rows (an empty slot reads row
// 0; its scores are masked to -inf).  Q rows are read the same way, from the
// reordered Q or, when tok.q is set, from the token of the sampled row.
template <int D, int K>
__global__ __launch_bounds__(kThreads) void est_pass_kernel(
    const __bf16* __restrict__ q_r, const __bf16* __restrict__ k_r, TokIO tok, int Npad, int Hh,
    float2* __restrict__ part, float* __restrict__ tmax, SampleGeom sg, float sl2) {
  using C = PassCfg<D>;
  // Distinct arrays with static roles in each half of the 2x-unrolled loop,
  // so the LDS reads of one are not made to wait for the copy into the other.
  __shared__ __attribute__((aligned(1024))) char Kc0[C::kBytes];
  __shared__ __attribute__((aligned(1024))) char Kc1[C::kBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  int bh, split, panel;
  wg_coords(sg, bh, split, panel);
  const int rq = panel * kQPerWg + wave * 32 + l32;
  const bool qok = rq < sg.nsp;

  // Copies: LDS byte 1024 n + 16 lane of a chunk holds padded unit p = 64 n +
  // lane, i.e. key row p / kRowU of the chunk, unit p % kRowU (the pad unit
  // repeats the row's last unit).  Surplus instructions repeat the chunk's
  // last one.
  // K rows per (batch, head): the reordered rows, or the gathered slot rows
  const int krows = sg.compact ? sg.nsp_pad : Npad;
  const auto rk = make_rsrc(k_r + (int64_t)bh * krows * D, (uint32_t)krows * (uint32_t)(D * 2));
  // rows between consecutive slots of a full block
  const int rstride = sg.compact ? 1 : sg.b >> sg.klog2;
  uint32_t voff[C::kPer];
#pragma unroll
  for (int i = 0; i < C::kPer; ++i) {
    const int n = min(wave + i * kWaves, C::kInstr - 1);
    const int p = 64 * n + lane;
    const int row = p / C::kRowU, c = min(p % C::kRowU, C::kRowU - 2);
    voff[i] = (uint32_t)(row * rstride * D * 2 + c * 16);
  }
  // From this slot on, chunks take the exact rows: the last block when it is
  // partial (its slots are spread over fewer than b rows), and the padding.
  // Every chunk takes them when the sample count is not a power of two.
  // (Gathered slot rows are read at unit stride throughout: their empty slots
  // and padding are zero rows, masked like the others.)
  const int exact_from = sg.compact ? sg.nsp_pad
                         : sg.kf < sg.k ? 0
                         : (sg.N < sg.nb * sg.b || sg.nsp % kChunk != 0) ? (sg.nb - 1) * sg.k : sg.nsp_pad;
  auto dma = [&](int ch, char* buf) {
    const int ck0 = ch * kChunk;
    if (ck0 + kChunk <= exact_from) {
#pragma unroll
      for (int i = 0; i < C::kPer; ++i) {
        const int n = min(wave + i * kWaves, C::kInstr - 1);
        copy16_lds(rk, buf + 1024 * n, voff[i], (uint32_t)ck0 * (uint32_t)(rstride * D * 2));
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::kPer; ++i) {
        const int n = min(wave + i * kWaves, C::kInstr - 1);
        const int p = 64 * n + lane;
        const int row = p / C::kRowU, c = min(p % C::kRowU, C::kRowU - 2);
        const int src = sg.row(ck0 + row);
        copy16_lds(rk, buf + 1024 * n, (uint32_t)((src < 0 ? 0 : src) * D * 2 + c * 16), 0u);
      }
    }
  };
  // The first chunk's copy is issued before the Q loads so that the two
  // latencies overlap.
  const int c0 = split * sg.cps, c1 = min(sg.nsp_pad / kChunk, c0 + sg.cps);
  dma(c0, Kc0);

  // Q^T operand: lane (l32, g) holds Q_s[rq][16 kk + 8 g .. +7]; zero for an
  // empty slot or padding.
  bf16x8_t qreg[D / 16];
  {
    const int src = sg.row(rq);
    if (src < 0) {
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) qreg[kk] = bf16x8_t{};
    } else if (tok.q == nullptr) {
      const __bf16* qp = q_r + ((int64_t)bh * Npad + src) * D + 8 * g;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) qreg[kk] = *reinterpret_cast<const bf16x8_t*>(qp + 16 * kk);
    } else {
      const int bi = bh / Hh, h = bh % Hh;
      int t = tok.perm[(int64_t)h * tok.perm_h_stride + src];
      t = t < 0 ? 0 : (t >= sg.N ? sg.N - 1 : t);
      const int64_t qo = bi * tok.qsb + (int64_t)t * tok.qsn + h * tok.qsh + 8 * g;
      if (tok.q_f32) {
        const float* qp = reinterpret_cast<const float*>(tok.q) + qo;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          const float4 a = reinterpret_cast<const float4*>(qp + 16 * kk)[0];
          const float4 c = reinterpret_cast<const float4*>(qp + 16 * kk)[1];
          const uint4 w = make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(c.x, c.y),
                                     pack_bf16x2(c.z, c.w));
          qreg[kk] = __builtin_bit_cast(bf16x8_t, w);
        }
      } else {
        const __bf16* qp = reinterpret_cast<const __bf16*>(tok.q) + qo;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) qreg[kk] = *reinterpret_cast<const bf16x8_t*>(qp + 16 * kk);
      }
    }
  }

  const int kbase = l32 * C::kStride + 16 * g;
  auto scores = [&](const char* kb, f32x16_t (&S)[2]) {
    S[0] = f32x16_t{};
    S[1] = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kb + kbase + kt * 32 * C::kStride + kk * 32);
        S[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[kk], S[kt], 0, 0, 0);
      }
    }
  };

  float m = -INFINITY, l = 0.f;
  float* trow = tmax + ((int64_t)bh * sg.nsp + (qok ? rq : 0)) * sg.ncell;
  CellStores<K> pend;
  pend.clear();
  // k = 16: the lane partial maxima of a chunk pair are completed across the
  // wave halves with one exchange per cell: half 0 finishes the pair's first
  // chunk and half 1 the second, so a lane stores its query's 4 cells of one
  // chunk as 16 contiguous bytes (and a query's 8 cells of the pair are 32).
  float held[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  float4 pv = make_float4(0.f, 0.f, 0.f, 0.f);
  int pcell = -1;                        // first cell of the pending 16-byte store, or -1
  const bool vec16 = (sg.ncell & 3) == 0 && (((uintptr_t)tmax) & 15u) == 0;
  auto pair16 = [&](int ch_first, const float (&px)[4]) {
    float c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(held[j]), __float_as_uint(px[j]), false, false);
      c[j] = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    pv = make_float4(c[0], c[1], c[2], c[3]);
    const int chunk = ch_first + g;
    pcell = chunk * kChunk < sg.nsp ? 4 * chunk : -1;
  };
  auto flush16 = [&]() {
    if (qok && pcell >= 0) {
      if (vec16 && 16 * (pcell + 3) < sg.nsp) {
        *reinterpret_cast<float4*>(trow + pcell) = pv;
      } else {
        const float vv[4] = {pv.x, pv.y, pv.z, pv.w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (16 * (pcell + j) < sg.nsp) trow[pcell + j] = vv[j];
      }
    }
    pcell = -1;
  };
  const int tail = (sg.nb - 1) * sg.k;   // first slot of the last block
  auto body = [&](int ch, f32x16_t (&S)[2], auto first) {
    const int ck0 = ch * kChunk;
    if (ck0 + kChunk > sg.nsp || (sg.kj_last < sg.k && ck0 + kChunk > tail) || sg.kf < sg.k) {
      // padding and empty slots score -inf (only the last chunks when the
      // sample count is a power of two)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (!sg.valid(ck0 + 32 * kt + (v >> 2) * 8 + 4 * g + (v & 3))) S[kt][v] = -INFINITY;
    }
    float mx;
    if constexpr (K == 16) {
      auto mx3 = [](float a, float b, float c) { return fmaxf(fmaxf(a, b), c); };
      auto max8 = [&](const f32x16_t& t, int v0) {
        return fmaxf(mx3(t[v0], t[v0 + 1], t[v0 + 2]), mx3(t[v0 + 3], mx3(t[v0 + 4], t[v0 + 5], t[v0 + 6]), t[v0 + 7]));
      };
      const float px[4] = {max8(S[0], 0), max8(S[0], 8), max8(S[1], 0), max8(S[1], 8)};
      if constexpr (decltype(first)::value) {
#pragma unroll
        for (int j = 0; j < 4; ++j) held[j] = px[j];
      } else {
        pair16(ch - 1, px);
      }
      mx = fmaxf(fmaxf(px[0], px[1]), fmaxf(px[2], px[3])) * sl2;
    } else {
      mx = cell_maxima<K>(S, ck0, g, sg.cell_log2, sg.nsp, pend) * sl2;
    }
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    float s0 = l * fast_exp2(m - m_use), s1 = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      s0 += fast_exp2(__builtin_fmaf(S[0][v], sl2, -m_use));
      s1 += fast_exp2(__builtin_fmaf(S[1][v], sl2, -m_use));
    }
    l = s0 + s1;
    m = m_new;
  };

  f32x16_t S[2];
  // The cell maxima of a chunk are stored after the next chunk's barrier, so
  // they have a whole chunk to complete before the next wait for the copies
  // (which also waits for stores).
  for (int ch = c0; ch < c1; ch += 2) {
    wait_dma();
    __syncthreads();
    if (ch + 1 < c1) dma(ch + 1, Kc1);
    if constexpr (K == 16) {
      flush16();
    } else {
      if (qok) pend.flush(trow);
    }
    scores(Kc0, S);
    body(ch, S, std::true_type{});
    if (ch + 1 < c1) {
      wait_dma();
      __syncthreads();
      if (ch + 2 < c1) dma(ch + 2, Kc0);
      if constexpr (K != 16) {
        if (qok) pend.flush(trow);
      }
      scores(Kc1, S);
      body(ch + 1, S, std::false_type{});
    }
  }
  if constexpr (K == 16) {
    if (((c1 - c0) & 1) != 0) {   // the last chunk had no partner: half 0 completes it
      const float none[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      pair16(c1 - 1, none);
      if (g == 1) pcell = -1;
    }
    flush16();
  } else {
    if (qok) pend.flush(trow);
  }
  // merge the two wave halves (each saw half of every chunk's keys)
  const auto rm = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  const float M = fmaxf(__uint_as_float(rm[0]), __uint_as_float(rm[1]));
  const float mine = (M == -INFINITY) ? 0.f : l * fast_exp2(m - M);
  const auto rl = __builtin_amdgcn_permlane32_swap(__float_as_uint(mine), __float_as_uint(mine), false, false);
  const float L = __uint_as_float(rl[0]) + __uint_as_float(rl[1]);
  if (g == 0 && qok) part[((int64_t)bh * sg.splits + split) * sg.nsp + rq] = make_float2(M, L);
}

// log2 of the softmax normaliser of sampled query rq from its per-split partials.
// The splits are merged in one sweep with a running maximum (the partials of
// up to 8 splits are loaded together).
__device__ __forceinline__ float merge_lse2(const float2* part_bh, const SampleGeom& sg, int rq) {
  float M = -INFINITY, L = 0.f;
  for (int s0 = 0; s0 < sg.splits; s0 += 8) {
    float2 p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      p[e] = s0 + e < sg.splits ? part_bh[(int64_t)(s0 + e) * sg.nsp + rq] : make_float2(-INFINITY, 0.f);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float Mn = fmaxf(M, p[e].x);
      if (Mn != -INFINITY) L = L * fast_exp2(M - Mn) + p[e].y * fast_exp2(p[e].x - Mn);
      M = Mn;
    }
  }
  return M == -INFINITY ? INFINITY : M + __log2f(L);
}

// P_imp of one (batch, head, query block I) row: lse2 of the block's valid
// sampled queries from the split partials (in LDS), then for every key block
// J the maximum over those queries of sl2 * t_qJ - lse2_q, and one exp2.
// An empty query slot contributes nothing; a block without valid query slots
// (impossible: k_J >= 1) would get exp2(-inf) = 0.
constexpr int kFinalThreads = 256;
constexpr int kMaxK = 128;   // k <= b <= 128

// The lse2 values of query block I's sampled queries (slots >= k_I: +inf),
// written by threads lane0 .. lane0 + k - 1 of the calling group.
__device__ __forceinline__ void row_lse(const float2* __restrict__ part, const SampleGeom& sg, int bh, int I,
                                        int kI, float* lse, int i) {
  if (i < sg.k) {
    const int rq = I * sg.k + i;
    lse[i] = i < kI ? merge_lse2(part + (int64_t)bh * sg.splits * sg.nsp, sg, rq) : INFINITY;
  }
}

// P_imp[I, J] from the row's lse2 values and the block maxima of its sampled
// queries (t0: the first of them).  Max is exact, so the order of the terms
// does not change the result.
__device__ __forceinline__ float pimp_value(const float* lse, const float* __restrict__ t0, const SampleGeom& sg,
                                            int kI, int J, float sl2) {
  const int cpb = sg.ncell / sg.nb;   // cells per block: 1, or k / 64
  float best = -INFINITY;
  // 8 sampled queries at a time, their loads issued together
  for (int t0q = 0; t0q < kI; t0q += 8) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = min(t0q + e, kI - 1);
      const float* tr = t0 + (int64_t)t * sg.ncell + J * cpb;
      v[e] = tr[0];
      for (int c = 1; c < cpb; ++c) v[e] = fmaxf(v[e], tr[c]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = min(t0q + e, kI - 1);
      best = fmaxf(best, __builtin_fmaf(v[e], sl2, -lse[t]));
    }
  }
  return fast_exp2(best);
}

__global__ __launch_bounds__(kFinalThreads) void est_final_kernel(const float2* __restrict__ part,
                                                                  const float* __restrict__ tmax,
                                                                  float* __restrict__ p_imp, SampleGeom sg,
                                                                  float sl2) {
  __shared__ float lse[kMaxK];
  const int I = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int kI = I < sg.nb - 1 ? sg.kf : sg.kj_last;
  row_lse(part, sg, bh, I, kI, lse, tid);
  __syncthreads();
  const float* t0 = tmax + ((int64_t)bh * sg.nsp + (int64_t)I * sg.k) * sg.ncell;
  float* prow = p_imp + ((int64_t)bh * sg.nb + I) * sg.nb;
  for (int J = tid; J < sg.nb; J += kFinalThreads) prow[J] = pimp_value(lse, t0, sg, kI, J, sl2);
}

// The lane's KPL consecutive P_imp entries J = lane * KPL + r of one row, all
// loads of a group of 16 sampled queries in flight together.  vec: one block
// per cell and 4 * KPL-byte aligned rows, so each sampled query's KPL maxima
// arrive in one vector load (a wavefront reads a contiguous row).  Same terms
// and the same exact max as pimp_value, so the same bits.
template <int KPL>
__device__ __forceinline__ void pimp_lane(const float* lse, const float* __restrict__ t0, const SampleGeom& sg, int kI,
                                          int lane, float sl2, bool vec, uint32_t (&out)[KPL]) {
  float best[KPL];
#pragma unroll
  for (int r = 0; r < KPL; ++r) best[r] = -INFINITY;
  const int J0 = lane * KPL;
  if (vec) {
    typedef float vf __attribute__((ext_vector_type(KPL)));
    if (J0 < sg.nb) {
      for (int t0q = 0; t0q < kI; t0q += 16) {
        vf v[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int t = min(t0q + e, kI - 1);
          v[e] = *reinterpret_cast<const vf*>(t0 + (int64_t)t * sg.ncell + J0);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float l = lse[min(t0q + e, kI - 1)];
#pragma unroll
          for (int r = 0; r < KPL; ++r) best[r] = fmaxf(best[r], __builtin_fmaf(v[e][r], sl2, -l));
        }
      }
    }
  } else {
    const int cpb = sg.ncell / sg.nb;
    for (int t0q = 0; t0q < kI; t0q += 8) {
      float v[8][KPL];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = min(t0q + e, kI - 1);
#pragma unroll
        for (int r = 0; r < KPL; ++r) {
          const int J = min(J0 + r, sg.nb - 1);
          const float* tr = t0 + (int64_t)t * sg.ncell + J * cpb;
          v[e][r] = tr[0];
          for (int c = 1; c < cpb; ++c) v[e][r] = fmaxf(v[e][r], tr[c]);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float l = lse[min(t0q + e, kI - 1)];
#pragma unroll
        for (int r = 0; r < KPL; ++r) best[r] = fmaxf(best[r], __builtin_fmaf(v[e][r], sl2, -l));
      }
    }
  }
#pragma unroll
  for (int r = 0; r < KPL; ++r) out[r] = J0 + r < sg.nb ? __float_as_uint(fast_exp2(best[r])) : 0u;
}

// The final step fused with the block selection (estimate and mask in one
// pass, as SPADE's prepass suggests): each P_imp row goes from registers
// straight into the mask selection and reaches HBM only when p_imp is given.
// Rows of up to 256 blocks: one wavefront per row, four per workgroup; lane l
// forms entries l * KPL .. l * KPL + KPL - 1, the layout the register sort
// takes.
template <int KPL>
__global__ __launch_bounds__(256) void est_mask_wave_kernel(const float2* __restrict__ part,
                                                            const float* __restrict__ tmax, SampleGeom sg, float sl2,
                                                            maskcore::Rule rule, float* __restrict__ p_imp,
                                                            int32_t* __restrict__ kv_count,
                                                            int32_t* __restrict__ kv_idx,
                                                            uint8_t* __restrict__ mask) {
  __shared__ float lse_all[4][kMaxK];
  __shared__ uint8_t flag_all[4][64 * KPL];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int I = blockIdx.x * 4 + w, bh = blockIdx.y;
  if (I >= sg.nb) return;   // whole wavefronts; no workgroup barrier follows
  const int kI = I < sg.nb - 1 ? sg.kf : sg.kj_last;
  float* lse = lse_all[w];
  for (int i = lane; i < sg.k; i += 64) row_lse(part, sg, bh, I, kI, lse, i);
  __builtin_amdgcn_wave_barrier();
  const int64_t row = (int64_t)bh * sg.nb + I;
  const float* t0 = tmax + ((int64_t)bh * sg.nsp + (int64_t)I * sg.k) * sg.ncell;
  const bool vec = sg.ncell == sg.nb && sg.nb % KPL == 0 && ((uintptr_t)tmax & (4 * KPL - 1)) == 0;
  uint32_t in[KPL];
  pimp_lane<KPL>(lse, t0, sg, kI, lane, sl2, vec, in);
  if (p_imp != nullptr) {
#pragma unroll
    for (int r = 0; r < KPL; ++r)
      if (lane * KPL + r < sg.nb) p_imp[row * sg.nb + lane * KPL + r] = __uint_as_float(in[r]);
  }
  maskcore::mask_row_wave<KPL>(in, row, sg.nb, rule, flag_all[w], kv_count, kv_idx, mask);
}

// Rows of 257..4096 blocks: one wavefront per row (four per workgroup), in
// two steps.  First the row's P_imp values are formed with coalesced loads
// (lane l forms entries 256 g + 4 l .. + 3 of each 256-entry group g, one
// 16-byte load per sampled query, pimp_value's terms, so the same bits) and
// parked in the wavefront's LDS area; then lane l takes entries l * KPL ..
// l * KPL + KPL - 1 from there, the layout of the radix selection, which
// reuses the same LDS area for its counters.
template <int KPL>
__global__ __launch_bounds__(256) void est_mask_radix_kernel(const float2* __restrict__ part,
                                                             const float* __restrict__ tmax, SampleGeom sg, float sl2,
                                                             maskcore::Rule rule, float* __restrict__ p_imp,
                                                             int32_t* __restrict__ kv_count,
                                                             int32_t* __restrict__ kv_idx,
                                                             uint8_t* __restrict__ mask) {
  constexpr int kWords = maskcore::RadixArea<KPL>::kWords;
  __shared__ float lse_all[4][kMaxK];
  __shared__ __attribute__((aligned(16))) unsigned long long area_all[4][kWords];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int I = blockIdx.x * 4 + w, bh = blockIdx.y;
  if (I >= sg.nb) return;   // whole wavefronts; no workgroup barrier follows
  const int kI = I < sg.nb - 1 ? sg.kf : sg.kj_last;
  float* lse = lse_all[w];
  for (int i = lane; i < sg.k; i += 64) row_lse(part, sg, bh, I, kI, lse, i);
  __builtin_amdgcn_wave_barrier();
  const int64_t row = (int64_t)bh * sg.nb + I;
  const float* t0 = tmax + ((int64_t)bh * sg.nsp + (int64_t)I * sg.k) * sg.ncell;
  float* pv = reinterpret_cast<float*>(area_all[w]);
  float* prow = p_imp != nullptr ? p_imp + row * sg.nb : nullptr;
  const bool vec = sg.ncell == sg.nb && sg.nb % 4 == 0 && ((uintptr_t)tmax & 15u) == 0;
  if (vec) {
#pragma unroll 1
    for (int g = 0; g < KPL / 4; ++g) {
      const int J = 256 * g + 4 * lane;
      const bool ok = J < sg.nb;   // nb % 4 == 0: then all four entries are
      const int Jc = ok ? J : 0;
      float best[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      for (int t0q = 0; t0q < kI; t0q += 16) {
        float4 vv[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int t = min(t0q + e, kI - 1);
          vv[e] = *reinterpret_cast<const float4*>(t0 + (int64_t)t * sg.ncell + Jc);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float l = lse[min(t0q + e, kI - 1)];
          best[0] = fmaxf(best[0], __builtin_fmaf(vv[e].x, sl2, -l));
          best[1] = fmaxf(best[1], __builtin_fmaf(vv[e].y, sl2, -l));
          best[2] = fmaxf(best[2], __builtin_fmaf(vv[e].z, sl2, -l));
          best[3] = fmaxf(best[3], __builtin_fmaf(vv[e].w, sl2, -l));
        }
      }
      float4 pq = make_float4(0.f, 0.f, 0.f, 0.f);
      if (ok) {
        pq = make_float4(fast_exp2(best[0]), fast_exp2(best[1]), fast_exp2(best[2]), fast_exp2(best[3]));
        if (prow != nullptr) *reinterpret_cast<float4*>(prow + J) = pq;
      }
      *reinterpret_cast<float4*>(pv + J) = pq;
    }
  } else {
#pragma unroll 1
    for (int r = 0; r < KPL; ++r) {
      const int J = 64 * r + lane;
      float v = 0.f;
      if (J < sg.nb) {
        v = pimp_value(lse, t0, sg, kI, J, sl2);
        if (prow != nullptr) prow[J] = v;
      }
      pv[J] = v;
    }
  }
  uint32_t in[KPL];
  maskcore::gather_lane_entries<KPL>(pv, lane, in);
  maskcore::mask_row_radix<KPL>(in, row, sg.nb, rule, area_all[w], kv_count, kv_idx, mask);
}

// The sampled K rows gathered from K in token order into the layout the pass
// reads at unit stride: row r of (batch, head) holds K at the token of
// sampled slot r, as dbs_reorder_kv's k_r holds it (bf16; float32 rounded to
// nearest even), and zeros for an empty slot or padding.  One thread per
// 16-byte chunk of a row.
template <int D>
__global__ __launch_bounds__(256) void gather_sampled_k_kernel(const void* __restrict__ key, int k_f32, int64_t sb,
                                                               int64_t sn, int64_t sh,
                                                               const int32_t* __restrict__ perm, int perm_h_stride,
                                                               int Hh, SampleGeom sg, __bf16* __restrict__ k_s) {
  constexpr int kCpr = D / 8;   // 16-byte chunks per bf16 row
  const int bh = blockIdx.y, bi = bh / Hh, h = bh % Hh;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)sg.nsp_pad * kCpr) return;
  const int r = (int)(i / kCpr), c = (int)(i % kCpr);
  const int row = sg.row(r);
  uint4 o = make_uint4(0u, 0u, 0u, 0u);
  if (row >= 0) {
    int t = perm[(int64_t)h * perm_h_stride + row];
    t = t < 0 ? 0 : (t >= sg.N ? sg.N - 1 : t);
    const int64_t off = bi * sb + (int64_t)t * sn + (int64_t)h * sh + 8 * c;
    if (k_f32) {
      const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(key) + off);
      const float4 a = p[0], b = p[1];
      o = make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y), pack_bf16x2(b.z, b.w));
    } else {
      o = *reinterpret_cast<const uint4*>(reinterpret_cast<const __bf16*>(key) + off);
    }
  }
  *reinterpret_cast<uint4*>(k_s + ((int64_t)bh * sg.nsp_pad + r) * D + 8 * c) = o;
}

// Key splits: about 768 workgroups in total (one and a half rounds of two
// 8-wavefront workgroups per CU), each streaming a contiguous range of 64-key
// chunks.  On the Wan-shaped layer, 768 measured 3 us faster than 1536 and
// 10 us faster than 576.
void split_plan(int BH, int nsp, int& splits, int& cps) {
  const int nsp_pad = (nsp + kChunk - 1) / kChunk * kChunk;
  const int nchunks = nsp_pad / kChunk;
  const int panels = (nsp + kQPerWg - 1) / kQPerWg;
  const int64_t wgs = (int64_t)panels * BH;
  int want = (int)((768 + wgs - 1) / wgs);
  want = want < 1 ? 1 : (want > nchunks ? nchunks : want);
  cps = (nchunks + want - 1) / want;
  if (cps > kMaxChunksPerSplit) cps = kMaxChunksPerSplit;
  splits = (nchunks + cps - 1) / cps;
}

template <int D>
hipError_t launch_d(const EstimateArgs& a) {
  SampleGeom sg;
  sg.N = a.N; sg.b = a.b; sg.nb = a.nb;
  sg.klog2 = 0;
  while ((1 << sg.klog2) < a.k) ++sg.klog2;
  sg.k = 1 << sg.klog2;
  sg.kf = a.k;
  sg.nsp = a.nb * sg.k;
  sg.nsp_pad = (sg.nsp + kChunk - 1) / kChunk * kChunk;
  sg.cell_log2 = sg.klog2 < 6 ? sg.klog2 : 6;
  sg.ncell = sg.nsp >> sg.cell_log2;
  const int Llast = a.N - (a.nb - 1) * a.b;
  sg.kj_last = a.k < Llast ? a.k : Llast;
  const float sl2 = a.scale * kLog2e;
  const int BH = a.B * a.Hh;
  split_plan(BH, sg.nsp, sg.splits, sg.cps);
  float2* part = reinterpret_cast<float2*>(a.workspace);
  float* tmax = reinterpret_cast<float*>(part + (int64_t)BH * sg.splits * sg.nsp);
  const __bf16* qr = (const __bf16*)a.q_r;
  const __bf16* kr = (const __bf16*)a.k_r;
  sg.compact = 0;
  if (a.k_tok != nullptr) {
    const size_t off = (estimate_workspace_bytes(a.B, a.Hh, a.nb, a.k, D) + 255) / 256 * 256;
    __bf16* ks = reinterpret_cast<__bf16*>(reinterpret_cast<char*>(a.workspace) + off);
    const int64_t chunks = (int64_t)sg.nsp_pad * (D / 8);
    hipLaunchKernelGGL((gather_sampled_k_kernel<D>), dim3((unsigned)((chunks + 255) / 256), (unsigned)BH), dim3(256),
                       0, a.stream, a.k_tok, a.k_f32, a.ksb, a.ksn, a.ksh, a.tok.perm, a.tok.perm_h_stride, a.Hh, sg,
                       ks);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    kr = ks;
    sg.compact = 1;
  }
  dim3 grid((unsigned)(((sg.nsp + kQPerWg - 1) / kQPerWg) * sg.splits * BH));
  switch (sg.k) {
    case 1: hipLaunchKernelGGL((est_pass_kernel<D, 1>), grid, dim3(kThreads), 0, a.stream, qr, kr, a.tok, a.Npad, a.Hh, part, tmax, sg, sl2); break;
    case 2: hipLaunchKernelGGL((est_pass_kernel<D, 2>), grid, dim3(kThreads), 0, a.stream, qr, kr, a.tok, a.Npad, a.Hh, part, tmax, sg, sl2); break;
    case 4: hipLaunchKernelGGL((est_pass_kernel<D, 4>), grid, dim3(kThreads), 0, a.stream, qr, kr, a.tok, a.Npad, a.Hh, part, tmax, sg, sl2); break;
    case 8: hipLaunchKernelGGL((est_pass_kernel<D, 8>), grid, dim3(kThreads), 0, a.stream, qr, kr, a.tok, a.Npad, a.Hh, part, tmax, sg, sl2); break;
    case 16: hipLaunchKernelGGL((est_pass_kernel<D, 16>), grid, dim3(kThreads), 0, a.stream, qr, kr, a.tok, a.Npad, a.Hh, part, tmax, sg, sl2); break;
    case 32: hipLaunchKernelGGL((est_pass_kernel<D, 32>), grid, dim3(kThreads), 0, a.stream, qr, kr, a.tok, a.Npad, a.Hh, part, tmax, sg, sl2); break;
    default: hipLaunchKernelGGL((est_pass_kernel<D, 64>), grid, dim3(kThreads), 0, a.stream, qr, kr, a.tok, a.Npad, a.Hh, part, tmax, sg, sl2); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.fuse == nullptr) {
    hipLaunchKernelGGL(est_final_kernel, dim3((unsigned)a.nb, (unsigned)BH), dim3(kFinalThreads), 0, a.stream,
                       (const float2*)part, (const float*)tmax, a.p_imp, sg, sl2);
    return hipGetLastError();
  }
  const MaskArgs& m = *a.fuse;
  const maskcore::Rule rule = maskcore::make_rule(m.rule, m.tau, m.topk, m.u);
  const float2* cp = part;
  const float* ct = tmax;
  const dim3 wgrid((unsigned)((a.nb + 3) / 4), (unsigned)BH);
  if (a.nb <= 64) {
    hipLaunchKernelGGL((est_mask_wave_kernel<1>), wgrid, dim3(256), 0, a.stream, cp, ct, sg, sl2, rule, a.p_imp,
                       m.kv_count, m.kv_idx, m.mask);
  } else if (a.nb <= 128) {
    hipLaunchKernelGGL((est_mask_wave_kernel<2>), wgrid, dim3(256), 0, a.stream, cp, ct, sg, sl2, rule, a.p_imp,
                       m.kv_count, m.kv_idx, m.mask);
  } else if (a.nb <= 256) {
    hipLaunchKernelGGL((est_mask_wave_kernel<4>), wgrid, dim3(256), 0, a.stream, cp, ct, sg, sl2, rule, a.p_imp,
                       m.kv_count, m.kv_idx, m.mask);
  } else if (a.nb <= 512) {
    hipLaunchKernelGGL((est_mask_radix_kernel<8>), wgrid, dim3(256), 0, a.stream, cp, ct, sg, sl2, rule, a.p_imp,
                       m.kv_count, m.kv_idx, m.mask);
  } else if (a.nb <= 1024) {
    hipLaunchKernelGGL((est_mask_radix_kernel<16>), wgrid, dim3(256), 0, a.stream, cp, ct, sg, sl2, rule, a.p_imp,
                       m.kv_count, m.kv_idx, m.mask);
  } else if (a.nb <= 1280) {
    hipLaunchKernelGGL((est_mask_radix_kernel<20>), wgrid, dim3(256), 0, a.stream, cp, ct, sg, sl2, rule, a.p_imp,
                       m.kv_count, m.kv_idx, m.mask);
  } else if (a.nb <= 2048) {
    hipLaunchKernelGGL((est_mask_radix_kernel<32>), wgrid, dim3(256), 0, a.stream, cp, ct, sg, sl2, rule, a.p_imp,
                       m.kv_count, m.kv_idx, m.mask);
  } else {
    hipLaunchKernelGGL((est_mask_radix_kernel<64>), wgrid, dim3(256), 0, a.stream, cp, ct, sg, sl2, rule, a.p_imp,
                       m.kv_count, m.kv_idx, m.mask);
  }
  if (m.order != nullptr) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_build_order(m);
  }
  return hipGetLastError();
}

}  // namespace

size_t estimate_kvtok_workspace_bytes(int B, int Hh, int nb, int k, int d) {
  int kp = 1;
  while (kp < k) kp <<= 1;
  const int64_t nsp_pad = ((int64_t)nb * kp + kChunk - 1) / kChunk * kChunk;
  return (estimate_workspace_bytes(B, Hh, nb, k, d) + 255) / 256 * 256 +
         (size_t)((int64_t)B * Hh * nsp_pad * d * 2);
}

size_t estimate_workspace_bytes(int B, int Hh, int nb, int k, int d) {
  int kp = 1;
  while (kp < k) kp <<= 1;
  const int64_t nsp = (int64_t)nb * kp;
  const int64_t nsp_pad = (nsp + kChunk - 1) / kChunk * kChunk;
  const int64_t BH = (int64_t)B * Hh;
  int splits, cps;
  split_plan((int)BH, (int)nsp, splits, cps);
  int klog2 = 0;
  while ((1 << klog2) < k) ++klog2;
  const int64_t cells = nsp >> (klog2 < 6 ? klog2 : 6);
  (void)nsp_pad;
  (void)d;
  return (size_t)(BH * splits * nsp * 8 + BH * nsp * cells * 4);
}

hipError_t launch_estimate(const EstimateArgs& a) {
  return a.d == 64 ? launch_d<64>(a) : launch_d<128>(a);
}

}  // namespace dbs
