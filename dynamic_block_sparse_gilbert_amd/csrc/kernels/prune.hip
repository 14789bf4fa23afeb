// BSA query pruning and token filling (gfx950).
//
// The BSA notes, key design 1: inside each query block, tokens nearly
// parallel to their window's centre token are left out of the attention and
// later take the centre's output.  A block of n valid tokens holding c centres
// keeps m = min(n, max(ceil(r * n), c)) rows: its centres (their outputs are
// needed for the filling) and the m - c other tokens of largest
// 1 - cos(q_centre, q_i), ties by smaller row.
//
// query_prune_kernel: one workgroup of 128 threads per (batch, head, block).
// Each thread first reads its row's token, centre and the centre's token.  The
// dissimilarities are then formed with D / 8 (bf16) or D / 4 (float32) lanes
// per row, 16 bytes each, so a wavefront's loads cover whole rows and a batch
// of them is in flight at once; each row's dot product and squared norms (in
// float32 from the bf16 values) are summed across its lanes.  Each thread
// then ranks its token among the block's non-centre tokens by counting, over
// the block's values in LDS, those that order before it.  A workgroup scan of
// the kept flags writes the kept rows in ascending order.
// fill_pruned_kernel: after the attention over the kept rows, every pruned
// row copies its centre's output row (and log-sum-exp), 16 bytes per thread.
#include <cmath>
#include <type_traits>

#include "common.h"
#include "../launch.h"

namespace dbs {
namespace {

constexpr int kPruneThreads = 128;   // >= b

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Sum over aligned groups of L lanes (L = 8, 16 or 32), in every lane of
// the group: DPP steps within rows of 16 lanes (neighbour pairs,
// pairs of pairs, then the row's two halves and its whole), and one exchange
// across rows for L = 32.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  auto dpp = [](float x, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value, 0xF, 0xF, false));
  };
  v += dpp(v, std::integral_constant<int, 0xB1>{});    // quad_perm [1, 0, 3, 2]
  v += dpp(v, std::integral_constant<int, 0x4E>{});    // quad_perm [2, 3, 0, 1]
  v += dpp(v, std::integral_constant<int, 0x141>{});   // row_half_mirror
  if constexpr (L >= 16) v += dpp(v, std::integral_constant<int, 0x140>{});   // row_mirror
  if constexpr (L == 32) v += __shfl_xor(v, 16, 64);
  return v;
}

template <int D, bool F32>
__global__ __launch_bounds__(kPruneThreads) void query_prune_kernel(PruneArgs a) {
  __shared__ int tok_s[2][kPruneThreads];   // token of the row, token of its centre
  __shared__ __attribute__((aligned(16))) float dis_s[kPruneThreads];
  __shared__ int cls_s[kPruneThreads];      // 0 invalid row, 1 centre, 2 other token
  __shared__ int wave_cnt[kPruneThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int I = blockIdx.x, bh = blockIdx.y;
  const int bi = bh / a.Hh, hh = bh % a.Hh;
  const int R = I * a.b + tid;
  const bool valid = tid < a.b && R < a.N;
  const int32_t* perm = a.perm + (int64_t)hh * a.perm_h_stride;
  const int32_t* anc = a.anchor + (int64_t)hh * a.perm_h_stride;
  auto clamp_n = [&](int t) { return t < 0 ? 0 : (t >= a.N ? a.N - 1 : t); };

  // The row's token and centre first; a centre inside the block (always so
  // when the windows nest in the blocks) takes its token from LDS.
  int cls = 0, tR = 0, A = 0;
  if (valid) {
    A = clamp_n(anc[R]);
    tR = clamp_n(perm[R]);
    cls = A == R ? 1 : 2;
  }
  tok_s[0][tid] = tR;
  __syncthreads();
  int tA = 0;
  if (valid) {
    const int Ab = A - I * a.b;
    tA = (Ab >= 0 && Ab < a.b) ? tok_s[0][Ab] : clamp_n(perm[A]);
  }
  tok_s[1][tid] = tA;
  cls_s[tid] = cls;
  __syncthreads();

  // Row `row` of the workgroup: lanes sub * LR .. of a group of LR lanes, 16
  // bytes each; wavefront w takes rows 64 w .. 64 w + 63, RPI per iteration.
  constexpr int kEl = F32 ? 4 : 8, LR = D / kEl, RPI = 64 / LR, IT = LR;
  constexpr int kBatch = IT < 8 ? IT : 8;
  const int sub = lane / LR, li = lane % LR;
  const int64_t es = F32 ? 4 : 2;
  const char* qbase = reinterpret_cast<const char*>(a.q) + (bi * a.qsb + hh * a.qsh) * es + 16 * li;
  const int64_t tstride = a.qsn * es;   // bytes between tokens
#pragma unroll
  for (int it0 = 0; it0 < IT; it0 += kBatch) {
    uint4 x[kBatch], y[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int row = wave * 64 + (it0 + j) * RPI + sub;
      x[j] = *reinterpret_cast<const uint4*>(qbase + tok_s[0][row] * tstride);
      y[j] = *reinterpret_cast<const uint4*>(qbase + tok_s[1][row] * tstride);
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const uint32_t xw[4] = {x[j].x, x[j].y, x[j].z, x[j].w}, yw[4] = {y[j].x, y[j].y, y[j].z, y[j].w};
      float dot = 0.f, nq = 0.f, na = 0.f;
      if constexpr (F32) {
        // the float32 input rounded to bf16, as the attention reads it
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = bf16_bits_to_f32(f32_to_bf16_bits(__uint_as_float(xw[e])));
          const float y0 = bf16_bits_to_f32(f32_to_bf16_bits(__uint_as_float(yw[e])));
          dot = __builtin_fmaf(x0, y0, dot);
          nq = __builtin_fmaf(x0, x0, nq);
          na = __builtin_fmaf(y0, y0, na);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = bf16_lo(xw[e]), x1 = bf16_hi(xw[e]), y0 = bf16_lo(yw[e]), y1 = bf16_hi(yw[e]);
          dot = __builtin_fmaf(x0, y0, __builtin_fmaf(x1, y1, dot));
          nq = __builtin_fmaf(x0, x0, __builtin_fmaf(x1, x1, nq));
          na = __builtin_fmaf(y0, y0, __builtin_fmaf(y1, y1, na));
        }
      }
      dot = group_sum<LR>(dot);
      nq = group_sum<LR>(nq);
      na = group_sum<LR>(na);
      const int row = wave * 64 + (it0 + j) * RPI + sub;
      if (li == LR - 1) {
        // a row that is not a candidate (centre or invalid) is stored as -inf,
        // so it never orders before a candidate below
        float dis = -INFINITY;
        if (cls_s[row] == 2) {
          if (nq == 0.f || na == 0.f) {
            dis = nq == na ? 0.f : 1.f;
          } else {
            dis = 1.f - dot / (sqrtf(nq) * sqrtf(na));
          }
        }
        dis_s[row] = dis;
      }
    }
  }
  const int n_valid = __syncthreads_count(valid);   // also orders the dis_s writes before the reads
  const int n_centre = __syncthreads_count(cls == 1);
  const int m = min(n_valid, max((int)ceil(a.r * (double)n_valid), n_centre));
  const int take = m - n_centre;
  bool keep = cls == 1;
  if (cls == 2) {
    // rank among the candidates: larger dissimilarity first, ties by smaller row
    const float dis = dis_s[tid];
    int rank = 0;
#pragma unroll 8
    for (int j4 = 0; j4 < kPruneThreads / 4; ++j4) {
      const float4 d4 = reinterpret_cast<const float4*>(dis_s)[j4];
      const float dj[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) rank += (dj[e] > dis || (dj[e] == dis && 4 * j4 + e < tid)) ? 1 : 0;
    }
    keep = rank < take;
  }
  // ascending compaction of the kept rows
  const uint64_t ball = __ballot(keep);
  if (lane == 0) wave_cnt[wave] = __popcll(ball);
  __syncthreads();
  int pos = __popcll(ball & ((1ull << lane) - 1ull));
  for (int w = 0; w < wave; ++w) pos += wave_cnt[w];
  const int64_t row = (int64_t)bh * a.nb + I;
  int32_t* sel = a.rowsel + row * a.b;
  if (keep) sel[pos] = R;
  if (tid < a.b && tid >= m) sel[tid] = -1;
  if (tid < a.b) a.keep[(int64_t)bh * a.Npad + I * a.b + tid] = keep ? 1 : 0;
  if (tid == 0) a.q_count[row] = m;
}

// One thread per 16-byte chunk of a row; rows whose keep flag is 0 take their
// centre's output row and log-sum-exp.
__global__ __launch_bounds__(256) void fill_pruned_kernel(FillArgs a) {
  const int cpr = a.row_bytes / 16;                      // chunks per row
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)a.B * a.Hh * a.N * cpr;
  if (gid >= total) return;
  const int c = (int)(gid % cpr);
  const int64_t rr = gid / cpr;
  const int R = (int)(rr % a.N);
  const int bh = (int)(rr / a.N);
  const int bi = bh / a.Hh, hh = bh % a.Hh;
  if (a.keep[(int64_t)bh * a.Npad + R] != 0) return;
  const int32_t* perm = a.perm + (int64_t)hh * a.perm_h_stride;
  int A = a.anchor[(int64_t)hh * a.perm_h_stride + R];
  A = A < 0 ? 0 : (A >= a.N ? a.N - 1 : A);
  auto tok = [&](int row) {
    const int t = perm[row];
    return t < 0 ? 0 : (t >= a.N ? a.N - 1 : t);
  };
  const int64_t es = a.out_f32 ? 4 : 2;
  char* base = reinterpret_cast<char*>(a.out) + (bi * a.osb + hh * a.osh) * es;
  const uint4 v = *reinterpret_cast<const uint4*>(base + (int64_t)tok(A) * a.osn * es + c * 16);
  *reinterpret_cast<uint4*>(base + (int64_t)tok(R) * a.osn * es + c * 16) = v;
  if (a.lse != nullptr && c == 0) a.lse[(int64_t)bh * a.Npad + R] = a.lse[(int64_t)bh * a.Npad + A];
}

}  // namespace

hipError_t launch_query_prune(const PruneArgs& a) {
  const dim3 grid((unsigned)a.nb, (unsigned)(a.B * a.Hh));
  if (a.d == 64) {
    if (a.q_f32) hipLaunchKernelGGL((query_prune_kernel<64, true>), grid, dim3(kPruneThreads), 0, a.stream, a);
    else hipLaunchKernelGGL((query_prune_kernel<64, false>), grid, dim3(kPruneThreads), 0, a.stream, a);
  } else {
    if (a.q_f32) hipLaunchKernelGGL((query_prune_kernel<128, true>), grid, dim3(kPruneThreads), 0, a.stream, a);
    else hipLaunchKernelGGL((query_prune_kernel<128, false>), grid, dim3(kPruneThreads), 0, a.stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_fill_pruned(const FillArgs& a) {
  const int64_t total = (int64_t)a.B * a.Hh * a.N * (a.row_bytes / 16);
  hipLaunchKernelGGL(fill_pruned_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, a.stream, a);
  return hipGetLastError();
}

}  // namespace dbs
