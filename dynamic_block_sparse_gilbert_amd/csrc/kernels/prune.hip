// BSA query pruning and token filling (gfx950).
//
// The BSA notes, key design 1: inside each query block, tokens nearly
// parallel to their window's centre token are left out of the attention and
// later take the centre's output.  A block of n valid tokens holding c centres
// keeps m = min(n, max(ceil(r * n), c)) rows: its centres (their outputs are
// needed for the filling) and the m - c other tokens of largest
// 1 - cos(q_centre, q_i), ties by smaller row.
//
// query_prune_kernel: one workgroup of 128 threads per (batch, head, block),
// one token per thread.  Each thread forms its token's dot product with its
// centre and both squared norms in float32 from the bf16 rows (read in token
// order through the permutation), then its rank among the block's
// non-centre tokens by counting, over the block's values in LDS, those that
// order before it.  A workgroup scan of the kept flags writes the kept rows in
// ascending order.
// fill_pruned_kernel: after the attention over the kept rows, every pruned
// row copies its centre's output row (and log-sum-exp), 16 bytes per thread.
#include <cmath>

#include "common.h"
#include "../launch.h"

namespace dbs {
namespace {

constexpr int kPruneThreads = 128;   // >= b

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__global__ __launch_bounds__(kPruneThreads) void query_prune_kernel(PruneArgs a) {
  __shared__ float dis_s[kPruneThreads];
  __shared__ int cls_s[kPruneThreads];      // 0 invalid row, 1 centre, 2 other token
  __shared__ int wave_cnt[kPruneThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int I = blockIdx.x, bh = blockIdx.y;
  const int bi = bh / a.Hh, hh = bh % a.Hh;
  const int R = I * a.b + tid;
  const bool valid = tid < a.b && R < a.N;
  const int32_t* perm = a.perm + (int64_t)hh * a.perm_h_stride;
  const int32_t* anc = a.anchor + (int64_t)hh * a.perm_h_stride;

  float dis = 0.f;
  int cls = 0;
  if (valid) {
    int A = anc[R];
    A = A < 0 ? 0 : (A >= a.N ? a.N - 1 : A);
    cls = A == R ? 1 : 2;
    if (cls == 2) {
      auto tok = [&](int row) {
        const int t = perm[row];
        return t < 0 ? 0 : (t >= a.N ? a.N - 1 : t);
      };
      const int64_t oq = bi * a.qsb + (int64_t)tok(R) * a.qsn + hh * a.qsh;
      const int64_t oa = bi * a.qsb + (int64_t)tok(A) * a.qsn + hh * a.qsh;
      float dot = 0.f, nq = 0.f, na = 0.f;
      if (a.q_f32) {
        const float4* qp = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.q) + oq);
        const float4* ap = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.q) + oa);
        for (int c = 0; c < a.d / 4; ++c) {
          const float4 x = qp[c], y = ap[c];
          // the float32 input rounded to bf16, as the attention reads it
          const float xs[4] = {bf16_bits_to_f32(f32_to_bf16_bits(x.x)), bf16_bits_to_f32(f32_to_bf16_bits(x.y)),
                               bf16_bits_to_f32(f32_to_bf16_bits(x.z)), bf16_bits_to_f32(f32_to_bf16_bits(x.w))};
          const float ys[4] = {bf16_bits_to_f32(f32_to_bf16_bits(y.x)), bf16_bits_to_f32(f32_to_bf16_bits(y.y)),
                               bf16_bits_to_f32(f32_to_bf16_bits(y.z)), bf16_bits_to_f32(f32_to_bf16_bits(y.w))};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            dot = __builtin_fmaf(xs[e], ys[e], dot);
            nq = __builtin_fmaf(xs[e], xs[e], nq);
            na = __builtin_fmaf(ys[e], ys[e], na);
          }
        }
      } else {
        const uint4* qp = reinterpret_cast<const uint4*>(reinterpret_cast<const __bf16*>(a.q) + oq);
        const uint4* ap = reinterpret_cast<const uint4*>(reinterpret_cast<const __bf16*>(a.q) + oa);
        for (int c = 0; c < a.d / 8; ++c) {
          const uint4 x = qp[c], y = ap[c];
          const uint32_t xw[4] = {x.x, x.y, x.z, x.w}, yw[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x0 = bf16_lo(xw[e]), x1 = bf16_hi(xw[e]), y0 = bf16_lo(yw[e]), y1 = bf16_hi(yw[e]);
            dot = __builtin_fmaf(x0, y0, __builtin_fmaf(x1, y1, dot));
            nq = __builtin_fmaf(x0, x0, __builtin_fmaf(x1, x1, nq));
            na = __builtin_fmaf(y0, y0, __builtin_fmaf(y1, y1, na));
          }
        }
      }
      if (nq == 0.f || na == 0.f) {
        dis = nq == na ? 0.f : 1.f;
      } else {
        dis = 1.f - dot / (sqrtf(nq) * sqrtf(na));
      }
    }
  }
  dis_s[tid] = dis;
  cls_s[tid] = cls;
  const int n_valid = __syncthreads_count(valid);
  const int n_centre = __syncthreads_count(cls == 1);
  const int m = min(n_valid, max((int)ceil(a.r * (double)n_valid), n_centre));
  const int take = m - n_centre;
  bool keep = cls == 1;
  if (cls == 2) {
    int rank = 0;
    for (int j = 0; j < kPruneThreads; ++j) {
      const float dj = dis_s[j];
      rank += (cls_s[j] == 2 && (dj > dis || (dj == dis && j < tid))) ? 1 : 0;
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
  hipLaunchKernelGGL(query_prune_kernel, dim3((unsigned)a.nb, (unsigned)(a.B * a.Hh)), dim3(kPruneThreads), 0,
                     a.stream, a);
  return hipGetLastError();
}

hipError_t launch_fill_pruned(const FillArgs& a) {
  const int64_t total = (int64_t)a.B * a.Hh * a.N * (a.row_bytes / 16);
  hipLaunchKernelGGL(fill_pruned_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, a.stream, a);
  return hipGetLastError();
}

}  // namespace dbs
