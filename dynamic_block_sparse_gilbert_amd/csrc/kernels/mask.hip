// Cumulative-threshold block mask (gfx950).
//
// Video-BLADE "Step 2.1": sort each P_imp row descending and keep the fewest
// key blocks whose cumulative score reaches tau of the row's mass.
//
// Exactness: every float32 in [0, 1] is an integer multiple of 2^-149 below
// 2^150, so a row of up to 4096 values sums exactly in a 192-bit integer
// (six 32-bit limbs).  The row total, the target ceil(tau * total) and the
// running prefix are all exact; "prefix >= tau * total" is then decided
// without rounding and the result cannot depend on the summation order.
//
// Rows of up to 256 blocks take one wavefront each (four rows per workgroup,
// no workgroup barrier): the 64-bit keys (~value bits, block index), which
// order by value descending and index ascending, are sorted in registers by
// a bitonic network with cross-lane exchanges; one wavefront scan of the
// lanes' exact sums finds the first prefix that reaches the target.  Longer
// rows also take one wavefront each, with no sort: a radix selection over the
// value bits with exact weights finds the last kept value and how many of its
// ties are kept.  The kept blocks are written in ascending index order by a
// compaction.  Optionally a second launch turns the kept counts
// into the attention kernel's work order.
#include "common.h"
#include "../launch.h"

#include "mask_core.h"

namespace dbs {
namespace {

using namespace maskcore;

template <int KPL>
__global__ __launch_bounds__(256) void build_mask_wave_kernel(
    const float* __restrict__ p_imp, int nb, int rows, Rule rule, int32_t* __restrict__ kv_count,
    int32_t* __restrict__ kv_idx, uint8_t* __restrict__ mask) {
  __shared__ uint8_t flag_all[4][64 * KPL];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + w;
  if (row >= rows) return;
  const uint32_t* prow = reinterpret_cast<const uint32_t*>(p_imp) + row * nb;
  uint32_t in[KPL];
#pragma unroll
  for (int r = 0; r < KPL; ++r) in[r] = lane * KPL + r < nb ? prow[lane * KPL + r] : 0u;
  mask_row_wave<KPL>(in, row, nb, rule, flag_all[w], kv_count, kv_idx, mask);
}

// Rows of 257..4096 blocks: one wavefront per row (four per workgroup).  The
// row is read coalesced (16 bytes per lane at 256 g + 4 l when the rows are
// 16-byte aligned) into the wavefront's LDS area, lane l then takes entries
// l * KPL .. l * KPL + KPL - 1 from there, and the radix selection runs (no
// sort), reusing the area for its counters.
template <int KPL>
__global__ __launch_bounds__(256) void build_mask_radix_kernel(
    const float* __restrict__ p_imp, int nb, int rows, Rule rule, int32_t* __restrict__ kv_count,
    int32_t* __restrict__ kv_idx, uint8_t* __restrict__ mask) {
  __shared__ __attribute__((aligned(16))) unsigned long long area_all[4][RadixArea<KPL>::kWords];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + w;
  if (row >= rows) return;   // whole wavefronts; no workgroup barrier follows
  const float* prow = p_imp + row * nb;
  float* pv = reinterpret_cast<float*>(area_all[w]);
  if ((nb & 3) == 0 && (((uintptr_t)p_imp) & 15u) == 0) {
#pragma unroll
    for (int g = 0; g < KPL / 4; ++g) {
      const int J = 256 * g + 4 * lane;
      float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
      if (J < nb) q = *reinterpret_cast<const float4*>(prow + J);   // nb % 4 == 0: all four valid
      *reinterpret_cast<float4*>(pv + J) = q;
    }
  } else {
#pragma unroll
    for (int r = 0; r < KPL; ++r) {
      const int J = 64 * r + lane;
      pv[J] = J < nb ? prow[J] : 0.f;
    }
  }
  uint32_t in[KPL];
  gather_lane_entries<KPL>(pv, lane, in);
  mask_row_radix<KPL>(in, row, nb, rule, area_all[w], kv_count, kv_idx, mask);
}


// Work order for the attention kernel: rows (b, h, I) are split into the
// eight contiguous ranges that the attention launch assigns to the eight
// XCDs (see xcd_range in common.h), and each range is listed by kept count
// descending, so every XCD starts its longest query blocks first (a
// longest-processing-time-first schedule; kept counts are very uneven).
// One workgroup per range: a counting sort over the counts 0..nb in LDS.
// Rows with equal counts come out in an arbitrary order.
constexpr int kOrderThreads = 1024;

__global__ __launch_bounds__(kOrderThreads) void build_order_kernel(const int32_t* __restrict__ kv_count,
                                                                    int nb, int total,
                                                                    int32_t* __restrict__ order) {
  __shared__ int cursor[kMaxNb + 1];
  __shared__ int wsum[kOrderThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63;
  int start, size;
  xcd_range(blockIdx.x, total, start, size);
  const int nbins = nb + 1;                       // bin nb - c holds count c
  for (int i = tid; i < nbins; i += kOrderThreads) cursor[i] = 0;
  __syncthreads();
  for (int i = tid; i < size; i += kOrderThreads) {
    const int c = min(max(kv_count[start + i], 0), nb);
    atomicAdd(&cursor[nb - c], 1);
  }
  __syncthreads();
  // Exclusive prefix over the bins: thread t owns a contiguous chunk.
  const int chunk = (nbins + kOrderThreads - 1) / kOrderThreads;
  const int b0 = min(tid * chunk, nbins), b1 = min(b0 + chunk, nbins);
  int local = 0;
  for (int b = b0; b < b1; ++b) local += cursor[b];
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(incl, off, 64);
    if (lane >= off) incl += t;
  }
  if (lane == 63) wsum[tid >> 6] = incl;
  __syncthreads();
  int run = incl - local;
  for (int w = 0; w < (tid >> 6); ++w) run += wsum[w];
  for (int b = b0; b < b1; ++b) {
    const int h = cursor[b];
    cursor[b] = run;
    run += h;
  }
  __syncthreads();
  for (int i = tid; i < size; i += kOrderThreads) {
    const int c = min(max(kv_count[start + i], 0), nb);
    const int pos = atomicAdd(&cursor[nb - c], 1);
    order[start + pos] = start + i;
  }
}

}  // namespace

hipError_t launch_build_mask(const MaskArgs& a) {
  const Rule rule = make_rule(a.rule, a.tau, a.topk, a.u);
  const dim3 wgrid((unsigned)((a.rows + 3) / 4));
  if (a.nb <= 64) {
    hipLaunchKernelGGL((build_mask_wave_kernel<1>), wgrid, dim3(256), 0, a.stream, a.p_imp, a.nb, a.rows,
                       rule, a.kv_count, a.kv_idx, a.mask);
  } else if (a.nb <= 128) {
    hipLaunchKernelGGL((build_mask_wave_kernel<2>), wgrid, dim3(256), 0, a.stream, a.p_imp, a.nb, a.rows,
                       rule, a.kv_count, a.kv_idx, a.mask);
  } else if (a.nb <= 256) {
    hipLaunchKernelGGL((build_mask_wave_kernel<4>), wgrid, dim3(256), 0, a.stream, a.p_imp, a.nb, a.rows,
                       rule, a.kv_count, a.kv_idx, a.mask);
  } else if (a.nb <= 512) {
    hipLaunchKernelGGL((build_mask_radix_kernel<8>), wgrid, dim3(256), 0, a.stream, a.p_imp, a.nb, a.rows, rule,
                       a.kv_count, a.kv_idx, a.mask);
  } else if (a.nb <= 1024) {
    hipLaunchKernelGGL((build_mask_radix_kernel<16>), wgrid, dim3(256), 0, a.stream, a.p_imp, a.nb, a.rows, rule,
                       a.kv_count, a.kv_idx, a.mask);
  } else if (a.nb <= 1280) {
    hipLaunchKernelGGL((build_mask_radix_kernel<20>), wgrid, dim3(256), 0, a.stream, a.p_imp, a.nb, a.rows, rule,
                       a.kv_count, a.kv_idx, a.mask);
  } else if (a.nb <= 2048) {
    hipLaunchKernelGGL((build_mask_radix_kernel<32>), wgrid, dim3(256), 0, a.stream, a.p_imp, a.nb, a.rows, rule,
                       a.kv_count, a.kv_idx, a.mask);
  } else {
    hipLaunchKernelGGL((build_mask_radix_kernel<64>), wgrid, dim3(256), 0, a.stream, a.p_imp, a.nb, a.rows, rule,
                       a.kv_count, a.kv_idx, a.mask);
  }
  if (a.order != nullptr) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_build_order(a);
  }
  return hipGetLastError();
}

hipError_t launch_build_order(const MaskArgs& a) {
  hipLaunchKernelGGL(build_order_kernel, dim3(kXcdRanges), dim3(kOrderThreads), 0, a.stream, a.kv_count,
                     a.nb, a.rows, a.order);
  return hipGetLastError();
}

}  // namespace dbs
