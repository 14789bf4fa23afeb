// Per-row mask selection shared by the mask kernels and the fused
// estimate-and-mask kernels: exact 192-bit sums, the selection rules, the
// register (one wavefront per row) and LDS (one workgroup per row) sorts.
// Included by one translation unit each; everything here is inline.
#pragma once
#include "common.h"

namespace dbs {
namespace maskcore {

constexpr int kMaxNb = 4096;
constexpr int kLimbs = 6;

struct U192 {
  uint32_t w[kLimbs];
};

__device__ __forceinline__ U192 u192_zero() {
  U192 r;
#pragma unroll
  for (int i = 0; i < kLimbs; ++i) r.w[i] = 0;
  return r;
}

__device__ __forceinline__ U192 u192_add(const U192& a, const U192& b) {
  U192 r;
  uint64_t c = 0;
#pragma unroll
  for (int i = 0; i < kLimbs; ++i) {
    const uint64_t s = (uint64_t)a.w[i] + b.w[i] + c;
    r.w[i] = (uint32_t)s;
    c = s >> 32;
  }
  return r;
}

__device__ __forceinline__ bool u192_ge(const U192& a, const U192& b) {
#pragma unroll
  for (int i = kLimbs - 1; i >= 0; --i) {
    if (a.w[i] != b.w[i]) return a.w[i] > b.w[i];
  }
  return true;
}

// Exact integer value (units of 2^-149) of a non-negative float32 <= 1.
__device__ __forceinline__ U192 f32_to_u192(uint32_t bits) {
  U192 r = u192_zero();
  const uint32_t e = bits >> 23, mant = bits & 0x7fffffu;
  uint64_t sig;
  int sh;
  if (e == 0) {
    sig = mant;
    sh = 0;
  } else {
    sig = mant | 0x800000u;
    sh = (int)e - 1;
  }
  const int limb = sh >> 5, off = sh & 31;
  const uint64_t v = sig << off;              // < 2^55
#pragma unroll
  for (int i = 0; i < kLimbs; ++i) {
    if (i == limb) r.w[i] = (uint32_t)v;
    if (i == limb + 1) r.w[i] = (uint32_t)(v >> 32);
  }
  return r;
}

__device__ __forceinline__ uint32_t shfl_xor_u32(uint32_t v, int mask) {
  const int lane = threadIdx.x & 63;
  return (uint32_t)__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, (int)v);
}

__device__ __forceinline__ uint32_t shfl_from_u32(uint32_t v, int src) {
  return (uint32_t)__builtin_amdgcn_ds_bpermute(src << 2, (int)v);
}

__device__ __forceinline__ U192 wave_sum(U192 x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    U192 o;
#pragma unroll
    for (int i = 0; i < kLimbs; ++i) o.w[i] = shfl_xor_u32(x.w[i], m);
    x = u192_add(x, o);
  }
  return x;
}

__device__ __forceinline__ U192 wave_inclusive_scan(U192 x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int src = lane >= d ? lane - d : lane;
    U192 o;
#pragma unroll
    for (int i = 0; i < kLimbs; ++i) o.w[i] = shfl_from_u32(x.w[i], src);
    if (lane >= d) x = u192_add(x, o);
  }
  return x;
}

// The selection rule (launch.h MaskRule): the cumulative threshold tau, the
// top-k budget, or the statistical cutoff p = mean + std * u over the row's
// scores (BSA notes, design 2, read as a per-block cutoff; at least the
// largest block is kept).  The statistics are float64 sums in a fixed order.
struct Rule {
  int kind;          // 0 cumulative, 1 top-k, 2 statistical
  uint32_t tau_bits;
  int topk;
  double u;
};

inline Rule make_rule(int kind, float tau, int topk, double u) {
  Rule r;
  r.kind = kind;
  __builtin_memcpy(&r.tau_bits, &tau, 4);
  r.topk = topk;
  r.u = u;
  return r;
}

__device__ __forceinline__ double xor_shfl_d(double v, int m) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const int lane = threadIdx.x & 63;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute((lane ^ m) << 2, (int)(uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute((lane ^ m) << 2, (int)(uint32_t)(b >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum over the 64 lanes, the same butterfly order in every lane.
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += xor_shfl_d(v, m);
  return v;
}

// kCap: largest nb of the size class (LDS is sized for it, so small rows keep
// many workgroups resident); kThreads: workgroup size.
// load(j) returns the float32 bits of the row's entry j < nb.  Every thread
// of the workgroup calls this once per row.
template <int kCap, int kThreads, class Load>
__device__ __forceinline__ void mask_row_lds(Load load, int64_t row, int nb, Rule rule, int32_t* __restrict__ kv_count,
                                             int32_t* __restrict__ kv_idx, uint8_t* __restrict__ mask) {
  const uint32_t tau_bits = rule.tau_bits;
  __shared__ uint64_t keys[kCap];
  __shared__ uint8_t flag[kCap];
  __shared__ uint32_t red[kThreads / 64][kLimbs];
  __shared__ double dred[kThreads / 64];
  __shared__ int s_invalid, s_m;
  __shared__ int s_wave_cnt[kThreads / 64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int P2 = 1;
  while (P2 < nb) P2 <<= 1;

  if (tid == 0) s_invalid = 0;
  __syncthreads();
  bool bad = false;
  for (int j = tid; j < P2; j += kThreads) {
    uint64_t key = ~0ull;
    if (j < nb) {
      uint32_t bits = load(j);
      if ((bits & 0x7fffffffu) == 0) bits = 0;          // -0 is 0
      if (bits > 0x3f800000u) bad = true;               // negative, > 1, inf, NaN
      key = ((uint64_t)(~bits) << 32) | (uint32_t)j;
    }
    keys[j] = key;
  }
  if (bad) s_invalid = 1;
  __syncthreads();
  const bool keep_all = s_invalid != 0 || (rule.kind == 0 && tau_bits >= 0x3f800000u) ||
                        (rule.kind == 1 && rule.topk >= nb);

  int m = nb;
  if (!keep_all) {
    // ---- bitonic sort, ascending keys ----------------------------------------
    for (int k = 2; k <= P2; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < (P2 >> 1); i += kThreads) {
          const int lo = ((i & ~(j - 1)) << 1) | (i & (j - 1)), hi = lo + j;   // j is a power of two
          const uint64_t a = keys[lo], b = keys[hi];
          const bool asc = (lo & k) == 0;
          if ((a > b) == asc) {
            keys[lo] = b;
            keys[hi] = a;
          }
        }
        __syncthreads();
      }
    }
  }
  if (!keep_all && rule.kind == 1) {
    m = rule.topk;
  } else if (!keep_all && rule.kind == 2) {
    // ---- statistical cutoff: mean, then the population deviation, float64 --------
    auto block_sum = [&](double v) {
      v = wave_sum_d(v);
      if (lane == 0) dred[wave] = v;
      __syncthreads();
      double t = 0.0;
      for (int w = 0; w < kThreads / 64; ++w) t += dred[w];
      __syncthreads();
      return t;
    };
    double s1 = 0.0;
    for (int j = tid; j < nb; j += kThreads) s1 += (double)__uint_as_float(~(uint32_t)(keys[j] >> 32));
    const double mean = block_sum(s1) / nb;
    double s2 = 0.0;
    for (int j = tid; j < nb; j += kThreads) {
      const double dv = (double)__uint_as_float(~(uint32_t)(keys[j] >> 32)) - mean;
      s2 += dv * dv;
    }
    const double p = mean + sqrt(block_sum(s2) / nb) * rule.u;
    double c = 0.0;
    for (int j = tid; j < nb; j += kThreads) c += (double)__uint_as_float(~(uint32_t)(keys[j] >> 32)) >= p ? 1.0 : 0.0;
    m = max(1, (int)block_sum(c));
  } else if (!keep_all) {
    // ---- exact row total ---------------------------------------------------------
    U192 part = u192_zero();
    for (int j = tid; j < nb; j += kThreads) part = u192_add(part, f32_to_u192(~(uint32_t)(keys[j] >> 32)));
    part = wave_sum(part);
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < kLimbs; ++i) red[wave][i] = part.w[i];
    }
    __syncthreads();
    if (wave == 0) {
      U192 total = u192_zero();
      for (int w = 0; w < kThreads / 64; ++w) {
        U192 t;
#pragma unroll
        for (int i = 0; i < kLimbs; ++i) t.w[i] = red[w][i];
        total = u192_add(total, t);
      }
      // target = ceil(tau * total), tau = tm * 2^-sh exactly
      const uint32_t te = tau_bits >> 23;
      const uint64_t tm = te ? ((tau_bits & 0x7fffffu) | 0x800000u) : (tau_bits & 0x7fffffu);
      const int sh = te ? 150 - (int)te : 149;
      uint32_t prod[kLimbs + 1];
      uint64_t c = 0;
#pragma unroll
      for (int i = 0; i < kLimbs; ++i) {
        const uint64_t s = (uint64_t)total.w[i] * tm + c;
        prod[i] = (uint32_t)s;
        c = s >> 32;
      }
      prod[kLimbs] = (uint32_t)c;
      // shift right by sh with a sticky bit for the ceiling
      U192 tgt = u192_zero();
      bool sticky = false;
      const int ls = sh >> 5, bs = sh & 31;
      for (int i = 0; i < kLimbs + 1; ++i) {
        const int src = i + ls;
        uint32_t v = 0;
        if (src <= kLimbs) {
          v = prod[src] >> bs;
          if (bs && src + 1 <= kLimbs) v |= prod[src + 1] << (32 - bs);
        }
        if (i < kLimbs) tgt.w[i] = v;
      }
      for (int i = 0; i < ls && i <= kLimbs; ++i) sticky |= prod[i] != 0;
      if (ls <= kLimbs && bs) sticky |= (prod[ls] & ((1u << bs) - 1u)) != 0;
      if (sticky) {
        U192 one = u192_zero();
        one.w[0] = 1;
        tgt = u192_add(tgt, one);
      }
      // ---- minimal prefix over the sorted values -----------------------------------
      U192 run = u192_zero();
      int found = nb;
      for (int base = 0; base < nb; base += 64) {
        const int j = base + lane;
        const U192 x = j < nb ? f32_to_u192(~(uint32_t)(keys[j] >> 32)) : u192_zero();
        const U192 inc = wave_inclusive_scan(x, lane);
        const U192 pref = u192_add(run, inc);
        const bool hit = j < nb && u192_ge(pref, tgt);
        const uint64_t ball = __ballot(hit);
        if (ball) {
          found = base + __ffsll((unsigned long long)ball);   // first hit index + 1
          break;
        }
        U192 last;
#pragma unroll
        for (int i = 0; i < kLimbs; ++i) last.w[i] = shfl_from_u32(inc.w[i], 63);
        run = u192_add(run, last);
      }
      if (lane == 0) s_m = found;
    }
    __syncthreads();
    m = s_m;
  }

  // ---- kept flags, then ascending compaction --------------------------------------------
  for (int j = tid; j < nb; j += kThreads) flag[j] = keep_all ? 1 : 0;
  __syncthreads();
  if (!keep_all) {
    for (int i = tid; i < m; i += kThreads) flag[(uint32_t)keys[i]] = 1;
    __syncthreads();
  }
  const int per = (nb + kThreads - 1) / kThreads;
  const int j0 = tid * per, j1 = min(nb, j0 + per);
  int cnt = 0;
  for (int j = j0; j < j1; ++j) cnt += flag[j];
  // exclusive scan of cnt over the workgroup
  int inc = cnt;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int src = lane >= d ? lane - d : lane;
    const int o = __builtin_amdgcn_ds_bpermute(src << 2, inc);
    if (lane >= d) inc += o;
  }
  if (lane == 63) s_wave_cnt[wave] = inc;
  __syncthreads();
  int pos = inc - cnt;
  for (int w = 0; w < wave; ++w) pos += s_wave_cnt[w];
  int32_t* irow = kv_idx + row * nb;
  for (int j = j0; j < j1; ++j) {
    if (flag[j]) irow[pos++] = j;
  }
  if (mask != nullptr) {
    uint8_t* mrow = mask + row * nb;
    for (int j = tid; j < nb; j += kThreads) mrow[j] = flag[j];
  }
  if (tid == 0) kv_count[row] = m;
}

// Rows of up to 256 blocks: one wavefront per row, four rows per workgroup,
// no workgroup barrier.  Lane l holds the KPL = P2 / 64 keys of elements
// l * KPL .. l * KPL + KPL - 1 in registers; the bitonic network compares
// element e with e ^ j: for j < KPL inside the lane, otherwise with lane
// l ^ (j / KPL) through a cross-lane exchange (ds_swizzle xor below 32,
// v_permlane32_swap at 32).  The exact sums are the same 192-bit integers as
// in build_mask_kernel, so the result is identical.
__device__ __forceinline__ uint32_t lane_xor(uint32_t v, int d) {
  switch (d) {   // ds_swizzle bit mode: and_mask 0x1f, xor_mask d (within 32 lanes)
    case 1: return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x041f);
    case 2: return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x081f);
    case 4: return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x101f);
    case 8: return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x201f);
    case 16: return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401f);
    default: {
      const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
      return (threadIdx.x & 32) ? r[0] : r[1];
    }
  }
}

// One wavefront, one row: lane l brings the float32 bits of entries
// l * KPL + r (r < KPL; entries >= nb are ignored); flag is the wavefront's
// own 64 * KPL bytes of LDS.
template <int KPL>
__device__ __forceinline__ void mask_row_wave(const uint32_t (&in)[KPL], int64_t row, int nb, Rule rule,
                                              uint8_t* flag, int32_t* __restrict__ kv_count,
                                              int32_t* __restrict__ kv_idx, uint8_t* __restrict__ mask) {
  const uint32_t tau_bits = rule.tau_bits;
  constexpr int P2 = 64 * KPL;
  const int lane = threadIdx.x & 63;

  uint64_t key[KPL];
  bool bad = false;
#pragma unroll
  for (int r = 0; r < KPL; ++r) {
    const int e = lane * KPL + r;
    key[r] = ~0ull;
    if (e < nb) {
      uint32_t bits = in[r];
      if ((bits & 0x7fffffffu) == 0) bits = 0;          // -0 is 0
      if (bits > 0x3f800000u) bad = true;               // negative, > 1, inf, NaN
      key[r] = ((uint64_t)(~bits) << 32) | (uint32_t)e;
    }
  }
  const bool keep_all = __ballot(bad) != 0 || (rule.kind == 0 && tau_bits >= 0x3f800000u) ||
                        (rule.kind == 1 && rule.topk >= nb);

  int m = nb;
  if (!keep_all) {
    // ---- bitonic sort, ascending keys ------------------------------------------
#pragma unroll
    for (int k = 2; k <= P2; k <<= 1) {
#pragma unroll
      for (int j = k >> 1; j > 0; j >>= 1) {
        if (j >= KPL) {
          const int d = j / KPL;
#pragma unroll
          for (int r = 0; r < KPL; ++r) {
            const int e = lane * KPL + r;
            const uint64_t o = ((uint64_t)lane_xor((uint32_t)(key[r] >> 32), d) << 32) |
                               lane_xor((uint32_t)key[r], d);
            const bool keep_min = ((e & j) == 0) == ((e & k) == 0);
            key[r] = keep_min ? (o < key[r] ? o : key[r]) : (o > key[r] ? o : key[r]);
          }
        } else {
#pragma unroll
          for (int r = 0; r < KPL; ++r) {
            if (r & j) continue;
            const int e = lane * KPL + r;
            const uint64_t a = key[r], b = key[r | j];
            const bool asc = (e & k) == 0;
            if ((a > b) == asc) {
              key[r] = b;
              key[r | j] = a;
            }
          }
        }
      }
    }
  }
  if (!keep_all && rule.kind == 1) {
    m = rule.topk;
  } else if (!keep_all && rule.kind == 2) {
    // ---- statistical cutoff: mean, then the population deviation, float64 ----------
    double s1 = 0.0;
#pragma unroll
    for (int r = 0; r < KPL; ++r)
      if (lane * KPL + r < nb) s1 += (double)__uint_as_float(~(uint32_t)(key[r] >> 32));
    const double mean = wave_sum_d(s1) / nb;
    double s2 = 0.0;
#pragma unroll
    for (int r = 0; r < KPL; ++r) {
      if (lane * KPL + r < nb) {
        const double dv = (double)__uint_as_float(~(uint32_t)(key[r] >> 32)) - mean;
        s2 += dv * dv;
      }
    }
    const double p = mean + sqrt(wave_sum_d(s2) / nb) * rule.u;
    int c = 0;
#pragma unroll
    for (int r = 0; r < KPL; ++r)
      c += (lane * KPL + r < nb && (double)__uint_as_float(~(uint32_t)(key[r] >> 32)) >= p) ? 1 : 0;
    m = max(1, (int)wave_sum_d((double)c));
  } else if (!keep_all) {
    // ---- exact row total and target ceil(tau * total) ----------------------------
    U192 val[KPL];
    U192 lsum = u192_zero();
#pragma unroll
    for (int r = 0; r < KPL; ++r) {
      val[r] = lane * KPL + r < nb ? f32_to_u192(~(uint32_t)(key[r] >> 32)) : u192_zero();
      lsum = u192_add(lsum, val[r]);
    }
    const U192 total = wave_sum(lsum);
    const uint32_t te = tau_bits >> 23;
    const uint64_t tm = te ? ((tau_bits & 0x7fffffu) | 0x800000u) : (tau_bits & 0x7fffffu);
    const int sh = te ? 150 - (int)te : 149;
    uint32_t prod[kLimbs + 1];
    uint64_t c = 0;
#pragma unroll
    for (int i = 0; i < kLimbs; ++i) {
      const uint64_t t = (uint64_t)total.w[i] * tm + c;
      prod[i] = (uint32_t)t;
      c = t >> 32;
    }
    prod[kLimbs] = (uint32_t)c;
    U192 tgt = u192_zero();
    bool sticky = false;
    const int ls = sh >> 5, bs = sh & 31;
    for (int i = 0; i < kLimbs; ++i) {
      const int src = i + ls;
      uint32_t v = 0;
      if (src <= kLimbs) {
        v = prod[src] >> bs;
        if (bs && src + 1 <= kLimbs) v |= prod[src + 1] << (32 - bs);
      }
      tgt.w[i] = v;
    }
    for (int i = 0; i < ls && i <= kLimbs; ++i) sticky |= prod[i] != 0;
    if (ls <= kLimbs && bs) sticky |= (prod[ls] & ((1u << bs) - 1u)) != 0;
    if (sticky) {
      U192 one = u192_zero();
      one.w[0] = 1;
      tgt = u192_add(tgt, one);
    }
    // ---- minimal prefix over the sorted values ------------------------------------
    // prefix of element e = (sums of lanes below) + (the lane's values up to e)
    const U192 incl = wave_inclusive_scan(lsum, lane);
    U192 run;
#pragma unroll
    for (int i = 0; i < kLimbs; ++i) run.w[i] = shfl_from_u32(incl.w[i], lane > 0 ? lane - 1 : 0);
    if (lane == 0) run = u192_zero();
    int first = KPL;   // first element of this lane whose prefix reaches the target
#pragma unroll
    for (int r = 0; r < KPL; ++r) {
      run = u192_add(run, val[r]);
      if (first == KPL && lane * KPL + r < nb && u192_ge(run, tgt)) first = r;
    }
    const uint64_t ball = __ballot(first < KPL);
    const int fl = ball ? __ffsll((unsigned long long)ball) - 1 : 63;
    const int fr = __shfl(first, fl, 64);
    m = ball ? fl * KPL + fr + 1 : nb;
  }

  // ---- kept flags, then ascending compaction ----------------------------------------
#pragma unroll
  for (int r = 0; r < KPL; ++r) flag[lane * KPL + r] = 0;
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int r = 0; r < KPL; ++r) {
    const int e = lane * KPL + r;
    if (e < m) flag[keep_all ? e : (uint32_t)key[r]] = 1;
  }
  __builtin_amdgcn_wave_barrier();
  int cnt = 0;
  uint8_t f[KPL];
#pragma unroll
  for (int r = 0; r < KPL; ++r) {
    f[r] = lane * KPL + r < nb ? flag[lane * KPL + r] : 0;
    cnt += f[r];
  }
  int inc = cnt;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int src = lane >= d ? lane - d : lane;
    const int o = __builtin_amdgcn_ds_bpermute(src << 2, inc);
    if (lane >= d) inc += o;
  }
  int pos = inc - cnt;
  int32_t* irow = kv_idx + row * nb;
#pragma unroll
  for (int r = 0; r < KPL; ++r) {
    if (f[r]) irow[pos++] = lane * KPL + r;
  }
  if (mask != nullptr) {
    uint8_t* mrow = mask + row * nb;
#pragma unroll
    for (int r = 0; r < KPL; ++r)
      if (lane * KPL + r < nb) mrow[lane * KPL + r] = f[r];
  }
  if (lane == 0) kv_count[row] = m;
}

}  // namespace maskcore
}  // namespace dbs
