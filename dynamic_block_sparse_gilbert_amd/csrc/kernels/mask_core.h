// Per-row mask selection shared by the mask kernels and the fused
// estimate-and-mask kernels: exact 192-bit sums, the selection rules, the
// register sort (rows of up to 256 blocks) and the radix selection (longer
// rows), both one wavefront per row.
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

// Rows of up to 256 blocks: one wavefront per row, four rows per workgroup,
// no workgroup barrier.  Lane l holds the KPL = P2 / 64 keys of elements
// l * KPL .. l * KPL + KPL - 1 in registers; the bitonic network compares
// element e with e ^ j: for j < KPL inside the lane, otherwise with lane
// l ^ (j / KPL) through a cross-lane exchange (ds_swizzle xor below 32,
// v_permlane32_swap at 32).  The row total, the target and the prefixes are
// exact 192-bit integers, so the result does not depend on the order of the
// additions.
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

// ---- radix selection: one wavefront per row, no sort ---------------------------------------
// The kept set of the cumulative rule is the top-m prefix of the order (value
// descending, index ascending), so it is fixed by its last element: the value
// v* of the m-th element and how many elements equal to v* (lowest indices
// first) it takes.  Both are found by a radix select on the value bits (for
// non-negative floats the bit pattern orders like the value) with exact
// weights: first over the exponent, then over three 8-bit digits of the
// significand of the elements in the crossing exponent.  Within one exponent
// every value's exact mass is its significand times the same power of two, so
// those sums are 64-bit integers; only the 128 exponent buckets need the
// 192-bit sums.  Top-k is the same search with weight 1 per element.  The
// result is the same set as the sort's, bit for bit.

// Significand of non-negative float32 bits (hidden bit included for normals):
// the exact value is sig * 2^(max(e, 1) - 150).
__device__ __forceinline__ uint32_t sig_of(uint32_t b) {
  const uint32_t e = b >> 23;
  return e ? ((b & 0x7fffffu) | 0x800000u) : (b & 0x7fffffu);
}

// x * 2^s as a 192-bit number (x < 2^64, s < 128).
__device__ __forceinline__ U192 u192_shl64(uint64_t x, int s) {
  U192 r = u192_zero();
  const int limb = s >> 5, off = s & 31;
  const uint64_t lo = x << off;
  const uint32_t top = off ? (uint32_t)(x >> (64 - off)) : 0u;
#pragma unroll
  for (int i = 0; i < kLimbs; ++i) {
    if (i == limb) r.w[i] = (uint32_t)lo;
    if (i == limb + 1) r.w[i] = (uint32_t)(lo >> 32);
    if (i == limb + 2) r.w[i] = top;
  }
  return r;
}

// a - b for a >= b.
__device__ __forceinline__ U192 u192_sub(const U192& a, const U192& b) {
  U192 r;
  uint32_t br = 0;
#pragma unroll
  for (int i = 0; i < kLimbs; ++i) {
    const uint64_t d = (uint64_t)a.w[i] - b.w[i] - br;
    r.w[i] = (uint32_t)d;
    br = (uint32_t)(d >> 63);
  }
  return r;
}

// ceil(a / 2^s) for a result below 2^64 (s < 160).
__device__ __forceinline__ uint64_t u192_shr_ceil64(const U192& a, int s) {
  const int limb = s >> 5, off = s & 31;
  uint32_t w0 = 0, w1 = 0, w2 = 0;
  bool rem = false;
#pragma unroll
  for (int i = 0; i < kLimbs; ++i) {
    if (i == limb) w0 = a.w[i];
    if (i == limb + 1) w1 = a.w[i];
    if (i == limb + 2) w2 = a.w[i];
    if (i < limb) rem |= a.w[i] != 0;
  }
  const uint64_t lo = ((uint64_t)w1 << 32) | w0;
  const uint64_t q = off ? ((lo >> off) | ((uint64_t)w2 << (64 - off))) : lo;
  if (off) rem |= (w0 & ((1u << off) - 1u)) != 0;
  return q + (rem ? 1u : 0u);
}

__device__ __forceinline__ bool u192_is_zero(const U192& a) {
  uint32_t o = 0;
#pragma unroll
  for (int i = 0; i < kLimbs; ++i) o |= a.w[i];
  return o == 0;
}

// ceil(tau * total) in units of 2^-149, tau = the float32 with bits tau_bits (in (0, 1)).
__device__ __forceinline__ U192 tau_target(const U192& total, uint32_t tau_bits) {
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
#pragma unroll
  for (int i = 0; i < kLimbs; ++i) {
    const int src = i + ls;
    uint32_t v = 0;
#pragma unroll
    for (int q = 0; q <= kLimbs; ++q) {
      if (q == src) v |= prod[q] >> bs;
      if (bs && q == src + 1) v |= prod[q] << (32 - bs);
    }
    tgt.w[i] = v;
  }
#pragma unroll
  for (int q = 0; q <= kLimbs; ++q) {
    if (q < ls) sticky |= prod[q] != 0;
    if (bs && q == ls) sticky |= (prod[q] & ((1u << bs) - 1u)) != 0;
  }
  if (sticky) {
    U192 one = u192_zero();
    one.w[0] = 1;
    tgt = u192_add(tgt, one);
  }
  return tgt;
}

__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  const uint32_t lo = shfl_from_u32((uint32_t)v, src), hi = shfl_from_u32((uint32_t)(v >> 32), src);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint64_t o = shfl_u64(x, lane >= d ? lane - d : lane);
    if (lane >= d) x += o;
  }
  return x;
}

// Narrows the selection to one value: among the candidates (cand[r]), the
// 8-bit digit (sig >> shift) & 255 whose cumulative weight, from the largest
// digit down, first reaches `need` (need >= 1 and reachable); `need` becomes
// what the elements at or below that digit must still supply.  hist: this
// wavefront's 256 LDS counters.
template <int KPL>
__device__ __forceinline__ uint32_t radix_digit(const uint32_t (&sg)[KPL], const bool (&cand)[KPL], int shift,
                                                bool by_mass, unsigned long long* hist, uint64_t& need) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 4; ++i) hist[lane + 64 * i] = 0ull;
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int r = 0; r < KPL; ++r)
    if (cand[r]) __hip_atomic_fetch_add(&hist[(sg[r] >> shift) & 255u], by_mass ? (unsigned long long)sg[r] : 1ull,
                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
  __builtin_amdgcn_wave_barrier();
  // lane l holds digits 255 - 4l .. 252 - 4l (descending)
  uint64_t h[4], lt = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    h[q] = __hip_atomic_load(&hist[255 - 4 * lane - q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
    lt += h[q];
  }
  const uint64_t incl = wave_incl_scan_u64(lt, lane);
  uint64_t cum = incl - lt;
  int hitq = 4;
  uint64_t above = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint64_t prev = cum;
    cum += h[q];
    if (hitq == 4 && cum >= need) {
      hitq = q;
      above = prev;
    }
  }
  const uint64_t ball = __ballot(hitq < 4);
  const int L = ball ? __ffsll((unsigned long long)ball) - 1 : 63;
  const int q = __shfl(hitq, L, 64);
  need -= shfl_u64(above, L);
  __builtin_amdgcn_wave_barrier();
  return (uint32_t)(255 - 4 * L - (q < 4 ? q : 3));
}

// LDS area of one wavefront in the radix kernels: first the row's 64 * KPL
// entries (float32 bits), written coalesced, then the selection's 512 64-bit
// counters.
template <int KPL>
struct RadixArea {
  static constexpr int kWords = KPL * 64 * 4 > 512 * 8 ? KPL * 32 : 512;   // 64-bit words
};

// in[r] = row entry lane * KPL + r from the wavefront's LDS area (16-byte
// reads), after the wavefront wrote every entry there.  The memory clobbers
// keep the reads after those writes and before the selection reuses the
// area; LDS operations of one wavefront complete in order.
template <int KPL>
__device__ __forceinline__ void gather_lane_entries(const float* pv, int lane, uint32_t (&in)[KPL]) {
  static_assert(KPL % 4 == 0, "16-byte reads");
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
#pragma unroll
  for (int r = 0; r < KPL; r += 4) {
    const uint4 q = *reinterpret_cast<const uint4*>(pv + lane * KPL + r);
    in[r] = q.x; in[r + 1] = q.y; in[r + 2] = q.z; in[r + 3] = q.w;
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

// One wavefront, one row: lane l brings the float32 bits of entries
// l * KPL + r (r < KPL; entries >= nb are ignored).  hist: this wavefront's 512
// 64-bit LDS counters.  Same result as mask_row_wave (and as a full sort) under the
// cumulative and top-k rules; the statistical rule sums its float64 statistics
// in this function's own fixed order.
template <int KPL>
__device__ __forceinline__ void mask_row_radix(const uint32_t (&in)[KPL], int64_t row, int nb, Rule rule,
                                               unsigned long long* hist, int32_t* __restrict__ kv_count,
                                               int32_t* __restrict__ kv_idx, uint8_t* __restrict__ mask) {
  const int lane = threadIdx.x & 63;
  uint32_t v[KPL];
  bool bad = false;
#pragma unroll
  for (int r = 0; r < KPL; ++r) {
    uint32_t b = 0;
    if (lane * KPL + r < nb) {
      b = in[r];
      if ((b & 0x7fffffffu) == 0) b = 0;      // -0 is 0
      if (b > 0x3f800000u) bad = true;        // negative, > 1, inf, NaN
    }
    v[r] = b;
  }
  const bool keep_all = __ballot(bad) != 0 || (rule.kind == 0 && rule.tau_bits >= 0x3f800000u) ||
                        (rule.kind == 1 && rule.topk >= nb);
  // kept: every valid element when keep_all; under the statistical cutoff with a
  // hit, the elements >= p; otherwise v > vstar, or v == vstar among the first
  // ceq such elements by index
  bool direct = false;
  double pcut = 0.0;
  uint32_t vstar = 0;
  uint64_t ceq = 0;
  if (!keep_all) {
    bool by_mass = rule.kind == 0;
    uint64_t need_count = rule.kind == 1 ? (uint64_t)rule.topk : 1ull;
    if (rule.kind == 2) {
      double s1 = 0.0;
#pragma unroll
      for (int r = 0; r < KPL; ++r)
        if (lane * KPL + r < nb) s1 += (double)__uint_as_float(v[r]);
      const double mean = wave_sum_d(s1) / nb;
      double s2 = 0.0;
#pragma unroll
      for (int r = 0; r < KPL; ++r) {
        if (lane * KPL + r < nb) {
          const double dv = (double)__uint_as_float(v[r]) - mean;
          s2 += dv * dv;
        }
      }
      pcut = mean + sqrt(wave_sum_d(s2) / nb) * rule.u;
      bool any = false;
#pragma unroll
      for (int r = 0; r < KPL; ++r) any |= lane * KPL + r < nb && (double)__uint_as_float(v[r]) >= pcut;
      direct = __ballot(any) != 0;
      by_mass = false;   // otherwise the largest element alone: top-1
    }
    if (!direct) {
      // ---- exponent buckets: four copies (lanes / 16) to spread the LDS atomics --------------
#pragma unroll
      for (int i = 0; i < 8; ++i) hist[lane + 64 * i] = 0ull;
      __builtin_amdgcn_wave_barrier();
      const int copy = (lane >> 4) * 128;
#pragma unroll
      for (int r = 0; r < KPL; ++r)
        if (lane * KPL + r < nb)
          __hip_atomic_fetch_add(&hist[copy + (v[r] >> 23)], by_mass ? (unsigned long long)sig_of(v[r]) : 1ull,
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
      __builtin_amdgcn_wave_barrier();
      // lane l: exponents 127 - 2l (first) and 126 - 2l
      const int eh = 127 - 2 * lane, el = 126 - 2 * lane;
      uint64_t hh = 0, hl = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        hh += __hip_atomic_load(&hist[c * 128 + eh], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
        hl += __hip_atomic_load(&hist[c * 128 + el], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
      }
      __builtin_amdgcn_wave_barrier();
      int estar;
      uint64_t need;
      if (by_mass) {
        const U192 mh = u192_shl64(hh, (eh > 1 ? eh : 1) - 1), ml = u192_shl64(hl, (el > 1 ? el : 1) - 1);
        const U192 pair = u192_add(mh, ml);
        const U192 incl = wave_inclusive_scan(pair, lane);
        const U192 excl = u192_sub(incl, pair);
        U192 total;
#pragma unroll
        for (int i = 0; i < kLimbs; ++i) total.w[i] = shfl_from_u32(incl.w[i], 63);
        const U192 tgt = tau_target(total, rule.tau_bits);
        if (u192_is_zero(tgt)) {
          // every value is 0: the first element alone (index 0)
          vstar = 0;
          ceq = 1;
          estar = -1;
          need = 0;
        } else {
          const U192 cum_h = u192_add(excl, mh);
          const bool hit_h = u192_ge(cum_h, tgt), hit_l = u192_ge(incl, tgt);
          const uint64_t ball = __ballot(hit_h || hit_l);
          const int L = __ffsll((unsigned long long)ball) - 1;   // a hit exists: the total reaches tgt
          const int which = __shfl(hit_h ? 0 : 1, L, 64);
          estar = 127 - 2 * L - which;
          U192 above;
#pragma unroll
          for (int i = 0; i < kLimbs; ++i) {
            const uint32_t a0 = shfl_from_u32(excl.w[i], L), a1 = shfl_from_u32(cum_h.w[i], L);
            above.w[i] = which ? a1 : a0;
          }
          need = u192_shr_ceil64(u192_sub(tgt, above), (estar > 1 ? estar : 1) - 1);
        }
      } else {
        const uint64_t pair = hh + hl;
        const uint64_t incl = wave_incl_scan_u64(pair, lane);
        const uint64_t cum_h = incl - pair + hh;
        const bool hit_h = cum_h >= need_count, hit_l = incl >= need_count;
        const uint64_t ball = __ballot(hit_h || hit_l);
        const int L = __ffsll((unsigned long long)ball) - 1;   // need_count <= valid elements
        const int which = __shfl(hit_h ? 0 : 1, L, 64);
        estar = 127 - 2 * L - which;
        need = need_count - shfl_u64(which ? cum_h : incl - pair, L);
      }
      if (estar >= 0) {
        // ---- significand digits of the elements in the crossing exponent ---------------------
        uint32_t sg[KPL];
        bool cand[KPL];
#pragma unroll
        for (int r = 0; r < KPL; ++r) {
          sg[r] = sig_of(v[r]);
          cand[r] = lane * KPL + r < nb && (int)(v[r] >> 23) == estar;
        }
        uint32_t pre = 0;
#pragma unroll
        for (int pass = 0; pass < 3; ++pass) {
          const int shift = 16 - 8 * pass;
          const uint32_t d = radix_digit<KPL>(sg, cand, shift, by_mass, hist, need);
          pre = (pre << 8) | d;
#pragma unroll
          for (int r = 0; r < KPL; ++r) cand[r] = cand[r] && ((sg[r] >> shift) & 255u) == d;
        }
        vstar = ((uint32_t)estar << 23) | (pre & 0x7fffffu);
        ceq = by_mass ? (need + pre - 1) / pre : need;
      }
    }
  }
  // ---- kept flags, then ascending compaction ----------------------------------------------
  // rank of the lane's first element equal to vstar among all such elements
  int neq = 0;
#pragma unroll
  for (int r = 0; r < KPL; ++r) neq += (lane * KPL + r < nb && v[r] == vstar) ? 1 : 0;
  int eq_incl = neq;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __builtin_amdgcn_ds_bpermute((lane >= d ? lane - d : lane) << 2, eq_incl);
    if (lane >= d) eq_incl += o;
  }
  uint64_t rank = (uint64_t)(eq_incl - neq);
  bool f[KPL];
  int cnt = 0;
#pragma unroll
  for (int r = 0; r < KPL; ++r) {
    const bool ok = lane * KPL + r < nb;
    bool k;
    if (keep_all) {
      k = ok;
    } else if (direct) {
      k = ok && (double)__uint_as_float(v[r]) >= pcut;
    } else {
      const bool eq = v[r] == vstar;
      k = ok && (v[r] > vstar || (eq && rank < ceq));
      if (ok && eq) ++rank;
    }
    f[r] = k;
    cnt += k ? 1 : 0;
  }
  int inc = cnt;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __builtin_amdgcn_ds_bpermute((lane >= d ? lane - d : lane) << 2, inc);
    if (lane >= d) inc += o;
  }
  int pos = inc - cnt;
  const int m = __shfl(inc, 63, 64);
  int32_t* irow = kv_idx + row * nb;
#pragma unroll
  for (int r = 0; r < KPL; ++r)
    if (f[r]) irow[pos++] = lane * KPL + r;
  if (mask != nullptr) {
    uint8_t* mrow = mask + row * nb;
#pragma unroll
    for (int r = 0; r < KPL; ++r)
      if (lane * KPL + r < nb) mrow[lane * KPL + r] = f[r] ? 1 : 0;
  }
  if (lane == 0) kv_count[row] = m;
}

}  // namespace maskcore
}  // namespace dbs
