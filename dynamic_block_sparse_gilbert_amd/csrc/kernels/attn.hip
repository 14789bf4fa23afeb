// Block-sparse flash attention forward over compacted KV-block lists (gfx950).
//
// Video-BLADE "Step 2.2": the binary block mask restricts attention; every
// query block walks only its kept KV blocks (the count/index-list form the
// BSA notes call q2k_num / q2k_index).  ASA_G appends the mean-pooled global
// tokens with a +ln(r) logit bias (BLADE notes, key design 2).
//
// Decomposition: one workgroup per (batch, head, query block of BLK rows);
// each wavefront owns 32 query rows (one MFMA tile).  Keys are consumed in
// stages of 64 (a kept block of 128 is two stages; global-token tiles
// likewise).
//   S^T = K Q^T      bf16 MFMA 32x32x16, Q^T resident in VGPRs.  The
//                    accumulator layout gives each lane the scores of single
//                    queries, so softmax statistics stay in the lane (one
//                    exchange between the two wave halves per stage).
//   P^T = exp2(S^T * scale*log2e - m)   fp32 (row sums in fp32), packed to
//                    bf16 by v_cvt_pk.
//   O^T += V^T P^T   bf16 MFMA 32x32x16; P^T comes straight from the score
//                    accumulators.  Inside each 16-key step the MFMA k index
//                    maps to keys {4g..4g+3, 8+4g..8+4g+3} (g = wave half) for
//                    both operands; V tiles store every 16 keys in the order
//                    0-3, 8-11, 4-7, 12-15, so a lane's 8 keys of one channel
//                    are one contiguous 16-byte LDS read.
//
// Software pipeline per stage u (two phases, a barrier before each):
//   phase A: score MFMAs of stage u+1   ||  exp / pack / row-sum of stage u
//   phase B: PV MFMAs of stage u        ||  row maximum of stage u+1
//   then, for partial stages and the last global-token tile only, the key mask
//   and bias and a fresh maximum (the other global-token tiles add ln n to the
//   maximum and the exponent offset instead), and the (rarely taken) lazy
//   rescale decided from stage u+1's maximum.  Two wavefronts per SIMD from different workgroups fill
//   each other's gaps; forcing an instruction interleave measured slower.
// K and V stages are copied global -> LDS by the buffer form of the DMA path
// (buffer_load_dwordx4 ... lds, no VGPR staging) into double buffers during
// the iteration before their use.  At d = 128, K of stage u+2 goes out among
// phase A's MFMAs and V of stage u+1 among phase B's.  Copies retire in order,
// so each phase waits only for what it reads: iteration u opens with a wait
// that leaves the previous phase B's V copies in flight (K of stage u+1 done)
// and a barrier, and phase B opens with a wait that leaves this phase A's K
// copies in flight (V of stage u done) and a second barrier.  Every copy thus
// gets about one iteration to land; a single full wait per iteration gave the
// last copies of phase B only a few MFMAs.  At d = 64 (VALU-bound) both copies
// go out after phase A's first MFMAs behind one full wait per iteration, which
// saves the second barrier.  The buffer form counts on vmcnt only, so the LDS
// operand reads keep partial lgkmcnt waits (the flat form of the same copy
// forces a full LDS drain after each issue).  One sched_group_barrier order
// per phase keeps every LDS operand read two MFMAs ahead of its use.  The kept-block list of
// the query block is staged in LDS once, so the stage descriptors read it
// there rather than with scalar loads; each stage descriptor is computed
// once, one iteration ahead of its score MFMAs.  LDS rows are padded by one 16-byte
// unit, so the 8 lanes that share a bank window read 8 different 16-byte bank
// groups and every read address is one per-lane base register plus an
// immediate.
// Online softmax with a lazy rescale: the running maximum is raised (and O, l
// rescaled) only when a stage's maximum exceeds it by more than 8 (log2
// units), so probabilities stay below 2^8 and most stages skip the rescale.
#include "common.h"
#include "../launch.h"

#include <type_traits>

namespace dbs {
namespace {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

template <int D, int BLK, int QB = BLK>
struct AttnCfg {
  static constexpr int kQW = 32;                 // query rows per wavefront
  static constexpr int kWaves = QB / kQW;        // query rows per workgroup / 32: 4 for QB = 128, 2 for 64
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kKT = 64;                 // keys per stage
  static constexpr int kSubs = BLK / kKT;        // stages per block
  // K stage in LDS: 64 key rows of D bf16, each padded by one 16-byte unit.
  static constexpr int kKRowU = D / 8 + 1;
  static constexpr int kKStride = kKRowU * 16;   // bytes per padded K row
  static constexpr int kKBytes = kKT * kKStride;
  static constexpr int kKInstr = kKBytes / 1024; // DMA instructions (1 KiB each) per K stage
  // V^T stage in LDS: D channel rows of 64 keys, each padded by one unit.
  static constexpr int kVRowU = kKT / 8 + 1;
  static constexpr int kVStride = kVRowU * 16;
  static constexpr int kVBytes = D * kVStride;
  static constexpr int kVInstr = kVBytes / 1024;
  static constexpr int kKPer = (kKInstr + kWaves - 1) / kWaves;   // per wave
  static constexpr int kVPer = (kVInstr + kWaves - 1) / kWaves;
  static_assert(kKBytes % 1024 == 0 && kVBytes % 1024 == 0, "stage must be whole DMA instructions");
};

constexpr float kLazyThreshold = 8.0f;

// Kept-block list words in LDS: bits 0-11 block index, bit 12 + h the stage
// (half block) h is partial or invalid, bit 14 the entry is invalid.
constexpr int kIndexMask = 0xFFF;
constexpr int kPartial = 0x1000;
constexpr int kInvalidBit = 0x4000;

// sched_group_barrier instruction classes
constexpr int kSgMfma = 0x008;
constexpr int kSgVmem = 0x020;   // vector-memory reads (the global -> LDS copies)
constexpr int kSgDsRead = 0x100;

__device__ __forceinline__ uint32_t cvt_pk(float a, float b) {
  bf16x2_t p;
  p[0] = (__bf16)a;
  p[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ float max_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Raw buffer descriptor over `bytes` bytes at `base` (gfx9 word 3: 32-bit data
// format, raw addressing).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// 16 bytes per lane from buffer offset soff + voff into LDS at lds + 16 * lane.
__device__ __forceinline__ void copy16_lds(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, voff, soff, 0, 0);
}

struct StageDesc {
  uint32_t koffs;      // byte offset of the stage's first K row in its head
  uint32_t voffs;      // byte offset of the stage's V^T columns in its head
  bool glob;           // global-token tile (K_g / V_g) rather than a kept block
  int key0;            // index of the stage's first key (token, or global token)
  int kind;            // 0 full, 1 partial / invalid (mask by key index), 2 global tokens (the
                       // last tile: per-key bias and mask), 3 global tokens that all carry the
                       // ln n bias (no mask; the bias enters the exponent offset)
  int limit;           // keys with index >= limit are masked (kind 1, 2)
  bool absent;         // mode 2: a block this wavefront's query block does not keep (contributes nothing)
};

// QB: query rows per workgroup.  MODE (BSA query pruning, rowsel lists the
// kept rows of each block, q_count[block] of them):
//   0  every row of the query block;
//   1  the kept rows of one block (rows sub * QB .. of its list);
//   2  a pair of blocks (2P, 2P + 1) whose kept rows fit half a workgroup
//      each: the first half of the wavefronts takes block 2P's rows, the
//      second half block 2P + 1's, over the union of their kept-block lists,
//      a wavefront masking the stages its block does not keep.  Mode 1 skips
//      the blocks mode 2 takes, and mode 2 exits for the others.  With a
//      work order, mode 2 walks the rows in that order and runs each pair
//      at its first block's place (the longest pairs start first).
//
// GLOB: the launch has ASA_G global tokens (k_g, v_g); without them the global
// tiles and the kind 3 exponent offset are compiled out.  The d = 64, b = 128
// plain kernel fits three workgroups per CU (168 VGPRs, 45 KB LDS): its softmax VALU
// work is that of d = 128 over half the MFMAs, and the third wavefront per SIMD
// fills more of the VALU gaps.
template <int D, int BLK, int QB, int MODE, bool GLOB = false>
__global__ __launch_bounds__(QB / 32 * 64)
__attribute__((amdgpu_waves_per_eu(D == 64 && BLK == 128 && MODE == 0 ? 3 : 2,
                                  D == 64 && BLK == 128 && MODE == 0 ? 3 : 2)))
void attn_fwd_kernel(
    const __bf16* __restrict__ q_r, const __bf16* __restrict__ k_r, const __bf16* __restrict__ v_t,
    const int32_t* __restrict__ kv_count, const int32_t* __restrict__ kv_idx,
    const int32_t* __restrict__ order,
    const __bf16* __restrict__ k_g, const __bf16* __restrict__ v_g,
    __bf16* __restrict__ o_r, float* __restrict__ lse,
    int Hh, int N, int Npad, int nb, int Ng, float sl2, float bias_n, float bias_last, int total, TokIO tok,
    const int32_t* __restrict__ q_count, const int32_t* __restrict__ rowsel) {
  using C = AttnCfg<D, BLK, QB>;
  // d = 128: each phase waits only for the copies it reads (two barriers per
  // iteration).  d = 64: the kernel is VALU-bound and a second barrier costs
  // more than the lead it buys, so both copies go out after phase A's first
  // MFMAs and one full wait opens the iteration (1.59 against 1.63-1.68 ms on
  // the CogVideoX-shaped layer, 3% slower at d = 128 on the long layer).
  constexpr bool kSplitWait = D == 128;
  constexpr int kSubQ = BLK / QB;   // work items per query block
  constexpr int kHalfW = C::kWaves / 2;
  static_assert(MODE != 2 || QB == BLK, "pairs take whole-block workgroups");
  // Four distinct arrays whose roles are static in each half of the 2x-unrolled
  // pipeline, so the compiler can prove LDS reads never alias a DMA in flight
  // and does not make them wait for it.
  __shared__ __attribute__((aligned(1024))) char Vb0[C::kVBytes];
  __shared__ __attribute__((aligned(1024))) char Vb1[C::kVBytes];
  __shared__ __attribute__((aligned(1024))) char Kb0[C::kKBytes];
  __shared__ __attribute__((aligned(1024))) char Kb1[C::kKBytes];
  // The kept-block list of this query block, one word per entry (index and
  // masking flags, see kIndexMask).
  __shared__ uint16_t idx_s[4096];
  // Mode 2: bit 14 + x of a list word is set when block 2P + x does not keep
  // the entry (the union holds no invalid entries, whose flag bit 14 is
  // otherwise).
  __shared__ int wtot_s[C::kWaves];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  // Work item: this XCD's next entry of the schedule (longest query blocks
  // first when build_mask wrote one), clamped so a bad schedule stays in bounds.
  const int slot = xcd_remap(blockIdx.x, total);
  int I, bh;
  if constexpr (MODE == 2) {
    if (order != nullptr) {
      // rows in the work order; a pair runs at its first block's place
      const int wid = min(max(__builtin_amdgcn_readfirstlane(order[slot]), 0), total - 1);
      if (wid % nb % 2 != 0) return;   // the whole workgroup, before any barrier
      I = wid % nb;
      bh = wid / nb;
    } else {
      const int np = (nb + 1) / 2;
      bh = slot / np;
      I = 2 * (slot % np);
    }
  } else {
    const int rows_total = total / kSubQ;
    const int wid = order == nullptr ? slot / kSubQ
                                     : min(max(__builtin_amdgcn_readfirstlane(order[slot / kSubQ]), 0),
                                           rows_total - 1);
    I = wid % nb;
    bh = wid / nb;
  }
  const int64_t rowbase = (int64_t)bh * Npad;
  // kept-row count of block J of this head, clamped
  auto kept_rows = [&](int J) {
    const int mq = __builtin_amdgcn_readfirstlane(q_count[(int64_t)bh * nb + J]);
    return mq < 0 ? 0 : (mq > BLK ? BLK : mq);
  };
  // blocks 2P, 2P + 1 go to mode 2 together when both fit half a workgroup
  auto paired = [&](int I0) { return I0 + 1 < nb && kept_rows(I0) <= QB / 2 && kept_rows(I0 + 1) <= QB / 2; };
  // this lane's query row (reordered index) and whether it is one
  int qrow = I * BLK + wave * C::kQW + l32;
  bool qvalid = qrow < N;
  int half = 0;   // mode 2: which block of the pair this wavefront serves
  if constexpr (MODE == 1) {
    const int sub = slot % kSubQ;
    const int mq = kept_rows(I);
    if (sub * QB >= mq || paired(I & ~1)) return;   // the whole workgroup, before any barrier
    const int s = sub * QB + wave * C::kQW + l32;
    qrow = s < mq ? rowsel[((int64_t)bh * nb + I) * BLK + s] : -1;
    qvalid = qrow >= 0 && qrow < N;
    if (!qvalid) qrow = 0;
  } else if constexpr (MODE == 2) {
    if (!paired(I)) return;                           // the whole workgroup, before any barrier
    half = wave / kHalfW;
    const int mq = kept_rows(I + half);
    const int s = (wave % kHalfW) * C::kQW + l32;
    qrow = s < mq ? rowsel[((int64_t)bh * nb + I + half) * BLK + s] : -1;
    qvalid = qrow >= 0 && qrow < N;
    if (!qvalid) qrow = 0;
  }

  // List word of kept-block index J (see kIndexMask).
  auto word_of = [&](int J) {
    const bool ok = J >= 0 && J < nb;
    int w = ok ? J : kInvalidBit;
#pragma unroll
    for (int h = 0; h < C::kSubs; ++h)
      if (!ok || J * BLK + (h + 1) * C::kKT > N) w |= kPartial << h;
    return w;
  };
  int cnt = __builtin_amdgcn_readfirstlane(kv_count[(int64_t)bh * nb + I]);
  cnt = cnt < 0 ? 0 : (cnt > nb ? nb : cnt);
  const int32_t* idx = kv_idx + ((int64_t)bh * nb + I) * nb;
  if constexpr (MODE == 2) {
    // The union of the two blocks' kept-block sets, ascending, with each
    // entry's membership, into idx_s: both lists become bitmaps over
    // the nb <= 4096 blocks (staged in the first K buffer, which the first
    // copies overwrite only after the barriers below), and a scan of the
    // union's popcounts places every block.  Entries out of [0, nb) and
    // repeats drop out (they add nothing to the attention).
    int c1 = __builtin_amdgcn_readfirstlane(kv_count[(int64_t)bh * nb + I + 1]);
    c1 = c1 < 0 ? 0 : (c1 > nb ? nb : c1);
    const int32_t* idx1 = idx + nb;
    uint32_t* bA = reinterpret_cast<uint32_t*>(Kb0);   // 128 words each
    uint32_t* bB = bA + 128;
    static_assert(C::kKBytes >= 1024, "a K buffer holds the two bitmaps");
    for (int t = threadIdx.x; t < 256; t += C::kThreads) bA[t] = 0u;   // bA and bB
    __syncthreads();
    for (int t = threadIdx.x; t < cnt; t += C::kThreads) {
      const int J = idx[t];
      if (J >= 0 && J < nb) atomicOr(&bA[J >> 5], 1u << (J & 31));
    }
    for (int t = threadIdx.x; t < c1; t += C::kThreads) {
      const int J = idx1[t];
      if (J >= 0 && J < nb) atomicOr(&bB[J >> 5], 1u << (J & 31));
    }
    __syncthreads();
    const uint32_t wa = threadIdx.x < 128 ? bA[threadIdx.x] : 0u;
    const uint32_t wb = threadIdx.x < 128 ? bB[threadIdx.x] : 0u;
    const int pc = __popc(wa | wb);
    int inc = pc;   // inclusive scan over the wavefront
#pragma unroll
    for (int dd = 1; dd < 64; dd <<= 1) {
      const int o = __shfl_up(inc, dd, 64);
      if (lane >= dd) inc += o;
    }
    if (lane == 63) wtot_s[wave] = inc;
    __syncthreads();
    int pos = inc - pc;
    for (int w = 0; w < wave; ++w) pos += wtot_s[w];
    for (uint32_t u = wa | wb; u != 0u; u &= u - 1u, ++pos) {
      const int bit = __ffs((int)u) - 1;
      const int absent = (((wa >> bit) & 1u) ? 0 : 0x4000) | (((wb >> bit) & 1u) ? 0 : 0x8000);
      idx_s[pos] = (uint16_t)(word_of(threadIdx.x * 32 + bit) | absent);
    }
    int u = 0;
    for (int w = 0; w < C::kWaves; ++w) u += wtot_s[w];
    __syncthreads();
    cnt = __builtin_amdgcn_readfirstlane(u);
  }
  const int Ngpad = (Ng + BLK - 1) / BLK * BLK;
  const int ntg = (GLOB && k_g != nullptr) ? Ngpad / BLK : 0;
  const int U = (cnt + ntg) * C::kSubs;

  // Buffer descriptors of this head's K rows, V^T tiles and global-token
  // tiles (raw addressing, 32-bit data format: word 3 = 0x00020000 on gfx9).
  // The copies address them with a per-stage scalar offset and per-lane
  // offsets; buffer copies to LDS count on vmcnt only.
  const auto rk = make_rsrc(k_r + rowbase * D, (uint32_t)Npad * (uint32_t)(D * 2));
  const auto rv = make_rsrc(v_t + (int64_t)bh * nb * (D * BLK), (uint32_t)nb * (uint32_t)(D * BLK * 2));
  const auto rkg = make_rsrc(ntg > 0 ? k_g + (int64_t)bh * Ngpad * D : k_r, (uint32_t)Ngpad * (uint32_t)(D * 2));
  const auto rvg = make_rsrc(ntg > 0 ? v_g + (int64_t)bh * Ngpad * D : v_t, (uint32_t)Ngpad * (uint32_t)(D * 2));

  // Stage u: kept block j = u / kSubs of the list, or global-token tile j - cnt.
  // Selects only (no branches), so the copies can be scheduled inside the
  // MFMA phases.  The list word carries the block index and the masking
  // flags, so a full stage costs a handful of scalar operations.
  const int cnt_m1 = cnt > 0 ? cnt - 1 : 0;
  // Stage u from the list word w of its block (ignored for global tiles).
  auto stage_w = [&](int u, int w) -> StageDesc {
    StageDesc s;
    const int j = (int)((unsigned)u / C::kSubs), h = (int)((unsigned)u % C::kSubs);
    const bool kept = j < cnt;
    const int Jx = kept ? (w & kIndexMask) : j - cnt;
    s.key0 = Jx * BLK + h * C::kKT;
    s.koffs = (uint32_t)s.key0 * (uint32_t)(D * 2);
    s.voffs = ((uint32_t)Jx * (uint32_t)(D * BLK) + (uint32_t)(h * C::kKT)) * 2u;
    s.glob = !kept;
    // a global tile whose keys all precede the last global token adds the same ln n to
    // every score: it needs neither the per-key bias nor a mask
    s.kind = kept ? ((w >> h) & kPartial ? 1 : 0) : (GLOB && s.key0 + C::kKT <= Ng - 1 ? 3 : 2);
    s.limit = kept ? ((MODE != 2 && (w & kInvalidBit)) ? -1 : N) : Ng;
    // mode 2: a block of the union that this wavefront's query block does
    // not keep; its probabilities are made zero through the exponent offset
    // (no per-key mask) and its maximum is ignored
    s.absent = MODE == 2 && kept && ((w >> (14 + half)) & 1);
    return s;
  };
  auto stage = [&](int u) -> StageDesc {
    const int j = (int)((unsigned)u / C::kSubs);
    return stage_w(u, __builtin_amdgcn_readfirstlane((int)idx_s[min(j, cnt_m1)]));
  };

  // Per-lane source offsets (elements) of the padded DMA: loop invariant.
  // LDS byte 1024 n + 16 lane of a stage holds padded unit p = 64 n + lane,
  // i.e. row p / rowU, unit p % rowU; the pad unit re-reads the row's last
  // unit (same cache line, no extra traffic).  Every wavefront issues kKPer
  // (kVPer) copies per stage; where the stage has fewer, the surplus ones
  // repeat the last copy, writing the same bytes (no branch in the issue).
  int koff[C::kKPer], voff[C::kVPer];
#pragma unroll
  for (int i = 0; i < C::kKPer; ++i) {
    const int n = min(wave + i * C::kWaves, C::kKInstr - 1);
    const int p = 64 * n + lane;
    const int row = p / C::kKRowU, c = min(p % C::kKRowU, C::kKRowU - 2);
    koff[i] = row * D + c * 8;
  }
#pragma unroll
  for (int i = 0; i < C::kVPer; ++i) {
    const int n = min(wave + i * C::kWaves, C::kVInstr - 1);
    const int p = 64 * n + lane;
    const int row = p / C::kVRowU, c = min(p % C::kVRowU, C::kVRowU - 2);
    voff[i] = row * BLK + c * 8;
  }
  auto dma_k = [&](const StageDesc& s, char* buf) {
#pragma unroll
    for (int i = 0; i < C::kKPer; ++i) {
      const int n = min(wave + i * C::kWaves, C::kKInstr - 1);
      copy16_lds((MODE == 0 && s.glob) ? rkg : rk, buf + 1024 * n, (uint32_t)koff[i] * 2u, s.koffs);
    }
  };
  auto dma_v = [&](const StageDesc& s, char* buf) {
#pragma unroll
    for (int i = 0; i < C::kVPer; ++i) {
      const int n = min(wave + i * C::kWaves, C::kVInstr - 1);
      copy16_lds((MODE == 0 && s.glob) ? rvg : rv, buf + 1024 * n, (uint32_t)voff[i] * 2u, s.voffs);
    }
  };

  // Per-lane LDS read bases (bytes): K row l32 at unit g; V^T row l32 at unit g.
  const int kbase = l32 * C::kKStride + 16 * g;
  const int vbase = l32 * C::kVStride + 16 * g;
  auto read_k = [&](const char* kb, int kt, int kk) {
    return *reinterpret_cast<const bf16x8_t*>(kb + kbase + kt * 32 * C::kKStride + kk * 32);
  };
  auto read_v = [&](const char* vb, int dt, int st) {
    return *reinterpret_cast<const bf16x8_t*>(vb + vbase + dt * 32 * C::kVStride + st * 32);
  };

  bf16x8_t qreg[D / 16];   // Q^T operand, loaded once the kept-block list is in LDS
  f32x16_t oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = f32x16_t{};
  float m = -INFINITY, mneg = 0.f, l = 0.f;
  bool cur_abs = false;   // mode 2: the current stage is absent for this wavefront
  // The current stage's constant logit bias in log2 units (kind 3 stages: ln n * log2 e); the
  // probabilities are exp2(S * sl2 + mneg + cur_eb).
  float cur_eb = 0.f;
  const float eb3 = bias_n * sl2;

  // S^T tiles of one stage: S[kt][v] is key 32 kt + (v/4)*8 + 4g + v%4 of
  // query l32.
  auto scores = [&](const char* kb, f32x16_t (&S)[2]) {
    S[0] = f32x16_t{};
    S[1] = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        S[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_k(kb, kt, kk), qreg[kk], S[kt], 0, 0, 0);
    }
  };

  // Partial and invalid stages and the last global-token tile: move the ASA_G
  // bias into the raw score domain (ln r / scale) and mask keys past the stage's
  // limit.  The other global-token tiles (kind 3) carry ln n on every key, which
  // shifts their maximum by ln n and their exponent offset by ln n * log2 e.
  auto fixup = [&](const StageDesc& s, f32x16_t (&S)[2]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = s.key0 + 32 * kt + (v >> 2) * 8 + 4 * g + (v & 3);
        float t = S[kt][v];
        if (s.kind == 2) t += (key < s.limit - 1) ? bias_n : bias_last;
        S[kt][v] = key >= s.limit ? -INFINITY : t;
      }
    }
  };

  // Maximum of the 32 scores of one stage as a tree of 3-input maxima (16 ops).
  auto row_max = [&](const f32x16_t (&S)[2]) {
    auto mx3 = [](float a, float b, float c) { return fmaxf(fmaxf(a, b), c); };
    float x[32];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      x[v] = S[0][v];
      x[16 + v] = S[1][v];
    }
    float a[10];
#pragma unroll
    for (int j = 0; j < 10; ++j) a[j] = mx3(x[3 * j], x[3 * j + 1], x[3 * j + 2]);
    const float c = mx3(a[9], x[30], x[31]);
    const float d = mx3(mx3(a[0], a[1], a[2]), mx3(a[3], a[4], a[5]), mx3(a[6], a[7], a[8]));
    return fmaxf(d, c);
  };

  // Raise the running maximum (log2 units) when the stage maximum mx_raw (raw
  // score units) exceeds it by more than the lazy threshold.
  auto decide = [&](float mx_raw) {
    const float mx = max_halves(mx_raw) * sl2;
    const bool need = mx > m + kLazyThreshold;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float alpha = need ? fast_exp2(m - mx) : 1.f;
      m = need ? mx : m;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) oacc[dt] *= alpha;
    }
    mneg = (m == -INFINITY) ? 0.f : -m;
  };

  // Phase A: probabilities of the current stage (and, with a next stage, the
  // next stage's score MFMAs interleaved with them and the K copies of the
  // stage after it).
  auto phase_a = [&](const f32x16_t (&Sc)[2], f32x16_t (&Sn)[2], const char* ksrc, uint32_t (&P)[16],
                     const StageDesc* dk, char* kdst, const StageDesc* dv, char* vdst, auto has_next) {
    constexpr bool kNext = decltype(has_next)::value;
    if constexpr (kNext) {
      scores(ksrc, Sn);
      dma_k(*dk, kdst);
      if constexpr (!kSplitWait) dma_v(*dv, vdst);
      // The phase's order: every LDS operand read runs 2 MFMAs ahead of its
      // use, and one K copy follows each of the first MFMAs (the earliest
      // issue gives the copies the most lead; one copy every third MFMA
      // measured 0.5-1% slower).
      constexpr int kL = 2, kMM = 2 * (D / 16);
      __builtin_amdgcn_sched_group_barrier(kSgDsRead, kL, 0);
#pragma unroll
      for (int i = 0; i < kMM; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        if (i + kL < kMM) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
        if (i < C::kKPer + (kSplitWait ? 0 : C::kVPer)) __builtin_amdgcn_sched_group_barrier(kSgVmem, 1, 0);
      }
    }
    const float mn = (MODE == 2 && cur_abs) ? -INFINITY : (GLOB ? mneg + cur_eb : mneg);
    float s0, s1;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int kt = st >> 1, o = (st & 1) * 8;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pa = fast_exp2(__builtin_fmaf(Sc[kt][o + 2 * e], sl2, mn));
        const float pb = fast_exp2(__builtin_fmaf(Sc[kt][o + 2 * e + 1], sl2, mn));
        P[4 * st + e] = cvt_pk(pa, pb);
        s0 = (st | e) == 0 ? pa : s0 + pa;
        s1 = (st | e) == 0 ? pb : s1 + pb;
      }
    }
    l += s0 + s1;
    asm volatile("" ::"v"(l));   // keep the row sums in this phase
  };

  // Phase B: O^T += V^T P^T for the current stage (and the next stage's
  // row maximum interleaved with it, and the next stage's V copies).
  auto phase_b = [&](const char* vsrc, const uint32_t (&P)[16], const f32x16_t (&Sn)[2],
                     const StageDesc* dv, char* vdst, auto has_next) {
    constexpr bool kNext = decltype(has_next)::value;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      uint4 w;
      w.x = P[4 * st + 0];
      w.y = P[4 * st + 1];
      w.z = P[4 * st + 2];
      w.w = P[4 * st + 3];
      const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, w);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_v(vsrc, dt, st), pb, oacc[dt], 0, 0, 0);
    }
    float mx = -INFINITY;
    if constexpr (kNext) {
      mx = row_max(Sn);
      if constexpr (kSplitWait) dma_v(*dv, vdst);
      // The same order for the PV MFMAs, one V copy after each of the first.
      constexpr int kL = 2, kMM = 4 * (D / 32), kVm = C::kVPer;
      __builtin_amdgcn_sched_group_barrier(kSgDsRead, kL, 0);
#pragma unroll
      for (int i = 0; i < kMM; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        if (i + kL < kMM) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
        if (kSplitWait && i < kVm) __builtin_amdgcn_sched_group_barrier(kSgVmem, 1, 0);
      }
    }
    return mx;
  };

  // One pipeline iteration for stage u with a next stage u+1.  kdst / vdst
  // receive the DMAs of stages u+2 (K) and u+1 (V); ksrc holds K of stage u+1
  // and vsrc holds V of stage u.
  auto iterate = [&](int u, const f32x16_t (&Sc)[2], f32x16_t (&Sn)[2], char* kdst, char* vdst,
                     const char* ksrc, const char* vsrc, const StageDesc& sn) {
    const StageDesc sk = stage(min(u + 2, U - 1));   // past the end: a harmless repeat
    uint32_t P[16];
    if constexpr (kSplitWait) {
      // K of stage u+1 (copied in the previous iteration's phase A) is complete
      // once at most its V copies (phase B) are outstanding
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(C::kVPer) : "memory");
      phase_a(Sc, Sn, ksrc, P, &sk, kdst, &sn, vdst, std::true_type{});
      // V of stage u: complete once at most this iteration's K copies are outstanding
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(C::kKPer) : "memory");
    } else {
      // every copy of the previous iteration (K of stage u+1, V of stage u) is complete
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      phase_a(Sc, Sn, ksrc, P, &sk, kdst, &sn, vdst, std::true_type{});
    }
    float mx = phase_b(vsrc, P, Sn, &sn, vdst, std::true_type{});
    // Pin the maximum inside the phase (otherwise it is sunk past the branch
    // below, away from the MFMAs it is meant to overlap).
    asm volatile("" ::"v"(mx));
    if (sn.kind == 1 || sn.kind == 2) {
      fixup(sn, Sn);
      mx = row_max(Sn);
    } else if (sn.kind == 3) {
      mx += bias_n;   // the maximum of the biased scores
    }
    if constexpr (MODE == 2) {
      if (sn.absent) mx = -INFINITY;
    }
    decide(mx);
    if constexpr (GLOB) cur_eb = sn.kind == 3 ? eb3 : 0.f;
    if constexpr (MODE == 2) cur_abs = sn.absent;
    return sk;
  };

  // The last stage: no next stage to score.
  auto last = [&](const f32x16_t (&Sc)[2], const char* vsrc) {
    wait_dma();
    __syncthreads();
    uint32_t P[16];
    f32x16_t unused[2];
    phase_a(Sc, unused, nullptr, P, nullptr, nullptr, nullptr, nullptr, std::false_type{});
    phase_b(vsrc, P, unused, nullptr, nullptr, std::false_type{});
  };

  // Prologue order matters because vector loads retire in order: this
  // thread's list entry first, then the token lookup, then the first copies;
  // the list word is then stored without waiting for the copies, and the Q
  // gather waits for the token lookup only.
  const int jt = (MODE != 2 && threadIdx.x < cnt) ? idx[threadIdx.x] : 0;

  // Q^T operand: lane (l32, g) holds Q[qrow][16 kk + 8 g .. +7], from the
  // reordered rows or, in token order, from the row's token (bf16, or float32
  // rounded to bf16 as the reorder rounds it; rows >= N are zero).
  const int bi = bh / Hh, hh = bh % Hh;
  auto token_of = [&](int row) {
    const int t = tok.perm[(int64_t)hh * tok.perm_h_stride + row];
    return t < 0 ? 0 : (t >= N ? N - 1 : t);
  };
  // token of this lane's query row (used again by the epilogue)
  const int qtok = (tok.perm != nullptr && qvalid) ? token_of(qrow) : 0;

  // The first two stages need list entries 0 and 1 only: their words come
  // straight from global memory, so the first copies start before the list
  // reaches LDS.
  StageDesc s0{}, sd{};
  if (U > 0) {
    const int w0 = MODE == 2 ? __builtin_amdgcn_readfirstlane((int)idx_s[0])
                             : word_of(__builtin_amdgcn_readfirstlane(idx[0]));
    const int w1 = MODE == 2 ? __builtin_amdgcn_readfirstlane((int)idx_s[min(1, cnt_m1)])
                             : word_of(__builtin_amdgcn_readfirstlane(idx[min(1, cnt_m1)]));
    const int u1 = min(1, U - 1);
    s0 = stage_w(0, w0);
    sd = stage_w(u1, u1 / C::kSubs == 0 ? w0 : w1);
    dma_k(s0, Kb0);
    dma_v(s0, Vb0);
    dma_k(sd, Kb1);
  }
  if (MODE != 2) {
    if (threadIdx.x < cnt) idx_s[threadIdx.x] = (uint16_t)word_of(jt);
    for (int t = threadIdx.x + C::kThreads; t < cnt; t += C::kThreads) idx_s[t] = (uint16_t)word_of(idx[t]);
  }
  // The list is in LDS: wait for the LDS writes only (a full __syncthreads
  // would also wait for the copies above and the Q loads below).
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  if (tok.q == nullptr && (MODE == 0 || qvalid)) {
    const __bf16* qp = q_r + (rowbase + qrow) * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qreg[kk] = *reinterpret_cast<const bf16x8_t*>(qp + 16 * kk);
  } else if (!qvalid) {
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qreg[kk] = bf16x8_t{};
  } else {
    const int64_t off = bi * tok.qsb + (int64_t)qtok * tok.qsn + hh * tok.qsh + 8 * g;
    if (tok.q_f32) {
      const float* qp = reinterpret_cast<const float*>(tok.q) + off;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const float4 a = reinterpret_cast<const float4*>(qp + 16 * kk)[0];
        const float4 c = reinterpret_cast<const float4*>(qp + 16 * kk)[1];
        const uint4 w = make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(c.x, c.y),
                                   pack_bf16x2(c.z, c.w));
        qreg[kk] = __builtin_bit_cast(bf16x8_t, w);
      }
    } else {
      const __bf16* qp = reinterpret_cast<const __bf16*>(tok.q) + off;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) qreg[kk] = *reinterpret_cast<const bf16x8_t*>(qp + 16 * kk);
    }
  }

  if (U > 0) {
    wait_dma();
    __syncthreads();
    f32x16_t SA[2], SB[2];
    scores(Kb0, SA);
    if (s0.kind == 1 || s0.kind == 2) fixup(s0, SA);
    decide((MODE == 2 && s0.absent) ? -INFINITY : row_max(SA) + (s0.kind == 3 ? bias_n : 0.f));
    if constexpr (GLOB) cur_eb = s0.kind == 3 ? eb3 : 0.f;
    if constexpr (MODE == 2) cur_abs = s0.absent;
    int u = 0;
    for (; u + 2 < U; u += 2) {
      sd = iterate(u, SA, SB, Kb0, Vb1, Kb1, Vb0, sd);
      sd = iterate(u + 1, SB, SA, Kb1, Vb0, Kb0, Vb1, sd);
    }
    if (u + 1 < U) {
      iterate(u, SA, SB, Kb0, Vb1, Kb1, Vb0, sd);
      last(SB, Vb1);
    } else {
      last(SA, Vb0);
    }
  }

  // ---- epilogue -------------------------------------------------------------------
  const float lt = sum_halves(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const int q = qrow;
  if (qvalid) {
    // lane (l32, g) holds channels 32 dt + 8 i + 4 g .. +3 of its query row
    if (tok.out != nullptr && tok.out_f32) {
      float* op = reinterpret_cast<float*>(tok.out) + bi * tok.osb + (int64_t)qtok * tok.osn +
                  hh * tok.osh + 4 * g;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // the bf16 value of the output, widened exactly
          const uint32_t lo = cvt_pk(oacc[dt][i * 4 + 0] * inv, oacc[dt][i * 4 + 1] * inv);
          const uint32_t hi = cvt_pk(oacc[dt][i * 4 + 2] * inv, oacc[dt][i * 4 + 3] * inv);
          *reinterpret_cast<float4*>(op + 32 * dt + 8 * i) =
              make_float4(__uint_as_float(lo << 16), __uint_as_float(lo & 0xffff0000u),
                          __uint_as_float(hi << 16), __uint_as_float(hi & 0xffff0000u));
        }
      }
    } else {
      __bf16* op = tok.out != nullptr
                       ? reinterpret_cast<__bf16*>(tok.out) + bi * tok.osb + (int64_t)qtok * tok.osn +
                             hh * tok.osh + 4 * g
                       : o_r + (rowbase + q) * D + 4 * g;
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
    }
    if (lse != nullptr && g == 0) {
      lse[rowbase + q] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
    }
  }
}

template <int D, int BLK, int QB = BLK, int MODE = 0, bool GLOB = false>
hipError_t launch(const AttnArgs& a) {
  // mode 2: one work item per pair, or per row (odd rows exit) when a work order is given
  const int total = (MODE == 2 && a.order == nullptr) ? a.B * a.Hh * ((a.nb + 1) / 2)
                                                      : a.B * a.Hh * a.nb * (BLK / QB);
  const float sl2 = a.scale * kLog2e;
  float bias_n = 0.f, bias_last = 0.f;
  if (a.k_g != nullptr) {
    // ln r in raw score units: the kernel multiplies scores by scale * log2(e)
    bias_n = (float)(std::log((double)a.n_pool) / a.scale);
    bias_last = (float)(std::log((double)(a.N - (a.Ng - 1) * a.n_pool)) / a.scale);
  }
  hipLaunchKernelGGL((attn_fwd_kernel<D, BLK, QB, MODE, GLOB>), dim3(total), dim3(AttnCfg<D, BLK, QB>::kThreads), 0,
                     a.stream, (const __bf16*)a.q_r, (const __bf16*)a.k_r, (const __bf16*)a.v_t,
                     a.kv_count, a.kv_idx, a.order, (const __bf16*)a.k_g, (const __bf16*)a.v_g,
                     (__bf16*)a.o_r, a.lse, a.Hh, a.N, a.Npad, a.nb, a.Ng, sl2, bias_n, bias_last,
                     total, a.tok, a.q_count, a.rowsel);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const AttnArgs& a) {
  if (a.rowsel != nullptr) {   // pruned queries: pairs of blocks, then the unpaired blocks
    hipError_t e;
    if (a.d == 64) e = a.b == 64 ? launch<64, 64, 64, 2>(a) : launch<64, 128, 128, 2>(a);
    else e = a.b == 64 ? launch<128, 64, 64, 2>(a) : launch<128, 128, 128, 2>(a);
    if (e != hipSuccess) return e;
    if (a.d == 64) return a.b == 64 ? launch<64, 64, 64, 1>(a) : launch<64, 128, 128, 1>(a);
    return a.b == 64 ? launch<128, 64, 64, 1>(a) : launch<128, 128, 128, 1>(a);
  }
  if (a.k_g != nullptr) {
    if (a.d == 64) return a.b == 64 ? launch<64, 64, 64, 0, true>(a) : launch<64, 128, 128, 0, true>(a);
    return a.b == 64 ? launch<128, 64, 64, 0, true>(a) : launch<128, 128, 128, 0, true>(a);
  }
  if (a.d == 64) return a.b == 64 ? launch<64, 64>(a) : launch<64, 128>(a);
  return a.b == 64 ? launch<128, 64>(a) : launch<128, 128>(a);
}

}  // namespace dbs
