// Backward of the block-sparse attention (plain ASA) over the kept-block
// lists (gfx950).
//
// The forward is Video-BLADE "Step 2.2": every query block attends to its
// kept key blocks.  Its gradient, with P = softmax(S), S = Q K^T * scale:
//     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D_q = sum_d dO_qd O_qd,
//     dQ = dS K * scale,  dK = dS^T Q * scale.
// P is recomputed from the scores and the forward's log-sum-exp, so nothing of
// size N x N is stored.  The key-to-query direction needs the lists the other
// way round (the BSA notes' reverse scatter of q2k_index): for every key block
// J, the query blocks whose list holds J.
//
// Launches:
//   transpose_lists: a bit matrix (query block x key block) per group of 32
//     key blocks in LDS, read out in ascending query block.
//   dq: one workgroup per (batch, head, query block), 32 query rows per
//     wavefront, over the block's kept key blocks in tiles of 32 keys:
//       S^T = K Q^T, dP^T = V dO^T (Q^T, dO^T in VGPRs), P^T, dS^T in the
//       lane's registers (each lane holds one query: lse and D are scalars),
//       dQ^T += K^T dS^T.  It also writes D for the next launch.
//   dkdv: one workgroup per (batch, head, key block), 32 keys per wavefront,
//     over the query blocks that keep it, in tiles of 32 queries:
//     S = Q K^T, dP = dO V^T (K^T, V^T in VGPRs), dV^T += dO^T P,
//     dK^T += Q^T dS.
// A stage (the tokens copied between two barriers) holds two tiles in a
// 128-row workgroup and one in a 64-row workgroup.
// All products are bf16 MFMA 32x32x16 with fp32 accumulation; P and dS are
// rounded to bf16 for the second product.  The products that contract over
// tokens (dV^T += dO^T P, dK^T += Q^T dS, dQ^T += K^T dS^T) take their A
// operand from the token rows already in LDS by transposing reads
// (ds_read_b64_tr_b16), so no transposed copy of Q, dO or K is made; the MFMA
// tile rows map to the stage's token rows through a fixed permutation that
// keeps both kinds of LDS read free of bank conflicts.  Stage data are copied
// global -> LDS by the buffer form of the DMA path into row-padded LDS through
// a ring of two stage buffers (one stage in flight while one computes), and
// both kernels are held to 256 VGPRs: two workgroups then share each CU (two
// wavefronts per SIMD).
#include "common.h"
#include "../launch.h"

namespace dbs {
namespace {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

__device__ __forceinline__ uint32_t cvt_pk(float a, float b) {
  bf16x2_t p;
  p[0] = (__bf16)a;
  p[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ float sum_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N vector-memory instructions of this wavefront are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void copy16_lds(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, voff, soff, 0, 0);
}

// Stage layouts in LDS (KT tokens per stage), each a whole number of 1 KiB
// copy instructions (a rows stage of 32 tokens leaves a spare half KiB that
// the surplus lanes of its last copy fill).
template <int D, int KT>
struct BwdCfg {
  static constexpr int kT = KT;
  static constexpr int kRowU = D / 8 + 1;          // rows stage: KT rows of D, padded by one 16-byte unit
  static constexpr int kRowStride = kRowU * 16;
  static constexpr int kRowInstr = (KT * kRowU + 63) / 64;
  static constexpr int kRowBytes = kRowInstr * 1024;
};

// Per-lane source offsets (elements) of the padded copies: LDS byte 1024 n +
// 16 lane of a stage holds padded unit p = 64 n + lane, i.e. row p / rowU,
// unit p % rowU (the pad unit re-reads the row's last unit).  Surplus
// instructions of a wavefront repeat the last one; surplus lanes of a rows
// stage read the rows just past it (out of range: zero) into the spare bytes.
template <int D, int BLK, int W, int KT>
struct StageCopies {
  using C = BwdCfg<D, KT>;
  static constexpr int kRowPer = (C::kRowInstr + W - 1) / W;
  uint32_t roff[kRowPer];
  int wave, lane;
  __device__ __forceinline__ void init(int w, int l) {
    wave = w;
    lane = l;
#pragma unroll
    for (int i = 0; i < kRowPer; ++i) {
      const int n = min(wave + i * W, C::kRowInstr - 1);
      const int p = 64 * n + lane;
      const int row = p / C::kRowU, c = min(p % C::kRowU, C::kRowU - 2);
      roff[i] = (uint32_t)(row * D + c * 8) * 2u;
    }
  }
  __device__ __forceinline__ void rows(__amdgpu_buffer_rsrc_t r, uint32_t soff, char* buf) const {
#pragma unroll
    for (int i = 0; i < kRowPer; ++i) {
      const int n = min(wave + i * W, C::kRowInstr - 1);
      copy16_lds(r, buf + 1024 * n, roff[i], soff);
    }
  }
};

// Tile row m of the first product of a stage (the MFMA row that lane l32 = m
// of the A operand feeds, and accumulator row acc_row) is stage row
// stage_row(m): within each group of 16, m = 8 h + 4 g + e goes to row
// 4 e + 2 h + g.  The LDS serves 16 lanes of a 16-byte read or 32 lanes of an
// 8-byte read per cycle from 64 banks; at the padded row stride (an odd
// number of 16-byte units) the 16 rows of a 16-byte row read start in distinct
// bank quads, and the 4 rows 4 e + c of a transposing read (64 bytes of each
// per 32 lanes) start in distinct quarters of the banks, so neither kind of
// read meets a bank conflict.
__device__ __forceinline__ int stage_row(int m) { return (m & ~15) | (((m >> 3) & 1) << 1) | ((m >> 2) & 1) | ((m & 3) << 2); }
__device__ __forceinline__ int tile_row(int r) { return (r & ~15) | (((r >> 1) & 1) << 3) | ((r & 1) << 2) | ((r >> 2) & 3); }

// MFMA operand read (16 bytes per lane): rows stage, tile row l32, k step kk
// (elements 16 kk + 8 g ..).
template <class C>
__device__ __forceinline__ bf16x8_t read_rows(const char* buf, int l32, int g, int kk) {
  return *reinterpret_cast<const bf16x8_t*>(buf + stage_row(l32) * C::kRowStride + 16 * g + kk * 32);
}
// A operand of a product contracting over the 32 token rows of a rows stage
// (dO^T, Q^T, K^T): lane (l32, g) receives column 32 dt + l32 of the stage rows
// of tile rows 16 st + 4 g + e and 16 st + 8 + 4 g + e (e < 4), the k order
// pack_half gives the B operand.  Two transposing LDS reads (ds_read_b64_tr_b16):
// in each group of 16 lanes, lane i points at 4 consecutive columns
// 4 (i & 3) .. of the (i >> 2)-th row of a 4-row set, and lane l receives
// column l of the set's 4 rows.
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;
template <class C>
__device__ __forceinline__ bf16x8_t read_rows_tr(const char* buf, int lane, int dt, int st) {
  const int grp = lane >> 4, i = lane & 15;
  const int row = 16 * st + (grp >> 1) + 4 * (i >> 2);   // stage_row(16 st + 4 g + (i >> 2))
  const int col = 32 * dt + 16 * (grp & 1) + 4 * (i & 3);
  const char* p = buf + row * C::kRowStride + 2 * col;
  const short4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)p);
  const short4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(p + 2 * C::kRowStride));
  typedef short short8_t __attribute__((ext_vector_type(8)));
  const short8_t ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, ab);
}

// B operand of a product contracting over the 32 rows of one accumulator tile
// T, 16-row step st: the lane's 8 values of that step (tile rows 16 st + 4 g + e and
// 16 st + 8 + 4 g + e, e < 4), the order read_rows_tr gives the A operand.
__device__ __forceinline__ bf16x8_t pack_half(const f32x16_t& T, int st) {
  const int o = st * 8;
  uint4 w;
  w.x = cvt_pk(T[o + 0], T[o + 1]);
  w.y = cvt_pk(T[o + 2], T[o + 3]);
  w.z = cvt_pk(T[o + 4], T[o + 5]);
  w.w = cvt_pk(T[o + 6], T[o + 7]);
  return __builtin_bit_cast(bf16x8_t, w);
}

__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row r of a 32 x 32 accumulator tile held in element v of lane half g.
__device__ __forceinline__ int acc_row(int v, int g) { return (v >> 2) * 8 + 4 * g + (v & 3); }

// The workgroup's block list in LDS (dynamic LDS sized by nb), one 16-bit word
// per entry (the block, or kNoBlock for an entry outside [0, nb)), so a stage
// reads its block from LDS instead of waiting on a scalar load from memory.
constexpr uint16_t kNoBlock = 0xFFFF;

__device__ __forceinline__ void stage_list(const int32_t* __restrict__ idx, int cnt, int nb, uint16_t* list_s) {
  for (int i = threadIdx.x; i < cnt; i += blockDim.x) {
    const int v = idx[i];
    list_s[i] = (v >= 0 && v < nb) ? (uint16_t)v : kNoBlock;
  }
}

// ---------------------------------------------------------------------------
// Key-to-query lists.  One workgroup per (32 key blocks, batch x head): it marks
// in an LDS bit matrix, for each of its key blocks J, the query blocks I whose
// list holds J (every list entry of the head, one wavefront per row), then each
// of its threads reads one J's row of bits in ascending I.  The result is the
// same whatever order the marks arrive in.
constexpr int kTrThreads = 1024;
constexpr int kTrJ = 32;          // key blocks per workgroup
constexpr int kTrMaxNb = 4096;

__global__ __launch_bounds__(kTrThreads) void transpose_lists_kernel(const int32_t* __restrict__ kv_count,
                                                                     const int32_t* __restrict__ kv_idx, int nb,
                                                                     int32_t* __restrict__ kvT_count,
                                                                     int32_t* __restrict__ kvT_idx) {
  __shared__ uint32_t bits[kTrJ][kTrMaxNb / 32];
  __shared__ uint16_t cnt_s[kTrMaxNb];
  const int J0 = blockIdx.x * kTrJ, bh = blockIdx.y, tid = threadIdx.x;
  const int words = (nb + 31) / 32;
  for (int i = tid; i < kTrJ * words; i += kTrThreads) bits[i / words][i % words] = 0u;
  for (int I = tid; I < nb; I += kTrThreads) cnt_s[I] = (uint16_t)min(max(kv_count[(int64_t)bh * nb + I], 0), nb);
  __syncthreads();
  // one wavefront per list row, its lanes over the row's entries
  const int32_t* irow = kv_idx + (int64_t)bh * nb * nb;
  const int wave = tid >> 6, lane = tid & 63;
  for (int I = wave; I < nb; I += kTrThreads / 64) {
    const int c = cnt_s[I];
    for (int pos = lane; pos < c; pos += 64) {
      const int J = irow[(int64_t)I * nb + pos] - J0;
      if (J >= 0 && J < kTrJ && J0 + J < nb) atomicOr(&bits[J][I >> 5], 1u << (I & 31));
    }
  }
  __syncthreads();
  if (tid < kTrJ && J0 + tid < nb) {
    const int J = J0 + tid;
    int32_t* out = kvT_idx + ((int64_t)bh * nb + J) * nb;
    int c = 0;
    for (int w = 0; w < words; ++w) {
      uint32_t m = bits[tid][w];
      while (m) {
        out[c++] = 32 * w + __builtin_ctz(m);
        m &= m - 1;
      }
    }
    kvT_count[(int64_t)bh * nb + J] = c;
  }
}

// ---------------------------------------------------------------------------
// Stages of 32 tokens in a ring of kRing buffers: the copies of stage
// u + kRing - 1 are issued right after the barrier that opens stage u (into the
// buffers stage u - 1 used), so kRing - 1 stages are in flight while stage u
// computes.  Stage u waits for its own copies only: every wavefront issues the
// same number of copies per stage, and vector-memory instructions retire in
// order.  The buffers are distinct arrays, each named at a fixed position of
// the kRing-times unrolled loop, so the compiler sees that no LDS read aliases
// a copy in flight.
constexpr int kKT = 32;
constexpr int kRing = 2;
constexpr int kDqKT = 64;   // dQ stages of 128-row workgroups: two 32-key tiles per barrier

// dQ.  Stage u: list entry u / kSubs, KT-key part u % kSubs, as 32-key tiles.
template <int D, int BLK>
__global__ __launch_bounds__(BLK / 32 * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_bwd_dq_kernel(
    const __bf16* __restrict__ q_r, const __bf16* __restrict__ k_r, const __bf16* __restrict__ v_r,
    const __bf16* __restrict__ o_r, const __bf16* __restrict__ do_r, const float* __restrict__ lse,
    const int32_t* __restrict__ kv_count, const int32_t* __restrict__ kv_idx,
    float* __restrict__ dq, float* __restrict__ dbuf, int Hh, int N, int Npad, int nb, float sl2, float scale) {
  constexpr int KT = BLK >= 128 ? kDqKT : kKT;   // 64-row workgroups keep 32-key stages (copy offsets)
  using C = BwdCfg<D, KT>;
  constexpr int W = BLK / 32, kSubs = BLK / KT;
  __shared__ __attribute__((aligned(1024))) char Ks0[C::kRowBytes];
  __shared__ __attribute__((aligned(1024))) char Vs0[C::kRowBytes];
  __shared__ __attribute__((aligned(1024))) char Ks1[C::kRowBytes];
  __shared__ __attribute__((aligned(1024))) char Vs1[C::kRowBytes];
  extern __shared__ uint16_t list_s[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int slot = xcd_remap(blockIdx.x, gridDim.x);
  const int I = slot % nb, bh = slot / nb;
  const int64_t rowbase = (int64_t)bh * Npad;
  const int q = I * BLK + wave * 32 + l32;
  const bool qok = q < N;

  // Q^T and dO^T operands (rows >= N zero), D = rowsum(dO o O), lse in log2 units.
  bf16x8_t qreg[D / 16], doreg[D / 16];
  float dpart = 0.f;
  {
    const int64_t off = (rowbase + (qok ? q : 0)) * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(q_r + off + 16 * kk);
      bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(do_r + off + 16 * kk);
      const bf16x8_t o = *reinterpret_cast<const bf16x8_t*>(o_r + off + 16 * kk);
      if (!qok) {
        a = bf16x8_t{};
        b = bf16x8_t{};
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) dpart += (float)b[e] * (float)o[e];
      qreg[kk] = a;
      doreg[kk] = b;
    }
  }
  const float Dq = qok ? sum_halves(dpart) : 0.f;
  const float lse2 = qok ? lse[rowbase + q] * kLog2e : INFINITY;   // +inf: P = 0 for rows >= N
  if (qok && g == 0) dbuf[rowbase + q] = Dq;

  f32x16_t acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16_t{};

  int cnt = __builtin_amdgcn_readfirstlane(kv_count[(int64_t)bh * nb + I]);
  cnt = cnt < 0 ? 0 : (cnt > nb ? nb : cnt);
  const int32_t* idx = kv_idx + ((int64_t)bh * nb + I) * nb;
  const auto rk = make_rsrc(k_r + rowbase * D, (uint32_t)Npad * (uint32_t)(D * 2));
  const auto rv = make_rsrc(v_r + rowbase * D, (uint32_t)Npad * (uint32_t)(D * 2));
  StageCopies<D, BLK, W, KT> cp;
  cp.init(wave, lane);
  stage_list(idx, cnt, nb, list_s);
  __syncthreads();

  const int U = cnt * kSubs;
  auto block_of = [&](int u) { return __builtin_amdgcn_readfirstlane((int)list_s[u / kSubs]); };
  // An invalid entry copies block 0 and computes nothing, as the forward skips it.
  auto issue = [&](int u, char* kb, char* vb) {
    const int J0 = block_of(u), h = u % kSubs;
    const int J = J0 == kNoBlock ? 0 : J0;
    const int key0 = J * BLK + h * KT;
    cp.rows(rk, (uint32_t)key0 * (uint32_t)(D * 2), kb);
    cp.rows(rv, (uint32_t)key0 * (uint32_t)(D * 2), vb);
  };
  auto compute = [&](int u, const char* kb_stage, const char* vb_stage) {
    const int J = block_of(u), h = u % kSubs;
    if (J == kNoBlock) return;
#pragma unroll
    for (int t = 0; t < KT / 32; ++t) {
    const char* kb = kb_stage + 32 * t * C::kRowStride;
    const char* vb = vb_stage + 32 * t * C::kRowStride;
    const int key0 = J * BLK + h * KT + 32 * t;
    // dP^T accumulates onto -D (each lane's column is one query), so it ends as dP^T - D
    f32x16_t S = f32x16_t{}, dP;
#pragma unroll
    for (int v = 0; v < 16; ++v) dP[v] = -Dq;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      S = mfma(read_rows<C>(kb, l32, g, kk), qreg[kk], S);
      dP = mfma(read_rows<C>(vb, l32, g, kk), doreg[kk], dP);
    }
    // dS^T = P^T (dP^T - D); keys >= N have P = 0.  Only a tile that runs
    // past N takes the masked form (a uniform branch).
    if (key0 + 32 > N) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float p = fast_exp2(__builtin_fmaf(S[v], sl2, -lse2));
        if (key0 + stage_row(acc_row(v, g)) >= N) p = 0.f;
        S[v] = p * dP[v];
      }
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) S[v] = fast_exp2(__builtin_fmaf(S[v], sl2, -lse2)) * dP[v];
    }
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const bf16x8_t bq = pack_half(S, st);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) acc[dt] = mfma(read_rows_tr<C>(kb, lane, dt, st), bq, acc[dt]);
    }
    }
  };
  constexpr int kCps = 2 * StageCopies<D, BLK, W, KT>::kRowPer;   // copies per stage and wavefront
  auto stage = [&](int u, const char* kb, const char* vb, char* nk, char* nv) {
    if (u + kRing - 2 < U) wait_vm<(kRing - 2) * kCps>();
    else wait_dma();
    __syncthreads();   // stage u landed; every wave is done with stage u - 1's buffers
    if (u + kRing - 1 < U) issue(u + kRing - 1, nk, nv);
    compute(u, kb, vb);
  };
  static_assert(kRing == 2, "the unrolled ring below names two buffers");
  if (U > 0) issue(0, Ks0, Vs0);
  for (int u = 0; u < U; u += kRing) {
    stage(u, Ks0, Vs0, Ks1, Vs1);
    if (u + 1 < U) stage(u + 1, Ks1, Vs1, Ks0, Vs0);
  }

  // lane (l32, g) holds dQ^T rows 32 dt + acc_row(v, g) of query q
  if (q < Npad) {
    float* out = dq + (rowbase + q) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 w = qok ? make_float4(acc[dt][4 * i] * scale, acc[dt][4 * i + 1] * scale,
                                           acc[dt][4 * i + 2] * scale, acc[dt][4 * i + 3] * scale)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
        *reinterpret_cast<float4*>(out + 32 * dt + 8 * i + 4 * g) = w;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dK, dV.  Stage u of the key block's query list: entry u / kSubs, KT-query
// part u % kSubs, as 32-query tiles computed one after the other (the score
// registers serve both).
template <int D, int BLK>
__global__ __launch_bounds__(BLK / 32 * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_bwd_dkdv_kernel(
    const __bf16* __restrict__ q_r, const __bf16* __restrict__ k_r, const __bf16* __restrict__ v_r,
    const __bf16* __restrict__ do_r, const float* __restrict__ lse, const float* __restrict__ dbuf,
    const int32_t* __restrict__ kvT_count,
    const int32_t* __restrict__ kvT_idx, float* __restrict__ dk, float* __restrict__ dv, int Hh, int N, int Npad,
    int nb, float sl2, float scale) {
  constexpr int KT = BLK >= 128 ? kDqKT : kKT;   // as dQ
  using C = BwdCfg<D, KT>;
  constexpr int W = BLK / 32, kSubs = BLK / KT;
  __shared__ __attribute__((aligned(1024))) char Qs0[C::kRowBytes];
  __shared__ __attribute__((aligned(1024))) char dOs0[C::kRowBytes];
  __shared__ __attribute__((aligned(1024))) char Qs1[C::kRowBytes];
  __shared__ __attribute__((aligned(1024))) char dOs1[C::kRowBytes];
  __shared__ __attribute__((aligned(16))) float ld_s[kRing][2 * KT];   // per buffer set: lse (log2), then D
  extern __shared__ uint16_t list_s[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int slot = xcd_remap(blockIdx.x, gridDim.x);
  const int J = slot % nb, bh = slot / nb;
  const int64_t rowbase = (int64_t)bh * Npad;
  const int key = J * BLK + wave * 32 + l32;
  const bool kok = key < N;

  // K^T and V^T operands of this wavefront's 32 keys (keys >= N zero).
  bf16x8_t kreg[D / 16], vreg[D / 16];
  {
    const int64_t off = (rowbase + (kok ? key : 0)) * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(k_r + off + 16 * kk);
      const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(v_r + off + 16 * kk);
      kreg[kk] = kok ? a : bf16x8_t{};
      vreg[kk] = kok ? b : bf16x8_t{};
    }
  }
  f32x16_t dka[D / 32], dva[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    dka[dt] = f32x16_t{};
    dva[dt] = f32x16_t{};
  }

  int cnt = __builtin_amdgcn_readfirstlane(kvT_count[(int64_t)bh * nb + J]);
  cnt = cnt < 0 ? 0 : (cnt > nb ? nb : cnt);
  const int32_t* idx = kvT_idx + ((int64_t)bh * nb + J) * nb;
  const auto rq = make_rsrc(q_r + rowbase * D, (uint32_t)Npad * (uint32_t)(D * 2));
  const auto rdo = make_rsrc(do_r + rowbase * D, (uint32_t)Npad * (uint32_t)(D * 2));
  StageCopies<D, BLK, W, KT> cp;
  cp.init(wave, lane);
  stage_list(idx, cnt, nb, list_s);
  __syncthreads();

  const int U = cnt * kSubs;
  auto block_of = [&](int u) { return __builtin_amdgcn_readfirstlane((int)list_s[u / kSubs]); };
  // The stage's lse and D (one query per thread of the first KT) are loaded
  // into registers with its copies and written to LDS only when the stage
  // opens, after the wait for its copies, so no wave stalls on them at issue.
  // An invalid entry copies block 0 and computes nothing.
  float l_in = 0.f, d_in = 0.f;
  bool ok_in = false;
  auto issue = [&](int u, char* qb, char* ob) {
    const int I0 = block_of(u), h = u % kSubs;
    const int I = I0 == kNoBlock ? 0 : I0;
    const int qs0 = I * BLK + h * KT;
    if (threadIdx.x < KT) {
      const int qq = qs0 + threadIdx.x;
      ok_in = qq < N;
      if (ok_in) {
        l_in = lse[rowbase + qq];
        d_in = dbuf[rowbase + qq];
      }
    }
    cp.rows(rq, (uint32_t)qs0 * (uint32_t)(D * 2), qb);
    cp.rows(rdo, (uint32_t)qs0 * (uint32_t)(D * 2), ob);
  };
  auto compute = [&](int u, const char* qb_stage, const char* ob_stage, const float* ls_stage) {
    const int I = block_of(u);
    if (I == kNoBlock) return;
#pragma unroll
    for (int t = 0; t < KT / 32; ++t) {
    const char* qb = qb_stage + 32 * t * C::kRowStride;
    const char* ob = ob_stage + 32 * t * C::kRowStride;
    const float* ls = ls_stage + 32 * t;   // lse of the tile; its D at ls + KT
    f32x16_t S = f32x16_t{}, dP = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      S = mfma(read_rows<C>(qb, l32, g, kk), kreg[kk], S);
      dP = mfma(read_rows<C>(ob, l32, g, kk), vreg[kk], dP);
    }
    // rows of S are tile rows acc_row(v, g): lse and D from LDS, 4 at a time
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int r0 = 8 * a + 4 * g;
      const float4 l4 = *reinterpret_cast<const float4*>(ls + r0);
      const float4 d4 = *reinterpret_cast<const float4*>(ls + KT + r0);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
      const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int v = 4 * a + j;
        const float p = fast_exp2(__builtin_fmaf(S[v], sl2, -lv[j]));
        S[v] = p;
        dP[v] = p * (dP[v] - dv4[j]);
      }
    }
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const bf16x8_t bp = pack_half(S, st), bs = pack_half(dP, st);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        dva[dt] = mfma(read_rows_tr<C>(ob, lane, dt, st), bp, dva[dt]);
        dka[dt] = mfma(read_rows_tr<C>(qb, lane, dt, st), bs, dka[dt]);
      }
    }
    }
  };
  // With one stage in flight, the wait that opens stage u covers its lse / D
  // loads (issued before its copies) as well as its copies.
  static_assert(kRing == 2, "the lse / D registers and the unrolled ring below hold one stage in flight");
  auto stage = [&](int u, const char* qb, const char* ob, float* ls, char* nq, char* no) {
    wait_dma();
    if (threadIdx.x < KT) {   // at its tile row, the order of the accumulator rows
      const int m = (threadIdx.x & ~31) | tile_row(threadIdx.x & 31);
      ls[m] = ok_in ? l_in * kLog2e : INFINITY;   // +inf: P = 0 for rows >= N
      ls[KT + m] = ok_in ? d_in : 0.f;
    }
    __syncthreads();   // stage u landed, its lse / D are in LDS; stage u - 1's buffers are free
    if (u + 1 < U) issue(u + 1, nq, no);
    compute(u, qb, ob, ls);
  };
  if (U > 0) issue(0, Qs0, dOs0);
  for (int u = 0; u < U; u += kRing) {
    stage(u, Qs0, dOs0, ld_s[0], Qs1, dOs1);
    if (u + 1 < U) stage(u + 1, Qs1, dOs1, ld_s[1], Qs0, dOs0);
  }

  // lane (l32, g) holds rows 32 dt + acc_row(v, g) of dK^T, dV^T for its key
  if (key < Npad) {
    float* ko = dk + (rowbase + key) * D;
    float* vo = dv + (rowbase + key) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 a = kok ? make_float4(dka[dt][4 * i] * scale, dka[dt][4 * i + 1] * scale,
                                           dka[dt][4 * i + 2] * scale, dka[dt][4 * i + 3] * scale)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
        const float4 b = kok ? make_float4(dva[dt][4 * i], dva[dt][4 * i + 1], dva[dt][4 * i + 2], dva[dt][4 * i + 3])
                             : make_float4(0.f, 0.f, 0.f, 0.f);
        *reinterpret_cast<float4*>(ko + 32 * dt + 8 * i + 4 * g) = a;
        *reinterpret_cast<float4*>(vo + 32 * dt + 8 * i + 4 * g) = b;
      }
    }
  }
}

template <int D, int BLK>
hipError_t launch_bwd_db(const AttnBwdArgs& a) {
  const int BH = a.B * a.Hh;
  float* dbuf = reinterpret_cast<float*>(a.workspace);
  const float sl2 = a.scale * kLog2e;
  const unsigned grid = (unsigned)(BH * a.nb);
  const size_t list_bytes = ((size_t)a.nb * 2 + 15) / 16 * 16;
  hipLaunchKernelGGL((attn_bwd_dq_kernel<D, BLK>), dim3(grid), dim3(BLK / 32 * 64), list_bytes, a.stream,
                     (const __bf16*)a.q_r, (const __bf16*)a.k_r, (const __bf16*)a.v_r, (const __bf16*)a.o_r,
                     (const __bf16*)a.do_r, a.lse, a.kv_count, a.kv_idx, a.dq, dbuf, a.Hh, a.N, a.Npad, a.nb, sl2,
                     a.scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, BLK>), dim3(grid), dim3(BLK / 32 * 64), list_bytes, a.stream,
                     (const __bf16*)a.q_r, (const __bf16*)a.k_r, (const __bf16*)a.v_r, (const __bf16*)a.do_r, a.lse,
                     (const float*)dbuf, a.kvT_count, a.kvT_idx, a.dk, a.dv, a.Hh, a.N, a.Npad, a.nb, sl2, a.scale);
  return hipGetLastError();
}

}  // namespace

size_t attn_bwd_workspace_bytes(int B, int Hh, int Npad, int d) {
  (void)d;
  return (size_t)((int64_t)B * Hh * Npad * 4);   // D = rowsum(dO o O) per row
}

hipError_t launch_transpose_lists(const TransposeListsArgs& a) {
  hipLaunchKernelGGL(transpose_lists_kernel, dim3((unsigned)((a.nb + kTrJ - 1) / kTrJ), (unsigned)(a.B * a.Hh)),
                     dim3(kTrThreads), 0, a.stream, a.kv_count, a.kv_idx, a.nb, a.kvT_count, a.kvT_idx);
  return hipGetLastError();
}

hipError_t launch_attn_bwd(const AttnBwdArgs& a) {
  if (a.d == 64) return a.b == 64 ? launch_bwd_db<64, 64>(a) : launch_bwd_db<64, 128>(a);
  return a.b == 64 ? launch_bwd_db<128, 64>(a) : launch_bwd_db<128, 128>(a);
}

}  // namespace dbs
