// gfx950 (CDNA4) kernels of the weight-only quantized GEMM and the qgemm_run entry point.
//
//   out[M, N] = A[M, K] . dequant(W)[K, N]   (times alpha for FP8 / FP4)
//
// Both kernels feed v_mfma_f32_16x16x32_{f16,bf16}.  Operand fragment of that MFMA, per
// 64-lane wavefront: lane l supplies row (A) or column (B) l & 15 and the eight
// consecutive K values 8 (l >> 4) .. 8 (l >> 4) + 7 of the 32-wide K step; the 16x16 fp32
// result sits in lane l as rows 4 (l >> 4) .. +3 of column l & 15.  The packed weight
// layout puts exactly one such B fragment per K step in each lane's 16-byte chunk, so a
// wavefront turns one coalesced 1 KiB load into MFMA operands with register-only
// unpacking: the dequantize-in-registers pattern of Low Bit Triton Kernels (GPU MODE
// lecture 034, core pattern), without the shared-memory re-layout that the Bitblas
// lecture 033 (layout section) measures as the dominant cost when fragments mismatch.
//
// Dequantization (value semantics of each format):
//   INT4: the nibble (stored value + 8) is OR-ed into the mantissa of an fp16 constant
//         (0x6400 = 1024 for a low nibble, 0x5400 = 64 for a nibble at bit 4), the
//         constant plus 8 is subtracted (exact), and the result is multiplied by the fp16
//         group scale: RNE_fp16((nibble - 8) * s), the 16-bit tile of the gemlite snippet.
//   FP8 : v_cvt_scalef32_pk_bf16_fp8 with scale 1.0 (OCP e4m3, exact in bf16); the
//         per-tensor alpha multiplies the fp32 accumulator in the epilogue (FlashInfer
//         PR #7495 analysis, introduction).
//   FP4 : v_cvt_scalef32_pk_f32_fp4 with scale 1.0, times the e4m3 block scale in fp32
//         (exact), then RNE to bf16 (exact).  The scale operand of the scalef32 converts
//         only honours its exponent, so it cannot carry an e4m3 block scale.
//
// Split-K (when the output tiles alone cannot fill 256 compute units): each K slice writes
// an fp32 partial tile to the workspace, then takes a ticket; the workgroup that draws the
// last ticket sums all partials in slice order (bitwise deterministic, whichever slice
// arrives last) and resets the ticket.  No workgroup ever waits for another, so nothing
// assumes co-residency (FlashInfer PR #7495 analysis, section 3(d), describes the deadlock
// that assumption caused and the slice-ordered sum that keeps results bitwise identical).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "qgemm_internal.h"

namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

struct KArgs {
  const uint16_t* A;          // [M][K] 16-bit
  const uint8_t* W;           // packed weights
  const void* S;              // packed scales (INT4: fp16, FP4: e4m3 bytes)
  const float* alpha;         // FP8 / FP4: device scalar
  void* out;                  // [M][N]
  unsigned* counters;         // split-K tickets, one per tile
  float* partials;            // split-K partial tiles
  int M, N, K;
  int out_dtype;
  int splits, kb_per_split;
  int tiles_n;                // prefill: output tiles along N
};

// ----------------------------------------------------------------------------- dequant
// (a & m) | o in one VALU op.  The compiler splits it into AND + OR because the two
// constants cannot both be instruction operands; as VGPR operands they can.
__device__ __forceinline__ unsigned and_or(unsigned a, unsigned m, unsigned o) {
  unsigned r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(o));
  return r;
}

__device__ __forceinline__ u32x4 dq_int4(unsigned w, unsigned s2) {
  const unsigned hi = w >> 8;
  const unsigned p0 = and_or(w, 0x000F000Fu, 0x64006400u);    // k slots j0, j1: 1024 + nibble
  const unsigned p1 = and_or(w, 0x00F000F0u, 0x54005400u);    // j2, j3: 64 + nibble
  const unsigned p2 = and_or(hi, 0x000F000Fu, 0x64006400u);   // j4, j5
  const unsigned p3 = and_or(hi, 0x00F000F0u, 0x54005400u);   // j6, j7
  const f16x2 s = __builtin_bit_cast(f16x2, s2);
  const f16x2 big = {(_Float16)1032.0f, (_Float16)1032.0f};
  const f16x2 small = {(_Float16)72.0f, (_Float16)72.0f};
  const f16x2 h0 = (__builtin_bit_cast(f16x2, p0) - big) * s;
  const f16x2 h1 = (__builtin_bit_cast(f16x2, p1) - small) * s;
  const f16x2 h2 = (__builtin_bit_cast(f16x2, p2) - big) * s;
  const f16x2 h3 = (__builtin_bit_cast(f16x2, p3) - small) * s;
  return u32x4{__builtin_bit_cast(unsigned, h0), __builtin_bit_cast(unsigned, h1),
               __builtin_bit_cast(unsigned, h2), __builtin_bit_cast(unsigned, h3)};
}

__device__ __forceinline__ u32x4 dq_fp8(unsigned lo, unsigned hi) {
  return u32x4{__builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false)),
               __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true)),
               __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false)),
               __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true))};
}

__device__ __forceinline__ unsigned pk_bf16(f32x2 f, float s) {
  bf16x2 r;
  r[0] = (__bf16)(f[0] * s);
  r[1] = (__bf16)(f[1] * s);
  return __builtin_bit_cast(unsigned, r);
}

__device__ __forceinline__ u32x4 dq_fp4(unsigned w, float s) {
  return u32x4{pk_bf16(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0), s),
               pk_bf16(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1), s),
               pk_bf16(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2), s),
               pk_bf16(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3), s)};
}

// Four e4m3 block-scale bytes -> fp32 (exact through the verified e4m3 -> bf16 convert).
__device__ __forceinline__ void fp4_scales(unsigned sw, float (&s)[4]) {
  const unsigned a = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(sw, 1.0f, false));
  const unsigned b = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(sw, 1.0f, true));
  s[0] = __builtin_bit_cast(float, a << 16);
  s[1] = __builtin_bit_cast(float, a & 0xFFFF0000u);
  s[2] = __builtin_bit_cast(float, b << 16);
  s[3] = __builtin_bit_cast(float, b & 0xFFFF0000u);
}

template <int FMT>
__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (FMT == qgemm::FMT_INT4)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Weights + scales of one (column block, 128-wide k block) as seen by one lane.  Scales
// are kept as loaded (raw bits) and expanded only where they are used, so that nothing
// consumes a load before the MFMA loop does (a consumer forces a wait for every load
// issued before it).
template <int FMT>
struct WFrag {
  u32x4 w[FMT == qgemm::FMT_FP8 ? 2 : 1];
  unsigned s[2];    // INT4: 1, 2 or 4 fp16 scales (G = 128|256, 64, 32); FP4: 4 e4m3 bytes
};

// G is the INT4 group size (a template parameter, so the scale load has no branches:
// a branch around a load ends in a wait for every outstanding load); 0 for FP8 / FP4.
// STREAM marks weights read once (decode: non-temporal loads keep them out of the way in
// the caches); prefill re-reads each weight fragment once per row tile and caches it.
template <bool STREAM>
__device__ __forceinline__ u32x4 wload(const u32x4* p) {
  if constexpr (STREAM) return __builtin_nontemporal_load(p);
  else return *p;
}

template <int FMT, int G, bool STREAM = true>
__device__ __forceinline__ void load_wfrag(const KArgs& a, int nb, int kb, int lane, WFrag<FMT>& f) {
  const int KB = a.K >> 7;
  if constexpr (FMT == qgemm::FMT_FP8) {
    const u32x4* p = reinterpret_cast<const u32x4*>(a.W + ((size_t)nb * (KB * 2) + 2 * kb) * 1024) + lane;
    f.w[0] = wload<STREAM>(p);
    f.w[1] = wload<STREAM>(p + 64);
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(a.W + ((size_t)nb * KB + kb) * 1024) + lane;
    f.w[0] = wload<STREAM>(p);
  }
  if constexpr (FMT == qgemm::FMT_INT4) {
    const uint16_t* S = static_cast<const uint16_t*>(a.S);
    const int c = lane & 15;
    if constexpr (G <= 128) {
      constexpr int T = 128 / G;
      const size_t base = ((size_t)nb * KB + kb) * 16 * T + (size_t)c * T;
      if constexpr (T == 4) {
        const u32x2 x = *reinterpret_cast<const u32x2*>(S + base);
        f.s[0] = x[0];
        f.s[1] = x[1];
      } else if constexpr (T == 2) {
        f.s[0] = *reinterpret_cast<const unsigned*>(S + base);
      } else {
        f.s[0] = S[base];
      }
    } else {   // G == 256: one scale per two k blocks
      f.s[0] = S[((size_t)nb * (KB >> 1) + (kb >> 1)) * 16 + c];
    }
  } else if constexpr (FMT == qgemm::FMT_FP4) {
    const uint8_t* S = static_cast<const uint8_t*>(a.S);
    f.s[0] = *reinterpret_cast<const unsigned*>(S + (((size_t)nb * KB + kb) * 16 + (lane & 15)) * 8 + 4 * (lane >> 5));
  }
}

// fp16 scale of K step t, duplicated into both halves (INT4).
template <int G>
__device__ __forceinline__ unsigned int4_scale_pair(const unsigned (&s)[2], int t) {
  unsigned h;
  if constexpr (G == 32) h = (t & 1) ? (s[t >> 1] >> 16) : (s[t >> 1] & 0xFFFFu);
  else if constexpr (G == 64) h = (t >> 1) ? (s[0] >> 16) : (s[0] & 0xFFFFu);
  else h = s[0] & 0xFFFFu;
  return h | (h << 16);
}

// The B operand (dequantized weights) of K step t.
template <int FMT, int G>
__device__ __forceinline__ u32x4 bfrag(const WFrag<FMT>& f, int t, const float (&fs)[4]) {
  if constexpr (FMT == qgemm::FMT_INT4) {
    return dq_int4(f.w[0][t], int4_scale_pair<G>(f.s, t));
  } else if constexpr (FMT == qgemm::FMT_FP8) {
    return dq_fp8(f.w[t >> 1][2 * (t & 1)], f.w[t >> 1][2 * (t & 1) + 1]);
  } else {
    return dq_fp4(f.w[0][t], fs[t]);
  }
}

// ----------------------------------------------------------------------------- epilogue
__device__ __forceinline__ void store_out(const KArgs& a, int m, int n, float v) {
  const size_t i = (size_t)m * a.N + n;
  if (a.out_dtype == QGEMM_DT_F32) {
    static_cast<float*>(a.out)[i] = v;
  } else if (a.out_dtype == QGEMM_DT_F16) {
    static_cast<_Float16*>(a.out)[i] = (_Float16)v;
  } else {
    static_cast<__bf16*>(a.out)[i] = (__bf16)v;
  }
}

// Split-K hand-off.  Every thread of the workgroup calls this with its NF fragments
// (`active` false for threads that hold none).  Returns true in the workgroup that must
// write the output; then `v` holds the slice-ordered sum of all partials.
//
// Visibility across XCDs without L2 maintenance: partials are written with device-scope
// stores (write-through past the XCD-private L2), every thread waits for its stores to
// be acknowledged before the barrier that precedes the ticket, and the last workgroup
// reads the partials back with device-scope loads.  A device-scope fence would instead
// write back and invalidate the whole XCD L2 in every workgroup.
__device__ __forceinline__ void store_dev(float* p, f32x4 v) {
#pragma unroll
  for (int r = 0; r < 4; ++r) __hip_atomic_store(p + r, v[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ f32x4 load_dev(const float* p) {
  f32x4 v;
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = __hip_atomic_load(p + r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return v;
}

template <int NF, int NT = 256>
__device__ bool splitk_finish(const KArgs& a, int tile, int split, int tile_elems, bool active, f32x4 (&v)[NF]) {
  __shared__ int s_last;
  const int tid = threadIdx.x;
  float* base = a.partials + (size_t)tile * a.splits * tile_elems;
  if (active) {
    float* mine = base + (size_t)split * tile_elems;
#pragma unroll
    for (int f = 0; f < NF; ++f) store_dev(mine + 4 * (f * NT + tid), v[f]);
  }
  __builtin_amdgcn_s_waitcnt(0);     // this thread's partial stores are complete
  __syncthreads();
  if (tid == 0) {
    const unsigned ticket = __hip_atomic_fetch_add(a.counters + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = ticket == (unsigned)(a.splits - 1);
  }
  __syncthreads();
  if (!s_last) return false;
  if (active) {
#pragma unroll
    for (int f = 0; f < NF; ++f) v[f] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < a.splits; ++s) {
      const float* p = base + (size_t)s * tile_elems;
#pragma unroll
      for (int f = 0; f < NF; ++f) v[f] += load_dev(p + 4 * (f * NT + tid));
    }
  }
  if (tid == 0) __hip_atomic_store(a.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// ============================================================================= decode
// M <= 16.  Workgroup = NW wavefronts; it owns CB column blocks (16 columns each) and one
// K slice (normally all of K: a split-K hand-off costs three dependent memory round trips,
// more than a whole small GEMM).  Wavefront w owns a contiguous share of the slice's k
// blocks, streamed in runs of up to KPW blocks: all weight and scale loads of a run are
// issued before any is consumed, and the k blocks are then consumed in load order, so each
// waits only for its own data.
// A fragments: with ASTAGE (small M) every thread first loads distinct 16-byte chunks of the
// A slice (M rows, at most 32 KiB) into LDS, because a wave's fragment loads would otherwise
// fetch each A value 16 times; otherwise (rows all distinct) each wavefront loads its
// fragments from global memory before the run's weights.  Rows at or beyond M read row
// M - 1 (MFMA output row m depends on A row m only; rows >= M are never stored).
// Control flow is wavefront-uniform and loads are clamped rather than predicated (the
// compiler waits for every outstanding load at the end of a branch that contains one).
// Each wavefront keeps two accumulators per column block (even / odd K steps) to halve the
// MFMA dependency chain; the NW wavefront tiles are summed through LDS in wave order.
constexpr int DEC_A_CHUNKS = 2048;                  // 32 KiB of staged A per workgroup
constexpr bool DEC_ACC2 = true;                     // two accumulators per column block

template <int FMT, int G, int CB, int KPW, int NW, bool ASTAGE>
__global__ __launch_bounds__(64 * NW) void qgemm_decode(KArgs a) {
  constexpr int NT = 64 * NW;
  constexpr int SCH = ASTAGE ? DEC_A_CHUNKS / NT : 1;   // staging chunks per thread
  __shared__ __attribute__((aligned(16))) uint16_t a_lds[ASTAGE ? DEC_A_CHUNKS * 8 + 16 * 8 : 8];
  __shared__ f32x4 red[NW][CB][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = blockIdx.x, split = blockIdx.y;
  const int KB = a.K >> 7, NB = a.N >> 4;
  const int kb_begin = split * a.kb_per_split;
  const int kb_end = min(KB, kb_begin + a.kb_per_split);
  const int nb0 = group * CB;
  const int kslice = (kb_end - kb_begin) * 128;     // halves per A row in this slice
  const int lda = kslice + 8;                        // LDS row stride (halves)
  // this wavefront's contiguous share of the slice
  const int share = (kb_end - kb_begin + NW - 1) / NW;
  const int w_begin = min(kb_end, kb_begin + wave * share);
  const int w_end = min(kb_end, w_begin + share);
  const int row = min(lane & 15, a.M - 1);

  int soff[SCH];
  u32x4 stage[SCH];
  if constexpr (ASTAGE) {
    const int cpr = kslice >> 3;                     // 16-byte chunks per row
    const int chunks = a.M * cpr;                    // <= DEC_A_CHUNKS by the launch plan
    const float inv_cpr = 1.0f / (float)cpr;
#pragma unroll
    for (int i = 0; i < SCH; ++i) {                  // no branch around a load: surplus threads re-load the last chunk
      const int q = tid + NT * i;
      const int qq = min(q, chunks - 1);
      const int r = (int)(((float)qq + 0.5f) * inv_cpr);
      const int c8 = qq - r * cpr;
      stage[i] = *reinterpret_cast<const u32x4*>(a.A + (size_t)r * a.K + (size_t)kb_begin * 128 + 8 * c8);
      soff[i] = q < chunks ? r * lda + 8 * c8 : -1;
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  f32x4 acc[CB][2];
#pragma unroll
  for (int c = 0; c < CB; ++c) acc[c][0] = acc[c][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint16_t* arow_g = a.A + (size_t)row * a.K + 8 * (lane >> 4);
  const uint16_t* arow_l = a_lds + row * lda + 8 * (lane >> 4);
  const int last = max(w_end - 1, w_begin);          // clamp target (valid even for an empty share)
  const int kb_cap = min(last, KB - 1);

  // one run: loads first (A fragments, then weights and scales), then the k blocks in
  // load order, each waiting only for its own data
  auto run_loads = [&](int run, u32x4 (&afr)[ASTAGE ? 1 : KPW][4], WFrag<FMT> (&wf)[KPW][CB]) {
    if constexpr (!ASTAGE) {
#pragma unroll
      for (int u = 0; u < KPW; ++u) {
        const u32x4* ap = reinterpret_cast<const u32x4*>(arow_g + (size_t)min(run + u, kb_cap) * 128);
#pragma unroll
        for (int t = 0; t < 4; ++t) afr[u][t] = ap[4 * t];
      }
    }
#pragma unroll
    for (int u = 0; u < KPW; ++u)
#pragma unroll
      for (int c = 0; c < CB; ++c) load_wfrag<FMT, G>(a, min(nb0 + c, NB - 1), min(run + u, kb_cap), lane, wf[u][c]);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto run_compute = [&](int run, const u32x4 (&afr)[ASTAGE ? 1 : KPW][4], const WFrag<FMT> (&wf)[KPW][CB]) {
#pragma unroll
    for (int u = 0; u < KPW; ++u) {
      if (run + u < w_end) {
        u32x4 al[4];
        if constexpr (ASTAGE) {
          const uint16_t* ap = arow_l + (run + u - kb_begin) * 128;
#pragma unroll
          for (int t = 0; t < 4; ++t) al[t] = *reinterpret_cast<const u32x4*>(ap + 32 * t);
        }
#pragma unroll
        for (int c = 0; c < CB; ++c) {
          float fs[4] = {0.f, 0.f, 0.f, 0.f};
          if constexpr (FMT == qgemm::FMT_FP4) fp4_scales(wf[u][c].s[0], fs);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const u32x4 av = ASTAGE ? al[t] : afr[ASTAGE ? 0 : u][t];
            acc[c][DEC_ACC2 ? (t & 1) : 0] = mfma<FMT>(av, bfrag<FMT, G>(wf[u][c], t, fs), acc[c][DEC_ACC2 ? (t & 1) : 0]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  {   // first run: every wavefront, with or without k blocks, also stages A and syncs
    u32x4 afr[ASTAGE ? 1 : KPW][4];
    WFrag<FMT> wf[KPW][CB];
    run_loads(w_begin, afr, wf);
    if constexpr (ASTAGE) {
#pragma unroll
      for (int i = 0; i < SCH; ++i)
        if (soff[i] >= 0) *reinterpret_cast<u32x4*>(a_lds + soff[i]) = stage[i];
      __syncthreads();
    }
    if (w_begin < w_end) run_compute(w_begin, afr, wf);
  }
  for (int run = w_begin + KPW; run < w_end; run += KPW) {
    u32x4 afr[ASTAGE ? 1 : KPW][4];
    WFrag<FMT> wf[KPW][CB];
    run_loads(run, afr, wf);
    run_compute(run, afr, wf);
  }

#pragma unroll
  for (int c = 0; c < CB; ++c) red[wave][c][lane] = DEC_ACC2 ? acc[c][0] + acc[c][1] : acc[c][0];
  __syncthreads();
  const bool active = tid < CB * 64;
  const int c = tid >> 6, ln = tid & 63;
  f32x4 v[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
  if (active) {
    v[0] = red[0][c][ln];
#pragma unroll
    for (int w = 1; w < NW; ++w) v[0] += red[w][c][ln];
  }
  if (a.splits > 1) {
    if (!splitk_finish<1, NT>(a, group, split, CB * 256, active, v)) return;
  }
  if (!active || nb0 + c >= NB) return;
  const float alpha = FMT == qgemm::FMT_INT4 ? 1.0f : *a.alpha;
  const int n = (nb0 + c) * 16 + (ln & 15);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * (ln >> 4) + r;
    if (m < a.M) store_out(a, m, n, FMT == qgemm::FMT_INT4 ? v[0][r] : v[0][r] * alpha);
  }
}

// ============================================================================= prefill
// Workgroup = WGM x WGN wavefronts; each wavefront owns TM x TN MFMA tiles (16 x 16), so
// the workgroup tile is (16 WGM TM) x (16 WGN TN); one 128-wide k block per step.
//
// A goes from HBM straight into LDS (buffer loads with the LDS-destination bit: no VGPR
// staging), double-buffered in two separate arrays so that the compiler can tell the
// buffer being read from the one being filled.  A DMA load writes its 64 lanes' 16 bytes
// contiguously, so LDS rows cannot be padded; instead the 16-byte chunk c of tile row r
// is stored at chunk position c ^ (r & 15).  The MFMA A-fragment read (lane l: row l & 15,
// chunk 4t + l / 16) then touches 16 distinct positions per 16 lanes: no bank conflicts.
// The buffer resource covers the tile's valid rows only and the row sits in the range-
// checked per-lane offset (the k block in the scalar offset never leaves its row), so rows
// at or beyond M read as zero (and are never stored).
//
// Each wavefront loads its own packed weight fragments into registers (one k block
// ahead) and dequantizes each once per K step, reusing it for its TM row tiles; the
// dequantization of K step t + 1 is issued with the MFMAs of step t.  A fragments are
// read from LDS in units of RU row tiles, LA units ahead of the MFMAs that consume them.
// One barrier per k block: step k issues the weight loads of block k + 1, computes block k
// while spreading the A DMA loads of block k + 1 over its first read units, waits for its
// own loads and meets the other wavefronts at the barrier.  The
// loop is unrolled by two so buffers and register sets alternate without copies; every
// load is unconditional (the last step re-loads its own block, never used) and
// sched_barrier pins the phase order (a load under a branch, or a consumer scheduled
// early, would make the wavefront wait for all outstanding loads).
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Output tile of workgroup b.  Workgroups are dispatched to the eight XCDs (each with its
// own L2) round-robin by id, so the id is first mapped to a position such that each XCD
// owns one contiguous range of positions; positions then walk the tile grid in bands of
// GM tile rows, column by column, so that the tiles an XCD runs at the same time share
// few A row blocks and weight column blocks.
#ifndef QGEMM_PF_GM
#define QGEMM_PF_GM 4
#endif
#ifndef QGEMM_PF_DS
#define QGEMM_PF_DS 1
#endif
__device__ __forceinline__ void pf_tile_of(int b, int tiles, int tiles_n, int& tm, int& tn) {
  const int x = b & 7, slot = b >> 3, q = tiles >> 3, r = tiles & 7;
  const int L = x < r ? x * (q + 1) + slot : r * (q + 1) + (x - r) * q + slot;
  const int tiles_m = tiles / tiles_n;
  const int band = L / (QGEMM_PF_GM * tiles_n), first = band * QGEMM_PF_GM;
  const int gm = min(QGEMM_PF_GM, tiles_m - first);
  const int in = L - band * QGEMM_PF_GM * tiles_n;
  tm = first + in % gm;
  tn = in / gm;
}

template <int FMT, int G, int WGM, int WGN, int TM, int TN, int RU, int LA>
__global__ __launch_bounds__(64 * WGM * WGN) void qgemm_prefill(KArgs a) {
  constexpr int NW = WGM * WGN;                      // wavefronts
  constexpr int NT = 64 * NW;                        // threads
  constexpr int BM = 16 * WGM * TM, BN = 16 * WGN * TN;
  constexpr int ROWB = 256;                          // bytes of one A row per k block
  constexpr int NDMA = BM / (4 * NW);                // 1 KiB DMA loads per wavefront per k block
  constexpr int TU = TM / RU;                        // read units per K step
  constexpr int NU = 4 * TU;                         // read units per k block
  static_assert(NDMA * 4 * NW == BM && (4 * NW) % 16 == 0, "A tile must split into whole 4-row DMA loads");
  static_assert(TU * RU == TM, "RU must divide TM");
  constexpr int DS = QGEMM_PF_DS;                    // read units between two DMA issues
  static_assert(DS * (NDMA - 1) < NU, "the DMA loads must all be issued within one k block");
  __shared__ __attribute__((aligned(1024))) unsigned char As0[BM * ROWB];
  __shared__ __attribute__((aligned(1024))) unsigned char As1[BM * ROWB];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int tile = blockIdx.x, split = blockIdx.y;
  int tm, tn;
  pf_tile_of(tile, gridDim.x, a.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int KB = a.K >> 7, NB = a.N >> 4;
  const int kb_begin = split * a.kb_per_split;
  const int kb_end = min(KB, kb_begin + a.kb_per_split);

  // DMA load i of this wavefront fills LDS bytes [(NW i + wave) KiB, +1 KiB): tile rows
  // 4 (NW i + wave) + lane / 16, chunk position lane & 15.  Since 4 NW is a multiple of 16,
  // the row's low four bits, and so the swizzled source chunk, do not depend on i.
  const int drow = 4 * wave + (lane >> 4);
  const int dchunk = (lane & 15) ^ (drow & 15);
  const int rows = min(a.M - m0, BM);
  const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.A + (size_t)m0 * a.K), (short)0, rows * a.K * 2, 0x00020000);
  const int dvoff = drow * a.K * 2 + 16 * dchunk;
  const int dstride = 4 * NW * a.K * 2;              // bytes between a wavefront's DMA loads
  auto load_a = [&](int kb, unsigned char* As, int i) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(arsrc, (lds_ptr_t)(As + (NW * i + wave) * 1024), 16,
                                             dvoff + i * dstride, kb * ROWB, 0, 0);
  };

  // A-fragment read offsets, one per K step: row 16 TM wm + 16 i + (l & 15), chunk 4t + l / 16.
  int aoff[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
    aoff[t] = (16 * TM * wm + (lane & 15)) * ROWB + 16 * ((4 * t + (lane >> 4)) ^ (lane & 15));

  int nbw[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) nbw[j] = min((n0 >> 4) + TN * wn + j, NB - 1);
  auto load_w = [&](int kb, WFrag<FMT> (&wf)[TN]) {
#pragma unroll
    for (int j = 0; j < TN; ++j) load_wfrag<FMT, G, false>(a, nbw[j], kb, lane, wf[j]);
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Computes one k block from As / wf while issuing the DMA loads of the next one (into
  // Ad), DS read units apart: issued all at once they would fill the memory pipeline's
  // queue and stall the wavefront's MFMAs behind it.
  auto compute = [&](const unsigned char* As, const WFrag<FMT> (&wf)[TN], int kb_next, unsigned char* Ad) {
    float fs[TN][4];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int t = 0; t < 4; ++t) fs[j][t] = 0.f;
      if constexpr (FMT == qgemm::FMT_FP4) fp4_scales(wf[j].s[0], fs[j]);
    }
    u32x4 af[LA + 1][RU];
    auto read_unit = [&](int u, u32x4 (&dst)[RU]) {
      const int t = u / TU, i0 = (u % TU) * RU;
#pragma unroll
      for (int r = 0; r < RU; ++r) dst[r] = *reinterpret_cast<const u32x4*>(As + aoff[t] + (i0 + r) * 16 * ROWB);
    };
    u32x4 b[2][TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) b[0][j] = bfrag<FMT, G>(wf[j], 0, fs[j]);
#pragma unroll
    for (int u = 0; u < LA && u < NU; ++u) read_unit(u, af[u]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int t = u / TU, i0 = (u % TU) * RU;
      if (u + LA < NU) read_unit(u + LA, af[(u + LA) % (LA + 1)]);
      if (u % DS == 0 && u / DS < NDMA) load_a(kb_next, Ad, u / DS);
      __builtin_amdgcn_sched_barrier(0);   // later units' reads go out before this unit's MFMAs
      if (i0 + RU == TM && t < 3) {
#pragma unroll
        for (int j = 0; j < TN; ++j) b[(t + 1) & 1][j] = bfrag<FMT, G>(wf[j], t + 1, fs[j]);
      }
#pragma unroll
      for (int r = 0; r < RU; ++r)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i0 + r][j] = mfma<FMT>(af[u % (LA + 1)][r], b[t & 1][j], acc[i0 + r][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  WFrag<FMT> w0[TN], w1[TN];
#pragma unroll
  for (int i = 0; i < NDMA; ++i) load_a(kb_begin, As0, i);
  load_w(kb_begin, w0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  for (int kb = kb_begin; kb < kb_end; kb += 2) {
    // even step: block kb from As0 / w0; loads of block kb + 1 into As1 / w1
    const int k1 = min(kb + 1, kb_end - 1);
    load_w(k1, w1);
    __builtin_amdgcn_sched_barrier(0);
    compute(As0, w0, k1, As1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kb + 1 >= kb_end) break;
    // odd step: block kb + 1 from As1 / w1; loads of block kb + 2 into As0 / w0
    const int k2 = min(kb + 2, kb_end - 1);
    load_w(k2, w0);
    __builtin_amdgcn_sched_barrier(0);
    compute(As1, w1, k2, As0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  f32x4 v[TM * TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) v[TN * i + j] = acc[i][j];
  if (a.splits > 1) {
    if (!splitk_finish<TM * TN, NT>(a, tile, split, BM * BN, true, v)) return;
  }
  const float alpha = FMT == qgemm::FMT_INT4 ? 1.0f : *a.alpha;
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int nb = (n0 >> 4) + TN * wn + j;
    if (nb >= NB) continue;
    const int n = nb * 16 + (lane & 15);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 16 * TM * wm + 16 * i + 4 * (lane >> 4) + r;
        if (m < a.M) store_out(a, m, n, FMT == qgemm::FMT_INT4 ? v[TN * i + j][r] : v[TN * i + j][r] * alpha);
      }
  }
}

// ----------------------------------------------------------------------------- launch
template <int FMT, int G, int CB, int KPW>
void launch_decode(const qgemm::Plan& pl, const KArgs& a, hipStream_t stream) {
  const dim3 grid(pl.grid_x, pl.grid_y);
  if (pl.astage)
    hipLaunchKernelGGL((qgemm_decode<FMT, G, CB, KPW, QGEMM_DEC_NW, true>), grid, dim3(64 * QGEMM_DEC_NW), 0, stream, a);
  else
    hipLaunchKernelGGL((qgemm_decode<FMT, G, CB, KPW, QGEMM_DEC_NW, false>), grid, dim3(64 * QGEMM_DEC_NW), 0, stream, a);
}

template <int FMT, int G, int WGM, int WGN, int TM, int TN, int RU, int LA>
void launch_prefill(const qgemm::Plan& pl, const KArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((qgemm_prefill<FMT, G, WGM, WGN, TM, TN, RU, LA>), dim3(pl.grid_x, pl.grid_y),
                     dim3(64 * WGM * WGN), 0, stream, a);
}

template <int FMT, int G>
hipError_t launch(const qgemm::Plan& pl, const KArgs& a, hipStream_t stream) {
  if (pl.kind == qgemm::KIND_PREFILL) {
    if (pl.bm == qgemm::pf_bm(qgemm::kPfLarge))
      launch_prefill<FMT, G, qgemm::kPfLarge.wgm, qgemm::kPfLarge.wgn, qgemm::kPfLarge.tm, qgemm::kPfLarge.tn,
                     qgemm::kPfLarge.ru, qgemm::kPfLarge.la>(pl, a, stream);
    else
      launch_prefill<FMT, G, qgemm::kPfMedium.wgm, qgemm::kPfMedium.wgn, qgemm::kPfMedium.tm, qgemm::kPfMedium.tn,
                     qgemm::kPfMedium.ru, qgemm::kPfMedium.la>(pl, a, stream);
  } else {
    switch (pl.cb * 16 + pl.kpw) {
      case 16 + 8: launch_decode<FMT, G, 1, 8>(pl, a, stream); break;
      case 16 + 5: launch_decode<FMT, G, 1, 5>(pl, a, stream); break;
      case 16 + 4: launch_decode<FMT, G, 1, 4>(pl, a, stream); break;
      case 16 + 2: launch_decode<FMT, G, 1, 2>(pl, a, stream); break;
      case 16 + 1: launch_decode<FMT, G, 1, 1>(pl, a, stream); break;
      case 32 + 4: launch_decode<FMT, G, 2, 4>(pl, a, stream); break;
      case 32 + 2: launch_decode<FMT, G, 2, 2>(pl, a, stream); break;
      case 32 + 1: launch_decode<FMT, G, 2, 1>(pl, a, stream); break;
      case 64 + 2: launch_decode<FMT, G, 4, 2>(pl, a, stream); break;
      case 64 + 1: launch_decode<FMT, G, 4, 1>(pl, a, stream); break;
      default: return hipErrorInvalidConfiguration;
    }
  }
  return hipGetLastError();
}

hipError_t launch_any(const qgemm::Plan& pl, int group_size, const KArgs& a, hipStream_t stream) {
  switch (pl.fmt) {
    case qgemm::FMT_INT4:
      switch (group_size) {
        case 32: return launch<qgemm::FMT_INT4, 32>(pl, a, stream);
        case 64: return launch<qgemm::FMT_INT4, 64>(pl, a, stream);
        case 128: return launch<qgemm::FMT_INT4, 128>(pl, a, stream);
        case 256: return launch<qgemm::FMT_INT4, 256>(pl, a, stream);
        default: return hipErrorInvalidValue;
      }
    case qgemm::FMT_FP8: return launch<qgemm::FMT_FP8, 0>(pl, a, stream);
    default: return launch<qgemm::FMT_FP4, 0>(pl, a, stream);
  }
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

}  // namespace

extern "C" qgemm_status_t qgemm_run(const qgemm_problem_t* p, const void* A, const void* w_packed,
                                    const void* s_packed, const float* alpha, void* out, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  using namespace qgemm;
  clear_error();
  qgemm_status_t st = validate_problem(p);
  if (st != QGEMM_OK) return st;
  const Format fmt = format_of(p);
  if (!A) return fail(QGEMM_ERR_INVALID_ARGUMENT, "A is NULL");
  if (!w_packed) return fail(QGEMM_ERR_INVALID_ARGUMENT, "w_packed is NULL");
  if (!out) return fail(QGEMM_ERR_INVALID_ARGUMENT, "out is NULL");
  if (fmt != FMT_FP8 && !s_packed) return fail(QGEMM_ERR_INVALID_ARGUMENT, "s_packed is NULL (needed for INT4 and FP4)");
  if (fmt != FMT_INT4 && !alpha) return fail(QGEMM_ERR_INVALID_ARGUMENT, "alpha is NULL (needed for FP8 and FP4)");
  if (!aligned(A, 16)) return fail(QGEMM_ERR_MISALIGNED, "A must be 16-byte aligned");
  if (!aligned(w_packed, 16)) return fail(QGEMM_ERR_MISALIGNED, "w_packed must be 16-byte aligned");
  if (s_packed && fmt != FMT_FP8 && !aligned(s_packed, 16)) return fail(QGEMM_ERR_MISALIGNED, "s_packed must be 16-byte aligned");
  if (alpha && fmt != FMT_INT4 && !aligned(alpha, 4)) return fail(QGEMM_ERR_MISALIGNED, "alpha must be 4-byte aligned");
  if (!aligned(out, 16)) return fail(QGEMM_ERR_MISALIGNED, "out must be 16-byte aligned");

  Plan pl;
  st = make_plan(p, &pl);
  if (st != QGEMM_OK) return st;
  if (pl.ws_bytes) {
    if (!workspace || workspace_bytes < pl.ws_bytes)
      return fail(QGEMM_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes needed, %zu given%s", pl.ws_bytes,
                  workspace ? workspace_bytes : (size_t)0, workspace ? "" : " (NULL)");
    if (!aligned(workspace, 256)) return fail(QGEMM_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  }

  KArgs a;
  std::memset(&a, 0, sizeof(a));
  a.A = static_cast<const uint16_t*>(A);
  a.W = static_cast<const uint8_t*>(w_packed);
  a.S = s_packed;
  a.alpha = alpha;
  a.out = out;
  if (pl.ws_bytes) {
    a.counters = static_cast<unsigned*>(workspace);
    a.partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.counters_bytes);
  }
  a.M = (int)p->M;
  a.N = (int)p->N;
  a.K = (int)p->K;
  a.out_dtype = p->out_dtype;
  a.splits = pl.splits;
  a.kb_per_split = pl.kb_per_split;
  a.tiles_n = (int)((p->N + pl.bn - 1) / (pl.bn ? pl.bn : 1));

  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = launch_any(pl, p->group_size, a, s);
  if (e != hipSuccess) return fail(QGEMM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return QGEMM_OK;
}
