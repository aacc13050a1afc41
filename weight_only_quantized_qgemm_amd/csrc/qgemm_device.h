// Device-side building blocks shared by the decode and prefill kernels of the weight-only
// quantized GEMM on gfx950 (CDNA4), and the launchers each kernel source defines.
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
//   NF4 : the nibble indexes a 16-entry fp16 code book held in registers as byte tables
//         (v_perm_b32 looks up four bytes at once), and the entry is multiplied by the fp16
//         group scale: RNE_fp16(T[code] * s).  Low Bit Triton Kernels (lecture 034) weighs
//         this against INT4: the table must live in registers and the unpack is about twice
//         as long.
//
// Split-K (when the output tiles alone cannot fill 256 compute units): each K slice writes
// an fp32 partial tile to the workspace, then takes a ticket; the workgroup that draws the
// last ticket sums all partials in slice order (bitwise deterministic, whichever slice
// arrives last) and resets the ticket.  No workgroup ever waits for another, so nothing
// assumes co-residency (FlashInfer PR #7495 analysis, section 3(d), describes the deadlock
// that assumption caused and the slice-ordered sum that keeps results bitwise identical).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "qgemm_internal.h"

namespace qgemm {
namespace dev {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
// LDS destination of a buffer-to-LDS DMA load
typedef __attribute__((address_space(3))) void* lds_ptr_t;

struct KArgs {
  const uint16_t* A;          // [M][K] 16-bit
  const uint8_t* W;           // packed weights
  const void* S;              // packed scales (INT4 / INT2 / NF4: fp16, FP4: e4m3 bytes)
  const unsigned* lut;        // NF4: code-book header (low-byte tables, then high-byte tables)
  const float* alpha;         // FP8 / FP4: device scalar
  void* out;                  // [M][N]
  const void* bias;           // [N] of out_dtype, added after alpha; NULL for none
  unsigned* counters;         // split-K tickets, one per tile
  float* partials;            // split-K partial tiles
  int M, N, K;
  int out_dtype;
  int splits, kb_per_split;
  int tiles_n;                // prefill: output tiles along N
  // persistent prefill (grid of `persist` workgroups, 0 = one tile per workgroup): tiles
  // 0 .. dp_tiles - 1 go round-robin to the workgroups, the k blocks of the rest (the stream-K
  // tail) are split into ranges of sk_q + 1 (the first sk_r workgroups) or sk_q
  int persist, tiles_total, dp_tiles;
  int sk_q, sk_r;
};

// ----------------------------------------------------------------------------- dequant
// (a & M) | O in one VALU op (v_and_or_b32).  With both constants as literals the compiler
// splits it into AND + OR (an instruction takes one literal); held in registers they fit
// one instruction.  The constants are moved into registers by an opaque (non-volatile,
// hence shared) asm statement, and the operation itself stays in C so the compiler sees
// every register it writes: an MFMA that reads a register a VALU op has just written needs
// wait states, which the compiler inserts only for instructions it knows.
template <unsigned C>
__device__ __forceinline__ unsigned vconst() {
  unsigned r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(C));
  return r;
}
template <unsigned M, unsigned O>
__device__ __forceinline__ unsigned and_or(unsigned a) {
  return (a & vconst<M>()) | vconst<O>();
}

__device__ __forceinline__ u32x4 dq_int4(unsigned w, unsigned s2) {
  const unsigned hi = w >> 8;
  const unsigned p0 = and_or<0x000F000Fu, 0x64006400u>(w);    // k slots j0, j1: 1024 + nibble
  const unsigned p1 = and_or<0x00F000F0u, 0x54005400u>(w);    // j2, j3: 64 + nibble
  const unsigned p2 = and_or<0x000F000Fu, 0x64006400u>(hi);   // j4, j5
  const unsigned p3 = and_or<0x00F000F0u, 0x54005400u>(hi);   // j6, j7
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

// INT2: byte b of either 16-bit half of dword w carries one K step, field f (bits 2f, 2f+1
// of the byte) the k pair (2f, 2f + 1), the even k in the low half.  OR-ing the masked
// field into the exponent of 2^(10 - 2f) gives 2^(10 - 2f) + code exactly; subtracting
// 2^(10 - 2f) + 2 leaves the signed value, which the scale multiplies (RNE_fp16, exact while
// the product stays in range: at most 12 significant bits).
__device__ __forceinline__ u32x4 dq_int2(unsigned w, int b, unsigned s2) {
  const unsigned x = b ? w >> 8 : w;
  const unsigned p0 = and_or<0x00030003u, 0x64006400u>(x);    // k 0, 1: 1024 + code
  const unsigned p1 = and_or<0x000C000Cu, 0x5C005C00u>(x);    // k 2, 3: 256 + code
  const unsigned p2 = and_or<0x00300030u, 0x54005400u>(x);    // k 4, 5: 64 + code
  const unsigned p3 = and_or<0x00C000C0u, 0x4C004C00u>(x);    // k 6, 7: 16 + code
  const f16x2 s = __builtin_bit_cast(f16x2, s2);
  const f16x2 b0 = {(_Float16)1026.0f, (_Float16)1026.0f}, b1 = {(_Float16)258.0f, (_Float16)258.0f};
  const f16x2 b2 = {(_Float16)66.0f, (_Float16)66.0f}, b3 = {(_Float16)18.0f, (_Float16)18.0f};
  return u32x4{__builtin_bit_cast(unsigned, (__builtin_bit_cast(f16x2, p0) - b0) * s),
               __builtin_bit_cast(unsigned, (__builtin_bit_cast(f16x2, p1) - b1) * s),
               __builtin_bit_cast(unsigned, (__builtin_bit_cast(f16x2, p2) - b2) * s),
               __builtin_bit_cast(unsigned, (__builtin_bit_cast(f16x2, p3) - b3) * s)};
}

// NF4 code book as byte tables: lo[q] byte j = low byte of T[4q + j], hi[q] the high bytes.
struct Lut {
  unsigned lo[4], hi[4];
};
template <int FMT>
__device__ __forceinline__ void load_lut(const KArgs& a, Lut& t) {
  if constexpr (FMT == qgemm::FMT_NF4) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      t.lo[q] = a.lut[q];
      t.hi[q] = a.lut[4 + q];
    }
  }
}

// Byte j of the result = byte sel_j of the 16-byte table t3:t2:t1:t0 (sel_j in 0..15).
// v_perm_b32 selects among 8 bytes, so entries 0..7 and 8..15 are looked up separately and
// bit 3 of each index picks one (hm: 0xFF in the bytes whose index has bit 3 set).
__device__ __forceinline__ unsigned lut16(unsigned t0, unsigned t1, unsigned t2, unsigned t3, unsigned sel,
                                          unsigned hm) {
  const unsigned a = __builtin_amdgcn_perm(t1, t0, sel);
  const unsigned b = __builtin_amdgcn_perm(t3, t2, sel);
  return (b & hm) | (a & ~hm);
}

// Dword w holds 8 nibbles; byte b carries the codes of k offsets b (low nibble) and b + 4
// (high nibble).  Returns the four fp16 pairs (k 0,1), (2,3), (4,5), (6,7), each times s.
__device__ __forceinline__ u32x4 dq_nf4(unsigned w, unsigned s2, const Lut& t) {
  const unsigned w4 = w >> 4;
  const unsigned sa = w & 0x07070707u, sb = w4 & 0x07070707u;
  // bytes 0xFF where bit 3 (sa) or bit 7 (sb) of the byte is set: the sign-replicating
  // selectors 8..11 of v_perm_b32 read bit 7 of bytes 1, 3, 5, 7 of {x << 8, x}
  const unsigned ha = __builtin_amdgcn_perm(w << 12, w << 4, 0x090B080Au);
  const unsigned hb = __builtin_amdgcn_perm(w << 8, w, 0x090B080Au);
  const unsigned la = lut16(t.lo[0], t.lo[1], t.lo[2], t.lo[3], sa, ha);   // low bytes, k 0..3
  const unsigned ua = lut16(t.hi[0], t.hi[1], t.hi[2], t.hi[3], sa, ha);   // high bytes, k 0..3
  const unsigned lb = lut16(t.lo[0], t.lo[1], t.lo[2], t.lo[3], sb, hb);   // k 4..7
  const unsigned ub = lut16(t.hi[0], t.hi[1], t.hi[2], t.hi[3], sb, hb);
  const f16x2 s = __builtin_bit_cast(f16x2, s2);
  const unsigned p0 = __builtin_amdgcn_perm(ua, la, 0x05010400u);   // fp16 of k 0 | k 1 << 16
  const unsigned p1 = __builtin_amdgcn_perm(ua, la, 0x07030602u);   // k 2, 3
  const unsigned p2 = __builtin_amdgcn_perm(ub, lb, 0x05010400u);   // k 4, 5
  const unsigned p3 = __builtin_amdgcn_perm(ub, lb, 0x07030602u);   // k 6, 7
  return u32x4{__builtin_bit_cast(unsigned, __builtin_bit_cast(f16x2, p0) * s),
               __builtin_bit_cast(unsigned, __builtin_bit_cast(f16x2, p1) * s),
               __builtin_bit_cast(unsigned, __builtin_bit_cast(f16x2, p2) * s),
               __builtin_bit_cast(unsigned, __builtin_bit_cast(f16x2, p3) * s)};
}

__device__ __forceinline__ u32x4 dq_fp8(unsigned lo, unsigned hi) {
  return u32x4{__builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false)),
               __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true)),
               __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false)),
               __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true))};
}

// e4m3 -> fp16 is exact too (fp16 covers e4m3's range and precision, subnormals included).
__device__ __forceinline__ u32x4 dq_fp8h(unsigned lo, unsigned hi) {
  return u32x4{__builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false)),
               __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true)),
               __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false)),
               __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true))};
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
  if constexpr (qgemm::f16_mfma(FMT))
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
  u32x4 w[qgemm::fp8_weights(FMT) ? 2 : 1];
  unsigned s[2];    // INT4: 1, 2 or 4 fp16 scales (G = 128|256, 64, 32); FP4: 4 e4m3 bytes
};

// G is the INT4 / INT2 group size (a template parameter, so the scale load has no branches:
// a branch around a load ends in a wait for every outstanding load); 0 for FP8 / FP4.
// STREAM marks weights read once (decode: non-temporal loads keep them out of the way in
// the caches); prefill re-reads each weight fragment once per row tile and caches it.
template <bool STREAM>
__device__ __forceinline__ u32x4 wload(const u32x4* p) {
  if constexpr (STREAM) return __builtin_nontemporal_load(p);
  else return *p;
}

template <int FMT, int G, bool STREAM = true, bool SCALES = true>
__device__ __forceinline__ void load_wfrag(const KArgs& a, int nb, int kb, int lane, WFrag<FMT>& f) {
  const int KB = a.K >> 7;
  if constexpr (qgemm::fp8_weights(FMT)) {
    const u32x4* p = reinterpret_cast<const u32x4*>(a.W + ((size_t)nb * (KB * 2) + 2 * kb) * 1024) + lane;
    f.w[0] = wload<STREAM>(p);
    f.w[1] = wload<STREAM>(p + 64);
  } else if constexpr (FMT == qgemm::FMT_INT2) {   // 512-byte blocks, 8 bytes per lane
    const u32x2* p = reinterpret_cast<const u32x2*>(a.W + ((size_t)nb * KB + kb) * 512) + lane;
    u32x2 x;
    if constexpr (STREAM) x = __builtin_nontemporal_load(p);
    else x = *p;
    f.w[0] = u32x4{x[0], x[1], 0u, 0u};
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(a.W + ((size_t)nb * KB + kb) * 1024) + lane;
    f.w[0] = wload<STREAM>(p);
  }
  if constexpr (!SCALES) {
    return;
  } else if constexpr (qgemm::group_scaled(FMT)) {
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

// ----------------------------------------------------------------------------- scales
// Byte offset, inside one column block's packed scales, of the scales k block kb uses
// (INT4 with G = 256: of its group, which spans two k blocks); sc_rel(KB) is the size of one
// column block's scales.  FP8 has none.
template <int FMT, int G>
__device__ __forceinline__ int sc_rel(int kb) {
  if constexpr (qgemm::group_scaled(FMT)) return G <= 128 ? kb * 32 * (128 / G) : (kb >> 1) * 32;
  else if constexpr (FMT == qgemm::FMT_FP4) return kb * 128;
  else return 0;
}
// End of the scale bytes that cover k blocks up to kb_end (exclusive); a group of 256 is kept whole.
template <int FMT, int G>
__device__ __forceinline__ int sc_end(int kb_end) {
  return sc_rel<FMT, G>(qgemm::group_scaled(FMT) && G > 128 ? kb_end + 1 : kb_end);
}

// Scales of k block kb for this lane's column, from an LDS copy of one column block's packed
// scales that starts with those of k block kb_begin.
template <int FMT, int G>
__device__ __forceinline__ void read_staged_scales(const unsigned char* s, int kb, int kb_begin, int lane,
                                                   WFrag<FMT>& f) {
  const unsigned char* p = s + (sc_rel<FMT, G>(kb) - sc_rel<FMT, G>(kb_begin));
  if constexpr (qgemm::group_scaled(FMT)) {
    constexpr int T = G <= 128 ? 128 / G : 1;
    p += (lane & 15) * T * 2;
    if constexpr (T == 4) {
      const u32x2 x = *reinterpret_cast<const u32x2*>(p);
      f.s[0] = x[0];
      f.s[1] = x[1];
    } else if constexpr (T == 2) {
      f.s[0] = *reinterpret_cast<const unsigned*>(p);
    } else {
      f.s[0] = *reinterpret_cast<const uint16_t*>(p);
    }
  } else if constexpr (FMT == qgemm::FMT_FP4) {
    f.s[0] = *reinterpret_cast<const unsigned*>(p + (lane & 15) * 8 + 4 * (lane >> 5));
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
__device__ __forceinline__ u32x4 bfrag(const WFrag<FMT>& f, int t, const float (&fs)[4], const Lut& lut) {
  if constexpr (FMT == qgemm::FMT_INT4) {
    return dq_int4(f.w[0][t], int4_scale_pair<G>(f.s, t));
  } else if constexpr (FMT == qgemm::FMT_NF4) {
    return dq_nf4(f.w[0][t], int4_scale_pair<G>(f.s, t), lut);
  } else if constexpr (FMT == qgemm::FMT_INT2) {
    return dq_int2(f.w[0][t >> 1], t & 1, int4_scale_pair<G>(f.s, t));
  } else if constexpr (FMT == qgemm::FMT_FP8) {
    return dq_fp8(f.w[t >> 1][2 * (t & 1)], f.w[t >> 1][2 * (t & 1) + 1]);
  } else if constexpr (FMT == qgemm::FMT_FP8H) {
    return dq_fp8h(f.w[t >> 1][2 * (t & 1)], f.w[t >> 1][2 * (t & 1) + 1]);
  } else {
    return dq_fp4(f.w[0][t], fs[t]);
  }
}

// ----------------------------------------------------------------------------- epilogue
// Bias of column n as fp32 (exact), 0 without a bias.  Wavefront-uniform branch.
__device__ __forceinline__ float bias_of(const KArgs& a, int n) {
  if (!a.bias) return 0.0f;
  if (a.out_dtype == QGEMM_DT_F32) return static_cast<const float*>(a.bias)[n];
  if (a.out_dtype == QGEMM_DT_F16) return (float)static_cast<const _Float16*>(a.bias)[n];
  return (float)static_cast<const __bf16*>(a.bias)[n];
}

// Bias of columns n .. n + 3 (n a multiple of 4) as fp32 (exact), zeros without a bias: one
// 16-byte (fp32) or 8-byte (16-bit) load, aligned since the bias is 16-byte aligned.
__device__ __forceinline__ f32x4 bias4_of(const KArgs& a, int n) {
  if (!a.bias) return f32x4{0.f, 0.f, 0.f, 0.f};
  if (a.out_dtype == QGEMM_DT_F32) return *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.bias) + n);
  const u32x2 h = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(a.bias) + n);
  const unsigned h0 = h[0], h1 = h[1];
  if (a.out_dtype == QGEMM_DT_F16) {
    const f16x2 lo = __builtin_bit_cast(f16x2, h0), hi = __builtin_bit_cast(f16x2, h1);
    return f32x4{(float)lo[0], (float)lo[1], (float)hi[0], (float)hi[1]};
  }
  const bf16x2 lo = __builtin_bit_cast(bf16x2, h0), hi = __builtin_bit_cast(bf16x2, h1);
  return f32x4{(float)lo[0], (float)lo[1], (float)hi[0], (float)hi[1]};
}

// Four fp32 results (alpha already applied) plus their biases in fp32, each rounded once to
// the 16-bit output type, packed in column order.
__device__ __forceinline__ u32x2 pack4_out16(const KArgs& a, f32x4 v, f32x4 bias) {
  const float v0 = v[0] + bias[0], v1 = v[1] + bias[1], v2 = v[2] + bias[2], v3 = v[3] + bias[3];
  if (a.out_dtype == QGEMM_DT_F16) {
    const f16x2 lo = {(_Float16)v0, (_Float16)v1}, hi = {(_Float16)v2, (_Float16)v3};
    return u32x2{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
  }
  const bf16x2 lo = {(__bf16)v0, (__bf16)v1}, hi = {(__bf16)v2, (__bf16)v3};
  return u32x2{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
}

// v is the final fp32 value (alpha and bias already applied), rounded once to the output type.
__device__ __forceinline__ void store_val(const KArgs& a, int m, int n, float v) {
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
// (sc1) stores, which write through the XCD-private L2, every thread waits for its stores
// to be acknowledged before the barrier that precedes the ticket, and the last workgroup
// reads the partials back with device-scope loads, which do not hit in its own L2.  A
// device-scope fence would instead write back and invalidate the whole XCD L2 in every
// workgroup.  The accesses are 16-byte buffer loads and stores carrying the sc1 policy
// (the relaxed device-scope atomics of the same bits move 4 bytes per instruction).
constexpr int kCPolDevice = 16;   // buffer-instruction cache policy: sc1 (device scope)

// Hand-off of one contributor's fp32 partial tile, shared by split-K and the stream-K tail of
// the persistent prefill.  The tile's contributors use partial slots base .. base + span - 1
// (slot = tile_elems fp32 values); this one writes its partial to slot `my`, then takes a
// ticket on `counter`; the contributor that draws ticket nslots - 1 sums the partials of
// contributors 0 .. nslots - 1 (slot rel(i)) in that order, resets the ticket and returns true.
template <int NF, int NT, class RelSlot>
__device__ bool fixup_finish(unsigned* counter, float* base, int span, int my, int nslots, RelSlot rel,
                             int tile_elems, bool active, f32x4 (&v)[NF]) {
  __shared__ int s_last;
  const int tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t part =
      __builtin_amdgcn_make_buffer_rsrc(base, (short)0, span * tile_elems * 4, 0x00020000);
  if (active) {
#pragma unroll
    for (int f = 0; f < NF; ++f)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v[f]), part,
                                             (my * tile_elems + 4 * (f * NT + tid)) * 4, 0, kCPolDevice);
  }
  __builtin_amdgcn_s_waitcnt(0);     // this thread's partial stores are complete
  __syncthreads();
  if (tid == 0) {
    const unsigned ticket = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = ticket == (unsigned)(nslots - 1);
  }
  __syncthreads();
  if (!s_last) return false;
  if (active) {
#pragma unroll
    for (int f = 0; f < NF; ++f) v[f] = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int B = NF < 8 ? NF : 8;                // loads in flight per batch
    for (int i = 0; i < nslots; ++i) {
      const int s = rel(i);
#pragma unroll
      for (int f0 = 0; f0 < NF; f0 += B) {
        f32x4 p[B];
#pragma unroll
        for (int f = 0; f < B; ++f)
          p[f] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                               part, (s * tile_elems + 4 * ((f0 + f) * NT + tid)) * 4, 0, kCPolDevice));
#pragma unroll
        for (int f = 0; f < B; ++f) v[f0 + f] += p[f];
        __builtin_amdgcn_sched_barrier(0);          // one batch at a time: bounded registers
      }
    }
  }
  if (tid == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// Split-K: the splits of a tile use slots tile * splits .. + splits - 1, contributor i = slot i.
template <int NF, int NT = 256>
__device__ bool splitk_finish(const KArgs& a, int tile, int split, int tile_elems, bool active, f32x4 (&v)[NF]) {
  return fixup_finish<NF, NT>(a.counters + tile, a.partials + (size_t)tile * a.splits * tile_elems, a.splits, split,
                              a.splits, [](int i) { return i; }, tile_elems, active, v);
}

// ----------------------------------------------------------------------------- barrier
// Workgroup barrier without the release fence of __syncthreads(), which waits for every
// outstanding load, the A stages still meant to be in flight included.  Callers first
// wait for the loads that must have landed; every LDS read before the barrier has been
// consumed (so completed) by then; the clobbers keep the compiler from moving memory
// operations across it.
__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ----------------------------------------------------------------------------- tile walk
// Output tile of workgroup b.  Workgroups are dispatched to the eight XCDs (each with its
// own L2) round-robin by id, so the id is first mapped to a position such that each XCD
// owns one contiguous range of positions; positions then walk the tile grid in bands of
// GM tile rows, column by column, so that the tiles an XCD runs at the same time share
// few A row blocks and weight column blocks.
#ifndef QGEMM_PF_GM
#define QGEMM_PF_GM 4
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


// ----------------------------------------------------------------------------- launchers
// Launch the kernel instance the plan names on `stream`; return hipGetLastError().
hipError_t launch_decode(const Plan& pl, int group_size, const KArgs& a, hipStream_t stream);
hipError_t launch_prefill(const Plan& pl, int group_size, const KArgs& a, hipStream_t stream);
// The same for one format; each kernel source instantiates these for one format per object.
template <int FMT>
hipError_t launch_decode_format(const Plan& pl, int group_size, const KArgs& a, hipStream_t stream);
template <int FMT>
hipError_t launch_prefill_format(const Plan& pl, int group_size, const KArgs& a, hipStream_t stream);
// The prefill kernel with dedicated dequantization wavefronts (kernel_hint PREFILL_TRANSFORM).
template <int FMT>
hipError_t launch_prefill_tw_format(const Plan& pl, int group_size, const KArgs& a, hipStream_t stream);

}  // namespace dev
}  // namespace qgemm
