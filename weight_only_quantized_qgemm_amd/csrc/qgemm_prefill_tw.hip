// The prefill kernel with dedicated dequantization ("transform") wavefronts, on gfx950.
//
// FlashInfer PR #7495 analysis, section 1, describes a Blackwell main loop in which a
// dedicated transform warpgroup turns the packed weights into 16-bit MMA operands in shared
// memory while the MMA warps only consume operands.  This is that split for gfx950: a
// 64 x 128 output tile per workgroup of 8 MFMA wavefronts and 4 transform wavefronts.
//   * The transform wavefronts issue every global access of the main loop: the A tile by
//     buffer-to-LDS DMA (four 16-byte chunks per lane and k block, chunk c of row r at
//     position c ^ (r & 15), the swizzle of the other prefill tiles) three k blocks ahead, and
//     the packed weights and scales of two 16-column blocks each, also three blocks ahead
//     into rotating register sets.  One k block ahead of the MFMAs they dequantize the
//     weights into an LDS stage in MFMA fragment order: fragment (column block c, K step t)
//     is 1 KiB, lane l's 16 bytes at 16 l, exactly the operand lane l of an MFMA wavefront
//     reads (one conflict-free ds_read_b128).
//   * MFMA wavefront w owns column block w of the tile and all four of its row tiles: per
//     K step one weight fragment and four A fragments from LDS, four MFMAs.  It issues no
//     global load and no VALU dequantization; its only waits are on LDS reads and barriers.
// One workgroup barrier per k block; both roles execute the same number, each on its own
// path.  Stages: A in four 16 KiB stages (block kb + 3 is loaded into the stage block kb - 1
// was read from), dequantized weights in two 32 KiB stages (block kb + 1 is written into
// the stage block kb - 1 was read from): 128 KiB of LDS, one workgroup per CU.
// The weights enter each MFMA as its first operand, so the accumulator is the transposed
// 16 x 16 tile: lane l holds output row l & 15, columns 4 (l >> 4) .. + 3 (one 8- or 16-byte
// store).  Split K uses the ticketed hand-off of the other kernels (slice-ordered sum).
#include "qgemm_device.h"

namespace qgemm {
namespace dev {
namespace {

constexpr int kTwMma = 8;     // MFMA wavefronts
constexpr int kTwXf = 4;      // transform wavefronts
constexpr int kTwStA = 4;     // A stages
constexpr int kTwBM = 64, kTwBN = 128;

template <int FMT, int G>
__global__ __launch_bounds__(64 * (kTwMma + kTwXf)) void qgemm_prefill_tw(KArgs a) {
  constexpr int BM = kTwBM, BN = kTwBN, NW = kTwMma, NX = kTwXf, ST = kTwStA;
  constexpr int ROWB = 256;                          // bytes of one A row per k block
  constexpr int TM = BM / 16;                        // row tiles of an MFMA wavefront
  constexpr int CBX = BN / 16 / NX;                  // column blocks of a transform wavefront
  constexpr int NDMA = BM / (4 * NX);                // 1 KiB A DMA loads per transform wavefront and k block
  constexpr int BSTAGE = BN / 16 * 4 * 1024;         // one k block of dequantized fragments
  static_assert(NDMA * 4 * NX == BM && (4 * NX) % 16 == 0, "A tile must split into whole 4-row DMA loads");
  static_assert(BN / 16 == NW && CBX * NX == NW, "one column block per MFMA wavefront");
  // Vector-memory loads per k block of a transform wavefront: NDMA A loads and two per column
  // block (the fragment and its scales, or FP8's two halves).  At the end of step kb, block
  // kb + 1's A must have landed while blocks kb + 2 and kb + 3 may still be in flight.
  constexpr int PEND = (ST - 2) * (NDMA + 2 * CBX);
  static_assert(PEND <= 63, "vmcnt counts at most 63 outstanding loads");
  // s_waitcnt vmcnt(PEND) lgkmcnt(0): the wavefront's fragment writes have landed as well
  constexpr int WAIT_PEND_LDS = (PEND & 15) | (7 << 4) | (0 << 8) | ((PEND >> 4) << 14);
  // Separate arrays, so that the compiler tells the stage being read from the ones being filled.
  __shared__ __attribute__((aligned(1024))) unsigned char As0[BM * ROWB];
  __shared__ __attribute__((aligned(1024))) unsigned char As1[BM * ROWB];
  __shared__ __attribute__((aligned(1024))) unsigned char As2[BM * ROWB];
  __shared__ __attribute__((aligned(1024))) unsigned char As3[BM * ROWB];
  __shared__ __attribute__((aligned(1024))) unsigned char Bs0[BSTAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char Bs1[BSTAGE];
  auto astage = [&](int i) -> unsigned char* { return i == 0 ? As0 : i == 1 ? As1 : i == 2 ? As2 : As3; };
  auto bstage = [&](int i) -> unsigned char* { return i == 0 ? Bs0 : Bs1; };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int KB = a.K >> 7, NB = a.N >> 4;
  int tm, tn;
  pf_tile_of(blockIdx.x, gridDim.x, a.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int kb_begin = blockIdx.y * a.kb_per_split;
  const int kb_end = min(KB, kb_begin + a.kb_per_split);

  f32x4 acc[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (wave >= NW) {
    // ------------------------------------------------------------- transform wavefront x
    const int x = wave - NW;
    Lut lut;                                         // NF4 code book (wavefront-uniform)
    load_lut<FMT>(a, lut);
    // DMA load i fills LDS bytes [(NX i + x) KiB, +1 KiB): tile rows 4 (NX i + x) + lane / 16,
    // chunk position lane & 15; since 4 NX is a multiple of 16, the row's low four bits (and
    // so the swizzled source chunk) do not depend on i.  The resource covers the tile's
    // valid rows only: rows at or beyond M read as zero.
    const int drow = 4 * x + (lane >> 4);
    const int dchunk = (lane & 15) ^ (drow & 15);
    const int rows = min(a.M - m0, BM);
    const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.A + (size_t)m0 * a.K), (short)0, rows * a.K * 2, 0x00020000);
    const int dvoff = drow * a.K * 2 + 16 * dchunk;
    const int dstride = 4 * NX * a.K * 2;
    auto load_a = [&](int kb, unsigned char* As) {
#pragma unroll
      for (int i = 0; i < NDMA; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(arsrc, (lds_ptr_t)(As + (NX * i + x) * 1024), 16, dvoff + i * dstride,
                                                 kb * ROWB, 0, 0);
    };
    int nbw[CBX];                                    // column blocks past N are clamped (never stored)
#pragma unroll
    for (int j = 0; j < CBX; ++j) nbw[j] = min((n0 >> 4) + CBX * x + j, NB - 1);
    auto load_w = [&](int kb, WFrag<FMT> (&wf)[CBX]) {
#pragma unroll
      for (int j = 0; j < CBX; ++j) load_wfrag<FMT, G, false>(a, nbw[j], kb, lane, wf[j]);
    };
    auto dequant = [&](const WFrag<FMT> (&wf)[CBX], unsigned char* Bs) {
#pragma unroll
      for (int j = 0; j < CBX; ++j) {
        float fs[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (FMT == qgemm::FMT_FP4) fp4_scales(wf[j].s[0], fs);
#pragma unroll
        for (int t = 0; t < 4; ++t)
          *reinterpret_cast<u32x4*>(Bs + ((CBX * x + j) * 4 + t) * 1024 + lane * 16) = bfrag<FMT, G>(wf[j], t, fs, lut);
      }
    };

    // Prologue: blocks kb_begin .. kb_begin + ST - 2 (weights, then A), block kb_begin's weights
    // dequantized into stage 0.  Step kb loads block kb + ST - 1 (into the register set and the
    // A stage block kb - 1 used) and dequantizes block kb + 1 into the other weight stage.
    WFrag<FMT> w[ST][CBX];
#pragma unroll
    for (int s = 0; s < ST - 1; ++s) {
      const int kb = min(kb_begin + s, kb_end - 1);
      load_w(kb, w[s]);
      load_a(kb, astage(s));
    }
    dequant(w[0], bstage(0));
    __builtin_amdgcn_s_waitcnt(WAIT_PEND_LDS);
    barrier_no_fence();
    for (int kb = kb_begin; kb < kb_end; kb += ST) {
#pragma unroll
      for (int j = 0; j < ST; ++j) {
        const int kn = min(kb + j + ST - 1, kb_end - 1);
        load_w(kn, w[(j + ST - 1) % ST]);
        load_a(kn, astage((j + ST - 1) % ST));
        __builtin_amdgcn_sched_barrier(0);
        dequant(w[(j + 1) % ST], bstage((j + 1) & 1));  // past the slice: a clamped block, never read
        __builtin_amdgcn_s_waitcnt(WAIT_PEND_LDS);
        barrier_no_fence();
        if (kb + j + 1 >= kb_end) break;
      }
    }
    // clamped re-loads past the slice may still be writing LDS
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    // ------------------------------------------------------------- MFMA wavefront w
    int aoff[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) aoff[t] = (lane & 15) * ROWB + 16 * ((4 * t + (lane >> 4)) ^ (lane & 15));
    const int boff = wave * 4 * 1024 + lane * 16;
    // a wavefront whose column block lies past N computes nothing (it still meets every barrier)
    const bool idle = (n0 >> 4) + wave >= NB;
    barrier_no_fence();                              // the prologue's stages are filled
    for (int kb = kb_begin; kb < kb_end; kb += ST) {
#pragma unroll
      for (int j = 0; j < ST; ++j) {
        if (!idle) {
          const unsigned char* As = astage(j);
          const unsigned char* Bs = bstage(j & 1);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const u32x4 b = *reinterpret_cast<const u32x4*>(Bs + boff + t * 1024);
            u32x4 af[TM];
#pragma unroll
            for (int i = 0; i < TM; ++i) af[i] = *reinterpret_cast<const u32x4*>(As + aoff[t] + i * 16 * ROWB);
#pragma unroll
            for (int i = 0; i < TM; ++i) acc[i] = mfma<FMT>(b, af[i], acc[i]);
          }
        }
        barrier_no_fence();
        if (kb + j + 1 >= kb_end) break;
      }
    }
  }

  const bool active = wave < NW;
  if (a.splits > 1) {
    if (!splitk_finish<TM, 64 * NW>(a, blockIdx.x, blockIdx.y, BM * BN, active, acc)) return;
  }
  if (!active) return;
  const int nb = (n0 >> 4) + wave;
  if (nb >= NB) return;
  const float alpha = qgemm::group_scaled(FMT) ? 1.0f : *a.alpha;
  const int n = nb * 16 + 4 * (lane >> 4);
  const f32x4 bv = bias4_of(a, n);
  // every value is formed before the first store (a wait for the bias load placed between
  // two stores would also wait for the stores before it)
  f32x4 o[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    f32x4 x = acc[i];
    if constexpr (!qgemm::group_scaled(FMT)) x = f32x4{x[0] * alpha, x[1] * alpha, x[2] * alpha, x[3] * alpha};
    if (a.out_dtype == QGEMM_DT_F32) x = f32x4{x[0] + bv[0], x[1] + bv[1], x[2] + bv[2], x[3] + bv[3]};
    asm volatile("" : "+v"(x));
    o[i] = x;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = m0 + 16 * i + (lane & 15);
    if (m >= a.M) continue;
    if (a.out_dtype == QGEMM_DT_F32)
      *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + (size_t)m * a.N + n) = o[i];
    else
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + (size_t)m * a.N + n) = pack4_out16(a, o[i], bv);
  }
}

template <int FMT, int G>
hipError_t launch_tw(const Plan& pl, const KArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((qgemm_prefill_tw<FMT, G>), dim3(pl.grid_x, pl.grid_y), dim3(64 * (kTwMma + kTwXf)), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

// The instances of one format (QGEMM_FMT_UNIT), one per group size where the format has them.
template <int FMT>
hipError_t launch_prefill_tw_format(const Plan& pl, int group_size, const KArgs& a, hipStream_t stream) {
  if (pl.bm != kTwBM || pl.bn != kTwBN || pl.persist) return hipErrorInvalidConfiguration;
  if constexpr (qgemm::group_scaled(FMT)) {
    switch (group_size) {
      case 32: return launch_tw<FMT, 32>(pl, a, stream);
      case 64: return launch_tw<FMT, 64>(pl, a, stream);
      case 128: return launch_tw<FMT, 128>(pl, a, stream);
      case 256: return launch_tw<FMT, 256>(pl, a, stream);
      default: return hipErrorInvalidValue;
    }
  } else {
    return launch_tw<FMT, 0>(pl, a, stream);
  }
}

#ifndef QGEMM_FMT_UNIT
#error "compile once per format with -DQGEMM_FMT_UNIT=<format>"
#endif
template hipError_t launch_prefill_tw_format<QGEMM_FMT_UNIT>(const Plan&, int, const KArgs&, hipStream_t);

}  // namespace dev
}  // namespace qgemm
