// The decode kernel (M <= 16) of the weight-only quantized GEMM on gfx950.
#include "qgemm_device.h"

namespace qgemm {
namespace dev {
namespace {

// ============================================================================= decode
// M <= 16.  Workgroup = NW wavefronts; it owns CB column blocks (16 columns each) and one
// K slice (normally all of K: a split-K hand-off costs three dependent memory round trips,
// more than a whole small GEMM).  Wavefront w owns a contiguous share of the slice's k
// blocks, streamed in runs of up to KPW blocks: all weight loads of a run are issued before
// any is consumed, and the k blocks are then consumed in load order, so each waits only for
// its own data.
//
// With ASTAGE (small M) each wavefront first stages its own share of A (M rows) and of the
// packed scales into a private LDS region, in 16-byte chunks, one load instruction per 64
// chunks: the MFMA fragment loads would otherwise fetch each A value 16 times, and the
// compute unit's vector-memory pipeline spends about the same time on a load instruction
// however few distinct bytes it carries.  Nothing staged is shared between wavefronts, so no
// workgroup barrier holds a wavefront back once its own data has arrived.  With larger M
// the rows are distinct: each wavefront loads its A fragments and its scales from global
// memory with its weights, either straight into registers (A_DIRECT) or, with A_DMA,
// through buffer-to-LDS DMA into a static LDS slot per k block of the run (4 KiB: 16 rows x
// 16 chunks of 16 bytes, chunk c of row r at position c ^ r, so that the fragment reads are
// free of bank conflicts); its fragments are then read from the slot.  A run overlapping the
// next one uses the other of two slot sets, each its own array, so that the compiler's wait
// before a slot read covers only the DMA loads of that set.  Rows at or beyond M read row
// M - 1 (MFMA output row m depends on A row m only; rows >= M are never stored).
// Control flow is wavefront-uniform and loads are clamped rather than predicated (the
// compiler waits for every outstanding load at the end of a branch that contains one).
// Each wavefront keeps two accumulators per column block (even / odd K steps) to halve the
// MFMA dependency chain; the NW wavefront tiles are summed through LDS in wave order.
// NR >= 2 (a share of NR runs): two register sets alternate and the loads of run r + 1
// are issued before run r is computed, so consecutive runs overlap their memory round
// trips.  The runs are unrolled (a loop carrying loads across its back edge defeats the
// compiler's wait tracking, which then drains every load at the loop head): up to four
// runs, or eight with A in DMA slots.  NR = 1: one run, or, for longer shares, runs one after
// another.
constexpr bool DEC_ACC2 = true;                     // two accumulators per column block

// The pointers and sizes that the first loads depend on come as separate leading
// arguments ahead of the full argument block: built with kernarg preloading, the dispatch
// places them in scalar registers, so the weight and A loads go out without first waiting
// for a scalar load of the argument block (2-4% of a decode launch).
template <int FMT, int G, int CB, int KPW, int NW, int AMODE, int NR>
__global__ __launch_bounds__(64 * NW) void qgemm_decode(const uint8_t* W, const void* S, const uint16_t* A,
                                                         const unsigned* code_book, int M, int N, int K,
                                                         int kb_per_split, KArgs a) {
  a.W = W;
  a.S = S;
  a.A = A;
  a.lut = code_book;
  a.M = M;
  a.N = N;
  a.K = K;
  a.kb_per_split = kb_per_split;
  constexpr bool MULTI = NR > 1;
  constexpr bool ASTAGE = qgemm::a_staged(AMODE), ADMA = AMODE == qgemm::A_DMA;
  constexpr int NT = 64 * NW;
  // Scales are staged with the A share (small M); otherwise each wavefront loads its own
  // with its weights (staging them alone measured slower at M = 16).
  constexpr bool HAS_S = !qgemm::fp8_weights(FMT) && ASTAGE;
  constexpr bool STAGE = ASTAGE;
  extern __shared__ __attribute__((aligned(16))) unsigned char dec_lds[];
  constexpr int DMA_SET = ADMA ? qgemm::dec_dma_set_bytes(NW, KPW) : 16;
  __shared__ __attribute__((aligned(1024))) unsigned char Ad0[DMA_SET];
  __shared__ __attribute__((aligned(1024))) unsigned char Ad1[ADMA && MULTI ? DMA_SET : 16];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = blockIdx.x, split = blockIdx.y;
  const int KB = a.K >> 7, NB = a.N >> 4;
  const int kb_begin = split * a.kb_per_split;
  const int kb_end = min(KB, kb_begin + a.kb_per_split);
  const int nb0 = group * CB;
  // this wavefront's contiguous share of the slice
  const int share = (kb_end - kb_begin + NW - 1) / NW;
  const int w_begin = min(kb_end, kb_begin + wave * share);
  const int w_end = min(kb_end, w_begin + share);
  const int row = min(lane & 15, a.M - 1);
  const int s_col = sc_rel<FMT, G>(KB);              // scale bytes of one whole column block

  // LDS (layout shared with the launch plan): one private region per wavefront ([its A share:
  // M rows of share x 128 + 8 halves][its scales: CB x SW bytes]), then the wave tiles of the
  // final reduction.
  Lut lut;                                           // NF4 code book (wavefront-uniform)
  load_lut<FMT>(a, lut);
  const int ldw = share * 128 + 8;                   // LDS A row stride (halves)
  const int aw_bytes = qgemm::dec_a_bytes(a.M, share, AMODE);
  const int SW = HAS_S ? qgemm::dec_scale_span(FMT, G, share) : 0;   // scale bytes of a share, per column block
  const int region = qgemm::dec_region_bytes(FMT, G, a.M, share, CB, AMODE);
  unsigned char* w_lds = dec_lds + wave * region;
  const unsigned char* s_lds = w_lds + aw_bytes;
  f32x4* red = reinterpret_cast<f32x4*>(dec_lds + NW * region);     // [NW][CB][64]

  // Staging of this wavefront's share, 16-byte chunks through buffer loads (32-bit offsets):
  // the A share (chunk q: row q / cpr, chunk q % cpr of the row), then its scales (chunk q:
  // column block q / spc, chunk q % spc of its range).  Iteration i covers chunks 64 i .. + 63
  // and is skipped (wavefront-uniformly) when all of them are past the end; lanes past the end
  // re-load the last chunk and write nothing.  Nothing here is shared with other wavefronts,
  // so no workgroup barrier delays the first k block.
  constexpr int SA = ASTAGE ? qgemm::kDecodeStageA : 0, SS = HAS_S ? qgemm::kDecodeStageS : 0;
  const int nkw = w_end - w_begin;                   // k blocks of this share (may be 0)
  const int cpr = nkw * 16;
  const int a_chunks = ASTAGE ? a.M * cpr : 0;
  const int sw0 = sc_rel<FMT, G>(w_begin);
  const int spc = (sc_end<FMT, G>(w_end) - sw0) >> 4;
  const int s_chunks = nkw > 0 ? CB * spc : 0;
  int soff[SA + SS + 1];
  u32x4 stage[SA + SS + 1];
  // A_STAGED_EARLY: the first weight block goes out before the staging loads, whose address
  // arithmetic otherwise delays it by ~0.5 us (M = 1 N = 4096 4.49 -> 4.27 us, M = 2 4.64 ->
  // 4.43, NF4 M = 1 5.32 -> 5.03).  Planned for one column block, runs of at most five k blocks
  // and at most one workgroup per CU: otherwise it measured 2-6% slower (M = 4 N = 11008, two
  // or three workgroups per CU; FP4 M = 1 K = 8192, runs of eight).
  constexpr bool W0FIRST = AMODE == qgemm::A_STAGED_EARLY;
  auto issue_staging = [&]() {
  if constexpr (ASTAGE) {
    const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.A + (size_t)w_begin * 128), (short)0, 0x7fffffff, 0x00020000);
    const float inv = 1.0f / (float)max(cpr, 1);
#pragma unroll
    for (int i = 0; i < SA; ++i) {
      soff[i] = -1;
      if (64 * i < a_chunks) {
        const int q = min(lane + 64 * i, a_chunks - 1);
        int r = (int)(((float)q + 0.5f) * inv);
        r -= r * cpr > q;
        const int c8 = q - r * cpr;
        stage[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ar, (r * a.K + 8 * c8) * 2, 0, 0));
        if (lane + 64 * i < a_chunks) soff[i] = r * ldw * 2 + 16 * c8;
      }
    }
  }
  if constexpr (HAS_S) {
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(static_cast<const unsigned char*>(a.S) + (size_t)nb0 * s_col + sw0), (short)0,
        0x7fffffff, 0x00020000);
    const int cmax = NB - 1 - nb0;                   // last column block of the matrix, relative
    const float inv = 1.0f / (float)max(spc, 1);
#pragma unroll
    for (int i = 0; i < SS; ++i) {
      soff[SA + i] = -1;
      if (64 * i < s_chunks) {
        const int q = min(lane + 64 * i, s_chunks - 1);
        int c = (int)(((float)q + 0.5f) * inv);
        c -= c * spc > q;
        const int o = q - c * spc;
        stage[SA + i] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(sr, min(c, cmax) * s_col + 16 * o, 0, 0));
        if (lane + 64 * i < s_chunks) soff[SA + i] = aw_bytes + c * SW + 16 * o;
      }
    }
  }
  if constexpr (STAGE) __builtin_amdgcn_sched_barrier(0);
  };
  if constexpr (!W0FIRST) issue_staging();

  f32x4 acc[CB][2];
#pragma unroll
  for (int c = 0; c < CB; ++c) acc[c][0] = acc[c][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint16_t* arow_g = a.A + (size_t)row * a.K + 8 * (lane >> 4);
  const uint16_t* arow_l = reinterpret_cast<const uint16_t*>(w_lds) + row * ldw + 8 * (lane >> 4);
  const int last = max(w_end - 1, w_begin);          // clamp target (valid even for an empty share)
  const int kb_cap = min(last, KB - 1);

  // A_DMA: load j (0..3) of a k block fills bytes [1024 j, +1024) of its slot, lane l the 16
  // bytes at 16 l: row r = 4 j + l / 16, position l & 15, which holds source chunk
  // (l & 15) ^ r of row min(r, M - 1) (the k block's byte offset goes in the scalar offset;
  // fetching nothing for rows >= M instead, through offsets past a bounded resource, measured
  // no faster at M = 5..12).  Fragment read t of a lane: row l & 15, source chunk 4 t + l / 16.
  // The A slots of a run go out before its weights: issued after them, they made the first
  // k block wait for the whole run's weights (M = 16, N = 4096: 5.4 -> 5.9 us).
  int aoff[ADMA ? 4 : 1];
  __amdgpu_buffer_rsrc_t drsrc;
  if constexpr (ADMA) {
    drsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.A), (short)0, 0x7fffffff, 0x00020000);
#pragma unroll
    for (int t = 0; t < 4; ++t) aoff[t] = (lane & 15) * 256 + 16 * ((4 * t + (lane >> 4)) ^ (lane & 15));
  }
  auto dma_slot = [&](unsigned char* set, int u) { return set + (wave * KPW + u) * 4096; };

  // one run: loads first (A fragments, then weights), then the k blocks in load order,
  // each waiting only for its own data
  constexpr int NAF = AMODE == qgemm::A_DIRECT ? KPW : 1;
  auto run_loads = [&](int run, u32x4 (&afr)[NAF][4], WFrag<FMT> (&wf)[KPW][CB], unsigned char* set, int u0 = 0,
                       int u1 = KPW) {
    if constexpr (ADMA) {
#pragma unroll
      for (int u = 0; u < KPW; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // the source offset is written out here: taken from a captured array or lambda, it
          // makes the host pass drop the kernel's launch stub
          const int r = 4 * j + (lane >> 4);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(drsrc, (lds_ptr_t)(dma_slot(set, u) + 1024 * j), 16,
                                                   min(r, a.M - 1) * a.K * 2 + 16 * ((lane & 15) ^ r),
                                                   min(run + u, kb_cap) * 256, 0, 0);
        }
    } else if constexpr (AMODE == qgemm::A_DIRECT) {
#pragma unroll
      for (int u = 0; u < KPW; ++u) {
        const u32x4* ap = reinterpret_cast<const u32x4*>(arow_g + (size_t)min(run + u, kb_cap) * 128);
#pragma unroll
        for (int t = 0; t < 4; ++t) afr[u][t] = ap[4 * t];
      }
    }
#pragma unroll
    for (int u = 0; u < KPW; ++u)
      if (u >= u0 && u < u1)                         // compile-time after unrolling
#pragma unroll
        for (int c = 0; c < CB; ++c)
          load_wfrag<FMT, G, true, !HAS_S>(a, min(nb0 + c, NB - 1), min(run + u, kb_cap), lane, wf[u][c]);
    __builtin_amdgcn_sched_barrier(0);
  };
  // MULTI: no branch around a k block (the compiler would wait for every load in flight,
  // the next run's included, at its end); a block past the share multiplies a zero A
  // fragment instead, and the staged reads stay inside the staged slice.
  auto run_compute = [&](int run, const u32x4 (&afr)[NAF][4], WFrag<FMT> (&wf)[KPW][CB], const unsigned char* set) {
#pragma unroll
    for (int u = 0; u < KPW; ++u) {
      const bool valid = run + u < w_end;
      if (MULTI || valid) {
        const int kbl = MULTI ? max(min(run + u, w_end - 1), w_begin) : run + u;   // inside the staged share
        u32x4 al[4];
        if constexpr (ASTAGE) {
          const uint16_t* ap = arow_l + (kbl - w_begin) * 128;
#pragma unroll
          for (int t = 0; t < 4; ++t) al[t] = *reinterpret_cast<const u32x4*>(ap + 32 * t);
        } else if constexpr (ADMA) {
          const unsigned char* ap = set + (wave * KPW + u) * 4096;
#pragma unroll
          for (int t = 0; t < 4; ++t) al[t] = *reinterpret_cast<const u32x4*>(ap + aoff[t]);
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t) al[t] = afr[u][t];
        }
        if constexpr (MULTI) {
#pragma unroll
          for (int t = 0; t < 4; ++t) al[t] = valid ? al[t] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int c = 0; c < CB; ++c) {
          if constexpr (HAS_S) {
            read_staged_scales<FMT, G>(s_lds + c * SW, kbl, w_begin, lane, wf[u][c]);
            if constexpr (MULTI) {                   // a block past the share: zero weights, never NaN
              wf[u][c].s[0] = valid ? wf[u][c].s[0] : 0u;
              wf[u][c].s[1] = valid ? wf[u][c].s[1] : 0u;
            }
          }
          float fs[4] = {0.f, 0.f, 0.f, 0.f};
          if constexpr (FMT == qgemm::FMT_FP4) fp4_scales(wf[u][c].s[0], fs);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const u32x4 av = al[t];
            acc[c][DEC_ACC2 ? (t & 1) : 0] = mfma<FMT>(av, bfrag<FMT, G>(wf[u][c], t, fs, lut), acc[c][DEC_ACC2 ? (t & 1) : 0]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  u32x4 afr[MULTI ? 2 : 1][NAF][4];
  WFrag<FMT> wf[MULTI ? 2 : 1][KPW][CB];
  // first run (every wavefront, with or without k blocks), then the staged share lands in LDS
  if constexpr (W0FIRST) {
    run_loads(w_begin, afr[0], wf[0], Ad0, 0, 1);
    issue_staging();
    run_loads(w_begin, afr[0], wf[0], Ad0, 1, KPW);
  } else {
    run_loads(w_begin, afr[0], wf[0], Ad0);
  }
  if constexpr (STAGE) {
#pragma unroll
    for (int i = 0; i < SA + SS; ++i)
      if (soff[i] >= 0) *reinterpret_cast<u32x4*>(w_lds + soff[i]) = stage[i];
    __builtin_amdgcn_s_waitcnt(0xC07F);              // lgkmcnt(0): the wavefront's own LDS writes have landed
    __builtin_amdgcn_wave_barrier();
    if constexpr (W0FIRST) __builtin_amdgcn_sched_barrier(0);   // the next run's loads stay behind
  }
  if constexpr (!MULTI) {
    if (w_begin < w_end) run_compute(w_begin, afr[0], wf[0], Ad0);
    for (int run = w_begin + KPW; run < w_end; run += KPW) {
      run_loads(run, afr[0], wf[0], Ad0);           // the previous run's slot reads fed its MFMAs already
      run_compute(run, afr[0], wf[0], Ad0);
    }
  } else {
    run_loads(w_begin + KPW, afr[1], wf[1], Ad1);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      run_compute(w_begin + r * KPW, afr[r & 1], wf[r & 1], (r & 1) ? Ad1 : Ad0);
      if (r + 2 < NR) run_loads(w_begin + (r + 2) * KPW, afr[r & 1], wf[r & 1], (r & 1) ? Ad1 : Ad0);
    }
  }
  // A_DMA: slots of k blocks past the share may still be filling; the workgroup's LDS must
  // not be released under them.
  if constexpr (ADMA) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0); expcnt and lgkmcnt left open

#pragma unroll
  for (int c = 0; c < CB; ++c) red[(wave * CB + c) * 64 + lane] = DEC_ACC2 ? acc[c][0] + acc[c][1] : acc[c][0];
  // Barrier without the release fence of __syncthreads(): that fence would also wait for
  // the clamped re-loads still in flight; the LDS writes above are what must land.
  __builtin_amdgcn_s_waitcnt(0xC07F);                // lgkmcnt(0): vmcnt and expcnt left open
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  const bool active = tid < CB * 64;
  const int c = tid >> 6, ln = tid & 63;
  f32x4 v[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
  if (active) {
    // every wave tile's read goes out before the first sum (summed in wave order as before):
    // read and summed one after another, the compiler kept two reads in flight
    f32x4 t[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) t[w] = red[(w * CB + c) * 64 + ln];
    __builtin_amdgcn_sched_barrier(0);
    v[0] = t[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) v[0] += t[w];
  }
  if (a.splits > 1) {
    if (!splitk_finish<1, NT>(a, group, split, CB * 256, active, v)) return;
  }
  if (!active || nb0 + c >= NB) return;
  const float alpha = qgemm::group_scaled(FMT) ? 1.0f : *a.alpha;
  const int n = (nb0 + c) * 16 + (ln & 15);
  const float bv = bias_of(a, n);
  // Every value is formed before the first store: a store counts as an outstanding memory
  // operation here, so a wait for the bias or alpha load placed between two stores also waited
  // for the stores before it (at M = 16, four write round trips in a row).
  // (the empty asm pins the four values ahead of the stores: the compiler would otherwise sink
  // each add into its store's branch)
  float o[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    o[r] = (qgemm::group_scaled(FMT) ? v[0][r] : v[0][r] * alpha) + bv;
    asm volatile("" : "+v"(o[r]));
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * (ln >> 4) + r;
    if (m < a.M) store_val(a, m, n, o[r]);
  }
}

template <int FMT, int G, int CB, int KPW, int NW, int AMODE, int NR>
bool launch_one(const Plan& pl, const KArgs& a, hipStream_t stream) {
  // five to eight overlapped runs only with A in DMA slots (A in registers or staged: at most four)
  if constexpr ((AMODE == qgemm::A_DMA && !qgemm::dec_dma_fits(NW, KPW, CB, NR)) || (NR > 4 && AMODE != qgemm::A_DMA)) {
    return false;                                    // not instantiated; never planned
  } else {
    // The instance's static LDS (slot sets, flags) plus the plan's dynamic region must fit the
    // workgroup limit: a larger request fails at dispatch, after the call has returned.
    static const size_t static_lds = [] {
      hipFuncAttributes at{};
      return hipFuncGetAttributes(&at, reinterpret_cast<const void*>(&qgemm_decode<FMT, G, CB, KPW, NW, AMODE, NR>)) ==
                     hipSuccess
                 ? at.sharedSizeBytes
                 : (size_t)qgemm::kMaxLds + 1;
    }();
    if (static_lds + (size_t)pl.lds_bytes > (size_t)qgemm::kMaxLds) return false;
    hipLaunchKernelGGL((qgemm_decode<FMT, G, CB, KPW, NW, AMODE, NR>), dim3(pl.grid_x, pl.grid_y), dim3(64 * NW),
                       pl.lds_bytes, stream, a.W, a.S, a.A, a.lut, a.M, a.N, a.K, a.kb_per_split, a);
    return true;
  }
}

template <int FMT, int G, int CB, int KPW, int NW, int AMODE>
bool launch_nr(const Plan& pl, const KArgs& a, hipStream_t stream) {
  switch (pl.nruns) {
    case 2: return launch_one<FMT, G, CB, KPW, NW, AMODE, 2>(pl, a, stream);
    case 3: return launch_one<FMT, G, CB, KPW, NW, AMODE, 3>(pl, a, stream);
    case 4: return launch_one<FMT, G, CB, KPW, NW, AMODE, 4>(pl, a, stream);
    case 5: return launch_one<FMT, G, CB, KPW, NW, AMODE, 5>(pl, a, stream);
    case 6: return launch_one<FMT, G, CB, KPW, NW, AMODE, 6>(pl, a, stream);
    case 7: return launch_one<FMT, G, CB, KPW, NW, AMODE, 7>(pl, a, stream);
    case 8: return launch_one<FMT, G, CB, KPW, NW, AMODE, 8>(pl, a, stream);
    default: return launch_one<FMT, G, CB, KPW, NW, AMODE, 1>(pl, a, stream);
  }
}

// Staged A always runs kDecodeWaves wavefronts; unstaged A with two or more column blocks
// runs kDecodeWavesWide (the plan's nw says which).
// Only the A path the build plans is instantiated (A_DIRECT only when built with the DMA path
// off, QGEMM_DEC_ADMA=0); a plan for the other one is refused.
template <int FMT, int G, int CB, int KPW, int NW>
bool launch_unstaged(const Plan& pl, const KArgs& a, hipStream_t stream) {
  constexpr int kPath = QGEMM_DEC_ADMA ? qgemm::A_DMA : qgemm::A_DIRECT;
  if (pl.amode != kPath) return false;
  return launch_nr<FMT, G, CB, KPW, NW, kPath>(pl, a, stream);
}
template <int FMT, int G, int CB, int KPW>
bool launch_cb(const Plan& pl, const KArgs& a, hipStream_t stream) {
  if (pl.amode == qgemm::A_STAGED) return launch_nr<FMT, G, CB, KPW, kDecodeWaves, qgemm::A_STAGED>(pl, a, stream);
  if (pl.amode == qgemm::A_STAGED_EARLY) {
    if constexpr (CB == 1 && KPW <= 5)
      return launch_nr<FMT, G, CB, KPW, kDecodeWaves, qgemm::A_STAGED_EARLY>(pl, a, stream);
    else
      return false;                                  // not instantiated; never planned
  }
  if constexpr (CB >= 2)
    return launch_unstaged<FMT, G, CB, KPW, kDecodeWavesWide>(pl, a, stream);
  else
    return launch_unstaged<FMT, G, CB, KPW, kDecodeWaves>(pl, a, stream);
}

template <int FMT, int G>
struct DecodeLauncher {
  static hipError_t run(const Plan& pl, const KArgs& a, hipStream_t stream) {
    bool ok = false;
    switch (pl.cb * 16 + pl.kpw) {
      case 16 + 8: ok = launch_cb<FMT, G, 1, 8>(pl, a, stream); break;
      case 16 + 5: ok = launch_cb<FMT, G, 1, 5>(pl, a, stream); break;
      case 16 + 4: ok = launch_cb<FMT, G, 1, 4>(pl, a, stream); break;
      case 16 + 2: ok = launch_cb<FMT, G, 1, 2>(pl, a, stream); break;
      case 16 + 1: ok = launch_cb<FMT, G, 1, 1>(pl, a, stream); break;
      case 32 + 4: ok = launch_cb<FMT, G, 2, 4>(pl, a, stream); break;
      case 32 + 2: ok = launch_cb<FMT, G, 2, 2>(pl, a, stream); break;
      case 32 + 1: ok = launch_cb<FMT, G, 2, 1>(pl, a, stream); break;
      case 48 + 2: ok = launch_cb<FMT, G, 3, 2>(pl, a, stream); break;
      case 48 + 1: ok = launch_cb<FMT, G, 3, 1>(pl, a, stream); break;
      case 64 + 2: ok = launch_cb<FMT, G, 4, 2>(pl, a, stream); break;
      case 64 + 1: ok = launch_cb<FMT, G, 4, 1>(pl, a, stream); break;
      default: ok = false;
    }
    if (!ok) return hipErrorInvalidConfiguration;
    return hipGetLastError();
  }
};

}  // namespace

// The instances of one format (QGEMM_FMT_UNIT): every group size it has (INT4, INT2, NF4:
// 32, 64, 128, 256; FP8 / FP4: none).  The source is compiled once per format, so that the
// many instances build in parallel; launch_decode dispatches to the format's unit.
template <int FMT>
hipError_t launch_decode_format(const Plan& pl, int group_size, const KArgs& a, hipStream_t stream) {
  if constexpr (qgemm::group_scaled(FMT)) {
    switch (group_size) {
      case 32: return DecodeLauncher<FMT, 32>::run(pl, a, stream);
      case 64: return DecodeLauncher<FMT, 64>::run(pl, a, stream);
      case 128: return DecodeLauncher<FMT, 128>::run(pl, a, stream);
      case 256: return DecodeLauncher<FMT, 256>::run(pl, a, stream);
      default: return hipErrorInvalidValue;
    }
  } else {
    return DecodeLauncher<FMT, 0>::run(pl, a, stream);
  }
}

#ifndef QGEMM_FMT_UNIT
#error "compile once per format with -DQGEMM_FMT_UNIT=<format>"
#endif
template hipError_t launch_decode_format<QGEMM_FMT_UNIT>(const Plan&, int, const KArgs&, hipStream_t);

}  // namespace dev
}  // namespace qgemm
