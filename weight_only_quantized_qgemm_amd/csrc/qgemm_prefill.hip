// The prefill kernel (MFMA tiles, any M) of the weight-only quantized GEMM on gfx950.
#include "qgemm_device.h"

namespace qgemm {
namespace dev {
namespace {

// ============================================================================= prefill
// Workgroup = WGM x WGN wavefronts; each wavefront owns TM x TN MFMA tiles (16 x 16), so
// the workgroup tile is (16 WGM TM) x (16 WGN TN); one 128-wide k block per step.
//
// A goes from HBM straight into LDS (buffer loads with the LDS-destination bit: no VGPR
// staging), in ST stages (two to eight), each its own array so that the compiler can tell
// the stage being read from the ones being filled.  A DMA load writes its 64 lanes' 16 bytes
// contiguously, so LDS rows cannot be padded; instead the 16-byte chunk c of tile row r
// is stored at chunk position c ^ (r & 15).  The MFMA A-fragment read (lane l: row l & 15,
// chunk 4t + l / 16) then touches 16 distinct positions per 16 lanes: no bank conflicts.
// The buffer resource covers the tile's valid rows only and the row sits in the range-
// checked per-lane offset (the k block in the scalar offset never leaves its row), so rows
// at or beyond M read as zero (and are never stored).
//
// Each wavefront loads its own packed weight fragments into registers (ST - BB k blocks
// ahead, like its A) and dequantizes each once per K step, reusing it for its TM row tiles; the
// dequantization of K step t + 1 is issued with the MFMAs of step t.  A fragments are
// read from LDS in units of RU row tiles, LA units ahead of the MFMAs that consume them.
// The weights enter each MFMA as its first operand and A as its second (both fragments
// have the same lane map), so the MFMA computes the transposed 16 x 16 tile: lane l holds
// output row l & 15, columns 4 (l >> 4) .. 4 (l >> 4) + 3, and the epilogue writes them
// with one 8-byte (16-bit output) or 16-byte (fp32) store.
// One barrier per BB k blocks: step k issues the weight loads of block k + ST - BB, computes
// block k while spreading the A DMA loads of that block over its first read units, and at the
// end of each window of BB blocks waits for its own loads and meets the other wavefronts at
// the barrier.  The loop is unrolled by ST so buffers and register sets rotate without copies; every
// load is unconditional (the last step re-loads its own block, never used) and
// sched_barrier pins the phase order (a load under a branch, or a consumer scheduled
// early, would make the wavefront wait for all outstanding loads).


#ifndef QGEMM_PF_DS
#define QGEMM_PF_DS 1
#endif
// wavefronts with no column inside N skip their MFMAs (0 turns it off)
#ifndef QGEMM_PF_IDLE
#define QGEMM_PF_IDLE 1
#endif
// One piece of work of a prefill workgroup: output tile (tm, tn), its k blocks
// [kb_begin, kb_end), and how the tile's sum is completed.  nslots == 1: this segment is the
// whole sum and writes the output.  Otherwise the tile's nslots contributors hand off fp32
// partials through slots base .. base + span - 1 (this one's is `my`), ticket `counter`; for
// split-K contributor i uses slot i (v0 < 0), for the stream-K tail contributor i is
// workgroup v0 + i, whose slot is 2 (v0 + i) + [the tile is not that workgroup's first].
struct PfSeg {
  int tm, tn, kb_begin, kb_end;
  int nslots, span, my, v0, t;
  unsigned* counter;
  float* base;
};

// Stream-K tail of the persistent schedule: the sk_units k blocks of the tail tiles are cut
// into P contiguous ranges of q or q + 1 units (the first r ranges are one longer; q and r are
// computed on the host), range v = [start(v), start(v + 1)).  owner(x) is the workgroup whose
// range holds unit x.  All of it fits 32-bit arithmetic (sk_units < 2^31).
__device__ __forceinline__ int sk_start(int v, int q, int r) { return v * q + min(v, r); }
__device__ __forceinline__ int sk_owner(int x, int q, int r) {
  const int big = r * (q + 1);                       // units in the r longer ranges
  return x < big ? x / (q + 1) : r + (x - big) / q;  // q > 0 whenever x >= big
}

// The item-th segment of this workgroup (false when it has no more).  Without persistence a
// workgroup owns one tile (blockIdx.x) and one K slice (blockIdx.y).  With it, workgroup w of
// the a.persist resident ones first takes the whole tiles w, w + P, ... below dp_tiles (the
// same XCD-aware walk of tile ids as the one-tile launch: id b runs on XCD b mod 8 in both,
// since P is a multiple of 8), then its contiguous range of the tail's k blocks, one segment
// per tail tile the range touches.
template <bool PERSIST>
__device__ __forceinline__ bool pf_next(const KArgs& a, int item, int KB, int tile_elems, PfSeg& g) {
  if constexpr (!PERSIST) {
    const int tile = blockIdx.x, split = blockIdx.y;
    pf_tile_of(tile, gridDim.x, a.tiles_n, g.tm, g.tn);
    g.kb_begin = split * a.kb_per_split;
    g.kb_end = min(KB, g.kb_begin + a.kb_per_split);
    g.nslots = a.splits;
    g.span = a.splits;
    g.my = split;
    g.v0 = -1;
    g.t = tile;
    g.counter = a.counters + tile;
    g.base = a.partials + (size_t)tile * a.splits * tile_elems;
    return item == 0;
  } else {
    const int P = a.persist, w = blockIdx.x;
    const int ndp = w < a.dp_tiles ? (a.dp_tiles - w + P - 1) / P : 0;
    if (item < ndp) {
      pf_tile_of(w + item * P, a.tiles_total, a.tiles_n, g.tm, g.tn);
      g.kb_begin = 0;
      g.kb_end = KB;
      g.nslots = 1;
      return true;
    }
    const int q = a.sk_q, r = a.sk_r;
    const int u0 = sk_start(w, q, r), u1 = sk_start(w + 1, q, r);
    const int t0 = u0 / KB;
    const int t = t0 + (item - ndp);
    const int s0 = max(u0, t * KB), s1 = min(u1, (t + 1) * KB);
    if (s0 >= s1) return false;
    g.kb_begin = s0 - t * KB;
    g.kb_end = s1 - t * KB;
    const int v0 = sk_owner(t * KB, q, r), vl = sk_owner((t + 1) * KB - 1, q, r);
    g.nslots = vl - v0 + 1;
    g.span = 2 * g.nslots;
    g.my = 2 * (w - v0) + (t == t0 ? 0 : 1);
    g.v0 = v0;
    g.t = t;
    g.counter = a.counters + t;
    g.base = a.partials + (size_t)(2 * v0) * tile_elems;
    pf_tile_of(a.dp_tiles + t, a.tiles_total, a.tiles_n, g.tm, g.tn);
    return true;
  }
}

template <int FMT, int G, int WGM, int WGN, int TM, int TN, int RU, int LA, int ST, int BB, bool PERSIST>
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
  static_assert(ST >= 2 && ST <= 8, "two to eight A stages");
  // BB k blocks between two workgroup barriers; block kb + D is loaded while block kb is
  // computed, into the stage block kb - BB left, which every wavefront finished reading before
  // the last barrier.
  static_assert(BB >= 1 && ST % BB == 0 && ST > BB, "whole barrier windows per stage ring");
  constexpr int D = ST - BB;
  // Each stage is its own array, so that the compiler can tell the buffer being read from
  // the ones being filled (it would otherwise wait for every DMA load before a read).
  __shared__ __attribute__((aligned(1024))) unsigned char As0[BM * ROWB];
  __shared__ __attribute__((aligned(1024))) unsigned char As1[BM * ROWB];
  __shared__ __attribute__((aligned(1024))) unsigned char As2[ST > 2 ? BM * ROWB : 16];
  __shared__ __attribute__((aligned(1024))) unsigned char As3[ST > 3 ? BM * ROWB : 16];
  __shared__ __attribute__((aligned(1024))) unsigned char As4[ST > 4 ? BM * ROWB : 16];
  __shared__ __attribute__((aligned(1024))) unsigned char As5[ST > 5 ? BM * ROWB : 16];
  __shared__ __attribute__((aligned(1024))) unsigned char As6[ST > 6 ? BM * ROWB : 16];
  __shared__ __attribute__((aligned(1024))) unsigned char As7[ST > 7 ? BM * ROWB : 16];
  auto stage = [&](int i) -> unsigned char* {
    return i == 0 ? As0 : i == 1 ? As1 : i == 2 ? As2 : i == 3 ? As3 : i == 4 ? As4 : i == 5 ? As5 : i == 6 ? As6 : As7;
  };
  // With three or more stages the first LA read units of the next block are read during
  // the current one (after its own last reads), so a block starts with its A fragments in
  // flight instead of behind the barrier; the unit ring must then line up across blocks.
  constexpr bool XPF = ST >= 3 && NU % (LA + 1) == 0;
  // Vector-memory instructions per k block per wavefront: NDMA A loads and, per weight
  // column block, two (the fragment and its scales, or FP8's two fragment halves).  At a
  // barrier the next window of BB blocks must have landed (with XPF one more, since the last
  // step of the window reads ahead into it) while the D - BB (- 1) blocks after them may
  // still be in flight; loads complete in issue order, so that is this many pending.
  static_assert(ST - 2 * BB - (XPF ? 1 : 0) >= 0, "the next window must be loaded before its barrier");
  constexpr int PEND = (ST - 2 * BB - (XPF ? 1 : 0)) * (NDMA + 2 * TN);
  static_assert(PEND <= 63, "vmcnt counts at most 63 outstanding loads");
  // s_waitcnt immediate: vmcnt = PEND (bits 3:0 and 15:14), expcnt and lgkmcnt left open.
  // Through the builtin (not inline asm) the compiler's own wait insertion knows of it.
  constexpr int WAIT_PEND = (PEND & 15) | (7 << 4) | (15 << 8) | ((PEND >> 4) << 14);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  Lut lut;                                           // NF4 code book (wavefront-uniform)
  load_lut<FMT>(a, lut);
  const int KB = a.K >> 7, NB = a.N >> 4;
  for (int item = 0; item < (PERSIST ? 0x7fffffff : 1); ++item) {
  PfSeg sg;
  if (!pf_next<PERSIST>(a, item, KB, BM * BN, sg)) break;
  if (item > 0) {
    // the previous segment's output stores and LDS reads are done before this one's loads
    // and DMA writes start (the load counts below assume nothing older is outstanding)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  const int tm = sg.tm, tn = sg.tn;
  const int m0 = tm * BM, n0 = tn * BN;
  const int kb_begin = sg.kb_begin, kb_end = sg.kb_end;

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

  // A-fragment read units: unit u of a k block sits in slot u % (LA + 1); with XPF the
  // first LA units of a block are read by the step before it.
  u32x4 af[LA + 1][RU];
  auto read_unit = [&](const unsigned char* As, int u, u32x4 (&dst)[RU]) {
    const int t = u / TU, i0 = (u % TU) * RU;
#pragma unroll
    for (int r = 0; r < RU; ++r) dst[r] = *reinterpret_cast<const u32x4*>(As + aoff[t] + (i0 + r) * 16 * ROWB);
  };

  // A wavefront whose column blocks all lie past N (the last tile column of an N that is not
  // a multiple of the tile width) computes nothing; it still issues its share of the A DMA
  // and its (clamped) weight loads, so the load counts the waits rely on stay the same.
  const bool idle = QGEMM_PF_IDLE && (n0 >> 4) + TN * wn >= NB;
  // Computes one k block from As / wf while issuing the DMA loads of a later one (into
  // Ad), DS read units apart: issued all at once they would fill the memory pipeline's
  // queue and stall the wavefront's MFMAs behind it.  An is the stage of the next block.
  auto compute = [&](const unsigned char* As, const WFrag<FMT> (&wf)[TN], int kb_next, unsigned char* Ad,
                     const unsigned char* An) {
    if (idle) {
#pragma unroll
      for (int i = 0; i < NDMA; ++i) load_a(kb_next, Ad, i);
      __builtin_amdgcn_sched_barrier(0);
      return;
    }
    float fs[TN][4];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int t = 0; t < 4; ++t) fs[j][t] = 0.f;
      if constexpr (FMT == qgemm::FMT_FP4) fp4_scales(wf[j].s[0], fs[j]);
    }
    u32x4 b[2][TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) b[0][j] = bfrag<FMT, G>(wf[j], 0, fs[j], lut);
    if constexpr (!XPF) {
#pragma unroll
      for (int u = 0; u < LA && u < NU; ++u) read_unit(As, u, af[u]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int t = u / TU, i0 = (u % TU) * RU;
      if (u + LA < NU) read_unit(As, u + LA, af[(u + LA) % (LA + 1)]);
      else if constexpr (XPF) read_unit(An, u + LA - NU, af[(u + LA) % (LA + 1)]);
      if (u % DS == 0 && u / DS < NDMA) load_a(kb_next, Ad, u / DS);
      __builtin_amdgcn_sched_barrier(0);   // later units' reads go out before this unit's MFMAs
      if (i0 + RU == TM && t < 3) {
#pragma unroll
        for (int j = 0; j < TN; ++j) b[(t + 1) & 1][j] = bfrag<FMT, G>(wf[j], t + 1, fs[j], lut);
      }
#pragma unroll
      for (int r = 0; r < RU; ++r)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i0 + r][j] = mfma<FMT>(b[t & 1][j], af[u % (LA + 1)][r], acc[i0 + r][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Prologue: blocks kb_begin .. kb_begin + D - 1 into stages 0 .. D - 1.  Step kb computes
  // stage kb mod ST while loading block kb + D into the stage block kb - BB was read from.
  WFrag<FMT> w[ST][TN];
#pragma unroll
  for (int s = 0; s < D; ++s) {
    const int kb = min(kb_begin + s, kb_end - 1);
    load_w(kb, w[s]);
#pragma unroll
    for (int i = 0; i < NDMA; ++i) load_a(kb, stage(s), i);
  }
  __builtin_amdgcn_s_waitcnt(WAIT_PEND);
  barrier_no_fence();
  if constexpr (XPF) {
#pragma unroll
    for (int u = 0; u < LA && u < NU; ++u) read_unit(stage(0), u, af[u]);
  }

  for (int kb = kb_begin; kb < kb_end; kb += ST) {
#pragma unroll
    for (int j = 0; j < ST; ++j) {
      const int sn = (j + D) % ST;                     // stage that receives block kn
      const int kn = min(kb + j + D, kb_end - 1);
      load_w(kn, w[sn]);
      __builtin_amdgcn_sched_barrier(0);
      compute(stage(j), w[j], kn, stage(sn), stage((j + 1) % ST));
      if ((j + 1) % BB == 0) {
        __builtin_amdgcn_s_waitcnt(WAIT_PEND);
        barrier_no_fence();
      }
      if (kb + j + 1 >= kb_end) break;
    }
  }
  // clamped re-loads past the last block may still be writing LDS
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  f32x4 v[TM * TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) v[TN * i + j] = acc[i][j];
  if (sg.nslots > 1) {
    const int v0 = sg.v0, t = sg.t;
    auto rel = [&](int i) {
      if constexpr (!PERSIST) return i;              // split-K
      else                                           // stream-K: workgroup v0 + i's slot for tail tile t
        return 2 * i + (t == sk_start(v0 + i, a.sk_q, a.sk_r) / KB ? 0 : 1);
    };
    if (!fixup_finish<TM * TN, NT>(sg.counter, sg.base, sg.span, sg.my, sg.nslots, rel, BM * BN, true, v))
      continue;                                      // another contributor completes this tile
  }
  const float alpha = qgemm::group_scaled(FMT) ? 1.0f : *a.alpha;
  auto scaled = [&](f32x4 x) {
    if constexpr (!qgemm::group_scaled(FMT)) {
      x[0] *= alpha;
      x[1] *= alpha;
      x[2] *= alpha;
      x[3] *= alpha;
    }
    return x;
  };
  if (a.out_dtype == QGEMM_DT_F32) {                 // fp32 output: 16-byte stores from the fragments
    // Every value is formed before the first store (the empty asm keeps the compiler from
    // sinking the adds into the stores' branches): a store counts as an outstanding memory
    // operation, so a wait for a bias load between two stores would also wait for the stores
    // before it.
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int nb = min((n0 >> 4) + TN * wn + j, NB - 1);    // a block past N is formed, never stored
      const f32x4 bv = bias4_of(a, nb * 16 + 4 * (lane >> 4));
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        f32x4 x = scaled(v[TN * i + j]);
        x = f32x4{x[0] + bv[0], x[1] + bv[1], x[2] + bv[2], x[3] + bv[3]};
        asm volatile("" : "+v"(x));
        v[TN * i + j] = x;
      }
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int nb = (n0 >> 4) + TN * wn + j;
      if (nb >= NB) continue;
      const int n = nb * 16 + 4 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int m = m0 + 16 * TM * wm + 16 * i + (lane & 15);
        if (m < a.M) *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + (size_t)m * a.N + n) = v[TN * i + j];
      }
    }
    continue;
  }

  // 16-bit output: the tile goes through the (now idle) A stages in LDS, row-major, so that
  // each store instruction writes whole rows.  Tile row R sits in stage R / RPA at row
  // R % RPA; its 16-byte chunk c at position c ^ (R & 15), which keeps both the fragment
  // writes (16 rows per instruction) and the row reads free of bank conflicts.
  constexpr int OROW = BN * 2;                       // bytes of one output row of the tile
  constexpr int OCH = OROW / 16;                     // 16-byte chunks per row
  constexpr int RPA = BM * ROWB / OROW;              // tile rows per stage
  constexpr int RPP = NT / OCH;                      // tile rows per store pass
  static_assert(OCH >= 16 && RPA % 16 == 0 && (BM + RPA - 1) / RPA <= ST && BM % RPP == 0,
                "the output tile must fit the A stages in whole swizzled rows");
  __syncthreads();                                   // every wavefront is done reading A
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int nb = (n0 >> 4) + TN * wn + j;
    if (nb >= NB) continue;                          // never stored
    const f32x4 bv = bias4_of(a, nb * 16 + 4 * (lane >> 4));
    const int c = 2 * (TN * wn + j) + (lane >> 5);   // chunk of columns 4 (lane >> 4) ..
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int R = 16 * TM * wm + 16 * i + (lane & 15);
      unsigned char* row = stage(R / RPA) + (R % RPA) * OROW;
      *reinterpret_cast<u32x2*>(row + 16 * (c ^ (R & 15)) + 8 * ((lane >> 4) & 1)) =
          pack4_out16(a, scaled(v[TN * i + j]), bv);
    }
  }
  __syncthreads();
  const int c = threadIdx.x % OCH;
  const bool col_ok = (n0 >> 4) + (c >> 1) < NB;     // a 16-column block is two chunks
  unsigned char* out = static_cast<unsigned char*>(a.out) + (size_t)n0 * 2 + 16 * c;
#pragma unroll
  for (int p = 0; p < BM / RPP; ++p) {
    const int R = p * RPP + threadIdx.x / OCH;
    const u32x4 x = *reinterpret_cast<const u32x4*>(stage(R / RPA) + (R % RPA) * OROW + 16 * (c ^ (R & 15)));
    if (col_ok && m0 + R < a.M) *reinterpret_cast<u32x4*>(out + (size_t)(m0 + R) * a.N * 2) = x;
  }
  }   // segments
}

template <int FMT, int G, int WGM, int WGN, int TM, int TN, int RU, int LA, int ST, int BB>
void launch_shape(const Plan& pl, const KArgs& a, hipStream_t stream) {
  if (pl.persist)
    hipLaunchKernelGGL((qgemm_prefill<FMT, G, WGM, WGN, TM, TN, RU, LA, ST, BB, true>), dim3(pl.grid_x, pl.grid_y),
                       dim3(64 * WGM * WGN), 0, stream, a);
  else
    hipLaunchKernelGGL((qgemm_prefill<FMT, G, WGM, WGN, TM, TN, RU, LA, ST, BB, false>), dim3(pl.grid_x, pl.grid_y),
                       dim3(64 * WGM * WGN), 0, stream, a);
}

template <int FMT, int G>
struct PrefillLauncher {
  static hipError_t run(const Plan& pl, const KArgs& a, hipStream_t stream) {
    constexpr PfShape L = kPfLarge, M = kPfMedium, S = kPfSmall;
    if (pl.bm == pf_bm(L))
      launch_shape<FMT, G, L.wgm, L.wgn, L.tm, L.tn, L.ru, L.la, L.st, L.bb>(pl, a, stream);
    else if (pl.bm == pf_bm(M))
      launch_shape<FMT, G, M.wgm, M.wgn, M.tm, M.tn, M.ru, M.la, M.st, M.bb>(pl, a, stream);
    else
      launch_shape<FMT, G, S.wgm, S.wgn, S.tm, S.tn, S.ru, S.la, S.st, S.bb>(pl, a, stream);
    return hipGetLastError();
  }
};

}  // namespace

// The instances of one format (QGEMM_FMT_UNIT): every group size it has (INT4, INT2, NF4:
// 32, 64, 128, 256; FP8 / FP4: none).  The source is compiled once per format, so that the
// many instances build in parallel; launch_prefill dispatches to the format's unit.
template <int FMT>
hipError_t launch_prefill_format(const Plan& pl, int group_size, const KArgs& a, hipStream_t stream) {
  if constexpr (qgemm::group_scaled(FMT)) {
    switch (group_size) {
      case 32: return PrefillLauncher<FMT, 32>::run(pl, a, stream);
      case 64: return PrefillLauncher<FMT, 64>::run(pl, a, stream);
      case 128: return PrefillLauncher<FMT, 128>::run(pl, a, stream);
      case 256: return PrefillLauncher<FMT, 256>::run(pl, a, stream);
      default: return hipErrorInvalidValue;
    }
  } else {
    return PrefillLauncher<FMT, 0>::run(pl, a, stream);
  }
}

#ifndef QGEMM_FMT_UNIT
#error "compile once per format with -DQGEMM_FMT_UNIT=<format>"
#endif
template hipError_t launch_prefill_format<QGEMM_FMT_UNIT>(const Plan&, int, const KArgs&, hipStream_t);

}  // namespace dev
}  // namespace qgemm
