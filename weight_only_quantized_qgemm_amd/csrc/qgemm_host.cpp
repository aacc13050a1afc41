// Host side of the library: status text, validation, launch planning, the offline
// quantizer and the offline packer.  Nothing in this file touches the GPU.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "qgemm_internal.h"

namespace qgemm {

static_assert(sizeof(qgemm_problem_t) == 56, "qgemm_problem_t layout is part of the ABI");

static thread_local std::string t_last_error;

qgemm_status_t fail(qgemm_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  t_last_error = buf;
  return st;
}

void clear_error() { t_last_error.clear(); }

static const char* dtype_name(int d) {
  switch (d) {
    case QGEMM_DT_F16: return "F16";
    case QGEMM_DT_BF16: return "BF16";
    case QGEMM_DT_F32: return "F32";
    case QGEMM_DT_INT4: return "INT4";
    case QGEMM_DT_FP8_E4M3: return "FP8_E4M3";
    case QGEMM_DT_FP4_E2M1: return "FP4_E2M1";
    case QGEMM_DT_INT2: return "INT2";
    case QGEMM_DT_NF4: return "NF4";
    default: return "?";
  }
}

Format format_of(const qgemm_problem_t* p) {
  if (p->w_dtype == QGEMM_DT_INT4) return FMT_INT4;
  if (p->w_dtype == QGEMM_DT_INT2) return FMT_INT2;
  if (p->w_dtype == QGEMM_DT_NF4) return FMT_NF4;
  if (p->w_dtype == QGEMM_DT_FP8_E4M3) return p->a_dtype == QGEMM_DT_F16 ? FMT_FP8H : FMT_FP8;
  return FMT_FP4;
}

// Each of M, N, K is limited to 2^24; the kernels address A, W, out and the workspace with
// 64-bit offsets, and grids are checked against the 2^31 - 1 workgroup limit when planned.
static const int64_t kMaxDim = int64_t(1) << 24;

qgemm_status_t validate_problem(const qgemm_problem_t* p) {
  if (!p) return fail(QGEMM_ERR_INVALID_ARGUMENT, "problem is NULL");
  for (int d : {p->a_dtype, p->w_dtype, p->out_dtype})
    if (d < QGEMM_DT_F16 || d > QGEMM_DT_NF4)
      return fail(QGEMM_ERR_INVALID_ARGUMENT, "dtype value %d is not a qgemm_dtype_t", d);
  if (p->scale_layout < QGEMM_SCALE_GROUP_F16 || p->scale_layout > QGEMM_SCALE_GROUP_F16_LUT16)
    return fail(QGEMM_ERR_INVALID_ARGUMENT, "scale_layout %d is not a qgemm_scale_layout_t", p->scale_layout);
  if (p->M < 0 || p->M > kMaxDim)
    return fail(QGEMM_ERR_INVALID_ARGUMENT, "M must be in [0, %lld], got %lld", (long long)kMaxDim, (long long)p->M);
  if (p->N < 16 || p->N % 16 || p->N > kMaxDim)
    return fail(QGEMM_ERR_INVALID_ARGUMENT, "N must be a positive multiple of 16 (<= %lld), got %lld",
                (long long)kMaxDim, (long long)p->N);
  if (p->K < 128 || p->K % 128 || p->K > kMaxDim)
    return fail(QGEMM_ERR_INVALID_ARGUMENT, "K must be a positive multiple of 128 (<= %lld), got %lld",
                (long long)kMaxDim, (long long)p->K);

  const int a = p->a_dtype, w = p->w_dtype, o = p->out_dtype, sl = p->scale_layout, g = p->group_size;
  if (w == QGEMM_DT_INT4 || w == QGEMM_DT_INT2 || w == QGEMM_DT_NF4) {
    const char* wn = dtype_name(w);
    const int want = w == QGEMM_DT_NF4 ? QGEMM_SCALE_GROUP_F16_LUT16 : QGEMM_SCALE_GROUP_F16;
    if (a != QGEMM_DT_F16 || sl != want || (o != QGEMM_DT_F16 && o != QGEMM_DT_F32))
      return fail(QGEMM_ERR_UNSUPPORTED, "%s weights need a_dtype F16, scale_layout %s and out_dtype F16 or F32; "
                  "got a=%s out=%s scale_layout=%d", wn, w == QGEMM_DT_NF4 ? "GROUP_F16_LUT16" : "GROUP_F16",
                  dtype_name(a), dtype_name(o), sl);
    if (g != 32 && g != 64 && g != 128 && g != 256)
      return fail(QGEMM_ERR_UNSUPPORTED, "%s group_size must be 32, 64, 128 or 256, got %d", wn, g);
    if (p->K % g) return fail(QGEMM_ERR_INVALID_ARGUMENT, "K (%lld) must be a multiple of group_size (%d)", (long long)p->K, g);
  } else if (w == QGEMM_DT_FP8_E4M3) {
    // mm_bf16_fp8 and mm_fp16_fp8: the output is the activations' 16-bit type or fp32
    if ((a != QGEMM_DT_BF16 && a != QGEMM_DT_F16) || sl != QGEMM_SCALE_TENSOR_F32 || (o != a && o != QGEMM_DT_F32))
      return fail(QGEMM_ERR_UNSUPPORTED, "FP8_E4M3 weights need a_dtype BF16 or F16, scale_layout TENSOR_F32 and out_dtype "
                  "a_dtype or F32; got a=%s out=%s scale_layout=%d", dtype_name(a), dtype_name(o), sl);
    if (g != 0) return fail(QGEMM_ERR_INVALID_ARGUMENT, "FP8_E4M3 takes group_size 0 (per-tensor scale), got %d", g);
  } else if (w == QGEMM_DT_FP4_E2M1) {
    if (a != QGEMM_DT_BF16 || sl != QGEMM_SCALE_BLOCK16_E4M3 || (o != QGEMM_DT_BF16 && o != QGEMM_DT_F32))
      return fail(QGEMM_ERR_UNSUPPORTED, "FP4_E2M1 weights need a_dtype BF16, scale_layout BLOCK16_E4M3 and out_dtype BF16 or F32; "
                  "got a=%s out=%s scale_layout=%d", dtype_name(a), dtype_name(o), sl);
    if (g != 16) return fail(QGEMM_ERR_INVALID_ARGUMENT, "FP4_E2M1 takes group_size 16 (one e4m3 scale per 16 K), got %d", g);
  } else {
    return fail(QGEMM_ERR_UNSUPPORTED, "w_dtype %s is not a weight format (INT4, INT2, NF4, FP8_E4M3, FP4_E2M1)", dtype_name(w));
  }

  if (p->kernel_hint < QGEMM_KERNEL_AUTO || p->kernel_hint > QGEMM_KERNEL_PREFILL_TRANSFORM)
    return fail(QGEMM_ERR_INVALID_ARGUMENT, "kernel_hint must be 0 to 4, got %d", p->kernel_hint);
  if (p->kernel_hint == QGEMM_KERNEL_PREFILL_TRANSFORM && p->tile_hint != 0 && p->tile_hint != pf_bm(kPfSmall))
    return fail(QGEMM_ERR_INVALID_ARGUMENT, "kernel_hint PREFILL_TRANSFORM has the %d x %d tile only; tile_hint must "
                "be 0 or %d, got %d", pf_bm(kPfSmall), pf_bn(kPfSmall), pf_bm(kPfSmall), p->tile_hint);
  if (p->kernel_hint == QGEMM_KERNEL_PREFILL_STREAMK && p->split_k_hint != 0)
    return fail(QGEMM_ERR_INVALID_ARGUMENT, "kernel_hint PREFILL_STREAMK splits K itself; split_k_hint must be 0, got %d",
                p->split_k_hint);
  if (p->kernel_hint == QGEMM_KERNEL_DECODE && p->M > 16)
    return fail(QGEMM_ERR_INVALID_ARGUMENT, "kernel_hint DECODE needs M <= 16, got M=%lld", (long long)p->M);
  if (p->split_k_hint < 0 || p->split_k_hint > 64)
    return fail(QGEMM_ERR_INVALID_ARGUMENT, "split_k_hint must be in [0, 64], got %d", p->split_k_hint);
  if (p->split_k_hint > p->K / 128)
    return fail(QGEMM_ERR_INVALID_ARGUMENT, "split_k_hint %d exceeds the %lld 128-wide K blocks",
                p->split_k_hint, (long long)(p->K / 128));
  const bool decode = p->kernel_hint == QGEMM_KERNEL_DECODE || (p->kernel_hint == QGEMM_KERNEL_AUTO && p->M <= 16);
  if (decode && (p->tile_hint < 0 || p->tile_hint > 4))
    return fail(QGEMM_ERR_INVALID_ARGUMENT, "tile_hint for the decode kernel must be 0 to 4, got %d", p->tile_hint);
  if (!decode && p->tile_hint != 0 && p->tile_hint != pf_bm(kPfSmall) && p->tile_hint != pf_bm(kPfMedium) &&
      p->tile_hint != pf_bm(kPfLarge))
    return fail(QGEMM_ERR_INVALID_ARGUMENT, "tile_hint for the prefill kernel must be 0, %d, %d or %d, got %d",
                pf_bm(kPfSmall), pf_bm(kPfMedium), pf_bm(kPfLarge), p->tile_hint);
  return QGEMM_OK;
}

// ----------------------------------------------------------------------------- planning
static int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// The chip has 256 compute units; grids are sized against that.
static const int kCUs = 256;

static void finish_split(Plan* pl, int kblocks, int requested) {
  int s = requested > 0 ? requested : pl->splits;
  if (s < 1) s = 1;
  if (s > kblocks) s = kblocks;
  pl->kb_per_split = ceil_div(kblocks, s);
  pl->splits = ceil_div(kblocks, pl->kb_per_split);   // no empty split
}

qgemm_status_t make_plan(const qgemm_problem_t* p, Plan* pl) {
  std::memset(pl, 0, sizeof(*pl));
  pl->fmt = format_of(p);
  if (p->M == 0) return QGEMM_OK;                    // empty product: no launch, no workspace
  const int kblocks = (int)(p->K / 128);
  const int nblocks = (int)(p->N / 16);
  const bool decode = p->kernel_hint == QGEMM_KERNEL_DECODE || (p->kernel_hint == QGEMM_KERNEL_AUTO && p->M <= 16);
  if (decode) {
    pl->kind = KIND_DECODE;
    // A is staged in LDS (at most 32 KiB per workgroup) when M is small: the MFMA fragment
    // loads would otherwise fetch each A value many times.  With larger M the rows are
    // distinct and fragments are loaded directly.
#ifndef QGEMM_DEC_ASTAGE_M
#define QGEMM_DEC_ASTAGE_M 4
#endif
    pl->astage = p->M <= QGEMM_DEC_ASTAGE_M;
    // Column blocks per workgroup.  Every workgroup reads all M x K of A once, so wider
    // workgroups cut A traffic; narrower ones put more compute units to work.  M <= 4 (A
    // staged per wavefront): one block each up to three workgroups per compute unit, two
    // beyond (M = 4: N = 4096 5.4 vs 6.2 us, N = 11008 8.4 vs 9.3 us, N = 14336 10.7 vs
    // 9.8 us).  Larger M: the fewest blocks (1 to 4) that keep the grid within one
    // workgroup per compute unit.
    int cb = 1;
    if (p->M > 4) {
      while (cb < 4 && ceil_div(nblocks, cb) > kCUs) ++cb;
    } else if (p->M > 1 && nblocks > 3 * kCUs) {
      cb = 2;
    }
    pl->cb = p->tile_hint ? p->tile_hint : cb;
    pl->nw = !pl->astage && pl->cb >= 2 ? kDecodeWavesWide : kDecodeWaves;
    const int groups = ceil_div(nblocks, pl->cb);
    // K is split only when needed to bound what a workgroup stages in LDS (its A slice and
    // its scales), or when the output alone gives fewer than 128 workgroups (a split-K
    // hand-off costs three dependent memory round trips); every wavefront keeps at least
    // one k block.
    // Each wavefront stages its own share (ceil(kb / waves) k blocks) of A and of the scales.
    auto staged_ok = [&](int kb) {
      const int share = ceil_div(kb, pl->nw);
      return (!pl->astage || 2 * 128 * p->M * (int64_t)share * pl->nw <= kDecodeMaxA) &&
             (!pl->astage ||
              (int64_t)pl->cb * dec_scale_span(pl->fmt, p->group_size, share) * pl->nw <= kDecodeMaxScales);
    };
    int max_kb = kblocks;
    while (max_kb > 1 && !staged_ok(max_kb)) --max_kb;
    int s = 1;
    while (ceil_div(kblocks, s) > max_kb) ++s;
    while (groups * s < kCUs / 2 && kblocks / (s * 2) >= pl->nw) s *= 2;
    pl->splits = s;
    finish_split(pl, kblocks, p->split_k_hint);
    if (pl->kb_per_split > max_kb)
      return fail(QGEMM_ERR_INVALID_ARGUMENT, "split_k_hint %d leaves %d k blocks per slice; the decode kernel "
                  "stages at most %d at M=%lld", p->split_k_hint, pl->kb_per_split, max_kb, (long long)p->M);
    // Each wavefront owns ceil(kb_per_split / waves) consecutive k blocks, streamed in runs
    // of KPW (at most 8 weight blocks in flight per wavefront): the whole share in one run
    // when an instance exists for it, else the largest instance below.  A share longer
    // than one run alternates two register sets, each KPW x (4 A fragments when A is loaded
    // straight into registers + CB weight fragments of 5 registers, FP8 8); the run is
    // shortened until both sets fit in 210 registers (measured: more spills).
    const int share = ceil_div(pl->kb_per_split, pl->nw);
    static const int kRuns[] = {8, 5, 4, 2, 1};            // instantiated KPW values
    auto instantiated = [&](int k) {
      return k * pl->cb <= 8 && (k != 5 || pl->cb == 1) && (k != 8 || pl->cb == 1);
    };
    auto choose_runs = [&](int amode, int kmax) {
      auto fits_twice = [&](int k) {
        const int wregs = fp8_weights(pl->fmt) ? 8 : 5;
        const int budget = pl->fmt == FMT_NF4 ? 202 : 210;   // NF4 keeps its code book in 8 registers
        return 2 * k * ((amode == A_DIRECT ? 16 : 0) + pl->cb * wregs) <= budget;
      };
      pl->kpw = 1;
      for (int k : kRuns)
        if (k <= kmax && instantiated(k) && k <= share && (k == share || (k < share && fits_twice(k)))) {
          pl->kpw = k;
          break;
        }
      const int runs = ceil_div(share, pl->kpw);
      // overlapped runs are unrolled at compile time: up to four, or eight with A in DMA slots
      // (M = 16 N = 11008 K = 8192 15.2 -> 12.9 us, M = 8 N = 10240 K = 5120 10.6 -> 8.7 us
      // against runs one after another)
      pl->nruns = runs >= 2 && runs <= (amode == A_DMA ? 8 : 4) ? runs : 1;
      pl->amode = amode;
      pl->lds_bytes = dec_lds_bytes(pl->fmt, p->group_size, (int)p->M, share, pl->cb, amode, pl->nw);
    };
    // Above the staging limit A goes through buffer-to-LDS DMA when its slots (one or two sets
    // of KPW k blocks per wavefront, next to the wave tiles) fit in LDS: a DMA load reads 256
    // contiguous bytes from each of 4 rows (8 whole cache lines) where a fragment load reads
    // 64 bytes from each of 16 rows (16 half lines), for the same kilobyte (M = 16: N = 4096
    // 6.9 -> 5.5 us, N = 11008 9.1 -> 8.3 us; FP4 8192 x 8192 16.4 -> 13.0 us).
    if (pl->astage) {
      choose_runs(A_STAGED, 8);
      if (pl->cb == 1 && pl->kpw <= 5 && (int64_t)groups * pl->splits <= kCUs) pl->amode = A_STAGED_EARLY;
    } else {
      // Runs are shortened until the slots fit (M = 16, N = 4096: K = 8192 11.6 -> 8.5 us with
      // runs of 2 instead of direct runs of 8, K = 14336 18.5 -> 12.4 us); runs of one k block
      // always fit (two sets of 8 x 4 KiB at most).
      choose_runs(QGEMM_DEC_ADMA ? A_DMA : A_DIRECT, 8);
      while (pl->amode == A_DMA && pl->kpw > 1 && !dec_dma_fits(pl->nw, pl->kpw, pl->cb, pl->nruns))
        choose_runs(A_DMA, pl->kpw - 1);
      if (pl->amode == A_DMA && !dec_dma_fits(pl->nw, pl->kpw, pl->cb, pl->nruns))
        return fail(QGEMM_ERR_UNSUPPORTED, "decode A slots of %d wavefronts x %d column blocks do not fit in LDS",
                    pl->nw, pl->cb);
    }
    pl->grid_x = (unsigned)groups;
    pl->grid_y = (unsigned)pl->splits;
    pl->tiles = groups;
    pl->tile_elems = pl->cb * 256;
  } else {
    pl->kind = KIND_PREFILL;
    // Tile shape and K split: the pair that minimises a time model of the launch, in
    // microseconds measured on MI355X: rounds of the grid over the CUs x (k blocks per slice
    // + pipeline fill) x the tile's time per k block under full load, plus, when split, the
    // fp32 partial tiles written and read back at HBM speed and one dependent partial read
    // per slice by the workgroup that finishes each tile.  The medium tile does a quarter of
    // the large tile's work per k block in about 0.38 of its time, so it wins whenever it
    // fills the CUs and the large tile cannot (e.g. M = 512..1024 at N = 4096, or
    // M = 2048 at N = 10240); the large one wins once both fill several rounds.  The small
    // tile does half the medium tile's work in about 0.62 of its time (the weight fragments
    // it dequantizes are the same), so it wins where rows are few: M <= 64 always, and up to
    // a few hundred rows when the medium tile would leave CUs idle or need a deep split.
    // A tile is only a candidate when M exceeds the next smaller tile's rows.
    struct Cand { PfShape sh; double t_kb; };
    const Cand cands[3] = {{kPfSmall, 0.8}, {kPfMedium, 1.3}, {kPfLarge, 3.4}};
    const double kFill = 3.0, kPartialLatency = 1.5, kBytesPerUs = 5.0e6;
    int best_c = -1, best = 1;
    double best_cost = 0.0;
    // Persistent schedule with a stream-K tail (split 0 below), on request only
    // (QGEMM_KERNEL_PREFILL_STREAMK): as many workgroups as are resident at once (as many per CU
    // as their A stages fit in its 160 KiB of LDS: pf_per_cu); each takes whole tiles
    // round-robin (the same tile ids, and so the same XCD-aware walk, as the one-tile launch)
    // for all rounds but the last full one, and the tiles left
    // (between one and two rounds' worth) are split evenly in K over all of them, so no round
    // runs partly idle.  Its cost: the k blocks of a workgroup's share plus two pipeline fills,
    // and about one partial tile per workgroup written and read back at once; the tile is the
    // one this model prices lowest.  The automatic plan never takes it: measured against the
    // one-tile launch it was at best even (FP8 32768 x 3200 x 5120, 6.5 rounds: 786.6 vs 786.0
    // us; 16384 x 12800 x 5120, 12.5 rounds: 1472 vs 1471 us; INT4 4352 x 4096 x 4096, 1.06
    // rounds: 171.0 vs 171.6 us with the 128 x 128 tile, 204 us with the 256 x 256 tile, whose
    // workgroup ranges cut nearly every tail tile) -- the chip's clock rises while a last round
    // runs partly idle -- and the one-tile launch needs no workspace.
    const bool sk_forced = p->kernel_hint == QGEMM_KERNEL_PREFILL_STREAMK;
    // The kernel with dedicated dequantization wavefronts (on request only) has the 64 x 128
    // tile; its split is priced like that tile's.
    const bool tw = p->kernel_hint == QGEMM_KERNEL_PREFILL_TRANSFORM;
    for (int c = 0; c < 3; ++c) {
      const PfShape sh = cands[c].sh;
      if (tw && c > 0) continue;
      if (!tw && (p->tile_hint ? p->tile_hint != pf_bm(sh) : (c > 0 && p->M <= pf_bm(cands[c - 1].sh)))) continue;
      if ((int64_t)pf_bm(sh) * p->K * 2 > 0x7fffffffLL) continue;     // the A tile uses 32-bit offsets
      const int64_t mt = (p->M + pf_bm(sh) - 1) / pf_bm(sh), nt = (p->N + pf_bn(sh) - 1) / pf_bn(sh);
      const int64_t T = mt * nt;
      const int P = kCUs * pf_per_cu(sh);            // resident workgroups
      for (int s = 0; s <= 64 && (s <= 1 || s <= kblocks / 2); ++s) {
        double cost;
        if (s == 0) {                                  // persistent, stream-K tail
          if (!sk_forced) continue;
          const int64_t dp = T > P ? (T / P - 1) * P : 0;
          const double tail = (double)((T - dp) * kblocks) / P;
          const double handoff = (double)P * pf_bm(sh) * pf_bn(sh) * 4 * 2 / kBytesPerUs + 2 * kPartialLatency;
          cost = ((double)(dp / P) * (kblocks + kFill) + tail + 2 * kFill) * cands[c].t_kb + handoff;
        } else {
          if (sk_forced) continue;
          const double rounds = (double)((T * s + kCUs - 1) / kCUs);
          const double partials = (double)(T * s) * pf_bm(sh) * pf_bn(sh) * 4 * 2 / kBytesPerUs;
          cost = rounds * (ceil_div(kblocks, s) + kFill) * cands[c].t_kb + (s > 1 ? partials + kPartialLatency * s : 0.0);
        }
        if (best_c < 0 || cost < best_cost) { best_c = c; best = s; best_cost = cost; }
      }
    }
    if (best_c < 0)
      return fail(QGEMM_ERR_UNSUPPORTED, "the prefill kernel needs %d * K * 2 < 2^31 (K = %lld)",
                  p->tile_hint ? p->tile_hint : pf_bm(kPfSmall), (long long)p->K);
    pl->bm = pf_bm(cands[best_c].sh);
    pl->bn = pf_bn(cands[best_c].sh);
    pl->transform = tw;
    const int64_t mt = (p->M + pl->bm - 1) / pl->bm, nt = (p->N + pl->bn - 1) / pl->bn;
    const bool persist = best == 0;
    pl->splits = persist ? 1 : best;
    finish_split(pl, kblocks, p->split_k_hint);
    if (mt * nt > 0x7fffffffLL) return fail(QGEMM_ERR_UNSUPPORTED, "too many output tiles (%lld)", (long long)(mt * nt));
    pl->grid_x = (unsigned)(mt * nt);
    pl->grid_y = (unsigned)pl->splits;
    pl->tiles = (int)(mt * nt);
    pl->tile_elems = pl->bm * pl->bn;
    const int64_t T = mt * nt;
    const PfShape chosen = cands[best_c].sh;
    const int P = kCUs * pf_per_cu(chosen);          // resident workgroups
    if (persist) {
      const int64_t dp = T > P ? (T / P - 1) * P : 0;
      if ((T - dp) * kblocks > 0x7fffffffLL)
        return fail(QGEMM_ERR_UNSUPPORTED, "the stream-K tail of %lld tiles x %d k blocks is too long",
                    (long long)(T - dp), kblocks);
      pl->persist = P;
      pl->dp_tiles = (int)dp;
      pl->sk_units = (long long)(T - dp) * kblocks;
      pl->splits = 1;
      pl->kb_per_split = kblocks;
      pl->grid_x = (unsigned)P;
      pl->grid_y = 1;
      pl->tiles = (int)(T - dp);                      // tickets: one per tail tile
      pl->counters_bytes = ((size_t)pl->tiles * 4 + 255) / 256 * 256;
      pl->ws_bytes = pl->counters_bytes + (size_t)2 * P * pl->tile_elems * 4;   // two partial slots per workgroup
    }
  }
  if ((int64_t)pl->grid_x * pl->grid_y > 0x7fffffffLL)
    return fail(QGEMM_ERR_UNSUPPORTED, "problem needs %lld workgroups, more than one launch allows",
                (long long)pl->grid_x * pl->grid_y);
  if (pl->splits > 1) {
    pl->counters_bytes = ((size_t)pl->tiles * 4 + 255) / 256 * 256;
    pl->ws_bytes = pl->counters_bytes + (size_t)pl->tiles * pl->splits * pl->tile_elems * 4;
  }
  return QGEMM_OK;
}

// ----------------------------------------------------------------------------- rounding
// Round-to-nearest-even of a double onto a binary format with `mant` explicit mantissa
// bits and smallest normal exponent `emin` (no overflow handling; callers clamp).
static double round_format(double x, int mant, int emin) {
  if (x == 0.0 || !std::isfinite(x)) return x;
  int e2;
  std::frexp(x, &e2);             // |x| = f * 2^e2, f in [0.5, 1)
  int e = e2 - 1;
  if (e < emin) e = emin;
  double q = std::ldexp(1.0, e - mant);
  return std::nearbyint(x / q) * q;   // default rounding mode is to-nearest-even
}

static uint16_t f16_bits_of(double v) {   // v already an fp16 value (finite)
  if (v == 0.0) return std::signbit(v) ? 0x8000 : 0;
  uint16_t s = std::signbit(v) ? 0x8000 : 0;
  double a = std::fabs(v);
  int e2;
  double f = std::frexp(a, &e2);        // a = f 2^e2
  int e = e2 - 1;                        // a = (2f) 2^e
  if (e < -14) {                         // subnormal: a = m 2^-24
    return (uint16_t)(s | (uint16_t)std::llround(a * 16777216.0));
  }
  int m = (int)std::llround((2.0 * f - 1.0) * 1024.0);
  return (uint16_t)(s | ((e + 15) << 10) | m);
}

// Standard normal quantile: bisection on Phi(x) = erfc(-x / sqrt 2) / 2 to double precision.
static double normal_quantile(double p) {
  double lo = -40.0, hi = 40.0;
  for (int i = 0; i < 200 && hi - lo > 0.0; ++i) {
    const double mid = 0.5 * (lo + hi);
    if (mid == lo || mid == hi) break;
    if (0.5 * std::erfc(-mid / std::sqrt(2.0)) < p) lo = mid;
    else hi = mid;
  }
  return 0.5 * (lo + hi);
}

// The NormalFloat-4 code book (QLoRA's construction), in fp16: quantiles of N(0,1) at 8
// evenly spaced probabilities from delta down to (not including) 1/2 for the positive
// values and at 7 for the negative ones, plus an exact 0, sorted and divided by the largest.
// delta = ((1 - 1/30) + (1 - 1/32)) / 2 sits between the outermost quantile estimates of a
// 15- and a 16-point grid.
static void nf4_codebook(double (&t)[16]) {
  const double delta = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0));
  double neg[7], pos[8];
  for (int i = 0; i < 7; ++i) neg[i] = -normal_quantile(delta + (0.5 - delta) * i / 7.0);   // -q .. nearest 0
  for (int i = 0; i < 8; ++i) pos[i] = normal_quantile(delta + (0.5 - delta) * i / 8.0);    // q .. nearest 0
  const double top = pos[0];
  int n = 0;
  for (int i = 0; i < 7; ++i) t[n++] = neg[i] / top;
  t[n++] = 0.0;
  for (int i = 7; i >= 0; --i) t[n++] = pos[i] / top;
  for (int i = 0; i < 16; ++i) t[i] = round_format(t[i], 10, -14);
}

static uint8_t e4m3_code_of(double v) {   // v already an e4m3 value, |v| <= 448
  if (v == 0.0) return 0;
  uint8_t s = std::signbit(v) ? 0x80 : 0;
  double a = std::fabs(v);
  if (a < std::ldexp(1.0, -6)) return (uint8_t)(s | (uint8_t)std::llround(a * 512.0));
  int e2;
  double f = std::frexp(a, &e2);
  int e = e2 - 1;
  int m = (int)std::llround((2.0 * f - 1.0) * 8.0);
  return (uint8_t)(s | ((e + 7) << 3) | m);
}

static double e4m3_value(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v = e == 0 ? std::ldexp(m / 8.0, -6) : std::ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

static uint8_t e2m1_code_of(double v) {   // v already an e2m1 value, |v| <= 6
  static const double mags[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  double a = std::fabs(v);
  int idx = 0;
  for (int i = 0; i < 8; ++i)
    if (mags[i] == a) idx = i;
  uint8_t s = (std::signbit(v) && a != 0.0) ? 8 : 0;
  return (uint8_t)(s | idx);
}

static double clampd(double x, double lo, double hi) { return x < lo ? lo : (x > hi ? hi : x); }

}  // namespace qgemm

using namespace qgemm;

// ============================================================================= C ABI
extern "C" {

const char* qgemm_status_string(qgemm_status_t status) {
  // A C caller may pass any int; read the raw value (in C++ a load of an enum object holding a
  // value outside the enumeration's range is undefined)
  int32_t st;
  std::memcpy(&st, &status, sizeof st);
  static_assert(sizeof(qgemm_status_t) == sizeof(int32_t), "status is passed as a 32-bit int");
  switch (st) {
    case QGEMM_OK: return "QGEMM_OK";
    case QGEMM_ERR_INVALID_ARGUMENT: return "QGEMM_ERR_INVALID_ARGUMENT";
    case QGEMM_ERR_UNSUPPORTED: return "QGEMM_ERR_UNSUPPORTED";
    case QGEMM_ERR_MISALIGNED: return "QGEMM_ERR_MISALIGNED";
    case QGEMM_ERR_WORKSPACE_TOO_SMALL: return "QGEMM_ERR_WORKSPACE_TOO_SMALL";
    case QGEMM_ERR_HIP: return "QGEMM_ERR_HIP";
    default: return "QGEMM_ERR_UNKNOWN_STATUS";
  }
}

const char* qgemm_last_error(void) { return t_last_error.c_str(); }

int32_t qgemm_version(void) { return 100; }

qgemm_status_t qgemm_workspace_bytes(const qgemm_problem_t* p, size_t* bytes) {
  clear_error();
  if (!bytes) return fail(QGEMM_ERR_INVALID_ARGUMENT, "bytes is NULL");
  qgemm_status_t st = validate_problem(p);
  if (st != QGEMM_OK) return st;
  Plan pl;
  st = make_plan(p, &pl);
  if (st != QGEMM_OK) return st;
  *bytes = pl.ws_bytes;
  return QGEMM_OK;
}

qgemm_status_t qgemm_plan_describe(const qgemm_problem_t* p, char* buf, size_t len) {
  clear_error();
  if (!buf || len == 0) return fail(QGEMM_ERR_INVALID_ARGUMENT, "buf is NULL or len is 0");
  buf[0] = '\0';
  qgemm_status_t st = validate_problem(p);
  if (st != QGEMM_OK) return st;
  Plan pl;
  st = make_plan(p, &pl);
  if (st != QGEMM_OK) return st;
  int n;
  if (p->M == 0) {
    n = std::snprintf(buf, len, "empty");
  } else if (pl.kind == KIND_DECODE) {
    static const char* const kA[] = {"direct", "staged", "dma", "staged-early"};
    n = std::snprintf(buf, len, "decode grid=%ux%u waves=%d cb=%d kpw=%d runs=%d a=%s splits=%d kb_per_split=%d "
                      "lds=%d ws=%zu", pl.grid_x, pl.grid_y, pl.nw, pl.cb, pl.kpw, pl.nruns, kA[pl.amode], pl.splits,
                      pl.kb_per_split, pl.lds_bytes, pl.ws_bytes);
  } else {
    n = std::snprintf(buf, len, "prefill grid=%ux%u tile=%dx%d splits=%d kb_per_split=%d persist=%d dp_tiles=%d "
                      "transform=%d ws=%zu", pl.grid_x, pl.grid_y, pl.bm, pl.bn, pl.splits, pl.kb_per_split, pl.persist,
                      pl.dp_tiles, pl.transform, pl.ws_bytes);
  }
  if (n < 0 || (size_t)n >= len) return fail(QGEMM_ERR_INVALID_ARGUMENT, "len %zu is too small (needs %d)", len, n + 1);
  return QGEMM_OK;
}

qgemm_status_t qgemm_quantize(const qgemm_problem_t* p, const float* w_nk, void* codes_canonical,
                              void* scales_canonical, float* alpha_out) {
  clear_error();
  qgemm_status_t st = validate_problem(p);
  if (st != QGEMM_OK) return st;
  if (!w_nk || !codes_canonical) return fail(QGEMM_ERR_INVALID_ARGUMENT, "w_nk and codes_canonical must not be NULL");
  const Format fmt = format_of(p);
  if (!fp8_weights(fmt) && !scales_canonical)
    return fail(QGEMM_ERR_INVALID_ARGUMENT, "scales_canonical must not be NULL for INT4 / INT2 / NF4 / FP4");
  if (!group_scaled(fmt) && !alpha_out) return fail(QGEMM_ERR_INVALID_ARGUMENT, "alpha_out must not be NULL for FP8 / FP4");
  const int64_t N = p->N, K = p->K;
  uint8_t* codes = static_cast<uint8_t*>(codes_canonical);

  if (fmt == FMT_NF4) {
    // s = RNE_fp16(absmax) per (group, column): the code book spans [-1, 1]; code = index of
    // the book entry nearest to w / s, ties to the lower index; 7 (the entry 0) when s = 0
    double book[16];
    nf4_codebook(book);
    const int G = p->group_size;
    uint16_t* sc = static_cast<uint16_t*>(scales_canonical);   // [16] book, then [K/G][N]
    for (int c = 0; c < 16; ++c) sc[c] = f16_bits_of(book[c]);
    sc += 16;
    std::vector<uint8_t> q(K);
    for (int64_t n = 0; n < N; ++n) {
      const float* row = w_nk + n * K;
      for (int64_t g = 0; g < K / G; ++g) {
        double amax = 0.0;
        for (int i = 0; i < G; ++i) {
          const double v = std::fabs((double)row[g * G + i]);
          if (!std::isfinite(v))
            return fail(QGEMM_ERR_INVALID_ARGUMENT, "w_nk[%lld] is not finite", (long long)(n * K + g * G + i));
          amax = v > amax ? v : amax;
        }
        const double s = round_format(amax, 10, -14);
        if (!(s <= 65504.0))
          return fail(QGEMM_ERR_INVALID_ARGUMENT, "column %lld group %lld: absmax %g overflows the fp16 scale",
                      (long long)n, (long long)g, amax);
        sc[g * N + n] = f16_bits_of(s);
        for (int i = 0; i < G; ++i) {
          int best = 7;
          if (s != 0.0) {
            const double x = (double)row[g * G + i] / s;
            double bd = std::fabs(x - book[0]);
            best = 0;
            for (int c = 1; c < 16; ++c) {
              const double d = std::fabs(x - book[c]);
              if (d < bd) { bd = d; best = c; }
            }
          }
          q[g * G + i] = (uint8_t)best;
        }
      }
      for (int64_t j = 0; j < K / 2; ++j) codes[n * (K / 2) + j] = (uint8_t)(q[2 * j] | (q[2 * j + 1] << 4));
    }
    if (alpha_out) *alpha_out = 1.0f;
    return QGEMM_OK;
  }

  if (group_scaled(fmt)) {
    // symmetric absmax per (group, column): s = RNE_fp16(absmax / qmax), code = clamp(rint(w / s),
    // -qmax-1, qmax) + qmax + 1 with qmax = 7 (INT4) or 1 (INT2)
    const bool i2 = fmt == FMT_INT2;
    const double qmax = i2 ? 1.0 : 7.0;
    const int G = p->group_size;
    uint16_t* sc = static_cast<uint16_t*>(scales_canonical);   // [K/G][N]
    std::vector<uint8_t> q(K);
    for (int64_t n = 0; n < N; ++n) {
      const float* row = w_nk + n * K;
      for (int64_t g = 0; g < K / G; ++g) {
        double amax = 0.0;
        for (int i = 0; i < G; ++i) {
          const double v = std::fabs((double)row[g * G + i]);
          if (!std::isfinite(v))
            return fail(QGEMM_ERR_INVALID_ARGUMENT, "w_nk[%lld] is not finite", (long long)(n * K + g * G + i));
          amax = v > amax ? v : amax;
        }
        double s = round_format(amax / qmax, 10, -14);
        if (!(s <= 65504.0))
          return fail(QGEMM_ERR_INVALID_ARGUMENT, "column %lld group %lld: absmax %g is not finite or its scale overflows fp16",
                      (long long)n, (long long)g, amax);
        sc[g * N + n] = f16_bits_of(s);
        for (int i = 0; i < G; ++i) {
          double v = s == 0.0 ? 0.0 : clampd(std::nearbyint((double)row[g * G + i] / s), -qmax - 1.0, qmax);
          q[g * G + i] = (uint8_t)((int)v + (int)qmax + 1);
        }
      }
      if (i2) {   // four codes per byte, lowest k in the lowest bits
        for (int64_t j = 0; j < K / 4; ++j)
          codes[n * (K / 4) + j] =
              (uint8_t)(q[4 * j] | (q[4 * j + 1] << 2) | (q[4 * j + 2] << 4) | (q[4 * j + 3] << 6));
      } else {    // two per byte, low nibble = even k
        for (int64_t j = 0; j < K / 2; ++j) codes[n * (K / 2) + j] = (uint8_t)(q[2 * j] | (q[2 * j + 1] << 4));
      }
    }
    if (alpha_out) *alpha_out = 1.0f;
    return QGEMM_OK;
  }

  double amax = 0.0;
  for (int64_t i = 0; i < N * K; ++i) {
    const double v = std::fabs((double)w_nk[i]);
    if (!std::isfinite(v)) return fail(QGEMM_ERR_INVALID_ARGUMENT, "w_nk[%lld] is not finite", (long long)i);
    amax = v > amax ? v : amax;
  }

  if (fp8_weights(fmt)) {
    const float alpha = (float)(amax / 448.0);
    *alpha_out = alpha;
    for (int64_t i = 0; i < N * K; ++i) {
      if (alpha == 0.0f) { codes[i] = 0; continue; }
      double x = clampd((double)w_nk[i] / (double)alpha, -448.0, 448.0);
      codes[i] = e4m3_code_of(round_format(x, 3, -6));
    }
    return QGEMM_OK;
  }

  // FP4
  const float alpha = (float)(amax / (6.0 * 448.0));
  *alpha_out = alpha;
  uint8_t* sf = static_cast<uint8_t*>(scales_canonical);   // [N][K/16]
  std::vector<uint8_t> q(K);
  for (int64_t n = 0; n < N; ++n) {
    const float* row = w_nk + n * K;
    for (int64_t b = 0; b < K / 16; ++b) {
      uint8_t scode = 0;
      if (alpha != 0.0f) {
        double bmax = 0.0;
        for (int i = 0; i < 16; ++i) bmax = std::fmax(bmax, std::fabs((double)row[b * 16 + i]));
        double t = bmax / (6.0 * (double)alpha);
        if (t > 448.0) t = 448.0;
        scode = e4m3_code_of(round_format(t, 3, -6));
      }
      sf[n * (K / 16) + b] = scode;
      const double den = e4m3_value(scode) * (double)alpha;
      for (int i = 0; i < 16; ++i) {
        if (den == 0.0) { q[b * 16 + i] = 0; continue; }
        double x = clampd((double)row[b * 16 + i] / den, -6.0, 6.0);
        q[b * 16 + i] = e2m1_code_of(round_format(x, 1, 0));
      }
    }
    for (int64_t j = 0; j < K / 2; ++j) codes[n * (K / 2) + j] = (uint8_t)(q[2 * j] | (q[2 * j + 1] << 4));
  }
  return QGEMM_OK;
}

qgemm_status_t qgemm_pack(const qgemm_problem_t* p, const void* w_canonical, const void* scales_canonical,
                          void* w_packed, size_t* w_packed_bytes, void* s_packed, size_t* s_packed_bytes) {
  clear_error();
  qgemm_status_t st = validate_problem(p);
  if (st != QGEMM_OK) return st;
  if (!w_packed_bytes || !s_packed_bytes)
    return fail(QGEMM_ERR_INVALID_ARGUMENT, "w_packed_bytes and s_packed_bytes must not be NULL");
  const Format fmt = format_of(p);
  const int64_t N = p->N, K = p->K, NB = N / 16;
  const size_t need_w = fp8_weights(fmt) ? (size_t)(N * K) : fmt == FMT_INT2 ? (size_t)(N * K / 4) : (size_t)(N * K / 2);
  size_t need_s = 0;
  if (group_scaled(fmt)) need_s = (size_t)(N * (K / p->group_size)) * 2 + (fmt == FMT_NF4 ? kLutHeaderBytes : 0);
  if (fmt == FMT_FP4) need_s = (size_t)(N * (K / 16));
  const size_t cap_w = *w_packed_bytes, cap_s = *s_packed_bytes;
  *w_packed_bytes = need_w;
  *s_packed_bytes = need_s;
  if (!w_packed && !s_packed) return QGEMM_OK;     // size query
  if (w_packed) {
    if (!w_canonical) return fail(QGEMM_ERR_INVALID_ARGUMENT, "w_canonical is NULL");
    if (cap_w < need_w) return fail(QGEMM_ERR_INVALID_ARGUMENT, "w_packed capacity %zu < %zu bytes", cap_w, need_w);
  }
  if (s_packed && need_s) {
    if (!scales_canonical) return fail(QGEMM_ERR_INVALID_ARGUMENT, "scales_canonical is NULL");
    if (cap_s < need_s) return fail(QGEMM_ERR_INVALID_ARGUMENT, "s_packed capacity %zu < %zu bytes", cap_s, need_s);
  }

  if (w_packed) {
    const uint8_t* src = static_cast<const uint8_t*>(w_canonical);
    uint8_t* dst = static_cast<uint8_t*>(w_packed);
    if (fp8_weights(fmt)) {
      // 1 KiB block = 16 columns x 64 k; lane l: column l & 15, k = 32t + 8(l >> 4) + j.
      const int64_t KB = K / 64;
      for (int64_t nb = 0; nb < NB; ++nb)
        for (int64_t kb = 0; kb < KB; ++kb) {
          uint8_t* blk = dst + (nb * KB + kb) * 1024;
          for (int lane = 0; lane < 64; ++lane) {
            const uint8_t* col = src + (nb * 16 + (lane & 15)) * K + kb * 64 + 8 * (lane >> 4);
            for (int t = 0; t < 2; ++t) std::memcpy(blk + 16 * lane + 8 * t, col + 32 * t, 8);
          }
        }
    } else if (fmt == FMT_INT2) {
      // 512-byte block = 16 columns x 128 k; lane l owns 2 dwords; bits 16h + 8b + 2f of dword
      // d hold column l & 15 at k = 32(2d + b) + 8(l >> 4) + 2f + h.
      const int64_t KB = K / 128;
      for (int64_t nb = 0; nb < NB; ++nb)
        for (int64_t kb = 0; kb < KB; ++kb) {
          uint8_t* blk = dst + (nb * KB + kb) * 512;
          for (int lane = 0; lane < 64; ++lane) {
            const uint8_t* col = src + (nb * 16 + (lane & 15)) * (K / 4);
            for (int d = 0; d < 2; ++d) {
              uint32_t word = 0;
              for (int h = 0; h < 2; ++h)
                for (int b = 0; b < 2; ++b)
                  for (int f = 0; f < 4; ++f) {
                    const int64_t k = kb * 128 + 32 * (2 * d + b) + 8 * (lane >> 4) + 2 * f + h;
                    const uint32_t code = (col[k >> 2] >> (2 * (k & 3))) & 3;
                    word |= code << (16 * h + 8 * b + 2 * f);
                  }
              std::memcpy(blk + 8 * lane + 4 * d, &word, 4);
            }
          }
        }
    } else {
      // 1 KiB block = 16 columns x 128 k; lane l owns 4 dwords, dword t holds the 8 nibbles
      // of column l & 15 at k = 32t + 8(l >> 4) + J[slot].
      static const int J_INT4[8] = {0, 2, 4, 6, 1, 3, 5, 7};
      static const int J_FP4[8] = {0, 1, 2, 3, 4, 5, 6, 7};
      static const int J_NF4[8] = {0, 4, 1, 5, 2, 6, 3, 7};
      const int* J = fmt == FMT_INT4 ? J_INT4 : fmt == FMT_NF4 ? J_NF4 : J_FP4;
      const int64_t KB = K / 128;
      for (int64_t nb = 0; nb < NB; ++nb)
        for (int64_t kb = 0; kb < KB; ++kb) {
          uint8_t* blk = dst + (nb * KB + kb) * 1024;
          for (int lane = 0; lane < 64; ++lane) {
            const uint8_t* col = src + (nb * 16 + (lane & 15)) * (K / 2);
            for (int t = 0; t < 4; ++t) {
              uint32_t word = 0;
              const int64_t k0 = kb * 128 + 32 * t + 8 * (lane >> 4);
              for (int slot = 0; slot < 8; ++slot) {
                const int64_t k = k0 + J[slot];
                const uint32_t nib = (col[k >> 1] >> (4 * (k & 1))) & 0xF;
                word |= nib << (4 * slot);
              }
              std::memcpy(blk + 16 * lane + 4 * t, &word, 4);
            }
          }
        }
    }
  }

  if (s_packed && need_s) {
    if (group_scaled(fmt)) {
      const int G = p->group_size;
      const int span = G > 128 ? G : 128;
      const int T = G < 128 ? 128 / G : 1;
      const int64_t KS = K / span, NG = K / G;
      const uint16_t* src = static_cast<const uint16_t*>(scales_canonical);   // [K/G][N]
      uint16_t* dst = static_cast<uint16_t*>(s_packed);
      if (fmt == FMT_NF4) {   // header: code-book low bytes in dwords 0..3, high bytes in 4..7
        uint8_t* h = static_cast<uint8_t*>(s_packed);
        std::memset(h, 0, kLutHeaderBytes);
        for (int c = 0; c < 16; ++c) {
          h[c] = (uint8_t)(src[c] & 0xFF);
          h[16 + c] = (uint8_t)(src[c] >> 8);
        }
        src += 16;
        dst += kLutHeaderBytes / 2;
      }
      for (int64_t nb = 0; nb < NB; ++nb)
        for (int64_t ks = 0; ks < KS; ++ks)
          for (int c = 0; c < 16; ++c)
            for (int t = 0; t < T; ++t) {
              const int64_t g = ks * (span / G) + t;
              if (g < NG) dst[((nb * KS + ks) * 16 + c) * T + t] = src[g * N + nb * 16 + c];
            }
    } else {
      const int64_t KB = K / 128;
      const uint8_t* src = static_cast<const uint8_t*>(scales_canonical);     // [N][K/16]
      uint8_t* dst = static_cast<uint8_t*>(s_packed);
      for (int64_t nb = 0; nb < NB; ++nb)
        for (int64_t kb = 0; kb < KB; ++kb)
          for (int c = 0; c < 16; ++c)
            for (int h = 0; h < 2; ++h)
              for (int t = 0; t < 4; ++t)
                dst[((nb * KB + kb) * 16 + c) * 8 + 4 * h + t] = src[(nb * 16 + c) * (K / 16) + 8 * kb + 2 * t + h];
    }
  }
  return QGEMM_OK;
}

}  // extern "C"
