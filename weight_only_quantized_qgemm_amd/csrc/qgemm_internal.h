// Internal declarations shared by the host library and the kernel launchers.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/qgemm.h"

namespace qgemm {

// Prefill workgroup shapes: one row of eight wavefronts (two per SIMD), each owning
// TM x TN MFMA tiles of 16 x 16.  The large shape amortises every dequantized weight
// fragment over 16 row tiles; the medium one (small M) has a quarter of the area, so its
// k steps are short and it keeps four A stages in flight instead of two; the small one
// (M up to a few hundred) halves the medium tile's rows again, doubling the workgroups.
// RU: row tiles per LDS read unit; LA: units read ahead of the MFMAs that consume them;
// ST: A stages in LDS; BB: k blocks per workgroup barrier (ST - BB k blocks are loaded ahead
// of the one being computed).
struct PfShape { int wgm, wgn, tm, tn, ru, la, st, bb; };
#ifndef QGEMM_PF_LARGE
#define QGEMM_PF_LARGE 1, 8, 16, 2, 4, 1, 2, 1
#define QGEMM_PF_MEDIUM 1, 8, 8, 1, 8, 1, 4, 1
#endif
// The small tile meets at a barrier every second k block, with six A stages (96 KiB, one
// workgroup per CU): FP4 128 x 8192 x 8192 28.4 -> 26.8 us, INT4 384 x 4096 x 4096 22.9 -> 21.2
// us against four stages and a barrier per block; eight stages measured slower (deeper
// prefetch alone: 28.2 and 23.0 us).
#ifndef QGEMM_PF_SMALL
#define QGEMM_PF_SMALL 1, 8, 4, 1, 4, 1, 6, 2
#endif
constexpr PfShape kPfLarge{QGEMM_PF_LARGE};    // 256 x 256 output tile
constexpr PfShape kPfMedium{QGEMM_PF_MEDIUM};  // 128 x 128 output tile
constexpr PfShape kPfSmall{QGEMM_PF_SMALL};    // 64 x 128 output tile
constexpr int pf_bm(PfShape s) { return 16 * s.wgm * s.tm; }
constexpr int pf_bn(PfShape s) { return 16 * s.wgn * s.tn; }
// Workgroups of a shape that fit one compute unit's 160 KiB of LDS (the A stages dominate).
constexpr int pf_per_cu(PfShape s) { return (160 * 1024) / (s.st * pf_bm(s) * 256 + 1024); }
// Decode kernel: wavefronts per workgroup (with A staged in LDS, and whenever a workgroup
// owns a single column block), and the smaller count for wider workgroups of unstaged A:
// half the wavefronts with twice the K share each pipeline longer runs (M = 16: N = 11008
// 9.58 -> 9.00 us, FP8 N = 10240 14.5 -> 12.8 us; with one column block 6.9 -> 7.8 us).
#ifndef QGEMM_DEC_NW
#define QGEMM_DEC_NW 8
#endif
constexpr int kDecodeWaves = QGEMM_DEC_NW;
constexpr int kDecodeWavesWide = 4;
// Decode staging pass (A slice and scales into LDS): the largest staged A slice and scale
// range per workgroup, and the 16-byte chunks per thread they take at most.
#ifndef QGEMM_DEC_MAXA
#define QGEMM_DEC_MAXA (32 * 1024)
#endif
constexpr int kDecodeMaxA = QGEMM_DEC_MAXA;
constexpr int kDecodeMaxScales = 16 * 1024;
constexpr int kDecodeStageA = kDecodeMaxA / (16 * 64 * kDecodeWaves);
constexpr int kDecodeStageS = kDecodeMaxScales / (16 * 64 * kDecodeWaves);
// Decode with M above the staging limit takes A through buffer-to-LDS DMA when its slots fit
// (0 turns it off).
#ifndef QGEMM_DEC_ADMA
#define QGEMM_DEC_ADMA 1
#endif

// Kernel formats.  FMT_FP8H is FP8 weights with fp16 activations (mm_fp16_fp8): the weight
// layout, quantization and alpha are FP8's, the MFMA is the fp16 one.  FMT_INT2 (W2A16)
// shares INT4's fp16 group scales and their layout; its weight blocks are 512 bytes.
// FMT_NF4 has INT4's block size and scale layout, behind a 256-byte code-book header.
enum Format : int { FMT_INT4 = 0, FMT_FP8 = 1, FMT_FP4 = 2, FMT_FP8H = 3, FMT_INT2 = 4, FMT_NF4 = 5 };
constexpr bool fp8_weights(int fmt) { return fmt == FMT_FP8 || fmt == FMT_FP8H; }
// fp16 scale per (group of G k, column), no alpha
constexpr bool group_scaled(int fmt) { return fmt == FMT_INT4 || fmt == FMT_INT2 || fmt == FMT_NF4; }
constexpr bool f16_mfma(int fmt) { return fmt == FMT_INT4 || fmt == FMT_FP8H || fmt == FMT_INT2 || fmt == FMT_NF4; }
// Bytes in front of the NF4 scales: the code book split into low- and high-byte tables.
constexpr int kLutHeaderBytes = 256;

// ---- Decode LDS layout, shared by the launch plan (which sizes the allocation) and the kernel.
// Packed scale bytes of one column block that nkb consecutive k blocks read, at most (an INT4
// group of 256 spans two k blocks and may be cut by a boundary).
constexpr int dec_scale_span(int fmt, int group_size, int nkb) {
  return fmt == FMT_FP4 ? 128 * nkb
         : fp8_weights(fmt) ? 0
         : group_size <= 128 ? 32 * (128 / group_size) * nkb
                             : 32 * (nkb / 2 + 1);
}
// How a decode wavefront gets its A fragments: straight from memory into registers
// (A_DIRECT), from its private LDS region after a register-staged copy of its whole A share
// and scales (A_STAGED, small M), or from LDS slots that buffer-to-LDS DMA fills run by run,
// 4 KiB (16 rows x 128 halves) per k block (A_DMA, larger M).  The A_DMA slots are static
// arrays of the kernel instance, not part of the dynamic region below.
// A_STAGED_EARLY is A_STAGED with the first weight block issued ahead of the staging loads
// (one column block, runs of at most five k blocks, a grid of at most one workgroup per CU).
enum AMode : int { A_DIRECT = 0, A_STAGED = 1, A_DMA = 2, A_STAGED_EARLY = 3 };
constexpr bool a_staged(int amode) { return amode == A_STAGED || amode == A_STAGED_EARLY; }
// LDS a workgroup may take (160 KiB on gfx950).
constexpr int kMaxLds = 160 * 1024;
// LDS the decode kernel holds besides its slot sets and its dynamic region: the split-K
// hand-off flag and the 1 KiB-aligned placeholder of an unused slot set, with their padding.
constexpr int kDecodeStaticReserve = 2048;
// A_DMA: bytes of one slot set (one k block per wavefront and run position); a kernel that
// overlaps runs (two or more runs per share) holds two sets.  An instance exists, and the plan
// takes A_DMA, only when its sets, the wave tiles of the final reduction and the reserve fit
// in LDS.
constexpr int dec_dma_set_bytes(int waves, int kpw) { return waves * kpw * 4096; }
constexpr bool dec_dma_fits(int waves, int kpw, int cb, int nruns) {
  return (nruns > 1 ? 2 : 1) * dec_dma_set_bytes(waves, kpw) + waves * cb * 64 * 16 + kDecodeStaticReserve <= kMaxLds;
}
// Per wavefront (dynamic region): its staged A share (M rows of share x 128 + 8 halves) and
// its staged scales (cb column blocks), each padded to 16 bytes; A_STAGED only.
constexpr int dec_a_bytes(int M, int share, int amode) {
  return a_staged(amode) ? (M * (share * 128 + 8) * 2 + 15) / 16 * 16 : 0;
}
constexpr int dec_s_bytes(int fmt, int group_size, int share, int cb, int amode) {
  return a_staged(amode) ? (cb * dec_scale_span(fmt, group_size, share) + 15) / 16 * 16 : 0;
}
constexpr int dec_region_bytes(int fmt, int group_size, int M, int share, int cb, int amode) {
  return dec_a_bytes(M, share, amode) + dec_s_bytes(fmt, group_size, share, cb, amode);
}
// Whole workgroup: the regions, then the wave tiles of the final reduction (64 lanes x 16 B
// per wavefront and column block).
constexpr int dec_lds_bytes(int fmt, int group_size, int M, int share, int cb, int amode, int waves) {
  return waves * dec_region_bytes(fmt, group_size, M, share, cb, amode) + waves * cb * 64 * 16;
}
enum Kind : int { KIND_DECODE = 1, KIND_PREFILL = 2 };

// Records a detail message for qgemm_last_error() and returns `st`.
qgemm_status_t fail(qgemm_status_t st, const char* fmt, ...);
void clear_error();

// Full validation of the descriptor (shapes, dtype combination, hints).
qgemm_status_t validate_problem(const qgemm_problem_t* p);
Format format_of(const qgemm_problem_t* p);

// Launch plan, a pure function of the problem (never of out_dtype or of pointers).
struct Plan {
  Kind kind;
  Format fmt;
  // decode: column blocks (16 columns each) per workgroup, k blocks per wavefront run
  int cb, kpw;
  bool astage;            // decode: stage the A slice in LDS (small M)
  int amode;              // decode: AMode (A_STAGED when astage)
  int nw;                 // decode: wavefronts per workgroup
  int nruns;              // decode: runs per wavefront share, pipelined when 2..8 (A_DMA) or 2..4 (else 1)
  int lds_bytes;          // decode: dynamic LDS per workgroup (staged A, staged scales, wave tiles)
  // prefill: workgroup tile (bm selects the shape: pf_bm of kPfSmall, kPfMedium or kPfLarge)
  int bm, bn;
  int transform;          // prefill: the kernel with dedicated dequantization wavefronts (64 x 128)
  // K split across workgroups (1 = none) and the 128-wide k-blocks each split covers
  int splits;
  int kb_per_split;
  // prefill, persistent schedule (0 = one tile per workgroup): resident workgroups, whole tiles
  // handed out round-robin, and the k blocks of the remaining (stream-K tail) tiles
  int persist;
  int dp_tiles;
  long long sk_units;
  // grid
  unsigned grid_x, grid_y;
  int tiles;              // output tiles that own a split-K counter
  int tile_elems;         // fp32 elements of one partial tile
  size_t counters_bytes;  // workspace prefix holding one 32-bit ticket per tile
  size_t ws_bytes;        // total workspace (0 when splits == 1)
};

qgemm_status_t make_plan(const qgemm_problem_t* p, Plan* plan);

}  // namespace qgemm
