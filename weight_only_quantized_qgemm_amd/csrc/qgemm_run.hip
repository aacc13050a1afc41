// qgemm_run: validation, planning and launch of the decode or prefill kernel.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "qgemm_device.h"

namespace {
bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }
}  // namespace

namespace qgemm {
namespace dev {

hipError_t launch_decode(const Plan& pl, int group_size, const KArgs& a, hipStream_t stream) {
  switch (pl.fmt) {
    case FMT_INT4: return launch_decode_format<FMT_INT4>(pl, group_size, a, stream);
    case FMT_FP8: return launch_decode_format<FMT_FP8>(pl, group_size, a, stream);
    case FMT_FP4: return launch_decode_format<FMT_FP4>(pl, group_size, a, stream);
    case FMT_FP8H: return launch_decode_format<FMT_FP8H>(pl, group_size, a, stream);
    case FMT_INT2: return launch_decode_format<FMT_INT2>(pl, group_size, a, stream);
    case FMT_NF4: return launch_decode_format<FMT_NF4>(pl, group_size, a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(const Plan& pl, int group_size, const KArgs& a, hipStream_t stream) {
  switch (pl.fmt) {
    case FMT_INT4: return launch_prefill_format<FMT_INT4>(pl, group_size, a, stream);
    case FMT_FP8: return launch_prefill_format<FMT_FP8>(pl, group_size, a, stream);
    case FMT_FP4: return launch_prefill_format<FMT_FP4>(pl, group_size, a, stream);
    case FMT_FP8H: return launch_prefill_format<FMT_FP8H>(pl, group_size, a, stream);
    case FMT_INT2: return launch_prefill_format<FMT_INT2>(pl, group_size, a, stream);
    case FMT_NF4: return launch_prefill_format<FMT_NF4>(pl, group_size, a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace dev
}  // namespace qgemm

extern "C" qgemm_status_t qgemm_run_bias(const qgemm_problem_t* p, const void* A, const void* w_packed,
                                         const void* s_packed, const float* alpha, const void* bias, void* out,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  using namespace qgemm;
  clear_error();
  qgemm_status_t st = validate_problem(p);
  if (st != QGEMM_OK) return st;
  if (p->M == 0) return QGEMM_OK;                    // empty product: nothing to enqueue
  const Format fmt = format_of(p);
  if (!A) return fail(QGEMM_ERR_INVALID_ARGUMENT, "A is NULL");
  if (!w_packed) return fail(QGEMM_ERR_INVALID_ARGUMENT, "w_packed is NULL");
  if (!out) return fail(QGEMM_ERR_INVALID_ARGUMENT, "out is NULL");
  if (!fp8_weights(fmt) && !s_packed) return fail(QGEMM_ERR_INVALID_ARGUMENT, "s_packed is NULL (needed for INT4, INT2, NF4 and FP4)");
  if (!group_scaled(fmt) && !alpha) return fail(QGEMM_ERR_INVALID_ARGUMENT, "alpha is NULL (needed for FP8 and FP4)");
  if (!aligned(A, 16)) return fail(QGEMM_ERR_MISALIGNED, "A must be 16-byte aligned");
  if (!aligned(w_packed, 16)) return fail(QGEMM_ERR_MISALIGNED, "w_packed must be 16-byte aligned");
  if (s_packed && !fp8_weights(fmt) && !aligned(s_packed, 16)) return fail(QGEMM_ERR_MISALIGNED, "s_packed must be 16-byte aligned");
  // a bias takes the alignment the FlashInfer fix requires of it (PR #7495 analysis,
  // section 3(a): 16 bytes when a bias is given, 4 for the scalar alpha)
  if (bias && !aligned(bias, 16)) return fail(QGEMM_ERR_MISALIGNED, "bias must be 16-byte aligned");
  if (alpha && !group_scaled(fmt) && !aligned(alpha, 4)) return fail(QGEMM_ERR_MISALIGNED, "alpha must be 4-byte aligned");
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

  dev::KArgs a;
  std::memset(&a, 0, sizeof(a));
  a.A = static_cast<const uint16_t*>(A);
  a.W = static_cast<const uint8_t*>(w_packed);
  a.S = s_packed;
  if (fmt == FMT_NF4) {   // the code book heads the packed scales
    a.lut = static_cast<const unsigned*>(s_packed);
    a.S = static_cast<const char*>(s_packed) + kLutHeaderBytes;
  }
  a.alpha = alpha;
  a.out = out;
  a.bias = bias;
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
  const hipError_t e = pl.kind == KIND_PREFILL ? dev::launch_prefill(pl, p->group_size, a, s)
                                                : dev::launch_decode(pl, p->group_size, a, s);
  if (e != hipSuccess) return fail(QGEMM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return QGEMM_OK;
}

extern "C" qgemm_status_t qgemm_run(const qgemm_problem_t* p, const void* A, const void* w_packed,
                                    const void* s_packed, const float* alpha, void* out, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return qgemm_run_bias(p, A, w_packed, s_packed, alpha, nullptr, out, workspace, workspace_bytes, stream);
}
