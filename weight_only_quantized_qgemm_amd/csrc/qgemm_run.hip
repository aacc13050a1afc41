// qgemm_run: validation, planning and launch of the decode or prefill kernel.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>

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
  if (pl.transform) {
    switch (pl.fmt) {
      case FMT_INT4: return launch_prefill_tw_format<FMT_INT4>(pl, group_size, a, stream);
      case FMT_FP8: return launch_prefill_tw_format<FMT_FP8>(pl, group_size, a, stream);
      case FMT_FP4: return launch_prefill_tw_format<FMT_FP4>(pl, group_size, a, stream);
      case FMT_FP8H: return launch_prefill_tw_format<FMT_FP8H>(pl, group_size, a, stream);
      case FMT_INT2: return launch_prefill_tw_format<FMT_INT2>(pl, group_size, a, stream);
      case FMT_NF4: return launch_prefill_tw_format<FMT_NF4>(pl, group_size, a, stream);
    }
    return hipErrorInvalidValue;
  }
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

namespace {

// Pointer checks of qgemm_run / qgemm_run_bias / qgemm_run_no_alloc (everything but the
// workspace), after validate_problem.
qgemm_status_t check_pointers(qgemm::Format fmt, const void* A, const void* w_packed, const void* s_packed,
                              const float* alpha, const void* bias, const void* out) {
  using namespace qgemm;
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
  return QGEMM_OK;
}

// Enqueue the planned kernel; counters / partials are the split-K tickets and fp32 partial
// tiles (unused when the plan has no split).
qgemm_status_t enqueue(const qgemm_problem_t* p, const qgemm::Plan& pl, const void* A, const void* w_packed,
                       const void* s_packed, const float* alpha, const void* bias, void* out, unsigned* counters,
                       float* partials, void* stream) {
  using namespace qgemm;
  dev::KArgs a;
  std::memset(&a, 0, sizeof(a));
  a.A = static_cast<const uint16_t*>(A);
  a.W = static_cast<const uint8_t*>(w_packed);
  a.S = s_packed;
  if (pl.fmt == FMT_NF4) {   // the code book heads the packed scales
    a.lut = static_cast<const unsigned*>(s_packed);
    a.S = static_cast<const char*>(s_packed) + kLutHeaderBytes;
  }
  a.alpha = alpha;
  a.out = out;
  a.bias = bias;
  if (pl.ws_bytes) {
    a.counters = counters;
    a.partials = partials;
  }
  a.M = (int)p->M;
  a.N = (int)p->N;
  a.K = (int)p->K;
  a.out_dtype = p->out_dtype;
  a.splits = pl.splits;
  a.kb_per_split = pl.kb_per_split;
  a.tiles_n = (int)((p->N + pl.bn - 1) / (pl.bn ? pl.bn : 1));
  a.persist = pl.persist;
  a.tiles_total = pl.persist ? (int)(((p->M + pl.bm - 1) / pl.bm) * a.tiles_n) : 0;
  a.dp_tiles = pl.dp_tiles;
  a.sk_q = pl.persist ? (int)(pl.sk_units / pl.persist) : 0;
  a.sk_r = pl.persist ? (int)(pl.sk_units % pl.persist) : 0;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = pl.kind == KIND_PREFILL ? dev::launch_prefill(pl, p->group_size, a, s)
                                                : dev::launch_decode(pl, p->group_size, a, s);
  if (e != hipSuccess) return fail(QGEMM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return QGEMM_OK;
}

}  // namespace

extern "C" qgemm_status_t qgemm_run_bias(const qgemm_problem_t* p, const void* A, const void* w_packed,
                                         const void* s_packed, const float* alpha, const void* bias, void* out,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  using namespace qgemm;
  clear_error();
  qgemm_status_t st = validate_problem(p);
  if (st != QGEMM_OK) return st;
  if (p->M == 0) return QGEMM_OK;                    // empty product: nothing to enqueue
  st = check_pointers(format_of(p), A, w_packed, s_packed, alpha, bias, out);
  if (st != QGEMM_OK) return st;
  Plan pl;
  st = make_plan(p, &pl);
  if (st != QGEMM_OK) return st;
  if (pl.ws_bytes) {
    if (!workspace || workspace_bytes < pl.ws_bytes)
      return fail(QGEMM_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes needed, %zu given%s", pl.ws_bytes,
                  workspace ? workspace_bytes : (size_t)0, workspace ? "" : " (NULL)");
    if (!aligned(workspace, 256)) return fail(QGEMM_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  }
  char* ws = static_cast<char*>(workspace);
  return enqueue(p, pl, A, w_packed, s_packed, alpha, bias, out, reinterpret_cast<unsigned*>(ws),
                 ws ? reinterpret_cast<float*>(ws + pl.counters_bytes) : nullptr, stream);
}

extern "C" qgemm_status_t qgemm_run(const qgemm_problem_t* p, const void* A, const void* w_packed,
                                    const void* s_packed, const float* alpha, void* out, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return qgemm_run_bias(p, A, w_packed, s_packed, alpha, nullptr, out, workspace, workspace_bytes, stream);
}

// ============================================================================= no-allocation entry
// For callers that cannot allocate device memory (code under graph capture, tight serving
// loops): the split-K workspace is a file-scope device array instead of a caller buffer.
// Each GPU holds its own copy at its own address, found once per device with
// hipGetSymbolAddress; host code uses only that address (the array's name is a host-side
// stand-in).  All calls on one GPU share the array.  Layout: a fixed ticket region (one
// 32-bit ticket per output tile, zero between calls: every completed call resets the tickets
// it took) and the fp32 partial tiles after it.  The tickets never share bytes with the
// partials of another call, whatever the two calls' plans, so only the ticket region has to
// start at zero.
namespace {

constexpr size_t kScratchBytes = QGEMM_NO_ALLOC_SCRATCH_BYTES;
constexpr size_t kScratchTicketBytes = 64 * 1024;
static_assert(kScratchBytes % 256 == 0 && kScratchTicketBytes % 256 == 0 && kScratchTicketBytes < kScratchBytes,
              "scratch regions stay 256-byte aligned");
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device, after set-up

__global__ void zero_fill(uint4* p, unsigned n) {
  for (unsigned i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Address of this device's scratch.  The first call on a device looks it up and enqueues a
// clear of the ticket region on `stream` (a fill kernel, so a capturing caller records a
// kernel node, not a memset).
qgemm_status_t scratch_for_device(hipStream_t stream, char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return qgemm::fail(QGEMM_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return qgemm::fail(QGEMM_ERR_UNSUPPORTED, "device %d is beyond the %d that qgemm_run_no_alloc supports", dev,
                       kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return qgemm::fail(QGEMM_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                         hipGetErrorString(e));
    hipLaunchKernelGGL(zero_fill, dim3(16), dim3(256), 0, stream, static_cast<uint4*>(ptr),
                       (unsigned)(kScratchTicketBytes / 16));
    e = hipGetLastError();
    if (e != hipSuccess) return qgemm::fail(QGEMM_ERR_HIP, "clearing the scratch tickets failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = static_cast<char*>(g_scratch_ptr[dev]);
  return QGEMM_OK;
}

}  // namespace

extern "C" qgemm_status_t qgemm_run_no_alloc(const qgemm_problem_t* p, const void* A, const void* w_packed,
                                             const void* s_packed, const float* alpha, const void* bias, void* out,
                                             void* stream) {
  using namespace qgemm;
  clear_error();
  qgemm_status_t st = validate_problem(p);
  if (st != QGEMM_OK) return st;
  if (p->M == 0) return QGEMM_OK;                    // empty product: nothing to enqueue
  st = check_pointers(format_of(p), A, w_packed, s_packed, alpha, bias, out);
  if (st != QGEMM_OK) return st;
  Plan pl;
  st = make_plan(p, &pl);
  if (st != QGEMM_OK) return st;
  char* sc = nullptr;
  if (pl.ws_bytes) {
    const size_t partial_bytes = pl.ws_bytes - pl.counters_bytes;
    if ((size_t)pl.tiles * 4 > kScratchTicketBytes || partial_bytes > kScratchBytes - kScratchTicketBytes)
      return fail(QGEMM_ERR_WORKSPACE_TOO_SMALL, "this problem's split-K plan needs %d tickets and %zu bytes of "
                  "partial tiles; the static scratch of qgemm_run_no_alloc holds %zu tickets and %zu bytes "
                  "(qgemm_run with a workspace has no such limit)", pl.tiles, partial_bytes,
                  kScratchTicketBytes / 4, kScratchBytes - kScratchTicketBytes);
    st = scratch_for_device(static_cast<hipStream_t>(stream), &sc);
    if (st != QGEMM_OK) return st;
  }
  return enqueue(p, pl, A, w_packed, s_packed, alpha, bias, out, reinterpret_cast<unsigned*>(sc),
                 sc ? reinterpret_cast<float*>(sc + kScratchTicketBytes) : nullptr, stream);
}
