// Measurement helpers for the benchmark, built as their own library (libqgemm_probe.so)
// next to libqgemm.so and outside its C ABI: nothing here is part of the GEMM.
//
//  * qgemm_probe_stream: a plain streaming read of one or two device buffers with
//    non-temporal 16-byte loads (the access pattern of the decode kernel's weight and scale
//    streams, without any arithmetic), so that the decode kernel can be compared with the
//    time a kernel needs just to read the same bytes at the same sizes.  Every loaded value
//    feeds an XOR whose per-workgroup result is stored, so no load can be dropped.
//  * qgemm_probe_host_ns: host time per qgemm_run call (validation, planning, launch) and
//    per qgemm_workspace_bytes call (validation and planning only), measured in C so that
//    no Python call overhead is counted.
#include <hip/hip_runtime.h>

#include <chrono>
#include <cstdint>

#include "../../include/qgemm.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Thread t of the grid reads chunks t, t + T, t + 2T, ... (T = threads in the grid, U chunks
// per thread at most), all loads issued before the first is consumed.  Chunks past the end
// are clamped to the last one (read again, not counted).
template <int U>
__global__ __launch_bounds__(512) void stream_read(const u32x4* __restrict__ a, long long na,
                                                   const u32x4* __restrict__ b, long long nb,
                                                   unsigned* __restrict__ sink) {
  const long long T = (long long)gridDim.x * blockDim.x;
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 x[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    long long i = t + u * T;
    i = i < na ? i : na - 1;
    x[u] = __builtin_nontemporal_load(a + i);
  }
  u32x4 y = {0u, 0u, 0u, 0u};
  if (nb > 0) {                                      // the second stream (scales): one chunk per thread at most
    long long i = t < nb ? t : nb - 1;
    y = __builtin_nontemporal_load(b + i);
  }
  unsigned acc = y[0] ^ y[1] ^ y[2] ^ y[3];
#pragma unroll
  for (int u = 0; u < U; ++u) acc ^= x[u][0] ^ x[u][1] ^ x[u][2] ^ x[u][3];
  // one value per workgroup: the XOR of every thread's loads (storing each thread's value
  // would add write traffic to a read measurement)
  __shared__ unsigned red[8];
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned r = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) r ^= red[w];
    sink[blockIdx.x] = r;
  }
}

}  // namespace

extern "C" {

// Threads per workgroup of the streaming probe.
int qgemm_probe_stream_threads(void) { return 512; }

// Workgroups the probe launches for `chunks` 16-byte chunks of the first buffer with U loads
// per thread (the sink needs at least this many 32-bit words).
long long qgemm_probe_stream_groups(long long chunks, int U) {
  const long long per = 512LL * U;
  return (chunks + per - 1) / per;
}

// Enqueue one streaming read of a (na_bytes) and optionally b (nb_bytes, at most one 16-byte
// chunk per thread of the grid); sizes must be multiples of 16, buffers 16-byte aligned.
// U in {1, 2, 4, 8}.  Returns 0 on success, else a HIP error code or -1 for bad arguments.
int qgemm_probe_stream(const void* a, long long na_bytes, const void* b, long long nb_bytes, void* sink, int U,
                       void* stream) {
  if (!a || na_bytes <= 0 || (na_bytes & 15) || (nb_bytes & 15) || nb_bytes < 0 || !sink) return -1;
  const long long na = na_bytes / 16, nb = nb_bytes / 16;
  const long long groups = qgemm_probe_stream_groups(na, U);
  if (groups > 0x7fffffffLL || nb > groups * 512) return -1;
  const dim3 grid((unsigned)groups), block(512);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const u32x4* pa = static_cast<const u32x4*>(a);
  const u32x4* pb = static_cast<const u32x4*>(b);
  unsigned* ps = static_cast<unsigned*>(sink);
  switch (U) {
    case 1: hipLaunchKernelGGL(stream_read<1>, grid, block, 0, s, pa, na, pb, nb, ps); break;
    case 2: hipLaunchKernelGGL(stream_read<2>, grid, block, 0, s, pa, na, pb, nb, ps); break;
    case 4: hipLaunchKernelGGL(stream_read<4>, grid, block, 0, s, pa, na, pb, nb, ps); break;
    case 8: hipLaunchKernelGGL(stream_read<8>, grid, block, 0, s, pa, na, pb, nb, ps); break;
    default: return -1;
  }
  return (int)hipGetLastError();
}

// Host nanoseconds per call, averaged over `iters` calls after 10 untimed ones:
// out_ns[0] = qgemm_workspace_bytes (validation + plan), out_ns[1] = qgemm_run (validation,
// plan and the kernel launch; the kernels are enqueued on `stream`).  Returns the first
// non-OK status, else QGEMM_OK.
int qgemm_probe_host_ns(const qgemm_problem_t* p, const void* A, const void* w, const void* s, const float* alpha,
                        void* out, void* ws, size_t ws_bytes, void* stream, int iters, double* out_ns) {
  using clk = std::chrono::steady_clock;
  size_t bytes = 0;
  for (int i = 0; i < 10; ++i) {
    const qgemm_status_t st = qgemm_workspace_bytes(p, &bytes);
    if (st != QGEMM_OK) return st;
  }
  auto t0 = clk::now();
  for (int i = 0; i < iters; ++i) qgemm_workspace_bytes(p, &bytes);
  auto t1 = clk::now();
  out_ns[0] = std::chrono::duration<double, std::nano>(t1 - t0).count() / iters;
  for (int i = 0; i < 10; ++i) {
    const qgemm_status_t st = qgemm_run(p, A, w, s, alpha, out, ws, ws_bytes, stream);
    if (st != QGEMM_OK) return st;
  }
  t0 = clk::now();
  for (int i = 0; i < iters; ++i) qgemm_run(p, A, w, s, alpha, out, ws, ws_bytes, stream);
  t1 = clk::now();
  out_ns[1] = std::chrono::duration<double, std::nano>(t1 - t0).count() / iters;
  return QGEMM_OK;
}

}  // extern "C"
