// Streaming-bandwidth probe for the benchmark (not part of the decode path).
//
// Measures what plain HIP kernels reach on the current GPU for a read-only
// stream, a write-only stream and a copy, with 16-byte accesses in grid-stride
// loops, so that the decode kernels' HBM figures can be read against the
// chip's attainable bandwidth as well as its published peak.  Each kind runs
// at several grid sizes and the best rate is reported.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

__global__ void k_stream_read(const uint4* __restrict__ a, size_t n, unsigned* __restrict__ sink) {
  unsigned acc = 0u;
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint4 v = a[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // a data-dependent store the compiler cannot drop; the buffer holds no
  // such pattern, so nothing is written in practice
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

__global__ void k_stream_write(uint4* __restrict__ a, size_t n) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
    a[i] = make_uint4(static_cast<unsigned>(i), 0u, 0u, 0u);
}

__global__ void k_stream_copy(const uint4* __restrict__ a, uint4* __restrict__ b, size_t n) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) b[i] = a[i];
}

constexpr int kThreads = 256;
constexpr int kGrids[] = {1024, 2048, 4096, 8192, 16384};
constexpr int kMaxGrid = 16384;

}  // namespace

// bytes: size of each of the two device buffers (a multiple of 16, at least
// 16 MiB); reps: timed launches per kind and grid.  Writes the best
// read-only, write-only and copy rates in GB/s (copy counts the bytes read
// plus the bytes written).  Allocates its buffers and frees them before
// returning.  Returns 0, or the HIP error code of the first failing call
// (the outputs are then unspecified).
extern "C" int stepq_stream_probe(size_t bytes, int reps, double* read_gbs, double* write_gbs,
                                  double* copy_gbs) {
  if (bytes % 16 != 0 || bytes < (size_t(16) << 20) || reps < 1 || !read_gbs || !write_gbs || !copy_gbs)
    return static_cast<int>(hipErrorInvalidValue);
  const size_t n = bytes / 16;
  uint4 *a = nullptr, *b = nullptr;
  unsigned* sink = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t err = hipSuccess;
  double best[3] = {0.0, 0.0, 0.0};
#define STEPQ_PROBE_CK(x) do { err = (x); if (err != hipSuccess) goto done; } while (0)
  STEPQ_PROBE_CK(hipMalloc(&a, bytes));
  STEPQ_PROBE_CK(hipMalloc(&b, bytes));
  STEPQ_PROBE_CK(hipMalloc(&sink, kMaxGrid * sizeof(unsigned)));
  STEPQ_PROBE_CK(hipMemset(a, 1, bytes));
  STEPQ_PROBE_CK(hipEventCreate(&e0));
  STEPQ_PROBE_CK(hipEventCreate(&e1));
  for (int grid : kGrids) {
    for (int kind = 0; kind < 3; ++kind) {
      auto launch = [&]() {
        if (kind == 0) k_stream_read<<<grid, kThreads>>>(a, n, sink);
        else if (kind == 1) k_stream_write<<<grid, kThreads>>>(b, n);
        else k_stream_copy<<<grid, kThreads>>>(a, b, n);
      };
      for (int w = 0; w < 2; ++w) launch();
      STEPQ_PROBE_CK(hipEventRecord(e0));
      for (int r = 0; r < reps; ++r) launch();
      STEPQ_PROBE_CK(hipEventRecord(e1));
      STEPQ_PROBE_CK(hipEventSynchronize(e1));
      STEPQ_PROBE_CK(hipGetLastError());
      float ms = 0.f;
      STEPQ_PROBE_CK(hipEventElapsedTime(&ms, e0, e1));
      const double moved = (kind == 2 ? 2.0 : 1.0) * static_cast<double>(bytes);
      const double gbs = moved / (static_cast<double>(ms) * 1e-3 / reps) / 1e9;
      if (gbs > best[kind]) best[kind] = gbs;
    }
  }
  *read_gbs = best[0];
  *write_gbs = best[1];
  *copy_gbs = best[2];
done:
#undef STEPQ_PROBE_CK
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (a) (void)hipFree(a);
  if (b) (void)hipFree(b);
  if (sink) (void)hipFree(sink);
  return static_cast<int>(err);
}
