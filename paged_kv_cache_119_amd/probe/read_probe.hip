// Measurement context for the roofline (not part of libpagedkv): a plain
// streaming read of a contiguous buffer, the practical read ceiling the
// decode kernels are compared with, and timing events for the benchmark.  Grid-stride over 16-byte pieces, four
// loads in flight per iteration; the XOR of what was read is written only if
// it equals an arbitrary constant, so the loads cannot be removed.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4 *p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <bool NT>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *__restrict__ p, int64_t n, uint32_t *out) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * 256;
  uint32_t acc = 0;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 a = ld<NT>(p + i), b = ld<NT>(p + i + stride), c = ld<NT>(p + i + 2 * stride),
                d = ld<NT>(p + i + 3 * stride);
    acc ^= a.x ^ b.y ^ c.z ^ d.w;
  }
  for (; i < n; i += stride) acc ^= ld<NT>(p + i).x;
  if (acc == 0x9E3779B9u) out[blockIdx.x & 1023] = acc;
}

}  // namespace

// Read `bytes` (a multiple of 16) at `p` with `grid` workgroups of 256
// threads; `out` is a device buffer of 1024 uint32 that is written only by
// accident of the data.  nt != 0: non-temporal loads.  Returns the HIP error.
extern "C" int pkvprobe_stream_read(const void *p, int64_t bytes, void *out, int grid, int nt, void *stream) {
  if (!p || !out || bytes < 16 || bytes % 16 != 0 || grid < 1) return (int)hipErrorInvalidValue;
  if (nt)
    hipLaunchKernelGGL((stream_read_kernel<true>), dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<const u32x4 *>(p), bytes / 16, reinterpret_cast<uint32_t *>(out));
  else
    hipLaunchKernelGGL((stream_read_kernel<false>), dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<const u32x4 *>(p), bytes / 16, reinterpret_cast<uint32_t *>(out));
  return (int)hipGetLastError();
}

// Timing events for per-launch durations: created with
// hipEventDisableSystemFence, so recording one does not add a system-scope
// cache writeback and invalidation between the launches it brackets (HIP
// documents the flag for events used only to measure time).  Elapsed times
// are read after a device synchronisation.  Each returns the HIP error.
extern "C" int pkvprobe_event_create(void **ev) {
  if (!ev) return (int)hipErrorInvalidValue;
  return (int)hipEventCreateWithFlags(reinterpret_cast<hipEvent_t *>(ev), hipEventDisableSystemFence);
}
extern "C" int pkvprobe_event_record(void *ev, void *stream) {
  return (int)hipEventRecord(reinterpret_cast<hipEvent_t>(ev), reinterpret_cast<hipStream_t>(stream));
}
extern "C" int pkvprobe_event_elapsed(float *ms, void *start, void *stop) {
  if (!ms) return (int)hipErrorInvalidValue;
  return (int)hipEventElapsedTime(ms, reinterpret_cast<hipEvent_t>(start), reinterpret_cast<hipEvent_t>(stop));
}
extern "C" int pkvprobe_event_destroy(void *ev) {
  return (int)hipEventDestroy(reinterpret_cast<hipEvent_t>(ev));
}
