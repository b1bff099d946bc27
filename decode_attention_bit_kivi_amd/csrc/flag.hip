// Ordering between two streams of one GPU through a flag in device memory instead of a queue
// barrier: the producer stream stores a sequence number once its earlier work is done, and a
// one-wave kernel on the consumer stream holds that stream until it reads a number at least as
// large.  In the overlapped decode loop the gather stream can wait this way for the compute
// stream's selection: a queue barrier between two streams releases the waiting stream ~11 µs
// after the work it waits for has ended, while the stream behind a polling kernel starts its
// next kernel within ~2 µs of the store.  The setter pays for its release instead (the
// device-scope write-back of the L2 lines its stream has dirtied, 4-12 µs after a decode step).
#include "../../include/specache.h"
#include "common.h"

namespace {

// The stream runs this after every earlier command on it has completed (in-order stream, end of
// kernel release), so the store publishes that work; release ordering at device scope.
__global__ __launch_bounds__(64) void flag_set_kernel(uint32_t* flag, uint32_t value) {
  if (threadIdx.x == 0) __hip_atomic_store(flag, value, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// Lane 0 polls the flag until it has reached `value` (wrap-around safe: value - flag taken as a
// signed distance) or `max_ticks` of the 100 MHz real-time counter have passed; a wait that ends
// on the time limit adds one to *timeouts, so every call ends and the caller can tell.  The polls
// are relaxed loads at device scope (they read past the non-coherent caches) about every 0.5 µs,
// and the acquire is one fence once the value is there: an acquire at device scope on every poll
// would invalidate caches that the kernels running beside the wait are using.
__global__ __launch_bounds__(64) void flag_wait_kernel(const uint32_t* flag, uint32_t value, uint64_t max_ticks,
                                                       uint32_t* timeouts) {
  if (threadIdx.x != 0) return;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (;;) {
    const uint32_t v = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((int32_t)(v - value) >= 0) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      return;
    }
    if (__builtin_amdgcn_s_memrealtime() - t0 > max_ticks) {
      atomicAdd(timeouts, 1u);
      return;
    }
    __builtin_amdgcn_s_sleep(16);
  }
}

}  // namespace

extern "C" {

int specache_flag_set(uint32_t* flag, uint32_t value, void* stream) {
  if (!flag) return SPECACHE_ERR_INVALID;
  flag_set_kernel<<<1, 64, 0, static_cast<hipStream_t>(stream)>>>(flag, value);
  return hipGetLastError() == hipSuccess ? SPECACHE_OK : SPECACHE_ERR_HIP;
}

int specache_flag_wait(const uint32_t* flag, uint32_t value, uint32_t max_wait_us, uint32_t* timeouts,
                       void* stream) {
  if (!flag || !timeouts || max_wait_us == 0) return SPECACHE_ERR_INVALID;
  flag_wait_kernel<<<1, 64, 0, static_cast<hipStream_t>(stream)>>>(flag, value, (uint64_t)max_wait_us * 100u,
                                                                   timeouts);
  return hipGetLastError() == hipSuccess ? SPECACHE_OK : SPECACHE_ERR_HIP;
}

}  // extern "C"
