// probe.hip -- libsvprobe: test and benchmark probes of libspecverify's device helpers (gfx950).
//
// NOT part of the product library: it is built into its own shared object, which only the GPU tests and
// the benchmark load.  It runs the product's own device code (sv_common.h) on inputs chosen by the host,
// so that the random stream and the race transform can be checked directly, element by element:
//   probe_philox       the Philox-4x32-10 block function on given counters and keys (known-answer tests);
//   probe_philox_uk    the same with one key for the whole launch, the form the verify kernels use;
//   probe_race_e2      for every 23-bit uniform code j (U = (j + 0.5) 2^-23): E2 = -log2 U as the draws
//                      compute it, and the race key scale rcp(E2) (the Gumbel-max draws of the AReno page
//                      "feat(engine): MTP training loss and speculative decoding for bailing_v3", its
//                      per-step optimisation table);
//   probe_u24          for every 24-bit code: the accept uniform (w >> 8) 2^-24 as the accept test sees it;
//   probe_read_stream  a plain read of a buffer with 16-byte loads (the bandwidth reference the benchmark
//                      quotes its kernels against);
//   probe_dispatch_id  the dispatch's 64-bit id and queue address as a kernel sees them (the per-call tag of
//                      cross-workgroup flags is built from them);
//   probe_occupancy    how many 256-thread workgroups the hardware holds at once for a kernel that reserves
//                      given numbers of scalar or vector registers.
// Every entry point takes device pointers, enqueues one kernel on `stream` and returns 0, or 1 for bad
// arguments (nothing enqueued).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_common.h"

namespace {

__global__ void k_philox(const uint32_t* ctr, const uint32_t* key, uint32_t* out, int n) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n) return;
  const uint4 c = make_uint4(ctr[4 * t], ctr[4 * t + 1], ctr[4 * t + 2], ctr[4 * t + 3]);
  const uint4 r = sv::philox10(c, key[2 * t], key[2 * t + 1]);
  out[4 * t] = r.x;
  out[4 * t + 1] = r.y;
  out[4 * t + 2] = r.z;
  out[4 * t + 3] = r.w;
}

// philox10_uk, the verify kernels' form: one key for the whole launch (kernel arguments, so uniform).
__global__ void k_philox_uk(const uint32_t* ctr, uint32_t k0, uint32_t k1, uint32_t* out, int n) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n) return;
  const uint4 c = make_uint4(ctr[4 * t], ctr[4 * t + 1], ctr[4 * t + 2], ctr[4 * t + 3]);
  const uint4 r = sv::philox10_uk(c, k0, k1);
  out[4 * t] = r.x;
  out[4 * t + 1] = r.y;
  out[4 * t + 2] = r.z;
  out[4 * t + 3] = r.w;
}

__global__ void k_race_e2(float* e2, float* scale) {
  const uint32_t j = blockIdx.x * blockDim.x + threadIdx.x;  // grid covers exactly 2^23 codes
  const uint32_t w = j << 9;                                  // (w >> 9) == j
  const float e = sv::exp_race_E2(w);
  e2[j] = e;
  scale[j] = __builtin_amdgcn_rcpf(e);
}

__global__ void k_u24(float* u) {
  const uint32_t j = blockIdx.x * blockDim.x + threadIdx.x;  // grid covers exactly 2^24 codes
  u[j] = sv::u24(j << 8);
}

// Each thread xors its 16-byte vectors (grid-stride); one word per workgroup keeps the loads alive.
__global__ __launch_bounds__(256) void k_read_stream(const uint4* src, size_t nvec, uint32_t* sink) {
  uint32_t acc = 0;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += (size_t)gridDim.x * blockDim.x) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  acc = sv::wave_or(acc);
  if ((threadIdx.x & 63) == 0 && acc == 0x9E3779B9u) sink[blockIdx.x] = acc;  // practically never stored
}

// Occupancy: each 256-thread workgroup stamps the wall clock (100 MHz) at its start, waits `spin` ticks and
// stamps its end; the most workgroups alive at once is what the hardware holds per dispatch.  The variants
// claim registers through empty inline-asm clobbers (no instruction is emitted): the compiler then reports
// that many, and the launch reserves them.
template <int REG>
__global__ __launch_bounds__(256) void k_occupancy(unsigned long long* out, unsigned long long spin) {
  if (REG == 1) asm volatile("" ::: "s73");  // 80 scalar registers in the compiler's total
  if (REG == 2) asm volatile("" ::: "s75");  // 82
  if (REG == 3) asm volatile("" ::: "s95");  // 102
  if (REG == 4) asm volatile("" ::: "v60");  // 61 vector registers
  if (REG == 5) asm volatile("" ::: "v68");  // 69
  const unsigned long long t0 = wall_clock64();
  while (wall_clock64() - t0 < spin) __builtin_amdgcn_s_sleep(2);
  __syncthreads();
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = t0;
    out[2 * blockIdx.x + 1] = wall_clock64();
  }
}

// The dispatch id (the LLVM intrinsic has no clang builtin of its own).
extern "C" __device__ unsigned long long sv_dispatch_id() __asm("llvm.amdgcn.dispatch.id");

__global__ void k_dispatch_id(unsigned long long* out) {
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = sv_dispatch_id();
    out[2 * blockIdx.x + 1] = (unsigned long long)(uintptr_t)__builtin_amdgcn_queue_ptr();
  }
}

}  // namespace

// out: device uint64 [2 * blocks]
extern "C" int probe_dispatch_id(unsigned long long* out, int32_t blocks, void* stream) {
  if (!out || blocks < 1) return 1;
  (void)hipGetLastError();  // so that the check below is about this launch alone
  hipLaunchKernelGGL(k_dispatch_id, dim3((unsigned)blocks), dim3(64), 0, (hipStream_t)stream, out);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

extern "C" int probe_philox(const uint32_t* ctr, const uint32_t* key, uint32_t* out, int32_t n, void* stream) {
  if (n < 1 || !ctr || !key || !out) return 1;
  (void)hipGetLastError();  // so that the check below is about this launch alone
  hipLaunchKernelGGL(k_philox, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream, ctr, key, out, n);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// As probe_philox with one key (k0, k1) for all n counters.
extern "C" int probe_philox_uk(const uint32_t* ctr, uint32_t k0, uint32_t k1, uint32_t* out, int32_t n, void* stream) {
  if (n < 1 || !ctr || !out) return 1;
  (void)hipGetLastError();  // so that the check below is about this launch alone
  hipLaunchKernelGGL(k_philox_uk, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream, ctr, k0, k1, out,
                     n);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// out: device uint64 [2 * blocks]; variant 0..5 (see k_occupancy); spin: wall-clock ticks each workgroup waits
extern "C" int probe_occupancy(int32_t variant, unsigned long long* out, int32_t blocks, unsigned long long spin,
                               void* stream) {
  if (!out || blocks < 1 || spin > 100000ull) return 1;
  (void)hipGetLastError();  // so that the check below is about this launch alone
  const dim3 g((unsigned)blocks), t(256);
  const hipStream_t st = (hipStream_t)stream;
  switch (variant) {
    case 0: hipLaunchKernelGGL(k_occupancy<0>, g, t, 0, st, out, spin); break;
    case 1: hipLaunchKernelGGL(k_occupancy<1>, g, t, 0, st, out, spin); break;
    case 2: hipLaunchKernelGGL(k_occupancy<2>, g, t, 0, st, out, spin); break;
    case 3: hipLaunchKernelGGL(k_occupancy<3>, g, t, 0, st, out, spin); break;
    case 4: hipLaunchKernelGGL(k_occupancy<4>, g, t, 0, st, out, spin); break;
    case 5: hipLaunchKernelGGL(k_occupancy<5>, g, t, 0, st, out, spin); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// e2, scale: device float [2^23]
extern "C" int probe_race_e2(float* e2, float* scale, void* stream) {
  if (!e2 || !scale) return 1;
  (void)hipGetLastError();  // so that the check below is about this launch alone
  hipLaunchKernelGGL(k_race_e2, dim3((1u << 23) / 256), dim3(256), 0, (hipStream_t)stream, e2, scale);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// u: device float [2^24]
extern "C" int probe_u24(float* u, void* stream) {
  if (!u) return 1;
  (void)hipGetLastError();  // so that the check below is about this launch alone
  hipLaunchKernelGGL(k_u24, dim3((1u << 24) / 256), dim3(256), 0, (hipStream_t)stream, u);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// src: device, nvec 16-byte vectors (16-byte aligned); sink: device uint32 [blocks]
extern "C" int probe_read_stream(const void* src, size_t nvec, uint32_t* sink, int32_t blocks, void* stream) {
  if (!src || !sink || nvec == 0 || blocks < 1 || ((uintptr_t)src & 15)) return 1;
  (void)hipGetLastError();  // so that the check below is about this launch alone
  hipLaunchKernelGGL(k_read_stream, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, (const uint4*)src, nvec,
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}
