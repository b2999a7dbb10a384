// Debug validation of the device-side preconditions of the routing and of a plan (off the hot
// path).  The pages require each token's top_k experts to be distinct (FlashInfer
// "flashinfer.fused_moe.CudnnGroupedGemmNvfp4Config", topk_ids bullet) and a pre-aligned plan's
// entries to name flat slots or the padding sentinel, with one valid expert per block
// (FlashInfer "flashinfer.fused_moe.alphamoe_nvfp4_aligned_moe", plan parameters).  The fused
// calls do not check these on the device; these kernels count violations into a three-int
// report that the caller reads back.
#include "bfp4moe.h"
#include "runtime.h"

namespace bfp4 {

namespace {

constexpr int kCheckThreads = 256;
constexpr int32_t kNoToken = 0x7FFFFFFF;

// report[0..1] = 0, report[2] = v2
__global__ void report_init_kernel(int32_t* __restrict__ report, int32_t v2) {
  if (threadIdx.x < 3) report[threadIdx.x] = threadIdx.x == 2 ? v2 : 0;
}

// One thread per token: ids outside [-1, num_experts) and ids >= 0 repeated within the token.
__global__ __launch_bounds__(kCheckThreads) void check_topk_kernel(
    const int32_t* __restrict__ ids, int64_t M, int top_k, int num_experts,
    int32_t* __restrict__ report) {
  const int64_t t = (int64_t)blockIdx.x * kCheckThreads + threadIdx.x;
  if (t >= M) return;
  const int32_t* r = ids + t * top_k;
  int dup = 0, bad = 0;
  for (int j = 0; j < top_k; ++j) {
    const int32_t v = r[j];
    if (v < -1 || v >= num_experts) {
      ++bad;
    } else if (v >= 0 && !dup) {
      for (int i = 0; i < j; ++i) {
        if (r[i] == v) {
          dup = 1;
          break;
        }
      }
    }
  }
  if (dup) atomicAdd(report + 0, 1);
  if (bad) atomicAdd(report + 1, bad);
  if (dup || bad) atomicMin(report + 2, (int32_t)t);
}

// One thread per plan entry.  The extent P must lie in [0, capacity] and be a multiple of
// block_m; entries below the (clamped) extent must lie in [0, sentinel], and the expert id of
// every block below it in [0, nloc).
__global__ __launch_bounds__(kCheckThreads) void check_plan_kernel(
    const int32_t* __restrict__ sorted, const int32_t* __restrict__ eids,
    const int32_t* __restrict__ ntpp, int64_t cap, int64_t sentinel, int block_m, int nloc,
    int32_t* __restrict__ report) {
  const int64_t P = *ntpp;
  const bool ok = P >= 0 && P <= cap && P % block_m == 0;
  const int64_t ext = P < 0 ? 0 : (P < cap ? P : cap) / block_m * block_m;
  const int64_t i = (int64_t)blockIdx.x * kCheckThreads + threadIdx.x;
  if (i == 0 && !ok) report[2] = 1;
  if (i < ext) {
    const int64_t f = sorted[i];
    if (f < 0 || f > sentinel) atomicAdd(report + 0, 1);
  }
  if (i < ext / block_m) {
    const int32_t e = eids[i];
    if (e < 0 || e >= nloc) atomicAdd(report + 1, 1);
  }
}

// XOR checksum of a device buffer, a diagnostic outside the MoE path (the benchmark times it as
// the HBM read rate a plain stream reaches on the same GPU): kXorWaves waves each read one
// contiguous slice, 16 bytes per lane per load with kXorDepth loads in flight, and write the XOR
// of the slice's 32-bit words to partial[wave].
constexpr int kXorGroups = 4096, kXorWaves = kXorGroups * 4, kXorDepth = 4;
static_assert(kXorWaves == BFP4_XOR_PARTIALS, "one partial word per wave");

typedef uint32_t xu32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void xor_checksum_kernel(const xu32x4_t* __restrict__ src,
                                                           int64_t n16, int64_t per_wave,
                                                           uint32_t* __restrict__ partial) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t base = wave * per_wave;
  const int64_t end = base + per_wave < n16 ? base + per_wave : n16;
  uint32_t acc = 0;
  for (int64_t i = base + lane; i < end; i += 64 * kXorDepth) {
    xu32x4_t v[kXorDepth];
#pragma unroll
    for (int d = 0; d < kXorDepth; ++d) {
      const int64_t j = i + 64 * d;
      v[d] = j < end ? src[j] : xu32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int d = 0; d < kXorDepth; ++d) acc ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  if (lane == 0) partial[wave] = acc;
}

}  // namespace

hipError_t launch_check_topk(const int32_t* ids, int64_t M, int top_k, int num_experts,
                             int32_t* report, hipStream_t s) {
  {
    KernelTimer t("check_init", s);
    hipLaunchKernelGGL(report_init_kernel, dim3(1), dim3(64), 0, s, report, kNoToken);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || M == 0) return e;
  KernelTimer t("check_topk", s);
  const dim3 grid((unsigned)((M + kCheckThreads - 1) / kCheckThreads));
  hipLaunchKernelGGL(check_topk_kernel, grid, dim3(kCheckThreads), 0, s, ids, M, top_k,
                     num_experts, report);
  return hipGetLastError();
}

hipError_t launch_check_plan(const int32_t* sorted, const int32_t* eids, const int32_t* ntpp,
                             int64_t cap, int64_t sentinel, int block_m, int nloc,
                             int32_t* report, hipStream_t s) {
  {
    KernelTimer t("check_init", s);
    hipLaunchKernelGGL(report_init_kernel, dim3(1), dim3(64), 0, s, report, 0);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  KernelTimer t("check_plan", s);
  const int64_t n = cap > 0 ? cap : 1;        // one thread reads the extent even when cap is 0
  const dim3 grid((unsigned)((n + kCheckThreads - 1) / kCheckThreads));
  hipLaunchKernelGGL(check_plan_kernel, grid, dim3(kCheckThreads), 0, s, sorted, eids, ntpp, cap,
                     sentinel, block_m, nloc, report);
  return hipGetLastError();
}

hipError_t launch_xor_checksum(const void* buf, int64_t bytes, uint32_t* partial,
                               hipStream_t s) {
  const int64_t n16 = bytes / 16;
  const int64_t per_wave = (n16 + kXorWaves - 1) / kXorWaves;
  KernelTimer t("xor_checksum", s);
  hipLaunchKernelGGL(xor_checksum_kernel, dim3(kXorGroups), dim3(256), 0, s,
                     static_cast<const xu32x4_t*>(buf), n16, per_wave, partial);
  return hipGetLastError();
}

}  // namespace bfp4
