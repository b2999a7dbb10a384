// Expert-sorted routing plan (FlashInfer "flashinfer.fused_moe.alphamoe_nvfp4_aligned_moe",
// plan paragraph: sorted_token_ids, expert_ids per block_m entries, num_tokens_post_padded;
// "flashinfer.fused_moe.CudnnGroupedGemmNvfp4Config": expert-sorted permutation, masked
// non-local experts).
//
// Plan contents: routed slots grouped by local expert (ascending), each group padded to a
// multiple of block_m; inside a group the flat slot indices f = t*top_k + j ascend; padding and
// the tail [extent, capacity) hold the sentinel M*top_k; expert_ids = local id per block, -1 past
// the extent; token_to_row = plan row per slot or -1.
//
// Three phases: histogram of local expert ids; prefix sum of the padded counts; a stable scatter
// in which one wavefront walks its slots 64 at a time and ranks equal ids with ballots (a lane's
// rank among the lanes holding the same id is the popcount of the matching lanes below it).
// Small inputs run all phases in one workgroup; large inputs split the slots into 1024-slot
// chunks (per-chunk histograms, one scan over (expert, chunk), per-chunk scatter).  The scatter
// is a serial chain of ballot rounds per wave, so spreading the chunks over many workgroups
// (one wave each, on different CUs) is faster than running more waves in one workgroup.
#include "device.h"
#include "runtime.h"

namespace bfp4 {

namespace {

constexpr int kMaxLocal = 1024;
constexpr int64_t kSmallMax = 2048;   // slots handled by the single-workgroup kernel
constexpr int kChunk = 1024;          // slots per chunk in the multi-workgroup path
constexpr int kScatterWaves = 4;      // waves ranking one chunk's slots in the scatter
constexpr int kScanCache = 24576;     // chunk counts the scan keeps in LDS (16 bits each)

__device__ __forceinline__ int local_id(int32_t id, int num_experts, int offset, int nloc) {
  int e = id - offset;
  return (id >= 0 && id < num_experts && e >= 0 && e < nloc) ? e : -1;
}

// Lanes of the current wave whose key equals this lane's key (keys < 2^nbits).
__device__ __forceinline__ uint64_t match_any(uint32_t key, int nbits) {
  uint64_t peers = __ballot(1);
  for (int b = 0; b < nbits; ++b) {
    uint32_t bit = (key >> b) & 1u;
    uint64_t m = __ballot(bit);
    peers &= bit ? m : ~m;
  }
  return peers;
}

__device__ __forceinline__ int key_bits(int nloc) {
  int b = 1;
  while ((1 << b) <= nloc) ++b;   // keys 0..nloc (nloc marks unrouted)
  return b;
}

// One wave ranks slots [f0, f1) in order and scatters them.  run[e] holds, for each local
// expert, the plan position of its next slot; it is advanced by the highest lane of each group.
// The ids of kIdBatch rounds of 64 slots are loaded together before any of those rounds
// scatters: the vector-memory counter covers loads and stores in issue order, so a load issued
// after a round's stores could only be waited for behind them, one store round trip per round.
__device__ void scatter_wave(const int32_t* ids, int64_t f0, int64_t f1,
                             int num_experts, int offset, int nloc, int* run,
                             int32_t* __restrict__ sorted, int32_t* __restrict__ ttr) {
  const int lane = threadIdx.x & 63;
  const int nbits = key_bits(nloc);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  constexpr int kIdBatch = 16;
  for (int64_t b0 = f0; b0 < f1; b0 += 64 * kIdBatch) {
    int32_t idv[kIdBatch];
#pragma unroll
    for (int i = 0; i < kIdBatch; ++i) {
      const int64_t fi = b0 + 64 * i + lane;
      idv[i] = fi < f1 ? ids[fi] : -1;
    }
#pragma unroll
    for (int i = 0; i < kIdBatch; ++i) {
      const int64_t base = b0 + 64 * i;
      if (base >= f1) break;
      const int64_t f = base + lane;
      if (f < f1) {
        const int e = local_id(idv[i], num_experts, offset, nloc);
        const uint32_t key = (e < 0) ? (uint32_t)nloc : (uint32_t)e;
        const uint64_t peers = match_any(key, nbits);
        if (e >= 0) {
          const int rank = __popcll(peers & below);
          const int pos = run[e] + rank;
          sorted[pos] = (int32_t)f;
          ttr[f] = pos;
          if ((peers >> lane) == 1ull) run[e] += __popcll(peers);   // highest lane of the group
        } else {
          ttr[f] = -1;
        }
      }
    }
  }
}

// Exclusive scan of one int per thread over a 1024-thread block (16 waves); returns the
// total.  Each wave scans its 64 values with lane shuffles; one barrier publishes the wave
// totals.
__device__ int block_excl_scan_1024(int v, int* tmp, int& total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) tmp[w] = x;
  __syncthreads();
  int pre = 0, all = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int t = tmp[i];
    pre += i < w ? t : 0;
    all += t;
  }
  total = all;
  __syncthreads();                       // tmp may be reused by the caller
  return pre + x - v;
}

// Writes num_tokens_post_padded, expert_ids and the sentinel entries, given each expert's
// count (cnt) and segment start (start) in LDS.
__device__ void write_plan_frame(const int* cnt, const int* start, int nloc, int block_m, int P,
                                 int64_t cap, int32_t sentinel, int32_t* __restrict__ sorted,
                                 int32_t* __restrict__ eids, int32_t* __restrict__ ntpp) {
  int tid = threadIdx.x;
  if (tid == 0) *ntpp = P;
  // blockDim / nloc threads per expert (at least one: nloc <= kMaxLocal = blockDim) write its
  // block ids and padding sentinels
  const int per = (int)blockDim.x / nloc;
  if (tid < per * nloc) {
    const int e = tid % nloc, part = tid / nloc;
    int c = cnt[e];
    if (c > 0) {
      int seg = (c + block_m - 1) / block_m * block_m;
      int s0 = start[e];
      for (int b = s0 / block_m + part; b < (s0 + seg) / block_m; b += per) eids[b] = e;
      for (int p = s0 + c + part; p < s0 + seg; p += per) sorted[p] = sentinel;
    }
  }
  for (int64_t b = P / block_m + tid; b < cap / block_m; b += blockDim.x) eids[b] = -1;
  for (int64_t p = P + tid; p < cap; p += blockDim.x) sorted[p] = sentinel;
}

// The whole plan in one 1024-thread workgroup (A <= kSmallMax slots).
__device__ void plan_small(const int32_t* __restrict__ ids, int64_t A, int num_experts,
                           int offset, int nloc, int block_m, int32_t* __restrict__ sorted,
                           int32_t* __restrict__ eids, int32_t* __restrict__ ntpp,
                           int32_t* __restrict__ ttr, int64_t cap) {
  __shared__ int cnt[kMaxLocal], start[kMaxLocal], tmp[1024];
  __shared__ int32_t sid[kSmallMax];          // the ids, read from memory once
  __shared__ int run[kMaxLocal];               // the scatter's running positions
  int tid = threadIdx.x;
  if (tid < nloc) cnt[tid] = 0;
  __syncthreads();
  for (int64_t f = tid; f < A; f += 1024) {
    const int32_t id = ids[f];
    sid[f] = id;
    int e = local_id(id, num_experts, offset, nloc);
    if (e >= 0) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  int seg = (tid < nloc) ? (cnt[tid] + block_m - 1) / block_m * block_m : 0;
  int P;
  int excl = block_excl_scan_1024(seg, tmp, P);
  if (tid < nloc) {
    start[tid] = excl;
    run[tid] = excl;
  }
  __syncthreads();
  // wave 0 scatters (advancing its own copy of the starts) while the other waves write the
  // frame, whose padding entries and tail the scatter never touches; wave 0 writes its share of
  // the frame afterwards
  if (tid < 64) scatter_wave(sid, 0, A, num_experts, offset, nloc, run, sorted, ttr);
  write_plan_frame(cnt, start, nloc, block_m, P, cap, (int32_t)A, sorted, eids, ntpp);
}

__global__ __launch_bounds__(1024) void plan_small_kernel(
    const int32_t* __restrict__ ids, int64_t A, int num_experts, int offset, int nloc,
    int block_m, int32_t* __restrict__ sorted, int32_t* __restrict__ eids,
    int32_t* __restrict__ ntpp, int32_t* __restrict__ ttr, int64_t cap) {
  plan_small(ids, A, num_experts, offset, nloc, block_m, sorted, eids, ntpp, ttr, cap);
}

// Maximum of v over the workgroup (blockDim a multiple of 64, at most 1024 threads).
__device__ float block_max_any(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6, nw = (int)blockDim.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = 0.0f;
  for (int i = 0; i < nw; ++i) r = __builtin_fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

// The plan (workgroup 0) and the per-token NVFP4 quantization of the activations (workgroup
// 1 + t quantizes row t) in one launch: the two are independent, and each part computes exactly
// what its own kernel does (the plan through plan_small; the row through the same amax, encode
// scale and block quantizer as the per-row quantizer, whose result does not depend on how the
// row's blocks are spread over threads).
__global__ __launch_bounds__(1024) void plan_quantize_kernel(
    const int32_t* __restrict__ ids, int64_t A, int num_experts, int offset, int nloc,
    int block_m, int32_t* __restrict__ sorted, int32_t* __restrict__ eids,
    int32_t* __restrict__ ntpp, int32_t* __restrict__ ttr, int64_t cap,
    const uint16_t* __restrict__ x, int64_t cols, int64_t stride, uint8_t* __restrict__ q,
    uint8_t* __restrict__ sf, float* __restrict__ dec) {
  if (blockIdx.x == 0) {
    plan_small(ids, A, num_experts, offset, nloc, block_m, sorted, eids, ntpp, ttr, cap);
    return;
  }
  __shared__ float red[16];
  const int64_t r = blockIdx.x - 1;
  const uint16_t* xr = x + r * stride;
  const int64_t nblk = cols >> 4;
  float m = 0.0f;
  for (int64_t b = threadIdx.x; b < nblk; b += blockDim.x) {
    float v[16];
    load_block16(xr + b * 16, v);
#pragma unroll
    for (int i = 0; i < 16; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(v[i]));
  }
  m = block_max_any(m, red);
  const float s_enc = encode_scale_from_amax(m);
  if (threadIdx.x == 0) dec[r] = 1.0f / s_enc;
  uint8_t* qr = q + r * (cols >> 1);
  uint8_t* sr = sf + r * nblk;
  for (int64_t b = threadIdx.x; b < nblk; b += blockDim.x) {
    float v[16];
    load_block16(xr + b * 16, v);
    uint32_t lo, hi;
    const uint32_t sc = quant_block16(v, s_enc, lo, hi);
    *reinterpret_cast<uint2*>(qr + b * 8) = make_uint2(lo, hi);
    sr[b] = (uint8_t)sc;
  }
}

__global__ __launch_bounds__(256) void plan_count_kernel(const int32_t* __restrict__ ids, int64_t A,
                                                         int num_experts, int offset, int nloc,
                                                         int32_t* __restrict__ hist) {
  __shared__ int h[kMaxLocal];
  for (int e = threadIdx.x; e < nloc; e += 256) h[e] = 0;
  __syncthreads();
  int64_t f0 = (int64_t)blockIdx.x * kChunk;
  int64_t f1 = f0 + kChunk < A ? f0 + kChunk : A;
  for (int64_t f = f0 + threadIdx.x; f < f1; f += 256) {
    int e = local_id(ids[f], num_experts, offset, nloc);
    if (e >= 0) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < nloc; e += 256) hist[(int64_t)blockIdx.x * nloc + e] = h[e];
}

// Turns the per-chunk histograms into per-chunk starting positions (in place), writes the
// extent and publishes each local expert's count and segment start (fr[e], fr[nloc + e]) for
// the scatter's workgroups, which write the rest of the plan frame.
__global__ __launch_bounds__(1024) void plan_scan_kernel(int32_t* __restrict__ hist,
                                                         int64_t nchunks, int nloc, int block_m,
                                                         int32_t* __restrict__ fr,
                                                         int32_t* __restrict__ ntpp) {
  __shared__ int cnt[kMaxLocal], start[kMaxLocal], tmp[1024];
  // the chunk counts (each at most kChunk, so 16 bits) when they fit: read once by all threads
  // with their loads in flight together, instead of twice by one thread per expert
  __shared__ uint16_t counts[kScanCache];
  int tid = threadIdx.x;
  const int64_t n = nchunks * nloc;
  if (n <= kScanCache) {
    constexpr int kLoads = 8;
    for (int64_t i0 = tid; i0 < n; i0 += kLoads * 1024) {
      int v[kLoads];
#pragma unroll
      for (int j = 0; j < kLoads; ++j) v[j] = i0 + j * 1024 < n ? hist[i0 + j * 1024] : 0;
#pragma unroll
      for (int j = 0; j < kLoads; ++j)
        if (i0 + j * 1024 < n) counts[i0 + j * 1024] = (uint16_t)v[j];
    }
    __syncthreads();
    int c = 0;
    if (tid < nloc) {
      for (int64_t g = 0; g < nchunks; ++g) c += counts[g * nloc + tid];
      cnt[tid] = c;
    }
    int seg = (tid < nloc) ? (c + block_m - 1) / block_m * block_m : 0;
    int P;
    int excl = block_excl_scan_1024(seg, tmp, P);
    if (tid < nloc) {
      start[tid] = excl;
      int pos = excl;
      for (int64_t g = 0; g < nchunks; ++g) {
        const int v = counts[g * nloc + tid];
        hist[g * nloc + tid] = pos;
        pos += v;
      }
      fr[tid] = c;
      fr[nloc + tid] = excl;
    }
    if (tid == 0) *ntpp = P;
    return;
  }
  // the chunk histograms are read kBatch at a time (independent loads in flight together)
  constexpr int kBatch = 16;
  int c = 0;
  if (tid < nloc) {
    for (int64_t g0 = 0; g0 < nchunks; g0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) v[i] = g0 + i < nchunks ? hist[(g0 + i) * nloc + tid] : 0;
#pragma unroll
      for (int i = 0; i < kBatch; ++i) c += v[i];
    }
    cnt[tid] = c;
  }
  int seg = (tid < nloc) ? (c + block_m - 1) / block_m * block_m : 0;
  int P;
  int excl = block_excl_scan_1024(seg, tmp, P);
  if (tid < nloc) {
    start[tid] = excl;
    int pos = excl;
    for (int64_t g0 = 0; g0 < nchunks; g0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) v[i] = g0 + i < nchunks ? hist[(g0 + i) * nloc + tid] : 0;
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        if (g0 + i < nchunks) hist[(g0 + i) * nloc + tid] = pos;
        pos += v[i];
      }
    }
    fr[tid] = c;
    fr[nloc + tid] = excl;
  }
  if (tid == 0) *ntpp = P;
}

// Ranks and scatters the slots of chunk blockIdx.x: wave w takes the slots of quarter w of the
// chunk, starting each local expert at the chunk's position plus the counts of the earlier
// quarters, so that the slots still land in ascending order within each expert.  The
// workgroups also share out the plan frame (expert_ids, the padding entries of every segment,
// the sentinel tail up to the capacity) from the counts and starts the scan published in fr.
__global__ __launch_bounds__(64 * kScatterWaves) void plan_scatter_kernel(
    const int32_t* __restrict__ ids, int64_t A, int num_experts, int offset, int nloc,
    const int32_t* __restrict__ pos0, const int32_t* __restrict__ fr,
    const int32_t* __restrict__ ntpp, int block_m, int64_t cap, int32_t* __restrict__ sorted,
    int32_t* __restrict__ eids, int32_t* __restrict__ ttr) {
  __shared__ int run[kScatterWaves * kMaxLocal];
  constexpr int kThreads = 64 * kScatterWaves, kSub = kChunk / kScatterWaves;
  static_assert(kSub == kThreads, "one slot of each quarter per thread in the count");
  const int tid = threadIdx.x, w = tid >> 6;
  const int64_t f0 = (int64_t)blockIdx.x * kChunk;
  const int64_t f1 = f0 + kChunk < A ? f0 + kChunk : A;
  for (int i = tid; i < kScatterWaves * nloc; i += kThreads) run[i] = 0;
  // the local ids of slot f0 + tid of every quarter, loads in flight together
  int ev[kScatterWaves];
#pragma unroll
  for (int q = 0; q < kScatterWaves; ++q) {
    const int64_t f = f0 + (int64_t)q * kSub + tid;
    ev[q] = f < f1 ? ids[f] : -1;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kScatterWaves; ++q) {
    const int e = local_id(ev[q], num_experts, offset, nloc);
    if (e >= 0) atomicAdd(&run[q * nloc + e], 1);
  }
  __syncthreads();
  // counts -> starting positions of each quarter, per expert
  for (int e = tid; e < nloc; e += kThreads) {
    int p = pos0[(int64_t)blockIdx.x * nloc + e];
#pragma unroll
    for (int q = 0; q < kScatterWaves; ++q) {
      const int c = run[q * nloc + e];
      run[q * nloc + e] = p;
      p += c;
    }
  }
  __syncthreads();
  const int64_t s0 = f0 + (int64_t)w * kSub;
  const int64_t s1 = s0 + kSub < f1 ? s0 + kSub : f1;
  if (s0 < s1) scatter_wave(ids, s0, s1, num_experts, offset, nloc, run + w * nloc, sorted, ttr);

  // plan frame.  Expert e = blockIdx.x + gridDim.x * (w + kScatterWaves * k) goes to wave w of
  // this workgroup: its lanes read the counts and starts of 64 such experts at a time, then the
  // wave writes each segment's block ids and padding entries with consecutive lanes on
  // consecutive words.
  const int lane = tid & 63;
  const int sentinel = (int)A;
  const int64_t stride_e = (int64_t)gridDim.x * kScatterWaves;
  for (int64_t k0 = 0; blockIdx.x + (int64_t)gridDim.x * w + stride_e * k0 < nloc; k0 += 64) {
    const int64_t el = blockIdx.x + (int64_t)gridDim.x * w + stride_e * (k0 + lane);
    const int c_l = el < nloc ? fr[el] : 0;
    const int s_l = el < nloc ? fr[nloc + el] : 0;
    for (int j = 0; j < 64; ++j) {
      const int64_t e = blockIdx.x + (int64_t)gridDim.x * w + stride_e * (k0 + j);
      if (e >= nloc) break;
      const int c = __builtin_amdgcn_readlane(c_l, j);
      if (c == 0) continue;
      const int st = __builtin_amdgcn_readlane(s_l, j);
      const int seg = (c + block_m - 1) / block_m * block_m;
      for (int b = st / block_m + lane; b < (st + seg) / block_m; b += 64) eids[b] = (int)e;
      for (int q = st + c + lane; q < st + seg; q += 64) sorted[q] = sentinel;
    }
  }
  // the tail past the extent P, in one slice per workgroup
  const int64_t P = *ntpp;
  const int64_t nb0 = P / block_m, nb1 = cap / block_m;
  const int64_t bl = (nb1 - nb0 + gridDim.x - 1) / gridDim.x;
  const int64_t b_lo = nb0 + bl * blockIdx.x, b_hi = b_lo + bl < nb1 ? b_lo + bl : nb1;
  for (int64_t b = b_lo + tid; b < b_hi; b += kThreads) eids[b] = -1;
  const int64_t pl = (cap - P + gridDim.x - 1) / gridDim.x;
  const int64_t p_lo = P + pl * blockIdx.x, p_hi = p_lo + pl < cap ? p_lo + pl : cap;
  for (int64_t p = p_lo + tid; p < p_hi; p += kThreads) sorted[p] = sentinel;
}

}  // namespace

hipError_t launch_plan_quantize(const int32_t* ids, int64_t A, int num_experts, int offset,
                                int nloc, int block_m, int32_t* sorted, int32_t* eids,
                                int32_t* ntpp, int32_t* ttr, int64_t cap, const uint16_t* x,
                                int64_t rows, int64_t cols, int64_t stride, uint8_t* q,
                                uint8_t* sf, float* dec, hipStream_t s) {
  KernelTimer t("plan_quantize", s);
  hipLaunchKernelGGL(plan_quantize_kernel, dim3((unsigned)(1 + rows)), dim3(1024), 0, s, ids, A,
                     num_experts, offset, nloc, block_m, sorted, eids, ntpp, ttr, cap, x, cols,
                     stride, q, sf, dec);
  return hipGetLastError();
}

bool plan_uses_small_kernel(int64_t A) { return A <= kSmallMax; }
int64_t plan_chunks(int64_t A) { return (A + kChunk - 1) / kChunk; }

hipError_t launch_plan(const int32_t* ids, int64_t A, int top_k, int num_experts, int offset,
                       int nloc, int block_m, int32_t* sorted, int32_t* eids, int32_t* ntpp,
                       int32_t* ttr, int64_t cap, void* ws, hipStream_t s) {
  (void)top_k;
  if (plan_uses_small_kernel(A)) {
    KernelTimer t("plan_small", s);
    hipLaunchKernelGGL(plan_small_kernel, dim3(1), dim3(1024), 0, s, ids, A, num_experts, offset,
                       nloc, block_m, sorted, eids, ntpp, ttr, cap);
    return hipGetLastError();
  }
  int64_t nch = plan_chunks(A);
  int32_t* hist = static_cast<int32_t*>(ws);
  {
    KernelTimer t("plan_count", s);
    hipLaunchKernelGGL(plan_count_kernel, dim3((unsigned)nch), dim3(256), 0, s, ids, A,
                       num_experts, offset, nloc, hist);
  }
  {
    KernelTimer t("plan_scan", s);
    hipLaunchKernelGGL(plan_scan_kernel, dim3(1), dim3(1024), 0, s, hist, nch, nloc, block_m,
                       hist + nch * nloc, ntpp);
  }
  KernelTimer t("plan_scatter", s);
  hipLaunchKernelGGL(plan_scatter_kernel, dim3((unsigned)nch), dim3(64 * kScatterWaves), 0, s, ids,
                     A, num_experts, offset, nloc, hist, hist + nch * nloc, ntpp, block_m, cap,
                     sorted, eids, ttr);
  return hipGetLastError();
}

}  // namespace bfp4
