// Block-scaled grouped GEMMs of the routed MoE on gfx950 MFMA, and the weight panel layout.
//
// What is computed (FlashInfer "flashinfer.fused_moe.alphamoe_nvfp4_aligned_moe": gate/up GEMM,
// SwiGLU, requantization and down GEMM on a pre-aligned plan, FP32 accumulation, per-expert
// output scales; "flashinfer.fused_moe.CudnnGroupedGemmNvfp4Config": GEMM1 rows times the
// expert's global dequant, BF16 intermediate re-quantized with a global scale of one;
// "flashinfer.fused_moe.FrostLowLatencyConfig": BF16 intermediate and BF16 expert outputs):
//   GEMM1  pre = (sum_h a[t,h] w1_e[n,h]) * s_tok * alpha1   ->  SwiGLU / ReLU^2  ->  BF16  ->
//          NVFP4 with fixed encode scale c2 (written in plan-row order, GEMM2's operand layout)
//   GEMM2  y = bf16((sum_i hq[r,i] w2_e[k,i]) * (1/c2) * alpha2)
//
// How (gfx950 design):
// * Operands are NVFP4 in memory and decoded exactly to FP16 in registers (every E2M1 x E4M3
//   product is exact in FP16), then fed to v_mfma_f32_32x32x16_f16 with FP32 accumulation.
// * MFMA A operand = 32 weight rows, B operand = 32 plan rows (tokens).  Weights stream from HBM
//   straight into registers (no LDS), one 16-byte load per lane per 64 K values.
// * Prefill: a workgroup of 8 waves (two per SIMD) owns a tile of up to 256 plan rows of one
//   expert and 8 weight row groups (one n-tile; the down GEMM streams up to 4 n-tiles of a tile
//   through one pipeline); the tile's token rows are copied per 128-K stage from an exact FP16
//   copy into LDS by direct buffer-to-LDS loads and shared by the 8 waves; each wave decodes its
//   own row group once per tile and multiplies it by every token fragment of the tile.
// * Decode: the few routed rows of a plan block are staged packed in LDS once; each wave then
//   streams its weight row groups without further barriers.
// * Weight panels put, for each 32-row group and each 64-value K chunk, exactly the 1 KiB a wave
//   loads in one instruction (lane l: row l%32, K half l/32), scales grouped per 512 K values.
// * Inside a 32-row group the rows are permuted so that each lane's 16 accumulator rows are 16
//   consecutive logical rows: the requantization block (16 values) stays within a lane pair, and
//   a GEMM2 lane stores 32 contiguous bytes.  A gated W1 group holds the gate rows of 16
//   intermediate indices in its first 16 logical rows and the up rows of the same indices in
//   the last 16, so the SwiGLU epilogue pairs lane l with lane l + 32.
// * Plan rows past the device-side extent, padding rows and 32-row token fragments with no valid
//   row are skipped.  Prefill tasks are handed out dynamically from one ticket queue per XCD;
//   the decode grid covers (plan block, row groups) tasks with a static stride.
#include <atomic>
#include <type_traits>
#include <utility>

#include "bfp4moe.h"
#include "device.h"
#include "runtime.h"

namespace bfp4 {

namespace {

constexpr int kGroupRows = 32;      // weight rows per MFMA A fragment
constexpr int kChunkK = 64;         // K values per 1 KiB data unit
constexpr int kSuperChunks = 8;     // chunks sharing one 1 KiB scale unit
constexpr int kUnit = 1024;
constexpr int kSuperBytes = (kSuperChunks + 1) * kUnit;
constexpr int kStageChunks = 2;     // chunks per pipeline stage (128 K values)
constexpr int kTokPitch = 256;      // LDS bytes per token row per stage: 128 FP16, swizzled slots
constexpr int kTokRegion = 128 * 1024;   // LDS bytes of prefill token stage buffers
constexpr int kTileRows = 256;      // plan rows per prefill tile (8 token fragments)
constexpr int kTileGroups = 8;      // weight row groups per prefill task (one per wave)
constexpr int kXcds = 8;            // accelerator complex dies (each with its own L2)
constexpr int kSpreadSteps = 4;     // 16-K steps of a stage over which its token loads go out
constexpr int kChainGemm1 = 1;      // prefill n-tiles per task, gate/up GEMM
static_assert(kChainGemm1 == 1, "the gate/up GEMM kernel runs one n-tile per task");
constexpr int kChainGemm2 = 4;      // prefill n-tiles per task, down GEMM (2 for short lists)
constexpr int kMinTasksPerCu = 6;   // down GEMM: fewer tasks per CU at kChainGemm2 halve it
constexpr int kCus = 256;           // compute units (one persistent workgroup each)

// Logical row (within a 32-row group) held at physical row rho: the MFMA 32x32 accumulator of
// lane l holds rows 8i + 4*(l/32) + j (i, j in 0..3); they are made logical rows
// 16*(l/32) + 4i + j.
__host__ __device__ __forceinline__ int group_perm(int rho) {
  return 16 * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3);
}

struct PanelGeom {
  int64_t ng, nch, nsc, rg_bytes, expert_bytes;
};

__host__ __device__ inline PanelGeom panel_geom(int64_t rows, int64_t K) {
  PanelGeom g;
  g.ng = rows / kGroupRows;
  g.nch = K / kChunkK;
  g.nsc = (g.nch + kSuperChunks - 1) / kSuperChunks;
  g.rg_bytes = (g.nsc + g.nch) * kUnit;
  g.expert_bytes = g.ng * g.rg_bytes;
  return g;
}

// One thread per 16-byte piece of the panel of one matrix type.
__global__ void prepare_kernel(const uint8_t* __restrict__ w_q, const uint8_t* __restrict__ w_sf,
                               int64_t rows, int64_t K, int64_t half_rows, int64_t total_pieces,
                               uint8_t* __restrict__ panel, int mx) {
  int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= total_pieces) return;
  PanelGeom g = panel_geom(rows, K);
  int lane = (int)(p & 63);
  int64_t unit = p >> 6;
  int64_t per_expert = g.ng * (g.nsc + g.nch);
  int64_t e = unit / per_expert;
  int64_t rem = unit - e * per_expert;
  int64_t grp = rem / (g.nsc + g.nch);
  int64_t u = rem - grp * (g.nsc + g.nch);
  int64_t sc = u / (kSuperChunks + 1);
  int64_t j = u - sc * (kSuperChunks + 1);
  int rho = lane & 31, h = lane >> 5;
  int64_t lr;
  if (half_rows > 0) {          // gated W1: gate rows 16*grp.. then the up rows of the same indices
    const int gp = group_perm(rho);
    lr = (gp >= 16 ? half_rows : 0) + grp * 16 + (gp & 15);
  } else {
    lr = grp * kGroupRows + group_perm(rho);
  }
  int64_t row = e * rows + lr;
  uint4 out;
  if (j == 0) {                 // scale unit: 2 bytes per chunk of the superchunk
    uint32_t b[16];
#pragma unroll
    for (int jj = 0; jj < kSuperChunks; ++jj) {
      int64_t c = sc * kSuperChunks + jj;
      bool ok = c < g.nch;
      if (mx) {                 // one E8M0 scale per 32 values fills both 16-value slots
        const uint8_t* s = w_sf + row * (K / 32) + 2 * c + h;
        b[2 * jj] = ok ? s[0] : 0u;
        b[2 * jj + 1] = ok ? s[0] : 0u;
      } else {
        const uint8_t* s = w_sf + row * (K / 16) + 4 * c + 2 * h;
        b[2 * jj] = ok ? s[0] : 0u;
        b[2 * jj + 1] = ok ? s[1] : 0u;
      }
    }
    out.x = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
    out.y = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
    out.z = b[8] | (b[9] << 8) | (b[10] << 16) | (b[11] << 24);
    out.w = b[12] | (b[13] << 8) | (b[14] << 16) | (b[15] << 24);
  } else {
    int64_t c = sc * kSuperChunks + (j - 1);
    out = *reinterpret_cast<const uint4*>(w_q + row * (K / 2) + c * 32 + h * 16);
  }
  *reinterpret_cast<uint4*>(panel + p * 16) = out;
}

struct GemmArgs {
  // token operand
  const uint8_t* a_q;
  const uint8_t* a_sf;
  int64_t a_rows;            // rows of a_q / a_sf (and of t16)
  const uint16_t* t16;       // prefill: exact FP16 copy of the token operand [a_rows, K]
  int64_t t16_rowb;          // bytes per t16 row (2 K)
  const float* a_dec;        // per-token decode scale (gather) or nullptr
  float a_const_scale;       // decode scale when a_dec is nullptr
  int64_t a_rowq;            // bytes per packed token row (K/2)
  int gather;                // 1: token = entry / top_k;  0: token row = plan row
  // plan
  const int32_t* sorted;
  const int32_t* eids;
  const int32_t* ntpp;
  int64_t cap;
  int64_t sentinel;
  int top_k, block_m, nloc;
  const int2* tiles;         // prefill tiles {first row, rows}, ordered by length
  const int32_t* n_tiles;
  uint32_t* task_counter;    // prefill: one ticket counter per XCD queue (cleared by the tile list)
  // weights
  const uint8_t* panel;
  int64_t expert_bytes, rg_bytes;
  int nch, N, n_nt;
  int chain, n_ct;           // prefill: n-tiles per task and tasks per tile (ceil(n_nt / chain))
  const float* alpha_a;      // GEMM1: alpha1_gate; GEMM2: alpha2
  const float* alpha_b;      // GEMM1: alpha1_up
  // GEMM1 epilogue
  int act;                   // activation code (EPI_ACT picks GELU, ReLU, SiLU or Identity by it)
  float c2;
  int64_t I;
  uint8_t* hq;               // null: the NVFP4 intermediate is not stored
  uint8_t* hsf;
  uint16_t* h16;             // prefill: FP16 copy of the requantized intermediate [cap, I] or null
  float* dbg_pre;
  uint16_t* dbg_inter;
  // GEMM2 epilogue
  uint16_t* y;
  int64_t Hout;
  // weight-only mode (BF16 token operand): token rows (x for GEMM1, the BF16 intermediate for
  // GEMM2) with their row stride in elements, and GEMM1's BF16 intermediate output [cap, I]
  const uint16_t* w16_x;
  int64_t w16_stride;
  uint16_t* w16_h;
};

// Epilogues: the two GEMM1 forms the hot paths use (SwiGLU, squared ReLU), the down GEMM, GeGLU,
// and the remaining one-projection activations (GELU, ReLU, SiLU, Identity) chosen at run time.
enum { EPI_SWIGLU = 0, EPI_RELU2 = 1, EPI_DOWN = 2, EPI_GEGLU = 3, EPI_ACT = 4 };

// GEMM1 epilogues whose intermediate value i comes from one pre-activation (no gate/up pairs)
constexpr bool one_projection(int epi) { return epi == EPI_RELU2 || epi == EPI_ACT; }


// Prefill tile list, built on the device from the plan by one workgroup before GEMM1:
//  1. tiles in plan order: for block_m < kTileRows, up to kTileRows / block_m consecutive plan
//     blocks of one local expert segment (aligned to the segment's first block); otherwise
//     kTileRows-row slices of each block of a local expert;
//  2. each tile's token-fragment count (up to its last routed row), tiles ranked by it
//     (counting sort) and handed to the dynamic schedule of the GEMMs either longest first
//     (the FP16-MFMA kernels) or interleaved longest / shortest (the MX kernels), whichever
//     measured faster for each;
//  3. the GEMMs' per-XCD ticket counters are cleared.
// tmp holds max_tiles int2 + max_tiles int; tiles max_tiles int2.
__device__ void tile_list_body(
    const int32_t* __restrict__ eids, const int32_t* __restrict__ sorted,
    const int32_t* __restrict__ ntpp, int64_t cap, int block_m, int64_t sentinel, int nloc,
    int2* __restrict__ tmp, int2* __restrict__ tiles, int32_t* __restrict__ n_tiles,
    uint32_t* __restrict__ counters, bool longest_first) {
  __shared__ int scan[1024];
  __shared__ int carry_start, carry_count;
  __shared__ int hist[9], offs[9];
  const int tid = threadIdx.x;
  int64_t P = *ntpp;
  if (P > cap) P = cap;
  if (P < 0) P = 0;
  const int nblk = (int)(P / block_m);
  const int tb = block_m < kTileRows ? kTileRows / block_m : 1;
  const int n_sub = block_m < kTileRows ? 1 : (block_m + kTileRows - 1) / kTileRows;
  if (tid == 0) {
    carry_start = 0;
    carry_count = 0;
  }
  if (tid < 9) hist[tid] = 0;
  __syncthreads();
  for (int base = 0; base < nblk; base += 1024) {
    const int b = base + tid;
    const bool valid = b < nblk;
    const int e = valid ? eids[b] : -2;
    const bool seg_start = valid && (b == 0 || eids[b - 1] != e);
    // inclusive max-scan of segment starts
    scan[tid] = seg_start ? b : -1;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      int v = (tid >= off) ? scan[tid - off] : -1;
      __syncthreads();
      scan[tid] = max(scan[tid], v);
      __syncthreads();
    }
    const int s0 = max(scan[tid], carry_start);
    const bool local = valid && e >= 0 && e < nloc;
    const int ntile = !local ? 0 : (tb > 1 ? ((b - s0) % tb == 0 ? 1 : 0) : n_sub);
    __syncthreads();
    // exclusive prefix sum of the tiles each block starts
    scan[tid] = ntile;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      int v = (tid >= off) ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const int first = carry_count + scan[tid] - ntile;
    const int total = scan[1023];
    if (ntile > 0) {
      if (tb > 1) {
        int nb = 1;
        while (nb < tb && b + nb < nblk && eids[b + nb] == e) ++nb;
        tmp[first] = make_int2(b * block_m, nb * block_m);
      } else {
        for (int u = 0; u < n_sub; ++u)
          tmp[first + u] = make_int2(b * block_m + u * kTileRows,
                                     min(kTileRows, block_m - u * kTileRows));
      }
    }
    __syncthreads();                         // every thread has read carry_start/count
    if (tid == min(1023, nblk - 1 - base)) carry_start = s0;
    if (tid == 0) carry_count += total;
    __syncthreads();
  }
  const int nt_all = carry_count;
  int* nfw_of = reinterpret_cast<int*>(tmp + nt_all);
  __syncthreads();
  for (int t = tid; t < nt_all; t += 1024) {
    // last routed row by bisection (an expert segment holds its routed rows first, then the
    // padding); the count only orders the tiles, the GEMMs find each tile's rows themselves
    const int2 tl = tmp[t];
    int lo = -1, hi = tl.y;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      const int ent = sorted[tl.x + mid];
      if (ent >= 0 && ent < sentinel) lo = mid;
      else hi = mid;
    }
    const int nfw = max(1, (lo + 32) >> 5);
    nfw_of[t] = nfw;
    atomicAdd(&hist[nfw], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int f = 8; f >= 1; --f) {             // rank 0: most fragments
      offs[f] = acc;
      acc += hist[f];
    }
    offs[0] = acc;
    *n_tiles = acc;
    for (int c = 0; c < 2 * kXcds; ++c) counters[c] = 0u;
  }
  __syncthreads();
  // rank r in decreasing fragment count -> position: r itself (the long tiles first, so the
  // short ones fill the end of the schedule), or the longest and the shortest tiles
  // alternating (r0, r(n-1), r1, r(n-2), ...), so that the tasks in flight at any time mix
  // MFMA-bound and weight-streaming-bound tiles
  const int n = offs[0];
  for (int t = tid; t < nt_all; t += 1024) {
    const int r = atomicAdd(&offs[nfw_of[t]], 1);
    const int pos = longest_first ? r : (r < (n + 1) / 2) ? 2 * r : 2 * (n - 1 - r) + 1;
    tiles[pos] = tmp[t];
  }
}

__global__ __launch_bounds__(1024) void tile_list_kernel(
    const int32_t* __restrict__ eids, const int32_t* __restrict__ sorted,
    const int32_t* __restrict__ ntpp, int64_t cap, int block_m, int64_t sentinel, int nloc,
    int2* __restrict__ tmp, int2* __restrict__ tiles, int32_t* __restrict__ n_tiles,
    uint32_t* __restrict__ counters) {
  tile_list_body(eids, sorted, ntpp, cap, block_m, sentinel, nloc, tmp, tiles, n_tiles, counters,
                 false);
}

// Exact FP16 copy of NVFP4 rows (E2M1 x E4M3, without the row's FP32 decode scale) for the
// values v0 = 8 i .. 8 i + 7 (8 values never straddle a row).
__device__ __forceinline__ void decode_rows_unit(const uint8_t* __restrict__ q,
                                                 const uint8_t* __restrict__ sf, int64_t i,
                                                 uint16_t* __restrict__ out) {
  const int64_t v0 = i * 8;
  const uint32_t w = *reinterpret_cast<const uint32_t*>(q + (v0 >> 1));
  const uint32_t sb = sf[v0 >> 4];
  *reinterpret_cast<h8_t*>(out + v0) = decode8(w, e4m3_scale_h2(sb));
}

// The NVFP4 prefill's two preparations of GEMM1 in one launch, as they are independent:
// workgroup 0 builds the tile list (tile_list_body), workgroup 1 + j decodes the activation
// values 8192 j .. 8192 j + 8191 into their exact FP16 copy (one thread per 8 values).
__global__ __launch_bounds__(1024) void tile_list_decode_kernel(
    const int32_t* __restrict__ eids, const int32_t* __restrict__ sorted,
    const int32_t* __restrict__ ntpp, int64_t cap, int block_m, int64_t sentinel, int nloc,
    int2* __restrict__ tmp, int2* __restrict__ tiles, int32_t* __restrict__ n_tiles,
    uint32_t* __restrict__ counters, const uint8_t* __restrict__ q,
    const uint8_t* __restrict__ sf, int64_t n8, uint16_t* __restrict__ out) {
  if (blockIdx.x == 0) {
    tile_list_body(eids, sorted, ntpp, cap, block_m, sentinel, nloc, tmp, tiles, n_tiles,
                   counters, true);
    return;
  }
  const int64_t i = (int64_t)(blockIdx.x - 1) * 1024 + threadIdx.x;
  if (i < n8) decode_rows_unit(q, sf, i, out);
}

struct Smem {
  uint8_t* tok;         // token stage buffers (kTokRegion bytes)
  int* row_src;
  float* row_scale;
  int* sh_nvalid;
  int* sh_task;
};


// SiLU x / (1 + e^-x) with the hardware exponential (2^y) and reciprocal, each within a few ulp
// of FP32: the result is rounded to BF16 next.  Saturates to -0 for large negative x (e^-x
// overflows to infinity, whose reciprocal is 0) and to x for large positive x.
__device__ __forceinline__ float silu(float x) {
  const float e = __builtin_amdgcn_exp2f(x * -1.44269504088896341f);
  return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// GELU in its erf form, x * Phi(x) with Phi(x) = erfc(-x / sqrt 2) / 2: the complementary error
// function keeps Phi's relative accuracy for large negative x, where 1 + erf(x / sqrt 2) would
// cancel.
__device__ __forceinline__ float gelu(float x) {
  return 0.5f * x * erfcf(x * -0.70710678118654752f);
}

// The one-projection activations other than squared ReLU, by activation code.
__device__ __forceinline__ float act_one(float x, int act) {
  if (act == BFP4_ACT_GELU) return gelu(x);
  if (act == BFP4_ACT_RELU) return x > 0.0f ? x : 0.0f;
  if (act == BFP4_ACT_SILU) return silu(x);
  return x;                                        // Identity
}

// Epilogue of one weight row group g for the plan row r of this lane's token column; the lane
// holds the group's logical rows 16h .. 16h + 15.
//   down:    outputs 32g + 16h + v  ->  BF16, 32 contiguous bytes per lane
//   ReLU^2:  intermediate 32g + 16h + v, one requantization block per lane
//   SwiGLU:  h = 0 holds gate, h = 1 up of intermediate 16g + v; lane h = 0 keeps 16g + 0..7 and
//            lane h = 1 keeps 16g + 8..15 after swapping halves with its partner (lane ^ 32);
//            the requantization block is the pair's 16 values.
// al is the lane's per-expert output scale (lane_alpha), read before the main loop so that its
// load latency is hidden.
template <int EPI>
__device__ __forceinline__ float lane_alpha(const GemmArgs& a, int e, int h) {
  if (EPI == EPI_DOWN) return a.alpha_a[e];
  if (one_projection(EPI)) return a.alpha_b[e];
  return h ? a.alpha_b[e] : a.alpha_a[e];
}

// O32: the intermediate's element offsets (r * I) fit in 32 bits (the tiled kernels' operands are
// checked to be below 2^31 bytes), so they are formed with 32-bit products.
template <int EPI, bool O32 = false>
__device__ __forceinline__ void epilogue_group(const GemmArgs& a, const f32x16_t& acc, float al,
                                               int64_t g, int h, float s_row, int64_t r) {
  // r * I / 16 (I is a multiple of 128); with O32, r < 2^23 (r * I * 2 < 2^31, I >= 128), so a
  // 24-bit product
  const int64_t r16 = O32 ? (int64_t)__umul24((uint32_t)r, (uint32_t)(a.I >> 4)) : r * (a.I >> 4);
  auto roff = [&](int64_t stride) -> int64_t {   // stride is I / 2, I / 16 or I
    return stride == (a.I >> 1) ? r16 << 3 : stride == (a.I >> 4) ? r16 : r16 << 4;
  };
  if (EPI == EPI_DOWN) {
    const float a2 = al;
    const int64_t k0 = g * kGroupRows + 16 * h;
    uint32_t pk[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const float y0 = (acc[2 * v] * s_row) * a2;
      const float y1 = (acc[2 * v + 1] * s_row) * a2;
      pk[v] = f32_to_bf16(y0) | (f32_to_bf16(y1) << 16);
    }
    uint4* dst = reinterpret_cast<uint4*>(a.y + r * a.Hout + k0);
    dst[0] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    dst[1] = make_uint4(pk[4], pk[5], pk[6], pk[7]);
    return;
  }
  if (one_projection(EPI)) {
    const float au = al;
    const int64_t i0 = g * kGroupRows + 16 * h;
    float pr[16], hv[16];
    uint32_t bb[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      pr[v] = (acc[v] * s_row) * au;
      if (EPI == EPI_RELU2) {
        const float q = pr[v] > 0.0f ? pr[v] : 0.0f;
        bb[v] = f32_to_bf16(q * q);
      } else {
        bb[v] = f32_to_bf16(act_one(pr[v], a.act));
      }
      hv[v] = bf16_to_f32(bb[v]);
    }
    if (a.dbg_pre) {
      float4* dp = reinterpret_cast<float4*>(a.dbg_pre + r * a.I + i0);
#pragma unroll
      for (int v = 0; v < 4; ++v)
        dp[v] = make_float4(pr[4 * v], pr[4 * v + 1], pr[4 * v + 2], pr[4 * v + 3]);
    }
    if (a.dbg_inter) {
      uint4* d = reinterpret_cast<uint4*>(a.dbg_inter + r * a.I + i0);
      d[0] = make_uint4(bb[0] | (bb[1] << 16), bb[2] | (bb[3] << 16), bb[4] | (bb[5] << 16),
                        bb[6] | (bb[7] << 16));
      d[1] = make_uint4(bb[8] | (bb[9] << 16), bb[10] | (bb[11] << 16), bb[12] | (bb[13] << 16),
                        bb[14] | (bb[15] << 16));
    }
    uint32_t lo, hi;
    const uint32_t sfb = quant_block16(hv, a.c2, lo, hi);
    if (a.hq) {                  // the tiled down GEMM reads only h16: hq is debug output there
      *reinterpret_cast<uint2*>(a.hq + roff(a.I >> 1) + (i0 >> 1)) = make_uint2(lo, hi);
      a.hsf[roff(a.I >> 4) + (i0 >> 4)] = (uint8_t)sfb;
    }
    if (a.h16) {                 // the same values, E2M1 x E4M3 exactly in FP16
      h8_t* d = reinterpret_cast<h8_t*>(a.h16 + roff(a.I) + i0);
      d[0] = decode8(lo, e4m3_scale_h2(sfb));
      d[1] = decode8(hi, e4m3_scale_h2(sfb));
    }
    return;
  }
  // SwiGLU, GeGLU
  const int64_t i0 = g * 16;
  float pre[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) pre[v] = (acc[v] * s_row) * al;
  if (a.dbg_pre) {
    float4* dp = reinterpret_cast<float4*>(a.dbg_pre + r * (2 * a.I) + h * a.I + i0);
#pragma unroll
    for (int v = 0; v < 4; ++v)
      dp[v] = make_float4(pre[4 * v], pre[4 * v + 1], pre[4 * v + 2], pre[4 * v + 3]);
  }
  float hv[8];
  uint32_t bb[8];
  float bmax = 0.0f;
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    // one lane swap gives every lane its gate and up value: lanes 0..31 keep pre[v] (gate of
    // 16g + v) and take their partner's pre[v] (up of 16g + v); lanes 32..63 take their
    // partner's pre[8 + v] (gate of 16g + 8 + v) and keep pre[8 + v] (up)
    const auto gu = __builtin_amdgcn_permlane32_swap(__float_as_uint(pre[v]),
                                                     __float_as_uint(pre[8 + v]), false, false);
    const float gt = __uint_as_float(gu[0]);
    const float up = __uint_as_float(gu[1]);
    bb[v] = f32_to_bf16((EPI == EPI_GEGLU ? gelu(gt) : silu(gt)) * up);
    hv[v] = bf16_to_f32(bb[v]);
    bmax = __builtin_fmaxf(bmax, __builtin_fabsf(hv[v]));
  }
  const int64_t ih = i0 + 8 * h;
  if (a.dbg_inter) {
    *reinterpret_cast<uint4*>(a.dbg_inter + r * a.I + ih) =
        make_uint4(bb[0] | (bb[1] << 16), bb[2] | (bb[3] << 16), bb[4] | (bb[5] << 16),
                   bb[6] | (bb[7] << 16));
  }
  {
    const auto mm = __builtin_amdgcn_permlane32_swap(__float_as_uint(bmax), __float_as_uint(bmax),
                                                     false, false);
    bmax = __builtin_fmaxf(__uint_as_float(mm[0]), __uint_as_float(mm[1]));   // this lane, partner
  }
  float inv;
  const uint32_t sfb = block_scale(bmax, a.c2, inv);
  const uint32_t codes = quant8(hv, inv);
  if (a.hq) {
    *reinterpret_cast<uint32_t*>(a.hq + roff(a.I >> 1) + (ih >> 1)) = codes;
    if (h == 0) a.hsf[roff(a.I >> 4) + (i0 >> 4)] = (uint8_t)sfb;
  }
  if (a.h16)                     // the same values, E2M1 x E4M3 exactly in FP16
    *reinterpret_cast<h8_t*>(a.h16 + roff(a.I) + ih) = decode8(codes, e4m3_scale_h2(sfb));
}

// f(integral_constant<int, I>) for I = 0, 1, ... in order
template <typename F, int... Is>
__device__ __forceinline__ void unroll_seq(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}

// Prefetch depths of a prefill tile with NFW token fragments, in 128-K stages: the weights of
// stage st + RW - 1 are loaded into registers and the FP16 token rows of stage st + NB - 1 into
// LDS while stage st computes.  A stage of token rows takes NFW * 8 KiB of the 128 KiB region,
// so short tiles (short stages) look further ahead.
template <int NFW, int G, int EPI> struct TileDepth {
  // 3 stages for short gate/up tiles measured faster than 4; the down GEMM keeps 4, which
  // divides its 16 stages per n-tile so that n-tiles stream through one pipeline.  With two
  // row groups per wave the weight ring takes twice the registers.
  static constexpr int RW = G == 2 ? (NFW <= 2 ? (EPI == EPI_DOWN ? 4 : 3) : 2)
                                   : NFW <= 4 ? (EPI == EPI_DOWN ? 4 : 3) : 2;
  static constexpr int NB0 = kTokRegion / (NFW * 32 * kTokPitch);
  static constexpr int NB = NB0 > 8 ? 8 : NB0;
};

// One prefill tile of up to kTileRows plan rows of one expert, against G n-tiles of kTileGroups
// weight row groups each.  Eight waves, two per SIMD: wave w owns row group g = kTileGroups * nt
// + w of each of the G n-tiles nt and all NFW token fragments of the tile (32 * NFW plan rows),
// so each weight fragment is decoded once per tile.  With G = 2 (short down-GEMM tiles) every
// token operand read from LDS feeds two MFMAs, and the tile's token rows are copied into LDS
// half as often.  The token operand comes from an exact FP16 copy (the decoded activations for
// GEMM1, the dequantized intermediate for GEMM2) and is copied into LDS by direct buffer-to-LDS
// loads: per 128-K stage each wave moves 4 rows of every fragment (one 1 KiB load per fragment),
// into a ring of NB stage buffers.  Inside a buffer row r's 16-byte slot u (K values 8u .. 8u+7
// of the stage) sits at slot u ^ (r & 15), so the MFMA operand reads are free of bank conflicts.
// Per 16-K step a wave issues its G * NFW MFMAs, each fragment's followed by the LDS read that
// refills the same token register for the next step, and decodes its weight fragments of the
// next step.  The task's n-tiles nt0 .. nt0 + nchain - 1 are taken G at a time (units); a unit
// past the matrix's last n-tile loads group 0 and skips its epilogue.
template <int NFW, int G, int EPI>
__device__ __forceinline__ void run_tile(const GemmArgs& a, const Smem& sm, int e, int nt0,
                                         int nchain, int64_t row0) {
  static_assert(NFW >= 1 && NFW <= 8, "at most 8 token fragments per tile");
  static_assert(G == 1 || (G == 2 && NFW <= 4), "two n-tiles at once for short tiles only");
  constexpr int RW = TileDepth<NFW, G, EPI>::RW, NB = TileDepth<NFW, G, EPI>::NB;
  static_assert(RW >= 2 && RW <= 8, "weight ring of 2 to 8 stages");
  static_assert(NB >= 2, "at least two token stage buffers");
  constexpr int SBUF = NFW * 32 * kTokPitch;      // bytes of one stage buffer
  // vector memory operations a wave issues per stage: 3 G weight loads, then NFW token loads
  constexpr int VM_W = 3 * G;
  constexpr int VM_STAGE = NFW + VM_W;
  // loads issued after the prologue's token load of stage 1: NB - 3 token stages, RW - 1 weight
  // stages, then stage 0's NFW + VM_W (the fewest behind any prologue-loaded stage).  The
  // prologue issues its token stages before its weight stages.
  constexpr int kEarlyWait = NB >= 3 ? (NB - 3) * NFW + VM_W * (RW - 1) + VM_STAGE : 0;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, col = lane & 31;
  const int nst = a.nch / kStageChunks;

  // Weight loads go through a buffer resource over the expert's panel: lane offset in a VGPR,
  // row-group and stage offsets in SGPRs.  A wave past the last row group of its n-tile streams
  // group 0 (every load and MFMA is unconditional) and skips that n-tile's epilogue.
  const __amdgpu_buffer_rsrc_t wrs =
      make_rsrc(a.panel + (int64_t)e * a.expert_bytes, (uint32_t)a.expert_bytes);
  const int wlane = lane * 16;
  auto group_of = [&](int nt) { return nt * kTileGroups + wave; };
  auto group_on = [&](int nt) { return (group_of(nt) + 1) * kGroupRows <= a.N; };
  const int nunits = (nchain + G - 1) / G;          // units of G n-tiles

  // token rows: this lane moves row 32 i + 4 wave + lane / 16 of fragment i, physical slot
  // lane % 16, i.e. logical slot u_l; rows without a routed slot read row 0 (their MFMA columns
  // are discarded).  The FP16 token operand is smaller than 2^31 bytes (checked at the entry
  // point), so offsets are 32-bit.
  const int trow = 4 * wave + (lane >> 4);
  const uint32_t u_l = (uint32_t)((lane & 15) ^ (trow & 15));
  const uint32_t rowb = (uint32_t)a.t16_rowb;
  const __amdgpu_buffer_rsrc_t trs = make_rsrc(a.t16, (uint32_t)(a.a_rows * (int64_t)rowb));
  uint32_t t_voff[NFW];
#pragma unroll
  for (int i = 0; i < NFW; ++i) {
    int src = sm.row_src[32 * i + trow];
    src = src < 0 ? 0 : src;
    t_voff[i] = (uint32_t)src * rowb + u_l * 16;
  }
  uint8_t* const tok_wave = sm.tok + 4 * wave * kTokPitch;       // row 4 * wave of a buffer
  // LDS byte offset of this lane's operand in fragment 0, step q of a stage buffer
  const int swz = col & 15;
  auto t_off = [&](int q) {
    const int u = 8 * (q >> 2) + 4 * h + (q & 3);
    return col * kTokPitch + ((u ^ swz) << 4);
  };

  const float al = lane_alpha<EPI>(a, e, h);
  f32x16_t acc[G][NFW];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int j = 0; j < NFW; ++j) acc[g][j] = f32x16_t{};

  uint4 W[RW][G][kStageChunks];
  uint32_t S[RW][G];
  h8_t T[NFW];
  h8_t Wc[G];

  // weights of local stage st of row-group offset go (bytes): the scale dword (load_s) and
  // 64-value chunk c (load_w1)
  auto load_s = [&](int go, int st) {
    const int sc = st / (kSuperChunks / kStageChunks);
    const int c0 = (st * kStageChunks) % kSuperChunks;
    return buffer_load_u32(wrs, wlane, go + sc * kSuperBytes + 2 * c0);
  };
  auto load_w1 = [&](int go, int st, int c) {
    const int sc = st / (kSuperChunks / kStageChunks);
    const int c0 = (st * kStageChunks) % kSuperChunks;
    return buffer_load_u128(wrs, wlane + (1 + c) * kUnit, go + sc * kSuperBytes + c0 * kUnit);
  };
  // token rows of fragment i (load_t1) or of every fragment (load_t) of stage st into stage
  // buffer b
  auto load_t1 = [&](int b, int st, int i) {
    buffer_load_lds16(trs, tok_wave + b * SBUF + i * 32 * kTokPitch, t_voff[i],
                      (uint32_t)st * kTokPitch);
  };
  auto load_t = [&](int b, int st) {
#pragma unroll
    for (int i = 0; i < NFW; ++i) load_t1(b, st, i);
  };
  auto dec_w = [&](const uint4 (&Wd)[kStageChunks], uint32_t Sd, int q) {
    const int c = q >> 2, s = q & 3;
    const uint32_t wd = (s == 0) ? Wd[c].x : (s == 1) ? Wd[c].y : (s == 2) ? Wd[c].z : Wd[c].w;
    const uint32_t sb = (Sd >> (8 * (2 * c + (s >> 1)))) & 0xFFu;
    return decode8(wd, e4m3_scale_h2(sb));
  };
  auto read_all = [&](const uint8_t* buf, int q) {
#pragma unroll
    for (int j = 0; j < NFW; ++j)
      T[j] = *reinterpret_cast<const h8_t*>(buf + j * 32 * kTokPitch + t_off(q));
  };

  // n-tiles nt0 .. nt0 + nchain - 1 of the tile run as one stream of nchain * nst stages when
  // the weight ring divides nst (then every n-tile starts in weight slot 0); otherwise one
  // stream per n-tile.  Inside a stream the loads of the next n-tile's first stages are in flight
  // while the previous n-tile's epilogue runs.  Only the down GEMM streams several n-tiles: the
  // larger gate/up epilogues inside the stage loop would push its registers past the file.
  constexpr bool kStream = EPI == EPI_DOWN;
  const int cc = (kStream && nst % RW == 0) ? nunits : 1;
  for (int c0 = 0; c0 < nunits; c0 += cc) {
    const int ub = c0, cnt = kStream ? min(cc, nunits - c0) : 1;
    const int NS = cnt * nst;                 // stages of this stream
    // first n-tile of unit u; weight row-group byte offset of n-tile g of the unit of global
    // stage gs, and its local stage
    auto unit_nt = [&](int u) { return nt0 + G * u; };
    auto wgo = [&](int gs, int g) {
      const int nt = unit_nt(kStream ? ub + gs / nst : ub) + g;
      return (group_on(nt) ? group_of(nt) : 0) * (int)a.rg_bytes;
    };
    auto local = [&](int gs) { return kStream ? gs % nst : gs; };
    auto load_w = [&](uint4 (&Wd)[G][kStageChunks], uint32_t (&Sd)[G], int gs) {
      const int ls = local(gs);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int go = wgo(gs, g);
        Sd[g] = load_s(go, ls);
#pragma unroll
        for (int c = 0; c < kStageChunks; ++c) Wd[g][c] = load_w1(go, ls, c);
      }
    };

    // ---- prologue: token stages 0 .. NB-2 into buffers 0 .. NB-2, weights of 0 .. RW-2 ----
    // Every load is unconditional (stage indices clamped; the loads past the end re-read the
    // last stage into buffers nobody reads again), and token loads and weight loads are issued
    // in a fixed order, so the explicit waits below count exactly.
#pragma unroll
    for (int b = 0; b < NB - 1; ++b) load_t(b, local(min(b, NS - 1)));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < RW - 1; ++r) load_w(W[r], S[r], min(r, NS - 1));
    __builtin_amdgcn_sched_barrier(0);
    // stage 0's rows have landed once at most the later loads are outstanding
    wait_vmcnt<(NB - 2) * NFW + 3 * (RW - 1)>();
    lds_barrier();
    read_all(sm.tok, 0);
#pragma unroll
    for (int g = 0; g < G; ++g) Wc[g] = dec_w(W[0][g], S[0][g], 0);

    // One stage st of the stream; R = st % RW gives the weight slot as a compile-time index;
    // the LDS stage buffer is st % NB.  Stage st refills buffer (st - 1) % NB (read by stage
    // st - 1, released by the barrier that ended it) with stage st + NB - 1, and the weight slot
    // freed by stage st - 1 with stage st + RW - 1.  Stages run in groups of RW.
    auto stage = [&](auto RR, int st) {
      constexpr int R = decltype(RR)::value;
      const uint8_t* buf = sm.tok + (st % NB) * SBUF;
      const uint8_t* nbuf = sm.tok + ((st + 1) % NB) * SBUF;
      const int tb = (st + NB - 1) % NB, ts = local(min(st + NB - 1, NS - 1));
      const int wslot = (R + RW - 1) % RW, wgs = min(st + RW - 1, NS - 1);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        h8_t Wn[G];
#pragma unroll
        for (int g = 0; g < G; ++g)
          Wn[g] = (q < 7) ? dec_w(W[R][g], S[R][g], q + 1)
                          : dec_w(W[(R + 1) % RW][g], S[(R + 1) % RW][g], 0);
#pragma unroll
        for (int j = 0; j < NFW; ++j) {
#pragma unroll
          for (int g = 0; g < G; ++g)
            acc[g][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Wc[g], T[j], acc[g][j], 0, 0, 0);
          if (q < 7)
            T[j] = *reinterpret_cast<const h8_t*>(buf + j * 32 * kTokPitch + t_off(q + 1));
          // The stage's vector memory operations go out in a fixed order: its weight loads
          // after the first MFMAs, then the token rows one at a time between the MFMAs of the
          // first half of the stage: a wave stalled issuing a burst of them behind other waves'
          // requests would have no MFMA in flight.  Only VALU and SALU work crosses these
          // points.
          const int m = q * NFW + j;
          if (m == 0) load_w(W[wslot], S[wslot], wgs);
#pragma unroll
          for (int i = 0; i < NFW; ++i)
            if (m == 1 + (i * (kSpreadSteps * NFW - 1)) / NFW) load_t1(tb, ts, i);
          if (m == 0) __builtin_amdgcn_sched_barrier(0);
          else __builtin_amdgcn_sched_barrier(0x006);
        }
#pragma unroll
        for (int g = 0; g < G; ++g) Wc[g] = Wn[g];
      }
      // stage st + 1's rows have landed once at most the loads issued after them are
      // outstanding.  In the steady state they were the last loads of the stage NB - 1 stages
      // ago, followed by NB - 2 full stages (and possibly an epilogue's stores, which only make
      // the wait stricter); while st + 1 <= NB - 2 they came from the prologue, followed by
      // fewer loads (the smallest count is at st = 0).
      if (st + 1 > NB - 2) wait_vmcnt<(NB - 2) * VM_STAGE>();
      else wait_vmcnt<kEarlyWait>();
      lds_barrier();
      read_all(nbuf, 0);
    };
    for (int c = 0; c < cnt; ++c) {
      const int s0 = c * nst;
      int ls = 0;
      for (; ls + RW - 1 < nst; ls += RW)
        unroll_seq([&](auto RR) { stage(RR, s0 + ls + decltype(RR)::value); },
                   std::make_integer_sequence<int, RW>{});
      const int rem = nst - ls;                // only when the stream is a single n-tile
      unroll_seq([&](auto RR) {
        if (decltype(RR)::value < rem) stage(RR, s0 + ls + decltype(RR)::value);
      }, std::make_integer_sequence<int, RW - 1>{});
      if (c == cnt - 1) {
        // The explicit waits count the weight loads of every stage, also in the last stages
        // whose weight registers are never read again; this use keeps the compiler from
        // deleting those loads.
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
          for (int g = 0; g < G; ++g)
            asm volatile("" ::"v"(__builtin_bit_cast(u32x4_t, W[r][g][0])),
                         "v"(__builtin_bit_cast(u32x4_t, W[r][g][1])), "v"(S[r][g]));
        // the clamped token loads of the last stages must land before LDS is reused
        wait_vmcnt<0>();
      }
      // ---- epilogue of unit ub + c ----
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int nt = unit_nt(ub + c) + g;
        if (!group_on(nt)) continue;
#pragma unroll
        for (int j = 0; j < NFW; ++j) {
          const int m = j * 32 + col;
          if (sm.row_src[m] < 0) continue;
          epilogue_group<EPI, true>(a, acc[g][j], al, group_of(nt), h, sm.row_scale[m],
                                    row0 + m);
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < NFW; ++j) acc[g][j] = f32x16_t{};
    }
  }
}

template <int EPI>
__device__ __forceinline__ void run_nfw(const GemmArgs& a, const Smem& sm, int e, int nt,
                                        int nchain, int64_t row0, int nfw) {
  // down-GEMM tiles of at most 4 fragments run two n-tiles at once (measured faster); the
  // gate/up GEMM, with its heavier epilogue, keeps one n-tile per pass (measured slower with two)
  constexpr int GS = EPI == EPI_DOWN ? 2 : 1;
  switch (nfw) {
    case 1: run_tile<1, GS, EPI>(a, sm, e, nt, nchain, row0); break;
    case 2: run_tile<2, GS, EPI>(a, sm, e, nt, nchain, row0); break;
    case 3: run_tile<3, GS, EPI>(a, sm, e, nt, nchain, row0); break;
    case 4: run_tile<4, GS, EPI>(a, sm, e, nt, nchain, row0); break;
    case 5: run_tile<5, 1, EPI>(a, sm, e, nt, nchain, row0); break;
    case 6: run_tile<6, 1, EPI>(a, sm, e, nt, nchain, row0); break;
    case 7: run_tile<7, 1, EPI>(a, sm, e, nt, nchain, row0); break;
    default: run_tile<8, 1, EPI>(a, sm, e, nt, nchain, row0); break;
  }
}

// Prefill-sized plan blocks.  Persistent grid of one 8-wave workgroup per CU with a dynamic
// schedule: a task is (tile, chain of up to `chain` consecutive n-tiles of kTileGroups weight
// row groups), task k = tile k / n_ct of the tile list, n-tiles from (k % n_ct) * chain; a
// workgroup takes its next task from a global counter while it works on the current one.
template <int EPI>
__global__ __launch_bounds__(512, 1) void moe_gemm_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  Smem sm;
  sm.tok = smem;
  sm.row_src = reinterpret_cast<int*>(smem + kTokRegion);
  sm.row_scale = reinterpret_cast<float*>(sm.row_src + kTileRows);
  sm.sh_nvalid = reinterpret_cast<int*>(sm.row_scale + kTileRows);
  sm.sh_task = sm.sh_nvalid + 1;

  const int tid = threadIdx.x;
  const int n_tiles = *a.n_tiles;
  // the down GEMM halves its n-tile chains when the tile list is short (fewer than
  // kMinTasksPerCu tasks per CU at the full chain), so that the dynamic schedule still has
  // tasks to balance; the choice depends on the device-side tile count only, so every
  // workgroup makes the same one
  int chain = a.chain;
  if (EPI == EPI_DOWN && chain > 2 &&
      (int64_t)n_tiles * a.n_nt < (int64_t)kMinTasksPerCu * kCus * chain)
    chain = 2;
  const int n_ct = (a.n_nt + chain - 1) / chain;
  // queue x holds tiles x, x + 8, ... (the tile list is ordered by length, so every queue gets
  // a similar mix); workgroups of XCD x (dispatch places workgroup i on XCD i % 8)
  // take tasks from queue x, so a tile's n-tile tasks share one L2, and move on to the next
  // queues when theirs is empty.  Thread 0 keeps the current queue in q.
  auto q_tasks = [&](int qq) -> int64_t {
    return n_tiles > qq ? (int64_t)((n_tiles - qq + kXcds - 1) / kXcds) * n_ct : 0;
  };
  // resolve a ticket of queue q into a task (tile * n_ct + chain), moving on while queues are
  // exhausted; -1 when every queue is
  auto resolve = [&](int& qq, uint32_t ticket) -> int {
    for (int tries = 0; tries < kXcds; ++tries) {
      if ((int64_t)ticket < q_tasks(qq)) {
        const int tile = qq + kXcds * (int)(ticket / n_ct);
        return tile * n_ct + (int)(ticket % n_ct);
      }
      if (tries == kXcds - 1) break;
      qq = (qq + 1) % kXcds;
      ticket = atomicAdd(a.task_counter + qq, 1u);
    }
    return -1;
  };
  int q = (int)(blockIdx.x % kXcds);
  if (tid == 0) *sm.sh_task = resolve(q, atomicAdd(a.task_counter + q, 1u));
  __syncthreads();
  int64_t k = *sm.sh_task;
  while (k >= 0) {
    uint32_t ticket = 0;
    if (tid == 0) ticket = atomicAdd(a.task_counter + q, 1u);   // in flight during this task
    const int2 t = a.tiles[k / n_ct];
    const int nt = (int)(k % n_ct) * chain;
    const int nchain = EPI == EPI_DOWN ? min(chain, a.n_nt - nt) : 1;
    const int64_t row0 = t.x;
    const int rows_here = min(kTileRows, t.y);
    const int e = a.eids[row0 / a.block_m];
    __syncthreads();                         // the previous task is done with LDS
    if (tid == 0) *sm.sh_nvalid = 0;
    __syncthreads();
    if (tid < kTileRows) {
      int src = -1;
      float sc = 0.0f;
      if (tid < rows_here) {
        const int64_t ent = a.sorted[row0 + tid];
        if (ent >= 0 && ent < a.sentinel) {
          if (a.gather) {
            const int64_t tk = ent / a.top_k;
            src = (int)tk;
            sc = a.a_dec[tk];
          } else {
            src = (int)(row0 + tid);
            sc = a.a_const_scale;
          }
        }
      }
      sm.row_src[tid] = src;
      sm.row_scale[tid] = sc;
      if (src >= 0) atomicMax(sm.sh_nvalid, tid + 1);
    }
    __syncthreads();
    const int nvalid = *sm.sh_nvalid;
    // the tile list holds local experts and tiles with a routed row only
    if (nvalid > 0 && e >= 0 && e < a.nloc)
      run_nfw<EPI>(a, sm, e, nt, nchain, row0, (nvalid + 31) >> 5);
    __syncthreads();                         // every thread has read sh_task
    if (tid == 0) *sm.sh_task = resolve(q, ticket);
    __syncthreads();
    k = *sm.sh_task;
  }
}

// Decode-sized plan blocks (block_m <= 32).  A workgroup task is (plan block, 4 * FN / KS weight
// row groups): the four waves form 4 / KS sets of KS waves, each set owns FN row groups, and the
// KS waves of a set take consecutive parts of the K stages of the same row groups.  The block's
// routed token rows (at most 32) are copied once, still packed (NVFP4 bytes and scale bytes for
// the whole K), into LDS; every wave streams its weights from HBM RING - 1 stages ahead in
// registers and reads its token operand from LDS with no barrier inside the K loop.  The first
// weight stages are requested before the token rows are staged (they depend only on the
// block's expert), so the weight stream's latency overlaps the token gather.  With KS > 1 the
// waves of a set hand their partial FP32 sums to the set's first wave through LDS, which adds
// them in wave order before the epilogue: a few-token GEMM with few row groups then keeps more
// waves streaming, each with a shorter dependent chain of loads.
template <int FN, int KS, int EPI, int RING, int OCC>
__global__ __launch_bounds__(256, OCC) void moe_gemv_kernel(GemmArgs a) {
  static_assert(KS == 1 || KS == 2 || KS == 4, "the four waves split K in 1, 2 or 4 parts");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int* row_src = reinterpret_cast<int*>(smem);
  float* row_scale = reinterpret_cast<float*>(smem + 32 * sizeof(int));
  uint8_t* tok = smem + 64 * sizeof(int);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int kp = wave % KS, set = wave / KS;           // K part and wave set
  // per staged row: K/2 packed bytes then K/16 scale bytes, rounded up to 16 bytes
  const int64_t pitch = (a.a_rowq + (a.a_rowq >> 3) + 15) & ~(int64_t)15;
  const int rows_max = min(a.block_m, 32);
  // partial sums of waves kp > 0: [set][kp - 1][fn][4 float4][64 lanes], after the token rows
  float4* red = reinterpret_cast<float4*>(tok + rows_max * pitch);
  // The first task's expert and plan entries are read together with the plan extent: block
  // blockIdx.x / n_nt is below capacity / block_m for every workgroup of the grid (at most
  // capacity / block_m * n_nt workgroups), so the reads stay inside expert_ids and
  // sorted_token_ids whatever the extent turns out to be.
  const int64_t b_first = blockIdx.x / a.n_nt;
  const int e_first = a.eids[b_first];
  const int ent_first = tid < rows_max ? a.sorted[b_first * a.block_m + tid] : -1;
  int64_t P = *a.ntpp;
  // all three values are taken here, so the compiler issues the three reads together instead
  // of sinking the first two to their uses behind the extent test
  asm volatile("" ::"s"(e_first), "v"(ent_first), "s"((int)P));
  if (P > a.cap) P = a.cap;
  if (P < 0) P = 0;
  const int64_t nblk = P / a.block_m;
  const int64_t ntask = nblk * a.n_nt;
  const int nst = a.nch / kStageChunks;
  // this wave's K stages [s_lo, s_lo + n); s_lo < nst, n may be 0 when nst < KS
  const int s_lo = kp * nst / KS, n = (kp + 1) * nst / KS - s_lo;

  for (int64_t task = blockIdx.x; task < ntask; task += gridDim.x) {
    const bool first = task == blockIdx.x;
    const int64_t b = task / a.n_nt;
    const int nt = (int)(task - b * a.n_nt);
    const int e = first ? e_first : a.eids[b];
    if (e < 0 || e >= a.nloc) continue;

    const int64_t g0 = (int64_t)nt * (4 / KS * FN) + (int64_t)set * FN;
    const bool wave_on = (g0 + FN) * kGroupRows <= a.N;
    const uint8_t* wbase = a.panel + (int64_t)e * a.expert_bytes +
                           (wave_on ? g0 : 0) * a.rg_bytes + lane * 16;
    uint4 W[RING][kStageChunks][FN];
    uint32_t S[RING][FN];
    auto load_w = [&](uint4 (&Wd)[kStageChunks][FN], uint32_t (&Sd)[FN], int st) {
      const int64_t sc = st / (kSuperChunks / kStageChunks);
      const int c0 = (st * kStageChunks) % kSuperChunks;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const uint8_t* base = wbase + fn * a.rg_bytes + sc * kSuperBytes;
        Sd[fn] = *reinterpret_cast<const uint32_t*>(base + 2 * c0);
#pragma unroll
        for (int c = 0; c < kStageChunks; ++c)
          Wd[c][fn] = *reinterpret_cast<const uint4*>(base + kUnit + (c0 + c) * kUnit);
      }
    };
    // the first RING - 1 stages (clamped to the wave's range; a wave with no stages re-reads
    // stage s_lo, which stays in range, and never uses it)
#pragma unroll
    for (int d = 0; d < RING - 1; ++d) load_w(W[d], S[d], s_lo + min(d, max(n - 1, 0)));

    // These barriers order LDS only (row table, token rows, partial sums), so they do not wait
    // for the weight loads in flight.
    lds_barrier();                                     // previous task done with LDS
    // row table: the source row of each of the block's plan rows (-1: padding or masked),
    // then its scale, read while the rows are staged
    int src = -1;
    if (tid < 32) {
      if (tid < rows_max) {
        const int ent = first ? ent_first : a.sorted[b * a.block_m + tid];
        if (ent >= 0 && ent < a.sentinel)
          src = a.gather ? (int)(ent / a.top_k) : (int)(b * a.block_m + tid);
      }
      row_src[tid] = src;
    }
    lds_barrier();
    const float sc_v =
        (tid < 32 && src >= 0) ? (a.gather ? a.a_dec[src] : a.a_const_scale) : 0.0f;
    // stage the routed rows: per row, its packed bytes in 16-byte units (K/2 is a multiple of
    // 64), then its scale bytes in 8-byte units (K/16 is a multiple of 8); the units of all rows
    // are spread over the threads, two loads in flight per thread before their LDS stores
    const int q16 = (int)(a.a_rowq >> 4), per_row = q16 + (int)(a.a_rowq >> 6);
    const int total = rows_max * per_row;
    for (int u0 = tid; u0 < total; u0 += 2 * 256) {
      uint4 v[2];
      int dst[2];                        // LDS byte offset of the unit, -1: nothing to stage
      bool wide[2];                      // a 16-byte unit (packed values), else 8 scale bytes
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int u = u0 + j * 256;
        dst[j] = -1;
        wide[j] = false;
        if (u < total) {
          const int r = u / per_row, i = u - r * per_row;
          const int sr = row_src[r];
          if (sr >= 0 && i < q16) {
            v[j] = *reinterpret_cast<const uint4*>(a.a_q + (int64_t)sr * a.a_rowq + 16 * i);
            dst[j] = r * (int)pitch + 16 * i;
            wide[j] = true;
          } else if (sr >= 0) {
            const uint2 t = *reinterpret_cast<const uint2*>(
                a.a_sf + (int64_t)sr * (a.a_rowq >> 3) + 8 * (i - q16));
            v[j] = make_uint4(t.x, t.y, 0u, 0u);
            dst[j] = r * (int)pitch + (int)a.a_rowq + 8 * (i - q16);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (dst[j] < 0) continue;
        if (wide[j]) *reinterpret_cast<uint4*>(tok + dst[j]) = v[j];
        else *reinterpret_cast<uint2*>(tok + dst[j]) = make_uint2(v[j].x, v[j].y);
      }
    }
    if (tid < 32) row_scale[tid] = sc_v;
    lds_barrier();

    // lanes past the staged rows read row 0; their MFMA columns are discarded
    const uint8_t* trow = tok + (col < rows_max ? col : 0) * pitch;
    const float al = lane_alpha<EPI>(a, e, h);
    f32x16_t acc[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) acc[fn] = f32x16_t{};

    auto compute = [&](const uint4 (&Wd)[kStageChunks][FN], const uint32_t (&Sd)[FN], int st) {
      const uint2 tsc = *reinterpret_cast<const uint2*>(trow + a.a_rowq + st * 8);
#pragma unroll
      for (int c = 0; c < kStageChunks; ++c) {
        const uint4 td4 = *reinterpret_cast<const uint4*>(trow + st * 64 + c * 32 + 16 * h);
        const uint32_t tsw = (c == 0) ? tsc.x : tsc.y;      // scale bytes of blocks 4c..4c+3
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint32_t td = (s == 0) ? td4.x : (s == 1) ? td4.y : (s == 2) ? td4.z : td4.w;
          const uint32_t tsb = (tsw >> (8 * (2 * h + (s >> 1)))) & 0xFFu;
          const h8_t Tv = decode8(td, e4m3_scale_h2(tsb));
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
            const uint32_t wd = (s == 0) ? Wd[c][fn].x : (s == 1) ? Wd[c][fn].y
                                : (s == 2) ? Wd[c][fn].z : Wd[c][fn].w;
            const uint32_t sb = (Sd[fn] >> (8 * (2 * c + (s >> 1)))) & 0xFFu;
            const h8_t Wv = decode8(wd, e4m3_scale_h2(sb));
            acc[fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Wv, Tv, acc[fn], 0, 0, 0);
          }
        }
      }
    };

    // weight loads are unconditional (stage index clamped to the wave's last stage) so the
    // compiler's waits count them exactly; the tail of the last ring pass leaves through the
    // break
    for (int st0 = 0; st0 < n; st0 += RING) {
#pragma unroll
      for (int d = 0; d < RING; ++d) {
        const int st = st0 + d;
        if (st >= n) break;
        const int nd = (d + RING - 1) % RING;
        load_w(W[nd], S[nd], s_lo + min(st + RING - 1, n - 1));
        compute(W[d], S[d], s_lo + st);
      }
    }
    if (KS > 1) {
      // waves kp > 0 hand their partial sums to wave kp = 0 of their set
      float4* mine = red + ((set * (KS - 1) + (kp > 0 ? kp - 1 : 0)) * FN) * 4 * 64 + lane;
      if (kp > 0) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            mine[(fn * 4 + i) * 64] = make_float4(acc[fn][4 * i], acc[fn][4 * i + 1],
                                                  acc[fn][4 * i + 2], acc[fn][4 * i + 3]);
      }
      lds_barrier();
      if (kp == 0) {
#pragma unroll
        for (int q = 1; q < KS; ++q) {
          const float4* part = red + ((set * (KS - 1) + q - 1) * FN) * 4 * 64 + lane;
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float4 v = part[(fn * 4 + i) * 64];
              acc[fn][4 * i] += v.x;
              acc[fn][4 * i + 1] += v.y;
              acc[fn][4 * i + 2] += v.z;
              acc[fn][4 * i + 3] += v.w;
            }
        }
      }
    }
    if (kp == 0 && wave_on && col < rows_max && row_src[col] >= 0) {
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        epilogue_group<EPI>(a, acc[fn], al, g0 + fn, h, row_scale[col], b * a.block_m + col);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// NVFP4 weight-only mode on BF16 activations, decode-sized plan blocks (block_m <= 32).
// Same tasks and weight stream as moe_gemv_kernel; the token operand is BF16 as given, read by
// each lane straight from memory (the block's few rows stay in L2), so nothing is staged in LDS
// but the row sources; each weight fragment is decoded exactly (E2M1 x E4M3 has at most 6
// significant bits) to BF16 and fed to v_mfma_f32_32x32x16_bf16.

typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));

typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));

// 8 E2M1 codes times one E4M3 scale -> 8 exact BF16 values: the codes convert to FP32 times
// 256 (only the exponent of the conversion's scale operand is used) and the scale enters as the
// FP32 value s * 2^-8 (read through its FP16 bit pattern, exact for every E4M3 code); every
// product has at most 6 significant bits, so the FP32 products and their BF16 conversion are
// exact.
__device__ __forceinline__ bf8_t decode8_bf16(uint32_t w, uint32_t sf_byte) {
  const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)((sf_byte & 0x7Fu) << 7));
  u32x4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float2 p;
    switch (i) {   // the byte selector must be a compile-time constant
      case 0: {
        const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 256.0f, 0);
        p = make_float2(v[0], v[1]);
        break;
      }
      case 1: {
        const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 256.0f, 1);
        p = make_float2(v[0], v[1]);
        break;
      }
      case 2: {
        const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 256.0f, 2);
        p = make_float2(v[0], v[1]);
        break;
      }
      default: {
        const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 256.0f, 3);
        p = make_float2(v[0], v[1]);
        break;
      }
    }
    const bf2_t b2 = {(__bf16)(p.x * s), (__bf16)(p.y * s)};
    r[i] = __builtin_bit_cast(uint32_t, b2);
  }
  return __builtin_bit_cast(bf8_t, r);
}

// 8 E2M1 codes times one E8M0 scale (MXFP4) -> 8 BF16 values in four conversions: the scale's
// code is the exponent field of an FP32 with the same bias (127), and the conversion applies only
// the exponent of its scale operand.  Exact while the products stay in BF16's normal range
// (scale codes 2..252).
__device__ __forceinline__ bf8_t decode8_mx(uint32_t w, uint32_t e8m0) {
  const float sc = __uint_as_float(e8m0 << 23);
  u32x4_t r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
  return __builtin_bit_cast(bf8_t, r);
}

// GEMM1 epilogue of the weight-only mode: pre = acc * alpha (FP32, reported to dbg_pre), rounded
// to BF16; the activation of the rounded values, rounded to BF16, is the intermediate h [cap, I]
// (GEMM2's BF16 token operand).  Gated forms exchange halves between lanes l and l + 32 as the
// NVFP4 epilogue does; one-projection forms keep 16 consecutive values per lane.
template <int EPI>
__device__ __forceinline__ void epilogue_w16(const GemmArgs& a, const f32x16_t& acc, float al,
                                             int64_t g, int h, int64_t r) {
  if (one_projection(EPI)) {
    const int64_t i0 = g * kGroupRows + 16 * h;
    float pr[16];
    uint32_t bb[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      pr[v] = acc[v] * al;
      const float pb = bf16_to_f32(f32_to_bf16(pr[v]));
      float hv;
      if (EPI == EPI_RELU2) {
        const float q = pb > 0.0f ? pb : 0.0f;
        hv = q * q;
      } else {
        hv = act_one(pb, a.act);
      }
      bb[v] = f32_to_bf16(hv);
    }
    if (a.dbg_pre) {
      float4* dp = reinterpret_cast<float4*>(a.dbg_pre + r * a.I + i0);
#pragma unroll
      for (int v = 0; v < 4; ++v)
        dp[v] = make_float4(pr[4 * v], pr[4 * v + 1], pr[4 * v + 2], pr[4 * v + 3]);
    }
    const uint4 w0 = make_uint4(bb[0] | (bb[1] << 16), bb[2] | (bb[3] << 16),
                                bb[4] | (bb[5] << 16), bb[6] | (bb[7] << 16));
    const uint4 w1 = make_uint4(bb[8] | (bb[9] << 16), bb[10] | (bb[11] << 16),
                                bb[12] | (bb[13] << 16), bb[14] | (bb[15] << 16));
    uint4* d = reinterpret_cast<uint4*>(a.w16_h + r * a.I + i0);
    d[0] = w0;
    d[1] = w1;
    if (a.dbg_inter) {
      uint4* dd = reinterpret_cast<uint4*>(a.dbg_inter + r * a.I + i0);
      dd[0] = w0;
      dd[1] = w1;
    }
    return;
  }
  // SwiGLU, GeGLU
  const int64_t i0 = g * 16;
  float pre[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) pre[v] = acc[v] * al;
  if (a.dbg_pre) {
    float4* dp = reinterpret_cast<float4*>(a.dbg_pre + r * (2 * a.I) + h * a.I + i0);
#pragma unroll
    for (int v = 0; v < 4; ++v)
      dp[v] = make_float4(pre[4 * v], pre[4 * v + 1], pre[4 * v + 2], pre[4 * v + 3]);
  }
  uint32_t bb[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const auto gu = __builtin_amdgcn_permlane32_swap(__float_as_uint(pre[v]),
                                                     __float_as_uint(pre[8 + v]), false, false);
    const float gt = bf16_to_f32(f32_to_bf16(__uint_as_float(gu[0])));
    const float up = bf16_to_f32(f32_to_bf16(__uint_as_float(gu[1])));
    bb[v] = f32_to_bf16((EPI == EPI_GEGLU ? gelu(gt) : silu(gt)) * up);
  }
  const int64_t ih = i0 + 8 * h;
  const uint4 w = make_uint4(bb[0] | (bb[1] << 16), bb[2] | (bb[3] << 16), bb[4] | (bb[5] << 16),
                             bb[6] | (bb[7] << 16));
  *reinterpret_cast<uint4*>(a.w16_h + r * a.I + ih) = w;
  if (a.dbg_inter) *reinterpret_cast<uint4*>(a.dbg_inter + r * a.I + ih) = w;
}

// MX: the weight panels carry MXFP4 (E8M0 scale codes, duplicated into the 16-value slots)
template <int FN, int EPI, int RING, bool MX>
__global__ __launch_bounds__(256, 4) void moe_gemv16_kernel(GemmArgs a) {
  __shared__ int row_src[32];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, col = lane & 31;
  int64_t P = *a.ntpp;
  if (P > a.cap) P = a.cap;
  if (P < 0) P = 0;
  const int64_t nblk = P / a.block_m;
  const int nst = a.nch / kStageChunks;
  const int rows_max = min(a.block_m, 32);
  const int64_t ntask = nblk * a.n_nt;

  for (int64_t task = blockIdx.x; task < ntask; task += gridDim.x) {
    const int64_t b = task / a.n_nt;
    const int nt = (int)(task - b * a.n_nt);
    const int e = a.eids[b];
    if (e < 0 || e >= a.nloc) continue;
    __syncthreads();                                   // previous task done with row_src
    if (tid < 32) {
      int src = -1;
      if (tid < rows_max) {
        const int64_t ent = a.sorted[b * a.block_m + tid];
        if (ent >= 0 && ent < a.sentinel) src = a.gather ? (int)(ent / a.top_k)
                                                         : (int)(b * a.block_m + tid);
      }
      row_src[tid] = src;
    }
    __syncthreads();

    const int64_t g0 = (int64_t)nt * (4 * FN) + (int64_t)wave * FN;
    const bool wave_on = (g0 + FN) * kGroupRows <= a.N;
    const uint8_t* wbase = a.panel + (int64_t)e * a.expert_bytes + (wave_on ? g0 : 0) * a.rg_bytes +
                           lane * 16;
    // only lanes of routed rows read token data; the others feed zeros (their columns are
    // dropped), which keeps the L2 traffic to the block's routed rows
    const int my_src = col < rows_max ? row_src[col] : -1;
    const bool tok_on = my_src >= 0;
    const uint16_t* trow = a.w16_x + (int64_t)(tok_on ? my_src : 0) * a.w16_stride + 32 * h;

    const float al = lane_alpha<EPI>(a, e, h);
    f32x16_t acc[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) acc[fn] = f32x16_t{};
    uint4 W[RING][kStageChunks][FN];
    uint32_t S[RING][FN];

    auto load_w = [&](uint4 (&Wd)[kStageChunks][FN], uint32_t (&Sd)[FN], int st) {
      const int64_t sc = st / (kSuperChunks / kStageChunks);
      const int c0 = (st * kStageChunks) % kSuperChunks;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const uint8_t* base = wbase + fn * a.rg_bytes + sc * kSuperBytes;
        Sd[fn] = *reinterpret_cast<const uint32_t*>(base + 2 * c0);
#pragma unroll
        for (int c = 0; c < kStageChunks; ++c)
          Wd[c][fn] = *reinterpret_cast<const uint4*>(base + kUnit + (c0 + c) * kUnit);
      }
    };
    // token operand of one 64-value chunk: lane (col, h) holds values 32h .. 32h + 31 of the
    // chunk, 8 per MFMA step (the K order the weight panels use)
    auto load_t = [&](uint4 (&T)[4], int64_t chunk) {
      const uint4* p = reinterpret_cast<const uint4*>(trow + chunk * 64);
#pragma unroll
      for (int s = 0; s < 4; ++s) T[s] = tok_on ? p[s] : make_uint4(0, 0, 0, 0);
    };
    auto compute = [&](const uint4 (&Wd)[kStageChunks][FN], const uint32_t (&Sd)[FN],
                       const uint4 (&T)[kStageChunks][4]) {
#pragma unroll
      for (int c = 0; c < kStageChunks; ++c) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf8_t Tv = __builtin_bit_cast(bf8_t, T[c][s]);
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
            const uint32_t wd = (s == 0) ? Wd[c][fn].x : (s == 1) ? Wd[c][fn].y
                                : (s == 2) ? Wd[c][fn].z : Wd[c][fn].w;
            const uint32_t sb = (Sd[fn] >> (8 * (2 * c + (s >> 1)))) & 0xFFu;
            const bf8_t Wv = MX ? decode8_mx(wd, sb) : decode8_bf16(wd, sb);
            acc[fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Wv, Tv, acc[fn], 0, 0, 0);
          }
        }
      }
    };

    uint4 T[kStageChunks][4];
#pragma unroll
    for (int d = 0; d < RING - 1; ++d) load_w(W[d], S[d], min(d, nst - 1));
    for (int st0 = 0; st0 < nst; st0 += RING) {
#pragma unroll
      for (int d = 0; d < RING; ++d) {
        const int st = st0 + d;
        if (st >= nst) break;
#pragma unroll
        for (int c = 0; c < kStageChunks; ++c) load_t(T[c], (int64_t)st * kStageChunks + c);
        const int nd = (d + RING - 1) % RING;
        load_w(W[nd], S[nd], min(st + RING - 1, nst - 1));
        compute(W[d], S[d], T);
      }
    }
    if (wave_on && tok_on) {
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        if (EPI == EPI_DOWN)
          epilogue_group<EPI_DOWN>(a, acc[fn], al, g0 + fn, h, 1.0f, b * a.block_m + col);
        else
          epilogue_w16<EPI>(a, acc[fn], al, g0 + fn, h, b * a.block_m + col);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// MXFP4 weights on MXFP8 activations, decode-sized plan blocks (block_m <= 32), on gfx950's
// block-scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4: A = 32 weight rows x 64 K as FP4, B = 64 K
// x 32 tokens as FP8, E8M0 scales per row or column and 32-value K block, the scale of K block kb
// given by lane col + 32 kb).  Operand lane layouts, as measured on gfx950 with an in-bounds
// probe of the instruction: an FP4 operand lane (col, h) holds K values 32 h .. 32 h + 31 of
// the 64 (low nibble first); an FP8 operand lane holds K values 16 h .. 16 h + 15 and
// 32 + 16 h .. 32 + 16 h + 15.  The MXFP4 panels already hold, per 64-value chunk, each lane's
// 16 bytes (row l % 32, K half l / 32: one MX block) and its E8M0 code, so weights go from the
// load straight into the MFMA with no decode; each lane reads its token's two 16-byte FP8 pieces
// of the chunk and the E8M0 code of K block h from memory one stage ahead (the block's few rows
// stay in L2).  Same tasks and weight stream as moe_gemv16_kernel.  The instruction's internal
// sum of a chunk's 64 products is not exact to FP32 (measured: within 2^-13.4 of the sum of the
// products' magnitudes); the running sum over chunks is FP32.
//   GEMM1  pre = sum_h a w1 (no FP32 scales: MX weights and activations carry only E8M0 block
//          scales) -> activation -> BF16 -> MXFP8 of each 32-value block of the intermediate
//   GEMM2  y = bf16(sum_i hq w2)

typedef int i32x8_t __attribute__((ext_vector_type(8)));

// GEMM1 epilogue of the MX mode for the wave's two row groups g0 (even) and g0 + 1, token row r:
// pre -> activation -> BF16 -> MXFP8 with one E8M0 scale per 32 intermediate values.  Gated: the
// groups hold the gate and up rows of intermediate values 16 g0 .. 16 g0 + 31, one MX block;
// after the lane-pair swap lane (col, h) holds 16 g + 8 h + 0..7 of each group.  One projection:
// group g holds the MX block 32 g .. 32 g + 31, lane h its values 16 h .. 16 h + 15.  The block
// maximum is taken over the lane pair (l, l ^ 32).
template <int EPI>
__device__ __forceinline__ void epilogue_mx(const GemmArgs& a, const f32x16_t& acc0,
                                            const f32x16_t& acc1, int64_t g0, int h, int64_t r) {
  const f32x16_t* acc[2] = {&acc0, &acc1};
  uint8_t* hq = a.hq + r * a.I;                     // MXFP8 intermediate: I bytes per row
  uint8_t* hsf = a.hsf + r * (a.I >> 5);
  if (one_projection(EPI)) {
#pragma unroll
    for (int fn = 0; fn < 2; ++fn) {
      const int64_t i0 = (g0 + fn) * kGroupRows + 16 * h;
      float pr[16], hv[16];
      uint32_t bb[16];
      float m = 0.0f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        pr[v] = (*acc[fn])[v];
        float q;
        if (EPI == EPI_RELU2) {
          const float t = pr[v] > 0.0f ? pr[v] : 0.0f;
          q = t * t;
        } else {
          q = act_one(pr[v], a.act);
        }
        bb[v] = f32_to_bf16(q);
        hv[v] = bf16_to_f32(bb[v]);
        m = __builtin_fmaxf(m, __builtin_fabsf(hv[v]));
      }
      if (a.dbg_pre) {
        float4* dp = reinterpret_cast<float4*>(a.dbg_pre + r * a.I + i0);
#pragma unroll
        for (int v = 0; v < 4; ++v)
          dp[v] = make_float4(pr[4 * v], pr[4 * v + 1], pr[4 * v + 2], pr[4 * v + 3]);
      }
      if (a.dbg_inter) {
        uint4* d = reinterpret_cast<uint4*>(a.dbg_inter + r * a.I + i0);
        d[0] = make_uint4(bb[0] | (bb[1] << 16), bb[2] | (bb[3] << 16), bb[4] | (bb[5] << 16),
                          bb[6] | (bb[7] << 16));
        d[1] = make_uint4(bb[8] | (bb[9] << 16), bb[10] | (bb[11] << 16),
                          bb[12] | (bb[13] << 16), bb[14] | (bb[15] << 16));
      }
      const auto mm = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m),
                                                       false, false);
      m = __builtin_fmaxf(__uint_as_float(mm[0]), __uint_as_float(mm[1]));
      uint32_t code;
      const float inv = mx_scale_inverse(m, kE4M3Emax, code);
      *reinterpret_cast<uint4*>(hq + i0) =
          make_uint4(e4m3_pack4(hv, inv), e4m3_pack4(hv + 4, inv), e4m3_pack4(hv + 8, inv),
                     e4m3_pack4(hv + 12, inv));
      if (h == 0) hsf[(g0 + fn)] = (uint8_t)code;
    }
    return;
  }
  // SwiGLU, GeGLU
  float hv[2][8];
  uint32_t bb[2][8];
  float m = 0.0f;
#pragma unroll
  for (int fn = 0; fn < 2; ++fn) {
    const int64_t i0 = (g0 + fn) * 16;
    if (a.dbg_pre) {
      float4* dp = reinterpret_cast<float4*>(a.dbg_pre + r * (2 * a.I) + h * a.I + i0);
#pragma unroll
      for (int v = 0; v < 4; ++v)
        dp[v] = make_float4((*acc[fn])[4 * v], (*acc[fn])[4 * v + 1], (*acc[fn])[4 * v + 2],
                            (*acc[fn])[4 * v + 3]);
    }
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const auto gu = __builtin_amdgcn_permlane32_swap(__float_as_uint((*acc[fn])[v]),
                                                       __float_as_uint((*acc[fn])[8 + v]), false,
                                                       false);
      const float gt = __uint_as_float(gu[0]);
      const float up = __uint_as_float(gu[1]);
      bb[fn][v] = f32_to_bf16((EPI == EPI_GEGLU ? gelu(gt) : silu(gt)) * up);
      hv[fn][v] = bf16_to_f32(bb[fn][v]);
      m = __builtin_fmaxf(m, __builtin_fabsf(hv[fn][v]));
    }
    if (a.dbg_inter) {
      *reinterpret_cast<uint4*>(a.dbg_inter + r * a.I + i0 + 8 * h) =
          make_uint4(bb[fn][0] | (bb[fn][1] << 16), bb[fn][2] | (bb[fn][3] << 16),
                     bb[fn][4] | (bb[fn][5] << 16), bb[fn][6] | (bb[fn][7] << 16));
    }
  }
  const auto mm = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m),
                                                   false, false);
  m = __builtin_fmaxf(__uint_as_float(mm[0]), __uint_as_float(mm[1]));
  uint32_t code;
  const float inv = mx_scale_inverse(m, kE4M3Emax, code);
#pragma unroll
  for (int fn = 0; fn < 2; ++fn)
    *reinterpret_cast<uint2*>(hq + (g0 + fn) * 16 + 8 * h) =
        make_uint2(e4m3_pack4(hv[fn], inv), e4m3_pack4(hv[fn] + 4, inv));
  if (h == 0) hsf[g0 >> 1] = (uint8_t)code;
}

template <int EPI, int RING>
__global__ __launch_bounds__(256, 4) void moe_gemv_mx_kernel(GemmArgs a) {
  constexpr int FN = 2;                       // the gated MX block spans two row groups
  __shared__ int row_src[32];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, col = lane & 31;
  int64_t P = *a.ntpp;
  if (P > a.cap) P = a.cap;
  if (P < 0) P = 0;
  const int64_t nblk = P / a.block_m;
  const int nst = a.nch / kStageChunks;
  const int rows_max = min(a.block_m, 32);
  const int64_t ntask = nblk * a.n_nt;
  const int64_t K = a.a_rowq;                 // FP8 token row: K bytes, then K / 32 scale codes

  for (int64_t task = blockIdx.x; task < ntask; task += gridDim.x) {
    const int64_t b = task / a.n_nt;
    const int nt = (int)(task - b * a.n_nt);
    const int e = a.eids[b];
    if (e < 0 || e >= a.nloc) continue;
    __syncthreads();                                   // previous task done with row_src
    if (tid < 32) {
      int src = -1;
      if (tid < rows_max) {
        const int64_t ent = a.sorted[b * a.block_m + tid];
        if (ent >= 0 && ent < a.sentinel) src = a.gather ? (int)(ent / a.top_k)
                                                         : (int)(b * a.block_m + tid);
      }
      row_src[tid] = src;
    }
    __syncthreads();

    const int64_t g0 = (int64_t)nt * (4 * FN) + (int64_t)wave * FN;
    const bool wave_on = (g0 + FN) * kGroupRows <= a.N;
    const uint8_t* wbase = a.panel + (int64_t)e * a.expert_bytes + (wave_on ? g0 : 0) * a.rg_bytes +
                           lane * 16;
    // only lanes of routed rows read token data; the others feed zeros (their columns are
    // dropped)
    const int my_src = col < rows_max ? row_src[col] : -1;
    const bool tok_on = my_src >= 0;
    const uint8_t* trow = a.a_q + (int64_t)(tok_on ? my_src : 0) * K + 16 * h;
    const uint8_t* tsf = a.a_sf + (int64_t)(tok_on ? my_src : 0) * (K >> 5);

    f32x16_t acc[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) acc[fn] = f32x16_t{};
    uint4 W[RING][kStageChunks][FN];
    uint32_t S[RING][FN];

    auto load_w = [&](uint4 (&Wd)[kStageChunks][FN], uint32_t (&Sd)[FN], int st) {
      const int64_t sc = st / (kSuperChunks / kStageChunks);
      const int c0 = (st * kStageChunks) % kSuperChunks;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const uint8_t* base = wbase + fn * a.rg_bytes + sc * kSuperBytes;
        Sd[fn] = *reinterpret_cast<const uint32_t*>(base + 2 * c0);
#pragma unroll
        for (int c = 0; c < kStageChunks; ++c)
          Wd[c][fn] = *reinterpret_cast<const uint4*>(base + kUnit + (c0 + c) * kUnit);
      }
    };
    // token operand of one stage: per chunk the FP8 bytes 16 h .. 16 h + 15 and 32 + 16 h ..
    // 32 + 16 h + 15 (the FP8 operand's lane layout), and the stage's four E8M0 codes (chunk c,
    // K block h: byte 2 c + h)
    auto load_t = [&](uint4 (&T)[kStageChunks][2], uint32_t& TS, int st) {
#pragma unroll
      for (int c = 0; c < kStageChunks; ++c) {
        const uint4* p =
            reinterpret_cast<const uint4*>(trow + (int64_t)(st * kStageChunks + c) * 64);
        T[c][0] = tok_on ? p[0] : make_uint4(0, 0, 0, 0);
        T[c][1] = tok_on ? p[2] : make_uint4(0, 0, 0, 0);
      }
      TS = tok_on ? *reinterpret_cast<const uint32_t*>(tsf + st * 4) : 0u;
    };
    auto compute = [&](const uint4 (&Wd)[kStageChunks][FN], const uint32_t (&Sd)[FN],
                       const uint4 (&T)[kStageChunks][2], uint32_t TS) {
#pragma unroll
      for (int c = 0; c < kStageChunks; ++c) {
        const i32x8_t B = {(int)T[c][0].x, (int)T[c][0].y, (int)T[c][0].z, (int)T[c][0].w,
                           (int)T[c][1].x, (int)T[c][1].y, (int)T[c][1].z, (int)T[c][1].w};
        const int sb = (int)((TS >> (8 * (2 * c + h))) & 0xFFu);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const i32x8_t A = {(int)Wd[c][fn].x, (int)Wd[c][fn].y, (int)Wd[c][fn].z,
                             (int)Wd[c][fn].w, 0, 0, 0, 0};
          const int sa = (int)((Sd[fn] >> (16 * c)) & 0xFFu);   // chunk c0 + c of the stage
          acc[fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc[fn], 4, 0, 0, sa, 0,
                                                                    sb);
        }
      }
    };

    uint4 T[RING][kStageChunks][2];
    uint32_t TS[RING];
#pragma unroll
    for (int d = 0; d < RING - 1; ++d) {
      load_w(W[d], S[d], min(d, nst - 1));
      load_t(T[d], TS[d], min(d, nst - 1));
    }
    for (int st0 = 0; st0 < nst; st0 += RING) {
#pragma unroll
      for (int d = 0; d < RING; ++d) {
        const int st = st0 + d;
        if (st >= nst) break;
        const int nd = (d + RING - 1) % RING;
        load_w(W[nd], S[nd], min(st + RING - 1, nst - 1));
        load_t(T[nd], TS[nd], min(st + RING - 1, nst - 1));
        compute(W[d], S[d], T[d], TS[d]);
      }
    }
    if (wave_on && tok_on) {
      const int64_t r = b * a.block_m + col;
      if (EPI == EPI_DOWN) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          epilogue_group<EPI_DOWN>(a, acc[fn], 1.0f, g0 + fn, h, 1.0f, r);
      } else {
        epilogue_mx<EPI>(a, acc[0], acc[1], g0, h, r);
      }
    }
  }
}

template <int EPI>
hipError_t launch_gemv_mx(const GemmArgs& a, int64_t cap_blocks, const char* name,
                          hipStream_t s) {
  const int64_t tasks = cap_blocks * a.n_nt;
  const int64_t max_wg = 256LL * 4;                  // resident workgroups (4 waves each)
  const int64_t grid = tasks < max_wg ? tasks : max_wg;
  if (grid == 0) return hipSuccess;
  KernelTimer t(name, s);
  hipLaunchKernelGGL((moe_gemv_mx_kernel<EPI, 2>), dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int FN, int EPI, bool MX>
hipError_t launch_gemv16(const GemmArgs& a, int64_t cap_blocks, const char* name,
                         hipStream_t s) {
  const int64_t tasks = cap_blocks * a.n_nt;
  const int64_t max_wg = 256LL * 4;                  // resident workgroups (4 waves each)
  const int64_t grid = tasks < max_wg ? tasks : max_wg;
  if (grid == 0) return hipSuccess;
  KernelTimer t(name, s);
  hipLaunchKernelGGL((moe_gemv16_kernel<FN, EPI, 2, MX>), dim3((unsigned)grid), dim3(256), 0, s,
                     a);
  return hipGetLastError();
}

constexpr int kMaxDevices = 64;

// Raises fn's dynamic LDS limit to at least `lds` bytes on the current device, once per device
// (done[dev] holds the largest limit set so far); several threads may race here harmlessly, since
// setting the same attribute twice is idempotent.
hipError_t ensure_dynamic_lds(const void* fn, size_t lds, std::atomic<size_t>* done) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  std::atomic<size_t>* slot = (dev >= 0 && dev < kMaxDevices) ? &done[dev] : nullptr;
  if (slot && slot->load(std::memory_order_acquire) >= lds) return hipSuccess;
  err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  if (slot) {
    size_t cur = slot->load(std::memory_order_acquire);
    while (cur < lds && !slot->compare_exchange_weak(cur, lds, std::memory_order_acq_rel)) {
    }
  }
  return hipSuccess;
}

// LDS of a decode task: the row table and staged token rows, then the partial sums that the
// waves with K part > 0 hand over (FN accumulators of 64 lanes x 16 floats each).
size_t gemv_lds_bytes(int block_m, int64_t K, int fn, int ks) {
  return moe_gemv_lds_bytes(block_m, K) + (size_t)(4 - 4 / ks) * fn * 64 * 16 * sizeof(float);
}

template <int FN, int KS, int RING, int OCC, int EPI>
hipError_t launch_gemv(const GemmArgs& a, int64_t cap_blocks, const char* name, hipStream_t s) {
  auto kern = moe_gemv_kernel<FN, KS, EPI, RING, OCC>;
  const size_t lds = gemv_lds_bytes(a.block_m, 2 * a.a_rowq, FN, KS);
  if (lds > kMaxLdsBytes) return hipErrorInvalidValue;
  static std::atomic<size_t> lds_set[kMaxDevices];
  hipError_t err = ensure_dynamic_lds(reinterpret_cast<const void*>(kern), lds, lds_set);
  if (err != hipSuccess) return err;
  const int64_t tasks = cap_blocks * a.n_nt;
  const int64_t max_wg = 256LL * OCC;                // resident workgroups (4 waves each)
  const int64_t grid = tasks < max_wg ? tasks : max_wg;
  if (grid == 0) return hipSuccess;
  KernelTimer t(name, s);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), lds, s, a);
  return hipGetLastError();
}

// Task shape of a decode GEMM with N weight rows and K values per row, for at most `blocks`
// plan blocks: FN row groups per wave and K split over KS waves.  With at least two tasks of 8
// row groups per CU (the 7168- and 4096-row matrices of an 8-token step) the weight stream is
// HBM-bound: two row groups per wave and the whole K, which amortizes the task set-up over the
// longest chains.  Below that (few tokens on small matrices) the GEMM is latency-bound: one
// row group per wave, and K split over the most waves (4 or 2) that keep the row-group streams
// times KS within twice the 4096 resident waves and give each wave at least two 128-K stages
// (measured on the 4-token, 2048 x 512 shape: 20 against 23 us for the gate/up GEMM, 13 against
// 14 us for the down GEMM).
struct GemvShape {
  int fn, ks;
};
GemvShape gemv_shape(int64_t blocks, int64_t N, int64_t K, int block_m) {
  const int64_t groups = (N + kGroupRows - 1) / kGroupRows;
  if (blocks * ((N + 255) / 256) >= 2 * kCus) return {2, 1};
  const int64_t streams = blocks * groups, nst = K / (kChunkK * kStageChunks);
  const size_t lds_cap = kMaxLdsBytes / 4;          // four workgroups per CU
  for (int ks = 4; ks > 1; ks /= 2)
    if (streams * ks <= 2 * 4LL * kCus * 4 && nst >= 2 * ks &&
        gemv_lds_bytes(block_m, K, 1, ks) <= lds_cap)
      return {1, ks};
  return {1, 1};
}

template <int EPI>
hipError_t launch_gemv_shape(const GemvShape& sh, const GemmArgs& a, int64_t cap_blocks,
                             const char* name, hipStream_t s) {
  if (sh.fn == 2) return launch_gemv<2, 1, 2, 4, EPI>(a, cap_blocks, name, s);
  if (sh.ks == 4) return launch_gemv<1, 4, 3, 4, EPI>(a, cap_blocks, name, s);
  if (sh.ks == 2) return launch_gemv<1, 2, 3, 4, EPI>(a, cap_blocks, name, s);
  return launch_gemv<1, 1, 2, 4, EPI>(a, cap_blocks, name, s);
}

// ---------------------------------------------------------------------------------------------
// MXFP4 weights on MXFP8 activations, prefill-sized plan blocks (block_m > 32), on the block-
// scaled MFMA.  Persistent grid of one 8-wave workgroup per CU (two waves per SIMD) taking tasks
// (tile of up to 256 plan rows of one expert, n-tile of 256 weight rows) from the per-XCD ticket
// queues of the prefill tile list.  Waves w and w + 4 own the two row groups 8 nt + 2 w and
// 8 nt + 2 w + 1 (so a gated MX block of 32 intermediate values stays inside one wave); wave w
// takes the first ceil(NFW / 2) token fragments of the tile, wave w + 4 the others, so a wave
// holds at most 8 accumulators of 16 values and each token fragment read from LDS feeds two
// MFMAs.  Per 128-K stage, the tile's FP8 token rows (128 bytes each) with their four E8M0
// codes, and the n-tile's MXFP4 weight chunks with their scale words, are copied into one
// stage buffer of an LDS ring by direct buffer-to-LDS loads shared out over the 8 waves; the ring
// holds NB stages, so both operands are requested NB - 1 stages ahead without holding registers.
// Inside a token row the 16-byte slot u sits at u ^ (row & 7), so the operand reads are free of
// bank conflicts; weight chunks keep the panel's lane order (lane l's 16 bytes at 16 l).
constexpr int kMxStageBytes = 128;        // FP8 token bytes per row per stage (128 K values)
constexpr int kMxTileRows = 256;
constexpr int kMxRingBytes = 158 * 1024;  // stage buffers: tokens, token scales, weights, scales
constexpr int kMxWBytes = kTileGroups * kStageChunks * kUnit;       // weight chunks per stage
constexpr int kMxWsBytes = kTileGroups * 256;                       // weight scale words per stage

template <int NFW> struct MxDepth {
  static constexpr int TDATA = NFW * 32 * kMxStageBytes;             // token rows
  static constexpr int TSC = TDATA;                                  // token scale dwords
  static constexpr int WOFF = TSC + kMxTileRows * 4;                 // weight chunks
  static constexpr int WSC = WOFF + kMxWBytes;                       // weight scale words
  static constexpr int SBUF = WSC + kMxWsBytes;
  static constexpr int NB0 = kMxRingBytes / SBUF;
  static constexpr int NB = NB0 > 6 ? 6 : NB0;
  static constexpr int NF0 = (NFW + 1) / 2;          // fragments of waves 0-3; the rest 4-7
};

template <int NFW, int NJ, int EPI>
__device__ __forceinline__ void run_tile_mx(const GemmArgs& a, uint8_t* ring, const int* row_src,
                                            int e, int nt, int64_t row0) {
  using D = MxDepth<NFW>;
  constexpr int NB = D::NB, SBUF = D::SBUF;
  constexpr int NF0 = D::NF0;
  constexpr int NA = NJ > 0 ? NJ : 1;                    // accumulator fragments declared
  static_assert(NB >= 3, "at least three stage buffers");
  // vector memory operations a wave issues per stage: one weight group (scale word and two
  // chunks), NP token data pieces and one token scale piece
  constexpr int NP = (4 * NFW + 7) / 8;
  constexpr int VM_STAGE = 3 + NP + 1;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wg = wave & 3, half = wave >> 2;
  const int h = lane >> 5, col = lane & 31;
  const int nst = a.nch / kStageChunks;
  const int64_t K = a.a_rowq;                            // FP8 bytes per token row

  // weights: wave w + 4 h copies row group 8 nt + 2 w + h of the n-tile (local group 2 w + h)
  // through a buffer resource over the expert; a wave pair past the last row group of the
  // matrix copies groups 0 and 1 instead and skips the epilogue
  const __amdgpu_buffer_rsrc_t wrs =
      make_rsrc(a.panel + (int64_t)e * a.expert_bytes, (uint32_t)a.expert_bytes);
  const int g0 = nt * kTileGroups + 2 * wg;
  const bool wave_on = (g0 + 2) * kGroupRows <= a.N;
  const int gl = 2 * wg + half;                          // local group this wave copies
  const int go = (wave_on ? g0 + half : half) * (int)a.rg_bytes;
  const uint32_t wlane = (uint32_t)lane * 16;

  // token rows: the stage's 4 NFW DMA pieces of 8 rows go round the 8 waves, piece
  // p = wave + 8 k (a wave past the last piece repeats it: the same bytes to the same place);
  // lane L moves row 8 p + L / 8 into physical slot L % 8 = logical slot (L % 8) ^ (row & 7).
  // The scale piece covers rows 64 wg .. 64 wg + 63, one dword per lane (waves w and w + 4 move
  // the same one), so every wave issues the same loads and no branch splits a stage.
  const __amdgpu_buffer_rsrc_t trs = make_rsrc(a.a_q, (uint32_t)(a.a_rows * K));
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(a.a_sf, (uint32_t)(a.a_rows * (K >> 5)));
  uint32_t t_voff[NP];
  int t_piece[NP];
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    t_piece[k] = min(wave + 8 * k, 4 * NFW - 1);
    const int row = 8 * t_piece[k] + (lane >> 3);
    const int src = row_src[row] < 0 ? 0 : row_src[row];
    const uint32_t u = (uint32_t)((lane & 7) ^ (row & 7));
    t_voff[k] = (uint32_t)src * (uint32_t)K + u * 16;
  }
  uint32_t s_voff;
  {
    const int row = 64 * wg + lane;
    const int src = (row < NFW * 32 && row_src[row] >= 0) ? row_src[row] : 0;
    s_voff = (uint32_t)src * (uint32_t)(K >> 5);
  }
  auto lds_ptr = [](uint8_t* p) { return (__attribute__((address_space(3))) void*)p; };
  // stage st into stage buffer b: weight scale word, the two weight chunks, token rows, token
  // scales (VM_STAGE vector memory operations, always in this order)
  auto load_stage = [&](int b, int st) {
    uint8_t* base = ring + b * SBUF;
    const int sc = st / (kSuperChunks / kStageChunks), c0 = (st * kStageChunks) % kSuperChunks;
    const int wsoff = go + sc * kSuperBytes;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, lds_ptr(base + D::WSC + gl * 256), 4, wlane,
                                             (uint32_t)(wsoff + 2 * c0), 0, 0);
#pragma unroll
    for (int c = 0; c < kStageChunks; ++c)
      buffer_load_lds16(wrs, base + D::WOFF + (gl * kStageChunks + c) * kUnit, wlane,
                        (uint32_t)(wsoff + (1 + c0 + c) * kUnit));
#pragma unroll
    for (int k = 0; k < NP; ++k)
      buffer_load_lds16(trs, base + 8 * t_piece[k] * kMxStageBytes, t_voff[k],
                        (uint32_t)st * kMxStageBytes);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, lds_ptr(base + D::TSC + 64 * wg * 4), 4, s_voff,
                                             (uint32_t)st * 4, 0, 0);
  };

  f32x16_t acc[2][NA];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int j = 0; j < NA; ++j) acc[g][j] = f32x16_t{};

  // ---- prologue: stages 0 .. NB-2 (stage indices clamped, so every wave issues the same
  // loads and the waits below count exactly) ----
#pragma unroll
  for (int b = 0; b < NB - 1; ++b) load_stage(b, min(b, nst - 1));
  wait_vmcnt<(NB - 2) * VM_STAGE>();                     // stage 0 has landed
  lds_barrier();

  // LDS operand addresses: this lane's row of fragment 0 of this wave's half of the tile, its
  // four 16-byte slots (chunk c, K halves) and its scale dword; fragment jj adds jj * 4 KiB.
  // The weight operand of group 2 wg + g, chunk c is this lane's 16 bytes of that chunk.
  const uint32_t sw = (uint32_t)(col & 7);               // row & 7 for every fragment's row
  const int j0 = half == 0 ? 0 : NF0;
  const int hoff = 32 * j0 * kMxStageBytes;              // wave-uniform
  const int soff = D::TSC + 32 * j0 * 4;
  uint32_t lb[kStageChunks][2];
#pragma unroll
  for (int c = 0; c < kStageChunks; ++c)
#pragma unroll
    for (int k = 0; k < 2; ++k)
      lb[c][k] = (uint32_t)(col * kMxStageBytes) + ((((uint32_t)(4 * c + 2 * k + h)) ^ sw) << 4);
  const uint32_t ls = (uint32_t)(col * 4);
  const int woff = D::WOFF + 2 * wg * kStageChunks * kUnit;
  const int wsc = D::WSC + 2 * wg * 256;

  // The MFMAs of one stage over NF fragments: two-deep pipeline over the fragments (the next
  // fragment's operand is read from LDS while the current one's two MFMAs issue), the next
  // chunk's weight operands read during the first fragment of a chunk; the scheduling fences
  // keep the compiler from hoisting more reads ahead.  Plain vector types for the LDS reads:
  // read through HIP's uint4 struct, the compiler makes every LDS read wait for the latest
  // buffer-to-LDS copy to land, which would stall each stage on the copies it has just issued.
  auto mfmas = [&](auto NJ_, const uint8_t* buf) {
    constexpr int NF = decltype(NJ_)::value;
    const uint8_t* hb = buf + hoff;
    const uint8_t* sbase = buf + soff;
    auto read_b = [&](int jj, int c, i32x8_t& B, int& sb) {
      const u32x4_t b0 =
          *reinterpret_cast<const u32x4_t*>(hb + lb[c][0] + jj * 32 * kMxStageBytes);
      const u32x4_t b1 =
          *reinterpret_cast<const u32x4_t*>(hb + lb[c][1] + jj * 32 * kMxStageBytes);
      B = i32x8_t{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                  (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
      const uint32_t tsc = *reinterpret_cast<const uint32_t*>(sbase + ls + jj * 32 * 4);
      sb = (int)((tsc >> (8 * (2 * c + h))) & 0xFFu);
    };
    auto read_a = [&](int c, u32x4_t (&A)[2], uint32_t (&S)[2]) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        A[g] = *reinterpret_cast<const u32x4_t*>(buf + woff + (g * kStageChunks + c) * kUnit +
                                                 wlane);
        S[g] = *reinterpret_cast<const uint32_t*>(buf + wsc + g * 256 + 4 * lane);
      }
    };
    u32x4_t Ac[2], An[2];
    uint32_t Sc[2], Sn[2];
    read_a(0, Ac, Sc);
#pragma unroll
    for (int c = 0; c < kStageChunks; ++c) {
      i32x8_t Bc, Bn;
      int sbc, sbn;
      read_b(0, c, Bc, sbc);
      if (c + 1 < kStageChunks) read_a(c + 1, An, Sn);
      i32x8_t A[2];
      int sa[2];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        A[g] = i32x8_t{(int)Ac[g].x, (int)Ac[g].y, (int)Ac[g].z, (int)Ac[g].w, 0, 0, 0, 0};
        sa[g] = (int)((Sc[g] >> (16 * c)) & 0xFFu);
      }
#pragma unroll
      for (int jj = 0; jj < NF; ++jj) {
        if (jj + 1 < NF) read_b(jj + 1, c, Bn, sbn);
#pragma unroll
        for (int g = 0; g < 2; ++g)
          acc[g][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[g], Bc, acc[g][jj], 4,
                                                                       0, 0, sa[g], 0, sbc);
        __builtin_amdgcn_sched_barrier(0);
        if (jj + 1 < NF) {
          Bc = Bn;
          sbc = sbn;
        }
      }
      if (c + 1 < kStageChunks) {
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          Ac[g] = An[g];
          Sc[g] = Sn[g];
        }
      }
    }
  };

  // one stage: stage st + NB - 1 goes out first into the buffer released by the barrier that
  // ended stage st - 1, then the stage's MFMAs; stage st + 1 has landed once at most the loads
  // issued after it are outstanding: it went out in stage st + 2 - NB (or in the prologue, which
  // is followed by fewer loads), followed by NB - 2 stages' loads
  for (int st = 0; st < nst; ++st) {
    const uint8_t* buf = ring + (st % NB) * SBUF;
    load_stage((st + NB - 1) % NB, min(st + NB - 1, nst - 1));
    if (NJ > 0) mfmas(std::integral_constant<int, NA>{}, buf);
    wait_vmcnt<(NB - 2) * VM_STAGE>();
    lds_barrier();
  }
  // the clamped loads of the last stages must land before the LDS ring is reused
  wait_vmcnt<0>();
  if (!wave_on) return;
  // one fragment's epilogue at a time: the fences keep the compiler from moving every
  // accumulator out at once
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) {
    __builtin_amdgcn_sched_barrier(0);
    const int m = 32 * (j0 + jj) + col;
    if (row_src[m] < 0) continue;
    if (EPI == EPI_DOWN) {
      epilogue_group<EPI_DOWN, true>(a, acc[0][jj], 1.0f, g0, h, 1.0f, row0 + m);
      epilogue_group<EPI_DOWN, true>(a, acc[1][jj], 1.0f, g0 + 1, h, 1.0f, row0 + m);
    } else {
      epilogue_mx<EPI>(a, acc[0][jj], acc[1][jj], g0, h, row0 + m);
    }
  }
}

template <int EPI>
__device__ __forceinline__ void run_nfw_mx(const GemmArgs& a, uint8_t* ring, const int* row_src,
                                           int e, int nt, int64_t row0, int nfw) {
  // waves 0-3 take the first ceil(nfw / 2) token fragments, waves 4-7 the others; each half
  // runs its own copy of the stage loop, specialised for its fragment count
  const bool lo = (threadIdx.x >> 6) < 4;
  switch (nfw) {
    case 1:
      if (lo) run_tile_mx<1, 1, EPI>(a, ring, row_src, e, nt, row0);
      else run_tile_mx<1, 0, EPI>(a, ring, row_src, e, nt, row0);
      break;
    case 2: run_tile_mx<2, 1, EPI>(a, ring, row_src, e, nt, row0); break;
    case 3:
      if (lo) run_tile_mx<3, 2, EPI>(a, ring, row_src, e, nt, row0);
      else run_tile_mx<3, 1, EPI>(a, ring, row_src, e, nt, row0);
      break;
    case 4: run_tile_mx<4, 2, EPI>(a, ring, row_src, e, nt, row0); break;
    case 5:
      if (lo) run_tile_mx<5, 3, EPI>(a, ring, row_src, e, nt, row0);
      else run_tile_mx<5, 2, EPI>(a, ring, row_src, e, nt, row0);
      break;
    case 6: run_tile_mx<6, 3, EPI>(a, ring, row_src, e, nt, row0); break;
    case 7:
      if (lo) run_tile_mx<7, 4, EPI>(a, ring, row_src, e, nt, row0);
      else run_tile_mx<7, 3, EPI>(a, ring, row_src, e, nt, row0);
      break;
    default: run_tile_mx<8, 4, EPI>(a, ring, row_src, e, nt, row0); break;
  }
}

template <int EPI>
__global__ __launch_bounds__(512, 1) void moe_gemm_mx_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* ring = smem;
  int* row_src = reinterpret_cast<int*>(smem + kMxRingBytes);
  int* sh_nvalid = row_src + kMxTileRows;
  int* sh_task = sh_nvalid + 1;
  const int tid = threadIdx.x;
  const int n_tiles = *a.n_tiles;
  // the ticket queues of moe_gemm_kernel: queue x holds tiles x, x + 8, ...; workgroups of XCD
  // x take from queue x and move on to the next queues when theirs is empty
  auto q_tasks = [&](int qq) -> int64_t {
    return n_tiles > qq ? (int64_t)((n_tiles - qq + kXcds - 1) / kXcds) * a.n_ct : 0;
  };
  auto resolve = [&](int& qq, uint32_t ticket) -> int {
    for (int tries = 0; tries < kXcds; ++tries) {
      if ((int64_t)ticket < q_tasks(qq)) {
        const int tile = qq + kXcds * (int)(ticket / a.n_ct);
        return tile * a.n_ct + (int)(ticket % a.n_ct);
      }
      if (tries == kXcds - 1) break;
      qq = (qq + 1) % kXcds;
      ticket = atomicAdd(a.task_counter + qq, 1u);
    }
    return -1;
  };
  int q = (int)(blockIdx.x % kXcds);
  if (tid == 0) *sh_task = resolve(q, atomicAdd(a.task_counter + q, 1u));
  __syncthreads();
  int64_t k = *sh_task;
  while (k >= 0) {
    uint32_t ticket = 0;
    if (tid == 0) ticket = atomicAdd(a.task_counter + q, 1u);   // in flight during this task
    const int2 t = a.tiles[k / a.n_ct];
    const int nt = (int)(k % a.n_ct);
    const int64_t row0 = t.x;
    const int rows_here = min(kMxTileRows, t.y);
    const int e = a.eids[row0 / a.block_m];
    __syncthreads();                         // the previous task is done with LDS
    if (tid == 0) *sh_nvalid = 0;
    __syncthreads();
    if (tid < kMxTileRows) {
      int src = -1;
      if (tid < rows_here) {
        const int64_t ent = a.sorted[row0 + tid];
        if (ent >= 0 && ent < a.sentinel)
          src = a.gather ? (int)(ent / a.top_k) : (int)(row0 + tid);
      }
      row_src[tid] = src;
      if (src >= 0) atomicMax(sh_nvalid, tid + 1);
    }
    __syncthreads();
    const int nvalid = *sh_nvalid;
    if (nvalid > 0 && e >= 0 && e < a.nloc)
      run_nfw_mx<EPI>(a, ring, row_src, e, nt, row0, (nvalid + 31) >> 5);
    __syncthreads();                         // every thread has read sh_task
    if (tid == 0) *sh_task = resolve(q, ticket);
    __syncthreads();
    k = *sh_task;
  }
}

template <int EPI>
hipError_t launch_gemm_mx(const GemmArgs& a, int64_t max_tiles, const char* name, hipStream_t s) {
  const size_t lds = (size_t)kMxRingBytes + kMxTileRows * sizeof(int) + 16;
  auto kern = moe_gemm_mx_kernel<EPI>;
  static std::atomic<size_t> lds_set[kMaxDevices];
  hipError_t err = ensure_dynamic_lds(reinterpret_cast<const void*>(kern), lds, lds_set);
  if (err != hipSuccess) return err;
  const int64_t total = max_tiles * a.n_ct;
  const int64_t maxwg = 256;                         // one workgroup per CU
  int64_t grid = total < maxwg ? total : maxwg;
  grid = (grid + 7) / 8 * 8;
  if (grid == 0) return hipSuccess;
  KernelTimer t(name, s);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(512), lds, s, a);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_gemm(const GemmArgs& a, int64_t max_tiles, const char* name, hipStream_t s) {
  const size_t lds = (size_t)kTokRegion + 2 * kTileRows * sizeof(int) + 16;
  auto kern = moe_gemm_kernel<EPI>;
  static std::atomic<size_t> lds_set[kMaxDevices];
  hipError_t err = ensure_dynamic_lds(reinterpret_cast<const void*>(kern), lds, lds_set);
  if (err != hipSuccess) return err;
  // the most tasks the kernel can make (the down GEMM may halve its chains to 2)
  const int64_t n_ct_max = EPI == EPI_DOWN ? (a.n_nt + 1) / 2 : a.n_ct;
  const int64_t total = max_tiles * n_ct_max;
  const int64_t maxwg = kCus;                        // one workgroup per CU
  int64_t grid = total < maxwg ? total : maxwg;
  grid = (grid + 7) / 8 * 8;
  if (grid == 0) return hipSuccess;
  KernelTimer t(name, s);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(512), lds, s, a);
  return hipGetLastError();
}

}  // namespace

int64_t panel_matrix_bytes(int num_experts, int64_t rows, int64_t K) {
  return (int64_t)num_experts * panel_geom(rows, K).expert_bytes;
}

hipError_t launch_prepare(const uint8_t* w_q, const uint8_t* w_sf, int num_experts, int64_t rows,
                          int64_t K, int gated_rows_half, uint8_t* panel, hipStream_t s, bool mx) {
  int64_t pieces = panel_matrix_bytes(num_experts, rows, K) / 16;
  if (pieces == 0) return hipSuccess;
  KernelTimer t("prepare_weights", s);
  hipLaunchKernelGGL(prepare_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, s, w_q,
                     w_sf, rows, K, (int64_t)gated_rows_half, pieces, panel, (int)mx);
  return hipGetLastError();
}

hipError_t launch_moe_gemms(const MoeGemmProblem& p, hipStream_t s) {
  const bool gated = p.act == BFP4_ACT_SWIGLU || p.act == BFP4_ACT_GEGLU;
  const int64_t N1 = gated ? 2 * p.I : p.I;
  const int64_t cap_blocks = p.cap / p.block_m;
  // Decode: one plan block of <= 32 rows per task; prefill: tiles of up to kTileRows plan rows
  // (several blocks of one expert, or slices of larger blocks) from the device-built tile list.
  const bool small = p.block_m <= 32;
  // row groups per task: tiled n-tiles are 4 * 2 groups (256 rows); a decode task takes
  // 4 FN / KS groups (gemv_shape), counting at most one plan block per assignment
  const int64_t est_blocks = std::min<int64_t>(cap_blocks, p.M * p.top_k);
  const GemvShape sh1 = small ? gemv_shape(est_blocks, N1, p.H, (int)p.block_m) : GemvShape{2, 1};
  const GemvShape sh2 = small ? gemv_shape(est_blocks, p.H, p.I, (int)p.block_m) : GemvShape{2, 1};
  const int64_t rows1 = 4 * sh1.fn / sh1.ks * kGroupRows, rows2 = 4 * sh2.fn / sh2.ks * kGroupRows;

  GemmArgs g1{};
  g1.a_q = p.a_q;
  g1.a_sf = p.a_sf;
  g1.a_rows = p.M;
  g1.a_dec = p.a_dec;
  g1.a_const_scale = 0.0f;
  g1.a_rowq = p.H / 2;
  g1.gather = 1;
  g1.sorted = p.sorted;
  g1.eids = p.eids;
  g1.ntpp = p.ntpp;
  g1.cap = p.cap;
  g1.sentinel = p.M * p.top_k;
  g1.top_k = p.top_k;
  g1.block_m = p.block_m;
  g1.nloc = p.nloc;
  const int64_t max_tiles = moe_gemm_max_tiles(p.cap, p.block_m);
  int2* tile_tmp = reinterpret_cast<int2*>(p.tile_ws);
  int2* tiles = tile_tmp + 2 * max_tiles;     // after max_tiles int2 + max_tiles int (rounded up)
  int32_t* n_tiles = reinterpret_cast<int32_t*>(tiles + max_tiles);
  uint32_t* counters = reinterpret_cast<uint32_t*>(n_tiles + 1);
  if (!small) {
    g1.tiles = tiles;
    g1.n_tiles = n_tiles;
    g1.task_counter = counters;
    const int64_t n8 = p.M * (p.H / 8);
    KernelTimer t("tile_list_decode_tokens", s);
    hipLaunchKernelGGL(tile_list_decode_kernel, dim3((unsigned)(1 + (n8 + 1023) / 1024)),
                       dim3(1024), 0, s, p.eids, p.sorted, p.ntpp, p.cap, p.block_m,
                       (int64_t)(p.M * p.top_k), p.nloc, tile_tmp, tiles, n_tiles, counters,
                       p.a_q, p.a_sf, n8, p.a16);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  PanelGeom pg1 = panel_geom(N1, p.H);
  g1.panel = p.panel1;
  g1.expert_bytes = pg1.expert_bytes;
  g1.rg_bytes = pg1.rg_bytes;
  g1.nch = (int)pg1.nch;
  g1.N = (int)N1;
  g1.n_nt = (int)((N1 + rows1 - 1) / rows1);
  g1.chain = kChainGemm1;
  g1.n_ct = (g1.n_nt + g1.chain - 1) / g1.chain;
  g1.alpha_a = p.alpha1_gate;
  g1.alpha_b = p.alpha1_up;
  g1.act = p.act;
  g1.c2 = p.c2;
  g1.I = p.I;
  // the tiled down GEMM reads the FP16 copy h16, so the tiled gate/up GEMM writes the NVFP4
  // intermediate only when the caller asks for it
  g1.hq = (small || p.keep_hq) ? p.hq : nullptr;
  g1.hsf = (small || p.keep_hq) ? p.hsf : nullptr;
  g1.t16 = small ? nullptr : p.a16;
  g1.t16_rowb = p.H * 2;
  g1.h16 = small ? nullptr : p.h16;
  g1.dbg_pre = p.dbg_pre;
  g1.dbg_inter = p.dbg_inter;

  GemmArgs g2 = g1;
  g2.a_q = p.hq;
  g2.a_sf = p.hsf;
  g2.a_rows = p.cap;
  g2.a_dec = nullptr;
  g2.a_const_scale = 1.0f / p.c2;
  g2.t16 = small ? nullptr : p.h16;
  g2.t16_rowb = p.I * 2;
  g2.h16 = nullptr;
  g2.task_counter = counters + kXcds;
  g2.a_rowq = p.I / 2;
  g2.gather = 0;
  PanelGeom pg2 = panel_geom(p.H, p.I);
  g2.panel = p.panel2;
  g2.expert_bytes = pg2.expert_bytes;
  g2.rg_bytes = pg2.rg_bytes;
  g2.nch = (int)pg2.nch;
  g2.N = (int)p.H;
  g2.n_nt = (int)((p.H + rows2 - 1) / rows2);
  g2.chain = kChainGemm2;
  g2.n_ct = (g2.n_nt + g2.chain - 1) / g2.chain;
  g2.alpha_a = p.alpha2;
  g2.alpha_b = nullptr;
  g2.y = p.y;
  g2.Hout = p.H;
  g2.dbg_pre = nullptr;
  g2.dbg_inter = nullptr;

  hipError_t err;
  if (small) {
    static const char* const kName[] = {
        "gemm1_swiglu_decode", "gemm1_relu2_decode", "gemm1_geglu_decode", "gemm1_gelu_decode",
        "gemm1_relu_decode", "gemm1_silu_decode", "gemm1_identity_decode"};
    const char* nm = kName[p.act];
    err = p.act == BFP4_ACT_SWIGLU ? launch_gemv_shape<EPI_SWIGLU>(sh1, g1, cap_blocks, nm, s)
        : p.act == BFP4_ACT_RELU2  ? launch_gemv_shape<EPI_RELU2>(sh1, g1, cap_blocks, nm, s)
        : p.act == BFP4_ACT_GEGLU  ? launch_gemv_shape<EPI_GEGLU>(sh1, g1, cap_blocks, nm, s)
                              : launch_gemv_shape<EPI_ACT>(sh1, g1, cap_blocks, nm, s);
    if (err != hipSuccess) return err;
    return launch_gemv_shape<EPI_DOWN>(sh2, g2, cap_blocks, "gemm2_down_decode", s);
  }
  // the prefill kernels address their FP16 token operands with 32-bit buffer offsets
  if (p.M * p.H * 2 >= (int64_t(1) << 31) || p.cap * p.I * 2 >= (int64_t(1) << 31))
    return hipErrorInvalidValue;
  static const char* const kName[] = {
      "gemm1_swiglu_prefill", "gemm1_relu2_prefill", "gemm1_geglu_prefill", "gemm1_gelu_prefill",
      "gemm1_relu_prefill", "gemm1_silu_prefill", "gemm1_identity_prefill"};
  const char* nm = kName[p.act];
  err = p.act == BFP4_ACT_SWIGLU ? launch_gemm<EPI_SWIGLU>(g1, max_tiles, nm, s)
      : p.act == BFP4_ACT_RELU2  ? launch_gemm<EPI_RELU2>(g1, max_tiles, nm, s)
      : p.act == BFP4_ACT_GEGLU  ? launch_gemm<EPI_GEGLU>(g1, max_tiles, nm, s)
                            : launch_gemm<EPI_ACT>(g1, max_tiles, nm, s);
  if (err != hipSuccess) return err;
  return launch_gemm<EPI_DOWN>(g2, max_tiles, "gemm2_down_prefill", s);
}

// row sources and scales (64 words), then each staged row: K/2 packed bytes and K/16 scale
// bytes, rounded up to 16 bytes
size_t moe_gemv_lds_bytes(int block_m, int64_t K) {
  const int64_t rows_max = block_m < 32 ? block_m : 32;
  return 64 * sizeof(int) + (size_t)rows_max * ((K / 2 + K / 16 + 15) & ~(int64_t)15);
}

template <bool MX>
hipError_t launch_moe_gemms_w16_fmt(const MoeGemmW16& w, hipStream_t s) {
  const MoeGemmProblem& p = w.p;
  const bool gated = p.act == BFP4_ACT_SWIGLU || p.act == BFP4_ACT_GEGLU;
  const int64_t N1 = gated ? 2 * p.I : p.I;
  const int64_t cap_blocks = p.cap / p.block_m;
  constexpr int FN = 2;
  if (p.block_m > 32) return hipErrorInvalidValue;

  GemmArgs g1{};
  g1.sorted = p.sorted;
  g1.eids = p.eids;
  g1.ntpp = p.ntpp;
  g1.cap = p.cap;
  g1.sentinel = p.M * p.top_k;
  g1.top_k = p.top_k;
  g1.block_m = p.block_m;
  g1.nloc = p.nloc;
  g1.gather = 1;
  const PanelGeom pg1 = panel_geom(N1, p.H);
  g1.panel = p.panel1;
  g1.expert_bytes = pg1.expert_bytes;
  g1.rg_bytes = pg1.rg_bytes;
  g1.nch = (int)pg1.nch;
  g1.N = (int)N1;
  g1.n_nt = (int)((N1 + 4 * FN * 32 - 1) / (4 * FN * 32));
  g1.alpha_a = p.alpha1_gate;
  g1.alpha_b = p.alpha1_up;
  g1.act = p.act;
  g1.I = p.I;
  g1.dbg_pre = p.dbg_pre;
  g1.dbg_inter = p.dbg_inter;
  g1.w16_x = w.x;
  g1.w16_stride = w.x_stride;
  g1.w16_h = w.h;

  GemmArgs g2 = g1;
  g2.gather = 0;
  const PanelGeom pg2 = panel_geom(p.H, p.I);
  g2.panel = p.panel2;
  g2.expert_bytes = pg2.expert_bytes;
  g2.rg_bytes = pg2.rg_bytes;
  g2.nch = (int)pg2.nch;
  g2.N = (int)p.H;
  g2.n_nt = (int)((p.H + 4 * FN * 32 - 1) / (4 * FN * 32));
  g2.alpha_a = p.alpha2;
  g2.alpha_b = nullptr;
  g2.y = p.y;
  g2.Hout = p.H;
  g2.dbg_pre = nullptr;
  g2.dbg_inter = nullptr;
  g2.w16_x = w.h;
  g2.w16_stride = p.I;
  g2.w16_h = nullptr;

  static const char* const kName[] = {
      "gemm1_swiglu_w16_decode", "gemm1_relu2_w16_decode", "gemm1_geglu_w16_decode",
      "gemm1_gelu_w16_decode", "gemm1_relu_w16_decode", "gemm1_silu_w16_decode",
      "gemm1_identity_w16_decode"};
  const char* nm = kName[p.act];
  hipError_t err =
      p.act == BFP4_ACT_SWIGLU ? launch_gemv16<FN, EPI_SWIGLU, MX>(g1, cap_blocks, nm, s)
      : p.act == BFP4_ACT_RELU2 ? launch_gemv16<FN, EPI_RELU2, MX>(g1, cap_blocks, nm, s)
      : p.act == BFP4_ACT_GEGLU ? launch_gemv16<FN, EPI_GEGLU, MX>(g1, cap_blocks, nm, s)
                                : launch_gemv16<FN, EPI_ACT, MX>(g1, cap_blocks, nm, s);
  if (err != hipSuccess) return err;
  return launch_gemv16<FN, EPI_DOWN, MX>(g2, cap_blocks, "gemm2_down_w16_decode", s);
}

hipError_t launch_moe_gemms_mx(const MoeGemmProblem& p, hipStream_t s) {
  const bool gated = p.act == BFP4_ACT_SWIGLU || p.act == BFP4_ACT_GEGLU;
  const int64_t N1 = gated ? 2 * p.I : p.I;
  const int64_t cap_blocks = p.cap / p.block_m;
  constexpr int FN = 2;
  const bool small = p.block_m <= 32;

  GemmArgs g1{};
  g1.a_q = p.a_q;
  g1.a_sf = p.a_sf;
  g1.a_rows = p.M;
  g1.a_rowq = p.H;                 // MXFP8 row: H bytes
  g1.gather = 1;
  g1.sorted = p.sorted;
  g1.eids = p.eids;
  g1.ntpp = p.ntpp;
  g1.cap = p.cap;
  g1.sentinel = p.M * p.top_k;
  g1.top_k = p.top_k;
  g1.block_m = p.block_m;
  g1.nloc = p.nloc;
  const PanelGeom pg1 = panel_geom(N1, p.H);
  g1.panel = p.panel1;
  g1.expert_bytes = pg1.expert_bytes;
  g1.rg_bytes = pg1.rg_bytes;
  g1.nch = (int)pg1.nch;
  g1.N = (int)N1;
  g1.n_nt = (int)((N1 + 4 * FN * 32 - 1) / (4 * FN * 32));
  g1.act = p.act;
  g1.I = p.I;
  g1.hq = p.hq;
  g1.hsf = p.hsf;
  g1.dbg_pre = p.dbg_pre;
  g1.dbg_inter = p.dbg_inter;

  GemmArgs g2 = g1;
  g2.a_q = p.hq;
  g2.a_sf = p.hsf;
  g2.a_rows = p.cap;
  g2.a_rowq = p.I;
  g2.gather = 0;
  const PanelGeom pg2 = panel_geom(p.H, p.I);
  g2.panel = p.panel2;
  g2.expert_bytes = pg2.expert_bytes;
  g2.rg_bytes = pg2.rg_bytes;
  g2.nch = (int)pg2.nch;
  g2.N = (int)p.H;
  g2.n_nt = (int)((p.H + 4 * FN * 32 - 1) / (4 * FN * 32));
  g2.y = p.y;
  g2.Hout = p.H;
  g2.hq = nullptr;
  g2.hsf = nullptr;
  g2.dbg_pre = nullptr;
  g2.dbg_inter = nullptr;

  if (!small) {
    // tiled kernels: the prefill tile list (tiles of up to 256 plan rows, per-XCD ticket queues)
    const int64_t max_tiles = moe_gemm_max_tiles(p.cap, p.block_m);
    int2* tile_tmp = reinterpret_cast<int2*>(p.tile_ws);
    int2* tiles = tile_tmp + 2 * max_tiles;
    int32_t* n_tiles = reinterpret_cast<int32_t*>(tiles + max_tiles);
    uint32_t* counters = reinterpret_cast<uint32_t*>(n_tiles + 1);
    {
      KernelTimer t("tile_list", s);
      hipLaunchKernelGGL(tile_list_kernel, dim3(1), dim3(1024), 0, s, p.eids, p.sorted, p.ntpp,
                         p.cap, p.block_m, (int64_t)(p.M * p.top_k), p.nloc, tile_tmp, tiles,
                         n_tiles, counters);
      hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
    if (p.M * p.H >= (int64_t(1) << 31) || p.cap * p.I >= (int64_t(1) << 31))
      return hipErrorInvalidValue;         // 32-bit buffer offsets of the token operands
    for (GemmArgs* g : {&g1, &g2}) {
      g->tiles = tiles;
      g->n_tiles = n_tiles;
      g->n_ct = g->n_nt;
      g->chain = 1;
    }
    g1.task_counter = counters;
    g2.task_counter = counters + kXcds;
    static const char* const kNameT[] = {
        "gemm1_swiglu_mx_prefill", "gemm1_relu2_mx_prefill", "gemm1_geglu_mx_prefill",
        "gemm1_gelu_mx_prefill", "gemm1_relu_mx_prefill", "gemm1_silu_mx_prefill",
        "gemm1_identity_mx_prefill"};
    const char* nm = kNameT[p.act];
    hipError_t err = p.act == BFP4_ACT_SWIGLU ? launch_gemm_mx<EPI_SWIGLU>(g1, max_tiles, nm, s)
                   : p.act == BFP4_ACT_RELU2  ? launch_gemm_mx<EPI_RELU2>(g1, max_tiles, nm, s)
                   : p.act == BFP4_ACT_GEGLU  ? launch_gemm_mx<EPI_GEGLU>(g1, max_tiles, nm, s)
                                              : launch_gemm_mx<EPI_ACT>(g1, max_tiles, nm, s);
    if (err != hipSuccess) return err;
    return launch_gemm_mx<EPI_DOWN>(g2, max_tiles, "gemm2_down_mx_prefill", s);
  }
  static const char* const kName[] = {
      "gemm1_swiglu_mx_decode", "gemm1_relu2_mx_decode", "gemm1_geglu_mx_decode",
      "gemm1_gelu_mx_decode", "gemm1_relu_mx_decode", "gemm1_silu_mx_decode",
      "gemm1_identity_mx_decode"};
  const char* nm = kName[p.act];
  hipError_t err = p.act == BFP4_ACT_SWIGLU ? launch_gemv_mx<EPI_SWIGLU>(g1, cap_blocks, nm, s)
                 : p.act == BFP4_ACT_RELU2  ? launch_gemv_mx<EPI_RELU2>(g1, cap_blocks, nm, s)
                 : p.act == BFP4_ACT_GEGLU  ? launch_gemv_mx<EPI_GEGLU>(g1, cap_blocks, nm, s)
                                            : launch_gemv_mx<EPI_ACT>(g1, cap_blocks, nm, s);
  if (err != hipSuccess) return err;
  return launch_gemv_mx<EPI_DOWN>(g2, cap_blocks, "gemm2_down_mx_decode", s);
}

hipError_t launch_moe_gemms_w16(const MoeGemmW16& w, hipStream_t s) {
  return w.mx ? launch_moe_gemms_w16_fmt<true>(w, s) : launch_moe_gemms_w16_fmt<false>(w, s);
}

int64_t moe_gemm_max_tiles(int64_t cap, int block_m) {
  return (cap / block_m) * ((block_m + kTileRows - 1) / kTileRows);
}

size_t moe_gemm_tile_ws_bytes(int64_t cap, int block_m) {
  // tile list scratch (int2 + int per tile, as two int2), the ordered list, the count and the
  // two GEMMs' per-XCD ticket counters
  return (size_t)moe_gemm_max_tiles(cap, block_m) * 3 * sizeof(int2) + 4 + 2 * kXcds * 4;
}

}  // namespace bfp4
