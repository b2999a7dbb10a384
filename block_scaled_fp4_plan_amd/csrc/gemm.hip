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
// * MFMA A operand = 32 weight rows, B operand = 32 plan rows (tokens).  Each wave owns FN weight
//   row groups and streams them from HBM straight into registers (no LDS), one 16-byte load per
//   lane per 64 K values; the token tile (32*FM plan rows) is decoded once per workgroup into LDS
//   as FP16 and shared by the four waves.
// * Weight panels put, for each 32-row group and each 64-value K chunk, exactly the 1 KiB a wave
//   loads in one instruction (lane l: row l%32, K half l/32), scales grouped per 512 K values.
// * Inside a 32-row group the rows are permuted so that each lane's 16 accumulator rows are 16
//   consecutive output indices: the requantization block (16 values) is lane-local, and a GEMM2
//   lane stores 32 contiguous bytes.  Gated W1 alternates gate and up row groups, so a wave
//   holds gate and up of the same 32 intermediate indices.
// * Plan rows past the device-side extent, padding rows and 32-row token fragments with no valid
//   row are skipped; a static schedule interleaves M tiles over the 8 XCDs.
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
constexpr int kTokPitch = 272;      // LDS bytes per token row per stage: 128 FP16 + 16 pad

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
                               uint8_t* __restrict__ panel) {
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
  if (half_rows > 0) {          // gated W1: groups alternate gate (even) and up (odd)
    lr = (grp & 1) * half_rows + (grp >> 1) * kGroupRows + group_perm(rho);
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
      const uint8_t* s = w_sf + row * (K / 16) + 4 * c + 2 * h;
      b[2 * jj] = ok ? s[0] : 0u;
      b[2 * jj + 1] = ok ? s[1] : 0u;
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
  int top_k, block_m, n_sub, nloc;
  const int2* tiles;         // nullptr: one tile per (block, sub-tile); else {first row, rows}
  const int32_t* n_tiles;
  // weights
  const uint8_t* panel;
  int64_t expert_bytes, rg_bytes;
  int nch, N, n_nt;
  const float* alpha_a;      // GEMM1: alpha1_gate; GEMM2: alpha2
  const float* alpha_b;      // GEMM1: alpha1_up
  // GEMM1 epilogue
  float c2;
  int64_t I;
  uint8_t* hq;
  uint8_t* hsf;
  float* dbg_pre;
  uint16_t* dbg_inter;
  // GEMM2 epilogue
  uint16_t* y;
  int64_t Hout;
};

enum { EPI_SWIGLU = 0, EPI_RELU2 = 1, EPI_DOWN = 2 };


// Tiles of up to `tb` consecutive plan blocks of one expert segment (aligned to the segment's
// first block), compacted into a list; run once per fused call by a single workgroup.
__global__ __launch_bounds__(1024) void tile_list_kernel(const int32_t* __restrict__ eids,
                                                         const int32_t* __restrict__ ntpp,
                                                         int64_t cap, int block_m, int tb,
                                                         int2* __restrict__ tiles,
                                                         int32_t* __restrict__ n_tiles) {
  __shared__ int scan[1024];
  __shared__ int carry_start, carry_count;
  const int tid = threadIdx.x;
  int64_t P = *ntpp;
  if (P > cap) P = cap;
  if (P < 0) P = 0;
  const int nblk = (int)(P / block_m);
  if (tid == 0) {
    carry_start = 0;
    carry_count = 0;
  }
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
    const bool is_tile = valid && ((b - s0) % tb == 0);
    __syncthreads();
    // exclusive prefix sum of tile starts
    scan[tid] = is_tile ? 1 : 0;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      int v = (tid >= off) ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const int incl = scan[tid];
    const int total = scan[1023];
    if (is_tile) {
      int nb = 1;
      while (nb < tb && b + nb < nblk && eids[b + nb] == e) ++nb;
      tiles[carry_count + incl - 1] = make_int2(b * block_m, nb * block_m);
    }
    __syncthreads();                         // every thread has read carry_start/count
    if (tid == min(1023, nblk - 1 - base)) carry_start = s0;
    if (tid == 0) carry_count += total;
    __syncthreads();
  }
  if (tid == 0) *n_tiles = carry_count;
}

struct Smem {
  uint8_t* tok;         // two token stages, MT rows each
  int* row_src;
  float* row_scale;
  int* sh_nvalid;
};

// LDS slot (16 bytes = 8 FP16) of the 8 token values a lane needs for chunk c, K half h, MFMA
// step s of a stage.  The writer of 16-value block blk (blk = 4c + 2h + s/2) stores its two
// halves at slots blk and 8 + blk, so eight consecutive writer lanes fill 128 contiguous bytes.
__device__ __forceinline__ int tok_slot(int c, int h, int s) {
  return ((s & 1) << 3) + 4 * c + 2 * h + (s >> 1);
}

// Epilogue of one token column held by this lane: the lane holds 16 consecutive output rows
// (16h + 0..15 of each of its FN weight row groups) for plan row r.
template <int FN, int EPI>
__device__ __forceinline__ void epilogue_frag(const GemmArgs& a, const f32x16_t (&acc)[FN], int e,
                                              int64_t g0, int h, float s_row, int64_t r) {
  if (EPI == EPI_DOWN) {
    const float a2 = a.alpha_a[e];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int64_t k0 = (g0 + fn) * kGroupRows + 16 * h;
      uint32_t pk[8];
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const float y0 = (acc[fn][2 * v] * s_row) * a2;
        const float y1 = (acc[fn][2 * v + 1] * s_row) * a2;
        pk[v] = f32_to_bf16(y0) | (f32_to_bf16(y1) << 16);
      }
      uint4* dst = reinterpret_cast<uint4*>(a.y + r * a.Hout + k0);
      dst[0] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      dst[1] = make_uint4(pk[4], pk[5], pk[6], pk[7]);
    }
    return;
  }
  const float au = a.alpha_b[e];
  const float ag = a.alpha_a[e];
  constexpr int NOUT = (EPI == EPI_SWIGLU) ? FN / 2 : FN;
#pragma unroll
  for (int p = 0; p < NOUT; ++p) {
    float hv[16];
    int64_t i0;
    if (EPI == EPI_SWIGLU) {
      i0 = ((g0 + 2 * p) >> 1) * kGroupRows + 16 * h;
      float gt[16], up[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        gt[v] = (acc[2 * p][v] * s_row) * ag;
        up[v] = (acc[2 * p + 1][v] * s_row) * au;
        hv[v] = (gt[v] / (1.0f + expf(-gt[v]))) * up[v];
      }
      if (a.dbg_pre) {
        float4* dg = reinterpret_cast<float4*>(a.dbg_pre + r * (2 * a.I) + i0);
        float4* du = reinterpret_cast<float4*>(a.dbg_pre + r * (2 * a.I) + a.I + i0);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          dg[v] = make_float4(gt[4 * v], gt[4 * v + 1], gt[4 * v + 2], gt[4 * v + 3]);
          du[v] = make_float4(up[4 * v], up[4 * v + 1], up[4 * v + 2], up[4 * v + 3]);
        }
      }
    } else {
      i0 = (g0 + p) * kGroupRows + 16 * h;
      float pr[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        pr[v] = (acc[p][v] * s_row) * au;
        const float q = pr[v] > 0.0f ? pr[v] : 0.0f;
        hv[v] = q * q;
      }
      if (a.dbg_pre) {
        float4* dp = reinterpret_cast<float4*>(a.dbg_pre + r * a.I + i0);
#pragma unroll
        for (int v = 0; v < 4; ++v)
          dp[v] = make_float4(pr[4 * v], pr[4 * v + 1], pr[4 * v + 2], pr[4 * v + 3]);
      }
    }
    uint32_t bb[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      bb[v] = f32_to_bf16(hv[v]);
      hv[v] = bf16_to_f32(bb[v]);
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
    *reinterpret_cast<uint2*>(a.hq + r * (a.I >> 1) + (i0 >> 1)) = make_uint2(lo, hi);
    a.hsf[r * (a.I >> 4) + (i0 >> 4)] = (uint8_t)sfb;
  }
}

// One tile.  WAVES waves per workgroup: wave % 4 selects FN weight row groups, wave / 4 selects
// the token fragments fm = j * WM + wave / 4 (j < NFW), WM = WAVES / 4.
template <int FN, int FM, int NFW, int EPI, int WAVES, int RING>
__device__ __forceinline__ void run_tile(const GemmArgs& a, const Smem& sm, int e, int nt,
                                         int64_t row0) {
  constexpr int MT = 32 * FM;
  constexpr int WM = WAVES / 4;
  constexpr int NT = 64 * WAVES;                 // threads
  constexpr int ROWS = 32 * NFW * WM;            // token rows staged
  constexpr int ITEMS = ROWS * 8 / NT;           // staging items per thread
  static_assert(ROWS * 8 % NT == 0, "staging items must divide evenly");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_n = wave & 3, wave_m = wave >> 2;
  const int h = lane >> 5, col = lane & 31;
  const int nst = a.nch / kStageChunks;
  const int64_t sf_rowb = a.a_rowq >> 3;

  const int64_t g0 = (int64_t)nt * (4 * FN) + (int64_t)wave_n * FN;
  const bool wave_on = (g0 + FN) * kGroupRows <= a.N;
  // a wave past the last row group still loads (group 0) so that every load is unconditional
  // and the compiler's wait counts stay exact; it skips the MFMAs and the epilogue
  const uint8_t* wbase = a.panel + (int64_t)e * a.expert_bytes + (wave_on ? g0 : 0) * a.rg_bytes +
                         lane * 16;

  // token loader: item = (row, 16-value block) of a 128-value stage; thread tid handles block
  // tid % 8 of rows tid / 8 + it * NT / 8.  Rows without a routed slot are not staged: their
  // LDS rows hold stale values, which only reach MFMA output columns that are discarded.
  const int blk = tid & 7;
  const int lds0 = (tid >> 3) * kTokPitch + blk * 16;
  // rows without a routed slot load token row 0 (any valid row) instead of branching
  int64_t it_src[ITEMS];
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const int src = sm.row_src[(tid >> 3) + it * (NT / 8)];
    it_src[it] = src < 0 ? 0 : src;
  }

  f32x16_t acc[FN][NFW];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < NFW; ++j) acc[i][j] = f32x16_t{};

  uint4 W[RING][kStageChunks][FN];
  uint32_t S[RING][FN];
  uint2 Tq[ITEMS];
  uint32_t Ts[ITEMS];

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
  auto load_t = [&](int st) {
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int64_t src = it_src[it];
      Tq[it] = *reinterpret_cast<const uint2*>(a.a_q + src * a.a_rowq + st * 64 + blk * 8);
      Ts[it] = a.a_sf[src * sf_rowb + st * 8 + blk];
    }
  };
  auto store_t = [&](uint8_t* buf) {
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const uint32_t s2 = e4m3_scale_h2(Ts[it]);
      uint8_t* d = buf + lds0 + it * (NT / 8) * kTokPitch;
      *reinterpret_cast<h8_t*>(d) = decode8(Tq[it].x, s2);
      *reinterpret_cast<h8_t*>(d + 128) = decode8(Tq[it].y, s2);
    }
  };
  auto compute = [&](const uint4 (&Wd)[kStageChunks][FN], const uint32_t (&Sd)[FN],
                     const uint8_t* buf) {
    if (!wave_on) return;
#pragma unroll
    for (int c = 0; c < kStageChunks; ++c) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        h8_t T[NFW];
#pragma unroll
        for (int j = 0; j < NFW; ++j)
          T[j] = *reinterpret_cast<const h8_t*>(buf + ((j * WM + wave_m) * 32 + col) * kTokPitch +
                                                tok_slot(c, h, s) * 16);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const uint32_t wd = (s == 0) ? Wd[c][fn].x : (s == 1) ? Wd[c][fn].y
                              : (s == 2) ? Wd[c][fn].z : Wd[c][fn].w;
          const uint32_t sb = (Sd[fn] >> (8 * (2 * c + (s >> 1)))) & 0xFFu;
          const h8_t Wv = decode8(wd, e4m3_scale_h2(sb));
#pragma unroll
          for (int j = 0; j < NFW; ++j)
            acc[fn][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Wv, T[j], acc[fn][j], 0, 0, 0);
        }
      }
    }
  };

  // ---- pipeline: weights RING-1 stages ahead in registers, tokens one stage ahead in LDS ----
  // Loads are never conditional (stage indices are clamped; the extra loads at the end re-read
  // the last stage), so the waits the compiler places before each use count exactly the loads
  // issued after it and the prefetch stays in flight.  The caller guarantees nst % RING == 0.
#pragma unroll
  for (int d = 0; d < RING - 1; ++d) load_w(W[d], S[d], min(d, nst - 1));
  load_t(0);
  store_t(sm.tok);
  lds_barrier();
  for (int st0 = 0; st0 < nst; st0 += RING) {
#pragma unroll
    for (int d = 0; d < RING; ++d) {
      const int st = st0 + d;
      // token loads first: the wait for them at the end of this stage (vmcnt counts in issue
      // order) must not also wait for the weight loads issued for a later stage
      load_t(min(st + 1, nst - 1));
      load_w(W[(d + RING - 1) % RING], S[(d + RING - 1) % RING], min(st + RING - 1, nst - 1));
      compute(W[d], S[d], sm.tok + (st & 1) * (MT * kTokPitch));
      store_t(sm.tok + ((st + 1) & 1) * (MT * kTokPitch));
      lds_barrier();
    }
  }

  // ---- epilogue ----
  if (!wave_on) return;
#pragma unroll
  for (int j = 0; j < NFW; ++j) {
    const int m = (j * WM + wave_m) * 32 + col;
    if (sm.row_src[m] < 0) continue;
    f32x16_t accj[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) accj[fn] = acc[fn][j];
    epilogue_frag<FN, EPI>(a, accj, e, g0, h, sm.row_scale[m], row0 + m);
  }
}

template <int FN, int FM, int EPI, int WAVES, int RING>
__device__ __forceinline__ void run_nfw(const GemmArgs& a, const Smem& sm, int e, int nt,
                                        int64_t row0, int nfw) {
  if constexpr (FM == 1) {
    run_tile<FN, FM, 1, EPI, WAVES, RING>(a, sm, e, nt, row0);
  } else {
    static_assert(FM / (WAVES / 4) == 4, "prefill tile: 4 token fragments per wave at most");
    switch (nfw) {
      case 1: run_tile<FN, FM, 1, EPI, WAVES, RING>(a, sm, e, nt, row0); break;
      case 2: run_tile<FN, FM, 2, EPI, WAVES, RING>(a, sm, e, nt, row0); break;
      case 3: run_tile<FN, FM, 3, EPI, WAVES, RING>(a, sm, e, nt, row0); break;
      default: run_tile<FN, FM, 4, EPI, WAVES, RING>(a, sm, e, nt, row0); break;
    }
  }
}

template <int FN, int FM, int EPI, int OCC, int WAVES, int RING>
__global__ __launch_bounds__(64 * WAVES, OCC) void moe_gemm_kernel(GemmArgs a) {
  constexpr int MT = 32 * FM;
  constexpr int WM = WAVES / 4;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  Smem sm;
  sm.tok = smem;
  sm.row_src = reinterpret_cast<int*>(smem + 2 * MT * kTokPitch);
  sm.row_scale = reinterpret_cast<float*>(sm.row_src + MT);
  sm.sh_nvalid = reinterpret_cast<int*>(sm.row_scale + MT);

  const int tid = threadIdx.x;
  int64_t P = *a.ntpp;
  if (P > a.cap) P = a.cap;
  if (P < 0) P = 0;
  const int64_t n_mt = a.tiles ? (int64_t)(*a.n_tiles) : (P / a.block_m) * a.n_sub;
  const int xcd = blockIdx.x & 7;
  const int64_t Q = gridDim.x >> 3;
  const int64_t li = blockIdx.x >> 3;
  const int64_t mts_here = (n_mt > xcd) ? (n_mt - xcd + 7) / 8 : 0;
  const int64_t ntask = mts_here * a.n_nt;

  for (int64_t k = li; k < ntask; k += Q) {
    const int64_t mt = xcd + 8 * (k / a.n_nt);
    const int nt = (int)(k % a.n_nt);
    int64_t row0;
    int rows_here;
    if (a.tiles) {
      const int2 t = a.tiles[mt];
      row0 = t.x;
      rows_here = min(MT, t.y);
    } else {
      const int64_t b = mt / a.n_sub;
      const int sub = (int)(mt % a.n_sub);
      row0 = b * a.block_m + (int64_t)sub * MT;
      rows_here = min(MT, a.block_m - sub * MT);
    }
    if (row0 < 0 || row0 + rows_here > P) continue;
    const int e = a.eids[row0 / a.block_m];
    if (e < 0 || e >= a.nloc) continue;

    __syncthreads();                         // the previous task is done with LDS
    if (tid == 0) *sm.sh_nvalid = 0;
    __syncthreads();
    if (tid < MT) {
      int src = -1;
      float sc = 0.0f;
      if (tid < rows_here) {
        const int64_t ent = a.sorted[row0 + tid];
        if (ent >= 0 && ent < a.sentinel) {
          if (a.gather) {
            const int64_t t = ent / a.top_k;
            src = (int)t;
            sc = a.a_dec[t];
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
    if (nvalid == 0) continue;
    // token fragments per wave: ceil(fragments holding a valid row / WM); a trailing fragment
    // with no valid row is computed and discarded
    const int nfw = (((nvalid + 31) >> 5) + WM - 1) / WM;
    const int nst = a.nch / kStageChunks;
    if (nst % RING == 0) {
      run_nfw<FN, FM, EPI, WAVES, RING>(a, sm, e, nt, row0, nfw);
    } else if (RING > 2 && nst % 2 == 0) {
      run_nfw<FN, FM, EPI, WAVES, 2>(a, sm, e, nt, row0, nfw);
    } else {
      run_nfw<FN, FM, EPI, WAVES, 1>(a, sm, e, nt, row0, nfw);
    }
  }
}

// Decode-sized plan blocks (block_m <= 32).  A workgroup task is (plan block, 4*FN weight row
// groups).  The block's routed token rows (at most 32) are copied once, still packed (NVFP4
// bytes and scale bytes for the whole K), into LDS; after one barrier every wave streams its own
// FN weight row groups from HBM RING-1 stages ahead in registers and reads its token operand
// from LDS, with no further barrier, so the four weight streams never wait for each other.
template <int FN, int EPI, int RING>
__global__ __launch_bounds__(256, 4) void moe_gemv_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int* row_src = reinterpret_cast<int*>(smem);
  float* row_scale = reinterpret_cast<float*>(smem + 32 * sizeof(int));
  uint8_t* tok = smem + 64 * sizeof(int);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  // per staged row: K/2 packed bytes then K/16 scale bytes, rounded up to 16 bytes
  const int64_t pitch = (a.a_rowq + (a.a_rowq >> 3) + 15) & ~(int64_t)15;
  int64_t P = *a.ntpp;
  if (P > a.cap) P = a.cap;
  if (P < 0) P = 0;
  const int64_t nblk = P / a.block_m;
  const int64_t ntask = nblk * a.n_nt;
  const int nst = a.nch / kStageChunks;
  const int rows_max = min(a.block_m, 32);

  for (int64_t task = blockIdx.x; task < ntask; task += gridDim.x) {
    const int64_t b = task / a.n_nt;
    const int nt = (int)(task - b * a.n_nt);
    const int e = a.eids[b];
    if (e < 0 || e >= a.nloc) continue;
    __syncthreads();                                   // previous task done with LDS
    if (tid < 32) {
      int src = -1;
      float sc = 0.0f;
      if (tid < rows_max) {
        const int64_t ent = a.sorted[b * a.block_m + tid];
        if (ent >= 0 && ent < a.sentinel) {
          if (a.gather) {
            src = (int)(ent / a.top_k);
            sc = a.a_dec[src];
          } else {
            src = (int)(b * a.block_m + tid);
            sc = a.a_const_scale;
          }
        }
      }
      row_src[tid] = src;
      row_scale[tid] = sc;
    }
    __syncthreads();
    // stage the routed rows: packed bytes in 16-byte units (K/2 is a multiple of 64), scale
    // bytes in 8-byte units (K/16 is a multiple of 8)
    const int64_t q16 = a.a_rowq >> 4, s8 = (a.a_rowq >> 3) >> 3;
    for (int r = 0; r < rows_max; ++r) {
      const int src = row_src[r];
      if (src < 0) continue;
      const uint4* sq = reinterpret_cast<const uint4*>(a.a_q + (int64_t)src * a.a_rowq);
      const uint2* ss = reinterpret_cast<const uint2*>(a.a_sf + (int64_t)src * (a.a_rowq >> 3));
      uint8_t* d = tok + r * pitch;
      for (int64_t i = tid; i < q16; i += 256) reinterpret_cast<uint4*>(d)[i] = sq[i];
      for (int64_t i = tid; i < s8; i += 256) reinterpret_cast<uint2*>(d + a.a_rowq)[i] = ss[i];
    }
    __syncthreads();

    const int64_t g0 = (int64_t)nt * (4 * FN) + (int64_t)wave * FN;
    const bool wave_on = (g0 + FN) * kGroupRows <= a.N;
    const uint8_t* wbase = a.panel + (int64_t)e * a.expert_bytes + (wave_on ? g0 : 0) * a.rg_bytes +
                           lane * 16;
    // lanes past the staged rows read row 0; their MFMA columns are discarded
    const uint8_t* trow = tok + (col < rows_max ? col : 0) * pitch;

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

    // weight loads are unconditional (stage index clamped) so the compiler's waits count them
    // exactly; the tail of the last ring pass leaves through the break
#pragma unroll
    for (int d = 0; d < RING - 1; ++d) load_w(W[d], S[d], min(d, nst - 1));
    for (int st0 = 0; st0 < nst; st0 += RING) {
#pragma unroll
      for (int d = 0; d < RING; ++d) {
        const int st = st0 + d;
        if (st >= nst) break;
        const int nd = (d + RING - 1) % RING;
        load_w(W[nd], S[nd], min(st + RING - 1, nst - 1));
        compute(W[d], S[d], st);
      }
    }
    if (wave_on && col < rows_max && row_src[col] >= 0)
      epilogue_frag<FN, EPI>(a, acc, e, g0, h, row_scale[col], b * a.block_m + col);
  }
}

template <int FN, int EPI>
hipError_t launch_gemv(const GemmArgs& a, int64_t cap_blocks, const char* name, hipStream_t s) {
  constexpr int RING = 3;
  auto kern = moe_gemv_kernel<FN, EPI, RING>;
  const int rows_max = a.block_m < 32 ? a.block_m : 32;
  const size_t lds = 64 * sizeof(int) +
                     (size_t)rows_max * ((a.a_rowq + (a.a_rowq >> 3) + 15) & ~(int64_t)15);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  static size_t attr_lds = 0;
  if (lds > attr_lds) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    attr_lds = lds;
  }
  const int64_t tasks = cap_blocks * a.n_nt;
  const int64_t max_wg = 256LL * 4;                  // resident workgroups (4 waves each)
  const int64_t grid = tasks < max_wg ? tasks : max_wg;
  if (grid == 0) return hipSuccess;
  KernelTimer t(name, s);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), lds, s, a);
  return hipGetLastError();
}

template <int FN, int FM, int EPI, int OCC, int WAVES, int RING>
hipError_t launch_gemm(const GemmArgs& a, int64_t max_tiles, const char* name, hipStream_t s) {
  constexpr int MT = 32 * FM;
  const size_t lds = 2 * (size_t)MT * kTokPitch + 2 * MT * sizeof(int) + 16;
  auto kern = moe_gemm_kernel<FN, FM, EPI, OCC, WAVES, RING>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  const int64_t total = max_tiles * a.n_nt;
  const int64_t maxwg = 256LL * OCC;
  int64_t grid = total < maxwg ? total : maxwg;
  grid = (grid + 7) / 8 * 8;
  if (grid == 0) return hipSuccess;
  KernelTimer t(name, s);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * WAVES), lds, s, a);
  return hipGetLastError();
}

}  // namespace

int64_t panel_matrix_bytes(int num_experts, int64_t rows, int64_t K) {
  return (int64_t)num_experts * panel_geom(rows, K).expert_bytes;
}

hipError_t launch_prepare(const uint8_t* w_q, const uint8_t* w_sf, int num_experts, int64_t rows,
                          int64_t K, int gated_rows_half, uint8_t* panel, hipStream_t s) {
  int64_t pieces = panel_matrix_bytes(num_experts, rows, K) / 16;
  if (pieces == 0) return hipSuccess;
  KernelTimer t("prepare_weights", s);
  hipLaunchKernelGGL(prepare_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, s, w_q,
                     w_sf, rows, K, (int64_t)gated_rows_half, pieces, panel);
  return hipGetLastError();
}

hipError_t launch_moe_gemms(const MoeGemmProblem& p, hipStream_t s) {
  const bool gated = (p.act == 0);
  const int64_t N1 = gated ? 2 * p.I : p.I;
  const int64_t cap_blocks = p.cap / p.block_m;
  // Decode tile: 32 plan rows (one plan block of <= 32 rows); prefill tile: 256 plan rows made
  // of up to 256/block_m consecutive blocks of one expert (or 256-row slices of larger blocks).
  const bool small = p.block_m <= 32;
  const int MT = small ? 32 : 256;
  const int FN = 2;

  GemmArgs g1{};
  g1.a_q = p.a_q;
  g1.a_sf = p.a_sf;
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
  g1.n_sub = (int)((p.block_m + MT - 1) / MT);
  g1.nloc = p.nloc;
  int64_t max_tiles = cap_blocks * g1.n_sub;
  if (!small && p.block_m < MT) {
    // list of multi-block tiles, built on the device from the plan
    const int tb = MT / p.block_m;
    g1.tiles = reinterpret_cast<const int2*>(p.tile_ws);
    g1.n_tiles = reinterpret_cast<const int32_t*>(p.tile_ws + cap_blocks * sizeof(int2));
    g1.n_sub = 1;
    max_tiles = cap_blocks;
    KernelTimer t("tile_list", s);
    hipLaunchKernelGGL(tile_list_kernel, dim3(1), dim3(1024), 0, s, p.eids, p.ntpp, p.cap,
                       p.block_m, tb, reinterpret_cast<int2*>(p.tile_ws),
                       reinterpret_cast<int32_t*>(p.tile_ws + cap_blocks * sizeof(int2)));
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  PanelGeom pg1 = panel_geom(N1, p.H);
  g1.panel = p.panel1;
  g1.expert_bytes = pg1.expert_bytes;
  g1.rg_bytes = pg1.rg_bytes;
  g1.nch = (int)pg1.nch;
  g1.N = (int)N1;
  g1.n_nt = (int)((N1 + 4 * FN * 32 - 1) / (4 * FN * 32));
  g1.alpha_a = p.alpha1_gate;
  g1.alpha_b = p.alpha1_up;
  g1.c2 = p.c2;
  g1.I = p.I;
  g1.hq = p.hq;
  g1.hsf = p.hsf;
  g1.dbg_pre = p.dbg_pre;
  g1.dbg_inter = p.dbg_inter;

  GemmArgs g2 = g1;
  g2.a_q = p.hq;
  g2.a_sf = p.hsf;
  g2.a_dec = nullptr;
  g2.a_const_scale = 1.0f / p.c2;
  g2.a_rowq = p.I / 2;
  g2.gather = 0;
  PanelGeom pg2 = panel_geom(p.H, p.I);
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

  hipError_t err;
  if (small) {
    err = gated ? launch_gemv<2, EPI_SWIGLU>(g1, cap_blocks, "gemm1_swiglu_decode", s)
                : launch_gemv<2, EPI_RELU2>(g1, cap_blocks, "gemm1_relu2_decode", s);
    if (err != hipSuccess) return err;
    return launch_gemv<2, EPI_DOWN>(g2, cap_blocks, "gemm2_down_decode", s);
  }
  err = gated ? launch_gemm<2, 8, EPI_SWIGLU, 1, 8, 2>(g1, max_tiles, "gemm1_swiglu_prefill", s)
              : launch_gemm<2, 8, EPI_RELU2, 1, 8, 2>(g1, max_tiles, "gemm1_relu2_prefill", s);
  if (err != hipSuccess) return err;
  return launch_gemm<2, 8, EPI_DOWN, 1, 8, 2>(g2, max_tiles, "gemm2_down_prefill", s);
}

size_t moe_gemm_tile_ws_bytes(int64_t cap, int block_m) {
  return (size_t)(cap / block_m) * sizeof(int2) + 16;
}

}  // namespace bfp4
