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

template <int FN, int FM, int EPI, int OCC>
__global__ __launch_bounds__(256, OCC) void moe_gemm_kernel(GemmArgs a) {
  constexpr int MT = 32 * FM;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* tok0 = smem;
  uint8_t* tok1 = smem + MT * kTokPitch;
  int* row_src = reinterpret_cast<int*>(smem + 2 * MT * kTokPitch);
  float* row_scale = reinterpret_cast<float*>(row_src + MT);
  int* sh_nvalid = reinterpret_cast<int*>(row_scale + MT);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  int64_t P = *a.ntpp;
  if (P > a.cap) P = a.cap;
  if (P < 0) P = 0;
  const int64_t n_mt = (P / a.block_m) * a.n_sub;
  const int xcd = blockIdx.x & 7;
  const int64_t Q = gridDim.x >> 3;
  const int64_t li = blockIdx.x >> 3;
  const int64_t mts_here = (n_mt > xcd) ? (n_mt - xcd + 7) / 8 : 0;
  const int64_t ntask = mts_here * a.n_nt;
  const int nst = a.nch / kStageChunks;
  const int64_t sf_rowb = a.a_rowq >> 3;

  for (int64_t k = li; k < ntask; k += Q) {
    const int64_t mt = xcd + 8 * (k / a.n_nt);
    const int nt = (int)(k % a.n_nt);
    const int64_t b = mt / a.n_sub;
    const int sub = (int)(mt % a.n_sub);
    const int64_t row0 = b * a.block_m + (int64_t)sub * MT;
    const int rows_here = min(MT, a.block_m - sub * MT);
    const int e = a.eids[b];
    if (e < 0 || e >= a.nloc) continue;

    __syncthreads();                         // the previous task is done with LDS
    if (tid == 0) *sh_nvalid = 0;
    __syncthreads();
    if (tid < MT) {
      int src = -1;
      float sc = 0.0f;
      if (tid < rows_here) {
        int64_t ent = a.sorted[row0 + tid];
        if (ent >= 0 && ent < a.sentinel) {
          if (a.gather) {
            int64_t t = ent / a.top_k;
            src = (int)t;
            sc = a.a_dec[t];
          } else {
            src = (int)(row0 + tid);
            sc = a.a_const_scale;
          }
        }
      }
      row_src[tid] = src;
      row_scale[tid] = sc;
      if (src >= 0) atomicMax(sh_nvalid, tid + 1);
    }
    __syncthreads();
    const int nvalid = *sh_nvalid;
    if (nvalid == 0) continue;
    const int fm_eff = (nvalid + 31) >> 5;

    // ---- this wave's weight row groups ----
    const int64_t g0 = (int64_t)nt * (4 * FN) + (int64_t)wave * FN;
    const bool wave_on = (g0 + FN) * kGroupRows <= a.N;
    const uint8_t* wbase = a.panel + (int64_t)e * a.expert_bytes + g0 * a.rg_bytes + lane * 16;

    // ---- token loader: FM items per thread, item = (row, 16-value block) of a stage ----
    int it_row[FM];
    const uint8_t* it_q[FM];
    const uint8_t* it_s[FM];
#pragma unroll
    for (int it = 0; it < FM; ++it) {
      int idx = tid + 256 * it;
      int r = idx >> 3, blk = idx & 7;
      it_row[it] = r * kTokPitch + blk * 32;
      int src = row_src[r];
      it_q[it] = (src >= 0) ? a.a_q + (int64_t)src * a.a_rowq + blk * 8 : nullptr;
      it_s[it] = (src >= 0) ? a.a_sf + (int64_t)src * sf_rowb + blk : nullptr;
    }

    f32x16_t acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) acc[i][j] = f32x16_t{};

    uint4 WA[kStageChunks][FN], WB[kStageChunks][FN];
    uint32_t SA[FN], SB[FN];
    uint2 TAq[FM], TBq[FM];
    uint32_t TAs[FM], TBs[FM];

    auto load_w = [&](uint4 (&W)[kStageChunks][FN], uint32_t (&S)[FN], int st) {
      if (!wave_on) return;
      const int64_t sc = st / (kSuperChunks / kStageChunks);
      const int c0 = (st * kStageChunks) % kSuperChunks;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const uint8_t* base = wbase + fn * a.rg_bytes + sc * kSuperBytes;
        S[fn] = *reinterpret_cast<const uint32_t*>(base + 2 * c0);
#pragma unroll
        for (int c = 0; c < kStageChunks; ++c)
          W[c][fn] = *reinterpret_cast<const uint4*>(base + kUnit + (c0 + c) * kUnit);
      }
    };
    auto load_t = [&](uint2 (&Tq)[FM], uint32_t (&Ts)[FM], int st) {
#pragma unroll
      for (int it = 0; it < FM; ++it) {
        if (it_q[it]) {
          Tq[it] = *reinterpret_cast<const uint2*>(it_q[it] + st * 64);
          Ts[it] = it_s[it][st * 8];
        } else {
          Tq[it] = make_uint2(0, 0);
          Ts[it] = 0;
        }
      }
    };
    auto store_t = [&](const uint2 (&Tq)[FM], const uint32_t (&Ts)[FM], uint8_t* buf) {
#pragma unroll
      for (int it = 0; it < FM; ++it) {
        uint32_t s2 = e4m3_scale_h2(Ts[it]);
        h8_t lo = decode8(Tq[it].x, s2);
        h8_t hi = decode8(Tq[it].y, s2);
        *reinterpret_cast<h8_t*>(buf + it_row[it]) = lo;
        *reinterpret_cast<h8_t*>(buf + it_row[it] + 16) = hi;
      }
    };
    auto compute = [&](const uint4 (&W)[kStageChunks][FN], const uint32_t (&S)[FN],
                       const uint8_t* buf) {
      if (!wave_on) return;
#pragma unroll
      for (int c = 0; c < kStageChunks; ++c) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          h8_t T[FM];
#pragma unroll
          for (int fm = 0; fm < FM; ++fm) {
            if (fm < fm_eff)
              T[fm] = *reinterpret_cast<const h8_t*>(buf + (fm * 32 + col) * kTokPitch + c * 128 +
                                                     h * 64 + s * 16);
          }
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
            uint32_t wd = (s == 0) ? W[c][fn].x : (s == 1) ? W[c][fn].y : (s == 2) ? W[c][fn].z
                                                                                   : W[c][fn].w;
            uint32_t sb = (S[fn] >> (8 * (2 * c + (s >> 1)))) & 0xFFu;
            h8_t Wd = decode8(wd, e4m3_scale_h2(sb));
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
              if (fm < fm_eff)
                acc[fn][fm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Wd, T[fm], acc[fn][fm], 0, 0, 0);
            }
          }
        }
      }
    };

    // ---- pipeline: stage s+1 loads in flight while stage s computes ----
    load_w(WA, SA, 0);
    load_t(TAq, TAs, 0);
    store_t(TAq, TAs, tok0);
    lds_barrier();
    for (int st = 0; st < nst; st += 2) {
      if (st + 1 < nst) {
        load_w(WB, SB, st + 1);
        load_t(TBq, TBs, st + 1);
      }
      compute(WA, SA, tok0);
      if (st + 1 < nst) store_t(TBq, TBs, tok1);
      lds_barrier();
      if (st + 1 >= nst) break;
      if (st + 2 < nst) {
        load_w(WA, SA, st + 2);
        load_t(TAq, TAs, st + 2);
      }
      compute(WB, SB, tok1);
      if (st + 2 < nst) store_t(TAq, TAs, tok0);
      lds_barrier();
    }

    // ---- epilogue ----
    if (!wave_on) continue;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      if (fm >= fm_eff) continue;
      const int m = fm * 32 + col;
      if (row_src[m] < 0) continue;
      const float s_row = row_scale[m];
      const int64_t r = row0 + m;
      if (EPI == EPI_DOWN) {
        const float a2 = a.alpha_a[e];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const int64_t k0 = (g0 + fn) * kGroupRows + 16 * h;
          uint32_t pk[8];
#pragma unroll
          for (int v = 0; v < 8; ++v) {
            float y0 = (acc[fn][fm][2 * v] * s_row) * a2;
            float y1 = (acc[fn][fm][2 * v + 1] * s_row) * a2;
            pk[v] = f32_to_bf16(y0) | (f32_to_bf16(y1) << 16);
          }
          uint4* dst = reinterpret_cast<uint4*>(a.y + r * a.Hout + k0);
          dst[0] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
          dst[1] = make_uint4(pk[4], pk[5], pk[6], pk[7]);
        }
      } else {
        const float au = a.alpha_b[e];
        const float ag = a.alpha_a[e];
        constexpr int NOUT = (EPI == EPI_SWIGLU) ? FN / 2 : FN;
#pragma unroll
        for (int p = 0; p < NOUT; ++p) {
          float hv[16];
          int64_t i0;
          if (EPI == EPI_SWIGLU) {
            i0 = ((g0 + 2 * p) >> 1) * kGroupRows + 16 * h;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              float gt = (acc[2 * p][fm][v] * s_row) * ag;
              float up = (acc[2 * p + 1][fm][v] * s_row) * au;
              if (a.dbg_pre) {
                a.dbg_pre[r * (2 * a.I) + i0 + v] = gt;
                a.dbg_pre[r * (2 * a.I) + a.I + i0 + v] = up;
              }
              float sg = gt / (1.0f + expf(-gt));
              hv[v] = sg * up;
            }
          } else {
            i0 = (g0 + p) * kGroupRows + 16 * h;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              float pr = (acc[p][fm][v] * s_row) * au;
              if (a.dbg_pre) a.dbg_pre[r * a.I + i0 + v] = pr;
              float q = pr > 0.0f ? pr : 0.0f;
              hv[v] = q * q;
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
            d[1] = make_uint4(bb[8] | (bb[9] << 16), bb[10] | (bb[11] << 16),
                              bb[12] | (bb[13] << 16), bb[14] | (bb[15] << 16));
          }
          uint32_t lo, hi;
          uint32_t sfb = quant_block16(hv, a.c2, lo, hi);
          *reinterpret_cast<uint2*>(a.hq + r * (a.I >> 1) + (i0 >> 1)) = make_uint2(lo, hi);
          a.hsf[r * (a.I >> 4) + (i0 >> 4)] = (uint8_t)sfb;
        }
      }
    }
  }
}

template <int FN, int FM, int EPI, int OCC>
hipError_t launch_gemm(const GemmArgs& a, int64_t cap_blocks, const char* name, hipStream_t s) {
  constexpr int MT = 32 * FM;
  const size_t lds = 2 * (size_t)MT * kTokPitch + 2 * MT * sizeof(int) + 16;
  auto kern = moe_gemm_kernel<FN, FM, EPI, OCC>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  int64_t total = cap_blocks * a.n_sub * a.n_nt;
  int64_t maxwg = 256LL * OCC;
  int64_t grid = total < maxwg ? total : maxwg;
  grid = (grid + 7) / 8 * 8;
  if (grid == 0) return hipSuccess;
  KernelTimer t(name, s);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), lds, s, a);
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
  const bool small = p.block_m <= 32;
  const int MT = small ? 32 : 128;
  const int FN = small ? 2 : 4;

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
    err = gated ? launch_gemm<2, 1, EPI_SWIGLU, 4>(g1, cap_blocks, "gemm1_swiglu_decode", s)
                : launch_gemm<2, 1, EPI_RELU2, 4>(g1, cap_blocks, "gemm1_relu2_decode", s);
    if (err != hipSuccess) return err;
    return launch_gemm<2, 1, EPI_DOWN, 4>(g2, cap_blocks, "gemm2_down_decode", s);
  }
  err = gated ? launch_gemm<4, 4, EPI_SWIGLU, 1>(g1, cap_blocks, "gemm1_swiglu_prefill", s)
              : launch_gemm<4, 4, EPI_RELU2, 1>(g1, cap_blocks, "gemm1_relu2_prefill", s);
  if (err != hipSuccess) return err;
  return launch_gemm<4, 4, EPI_DOWN, 1>(g2, cap_blocks, "gemm2_down_prefill", s);
}

}  // namespace bfp4
