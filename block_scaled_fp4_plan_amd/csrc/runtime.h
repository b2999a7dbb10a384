// Host-side internals of the bfp4moe library: kernel launchers and the optional event timer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bfp4 {

// Records a pair of HIP events around one kernel launch when timing is enabled
// (bfp4_profile_begin); otherwise does nothing.
class KernelTimer {
 public:
  KernelTimer(const char* name, hipStream_t stream);
  ~KernelTimer();

 private:
  int slot_;
  hipStream_t stream_;
};

// ---- launchers (arguments already validated by the C entry points) ----
hipError_t launch_plan(const int32_t* ids, int64_t A, int top_k, int num_experts, int offset,
                       int nloc, int block_m, int32_t* sorted, int32_t* eids, int32_t* ntpp,
                       int32_t* ttr, int64_t cap, void* ws, hipStream_t s);
bool plan_uses_small_kernel(int64_t A);
// plan (A <= the one-workgroup limit) and per-row activation quantization in one launch
hipError_t launch_plan_quantize(const int32_t* ids, int64_t A, int num_experts, int offset,
                                int nloc, int block_m, int32_t* sorted, int32_t* eids,
                                int32_t* ntpp, int32_t* ttr, int64_t cap, const uint16_t* x,
                                int64_t rows, int64_t cols, int64_t stride, uint8_t* q,
                                uint8_t* sf, float* dec, hipStream_t s);
int64_t plan_chunks(int64_t A);

hipError_t launch_quantize_mxfp8(const uint16_t* x, int64_t rows, int64_t cols, int64_t stride,
                                uint8_t* q, uint8_t* sf, hipStream_t s);
hipError_t launch_quantize_mxfp4(const uint16_t* x, int64_t rows, int64_t cols, int64_t stride,
                                uint8_t* q, uint8_t* sf, hipStream_t s);
hipError_t launch_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t stride, int mode,
                           int64_t group_rows, float fixed, uint8_t* q, uint8_t* sf, float* dec,
                           void* ws, hipStream_t s);

hipError_t launch_permute(const uint8_t* q, const uint8_t* sf, const float* dec, int64_t M,
                          int64_t H, int top_k, const int32_t* sorted, const int32_t* ntpp,
                          int64_t cap, uint8_t* qp, uint8_t* sp, float* spd, hipStream_t s);

// Debug validation (validate.hip): counts into report[3], which the launchers initialize.
hipError_t launch_check_topk(const int32_t* ids, int64_t M, int top_k, int num_experts,
                             int32_t* report, hipStream_t s);
hipError_t launch_check_plan(const int32_t* sorted, const int32_t* eids, const int32_t* ntpp,
                             int64_t cap, int64_t sentinel, int block_m, int nloc,
                             int32_t* report, hipStream_t s);

hipError_t launch_xor_checksum(const void* buf, int64_t bytes, uint32_t* partial,
                               hipStream_t s);

hipError_t launch_unpack_routing(const int32_t* packed, int64_t n, int32_t* ids,
                                uint16_t* weights, hipStream_t s);

hipError_t launch_finalize(const uint16_t* y, const void* w, bool w_bf16, const int32_t* ttr,
                           int64_t M, int64_t H, int top_k, float rsf, uint16_t* out,
                           hipStream_t s);

// Weight panels: see gemm.hip for the layout.
int64_t panel_matrix_bytes(int num_experts, int64_t rows, int64_t K);
// mx: w_sf holds one E8M0 scale per 32 values (MXFP4), each written to both 16-value slots of
// the panel; otherwise one E4M3 scale per 16 values (NVFP4)
hipError_t launch_prepare(const uint8_t* w_q, const uint8_t* w_sf, int num_experts, int64_t rows,
                          int64_t K, int gated_rows_half, uint8_t* panel, hipStream_t s,
                          bool mx = false);

struct MoeGemmProblem {
  const uint8_t* a_q;
  const uint8_t* a_sf;
  const float* a_dec;
  const uint8_t* panel1;
  const uint8_t* panel2;
  const float* alpha1_gate;
  const float* alpha1_up;
  const float* alpha2;
  float c2;
  const int32_t* sorted;
  const int32_t* eids;
  const int32_t* ntpp;
  int64_t cap;
  int64_t M, H, I;
  int nloc, top_k, block_m, act;
  uint8_t* hq;      // [cap, I/2]
  uint8_t* hsf;     // [cap, I/16]
  bool keep_hq;     // block_m > 32: also store hq / hsf (GEMM2 reads h16 there)
  uint16_t* y;      // [cap, H]
  float* dbg_pre;
  uint16_t* dbg_inter;
  uint8_t* tile_ws;  // moe_gemm_tile_ws_bytes() of scratch for the prefill tile list
  uint16_t* a16;     // block_m > 32: [M, H] FP16 copy of the activations
  uint16_t* h16;     // block_m > 32: [cap, I] FP16 copy of the requantized intermediate
};
hipError_t launch_moe_gemms(const MoeGemmProblem& p, hipStream_t s);
// MXFP4 weights (MXFP4 panels) on MXFP8 activations, block_m <= 32: a_q [M, H] E4M3 bytes, a_sf
// [M, H/32] E8M0; hq [cap, I] and hsf [cap, I/32] the MXFP8 intermediate; a_dec, alphas, c2,
// tile_ws, a16, h16 unused.
hipError_t launch_moe_gemms_mx(const MoeGemmProblem& p, hipStream_t s);

// NVFP4 weight-only mode on BF16 activations (block_m <= 32): the plan, panels, alphas, act,
// dbg_* and y fields of MoeGemmProblem as above; a_q, a_sf, a_dec, c2, hq, hsf, tile_ws, a16,
// h16 unused.
struct MoeGemmW16 {
  MoeGemmProblem p;
  const uint16_t* x;    // [M rows, stride x_stride] BF16 activations
  int64_t x_stride;
  uint16_t* h;          // [cap, I] BF16 intermediate
  bool mx;              // panels hold MXFP4 (E8M0 scales per 32) instead of NVFP4
};
hipError_t launch_moe_gemms_w16(const MoeGemmW16& w, hipStream_t s);
int64_t moe_gemm_max_tiles(int64_t cap, int block_m);
size_t moe_gemm_tile_ws_bytes(int64_t cap, int block_m);
// LDS bytes of a decode-GEMM workgroup (block_m <= 32) whose token rows have K values
size_t moe_gemv_lds_bytes(int block_m, int64_t K);
constexpr size_t kMaxLdsBytes = 160 * 1024;

}  // namespace bfp4
