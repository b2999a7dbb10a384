// C entry points of the bfp4moe library: host-side validation, workspace sizing, launch
// sequencing on the caller's stream, and the optional HIP-event kernel timer.
// The contracts are documented in include/bfp4moe.h.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <string>
#include <vector>

#include "bfp4moe.h"
#include "runtime.h"

namespace bfp4 {

namespace {

struct TimerState {
  bool on = false;
  std::vector<hipEvent_t> start, stop;
  std::vector<const char*> name;
  std::string prefix;          // record only kernels whose name starts with it (empty: all)
  int used = 0;
  int launched = 0;
};
TimerState g_timer;

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// [lo, lo+n) and [lo2, lo2+n2) intersect (byte ranges, empty ranges never intersect)
inline bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// The current device is a gfx950; the answer is kept per device (0 unknown, 1 yes, 2 no), so a
// call after the first makes no device query (none inside a stream capture either).
int device_check() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BFP4_ERR_DEVICE;
  constexpr int kMaxDevices = 64;
  static std::atomic<int> state[kMaxDevices];
  const bool cached = dev >= 0 && dev < kMaxDevices;
  int st = cached ? state[dev].load(std::memory_order_relaxed) : 0;
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return BFP4_ERR_DEVICE;
    st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    if (cached) state[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? BFP4_OK : BFP4_ERR_DEVICE;
}

inline int launched(hipError_t e) { return e == hipSuccess ? BFP4_OK : BFP4_ERR_LAUNCH; }

inline size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

bool valid_block_m(int bm) { return bm >= 8 && bm % 8 == 0; }

// Host-side argument checks of the plan (bfp4_moe_plan's contract): BFP4_OK or the status.
int check_plan_args(const int32_t* topk_ids, int64_t M, int top_k, int num_experts,
                    int local_expert_offset, int num_local_experts, int block_m,
                    const int32_t* sorted_token_ids, const int32_t* expert_ids,
                    const int32_t* num_tokens_post_padded, const int32_t* token_to_row,
                    size_t capacity, const void* workspace, size_t workspace_bytes) {
  if (M < 0 || top_k <= 0 || M * (int64_t)top_k >= (1LL << 31)) return BFP4_ERR_SHAPE;
  if (!valid_block_m(block_m)) return BFP4_ERR_BLOCK_M;
  if (num_experts <= 0 || num_local_experts <= 0 || num_local_experts > 1024 ||
      local_expert_offset < 0 || (int64_t)local_expert_offset + num_local_experts > num_experts)
    return BFP4_ERR_EXPERTS;
  size_t need = bfp4_plan_capacity(M, top_k, num_local_experts, block_m);
  if (capacity < need || capacity % block_m || capacity >= (1ULL << 31)) return BFP4_ERR_CAPACITY;
  if (!num_tokens_post_padded || (capacity && (!sorted_token_ids || !expert_ids)) ||
      (M && (!topk_ids || !token_to_row)))
    return BFP4_ERR_NULL;
  if (!aligned(topk_ids, 4) || !aligned(sorted_token_ids, 4) || !aligned(expert_ids, 4) ||
      !aligned(num_tokens_post_padded, 4) || !aligned(token_to_row, 4))
    return BFP4_ERR_ALIGN;
  size_t ws = bfp4_plan_workspace_size(M, top_k, num_local_experts);
  if (workspace_bytes < ws || (ws && !workspace)) return BFP4_ERR_WORKSPACE;
  return BFP4_OK;
}

// Host-side argument checks of the quantizer (bfp4_quantize_nvfp4's contract).
int check_quant_args(const uint16_t* x_bf16, int64_t rows, int64_t cols, int64_t row_stride,
                     int mode, int64_t group_rows, float fixed_encode_scale, const uint8_t* q,
                     const uint8_t* sf, const float* dec_scale, const void* workspace,
                     size_t workspace_bytes) {
  if (mode < 0 || mode > 2) return BFP4_ERR_MODE;
  if (rows < 0 || cols <= 0 || cols % 32 || row_stride < cols || row_stride % 8 ||
      rows >= (1LL << 31))
    return BFP4_ERR_SHAPE;
  if (mode == BFP4_SCALE_PER_GROUP && (group_rows <= 0 || rows % group_rows)) return BFP4_ERR_SHAPE;
  if (mode == BFP4_SCALE_FIXED && !(isfinite(fixed_encode_scale) && fixed_encode_scale > 0.0f))
    return BFP4_ERR_SCALAR;
  if (rows == 0) return BFP4_OK;
  if (!x_bf16 || !q || !sf || (mode != BFP4_SCALE_FIXED && !dec_scale)) return BFP4_ERR_NULL;
  if (!aligned(x_bf16, 16) || !aligned(q, 8) || !aligned(dec_scale, 4)) return BFP4_ERR_ALIGN;
  size_t ws = bfp4_quantize_workspace_size(rows, mode, group_rows);
  if (workspace_bytes < ws || (ws && !workspace)) return BFP4_ERR_WORKSPACE;
  if (!aligned(workspace, 4)) return BFP4_ERR_ALIGN;
  size_t xb = (size_t)((rows - 1) * row_stride + cols) * 2;
  if (overlaps(x_bf16, xb, q, rows * cols / 2) || overlaps(x_bf16, xb, sf, rows * cols / 16))
    return BFP4_ERR_OVERLAP;
  return BFP4_OK;
}


}  // namespace

KernelTimer::KernelTimer(const char* name, hipStream_t stream) : slot_(-1), stream_(stream) {
  if (!g_timer.on) return;
  g_timer.launched++;
  if (!g_timer.prefix.empty() && strncmp(name, g_timer.prefix.c_str(), g_timer.prefix.size()) != 0)
    return;
  if (g_timer.used >= (int)g_timer.start.size()) return;
  slot_ = g_timer.used++;
  g_timer.name[slot_] = name;
  if (hipEventRecord(g_timer.start[slot_], stream_) != hipSuccess) {
    g_timer.name[slot_] = nullptr;                   // slot left out of the report
    slot_ = -1;
  }
}

KernelTimer::~KernelTimer() {
  if (slot_ >= 0 && hipEventRecord(g_timer.stop[slot_], stream_) != hipSuccess)
    g_timer.name[slot_] = nullptr;
}

}  // namespace bfp4

using namespace bfp4;

namespace {

// Static scratch for bfp4_fused_moe_nvfp4_noalloc: every GPU the library runs on holds one copy
// of this array (BFP4_NOALLOC_SCRATCH_BYTES) until the process ends.  Host code never uses its
// name as an address: scratch_address() asks the runtime for the current device's copy once and
// keeps it per device.
__device__ __align__(256) uint8_t scratch[BFP4_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];

// The current device's address of `scratch`: looked up with the device current on the first call
// on that device (several threads may race here; they store the same address), then cached.
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BFP4_ERR_DEVICE;
  if (dev < 0 || dev >= kMaxScratchDevices) return BFP4_ERR_DEVICE;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BFP4_ERR_DEVICE;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return BFP4_OK;
}

int fused_nvfp4_impl(const uint8_t* a_q, const uint8_t* a_sf, const float* a_dec,
                         const void* panels, size_t panels_bytes, const float* alpha1_gate,
                         const float* alpha1_up, const float* alpha2, float c2,
                         const int32_t* sorted_token_ids, const int32_t* expert_ids,
                         const int32_t* num_tokens_post_padded, const int32_t* token_to_row,
                         size_t capacity, const void* topk_weights, int weights_dtype,
                         int64_t M, int64_t H, int64_t I, int num_local_experts, int top_k,
                         int block_m, int act,
                         float routed_scaling_factor, int do_finalize, uint16_t* out,
                         uint16_t* gemm2_out, const bfp4_debug* debug, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (act < BFP4_ACT_SWIGLU || act > BFP4_ACT_IDENTITY) return BFP4_ERR_MODE;
  if (weights_dtype != BFP4_WEIGHTS_F32 && weights_dtype != BFP4_WEIGHTS_BF16) return BFP4_ERR_MODE;
  const size_t wsz = weights_dtype == BFP4_WEIGHTS_BF16 ? 2 : 4;
  const int gated = act == BFP4_ACT_SWIGLU || act == BFP4_ACT_GEGLU;
  if (M < 0 || top_k <= 0 || M * (int64_t)top_k >= (1LL << 31)) return BFP4_ERR_SHAPE;
  if (H < 256 || H % 256 || I < 128 || I % 128) return BFP4_ERR_SHAPE;
  if (!valid_block_m(block_m)) return BFP4_ERR_BLOCK_M;
  if (num_local_experts <= 0 || num_local_experts > 1024) return BFP4_ERR_EXPERTS;
  if (!(isfinite(c2) && c2 > 0.0f) || !isfinite(routed_scaling_factor)) return BFP4_ERR_SCALAR;
  // the tiled (block_m > 32) GEMMs address their FP16 token operands with 32-bit offsets
  if (block_m > 32 && (M * H * 2 >= (1LL << 31) || (int64_t)capacity * I * 2 >= (1LL << 31)))
    return BFP4_ERR_SHAPE;
  // the decode kernels (block_m <= 32) stage a plan block's token rows whole in LDS
  if (block_m <= 32 && (moe_gemv_lds_bytes(block_m, H) > kMaxLdsBytes ||
                        moe_gemv_lds_bytes(block_m, I) > kMaxLdsBytes))
    return BFP4_ERR_SHAPE;
  // ... and an expert's weight panels with 32-bit offsets
  if (block_m > 32 &&
      (panel_matrix_bytes(1, gated ? 2 * I : I, H) >= (1LL << 31) ||
       panel_matrix_bytes(1, H, I) >= (1LL << 31)))
    return BFP4_ERR_SHAPE;
  size_t need_cap = bfp4_plan_capacity(M, top_k, num_local_experts, block_m);
  if (capacity < need_cap || capacity % block_m || capacity >= (1ULL << 31))
    return BFP4_ERR_CAPACITY;
  if (M == 0) return BFP4_OK;
  if (!a_q || !a_sf || !a_dec || !panels || !alpha1_gate || !alpha1_up || !alpha2 ||
      !sorted_token_ids || !expert_ids || !num_tokens_post_padded || !token_to_row ||
      !topk_weights || (do_finalize && !out) || (!do_finalize && !gemm2_out))
    return BFP4_ERR_NULL;
  if (!aligned(a_q, 16) || !aligned(a_sf, 16) || !aligned(panels, 16) || !aligned(out, 16) ||
      !aligned(gemm2_out, 16) || !aligned(a_dec, 4) || !aligned(alpha1_gate, 4) ||
      !aligned(alpha1_up, 4) || !aligned(alpha2, 4) || !aligned(topk_weights, wsz) ||
      !aligned(sorted_token_ids, 4) || !aligned(expert_ids, 4) || !aligned(token_to_row, 4) ||
      !aligned(workspace, 256))
    return BFP4_ERR_ALIGN;
  if (panels_bytes < bfp4_panel_bytes(num_local_experts, H, I, gated)) return BFP4_ERR_WORKSPACE;
  size_t ws = bfp4_workspace_size(M, H, I, top_k, num_local_experts, block_m, do_finalize);
  if (workspace_bytes < ws || !workspace) return BFP4_ERR_WORKSPACE;
  const int64_t N1 = gated ? 2 * I : I;
  if (debug) {
    if (!aligned(debug->preact, 4) || !aligned(debug->inter, 16) || !aligned(debug->inter_q, 8) ||
        !aligned(debug->inter_f16, 16))
      return BFP4_ERR_ALIGN;
  }
  {
    // the destination (out [M, H] when finalizing, else gemm2_out [capacity, H]) overlaps no
    // input and not the workspace
    const uint16_t* d = do_finalize ? out : gemm2_out;
    const size_t ob = (do_finalize ? (size_t)M : capacity) * (size_t)H * 2;
    const size_t nl = (size_t)num_local_experts * 4, mk = (size_t)M * top_k * 4;
    if (overlaps(d, ob, a_q, M * H / 2) || overlaps(d, ob, a_sf, M * H / 16) ||
        overlaps(d, ob, a_dec, M * 4) || overlaps(d, ob, panels, panels_bytes) ||
        overlaps(d, ob, alpha1_gate, nl) || overlaps(d, ob, alpha1_up, nl) ||
        overlaps(d, ob, alpha2, nl) || overlaps(d, ob, sorted_token_ids, capacity * 4) ||
        overlaps(d, ob, expert_ids, capacity / block_m * 4) ||
        overlaps(d, ob, num_tokens_post_padded, 4) || overlaps(d, ob, token_to_row, mk) ||
        overlaps(d, ob, topk_weights, (size_t)M * top_k * wsz) ||
        overlaps(d, ob, workspace, ws))
      return BFP4_ERR_OVERLAP;
  }
  int dc = device_check();
  if (dc) return dc;

  uint8_t* w = static_cast<uint8_t*>(workspace);
  uint8_t* hq = (debug && debug->inter_q) ? debug->inter_q : w;
  w += align_up(capacity * (size_t)(I / 2));
  uint8_t* hsf = (debug && debug->inter_sf) ? debug->inter_sf : w;
  w += align_up(capacity * (size_t)(I / 16));
  uint8_t* tile_ws = w;
  w += align_up(moe_gemm_tile_ws_bytes((int64_t)capacity, block_m));
  uint16_t* a16 = nullptr;
  uint16_t* h16 = nullptr;
  if (block_m > 32) {
    a16 = reinterpret_cast<uint16_t*>(w);
    w += align_up((size_t)M * H * 2);
    h16 = (debug && debug->inter_f16) ? debug->inter_f16 : reinterpret_cast<uint16_t*>(w);
    w += align_up(capacity * (size_t)I * 2);
  }
  uint16_t* y = do_finalize ? reinterpret_cast<uint16_t*>(w) : gemm2_out;

  MoeGemmProblem p{};
  p.a_q = a_q;
  p.a_sf = a_sf;
  p.a_dec = a_dec;
  p.panel1 = static_cast<const uint8_t*>(panels);
  p.panel2 = p.panel1 + panel_matrix_bytes(num_local_experts, N1, H);
  p.alpha1_gate = alpha1_gate;
  p.alpha1_up = alpha1_up;
  p.alpha2 = alpha2;
  p.c2 = c2;
  p.sorted = sorted_token_ids;
  p.eids = expert_ids;
  p.ntpp = num_tokens_post_padded;
  p.cap = (int64_t)capacity;
  p.M = M;
  p.H = H;
  p.I = I;
  p.nloc = num_local_experts;
  p.top_k = top_k;
  p.block_m = block_m;
  p.act = act;
  p.hq = hq;
  p.hsf = hsf;
  p.keep_hq = debug && (debug->inter_q || debug->inter_sf);
  p.y = y;
  p.dbg_pre = debug ? debug->preact : nullptr;
  p.dbg_inter = debug ? debug->inter : nullptr;
  p.tile_ws = tile_ws;
  p.a16 = a16;
  p.h16 = h16;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_moe_gemms(p, s);
  if (e != hipSuccess) return BFP4_ERR_LAUNCH;
  if (!do_finalize) return BFP4_OK;
  return launched(launch_finalize(y, topk_weights, weights_dtype == BFP4_WEIGHTS_BF16,
                                  token_to_row, M, H, top_k, routed_scaling_factor, out, s));
}

}  // namespace

extern "C" {

const char* bfp4_status_string(int status) {
  switch (status) {
    case BFP4_OK: return "ok";
    case BFP4_ERR_NULL: return "required pointer is NULL";
    case BFP4_ERR_SHAPE: return "size out of range or not a required multiple";
    case BFP4_ERR_ALIGN: return "pointer or stride misaligned";
    case BFP4_ERR_BLOCK_M: return "block_m must be >= 8 and a multiple of 8";
    case BFP4_ERR_CAPACITY: return "plan capacity too small";
    case BFP4_ERR_WORKSPACE: return "workspace or panel buffer too small";
    case BFP4_ERR_OVERLAP: return "output overlaps an input";
    case BFP4_ERR_EXPERTS: return "invalid expert range";
    case BFP4_ERR_MODE: return "unknown activation or scale mode";
    case BFP4_ERR_SCALAR: return "scalar argument not finite or not positive";
    case BFP4_ERR_DEVICE: return "no gfx950 HIP device";
    case BFP4_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

const char* bfp4_version(void) { return "bfp4moe 0.1 (gfx950)"; }

size_t bfp4_plan_capacity(int64_t M, int top_k, int num_local_experts, int block_m) {
  if (M < 0 || top_k <= 0 || num_local_experts <= 0 || !valid_block_m(block_m)) return 0;
  int64_t A = M * top_k;
  int64_t ne = (int64_t)num_local_experts < A ? num_local_experts : A;
  int64_t v = A + ne * (block_m - 1);
  return (size_t)((v + block_m - 1) / block_m * block_m);
}

size_t bfp4_plan_workspace_size(int64_t M, int top_k, int num_local_experts) {
  if (M < 0 || top_k <= 0 || num_local_experts <= 0) return 0;
  int64_t A = M * top_k;
  if (plan_uses_small_kernel(A)) return 0;
  // one count per chunk and local expert, then each local expert's count and segment start
  return (size_t)((plan_chunks(A) + 2) * num_local_experts * sizeof(int32_t));
}

int bfp4_moe_plan(const int32_t* topk_ids, int64_t M, int top_k, int num_experts,
                  int local_expert_offset, int num_local_experts, int block_m,
                  int32_t* sorted_token_ids, int32_t* expert_ids, int32_t* num_tokens_post_padded,
                  int32_t* token_to_row, size_t capacity, void* workspace, size_t workspace_bytes,
                  void* stream) {
  int st = check_plan_args(topk_ids, M, top_k, num_experts, local_expert_offset,
                           num_local_experts, block_m, sorted_token_ids, expert_ids,
                           num_tokens_post_padded, token_to_row, capacity, workspace,
                           workspace_bytes);
  if (st) return st;
  int dc = device_check();
  if (dc) return dc;
  return launched(launch_plan(topk_ids, M * top_k, top_k, num_experts, local_expert_offset,
                              num_local_experts, block_m, sorted_token_ids, expert_ids,
                              num_tokens_post_padded, token_to_row, (int64_t)capacity, workspace,
                              (hipStream_t)stream));
}

size_t bfp4_quantize_workspace_size(int64_t rows, int mode, int64_t group_rows) {
  if (mode != BFP4_SCALE_PER_GROUP || rows <= 0 || group_rows <= 0) return 0;
  return (size_t)((rows / group_rows) * sizeof(uint32_t));
}

int bfp4_quantize_nvfp4(const uint16_t* x_bf16, int64_t rows, int64_t cols, int64_t row_stride,
                        int mode, int64_t group_rows, float fixed_encode_scale, uint8_t* q,
                        uint8_t* sf, float* dec_scale, void* workspace, size_t workspace_bytes,
                        void* stream) {
  int st = check_quant_args(x_bf16, rows, cols, row_stride, mode, group_rows, fixed_encode_scale,
                            q, sf, dec_scale, workspace, workspace_bytes);
  if (st) return st;
  if (rows == 0) return BFP4_OK;
  int dc = device_check();
  if (dc) return dc;
  return launched(launch_quantize(x_bf16, rows, cols, row_stride, mode, group_rows,
                                  fixed_encode_scale, q, sf, dec_scale, workspace,
                                  (hipStream_t)stream));
}

int bfp4_moe_plan_quantize(const int32_t* topk_ids, int64_t M, int top_k, int num_experts,
                           int local_expert_offset, int num_local_experts, int block_m,
                           int32_t* sorted_token_ids, int32_t* expert_ids,
                           int32_t* num_tokens_post_padded, int32_t* token_to_row,
                           size_t capacity, void* plan_workspace, size_t plan_workspace_bytes,
                           const uint16_t* x_bf16, int64_t H, int64_t row_stride, uint8_t* q,
                           uint8_t* sf, float* dec_scale, void* stream) {
  int st = check_plan_args(topk_ids, M, top_k, num_experts, local_expert_offset,
                           num_local_experts, block_m, sorted_token_ids, expert_ids,
                           num_tokens_post_padded, token_to_row, capacity, plan_workspace,
                           plan_workspace_bytes);
  if (st) return st;
  st = check_quant_args(x_bf16, M, H, row_stride, BFP4_SCALE_PER_ROW, 0, 1.0f, q, sf, dec_scale,
                        nullptr, 0);
  if (st) return st;
  int dc = device_check();
  if (dc) return dc;
  const int64_t A = M * top_k;
  hipStream_t s = (hipStream_t)stream;
  if (M > 0 && plan_uses_small_kernel(A))
    return launched(launch_plan_quantize(topk_ids, A, num_experts, local_expert_offset,
                                         num_local_experts, block_m, sorted_token_ids,
                                         expert_ids, num_tokens_post_padded, token_to_row,
                                         (int64_t)capacity, x_bf16, M, H, row_stride, q, sf,
                                         dec_scale, s));
  hipError_t e = launch_plan(topk_ids, A, top_k, num_experts, local_expert_offset,
                             num_local_experts, block_m, sorted_token_ids, expert_ids,
                             num_tokens_post_padded, token_to_row, (int64_t)capacity,
                             plan_workspace, s);
  if (e != hipSuccess || M == 0) return launched(e);
  return launched(launch_quantize(x_bf16, M, H, row_stride, BFP4_SCALE_PER_ROW, 0, 1.0f, q, sf,
                                  dec_scale, nullptr, s));
}

int bfp4_moe_permute(const uint8_t* q, const uint8_t* sf, const float* dec_scale, int64_t M,
                     int64_t H, int top_k, const int32_t* sorted_token_ids,
                     const int32_t* num_tokens_post_padded, size_t capacity, uint8_t* q_perm,
                     uint8_t* sf_perm, float* s_perm, void* stream) {
  if (M < 0 || H <= 0 || H % 32 || top_k <= 0 || capacity >= (1ULL << 31)) return BFP4_ERR_SHAPE;
  if (capacity == 0) return BFP4_OK;
  if (!sorted_token_ids || !num_tokens_post_padded || !q_perm || !sf_perm || !s_perm ||
      (M && (!q || !sf || !dec_scale)))
    return BFP4_ERR_NULL;
  if (!aligned(q, 16) || !aligned(sf, 16) || !aligned(q_perm, 16) || !aligned(sf_perm, 16) ||
      !aligned(dec_scale, 4) || !aligned(s_perm, 4) || !aligned(sorted_token_ids, 4))
    return BFP4_ERR_ALIGN;
  int dc = device_check();
  if (dc) return dc;
  return launched(launch_permute(q, sf, dec_scale, M, H, top_k, sorted_token_ids,
                                 num_tokens_post_padded, (int64_t)capacity, q_perm, sf_perm,
                                 s_perm, (hipStream_t)stream));
}

size_t bfp4_panel_bytes(int num_local_experts, int64_t H, int64_t I, int gated) {
  if (num_local_experts <= 0 || H <= 0 || I <= 0 || H % 256 || I % 128) return 0;
  int64_t N1 = gated ? 2 * I : I;
  return (size_t)(panel_matrix_bytes(num_local_experts, N1, H) +
                  panel_matrix_bytes(num_local_experts, H, I));
}

int bfp4_prepare_weights(const uint8_t* w1_q, const uint8_t* w1_sf, const uint8_t* w2_q,
                         const uint8_t* w2_sf, int num_local_experts, int64_t H, int64_t I,
                         int gated, void* panels, size_t panels_bytes, void* stream) {
  if (num_local_experts <= 0 || num_local_experts > 1024) return BFP4_ERR_EXPERTS;
  if (H < 256 || H % 256 || I < 128 || I % 128) return BFP4_ERR_SHAPE;
  if (!w1_q || !w1_sf || !w2_q || !w2_sf || !panels) return BFP4_ERR_NULL;
  if (!aligned(w1_q, 16) || !aligned(w1_sf, 16) || !aligned(w2_q, 16) || !aligned(w2_sf, 16) ||
      !aligned(panels, 16))
    return BFP4_ERR_ALIGN;
  if (panels_bytes < bfp4_panel_bytes(num_local_experts, H, I, gated)) return BFP4_ERR_WORKSPACE;
  int dc = device_check();
  if (dc) return dc;
  int64_t N1 = gated ? 2 * I : I;
  uint8_t* p1 = static_cast<uint8_t*>(panels);
  uint8_t* p2 = p1 + panel_matrix_bytes(num_local_experts, N1, H);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_prepare(w1_q, w1_sf, num_local_experts, N1, H, gated ? (int)I : 0, p1, s);
  if (e != hipSuccess) return BFP4_ERR_LAUNCH;
  return launched(launch_prepare(w2_q, w2_sf, num_local_experts, H, I, 0, p2, s));
}

size_t bfp4_workspace_size(int64_t M, int64_t H, int64_t I, int top_k, int num_local_experts,
                           int block_m, int do_finalize) {
  size_t cap = bfp4_plan_capacity(M, top_k, num_local_experts, block_m);
  if (H <= 0 || I <= 0) return 0;
  size_t ws = align_up(cap * (size_t)(I / 2)) + align_up(cap * (size_t)(I / 16)) +
              align_up(moe_gemm_tile_ws_bytes((int64_t)cap, block_m));
  // tiled prefill kernels: FP16 copies of the activations and of the requantized intermediate
  if (block_m > 32) ws += align_up((size_t)M * H * 2) + align_up(cap * (size_t)I * 2);
  if (do_finalize) ws += align_up(cap * (size_t)H * 2);
  return ws;
}

int bfp4_fused_moe_nvfp4(const uint8_t* a_q, const uint8_t* a_sf, const float* a_dec,
                         const void* panels, size_t panels_bytes, const float* alpha1_gate,
                         const float* alpha1_up, const float* alpha2, float c2,
                         const int32_t* sorted_token_ids, const int32_t* expert_ids,
                         const int32_t* num_tokens_post_padded, const int32_t* token_to_row,
                         size_t capacity, const void* topk_weights, int weights_dtype,
                         int64_t M, int64_t H, int64_t I, int num_local_experts, int top_k,
                         int block_m, int act,
                         float routed_scaling_factor, int do_finalize, uint16_t* out,
                         uint16_t* gemm2_out, const bfp4_debug* debug, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return fused_nvfp4_impl(a_q, a_sf, a_dec, panels, panels_bytes, alpha1_gate, alpha1_up, alpha2,
                          c2, sorted_token_ids, expert_ids, num_tokens_post_padded, token_to_row,
                          capacity, topk_weights, weights_dtype, M, H, I, num_local_experts,
                          top_k, block_m, act, routed_scaling_factor, do_finalize, out,
                          gemm2_out, debug, workspace, workspace_bytes, stream);
}

int bfp4_fused_moe_nvfp4_noalloc(const uint8_t* a_q, const uint8_t* a_sf, const float* a_dec,
                                 const void* panels, size_t panels_bytes,
                                 const float* alpha1_gate, const float* alpha1_up,
                                 const float* alpha2, float c2, const int32_t* sorted_token_ids,
                                 const int32_t* expert_ids,
                                 const int32_t* num_tokens_post_padded,
                                 const int32_t* token_to_row, size_t capacity,
                                 const void* topk_weights, int weights_dtype, int64_t M,
                                 int64_t H, int64_t I, int num_local_experts, int top_k,
                                 int block_m, int act, float routed_scaling_factor,
                                 int do_finalize, uint16_t* out, uint16_t* gemm2_out,
                                 const bfp4_debug* debug, void* stream) {
  // the workspace this call needs must fit the static scratch array; checked before any device
  // query, so an oversized call fails without touching the device
  const size_t need = bfp4_workspace_size(M, H, I, top_k, num_local_experts, block_m, do_finalize);
  if (need > (size_t)BFP4_NOALLOC_SCRATCH_BYTES) return BFP4_ERR_WORKSPACE;
  int dc = device_check();
  if (dc) return dc;
  void* ws = nullptr;
  dc = scratch_address(&ws);
  if (dc) return dc;
  return fused_nvfp4_impl(a_q, a_sf, a_dec, panels, panels_bytes, alpha1_gate, alpha1_up, alpha2,
                          c2, sorted_token_ids, expert_ids, num_tokens_post_padded, token_to_row,
                          capacity, topk_weights, weights_dtype, M, H, I, num_local_experts,
                          top_k, block_m, act, routed_scaling_factor, do_finalize, out,
                          gemm2_out, debug, ws, (size_t)BFP4_NOALLOC_SCRATCH_BYTES, stream);
}

size_t bfp4_workspace_size_w4a16(int64_t M, int64_t H, int64_t I, int top_k,
                                 int num_local_experts, int block_m, int do_finalize) {
  size_t cap = bfp4_plan_capacity(M, top_k, num_local_experts, block_m);
  if (H <= 0 || I <= 0) return 0;
  size_t ws = align_up(cap * (size_t)I * 2);       // BF16 intermediate
  if (do_finalize) ws += align_up(cap * (size_t)H * 2);
  return ws;
}

int bfp4_quantize_mxfp4(const uint16_t* x_bf16, int64_t rows, int64_t cols, int64_t row_stride,
                        uint8_t* q, uint8_t* sf, void* stream) {
  if (rows < 0 || cols <= 0 || cols % 32 || row_stride < cols || row_stride % 8 ||
      rows >= (1LL << 31))
    return BFP4_ERR_SHAPE;
  if (rows == 0) return BFP4_OK;
  if (!x_bf16 || !q || !sf) return BFP4_ERR_NULL;
  if (!aligned(x_bf16, 16) || !aligned(q, 16)) return BFP4_ERR_ALIGN;
  size_t xb = (size_t)((rows - 1) * row_stride + cols) * 2;
  if (overlaps(x_bf16, xb, q, rows * cols / 2) || overlaps(x_bf16, xb, sf, rows * cols / 32))
    return BFP4_ERR_OVERLAP;
  int dc = device_check();
  if (dc) return dc;
  return launched(launch_quantize_mxfp4(x_bf16, rows, cols, row_stride, q, sf,
                                        (hipStream_t)stream));
}

int bfp4_quantize_mxfp8(const uint16_t* x_bf16, int64_t rows, int64_t cols, int64_t row_stride,
                        uint8_t* q, uint8_t* sf, void* stream) {
  if (rows < 0 || cols <= 0 || cols % 32 || row_stride < cols || row_stride % 8 ||
      rows >= (1LL << 31))
    return BFP4_ERR_SHAPE;
  if (rows == 0) return BFP4_OK;
  if (!x_bf16 || !q || !sf) return BFP4_ERR_NULL;
  if (!aligned(x_bf16, 16) || !aligned(q, 16)) return BFP4_ERR_ALIGN;
  size_t xb = (size_t)((rows - 1) * row_stride + cols) * 2;
  if (overlaps(x_bf16, xb, q, rows * cols) || overlaps(x_bf16, xb, sf, rows * cols / 32))
    return BFP4_ERR_OVERLAP;
  int dc = device_check();
  if (dc) return dc;
  return launched(launch_quantize_mxfp8(x_bf16, rows, cols, row_stride, q, sf,
                                        (hipStream_t)stream));
}

size_t bfp4_workspace_size_mx(int64_t M, int64_t H, int64_t I, int top_k, int num_local_experts,
                              int block_m, int do_finalize) {
  size_t cap = bfp4_plan_capacity(M, top_k, num_local_experts, block_m);
  if (H <= 0 || I <= 0) return 0;
  size_t ws = align_up(cap * (size_t)I) + align_up(cap * (size_t)(I / 32)) +
              align_up(moe_gemm_tile_ws_bytes((int64_t)cap, block_m));
  if (do_finalize) ws += align_up(cap * (size_t)H * 2);
  return ws;
}

int bfp4_fused_moe_mx(const uint8_t* a_q, const uint8_t* a_sf, const void* panels,
                      size_t panels_bytes, const int32_t* sorted_token_ids,
                      const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                      const int32_t* token_to_row, size_t capacity, const void* topk_weights,
                      int weights_dtype, int64_t M, int64_t H, int64_t I, int num_local_experts,
                      int top_k, int block_m, int act, float routed_scaling_factor,
                      int do_finalize, uint16_t* out, uint16_t* gemm2_out,
                      const bfp4_debug* debug, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (act < BFP4_ACT_SWIGLU || act > BFP4_ACT_IDENTITY) return BFP4_ERR_MODE;
  if (weights_dtype != BFP4_WEIGHTS_F32 && weights_dtype != BFP4_WEIGHTS_BF16) return BFP4_ERR_MODE;
  const size_t wsz = weights_dtype == BFP4_WEIGHTS_BF16 ? 2 : 4;
  const int gated = act == BFP4_ACT_SWIGLU || act == BFP4_ACT_GEGLU;
  if (M < 0 || top_k <= 0 || M * (int64_t)top_k >= (1LL << 31)) return BFP4_ERR_SHAPE;
  if (H < 256 || H % 256 || I < 128 || I % 128) return BFP4_ERR_SHAPE;
  if (!valid_block_m(block_m)) return BFP4_ERR_BLOCK_M;
  if (num_local_experts <= 0 || num_local_experts > 1024) return BFP4_ERR_EXPERTS;
  if (!isfinite(routed_scaling_factor)) return BFP4_ERR_SCALAR;
  size_t need_cap = bfp4_plan_capacity(M, top_k, num_local_experts, block_m);
  if (capacity < need_cap || capacity % block_m || capacity >= (1ULL << 31))
    return BFP4_ERR_CAPACITY;
  // the tiled (block_m > 32) kernels address their FP8 token operands and an expert's panels
  // with 32-bit offsets
  if (block_m > 32 && (M * H >= (1LL << 31) || (int64_t)capacity * I >= (1LL << 31) ||
                       panel_matrix_bytes(1, gated ? 2 * I : I, H) >= (1LL << 31) ||
                       panel_matrix_bytes(1, H, I) >= (1LL << 31)))
    return BFP4_ERR_SHAPE;
  if (M == 0) return BFP4_OK;
  if (!a_q || !a_sf || !panels || !sorted_token_ids || !expert_ids || !num_tokens_post_padded ||
      !token_to_row || !topk_weights || (do_finalize && !out) || (!do_finalize && !gemm2_out))
    return BFP4_ERR_NULL;
  if (!aligned(a_q, 16) || !aligned(a_sf, 4) || !aligned(panels, 16) || !aligned(out, 16) ||
      !aligned(gemm2_out, 16) || !aligned(topk_weights, wsz) || !aligned(sorted_token_ids, 4) ||
      !aligned(expert_ids, 4) || !aligned(token_to_row, 4) || !aligned(workspace, 256))
    return BFP4_ERR_ALIGN;
  if (panels_bytes < bfp4_panel_bytes(num_local_experts, H, I, gated)) return BFP4_ERR_WORKSPACE;
  size_t ws = bfp4_workspace_size_mx(M, H, I, top_k, num_local_experts, block_m, do_finalize);
  if (workspace_bytes < ws || !workspace) return BFP4_ERR_WORKSPACE;
  const int64_t N1 = gated ? 2 * I : I;
  if (debug) {
    if (!aligned(debug->preact, 4) || !aligned(debug->inter, 16) || !aligned(debug->inter_q, 16))
      return BFP4_ERR_ALIGN;
  }
  {
    const uint16_t* d = do_finalize ? out : gemm2_out;
    const size_t ob = (do_finalize ? (size_t)M : capacity) * (size_t)H * 2;
    const size_t mk = (size_t)M * top_k * 4;
    if (overlaps(d, ob, a_q, M * H) || overlaps(d, ob, a_sf, M * H / 32) ||
        overlaps(d, ob, panels, panels_bytes) ||
        overlaps(d, ob, sorted_token_ids, capacity * 4) ||
        overlaps(d, ob, expert_ids, capacity / block_m * 4) ||
        overlaps(d, ob, num_tokens_post_padded, 4) || overlaps(d, ob, token_to_row, mk) ||
        overlaps(d, ob, topk_weights, (size_t)M * top_k * wsz) ||
        overlaps(d, ob, workspace, ws))
      return BFP4_ERR_OVERLAP;
  }
  int dc = device_check();
  if (dc) return dc;

  uint8_t* w = static_cast<uint8_t*>(workspace);
  uint8_t* hq = (debug && debug->inter_q) ? debug->inter_q : w;
  w += align_up(capacity * (size_t)I);
  uint8_t* hsf = (debug && debug->inter_sf) ? debug->inter_sf : w;
  w += align_up(capacity * (size_t)(I / 32));
  uint8_t* tile_ws = w;
  w += align_up(moe_gemm_tile_ws_bytes((int64_t)capacity, block_m));
  uint16_t* y = do_finalize ? reinterpret_cast<uint16_t*>(w) : gemm2_out;

  MoeGemmProblem p{};
  p.a_q = a_q;
  p.a_sf = a_sf;
  p.tile_ws = tile_ws;
  p.panel1 = static_cast<const uint8_t*>(panels);
  p.panel2 = p.panel1 + panel_matrix_bytes(num_local_experts, N1, H);
  p.sorted = sorted_token_ids;
  p.eids = expert_ids;
  p.ntpp = num_tokens_post_padded;
  p.cap = (int64_t)capacity;
  p.M = M;
  p.H = H;
  p.I = I;
  p.nloc = num_local_experts;
  p.top_k = top_k;
  p.block_m = block_m;
  p.act = act;
  p.hq = hq;
  p.hsf = hsf;
  p.y = y;
  p.dbg_pre = debug ? debug->preact : nullptr;
  p.dbg_inter = debug ? debug->inter : nullptr;
  hipStream_t s = (hipStream_t)stream;
  if (launch_moe_gemms_mx(p, s) != hipSuccess) return BFP4_ERR_LAUNCH;
  if (!do_finalize) return BFP4_OK;
  return launched(launch_finalize(y, topk_weights, weights_dtype == BFP4_WEIGHTS_BF16,
                                  token_to_row, M, H, top_k, routed_scaling_factor, out, s));
}

int bfp4_prepare_weights_mxfp4(const uint8_t* w1_q, const uint8_t* w1_sf, const uint8_t* w2_q,
                               const uint8_t* w2_sf, int num_local_experts, int64_t H, int64_t I,
                               int gated, void* panels, size_t panels_bytes, void* stream) {
  if (num_local_experts <= 0 || num_local_experts > 1024) return BFP4_ERR_EXPERTS;
  if (H < 256 || H % 256 || I < 128 || I % 128) return BFP4_ERR_SHAPE;
  if (!w1_q || !w1_sf || !w2_q || !w2_sf || !panels) return BFP4_ERR_NULL;
  if (!aligned(w1_q, 16) || !aligned(w2_q, 16) || !aligned(panels, 16)) return BFP4_ERR_ALIGN;
  if (panels_bytes < bfp4_panel_bytes(num_local_experts, H, I, gated)) return BFP4_ERR_WORKSPACE;
  int dc = device_check();
  if (dc) return dc;
  int64_t N1 = gated ? 2 * I : I;
  uint8_t* p1 = static_cast<uint8_t*>(panels);
  uint8_t* p2 = p1 + panel_matrix_bytes(num_local_experts, N1, H);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e =
      launch_prepare(w1_q, w1_sf, num_local_experts, N1, H, gated ? (int)I : 0, p1, s, true);
  if (e != hipSuccess) return BFP4_ERR_LAUNCH;
  return launched(launch_prepare(w2_q, w2_sf, num_local_experts, H, I, 0, p2, s, true));
}

int bfp4_fused_moe_w4a16(const uint16_t* x_bf16, int64_t row_stride, const void* panels,
                         size_t panels_bytes, int weight_format, const float* alpha1_gate,
                         const float* alpha1_up,
                         const float* alpha2, const int32_t* sorted_token_ids,
                         const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                         const int32_t* token_to_row, size_t capacity, const void* topk_weights,
                         int weights_dtype, int64_t M, int64_t H, int64_t I,
                         int num_local_experts, int top_k, int block_m, int act,
                         float routed_scaling_factor, int do_finalize, uint16_t* out,
                         uint16_t* gemm2_out, const bfp4_debug* debug, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (act < BFP4_ACT_SWIGLU || act > BFP4_ACT_IDENTITY) return BFP4_ERR_MODE;
  if (weights_dtype != BFP4_WEIGHTS_F32 && weights_dtype != BFP4_WEIGHTS_BF16) return BFP4_ERR_MODE;
  if (weight_format != BFP4_FORMAT_NVFP4 && weight_format != BFP4_FORMAT_MXFP4)
    return BFP4_ERR_MODE;
  const size_t wsz = weights_dtype == BFP4_WEIGHTS_BF16 ? 2 : 4;
  const int gated = act == BFP4_ACT_SWIGLU || act == BFP4_ACT_GEGLU;
  if (M < 0 || top_k <= 0 || M * (int64_t)top_k >= (1LL << 31)) return BFP4_ERR_SHAPE;
  if (H < 256 || H % 256 || I < 128 || I % 128) return BFP4_ERR_SHAPE;
  if (row_stride < H || row_stride % 8) return BFP4_ERR_SHAPE;
  if (!valid_block_m(block_m) || block_m > 32) return BFP4_ERR_BLOCK_M;
  if (num_local_experts <= 0 || num_local_experts > 1024) return BFP4_ERR_EXPERTS;
  if (!isfinite(routed_scaling_factor)) return BFP4_ERR_SCALAR;
  size_t need_cap = bfp4_plan_capacity(M, top_k, num_local_experts, block_m);
  if (capacity < need_cap || capacity % block_m || capacity >= (1ULL << 31))
    return BFP4_ERR_CAPACITY;
  if (M == 0) return BFP4_OK;
  if (!x_bf16 || !panels || !alpha1_gate || !alpha1_up || !alpha2 || !sorted_token_ids ||
      !expert_ids || !num_tokens_post_padded || !token_to_row || !topk_weights ||
      (do_finalize && !out) || (!do_finalize && !gemm2_out))
    return BFP4_ERR_NULL;
  if (!aligned(x_bf16, 16) || !aligned(panels, 16) || !aligned(out, 16) ||
      !aligned(gemm2_out, 16) || !aligned(alpha1_gate, 4) || !aligned(alpha1_up, 4) ||
      !aligned(alpha2, 4) || !aligned(topk_weights, wsz) || !aligned(sorted_token_ids, 4) ||
      !aligned(expert_ids, 4) || !aligned(token_to_row, 4) || !aligned(workspace, 256))
    return BFP4_ERR_ALIGN;
  if (panels_bytes < bfp4_panel_bytes(num_local_experts, H, I, gated)) return BFP4_ERR_WORKSPACE;
  size_t ws = bfp4_workspace_size_w4a16(M, H, I, top_k, num_local_experts, block_m, do_finalize);
  if (workspace_bytes < ws || !workspace) return BFP4_ERR_WORKSPACE;
  const int64_t N1 = gated ? 2 * I : I;
  if (debug) {
    if (!aligned(debug->preact, 4) || !aligned(debug->inter, 16)) return BFP4_ERR_ALIGN;
  }
  {
    // the destination (out [M, H] when finalizing, else gemm2_out [capacity, H]) overlaps no
    // input and not the workspace
    const uint16_t* d = do_finalize ? out : gemm2_out;
    const size_t ob = (do_finalize ? (size_t)M : capacity) * (size_t)H * 2;
    const size_t nl = (size_t)num_local_experts * 4, mk = (size_t)M * top_k * 4;
    const size_t xb = (size_t)((M - 1) * row_stride + H) * 2;
    if (overlaps(d, ob, x_bf16, xb) || overlaps(d, ob, panels, panels_bytes) ||
        overlaps(d, ob, alpha1_gate, nl) || overlaps(d, ob, alpha1_up, nl) ||
        overlaps(d, ob, alpha2, nl) || overlaps(d, ob, sorted_token_ids, capacity * 4) ||
        overlaps(d, ob, expert_ids, capacity / block_m * 4) ||
        overlaps(d, ob, num_tokens_post_padded, 4) || overlaps(d, ob, token_to_row, mk) ||
        overlaps(d, ob, topk_weights, (size_t)M * top_k * wsz) ||
        overlaps(d, ob, workspace, ws))
      return BFP4_ERR_OVERLAP;
  }
  int dc = device_check();
  if (dc) return dc;

  uint8_t* w = static_cast<uint8_t*>(workspace);
  uint16_t* hbuf = reinterpret_cast<uint16_t*>(w);
  w += align_up(capacity * (size_t)I * 2);
  uint16_t* y = do_finalize ? reinterpret_cast<uint16_t*>(w) : gemm2_out;

  MoeGemmW16 g{};
  MoeGemmProblem& p = g.p;
  p.panel1 = static_cast<const uint8_t*>(panels);
  p.panel2 = p.panel1 + panel_matrix_bytes(num_local_experts, N1, H);
  p.alpha1_gate = alpha1_gate;
  p.alpha1_up = alpha1_up;
  p.alpha2 = alpha2;
  p.sorted = sorted_token_ids;
  p.eids = expert_ids;
  p.ntpp = num_tokens_post_padded;
  p.cap = (int64_t)capacity;
  p.M = M;
  p.H = H;
  p.I = I;
  p.nloc = num_local_experts;
  p.top_k = top_k;
  p.block_m = block_m;
  p.act = act;
  p.y = y;
  p.dbg_pre = debug ? debug->preact : nullptr;
  p.dbg_inter = debug ? debug->inter : nullptr;
  g.x = x_bf16;
  g.x_stride = row_stride;
  g.h = hbuf;
  g.mx = weight_format == BFP4_FORMAT_MXFP4;
  hipStream_t s = (hipStream_t)stream;
  if (launch_moe_gemms_w16(g, s) != hipSuccess) return BFP4_ERR_LAUNCH;
  if (!do_finalize) return BFP4_OK;
  return launched(launch_finalize(y, topk_weights, weights_dtype == BFP4_WEIGHTS_BF16,
                                  token_to_row, M, H, top_k, routed_scaling_factor, out, s));
}

int bfp4_moe_finalize(const uint16_t* gemm2_out, const void* topk_weights, int weights_dtype,
                      const int32_t* token_to_row, int64_t M, int64_t H, int top_k,
                      float routed_scaling_factor, uint16_t* out, void* stream) {
  if (weights_dtype != BFP4_WEIGHTS_F32 && weights_dtype != BFP4_WEIGHTS_BF16) return BFP4_ERR_MODE;
  const size_t wsz = weights_dtype == BFP4_WEIGHTS_BF16 ? 2 : 4;
  if (M < 0 || H <= 0 || H % 8 || top_k <= 0) return BFP4_ERR_SHAPE;
  if (!isfinite(routed_scaling_factor)) return BFP4_ERR_SCALAR;
  if (M == 0) return BFP4_OK;
  if (!gemm2_out || !topk_weights || !token_to_row || !out) return BFP4_ERR_NULL;
  if (!aligned(gemm2_out, 16) || !aligned(out, 16) || !aligned(topk_weights, wsz) ||
      !aligned(token_to_row, 4))
    return BFP4_ERR_ALIGN;
  size_t ob = (size_t)M * H * 2, mk = (size_t)M * top_k * 4;
  if (overlaps(out, ob, topk_weights, (size_t)M * top_k * wsz) ||
      overlaps(out, ob, token_to_row, mk))
    return BFP4_ERR_OVERLAP;
  int dc = device_check();
  if (dc) return dc;
  return launched(launch_finalize(gemm2_out, topk_weights, weights_dtype == BFP4_WEIGHTS_BF16,
                                  token_to_row, M, H, top_k, routed_scaling_factor, out,
                                  (hipStream_t)stream));
}

int bfp4_xor_checksum(const void* buf, size_t bytes, uint32_t* partial, void* stream) {
  if (bytes % 16 || bytes >= (1ULL << 62)) return BFP4_ERR_SHAPE;
  if (!partial || (bytes && !buf)) return BFP4_ERR_NULL;
  if (!aligned(buf, 16) || !aligned(partial, 4)) return BFP4_ERR_ALIGN;
  if (overlaps(buf, bytes, partial, (size_t)BFP4_XOR_PARTIALS * 4)) return BFP4_ERR_OVERLAP;
  int dc = device_check();
  if (dc) return dc;
  return launched(launch_xor_checksum(buf, (int64_t)bytes, partial, (hipStream_t)stream));
}

int bfp4_unpack_routing(const int32_t* packed, int64_t M, int top_k, int32_t* topk_ids,
                        uint16_t* topk_weights, void* stream) {
  if (M < 0 || top_k <= 0 || M * (int64_t)top_k >= (1LL << 31)) return BFP4_ERR_SHAPE;
  if (M == 0) return BFP4_OK;
  if (!packed || !topk_ids || !topk_weights) return BFP4_ERR_NULL;
  if (!aligned(packed, 4) || !aligned(topk_ids, 4) || !aligned(topk_weights, 2))
    return BFP4_ERR_ALIGN;
  const size_t n = (size_t)M * top_k;
  if (overlaps(packed, n * 4, topk_ids, n * 4) || overlaps(packed, n * 4, topk_weights, n * 2) ||
      overlaps(topk_ids, n * 4, topk_weights, n * 2))
    return BFP4_ERR_OVERLAP;
  int dc = device_check();
  if (dc) return dc;
  return launched(launch_unpack_routing(packed, (int64_t)n, topk_ids, topk_weights,
                                        (hipStream_t)stream));
}

int bfp4_check_topk_ids(const int32_t* topk_ids, int64_t M, int top_k, int num_experts,
                        int32_t* report, void* stream) {
  if (M < 0 || top_k <= 0 || M * (int64_t)top_k >= (1LL << 31)) return BFP4_ERR_SHAPE;
  if (num_experts <= 0) return BFP4_ERR_EXPERTS;
  if (!report || (M && !topk_ids)) return BFP4_ERR_NULL;
  if (!aligned(report, 4) || !aligned(topk_ids, 4)) return BFP4_ERR_ALIGN;
  if (overlaps(report, 12, topk_ids, (size_t)M * top_k * 4)) return BFP4_ERR_OVERLAP;
  int dc = device_check();
  if (dc) return dc;
  return launched(launch_check_topk(topk_ids, M, top_k, num_experts, report,
                                    (hipStream_t)stream));
}

int bfp4_check_plan(const int32_t* sorted_token_ids, const int32_t* expert_ids,
                    const int32_t* num_tokens_post_padded, size_t capacity, int64_t M, int top_k,
                    int num_local_experts, int block_m, int32_t* report, void* stream) {
  if (M < 0 || top_k <= 0 || M * (int64_t)top_k >= (1LL << 31)) return BFP4_ERR_SHAPE;
  if (!valid_block_m(block_m)) return BFP4_ERR_BLOCK_M;
  if (num_local_experts <= 0 || num_local_experts > 1024) return BFP4_ERR_EXPERTS;
  if (capacity % block_m || capacity >= (1ULL << 31)) return BFP4_ERR_CAPACITY;
  if (!report || !num_tokens_post_padded || (capacity && (!sorted_token_ids || !expert_ids)))
    return BFP4_ERR_NULL;
  if (!aligned(report, 4) || !aligned(sorted_token_ids, 4) || !aligned(expert_ids, 4) ||
      !aligned(num_tokens_post_padded, 4))
    return BFP4_ERR_ALIGN;
  if (overlaps(report, 12, sorted_token_ids, capacity * 4) ||
      overlaps(report, 12, expert_ids, capacity / block_m * 4) ||
      overlaps(report, 12, num_tokens_post_padded, 4))
    return BFP4_ERR_OVERLAP;
  int dc = device_check();
  if (dc) return dc;
  return launched(launch_check_plan(sorted_token_ids, expert_ids, num_tokens_post_padded,
                                    (int64_t)capacity, M * top_k, block_m, num_local_experts,
                                    report, (hipStream_t)stream));
}

int bfp4_profile_begin(int capacity, const char* name_prefix) {
  if (capacity <= 0 || capacity > (1 << 20)) return BFP4_ERR_SHAPE;
  int dc = device_check();
  if (dc) return dc;
  TimerState& t = g_timer;
  for (auto ev : t.start) (void)hipEventDestroy(ev);   // a failed destroy only leaks the event
  for (auto ev : t.stop) (void)hipEventDestroy(ev);
  t.start.assign(capacity, nullptr);
  t.stop.assign(capacity, nullptr);
  t.name.assign(capacity, nullptr);
  for (int i = 0; i < capacity; ++i) {
    if (hipEventCreate(&t.start[i]) != hipSuccess || hipEventCreate(&t.stop[i]) != hipSuccess)
      return BFP4_ERR_LAUNCH;
  }
  t.prefix = name_prefix ? name_prefix : "";
  t.used = 0;
  t.launched = 0;
  t.on = true;
  return BFP4_OK;
}

int bfp4_profile_end(char* buf, size_t len) {
  TimerState& t = g_timer;
  if (!t.on) return BFP4_ERR_SHAPE;
  t.on = false;
  std::vector<std::string> names;
  std::vector<double> total;
  std::vector<int> count;
  for (int i = 0; i < t.used; ++i) {
    if (t.name[i] == nullptr) continue;              // an event of this slot was not recorded
    if (hipEventSynchronize(t.stop[i]) != hipSuccess) return BFP4_ERR_LAUNCH;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, t.start[i], t.stop[i]) != hipSuccess) return BFP4_ERR_LAUNCH;
    size_t k = 0;
    while (k < names.size() && names[k] != t.name[i]) ++k;
    if (k == names.size()) {
      names.push_back(t.name[i]);
      total.push_back(0.0);
      count.push_back(0);
    }
    total[k] += ms;
    count[k] += 1;
  }
  std::string text;
  char line[256];
  for (size_t k = 0; k < names.size(); ++k) {
    snprintf(line, sizeof(line), "%s %d %.6f\n", names[k].c_str(), count[k], total[k]);
    text += line;
  }
  if (buf && len) {
    size_t n = text.size() < len - 1 ? text.size() : len - 1;
    memcpy(buf, text.data(), n);
    buf[n] = 0;
  }
  return t.launched;
}

}  // extern "C"
