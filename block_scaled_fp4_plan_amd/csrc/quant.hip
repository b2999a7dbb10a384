// NVFP4 quantization, permutation into plan order, and the ordered FP32 combine (finalize).
//
// Quantization follows Megatron-Core "core.inference.moe.flashinfer_nvfp4" (one FP32 scale per
// token or per expert matrix, block size 16, E2M1 max 6, E4M3 max 448), FlashInfer
// "flashinfer.fused_moe.alphamoe_nvfp4_aligned_moe" (packing, linear scales) and vLLM
// "flashinfer_utils" quantize_nvfp4_per_token_input (the FP32 scale returned is the decode
// scale).  The combine follows FlashInfer "flashinfer.fused_moe.FrostLowLatencyConfig" (ordered,
// separate FP32 multiplication and addition) and the alphamoe page's out parameter
// (contributions added to out in FP32, one BF16 conversion).
#include "device.h"
#include "runtime.h"

namespace bfp4 {

namespace {

constexpr int kQuantThreads = 256;

__device__ float block_max_256(float v, float* red) {
  v = wave_max(v);
  int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}

// Row amax of each row, folded into its group's maximum with an integer atomic max (the bit
// pattern of a non-negative float orders like the float).
__global__ __launch_bounds__(kQuantThreads) void group_amax_kernel(const uint16_t* __restrict__ x,
                                                                   int64_t cols, int64_t stride,
                                                                   int64_t group_rows,
                                                                   uint32_t* __restrict__ gmax) {
  __shared__ float red[4];
  int64_t r = blockIdx.x;
  const uint16_t* xr = x + r * stride;
  int64_t nblk = cols >> 4;
  float m = 0.0f;
  for (int64_t b = threadIdx.x; b < nblk; b += kQuantThreads) {
    float v[16];
    load_block16(xr + b * 16, v);
#pragma unroll
    for (int i = 0; i < 16; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(v[i]));
  }
  m = block_max_256(m, red);
  if (threadIdx.x == 0) atomicMax(gmax + r / group_rows, __float_as_uint(m));
}

__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// One workgroup per row.  MODE 0: per-row scale from the row amax; 1: per-group scale from the
// group maxima in gmax; 2: fixed encode scale.
template <int MODE>
__global__ __launch_bounds__(kQuantThreads) void quantize_rows_kernel(
    const uint16_t* __restrict__ x, int64_t cols, int64_t stride, int64_t group_rows, float fixed,
    const uint32_t* __restrict__ gmax, uint8_t* __restrict__ q, uint8_t* __restrict__ sf,
    float* __restrict__ dec) {
  __shared__ float red[4];
  int64_t r = blockIdx.x;
  const uint16_t* xr = x + r * stride;
  int64_t nblk = cols >> 4;
  float s_enc;
  // the first kCached blocks of this thread stay in registers between the amax and the
  // quantization pass (all of them for rows up to kCached * 4096 values)
  constexpr int kCached = 2;
  static_assert(kCached == 2, "the quantization pass below selects between two cached blocks");
  float vc[kCached][16];
  if (MODE == 0) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < kCached; ++i) {
      const int64_t b = threadIdx.x + (int64_t)i * kQuantThreads;
      if (b < nblk) {
        load_block16(xr + b * 16, vc[i]);
#pragma unroll
        for (int k = 0; k < 16; ++k) m = __builtin_fmaxf(m, __builtin_fabsf(vc[i][k]));
      }
    }
    for (int64_t b = threadIdx.x + (int64_t)kCached * kQuantThreads; b < nblk;
         b += kQuantThreads) {
      float v[16];
      load_block16(xr + b * 16, v);
#pragma unroll
      for (int i = 0; i < 16; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(v[i]));
    }
    m = block_max_256(m, red);
    s_enc = encode_scale_from_amax(m);
    if (threadIdx.x == 0) dec[r] = 1.0f / s_enc;
  } else if (MODE == 1) {
    s_enc = encode_scale_from_amax(__uint_as_float(gmax[r / group_rows]));
    if (threadIdx.x == 0 && (r % group_rows) == 0) dec[r / group_rows] = 1.0f / s_enc;
  } else {
    s_enc = fixed;
    if (threadIdx.x == 0 && r == 0 && dec) dec[0] = 1.0f / s_enc;
  }
  uint8_t* qr = q + r * (cols >> 1);
  uint8_t* sr = sf + r * nblk;
  for (int64_t b = threadIdx.x, i = 0; b < nblk; b += kQuantThreads, ++i) {
    float v[16];
    if (MODE == 0 && i < kCached) {
#pragma unroll
      for (int k = 0; k < 16; ++k) v[k] = i == 0 ? vc[0][k] : vc[kCached - 1][k];
    } else {
      load_block16(xr + b * 16, v);
    }
    uint32_t lo, hi;
    uint32_t s = quant_block16(v, s_enc, lo, hi);
    *reinterpret_cast<uint2*>(qr + b * 8) = make_uint2(lo, hi);
    sr[b] = (uint8_t)s;
  }
}

// MXFP4 (E2M1 with one E8M0 scale per 32 values): one workgroup per row, one thread per block of
// 32.  Shared exponent X = floor(log2(amax)) - 2 (2: the exponent of the largest E2M1 magnitude),
// clamped to [-127, 127], scale code X + 127; amax 0 (or below the FP32 normal range, which BF16
// inputs only reach with X < -127) gives code 0; elements are E2M1 of x * 2^-X (an exact
// power-of-two product), nearest with ties to even, saturating at 6.
__global__ __launch_bounds__(kQuantThreads) void quantize_mxfp4_kernel(
    const uint16_t* __restrict__ x, int64_t cols, int64_t stride, uint8_t* __restrict__ q,
    uint8_t* __restrict__ sf) {
  const int64_t r = blockIdx.x;
  const uint16_t* xr = x + r * stride;
  const int64_t nblk = cols >> 5;
  for (int64_t b = threadIdx.x; b < nblk; b += kQuantThreads) {
    float v[32];
    load_block16(xr + b * 32, *reinterpret_cast<float(*)[16]>(v));
    load_block16(xr + b * 32 + 16, *reinterpret_cast<float(*)[16]>(v + 16));
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
    const int ebits = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
    int X = ebits == 0 ? -127 : ebits - 127 - 2;
    X = X < -127 ? -127 : (X > 127 ? 127 : X);
    const uint32_t code = (amax == 0.0f || ebits == 0) ? 0u : (uint32_t)(X + 127);
    const float inv = ldexpf(1.0f, -X);
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = quant8(v + 8 * k, inv);
    *reinterpret_cast<uint4*>(q + r * (cols >> 1) + b * 16) = make_uint4(w[0], w[1], w[2], w[3]);
    sf[r * nblk + b] = (uint8_t)code;
  }
}

// MXFP8 (E4M3 elements with one E8M0 scale per 32 values): one workgroup per row, one thread per
// block of 32.  Shared exponent X = floor(log2(amax)) - 8 (8: the exponent of E4M3's largest
// magnitude, 448 = 1.75 * 2^8), clamped to [-127, 127], scale code X + 127; amax 0 (or below the
// FP32 normal range, where the clamp gives X = -127 anyway) gives code 0; elements are E4M3 of
// x * 2^-X (an exact power-of-two product), nearest with ties to even, saturating at 448, with
// the input's sign bit.
__global__ __launch_bounds__(kQuantThreads) void quantize_mxfp8_kernel(
    const uint16_t* __restrict__ x, int64_t cols, int64_t stride, uint8_t* __restrict__ q,
    uint8_t* __restrict__ sf) {
  const int64_t r = blockIdx.x;
  const uint16_t* xr = x + r * stride;
  const int64_t nblk = cols >> 5;
  for (int64_t b = threadIdx.x; b < nblk; b += kQuantThreads) {
    float v[32];
    load_block16(xr + b * 32, *reinterpret_cast<float(*)[16]>(v));
    load_block16(xr + b * 32 + 16, *reinterpret_cast<float(*)[16]>(v + 16));
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
    uint32_t code;
    const float inv = mx_scale_inverse(amax, kE4M3Emax, code);
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] = e4m3_pack4(v + 4 * k, inv);
    uint4* dst = reinterpret_cast<uint4*>(q + r * cols + b * 32);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
    sf[r * nblk + b] = (uint8_t)code;
  }
}

// Permute: one workgroup of 64 threads per capacity row.
__global__ __launch_bounds__(64) void permute_kernel(const uint8_t* __restrict__ q,
                                                     const uint8_t* __restrict__ sf,
                                                     const float* __restrict__ dec, int64_t M,
                                                     int64_t H, int top_k,
                                                     const int32_t* __restrict__ sorted,
                                                     const int32_t* __restrict__ ntpp,
                                                     uint8_t* __restrict__ qp,
                                                     uint8_t* __restrict__ sp,
                                                     float* __restrict__ spd) {
  int64_t r = blockIdx.x;
  int64_t P = *ntpp;
  int64_t f = (r < P) ? (int64_t)sorted[r] : -1;
  bool valid = f >= 0 && f < M * top_k;
  int64_t t = valid ? f / top_k : 0;
  int64_t qbytes = H >> 1, sbytes = H >> 4;
  const uint4* srcq = reinterpret_cast<const uint4*>(q + t * qbytes);
  uint4* dstq = reinterpret_cast<uint4*>(qp + r * qbytes);
  const uint4 z = make_uint4(0, 0, 0, 0);
  for (int64_t i = threadIdx.x; i < qbytes / 16; i += 64) dstq[i] = valid ? srcq[i] : z;
  const uint8_t* srcs = sf + t * sbytes;
  uint8_t* dsts = sp + r * sbytes;
  if ((sbytes & 15) == 0) {
    for (int64_t i = threadIdx.x; i < sbytes / 16; i += 64)
      reinterpret_cast<uint4*>(dsts)[i] = valid ? reinterpret_cast<const uint4*>(srcs)[i] : z;
  } else {
    for (int64_t i = threadIdx.x; i < sbytes; i += 64) dsts[i] = valid ? srcs[i] : (uint8_t)0;
  }
  if (threadIdx.x == 0) spd[r] = valid ? dec[t] : 0.0f;
}

// Packed routing slots -> expert ids and BF16 scores, one thread per slot.  A packed slot is one
// 32-bit word: the score's BF16 bits in the high half, the expert id as a signed 16-bit integer
// in the low half (sign-extended here; -1, an empty slot, is 0xFFFF).
__global__ __launch_bounds__(256) void unpack_routing_kernel(const int32_t* __restrict__ packed,
                                                             int64_t n, int32_t* __restrict__ ids,
                                                             uint16_t* __restrict__ weights) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t w = (uint32_t)packed[i];
  ids[i] = (int32_t)(int16_t)(uint16_t)(w & 0xFFFFu);
  weights[i] = (uint16_t)(w >> 16);
}

// Finalize: one thread per (token, 8 consecutive hidden values).
// WBF16: the routing weights are BF16 bit patterns, used as their exact FP32 values
template <bool WBF16>
__global__ __launch_bounds__(256) void finalize_kernel(const uint16_t* __restrict__ y,
                                                       const void* __restrict__ w,
                                                       const int32_t* __restrict__ ttr, int64_t M,
                                                       int64_t H, int top_k, float rsf,
                                                       uint16_t* __restrict__ out) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t per_row = H >> 3;
  if (i >= M * per_row) return;
  int64_t t = i / per_row;
  int64_t h = (i - t * per_row) * 8;
  uint4 o = *reinterpret_cast<const uint4*>(out + t * H + h);
  uint32_t ow[4] = {o.x, o.y, o.z, o.w};
  float acc[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    acc[2 * k] = bf16_to_f32(ow[k] & 0xFFFFu);
    acc[2 * k + 1] = bf16_to_f32(ow[k] >> 16);
  }
  const bool scaled = (rsf != 1.0f);
  // slots in groups of 8: the group's rows, then its weights and expert-output rows are loaded
  // together, then added in ascending slot order (unrouted slots: weight never read)
  for (int j0 = 0; j0 < top_k; j0 += 8) {
    int32_t r[8];
    float wt[8];
    uint4 yy[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) r[u] = (j0 + u < top_k) ? ttr[t * top_k + j0 + u] : -1;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (r[u] >= 0) {
        const int64_t wi = t * top_k + j0 + u;
        wt[u] = WBF16 ? bf16_to_f32(static_cast<const uint16_t*>(w)[wi])
                      : static_cast<const float*>(w)[wi];
        yy[u] = *reinterpret_cast<const uint4*>(y + (int64_t)r[u] * H + h);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (r[u] < 0) continue;
      const uint32_t yw[4] = {yy[u].x, yy[u].y, yy[u].z, yy[u].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float p0 = wt[u] * bf16_to_f32(yw[k] & 0xFFFFu);
        float p1 = wt[u] * bf16_to_f32(yw[k] >> 16);
        if (scaled) {
          p0 = p0 * rsf;
          p1 = p1 * rsf;
        }
        acc[2 * k] = acc[2 * k] + p0;
        acc[2 * k + 1] = acc[2 * k + 1] + p1;
      }
    }
  }
  uint4 res;
  res.x = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
  res.y = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
  res.z = f32_to_bf16(acc[4]) | (f32_to_bf16(acc[5]) << 16);
  res.w = f32_to_bf16(acc[6]) | (f32_to_bf16(acc[7]) << 16);
  *reinterpret_cast<uint4*>(out + t * H + h) = res;
}

}  // namespace

hipError_t launch_quantize_mxfp4(const uint16_t* x, int64_t rows, int64_t cols, int64_t stride,
                                uint8_t* q, uint8_t* sf, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  KernelTimer t("quantize_mxfp4", s);
  hipLaunchKernelGGL(quantize_mxfp4_kernel, dim3((unsigned)rows), dim3(kQuantThreads), 0, s, x,
                     cols, stride, q, sf);
  return hipGetLastError();
}

hipError_t launch_quantize_mxfp8(const uint16_t* x, int64_t rows, int64_t cols, int64_t stride,
                                uint8_t* q, uint8_t* sf, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  KernelTimer t("quantize_mxfp8", s);
  hipLaunchKernelGGL(quantize_mxfp8_kernel, dim3((unsigned)rows), dim3(kQuantThreads), 0, s, x,
                     cols, stride, q, sf);
  return hipGetLastError();
}

hipError_t launch_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t stride, int mode,
                           int64_t group_rows, float fixed, uint8_t* q, uint8_t* sf, float* dec,
                           void* ws, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  dim3 grid((unsigned)rows), block(kQuantThreads);
  if (mode == 0) {
    KernelTimer t("quantize_rows", s);
    hipLaunchKernelGGL(quantize_rows_kernel<0>, grid, block, 0, s, x, cols, stride, group_rows,
                       fixed, nullptr, q, sf, dec);
  } else if (mode == 1) {
    uint32_t* gmax = static_cast<uint32_t*>(ws);
    int64_t ng = rows / group_rows;
    {
      KernelTimer t("fill_u32", s);
      hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)((ng + 255) / 256)), dim3(256), 0, s,
                         gmax, ng, 0u);
    }
    {
      KernelTimer t("group_amax", s);
      hipLaunchKernelGGL(group_amax_kernel, grid, block, 0, s, x, cols, stride, group_rows, gmax);
    }
    KernelTimer t("quantize_rows_group", s);
    hipLaunchKernelGGL(quantize_rows_kernel<1>, grid, block, 0, s, x, cols, stride, group_rows,
                       fixed, gmax, q, sf, dec);
  } else {
    KernelTimer t("quantize_rows_fixed", s);
    hipLaunchKernelGGL(quantize_rows_kernel<2>, grid, block, 0, s, x, cols, stride, group_rows,
                       fixed, nullptr, q, sf, dec);
  }
  return hipGetLastError();
}

hipError_t launch_unpack_routing(const int32_t* packed, int64_t n, int32_t* ids,
                                uint16_t* weights, hipStream_t s) {
  if (n == 0) return hipSuccess;
  KernelTimer t("unpack_routing", s);
  hipLaunchKernelGGL(unpack_routing_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     packed, n, ids, weights);
  return hipGetLastError();
}

hipError_t launch_permute(const uint8_t* q, const uint8_t* sf, const float* dec, int64_t M,
                          int64_t H, int top_k, const int32_t* sorted, const int32_t* ntpp,
                          int64_t cap, uint8_t* qp, uint8_t* sp, float* spd, hipStream_t s) {
  if (cap == 0) return hipSuccess;
  KernelTimer t("permute", s);
  hipLaunchKernelGGL(permute_kernel, dim3((unsigned)cap), dim3(64), 0, s, q, sf, dec, M, H, top_k,
                     sorted, ntpp, qp, sp, spd);
  return hipGetLastError();
}

hipError_t launch_finalize(const uint16_t* y, const void* w, bool w_bf16, const int32_t* ttr,
                           int64_t M, int64_t H, int top_k, float rsf, uint16_t* out,
                           hipStream_t s) {
  int64_t n = M * (H >> 3);
  if (n == 0) return hipSuccess;
  KernelTimer t("finalize", s);
  const dim3 grid((unsigned)((n + 255) / 256));
  if (w_bf16)
    hipLaunchKernelGGL(finalize_kernel<true>, grid, dim3(256), 0, s, y, w, ttr, M, H, top_k, rsf,
                       out);
  else
    hipLaunchKernelGGL(finalize_kernel<false>, grid, dim3(256), 0, s, y, w, ttr, M, H, top_k, rsf,
                       out);
  return hipGetLastError();
}

}  // namespace bfp4
