"""Python binding of the bfp4moe C ABI (include/bfp4moe.h): argument marshalling only.

Every function has the name of its C entry point and takes the same arguments in the same
order.  Device buffers may be passed as torch tensors (their data pointer is used) or as integer
addresses; ``stream`` defaults to torch's current HIP stream.  A non-zero status raises
``Bfp4Error``.  All computation happens in the HIP library; if it is not built, importing this
package fails.
"""

import ctypes
import os

import torch  # loads the HIP runtime first, so the library binds to the same one

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbfp4moe.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        "libbfp4moe.so is not built; run `python block_scaled_fp4_plan_amd/build.py` "
        "(or __graft_entry__.build())")

_lib = ctypes.CDLL(LIB_PATH)

BFP4_ACT_SWIGLU = 0
BFP4_ACT_RELU2 = 1
BFP4_ACT_GEGLU = 2
BFP4_ACT_GELU = 3
BFP4_ACT_RELU = 4
BFP4_ACT_SILU = 5
BFP4_ACT_IDENTITY = 6
GATED_ACTS = (BFP4_ACT_SWIGLU, BFP4_ACT_GEGLU)
BFP4_SCALE_PER_ROW = 0
BFP4_SCALE_PER_GROUP = 1
BFP4_SCALE_FIXED = 2
BFP4_WEIGHTS_F32 = 0
BFP4_WEIGHTS_BF16 = 1
BFP4_FORMAT_NVFP4 = 0
BFP4_FORMAT_MXFP4 = 1

STATUS = {
    0: "BFP4_OK", -1: "BFP4_ERR_NULL", -2: "BFP4_ERR_SHAPE", -3: "BFP4_ERR_ALIGN",
    -4: "BFP4_ERR_BLOCK_M", -5: "BFP4_ERR_CAPACITY", -6: "BFP4_ERR_WORKSPACE",
    -7: "BFP4_ERR_OVERLAP", -8: "BFP4_ERR_EXPERTS", -9: "BFP4_ERR_MODE", -10: "BFP4_ERR_SCALAR",
    -11: "BFP4_ERR_DEVICE", -12: "BFP4_ERR_LAUNCH",
}
EXPORTS = [
    "bfp4_status_string", "bfp4_version", "bfp4_plan_capacity", "bfp4_plan_workspace_size",
    "bfp4_moe_plan", "bfp4_quantize_workspace_size", "bfp4_quantize_nvfp4", "bfp4_moe_permute",
    "bfp4_panel_bytes", "bfp4_prepare_weights", "bfp4_workspace_size", "bfp4_fused_moe_nvfp4",
    "bfp4_moe_finalize", "bfp4_profile_begin", "bfp4_profile_end", "bfp4_workspace_size_w4a16",
    "bfp4_fused_moe_w4a16", "bfp4_quantize_mxfp4", "bfp4_prepare_weights_mxfp4",
    "bfp4_check_topk_ids", "bfp4_check_plan", "bfp4_fused_moe_nvfp4_noalloc",
    "bfp4_moe_plan_quantize", "bfp4_quantize_mxfp8", "bfp4_workspace_size_mx", "bfp4_fused_moe_mx",
    "bfp4_unpack_routing", "bfp4_xor_checksum",
]
XOR_PARTIALS = 16384                      # BFP4_XOR_PARTIALS
NOALLOC_SCRATCH_BYTES = 64 << 20          # BFP4_NOALLOC_SCRATCH_BYTES


class Bfp4Error(RuntimeError):
    def __init__(self, status, fn):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (fn, STATUS.get(status, status),
                                                 _lib.bfp4_status_string(status).decode()))


class bfp4_debug(ctypes.Structure):
    _fields_ = [("preact", ctypes.c_void_p), ("inter", ctypes.c_void_p),
                ("inter_q", ctypes.c_void_p), ("inter_sf", ctypes.c_void_p),
                ("inter_f16", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_F = ctypes.c_float
_SZ = ctypes.c_size_t


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_sig("bfp4_status_string", ctypes.c_char_p, [_I])
_sig("bfp4_version", ctypes.c_char_p, [])
_sig("bfp4_plan_capacity", _SZ, [_I64, _I, _I, _I])
_sig("bfp4_plan_workspace_size", _SZ, [_I64, _I, _I])
_sig("bfp4_moe_plan", _I, [_P, _I64, _I, _I, _I, _I, _I, _P, _P, _P, _P, _SZ, _P, _SZ, _P])
_sig("bfp4_quantize_workspace_size", _SZ, [_I64, _I, _I64])
_sig("bfp4_quantize_nvfp4", _I, [_P, _I64, _I64, _I64, _I, _I64, _F, _P, _P, _P, _P, _SZ, _P])
_sig("bfp4_moe_plan_quantize", _I, [_P, _I64, _I, _I, _I, _I, _I, _P, _P, _P, _P, _SZ, _P, _SZ,
                                    _P, _I64, _I64, _P, _P, _P, _P])
_sig("bfp4_moe_permute", _I, [_P, _P, _P, _I64, _I64, _I, _P, _P, _SZ, _P, _P, _P, _P])
_sig("bfp4_panel_bytes", _SZ, [_I, _I64, _I64, _I])
_sig("bfp4_prepare_weights", _I, [_P, _P, _P, _P, _I, _I64, _I64, _I, _P, _SZ, _P])
_sig("bfp4_workspace_size", _SZ, [_I64, _I64, _I64, _I, _I, _I, _I])
_sig("bfp4_fused_moe_nvfp4", _I,
     [_P, _P, _P, _P, _SZ, _P, _P, _P, _F, _P, _P, _P, _P, _SZ, _P, _I, _I64, _I64, _I64, _I, _I,
      _I, _I, _F, _I, _P, _P, ctypes.POINTER(bfp4_debug), _P, _SZ, _P])
_sig("bfp4_fused_moe_nvfp4_noalloc", _I,
     [_P, _P, _P, _P, _SZ, _P, _P, _P, _F, _P, _P, _P, _P, _SZ, _P, _I, _I64, _I64, _I64, _I, _I,
      _I, _I, _F, _I, _P, _P, ctypes.POINTER(bfp4_debug), _P])
_sig("bfp4_moe_finalize", _I, [_P, _P, _I, _P, _I64, _I64, _I, _F, _P, _P])
_sig("bfp4_workspace_size_w4a16", _SZ, [_I64, _I64, _I64, _I, _I, _I, _I])
_sig("bfp4_fused_moe_w4a16", _I,
     [_P, _I64, _P, _SZ, _I, _P, _P, _P, _P, _P, _P, _P, _SZ, _P, _I, _I64, _I64, _I64, _I, _I,
      _I, _I, _F, _I, _P, _P, ctypes.POINTER(bfp4_debug), _P, _SZ, _P])
_sig("bfp4_quantize_mxfp4", _I, [_P, _I64, _I64, _I64, _P, _P, _P])
_sig("bfp4_quantize_mxfp8", _I, [_P, _I64, _I64, _I64, _P, _P, _P])
_sig("bfp4_workspace_size_mx", _SZ, [_I64, _I64, _I64, _I, _I, _I, _I])
_sig("bfp4_fused_moe_mx", _I,
     [_P, _P, _P, _SZ, _P, _P, _P, _P, _SZ, _P, _I, _I64, _I64, _I64, _I, _I, _I, _I, _F, _I, _P,
      _P, ctypes.POINTER(bfp4_debug), _P, _SZ, _P])
_sig("bfp4_prepare_weights_mxfp4", _I, [_P, _P, _P, _P, _I, _I64, _I64, _I, _P, _SZ, _P])
_sig("bfp4_unpack_routing", _I, [_P, _I64, _I, _P, _P, _P])
_sig("bfp4_xor_checksum", _I, [_P, _SZ, _P, _P])
_sig("bfp4_check_topk_ids", _I, [_P, _I64, _I, _I, _P, _P])
_sig("bfp4_check_plan", _I, [_P, _P, _P, _SZ, _I64, _I, _I, _I, _P, _P])
_sig("bfp4_profile_begin", _I, [_I, ctypes.c_char_p])
_sig("bfp4_profile_end", _I, [ctypes.c_char_p, _SZ])


def _p(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.data_ptr()
    return int(x)


def _s(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(st, fn):
    if st != 0:
        raise Bfp4Error(st, fn)
    return st


def bfp4_status_string(status):
    return _lib.bfp4_status_string(status).decode()


def bfp4_version():
    return _lib.bfp4_version().decode()


def bfp4_plan_capacity(M, top_k, num_local_experts, block_m):
    return _lib.bfp4_plan_capacity(M, top_k, num_local_experts, block_m)


def bfp4_plan_workspace_size(M, top_k, num_local_experts):
    return _lib.bfp4_plan_workspace_size(M, top_k, num_local_experts)


def bfp4_moe_plan(topk_ids, M, top_k, num_experts, local_expert_offset, num_local_experts,
                  block_m, sorted_token_ids, expert_ids, num_tokens_post_padded, token_to_row,
                  capacity, workspace=None, workspace_bytes=0, stream=None):
    return _check(_lib.bfp4_moe_plan(
        _p(topk_ids), M, top_k, num_experts, local_expert_offset, num_local_experts, block_m,
        _p(sorted_token_ids), _p(expert_ids), _p(num_tokens_post_padded), _p(token_to_row),
        capacity, _p(workspace), workspace_bytes, _s(stream)), "bfp4_moe_plan")


def bfp4_quantize_workspace_size(rows, mode, group_rows):
    return _lib.bfp4_quantize_workspace_size(rows, mode, group_rows)


def bfp4_quantize_nvfp4(x_bf16, rows, cols, row_stride, mode, group_rows, fixed_encode_scale, q,
                        sf, dec_scale, workspace=None, workspace_bytes=0, stream=None):
    return _check(_lib.bfp4_quantize_nvfp4(
        _p(x_bf16), rows, cols, row_stride, mode, group_rows, fixed_encode_scale, _p(q), _p(sf),
        _p(dec_scale), _p(workspace), workspace_bytes, _s(stream)), "bfp4_quantize_nvfp4")


def bfp4_moe_plan_quantize(topk_ids, M, top_k, num_experts, local_expert_offset,
                           num_local_experts, block_m, sorted_token_ids, expert_ids,
                           num_tokens_post_padded, token_to_row, capacity, plan_workspace,
                           plan_workspace_bytes, x_bf16, H, row_stride, q, sf, dec_scale,
                           stream=None):
    return _check(_lib.bfp4_moe_plan_quantize(
        _p(topk_ids), M, top_k, num_experts, local_expert_offset, num_local_experts, block_m,
        _p(sorted_token_ids), _p(expert_ids), _p(num_tokens_post_padded), _p(token_to_row),
        capacity, _p(plan_workspace), plan_workspace_bytes, _p(x_bf16), H, row_stride, _p(q),
        _p(sf), _p(dec_scale), _s(stream)), "bfp4_moe_plan_quantize")


def bfp4_moe_permute(q, sf, dec_scale, M, H, top_k, sorted_token_ids, num_tokens_post_padded,
                     capacity, q_perm, sf_perm, s_perm, stream=None):
    return _check(_lib.bfp4_moe_permute(
        _p(q), _p(sf), _p(dec_scale), M, H, top_k, _p(sorted_token_ids),
        _p(num_tokens_post_padded), capacity, _p(q_perm), _p(sf_perm), _p(s_perm), _s(stream)),
        "bfp4_moe_permute")


def bfp4_panel_bytes(num_local_experts, H, I, gated):
    return _lib.bfp4_panel_bytes(num_local_experts, H, I, gated)


def bfp4_prepare_weights(w1_q, w1_sf, w2_q, w2_sf, num_local_experts, H, I, gated, panels,
                         panels_bytes, stream=None):
    return _check(_lib.bfp4_prepare_weights(
        _p(w1_q), _p(w1_sf), _p(w2_q), _p(w2_sf), num_local_experts, H, I, gated, _p(panels),
        panels_bytes, _s(stream)), "bfp4_prepare_weights")


def bfp4_workspace_size(M, H, I, top_k, num_local_experts, block_m, do_finalize):
    return _lib.bfp4_workspace_size(M, H, I, top_k, num_local_experts, block_m, do_finalize)


def bfp4_fused_moe_nvfp4(a_q, a_sf, a_dec, panels, panels_bytes, alpha1_gate, alpha1_up, alpha2,
                         c2, sorted_token_ids, expert_ids, num_tokens_post_padded, token_to_row,
                         capacity, topk_weights, weights_dtype, M, H, I, num_local_experts, top_k,
                         block_m, act, routed_scaling_factor, do_finalize, out, gemm2_out, debug,
                         workspace, workspace_bytes, stream=None):
    dbg = None
    if debug is not None:
        dbg = ctypes.byref(bfp4_debug(*(_p(debug.get(k)) for k in
                                        ("preact", "inter", "inter_q", "inter_sf",
                                         "inter_f16"))))
    return _check(_lib.bfp4_fused_moe_nvfp4(
        _p(a_q), _p(a_sf), _p(a_dec), _p(panels), panels_bytes, _p(alpha1_gate), _p(alpha1_up),
        _p(alpha2), c2, _p(sorted_token_ids), _p(expert_ids), _p(num_tokens_post_padded),
        _p(token_to_row), capacity, _p(topk_weights), weights_dtype, M, H, I, num_local_experts,
        top_k, block_m,
        act, routed_scaling_factor, do_finalize, _p(out), _p(gemm2_out), dbg, _p(workspace),
        workspace_bytes, _s(stream)), "bfp4_fused_moe_nvfp4")


def bfp4_fused_moe_nvfp4_noalloc(a_q, a_sf, a_dec, panels, panels_bytes, alpha1_gate, alpha1_up,
                                 alpha2, c2, sorted_token_ids, expert_ids,
                                 num_tokens_post_padded, token_to_row, capacity, topk_weights,
                                 weights_dtype, M, H, I, num_local_experts, top_k, block_m, act,
                                 routed_scaling_factor, do_finalize, out, gemm2_out, debug,
                                 stream=None):
    dbg = None
    if debug is not None:
        dbg = ctypes.byref(bfp4_debug(*(_p(debug.get(k)) for k in
                                        ("preact", "inter", "inter_q", "inter_sf",
                                         "inter_f16"))))
    return _check(_lib.bfp4_fused_moe_nvfp4_noalloc(
        _p(a_q), _p(a_sf), _p(a_dec), _p(panels), panels_bytes, _p(alpha1_gate), _p(alpha1_up),
        _p(alpha2), c2, _p(sorted_token_ids), _p(expert_ids), _p(num_tokens_post_padded),
        _p(token_to_row), capacity, _p(topk_weights), weights_dtype, M, H, I, num_local_experts,
        top_k, block_m, act, routed_scaling_factor, do_finalize, _p(out), _p(gemm2_out), dbg,
        _s(stream)), "bfp4_fused_moe_nvfp4_noalloc")


def bfp4_workspace_size_w4a16(M, H, I, top_k, num_local_experts, block_m, do_finalize):
    return _lib.bfp4_workspace_size_w4a16(M, H, I, top_k, num_local_experts, block_m, do_finalize)


def bfp4_quantize_mxfp4(x_bf16, rows, cols, row_stride, q, sf, stream=None):
    return _check(_lib.bfp4_quantize_mxfp4(_p(x_bf16), rows, cols, row_stride, _p(q), _p(sf),
                                           _s(stream)), "bfp4_quantize_mxfp4")


def bfp4_quantize_mxfp8(x_bf16, rows, cols, row_stride, q, sf, stream=None):
    return _check(_lib.bfp4_quantize_mxfp8(_p(x_bf16), rows, cols, row_stride, _p(q), _p(sf),
                                           _s(stream)), "bfp4_quantize_mxfp8")


def bfp4_workspace_size_mx(M, H, I, top_k, num_local_experts, block_m, do_finalize):
    return _lib.bfp4_workspace_size_mx(M, H, I, top_k, num_local_experts, block_m, do_finalize)


def bfp4_fused_moe_mx(a_q, a_sf, panels, panels_bytes, sorted_token_ids, expert_ids,
                      num_tokens_post_padded, token_to_row, capacity, topk_weights, weights_dtype,
                      M, H, I, num_local_experts, top_k, block_m, act, routed_scaling_factor,
                      do_finalize, out, gemm2_out, debug, workspace, workspace_bytes,
                      stream=None):
    dbg = None
    if debug is not None:
        dbg = ctypes.byref(bfp4_debug(*(_p(debug.get(k)) for k in
                                        ("preact", "inter", "inter_q", "inter_sf",
                                         "inter_f16"))))
    return _check(_lib.bfp4_fused_moe_mx(
        _p(a_q), _p(a_sf), _p(panels), panels_bytes, _p(sorted_token_ids), _p(expert_ids),
        _p(num_tokens_post_padded), _p(token_to_row), capacity, _p(topk_weights), weights_dtype,
        M, H, I, num_local_experts, top_k, block_m, act, routed_scaling_factor, do_finalize,
        _p(out), _p(gemm2_out), dbg, _p(workspace), workspace_bytes, _s(stream)),
        "bfp4_fused_moe_mx")


def bfp4_prepare_weights_mxfp4(w1_q, w1_sf, w2_q, w2_sf, num_local_experts, H, I, gated, panels,
                               panels_bytes, stream=None):
    return _check(_lib.bfp4_prepare_weights_mxfp4(
        _p(w1_q), _p(w1_sf), _p(w2_q), _p(w2_sf), num_local_experts, H, I, gated, _p(panels),
        panels_bytes, _s(stream)), "bfp4_prepare_weights_mxfp4")


def bfp4_fused_moe_w4a16(x_bf16, row_stride, panels, panels_bytes, weight_format, alpha1_gate,
                         alpha1_up, alpha2, sorted_token_ids, expert_ids, num_tokens_post_padded,
                         token_to_row, capacity, topk_weights, weights_dtype, M, H, I,
                         num_local_experts, top_k, block_m, act, routed_scaling_factor,
                         do_finalize, out, gemm2_out, debug, workspace, workspace_bytes,
                         stream=None):
    dbg = None
    if debug is not None:
        dbg = ctypes.byref(bfp4_debug(*(_p(debug.get(k)) for k in
                                        ("preact", "inter", "inter_q", "inter_sf",
                                         "inter_f16"))))
    return _check(_lib.bfp4_fused_moe_w4a16(
        _p(x_bf16), row_stride, _p(panels), panels_bytes, weight_format, _p(alpha1_gate),
        _p(alpha1_up),
        _p(alpha2), _p(sorted_token_ids), _p(expert_ids), _p(num_tokens_post_padded),
        _p(token_to_row), capacity, _p(topk_weights), weights_dtype, M, H, I, num_local_experts,
        top_k, block_m, act, routed_scaling_factor, do_finalize, _p(out), _p(gemm2_out), dbg,
        _p(workspace), workspace_bytes, _s(stream)), "bfp4_fused_moe_w4a16")


def bfp4_moe_finalize(gemm2_out, topk_weights, weights_dtype, token_to_row, M, H, top_k,
                      routed_scaling_factor, out, stream=None):
    return _check(_lib.bfp4_moe_finalize(
        _p(gemm2_out), _p(topk_weights), weights_dtype, _p(token_to_row), M, H, top_k,
        routed_scaling_factor, _p(out), _s(stream)), "bfp4_moe_finalize")


def bfp4_unpack_routing(packed, M, top_k, topk_ids, topk_weights, stream=None):
    return _check(_lib.bfp4_unpack_routing(_p(packed), M, top_k, _p(topk_ids), _p(topk_weights),
                                           _s(stream)), "bfp4_unpack_routing")


def bfp4_xor_checksum(buf, nbytes, partial, stream=None):
    return _check(_lib.bfp4_xor_checksum(_p(buf), nbytes, _p(partial), _s(stream)),
                  "bfp4_xor_checksum")


def bfp4_check_topk_ids(topk_ids, M, top_k, num_experts, report, stream=None):
    return _check(_lib.bfp4_check_topk_ids(_p(topk_ids), M, top_k, num_experts, _p(report),
                                           _s(stream)), "bfp4_check_topk_ids")


def bfp4_check_plan(sorted_token_ids, expert_ids, num_tokens_post_padded, capacity, M, top_k,
                    num_local_experts, block_m, report, stream=None):
    return _check(_lib.bfp4_check_plan(
        _p(sorted_token_ids), _p(expert_ids), _p(num_tokens_post_padded), capacity, M, top_k,
        num_local_experts, block_m, _p(report), _s(stream)), "bfp4_check_plan")


def bfp4_profile_begin(capacity, name_prefix=None):
    pre = name_prefix.encode() if name_prefix else None
    return _check(_lib.bfp4_profile_begin(capacity, pre), "bfp4_profile_begin")


def bfp4_profile_end():
    """Returns (kernels launched while recording, {name: (count, total_ms)})."""
    buf = ctypes.create_string_buffer(1 << 16)
    n = _lib.bfp4_profile_end(buf, len(buf))
    if n < 0:
        raise Bfp4Error(n, "bfp4_profile_end")
    table = {}
    for line in buf.value.decode().splitlines():
        name, cnt, ms = line.split()
        table[name] = (int(cnt), float(ms))
    return n, table
