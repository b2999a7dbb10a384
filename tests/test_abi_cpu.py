"""The C-ABI library loads, exports every function declared in include/bfp4moe.h, and rejects
invalid arguments on the host (no GPU needed: validation reads no device memory, and valid
arguments without a gfx950 device give BFP4_ERR_DEVICE before anything is launched)."""

import ctypes
import os
import re

import pytest
import torch

import block_scaled_fp4_plan_amd as bf
from block_scaled_fp4_plan_amd import Bfp4Error

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bfp4moe.h")

NO_GPU = not torch.cuda.is_available()
cpu_only = pytest.mark.skipif(not NO_GPU, reason="checks the no-device error path")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bfp4_\w+)\s*\(", text)))


def test_header_and_binding_agree():
    names = declared_functions()
    assert "bfp4_fused_moe_nvfp4" in names and "bfp4_moe_plan" in names
    assert sorted(bf.EXPORTS) == names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(bf.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_status_strings_and_sizes():
    assert bf.bfp4_status_string(0) == "ok"
    assert "block_m" in bf.bfp4_status_string(-4)
    assert bf.bfp4_version().startswith("bfp4moe")
    # capacity = round_up(M*k + min(E, M*k) * (block_m - 1), block_m)
    assert bf.bfp4_plan_capacity(16, 2, 8, 8) == 32 + 8 * 7 == 88
    assert bf.bfp4_plan_capacity(16, 2, 8, 128) == 1152
    assert bf.bfp4_plan_capacity(4096, 8, 256, 128) == 65280
    assert bf.bfp4_plan_capacity(8, 8, 256, 8) == 64 + 64 * 7
    assert bf.bfp4_plan_capacity(16, 2, 8, 12) == 0            # invalid block_m
    # panel bytes: per 32-row group, 1 KiB per 64 K values + 1 KiB per 512 K values
    assert bf.bfp4_panel_bytes(1, 256, 128, 1) == (8 * (4 + 1) + 8 * (2 + 1)) * 1024
    assert bf.bfp4_panel_bytes(2, 7168, 2048, 1) == 2 * (128 * (112 + 14) + 224 * (32 + 4)) * 1024
    assert bf.bfp4_panel_bytes(1, 250, 128, 1) == 0
    # hq [88, 64] + hsf [88, 8] + tile list [11 x 8 B + 16] (each rounded up to 256 B)
    # + y [88, 256] BF16
    # hq | hsf | tile list (11 tiles x 24 bytes + 16) | y, each rounded up to 256 bytes
    assert bf.bfp4_workspace_size(16, 256, 128, 2, 8, 8, 1) == 5632 + 768 + 512 + 88 * 512
    assert bf.bfp4_quantize_workspace_size(64, bf.BFP4_SCALE_PER_GROUP, 16) == 16


A = 1 << 20   # a fake, 256-byte aligned "device" address: never dereferenced on the host


def _plan(**kw):
    args = dict(topk_ids=A, M=16, top_k=2, num_experts=8, local_expert_offset=0,
                num_local_experts=8, block_m=8, sorted_token_ids=A + 4096, expert_ids=A + 8192,
                num_tokens_post_padded=A + 12288, token_to_row=A + 16384, capacity=88,
                workspace=None, workspace_bytes=0, stream=0)
    args.update(kw)
    with pytest.raises(Bfp4Error) as ei:
        bf.bfp4_moe_plan(**args)
    return bf.STATUS[ei.value.status]


def test_plan_validation():
    assert _plan(block_m=12) == "BFP4_ERR_BLOCK_M"
    assert _plan(block_m=4) == "BFP4_ERR_BLOCK_M"
    assert _plan(capacity=80) == "BFP4_ERR_CAPACITY"
    assert _plan(capacity=92) == "BFP4_ERR_CAPACITY"          # not a multiple of block_m
    assert _plan(local_expert_offset=4, num_local_experts=8) == "BFP4_ERR_EXPERTS"
    assert _plan(num_local_experts=2000, num_experts=4000) == "BFP4_ERR_EXPERTS"
    assert _plan(topk_ids=None) == "BFP4_ERR_NULL"
    assert _plan(token_to_row=A + 2) == "BFP4_ERR_ALIGN"
    assert _plan(M=-1) == "BFP4_ERR_SHAPE"
    assert _plan(M=4096, top_k=8, capacity=65280 * 8 // 128 * 16, num_experts=256,
                 num_local_experts=256, block_m=8, workspace=None) in ("BFP4_ERR_WORKSPACE",
                                                                        "BFP4_ERR_CAPACITY")


@cpu_only
def test_plan_valid_args_without_device():
    assert _plan() == "BFP4_ERR_DEVICE"


def _quant(**kw):
    args = dict(x_bf16=A, rows=4, cols=256, row_stride=256, mode=0, group_rows=0,
                fixed_encode_scale=1.0, q=A + (1 << 16), sf=A + (2 << 16), dec_scale=A + (3 << 16),
                workspace=None, workspace_bytes=0, stream=0)
    args.update(kw)
    with pytest.raises(Bfp4Error) as ei:
        bf.bfp4_quantize_nvfp4(**args)
    return bf.STATUS[ei.value.status]


def test_quantize_validation():
    assert _quant(cols=48) == "BFP4_ERR_SHAPE"
    assert _quant(row_stride=200) == "BFP4_ERR_SHAPE"
    assert _quant(row_stride=260) == "BFP4_ERR_SHAPE"
    assert _quant(mode=7) == "BFP4_ERR_MODE"
    assert _quant(mode=2, fixed_encode_scale=float("inf")) == "BFP4_ERR_SCALAR"
    assert _quant(mode=2, fixed_encode_scale=0.0) == "BFP4_ERR_SCALAR"
    assert _quant(mode=1, group_rows=3) == "BFP4_ERR_SHAPE"
    assert _quant(mode=1, group_rows=2) == "BFP4_ERR_WORKSPACE"
    assert _quant(x_bf16=A + 8) == "BFP4_ERR_ALIGN"
    assert _quant(q=None) == "BFP4_ERR_NULL"
    assert _quant(q=A + 16) == "BFP4_ERR_OVERLAP"


@cpu_only
def test_quantize_valid_args_without_device():
    assert _quant() == "BFP4_ERR_DEVICE"


def _fused(**kw):
    args = dict(a_q=A, a_sf=A + (1 << 16), a_dec=A + (2 << 16), panels=A + (3 << 16),
                panels_bytes=bf.bfp4_panel_bytes(8, 256, 128, 1), alpha1_gate=A + (40 << 16),
                alpha1_up=A + (41 << 16), alpha2=A + (42 << 16), c2=1.0,
                sorted_token_ids=A + (43 << 16), expert_ids=A + (44 << 16),
                num_tokens_post_padded=A + (45 << 16), token_to_row=A + (46 << 16), capacity=88,
                topk_weights=A + (47 << 16), weights_dtype=0, M=16, H=256, I=128, num_local_experts=8, top_k=2,
                block_m=8, act=0, routed_scaling_factor=1.0, do_finalize=1, out=A + (48 << 16),
                gemm2_out=None, debug=None, workspace=A + (50 << 16),
                workspace_bytes=bf.bfp4_workspace_size(16, 256, 128, 2, 8, 8, 1), stream=0)
    args.update(kw)
    with pytest.raises(Bfp4Error) as ei:
        bf.bfp4_fused_moe_nvfp4(**args)
    return bf.STATUS[ei.value.status]


def test_fused_validation():
    assert _fused(H=200) == "BFP4_ERR_SHAPE"
    assert _fused(H=128) == "BFP4_ERR_SHAPE"                   # H >= 256 and % 256
    assert _fused(I=96) == "BFP4_ERR_SHAPE"                    # I % 128
    assert _fused(block_m=9) == "BFP4_ERR_BLOCK_M"
    assert _fused(act=7) == "BFP4_ERR_MODE"
    assert _fused(weights_dtype=2) == "BFP4_ERR_MODE"
    assert _fused(topk_weights=A + (47 << 16) + 2) == "BFP4_ERR_ALIGN"      # FP32 needs 4 bytes
    assert _fused(act=-1) == "BFP4_ERR_MODE"
    # a gated activation (GeGLU) needs the larger, gated panels
    assert _fused(act=2, panels_bytes=bf.bfp4_panel_bytes(8, 256, 128, 0)) == "BFP4_ERR_WORKSPACE"
    assert _fused(c2=0.0) == "BFP4_ERR_SCALAR"
    assert _fused(routed_scaling_factor=float("nan")) == "BFP4_ERR_SCALAR"
    assert _fused(capacity=80) == "BFP4_ERR_CAPACITY"
    assert _fused(panels_bytes=1024) == "BFP4_ERR_WORKSPACE"
    assert _fused(workspace_bytes=100) == "BFP4_ERR_WORKSPACE"
    assert _fused(a_q=A + 4) == "BFP4_ERR_ALIGN"
    assert _fused(out=A + 8) == "BFP4_ERR_ALIGN"
    assert _fused(a_dec=None) == "BFP4_ERR_NULL"
    assert _fused(do_finalize=0) == "BFP4_ERR_NULL"            # gemm2_out required
    assert _fused(out=A + (1 << 16) + 64) == "BFP4_ERR_OVERLAP"  # out over a_sf
    assert _fused(out=A + (50 << 16) + 512) == "BFP4_ERR_OVERLAP"  # out over workspace
    # unfinalized: gemm2_out [capacity, H] BF16 (88 x 512 bytes) must not reach an input either
    assert _fused(do_finalize=0, gemm2_out=A + (46 << 16) - 88 * 512 + 16) == "BFP4_ERR_OVERLAP"
    assert _fused(do_finalize=0, gemm2_out=A + (50 << 16) + 256) == "BFP4_ERR_OVERLAP"
    assert _fused(num_local_experts=0) == "BFP4_ERR_EXPERTS"
    # decode kernels (block_m <= 32) stage a block's rows whole in LDS: H <= 8960 at block_m 32
    assert _fused(H=9216, block_m=32, capacity=bf.bfp4_plan_capacity(16, 2, 8, 32),
                  panels_bytes=bf.bfp4_panel_bytes(8, 9216, 128, 1)) == "BFP4_ERR_SHAPE"
    # tiled kernels (block_m > 32) read FP16 token copies with 32-bit offsets: M*H*2 < 2^31
    assert _fused(M=1 << 24, top_k=1, block_m=128) == "BFP4_ERR_SHAPE"


@cpu_only
def test_fused_valid_args_without_device():
    assert _fused() == "BFP4_ERR_DEVICE"
    for act in range(7):                         # every activation code is accepted
        nb = bf.bfp4_panel_bytes(8, 256, 128, int(act in bf.GATED_ACTS))
        assert _fused(act=act, panels_bytes=nb) == "BFP4_ERR_DEVICE"
    # the largest decode-kernel shape at block_m 32 passes validation
    assert _fused(H=8960, block_m=32, capacity=bf.bfp4_plan_capacity(16, 2, 8, 32),
                  panels_bytes=bf.bfp4_panel_bytes(8, 8960, 128, 1),
                  workspace_bytes=bf.bfp4_workspace_size(16, 8960, 128, 2, 8, 32, 1),
                  out=1 << 40) == "BFP4_ERR_DEVICE"
    # BF16 routing weights need 2-byte alignment only
    assert _fused(weights_dtype=1, topk_weights=A + (47 << 16) + 2) == "BFP4_ERR_DEVICE"
    # unfinalized: gemm2_out ending right where token_to_row starts is accepted
    assert _fused(do_finalize=0, gemm2_out=A + (46 << 16) - 88 * 512) == "BFP4_ERR_DEVICE"


def test_finalize_and_prepare_validation():
    with pytest.raises(Bfp4Error) as ei:
        bf.bfp4_moe_finalize(A, A + 4096, 0, A + 8192, 4, 12, 2, 1.0, A + (1 << 16), 0)
    assert bf.STATUS[ei.value.status] == "BFP4_ERR_SHAPE"
    with pytest.raises(Bfp4Error) as ei:
        bf.bfp4_moe_finalize(A, A + 4096, 0, A + 8192, 4, 256, 2, 1.0, A + 4096, 0)
    assert bf.STATUS[ei.value.status] == "BFP4_ERR_OVERLAP"
    with pytest.raises(Bfp4Error) as ei:                       # unknown routing-weight dtype
        bf.bfp4_moe_finalize(A, A + 4096, 3, A + 8192, 4, 256, 2, 1.0, A + (1 << 16), 0)
    assert bf.STATUS[ei.value.status] == "BFP4_ERR_MODE"
    with pytest.raises(Bfp4Error) as ei:                       # FP32 weights 2-byte aligned
        bf.bfp4_moe_finalize(A, A + 4098, 0, A + 8192, 4, 256, 2, 1.0, A + (1 << 16), 0)
    assert bf.STATUS[ei.value.status] == "BFP4_ERR_ALIGN"
    with pytest.raises(Bfp4Error) as ei:
        bf.bfp4_prepare_weights(A, A, A, A, 1, 256, 100, 1, A, 1 << 20, 0)
    assert bf.STATUS[ei.value.status] == "BFP4_ERR_SHAPE"
    with pytest.raises(Bfp4Error) as ei:
        bf.bfp4_prepare_weights(A, A, A, A, 1, 256, 128, 1, A, 100, 0)
    assert bf.STATUS[ei.value.status] == "BFP4_ERR_WORKSPACE"
    with pytest.raises(Bfp4Error) as ei:
        bf.bfp4_moe_permute(A, A, A, 4, 48, 2, A, A, 16, A, A, A, 0)
    assert bf.STATUS[ei.value.status] == "BFP4_ERR_SHAPE"


def _w16(**kw):
    args = dict(x_bf16=A, row_stride=256, panels=A + (3 << 16),
                panels_bytes=bf.bfp4_panel_bytes(8, 256, 128, 1), weight_format=0,
                alpha1_gate=A + (40 << 16),
                alpha1_up=A + (41 << 16), alpha2=A + (42 << 16), sorted_token_ids=A + (43 << 16),
                expert_ids=A + (44 << 16), num_tokens_post_padded=A + (45 << 16),
                token_to_row=A + (46 << 16), capacity=88, topk_weights=A + (47 << 16),
                weights_dtype=0, M=16, H=256, I=128, num_local_experts=8, top_k=2, block_m=8,
                act=0, routed_scaling_factor=1.0, do_finalize=1, out=A + (48 << 16),
                gemm2_out=None, debug=None, workspace=A + (50 << 16),
                workspace_bytes=bf.bfp4_workspace_size_w4a16(16, 256, 128, 2, 8, 8, 1), stream=0)
    args.update(kw)
    with pytest.raises(Bfp4Error) as ei:
        bf.bfp4_fused_moe_w4a16(**args)
    return bf.STATUS[ei.value.status]


def test_w4a16_validation():
    # hq [88, 128] BF16 intermediate + y [88, 256] BF16, each rounded up to 256 bytes
    assert bf.bfp4_workspace_size_w4a16(16, 256, 128, 2, 8, 8, 1) == 88 * 256 + 88 * 512
    assert _w16(block_m=128, capacity=bf.bfp4_plan_capacity(16, 2, 8, 128)) == "BFP4_ERR_BLOCK_M"
    assert _w16(row_stride=200) == "BFP4_ERR_SHAPE"
    assert _w16(row_stride=260) == "BFP4_ERR_SHAPE"
    assert _w16(H=200) == "BFP4_ERR_SHAPE"
    assert _w16(act=9) == "BFP4_ERR_MODE"
    assert _w16(weights_dtype=5) == "BFP4_ERR_MODE"
    assert _w16(x_bf16=A + 8) == "BFP4_ERR_ALIGN"
    assert _w16(x_bf16=None) == "BFP4_ERR_NULL"
    assert _w16(workspace_bytes=64) == "BFP4_ERR_WORKSPACE"
    assert _w16(out=A + 64) == "BFP4_ERR_OVERLAP"                 # out over x
    assert _w16(do_finalize=0, gemm2_out=A + (45 << 16)) == "BFP4_ERR_OVERLAP"  # over the extent
    assert _w16(capacity=80) == "BFP4_ERR_CAPACITY"
    assert _w16(weight_format=2) == "BFP4_ERR_MODE"


def test_mxfp4_quantize_and_prepare_validation():
    def quant(**kw):
        args = dict(x_bf16=A, rows=4, cols=256, row_stride=256, q=A + (1 << 16), sf=A + (2 << 16),
                    stream=0)
        args.update(kw)
        with pytest.raises(Bfp4Error) as ei:
            bf.bfp4_quantize_mxfp4(**args)
        return bf.STATUS[ei.value.status]

    assert quant(cols=48) == "BFP4_ERR_SHAPE"                   # multiple of 32
    assert quant(row_stride=200) == "BFP4_ERR_SHAPE"
    assert quant(q=A + 8) == "BFP4_ERR_ALIGN"
    assert quant(sf=None) == "BFP4_ERR_NULL"
    assert quant(q=A + 64) == "BFP4_ERR_OVERLAP"
    if NO_GPU:
        assert quant() == "BFP4_ERR_DEVICE"
    with pytest.raises(Bfp4Error) as ei:
        bf.bfp4_prepare_weights_mxfp4(A, A, A, A, 1, 256, 100, 1, A, 1 << 20, 0)
    assert bf.STATUS[ei.value.status] == "BFP4_ERR_SHAPE"
    with pytest.raises(Bfp4Error) as ei:
        bf.bfp4_prepare_weights_mxfp4(A, A, A, A, 1, 256, 128, 1, A, 100, 0)
    assert bf.STATUS[ei.value.status] == "BFP4_ERR_WORKSPACE"


@cpu_only
def test_w4a16_valid_args_without_device():
    assert _w16() == "BFP4_ERR_DEVICE"
    assert _w16(block_m=32, capacity=bf.bfp4_plan_capacity(16, 2, 8, 32),
                workspace_bytes=bf.bfp4_workspace_size_w4a16(16, 256, 128, 2, 8, 32, 1)) == \
        "BFP4_ERR_DEVICE"


def _status(fn, **args):
    with pytest.raises(Bfp4Error) as ei:
        fn(**args)
    return bf.STATUS[ei.value.status]


def test_check_entry_points_validation():
    def topk(**kw):
        args = dict(topk_ids=A, M=4, top_k=2, num_experts=8, report=A + (1 << 16), stream=0)
        args.update(kw)
        return _status(bf.bfp4_check_topk_ids, **args)

    def plan(**kw):
        args = dict(sorted_token_ids=A, expert_ids=A + (1 << 16), num_tokens_post_padded=A + (2 << 16),
                    capacity=88, M=16, top_k=2, num_local_experts=8, block_m=8,
                    report=A + (3 << 16), stream=0)
        args.update(kw)
        return _status(bf.bfp4_check_plan, **args)

    assert topk(M=-1) == "BFP4_ERR_SHAPE"
    assert topk(top_k=0) == "BFP4_ERR_SHAPE"
    assert topk(num_experts=0) == "BFP4_ERR_EXPERTS"
    assert topk(report=None) == "BFP4_ERR_NULL"
    assert topk(topk_ids=None) == "BFP4_ERR_NULL"
    assert topk(report=A + (1 << 16) + 2) == "BFP4_ERR_ALIGN"
    assert topk(report=A + 28) == "BFP4_ERR_OVERLAP"          # inside topk_ids [4, 2] int32
    assert plan(block_m=12) == "BFP4_ERR_BLOCK_M"
    assert plan(num_local_experts=0) == "BFP4_ERR_EXPERTS"
    assert plan(capacity=84) == "BFP4_ERR_CAPACITY"           # not a multiple of block_m
    assert plan(num_tokens_post_padded=None) == "BFP4_ERR_NULL"
    assert plan(expert_ids=A + (1 << 16) + 1) == "BFP4_ERR_ALIGN"
    assert plan(report=A + 344) == "BFP4_ERR_OVERLAP"         # the last entry of sorted [88]
    if NO_GPU:
        assert topk() == "BFP4_ERR_DEVICE"
        assert topk(M=0, topk_ids=None) == "BFP4_ERR_DEVICE"  # an empty routing still reports
        assert plan() == "BFP4_ERR_DEVICE"
        assert plan(capacity=0, sorted_token_ids=None, expert_ids=None) == "BFP4_ERR_DEVICE"


def test_unpack_routing_validation():
    def unpack(**kw):
        args = dict(packed=A, M=4, top_k=2, topk_ids=A + (1 << 16), topk_weights=A + (2 << 16),
                    stream=0)
        args.update(kw)
        with pytest.raises(Bfp4Error) as ei:
            bf.bfp4_unpack_routing(**args)
        return bf.STATUS[ei.value.status]

    assert unpack(M=-1) == "BFP4_ERR_SHAPE"
    assert unpack(top_k=0) == "BFP4_ERR_SHAPE"
    assert unpack(M=1 << 28, top_k=8) == "BFP4_ERR_SHAPE"        # M * top_k = 2^31
    assert unpack(packed=None) == "BFP4_ERR_NULL"
    assert unpack(topk_weights=None) == "BFP4_ERR_NULL"
    assert unpack(topk_ids=A + (1 << 16) + 2) == "BFP4_ERR_ALIGN"
    assert unpack(topk_weights=A + (2 << 16) + 1) == "BFP4_ERR_ALIGN"
    assert unpack(topk_ids=A + 28) == "BFP4_ERR_OVERLAP"          # inside packed [4, 2] int32
    assert unpack(topk_weights=A + (1 << 16) + 30) == "BFP4_ERR_OVERLAP"   # inside topk_ids
    assert bf.bfp4_unpack_routing(None, 0, 2, None, None) == 0     # empty: nothing to do
    if NO_GPU:
        assert unpack() == "BFP4_ERR_DEVICE"


def test_xor_checksum_validation():
    def xs(**kw):
        args = dict(buf=A, nbytes=4096, partial=A + (1 << 20), stream=0)
        args.update(kw)
        with pytest.raises(Bfp4Error) as ei:
            bf.bfp4_xor_checksum(**args)
        return bf.STATUS[ei.value.status]

    assert xs(nbytes=4100) == "BFP4_ERR_SHAPE"                  # not a multiple of 16
    assert xs(partial=None) == "BFP4_ERR_NULL"
    assert xs(buf=None) == "BFP4_ERR_NULL"
    assert xs(buf=A + 8) == "BFP4_ERR_ALIGN"
    assert xs(partial=A + (1 << 20) + 2) == "BFP4_ERR_ALIGN"
    assert xs(partial=A + 4092) == "BFP4_ERR_OVERLAP"
    if NO_GPU:
        assert xs() == "BFP4_ERR_DEVICE"


def _pq(**kw):
    args = dict(topk_ids=A, M=16, top_k=2, num_experts=8, local_expert_offset=0,
                num_local_experts=8, block_m=8, sorted_token_ids=A + 4096, expert_ids=A + 8192,
                num_tokens_post_padded=A + 12288, token_to_row=A + 16384, capacity=88,
                plan_workspace=None, plan_workspace_bytes=0, x_bf16=A + 65536, H=256,
                row_stride=256, q=A + 2 * 65536, sf=A + 3 * 65536, dec_scale=A + 4 * 65536,
                stream=0)
    args.update(kw)
    with pytest.raises(Bfp4Error) as ei:
        bf.bfp4_moe_plan_quantize(**args)
    return bf.STATUS[ei.value.status]


def test_plan_quantize_validation():
    """The combined call rejects what either of the two calls it replaces rejects."""
    assert _pq(block_m=12) == "BFP4_ERR_BLOCK_M"
    assert _pq(capacity=80) == "BFP4_ERR_CAPACITY"
    assert _pq(num_local_experts=9) == "BFP4_ERR_EXPERTS"
    assert _pq(H=250, row_stride=256) == "BFP4_ERR_SHAPE"          # H % 32
    assert _pq(row_stride=128) == "BFP4_ERR_SHAPE"                  # stride < H
    assert _pq(x_bf16=A + 65536 + 2) == "BFP4_ERR_ALIGN"
    assert _pq(q=None) == "BFP4_ERR_NULL"
    assert _pq(q=A + 65536) == "BFP4_ERR_OVERLAP"                   # q inside x
    if NO_GPU:
        assert _pq() == "BFP4_ERR_DEVICE"
