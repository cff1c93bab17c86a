"""The C-ABI library loads and exports every entry point include/moe_ffn.h
declares; host-side argument validation (which returns before any device
work, so it runs without a GPU)."""
import ctypes
import os
import re

import pytest

from moe_expert_ffn_amd import binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "moe_ffn.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = B.load()
    names = _declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(B.EXPORTS)


def test_version_and_status_strings():
    lib = B.load()
    assert lib.moe_abi_version() == B.ABI_VERSION == 5
    assert lib.moe_status_str(0) == b"ok"
    assert b"workspace" in lib.moe_status_str(-3)


def test_size_helpers():
    assert B.max_slots(8192, 8, 128, 128) == 65536 + 128 * 127
    assert B.max_blocks(8192, 8, 128, 128) == (65536 + 128 * 127) // 128
    assert B.max_slots(-1, 8, 128, 128) == 0


def _layer(E=8, d=128, dff=64, act=B.MOE_F32, w=B.MOE_F32):
    return B.Layer(E, d, dff, act, w, 16, 32, None, None)


def test_workspace_size_and_rejections():
    lib = B.load()
    L = _layer()
    f = lib.moe_workspace_size(ctypes.byref(L), 256, 2, 16, 4, 1, 0)
    b = lib.moe_workspace_size(ctypes.byref(L), 256, 2, 16, 4, 1, 1)
    assert 0 < f <= b
    assert lib.moe_workspace_size(ctypes.byref(L), 256, 2, 16, 3, 1, 0) == 0    # P not in {1,2,4,8}
    assert lib.moe_workspace_size(ctypes.byref(L), 256, 2, 0, 4, 1, 0) == 0     # beta < 1


def test_operands_of_2gib_or_more_rejected():
    """The GEMM kernels address operands with 32-bit byte offsets and read
    masked rows at offset 2^31: sizes whose token rows, slot buffers or expert
    weights reach 2 GiB (in their own dtypes) are refused before anything is
    launched."""
    lib = B.load()
    P = ctypes.c_void_p(16)
    L = _layer()                                            # d = 128, d_ff = 64
    T = 1 << 22                                             # T * d * 4 = 2 GiB exactly
    assert lib.moe_workspace_size(ctypes.byref(L), T, 2, 16, 4, 1, 1) == 0
    # 2^19 tokens, top-2: token rows 256 MiB, slot buffers about 512 MiB each
    assert lib.moe_workspace_size(ctypes.byref(L), 1 << 19, 2, 16, 4, 1, 1) > 0
    assert lib.moe_forward(ctypes.byref(L), P, P, P, T, 2, 16, 4, *([P] * 8), P, 1 << 30, 0,
                           None, None, None) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_backward(ctypes.byref(L), P, P, P, P, P, T, 2, 16, 4, 1, *([P] * 10), P,
                            1 << 30, 0, None, None, None) == B.MOE_ERR_UNSUPPORTED
    # one expert's weights: 2 d_ff d fp32 elements must stay below 2 GiB
    wide = _layer(d=16384, dff=16384)
    assert lib.moe_workspace_size(ctypes.byref(wide), 16, 2, 16, 4, 1, 0) == 0
    # the DeepSeek-V3 share (bf16 activations, e4m3 weights): 10.8k tokens at top-8 reserve
    # about 90k slots, 1.3 GB of bf16 O rows, which the bf16 extent admits
    ds = B.Layer(32, 7168, 2048, B.MOE_BF16, B.MOE_FP8_E4M3, 16, 32, 64, 64)
    assert lib.moe_workspace_size(ctypes.byref(ds), 10800, 8, 128, 8, 4, 1) > 0
    # the same shapes in fp32 would need 2.6 GB of O rows
    ds32 = _layer(E=32, d=7168, dff=2048)
    assert lib.moe_workspace_size(ctypes.byref(ds32), 10800, 8, 128, 8, 4, 1) == 0


def test_host_validation_errors():
    lib = B.load()
    P = ctypes.c_void_p(16)
    # route stats: bad sizes / null pointers / missing workspace
    assert lib.moe_route_stats(P, 4, 2, 0, 16, *([P] * 8), P, 1 << 20, None) == B.MOE_ERR_ARG
    assert lib.moe_route_stats(P, 4, 2, 2000, 16, *([P] * 8), P, 1 << 20, None) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_route_stats(None, 4, 2, 8, 16, *([P] * 8), P, 1 << 20, None) == B.MOE_ERR_ARG
    assert lib.moe_route_stats(P, 4, 2, 8, 16, *([P] * 8), None, 0, None) == B.MOE_ERR_WORKSPACE
    assert lib.moe_route_stats(P, 4, 2, 8, 16, *([P] * 8), ctypes.c_void_p(17), 1 << 20,
                               None) == B.MOE_ERR_WORKSPACE
    # planner
    assert lib.moe_plan(P, P, P, 8, 3, 1, 0, 12, P, P, P, 64, P, P, P, 0, None) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_plan(P, P, P, 8, 4, -1, 0, 12, P, P, P, 64, P, P, P, 0, None) == B.MOE_ERR_ARG
    assert lib.moe_plan(P, P, P, 8, 4, 1, 3, 12, P, P, P, 64, P, P, P, 0, None) == B.MOE_ERR_ARG
    # quota mode: lambda is the quota floor and must be at least one block
    assert lib.moe_plan(P, P, P, 8, 4, 1, B.PLAN_QUOTA, 0, P, P, P, 64, P, P, P, 0, None) == B.MOE_ERR_ARG
    assert lib.moe_plan(P, P, P, 8, 4, 1, 0, -1, P, P, P, 64, P, P, P, 0, None) == B.MOE_ERR_ARG
    assert lib.moe_plan(P, P, P, 600, 4, 1, 0, 12, P, P, P, 64, P, P, P, 0, None) == B.MOE_ERR_UNSUPPORTED
    # block_worker capacity is a size
    assert lib.moe_plan(P, P, P, 8, 4, 1, 0, 12, P, P, P, -1, P, P, P, 0, None) == B.MOE_ERR_ARG
    # replication gate: price >= 0, P in {1,2,4,8}, E <= 512, no null pointers
    assert lib.moe_plan_gate(P, P, P, 8, 4, -1, P, P, P, 64, P, P, None) == B.MOE_ERR_ARG
    assert lib.moe_plan_gate(P, P, P, 0, 4, 1000, P, P, P, 64, P, P, None) == B.MOE_ERR_ARG
    assert lib.moe_plan_gate(P, P, P, 8, 3, 1000, P, P, P, 64, P, P, None) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_plan_gate(P, P, P, 600, 4, 1000, P, P, P, 64, P, P, None) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_plan_gate(P, None, P, 8, 4, 1000, P, P, P, 64, P, P, None) == B.MOE_ERR_ARG
    assert lib.moe_plan_gate(P, P, P, 8, 4, 1000, P, P, P, -1, P, P, None) == B.MOE_ERR_ARG
    # cost model: sizes, P, shapes the model covers, workgroups divisible by P
    assert lib.moe_predict_cost(*([P] * 5), 8, 128, 4, 256, 0, 256, P, P, None) == B.MOE_ERR_ARG
    assert lib.moe_predict_cost(*([P] * 5), 8, 128, 3, 256, 256, 256, P, P, None) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_predict_cost(*([P] * 5), 8, 128, 4, 384, 256, 256, P, P, None) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_predict_cost(*([P] * 5), 8, 128, 4, 256, 256, 254, P, P, None) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_predict_cost(*([P] * 5), 8, 128, 1, 256, 256, 512, P, P, None) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_predict_cost(*([P] * 4), None, 8, 128, 4, 256, 256, 256, P, P, None) == B.MOE_ERR_ARG
    # forward / backward layer checks
    bad_d = _layer(d=96)
    assert lib.moe_forward(ctypes.byref(bad_d), P, P, P, 4, 2, 16, 4, *([P] * 8), P, 1 << 30, 0,
                           None, None, None) == B.MOE_ERR_UNSUPPORTED
    mixed = _layer(act=B.MOE_F32, w=B.MOE_BF16)
    assert lib.moe_forward(ctypes.byref(mixed), P, P, P, 4, 2, 16, 4, *([P] * 8), P, 1 << 30, 0,
                           None, None, None) == B.MOE_ERR_UNSUPPORTED
    fp8 = B.Layer(8, 128, 128, B.MOE_BF16, B.MOE_FP8_E4M3, 16, 32, 64, 64)
    # fp8 weights have a backward (token-axis requantization): the call gets past
    # the layer checks and stops at a workspace too small for the e4m3 buffers
    assert lib.moe_backward(ctypes.byref(fp8), P, P, P, P, P, 4, 2, 16, 4, 1, *([P] * 10), P,
                            16, 0, None, None, None) == B.MOE_ERR_WORKSPACE
    nofp8 = B.Layer(8, 128, 192, B.MOE_BF16, B.MOE_FP8_E4M3, 16, 32, 64, 64)   # d_ff % 128
    assert lib.moe_backward(ctypes.byref(nofp8), P, P, P, P, P, 4, 2, 16, 4, 1, *([P] * 10), P,
                            1 << 30, 0, None, None, None) == B.MOE_ERR_UNSUPPORTED
    # token-axis quantization: shapes and pointers are checked on the host
    # (src, ld, src_rows, row_map, gather, row_div, row_scale, rows, cols, block_rows, codes,
    #  scales, stream)
    q = lib.moe_quantize_token_blocks
    assert q(P, 16, 4, None, 0, 1, None, 4, 12, 128, P, P, None) == B.MOE_ERR_ARG     # cols % 8
    assert q(P, 8, 4, None, 0, 1, None, 4, 16, 128, P, P, None) == B.MOE_ERR_ARG      # ld < cols
    assert q(P, 20, 4, None, 0, 1, None, 4, 16, 128, P, P, None) == B.MOE_ERR_ARG     # ld % 8
    assert q(P, 16, 4, None, 0, 1, None, -1, 16, 128, P, P, None) == B.MOE_ERR_ARG    # rows
    assert q(P, 16, 4, None, 0, 1, None, 4, 16, 0, P, P, None) == B.MOE_ERR_ARG       # block rows
    assert q(P, 16, 4, None, 0, 0, None, 4, 16, 128, P, P, None) == B.MOE_ERR_ARG     # row_div
    assert q(None, 16, 4, None, 0, 1, None, 4, 16, 128, P, P, None) == B.MOE_ERR_ARG  # src
    assert q(P, 16, 4, None, 0, 1, None, 4, 16, 128, None, P, None) == B.MOE_ERR_ARG  # codes
    assert q(P, 16, -1, P, 1, 1, None, 4, 16, 128, P, P, None) == B.MOE_ERR_ARG       # src_rows
    assert q(P, 16, 3, None, 0, 1, None, 4, 16, 128, P, P, None) == B.MOE_ERR_ARG     # rows in place
    assert q(P, 16, 3, P, 0, 1, None, 4, 16, 128, P, P, None) == B.MOE_ERR_ARG        # > src_rows
    big = 65535 * 128 + 8                                                            # > 65535 column tiles
    assert q(P, big, 4, None, 0, 1, None, 4, big, 128, P, P, None) == B.MOE_ERR_ARG
    # activation rows for the fp8 MFMA: (src, rows, cols, codes, exps, stream)
    qa = lib.moe_quantize_act_rows
    assert qa(P, -1, 128, P, P, None) == B.MOE_ERR_ARG                               # rows
    assert qa(P, 4, 192, P, P, None) == B.MOE_ERR_ARG                                # cols % 128
    assert qa(P, 4, 0, P, P, None) == B.MOE_ERR_ARG                                  # cols
    assert qa(None, 4, 128, P, P, None) == B.MOE_ERR_ARG                             # src
    assert qa(P, 4, 128, None, P, None) == B.MOE_ERR_ARG                             # codes
    assert qa(P, 4, 128, P, None, None) == B.MOE_ERR_ARG                             # exps
    assert qa(None, 0, 128, None, None, None) == B.MOE_OK                            # nothing to do
    ok = _layer()
    assert lib.moe_forward(ctypes.byref(ok), P, P, P, 4, 2, 16, 4, *([P] * 8), P, 16, 0, None,
                           None, None) == B.MOE_ERR_WORKSPACE
    assert lib.moe_forward(ctypes.byref(ok), P, P, P, 4, 2, 16, 5, *([P] * 8), P, 1 << 30, 0, None,
                           None, None) == B.MOE_ERR_UNSUPPORTED
    # unknown exec_flags; MOE_EXEC_FP8_ACT on a bf16 layer
    assert lib.moe_forward(ctypes.byref(ok), P, P, P, 4, 2, 16, 4, *([P] * 8), P, 1 << 30, 4, None,
                           None, None) == B.MOE_ERR_ARG
    assert lib.moe_forward(ctypes.byref(ok), P, P, P, 4, 2, 16, 4, *([P] * 8), P, 1 << 30,
                           B.EXEC_FP8_ACT, None, None, None) == B.MOE_ERR_ARG
    # ... on an e4m3 layer together with the two-phase launch, or off the 256 grid,
    # in either direction; the backward refuses it on a bf16 layer too
    f8 = B.Layer(8, 256, 256, B.MOE_BF16, B.MOE_FP8_E4M3, 16, 32, 64, 64)
    f8small = B.Layer(8, 128, 128, B.MOE_BF16, B.MOE_FP8_E4M3, 16, 32, 64, 64)
    for lay, fl in ((f8, B.EXEC_FP8_ACT | B.EXEC_TWO_PHASE), (f8small, B.EXEC_FP8_ACT)):
        assert lib.moe_forward(ctypes.byref(lay), P, P, P, 4, 2, 16, 4, *([P] * 8), P, 1 << 30,
                               fl, None, None, None) == B.MOE_ERR_ARG
        assert lib.moe_backward(ctypes.byref(lay), P, P, P, P, P, 4, 2, 16, 4, 1, *([P] * 10), P,
                                1 << 30, fl, None, None, None) == B.MOE_ERR_ARG
    assert lib.moe_backward(ctypes.byref(ok), P, P, P, P, P, 4, 2, 16, 4, 1, *([P] * 10), P,
                            1 << 30, B.EXEC_FP8_ACT, None, None, None) == B.MOE_ERR_ARG
    assert lib.moe_backward(ctypes.byref(ok), P, P, P, P, P, 4, 2, 16, 4, 1, *([P] * 10), P,
                            1 << 30, 4, None, None, None) == B.MOE_ERR_ARG
    # a producer/consumer split without the two-phase launch, or bits past 15
    for bad in (1 << 8, 1 | (1 << 16)):
        assert lib.moe_forward(ctypes.byref(ok), P, P, P, 4, 2, 16, 4, *([P] * 8), P, 1 << 30, bad,
                               None, None, None) == B.MOE_ERR_ARG
        assert lib.moe_backward(ctypes.byref(ok), P, P, P, P, P, 4, 2, 16, 4, 1, *([P] * 10), P,
                                1 << 30, bad, None, None, None) == B.MOE_ERR_ARG
    # split model: (counts, offsets, block_worker, E, beta, P, d, d_ff, G, backward,
    #  costs, choice, status, stream)
    ps = lib.moe_predict_split
    assert ps(P, P, P, 0, 16, 4, 256, 256, 256, 0, P, P, P, None) == B.MOE_ERR_ARG      # E
    assert ps(P, P, P, 8, 0, 4, 256, 256, 256, 0, P, P, P, None) == B.MOE_ERR_ARG      # beta
    assert ps(P, P, None, 8, 16, 4, 256, 256, 256, 0, P, P, P, None) == B.MOE_ERR_ARG  # plan
    assert ps(P, P, P, 8, 16, 4, 256, 256, 256, 0, P, None, P, None) == B.MOE_ERR_ARG  # choice
    assert ps(P, P, P, 8, 16, 3, 256, 256, 256, 0, P, P, P, None) == B.MOE_ERR_UNSUPPORTED  # P
    assert ps(P, P, P, 8, 16, 4, 384, 256, 256, 0, P, P, P, None) == B.MOE_ERR_UNSUPPORTED  # d
    assert ps(P, P, P, 8, 16, 4, 256, 256, 254, 0, P, P, P, None) == B.MOE_ERR_UNSUPPORTED  # G % P
    assert ps(P, P, P, 8, 16, 1, 256, 256, 512, 0, P, P, P, None) == B.MOE_ERR_UNSUPPORTED  # G/P
    # the binding builds the flags and refuses a split without the two-phase launch
    assert B.exec_flags(True, 12) == 1 | (12 << 8)
    with pytest.raises(B.MoeError):
        B.exec_flags(False, 3)
    with pytest.raises(B.MoeError):
        B.exec_flags(True, 256)


def test_quantizer_binding_checks_buffers():
    """The Python binding refuses buffers of the wrong element type or size
    before anything reaches the device (no GPU needed: the checks come first)."""
    import torch

    class FakeDev:
        """A tensor stand-in that claims to be a contiguous device tensor."""
        def __init__(self, dtype, n):
            self.dtype, self._n = dtype, n
            self.is_cuda = True

        def is_contiguous(self):
            return True

        def numel(self):
            return self._n

    src = FakeDev(torch.bfloat16, 64 * 16)
    ok_codes, ok_scales = FakeDev(torch.uint8, 64 * 16), FakeDev(torch.float32, 16)
    with pytest.raises(B.MoeError, match="codes"):
        B.quantize_token_blocks(src, 64, 16, 128, FakeDev(torch.uint8, 10), ok_scales)
    with pytest.raises(B.MoeError, match="scales"):
        B.quantize_token_blocks(src, 64, 16, 128, ok_codes, FakeDev(torch.float16, 16))
    with pytest.raises(B.MoeError, match="src"):
        B.quantize_token_blocks(FakeDev(torch.float32, 64 * 16), 64, 16, 128, ok_codes, ok_scales)
    with pytest.raises(B.MoeError, match="row_map"):
        B.quantize_token_blocks(src, 64, 16, 128, ok_codes, ok_scales,
                                row_map=FakeDev(torch.int64, 64))
    # gathered rows: src_rows is required, src must hold that many rows and the
    # row scales one entry per (src row, map divisor)
    rmap = FakeDev(torch.int32, 64)
    with pytest.raises(B.MoeError, match="src_rows"):
        B.quantize_token_blocks(src, 64, 16, 128, ok_codes, ok_scales, row_map=rmap, gather=True,
                                row_div=8)
    with pytest.raises(B.MoeError, match="src"):
        B.quantize_token_blocks(src, 64, 16, 128, ok_codes, ok_scales, row_map=rmap, gather=True,
                                row_div=8, src_rows=65)
    with pytest.raises(B.MoeError, match="row_scale"):
        B.quantize_token_blocks(src, 64, 16, 128, ok_codes, ok_scales, row_map=rmap, gather=True,
                                row_div=8, src_rows=64, row_scale=FakeDev(torch.float32, 64 * 8 - 1))


def test_executor_bindings_check_buffers():
    """route_stats, plan, forward and backward refuse tensors of the wrong
    element type or too few elements before anything reaches the device (an
    undersized output would be written past its end)."""
    import torch

    class FakeDev:
        def __init__(self, dtype, n, shape=None):
            self.dtype, self._n, self.shape = dtype, n, shape if shape is not None else (n,)
            self.is_cuda = True

        def is_contiguous(self):
            return True

        def numel(self):
            return self._n

        def dim(self):
            return len(self.shape)

        def data_ptr(self):
            return 16

    T, k, E, beta, P, d, dff = 32, 2, 8, 16, 4, 128, 64
    i32, f32 = torch.int32, torch.float32
    ids = FakeDev(i32, T * k, (T, k))
    S = B.max_slots(T, k, E, beta)
    rs = {"counts": FakeDev(i32, E), "offsets": FakeDev(i32, E + 1),
          "block_counts": FakeDev(i32, E), "block_offsets": FakeDev(i32, E + 1),
          "row_to_slot": FakeDev(i32, T * k), "slot_to_row": FakeDev(i32, S),
          "kappa": FakeDev(torch.float64, 1)}
    ws, st = FakeDev(torch.uint8, 1 << 20), FakeDev(i32, 1)
    with pytest.raises(B.MoeError, match="slot_to_row"):
        B.route_stats(ids, E, beta, {**rs, "slot_to_row": FakeDev(i32, S - 1)}, ws, st)
    with pytest.raises(B.MoeError, match="kappa"):
        B.route_stats(ids, E, beta, {**rs, "kappa": FakeDev(f32, 1)}, ws, st)
    with pytest.raises(B.MoeError, match="topk_ids"):
        B.route_stats(FakeDev(i32, T * k, (T * k,)), E, beta, rs, ws, st)
    plan = {"q": FakeDev(i32, E * P), "load": FakeDev(i32, P), "block_worker": FakeDev(i32, 64),
            "plan_info": FakeDev(i32, 4)}
    with pytest.raises(B.MoeError, match="q"):
        B.plan(rs["block_counts"], rs["block_offsets"], FakeDev(i32, E), P, 1, 0, 12,
               {**plan, "q": FakeDev(i32, E * P - 1)}, ws, st)
    with pytest.raises(B.MoeError, match="owner"):
        B.plan(rs["block_counts"], rs["block_offsets"], FakeDev(torch.int64, E), P, 1, 0, 12, plan,
               ws, st)
    L = B.Layer(E, d, dff, B.MOE_BF16, B.MOE_BF16, 16, 32, None, None)
    bf = torch.bfloat16
    x, g = FakeDev(bf, T * d), FakeDev(f32, T * k)
    z = FakeDev(bf, S * 2 * dff)
    bw = FakeDev(i32, B.max_blocks(T, k, E, beta))
    with pytest.raises(B.MoeError, match="block_worker"):
        B.forward(L, x, g, ids, beta, P, rs, FakeDev(i32, B.max_blocks(T, k, E, beta) - 1),
                  FakeDev(bf, T * d), z, ws, st)
    with pytest.raises(B.MoeError, match="y"):
        B.forward(L, x, g, ids, beta, P, rs, bw, FakeDev(f32, T * d), z, ws, st)
    with pytest.raises(B.MoeError, match="z_save"):
        B.forward(L, x, g, ids, beta, P, rs, bw, FakeDev(bf, T * d), FakeDev(bf, S * dff), ws, st)
    own = FakeDev(i32, E)
    dw1, dw2 = FakeDev(f32, E * 2 * dff * d), FakeDev(f32, E * d * dff)
    with pytest.raises(B.MoeError, match="dw1"):
        B.backward(L, x, g, x, z, ids, beta, P, 1, rs, own, bw, FakeDev(bf, T * d),
                   FakeDev(f32, E * 2 * dff * d - 1), dw2, ws, st)
    with pytest.raises(B.MoeError, match="gates"):
        B.backward(L, x, FakeDev(bf, T * k), x, z, ids, beta, P, 1, rs, own, bw,
                   FakeDev(bf, T * d), dw1, dw2, ws, st)


def test_make_layer_checks_weights():
    """make_layer refuses mismatched weight shapes or types and e4m3 weights
    without correctly sized block scales."""
    import torch

    class FakeW:
        def __init__(self, dtype, shape):
            self.dtype, self.shape = dtype, shape
            self.is_cuda = True

        def is_contiguous(self):
            return True

        def dim(self):
            return len(self.shape)

        def numel(self):
            n = 1
            for v in self.shape:
                n *= v
            return n

        def data_ptr(self):
            return 16

    E, d, dff = 4, 256, 128
    bf = torch.bfloat16
    L = B.make_layer(FakeW(bf, (E, 2 * dff, d)), FakeW(bf, (E, d, dff)))
    assert (L.E, L.d, L.d_ff, L.w_dtype) == (E, d, dff, B.MOE_BF16)
    with pytest.raises(B.MoeError, match="w2"):
        B.make_layer(FakeW(bf, (E, 2 * dff, d)), FakeW(bf, (E, dff, d)))
    with pytest.raises(B.MoeError, match="w2"):
        B.make_layer(FakeW(bf, (E, 2 * dff, d)), FakeW(torch.float32, (E, d, dff)))
    u8 = torch.uint8
    w1, w2 = FakeW(u8, (E, 2 * dff, d)), FakeW(u8, (E, d, dff))
    with pytest.raises(B.MoeError, match="scale"):
        B.make_layer(w1, w2)
    s1, s2 = FakeW(torch.float32, (E, 2, 2)), FakeW(torch.float32, (E, 2, 1))
    assert B.make_layer(w1, w2, s1, s2).w_dtype == B.MOE_FP8_E4M3
    with pytest.raises(B.MoeError, match="w2_scale"):
        B.make_layer(w1, w2, s1, FakeW(torch.float32, (E, 1, 1)))
