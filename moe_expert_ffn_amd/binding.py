"""Thin ctypes binding of libmoe_ffn.so (C ABI in include/moe_ffn.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  torch provides device memory and the current HIP stream.  The
library must have been built (``python moe_expert_ffn_amd/build.py`` or
``__graft_entry__.build()``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_ffn.so")

ABI_VERSION = 5                 # MOE_ABI_VERSION of the header these signatures follow
MOE_OK, MOE_ERR_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
PLAN_FWD, PLAN_BWD, PLAN_QUOTA = 0, 1, 2
DEV_BAD_EXPERT, DEV_BAD_PLAN, DEV_BAD_OWNER, DEV_WAIT_TIMEOUT = 1, 2, 4, 8
EXEC_TWO_PHASE = 1              # MOE_EXEC_TWO_PHASE
EXEC_SPLIT_SHIFT = 8            # MOE_EXEC_SPLIT(n1) = n1 << 8
EXEC_FP8_ACT = 2                # MOE_EXEC_FP8_ACT


def exec_flags(two_phase=False, split=0, fp8_act=False):
    """exec_flags of moe_forward / moe_backward: the two-phase launch and its
    producer workgroups per worker (0: every workgroup runs both phases)."""
    split = int(split)
    if split and not two_phase:
        raise MoeError("a producer/consumer split needs the two-phase launch")
    if not 0 <= split <= 0xFF:
        raise MoeError(f"split={split} outside 0..255")
    return ((EXEC_TWO_PHASE if two_phase else 0) | (split << EXEC_SPLIT_SHIFT) |
            (EXEC_FP8_ACT if fp8_act else 0))
TIMELINE_MAX_WG, TL_PHASES = 1024, 5          # MOE_TIMELINE_MAX_WG, MOE_TL_PHASES
TL_FC1, TL_FC2, TL_DA, TL_DX, TL_DW = range(5)

EXPORTS = ["moe_abi_version", "moe_status_str", "moe_max_slots", "moe_max_blocks",
           "moe_workspace_size", "moe_route_stats", "moe_route_stats_noalloc", "moe_plan",
           "moe_plan_gate",
           "moe_predict_cost", "moe_predict_split", "moe_quantize_token_blocks",
           "moe_quantize_act_rows", "moe_forward",
           "moe_backward",
           "moe_event_create", "moe_event_destroy", "moe_event_record", "moe_event_elapsed_ms",
           "moe_device_info"]


class MoeError(RuntimeError):
    pass


class Layer(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int), ("d", ctypes.c_int), ("d_ff", ctypes.c_int),
                ("act_dtype", ctypes.c_int), ("w_dtype", ctypes.c_int),
                ("w1", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("w1_scale", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p)]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t


def load():
    """Load the built library (raises MoeError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise MoeError(f"{LIB_PATH} is missing: build it with moe_expert_ffn_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    lib.moe_abi_version.restype = _I
    lib.moe_status_str.restype = ctypes.c_char_p
    lib.moe_status_str.argtypes = [_I]
    lib.moe_max_slots.restype = _SZ
    lib.moe_max_slots.argtypes = [_I, _I, _I, _I]
    lib.moe_max_blocks.restype = _SZ
    lib.moe_max_blocks.argtypes = [_I, _I, _I, _I]
    lib.moe_workspace_size.restype = _SZ
    lib.moe_workspace_size.argtypes = [ctypes.POINTER(Layer), _I, _I, _I, _I, _I, _I]
    lib.moe_route_stats.restype = _I
    lib.moe_route_stats.argtypes = [_P, _I, _I, _I, _I] + [_P] * 8 + [_P, _SZ, _P]
    lib.moe_route_stats_noalloc.restype = _I
    lib.moe_route_stats_noalloc.argtypes = [_P, _I, _I, _I, _I] + [_P] * 8 + [_P]
    lib.moe_plan.restype = _I
    lib.moe_plan.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I] + [_P] * 3 + [_I] + [_P] * 2 + [_P, _SZ, _P]
    lib.moe_quantize_token_blocks.restype = _I
    lib.moe_quantize_token_blocks.argtypes = [_P, _I, _I, _P, _I, _I, _P, _I, _I, _I, _P, _P, _P]
    lib.moe_predict_cost.restype = _I
    lib.moe_predict_cost.argtypes = [_P] * 5 + [_I] * 6 + [_P, _P, _P]
    lib.moe_quantize_act_rows.restype = _I
    lib.moe_quantize_act_rows.argtypes = [_P, _I, _I, _P, _P, _P]
    lib.moe_predict_split.restype = _I
    lib.moe_predict_split.argtypes = [_P] * 3 + [_I] * 7 + [_P, _P, _P, _P]
    lib.moe_plan_gate.restype = _I
    lib.moe_plan_gate.argtypes = [_P, _P, _P, _I, _I, _I] + [_P] * 3 + [_I] + [_P] * 2 + [_P]
    lib.moe_forward.restype = _I
    lib.moe_forward.argtypes = ([ctypes.POINTER(Layer), _P, _P, _P, _I, _I, _I, _I]
                                + [_P] * 8 + [_P, _SZ, _I, _P, _P, _P])
    lib.moe_backward.restype = _I
    lib.moe_backward.argtypes = ([ctypes.POINTER(Layer), _P, _P, _P, _P, _P, _I, _I, _I, _I, _I]
                                 + [_P] * 10 + [_P, _SZ, _I, _P, _P, _P])
    lib.moe_event_create.argtypes = [ctypes.POINTER(_P)]
    lib.moe_event_destroy.argtypes = [_P]
    lib.moe_event_record.argtypes = [_P, _P]
    lib.moe_event_elapsed_ms.argtypes = [_P, _P, ctypes.POINTER(ctypes.c_float)]
    lib.moe_device_info.argtypes = [ctypes.POINTER(_I)] * 3
    if lib.moe_abi_version() != ABI_VERSION:
        raise MoeError(f"{LIB_PATH} has ABI {lib.moe_abi_version()}, the binding expects "
                       f"{ABI_VERSION}: rebuild it")
    _lib = lib
    return lib


def _check(rc):
    if rc != MOE_OK:
        raise MoeError(f"libmoe_ffn: {load().moe_status_str(rc).decode()} ({rc})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _require_device(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise MoeError("all buffers must be contiguous device tensors")


def _expect(t, dtype, min_numel, name):
    """Element type and minimum size of a buffer the library writes or reads."""
    if t.dtype != dtype:
        raise MoeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.numel() < min_numel:
        raise MoeError(f"{name}: needs at least {min_numel} elements, has {t.numel()}")


def act_code(dtype) -> int:
    return MOE_F32 if dtype == torch.float32 else MOE_BF16


def _act_dtype(layer) -> torch.dtype:
    return torch.float32 if layer.act_dtype == MOE_F32 else torch.bfloat16


def _ids_shape(topk_ids):
    if topk_ids.dim() != 2:
        raise MoeError(f"topk_ids: expected [T][k], got {tuple(topk_ids.shape)}")
    _expect(topk_ids, torch.int32, 0, "topk_ids")
    return topk_ids.shape


def _expect_route(rs, T, k, E, beta):
    """The routing statistics the executors read (from route_stats)."""
    _expect(rs["counts"], torch.int32, E, "counts")
    _expect(rs["block_offsets"], torch.int32, E + 1, "block_offsets")
    _expect(rs["row_to_slot"], torch.int32, T * k, "row_to_slot")
    _expect(rs["slot_to_row"], torch.int32, max_slots(T, k, E, beta), "slot_to_row")


def _expect_plan_out(out, E, P):
    _expect(out["q"], torch.int32, E * P, "q")
    _expect(out["load"], torch.int32, P, "load")
    # block_worker [>= sum b]: its size goes to the library, which writes nothing
    # (and flags the plan) when the blocks do not fit
    _expect(out["block_worker"], torch.int32, 1, "block_worker")
    _expect(out["plan_info"], torch.int32, 4, "plan_info")


def make_layer(w1, w2, w1_scale=None, w2_scale=None, act_dtype=torch.bfloat16) -> Layer:
    _require_device(w1, w2, w1_scale, w2_scale)
    if w1.dim() != 3 or w2.dim() != 3:
        raise MoeError("w1 and w2 are [E][2 d_ff][d] and [E][d][d_ff]")
    E, two_dff, d = w1.shape
    if tuple(w2.shape) != (E, d, two_dff // 2) or two_dff % 2:
        raise MoeError(f"w2: expected {(E, d, two_dff // 2)}, got {tuple(w2.shape)}")
    if w2.dtype != w1.dtype:
        raise MoeError(f"w2: expected {w1.dtype}, got {w2.dtype}")
    if w1.dtype == torch.uint8:
        wcode = MOE_FP8_E4M3
        if w1_scale is None or w2_scale is None:
            raise MoeError("e4m3 weights need w1_scale and w2_scale")
        _expect(w1_scale, torch.float32, E * -(-two_dff // 128) * -(-d // 128), "w1_scale")
        _expect(w2_scale, torch.float32, E * -(-d // 128) * -(-(two_dff // 2) // 128), "w2_scale")
    elif w1.dtype == torch.float32:
        wcode = MOE_F32
    elif w1.dtype == torch.bfloat16:
        wcode = MOE_BF16
    else:
        raise MoeError(f"w1: unsupported element type {w1.dtype}")
    return Layer(E, d, two_dff // 2, act_code(act_dtype), wcode, w1.data_ptr(), w2.data_ptr(),
                 w1_scale.data_ptr() if w1_scale is not None else None,
                 w2_scale.data_ptr() if w2_scale is not None else None)


def max_slots(T, k, E, beta) -> int:
    return int(load().moe_max_slots(T, k, E, beta))


def max_blocks(T, k, E, beta) -> int:
    return int(load().moe_max_blocks(T, k, E, beta))


def workspace(layer: Layer, T, k, beta, P, s, with_backward, device) -> torch.Tensor:
    n = int(load().moe_workspace_size(ctypes.byref(layer), T, k, beta, P, s, int(with_backward)))
    if n == 0:
        raise MoeError("moe_workspace_size rejected the sizes")
    return torch.empty(n + 256, dtype=torch.uint8, device=device)


def _aligned(ws: torch.Tensor):
    p = ws.data_ptr()
    off = (-p) % 256
    return ctypes.c_void_p(p + off), ws.numel() - off


def alloc_route(T, k, E, beta, device):
    i32 = dict(dtype=torch.int32, device=device)
    return {
        "counts": torch.empty(E, **i32), "offsets": torch.empty(E + 1, **i32),
        "block_counts": torch.empty(E, **i32), "block_offsets": torch.empty(E + 1, **i32),
        "row_to_slot": torch.empty(max(T * k, 1), **i32),
        "slot_to_row": torch.empty(max(max_slots(T, k, E, beta), 1), **i32),
        "kappa": torch.empty(1, dtype=torch.float64, device=device),
    }


def route_stats(topk_ids: torch.Tensor, E: int, beta: int, out: dict, ws: torch.Tensor,
                status: torch.Tensor):
    _require_device(topk_ids, ws, status, *out.values())
    T, k = _ids_shape(topk_ids)
    _expect(out["counts"], torch.int32, E, "counts")
    _expect(out["offsets"], torch.int32, E + 1, "offsets")
    _expect(out["block_counts"], torch.int32, E, "block_counts")
    _expect(out["block_offsets"], torch.int32, E + 1, "block_offsets")
    _expect(out["row_to_slot"], torch.int32, T * k, "row_to_slot")
    _expect(out["slot_to_row"], torch.int32, max_slots(T, k, E, beta), "slot_to_row")
    _expect(out["kappa"], torch.float64, 1, "kappa")
    _expect(status, torch.int32, 1, "status")
    wsp, wsn = _aligned(ws)
    _check(load().moe_route_stats(_ptr(topk_ids), T, k, E, beta, _ptr(out["counts"]),
                                  _ptr(out["offsets"]), _ptr(out["block_counts"]),
                                  _ptr(out["block_offsets"]), _ptr(out["row_to_slot"]),
                                  _ptr(out["slot_to_row"]), _ptr(out["kappa"]), _ptr(status),
                                  wsp, wsn, _stream()))
    return out


def route_stats_noalloc(topk_ids: torch.Tensor, E: int, beta: int, out: dict,
                        status: torch.Tensor):
    """route_stats without a workspace (moe_route_stats_noalloc): the library's
    own scratch array holds the per-chunk counts."""
    _require_device(topk_ids, status, *out.values())
    T, k = _ids_shape(topk_ids)
    _expect(out["counts"], torch.int32, E, "counts")
    _expect(out["offsets"], torch.int32, E + 1, "offsets")
    _expect(out["block_counts"], torch.int32, E, "block_counts")
    _expect(out["block_offsets"], torch.int32, E + 1, "block_offsets")
    _expect(out["row_to_slot"], torch.int32, T * k, "row_to_slot")
    _expect(out["slot_to_row"], torch.int32, max_slots(T, k, E, beta), "slot_to_row")
    _expect(out["kappa"], torch.float64, 1, "kappa")
    _expect(status, torch.int32, 1, "status")
    _check(load().moe_route_stats_noalloc(_ptr(topk_ids), T, k, E, beta, _ptr(out["counts"]),
                                          _ptr(out["offsets"]), _ptr(out["block_counts"]),
                                          _ptr(out["block_offsets"]), _ptr(out["row_to_slot"]),
                                          _ptr(out["slot_to_row"]), _ptr(out["kappa"]),
                                          _ptr(status), _stream()))
    return out


def alloc_plan(E, P, nblocks_cap, device):
    i32 = dict(dtype=torch.int32, device=device)
    return {"q": torch.empty((E, P), **i32), "load": torch.empty(P, **i32),
            "block_worker": torch.full((max(nblocks_cap, 1),), -1, **i32),
            "plan_info": torch.empty(4, **i32)}


def predict_cost(counts, block_offsets, bw_fwd, bw_bwd, owner, beta, P, d, d_ff, cost, status,
                 num_workgroups=0):
    """Wave-quantized predicted cost (int64, thousandths of a K step) into cost[0]."""
    _require_device(counts, block_offsets, bw_fwd, bw_bwd, owner, cost, status)
    _check(load().moe_predict_cost(_ptr(counts), _ptr(block_offsets), _ptr(bw_fwd), _ptr(bw_bwd),
                                   _ptr(owner), counts.numel(), beta, P, d, d_ff, num_workgroups,
                                   _ptr(cost), _ptr(status), _stream()))
    return cost


def predict_split(counts, block_offsets, block_worker, beta, P, d, d_ff, backward, costs, choice,
                  status, num_workgroups=0):
    """Predicted time (int64, thousandths of a K step) of every two-phase mode
    into costs[m + 1] (m = -1 two launches, 0 one launch, n1 > 0 producer /
    consumer split) and the chosen mode into choice[0]."""
    _require_device(counts, block_offsets, block_worker, costs, choice, status)
    _expect(costs, torch.int64, costs.numel(), "costs")
    _expect(choice, torch.int32, 1, "choice")
    G = num_workgroups if num_workgroups > 0 else device_info()["num_cus"]
    if P > 0 and G % P == 0 and costs.numel() < G // P + 1:
        raise MoeError(f"costs holds {costs.numel()} entries, the model writes {G // P + 1}")
    _check(load().moe_predict_split(_ptr(counts), _ptr(block_offsets), _ptr(block_worker),
                                    counts.numel(), beta, P, d, d_ff, num_workgroups,
                                    1 if backward else 0, _ptr(costs), _ptr(choice), _ptr(status),
                                    _stream()))
    return costs, choice


def quantize_act_rows(src, codes, exps):
    """e4m3 codes [rows][cols] and power-of-two exponents [cols/128][rows]
    (int32) of the bf16 rows src [rows][cols], blocks of 128 features."""
    _require_device(src, codes, exps)
    if src.dim() != 2:
        raise MoeError("src must be [rows][cols]")
    rows, cols = src.shape
    _expect(src, torch.bfloat16, rows * cols, "src")
    _expect(codes, torch.uint8, rows * cols, "codes")
    _expect(exps, torch.int32, rows * (cols // 128), "exps")
    _check(load().moe_quantize_act_rows(_ptr(src), rows, cols, _ptr(codes), _ptr(exps), _stream()))
    return codes, exps


def quantize_token_blocks(src, rows, cols, block_rows, codes, scales, row_map=None, gather=False,
                          row_div=1, row_scale=None, ld=None, src_rows=None):
    """Token-axis e4m3 codes [rows][cols] and scales [ceil(rows/block_rows)][cols].

    src holds src_rows rows of ld elements (default: rows, the rows read in
    place); gathered map values past src_rows * row_div read as zero rows, and
    row_scale must hold src_rows * row_div entries."""
    _require_device(src, codes, scales, *[t for t in (row_map, row_scale) if t is not None])
    ld = cols if ld is None else ld
    if src_rows is None:
        if gather:
            raise MoeError("gathered rows need src_rows (the rows of src)")
        src_rows = rows
    if rows > 0 and block_rows > 0:
        nblk = (rows + block_rows - 1) // block_rows
        _expect(codes, torch.uint8, rows * cols, "codes")
        _expect(scales, torch.float32, nblk * cols, "scales")
        _expect(src, torch.bfloat16, (src_rows - 1) * ld + cols if src_rows > 0 else 0, "src")
        if row_map is not None:
            _expect(row_map, torch.int32, rows, "row_map")
        if row_scale is not None:
            _expect(row_scale, torch.float32, src_rows * row_div, "row_scale")
    _check(load().moe_quantize_token_blocks(
        _ptr(src), ld, src_rows, _ptr(row_map) if row_map is not None else None,
        1 if gather else 0, row_div, _ptr(row_scale) if row_scale is not None else None, rows, cols,
        block_rows, _ptr(codes), _ptr(scales), _stream()))
    return codes, scales


def plan_gate(block_counts, block_offsets, owner, P, rho_milli, out, status):
    _require_device(block_counts, block_offsets, owner, status, *out.values())
    E = block_counts.numel()
    _expect(block_counts, torch.int32, E, "block_counts")
    _expect(block_offsets, torch.int32, E + 1, "block_offsets")
    _expect(owner, torch.int32, E, "owner")
    _expect_plan_out(out, E, P)
    _expect(status, torch.int32, 1, "status")
    _check(load().moe_plan_gate(_ptr(block_counts), _ptr(block_offsets), _ptr(owner), E, P,
                                rho_milli, _ptr(out["q"]), _ptr(out["load"]),
                                _ptr(out["block_worker"]), out["block_worker"].numel(),
                                _ptr(out["plan_info"]), _ptr(status), _stream()))
    return out


def plan(block_counts, block_offsets, owner, P, s, mode, lam, out, ws, status):
    _require_device(block_counts, block_offsets, owner, ws, status, *out.values())
    E = block_counts.numel()
    _expect(block_counts, torch.int32, E, "block_counts")
    _expect(block_offsets, torch.int32, E + 1, "block_offsets")
    _expect(owner, torch.int32, E, "owner")
    _expect_plan_out(out, E, P)
    _expect(status, torch.int32, 1, "status")
    wsp, wsn = _aligned(ws)
    _check(load().moe_plan(_ptr(block_counts), _ptr(block_offsets), _ptr(owner), E, P, s, mode,
                           lam, _ptr(out["q"]), _ptr(out["load"]), _ptr(out["block_worker"]),
                           out["block_worker"].numel(), _ptr(out["plan_info"]), _ptr(status),
                           wsp, wsn, _stream()))
    return out


def alloc_timeline(device):
    """Timeline buffer [TL_PHASES][TIMELINE_MAX_WG][2] of the GPU's 100 MHz counter."""
    return torch.zeros((TL_PHASES, TIMELINE_MAX_WG, 2), dtype=torch.int64, device=device)


def _expect_timeline(timeline):
    if timeline is not None:
        _expect(timeline, torch.int64, TL_PHASES * TIMELINE_MAX_WG * 2, "timeline")


def forward(layer: Layer, x, gates, topk_ids, beta, P, rs, block_worker, y, z_save, ws, status,
            events=None, timeline=None, two_phase=False, split=0, fp8_act=False):
    _require_device(x, gates, topk_ids, y, z_save, ws, status, block_worker, timeline)
    _expect_timeline(timeline)
    T, k = _ids_shape(topk_ids)
    act, E, d, dff = _act_dtype(layer), layer.E, layer.d, layer.d_ff
    _expect(x, act, T * d, "x")
    _expect(gates, torch.float32, T * k, "gates")
    _expect(y, act, T * d, "y")
    if z_save is not None:
        _expect(z_save, act, max_slots(T, k, E, beta) * 2 * dff, "z_save")
    _expect_route(rs, T, k, E, beta)
    _expect(block_worker, torch.int32, max_blocks(T, k, E, beta), "block_worker")
    _expect(status, torch.int32, 1, "status")
    wsp, wsn = _aligned(ws)
    ev = None if events is None else (ctypes.c_void_p * len(events))(*events)
    _check(load().moe_forward(ctypes.byref(layer), _ptr(x), _ptr(gates), _ptr(topk_ids), T, k,
                              beta, P, _ptr(rs["counts"]), _ptr(rs["block_offsets"]),
                              _ptr(rs["row_to_slot"]), _ptr(rs["slot_to_row"]),
                              _ptr(block_worker), _ptr(y), _ptr(z_save), _ptr(status), wsp, wsn,
                              exec_flags(two_phase, split, fp8_act), ev, _ptr(timeline),
                              _stream()))


def backward(layer: Layer, x, gates, dy, z_save, topk_ids, beta, P, s, rs, owner, block_worker,
             dx, dw1, dw2, ws, status, events=None, timeline=None, two_phase=False, split=0,
             fp8_act=False):
    _require_device(x, gates, dy, z_save, topk_ids, owner, block_worker, dx, dw1, dw2, ws, status,
                    timeline)
    _expect_timeline(timeline)
    T, k = _ids_shape(topk_ids)
    act, E, d, dff = _act_dtype(layer), layer.E, layer.d, layer.d_ff
    _expect(x, act, T * d, "x")
    _expect(gates, torch.float32, T * k, "gates")
    _expect(dy, act, T * d, "dy")
    _expect(z_save, act, max_slots(T, k, E, beta) * 2 * dff, "z_save")
    _expect_route(rs, T, k, E, beta)
    _expect(owner, torch.int32, E, "owner")
    _expect(block_worker, torch.int32, max_blocks(T, k, E, beta), "block_worker")
    _expect(dx, act, T * d, "dx")
    _expect(dw1, torch.float32, E * 2 * dff * d, "dw1")
    _expect(dw2, torch.float32, E * d * dff, "dw2")
    _expect(status, torch.int32, 1, "status")
    wsp, wsn = _aligned(ws)
    ev = None if events is None else (ctypes.c_void_p * len(events))(*events)
    _check(load().moe_backward(ctypes.byref(layer), _ptr(x), _ptr(gates), _ptr(dy), _ptr(z_save),
                               _ptr(topk_ids), T, k, beta, P, s, _ptr(rs["counts"]),
                               _ptr(rs["block_offsets"]), _ptr(rs["row_to_slot"]),
                               _ptr(rs["slot_to_row"]), _ptr(owner), _ptr(block_worker), _ptr(dx),
                               _ptr(dw1), _ptr(dw2), _ptr(status), wsp, wsn,
                               exec_flags(two_phase, split, fp8_act), ev, _ptr(timeline),
                               _stream()))


class Events:
    """n hipEvent_t created through the library, for stage timing on the
    stream the kernels run on."""

    def __init__(self, n):
        lib = load()
        self.ev = []
        for _ in range(n):
            p = ctypes.c_void_p()
            _check(lib.moe_event_create(ctypes.byref(p)))
            self.ev.append(p.value)

    def elapsed_ms(self, i, j) -> float:
        ms = ctypes.c_float()
        _check(load().moe_event_elapsed_ms(ctypes.c_void_p(self.ev[i]), ctypes.c_void_p(self.ev[j]),
                                          ctypes.byref(ms)))
        return float(ms.value)

    def record(self, i):
        _check(load().moe_event_record(ctypes.c_void_p(self.ev[i]), _stream()))

    def __del__(self):
        try:
            lib = load()
            for e in self.ev:
                lib.moe_event_destroy(ctypes.c_void_p(e))
        except Exception:
            pass


def device_info():
    a, b, c = _I(), _I(), _I()
    _check(load().moe_device_info(ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return {"num_cus": a.value, "num_xcds": b.value, "gemm_wg_per_cu": c.value}
