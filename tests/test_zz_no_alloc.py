"""moe_route_stats_noalloc -- the routing statistics with the library's own
scratch array instead of a caller workspace -- against moe_route_stats on the
same ids: every output bit for bit, on two calls in a row (the second with a
smaller input, so stale counts of the first would show), and the size limit
refused on the host."""
import ctypes

import numpy as np
import pytest
import torch

from moe_expert_ffn_amd import binding as B
from moe_expert_ffn_amd.inputs import WORKLOADS, make_routing
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def _both(ids_np, E, beta):
    dev = torch.device("cuda")
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).to(dev)
    T, k = ids_np.shape
    ref = B.alloc_route(T, k, E, beta, dev)
    got = B.alloc_route(T, k, E, beta, dev)
    for t in got.values():                            # stale garbage in every output
        t.fill_(-7)
    st_ref = torch.zeros(1, dtype=torch.int32, device=dev)
    st_got = torch.zeros(1, dtype=torch.int32, device=dev)
    lay = B.Layer(E, 128, 64, B.MOE_BF16, B.MOE_BF16, 16, 16, None, None)
    n = int(B.load().moe_workspace_size(ctypes.byref(lay), T, k, beta, 1, 0, 0))
    ws = torch.empty(n + 256, dtype=torch.uint8, device=dev)
    B.route_stats(ids, E, beta, ref, ws, st_ref)
    B.route_stats_noalloc(ids, E, beta, got, st_got)
    torch.cuda.synchronize()
    return ref, got, int(st_ref.item()), int(st_got.item())


def _same(ref, got, T, k, E, beta):
    ms = B.max_slots(T, k, E, beta)
    lim = {"counts": E, "offsets": E + 1, "block_counts": E, "block_offsets": E + 1,
           "row_to_slot": T * k, "slot_to_row": ms, "kappa": 1}
    for name, n in lim.items():
        a, b = ref[name][:n].cpu(), got[name][:n].cpu()
        assert torch.equal(a, b), name


def test_noalloc_route_stats_matches_twice_then_smaller():
    w = WORKLOADS["qwen3_bf16"]
    cases = []
    ids8, _ = make_routing(w, 8)                      # skewed, 65,536 rows
    cases.append((ids8, w.E, w.beta))
    rng = np.random.default_rng(3)
    small = rng.integers(-1, 64, size=(300, 4)).astype(np.int32)   # fewer chunks, E = 64, ids < 0
    cases.append((small, 64, 32))
    for ids_np, E, beta in cases:
        T, k = ids_np.shape
        say(f"[noalloc] T={T} k={k} E={E} beta={beta}")
        ref, got, s_ref, s_got = _both(ids_np, E, beta)
        assert s_ref == s_got == 0
        _same(ref, got, T, k, E, beta)


def test_noalloc_route_stats_flags_bad_expert_like_the_workspace_call():
    ids = np.array([[0, 5], [9, 1], [2, -1]], dtype=np.int32)      # 9 >= E
    ref, got, s_ref, s_got = _both(ids, 8, 4)
    assert s_ref == s_got == B.DEV_BAD_EXPERT
    _same(ref, got, 3, 2, 8, 4)


def test_noalloc_route_stats_refuses_sizes_beyond_its_array():
    lib = B.load()
    P = ctypes.c_void_p(16)
    # ceil(T k / 256) * E * 4 bytes must fit MOE_ROUTE_SCRATCH_BYTES (4 MiB):
    # T k = 2^21 rows at E = 128 is the largest; one chunk more is refused
    E, k = 128, 8
    T_ok = (1 << 21) // k
    T_bad = T_ok + 256 // k
    assert lib.moe_route_stats_noalloc(P, T_bad, k, E, 128, *([P] * 8), None) == B.MOE_ERR_UNSUPPORTED
    with pytest.raises(B.MoeError, match="unsupported"):
        dev = torch.device("cuda")
        ids = torch.zeros((T_bad, k), dtype=torch.int32, device=dev)
        B.route_stats_noalloc(ids, E, 128, B.alloc_route(T_bad, k, E, 128, dev),
                              torch.zeros(1, dtype=torch.int32, device=dev))
