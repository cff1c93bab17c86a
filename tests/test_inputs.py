"""The seeded workload generator: shapes, determinism, skew targets, and the
e4m3 block storage it produces (decoded by the oracle within the format's
half-ulp bound)."""
import numpy as np
import pytest
import torch

from moe_expert_ffn_amd.inputs import (WORKLOADS, Workload, make_layer, make_routing,
                                       realised_kappa)
from oracle.fp8 import dequant_blocks


@pytest.mark.parametrize("name", ["tiny_f32", "olmoe_bf16", "qwen3_bf16", "dsv3_fp8"])
def test_routing_shapes_and_skew(name):
    w = WORKLOADS[name]
    for kap in w.kappas:
        ids, gates = make_routing(w, kap)
        assert ids.dtype == np.int32 and gates.dtype == np.float32
        assert ids.shape[1] == w.k and ((ids >= -1) & (ids < w.E)).all()
        for row in ids:                          # distinct experts within a token
            v = row[row >= 0]
            assert len(set(v.tolist())) == len(v)
        assert (ids >= 0).sum() == w.routed_rows
        if kap:
            assert abs(realised_kappa(ids, w.E) - kap) <= 0.02 * kap
        ids2, gates2 = make_routing(w, kap)
        np.testing.assert_array_equal(ids, ids2)
        np.testing.assert_array_equal(gates, gates2)
    if name != "dsv3_fp8":
        np.testing.assert_allclose(gates.sum(axis=1), 1.0, rtol=1e-5)


def test_fp8_storage_error_bound():
    w = Workload("q", "bf16", "fp8", T=4, k=1, E=2, d=256, d_ff=128, beta=16, P=1, s=0,
                 kappas=(1,), cfg_id=9)
    lay = make_layer(w)
    g = torch.Generator()
    g.manual_seed(1000 * 9 + 1)
    ref = (torch.randn((2, 256, 256), generator=g) / 16.0).double().numpy()
    deq = dequant_blocks(lay["w1"].numpy(), lay["w1_scale"].numpy())
    # e4m3 with 3 mantissa bits: relative error <= 2^-4 above the subnormal range
    scale = np.repeat(np.repeat(lay["w1_scale"].double().numpy(), 128, 1), 128, 2)
    err = np.abs(deq - ref)
    assert (err <= np.maximum(np.abs(ref) * 2.0 ** -4, scale * 2.0 ** -10)).all()
