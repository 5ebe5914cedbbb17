"""GPU parity of the forward: the HIP path (through the C ABI) against the fp64
oracle on the same seeded inputs, element by element (relative L2 per output
tensor: <= 1e-5 for fp32 I/O, <= 5e-3 for bf16 I/O)."""
import os

import numpy as np
import pytest
import torch

from chunkwise_linear_rnn_gla_amd.inputs import WORKLOADS, make_inputs, workload_inputs
from gpu_util import TOL, dtype_name, oracle_fwd, rel_l2, run_fwd, say

pytestmark = pytest.mark.gpu


@pytest.fixture(params=["auto", "fused", "materialized"], autouse=True)
def forward_path(request, monkeypatch):
    """Run every forward case through each forward path: the default (the
    two-pass chunk prep + recurrence wherever it applies), the single-pass
    fused segment kernel (GLA_FORWARD=fused, where it applies) and the
    materialised-state kernels (GLA_FORWARD=materialized)."""
    if request.param == "auto":
        monkeypatch.delenv("GLA_FORWARD", raising=False)
    else:
        monkeypatch.setenv("GLA_FORWARD", request.param)
    return request.param


def check_fwd(x, chunk, tag=""):
    dt = dtype_name(x)
    say(f"[fwd] {tag} dtype={dt} shape={tuple(x.q.shape)} dv={x.v.shape[-1]} C={chunk}")
    o, hT = run_fwd(x, chunk)
    ro, rh = oracle_fwd(x)
    eo, eh = rel_l2(o, ro), rel_l2(hT, rh)
    say(f"      rel_l2 o={eo:.3e} hT={eh:.3e}")
    assert np.isfinite(o).all() and np.isfinite(hT).all()
    assert eo <= TOL[dt], f"o rel_l2 {eo}"
    assert eh <= TOL[dt], f"hT rel_l2 {eh}"
    return eo, eh


def test_tiny_fp32_workload():
    w = WORKLOADS["tiny_fp32"]
    check_fwd(workload_inputs(w), w.chunk, "tiny_fp32")


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("dk,dv", [(16, 32), (48, 80), (64, 128)])
def test_fp32_tiles_and_ragged_tail(C, dk, dv):
    x = make_inputs(2, 3, 200, dk, dv, "fp32", seed=100 + C + dk, h0_std=0.5)
    check_fwd(x, C, "fp32-ragged")


@pytest.mark.parametrize("C", [32, 64])
@pytest.mark.parametrize("dk,dv", [(32, 64), (64, 96), (128, 256)])
def test_bf16_tiles_and_ragged_tail(C, dk, dv):
    x = make_inputs(2, 2, 300, dk, dv, "bf16", seed=200 + C + dk, h0_std=0.3)
    check_fwd(x, C, "bf16-ragged")


def test_bf16_max_head_dims():
    x = make_inputs(1, 2, 130, 256, 512, "bf16", seed=301, h0_std=0.1)
    check_fwd(x, 64, "bf16-max-dims")


@pytest.mark.parametrize("dt", ["fp32", "bf16"])
def test_segmented_state_recurrence(dt):
    # few (batch, head) tiles and many chunks: the state recurrence runs as
    # per-segment local states + a scan over segments + a fill pass
    x = make_inputs(1, 1, 1000, 32, 64, dt, seed=302, h0_std=0.4)
    check_fwd(x, 32, "segmented")


@pytest.mark.parametrize("gate", ["zero", "extreme", "const", "channel_const"])
@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 128)])
def test_gate_edge_cases(gate, dk, dv):
    x = make_inputs(2, 2, 192, dk, dv, "fp32", seed=303, gate=gate, h0_std=0.2,
                    gate_value=-0.3)
    check_fwd(x, 64, f"gate-{gate}")


@pytest.mark.parametrize("dt,dk,dv,L", [("fp32", 64, 128, 1000), ("fp32", 128, 128, 333),
                                        ("bf16", 128, 256, 700), ("bf16", 64, 256, 1100),
                                        ("bf16", 256, 512, 450)])
def test_fused_segments(dt, dk, dv, L):
    # few heads, many chunks: the fused forward splits the sequence into
    # segments whose entry states come from the local-state pass and scan
    x = make_inputs(1, 2, L, dk, dv, dt, seed=311 + dk + L, h0_std=0.3)
    check_fwd(x, 64, "fused-segments")


@pytest.mark.parametrize("waves", [1, 2, 4])
@pytest.mark.parametrize("dt,dk", [("fp32", 64), ("bf16", 128)])
def test_recurrence_workgroup_shapes(waves, dt, dk, monkeypatch):
    # 32 (batch, head) pairs: one segment per sequence, 16 state columns per
    # wave and 1, 2 or 4 waves per workgroup
    monkeypatch.setenv("GLA_RECUR_WAVES", str(waves))
    x = make_inputs(4, 8, 300, dk, 128, dt, seed=320 + waves + dk, h0_std=0.3)
    check_fwd(x, 64, f"recur-waves{waves}")


def test_single_chunk_and_single_token():
    check_fwd(make_inputs(1, 2, 64, 32, 64, "fp32", seed=304, h0_std=1.0), 64, "L=C")
    check_fwd(make_inputs(1, 2, 1, 32, 64, "fp32", seed=305, h0_std=1.0), 64, "L=1")
    check_fwd(make_inputs(1, 2, 17, 64, 64, "bf16", seed=306, h0_std=1.0), 32, "L=17 bf16")


def test_empty_sequence_copies_h0():
    x = make_inputs(2, 2, 0, 32, 64, "fp32", seed=307, h0_std=1.0)
    o, hT = run_fwd(x, 64)
    assert o.shape == (2, 2, 0, 64)
    assert np.array_equal(hT, x.h0.double().numpy())
    x = make_inputs(1, 1, 0, 32, 64, "bf16", seed=308)
    _, hT = run_fwd(x, 64)
    assert not hT.any()


def test_zero_batch():
    x = make_inputs(0, 2, 64, 32, 64, "bf16", seed=309)
    o, hT = run_fwd(x, 64)
    assert o.shape == (0, 2, 64, 64) and hT.shape == (0, 2, 32, 64)


def test_deterministic():
    x = make_inputs(2, 2, 256, 64, 128, "bf16", seed=310, h0_std=0.2)
    a = run_fwd(x, 64)
    b = run_fwd(x, 64)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.slow
@pytest.mark.parametrize("name", ["gla340m_fwd", "gla1p3b_fwd", "long16k_fwd"])
def test_full_size_workloads(name):
    w = WORKLOADS[name]
    check_fwd(workload_inputs(w), w.chunk, name)
