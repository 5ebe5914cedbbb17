"""GPU parity of the forward: the HIP path (through the C ABI) against the fp64
oracle on the same seeded inputs, element by element (relative L2 per output
tensor: <= 1e-5 for fp32 I/O, <= 5e-3 for bf16 I/O)."""
import numpy as np
import pytest
import torch

from chunkwise_linear_rnn_gla_amd.inputs import WORKLOADS, make_inputs, workload_inputs
from gpu_util import (PATH_KERNEL, TOL, dtype_name, fwd_path_supported, oracle_fwd, rel_l2,
                      run_fwd, say)

pytestmark = pytest.mark.gpu

# The forward path of the running test (set by the autouse fixture below).
_PATH = {"algo": "auto"}


@pytest.fixture(params=["auto", "fused", "materialized"], autouse=True)
def forward_path(request):
    """Run every forward case through each forward path, requested explicitly
    through gla_fwd_ex: the default (the two-pass chunk prep + recurrence
    wherever it applies), the single-pass fused segment kernel and the
    materialised-state kernels.  A case whose shape a path does not support
    is skipped for that path (the library refuses it rather than running
    another one)."""
    _PATH["algo"] = request.param
    yield request.param
    _PATH["algo"] = "auto"


def skip_unsupported(x, chunk, **cfg):
    algo = _PATH["algo"]
    if not fwd_path_supported(x, chunk, algo, **cfg):
        pytest.skip(f"the {algo} forward does not support dk={x.q.shape[-1]} "
                    f"dv={x.v.shape[-1]} C={chunk} {dtype_name(x)} {cfg or ''}")
    return algo


def check_fwd(x, chunk, tag="", **cfg):
    dt = dtype_name(x)
    algo = skip_unsupported(x, chunk, **cfg)
    say(f"[fwd] {tag} path={algo} dtype={dt} shape={tuple(x.q.shape)} dv={x.v.shape[-1]} "
        f"C={chunk} {cfg or ''}")
    o, hT, names = run_fwd(x, chunk, algo=algo, **cfg)
    if algo in PATH_KERNEL and x.q.shape[2] > 0 and x.q.shape[0] * x.q.shape[1] > 0:
        assert PATH_KERNEL[algo] in names, (algo, names)
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
def test_recurrence_workgroup_shapes(waves, dt, dk, forward_path):
    # 32 (batch, head) pairs: one segment per sequence, 16 state columns per
    # wave and 1, 2 or 4 waves per workgroup (a two-pass setting)
    if forward_path != "auto":
        pytest.skip("recurrence workgroup shapes are a setting of the two-pass forward")
    x = make_inputs(4, 8, 300, dk, 128, dt, seed=320 + waves + dk, h0_std=0.3)
    check_fwd(x, 64, f"recur-waves{waves}", recur_waves=waves)


@pytest.mark.parametrize("dt,dk", [("fp32", 64), ("bf16", 128)])
def test_recurrence_workgroup_shapes_bitwise(dt, dk, forward_path):
    # Each wave of the recurrence owns 16 state columns and runs the same
    # instructions on them whatever the number of waves per workgroup, so with
    # the sequence split the same way (one segment) the outputs are identical
    # to the bit.  (Other settings change the arithmetic: segments re-associate
    # the state sum over chunks, and the fused and materialised forwards order
    # their products differently; those are compared with the oracle.)
    if forward_path != "auto":
        pytest.skip("recurrence workgroup shapes are a setting of the two-pass forward")
    x = make_inputs(2, 4, 300, dk, 128, dt, seed=330 + dk, h0_std=0.3)
    runs = {}
    for waves in (1, 2, 4):
        if not fwd_path_supported(x, 64, "two_pass", recur_waves=waves, recur_segments=1):
            continue
        say(f"[fwd] bitwise recur_waves={waves} dtype={dt} dk={dk}")
        o, hT, names = run_fwd(x, 64, algo="two_pass", recur_waves=waves, recur_segments=1)
        assert "chunk_recur" in names, names
        runs[waves] = (o, hT)
    assert len(runs) >= 2, "fewer than two workgroup shapes to compare"
    (w0, (o0, h0)), *rest = sorted(runs.items())
    for w, (o, h) in rest:
        assert np.array_equal(o, o0), f"o differs between {w0} and {w} waves"
        assert np.array_equal(h, h0), f"hT differs between {w0} and {w} waves"


def _slice(x, a, b, h0):
    """Tokens [a, b) of every sequence, entering with state h0."""
    from chunkwise_linear_rnn_gla_amd.inputs import Inputs
    t = lambda z: z[:, :, a:b].contiguous()
    return Inputs(t(x.q), t(x.k), t(x.v), t(x.log_alpha), h0, None, None)


@pytest.mark.parametrize("dt", ["fp32", "bf16"])
@pytest.mark.parametrize("split", [256, 200])
def test_segment_split_carries_the_state(dt, split, forward_path):
    # A sequence run as two calls, the second entering with the first's final
    # state (papercache.org notes §2.2: the recurrence only needs the previous
    # state; the zako-mio report ch. 4.5 trains this way across segments),
    # against one call and against the oracle.
    x = make_inputs(2, 3, 512, 64, 128, dt, seed=340 + split, h0_std=0.3)
    algo = skip_unsupported(x, 64)

    def split_run(**cfg):
        o1, h1, _ = run_fwd(_slice(x, 0, split, x.h0), 64, algo=algo, **cfg)
        o2, h2, _ = run_fwd(_slice(x, split, 512, torch.from_numpy(h1).float()), 64, algo=algo,
                            **cfg)
        return np.concatenate([o1, o2], axis=2), h2

    say(f"[fwd] segment split at {split} path={algo} dtype={dt}")
    o, hT, _ = run_fwd(x, 64, algo=algo)
    os_, hs = split_run()
    ro, rh = oracle_fwd(x)
    eo, eh = rel_l2(os_, ro), rel_l2(hs, rh)
    say(f"      rel_l2 vs oracle o={eo:.3e} hT={eh:.3e}; vs one call "
        f"o={rel_l2(os_, o):.3e} hT={rel_l2(hs, hT):.3e}")
    assert eo <= TOL[dt] and eh <= TOL[dt]
    assert rel_l2(os_, o) <= TOL[dt] and rel_l2(hs, hT) <= TOL[dt]
    if algo == "two_pass" or (algo == "auto" and fwd_path_supported(x, 64, "two_pass")):
        if split % 64 == 0:
            # On a chunk boundary, with the sequence in one recurrence segment
            # in every call, each chunk sees the same tokens and the same fp32
            # entering state (held in the accumulators, or loaded from h0), so
            # the two-pass forward matches one call to the bit.
            algo = "two_pass"
            o, hT, _ = run_fwd(x, 64, algo=algo, recur_segments=1)
            os_, hs = split_run(recur_segments=1)
            assert np.array_equal(os_, o) and np.array_equal(hs, hT)


def test_single_chunk_and_single_token():
    check_fwd(make_inputs(1, 2, 64, 32, 64, "fp32", seed=304, h0_std=1.0), 64, "L=C")
    check_fwd(make_inputs(1, 2, 1, 32, 64, "fp32", seed=305, h0_std=1.0), 64, "L=1")
    check_fwd(make_inputs(1, 2, 17, 64, 64, "bf16", seed=306, h0_std=1.0), 32, "L=17 bf16")


def test_empty_sequence_copies_h0():
    x = make_inputs(2, 2, 0, 32, 64, "fp32", seed=307, h0_std=1.0)
    o, hT, _ = run_fwd(x, 64, algo=skip_unsupported(x, 64))
    assert o.shape == (2, 2, 0, 64)
    assert np.array_equal(hT, x.h0.double().numpy())
    x = make_inputs(1, 1, 0, 32, 64, "bf16", seed=308)
    _, hT, _ = run_fwd(x, 64, algo=skip_unsupported(x, 64))
    assert not hT.any()


def test_zero_batch():
    x = make_inputs(0, 2, 64, 32, 64, "bf16", seed=309)
    o, hT, _ = run_fwd(x, 64, algo=skip_unsupported(x, 64))
    assert o.shape == (0, 2, 64, 64) and hT.shape == (0, 2, 32, 64)


def test_deterministic():
    x = make_inputs(2, 2, 256, 64, 128, "bf16", seed=310, h0_std=0.2)
    algo = skip_unsupported(x, 64)
    a = run_fwd(x, 64, algo=algo)
    b = run_fwd(x, 64, algo=algo)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.slow
@pytest.mark.parametrize("name", ["gla340m_fwd", "gla1p3b_fwd", "long16k_fwd"])
def test_full_size_workloads(name):
    w = WORKLOADS[name]
    check_fwd(workload_inputs(w), w.chunk, name)


def test_wrong_out_buffer_is_rejected():
    # a caller-supplied output of the wrong dtype or shape never reaches the
    # kernels (they would write past it)
    from chunkwise_linear_rnn_gla_amd import fwd
    d = make_inputs(1, 2, 64, 32, 64, "bf16", seed=312).to("cuda")
    with pytest.raises(TypeError):
        fwd(d.q, d.k, d.v, d.log_alpha, out=torch.empty(1, 2, 64, 64, device="cuda"))
    with pytest.raises(ValueError):
        fwd(d.q, d.k, d.v, d.log_alpha,
            out=torch.empty(1, 2, 32, 64, dtype=torch.bfloat16, device="cuda"))
