"""CPU tests of the C ABI: the library loads, exports every symbol that
include/gla.h declares, and rejects bad arguments before enqueueing anything.
No call here reaches a kernel launch (each one fails validation first)."""
import ctypes
import os
import re

import pytest

from chunkwise_linear_rnn_gla_amd import _abi
from chunkwise_linear_rnn_gla_amd._abi import GLA_BF16, GLA_FP32, GlaDims

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gla.h")

FAKE = 0x10000  # a 16-byte aligned non-null address; never dereferenced here


@pytest.fixture(scope="module")
def lib():
    return _abi.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(g?gla_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(_abi.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert _abi.gla_abi_version() == 2
    for s in range(7):
        assert _abi.status_string(s) and _abi.status_string(s) != "unknown status"
    assert _abi.status_string(99) == "unknown status"


def good_dims(**kw):
    d = dict(B=2, H=4, L=2048, dk=128, dv=256, chunk=64, subchunk=16)
    d.update(kw)
    return GlaDims(**d)


def ws_status(d, dtype):
    n = ctypes.c_size_t(0)
    return _abi.load().gla_fwd_workspace_size(ctypes.byref(d), dtype, ctypes.byref(n)), n.value


def test_workspace_size_valid_and_monotone():
    st, n1 = ws_status(good_dims(L=1024), GLA_BF16)
    st2, n2 = ws_status(good_dims(L=2048), GLA_BF16)
    assert st == 0 and st2 == 0 and 0 < n1 < n2
    assert _abi.gla_bwd_workspace_size(good_dims(), GLA_BF16) > _abi.gla_fwd_workspace_size(
        good_dims(), GLA_BF16)


@pytest.mark.parametrize("kw,dtype", [
    (dict(chunk=48), GLA_BF16),
    (dict(chunk=16), GLA_BF16),      # bf16 needs chunk 32 or 64
    (dict(chunk=128), GLA_FP32),
    (dict(subchunk=8), GLA_FP32),
    (dict(dk=48), GLA_BF16),         # bf16 needs multiples of 32
    (dict(dk=40), GLA_FP32),
    (dict(dv=1024), GLA_BF16),
    (dict(dk=512), GLA_FP32),
    (dict(L=-1), GLA_FP32),
    (dict(B=-2), GLA_FP32),
    (dict(B=256, H=257), GLA_FP32),  # B * H is a grid dimension: at most 65535
])
def test_shape_errors(kw, dtype):
    st, _ = ws_status(good_dims(**kw), dtype)
    assert st == 2  # GLA_ERR_SHAPE
    st = _abi.gla_fwd(good_dims(**kw), dtype, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE,
                      1 << 40, None)
    assert st == 2


def test_dtype_error():
    assert ws_status(good_dims(), 7)[0] == 3
    assert _abi.gla_fwd(good_dims(), 2, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, 1 << 40,
                        None) == 3


def test_null_errors():
    lib = _abi.load()
    n = ctypes.c_size_t(0)
    assert lib.gla_fwd_workspace_size(None, GLA_BF16, ctypes.byref(n)) == 1
    assert lib.gla_fwd_workspace_size(ctypes.byref(good_dims()), GLA_BF16, None) == 1
    d = good_dims()
    for i in range(5):  # q, k, v, log_alpha, o are required
        args = [FAKE] * 5
        args[i] = None
        q, k, v, a, o = args
        assert _abi.gla_fwd(d, GLA_BF16, q, k, v, a, None, o, None, FAKE, 1 << 40, None) == 1
    bargs = [FAKE] * 9  # q k v a dout dq dk dv dla
    for i in range(9):
        a = list(bargs)
        a[i] = None
        q, k, v, la, do, dq, dk, dv, dla = a
        assert _abi.gla_bwd(d, GLA_BF16, q, k, v, la, None, do, None, dq, dk, dv, dla, None,
                            FAKE, 1 << 40, None) == 1


def test_alignment_errors():
    d = good_dims()
    bad = FAKE + 8
    assert _abi.gla_fwd(d, GLA_BF16, bad, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, 1 << 40,
                        None) == 4
    assert _abi.gla_fwd(d, GLA_BF16, FAKE, FAKE, FAKE, FAKE, bad, FAKE, None, FAKE, 1 << 40,
                        None) == 4   # optional h0 misaligned
    assert _abi.gla_fwd(d, GLA_BF16, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, bad, 1 << 40,
                        None) == 4   # workspace misaligned


def test_workspace_errors():
    d = good_dims()
    need = _abi.gla_fwd_workspace_size(d, GLA_BF16)
    assert _abi.gla_fwd(d, GLA_BF16, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None, need,
                        None) == 5
    assert _abi.gla_fwd(d, GLA_BF16, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, need - 1,
                        None) == 5
    needb = _abi.gla_bwd_workspace_size(d, GLA_BF16)
    assert _abi.gla_bwd(d, GLA_BF16, *([FAKE] * 4), None, FAKE, None, *([FAKE] * 4), None,
                        FAKE, needb - 1, None) == 5


def test_empty_batch_is_a_no_op():
    # B * H == 0: nothing to do, nothing launched, pointers not required
    d = good_dims(B=0)
    assert _abi.gla_fwd(d, GLA_BF16, None, None, None, None, None, None, None, None, 0, None) == 0
    assert _abi.gla_bwd(d, GLA_BF16, *([None] * 12), None, 0, None) == 0


def test_decode_errors():
    # validation of the one-token step happens before any launch
    d = good_dims(L=0, chunk=0, subchunk=0)  # sequence and chunk fields are not used
    assert _abi.gla_decode(d, 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 3
    assert _abi.load().gla_decode(None, GLA_BF16, *([FAKE] * 6), None) == 1
    assert _abi.gla_decode(good_dims(dk=20), GLA_BF16, *([FAKE] * 6), None) == 2
    assert _abi.gla_decode(good_dims(dv=1024), GLA_FP32, *([FAKE] * 6), None) == 2
    assert _abi.gla_decode(d, GLA_BF16, FAKE, FAKE, None, FAKE, FAKE, FAKE, None) == 1
    assert _abi.gla_decode(d, GLA_BF16, FAKE, FAKE, FAKE, FAKE, FAKE + 8, FAKE, None) == 4
    assert _abi.gla_decode(good_dims(B=0), GLA_BF16, *([None] * 6), None) == 0


def test_general_gate_errors():
    # ggla_*: validation happens before any launch; chunk fields are not used
    d = good_dims(L=64, chunk=0, subchunk=0)
    n_fwd = _abi.ggla_fwd_workspace_size(d, GLA_BF16)
    n_bwd = _abi.ggla_bwd_workspace_size(d, GLA_BF16)
    assert 0 < n_fwd < n_bwd
    args = [FAKE] * 5 + [None, FAKE, None]
    assert _abi.ggla_fwd(d, 2, *args, FAKE, n_fwd, None) == 3
    assert _abi.load().ggla_fwd(None, GLA_BF16, *([FAKE] * 8), FAKE, n_fwd, None) == 1
    assert _abi.ggla_fwd(good_dims(dv=544), GLA_BF16, *args, FAKE, n_fwd, None) == 2
    assert _abi.ggla_fwd(good_dims(dk=512), GLA_BF16, *args, FAKE, n_fwd, None) == 2
    assert _abi.ggla_fwd(good_dims(dk=48), GLA_BF16, *args, FAKE, n_fwd, None) == 2
    assert _abi.ggla_fwd(good_dims(B=300, H=300), GLA_BF16, *args, FAKE, n_fwd, None) == 2
    assert _abi.ggla_fwd(d, GLA_BF16, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None, FAKE,
                         n_fwd, None) == 1
    assert _abi.ggla_fwd(d, GLA_BF16, FAKE, FAKE, FAKE, FAKE, FAKE + 4, None, FAKE, None, FAKE,
                         n_fwd, None) == 4
    assert _abi.ggla_fwd(d, GLA_BF16, *args, FAKE, n_fwd - 1, None) == 5
    bargs = [FAKE] * 5 + [None, FAKE, None] + [FAKE] * 5 + [None]
    assert _abi.ggla_bwd(d, GLA_BF16, *bargs, FAKE, n_bwd - 1, None) == 5
    bad = list(bargs)
    bad[12] = None  # dlog_beta
    assert _abi.ggla_bwd(d, GLA_BF16, *bad, FAKE, n_bwd, None) == 1
    assert _abi.ggla_fwd(good_dims(B=0), GLA_BF16, *([None] * 8), None, 0, None) == 0
    assert _abi.ggla_bwd(good_dims(B=0), GLA_BF16, *([None] * 14), None, 0, None) == 0


def cfg_status(d, dtype, algo, waves=0, segs=0):
    n = ctypes.c_size_t(0)
    c = _abi.GlaFwdConfig(algo, waves, segs)
    return _abi.load().gla_fwd_ex_workspace_size(ctypes.byref(d), dtype, ctypes.byref(c),
                                                 ctypes.byref(n)), n.value


def test_forward_config_validation():
    d = good_dims()
    st_auto, n_auto = cfg_status(d, GLA_BF16, _abi.GLA_FWD_AUTO)
    st_two, n_two = cfg_status(d, GLA_BF16, _abi.GLA_FWD_TWO_PASS)
    st_mat, n_mat = cfg_status(d, GLA_BF16, _abi.GLA_FWD_MATERIALIZED)
    st_fus, n_fus = cfg_status(d, GLA_BF16, _abi.GLA_FWD_FUSED)
    assert st_auto == st_two == st_mat == st_fus == 0
    # the automatic choice is the two-pass forward here, and gla_fwd's query
    # agrees with gla_fwd_ex's for a NULL config
    assert n_auto == n_two == _abi.gla_fwd_workspace_size(d, GLA_BF16)
    n = ctypes.c_size_t(0)
    assert _abi.load().gla_fwd_ex_workspace_size(ctypes.byref(d), GLA_BF16, None,
                                                 ctypes.byref(n)) == 0 and n.value == n_auto
    # the materialised states need more workspace than the two-pass records
    assert n_mat > n_two > 0 and n_fus > 0
    # requested paths and settings the shape does not support are refused
    assert cfg_status(good_dims(dk=32), GLA_BF16, _abi.GLA_FWD_FUSED)[0] == 2   # fused: dk 64+
    assert cfg_status(good_dims(chunk=32), GLA_BF16, _abi.GLA_FWD_FUSED)[0] == 2
    assert cfg_status(d, GLA_BF16, 7)[0] == 2
    assert cfg_status(d, GLA_BF16, -1)[0] == 2
    assert cfg_status(d, GLA_BF16, _abi.GLA_FWD_TWO_PASS, waves=3)[0] == 2
    assert cfg_status(good_dims(dk=256), GLA_BF16, _abi.GLA_FWD_TWO_PASS, waves=1)[0] == 2
    assert cfg_status(d, GLA_BF16, _abi.GLA_FWD_MATERIALIZED, waves=2)[0] == 2
    assert cfg_status(d, GLA_BF16, _abi.GLA_FWD_FUSED, segs=2)[0] == 2
    assert cfg_status(d, GLA_BF16, _abi.GLA_FWD_TWO_PASS, segs=-1)[0] == 2
    for w in (1, 2, 4):
        assert cfg_status(d, GLA_BF16, _abi.GLA_FWD_TWO_PASS, waves=w)[0] == 0
    # more recurrence segments need more workspace (segment states)
    st1, n1 = cfg_status(d, GLA_BF16, _abi.GLA_FWD_TWO_PASS, segs=1)
    st4, n4 = cfg_status(d, GLA_BF16, _abi.GLA_FWD_TWO_PASS, segs=4)
    assert st1 == st4 == 0 and n4 > n1
    # gla_fwd_ex validates like the query, before anything is launched
    c = _abi.GlaFwdConfig(_abi.GLA_FWD_FUSED, 0, 0)
    assert _abi.gla_fwd_ex(good_dims(dk=32), GLA_BF16, c, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                           None, FAKE, 1 << 40, None) == 2
    assert _abi.gla_fwd_ex(d, GLA_BF16, None, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE,
                           n_auto - 1, None) == 5


def test_python_argument_checks_before_any_call():
    """The binding rejects buffers the kernels would misuse (the C side sees
    only pointers): wrong dtype, shape, layout or device of an output."""
    import torch
    from chunkwise_linear_rnn_gla_amd import _check, fwd_config
    o = torch.empty(2, 3, 5, 8, dtype=torch.bfloat16)
    _check(o, "out", torch.bfloat16, (2, 3, 5, 8), o.device, require_device=False)
    with pytest.raises(TypeError):
        _check(o, "out", torch.float32, (2, 3, 5, 8), o.device, require_device=False)
    with pytest.raises(ValueError):
        _check(o, "out", torch.bfloat16, (2, 3, 5, 16), o.device, require_device=False)
    with pytest.raises(ValueError):
        _check(o.transpose(2, 3), "out", torch.bfloat16, None, o.device, require_device=False)
    with pytest.raises(ValueError):
        _check(o, "out", torch.bfloat16, (2, 3, 5, 8), torch.device("meta"),
               require_device=False)
    with pytest.raises(ValueError):
        _check(o, "out", torch.bfloat16, (2, 3, 5, 8))   # not a device tensor
    with pytest.raises(ValueError):
        fwd_config("bogus")
    c = fwd_config("two_pass", recur_waves=2, recur_segments=3)
    assert (c.algo, c.recur_waves, c.recur_segments) == (_abi.GLA_FWD_TWO_PASS, 2, 3)


def test_noalloc_forward_rejects_before_any_device_call():
    # sizes are validated before the entry point touches the device: shapes
    # outside the two-pass forward, and records beyond the static scratch
    text = open(HEADER).read()
    limit = int(re.search(r"#define GLA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
                .group(1)) << int(re.search(r"<< (\d+)\)", text).group(1))
    big = good_dims(B=16)
    assert _abi.gla_fwd_ex_workspace_size(big, GLA_BF16, _abi.GlaFwdConfig(1, 0, 0)) > limit
    assert _abi.gla_fwd_ex_workspace_size(good_dims(B=8), GLA_BF16,
                                          _abi.GlaFwdConfig(1, 0, 0)) <= limit
    assert _abi.gla_fwd_noalloc(big, GLA_BF16, FAKE, FAKE, FAKE, FAKE, None, FAKE, None,
                                None) == 5
    assert _abi.gla_fwd_noalloc(good_dims(dk=256), GLA_FP32, FAKE, FAKE, FAKE, FAKE, None,
                                FAKE, None, None) == 2
    assert _abi.gla_fwd_noalloc(good_dims(), 9, FAKE, FAKE, FAKE, FAKE, None, FAKE, None,
                                None) == 3
    assert _abi.load().gla_fwd_noalloc(None, GLA_BF16, *([FAKE] * 7), None) == 1
