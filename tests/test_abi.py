"""C ABI on the host (no GPU needed): the library loads, exports every declared
symbol, sizes its workspace, and rejects invalid calls before any HIP call."""
import os
import re

import pytest

import rank_orthonormalized_optimizer_amd as dion
from rank_orthonormalized_optimizer_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "dion.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dion_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = dion.load()
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS), names
    for name in names:
        assert hasattr(lib, name), name


def test_header_enums_match_binding():
    text = open(HEADER).read()
    vals = dict((k, int(v)) for k, v in re.findall(r"\b(DION_\w+)\s*=\s*(-?\d+)", text))
    assert vals["DION_F32"] == _lib.F32 and vals["DION_BF16"] == _lib.BF16
    assert vals["DION_OPT_STICKY_F64"] == _lib.OPT_STICKY_F64 and vals["DION_OPT_FORCE_F64"] == _lib.OPT_FORCE_F64
    assert vals["DION_OPT_FORCE_F32"] == _lib.OPT_FORCE_F32
    assert vals["DION_OPT_HOUSEHOLDER"] == _lib.OPT_HOUSEHOLDER
    assert vals["DION_OPT_SPECTRAL_SHIFT"] == _lib.OPT_SPECTRAL_SHIFT
    assert vals["DION_OPT_EXACT_PRODUCTS"] == _lib.OPT_EXACT_PRODUCTS
    assert vals["DION_FLAG_F64"] == _lib.FLAG_F64 and vals["DION_FLAG_NONFINITE"] == _lib.FLAG_NONFINITE
    assert vals["DION_NUM_PHASES"] == _lib.NUM_PHASES == len(_lib.PHASES)
    for k, v in vals.items():
        if k.startswith("DION_ERR_"):
            assert getattr(_lib, k[5:]) == v, k


def test_workspace_size():
    assert dion.workspace_size(256, 512, 1, 32) > 0
    a = dion.workspace_size(1024, 1024, 24, 256)
    # at least P (fp32 + fp64) and R (fp32 + fp64) for every matrix
    assert a >= 24 * (1024 * 256 * 12 * 2)
    assert dion.workspace_size(1024, 1024, 24, 128) < a
    assert dion.workspace_size(0, 5, 1, 0) == 0
    assert dion.workspace_size(64, 96, 2, 0) > 0      # rank 0 is valid (M <- M + G only)
    assert dion.workspace_size(64, 96, 0, 8) >= 0     # empty stack
    assert dion.workspace_size(4, 5, 1, 5) == 0      # rank > min(m, n)
    assert dion.workspace_size(4, 5, -1, 1) == 0
    assert dion.workspace_size(1 << 45, 1 << 45, 1, 1) == 0


def test_version_and_strerror():
    assert dion.version() >= 100
    for st in (0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -100, -105, 7):
        assert isinstance(dion.strerror(st), str) and dion.strerror(st)


# Fake device addresses: every case below must be rejected by host validation before
# anything is enqueued, so no GPU (and no real memory) is touched.
BASE = 1 << 40
MB = 1 << 20


def call(**kw):
    a = dict(X=BASE, G=BASE + 64 * MB, M=BASE + 128 * MB, Q=BASE + 192 * MB, m=64, n=96, batch=2, rank=8,
             mu=0.95, lr=0.01, eps=1e-8, x_dtype=0, g_dtype=0, workspace=BASE + 256 * MB,
             workspace_bytes=1 << 30, flags=0, options=0, stream=0)
    a.update(kw)
    return _lib.step_batched_raw(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(m=0), _lib.ERR_SHAPE),
    (dict(n=-3), _lib.ERR_SHAPE),
    (dict(batch=-1), _lib.ERR_SHAPE),
    (dict(rank=65), _lib.ERR_RANK),
    (dict(rank=-1), _lib.ERR_RANK),
    (dict(mu=1.0), _lib.ERR_HYPER),
    (dict(mu=-0.1), _lib.ERR_HYPER),
    (dict(lr=float("nan")), _lib.ERR_HYPER),
    (dict(eps=-1e-8), _lib.ERR_HYPER),
    (dict(eps=float("inf")), _lib.ERR_HYPER),
    (dict(x_dtype=2), _lib.ERR_DTYPE),
    (dict(g_dtype=-1), _lib.ERR_DTYPE),
    (dict(options=8), _lib.ERR_OPTION),
    (dict(options=_lib.OPT_FORCE_F32 | _lib.OPT_FORCE_F64), _lib.ERR_OPTION),
    (dict(options=_lib.OPT_HOUSEHOLDER | _lib.OPT_FORCE_F32), _lib.ERR_OPTION),
    (dict(options=_lib.OPT_HOUSEHOLDER, m=4097, n=4097, batch=1, rank=4097), _lib.ERR_OPTION),
    (dict(options=128), _lib.ERR_OPTION),
    (dict(options=_lib.OPT_SPECTRAL_SHIFT | _lib.OPT_FORCE_F32), _lib.ERR_OPTION),
    (dict(X=0), _lib.ERR_NULL),
    (dict(Q=0), _lib.ERR_NULL),
    (dict(workspace=0), _lib.ERR_NULL),
    (dict(M=BASE + 128 * MB + 4), _lib.ERR_ALIGN),
    (dict(flags=BASE + 300 * MB + 8), _lib.ERR_ALIGN),
    (dict(workspace=BASE + 256 * MB + 16), _lib.ERR_ALIGN),
    (dict(workspace_bytes=1024), _lib.ERR_WORKSPACE),
    (dict(G=BASE + 1024), _lib.ERR_OVERLAP),
    (dict(Q=BASE + 128 * MB + 4096), _lib.ERR_OVERLAP),
    (dict(flags=BASE + 256 * MB + 512), _lib.ERR_OVERLAP),
])
def test_invalid_calls_rejected_on_host(kw, status):
    assert call(**kw) == status


def test_empty_batch_is_a_noop():
    assert call(batch=0, X=0, G=0, M=0, Q=0, workspace=0) == _lib.OK


def test_rank_zero_needs_no_q_but_still_validates():
    assert call(rank=0, Q=0, m=0) == _lib.ERR_SHAPE
    assert call(rank=0, Q=0, workspace_bytes=0) == _lib.ERR_WORKSPACE


def test_group_matrices_rejects_1d():
    import torch
    ps = [torch.zeros(4, 5), torch.zeros(4, 5), torch.zeros(3, 3, dtype=torch.bfloat16)]
    g = dion.group_matrices(ps)
    assert list(g) == [((4, 5), torch.float32), ((3, 3), torch.bfloat16)]
    assert len(g[((4, 5), torch.float32)]) == 2
    with pytest.raises(ValueError, match="only 2-D"):
        dion.group_matrices([torch.zeros(4, 5), torch.zeros(5)])


def adamw(**kw):
    a = dict(param=BASE, grad=BASE + 64 * MB, exp_avg=BASE + 128 * MB, exp_avg_sq=BASE + 192 * MB, n=1000, t=1,
             lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, p_dtype=0, g_dtype=0, stream=0)
    a.update(kw)
    return _lib.adamw_step_raw(**a)


def lion(**kw):
    a = dict(param=BASE, grad=BASE + 64 * MB, exp_avg=BASE + 128 * MB, n=1000, lr=1e-4, beta1=0.9, beta2=0.99,
             weight_decay=0.0, p_dtype=0, g_dtype=0, stream=0)
    a.update(kw)
    return _lib.lion_step_raw(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(n=-1), _lib.ERR_SHAPE),
    (dict(t=0), _lib.ERR_HYPER),
    (dict(beta1=1.0), _lib.ERR_HYPER),
    (dict(beta2=-0.5), _lib.ERR_HYPER),
    (dict(eps=-1.0), _lib.ERR_HYPER),
    (dict(lr=float("inf")), _lib.ERR_HYPER),
    (dict(weight_decay=float("nan")), _lib.ERR_HYPER),
    (dict(p_dtype=3), _lib.ERR_DTYPE),
    (dict(param=0), _lib.ERR_NULL),
    (dict(exp_avg_sq=0), _lib.ERR_NULL),
    (dict(grad=BASE + 64 * MB + 8), _lib.ERR_ALIGN),
    (dict(grad=BASE + 2048), _lib.ERR_OVERLAP),
    (dict(exp_avg_sq=BASE + 128 * MB + 1024), _lib.ERR_OVERLAP),
])
def test_adamw_invalid_calls_rejected_on_host(kw, status):
    assert adamw(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(n=-1), _lib.ERR_SHAPE),
    (dict(beta1=-0.1), _lib.ERR_HYPER),
    (dict(beta2=1.0), _lib.ERR_HYPER),
    (dict(lr=float("nan")), _lib.ERR_HYPER),
    (dict(g_dtype=7), _lib.ERR_DTYPE),
    (dict(exp_avg=0), _lib.ERR_NULL),
    (dict(param=BASE + 4), _lib.ERR_ALIGN),
    (dict(exp_avg=BASE + 1024), _lib.ERR_OVERLAP),
])
def test_lion_invalid_calls_rejected_on_host(kw, status):
    assert lion(**kw) == status


def test_elementwise_empty_is_a_noop():
    assert adamw(n=0, param=0, grad=0, exp_avg=0, exp_avg_sq=0) == _lib.OK
    assert lion(n=0, param=0, grad=0, exp_avg=0) == _lib.OK


def lam(**kw):
    a = dict(W=BASE, r=256, batch=4, V0=0, k=32, iters=10, lam=BASE + 64 * MB, workspace=BASE + 128 * MB,
             workspace_bytes=_lib.lambda_max_workspace_size(256, 4, 32), stream=0)
    a.update(kw)
    return _lib.lambda_max_raw(**a)


def test_lambda_max_workspace_size():
    assert _lib.lambda_max_workspace_size(256, 4, 32) == 4 * (2 * 256 * 32 + 2) * 8
    assert _lib.lambda_max_workspace_size(7, 3, 5) == 3 * (2 * 7 * 5 + 2) * 8
    assert _lib.lambda_max_workspace_size(256, 0, 32) == 0
    for bad in ((0, 4, 32), (256, -1, 32), (256, 4, 0), (256, 4, 33), (256, 65536, 1)):
        assert _lib.lambda_max_workspace_size(*bad) == 0, bad


@pytest.mark.parametrize("kw,status", [
    (dict(r=0), _lib.ERR_SHAPE),
    (dict(batch=-1), _lib.ERR_SHAPE),
    (dict(batch=65536), _lib.ERR_SHAPE),
    (dict(k=0), _lib.ERR_SHAPE),
    (dict(k=33), _lib.ERR_SHAPE),
    (dict(iters=-1), _lib.ERR_HYPER),
    (dict(iters=65), _lib.ERR_HYPER),
    (dict(W=0), _lib.ERR_NULL),
    (dict(lam=0), _lib.ERR_NULL),
    (dict(workspace=0), _lib.ERR_NULL),
    (dict(W=BASE + 4), _lib.ERR_ALIGN),
    (dict(V0=BASE + 32 * MB + 12), _lib.ERR_ALIGN),
    (dict(workspace=BASE + 128 * MB + 64), _lib.ERR_ALIGN),
    (dict(workspace_bytes=1000), _lib.ERR_WORKSPACE),
    (dict(lam=BASE + 8), _lib.ERR_OVERLAP),                 # inside W
    (dict(lam=BASE + 128 * MB + 4096), _lib.ERR_OVERLAP),   # inside the workspace
    (dict(V0=BASE + 128 * MB), _lib.ERR_OVERLAP),           # start vectors in the workspace
])
def test_lambda_max_invalid_calls_rejected_on_host(kw, status):
    assert lam(**kw) == status


def test_lambda_max_empty_batch_is_a_noop():
    assert lam(batch=0, W=0, lam=0, workspace=0, workspace_bytes=0) == _lib.OK
