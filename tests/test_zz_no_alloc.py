"""The allocation-free entry point (sgmv_lora_add_host_ids_noalloc), through the C ABI:
its output equals the workspace-taking sgmv_lora_add_host_ids bit for bit (same kernel)
and the fp64 oracle within tolerance, on consecutive calls that share the library's
static scratch, the later ones on smaller inputs."""
import sys

import numpy as np
import pytest

import oracle
from workloads import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _storage(y, dtype):
    from adapter_gemv_amd.device_problem import to_numpy_storage
    return to_numpy_storage(y, dtype)


def _noalloc(dp, y, ids):
    from adapter_gemv_amd import _lib, sgmv
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    st = sgmv.sgmv_lora_add_host_ids_noalloc(
        sgmv._stream_handle(), sgmv.dtype_code(y), y.data_ptr(), y.stride(0), dp.x.data_ptr(),
        dp.x.stride(0), ids.ctypes.data, int(ids.shape[0]), dp.A.data_ptr(), dp.A.stride(0),
        dp.B.data_ptr(), dp.B.stride(0), int(dp.A.shape[0]), int(dp.x.shape[1]),
        int(y.shape[1]), int(dp.A.shape[1]), dp.scale)
    assert st == _lib.OK, _lib.status_string(st)
    return y


def test_noalloc_equals_workspace_call_on_consecutive_calls(torch_cuda):
    torch = torch_cuda
    from adapter_gemv_amd.device_problem import DeviceProblem
    problems = [
        synth.decode7b(),                                                   # 32 x 4096 -> 4096
        synth.random_problem((97, 1), n=5, h_in=1032, h_out=520, r=64, n_adapters=3,
                             dtype="bf16", id_dist="uniform"),              # smaller, r = 64
        synth.random_problem((97, 2), n=3, h_in=264, h_out=136, r=16, n_adapters=2,
                             dtype="f16", id_dist="uniform"),               # smaller still
    ]
    for i, p in enumerate(problems):
        _say(f"[noalloc] call {i}: {p.name} n={p.n} h_in={p.h_in} h_out={p.h_out} r={p.r} {p.dtype}")
        dp = DeviceProblem.upload(p)
        y_ws = dp.lora_add_host_ids()          # the existing entry point, fresh workspace
        y_na = _noalloc(dp, dp.fresh_y(), p.ids)
        torch.cuda.synchronize()
        assert torch.equal(y_na, y_ws), f"call {i}: differs from sgmv_lora_add_host_ids"
        ref = oracle.lora_add_problem(p)
        got = oracle.decode(_storage(y_na, p.dtype), p.dtype)
        err = np.abs(got - ref)
        tol = 1e-2 + 1e-2 * np.abs(ref)
        _say(f"[noalloc] call {i}: max|err| {err.max():.3e}")
        assert np.all(err <= tol)
    # the first shape again: the scratch the smaller calls used is back at zero
    p = problems[0]
    dp = DeviceProblem.upload(p)
    y_na = _noalloc(dp, dp.fresh_y(), p.ids)
    y_ws = dp.lora_add_host_ids()
    torch.cuda.synchronize()
    assert torch.equal(y_na, y_ws)
