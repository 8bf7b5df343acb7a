"""On-demand adapter loading (AdapterPool: the native slot cache + sgmv_upload_adapter from
pinned host copies) and stacked multi-layer pools, on the GPU, against the fp64 oracle:
every batch's result uses exactly the adapters its keys name, whichever slots they landed
in, after evictions and re-registrations."""
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


def _assert_close(got, ref, what):
    err = np.abs(got - ref)
    tol = 1e-2 + 1e-2 * np.abs(ref)
    _say(f"{what}: max|err| {err.max():.3e}, worst err/tol {np.max(err / tol):.3f}")
    assert np.all(err <= tol), f"{what}: {int((err > tol).sum())} outside tolerance"


def _storage(y, dtype):
    from adapter_gemv_amd.device_problem import to_numpy_storage
    return to_numpy_storage(y, dtype)


def _stacked_adapters(seed, layers, P, r, h_in, h_out, dtype):
    """Adapters of ``layers`` layers in the generator's storage format: A [layers, P, r, h_in],
    B [layers, P, h_out, r] (each layer drawn like one projection's pool)."""
    As, Bs = [], []
    for layer in range(layers):
        p = synth.random_problem((seed, layer), n=1, h_in=h_in, h_out=h_out, r=r, n_adapters=P,
                                 dtype=dtype, ids=np.zeros(1, np.int32))
        As.append(p.A)
        Bs.append(p.B)
    return np.stack(As), np.stack(Bs)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_adapter_pool_on_demand_batches(torch_cuda, dtype):
    torch = torch_cuda
    from adapter_gemv_amd import sgmv
    from adapter_gemv_amd.adapter_pool import AdapterPool
    layers, n_keys, r, h_in, h_out = 2, 10, 16, 1032, 520
    A_all, B_all = _stacked_adapters(60, layers, n_keys, r, h_in, h_out, dtype)
    keys = [1000 + 17 * i for i in range(n_keys)]          # arbitrary adapter keys
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    pool = AdapterPool(6, r, h_in, h_out, layers=layers, dtype=tdt)
    for i, k in enumerate(keys):
        pool.register(k, sgmv.as_tensor(A_all[:, i], dtype), sgmv.as_tensor(B_all[:, i], dtype))
    rng = np.random.default_rng(61)
    # batches of 12 (one launch, host ids) and 150 (device ids) tokens over 1..6 distinct
    # adapters each: later batches evict what earlier ones loaded
    plan = [(12, [0, 1, 2]), (12, [3, 4, 5, 0]), (150, [6, 7, 1]), (12, [8, 9, 2, 3, 4, 6]),
            (150, [0, 1, 2, 3, 4, 5]), (12, [9])]
    for b, (n, which) in enumerate(plan):
        idx = np.asarray(which)[rng.integers(0, len(which), n)].astype(np.int32)
        p = synth.random_problem((62, b), n=n, h_in=h_in, h_out=h_out, r=r, n_adapters=1,
                                 dtype=dtype, ids=np.zeros(n, np.int32), scale=1.5)
        x = sgmv.as_tensor(p.x, dtype, "cuda")
        slots = pool.prepare([keys[i] for i in idx])
        for layer in range(layers):
            y = sgmv.as_tensor(p.y, dtype, "cuda")
            pool.lora_add(y, x, slots, p.scale, layer=layer)
            torch.cuda.synchronize()
            ref = oracle.lora_add(p.y, p.x, idx, A_all[layer], B_all[layer], p.scale, dtype)
            _assert_close(oracle.decode(_storage(y, dtype), dtype), ref,
                          f"pool batch {b} layer {layer} ({n} tokens, slots {sorted(set(slots.tolist()))})")
    _say(f"[adapter pool] stats {pool.stats}")
    assert pool.stats["misses"] > pool.n_slots          # evictions happened
    # a re-registered adapter is uploaded again on its next use
    A_new, B_new = _stacked_adapters(63, layers, 1, r, h_in, h_out, dtype)
    pool.register(keys[9], sgmv.as_tensor(A_new[:, 0], dtype), sgmv.as_tensor(B_new[:, 0], dtype))
    p = synth.random_problem((64,), n=5, h_in=h_in, h_out=h_out, r=r, n_adapters=1, dtype=dtype,
                             ids=np.zeros(5, np.int32))
    before = pool.stats["misses"]
    slots = pool.prepare([keys[9]] * 5)
    assert pool.stats["misses"] == before + 1
    y = sgmv.as_tensor(p.y, dtype, "cuda")
    pool.lora_add(y, sgmv.as_tensor(p.x, dtype, "cuda"), slots, p.scale, layer=1)
    torch.cuda.synchronize()
    ref = oracle.lora_add(p.y, p.x, np.zeros(5, np.int32), A_new[1], B_new[1], p.scale, dtype)
    _assert_close(oracle.decode(_storage(y, dtype), dtype), ref, "re-registered adapter")
    pool.close()


@pytest.mark.parametrize("layer", [0, 2])
def test_stacked_multilayer_pool(torch_cuda, layer):
    """A [layers, P, r, h] pool: layer l's adapters at a pointer offset of l * P adapters,
    through the one-launch paths (device and host ids), the device-id table path and the
    host-table path; each against the oracle on that layer's adapters."""
    torch = torch_cuda
    from adapter_gemv_amd import sgmv
    layers, P, r, h_in, h_out, dtype = 3, 7, 32, 2056, 1032, "bf16"
    A_all, B_all = _stacked_adapters(70, layers, P, r, h_in, h_out, dtype)
    A = sgmv.as_tensor(A_all, dtype, "cuda")
    B = sgmv.as_tensor(B_all, dtype, "cuda")
    for n in (40, 300):
        p = synth.random_problem((71, n, layer), n=n, h_in=h_in, h_out=h_out, r=r, n_adapters=P,
                                 dtype=dtype, id_dist="zipf", zipf_s=1.1)
        x = sgmv.as_tensor(p.x, dtype, "cuda")
        ref = oracle.lora_add(p.y, p.x, p.ids, A_all[layer], B_all[layer], p.scale, dtype)
        ids_dev = torch.as_tensor(p.ids, device="cuda")
        outs = {}
        y = sgmv.as_tensor(p.y, dtype, "cuda")
        outs["device ids"] = sgmv.lora_add_pool(y, x, ids_dev, A, B, p.scale, layer=layer)
        if n <= 64:
            y = sgmv.as_tensor(p.y, dtype, "cuda")
            outs["host ids"] = sgmv.lora_add_host_ids(y, x, p.ids, A, B, p.scale, layer=layer)
        y = sgmv.as_tensor(p.y, dtype, "cuda")
        b = sgmv.Batch.build(p.ids, A[layer], B[layer])
        outs["host tables"] = sgmv.lora_add(y, x, b, p.scale)
        torch.cuda.synchronize()
        for k, out in outs.items():
            _assert_close(oracle.decode(_storage(out, dtype), dtype), ref,
                          f"stacked layer {layer} n={n} {k}")
    with pytest.raises(ValueError):
        sgmv.lora_add_pool(y, x, ids_dev, A, B, p.scale)        # no layer for stacked pools
