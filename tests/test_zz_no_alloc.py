"""GPU: the no-allocation permutation (its workspace a fixed device array)
gives exactly moelb_permute's outputs, on two calls in a row, the second with
a smaller input, and refuses a workspace beyond its array's size."""
import ctypes

import numpy as np
import pytest
import torch

from tests.gpu_layer import log

pytestmark = pytest.mark.gpu


def _case(T, d, E, k, G, N, L, seed):
    from routed_expert_ffn_gate_amd import moelb as M
    dev = torch.device("cuda")
    rng = np.random.default_rng(seed)
    p = 1.0 / np.arange(1, E + 1) ** 1.2
    idx = np.stack([rng.choice(E, size=k, replace=False, p=p / p.sum()) for _ in range(T)]).astype(np.int32)
    i32 = dict(dtype=torch.int32, device=dev)
    idx_t = torch.from_numpy(idx).to(dev)
    home = torch.arange(E, **i32) // (E // G)
    counts = torch.empty((G, E), **i32)
    replica = torch.empty((G, N), **i32)
    host_count = torch.empty((E, G), **i32)
    load = torch.empty((G,), **i32)
    M.moelb_histogram(idx_t, G, counts)
    M.moelb_plan(counts, home, L, replica)
    M.moelb_split(counts, home, replica, host_count, load)
    h = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to(dev).to(torch.bfloat16)
    return M, idx_t, home, replica, host_count, h


def _outputs(T, d, E, k, G, dev):
    i32 = dict(dtype=torch.int32, device=dev)
    return (torch.full((2 * G * E + 1,), -7, **i32), torch.full((T * k,), -7, **i32),
            torch.full((T * k,), -7, **i32), torch.zeros((T * k, d), dtype=torch.bfloat16, device=dev))


@pytest.mark.parametrize("first,second", [((8192, 256, 128, 8, 8, 4, 2), (512, 128, 64, 6, 4, 2, 1))])
def test_noalloc_permute_equals_permute_twice(moelb, first, second):
    for n, (T, d, E, k, G, N, L) in enumerate((first, second)):
        log(f"[noalloc permute] call {n}: T={T} d={d} E={E} k={k} G={G} N={N}")
        M, idx, home, replica, host_count, h = _case(T, d, E, k, G, N, L, seed=n)
        ws = torch.empty((M.moelb_permute_workspace_bytes(T, k, E, G),), dtype=torch.uint8, device=h.device)
        assert ws.numel() <= (32 << 20)
        a = _outputs(T, d, E, k, G, h.device)
        b = _outputs(T, d, E, k, G, h.device)
        M.moelb_permute(h, idx, G, home, replica, host_count, ws, *a)
        M.moelb_permute_noalloc(h, idx, G, home, replica, host_count, *b)
        torch.cuda.synchronize()
        for name, x, y in zip(("group_off", "perm", "pos", "x_perm"), a, b):
            assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                               y.view(torch.int16) if y.dtype == torch.bfloat16 else y), name
        # indices only (no rows) as well
        c = _outputs(T, d, E, k, G, h.device)
        M.moelb_permute_noalloc(None, idx, G, home, replica, host_count, c[0], c[1], c[2], None, d=d,
                                dtype=M.MOELB_BF16)
        torch.cuda.synchronize()
        for name, x, y in zip(("group_off", "perm", "pos"), a[:3], c[:3]):
            assert torch.equal(x, y), name


def test_noalloc_permute_refuses_oversized_workspace(moelb):
    from routed_expert_ffn_gate_amd import moelb as M
    lib = M.lib()
    P = ctypes.c_void_p(16)  # never dereferenced: the size check fails first
    T, k, E, G = 1 << 22, 8, 256, 64
    assert M.moelb_permute_workspace_bytes(T, k, E, G) > (32 << 20)
    assert lib.moelb_permute_noalloc(None, P, T, 64, k, E, G, 1, M.MOELB_BF16, P, P, P, P, P, P, None,
                                     None) == M.MOELB_EWORKSPACE
