"""kivi_append_decode_noalloc (the decode step for callers that cannot allocate) against
kivi_append_decode with a workspace, through the C ABI.

Two calls in a row, the second on a smaller batch than the first, each on two
identically prefilled caches: the cache bytes must be equal (integer data, bit for
bit), the two outputs within the stated tolerance |x - y| <= 2e-3 + 1e-3 |y| of each
other (the same kernels; which wave takes which block varies, so float sums may round
differently), and both within that tolerance of the oracle.  A flush step (window
full) and a plain step are both covered.
"""
import math

import numpy as np
import pytest

import oracle as O
import workloads as W
from tests.test_gpu_parity import assert_close, dims_of, gpu_prefill, rand_kv

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def one_step(B, H, g, T0, R, bits, seed):
    from bit_quantization_amd import kivi as k
    d = 128
    print(f"[noalloc] B={B} H={H} g={g} T_before={T0} R={R} bits={bits}", flush=True)
    w = W.Workload("noalloc", 97, 1, B, H, H * g, d, T0, bits, 32, d, R, stream_steps=4)
    dims = dims_of(w, w.max_tokens())
    K, V = rand_kv(B, H, T0 + 1, d, seed=seed)
    ca = gpu_prefill(w, dims, K, V, T0)
    cb = gpu_prefill(w, dims, K, V, T0)
    q = torch.randn((B, H * g, d), device="cuda").to(torch.float16)
    sm = 1 / math.sqrt(d)
    kn, vn = K[:, :, T0].contiguous(), V[:, :, T0].contiguous()
    oa = torch.empty((B, H * g, d), dtype=torch.float32, device="cuda")
    ob = torch.full_like(oa, float("nan"))
    ws = k.new_workspace(dims, T0 + 1)
    k.kivi_append_decode(dims, ca, 0, T0, kn, vn, q, sm, oa, ws)
    k.kivi_append_decode_noalloc(dims, cb, 0, T0, kn, vn, q, sm, ob)
    torch.cuda.synchronize()
    for name in k.BUFFERS:
        assert torch.equal(ca.view(name).cpu(), cb.view(name).cpu()), f"{name} differs"
    a, b = oa.cpu().numpy(), ob.cpu().numpy()
    assert_close(b, a, f"noalloc against the workspace call B={B} H={H}")
    oc = O.LayerCache(B, H, d, bits, 32, d, R, w.max_tokens())
    oc.prefill(K[:, :, :T0].cpu().numpy(), V[:, :, :T0].cpu().numpy())
    oc.append(kn.cpu().numpy(), vn.cpu().numpy())
    assert_close(b, oc.attend(q.cpu().numpy(), sm), f"noalloc B={B} H={H} T={T0 + 1}")


def test_noalloc_step_equals_workspace_step_twice_shrinking():
    # first call: 8 pairs, GQA 4, a full window (the step flushes), 2-bit
    one_step(B=2, H=4, g=4, T0=2048, R=128, bits=2, seed=41)
    # second call, smaller: 2 pairs, GQA 2, a plain step, 4-bit
    one_step(B=1, H=2, g=2, T0=700, R=64, bits=4, seed=42)
