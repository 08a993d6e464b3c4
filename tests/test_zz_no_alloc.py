"""The allocation-free route prep (moe_route_prep_noalloc, for callers that
cannot allocate device memory) against moe_route_prep with a caller's
workspace: equal tables on two calls in a row through the C ABI, the second
with a smaller input, both large enough to use the library's fixed device
array; sizes beyond that array are refused on the host."""
import ctypes as C

import numpy as np
import pytest
import torch

import synth
import quantized_moe_grouped_route_amd as mq

pytestmark = pytest.mark.gpu


def _outs(T, k, E):
    i32 = dict(dtype=torch.int32, device="cuda")
    return (torch.full((E + 1,), -7, **i32), torch.full((T * k,), -7, **i32), torch.full((T * k,), -7, **i32),
            torch.full((1,), -7, **i32))


def _noalloc_abi(ids, E, outs):
    # straight through the C entry point (ctypes), no Python-side allocation
    T, k = ids.shape
    L = mq.lib()
    st = L.moe_route_prep_noalloc(C.c_void_p(ids.data_ptr()), T, k, E, *(C.c_void_p(t.data_ptr()) for t in outs),
                                  C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == mq.OK, L.moeq_last_error()
    return outs


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mq.lib()


def test_noalloc_route_equals_workspace_route_two_calls_second_smaller():
    rng = np.random.default_rng(3)
    cases = [(synth.zipf_ids(rng, 4096, 8, 256), 256),                  # 32768 pairs, 32 chunks
             (np.where(rng.random((1500, 3)) < 0.1, -1,                 # 4500 pairs with -1 and
                       rng.integers(-2, 40, size=(1500, 3))).astype(np.int32), 37)]   # out-of-range ids
    for ids_np, E in cases:
        ids = torch.from_numpy(ids_np).cuda()
        T, k = ids.shape
        assert mq.route_workspace_bytes(T, k, E) > 0                   # the fixed array is used
        got = _noalloc_abi(ids, E, _outs(T, k, E))
        ref = mq.moe_route_prep(ids, E)
        torch.cuda.synchronize()
        for g, r in zip(got, ref):
            assert torch.equal(g, r)


def test_noalloc_route_small_sizes_and_the_limit():
    ids = torch.from_numpy(synth.distinct_uniform_ids(np.random.default_rng(4), 8, 8, 256)).cuda()
    got = mq.moe_route_prep_noalloc(ids, 256, out=_outs(8, 8, 256))
    ref = mq.moe_route_prep(ids, 256)
    for g, r in zip(got, ref):
        assert torch.equal(g, r)
    # the largest pair count the fixed array serves at E = 1024, and one chunk more
    E = 1024
    chunks = mq.ROUTE_NOALLOC_SCRATCH_BYTES // ((E + 1) * 4)
    big = torch.zeros((chunks * 1024 + 1, 1), dtype=torch.int32, device="cuda")
    with pytest.raises(mq.MoeqError, match="fixed"):
        mq.moe_route_prep_noalloc(big, E, out=_outs(big.shape[0], 1, E))
    ok = big[: chunks * 1024]
    got = mq.moe_route_prep_noalloc(ok, E, out=_outs(ok.shape[0], 1, E))
    ref = mq.moe_route_prep(ok, E)
    torch.cuda.synchronize()
    for g, r in zip(got, ref):
        assert torch.equal(g, r)
