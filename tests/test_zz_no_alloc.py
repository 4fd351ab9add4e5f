"""moe_permute_noalloc (the grouping with its count table in the library's static device array,
for callers that cannot allocate) through the C ABI, against moe_permute with a caller
workspace and against the oracle: bit-exact, on consecutive calls whose sizes shrink (the array
keeps the previous call's table), up to the largest table the array holds."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import routed_expert_grouped_amd as moe
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _buffers(T, k, E, fill):
    i32 = torch.int32
    return (torch.full((E,), fill, dtype=i32, device=DEV),
            torch.full((E + 1,), fill, dtype=i32, device=DEV),
            torch.full((T * k,), fill, dtype=i32, device=DEV),
            torch.full((T * k,), fill, dtype=i32, device=DEV))


def _noalloc(ids, E, fill, stream=None):
    T, k = ids.shape
    counts, offsets, perm, inv = _buffers(T, k, E, fill)
    stream = torch.cuda.current_stream() if stream is None else stream
    st = moe.lib().moe_permute_noalloc(
        ctypes.c_void_p(ids.data_ptr()), T, k, E, ctypes.c_void_p(counts.data_ptr()),
        ctypes.c_void_p(offsets.data_ptr()), ctypes.c_void_p(perm.data_ptr()),
        ctypes.c_void_p(inv.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
    return st, (counts, offsets, perm, inv)


def test_noalloc_matches_the_workspace_call_on_shrinking_inputs():
    # the largest table the array holds (256 blocks x 1024 experts x 4 bytes = 1 MiB), then
    # smaller and smaller inputs: each call must not depend on what the previous one left
    cases = [(65536, 8, 1024), (32768, 8, 256), (4096, 8, 256), (300, 8, 256), (16, 8, 256)]
    for T, k, E in cases:
        ids = synth.random_topk_ids(T, E, k, seed=T + E).to(DEV)
        table = 0 if T * k <= 2048 else -(-T * k // 2048) * E * 4
        assert table <= moe.PERMUTE_NOALLOC_MAX_BYTES
        side = torch.cuda.Stream()  # a stream of its own (the current device's): same result
        side.wait_stream(torch.cuda.current_stream())
        st, got = _noalloc(ids, E, fill=-7, stream=side if T == 4096 else None)
        assert st == moe.MOE_OK, moe.moe_status_string(st)
        torch.cuda.synchronize()
        want = moe.moe_permute(ids, E)
        torch.cuda.synchronize()
        ref = oracle.permute(ids.cpu().numpy(), E)
        for a, b, r in zip(got, want, ref):
            np.testing.assert_array_equal(a.cpu().numpy(), b.cpu().numpy())
            np.testing.assert_array_equal(a.cpu().numpy(), r)


def test_noalloc_rejects_a_table_beyond_the_array():
    """One block more than the array holds is UNSUPPORTED, checked before anything is enqueued
    (the output buffers keep their contents)."""
    T, k, E = 257 * 2048 // 8, 8, 1024  # 257 blocks of 2048 assignments
    ids = torch.zeros((T, k), dtype=torch.int32, device=DEV)
    st, bufs = _noalloc(ids, E, fill=-7)
    torch.cuda.synchronize()
    assert st == moe.MOE_ERR_UNSUPPORTED
    assert all(bool((b == -7).all()) for b in bufs)


def test_noalloc_in_a_graph():
    """The call captured into a HIP graph (the use it is for: nothing to allocate while
    capturing) replays to moe_permute's result, also after new ids are copied into the captured
    input and with other eager work between the replays."""
    T, k, E = 4096, 8, 256
    ids = synth.random_topk_ids(T, E, k, seed=5).to(DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st, _ = _noalloc(ids, E, fill=0)  # first call on the device outside the capture
    torch.cuda.synchronize()
    assert st == moe.MOE_OK
    outs = _buffers(T, k, E, fill=-7)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cur = torch.cuda.current_stream()
        st = moe.lib().moe_permute_noalloc(
            ctypes.c_void_p(ids.data_ptr()), T, k, E, *[ctypes.c_void_p(b.data_ptr()) for b in outs],
            ctypes.c_void_p(cur.cuda_stream))
    assert st == moe.MOE_OK, moe.moe_status_string(st)
    for rep in range(4):
        if rep == 3:  # new inputs, copied into the captured buffer
            ids.copy_(synth.random_topk_ids(T, E, k, seed=6).to(DEV))
        for b in outs:
            b.fill_(-7)
        junk = torch.randn(1 << 20, device=DEV).sum()  # unrelated eager work
        graph.replay()
        torch.cuda.synchronize()
        want = oracle.permute(ids.cpu().numpy(), E)
        for a, r in zip(outs, want):
            np.testing.assert_array_equal(a.cpu().numpy(), r)
        del junk
