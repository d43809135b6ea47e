"""The arena's call rules through the C ABI ("Arenas" page, `uform_arena_t`: an arena
serves one call at a time and a second call naming it finishes `contended`; on failure
the outputs are empty; "Python" page, "Errors": out-of-memory without a host fallback).
"""
import ctypes as C
import threading

import numpy as np
import pytest

from multimodal_embeddings_amd import configs, synth
from tests.gpu_util import device_bytes, say

pytestmark = pytest.mark.gpu


def _raw_text_encode(ube, model, arena, data, offsets):
    """One ube_text_encode call -> (status name, rows view fields); no exception on failure."""
    tape, off = ube._tape(data, offsets)
    rows, stats, outcome = ube.ube_rows_view_t(), ube.ube_encode_stats_t(), ube.ube_outcome_t()
    states, vectors = ube.ube_rows_tape_view_t(), ube.ube_rows_tape_view_t()
    # non-NULL garbage in the output views: a failed call must reset it
    rows.data, rows.count, rows.columns = 0x1234, 7, 7
    args = ube.ube_text_encode_t(model.handle, arena.handle, None, C.pointer(outcome), 0, tape, ube.SCALAR["f32"],
                                 C.pointer(rows), C.pointer(stats), None, 0, C.pointer(states), C.pointer(vectors))
    ube.lib().ube_text_encode(C.byref(args))
    return ube.STATUS[outcome.status], (rows.data, rows.count, rows.columns, rows.stride)


def test_a_second_concurrent_call_on_an_arena_is_contended():
    import torch
    import multimodal_embeddings_amd as ube
    w = synth.make_weights(configs.geometry("text512"))
    model, arena = ube.Model(w, 0), ube.Arena(0)
    batch = synth.workload_inputs("throughput")  # ~0.15 s per call: the first caller holds the arena that long
    data = device_bytes(batch.data)
    want, _ = ube.text_encode(model, arena, data, batch.offsets)  # grows the arena once
    want = want.tensor().clone()
    torch.cuda.synchronize()
    n = 4
    gate = threading.Barrier(n)
    results = [None] * n

    def call(i):
        gate.wait()
        results[i] = _raw_text_encode(ube, model, arena, data, batch.offsets)

    threads = [threading.Thread(target=call, args=(i,)) for i in range(n)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    statuses = [r[0] for r in results]
    say(f"  concurrent calls on one arena: {statuses}")
    assert set(statuses) <= {"success", "contended"}
    assert statuses.count("success") >= 1 and statuses.count("contended") >= 1
    for status, view in results:
        if status == "contended":
            assert view == (None, 0, 0, 0)
        else:
            assert view[1:] == (1024, 512, 2048)
    # the call that held the arena left the same rows as a call alone
    rows, _ = ube.text_encode(model, arena, data, batch.offsets)
    np.testing.assert_array_equal(rows.tensor().cpu().numpy(), want.cpu().numpy())
    arena.close()
    model.close()


def test_arena_capacity_limit_reports_out_of_memory():
    import multimodal_embeddings_amd as ube
    w = synth.make_weights(configs.geometry("tiny"))
    model = ube.Model(w, 0)
    limit = 4 << 20
    arena = ube.Arena(0, capacity_limit=limit)
    small = synth.text_batch(2, 16, 17, 0, 256, seed=5)
    big = synth.text_batch(8, 1024, 1025, 0, 256, seed=6)
    rows, _ = ube.text_encode(model, arena, device_bytes(small.data), small.offsets)
    got_small = rows.tensor().cpu().numpy().copy()
    cap = arena.capacity
    assert 0 < cap <= limit
    status, view = _raw_text_encode(ube, model, arena, device_bytes(big.data), big.offsets)
    say(f"  8 x 1024 tokens in a {limit >> 20} MiB arena: {status}")
    assert status == "out_of_memory" and view == (None, 0, 0, 0)
    assert arena.capacity == cap  # the arena keeps what it held and still serves calls that fit
    rows, _ = ube.text_encode(model, arena, device_bytes(small.data), small.offsets)
    np.testing.assert_array_equal(rows.tensor().cpu().numpy(), got_small)
    # without the limit the same call succeeds
    free = ube.Arena(0)
    rows, stats = ube.text_encode(model, free, device_bytes(big.data), big.offsets)
    assert stats == (0, 8 * 1024) and free.capacity > limit
    free.close()
    arena.close()
    model.close()
