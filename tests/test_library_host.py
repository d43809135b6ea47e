"""Host-side checks of libube that need no GPU: exports, tape plan, argument refusals."""
import ctypes as C
import glob
import os
import re

import numpy as np
import pytest

import oracle
import multimodal_embeddings_amd as ube

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w \*]*?\b(ube_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert {"ube_text_encode", "ube_model_init", "ube_arena_init", "ube_tape_plan", "ube_step_gemm"} <= names
    L = ube.lib()
    missing = [n for n in sorted(names) if not hasattr(L, n)]
    assert not missing, missing
    assert set(ube._SIGNATURES) == names  # the binding marshals exactly the declared calls


def test_tape_plan_matches_oracle_bit_exact():
    rng = np.random.default_rng(3)
    for _ in range(30):
        n = int(rng.integers(0, 40))
        lens = rng.integers(0, 3000, size=n)
        start = int(rng.integers(0, 7))
        offsets = np.concatenate([[start], start + np.cumsum(lens)]).astype(np.uint64)
        ctx = int(rng.integers(1, 2049))
        l1, cu1, s1 = ube.tape_plan(offsets, ctx)
        l2, cu2, s2 = oracle.tape_plan(offsets, ctx)
        assert l1.tolist() == l2.tolist() and cu1.tolist() == cu2.tolist() and s1 == s2


def test_tape_plan_worked_example_and_refusal():
    l, cu, s = ube.tape_plan(np.array([0, 14, 24], np.uint64), 8)
    assert l.tolist() == [8, 8] and cu.tolist() == [0, 8, 16] and s == (2, 16)
    with pytest.raises(ube.UbeError) as e:
        ube.tape_plan(np.array([0, 14, 10], np.uint64), 8)
    assert e.value.status == "invalid_argument"


def test_status_and_kernel_names():
    L = ube.lib()
    assert L.ube_status_name(0) == b"success" and L.ube_status_name(5) == b"contended"
    assert [L.ube_kernel_name(i).decode() for i in range(len(ube.KERNELS))] == ube.KERNELS


def test_encode_refuses_null_arena_before_any_device_work():
    outcome = ube.ube_outcome_t()
    rows = ube.ube_rows_view_t()
    rows.count = 99
    off = np.array([0, 3], np.uint64)
    data = np.zeros(3, np.uint8)
    tape = ube.ube_tape_view_t(data.ctypes.data, off.ctypes.data_as(C.POINTER(C.c_size_t)), 1)
    args = ube.ube_text_encode_t(None, None, None, C.pointer(outcome), 0, tape, 3, C.pointer(rows), None, None)
    ube.lib().ube_text_encode(C.byref(args))
    assert ube.STATUS[outcome.status] == "invalid_argument"
    assert rows.data is None and rows.count == 0  # outputs stay NULL on failure


def test_model_init_refuses_missing_weights():
    outcome = ube.ube_outcome_t()
    handle = C.c_void_p(1234)
    args = ube.ube_model_init_t(C.pointer(handle), C.pointer(outcome), 0, ube.ube_geometry_t(), None)
    ube.lib().ube_model_init(C.byref(args))
    assert ube.STATUS[outcome.status] == "invalid_argument" and not handle.value


def test_free_calls_are_null_safe():
    ube.lib().ube_model_free(None)
    ube.lib().ube_arena_free(None)
    assert ube.lib().ube_arena_capacity(None) == 0


def test_trainer_calls_refuse_null_arguments_before_any_device_work():
    L = ube.lib()
    outcome = ube.ube_outcome_t()
    handle = C.c_void_p(1234)
    init = ube.ube_trainer_init_t(C.pointer(handle), C.pointer(outcome), None, None, 0.0, 0.0, 0.0, 0.0, 0)
    L.ube_trainer_init(C.byref(init))
    assert ube.STATUS[outcome.status] == "invalid_argument" and not handle.value
    rows = ube.ube_rows_view_t()
    rows.count = 7
    fwd = ube.ube_trainer_forward_t(None, None, None, C.pointer(outcome), 0, ube.ube_tape_view_t(), C.pointer(rows),
                                    None)
    L.ube_trainer_forward(C.byref(fwd))
    assert ube.STATUS[outcome.status] == "invalid_argument" and rows.data is None and rows.count == 0
    bwd = ube.ube_trainer_backward_t(None, None, None, C.pointer(outcome), 0, ube.ube_tape_view_t(), None, 0, None, 1)
    L.ube_trainer_backward(C.byref(bwd))
    assert ube.STATUS[outcome.status] == "invalid_argument"
    step = ube.ube_trainer_step_t(None, None, C.pointer(outcome), 0, 1e-3)
    L.ube_trainer_step(C.byref(step))
    assert ube.STATUS[outcome.status] == "invalid_argument"
    assert L.ube_trainer_tensors(None, None, 0) == 0
    L.ube_trainer_free(None)


def test_contrastive_refuses_null_arena():
    outcome = ube.ube_outcome_t()
    args = ube.ube_contrastive_t()
    args.outcome = C.pointer(outcome)
    ube.lib().ube_contrastive(C.byref(args))
    assert ube.STATUS[outcome.status] == "invalid_argument"
