"""Host-side checks of the C ABI (no GPU needed: nothing here launches work).

The library must load, export every function include/headloss.h declares,
and reject every invalid argument on the host with the documented status.
"""

import ctypes
import math

import pytest

import lm_head_vocab_amd as hl
from lm_head_vocab_amd._binding import Weights

lib = hl.load_library()
VP = ctypes.c_void_p


def _plan(V=1000, dtype=hl.HL_BF16, flags=hl.CE, w=None, tau=1.0, eps=0.2, scale=1.0, cap=0.0):
    h = VP()
    w = w or Weights(1.0, 0.0, 0.0, 0.0, 1.0, 0.0)
    st = lib.hl_plan(ctypes.byref(h), V, dtype, flags, ctypes.byref(w), tau, eps, scale, cap)
    return st, h


def test_every_declared_symbol_is_exported():
    names = hl.exported_functions_in_header()
    assert {"hl_plan", "hl_forward_backward", "hl_forward_backward_segments", "hl_plan_destroy",
            "hl_workspace_bytes", "hl_plan_set_workspace", "hl_status_str"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings():
    for code in range(6):
        assert isinstance(hl.status_str(code), str) and hl.status_str(code)
    assert hl.status_str(99) == "unknown status"


@pytest.mark.parametrize("kwargs,status", [
    (dict(V=0), hl.HL_ERR_INVALID_ARG),
    (dict(V=-5), hl.HL_ERR_INVALID_ARG),
    (dict(dtype=7), hl.HL_ERR_INVALID_ARG),
    (dict(flags=0), hl.HL_ERR_INVALID_ARG),
    (dict(flags=hl.ACCUMULATE), hl.HL_ERR_INVALID_ARG),
    (dict(flags=1 << 9), hl.HL_ERR_INVALID_ARG),
    (dict(flags=hl.FKL | hl.RKL), hl.HL_ERR_INVALID_ARG),
    (dict(flags=hl.FKL | hl.FDCE), hl.HL_ERR_INVALID_ARG),
    (dict(flags=hl.RKL | hl.FDCE), hl.HL_ERR_INVALID_ARG),
    (dict(flags=hl.FDCE, tau=0.0), hl.HL_ERR_INVALID_ARG),
    (dict(flags=hl.FKL, tau=0.0), hl.HL_ERR_INVALID_ARG),
    (dict(flags=hl.RKL, tau=-1.0), hl.HL_ERR_INVALID_ARG),
    (dict(flags=hl.RKL, tau=math.inf), hl.HL_ERR_INVALID_ARG),
    (dict(flags=hl.GRPO, eps=0.0), hl.HL_ERR_INVALID_ARG),
    (dict(flags=hl.GRPO, eps=1.0), hl.HL_ERR_INVALID_ARG),
    (dict(flags=hl.GRPO, eps=math.nan), hl.HL_ERR_INVALID_ARG),
    (dict(flags=hl.GSPO, eps=0.0), hl.HL_ERR_INVALID_ARG),
    (dict(flags=hl.GSPO, eps=1.5), hl.HL_ERR_INVALID_ARG),
    (dict(flags=hl.GRPO | hl.GSPO), hl.HL_ERR_INVALID_ARG),
    (dict(flags=hl.CE | hl.HINTON), hl.HL_ERR_INVALID_ARG),
    (dict(flags=hl.FKL | hl.HINTON, tau=0.0), hl.HL_ERR_INVALID_ARG),
    (dict(scale=0.0), hl.HL_ERR_INVALID_ARG),
    (dict(scale=-1.0), hl.HL_ERR_INVALID_ARG),
    (dict(scale=math.inf), hl.HL_ERR_INVALID_ARG),
    (dict(cap=-1.0), hl.HL_ERR_INVALID_ARG),
    (dict(cap=math.nan), hl.HL_ERR_INVALID_ARG),
    (dict(w=Weights(math.nan, 0, 0, 0, 1, 0)), hl.HL_ERR_INVALID_ARG),
    (dict(w=Weights(1, 0, 0, 0, math.inf, 0)), hl.HL_ERR_INVALID_ARG),
    (dict(V=2**31), hl.HL_ERR_UNSUPPORTED),                        # 32-bit element indices
])
def test_plan_rejects(kwargs, status):
    st, h = _plan(**kwargs)
    assert st == status
    assert not h.value


@pytest.mark.parametrize("kwargs", [
    dict(V=10**9), dict(V=2**31 - 1), dict(V=1_500_000),
    dict(V=1_474_561 + 8),                                 # past 9 x 1024 x 20 student vectors
    dict(V=737_280 + 8, flags=hl.RKL),                     # past 9 x 1024 x 10 teacher vectors
    dict(V=655_360 + 8, flags=hl.FDCE | hl.HINTON),        # 8 chunks at most there
    dict(V=368_640 + 4, dtype=hl.HL_F32, flags=hl.FKL),    # fp32: 4 elements per vector
])
def test_rows_past_every_exchanged_slice_plan_two_launches(kwargs):
    """Rows longer than any slice set the chunk exchange serves: statistics
    streamed first, the gradient from the fused kernel in load mode with as many
    1024-thread chunks as the row needs."""
    st, h = _plan(**kwargs)
    assert st == hl.HL_OK
    c, b, n = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    assert lib.hl_plan_describe(h, ctypes.byref(c), ctypes.byref(b), ctypes.byref(n)) == hl.HL_OK
    vec = 4 if kwargs.get("dtype") == hl.HL_F32 else 8
    teacher = kwargs.get("flags", hl.CE) & (hl.FKL | hl.RKL | hl.FDCE)
    assert b.value == 1024 and n.value <= (10 if teacher else 20) and c.value >= 8
    assert c.value * b.value * n.value * vec >= kwargs["V"] - vec      # the slices cover the row
    # a forced chunk count still has to fit a slice the exchange serves
    before = (c.value, b.value, n.value)
    assert lib.hl_plan_set_chunks(h, 9) == hl.HL_ERR_UNSUPPORTED
    assert lib.hl_plan_describe(h, ctypes.byref(c), ctypes.byref(b), ctypes.byref(n)) == hl.HL_OK
    assert (c.value, b.value, n.value) == before
    lib.hl_plan_destroy(h)
    # no chunk-exchange words for such a plan: its workspace is a one-chunk plan's
    st, h = _plan(**kwargs)
    flags = kwargs.get("flags", hl.CE)
    st1, h1 = _plan(V=1000, dtype=kwargs.get("dtype", hl.HL_BF16), flags=flags)
    assert st == st1 == hl.HL_OK
    lib.hl_plan_describe(h1, ctypes.byref(c), None, None)
    assert c.value == 1
    for n_rows in (0, 1, 777, 32768):
        assert lib.hl_workspace_bytes(h, n_rows) == lib.hl_workspace_bytes(h1, n_rows)
    lib.hl_plan_destroy(h)
    lib.hl_plan_destroy(h1)
    # one element shorter than a full slice set still plans a register-resident variant
    if kwargs["V"] < 10**6 and "dtype" not in kwargs:
        st, h = _plan(**dict(kwargs, V=kwargs["V"] - 8))
        assert st == hl.HL_OK
        lib.hl_plan_describe(h, ctypes.byref(c), ctypes.byref(b), ctypes.byref(n))
        assert n.value > 0
        lib.hl_plan_destroy(h)


def test_plan_accepts_and_describes_the_baseline_shapes():
    cases = [  # (V, dtype, flags, expected chunks, expected threads per workgroup)
        (1024, hl.HL_F32, hl.CE | hl.ZLOSS, 1, 256),
        (128256, hl.HL_BF16, hl.CE | hl.ZLOSS, 2, 1024),
        (151936, hl.HL_BF16, hl.CE | hl.FKL, 4, 512),
        (151936, hl.HL_BF16, hl.CE | hl.RKL, 4, 512),
        (151936, hl.HL_BF16, hl.GRPO | hl.ZLOSS | hl.ENTROPY, 2, 1024),
        (60000, hl.HL_BF16, hl.CE, 1, 1024),
        (256000, hl.HL_BF16, hl.CE | hl.ZLOSS | hl.RKL | hl.GRPO | hl.ENTROPY | hl.ACCUMULATE, 7, 512),
        (1_400_000, hl.HL_BF16, hl.CE, 9, 1024),
        (151936, hl.HL_BF16, hl.CE | hl.FDCE, 4, 512),
        (151936, hl.HL_F16, hl.CE | hl.ZLOSS, 2, 1024),
    ]
    for V, dt, flags, chunks, block in cases:
        st, h = _plan(V=V, dtype=dt, flags=flags, cap=30.0 if V == 256000 else 0.0)
        assert st == hl.HL_OK, (V, flags)
        c, b, n = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
        assert lib.hl_plan_describe(h, ctypes.byref(c), ctypes.byref(b), ctypes.byref(n)) == 0
        assert (c.value, b.value) == (chunks, block), (V, flags, c.value, b.value)
        vec = 4 if dt == hl.HL_F32 else 8
        # every body vector of a chunk has a thread slot
        assert c.value * b.value * n.value * vec >= V - 2 * vec
        assert lib.hl_workspace_bytes(h, 1000) > 0
        assert lib.hl_workspace_bytes(h, -1) == 0
        lib.hl_plan_destroy(h)


def test_set_chunks_and_errors():
    st, h = _plan(V=20000)
    assert st == 0
    assert lib.hl_plan_set_chunks(h, -1) == hl.HL_ERR_INVALID_ARG
    assert lib.hl_plan_set_chunks(h, 10) == hl.HL_ERR_INVALID_ARG
    assert lib.hl_plan_set_variant(h, 2, 300) == hl.HL_ERR_INVALID_ARG
    assert lib.hl_plan_set_variant(h, 0, 512) == hl.HL_ERR_INVALID_ARG
    assert lib.hl_plan_set_chunks(h, 3) == hl.HL_OK
    c = ctypes.c_int()
    lib.hl_plan_describe(h, ctypes.byref(c), None, None)
    assert c.value == 3
    assert lib.hl_plan_set_chunks(h, 0) == hl.HL_OK
    lib.hl_plan_describe(h, ctypes.byref(c), None, None)
    assert c.value == 1
    lib.hl_plan_destroy(h)
    # a chunk count that leaves a too-long slice is refused and the plan kept
    st, h = _plan(V=256000, flags=hl.CE | hl.RKL)
    assert lib.hl_plan_set_chunks(h, 1) == hl.HL_ERR_UNSUPPORTED
    lib.hl_plan_describe(h, ctypes.byref(c), None, None)
    assert c.value == 7
    lib.hl_plan_destroy(h)


def test_variant_change_invalidates_a_caller_workspace():
    st, h = _plan(V=5000, flags=hl.CE)
    fake = VP(4096)
    fb = lib.hl_forward_backward
    # a caller workspace that is too small is refused before any HIP call
    assert lib.hl_plan_set_workspace(h, fake, 8) == hl.HL_OK
    assert fb(h, 4, fake, fake, None, None, None, None, None, fake, None) == hl.HL_ERR_WORKSPACE
    assert lib.hl_plan_set_workspace(h, fake, 1 << 30) == hl.HL_OK
    assert lib.hl_plan_set_variant(h, 3, 256) == hl.HL_OK
    # the layout changed: the caller's workspace must be handed over again
    assert fb(h, 4, fake, fake, None, None, None, None, None, fake, None) == hl.HL_ERR_WORKSPACE
    lib.hl_plan_destroy(h)


def test_forward_backward_host_checks_enqueue_nothing():
    # every case below fails before any HIP call (works without a GPU)
    st, h = _plan(V=64, flags=hl.CE | hl.GRPO | hl.FKL, w=Weights(1, 0, 1, 1, 1, 0))
    assert st == 0
    fake = VP(4096)           # 16-byte aligned stand-in pointer, never dereferenced
    mis = VP(4097)            # not aligned to the bf16 element size (a 16-byte misalignment that
                              # keeps element alignment is valid: it selects the row-wise kernel)
    fb = lib.hl_forward_backward
    assert fb(None, 4, fake, fake, None, fake, fake, fake, fake, fake, None) == hl.HL_ERR_INVALID_ARG
    assert fb(h, -1, fake, fake, None, fake, fake, fake, fake, fake, None) == hl.HL_ERR_INVALID_ARG
    assert fb(h, 4, fake, fake, None, fake, fake, fake, fake, None, None) == hl.HL_ERR_INVALID_ARG
    assert fb(h, 4, None, fake, None, fake, fake, fake, fake, fake, None) == hl.HL_ERR_INVALID_ARG
    assert fb(h, 4, fake, None, None, fake, fake, fake, fake, fake, None) == hl.HL_ERR_MISSING_INPUT
    assert fb(h, 4, fake, fake, None, None, fake, fake, fake, fake, None) == hl.HL_ERR_MISSING_INPUT
    assert fb(h, 4, fake, fake, None, fake, None, fake, fake, fake, None) == hl.HL_ERR_MISSING_INPUT
    assert fb(h, 4, fake, fake, None, fake, fake, None, fake, fake, None) == hl.HL_ERR_MISSING_INPUT
    assert fb(h, 4, mis, fake, None, fake, fake, fake, fake, fake, None) == hl.HL_ERR_INVALID_ARG
    assert fb(h, 4, fake, fake, None, mis, fake, fake, fake, fake, None) == hl.HL_ERR_INVALID_ARG
    assert fb(h, 4, fake, fake, None, fake, fake, fake, mis, fake, None) == hl.HL_ERR_INVALID_ARG
    # a caller workspace that is too small
    assert lib.hl_plan_set_workspace(h, None, 0) == hl.HL_ERR_INVALID_ARG
    assert lib.hl_plan_set_workspace(h, VP(4096 + 16), 1 << 20) == hl.HL_ERR_INVALID_ARG
    assert lib.hl_plan_set_workspace(h, fake, 8) == hl.HL_OK
    assert fb(h, 4, fake, fake, None, fake, fake, fake, fake, fake, None) == hl.HL_ERR_WORKSPACE
    lib.hl_plan_destroy(h)
    lib.hl_plan_destroy(None)


def test_hinton_plans_and_the_eight_statistic_chunk_cap():
    for mode in (hl.FKL, hl.RKL, hl.FDCE):
        st, h = _plan(V=151936, flags=hl.CE | mode | hl.HINTON, w=Weights(1, 0, 1, 0, 1, 0), tau=2.0)
        assert st == 0
        c, b, n = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
        assert lib.hl_plan_describe(h, ctypes.byref(c), ctypes.byref(b), ctypes.byref(n)) == 0
        # the 16-bit Hinton instances hold 9 register + 4 LDS vectors per tensor
        assert (c.value, b.value, n.value) == (3, 512, 13)
        # the from-distribution mode with Hinton exchanges 8 statistics per
        # chunk: one wave polls at most 64 words, so 8 chunks at most
        expect9 = hl.HL_ERR_UNSUPPORTED if mode == hl.FDCE else hl.HL_OK
        assert lib.hl_plan_set_chunks(h, 9) == expect9
        assert lib.hl_plan_set_chunks(h, 8) == hl.HL_OK
        lib.hl_plan_destroy(h)


def test_fp32_chunk_caps():
    """fp32 plans also exchange the low parts of their normalizers (Z; + Zt
    with a teacher; + Zs with Hinton), so their chunk caps are 64 // words:
    9 student-only, 8 forward / reverse KL, 7 FDCE, 6 Hinton KL, 5 Hinton
    FDCE."""
    cases = [(hl.CE, 9), (hl.CE | hl.FKL, 8), (hl.CE | hl.RKL, 8), (hl.CE | hl.FDCE, 7),
             (hl.CE | hl.FKL | hl.HINTON, 6), (hl.CE | hl.RKL | hl.HINTON, 6), (hl.CE | hl.FDCE | hl.HINTON, 5)]
    for flags, cap in cases:
        st, h = _plan(V=20011, dtype=hl.HL_F32, flags=flags, w=Weights(1, 0, 1, 0, 1, 0), tau=2.0)
        assert st == hl.HL_OK
        assert lib.hl_plan_set_chunks(h, cap) == hl.HL_OK, (flags, cap)
        if cap < 9:
            assert lib.hl_plan_set_chunks(h, cap + 1) == hl.HL_ERR_UNSUPPORTED, (flags, cap)
        lib.hl_plan_destroy(h)


def test_segment_call_host_checks_enqueue_nothing():
    st, h = _plan(V=64, flags=hl.CE | hl.GSPO | hl.RKL, w=Weights(1, 0, 1, 1, 1, 0))
    assert st == 0
    fake = VP(4096)
    fs = lib.hl_forward_backward_segments
    fb = lib.hl_forward_backward
    # a GSPO plan needs segments: the plain entry point cannot serve it
    assert fb(h, 4, fake, fake, None, fake, fake, fake, fake, fake, None) == hl.HL_ERR_MISSING_INPUT
    assert fs(h, 4, fake, fake, None, fake, fake, fake, None, 2, fake, fake, None) == hl.HL_ERR_MISSING_INPUT
    for n_seg in (0, 5, -1):   # 1 <= n_segments <= n_rows
        assert fs(h, 4, fake, fake, None, fake, fake, fake, fake, n_seg, fake, fake, None) == hl.HL_ERR_INVALID_ARG
    assert fs(h, 4, fake, fake, None, None, fake, fake, fake, 2, fake, fake, None) == hl.HL_ERR_MISSING_INPUT
    assert fs(h, 4, fake, fake, None, fake, None, fake, fake, 2, fake, fake, None) == hl.HL_ERR_MISSING_INPUT
    assert fs(h, 4, fake, fake, None, fake, fake, None, fake, 2, fake, fake, None) == hl.HL_ERR_MISSING_INPUT
    assert lib.hl_plan_set_workspace(h, fake, 8) == hl.HL_OK
    assert fs(h, 4, fake, fake, None, fake, fake, fake, fake, 2, fake, fake, None) == hl.HL_ERR_WORKSPACE
    # the GSPO regions grow the workspace with the row count
    st2, h2 = _plan(V=64, flags=hl.CE | hl.GRPO, w=Weights(1, 0, 1, 1, 1, 0))
    assert lib.hl_workspace_bytes(h, 1000) > lib.hl_workspace_bytes(h2, 1000)
    lib.hl_plan_destroy(h)
    lib.hl_plan_destroy(h2)


def test_binding_marshalling_errors_without_gpu():
    torch = pytest.importorskip("torch")
    p = hl.Plan(64, torch.bfloat16, hl.CE)
    with pytest.raises(ValueError):
        p(torch.zeros(4, 63, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        p(torch.zeros(4, 64, dtype=torch.bfloat16), labels=torch.zeros(4, dtype=torch.int64))
    with pytest.raises(hl.HeadLossError):
        hl.Plan(64, torch.bfloat16, hl.FKL | hl.RKL)
    with pytest.raises(ValueError):
        hl.Plan(64, torch.int8, hl.CE)


def test_layout_without_an_instance_is_refused_and_the_plan_kept():
    # 6 chunks of 256 threads x 4 vectors hold 49152 bf16 elements: no instance serves V = 60013
    st, h = _plan(V=60013, flags=hl.CE | hl.ZLOSS)
    assert st == 0
    c, b = ctypes.c_int(), ctypes.c_int()
    lib.hl_plan_describe(h, ctypes.byref(c), ctypes.byref(b), None)
    before = (c.value, b.value)
    assert lib.hl_plan_set_variant(h, 6, 256) == hl.HL_ERR_UNSUPPORTED
    lib.hl_plan_describe(h, ctypes.byref(c), ctypes.byref(b), None)
    assert (c.value, b.value) == before
    assert lib.hl_plan_set_variant(h, 8, 256) == hl.HL_OK
    lib.hl_plan_destroy(h)


def test_fp32_teacher_slices_respect_their_register_cap():
    # fp32 instances evaluate gradient elements in fp64: teacher slices hold at
    # most 8 vectors per tensor, 4 in the Hinton modes
    for extra, cap in ((0, 8), (hl.HINTON, 4)):
        for V in (20011, 60000, 151936, 300007):
            st, h = _plan(V=V, flags=hl.CE | hl.FKL | extra, dtype=hl.HL_F32, w=Weights(1, 0, 1, 0, 1, 0), tau=2.0)
            assert st == 0, (V, extra)
            n = ctypes.c_int()
            assert lib.hl_plan_describe(h, None, None, ctypes.byref(n)) == 0
            assert n.value <= cap, (V, extra, n.value)
            for chunks in range(1, 10):
                if lib.hl_plan_set_chunks(h, chunks) == hl.HL_OK:
                    lib.hl_plan_describe(h, None, None, ctypes.byref(n))
                    assert n.value <= cap, (V, extra, chunks, n.value)
            lib.hl_plan_destroy(h)


def test_exchange_test_hook_arguments():
    st, h = _plan(V=20000, flags=hl.CE | hl.RKL, w=Weights(1, 0, 1, 0, 1, 0))
    assert st == 0
    hook = lib.hl_plan_set_exchange_test
    assert hook(None, 64, 0, 0) == hl.HL_ERR_INVALID_ARG
    assert hook(h, 0, 0, 0) == hl.HL_ERR_INVALID_ARG            # the wait needs at least one poll
    assert hook(h, 64, 1 << 32, 0) == hl.HL_ERR_INVALID_ARG     # rows are 32-bit there
    assert hook(h, 64, 3, 1) == hl.HL_OK
    assert hook(h, 1 << 20, -1, -1) == hl.HL_OK                  # back to the default
    lib.hl_plan_destroy(h)


def test_noalloc_checks_before_any_hip_call():
    # argument checks and the static-workspace size limit are host checks
    st, h = _plan(V=151936, flags=hl.CE | hl.FKL, w=Weights(1, 0, 1, 0, 1, 0), tau=2.0)
    assert st == 0
    fake = VP(4096)
    na = lib.hl_forward_backward_noalloc
    assert na(None, 4, fake, fake, None, fake, None, None, None, 0, fake, fake, None) == hl.HL_ERR_INVALID_ARG
    assert na(h, 4, fake, fake, None, None, None, None, None, 0, fake, fake, None) == hl.HL_ERR_MISSING_INPUT
    n = 1
    while lib.hl_workspace_bytes(h, n) <= 32 * 1024 * 1024:
        n *= 2
    assert na(h, n, fake, fake, None, fake, None, None, None, 0, fake, fake, None) == hl.HL_ERR_WORKSPACE
    msg = lib.hl_last_error().decode()
    assert "HL_STATIC_WORKSPACE_BYTES" in msg and str(n) in msg
    lib.hl_plan_destroy(h)


def test_stream_ceiling_host_checks():
    """The measurement aid refuses bad arguments on the host, before any HIP call."""
    ms = ctypes.c_float()
    f = lib.hl_stream_ceiling
    assert f(None, None, VP(4096), 1 << 20, 1024, 10, 1, None, ctypes.byref(ms)) == hl.HL_ERR_INVALID_ARG
    assert f(VP(4096), None, VP(8192), 1 << 20, 1024, 10, 0, None, ctypes.byref(ms)) == hl.HL_ERR_INVALID_ARG
    assert f(VP(4096), None, VP(8192), 1000, 1024, 10, 1, None, ctypes.byref(ms)) == hl.HL_ERR_INVALID_ARG
    assert f(VP(4096 + 8), None, VP(8192), 1 << 20, 1024, 10, 1, None, ctypes.byref(ms)) == hl.HL_ERR_INVALID_ARG
    assert f(VP(4096), None, VP(8192), 1 << 20, 256, 10, 1, None, ctypes.byref(ms)) == hl.HL_ERR_UNSUPPORTED
    assert f(VP(4096), None, VP(8192), 1 << 20, 1024, 13, 1, None, ctypes.byref(ms)) == hl.HL_ERR_UNSUPPORTED
    assert f(VP(4096), VP(12288), VP(8192), 1 << 20, 512, 7, 1, None, ctypes.byref(ms)) == hl.HL_ERR_UNSUPPORTED
