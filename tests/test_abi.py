"""Host-side checks of the C ABI: the library loads without a GPU, exports every
function include/sscan.h declares, and rejects bad arguments before it touches
the HIP runtime.  Every call here fails validation, so nothing is launched."""
import ctypes
import os
import re

import pytest

from selective_state_space_sscan_amd import _lib
from selective_state_space_sscan_amd._lib import sscan_desc, sscan_plan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sscan.h")

OK, E_NULL, E_SHAPE, E_DTYPE, E_UNSUP, E_ALIGN, E_WS, E_HIP = range(8)
FAKE = 0x100000  # a 16-byte aligned address that is never dereferenced: validation fails first


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char\s*\*|const char\s*\*)\s*\**\s*(sscan_\w+)\s*\(",
                                 text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def desc(B=2, T=8, D=16, DS=4, io=0, **kw):
    d = sscan_desc()
    d.B, d.T, d.D, d.DS, d.io = B, T, D, DS, io
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def fwd(lib, d, plan=None, x=FAKE, delta=FAKE, A=FAKE, b=FAKE, c=FAKE, h0=None, y=FAKE, hT=FAKE, H=None, ws=None,
        ws_bytes=0):
    v = lambda p: None if p is None else ctypes.c_void_p(p)
    return lib.sscan_fwd(None if d is None else ctypes.byref(d), None if plan is None else ctypes.byref(plan), v(x),
                         v(delta), v(A), v(b), v(c), v(h0), v(y), v(hT), v(H), v(ws), ctypes.c_size_t(ws_bytes), None)


def bwd(lib, d, dy=FAKE, x=FAKE, delta=FAKE, A=FAKE, b=FAKE, c=FAKE, h0=None, H=FAKE, gx=FAKE, gd=FAKE, gb=FAKE,
        gc=FAKE, gA=FAKE, gh0=None, ws=None, ws_bytes=0, plan=None):
    v = lambda p: None if p is None else ctypes.c_void_p(p)
    return lib.sscan_bwd(ctypes.byref(d), None if plan is None else ctypes.byref(plan), v(dy), None, v(x), v(delta),
                         v(A), v(b), v(c), v(h0), v(H), v(gx), v(gd), v(gb), v(gc), v(gA), v(gh0), v(ws),
                         ctypes.c_size_t(ws_bytes), None)


def test_header_declares_the_expected_functions():
    assert header_functions() == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_version_and_status_strings(lib):
    assert lib.sscan_version() == 1
    for s in range(8):
        assert lib.sscan_status_str(s)
    assert lib.sscan_status_str(99) == b"unknown status"


def test_struct_layout_matches_header():
    assert ctypes.sizeof(sscan_desc) == 8 * 4 + 4 * 2 + 8 * 3
    assert ctypes.sizeof(sscan_plan) == 4 * 8


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), E_SHAPE), (dict(T=-3), E_SHAPE), (dict(D=-1), E_SHAPE),
    (dict(DS=3), E_UNSUP), (dict(DS=32), E_UNSUP), (dict(DS=0), E_UNSUP),
    (dict(io=2), E_DTYPE), (dict(reserved=1), E_UNSUP), (dict(B=70000), E_UNSUP),
    (dict(x_bstride=10), E_SHAPE), (dict(bc_bstride=5), E_SHAPE), (dict(y_bstride=100), E_SHAPE),
])
def test_descriptor_validation(lib, kw, status):
    assert fwd(lib, desc(**kw)) == status
    assert lib.sscan_last_error()


def test_size_limits_are_exact(lib):
    """The largest accepted sizes (B = 65535, D*DS = 2^22, T = 2^31 - 1) pass validation,
    one more is refused: the kernels' 32-bit tile offsets are sized for exactly these."""
    def sizes_ok(**kw):
        n = ctypes.c_size_t()
        return lib.sscan_fwd_workspace(ctypes.byref(desc(**kw)), None, ctypes.byref(n))
    assert sizes_ok(B=65535) == OK and sizes_ok(B=65536) == E_UNSUP
    assert sizes_ok(D=2 ** 18, DS=16) == OK and sizes_ok(D=2 ** 18 + 1, DS=16) == E_UNSUP
    assert sizes_ok(D=2 ** 22, DS=1) == OK and sizes_ok(D=2 ** 22 + 1, DS=1) == E_UNSUP
    assert sizes_ok(B=1, T=2 ** 31 - 1) == OK and sizes_ok(B=1, T=2 ** 31) == E_UNSUP


def test_last_error_is_per_thread(lib):
    """sscan_last_error reports the last failure of the calling thread: threads that fail
    validation with different sizes at the same time each read back their own message
    (the ctypes calls release the interpreter lock, so the calls do overlap)."""
    import threading

    errors = []

    def worker(k):
        d = desc(B=-1 - k)
        for _ in range(300):
            if fwd(lib, d) != E_SHAPE:
                errors.append((k, "status"))
                return
            msg = lib.sscan_last_error().decode()
            if f"B={-1 - k} " not in msg:
                errors.append((k, msg))
                return

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:3]


def test_null_descriptor(lib):
    assert fwd(lib, None) == E_NULL
    n = ctypes.c_size_t()
    assert lib.sscan_fwd_workspace(None, None, ctypes.byref(n)) == E_NULL


@pytest.mark.parametrize("missing", ["x", "delta", "A", "b", "c", "y"])
def test_forward_required_pointers(lib, missing):
    assert fwd(lib, desc(), **{missing: None}) == E_NULL


@pytest.mark.parametrize("arg,addr", [("x", FAKE + 2), ("y", FAKE + 1), ("A", FAKE + 4), ("H", FAKE + 8),
                                      ("h0", FAKE + 4), ("hT", FAKE + 12)])
def test_forward_alignment(lib, arg, addr):
    assert fwd(lib, desc(), **{arg: addr}) == E_ALIGN


def test_bf16_io_needs_only_two_byte_alignment_but_not_odd(lib):
    assert fwd(lib, desc(io=1), x=FAKE + 1) == E_ALIGN


def test_plan_validation(lib):
    p = sscan_plan()
    p.lanes = 3
    assert fwd(lib, desc(), plan=p) == E_UNSUP
    p.lanes = 8  # more lanes than DS=4 states
    assert fwd(lib, desc(), plan=p) == E_UNSUP
    p.lanes = 0
    p.chunks = -1
    assert fwd(lib, desc(), plan=p) == E_UNSUP
    p.chunks = 0
    p.reserved[2] = 1
    assert fwd(lib, desc(), plan=p) == E_UNSUP


def test_layout_validation_and_choice(lib):
    LANES, SG = 1, 2
    p = sscan_plan()
    p.layout = 3
    assert fwd(lib, desc(), plan=p) == E_UNSUP
    p.layout = SG
    assert fwd(lib, desc(DS=8), plan=p, H=FAKE) == E_UNSUP    # it writes H only at DS = 16
    assert fwd(lib, desc(DS=16), plan=p, H=FAKE) == E_WS      # valid; b/c packing needs workspace
    assert fwd(lib, desc(DS=2), plan=p) == E_UNSUP            # DS in {4, 8, 16}
    assert fwd(lib, desc(DS=16, D=18), plan=p) == E_UNSUP     # D a multiple of 4
    p.lanes = 4                                                # it runs DS/2 = 8 threads per channel
    assert fwd(lib, desc(DS=16), plan=p) == E_UNSUP
    p.lanes = 0
    assert fwd(lib, desc(DS=16), plan=p) == E_WS               # valid plan; b/c packing needs workspace
    assert bwd(lib, desc(DS=16), plan=p) == E_UNSUP           # the backward runs the lanes layout only
    # the library's choice for the plain forward: state groups wherever they apply, one pass
    # from 512 compute waves (B*D*DS/2 lanes / 64) up, else T-chunks towards 2048 waves (a
    # power of two up to 16) if the chunks keep 256 steps; the lanes layout otherwise, split
    # below one wave per SIMD into chunks of whole tiles for at most four waves per SIMD
    for (B, T, D, DS), (layout, lanes, chunks) in {(16, 4096, 1024, 16): (SG, 8, 1), (8, 1024, 256, 16): (LANES, 8, 16),
                                                   (4, 2048, 2048, 16): (SG, 8, 1), (8, 2048, 768, 16): (SG, 8, 1),
                                                   (2, 4096, 1024, 16): (SG, 8, 8), (1, 8192, 2048, 16): (SG, 8, 8),
                                                   (4, 4096, 1536, 8): (SG, 4, 8), (8, 2048, 1024, 8): (SG, 4, 1),
                                                   (2, 8192, 512, 8): (SG, 4, 16), (16, 2048, 2048, 4): (SG, 2, 1),
                                                   (8, 1024, 256, 2): (LANES, 2, 16), (8, 1024, 258, 16): (LANES, 8, 8),
                                                   (1, 300, 64, 16): (LANES, 8, 5), (1, 4096, 1024, 16): (SG, 8, 16)}.items():
        d = desc(B=B, T=T, D=D, DS=DS)
        q = sscan_plan()
        assert lib.sscan_plan_select(ctypes.byref(d), 0, ctypes.byref(q)) == OK
        assert (q.layout, q.lanes, q.chunks) == (layout, lanes, chunks), (B, T, D, DS)
    # its workspace holds fp32 b and c for every step rounded up to 64
    d = desc(B=16, T=4000, D=1024, DS=16)
    n = ctypes.c_size_t()
    assert lib.sscan_fwd_workspace(ctypes.byref(d), None, ctypes.byref(n)) == OK
    assert n.value >= 16 * 4032 * 2 * 16 * 4


def test_state_group_layout_stops_below_2_24_steps(lib):
    """The state-group forward addresses a batch row's packed b/c (8 DS bytes per step)
    with 32-bit buffer offsets below 2^31, so it runs only for T < 2^24: at T = 2^24 the
    library picks the lanes layout by itself and refuses an explicit state-group plan."""
    LANES, SG = 1, 2
    for kind in (0, 4):  # the forward, and the forward keeping boundary states
        for T, layout in ((2 ** 24 - 64, SG), (2 ** 24 - 1, SG), (2 ** 24, LANES), (2 ** 24 + 64, LANES)):
            d = desc(B=1, T=T, D=4, DS=4)
            q = sscan_plan()
            assert lib.sscan_plan_select(ctypes.byref(d), kind, ctypes.byref(q)) == OK
            assert q.layout == layout, (kind, T)
    p = sscan_plan()
    p.layout = SG
    assert fwd(lib, desc(B=1, T=2 ** 24 - 1, D=4, DS=4), plan=p) == E_WS  # valid; needs its workspace
    assert fwd(lib, desc(B=1, T=2 ** 24, D=4, DS=4), plan=p) == E_UNSUP


def test_plan_select_per_forward_kind(lib):
    # 8x2048x768x16 (0.75 waves per SIMD in one pass): every forward, without H, keeping
    # boundary states or writing H, runs the state-group layout in one pass (192 workgroups
    # of 32 channels)
    d = desc(B=8, T=2048, D=768, DS=16)
    want = {0: (2, 8, 1), 3: (2, 8, 1), 4: (2, 8, 1)}
    for kind, (layout, lanes, chunks) in want.items():
        p = sscan_plan()
        assert lib.sscan_plan_select(ctypes.byref(d), kind, ctypes.byref(p)) == OK
        assert (p.layout, p.lanes, p.chunks) == (layout, lanes, chunks), kind
    # where the state-group layout cannot run (D not a multiple of 4), the forward keeping
    # boundary states splits the lanes layout to three waves per SIMD
    d = desc(B=8, T=2048, D=770, DS=16)
    p = sscan_plan()
    assert lib.sscan_plan_select(ctypes.byref(d), 4, ctypes.byref(p)) == OK
    assert (p.layout, p.lanes, p.chunks) == (1, 8, 4)
    # the forward writing H runs the state-group layout only at DS = 16, with 32-channel
    # workgroups from 128 of them up: 8x2048x768x8 and 2x2048x768x16 (48 workgroups) run lanes
    for B, DS in ((8, 8), (2, 16)):
        d = desc(B=B, T=2048, D=768, DS=DS)
        assert lib.sscan_plan_select(ctypes.byref(d), 3, ctypes.byref(p)) == OK
        assert p.layout == 1, (B, DS)
    # at two waves per SIMD or more nothing is split
    d = desc(B=16, T=4096, D=1024, DS=16)
    p = sscan_plan()
    assert lib.sscan_plan_select(ctypes.byref(d), 4, ctypes.byref(p)) == OK
    assert (p.layout, p.chunks) == (2, 1)
    # too few workgroups for one state-group pass: short sequences keep at least 128 steps
    # per chunk
    d = desc(B=1, T=300, D=64, DS=16)
    assert lib.sscan_plan_select(ctypes.byref(d), 4, ctypes.byref(p)) == OK
    assert (p.layout, p.chunks) == (1, 2)


def test_forward_workspace_covers_the_hfree_split(lib):
    # 8x2048x770x16 (the lanes layout: D is not a multiple of 4): the forward without H
    # splits into 5 T-chunks (800 waves in one pass: at most 5 chunks for four per SIMD),
    # the forward keeping boundary states into 4; one query serves both calls
    d = desc(B=8, T=2048, D=770, DS=16)
    n = ctypes.c_size_t()
    assert lib.sscan_fwd_workspace(ctypes.byref(d), None, ctypes.byref(n)) == OK
    assert n.value >= 3 * 8 * 770 * 16 * 8
    p = sscan_plan()
    assert lib.sscan_plan_select(ctypes.byref(d), 0, ctypes.byref(p)) == OK
    assert (p.layout, p.chunks) == (1, 5)  # the lanes layout, 5 chunks of at most 7 tiles
    # 8x2048x768x16: both forwards run one state-group pass (packed b/c, 2 MB)
    d = desc(B=8, T=2048, D=768, DS=16)
    assert lib.sscan_fwd_workspace(ctypes.byref(d), None, ctypes.byref(n)) == OK
    assert n.value >= 8 * 2048 * 2 * 16 * 4
    # a chunk count the caller fixes is used as given for both calls
    p = sscan_plan()
    p.lanes, p.chunks = 8, 2
    assert lib.sscan_fwd_workspace(ctypes.byref(d), ctypes.byref(p), ctypes.byref(n)) == OK
    # (one block of carry pairs, plus the state-group layout's packed b/c for the plain forward)
    assert 1 * 8 * 768 * 16 * 8 <= n.value < 3 * 8 * 768 * 16 * 8 + 8 * 2048 * 2 * 16 * 4 + 4096


def test_forward_workspace_required_for_chunked_plan(lib):
    p = sscan_plan()
    p.lanes, p.chunks = 4, 4
    n = ctypes.c_size_t()
    d = desc(B=2, T=64, D=16, DS=4)
    assert lib.sscan_fwd_workspace(ctypes.byref(d), ctypes.byref(p), ctypes.byref(n)) == OK
    assert n.value > 0
    assert fwd(lib, d, plan=p) == E_WS
    assert fwd(lib, d, plan=p, ws=FAKE, ws_bytes=n.value - 1) == E_WS


def test_backward_validation(lib):
    assert bwd(lib, desc(), H=None) == E_NULL
    assert bwd(lib, desc(), gA=None) == E_NULL
    assert bwd(lib, desc(), dy=None) == E_NULL
    assert bwd(lib, desc(), gA=FAKE + 4) == E_ALIGN
    assert bwd(lib, desc(), gx=FAKE + 2) == E_ALIGN
    assert bwd(lib, desc()) == E_WS  # workspace is always needed when there are steps
    p = sscan_plan()
    p.chunks = -2
    d = desc()
    assert lib.sscan_bwd(ctypes.byref(d), ctypes.byref(p), *([None] * 15), None, ctypes.c_size_t(0), None) == E_UNSUP


def test_backward_chunked_workspace_grows_with_chunks(lib):
    d = desc(B=2, T=1000, D=64, DS=16)
    sizes = []
    for c in (1, 2, 4):
        p = sscan_plan()
        p.lanes, p.chunks = 16, c
        n = ctypes.c_size_t()
        assert lib.sscan_bwd_workspace(ctypes.byref(d), ctypes.byref(p), ctypes.byref(n)) == OK
        sizes.append(n.value)
    assert sizes[0] < sizes[1] < sizes[2]


def test_empty_problems_need_no_pointers(lib):
    # B == 0 or D == 0: nothing to compute and nothing to write in the forward.
    assert fwd(lib, desc(B=0), x=None, delta=None, A=None, b=None, c=None, y=None, hT=None) == OK
    assert fwd(lib, desc(D=0), x=None, delta=None, A=None, b=None, c=None, y=None, hT=None) == OK
    # T == 0 with no hT requested: nothing to write.
    assert fwd(lib, desc(T=0), x=None, delta=None, A=None, b=None, c=None, y=None, hT=None) == OK


def test_plan_select_and_workspace_sizes(lib):
    cases = {(16, 4096, 1024, 16): 8, (4, 2048, 2048, 16): 8, (8, 2048, 768, 16): 8, (1, 64, 16, 4): 4,
             (16, 2048, 2048, 4): 2}  # state groups run DS/2 threads per channel
    for (B, T, D, DS), lanes in cases.items():
        d = desc(B=B, T=T, D=D, DS=DS)
        p = sscan_plan()
        assert lib.sscan_plan_select(ctypes.byref(d), 0, ctypes.byref(p)) == OK
        assert p.lanes == lanes, (B, T, D, DS, p.lanes)
    # the small fp32 workload splits its sequence to fill the GPU (256 waves in one pass:
    # 16 chunks of one 64-step tile, four waves per SIMD)
    d = desc(B=8, T=1024, D=256, DS=16)
    p = sscan_plan()
    assert lib.sscan_plan_select(ctypes.byref(d), 0, ctypes.byref(p)) == OK
    assert p.lanes == 8 and p.chunks == 16
    assert lib.sscan_plan_select(ctypes.byref(d), 1, ctypes.byref(p)) == OK
    assert p.lanes == 4 and p.chunks == 16  # 2048 channels x 4 lanes x 16 chunks = 2 waves per SIMD (T caps it)
    d = desc(B=8, T=2048, D=768, DS=16)
    assert lib.sscan_plan_select(ctypes.byref(d), 1, ctypes.byref(p)) == OK
    assert p.lanes == 4 and p.chunks == 8  # 0.375 -> 3 waves per SIMD
    # below DS = 16: four states per lane, more lanes per channel where 16 chunks would still
    # leave under three waves per SIMD
    for (B, T, D, DS), lanes in {(16, 2048, 2048, 4): 1, (32, 1024, 1024, 8): 2, (2, 8192, 512, 8): 8,
                                 (8, 4096, 256, 4): 4, (2, 50, 7, 2): 2}.items():
        dd = desc(B=B, T=T, D=D, DS=DS)
        assert lib.sscan_plan_select(ctypes.byref(dd), 1, ctypes.byref(p)) == OK
        assert p.lanes == lanes, (B, T, D, DS, p.lanes)
    assert lib.sscan_plan_select(ctypes.byref(d), 2, ctypes.byref(p)) == OK  # the wrapper's backward
    assert p.lanes == 4 and p.chunks == 8
    # backward partial buffers: one (gb, gc) pair per channel tile, step and state, plus gA per batch row
    d = desc(B=8, T=2048, D=768, DS=16)
    n = ctypes.c_size_t()
    assert lib.sscan_bwd_workspace(ctypes.byref(d), None, ctypes.byref(n)) == OK
    tiles = (768 + 63) // 64
    assert n.value >= tiles * 8 * 2048 * 16 * 8 + 8 * 768 * 16 * 4


def dec(lib, d, x=FAKE, delta=FAKE, A=FAKE, b=FAKE, c=FAKE, si=FAKE, so=FAKE + 0x10000, y=FAKE):
    v = lambda p: None if p is None else ctypes.c_void_p(p)
    return lib.sscan_decode(ctypes.byref(d), v(x), v(delta), v(A), v(b), v(c), v(si), v(so), v(y), None)


def test_decode_validation(lib):
    assert dec(lib, desc(T=2)) == E_SHAPE           # one step only
    assert dec(lib, desc(T=0)) == E_SHAPE
    assert dec(lib, desc(T=1), si=None) == E_NULL
    assert dec(lib, desc(T=1), y=None) == E_NULL
    assert dec(lib, desc(T=1), si=FAKE + 4) == E_ALIGN
    assert dec(lib, desc(T=1, io=1), x=FAKE + 1) == E_ALIGN
    # B=2, D=16, DS=4: the state is 512 bytes; a partial overlap is refused, identity is not
    assert dec(lib, desc(T=1), si=FAKE, so=FAKE + 256) == E_SHAPE
    assert dec(lib, desc(T=1, DS=3)) == E_UNSUP
    # nothing to do: no pointer is looked at
    assert dec(lib, desc(B=0, T=1), x=None, delta=None, A=None, b=None, c=None, si=None, so=None, y=None) == OK


def test_ckpt_validation(lib):
    p = sscan_plan()
    n = ctypes.c_size_t()
    # the H-free backward runs 8 or 16 lanes per channel: DS >= 8, plan.lanes >= 8
    assert lib.sscan_bwd_ckpt_workspace(ctypes.byref(desc(DS=4)), None, 0, ctypes.byref(n)) == E_UNSUP
    p.lanes = 4
    assert lib.sscan_bwd_ckpt_workspace(ctypes.byref(desc(DS=16)), ctypes.byref(p), 0, ctypes.byref(n)) == E_UNSUP
    assert lib.sscan_bwd_ckpt_workspace(ctypes.byref(desc(DS=16)), None, 7, ctypes.byref(n)) == E_UNSUP
    assert lib.sscan_bwd_ckpt_workspace(ctypes.byref(desc(DS=16)), None, 1, ctypes.byref(n)) == OK
    v = lambda a: ctypes.c_void_p(a)
    # forward: hck required, H-free and wrapper checks happen before any launch
    d = desc(DS=16)
    assert lib.sscan_fwd_ckpt(ctypes.byref(d), None, 0, *([v(FAKE)] * 5), None, None, v(FAKE), None, None, None,
                              ctypes.c_size_t(0), None) == E_NULL
    assert lib.sscan_fwd_ckpt(ctypes.byref(d), None, 3, *([v(FAKE)] * 5), None, None, v(FAKE), None, v(FAKE), None,
                              ctypes.c_size_t(0), None) == E_UNSUP
    assert lib.sscan_fwd_ckpt(ctypes.byref(d), None, 0, *([v(FAKE)] * 5), None, None, v(FAKE), None, v(FAKE + 4),
                              None, ctypes.c_size_t(0), None) == E_ALIGN
    # backward: hck required
    assert lib.sscan_bwd_ckpt(ctypes.byref(d), None, 0, *([None] * 16), None, ctypes.c_size_t(0), None) == E_NULL


def test_micro_library_rejects_bad_arguments_before_any_gpu_call():
    # the microbenchmark library (bench.py --micro) is built with libsscan and checks its
    # arguments on the host: these return 1 without touching a device
    path = os.path.join(os.path.dirname(_lib.LIB_PATH), "libsscan_micro.so")
    if not os.path.exists(path):
        pytest.skip("libsscan_micro.so is not built")
    m = ctypes.CDLL(path)
    m.sscan_micro_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.POINTER(ctypes.c_double)]
    m.sscan_micro_rate.restype = ctypes.c_int
    r = ctypes.c_double()
    assert m.sscan_micro_rate(0, 1, 0, None) == 1                         # no output
    assert m.sscan_micro_rate(9, 1, 0, ctypes.byref(r)) == 1              # unknown kernel
    assert m.sscan_micro_rate(-1, 1, 0, ctypes.byref(r)) == 1
    assert m.sscan_micro_rate(0, 0, 0, ctypes.byref(r)) == 1              # waves per SIMD out of 1..8
    assert m.sscan_micro_rate(0, 9, 0, ctypes.byref(r)) == 1
    assert m.sscan_micro_rate(5, 1, 0, ctypes.byref(r)) == 1              # stream size missing
    assert m.sscan_micro_rate(6, 1, 1000, ctypes.byref(r)) == 1           # not a multiple of 16
    assert m.sscan_micro_rate(7, 1, (16 << 30) + 16, ctypes.byref(r)) == 1  # above 16 GiB


def noalloc(lib, d, plan=None, x=FAKE, delta=FAKE, A=FAKE, b=FAKE, c=FAKE, h0=None, y=FAKE, hT=FAKE, H=None):
    v = lambda p: None if p is None else ctypes.c_void_p(p)
    return lib.sscan_fwd_noalloc(ctypes.byref(d), None if plan is None else ctypes.byref(plan), v(x), v(delta),
                                 v(A), v(b), v(c), v(h0), v(y), v(hT), v(H), None)


def test_noalloc_forward_validates_before_any_gpu_call(lib):
    """The allocation-free forward rejects, without a GPU, bad arguments and a problem whose
    scratch exceeds its static array (the state-group layout packs B*T*2*DS floats of b, c:
    64 x 65536 x 32 x 4 B = 512 MiB > 32 MiB)."""
    assert noalloc(lib, desc(), x=None) == E_NULL
    assert noalloc(lib, desc(), y=FAKE + 2) == E_ALIGN
    assert noalloc(lib, desc(DS=3)) == E_UNSUP
    big = desc(B=64, T=65536, D=4, DS=16)
    plan = sscan_plan()
    plan.layout = 2  # state groups
    plan.chunks = 1
    assert noalloc(lib, big, plan=plan) == E_WS
    assert b"32 MiB" in lib.sscan_last_error() or b"33554432" in lib.sscan_last_error()
    n = ctypes.c_size_t(0)
    assert lib.sscan_fwd_workspace(ctypes.byref(big), ctypes.byref(plan), ctypes.byref(n)) == OK
    assert n.value > _lib.SSCAN_NOALLOC_SCRATCH_BYTES
    # problems with nothing to do need no scratch and no GPU
    assert noalloc(lib, desc(B=0)) == OK
    assert noalloc(lib, desc(D=0)) == OK


def test_forward_workspace_with_a_state_group_plan_below_ds16(lib):
    # a plan forcing the state-group layout at DS = 8 is valid for the forwards without H
    # (the query sizes them) and not for one writing H (which the query then leaves out)
    p = sscan_plan()
    p.layout, p.chunks = 2, 2
    d = desc(B=2, T=63, D=4, DS=8)
    n = ctypes.c_size_t()
    assert lib.sscan_fwd_workspace(ctypes.byref(d), ctypes.byref(p), ctypes.byref(n)) == OK
    assert n.value >= 2 * 64 * 2 * 8 * 4
    assert fwd(lib, d, plan=p, H=FAKE) == E_UNSUP
