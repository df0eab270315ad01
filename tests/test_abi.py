"""C ABI checks that need no GPU: the library loads, exports every function
the header declares, and rejects bad arguments on the host before any HIP
call (only invalid argument sets are passed here, so nothing is launched)."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

q4 = pytest.importorskip("bit_weight_only_q4g128_amd")
lib = q4.lib

OK, EPTR, ESHAPE, EALIGN, EALIAS, ELAUNCH, EVARIANT = 0, -1, -2, -3, -4, -5, -6
A = 0x10000000  # a 16-byte aligned fake device address; never dereferenced


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names += re.findall(r"^\s*(?:int|size_t|const\s+char\s*\*)\s+(\w+)\s*\(", src, flags=re.M)
    return names


def test_header_declares_the_boundary():
    names = set(declared_functions())
    for must in ("q4g128_gemv", "nvfp4g16_gemv", "bf16_gemv", "q4g128_dequant_f32", "nvfp4g16_dequant_f32"):
        assert must in names


@pytest.mark.parametrize("name", declared_functions())
def test_symbol_exported(name):
    assert hasattr(lib, name), name


def test_version_and_strerror():
    assert lib.q4gemv_version() >= 100
    for rc in (OK, EPTR, ESHAPE, EALIGN, EALIAS, ELAUNCH, EVARIANT):
        assert q4.strerror(rc) and q4.strerror(rc) != "unknown status"
    assert q4.strerror(-99) == "unknown status"


def q4call(x=A, M=1, K=2048, qw=A + (1 << 24), sc=A + (2 << 24), mn=A + (3 << 24), N=2048, y=A + (4 << 24), variant=0):
    return lib.q4g128_gemv_variant(x, M, K, qw, sc, mn, N, y, variant, None)


@pytest.mark.parametrize("kw,rc", [
    (dict(x=None), EPTR), (dict(qw=None), EPTR), (dict(sc=None), EPTR), (dict(mn=None), EPTR), (dict(y=None), EPTR),
    (dict(M=0), ESHAPE), (dict(M=65), ESHAPE), (dict(N=0), ESHAPE), (dict(K=0), ESHAPE), (dict(K=192), ESHAPE),
    (dict(K=2048 + 64), ESHAPE), (dict(x=A + 2), EALIGN), (dict(qw=A + (1 << 24) + 8), EALIGN),
    (dict(sc=A + (2 << 24) + 1), EALIGN), (dict(y=A + (4 << 24) + 1), EALIGN),
    (dict(y=A + (1 << 24) + 64), EALIAS), (dict(y=A + 16), EALIAS), (dict(y=A + (3 << 24)), EALIAS),
    (dict(variant=5), EVARIANT), (dict(variant=-1), EVARIANT), (dict(variant=3, M=5), EVARIANT),
    (dict(variant=4, M=64, K=32768, N=64), EVARIANT),
    (dict(variant=3, K=1024), EVARIANT),
])
def test_q4_validation(kw, rc):
    assert q4call(**kw) == rc


def nvcall(x=A, M=1, K=2048, qw=A + (1 << 24), sc=A + (2 << 24), G=1.0, N=2048, y=A + (4 << 24), variant=0):
    return lib.nvfp4g16_gemv_variant(x, M, K, qw, sc, G, N, y, variant, None)


@pytest.mark.parametrize("kw,rc", [
    (dict(x=None), EPTR), (dict(sc=None), EPTR), (dict(K=48), ESHAPE), (dict(M=100), ESHAPE),
    (dict(qw=A + (1 << 24) + 4), EALIGN), (dict(y=A + (2 << 24)), EALIAS), (dict(variant=9), EVARIANT),
])
def test_nvfp4_validation(kw, rc):
    assert nvcall(**kw) == rc


def bfcall(x=A, M=1, K=2048, w=A + (1 << 24), N=2049, y=A + (4 << 24), variant=0):
    return lib.bf16_gemv_variant(x, M, K, w, N, y, variant, None)


@pytest.mark.parametrize("kw,rc", [
    (dict(w=None), EPTR), (dict(K=12), ESHAPE), (dict(N=-1), ESHAPE), (dict(w=A + (1 << 24) + 2), EALIGN),
    (dict(y=A + (1 << 24) + 100), EALIAS), (dict(variant=5), EVARIANT),
])
def test_bf16_validation(kw, rc):
    assert bfcall(**kw) == rc


def test_dequant_validation():
    assert lib.q4g128_dequant_f32(None, A, A, 1, 128, A, None) == EPTR
    assert lib.q4g128_dequant_f32(A, A + (1 << 24), A + (2 << 24), 1, 100, A + (3 << 24), None) == ESHAPE
    assert lib.q4g128_dequant_f32(A, A + (1 << 24), A + (2 << 24), 1, 128, A + (3 << 24) + 4, None) == EALIGN
    assert lib.q4g128_dequant_f32(A, A + (1 << 24), A + (2 << 24), 4, 128, A, None) == EALIAS
    assert lib.nvfp4g16_dequant_f32(A, None, 1.0, 1, 32, A, None) == EPTR
    assert lib.nvfp4g16_dequant_f32(A, A + (1 << 24), 1.0, 1, 16, A + (2 << 24), None) == ESHAPE


def test_variant_names():
    assert q4.variant_name(q4.FMT_Q4G128, q4.VARIANT_AUTO, 1, 2048, 2048) == "stream"
    assert q4.variant_name(q4.FMT_Q4G128, q4.VARIANT_AUTO, 2, 2048, 8192) == "stream"
    assert q4.variant_name(q4.FMT_Q4G128, q4.VARIANT_AUTO, 1, 256, 512) == "dot2"
    assert q4.variant_name(q4.FMT_Q4G128, q4.VARIANT_STREAM, 5, 2048, 2048) == "invalid"
    assert q4.variant_name(q4.FMT_BF16, q4.VARIANT_AUTO, 1, 16385, 2048) == "stream"
    assert q4.variant_name(q4.FMT_Q4G128, q4.VARIANT_AUTO, 48, 2048, 2048) == "skinny"
    assert q4.variant_name(q4.FMT_Q4G128, q4.VARIANT_AUTO, 5, 2048, 2048) == "skinny"
    assert q4.variant_name(q4.FMT_Q4G128, q4.VARIANT_AUTO, 49, 2048, 2048) == "tiled"
    assert q4.variant_name(q4.FMT_Q4G128, q4.VARIANT_AUTO, 48, 2048, 8192) == "tiled"     # no workspace: K > 16 groups
    assert q4.variant_name(q4.FMT_Q4G128, q4.VARIANT_TILED, 48, 2048, 2048) == "tiled"
    assert q4.variant_name(q4.FMT_Q4G128, 6, 4, 2048, 2048) == "invalid"                   # skinny: M >= 5
    assert q4.variant_name(q4.FMT_NVFP4G16, 6, 48, 2048, 2048) == "skinny"                 # skinny: every format
    assert q4.variant_name(q4.FMT_BF16, 6, 48, 2048, 1024) == "skinny"
    assert q4.variant_name(q4.FMT_BF16, 6, 48, 2048, 2048) == "invalid"                    # BF16 slices: 8 groups, no workspace
    assert q4.variant_name(q4.FMT_NVFP4G16, 6, 48, 2048, 2080) == "invalid"                # K % 128
    assert q4.variant_name(q4.FMT_Q4G128, q4.VARIANT_AUTO, 48, 2048, 16384) == "mfma"
    assert q4.variant_name(q4.FMT_Q4G128, q4.VARIANT_MFMA, 1, 2048, 2048) == "mfma"
    assert q4.variant_name(q4.FMT_BF16, q4.VARIANT_DOT2, 3, 16385, 2048) == "dot2"
    assert q4.variant_name(q4.FMT_NVFP4G16, q4.VARIANT_AUTO, 48, 8192, 2048) == "skinny"   # one slice of 16 groups
    assert q4.variant_name(q4.FMT_NVFP4G16, q4.VARIANT_AUTO, 48, 8192, 4096) == "mfma"    # no workspace: rows alone too few
    assert q4.variant_name(q4.FMT_NVFP4G16, q4.VARIANT_AUTO, 48, 16384, 2048) == "skinny"
    assert q4.variant_name(q4.FMT_NVFP4G16, q4.VARIANT_AUTO, 48, 16384, 4096) == "tiled"   # no workspace: K > 16 groups
    assert q4.variant_name(q4.FMT_NVFP4G16, q4.VARIANT_TILED, 48, 8192, 2048) == "tiled"
    assert q4.variant_name(q4.FMT_NVFP4G16, q4.VARIANT_AUTO, 48, 8192, 2080) == "mfma"   # K % 128 != 0
    assert q4.variant_name(q4.FMT_BF16, q4.VARIANT_AUTO, 48, 16385, 2048) == "tiled"      # no workspace: K > 8 groups
    assert q4.variant_name(q4.FMT_BF16, q4.VARIANT_AUTO, 48, 16385, 1024) == "skinny"
    assert q4.variant_name(q4.FMT_BF16, q4.VARIANT_AUTO, 48, 16385, 2056) == "mfma"
    assert q4.variant_name(q4.FMT_BF16, q4.VARIANT_TILED, 48, 16385, 2056) == "invalid"
    assert q4.variant_name(7, 0, 1, 1, 128) == "invalid"
    assert q4.variant_name(0, 0, 0, 1, 128) == "invalid"


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        q4.q4g128_gemv(x, torch.zeros(1, 64, dtype=torch.uint8), torch.zeros(1, 1, dtype=torch.float16),
                       torch.zeros(1, 1, dtype=torch.float16))


def test_grouped_validation():
    T = q4.Q4Task
    def task(i, **kw):
        base = dict(x=A + (i << 26), qweight=A + (i << 26) + (1 << 24), scale=A + (i << 26) + (2 << 24),
                    minv=A + (i << 26) + (3 << 24), y=A + (i << 26) + (4 << 24), N=2048, K=2048)
        base.update(kw)
        return T(**base)
    arr = (T * 3)(task(0), task(1), task(2))
    assert lib.q4g128_gemv_grouped(None, 1, 1, 0, None) == EPTR
    assert lib.q4g128_gemv_grouped(arr, 0, 1, 0, None) == ESHAPE
    assert lib.q4g128_gemv_grouped(arr, 9, 1, 0, None) == ESHAPE
    assert lib.q4g128_gemv_grouped(arr, 3, 0, 0, None) == ESHAPE
    assert lib.q4g128_gemv_grouped(arr, 3, 1, 5, None) == EVARIANT
    assert lib.q4g128_gemv_grouped_ws(arr, 3, 1, 0, A + 1, 4096, None) == EALIGN
    import ctypes
    assert lib.q4g128_workspace_bytes(arr, 3, 48, None) == EPTR
    def far(i):   # disjoint address ranges (nothing is launched)
        b = A + (i << 29)
        return T(x=b, qweight=b + (1 << 26), scale=b + (2 << 26), minv=b + (3 << 26), y=b + (4 << 26), N=2048, K=2048)
    ok3 = (T * 3)(far(0), far(1), far(2))
    nb = ctypes.c_size_t(123)
    assert lib.q4g128_workspace_bytes(ok3, 3, 1, ctypes.byref(nb)) == OK and nb.value == 0   # M = 1 never splits
    # three 2048-row tasks at M = 48, K = 2048: the skinny kernel's 32-row
    # blocks fill the GPU whole (192 workgroups), no split
    assert lib.q4g128_workspace_bytes(ok3, 3, 48, ctypes.byref(nb)) == OK and nb.value == 0
    # K = 8192 exceeds one workgroup slice: split with a workspace
    ok3k = (T * 3)(*[T(x=t.x, qweight=t.qweight, scale=t.scale, minv=t.minv, y=t.y, N=2048, K=8192) for t in ok3])
    assert lib.q4g128_workspace_bytes(ok3k, 3, 48, ctypes.byref(nb)) == OK and nb.value > 64 * 1024
    # the tiled kernel (M = 64) splits the 2048-column tasks
    assert lib.q4g128_workspace_bytes(ok3, 3, 64, ctypes.byref(nb)) == OK and nb.value > 0
    bad = (T * 2)(task(0), task(1, K=100))
    assert lib.q4g128_gemv_grouped(bad, 2, 1, 0, None) == ESHAPE
    # task 1 writes over task 0's weights
    alias = (T * 2)(task(0), task(1, y=A + (1 << 24) + 4096))
    assert lib.q4g128_gemv_grouped(alias, 2, 1, 0, None) == EALIAS
    # two tasks share an output
    same = (T * 2)(task(0), task(1, y=A + (4 << 24)))
    assert lib.q4g128_gemv_grouped(same, 2, 1, 0, None) == EALIAS


def test_grouped_nvfp4_bf16_validation():
    import ctypes
    NT, BT = q4.NvTask, q4.BfTask
    def nv(i, **kw):
        b = A + (i << 29)
        base = dict(x=b, qweight=b + (1 << 26), scale_e4m3=b + (2 << 26), global_scale=1.0, y=b + (4 << 26), N=2048, K=2048)
        base.update(kw)
        return NT(**base)
    def bf(i, **kw):
        b = A + (i << 29)
        base = dict(x=b, w=b + (1 << 26), y=b + (4 << 26), N=2048, K=2048)
        base.update(kw)
        return BT(**base)
    for fn, mk, T in ((lib.nvfp4g16_gemv_grouped_ws, nv, NT), (lib.bf16_gemv_grouped_ws, bf, BT)):
        arr = (T * 2)(mk(0), mk(1))
        assert fn(None, 1, 1, 0, None, 0, None) == EPTR
        assert fn(arr, 0, 1, 0, None, 0, None) == ESHAPE
        assert fn(arr, 9, 1, 0, None, 0, None) == ESHAPE
        assert fn(arr, 2, 65, 0, None, 0, None) == ESHAPE
        assert fn(arr, 2, 1, 7, None, 0, None) == EVARIANT
        assert fn(arr, 2, 48, 4, A + 8, 4096, None) == EALIGN
        assert fn((T * 2)(mk(0), mk(1, x=None)), 2, 1, 0, None, 0, None) == EPTR
        same = (T * 2)(mk(0), mk(1, y=A + (4 << 26)))
        assert fn(same, 2, 1, 0, None, 0, None) == EALIAS
        over = (T * 2)(mk(0), mk(1, y=A + (1 << 26) + 64))   # task 1 writes over task 0's weights
        assert fn(over, 2, 1, 0, None, 0, None) == EALIAS
    assert lib.nvfp4g16_gemv_grouped_ws((NT * 1)(nv(0, K=48)), 1, 1, 0, None, 0, None) == ESHAPE
    assert lib.nvfp4g16_gemv_grouped_ws((NT * 1)(nv(0, qweight=A + (1 << 26) + 8)), 1, 1, 0, None, 0, None) == EALIGN
    assert lib.bf16_gemv_grouped_ws((BT * 1)(bf(0, K=12)), 1, 1, 0, None, 0, None) == ESHAPE
    # the tiled kernel needs K % 128 == 0
    assert lib.bf16_gemv_grouped_ws((BT * 1)(bf(0, K=2056)), 1, 48, 4, None, 0, None) == EVARIANT
    nb = ctypes.c_size_t(123)
    for fnb, mk, T in ((lib.nvfp4g16_workspace_bytes, nv, NT), (lib.bf16_workspace_bytes, bf, BT)):
        arr = (T * 2)(mk(0), mk(1))
        assert fnb(arr, 2, 48, None) == EPTR
        assert fnb(arr, 2, 1, ctypes.byref(nb)) == OK and nb.value == 0     # M = 1 never splits
        assert fnb(arr, 2, 48, ctypes.byref(nb)) == OK
        # the skinny kernel: NVFP4 K = 2048 is one slice of 16 groups; BF16
        # slices hold 8 groups, so its K = 2048 is split
        assert (nb.value > 0) == (T is BT)


def test_fused_validation():
    """q4g128_gemv_fused / q4g128_fused_workspace_bytes reject bad arguments
    on the host (the size query never launches anything)."""
    FT = q4.FusedTask

    def ft(i, **kw):
        b = A + (i << 29)
        base = dict(x=b, up=b + (5 << 26), qweight=b + (1 << 26), scale=b + (2 << 26), minv=b + (3 << 26),
                    residual=b + (6 << 26), y=b + (4 << 26), N=2048, K=2048)
        base.update(kw)
        return FT(**base)

    nb = ctypes.c_size_t(123)

    def size(tasks, M=1):
        arr = (FT * len(tasks))(*tasks)
        return lib.q4g128_fused_workspace_bytes(arr, len(tasks), M, ctypes.byref(nb))

    def call(tasks, M=1):
        arr = (FT * len(tasks))(*tasks)
        return lib.q4g128_gemv_fused(arr, len(tasks), M, None, 0, None)

    assert lib.q4g128_gemv_fused(None, 1, 1, None, 0, None) == EPTR
    assert lib.q4g128_fused_workspace_bytes((FT * 1)(ft(0)), 1, 1, None) == EPTR
    assert size([ft(0)]) == OK and nb.value == 0                       # M = 1: the streaming kernel, no split
    assert size([ft(0), ft(1)], M=48) == OK and nb.value > 0            # M = 48: the tiled kernel splits K
    assert size([ft(0, up=None, residual=None)]) == OK
    assert size([ft(0, residual=A + (4 << 26))]) == OK                  # in place: residual is y
    assert call([ft(i) for i in range(9)]) == ESHAPE
    assert call([ft(0)], M=0) == ESHAPE
    assert call([ft(0)], M=65) == ESHAPE
    assert call([ft(0, x=None)]) == EPTR
    assert call([ft(0, up=A + (5 << 26) + 8)]) == EALIGN
    assert call([ft(0, residual=A + (6 << 26) + 1)]) == EALIGN
    assert call([ft(0, y=A + (5 << 26) + 64)]) == EALIAS               # over its own up activations
    assert call([ft(0, residual=A + (4 << 26) + 2)]) == EALIAS         # residual partly over y
    # a workspace must be 256-byte aligned (rejected before anything is planned)
    assert lib.q4g128_gemv_fused((FT * 1)(ft(0)), 1, 48, A + (7 << 26) + 16, 1 << 20, None) == EALIGN
    # the h buffers never start inside the 64 KiB counter region, also when no K split is planned
    assert size([ft(0, K=512, N=256, residual=None)], M=16) == OK and nb.value >= 64 * 1024 + 16 * 512 * 2
    assert call([ft(0), ft(1, y=A + (6 << 26))]) == EALIAS              # over another task's residual
    assert call([ft(0), ft(1, y=A + (4 << 26))]) == EALIAS              # two tasks share an output
    assert call([ft(0, K=32768, N=64)], M=64) == EVARIANT               # unsplit tiled kernel: too many groups


def test_sample_validation():
    """q4_sample_topk / bf16_head_sample reject bad arguments before any launch."""
    L, U, T = A, A + (1 << 26), A + (2 << 26)          # logits, u, token
    TI, TP = A + (3 << 26), A + (4 << 26)
    f = ctypes.c_float

    def s(logits=L, M=1, V=2049, temp=0.8, k=30, u=U, tok=T, ti=TI, tp=TP):
        return lib.q4_sample_topk(logits, M, V, f(temp), k, u, tok, ti, tp, None)

    assert s(logits=None) == EPTR and s(u=None) == EPTR and s(tok=None) == EPTR
    for kw in (dict(M=0), dict(V=0), dict(V=30721), dict(k=0), dict(k=65), dict(V=20, k=21), dict(temp=0.0), dict(temp=-1.0),
               dict(temp=float("inf")), dict(temp=float("nan"))):
        assert s(**kw) == ESHAPE, kw
    assert s(logits=L + 1) == EALIGN and s(u=U + 2) == EALIGN and s(tok=T + 2) == EALIGN and s(tp=TP + 2) == EALIGN
    assert s(tok=L + 64) == EALIAS            # token over the logits
    assert s(ti=U) == EALIAS                  # indices over the draws
    assert s(tp=T) == EALIAS                  # probabilities over the tokens
    X, W, LG = A + (5 << 29), A + (6 << 29), A + (7 << 29)   # far apart: a 40000 x 2048 weight spans 164 MB

    def h(x=X, w=W, lg=LG, tok=T, ti=None, tp=None, M=1, K=2048, N=2049, k=30):
        return lib.bf16_head_sample(x, M, K, w, N, lg, f(0.8), k, U, tok, ti, tp, None)

    assert h(x=None) == EPTR and h(lg=None) == EPTR
    assert h(M=0) == ESHAPE and h(K=12) == ESHAPE and h(N=40000) == ESHAPE
    assert h(lg=W + 64) == EALIAS             # logits over the weights
    assert h(tok=X) == EALIAS                 # token over the activations
    assert h(ti=W + 128) == EALIAS
    assert h(lg=U - 64) == EALIAS             # logits written over the uniforms before they are read

    # the one-launch form: workspace size rule, alignment and aliasing (checked before any launch)
    wsb = lib.bf16_head_sample_workspace_bytes
    wsb.restype = ctypes.c_size_t
    assert wsb(1, 2049, 2048, 30) > 0                      # one block of workgroups: counters only
    assert wsb(1, 16385, 2048, 30) > wsb(1, 2049, 2048, 30)   # blocks of workgroups: counters + candidates
    assert wsb(1, 2049, 1000, 30) == 0 and wsb(1, 2049, 2048, 65) == 0
    # a batch: the split sampler (counters a cache line apart per row, then
    # ceil(N / 1024) x top_k candidates per row), any K; nothing for one block
    assert wsb(2, 2049, 1000, 30) == 2 * 128 + 2 * 3 * 30 * 4
    assert wsb(48, 16385, 2048, 64) == 48 * 128 + 48 * 17 * 64 * 4
    assert wsb(2, 1024, 2048, 30) == 0 and wsb(65, 2049, 2048, 30) == 0 and wsb(2, 30721, 2048, 30) == 0
    WS = A + (1 << 30) + (1 << 29)

    def hw(ws=WS, nb=1 << 20, lg=LG, tok=T, N=16385):
        return lib.bf16_head_sample_ws(X, 1, 2048, W, N, lg, f(0.8), 30, U, tok, None, None, ws, nb, None)

    assert hw(ws=WS + 2) == EALIGN
    assert hw(ws=LG + 4096) == EALIAS                       # over the logits
    assert hw(ws=W + 4096) == EALIAS                        # over the weights
    assert hw(ws=T - 128) == EALIAS                         # over the tokens
    assert hw(lg=W + 64) == EALIAS                          # the head checks still apply


def test_mixed_validation():
    """q4gemv_grouped_mixed / q4gemv_mixed_workspace_bytes reject bad arguments
    on the host (the size query never launches anything)."""
    MT = q4.MixedTask
    FQ, FN, FB = q4.FMT_Q4G128, q4.FMT_NVFP4G16, q4.FMT_BF16

    def mt(i, fmt=FQ, **kw):
        b = A + (i << 29)
        base = dict(format=fmt, x=b, weight=b + (1 << 26), scale=b + (2 << 26), minv=b + (3 << 26), global_scale=1.0,
                    y=b + (4 << 26), N=2048, K=2048)
        base.update(kw)
        return MT(**base)

    nb = ctypes.c_size_t(7)

    def size(tasks, M=1):
        return lib.q4gemv_mixed_workspace_bytes((MT * len(tasks))(*tasks), len(tasks), M, ctypes.byref(nb))

    def call(tasks, M=1):
        return lib.q4gemv_grouped_mixed((MT * len(tasks))(*tasks), len(tasks), M, None, 0, None)

    mixed = [mt(0, FN), mt(1, FB), mt(2, FQ)]
    assert size(mixed) == OK and nb.value == 0                 # one streaming launch: no workspace
    assert size(mixed, M=48) == OK and nb.value > 0            # one tiled launch per format, K splits
    assert lib.q4gemv_grouped_mixed(None, 1, 1, None, 0, None) == EPTR
    assert call([mt(i) for i in range(9)]) == ESHAPE
    assert call([mt(0, fmt=5)]) == ESHAPE
    assert call([mt(0, FN, scale=None)]) == EPTR
    assert call([mt(0, FB, K=12)]) == ESHAPE
    assert call([mt(0, FN, weight=A + (1 << 26) + 8)]) == EALIGN
    assert call([mt(0, FN), mt(1, FB, y=A + (1 << 26) + 64)]) == EALIAS   # over another task's weights
    assert call([mt(0, FN), mt(1, FB, y=A + (4 << 26))]) == EALIAS        # two tasks share an output


def test_gemm_validation():
    """q4g128_gemm_variant rejects bad arguments on the host: the variant (only
    AUTO, TILED and GEMM), M, K, pointers, alignment and aliasing; the chunked
    kernel's K limit under an explicit TILED; M <= 64 under AUTO is the GEMV
    (the GEMV's M limit does not apply to the prefill variants)."""
    lib.q4g128_gemm_variant.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]

    def call(x=A, M=1024, K=2048, qw=A + (1 << 28), sc=A + (2 << 28), mn=A + (3 << 28), N=2048, y=A + (4 << 28), variant=5):
        return lib.q4g128_gemm_variant(x, M, K, qw, sc, mn, N, y, variant, None)

    assert call(variant=1) == EVARIANT                     # a GEMV-only variant
    assert call(variant=3) == EVARIANT
    assert call(variant=9) == EVARIANT
    assert call(M=0) == ESHAPE
    assert call(M=(1 << 19) + 1) == ESHAPE
    assert call(K=2000) == ESHAPE                          # K % 128
    assert call(K=65536) == ESHAPE                         # beyond the library's K limit
    assert call(x=None) == EPTR
    assert call(mn=None) == EPTR
    assert call(qw=A + (1 << 28) + 8) == EALIGN
    assert call(y=A + (1 << 21)) == EALIAS                 # y [1024, 2048] overlaps x [1024, 2048] (4 MiB)
    assert call(K=32768, variant=4) == EVARIANT            # the chunked kernel's LDS limit
    assert call(M=65, variant=0, x=None) == EPTR           # AUTO above 64 rows: prefill checks
    assert call(M=1, variant=0, K=2000) == ESHAPE          # AUTO at M <= 64: the GEMV's checks


def test_stream_read_validation():
    import ctypes
    lib.q4gemv_stream_read.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_size_t), ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.q4gemv_stream_read_sink_words.argtypes = [ctypes.POINTER(ctypes.c_size_t), ctypes.c_int]
    lib.q4gemv_stream_read_sink_words.restype = ctypes.c_size_t
    P, S = ctypes.c_void_p, ctypes.c_size_t
    bufs = (P * 2)(A, A + (1 << 24))
    sizes = (S * 2)(1 << 20, 4096)
    # 16 KB per workgroup, 4 words per workgroup: 64 + 1 workgroups
    need = lib.q4gemv_stream_read_sink_words(sizes, 2)
    assert need == (64 + 1) * 4
    assert lib.q4gemv_stream_read_sink_words(sizes, 0) == 0
    assert lib.q4gemv_stream_read_sink_words((S * 1)(8), 1) == 0
    sink = A + (2 << 24)
    assert lib.q4gemv_stream_read(None, sizes, 2, sink, need, None) == EPTR
    assert lib.q4gemv_stream_read(bufs, sizes, 2, None, need, None) == EPTR
    assert lib.q4gemv_stream_read((P * 2)(A, None), sizes, 2, sink, need, None) == EPTR
    assert lib.q4gemv_stream_read(bufs, sizes, 0, sink, need, None) == ESHAPE
    assert lib.q4gemv_stream_read(bufs, sizes, 33, sink, need, None) == ESHAPE
    assert lib.q4gemv_stream_read(bufs, (S * 2)(1 << 20, 8), 2, sink, need, None) == ESHAPE
    assert lib.q4gemv_stream_read(bufs, sizes, 2, sink, need - 1, None) == ESHAPE
    assert lib.q4gemv_stream_read((P * 2)(A + 2, A + (1 << 24)), sizes, 2, sink, need, None) == EALIGN
    assert lib.q4gemv_stream_read(bufs, sizes, 2, sink + 2, need, None) == EALIGN
    assert lib.q4gemv_stream_read(bufs, sizes, 2, A + 4096, need, None) == EALIAS
