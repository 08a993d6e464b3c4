"""C-ABI library: it loads, exports every function include/moeq.h declares,
and rejects bad arguments on the host with the documented status before any
HIP call (these tests need no GPU)."""
import ctypes as C
import os
import re

import pytest

import quantized_moe_grouped_route_amd as mq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moeq.h")

# Fake device addresses: only their values are inspected on these paths.
A16 = 0x10000
ODD = 0x10001


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                          text, flags=re.M))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mq.LIB_PATH):
        pytest.skip("libmoeq.so not built")
    return mq.lib()


def test_header_declares_the_five_entry_points():
    fns = declared_functions()
    for f in ("moe_route_prep", "grouped_gemm_qint4", "grouped_gemm_qfp8_block",
              "grouped_gemm_qnvfp4", "moe_scatter_combine", "moeq_last_error",
              "moe_route_prep_workspace_bytes", "moeq_abi_version", "moe_quantize_int4"):
        assert f in fns
    assert set(mq.EXPORTS) == fns


def test_library_exports_every_declared_symbol(L):
    raw = C.CDLL(mq.LIB_PATH)
    for f in declared_functions():
        assert hasattr(raw, f), f
    assert L.moeq_abi_version() == 3


def test_workspace_bytes(L):
    assert L.moe_route_prep_workspace_bytes(64, 2, 4) == 0          # one chunk: fused kernel
    assert L.moe_route_prep_workspace_bytes(4096, 8, 256) == 32 * 257 * 4
    assert L.moe_route_prep_workspace_bytes(-1, 2, 4) == 0
    # out-of-range sizes give 0, with T bounded before T*topk is formed
    assert L.moe_route_prep_workspace_bytes(2 ** 62, 4, 256) == 0
    assert L.moe_route_prep_workspace_bytes(2 ** 28, 8, 256) == 0
    assert L.moe_route_prep_workspace_bytes(4096, 65, 256) == 0
    assert L.moe_route_prep_workspace_bytes(4096, 8, 1025) == 0


def _route(L, T=4, topk=2, E=4, ids=A16, offs=A16, srt=A16, p2s=A16, ninv=A16, ws=None, wsb=0):
    return L.moe_route_prep(ids, T, topk, E, offs, srt, p2s, ninv, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), mq.EINVAL), (dict(topk=0), mq.EINVAL), (dict(topk=65), mq.EINVAL),
    (dict(E=0), mq.EINVAL), (dict(E=1025), mq.EINVAL), (dict(ids=None), mq.EINVAL),
    (dict(offs=None), mq.EINVAL), (dict(srt=ODD), mq.EALIGN),
    (dict(T=5000, topk=8, E=16), mq.EINVAL),            # needs a workspace
    (dict(T=2 ** 28, topk=8), mq.EINVAL),               # T*topk >= 2^31
    (dict(T=2 ** 62, topk=4), mq.EINVAL),               # T*topk would overflow int64
])
def test_route_prep_rejects(L, kw, status):
    assert _route(L, **kw) == status
    assert L.moeq_last_error()


def _int4(L, **kw):
    a = dict(a=A16, sa=A16, rows=16, arow=0, w=A16, sw=A16, off=A16, srt=A16, P=16, topk=2, E=4,
             N=256, K=256, act=0, od=mq.F16, out=A16, sched=0)
    a.update(kw)
    return L.grouped_gemm_qint4(a["a"], a["sa"], a["rows"], a["arow"], a["w"], a["sw"], a["off"],
                                a["srt"], a["P"], a["topk"], a["E"], a["N"], a["K"], a["act"],
                                a["od"], a["out"], a["sched"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=192), mq.EALIGN), (dict(N=80), mq.EALIGN), (dict(N=48, act=1), mq.EALIGN), (dict(E=0), mq.EINVAL),
    (dict(E=2000), mq.EINVAL), (dict(topk=0), mq.EINVAL), (dict(P=-1), mq.EINVAL),
    (dict(a=None), mq.EINVAL), (dict(w=ODD), mq.EALIGN), (dict(out=ODD), mq.EALIGN),
    (dict(sa=None), mq.EINVAL), (dict(act=7), mq.EUNSUPPORTED), (dict(od=9), mq.EUNSUPPORTED),
    (dict(od=mq.I32, act=1), mq.EUNSUPPORTED), (dict(arow=5), mq.EINVAL), (dict(act=2), mq.EUNSUPPORTED),
    (dict(srt=None, rows=8, P=16), mq.EINVAL), (dict(sched=9), mq.EINVAL),
    (dict(rows=0), mq.EINVAL), (dict(K=1 << 18), mq.EINVAL),
    # K = 2^17 with every code -8 would sum 2^17 products of 2^14 to 2^31 in
    # the int32 accumulator; the largest accepted K is 2^17 - 128
    (dict(K=1 << 17), mq.EINVAL),
    # the streaming schedule reads whole 256-value K groups
    (dict(K=384, sched=1), mq.EALIGN),
])
def test_int4_rejects(L, kw, status):
    assert _int4(L, **kw) == status


def _fp8(L, **kw):
    a = dict(a=A16, sa=A16, rows=16, arow=0, w=A16, sw=A16, off=A16, srt=A16, P=16, topk=1, E=1,
             N=256, K=256, od=mq.BF16, out=A16, sched=0)
    a.update(kw)
    return L.grouped_gemm_qfp8_block(a["a"], a["sa"], a["rows"], a["arow"], a["w"], a["sw"],
                                     a["off"], a["srt"], a["P"], a["topk"], a["E"], a["N"], a["K"],
                                     a["od"], a["out"], a["sched"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=64), mq.EALIGN), (dict(N=64), mq.EALIGN), (dict(od=mq.I32), mq.EUNSUPPORTED),
    (dict(sw=None), mq.EINVAL), (dict(sa=ODD), mq.EALIGN), (dict(off=None), mq.EINVAL),
])
def test_fp8_rejects(L, kw, status):
    assert _fp8(L, **kw) == status


def _nvfp4(L, **kw):
    a = dict(x=A16, xd=mq.BF16, rows=16, arow=0, w=A16, wl=0, sf=A16, sfl=0, gs=A16, off=A16, srt=A16, P=16,
             topk=2, E=4, N=256, K=256, act=0, lim=0.0, pw=None, od=mq.BF16, out=A16, wq=None, sched=0)
    a.update(kw)
    return L.grouped_gemm_qnvfp4(a["x"], a["xd"], a["rows"], a["arow"], a["w"], a["wl"], a["sf"], a["sfl"],
                                 a["gs"], a["off"],
                                 a["srt"], a["P"], a["topk"], a["E"], a["N"], a["K"], a["act"],
                                 a["lim"], a["pw"], a["od"], a["out"], a["wq"], a["sched"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=96), mq.EALIGN), (dict(N=48), mq.EALIGN), (dict(N=16, act=1), mq.EALIGN), (dict(sf=ODD), mq.EALIGN),
    (dict(gs=None), mq.EINVAL), (dict(od=mq.I32), mq.EUNSUPPORTED), (dict(act=3), mq.EUNSUPPORTED),
    (dict(x=None), mq.EINVAL), (dict(act=2, lim=0.0, K=96), mq.EALIGN),
    (dict(act=2, lim=0.0), mq.EINVAL), (dict(act=2, lim=-1.0), mq.EINVAL),
    (dict(act=2, lim=float("nan")), mq.EINVAL),
    (dict(pw=A16, act=1), mq.EUNSUPPORTED), (dict(pw=A16, srt=None), mq.EINVAL),
    (dict(pw=ODD), mq.EALIGN), (dict(xd=mq.F32), mq.EUNSUPPORTED), (dict(xd=mq.I32), mq.EUNSUPPORTED),
    (dict(sfl=2), mq.EINVAL), (dict(sfl=-1), mq.EINVAL), (dict(wl=2), mq.EINVAL),
    (dict(wq=ODD), mq.EALIGN),
])
def test_nvfp4_rejects(L, kw, status):
    assert _nvfp4(L, **kw) == status


def _combine(L, **kw):
    a = dict(y=A16, yd=mq.BF16, p2s=A16, tw=A16, T=8, topk=2, N=256, od=mq.BF16, out=A16)
    a.update(kw)
    return L.moe_scatter_combine(a["y"], a["yd"], a["p2s"], a["tw"], a["T"], a["topk"], a["N"],
                                 a["od"], a["out"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(N=12), mq.EALIGN), (dict(T=-2), mq.EINVAL), (dict(topk=0), mq.EINVAL),
    (dict(yd=mq.I32), mq.EUNSUPPORTED), (dict(od=7), mq.EUNSUPPORTED), (dict(y=None), mq.EINVAL),
    (dict(out=ODD), mq.EALIGN), (dict(T=2 ** 28, topk=8), mq.EINVAL), (dict(T=2 ** 62, topk=4), mq.EINVAL),
])
def test_combine_rejects(L, kw, status):
    assert _combine(L, **kw) == status


def _quant(L, **kw):
    a = dict(x=A16, xd=mq.F16, rows=8, K=256, q=A16, sc=A16)
    a.update(kw)
    return L.moe_quantize_int4(a["x"], a["xd"], a["rows"], a["K"], a["q"], a["sc"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=40), mq.EALIGN), (dict(K=0), mq.EINVAL), (dict(rows=-1), mq.EINVAL),
    (dict(xd=mq.I32), mq.EUNSUPPORTED), (dict(x=None), mq.EINVAL), (dict(q=ODD), mq.EALIGN),
    (dict(sc=ODD), mq.EALIGN),
])
def test_quantize_rejects(L, kw, status):
    assert _quant(L, **kw) == status


def test_error_text_names_the_call(L):
    assert _int4(L, K=192) == mq.EALIGN
    assert b"grouped_gemm_qint4" in L.moeq_last_error() and b"K=192" in L.moeq_last_error()


def test_binding_raises_without_gpu_tensors():
    import torch
    with pytest.raises(ValueError, match="on the GPU"):
        mq.moe_route_prep(torch.zeros(4, 2, dtype=torch.int32), 4)


def test_n_alignment_of_each_gemm(L):
    # INT4 and NVFP4 take N % 32 == 0 (the W4A4 launcher's check); FP8 keeps
    # N % 128 == 0 for its 128 x 128 weight-scale blocks.  Accepted shapes are
    # not called here (that would launch); the next multiple of 16 is refused.
    assert _int4(L, N=112) == mq.EALIGN and b"multiple of 32" in L.moeq_last_error()
    assert _nvfp4(L, N=112) == mq.EALIGN and b"multiple of 32" in L.moeq_last_error()
    assert _fp8(L, N=160) == mq.EALIGN and b"multiple of 128" in L.moeq_last_error()


def test_binding_checks_combine_out_shape():
    # a too-small caller-supplied out would let the kernel write [T][N] past
    # its end; the binding refuses it before anything is launched
    import torch
    y = torch.zeros(8, 64, dtype=torch.float16)
    p2s = torch.zeros(8, dtype=torch.int32)
    tw = torch.zeros(4, 2, dtype=torch.float32)
    with pytest.raises(ValueError, match=r"out must be \[4\]\[64\]"):
        mq.moe_scatter_combine(y, p2s, tw, out=torch.zeros(3, 64, dtype=torch.float16))
    with pytest.raises(ValueError, match=r"out must be \[4\]\[64\]"):
        mq.moe_scatter_combine(y, p2s, tw, out=torch.zeros(4, 32, dtype=torch.float16))
    with pytest.raises(ValueError, match="on the GPU"):       # right shape: reaches the device check
        mq.moe_scatter_combine(y, p2s, tw, out=torch.zeros(4, 64, dtype=torch.float16))


def test_binding_checks_sum_pairs_out_shape():
    import torch
    y = torch.zeros(8, 64, dtype=torch.bfloat16)
    p2s = torch.zeros(8, dtype=torch.int32)
    with pytest.raises(ValueError, match=r"out must be \[4\]\[64\]"):
        mq.moe_sum_pairs(y, p2s, 4, 2, out=torch.zeros(2, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="on the GPU"):
        mq.moe_sum_pairs(y, p2s, 4, 2, out=torch.zeros(4, 64, dtype=torch.bfloat16))


def test_binding_checks_pair_weights_rows():
    # with pair_weights, FC2 writes rows at pair ids up to the pair count - 1:
    # an explicit P below that count is refused
    import torch
    E, N, K, pairs = 2, 32, 128, 8
    x = torch.zeros(pairs, K, dtype=torch.float16)
    w = torch.zeros(E, N, K // 2, dtype=torch.uint8)
    sf = torch.zeros(E, N, K // 16, dtype=torch.uint8)
    g = torch.ones(E, dtype=torch.float32)
    offs = torch.zeros(E + 1, dtype=torch.int32)
    srt = torch.zeros(pairs, dtype=torch.int32)
    pw = torch.ones(pairs, dtype=torch.float32)
    with pytest.raises(ValueError, match="P must be at least"):
        mq.grouped_gemm_qnvfp4(x, w, sf, g, offs, srt, 2, a_row="sorted", pair_weights=pw, P=pairs - 1)
    with pytest.raises(ValueError, match="on the GPU"):
        mq.grouped_gemm_qnvfp4(x, w, sf, g, offs, srt, 2, a_row="sorted", pair_weights=pw, P=pairs)


def _repack(L, **kw):
    a = dict(w=A16, sf=0x20000, E=2, N=256, K=128, swap=1, wlay=0, lay=0, wo=0x40000, so=0x80000)
    a.update(kw)
    return L.moe_nvfp4_repack(a["w"], a["sf"], a["E"], a["N"], a["K"], a["swap"], a["wlay"], a["lay"], a["wo"],
                              a["so"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(N=192), mq.EALIGN), (dict(K=96), mq.EALIGN), (dict(E=0), mq.EINVAL),
    (dict(E=1025), mq.EINVAL), (dict(swap=2), mq.EINVAL), (dict(w=None), mq.EINVAL),
    (dict(so=None), mq.EINVAL), (dict(sf=0x20008), mq.EALIGN), (dict(wo=ODD), mq.EALIGN),
    (dict(wo=A16), mq.EINVAL),                          # in place
    (dict(wo=0x10000 + 0x3000), mq.EINVAL),             # overlaps the tail of w_in
    (dict(so=0x40000 + 0x7000), mq.EINVAL),             # overlaps w_out
    (dict(so=0x20000), mq.EINVAL),                      # scales in place
    (dict(N=1 << 20, K=1 << 17), mq.EINVAL),            # N*K too large
    (dict(lay=3), mq.EINVAL), (dict(wlay=5), mq.EINVAL),
])
def test_repack_rejects(L, kw, status):
    assert _repack(L, **kw) == status
    assert b"moe_nvfp4_repack" in L.moeq_last_error()


def _sum_pairs(L, **kw):
    a = dict(y=A16, yd=mq.BF16, p2s=A16, T=8, topk=2, N=256, od=mq.BF16, out=A16)
    a.update(kw)
    return L.moe_sum_pairs(a["y"], a["yd"], a["p2s"], a["T"], a["topk"], a["N"], a["od"], a["out"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(N=12), mq.EALIGN), (dict(T=-2), mq.EINVAL), (dict(topk=0), mq.EINVAL),
    (dict(yd=mq.I32), mq.EUNSUPPORTED), (dict(od=7), mq.EUNSUPPORTED), (dict(y=None), mq.EINVAL),
    (dict(p2s=None), mq.EINVAL), (dict(out=ODD), mq.EALIGN), (dict(T=2 ** 62, topk=4), mq.EINVAL),
])
def test_sum_pairs_rejects(L, kw, status):
    assert _sum_pairs(L, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(n=12), mq.EALIGN), (dict(n=-8), mq.EINVAL), (dict(x=None), mq.EINVAL), (dict(y=ODD), mq.EALIGN),
    (dict(y=A16 + 16), mq.EINVAL),                       # partial overlap
])
def test_cast_rejects(L, kw, status):
    a = dict(x=A16, n=64, y=0x20000)
    a.update(kw)
    assert L.moe_cast_bf16_to_f16(a["x"], a["n"], a["y"], None) == status


def test_noalloc_route_rejects_before_any_device_call(L):
    # argument checks and the fixed-array limit come before the device
    # address lookup, so they run without a GPU
    f = L.moe_route_prep_noalloc
    assert f(A16, -1, 2, 4, A16, A16, A16, A16, None) == mq.EINVAL
    assert f(A16, 4, 0, 4, A16, A16, A16, A16, None) == mq.EINVAL
    assert f(A16, 4, 2, 4, A16, ODD, A16, A16, None) == mq.EALIGN
    assert f(A16, 2 ** 62, 4, 4, A16, A16, A16, A16, None) == mq.EINVAL
    chunks = mq.ROUTE_NOALLOC_SCRATCH_BYTES // ((256 + 1) * 4)
    assert f(A16, chunks * 1024 + 1, 1, 256, A16, A16, A16, A16, None) == mq.EINVAL
    assert b"fixed" in L.moeq_last_error()
