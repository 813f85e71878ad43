"""The C-ABI library: it loads on a CPU-only host, exports every function that
include/kvc.h declares, and rejects bad arguments synchronously before any
HIP call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

import long_context_kv_kmeans_amd as kvc

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "kvc.h")

pytestmark = pytest.mark.skipif(not os.path.exists(kvc.LIB_PATH),
                                reason="libkvc.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kv_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(kvc.EXPORTED)


def test_every_declared_symbol_is_exported():
    L = kvc.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings():
    for code, name in [(0, "KV_OK"), (-1, "KV_ERR_INVALID_ARG"), (-2, "KV_ERR_UNSUPPORTED"),
                       (-3, "KV_ERR_WORKSPACE"), (-4, "KV_ERR_CAPACITY"), (-5, "KV_ERR_HIP")]:
        assert kvc.status_string(code) == name


def _fake_pool(**kw):
    # Non-null dummy addresses: validation only inspects them, never dereferences.
    a = 0x10000
    p = kvc.KVPool(kw.get("batch", 1), kw.get("n_kv_heads", 8), kw.get("head_dim", 128),
                   kw.get("dtype", kvc.KV_BF16), kw.get("row_cap", 4096), kw.get("unit_cap", 256),
                   a, a, a, a, a, a, a, a, a, kw.get("buf_cap", 0), a, a,
                   kw.get("seg_sum", None), a)
    return p


def test_boundary_validation():
    L = kvc.lib()
    f = ctypes.c_float(0.7)
    a = ctypes.c_void_p(0x10000)
    assert L.kv_boundary(None, None, 1, 4, 64, 0, f, a, None, None) == kvc.KV_ERR_INVALID_ARG
    assert L.kv_boundary(None, a, 0, 4, 64, 0, f, a, None, None) == kvc.KV_ERR_INVALID_ARG
    assert L.kv_boundary(None, a, 1, 4, 96, 0, f, a, None, None) == kvc.KV_ERR_UNSUPPORTED
    assert L.kv_boundary(None, a, 1, 4, 64, 7, f, a, None, None) == kvc.KV_ERR_UNSUPPORTED
    assert L.kv_boundary(None, a, 1, 4, 64, 0, ctypes.c_float(float("nan")), a, None,
                         None) == kvc.KV_ERR_INVALID_ARG


def test_boundary_select_validation():
    L = kvc.lib()
    a = ctypes.c_void_p(0x10000)
    f = ctypes.c_float(0.7)
    p = _fake_pool()
    need = L.kv_select_workspace(ctypes.byref(p), 32)
    assert need > 0
    # the same checks as kv_select, plus flag out and a finite tau
    assert L.kv_boundary_select(ctypes.byref(p), None, a, 32, f, 64, None, None, a, 256, a, a,
                                None, None, a, need, None) == kvc.KV_ERR_INVALID_ARG
    assert L.kv_boundary_select(ctypes.byref(p), None, a, 32, ctypes.c_float(float("nan")), 64,
                                a, None, a, 256, a, a, None, None, a, need,
                                None) == kvc.KV_ERR_INVALID_ARG
    assert L.kv_boundary_select(ctypes.byref(p), None, a, 24, f, 64, a, None, a, 256, a, a,
                                None, None, a, need, None) == kvc.KV_ERR_UNSUPPORTED  # G = 3
    assert L.kv_boundary_select(ctypes.byref(p), None, a, 32, f, 64, a, None, a, 256, a, a,
                                None, None, a, need - 1, None) == kvc.KV_ERR_WORKSPACE
    pb = _fake_pool(buf_cap=64, seg_sum=0x10000)
    assert L.kv_boundary_select(ctypes.byref(pb), None, a, 32, f, 64, a, None, a, 256, a, a,
                                None, None, a, need, None) == kvc.KV_ERR_UNSUPPORTED  # local buffer


def test_boundary_segment_append_validation():
    L = kvc.lib()
    a = ctypes.c_void_p(0x10000)
    f = ctypes.c_float(0.7)
    pb = _fake_pool(buf_cap=64, seg_sum=0x10000)
    assert L.kv_boundary_segment_append(ctypes.byref(pb), None, None, 32, f, a, a, a,
                                        None, None) == kvc.KV_ERR_INVALID_ARG  # q_cur
    assert L.kv_boundary_segment_append(ctypes.byref(pb), None, a, 32, f, a, a, None,
                                        None, None) == kvc.KV_ERR_INVALID_ARG  # flag out
    assert L.kv_boundary_segment_append(ctypes.byref(pb), None, a, 32,
                                        ctypes.c_float(float("nan")), a, a, a, None,
                                        None) == kvc.KV_ERR_INVALID_ARG
    p = _fake_pool()  # no local buffer
    assert L.kv_boundary_segment_append(ctypes.byref(p), None, a, 32, f, a, a, a, None,
                                        None) == kvc.KV_ERR_INVALID_ARG


def test_pool_validation():
    L = kvc.lib()
    a = ctypes.c_void_p(0x10000)
    ws = ctypes.c_void_p(0x10000)  # 256-aligned dummy
    p = _fake_pool(head_dim=96)
    assert L.kv_select(ctypes.byref(p), a, 32, 512, None, a, 512, a, a, None, None, ws, 1 << 30,
                       None) == kvc.KV_ERR_UNSUPPORTED
    p = _fake_pool(batch=0)
    assert L.kv_select(ctypes.byref(p), a, 32, 512, None, a, 512, a, a, None, None, ws, 1 << 30,
                       None) == kvc.KV_ERR_INVALID_ARG
    p = _fake_pool()
    # query heads not a multiple of KV heads
    assert L.kv_select(ctypes.byref(p), a, 30, 512, None, a, 512, a, a, None, None, ws, 1 << 30,
                       None) == kvc.KV_ERR_INVALID_ARG
    # negative budget
    assert L.kv_select(ctypes.byref(p), a, 32, -1, None, a, 512, a, a, None, None, ws, 1 << 30,
                       None) == kvc.KV_ERR_INVALID_ARG
    # selection capacity below min(budget, unit_cap)
    assert L.kv_select(ctypes.byref(p), a, 32, 512, None, a, 100, a, a, None, None, ws, 1 << 30,
                       None) == kvc.KV_ERR_CAPACITY
    # workspace too small / misaligned
    assert L.kv_select(ctypes.byref(p), a, 32, 128, None, a, 256, a, a, None, None, ws, 16,
                       None) == kvc.KV_ERR_WORKSPACE
    assert L.kv_select(ctypes.byref(p), a, 32, 128, None, a, 256, a, a, None, None,
                       ctypes.c_void_p(0x10004), 1 << 30, None) == kvc.KV_ERR_WORKSPACE
    # group size 3 unsupported
    p3 = _fake_pool(n_kv_heads=2)
    assert L.kv_select(ctypes.byref(p3), a, 6, 128, None, a, 256, a, a, None, None, ws, 1 << 30,
                       None) == kvc.KV_ERR_UNSUPPORTED
    # segments need a local buffer and seg_sum
    assert L.kv_segment_append(ctypes.byref(p), a, a, a, None) == kvc.KV_ERR_INVALID_ARG
    pb = _fake_pool(buf_cap=16)  # seg_sum NULL
    assert L.kv_segment_append(ctypes.byref(pb), a, a, a, None) == kvc.KV_ERR_INVALID_ARG
    assert L.kv_select(None, a, 32, 128, None, a, 256, a, a, None, None, ws, 1 << 30,
                       None) == kvc.KV_ERR_INVALID_ARG


def test_attend_validation():
    L = kvc.lib()
    a = ctypes.c_void_p(0x10000)
    p = _fake_pool()
    need = L.kv_gather_attend_workspace(ctypes.byref(p), 32, 512)
    assert need > 0
    c01 = ctypes.c_float(0.1)
    assert L.kv_gather_attend(ctypes.byref(p), a, 32, c01, a, None, 5000, a, 512, a, a, need,
                              None) == kvc.KV_ERR_UNSUPPORTED  # sel_cap > 4096
    assert L.kv_gather_attend(ctypes.byref(p), a, 32, c01, a, None, 512, a, 512, a, a, need - 1,
                              None) == kvc.KV_ERR_WORKSPACE
    assert L.kv_gather_attend(ctypes.byref(p), None, 32, c01, a, None, 512, a, 512, a, a, need,
                              None) == kvc.KV_ERR_INVALID_ARG
    # neither ids nor spans
    assert L.kv_gather_attend(ctypes.byref(p), a, 32, c01, None, None, 512, a, 512, a, a, need,
                              None) == kvc.KV_ERR_INVALID_ARG


def test_cluster_build_validation():
    L = kvc.lib()
    a = ctypes.c_void_p(0x10000)
    p = _fake_pool(row_cap=1000, unit_cap=64)
    ws_need = L.kv_cluster_build_workspace(1, 8, 1000, 128, 64, kvc.KV_BF16)
    assert ws_need > 0
    assert L.kv_cluster_build(ctypes.byref(p), a, a, 1000, 65, 10, a, None, None, None, None, a, ws_need,
                              None) == kvc.KV_ERR_CAPACITY  # clusters > unit_cap
    assert L.kv_cluster_build(ctypes.byref(p), a, a, 1001, 64, 10, a, None, None, None, None, a, ws_need,
                              None) == kvc.KV_ERR_CAPACITY  # keys > row_cap
    assert L.kv_cluster_build(ctypes.byref(p), a, a, 50, 64, 10, a, None, None, None, None, a, ws_need,
                              None) == kvc.KV_ERR_INVALID_ARG  # clusters > keys
    assert L.kv_cluster_build(ctypes.byref(p), a, a, 1000, 64, 0, a, None, None, None, None, a, ws_need,
                              None) == kvc.KV_ERR_INVALID_ARG  # no iterations, no labels
    assert L.kv_cluster_build(ctypes.byref(p), a, a, 1000, 64, 10, None, None, None, None, None, a, ws_need,
                              None) == kvc.KV_ERR_INVALID_ARG
    assert L.kv_cluster_build(ctypes.byref(p), a, a, 1000, 64, 10, a, None, None, None, None, a, ws_need - 1,
                              None) == kvc.KV_ERR_WORKSPACE
    assert L.kv_kmeans_assign(a, a, 8, 1000, 128, 40000, kvc.KV_BF16, a, a, 1 << 30,
                              None) == kvc.KV_ERR_UNSUPPORTED  # too many clusters
    need = L.kv_kmeans_assign_workspace(8, 64, 128, kvc.KV_BF16)
    assert L.kv_kmeans_prepare(a, 8, 128, 64, kvc.KV_BF16, a, need - 1,
                               None) == kvc.KV_ERR_WORKSPACE
    assert L.kv_kmeans_prepare(None, 8, 128, 64, kvc.KV_BF16, a, need,
                               None) == kvc.KV_ERR_INVALID_ARG
    assert L.kv_kmeans_prepare(a, 8, 96, 64, kvc.KV_BF16, a, need,
                               None) == kvc.KV_ERR_UNSUPPORTED  # head_dim
    assert L.kv_kmeans_assign_prepared(a, a, 8, 0, 128, 64, kvc.KV_BF16, a, a, need,
                                       None) == kvc.KV_ERR_INVALID_ARG  # no keys
    assert L.kv_kmeans_assign_prepared(a, a, 8, 1000, 128, 64, kvc.KV_BF16, a,
                                       ctypes.c_void_p(0x10010), need,
                                       None) == kvc.KV_ERR_WORKSPACE  # misaligned
    assert L.kv_kmeans_update(a, a, a, a, None, 8, 1000, 128, 64, kvc.KV_BF16, a, 10,
                              None) == kvc.KV_ERR_WORKSPACE


def test_fetch_selected_validation():
    L = kvc.lib()
    a = ctypes.c_void_p(0x10000)
    src = _fake_pool()
    dst = _fake_pool(row_cap=512, unit_cap=1)
    dst.k, dst.v = 0x20000, 0x30000
    S, D = ctypes.byref(src), ctypes.byref(dst)

    def call(src_=S, dst_=D, flag=a, su=a, sp=None, cap=64, sn=a, ds=a, dn=a):
        return L.kv_fetch_selected(src_, flag, su, sp, cap, sn, dst_, ds, dn, None)

    for kw in ({"src_": None}, {"dst_": None}, {"flag": None}, {"su": None}, {"sn": None},
               {"ds": None}, {"dn": None}, {"cap": 0}):
        assert call(**kw) == kvc.KV_ERR_INVALID_ARG, kw
    assert call(cap=4097) == kvc.KV_ERR_UNSUPPORTED
    for field, val in (("batch", 2), ("n_kv_heads", 4), ("head_dim", 64), ("dtype", kvc.KV_F32)):
        bad = _fake_pool(row_cap=512, unit_cap=1)
        bad.k, bad.v = 0x20000, 0x30000
        setattr(bad, field, val)
        assert call(dst_=ctypes.byref(bad)) == kvc.KV_ERR_INVALID_ARG, field
    same = _fake_pool(row_cap=512, unit_cap=1)  # k, v alias the source's
    assert call(dst_=ctypes.byref(same)) == kvc.KV_ERR_INVALID_ARG
    dseg = _fake_pool(row_cap=512, unit_cap=1, buf_cap=8, seg_sum=0x10000)
    dseg.k, dseg.v = 0x20000, 0x30000
    assert call(dst_=ctypes.byref(dseg)) == kvc.KV_ERR_UNSUPPORTED  # a working set has no buffer


def test_fetch_attend_validation():
    L = kvc.lib()
    a = ctypes.c_void_p(0x10000)
    src = _fake_pool()
    dst = _fake_pool(row_cap=512, unit_cap=1)
    dst.k, dst.v = 0x20000, 0x30000
    S, D = ctypes.byref(src), ctypes.byref(dst)
    need = L.kv_gather_attend_workspace(D, 32, 512)
    assert need > 0
    f = ctypes.c_float(0.1)

    def call(src_=S, dst_=D, q=a, hq=32, scale=f, flag=a, su=a, cap=64, sn=a, rows=512, ds=a,
             dn=a, out=a, ws=a, nbytes=need):
        return L.kv_fetch_attend(src_, q, hq, scale, flag, su, None, cap, sn, rows, dst_, ds, dn,
                                 out, ws, nbytes, None)

    for kw in ({"src_": None}, {"dst_": None}, {"q": None}, {"flag": None}, {"su": None},
               {"sn": None}, {"ds": None}, {"dn": None}, {"out": None}, {"cap": 0},
               {"hq": 12}, {"rows": -1}, {"scale": ctypes.c_float(float("nan"))}):
        assert call(**kw) == kvc.KV_ERR_INVALID_ARG, kw
    assert call(hq=24) == kvc.KV_ERR_UNSUPPORTED  # G = 3
    assert call(cap=4097) == kvc.KV_ERR_UNSUPPORTED
    assert call(nbytes=need - 1) == kvc.KV_ERR_WORKSPACE
    assert call(ws=ctypes.c_void_p(0x10010)) == kvc.KV_ERR_WORKSPACE  # misaligned
    same = _fake_pool(row_cap=512, unit_cap=1)
    assert call(dst_=ctypes.byref(same)) == kvc.KV_ERR_INVALID_ARG
    seg = _fake_pool(buf_cap=64, seg_sum=0x10000)  # local buffer without an HBM copy
    assert call(src_=ctypes.byref(seg)) == kvc.KV_ERR_UNSUPPORTED
    segf = _fake_pool(buf_cap=64, seg_sum=0x10000, dtype=kvc.KV_F32)  # fp32 with a copy
    segf.buf_k, segf.buf_v, segf.buf_ring = 0x40000, 0x50000, 64
    dstf = _fake_pool(row_cap=512, unit_cap=1, dtype=kvc.KV_F32)
    dstf.k, dstf.v = 0x20000, 0x30000
    assert call(src_=ctypes.byref(segf), dst_=ctypes.byref(dstf)) == kvc.KV_ERR_UNSUPPORTED


def test_local_buffer_copy_validation():
    # buf_k / buf_v: both or neither, only with a local buffer, ring >= buf_cap
    L = kvc.lib()
    ok = _fake_pool(buf_cap=64, seg_sum=0x10000)
    ok.buf_k, ok.buf_v, ok.buf_ring = 0x40000, 0x50000, 64
    assert L.kv_gather_attend_workspace(ctypes.byref(ok), 32, 512) > 0
    for field, val in (("buf_v", None), ("buf_ring", 63)):
        bad = _fake_pool(buf_cap=64, seg_sum=0x10000)
        bad.buf_k, bad.buf_v, bad.buf_ring = 0x40000, 0x50000, 64
        setattr(bad, field, val)
        assert L.kv_gather_attend_workspace(ctypes.byref(bad), 32, 512) == 0, field
    nobuf = _fake_pool()
    nobuf.buf_k, nobuf.buf_v, nobuf.buf_ring = 0x40000, 0x50000, 64
    assert L.kv_gather_attend_workspace(ctypes.byref(nobuf), 32, 512) == 0


def test_host_device_pointer_rejects_unpinned_memory():
    L = kvc.lib()
    out = ctypes.c_void_p()
    assert L.kv_host_device_pointer(None, ctypes.byref(out)) == kvc.KV_ERR_INVALID_ARG
    buf = ctypes.create_string_buffer(4096)
    assert L.kv_host_device_pointer(ctypes.cast(buf, ctypes.c_void_p), None) == \
        kvc.KV_ERR_INVALID_ARG
    # pageable memory (and, on a host without a GPU, any memory) has no device address
    assert L.kv_host_device_pointer(ctypes.cast(buf, ctypes.c_void_p),
                                    ctypes.byref(out)) == kvc.KV_ERR_INVALID_ARG


def test_workspace_sizes_scale():
    L = kvc.lib()
    small = L.kv_cluster_build_workspace(1, 8, 32768, 128, 2048, kvc.KV_BF16)
    big = L.kv_cluster_build_workspace(1, 8, 131072, 128, 8192, kvc.KV_BF16)
    assert 0 < small < big < 256 << 20
    assert L.kv_cluster_build_workspace(0, 8, 10, 128, 2, 1) == 0


def test_product_path_has_no_oracle_dependency():
    root = os.path.dirname(os.path.abspath(kvc.__file__))
    for dirpath, _, files in os.walk(root):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f


def test_ranges_beyond_the_kernels_limits_are_refused():
    """Clusters above 8192 (one counting-sort chunk's label counts must fit
    64 KB of LDS) and pools of more than 8192 units (8 selection keys per
    thread of a 1024-thread workgroup) are refused before any launch."""
    L = kvc.lib()
    a = ctypes.c_void_p(0x10000)
    big = 1 << 30
    assert L.kv_kmeans_assign(a, a, 8, 20000, 128, 8193, kvc.KV_BF16, a, a, big,
                              None) == kvc.KV_ERR_UNSUPPORTED
    assert L.kv_kmeans_prepare(a, 8, 128, 8193, kvc.KV_BF16, a, big, None) == kvc.KV_ERR_UNSUPPORTED
    assert L.kv_kmeans_assign_prepared(a, a, 8, 20000, 128, 8193, kvc.KV_BF16, a, a, big,
                                       None) == kvc.KV_ERR_UNSUPPORTED
    assert L.kv_kmeans_update(a, a, a, a, None, 8, 20000, 128, 8193, kvc.KV_BF16, a, big,
                              None) == kvc.KV_ERR_UNSUPPORTED
    p = _fake_pool(row_cap=20000, unit_cap=9000)
    assert L.kv_cluster_build(ctypes.byref(p), a, a, 20000, 8193, 10, a, None, None, None, None, a, big,
                              None) == kvc.KV_ERR_UNSUPPORTED
    # 8192 clusters and 8192 units are inside the limits (only the workspace is short here)
    p = _fake_pool(row_cap=20000, unit_cap=8192)
    assert L.kv_cluster_build(ctypes.byref(p), a, a, 20000, 8192, 10, a, None, None, None, None, a, 256,
                              None) == kvc.KV_ERR_WORKSPACE
    assert L.kv_select(ctypes.byref(p), a, 32, 512, None, a, 512, a, a, None, None, a, 16,
                       None) == kvc.KV_ERR_WORKSPACE
    p = _fake_pool(row_cap=20000, unit_cap=8193)
    assert L.kv_select(ctypes.byref(p), a, 32, 512, None, a, 512, a, a, None, None, a, big,
                       None) == kvc.KV_ERR_UNSUPPORTED
    assert L.kv_boundary_select(ctypes.byref(p), None, a, 32, ctypes.c_float(0.7), 512, a, None,
                                a, 512, a, a, None, None, a, big,
                                None) == kvc.KV_ERR_UNSUPPORTED


def _cpu_pool(dtype=None, B=1, H=2, D=64, row_cap=64, unit_cap=8):
    import torch
    return kvc.Pool(B, H, D, dtype or torch.bfloat16, row_cap=row_cap, unit_cap=unit_cap,
                    device="cpu")


def test_binding_rejects_wrong_element_types_and_shapes():
    """The binding checks every tensor's element type and extent against the
    pool (and against each other) before a pointer reaches the library: the C
    ABI has no way to tell a bf16 query from an fp32 one or a short buffer
    from a long one. CPU tensors are used, so a call that passes the checks
    stops at the 'must live on the GPU' error instead."""
    import torch
    B, H, Hq, D = 1, 2, 8, 64
    pool = _cpu_pool()
    bf, f32, i32, u8 = torch.bfloat16, torch.float32, torch.int32, torch.uint8

    def z(*shape, dt=i32):
        return torch.zeros(*shape, dtype=dt)

    q = z(B, Hq, D, dt=bf)
    sel, sel_n, sel_rows = z(B, H, 16), z(B, H), z(B, H)
    flag = z(B, dt=u8)
    out = z(B, Hq, D, dt=f32)

    def raises(match, fn, *a, **k):
        with pytest.raises(ValueError, match=match):
            fn(*a, **k)

    # a call that passes every check reaches the device-pointer check
    ws = z(256, dt=u8)
    raises("must live on the GPU", kvc.kv_select, pool, q, 16, flag, sel, sel_n, sel_rows, ws=ws)
    raises("q: element type", kvc.kv_select, pool, q.float(), 16, flag, sel, sel_n, sel_rows)
    raises("q: shape", kvc.kv_select, pool, z(B, Hq, 128, dt=bf), 16, flag, sel, sel_n, sel_rows)
    raises("flag: element type", kvc.kv_select, pool, q, 16, flag.int(), sel, sel_n, sel_rows)
    raises("sel_n: shape", kvc.kv_select, pool, q, 16, flag, sel, z(B, H + 1), sel_rows)
    raises("sel_spans: shape", kvc.kv_select, pool, q, 16, flag, sel, sel_n, sel_rows,
           sel_spans=z(B, H, 15, 2))
    raises("scores_out: shape", kvc.kv_select, pool, q, 16, flag, sel, sel_n, sel_rows,
           scores_out=z(B, H, 7, dt=f32))
    raises("q_prev: element type", kvc.kv_boundary_select, pool, q.float(), q, 0.7, 16, flag,
           sel, sel_n, sel_rows)
    # attention: output type and extent, span/id capacity agreement
    raises("must live on the GPU", kvc.kv_gather_attend, pool, q, 0.1, sel, sel_n, 16, out, ws=ws)
    raises("out: element type", kvc.kv_gather_attend, pool, q, 0.1, sel, sel_n, 16, out.bfloat16())
    raises("out: shape", kvc.kv_gather_attend, pool, q, 0.1, sel, sel_n, 16, z(B, Hq, 32, dt=f32))
    raises("sel_spans: shape", kvc.kv_gather_attend, pool, q, 0.1, sel, sel_n, 16, out,
           sel_spans=z(B, H, 8, 2))
    raises("required", kvc.kv_gather_attend, pool, q, 0.1, None, sel_n, 16, out)
    wset = _cpu_pool(row_cap=16, unit_cap=1)
    raises("dst_spans", kvc.kv_fetch_attend, pool, q, 0.1, flag, sel, sel_n, 16, wset,
           z(B, H, 2, 2), z(B, H), out)
    raises("dst_n: shape", kvc.kv_fetch_selected, pool, flag, sel, sel_n, wset, z(B, H, 1, 2),
           z(B))
    # prefill: keys/values against the pool, init and labels against the keys
    keys, vals = z(B, H, 32, D, dt=bf), z(B, H, 32, D, dt=bf)
    init = z(B, H, 4)
    raises("must live on the GPU", kvc.kv_cluster_build, pool, keys, vals, 4, 1, init, ws=ws)
    raises("keys: element type", kvc.kv_cluster_build, pool, keys.float(), vals, 4, 1, init)
    raises("keys: shape", kvc.kv_cluster_build, pool, z(B, H + 1, 32, D, dt=bf), vals, 4, 1, init)
    raises("values: shape", kvc.kv_cluster_build, pool, keys, z(B, H, 31, D, dt=bf), 4, 1, init)
    raises("init_idx: shape", kvc.kv_cluster_build, pool, keys, vals, 5, 1, init)
    raises("init_idx: element type", kvc.kv_cluster_build, pool, keys, vals, 4, 1, init.long())
    raises("assign_in: shape", kvc.kv_cluster_build, pool, keys, vals, 4, 1, init,
           assign_in=z(B, H, 31))
    raises("assign_out: element type", kvc.kv_cluster_build, pool, keys, vals, 4, 1, init,
           assign_out=z(B, H, 32, dt=torch.int64))
    # K-means steps: centroids fp32 [BH, C, D], labels int32 [BH, N]
    k3, c3, lab = z(2, 32, D, dt=bf), z(2, 4, D, dt=f32), z(2, 32)
    raises("centroids: element type", kvc.kv_kmeans_assign, k3, c3.bfloat16(), lab)
    raises("labels: shape", kvc.kv_kmeans_assign, k3, c3, z(2, 31))
    raises("centroids_out: shape", kvc.kv_kmeans_update, k3, lab, c3, z(2, 5, D, dt=f32))
    raises("counts: element type", kvc.kv_kmeans_update, k3, lab, c3, c3.clone(),
           counts=z(2, 4, dt=f32))
    # decode-step tensors of the segment append
    kt = z(B, H, D, dt=bf)
    raises("k_t: shape", kvc.kv_segment_append, pool, z(B, H, 32, dt=bf), kt, flag)
    raises("v_t: element type", kvc.kv_segment_append, pool, kt, kt.float(), flag)
    raises("r: element type", kvc.kv_boundary, q, q, 0.7, flag, r=z(B))


def test_noalloc_attention_validation():
    """kv_gather_attend_noalloc validates like kv_gather_attend and refuses a
    launch whose partials would not fit its 4 MiB static scratch, all before
    it touches the device."""
    L = kvc.lib()
    a = ctypes.c_void_p(0x10000)
    c01 = ctypes.c_float(0.1)
    p = _fake_pool()
    assert L.kv_gather_attend_noalloc(ctypes.byref(p), None, 32, c01, a, None, 512, a, 512, a,
                                      None) == kvc.KV_ERR_INVALID_ARG
    assert L.kv_gather_attend_noalloc(ctypes.byref(p), a, 32, c01, None, None, 512, a, 512, a,
                                      None) == kvc.KV_ERR_INVALID_ARG
    assert L.kv_gather_attend_noalloc(ctypes.byref(p), a, 24, c01, a, None, 512, a, 512, a,
                                      None) == kvc.KV_ERR_UNSUPPORTED  # G = 3
    assert L.kv_gather_attend_noalloc(ctypes.byref(p), a, 32, c01, a, None, 5000, a, 512, a,
                                      None) == kvc.KV_ERR_UNSUPPORTED  # sel_cap > 4096
    big = _fake_pool(batch=256)
    assert L.kv_gather_attend_workspace(ctypes.byref(big), 64, 4096) > 4 << 20
    assert L.kv_gather_attend_noalloc(ctypes.byref(big), a, 64, c01, a, None, 4096, a, 4096, a,
                                      None) == kvc.KV_ERR_WORKSPACE


def test_decode_step_validation():
    """kv_decode_step: bf16 pools without a local buffer, a distinct working set of the
    same shape, every output pointer, a big enough selection list and workspace."""
    L = kvc.lib()
    a = ctypes.c_void_p(0x10000)
    f07, c01 = ctypes.c_float(0.7), ctypes.c_float(0.1)
    src = _fake_pool()
    dst = _fake_pool(row_cap=512, unit_cap=1)
    dst.k, dst.v = 0x20000, 0x30000
    need = L.kv_decode_step_workspace(ctypes.byref(src), 32, 512)
    assert need > L.kv_gather_attend_workspace(ctypes.byref(src), 32, 512)

    def call(src_=None, dst_=None, hq=32, budget=512, su=a, sp=a, cap=512, out=a, ws_bytes=need,
             q=a, tau=f07):
        return L.kv_decode_step(ctypes.byref(src_ or src), None, q, hq, tau, c01, budget, a,
                                None, su, sp, cap, a, a, ctypes.byref(dst_ or dst), a, a, out, a,
                                ws_bytes, None)
    # everything valid except the (dummy) workspace size: KV_ERR_WORKSPACE comes last
    assert call(ws_bytes=need - 1) == kvc.KV_ERR_WORKSPACE
    assert call(q=None) == kvc.KV_ERR_INVALID_ARG
    assert call(su=None) == kvc.KV_ERR_INVALID_ARG
    assert call(sp=None) == kvc.KV_ERR_INVALID_ARG
    assert call(out=None) == kvc.KV_ERR_INVALID_ARG
    assert call(tau=ctypes.c_float(float("nan"))) == kvc.KV_ERR_INVALID_ARG
    assert call(hq=24) == kvc.KV_ERR_UNSUPPORTED  # G = 3
    assert call(cap=100) == kvc.KV_ERR_CAPACITY    # below min(budget, unit_cap)
    assert call(budget=5000, cap=4097) == kvc.KV_ERR_UNSUPPORTED
    assert call(src_=_fake_pool(dtype=kvc.KV_F32)) == kvc.KV_ERR_UNSUPPORTED
    assert call(src_=_fake_pool(buf_cap=64, seg_sum=0x10000)) == kvc.KV_ERR_UNSUPPORTED
    assert call(src_=_fake_pool(unit_cap=8193)) == kvc.KV_ERR_UNSUPPORTED
    same = _fake_pool(row_cap=512, unit_cap=1)  # k, v alias the source's
    assert call(dst_=same) == kvc.KV_ERR_INVALID_ARG
    other = _fake_pool(row_cap=512, unit_cap=1, n_kv_heads=4)
    other.k, other.v = 0x20000, 0x30000
    assert call(dst_=other) == kvc.KV_ERR_INVALID_ARG
