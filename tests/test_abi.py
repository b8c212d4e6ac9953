"""CPU tests of the C ABI: the library loads and exports every declared entry point,
the planner's work list covers each request's visible tokens exactly once, and
malformed or unsupported inputs return the documented status without launching."""
import ctypes
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from paged_split_kv_stage1_amd import _lib
from paged_split_kv_stage1_amd._lib import (PA_ERR_INSUFFICIENT_WORKSPACE, PA_ERR_INVALID_ARGUMENT,
                                            PA_ERR_UNSUPPORTED, PaError, pa_plan_splits)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "pa.h")).read()
    declared = set(re.findall(r"^(?:pa_status|const char\*)\s+(pa_\w+)\(", header, flags=re.M))
    assert {"pa_plan_splits", "pa_decode_stage1", "pa_decode_merge", "pa_kv_quantize_fp8", "pa_kv_append",
            "pa_kv_quantize_fp8_per_head", "pa_kv_quantize_int8", "pa_debug_gather", "pa_last_error"} <= declared
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def _plan(B=2, rows=(1, 4), kv=(100, 3000), window=None, R=8, P=16, Hq=16, Hkv=2, d=256, q="bf16", kvd="bf16",
          mode="none", cus=256, max_splits=0, force=0, orientation="kv_on_m"):
    rows = np.asarray(rows)
    kv = np.asarray(kv)
    qo = np.concatenate([[0], np.cumsum(rows)])
    kvi = np.concatenate([[0], np.cumsum((kv + P - 1) // P)])
    return pa_plan_splits(qo, kvi, kv, window, R, P, Hq, Hkv, d, q, kvd, mode, num_cus=cus, max_splits=max_splits,
                          force_splits=force, orientation=orientation)


def _items(info, plan):
    n = info.num_items
    return plan[: n * 64].view(np.int32).reshape(n, 16), plan[n * 64:].view(np.int32)


def _check_cover(info, plan, rows, kv, window, Hkv, G=8, d=128):
    # every (request, KV head, query-block group) has splits 0..S-1 covering the visible
    # range once; the groups (runs of four 16-row blocks) cover the request's rows x heads
    it, row_ns = _items(info, plan)
    qo = np.concatenate([[0], np.cumsum(rows)])
    for b in range(len(kv)):
        n, L = rows[b], kv[b]
        W = 0 if window is None else window[b]
        lo = max(0, L - n - W + 1) if W > 0 else 0
        sel_b = it[it[:, 10] == b]
        assert np.all(sel_b[:, 7] == sel_b[0, 7])                  # same nsplit for the request
        assert np.all(row_ns[qo[b]:qo[b + 1]] == sel_b[0, 7])
        nb16 = -(-n * G // 16)
        per = 4 if (d == 512 and nb16 > 4) else max(nb16, 1)       # blocks one item covers
        assert sorted(set(sel_b[:, 11].tolist())) == list(range(0, nb16, per))
        for g in range(Hkv):
            for q0 in range(0, nb16, per):
                sel = sel_b[(sel_b[:, 5] == g) & (sel_b[:, 11] == q0)]
                sel = sel[np.argsort(sel[:, 6])]
                assert sel[:, 6].tolist() == list(range(len(sel)))
                assert sel[0, 8] <= lo and sel[0, 8] % 64 == 0
                assert np.all(sel[:-1, 9] == sel[1:, 8])             # contiguous, no overlap
                assert sel[-1, 9] == L
                assert np.all(sel[:, 9] >= sel[:, 8])
                assert np.all(sel[:, 0] == qo[b]) and np.all(sel[:, 1] == n) and np.all(sel[:, 2] == L)


def test_plan_covers_visible_tokens_exactly_once():
    rows, kv, win = [1, 4, 8, 2], [100, 3000, 8, 70000], [0, 64, 0, 5]
    info, plan = _plan(B=4, rows=rows, kv=kv, window=win)
    _check_cover(info, plan, np.array(rows), np.array(kv), win, 2)
    assert info.total_rows == sum(rows)
    assert info.plan_bytes == info.num_items * 64 + sum(rows) * 4
    assert info.partial_o_bytes == (sum(rows) * 16 * info.max_splits * 256 * 4 if info.max_splits > 1 else 0)
    info2, plan2 = _plan(B=4, rows=rows, kv=kv, window=[0, 0, 0, 0])
    assert info2.max_splits > 1 and info2.needs_merge
    assert info2.partial_o_bytes == sum(rows) * 16 * info2.max_splits * 256 * 4
    _check_cover(info2, plan2, np.array(rows), np.array(kv), None, 2)


@settings(max_examples=60, deadline=None)
@given(st.data())
def test_plan_properties(data):
    B = data.draw(st.integers(1, 12))
    rows = np.array(data.draw(st.lists(st.integers(1, 8), min_size=B, max_size=B)))
    kv = np.array([r + data.draw(st.integers(0, 40000)) for r in rows])
    win = data.draw(st.one_of(st.none(), st.lists(st.sampled_from([0, 1, 7, 64, 1000]), min_size=B, max_size=B)))
    cus = data.draw(st.sampled_from([1, 8, 256, 304]))
    cap = data.draw(st.sampled_from([0, 1, 3, 64]))
    Hkv = data.draw(st.sampled_from([1, 2, 8]))
    G = data.draw(st.sampled_from([1, 8, 24]))
    d = data.draw(st.sampled_from([128, 512])) if G * 8 <= 192 else 128
    info, plan = _plan(B=B, rows=rows, kv=kv, window=win, cus=cus, max_splits=cap, Hq=Hkv * G, Hkv=Hkv, d=d)
    _check_cover(info, plan, rows, kv, win, Hkv, G, d)
    if cap:
        assert info.max_splits <= cap
    it, _ = _items(info, plan)
    slots = cus if d == 512 else 2 * cus
    if info.num_items <= slots and slots % 16 == 0:
        return          # one round: splits cut by XCD streaming rate (test_one_round_splits_follow_xcd_rate)
    # heaviest first: within a request (same rows, same split status) longer items come first
    for b in range(B):
        for grp in np.unique(it[it[:, 10] == b, 11]):
            sel = (it[:, 10] == b) & (it[:, 11] == grp)
            tok = (it[sel, 9] - it[sel, 8]).astype(np.int64)
            assert np.all(tok[:-1] >= tok[1:])


def test_force_splits_gives_exact_count():
    info, plan = _plan(rows=[1, 1], kv=[512, 70], force=4)
    it, row_ns = _items(info, plan)
    assert info.num_items == 2 * 2 * 4 and info.max_splits == 4
    assert row_ns.tolist() == [4, 4]


def test_single_split_plan_needs_no_merge():
    info, _ = _plan(rows=[1], kv=[64], B=1)
    assert info.max_splits == 1 and not info.needs_merge and info.partial_o_bytes == 0


@pytest.mark.parametrize("kw,status", [
    (dict(R=9, rows=[9, 1]), PA_ERR_UNSUPPORTED),
    (dict(d=64), PA_ERR_UNSUPPORTED),
    (dict(d=192), PA_ERR_UNSUPPORTED),
    (dict(Hq=15), PA_ERR_INVALID_ARGUMENT),
    (dict(rows=[5, 1], kv=[4, 100]), PA_ERR_INVALID_ARGUMENT),
    (dict(rows=[0, 1]), PA_ERR_INVALID_ARGUMENT),
    (dict(R=2, rows=[3, 1]), PA_ERR_INVALID_ARGUMENT),
    (dict(window=[-1, 0]), PA_ERR_INVALID_ARGUMENT),
    (dict(q="fp8"), PA_ERR_UNSUPPORTED),
    (dict(mode="per_tensor"), PA_ERR_INVALID_ARGUMENT),
    (dict(kvd="fp8"), PA_ERR_INVALID_ARGUMENT),
    (dict(P=24), PA_ERR_UNSUPPORTED),
    (dict(P=8), PA_ERR_UNSUPPORTED),
    (dict(force=5, max_splits=4), PA_ERR_INVALID_ARGUMENT),
])
def test_plan_errors(kw, status):
    with pytest.raises(PaError) as e:
        _plan(**kw)
    assert e.value.status == status


def test_plan_rejects_inconsistent_page_counts():
    with pytest.raises(PaError) as e:
        pa_plan_splits([0, 1], [0, 3], [100], None, 1, 16, 8, 1, 128, "bf16", "bf16", "none", num_cus=8)
    assert e.value.status == PA_ERR_INVALID_ARGUMENT
    with pytest.raises(PaError) as e:
        pa_plan_splits([1, 2], [0, 7], [100], None, 1, 16, 8, 1, 128, "bf16", "bf16", "none", num_cus=8)
    assert e.value.status == PA_ERR_INVALID_ARGUMENT


def test_plan_buffer_too_small():
    L = _lib.lib()
    qo = (ctypes.c_int32 * 2)(0, 1)
    kvi = (ctypes.c_int32 * 2)(0, 4)
    kvl = (ctypes.c_int32 * 1)(64)
    a = _lib.PlanArgs(1, qo, kvi, kvl, None, 1, 16, 8, 1, 128, 0, 0, 0, 8, 0, 0)
    info = _lib.PlanInfo()
    buf = (ctypes.c_uint8 * 8)()
    st_ = L.pa_plan_splits(ctypes.byref(a), ctypes.addressof(buf), 8, ctypes.byref(info))
    assert st_ == PA_ERR_INSUFFICIENT_WORKSPACE and info.plan_bytes > 8
    assert b"plan buffer" in L.pa_last_error()


def test_stage1_validates_before_launch():
    info, _ = _plan(rows=[1, 1], kv=[512, 70])
    lay = (16 * 256 * 2, 16 * 256, 256)
    fake = 1 << 20        # never dereferenced: validation fails first
    with pytest.raises(PaError) as e:          # misaligned cache pointer
        _lib.pa_decode_stage1(info, fake, fake, None, fake + 8, fake, lay, None, None, None, fake, 0.1, fake, fake,
                              fake, "bf16")
    assert e.value.status == PA_ERR_INVALID_ARGUMENT
    with pytest.raises(PaError) as e:          # stride not a multiple of 16 bytes
        _lib.pa_decode_stage1(info, fake, fake, None, fake, fake, (1000, 8, 4), None, None, None, fake, 0.1, fake,
                              fake, fake, "bf16")
    assert e.value.status == PA_ERR_INVALID_ARGUMENT
    with pytest.raises(PaError) as e:          # missing output
        _lib.pa_decode_stage1(info, fake, fake, None, fake, fake, lay, None, None, None, fake, 0.1, fake, fake, None,
                              "bf16")
    assert e.value.status == PA_ERR_INVALID_ARGUMENT
    with pytest.raises(PaError) as e:          # bad output dtype
        _lib.pa_decode_stage1(info, fake, fake, None, fake, fake, lay, None, None, None, fake, 0.1, fake, fake, fake,
                              "fp8")
    assert e.value.status == PA_ERR_INVALID_ARGUMENT


def test_fp8_kv_needs_scales():
    info, _ = _plan(rows=[1, 1], kv=[512, 70], kvd="fp8", mode="per_token_head")
    fake = 1 << 20
    with pytest.raises(PaError) as e:
        _lib.pa_decode_stage1(info, fake, fake, None, fake, fake, (4096, 256, 256), None, None, (32, 16, 1), fake,
                              0.1, fake, fake, fake, "bf16")
    assert e.value.status == PA_ERR_INVALID_ARGUMENT


def test_quantize_validates():
    fake = 1 << 20
    with pytest.raises(PaError) as e:
        _lib.pa_kv_quantize_fp8(fake, "bf16", 10, 96, "per_token_head", fake, fake)
    assert e.value.status == PA_ERR_UNSUPPORTED
    with pytest.raises(PaError) as e:
        _lib.pa_kv_quantize_fp8(fake, "bf16", 10, 128, "none", fake, fake)
    assert e.value.status == PA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("case,status", [
    (dict(kv_dtype="bf16", mode="per_tensor"), PA_ERR_INVALID_ARGUMENT),       # dtype/mode combination
    (dict(kv_dtype="fp8", mode="none"), PA_ERR_INVALID_ARGUMENT),
    (dict(head_dim=96), PA_ERR_UNSUPPORTED),
    (dict(page_size=48), PA_ERR_UNSUPPORTED),
    (dict(k_scale=None), PA_ERR_INVALID_ARGUMENT),                             # FP8 without scales
    (dict(scale_layout=None), PA_ERR_INVALID_ARGUMENT),                        # per-token-head without layout
    (dict(k_new=(1 << 20) + 8), PA_ERR_INVALID_ARGUMENT),                      # misaligned source
    (dict(kv_layout=(4096, 256, 24)), PA_ERR_INVALID_ARGUMENT),                # slot stride not 16 B
    (dict(n_tokens=1 << 29, num_kv_heads=2), PA_ERR_UNSUPPORTED),              # row index past 32 bits
])
def test_append_validates(case, status):
    fake = 1 << 20
    args = dict(k_new=fake, v_new=fake, src_dtype="bf16", n_tokens=4, num_kv_heads=2, head_dim=128, page_size=16,
                slot_mapping=fake, k_cache=fake, v_cache=fake, kv_dtype="fp8", mode="per_token_head",
                kv_layout=(4096, 2048, 128), k_scale=fake, v_scale=fake, scale_layout=(32, 16, 1))
    args.update(case)
    with pytest.raises(PaError) as e:
        _lib.pa_kv_append(**args)
    assert e.value.status == status


@pytest.mark.parametrize("args,status", [
    (dict(num_heads=0), PA_ERR_UNSUPPORTED),
    (dict(num_heads=1025), PA_ERR_UNSUPPORTED),
    (dict(head_dim=96), PA_ERR_UNSUPPORTED),
    (dict(src=(1 << 20) + 8), PA_ERR_INVALID_ARGUMENT),
    (dict(dst=(1 << 20) + 4), PA_ERR_INVALID_ARGUMENT),
    (dict(scale=None), PA_ERR_INVALID_ARGUMENT),
    (dict(n_tokens=-1), PA_ERR_INVALID_ARGUMENT),
    (dict(src_dtype="fp8"), PA_ERR_INVALID_ARGUMENT),
])
def test_quantize_per_head_validates(args, status):
    fake = 1 << 20
    kw = dict(src=fake, src_dtype="bf16", n_tokens=10, num_heads=8, head_dim=128, dst=fake, scale=fake)
    kw.update(args)
    with pytest.raises(PaError) as e:
        _lib.pa_kv_quantize_fp8_per_head(**kw)
    assert e.value.status == status


def test_per_head_mode_needs_fp8_kv_and_plans_like_per_tensor():
    with pytest.raises(PaError) as e:
        _plan(kvd="bf16", mode="per_head")
    assert e.value.status == PA_ERR_INVALID_ARGUMENT
    a, _ = _plan(kvd="fp8", mode="per_head")
    b, _ = _plan(kvd="fp8", mode="per_tensor")
    assert (a.num_items, a.max_splits, a.variant) == (b.num_items, b.max_splits, b.variant)


def test_int8_kv_modes_and_queries():
    # INT8 KV: bf16 queries, per-tensor or per-token-head scales; it plans on the
    # per-token kernel path
    a, _ = _plan(kvd="int8", mode="per_token_head")
    b, _ = _plan(kvd="int8", mode="per_tensor")
    assert a.variant == b.variant and (a.variant >> 12) & 1 and (a.variant >> 3) & 1
    for kw in (dict(kvd="int8", mode="per_head"), dict(kvd="int8", mode="none"), dict(kvd="int8", q="fp8",
                                                                                      mode="per_tensor")):
        with pytest.raises(PaError) as e:
            _plan(**kw)
        assert e.value.status in (PA_ERR_INVALID_ARGUMENT, PA_ERR_UNSUPPORTED)
    fake = 1 << 20
    with pytest.raises(PaError) as e:
        _lib.pa_kv_quantize_int8(fake, "bf16", 10, 128, "per_head", fake, fake)
    assert e.value.status == PA_ERR_INVALID_ARGUMENT
    with pytest.raises(PaError) as e:
        _lib.pa_kv_quantize_int8(fake, "bf16", 10, 96, "per_tensor", fake, fake)
    assert e.value.status == PA_ERR_UNSUPPORTED
    with pytest.raises(PaError) as e:
        _lib.pa_kv_append(fake, fake, "bf16", 4, 2, 128, 16, fake, fake, fake, "int8", "per_head",
                          (4096, 2048, 128), fake, fake)
    assert e.value.status == PA_ERR_INVALID_ARGUMENT


def test_merge_without_splits_is_a_noop():
    info, _ = _plan(rows=[1], kv=[64], B=1)
    fake = 1 << 20
    _lib.pa_decode_merge(info, fake, None, None, fake, "bf16")      # launches nothing, returns OK


def test_head_dim_512_plans_and_round_trips_its_variant():
    # head_dim 512 (bf16 KV or per-token-head FP8 KV) plans one item per CU slot and query
    # block group, each wave one 16-row block, and its tile variant names head_dim 512; a
    # per-tensor FP8 cache, INT8 or FP8 queries are refused
    for kw in (dict(), dict(kvd="fp8", mode="per_token_head")):
        info, _ = _plan(B=1, rows=[8], kv=[131072], R=8, P=16, Hq=8, Hkv=1, d=512, **kw)
        assert info.head_dim == 512 and (info.variant >> 13) & 1 and info.num_items == 256
    info, plan = _plan(B=1, rows=[8], kv=[131072], R=8, P=16, Hq=16, Hkv=1, d=512)   # 128 rows x heads
    it, _ = _items(info, plan)
    assert sorted(set(it[:, 11].tolist())) == [0, 4] and info.num_items % 2 == 0
    for kw in (dict(kvd="fp8", mode="per_tensor"), dict(kvd="int8", mode="per_token_head"),
               dict(kvd="fp8", mode="per_token_head", q="fp8")):
        args = dict(B=1, rows=[8], kv=[131072], R=8, P=16, Hq=8, Hkv=1, d=512)
        args.update(kw)
        with pytest.raises(PaError) as e:
            _plan(**args)
        assert e.value.status == PA_ERR_UNSUPPORTED


def test_query_block_groups_cover_rows_x_heads():
    # head_dim 512 with more than four 16-row blocks per KV head (8 rows x group 24 = 12
    # blocks; group 128 = 64 blocks): one item per run of four blocks and split
    for Hq, Hkv, ngrp in ((48, 2, 3), (128, 1, 16)):
        rows, kv = np.array([8, 3, 1]), np.array([5000, 900, 64])
        info, plan = _plan(B=3, rows=rows, kv=kv, Hq=Hq, Hkv=Hkv, d=512)
        G = Hq // Hkv
        _check_cover(info, plan, rows, kv, None, Hkv, G, 512)
        assert ((info.variant >> 4) & 15, (info.variant >> 8) & 15) == (4, 1)
        it, _ = _items(info, plan)
        assert it[it[:, 10] == 0][:, 11].max() == 4 * (ngrp - 1)


def test_noalloc_rejects_plans_beyond_its_scratch():
    # 8 rows x 16 heads x 1024 splits x d 256 float32 partials = 128 MiB + LSE: above the
    # allocation-free entry point's scratch array, refused before any device call
    info, _ = _plan(B=1, rows=[8], kv=[131072], force=1024)
    assert info.partial_o_bytes + info.partial_lse_bytes > 128 << 20
    fake = 1 << 20
    with pytest.raises(PaError) as e:
        _lib.pa_decode_noalloc(info, fake, fake, None, fake, fake, (16 * 256 * 2, 16 * 256, 256), None, None, None,
                               fake, 0.1, fake, "bf16")
    assert e.value.status == PA_ERR_INSUFFICIENT_WORKSPACE
    assert "scratch" in str(e.value)


def test_gather_hooks_refuse_the_other_kernels_plans():
    # each test hook covers its own kernel family; the check comes before any device call
    fake = 1 << 20
    lay = (16 * 256, 256, 256)
    info, _ = _plan(rows=[1, 1], kv=[512, 70])
    with pytest.raises(PaError) as e:
        _lib.pa_debug_gather_rope(info, fake, fake, lay, None, lay, None, fake)
    assert e.value.status == PA_ERR_UNSUPPORTED
    qo, kvi, kv = [0, 1], [0, 5], [70]
    info, _ = pa_plan_splits(qo, kvi, kv, None, 1, 16, 32, 4, 192, "bf16", "bf16", "none", num_cus=8, head_dim_v=128)
    with pytest.raises(PaError) as e:
        _lib.pa_debug_gather(info, fake, fake, lay, None, fake)
    assert e.value.status == PA_ERR_UNSUPPORTED
    with pytest.raises(PaError) as e:          # 192/128 needs the V layout
        _lib.pa_debug_gather_rope(info, fake, fake, lay, None, None, None, fake)
    assert e.value.status == PA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw", [dict(), dict(kvd="fp8", mode="per_token_head"),
                                dict(d=128, Hq=48, kvd="fp8", mode="per_token_head"),
                                dict(d=128, Hq=32, R=4, rows=(3, 4))])
def test_query_rows_on_m_plans_the_same_work(kw):
    """The orientation changes only the kernel: the same work list, the variant with its bit."""
    a_info, a_plan = _plan(**kw)
    b_info, b_plan = _plan(orientation="q_on_m", **kw)
    assert b_info.variant == a_info.variant | (1 << 16)
    assert (a_info.num_items, a_info.max_splits, a_info.plan_bytes) == (b_info.num_items, b_info.max_splits,
                                                                        b_info.plan_bytes)
    assert np.array_equal(a_plan, b_plan)


@pytest.mark.parametrize("kw", [
    dict(q="fp8", kvd="fp8", mode="per_tensor"),             # e4m3 P.V
    dict(kvd="fp8", mode="per_tensor"),
    dict(kvd="int8", mode="per_token_head"),
    dict(R=4, rows=(1, 4)),                                  # bf16, d256, 32 rows x heads: two-wave tiles
    dict(d=128, Hq=48, R=8, rows=(8, 1)),                    # bf16, d128, 3 blocks per wave
    dict(d=512, Hq=8, Hkv=1),
])
def test_query_rows_on_m_refuses_what_it_is_not_built_for(kw):
    _plan(**kw)                                              # the default orientation plans it
    with pytest.raises(PaError) as e:
        _plan(orientation="q_on_m", **kw)
    assert e.value.status == PA_ERR_UNSUPPORTED


def test_orientation_value_is_checked():
    with pytest.raises(PaError) as e:
        _plan(orientation=2)
    assert e.value.status == PA_ERR_INVALID_ARGUMENT


def test_one_round_splits_follow_xcd_rate():
    """A one-round plan of memory-bound requests cuts each range so that items at odd
    positions (odd XCDs, measured ~10% slower at streaming) get ~0.9x the tokens of those at
    even positions; the splits still cover every visible token once."""
    B, R = 16, 1
    rows, kv = np.full(B, R), np.full(B, 32768)
    info, plan = _plan(B=B, rows=rows, kv=kv, R=R, Hq=16, Hkv=2, d=256)
    assert info.num_items == 512
    _check_cover(info, plan, rows, kv, None, 2)
    it, _ = _items(info, plan)
    tok = (it[:, 9] - it[:, 8]).astype(np.float64)
    ratio = tok[1::2].mean() / tok[0::2].mean()
    assert 0.85 <= ratio <= 0.95, ratio
    assert info.max_item_tokens == int(tok.max())
    # a compute-bound shape (per-token-head FP8, 8 rows) keeps equal splits
    info2, plan2 = _plan(B=B, rows=np.full(B, 8), kv=np.full(B, 131072), R=8, Hq=16, Hkv=2, d=256, kvd="fp8",
                         mode="per_token_head")
    it2, _ = _items(info2, plan2)
    assert len(set((it2[:, 9] - it2[:, 8]).tolist())) == 1
