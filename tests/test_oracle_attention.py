"""Pins of the fp64 attention oracle: a 40-digit decimal brute force on tiny cases,
closed forms, and the invariants the method must satisfy (rows ignore positions
past their own, split count does not change the result, R=1 equals single-row
decode, GQA head mapping)."""
from decimal import Decimal, getcontext

import numpy as np
import pytest

from oracle.attention import (PagedKV, attend, decode_attention, decode_attention_one, gather_slots,
                              merge_partials, split_partials, visible_range)
from oracle.formats import bf16_bits_to_f64
from tests.oracle_cases import bf16_bits, tiny_problem


def _run(pb, q64=None):
    q64 = bf16_bits_to_f64(pb["q"]) if q64 is None else q64
    return decode_attention(q64, pb["k"], pb["v"], pb["page_indices"], pb["kv_indptr"], pb["kv_len"],
                            pb["qo_indptr"], pb["window"], pb["sm_scale"])


def _brute_force(pb):
    """Decimal (40 digits) evaluation with its own page walk: enumerate the
    request's pages in table order, then the slots inside each page."""
    getcontext().prec = 40
    q = bf16_bits_to_f64(pb["q"])
    P, Hq, Hkv = pb["P"], pb["Hq"], pb["Hkv"]
    k = bf16_bits_to_f64(pb["k"].data)
    v = bf16_bits_to_f64(pb["v"].data)
    out = {}
    for b in range(len(pb["kv_len"])):
        toks = []
        for pi in range(pb["kv_indptr"][b], pb["kv_indptr"][b + 1]):
            for slot in range(P):
                if len(toks) < pb["kv_len"][b]:
                    toks.append((int(pb["page_indices"][pi]), slot))
        n = pb["qo_indptr"][b + 1] - pb["qo_indptr"][b]
        for r in range(n):
            t = pb["qo_indptr"][b] + r
            pos = pb["kv_len"][b] - n + r
            W = pb["window"][b]
            keys = [j for j in range(len(toks)) if j <= pos and (W == 0 or j > pos - W)]
            for h in range(Hq):
                g = h * Hkv // Hq
                sc = Decimal(pb["sm_scale"])
                s = []
                for j in keys:
                    pg, sl = toks[j]
                    s.append(sc * sum(Decimal(q[t, h, c]) * Decimal(k[pg, g, sl, c]) for c in range(pb["d"])))
                m = max(s)
                e = [(x - m).exp() for x in s]
                l = sum(e)
                o = []
                for c in range(pb["d"]):
                    acc = Decimal(0)
                    for j, ej in zip(keys, e):
                        pg, sl = toks[j]
                        acc += ej * Decimal(v[pg, g, sl, c])
                    o.append(acc / l)
                out[(t, h)] = (np.array([float(x) for x in o]), float(m + l.ln()))
    return out


@pytest.mark.parametrize("seed,kw", [
    (0, {}),
    (1, dict(B=3, rows=(1, 4, 2), kv_len=(1, 9, 40), window=(0, 3, 1), P=8, Hq=6, Hkv=2, d=5)),
    (2, dict(B=1, rows=(8,), kv_len=(30,), window=(7,), P=16, Hq=4, Hkv=1, d=4)),
    (3, dict(B=2, rows=(3, 1), kv_len=(3, 17), window=(2, 0), P=2, Hq=3, Hkv=3, d=6)),
])
def test_matches_decimal_brute_force(seed, kw):
    pb = tiny_problem(seed, **kw)
    out, lse = _run(pb)
    ref = _brute_force(pb)
    for (t, h), (o_ref, l_ref) in ref.items():
        assert np.max(np.abs(out[t, h] - o_ref)) <= 1e-13 * max(1.0, np.max(np.abs(o_ref)))
        assert abs(lse[t, h] - l_ref) <= 1e-13 * max(1.0, abs(l_ref))
    assert not np.isnan(out).any()


def test_gather_hand_built_table():
    # P = 4; request 0 has 6 tokens on pages [7, 2]; request 1 has 3 tokens on page [5]
    kv_indptr = np.array([0, 2, 3])
    page_indices = np.array([7, 2, 5])
    kv_len = np.array([6, 3])
    assert gather_slots(kv_indptr, page_indices, kv_len, 4, 0).tolist() == [28, 29, 30, 31, 8, 9]
    assert gather_slots(kv_indptr, page_indices, kv_len, 4, 1).tolist() == [20, 21, 22]


def test_visible_range_edges():
    # 3 rows, 10 tokens: rows sit at positions 7, 8, 9
    assert [visible_range(10, 3, r, 0) for r in range(3)] == [(0, 7), (0, 8), (0, 9)]
    assert [visible_range(10, 3, r, 4) for r in range(3)] == [(4, 7), (5, 8), (6, 9)]
    assert visible_range(10, 3, 0, 1) == (7, 7)
    assert visible_range(3, 3, 0, 50) == (0, 0)


@pytest.mark.parametrize("window", [0, 1, 3, 7])
def test_zero_query_gives_mean_of_visible_values(window):
    # q = 0: all scores equal, so o = mean of the visible V; with V[j, 0] = j the
    # first component is exactly (lo + p) / 2, which pins the causal and window edges.
    B, P, Hq, Hkv, d = 1, 4, 2, 1, 4
    L, n = 22, 5
    npages = (L + P - 1) // P
    rng = np.random.default_rng(5)
    page_indices = rng.permutation(npages).astype(np.int32)
    vals = np.zeros((npages, Hkv, P, d))
    for t in range(L):
        pg = page_indices[t // P]
        vals[pg, 0, t % P, 0] = t
        vals[pg, 0, t % P, 1:] = rng.standard_normal(d - 1)
    k = PagedKV(bf16_bits(rng.standard_normal((npages, Hkv, P, d))), "bf16")
    v = PagedKV(bf16_bits(vals), "bf16")
    q64 = np.zeros((n, Hq, d))
    out, lse = decode_attention(q64, k, v, page_indices, np.array([0, npages]), np.array([L]),
                                np.array([0, n]), np.array([window]), 0.125)
    for r in range(n):
        lo, p = visible_range(L, n, r, window)
        assert out[r, 0, 0] == (lo + p) / 2
        assert lse[r, 0] == pytest.approx(np.log(p - lo + 1), abs=1e-15)


def test_single_visible_key_returns_its_value():
    pb = tiny_problem(7, B=1, rows=(3,), kv_len=(11,), window=(1,), P=4, Hq=2, Hkv=1, d=8)
    out, lse = _run(pb)
    q64 = bf16_bits_to_f64(pb["q"])
    slots = gather_slots(pb["kv_indptr"], pb["page_indices"], pb["kv_len"], 4, 0)
    K = pb["k"].tokens(slots, 0)
    V = pb["v"].tokens(slots, 0)
    for r in range(3):
        p = 11 - 3 + r
        for h in range(2):
            assert np.array_equal(out[r, h], V[p])
            assert lse[r, h] == pb["sm_scale"] * float(q64[r, h] @ K[p])


def test_two_keys_give_sigmoid_weights():
    q = np.array([[0.5, -1.0, 2.0]])
    k = np.array([[1.0, 0.0, 1.0], [-1.0, 2.0, 0.5]])
    v = np.array([[3.0, -1.0, 0.0], [1.0, 1.0, 4.0]])
    o, lse = attend(q, k, v, 0.7)
    s1, s2 = 0.7 * 2.5, 0.7 * (-0.5 - 2.0 + 1.0)
    w1 = 1.0 / (1.0 + np.exp(s2 - s1))
    assert np.allclose(o[0], w1 * v[0] + (1 - w1) * v[1], rtol=0, atol=1e-15)
    assert lse[0] == pytest.approx(np.logaddexp(s1, s2), abs=1e-15)


def test_identical_keys_and_dominant_key():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((9, 4))
    k = np.tile(rng.standard_normal((1, 4)), (9, 1))
    o, lse = attend(rng.standard_normal((1, 4)), k, v, 0.5)
    assert np.allclose(o[0], v.mean(axis=0), atol=1e-15)
    k2 = np.zeros((9, 4)); k2[4, 0] = 100.0
    o2, _ = attend(np.array([[1.0, 0, 0, 0]]), k2, v, 0.5)      # key 4 is 50 above the rest
    assert np.allclose(o2[0], v[4], atol=1e-20 + 1e-15 * np.abs(v).max() + 9 * np.exp(-50) * np.abs(v).max())


def test_weights_sum_to_one_and_masked_weights_are_zero():
    # V = identity rows: the output is the weight vector itself
    L, n, d = 12, 4, 12
    P = 4
    npages = 3
    page_indices = np.array([2, 0, 1], dtype=np.int32)
    eye = np.zeros((npages, 1, P, d))
    for t in range(L):
        eye[page_indices[t // P], 0, t % P, t] = 1.0
    rng = np.random.default_rng(11)
    k = PagedKV(bf16_bits(rng.standard_normal((npages, 1, P, d))), "bf16")
    v = PagedKV(bf16_bits(eye), "bf16")
    q64 = bf16_bits_to_f64(bf16_bits(rng.standard_normal((n, 2, d))))
    out, _ = decode_attention(q64, k, v, page_indices, np.array([0, 3]), np.array([L]), np.array([0, n]),
                              np.array([3]), 0.3)
    for r in range(n):
        lo, p = visible_range(L, n, r, 3)
        for h in range(2):
            w = out[r, h]
            assert abs(w.sum() - 1.0) <= 1e-15
            assert np.all(w[lo:p + 1] > 0)
            assert np.all(w[:lo] == 0) and np.all(w[p + 1:] == 0)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_split_merge_equals_unsplit(seed):
    pb = tiny_problem(seed, B=2, rows=(4, 2), kv_len=(37, 25), window=(0, 6), P=4, Hq=6, Hkv=2, d=8)
    out, lse = _run(pb)
    q64 = bf16_bits_to_f64(pb["q"])
    rng = np.random.default_rng(seed)
    for b in range(2):
        L = int(pb["kv_len"][b])
        cuts = sorted(set([0, L] + rng.integers(1, L, size=3).tolist()))
        splits = list(zip(cuts[:-1], cuts[1:]))
        o_p, l_p = split_partials(q64, pb["k"], pb["v"], pb["page_indices"], pb["kv_indptr"], pb["kv_len"],
                                  pb["qo_indptr"], pb["window"], pb["sm_scale"], b, splits)
        o_m, l_m = merge_partials(o_p, l_p)
        t0, t1 = pb["qo_indptr"][b], pb["qo_indptr"][b + 1]
        assert np.max(np.abs(o_m - out[t0:t1])) <= 1e-14
        assert np.max(np.abs(l_m - lse[t0:t1])) <= 1e-14
        if b == 1:   # the windowed request: some splits are empty for some rows
            assert np.isneginf(l_p).any()


def test_multi_row_equals_single_row_requests():
    pb = tiny_problem(4, B=1, rows=(5,), kv_len=(29,), window=(0,), P=8, Hq=4, Hkv=2, d=8)
    out, lse = _run(pb)
    q64 = bf16_bits_to_f64(pb["q"])
    for r in range(5):
        p = 29 - 5 + r
        o1, l1 = decode_attention(q64[r:r + 1], pb["k"], pb["v"], pb["page_indices"], pb["kv_indptr"],
                                  np.array([p + 1]), np.array([0, 1]), np.array([0]), pb["sm_scale"])
        assert np.array_equal(o1[0], out[r]) and np.array_equal(l1[0], lse[r])


def test_rows_ignore_positions_past_their_own_and_before_window():
    pb = tiny_problem(6, B=1, rows=(4,), kv_len=(26,), window=(5,), P=4, Hq=4, Hkv=2, d=8)
    out, _ = _run(pb)
    slots = gather_slots(pb["kv_indptr"], pb["page_indices"], pb["kv_len"], 4, 0)
    r = 1
    lo, p = visible_range(26, 4, r, 5)
    k2 = pb["k"].data.copy()
    v2 = pb["v"].data.copy()
    rng = np.random.default_rng(9)
    for j in list(range(0, lo)) + list(range(p + 1, 26)):
        pg, sl = divmod(int(slots[j]), 4)
        k2[pg, :, sl] = bf16_bits(rng.standard_normal(k2[pg, :, sl].shape) * 30)
        v2[pg, :, sl] = bf16_bits(rng.standard_normal(v2[pg, :, sl].shape) * 30)
    pb2 = dict(pb, k=PagedKV(k2, "bf16"), v=PagedKV(v2, "bf16"))
    out2, _ = _run(pb2)
    assert np.array_equal(out2[r], out[r])
    assert not np.array_equal(out2[3], out[3])      # the last row does see position p+1..


def test_head_permutation_within_group_permutes_outputs():
    pb = tiny_problem(8, B=1, rows=(2,), kv_len=(19,), window=(0,), P=4, Hq=6, Hkv=2, d=8)
    out, _ = _run(pb)
    q64 = bf16_bits_to_f64(pb["q"])
    perm = np.array([2, 0, 1, 5, 3, 4])                 # stays inside each group of 3
    out_p, _ = _run(pb, q64=q64[:, perm])
    assert np.array_equal(out_p, out[:, perm])


def test_group_24_matches_per_head_problems():
    # 48 query heads on 2 KV heads (a group that is not a multiple of 16): every
    # head must equal a 1-query-head / 1-KV-head problem on its own KV head.
    pb = tiny_problem(10, B=1, rows=(2,), kv_len=(15,), window=(0,), P=4, Hq=48, Hkv=2, d=4)
    out, _ = _run(pb)
    q64 = bf16_bits_to_f64(pb["q"])
    for h in [0, 5, 23, 24, 30, 47]:
        g = h // 24
        k1 = PagedKV(pb["k"].data[:, g:g + 1], "bf16")
        v1 = PagedKV(pb["v"].data[:, g:g + 1], "bf16")
        o1, _ = decode_attention(q64[:, h:h + 1], k1, v1, pb["page_indices"], pb["kv_indptr"], pb["kv_len"],
                                 pb["qo_indptr"], pb["window"], pb["sm_scale"])
        assert np.max(np.abs(o1[:, 0] - out[:, h])) <= 1e-14


def test_layouts_agree():
    a = tiny_problem(12, layout="HPD")
    b = dict(a)
    b["k"] = PagedKV(np.ascontiguousarray(a["k"].data.transpose(0, 2, 1, 3)), "bf16", "PHD")
    b["v"] = PagedKV(np.ascontiguousarray(a["v"].data.transpose(0, 2, 1, 3)), "bf16", "PHD")
    oa, la = _run(a)
    ob, lb = _run(b)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


@pytest.mark.parametrize("layout", ["HPD", "PHD"])
def test_single_vector_oracle_equals_full_oracle_and_brute_force(layout):
    # decode_attention_one (the checker of the full-size sampled GPU tests) must give, for
    # every (row, head) of a ragged, windowed, multi-row GQA problem, the full oracle's
    # vector and LSE (up to the BLAS summation order: one row against a group of rows)
    # and agree with the decimal brute force
    pb = tiny_problem(17, B=3, rows=(3, 1, 4), kv_len=(9, 14, 22), window=(0, 4, 6), P=4, Hq=6, Hkv=2, d=8,
                      layout=layout)
    q64 = bf16_bits_to_f64(pb["q"])
    full, lse = _run(pb)
    bf = _brute_force(pb) if layout == "HPD" else None
    for t in range(q64.shape[0]):
        for h in range(pb["Hq"]):
            o, l = decode_attention_one(q64[t, h], pb["k"], pb["v"], pb["page_indices"], pb["kv_indptr"],
                                        pb["kv_len"], pb["qo_indptr"], pb["window"], pb["sm_scale"], t, h,
                                        pb["Hkv"], pb["Hq"])
            assert np.max(np.abs(o - full[t, h])) <= 1e-14 * np.max(np.abs(full[t, h]))
            assert abs(l - lse[t, h]) <= 1e-14 * max(1.0, abs(lse[t, h]))
            if bf is not None:
                assert np.max(np.abs(o - bf[(t, h)][0])) <= 1e-13 * np.max(np.abs(bf[(t, h)][0]))
                assert abs(l - bf[(t, h)][1]) <= 1e-13 * max(1.0, abs(bf[(t, h)][1]))


def _brute_force_kv(q, k_tok, v_tok, kv_len, qo_indptr, window, sm_scale, Hq, Hkv):
    """Decimal (40 digits) attention with separate key and value widths: q [T, Hq, dk]
    float64, k_tok / v_tok[b] = [kv_len[b], dk] / [kv_len[b], dv] float64 per (request,
    KV head) in logical token order.  Returns {(t, h): (o, lse)}."""
    getcontext().prec = 40
    out = {}
    for b in range(len(kv_len)):
        n = qo_indptr[b + 1] - qo_indptr[b]
        for r in range(n):
            t = qo_indptr[b] + r
            pos = kv_len[b] - n + r
            W = window[b]
            keys = [j for j in range(kv_len[b]) if j <= pos and (W == 0 or j > pos - W)]
            for h in range(Hq):
                g = h * Hkv // Hq
                K, V = k_tok[b][g], v_tok[b][g]
                s = [Decimal(sm_scale) * sum(Decimal(q[t, h, c]) * Decimal(K[j, c]) for c in range(K.shape[1]))
                     for j in keys]
                m = max(s)
                e = [(x - m).exp() for x in s]
                l = sum(e)
                o = [sum(ej * Decimal(V[j, c]) for j, ej in zip(keys, e)) / l for c in range(V.shape[1])]
                out[(t, h)] = (np.array([float(x) for x in o]), float(m + l.ln()))
    return out


def test_key_and_value_widths_differ_decimal_brute_force():
    # 12-channel keys, 8-channel values (separate head_dim_qk and head_dim_v)
    rng = np.random.default_rng(21)
    B, P, Hq, Hkv, dk, dv = 2, 4, 4, 2, 12, 8
    kv_len = np.array([9, 14]); rows = np.array([2, 3]); window = np.array([0, 5])
    qo = np.concatenate([[0], np.cumsum(rows)])
    pages_b = (kv_len + P - 1) // P
    kvi = np.concatenate([[0], np.cumsum(pages_b)])
    npages = int(pages_b.sum()) + 2
    pidx = rng.permutation(npages)[: int(pages_b.sum())].astype(np.int32)
    k = PagedKV(bf16_bits(rng.standard_normal((npages, Hkv, P, dk))), "bf16")
    v = PagedKV(bf16_bits(rng.standard_normal((npages, Hkv, P, dv))), "bf16")
    qb = bf16_bits(rng.standard_normal((int(qo[-1]), Hq, dk)))
    q = bf16_bits_to_f64(qb)
    sm = float(np.float32(1 / np.sqrt(dk)))
    out, lse = decode_attention(q, k, v, pidx, kvi, kv_len, qo, window, sm)
    assert out.shape == (int(qo[-1]), Hq, dv)
    kt = [[bf16_bits_to_f64(k.data[pidx[kvi[b] + np.arange(kv_len[b]) // P], g, np.arange(kv_len[b]) % P])
           for g in range(Hkv)] for b in range(B)]
    vt = [[bf16_bits_to_f64(v.data[pidx[kvi[b] + np.arange(kv_len[b]) // P], g, np.arange(kv_len[b]) % P])
           for g in range(Hkv)] for b in range(B)]
    bf = _brute_force_kv(q, kt, vt, kv_len, qo, window, sm, Hq, Hkv)
    for (t, h), (o, l) in bf.items():
        assert np.max(np.abs(out[t, h] - o)) <= 1e-13 * np.max(np.abs(o)) and abs(lse[t, h] - l) <= 1e-13 * max(1, abs(l))


def test_latent_cache_against_torch_decode_and_decimal_brute_force():
    # MLA-style cache: key = [latent codes x per-(token, 128 channel) scale, bf16 rotary],
    # value = the latent; the dequantisation against torch's own float8 decode, the
    # attention against a decimal brute force built from those values
    import torch
    from oracle.attention import LatentKV, dequant_q_latent
    rng = np.random.default_rng(22)
    B, P, Hq, Hkv, dv, dr = 2, 4, 3, 1, 256, 8
    kv_len = np.array([7, 11]); rows = np.array([1, 2]); window = np.array([0, 0])
    qo = np.concatenate([[0], np.cumsum(rows)])
    pages_b = (kv_len + P - 1) // P
    kvi = np.concatenate([[0], np.cumsum(pages_b)])
    npages = int(pages_b.sum())
    pidx = rng.permutation(npages).astype(np.int32)
    codes = rng.integers(0, 256, (npages, Hkv, P, dv)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x2A
    scale = (rng.random((npages, Hkv, P, dv // 128)) * 0.05 + 0.001).astype(np.float32)
    rope = bf16_bits(rng.standard_normal((npages, Hkv, P, dr)))
    lkv = LatentKV(codes, scale, rope)
    slots = np.array([0, 5, 13])
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    for s in slots:
        pg, sl = s // P, s % P
        ref = dec[pg, 0, sl] * np.repeat(scale[pg, 0, sl].astype(np.float64), 128)
        assert np.array_equal(lkv.latent(np.array([s]), 0)[0], ref)
        assert np.array_equal(lkv.key_view().tokens(np.array([s]), 0)[0],
                              np.concatenate([ref, bf16_bits_to_f64(rope[pg, 0, sl])]))
    T = int(qo[-1])
    qc = rng.integers(0, 256, (T, Hq, dv)).astype(np.uint8)
    qc[(qc & 0x7F) == 0x7F] = 0x33
    qs = (rng.random((T, Hq, dv // 128)) + 0.5).astype(np.float32)
    qr = bf16_bits(rng.standard_normal((T, Hq, dr)))
    q = dequant_q_latent(qc, qs, qr)
    qref = np.concatenate([torch.from_numpy(qc).view(torch.float8_e4m3fn).double().numpy() *
                           np.repeat(qs.astype(np.float64), 128, axis=2), bf16_bits_to_f64(qr)], axis=2)
    assert np.array_equal(q, qref)
    sm = float(np.float32(1 / np.sqrt(dv + dr)))
    out, lse = decode_attention(q, lkv.key_view(), lkv.value_view(), pidx, kvi, kv_len, qo, window, sm)
    kt = [[lkv.key_view().tokens(pidx[kvi[b] + np.arange(kv_len[b]) // P] * P + np.arange(kv_len[b]) % P, 0)]
          for b in range(B)]
    vt = [[x[0][:, :dv]] for x in kt]
    bf = _brute_force_kv(q, kt, vt, kv_len, qo, window, sm, Hq, Hkv)
    for (t, h), (o, l) in bf.items():
        assert np.max(np.abs(out[t, h] - o)) <= 1e-12 * np.max(np.abs(o)) and abs(lse[t, h] - l) <= 1e-12 * max(1, abs(l))
