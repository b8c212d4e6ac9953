"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the same
seeded inputs (element by element), plus the method's invariants on the GPU."""
import numpy as np
import pytest
import torch

from oracle.attention import decode_attention, gather_slots
from oracle.quantize import (quantize_int8_per_row, quantize_int8_per_tensor, quantize_per_head, quantize_per_row,
                             quantize_per_tensor)
from paged_split_kv_stage1_amd import (pa_debug_gather, pa_kv_quantize_fp8, pa_kv_quantize_fp8_per_head,
                                       pa_kv_quantize_int8)
from paged_split_kv_stage1_amd.decode import PagedDecode
from paged_split_kv_stage1_amd.device_inputs import to_device
from paged_split_kv_stage1_amd.inputs import make_workload
from tests.gpu_run import run_decode
from tests.oracle_inputs import max_rel_err, oracle_inputs

pytestmark = pytest.mark.gpu

# max relative error (per row-head, inf-norm); INT8 KV (not among the pages' bars) is held
# to the FP8 one
BAR = {"bf16": 2e-3, "fp8": 2e-2, "int8": 2e-2}
BF16_OUT_EXTRA = 2.0 ** -8              # bf16 output rounding on top of the bar

# Shapes of the five workloads at sizes the oracle finishes in seconds; contexts are
# not multiples of the page or tile size, so the last page is ragged.
SMALL = {
    "c1": dict(),
    "c2": dict(batch=6, ctx=[2048, 1000, 77, 1, 640, 1999]),
    "c2_ph": dict(batch=6, ctx=[2048, 1000, 77, 1, 640, 1999]),
    "c3": dict(batch=3, ctx=[3001, 517, 4]),
    "c3_r1": dict(batch=3, ctx=[2500, 130, 1]),
    "c3_r8": dict(batch=2, ctx=[1500, 9]),
    "c4": dict(batch=2, ctx=[2500, 700]),
    "c4_i8": dict(batch=2, ctx=[2500, 700]),
    "c4_i8t": dict(batch=2, ctx=[1300, 45]),
    "c4_r1": dict(batch=2, ctx=[1800, 33]),
    "c5": dict(batch=10, ctx_range=(60, 2500)),
    "c6": dict(batch=2, ctx=[3001, 129]),
    "c6_r4": dict(batch=3, ctx=[2100, 700, 4]),
    "c6_f8": dict(batch=2, ctx=[3001, 129]),
}


def _oracle(w, layout="HPD"):
    oi = oracle_inputs(w, layout)
    out, lse = decode_attention(oi["q64"], oi["k"], oi["v"], w.page_indices, w.kv_indptr, w.kv_len, w.qo_indptr,
                                w.window, w.sm_scale)
    return out, lse


def _bar(w):
    return BAR[w.kv_dtype]


@pytest.mark.parametrize("name", list(SMALL))
def test_parity_fp32_out(name):
    print(f"[parity] {name}", flush=True)
    w = make_workload(name, **SMALL[name], out_dtype="fp32")
    di = to_device(w)
    o, pd, lse = run_decode(w, di, out_lse=True)
    ref, ref_lse = _oracle(w)
    err = max_rel_err(o, ref)
    print(f"  items={pd.num_items} S_max={pd.max_splits} maxrel={err:.3e}")
    assert not np.isnan(o).any()
    assert err <= _bar(w), err
    # stage 1 writes the LSE of single-split rows, the merge that of split rows: every row
    assert not np.isnan(lse).any()
    assert np.max(np.abs(lse - ref_lse)) <= 1e-3 * max(1.0, np.max(np.abs(ref_lse)))


@pytest.mark.parametrize("name", ["c1", "c2", "c2_ph", "c3", "c4", "c4_i8", "c5", "c6", "c6_f8"])
def test_parity_bf16_out(name):
    print(f"[parity-bf16] {name}", flush=True)
    w = make_workload(name, **SMALL[name], out_dtype="bf16")
    di = to_device(w)
    o, pd, _ = run_decode(w, di)
    ref, _ = _oracle(w)
    err = max_rel_err(o, ref)
    print(f"  maxrel={err:.3e}")
    assert err <= _bar(w) + BF16_OUT_EXTRA, err


@pytest.mark.parametrize("mode", ["per_token_head", "per_tensor"])
@pytest.mark.parametrize("d", [64, 128, 256, 512, 1024])
def test_quantizer_bit_exact(mode, d):
    g = torch.Generator().manual_seed(d)
    x = (torch.randn(333, d, generator=g) * torch.rand(333, 1, generator=g) * 5).to(torch.bfloat16)
    x[7] = 0
    x[11, :3] = torch.tensor([1e-30, 3e4, -2.0])
    x[13, :4] = torch.tensor([-0.0, 9.2e-41, -9.2e-41, 0.0])          # signed zeros, bf16 subnormals
    xd = x.cuda()
    n = x.shape[0]
    codes = torch.empty(n, d, dtype=torch.uint8, device="cuda")
    scale = torch.empty(n if mode == "per_token_head" else 1, dtype=torch.float32, device="cuda")
    pa_kv_quantize_fp8(xd, "bf16", n, d, mode, codes, scale)
    torch.cuda.synchronize()
    bits = x.view(torch.int16).numpy().astype(np.uint16)
    rc, rs = quantize_per_row(bits, "bf16") if mode == "per_token_head" else quantize_per_tensor(bits, "bf16")
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scale.cpu().numpy().reshape(np.shape(rs)), rs)


@pytest.mark.parametrize("mode", ["per_token_head", "per_tensor"])
def test_quantizer_division_stress(mode):
    # fp32 values with arbitrary mantissas over 2^-20..2^20: the quotient x / scale must
    # be the IEEE fp32 one for every element (the kernel divides once per row and
    # corrects each element's product with the reciprocal)
    rng = np.random.default_rng(17)
    n, d = 2048, 64
    x = (rng.uniform(1.0, 2.0, (n, d)) * np.exp2(rng.integers(-20, 21, (n, d)))
         * rng.choice([-1.0, 1.0], (n, d))).astype(np.float32)
    x[::7, 5] = -0.0
    codes = torch.empty(n, d, dtype=torch.uint8, device="cuda")
    scale = torch.empty(n if mode == "per_token_head" else 1, dtype=torch.float32, device="cuda")
    pa_kv_quantize_fp8(torch.from_numpy(x).cuda(), "fp32", n, d, mode, codes, scale)
    torch.cuda.synchronize()
    rc, rs = quantize_per_row(x, "fp32") if mode == "per_token_head" else quantize_per_tensor(x, "fp32")
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scale.cpu().numpy().reshape(np.shape(rs)), rs)


# Row counts at which the launch takes four row groups per wave (two for d = 1024), plus a
# ragged tail; and a per-tensor size whose grid-stride loop runs twice and then a tail.
MANY_ROWS = {64: 262144 + 37, 128: 131072 + 37, 256: 65536 + 37, 512: 32768 + 37, 1024: 16384 + 37}


@pytest.mark.parametrize("d", list(MANY_ROWS))
def test_quantizer_many_rows_bit_exact(d):
    n = MANY_ROWS[d]
    print(f"[quant many] d={d} rows={n}", flush=True)
    g = torch.Generator().manual_seed(d + 1)
    x = (torch.randn(n, d, generator=g) * torch.rand(n, 1, generator=g) * 5).to(torch.bfloat16)
    codes = torch.empty(n, d, dtype=torch.uint8, device="cuda")
    scale = torch.empty(n, dtype=torch.float32, device="cuda")
    pa_kv_quantize_fp8(x.cuda(), "bf16", n, d, "per_token_head", codes, scale)
    torch.cuda.synchronize()
    rc, rs = quantize_per_row(x.view(torch.int16).numpy().view(np.uint16), "bf16")
    assert np.array_equal(scale.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_quantizer_per_tensor_many_groups_bit_exact():
    n, d = 133000, 128
    g = torch.Generator().manual_seed(3)
    x = (torch.randn(n, d, generator=g) * 2).to(torch.bfloat16)
    x[n - 1, d - 1] = -37.5                                          # the amax sits in the tail
    codes = torch.empty(n, d, dtype=torch.uint8, device="cuda")
    scale = torch.empty(1, dtype=torch.float32, device="cuda")
    pa_kv_quantize_fp8(x.cuda(), "bf16", n, d, "per_tensor", codes, scale)
    torch.cuda.synchronize()
    rc, rs = quantize_per_tensor(x.view(torch.int16).numpy().view(np.uint16), "bf16")
    assert scale.cpu().numpy()[0] == rs
    assert np.array_equal(codes.cpu().numpy(), rc)


# (tokens, heads, d): few tokens (one small launch), and enough rows for four row groups
# per wave with a ragged tail; 64 query heads as in the per-head FP8 workload.
PER_HEAD_SHAPES = [(37, 3, 64), (129, 8, 128), (5, 2, 256), (9, 1, 512), (3, 64, 128), (16384 + 7, 8, 128),
                   (4101, 2, 1024)]


@pytest.mark.parametrize("n,h,d", PER_HEAD_SHAPES)
@pytest.mark.parametrize("src", ["bf16", "fp32"])
def test_quantizer_per_head_bit_exact(n, h, d, src):
    print(f"[quant per-head] n={n} H={h} d={d} {src}", flush=True)
    g = torch.Generator().manual_seed(n + h + d)
    x = torch.randn(n, h, d, generator=g) * (torch.rand(1, h, 1, generator=g) * 8)
    x[0, 0, :4] = torch.tensor([-0.0, 9.2e-41, -9.2e-41, 0.0])        # signed zeros, bf16 subnormals
    if h > 1:
        x[:, h - 1] = 0                                                # an all-zero head: scale 1
    x = x.to(torch.bfloat16) if src == "bf16" else x
    codes = torch.empty(n, h, d, dtype=torch.uint8, device="cuda")
    scale = torch.full((h,), float("nan"), dtype=torch.float32, device="cuda")
    pa_kv_quantize_fp8_per_head(x.cuda(), src, n, h, d, codes, scale)
    torch.cuda.synchronize()
    xs = x.view(torch.int16).numpy().view(np.uint16) if src == "bf16" else x.numpy()
    rc, rs = quantize_per_head(xs, src, 1)
    assert np.array_equal(scale.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_quantizer_per_head_twice_in_a_row():
    # the amax words are cleared by every call: a second, smaller call gives its own scales
    for n, amp in ((500, 30.0), (20, 0.5)):
        x = (torch.randn(n, 4, 128, generator=torch.Generator().manual_seed(n)) * amp).to(torch.bfloat16)
        codes = torch.empty(n, 4, 128, dtype=torch.uint8, device="cuda")
        scale = torch.empty(4, dtype=torch.float32, device="cuda")
        pa_kv_quantize_fp8_per_head(x.cuda(), "bf16", n, 4, 128, codes, scale)
        torch.cuda.synchronize()
        rc, rs = quantize_per_head(x.view(torch.int16).numpy().view(np.uint16), "bf16", 1)
        assert np.array_equal(scale.cpu().numpy(), rs) and np.array_equal(codes.cpu().numpy(), rc)


@pytest.mark.parametrize("mode", ["per_token_head", "per_tensor"])
@pytest.mark.parametrize("d,n", [(64, 333), (128, 131072 + 37), (256, 45), (512, 32768 + 37), (1024, 16384 + 37)])
def test_quantizer_int8_bit_exact(mode, d, n):
    # ties: rows whose amax is 127 (scale 1) hold exact halves, which round to even
    print(f"[quant int8] {mode} d={d} n={n}", flush=True)
    g = torch.Generator().manual_seed(d + n)
    x = torch.randn(n, d, generator=g) * torch.rand(n, 1, generator=g) * 4
    x[3] = 0
    x[5, :6] = torch.tensor([127.0, 2.5, 3.5, -0.5, -1.5, 0.5])
    x[5, 6:] = 0.25
    x[7, :4] = torch.tensor([-0.0, 9.2e-41, -9.2e-41, 0.0])
    for src in ("bf16", "fp32"):
        xs = x.to(torch.bfloat16) if src == "bf16" else x
        codes = torch.empty(n, d, dtype=torch.int8, device="cuda")
        scale = torch.empty(n if mode == "per_token_head" else 1, dtype=torch.float32, device="cuda")
        pa_kv_quantize_int8(xs.cuda(), src, n, d, mode, codes, scale)
        torch.cuda.synchronize()
        host = xs.view(torch.int16).numpy().view(np.uint16) if src == "bf16" else xs.numpy()
        rc, rs = quantize_int8_per_row(host, src) if mode == "per_token_head" else quantize_int8_per_tensor(host, src)
        assert np.array_equal(scale.cpu().numpy().reshape(np.shape(rs)), rs)
        assert np.array_equal(codes.cpu().numpy(), rc)


def test_quantizer_fp32_source_bit_exact():
    g = torch.Generator().manual_seed(5)
    x = torch.randn(100, 128, generator=g) * 3
    codes = torch.empty(100, 128, dtype=torch.uint8, device="cuda")
    scale = torch.empty(100, dtype=torch.float32, device="cuda")
    pa_kv_quantize_fp8(x.cuda(), "fp32", 100, 128, "per_token_head", codes, scale)
    torch.cuda.synchronize()
    rc, rs = quantize_per_row(x.numpy(), "fp32")
    assert np.array_equal(codes.cpu().numpy(), rc) and np.array_equal(scale.cpu().numpy(), rs)


GATHER_CASES = [("c1", "HPD"), ("c2", "HPD"), ("c2", "PHD"), ("c3", "HPD"), ("c3", "PHD"), ("c3_r1", "PHD"),
                ("c3_r8", "HPD"), ("c4", "HPD"), ("c4", "PHD"), ("c4_r1", "HPD"), ("c4_i8", "PHD"),
                ("c4_i8t", "HPD"), ("c5", "HPD"), ("c5", "PHD"), ("c6", "HPD"), ("c6_f8", "PHD")]


@pytest.mark.parametrize("name,layout", GATHER_CASES)
def test_gather_bit_exact(name, layout):
    # Stage 1's own KV address code (run by the gather hook over every tile of every work
    # item, every KV head and query-block group) against the oracle's page gather and the
    # cache strides: byte offsets of every 16-byte K/V chunk and element offsets of every
    # per-token scale, bit-exact; entries past an item's token range stay untouched.
    print(f"[gather] {name} {layout}", flush=True)
    w = make_workload(name, **SMALL[name])
    di = to_device(w, layout=layout)
    pd = PagedDecode(w.qo_indptr, w.kv_indptr, w.kv_len, w.window, w.max_q_len, w.page_size, w.num_q_heads,
                     w.num_kv_heads, w.head_dim, w.q_dtype, w.kv_dtype, w.kv_scale_mode, di.q.device,
                     force_splits=w.forced_splits or 0)
    M = int(pd.info.max_item_tokens)
    esz = 2 if w.kv_dtype == "bf16" else 1
    C = w.head_dim * esz // 16
    per_tok = w.kv_scale_mode == "per_token_head" or w.kv_dtype == "int8"
    kv_off = torch.full((pd.num_items, M, C), -1, dtype=torch.int64, device="cuda")
    sc_off = torch.full((pd.num_items, M, 2), -1, dtype=torch.int64, device="cuda") if per_tok else None
    pa_debug_gather(pd.info, pd.plan, di.page_indices, di.kv_layout, di.scale_layout, kv_off, sc_off)
    torch.cuda.synchronize()
    got = kv_off.cpu().numpy()
    got_sc = sc_off.cpu().numpy() if per_tok else None
    sp, sh, ss = di.kv_layout
    csp, csh, css = di.scale_layout if di.scale_layout is not None else (0, 0, 0)
    P = w.page_size
    items = pd.items()
    assert items[:, 9].max() - items[:, 8].min() > 0
    slots_of = {b: gather_slots(w.kv_indptr, w.page_indices, w.kv_len, P, b) for b in range(w.batch)}
    for i, it in enumerate(items):
        b, kvh, t0, t1 = int(it[10]), int(it[5]), int(it[8]), int(it[9])
        phys = slots_of[b][t0:t1]
        page, slot = phys // P, phys % P
        exp = ((page * sp + kvh * sh + slot * ss) * esz)[:, None] + 16 * np.arange(C)[None, :]
        assert np.array_equal(got[i, :t1 - t0], exp), (i, b, kvh, t0, t1)
        assert (got[i, t1 - t0:] == -1).all()
        if per_tok:
            sexp = page * csp + kvh * csh + slot * css
            assert np.array_equal(got_sc[i, :t1 - t0, 0], sexp) and np.array_equal(got_sc[i, :t1 - t0, 1], sexp)
            assert (got_sc[i, t1 - t0:] == -1).all()


# With bf16 two-term P (bf16 KV) the split count only moves fp32 rounding.  Where P
# is rounded relative to each split's running maximum the rounding of P itself
# changes with the splits: per-tensor FP8 V requantises P to two e4m3 terms (about
# 1e-3 here), per-token-head FP8 KV carries P as one bf16 term (relative rounding
# <= 2^-9 per probability; 4 x 2^-9 bounds the difference of two such sums).  With
# one-byte KV codes the split partials are stored in bf16 (2^-9 relative each, so the
# merged row moves by at most 2^-9 more).
SPLIT_TOL = {"c3": 2e-5, "c4": 5 * 2.0 ** -9, "c4_i8": 5 * 2.0 ** -9, "c2": 3e-3 + 2.0 ** -9,
             "c2_ph": 3e-3 + 2.0 ** -9, "c6": 2e-5, "c6_f8": 5 * 2.0 ** -9}


@pytest.mark.parametrize("name", ["c3", "c4", "c4_i8", "c2", "c2_ph", "c6", "c6_f8"])
def test_split_count_invariance(name):
    w = make_workload(name, **SMALL[name], out_dtype="fp32")
    di = to_device(w)
    outs = [run_decode(w, di, force_splits=s)[0] for s in (1, 2, 5, 13)]
    for o in outs[1:]:
        assert max_rel_err(o, outs[0]) <= SPLIT_TOL[name]


def test_multi_row_equals_single_row_requests():
    w = make_workload("c3", batch=1, ctx=[1234], out_dtype="fp32")
    di = to_device(w)
    o, _, _ = run_decode(w, di)
    n = w.total_rows
    for r in range(n):
        w1 = make_workload("c3", batch=1, ctx=[1234], out_dtype="fp32")
        p = 1234 - n + r
        w1.qo_indptr = np.array([0, 1], np.int32)
        w1.kv_len = np.array([p + 1], np.int32)
        w1.kv_indptr = np.array([0, (p + 1 + w.page_size - 1) // w.page_size], np.int32)
        w1.page_indices = w.page_indices[: w1.kv_indptr[1]]
        w1.q = w.q[r:r + 1].clone()
        di1 = to_device(w1)
        di1.k, di1.v, di1.page_indices = di.k, di.v, di.page_indices[: w1.kv_indptr[1]].contiguous()
        o1, _, _ = run_decode(w1, di1)
        assert max_rel_err(o1[0], o[r]) <= 2e-5


@pytest.mark.parametrize("name", ["c3", "c4", "c5"])
def test_masked_positions_do_not_change_output(name):
    # finite changes of K/V at positions a row may not see leave that row bit-identical
    shape = {"c3": dict(batch=2, ctx=[900, 300]), "c4": dict(batch=2, ctx=[700, 260]),
             "c5": dict(batch=4, ctx_range=(200, 900))}[name]
    w = make_workload(name, **shape, out_dtype="fp32")
    if name == "c5":
        w.window[:] = [64, 0, 64, 0]
    di = to_device(w)
    o, _, _ = run_decode(w, di, force_splits=3)
    b = 0
    n = int(w.qo_indptr[b + 1] - w.qo_indptr[b])
    L = int(w.kv_len[b])
    slots = gather_slots(w.kv_indptr, w.page_indices, w.kv_len, w.page_size, b)
    r = 0
    p = L - n + r
    lo = max(0, p - int(w.window[b]) + 1) if w.window[b] > 0 else 0
    hidden = list(range(p + 1, L)) + list(range(0, lo))
    if not hidden:
        pytest.skip("no hidden positions")
    g = torch.Generator().manual_seed(3)
    for j in hidden:
        pg, sl = divmod(int(slots[j]), w.page_size)
        w.k[pg, :, sl] = (torch.randn(w.k[pg, :, sl].shape, generator=g) * 7).to(torch.bfloat16)
        w.v[pg, :, sl] = (torch.randn(w.v[pg, :, sl].shape, generator=g) * 7).to(torch.bfloat16)
    di2 = to_device(w)
    if w.kv_scale_mode == "per_tensor":
        pytest.skip("per-tensor scale changes with the data")
    o2, _, _ = run_decode(w, di2, force_splits=3)
    t = int(w.qo_indptr[b]) + r
    assert np.array_equal(o2[t], o[t])
    if n > 1:
        assert not np.array_equal(o2[t + n - 1], o[t + n - 1]) or p + 1 >= L


def test_phd_layout_matches_hpd():
    w = make_workload("c4", **SMALL["c4"], out_dtype="fp32")
    a, _, _ = run_decode(w, to_device(w, layout="HPD"))
    b, _, _ = run_decode(w, to_device(w, layout="PHD"))
    assert np.array_equal(a, b)
    ref, _ = _oracle(w, layout="PHD")
    assert max_rel_err(b, ref) <= BAR["fp8"]


@pytest.mark.parametrize("case", [
    dict(ctx=[1, 5, 8], rows=[1, 5, 8]),          # every key is a new row (kv_len == rows)
    dict(ctx=[64, 65, 63], rows=[8, 1, 3]),       # tile-boundary lengths
])
def test_edge_lengths(case):
    w = make_workload("c3", batch=3, ctx=case["ctx"], rows=case["rows"], out_dtype="fp32")
    di = to_device(w)
    for fs in (0, 1, 4):
        o, _, _ = run_decode(w, di, force_splits=fs)
        ref, _ = _oracle(w)
        assert max_rel_err(o, ref) <= BAR["bf16"]


@pytest.mark.parametrize("window", [1, 2, 63, 64, 65, 200])
def test_window_edges(window):
    w = make_workload("c5", batch=3, ctx=[700, 129, 64], rows=[8, 3, 1], out_dtype="fp32")
    w.window[:] = window
    di = to_device(w)
    o, _, _ = run_decode(w, di, force_splits=4)
    ref, _ = _oracle(w)
    assert max_rel_err(o, ref) <= BAR["fp8"]


@pytest.mark.parametrize("name", ["c3", "c4"])
@pytest.mark.parametrize("fs", [64, 81])
def test_many_splits_workgroup_merge(fs, name):
    # 64 or more splits take the merge shape in which four waves share one
    # (row, head, d slice); fewer take the one-wave-per-slice shape.  bf16 KV merges
    # float32 partials, FP8 KV bf16 partials.
    print(f"[many-splits] {name} {fs}", flush=True)
    w = make_workload(name, batch=2, ctx=[5300, 4100], out_dtype="fp32")
    di = to_device(w)
    o, pd, lse = run_decode(w, di, force_splits=fs, out_lse=True)
    assert pd.max_splits >= 64
    ref, ref_lse = _oracle(w)
    assert max_rel_err(o, ref) <= _bar(w)
    assert np.max(np.abs(lse - ref_lse)) <= 1e-3 * max(1.0, np.max(np.abs(ref_lse)))


def test_head_permutation_within_group_permutes_outputs():
    # heads of one KV group share the MFMA row blocks; every row's softmax and P.V are
    # independent of the other rows, so permuting them permutes the outputs bit for bit
    w = make_workload("c5", batch=3, ctx=[900, 130, 64], rows=[8, 3, 1], out_dtype="fp32")
    di = to_device(w)
    o, _, _ = run_decode(w, di)
    G = w.num_q_heads // w.num_kv_heads
    perm = np.concatenate([g * G + np.random.default_rng(g).permutation(G) for g in range(w.num_kv_heads)])
    di.q = di.q[:, torch.as_tensor(perm, device=di.q.device)].contiguous()
    o2, _, _ = run_decode(w, di)
    assert np.array_equal(o2, o[:, perm])


@pytest.mark.parametrize("name,page", [("c2", 128), ("c2", 1024), ("c2_ph", 128), ("c3", 256), ("c4", 1024),
                                       ("c4_i8", 128), ("c5", 128)])
@pytest.mark.parametrize("layout", ["HPD", "PHD"])
def test_large_pages(name, page, layout):
    # pages of 128..1024 tokens: several tiles (and whole splits) inside one page, and a
    # split boundary inside a page
    print(f"[large-pages] {name} P={page} {layout}", flush=True)
    w = make_workload(name, **SMALL[name], page=page, out_dtype="fp32")
    di = to_device(w, layout=layout)
    for fs in (0, 3):
        o, _, _ = run_decode(w, di, force_splits=fs)
        ref, _ = _oracle(w, layout=layout)
        assert max_rel_err(o, ref) <= _bar(w)


def test_more_splits_than_blocks_gives_empty_splits():
    w = make_workload("c1", ctx=100, out_dtype="fp32")
    di = to_device(w)
    o, pd, _ = run_decode(w, di, force_splits=7)
    ref, _ = _oracle(w)
    assert max_rel_err(o, ref) <= BAR["bf16"]


def test_graph_capture_replay():
    w = make_workload("c3", **SMALL["c3"], out_dtype="fp32")
    di = to_device(w)
    o_eager, pd, _ = run_decode(w, di)
    out = torch.zeros(w.total_rows, w.num_q_heads, w.head_dim, dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        pd.run(di.q, di.q_scale, di.k, di.v, di.kv_layout, di.k_scale, di.v_scale, di.scale_layout, di.page_indices,
               w.sm_scale, out, "fp32", stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pd.run(di.q, di.q_scale, di.k, di.v, di.kv_layout, di.k_scale, di.v_scale, di.scale_layout, di.page_indices,
               w.sm_scale, out, "fp32", stream=torch.cuda.current_stream())
    for _ in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().astype(np.float64), o_eager)


@pytest.mark.parametrize("name", ["c4", "c4_i8", "c6_f8"])
def test_query_rows_with_outliers_tiny_tails_and_zeros(name):
    # The four-wave kernels of these shapes carry each bf16 query row as two 8-bit terms
    # under the row's own scale (amax/448 for e4m3, amax/127 for int8).  Rows dominated by
    # one element, rows with a tail of elements a thousand times smaller, and all-zero rows
    # (scale 1, every code 0: uniform weights) must still meet the bar.
    print(f"[query-outliers] {name}", flush=True)
    w = make_workload(name, **SMALL[name], out_dtype="fp32")
    q = w.q.float()
    q[:, :, 7] *= 40.0
    q[-1, :, 100:] *= 1e-3
    q[0] = 0.0
    q[1, 3] = 0.0
    w.q = q.to(torch.bfloat16)
    di = to_device(w)
    o, pd, _ = run_decode(w, di)
    ref, _ = _oracle(w)
    err = max_rel_err(o, ref)
    print(f"  items={pd.num_items} maxrel={err:.3e}", flush=True)
    assert not np.isnan(o).any()
    assert err <= _bar(w), err
