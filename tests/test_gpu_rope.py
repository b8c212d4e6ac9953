"""GPU parity of keys wider than values (pa_decode_stage1_rope): bf16 192/128 keys/values
and the MLA-style latent cache (576/512: e4m3 latent with a scale per (token, 128
channels), bf16 rotary part, value = latent), against the fp64 oracle on the same
quantised inputs.  Bars: 2e-3 for bf16 KV, 2e-2 for the e4m3 latent."""
import numpy as np
import pytest

from oracle.attention import decode_attention
from paged_split_kv_stage1_amd.device_inputs import to_device
from paged_split_kv_stage1_amd.inputs import make_workload
from tests.gpu_run import run_decode
from tests.oracle_inputs import max_rel_err, oracle_inputs

pytestmark = pytest.mark.gpu

BAR = {"bf16": 2e-3, "fp8": 2e-2}
SMALL = {
    "f3": dict(batch=3, ctx=[1000, 77, 2500]),
    "f3_r4": dict(batch=3, ctx=[1000, 5, 2049]),
    "mla": dict(batch=4, ctx=[300, 1000, 64, 2001]),
    "mla_r2": dict(batch=3, ctx=[2, 1500, 129]),
}


def _oracle(w):
    oi = oracle_inputs(w)
    return decode_attention(oi["q64"], oi["k"], oi["v"], w.page_indices, w.kv_indptr, w.kv_len, w.qo_indptr,
                            w.window, w.sm_scale)


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("splits", [0, 1, 5])
def test_rope_parity(name, splits):
    print(f"[rope] {name} splits={splits}", flush=True)
    w = make_workload(name, **SMALL[name], out_dtype="fp32")
    di = to_device(w)
    o, pd, lse = run_decode(w, di, force_splits=splits, out_lse=True)
    ref, ref_lse = _oracle(w)
    err = max_rel_err(o, ref)
    print(f"  items={pd.num_items} S_max={pd.max_splits} maxrel={err:.3e}", flush=True)
    assert o.shape[-1] == w.dv and not np.isnan(o).any()
    assert err <= BAR[w.kv_dtype], err
    assert not np.isnan(lse).any()
    assert np.max(np.abs(lse - ref_lse)) <= 1e-3 * max(1.0, np.max(np.abs(ref_lse)))


@pytest.mark.parametrize("name", ["f3", "mla"])
def test_rope_bf16_output_and_split_invariance(name):
    w = make_workload(name, **SMALL[name], out_dtype="bf16")
    di = to_device(w)
    o, _, _ = run_decode(w, di)
    ref, _ = _oracle(w)
    assert max_rel_err(o, ref) <= BAR[w.kv_dtype] + 2.0 ** -8
    w32 = make_workload(name, **SMALL[name], out_dtype="fp32")
    outs = [run_decode(w32, di, force_splits=s)[0] for s in (1, 2, 7)]
    # bf16 KV: P in two bf16 terms, only fp32 rounding moves; the latent: one bf16 term of P
    # rounded per split, and bf16 partials (2^-9 each), as the per-token-head FP8 path
    tol = 2e-5 if w.kv_dtype == "bf16" else 5 * 2.0 ** -9
    for x in outs[1:]:
        assert max_rel_err(x, outs[0]) <= tol


@pytest.mark.parametrize("hq,rows", [(48, 2), (128, 1), (64, 2)])
def test_latent_many_heads_query_block_groups(hq, rows):
    # more than 64 rows x heads per KV head run as several work items per split (groups of
    # four 16-row blocks); 128 heads is the full MLA head count of the model family
    w = make_workload("mla", batch=2, ctx=[700, 1500], rows=rows, out_dtype="fp32", overrides={"hq": hq})
    di = to_device(w)
    o, pd, _ = run_decode(w, di, force_splits=3)
    ref, _ = _oracle(w)
    assert max_rel_err(o, ref) <= BAR["fp8"]


def test_keys_wider_than_values_masked_positions():
    # windowed rows of the 192/128 form: keys outside a row's window leave it bit-identical
    w = make_workload("f3_r4", batch=2, ctx=[600, 300], out_dtype="fp32")
    w.window[:] = [50, 0]
    di = to_device(w)
    o, _, _ = run_decode(w, di, force_splits=3)
    ref, _ = _oracle(w)
    assert max_rel_err(o, ref) <= BAR["bf16"]
    di.k[di.page_indices[0].item()].fill_(3.0)         # page 0 of request 0: outside every window
    di.v[di.page_indices[0].item()].fill_(-2.0)
    o2, _, _ = run_decode(w, di, force_splits=3)
    n0 = int(w.qo_indptr[1])
    assert np.array_equal(o2[:n0], o[:n0])


@pytest.mark.parametrize("page", [16, 128])
@pytest.mark.parametrize("hq", [16, 48])
def test_latent_windows_ragged_rows_and_page_sizes(page, hq):
    # ragged rows (1-4 per request), sliding windows on half the requests, pages of 16 and
    # 128 tokens (a 16-token load span then lies in one page either way), 16 or 48 heads
    # (one block per item, or three blocks in a four-block item: the fourth team idle)
    print(f"[rope] latent page={page} hq={hq}", flush=True)
    w = make_workload("mla", batch=4, ctx=[900, 130, 2100, 47], rows=[1, 3, 4, 2], page=page, out_dtype="fp32",
                      overrides={"hq": hq})
    w.window[:] = [0, 20, 0, 5]
    di = to_device(w)
    for splits in (0, 3):
        o, pd, lse = run_decode(w, di, force_splits=splits, out_lse=True)
        ref, ref_lse = _oracle(w)
        err = max_rel_err(o, ref)
        print(f"  splits={splits} items={pd.num_items} maxrel={err:.3e}", flush=True)
        assert err <= BAR["fp8"], err
        assert np.max(np.abs(lse - ref_lse)) <= 1e-3 * max(1.0, np.max(np.abs(ref_lse)))


def test_latent_masked_positions_do_not_change_output():
    # keys before a row's window leave the latent kernel's output bit-identical
    w = make_workload("mla_r2", batch=2, ctx=[700, 300], out_dtype="fp32")
    w.window[:] = [64, 0]
    di = to_device(w)
    o, _, _ = run_decode(w, di, force_splits=3)
    ref, _ = _oracle(w)
    assert max_rel_err(o, ref) <= BAR["fp8"]
    di.k[di.page_indices[0].item()].fill_(0x38)        # page 0 of request 0 (tokens 0..63): e4m3 1.0
    di.k_rope[di.page_indices[0].item()].fill_(5.0)
    o2, _, _ = run_decode(w, di, force_splits=3)
    n0 = int(w.qo_indptr[1])
    assert np.array_equal(o2[:n0], o[:n0])


@pytest.mark.parametrize("name,window", [("f3", 0), ("f3_r4", 40), ("mla", 0), ("mla_r2", 30)])
def test_wider_key_gather_bit_exact(name, window):
    # the wider-key kernels' own load enumerators (run by the gather hook over every tile
    # of every work item) against the oracle's page gather and the cache strides: byte
    # offsets of every 16-byte chunk (K main / latent, rotary, V) and element offsets of
    # every latent block scale, bit-exact, including each split's clamped last tile
    import torch

    from oracle.attention import gather_slots
    from paged_split_kv_stage1_amd._lib import pa_debug_gather_rope
    from paged_split_kv_stage1_amd.decode import PagedDecode

    print(f"[gather-rope] {name} window={window}", flush=True)
    w = make_workload(name, **SMALL[name])
    w.window[:] = window
    di = to_device(w)
    pd = PagedDecode(w.qo_indptr, w.kv_indptr, w.kv_len, w.window, w.max_q_len, w.page_size, w.num_q_heads,
                     w.num_kv_heads, w.head_dim, w.q_dtype, w.kv_dtype, w.kv_scale_mode, di.q.device,
                     force_splits=3, head_dim_v=w.head_dim_v)
    M = int(pd.info.max_item_tokens)
    N = 44 if w.latent else 40
    off = torch.full((pd.num_items, M, N), -1, dtype=torch.int64, device="cuda")
    pa_debug_gather_rope(pd.info, pd.plan, di.page_indices, di.kv_layout, di.rope_layout, di.v_layout,
                         di.scale_layout, off)
    torch.cuda.synchronize()
    got = off.cpu().numpy()
    P = w.page_size
    items = pd.items()
    slots_of = {b: gather_slots(w.kv_indptr, w.page_indices, w.kv_len, P, b) for b in range(w.batch)}
    ksp, ksh, kss = di.kv_layout
    for i, it in enumerate(items):
        b, kvh, t0, t1 = int(it[10]), int(it[5]), int(it[8]), int(it[9])
        phys = slots_of[b][t0:t1]
        page, slot = phys // P, phys % P
        if w.latent:
            rsp, rsh, rss = di.rope_layout
            ssp, ssh, sss = di.scale_layout
            exp = np.concatenate([
                (page * ksp + kvh * ksh + slot * kss)[:, None] + 16 * np.arange(32)[None, :],
                ((page * rsp + kvh * rsh + slot * rss) * 2)[:, None] + 16 * np.arange(8)[None, :],
                (page * ssp + kvh * ssh + slot * sss)[:, None] + np.arange(4)[None, :]], axis=1)
        else:
            vsp, vsh, vss = di.v_layout
            krow = (page * ksp + kvh * ksh + slot * kss) * 2
            exp = np.concatenate([krow[:, None] + 16 * np.arange(16)[None, :],
                                  krow[:, None] + 16 * np.arange(8)[None, :],
                                  ((page * vsp + kvh * vsh + slot * vss) * 2)[:, None] + 16 * np.arange(16)[None, :]],
                                 axis=1)
        assert np.array_equal(got[i, :t1 - t0], exp), (i, b, kvh, t0, t1)
        assert (got[i, t1 - t0:] == -1).all()
