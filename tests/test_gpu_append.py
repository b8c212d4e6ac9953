"""KV append through the C ABI, element by element against oracle.cache."""
import numpy as np
import pytest
import torch

from oracle.cache import append_kv
from paged_split_kv_stage1_amd import pa_kv_append
from paged_split_kv_stage1_amd.device_inputs import to_device
from paged_split_kv_stage1_amd.inputs import BF16_NAN_BITS, E4M3_NAN_CODE, INT8_POISON_CODE, make_workload
from tests.gpu_run import run_decode

pytestmark = pytest.mark.gpu


MODE = {"bf16": "none", "fp8_per_tensor": "per_tensor", "fp8_per_head": "per_head",
        "fp8_per_token_head": "per_token_head", "int8_per_tensor": "per_tensor", "int8_per_token_head": "per_token_head"}


def _kvd(kind):
    return kind.split("_")[0]


def _strides(layout, P, hkv, d):
    return (hkv * P * d, P * d, d) if layout == "HPD" else (P * hkv * d, d, hkv * d)


def _scale_strides(layout, P, hkv):
    return (hkv * P, P, 1) if layout == "HPD" else (P * hkv, 1, hkv)


@pytest.mark.parametrize("kind", ["bf16", "fp8_per_tensor", "fp8_per_head", "fp8_per_token_head", "int8_per_tensor",
                                  "int8_per_token_head"])
@pytest.mark.parametrize("src", ["bf16", "fp32"])
@pytest.mark.parametrize("layout", ["HPD", "PHD"])
@pytest.mark.parametrize("d", [128, 256])
def test_append_matches_oracle(kind, src, layout, d):
    print(f"[append] {kind} {src} {layout} d={d}", flush=True)
    P, pages, hkv, n = 16, 9, 2, 37
    rng = np.random.default_rng(d + 7 * len(kind) + len(src))
    shape = (pages, hkv, P, d) if layout == "HPD" else (pages, P, hkv, d)
    # the caches start with arbitrary contents, which must survive wherever nothing lands
    if kind == "bf16":
        k0, v0 = (rng.integers(0, 1 << 16, shape).astype(np.uint16) for _ in range(2))
    else:
        k0, v0 = (rng.integers(0, 256, shape).astype(np.uint8) for _ in range(2))
    pt = kind.endswith("per_token_head")
    ks0, vs0 = (rng.random(shape[:3]).astype(np.float32) for _ in range(2)) if pt else (None, None)
    slots = rng.permutation(pages * P)[:n].astype(np.int64)
    slots[[3, 20]] = -1                                          # padding tokens
    kx = (torch.randn(n, hkv, d) * 3).float()
    vx = (torch.randn(n, hkv, d) * torch.rand(n, hkv, 1) * 5).float()
    if src == "bf16":
        kx, vx = kx.to(torch.bfloat16), vx.to(torch.bfloat16)
        k_rows = kx.view(torch.int16).numpy().view(np.uint16)
        v_rows = vx.view(torch.int16).numpy().view(np.uint16)
    else:
        k_rows, v_rows = kx.numpy(), vx.numpy()
    if kind == "fp8_per_head":
        ts_k = (np.float32(0.021) * (1 + np.arange(hkv))).astype(np.float32)
        ts_v = (np.float32(0.033) / (1 + np.arange(hkv))).astype(np.float32)
    else:
        ts_k, ts_v = np.float32(0.021), np.float32(0.033)

    as_t = (lambda a: torch.from_numpy(a.view(np.int16).copy())) if kind == "bf16" else (lambda a: torch.from_numpy(a.copy()))
    kc, vc = as_t(k0).cuda(), as_t(v0).cuda()
    if pt:
        ksc, vsc = torch.from_numpy(ks0.copy()).cuda(), torch.from_numpy(vs0.copy()).cuda()
    elif kind.endswith("per_tensor"):
        ksc, vsc = torch.tensor([ts_k]).cuda(), torch.tensor([ts_v]).cuda()
    elif kind == "fp8_per_head":
        ksc, vsc = torch.from_numpy(ts_k).cuda(), torch.from_numpy(ts_v).cuda()
    else:
        ksc = vsc = None
    pa_kv_append(kx.cuda(), vx.cuda(), src, n, hkv, d, P, torch.from_numpy(slots).cuda(), kc, vc,
                 _kvd(kind), MODE[kind],
                 _strides(layout, P, hkv, d), ksc, vsc, _scale_strides(layout, P, hkv) if pt else None)
    torch.cuda.synchronize()
    rk, rks = append_kv(k0, ks0, k_rows, src, slots, P, kind, layout, tensor_scale=ts_k)
    rv, rvs = append_kv(v0, vs0, v_rows, src, slots, P, kind, layout, tensor_scale=ts_v)
    got_k, got_v = kc.cpu().numpy(), vc.cpu().numpy()
    if kind == "bf16":
        got_k, got_v = got_k.view(np.uint16), got_v.view(np.uint16)
    assert np.array_equal(got_k, rk) and np.array_equal(got_v, rv)
    if pt:
        assert np.array_equal(ksc.cpu().numpy(), rks) and np.array_equal(vsc.cpu().numpy(), rvs)


@pytest.mark.parametrize("name", ["c2", "c2_ph", "c3", "c4", "c4_i8", "c4_i8t"])
def test_appended_tokens_are_what_decode_reads(name):
    # poison the slots of each request's last 8 tokens, then append those tokens back
    # through pa_kv_append from their bf16 rows: the cache must come back byte for byte
    # (the append encodes exactly like the quantiser that built it) and so must the
    # decode output
    print(f"[append e2e] {name}", flush=True)
    w = make_workload(name, batch=2, ctx=[300, 77], out_dtype="fp32")
    di = to_device(w)
    o_ref, _, _ = run_decode(w, di)
    ref = [None if t is None else t.clone() for t in (di.k, di.v, di.k_scale, di.v_scale)]
    P, hkv, d = w.page_size, w.num_kv_heads, w.head_dim
    toks = []
    for b in range(w.batch):
        for j in range(int(w.kv_len[b]) - 8, int(w.kv_len[b])):
            toks.append((int(w.page_indices[w.kv_indptr[b] + j // P]), j % P))
    slots = torch.tensor([p * P + s for p, s in toks], dtype=torch.int64)
    k_new = torch.stack([w.k[p, :, s] for p, s in toks]).contiguous()      # bf16 [n, Hkv, d]
    v_new = torch.stack([w.v[p, :, s] for p, s in toks]).contiguous()
    for p, s in toks:
        if w.kv_dtype == "bf16":
            di.k.view(torch.int16)[p, :, s] = BF16_NAN_BITS
            di.v.view(torch.int16)[p, :, s] = BF16_NAN_BITS
        else:
            code = INT8_POISON_CODE if w.kv_dtype == "int8" else E4M3_NAN_CODE
            di.k[p, :, s] = code
            di.v[p, :, s] = code
        if w.kv_scale_mode == "per_token_head":
            di.k_scale[p, :, s] = float("nan")
            di.v_scale[p, :, s] = float("nan")
    pa_kv_append(k_new.cuda(), v_new.cuda(), "bf16", len(toks), hkv, d, P, slots.cuda(), di.k, di.v, w.kv_dtype,
                 w.kv_scale_mode, di.kv_layout, di.k_scale, di.v_scale, di.scale_layout)
    torch.cuda.synchronize()
    for got, want in zip((di.k, di.v, di.k_scale, di.v_scale), ref):
        if want is not None:
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8))
    o, _, _ = run_decode(w, di)
    assert np.array_equal(o, o_ref)


# Enough rows for the launch to take four row groups per wave (2048 workgroups and more),
# with a ragged last workgroup: (kind, Hkv, d, P, tokens, source dtype).
MANY = [
    ("fp8_per_token_head", 2, 256, 16, 16384 + 11, "bf16"),
    ("fp8_per_tensor", 8, 128, 64, 8192 + 5, "fp32"),
    ("fp8_per_head", 8, 128, 64, 8192 + 5, "bf16"),
    ("int8_per_token_head", 2, 256, 16, 16384 + 11, "fp32"),
    ("bf16", 2, 256, 16, 16384 + 11, "bf16"),
]


@pytest.mark.parametrize("kind,hkv,d,P,n,src", MANY)
def test_append_many_rows_matches_oracle(kind, hkv, d, P, n, src):
    print(f"[append many] {kind} Hkv={hkv} d={d} n={n} {src}", flush=True)
    rng = np.random.default_rng(n + d)
    pages = (n + P - 1) // P + 9
    shape = (pages, hkv, P, d)
    if kind == "bf16":
        c0 = [rng.integers(0, 1 << 16, shape).astype(np.uint16) for _ in range(2)]
    else:
        c0 = [rng.integers(0, 256, shape).astype(np.uint8) for _ in range(2)]
    pt = kind.endswith("per_token_head")
    s0 = [rng.random(shape[:3]).astype(np.float32) for _ in range(2)] if pt else [None, None]
    slots = rng.permutation(pages * P)[:n].astype(np.int64)
    slots[rng.choice(n, 40, replace=False)] = -1
    new = [torch.randn(n, hkv, d) * 4, torch.randn(n, hkv, d) * torch.rand(n, hkv, 1) * 6]
    if src == "bf16":
        new = [t.to(torch.bfloat16) for t in new]
        rows = [t.view(torch.int16).numpy().view(np.uint16) for t in new]
    else:
        rows = [t.numpy() for t in new]
    if kind == "fp8_per_head":
        ts = [(np.float32(0.03) * (1 + np.arange(hkv))).astype(np.float32),
              (np.float32(0.05) / (1 + np.arange(hkv))).astype(np.float32)]
    else:
        ts = [np.float32(0.03), np.float32(0.05)]
    as_t = (lambda a: torch.from_numpy(a.view(np.int16).copy())) if kind == "bf16" else \
           (lambda a: torch.from_numpy(a.copy()))
    caches = [as_t(c).cuda() for c in c0]
    if pt:
        scales = [torch.from_numpy(s.copy()).cuda() for s in s0]
    elif kind.endswith("per_tensor"):
        scales = [torch.tensor([t]).cuda() for t in ts]
    elif kind == "fp8_per_head":
        scales = [torch.from_numpy(t).cuda() for t in ts]
    else:
        scales = [None, None]
    pa_kv_append(new[0].cuda(), new[1].cuda(), src, n, hkv, d, P, torch.from_numpy(slots).cuda(), caches[0],
                 caches[1], _kvd(kind), MODE[kind],
                 (hkv * P * d, P * d, d), scales[0], scales[1], (hkv * P, P, 1) if pt else None)
    torch.cuda.synchronize()
    for i in range(2):
        rc, rs = append_kv(c0[i], s0[i], rows[i], src, slots, P, kind, "HPD", tensor_scale=ts[i])
        got = caches[i].cpu().numpy()
        assert np.array_equal(got.view(np.uint16) if kind == "bf16" else got, rc)
        if pt:
            assert np.array_equal(scales[i].cpu().numpy(), rs)
