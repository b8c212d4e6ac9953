"""GPU parity of stage 1 with the query rows on the MFMA M axis (S = Q K^T, O = P V, P
transposed through LDS) -- the alternative to the default key-tokens-on-M orientation --
against the fp64 oracle, over every tile shape that orientation is built for."""
import numpy as np
import pytest

from paged_split_kv_stage1_amd.device_inputs import to_device
from paged_split_kv_stage1_amd.inputs import make_workload
from tests.gpu_run import run_decode
from tests.oracle_inputs import max_rel_err
from tests.test_gpu_parity import SMALL, _bar, _oracle

pytestmark = pytest.mark.gpu

BF16_KV = dict(kv="bf16", scale="none")
# (name, make_workload keyword arguments, expected tile shape (waves per row block, blocks per wave))
CASES = [
    ("c1", dict(), (1, 1)),                                                        # d128 bf16, 4 forced splits
    ("c3_r8", SMALL["c3_r8"], (4, 1)),                                             # d256 bf16, causal rows
    ("c4", SMALL["c4"], (4, 1)),                                                   # d256 e4m3 per token-head
    ("c4_r1", SMALL["c4_r1"], (2, 1)),
    ("c5", SMALL["c5"], (4, 3)),                                                   # d128, group 24, windows
    ("c5", dict(batch=5, ctx_range=(60, 2000), rows=1), (2, 1)),
    ("c5", dict(batch=5, ctx_range=(60, 2000), rows=2), (4, 1)),
    ("c5", dict(batch=5, ctx_range=(60, 2000), rows=[5, 1, 3, 2, 4], overrides=BF16_KV), (4, 2)),
    ("c5", dict(batch=4, ctx_range=(60, 2000), rows=1, overrides=BF16_KV), (2, 1)),
    ("c5", dict(batch=4, ctx_range=(60, 2000), rows=2, overrides=BF16_KV), (4, 1)),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_query_rows_on_m_parity(case):
    name, kw, (wq, nqb) = CASES[case]
    print(f"[q_on_m] {name} {kw}", flush=True)
    w = make_workload(name, **kw, out_dtype="fp32")
    di = to_device(w)
    o, pd, lse = run_decode(w, di, out_lse=True, orientation="q_on_m")
    v = int(pd.info.variant)
    assert (v >> 16) & 1 and ((v >> 4) & 15, (v >> 8) & 15) == (wq, nqb)
    ref, ref_lse = _oracle(w)
    err = max_rel_err(o, ref)
    print(f"  items={pd.num_items} S_max={pd.max_splits} maxrel={err:.3e}")
    assert not np.isnan(o).any()
    assert err <= _bar(w), err
    assert not np.isnan(lse).any()
    assert np.max(np.abs(lse - ref_lse)) <= 1e-3 * max(1.0, np.max(np.abs(ref_lse)))


@pytest.mark.parametrize("name", ["c3_r8", "c4"])
def test_orientations_agree(name):
    """Both orientations run the same plan on the same inputs: their outputs differ only by
    rounding order (and by the two-term query of the four-wave FP8 shape, the same in
    both), far inside the bar."""
    print(f"[q_on_m vs kv_on_m] {name}", flush=True)
    w = make_workload(name, **SMALL[name], out_dtype="fp32")
    di = to_device(w)
    a, pa, _ = run_decode(w, di)
    b, pb, _ = run_decode(w, di, orientation="q_on_m")
    assert pa.num_items == pb.num_items
    assert max_rel_err(b, a) <= _bar(w) / 4
