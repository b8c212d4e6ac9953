"""The byte/flop accounting reproduces the numbers printed in hpc-ops issue #4."""
import json
import os

from paged_split_kv_stage1_amd.accounting import step_accounting

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hpcops_h200_fp8_decode.json")


def test_reproduces_hpcops_printout():
    g = json.load(open(GOLDEN))
    s = g["shape"]
    B = s["batch"]
    acc = step_accounting(B, list(range(B + 1)), [s["kv_len"]] * B, None, s["block_size"],
                          s["num_q_heads"], s["num_kv_heads"], s["head_dim"], "fp8", "fp8", "per_tensor", "bf16")
    q_bytes = acc["q"] - 4                            # the printout carries no scale bytes
    moved = acc["kv"] + q_bytes + acc["out"]
    assert moved == 540_016_640
    for key in ("printed", "printed_fa3"):
        it = g[key]["throughput_iter_per_s"]
        assert round(moved * it / 1e9, 1) == g[key]["bandwidth_GBps"]
        assert round(acc["flops"] * it / 1e12, 2) == g[key]["tflops"]
    assert acc["page_table"] == B * (s["kv_len"] // s["block_size"]) * 4
