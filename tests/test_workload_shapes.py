"""The layer shapes of workloads.py pinned to the model description on the pages
(tests/golden/puro2b_shapes.json: 28 layers, hidden 2048, 4096-token context,
Qwen3-1.7B-compatible: 16 query and 8 key/value heads of 128, MLP width 6144),
and every workload tensor's shape derived from those numbers.  Host only."""
import json
import os

import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "puro2b_shapes.json")


def model():
    with open(GOLDEN) as fh:
        return json.load(fh)


def test_linears_follow_the_model():
    m = model()
    q = m["qwen3_1_7b_compatible"]
    hidden, inter = m["hidden"], q["intermediate"]
    qkv_out = (q["query_heads"] + 2 * q["kv_heads"]) * q["head_dim"]
    assert workloads.HIDDEN == hidden
    assert workloads.INTER == inter
    assert workloads.QKV_OUT == qkv_out == 4096
    assert workloads.LINEARS == {                     # (in_features, out_features)
        "qkv": (hidden, qkv_out),
        "o": (q["query_heads"] * q["head_dim"], hidden),
        "gate_up": (hidden, 2 * inter),
        "down": (inter, hidden),
    }


def test_workload_tensor_shapes():
    m = model()
    hidden, ctx, inter = m["hidden"], m["context"], m["qwen3_1_7b_compatible"]["intermediate"]
    shapes = {name: {s.name: s.shape for s in specs} for name, specs in workloads.WORKLOADS.items()}
    assert shapes["qkv_fprop"] == {"x": (ctx, hidden), "w": (workloads.QKV_OUT, hidden)}
    assert shapes["mlp_fprop"] == {"x_gate_up": (2 * ctx, hidden), "w_gate_up": (2 * inter, hidden),
                                   "x_down": (2 * ctx, inter), "w_down": (hidden, inter)}
    assert shapes["mlp_down_bwd"] == {"dy": (2 * ctx, hidden), "w": (hidden, inter), "x": (2 * ctx, inter)}
    layer = shapes["layer"]
    for lin, (kin, kout) in workloads.LINEARS.items():
        assert layer["x_" + lin] == (4 * ctx, kin)
        assert layer["w_" + lin] == (kout, kin)
        assert layer["dy_" + lin] == (4 * ctx, kout)
