"""Host-side logic of bench.py (no GPU): the one-GPU guard, the algorithmic
byte and flop counts the roofline divides by, and the source hash that keys
the stored LM-head traffic figure."""
import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_headline_algorithmic_bytes_and_flops():
    cfg = synth.make_inputs(synth.HEADLINE, with_weight=False).cfg
    nb, M = cfg.k + 1, 111
    a = bench.algorithmic(cfg, nb, M)
    # W once (152064 x 3584 bf16), the 111 listed H rows, conf + arg
    assert a["w_bytes"] == 152064 * 3584 * 2
    assert a["head_bytes"] == 152064 * 3584 * 2 + 111 * 3584 * 2 + 111 * 8 == 1_090_791_288
    assert a["head_flops"] == 2.0 * 111 * 3584 * 152064
    # prefix K and V, every branch's Q/K/V and H
    assert a["attn_bytes"] == (2 * 512 * 4 * 128 + 5 * 32 * 36 * 128) * 2 + 5 * 32 * 3584 * 2
    assert a["attn_flops"] == 4.0 * 5 * 32 * 28 * (512 + 32) * 128
    assert a["step_bytes"] > a["head_bytes"] + a["attn_bytes"]


def test_model_forward_bytes():
    import lookahead_decoding_amd as lopa
    from lookahead_decoding_amd.model import QWEN7B, model_dims
    d = lopa.Dims(L=512, B=32, Hq=28, Hkv=4, d=128, V=152064, k_max=4, dtype=lopa.BF16)
    m = bench.model_bytes(d, model_dims(**QWEN7B))
    layer = (4608 * 3584 + 4608 + 3584 * 3584 + 2 * 3584 + 2 * 18944 * 3584 + 3584 * 18944) * 2
    assert m["weight_bytes"] == 28 * layer + 3584 * 2
    assert m["forward_bytes"] == 13_092_072_448


def test_source_hash_is_stable_and_keys_the_traffic_table():
    h = bench.head_source_hash()
    assert h == bench.head_source_hash() and len(h) == 16 and int(h, 16) >= 0
    for name, (key, traffic) in bench.HEAD_TRAFFIC.items():
        assert len(key) == 16 and traffic > 0
        assert name in synth.SEVEN_B
