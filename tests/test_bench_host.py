"""CPU tests of bench.py's host-side accounting: the useful-FLOP pair count it
reports against the oracle's dense mask, with and without a KV range, and the
check that its stored HBM-traffic figures belong to the current kernel."""
import dataclasses
import json
import os

import numpy as np
import pytest

import bench
import oracle
from workloads import CONFIGS, Layout, layout_from_chunks, streaming_layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_useful_pairs_match_golden_mask_areas():
    with open(os.path.join(ROOT, "tests", "golden", "unmasked_pairs.json")) as f:
        gold = json.load(f)["pairs_per_head"]
    for c in CONFIGS:
        assert bench.useful_pairs(c.layout) == gold[c.name], c.name


@pytest.mark.parametrize("R", [0, 1, 2, 3, 5])
@pytest.mark.parametrize("last_global", [0, 1])
def test_useful_pairs_match_dense_mask_with_window(R, last_global):
    lays = [layout_from_chunks([[7, 5, 9, 3], [4, 4]]), streaming_layout(3, 2, 6),
            Layout((0, 3, 3, 8, 10), (0, 4, 9, 11, 15), (0, 2, 4))]
    for lay in lays:
        lw = dataclasses.replace(lay, kv_range=R, last_global=last_global)
        assert bench.useful_pairs(lw) == int(oracle.block_causal_mask(lw).sum())


def test_stored_traffic_is_tied_to_the_kernel_source():
    for name in ("video480x832", "streaming"):
        path = os.path.join(ROOT, "profiles", f"fwd_bf16_{name}_traffic.json")
        if not os.path.exists(path):
            continue
        with open(path) as f:
            doc = json.load(f)
        if doc.get("kernel_sha256_16") == bench.kernel_hash():
            assert bench.stored_traffic(name) == doc["hbm_bytes_per_launch"]
        else:
            assert bench.stored_traffic(name) is None
    assert bench.stored_traffic("no-such-workload") is None


def test_stored_backward_traffic_is_tied_to_the_backward_source(tmp_path, monkeypatch):
    path = os.path.join(ROOT, "profiles", "bwd_bf16_video480x832_traffic.json")
    if os.path.exists(path):
        with open(path) as f:
            doc = json.load(f)
        want = doc["hbm_bytes_per_call"] if doc.get("kernel_sha256_16") == bench.kernel_hash(bench.BWD_KERNEL_SRC) else None
        assert bench.stored_backward_traffic("video480x832") == want
    # a changed source (comments aside) makes the stored figure stale
    src = tmp_path / "bwd.hip"
    with open(bench.BWD_KERNEL_SRC) as f:
        text = f.read()
    src.write_text(text + "\n// a comment changes nothing\n")
    assert bench.kernel_hash(str(src)) == bench.kernel_hash(bench.BWD_KERNEL_SRC)
    src.write_text(text + "\nint changed;\n")
    assert bench.kernel_hash(str(src)) != bench.kernel_hash(bench.BWD_KERNEL_SRC)
    monkeypatch.setattr(bench, "BWD_KERNEL_SRC", str(src))
    assert bench.stored_backward_traffic("video480x832") is None
    assert bench.stored_backward_traffic("no-such-workload") is None


def test_more_than_one_gpu_is_refused(monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err


def test_parallel_backward_is_refused(monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--backward", "--attention", "parallel"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "self or cross" in capsys.readouterr().err


def test_useful_text_pairs_match_oracle():
    from workloads import text_layout
    for c in CONFIGS:
        t = text_layout(c)
        assert bench.useful_text_pairs(c.layout, t) == oracle.text_pairs(c.layout.q_offsets, t), c.name
