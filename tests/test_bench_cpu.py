"""Host logic of bench.py (CPU only): the metric's FLOP counts, the block-sparse and KV-cache pair
counts, the staleness rule of the committed traffic summaries and the one-GPU guard.

The pair counts are checked against a brute-force count of the admission rule written out here
(keys j with 0 <= j < Nk, j <= i + off under the causal mask, and i + off - wl <= j <= i + off + wr
for a window, off = Nk - Nq) and against the oracle's own admission mask.
"""
import json
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest
import torch

import bench
from exact_attention_09_amd.inputs import SPARSE_WORKLOADS, WORKLOADS, KVCacheWorkload, sparse_block_mask
from oracle import admitted

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def brute_pairs(Nq, Nk, causal, wl, wr):
    off = Nk - Nq
    n = 0
    for i in range(Nq):
        for j in range(Nk):
            ok = (not causal or j <= i + off) and (wl < 0 or j >= i + off - wl) and (wr < 0 or j <= i + off + wr)
            n += ok
    return n


@pytest.mark.parametrize("Nq,Nk", [(1, 1), (7, 7), (5, 19), (19, 5), (33, 64), (64, 33)])
@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (False, (3, 0)), (True, (4, -1)),
                                           (False, (0, 0)), (False, (2, 5)), (True, (100, 100))])
def test_admitted_pairs_is_the_admission_count(Nq, Nk, causal, window):
    got = bench.admitted_pairs(Nq, Nk, causal, window)
    assert got == brute_pairs(Nq, Nk, causal, *window)
    assert got == int(admitted(Nq, Nk, causal, window[0], window[1]).sum())


def test_metric_flops_of_the_headline_and_window_workloads():
    w = WORKLOADS["causal_b4_h32_n4096_d64_f16"]
    assert bench.metric_flops(w) == 4.0 * 4 * 32 * 4096 * 4096 * 64 / 2 == 274877906944.0
    for name, w in WORKLOADS.items():
        if w.window != (-1, -1):
            assert bench.metric_flops(w) == 4.0 * w.B * w.Hq * w.D * bench.admitted_pairs(w.Nq, w.Nk, w.causal, w.window)


@pytest.mark.parametrize("causal", [True, False])
def test_sparse_pairs_match_brute_force(causal):
    class Small:   # a short sequence (the pair count only reads N and causal)
        N = 700
    Small.causal = causal
    w = SPARSE_WORKLOADS["blocksparse_b1_h16_n65536_d64_f16"]
    # the benchmark's mask recipe (band, sinks, random blocks) on the short sequence, two heads
    mask = sparse_block_mask(Small.N, Small.N, 2, w.band, w.sinks, 0.3, seed=1, causal=causal)
    assert mask.shape == (2, 6, 11)
    got = bench.sparse_pairs(Small, mask)
    causal_mask = admitted(Small.N, Small.N, causal)
    for hm in range(2):
        rows = np.repeat(mask[hm].numpy() != 0, 128, axis=0)[:Small.N]
        blocks = np.repeat(rows, 64, axis=1)[:, :Small.N]
        assert got[hm] == int((blocks & causal_mask).sum())


def test_kvcache_flops_count_each_sequences_pairs():
    w = KVCacheWorkload("t", 3, 4, 10, 50, 8, 2, 64, "bf16", 16, True)
    lengths = [0, 3, 50]
    want = sum(brute_pairs(w.Nq, n, True, -1, -1) for n in lengths if n > 0)
    assert bench.kvcache_flops(w, lengths) == 4.0 * w.Hq * w.D * want


def test_committed_traffic_is_dropped_when_the_kernel_source_changed(tmp_path, monkeypatch):
    for p in bench.KERNEL_SOURCES["fwd"]:
        dst = tmp_path / p
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, p), dst)
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.committed_traffic("some_workload") is None                      # no summary
    h = bench.kernel_source_hash("fwd")
    with open(tmp_path / "profiles" / "traffic_some_workload.txt", "w") as f:
        json.dump({"kernel_source_hash": h, "hbm_bytes_per_launch": 1234}, f)
    assert bench.committed_traffic("some_workload") == 1234                      # same sources
    with open(tmp_path / bench.KERNEL_SOURCES["fwd"][0], "a") as f:
        f.write("\n// changed\n")
    assert bench.kernel_source_hash("fwd") != h
    assert bench.committed_traffic("some_workload") is None                      # stale: dropped


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "error" in line and line["n_gpus"] == 2


def test_roofline_bound_of_the_workloads():
    # the window workloads move more bytes at 8 TB/s than they compute at the MFMA peak; the
    # causal and full workloads are the other way round
    for name, w in WORKLOADS.items():
        flops, nbytes = bench.metric_flops(w), bench.algorithmic_bytes(w)
        want = "hbm" if w.window != (-1, -1) else "mfma"
        if name.startswith("mha_"):   # the small parity cases (launch-bound in practice): 0.13 MB
            want = "hbm"              # against 8 MFLOP, 4.2 MB against 1.07 GFLOP
        assert bench.roofline_bound(flops, nbytes, bench.PEAK_TFLOPS[w.dtype]) == want, name
    w = WORKLOADS["gqa_win256_b1_hq32_hkv8_n16384_d128_bf16"]
    assert bench.algorithmic_bytes(w) == 337641472
    assert bench.roofline_bound(bench.metric_flops(w), 337641472, 2516.6) == "hbm"
    assert bench.roofline_bound(bench.metric_flops(w), 337641472, 1e9) == "hbm"
    assert bench.roofline_bound(bench.metric_flops(w), 1, 2516.6) == "mfma"


def test_bar_workloads_cover_every_bar_configuration():
    """The default line's `bars`: each entry names a dense workload; the backward entry takes fp16 or
    bf16; together with the default workload they cover both dtypes of the 4096-token causal
    shape, the fp8 run, and the GQA and MQA runs with and without the window."""
    names = [n for n, _ in bench.BAR_WORKLOADS]
    assert all(n in WORKLOADS for n in names)
    assert all(WORKLOADS[n].dtype != "e4m3" for n, bwd in bench.BAR_WORKLOADS if bwd)
    covered = set(names) | {bench.DEFAULT_WORKLOAD}
    assert {"causal_b4_h32_n4096_d64_f16", "causal_b4_h32_n4096_d64_bf16", "causal_fp8_b2_h32_n4096_d64_e4m3",
            "gqa_b1_hq32_hkv8_n16384_d128_bf16", "mqa_b1_hq32_hkv1_n16384_d128_bf16",
            "gqa_win256_b1_hq32_hkv8_n16384_d128_bf16", "mqa_win256_b1_hq32_hkv1_n16384_d128_bf16"} <= covered
    assert len({(n, b) for n, b in bench.BAR_WORKLOADS}) == len(bench.BAR_WORKLOADS)
