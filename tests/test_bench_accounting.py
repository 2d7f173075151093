"""CPU pins of the benchmark's work accounting: the closed-form pair counts equal a
pair-by-pair count from the oracle's visibility rule, and the padding count
reproduces the worked example of the nalar.dev padding-mask article."""

import json
import os

import numpy as np
import pytest

import bench
from oracle import masks as M

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_padding_example_from_page():
    g = json.load(open(os.path.join(GOLDEN, "padding_example.json")))
    assert bench.padding_positions(g["lengths"], g["padded_to"]) == g["padding_positions"]
    assert g["padded_to"] - g["lengths"][0] == g["padding_positions_of_first_sequence"]


@pytest.mark.parametrize("mask", [M.MASK_CAUSAL, M.MASK_NONE, M.MASK_ALIBI_SQRT])
def test_visible_pairs_match_rule(mask):
    rng = np.random.default_rng(mask)
    L = rng.integers(0, 50, size=5)
    kv = L + rng.integers(0, 40, size=5)
    count = 0
    for Lb, kvb in zip(L, kv):
        a = (kvb - Lb) + np.arange(Lb)[:, None]
        j = np.arange(kvb)[None, :]
        count += int(M.visible(mask, a, j, kvb).sum())
    assert bench.visible_pairs(L, kv, mask != M.MASK_NONE) == count
    assert bench.prefill_valid_flops(L, kv, mask != M.MASK_NONE, 3, 64) == count * 3 * 4 * 64


def test_mla_accounting():
    ctx = [10, 20]
    assert bench.mla_flops(ctx, None, 2, False) == 30 * 2 * 2176
    # SPEC: token t of 3 sees ctx - 3 + t + 1 keys
    assert bench.mla_flops(ctx, [3, 3], 1, True) == ((8 + 9 + 10) + (18 + 19 + 20)) * 2176
    assert bench.mla_bytes(ctx, 2, 4, max_blocks=3) == 30 * 1152 + 2 * 4 * (1152 + 1024 + 4) + 2 * 3 * 4


def test_gpus_above_one_exit_with_message():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(os.path.dirname(GOLDEN), "..", "bench.py"),
                        "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_short_kernel_names():
    assert bench.short_kernel_name(
        "_ZN3mpa12_GLOBAL__N_118prefill_fwd_kernelIDF16bLi128ELi9EEEvNS_13PrefillParamsE") == \
        "prefill_fwd_kernel<bf16,128,9>"
    assert bench.short_kernel_name("_ZN3mpa12_GLOBAL__N_116mla_split_kernelIDF16_EEvNS_9MlaParamsEPKi") == \
        "mla_split_kernel<fp16>"


def test_traffic_summary_tracks_kernel_sources(tmp_path):
    digest = bench.kernel_source_digest()
    good = tmp_path / "t.txt"
    good.write_text(f"# x\nsource_digest {digest}\n"
                    "traffic prefill_fwd_kernel<bf16,128,9> 4 10.0 20.0 40960\n")
    assert bench.read_traffic("prefill_fwd_kernel", str(good)) == 40960
    assert bench.read_traffic("mla_split_kernel", str(good)) is None
    stale = tmp_path / "s.txt"
    stale.write_text("source_digest 0000000000000000\n"
                     "traffic prefill_fwd_kernel<bf16,128,9> 4 10.0 20.0 40960\n")
    assert bench.read_traffic("prefill_fwd_kernel", str(stale)) is None
    assert bench.read_traffic("prefill_fwd_kernel", str(tmp_path / "missing.txt")) is None


def test_short_kernel_names_bool_and_demangled():
    assert bench.short_kernel_name(
        "_ZN3mpa12_GLOBAL__N_116mla_split_kernelIDF16bLb1EEEvNS_9MlaParamsEPKi") == "mla_split_kernel<bf16,true>"
    assert bench.short_kernel_name(
        "void mpa::(anonymous namespace)::mla_split_kernel<bool _Accum, bool, E>(mpa::MlaParams)") == \
        "mla_split_kernel<bf16,true>"
    assert bench.short_kernel_name(
        "void mpa::(anonymous namespace)::mla_split_kernel<bool _Accum, bool, E, false>(mpa::MlaParams)") == \
        "mla_split_kernel<bf16,true,false>"


def test_short_kernel_name_of_the_dma_prefill_kernel():
    import bench
    assert bench.short_kernel_name(
        "_ZN3mpa12_GLOBAL__N_118prefill_dma_kernelIDF16bLi9EEEvNS_13PrefillParamsEPKi") == \
        "prefill_dma_kernel<bf16,9>"


def test_chunked_valid_flops_match_brute_force():
    import bench
    L, kv, C = [7, 5], [20, 5], 6
    pairs = 0
    for l_, k_ in zip(L, kv):
        for i in range(l_):
            a = k_ - l_ + i
            pairs += sum(1 for j in range(k_) if j <= a and j // C == a // C)
    assert bench.prefill_valid_flops_chunked(L, kv, C, 3, 64) == pairs * 3 * 4 * 64
