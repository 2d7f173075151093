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


class _FakeEvent:
    def __init__(self, log):
        self.log = log

    def record(self):
        pass

    def elapsed_time(self, other):
        return 1.0


class _FakeCuda:
    def __init__(self, log):
        self.log = log

    def Event(self, enable_timing=True):
        return _FakeEvent(self.log)

    def synchronize(self):
        self.log.append(("sync",))


class _FakeTorch:
    def __init__(self, log):
        self.cuda = _FakeCuda(log)


class _FakeOp:
    def __init__(self, log):
        self.log = log
        self.ev = None

    def set_launch_events(self, a, b):
        self.ev = (a, b)

    def run(self):
        self.log.append(("run", self.ev))


@pytest.mark.parametrize("iters,warmup", [(10, 3), (20, 4), (4, 9)])
def test_every_timing_event_is_used_once_before_its_timed_launch(iters, warmup):
    # a launch that records an event on its kernels for the first time runs
    # several times slower: time_ops must give every event pair an untimed launch
    # first, and time exactly `iters` launches after the last synchronisation
    log = []
    ops = [_FakeOp(log), _FakeOp(log)]
    ms = bench.time_ops(_FakeTorch(log), ops, iters, warmup)
    assert ms == 1.0
    syncs = [i for i, e in enumerate(log) if e[0] == "sync"]
    runs = [(i, e[1]) for i, e in enumerate(log) if e[0] == "run"]
    timed = [ev for i, ev in runs if syncs[-2] < i < syncs[-1]]
    untimed = [ev for i, ev in runs if i < syncs[-2]]
    assert len(timed) == iters and all(ev is not None for ev in timed)
    assert len(untimed) >= max(warmup, iters)
    warmed = {(id(a), id(b)) for a, b in untimed if a is not None}
    assert all((id(a), id(b)) in warmed for a, b in timed)


def test_counter_summary_clock_column(tmp_path):
    # GRBM_GUI_ACTIVE summed over the 8 dies: 8 x 2.0e6 cycles over a 1 ms dispatch
    # is a 2.0 GHz engine clock; the calibration copy is left out.
    hdr = ("Correlation_Id,Dispatch_Id,Agent_Id,Queue_Id,Process_Id,Thread_Id,Grid_Size,Kernel_Id,"
           "Kernel_Name,Workgroup_Size,LDS_Block_Size,Scratch_Size,VGPR_Count,Accum_VGPR_Count,"
           "SGPR_Count,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp")
    rows = [
        '1,1,"Agent 1",1,1,1,512,7,"__amd_rocclr_copyBuffer",512,0,0,8,0,32,"GRBM_GUI_ACTIVE",5.0e6,0,1000',
        '2,2,"Agent 1",1,1,1,512,8,"mla_combine_kernel",256,0,0,8,0,32,"GRBM_GUI_ACTIVE",1.6e7,0,1000000',
        '3,3,"Agent 1",1,1,1,512,8,"mla_combine_kernel",256,0,0,8,0,32,"GRBM_GUI_ACTIVE",1.2e7,0,1000000',
    ]
    p = tmp_path / "pmc.csv"
    p.write_text(hdr + "\n" + "\n".join(rows) + "\n")
    out = bench.summarize_counters(str(p), "cmd").splitlines()
    head = [l for l in out if l.startswith("kernel")][0].split()
    line = [l for l in out if l.startswith("mla_combine")][0].split()
    assert head[-1] == "clock_GHz" and line[1] == "2"
    assert float(line[head.index("clock_GHz")]) == pytest.approx(1.75)
    assert float(line[head.index("GRBM_GUI_ACTIVE")]) == pytest.approx(1.4e7)


def test_counter_summary_lds_busy_column(tmp_path):
    # 8 dies x 1.0e6 active cycles; 256 CUs x 1.0e6 x 25% = 6.4e7 LDS-busy cycles
    hdr = ("Correlation_Id,Dispatch_Id,Agent_Id,Queue_Id,Process_Id,Thread_Id,Grid_Size,Kernel_Id,"
           "Kernel_Name,Workgroup_Size,LDS_Block_Size,Scratch_Size,VGPR_Count,Accum_VGPR_Count,"
           "SGPR_Count,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp")
    rows = [
        '1,1,"Agent 1",1,1,1,512,8,"k",256,0,0,8,0,32,"GRBM_GUI_ACTIVE",8.0e6,0,500000',
        '1,1,"Agent 1",1,1,1,512,8,"k",256,0,0,8,0,32,"SQ_LDS_IDX_ACTIVE",6.4e7,0,500000',
    ]
    p = tmp_path / "pmc.csv"
    p.write_text(hdr + "\n" + "\n".join(rows) + "\n")
    out = bench.summarize_counters(str(p), "cmd").splitlines()
    head = [l for l in out if l.startswith("kernel")][0].split()
    line = [l for l in out if l.startswith("k ")][0].split()
    assert float(line[head.index("lds_busy_pct")]) == pytest.approx(25.0)
    assert float(line[head.index("clock_GHz")]) == pytest.approx(2.0)
