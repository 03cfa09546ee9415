"""Pin of the byte accounting against the cartridge page's payload table."""
import json
import os

from oracle.accounting import MIB, payload_table, raw_bytes_per_token, token_head_bytes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_payload_table_matches_printed_values():
    g = json.load(open(os.path.join(GOLDEN, "cartridge_payload_table.json")))
    rows = payload_table(g["full_kv_tokens"], g["cartridge_positions"])
    for (name, kib, gib, mib), ref in zip(rows, g["rows"]):
        assert name == ref["layout"]
        assert kib == ref["kib_per_token"]
        assert round(gib, 3) == ref["gib_full"]
        assert round(mib, 3) == ref["mib_cartridge"]
    saving = (raw_bytes_per_token("bf16", "bf16") - raw_bytes_per_token("bf16", "fp8")) * 632 / MIB
    assert round(saving, 3) == g["k16v8_saving_mib"]
    assert saving / (raw_bytes_per_token("bf16", "bf16") * 632 / MIB) == g["k16v8_saving_fraction"]


def test_token_head_bytes_of_the_workloads():
    # K8/V8 per-token scales + exact bf16 K + 16-band fp16 witness
    assert token_head_bytes("fp8", "fp8", exact_k=True, witness=True) == 552
    assert token_head_bytes("fp8", "fp8", exact_k=False, witness=True) == 296
    # K16/V8 cartridge: the exact keys are the stored keys
    assert token_head_bytes("bf16", "fp8", exact_k=False, witness=False) == 388
    assert token_head_bytes("bf16", "bf16", exact_k=False, witness=False) == 512
    # dithered INT8 with per-(256-token block, channel) fp16 scales
    assert token_head_bytes("int8", "int8", exact_k=True, witness=True) == 546


def test_group_scale_keys_match_table6_without_pairs():
    """Keys of the per-token group-scale INT8 format: 128 codes + 4 fp16
    scales = 136 B per token-head, Table 6's m = 0 row (WitCert Sec. 6.2.5)."""
    g = json.load(open(os.path.join(GOLDEN, "witcert_table6_outlier_bytes.json")))
    k_only = token_head_bytes("int8g32", "int8g32", exact_k=False, witness=False) / 2
    assert k_only == g["printed"]["0"]


def test_bench_byte_count_agrees_with_the_accounting():
    """bench.py's algorithmic bytes per token-head (its own count) agree with
    the accounting here for every stored format."""
    import bench
    for kf in ("bf16", "fp8", "int8", "int8g32"):
        for vf in ("bf16", "fp8", "int8", "int8g32"):
            for ex in (False, True):
                for wit in (False, True):
                    assert bench.token_head_bytes(kf, vf, ex, wit) == token_head_bytes(kf, vf, exact_k=ex,
                                                                                        witness=wit), (kf, vf)


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_bench_rejects_a_gqa_group_the_kernels_do_not_take():
    """--q-heads must give 1, 2, 4 or 8 query heads per KV head of the
    workload; the check runs before any device work."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for extra in (["--workload", "3", "--q-heads", "24"], ["--workload", "3", "--q-heads", "12"],
                  ["--q-heads", "64"]):
        r = subprocess.run([sys.executable, os.path.join(root, "bench.py")] + extra, capture_output=True,
                           text=True, timeout=300)
        assert r.returncode == 1 and "--q-heads needs" in r.stderr, (extra, r.stderr[-300:])
