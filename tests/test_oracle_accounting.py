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
