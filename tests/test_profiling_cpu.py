"""Host logic of the measurement records: a traffic record stored under
profiles/ is used by bench.py only while the kernel sources and their
per-file compiler flags are the ones it was measured on."""

import json
import os

from windowed_gqa_kv_amd import build, profiling

DEC = ["decode_mfma.hip", "common.h", "kernels.h"]
PF = ["prefill_mfma.hip", "common.h", "kernels.h"]


def test_source_hash_covers_per_file_flags(monkeypatch):
    h0 = profiling.src_hash(DEC)
    assert h0 == profiling.src_hash(DEC)  # deterministic
    flags = dict(build.FILE_FLAGS)
    flags["decode_mfma.hip"] = flags.get("decode_mfma.hip", []) + ["-mllvm", "-some-other-option"]
    monkeypatch.setattr(build, "FILE_FLAGS", flags)
    assert profiling.src_hash(DEC) != h0
    # a flag of another source does not touch the decode's hash
    monkeypatch.setattr(build, "FILE_FLAGS", dict(flags, **{"rotary.hip": ["-O1"]}))
    assert profiling.src_hash(DEC) == profiling.src_hash(DEC)
    h1 = profiling.src_hash(DEC)
    monkeypatch.setattr(build, "FILE_FLAGS", flags)
    assert profiling.src_hash(DEC) == h1


def test_source_hash_differs_between_kernels():
    assert profiling.src_hash(DEC) != profiling.src_hash(PF)


def test_committed_traffic_records_match_the_sources():
    """Every record bench.py reads was measured on the current kernels.  A
    stale record makes bench.py print a null traffic figure; this test then
    reports it as skipped (with the key), so that a kernel change can be
    committed before its counters are taken again."""
    import pytest
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles", "traffic.json")
    with open(path) as f:
        table = json.load(f)
    want = {"append_decode": profiling.src_hash(DEC), "decode": profiling.src_hash(DEC),
            "prefill": profiling.src_hash(PF)}
    assert table, "no traffic records"
    stale = [key for key, rec in table.items() if rec["src_hash"] != want[key.split("/")[0]]]
    for rec in table.values():
        assert rec["bytes_per_launch"] > 0
    if stale:
        pytest.skip(f"traffic records measured on other sources: {stale}")
