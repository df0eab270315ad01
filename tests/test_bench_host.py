"""Host-side checks of bench.py that need no GPU: a multi-GPU request is
refused before anything touches a device, and every committed traffic record
under profiles/ was taken from the kernel sources as they stand (bench.py
reports a record's traffic only while the code of its sources hashes to the
recorded digest, so a stale record would silently turn the bench line's
`traffic` fields into null)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402  (the module only defines functions at import)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


RECORDS = {
    "gemv_stream_q4_M1_grouped_traffic.json": bench.KERNELS[1],
    "skinny_q4_M48_grouped_traffic.json": bench.KERNELS[48],
    "gemv_stream_nvfp4_M1_traffic.json": bench.NVFP4_KERNEL,
    "gemv_stream_mixed_nvfp4_M1_grouped_traffic.json": bench.NVFP4_KERNEL_M1_GROUPED,
    "skinny_nvfp4_bf16_M48_grouped_traffic.json": bench.NVFP4_KERNEL_M48,
}


@pytest.mark.parametrize("name", sorted(RECORDS))
def test_traffic_record_is_current(name):
    kern = RECORDS[name]
    assert os.path.basename(kern[2]) == name
    with open(os.path.join(ROOT, "profiles", name)) as f:
        rec = json.load(f)
    assert rec["csrc_digest"] == bench.csrc_digest_of(kern[1]), f"{name}: counters taken from other kernel sources"
    assert rec["traffic_bytes_per_launch"] > 0
    md = os.path.join(ROOT, "profiles", name[:-len(".json")] + ".md")
    with open(md) as f:
        text = f.read()
    assert rec["csrc_digest"] in text and f"{rec['traffic_bytes_per_launch']:,}" in text, f"{md} disagrees with {name}"


def test_digest_ignores_comments_and_layout():
    src = "int f(int x) {\n    // a comment\n    return x + 1;  /* another */\n}\n"
    same = "int f(int x)\n{ return x + 1; }\n"
    assert bench._code_only(src) == bench._code_only(same)
    assert bench._code_only(src) != bench._code_only(src.replace("x + 1", "x + 2"))
