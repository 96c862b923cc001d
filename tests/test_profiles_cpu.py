"""The committed profiler summaries say how they were made, and only with committed files.

Each summary under profiles/ opens with the rocprofv3 command that produced it. The
command must run the profiler directly on a program of this repository (the program
right after `--`) and must name no scratch or working folder.
"""
import json
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")
SUMMARIES = sorted(f for f in os.listdir(PROFILES) if f.endswith(".md"))


def test_there_are_summaries():
    assert any(f.endswith("_kernel_trace.md") for f in SUMMARIES)
    assert any(f.endswith("_hbm_traffic.md") for f in SUMMARIES)
    assert any(f.endswith("_mfma_lds.md") for f in SUMMARIES)


@pytest.mark.parametrize("name", SUMMARIES)
def test_summary_names_its_command(name):
    with open(os.path.join(PROFILES, name)) as fh:
        first = fh.readline()
    m = re.match(r"Command: `(.+)`", first)
    assert m, "%s does not open with its command" % name
    cmd = m.group(1)
    assert "rocprofv3" in cmd and "_work" not in cmd and "/root/reference" not in cmd
    # every program run under the profiler comes right after `--` and is a committed file
    progs = re.findall(r"-- python3 \$REPO/(\S+)", cmd)
    assert progs, "%s: no program after --" % name
    for p in progs:
        assert os.path.isfile(os.path.join(ROOT, p)), p
    assert not re.search(r"-- (env|bash|sh|taskset|numactl)\b", cmd)


@pytest.mark.parametrize("name", ["traffic.json", "mfma.json"])
def test_counter_records_carry_command_and_sources(name):
    with open(os.path.join(PROFILES, name)) as fh:
        rec = json.load(fh)
    text = json.dumps(rec)
    assert "rocprofv3" in text and "_work" not in text
    assert re.search(r"[0-9a-f]{16,}", text), "no source hash recorded"
