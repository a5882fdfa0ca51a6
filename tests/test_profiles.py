"""The committed rocprofv3 summaries under profiles/ describe the kernels as
they are now: each summary names the command that produced it, and each one
that records a kernel-source hash matches the current sources (bench.py only
takes counter traffic from a summary whose hash matches, so a stale one would
silently drop the bench line's `traffic`)."""
import importlib.util
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")


def _bench():
    spec = importlib.util.spec_from_file_location("bench_for_profiles", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


SUMMARIES = sorted(f for f in os.listdir(PROFILES) if f.endswith(".txt"))
HASH = re.compile(r"(?:kernel source sha256\[:16\]|kernel_source_sha256_16)\s*=\s*([0-9a-f]{16})")


def test_there_are_summaries():
    assert any(f.startswith("gdn_decode_rows__decode_b512_hk16_hv32") for f in SUMMARIES)
    assert any(f.startswith("gdn_chunk_prep+gdn_chunk_state__") for f in SUMMARIES)


@pytest.mark.parametrize("name", SUMMARIES)
def test_summary_names_its_command(name):
    text = open(os.path.join(PROFILES, name)).read()
    assert re.search(r"^# command", text, re.M), f"{name} does not give the command that made it"


@pytest.mark.parametrize("name", SUMMARIES)
def test_summary_matches_current_sources(name):
    text = open(os.path.join(PROFILES, name)).read()
    m = HASH.search(text)
    if m is None:
        return   # a summary of probes or of the CPU oracle: no kernel source to match
    kernel = name.split("__")[0]
    assert m.group(1) == _bench().kernel_source_hash(kernel), \
        f"{name} was taken with other sources of {kernel}; profile it again"
