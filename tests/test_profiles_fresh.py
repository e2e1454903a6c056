"""The committed rocprofv3 summaries describe the committed kernels: each
summary's source_digest (the first 16 hex digits of the sha256 that bench.py
computes over a kernel's sources and include/p3d.h) equals the digest of the
sources as they are now. A kernel edited after its counters were taken fails
here until its profiles are taken again (bench.py would already report such
a kernel's traffic as null). CPU only."""
import glob
import os
import re

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUMMARIES = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md")))


def _digests(path):
    """(kernel, digest) pairs named by a summary's source_digest line; a
    line with a bare digest covers the kernel its file name starts with."""
    for line in open(path):
        m = re.match(r"source_digest: (.+)$", line.strip())
        if not m:
            continue
        body = m.group(1)
        pairs = re.findall(r"([a-z_0-9]+) ([0-9a-f]{16})", body)
        if pairs:
            return pairs
        if re.fullmatch(r"[0-9a-f]{16}", body):
            name = os.path.basename(path)
            kern = [k for k in bench.KERNEL_SOURCES if name.startswith(k + "_")]
            assert len(kern) == 1, name
            return [(kern[0], body)]
    return []


def test_there_are_summaries():
    assert len(SUMMARIES) >= 10


@pytest.mark.parametrize("path", SUMMARIES, ids=[os.path.basename(p) for p in SUMMARIES])
def test_summary_digest_matches_the_sources(path):
    pairs = _digests(path)
    assert pairs, "no source_digest line in %s" % os.path.basename(path)
    for kern, dig in pairs:
        assert kern in bench.KERNEL_SOURCES, kern
        assert dig == bench.kernel_source_digest(kern), (
            "%s was taken on other %s sources (%s, now %s): take the profiles again"
            % (os.path.basename(path), kern, dig, bench.kernel_source_digest(kern)))
