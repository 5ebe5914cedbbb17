"""CPU tests of bench.py's host logic: which sources a stored counter record
depends on (a record is reported only while those files are unchanged)."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def names(paths):
    return {os.path.basename(p) for p in paths}


def test_kernel_sources_follow_the_defining_file_and_its_headers():
    # the forward's prep: its own file, the headers it includes (also through
    # other headers), the planner and the build flags; no backward source
    s = names(bench.kernel_sources("chunk_prep"))
    assert {"gla_prep.hip", "gla_records.h", "gla_dma.h", "gla_common.h", "gla_pblock.h",
            "gla_internal.h", "gla_api.hip", "build.py"} <= s
    assert not s & {"gla_bwd.hip", "gla_bwd_recur.hip", "gla_ggate.hip", "gla_recur.hip"}
    # the time-reversed and the local-state variants map to the same kernels
    assert names(bench.kernel_sources("chunk_prep_rev")) == s
    assert names(bench.kernel_sources("recur_local")) == names(bench.kernel_sources("chunk_recur"))
    assert "gla_recur.hip" in names(bench.kernel_sources("chunk_recur"))
    # launch names that differ from the kernel's name
    assert "gla_fwd.hip" in names(bench.kernel_sources("chunk_cumsum"))
    assert "gla_ggate.hip" in names(bench.kernel_sources("gg_recur_f32_r256"))
    assert "gla_bwd_recur.hip" in names(bench.kernel_sources("bwd_inter"))
    assert "gla_bwd.hip" in names(bench.kernel_sources("chunk_dqdk"))


def test_unknown_kernel_depends_on_every_source():
    assert bench.kernel_sources("no_such_kernel") == list(bench.KERNEL_SOURCES)


def test_every_listed_source_exists():
    for n in ("chunk_prep", "chunk_recur", "bwd_inter", "chunk_dqdk", "gg_prep", "decode"):
        for rel in bench.kernel_sources(n):
            assert os.path.isfile(os.path.join(ROOT, rel)), rel
