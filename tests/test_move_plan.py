"""CPU emulation of the handed-over compaction protocol of kve_step_ws.

The kernels take every decision about a handed-over move -- whether a move is
handed over, its chunks, which rows the step parks, where each chunk reads
its sources, whether a pool reservation fits, how many items the move kernel
reads -- from kv_cache_eviction_step_amd/csrc/kve_move_plan.h.
``move_plan_emulation.cpp`` compiles that same header with g++ and runs the
protocol on the host: chunks in random orders and interleavings, many
caches sharing pools from one item to more than enough, and the pool's
header over tens of thousands of calls.  It checks that no chunk reads a row
another chunk writes, that every index stays in bounds, that the move kernel
reads only items this launch wrote, that every call starts on a zero counter
and every move workgroup reads that call's count, and that every cache ends
as keyformer_update step 3 leaves it (later rows one slot down, the incoming
row last).
"""
from __future__ import annotations

import os
import re
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "kv_cache_eviction_step_amd", "csrc")


def test_kernels_take_the_move_plan_from_the_shared_header():
    """The emulation proves something about the kernels only if they call the
    header's functions rather than restating its arithmetic."""
    src = open(os.path.join(CSRC, "kve_step.hip")).read()
    for fn in ("move_handed_over", "move_chunks", "parked_row", "chunk_first_dst",
               "move_last_dst", "chunk_source_row", "reservation_fits", "items_queued",
               "pool_counter", "pool_next_phase"):
        assert re.search(rf"\b{fn}\(", src), fn
    assert '#include "kve_move_plan.h"' in open(os.path.join(CSRC, "kve_step.h")).read()
    api = open(os.path.join(CSRC, "kve_api.hip")).read()
    assert "max_move_chunks(" in open(os.path.join(CSRC, "kve_move_plan.h")).read()
    assert "kve::max_move_chunks(" in api        # the workspace size of every move


def test_move_protocol_emulation(tmp_path):
    exe = str(tmp_path / "move_plan_emulation")
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-Wextra", "-Werror", "-I", CSRC,
                    os.path.join(HERE, "move_plan_emulation.cpp"), "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    m = re.search(r"ok: (\d+) handed-over moves, (\d+) pooled launches, (\d+) calls", r.stdout)
    assert m and int(m.group(1)) > 10_000 and int(m.group(2)) > 50 and int(m.group(3)) > 10_000, \
        r.stdout
