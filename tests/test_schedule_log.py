"""JFA_LOG schedule statistics (host only): the line the library prints for a schedule
agrees with the schedule jfa_schedule returns (tile and program counts, the cost of
each segment computed here from the returned tiles)."""

import os
import re
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import json, sys
import numpy as np
from variable_length_flash_jagged_amd import binding as B
lengths = [700, 5, 0, 3000, 64, 1, 300]
off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
shape = B.make_shape(len(lengths), 3, 128, int(off[-1]), 0, 0)
out = []
for sched in (0, 1):
    tiles, seg, progs, rows = B.schedule(shape, B.MODE_SELF, B.PASS_BWD, off, B.make_opts(sched=sched, num_programs=16))
    out.append(dict(tiles=tiles.tolist(), seg=seg.tolist(), programs=progs, rows=rows))
sys.stderr.flush()
print(json.dumps(dict(lengths=lengths, runs=out)))
"""

LINE = re.compile(r"jfa schedule (?P<what>[^:]+): tiles (?P<tiles>\d+), programs (?P<programs>\d+), "
                  r"(?P<kind>counter groups|static segments) (?P<segs>\d+), tile rows (?P<rows>\d+), "
                  r"cost (?P<cost>\d+), per segment max (?P<max>\d+) mean (?P<mean>[\d.]+) \(max/mean (?P<ratio>[\d.]+)\)")


def _run(env_value):
    env = dict(os.environ, JFA_LOG=env_value)
    r = subprocess.run([sys.executable, "-c", CHILD], cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    import json
    return json.loads(r.stdout.strip().splitlines()[-1]), [m for m in map(LINE.search, r.stderr.splitlines()) if m]


def test_log_lines_match_returned_schedules():
    data, lines = _run("1")
    # each jfa_schedule call of the child builds its schedule twice (count query, fill)
    bwd = [m for m in lines if m["what"] == "self backward sorted zigzag"]
    assert len(bwd) == 4, [m.group(0) for m in lines]
    lengths = np.array(data["lengths"])
    for run, m in zip(data["runs"], bwd[::2]):
        tiles, seg = np.array(run["tiles"]), np.array(run["seg"])
        assert int(m["tiles"]) == len(tiles) and int(m["programs"]) == run["programs"]
        assert int(m["rows"]) == run["rows"]
        assert int(m["segs"]) == len(seg) - 1
        costs = [int(lengths[tiles[a:b, 0]].sum()) for a, b in zip(seg[:-1], seg[1:])]
        assert int(m["cost"]) == sum(costs) and int(m["max"]) == max(costs)
        assert abs(float(m["mean"]) - sum(costs) / len(costs)) <= 0.05
    assert bwd[0]["kind"] == "static segments" and bwd[2]["kind"] == "counter groups"


def test_no_lines_without_the_variable():
    _, lines = _run("0")
    assert lines == []
