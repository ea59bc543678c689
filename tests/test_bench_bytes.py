"""The benchmark's algorithmic-byte counts (the roofline's numerator), worked
out by hand on the hand-worked example of tests/golden/handworked.json:
T = 2 tables (3 rows x D 2, 2 rows x D 1), B = 2, fp32 weights,
indices [0, 2, 1, 1, 1, 0], offsets [0, 2, 4, 4, 6].

By hand: 6 lookups, 5 offsets; the batch touches table 0 rows {0, 1, 2}
(3 x 2 x 4 = 24 bytes) and table 1 rows {0, 1} (2 x 1 x 4 = 8 bytes), so 32
bytes of distinct rows and 5 runs; per lookup the rows read are 4 x 8 + 2 x 4
= 40 bytes; the output is 2 x 3 x 4 = 24 bytes; 5 rows in all need 3 key bits,
one radix pass.
"""
import json
import os

import numpy as np

import bench
from pooling_tbe_forward_amd import datagen as dg

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "handworked.json")))


def _problem(weighted):
    T, B = GOLD["T"], GOLD["B"]
    N = len(GOLD["indices"])
    return dg.Problem(name="gold", seed=0, T=T, B=B, rows=np.array(GOLD["rows"], np.int64),
                      dims=np.array(GOLD["dims"], np.int32), wdtype="f32", wdist=("explicit",),
                      weighted=np.full(T, weighted), lengths=np.diff(GOLD["offsets"]).reshape(T, B),
                      offsets=np.array(GOLD["offsets"], np.int64),
                      indices=np.array(GOLD["indices"], np.int64),
                      psw=np.ones(N, np.float32) if weighted else None,
                      grad=np.zeros((B, 3), np.float32), lr=0.5)


def test_unweighted_counts():
    b = bench.algorithmic_bytes(_problem(False))
    jag = 6 * 4 + 5 * 4                       # indices + offsets
    assert b["N"] == 6 and b["unique_rows"] == 5 and b["passes"] == 1
    assert b["fwd_min"] == jag + 32 + 24
    assert b["fwd_lookup"] == jag + 40 + 24
    # one pass moving (4-byte key + 4-byte sample id) in and out per lookup,
    # 16 bytes per run record
    assert b["bwd_min"] == jag + 24 + 2 * 32 + 6 * 8 * 2 + 5 * 16
    # segment kernel: rows read and written, grad_output once, the sorted
    # payload, the run records; Adagrad adds a 4-byte state read and write
    assert b["seg_min"] == 2 * 32 + 24 + 6 * 4 + 5 * 16
    assert b["seg_min_adagrad"] == b["seg_min"] + 5 * 8


def test_weighted_counts():
    b = bench.algorithmic_bytes(_problem(True))
    jag = 6 * 4 + 5 * 4 + 6 * 4               # + per-sample weights
    assert b["fwd_min"] == jag + 32 + 24
    # the payload is a (sample, weight) pair: 8 bytes
    assert b["bwd_min"] == jag + 24 + 2 * 32 + 6 * 12 * 2 + 5 * 16
    assert b["seg_min"] == 2 * 32 + 24 + 6 * 8 + 5 * 16


def test_traffic_keyed_to_source_and_tuning(tmp_path, monkeypatch):
    """A committed PMC summary counts only for the kernel source and the
    launch knobs it was taken with."""
    tun = dict(tau=64, chunk=256, seg_slab_kib=1024)
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "traffic_file", lambda w: str(path))
    rec = dict(source_sha256_16=bench.source_hash(bench.SEGMENT_SRC), tuning=tun,
               traffic_bytes=12345)
    path.write_text(json.dumps(rec))
    assert bench.measured_traffic("mixed", tun) == 12345
    assert bench.measured_traffic("mixed", dict(tun, tau=128)) is None
    path.write_text(json.dumps(dict(rec, source_sha256_16="0" * 16)))
    assert bench.measured_traffic("mixed", tun) is None
    path.write_text(json.dumps({k: v for k, v in rec.items() if k != "tuning"}))
    assert bench.measured_traffic("mixed", tun) is None


def test_source_hash_ignores_comments(tmp_path):
    a = tmp_path / "a.hip"
    a.write_text("// header\nint f(int x) { return x + 1; }  // inline\n\n/* block\n */\n")
    b = tmp_path / "b.hip"
    b.write_text("// other words\n\nint f(int x) { return x + 1; }\n")
    c = tmp_path / "c.hip"
    c.write_text("int f(int x) { return x + 2; }\n")
    assert bench.source_hash(str(a)) == bench.source_hash(str(b))
    assert bench.source_hash(str(a)) != bench.source_hash(str(c))
