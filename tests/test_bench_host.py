"""Host-side logic of bench.py and the block-flag generator (no GPU)."""
import numpy as np

import bench
import synth


def test_attended_pairs_against_brute_force():
    for N, blk, causal in ((300, 64, True), (300, 64, False), (777, 96, True), (128, 32, True), (65, 64, True)):
        bm = synth.block_mask(2, 2, N, blk, 3, "random", 0.4)
        tot = 0
        for b in range(2):
            for h in range(2):
                f = np.repeat(np.repeat(bm[b, h], blk, 0), blk, 1)[:N, :N].astype(bool)
                if causal:
                    f &= np.tril(np.ones((N, N), bool))
                tot += int(f.sum())
        assert bench.attended_pairs(bm, N, blk, causal) == tot, (N, blk, causal)


def test_block_mask_patterns():
    bm = synth.block_mask(1, 2, 1000, 64, 1, "local_global", band=2, n_global=1)
    assert bm.shape == (1, 2, 16, 16) and bm.dtype == np.uint8
    i, j = np.indices((16, 16))
    want = ((np.abs(i - j) <= 2) | (i < 1) | (j < 1)).astype(np.uint8)
    assert np.array_equal(bm[0, 0], want) and np.array_equal(bm[0, 1], want)
    r1 = synth.block_mask(2, 3, 500, 32, 7, "random", 0.3)
    r2 = synth.block_mask(2, 3, 500, 32, 7, "random", 0.3)
    assert np.array_equal(r1, r2) and r1.shape == (2, 3, 16, 16)
    assert 0.2 < r1.mean() < 0.4


def test_environment_record_keys():
    """The env object of a bench line names the GPU, its architecture and the
    software versions; checked with stand-ins for torch and the library."""
    import types

    props = types.SimpleNamespace(name="gpu-name", gcnArchName="gfx950:sramecc+:xnack-")
    torch = types.SimpleNamespace(
        __version__="9.9", version=types.SimpleNamespace(hip="7.0"),
        cuda=types.SimpleNamespace(get_device_properties=lambda i: props))
    A = types.SimpleNamespace(lib=lambda: types.SimpleNamespace(attn_version=lambda: 100))
    env = bench.environment(torch, A)
    assert env["gpu"] == "gpu-name" and env["arch"].startswith("gfx950")
    assert env["hip_runtime"] == "7.0" and env["torch"] == "9.9" and env["libattn_version"] == 100
    assert "rocm" in env and env["dropout"] is None
    assert "host_cpu" in env and env["host_threads"] >= 1


def test_traffic_record_follows_its_sources(tmp_path, monkeypatch):
    """A counter record is used only while the sources it names are unchanged;
    records without a source list are tied to the forward kernel's source."""
    import json

    csrc = tmp_path / "tiled_online_softmax_fwd_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    for f in bench.KERNEL_SOURCES:
        (csrc / f).write_text(f"{f} v1")
    (csrc / "decode.hip").write_text("decode v1")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    recs = {"fwd": {"kernel_hash": bench.kernel_hash(), "hbm_bytes_per_launch": 1.0},
            "dec": {"kernel_hash": bench.kernel_hash(["decode.hip"]), "sources": ["decode.hip"],
                    "hbm_bytes_per_launch": 2.0}}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(recs))
    assert bench.traffic_record("fwd")["hbm_bytes_per_launch"] == 1.0
    assert bench.traffic_record("dec")["hbm_bytes_per_launch"] == 2.0
    assert bench.traffic_record("missing") is None
    for f in bench.KERNEL_SOURCES:     # a change to any default source drops the record
        (csrc / f).write_text(f"{f} v2")
        assert bench.traffic_record("fwd") is None
        (csrc / f).write_text(f"{f} v1")
        assert bench.traffic_record("fwd")["hbm_bytes_per_launch"] == 1.0
    (csrc / "fwd_kernel.h").write_text("forward v2")
    assert bench.traffic_record("fwd") is None
    assert bench.traffic_record("dec")["hbm_bytes_per_launch"] == 2.0
    (csrc / "decode.hip").write_text("decode v2")
    assert bench.traffic_record("dec") is None


def test_committed_traffic_records_are_complete():
    """Every committed counter record carries what the bench and its summary
    need: the kernel, both counters, both calibration factors and the bytes."""
    import json
    import os

    with open(os.path.join(bench.ROOT, "profiles", "traffic.json")) as f:
        recs = json.load(f)
    assert recs
    for key, r in recs.items():
        for field in ("kernel", "kernel_hash", "fetch_kib", "write_kib", "fetch_scale", "write_scale",
                      "hbm_bytes_per_launch", "summary"):
            assert field in r, (key, field)
        want = (r["fetch_kib"] * r["fetch_scale"] + r["write_kib"] * r["write_scale"]) * 1024
        assert abs(r["hbm_bytes_per_launch"] - want) <= 1e-6 * want, key
        assert os.path.exists(os.path.join(bench.ROOT, "profiles", r["summary"])), key
