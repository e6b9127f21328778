"""Host-side behaviour of bench.py (CPU only): one GPU only, and the counter-measured
HBM traffic is reported only while the kernel sources still hash the same."""
import hashlib
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT,
                          capture_output=True, text=True, env=e, timeout=120)


def test_more_than_one_gpu_exits_with_a_message():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_world_size_above_one_exits():
    r = _run([], env={"WORLD_SIZE": "2"})
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_help():
    r = _run(["--help"])
    assert r.returncode == 0 and "--no-parts-bench" in r.stdout


def test_traffic_only_while_sources_match(tmp_path):
    sys.path.insert(0, ROOT)
    import bench
    src = "long_context_exact_block_amd/csrc/elementwise.hip"
    h = hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest()
    rel = os.path.relpath(str(tmp_path / "t.json"), ROOT)
    with open(tmp_path / "t.json", "w") as f:
        json.dump({"kernel_sources_sha256": h, "hbm_bytes_per_launch": 123.0}, f)
    assert bench.traffic_from_profile([src], rel) == 123.0
    with open(tmp_path / "t.json", "w") as f:
        json.dump({"kernel_sources_sha256": "0" * 64, "hbm_bytes_per_launch": 123.0}, f)
    assert bench.traffic_from_profile([src], rel) is None
    assert bench.traffic_from_profile([src], rel + ".missing") is None


def test_committed_traffic_summaries_match_the_sources():
    """The committed counter summaries were taken on the current kernel sources."""
    sys.path.insert(0, ROOT)
    import bench
    for summary in ("profiles/attn_packed_1M_share_traffic.json", "profiles/merge_traffic.json"):
        prof = json.load(open(os.path.join(ROOT, summary)))
        assert bench.traffic_from_profile(prof["kernel_sources"], summary) == \
            prof["hbm_bytes_per_launch"], (
                "%s: the kernel sources changed since FETCH_SIZE / WRITE_SIZE were taken; "
                "re-take them with the commands the file lists" % summary)


def test_forwarded_bytes_counted_only_where_the_kernel_forwards():
    """The FORWARD hand-off writes blocks on from the block kernel only on hops the thin
    side copy cannot hide (the library's rule); only then do the launch's algorithmic bytes
    include the blocks it writes on (K and packed V of every sending rank, no hop after the
    last)."""
    sys.path.insert(0, ROOT)
    import bench
    from long_context_exact_block_amd import binding as rb
    from long_context_exact_block_amd import configs
    c5 = configs.SHORT_512
    assert bench.forwards_in_kernel(rb, c5, "forward")
    assert not bench.forwards_in_kernel(rb, c5, "copy")
    for w in (configs.SHARE_1M, configs.MHA_32K, configs.GQA_128K, configs.TINY):
        assert not bench.forwards_in_kernel(rb, w, "forward"), w.name
    fb = bench.hop_forward_bytes(c5)
    per_rank = c5.B * c5.Hkv * (c5.n * c5.d + c5.d * c5.n) * 2  # n = 512: no padding
    assert fb == [per_rank * c5.R] * (c5.R - 1) + [0]
    sub = configs.SHARE_1M  # one computed rank: it sends nothing in the kernel
    assert bench.hop_forward_bytes(sub) == [0] * sub.R
    assert bench.kernel_name(c5, True, True) == "attn_lean64_kernel<fp16> (forwarding)"
    assert bench.kernel_name(c5, False) == "attn_lean64_kernel<fp16, exact>"
    assert bench.kernel_name(configs.SHARE_1M) == "attn_packed_kernel<128,bf16>"
