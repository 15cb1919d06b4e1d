"""Host logic of bench.py, on the CPU: the hash that ties the stored HBM
traffic figures to the kernel sources they were measured on, and the
single-GPU contract of the command line."""
import json
import os

import pytest

import bench


def _reader(files):
    return lambda rel: files[rel]


def _files():
    launch = ("struct Other {\n  int x;\n};\nstruct DecodeLaunch {\n  int a;\n};\n"
              "struct PrefillLaunch {\n  int b;\n};\n")
    return {bench.CSRC + "decode.hip": b"decode v1", bench.CSRC + "prefill_mfma.hip": b"prefill v1",
            bench.CSRC + "common.h": b"common v1", bench.API_CPP: b"host v1", bench.BUILD_PY: b"flags v1",
            bench.CSRC + "launch.h": launch.encode()}


def test_source_hash_follows_every_input_of_the_kernels():
    base = bench.source_sha("decode", read=_reader(_files()))
    for rel in (bench.CSRC + "decode.hip", bench.CSRC + "common.h", bench.API_CPP, bench.BUILD_PY):
        f = _files()
        f[rel] += b" changed"
        assert bench.source_sha("decode", read=_reader(f)) != base, rel
    # the launch struct the kernels compile against counts; other structs do not
    f = _files()
    f[bench.CSRC + "launch.h"] = f[bench.CSRC + "launch.h"].replace(b"int a;", b"int a, c;")
    assert bench.source_sha("decode", read=_reader(f)) != base
    f = _files()
    f[bench.CSRC + "launch.h"] = f[bench.CSRC + "launch.h"].replace(b"int x;", b"int x, y;")
    assert bench.source_sha("decode", read=_reader(f)) == base
    # comments and layout do not count
    f = _files()
    f[bench.CSRC + "decode.hip"] = b"// a note\ndecode   /* inline */ v1\n"
    assert bench.source_sha("decode", read=_reader(f)) == base
    # the prefill kernels' hash does not see the decode source
    f = _files()
    f[bench.CSRC + "decode.hip"] += b" changed"
    assert bench.source_sha("prefill", read=_reader(f)) == bench.source_sha("prefill", read=_reader(_files()))


def test_traffic_is_reported_only_for_the_sources_it_was_measured_on(monkeypatch):
    with open(os.path.join(bench.ROOT, "profiles", "traffic.json")) as fh:
        stored = json.load(fh)["workloads"]
    for w, entry in stored.items():
        kind = bench.WORKLOAD_KERNELS[w]
        monkeypatch.setattr(bench, "source_sha", lambda k, read=None, h=entry["source_sha256"]: h)
        assert bench.traffic(w) == entry["bytes_per_launch"], w
        monkeypatch.setattr(bench, "source_sha", lambda k, read=None: "0" * 64)
        assert bench.traffic(w) is None, w
        assert kind in bench.KERNEL_SOURCES
    assert bench.traffic("no-such-workload") is None


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_every_leg_is_known():
    for name in bench.LEGS:
        assert name in ("tiny", "padded32", "longctx70b", "verify8b", "prefill8k", "chunkprefill",
                        "chunkprefill_fp8", "cowcopy", "beamreorder", "stream")
    with pytest.raises(ValueError):
        bench.run_leg("no-such-leg", None, False)


def test_kernel_times_are_stored_figures_of_the_same_sources(monkeypatch):
    with open(os.path.join(bench.ROOT, "profiles", "traffic.json")) as fh:
        entry = json.load(fh)["workloads"]["decode8b"]
    monkeypatch.setattr(bench, "source_sha", lambda k, read=None: entry["source_sha256"])
    rec = bench.kernel_times("decode8b", 1e9, bench.HBM_PEAK_GBS, "GB/s")
    us = sum(entry["kernel_avg_us"].values())
    assert rec["us_per_call"] == pytest.approx(us)
    assert rec["achieved"] == pytest.approx(1.0 / (us * 1e-6))          # 1e9 bytes per call, in GB/s
    assert rec["frac"] == pytest.approx(rec["achieved"] / bench.HBM_PEAK_GBS)
    monkeypatch.setattr(bench, "source_sha", lambda k, read=None: "0" * 64)
    assert bench.kernel_times("decode8b", 1e9, bench.HBM_PEAK_GBS, "GB/s") is None
