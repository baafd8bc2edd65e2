"""bench.py's one JSON line, as the harness parses it: run in this
process (no child process once the GPU is initialised) on the default
workload with few steps; and the refusal of more than one GPU (CPU)."""
import json
import sys

import pytest

import bench


def _main(capsys, monkeypatch, *argv):
    monkeypatch.setattr(sys, "argv", ["bench.py", *argv])
    bench.main()
    lines = [l for l in capsys.readouterr().out.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    return json.loads(lines[0])


def test_more_than_one_gpu_is_refused(capsys, monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code != 0
    assert "one GPU" in capsys.readouterr().err


@pytest.mark.gpu
def test_headline_line_keeps_the_contract(capsys, monkeypatch):
    r = _main(capsys, monkeypatch, "--steps", "3", "--warmup", "1", "--headline-only",
              "--no-cpu-baseline")
    assert r["metric"] == bench.METRIC and r["unit"] == "completion tokens/s"
    assert r["n_gpus"] == 1 and r["steps"] == 3 and r["warmup"] == 1
    assert r["higher_is_better"] is True and r["scaling"] == "weak"
    assert r["vs_baseline"] is None and r["dtype"] == "bf16"
    assert "synthetic" in r["data"]
    c = r["config"]
    assert c["workload"] == "qwen_b8g8c256" and (c["B"], c["G"], c["C"], c["V"]) == (8, 8, 256,
                                                                                     151936)
    # value: completion tokens (B*G*C) per second of the timed steps
    assert r["value"] == pytest.approx(8 * 8 * 256 / (r["ms_per_step"] / 1e3), rel=1e-9)
    f = r["roofline"]
    assert f["bound"] == "hbm" and f["unit"] == "GB/s" and f["peak"] == 8000.0
    assert f["achieved"] > 0 and f["frac"] == pytest.approx(f["achieved"] / f["peak"])
    # achieved: algorithmic bytes per launch over the row kernel's mean launch time
    assert f["achieved"] == pytest.approx(
        f["alg_bytes_per_launch"] / (f["kernel_ms"] / 1e3) / 1e9, rel=1e-9)
    assert f["kernel_ms"] <= r["ms_per_step"] * 1.05
    assert f["traffic"] is None or f["traffic"] > 0.99 * f["alg_bytes_per_launch"]
    assert "provenance" in r and r["provenance"]["device"]["arch"].startswith("gfx950")
