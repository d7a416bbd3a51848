"""bench.py's parity gate (host logic, no GPU): fed the oracle's own step it
passes; one wrong code byte, or an h or y output off by more than the bar,
each make it fail."""
import numpy as np

import bench
import oracle
import workloads as wl


def _step():
    g = wl.rng(wl.SEEDS["ffn_up"])
    w_up = wl.q4k_weights(*bench.UP, g)
    x = wl.activations(1, bench.UP[1], g)
    w_dn = wl.q4k_weights(*bench.DOWN, wl.rng(wl.SEEDS["ffn_down"]))
    o = oracle.default()
    xq_x = o.quantize_q8k(x)
    h, Th = o.gemv_q4k(w_up, xq_x, *bench.UP)
    xq_h = o.quantize_q8k(h.astype(np.float32).reshape(1, -1))
    y, Ty = o.gemv_q4k(w_dn, xq_h, *bench.DOWN)
    fp = {"xq_x": xq_x.copy(), "h": h.astype(np.float64), "xq_h": xq_h.copy(),
          "y": y.astype(np.float64)}
    return o, x, w_up, w_dn, fp, Th, Ty


def test_bench_parity_gate():
    o, x, w_up, w_dn, fp, Th, Ty = _step()
    assert bench._parity_gate(o, x, w_up, w_dn, fp)["passed"]

    bad = dict(fp, xq_x=fp["xq_x"].copy())
    bad["xq_x"].reshape(-1)[5] ^= 1
    r = bench._parity_gate(o, x, w_up, w_dn, bad)
    assert not r["passed"] and not r["q8k_x_bytes"]

    i = int(np.argmax(Th))
    bad = dict(fp, h=fp["h"].copy())
    bad["h"][i] += 1e-4 * Th[i]
    r = bench._parity_gate(o, x, w_up, w_dn, bad)
    assert not r["passed"] and not r["h"]

    j = int(np.argmax(Ty))
    bad = dict(fp, y=fp["y"].copy())
    bad["y"][j] += 2e-5 * Ty[j]
    r = bench._parity_gate(o, x, w_up, w_dn, bad)
    assert not r["passed"] and not r["y"]


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
