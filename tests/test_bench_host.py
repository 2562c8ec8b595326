"""Host-side pieces of bench.py that need no GPU: the shader-clock readout and
the algorithmic byte count the roofline fractions divide by."""
import importlib.util
import os

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_host", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_sclk_readout(tmp_path):
    b = _bench()
    for text, want in (("S: 125Mhz *\n0: 500Mhz\n1: 2400Mhz\n", 125.0),
                       ("S: 2177Mhz *\n0: 500Mhz\n1: 2400Mhz\n", 2177.0),
                       ("0: 500Mhz\n1: 2400Mhz *\n", 2400.0),
                       ("0: 500Mhz\n1: 2400Mhz\n", None)):
        p = tmp_path / "pp_dpm_sclk"
        p.write_text(text)
        assert b.read_sclk_mhz(str(p)) == want, text


def test_layer_bytes_qwen3_shape():
    """Per-stage algorithmic bytes of the Qwen3-30B-A3B-shaped layer at T = 4096
    with every expert used: quantized rows are C/2 + C/16 + 4 bytes."""
    b = _bench()
    T, H, E, K, I = 4096, 2048, 128, 8, 768
    by = b.layer_bytes(T, H, E, K, I, np.full(E, T * K // E))
    qh, qi = H // 2 + H // 16 + 4, I // 2 + I // 16 + 4
    assert (qh, qi) == (1156, 436)
    assert by["weights"] == E * (2 * I * qh + H * qi)
    P = T * K
    assert by["fc1"] == P * qh + E * 2 * I * qh + P * I * 2
    assert by["compulsory"] == by["weights"] + 2 * T * H * 2 + T * K * 8
    assert by["total"] == by["compulsory"] + 2 * (P * qh + P * I * 2 + P * qi + P * H * 2)
