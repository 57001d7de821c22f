"""Host-side checks of the seeded input generators (no method arithmetic)."""
import math

import pytest
import torch

from long_context_decode_s4r_amd import configs, synth


def test_deterministic_and_shapes():
    w = configs.TINY_F32
    a = synth.make_prompt(w)
    b = synth.make_prompt(w)
    assert a.K.shape == (1, 1024, 64) and a.K.dtype == torch.float32
    assert torch.equal(a.K, b.K) and torch.equal(a.V, b.V)
    assert not torch.equal(a.K, a.V)
    d = synth.make_decode_inputs(w, a, 3)
    assert d.q.shape == (3, 1, 1, 64) and d.k.shape == (3, 1, 1, 64)


def test_factor_model_rank_and_sinks():
    w = configs.TINY_F32.with_(noise=0.0)
    p = synth.make_prompt(w)
    X = p.K[0].double()
    sv = torch.linalg.svdvals(X[w.n_sink:])
    assert sv[w.factor_rank] < 1e-4 * sv[0]
    # sink rows scaled 10x relative to the same draw
    assert X[: w.n_sink].norm(dim=1).mean() > 5 * X[w.n_sink:].norm(dim=1).mean()


def test_power_spectrum_and_rms():
    s = synth.power_spectrum(1024, 0.8).double()
    assert abs(float((s * s).sum()) - 1024) < 1e-2
    assert float(s[0] / s[1]) == pytest.approx(2 ** 0.8, rel=1e-5)
    w = configs.LLAMA8B_32K
    p = synth.make_prompt(w, L=512, batch=1)
    rms = p.K.float().pow(2).mean().sqrt().item()
    assert 0.8 < rms < 1.2


def test_planted_positions():
    w = configs.LLAMA8B_128K
    L = 131072
    pos = synth.planted_positions(w, 0, L)
    assert len(pos) == math.floor(0.02 * L) == len(set(pos.tolist()))
    assert pos.min() >= L // 4 and pos.max() < 3 * L // 4
    assert not torch.equal(pos, synth.planted_positions(w, 1, L))


def test_qwen_exponents():
    w = configs.QWEN7B_64K
    assert w.exponent(0) == pytest.approx(0.5) and w.exponent(27) == pytest.approx(1.2)
    assert w.G == 7 and w.D == 512


def test_layer_slices_match_whole_model():
    """A layer generated on its own equals the same layer generated with the
    others (the 28-layer workload is built one layer at a time)."""
    w = configs.QWEN7B_64K
    a = synth.make_prompt(w, L=64, batch=2, n_layers=3)
    b = synth.make_prompt(w, L=64, batch=2, n_layers=1, first_layer=2)
    assert torch.equal(a.K[4:6], b.K) and torch.equal(a.V[4:6], b.V)
    da = synth.make_decode_inputs(w, a, 2, batch=2)
    db = synth.make_decode_inputs(w, b, 2, batch=2, first_layer=2)
    assert torch.equal(da.q[:, 4:6], db.q) and torch.equal(da.v[:, 4:6], db.v)
