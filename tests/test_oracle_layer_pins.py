"""Pins of the decoder-layer oracle (oracle/layer.py) to closed forms, invariants, a library
rounding routine and the already pinned attention oracle; CPU only."""
import numpy as np
import pytest
import torch

from oracle import layer as lo
from oracle import oracle as orc


# ------------------------------------------------------------------------------ bf16

def test_bf16_round_hand_values():
    ulp = 2.0 ** -7  # bf16 spacing in [1, 2)
    assert lo.bf16_round(1.0) == 1.0
    assert lo.bf16_round(1 + ulp / 2) == 1.0                 # tie, even neighbour below
    assert lo.bf16_round(1 + 3 * ulp / 2) == 1 + 2 * ulp     # tie, even neighbour above
    assert lo.bf16_round(1 + 0.6 * ulp) == 1 + ulp
    assert lo.bf16_round(-3.0) == -3.0
    assert lo.bf16_round(0.0) == 0.0


def test_bf16_round_matches_torch_conversion():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.normal(size=4000) * 10.0 ** rng.integers(-8, 8, size=4000),
                        [1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 65504.0, 1e-30]])
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(lo.bf16_round(x), ref)


# ------------------------------------------------------------------------ rmsnorm, silu

def test_rmsnorm_closed_forms():
    g = np.linspace(0.5, 2.0, 16)
    for c in (3.0, -0.25):
        y = lo.rmsnorm(np.full(16, c), g, eps=0.0)
        assert np.allclose(y, np.sign(c) * g, rtol=0, atol=1e-15)
        y = lo.rmsnorm(np.full(16, c), g, eps=1e-2)
        assert np.allclose(y, c / np.sqrt(c * c + 1e-2) * g, rtol=1e-15)
    x = np.random.default_rng(1).normal(size=(3, 64))
    y = lo.rmsnorm(x, np.ones(64), eps=0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, atol=1e-14)  # unit RMS
    assert np.allclose(lo.rmsnorm(7.5 * x, np.ones(64), 0.0), y, atol=1e-14)  # scale invariant


def test_silu_closed_forms():
    assert lo.silu(0.0) == 0.0
    assert np.isclose(lo.silu(1.0), 0.7310585786300049, rtol=1e-15)   # 1 / (1 + e^-1)
    assert np.isclose(lo.silu(-1.0), -0.2689414213699951, rtol=1e-15)  # -1 / (1 + e)
    assert np.isclose(lo.silu(50.0), 50.0, rtol=1e-15)
    big_neg = lo.silu(-800.0)
    assert big_neg == 0.0 and not np.isnan(big_neg)


# ---------------------------------------------------------------------------- the layer

def _weights(rng, dm, Hq, Hkv, d, f, std=0.05):
    r = lambda *shape: lo.bf16_round(rng.normal(size=shape) * std)
    return lo.LayerWeights(g_attn=lo.bf16_round(1 + 0.1 * rng.normal(size=dm)), w_qkv=r((Hq + 2 * Hkv) * d, dm),
                           w_o=r(dm, Hq * d), g_mlp=lo.bf16_round(1 + 0.1 * rng.normal(size=dm)),
                           w_gate_up=r(2 * f, dm), w_down=r(dm, f))


def test_layer_with_zero_output_projections_leaves_x_and_appends_kv():
    rng = np.random.default_rng(2)
    dm, Hq, Hkv, d, f = 32, 4, 2, 8, 48
    wts = _weights(rng, dm, Hq, Hkv, d, f)
    wts.w_o[:] = 0.0
    wts.w_down[:] = 0.0
    x = rng.normal(size=(2, dm))
    hist = [lo.History(), lo.History()]
    y = lo.layer_step(x, wts, hist, [5, 9], Hq, Hkv, d, w=4, s=1, scale=0.3, conv=0, eps=1e-5)
    assert np.array_equal(y, x)
    h = lo.bf16_round(lo.rmsnorm(x, wts.g_attn, 1e-5))
    kv = lo.bf16_round(h @ wts.w_qkv[Hq * d:].T)
    for b, p in enumerate([5, 9]):
        assert hist[b].pos == [p]
        assert np.array_equal(hist[b].k[0].reshape(-1), kv[b, :Hkv * d])
        assert np.array_equal(hist[b].v[0].reshape(-1), kv[b, Hkv * d:])


@pytest.mark.parametrize("w,s", [(3, 0), (3, 2), (64, 0)])
def test_layer_zero_keys_give_mean_of_allowed_values(w, s):
    """k = 0 makes every allowed weight equal, so the attention output is the plain mean of
    the values at the allowed positions: x1 - x = bf16(mean_{j in A(t)} v_j) with W_o = I."""
    rng = np.random.default_rng(3)
    Hq = Hkv = 1
    d = dm = 16
    wts = _weights(rng, dm, Hq, Hkv, d, f=8)
    wts.w_qkv[d:2 * d] = 0.0                    # keys
    wts.w_qkv[2 * d:] = np.eye(d)               # values = h
    wts.w_o[:] = np.eye(dm)
    wts.w_down[:] = 0.0
    hist = [lo.History()]
    vs = []
    for t in range(9):
        x = rng.normal(size=(1, dm))
        y = lo.layer_step(x, wts, hist, [t], Hq, Hkv, d, w, s, scale=0.5, conv=0, eps=1e-6)
        vs.append(lo.bf16_round(lo.rmsnorm(x, wts.g_attn, 1e-6))[0])
        keep = [j for j in range(t + 1) if j > t - w or j < s]
        assert np.allclose(y - x, lo.bf16_round(np.mean([vs[j] for j in keep], axis=0)), rtol=0, atol=1e-12)


def test_layer_mlp_gate_up_order_and_silu():
    """W_o = 0, gate rows = 1000 I, up rows = I, W_down = I: for h2 > 0, silu(1000 h2) = 1000 h2 up
    to e^-1000, so x2 - x = bf16(1000 h2^2); for h2 < 0 the gate is ~0 and so is the update.
    Swapping gate and up rows would give silu(h2) * 1000 h2 instead."""
    rng = np.random.default_rng(4)
    dm = f = 16
    Hq = Hkv = 1
    d = 4
    wts = _weights(rng, dm, Hq, Hkv, d, f)
    wts.w_o[:] = 0.0
    wts.w_gate_up[:f] = 1000.0 * np.eye(f)
    wts.w_gate_up[f:] = np.eye(f)
    wts.w_down[:] = np.eye(dm)
    x = rng.normal(size=(1, dm))
    y = lo.layer_step(x, wts, [lo.History()], [0], Hq, Hkv, d, w=2, s=0, scale=1.0, conv=0, eps=1e-6)
    h2 = lo.bf16_round(lo.rmsnorm(x, wts.g_mlp, 1e-6))[0]
    want = np.where(h2 > 0, lo.bf16_round(1000.0 * h2 * h2), 0.0)
    assert np.allclose((y - x)[0], want, rtol=0, atol=1e-9)


def test_layer_is_invariant_to_the_scale_of_x():
    """With eps = 0 both norms remove the scale of x, so the update x' - x does not change
    when x is multiplied by a constant (a missing or misplaced norm breaks this)."""
    rng = np.random.default_rng(6)
    dm, Hq, Hkv, d, f = 32, 4, 2, 8, 40
    wts = _weights(rng, dm, Hq, Hkv, d, f)
    wts.w_o[:] = 0.0  # the second norm then sees c x exactly
    x = rng.normal(size=(1, dm))
    d1 = lo.layer_step(x, wts, [lo.History()], [0], Hq, Hkv, d, 4, 1, 0.3, 0, 0.0) - x
    d2 = lo.layer_step(8.0 * x, wts, [lo.History()], [0], Hq, Hkv, d, 4, 1, 0.3, 0, 0.0) - 8.0 * x
    assert np.allclose(d1, d2, rtol=0, atol=1e-12)


def test_layer_attention_over_steps_equals_prefill_rows():
    """W_o = I and W_down = 0: the update of step t is bf16 of the SWA(w,s) prefill row t of the
    q, k, v sequences the steps produced (the prefill oracle is pinned on its own)."""
    rng = np.random.default_rng(7)
    Hq, Hkv, d = 4, 2, 8
    dm = Hq * d
    w, s, T = 5, 2, 14
    wts = _weights(rng, dm, Hq, Hkv, d, f=24, std=0.3)
    wts.w_o[:] = np.eye(dm)
    wts.w_down[:] = 0.0
    hist = [lo.History()]
    xs, ups, qs = [], [], []
    for t in range(T):
        x = rng.normal(size=(1, dm))
        y = lo.layer_step(x, wts, hist, [t], Hq, Hkv, d, w, s, scale=0.4, conv=0, eps=1e-5)
        h = lo.bf16_round(lo.rmsnorm(x, wts.g_attn, 1e-5))
        qs.append(lo.bf16_round(h @ wts.w_qkv[:Hq * d].T).reshape(Hq, d))
        ups.append((y - x)[0])
    q = np.stack(qs)[None]
    k = np.stack(hist[0].k)[None]
    v = np.stack(hist[0].v)[None]
    ref = orc.prefill(q, k, v, w, s, 0.4, 0)[0].reshape(T, dm)
    assert np.allclose(np.stack(ups), lo.bf16_round(ref), rtol=0, atol=1e-12)


def test_layer_mlp_sees_the_residual_after_attention():
    """One step at t = 0 with zero keys and identity values attends to itself: the attention
    update is bf16(h).  The MLP (gate 1000 I, up I, down I) must then normalise x1 = x + bf16(h),
    not x."""
    rng = np.random.default_rng(8)
    Hq = Hkv = 1
    d = dm = f = 16
    wts = _weights(rng, dm, Hq, Hkv, d, f)
    wts.w_qkv[d:2 * d] = 0.0
    wts.w_qkv[2 * d:] = np.eye(d)
    wts.w_o[:] = np.eye(dm)
    wts.w_gate_up[:f] = 1000.0 * np.eye(f)
    wts.w_gate_up[f:] = np.eye(f)
    wts.w_down[:] = np.eye(dm)
    x = rng.normal(size=(1, dm))
    y = lo.layer_step(x, wts, [lo.History()], [0], Hq, Hkv, d, w=3, s=0, scale=1.0, conv=0, eps=1e-6)[0]
    h = lo.bf16_round(lo.rmsnorm(x, wts.g_attn, 1e-6))[0]
    x1 = x[0] + lo.bf16_round(h)
    h2 = lo.bf16_round(lo.rmsnorm(x1, wts.g_mlp, 1e-6))
    want = x1 + np.where(h2 > 0, lo.bf16_round(1000.0 * h2 * h2), 0.0)
    assert np.allclose(y, want, rtol=0, atol=1e-9)
