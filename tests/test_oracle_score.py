"""Pins of the oracle's indexer score and cache layout.

The score reading (s(p) = sum_h w_h ReLU(q_h . k_{p,h}) in a fixed fp32 order) is pinned
by exact rational arithmetic (fractions.Fraction) on dequantised values:
* on inputs built so that every fp32 step is exact, the oracle must equal the exact value;
* on N(0,1) inputs it must lie within the fp32 rounding bound of the exact value;
* with one head and w = 1 it reduces to ReLU of a textbook dot product.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth_inputs as si
from harness import make_table

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _cfg(H, d):
    return oracle.cfg(H, d, 512, 16, 128, 4, 8, 1.0 / np.sqrt(512))


def _pack_keys(c, keys):
    """keys fp32 [L, H, d] -> oracle idx cache with an identity-free permuted table."""
    L = keys.shape[0]
    table, n_blocks = make_table([L], seed=L)
    kv, idx = oracle.alloc_caches(c, table, n_blocks)
    oracle.append_global(c, None, keys[None], table, np.array([0], np.int32), None, idx)
    return table, idx


def _exact_scores(qvals, kvals, w):
    """qvals [H, d], kvals [L, H, d] exact dequantised values (float64, exactly
    representable), w [H] float32 -> exact rational scores."""
    out = []
    for p in range(kvals.shape[0]):
        s = Fraction(0)
        for h in range(qvals.shape[0]):
            dot = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qvals[h], kvals[p, h]))
            s += Fraction(float(w[h])) * max(dot, Fraction(0))
        out.append(s)
    return out


def _grid_vectors(rng, shape, e_choices):
    """Values exactly on the E2M1 grid times 2^e, one 6*2^e element per 32-group so the
    quantiser picks exponent e and round-trips every value."""
    v = rng.choice(GRID, shape) * rng.choice([-1.0, 1.0], shape)
    flat = v.reshape(-1, 32)
    e = rng.choice(e_choices, flat.shape[0])
    flat[:, 0] = 6.0 * rng.choice([-1.0, 1.0], flat.shape[0])
    flat *= (2.0 ** e)[:, None]
    return flat.reshape(shape).astype(np.float32)


@pytest.mark.parametrize("H,d", [(1, 32), (2, 64), (4, 64), (8, 128)])
def test_score_exact_when_every_step_is_exact(H, d):
    rng = np.random.default_rng(H * 1000 + d)
    c = _cfg(H, d)
    L = 21
    # one common exponent per vector keeps every partial sum an exact fp32 integer multiple
    q = _grid_vectors(rng, (H, d), [-1])
    keys = _grid_vectors(rng, (L, H, d), [-2])
    w = rng.choice([0.25, 0.5, 1.0, 2.0], H).astype(np.float32)
    qc, qs = oracle.quantize_mxfp4(q.reshape(1, -1))
    assert np.array_equal(oracle.dequant_mxfp4(qc, qs)[0], q.reshape(-1).astype(np.float64))
    table, idx = _pack_keys(c, keys)
    s = oracle.index_scores(c, qc[0], qs[0], w, idx, table[0], L)
    exact = _exact_scores(q.astype(np.float64), keys.astype(np.float64), w)
    for p in range(L):
        assert Fraction(float(s[p])) == exact[p], p


@pytest.mark.parametrize("H,d,mixed", [(4, 64, False), (8, 128, False), (4, 64, True)])
def test_score_within_fp32_bound_on_normal_data(H, d, mixed):
    wl = si.small("score", 11 + H, [40], H_I=H, d_I=d)
    c = oracle.cfg_of(wl)
    keys = si.idx_keys(wl, 0)
    q = si.layer_idx_q(wl, 0)[0]
    w = si.layer_idx_w(wl, 0, mixed_sign=mixed)[0]
    qc, qs = oracle.quantize_mxfp4(q.reshape(1, -1))
    kc, ks = oracle.quantize_mxfp4(keys.reshape(40, -1))
    qv = oracle.dequant_mxfp4(qc, qs)[0].reshape(H, d)
    kvv = oracle.dequant_mxfp4(kc, ks).reshape(40, H, d)
    table, idx = _pack_keys(c, keys)
    s = oracle.index_scores(c, qc[0], qs[0], w, idx, table[0], 40)
    exact = _exact_scores(qv, kvv, w)
    for p in range(40):
        # per head: group sum rounds <= G-1 times, the fma chain rounds H times
        mag = sum(abs(float(w[h])) * max(0.0, float(np.dot(qv[h], kvv[p, h]))) for h in range(H))
        dmax = max(abs(float(np.dot(qv[h], kvv[p, h]))) for h in range(H))
        bound = (H + d // 32) * 2.0 ** -23 * (mag + sum(abs(w)) * dmax) + 1e-30
        assert abs(float(s[p]) - float(exact[p])) <= bound, p


def test_single_head_unit_weight_is_relu_of_dot():
    wl = si.small("dot", 5, [64], H_I=1, d_I=64)
    c = oracle.cfg_of(wl)
    keys = si.idx_keys(wl, 0)
    q = si.layer_idx_q(wl, 0)[0]
    qc, qs = oracle.quantize_mxfp4(q.reshape(1, -1))
    kc, ks = oracle.quantize_mxfp4(keys.reshape(64, -1))
    qv = oracle.dequant_mxfp4(qc, qs)[0]
    kvv = oracle.dequant_mxfp4(kc, ks)
    table, idx = _pack_keys(c, keys)
    s = oracle.index_scores(c, qc[0], qs[0], np.ones(1, np.float32), idx, table[0], 64)
    ref = np.maximum(kvv @ qv, 0.0)  # fp64 textbook dot; 2 groups -> one fp32 rounding
    assert np.all(np.abs(s - ref) <= 2.0 ** -24 * np.abs(ref) + 1e-30)
    assert np.all(s[ref == 0] == 0) and np.any(ref == 0) and np.any(ref > 0)


def test_score_never_negative_zero_and_sign_of_weights():
    rng = np.random.default_rng(3)
    c = _cfg(2, 64)
    q = _grid_vectors(rng, (2, 64), [0])
    keys = np.stack([q, -q, np.zeros_like(q)])  # dot > 0, dot < 0, dot = 0
    qc, qs = oracle.quantize_mxfp4(q.reshape(1, -1))
    table, idx = _pack_keys(c, keys.astype(np.float32))
    w = np.array([-1.0, 0.5], np.float32)
    s = oracle.index_scores(c, qc[0], qs[0], w, idx, table[0], 3)
    d0 = sum(float(x) ** 2 for x in q[0].astype(np.float64))
    d1 = sum(float(x) ** 2 for x in q[1].astype(np.float64))
    assert s[0] == np.float32(-d0 + 0.5 * d1)
    for p in (1, 2):  # ReLU gives +0 and the fma chain keeps +0
        assert s[p] == 0.0 and not np.signbit(s[p])


def test_index_key_block_layout_offsets():
    # H = 2, d = 64 (G = 2): block = 8 * 2 * 32 code bytes + 8 * 2 * 2 scale bytes = 544
    c = _cfg(2, 64)
    assert oracle.idx_block_bytes(c) == 544
    keys = np.zeros((8, 2, 64), np.float32)
    keys[3, 1, 32] = 6.0        # slot 3, head 1, group 1, element 0 -> code 7, scale 127
    keys[3, 1, 33] = -0.5 * 1   # element 1 -> -0.5 -> code 0x9
    keys[3, 1, 63] = 1.0        # element 31 -> code 2 in the high nibble of byte 15
    table = np.array([[0]], np.int32)
    kv, idx = oracle.alloc_caches(c, table, 1)
    oracle.append_global(c, None, keys[None], table, np.array([0], np.int32), None, idx)
    blk = idx[0]
    off = ((1 * 8 + 3) * 2 + 1) * 16        # ((g*8 + s)*H + h) * 16
    assert blk[off] == 0x97 and blk[off + 15] == 0x20
    assert blk[512 + (3 * 2 + 1) * 2 + 1] == 127
    # every other code byte is zero and every other scale byte is code 0 (zero groups)
    mask = np.ones(544, bool)
    mask[[off, off + 15, 512 + 15]] = False
    assert not blk[mask].any()


def test_main_kv_and_window_layouts():
    c = _cfg(1, 32)
    lat = np.zeros((1, 10, 512), np.float32)
    lat[0, 9, 2] = 6.0            # position 9 -> block 1, slot 1
    table = np.array([[1, 0]], np.int32)   # logical block 1 in physical block 0
    kv, idx = oracle.alloc_caches(c, table, 2)
    oracle.append_global(c, lat, np.zeros((1, 10, 1, 32), np.float32), table,
                         np.array([0], np.int32), kv, idx)
    row = 272
    assert kv.shape == (2, 8 * row)
    assert kv[0, 1 * row + 1] == 0x07 and kv[0, 1 * row + 256] == 127
    swa = oracle.alloc_swa(c, 1, 4)
    rows = np.zeros((1, 2, 512), np.float32)
    rows[0, 1, 0] = 448.0
    oracle.append_swa(c, rows, np.array([6], np.int32), swa, 4)   # positions 6, 7 -> slots 2, 3
    assert swa[0, 3, 0] == 0x7E and swa[0, 3, 512] == 127 and not swa[0, 2].any()
