"""Pins of the CPU oracle against things other than itself (CPU only).

Each test ties one oracle function to a closed form, a library routine, exact
rational arithmetic or brute force, chosen so that a plausible slip (wrong
bias, wrong tie rule, a dropped scale, a transposed operand, a wrong nibble
order) fails at least one of them.
"""
from __future__ import annotations

import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from exact_ref import (E4M3_POS, best_pair, bf16_value, decode_exact, f32_round, nearest_e4m3,
                       quantize_exact)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32(x):
    return struct.unpack("<f", struct.pack("<f", x))[0]


# ------------------------------------------------------------ e4m3 decode ---

def test_decode_golden_points():
    with open(os.path.join(GOLDEN, "e4m3_points.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(rows) >= 10
    for code, val in rows:
        got = oracle.e4m3_decode(int(code, 16))
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val))


def test_decode_all_codes_vs_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_decode_table()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(got[~nan], ref[~nan])


def test_decode_vs_exact_table():
    for code, val in E4M3_POS:
        assert Fraction(oracle.e4m3_decode(code)) == val
        assert Fraction(oracle.e4m3_decode(code | 0x80)) == -val


# ------------------------------------------------------------ e4m3 encode ---

def test_encode_roundtrip_all_codes():
    for c in range(256):
        v = oracle.e4m3_decode(c)
        e = oracle.e4m3_encode(v)
        if c in (0x7F, 0xFF):
            assert e in (0x7F, 0xFF)
        else:
            assert e == c, (hex(c), v, hex(e))


def test_encode_saturation_and_specials():
    assert oracle.e4m3_encode(448.0) == 0x7E
    assert oracle.e4m3_encode(449.0) == 0x7E
    assert oracle.e4m3_encode(1e30) == 0x7E
    assert oracle.e4m3_encode(math.inf) == 0x7E
    assert oracle.e4m3_encode(-math.inf) == 0xFE
    assert oracle.e4m3_encode(-500.0) == 0xFE
    assert oracle.e4m3_encode(math.nan) in (0x7F, 0xFF)
    assert oracle.e4m3_encode(0.0) == 0x00
    assert oracle.e4m3_encode(-0.0) == 0x80
    assert oracle.e4m3_encode(-1e-30) == 0x80          # negative underflow keeps the sign
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00      # tie between 0 and 2^-9 -> even (0)
    assert oracle.e4m3_encode(3 * 2.0 ** -10) == 0x02  # tie between codes 1 and 2 -> 2
    assert oracle.e4m3_encode(432.0) == 0x7E           # tie 416 / 448 -> 0x7E (even)
    assert oracle.e4m3_encode(f32(432.0 - 2 ** -15)) == 0x7D


def test_encode_all_bf16_vs_torch_cast():
    """Every bf16 value with |v| <= 448: torch's RNE cast is an independent encoder."""
    bits = np.arange(65536, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    ok = np.isfinite(vals) & (np.abs(vals) <= 448)
    v = vals[ok]
    ref = torch.from_numpy(v.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_encode_array(v.astype(np.float64))
    assert np.array_equal(got, ref)
    # above 448 torch does not saturate; the rule is saturation
    big = vals[np.isfinite(vals) & (np.abs(vals) > 448)]
    got_big = oracle.e4m3_encode_array(big.astype(np.float64))
    assert np.array_equal(got_big, np.where(big > 0, 0x7E, 0xFE).astype(np.uint8))


def test_encode_near_midpoints_vs_brute_force():
    """fp32 values at and one ulp around every midpoint: exhaustive nearest search."""
    vals = [v for _, v in E4M3_POS]
    cases = []
    for lo, hi in zip(vals[:-1], vals[1:]):
        mid = float((lo + hi) / 2)
        cases += [mid, float(np.nextafter(np.float32(mid), np.float32(0))),
                  float(np.nextafter(np.float32(mid), np.float32(1000)))]
    for v in cases:
        for sgn in (1.0, -1.0):
            want = nearest_e4m3(Fraction(v), negative=sgn < 0)
            assert oracle.e4m3_encode(sgn * v) == want, (v, sgn)


def test_encode_random_fp32_vs_torch():
    rng = np.random.default_rng(7)
    v = (rng.standard_normal(200000) * np.exp(rng.uniform(-14, 6.2, 200000))).astype(np.float32)
    v = v[np.abs(v) <= 448]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_encode_array(v.astype(np.float64))
    assert np.array_equal(got, ref)


# ------------------------------------------------- activation quantization ---

def _bf16_bits(vals):
    return si.to_bf16_bits(torch.tensor(np.asarray(vals, dtype=np.float32)))


def test_quant_act_exact_small():
    """Whole-path check on a small X with crafted groups, against exact arithmetic."""
    rng = np.random.default_rng(11)
    M, K = 5, 384
    x = rng.standard_normal((M, K)).astype(np.float32) * np.exp(rng.uniform(-3, 3, (M, 1))).astype(np.float32)
    x[1, 128:256] = 0.0                                   # all-zero group
    x[1, 130] = -0.0
    x[2, 0:128] = rng.standard_normal(128).astype(np.float32) * 1e-39  # bf16 subnormals
    x[3, 256:384] = 1e20 * rng.standard_normal(128).astype(np.float32)
    xb = _bf16_bits(x)
    q, s = oracle.quant_act(xb)
    for m in range(M):
        for kb in range(K // 128):
            g = [bf16_value(int(b)) for b in xb[m, kb * 128:(kb + 1) * 128]]
            s_ref, codes = quantize_exact(g)
            assert s[m, kb] == np.float32(s_ref), (m, kb)
            assert q[m, kb * 128:(kb + 1) * 128].tolist() == codes, (m, kb)
    assert s[1, 1] == 0.0 and q[1, 130] == 0x80
    assert 0 < s[2, 0] < np.finfo(np.float32).tiny   # subnormal fp32 scale


def _nearest_code_of_quotient(x: Fraction, s: Fraction, negative: bool) -> int:
    """E4M3 code nearest to the exact quotient x / s (one rounding, ties to the even
    code, saturating): bisection over the 127 non-negative values, then an exact
    comparison with the midpoint of the two neighbours."""
    a = abs(x) / s
    sign = 0x80 if negative else 0x00
    if a >= 448:
        return sign | 0x7E
    lo, hi = 0, len(E4M3_POS) - 1          # E4M3_POS is sorted by value
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if E4M3_POS[mid][1] <= a:
            lo = mid
        else:
            hi = mid
    (c0, v0), (c1, v1) = E4M3_POS[lo], E4M3_POS[hi]
    d0, d1 = a - v0, v1 - a
    if d0 < d1 or (d0 == d1 and c0 % 2 == 0):
        return sign | c0
    return sign | c1


def test_quant_act_codes_round_the_fp32_quotient_not_the_exact_one():
    """Which quotient the codes round.  The codes are enc(fl32(x / s)): the IEEE fp32
    quotient, then one rounding to e4m3.  That is the exact quotient rounded once
    except where fl32(x / s) lands exactly on an e4m3 rounding midpoint while the
    exact quotient lies off it (a double rounding: x has 8 significant bits and s 24,
    so x / s can sit within 2^-25 of a midpoint).  Checked with exact rational
    arithmetic on random bf16 groups with maxima from 2^-120 to 2^120, and on crafted
    groups whose quotients sit within a few fp32 ulps of midpoints: every code equals
    the rounding of the correctly rounded fp32 quotient, and every code that differs
    from the single rounding of the exact quotient is such a double-rounding case."""
    rng = np.random.default_rng(23)
    mids = [(E4M3_POS[i][1] + E4M3_POS[i + 1][1]) / 2 for i in range(len(E4M3_POS) - 1)]
    mid_set = set(mids)
    groups = []
    for _ in range(96):                                # random groups
        g = rng.standard_normal(128) * 2.0 ** rng.uniform(-120, 120)
        groups.append(g.astype(np.float32))
    for _ in range(160):                               # crafted: quotients next to midpoints
        amax = np.float32(2.0 ** rng.uniform(-60, 60))
        s32 = np.float32(amax / np.float32(448))
        picks = rng.choice(len(mids), 127)
        x = np.array([float(mids[i]) * float(s32) for i in picks]) * (1 + rng.integers(-4, 5, 127) * 2.0 ** -9)
        x = np.clip(x, -float(amax), float(amax)) * rng.choice([-1.0, 1.0], 127)
        groups.append(np.concatenate([[amax], x]).astype(np.float32))
    xb = _bf16_bits(np.stack(groups))                  # [groups, 128] bf16, one group per row
    q, s = oracle.quant_act(xb)
    near = double_rounded = 0
    for r in range(xb.shape[0]):
        sr = Fraction(float(s[r, 0]))
        assert sr == f32_round(Fraction(max(abs(bf16_value(int(b))) for b in xb[r])) / 448)
        for k in range(128):
            xv = bf16_value(int(xb[r, k]))
            if xv == 0.0 or sr == 0:
                continue
            exact = Fraction(xv) / sr
            q32 = Fraction(f32_round(exact))
            assert q[r, k] == _nearest_code_of_quotient(q32, Fraction(1), xv < 0), (r, k, xv, float(sr))
            once = _nearest_code_of_quotient(exact, Fraction(1), xv < 0)
            if q[r, k] != once:
                assert abs(q32) in mid_set and abs(q32) != abs(exact), (r, k, xv, float(sr))
                double_rounded += 1
            a, c = abs(exact), once & 0x7F
            near += any(abs(a - m) <= m * Fraction(1, 2 ** 20) for m in mids[max(0, c - 1):c + 1])
    assert near > 300             # the crafted groups do reach the midpoints
    assert double_rounded > 0     # and the two readings do differ there


def test_quant_act_division_is_not_reciprocal():
    """Codes follow x/s, which differs from x*(448/amax) in rare cases."""
    xb = si.activations(64, 4096, outliers=False)
    q, s = oracle.quant_act(xb)
    x = si.bf16_bits_to_f32(xb).reshape(64, 32, 128)
    amax = np.abs(x).max(axis=2, keepdims=True)
    recip = (np.float32(448) / amax).astype(np.float32)
    alt = torch.from_numpy((x * recip).astype(np.float32).reshape(64, 4096)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    div = torch.from_numpy((x / s.reshape(64, 32, 1)).astype(np.float32).reshape(64, 4096)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, div)
    assert not np.array_equal(q, alt)


def test_quant_act_invariants():
    xb = si.activations(32, 4096)
    q, s = oracle.quant_act(xb)
    x = si.bf16_bits_to_f32(xb).astype(np.float64).reshape(32, 32, 128)
    qq = q.reshape(32, 32, 128)
    # every non-zero group reaches the largest code
    assert np.all((qq & 0x7F).max(axis=2) == 0x7E)
    # reconstruction within half an e4m3 step (relative 2^-4, absolute 2^-10 in the subnormal range)
    dec = oracle.e4m3_decode_table()[qq]
    r = x / s.reshape(32, 32, 1).astype(np.float64)
    step = np.where(np.abs(r) >= 2.0 ** -6, 2.0 ** np.floor(np.log2(np.maximum(np.abs(r), 1e-300))) / 8, 2.0 ** -9)
    assert np.all(np.abs(dec - r) <= step / 2 * (1 + 1e-6))


def test_quant_act_scale_invariance():
    xb = si.activations(8, 1024, outliers=False)
    q, s = oracle.quant_act(xb)
    for j in (-5, 3, 17):
        xj = si.to_bf16_bits(torch.from_numpy(si.bf16_bits_to_f32(xb) * np.float32(2.0 ** j)))
        qj, sj = oracle.quant_act(xj)
        assert np.array_equal(qj, q)
        assert np.array_equal(sj, (s * np.float32(2.0 ** j)).astype(np.float32))


def test_quant_act_token_and_group_independence():
    """Changing one group changes only that group's codes and scale (no transposition)."""
    xb = si.activations(6, 512, outliers=False)
    q, s = oracle.quant_act(xb)
    xb2 = xb.copy()
    xb2[4, 256:384] = _bf16_bits(np.linspace(-3, 5, 128))
    q2, s2 = oracle.quant_act(xb2)
    diff = q != q2
    assert diff[4, 256:384].any() and not diff[:4].any() and not diff[5].any()
    assert not diff[4, :256].any() and not diff[4, 384:].any()
    sd = s != s2
    assert sd[4, 2] and sd.sum() == 1


# ---------------------------------------------------- weight quantization ---

@pytest.mark.parametrize("N,K", [(128, 128), (256, 128), (128, 256)])
def test_quant_wblock_exact(N, K):
    w = si.weights(N, K)
    w[0, 0] = _bf16_bits([3.0])[0]   # one large value in block (0,0)
    q, s = oracle.quant_wblock(w)
    for nb in range(N // 128):
        for kb in range(K // 128):
            blk = w[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128].ravel()
            vals = [bf16_value(int(b)) for b in blk]
            s_ref, codes = quantize_exact(vals)
            assert s[nb, kb] == np.float32(s_ref)
            got = q[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128].ravel().tolist()
            assert got == codes


def test_quant_wblock_block_scale_layout():
    """Scale (nb,kb) depends only on its block: planting a big value moves one scale."""
    w = si.weights(256, 384)
    _, s = oracle.quant_wblock(w)
    w2 = w.copy()
    w2[200, 300] = _bf16_bits([10.0])[0]   # block (1, 2)
    _, s2 = oracle.quant_wblock(w2)
    changed = np.argwhere(s != s2)
    assert changed.tolist() == [[1, 2]]
    assert s2[1, 2] == np.float32(10.0) / np.float32(448.0)


# ------------------------------------------------------------------ 2:4 ------

def test_prune_golden_groups():
    with open(os.path.join(GOLDEN, "prune24_groups.txt")) as f:
        rows = [ln for ln in f if ln.strip() and not ln.startswith("#")]
    for ln in rows:
        wv, cv, kv = [p.split() for p in ln.split("|")]
        w = np.zeros((1, 128), np.float32)
        c = np.ones(128, np.float32)
        w[0, 4:8] = [float(t) for t in wv]
        c[4:8] = [float(t) for t in cv]
        keep = oracle.prune24_mask(_bf16_bits(w), c)
        assert np.nonzero(keep[0, 4:8])[0].tolist() == [int(t) for t in kv], ln


def test_prune_brute_force_with_ties():
    rng = np.random.default_rng(3)
    N, K = 16, 256
    w = rng.integers(-3, 4, (N, K)).astype(np.float32)   # many ties
    c = rng.integers(0, 3, K).astype(np.float32)
    wb = _bf16_bits(w)
    for cn in (None, c):
        keep = oracle.prune24_mask(wb, cn)
        assert np.all(keep.reshape(N, K // 4, 4).sum(axis=2) == 2)
        for n in range(N):
            for g in range(K // 4):
                sc = [abs(Fraction(float(w[n, 4 * g + j]))) * (1 if cn is None else Fraction(float(cn[4 * g + j])))
                      for j in range(4)]
                i, j = best_pair(sc)
                assert np.nonzero(keep[n, 4 * g:4 * g + 4])[0].tolist() == [i, j]


def test_prune_activation_aware_exact_scores():
    """Scores are exact products: an fp32 product would tie these two, fp64 does not."""
    w = np.zeros((1, 128), np.float32)
    c = np.ones(128, np.float32)
    a = f32(1.0 + 2 ** -7)          # bf16-exact
    b = f32(1.0)
    ca = f32(1.0 - 2 ** -23)
    cb = f32(1.0 + 2 ** -7 - 2 ** -22)
    # a*ca = 1 + 2^-7 - 2^-23 - 2^-30 ; b*cb = 1 + 2^-7 - 2^-22  -> a*ca is larger
    w[0, :4] = [a, b, 0.0, 0.0]
    c[:4] = [ca, cb, 1.0, 1.0]
    keep = oracle.prune24_mask(_bf16_bits(w), c)
    assert keep[0, :4].tolist() == [True, True, False, False]
    w[0, :4] = [0.0, b, a, 0.0]
    c[:4] = [1.0, cb, ca, 1.0]
    keep = oracle.prune24_mask(_bf16_bits(w), c)
    assert keep[0, :4].tolist() == [False, True, True, False]
    # now three candidates: a*ca > b*cb, so with a third big value b is dropped
    w[0, :4] = [0.0, b, a, 4.0]
    c[:4] = [1.0, cb, ca, 1.0]
    keep = oracle.prune24_mask(_bf16_bits(w), c)
    assert keep[0, :4].tolist() == [False, False, True, True]


def test_prune_matches_best_pair_over_many_random_groups():
    """Over whole random weights (magnitude and activation-aware), every group keeps
    the pair of positions with the largest score sum, the first such pair in
    lexicographic order when sums tie: an enumeration of the six pairs with exact
    fp64 sums, a different procedure from the oracle's ranking."""
    pairs = [(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)]
    w = si.weights(128, 1024)
    c = si.column_norms(si.calibration_batch(1024))
    for cn in (None, c):
        keep = oracle.prune24_mask(w, cn).reshape(128, 256, 4)
        score = np.abs(si.bf16_bits_to_f32(w).astype(np.float64))
        if cn is not None:
            score = score * cn.astype(np.float64)[None, :]
        score = score.reshape(128, 256, 4)
        sums = np.stack([score[..., i] + score[..., j] for i, j in pairs], axis=-1)
        best = np.argmax(sums, axis=-1)  # first maximum: the lexicographically smallest pair
        want = np.zeros_like(keep)
        for p, (i, j) in enumerate(pairs):
            sel = best == p
            want[..., i] |= sel
            want[..., j] |= sel
        assert np.array_equal(keep, want)


def test_compress_roundtrip_and_cross_path_identity():
    w = si.weights(256, 512)
    c = si.column_norms(si.calibration_batch(512))
    for cn in (None, c):
        vals, meta, s = oracle.prune24_compress(w, cn)
        keep = oracle.prune24_mask(w, cn)
        # pruned bf16 weights, then plain block quantization
        wp = np.where(keep, w, np.uint16(0)).astype(np.uint16)
        qd, sd = oracle.quant_wblock(wp)
        assert np.array_equal(s, sd)
        dense = oracle.decompress24(vals, meta)
        assert np.array_equal(dense, qd)
        # nibbles are valid (i0 < i1) and describe the mask
        nib = np.stack([meta & 15, meta >> 4], axis=-1).reshape(256, 128)
        assert set(np.unique(nib).tolist()) <= {4, 8, 12, 9, 13, 14}
        i0, i1 = nib & 3, nib >> 2
        km = keep.reshape(256, 128, 4)
        rows = np.arange(256)[:, None]
        grp = np.arange(128)[None, :]
        assert km[rows, grp, i0].all() and km[rows, grp, i1].all()
        # values in index order
        assert np.array_equal(vals.reshape(256, 128, 2)[..., 0], qd.reshape(256, 128, 4)[rows, grp, i0])


def test_compress_tensor_equals_tensor_quantization_of_the_pruned_weight():
    """Per-tensor 2:4 compression is the per-tensor quantization of mask * W, packed:
    the same mask as the block form, one scale (amax over the kept values / 448), and
    codes equal to those the per-tensor weight quantizer gives the pruned weight."""
    w = si.weights(384, 640)
    c = si.column_norms(si.calibration_batch(640))
    for cn in (None, c):
        vals, meta, s = oracle.prune24_compress_tensor(w, cn)
        keep = oracle.prune24_mask(w, cn)
        vb, mb, _ = oracle.prune24_compress(w, cn)
        assert np.array_equal(meta, mb)                      # the mask does not depend on the scale
        wp = np.where(keep, w, np.uint16(0)).astype(np.uint16)
        q, st = oracle.quant_weight_tensor(wp)
        assert np.all(s == s.flat[0]) and np.array_equal(s, st)
        kept_amax = np.abs(si.bf16_bits_to_f32(w)[keep]).max()
        assert s.flat[0] == np.float32(kept_amax) / np.float32(448)
        assert np.array_equal(oracle.decompress24(vals, meta), q)


def test_compress_tensor_exact_small():
    """Exact rational arithmetic on one 128 x 128 weight: the tensor scale and every kept code."""
    rng = np.random.default_rng(31)
    x = (rng.standard_normal((128, 128)) * 2.0 ** rng.integers(-8, 8, (128, 1))).astype(np.float32)
    w = _bf16_bits(x)
    vals, meta, s = oracle.prune24_compress_tensor(w)
    keep = oracle.prune24_mask(w)
    kept = [bf16_value(int(b)) for b in w[keep]]
    s_ref, codes = quantize_exact(kept, amax=max(abs(v) for v in kept))
    assert s[0, 0] == np.float32(s_ref)
    assert oracle.decompress24(vals, meta)[keep].tolist() == codes


def test_compress_tensor_equals_block_form_when_blocks_share_the_amax():
    """Where every 128 x 128 block's kept maximum is the tensor's, the two forms agree."""
    w = si.weights(256, 512).copy()
    big = _bf16_bits([3.0])[0]
    for nb in range(2):
        for kb in range(4):
            w[nb * 128 + 5, kb * 128 + 8] = big                    # a kept value (largest of its group)
    vb, mb, sb = oracle.prune24_compress(w)
    vt, mt, st = oracle.prune24_compress_tensor(w)
    assert np.array_equal(sb, st) and np.array_equal(vb, vt) and np.array_equal(mb, mt)


def test_compress_nibble_order_by_hand():
    w = np.zeros((128, 128), np.float32)
    w[0, 0:4] = [0, 5, 0, 7]       # group 0 keeps (1,3) -> nibble 1 | 3<<2 = 13
    w[0, 4:8] = [9, 0, 8, 0]       # group 1 keeps (0,2) -> nibble 0 | 2<<2 = 8
    vals, meta, s = oracle.prune24_compress(_bf16_bits(w))
    assert meta[0, 0] == 13 | (8 << 4)
    assert s[0, 0] == np.float32(9.0) / np.float32(448.0)
    enc = lambda v: oracle.e4m3_encode(f32(np.float32(v) / s[0, 0]))
    assert vals[0, :4].tolist() == [enc(5), enc(7), 0x7E, enc(8)]
    assert enc(7) == 123 and enc(5) == 120 and enc(8) == 124


def test_postprune_scale_uses_kept_values_only():
    w = np.full((128, 128), 0.01, np.float32)
    w[5, 8:12] = [100.0, 0.5, 0.6, 0.0]     # 100 is kept
    w[6, 8:12] = [0.0, 200.0, 300.0, 400.0]  # 200 is dropped
    _, _, s = oracle.prune24_compress(_bf16_bits(w))
    assert s[0, 0] == np.float32(400.0) / np.float32(448.0)
    w[6, 8:12] = [0.0, 0.0, 300.0, 0.0]
    w[7, 0:4] = [500.0, 600.0, 700.0, 800.0]  # 500, 600 dropped
    _, _, s = oracle.prune24_compress(_bf16_bits(w))
    assert s[0, 0] == np.float32(800.0) / np.float32(448.0)


# ------------------------------------------------------------------ GEMM -----

def _dequant(q, s, rows_per_scale_row, blocks_along_rows=False):
    dec = np.array([float(decode_exact(c)) if c not in (0x7F, 0xFF) else np.nan for c in range(256)])
    return dec[q]


def test_gemm_exact_fraction_tiny():
    rng = np.random.default_rng(5)
    M, N, K = 3, 128, 256
    xq, xs = oracle.quant_act(si.to_bf16_bits(torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32))))
    wq, ws = oracle.quant_wblock(si.weights(N, K))
    y = oracle.gemm(xq, xs, wq, ws)
    for m in range(M):
        for n in range(0, N, 7):
            acc = Fraction(0)
            for kb in range(K // 128):
                p = sum(decode_exact(int(xq[m, k])) * decode_exact(int(wq[n, k])) for k in range(kb * 128, kb * 128 + 128))
                acc += Fraction(float(xs[m, kb])) * Fraction(float(ws[n // 128, kb])) * p
            assert abs(Fraction(y[m, n]) - acc) <= abs(acc) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 1000)


def test_gemm_vs_numpy_dequant_matmul():
    M, N, K = 40, 384, 512
    xq, xs = oracle.quant_act(si.activations(M, K))
    wq, ws = oracle.quant_wblock(si.weights(N, K))
    dec = np.array([float(decode_exact(c)) if c not in (0x7F, 0xFF) else np.nan for c in range(256)])
    xd = dec[xq] * np.repeat(xs.astype(np.float64), 128, axis=1)
    wd = dec[wq] * np.repeat(np.repeat(ws.astype(np.float64), 128, axis=0), 128, axis=1)
    ref = xd @ wd.T
    y = oracle.gemm(xq, xs, wq, ws)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    rows = np.array([0, 7, 39], np.int64)
    assert np.array_equal(oracle.gemm(xq, xs, wq, ws, rows=rows), y[rows])


def test_gemm_integer_special_case():
    """Power-of-two scales and small-integer codes: Y is an exact int64 matmul."""
    rng = np.random.default_rng(9)
    M, N, K = 16, 256, 384
    int_codes = {v: c for c, v in ((c, float(decode_exact(c))) for c in range(256) if c not in (0x7F, 0xFF))
                 if float(v).is_integer() and abs(v) <= 16}
    vals = np.array(sorted(int_codes))
    xi = rng.choice(vals, (M, K))
    wi = rng.choice(vals, (N, K))
    xq = np.vectorize(int_codes.get)(xi).astype(np.uint8)
    wq = np.vectorize(int_codes.get)(wi).astype(np.uint8)
    xe = rng.integers(-3, 4, (M, K // 128))
    we = rng.integers(-3, 4, (N // 128, K // 128))
    xs = (2.0 ** xe).astype(np.float32)
    ws = (2.0 ** we).astype(np.float32)
    y = oracle.gemm(xq, xs, wq, ws)
    # exact: scale everything by 2^6 to stay integral
    ref = np.zeros((M, N), dtype=object)
    xi64 = xi.astype(np.int64)
    wi64 = wi.astype(np.int64)
    for kb in range(K // 128):
        p = xi64[:, kb * 128:(kb + 1) * 128] @ wi64[:, kb * 128:(kb + 1) * 128].T
        sc = xe[:, kb][:, None] + np.repeat(we[:, kb], 128)[None, :]
        ref = ref + np.vectorize(lambda a, e: Fraction(int(a)) * Fraction(2) ** int(e))(p, sc)
    assert all(Fraction(y[m, n]) == ref[m, n] for m in range(M) for n in range(N))


def test_gemm_block_identity():
    """W = identity blocks with code 1.0 and scale 1: Y equals dequantized X."""
    M, K = 8, 256
    xq, xs = oracle.quant_act(si.activations(M, K))
    wq = np.zeros((K, K), np.uint8)
    np.fill_diagonal(wq, 0x38)   # 1.0
    ws = np.ones((K // 128, K // 128), np.float32)
    y = oracle.gemm(xq, xs, wq, ws)
    dec = oracle.e4m3_decode_table()
    ref = dec[xq] * np.repeat(xs.astype(np.float64), 128, axis=1)
    assert np.array_equal(y, ref)
    # and the scale of W's block row scales the matching outputs only
    ws2 = ws.copy()
    ws2[1, :] = 2.0
    y2 = oracle.gemm(xq, xs, wq, ws2)
    assert np.array_equal(y2[:, :128], ref[:, :128]) and np.array_equal(y2[:, 128:], 2 * ref[:, 128:])


def test_sparse_gemm_equals_dense_on_decompressed():
    M, N, K = 16, 256, 512
    xq, xs = oracle.quant_act(si.activations(M, K))
    w = si.weights(N, K)
    vals, meta, s = oracle.prune24_compress(w)
    y = oracle.sparse24_gemm(xq, xs, vals, meta, s)
    keep = oracle.prune24_mask(w)
    wq, ws = oracle.quant_wblock(np.where(keep, w, np.uint16(0)).astype(np.uint16))
    assert np.array_equal(y, oracle.gemm(xq, xs, wq, ws))


# ----------------------------------------------------------------- SwiGLU ---

def test_swiglu_against_library_sigmoid_and_identities():
    """silu(g) * u against scipy's logistic function, and silu(x) - silu(-x) = x."""
    from scipy.special import expit
    g = np.concatenate([np.linspace(-60, 60, 2001), [0.0, 1e-30, -1e-30, 700.0, -700.0, -1e4]])
    u = np.cos(np.arange(g.size))
    assert np.allclose(oracle.swiglu(g, u), g * expit(g) * u, rtol=1e-14, atol=1e-300)
    assert np.allclose(oracle.swiglu(g, 1.0) - oracle.swiglu(-g, 1.0), g, rtol=1e-13, atol=1e-13)
    assert oracle.swiglu(0.0, 5.0) == 0.0
    assert oracle.swiglu(-1e4, 3.0) == 0.0 and oracle.swiglu(1e4, 3.0) == 3e4


def test_gemm_swiglu_uses_gate_then_up_halves():
    """Swapping the gate and up halves changes the result as silu's asymmetry says
    (a transposed stacking fails); each half is the dense GEMM of its rows."""
    rng = np.random.default_rng(11)
    M, K, I = 3, 256, 128
    xq, xs = oracle.quant_act(si.to_bf16_bits(torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32))))
    w = si.to_bf16_bits(torch.from_numpy((rng.standard_normal((2 * I, K)) * 0.05).astype(np.float32)))
    wq, ws = oracle.quant_wblock(w)
    h = oracle.gemm_swiglu(xq, xs, wq, ws)
    g = oracle.gemm(xq, xs, wq[:I], ws[:1])
    u = oracle.gemm(xq, xs, wq[I:], ws[1:])
    assert np.array_equal(h, oracle.swiglu(g, u))
    swapped = oracle.gemm_swiglu(xq, xs, np.concatenate([wq[I:], wq[:I]]), np.concatenate([ws[1:], ws[:1]]))
    assert not np.allclose(h, swapped)
    rows = np.array([2, 0])
    assert np.array_equal(oracle.gemm_swiglu(xq, xs, wq, ws, rows=rows), h[rows])


# ----------------------------------------------------------- UE8M0 scales ---

def _ue8m0_groups():
    """[8, 1024] bf16 groups of 128: exact powers of two times 448, just above them,
    zero, bf16 subnormals, the bf16 maximum, random normals and heavy tails."""
    rng = np.random.default_rng(21)
    x = rng.standard_normal((8, 1024)).astype(np.float32)
    x[0, :128] = 0.0
    x[0, 128:256] = np.float32(448.0) * np.linspace(-1, 1, 128, dtype=np.float32)   # amax = 448 exactly
    x[0, 256:384] = np.float32(448.0 * 2 ** -20) * np.sign(rng.standard_normal(128)).astype(np.float32)
    x[0, 384:512] = rng.standard_normal(128).astype(np.float32) * 1e-39            # bf16 subnormals
    x[1, :128] = np.float32(3.3895314e38) * np.linspace(-1, 1, 128, dtype=np.float32)  # near the bf16 max
    x[1, 128:256] = np.float32(450.0)                                               # next bf16 above 448
    x[1, 256:384] = np.float32(448.0 * (1 + 2 ** -7)) * np.linspace(-1, 1, 128, dtype=np.float32)
    z = rng.standard_normal((4, 2, 1024))
    x[2:4] = (z[0] / np.sqrt((z[1] ** 2 + z[2] ** 2 + z[3] ** 2) / 3)).astype(np.float32)
    return si.to_bf16_bits(torch.from_numpy(x))


def test_ue8m0_exponent_is_the_smallest_covering_power_of_two():
    xb = _ue8m0_groups()
    q, e = oracle.quant_act_ue8m0(xb)
    vals = si.bf16_bits_to_f32(xb)
    for m in range(vals.shape[0]):
        for kb in range(vals.shape[1] // 128):
            amax = Fraction(float(np.abs(vals[m, 128 * kb:128 * kb + 128]).max()))
            ek = int(e[m, kb])
            assert Fraction(448) * Fraction(2) ** (ek - 127) >= amax
            assert ek == 0 or Fraction(448) * Fraction(2) ** (ek - 128) < amax
    assert e[0, 0] == 0 and e[0, 1] == 127 and e[0, 2] == 107 and e[0, 3] == 0
    assert e[1, 1] == 128 and e[1, 2] == 128


def test_ue8m0_codes_are_the_nearest_of_the_exact_quotient():
    """Exhaustive nearest-value search on x / 2^(e-127) (an exact rational), independent
    of the oracle's bisection encoder."""
    xb = _ue8m0_groups()
    q, e = oracle.quant_act_ue8m0(xb)
    vals = si.bf16_bits_to_f32(xb)
    rng = np.random.default_rng(3)
    for m in range(vals.shape[0]):
        for k in rng.choice(vals.shape[1], 48, replace=False):
            x = float(vals[m, k])
            neg = math.copysign(1.0, x) < 0
            ek = int(e[m, k // 128])
            want = nearest_e4m3(Fraction(x) / Fraction(2) ** (ek - 127), negative=neg)
            assert q[m, k] == want, (m, k, x, ek)


def test_ue8m0_matches_fp32_scales_when_amax_over_448_is_a_power_of_two():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((4, 512)).astype(np.float32)
    for m in range(4):
        for kb in range(4):
            g = x[m, 128 * kb:128 * kb + 128]
            g[np.argmax(np.abs(g))] = np.float32(448.0 * 2.0 ** (kb - m * 3))   # amax = 448 * 2^k
            g[:] = np.clip(g, -448.0 * 2.0 ** (kb - m * 3), 448.0 * 2.0 ** (kb - m * 3))
    xb = si.to_bf16_bits(torch.from_numpy(x))
    q8, e = oracle.quant_act_ue8m0(xb)
    q32, s = oracle.quant_act(xb)
    assert np.array_equal(q8, q32)
    assert np.array_equal(oracle.ue8m0_to_f32(e), s)


def test_ue8m0_scale_invariance_and_values():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((4, 256)).astype(np.float32)
    q0, e0 = oracle.quant_act_ue8m0(si.to_bf16_bits(torch.from_numpy(x)))
    for j in (-30, -1, 5, 40):
        qj, ej = oracle.quant_act_ue8m0(si.to_bf16_bits(torch.from_numpy(x * np.float32(2.0 ** j))))
        assert np.array_equal(qj, q0) and np.array_equal(ej.astype(int), e0.astype(int) + j)
    v = oracle.ue8m0_to_f32(np.array([0, 1, 126, 127, 128, 254], np.uint8))
    assert v[3] == 1.0 and v[4] == 2.0 and v[2] == 0.5 and v[5] == 2.0 ** 127
    assert v[0] == np.float32(2.0 ** -127) and 0 < v[0] < np.finfo(np.float32).tiny


def test_ue8m0_weight_blocks_exact():
    rng = np.random.default_rng(8)
    w = (rng.standard_normal((256, 384)) * 0.02).astype(np.float32)
    w[:128, 128:256] *= 1e4
    w[128:, :128] = 0.0
    wb = si.to_bf16_bits(torch.from_numpy(w))
    q, e = oracle.quant_wblock_ue8m0(wb)
    vals = si.bf16_bits_to_f32(wb)
    for nb in range(2):
        for kb in range(3):
            blk = vals[128 * nb:128 * nb + 128, 128 * kb:128 * kb + 128]
            amax = Fraction(float(np.abs(blk).max()))
            ek = int(e[nb, kb])
            assert Fraction(448) * Fraction(2) ** (ek - 127) >= amax
            assert ek == 0 or Fraction(448) * Fraction(2) ** (ek - 128) < amax
            for (i, j) in [(0, 0), (5, 77), (127, 127), (64, 3)]:
                x = float(blk[i, j])
                want = nearest_e4m3(Fraction(x) / Fraction(2) ** (ek - 127), negative=math.copysign(1.0, x) < 0)
                assert q[128 * nb + i, 128 * kb + j] == want
    assert e[1, 0] == 0 and np.all(q[128:, :128] == 0)


def test_gemm_ue8m0_is_the_gemm_with_power_of_two_scales():
    rng = np.random.default_rng(10)
    x = si.to_bf16_bits(torch.from_numpy(rng.standard_normal((8, 256)).astype(np.float32)))
    w = si.to_bf16_bits(torch.from_numpy((rng.standard_normal((128, 256)) * 0.02).astype(np.float32)))
    xq, xe = oracle.quant_act_ue8m0(x)
    wq, we = oracle.quant_wblock_ue8m0(w)
    y = oracle.gemm_ue8m0(xq, xe, wq, we)
    # exact: every product is a multiple of 2^-18 times 2^(ex+ew-254); sum exactly with Fractions
    for m, n in [(0, 0), (3, 77), (7, 127)]:
        acc = Fraction(0)
        for kb in range(2):
            blk = sum(decode_exact(int(xq[m, k])) * decode_exact(int(wq[n, k])) for k in range(128 * kb, 128 * kb + 128))
            acc += blk * Fraction(2) ** (int(xe[m, kb]) - 127) * Fraction(2) ** (int(we[0, kb]) - 127)
        assert y[m, n] == float(acc)


# ---------------------------------------------------------- grouped GEMM ---

def test_grouped_gemm_oracle_routes_rows_to_their_expert():
    rng = np.random.default_rng(12)
    M, K, N, G = 40, 256, 128, 3
    xq, xs = oracle.quant_act(si.to_bf16_bits(torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32))))
    ws_, wq_ = [], []
    for g in range(G):
        q, s = oracle.quant_wblock(si.to_bf16_bits(torch.from_numpy((rng.standard_normal((N, K)) * 0.02 * (g + 1)).astype(np.float32))))
        wq_.append(q)
        ws_.append(s)
    wq, ws = np.stack(wq_), np.stack(ws_)
    offsets = np.array([0, 17, 17, 40])          # expert 1 gets no tokens
    y = oracle.grouped_gemm(xq, xs, wq, ws, offsets)
    assert np.array_equal(y[:17], oracle.gemm(xq[:17], xs[:17], wq[0], ws[0]))
    assert np.array_equal(y[17:], oracle.gemm(xq[17:], xs[17:], wq[2], ws[2]))
    # one group covering everything is the plain GEMM
    assert np.array_equal(oracle.grouped_gemm(xq, xs, wq[1:2], ws[1:2], np.array([0, M])),
                          oracle.gemm(xq, xs, wq[1], ws[1]))
    # rows are independent of the order experts are listed in (a swapped lookup fails)
    perm = oracle.grouped_gemm(xq, xs, wq[::-1].copy(), ws[::-1].copy(), np.array([0, 0, 23, 40]))
    assert np.array_equal(perm[:23], oracle.gemm(xq[:23], xs[:23], wq[1], ws[1]))
    assert np.array_equal(perm[23:], oracle.gemm(xq[23:], xs[23:], wq[0], ws[0]))
    rows = np.array([39, 0, 16, 17])
    assert np.array_equal(oracle.grouped_gemm(xq, xs, wq, ws, offsets, rows=rows), y[rows])


# ------------------------------------------ per-tensor and static scales ---

def test_quant_act_tensor_and_static_against_exact_arithmetic():
    rng = np.random.default_rng(14)
    x = rng.standard_normal((6, 384)).astype(np.float32)
    x[2, 5] = 37.0                                              # the tensor's amax
    xb = si.to_bf16_bits(torch.from_numpy(x))
    q, s = oracle.quant_act_tensor(xb)
    vals = si.bf16_bits_to_f32(xb)
    s_ref, codes = quantize_exact([float(v) for v in vals.ravel()], amax=float(np.abs(vals).max()))
    assert np.all(s == np.float32(s_ref)) and s.shape == (6, 3)
    assert np.array_equal(q.ravel(), np.array(codes, np.uint8))
    # static with that scale gives the same; a smaller static scale saturates the large values
    qs, ss = oracle.quant_act_static(xb, s_ref)
    assert np.array_equal(qs, q) and np.all(ss == np.float32(s_ref))
    q2, _ = oracle.quant_act_static(xb, s_ref / 4)
    assert q2[2, 5] == 0x7E and np.all(np.abs(q2.astype(np.int16) & 0x7F) <= 0x7E)
    _, codes2 = quantize_exact([float(v) for v in vals.ravel()], amax=float(np.abs(vals).max()) / 4)
    assert np.array_equal(q2.ravel(), np.array(codes2, np.uint8))


def test_quant_act_tensor_equals_block_scaling_when_every_group_shares_the_amax():
    rng = np.random.default_rng(15)
    x = rng.standard_normal((4, 512)).astype(np.float32)
    x[:, ::128] = 9.0                                          # every 1x128 group has amax 9
    xb = si.to_bf16_bits(torch.from_numpy(x))
    qt, st = oracle.quant_act_tensor(xb)
    qb, sb = oracle.quant_act(xb)
    assert np.array_equal(qt, qb) and np.array_equal(st, sb)


def test_quant_weight_tensor_equals_block_scaling_when_every_block_shares_the_amax():
    rng = np.random.default_rng(16)
    w = (0.02 * rng.standard_normal((256, 384))).astype(np.float32)
    w[::128, ::128] = -0.75                                    # every 128x128 block has amax 0.75
    wb = si.to_bf16_bits(torch.from_numpy(w))
    qt, st = oracle.quant_weight_tensor(wb)
    qb, sb = oracle.quant_wblock(wb)
    assert st.shape == (2, 3) and np.array_equal(qt, qb) and np.array_equal(st, sb)
    w[7, 300] = 3.0                                            # one block now holds the tensor amax
    qt2, st2 = oracle.quant_weight_tensor(si.to_bf16_bits(torch.from_numpy(w)))
    assert np.all(st2 == np.float32(3.0) / np.float32(448.0)) and qt2[7, 300] == 0x7E
