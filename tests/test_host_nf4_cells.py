"""The quantise kernel's NF4 code lookup: a 256-cell table over [-1, 1) (cell width
1/128) holding, per cell i, the number of midpoints below -1 + (i - 1)/128 and the one
midpoint in the three-cell window [-1 + (i - 1)/128, -1 + (i + 2)/128) (or +inf); the
code of t is that count plus (midpoint < t), with the cell index trunc((t + 1) * 128) in
binary32, clamped to 0..255.  Checked here, in binary32 as the kernel computes it, to
equal the number of midpoints strictly below t (the codec's definition, QLoRA's NF4
midpoints as the oracle builds them) for every t near a midpoint or a cell edge, across
[-1.1, 1.1], and far outside (saturated fp16 scales)."""
import numpy as np

import oracle as O

F32 = np.float32


def _cells(mid):
    lo = F32(-1.0) + np.arange(-1, 255, dtype=F32) * F32(1.0 / 128.0)
    hi = F32(-1.0) + np.arange(2, 258, dtype=F32) * F32(1.0 / 128.0)
    cnt = (mid[None, :] < lo[:, None]).sum(1)
    inwin = (mid[None, :] >= lo[:, None]) & (mid[None, :] < hi[:, None])
    assert inwin.sum(1).max() <= 1, "a window holds two midpoints"
    cand = np.where(inwin.any(1), np.where(inwin, mid[None, :], 0).sum(1), np.inf).astype(F32)
    return cnt, cand


def _lookup(t, cnt, cand):
    x = (t + F32(1.0)) * F32(128.0)                      # two binary32 roundings, as in the kernel
    ci = np.clip(np.trunc(x), 0, 255).astype(np.int64)   # trunc toward zero (v_cvt_i32_f32)
    return cnt[ci] + (cand[ci] < t)


def _edge_cases(mid):
    pts = [F32(-1.0) + F32(k / 128.0) for k in range(-2, 260)] + list(mid)
    out = []
    for p in pts:
        x = F32(p)
        for _ in range(4):
            out += [x]
            x = np.nextafter(x, F32(np.inf))
        x = F32(p)
        for _ in range(4):
            x = np.nextafter(x, F32(-np.inf))
            out += [x]
    return np.array(out, dtype=F32)


def test_cell_lookup_counts_the_midpoints_below_t():
    mid = O.codec.nf4_midpoints().astype(F32)
    cnt, cand = _cells(mid)
    rng = np.random.default_rng(5)
    t = np.concatenate([_edge_cases(mid), rng.uniform(-1.1, 1.1, 400000).astype(F32),
                        np.array([-60000.0, -3.0, -1.0005, 1.0005, 3.0, 60000.0, 0.0, -0.0], F32)])
    ref = (mid[None, :] < t[:, None]).sum(1)
    assert np.array_equal(_lookup(t, cnt, cand), ref)


def test_the_three_cell_window_absorbs_an_index_one_cell_off():
    """An index one cell low (what rounding near a cell edge can give) miscounts with a
    table whose window is the cell alone, and not with the three-cell window."""
    mid = O.codec.nf4_midpoints().astype(F32)
    lo = F32(-1.0) + np.arange(0, 256, dtype=F32) * F32(1.0 / 128.0)
    hi = lo + F32(1.0 / 128.0)
    cnt1 = (mid[None, :] < lo[:, None]).sum(1)
    inwin = (mid[None, :] >= lo[:, None]) & (mid[None, :] < hi[:, None])
    cand1 = np.where(inwin.any(1), np.where(inwin, mid[None, :], 0).sum(1), np.inf).astype(F32)
    t = _edge_cases(mid)
    ref = (mid[None, :] < t[:, None]).sum(1)
    ci = np.clip(np.trunc((t + F32(1.0)) * F32(128.0)) - 1, 0, 255).astype(np.int64)
    assert not np.array_equal(cnt1[ci] + (cand1[ci] < t), ref)
    cnt3, cand3 = _cells(mid)
    assert np.array_equal(cnt3[ci] + (cand3[ci] < t), ref)
