"""Pins of the oracle's sparse attention with K = V and inverse RoPE (CPU only).

* Dense special case: with k >= the number of causal entries the result is
  plain softmax attention over all causal entries plus the window
  ([vLLM-V4] appendix, c128a framed as top-k 8192), checked against torch's
  scaled_dot_product_attention in float64 with K = V.
* Translation invariance: shifting every position by a multiple of 256 with
  the same pre-rotation content leaves the output unchanged ([vLLM-V4]
  appendix: after R_m^{-1} only R_{n-m} remains).
* Single row: one window row and no entries gives out = the row before
  rotation ([vLLM-V4] appendix; K = V).
* Window edges: rows t-127 .. t are used, t-128 and t+1 are not ([vLLM-V4]
  appendix, why the short window).
* c128a queries at t < 127 see no compressed entry.
"""

import numpy as np
import pytest
import torch

from oracle import attention, geometry
from oracle.paged import PagedCache
from tests._rot import close, rotate

D = 576


def fill(cache, b, idx, rows):
    for r, v in zip(idx, rows):
        cache.write(b, int(r), v)


def make_caches(rng, ratio, L, dtype="f32", d=D, pre=None):
    n = geometry.num_entries(L, ratio)
    kv = PagedCache.empty(1, max(n, 1), geometry.entries_per_block(ratio), d, dtype, perm_seed=1)
    swa = PagedCache.empty(1, L, 256, d, dtype, perm_seed=2)
    ent = rng.standard_normal((n, d)) if pre is None else pre[0]
    raw = rng.standard_normal((L, d)) if pre is None else pre[1]
    fill(kv, 0, range(n), ent)
    fill(swa, 0, range(L), raw)
    return kv, swa


@pytest.mark.parametrize("ratio,L,H,W", [(4, 300, 3, 128), (128, 1000, 2, 128), (4, 64, 2, 16)])
def test_dense_equals_sdpa(ratio, L, H, W):
    rng = np.random.default_rng(0)
    kv, swa = make_caches(rng, ratio, L)
    t = L - 1
    q = rng.standard_normal((1, H, D))
    n = geometry.visible_entries(t, ratio)
    scale = 1 / 24
    out, lse = attention.sparse_attn_decode([0, 1], [t], q, kv, ratio, None, swa, W, scale, 1e4, 64)
    # the same result through a top-k list that names every causal entry, in shuffled order
    ids = rng.permutation(n)[None, :]
    out2, _ = attention.sparse_attn_decode([0, 1], [t], q, kv, ratio, np.concatenate(
        [ids, -np.ones((1, 5), np.int64)], axis=1), swa, W, scale, 1e4, 64)
    assert close(out, out2, 1e-12)
    rows = np.concatenate([kv.read(0, np.arange(n)), swa.read(0, np.arange(max(0, t - W + 1), t + 1))])
    kt = torch.from_numpy(rows)[None, None].expand(1, H, -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q[0])[None, :, None, :], kt, kt, scale=scale)[0, :, 0].numpy()
    assert close(out[0], rotate(ref, -t), 1e-10)
    z = scale * q[0] @ rows.T
    assert close(lse[0], np.log(np.exp(z).sum(axis=1)), 1e-10)


def test_translation_invariance():
    rng = np.random.default_rng(1)
    L, delta, H, W = 700, 512, 2, 128
    n = geometry.num_entries(L, 4)
    norm_ent = rng.standard_normal((n, D))
    raw = rng.standard_normal((L, D))
    q0 = rng.standard_normal((H, D))
    t = L - 1
    sel = rng.choice(n, 40, replace=False)

    def run(shift):
        sh_e = shift // 4
        ent = np.zeros((n + sh_e, D))
        for j in range(n):
            ent[j + sh_e] = rotate(norm_ent[j], geometry.entry_anchor(j + sh_e, 4))
        win = np.zeros((L + shift, D))
        for p in range(max(0, t - W + 1), L):
            win[p + shift] = rotate(raw[p], p + shift)
        kv, swa = make_caches(rng, 4, L + shift, pre=(ent, win))
        q = rotate(q0, t + shift)[None]
        out, _ = attention.sparse_attn_decode([0, 1], [t + shift], q, kv, 4, (sel + sh_e)[None],
                                              swa, W, 0.05, 1e4, 64)
        return out

    # rows are stored as float32, so agreement is to float32 rounding
    assert close(run(0), run(delta), 1e-6)


def test_single_row_returns_unrotated_row():
    rng = np.random.default_rng(2)
    L = 50
    x = rng.standard_normal((L, D))
    win = np.stack([rotate(x[p], p) for p in range(L)])
    kv, swa = make_caches(rng, 4, L, pre=(rng.standard_normal((geometry.num_entries(L, 4), D)), win))
    q = rng.standard_normal((1, 3, D))
    out, _ = attention.sparse_attn_decode([0, 1], [L - 1], q, kv, 4, -np.ones((1, 8), np.int64),
                                          swa, 1, 0.04, 1e4, 64)
    for h in range(3):          # the window row went through float32 storage
        assert close(out[0, h], x[L - 1], 1e-6)


def test_c128a_early_queries_see_window_only():
    rng = np.random.default_rng(3)
    kv, swa = make_caches(rng, 128, 200)
    q = rng.standard_normal((1, 2, D))
    for t in (0, 60, 126):
        a, _ = attention.sparse_attn_decode([0, 1], [t], q, kv, 128, None, swa, 128, 0.04, 1e4, 64)
        kv2 = kv.copy()
        kv2.rows[:] = 1e3                                 # compressed entries are invisible
        b, _ = attention.sparse_attn_decode([0, 1], [t], q, kv2, 128, None, swa, 128, 0.04, 1e4, 64)
        assert np.array_equal(a, b)


def test_window_edges():
    rng = np.random.default_rng(4)
    L, t, W = 600, 400, 128
    kv, swa = make_caches(rng, 4, L)
    q = rng.standard_normal((1, 2, D))
    ids = np.array([[3, 9, -1]])
    base, _ = attention.sparse_attn_decode([0, 1], [t], q, kv, 4, ids, swa, W, 0.04, 1e4, 64)
    for p, used in [(t - 128, False), (t + 1, False), (t - 127, True), (t, True)]:
        s2 = swa.copy()
        s2.write(0, p, np.full(D, 50.0))
        o, _ = attention.sparse_attn_decode([0, 1], [t], q, kv, 4, ids, s2, W, 0.04, 1e4, 64)
        assert (not np.array_equal(o, base)) == used, p
    # non-causal or padded list entries are skipped
    n_vis = geometry.visible_entries(t, 4)
    o, _ = attention.sparse_attn_decode([0, 1], [t], q, kv, 4, np.array([[3, 9, n_vis, -1]]), swa,
                                        W, 0.04, 1e4, 64)
    assert np.array_equal(o, base)


def test_output_fp8_rows():
    """The fp8 output rows ([vLLM-V4] second fusion): per (query, head) row, scale = amax/448
    in float32 and codes that decode (code value * scale) to within half an E4M3 step of the
    row; the row's largest magnitude is exactly code 448 (0x7E or 0xFE); an all-zero row has
    scale 1 and zero codes."""
    from oracle.attention import output_fp8
    from oracle import formats
    rng = np.random.default_rng(11)
    out = rng.standard_normal((3, 2, 576)) * rng.uniform(0.01, 50.0, size=(3, 2, 1))
    out[2, 1] = 0.0
    codes, scales = output_fp8(out)
    assert codes.shape == out.shape and codes.dtype == np.uint8 and scales.shape == (3, 2)
    for i in range(3):
        for h in range(2):
            row = out[i, h]
            amax = np.max(np.abs(row))
            if amax == 0:
                assert scales[i, h] == 1.0 and not codes[i, h].any()
                continue
            assert scales[i, h] == np.float32(amax / 448.0)
            dec = formats.fp8_e4m3_to_f64(codes[i, h]) * np.float64(scales[i, h])
            q = row / np.float64(scales[i, h])
            # half an E4M3 step of each value (normal binades: 2^(e-4); subnormals: 2^-10)
            e = np.floor(np.log2(np.maximum(np.abs(q), 2.0 ** -6)))
            half = np.ldexp(1.0, (e - 4).astype(int)) * np.float64(scales[i, h])
            assert np.all(np.abs(dec - row) <= half * (1 + 1e-12))
            j = int(np.argmax(np.abs(row)))
            assert codes[i, h, j] in (0x7E, 0xFE)
