"""Pins of the oracle's compressor and entry geometry (CPU only).

What the pages fix, and how each is checked:
* entry counts: 256/4 = 64 and 256/128 = 2 entries per 256-position block
  ([vLLM-V4] section 3 part 1); about 250K c4a entries and at most about 8000
  c128a entries at 1M tokens ([vLLM-V4] section 2 and appendix, k values);
* coverage: c4a entry i is built from positions [4i-4, 4i+3], c128a entry i
  from [128i, 128i+127] ([vLLM-V4] appendix, exact position ranges) --
  checked by one-hot raw tokens;
* combine-then-RoPE-once at the anchor, then RMSNorm before RoPE
  ([vLLM-V4] appendix and section 3 part 2) -- closed forms on rows whose
  mean square is exactly 1 with eps = 0;
* the rolling residual is a handoff: any split of the raw stream gives
  bit-identical entries ([vLLM-V4] section 3 part 1, prefix caching at block
  boundaries);
* the Ref workload's indexing (entry i over [4i, 4i+8), RoPE at 4i+7) is the
  pages' entry i+1.
"""

import numpy as np
import pytest

from oracle import compress, geometry
from oracle.paged import PagedCache
from tests._rot import close, rotate, unit_rms_row


def run_stream(raw, ratio, splits, logits_all, eps=1e-6, gamma=None, dtype="f32", perm_seed=None,
               swa=False):
    """Feed raw rows [L, d] (float32) in the given chunk sizes; return (out cache, state, swa cache)."""
    L, d = raw.shape
    n = geometry.num_entries(L, ratio)
    out = PagedCache.empty(1, max(n, 1), geometry.entries_per_block(ratio), d, dtype, perm_seed)
    state = PagedCache.empty(1, L, 256, d, "f32", perm_seed)
    swac = PagedCache.empty(1, L, 256, d, "f32", perm_seed) if swa else None
    pos = 0
    for size in splits:
        L_old, L_new = pos, pos + size
        j0, j1 = geometry.num_entries(L_old, ratio), geometry.num_entries(L_new, ratio)
        compress.compress_insert(ratio, [L_old], [0, size], raw[L_old:L_new], "f32", [0, j1 - j0],
                                 logits_all[j0:j1], gamma, eps, 10000.0, 64, state, out, swac)
        pos = L_new
    assert pos == L
    return out, state, swac


def entries_of(out, n):
    return out.read(0, np.arange(n))


def test_counts_pinned_by_pages():
    assert geometry.num_entries(2 ** 20, 4) == 262144
    assert abs(geometry.num_entries(2 ** 20, 4) - 250_000) / 250_000 < 0.05
    assert geometry.num_entries(2 ** 20, 128) == 8192
    for ratio, per_block in [(4, 64), (128, 2)]:
        assert geometry.entries_per_block(ratio) == per_block
        # the anchors themselves fall 64 (resp. 2) to every 256-position block, the first included
        anchors = [geometry.entry_anchor(j, ratio) for j in range(geometry.num_entries(4096, ratio))]
        counts = np.bincount(np.array(anchors) // 256)
        assert np.all(counts == per_block)
        # and entry j lives in logical block j // per_block
        assert all(a // 256 == j // per_block for j, a in enumerate(anchors))


def test_window_lengths_and_causality():
    assert geometry.window_len(4) == 8 and geometry.window_len(128) == 128
    # query m may use entry i only when its anchor 4i+3 (128i+127) is <= m
    assert geometry.visible_entries(2, 4) == 0 and geometry.visible_entries(3, 4) == 1
    assert geometry.visible_entries(126, 128) == 0 and geometry.visible_entries(127, 128) == 1


@pytest.mark.parametrize("ratio", [4, 128])
def test_one_hot_coverage(ratio):
    d, L = 80, 768
    rng = np.random.default_rng(0)
    n = geometry.num_entries(L, ratio)
    logits = rng.standard_normal((n, geometry.window_len(ratio))).astype(np.float32)
    for p in [0, 3, 4, 5, 130, 255, 256, 511, 767]:
        raw = np.zeros((L, d), np.float32)
        raw[p] = rng.standard_normal(d)
        out, _, _ = run_stream(raw, ratio, [L], logits, eps=1e-30)
        nz = [j for j in range(n) if np.any(entries_of(out, n)[j] != 0)]
        if ratio == 4:
            expect = [j for j in (p // 4, p // 4 + 1) if j < n]
        else:
            expect = [p // 128] if p // 128 < n else []
        assert nz == expect, (p, nz, expect)


@pytest.mark.parametrize("ratio", [4, 128])
def test_identical_rows_closed_form(ratio):
    """All raw rows equal to x with mean(x^2) = 1, eps = 0: every entry is RoPE_anchor(x)."""
    rng = np.random.default_rng(1)
    d, L = 96, 512
    x = unit_rms_row(rng, d)
    raw = np.tile(x, (L, 1)).astype(np.float32)
    n = geometry.num_entries(L, ratio)
    logits = (rng.standard_normal((n, geometry.window_len(ratio))) * 3).astype(np.float32)
    out, _, _ = run_stream(raw, ratio, [L], logits, eps=0.0)
    ent = entries_of(out, n)
    for j in range(n):
        # entry 0 of c4a has four zero-padded slots: the weighted sum is a scalar times x,
        # which RMSNorm removes
        assert close(ent[j], rotate(x, geometry.entry_anchor(j, ratio)), 1e-6), j


def test_single_slot_weight_and_scale_invariance():
    rng = np.random.default_rng(2)
    d, L = 64 + 32, 64
    raw = np.stack([unit_rms_row(rng, d) for _ in range(L)]).astype(np.float32)
    n = geometry.num_entries(L, 4)
    logits = np.full((n, 8), -1e4, np.float32)
    logits[:, 5] = 0.0                         # all weight on slot 5 = position 4j+1
    out, _, _ = run_stream(raw, 4, [L], logits, eps=0.0)
    ent = entries_of(out, n)
    for j in range(1, n):
        assert close(ent[j], rotate(raw[4 * j + 1], 4 * j + 3), 1e-6)
    # adding a constant to an entry's logits changes nothing; scaling the rows changes nothing
    logits2 = rng.standard_normal((n, 8)).astype(np.float32)
    a, _, _ = run_stream(raw, 4, [L], logits2, eps=0.0)
    b, _, _ = run_stream(raw, 4, [L], logits2 + np.float32(5.0), eps=0.0)
    c, _, _ = run_stream(raw * np.float32(8.0), 4, [L], logits2, eps=0.0)
    assert close(entries_of(a, n), entries_of(b, n), 1e-6)
    assert close(entries_of(a, n), entries_of(c, n), 1e-9)
    # gamma multiplies the normalised row before rotation
    g = np.full(d, 2.0)
    e, _, _ = run_stream(raw, 4, [L], logits2, eps=0.0, gamma=g)
    assert close(entries_of(e, n), 2 * entries_of(a, n), 1e-9)


def test_rms_norm_hand_example():
    y = np.array([3.0, 4.0])
    assert close(compress.rms_norm(y, None, 0.0), y / np.sqrt(12.5))
    assert close(compress.rms_norm(y, np.array([1.0, 0.5]), 0.0), np.array([3.0, 2.0]) / np.sqrt(12.5))


def test_ref_workload_indexing_is_shifted_by_one():
    """Entry i of the Ref workload (window [4i, 4i+8), RoPE at 4i+7) equals the pages' entry i+1."""
    rng = np.random.default_rng(4)
    d, L = 576, 96
    raw = rng.standard_normal((L, d)).astype(np.float32)
    n = geometry.num_entries(L, 4)
    logits = rng.standard_normal((n, 8)).astype(np.float32)
    out, _, _ = run_stream(raw, 4, [L], logits, eps=1e-6)
    ent = entries_of(out, n)
    for i in range(n - 1):
        j = i + 1
        lw = logits[j].astype(np.float64)
        w = np.exp(lw - lw.max())
        w /= w.sum()
        y = w @ raw[4 * i:4 * i + 8].astype(np.float64)
        nrm = y / np.sqrt(np.mean(y ** 2) + 1e-6)
        assert close(ent[j], rotate(nrm, 4 * i + 7), 1e-6)


@pytest.mark.parametrize("ratio", [4, 128])
def test_chunk_invariance(ratio):
    rng = np.random.default_rng(5)
    d, L = 64, 1100
    raw = rng.standard_normal((L, d)).astype(np.float32)
    n = geometry.num_entries(L, ratio)
    logits = rng.standard_normal((n, geometry.window_len(ratio))).astype(np.float32)
    ref, ref_state, ref_swa = run_stream(raw, ratio, [L], logits, perm_seed=0, swa=True)
    for splits in ([1] * 40 + [L - 40], [3, 4, 7, 255, 256, 257, L - 782], [256] * 4 + [L - 1024],
                   [127, 1, 128, 129, L - 385]):
        out, state, swa = run_stream(raw, ratio, splits, logits, perm_seed=1, swa=True)
        assert np.array_equal(entries_of(out, n), entries_of(ref, n))
        W = geometry.window_len(ratio)
        tail = np.arange(L - W, L)
        assert np.array_equal(state.read(0, tail), raw[tail].astype(np.float64))
        assert np.array_equal(swa.read(0, np.arange(L)), ref_swa.read(0, np.arange(L)))


def test_window_rows_are_rotated_raw_rows():
    rng = np.random.default_rng(6)
    d, L = 576, 300
    raw = rng.standard_normal((L, d)).astype(np.float32)
    logits = rng.standard_normal((geometry.num_entries(L, 4), 8)).astype(np.float32)
    _, _, swa = run_stream(raw, 4, [100, 200], logits, swa=True)
    for p in [0, 1, 99, 100, 255, 256, 299]:
        assert close(swa.read(0, p), rotate(raw[p], p), 1e-6)   # float32 storage
