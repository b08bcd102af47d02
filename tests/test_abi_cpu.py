"""The C ABI on the CPU: the library loads, exports every function include/csa.h declares,
and rejects bad host-visible arguments before launching anything (no GPU needed)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")


@pytest.fixture(scope="module")
def csa():
    import compressed_sparse_long_c4a_amd as m
    if not os.path.exists(m.LIB_PATH):
        from compressed_sparse_long_c4a_amd import build
        build.build()
    m.lib()
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree(csa):
    assert set(declared_functions()) == set(csa.EXPORTED)


def test_exports_every_declared_symbol(csa):
    L = ctypes.CDLL(csa.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name


def test_host_helpers(csa):
    L = csa.lib()
    assert L.csa_abi_version() == 1
    assert L.csa_num_entries(4, 1 << 20) == 262144
    assert L.csa_num_entries(128, 1 << 20) == 8192
    assert L.csa_num_entries(4, 1023) == 255
    assert L.csa_num_entries(5, 10) == -1
    assert csa.status_str(csa.EINVAL) == "invalid argument"
    assert L.csa_index_workspace_size(0, 100, 4) == 0
    assert L.csa_index_workspace_size(4, 1 << 20, 2048) > 4 * 262144 * 12
    assert L.csa_sparse_attn_workspace_size(4, 128, 576, 4, 1, 2048, 1 << 20, 128) > 0


def test_validation_rejects_before_launch(csa):
    L = csa.lib()
    c = csa._CCache(1, None, csa.BF16, 576, 64, 10, 1, 8)     # fake (never dereferenced) pointers
    st = csa._CCache(1, None, csa.BF16, 576, 256, 10, 1, 8)
    P = ctypes.pointer
    # bad ratio
    assert L.csa_compress_insert(None, 5, 1, 1, 1, 1, 1, csa.BF16, 1, 1, 1, None, 1e-6, 1e4, 64,
                                 P(st), P(c), None) == csa.EINVAL
    # state dtype must equal the raw dtype
    assert L.csa_compress_insert(None, 4, 1, 1, 1, 1, 1, csa.F32, 1, 1, 1, None, 1e-6, 1e4, 64,
                                 P(st), P(c), None) == csa.EINVAL
    # fp8 cache without scales
    c8 = csa._CCache(1, None, csa.FP8_E4M3, 576, 64, 10, 1, 8)
    assert L.csa_compress_insert(None, 4, 1, 1, 1, 1, 1, csa.BF16, 1, 1, 1, None, 1e-6, 1e4, 64,
                                 P(st), P(c8), None) == csa.EINVAL
    # odd rope dims
    assert L.csa_compress_insert(None, 4, 1, 1, 1, 1, 1, csa.BF16, 1, 1, 1, None, 1e-6, 1e4, 63,
                                 P(st), P(c), None) == csa.EINVAL
    # index: workspace too small, k out of range, unsupported heads
    ic = csa._CCache(1, 1, csa.FP8_E4M3, 128, 64, 10, 1, 8)
    assert L.csa_index_topk(None, 1, 1, 1, 1, 1024, 1, csa.BF16, 64, 1, P(ic), 8, 1, None, 1, 16) \
        == csa.EWORKSPACE
    # csa_index_topk takes its queries in slices: one query's workspace is the least it accepts,
    # while the score and select halves need the whole call's
    one = L.csa_index_workspace_size(1, 1 << 20, 8)
    four = L.csa_index_workspace_size(4, 1 << 20, 8)
    assert one < four
    assert L.csa_index_topk(None, 1, 1, 1, 4, 1 << 20, 1, csa.BF16, 64, 1, P(ic), 8, 1, None, 1, one - 1) \
        == csa.EWORKSPACE
    assert L.csa_index_score(None, 1, 1, 1, 4, 1 << 20, 1, csa.BF16, 64, 1, P(ic), 8, 1, four - 1) \
        == csa.EWORKSPACE
    assert L.csa_index_select(None, 1, 1, 1, 4, 1 << 20, 8, 1, None, 1, four - 1) == csa.EWORKSPACE
    assert L.csa_index_topk(None, 1, 1, 1, 1, 1024, 1, csa.BF16, 64, 1, P(ic), 0, 1, None, 1, 1 << 40) \
        == csa.EINVAL
    assert L.csa_index_topk(None, 1, 1, 1, 1, 1024, 1, csa.BF16, 65, 1, P(ic), 8, 1, None, 1, 1 << 40) \
        == csa.ENOTSUP
    # attention: dim, heads, rope dims, dtype mismatch
    kv = csa._CCache(1, None, csa.BF16, 576, 64, 10, 1, 8)
    sw = csa._CCache(1, None, csa.BF16, 576, 256, 10, 1, 8)
    args = [None, 1, 1, 1, 1, 1024, 1, csa.BF16, 64, P(kv), 4, 1, 16, P(sw), 128, 0.04, 1e4, 64, 1,
            None, 1, 1 << 40]
    # (the unmodified argument list is valid and is never passed: it would launch)
    bad = list(args)
    bad[8] = 129
    assert L.csa_sparse_attn_decode(*bad) == csa.ENOTSUP
    bad = list(args)
    bad[17] = 32
    assert L.csa_sparse_attn_decode(*bad) == csa.ENOTSUP
    sw8 = csa._CCache(1, 1, csa.FP8_E4M3, 576, 256, 10, 1, 8)
    bad = list(args)
    bad[13] = P(sw8)
    assert L.csa_sparse_attn_decode(*bad) == csa.ENOTSUP
    bad = list(args)
    bad[21] = 8
    assert L.csa_sparse_attn_decode(*bad) == csa.EWORKSPACE


def test_compress_many_validation(csa):
    """csa_compress_insert_many rejects an empty or oversized job list and a bad job before
    launching (fake, never dereferenced pointers)."""
    L = csa.lib()
    st = csa._CCache(1, None, csa.BF16, 576, 256, 10, 1, 8)
    out = csa._CCache(1, None, csa.BF16, 576, 64, 10, 1, 8)
    P = ctypes.pointer
    job = csa._CJob(4, 1, csa.BF16, 1, 1, 1, None, 1e-6, 1e4, 64, P(st), P(out), None)
    arr = (csa._CJob * 5)(*([job] * 5))
    assert L.csa_compress_insert_many(None, 1, 1, 1, 1, 0, arr) == csa.EINVAL
    assert L.csa_compress_insert_many(None, 1, 1, 1, 1, 5, arr) == csa.EINVAL
    bad = (csa._CJob * 2)(job, csa._CJob(5, 1, csa.BF16, 1, 1, 1, None, 1e-6, 1e4, 64, P(st), P(out), None))
    assert L.csa_compress_insert_many(None, 1, 1, 1, 1, 2, bad) == csa.EINVAL
    mismatch = (csa._CJob * 1)(csa._CJob(4, 1, csa.F32, 1, 1, 1, None, 1e-6, 1e4, 64, P(st), P(out), None))
    assert L.csa_compress_insert_many(None, 1, 1, 1, 1, 1, mismatch) == csa.EINVAL


def test_q_norm_rope_swa_validation(csa):
    """csa_q_norm_rope_swa rejects bad dtypes, dims, rope spans and window arguments before
    launching (fake, never dereferenced pointers); empty calls launch nothing."""
    L = csa.lib()
    P = ctypes.pointer
    sw = csa._CCache(1, None, csa.BF16, 576, 256, 10, 1, 8)
    sw_bad = csa._CCache(1, None, csa.BF16, 512, 256, 10, 1, 8)
    # (stream, total_q, q_pos, q_in, q_out, q_dtype, heads, dim, gamma, eps, base, rope_dims,
    #  batch, ctx_lens, cu_new, total_new, new_raw, raw_dtype, swa)
    args = [None, 4, 1, 1, 1, csa.BF16, 128, 576, None, 1e-6, 1e4, 64, 4, 1, 1, 4, 1, csa.BF16, P(sw)]
    # (the unmodified argument list is valid and is never passed: it would launch)

    def with_(**kw):
        names = ["stream", "total_q", "q_pos", "q_in", "q_out", "q_dtype", "heads", "dim", "gamma",
                 "eps", "base", "rope_dims", "batch", "ctx_lens", "cu_new", "total_new", "new_raw",
                 "raw_dtype", "swa"]
        a = list(args)
        for k, v in kw.items():
            a[names.index(k)] = v
        return L.csa_q_norm_rope_swa(*a)

    assert with_(q_dtype=csa.FP8_E4M3) == csa.ENOTSUP
    assert with_(dim=580) == csa.ENOTSUP
    assert with_(dim=2048) == csa.ENOTSUP
    assert with_(rope_dims=60) == csa.EINVAL
    assert with_(rope_dims=256) == csa.EINVAL
    assert with_(eps=-1.0) == csa.EINVAL
    assert with_(heads=0) == csa.EINVAL
    assert with_(q_out=None) == csa.EINVAL
    assert with_(swa=P(sw_bad)) == csa.EINVAL          # window cache of another dim
    assert with_(cu_new=None) == csa.EINVAL
    assert with_(raw_dtype=csa.FP8_E4M3) == csa.ENOTSUP
    # nothing to do: returns without launching
    assert with_(total_q=0, q_pos=None, q_in=None, q_out=None, swa=None) == csa.OK
    assert with_(total_q=0, q_pos=None, q_in=None, q_out=None, total_new=0, new_raw=None) == csa.OK


def test_fp4_cache_validation(csa):
    """FP4 caches (CSA_FP4_E2M1): scales required, dim a multiple of 16; accepted as the
    indexer cache and the compressor's entry cache, refused for attention and window caches
    (fake, never dereferenced pointers)."""
    L = csa.lib()
    P = ctypes.pointer
    st = csa._CCache(1, None, csa.BF16, 576, 256, 10, 1, 8)
    st128 = csa._CCache(1, None, csa.BF16, 128, 256, 10, 1, 8)
    out4 = csa._CCache(1, 1, csa.FP4_E2M1, 128, 64, 10, 1, 8)
    out4_noscale = csa._CCache(1, None, csa.FP4_E2M1, 128, 64, 10, 1, 8)
    out4_dim = csa._CCache(1, 1, csa.FP4_E2M1, 584, 64, 10, 1, 8)
    st584 = csa._CCache(1, None, csa.BF16, 584, 256, 10, 1, 8)
    sw4 = csa._CCache(1, 1, csa.FP4_E2M1, 128, 256, 10, 1, 8)
    # compressor: fp4 entry cache needs scales and dim % 16 == 0; fp4 window output refused
    assert L.csa_compress_insert(None, 4, 1, 1, 1, 1, 1, csa.BF16, 1, 1, 1, None, 1e-6, 1e4, 64,
                                 P(st128), P(out4_noscale), None) == csa.EINVAL
    assert L.csa_compress_insert(None, 4, 1, 1, 1, 1, 1, csa.BF16, 1, 1, 1, None, 1e-6, 1e4, 64,
                                 P(st584), P(out4_dim), None) == csa.EINVAL
    assert L.csa_compress_insert(None, 4, 1, 1, 1, 1, 1, csa.BF16, 1, 1, 1, None, 1e-6, 1e4, 64,
                                 P(st128), P(out4), P(sw4)) == csa.ENOTSUP
    # indexer: an fp4 cache passes the cache checks (the small workspace is what fails)
    assert L.csa_index_topk(None, 1, 1, 1, 1, 1024, 1, csa.BF16, 64, 1, P(out4), 8, 1, None, 1, 16) \
        == csa.EWORKSPACE
    assert L.csa_index_topk(None, 1, 1, 1, 1, 1024, 1, csa.BF16, 64, 1, P(out4_noscale), 8, 1, None,
                            1, 1 << 40) == csa.EINVAL
    # attention: fp4 main / window caches are not supported
    kv4 = csa._CCache(1, 1, csa.FP4_E2M1, 576, 64, 10, 1, 8)
    sw4a = csa._CCache(1, 1, csa.FP4_E2M1, 576, 256, 10, 1, 8)
    assert L.csa_sparse_attn_decode(None, 1, 1, 1, 1, 1024, 1, csa.BF16, 64, P(kv4), 4, 1, 16, P(sw4a),
                                    128, 0.04, 1e4, 64, 1, None, 1, 1 << 40) == csa.ENOTSUP
    # query norm: an fp4 window cache is refused
    assert L.csa_q_norm_rope_swa(None, 4, 1, 1, 1, csa.BF16, 128, 576, None, 1e-6, 1e4, 64, 4, 1, 1,
                                 4, 1, csa.BF16, P(sw4a)) == csa.ENOTSUP
    del st


def test_read_probe_validation(csa):
    """The read probe refuses a NULL buffer or sink, an empty or ragged size and a misaligned
    buffer before launching (fake, never dereferenced pointers)."""
    L = csa.lib()
    assert L.csa_read_probe_sink_words() > 0
    assert L.csa_read_probe(None, None, 1024, 16) == csa.EINVAL
    assert L.csa_read_probe(None, 16, 1024, None) == csa.EINVAL
    assert L.csa_read_probe(None, 16, 0, 16) == csa.EINVAL
    assert L.csa_read_probe(None, 16, 1000, 16) == csa.EINVAL
    assert L.csa_read_probe(None, 8, 1024, 16) == csa.EINVAL


def test_compress_index_score_validation(csa):
    """csa_compress_index_score checks the compressor jobs, the index arguments and that the
    indexer-key job writes the indexer cache, before launching (fake pointers)."""
    L = csa.lib()
    P = ctypes.pointer
    st = csa._CCache(1, None, csa.BF16, 576, 256, 10, 1, 8)
    kv = csa._CCache(1, 1, csa.FP8_E4M3, 576, 64, 10, 1, 8)
    ist = csa._CCache(2, None, csa.BF16, 128, 256, 10, 3, 8)
    idx = csa._CCache(4, 5, csa.FP8_E4M3, 128, 64, 10, 6, 8)
    other = csa._CCache(7, 5, csa.FP8_E4M3, 128, 64, 10, 6, 8)
    main = csa._CJob(4, 1, csa.BF16, 1, 1, 1, None, 1e-6, 1e4, 64, P(st), P(kv), None)
    ij = csa._CJob(4, 1, csa.BF16, 1, 1, 1, None, 1e-6, 1e4, 64, P(ist), P(idx), None)
    ij_other = csa._CJob(4, 1, csa.BF16, 1, 1, 1, None, 1e-6, 1e4, 64, P(ist), P(other), None)
    jobs = (csa._CJob * 2)(main, ij)

    def call(jobs_arr, n, idx_job, ws_bytes=1 << 40, cache=idx):
        return L.csa_compress_index_score(None, 1, 1, 1, 1, n, jobs_arr, idx_job, 1, 1, 1, 1024, 1,
                                          csa.BF16, 64, 1, P(cache), 8, 1, ws_bytes)

    assert call(jobs, 2, 2) == csa.EINVAL            # idx_job out of range
    assert call(jobs, 2, -1) == csa.EINVAL
    assert call(jobs, 2, 0) == csa.EINVAL            # job 0 does not write the indexer cache
    assert call((csa._CJob * 2)(main, ij_other), 2, 1) == csa.EINVAL
    assert call(jobs, 2, 1, ws_bytes=16) == csa.EWORKSPACE
    assert call(jobs, 0, 0) == csa.EINVAL            # no job


def test_compress_index_score_launch_count(csa):
    """The library's own choice between one launch (compressors inside the score launch) and
    two (compressor, then score): host-only, nothing is launched."""
    L = csa.lib()
    P = ctypes.pointer
    st = csa._CCache(1, None, csa.BF16, 576, 256, 10, 1, 8)
    kv = csa._CCache(1, 1, csa.FP8_E4M3, 576, 64, 10, 1, 8)
    idx = csa._CCache(4, 5, csa.FP8_E4M3, 128, 64, 10, 6, 8)

    def jobs(entries, ratio=4):
        main = csa._CJob(ratio, 1, csa.BF16, 1, entries, 1, None, 1e-6, 1e4, 64, P(st), P(kv), None)
        ij = csa._CJob(4, 1, csa.BF16, 1, entries, 1, None, 1e-6, 1e4, 64, P(st), P(idx), None)
        return (csa._CJob * 2)(main, ij)

    n = L.csa_compress_index_score_launches
    assert n(2, jobs(1), 1, 4, 4, csa.BF16, 64) == 1          # decode: one launch
    assert n(2, jobs(1), 1, 4, 4, csa.F32, 64) == 2           # float32 queries
    assert n(2, jobs(1), 1, 4, 4, csa.BF16, 65) == 2          # more than 64 indexer heads
    assert n(2, jobs(1024), 1, 4096, 4096, csa.BF16, 64) == 2  # prefill chunk: 4M (entry, query) pairs
    assert n(2, jobs(1, ratio=128), 1, 4, 4, csa.BF16, 64) == 2
    assert n(2, jobs(0), 1, 0, 4, csa.BF16, 64) == 1          # nothing to compress: the score only
    assert n(2, jobs(1), 1, 4, 0, csa.BF16, 64) == 1          # no queries: the compressor only
    assert n(2, jobs(1), 2, 4, 4, csa.BF16, 64) == csa.EINVAL
    assert n(2, None, 1, 4, 4, csa.BF16, 64) == csa.EINVAL


def test_noalloc_attention_refuses_scratch_beyond_its_array(csa):
    """csa_sparse_attn_decode_noalloc serves at most 16 MiB of split partials from the library's
    own array; a larger request returns CSA_EWORKSPACE before any HIP call (fake pointers)."""
    L = csa.lib()
    P = ctypes.pointer
    kv = csa._CCache(1, 1, csa.FP8_E4M3, 576, 64, 10, 1, 8)
    swa = csa._CCache(2, 2, csa.FP8_E4M3, 576, 256, 10, 1, 8)
    # 256 queries x 128 heads x 2,176 rows: far more split partials than 16 MiB
    need = L.csa_sparse_attn_workspace_size(256, 128, 576, 4, 1, 2048, 1 << 20, 128)
    assert need > 16 << 20
    st = L.csa_sparse_attn_decode_noalloc(None, 1, 1, 1, 256, 1 << 20, 1, csa.BF16, 128, P(kv), 4, 1, 2048,
                                          P(swa), 128, 0.04, 1e4, 64, 1, None)
    assert st == csa.EWORKSPACE
    # and the usual argument checks come first
    assert L.csa_sparse_attn_decode_noalloc(None, 1, 1, 1, 4, 1 << 20, 1, csa.BF16, 128, P(kv), 4, 1, 2048,
                                            P(swa), 128, 0.04, 1e4, 64, None, None) == csa.EINVAL
