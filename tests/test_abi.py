"""The C-ABI library loads, exports every entry point include/qgemv.h
declares, answers the host-only size queries and rejects bad arguments with
the documented status codes before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

import compressed_gemv_amd as cg

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "qgemv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(cg.lib_path()):
        import __graft_entry__
        __graft_entry__.build()
    return cg.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) == 32, names
    for n in names:
        assert hasattr(lib, n), n


def test_versions_and_status_strings(lib):
    assert cg.q_abi_version() == 3
    assert cg.q_format_version() == 1
    for st in (0, -1, -2, -3, -4, -5, -6):
        s = cg.q_status_str(st)
        assert s and s != "unknown status"
    assert cg.q_status_str(-99) == "unknown status"


def test_size_queries(lib):
    assert cg.qgroup_sizes(28672, 8192, 4, 64) == (117_440_512, 14_680_064)
    assert cg.qgroup_sizes(512, 512, 4, 32) == (131_072, 32_768)
    for b in (2, 3, 5, 6):
        c, m = cg.qgroup_sizes(8192, 8192, b, 32)
        assert c == 8192 * 8192 * b // 8 and m == 8192 * 256 * 4
    ub, vb, ws = cg.qbinlr_sizes(28672, 8192, 4096, 1)
    # workspace: stage-2 table (4 B per entry of t, whole 512-entry steps)
    # + (C, V) partials of one stage-1 workgroup per 16 rows, 16-byte rounded
    assert ub == 14_680_064 and vb == 4_194_304 and ws == 4096 * 4 + 256 * 8
    ub, vb, ws = cg.qbinlr_sizes(10, 40, 3, 2)   # padding to 4-word rows
    assert ub == 10 * 16 and vb == 3 * 16 and ws == 2 * (2048 + 16)
    w = cg.qweight(cg.Q_FMT_BINLR, 28672, 8192, 0, 0, None, None, 4096, None, None, None, None)
    assert cg.qgemm_prefill_ws(w, 512) == 512 * 4096 * 2
    # short reductions keep T in fp32 (split-precision passes)
    w = cg.qweight(cg.Q_FMT_BINLR, 1000, 256, 0, 0, None, None, 300, None, None, None, None)
    assert cg.qgemm_prefill_ws(w, 70) == 70 * 384 * 4
    w = cg.qweight(cg.Q_FMT_GROUP, 28672, 8192, 4, 64, None, None, 0, None, None, None, None)
    assert cg.qgemm_prefill_ws(w, 512) == 0


@pytest.mark.parametrize("args", [
    (100, 100, 4, 32),      # K not a multiple of the group
    (100, 128, 7, 32),      # bits out of range
    (100, 128, 4, 48),      # group not 32/64
    (0, 128, 4, 32),        # empty
])
def test_size_query_rejects(lib, args):
    c, m = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.qgroup_sizes(*args, ctypes.byref(c), ctypes.byref(m)) == cg.Q_EINVAL


def test_entry_points_validate_before_touching_the_gpu(lib):
    P = ctypes.c_void_p
    good, odd = P(0x10000), P(0x10004)
    s = P(0)
    # null pointers
    assert lib.qgemv_group(P(0), good, 64, 128, 4, 32, good, cg.Q_BF16, 1, good, cg.Q_F32, s) == cg.Q_EINVAL
    # batch out of range
    assert lib.qgemv_group(good, good, 64, 128, 4, 32, good, cg.Q_BF16, 17, good, cg.Q_F32, s) == cg.Q_EINVAL
    # misaligned codes
    assert lib.qgemv_group(odd, good, 64, 128, 4, 32, good, cg.Q_BF16, 1, good, cg.Q_F32, s) == cg.Q_EALIGN
    # x must be 16-byte aligned (the header's rule); y 4-byte aligned is enough
    assert lib.qgemv_group(good, good, 64, 128, 4, 32, odd, cg.Q_BF16, 1, good, cg.Q_F32, s) == cg.Q_EALIGN
    assert lib.qgemv_group(good, good, 64, 128, 4, 32, P(0x10008), cg.Q_BF16, 1, good, cg.Q_F32, s) == cg.Q_EALIGN
    # unsupported: fp32 activations with B > 1, K beyond the register-resident limit
    assert lib.qgemv_group(good, good, 64, 128, 4, 32, good, cg.Q_F32, 2, good, cg.Q_F32, s) == cg.Q_EUNSUPPORTED
    assert lib.qgemv_group(good, good, 64, 131072, 4, 32, good, cg.Q_BF16, 1, good, cg.Q_F32, s) == cg.Q_EUNSUPPORTED
    assert lib.qgemv_group(good, good, 64, 65536, 4, 32, good, cg.Q_F32, 1, good, cg.Q_F32, s) == cg.Q_EUNSUPPORTED
    # bad dtype
    assert lib.qgemv_group(good, good, 64, 128, 4, 32, good, 7, 1, good, cg.Q_F32, s) == cg.Q_EINVAL
    # packer: bad shape, alignment
    assert lib.qpack_group(good, 64, 100, 4, 32, good, good, s) == cg.Q_EINVAL
    assert lib.qpack_group(good, 64, 128, 4, 32, odd, good, s) == cg.Q_EALIGN
    # binary: workspace too small
    assert lib.qgemv_binlr(good, good, good, good, 64, 128, 16, good, cg.Q_BF16, 1, good, cg.Q_F32,
                           good, 4, s) == cg.Q_EWORKSPACE
    assert lib.qgemv_binlr(good, good, good, good, 64, 128, 16, good, cg.Q_BF16, 1, good, cg.Q_F32,
                           P(0), 1 << 20, s) == cg.Q_EWORKSPACE
    assert lib.qpack_binlr(good, good, 64, 128, 0, good, good, s) == cg.Q_EINVAL
    # streaming-read reference: sizes and alignment
    assert lib.qstream_read(good, 100, good, s) == cg.Q_EINVAL
    assert lib.qstream_read(odd, 128, good, s) == cg.Q_EALIGN
    # binary without a workspace argument: the scratch array's limit, nulls, alignment
    assert lib.qgemv_binlr_noalloc(good, good, good, good, 64, 128, 65536, good, cg.Q_BF16, 16, good, cg.Q_F32,
                                   s) == cg.Q_EUNSUPPORTED
    assert lib.qgemv_binlr_noalloc(good, P(0), good, good, 64, 128, 16, good, cg.Q_BF16, 1, good, cg.Q_F32,
                                   s) == cg.Q_EINVAL
    assert lib.qgemv_binlr_noalloc(odd, good, good, good, 64, 128, 16, good, cg.Q_BF16, 1, good, cg.Q_F32,
                                   s) == cg.Q_EALIGN
    assert lib.qgemv_binlr_noalloc(good, good, good, good, 64, 128, 16, good, cg.Q_BF16, 17, good, cg.Q_F32,
                                   s) == cg.Q_EINVAL
    # grouped GEMV: count and per-matrix checks
    mats = (cg.qgroup_mat * 5)(*[cg.qgroup_mat(0x10000, 0x10000, 64, 0x10000) for _ in range(5)])
    assert lib.qgemv_group_multi(mats, 5, 128, 4, 32, good, cg.Q_BF16, 1, cg.Q_F32, s) == cg.Q_EINVAL
    assert lib.qgemv_group_multi(mats, 0, 128, 4, 32, good, cg.Q_BF16, 1, cg.Q_F32, s) == cg.Q_EINVAL
    mats[1].codes = 0x10004
    assert lib.qgemv_group_multi(mats, 2, 128, 4, 32, good, cg.Q_BF16, 1, cg.Q_F32, s) == cg.Q_EALIGN
    mats[1].codes = 0x10000
    mats[2].N = 0
    assert lib.qgemv_group_multi(mats, 3, 128, 4, 32, good, cg.Q_BF16, 1, cg.Q_F32, s) == cg.Q_EINVAL
    assert lib.qgemv_group_multi(mats, 2, 100, 4, 32, good, cg.Q_BF16, 1, cg.Q_F32, s) == cg.Q_EINVAL
    # outlier columns: count limits, workspace, alignment
    assert cg.qgroup_outlier_ws(8192, 8) == (8192 + 256) * 4
    assert cg.qgroup_outlier_ws(100, 3) == (100 + 4) * 4
    n = ctypes.c_size_t()
    assert lib.qgroup_outlier_ws(128, 65, ctypes.byref(n)) == cg.Q_EINVAL
    assert lib.qgroup_outlier_ws(32, 33, ctypes.byref(n)) == cg.Q_EINVAL
    assert lib.qpack_group_outlier(good, 64, 128, 4, 32, 4, good, good, good, good, good, 16, s) == cg.Q_EWORKSPACE
    assert lib.qpack_group_outlier(good, 64, 128, 4, 32, 4, good, good, P(0x10001), good, good, 1 << 20,
                                   s) == cg.Q_EALIGN
    assert lib.qpack_group_outlier(good, 64, 128, 4, 32, 4, good, good, P(0), good, good, 1 << 20,
                                   s) == cg.Q_EINVAL
    assert lib.qgemv_group_outlier(good, good, good, good, 65, 64, 128, 4, 32, good, cg.Q_BF16, 1, good,
                                   cg.Q_F32, s) == cg.Q_EINVAL
    assert lib.qgemv_group_outlier(good, good, P(0), good, 2, 64, 128, 4, 32, good, cg.Q_BF16, 1, good,
                                   cg.Q_F32, s) == cg.Q_EINVAL
    assert lib.qgemv_group_outlier(good, good, good, P(0x10002), 2, 64, 128, 4, 32, good, cg.Q_BF16, 1, good,
                                   cg.Q_F32, s) == cg.Q_EALIGN
    wo = cg.qweight(cg.Q_FMT_GROUP, 64, 128, 4, 32, 0x10000, 0x10000, 0, None, None, None, None, 0x10000,
                    0x10000, 65)
    assert lib.qgemm_prefill(ctypes.byref(wo), good, cg.Q_BF16, 16, good, cg.Q_F32, P(0), 0, s) == cg.Q_EINVAL
    # prefill
    w = cg.qweight(cg.Q_FMT_GROUP, 64, 128, 4, 32, 0x10000, 0x10000, 0, None, None, None, None)
    assert lib.qgemm_prefill(ctypes.byref(w), good, cg.Q_F32, 16, good, cg.Q_F32, P(0), 0, s) == cg.Q_EUNSUPPORTED
    w.format = 9
    assert lib.qgemm_prefill(ctypes.byref(w), good, cg.Q_BF16, 16, good, cg.Q_F32, P(0), 0, s) == cg.Q_EINVAL
    wb = cg.qweight(cg.Q_FMT_BINLR, 64, 128, 0, 0, None, None, 16, 0x10000, 0x10000, 0x10000, 0x10000)
    assert lib.qgemm_prefill(ctypes.byref(wb), good, cg.Q_BF16, 16, good, cg.Q_F32, P(0), 0, s) == cg.Q_EWORKSPACE
    # 32-bit tile offsets: 256 rows of K bf16 inputs, 256 rows of the padded
    # rank in fp32, and the tile count must fit
    wk = cg.qweight(cg.Q_FMT_GROUP, 1, 1 << 23, 2, 32, 0x10000, 0x10000, 0, None, None, None, None)
    assert lib.qgemm_prefill(ctypes.byref(wk), good, cg.Q_BF16, 16, good, cg.Q_F32, P(0), 0, s) == cg.Q_EUNSUPPORTED
    wk.K = (1 << 23) - 32
    assert lib.qgemm_prefill(ctypes.byref(wk), P(0), cg.Q_BF16, 16, good, cg.Q_F32, P(0), 0, s) == cg.Q_EINVAL
    wr = cg.qweight(cg.Q_FMT_BINLR, 1, 64, 0, 0, None, None, 1 << 22, 0x10000, 0x10000, 0x10000, 0x10000)
    assert lib.qgemm_prefill(ctypes.byref(wr), good, cg.Q_BF16, 16, good, cg.Q_F32, good, 1 << 40,
                             s) == cg.Q_EUNSUPPORTED
    wt = cg.qweight(cg.Q_FMT_GROUP, 32768, 32, 2, 32, 0x10000, 0x10000, 0, None, None, None, None)
    assert lib.qgemm_prefill(ctypes.byref(wt), good, cg.Q_BF16, 1 << 30, good, cg.Q_F32, P(0), 0,
                             s) == cg.Q_EUNSUPPORTED   # 2^24 x 256 tiles of 64 x 128
    assert lib.qgemm_prefill(ctypes.byref(wt), P(0), cg.Q_BF16, 1 << 20, good, cg.Q_F32, P(0), 0,
                             s) == cg.Q_EINVAL         # 2^14 x 256 tiles: past the size checks
    # batched GEMV: B * K * 2 bytes of activations addressed in 32 bits
    assert lib.qgemv_group(good, good, 1, 1 << 26, 2, 32, good, cg.Q_BF16, 16, good, cg.Q_F32,
                           s) == cg.Q_EUNSUPPORTED
    assert lib.qgemv_group(good, good, 1, 1 << 26, 2, 32, good, cg.Q_BF16, 1, good, cg.Q_F32,
                           s) == cg.Q_EUNSUPPORTED   # batch 1: K past its own limit
    # codebook prefill: ids present, no outlier columns with books, widths 2..4
    wc = cg.qweight(cg.Q_FMT_GROUP, 64, 128, 4, 32, 0x10000, 0x10000, 0, None, None, None, None, None, None, 0,
                    None, 0x10000, 8)
    assert lib.qgemm_prefill(ctypes.byref(wc), good, cg.Q_BF16, 16, good, cg.Q_F32, P(0), 0, s) == cg.Q_EINVAL
    wc.book_ids = 0x10000
    wc.bits = 5
    assert lib.qgemm_prefill(ctypes.byref(wc), good, cg.Q_BF16, 16, good, cg.Q_F32, P(0), 0, s) == cg.Q_EINVAL
    wc.bits, wc.n_books = 4, 17
    assert lib.qgemm_prefill(ctypes.byref(wc), good, cg.Q_BF16, 16, good, cg.Q_F32, P(0), 0, s) == cg.Q_EINVAL
    wc.n_books, wc.n_out, wc.side, wc.oidx = 8, 2, 0x10000, 0x10000
    assert lib.qgemm_prefill(ctypes.byref(wc), good, cg.Q_BF16, 16, good, cg.Q_F32, P(0), 0, s) == cg.Q_EINVAL
    # codebooks: widths 2..4, 1..16 books, books and ids present
    assert lib.qpack_group_cb(good, 64, 128, 5, 32, good, 8, good, good, good, s) == cg.Q_EINVAL
    assert lib.qpack_group_cb(good, 64, 128, 4, 32, good, 0, good, good, good, s) == cg.Q_EINVAL
    assert lib.qpack_group_cb(good, 64, 128, 4, 32, good, 17, good, good, good, s) == cg.Q_EINVAL
    assert lib.qpack_group_cb(good, 64, 128, 4, 32, P(0), 8, good, good, good, s) == cg.Q_EINVAL
    assert lib.qpack_group_cb(good, 64, 128, 4, 32, good, 8, good, good, P(0), s) == cg.Q_EINVAL
    assert lib.qpack_group_cb(good, 64, 128, 4, 32, good, 8, odd, good, good, s) == cg.Q_EALIGN
    assert lib.qgemv_group_cb(good, good, P(0), good, 8, 64, 128, 4, 32, good, cg.Q_BF16, 1, good, cg.Q_F32,
                              s) == cg.Q_EINVAL
    assert lib.qgemv_group_cb(good, good, good, good, 8, 64, 128, 6, 32, good, cg.Q_BF16, 1, good, cg.Q_F32,
                              s) == cg.Q_EINVAL
    assert lib.qgemv_group_cb(good, odd, good, good, 8, 64, 128, 2, 32, good, cg.Q_BF16, 1, good, cg.Q_F32,
                              s) == cg.Q_EALIGN
    assert lib.qgemv_group_cb(good, good, good, good, 8, 64, 128, 3, 64, good, cg.Q_F32, 4, good, cg.Q_F32,
                              s) == cg.Q_EUNSUPPORTED


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_default_codebooks_match_the_oracle(lib, bits):
    """The library's default dictionary is the one the oracle defines."""
    from oracle import codebook
    assert np.array_equal(cg.qcodebook_default(bits).numpy(), codebook.default_dictionary(bits))


def test_default_codebooks_reject_widths(lib):
    buf = (ctypes.c_uint8 * 256)()
    assert lib.qcodebook_default(5, buf, None) == cg.Q_EINVAL
    assert lib.qcodebook_default(4, None, None) == cg.Q_EINVAL


@pytest.mark.parametrize("d", [64, 128])
def test_key_centroids_and_rotation_match_the_oracle(lib, d):
    """The library's Lloyd-Max tables and Gram-Schmidt rotation equal the
    oracle's (incomplete-beta centroids, numpy QR with the sign fix)."""
    from oracle import turboquant as tq
    for m in (1, 2, 3, 4):
        dl, t = cg.qtq_centroids(d, m)
        d2, t2 = tq.stored_table(tq.lloyd_max(d, m))
        assert np.float32(dl) == d2 and np.array_equal(t, t2), (m, dl, d2)
    G = np.random.default_rng(d).standard_normal((d, d))
    assert np.abs(cg.qtq_rotation(G) - tq.rotation(G)).max() < 1e-11


def test_key_cache_entry_points_validate(lib):
    P = ctypes.c_void_p
    good, odd = P(0x10000), P(0x10004)
    s = P(0)
    t = (ctypes.c_uint8 * 8)(1, 24, 42, 57, 71, 86, 104, 127)
    bad = (ctypes.c_uint8 * 8)(0, 24, 42, 57, 71, 86, 104, 127)
    f = ctypes.c_float
    assert lib.qtq_quant_keys(good, 16, 5, good, good, f(0.003), t, good, good, good, s) == cg.Q_EINVAL
    assert lib.qtq_quant_keys(good, 16, 4, good, good, f(0.0), t, good, good, good, s) == cg.Q_EINVAL
    assert lib.qtq_quant_keys(good, 16, 4, good, good, f(0.003), bad, good, good, good, s) == cg.Q_EINVAL
    assert lib.qtq_quant_keys(good, 16, 4, odd, good, f(0.003), t, good, good, good, s) == cg.Q_EALIGN
    assert lib.qtq_quant_keys(good, 1 << 26, 4, good, good, f(0.003), t, good, good, good, s) == cg.Q_EUNSUPPORTED
    n = ctypes.c_size_t()
    assert lib.qtq_logits_ws(2, 4, ctypes.byref(n)) == 0 and n.value == 2 * 4 * 132 * 4
    assert lib.qtq_logits(good, good, good, 64, 2, 4, f(0.003), t, good, good, good, 4, good, good, 16,
                          s) == cg.Q_EWORKSPACE
    assert lib.qtq_logits(good, good, good, 64, 2, 4, f(0.003), t, good, good, good, 4, good, P(0), 1 << 20,
                          s) == cg.Q_EWORKSPACE
    assert lib.qtq_logits(good, good, good, 64, 0, 4, f(0.003), t, good, good, good, 4, good, good, 1 << 20,
                          s) == cg.Q_EINVAL
    assert lib.qtq_logits(good, good, good, 64, 2, 4, f(0.003), t, good, good, good, 4, good, P(0x10008), 1 << 20,
                          s) == cg.Q_EALIGN
    cb, sb, nb = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.qtq_sizes(1000, 4, ctypes.byref(cb), ctypes.byref(sb), ctypes.byref(nb)) == 0
    assert (cb.value, sb.value, nb.value) == (48000, 16000, 4000)
    buf = (ctypes.c_uint8 * 16)()
    assert lib.qtq_centroids(2, 3, ctypes.byref(f()), buf) == cg.Q_EINVAL
    assert lib.qtq_centroids(128, 5, ctypes.byref(f()), buf) == cg.Q_EINVAL
