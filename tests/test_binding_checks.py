"""The Python binding checks every tensor against the sizes the C ABI's
queries give before it passes a pointer: the C entry points receive bare
device pointers and cannot see a short buffer, a wrong shape or a host
tensor.  No GPU needed: every call here raises before any HIP call (the
tensors are host tensors, so one that passed the checks would be refused
as not on the device)."""
import os

import pytest
import torch

import compressed_gemv_amd as cg

pytestmark = pytest.mark.skipif(not os.path.exists(cg.lib_path()), reason="libqgemv.so not built")

N, K, BITS, G = 64, 256, 4, 64


def _group_bufs():
    cb, mb = cg.qgroup_sizes(N, K, BITS, G)
    return torch.zeros(cb, dtype=torch.uint8), torch.zeros(mb // 4, dtype=torch.int32)


def _raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_group_gemv_sizes():
    codes, meta = _group_bufs()
    x = torch.zeros(1, K, dtype=torch.bfloat16)
    _raises("codes", cg.qgemv_group, codes[:-16], meta, N, K, BITS, G, x)
    _raises("meta", cg.qgemv_group, codes, meta[:-1], N, K, BITS, G, x)
    _raises("x", cg.qgemv_group, codes, meta, N, K, BITS, G, torch.zeros(1, K + 32, dtype=torch.bfloat16))
    _raises("x", cg.qgemv_group, codes, meta, N, K, BITS, G, torch.zeros(2, K, dtype=torch.float64))
    _raises("y", cg.qgemv_group, codes, meta, N, K, BITS, G, x, y=torch.zeros(1, N - 1))
    _raises("y", cg.qgemv_group, codes, meta, N, K, BITS, G, x, y=torch.zeros(1, N, dtype=torch.float16))
    # right sizes, host memory: refused as not on the device
    _raises("CUDA", cg.qgemv_group, codes, meta, N, K, BITS, G, x, y=torch.zeros(1, N))


def test_group_unpack_and_pack_sizes():
    codes, meta = _group_bufs()
    _raises("codes", cg.qunpack_group, codes[:8], meta, N, K, BITS, G)
    _raises("CUDA", cg.qunpack_group, codes, meta, N, K, BITS, G)
    _raises("CUDA", cg.qpack_group, torch.zeros(N, K), BITS, G)


def test_grouped_sizes():
    codes, meta = _group_bufs()
    x = torch.zeros(1, K, dtype=torch.bfloat16)
    _raises("codes", cg.qgemv_group_multi, [(codes, meta, N), (codes, meta, 2 * N)], K, BITS, G, x)
    _raises("one output per matrix", cg.qgemv_group_multi, [(codes, meta, N)], K, BITS, G, x,
            ys=[torch.zeros(1, N), torch.zeros(1, N)])


def test_outlier_and_codebook_sizes():
    codes, meta = _group_bufs()
    x = torch.zeros(1, K, dtype=torch.bfloat16)
    idx = torch.zeros(3, dtype=torch.int32)
    _raises("side", cg.qgemv_group_outlier, codes, meta, torch.zeros(N, 2, dtype=torch.int16), idx, N, K, BITS, G, x)
    _raises("idx", cg.qgemv_group_outlier, codes, meta, torch.zeros(N, 3, dtype=torch.int16), idx.long(), N, K, BITS,
            G, x)
    books = torch.zeros(8, 16, dtype=torch.uint8)
    _raises("book_ids", cg.qgemv_group_cb, codes, meta, torch.zeros(N, K // G - 1, dtype=torch.uint8), books, N, K,
            BITS, G, x)
    _raises("books", cg.qgemv_group_cb, codes, meta, torch.zeros(N, K // G, dtype=torch.uint8), books[:, :8], N, K,
            BITS, G, x)


def test_binlr_sizes():
    r = 100
    ub, vb, ws = cg.qbinlr_sizes(N, K, r, 1)
    ubits, vtbits = torch.zeros(ub // 4, dtype=torch.int32), torch.zeros(vb // 4, dtype=torch.int32)
    s1, s2 = torch.zeros(N, dtype=torch.int16), torch.zeros(K, dtype=torch.int16)
    x = torch.zeros(1, K, dtype=torch.bfloat16)
    _raises("ubits", cg.qgemv_binlr, ubits[:-1], vtbits, s1, s2, N, K, r, x)
    _raises("vtbits", cg.qgemv_binlr, ubits, vtbits[:-4], s1, s2, N, K, r, x)
    _raises("s1", cg.qgemv_binlr, ubits, vtbits, s1[:-1], s2, N, K, r, x)
    _raises("s2", cg.qgemv_binlr, ubits, vtbits, s1, s2[:-1], N, K, r, x)
    _raises("ws", cg.qgemv_binlr, ubits, vtbits, s1, s2, N, K, r, x, ws=torch.zeros(ws - 16, dtype=torch.uint8))
    _raises("s1", cg.make_qweight_binlr, ubits, vtbits, s1[:3], s2, N, K, r)
    _raises("U", cg.qpack_binlr, torch.zeros(N, r, dtype=torch.int8), torch.zeros(K, r + 1, dtype=torch.int8))


def test_prefill_sizes():
    codes, meta = _group_bufs()
    _raises("codes", cg.make_qweight_group, codes[:16], meta, N, K, BITS, G)
    _raises("CUDA", cg.make_qweight_group, codes, meta, N, K, BITS, G)
    w = cg.qweight(cg.Q_FMT_GROUP, N, K, BITS, G)   # a bare descriptor (no buffers)
    w._tensors = ()
    _raises("X", cg.qgemm_prefill, w, torch.zeros(4, K + 8, dtype=torch.bfloat16))
    _raises("CUDA", cg.qgemm_prefill, w, torch.zeros(4, K, dtype=torch.bfloat16))


def test_key_cache_sizes():
    Pi = torch.zeros(128, 128, dtype=torch.float64)
    _raises("keys", cg.qtq_quant_keys, torch.zeros(4, 64), 4, Pi, Pi, 0.01, [64] * 8)
    _raises("Pi", cg.qtq_project, Pi, Pi[:64])
    n, H = 10, 2
    codes = torch.zeros(n * H * 12, dtype=torch.int32)
    signs = torch.zeros(n * H, 4, dtype=torch.int32)
    norms = torch.zeros(n * H, dtype=torch.int32)
    Qv = torch.zeros(H, 3, 128)
    _raises("codes", cg.qtq_logits, codes[:-1], signs, norms, n, H, 4, 0.01, [64] * 8, Pi, Pi, Qv)
    _raises("queries", cg.qtq_logits, codes, signs, norms, n, H, 4, 0.01, [64] * 8, Pi, Pi, Qv[:1])
    _raises("weights", cg.qtq_attend, codes, norms, n, H, 3, 0.01, [64] * 8, Pi, torch.zeros(H, 3, n + 1))
