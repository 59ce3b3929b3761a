"""The Python binding refuses tensors that do not fit the entry point it calls.

CPU only.  Every call below passes CPU tensors, so a call that got past its
checks would fail at the last one (GPU memory required) rather than reach the
library: each case asserts the status of the specific check it breaks.  The
shapes, dtypes and layouts are those of the C ABI in include/kvsel.h.
"""

import pytest
import torch

from query_guided_kv_amd import kvsel as K

SHAPE, DTYPE, UNSUP, WS, NULL = K.ERR_SHAPE, K.ERR_DTYPE, K.ERR_UNSUPPORTED, K.ERR_WORKSPACE, K.ERR_NULL


@pytest.fixture(scope="module", autouse=True)
def lib():
    import os
    if not os.path.exists(K.LIB_PATH):
        from query_guided_kv_amd import build
        build.build()
    return K.load()


def refused(status, fn, *args, **kw):
    with pytest.raises(K.KvselError) as e:
        fn(*args, **kw)
    assert e.value.status == status, str(e.value)


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


B, N, H, D, Hq, T, U = 2, 1024, 8, 128, 32, 1, 256


def cache():
    return bf(B, N, H, D), bf(B, N, H, D)


def test_score_query_must_fit_the_cache():
    k, _ = cache()
    refused(SHAPE, K.score, bf(B + 1, T, Hq, D), k, U)          # more queries than caches
    refused(SHAPE, K.score, bf(B, T, Hq, D), bf(B + 2, N, H, D), U)   # more caches than queries
    refused(SHAPE, K.score, bf(B, T, Hq, 64), k, U)             # head dim
    refused(SHAPE, K.score, bf(B, T, 30, D), k, U)              # Hq not a multiple of H
    refused(SHAPE, K.score, bf(B, T, Hq), k, U)                 # not 4-D
    refused(DTYPE, K.score, torch.zeros(B, T, Hq, D), k, U)     # fp32 query, bf16 cache
    refused(UNSUP, K.score, bf(B, Hq, T, D).transpose(1, 2), k, U)   # not contiguous
    refused(SHAPE, K.score, bf(B, T, Hq, D), k, 300)            # unit_len does not divide N
    refused(SHAPE, K.score, bf(B, T, Hq, D), k, U, part_out=torch.zeros(B, Hq, T, 3, 2))
    refused(DTYPE, K.score, bf(B, T, Hq, D), k, U, part_out=torch.zeros(B, Hq, T, 4, 2,
                                                                       dtype=torch.float64))
    refused(UNSUP, K.score, bf(B, T, Hq, D), k, U)              # everything fits: CPU memory


def test_score_reposition_delta():
    k, _ = cache()
    q = bf(B, T, Hq, D)
    refused(DTYPE, K.score_reposition, q, k, torch.zeros(4, dtype=torch.int32), U, U)
    refused(SHAPE, K.score_reposition, q, k, torch.zeros(5, dtype=torch.int64), U, U)
    refused(SHAPE, K.score_reposition, q, k, torch.zeros(B + 1, 4, dtype=torch.int64), U, U)
    refused(UNSUP, K.score_reposition, q, k, torch.zeros(8, dtype=torch.int64)[::2], U, U)
    refused(SHAPE, K.score_reposition, q, k, torch.zeros(4, dtype=torch.int64), U, U,
            k_out=bf(B, N // 2, H, D))
    refused(UNSUP, K.score_reposition, q, k, torch.zeros(B, 4, dtype=torch.int64), U, U)


def test_reposition_out_and_delta():
    k, _ = cache()
    d = torch.zeros(4, dtype=torch.int64)
    refused(SHAPE, K.reposition, k, d, U, out=bf(B, N, H, D).transpose(0, 1).contiguous()
            .transpose(0, 1))                                   # other strides
    refused(DTYPE, K.reposition, k, d, U, out=torch.zeros(B, N, H, D))
    refused(DTYPE, K.reposition, k, d.int(), U)
    refused(UNSUP, K.reposition, k, d, U)


def test_score_units_list():
    k, _ = cache()
    q = bf(B, 32, 28, D)
    k4 = bf(B, N, 4, D)
    refused(DTYPE, K.score_units, q, k4, torch.zeros(B, 3, dtype=torch.int64), U)
    refused(SHAPE, K.score_units, q, k4, torch.zeros(B + 1, 3, dtype=torch.int32), U)
    refused(SHAPE, K.score_units, q, k4, torch.zeros(B, 3, dtype=torch.int32), U,
            delta=torch.zeros(4, dtype=torch.int64))
    refused(UNSUP, K.score_units, q, k4, torch.zeros(B, 3, dtype=torch.int32), U)


def test_aggregate_inputs():
    k, v = cache()
    q = bf(B, T, Hq, D)
    rm = torch.zeros(B, Hq, T)
    part = torch.zeros(B, Hq, T, N // U, 2)
    refused(SHAPE, K.aggregate, U, part=torch.zeros(B, Hq, T, 3, 2), k=k)
    refused(DTYPE, K.aggregate, U, part=part.double(), k=k)
    refused(SHAPE, K.aggregate, U, 3, part=part, k=k)           # group does not divide B
    refused(NULL, K.aggregate, U, signal="vnorm", q=q, k=k, row_max=rm, row_sum=rm)
    refused(SHAPE, K.aggregate, U, signal="vnorm", q=q, k=k, v=bf(B, N // 2, H, D),
            row_max=rm, row_sum=rm)
    refused(DTYPE, K.aggregate, U, signal="vnorm", q=q, k=k, v=v, row_max=rm.double(),
            row_sum=rm)
    refused(SHAPE, K.aggregate, U, q=bf(B + 1, T, Hq, D), k=k, row_max=rm, row_sum=rm)
    refused(NULL, K.aggregate, U, part=part, k=k, accumulate=True)
    refused(SHAPE, K.aggregate, U, part=part, k=k, out=torch.zeros(B, 5))
    refused(WS, K.aggregate, U, part=part, k=k, ws=torch.zeros(4, dtype=torch.uint8))
    refused(UNSUP, K.aggregate, U, part=part, k=k)


def test_topk_order_take_scores_and_lists():
    s = torch.zeros(2, 10)
    refused(DTYPE, K.topk, s.double(), 3)
    refused(UNSUP, K.topk, torch.zeros(10, 2).t(), 3)
    refused(SHAPE, K.topk, torch.zeros(20), 3)
    refused(SHAPE, K.topk, s, 3, idx_out=torch.zeros(2, 4, dtype=torch.int32))
    refused(UNSUP, K.topk, s, 3)
    i = torch.zeros(2, 3, dtype=torch.int32)
    refused(DTYPE, K.order, s, i.long())
    refused(SHAPE, K.order, s, torch.zeros(3, 3, dtype=torch.int32))
    refused(UNSUP, K.order, s, i)
    refused(DTYPE, K.take, i.long(), i)
    refused(SHAPE, K.take, i, torch.zeros(3, 3, dtype=torch.int32))
    refused(UNSUP, K.take, i, i)
    refused(DTYPE, K.unit_fractions, i.long(), 256, 4)
    refused(UNSUP, K.unit_fractions, i, 256, 4)
    refused(DTYPE, K.slot_starts, i.long(), 256)
    refused(UNSUP, K.slot_starts, i, 256)


def test_gather_index_lists():
    k, v = cache()
    idx = torch.zeros(B, 2, dtype=torch.int32)
    refused(DTYPE, K.gather, k, v, idx.long(), U)               # torch.topk's int64
    refused(SHAPE, K.gather, k, v, torch.zeros(B + 1, 2, dtype=torch.int32), U)
    refused(SHAPE, K.gather, k, v, idx, U, idx_group=3)
    refused(SHAPE, K.gather, k, v, torch.zeros(2, dtype=torch.int32), U)
    refused(SHAPE, K.gather, k, bf(B, N, H, D).transpose(0, 1).contiguous().transpose(0, 1),
            idx, U)                                             # v with other strides
    refused(DTYPE, K.gather, k, v, idx, U, src_start=torch.zeros(4, dtype=torch.int32))
    refused(SHAPE, K.gather, k, v, idx, U, k_out=bf(B, 3 * U, H, D))
    refused(UNSUP, K.gather, k, v, idx, U)


def test_decode_and_gather_decode_queries():
    k, v = cache()
    idx = torch.zeros(B, 2, dtype=torch.int32)
    q = bf(B, T, Hq, D)
    # the case of more caches than query blocks: the kernels would run B
    # instances and read q and write out past their ends
    refused(SHAPE, K.gather_decode, bf(B - 1, T, Hq, D), k, v, idx, U)
    refused(SHAPE, K.decode_attn, bf(B - 1, T, Hq, D), [(k, v)])
    refused(DTYPE, K.gather_decode, q, k, v, idx.long(), U)
    refused(DTYPE, K.gather_decode, q.float(), k, v, idx, U)
    refused(UNSUP, K.gather_decode, bf(B, Hq, T, D).transpose(1, 2), k, v, idx, U)
    refused(SHAPE, K.gather_decode, q, k, bf(B, N, H // 2, D), idx, U)
    refused(SHAPE, K.gather_decode, q, k, v, idx, U, extra=[(k, bf(B, N // 2, H, D))])
    refused(SHAPE, K.gather_decode, q, k, v, idx, U, out=torch.zeros(B, T, Hq, D + 1))
    refused(SHAPE, K.decode_attn, q, [])
    refused(SHAPE, K.decode_attn, q, [(k, v), (bf(B, N, 4, D), bf(B, N, 4, D))])
    refused(UNSUP, K.gather_decode, q, k, v, idx, U)
    refused(UNSUP, K.decode_attn, q, [(k, v)])


def test_index_attn_positions():
    k, v = cache()
    q = bf(B, 5, Hq, D)
    refused(DTYPE, K.index_attn, q, k, v, torch.zeros(B, 5, dtype=torch.int64))
    refused(SHAPE, K.index_attn, q, k, v, torch.zeros(B, 4, dtype=torch.int32))
    refused(SHAPE, K.index_attn, q, k, bf(B, N - 8, H, D), torch.zeros(B, 5, dtype=torch.int32))
    refused(UNSUP, K.index_attn, q, k, v, torch.zeros(B, 5, dtype=torch.int32))
