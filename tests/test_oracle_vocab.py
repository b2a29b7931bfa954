"""Pins for the oracle's int4 vocabulary table lookup (CPU only).

"Gemma 4 E2B" article, tip on the int4 vocabulary tables, and "Gemma 4 From
E2B to 31B", "Tip: int4 Embedding Tables Cost More at Larger Sizes": the
embedding, untied lm_head and per-layer embedding tables are packed int4 in
groups of 32 as trained. A looked-up row must be the stored bf16 row of the
QAT table bit for bit (the q4_0 repack reproduces every stored value); the
untied lm_head is the W4A16 GEMM, pinned with the GEMMs.
"""

import numpy as np

import gen


def test_embed_rows_are_the_stored_bf16_rows(oracle):
    d = gen.vocab_config(V=300, D=96, T=40, seed=3)
    p, st, amb = oracle.repack_q4_0(d["w_bf16"])
    assert amb == 0
    ids = d["ids"].copy()
    ids[5] = ids[6]  # repeated token
    out = oracle.embed_q4(ids, p, st)
    assert np.array_equal(out, d["w_bf16"][ids])


def test_embed_invalid_ids_give_zero_rows(oracle):
    d = gen.vocab_config(V=64, D=64, T=6, seed=4)
    p, st, _ = oracle.repack_q4_0(d["w_bf16"])
    ids = np.int32([0, -1, 63, 64, 1 << 30, 7])
    out = oracle.embed_q4(ids, p, st)
    assert not out[[1, 3, 4]].any()
    assert np.array_equal(out[[0, 2, 5]], d["w_bf16"][[0, 63, 7]])


def test_embed_matches_one_hot_lm_head(oracle):
    """The lookup and the lm_head read the same table values: the W4A16 GEMM
    of the one-hot row e_k against the table is column k of every looked-up
    row, exactly."""
    d = gen.vocab_config(V=64, D=64, T=4, seed=5)
    p, st, _ = oracle.repack_q4_0(d["w_bf16"])
    table = gen.bf16_bits_to_f32(oracle.embed_q4(np.arange(64, dtype=np.int32), p, st))
    for k in (0, 31, 63):
        x = np.zeros((1, 64), np.uint16)
        x[0, k] = 0x3F80  # bf16 1.0
        y32, _ = oracle.gemm_w4a16(x, p, st)
        assert np.array_equal(y32[0], table[:, k])
