"""Pins of the attention oracle against things other than itself.

* brute force on tiny inputs (pure-Python loops, exp without max subtraction);
* the self-only special case equals a library SDPA routine (torch CPU, fp64);
* invariants that hold for softmax attention over a key set: duplicated keys,
  permutations, constant V, zero queries, one key, widely separated scores.

A dropped segment, a wrong head slice, a per-frame segment read at the wrong
frame, a wrong scale or a transposed operand each fail at least one test.
"""

import math

import numpy as np
import pytest

from oracle import refbank_attention, attend_rows, concat_segments


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _segments(rng, F, C, lens, shared_flags):
    segs = []
    for ls, sh in zip(lens, shared_flags):
        shape = (ls, C) if sh else (F, ls, C)
        segs.append((_rand(rng, *shape), _rand(rng, *shape), sh))
    return segs


def _brute(q, segs, heads, scale):
    """Pure-Python loops: exp without max subtraction, explicit sums."""
    F, L, C = q.shape
    d = C // heads
    out = np.zeros((F, L, C))
    for f in range(F):
        keys, vals = [], []
        for k, v, sh in segs:
            kk = k if sh else k[f]
            vv = v if sh else v[f]
            for j in range(kk.shape[0]):
                keys.append(kk[j])
                vals.append(vv[j])
        for h in range(heads):
            for i in range(L):
                w = []
                for key in keys:
                    s = 0.0
                    for c in range(d):
                        s += q[f, i, h * d + c] * key[h * d + c]
                    w.append(math.exp(s * scale))
                z = sum(w)
                for c in range(d):
                    acc = 0.0
                    for wj, val in zip(w, vals):
                        acc += wj * val[h * d + c]
                    out[f, i, h * d + c] = acc / z
    return out


@pytest.mark.parametrize("nseg", [1, 2, 3, 5])
def test_brute_force_tiny(nseg):
    rng = np.random.default_rng(100 + nseg)
    F, L, H, d = 2, 5, 2, 4
    C = H * d
    lens = [3, 7, 1, 4, 6][:nseg]
    shared = [False, True, True, True, True][:nseg]
    q = _rand(rng, F, L, C)
    segs = _segments(rng, F, C, lens, shared)
    scale = 1.0 / math.sqrt(d)
    got = refbank_attention(q, segs, H)
    ref = _brute(q, segs, H, scale)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_brute_force_shared_first_and_per_frame_late():
    # segment kinds in an unusual order: the frame index must follow each segment's kind
    rng = np.random.default_rng(7)
    F, L, H, d = 3, 4, 2, 8
    C = H * d
    segs = _segments(rng, F, C, [5, 2, 3], [True, False, True])
    q = _rand(rng, F, L, C)
    got = refbank_attention(q, segs, H, scale=0.3)
    ref = _brute(q, segs, H, 0.3)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_self_only_equals_library_sdpa():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    F, L, H, d = 3, 9, 2, 8
    C = H * d
    q = _rand(rng, F, L, C)
    k = _rand(rng, F, L, C)
    v = _rand(rng, F, L, C)
    got = refbank_attention(q, [(k, v, False)], H)

    def heads(x):
        return torch.from_numpy(x).reshape(F, L, H, d).permute(0, 2, 1, 3).contiguous()

    ref = torch.nn.functional.scaled_dot_product_attention(heads(q), heads(k), heads(v))
    ref = ref.permute(0, 2, 1, 3).reshape(F, L, C).numpy()
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_bank_with_bank_equals_concatenated_library_sdpa():
    # self + shared bank equals SDPA over keys that were concatenated by hand
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(2)
    F, L, H, d, Lb = 2, 6, 2, 4, 5
    C = H * d
    q = _rand(rng, F, L, C)
    k = _rand(rng, F, L, C)
    v = _rand(rng, F, L, C)
    bk = _rand(rng, Lb, C)
    bv = _rand(rng, Lb, C)
    got = refbank_attention(q, [(k, v, False), (bk, bv, True)], H)
    kc = np.concatenate([k, np.broadcast_to(bk, (F, Lb, C))], axis=1)
    vc = np.concatenate([v, np.broadcast_to(bv, (F, Lb, C))], axis=1)

    def heads(x, n):
        return torch.from_numpy(np.ascontiguousarray(x)).reshape(F, n, H, d).permute(0, 2, 1, 3).contiguous()

    ref = torch.nn.functional.scaled_dot_product_attention(heads(q, L), heads(kc, L + Lb), heads(vc, L + Lb))
    ref = ref.permute(0, 2, 1, 3).reshape(F, L, C).numpy()
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_bank_copy_of_own_tokens_leaves_output_unchanged():
    rng = np.random.default_rng(3)
    F, L, H, d = 1, 7, 2, 4
    C = H * d
    q = _rand(rng, F, L, C)
    k = _rand(rng, F, L, C)
    v = _rand(rng, F, L, C)
    alone = refbank_attention(q, [(k, v, False)], H)
    for copies in (1, 3):
        segs = [(k, v, False)] + [(k[0], v[0], True)] * copies
        assert np.max(np.abs(refbank_attention(q, segs, H) - alone)) <= 1e-12


def test_permutation_of_segments_and_keys():
    rng = np.random.default_rng(4)
    F, L, H, d = 2, 5, 2, 4
    C = H * d
    segs = _segments(rng, F, C, [6, 4, 3], [False, True, True])
    q = _rand(rng, F, L, C)
    base = refbank_attention(q, segs, H)
    perm = [segs[2], segs[0], segs[1]]
    assert np.max(np.abs(refbank_attention(q, perm, H) - base)) <= 1e-12
    k, v, sh = segs[0]
    idx = rng.permutation(k.shape[1])
    shuffled = [(k[:, idx], v[:, idx], sh)] + segs[1:]
    assert np.max(np.abs(refbank_attention(q, shuffled, H) - base)) <= 1e-12


def test_constant_values_give_that_constant():
    rng = np.random.default_rng(5)
    F, L, H, d = 2, 4, 2, 4
    C = H * d
    row = rng.standard_normal(C)
    k1 = _rand(rng, F, 6, C)
    k2 = _rand(rng, 3, C)
    v1 = np.broadcast_to(row, (F, 6, C)).copy()
    v2 = np.broadcast_to(row, (3, C)).copy()
    out = refbank_attention(_rand(rng, F, L, C), [(k1, v1, False), (k2, v2, True)], H)
    assert np.max(np.abs(out - row)) <= 1e-12


def test_zero_queries_give_mean_of_all_values():
    rng = np.random.default_rng(6)
    F, L, H, d = 2, 3, 2, 4
    C = H * d
    segs = _segments(rng, F, C, [5, 4, 2], [False, True, True])
    out = refbank_attention(np.zeros((F, L, C)), segs, H)
    for f in range(F):
        vals = np.concatenate([v if sh else v[f] for _, v, sh in segs], axis=0)
        assert np.max(np.abs(out[f] - vals.mean(axis=0))) <= 1e-12


def test_one_key_gives_its_value():
    rng = np.random.default_rng(8)
    F, L, H, d = 2, 4, 2, 4
    C = H * d
    k = _rand(rng, F, 1, C)
    v = _rand(rng, F, 1, C)
    out = refbank_attention(_rand(rng, F, L, C), [(k, v, False)], H)
    assert np.max(np.abs(out - v)) <= 1e-12


def test_separated_scores_select_the_argmax_value():
    # key j points along e_j with growing length; the query along e_3 picks key 3
    F, L, H, d = 1, 1, 1, 8
    C = d
    keys = np.zeros((1, 5, C))
    for j in range(5):
        keys[0, j, j] = 1.0
    q = np.zeros((1, 1, C))
    q[0, 0, 3] = 400.0
    vals = np.arange(5 * C, dtype=np.float64).reshape(1, 5, C)
    out = refbank_attention(q, [(keys, vals, False)], H, scale=1.0)
    assert np.max(np.abs(out[0, 0] - vals[0, 3])) <= 1e-12


def test_scale_defaults_to_inverse_sqrt_head_dim():
    rng = np.random.default_rng(9)
    F, L, H, d = 1, 3, 4, 5
    C = H * d
    segs = _segments(rng, F, C, [4], [False])
    q = _rand(rng, F, L, C)
    assert np.max(np.abs(refbank_attention(q, segs, H) - refbank_attention(q, segs, H, scale=1 / math.sqrt(d)))) == 0.0
    assert np.max(np.abs(refbank_attention(q, segs, H) - refbank_attention(q, segs, H, scale=1 / math.sqrt(C)))) > 1e-6


def test_restricted_rows_match_full_output():
    rng = np.random.default_rng(10)
    F, L, H, d = 2, 9, 2, 4
    C = H * d
    segs = _segments(rng, F, C, [9, 9], [False, True])
    q = _rand(rng, F, L, C)
    full = refbank_attention(q, segs, H)
    rows = [0, 4, 8]
    part = refbank_attention(q, segs, H, frames=[1], head_list=[0, 1], rows=rows)
    for h in range(H):
        assert np.max(np.abs(part[(1, h)] - full[1][rows][:, h * d:(h + 1) * d])) == 0.0


def test_fp16_inputs_are_upcast_exactly():
    rng = np.random.default_rng(11)
    F, L, H, d = 1, 4, 1, 8
    q = rng.standard_normal((F, L, d)).astype(np.float16)
    k = rng.standard_normal((F, 6, d)).astype(np.float16)
    v = rng.standard_normal((F, 6, d)).astype(np.float16)
    a = refbank_attention(q, [(k, v, False)], H)
    b = refbank_attention(q.astype(np.float64), [(k.astype(np.float64), v.astype(np.float64), False)], H)
    assert np.array_equal(a, b)


def test_attend_rows_and_concat_helpers():
    rng = np.random.default_rng(12)
    segs = _segments(rng, 2, 4, [3, 2], [False, True])
    k, v = concat_segments(segs, 1)
    assert k.shape == (5, 4)
    assert np.array_equal(k[:3], segs[0][0][1]) and np.array_equal(k[3:], segs[1][0])
    o = attend_rows(np.zeros((1, 4)), k, v, 1.0)
    assert np.max(np.abs(o[0] - v.mean(axis=0))) <= 1e-12


# ---- block-causal attention over a chunked sequence --------------------------------
def _chunk_inputs(seed, F, L, C, n_shared=1, Ls=5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((F, L, C))
    kv = (rng.standard_normal((F, L, C)), rng.standard_normal((F, L, C)))
    shared = [(rng.standard_normal((Ls, C)), rng.standard_normal((Ls, C))) for _ in range(n_shared)]
    return q, kv, shared


def test_chunk_causal_one_chunk_is_plain_attention():
    # a chunk as long as the sequence (and unlimited history) masks nothing
    from oracle import chunk_causal_attention
    q, kv, shared = _chunk_inputs(1, 2, 7, 8)
    got = chunk_causal_attention(q, kv, shared, 2, chunk_len=7)
    segs = [(kv[0], kv[1], False)] + [(k, v, True) for k, v in shared]
    assert np.allclose(got, refbank_attention(q, segs, 2), atol=1e-13)


def test_chunk_causal_token_chunks_are_causal_sdpa():
    # chunks of one token, no shared keys: textbook causal attention (library routine)
    torch = pytest.importorskip("torch")
    from oracle import chunk_causal_attention
    q, kv, _ = _chunk_inputs(2, 1, 9, 6)
    got = chunk_causal_attention(q, kv, [], 2, chunk_len=1)
    tq, tk, tv = (torch.from_numpy(a[0].reshape(9, 2, 3).transpose(1, 0, 2).copy()) for a in (q, kv[0], kv[1]))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    assert np.allclose(got[0], ref.numpy().transpose(1, 0, 2).reshape(9, 6), atol=1e-13)


def test_chunk_causal_brute_force_with_history_limit():
    # each row by hand: its visible self keys are the chunks [c - H, c], plus the shared rows
    from oracle import chunk_causal_attention
    q, kv, shared = _chunk_inputs(3, 2, 11, 4, n_shared=2, Ls=3)
    cl, hist = 3, 1
    got = chunk_causal_attention(q, kv, shared, 1, chunk_len=cl, max_history=hist)
    for f in range(2):
        for r in range(11):
            c = r // cl
            keys = [j for j in range(11) if max(0, c - hist) <= j // cl <= c]
            kk = np.concatenate([kv[0][f][keys]] + [k for k, _ in shared])
            vv = np.concatenate([kv[1][f][keys]] + [v for _, v in shared])
            s = kk @ q[f][r] / 2.0
            w = [math.exp(x) for x in s]
            want = sum(wi * vi for wi, vi in zip(w, vv)) / sum(w)
            assert np.allclose(got[f, r], want, atol=1e-12)


def test_chunk_causal_never_sees_later_chunks():
    # changing a later chunk's keys and values leaves earlier rows unchanged
    from oracle import chunk_causal_attention
    q, kv, shared = _chunk_inputs(4, 1, 12, 4)
    a = chunk_causal_attention(q, kv, shared, 1, chunk_len=4)
    k2, v2 = kv[0].copy(), kv[1].copy()
    k2[0, 8:] += 5.0
    v2[0, 8:] -= 3.0
    b = chunk_causal_attention(q, (k2, v2), shared, 1, chunk_len=4)
    assert np.array_equal(a[0, :8], b[0, :8])
    assert not np.allclose(a[0, 8:], b[0, 8:])
