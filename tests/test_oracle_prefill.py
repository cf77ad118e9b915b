"""Pins for the oracle's paged multi-token (chunked prefill) attention, CPU only.

Each test ties oracle.prefill to something other than itself: torch's float64
scaled_dot_product_attention with an explicit causal mask on contiguous K/V
built before paging, closed forms that fix the causal extent of every row,
the single-token case (the pinned decode oracle), and the chunking identity
(a prompt fed in chunks gives the rows of the whole prompt at once).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from test_oracle_attention import BS, page_into_pool


def causal_sdpa(q_rows, K, V, L, scale):
    """Contiguous float64 SDPA, the last T = len(q_rows) positions as queries.

    The mask comes from torch.tril with diagonal L - T: query row i may see
    key t exactly when t <= L - T + i.
    """
    T = q_rows.shape[0]
    mask = torch.ones(T, L, dtype=torch.bool).tril(diagonal=L - T)
    qt = torch.from_numpy(q_rows.transpose(1, 0, 2)[None])  # [1][Hq][T][D]
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, torch.from_numpy(K[None]), torch.from_numpy(V[None]), attn_mask=mask,
        scale=float(scale), enable_gqa=True)
    return o[0].numpy().transpose(1, 0, 2)  # [T][Hq][D]


def _batch(rng, lens, chunks, hkv, g, d):
    K = [rng.standard_normal((hkv, L, d)) for L in lens]
    V = [rng.standard_normal((hkv, L, d)) for L in lens]
    qstart = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int64)
    q = rng.standard_normal((int(qstart[-1]), hkv * g, d))
    return K, V, q, qstart


@pytest.mark.parametrize("seed", range(8))
def test_matches_masked_sdpa_on_contiguous(seed):
    rng = np.random.default_rng(300 + seed)
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice([8, 16, 64]))
    B = int(rng.integers(1, 5))
    lens = [int(x) for x in rng.integers(1, 70, size=B)]
    chunks = [int(rng.integers(0, L + 1)) for L in lens]
    K, V, q, qstart = _batch(rng, lens, chunks, hkv, g, d)
    scale = float(np.float32(1 / math.sqrt(d)))
    nb = sum(-(-L // BS) for L in lens) + 3
    kp, vp, tables = page_into_pool(K, V, nb, rng)
    got = oracle.prefill(q, kp, vp, tables, lens, qstart, scale, "fp32")
    for s in range(B):
        a, b = qstart[s], qstart[s + 1]
        if a == b:
            continue
        want = causal_sdpa(q[a:b], K[s], V[s], lens[s], np.float32(scale))
        np.testing.assert_allclose(got[a:b], want, rtol=0, atol=1e-12)


def test_identical_keys_give_running_means():
    """Equal scores: row i is the mean of V over positions 0..L-T+i exactly.

    Pins the causal extent of each row: an off-by-one in the position or the
    mask changes the count in the mean.
    """
    rng = np.random.default_rng(1)
    hkv, g, d, L, T = 2, 3, 8, 45, 29
    K = rng.standard_normal((hkv, L, d))
    K[:] = K[:, :1, :]
    V = rng.standard_normal((hkv, L, d))
    q = rng.standard_normal((T, hkv * g, d))
    kp, vp, t = page_into_pool([K], [V], 6, rng)
    out = oracle.prefill(q, kp, vp, t, [L], [0, T], 0.3, "fp32")
    run_mean = np.cumsum(V, axis=1) / np.arange(1, L + 1)[None, :, None]
    for i in range(T):
        for h in range(hkv * g):
            np.testing.assert_allclose(out[i, h], run_mean[h // g, L - T + i], rtol=0, atol=1e-13)


def test_whole_prompt_first_row_is_v0():
    """T = L: the first token sees only itself."""
    rng = np.random.default_rng(2)
    hkv, g, d, L = 1, 4, 16, 33
    K = rng.standard_normal((hkv, L, d))
    V = rng.standard_normal((hkv, L, d))
    q = rng.standard_normal((L, g, d))
    kp, vp, t = page_into_pool([K], [V], 4, rng)
    out = oracle.prefill(q, kp, vp, t, [L], [0, L], 0.25, "fp32")
    for h in range(g):
        assert np.array_equal(out[0, h], V[0, 0])


def test_single_token_chunks_equal_decode():
    rng = np.random.default_rng(3)
    lens = [1, 16, 17, 100]
    K, V, q, qstart = _batch(rng, lens, [1] * 4, 2, 4, 32)
    kp, vp, t = page_into_pool(K, V, 20, rng)
    a = oracle.prefill(q, kp, vp, t, lens, qstart, 0.125, "fp32")
    b = oracle.decode(q, kp, vp, t, lens, 0.125, "fp32")
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-15)


def test_chunks_reproduce_the_whole_prompt():
    """Feeding a prompt as chunks [0,a), [a,b), [b,L) -- each step with the
    context written so far -- gives the same rows as the whole prompt at once
    (Batching and PagedAttention, chunked prefill)."""
    rng = np.random.default_rng(4)
    hkv, g, d, L = 2, 2, 16, 77
    K = rng.standard_normal((hkv, L, d))
    V = rng.standard_normal((hkv, L, d))
    q = rng.standard_normal((L, hkv * g, d))
    kp, vp, t = page_into_pool([K], [V], 8, rng)
    whole = oracle.prefill(q, kp, vp, t, [L], [0, L], 0.2, "fp32")
    parts = []
    for lo, hi in [(0, 20), (20, 21), (21, 77)]:
        parts.append(oracle.prefill(q[lo:hi], kp, vp, t, [hi], [0, hi - lo], 0.2, "fp32"))
    np.testing.assert_allclose(np.concatenate(parts), whole, rtol=0, atol=1e-15)


def test_future_positions_never_read():
    """Poisoning every position after a row's own with NaN leaves that row
    finite and unchanged: row i reads nothing past L - T + i."""
    rng = np.random.default_rng(5)
    hkv, g, d, L, T = 1, 2, 8, 40, 12
    K = rng.standard_normal((hkv, L, d))
    V = rng.standard_normal((hkv, L, d))
    q = rng.standard_normal((T, g, d))
    kp, vp, t = page_into_pool([K], [V], 5, np.random.default_rng(0))
    ref = oracle.prefill(q, kp, vp, t, [L], [0, T], 0.3, "fp32")
    for i in range(T):
        p = L - T + i
        K2 = K.copy()
        V2 = V.copy()
        K2[:, p + 1:] = np.nan
        V2[:, p + 1:] = np.nan
        kp2, vp2, t2 = page_into_pool([K2], [V2], 5, np.random.default_rng(0))
        row = oracle.prefill(q[:i + 1], kp2, vp2, t2, [p + 1], [0, i + 1], 0.3, "fp32")[i]
        assert np.all(np.isfinite(row))
        assert np.array_equal(row, ref[i])


def test_empty_chunks_and_empty_batch():
    rng = np.random.default_rng(6)
    lens = [5, 9]
    K, V, q, qstart = _batch(rng, lens, [0, 0], 1, 1, 8)
    kp, vp, t = page_into_pool(K, V, 4, rng)
    out = oracle.prefill(q, kp, vp, t, lens, qstart, 0.5, "fp32")
    assert out.shape == (0, 1, 8)


def test_bf16_storage_matches_upcast_then_sdpa():
    from workloads import bf16_bits_from_f32

    rng = np.random.default_rng(7)
    hkv, g, d, L, T = 2, 2, 16, 50, 18
    Kf = rng.standard_normal((hkv, L, d)).astype(np.float32)
    Vf = rng.standard_normal((hkv, L, d)).astype(np.float32)
    qf = rng.standard_normal((T, hkv * g, d)).astype(np.float32)
    Kb, Vb, qb = (bf16_bits_from_f32(x) for x in (Kf, Vf, qf))
    up = lambda bits: torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()  # noqa: E731
    kp, vp, t = page_into_pool([up(Kb)], [up(Vb)], 6, rng)
    # store the pool as bf16 bits again (exact: the values are bf16 already)
    kpb = bf16_bits_from_f32(np.nan_to_num(kp).astype(np.float32))
    vpb = bf16_bits_from_f32(np.nan_to_num(vp).astype(np.float32))
    got = oracle.prefill(qb, kpb, vpb, t, [L], [0, T], 0.25, "bf16")
    want = causal_sdpa(up(qb), up(Kb), up(Vb), L, np.float32(0.25))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
