"""Pins for the oracle's paged decode attention (CPU only).

Each test ties oracle.decode to something other than itself: a library
routine on contiguous inputs built before paging, closed forms, or the pages'
invariants (placement independence, shared == duplicated, exact merging of
partitions).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import storage_to_f64
from workloads import bf16_bits_from_f32

BS = 16


def page_into_pool(K, V, num_blocks, rng, bs=BS, fill=np.nan):
    """Scatter contiguous per-sequence K/V ([Hkv][L][D] each) into a pool.

    Written here, independently of the oracle's gather: position t of
    sequence s goes to block table[s][t // bs], slot t % bs.  Unused slots
    hold ``fill``.
    """
    hkv, _, d = K[0].shape
    kp = np.full((num_blocks, hkv, bs, d), fill, dtype=np.float64)
    vp = np.full_like(kp, fill)
    perm = rng.permutation(num_blocks)
    nxt = 0
    maxb = max(1, max(-(-k.shape[1] // bs) for k in K))
    tables = np.full((len(K), maxb), -1, dtype=np.int32)
    for s, (k, v) in enumerate(zip(K, V)):
        L = k.shape[1]
        for j in range(-(-L // bs)):
            b = perm[nxt]
            nxt += 1
            tables[s, j] = b
        for t in range(L):
            kp[tables[s, t // bs], :, t % bs, :] = k[:, t, :]
            vp[tables[s, t // bs], :, t % bs, :] = v[:, t, :]
    return kp, vp, tables


def sdpa_reference(q, K, V, scale):
    """torch float64 SDPA on contiguous inputs, one sequence at a time."""
    outs = []
    for s in range(q.shape[0]):
        qt = torch.from_numpy(q[s][None, :, None, :])  # [1][Hq][1][D]
        kt = torch.from_numpy(K[s][None])  # [1][Hkv][L][D]
        vt = torch.from_numpy(V[s][None])
        o = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, scale=float(scale), enable_gqa=True)
        outs.append(o[0, :, 0, :].numpy())
    return np.stack(outs)


@pytest.mark.parametrize("seed", range(8))
def test_matches_sdpa_on_contiguous(seed):
    rng = np.random.default_rng(100 + seed)
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice([8, 16, 64]))
    B = int(rng.integers(1, 5))
    lens = [int(x) for x in rng.integers(1, 65, size=B)]
    K = [rng.standard_normal((hkv, L, d)) for L in lens]
    V = [rng.standard_normal((hkv, L, d)) for L in lens]
    q = rng.standard_normal((B, hkv * g, d))
    scale = float(np.float32(1 / math.sqrt(d)))
    nb = sum(-(-L // BS) for L in lens) + 3
    kp, vp, tables = page_into_pool(K, V, nb, rng)
    got = oracle.decode(q, kp, vp, tables, np.array(lens), scale, "fp32")
    want = sdpa_reference(q, K, V, scale)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_half_and_bf16_upcast_match_torch():
    rng = np.random.default_rng(7)
    x = rng.standard_normal(4096).astype(np.float32)
    bits = bf16_bits_from_f32(x)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(storage_to_f64(bits, "bf16"), ref)
    h = x.astype(np.float16)
    assert np.array_equal(storage_to_f64(h, "fp16"), torch.from_numpy(h).double().numpy())


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(8)
    x = rng.standard_normal(1 << 16).astype(np.float32)
    # exact ties: low 16 bits 0x8000 with both parities of bit 16
    ties = (np.arange(64, dtype=np.uint32) * np.uint32(0x10000) + np.uint32(0x3F808000)).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    got = bf16_bits_from_f32(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def _one_seq(rng, L, hkv=2, g=2, d=16):
    K = rng.standard_normal((hkv, L, d))
    V = rng.standard_normal((hkv, L, d))
    q = rng.standard_normal((1, hkv * g, d))
    return q, K, V


def test_length_one_returns_v0_exactly():
    rng = np.random.default_rng(1)
    q, K, V = _one_seq(rng, 1)
    kp, vp, t = page_into_pool([K], [V], 4, rng)
    out = oracle.decode(q, kp, vp, t, [1], 0.25, "fp32")
    for h in range(q.shape[1]):
        assert np.array_equal(out[0, h], V[h // 2, 0])


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(2)
    q, K, V = _one_seq(rng, 37)
    q[:] = 0
    kp, vp, t = page_into_pool([K], [V], 8, rng)
    out = oracle.decode(q, kp, vp, t, [37], 0.25, "fp32")
    for h in range(q.shape[1]):
        np.testing.assert_allclose(out[0, h], V[h // 2].mean(axis=0), rtol=0, atol=1e-14)


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(3)
    q, K, V = _one_seq(rng, 50)
    K[:] = K[:, :1, :]
    kp, vp, t = page_into_pool([K], [V], 8, rng)
    out = oracle.decode(q, kp, vp, t, [50], 0.25, "fp32")
    for h in range(q.shape[1]):
        np.testing.assert_allclose(out[0, h], V[h // 2].mean(axis=0), rtol=0, atol=1e-14)


def test_dominant_score_selects_its_row():
    rng = np.random.default_rng(4)
    q, K, V = _one_seq(rng, 33, hkv=1, g=1)
    K *= 1e-3
    K[0, 21] = 200.0 * q[0, 0] / np.linalg.norm(q[0, 0])  # score gap >= 50
    kp, vp, t = page_into_pool([K], [V], 8, rng)
    out = oracle.decode(q, kp, vp, t, [33], 1.0, "fp32")
    np.testing.assert_allclose(out[0, 0], V[0, 21], rtol=0, atol=1e-15)


def test_gqa_mapping_contiguous_groups():
    rng = np.random.default_rng(5)
    hkv, g, d, L = 4, 3, 8, 20
    K = rng.standard_normal((hkv, L, d))
    V = np.empty((hkv, L, d))
    for j in range(hkv):
        V[j] = j + 1.0
    q = rng.standard_normal((1, hkv * g, d))
    kp, vp, t = page_into_pool([K], [V], 6, rng)
    out = oracle.decode(q, kp, vp, t, [L], 0.5, "fp32")
    for h in range(hkv * g):
        np.testing.assert_allclose(out[0, h], h // g + 1.0, rtol=0, atol=1e-14)


def test_zero_length_gives_zero_row():
    rng = np.random.default_rng(6)
    q, K, V = _one_seq(rng, 5)
    kp, vp, t = page_into_pool([K], [V], 4, rng)
    out = oracle.decode(q, kp, vp, t, [0], 0.25, "fp32")
    assert np.all(out == 0)


def test_placement_invariance_bitwise():
    """Permuting physical blocks (pool and table together) changes nothing."""
    rng = np.random.default_rng(9)
    lens = [1, 15, 16, 17, 100, 257]
    K = [rng.standard_normal((2, L, 32)) for L in lens]
    V = [rng.standard_normal((2, L, 32)) for L in lens]
    q = rng.standard_normal((len(lens), 8, 32))
    nb = sum(-(-L // BS) for L in lens) + 5
    kp, vp, t = page_into_pool(K, V, nb, rng)
    base = oracle.decode(q, kp, vp, t, lens, 0.125, "fp32")
    p = rng.permutation(nb)  # new id of old block b is p[b]
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[p] = kp
    vp2[p] = vp
    t2 = np.where(t >= 0, p[np.maximum(t, 0)], -1)
    assert np.array_equal(base, oracle.decode(q, kp2, vp2, t2, lens, 0.125, "fp32"))


def test_shared_prefix_equals_duplicated_bitwise():
    rng = np.random.default_rng(10)
    hkv, d, prefix = 2, 16, 48  # three full shared blocks
    Kp = rng.standard_normal((hkv, prefix, d))
    Vp = rng.standard_normal((hkv, prefix, d))
    tails = [5, 20]
    Kt = [rng.standard_normal((hkv, n, d)) for n in tails]
    Vt = [rng.standard_normal((hkv, n, d)) for n in tails]
    K = [np.concatenate([Kp, k], axis=1) for k in Kt]
    V = [np.concatenate([Vp, v], axis=1) for v in Vt]
    lens = [prefix + n for n in tails]
    q = rng.standard_normal((2, 4, d))
    # duplicated: every sequence owns its own copy of the prefix
    kp, vp, t = page_into_pool(K, V, 20, rng)
    dup = oracle.decode(q, kp, vp, t, lens, 0.25, "fp32")
    # shared: both tables point at sequence 0's prefix blocks
    t_sh = t.copy()
    t_sh[1, :3] = t[0, :3]
    kp_sh = kp.copy()
    vp_sh = vp.copy()
    kp_sh[t[1, :3]] = np.nan  # the private copies are gone
    vp_sh[t[1, :3]] = np.nan
    assert np.array_equal(dup, oracle.decode(q, kp_sh, vp_sh, t_sh, lens, 0.25, "fp32"))


def test_unfilled_slots_and_unused_blocks_do_not_leak():
    rng = np.random.default_rng(11)
    lens = [3, 16, 31]
    K = [rng.standard_normal((1, L, 8)) for L in lens]
    V = [rng.standard_normal((1, L, 8)) for L in lens]
    q = rng.standard_normal((3, 2, 8))
    kp, vp, t = page_into_pool(K, V, 10, np.random.default_rng(0), fill=np.nan)
    kz, vz, _ = page_into_pool(K, V, 10, np.random.default_rng(0), fill=0.0)
    a = oracle.decode(q, kp, vp, t, lens, 0.3, "fp32")
    b = oracle.decode(q, kz, vz, t, lens, 0.3, "fp32")
    assert np.all(np.isfinite(a))
    assert np.array_equal(a, b)


@pytest.mark.parametrize("psize", [16, 64, 512])
def test_partition_merge_identity(psize):
    """Partitions merged with log-sum-exp weights equal the unsplit softmax.

    Per-partition (m_p, l_p, o_p = sum_t e^{x_t-m_p} v_t / l_p) merged as
    w_p = l_p e^{m_p - M}, out = sum_p w_p o_p / sum_p w_p.  Adding
    per-partition normalised outputs without the weights is wrong
    (PagedAttention (tensortonic), "5. Reading the Cache During Attention").
    """
    rng = np.random.default_rng(12)
    L, d = 2000, 64
    K = rng.standard_normal((1, L, d))
    V = rng.standard_normal((1, L, d))
    q = rng.standard_normal((1, 1, d))
    scale = 1 / 8
    kp, vp, t = page_into_pool([K], [V], 130, rng)
    want = oracle.decode(q, kp, vp, t, [L], scale, "fp32")[0, 0]
    x = scale * (K[0] @ q[0, 0])
    ms, ls, os_ = [], [], []
    for lo in range(0, L, psize):
        xp = x[lo:lo + psize]
        m = xp.max()
        e = np.exp(xp - m)
        ms.append(m)
        ls.append(e.sum())
        os_.append(e @ V[0, lo:lo + psize] / e.sum())
    M = max(ms)
    w = np.array([l * math.exp(m - M) for m, l in zip(ms, ls)])
    merged = (w[:, None] * np.array(os_)).sum(0) / w.sum()
    np.testing.assert_allclose(merged, want, rtol=0, atol=1e-13)
    if len(ms) > 1:
        naive = np.array(os_).sum(0)
        assert np.abs(naive - want).max() > 1e-3


def test_config_c1_matches_sdpa_after_gather():
    """The tiny fp32 config, end to end through the oracle block manager."""
    from workloads import make_workload

    w = make_workload("c1")
    bm = oracle.BlockManager(w.num_blocks, w.block_size, w.perm)
    bm.replay(w.ops)
    slots = bm.append_batch(w.seq_ids)
    k, v = oracle.write_kv(w.k_pool, w.v_pool, w.k_new, w.v_new, slots, w.block_size)
    maxb = w.max_blocks_per_seq
    tables = np.full((w.num_seqs, maxb), -1, np.int32)
    for s, sid in enumerate(w.seq_ids):
        tb = bm.table(sid)
        tables[s, :len(tb)] = tb
    got = oracle.decode(w.q, k, v, tables, w.context_lens, w.scale, w.dtype)
    # contiguous reference built by walking slots position by position
    Ks, Vs = [], []
    for s, sid in enumerate(w.seq_ids):
        L = int(w.context_lens[s])
        kk = np.empty((w.num_kv_heads, L, w.head_dim))
        vv = np.empty_like(kk)
        for pos in range(L):
            b = bm.table(sid)[pos // 16]
            kk[:, pos] = k[b, :, pos % 16]
            vv[:, pos] = v[b, :, pos % 16]
        assert np.array_equal(kk[:, L - 1], w.k_new[s])  # this step's token is attended
        Ks.append(kk)
        Vs.append(vv)
    want = sdpa_reference(w.q.astype(np.float64), Ks, Vs, np.float32(w.scale))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
