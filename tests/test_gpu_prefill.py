"""GPU parity of pa_prefill (chunked-prefill attention) against the oracle.

Every case runs the whole step through the library -- block manager,
pa_write_kv of the chunk, pa_prefill -- on pools whose unused elements are
NaN, and compares with the oracle's float64 result element by element.
Small cases are checked on every row, and so are the full-size P3, P4 and
P5 steps; P1 and P2 on sampled rows (first, last and random rows of every
sequence), which the oracle computes one at a time.
"""

import numpy as np
import pytest

import oracle
from harness import (TOL, GpuPrefillStep, oracle_prefill_pools, oracle_prefill_rows, to_device, to_f64,
                     to_host_storage)
from workloads import make_prefill_custom, make_prefill_workload

pytestmark = pytest.mark.gpu


def _check(got, want, dtype, what=""):
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - want).max() if got.size else 0.0
    assert err <= TOL[dtype], f"{what}: max abs error {err} > {TOL[dtype]}"
    return err


def _bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint16) if a.dtype.itemsize == 2 else a.view(np.uint32)


def _full_parity(w):
    g = GpuPrefillStep(w)
    out = g.run()
    st, k, v = oracle_prefill_pools(w)
    want = oracle.prefill(w.q, k, v, st.tables, w.context_lens, w.query_start, w.scale, w.dtype)
    got = to_f64(out, w.dtype)
    # the chunk's K/V landed in the same slots, bit for bit
    assert np.array_equal(_bits(to_host_storage(g.k, w.dtype)), _bits(k))
    assert np.array_equal(_bits(to_host_storage(g.v, w.dtype)), _bits(v))
    return _check(got, want, w.dtype, w.name)


def test_tiny_bf16_every_row():
    print("case p0", flush=True)
    _full_parity(make_prefill_workload("p0"))


def test_tiny_fp16_every_row():
    w = make_prefill_custom("p0h", "fp16", [0, 20, 5, 64, 100, 9], [1, 7, 16, 33, 130, 0], 8, 2, 64, seed=20)
    _full_parity(w)


# (g, D, dtype): group sizes that fill 16-row columns in different ways
SHAPES = [(1, 128, "fp16"), (2, 64, "bf16"), (4, 128, "bf16"), (5, 64, "fp16"), (8, 128, "fp16"),
          (16, 64, "bf16"), (3, 128, "bf16"), (32, 128, "bf16")]


@pytest.mark.parametrize("g,D,dtype", SHAPES)
def test_random_chunks_every_row(g, D, dtype):
    rng = np.random.default_rng(1000 + 17 * g + D)
    B = 5
    prior = rng.integers(0, 300, size=B)
    chunk = rng.integers(1, 200, size=B)
    chunk[1] = 0  # an empty chunk among the others
    prior[2] = 0  # a whole prompt in one step
    w = make_prefill_custom(f"r{g}_{D}", dtype, prior, chunk, 2 * g, 2, D, seed=int(rng.integers(1 << 30)))
    print(f"case g={g} D={D} {dtype} prior={prior.tolist()} chunk={chunk.tolist()}", flush=True)
    _full_parity(w)


@pytest.mark.parametrize("T", [1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 257])
def test_chunk_lengths_around_tile_edges(T):
    """Row tiles are 128 rows (32 tokens at g = 4) and steps 32 positions."""
    w = make_prefill_custom(f"t{T}", "bf16", [0, 13, 32, 100], [T, T, T, T], 8, 2, 128, seed=300 + T)
    _full_parity(w)


def _sampled(w, nrand=8, seed=0):
    rng = np.random.default_rng(seed)
    qs = w.query_start
    rows = []
    for s in range(w.num_seqs):
        a, b = int(qs[s]), int(qs[s + 1])
        if a == b:
            continue
        rows += [a, b - 1] + [int(x) for x in rng.integers(a, b, size=min(nrand, b - a))]
    return np.unique(np.asarray(rows))


@pytest.mark.parametrize("key", ["p1", "p2", "p3", "p4", "p5"])
def test_full_size_sampled_rows(key):
    w = make_prefill_workload(key)
    print(f"case {key}", flush=True)
    g = GpuPrefillStep(w)
    out = to_f64(g.run(), w.dtype)
    assert np.isfinite(out).all()
    st, k, v = oracle_prefill_pools(w)
    rows = _sampled(w, nrand=4 if key not in ("p3", "p5") else 1, seed=7)
    want = oracle_prefill_rows(w, st, k, v, rows)
    _check(out[rows], want, w.dtype, key)


def test_deterministic_and_placement_invariant():
    """Same inputs, same bits; a different physical placement of the same
    logical cache gives the same bits too (arithmetic order depends only on
    logical positions)."""
    import torch

    # (the last two sequences have 4 and 12 rows: decode-shaped items)
    w = make_prefill_custom("pl", "bf16", [40, 0, 77, 500, 61], [90, 33, 5, 1, 3], 8, 2, 128, seed=5)
    g = GpuPrefillStep(w)
    a = g.run().clone()
    b = g.attend().clone()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # permute the physical blocks: pool[p[i]] = pool[i], tables through p
    nb = w.num_blocks
    p = torch.from_numpy(np.random.default_rng(3).permutation(nb)).cuda()
    k2 = torch.empty_like(g.k)
    v2 = torch.empty_like(g.v)
    k2[p] = g.k
    v2[p] = g.v
    t = g.tables.long()
    t2 = torch.where(t >= 0, p[t.clamp(min=0)], t).int().contiguous()
    import paged_kv_cache_117_amd as pa

    c = pa.prefill(g.q, k2, v2, t2, g.lens, g.qstart, w.scale, w.max_query_len, w.max_context_len)
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


def test_single_token_chunks_match_decode_within_tolerance():
    import paged_kv_cache_117_amd as pa

    w = make_prefill_custom("dec", "bf16", [15, 16, 200, 1000], [1, 1, 1, 1], 32, 8, 128, seed=9)
    g = GpuPrefillStep(w)
    a = to_f64(g.run(), w.dtype)
    d = pa.decode(g.q, g.k, g.v, g.tables, g.lens, w.scale, w.max_context_len)
    st, k, v = oracle_prefill_pools(w)
    want = oracle.decode(w.q, k, v, st.tables, w.context_lens, w.scale, w.dtype)
    _check(a, want, w.dtype, "prefill T=1")
    _check(to_f64(d, w.dtype), want, w.dtype, "decode")


@pytest.mark.parametrize("scale", [0.0, -0.0883883461356163, 0.5])
def test_scales(scale):
    # chunks of 40 and 70 tokens (matrix tiles) and of 1 and 3 (decode-shaped items)
    w = make_prefill_custom("sc", "fp16", [10, 50, 300, 17], [40, 70, 1, 3], 8, 2, 64, seed=11)
    w.scale = float(np.float32(scale))
    _full_parity(w)


def test_bad_block_id_and_bad_lengths_give_nan_rows():
    import torch

    import paged_kv_cache_117_amd as pa

    w = make_prefill_custom("bad", "bf16", [20, 20, 20], [10, 10, 10], 8, 2, 64, seed=12)
    g = GpuPrefillStep(w)
    good = to_f64(g.run(), w.dtype)
    qs = w.query_start
    # sequence 1: a block id past the pool
    t = g.tables.clone()
    t[1, 0] = w.num_blocks + 5
    out = to_f64(pa.prefill(g.q, g.k, g.v, t, g.lens, g.qstart, w.scale, w.max_query_len, w.max_context_len),
                 w.dtype)
    assert np.isnan(out[qs[1]:qs[2]]).all()
    assert np.array_equal(out[qs[0]:qs[1]], good[qs[0]:qs[1]])
    assert np.array_equal(out[qs[2]:], good[qs[2]:])
    # sequence 2: T > L
    lens = g.lens.clone()
    lens[2] = 5
    out = to_f64(pa.prefill(g.q, g.k, g.v, g.tables, lens, g.qstart, w.scale, w.max_query_len,
                            w.max_context_len), w.dtype)
    assert np.isnan(out[qs[2]:qs[3]]).all()
    assert np.array_equal(out[:qs[2]], good[:qs[2]])
    # sequence 0: T larger than the max_query_len hint
    qst = torch.tensor([0, 14, 20, 30], dtype=torch.int32, device="cuda")
    out = to_f64(pa.prefill(g.q, g.k, g.v, g.tables, g.lens, qst, w.scale, 10, w.max_context_len), w.dtype)
    assert np.isnan(out[0:14]).all()


def test_empty_chunks_between_others():
    import torch

    import paged_kv_cache_117_amd as pa

    w = make_prefill_custom("emp", "bf16", [5, 9, 30], [0, 12, 0], 8, 2, 64, seed=13)
    g = GpuPrefillStep(w)
    g.write()
    out = torch.full_like(g.q, 7.0)
    pa.prefill(g.q, g.k, g.v, g.tables, g.lens, g.qstart, w.scale, w.max_query_len, w.max_context_len, out=out)
    st, k, v = oracle_prefill_pools(w)
    want = oracle.prefill(w.q, k, v, st.tables, w.context_lens, w.query_start, w.scale, w.dtype)
    _check(to_f64(out, w.dtype), want, w.dtype, "emp")


@pytest.mark.parametrize("psize", [64, 128, 512, 2048])
def test_split_partitions_every_row(psize):
    """Position partitions merged with log-sum-exp weights equal the unsplit
    attention (a partition of one step upward; rows whose causal limit stops
    before a partition take no part in it)."""
    w = make_prefill_custom(f"sp{psize}", "bf16", [0, 300, 1000, 77], [130, 40, 200, 1], 8, 2, 128,
                            seed=700 + psize)
    print(f"case split psize={psize}", flush=True)
    g = GpuPrefillStep(w)
    out = to_f64(g.run(partition_size=psize), "bf16")
    st, k, v = oracle_prefill_pools(w)
    want = oracle.prefill(w.q, k, v, st.tables, w.context_lens, w.query_start, w.scale, w.dtype)
    _check(out, want, "bf16", f"split {psize}")


def test_auto_split_short_chunk_long_context():
    """A prefix-cache continuation: 64 new tokens after 20k-30k cached ones.
    The automatic split cuts the walk into partitions (sampled rows)."""
    import paged_kv_cache_117_amd as pa

    w = make_prefill_custom("cont", "bf16", [20000, 31000], [64, 50], 32, 8, 128, seed=710)
    assert pa.prefill_workspace_bytes(w.num_seqs, w.num_tokens, 32, 8, 128, w.max_query_len,
                                      w.max_context_len, 0) > 0
    g = GpuPrefillStep(w)
    out = to_f64(g.run(), "bf16")
    assert np.isfinite(out).all()
    st, k, v = oracle_prefill_pools(w)
    rows = _sampled(w, nrand=6, seed=3)
    _check(out[rows], oracle_prefill_rows(w, st, k, v, rows), "bf16", "cont")
    # the unsplit launch agrees within rounding
    one = to_f64(g.attend(partition_size=1 << 20), "bf16")
    assert np.abs(one - out).max() <= TOL["bf16"]


def test_split_with_context_past_the_hint_gives_nan_rows():
    import paged_kv_cache_117_amd as pa

    w = make_prefill_custom("hint", "bf16", [500, 100], [20, 30], 8, 2, 64, seed=720)
    g = GpuPrefillStep(w)
    g.write()
    good = to_f64(g.attend(partition_size=128), "bf16")
    lens = g.lens.clone()
    lens[0] = w.max_context_len + 1  # longer than the max_context_len hint
    out = to_f64(pa.prefill(g.q, g.k, g.v, g.tables, lens, g.qstart, w.scale, w.max_query_len,
                            w.max_context_len, partition_size=128), "bf16")
    qs = w.query_start
    assert np.isnan(out[qs[0]:qs[1]]).all()
    assert np.array_equal(out[qs[1]:], good[qs[1]:])


@pytest.mark.parametrize("g,D,bs", [(1, 64, 16), (3, 128, 32), (4, 64, 128), (8, 128, 16)])
def test_fp32_every_row(g, D, bs):
    """fp32 KV goes through the VALU kernel, one query token per work item
    (tolerance 1e-5)."""
    w = make_prefill_custom(f"f32_{g}_{D}_{bs}", "fp32", [0, 45, 130, 9], [40, 1, 77, 0], 2 * g, 2, D,
                            seed=800 + g + D + bs, block_size=bs)
    print(f"case fp32 g={g} D={D} bs={bs}", flush=True)
    _full_parity(w)


def test_fp32_bad_lengths_give_nan_rows():
    import paged_kv_cache_117_amd as pa

    w = make_prefill_custom("f32bad", "fp32", [20, 20], [10, 10], 4, 2, 64, seed=810)
    g = GpuPrefillStep(w)
    good = to_f64(g.run(), "fp32")
    lens = g.lens.clone()
    lens[1] = 5  # T > L
    out = to_f64(pa.prefill(g.q, g.k, g.v, g.tables, lens, g.qstart, w.scale, w.max_query_len,
                            w.max_context_len), "fp32")
    qs = w.query_start
    assert np.isnan(out[qs[1]:qs[2]]).all()
    assert np.array_equal(out[:qs[1]], good[:qs[1]])


# The kernel variants stay correct beside each other: PA_PREFILL_KERNEL=regs
# (K/V staged in LDS through registers, V read with plain LDS reads), dma
# (K/V loaded straight into LDS, V read transposed) and w8 (the same with
# 8-wavefront workgroups of 256 rows); the library picks dma or w8 from the
# launch's sizes.
@pytest.mark.parametrize("variant", ["regs", "dma", "w8"])
@pytest.mark.parametrize("g,D,dtype", [(1, 128, "fp16"), (5, 64, "fp16"), (4, 128, "bf16"), (16, 64, "bf16")])
def test_kernel_variants_every_row(monkeypatch, variant, g, D, dtype):
    monkeypatch.setenv("PA_PREFILL_KERNEL", variant)
    w = make_prefill_custom(f"v{variant}{g}_{D}", dtype, [0, 37, 300, 5], [150, 64, 33, 1], 2 * g, 2, D,
                            seed=900 + g + D)
    print(f"case variant={variant} g={g} D={D} {dtype}", flush=True)
    _full_parity(w)


@pytest.mark.parametrize("psize", [64, 512])
def test_kernel_variants_agree_on_split_partitions(monkeypatch, psize):
    """Both variants also feed the partition merge; each is within tolerance
    of the oracle and of the other."""
    w = make_prefill_custom(f"vsp{psize}", "bf16", [0, 300, 1000], [130, 40, 200], 8, 2, 128, seed=950 + psize)
    g = GpuPrefillStep(w)
    g.write()
    res = {}
    for variant in ("regs", "dma", "w8"):
        monkeypatch.setenv("PA_PREFILL_KERNEL", variant)
        res[variant] = to_f64(g.attend(partition_size=psize), "bf16")
    st, k, v = oracle_prefill_pools(w)
    want = oracle.prefill(w.q, k, v, st.tables, w.context_lens, w.query_start, w.scale, w.dtype)
    for variant, got in res.items():
        _check(got, want, "bf16", f"{variant} split {psize}")
    assert np.abs(res["regs"] - res["dma"]).max() <= TOL["bf16"]
    assert np.array_equal(res["dma"], res["w8"])


@pytest.mark.parametrize("variant", ["dma", "w8"])
@pytest.mark.parametrize("B,Hkv,g", [(150, 4, 2), (512, 4, 1), (514, 4, 1), (530, 4, 1)])
def test_many_items_every_row(monkeypatch, variant, B, Hkv, g):
    """Workgroups run longest walk first within each XCD: 150 x 4 items put
    75 on each XCD (two per lane of the in-kernel order); 512 x 4 put
    exactly its 256 (four per lane); 514 x 4 (257 per XCD) and 530 x 4
    exceed it and take the plain tile order.  Empty chunks and one
    unservable sequence included."""
    import paged_kv_cache_117_amd as pa

    monkeypatch.setenv("PA_PREFILL_KERNEL", variant)
    rng = np.random.default_rng(40 + B)
    prior = rng.integers(0, 70, size=B)
    chunk = rng.integers(0, 6, size=B)
    chunk[::17] = 0
    w = make_prefill_custom(f"many{B}", "bf16", prior, chunk, g * Hkv, Hkv, 64, seed=41 + B)
    print(f"case many items B={B} Hkv={Hkv} g={g} {variant}", flush=True)
    g_ = GpuPrefillStep(w)
    g_.write()
    lens = g_.lens.clone()
    bad = int(np.nonzero(chunk)[0][3])
    lens[bad] = int(chunk[bad]) - 1  # T > L: NaN rows for this sequence only
    out = to_f64(pa.prefill(g_.q, g_.k, g_.v, g_.tables, lens, g_.qstart, w.scale, w.max_query_len,
                            w.max_context_len), "bf16")
    st, k, v = oracle_prefill_pools(w)
    want = oracle.prefill(w.q, k, v, st.tables, w.context_lens, w.query_start, w.scale, w.dtype)
    qs = w.query_start
    assert np.isnan(out[qs[bad]:qs[bad + 1]]).all()
    keep = np.ones(len(out), bool)
    keep[qs[bad]:qs[bad + 1]] = False
    _check(out[keep], want[keep], "bf16", f"many {B}")


@pytest.mark.parametrize("key", ["p0", "p1", "p3", "p4", "p5"])
def test_8_wavefront_kernel_bit_identical_to_4_wavefront_kernel(monkeypatch, key):
    """Per row the 8-wavefront kernel (w8) does the arithmetic of the
    4-wavefront direct-load kernel in the same order (same 32-row wavefront
    groups, passes in position order, the same rescale decisions), so the
    outputs agree to the bit; only the workgroups' tiles differ (256 rows,
    not 128).  The default call picks one of the two."""
    import torch

    w = make_prefill_workload(key)
    print(f"case w8 == dma {key}", flush=True)
    g = GpuPrefillStep(w)
    g.write()
    out = {"auto": g.attend().clone()}
    for variant in ("dma", "w8"):
        monkeypatch.setenv("PA_PREFILL_KERNEL", variant)
        out[variant] = g.attend().clone()
    torch.cuda.synchronize()
    assert torch.equal(out["dma"].view(torch.int16), out["w8"].view(torch.int16))
    assert torch.equal(out["dma"].view(torch.int16), out["auto"].view(torch.int16))


@pytest.mark.parametrize("bs,D,dtype", [(8, 128, "bf16"), (8, 64, "fp16"), (128, 128, "fp16")])
def test_8_wavefront_kernel_block_sizes_every_row(monkeypatch, bs, D, dtype):
    """The 8-wavefront kernel loads 8-row halves from one block each: at 8
    slots a half is exactly one block, at 128 sixteen halves share one."""
    monkeypatch.setenv("PA_PREFILL_KERNEL", "w8")
    w = make_prefill_custom(f"w8bs{bs}_{D}", dtype, [0, 45, 300, 7], [140, 64, 37, 1], 8, 2, D,
                            seed=960 + bs + D, block_size=bs)
    print(f"case w8 bs={bs} D={D} {dtype}", flush=True)
    _full_parity(w)


def _walk_bound_cases():
    rng = np.random.default_rng(77)
    # Hkv = 1: sequence s is XCD s mod 8's item, and every chunk sits on XCD 0
    # (129 rows: two 128-row tiles each, the rounding the bound allows for)
    c1 = np.zeros(40, np.int64)
    c1[::8] = 129
    # Hkv = 12: two KV heads of a sequence on one XCD (m = 2)
    c2 = np.array([300, 1, 1, 1, 1, 1, 1, 77, 1, 1])
    # two long chunks beside single tokens (a mixed chunked-prefill step)
    c3 = np.ones(40, np.int64)
    c3[[5, 22]] = 257
    return {
        "one_xcd_g1": (rng.integers(0, 300, size=40), c1, 1, 1, 64, "fp16"),
        "hkv12_g2": (rng.integers(0, 600, size=10), c2, 24, 12, 64, "bf16"),
        "singles_and_chunks": (rng.integers(0, 900, size=40), c3, 32, 8, 128, "bf16"),
    }


@pytest.mark.parametrize("variant", ["dma", "w8"])
@pytest.mark.parametrize("case", ["one_xcd_g1", "hkv12_g2", "singles_and_chunks"])
def test_launch_covers_every_walk_every_row(monkeypatch, variant, case):
    """Unsplit launches in the longest-first order size their grid by the
    walks the batch can hold (chunks of num_tokens tokens in all), not by
    max_query_len's row tiles for every sequence: batches whose walks all sit
    on one XCD, with two KV heads of a sequence per XCD, or with single
    tokens beside long chunks, every row against the oracle -- also when
    max_query_len overstates the longest chunk."""
    import paged_kv_cache_117_amd as pa

    monkeypatch.setenv("PA_PREFILL_KERNEL", variant)
    prior, chunk, Hq, Hkv, D, dtype = _walk_bound_cases()[case]
    w = make_prefill_custom(f"walks_{case}", dtype, prior, chunk, Hq, Hkv, D, seed=780 + len(case))
    print(f"case walk bound {case} {variant}", flush=True)
    g = GpuPrefillStep(w)
    g.write()
    st, k, v = oracle_prefill_pools(w)
    want = oracle.prefill(w.q, k, v, st.tables, w.context_lens, w.query_start, w.scale, w.dtype)
    for max_q in (w.max_query_len, int(w.query_start[-1])):
        out = to_f64(pa.prefill(g.q, g.k, g.v, g.tables, g.lens, g.qstart, w.scale, max_q, w.max_context_len),
                     dtype)
        _check(out, want, dtype, f"{case} {variant} max_query_len={max_q}")


# Items whose rows fit one 16-row matrix column group (T * g <= 16) on blocks
# of 16 or more slots run decode-shaped inside the prefill kernel (four
# wavefronts deal the 16-slot tiles, K and V straight into the matrix
# operands, per-row causal limits in the lane's column).  (prior, chunk,
# Hq, Hkv, D, dtype, block size) per case; every row against the oracle.
SHORT_ROW_CASES = {
    # single tokens beside chunks, Llama-like heads
    "singles_g4": ([0, 700, 33, 1500, 15, 4000, 64, 0], [300, 1, 1, 1, 1, 1, 1, 1], 32, 8, 128, "bf16", 16),
    # T = 2 after 31 cached positions: the tile holding position 32 lies
    # wholly past rows 0-3's limit, and it is the only tile of wave 2
    "t2_tile_past_limit": ([31, 31, 95, 0], [2, 2, 2, 2], 8, 2, 128, "fp16", 16),
    # g = 1: 16 rows exactly (this path) next to 17 (the matrix-tile path)
    "rows_16_and_17": ([40, 200, 900, 3], [16, 17, 1, 5], 2, 2, 64, "bf16", 16),
    # g = 8 (two tokens fill the column group), blocks of 32 and of 128 slots
    "g8_bs32": ([100, 2000, 513, 7], [2, 1, 2, 1], 16, 2, 128, "fp16", 32),
    "g4_bs128": ([129, 3000, 1, 700], [1, 3, 4, 1], 8, 2, 64, "bf16", 128),
    # blocks of 8 slots keep the matrix-tile path
    "singles_bs8": ([100, 300, 17, 0], [1, 1, 2, 1], 8, 2, 128, "bf16", 8),
    # a context past 64 tiles per wavefront: table entries in two groups
    "long_single": ([5200, 4200, 64], [1, 2, 1], 8, 2, 128, "bf16", 16),
}


@pytest.mark.parametrize("case", sorted(SHORT_ROW_CASES))
def test_short_row_items_every_row(case):
    prior, chunk, Hq, Hkv, D, dtype, bs = SHORT_ROW_CASES[case]
    w = make_prefill_custom(f"short_{case}", dtype, prior, chunk, Hq, Hkv, D, seed=500 + len(case), block_size=bs)
    print(f"case short rows {case}", flush=True)
    _full_parity(w)


@pytest.mark.parametrize("variant", ["dma", "w8"])
@pytest.mark.parametrize("psize", [64, 512])
def test_short_row_items_split_every_row(monkeypatch, variant, psize):
    """Decode-shaped items in a split launch write partials in the main
    path's format (normalised rows, base-2 max, sum) for the rows that reach
    the partition; the merge reads them beside the chunks' partials."""
    monkeypatch.setenv("PA_PREFILL_KERNEL", variant)
    w = make_prefill_custom(f"short_split{psize}", "bf16", [2100, 0, 1337, 64, 700], [1, 300, 2, 1, 4], 16, 4, 128,
                            seed=610 + psize)
    print(f"case short rows split {psize} {variant}", flush=True)
    g = GpuPrefillStep(w)
    out = to_f64(g.run(partition_size=psize), w.dtype)
    st, k, v = oracle_prefill_pools(w)
    want = oracle.prefill(w.q, k, v, st.tables, w.context_lens, w.query_start, w.scale, w.dtype)
    _check(out, want, w.dtype, f"short split {psize} {variant}")


def test_short_row_item_with_bad_block_id_gives_nan_rows():
    """An out-of-range block id in a decode-shaped item's table is never
    dereferenced: that item's rows become NaN, the others are computed."""
    import paged_kv_cache_117_amd as pa

    w = make_prefill_custom("short_bad", "bf16", [300, 90, 500], [1, 1, 200], 8, 2, 128, seed=620)
    print("case short rows bad block id", flush=True)
    g = GpuPrefillStep(w)
    g.write()
    tables = g.tables.clone()
    tables[0, 5] = w.num_blocks + 7
    out = to_f64(pa.prefill(g.q, g.k, g.v, tables, g.lens, g.qstart, w.scale, w.max_query_len,
                            w.max_context_len), w.dtype)
    st, k, v = oracle_prefill_pools(w)
    want = oracle.prefill(w.q, k, v, st.tables, w.context_lens, w.query_start, w.scale, w.dtype)
    qs = w.query_start
    assert np.isnan(out[qs[0]:qs[1]]).all()
    _check(out[qs[1]:], want[qs[1]:], w.dtype, "short bad id: the other sequences")


@pytest.mark.parametrize("key", ["p3", "p4", "p5"])
def test_full_size_every_row(key):
    """Every row of the mixed steps (P3, P5: decode-shaped single tokens beside
    chunks, the walk-sized grid) and of the long continuation (P4: split walks
    merged by the reduce) against the oracle; P1 and P2 are checked on sampled
    rows above (the oracle needs minutes for all of theirs)."""
    w = make_prefill_workload(key)
    print(f"case {key} every row", flush=True)
    _full_parity(w)
