"""Seeded generators for the decode-step workloads.

Shapes follow the decode layers named in the configs below: a tiny fp32 case,
a Llama-3.1-8B layer (GQA 32/8, bf16), an OPT-13B layer (MHA 40/40, fp16), a
parallel-sampling prefix share on Llama shapes, and a Qwen2.5-72B layer (GQA
64/8, fp16).  Values are N(0,1) drawn in fp32 and rounded to the storage type
with round-to-nearest-even.  Block placement is not computed here: the
workload carries a list of block-manager operations and a pool permutation
that seeds the free list ("shuffled pool"); each consumer replays them through
its own block manager.

Draw order (one child seed per stream, in this order): context lengths (and
tails) -> pool permutation -> q -> K pool -> V pool -> new K -> new V.
Large arrays are drawn in fixed-size chunks, chunk ``c`` of stream ``s`` from
``SeedSequence(seed, spawn_key=(s, c))``, so the values do not depend on how
many threads draw them.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BLOCK_SIZE = 16
_CHUNK = 1 << 22  # elements per independently seeded chunk

# stream ids (draw order)
_S_LENS, _S_PERM, _S_Q, _S_K, _S_V, _S_KNEW, _S_VNEW = range(7)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def _storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "fp32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "fp16":
        return x.astype(np.float16)  # numpy rounds to nearest even
    if dtype == "bf16":
        return bf16_bits_from_f32(x)
    raise ValueError(dtype)


def _storage_dtype(dtype: str):
    return {"fp32": np.float32, "fp16": np.float16, "bf16": np.uint16}[dtype]


def _normal_storage(seed: int, stream: int, shape, dtype: str) -> np.ndarray:
    """N(0,1) fp32 draws in seeded chunks, rounded to the storage dtype."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=_storage_dtype(dtype))
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def fill(c):
        lo = c * _CHUNK
        hi = min(n, lo + _CHUNK)
        rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(stream, c)))
        out[lo:hi] = _storage(rng.standard_normal(hi - lo, dtype=np.float32), dtype)

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        workers = max(1, min(16, os.cpu_count() or 1, nchunks))
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(stream,)))


@dataclass
class Workload:
    """One decode step's inputs, as host arrays.

    ``context_lens[s]`` is the length row ``s`` attends over in this step and
    includes the token the step writes (at position ``context_lens[s]-1``).
    Before the step, the block manager holds ``context_lens[s]-1`` tokens for
    the sequence; ``ops`` builds that state and the step appends one token
    per sequence.
    """

    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    scale: float
    context_lens: np.ndarray  # int32 [B]
    perm: np.ndarray  # int32 [num_blocks] free-list seed order
    q: np.ndarray  # storage [B][Hq][D]
    k_pool: np.ndarray  # storage [num_blocks][Hkv][bs][D]
    v_pool: np.ndarray
    k_new: np.ndarray  # storage [B][Hkv][D]
    v_new: np.ndarray
    ops: list  # ("add", seq) | ("append", seq, n) | ("fork", parent, child)
    seq_ids: list  # batch row s <-> sequence id seq_ids[s]
    block_size: int = BLOCK_SIZE
    partition_size: int = 512
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return len(self.seq_ids)

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if len(self.context_lens) else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return max(1, -(-self.max_context_len // self.block_size))


CONFIGS = {
    "c1": "tiny fp32: 4 seqs, lens {1,5,16,37}, Hq=Hkv=2, D=64, 16-block pool",
    "c2": "Llama-3.1-8B layer, bf16: B=64, Hq=32, Hkv=8, D=128, L~U[128,4096]",
    "c3": "OPT-13B layer MHA, fp16: B=256, H=40, D=128, L~U[64,2048]",
    "c4": "prefix share, Llama shapes, bf16: 32 prompts x 8 samples, prefix 1024, tails U[0,512]",
    "c4b": "fork step, Llama shapes, bf16: 32 prompts x 8 samples, prefix 1000, first token after fork",
    "c5": "Qwen2.5-72B layer, fp16: B=128, Hq=64, Hkv=8, D=128, L~U[4096,8192], 512-token partitions",
    "c5tp8": "one GPU's share of the Qwen2.5-72B layer at tensor parallel degree 8 (its KV head and 8 query "
             "heads): C5's sequences and lengths with Hq=8, Hkv=1",
}


def _pool_blocks(lens, factor=1.25, block_size=BLOCK_SIZE):
    need = int(sum(-(-int(l) // block_size) for l in lens))
    return need, int(math.ceil(factor * need))


def make_custom(
    name: str,
    dtype: str,
    context_lens,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    seed: int,
    num_blocks: int | None = None,
    pool_factor: float = 1.25,
    partition_size: int = 512,
    block_size: int = BLOCK_SIZE,
) -> Workload:
    """Independent sequences: each prefilled with L-1 tokens, then one step.

    ``context_lens`` may be a list of lengths or a callable ``rng -> lengths``
    (drawn from the lengths stream).
    """
    if callable(context_lens):
        lens = np.asarray(context_lens(_rng(seed, _S_LENS)), dtype=np.int32)
    else:
        lens = np.asarray(context_lens, dtype=np.int32)
    need, sized = _pool_blocks(lens, pool_factor, block_size)
    nb = sized if num_blocks is None else int(num_blocks)
    if nb < need:
        raise ValueError(f"pool of {nb} blocks < {need} needed")
    B = len(lens)
    perm = _rng(seed, _S_PERM).permutation(nb).astype(np.int32)
    D, Hq, Hkv = head_dim, num_q_heads, num_kv_heads
    q = _normal_storage(seed, _S_Q, (B, Hq, D), dtype)
    k_pool = _normal_storage(seed, _S_K, (nb, Hkv, block_size, D), dtype)
    v_pool = _normal_storage(seed, _S_V, (nb, Hkv, block_size, D), dtype)
    k_new = _normal_storage(seed, _S_KNEW, (B, Hkv, D), dtype)
    v_new = _normal_storage(seed, _S_VNEW, (B, Hkv, D), dtype)
    ops = []
    for s in range(B):
        ops.append(("add", s))
        if lens[s] > 1:
            ops.append(("append", s, int(lens[s]) - 1))
    return Workload(
        name=name, dtype=dtype, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
        num_blocks=nb, scale=float(np.float32(1.0) / np.sqrt(np.float32(D))),
        context_lens=lens, perm=perm, q=q, k_pool=k_pool, v_pool=v_pool,
        k_new=k_new, v_new=v_new, ops=ops, seq_ids=list(range(B)), block_size=block_size,
        partition_size=partition_size, meta={"seed": seed, "pool_need": need},
    )


def _make_prefix_share(name, seed, prefix, tails_fn, prompts=32, n=8):
    """Parallel sampling: each prompt's prefix is stored once; n samples fork it."""
    tails = np.asarray(tails_fn(_rng(seed, _S_LENS), prompts * n), dtype=np.int32)
    lens = (prefix + tails + 1).astype(np.int32)
    pre_blocks = -(-prefix // BLOCK_SIZE)
    full_shared = prefix // BLOCK_SIZE
    need = prompts * pre_blocks
    for L in lens:
        need += -(-int(L) // BLOCK_SIZE) - full_shared
    nb = int(math.ceil(1.25 * need))
    perm = _rng(seed, _S_PERM).permutation(nb).astype(np.int32)
    Hq, Hkv, D, dtype = 32, 8, 128, "bf16"
    B = prompts * n
    q = _normal_storage(seed, _S_Q, (B, Hq, D), dtype)
    k_pool = _normal_storage(seed, _S_K, (nb, Hkv, BLOCK_SIZE, D), dtype)
    v_pool = _normal_storage(seed, _S_V, (nb, Hkv, BLOCK_SIZE, D), dtype)
    k_new = _normal_storage(seed, _S_KNEW, (B, Hkv, D), dtype)
    v_new = _normal_storage(seed, _S_VNEW, (B, Hkv, D), dtype)
    ops = []
    for p in range(prompts):
        root = p * n
        ops.append(("add", root))
        ops.append(("append", root, prefix))
        for c in range(1, n):
            ops.append(("fork", root, root + c))
        for c in range(n):
            if tails[root + c] > 0:
                ops.append(("append", root + c, int(tails[root + c])))
    return Workload(
        name=name, dtype=dtype, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
        num_blocks=nb, scale=float(np.float32(1.0) / np.sqrt(np.float32(D))),
        context_lens=lens, perm=perm, q=q, k_pool=k_pool, v_pool=v_pool,
        k_new=k_new, v_new=v_new, ops=ops, seq_ids=list(range(B)),
        meta={"seed": seed, "prompts": prompts, "samples": n, "prefix": prefix,
              "tails": tails, "pool_need": need},
    )


def make_workload(key: str, block_size: int = BLOCK_SIZE) -> Workload:
    """The named decode-step workloads (see CONFIGS); ``block_size`` resizes
    the pool's blocks (independent-sequence workloads only)."""
    key = key.lower()
    if block_size != BLOCK_SIZE:
        if key in ("c4", "c4b"):
            raise ValueError("the prefix-share workloads use 16-slot blocks")
        w = make_workload(key)
        return make_custom(w.name, w.dtype, w.context_lens, w.num_q_heads, w.num_kv_heads, w.head_dim,
                           seed=w.meta["seed"], partition_size=w.partition_size, block_size=block_size)
    if key == "c1":
        return make_custom("c1", "fp32", [1, 5, 16, 37], 2, 2, 64, seed=1, num_blocks=16)
    if key == "c2":
        return make_custom(
            "c2", "bf16", lambda r: r.integers(128, 4096, size=64, endpoint=True),
            32, 8, 128, seed=2)
    if key == "c3":
        return make_custom(
            "c3", "fp16", lambda r: r.integers(64, 2048, size=256, endpoint=True),
            40, 40, 128, seed=3)
    if key == "c4":
        return _make_prefix_share(
            "c4", 4, 1024, lambda r, m: r.integers(0, 512, size=m, endpoint=True))
    if key == "c4b":
        return _make_prefix_share("c4b", 4, 1000, lambda r, m: np.zeros(m, np.int64))
    if key == "c5":
        return make_custom(
            "c5", "fp16", lambda r: r.integers(4096, 8192, size=128, endpoint=True),
            64, 8, 128, seed=5, partition_size=512)
    if key == "c5tp8":
        # the same length draw as c5 (same seed and stream): one KV head's
        # share, with the automatic split -- at one KV head C5's 512-position
        # partitions are only 1.5 per wavefront, too coarse to balance
        return make_custom(
            "c5tp8", "fp16", lambda r: r.integers(4096, 8192, size=128, endpoint=True),
            8, 1, 128, seed=5)
    raise KeyError(key)


# ----------------------------------------------------------------------------
# Chunked-prefill steps
# ----------------------------------------------------------------------------

@dataclass
class PrefillWorkload:
    """One chunked-prefill step's inputs, as host arrays.

    Sequence s holds ``prior_lens[s]`` cached tokens before the step; the
    step appends ``chunk_lens[s]`` new tokens (their K/V in ``k_new`` /
    ``v_new``, their queries in ``q``, rows ``query_start[s]`` ..
    ``query_start[s+1]-1``) and attends over ``context_lens = prior + chunk``
    positions.  ``ops`` builds the pre-step state.
    """

    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    scale: float
    prior_lens: np.ndarray  # int32 [B]
    chunk_lens: np.ndarray  # int32 [B]
    perm: np.ndarray  # int32 [num_blocks]
    q: np.ndarray  # storage [N][Hq][D]
    k_pool: np.ndarray  # storage [num_blocks][Hkv][bs][D]
    v_pool: np.ndarray
    k_new: np.ndarray  # storage [N][Hkv][D]
    v_new: np.ndarray
    ops: list
    seq_ids: list
    block_size: int = BLOCK_SIZE
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return len(self.seq_ids)

    @property
    def num_tokens(self) -> int:
        return int(self.chunk_lens.sum())

    @property
    def context_lens(self) -> np.ndarray:
        return (self.prior_lens + self.chunk_lens).astype(np.int32)

    @property
    def query_start(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.chunk_lens)]).astype(np.int32)

    @property
    def max_query_len(self) -> int:
        return int(self.chunk_lens.max()) if len(self.chunk_lens) else 0

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if len(self.chunk_lens) else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return max(1, -(-self.max_context_len // self.block_size))


PREFILL_CONFIGS = {
    "p0": "tiny bf16: 6 seqs, chunks {1,7,16,33,130,0}, priors {0,20,5,64,100,9}, Hq=8, Hkv=2, D=64",
    "p1": "Llama-3.1-8B layer, bf16: 8 seqs x 512-token chunks, prior context U[0,3584], Hq=32, Hkv=8, D=128",
    "p2": "Qwen2.5-72B layer, fp16: 4 seqs x 1024-token chunks, prior context U[0,7168], Hq=64, Hkv=8, D=128",
    "p3": "mixed step, Llama shapes, bf16: 4 chunks of 512 (prior U[0,3584]) + 60 single tokens (prior U[127,4095])",
    "p4": "prefix-cache continuation, Llama shapes, bf16: 4 seqs x 64 new tokens after U[24576,32704] cached",
    "p5": "mixed step with a long chunk, Llama shapes, bf16: one 4096-token chunk (no prior) + 127 single tokens "
          "(prior U[127,4095])",
}


def make_prefill_custom(name, dtype, prior_lens, chunk_lens, num_q_heads, num_kv_heads, head_dim, seed,
                        pool_factor: float = 1.25, block_size: int = BLOCK_SIZE) -> PrefillWorkload:
    """Independent sequences: each holds its prior tokens, then one chunk is appended.

    ``prior_lens`` / ``chunk_lens`` may be lists or one callable
    ``rng -> (prior, chunk)`` drawn from the lengths stream.
    """
    if callable(prior_lens):
        prior, chunk = prior_lens(_rng(seed, _S_LENS))
    else:
        prior, chunk = prior_lens, chunk_lens
    prior = np.asarray(prior, dtype=np.int32)
    chunk = np.asarray(chunk, dtype=np.int32)
    assert prior.shape == chunk.shape and (prior >= 0).all() and (chunk >= 0).all()
    need, nb = _pool_blocks(prior + chunk, pool_factor, block_size)
    nb = max(nb, need, 1)
    B, N = len(prior), int(chunk.sum())
    D, Hq, Hkv = head_dim, num_q_heads, num_kv_heads
    perm = _rng(seed, _S_PERM).permutation(nb).astype(np.int32)
    q = _normal_storage(seed, _S_Q, (N, Hq, D), dtype)
    k_pool = _normal_storage(seed, _S_K, (nb, Hkv, block_size, D), dtype)
    v_pool = _normal_storage(seed, _S_V, (nb, Hkv, block_size, D), dtype)
    k_new = _normal_storage(seed, _S_KNEW, (N, Hkv, D), dtype)
    v_new = _normal_storage(seed, _S_VNEW, (N, Hkv, D), dtype)
    ops = []
    for s in range(B):
        ops.append(("add", s))
        if prior[s] > 0:
            ops.append(("append", s, int(prior[s])))
    return PrefillWorkload(
        name=name, dtype=dtype, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, num_blocks=nb,
        scale=float(np.float32(1.0) / np.sqrt(np.float32(D))), prior_lens=prior, chunk_lens=chunk,
        perm=perm, q=q, k_pool=k_pool, v_pool=v_pool, k_new=k_new, v_new=v_new, ops=ops,
        seq_ids=list(range(B)), block_size=block_size, meta={"seed": seed, "pool_need": need})


def make_prefill_workload(key: str, block_size: int = BLOCK_SIZE) -> PrefillWorkload:
    """The named chunked-prefill workloads (see PREFILL_CONFIGS)."""
    key = key.lower()
    if block_size != BLOCK_SIZE:
        w = make_prefill_workload(key)
        return make_prefill_custom(w.name, w.dtype, w.prior_lens, w.chunk_lens, w.num_q_heads, w.num_kv_heads,
                                   w.head_dim, seed=w.meta["seed"], block_size=block_size)
    if key == "p0":
        return make_prefill_custom("p0", "bf16", [0, 20, 5, 64, 100, 9], [1, 7, 16, 33, 130, 0], 8, 2, 64, seed=10)
    if key == "p1":
        return make_prefill_custom(
            "p1", "bf16", lambda r: (r.integers(0, 3584, size=8, endpoint=True), np.full(8, 512)),
            None, 32, 8, 128, seed=11)
    if key == "p2":
        return make_prefill_custom(
            "p2", "fp16", lambda r: (r.integers(0, 7168, size=4, endpoint=True), np.full(4, 1024)),
            None, 64, 8, 128, seed=12)
    if key == "p3":
        def lens(r):
            pri = np.concatenate([r.integers(0, 3584, size=4, endpoint=True),
                                  r.integers(127, 4095, size=60, endpoint=True)])
            return pri, np.concatenate([np.full(4, 512), np.ones(60, np.int64)])
        return make_prefill_custom("p3", "bf16", lens, None, 32, 8, 128, seed=13)
    if key == "p4":
        return make_prefill_custom(
            "p4", "bf16", lambda r: (r.integers(24576, 32704, size=4, endpoint=True), np.full(4, 64)),
            None, 32, 8, 128, seed=14)
    if key == "p5":
        def lens5(r):
            pri = np.concatenate([[0], r.integers(127, 4095, size=127, endpoint=True)])
            return pri, np.concatenate([[4096], np.ones(127, np.int64)])
        return make_prefill_custom("p5", "bf16", lens5, None, 32, 8, 128, seed=15)
    raise KeyError(key)
