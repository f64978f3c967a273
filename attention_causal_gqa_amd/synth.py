"""Seeded synthetic inputs for the five attention workloads.

This module holds no attention arithmetic: it only draws random tensors and
lays them out (dense BHTD tensors, a page pool and its block table).  The GPU
tests, the oracle checks and the benchmark all take their inputs from here, so
both sides of every comparison see exactly the same values.

Draws use a CPU ``torch.Generator`` seeded per workload: values are iid
N(0, 1) in float32, drawn in the order Q, K, V, then rounded to the target
dtype (round to nearest even for bfloat16).  Paged inputs draw seq_lens
first, then the page permutation, then q, then the K and V pools.
"""

from dataclasses import dataclass
import math

import torch

PAGE_SIZE = 16


@dataclass(frozen=True)
class PrefillShape:
    B: int
    Hq: int
    Hkv: int
    T: int
    d: int
    dtype: torch.dtype

    def flops(self) -> int:
        """Algorithmic flops: QK^T and PV over the causal triangle, diagonal included."""
        return 2 * self.B * self.Hq * self.d * self.T * (self.T + 1)


@dataclass(frozen=True)
class DecodeShape:
    B: int
    Hq: int
    Hkv: int
    d: int
    page_size: int
    L_lo: int
    L_hi: int
    dtype: torch.dtype

    @property
    def max_pages_per_seq(self) -> int:
        return -(-self.L_hi // self.page_size)


@dataclass(frozen=True)
class ChunkShape:
    """Chunked prefill over a paged cache: the last Tq tokens of sequences of L ~ U{L_lo..L_hi} cached tokens."""
    B: int
    Hq: int
    Hkv: int
    Tq: int
    d: int
    page_size: int
    L_lo: int
    L_hi: int
    dtype: torch.dtype

    @property
    def max_pages_per_seq(self) -> int:
        return -(-self.L_hi // self.page_size)


def chunk_flops(Hq, d, Tq, seq_lens) -> int:
    """Algorithmic flops of a chunked prefill: QK^T and PV over each query's visible keys.

    Query t of a sequence of L tokens sees L - Tq + t + 1 keys, so a sequence contributes
    Tq (L - Tq) + Tq (Tq + 1) / 2 query-key pairs, at 2 flops per multiply-add and two products.
    """
    pairs = sum(Tq * (int(L) - Tq) + Tq * (Tq + 1) // 2 for L in seq_lens)
    return 4 * Hq * d * pairs


@dataclass(frozen=True)
class VarlenShape:
    """Ragged prefill: S sequences of T ~ U{T_lo..T_hi} tokens packed along the token axis."""
    S: int
    Hq: int
    Hkv: int
    d: int
    T_lo: int
    T_hi: int
    dtype: torch.dtype


def varlen_flops(Hq, d, lens) -> int:
    """Algorithmic flops of a ragged prefill: each sequence's causal triangle, diagonal included."""
    return sum(2 * Hq * d * int(T) * (int(T) + 1) for T in lens)


def varlen_inputs(shape: VarlenShape, seed: int, *, lens=None):
    """q [N,Hq,d], k, v [N,Hkv,d] (CPU), cu_seqlens int32 [S+1] and max_seqlen.

    Draw order: lengths (unless given), then Q, K, V, iid N(0,1) rounded to shape.dtype."""
    g = torch.Generator().manual_seed(seed)
    if lens is None:
        lens = torch.randint(shape.T_lo, shape.T_hi + 1, (shape.S,), generator=g)
    lens = torch.as_tensor(lens, dtype=torch.int64)
    N = int(lens.sum())
    cu = torch.zeros(lens.numel() + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(lens, 0)
    q = torch.randn(N, shape.Hq, shape.d, generator=g).to(shape.dtype)
    k = torch.randn(N, shape.Hkv, shape.d, generator=g).to(shape.dtype)
    v = torch.randn(N, shape.Hkv, shape.d, generator=g).to(shape.dtype)
    return q, k, v, cu.to(torch.int32), int(lens.max()) if lens.numel() else 0


# The five workloads.  Prefill inputs are drawn with seed = workload number,
# decode inputs with seed = 100 + workload number.
WORKLOADS = {
    1: {"prefill": PrefillShape(1, 4, 4, 128, 64, torch.float32)},
    2: {"prefill": PrefillShape(1, 16, 8, 512, 128, torch.bfloat16)},
    3: {"prefill": PrefillShape(2, 32, 8, 2048, 128, torch.bfloat16)},
    4: {"decode": DecodeShape(32, 16, 8, 128, PAGE_SIZE, 32, 2048, torch.bfloat16)},
    5: {
        "prefill": PrefillShape(1, 32, 8, 8192, 128, torch.bfloat16),
        "decode": DecodeShape(64, 32, 8, 128, PAGE_SIZE, 1024, 8192, torch.bfloat16),
    },
}

# Chunked prefill (seed 6): 2048-token chunks at the end of sequences of 4096..16384 cached tokens.
WORKLOADS[6] = {"chunk": ChunkShape(4, 32, 8, 2048, 128, PAGE_SIZE, 4096, 16384, torch.bfloat16)}

# KV append (seed 7): the 2048-token chunks of workload 6's shape written into the paged cache.
WORKLOADS[7] = {"append": ChunkShape(4, 32, 8, 2048, 128, PAGE_SIZE, 4096, 16384, torch.bfloat16)}

# KV append fused with the chunked prefill (seed 11): workload 6's shape, the chunk's keys and values
# arriving as dense tensors instead of already cached.
WORKLOADS[11] = {"fused": ChunkShape(4, 32, 8, 2048, 128, PAGE_SIZE, 4096, 16384, torch.bfloat16)}

# Paged decode with the newest token's KV append fused (seed 112): workload 4's decode shape.
WORKLOADS[12] = {"decode_append": DecodeShape(32, 16, 8, 128, PAGE_SIZE, 32, 2048, torch.bfloat16)}

# Ragged prefill (seed 8): 16 sequences of 256..4096 tokens packed along the token axis.
WORKLOADS[8] = {"varlen": VarlenShape(16, 32, 8, 128, 256, 4096, torch.bfloat16)}

# Paged decode over an FP8 E4M3 cache (seed 109): workload 5's decode shape.
WORKLOADS[9] = {"decode_fp8": DecodeShape(64, 32, 8, 128, PAGE_SIZE, 1024, 8192, torch.bfloat16)}

# A serving-size decode batch (seed 110): 1024 short ragged sequences, K/V (1.1 GB) far larger than the MALL.
WORKLOADS[10] = {"decode": DecodeShape(1024, 32, 8, 128, PAGE_SIZE, 16, 512, torch.bfloat16)}

WORKLOAD_NAMES = {
    1: "causal MHA prefill fp32 B1 H4 T128 d64",
    2: "causal GQA prefill bf16 B1 Hq16 Hkv8 T512 d128",
    3: "causal GQA prefill bf16 B2 Hq32 Hkv8 T2048 d128",
    4: "paged decode bf16 B32 Hq16 Hkv8 d128 page16 L~U[32,2048]",
    5: "mixed: prefill bf16 B1 Hq32 Hkv8 T8192 d128 + paged decode bf16 B64 Hq32 Hkv8 d128 page16 L~U[1024,8192]",
    6: "chunked prefill bf16 over a paged cache B4 Hq32 Hkv8 Tq2048 d128 page16 L~U[4096,16384]",
    7: "KV append bf16 into a paged cache B4 Hkv8 Tn2048 d128 page16 L~U[4096,16384]",
    8: "ragged prefill bf16 over packed tokens S16 Hq32 Hkv8 d128 T~U[256,4096]",
    9: "paged decode over an FP8 E4M3 cache B64 Hq32 Hkv8 d128 page16 L~U[1024,8192]",
    10: "paged decode bf16 serving batch B1024 Hq32 Hkv8 d128 page16 L~U[16,512]",
    11: "KV append + chunked prefill bf16 in one launch B4 Hq32 Hkv8 Tq2048 d128 page16 L~U[4096,16384]",
    12: "paged decode bf16 with the newest token's KV append fused B32 Hq16 Hkv8 d128 page16 L~U[32,2048]",
}


def prefill_inputs(shape: PrefillShape, seed: int):
    """q [B,Hq,T,d], k, v [B,Hkv,T,d] on the CPU, iid N(0,1) rounded to shape.dtype."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(shape.B, shape.Hq, shape.T, shape.d, generator=g)
    k = torch.randn(shape.B, shape.Hkv, shape.T, shape.d, generator=g)
    v = torch.randn(shape.B, shape.Hkv, shape.T, shape.d, generator=g)
    return q.to(shape.dtype), k.to(shape.dtype), v.to(shape.dtype)


@dataclass
class PagedInputs:
    q: torch.Tensor            # [B, Hq, d]
    k_pages: torch.Tensor      # [num_pages, Hkv, page_size, d]
    v_pages: torch.Tensor      # [num_pages, Hkv, page_size, d]
    block_table: torch.Tensor  # [B, W] int32, unused entries -1
    seq_lens: torch.Tensor     # [B] int32
    page_size: int

    @property
    def max_pages_per_seq(self) -> int:
        return self.block_table.shape[1]

    def kv_bytes(self) -> int:
        """Bytes of K and V that valid tokens occupy (unused slots excluded)."""
        Hkv, d = self.k_pages.shape[1], self.k_pages.shape[3]
        return 2 * int(self.seq_lens.sum()) * Hkv * d * self.k_pages.element_size()

    def algorithmic_bytes(self) -> int:
        """K/V of valid tokens + q + out + used block-table entries + seq_lens."""
        es = self.q.element_size()
        used_pages = int(((self.seq_lens.long() + self.page_size - 1) // self.page_size).sum())
        return self.kv_bytes() + 2 * self.q.numel() * es + 4 * used_pages + 4 * self.seq_lens.numel()


def _pool_layout(seq_lens, page_size, W, g, extra_pages):
    """Block table over a pool of exactly sum(ceil(L/page_size)) pages (+ extra), in randperm order."""
    B = seq_lens.shape[0]
    npages = (seq_lens + page_size - 1) // page_size
    used = int(npages.sum())
    num_pages = used + extra_pages
    perm = torch.randperm(num_pages, generator=g)
    table = torch.full((B, W), -1, dtype=torch.int32)
    off = 0
    for b in range(B):
        n = int(npages[b])
        table[b, :n] = perm[off : off + n].to(torch.int32)
        off += n
    return table, num_pages


def _poison(pages, table, seq_lens, page_size, extra_pages, value):
    """Write ``value`` into every slot no valid token occupies."""
    referenced = torch.zeros(pages.shape[0], dtype=torch.bool)
    for b in range(table.shape[0]):
        L = int(seq_lens[b])
        n = -(-L // page_size)
        if n:
            referenced[table[b, :n].long()] = True
            tail = L - (n - 1) * page_size
            pages[int(table[b, n - 1]), :, tail:, :] = value
    pages[~referenced] = value


def paged_inputs(shape: DecodeShape, seed: int, *, seq_lens=None, extra_pages=0, poison=None, B=None):
    """Paged decode inputs: seq_lens ~ U{L_lo..L_hi} (unless given), pool in randperm order.

    ``poison`` (e.g. float('nan')) fills every slot no valid token occupies,
    including ``extra_pages`` pages that no sequence references.
    """
    g = torch.Generator().manual_seed(seed)
    B = shape.B if B is None else B
    if seq_lens is None:
        seq_lens = torch.randint(shape.L_lo, shape.L_hi + 1, (B,), generator=g)
    seq_lens = torch.as_tensor(seq_lens, dtype=torch.int64)
    W = shape.max_pages_per_seq
    table, num_pages = _pool_layout(seq_lens, shape.page_size, W, g, extra_pages)
    q = torch.randn(B, shape.Hq, shape.d, generator=g).to(shape.dtype)
    pool_shape = (num_pages, shape.Hkv, shape.page_size, shape.d)
    k_pages = torch.randn(pool_shape, generator=g).to(shape.dtype)
    v_pages = torch.randn(pool_shape, generator=g).to(shape.dtype)
    if poison is not None:
        _poison(k_pages, table, seq_lens, shape.page_size, extra_pages, poison)
        _poison(v_pages, table, seq_lens, shape.page_size, extra_pages, poison)
    return PagedInputs(q, k_pages, v_pages, table, seq_lens.to(torch.int32), shape.page_size)


@dataclass
class ChunkInputs:
    q: torch.Tensor            # [B, Hq, Tq, d]
    k_pages: torch.Tensor      # [num_pages, Hkv, page_size, d]
    v_pages: torch.Tensor      # [num_pages, Hkv, page_size, d]
    block_table: torch.Tensor  # [B, W] int32, unused entries -1
    seq_lens: torch.Tensor     # [B] int32, each >= Tq
    page_size: int


def chunk_inputs(shape: ChunkShape, seed: int, *, seq_lens=None, poison=None, B=None):
    """Chunked-prefill inputs: seq_lens ~ U{L_lo..L_hi} (unless given), pool in randperm order, q for the chunk.

    Draw order: seq_lens, page permutation, q, K pool, V pool.  ``poison`` fills every unused slot.
    """
    g = torch.Generator().manual_seed(seed)
    B = shape.B if B is None else B
    if seq_lens is None:
        seq_lens = torch.randint(shape.L_lo, shape.L_hi + 1, (B,), generator=g)
    seq_lens = torch.as_tensor(seq_lens, dtype=torch.int64)
    W = shape.max_pages_per_seq
    table, num_pages = _pool_layout(seq_lens, shape.page_size, W, g, 0)
    q = torch.randn(B, shape.Hq, shape.Tq, shape.d, generator=g).to(shape.dtype)
    pool_shape = (num_pages, shape.Hkv, shape.page_size, shape.d)
    k_pages = torch.randn(pool_shape, generator=g).to(shape.dtype)
    v_pages = torch.randn(pool_shape, generator=g).to(shape.dtype)
    if poison is not None:
        _poison(k_pages, table, seq_lens, shape.page_size, 0, poison)
        _poison(v_pages, table, seq_lens, shape.page_size, 0, poison)
    return ChunkInputs(q, k_pages, v_pages, table, seq_lens.to(torch.int32), shape.page_size)


@dataclass
class AppendInputs:
    k_new: torch.Tensor        # [B, Hkv, Tn, d]
    v_new: torch.Tensor        # [B, Hkv, Tn, d]
    k_pages: torch.Tensor      # [num_pages, Hkv, page_size, d]
    v_pages: torch.Tensor      # [num_pages, Hkv, page_size, d]
    block_table: torch.Tensor  # [B, W] int32, unused entries -1
    seq_lens: torch.Tensor     # [B] int32, lengths after the append (>= Tn)
    page_size: int

    def algorithmic_bytes(self) -> int:
        """k_new and v_new read once and written once, plus the block-table entries and seq_lens read."""
        B, Hkv, Tn, d = self.k_new.shape
        return 4 * self.k_new.numel() * self.k_new.element_size() + 4 * B * (-(-Tn // self.page_size) + 1)


def append_inputs(shape: ChunkShape, seed: int, *, seq_lens=None, poison=None):
    """KV-append inputs: seq_lens ~ U{L_lo..L_hi} (lengths after the append), pool in randperm order,
    k_new / v_new [B, Hkv, Tq, d] for the last Tq tokens.  Draw order: seq_lens, page permutation,
    K pool, V pool, k_new, v_new.  ``poison`` fills every unused slot of the pools."""
    g = torch.Generator().manual_seed(seed)
    B = shape.B
    if seq_lens is None:
        seq_lens = torch.randint(shape.L_lo, shape.L_hi + 1, (B,), generator=g)
    seq_lens = torch.as_tensor(seq_lens, dtype=torch.int64)
    table, num_pages = _pool_layout(seq_lens, shape.page_size, shape.max_pages_per_seq, g, 0)
    pool_shape = (num_pages, shape.Hkv, shape.page_size, shape.d)
    k_pages = torch.randn(pool_shape, generator=g).to(shape.dtype)
    v_pages = torch.randn(pool_shape, generator=g).to(shape.dtype)
    if poison is not None:
        _poison(k_pages, table, seq_lens, shape.page_size, 0, poison)
        _poison(v_pages, table, seq_lens, shape.page_size, 0, poison)
    k_new = torch.randn(B, shape.Hkv, shape.Tq, shape.d, generator=g).to(shape.dtype)
    v_new = torch.randn(B, shape.Hkv, shape.Tq, shape.d, generator=g).to(shape.dtype)
    return AppendInputs(k_new, v_new, k_pages, v_pages, table, seq_lens.to(torch.int32), shape.page_size)


@dataclass
class FusedInputs:
    q: torch.Tensor            # [B, Hq, Tq, d]
    k_new: torch.Tensor        # [B, Hkv, Tq, d]: the chunk's keys
    v_new: torch.Tensor        # [B, Hkv, Tq, d]: the chunk's values
    k_pages: torch.Tensor      # [num_pages, Hkv, page_size, d]
    v_pages: torch.Tensor      # [num_pages, Hkv, page_size, d]
    block_table: torch.Tensor  # [B, W] int32, unused entries -1
    seq_lens: torch.Tensor     # [B] int32, lengths after the append (>= Tq)
    page_size: int


def chunk_slots(block_table, seq_lens, Tq, page_size):
    """(pages, slots) of the last Tq positions of every sequence, sequence-major, position order."""
    pages, slots = [], []
    for b, L in enumerate(seq_lens.tolist()):
        pos = torch.arange(L - Tq, L)
        pages.append(block_table[b].long()[pos // page_size])
        slots.append(pos % page_size)
    return torch.cat(pages), torch.cat(slots)


def fused_inputs(shape: ChunkShape, seed: int, *, seq_lens=None, poison=None, stale=None):
    """Inputs of the KV append fused with the chunked prefill: append_inputs(shape, seed, ...) (pools,
    table, lengths, the chunk's k_new / v_new), then q [B, Hq, Tq, d] from a generator seeded
    seed + 1000000.  ``stale``, if given, fills the chunk's own slots of the pools (values the
    fused call overwrites and must never read)."""
    a = append_inputs(shape, seed, seq_lens=seq_lens, poison=poison)
    g = torch.Generator().manual_seed(seed + 1000000)
    q = torch.randn(shape.B, shape.Hq, shape.Tq, shape.d, generator=g).to(shape.dtype)
    if stale is not None:
        pages, slots = chunk_slots(a.block_table, a.seq_lens, shape.Tq, a.page_size)
        a.k_pages[pages, :, slots] = stale
        a.v_pages[pages, :, slots] = stale
    return FusedInputs(q, a.k_new, a.v_new, a.k_pages, a.v_pages, a.block_table, a.seq_lens, a.page_size)


def decode_append_inputs(shape: DecodeShape, seed: int, *, seq_lens=None, poison=None, stale=None):
    """Inputs of the decode with the newest token's append fused: paged_inputs(shape, seed, ...) (seq_lens
    are the lengths after the append), then k_new, v_new [B, Hkv, d] from a generator seeded seed + 1000000.
    ``stale``, if given, fills each sequence's newest-token slot in the pools (values the call overwrites and
    must never read).  Returns (PagedInputs, k_new, v_new)."""
    inp = paged_inputs(shape, seed, seq_lens=seq_lens, poison=poison)
    B = inp.q.shape[0]
    g = torch.Generator().manual_seed(seed + 1000000)
    k_new = torch.randn(B, shape.Hkv, shape.d, generator=g).to(shape.dtype)
    v_new = torch.randn(B, shape.Hkv, shape.d, generator=g).to(shape.dtype)
    if stale is not None:
        for b, L in enumerate(inp.seq_lens.tolist()):
            if L > 0:
                page = int(inp.block_table[b, (L - 1) // shape.page_size])
                inp.k_pages[page, :, (L - 1) % shape.page_size] = stale
                inp.v_pages[page, :, (L - 1) % shape.page_size] = stale
    return inp, k_new, v_new


@dataclass
class Fp8PagedInputs:
    q: torch.Tensor            # [B, Hq, d] bf16
    k_codes: torch.Tensor      # [num_pages, Hkv, page_size, d] uint8, FP8 E4M3 codes
    v_codes: torch.Tensor
    k_scale: float
    v_scale: float
    block_table: torch.Tensor  # [B, W] int32
    seq_lens: torch.Tensor     # [B] int32
    page_size: int

    def algorithmic_bytes(self) -> int:
        """K/V codes of valid tokens (one byte each) + q + out + used block-table entries + seq_lens."""
        Hkv, d = self.k_codes.shape[1], self.k_codes.shape[3]
        used = int(((self.seq_lens.long() + self.page_size - 1) // self.page_size).sum())
        return 2 * int(self.seq_lens.sum()) * Hkv * d + 2 * self.q.numel() * 2 + 4 * used + 4 * self.seq_lens.numel()


def fp8_paged_inputs(shape: DecodeShape, seed: int, *, seq_lens=None, poison_nan=False):
    """Paged decode inputs quantised to FP8 E4M3: draw as paged_inputs (seq_lens, permutation, q, K, V in
    float32), then scale each pool by 448 / max|x| and round to the nearest E4M3 code (torch's float8_e4m3fn
    cast); k_scale / v_scale are the inverse factors, so code value * scale approximates the drawn value.
    ``poison_nan`` writes the NaN code 0x7F into every slot no valid token occupies."""
    g = torch.Generator().manual_seed(seed)
    B = shape.B
    if seq_lens is None:
        seq_lens = torch.randint(shape.L_lo, shape.L_hi + 1, (B,), generator=g)
    seq_lens = torch.as_tensor(seq_lens, dtype=torch.int64)
    table, num_pages = _pool_layout(seq_lens, shape.page_size, shape.max_pages_per_seq, g, 0)
    q = torch.randn(B, shape.Hq, shape.d, generator=g).to(torch.bfloat16)
    pool_shape = (num_pages, shape.Hkv, shape.page_size, shape.d)
    codes, scales = [], []
    for _ in range(2):
        x = torch.randn(pool_shape, generator=g)
        s = float(x.abs().max()) / 448.0
        c = (x / s).to(torch.float8_e4m3fn).view(torch.uint8).clone()
        if poison_nan:
            _poison(c, table, seq_lens, shape.page_size, 0, 0x7F)
        codes.append(c)
        scales.append(s)
    return Fp8PagedInputs(q, codes[0], codes[1], scales[0], scales[1], table, seq_lens.to(torch.int32),
                          shape.page_size)


def paged_from_dense(k, v, seq_lens, page_size, seed, W=None, poison=None):
    """Scatter dense K/V [B,Hkv,T,d] (tokens 0..L_b-1 of each b) into a permuted page pool.

    Returns (k_pages, v_pages, block_table int32, seq_lens int32).
    """
    B, Hkv, T, d = k.shape
    seq_lens = torch.as_tensor(seq_lens, dtype=torch.int64)
    W = W if W is not None else -(-T // page_size)
    g = torch.Generator().manual_seed(seed)
    table, num_pages = _pool_layout(seq_lens, page_size, W, g, 0)
    fill = float("nan") if poison is None else poison
    k_pages = torch.full((num_pages, Hkv, page_size, d), fill, dtype=k.dtype)
    v_pages = torch.full((num_pages, Hkv, page_size, d), fill, dtype=v.dtype)
    for b in range(B):
        L = int(seq_lens[b])
        for j in range(0, L, page_size):
            n = min(page_size, L - j)
            p = int(table[b, j // page_size])
            k_pages[p, :, :n] = k[b, :, j : j + n]
            v_pages[p, :, :n] = v[b, :, j : j + n]
    return k_pages, v_pages, table, seq_lens.to(torch.int32)


def permute_pages(k_pages, v_pages, block_table, seed):
    """Same cache under a different physical page order: pages moved, table rewritten."""
    g = torch.Generator().manual_seed(seed)
    P = k_pages.shape[0]
    perm = torch.randperm(P, generator=g)          # new position of old page i is perm[i]
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(P)
    k2 = k_pages[inv]
    v2 = v_pages[inv]
    t2 = block_table.clone()
    used = t2 >= 0
    t2[used] = perm[t2[used].long()].to(torch.int32)
    return k2, v2, t2


def fp32_scale(d: int) -> float:
    """1/sqrt(d) rounded to float32: the value the kernels receive."""
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))
