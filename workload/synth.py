"""Seeded synthetic inputs for the paged KV-cache data plane.

Test and benchmark infrastructure, shared by the fp64 oracle and the GPU path.
It stands in for the CPU control plane that the Nano-vLLM write-up describes
(the scheduler and the block manager, "Nano-vLLM part 1", sections 3-4 and
5.2): it draws sequence lengths and physical block ids and emits what that
control plane hands to the GPU -- block tables, context lengths, cu_seqlens
and slot mappings.  It also draws the bf16 Q/K/V values and lays out the
starting cache image: every slot holds a NaN poison (freed blocks are never
zeroed, section 4.3 of the same page) except the slots of tokens that earlier
steps already stored.  It contains none of the attention arithmetic.

Values are counter-based: element ``e`` of tensor ``tag`` is a pure function
of ``(seed, tag, e)`` built from integer hashing plus one IEEE fp32 multiply
and an integer round-to-nearest-even to bf16, so CPU and GPU produce the same
bits and any row can be regenerated on its own (the oracle regenerates the
rows of a few sampled sequences instead of holding a 43 GB cache image).

Layout conventions (the readings the whole repository uses):
  * K/V cache: one bf16 tensor each, ``[num_blocks * block_size, Hkv, d]``,
    row-major; a slot is one token's ``Hkv * d`` elements.
  * block_tables: int32 ``[num_seqs, max_blocks_per_seq]``, padded with -1.
  * slot_mapping: int32 ``[num_new_tokens]``; -1 marks a padding entry.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch

BF16_POISON = 0x7FC0  # quiet NaN in bf16; marks slots that hold no live token

TAG_Q, TAG_K, TAG_V, TAG_PAD = 1, 2, 3, 4
_M32 = 0xFFFFFFFF
_MUL = 0x45D9F3B  # odd 32-bit hash multiplier
# four 16-bit uniforms: mean 4 * 32767.5, variance 4 * (65536**2 - 1) / 12
_IH_MEAN = 131070
_IH_INV_STD = float(np.float32(1.0 / math.sqrt((65536.0 ** 2 - 1.0) / 3.0)))


def _hash32_int(x: int) -> int:
    x &= _M32
    x = (((x >> 16) ^ x) * _MUL) & _M32
    x = (((x >> 16) ^ x) * _MUL) & _M32
    return (x >> 16) ^ x


def _hash32(x: torch.Tensor) -> torch.Tensor:
    # x: int32 tensor; products wrap modulo 2**32, shifts are made logical by masking
    x = (((x >> 16) & 0xFFFF) ^ x) * _MUL
    x = (((x >> 16) & 0xFFFF) ^ x) * _MUL
    return ((x >> 16) & 0xFFFF) ^ x


def _stream_keys(seed: int, tag: int):
    k1 = _hash32_int(seed * 0x9E3779B1 + tag * 0x85EBCA6B + 0x27D4EB2F)
    k2 = _hash32_int(k1 ^ 0x165667B1)
    k3 = _hash32_int(k2 ^ 0x61C88647)
    return k1, k2, k3


def _as_i32(v: int) -> int:
    v &= _M32
    return v - (1 << 32) if v >= (1 << 31) else v


def bf16_values(seed: int, tag: int, elem: torch.Tensor) -> torch.Tensor:
    """Approximately N(0,1) bf16 values for int64 element indices ``elem``.

    Irwin-Hall sum of four 16-bit uniforms taken from two 32-bit hashes,
    standardised, rounded to fp32 by one multiply, then to bf16 by integer
    round-to-nearest-even.  Identical bits on every torch device
    (``bf16_value_ref`` is the same map on Python integers).
    """
    k1, k2, k3 = (_as_i32(k) for k in _stream_keys(seed, tag))
    lo = (elem & _M32).to(torch.int32)  # wraps into int32: same low 32 bits
    hi = ((elem >> 32) & _M32).to(torch.int32)
    a = _hash32(lo ^ k1)
    b = _hash32(a ^ hi ^ k2)
    c = _hash32(b ^ k3)
    u = (b & 0xFFFF) + ((b >> 16) & 0xFFFF) + (c & 0xFFFF) + ((c >> 16) & 0xFFFF)
    del a, b, c
    x = (u - _IH_MEAN).to(torch.float32) * torch.tensor(_IH_INV_STD, dtype=torch.float32,
                                                         device=elem.device)
    bits = x.view(torch.int32)
    r = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16) & 0xFFFF
    r = r - ((r >> 15) & 1) * 0x10000
    return r.to(torch.int16).view(torch.bfloat16)


def bf16_value_ref(seed: int, tag: int, e: int) -> int:
    """bf16 bit pattern of one element, on Python integers (checks ``bf16_values``)."""
    k1, k2, k3 = _stream_keys(seed, tag)
    a = _hash32_int((e & _M32) ^ k1)
    b = _hash32_int(a ^ ((e >> 32) & _M32) ^ k2)
    c = _hash32_int(b ^ k3)
    u = (b & 0xFFFF) + (b >> 16) + (c & 0xFFFF) + (c >> 16)
    x = np.float32(u - _IH_MEAN) * np.float32(_IH_INV_STD)
    bits = int(np.array([x], dtype=np.float32).view(np.uint32)[0])
    return ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16) & 0xFFFF


def rows_values(seed: int, tag: int, rows: torch.Tensor, heads: int, head_dim: int,
                max_elems: Optional[int] = None) -> torch.Tensor:
    """bf16 ``[len(rows), heads, head_dim]`` for logical row ids ``rows`` (int64)."""
    if max_elems is None:  # small chunks stay in the host caches; big ones fill the GPU
        max_elems = (1 << 22) if rows.device.type == "cpu" else (1 << 26)
    width = heads * head_dim
    out = torch.empty((rows.numel(), width), dtype=torch.bfloat16, device=rows.device)
    step = max(1, max_elems // width)
    col = torch.arange(width, dtype=torch.int64, device=rows.device)
    for s in range(0, rows.numel(), step):
        r = rows[s:s + step].to(torch.int64)
        out[s:s + step] = bf16_values(seed, tag, r[:, None] * width + col[None, :])
    return out.view(rows.numel(), heads, head_dim)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw uint16 bit patterns of a bf16 tensor (on the host)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


@dataclasses.dataclass
class Workload:
    """A batch of sequences as the control plane hands it to the data plane.

    Every sequence ``s`` has ``Lk[s] = prefix_len + hist[s] + lq[s]`` key
    positions.  Positions ``< prefix_len`` are the shared prefix (logical K/V
    rows ``0 .. prefix_len-1``, the same physical blocks in every table);
    the next ``hist[s]`` positions were stored by earlier steps; the last
    ``lq[s]`` positions are this step's new tokens: their K/V go through the
    store, and in prefill they are also the query rows.  Decode has
    ``lq = 1`` (or 0 for an empty context) and one query row per sequence.
    """

    name: str
    kind: str  # "decode" | "prefill"
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    scale: float
    causal: bool
    prefix_len: int
    hist: np.ndarray        # int64 [S]
    lq: np.ndarray          # int64 [S]
    q_row0: np.ndarray      # int64 [S]: logical Q row of the sequence's first query
    kv_row0: np.ndarray     # int64 [S]: logical K/V row of position prefix_len
    block_tables: np.ndarray  # int32 [S, max_blocks_per_seq]
    pad_tokens: int = 0     # extra store entries with slot -1
    seq_ids: Optional[np.ndarray] = None  # indices into the parent workload

    # ---- derived metadata (control-plane outputs) -------------------------------
    @property
    def num_seqs(self) -> int:
        return int(self.lq.shape[0])

    @property
    def lk(self) -> np.ndarray:
        return self.prefix_len + self.hist + self.lq

    @property
    def context_lens(self) -> np.ndarray:
        return self.lk.astype(np.int32)

    @property
    def cu_seqlens_q(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lq)]).astype(np.int32)

    @property
    def cu_seqlens_k(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lk)]).astype(np.int32)

    @property
    def num_slots(self) -> int:
        return self.num_blocks * self.block_size

    @property
    def num_q_rows(self) -> int:
        return self.num_seqs if self.kind == "decode" else int(self.lq.sum())

    def kv_rows(self, s: int, positions: np.ndarray) -> np.ndarray:
        """Logical K/V row ids of key positions of sequence ``s``."""
        positions = np.asarray(positions, dtype=np.int64)
        own = self.kv_row0[s] + (positions - self.prefix_len)
        return np.where(positions < self.prefix_len, positions, own)

    def slots(self, s: int, positions: np.ndarray) -> np.ndarray:
        """Physical slot of key positions of sequence ``s`` (block manager's map)."""
        positions = np.asarray(positions, dtype=np.int64)
        blk = self.block_tables[s, positions // self.block_size].astype(np.int64)
        assert (blk >= 0).all(), "position beyond the sequence's allocated blocks"
        return blk * self.block_size + positions % self.block_size

    def q_rows(self, s: int) -> np.ndarray:
        if self.kind == "decode":
            return np.array([self.q_row0[s]], dtype=np.int64)
        return self.q_row0[s] + np.arange(self.lq[s], dtype=np.int64)

    def new_tokens(self):
        """(logical K/V rows, slots) of this step's stores, in slot_mapping order."""
        rows, slots = [], []
        for s in range(self.num_seqs):
            pos = np.arange(self.lk[s] - self.lq[s], self.lk[s], dtype=np.int64)
            rows.append(self.kv_rows(s, pos))
            slots.append(self.slots(s, pos))
        rows = np.concatenate(rows) if rows else np.zeros(0, np.int64)
        slots = np.concatenate(slots) if slots else np.zeros(0, np.int64)
        return rows, slots

    def history_tokens(self):
        """(logical rows, slots) of positions stored before this step."""
        rows, slots = [], []
        if self.prefix_len and self.num_seqs:
            pos = np.arange(self.prefix_len, dtype=np.int64)
            rows.append(self.kv_rows(0, pos))
            slots.append(self.slots(0, pos))
        for s in range(self.num_seqs):
            pos = np.arange(self.prefix_len, self.prefix_len + self.hist[s], dtype=np.int64)
            rows.append(self.kv_rows(s, pos))
            slots.append(self.slots(s, pos))
        rows = np.concatenate(rows) if rows else np.zeros(0, np.int64)
        slots = np.concatenate(slots) if slots else np.zeros(0, np.int64)
        return rows, slots

    @property
    def slot_mapping(self) -> np.ndarray:
        _, slots = self.new_tokens()
        return np.concatenate([slots, -np.ones(self.pad_tokens, np.int64)]).astype(np.int32)

    @property
    def num_new_tokens(self) -> int:
        return int(self.lq.sum()) + self.pad_tokens

    @property
    def max_context_len(self) -> int:
        return int(self.lk.max()) if self.num_seqs else 0

    # ---- values -------------------------------------------------------------------
    def q_all_rows(self) -> np.ndarray:
        if self.kind == "decode":
            return self.q_row0.astype(np.int64)
        if self.num_seqs == 0:
            return np.zeros(0, np.int64)
        return np.concatenate([self.q_rows(s) for s in range(self.num_seqs)])

    def _pad_rows(self) -> np.ndarray:
        return np.arange(self.pad_tokens, dtype=np.int64)

    def materialize(self, device="cpu", with_history: bool = True) -> dict:
        """Device tensors for one step: inputs plus the starting cache image."""
        dev = torch.device(device)
        H, Hkv, d = self.num_q_heads, self.num_kv_heads, self.head_dim
        t = {}
        qr = torch.from_numpy(self.q_all_rows()).to(dev)
        t["q"] = rows_values(self.seed, TAG_Q, qr, H, d)
        rows, _ = self.new_tokens()
        r = torch.from_numpy(rows).to(dev)
        k_new = rows_values(self.seed, TAG_K, r, Hkv, d)
        v_new = rows_values(self.seed, TAG_V, r, Hkv, d)
        if self.pad_tokens:
            pr = torch.from_numpy(self._pad_rows()).to(dev)
            k_new = torch.cat([k_new, rows_values(self.seed, TAG_PAD, pr, Hkv, d)])
            v_new = torch.cat([v_new, rows_values(self.seed + 1, TAG_PAD, pr, Hkv, d)])
        t["k_new"], t["v_new"] = k_new.contiguous(), v_new.contiguous()
        t["slot_mapping"] = torch.from_numpy(self.slot_mapping).to(dev)
        t["block_tables"] = torch.from_numpy(np.ascontiguousarray(self.block_tables)).to(dev)
        t["context_lens"] = torch.from_numpy(self.context_lens).to(dev)
        t["cu_seqlens_q"] = torch.from_numpy(self.cu_seqlens_q).to(dev)
        t["cu_seqlens_k"] = torch.from_numpy(self.cu_seqlens_k).to(dev)
        t["k_cache"], t["v_cache"] = self.cache_image(dev, with_history)
        return t

    def cache_image(self, device, with_history: bool = True):
        dev = torch.device(device)
        Hkv, d = self.num_kv_heads, self.head_dim
        shape = (self.num_slots, Hkv, d)
        kc = torch.full(shape, BF16_POISON, dtype=torch.int16, device=dev)  # 0x7FC0 < 2**15
        vc = kc.clone()
        kc, vc = kc.view(torch.bfloat16), vc.view(torch.bfloat16)
        if with_history:
            rows, slots = self.history_tokens()
            step = max(1, (1 << 24) // (Hkv * d))
            for s0 in range(0, rows.shape[0], step):
                r = torch.from_numpy(rows[s0:s0 + step]).to(dev)
                sl = torch.from_numpy(slots[s0:s0 + step]).to(dev)
                kc[sl] = rows_values(self.seed, TAG_K, r, Hkv, d)
                vc[sl] = rows_values(self.seed, TAG_V, r, Hkv, d)
        return kc, vc

    def dense(self, s: int):
        """Host uint16 bits: (q [Lq or 1, Hq, d], k [Lk, Hkv, d], v [Lk, Hkv, d]).

        The contiguous, unpaged tokens of sequence ``s`` straight from the value
        generator; they never pass through a cache image.
        """
        H, Hkv, d = self.num_q_heads, self.num_kv_heads, self.head_dim
        qr = torch.from_numpy(self.q_rows(s))
        kr = torch.from_numpy(self.kv_rows(s, np.arange(self.lk[s])))
        return (bf16_bits(rows_values(self.seed, TAG_Q, qr, H, d)),
                bf16_bits(rows_values(self.seed, TAG_K, kr, Hkv, d)),
                bf16_bits(rows_values(self.seed, TAG_V, kr, Hkv, d)))

    def host_inputs(self, with_history: bool = True) -> dict:
        """materialize() on the CPU, as host numpy arrays (bf16 as uint16 bits)."""
        t = self.materialize("cpu", with_history)
        out = {}
        for k, v in t.items():
            out[k] = bf16_bits(v) if v.dtype == torch.bfloat16 else v.numpy()
        return out

    # ---- restriction ---------------------------------------------------------------
    def subset(self, idx: Sequence[int], name: Optional[str] = None) -> "Workload":
        """The same logical tokens for a few sequences, on a compact block pool.

        Physical ids are renumbered in order of first appearance; values are keyed by
        logical rows, so every sequence sees the same K/V as in the full workload.
        """
        idx = np.asarray(idx, dtype=np.int64)
        bt = self.block_tables[idx]
        used = [int(b) for b in bt.reshape(-1) if b >= 0]
        remap = {}
        for b in used:
            if b not in remap:
                remap[b] = len(remap)
        new_bt = np.full_like(bt, -1)
        for (i, j), b in np.ndenumerate(bt):
            if b >= 0:
                new_bt[i, j] = remap[int(b)]
        parent = self.seq_ids if self.seq_ids is not None else np.arange(self.num_seqs)
        return dataclasses.replace(
            self, name=name or f"{self.name}[subset {len(idx)}]",
            num_blocks=max(1, len(remap)), hist=self.hist[idx].copy(), lq=self.lq[idx].copy(),
            q_row0=self.q_row0[idx].copy(), kv_row0=self.kv_row0[idx].copy(),
            block_tables=new_bt, pad_tokens=0, seq_ids=parent[idx])

    def permute_blocks(self, perm: np.ndarray) -> "Workload":
        """Same sequences with physical block b moved to perm[b]."""
        perm = np.asarray(perm, dtype=np.int64)
        bt = np.where(self.block_tables >= 0, perm[np.maximum(self.block_tables, 0)], -1)
        return dataclasses.replace(self, block_tables=bt.astype(np.int32),
                                   name=self.name + "[permuted]")


def _tables_from_ids(nblk: np.ndarray, ids: np.ndarray, max_blocks: int,
                     shared: Optional[np.ndarray] = None) -> np.ndarray:
    S = nblk.shape[0]
    bt = np.full((S, max_blocks), -1, dtype=np.int32)
    pos = 0
    ns = 0 if shared is None else shared.shape[0]
    for s in range(S):
        if ns:
            bt[s, :ns] = shared
        n = int(nblk[s])
        bt[s, ns:ns + n] = ids[pos:pos + n]
        pos += n
    return bt


def build(kind: str, lq, hist, *, num_q_heads: int, num_kv_heads: int, head_dim: int,
          block_size: int, seed: int, prefix_len: int = 0, num_blocks: Optional[int] = None,
          id_mode: str = "choice", pool_factor: float = 1.1, max_blocks_per_seq: Optional[int] = None,
          scale: Optional[float] = None, causal: bool = True, pad_tokens: int = 0,
          rng: Optional[np.random.Generator] = None, name: str = "custom") -> Workload:
    """Allocate blocks for the given per-sequence lengths and return the workload.

    ``id_mode``: "choice" draws ``demand`` distinct ids from the pool (fragmented,
    assigned in sequence order); "perm" walks a random permutation of the pool;
    "ordered" assigns ids 0, 1, 2, ... in order.
    """
    rng = rng if rng is not None else np.random.Generator(np.random.PCG64(seed))
    lq = np.asarray(lq, dtype=np.int64)
    hist = np.asarray(hist, dtype=np.int64)
    S = lq.shape[0]
    assert prefix_len % block_size == 0, "a shared prefix covers whole blocks"
    n_prefix_blocks = prefix_len // block_size
    own = hist + lq
    own_blocks = -(-own // block_size)  # the prefix ends on a block boundary
    demand = int(n_prefix_blocks + own_blocks.sum())
    if num_blocks is None:
        num_blocks = max(1, int(math.ceil(pool_factor * demand)))
    if num_blocks < demand:
        raise ValueError(f"block pool of {num_blocks} cannot hold {demand} blocks")
    if id_mode == "choice":
        ids = rng.choice(num_blocks, size=demand, replace=False).astype(np.int32)
    elif id_mode == "perm":
        ids = rng.permutation(num_blocks)[:demand].astype(np.int32)
    elif id_mode == "ordered":
        ids = np.arange(demand, dtype=np.int32)
    else:
        raise ValueError(id_mode)
    shared = ids[:n_prefix_blocks] if n_prefix_blocks else None
    if max_blocks_per_seq is None:
        max_blocks_per_seq = max(1, int(n_prefix_blocks + (own_blocks.max() if S else 0)))
    bt = _tables_from_ids(own_blocks, ids[n_prefix_blocks:], max_blocks_per_seq, shared)
    if kind == "decode":
        assert ((lq == 1) | ((lq == 0) & (hist == 0))).all() and prefix_len == 0
        q_row0 = np.arange(S, dtype=np.int64)
    else:
        q_row0 = np.concatenate([[0], np.cumsum(lq)[:-1]]).astype(np.int64) if S else lq.copy()
    kv_row0 = prefix_len + (np.concatenate([[0], np.cumsum(own)[:-1]]).astype(np.int64)
                            if S else own.copy())
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(head_dim)))
    return Workload(name=name, kind=kind, seed=seed, num_q_heads=num_q_heads,
                    num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
                    num_blocks=num_blocks, max_blocks_per_seq=max_blocks_per_seq,
                    scale=float(np.float32(scale)), causal=causal, prefix_len=prefix_len,
                    hist=hist, lq=lq, q_row0=q_row0, kv_row0=kv_row0, block_tables=bt,
                    pad_tokens=pad_tokens)


def decode(context_lens, **kw) -> Workload:
    ctx = np.asarray(context_lens, dtype=np.int64)
    lq = (ctx > 0).astype(np.int64)
    return build("decode", lq, np.maximum(ctx - 1, 0), **kw)


def prefill(q_lens, hist=None, **kw) -> Workload:
    lq = np.asarray(q_lens, dtype=np.int64)
    h = np.zeros_like(lq) if hist is None else np.asarray(hist, dtype=np.int64)
    return build("prefill", lq, h, **kw)
