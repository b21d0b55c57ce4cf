"""Plain fp64 CPU oracle for the paged KV-cache data plane.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports or calls this
module; only the tests, the smoke check and the benchmark's CPU-baseline leg do.
It shares no code with the HIP library.

What it computes, and where the pages define it:

* Block arithmetic -- a sequence is cut into fixed-size blocks (256 tokens by
  default); a 700-token sequence takes three blocks, the last holding 188
  tokens with 68 slots idle, and a long sequence spans several blocks
  ["Nano-vLLM part 1" (neutree.ai, translated on blog.itpub.net), section 4.1
  "From sequences to blocks"].
* Slot of a key position -- the cache is a flat array of token slots addressed
  through a per-token slot mapping ["Nano-vLLM inference engine architecture"
  (blog.hotdry.top), section on the lightweight PagedAttention implementation];
  the pages print no formula, so this follows the plainest reading of the two
  passages above: slot = block_table[j // block_size] * block_size
  + j % block_size.
* Store -- each new token's K and V rows are written at its slot-mapping offset
  in the preallocated cache (hotdry.top page, same section, on the
  store_kvcache kernel); a negative slot marks a padding entry and is skipped.
* Attention -- prefill attends all prompt tokens at once, decode attends one new
  token per sequence against everything cached before it ["Nano-vLLM part 1",
  section 2.4 "Prefill and decode", section 5.2 "Preparing the inputs"; hotdry.top
  page, "low-level optimisation details", on the varlen prefill and the
  cached-KV decode calls].  Paging is addressing only, so the result is plain
  scaled dot-product softmax attention over the gathered keys, written out
  here: s = scale * q.k, p = softmax(s), out = sum_j p_j v_j.  Query head h uses
  KV head h // (Hq / Hkv).  A causal prefill row r of a sequence with Lq queries
  and Lk keys sits at absolute position (Lk - Lq) + r and sees keys 0 .. that
  position.  A row that sees no key returns zeros.

Every bf16 input arrives as its uint16 bit pattern and is widened exactly to fp64.
"""
from __future__ import annotations

import numpy as np

BF16_NAN_CHECK = True


# ---- number formats ----------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---- block arithmetic ("Nano-vLLM part 1", section 4.1) -----------------------------
def blocks_for(num_tokens: int, block_size: int) -> int:
    """Blocks a sequence of ``num_tokens`` occupies."""
    return -(-int(num_tokens) // int(block_size))


def block_fill(num_tokens: int, block_size: int):
    """(blocks used, tokens in the last block, idle slots in the last block)."""
    n = blocks_for(num_tokens, block_size)
    last = num_tokens - (n - 1) * block_size if n else 0
    return n, last, (block_size - last) if n else 0


def logical_block(position, block_size):
    """(logical block index, offset inside it) of a key position."""
    position = np.asarray(position, dtype=np.int64)
    return position // block_size, position % block_size


def slot_of(block_table_row: np.ndarray, position, block_size: int) -> np.ndarray:
    """Physical cache slot of key position(s) of one sequence."""
    lb, off = logical_block(position, block_size)
    phys = np.asarray(block_table_row, dtype=np.int64)[lb]
    if np.any(phys < 0):
        raise IndexError("key position lies in an unallocated (-1) block")
    return phys * block_size + off


# ---- store (hotdry.top page, PagedAttention section) --------------------------------
def store_kvcache(k_cache, v_cache, k, v, slot_mapping):
    """Return copies of the cache images with each new token written at its slot.

    ``k_cache``/``v_cache``: uint16 ``[num_slots, Hkv, d]``; ``k``/``v``: uint16
    ``[N, Hkv, d]``; ``slot_mapping``: ``[N]``, negative entries skipped.  Raises on
    a slot beyond the cache and on two tokens sharing a slot (then more than one
    image would be a correct result).
    """
    kc = np.array(k_cache, dtype=np.uint16, copy=True)
    vc = np.array(v_cache, dtype=np.uint16, copy=True)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    live = slots[slots >= 0]
    if live.size and live.max() >= kc.shape[0]:
        raise IndexError("slot beyond the cache")
    if np.unique(live).size != live.size:
        raise ValueError("two tokens map to one slot")
    for i, s in enumerate(slots):
        if s < 0:
            continue
        kc[s] = k[i]
        vc[s] = v[i]
    return kc, vc


def check_store_targets(slot_mapping, block_tables, block_size: int) -> None:
    """Raise if a store targets a block that several tables reference.

    Blocks found by prefix hashing are shared through reference counts and are
    only read afterwards ("Nano-vLLM part 1", section 4.2; tokens of different
    sequences never share a writable block, section 4.1).
    """
    bt = np.asarray(block_tables)
    ids, counts = np.unique(bt[bt >= 0], return_counts=True)
    shared = ids[counts > 1]
    slots = np.asarray(slot_mapping, dtype=np.int64)
    written = np.unique(slots[slots >= 0] // block_size)
    bad = np.intersect1d(written, shared)
    if bad.size:
        raise ValueError(f"store into shared block(s) {bad[:4].tolist()}")


# ---- attention (plain definition) ---------------------------------------------------
def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """KV head that query head ``h`` reads (consecutive query heads share one)."""
    return h // (num_q_heads // num_kv_heads)


def visible_keys(row: int, offset: int, lk: int, causal: bool) -> int:
    """Number of keys query row ``row`` attends to (keys 0 .. that count - 1)."""
    if not causal:
        return lk
    return max(0, min(lk, offset + row + 1))


def softmax_weights(q: np.ndarray, k: np.ndarray, scale: float, causal: bool = False,
                    offset: int = 0) -> np.ndarray:
    """Attention weights ``[Hq, Lq, Lk]`` (fp64); masked keys get weight 0.

    ``q``: fp64 ``[Lq, Hq, d]``; ``k``: fp64 ``[Lk, Hkv, d]``.
    """
    lq, hq, _ = q.shape
    lk, hkv, _ = k.shape
    w = np.zeros((hq, lq, lk), dtype=np.float64)
    if lk == 0 or lq == 0:
        return w
    nvis = np.array([visible_keys(r, offset, lk, causal) for r in range(lq)], dtype=np.int64)
    mask = np.arange(lk)[None, :] < nvis[:, None]  # [Lq, Lk]
    for h in range(hq):
        g = kv_head_of(h, hq, hkv)
        s = (q[:, h, :] @ k[:, g, :].T) * float(scale)
        s = np.where(mask, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        m = np.where(np.isfinite(m), m, 0.0)
        e = np.where(mask, np.exp(s - m), 0.0)
        tot = e.sum(axis=1, keepdims=True)
        w[h] = np.divide(e, tot, out=np.zeros_like(e), where=tot > 0)
    return w


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal: bool = False,
              offset: int = 0) -> np.ndarray:
    """Scaled dot-product softmax attention, fp64: ``[Lq, Hq, d]``."""
    lq, hq, d = q.shape
    hkv = k.shape[1]
    w = softmax_weights(q, k, scale, causal, offset)
    out = np.zeros((lq, hq, v.shape[2]), dtype=np.float64)
    for h in range(hq):
        out[:, h, :] = w[h] @ v[:, kv_head_of(h, hq, hkv), :]
    return out


def _gather(cache_bits: np.ndarray, block_table_row, n: int, block_size: int) -> np.ndarray:
    if n == 0:
        return np.zeros((0,) + cache_bits.shape[1:], dtype=np.float64)
    slots = slot_of(block_table_row, np.arange(n), block_size)
    rows = bf16_to_f64(cache_bits[slots])
    if BF16_NAN_CHECK and np.isnan(rows).any():
        raise ValueError("gathered a poisoned (never written) cache slot")
    return rows


# ---- paged decode and paged varlen prefill -----------------------------------------
def paged_decode(q_bits, k_cache, v_cache, block_tables, context_lens, block_size: int,
                 scale: float) -> np.ndarray:
    """One query token per sequence against its cached keys: fp64 ``[B, Hq, d]``.

    ``context_lens[b]`` counts every cached position of sequence b, the token just
    stored included; a zero context returns a zero row.
    """
    q = bf16_to_f64(q_bits)
    B = q.shape[0]
    out = np.zeros(q.shape, dtype=np.float64)
    for b in range(B):
        n = int(context_lens[b])
        if n == 0:
            continue
        kb = _gather(k_cache, block_tables[b], n, block_size)
        vb = _gather(v_cache, block_tables[b], n, block_size)
        out[b] = attention(q[b:b + 1], kb, vb, scale)[0]
    return out


def paged_prefill(q_bits, k_cache, v_cache, cu_seqlens_q, cu_seqlens_k, block_tables,
                  block_size: int, scale: float, causal: bool = True, seqs=None) -> np.ndarray:
    """Variable-length prefill over packed queries: fp64 ``[total_q, Hq, d]``.

    Keys of sequence i are its positions 0 .. Lk_i - 1, read through its block
    table (a shared prefix is just the same block ids in several tables).  With
    ``seqs`` only those sequences' rows are computed (the rest stay zero).
    """
    q = bf16_to_f64(q_bits)
    out = np.zeros(q.shape, dtype=np.float64)
    n_seq = len(cu_seqlens_q) - 1
    for i in (range(n_seq) if seqs is None else seqs):
        q0, q1 = int(cu_seqlens_q[i]), int(cu_seqlens_q[i + 1])
        lk = int(cu_seqlens_k[i + 1]) - int(cu_seqlens_k[i])
        lq = q1 - q0
        if lq == 0:
            continue
        if causal and lk < lq:
            raise ValueError("causal prefill needs at least as many keys as queries")
        kb = _gather(k_cache, block_tables[i], lk, block_size)
        vb = _gather(v_cache, block_tables[i], lk, block_size)
        out[q0:q1] = attention(q[q0:q1], kb, vb, scale, causal, lk - lq)
    return out
