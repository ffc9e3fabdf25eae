"""Host-side helpers of the parity tests past 4 GiB: the rows of their tensors
(a short seeded table repeated by position, inputs.periodic_table) and the
smaller problems the oracle runs for sampled rows.  test_large_reduction.py
checks on the CPU that each smaller problem gives the rows of the whole one."""
import numpy as np

from transformer_attention_fa_amd import inputs


def host_rows(table_bits, start, stop, shift):
    return table_bits[inputs.periodic_rows(start, stop, shift)]


def prefill_sub(tables, shifts, h, i0, i1, window):
    """q [1,1,i1-i0,d] and k, v [1,1,i1-k0,d] for query rows [i0, i1) of head h
    of a causal problem with N_q = N_k; k0 = max(0, i0 - window)."""
    k0 = max(0, i0 - window)
    q = host_rows(tables["q"], i0, i1, shifts["q"][h])[None, None]
    k = host_rows(tables["k"], k0, i1, shifts["k"][h])[None, None]
    v = host_rows(tables["v"], k0, i1, shifts["v"][h])[None, None]
    return q, k, v


def decode_sub(tk, tv, shift, b, length, window, H_kv):
    """k, v caches [1,H_kv,window+3,d]: rows [length-window-3, length) of sequence b."""
    lo = length - window - 3
    k = np.stack([host_rows(tk, lo, length, shift(1, b, g)) for g in range(H_kv)])[None]
    v = np.stack([host_rows(tv, lo, length, shift(2, b, g)) for g in range(H_kv)])[None]
    return k, v, length - lo


def pool_rows(bits, page, g, ps, shift):
    """Rows of page `page`, KV head g, of a pool whose flat row r (page*ps + s) is table row r + shift + 7g."""
    return host_rows(bits, page * ps, page * ps + ps, shift + 7 * g)


def paged_compact(table, bits, shift, H_kv, ps):
    """The pages the table names, renumbered in ascending order, and the table over them."""
    used = np.unique(table[table >= 0])
    compact = np.where(table >= 0, np.searchsorted(used, table), -1).astype(np.int32)
    hp = np.empty((used.size, H_kv, ps, bits.shape[1]), dtype=np.uint16)
    for j, page in enumerate(used):
        for g in range(H_kv):
            hp[j, g] = pool_rows(bits, int(page), g, ps, shift)
    return hp, compact


def decode_shift(tag, b, g):
    return 97 * tag + 1000 * b + 31 * g
