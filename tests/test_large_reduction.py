"""CPU checks of the reductions the parity tests past 4 GiB rely on.

Those tests cannot hand the oracle their whole tensors, so each sampled block of
rows is computed by the oracle on a smaller problem (tests/large_util.py).
Here, at a size the oracle runs whole, each smaller problem must give the same
rows as the whole problem, and the repeated-table inputs must tell a wrapped
32-bit address apart from the right one.
"""
import numpy as np

import oracle
from tests.large_util import decode_shift, decode_sub, host_rows, paged_compact, pool_rows, prefill_sub
from transformer_attention_fa_amd import inputs

D = 128
SEED = 52


def _tables(tags):
    return {name: inputs.periodic_table(SEED, tag, D) for name, tag in tags.items()}


def test_periodic_rows_tell_wrapped_addresses_apart():
    t = inputs.periodic_table(SEED, 0, D)
    assert t.shape == (inputs.LARGE_PERIOD, D) and t.dtype == np.uint16
    assert np.unique(t, axis=0).shape[0] == inputs.LARGE_PERIOD          # no two table rows alike
    rows = np.array([0, 1, 12345, (1 << 23) - 1, 1 << 23, (1 << 24) + 77], dtype=np.int64)
    for shift in (0, 17, 5003):
        right = inputs.periodic_rows(0, 1 << 25, shift)[rows]
        # a 256-byte-row address wrapped at 2^31, 2^32 or 2^33 bytes is off by 2^23, 2^24 or 2^25 rows
        for k in (23, 24, 25):
            wrapped = (rows + (1 << k) + shift) % inputs.LARGE_PERIOD
            assert np.all(wrapped != right)


def test_prefill_sub_problem_gives_the_whole_problems_rows():
    N, H, W = 700, 2, 160
    scale = D ** -0.5
    tabs = _tables({"q": 0, "k": 1, "v": 2})
    shifts = {"q": [0, 4099], "k": [17, 2500], "v": [1234, 77]}
    whole = {n: np.stack([host_rows(tabs[n], 0, N, shifts[n][h]) for h in range(H)])[None] for n in tabs}
    o, lse = oracle.attention(whole["q"], whole["k"], whole["v"], scale, True, window=W)
    for h in range(H):
        for i0, i1 in ((0, 100), (150, 170), (300, 420), (600, 700)):
            q, k, v = prefill_sub(tabs, shifts, h, i0, i1, W)
            o_s, lse_s = oracle.attention(q, k, v, scale, True, window=W)
            np.testing.assert_allclose(o_s[0, 0], o[0, h, i0:i1], rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse_s[0, 0], lse[0, h, i0:i1], rtol=0, atol=1e-12)


def test_decode_window_sub_cache_gives_the_whole_caches_result():
    B, H, H_kv, N_max, W = 2, 4, 2, 900, 250
    scale = D ** -0.5
    tk, tv = inputs.periodic_table(SEED, 1, D), inputs.periodic_table(SEED, 2, D)
    q = inputs.periodic_table(SEED, 3, D, period=B * H).reshape(B, H, D)
    lens = np.array([N_max, 700], dtype=np.int32)
    kc = np.stack([np.stack([host_rows(tk, 0, N_max, decode_shift(1, b, g)) for g in range(H_kv)])
                   for b in range(B)])
    vc = np.stack([np.stack([host_rows(tv, 0, N_max, decode_shift(2, b, g)) for g in range(H_kv)])
                   for b in range(B)])
    o, lse = oracle.decode(q, kc, vc, lens, scale, window=W)
    for b in range(B):
        k, v, n = decode_sub(tk, tv, decode_shift, b, int(lens[b]), W, H_kv)
        o_s, lse_s = oracle.decode(q[b:b + 1], k, v, [n], scale, window=W)
        np.testing.assert_allclose(o_s[0], o[b], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse_s[0], lse[b], rtol=0, atol=1e-12)


def test_compact_page_pool_gives_the_whole_pools_result():
    B, H, H_kv, ps, num_pages = 2, 4, 2, 16, 40
    scale = D ** -0.5
    tk, tv = inputs.periodic_table(SEED, 1, D), inputs.periodic_table(SEED, 2, D)
    q = inputs.periodic_table(SEED, 4, D, period=B * H).reshape(B, H, D)
    lens = np.array([100, 70], dtype=np.int32)
    table = inputs.scattered_page_table(lens, ps, num_pages, SEED)
    assert np.unique(table[table >= 0]).size == np.count_nonzero(table >= 0)   # distinct pages
    pools = [np.stack([np.stack([pool_rows(bits, p, g, ps, shift) for g in range(H_kv)]) for p in range(num_pages)])
             for bits, shift in ((tk, 11), (tv, 5003))]
    o, lse = oracle.decode_paged(q, pools[0], pools[1], np.maximum(table, 0), lens, scale)
    hk, compact = paged_compact(table, tk, 11, H_kv, ps)
    hv, _ = paged_compact(table, tv, 5003, H_kv, ps)
    assert hk.shape[0] == np.count_nonzero(table >= 0)
    o_s, lse_s = oracle.decode_paged(q, hk, hv, np.maximum(compact, 0), lens, scale)
    np.testing.assert_allclose(o_s, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_s, lse, rtol=0, atol=1e-12)


def test_scattered_page_table_reaches_the_large_pools_far_pages():
    lens = np.array([5000, 3333], dtype=np.int32)
    num_pages = (1 << 17) + 300
    table = inputs.scattered_page_table(lens, 64, num_pages, 51)
    used = table[table >= 0]
    assert used.size == 79 + 53 and np.unique(used).size == used.size
    assert used.max() < num_pages and used.min() >= 0
    assert np.any(used >= 1 << 17)                               # past 4 GiB (32 KB pages)
    assert np.any((used >= (1 << 16) - 64) & (used < (1 << 16) + 64))   # around 2 GiB
    assert np.all(table[1, 53:] == -1)
