"""GPU parity past 4 GiB: tensors whose byte offsets cross 2^31 and 2^32.

The rows of these tensors repeat a short seeded table (inputs.periodic_table,
period 8191), so a wrapped 32-bit address would read a different row than the
right one.  The oracle cannot take tensors of this size whole; each sampled
block of query rows is checked against the oracle run on the keys those rows
can see.  A row's result depends only on its visible keys, so that smaller
problem, with the same causal alignment and window, has the same rows:

* prefill (N_q = N_k): rows [i0, i1) with a window of W keys see keys
  (i - W, i].  Passing keys [k0, i1), k0 <= i0 - W + 1, makes the sub-problem's
  bottom-right offset i0 - k0, which puts row i0 + t on key k0 + (t + i0 - k0) = i.
* windowed decode: the query sees the last W rows of its cache; a cache cut
  down to rows [len - W - 3, len) has the same last W rows.
* paged decode: the pool is read only through the block table; the pages the
  table names, renumbered, form the same sequences.
"""
import numpy as np
import pytest

import oracle
from tests.gpu_util import BF16_LSE_REL_TOL, BF16_O_TOL, compare, say, to_f64
from tests.large_util import decode_shift, decode_sub, paged_compact, prefill_sub
from transformer_attention_fa_amd import api, inputs

pytestmark = pytest.mark.gpu

D = 128
SEED = 51


@pytest.fixture(scope="module", autouse=True)
def _gpu(require_gpu):
    api.load()


@pytest.fixture(autouse=True)
def _free():
    yield
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _table(tag):
    import torch
    bits = inputs.periodic_table(SEED, tag, D)
    return bits, torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)


def _fill_rows(dst, table_dev, start, stop, shift):
    """dst [stop-start, D] (contiguous, on the device) = table rows of rows start..stop-1."""
    import torch
    idx = torch.from_numpy(inputs.periodic_rows(start, stop, shift)).cuda()
    torch.index_select(table_dev, 0, idx, out=dst)


def test_fwd_window_rows_past_4gib():
    import torch
    N = (1 << 24) + 3 * 64 + 17          # 256-byte rows: a head spans 2^32 + 53504 bytes
    H = 2
    W = 160
    scale = D ** -0.5
    shifts = {"q": [0, 4099], "k": [17, 2500], "v": [1234, 77]}
    say(f"fa_fwd_window past 4 GiB: B=1 H={H} H_kv={H} N={N} d={D} window={W}")
    tabs = {name: _table(tag) for tag, name in enumerate(("q", "k", "v"))}
    dev = {}
    for name in ("q", "k", "v"):
        t = torch.empty((1, H, N, D), dtype=torch.bfloat16, device="cuda")
        for h in range(H):
            _fill_rows(t[0, h], tabs[name][1], 0, N, shifts[name][h])
        dev[name] = t
    o, lse = api.fwd(dev["q"], dev["k"], dev["v"], causal=True, scale=scale, window=W)
    torch.cuda.synchronize()
    blocks = [(0, 300), ((1 << 23) - 150, (1 << 23) + 150), ((1 << 24) - 150, (1 << 24) + 150), (N - 300, N)]
    for h in range(H):
        for i0, i1 in blocks:
            q_sub, k_sub, v_sub = prefill_sub({n: tabs[n][0] for n in tabs}, shifts, h, i0, i1, W)
            o_ref, lse_ref = oracle.attention(q_sub, k_sub, v_sub, scale, True, window=W)
            compare(to_f64(o[0, h, i0:i1]), to_f64(lse[0, h, i0:i1]), o_ref[0, 0], lse_ref[0, 0],
                    BF16_O_TOL, BF16_LSE_REL_TOL, label=f"head {h} rows {i0}..{i1 - 1}")


def test_decode_window_cache_past_4gib():
    import torch
    B, H, H_kv = 2, 8, 2
    N_max = (1 << 23) + 77               # a (b, g) block spans 2^31 + 19712 bytes
    W = 2500
    splits = 3
    scale = D ** -0.5
    lens = np.array([N_max, N_max - 1000], dtype=np.int32)
    say(f"fa_decode_window past 4 GiB: B={B} H={H} H_kv={H_kv} N_max={N_max} lens={lens.tolist()} window={W}")
    tk, tv = _table(1), _table(2)
    q_bits = inputs.periodic_table(SEED, 3, D, period=B * H).reshape(B, H, D)
    sh = decode_shift
    caches = []
    for tag, (bits, tdev) in ((1, tk), (2, tv)):
        c = torch.empty((B, H_kv, N_max, D), dtype=torch.bfloat16, device="cuda")
        for b in range(B):
            for g in range(H_kv):
                _fill_rows(c[b, g], tdev, 0, N_max, sh(tag, b, g))
        caches.append(c)
    q = torch.from_numpy(q_bits.view(np.int16)).cuda().view(torch.bfloat16)
    o, lse = api.decode(q, caches[0], caches[1], torch.from_numpy(lens).cuda(), num_splits=splits,
                        scale=scale, window=W)
    torch.cuda.synchronize()
    for b in range(B):
        k_sub, v_sub, n = decode_sub(tk[0], tv[0], sh, b, int(lens[b]), W, H_kv)
        o_ref, lse_ref = oracle.decode(q_bits[b:b + 1], k_sub, v_sub, [n], scale, window=W)
        compare(to_f64(o[b:b + 1]), to_f64(lse[b:b + 1]), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL,
                label=f"sequence {b} (len {int(lens[b])})")


def test_decode_paged_pool_past_4gib():
    import torch
    B, H, H_kv, ps = 2, 8, 2, 64
    num_pages = (1 << 17) + 300          # 32 KB pages: page 2^17 starts at 4 GiB
    scale = D ** -0.5
    lens = np.array([5000, 3333], dtype=np.int32)
    table = inputs.scattered_page_table(lens, ps, num_pages, SEED)
    say(f"fa_decode_paged past 4 GiB: pool of {num_pages} pages of {ps} rows, lens={lens.tolist()}, "
        f"pages {int(table[table >= 0].min())}..{int(table.max())}")
    tk, tv = _table(1), _table(2)
    q_bits = inputs.periodic_table(SEED, 4, D, period=B * H).reshape(B, H, D)
    pools = []
    for (bits, tdev), shift in ((tk, 11), (tv, 5003)):
        p = torch.empty((num_pages, H_kv, ps, D), dtype=torch.bfloat16, device="cuda")
        for g in range(H_kv):
            tmp = torch.empty((num_pages * ps, D), dtype=torch.bfloat16, device="cuda")
            _fill_rows(tmp, tdev, 0, num_pages * ps, shift + 7 * g)
            p[:, g].copy_(tmp.view(num_pages, ps, D))
            del tmp
        pools.append(p)
    q = torch.from_numpy(q_bits.view(np.int16)).cuda().view(torch.bfloat16)
    o, lse = api.decode_paged(q, pools[0], pools[1], torch.from_numpy(table).cuda(),
                              torch.from_numpy(lens).cuda(), num_splits=5, scale=scale)
    torch.cuda.synchronize()
    hk, compact = paged_compact(table, tk[0], 11, H_kv, ps)
    hv, _ = paged_compact(table, tv[0], 5003, H_kv, ps)
    o_ref, lse_ref = oracle.decode_paged(q_bits, hk, hv, np.maximum(compact, 0), lens, scale)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL, label="paged pool past 4 GiB")
