"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every comparison covers the whole output, element by element: small problems
that span several query and key tiles and end in ragged tails, and the
full-size workloads in the launch configuration the benchmark times.
"""
import os

import numpy as np
import pytest

import oracle
from tests.gpu_util import (BF16_LSE_REL_TOL, BF16_O_TOL, F32_TOL, bf16_to_device, compare, f32_to_device,
                            fwd_capped, say, to_f64)
from transformer_attention_fa_amd import api, inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(require_gpu):
    api.load()


def _spec(B, H, H_kv, N_q, N_k, d, causal, dtype="bf16", seed=7, k_scale=1.0):
    name = f"B{B}_H{H}_Hkv{H_kv}_Nq{N_q}_Nk{N_k}_d{d}_{'causal' if causal else 'full'}_{dtype}"
    return inputs.Prefill(name, B, H, H_kv, N_q, N_k, d, causal, dtype, seed, k_scale)


def _run_fwd(data):
    s = data.spec
    if s.dtype == "bf16":
        q, k, v = (bf16_to_device(x) for x in (data.q, data.k, data.v))
        o, lse = api.fwd(q, k, v, causal=s.causal, scale=s.scale)
    else:
        q, k, v = (f32_to_device(x) for x in (data.q, data.k, data.v))
        o, lse = api.fwd_f32(q, k, v, causal=s.causal, scale=s.scale)
    import torch
    torch.cuda.synchronize()
    return o, lse


SMALL_BF16 = [
    (1, 2, 2, 300, 300, 128, False),
    (1, 2, 2, 300, 300, 128, True),
    (2, 8, 2, 200, 333, 128, True),      # GQA, N_q < N_k: bottom-right causal
    (2, 8, 2, 200, 333, 128, False),
    (1, 4, 1, 129, 64, 64, False),       # MQA, d = 64
    (1, 4, 1, 129, 64, 64, True),        # N_q > N_k: leading rows see no key
    (1, 3, 3, 1, 1, 128, False),
    (1, 3, 1, 1, 17, 128, True),
    (2, 4, 4, 517, 517, 64, True),
    (1, 2, 1, 1000, 1000, 128, True),
]


@pytest.mark.parametrize("shape", SMALL_BF16, ids=lambda s: "x".join(map(str, s)))
def test_fwd_bf16_small_full_compare(shape):
    spec = _spec(*shape)
    say(f"fa_fwd bf16 {spec.name}")
    data = inputs.prefill_inputs(spec)
    o, lse = _run_fwd(data)
    o_ref, lse_ref = oracle.attention(data.q, data.k, data.v, spec.scale, spec.causal)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL, label=spec.name)


def test_fwd_bf16_sharp_softmax():
    """K scaled by 4: scores ~ N(0, 16); rows are nearly one-hot."""
    spec = _spec(1, 4, 2, 256, 256, 128, True, k_scale=4.0)
    data = inputs.prefill_inputs(spec)
    o, lse = _run_fwd(data)
    o_ref, lse_ref = oracle.attention(data.q, data.k, data.v, spec.scale, spec.causal)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL, label="sharp")


SMALL_F32 = [
    inputs.SINGLE_HEAD_F32,
    inputs.SINGLE_HEAD_F32_CAUSAL,
    _spec(2, 4, 2, 77, 190, 128, True, dtype="f32"),
    _spec(2, 4, 2, 190, 77, 128, True, dtype="f32"),
    _spec(1, 6, 3, 100, 300, 64, False, dtype="f32"),
]


@pytest.mark.parametrize("spec", SMALL_F32, ids=lambda s: s.name)
def test_fwd_f32_full_compare(spec):
    say(f"fa_fwd_f32 {spec.name}")
    data = inputs.prefill_inputs(spec)
    o, lse = _run_fwd(data)
    o_ref, lse_ref = oracle.attention(data.q, data.k, data.v, spec.scale, spec.causal)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, F32_TOL, F32_TOL, lse_relative=False, label=spec.name)


def _whole_compare(spec, o, lse, data):
    """Every O and LSE element of a full-size run against the oracle's whole
    tensors (the tiled method reaches the very same numbers as the plain
    definition: "Attention variants" §3)."""
    say(f"  oracle on the whole {spec.name} ({spec.B * spec.H * spec.N_q} rows)")
    o_ref, lse_ref = oracle.attention(data.q, data.k, data.v, spec.scale, spec.causal, window=spec.window or None)
    return compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL,
                   label=f"{spec.name} (whole)")


@pytest.mark.parametrize("spec", [inputs.MHA_PREFILL, inputs.GQA_PREFILL, inputs.MQA_PREFILL], ids=lambda s: s.name)
def test_fwd_bf16_workloads_whole(spec):
    """The full-size prefill workloads, in the launch configuration the
    benchmark times, compared element by element over the whole output."""
    import torch
    say(f"fa_fwd bf16 full-size workload {spec.name}")
    data = inputs.prefill_inputs(spec)
    q, k, v = (bf16_to_device(x) for x in (data.q, data.k, data.v))
    o, lse = api.fwd(q, k, v, causal=spec.causal, scale=spec.scale)
    torch.cuda.synchronize()
    del q, k, v
    _whole_compare(spec, o, lse, data)


def test_fwd_zero_query_closed_form():
    """Q = 0: every visible key has equal weight, o_i = mean(V[0..i]) (causal), lse_i = ln(i+1)."""
    import torch
    spec = _spec(1, 2, 1, 300, 300, 128, True)
    data = inputs.prefill_inputs(spec)
    q = torch.zeros((1, 2, 300, 128), dtype=torch.bfloat16, device="cuda")
    k, v = bf16_to_device(data.k), bf16_to_device(data.v)
    o, lse = api.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    vv = inputs.bf16_bits_to_f32(data.v).astype(np.float64)[0, 0]
    mean = np.cumsum(vv, axis=0) / np.arange(1, 301)[:, None]
    ref_o = np.broadcast_to(mean, (2, 300, 128))
    ref_lse = np.broadcast_to(np.log(np.arange(1, 301)), (2, 300))
    compare(to_f64(o)[0], to_f64(lse)[0], ref_o, ref_lse, BF16_O_TOL, BF16_LSE_REL_TOL, label="Q=0")


def test_fwd_deterministic_and_no_out_of_bounds_writes():
    import torch
    spec = _spec(2, 4, 2, 333, 333, 128, True)
    data = inputs.prefill_inputs(spec)
    q, k, v = (bf16_to_device(x) for x in (data.q, data.k, data.v))
    n_o, n_l, G = q.numel(), 2 * 4 * 333, 4096
    o_buf = torch.full((n_o + 2 * G,), 7.0, dtype=torch.bfloat16, device="cuda")
    l_buf = torch.full((n_l + 2 * G,), 7.0, dtype=torch.float32, device="cuda")
    o = o_buf[G:G + n_o].view(q.shape)
    lse = l_buf[G:G + n_l].view(2, 4, 333)
    api.fwd(q, k, v, causal=True, out=o, lse=lse)
    first_o, first_l = o.clone(), lse.clone()
    api.fwd(q, k, v, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(o, first_o) and torch.equal(lse, first_l)
    assert bool((o_buf[:G] == 7.0).all()) and bool((o_buf[G + n_o:] == 7.0).all())
    assert bool((l_buf[:G] == 7.0).all()) and bool((l_buf[G + n_l:] == 7.0).all())


def test_fwd_without_lse():
    import torch
    spec = _spec(1, 2, 2, 128, 128, 128, False)
    data = inputs.prefill_inputs(spec)
    q, k, v = (bf16_to_device(x) for x in (data.q, data.k, data.v))
    o1, _ = api.fwd(q, k, v)
    o2, l2 = api.fwd(q, k, v, lse=False)
    torch.cuda.synchronize()
    assert l2 is None and torch.equal(o1, o2)


# ------------------------------------------------------------------ decode
def _decode_run(data, num_splits):
    import torch
    s = data.spec
    q = bf16_to_device(data.q)
    kc, vc = bf16_to_device(data.k_cache), bf16_to_device(data.v_cache)
    lens = torch.from_numpy(data.seq_lens).cuda()
    o, lse = api.decode(q, kc, vc, lens, num_splits=num_splits, scale=s.scale)
    torch.cuda.synchronize()
    return o, lse


def test_decode_workload_full_compare():
    spec = inputs.GQA_DECODE
    say(f"fa_decode full-size workload {spec.name}")
    data = inputs.decode_inputs(spec)           # padding rows hold NaN
    o, lse = _decode_run(data, spec.num_splits)
    o_ref, lse_ref = oracle.decode(data.q, data.k_cache, data.v_cache, data.seq_lens, spec.scale)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL, label=spec.name)


def _small_decode_spec(H=8, H_kv=2, d=128, N_max=3000, B=6, seed=11):
    return inputs.Decode(f"decode_B{B}_H{H}_Hkv{H_kv}_d{d}", B, H, H_kv, d, 1, N_max, N_max, 16, seed)


@pytest.mark.parametrize("num_splits", [1, 4, 16, 64, 256])
def test_decode_split_counts_and_edge_lengths(num_splits):
    spec = _small_decode_spec()
    lens = np.array([1, 2, 15, 16, 17, 3000], np.int32)      # shorter than the split count, and N_max
    data = inputs.decode_inputs(spec, seq_lens=lens)          # rows past each length hold NaN
    o, lse = _decode_run(data, num_splits)
    o_ref, lse_ref = oracle.decode(data.q, data.k_cache, data.v_cache, lens, spec.scale)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL, label=f"S={num_splits}")


@pytest.mark.parametrize("H,H_kv,d", [(16, 1, 64), (12, 4, 128), (8, 8, 128), (64, 8, 128),
                                      (40, 2, 128), (48, 1, 64), (64, 2, 128)])
def test_decode_head_sharing(H, H_kv, d):
    spec = _small_decode_spec(H=H, H_kv=H_kv, d=d, N_max=1200, B=3, seed=13)
    data = inputs.decode_inputs(spec)
    o, lse = _decode_run(data, 8)
    o_ref, lse_ref = oracle.decode(data.q, data.k_cache, data.v_cache, data.seq_lens, spec.scale)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL, label=spec.name)


def test_decode_lengths_outside_the_cache_are_clamped():
    """A length <= 0 gives the empty result (o = 0, lse = -inf); one past N_max
    attends to the whole cache and reads nothing beyond it."""
    import torch
    spec = _small_decode_spec(H=8, H_kv=2, d=128, N_max=700, B=6, seed=19)
    dev_lens = np.array([0, 5, 700 + 333, -3, 1, 700], np.int32)
    host_lens = np.array([1, 5, 700, 1, 1, 700], np.int32)   # clamped; rows 0 and 3 are replaced below
    data = inputs.decode_inputs(spec, seq_lens=host_lens)
    q = bf16_to_device(data.q)
    kc, vc = bf16_to_device(data.k_cache), bf16_to_device(data.v_cache)
    o, lse = api.decode(q, kc, vc, torch.from_numpy(dev_lens).cuda(), num_splits=8, scale=spec.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode(data.q, data.k_cache, data.v_cache, host_lens, spec.scale)
    for b in (0, 3):
        o_ref[b] = 0.0
        lse_ref[b] = -np.inf
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL, label="clamped lengths")


def test_decode_deterministic():
    import torch
    spec = _small_decode_spec(seed=17)
    data = inputs.decode_inputs(spec)
    o1, l1 = _decode_run(data, 16)
    o2, l2 = _decode_run(data, 16)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ------------------------------------------------------------------ persistent prefill grid
# A cap on the workgroups makes every workgroup of the persistent d=128 kernel
# run many items in a row (item switches, the next item's Q and first K tile
# loaded during the current one, slot parity carried across items), at sizes
# the oracle checks element by element.
PERSIST_CASES = [
    # B, H, H_kv, N_q, N_k, d, causal, window
    (2, 8, 2, 600, 600, 128, True, None),      # 48 items; per-XCD list at caps >= 8
    (1, 3, 1, 700, 700, 128, False, None),     # 9 items; whole-list rounds
    (1, 8, 2, 900, 900, 128, True, 70),        # window: first tile parity changes between items
    (1, 8, 1, 900, 300, 128, True, None),      # N_q > N_k: items whose rows see no key
    (2, 4, 4, 300, 1000, 128, True, None),     # N_q < N_k
    (1, 4, 2, 517, 517, 64, True, None),       # d = 64 runs one item per workgroup: cap has no effect
]


@pytest.mark.parametrize("cap", [1, 3, 8, 13])
@pytest.mark.parametrize("case", PERSIST_CASES, ids=lambda c: "x".join(str(x) for x in c))
def test_fwd_persistent_rounds(case, cap):
    import torch
    B, H, H_kv, N_q, N_k, d, causal, window = case
    spec = _spec(B, H, H_kv, N_q, N_k, d, causal, seed=31)
    say(f"fa_fwd persistent cap={cap} {spec.name} window={window}")
    data = inputs.prefill_inputs(spec)
    q, k, v = (bf16_to_device(x) for x in (data.q, data.k, data.v))
    o, lse = fwd_capped(q, k, v, causal, spec.scale, cap, window)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(data.q, data.k, data.v, spec.scale, causal, window=window)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL, label=f"cap {cap}")
    # the same launch without a cap gives the same bits
    o2, lse2 = api.fwd(q, k, v, causal=causal, scale=spec.scale, window=window)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


# ------------------------------------------------------------------ random sweep
def _random_cases(n, seed=2024):
    """Seeded shapes that mix what the fixed cases test one at a time: lengths on
    and around tile (64 keys) and wave (32 rows) boundaries, N_q != N_k, head
    sharing, both head sizes, causal or not, sliding windows, and caps on the
    persistent grid (several items per workgroup)."""
    rng = np.random.default_rng(seed)
    edges = [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 383, 511, 513]
    cases = []
    for _ in range(n):
        n_q = int(rng.choice(edges)) if rng.random() < 0.6 else int(rng.integers(1, 600))
        n_k = int(rng.choice(edges)) if rng.random() < 0.6 else int(rng.integers(1, 600))
        h_kv = int(rng.choice([1, 2, 4]))
        rep = int(rng.choice([1, 2, 3, 4]))
        b = int(rng.integers(1, 4))
        d = int(rng.choice([64, 128]))
        causal = bool(rng.random() < 0.65)
        window = int(rng.integers(1, n_k + 64)) if causal and rng.random() < 0.4 else None
        cap = int(rng.choice([0, 0, 1, 3, 8]))
        cases.append((b, h_kv * rep, h_kv, n_q, n_k, d, causal, window, cap))
    return cases


RANDOM_CASES = _random_cases(24)


@pytest.mark.parametrize("case", RANDOM_CASES, ids=lambda c: "x".join(str(x) for x in c))
def test_fwd_random_shapes(case):
    import torch
    B, H, H_kv, N_q, N_k, d, causal, window, cap = case
    spec = _spec(B, H, H_kv, N_q, N_k, d, causal, seed=41)
    say(f"fa_fwd random {spec.name} window={window} cap={cap}")
    data = inputs.prefill_inputs(spec)
    q, k, v = (bf16_to_device(x) for x in (data.q, data.k, data.v))
    if cap:
        o, lse = fwd_capped(q, k, v, causal, spec.scale, cap, window)
    else:
        o, lse = api.fwd(q, k, v, causal=causal, scale=spec.scale, window=window)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(data.q, data.k, data.v, spec.scale, causal, window=window)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL, label=spec.name)


# Causal launches with an even GQA ratio at d = 128 pair two heads per item
# (128 rows each): several blocks per head pair, ragged last blocks, windows
# that cross blocks, N_q below and above N_k, and capped grids that force
# several rounds of items per workgroup.
PAIRED_CASES = [(2, 8, 4, 300, 300, None, 0), (1, 8, 2, 700, 900, None, 3), (2, 4, 1, 513, 513, 100, 5),
                (1, 6, 3, 1000, 600, None, 2), (3, 4, 2, 129, 2000, 300, 0), (1, 16, 4, 1024, 1024, 200, 8)]


@pytest.mark.parametrize("case", PAIRED_CASES, ids=lambda c: "x".join(str(x) for x in c))
def test_fwd_paired_items(case):
    import torch
    B, H, H_kv, N_q, N_k, window, cap = case
    spec = _spec(B, H, H_kv, N_q, N_k, 128, True, seed=43)
    say(f"fa_fwd paired items {spec.name} window={window} cap={cap}")
    data = inputs.prefill_inputs(spec)
    q, k, v = (bf16_to_device(x) for x in (data.q, data.k, data.v))
    if cap:
        o, lse = fwd_capped(q, k, v, True, spec.scale, cap, window)
    else:
        o, lse = api.fwd(q, k, v, causal=True, scale=spec.scale, window=window)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(data.q, data.k, data.v, spec.scale, True, window=window)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL, label=spec.name)


def _random_f32_cases(n, seed=2027):
    """Seeded fp32 shapes: lengths on and around its 32-key tiles and its
    query blocks, N_q != N_k (both ways), head sharing, both head sizes,
    causal or not."""
    rng = np.random.default_rng(seed)
    edges = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 257]
    cases = []
    for _ in range(n):
        n_q = int(rng.choice(edges)) if rng.random() < 0.6 else int(rng.integers(1, 400))
        n_k = int(rng.choice(edges)) if rng.random() < 0.6 else int(rng.integers(1, 400))
        h_kv = int(rng.choice([1, 2, 3]))
        rep = int(rng.choice([1, 2, 4]))
        cases.append((int(rng.integers(1, 3)), h_kv * rep, h_kv, n_q, n_k, int(rng.choice([64, 128])),
                      bool(rng.random() < 0.6)))
    return cases


@pytest.mark.parametrize("case", _random_f32_cases(12), ids=lambda c: "x".join(str(x) for x in c))
def test_fwd_f32_random_shapes(case):
    spec = _spec(*case, dtype="f32", seed=43)
    say(f"fa_fwd_f32 random {spec.name}")
    data = inputs.prefill_inputs(spec)
    o, lse = _run_fwd(data)
    o_ref, lse_ref = oracle.attention(data.q, data.k, data.v, spec.scale, spec.causal)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, F32_TOL, F32_TOL, lse_relative=False, label=spec.name)


# ------------------------------------------------------------------ sliding window
WINDOW_BF16 = [
    # B, H, H_kv, N_q, N_k, d, window
    (1, 4, 2, 300, 300, 128, 64),
    (1, 4, 2, 300, 300, 128, 1),
    (1, 2, 2, 333, 333, 128, 65),        # window edge inside a tile, ragged tail
    (2, 2, 1, 517, 517, 64, 100),
    (1, 2, 2, 200, 700, 128, 150),       # N_q < N_k: the window ends at i + 500
    (1, 2, 1, 700, 300, 128, 50),        # N_q > N_k: leading rows see no key
    (1, 4, 4, 1024, 1024, 128, 256),     # tile-aligned window
    (1, 2, 1, 1000, 1000, 128, 700),
]


@pytest.mark.parametrize("shape", WINDOW_BF16, ids=lambda s: "x".join(map(str, s)))
def test_fwd_window_full_compare(shape):
    import torch
    B, H, H_kv, N_q, N_k, d, w = shape
    spec = _spec(B, H, H_kv, N_q, N_k, d, True, seed=23)
    say(f"fa_fwd_window {spec.name} window={w}")
    data = inputs.prefill_inputs(spec)
    q, k, v = (bf16_to_device(x) for x in (data.q, data.k, data.v))
    o, lse = api.fwd(q, k, v, causal=True, scale=spec.scale, window=w)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(data.q, data.k, data.v, spec.scale, True, window=w)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL, label=f"window {w}")


def test_fwd_window_covering_the_keys_equals_causal():
    import torch
    spec = _spec(2, 4, 2, 600, 600, 128, True, seed=29)
    data = inputs.prefill_inputs(spec)
    q, k, v = (bf16_to_device(x) for x in (data.q, data.k, data.v))
    o_c, l_c = api.fwd(q, k, v, causal=True, scale=spec.scale)
    o_w, l_w = api.fwd(q, k, v, causal=True, scale=spec.scale, window=600)
    torch.cuda.synchronize()
    assert torch.equal(o_c, o_w) and torch.equal(l_c, l_w)


@pytest.mark.parametrize("window", [1, 15, 16, 17, 300, 5000])
@pytest.mark.parametrize("num_splits", [1, 5, 16])
def test_decode_window(window, num_splits):
    import torch
    spec = _small_decode_spec(H=8, H_kv=2, d=128, N_max=3000, B=6, seed=31)
    lens = np.array([1, 2, 16, 17, 1200, 3000], np.int32)
    data = inputs.decode_inputs(spec, seq_lens=lens)
    # rows before each window are never read: poison them
    k_c, v_c = data.k_cache.copy(), data.v_cache.copy()
    for b, n in enumerate(lens):
        k_c[b, :, :max(0, n - window)] = inputs.BF16_QNAN
        v_c[b, :, :max(0, n - window)] = inputs.BF16_QNAN
    q = bf16_to_device(data.q)
    kc, vc = bf16_to_device(k_c), bf16_to_device(v_c)
    o, lse = api.decode(q, kc, vc, torch.from_numpy(lens).cuda(), num_splits=num_splits, scale=spec.scale,
                        window=window)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode(data.q, data.k_cache, data.v_cache, lens, spec.scale, window=window)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL,
            label=f"window {window} S={num_splits}")


def _random_decode_cases(n, seed=2025):
    """Seeded decode shapes: one or several head groups per KV head (up to 16
    query heads per group), both head sizes, cache lengths from 1 to N_max
    (padding rows poisoned), split counts that do and do not divide them, and
    sliding windows."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        b = int(rng.integers(1, 9))
        h_kv = int(rng.choice([1, 2, 4, 8]))
        rep = int(rng.choice([1, 2, 3, 4, 8, 16, 20]))
        d = int(rng.choice([64, 128]))
        n_max = int(rng.choice([1, 17, 300, 2000]))
        lens = rng.integers(1, n_max + 1, size=b)
        lens[rng.random(b) < 0.25] = n_max
        lens[rng.random(b) < 0.15] = 1
        splits = int(rng.choice([1, 3, 16, 37]))
        window = int(rng.integers(1, n_max + 20)) if rng.random() < 0.35 else None
        cases.append((b, h_kv * rep, h_kv, d, n_max, tuple(int(x) for x in lens), splits, window))
    return cases


RANDOM_DECODE_CASES = _random_decode_cases(16)


@pytest.mark.parametrize("case", RANDOM_DECODE_CASES,
                         ids=lambda c: f"B{c[0]}_H{c[1]}_Hkv{c[2]}_d{c[3]}_N{c[4]}_S{c[6]}_w{c[7]}")
def test_decode_random_shapes(case):
    import torch
    B, H, H_kv, d, N_max, lens, S, window = case
    spec = inputs.Decode(f"decode_B{B}_H{H}_Hkv{H_kv}_d{d}_N{N_max}", B, H, H_kv, d, 1, N_max, N_max, S, 43)
    lens = np.array(lens, np.int32)
    say(f"fa_decode random {spec.name} lens={lens.tolist()} splits={S} window={window}")
    data = inputs.decode_inputs(spec, seq_lens=lens)          # rows past each length hold NaN
    q = bf16_to_device(data.q)
    kc, vc = bf16_to_device(data.k_cache), bf16_to_device(data.v_cache)
    o, lse = api.decode(q, kc, vc, torch.from_numpy(lens).cuda(), num_splits=S, scale=spec.scale, window=window)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode(data.q, data.k_cache, data.v_cache, lens, spec.scale, window=window)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL, label=spec.name)


@pytest.mark.parametrize("spec", [inputs.SWA_PREFILL, inputs.CHUNKED_PREFILL], ids=lambda s: s.name)
def test_fwd_next_workloads_whole(spec):
    import torch
    say(f"fa_fwd full-size workload {spec.name}")
    data = inputs.prefill_inputs(spec)
    q, k, v = (bf16_to_device(x) for x in (data.q, data.k, data.v))
    o, lse = api.fwd(q, k, v, causal=spec.causal, scale=spec.scale, window=spec.window or None)
    torch.cuda.synchronize()
    del q, k, v
    _whole_compare(spec, o, lse, data)


def test_decode_window_workload_full_compare():
    spec = inputs.SWA_DECODE
    say(f"fa_decode_window full-size workload {spec.name}")
    data = inputs.decode_inputs(spec)
    import torch
    q = bf16_to_device(data.q)
    kc, vc = bf16_to_device(data.k_cache), bf16_to_device(data.v_cache)
    o, lse = api.decode(q, kc, vc, torch.from_numpy(data.seq_lens).cuda(), num_splits=spec.num_splits,
                        scale=spec.scale, window=spec.window)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode(data.q, data.k_cache, data.v_cache, data.seq_lens, spec.scale,
                                   window=spec.window)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL, label=spec.name)


# ------------------------------------------------------------------ paged KV cache
def _paged(data, page_size, seed):
    table, num_pages = inputs.page_table(data.seq_lens, page_size, seed)
    kp = inputs.to_pages(data.k_cache, data.seq_lens, table, num_pages, page_size, inputs.BF16_QNAN)
    vp = inputs.to_pages(data.v_cache, data.seq_lens, table, num_pages, page_size, inputs.BF16_QNAN)
    return kp, vp, table


@pytest.mark.parametrize("page_size", [16, 32, 64, 256])
@pytest.mark.parametrize("num_splits", [1, 7, 16])
def test_decode_paged(page_size, num_splits):
    import torch
    spec = _small_decode_spec(H=8, H_kv=2, d=128, N_max=3000, B=6, seed=37)
    lens = np.array([1, 2, 15, 16, 17, 3000], np.int32)
    data = inputs.decode_inputs(spec, seq_lens=lens)
    kp, vp, table = _paged(data, page_size, 41)
    q = bf16_to_device(data.q)
    o, lse = api.decode_paged(q, bf16_to_device(kp), bf16_to_device(vp), torch.from_numpy(table).cuda(),
                              torch.from_numpy(lens).cuda(), num_splits=num_splits, scale=spec.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_paged(data.q, kp, vp, np.maximum(table, 0), lens, spec.scale)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL,
            label=f"page {page_size} S={num_splits}")


@pytest.mark.parametrize("d,page_size,num_splits", [(128, 16, 1), (128, 64, 2), (64, 32, 1)])
def test_decode_paged_long_chunks(d, page_size, num_splits):
    """Chunks of more than 64 tiles per wave (over 4096 keys): the kernel holds
    the first 64 block-table entries of each wave in its lanes and reads the
    later ones one by one."""
    import torch
    spec = _small_decode_spec(H=4, H_kv=1, d=d, N_max=9000, B=3, seed=53)
    lens = np.array([4097, 9000, 6000], np.int32)
    data = inputs.decode_inputs(spec, seq_lens=lens)
    kp, vp, table = _paged(data, page_size, 59)
    o, lse = api.decode_paged(bf16_to_device(data.q), bf16_to_device(kp), bf16_to_device(vp),
                              torch.from_numpy(table).cuda(), torch.from_numpy(lens).cuda(), num_splits=num_splits,
                              scale=spec.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode(data.q, data.k_cache, data.v_cache, lens, spec.scale)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL,
            label=f"paged long d{d} p{page_size} S={num_splits}")


def test_decode_paged_d64_mqa():
    import torch
    spec = _small_decode_spec(H=16, H_kv=1, d=64, N_max=900, B=3, seed=43)
    data = inputs.decode_inputs(spec)
    kp, vp, table = _paged(data, 32, 47)
    o, lse = api.decode_paged(bf16_to_device(data.q), bf16_to_device(kp), bf16_to_device(vp),
                              torch.from_numpy(table).cuda(), torch.from_numpy(data.seq_lens).cuda(), num_splits=8,
                              scale=spec.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode(data.q, data.k_cache, data.v_cache, data.seq_lens, spec.scale)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL, label="paged d64")


def test_decode_paged_clamps_bad_table_entries():
    """Entries past the used blocks are never read; a bad entry of a used block
    is clamped into the pool (so the result is that of the clamped table)."""
    import torch
    spec = _small_decode_spec(H=8, H_kv=2, d=128, N_max=500, B=3, seed=53)
    lens = np.array([100, 260, 500], np.int32)
    data = inputs.decode_inputs(spec, seq_lens=lens)
    kp, vp, table = _paged(data, 64, 59)
    bad = table.copy()
    bad[0, 2:] = 1 << 30                  # blocks past 100 rows: never read
    bad[1, 5] = -7                        # 260 rows use blocks 0..4: block 5 is never read
    bad[2, 3] = 1 << 30                   # used: clamped to the last page
    o, lse = api.decode_paged(bf16_to_device(data.q), bf16_to_device(kp), bf16_to_device(vp),
                              torch.from_numpy(bad).cuda(), torch.from_numpy(lens).cuda(), num_splits=4,
                              scale=spec.scale)
    torch.cuda.synchronize()
    clamped = np.clip(bad, 0, kp.shape[0] - 1)
    o_ref, lse_ref = oracle.decode_paged(data.q, kp, vp, clamped, lens, spec.scale)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL, label="clamped table")


def test_decode_paged_workload_full_compare():
    import torch
    spec = inputs.PAGED_DECODE
    say(f"fa_decode_paged full-size workload {spec.name}")
    data = inputs.decode_inputs(spec)
    kp, vp, table = _paged(data, spec.page_size, spec.seed)
    o, lse = api.decode_paged(bf16_to_device(data.q), bf16_to_device(kp), bf16_to_device(vp),
                              torch.from_numpy(table).cuda(), torch.from_numpy(data.seq_lens).cuda(),
                              num_splits=spec.num_splits, scale=spec.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode(data.q, data.k_cache, data.v_cache, data.seq_lens, spec.scale)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL, label=spec.name)


# ------------------------------------------------------------------ FP8 KV cache
def _fp8_run(data, num_splits, k_scale, v_scale):
    import torch
    s = data.spec
    q = bf16_to_device(data.q)
    kc = torch.from_numpy(data.k_cache).cuda()
    vc = torch.from_numpy(data.v_cache).cuda()
    o, lse = api.decode_fp8(q, kc, vc, k_scale, v_scale, torch.from_numpy(data.seq_lens).cuda(),
                            num_splits=num_splits, scale=s.scale)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("H,H_kv,d", [(8, 2, 128), (16, 1, 64), (12, 4, 128), (40, 2, 128)])
@pytest.mark.parametrize("num_splits", [1, 7, 16])
def test_decode_fp8(H, H_kv, d, num_splits):
    spec = inputs.Decode(f"fp8_B6_H{H}_Hkv{H_kv}_d{d}", 6, H, H_kv, d, 1, 3000, 3000, num_splits, 61,
                         dtype="e4m3", k_scale=2.0 ** -6, v_scale=2.0 ** -5)
    lens = np.array([1, 2, 15, 16, 17, 3000], np.int32)
    data = inputs.decode_inputs_fp8(spec, seq_lens=lens)
    o, lse = _fp8_run(data, num_splits, spec.k_scale, spec.v_scale)
    o_ref, lse_ref = oracle.decode_fp8(data.q, data.k_cache, data.v_cache, spec.k_scale, spec.v_scale, lens,
                                       spec.scale)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL, label=spec.name)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("num_splits", [1, 3, 5])
def test_decode_fp8_tile_boundaries(d, num_splits):
    """The FP8 cache streams 32-key tiles, each two 16-key score blocks: lengths
    and chunk ends on and around 16, 32, 48 and 64 keys (a tile whose second
    block is empty, partly filled or whole), one query head per KV head and a
    full group of 16."""
    lens = np.array([1, 15, 16, 17, 31, 32, 33, 47, 48, 49, 63, 64, 65, 97, 160, 161], np.int32)
    for H, H_kv in ((4, 4), (32, 2)):
        spec = inputs.Decode(f"fp8_tiles_H{H}_Hkv{H_kv}_d{d}", len(lens), H, H_kv, d, 1, 200, 200, num_splits, 67,
                             dtype="e4m3", k_scale=0.013, v_scale=2.0 ** -4)
        say(f"fa_decode_fp8 tile boundaries {spec.name} S={num_splits}")
        data = inputs.decode_inputs_fp8(spec, seq_lens=lens)
        o, lse = _fp8_run(data, num_splits, spec.k_scale, spec.v_scale)
        o_ref, lse_ref = oracle.decode_fp8(data.q, data.k_cache, data.v_cache, spec.k_scale, spec.v_scale, lens,
                                           spec.scale)
        compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL, label=spec.name)


def _random_cache_cases(n, seed=2026):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        b = int(rng.integers(1, 7))
        h_kv = int(rng.choice([1, 2, 4]))
        rep = int(rng.choice([1, 3, 4, 16, 18]))
        d = int(rng.choice([64, 128]))
        n_max = int(rng.choice([16, 100, 1500]))
        lens = rng.integers(1, n_max + 1, size=b)
        lens[rng.random(b) < 0.25] = n_max
        splits = int(rng.choice([1, 5, 16]))
        page = int(rng.choice([16, 32, 48, 128]))
        cases.append((b, h_kv * rep, h_kv, d, n_max, tuple(int(x) for x in lens), splits, page))
    return cases


RANDOM_CACHE_CASES = _random_cache_cases(10)


@pytest.mark.parametrize("case", RANDOM_CACHE_CASES,
                         ids=lambda c: f"B{c[0]}_H{c[1]}_Hkv{c[2]}_d{c[3]}_N{c[4]}_S{c[6]}_p{c[7]}")
def test_decode_paged_and_fp8_random_shapes(case):
    """Seeded shapes for the paged cache (page sizes that are multiples of 16,
    pages in shuffled order) and the FP8 cache (scales that are powers of two and
    not), each against its oracle."""
    import torch
    B, H, H_kv, d, N_max, lens, S, page = case
    lens = np.array(lens, np.int32)
    spec = inputs.Decode(f"rnd_B{B}_H{H}_Hkv{H_kv}_d{d}_N{N_max}", B, H, H_kv, d, 1, N_max, N_max, S, 47)
    data = inputs.decode_inputs(spec, seq_lens=lens)
    kp, vp, table = _paged(data, page, 53)
    say(f"fa_decode_paged random {spec.name} lens={lens.tolist()} S={S} page={page}")
    o, lse = api.decode_paged(bf16_to_device(data.q), bf16_to_device(kp), bf16_to_device(vp),
                              torch.from_numpy(table).cuda(), torch.from_numpy(lens).cuda(), num_splits=S,
                              scale=spec.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_paged(data.q, kp, vp, np.maximum(table, 0), lens, spec.scale)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL, label=f"paged {spec.name}")

    k_scale, v_scale = (2.0 ** -6, 0.0173) if B % 2 else (0.011, 2.0 ** -5)
    fspec = inputs.Decode(f"rnd8_B{B}_H{H}_Hkv{H_kv}_d{d}_N{N_max}", B, H, H_kv, d, 1, N_max, N_max, S, 59,
                          dtype="e4m3", k_scale=k_scale, v_scale=v_scale)
    fdata = inputs.decode_inputs_fp8(fspec, seq_lens=lens)
    say(f"fa_decode_fp8 random {fspec.name} k_scale={k_scale} v_scale={v_scale}")
    o, lse = _fp8_run(fdata, S, k_scale, v_scale)
    o_ref, lse_ref = oracle.decode_fp8(fdata.q, fdata.k_cache, fdata.v_cache, k_scale, v_scale, lens, fspec.scale)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL, label=f"fp8 {fspec.name}")


def test_decode_fp8_every_code():
    """Random codes over the whole finite range (subnormals, zeros of both signs,
    +-448) with scales that are not powers of two."""
    import torch
    B, H, H_kv, N, d = 2, 8, 2, 700, 128
    rng = np.random.default_rng(67)
    kc = rng.integers(0, 256, (B, H_kv, N, d)).astype(np.uint8)
    vc = rng.integers(0, 256, (B, H_kv, N, d)).astype(np.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x00       # the NaN codes become zeros
    vc[(vc & 0x7F) == 0x7F] = 0x80
    q = inputs.f32_to_bf16_bits(rng.standard_normal((B, H, d), dtype=np.float32) * np.float32(0.05))
    lens = np.array([333, 700], np.int32)
    k_scale, v_scale = 0.0123, 0.37
    spec = inputs.Decode("fp8_codes", B, H, H_kv, d, 1, N, N, 8, 0, dtype="e4m3")
    data = inputs.DecodeData(spec, q, kc, vc, lens)
    o, lse = _fp8_run(data, 8, k_scale, v_scale)
    o_ref, lse_ref = oracle.decode_fp8(q, kc, vc, k_scale, v_scale, lens, spec.scale)
    # values up to 448 * 0.37: the O tolerance scales with the value range (bf16 output rounding)
    tol = BF16_O_TOL * float(np.max(np.abs(o_ref)))
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, max(tol, BF16_O_TOL), BF16_LSE_REL_TOL, label="every code")


def test_decode_fp8_workload_full_compare():
    spec = inputs.FP8_DECODE
    say(f"fa_decode_fp8 full-size workload {spec.name}")
    data = inputs.decode_inputs_fp8(spec)
    o, lse = _fp8_run(data, spec.num_splits, spec.k_scale, spec.v_scale)
    o_ref, lse_ref = oracle.decode_fp8(data.q, data.k_cache, data.v_cache, spec.k_scale, spec.v_scale,
                                       data.seq_lens, spec.scale)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL, label=spec.name)


def test_fwd_clock_record_hook():
    """The test hook's clock-recording instantiation gives fa_fwd's bits, and
    its records are plausible: XCC ids 0-7, end after start, and a shader
    clock between 0.3 and 3 GHz."""
    import ctypes
    import torch
    spec = _spec(2, 8, 2, 1000, 1000, 128, True, seed=97)
    data = inputs.prefill_inputs(spec)
    q, k, v = (bf16_to_device(x) for x in (data.q, data.k, data.v))
    o_ref, l_ref = api.fwd(q, k, v, causal=True, scale=spec.scale)
    lib = api.load()
    fn = lib.fa_testing_fwd_capped
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    fn.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, i, vp, vp]
    fn.restype = i
    stamps = torch.zeros(64, dtype=torch.int64, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty_like(l_ref)
    api.check(fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), 2, 8, 2, 1000, 1000, 128,
                 float(spec.scale), 1, 0, 0, stamps.data_ptr(), torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)) and torch.equal(lse, l_ref)
    rec = stamps.cpu().numpy().reshape(8, 8)
    assert ((rec[:, 2] >= 0) & (rec[:, 2] < 8)).all()
    say(f"  XCC ids of workgroups 0-7: {rec[:, 2].tolist()}")
    cyc, ticks = rec[:, 3] - rec[:, 0], rec[:, 4] - rec[:, 1]
    assert (ticks > 0).all() and (cyc > 0).all()
    ghz = cyc / ticks * 0.1
    say(f"  clock record: {np.round(ghz, 3).tolist()} GHz")
    assert ((ghz > 0.3) & (ghz < 3.0)).all()


# ------------------------------------------------------------------ scale = 0
@pytest.mark.parametrize("causal,window,d", [(True, None, 128), (False, None, 128), (True, 50, 128), (True, None, 64)])
def test_fwd_scale_zero(causal, window, d):
    """scale = 0: every visible key has weight 1 / #visible, so o is the mean of
    the visible V rows and lse = ln(#visible); checked against the oracle and
    the closed form."""
    import torch
    spec = _spec(1, 4, 2, 300, 300, d, causal, seed=71)
    say(f"fa_fwd scale 0 causal={causal} window={window} d={d}")
    data = inputs.prefill_inputs(spec)
    q, k, v = (bf16_to_device(x) for x in (data.q, data.k, data.v))
    o, lse = api.fwd(q, k, v, causal=causal, scale=0.0, window=window)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(data.q, data.k, data.v, 0.0, causal, window=window)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL, label="scale 0")
    i = np.arange(300)
    first = np.maximum(0, i - window + 1) if window else np.zeros_like(i)
    n_vis = (i + 1 - first) if causal else np.full_like(i, 300)
    assert np.allclose(lse_ref[0, 0], np.log(n_vis), atol=1e-12)
    vv = inputs.bf16_bits_to_f32(data.v).astype(np.float64)[0, 0]
    mean = np.array([vv[first[r]:first[r] + n_vis[r]].mean(axis=0) for r in range(300)])
    assert np.allclose(o_ref[0, 0], mean, atol=1e-12)


@pytest.mark.parametrize("num_splits", [1, 5, 16])
def test_decode_scale_zero(num_splits):
    spec = _small_decode_spec(seed=73)
    lens = np.array([1, 2, 15, 16, 17, 3000], np.int32)
    data = inputs.decode_inputs(spec, seq_lens=lens)
    import torch
    q = bf16_to_device(data.q)
    kc, vc = bf16_to_device(data.k_cache), bf16_to_device(data.v_cache)
    o, lse = api.decode(q, kc, vc, torch.from_numpy(lens).cuda(), num_splits=num_splits, scale=0.0)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode(data.q, data.k_cache, data.v_cache, lens, 0.0)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL, label=f"decode scale 0 S={num_splits}")
    assert np.allclose(lse_ref, np.log(lens.astype(np.float64))[:, None], atol=1e-12)


# ------------------------------------------------------------------ decode outputs
def test_decode_rejects_wrong_output_shapes():
    """Caller-supplied o and lse must have shapes [B,H,d] and [B,H]: the kernels
    write that many values, so a smaller buffer is refused before any launch."""
    import torch
    spec = _small_decode_spec(B=3, N_max=200, seed=79)
    data = inputs.decode_inputs(spec)
    q = bf16_to_device(data.q)
    kc, vc = bf16_to_device(data.k_cache), bf16_to_device(data.v_cache)
    lens = torch.from_numpy(data.seq_lens).cuda()
    B, H, d = q.shape
    bad_o = [torch.empty((B, H - 1, d), dtype=torch.bfloat16, device="cuda"),
             torch.empty((B, H, d // 2), dtype=torch.bfloat16, device="cuda")]
    bad_l = [torch.empty((B, H - 1), dtype=torch.float32, device="cuda"),
             torch.empty((B - 1, H), dtype=torch.float32, device="cuda")]
    for o in bad_o:
        with pytest.raises(ValueError, match="out must have shape"):
            api.decode(q, kc, vc, lens, num_splits=4, out=o)
        with pytest.raises(ValueError, match="out must have shape"):
            api.decode(q, kc, vc, lens, num_splits=4, out=o, window=50)
    for lse in bad_l:
        with pytest.raises(ValueError, match="lse must have shape"):
            api.decode(q, kc, vc, lens, num_splits=4, lse=lse)
    codes = torch.zeros(kc.shape, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="out must have shape"):
        api.decode_fp8(q, codes, codes, 1.0, 1.0, lens, num_splits=4, out=bad_o[0])
    with pytest.raises(ValueError, match="lse must have shape"):
        api.decode_fp8(q, codes, codes, 1.0, 1.0, lens, num_splits=4, lse=bad_l[0])
    table = torch.zeros((B, 13), dtype=torch.int32, device="cuda")
    pool = torch.zeros((8, spec.H_kv, 16, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="out must have shape"):
        api.decode_paged(q, pool, pool, table, lens, num_splits=4, out=bad_o[1])
    with pytest.raises(ValueError, match="lse must have shape"):
        api.decode_paged(q, pool, pool, table, lens, num_splits=4, lse=bad_l[1])
    torch.cuda.synchronize()


@pytest.mark.parametrize("num_splits", [1, 16])
def test_decode_deterministic_and_no_out_of_bounds_writes(num_splits):
    """Decode writes exactly o [B,H,d] and lse [B,H]: guard bands on both sides
    keep their fill, and a second call gives the same bits."""
    import torch
    spec = _small_decode_spec(B=5, H=12, H_kv=4, N_max=900, seed=83)
    data = inputs.decode_inputs(spec)
    q = bf16_to_device(data.q)
    kc, vc = bf16_to_device(data.k_cache), bf16_to_device(data.v_cache)
    lens = torch.from_numpy(data.seq_lens).cuda()
    n_o, n_l, G = q.numel(), 5 * 12, 4096
    o_buf = torch.full((n_o + 2 * G,), 7.0, dtype=torch.bfloat16, device="cuda")
    l_buf = torch.full((n_l + 2 * G,), 7.0, dtype=torch.float32, device="cuda")
    o = o_buf[G:G + n_o].view(q.shape)
    lse = l_buf[G:G + n_l].view(5, 12)
    api.decode(q, kc, vc, lens, num_splits=num_splits, out=o, lse=lse)
    first_o, first_l = o.clone(), lse.clone()
    api.decode(q, kc, vc, lens, num_splits=num_splits, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(o, first_o) and torch.equal(lse, first_l)
    assert bool((o_buf[:G] == 7.0).all()) and bool((o_buf[G + n_o:] == 7.0).all())
    assert bool((l_buf[:G] == 7.0).all()) and bool((l_buf[G + n_l:] == 7.0).all())
    o_ref, lse_ref = oracle.decode(data.q, data.k_cache, data.v_cache, data.seq_lens, spec.scale)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL, label=f"guarded S={num_splits}")


# ------------------------------------------------------------------ decode chunk queue
# 32 sequences x 8 KV heads x 16 splits = 4096 chunks: more than the
# workgroups that fit on the device at once, so the split kernel's resident
# workgroups take chunks from the counter in the workspace.
def _queue_spec(seed):
    return inputs.Decode("decode_queue_B32_H16_Hkv8", 32, 16, 8, 128, 1, 640, 640, 16, seed)


def _queue_run(spec, dev_lens, host_lens, ws, out=None, lse=None):
    """Decode with device lengths dev_lens (0 = empty sequence) on caches drawn
    for host_lens (1 where dev_lens is 0); returns the result and the oracle's."""
    import torch
    data = inputs.decode_inputs(spec, seq_lens=host_lens)
    q = bf16_to_device(data.q)
    kc, vc = bf16_to_device(data.k_cache), bf16_to_device(data.v_cache)
    o, l = api.decode(q, kc, vc, torch.from_numpy(dev_lens).cuda(), num_splits=spec.num_splits, scale=spec.scale,
                      workspace=ws, out=out, lse=lse)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode(data.q, data.k_cache, data.v_cache, host_lens, spec.scale)
    for b in np.nonzero(dev_lens == 0)[0]:
        o_ref[b] = 0.0
        lse_ref[b] = -np.inf
    return o, l, o_ref, lse_ref


# the queue word's tag (high half) as the library leaves it
QUEUE_TAG = 0x46416451


def test_decode_chunk_queue_garbage_and_reused_workspace():
    """With the chunk queue in use, workspaces whose queue word the library did
    not leave give the oracle's result: all bytes 0xff, the tag minus one with
    an all-ones count (the first claim carries into the tag) and another tag
    with a small count.  Each is followed by a second call on the same
    workspace with other lengths: empty sequences, single keys and chunk edges
    (chunks of 0, 1, 2 and 3 keys, 16-key tile edges)."""
    import torch
    spec = _queue_spec(89)
    rng = np.random.default_rng(89)
    lens_a = rng.integers(1, spec.N_max + 1, spec.B).astype(np.int32)
    lens_b = lens_a.copy()
    lens_b[:12] = [0, 0, 1, 2, 15, 16, 17, 33, 48, 257, 639, 640]
    rng.shuffle(lens_b)
    nbytes = api.decode_workspace_bytes(spec.B, spec.H, spec.d, spec.num_splits)
    words = (("0xff bytes", None), ("tag - 1, count 2^32 - 1", ((QUEUE_TAG - 1) << 32) | 0xFFFFFFFF),
             ("other tag, count 5", (0x12345678 << 32) | 5))
    for name, word in words:
        ws = torch.full((nbytes,), 255, dtype=torch.uint8, device="cuda")
        if word is not None:
            ws[:8].view(torch.int64).fill_(word - (1 << 64) if word >= 1 << 63 else word)
        for label, dev_lens in ((f"{name}: first call", lens_a), (f"{name}: reused", lens_b)):
            say(f"decode chunk queue, {label}")
            o, lse, o_ref, lse_ref = _queue_run(spec, dev_lens, np.maximum(dev_lens, 1), ws)
            compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL, label=label)
        # the merge left the queue idle: the tag and a zero count
        torch.cuda.synchronize()
        assert int(ws[:8].view(torch.int64).item()) == QUEUE_TAG << 32


def test_decode_chunk_queue_graph_replays_match_eager():
    """A decode step whose split kernel takes chunks from the queue (with the
    kernel that zeroes the counter ahead of it), captured in a HIP graph,
    replays to the eager result bit for bit, with eager calls on the same
    workspace between the replays."""
    import torch
    spec = _queue_spec(97)
    data = inputs.decode_inputs(spec)
    q = bf16_to_device(data.q)
    kc, vc = bf16_to_device(data.k_cache), bf16_to_device(data.v_cache)
    lens = torch.from_numpy(data.seq_lens).cuda()
    ws = torch.empty(api.decode_workspace_bytes(spec.B, spec.H, spec.d, spec.num_splits), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")

    def step():
        api.decode(q, kc, vc, lens, num_splits=spec.num_splits, scale=spec.scale, out=o, lse=lse, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = (o.clone(), lse.clone())
    o_ref, lse_ref = oracle.decode(data.q, data.k_cache, data.v_cache, data.seq_lens, spec.scale)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL, label="eager decode")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), ref[0].view(torch.int16)), rep
        assert torch.equal(lse.view(torch.int32), ref[1].view(torch.int32)), rep
        api.decode(q, kc, vc, lens, num_splits=spec.num_splits, scale=spec.scale, workspace=ws)
        torch.cuda.synchronize()


# Each kernel variant with more chunks than the device holds at once (512
# workgroups at d = 128, 768 at d = 64 on 256 CUs), so the queue runs in all of
# them: more than 64 sequences (index order, lengths read per chunk), d = 64,
# a sliding window, the FP8 and the paged cache.
QUEUE_CASES = [
    # name, B, H, H_kv, d, N_max, splits, kind
    ("bf16_B80", 80, 8, 2, 128, 300, 8, "bf16"),
    ("bf16_d64", 16, 16, 4, 64, 500, 16, "bf16"),
    ("window_d128", 16, 8, 4, 128, 600, 16, "window"),
    ("fp8_d64", 16, 16, 4, 64, 600, 16, "fp8"),
    ("fp8_B70", 70, 4, 2, 128, 256, 4, "fp8"),
    ("paged_d64", 16, 16, 4, 64, 512, 16, "paged"),
]


@pytest.mark.parametrize("case", QUEUE_CASES, ids=lambda c: c[0])
def test_decode_chunk_queue_kernel_variants(case):
    import torch
    name, B, H, H_kv, d, N_max, S, kind = case
    assert B * H_kv * S > (512 if d == 128 else 768)
    rng = np.random.default_rng(B * 1000 + d)
    lens = rng.integers(1, N_max + 1, B).astype(np.int32)
    lens[:3] = [1, 17, N_max]
    say(f"decode chunk queue variant {name}")
    if kind == "fp8":
        k_scale, v_scale = 0.011, 2.0 ** -5
        fspec = inputs.Decode(f"queue_{name}", B, H, H_kv, d, 1, N_max, N_max, S, 97, dtype="e4m3",
                              k_scale=k_scale, v_scale=v_scale)
        fdata = inputs.decode_inputs_fp8(fspec, seq_lens=lens)
        o, lse = _fp8_run(fdata, S, k_scale, v_scale)
        o_ref, lse_ref = oracle.decode_fp8(fdata.q, fdata.k_cache, fdata.v_cache, k_scale, v_scale, lens,
                                           fspec.scale)
    else:
        spec = inputs.Decode(f"queue_{name}", B, H, H_kv, d, 1, N_max, N_max, S, 97)
        data = inputs.decode_inputs(spec, seq_lens=lens)
        dl = torch.from_numpy(lens).cuda()
        if kind == "paged":
            kp, vp, table = _paged(data, 16, 101)
            o, lse = api.decode_paged(bf16_to_device(data.q), bf16_to_device(kp), bf16_to_device(vp),
                                      torch.from_numpy(table).cuda(), dl, num_splits=S, scale=spec.scale)
            o_ref, lse_ref = oracle.decode_paged(data.q, kp, vp, np.maximum(table, 0), lens, spec.scale)
        else:
            window = 200 if kind == "window" else None
            o, lse = api.decode(bf16_to_device(data.q), bf16_to_device(data.k_cache), bf16_to_device(data.v_cache),
                                dl, num_splits=S, scale=spec.scale, window=window)
            o_ref, lse_ref = oracle.decode(data.q, data.k_cache, data.v_cache, lens, spec.scale, window=window)
    torch.cuda.synchronize()
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL, label=name)


# ------------------------------------------------------------------ HIP graph capture
def test_hip_graph_capture_replays_match_eager():
    """A prefill call and a decode step captured in one HIP graph (through
    torch.cuda.graph, on the capture stream the binding passes down) replay
    to the eager results bit for bit, replay after replay, with other eager
    work between the replays.  The library allocates, clears and syncs
    nothing on the call path, so nothing else needs to be captured."""
    import torch
    pspec = _spec(1, 4, 2, 300, 300, 128, True, seed=41)
    pd = inputs.prefill_inputs(pspec)
    q, k, v = (bf16_to_device(x) for x in (pd.q, pd.k, pd.v))
    dspec = inputs.Decode("graph_decode", 2, 8, 2, 128, 1, 700, 700, 4, 43)
    dd = inputs.decode_inputs(dspec)
    dq, kc, vc = (bf16_to_device(x) for x in (dd.q, dd.k_cache, dd.v_cache))
    lens = torch.from_numpy(dd.seq_lens).to("cuda")
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")
    do = torch.empty_like(dq)
    dl = torch.empty(dq.shape[:-1], dtype=torch.float32, device="cuda")
    ws = torch.empty(api.decode_workspace_bytes(2, 8, 128, 4), dtype=torch.uint8, device="cuda")

    def step():
        api.fwd(q, k, v, causal=True, scale=pspec.scale, out=o, lse=lse)
        api.decode(dq, kc, vc, lens, num_splits=4, scale=dspec.scale, out=do, lse=dl, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, lse, do, dl)]
    o_ref, lse_ref = oracle.attention(pd.q, pd.k, pd.v, pspec.scale, True)
    compare(to_f64(o), to_f64(lse), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL, label="eager prefill")

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    other = torch.randn(1, 4, 300, 128, device="cuda").to(torch.bfloat16)
    for rep in range(4):
        for t in (o, lse, do, dl):
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((o, lse, do, dl), ref):
            assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got.view(torch.int32),
                               want.view(torch.int16) if want.dtype == torch.bfloat16 else want.view(torch.int32)), rep
        # eager work between replays, on other buffers
        api.fwd(other, k, v, causal=True, scale=pspec.scale)
        torch.cuda.synchronize()


def test_concurrent_streams_match_sequential():
    """A persistent prefill launch and a decode step in flight together on two
    streams (plus a second prefill on a third) give the same bits as when run
    one at a time: the kernels keep no state between or across launches."""
    import torch
    torch.manual_seed(47)
    q = torch.randn(2, 8, 1500, 128, device="cuda").to(torch.bfloat16)
    k = torch.randn(2, 2, 1500, 128, device="cuda").to(torch.bfloat16)
    v = torch.randn(2, 2, 1500, 128, device="cuda").to(torch.bfloat16)
    q2 = torch.randn(1, 4, 900, 64, device="cuda").to(torch.bfloat16)
    k2 = torch.randn(1, 4, 900, 64, device="cuda").to(torch.bfloat16)
    v2 = torch.randn(1, 4, 900, 64, device="cuda").to(torch.bfloat16)
    dspec = inputs.Decode("streams_decode", 4, 16, 4, 128, 1, 3000, 9000, 8, 53)
    dd = inputs.decode_inputs(dspec)
    dq, kc, vc = (bf16_to_device(x) for x in (dd.q, dd.k_cache, dd.v_cache))
    lens = torch.from_numpy(dd.seq_lens).to("cuda")
    o_a, l_a = api.fwd(q, k, v, causal=True)
    o_b, l_b = api.fwd(q2, k2, v2, causal=False)
    do_a, dl_a = api.decode(dq, kc, vc, lens, num_splits=8)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(3)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        with torch.cuda.stream(streams[0]):
            o1, l1 = api.fwd(q, k, v, causal=True)
        with torch.cuda.stream(streams[1]):
            do1, dl1 = api.decode(dq, kc, vc, lens, num_splits=8)
        with torch.cuda.stream(streams[2]):
            o2, l2 = api.fwd(q2, k2, v2, causal=False)
        torch.cuda.synchronize()
        assert torch.equal(o1, o_a) and torch.equal(l1, l_a)
        assert torch.equal(o2, o_b) and torch.equal(l2, l_b)
        assert torch.equal(do1, do_a) and torch.equal(dl1, dl_a)


# ------------------------------------------------------------------ race hunting
DEBUG_BARRIER_CASES = [
    # B, H, H_kv, N_q, N_k, d, causal, window, cap
    (2, 8, 2, 600, 600, 128, True, None, 3),
    (1, 8, 1, 900, 900, 128, False, None, 5),
    (1, 8, 2, 900, 900, 128, True, 70, 8),
    (1, 8, 1, 900, 300, 128, True, None, 2),
    (2, 4, 4, 300, 1000, 128, True, None, 0),
    (1, 4, 2, 517, 517, 64, True, None, 0),
]


@pytest.mark.parametrize("case", DEBUG_BARRIER_CASES, ids=lambda c: "x".join(str(x) for x in c))
def test_fwd_debug_barrier_build_is_bit_identical(case):
    """libfa_debug_barriers.so puts a full wait and a barrier between the two
    phases of every period; the arithmetic is the same, so any difference from
    libfa.so would come from a race between waves."""
    import torch
    from transformer_attention_fa_amd import build
    B, H, H_kv, N_q, N_k, d, causal, window, cap = case
    if not os.path.exists(build.DEBUG_LIB):
        pytest.fail(f"{build.DEBUG_LIB} is not built (python -m transformer_attention_fa_amd.build --debug-barriers)")
    dbg = api.open_library(build.DEBUG_LIB)
    spec = _spec(B, H, H_kv, N_q, N_k, d, causal, seed=53)
    say(f"debug-barrier build vs libfa.so: {spec.name} window={window} cap={cap}")
    data = inputs.prefill_inputs(spec)
    q, k, v = (bf16_to_device(x) for x in (data.q, data.k, data.v))
    o, lse = fwd_capped(q, k, v, causal, spec.scale, cap, window)
    o2, lse2 = fwd_capped(q, k, v, causal, spec.scale, cap, window, lib=dbg)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
