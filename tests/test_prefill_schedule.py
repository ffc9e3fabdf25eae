"""The prefill kernel's item schedule, modelled on the CPU (no GPU needed).

A Python model of the item loop of csrc/fwd_bf16.hip -- the persistent grid's
item order, each wave's periods (idle, first, general/steady, last) between
switch periods, the slot parity of the K/V tiles, the tile loads of waves 0-3
and the next item's Q slices -- run over the benchmark shapes and random ones.
It checks what the kernel relies on and a GPU run would only show as a hang or
a wrong result: every wave of a workgroup passes the same number of barriers;
every tile a wave owns gets S, then its softmax, then PV, in the periods its
role fixes; every LDS slot a period reads holds the tile it should, and no
period loads into a slot it reads; the entered item's Q block is complete in
the Q area when the switch period reads it, and no Q slice loads in a switch
period; every item's rows are written once by every wave, and every 32-row
group of every head's output by exactly one wave (causal launches with an even
GQA ratio pair two heads per item: half the rows, waves 0-3 on the first head
and waves 4-7 on the second).  The model follows the kernel's code and must be
kept in step with it.
"""
import random

import pytest

_FLIP = False  # plants a slot-parity mistake (test of the checker itself)
_SAME_HEAD = False  # plants a paired-item mistake: waves 4-7 on the first head too

BM, BN, NW = 256, 64, 8

def cdiv(a, b): return -(-a // b)
def tdiv(a, b):  # C++ truncating division
    q = abs(a) // abs(b)
    return q if (a >= 0) == (b > 0) else -q

def run(B, H, Hkv, Nq, Nk, causal, window, cap, persist=True, group=4, resident=256, max_groups=None):
    rep = H // Hkv
    pair = persist and causal and rep % 2 == 0
    BMI = BM // 2 if pair else BM
    hpb = H // 2 if pair else H
    nqb = cdiv(Nq, BMI)
    items = nqb * hpb * B
    if items == 0: return
    grid = items; xcd = 0
    if persist:
        grid = min(grid, resident)
        if cap > 0: grid = min(grid, cap)
        if ((hpb * B) & 7) == 0 and grid >= 8:
            grid = grid // 8 * 8; xcd = 1
    off = Nk - Nq
    win = window if causal else 0
    QPARTS = 8
    def decompose(i):
        HB = hpb * B; head0, nheads, slot = 0, HB, i
        if (HB & 7) == 0:
            nheads = HB >> 3; head0 = (i & 7) * nheads; slot = i >> 3
        gsz = min(max(1, group // 2) if pair else group, nheads)
        grp = slot // (gsz * nqb); rem = slot - grp * gsz * nqb
        g0 = grp * gsz; gcount = min(gsz, nheads - g0)
        j = rem // gcount; bh = head0 + g0 + rem % gcount
        qb = nqb - 1 - j if causal else j
        return qb, bh % hpb, bh // hpb
    def item_at(i):
        qb, hh, b = decompose(i)
        h = 2 * hh if pair else hh
        q0 = qb * BMI
        kend = Nk
        if causal: kend = min(Nk, q0 + BMI + off)
        nkb = cdiv(kend, BN) if kend > 0 else 0
        kb_lo = 0
        if causal and win > 0: kb_lo = min(nkb, max(0, q0 + off - win + 1) // BN)
        nkb = max(nkb, kb_lo + (2 if persist else 1))
        return dict(bh=b * H + h, bh2=b * H + h + (1 if pair and not _SAME_HEAD else 0), bg=b * Hkv + h // rep,
                    q0=q0, nkb=nkb, kb_lo=kb_lo, id=i)
    def item_id(g, r):
        if not persist: return g if r == 0 else -1
        if xcd:
            S = grid >> 3; sl = g >> 3; x = g & 7
            k = r * S + ((S - 1 - sl) if (r & 1) else sl)
            return k * 8 + x if k < (items >> 3) else -1
        k = r * grid + ((grid - 1 - g) if (r & 1) else g)
        return k if k < items else -1
    covered = set()
    rows_out = {}
    groups = range(grid) if max_groups is None else range(min(grid, max_groups))
    for g in groups:
        logs = {}
        for w in range(NW):
            role = w >> 2; wr = w ^ 4
            ev = []; bars = 0
            r = 0
            iid = item_id(g, 0)
            if iid < 0: break
            cur = item_at(iid); sb = 0
            def look_ahead(r):
                nid = item_id(g, r + 1)
                hn = persist and nid >= 0
                return hn, (item_at(nid) if hn else cur)
            has_next, nxt = look_ahead(r)
            # prologue
            ev.append(('loadK', 0, (cur['id'], cur['kb_lo']), cur['kb_lo'] & 1)); bars += 1; period = 1
            if role == 0:   # the first switch period's tiles, issued in the prologue
                ev.append(('loadK', 0, (cur['id'], cur['kb_lo'] + 1), (cur['kb_lo'] & 1) ^ 1))
                ev.append(('loadV', 0, (cur['id'], cur['kb_lo']), cur['kb_lo'] & 1))
            for part in range(8): ev.append(('loadQ', 0, cur['id'], part))
            def geom(it):
                qw0 = it['q0'] + ((w & 3) if pair else wr) * 32
                nkb_w = it['nkb']
                if causal: nkb_w = max(0, min(it['nkb'], tdiv(qw0 + 31 + off, BN) + 1))
                windowed = causal and win > 0
                a_w = min(nkb_w, max(0, qw0 + off - win + 1) // BN) if windowed else 0
                return qw0, nkb_w, a_w
            has_prev = False; has_cur = True; do_pv = False; j_last = 0; prev = None
            mb = cur['kb_lo'] & 1
            j_knext = max(cur['kb_lo'], cur['nkb'] - 1)
            wave_g = None
            def per(kind, j, slots, reads, loads):
                ev.append((kind, period, j, slots, reads, loads))
            while True:
                # switch period
                bars += 1
                if role == 1 and do_pv: ev.append(('SM', period, prev['id'], j_last))
                if do_pv: ev.append(('PV', period, prev['id'], j_last, ('V', mb ^ 1)))
                if has_cur:
                    qw0, nkb_w, a_w = geom(cur); wave_g = (qw0, nkb_w, a_w)
                    ev.append(('readQ', period, cur['id']))
                if has_prev:
                    ev.append(('out', period, prev['id'], prev['bh2'] if pair and role == 1 else prev['bh'],
                               geom(prev)[0]))
                if not has_cur:
                    period += 1; break
                do_s = nkb_w > a_w and a_w == cur['kb_lo']
                j = cur['kb_lo']
                if role == 0 and has_prev:
                    ldk = j + 1 < cur['nkb'] or (has_next and j == j_knext)
                    ktile = (cur['id'], j + 1) if j + 1 < cur['nkb'] else (nxt['id'], nxt['kb_lo'])
                    if ldk: ev.append(('loadK', period, ktile, mb ^ 1))
                    ev.append(('loadV', period, (cur['id'], j), mb))
                if do_s:
                    ev.append(('S', period, cur['id'], j, ('K', mb)))
                    if role == 0: ev.append(('SM', period, cur['id'], j))
                period += 1
                # item periods
                q_first = cur['kb_lo'] + 1
                qcount = cur['nkb'] - q_first
                qpp = 1
                while qpp < 8 and qpp * qcount < 8: qpp *= 2
                started = a_w == cur['kb_lo']; ends = nkb_w == cur['nkb']
                def run_period(j, first, last_, sm, rl):
                    # first/last: 'S' steps, 'PV' steps flags; sm: 1 softmax j-1 before, 2 softmax j after
                    nonlocal period, bars
                    bars += 1
                    b = (j + sb) & 1
                    ldk = j + 1 < cur['nkb'] or (has_next and j == j_knext)
                    ldv = j < cur['nkb']
                    if role == 0:
                        ktile = (cur['id'], j + 1) if j + 1 < cur['nkb'] else (nxt['id'], nxt['kb_lo'])
                        if ldk: ev.append(('loadK', period, ktile, b ^ 1))
                        if ldv: ev.append(('loadV', period, (cur['id'], j), b))
                    if has_next:
                        for part in range(min(8, (j - q_first) * qpp), min(8, (j - q_first + 1) * qpp)):
                            ev.append(('loadQ', period, nxt['id'], part))
                    if sm == 1: ev.append(('SM', period, cur['id'], j - 1))
                    if 'PV' in first: ev.append(('PV', period, cur['id'], j - 1, ('V', b ^ 1)))
                    if 'S' in first: ev.append(('S', period, cur['id'], j, ('K', b)))
                    if sm == 2: ev.append(('SM', period, cur['id'], j))
                    period += 1
                j = q_first
                while j < a_w: run_period(j, (), None, 0, 2); j += 1
                if nkb_w > a_w:
                    if role == 0:
                        if not started: run_period(j, ('S',), None, 2, 0); j += 1
                        while j < nkb_w: run_period(j, ('PV', 'S'), None, 2, 0); j += 1
                        if not ends: run_period(j, ('PV',), None, 0, 0); j += 1
                    else:
                        if not started: run_period(j, ('S',), None, 0, 1); j += 1
                        while j < nkb_w: run_period(j, ('PV', 'S'), None, 1, 1); j += 1
                        if not ends: run_period(j, ('PV',), None, 1, 1); j += 1
                while j < cur['nkb']: run_period(j, (), None, 0, 2); j += 1
                assert j == cur['nkb']
                has_prev = True
                do_pv = nkb_w > a_w and nkb_w == cur['nkb']
                j_last = cur['nkb'] - 1
                prev = cur
                mb = (cur['nkb'] + sb) & 1
                has_cur = has_next
                if has_next:
                    sb = ((j_knext + 1 + sb - nxt['kb_lo']) & 1) ^ (1 if _FLIP else 0)
                    cur = nxt; r += 1
                    has_next, nxt = look_ahead(r)
                    j_knext = max(cur['kb_lo'], cur['nkb'] - 1)
            logs[w] = (bars, ev)
        if not logs: continue
        bs = {w: logs[w][0] for w in logs}
        assert len(set(bs.values())) == 1, ('barrier counts differ', g, bs)
        # slot contents: loads in period p visible from period p+1 on
        kslot = {}; vslot = {}
        loads = sorted([e for w in logs for e in logs[w][1] if e[0] in ('loadK', 'loadV')], key=lambda e: e[1])
        byp = {}
        for e in loads: byp.setdefault(e[1], []).append(e)
        maxp = max(e[1] for w in logs for e in logs[w][1])
        state_k = {}; state_v = {}
        snapshot = {}
        for pp in range(0, maxp + 2):
            snapshot[pp] = (dict(state_k), dict(state_v))
            for e in byp.get(pp, []):
                (state_k if e[0] == 'loadK' else state_v)[e[3]] = e[2]
        # loads of one period go to slots not read in that period
        for w in logs:
            for e in logs[w][1]:
                if e[0] in ('S', 'PV'):
                    pp = e[1]; kind, slot = e[-1]
                    sk, sv = snapshot[pp]
                    want = (e[2], e[3])
                    have = (sk if kind == 'K' else sv).get(slot)
                    assert have == want, ('slot holds the wrong tile', g, w, e, have)
                    for le in byp.get(pp, []):
                        if le[0] == ('loadK' if kind == 'K' else 'loadV'):
                            assert le[3] != slot, ('load into a slot read in the same period', g, w, e, le)
        # Q area: every slice holds the item when a wave reads its fragments;
        # no slice load lands in a period where the wave stages its rows there
        qloads = {}
        for w in logs:
            for e in logs[w][1]:
                if e[0] == 'loadQ': qloads.setdefault(e[1], {})[e[3]] = e[2]
        qstate = {}; qsnap = {}
        for pp in range(0, maxp + 2):
            qsnap[pp] = dict(qstate)
            qstate.update(qloads.get(pp, {}))
        for w in logs:
            for e in logs[w][1]:
                if e[0] == 'readQ':
                    assert all(qsnap[e[1]].get(part) == e[2] for part in range(8)), ('Q area', g, w, e, qsnap[e[1]])
                    assert not qloads.get(e[1]), ('Q load in a switch period', g, e)
        # per wave order and coverage
        for w in logs:
            role = w >> 2
            seen = {}
            for e in logs[w][1]:
                if e[0] in ('S', 'SM', 'PV'):
                    key = (e[2], e[3])
                    seen.setdefault(key, []).append((e[0], e[1]))
            for key, lst in seen.items():
                kinds = [k for k, _ in lst]
                assert kinds == ['S', 'SM', 'PV'], (g, w, key, lst)
                ps = {k: p for k, p in lst}
                if role == 0: assert ps['S'] == ps['SM'] and ps['PV'] == ps['S'] + 1, (g, w, key, lst)
                else: assert ps['SM'] == ps['S'] + 1 and ps['PV'] == ps['SM'], (g, w, key, lst)
            # the wave's tiles: exactly [a_w, nkb_w) of each item it runs
            outs = [e for e in logs[w][1] if e[0] == 'out']
            for e in outs:
                covered.add((e[2], w))
                if e[4] < Nq: rows_out[(e[3], e[4])] = rows_out.get((e[3], e[4]), 0) + 1
    # every item's rows written once per wave
    if max_groups is None:
        assert len(covered) == items * NW, (len(covered), items * NW)
        want = {(bh, q) for bh in range(B * H) for q in range(0, Nq, 32)}
        assert set(rows_out) == want and all(c == 1 for c in rows_out.values()), \
            ('output rows', sorted(set(rows_out) ^ want)[:8], [k for k, c in rows_out.items() if c != 1][:8])


WORKLOADS = [(4, 64, 1, 4096, 4096, False, 0, 0), (8, 32, 32, 2048, 2048, True, 0, 0),
             (1, 32, 8, 8192, 8192, True, 0, 0), (1, 32, 8, 16384, 16384, True, 4096, 0),
             (4, 32, 8, 512, 8192, True, 0, 0)]


@pytest.mark.parametrize("case", WORKLOADS, ids=lambda c: "x".join(str(x) for x in c))
def test_benchmark_shapes(case):
    run(*case, max_groups=24)


def _random_cases(n, seed=7):
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        B = rng.randint(1, 3)
        Hkv = rng.choice([1, 2, 4])
        H = Hkv * rng.choice([1, 2, 3, 4])
        Nq = rng.choice([1, 31, 64, 65, 255, 256, 257, 511, 600, 900, rng.randint(1, 1500)])
        Nk = rng.choice([1, 31, 64, 65, 127, 255, 256, 257, 300, 600, 1000, rng.randint(1, 1500)])
        causal = rng.random() < 0.6
        window = rng.randint(1, Nk + 64) if causal and rng.random() < 0.4 else 0
        cap = rng.choice([0, 1, 2, 3, 5, 8, 13])
        persist = rng.random() < 0.85
        out.append((B, H, Hkv, Nq, Nk, causal, window, cap, persist, 4, rng.choice([256, 16, 8])))
    return out


@pytest.mark.parametrize("case", _random_cases(60), ids=lambda c: "x".join(str(x) for x in c))
def test_random_shapes(case):
    run(*case)


def test_model_catches_a_slot_parity_mistake(monkeypatch):
    """The slot check is live: with the parity of the next item's first tile
    flipped, some read finds the wrong tile."""
    global _FLIP
    _FLIP = True
    try:
        with pytest.raises(AssertionError):
            run(2, 8, 2, 600, 600, True, 0, 3)
    finally:
        _FLIP = False


def test_model_catches_a_paired_head_mistake():
    """The output-row check is live: with both wave groups of a paired item on
    the same head, one head's rows are written twice and the other's never."""
    global _SAME_HEAD
    _SAME_HEAD = True
    try:
        with pytest.raises(AssertionError):
            run(1, 4, 2, 300, 300, True, 0, 2)
    finally:
        _SAME_HEAD = False
