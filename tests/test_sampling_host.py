"""Host emulation of how the sampling kernel locates the inverse-CDF crossing.

The kernel (one 1024-thread workgroup per row, 16 waves, 8 entries per
thread per 8192-entry super-tile) forms fp32 sums in fixed orders: each
thread's 8 weights in order, a butterfly sum per wave, the 16 wave totals in
wave order, the super-tile totals in order, and a Hillis-Steele scan of the
threads' sums inside a wave.  This file repeats exactly that arithmetic in
numpy float32 and checks the property the kernel relies on: the threads'
claimed ranges of running weight tile [0, total) without gaps, so every
target below the total is claimed and the pick lies at the crossing of the
row's distribution (Microgpt, "Inference": the next token is drawn from the
predicted distribution).  A variant that forms each thread's range on its
own (the lower bound from the scan, the upper bound as lower bound plus the
thread's sum) leaves gaps; the last test shows the check catches that.

No GPU is used; the expected answer is the float64 cumulative distribution
of the same float32 weights.
"""
import numpy as np

F = np.float32
NW, LANES, PER = 16, 64, 8
TILE = NW * LANES * PER


def _seq_sum(a, axis):
    """Sum along `axis` one element after another, in float32."""
    a = np.moveaxis(a, axis, 0)
    s = np.zeros(a.shape[1:], F)
    for x in a:
        s = (s + x).astype(F)
    return s


def _seq_excl(a, axis):
    """Exclusive running sums along `axis`, one element after another, in float32."""
    a = np.moveaxis(a, axis, 0)
    out = np.empty_like(a)
    s = np.zeros(a.shape[1:], F)
    for i, x in enumerate(a):
        out[i] = s
        s = (s + x).astype(F)
    return np.moveaxis(out, 0, axis)


def _butterfly(v):
    """Wave sum by xor shuffles over the last axis (64 lanes)."""
    lanes = np.arange(LANES)
    for o in (32, 16, 8, 4, 2, 1):
        v = (v + v[..., lanes ^ o]).astype(F)
    return v[..., 0]


def _scan(v):
    """Inclusive Hillis-Steele scan over the last axis (64 lanes)."""
    for o in (1, 2, 4, 8, 16, 32):
        sh = np.zeros_like(v)
        sh[..., o:] = v[..., :-o]
        v = (v + sh).astype(F)
    return v


def ranges(e, tiled=True):
    """Per-thread [lo, hi) of the running weight for every super-tile, the
    super-tile totals and their exclusive running sums, and the row total.
    e: float32 [NS, NW, LANES, PER]."""
    mine = _seq_sum(e, axis=3)                       # [NS, NW, LANES]
    wtot = _butterfly(mine)                          # [NS, NW]
    T = _seq_sum(wtot, axis=1)                       # [NS]
    run = _seq_excl(T, axis=0)                       # [NS]
    total = _seq_sum(T, axis=0)
    before = _seq_excl(wtot, axis=1)                 # [NS, NW]
    base_w = (run[:, None] + before).astype(F)
    incl = _scan(mine)
    excl = np.zeros_like(incl)
    excl[..., 1:] = incl[..., :-1]
    lo = (base_w[..., None] + excl).astype(F)
    if tiled:
        base_n = (run[:, None] + (before + wtot).astype(F)).astype(F)
        hi = np.empty_like(lo)
        hi[..., :-1] = lo[..., 1:]
        hi[..., -1] = base_n
    else:
        # each thread on its own: excl = (base + incl) - mine, hi = excl + mine
        lo = ((base_w[..., None] + incl).astype(F) - mine).astype(F)
        hi = (lo + mine).astype(F)
    return lo, hi, T, run, total


def picks(e, us, tiled=True):
    """Emulated kernel choice for each uniform in `us` (float32); -2 where no
    thread claims a target below the total."""
    NS = e.shape[0]
    lo, hi, T, run, total = ranges(e, tiled)
    flat_e = e.reshape(NS, NW * LANES, PER)
    lo = lo.reshape(NS, -1)
    hi = hi.reshape(NS, -1)
    pos = flat_e > 0
    idx = np.arange(NS * TILE).reshape(NS, NW * LANES, PER)
    lastpos = np.where(pos, idx, -1).max(axis=2)                # [NS, threads]
    prefmax = np.maximum.accumulate(lastpos, axis=1)
    row_last = int(np.max(np.where(pos, idx, -1)))
    out = np.empty(len(us), np.int64)
    for i, u in enumerate(us):
        target = F(F(u) * total)
        hit = np.nonzero((run + T).astype(F) > target)[0]
        if len(hit) == 0:
            out[i] = row_last
            continue
        sx = hit[0]
        claim = np.nonzero((lo[sx] <= target) & (target < hi[sx]))[0]
        if len(claim) == 0:
            out[i] = -2
            continue
        best = None
        for t in claim:
            cum = lo[sx, t]
            pick = -1
            for j in range(PER):
                cum = F(cum + flat_e[sx, t, j])
                if pick < 0 and cum > target:
                    pick = int(idx[sx, t, j])
            if pick < 0:
                pick = int(prefmax[sx, t])
            if pick >= 0:
                best = pick if best is None else min(best, pick)
        out[i] = best if best is not None else -2
    return out


def weights(logits, T=0.7):
    x = logits.astype(F)
    sc = F(F(1.0 / T) * F(1.4426950408889634))
    return np.exp2(((x - x.max()) * sc).astype(F)).astype(F)


def boundary_uniforms(e, rng, n):
    """Uniforms aimed at the running weight just before and after thread,
    wave and super-tile boundaries, plus plain draws."""
    c = np.cumsum(e.astype(np.float64))
    c /= c[-1]
    b = rng.choice([PER, PER * LANES, TILE], size=n)
    k = (rng.integers(1, len(c) // b) * b)
    eps = rng.choice([-1, 1], size=n) * 10.0 ** rng.uniform(-9, -6, size=n)
    u = np.clip(c[k - 1] + eps, 0, 1 - 2 ** -24)
    u[: n // 4] = rng.random(n // 4)
    return u.astype(F)


def check_row(logits, rng, n=600, tiled=True):
    V = logits.shape[0]
    ns = (V + TILE - 1) // TILE
    e = np.zeros(ns * TILE, F)
    e[:V] = weights(logits)
    us = boundary_uniforms(e[:V], rng, n)
    got = picks(e.reshape(ns, NW, LANES, PER), us, tiled)
    c = np.cumsum(e[:V].astype(np.float64))
    c /= c[-1]
    bad = 0
    for u, k in zip(us, got):
        if k < 0:
            bad += 1
            continue
        lo = c[k - 1] if k > 0 else 0.0
        if not (lo - 1e-5 <= u <= c[k] + 1e-5):
            bad += 1
    return bad


def test_tiled_ranges_claim_every_target():
    """Flat random-weight rows (logit std 0.8, T = 0.7) and peaked rows where
    most weights underflow to zero, with uniforms aimed at every kind of
    boundary: every target is claimed and every pick is at its crossing."""
    rng = np.random.default_rng(5)
    for r in range(24):
        V = 65536 if r % 3 else 40000
        lg = rng.standard_normal(V) * (0.8 if r % 2 else 40.0)
        assert check_row(lg, rng) == 0, r


def test_ranges_tile_exactly():
    """The upper bound of each thread is the lower bound of the next, across
    lanes, waves and (through the running total) super-tiles."""
    rng = np.random.default_rng(6)
    e = weights(rng.standard_normal(65536) * 0.8).reshape(8, NW, LANES, PER)
    lo, hi, T, run, total = ranges(e)
    flo, fhi = lo.reshape(8, -1), hi.reshape(8, -1)
    assert np.array_equal(fhi[:, :-1], flo[:, 1:])
    assert np.array_equal(flo[:, 0], run)
    assert np.array_equal(fhi[:, -1], (run + T).astype(F))


def test_independent_ranges_leave_gaps():
    """The check above has teeth: ranges formed thread by thread leave
    targets that no thread claims, or send them far from the crossing."""
    rng = np.random.default_rng(5)
    bad = sum(check_row(rng.standard_normal(65536) * 0.8, rng, n=1500, tiled=False) for _ in range(6))
    assert bad > 0
