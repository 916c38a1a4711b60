"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

The pages print no worked numeric example, so every pin comes from the
mathematics of softmax attention and from invariants the method must keep:

1. brute force: an independent pure-Python implementation (its own bf16
   decoding, token slots found by walking each request's page list, math.fsum
   sums) on tiny batches;
2. seq_len = 1 returns that token's V row exactly;
3. relabelling the physical pages (and the page table with them) changes no bit;
4. any split count merges to the unsplit result (empty splits included);
5. q = 0 gives the uniform average of the V rows;
6. constant V returns the constant; one dominant key returns its V row;
7. with an identity page table the result is torch's scaled_dot_product_attention
   in float64 with the KV heads repeated;
8. integer parts: kv_indptr page counts bracket the lengths, the split plan
   equals a search-based re-derivation of its rule, the append writes exactly
   the slot of the newest token;
9. NaN poison in free pages and past-the-end slots never reaches an output;
10. the keep mask: brute force over the kept tokens only, an all-true mask is the
    unmasked decode bit for bit, an all-false row is zero, masking a request's
    newest token equals decoding one token shorter, and mask entries past
    seq_len change nothing;
11. prefill: brute force over each row's visible keys, one-row requests are the
    decode bit for bit, causal row i is the decode of the first L - n + i + 1
    tokens, the non-causal rows all see L tokens, and with an identity page
    table and no prefix the causal result is torch's scaled_dot_product_attention
    (is_causal) in float64;
12. token-major K/V: brute force over each request's slots (table and
    contiguous), the paged batches stored token-major give the paged decode
    bit for bit, the contiguous layout equals the table b * stride + t, and a
    one-token request returns that slot's V row.

``test_planted_mistakes`` plants plausible mistakes in the oracle (on the CPU)
and checks that at least one pin fails for each.
"""

import math
import struct

import numpy as np
import pytest
import torch

import oracle.attention as OA
import workloads as W


# ----------------------------------------------------------------- fixtures

def tiny_batch(seed=11, poison=True, lengths=(1, 23, 9, 0)):
    return W.make_batch(
        name="tiny4", seed=seed, B=len(lengths), Hq=4, Hkv=2, D=16, P=4,
        lengths=np.array(lengths), num_pages=24, poison=poison,
    )


def gqa8_batch(seed=12):
    # G = 4 with 8 query heads; ragged lengths with a partial last page.
    return W.make_batch(
        name="gqa8", seed=seed, B=2, Hq=8, Hkv=2, D=8, P=4,
        lengths=np.array([13, 6]), num_pages=12,
    )


def run_decode(mod, batch):
    ip = mod.kv_indptr(batch.seq_lens, batch.P)
    return mod.decode(batch.q, batch.k_pool, batch.v_pool, ip, batch.kv_indices,
                      batch.seq_lens, batch.sm_scale, batch.P)


# --------------------------------------------------------- brute force (pin 1)

def _bf16_py(bits) -> float:
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def _token_slots(batch, b):
    """(page, offset) of request b's tokens, found by walking its pages in order."""
    slots = []
    for page in batch.page_lists[b]:
        for off in range(batch.P):
            slots.append((int(page), off))
    return slots[: int(batch.seq_lens[b])]


def brute_force(batch):
    B, Hq, Hkv, D = batch.B, batch.Hq, batch.Hkv, batch.D
    out = np.zeros((B, Hq, D))
    for b in range(B):
        slots = _token_slots(batch, b)
        if not slots:
            continue
        for hq in range(Hq):
            h = (hq * Hkv) // Hq
            qv = [_bf16_py(batch.q[b, hq, d]) for d in range(D)]
            xs = []
            for page, off in slots:
                kv = [_bf16_py(batch.k_pool[page, h, off, d]) for d in range(D)]
                xs.append(batch.sm_scale * math.fsum(a * c for a, c in zip(qv, kv)))
            m = max(xs)
            ws = [math.exp(x - m) for x in xs]
            den = math.fsum(ws)
            for d in range(D):
                num = math.fsum(w * _bf16_py(batch.v_pool[p, h, o, d]) for w, (p, o) in zip(ws, slots))
                out[b, hq, d] = num / den
    return out


def pin_brute_force(mod):
    for batch in (W.config(1), tiny_batch(), gqa8_batch()):
        got = run_decode(mod, batch)
        ref = brute_force(batch)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


# ------------------------------------------------------ invariants (pins 2-6)

def pin_seq_len_one(mod):
    batch = W.make_batch(name="len1", seed=21, B=3, Hq=8, Hkv=2, D=32, P=16,
                         lengths=np.ones(3, np.int64), num_pages=8)
    got = run_decode(mod, batch)
    G = batch.Hq // batch.Hkv
    for b in range(batch.B):
        page = int(batch.page_lists[b][0])
        for hq in range(batch.Hq):
            row = W.bf16_bits_to_f32(batch.v_pool[page, hq // G, 0]).astype(np.float64)
            assert np.array_equal(got[b, hq], row)


def pin_permutation(mod):
    for batch in (W.config(1), tiny_batch()):
        a = run_decode(mod, batch)
        b = run_decode(mod, W.permute_pool(batch, seed=99))
        assert np.array_equal(a, b, equal_nan=False)


def pin_split_invariance(mod):
    for batch in (W.config(1), tiny_batch(), gqa8_batch()):
        ip = mod.kv_indptr(batch.seq_lens, batch.P)
        ref = run_decode(mod, batch)
        npages = [len(pl) for pl in batch.page_lists]
        for k in range(1, max(npages) + 3):
            # k splits where possible; requests with fewer pages also get empty splits
            ns = np.full(batch.B, k)
            got = mod.decode_split(batch.q, batch.k_pool, batch.v_pool, ip, batch.kv_indices,
                                   batch.seq_lens, batch.sm_scale, batch.P, ns)
            np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def _valid_rows(pool, batch, b, h):
    return np.array([W.bf16_bits_to_f32(pool[p, h, o]) for p, o in _token_slots(batch, b)],
                    dtype=np.float64)


def pin_q_zero(mod):
    for batch in (tiny_batch(), gqa8_batch()):
        batch.q[:] = 0
        got = run_decode(mod, batch)
        G = batch.Hq // batch.Hkv
        for b in range(batch.B):
            if batch.seq_lens[b] == 0:
                continue
            for hq in range(batch.Hq):
                mean = _valid_rows(batch.v_pool, batch, b, hq // G).mean(axis=0)
                np.testing.assert_allclose(got[b, hq], mean, rtol=0, atol=1e-12)


def pin_constant_v(mod):
    batch = tiny_batch(poison=False, lengths=(5, 17, 3))
    c = W.f32_to_bf16_bits(np.float32(0.7109375))
    batch.v_pool[:] = c
    got = run_decode(mod, batch)
    np.testing.assert_allclose(got, np.full(got.shape, 0.7109375), rtol=0, atol=1e-12)


def pin_dominant_key(mod):
    batch = tiny_batch(poison=True, lengths=(9, 14, 6))
    rng = np.random.default_rng(5)
    G = batch.Hq // batch.Hkv
    for b in range(batch.B):
        slots = _token_slots(batch, b)
        j = int(rng.integers(len(slots)))
        p, o = slots[j]
        for h in range(batch.Hkv):
            big = W.bf16_bits_to_f32(batch.k_pool[p, h, o]) * np.float32(4.0)
            batch.k_pool[p, h, o] = W.f32_to_bf16_bits(big)
            for g in range(G):
                batch.q[b, h * G + g] = W.f32_to_bf16_bits(big * np.float32(16.0))
        batch.notes[b] = (p, o)
    got = run_decode(mod, batch)
    for b in range(batch.B):
        p, o = batch.notes[b]
        for hq in range(batch.Hq):
            row = W.bf16_bits_to_f32(batch.v_pool[p, hq // G, o]).astype(np.float64)
            np.testing.assert_allclose(got[b, hq], row, rtol=0, atol=1e-9)


# ------------------------------------------------- library special case (pin 7)

def pin_sdpa(mod):
    for batch in (W.identity_layout(W.config(1)), W.identity_layout(tiny_batch()),
                  W.identity_layout(gqa8_batch())):
        got = run_decode(mod, batch)
        G = batch.Hq // batch.Hkv
        for b in range(batch.B):
            L = int(batch.seq_lens[b])
            if L == 0:
                continue
            pages = batch.page_lists[b]
            p0, n = int(pages[0]), len(pages)

            def dense(pool):
                blk = W.bf16_bits_to_f32(pool[p0 : p0 + n]).astype(np.float64)  # [n, Hkv, P, D]
                blk = np.transpose(blk, (1, 0, 2, 3)).reshape(batch.Hkv, n * batch.P, batch.D)
                t = torch.from_numpy(np.ascontiguousarray(blk[:, :L]))
                return t.repeat_interleave(G, dim=0)[None]  # [1, Hq, L, D]

            q = torch.from_numpy(W.bf16_bits_to_f32(batch.q[b]).astype(np.float64))[None, :, None, :]
            ref = torch.nn.functional.scaled_dot_product_attention(
                q, dense(batch.k_pool), dense(batch.v_pool), scale=batch.sm_scale)
            np.testing.assert_allclose(got[b], ref[0, :, 0].numpy(), rtol=0, atol=1e-12)


# ----------------------------------------------------- integer parts (pin 8)

def pin_kv_indptr(mod):
    ragged = W.make_batch(name="ragged_small_d", seed=3, B=16, Hq=4, Hkv=1, D=8, P=16,
                          lengths=lambda r: r.integers(1, 4097, size=16), poison=False)
    for batch in (W.config(1), ragged, tiny_batch()):
        ip = np.asarray(mod.kv_indptr(batch.seq_lens, batch.P))
        assert ip.shape == (batch.B + 1,) and ip[0] == 0
        for b in range(batch.B):
            n = int(ip[b + 1] - ip[b])
            L = int(batch.seq_lens[b])
            assert n == len(batch.page_lists[b])
            assert (n == 0 and L == 0) or ((n - 1) * batch.P < L <= n * batch.P)


def _enumerate_tiles(seq_lens, P, U):
    """Every (request, head group, page) tile, listed one by one."""
    tiles = []
    for b, L in enumerate(seq_lens):
        n = 0
        while n * P < L:
            n += 1
        for u in range(U):
            for p in range(n):
                tiles.append((b, u, p))
    return tiles


def _pieces_of_plan(tiles, waves):
    """(b, u, first page, pages) pieces: each wave's range cut at segment borders."""
    pieces, pos = [], 0
    for b, u, p, cnt in waves:
        if cnt == 0:
            continue
        pos = tiles.index((b, u, p), pos)
        run = tiles[pos:pos + cnt]
        assert len(run) == cnt
        start = run[0]
        n = 1
        for prev, cur in zip(run, run[1:]):
            if cur[:2] == prev[:2]:
                n += 1
            else:
                pieces.append((*start, n))
                start, n = cur, 1
        pieces.append((*start, n))
        pos += cnt
    return pieces


def pin_plan(mod):
    rng = np.random.default_rng(7)
    cases = [(np.array([37]), 16, 8, 256, 8, 0), (np.array([0, 0]), 16, 8, 4, 8, 0)]
    for _ in range(40):
        B = int(rng.integers(1, 12))
        seq = rng.integers(0, 700, size=B)
        cases.append((seq, int(rng.choice([1, 4, 16])), int(rng.choice([1, 2, 8])),
                      int(rng.integers(1, 64)), int(rng.integers(1, 12)),
                      int(rng.choice([0, 0, 1, 3, 50]))))
    for seq, P, U, groups, mt, forced in cases:
        plan = mod.plan_stream(seq, P, U, groups, mt, forced)
        tiles = _enumerate_tiles(list(seq), P, U)
        T = len(tiles)
        assert plan["tiles"] == T
        # workgroups: fewest with min_tiles each, capped by the grid (or forced)
        if T == 0:
            W = 0
        elif forced:
            W = min(forced, groups, T)
        else:
            W = 1
            while W * mt < T and W < groups:
                W += 1
        assert plan["groups"] == W
        waves = [tuple(int(x) for x in r) for r in plan["waves"]]
        assert len(waves) == groups * 8
        # every tile exactly once, in order, and equal shares per workgroup and wave
        covered = []
        pos = 0
        for i in range(groups):
            share = []
            for w in range(8):
                b, u, p, cnt = waves[i * 8 + w]
                if cnt:
                    assert tiles[pos] == (b, u, p)
                share.append(cnt)
                covered.extend(tiles[pos:pos + cnt])
                pos += cnt
            if i < W:
                tot = sum(share)
                assert abs(tot - T / W) < 1 and max(share) - min(share) <= 1
            else:
                assert sum(share) == 0
        assert covered == tiles


def pin_head_groups(mod):
    """The decode plan's head grouping (a rule of this library's plan; the pages
    only say that the query heads of one KV head read its K/V together).

    Three statements of it: the table of head-group sizes that the library
    header documents, written out by hand (the largest of 1 .. 8, 12 and 16
    that divides G: all of a KV head's query heads up to eight, then sixteen,
    twelve, eight, seven, ..., one); the same sizes found by counting, for every size built,
    the passes over each KV head it needs (G / HG, fewest wins, only sizes that
    divide G allowed); and the structure every grouping must have (a group
    lies inside one KV head, and the groups cover the query heads exactly
    once)."""
    table = {1: 1, 2: 2, 3: 3, 4: 4, 5: 5, 6: 6, 7: 7, 8: 8, 9: 3, 10: 5, 11: 1, 12: 12,
             13: 1, 14: 7, 15: 5, 16: 16, 18: 6, 20: 5, 21: 7, 24: 12, 28: 7, 32: 16,
             36: 12, 40: 8, 44: 4, 48: 16, 60: 12}
    for G, hg in table.items():
        for Hkv in (1, 2, 8):
            assert mod.head_groups(G * Hkv, Hkv) == (hg, G * Hkv // hg), (G, Hkv)
    built = (1, 2, 3, 4, 5, 6, 7, 8, 12, 16)
    for G in range(1, 65):
        for Hkv in (1, 3, 8):
            Hq = G * Hkv
            HG, U = mod.head_groups(Hq, Hkv)
            passes = {h: G // h for h in built if G % h == 0}
            assert passes[HG] == min(passes.values()), (G, Hkv, HG)
            assert HG * U == Hq
            heads = []
            for u in range(U):
                grp = list(range(u * HG, (u + 1) * HG))
                assert len({mod.kv_head_of(h, G) for h in grp}) == 1, (G, u)
                heads.extend(grp)
            assert heads == list(range(Hq))


def pin_stream_pieces(mod):
    """The plan's pieces merge to the unsplit result for many grid sizes."""
    for batch in (tiny_batch(), gqa8_batch(), W.config(1)):
        HG, U = mod.head_groups(batch.Hq, batch.Hkv)
        ip = mod.kv_indptr(batch.seq_lens, batch.P)
        ref = run_decode(mod, batch)
        tiles = _enumerate_tiles(list(batch.seq_lens), batch.P, U)
        for groups, mt, forced in ((1, 8, 0), (3, 1, 0), (64, 1, 0), (5, 8, 2), (7, 1, 7)):
            plan = mod.plan_stream(batch.seq_lens, batch.P, U, groups, mt, forced)
            pieces = _pieces_of_plan(tiles, plan["waves"])
            got = mod.decode_pieces(batch.q, batch.k_pool, batch.v_pool, ip, batch.kv_indices,
                                    batch.seq_lens, batch.sm_scale, batch.P, pieces)
            np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def pin_append(mod):
    batch = W.make_batch(name="append_small", seed=31, B=6, Hq=4, Hkv=2, D=8, P=4,
                         lengths=np.array([1, 4, 5, 8, 13, 2]), num_pages=40, append=True)
    ip = mod.kv_indptr(batch.seq_lens, batch.P)
    k2, v2 = mod.append_kv(batch.k_pool, batch.v_pool, batch.k_new, batch.v_new, ip,
                           batch.kv_indices, batch.seq_lens, batch.P)
    changed = np.zeros(batch.k_pool.shape[:1] + batch.k_pool.shape[2:3], bool)
    for b in range(batch.B):
        p, o = _token_slots(batch, b)[-1]
        assert np.array_equal(k2[p, :, o], batch.k_new[b])
        assert np.array_equal(v2[p, :, o], batch.v_new[b])
        changed[p, o] = True
    keep = np.broadcast_to(~changed[:, None, :, None], k2.shape)
    assert np.array_equal(k2[keep], batch.k_pool[keep])
    assert np.array_equal(v2[keep], batch.v_pool[keep])
    # the appended batch is now fully written: poison must not reach any output
    out = mod.decode(batch.q, k2, v2, ip, batch.kv_indices, batch.seq_lens,
                     batch.sm_scale, batch.P)
    assert np.isfinite(out).all()


def pin_append_rows(mod):
    """The extend append: byte-level slots found by walking page lists, one
    token per request equals the single-token append, n tokens equal n
    single-token appends at growing lengths, and the written batch reads no
    poison."""
    batch = prefill_batch(seed=35, q_lens=(0, 1, 4, 5, 9, 3), prefix_lens=(6, 0, 3, 4, 0, 1),
                          new_rows=True)
    ip = mod.kv_indptr(batch.seq_lens, batch.P)
    k2, v2 = mod.append_kv_rows(batch.k_pool, batch.v_pool, batch.k_rows, batch.v_rows,
                                batch.qo_indptr, ip, batch.kv_indices, batch.seq_lens, batch.P)
    changed = np.zeros((batch.num_pages, batch.P), bool)
    for b in range(batch.B):
        q0, q1 = int(batch.qo_indptr[b]), int(batch.qo_indptr[b + 1])
        slots = _token_slots(batch, b)
        for i, (p, o) in enumerate(slots[len(slots) - (q1 - q0):]):
            assert np.array_equal(k2[p, :, o], batch.k_rows[q0 + i])
            assert np.array_equal(v2[p, :, o], batch.v_rows[q0 + i])
            changed[p, o] = True
    keep = np.broadcast_to(~changed[:, None, :, None], k2.shape)
    assert np.array_equal(k2[keep], batch.k_pool[keep])
    assert np.array_equal(v2[keep], batch.v_pool[keep])
    # every new slot written: the causal prefill over the batch reads no poison
    out = mod.prefill(batch.q_rows, k2, v2, ip, batch.kv_indices, batch.seq_lens,
                      batch.qo_indptr, batch.sm_scale, batch.P, True)
    assert np.isfinite(out).all()
    # n new tokens = n single-token appends, the length growing by one each time
    kk, vv = batch.k_pool, batch.v_pool
    nmax = int(np.max(np.diff(batch.qo_indptr)))
    for j in range(nmax):
        sl = batch.seq_lens.copy()
        sel = []
        for b in range(batch.B):
            n = int(batch.qo_indptr[b + 1] - batch.qo_indptr[b])
            # request b's j-th new token, at length seq_len - n + j + 1; none past n
            sl[b] = sl[b] - n + j + 1 if j < n else 0
            sel.append(int(batch.qo_indptr[b]) + min(j, max(n - 1, 0)))
        kk, vv = mod.append_kv(kk, vv, batch.k_rows[sel], batch.v_rows[sel], ip,
                               batch.kv_indices, sl, batch.P)
    assert np.array_equal(kk, k2) and np.array_equal(vv, v2)
    # one new token per request: exactly the single-token append
    one = prefill_batch(seed=36, q_lens=(1, 1, 1, 1), prefix_lens=(0, 4, 7, 15), new_rows=True)
    ip1 = mod.kv_indptr(one.seq_lens, one.P)
    a = mod.append_kv_rows(one.k_pool, one.v_pool, one.k_rows, one.v_rows, one.qo_indptr, ip1,
                           one.kv_indices, one.seq_lens, one.P)
    b_ = mod.append_kv(one.k_pool, one.v_pool, one.k_rows, one.v_rows, ip1, one.kv_indices,
                       one.seq_lens, one.P)
    assert np.array_equal(a[0], b_[0]) and np.array_equal(a[1], b_[1])


# ------------------------------------------------------------ poison (pin 9)

def pin_poison(mod):
    for batch in (W.config(1), W.config(2), tiny_batch(), gqa8_batch()):
        assert batch.poisoned
        out = run_decode(mod, batch)
        assert np.isfinite(out).all()


# -------------------------------------------------------------- mask (pin 10)

def brute_force_masked(batch, mask):
    """Pin-1 brute force over the kept tokens only (its own walk of the pages)."""
    B, Hq, Hkv, D = batch.B, batch.Hq, batch.Hkv, batch.D
    out = np.zeros((B, Hq, D))
    for b in range(B):
        slots = [s for t, s in enumerate(_token_slots(batch, b)) if mask[b][t]]
        if not slots:
            continue
        for hq in range(Hq):
            h = (hq * Hkv) // Hq
            qv = [_bf16_py(batch.q[b, hq, d]) for d in range(D)]
            xs = [batch.sm_scale * math.fsum(a * _bf16_py(batch.k_pool[p, h, o, d])
                                             for d, a in enumerate(qv)) for p, o in slots]
            m = max(xs)
            ws = [math.exp(x - m) for x in xs]
            den = math.fsum(ws)
            for d in range(D):
                out[b, hq, d] = math.fsum(w * _bf16_py(batch.v_pool[p, h, o, d])
                                          for w, (p, o) in zip(ws, slots)) / den
    return out


def run_masked(mod, batch, mask):
    ip = mod.kv_indptr(batch.seq_lens, batch.P)
    return mod.decode_masked(batch.q, batch.k_pool, batch.v_pool, ip, batch.kv_indices,
                             batch.seq_lens, batch.sm_scale, batch.P, mask)


def pin_mask(mod):
    batch = tiny_batch(seed=21)
    S = int(batch.seq_lens.max()) + 5
    rng = np.random.default_rng(22)
    mask = rng.random((batch.B, S)) < 0.6
    mask[1, :] = False  # a request that keeps nothing
    got = run_masked(mod, batch, mask)
    assert np.max(np.abs(got - brute_force_masked(batch, mask))) < 1e-12
    assert not got[1].any()
    # all kept: the unmasked decode, bit for bit
    assert np.array_equal(run_masked(mod, batch, np.ones((batch.B, S), bool)), run_decode(mod, batch))
    # entries past seq_len are ignored
    tail = mask.copy()
    for b in range(batch.B):
        tail[b, int(batch.seq_lens[b]):] = ~tail[b, int(batch.seq_lens[b]):]
    assert np.array_equal(run_masked(mod, batch, tail), got)
    # masking the newest token of every request = decoding one token shorter
    g8 = gqa8_batch(seed=23)
    S8 = int(g8.seq_lens.max())
    newest = np.ones((g8.B, S8), bool)
    for b in range(g8.B):
        newest[b, int(g8.seq_lens[b]) - 1] = False
    ip = mod.kv_indptr(g8.seq_lens, g8.P)
    short = mod.decode(g8.q, g8.k_pool, g8.v_pool, ip, g8.kv_indices, g8.seq_lens - 1,
                       g8.sm_scale, g8.P)
    assert np.array_equal(run_masked(mod, g8, newest), short)


# ----------------------------------------------------------- prefill (pin 11)

def prefill_batch(seed=31, q_lens=(3, 1, 6, 2), prefix_lens=(5, 0, 3, 9), **kw):
    args = dict(name="pf", seed=seed, Hq=4, Hkv=2, D=8, P=4, q_lens=q_lens,
                prefix_lens=prefix_lens)
    args.update(kw)
    return W.make_prefill(**args)


def run_prefill(mod, batch, causal, seq_lens=None):
    sl = batch.seq_lens if seq_lens is None else seq_lens
    ip = mod.kv_indptr(batch.seq_lens, batch.P)
    return mod.prefill(batch.q_rows, batch.k_pool, batch.v_pool, ip, batch.kv_indices, sl,
                       batch.qo_indptr, batch.sm_scale, batch.P, causal)


def brute_force_prefill(batch, causal):
    total, Hq, D = batch.q_rows.shape
    Hkv = batch.Hkv
    out = np.zeros((total, Hq, D))
    for b in range(batch.B):
        q0, q1 = int(batch.qo_indptr[b]), int(batch.qo_indptr[b + 1])
        n, L = q1 - q0, int(batch.seq_lens[b])
        slots = _token_slots(batch, b)
        for i in range(n):
            vis = slots[: L - n + i + 1] if causal else slots
            if not vis:
                continue
            for hq in range(Hq):
                h = (hq * Hkv) // Hq
                qv = [_bf16_py(batch.q_rows[q0 + i, hq, d]) for d in range(D)]
                xs = [batch.sm_scale * math.fsum(a * _bf16_py(batch.k_pool[p, h, o, d])
                                                 for d, a in enumerate(qv)) for p, o in vis]
                m = max(xs)
                ws = [math.exp(x - m) for x in xs]
                den = math.fsum(ws)
                for d in range(D):
                    out[q0 + i, hq, d] = math.fsum(w * _bf16_py(batch.v_pool[p, h, o, d])
                                                   for w, (p, o) in zip(ws, vis)) / den
    return out


def pin_prefill(mod):
    batch = prefill_batch()
    for causal in (True, False):
        got = run_prefill(mod, batch, causal)
        assert np.max(np.abs(got - brute_force_prefill(batch, causal))) < 1e-12
    causal = run_prefill(mod, batch, True)
    full = run_prefill(mod, batch, False)
    ip = mod.kv_indptr(batch.seq_lens, batch.P)
    for b in range(batch.B):
        q0, q1 = int(batch.qo_indptr[b]), int(batch.qo_indptr[b + 1])
        n, L = q1 - q0, int(batch.seq_lens[b])
        for i in range(n):
            # the row as a decode query: all L keys, or the first L - n + i + 1
            qd = np.repeat(batch.q_rows[q0 + i][None], batch.B, axis=0)
            for lim, ref in ((L, full), (L - n + i + 1, causal)):
                sl = batch.seq_lens.copy()
                sl[b] = lim
                dec = mod.decode(qd, batch.k_pool, batch.v_pool, ip, batch.kv_indices, sl,
                                 batch.sm_scale, batch.P)
                assert np.array_equal(dec[b], ref[q0 + i])
    # one-row requests: the decode of those rows, bit for bit
    one = prefill_batch(seed=32, q_lens=(1, 1, 1), prefix_lens=(6, 0, 11))
    ip1 = mod.kv_indptr(one.seq_lens, one.P)
    dec = mod.decode(one.q_rows, one.k_pool, one.v_pool, ip1, one.kv_indices, one.seq_lens,
                     one.sm_scale, one.P)
    assert np.array_equal(run_prefill(mod, one, True), dec)
    # identity page table, no prefix, causal: torch SDPA (square, so both
    # alignments of the causal mask agree) in float64
    sq = W.identity_layout(prefill_batch(seed=33, q_lens=(7,), prefix_lens=(0,), poison=False))
    got = run_prefill(mod, sq, True)
    L = int(sq.seq_lens[0])
    # token-major [pages, P, Hkv, D] -> [tokens, Hkv, D]
    k = torch.from_numpy(np.swapaxes(mod.bf16_to_f64(sq.k_pool), 1, 2).reshape(-1, sq.Hkv, sq.D)[:L])
    v = torch.from_numpy(np.swapaxes(mod.bf16_to_f64(sq.v_pool), 1, 2).reshape(-1, sq.Hkv, sq.D)[:L])
    G = sq.Hq // sq.Hkv
    qt = torch.from_numpy(mod.bf16_to_f64(sq.q_rows)).permute(1, 0, 2)  # [Hq, L, D]
    kt = k.permute(1, 0, 2).repeat_interleave(G, dim=0)
    vt = v.permute(1, 0, 2).repeat_interleave(G, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                           scale=sq.sm_scale)
    assert np.max(np.abs(got - ref.permute(1, 0, 2).numpy())) < 1e-12


# ------------------------------------------------------ token-major (pin 12)

def token_batches():
    lens = np.array([7, 0, 1, 12])
    return (W.make_tokens(name="tok", seed=41, B=4, Hq=4, Hkv=2, D=8, lengths=lens),
            W.make_tokens(name="contig", seed=42, B=4, Hq=8, Hkv=2, D=8, lengths=lens,
                          table=False, stride=13))


def run_tokens(mod, tb):
    return mod.decode_tokens(tb.q, tb.k_cache, tb.v_cache, tb.seq_lens, tb.sm_scale,
                             tb.slot_table, tb.stride)


def brute_force_tokens(tb):
    out = np.zeros((tb.B, tb.Hq, tb.D))
    for b in range(tb.B):
        L = int(tb.seq_lens[b])
        slots = [int(tb.slot_table[b][t]) if tb.slot_table is not None else b * tb.stride + t
                 for t in range(L)]
        if not slots:
            continue
        for hq in range(tb.Hq):
            h = (hq * tb.Hkv) // tb.Hq
            qv = [_bf16_py(tb.q[b, hq, d]) for d in range(tb.D)]
            xs = [tb.sm_scale * math.fsum(a * _bf16_py(tb.k_cache[sl, h, d])
                                          for d, a in enumerate(qv)) for sl in slots]
            m = max(xs)
            ws = [math.exp(x - m) for x in xs]
            den = math.fsum(ws)
            for d in range(tb.D):
                out[b, hq, d] = math.fsum(w * _bf16_py(tb.v_cache[sl, h, d])
                                          for w, sl in zip(ws, slots)) / den
    return out


def pin_tokens(mod):
    for tb in token_batches():
        got = run_tokens(mod, tb)
        assert np.isfinite(got).all()
        assert np.max(np.abs(got - brute_force_tokens(tb))) < 1e-12
    # the paged batches stored token-major: the paged decode, bit for bit
    for batch in (W.config(1), tiny_batch(), gqa8_batch()):
        assert np.array_equal(run_tokens(mod, W.tokens_from_pages(batch)), run_decode(mod, batch))
    # the contiguous layout is the table b * stride + t
    _, contig = token_batches()
    ident = np.full((contig.B, contig.stride), -1, np.int32)
    for b in range(contig.B):
        L = int(contig.seq_lens[b])
        ident[b, :L] = b * contig.stride + np.arange(L)
    with_table = mod.decode_tokens(contig.q, contig.k_cache, contig.v_cache, contig.seq_lens,
                                   contig.sm_scale, ident, 0)
    assert np.array_equal(with_table, run_tokens(mod, contig))
    # one token: its V row
    one = W.make_tokens(name="one", seed=43, B=2, Hq=4, Hkv=2, D=8, lengths=np.array([1, 1]))
    got = run_tokens(mod, one)
    for b in range(2):
        for hq in range(4):
            row = W.bf16_bits_to_f32(one.v_cache[one.slot_table[b, 0], hq // 2]).astype(np.float64)
            assert np.array_equal(got[b, hq], row)


PINS = [pin_brute_force, pin_seq_len_one, pin_permutation, pin_split_invariance, pin_q_zero,
        pin_constant_v, pin_dominant_key, pin_sdpa, pin_kv_indptr, pin_plan, pin_head_groups,
        pin_stream_pieces, pin_append_rows,
        pin_append, pin_poison, pin_mask, pin_prefill, pin_tokens]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(OA)


def test_poison_large_configs():
    # full-size ragged batch: the oracle never touches a NaN slot
    batch = W.config(3)
    out = run_decode(OA, batch)
    assert np.isfinite(out).all()


# ----------------------------------------------------------- planted mistakes

def _mutants():
    m = {}

    m["gqa_head_interleaved"] = {"kv_head_of": lambda hq, G: hq % 2}

    def gather_off_by_one(pool_bits, indptr, indices, b, L, P):
        pool = np.asarray(pool_bits)
        out = np.empty((L, pool.shape[1], pool.shape[3]))
        for t in range(L):
            page = int(indices[int(indptr[b]) + (t + 1) // P])
            out[t] = OA.bf16_to_f64(pool[page, :, (t + 1) % P, :])
        return out
    m["gather_shifted_token"] = {"gather_request": gather_off_by_one}

    def gather_swapped_page_offset(pool_bits, indptr, indices, b, L, P):
        pool = np.asarray(pool_bits)
        out = np.empty((L, pool.shape[1], pool.shape[3]))
        for t in range(L):
            page = int(indices[int(indptr[b]) + t % P])
            out[t] = OA.bf16_to_f64(pool[page, :, t // P, :])
        return out
    m["gather_swapped_page_offset"] = {"gather_request": gather_swapped_page_offset}

    def attend_no_scale(qv, Kd, Vd, sm_scale):
        return OA.__dict__["_orig_softmax_attend"](qv, Kd, Vd, 1.0)
    m["missing_sm_scale"] = {"softmax_attend": attend_no_scale}

    def attend_scores_from_v(qv, Kd, Vd, sm_scale):
        return OA.__dict__["_orig_softmax_attend"](qv, Vd, Vd, sm_scale)
    m["scores_use_v"] = {"softmax_attend": attend_scores_from_v}

    def attend_neg(qv, Kd, Vd, sm_scale):
        return OA.__dict__["_orig_softmax_attend"](qv, Kd, Vd, -sm_scale)
    m["score_sign_flipped"] = {"softmax_attend": attend_neg}

    def attend_drop_last(qv, Kd, Vd, sm_scale):
        n = max(1, Kd.shape[0] - 1) if Kd.shape[0] else 0
        return OA.__dict__["_orig_softmax_attend"](qv, Kd[:n], Vd[:n], sm_scale)
    m["drops_newest_token"] = {"softmax_attend": attend_drop_last}

    def merge_plain_mean(parts):
        live = [o for o, lse in parts if lse != -math.inf]
        return np.mean(live, axis=0) if live else np.zeros(parts[0][0].shape[0])
    m["merge_without_weights"] = {"merge_partials": merge_plain_mean}

    def partial_lse_missing_max(qv, Kd, Vd, sm_scale):
        o, lse = OA.__dict__["_orig_chunk_partial"](qv, Kd, Vd, sm_scale)
        if lse == -math.inf:
            return o, lse
        x = sm_scale * (Kd @ qv)
        return o, lse - float(np.max(x))
    m["lse_missing_max"] = {"chunk_partial": partial_lse_missing_max}

    def ranges_drop_last_page(n, k):
        r = [((s * n) // k, ((s + 1) * n) // k) for s in range(k)]
        r[-1] = (r[-1][0], max(r[-1][0], n - 1))
        return r
    m["ranges_drop_last_page"] = {"even_page_ranges": ranges_drop_last_page}

    # the grouping before groups of eight existed: four heads whenever G > 4
    m["head_groups_four_at_g8"] = {
        "head_groups": lambda Hq, Hkv: ((Hq // Hkv if Hq // Hkv <= 4 else 4),
                                        Hq // (Hq // Hkv if Hq // Hkv <= 4 else 4))}
    # the grouping before groups of twelve existed: four heads at G = 12
    m["head_groups_four_at_g12"] = {
        "head_groups": lambda Hq, Hkv: ((Hq // Hkv if Hq // Hkv <= 4 else
                                         (8 if (Hq // Hkv) % 8 == 0 else 4)),
                                        Hq // (Hq // Hkv if Hq // Hkv <= 4 else
                                               (8 if (Hq // Hkv) % 8 == 0 else 4)))}
    # the grouping before groups of five to seven existed: four heads at G = 6
    m["head_groups_four_at_g6"] = {
        "head_groups": lambda Hq, Hkv: ((Hq // Hkv if Hq // Hkv <= 4 else
                                         (12 if (Hq // Hkv) % 12 == 0 else
                                          (8 if (Hq // Hkv) % 8 == 0 else 4))),
                                        Hq // (Hq // Hkv if Hq // Hkv <= 4 else
                                               (12 if (Hq // Hkv) % 12 == 0 else
                                                (8 if (Hq // Hkv) % 8 == 0 else 4))))}
    # groups of eight for any G above four (splits a KV head's heads at G = 12)
    m["head_groups_eight_above_four"] = {
        "head_groups": lambda Hq, Hkv: ((Hq // Hkv if Hq // Hkv <= 4 else 8),
                                        Hq // (Hq // Hkv if Hq // Hkv <= 4 else 8))}

    def rows_reversed(k_pool, v_pool, k_rows, v_rows, qo, indptr, indices, seq_lens, P):
        k_r, v_r = np.array(k_rows), np.array(v_rows)
        for b in range(len(seq_lens)):
            k_r[qo[b]:qo[b + 1]] = k_r[qo[b]:qo[b + 1]][::-1]
            v_r[qo[b]:qo[b + 1]] = v_r[qo[b]:qo[b + 1]][::-1]
        return OA.__dict__["_orig_append_kv_rows"](k_pool, v_pool, k_r, v_r, qo, indptr, indices,
                                                    seq_lens, P)
    m["append_rows_reversed"] = {"append_kv_rows": rows_reversed}

    def rows_from_prefix_end(k_pool, v_pool, k_rows, v_rows, qo, indptr, indices, seq_lens, P):
        # a plausible slip: new tokens placed right after a prefix of seq_len - n - 1
        sl = np.maximum(np.asarray(seq_lens) - 1, 0)
        return OA.__dict__["_orig_append_kv_rows"](k_pool, v_pool, k_rows, v_rows, qo, indptr,
                                                    indices, sl, P)
    m["append_rows_one_early"] = {"append_kv_rows": rows_from_prefix_end}

    m["page_count_floor"] = {"page_counts": lambda L, P: np.asarray(L, np.int64) // P}

    def plan_group_bounds_ceil(seq_lens, P, units, groups, min_tiles, forced=0, waves_per_group=8):
        p = OA.__dict__["_orig_plan_stream"](seq_lens, P, units, groups, min_tiles, forced,
                                              waves_per_group)
        # a plausible slip: the last wave of every group starts one tile late
        for i in range(p["groups"]):
            r = p["waves"][i * waves_per_group + waves_per_group - 1]
            if r[3] > 1:
                b, u, pg = OA.tile_of(p["kv_indptr"], units,
                                      sum(int(x[3]) for x in p["waves"][:i * waves_per_group + 7]) + 1)
                r[:] = (b, u, pg, r[3] - 1)
        return p
    m["plan_wave_start_shifted"] = {"plan_stream": plan_group_bounds_ceil}

    def pieces_drop_first_page(q, k, v, ip, idx, sl, sc, P, pieces):
        pieces = [(b, u, p0 + (1 if n > 1 else 0), n - (1 if n > 1 else 0)) for b, u, p0, n in pieces]
        return OA.__dict__["_orig_decode_pieces"](q, k, v, ip, idx, sl, sc, P, pieces)
    m["pieces_skip_a_page"] = {"decode_pieces": pieces_drop_first_page}

    def append_at_len(k_pool, v_pool, k_new, v_new, indptr, indices, seq_lens, P):
        return OA.__dict__["_orig_append_kv"](k_pool, v_pool, k_new, v_new, indptr, indices,
                                              np.asarray(seq_lens) + 1, P)
    m["append_one_slot_late"] = {"append_kv": append_at_len}

    def masked_inverted(q, k, v, ip, idx, sl, sc, P, mask):
        return OA.__dict__["_orig_decode_masked"](q, k, v, ip, idx, sl, sc, P,
                                                  ~np.asarray(mask, bool))
    m["mask_inverted"] = {"decode_masked": masked_inverted}

    def masked_shifted(q, k, v, ip, idx, sl, sc, P, mask):
        return OA.__dict__["_orig_decode_masked"](q, k, v, ip, idx, sl, sc, P,
                                                  np.roll(np.asarray(mask, bool), 1, axis=1))
    m["mask_shifted_one_token"] = {"decode_masked": masked_shifted}

    def prefill_causal_top_left(q, k, v, ip, idx, sl, qo, sc, P, causal):
        # a plausible slip: the causal mask aligned to the start of the keys
        out = OA.__dict__["_orig_prefill"](q, k, v, ip, idx, sl, qo, sc, P, False)
        if not causal:
            return out
        for b in range(len(qo) - 1):
            n = int(qo[b + 1]) - int(qo[b])
            sl_b = np.zeros_like(np.asarray(sl))
            for i in range(n):
                sl_b[:] = 0
                sl_b[b] = min(i + 1, int(sl[b]))
                qi = np.repeat(np.asarray(q)[int(qo[b]) + i][None], len(sl), axis=0)
                out[int(qo[b]) + i] = OA.decode(qi, k, v, ip, idx, sl_b, sc, P)[b]
        return out
    m["prefill_causal_top_left"] = {"prefill": prefill_causal_top_left}

    def prefill_causal_one_short(q, k, v, ip, idx, sl, qo, sc, P, causal):
        out = OA.__dict__["_orig_prefill"](q, k, v, ip, idx, sl, qo, sc, P, causal)
        if causal:
            # each row loses its own key
            for b in range(len(qo) - 1):
                n = int(qo[b + 1]) - int(qo[b])
                L = int(sl[b])
                for i in range(n):
                    sl_b = np.zeros_like(np.asarray(sl))
                    sl_b[b] = max(0, L - n + i)
                    qi = np.repeat(np.asarray(q)[int(qo[b]) + i][None], len(sl), axis=0)
                    out[int(qo[b]) + i] = OA.decode(qi, k, v, ip, idx, sl_b, sc, P)[b]
        return out
    m["prefill_causal_one_short"] = {"prefill": prefill_causal_one_short}

    def tokens_next_slot(q, k, v, sl, sc, table=None, stride=0):
        # a slip in the table walk: every token read from the slot after its own
        if table is None:
            return OA.__dict__["_orig_decode_tokens"](q, k[1:], v[1:], sl, sc, None, stride)
        return OA.__dict__["_orig_decode_tokens"](q, k, v, sl, sc,
                                                  np.where(np.asarray(table) >= 0,
                                                           (np.asarray(table) + 1) % len(k), -1),
                                                  stride)
    m["tokens_next_slot"] = {"decode_tokens": tokens_next_slot}

    def tokens_packed_rows(q, k, v, sl, sc, table=None, stride=0):
        # contiguous rows read back to back, ignoring the row stride
        if table is not None:
            return OA.__dict__["_orig_decode_tokens"](q, k, v, sl, sc, table, stride)
        starts = np.concatenate([[0], np.cumsum(np.asarray(sl, np.int64))[:-1]])
        packed = np.full((len(sl), max(1, stride)), -1, np.int64)
        for b in range(len(sl)):
            packed[b, : int(sl[b])] = starts[b] + np.arange(int(sl[b]))
        return OA.__dict__["_orig_decode_tokens"](q, k, v, sl, sc, packed, 0)
    m["tokens_packed_rows"] = {"decode_tokens": tokens_packed_rows}
    return m


MUTANTS = _mutants()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes(name, monkeypatch):
    for fn in ("softmax_attend", "chunk_partial", "plan_stream", "decode_pieces", "append_kv",
               "append_kv_rows",
               "decode_masked", "prefill", "decode_tokens"):
        monkeypatch.setitem(OA.__dict__, "_orig_" + fn, getattr(OA, fn))
    for attr, repl in MUTANTS[name].items():
        monkeypatch.setattr(OA, attr, repl)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(OA)
        except (AssertionError, IndexError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name!r} passed every pin"
