"""Pins for the fp64 CPU oracle: checks against what the pages and the
mathematics fix, never against the oracle itself.

Each group targets a plausible mistake:
  * ownership: rank formula from the pages' worked table, the N x I period
  * local lengths / slots: the pages' token-count examples, partition and
    balance invariants, -1 on non-owners, injectivity, order preservation,
    virtual-block filling
  * head-tail split: the pages' PCP2/PCP3/PCP4/PCP8 examples and the closed-form
    causal work per rank
  * element decoding: torch's own bf16 / float8_e4m3fn conversions and the OCP
    format's special values
  * attention: torch's fp64 scaled_dot_product_attention and logsumexp (library
    routines), closed forms (q = 0, V = 1, one dominant key, empty set)
  * merge: merge of shard partials == unsharded attention (the pages' exactness
    claim), N = 1 identity, associativity, -inf parts
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


# ---------------------------------------------------------------------------
# ownership
# ---------------------------------------------------------------------------

def test_owner_matches_printed_table():
    # Breaking the Long-Sequence Inference Bottleneck ..., section 2 table + D20/D27
    for first, last, rank in _rows("interleave_table.txt"):
        for t in range(int(first), int(last) + 1):
            assert oracle.owner(t, 4, 4) == int(rank), t


@pytest.mark.parametrize("N,I", [(1, 1), (2, 1), (4, 4), (8, 16), (3, 5), (8, 1), (5, 64)])
def test_owner_period_is_N_times_I(N, I):
    # vLLM DCP and PCP ..., TL;DR: ownership repeats every N x I tokens
    for t in range(0, 3 * N * I + 7):
        assert oracle.owner(t + N * I, N, I) == oracle.owner(t, N, I)
    # and within one period every rank owns exactly I consecutive positions
    counts = np.bincount([oracle.owner(t, N, I) for t in range(N * I)], minlength=N)
    assert (counts == I).all()


# ---------------------------------------------------------------------------
# local lengths
# ---------------------------------------------------------------------------

def test_local_lens_printed_examples():
    for name, L, N, I, *expect in _rows("capacity_examples.txt"):
        got = [int(oracle.local_lens([int(L)], r, int(N), int(I))[0]) for r in range(int(N))]
        assert got == [int(x) for x in expect], name


def test_local_lens_tiny_gqa_config():
    # 1,000 tokens, 4 shards, interleave 4: 62 full rounds of 16 tokens (248 each),
    # then 8 tokens: 4 to rank 0, 4 to rank 1
    got = [int(oracle.local_lens([1000], r, 4, 4)[0]) for r in range(4)]
    assert got == [252, 252, 248, 248]


@pytest.mark.parametrize("N,I", [(2, 1), (4, 2), (8, 16), (3, 7), (8, 1)])
def test_local_lens_partition_and_balance(N, I):
    # vLLM DCP and PCP ..., Deep Dive 5: lengths differ by at most one interleave group
    rng = np.random.default_rng(N * 100 + I)
    seq = rng.integers(0, 500, size=40).astype(np.int32)
    lens = np.stack([oracle.local_lens(seq, r, N, I) for r in range(N)])
    assert (lens.sum(axis=0) == seq).all()
    assert (lens.max(axis=0) - lens.min(axis=0) <= I).all()
    # ranks earlier in the round never hold fewer tokens than later ones
    assert (np.diff(lens, axis=0) <= 0).all()


# ---------------------------------------------------------------------------
# slot mapping
# ---------------------------------------------------------------------------

def _tables(seq, N, I, bs, rng, pool_factor=2):
    """Random-permutation block tables per rank, sized from the local lengths."""
    tabs = []
    for r in range(N):
        need = (oracle.local_lens(seq, r, N, I) + bs - 1) // bs
        width = max(int(need.max()), 1)
        pool = max(int(need.sum()) * pool_factor, 1)
        perm = rng.permutation(pool).astype(np.int32)
        bt = np.full((len(seq), width), -1, dtype=np.int32)
        off = 0
        for b, n in enumerate(need):
            bt[b, :n] = perm[off:off + n]
            off += n
        tabs.append((bt, need))
    return tabs


@pytest.mark.parametrize("N,I,bs", [(4, 4, 16), (8, 16, 16), (8, 1, 64), (3, 5, 4), (4, 2, 3)])
def test_slot_map_invariants(N, I, bs):
    rng = np.random.default_rng(7 + N + I + bs)
    seq = rng.integers(1, 300, size=6).astype(np.int32)
    req = np.concatenate([np.full(L, b) for b, L in enumerate(seq)]).astype(np.int32)
    pos = np.concatenate([np.arange(L) for L in seq]).astype(np.int32)
    perm = rng.permutation(len(req))  # token order must not matter
    req, pos = req[perm], pos[perm]
    tabs = _tables(seq, N, I, bs, rng)
    owned_total = 0
    for r, (bt, need) in enumerate(tabs):
        slots = oracle.slot_map(req, pos, bt, r, N, I, bs)
        own = np.array([oracle.owner(int(t), N, I) == r for t in pos])
        # -1 exactly on positions another rank owns (section 2, slot mapping diagram)
        assert ((slots == -1) == ~own).all()
        s = slots[own]
        owned_total += own.sum()
        assert len(np.unique(s)) == len(s)          # injective on this rank
        for b in range(len(seq)):
            m = own & (req == b)
            sb, pb = slots[m], pos[m]
            order = np.argsort(pb)
            sb = sb[order]
            # every slot lies in one of the request's listed blocks
            blocks = list(bt[b, :need[b]])
            idx = np.array([blocks.index(x // bs) for x in sb], dtype=np.int64)
            local = idx * bs + sb % bs
            # local indices are 0..len-1 in position order
            assert (local == np.arange(len(sb))).all()
    assert owned_total == len(pos)                  # each token stored exactly once


def test_virtual_block_fills_one_physical_block_per_rank():
    # Breaking ..., section 2 "Virtual Block"; vLLM DCP and PCP ..., Deep Dive 5:
    # a virtual block of block_size x N positions fills exactly one physical block
    # per rank when the interleave divides the block size.
    N, I, bs = 4, 4, 16
    L = 5 * bs * N
    rng = np.random.default_rng(3)
    (tabs) = _tables(np.array([L], dtype=np.int32), N, I, bs, rng)
    pos = np.arange(L, dtype=np.int32)
    req = np.zeros(L, dtype=np.int32)
    for r, (bt, need) in enumerate(tabs):
        slots = oracle.slot_map(req, pos, bt, r, N, I, bs)
        for vb in range(5):
            s = slots[vb * bs * N:(vb + 1) * bs * N]
            s = s[s >= 0]
            assert len(s) == bs
            assert set(s // bs) == {bt[0, vb]}


def test_slot_map_past_table_is_minus_two():
    bt = np.array([[5, 9]], dtype=np.int32)
    pos = np.arange(0, 80, dtype=np.int32)
    req = np.zeros_like(pos)
    s = oracle.slot_map(req, pos, bt, 0, 2, 4, 8)  # rank 0 owns 40 of 80 -> needs 5 blocks
    owned = s[s != -1]
    assert (owned[:16] >= 0).all() and (owned[16:] == -2).all()


# ---------------------------------------------------------------------------
# PCP head-tail split
# ---------------------------------------------------------------------------

def test_pcp_pieces_printed_examples():
    for N, r, a, b in _rows("pcp_pieces.txt"):
        assert oracle.pcp_pieces(int(N), int(r)) == (int(a), int(b))


def test_pcp2_token_lists():
    for rank, *toks in _rows("pcp2_tokens.txt"):
        got = oracle.pcp_rank_positions(8, 2, int(rank)).tolist()
        assert got == [int(t) for t in toks]


def test_pcp8_uses_sixteen_pieces_and_covers_everything():
    # GLM-5.3 page: PCP8 divides the prompt into 16 chunks, early paired with late
    C, N = 32768, 8
    allpos = np.concatenate([oracle.pcp_rank_positions(C, N, r) for r in range(N)])
    assert sorted(allpos.tolist()) == list(range(C))
    assert {oracle.pcp_pieces(N, r) for r in range(N)} == {(r, 15 - r) for r in range(8)}
    with pytest.raises(AssertionError):
        oracle.pcp_rank_positions(C + 8, N, 0)   # not aligned to 2N


@pytest.mark.parametrize("C,N", [(8, 2), (48, 3), (64, 4), (256, 8)])
def test_pcp_balance_closed_form(C, N):
    # causal pairs of a query at chunk index i: i + 1 keys (itself and everything before)
    c = C // (2 * N)
    closed = c * c * (2 * N - 1) + c * (c + 1)
    for r in range(N):
        pairs = int(sum(int(p) + 1 for p in oracle.pcp_rank_positions(C, N, r)))
        assert pairs == closed
    assert N * closed == C * (C + 1) // 2


def test_pcp_balance_at_full_prefill_size_and_contiguous_skew():
    C, N = 32768, 8
    c = C // (2 * N)
    per_rank = [int((oracle.pcp_rank_positions(C, N, r) + 1).sum()) for r in range(N)]
    assert per_rank == [67_110_912] * N
    # a contiguous 8-way split instead: the last rank does ~15x the first one's work
    w = C // N
    contig = [sum(range(r * w + 1, (r + 1) * w + 1)) for r in range(N)]
    assert abs(contig[-1] / contig[0] - 15.0) < 0.01


# ---------------------------------------------------------------------------
# element decoding
# ---------------------------------------------------------------------------

def test_decode_e4m3fn_matches_torch_and_format():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    m = ~np.isnan(ref)
    assert np.array_equal(ours[m], ref[m])
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])
    # every finite e4m3fn value is exactly representable in bf16
    bf = torch.from_numpy(ours[m]).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf, ours[m])


def test_decode_bf16_matches_torch():
    rng = np.random.default_rng(0)
    codes = np.concatenate([rng.integers(0, 65536, 4000), [0, 0x8000, 0x3F80, 0x7F80, 0xFF80]])
    codes = codes.astype(np.uint16)
    ours = oracle.decode_bf16(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def _sdpa(q, k, v, scale, mask=None):
    """torch fp64 SDPA + logsumexp: q [Hq, n_q, D], k/v [Hkv, n_k, D] (GQA by
    repeating kv heads in contiguous groups)."""
    rep = q.shape[0] // k.shape[0]
    k = k.repeat_interleave(rep, dim=0)
    v = v.repeat_interleave(rep, dim=0)
    out = F.scaled_dot_product_attention(q[None], k[None], v[None], attn_mask=mask, scale=scale)[0]
    s = (q @ k.transpose(-1, -2)) * scale
    if mask is not None:
        s = s.masked_fill(~mask, float("-inf"))
    return out, torch.logsumexp(s, dim=-1)


@pytest.mark.parametrize("Hq,Hkv,Dk,Dv,nk", [(8, 2, 16, 16, 37), (4, 4, 8, 8, 5),
                                              (6, 1, 24, 16, 50), (8, 1, 9, 5, 3)])
def test_attention_matches_torch_sdpa(Hq, Hkv, Dk, Dv, nk):
    rng = np.random.default_rng(Hq * 10 + nk)
    q = rng.standard_normal((1, Hq, Dk)).astype(np.float32)
    k = rng.standard_normal((nk, Hkv, Dk)).astype(np.float32)
    v = rng.standard_normal((nk, Hkv, Dv)).astype(np.float32)
    scale = 1.0 / math.sqrt(Dk)
    out, lse = oracle.attention(q, k, v, key_begin=0, key_end=nk, scale=scale,
                                q_dtype="f32", kv_dtype="f32")
    tq = torch.from_numpy(q).double().permute(1, 0, 2)
    tk = torch.from_numpy(k).double().permute(1, 0, 2)
    tv = torch.from_numpy(v).double().permute(1, 0, 2)
    ro, rl = _sdpa(tq, tk, tv, scale)
    np.testing.assert_allclose(out[0], ro[:, 0].numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse[0], rl[:, 0].numpy(), rtol=1e-12, atol=1e-13)


def test_attention_mla_layout_latent_as_k_and_v():
    # absorbed MLA: one shared latent row serves as the key (all columns) and the
    # value (leading columns) for every query head
    rng = np.random.default_rng(11)
    H, Dk, Dv, n = 16, 40, 32, 29
    q = rng.standard_normal((1, H, Dk)).astype(np.float32)
    c = rng.standard_normal((n, 1, Dk)).astype(np.float32)
    out, lse = oracle.attention(q, c, c, key_begin=0, key_end=n, Dv=Dv, scale=0.2,
                                q_dtype="f32", kv_dtype="f32")
    tq = torch.from_numpy(q).double().permute(1, 0, 2)
    tc = torch.from_numpy(c).double().permute(1, 0, 2)
    ro, rl = _sdpa(tq, tc, tc[..., :Dv].contiguous(), 0.2)
    np.testing.assert_allclose(out[0], ro[:, 0].numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse[0], rl[:, 0].numpy(), rtol=1e-12, atol=1e-13)


def test_attention_causal_rows_match_masked_sdpa():
    # prefill rows: query i of a chunk starting at position P sees keys [0, P + i]
    rng = np.random.default_rng(5)
    P, C, H, D = 13, 11, 4, 8
    q = rng.standard_normal((C, H, D)).astype(np.float32)
    k = rng.standard_normal((P + C, 2, D)).astype(np.float32)
    v = rng.standard_normal((P + C, 2, D)).astype(np.float32)
    ends = P + np.arange(C) + 1
    out, lse = oracle.attention(q, k, v, key_begin=0, key_end=ends, scale=0.3,
                                q_dtype="f32", kv_dtype="f32")
    mask = torch.arange(P + C)[None, :] < torch.from_numpy(ends)[:, None]
    ro, rl = _sdpa(torch.from_numpy(q).double().permute(1, 0, 2),
                   torch.from_numpy(k).double().permute(1, 0, 2),
                   torch.from_numpy(v).double().permute(1, 0, 2), 0.3, mask)
    np.testing.assert_allclose(out, ro.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, rl.permute(1, 0).numpy(), rtol=1e-12, atol=1e-13)


def test_attention_shard_filter_equals_sdpa_on_owned_keys():
    rng = np.random.default_rng(9)
    n, N, I = 61, 4, 3
    q = rng.standard_normal((1, 4, 8)).astype(np.float32)
    k = rng.standard_normal((n, 2, 8)).astype(np.float32)
    v = rng.standard_normal((n, 2, 8)).astype(np.float32)
    for r in range(N):
        own = np.array([oracle.owner(t, N, I) == r for t in range(n)])
        out, lse = oracle.attention(q, k, v, key_begin=0, key_end=n, scale=0.5,
                                    q_dtype="f32", kv_dtype="f32", shard=(N, I, r))
        ro, rl = _sdpa(torch.from_numpy(q).double().permute(1, 0, 2),
                       torch.from_numpy(k[own]).double().permute(1, 0, 2),
                       torch.from_numpy(v[own]).double().permute(1, 0, 2), 0.5)
        np.testing.assert_allclose(out[0], ro[:, 0].numpy(), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[0], rl[:, 0].numpy(), rtol=1e-12, atol=1e-13)


def test_attention_closed_forms():
    rng = np.random.default_rng(1)
    n, D = 23, 8
    k = rng.standard_normal((n, 1, D)).astype(np.float32)
    v = rng.standard_normal((n, 1, D)).astype(np.float32)
    # q = 0: uniform weights -> mean of the values, LSE = ln n
    q0 = np.zeros((1, 2, D), dtype=np.float32)
    out, lse = oracle.attention(q0, k, v, key_begin=0, key_end=n, scale=1.0,
                                q_dtype="f32", kv_dtype="f32")
    np.testing.assert_allclose(out[0, 0], v[:, 0].astype(np.float64).mean(0), rtol=1e-12)
    assert abs(lse[0, 0] - math.log(n)) < 1e-12
    # all values one: weights sum to one -> output exactly ~1
    q = rng.standard_normal((1, 2, D)).astype(np.float32)
    ones = np.ones((n, 1, D), dtype=np.float32)
    out, _ = oracle.attention(q, k, ones, key_begin=0, key_end=n, scale=0.7,
                              q_dtype="f32", kv_dtype="f32")
    np.testing.assert_allclose(out, 1.0, rtol=1e-13)
    # one dominant key: output -> its value row
    kd = np.zeros_like(k)
    kd[7, 0, 0] = 1.0
    qd = np.zeros((1, 1, D), dtype=np.float32)
    qd[0, 0, 0] = 1.0
    out, lse = oracle.attention(qd, kd, v, key_begin=0, key_end=n, scale=200.0,
                                q_dtype="f32", kv_dtype="f32")
    np.testing.assert_allclose(out[0, 0], v[7, 0], rtol=1e-12, atol=1e-12)
    assert abs(lse[0, 0] - 200.0) < 1e-12
    # empty key set
    out, lse = oracle.attention(q, k, v, key_begin=5, key_end=5, scale=1.0,
                                q_dtype="f32", kv_dtype="f32")
    assert (out == 0).all() and np.isneginf(lse).all()


def test_attention_decodes_bf16_and_fp8_inputs():
    rng = np.random.default_rng(2)
    n, H, D = 19, 4, 16
    qf = torch.from_numpy(rng.standard_normal((1, H, D)).astype(np.float32)).to(torch.bfloat16)
    kf = torch.from_numpy(rng.standard_normal((n, 1, D)).astype(np.float32))
    scale_kv = float(kf.abs().max()) / 448.0
    k8 = (kf / scale_kv).clamp(-448, 448).to(torch.float8_e4m3fn)
    qbits = qf.view(torch.int16).numpy().view(np.uint16)
    kbits = k8.view(torch.uint8).numpy()
    out, lse = oracle.attention(qbits, kbits, kbits, key_begin=0, key_end=n, Dv=10, scale=0.25,
                                q_dtype="bf16", kv_dtype="fp8_e4m3fn", kv_scale=scale_kv)
    tq = qf.double().permute(1, 0, 2)
    tk = (k8.double() * scale_kv).permute(1, 0, 2)
    ro, rl = _sdpa(tq, tk, tk[..., :10].contiguous(), 0.25)
    np.testing.assert_allclose(out[0], ro[:, 0].numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse[0], rl[:, 0].numpy(), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# merge
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,I", [(4, 4), (8, 16), (3, 1), (5, 7)])
def test_merge_of_shard_partials_is_unsharded_attention(N, I):
    # vLLM DCP and PCP ..., Deep Dive 6: the shards partition the context, so the
    # merged result is the exact logical global output
    rng = np.random.default_rng(N + I)
    n, Hq, Hkv, D = 150, 8, 2, 16
    q = rng.standard_normal((1, Hq, D)).astype(np.float32)
    k = (3 * rng.standard_normal((n, Hkv, D))).astype(np.float32)
    v = rng.standard_normal((n, Hkv, D)).astype(np.float32)
    full_o, full_l = oracle.attention(q, k, v, key_begin=0, key_end=n, scale=0.25,
                                      q_dtype="f32", kv_dtype="f32")
    parts = [oracle.attention(q, k, v, key_begin=0, key_end=n, scale=0.25, q_dtype="f32",
                              kv_dtype="f32", shard=(N, I, r)) for r in range(N)]
    po = np.stack([p[0].reshape(Hq, D) for p in parts])
    pl = np.stack([p[1].reshape(Hq) for p in parts])
    mo, ml = oracle.lse_merge(po, pl)
    np.testing.assert_allclose(mo, full_o.reshape(Hq, D), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ml, full_l.reshape(Hq), rtol=1e-12)
    # summing normalised partial outputs would be wrong (a sanity check that the
    # identity above is not trivially satisfied)
    assert np.abs(po.sum(0) - full_o.reshape(Hq, D)).max() > 1e-3


def test_merge_identity_associativity_and_empty_parts():
    rng = np.random.default_rng(4)
    n, rows, Dv = 6, 10, 5
    po = rng.standard_normal((n, rows, Dv))
    pl = 10 * rng.standard_normal((n, rows))
    one_o, one_l = oracle.lse_merge(po[:1], pl[:1])
    np.testing.assert_array_equal(one_o, po[0])
    np.testing.assert_array_equal(one_l, pl[0])
    flat_o, flat_l = oracle.lse_merge(po, pl)
    a_o, a_l = oracle.lse_merge(po[:2], pl[:2])
    b_o, b_l = oracle.lse_merge(po[2:], pl[2:])
    two_o, two_l = oracle.lse_merge(np.stack([a_o, b_o]), np.stack([a_l, b_l]))
    np.testing.assert_allclose(two_o, flat_o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(two_l, flat_l, rtol=1e-12)
    # an empty part (-inf) contributes nothing, even if its output holds garbage
    pl2 = pl.copy()
    po2 = po.copy()
    pl2[3] = -np.inf
    po2[3] = np.nan
    m_o, m_l = oracle.lse_merge(po2, pl2)
    keep = [0, 1, 2, 4, 5]
    r_o, r_l = oracle.lse_merge(po[keep], pl[keep])
    np.testing.assert_allclose(m_o, r_o, rtol=1e-12)
    np.testing.assert_allclose(m_l, r_l, rtol=1e-12)
    # all parts empty -> zero output, -inf LSE (never NaN)
    z_o, z_l = oracle.lse_merge(po2[3:4], pl2[3:4])
    assert (z_o == 0).all() and np.isneginf(z_l).all()
    # large LSE spread: stays finite
    pl3 = np.array([[1000.0], [-1000.0]])
    po3 = np.array([[[1.0]], [[2.0]]])
    o3, l3 = oracle.lse_merge(po3, pl3)
    assert o3[0, 0] == 1.0 and l3[0] == 1000.0


# ---------------------------------------------------------------------------
# KV gather ([P1] section 3 "MLA path"): the inverse of the placement
# ---------------------------------------------------------------------------

def _scatter_shards(L, N, I, bs, row_shape, dtype, rng, poison):
    """Seeded logical KV per request, written into N shard pools (random block
    permutations, unused blocks and slots poisoned) through oracle.slot_map."""
    B = len(L)
    hi = 255 if dtype == np.uint8 else 65535
    kv = [rng.integers(0, hi, size=(int(l),) + row_shape, dtype=dtype) for l in L]
    caches, bts = [], []
    for r in range(N):
        ll = oracle.local_lens(np.asarray(L), r, N, I)
        need = (ll + bs - 1) // bs
        stride = int(need.max()) + 2
        nblk = int(need.sum()) + 3
        perm = rng.permutation(nblk)
        bt = np.full((B, stride), -7, dtype=np.int32)
        k = 0
        for b in range(B):
            for j in range(need[b]):
                bt[b, j] = perm[k]
                k += 1
        Hkv = row_shape[0] if len(row_shape) == 2 else 1
        D = row_shape[-1]
        cache = np.full((nblk, Hkv, bs, D), poison, dtype=dtype)
        for b in range(B):
            pos = np.arange(L[b], dtype=np.int32)
            sl = oracle.slot_map(np.full(L[b], b, dtype=np.int32), pos, bt, r, N, I, bs)
            for t in np.nonzero(sl >= 0)[0]:
                cache[sl[t] // bs, :, sl[t] % bs, :] = kv[b][t].reshape(Hkv, D)
        caches.append(cache if len(row_shape) == 2 else cache[:, 0])  # latent: [nblk][bs][D]
        bts.append(bt)
    return kv, caches, bts


@pytest.mark.parametrize("N,I,bs,row_shape,dtype", [
    (4, 4, 16, (2, 8), np.uint16),      # the pages' I=4, N=4 ownership table
    (3, 5, 16, (2, 8), np.uint16),      # I does not divide bs
    (8, 16, 16, (4, 4), np.uint16),     # one virtual block fills one physical block per rank
    (2, 1, 64, (12,), np.uint8),        # latent rows (Hkv = 1, [nblk][bs][D] cache), fp8 bytes
    (5, 32, 16, (1, 8), np.uint16),     # I > bs
])
def test_kv_gather_inverts_the_placement(N, I, bs, row_shape, dtype):
    rng = np.random.default_rng(11 + N + I + bs)
    L = [200, 37, 0, 130, 1]
    kv, caches, bts = _scatter_shards(L, N, I, bs, row_shape, dtype, rng, poison=0xFE)
    full = oracle.kv_gather(caches, bts, L, N, I, bs, 0, 200)
    for b, l in enumerate(L):
        assert np.array_equal(full[b, :l].reshape((l,) + row_shape), kv[b]), b
        assert (full[b, l:] == 0).all()          # past the request's end: zero rows
    # a window straddling the ends
    win = oracle.kv_gather(caches, bts, L, N, I, bs, 33, 100)
    for b, l in enumerate(L):
        n = max(0, min(100, l - 33))
        assert np.array_equal(win[b, :n].reshape((n,) + row_shape), kv[b][33:33 + n])
        assert (win[b, n:] == 0).all()
    # a planted mistake: reading with the wrong interleave size must not pass
    wrong = oracle.kv_gather(caches, bts, L, N, I + 1, bs, 0, 200)
    assert not np.array_equal(wrong, full)


def test_kv_gather_marks_bad_block_ids():
    rng = np.random.default_rng(5)
    N, I, bs = 2, 4, 16
    L = [100]
    kv, caches, bts = _scatter_shards(L, N, I, bs, (2, 8), np.uint16, rng, poison=0)
    bts[1][0, 1] = 10 ** 6                # rank 1's local block 1: out of the pool
    g = oracle.kv_gather(caches, bts, L, N, I, bs, 0, 100)
    # rank 1 owns t with floor(t/4) odd, at local index floor(t/8)*4 + t%4; its
    # local indices 16..31 (block 1) are positions 36..39, 44..47, 52..55, 60..63
    bad = [t for t in range(100) if (t // I) % N == 1 and 16 <= (t // 8) * 4 + t % 4 < 32]
    assert bad == [36, 37, 38, 39, 44, 45, 46, 47, 52, 53, 54, 55, 60, 61, 62, 63]
    for t in range(100):
        if t in bad:
            assert (g[0, t] == 0xFFFF).all()
        else:
            assert np.array_equal(g[0, t], kv[0][t])


@pytest.mark.parametrize("N,I", [(3, 5), (4, 64), (2, 1)])
def test_merge_of_causal_shard_partials_is_causal_attention(N, I):
    """DCP-sharded causal prefill ([P1] section 5, "AllGather Q path" with the
    chunk's KV interleaved like the prefix's): each shard's partial over its
    own keys at positions <= the query's, merged exactly, is the causal
    attention over prefix and chunk -- including rows for which a shard owns
    no visible key (empty partial, LSE -inf)."""
    rng = np.random.default_rng(900 + N + I)
    P, C, H, D = 37, 48, 2, 8
    q = rng.standard_normal((C, H, D)).astype(np.float32)
    k = rng.standard_normal((P + C, H, D)).astype(np.float32)
    v = rng.standard_normal((P + C, H, D)).astype(np.float32)
    rows = np.arange(C)
    ends = P + rows + 1
    po, pl = [], []
    for s in range(N):
        o, l = oracle.attention(q, k, v, key_begin=0, key_end=ends, scale=0.3, q_dtype="f32",
                                kv_dtype="f32", shard=(N, I, s))
        po.append(o)
        pl.append(l)
    if I == 64:
        assert np.isneginf(pl[1][0]).all()   # shard 1 owns no position below P + 1 = 38
    mo, ml = oracle.lse_merge(np.stack(po).reshape(N, C * H, D), np.stack(pl).reshape(N, C * H))
    ro, rl = oracle.attention(q, k, v, key_begin=0, key_end=ends, scale=0.3, q_dtype="f32",
                              kv_dtype="f32")
    ro, rl = ro.reshape(C * H, D), rl.reshape(C * H)
    assert np.allclose(mo, ro, rtol=1e-12, atol=1e-12)
    assert np.allclose(ml, rl, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Head-scattered exchanges ([P3] Deep Dive 6: AG+RS, and the all-to-all path)
# ---------------------------------------------------------------------------

def _shard_partials(rng, n, B, Hq, Hkv, D, N, I, scale):
    """Every DCP shard's partial over its own keys, and torch fp64 SDPA over all
    keys: B query rows (one per decode request, sharing one context here)."""
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    k = (3 * rng.standard_normal((n, Hkv, D))).astype(np.float32)
    v = rng.standard_normal((n, Hkv, D)).astype(np.float32)
    parts = [oracle.attention(q, k, v, key_begin=0, key_end=n, scale=scale, q_dtype="f32",
                              kv_dtype="f32", shard=(N, I, r)) for r in range(N)]
    tq = torch.from_numpy(q).double().permute(1, 0, 2)
    tk = torch.from_numpy(k).double().permute(1, 0, 2)
    tv = torch.from_numpy(v).double().permute(1, 0, 2)
    ro, rl = _sdpa(tq, tk, tv, scale)
    return parts, ro.permute(1, 0, 2).numpy(), rl.permute(1, 0).numpy()


@pytest.mark.parametrize("N,I,n", [(4, 4, 150), (8, 16, 300), (4, 4, 5), (3, 1, 2)])
def test_ag_rs_corrected_partials_sum_to_unsharded_attention(N, I, n):
    """AG+RS: after the LSE all-gather each rank scales its own output by
    exp(L_i - L); adding the N corrected outputs (what the reduce-scatter does,
    head slice by head slice) gives exact attention over all keys.  With n = 5
    (N = 4, I = 4) or n = 2 (N = 3) some shards own no key: LSE -inf, factor 0."""
    rng = np.random.default_rng(1200 + N + n)
    B, Hq, Hkv, D = 3, 8, 2, 16
    parts, ro, rl = _shard_partials(rng, n, B, Hq, Hkv, D, N, I, 0.25)
    pl = np.stack([p[1].reshape(B * Hq) for p in parts])
    if n < N * I:
        assert np.isneginf(pl[-1]).all()
    total = np.zeros((B * Hq, D))
    for r in range(N):
        po_r = parts[r][0].reshape(B * Hq, D).copy()
        if np.isneginf(pl[r]).all():
            po_r[:] = np.nan     # an empty partial's output is never read
        c, L = oracle.lse_correct(po_r, pl, r)
        np.testing.assert_allclose(L, rl.reshape(-1), rtol=1e-12)
        total += c
    np.testing.assert_allclose(total, ro.reshape(B * Hq, D), rtol=1e-11, atol=1e-13)
    # rank 0 alone is not the answer (the factors matter)
    assert np.abs(parts[0][0].reshape(B * Hq, D) - ro.reshape(B * Hq, D)).max() > 1e-3


def test_ag_rs_correction_special_rows():
    pl = np.array([[0.0, -np.inf, np.log(3.0)], [np.log(3.0), -np.inf, -np.inf]])
    po = np.array([[2.0, 4.0], [5.0, 6.0], [1.0, -1.0]])
    c, L = oracle.lse_correct(po, pl, 0)
    # row 0: L = log(1 + 3), factor 1/4; row 1: every part empty; row 2: the
    # other part is empty, factor 1
    np.testing.assert_allclose(L, [np.log(4.0), -np.inf, np.log(3.0)])
    np.testing.assert_allclose(c, [[0.5, 1.0], [0.0, 0.0], [1.0, -1.0]])


@pytest.mark.parametrize("N,Hq,Hkv", [(4, 8, 2), (2, 8, 8), (8, 16, 1)])
def test_a2a_pack_exchange_merge_gives_head_slices(N, Hq, Hkv):
    """All-to-all path: every rank packs its partial (outputs + fp32 LSE per
    row) by destination head partition; after the exchange rank d merges the N
    packed parts it received into heads d*H/N .. (d+1)*H/N - 1 of the exact
    attention over all keys."""
    rng = np.random.default_rng(1300 + N + Hq)
    B, D, n = 3, 16, 90
    parts, ro, rl = _shard_partials(rng, n, B, Hq, Hkv, D, N, 4, 0.25)
    send = np.stack([oracle.a2a_pack(p[0].reshape(B, Hq, D), p[1].reshape(B, Hq), N)
                     for p in parts])
    hs = Hq // N
    assert send.shape == (N, N, B, hs, D + 4) and send.dtype == np.float32
    # layout: part s's slot d holds heads d*hs.., LSE in float32, three zeros
    s, d = N - 1, N // 2
    np.testing.assert_array_equal(send[s, d, :, :, :D],
                                  parts[s][0].reshape(B, Hq, D)[:, d * hs:(d + 1) * hs]
                                  .astype(np.float32))
    np.testing.assert_array_equal(send[s, d, :, :, D],
                                  parts[s][1].reshape(B, Hq)[:, d * hs:(d + 1) * hs]
                                  .astype(np.float32))
    assert (send[..., D + 1:] == 0).all()
    recv = oracle.all_to_all(send)
    assert np.array_equal(recv[d, s], send[s, d])
    got = np.concatenate([oracle.lse_merge_packed(recv[d], D)[0] for d in range(N)], axis=1)
    # float32 partials and LSEs on the wire: agreement to float32 rounding
    np.testing.assert_allclose(got, ro, rtol=2e-5, atol=2e-6)
    lse = np.concatenate([oracle.lse_merge_packed(recv[d], D)[1] for d in range(N)], axis=1)
    np.testing.assert_allclose(lse, rl, rtol=1e-6, atol=1e-6)


# ---------------------------------------------------------------------------
# multi-token decode queries (speculative decoding / MTP)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,L,Hq,Hkv", [(2, 37, 8, 2), (4, 20, 4, 4), (3, 3, 2, 1), (1, 15, 4, 2)])
def test_decode_mtp_is_the_last_rows_of_causal_sdpa(T, L, Hq, Hkv):
    """Token t of the last T positions sees positions <= L - T + t: the last T
    rows of torch's fp64 causal attention over the whole sequence."""
    rng = np.random.default_rng(100 * T + L)
    D = 8
    q = rng.standard_normal((T, Hq, D)).astype(np.float32)
    k = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    out, lse = oracle.decode_mtp(q, k, v, L=L, scale=0.4, q_dtype="f32", kv_dtype="f32")
    # full causal attention of L queries, of which the last T are ours
    qa = np.concatenate([rng.standard_normal((L - T, Hq, D)).astype(np.float32), q])
    mask = torch.tril(torch.ones(L, L, dtype=torch.bool))
    ro, rl = _sdpa(torch.from_numpy(qa).double().permute(1, 0, 2),
                   torch.from_numpy(k).double().permute(1, 0, 2),
                   torch.from_numpy(v).double().permute(1, 0, 2), 0.4, mask)
    np.testing.assert_allclose(out, ro.permute(1, 0, 2).numpy()[L - T:], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, rl.permute(1, 0).numpy()[L - T:], rtol=1e-12, atol=1e-13)
    if T == 1:  # one token is plain decode over the whole context
        o1, l1 = oracle.attention(q, k, v, key_begin=0, key_end=L, scale=0.4, q_dtype="f32",
                                  kv_dtype="f32")
        assert np.array_equal(o1, out) and np.array_equal(l1, lse)


@pytest.mark.parametrize("N,I,T,L", [(4, 4, 2, 50), (8, 16, 4, 70), (3, 1, 3, 10), (4, 8, 2, 9)])
def test_merge_of_mtp_shard_partials_is_causal_attention(N, I, T, L):
    """Each shard's partial of the T tokens (keys it owns, positions <= the
    token's) merges exactly into the unsharded causal result; a token whose
    shard owns no visible key has o = 0 and LSE -inf there."""
    rng = np.random.default_rng(N * 1000 + L)
    Hq, Hkv, D = 4, 2, 8
    q = rng.standard_normal((T, Hq, D)).astype(np.float32)
    k = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    ro, rl = oracle.decode_mtp(q, k, v, L=L, scale=0.3, q_dtype="f32", kv_dtype="f32")
    parts = [oracle.decode_mtp(q, k, v, L=L, scale=0.3, q_dtype="f32", kv_dtype="f32",
                               shard=(N, I, r)) for r in range(N)]
    po = np.stack([p[0] for p in parts])
    pl = np.stack([p[1] for p in parts])
    mo, ml = oracle.lse_merge(po.reshape(N, T * Hq, D), pl.reshape(N, T * Hq))
    np.testing.assert_allclose(mo.reshape(T, Hq, D), ro, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ml.reshape(T, Hq), rl, rtol=1e-12, atol=1e-13)
    for r in range(N):
        for t in range(T):
            visible = [p for p in range(L - T + t + 1) if oracle.owner(p, N, I) == r]
            if not visible:
                assert np.all(parts[r][0][t] == 0) and np.all(np.isneginf(parts[r][1][t]))
