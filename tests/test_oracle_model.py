"""Pins of the oracle's routing, permutation, expert FFN, OFT, chunking and
LM-head log-prob (CPU only).

The method (Orbit announcement, 技术细节, active-expert-chunked
dequantization): router-selected experts, grouped in fixed-size chunks,
dequantized temporarily, grouped GEMM, weights released.  Chunking must not
change the result.  OFT adapter: an orthogonal transform (Orbit analysis
page, "为什么 OFT 重要").  Log-prob agreement metric: NeMo RL FP8 post,
token-mult-prob-error formula."""
import math

import numpy as np
import pytest

import oracle
from precision_moe_expert_amd import synth
from tests import refimpl


def tiny(fmt=1, T=24, H=128, I=128, E=6, k=2, oft=False, zipf=0.0, chunk=2):
    return synth.LayerConfig("tiny_pin", 90 + fmt, T=T, H=H, E=E, k=k, I=I, fmt=fmt, chunk=chunk,
                             oft=oft, zipf_alpha=zipf)


# ------------------------------------------------------------------ routing
@pytest.mark.parametrize("E,k", [(8, 2), (64, 8), (384, 8), (256, 8), (5, 5), (130, 16)])
def test_route_bruteforce(E, k):
    r = np.random.default_rng(E * 100 + k)
    lg = r.standard_normal((50, E)).astype(np.float32)
    lg[7, :] = 0.5                      # all equal -> ids 0..k-1
    lg[8, ::3] = 1.25                   # many ties
    lg[9, :] = -0.0; lg[9, 1::2] = 0.0  # -0 == +0
    ids, w = oracle.route(lg, k)
    ids2, w2 = refimpl.route_bruteforce(lg, k)
    assert np.array_equal(ids, ids2)
    assert np.max(np.abs(w - w2)) <= 1e-7
    assert np.array_equal(ids[7], np.arange(k)) and np.all(w[7] == np.float32(1.0 / k))
    assert np.array_equal(ids[9], np.arange(k))
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1) <= 1e-6)
    assert np.all(np.diff(w, axis=1) <= 0) and np.all(w > 0)


def test_route_k2_closed_form():
    r = np.random.default_rng(3)
    lg = r.standard_normal((200, 16)).astype(np.float32)
    ids, w = oracle.route(lg, 2)
    l0 = lg[np.arange(200), ids[:, 0]].astype(np.float64)
    l1 = lg[np.arange(200), ids[:, 1]].astype(np.float64)
    sig = 1.0 / (1.0 + np.exp(l1 - l0))
    assert np.max(np.abs(w[:, 0] - sig)) <= 1e-7


# -------------------------------------------------------------- permutation
@pytest.mark.parametrize("T,E,k", [(64, 8, 2), (333, 40, 8), (1, 4, 4), (100, 300, 3)])
def test_permute_bruteforce(T, E, k):
    r = np.random.default_rng(T + E + k)
    lg = r.standard_normal((T, E)).astype(np.float32)
    lg[:, 0] += 3.0  # a hot expert
    ids, _ = oracle.route(lg, k)
    P = oracle.permute(ids, E)
    trip = sorted((int(ids[t, j]), t, j) for t in range(T) for j in range(k))
    assert np.array_equal(P["sorted_rows"], np.array([t * k + j for _, t, j in trip], np.int32))
    assert np.array_equal(P["row_of"][P["sorted_rows"]], np.arange(T * k))
    assert np.array_equal(P["counts"], np.bincount(ids.ravel(), minlength=E))
    assert P["offsets"][0] == 0 and P["offsets"][E] == T * k and np.all(np.diff(P["offsets"]) >= 0)
    assert np.array_equal(P["active"], np.nonzero(P["counts"])[0])


# ----------------------------------------------------------- expert FFN: brute force
@pytest.mark.parametrize("fmt", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("oft", [False, True])
def test_forward_vs_dense_bruteforce(fmt, oft):
    cfg = tiny(fmt=fmt, oft=oft)
    li = synth.make_inputs(cfg)
    out = oracle.forward_inputs(li)
    ref, _, _ = refimpl.dense_moe(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, fmt, li.x, li.logits,
                                   li.w13, li.w2, li.s13, li.s2, oft=li.oft, g13=li.g13, g2=li.g2)
    rel = np.linalg.norm(out - ref, axis=1) / np.linalg.norm(ref, axis=1)
    # quantized-activation formats may flip a code where the two fp64 sums round
    # differently to fp32; all rows agree to 1e-3 and nearly all to 1e-6
    assert rel.max() <= (1e-6 if fmt in (1, 5) else 1e-3), rel.max()
    assert np.mean(rel <= 1e-6) >= 0.9


def test_forward_c1_vs_dense_bruteforce():
    cfg = synth.CONFIGS["c1"]
    li = synth.make_inputs(cfg)
    out = oracle.forward_inputs(li)
    ref, _, _ = refimpl.dense_moe(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.fmt, li.x, li.logits,
                                   li.w13, li.w2, li.s13, li.s2)
    rel = np.linalg.norm(out - ref, axis=1) / np.linalg.norm(ref, axis=1)
    assert rel.max() <= 1e-6


def test_single_expert_is_textbook_swiglu():
    cfg = tiny(fmt=1, E=1, k=1, T=9)
    li = synth.make_inputs(cfg)
    out = oracle.forward_inputs(li)
    W13 = refimpl.dequant(1, li.w13[0], li.s13[0], 2 * cfg.I, cfg.H)
    W2 = refimpl.dequant(1, li.w2[0], li.s2[0], cfg.H, cfg.I)
    x = refimpl.bf16_to_f32(li.x).astype(np.float64)
    g, u = x @ W13[:cfg.I].T, x @ W13[cfg.I:].T
    ref = (g / (1 + np.exp(-g)) * u) @ W2.T
    assert np.allclose(out, ref, rtol=1e-5, atol=1e-5)


def test_identical_experts_make_routing_irrelevant():
    cfg = tiny(fmt=1, E=5, k=3)
    li = synth.make_inputs(cfg)
    for a in (li.w13, li.w2, li.s13, li.s2):
        a[:] = a[0]
    out1 = oracle.forward_inputs(li)
    li.logits = np.random.default_rng(9).standard_normal(li.logits.shape).astype(np.float32)
    out2 = oracle.forward_inputs(li)
    assert np.allclose(out1, out2, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_zero_up_projection_gives_zero(fmt):
    cfg = tiny(fmt=fmt)
    li = synth.make_inputs(cfg)
    I = cfg.I
    if fmt == 2:
        li.w13[:, I:, :] = 0
    else:
        li.w13[:, I:, :] = 0  # nibble code 0 is value 0 for int4 and e2m1
    out = oracle.forward_inputs(li)
    assert not out.any()


# ----------------------------------------------------------------- chunking
@pytest.mark.parametrize("fmt", [1, 3])
def test_chunk_size_does_not_change_output(fmt):
    cfg = tiny(fmt=fmt, E=7, k=3, zipf=1.2)
    li = synth.make_inputs(cfg)
    outs = [oracle.forward_inputs(li, chunk_experts=c) for c in (1, 2, 3, 7, 100)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_token_subset_matches_full():
    cfg = tiny(fmt=2, T=40, E=6, k=2)
    li = synth.make_inputs(cfg)
    full = oracle.forward_inputs(li)
    sub = np.array([39, 0, 17, 5], np.int32)
    part = oracle.forward_inputs(li, tokens=sub)
    assert np.array_equal(part, full[sub])


# ---------------------------------------------------------------------- OFT
def test_oft_rotation_is_orthogonal():
    cfg = tiny(fmt=1, oft=True, E=3, H=128)
    # float64 Cayley transform as the generator builds it
    r = np.random.default_rng(0)
    u = np.triu(r.standard_normal((32, 32)) * 0.1, 1)
    S = u - u.T
    R = (np.eye(32) - S) @ np.linalg.inv(np.eye(32) + S)
    assert np.max(np.abs(R.T @ R - np.eye(32))) <= 1e-12
    x = r.standard_normal(32)
    assert abs(np.linalg.norm(x @ R) - np.linalg.norm(x)) <= 1e-12
    # bf16-stored R of the generator: norm kept to ~1e-3
    Rb = refimpl.bf16_to_f32(synth.gen_oft(cfg)).astype(np.float64)
    xs = r.standard_normal((100, 32))
    ratio = np.linalg.norm(np.einsum("ti,bij->btj", xs, Rb.reshape(-1, 32, 32)), axis=2) / np.linalg.norm(xs, axis=1)
    assert np.max(np.abs(ratio - 1)) <= 1e-2


def test_oft_identity_equals_no_adapter():
    cfg = tiny(fmt=2, oft=True)
    li = synth.make_inputs(cfg)
    li.oft[:] = 0
    li.oft[:, :, np.arange(32), np.arange(32)] = 0x3F80  # bf16 1.0
    a = oracle.forward_inputs(li)
    li.oft = None
    b = oracle.forward_inputs(li)
    assert np.array_equal(a, b)


def test_oft_shared_stride_zero():
    cfg = tiny(fmt=1, oft=True, E=4)
    li = synth.make_inputs(cfg)
    shared = li.oft[2].copy()
    li_all = synth.make_inputs(cfg)
    li_all.oft[:] = shared
    a = oracle.forward_inputs(li_all)
    c = cfg
    b = oracle.forward(c.T, c.H, c.I, c.E, c.k, c.fmt, li.x, li.logits, li.w13, li.w2, li.s13, li.s2,
                       oft=shared, chunk_experts=c.chunk, adapter_expert_stride=0)
    assert np.array_equal(a, b)


def test_oft_block_locality():
    """Changing R's block b changes the rotated input only on dims 32b..32b+31:
    with an FFN whose gate/up weights are zero outside block 1's columns, a change
    of block 0 leaves the output unchanged and a change of block 1 does not."""
    cfg = tiny(fmt=1, oft=True, E=2, k=1, H=128)
    li = synth.make_inputs(cfg)
    q = li.w13.reshape(cfg.E, 2 * cfg.I, cfg.H // 2)
    q[:, :, :16] = 0      # columns 0..31 (block 0) zero
    q[:, :, 32:] = 0      # columns 64.. zero -> only block 1 (cols 32..63) feeds the FFN
    base = oracle.forward_inputs(li)
    li0 = synth.make_inputs(cfg); li0.w13[:] = li.w13; li0.oft[:, 0] = li.oft[:, 2]
    assert np.array_equal(oracle.forward_inputs(li0), base)
    li1 = synth.make_inputs(cfg); li1.w13[:] = li.w13; li1.oft[:, 1] = li.oft[:, 3]
    assert not np.array_equal(oracle.forward_inputs(li1), base)


# ------------------------------------------------------------------ LM head
def test_logprob_uniform_closed_form():
    T, H, V = 3, 64, 32000
    h = np.random.default_rng(1).standard_normal((T, H)).astype(np.float32)
    w = np.zeros((V, H), np.uint16)
    lp = oracle.lm_head_logprob(h, w, np.array([0, 31999, 12345], np.int32))
    assert np.allclose(lp, -math.log(V), atol=1e-6)
    assert abs(-math.log(V) - (-10.373491181781864)) < 1e-12


def test_logprob_normalised_and_bruteforce():
    r = np.random.default_rng(2)
    T, H, V = 4, 96, 300
    h = (r.standard_normal((T, H)) * 30).astype(np.float32)
    wb = refimpl.torch.from_numpy((r.standard_normal((V, H)) / np.sqrt(H)).astype(np.float32)).to(refimpl.torch.bfloat16).view(refimpl.torch.int16).numpy().view(np.uint16)
    W = refimpl.bf16_to_f32(wb).astype(np.float64)
    # all targets of token 0 -> probabilities sum to one
    lp_all = oracle.lm_head_logprob(np.repeat(h[:1], V, 0), wb, np.arange(V, dtype=np.int32))
    assert abs(np.exp(lp_all.astype(np.float64)).sum() - 1.0) <= 1e-5
    tg = r.integers(0, V, T).astype(np.int32)
    lp = oracle.lm_head_logprob(h, wb, tg)
    hd = h.astype(np.float64)
    z = hd / np.sqrt((hd ** 2).mean(1, keepdims=True) + 1e-6)
    lg = z @ W.T
    m = lg.max(1, keepdims=True)
    ref = lg[np.arange(T), tg] - (m[:, 0] + np.log(np.exp(lg - m).sum(1)))
    assert np.max(np.abs(lp - ref)) <= 1e-5


def _bf16_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("T,k,H,seed", [(1, 1, 8, 0), (13, 4, 32, 1), (40, 16, 24, 2), (7, 8, 64, 3)])
def test_combine_matches_gather_sum(T, k, H, seed):
    """oracle.combine against a brute-force gather: out[t] = sum_j w[t, j] *
    y_perm[row_of[t*k + j]], summed in fp64 in ascending j, with row_of a
    random permutation of the T*k permuted rows and y_perm bf16."""
    r = np.random.default_rng(seed)
    R = T * k
    row_of = r.permutation(R).astype(np.int32)
    y = synth._to_bf16_bits((r.standard_normal((R, H)) * 4).astype(np.float32))
    w = r.random((T, k)).astype(np.float32)
    got = oracle.combine(y, w, row_of)
    yv = _bf16_f64(y)
    ref = np.zeros((T, H))
    for t in range(T):
        acc = np.zeros(H)
        for j in range(k):
            acc = acc + np.float64(w[t, j]) * yv[row_of[t * k + j]]
        ref[t] = acc
    assert np.array_equal(got, ref.astype(np.float32))


def test_combine_one_hot_reveals_pair_indexing():
    """With y_perm row r = 2^-r at column r (one-hot) and weights 1, output
    row t holds 2^-row_of[t*k+j] exactly at columns row_of[t*k+j] for its k
    slots and zeros elsewhere: a transposed (j*T + t) or inverse
    (sorted_rows) index lands on other columns."""
    T, k = 5, 3
    R = T * k
    row_of = np.random.default_rng(9).permutation(R).astype(np.int32)
    vals = np.float32(2.0) ** -np.arange(R, dtype=np.float32)
    y = np.zeros((R, R), np.float32)
    y[np.arange(R), np.arange(R)] = vals
    out = oracle.combine(synth._to_bf16_bits(y), np.ones((T, k), np.float32), row_of)
    expect = np.zeros((T, R), np.float32)
    for t in range(T):
        for j in range(k):
            r = row_of[t * k + j]
            expect[t, r] = vals[r]
    assert np.array_equal(out, expect)


def test_combine_weights_weight_slots_in_order():
    """Distinct power-of-two weights per slot on identical y rows of ones:
    out[t] = sum_j w[t, j], and swapping two slots' weights changes nothing
    only when their rows are equal, so slot j must read w[t, j]."""
    T, k, H = 3, 4, 8
    row_of = np.arange(T * k, dtype=np.int32)
    y = np.zeros((T * k, H), np.float32)
    for r in range(T * k):
        y[r] = r + 1                      # row r holds the value r + 1
    w = np.array([[2.0 ** -(j + 1) for j in range(k)]] * T, np.float32)
    out = oracle.combine(synth._to_bf16_bits(y), w, row_of)
    for t in range(T):
        expect = sum((t * k + j + 1) * 2.0 ** -(j + 1) for j in range(k))
        assert np.all(out[t] == np.float32(expect))
