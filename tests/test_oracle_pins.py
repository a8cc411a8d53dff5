"""Pins for the CPU oracle: each test ties it to something other than itself.

Kinds of pin used here:
  * worked examples from the pages (tests/golden, each with its citation);
  * a brute force of the placement definition, O((T*K)^2), that shares
    nothing with the oracle's counting-sort algorithm, run exhaustively on
    tiny inputs and on random small ones;
  * a library routine: numpy's stable argsort gives the row -> slot map;
  * closed forms for combine on exactly representable values (one-hot rows,
    K = 1 with weight 1, identity expert with weights summing to 1);
  * torch's float -> bf16 conversion (round to nearest even) for the bf16
    encoder, and hand-checked ties for the large-batch expert stand-in;
  * invariants (counts sum, contiguous blocks, bijection, row copies).
"""
import itertools

import numpy as np
import pytest

import oracle
from conftest import load_golden
from oracle import OracleError


# --------------------------------------------------------------- helpers --

def brute_force(topk, E, R, alignment=0):
    """Every quantity straight from its definition, by enumeration. With an
    alignment a > 1, expert e's block holds the smallest multiple of a that
    is >= its count, and rows holding no slot are marked -1."""
    T, K = topk.shape
    slots = [(t, k) for t in range(T) for k in range(K)]
    epr = E // R
    cnt = [sum(1 for (t, k) in slots if topk[t, k] == e) for e in range(E)]
    in_rank = [[int(any(topk[t, k] >= 0 and topk[t, k] // epr == r for k in range(K)))
                for r in range(R)] for t in range(T)]
    per_rank = [sum(in_rank[t][r] for t in range(T)) for r in range(R)]
    a = max(alignment, 1)
    size = [min(m for m in range(0, c + a, a) if m >= c) for c in cnt]
    start = [sum(size[:e]) for e in range(E)]
    oi = [[-1] * K for _ in range(T)]
    for (t, k) in slots:
        e = topk[t, k]
        if e < 0:
            continue
        earlier = sum(1 for (t2, k2) in slots if topk[t2, k2] == e and (t2, k2) < (t, k))
        oi[t][k] = start[e] + earlier
    N = sum(size)
    m = [-1] * N
    for (t, k) in slots:
        if oi[t][k] >= 0:
            m[oi[t][k]] = topk[t, k]
    return dict(cnt=np.array(cnt), per_rank=np.array(per_rank), in_rank=np.array(in_rank),
                start=np.array(start), total=N, oi=np.array(oi), m=np.array(m, dtype=np.int64))


def run_oracle(topk, E, R, x=None, x_scale=None, orc=None, alignment=0):
    orc = orc or oracle.default()
    cnt, per_rank, in_rank = orc.layout(topk, E, R)
    start, total = orc.scan(cnt, alignment)
    out, out_scale, m, oi = orc.scatter(x, x_scale, topk, start, total)
    return dict(cnt=cnt, per_rank=per_rank, in_rank=in_rank, start=start, total=total,
                out=out, out_scale=out_scale, m=m, oi=oi)


def assert_same_as_brute(topk, E, R, orc=None, alignment=0):
    got = run_oracle(topk, E, R, orc=orc, alignment=alignment)
    want = brute_force(topk, E, R, alignment=alignment)
    np.testing.assert_array_equal(got["cnt"], want["cnt"])
    np.testing.assert_array_equal(got["per_rank"], want["per_rank"])
    np.testing.assert_array_equal(got["in_rank"], want["in_rank"].reshape(got["in_rank"].shape))
    np.testing.assert_array_equal(got["start"], want["start"])
    assert got["total"] == want["total"]
    np.testing.assert_array_equal(got["oi"], want["oi"].reshape(got["oi"].shape))
    np.testing.assert_array_equal(got["m"], want["m"])


# ------------------------------------------------------ worked examples --

def test_golden_scan_prefix_example():
    g = load_golden("scan_prefix_example.txt")
    start, total = oracle.scan(np.array(g["counts"]))
    assert start.tolist() == g["expert_start_loc"]
    assert total == g["total"][0]


def test_golden_route_token_3_7():
    g = load_golden("route_token_3_7.txt")
    E, R = g["num_experts"][0], g["num_ranks"][0]
    topk = np.array([g["topk_idx"]], dtype=np.int64)
    cnt, per_rank, in_rank = oracle.layout(topk, E, R)
    assert cnt.tolist() == g["num_tokens_per_expert"]
    assert per_rank.tolist() == g["num_tokens_per_rank"]
    assert in_rank[0].tolist() == g["is_token_in_rank"]


def brute_rdma(topk, E, R, G):
    """Tokens per node straight from topk_idx: node of a slot = its owner
    rank // G; a token counts once per node it reaches."""
    T, K = topk.shape
    epr = E // R
    return np.array([sum(1 for t in range(T)
                         if any(topk[t, k] >= 0 and (topk[t, k] // epr) // G == n
                                for k in range(K)))
                     for n in range(R // G)])


def test_golden_rdma_counts_example():
    g = load_golden("rdma_counts_example.txt")
    E, R = g["num_experts"][0], g["num_ranks"][0]
    topk = np.array(g["topk_idx"], dtype=np.int64)
    _, _, in_rank = oracle.layout(topk, E, R)
    for G in (1, 2, 4):
        assert oracle.rdma_counts(in_rank, G).tolist() == g[f"rdma_g{G}"], G
    assert oracle.rdma_counts(in_rank, 8) is None          # one node
    assert oracle.rdma_counts(in_rank, 0) is None          # not asked for


@pytest.mark.parametrize("seed", range(6))
def test_rdma_counts_against_brute_force(seed):
    rng = np.random.default_rng(300 + seed)
    R = int(rng.choice([2, 4, 6, 8, 12]))
    E = R * int(rng.integers(1, 4))
    T, K = int(rng.integers(0, 40)), int(rng.integers(1, 6))
    topk = rng.integers(-1, E, size=(T, K)).astype(np.int64)
    _, per_rank, in_rank = oracle.layout(topk, E, R)
    for G in [g for g in range(1, R) if R % g == 0]:
        got = oracle.rdma_counts(in_rank, G)
        np.testing.assert_array_equal(got, brute_rdma(topk, E, R, G))
        nodes = per_rank.reshape(R // G, G)
        # a node gets at least as many tokens as its busiest rank and at
        # most the sum over its ranks
        assert (got >= nodes.max(axis=1)).all() and (got <= nodes.sum(axis=1)).all()
    np.testing.assert_array_equal(oracle.rdma_counts(in_rank, 1), per_rank)


def test_golden_scatter_hand_example():
    g = load_golden("scatter_hand_example.txt")
    E, R = g["num_experts"][0], g["num_ranks"][0]
    topk = np.array(g["topk_idx"], dtype=np.int64)
    T, K = topk.shape
    H = 8
    x = (np.arange(T * H, dtype=np.uint16) + 1).reshape(T, H)
    got = run_oracle(topk, E, R, x=x)
    assert got["cnt"].tolist() == g["num_tokens_per_expert"]
    assert got["start"].tolist() == g["expert_start_loc"]
    assert got["total"] == g["total"][0]
    assert got["oi"].tolist() == g["output_index"]
    assert got["m"].tolist() == g["m_indices"]
    assert got["per_rank"].tolist() == g["num_tokens_per_rank"]
    for row, src in enumerate(g["row_source_token"]):
        np.testing.assert_array_equal(got["out"][row], x[src])


# ------------------------------------------------------------ brute force --

EXHAUSTIVE_SHAPES = [
    # (T, K, E, R)
    (1, 3, 4, 4),
    (2, 2, 4, 2),
    (3, 2, 3, 3),
    (3, 2, 3, 1),
    (4, 1, 2, 1),
    (2, 3, 2, 2),
]


@pytest.mark.parametrize("T,K,E,R", EXHAUSTIVE_SHAPES)
def test_exhaustive_tiny_against_brute_force(T, K, E, R):
    """Every topk_idx matrix with entries in {-1, 0, .., E-1}: duplicates
    within a token, all -1 rows and empty experts included."""
    for vals in itertools.product(range(-1, E), repeat=T * K):
        topk = np.array(vals, dtype=np.int64).reshape(T, K)
        assert_same_as_brute(topk, E, R)


@pytest.mark.parametrize("seed", range(40))
def test_random_small_against_brute_force(seed):
    rng = np.random.default_rng(1000 + seed)
    R = int(rng.integers(1, 5))
    E = R * int(rng.integers(1, 5))
    T = int(rng.integers(0, 14))
    K = int(rng.integers(1, 5))
    topk = rng.integers(-1, E, size=(T, K)).astype(np.int64)
    assert_same_as_brute(topk, E, R)


@pytest.mark.parametrize("T,K,E,R,a", [(2, 2, 3, 3, 2), (3, 2, 2, 1, 3), (1, 3, 4, 2, 4)])
def test_exhaustive_tiny_aligned_against_brute_force(T, K, E, R, a):
    for vals in itertools.product(range(-1, E), repeat=T * K):
        topk = np.array(vals, dtype=np.int64).reshape(T, K)
        assert_same_as_brute(topk, E, R, alignment=a)


@pytest.mark.parametrize("seed", range(20))
def test_random_small_aligned_against_brute_force(seed):
    rng = np.random.default_rng(3000 + seed)
    R = int(rng.integers(1, 4))
    E = R * int(rng.integers(1, 4))
    T, K = int(rng.integers(0, 12)), int(rng.integers(1, 4))
    a = int(rng.integers(0, 7))
    topk = rng.integers(-1, E, size=(T, K)).astype(np.int64)
    assert_same_as_brute(topk, E, R, alignment=a)


def test_golden_alignment_example():
    g = load_golden("scan_alignment_example.txt")
    start, total = oracle.scan(np.array(g["counts"]), g["alignment"][0])
    assert start.tolist() == g["expert_start_loc"]
    assert total == g["total"][0]


@pytest.mark.parametrize("a", [1, 2, 16, 256])
def test_aligned_total_within_the_pages_upper_bound(a):
    """The vLLM fork's bound for the permuted row count with block_m padding:
    round_up(T*K + E*(a-1), a) ([SGLANG] section 4, compute_aligned_M). Every
    block is a multiple of a, holds its expert's rows first and pads with
    fewer than a rows marked -1."""
    from permute_ep_layout_amd import workloads
    w = workloads.get("small").with_(num_tokens=700)
    topk = workloads.make_topk(w)
    E, R = w.num_experts, w.num_ranks
    T, K = topk.shape
    got = run_oracle(topk, E, R, alignment=a)
    bound = -(-(T * K + E * (a - 1)) // a) * a
    assert got["total"] <= bound and got["total"] % a == 0
    ends = list(got["start"][1:]) + [got["total"]]
    for e in range(E):
        size = ends[e] - got["start"][e]
        assert size % a == 0 and 0 <= size - got["cnt"][e] < a
        blk = got["m"][got["start"][e]:ends[e]]
        assert (blk[:got["cnt"][e]] == e).all() and (blk[got["cnt"][e]:] == -1).all()


# ------------------------------------------------- library routine: argsort --

@pytest.mark.parametrize("seed", range(5))
def test_row_order_is_numpy_stable_argsort(seed):
    """Rows in expert order, ties by (token, k): exactly a stable sort of the
    flattened slot keys with the -1 slots (which sort first) dropped."""
    rng = np.random.default_rng(seed)
    T, K, E, R = 700, 6, 48, 8
    topk = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    topk[rng.random(topk.shape) < 0.1] = -1
    got = run_oracle(topk, E, R)
    flat = topk.ravel()
    order = np.argsort(flat, kind="stable")
    order = order[flat[order] >= 0]
    N = order.size
    assert got["total"] == N
    np.testing.assert_array_equal(got["oi"].ravel()[order], np.arange(N))
    np.testing.assert_array_equal(got["m"], flat[order])
    np.testing.assert_array_equal(got["oi"].ravel()[flat < 0], -1)


# ------------------------------------------------- byte rows, scale words --

def test_golden_scale_words_column_major():
    g = load_golden("scatter_scale_cols_example.txt")
    E, R = g["num_experts"][0], g["num_ranks"][0]
    topk = np.array(g["topk_idx"], dtype=np.int64)
    words = np.array(g["scale_words"], dtype=np.uint32)
    orc = oracle.default()
    cnt, _, _ = orc.layout(topk, E, R)
    start, total = orc.scan(cnt)
    _, out_scale, m, oi = orc.scatter_rows(None, words, orc.SCALE_COLS, topk, start, total,
                                          scale_ld=g["ld"][0])
    want = g["out_scale_flat"]
    for i, v in enumerate(want):
        if v >= 0:
            assert int(out_scale[i]) == v, i


@pytest.mark.parametrize("seed,ld_extra", [(0, 0), (1, 5), (2, 1000)])
def test_byte_rows_and_transposed_scales_match_numpy(seed, ld_extra):
    """FP8 rows move as bytes; the column-major scale buffer, read back with
    numpy's transpose, holds each row's token's words (row -> token map from
    numpy's stable argsort)."""
    rng = np.random.default_rng(seed)
    T, K, E, R, B, W = 300, 5, 24, 6, 96, 3
    topk = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    topk[rng.random(topk.shape) < 0.1] = -1
    x = rng.integers(0, 256, size=(T, B), dtype=np.uint8)
    words = rng.integers(0, 1 << 32, size=(T, W), dtype=np.uint64).astype(np.uint32)
    orc = oracle.default()
    cnt, _, _ = orc.layout(topk, E, R)
    start, total = orc.scan(cnt)
    ld = total + ld_extra
    out, cols, m, oi = orc.scatter_rows(x, words, orc.SCALE_COLS, topk, start, total, scale_ld=ld)
    _, rows, m2, oi2 = orc.scatter_rows(x, words, orc.SCALE_ROWS, topk, start, total)
    flat = topk.ravel()
    order = np.argsort(flat, kind="stable")
    src = (order[flat[order] >= 0]) // K            # token of each row
    np.testing.assert_array_equal(out, x[src])
    np.testing.assert_array_equal(cols.reshape(W, ld)[:, :total].T, words[src])
    np.testing.assert_array_equal(rows, words[src])
    np.testing.assert_array_equal(m, m2)
    np.testing.assert_array_equal(oi, oi2)


def test_byte_rows_agree_with_bf16_scatter():
    from permute_ep_layout_amd import workloads
    w = workloads.get("dsv3").with_(num_tokens=200, hidden=256)
    inp = workloads.make_inputs(w)
    orc = oracle.default()
    cnt, _, _ = orc.layout(inp["topk_idx"], w.num_experts, w.num_ranks)
    start, total = orc.scan(cnt, 8)
    out, out_s, m, oi = orc.scatter(inp["x"], inp["x_scale"], inp["topk_idx"], start, total)
    outb, rows, mb, oib = orc.scatter_rows(inp["x"].view(np.uint8), inp["x_scale"].view(np.uint32),
                                           orc.SCALE_ROWS, inp["topk_idx"], start, total)
    real = m >= 0
    np.testing.assert_array_equal(outb.view(np.uint16)[real], out[real])
    np.testing.assert_array_equal(rows[real], out_s.view(np.uint32)[real])
    np.testing.assert_array_equal(mb, m)
    np.testing.assert_array_equal(oib, oi)


# ------------------------------------------------------------- invariants --

def test_invariants_on_generated_workload():
    from permute_ep_layout_amd import workloads
    w = workloads.get("small").with_(num_tokens=300, hidden=64)
    inp = workloads.make_inputs(w)
    topk, x = inp["topk_idx"], inp["x"]
    E, R = w.num_experts, w.num_ranks
    got = run_oracle(topk, E, R, x=x)
    valid = topk >= 0
    assert got["cnt"].sum() == valid.sum() == got["total"]
    # each expert's rows are the contiguous block starting at its offset
    for e in range(E):
        blk = got["m"][got["start"][e]:got["start"][e] + got["cnt"][e]]
        assert (blk == e).all()
    assert (np.diff(got["m"]) >= 0).all()
    # output_index is a bijection from the valid slots onto [0, N)
    placed = got["oi"][valid]
    assert np.array_equal(np.sort(placed), np.arange(got["total"]))
    assert (got["oi"][~valid] == -1).all()
    # every placed row is a bit copy of its token's row
    tt, kk = np.nonzero(valid)
    np.testing.assert_array_equal(got["out"][got["oi"][tt, kk]], x[tt])
    # per-rank counts: column sums of the mask, bounded by the rank's slot count
    np.testing.assert_array_equal(got["per_rank"], got["in_rank"].sum(axis=0))
    epr = E // R
    for r in range(R):
        assert got["per_rank"][r] <= got["cnt"][r * epr:(r + 1) * epr].sum()
    assert got["total"] <= topk.size


def test_scale_rows_follow_their_rows():
    rng = np.random.default_rng(7)
    T, K, E, R, H = 50, 4, 16, 4, 256
    topk = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    x = rng.integers(0, 1 << 16, size=(T, H), dtype=np.uint16)
    xs = rng.uniform(0.01, 1.0, size=(T, H // 128)).astype(np.float32)
    got = run_oracle(topk, E, R, x=x, x_scale=xs)
    tt, kk = np.nonzero(topk >= 0)
    rows = got["oi"][tt, kk]
    np.testing.assert_array_equal(got["out_scale"][rows].view(np.uint32), xs[tt].view(np.uint32))


def test_empty_and_all_invalid():
    E, R = 8, 4
    got = run_oracle(np.zeros((0, 3), np.int64), E, R)
    assert got["total"] == 0 and got["cnt"].sum() == 0 and (got["start"] == 0).all()
    topk = -np.ones((5, 3), np.int64)
    got = run_oracle(topk, E, R)
    assert got["total"] == 0 and (got["oi"] == -1).all() and got["in_rank"].sum() == 0
    y = oracle.combine(np.zeros((0, 16), np.uint16), got["oi"], np.ones((5, 3), np.float32))
    assert (y == 0).all() and not np.signbit(y).any()


def test_errors():
    with pytest.raises(OracleError) as ei:
        oracle.layout(np.array([[0, 8]], np.int64), 8, 4)
    assert ei.value.code == oracle.ERANGE
    with pytest.raises(OracleError) as ei:
        oracle.layout(np.array([[0, -2]], np.int64), 8, 4)
    assert ei.value.code == oracle.ERANGE
    with pytest.raises(OracleError) as ei:
        oracle.layout(np.array([[0, 1]], np.int64), 9, 4)       # E % R != 0
    assert ei.value.code == oracle.EINVAL


# ---------------------------------------------------------------- combine --

def _bf16(values):
    return np.asarray(np.asarray(values, np.float32).view(np.uint32) >> 16, dtype=np.uint16)


def test_combine_one_hot_rows():
    """With row p of the expert output equal to the unit vector e_p, token t's
    result holds w[t,k] in column output_index[t,k] and zeros elsewhere:
    this pins which row each slot reads and which weight multiplies it."""
    rng = np.random.default_rng(3)
    T, K, E, R = 12, 3, 8, 2
    topk = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    topk[rng.random(topk.shape) < 0.2] = -1
    got = run_oracle(topk, E, R)
    N = got["total"]
    eye = _bf16(np.eye(N, dtype=np.float32))
    w = rng.uniform(0.05, 1.0, size=(T, K)).astype(np.float32)
    y = oracle.combine(eye, got["oi"], w)
    expect = np.zeros((T, N))
    for t in range(T):
        for k in range(K):
            if topk[t, k] >= 0:
                expect[t, got["oi"][t, k]] = np.float64(w[t, k])
    np.testing.assert_array_equal(y, expect)


def test_combine_k1_weight1_is_identity():
    rng = np.random.default_rng(4)
    T, E, R, H = 40, 8, 4, 96
    topk = rng.integers(0, E, size=(T, 1)).astype(np.int64)
    x = _bf16(rng.standard_normal((T, H)).astype(np.float32))
    got = run_oracle(topk, E, R, x=x)
    y = oracle.combine(got["out"], got["oi"], np.ones((T, 1), np.float32))
    np.testing.assert_array_equal(y, (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64))


def test_combine_identity_expert_returns_input():
    """Scatter then an identity-expert combine with weights that sum to 1
    returns x, up to the weights' own fp32 rounding (|sum w - 1|)."""
    from permute_ep_layout_amd import workloads
    w = workloads.get("small").with_(num_tokens=200, hidden=128)
    inp = workloads.make_inputs(w)
    topk, x, wt = inp["topk_idx"], inp["x"], inp["topk_weights"]
    got = run_oracle(topk, w.num_experts, w.num_ranks, x=x)
    y = oracle.combine(got["out"], got["oi"], wt)
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    has = (topk >= 0).any(axis=1)
    wsum = wt.astype(np.float64).sum(axis=1, keepdims=True)
    assert np.abs(wsum[has] - 1).max() < 1e-6
    bound = (np.abs(wsum - 1) + 1e-15) * np.abs(xf)
    assert (np.abs(y - xf)[has] <= bound[has]).all()
    assert (y[~has] == 0).all()


def test_combine_rejects_row_beyond_expert_output():
    with pytest.raises(OracleError):
        oracle.combine(np.zeros((2, 4), np.uint16), np.array([[0, 2]], np.int32),
                       np.ones((1, 2), np.float32))


def test_combine_token_subset_matches_full():
    rng = np.random.default_rng(5)
    T, K, E, R, H = 30, 4, 16, 4, 32
    topk = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    x = _bf16(rng.standard_normal((T, H)).astype(np.float32))
    got = run_oracle(topk, E, R, x=x)
    wt = rng.uniform(0, 1, (T, K)).astype(np.float32)
    full = oracle.combine(got["out"], got["oi"], wt)
    sel = np.array([29, 0, 7, 7])
    np.testing.assert_array_equal(oracle.combine(got["out"], got["oi"], wt, tokens=sel), full[sel])


# ------------------------------------------------------------------ bf16 --

def test_bf16_decode_is_upper_half_of_binary32():
    bits = np.arange(0, 1 << 16, 97, dtype=np.uint16)
    want32 = (bits.astype(np.uint32) << 16).view(np.float32)
    finite = np.isfinite(want32)
    want = want32[finite].astype(np.float64)
    got = np.array([oracle.bf16_to_double(int(b)) for b in bits[finite]])
    np.testing.assert_array_equal(got, want)


def test_bf16_encoder_matches_torch_round_to_nearest_even():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    u = rng.integers(0, 1 << 32, size=20000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    # add exact ties and near-ties around a few binades, subnormals, extremes
    ties = (np.arange(1, 2000, dtype=np.uint32) << 16 | np.uint32(0x8000)).view(np.float32)
    extra = np.array([0.0, -0.0, 1e-45, -1e-45, 1.17549435e-38, 3.4028235e38, -3.4028235e38,
                      3.3895314e38, 3.3961776e38], dtype=np.float32)
    f = np.concatenate([f, ties, -ties, extra])
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_from_double_array(f.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_expert_scale_hand_checked_values():
    """bf16(x * (1 + e/256)) on hand-worked cases, including an exact tie."""
    cases = [
        (0x3F80, 0, 0x3F80),     # 1 * 1 = 1
        (0x3F80, 128, 0x3FC0),   # 1 * 1.5 = 1.5
        (0x3F80, 255, 0x4000),   # 1 + 255/256: exactly half an ulp above 1.9921875 -> even -> 2
        (0x3F80, 254, 0x3FFF),   # 1 + 254/256 = 1.9921875, representable
        (0x3F81, 1, 0x3F82),     # (1+2^-7)(1+2^-8) = 1+2^-7+2^-8+2^-15 > halfway -> up
        (0x3F80, 1, 0x3F80),     # 1 + 2^-8: exactly halfway between 1 and 1+2^-7 -> even -> 1
        (0xBF80, 64, 0xBFA0),    # -1 * 1.25 = -1.25
        (0x0000, 200, 0x0000),
    ]
    rows = np.array([[c[0]] for c in cases], np.uint16)
    m = np.array([c[1] for c in cases], np.int32)
    got = oracle.expert_scale(rows, m)[:, 0]
    assert [hex(v) for v in got] == [hex(c[2]) for c in cases]


# ------------------------------------------------- receive side (local ids) --

def _to_local(topk, r, El):
    """The batch rank r holds after the dispatch: tokens that pick one of its
    experts [r*El, (r+1)*El), ids made local, -1 for other ranks' experts."""
    mine = (topk >= r * El) & (topk < (r + 1) * El)
    keep = np.nonzero(mine.any(axis=1))[0]
    return keep, np.where(mine[keep], topk[keep] - r * El, -1)


@pytest.mark.parametrize("seed,a", [(0, 0), (1, 0), (2, 4), (3, 3)])
def test_local_mode_is_the_global_buffer_restricted(seed, a):
    """With contiguous ownership, rank r's experts form one stretch of the
    global expert-contiguous buffer. Run on the rank's received batch with
    local ids, the path must produce exactly that stretch: the same rows in
    the same order, m_indices shifted by r*El, output_index shifted by the
    stretch's start."""
    rng = np.random.default_rng(500 + seed)
    T, K, R, El, H = 150, 4, 6, 4, 8
    E = R * El
    topk = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    topk[rng.random(topk.shape) < 0.15] = -1
    x = rng.integers(0, 1 << 15, size=(T, H), dtype=np.uint16)
    xs = rng.uniform(0.01, 1, size=(T, 1)).astype(np.float32)
    g = run_oracle(topk, E, R, x=x, x_scale=xs, alignment=a)
    for r in range(R):
        keep, lt = _to_local(topk, r, El)
        loc = run_oracle(lt, El, 1, x=x[keep], x_scale=xs[keep], alignment=a)
        lo = g["start"][r * El]
        hi = g["start"][(r + 1) * El] if r + 1 < R else g["total"]
        assert loc["total"] == hi - lo
        np.testing.assert_array_equal(loc["cnt"], g["cnt"][r * El:(r + 1) * El])
        m = g["m"][lo:hi]
        np.testing.assert_array_equal(loc["m"], np.where(m >= 0, m - r * El, -1))
        real = m >= 0
        np.testing.assert_array_equal(loc["out"][real], g["out"][lo:hi][real])
        np.testing.assert_array_equal(loc["out_scale"][real], g["out_scale"][lo:hi][real])
        want_oi = np.where(lt >= 0, g["oi"][keep] - lo, -1)
        np.testing.assert_array_equal(loc["oi"], want_oi)
        assert loc["per_rank"].tolist() == [len(keep)]


def test_local_partial_combines_sum_to_the_global_combine():
    """Each rank combines only its own slots; adding the partial sums of all
    ranks per source token gives the global combine (fp64, up to rounding)."""
    rng = np.random.default_rng(77)
    T, K, R, El, H = 120, 5, 4, 6, 16
    E = R * El
    topk = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    topk[rng.random(topk.shape) < 0.1] = -1
    x = rng.integers(0, 1 << 15, size=(T, H), dtype=np.uint16) & np.uint16(0xBFFF)  # finite
    w = rng.uniform(0.05, 1, size=(T, K)).astype(np.float32)
    g = run_oracle(topk, E, R, x=x)
    y = oracle.combine(g["out"], g["oi"], w)
    acc = np.zeros((T, H))
    for r in range(R):
        keep, lt = _to_local(topk, r, El)
        loc = run_oracle(lt, El, 1, x=x[keep])
        acc[keep] += oracle.combine(loc["out"], loc["oi"], w[keep])
    xv = np.array([[oracle.bf16_to_double(int(v)) for v in row] for row in x])
    bound = np.abs(w.astype(np.float64)).sum(axis=1, keepdims=True) * np.abs(xv)
    assert np.all(np.abs(acc - y) <= 1e-12 * bound + 1e-300)


# ------------------------------------------------------ FP8 e4m3 encoding --

def _e4m3_values():
    """Every finite e4m3 value, decoded by torch (the encoding's own
    decoder), sorted."""
    torch = pytest.importorskip("torch")
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    return codes, vals


def test_e4m3_encoder_matches_torch():
    """Every finite code round-trips; midpoints between neighbours (ties)
    and random values in range round as torch's float8_e4m3fn conversion
    does (round to nearest even)."""
    torch = pytest.importorskip("torch")
    codes, vals = _e4m3_values()
    np.testing.assert_array_equal(oracle.e4m3_from_double_array(vals), codes)
    pos = np.unique(vals[vals >= 0])
    mids = (pos[1:] + pos[:-1]) / 2                      # exact in binary32
    rng = np.random.default_rng(12)
    rnd = rng.standard_normal(4000) * np.exp2(rng.integers(-12, 9, 4000))
    v = np.concatenate([mids, -mids, rnd[np.abs(rnd) < 464]]).astype(np.float32)
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.e4m3_from_double_array(v.astype(np.float64)), want)


def _bf16(a):
    import torch
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def test_quantize_matches_float32_reference():
    """The quantiser against the same steps done with numpy binary32
    arithmetic and torch's e4m3 conversion: bit-exact codes and scales."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(21)
    T, H = 40, 512
    f = rng.standard_normal((T, H)).astype(np.float32) * np.exp2(
        rng.integers(-20, 20, (T, H // 128, 1)).astype(np.float32)).repeat(128, axis=2).reshape(T, H)
    f[3, :128] = 0.0                                  # an all-zero group
    f[4, 128:256] = 0.0
    f[4, 200] = -3.0                                  # one negative value carries the max
    x = _bf16(f)
    q, sc = oracle.quantize_e4m3(x)
    xf = (x.astype(np.uint32) << 16).view(np.float32).reshape(T, H // 128, 128)
    amax = np.abs(xf).max(axis=2)
    s_ref = (amax / np.float32(448)).astype(np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(amax > 0, np.float32(448) / amax, np.float32(0)).astype(np.float32)
    p = (xf * inv[:, :, None]).astype(np.float32).reshape(T, H)
    q_ref = torch.from_numpy(p).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(sc, s_ref)
    np.testing.assert_array_equal(q, q_ref)


def tiny_group_pair(seed=31, shift=120):
    """Groups g of bf16 values with magnitudes in [2^-5, 1.5) (a sixth of
    them zero, signs mixed) and the same groups times 2^-shift, built by
    lowering the bf16 exponent field, which is exact while the values stay
    normal (shift 120 keeps them in [2^-125, 1.5 * 2^-120), above bf16's
    smallest normal 2^-126). Returns (g, x) as uint16 bit patterns."""
    rng = np.random.default_rng(seed)
    T, H = 8, 256
    mag = np.exp2(rng.uniform(-5, np.log2(1.5), (T, H))).astype(np.float32)
    f = np.where(rng.random((T, H)) < 0.5, -mag, mag)
    f[rng.random((T, H)) < 1 / 6] = 0.0
    g = (f.view(np.uint32) >> 16).astype(np.uint16)        # truncate to bf16: exact values
    exp = (g >> 7) & 0xFF
    x = np.where(exp > 0, g - np.uint16(shift << 7), g).astype(np.uint16)
    assert ((x >> 7) & 0xFF)[exp > 0].min() >= 1           # still normal
    return g, x


def test_quantize_tiny_groups_encode_like_scaled_groups():
    """A group's codes do not depend on a power-of-two scale of the group:
    x * (448 / amax) is the same real number after the scale cancels, so
    groups whose amax is below 448 / FLT_MAX (where binary32's 448 / amax
    overflows) encode exactly like the same groups scaled up by 2^120 (zeros
    stay zero codes, nothing saturates); their scales are binary32's
    amax / 448, subnormal here, as numpy's IEEE division gives them."""
    g, x = tiny_group_pair()
    xf = (x.astype(np.uint32) << 16).view(np.float32).reshape(x.shape[0], -1, 128)
    amax = np.abs(xf).max(axis=2)
    assert (amax < np.float32(448) / np.finfo(np.float32).max).all()   # the overflow range
    qg, _ = oracle.quantize_e4m3(g)
    qx, sx = oracle.quantize_e4m3(x)
    np.testing.assert_array_equal(qx, qg)
    np.testing.assert_array_equal(qx == 0, g == 0)          # zeros, and only zeros, code 0
    assert not (qx == 0x7F).any() and not (qx == 0xFF).any()
    np.testing.assert_array_equal(sx, (amax / np.float32(448)).astype(np.float32))
    assert (sx < np.finfo(np.float32).tiny).all() and (sx > 0).all()


def test_quantize_properties():
    """The largest magnitude of each group encodes to +-448; q * scale is
    within e4m3's half-spacing of x (relative 2^-4 for normal codes); an
    all-zero group gives zero codes and scale 0."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(22)
    f = rng.standard_normal((16, 256)).astype(np.float32)
    f[5, 128:] = 0.0
    x = _bf16(f)
    q, sc = oracle.quantize_e4m3(x)
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    deq = torch.from_numpy(q).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    deq = deq * np.repeat(sc.astype(np.float64), 128, axis=1)
    for t in range(16):
        for g in range(2):
            blk = slice(128 * g, 128 * (g + 1))
            i = np.argmax(np.abs(xf[t, blk]))
            if sc[t, g] == 0:
                assert (q[t, blk] == 0).all()
                continue
            assert q[t, blk][i] in (0x7E, 0xFE)
            err = np.abs(deq[t, blk] - xf[t, blk])
            tol = np.maximum(np.abs(xf[t, blk]) * 2.0 ** -4, 2.0 ** -10 * sc[t, g]) * (1 + 1e-6)
            assert (err <= tol).all()
    assert sc[5, 1] == 0


# ------------------------------------------- low-latency fixed rectangle --

def test_golden_ll_rectangle_example():
    g = load_golden("ll_rectangle_example.txt")
    topk = np.array(g["topk_idx"], np.int64)
    E, M = g["num_experts"][0], g["tokens_per_segment"][0]
    r = oracle.ll_dispatch(None, topk, E, M, 4, hidden=128)
    assert r["output_index"].tolist() == g["cap4_output_index"]
    assert r["recv_count"].tolist() == g["cap4_recv_count"] and not r["overflow"]
    for e in (1, 3, 7):
        assert r["layout_range"][e].ravel().tolist() == g[f"cap4_range_e{e}"]
    assert (r["src_info"][[3, 3, 7, 7, 1], [0, 1, 0, 1, 0]] == 0).all()
    r1 = oracle.ll_dispatch(None, topk, E, M, 1, hidden=128)
    assert r1["output_index"].tolist() == g["cap1_output_index"]
    assert r1["recv_count"].tolist() == g["cap1_recv_count"] and r1["overflow"]


@pytest.mark.parametrize("seed,M", [(0, 16), (1, 7), (2, 1), (3, 50)])
def test_ll_rectangle_against_exact_layout(seed, M):
    """Within each expert the rectangle holds the same rows in the same order
    as the exact (prefix-sum) layout: row - e*cap == exact row - start[e].
    Rows are the quantised token rows, scales column-major per expert;
    src_info and layout_range follow from the token's segment."""
    rng = np.random.default_rng(600 + seed)
    nseg, K, E, H = 6, 4, 12, 256
    T = nseg * M
    topk = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    topk[rng.random(topk.shape) < 0.2] = -1
    x = _bf16(rng.standard_normal((T, H)).astype(np.float32))
    cap = T                                   # the worst case: every token at one expert
    r = oracle.ll_dispatch(x, topk, E, M, cap)
    assert not r["overflow"]
    cnt, _, _ = oracle.layout(topk, E, 1)
    start, total = oracle.scan(cnt)
    _, _, m, oi = oracle.scatter(None, None, topk, start, total)
    np.testing.assert_array_equal(r["recv_count"], cnt)
    valid = topk >= 0
    e_of = np.where(valid, topk, 0)
    want = np.where(valid, oi - start[e_of] + e_of * cap, -1)
    np.testing.assert_array_equal(r["output_index"], want)
    q, sc = oracle.quantize_e4m3(x)
    out = r["out"].reshape(E * cap, -1)
    tt, kk = np.nonzero(valid)
    rows = r["output_index"][tt, kk]
    np.testing.assert_array_equal(out[rows], q[tt])
    ee, jj = rows // cap, rows % cap
    np.testing.assert_array_equal(r["out_scale"][ee, :, jj], sc[tt])
    np.testing.assert_array_equal(r["src_info"].reshape(-1)[rows], tt % M)
    seg_counts = np.zeros((E, nseg), np.int64)
    np.add.at(seg_counts, (e_of[valid], tt // M), 1)
    np.testing.assert_array_equal(r["layout_range"][:, :, 1], seg_counts)
    np.testing.assert_array_equal(r["layout_range"][:, :, 0],
                                  np.cumsum(seg_counts, axis=1) - seg_counts)
    # the rows of segment s within expert e are exactly its layout_range
    for e in range(E):
        for s in range(nseg):
            b, c = r["layout_range"][e, s]
            assert (r["src_info"][e, b:b + c] >= 0).all()
            seg_rows = rows[(ee == e) & (tt // M == s)] % cap
            assert sorted(seg_rows.tolist()) == list(range(b, b + c))


def test_ll_rectangle_overflow_keeps_the_first_rows():
    rng = np.random.default_rng(44)
    T, K, E, M, cap = 64, 3, 4, 8, 20
    topk = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    r = oracle.ll_dispatch(None, topk, E, M, cap, hidden=128)
    big = oracle.ll_dispatch(None, topk, E, M, T, hidden=128)
    assert r["overflow"] and not big["overflow"]
    np.testing.assert_array_equal(r["recv_count"], np.minimum(big["recv_count"], cap))
    # slots within capacity keep their rows (re-based to the smaller stride)
    b = big["output_index"]
    j = np.where(b >= 0, b % T, -1)
    e = np.where(b >= 0, b // T, 0)
    want = np.where((b >= 0) & (j < cap), e * cap + j, -1)
    np.testing.assert_array_equal(r["output_index"], want)
