"""GPU parity of the low-latency (fixed-rectangle) dispatch against the CPU
oracle, through the C ABI: recv_count, layout_range, output_index and
src_info bit-exact; the FP8 codes and fp32 scales of every placed row
bit-exact (the quantisation decision is taken in binary32 on both sides);
rows past an expert's recv_count untouched (poisoned buffers); nothing written
past either end of a buffer (red zones, tests/redzones.py)."""
import zlib

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import permute_ep_layout_amd as epl  # noqa: E402
from permute_ep_layout_amd import workloads  # noqa: E402

import redzones  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
POISON = 0x5A


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    epl.load()


def poisoned(shape, dtype):
    return redzones.poisoned(shape, dtype, POISON, DEV)


@pytest.fixture(autouse=True)
def _red_zones():
    """Every buffer from poisoned() has red zones; a write past either end
    of one fails the test."""
    yield
    redzones.check()


def gpu_ll(topk, x, E, M, cap, stream=None, ws=None):
    T, K = topk.shape
    H = x.shape[1]
    p = epl.Problem.make(T, K, E, 1, H, H // 128)
    if ws is None:
        ws = poisoned(epl.epl_ll_workspace_bytes(p, M), torch.uint8)
    r = dict(out=poisoned((E, cap, H), torch.uint8),
             out_scale=poisoned((E, H // 128, cap), torch.float32),
             recv_count=poisoned(E, torch.int32), src_info=poisoned((E, cap), torch.int32),
             layout_range=poisoned((E, T // M, 2), torch.int32),
             output_index=poisoned((T, K), torch.int32), ws=ws)
    xd = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV).view(torch.bfloat16)
    epl.epl_ll_dispatch(p, M, cap, torch.from_numpy(topk).to(DEV), xd, r["out"], r["out_scale"],
                        r["recv_count"], r["src_info"], r["layout_range"], r["output_index"], ws,
                        stream)
    return r


def check_ll(topk, x, E, M, cap, expect_overflow=False, untouched_sample=64, ws=None):
    """One low-latency dispatch against the oracle. Ids outside [-1, E) must
    act as -1 and make the status EPL_ERANGE. `ws` reuses a workspace."""
    print(f"[ll] T={topk.shape[0]} K={topk.shape[1]} E={E} M={M} cap={cap} H={x.shape[1]}",
          flush=True)
    orc = oracle.default()
    bad_ids = bool(((topk < -1) | (topk >= E)).any())
    clean = np.where((topk < -1) | (topk >= E), -1, topk)
    ref = orc.ll_dispatch(None, clean, E, M, cap, hidden=x.shape[1])
    q, sc = orc.quantize_e4m3(x)
    r = gpu_ll(topk, x, E, M, cap, ws=ws)
    torch.cuda.synchronize()
    st = epl.epl_status(r["ws"])
    assert st == (epl.EPL_ERANGE if bad_ids else
                  epl.EPL_ECAPACITY if expect_overflow else epl.EPL_OK)
    assert ref["overflow"] == expect_overflow
    np.testing.assert_array_equal(r["recv_count"].cpu().numpy(), ref["recv_count"])
    np.testing.assert_array_equal(r["layout_range"].cpu().numpy(), ref["layout_range"])
    oi = r["output_index"].cpu().numpy()
    np.testing.assert_array_equal(oi, ref["output_index"])
    tt, kk = np.nonzero(oi >= 0)
    rows = oi[tt, kk].astype(np.int64)
    ee, jj = rows // cap, rows % cap
    np.testing.assert_array_equal(r["src_info"].view(-1).cpu().numpy()[rows], tt % M)
    rows_d = torch.from_numpy(rows).to(DEV)
    got = r["out"].view(E * cap, -1)[rows_d].cpu().numpy()
    np.testing.assert_array_equal(got, q[tt])
    got_s = r["out_scale"][torch.from_numpy(ee).to(DEV), :, torch.from_numpy(jj).to(DEV)]
    np.testing.assert_array_equal(got_s.cpu().numpy().view(np.uint32), sc[tt].view(np.uint32))
    # rows past recv_count stay untouched
    rc = ref["recv_count"]
    rng = np.random.default_rng(0)
    free = [(e, j) for e in rng.permutation(E)[:untouched_sample] for j in (rc[e], cap - 1)
            if j < cap and j >= rc[e]]
    for e, j in free:
        assert (r["out"][e, j] == POISON).all()
        assert (r["src_info"][e, j:j + 1].view(torch.uint8) == POISON).all()
    return r, ref


def _topk(rng, T, K, E, drop=0.0):
    topk = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    if drop:
        topk[rng.random(topk.shape) < drop] = -1
    return topk


def _x(rng, T, H, spread=True):
    f = rng.standard_normal((T, H)).astype(np.float32)
    if spread:   # groups of very different magnitude, and tiny values next to big ones
        f *= np.exp2(rng.integers(-30, 30, (T, H // 128, 1))).repeat(128, axis=2).reshape(T, H)
        f[:, ::37] *= 1e-4
    return workloads.fp32_to_bf16_bits(f)


def test_dsv3_ll_full_size():
    """The DeepSeek-V3-shaped batch as 32 segments of 128 tokens, every
    expert's rectangle sized for the worst case (4096 rows)."""
    w = workloads.get("dsv3_ll")
    inp = workloads.make_inputs(w)
    M = w.ll_segment
    check_ll(inp["topk_idx"], inp["x"], w.num_experts, M, w.num_tokens)


LL_CASES = [
    # (name, segments, M, K, E, H, cap, drop)
    ("ragged_m7", 6, 7, 4, 12, 256, 42, 0.2),
    ("h128", 5, 32, 3, 16, 128, 160, 0.0),
    ("h9216", 4, 16, 2, 8, 9216, 64, 0.1),
    ("h16512_two_passes", 4, 16, 2, 8, 16512, 64, 0.1),
    ("k1", 8, 64, 1, 32, 512, 512, 0.0),
    ("prime_m", 3, 127, 8, 64, 256, 381, 0.05),
    ("e1_all_one_expert", 4, 50, 2, 1, 256, 400, 0.3),
]


@pytest.mark.parametrize("case", LL_CASES, ids=[c[0] for c in LL_CASES])
def test_ll_shapes(case):
    name, nseg, M, K, E, H, cap, drop = case
    rng = np.random.default_rng(zlib.crc32(name.encode()))   # stable across processes
    T = nseg * M
    topk = _topk(rng, T, K, E, drop) if K <= E else rng.integers(-1, E, (T, K)).astype(np.int64)
    check_ll(topk, _x(rng, T, H), E, M, cap)


# Decode-sized batches (at most 4096 slots and at most 14336 (segment,
# expert) counters) are dispatched in one launch, with 2 slots per thread up
# to 2048 slots and 4 above; these cases sit on both sides of those limits,
# and one has rows longer than a workgroup's pass.
LL_DECODE_CASES = [
    # (name, segments, M, K, E, H, cap, drop)
    ("decode_dsv3_t128", 1, 128, 8, 256, 7168, 128, 0.0),
    ("decode_dsv3_8_segments", 8, 32, 8, 256, 7168, 256, 0.05),
    ("decode_slot_limit_2048", 2, 128, 8, 256, 1024, 256, 0.1),
    ("decode_wide_2056_slots", 1, 257, 8, 256, 1024, 257, 0.1),
    ("decode_wide_limit_4096", 4, 128, 8, 256, 7168, 512, 0.05),
    ("decode_wide_limit_plus_one_token", 1, 513, 8, 256, 1024, 513, 0.1),
    ("decode_counter_limit_14336", 56, 2, 4, 256, 256, 112, 0.0),
    ("decode_counter_limit_plus_one_segment", 57, 2, 4, 256, 256, 114, 0.0),
    ("decode_k16_two_passes", 2, 16, 16, 64, 16512, 32, 0.1),
    ("decode_e1000", 2, 64, 6, 1000, 384, 128, 0.0),
    ("decode_k64_2048_slots", 1, 32, 64, 128, 256, 32, 0.1),
]


# Above the decode size, up to 64 layout blocks the cast kernel sums the
# block offsets itself (no reduce launch); more blocks keep the reduce. With
# M = 1 every token is a layout block of its own.
LL_BLOCK_CASES = [
    # (name, segments, M, K, E, H, cap, drop)
    ("summed_limit_64_blocks", 64, 1, 40, 64, 256, 64, 0.1),
    ("reduce_65_blocks", 65, 1, 40, 64, 256, 65, 0.1),
    ("reduce_600_blocks_m7", 600, 7, 2, 16, 128, 4200, 0.1),
    ("summed_dsv3_t1024_tight_cap", 8, 128, 8, 256, 7168, 40, 0.0),
    # the widest expert count and the largest top-k above the decode size
    ("e2048_40_segments_tight_cap", 40, 128, 8, 2048, 256, 28, 0.1),
    ("k64_16_segments", 16, 64, 64, 512, 128, 192, 0.1),
]


@pytest.mark.parametrize("case", LL_BLOCK_CASES, ids=[c[0] for c in LL_BLOCK_CASES])
def test_ll_block_offsets_summed_or_reduced(case):
    name, nseg, M, K, E, H, cap, drop = case
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    T = nseg * M
    topk = _topk(rng, T, K, E, drop)
    over = bool((np.bincount(topk[topk >= 0], minlength=E) > cap).any())
    check_ll(topk, _x(rng, T, H), E, M, cap, expect_overflow=over)


@pytest.mark.parametrize("case", LL_DECODE_CASES, ids=[c[0] for c in LL_DECODE_CASES])
def test_ll_decode_sizes(case):
    name, nseg, M, K, E, H, cap, drop = case
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    T = nseg * M
    check_ll(_topk(rng, T, K, E, drop), _x(rng, T, H), E, M, cap)


@pytest.mark.parametrize("T", [128, 1024])
def test_ll_overflow_and_bad_ids_then_reset(T):
    """DeepSeek-V3-shaped batches (128 tokens: one launch; 1024 tokens: the
    cast kernel summing its block offsets) with 2 rows per expert: the
    capacity bit, the first rows kept; then ids outside [-1, E) in the same
    workspace: the id bit; then clean ids: the status clears."""
    rng = np.random.default_rng(41)
    K, E, H, M = 8, 256, 7168, 128
    topk, x = _topk(rng, T, K, E), _x(rng, T, H)
    r, _ = check_ll(topk, x, E, M, 2, expect_overflow=True)
    bad = topk.copy()
    bad[3, 1] = E
    bad[77, 0] = 1 << 40
    bad[100, 7] = -5
    check_ll(bad, x, E, M, T, ws=r["ws"])
    check_ll(topk, x, E, M, T, ws=r["ws"])


def test_ll_decode_receive_side_local_ids():
    """128 tokens of the DeepSeek-V3 batch seen by one receiver: local ids of
    its 8 experts, -1 elsewhere (most tokens select none of them)."""
    w = workloads.get("dsv3_ll")
    inp = workloads.make_inputs(w)
    El, r, T = 8, 5, 128
    topk = inp["topk_idx"][:T]
    mine = (topk >= r * El) & (topk < (r + 1) * El)
    local = np.ascontiguousarray(np.where(mine, topk - r * El, -1))
    check_ll(local, np.ascontiguousarray(inp["x"][:T]), El, T, T)


@pytest.mark.parametrize("seed", range(24))
def test_ll_random_shape_sweep(seed):
    """24 seeded random low-latency problems against the oracle: segment
    sizes and counts that land in the one-launch kernel (2 or 4 slots per
    thread), the cast kernel summing its block offsets, or the reduce launch;
    top-k up to 16, drops, receive-side-like sparse ids, rectangles from
    tight (overflowing) to the worst case, hidden widths from 128 to 8192."""
    rng = np.random.default_rng(11000 + seed)
    K = int(rng.integers(1, 17))
    E = int(rng.choice([K, 16, 64, 256]))
    M = int(rng.choice([1, 7, 32, 128, 200]))
    nseg = int(np.exp(rng.uniform(0, np.log(max(2, 6000 // M)))))
    T = M * max(1, nseg)
    H = 128 * int(rng.integers(1, 65))
    drop = float(rng.choice([0.0, 0.1, 0.85]))
    worst = M * (T // M)
    cap = int(rng.choice([worst, max(1, worst // 4), max(1, T * K // max(E, 1) // 2)]))
    print(f"[ll] sweep seed={seed} T={T} M={M} K={K} E={E} H={H} cap={cap} drop={drop}",
          flush=True)
    topk = _topk(rng, T, K, E, drop) if K <= E else rng.integers(-1, E, (T, K)).astype(np.int64)
    over = bool((np.bincount(topk[topk >= 0], minlength=E) > cap).any())
    check_ll(topk, _x(rng, T, H), E, M, cap, expect_overflow=over, untouched_sample=16)


def test_ll_receive_side_local_ids():
    """One receiver's rectangle: local ids (8 experts), -1 elsewhere."""
    w = workloads.get("dsv3_ll")
    inp = workloads.make_inputs(w)
    El, r = 8, 5
    topk = inp["topk_idx"]
    mine = (topk >= r * El) & (topk < (r + 1) * El)
    local = np.ascontiguousarray(np.where(mine, topk - r * El, -1))
    check_ll(local, inp["x"], El, w.ll_segment, w.num_tokens)


def test_ll_overflow_is_flagged_and_keeps_the_first_rows():
    rng = np.random.default_rng(3)
    topk = _topk(rng, 256, 4, 8)
    check_ll(topk, _x(rng, 256, 256), 8, 64, 100, expect_overflow=True)


def test_ll_zero_tokens_and_all_invalid():
    rng = np.random.default_rng(4)
    check_ll(np.zeros((0, 4), np.int64), np.zeros((0, 256), np.uint16), 8, 16, 32)
    check_ll(-np.ones((64, 4), np.int64), _x(rng, 64, 256), 8, 16, 32)


def test_ll_zero_groups_and_exact_powers():
    """All-zero groups (scale 0, codes 0), groups whose values are exact
    powers of two (codes hit exact binary32 products), and a negative
    group maximum."""
    rng = np.random.default_rng(5)
    T, H = 64, 512
    f = rng.standard_normal((T, H)).astype(np.float32)
    f[::3, :128] = 0.0
    f[1::3, 128:256] = np.exp2(rng.integers(-10, 10, (len(range(1, T, 3)), 128))).astype(np.float32)
    f[2::3, 256:384] = -np.abs(f[2::3, 256:384]) * 1000
    x = workloads.fp32_to_bf16_bits(f)
    check_ll(_topk(rng, T, 4, 16), x, 16, 16, 64)


def test_ll_tiny_groups_encode_like_scaled_groups():
    """Groups of bf16 values far below 1e-36 mixed with zeros, where
    binary32's 448 / amax overflows: the kernel's codes equal the oracle's
    (and those of the same groups scaled up by 2^120), zeros stay zero codes,
    and the scales are binary32's subnormal amax / 448 -- also for bf16
    subnormal values and groups of a single smallest subnormal."""
    from test_oracle_pins import tiny_group_pair

    g, x = tiny_group_pair(seed=33)
    x = x.copy()
    x[0, :128] = 0x0001                                 # the smallest bf16 subnormal, 2^-133
    x[1, 128:256] = 0x0000
    x[1, 130] = 0x8003                                  # one negative subnormal in zeros
    x[2, :128] = np.where(np.arange(128) % 2, 0x0040, 0x0000).astype(np.uint16)   # 2^-127
    q, sc = oracle.default().quantize_e4m3(x)
    qg, _ = oracle.default().quantize_e4m3(g)
    np.testing.assert_array_equal(q[3:], qg[3:])
    assert not (q == 0x7F).any() and q[0, 0] == 0x7E and q[1, 130] == 0xFE
    rng = np.random.default_rng(34)
    T = x.shape[0]
    check_ll(_topk(rng, T, 3, 8), x, 8, 4, T)


def test_ll_non_finite_values_encode_like_the_oracle():
    """NaN and +-Inf in the token rows: a group's amax skips NaN (a group of
    NaNs only gets scale 0), an Inf makes the scale Inf and the factor 0, and
    every NaN that reaches the encoder (a NaN value, or Inf * 0) is the code
    0x7F; codes and scales bit-exact against the oracle."""
    rng = np.random.default_rng(31)
    nseg, M, K, E, H = 4, 32, 4, 16, 512
    T = nseg * M
    topk = _topk(rng, T, K, E)
    x = _x(rng, T, H, spread=False)
    specials = np.array([0x7FC0, 0xFFC0, 0x7F80, 0xFF80], np.uint16)   # +-NaN, +-Inf
    hit = rng.random(x.shape) < 0.004
    x[hit] = specials[rng.integers(0, 4, int(hit.sum()))]
    x[5, 128:256] = 0x7FC0          # a group of NaNs only
    x[9, 0:128] = 0x0000            # an all-zero group
    x[9, 7] = 0xFF80                # ... but for one -Inf
    q, sc = oracle.default().quantize_e4m3(x)
    assert (q == 0x7F).any() and np.isinf(sc).any() and sc[5, 1] == 0.0
    check_ll(topk, x, E, M, T)


def test_ll_side_stream_and_repeat_is_deterministic():
    rng = np.random.default_rng(6)
    topk, x = _topk(rng, 512, 6, 32, 0.1), _x(rng, 512, 1024)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        a = gpu_ll(topk, x, 32, 128, 512, stream=s)
        b = gpu_ll(topk, x, 32, 128, 512, stream=s)
    s.synchronize()
    for key in ("recv_count", "layout_range", "output_index"):
        assert torch.equal(a[key], b[key]), key
    oi = a["output_index"].view(-1)
    rows = oi[oi >= 0].long()
    assert torch.equal(a["out"].view(32 * 512, -1)[rows], b["out"].view(32 * 512, -1)[rows])


def test_ll_rows_feed_the_combine():
    """The rectangle's output_index drives epl_combine over a bf16 [E*cap, H]
    expert-output buffer (rows of the rectangle); the sums match the fp64
    oracle within 1e-5 of sum |w v|."""
    rng = np.random.default_rng(8)
    nseg, M, K, E, H = 4, 64, 6, 16, 512
    T, cap = nseg * M, nseg * M
    topk = _topk(rng, T, K, E, 0.15)
    x = _x(rng, T, H, spread=False)
    wt = rng.uniform(0.05, 1.0, (T, K)).astype(np.float32)
    r = gpu_ll(topk, x, E, M, cap)
    oi = r["output_index"]
    # expert output = the token's own bf16 row, placed at its rectangle row
    eo = torch.zeros((E * cap, H), dtype=torch.bfloat16, device=DEV)
    flat = oi.view(-1).long()
    sel = flat >= 0
    tok = torch.arange(T, device=DEV).repeat_interleave(K)[sel]
    xd = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV).view(torch.bfloat16)
    eo[flat[sel]] = xd[tok]
    p = epl.Problem.make(T, K, E, 1, H, 0)
    y = poisoned((T, H), torch.float32)
    epl.epl_combine(p, eo, E * cap, oi, torch.from_numpy(wt).to(DEV), epl.EPL_OUT_F32, y, r["ws"])
    torch.cuda.synchronize()
    assert epl.epl_status(r["ws"]) == epl.EPL_OK
    orc = oracle.default()
    oi_h = oi.cpu().numpy()
    valid = oi_h >= 0
    compact = np.full(oi_h.shape, -1, np.int32)
    compact[valid] = np.arange(int(valid.sum()), dtype=np.int32)
    rows = np.repeat(x, K, axis=0)[valid.ravel()]
    y_ref = orc.combine(rows, compact, wt)
    bound = orc.combine(rows & np.uint16(0x7FFF), compact, np.abs(wt))
    d = np.abs(y.cpu().numpy().astype(np.float64) - y_ref)
    assert (d <= 1e-5 * bound).all()
