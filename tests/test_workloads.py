"""The seeded input generator: reproducible, and shaped like each workload."""
import numpy as np
import pytest

from permute_ep_layout_amd import workloads


def test_same_seed_same_bytes():
    w = workloads.get("small").with_(num_tokens=256, hidden=256)
    a, b = workloads.make_inputs(w), workloads.make_inputs(w)
    for key in ("topk_idx", "topk_weights", "x"):
        assert a[key].tobytes() == b[key].tobytes()
    c = workloads.make_inputs(w.with_(seed=w.seed + 1))
    assert a["topk_idx"].tobytes() != c["topk_idx"].tobytes()


def test_tensor_streams_are_independent():
    """Changing the routing recipe must not change x (its own stream)."""
    w = workloads.get("tiny")
    assert workloads.make_x(w).tobytes() == workloads.make_x(w.with_(drop_rate=0.3)).tobytes()


@pytest.mark.parametrize("name", ["tiny", "small", "dsv3", "large"])
def test_uniform_routing_distinct_and_in_range(name):
    w = workloads.get(name)
    topk = workloads.make_topk(w)
    assert topk.shape == (w.num_tokens, w.num_topk) and topk.dtype == np.int64
    valid = topk >= 0
    assert (topk[valid] < w.num_experts).all() and (topk[~valid] == -1).all()
    srt = np.sort(np.where(valid, topk, -np.arange(1, w.num_topk + 1)), axis=1)
    assert (np.diff(srt, axis=1) != 0).all(), "experts within a token must be distinct"
    if w.drop_rate == 0.0:
        assert valid.all()
    if w.drop_rate == 0.0 and w.num_tokens * w.num_topk >= 100 * w.num_experts:
        # uniform: every expert's share is close to K/E of the tokens
        cnt = np.bincount(topk.ravel(), minlength=w.num_experts)
        mean = w.num_tokens * w.num_topk / w.num_experts
        assert cnt.min() > 0.5 * mean and cnt.max() < 1.5 * mean


def test_small_drop_rate():
    w = workloads.get("small")
    topk = workloads.make_topk(w)
    rate = (topk < 0).mean()
    assert abs(rate - 0.05) < 0.005


def test_skew_has_cold_experts_and_a_hot_one():
    w = workloads.get("skew")
    topk = workloads.make_topk(w)
    cnt = np.bincount(topk.ravel(), minlength=w.num_experts)
    cold = workloads.cold_experts(w)
    assert cold.size == 8 and (cnt[cold] == 0).all()
    assert (cnt == 0).sum() == 8
    assert cnt.max() > 0.8 * w.num_tokens        # the hottest expert is in most tokens
    srt = np.sort(topk, axis=1)
    assert (np.diff(srt, axis=1) != 0).all()


@pytest.mark.parametrize("name", ["tiny", "small", "skew"])
def test_weights_softmax_over_valid(name):
    w = workloads.get(name)
    topk = workloads.make_topk(w)
    wt = workloads.make_weights(w, topk)
    assert wt.dtype == np.float32 and wt.shape == topk.shape
    valid = topk >= 0
    assert (wt[~valid] == 0).all() and (wt[valid] > 0).all()
    s = wt.astype(np.float64).sum(axis=1)
    has = valid.any(axis=1)
    assert np.abs(s[has] - 1).max() < 1e-6


def test_x_is_bf16_of_standard_normal():
    w = workloads.get("small").with_(num_tokens=512)
    x = workloads.make_x(w)
    assert x.dtype == np.uint16 and x.shape == (512, w.hidden)
    f = (x.astype(np.uint32) << 16).view(np.float32)
    assert abs(f.mean()) < 0.01 and abs(f.std() - 1) < 0.01


def test_x_row_subset_matches_full():
    w = workloads.get("small").with_(num_tokens=3000, hidden=1024)
    full = workloads.make_x(w)
    rows = np.array([2999, 0, 1500, 17, 17])
    np.testing.assert_array_equal(workloads.make_x(w, rows=rows), full[rows])


def test_fp32_to_bf16_rounding():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -8 + 2 ** -20],
                 dtype=np.float32)
    got = workloads.fp32_to_bf16_bits(f)
    assert [hex(v) for v in got] == ["0x3f80", "0x3f80", "0x3f82", "0xc020", "0x3f81"]


def test_scales():
    w = workloads.get("dsv3").with_(num_tokens=300)
    s = workloads.make_scales(w)
    assert s.shape == (300, 56) and s.dtype == np.float32
    assert s.min() >= 0.01 and s.max() <= 1.0
    assert workloads.make_scales(workloads.get("small")) is None


def test_receive_side_batch():
    """dsv3_recv: every kept token picks at least one of the rank's experts;
    ids are local or -1; local slots average K*El/Eg / P(hit) per token."""
    w = workloads.get("dsv3_recv")
    topk = workloads.make_topk(w)
    assert topk.shape == (29765, 8) and topk.dtype == np.int64
    valid = topk >= 0
    assert valid.any(axis=1).all()
    assert (topk[valid] < 8).all() and (topk[~valid] == -1).all()
    srt = np.sort(np.where(valid, topk, -np.arange(1, 9)), axis=1)
    assert (np.diff(srt, axis=1) != 0).all()
    p_hit = 1.0 - np.prod([(248 - i) / (256 - i) for i in range(8)])
    assert abs(valid.sum(axis=1).mean() - 8 * 8 / 256 / p_hit) < 0.01
    cnt = np.bincount(topk[valid], minlength=8)
    assert cnt.min() > 0.95 * cnt.mean() and cnt.max() < 1.05 * cnt.mean()
    # the sender's weights: positive on local slots, 0 elsewhere, sum <= 1
    wt = workloads.make_weights(w, topk)
    assert (wt[~valid] == 0).all() and (wt[valid] > 0).all()
    assert wt.astype(np.float64).sum(axis=1).max() <= 1.0 + 1e-6
    # the same draws as the send side: a global row with all K experts valid
    g = workloads._received_global(w)
    np.testing.assert_array_equal(np.where(valid, topk, -1), np.where(g < 8, g, -1))
