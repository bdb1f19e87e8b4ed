"""The seeded input generator: determinism and distribution sanity (no GPU)."""
import numpy as np
import pytest
import torch

import workloads as W


def test_table_shapes():
    c = W.CONFIGS
    assert (c["tiny"].num_experts, c["tiny"].top_k, c["tiny"].hidden, c["tiny"].intermediate) == (8, 2, 256, 512)
    assert (c["mixtral"].num_tokens, c["mixtral"].hidden, c["mixtral"].intermediate) == (4096, 4096, 14336)
    for t in (1, 8, 32, 128):
        k = c[f"ep_decode_T{t}"]
        assert (k.num_tokens, k.num_experts, k.pool, k.top_k, k.hidden, k.intermediate) == (t, 96, 384, 6, 7168, 3072)
    s = c["static_capacity"]
    assert (s.num_tokens, s.top_k, s.num_experts, s.hidden, s.intermediate, s.cap) == (2048, 8, 128, 2048, 768, 16384)


def test_deterministic():
    cfg = W.CONFIGS["tiny"]
    a, b = W.make_inputs(cfg, 3), W.make_inputs(cfg, 3)
    for k in a:
        assert torch.equal(a[k].view(torch.uint8) if a[k].dtype == torch.bfloat16 else a[k],
                           b[k].view(torch.uint8) if b[k].dtype == torch.bfloat16 else b[k])
    c = W.make_inputs(cfg, 4)
    assert not torch.equal(a["topk_ids"], c["topk_ids"])


@pytest.mark.parametrize("name", ["tiny", "ep_decode_T128", "ep_prefill_T2048_zipf", "static_capacity"])
def test_routing_sane(name):
    cfg = W.CONFIGS[name]
    ids, w = W.make_routing(cfg, 0)
    T, K = cfg.num_tokens, cfg.top_k
    assert ids.shape == (T, K) and w.shape == (T, K)
    assert ids.dtype == torch.int32 and w.dtype == torch.float32
    assert int(ids.min()) >= 0 and int(ids.max()) < cfg.pool
    srt = torch.sort(ids, dim=1).values
    assert bool((srt[:, 1:] != srt[:, :-1]).all())        # distinct per token
    np.testing.assert_allclose(w.sum(1).numpy(), 1.0, rtol=1e-5)
    assert bool((w > 0).all())


def test_softmax_topk_picks_largest():
    cfg = W.CONFIGS["tiny"]
    ids, w = W.make_routing(cfg, 1)
    # weights are sorted descending because the selected logits are
    assert bool((w[:, 0] >= w[:, 1]).all())


def test_zipf_rank_frequencies():
    cfg = W.CONFIGS["ep_prefill_T8192_zipf"]
    ids, _ = W.make_routing(cfg, 0)
    freq = torch.bincount(ids.reshape(-1).long(), minlength=384).double() / ids.shape[0]
    top = torch.sort(freq, descending=True).values
    # With s = 1.2 the most popular expert is in nearly every token's top-6 and
    # the tail is thin.
    assert float(top[0]) > 0.8
    assert float(top[-50:].mean()) < 0.01
    u_ids, _ = W.make_routing(W.CONFIGS["ep_prefill_T8192"], 0)
    ufreq = torch.bincount(u_ids.reshape(-1).long(), minlength=384).double() / u_ids.shape[0]
    assert float(ufreq.max()) < 0.03 and float(ufreq.min()) > 0.008   # ~6/384 each


def test_static_token_counts():
    tv = W.make_static_token_counts(0)
    assert len(tv) == 50 and min(tv) >= 1 and max(tv) <= 2048
    assert tv == W.make_static_token_counts(0)


def test_weight_scale():
    cfg = W.CONFIGS["tiny"]
    wgu, wd = W.make_weights(cfg, 0)
    assert wgu.shape == (8, 1024, 256) and wd.shape == (8, 256, 512)
    assert abs(float(wgu.float().std()) - 256 ** -0.5) < 0.01 * 256 ** -0.5 * 10
    assert abs(float(wd.float().std()) - 512 ** -0.5) < 0.01 * 512 ** -0.5 * 10
