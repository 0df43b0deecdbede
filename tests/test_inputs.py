"""Seeded generator: determinism and the layout conventions it promises."""
import hashlib

import numpy as np
import torch

from prefill_decode_hybrid_amd import inputs


def _digest(b):
    h = hashlib.sha256()
    for t in (b.q_prefill, b.q_decode, b.k_pool, b.v_pool, b.page_table_prefill,
              b.page_table_decode, b.context_lens):
        if t is not None:
            h.update(t.contiguous().view(torch.uint8).numpy().tobytes() if t.dtype != torch.int32
                     else t.numpy().tobytes())
    return h.hexdigest()


SMALL = dict(name="small", dtype="bf16", num_q_heads=8, num_kv_heads=2, head_dim=32,
             chunk_len=40, chunk_offset=25, decode_lens=("loguniform", 6, 5, 300),
             contiguous=False, k_outlier_frac=0.05)


def test_deterministic_per_seed():
    a, b, c = inputs.make_batch(SMALL, 0), inputs.make_batch(SMALL, 0), inputs.make_batch(SMALL, 1)
    assert _digest(a) == _digest(b)
    assert _digest(a) != _digest(c)


def test_layout_conventions():
    b = inputs.make_batch(SMALL, 3)
    B = inputs.PAGE_SIZE
    lp = b.chunk_offset + b.chunk_len
    assert b.page_table_prefill.numel() == -(-lp // B)
    # every page is used once, the guard page is all NaN
    used = torch.cat([b.page_table_prefill] + [b.page_table_decode[i, :-(-int(L) // B)]
                                               for i, L in enumerate(b.context_lens)])
    assert sorted(used.tolist()) == list(range(b.guard_page))
    assert torch.isnan(b.k_pool[b.guard_page].float()).all()
    # table padding points at the guard page; tails are NaN, visible keys finite
    for i, L in enumerate(b.context_lens.tolist()):
        n = -(-L // B)
        assert (b.page_table_decode[i, n:] == b.guard_page).all()
        last = int(b.page_table_decode[i, n - 1])
        tail = L - (n - 1) * B
        assert torch.isfinite(b.k_pool[last, :tail].float()).all()
        assert torch.isnan(b.v_pool[last, tail:].float()).all()
    # outliers: exactly round(frac * rows) K rows scaled by 8
    assert b.outlier_rows == round(0.05 * (lp + int(b.context_lens.sum())) * b.num_kv_heads)


def test_config_lengths_rules():
    rng_b = inputs.make_batch(2, 0, with_prefill=False)
    lens = rng_b.context_lens.numpy()
    assert len(lens) == 32 and lens.min() >= 1024 and lens.max() <= 4096
    c1 = inputs.make_batch(1, 0)
    assert c1.context_lens.tolist() == [37, 100, 256, 511]
    assert c1.dtype == torch.float32 and c1.sm_scale == 0.125
    assert c1.page_table_prefill.tolist() == list(range(8))  # contiguous: sequential pages


def test_loguniform_rule_bounds():
    rng = np.random.default_rng(0)
    x = inputs._draw_lengths(("loguniform", 10000, 128, 32768), rng)
    assert x.min() >= 128 and x.max() <= 32768
    # median of a log-uniform on [128, 32768] is 2048
    assert 1700 < np.median(x) < 2500
