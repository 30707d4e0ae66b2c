"""Host checks of the synthetic-layer generator (no method arithmetic lives there)."""
import numpy as np

from datagen import block_mask, get_config
from datagen.video_layers import budgets


def test_uniform_local_mask_rows_hold_k_blocks_with_the_diagonal():
    cfg = get_config("small_bf16")
    m = block_mask(cfg)
    assert m.shape == (1, cfg.num_blocks, cfg.num_blocks)
    assert (m[0].sum(axis=1) == cfg.blocks_per_row).all()
    assert (np.diagonal(m[0]) == 1).all()


def test_budget_masks_follow_their_budgets():
    cfg = get_config("small_budget_bf16")
    kk = budgets(cfg)
    m = block_mask(cfg)
    assert m.shape == (cfg.heads, cfg.num_blocks, cfg.num_blocks)
    assert (m.sum(axis=2) == kk).all()                      # row b of head h keeps k[h][b]
    assert (np.diagonal(m, axis1=1, axis2=2) == 1).all()    # the nearest block is itself
    assert kk.min() >= 1 and kk.max() <= cfg.num_blocks
    assert abs(kk.mean() - cfg.blocks_per_row) < 0.5        # mean budget is k
    assert kk.mean(axis=1).max() > 1.5 * kk.mean(axis=1).min()   # heads differ
    # nested: a larger budget of the same query block extends the smaller one
    order_ok = True
    for b in range(cfg.num_blocks):
        rows = sorted(range(cfg.heads), key=lambda h: kk[h, b])
        for h0, h1 in zip(rows, rows[1:]):
            order_ok &= bool(((m[h0, b] <= m[h1, b])).all())
    assert order_ok


def test_budgets_are_seeded():
    cfg = get_config("hunyuan13b_budget_bf16")
    a, b = budgets(cfg), budgets(cfg)
    assert (a == b).all() and a.shape == (cfg.heads, cfg.num_blocks)
    assert abs(a.mean() - cfg.blocks_per_row) < 0.5
