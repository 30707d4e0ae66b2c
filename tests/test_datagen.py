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


def test_key_block_masks_keep_k_key_blocks_around_the_query_block():
    import dataclasses
    for rule in ("centre", "reach"):
        cfg = dataclasses.replace(get_config("small_sub32_bf16"), local_rule=rule)
        m = block_mask(cfg)[0]
        S, B = cfg.kblock, cfg.block
        assert m.shape == (cfg.num_blocks, cfg.num_key_blocks)
        assert (m.sum(axis=1) == cfg.blocks_per_row).all()
        # the query block's own keys are the nearest: all B/S of its key blocks are kept
        for b in range(cfg.num_blocks):
            own = range(b * B // S, min(cfg.num_key_blocks, (b + 1) * B // S))
            assert all(m[b, kb] for kb in own), (rule, b)


def test_reach_rule_covers_the_query_block_ends():
    """With 32-key blocks and query blocks of 1.6 raster rows (80 wide, as in the 13B-class
    latent), the reach rule keeps key blocks next to both ends of the query block; the
    centre rule keeps a ball around its middle that reaches less far along it."""
    import dataclasses
    from datagen.video_layers import _token_coords
    base = dataclasses.replace(get_config("small_sub32_bf16"), frames=4, height=24, width=80)
    cen, rea = (block_mask(dataclasses.replace(base, local_rule=r))[0] for r in ("centre", "reach"))
    xyz = _token_coords(base) * np.array([base.local_scale, 1.0, 1.0])
    S, B = base.kblock, base.block

    def worst_reach(m):
        # largest distance from a query token to the nearest kept key, over all queries
        worst = 0.0
        for b in range(0, base.num_blocks, 7):
            keys = np.concatenate([np.arange(kb * S, (kb + 1) * S) for kb in np.nonzero(m[b])[0]])
            q = xyz[b * B:(b + 1) * B]
            d = ((q[:, None, :] - xyz[keys][None, :, :]) ** 2).sum(axis=2).min(axis=1)
            worst = max(worst, float(d.max()))
        return worst

    def mean_kernel(m, ell=6.0):
        # mean over queries of the kept Gaussian-kernel mass of 3D distance
        tot = 0.0
        for b in range(0, base.num_blocks, 7):
            keys = np.concatenate([np.arange(kb * S, (kb + 1) * S) for kb in np.nonzero(m[b])[0]])
            q = xyz[b * B:(b + 1) * B]
            d2 = ((q[:, None, :] - xyz[keys][None, :, :]) ** 2).sum(axis=2)
            tot += float(np.exp(-d2 / (2 * ell * ell)).sum())
        return tot

    assert worst_reach(rea) <= worst_reach(cen)
    assert mean_kernel(rea) > mean_kernel(cen)


def test_key_offset_shifts_the_centres_and_draws_nothing():
    import dataclasses
    from datagen.video_layers import head_tensors, to_f32
    base = get_config("small_bf16")
    a = head_tensors(base, 1)
    b = head_tensors(dataclasses.replace(base, key_offset=3.0), 1)
    assert (a["V"] == b["V"]).all() and (a["k_component"] == b["k_component"]).all()
    ka, kb = to_f32(base, a["K"]), to_f32(base, b["K"])
    # the same noise, shifted by 3 in every coordinate (up to the bf16 rounding of both)
    assert np.abs((kb - ka) - 3.0).max() <= 2 ** -8 * (np.abs(kb).max() + np.abs(ka).max())
    assert abs(float(kb.mean()) - float(ka.mean()) - 3.0) < 1e-2


def test_generator_is_deterministic_and_per_head():
    """Same seed, same bytes; a head generated alone equals that head of the whole layer."""
    from datagen import make_layer
    cfg = get_config("small_bf16")
    a = make_layer(cfg, threads=2)
    b = make_layer(cfg, threads=8)
    for k in ("Q", "K", "V", "mask", "cache_init"):
        assert np.array_equal(a[k], b[k]), k
    one = make_layer(cfg, heads=[5], threads=1)
    for k in ("Q", "K", "V", "cache_init"):
        assert np.array_equal(one[k][0], a[k][5]), k
    assert not np.array_equal(a["K"][4], a["K"][5])       # heads draw their own streams
