"""Host checks of the stream-K schedule (the kernel's own code, exported as
gemm_streamk_pieces) and of forced stream-K plans (no GPU).

"Hopper Support in Triton", the SplitK / stream-K slides: the K steps of all
output tiles are dealt out evenly to a fixed set of workgroups, and the tiles
cut between workgroups are summed from their parts.  The schedule must cover
every (tile, K step) exactly once, number each tile's parts 0..n-1 in K
order, and give every part of a cut tile its own workspace slot."""
import pytest

import dense_tiled_gemm_02_amd as g

from test_abi import fake_gfx950, plan


CASES = [(1, 1, 1), (1, 64, 7), (3, 10, 30), (144, 64, 256), (100, 64, 256), (7, 5, 3), (400, 64, 256),
         (2, 100, 9), (13, 17, 221), (64, 16, 256), (576, 64, 256), (5, 33, 64)]


@pytest.mark.parametrize("tiles,nkt,W", CASES)
def test_schedule_covers_every_step_once_and_numbers_parts(tiles, nkt, W):
    seen = {}
    parts = {}
    slots = {}
    for w in range(W):
        pieces = g.gemm_streamk_pieces(tiles, nkt, W, w)
        lo, hi = w * tiles * nkt // W, (w + 1) * tiles * nkt // W
        it = lo
        for (t, k0, k1, part, nparts, slot) in pieces:
            assert 0 <= t < tiles and 0 <= k0 < k1 <= nkt
            assert t * nkt + k0 == it                  # pieces are contiguous, in order
            it = t * nkt + k1
            for k in range(k0, k1):
                assert (t, k) not in seen
                seen[(t, k)] = w
            parts.setdefault(t, []).append((k0, k1, part, nparts))
            if nparts == 1:
                assert (k0, k1, slot) == (0, nkt, -1)
            else:
                assert 0 <= slot < 2 * W and slot not in slots, (t, part, slot)
                slots[slot] = (t, part)
        assert it == hi
        # a range has at most two cut pieces: its first and its last
        assert sum(1 for p in pieces if p[4] > 1) <= 2
    assert len(seen) == tiles * nkt
    for t, ps in parts.items():
        ps.sort()
        n = ps[0][3]
        assert [p[2] for p in ps] == list(range(n)) and all(p[3] == n for p in ps)
        assert ps[0][0] == 0 and ps[-1][1] == nkt
        assert all(a[1] == b[0] for a, b in zip(ps, ps[1:]))


def test_schedule_rejects_bad_arguments():
    for args in ((0, 4, 1, 0), (4, 4, 0, 0), (4, 4, 2, 2), (1, 4, 5, 0), (-1, 4, 1, 0), (65536, 1024, 64, 0)):
        with pytest.raises(g.GemmError) as e:
            g.gemm_streamk_pieces(*args)
        assert e.value.status == g.GEMM_ERR_INVALID_ARG, args


def test_planner_keeps_stream_k_forced_only():
    """Measured slower than the data-parallel tiles at every shape tried
    (partial rounds included), so the planner never picks it."""
    for shape in ((3072, 3072, 4096), (5120, 5120, 4096), (2560, 2560, 4096), (4096, 14336, 4096)):
        assert plan(*shape).config.kernel == 3, shape


def test_forced_stream_k_configurations():
    p = plan(1024, 1024, 1024, force={"kernel": g.KERNEL_DMA_SK, "bm": 256, "bn": 256, "splitk": 7})
    c = p.config
    assert (c.kernel, c.splitk) == (g.KERNEL_DMA_SK, 7)
    assert g.gemm_plan_launch(p)[0] == 7
    assert g.gemm_workspace_size(p) == 16384 + 2 * 7 * 256 * 256 * 4
    assert "gemm_dma_sk_kernel<256,256" in p.describe()
    p = plan(1000, 520, 1000, force={"kernel": g.KERNEL_DMA_SK, "bm": 256, "bn": 128})
    assert p.config.splitk == min(256, (4 * 5 * 16) // 16)
    big = plan(8192, 8192, 8192, force={"kernel": g.KERNEL_DMA_SK, "bm": 256, "bn": 256, "splitk": 4000})
    assert big.config.splitk == 4000
    with pytest.raises(g.GemmError):                                        # 2 x 4096 parts of 256 KiB: 2 GiB
        plan(8192, 8192, 8192, force={"kernel": g.KERNEL_DMA_SK, "bm": 256, "bn": 256, "splitk": 4096})
    for bad in ({"kernel": g.KERNEL_DMA_SK, "splitk": 16 * 16 + 1},):       # more workgroups than K steps
        with pytest.raises(g.GemmError) as e:
            plan(1024, 1024, 1024, force=dict(bad, bm=256, bn=256))
        assert e.value.status == g.GEMM_ERR_UNSUPPORTED
