"""Host replay of the backward row kernel's row walk at the planner's launch shapes (no GPU).

The backward row kernel (``bwd_kernel`` in csrc/bwd.hip) runs a persistent grid of G
workgroups, each of T teams. Workgroup b makes n = ceil((rows - b*T) / (G*T)) steps (none when
b*T >= rows) at base rows b*T, b*T + G*T, ..., as n // 2 two-step trips (two row buffers used in
turn) and a last single step when n is odd; team t handles row base + t. A team's row past the
end reads zeros and its dx stores are dropped (their offset lies past the row's resource), the
guard ``row < rows``. The planner's launch shape (layout, W, KC, T, G) comes from the library
itself (``norm_bwd_launch_shape``), so this test follows the planner as built; the walk below
restates the kernel's loop.

[NVRTC-PR] "Migrate norms and softmax kernels to NVRTC", Flowchart: the backward's per-workgroup
partial kernels and the grid sized from occupancy and the SM margin.
"""
import ctypes
import os

import pytest

L = pytest.importorskip("rmsnorm_fp8_quantization_amd._lib")


def _lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libnormfp8.so not built (run __graft_entry__.build())")
    return L.load()


def launch_shape(rows, hidden, norm=L.NORM_LAYERNORM, with_add=0, cus=256, margin=0, occ=1,
                 in_dt=L.NORM_BF16, w_dt=L.NORM_F32):
    _lib()
    shape = (ctypes.c_int64 * 5)()
    L.call("norm_bwd_launch_shape", rows, hidden, in_dt, w_dt, norm, with_add, cus, margin, occ, shape)
    return tuple(int(v) for v in shape)


def walk(rows, T, G, teams=None, guarded=True):
    """Rows the kernel stores dx for: workgroup b makes n steps (the trip count computed from
    its first base row b*T and the stride G*T), n // 2 trips of two steps and one more step
    when n is odd, at base = b*T, b*T + G*T, ...; team t stores row base + t when it is < rows
    (``guarded``) or always (the unguarded form). ``teams`` is the number of teams actually
    launched (T unless the kernel and the planner disagree on T)."""
    teams = T if teams is None else teams
    stride = G * T
    stored = []

    def step(base):
        for t in range(teams):
            if not guarded or base + t < rows:
                stored.append(base + t)

    for b in range(G):
        first = b * T
        n = (rows - first + stride - 1) // stride if first < rows else 0
        base = first
        for _ in range(n // 2):
            step(base)
            step(base + stride)
            base += 2 * stride
        if n % 2:
            step(base)
    return stored


LAYOUTS = range(14)  # every backward layout of the library's shape table


@pytest.mark.parametrize("cfg", LAYOUTS)
def test_every_layout_stores_each_row_once_and_never_past_the_end(cfg):
    for hidden in (8, 1024, 4096):
        for k in (1, 2, 3, 257, 1025, 4097):
            for occ in (1, 2, 8):
                for margin in (0, 7):
                    with L.tuning(NORMFP8_BWD_CFG=cfg):
                        c0, W, KC, T, G = launch_shape(8, hidden)
                        if c0 != cfg:  # this layout does not cover the row
                            continue
                        for rows in (T * k - 1, T * k, T * k + 1):
                            if rows == 0:  # no rows: one workgroup, no row visited
                                assert walk(0, T, launch_shape(0, hidden)[4]) == []
                                continue
                            c, W, KC, T, G = launch_shape(rows, hidden, occ=occ, margin=margin)
                            assert c == cfg
                            assert 1 <= G and (G - 1) * T < rows, (cfg, rows, G, T)  # no idle workgroup
                            stored = walk(rows, T, G)
                            assert max(stored) < rows and sorted(stored) == list(range(rows)), (cfg, rows, G, T)


def test_default_plans_with_ragged_row_counts():
    """Planner defaults (no override) at row counts that are not multiples of T: the team
    layouts T = 2 and T = 4 are chosen at 2048 / 4096 rows and more."""
    seen_t = set()
    for norm, add in ((L.NORM_LAYERNORM, 0), (L.NORM_RMSNORM, 0), (L.NORM_RMSNORM, 1)):
        for hidden in (512, 1024, 2048, 4096, 8192):
            for rows in (2047, 2049, 4095, 4097, 16383, 16385, 32769):
                c, W, KC, T, G = launch_shape(rows, hidden, norm=norm, with_add=add)
                seen_t.add(T)
                stored = walk(rows, T, G)
                assert max(stored) < rows and len(stored) == rows, (norm, hidden, rows, c, T, G)
    assert {2, 4} <= seen_t


def test_unguarded_walk_would_store_past_the_end():
    """The replay is sensitive to the guard: without it, a T > 1 layout at rows % T != 0 stores
    rows beyond the tensor (the defect the guard closes)."""
    c, W, KC, T, G = launch_shape(4097, 1024)
    assert T == 4
    assert max(walk(4097, T, G, guarded=False)) >= 4097


def test_kernel_and_planner_disagreeing_on_t_store_past_the_end():
    """A library assembled from objects built with different team counts (kernel T = 3, planner
    T = 2: 512 threads launched, two teams) at LayerNorm 16384 x 4096: with the row guard
    defeated, the walk stores row 16384, 8 KB past a 16384-row bf16 dx; with the guard it stores
    nothing past the end (and leaves rows unvisited, the wrong-answer half of such a mismatch)."""
    c, W, KC, T, G = launch_shape(16384, 4096, occ=1)
    assert (W, KC, T) == (4, 2, 2) and G == 256
    bad = walk(16384, 3, G, teams=2, guarded=False)
    assert max(bad) == 16384
    ok = walk(16384, 3, G, teams=2, guarded=True)
    assert max(ok) < 16384 and len(set(ok)) < 16384


# default backward layout per row width (many rows: 16384; few rows: under four per team)
@pytest.mark.parametrize("hidden,many,few", [
    (1024, (0, 2, 1, 4), (8, 2, 1, 1)),
    (2048, (1, 4, 1, 2), (9, 4, 1, 1)),
    (4096, (2, 4, 2, 2), (10, 4, 2, 1)),
    (4104, (12, 5, 2, 2), (13, 5, 2, 1)),
    (5120, (12, 5, 2, 2), (13, 5, 2, 1)),
    (5128, (3, 8, 2, 1), (3, 8, 2, 1)),
    (8192, (3, 8, 2, 1), (3, 8, 2, 1)),
    (12288, (11, 8, 3, 1), (11, 8, 3, 1)),
    (16384, (4, 16, 2, 1), (4, 16, 2, 1)),
])
def test_default_layout_per_width(hidden, many, few):
    assert launch_shape(16384, hidden)[:4] == many
    assert launch_shape(16384, hidden, norm=L.NORM_RMSNORM)[:4] == many
    assert launch_shape(256 * many[3] * 4 - 1, hidden)[:4] == few
    assert launch_shape(256 * many[3] * 4, hidden)[:4] == many
