"""The kernel's group-score merge, emulated lane by lane on the CPU.

Lanes of a wave hold 8 consecutive experts each, so a group of E / n_group
experts spans gl = E / n_group / 8 consecutive lanes.  The kernel gives every
lane of a group the group's two largest keys by merging, over gl - 1
rotations inside the group, the own top-2 of each other lane into its pair.
This test runs the same steps on numpy arrays for every group width the
configuration check accepts (gl = 1 .. 64 / n_group) and compares with the
two largest keys of each group taken directly; a butterfly over power-of-two
offsets, which leaves the group when gl is not a power of two, fails it.
"""
import numpy as np
import pytest


def lane_merge(keys, gl):
    """keys [64 lanes, 8] -> per-lane (a1, a2) after the kernel's rotations."""
    srt = -np.sort(-keys, axis=1)
    o1, o2 = srt[:, 0].copy(), srt[:, 1].copy()
    a1, a2 = o1.copy(), o2.copy()
    lanes = np.arange(64)
    gb = (lanes // gl) * gl
    li = lanes - gb
    for s in range(1, gl):
        src = gb + np.where(li + s < gl, li + s, li + s - gl)
        src %= 64  # the lane crossbar wraps; lanes past the experts hold no group
        b1, b2 = o1[src], o2[src]
        n2 = np.where(a1 >= b1, np.maximum(b1, a2), np.maximum(a1, b2))
        a1 = np.maximum(a1, b1)
        a2 = n2
    return a1, a2


def butterfly_merge(keys, gl):
    srt = -np.sort(-keys, axis=1)
    a1, a2 = srt[:, 0].copy(), srt[:, 1].copy()
    off = 1
    while off < gl:
        src = np.arange(64) ^ off
        b1, b2 = a1[src], a2[src]
        n2 = np.where(a1 >= b1, np.maximum(b1, a2), np.maximum(a1, b2))
        a1, a2 = np.maximum(a1, b1), n2
        off <<= 1
    return a1, a2


@pytest.mark.parametrize("experts,n_group", [(e, n) for e in (64, 96, 128, 192, 256, 320, 384, 448, 512)
                                             for n in (2, 3, 4, 5, 6, 8, 16) if e % n == 0 and (e // n) % 8 == 0])
def test_rotation_merge_gives_each_group_its_top2(experts, n_group):
    rng = np.random.default_rng(experts * 31 + n_group)
    gl = experts // n_group // 8
    for trial in range(20):
        k = rng.standard_normal(512)
        k[experts:] = -np.inf
        keys = k.reshape(64, 8)
        a1, a2 = lane_merge(keys, gl)
        for g in range(n_group):
            top = -np.sort(-k[g * experts // n_group:(g + 1) * experts // n_group])[:2]
            for lane in range(g * gl, (g + 1) * gl):
                assert a1[lane] == top[0] and a2[lane] == top[1], (experts, n_group, g, lane)


def test_butterfly_leaves_the_group_when_the_width_is_not_a_power_of_two():
    """The planted mistake the test above guards against (gl = 6: 384 experts, 8 groups)."""
    rng = np.random.default_rng(1)
    bad = 0
    for trial in range(50):
        k = rng.standard_normal(512)
        k[384:] = -np.inf
        a1, a2 = butterfly_merge(k.reshape(64, 8), 6)
        for g in range(8):
            top = -np.sort(-k[g * 48:(g + 1) * 48])[:2]
            bad += any(a1[l] != top[0] or a2[l] != top[1] for l in range(g * 6, (g + 1) * 6))
    assert bad > 0
