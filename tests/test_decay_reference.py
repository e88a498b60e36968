"""The decay-reference rule of the chunked forward kernels, restated on the
host in fp64: for every 16-token chunk and channel, the integer
L = sum_t (e_t - 1) (e_t the binary exponent of alpha_t) bounds the chunk's
decay product, 2^L <= G_15 < 2^(L + 16); the reference c = 2^m (m = 0 for
L >= -100, else ceil(L / 2)) keeps G_t / c and c / G_t within 2^112 of one;
and where L < -224 raising the alphas below 2^-14 to 2^-14 brings the chunk
back inside that range.  (The kernels' fp32 arithmetic is checked against the
oracle by the small-alpha GPU parity tests; this pins the rule itself.)"""
import numpy as np

FLOOR, L_FREE, L_FLOOR, E_FLOOR = 2.0 ** -14, -100, -224, -14


def decay_lb(a):
    a = np.asarray(a, np.float64)
    _, e = np.frexp(np.where(a >= 2.0 ** -120, a, 1.0))
    return np.where(a >= 2.0 ** -120, e - 1, -1000)


def reference(al):
    L = int(decay_lb(al).sum())
    floor = L < L_FLOOR
    if floor:
        L = int(np.maximum(decay_lb(al), E_FLOOR).sum())
    m = 0 if L >= L_FREE else -((-L) >> 1)
    return floor, m, L


def chunks(rng, n):
    out = []
    for _ in range(n):
        kind = rng.integers(0, 5)
        if kind == 0:
            al = 1.0 / (1.0 + np.exp(-rng.normal(2.0, 2.0, 16)))
        elif kind == 1:
            al = 10.0 ** rng.uniform(-3.0, -2.0, 16)
        elif kind == 2:
            al = 10.0 ** rng.uniform(-6.0, -3.0, 16)
        elif kind == 3:
            al = np.where(rng.random(16) < 0.2, 0.0, 10.0 ** rng.uniform(-8.0, 0.0, 16))
        else:
            al = 10.0 ** rng.uniform(-40.0, 0.0, 16)
        out.append(al.astype(np.float32).astype(np.float64))
    return out


def test_bound_on_the_chunk_product():
    rng = np.random.default_rng(5)
    for al in chunks(rng, 4000):
        if np.any(al < 2.0 ** -120):
            continue
        L = int(decay_lb(al).sum())
        logG = np.sum(np.log2(al))
        assert L <= logG < L + 16


def test_reference_keeps_both_factors_in_range():
    rng = np.random.default_rng(6)
    floored = referenced = 0
    for al in chunks(rng, 4000):
        floor, m, L = reference(al)
        a2 = np.maximum(al, FLOOR) if floor else al
        logG = np.cumsum(np.log2(np.maximum(a2, 1e-300)))
        assert logG[-1] >= L_FLOOR if floor else True
        hi = np.max(np.abs(logG - m))      # |log2(G_t / c)| = |log2(c / G_t)|
        bound = 100 if m == 0 else 112
        assert hi <= bound + 1e-9, (L, m, hi)
        floored += floor
        referenced += (m != 0)
    assert floored > 100 and referenced > 100


def test_floor_changes_only_alphas_below_it():
    al = np.array([0.9] * 8 + [1e-7] * 8)
    floor, m, L = reference(al)
    assert not floor and m != 0          # 8 x 1e-7 spans about 2^-186: a reference suffices
    al = np.array([1e-7] * 16)
    floor, m, L = reference(al)
    assert floor and L == 16 * E_FLOOR and m == -112
