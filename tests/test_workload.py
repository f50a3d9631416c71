"""The seeded input generator: Philox4x32-10 known answers, fast path == definition."""
import numpy as np

from workload import configs as C
from workload import gen


def test_philox_known_answers():
    # Known-answer vectors of Philox4x32-10 published with Random123 (Salmon et al., SC'11)
    kat = [
        ((0, 0, 0, 0), (0, 0), (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
        ((0xffffffff,) * 4, (0xffffffff,) * 2, (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
        ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
         (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
    ]
    for ctr, key, want in kat:
        got = gen.philox4x32_10(*[[c] for c in ctr], *key)
        assert tuple(int(x[0]) for x in got) == want


def test_fast_path_equals_definition():
    for seed, stream, start, n in ((0, 5, 0, 1000), (7, 0x10003, 12345, 777), (2**40 + 3, 9, 3, 5)):
        assert np.array_equal(gen.fast_words(seed, stream, start, n),
                              gen.words_range(seed, stream, start, n))
        assert np.array_equal(gen.fast_normal(seed, stream, (n,), 0.02, start),
                              gen.normal_f32(seed, stream, (n,), 0.02, start))
        assert np.array_equal(gen.fast_normal(seed, stream, (n,), 0.02, start, bf16=True),
                              gen.f32_to_bf16_bits(gen.normal_f32(seed, stream, (n,), 0.02, start)))
    idx = np.array([5, 0, 99, 4, 1 << 33])
    w = gen.words(3, 4, idx)
    for i, e in enumerate(idx):
        assert w[i] == gen.words_range(3, 4, int(e), 1)[0]


def test_normal_moments_and_grid():
    x = gen.fast_normal(0, 1, (1 << 20,), 1.0)
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1.0) < 5e-3
    assert np.all(np.abs(x) <= 1535 / 512)
    # unit-variance values sit on the k/512 grid exactly (fp32 product by a power of two)
    k = x.astype(np.float64) * 512
    assert np.array_equal(k, np.round(k))
    # most of them need more than bf16's 8 significant bits: an fp32-mode input rounded
    # to bf16 anywhere on the way would change
    assert np.mean(gen.round_bf16(x) != x) > 0.4
    # the integer variate itself: exact mean 0 and variance 2^18 over all 2^32 words
    # follow from the uniform parts; check the extremes and a few words by hand
    assert gen.normal_k(np.array([0, 0xFFFFFFFF], np.uint32)).tolist() == [-1535, 1535]
    assert gen.normal_k(np.array([1 | (2 << 10) | (3 << 20) | (1 << 30)], np.uint32)).tolist() == [1 + 2 + 3 + 1 - 1535]


def test_open01_is_exact_and_strictly_inside():
    w = np.array([0, 1, 511, 512, 0x80000000, 0xFFFFFE00, 0xFFFFFFFF], np.uint32)
    u = gen.open01_of_words(w)
    exact = ((w.astype(np.float64) // 512) + 0.5) * 2.0 ** -23
    assert np.array_equal(u.astype(np.float64), exact)          # no rounding in fp32
    assert u[0] == 2.0 ** -24 and u[-1] == 1.0 - 2.0 ** -24       # never 0 or 1
    assert np.all((u > 0) & (u < 1))


def test_bf16_round_to_nearest_even():
    vals = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5e-3], np.float32)
    b = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(vals))
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even (1.0)
    assert b[0] == 1.0 and b[1] == 1.0 and b[2] == np.float32(1.0 + 2**-6) and b[3] == 1.0
    assert abs(b[4] - vals[4]) <= abs(vals[4]) * 2**-8


def test_configs_inputs():
    w = C.c4()
    codes = C.maskgit_codes(w)
    assert codes.shape == (8, 750) and (codes == 1024).sum() == 3000
    assert codes.max() == 1024 and codes.min() >= 0
    L = C.c5_lengths(C.c5())
    assert L.min() >= 200 and L.max() <= 4000 and L.size == 64
    pt, n = C.page_table(7, [33, 16, 1])
    used = pt[pt >= 0]
    assert n == 5 and sorted(used.tolist()) == list(range(5))
    t = C.LazyTable(0, gen.KIND_TEXT_TABLE, 0, 151676, 64, True)
    full_row = gen.bf16_bits_to_f32(C.table(0, gen.KIND_TEXT_TABLE, 0, 3, 64, True))
    assert np.array_equal(t[np.array([2, 0])], full_row[[2, 0]])
