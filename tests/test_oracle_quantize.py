"""Pins for the oracle's two-level quantisation: the page's worked tile, the
block-amax-to-6 mapping, invariances, 2D transpose consistency, brute force
on tiny tensors, and the degenerate cases."""
import os

import numpy as np
import pytest

import oracle as O
from tests import bruteforce as BF

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _toy():
    d = {"scaled": [], "rounded": [], "sr": []}
    with open(os.path.join(GOLDEN, "toy_tile.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, *v = line.split()
            v = [float(t) for t in v]
            if k in d:
                d[k].append(v)
            else:
                d[k] = v[0]
    return d


def _nib(codes, j):
    b = codes[:, j // 2]
    return (b & 0xF) if j % 2 == 0 else (b >> 4)


def _code_value(c):
    return O.e2m1_decode(int(c))


def test_worked_tile_whole_tensor():
    """Page toy example: a block with amax 6.2 gets s_b = 6/6.2 ~ 0.968 and the
    listed elements scale to 6.00, -4.16, 0.465 and round to 6, -4, 0.5.
    Taken as the whole tensor, the global scale and E4M3 block scale together
    give the element multiplier r_b = s_enc/d_b, which must equal the printed
    s_b to the printed precision."""
    toy = _toy()
    raw = [r for r, _ in toy["scaled"]]
    x = np.zeros((1, 16), np.float32)
    x[0, :len(raw)] = raw
    q = O.quantize(x)
    assert abs(max(abs(v) for v in raw) - toy["block_amax"]) < 1e-6
    d_b = O.e4m3_decode(int(q.scales[0, 0]))
    r_b = np.float32(np.float32(1.0) / q.g) / np.float32(d_b)
    assert abs(float(r_b) - toy["block_scale"]) < 5e-4
    for j, (raw_v, printed) in enumerate(toy["scaled"]):
        assert abs(float(np.float32(raw_v) * r_b) - printed) < 5e-3
    rounded = {a: b for a, b in toy["rounded"]}
    for j, (raw_v, printed_scaled) in enumerate(toy["scaled"]):
        assert _code_value(_nib(q.codes, j)[0]) == rounded[printed_scaled]


def test_worked_tile_rounding_steps():
    """Every printed 'scaled value -> FP4 value' pair of the toy example."""
    toy = _toy()
    for v, want in toy["rounded"]:
        idx = O.e2m1_rn_index(abs(v))
        got = _code_value(idx | (8 if v < 0 else 0))
        assert got == want, (v, got, want)


@pytest.mark.parametrize("prescale", [False, True])
def test_worked_tile_all_listed_elements(prescale):
    """The tile's other listed values (1.7, -0.6, 3.2, -1.1) are read both as
    already-scaled values (divide by s_b to get raw) and as raw values: the
    codes come out as printed either way."""
    toy = _toy()
    rounded = toy["rounded"]
    s_b = 6.0 / 6.2
    raw = [6.2, -4.3, 0.48]
    extra = [v for v, _ in rounded[3:]]
    raw += [v / s_b for v in extra] if prescale else extra
    x = np.zeros((1, 16), np.float32)
    x[0, :len(raw)] = raw
    q = O.quantize(x)
    want = [b for _, b in rounded]
    for j in range(len(raw)):
        assert _code_value(_nib(q.codes, j)[0]) == want[j], (j, raw[j])


def _gen(shape, seed, outlier_p=0.01, outlier_mul=30.0):
    g = np.random.default_rng(seed)
    x = g.standard_normal(shape)
    mask = g.random(shape) < outlier_p
    x[mask] *= outlier_mul
    return x.astype(np.float32)


def test_block_amax_maps_to_fp4_max():
    """Each block's largest element is scaled onto the FP4 maximum (code +-6)
    and is reconstructed within E4M3's relative rounding (2^-4) plus fp32
    slack, for every block whose scale is a normal E4M3 value."""
    x = _gen((64, 512), 3)
    q = O.quantize(x)
    xh = O.dequant(q)
    for i in range(64):
        for b in range(32):
            blk = x[i, b * 16:(b + 1) * 16]
            j = int(np.argmax(np.abs(blk)))
            d = O.e4m3_decode(int(q.scales[i, b]))
            if d < 2.0 ** -6:
                continue
            code = int(_nib(q.codes, b * 16 + j)[i])
            assert code & 7 == 7
            amax_b = float(abs(blk[j]))
            assert abs(6.0 * d * float(q.g) - amax_b) <= 2 ** -4 * amax_b * (1 + 1e-6)
            assert abs(abs(xh[i, b * 16 + j]) - amax_b) <= 2 ** -4 * amax_b * (1 + 1e-6)


def test_tensor_amax_block_gets_e4m3_max():
    x = _gen((32, 256), 4)
    q = O.quantize(x)
    amax = np.max(np.abs(x))
    i, j = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert q.scales[i, j // 16] == 0x7E  # 448
    assert abs(float(q.g) - amax / 2688.0) <= 1e-6 * amax / 2688.0


@pytest.mark.parametrize("k", [-3, 1, 5])
def test_power_of_two_invariance(k):
    """Codes and block scales of 2^k x equal those of x; g scales by 2^k."""
    x = _gen((32, 256), 5)
    q0 = O.quantize(x)
    q1 = O.quantize(x * np.float32(2.0 ** k))
    assert np.array_equal(q0.codes, q1.codes)
    assert np.array_equal(q0.scales, q1.scales)
    assert float(q1.g) == float(q0.g) * 2.0 ** k


def test_sign_symmetry_rn():
    """Nearest-even is sign-symmetric: codes(-x) = codes(x) with both sign bits
    flipped, same scales and g."""
    x = _gen((32, 256), 6)
    x[x == 0] = 1.0  # a zero would keep its own sign bit
    q0, q1 = O.quantize(x), O.quantize(-x)
    assert np.array_equal(q0.codes ^ 0x88, q1.codes)
    assert np.array_equal(q0.scales, q1.scales) and q0.g == q1.g


def test_2d_transpose_consistency():
    """With 16x16 weight scales the transposed copy is exactly the quantised
    weight transposed, and quantising W^T directly gives the same bytes:
    forward and backward GEMMs see one quantised weight."""
    w = (_gen((96, 160), 7) * 0.02).astype(np.float32)
    q, qt = O.quantize_2d(w)
    q_of_t, _ = O.quantize_2d(np.ascontiguousarray(w.T))
    assert np.array_equal(qt.codes, q_of_t.codes)
    assert np.array_equal(qt.scales, q_of_t.scales)
    assert qt.g == q.g == q_of_t.g
    assert np.array_equal(O.dequant(qt), O.dequant(q).T)


def test_2d_vs_1d_scale_grid_shape_and_values():
    w = (_gen((32, 64), 8) * 0.02).astype(np.float32)
    q, _ = O.quantize_2d(w)
    assert q.scales.shape == (2, 4)
    for bi in range(2):
        for bj in range(4):
            tile = w[bi * 16:(bi + 1) * 16, bj * 16:(bj + 1) * 16]
            t = np.float32(np.max(np.abs(tile))) * np.float32(np.float32(2688.0 / np.max(np.abs(w))) / np.float32(6.0))
            assert q.scales[bi, bj] == O.e4m3_encode(float(t))


# ------------------------------------------------------------ brute force


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("sr", [False, True])
def test_brute_force_1x16(seed, sr):
    x = _gen((3, 32), 100 + seed, outlier_p=0.1)
    codes, scales, g = BF.quantize(x, sr=sr, seed=77, offset=48, stream=3)
    q = O.quantize(x, sr=sr, seed=77, offset=48, stream=3)
    assert np.array_equal(q.codes, codes)
    assert np.array_equal(q.scales, scales)
    assert q.g == g


@pytest.mark.parametrize("sr", [False, True])
def test_brute_force_transpose_rht(sr):
    """Transposed operand with the RHT along the block axis.  Inputs are small
    multiples of 1/16 so the transform is exact in fp32 and the brute force
    can use the float64 matrix form."""
    g = np.random.default_rng(11)
    x = (g.integers(-512, 512, size=(32, 5)) / 16.0).astype(np.float32)
    signs = 0xB5C3
    codes, scales, gg = BF.quantize(x, transpose=True, rht=True, signs=signs, sr=sr, seed=9,
                                    stream=1)
    q = O.quantize(x, transpose=True, rht=True, signs=signs, sr=sr, seed=9, stream=1)
    assert np.array_equal(q.codes, codes) and np.array_equal(q.scales, scales) and q.g == gg


def test_brute_force_2d():
    w = (_gen((32, 48), 12, outlier_p=0.05) * 0.02).astype(np.float32)
    codes, grid, g = BF.quantize_2d(w)
    q, _ = O.quantize_2d(w)
    assert np.array_equal(q.codes, codes) and np.array_equal(q.scales, grid) and q.g == g


def test_brute_force_dequant():
    x = _gen((4, 48), 13)
    q = O.quantize(x)
    assert np.array_equal(O.dequant(q), BF.decode(q.codes, q.scales, q.g))
    w = _gen((32, 32), 14)
    q2, _ = O.quantize_2d(w)
    assert np.array_equal(O.dequant(q2), BF.decode(q2.codes, q2.scales, q2.g, mode=1))


# ------------------------------------------------------------ degenerate cases


def test_zero_tensor():
    q = O.quantize(np.zeros((2, 32), np.float32))
    assert q.g == 1.0 and not q.scales.any() and not q.codes.any()
    xz = np.zeros((1, 16), np.float32)
    xz[0, 3] = -0.0
    q = O.quantize(xz)
    assert _nib(q.codes, 3)[0] == 8  # negative zero keeps its sign bit


def test_zero_block_in_nonzero_tensor():
    x = _gen((1, 32), 15)
    x[0, :16] = 0
    q = O.quantize(x)
    assert q.scales[0, 0] == 0 and not q.codes[0, :8].any()


def test_tiny_block_scale_flushes_to_zero():
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 1.0
    x[0, 16] = 1e-9  # t = 1e-9 * 448 far below E4M3's smallest subnormal / 2
    q = O.quantize(x)
    assert q.scales[0, 1] == 0 and not q.codes[0, 8:].any()


def test_nonfinite_raises():
    for bad in (np.inf, -np.inf, np.nan):
        x = np.ones((1, 16), np.float32)
        x[0, 5] = bad
        with pytest.raises(O.OracleError) as e:
            O.quantize(x)
        assert e.value.status == O.ERR_NONFINITE
    with pytest.raises(O.OracleError):
        O.quantize_2d(np.full((16, 16), np.nan, np.float32))


def test_shape_errors():
    with pytest.raises(O.OracleError):
        O.quantize(np.ones((2, 24), np.float32))
    with pytest.raises(O.OracleError):
        O.quantize_2d(np.ones((24, 32), np.float32))


def test_subnormal_tensor_scale_saturates():
    """amax below 2688/FLT_MAX: s_enc saturates to FLT_MAX (a stated reading);
    the results stay finite and deterministic."""
    x = np.zeros((1, 16), np.float32)
    x[0, 0] = 1e-39
    x[0, 1] = -5e-40
    q = O.quantize(x)
    assert np.isfinite(q.g) and q.g > 0
    assert np.all(np.isfinite(O.dequant(q)))
