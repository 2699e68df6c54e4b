"""The fp8 grouped GEMM's handling of the two block scales, modelled in float32 on the CPU.

The FP8 layer (StackedMoE page, quant_config with block scaling) has one fp32
scale per 128-column group of each activation row and one per 128 x 128 block
of each expert weight.  One output element of the GEMM is

    C = sum over 128-wide k blocks kb of  xs[kb] * ws[kb] * P[kb]

where P[kb] is the dot product of the raw e4m3 values over block kb.  The
kernel cannot add blocks with different scales in one accumulator directly,
so it keeps the running sum in units of the current block's scale and
rescales between blocks.  This file models that recurrence with float32
arithmetic, as the kernel runs it, on scales the tiny-valued activations and
weights of real data can produce (a 128-group at amax 1e-35, a group of bf16
subnormals, a weight block of amax 1e-30):

* the first form (unit = xs * ws, rescale by unit_prev / unit) fails: where
  the product of two small scales is subnormal its reciprocal is infinite
  and the accumulator becomes inf or NaN; where the product underflows to
  zero the block is added in the previous block's units;
* the committed form splits each scale into a power of two, which the
  matrix instruction applies to the product in hardware (one E8M0 exponent
  byte per operand), and a factor in [2^-23, 4) that stays in software;
  its recurrence stays finite and matches the exact sum.

These are CPU models of the kernel's arithmetic, not the oracle.
"""
import numpy as np

from oracle import moe_oracle as O

f32 = np.float32


def _block_products(rng, nblk):
    """Exact dot products of 128 random e4m3 values per block (float64)."""
    xc = rng.integers(0, 256, size=(nblk, 128), dtype=np.uint8)
    wc = rng.integers(0, 256, size=(nblk, 128), dtype=np.uint8)
    xc[(xc & 0x7F) == 0x7F] = 0                 # no NaN codes
    wc[(wc & 0x7F) == 0x7F] = 0
    return np.sum(O.e4m3_decode(xc) * O.e4m3_decode(wc), axis=1)


def _rcp32(v):
    """float32 reciprocal (correctly rounded; overflows to inf like the hardware)."""
    with np.errstate(divide="ignore", over="ignore"):
        return f32(f32(1.0) / f32(v))


def _old_recurrence(xs, ws, P):
    unit = f32(1.0)
    acc = f32(0.0)
    with np.errstate(over="ignore", invalid="ignore", under="ignore"):
        for kb in range(len(P)):
            s = f32(f32(xs[kb]) * f32(ws[kb]))
            s = s if s != 0 else unit
            ratio = f32(unit * _rcp32(s))
            unit = s
            acc = f32(f32(acc * ratio) + f32(P[kb]))
        return f32(acc * unit)


def split_scale(s):
    """(E8M0 byte e in [1, 253], factor m) with s = 2^(e - 127) * m exactly:
    e is the float32 exponent field clamped to [1, 253], m = s * 2^(127 - e)."""
    s = f32(s)
    ef = int((np.array([s], f32).view(np.uint32)[0] >> 23) & 0xFF)
    e = min(max(ef, 1), 253)
    return e, f32(np.ldexp(np.float64(s), 127 - e))


def _new_recurrence(xs, ws, P):
    unit = f32(1.0)
    acc = f32(0.0)
    with np.errstate(over="ignore", invalid="ignore", under="ignore"):
        for kb in range(len(P)):
            ex, mx = split_scale(xs[kb])
            ew, mw = split_scale(ws[kb])
            u = f32(mx * mw)
            if u == 0:                       # a zero scale: its codes are zeroed, the unit kept
                continue
            ratio = f32(unit * _rcp32(u))
            unit = u
            # the matrix instruction scales the exact block product by the two
            # power-of-two exponents, then accumulates in float32
            prod = f32(np.ldexp(P[kb], ex + ew - 254))
            acc = f32(f32(acc * ratio) + prod)
        return f32(acc * unit)


def _case(name, rng):
    nblk = 56                                    # hidden 7168: the fp8 layer's gate_up K
    P = _block_products(rng, nblk)
    xs = (rng.random(nblk) * 4 + 1).astype(f32) / f32(448)     # amax of N(0,1) groups
    ws = np.full(nblk, f32(0.08 / 448), f32)                    # weights ~N(0, 0.02)
    if name == "tiny_group":
        xs[7] = f32(1e-35) / f32(448)                            # a 128-group at amax 1e-35
    elif name == "subnormal_group":
        xs[3] = f32(2.0 ** -130) / f32(448)                      # a group of bf16 subnormals
        xs[40] = f32(1e-39) / f32(448)
    elif name == "tiny_weight_block":
        ws[11] = f32(1e-30) / f32(448)                           # a weight block of amax 1e-30
        xs[11] = f32(1e-20)
    elif name == "all_tiny_row":
        xs[:] = f32(1e-36) / f32(448)                            # a token whose values are all tiny
    return xs, ws, P


def _exact(xs, ws, P):
    return float(np.sum(np.asarray(xs, np.float64) * np.asarray(ws, np.float64) * P))


def test_first_form_fails_on_tiny_scales():
    """The recurrence of the first kernel gives inf / NaN where the product of
    the two scales is subnormal (tiny group), and adds the block at the wrong
    scale where the product underflows to zero (subnormal group)."""
    rng = np.random.default_rng(0)
    xs, ws, P = _case("tiny_group", rng)
    assert np.isfinite(_exact(xs, ws, P))
    assert not np.isfinite(_old_recurrence(xs, ws, P))
    xs, ws, P = _case("subnormal_group", rng)
    want = _exact(xs, ws, P)
    got = float(_old_recurrence(xs, ws, P))
    scale = float(np.sum(np.abs(np.asarray(xs, np.float64) * ws * P)))
    assert not np.isfinite(got) or abs(got - want) > 1e-2 * scale


def test_split_scale_is_exact():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        (rng.random(2000) * 10).astype(f32),
        np.ldexp(rng.random(2000) + 1, rng.integers(-149, 128, 2000)).astype(f32),
        np.array([2.0 ** -149, 2.0 ** -126, 2.0 ** -127, 3.4e38, 2.0 ** 127, 1e-45, 1.0], f32),
    ])
    for s in vals:
        e, m = split_scale(s)
        assert 1 <= e <= 253
        assert np.ldexp(np.float64(m), e - 127) == np.float64(s), s
        if s != 0:
            assert 2.0 ** -23 <= m < 4.0, (s, m)


def test_split_form_is_finite_and_exact_to_float32():
    rng = np.random.default_rng(2)
    for name in ("plain", "tiny_group", "subnormal_group", "tiny_weight_block", "all_tiny_row"):
        for _ in range(20):
            xs, ws, P = _case(name, rng)
            want = _exact(xs, ws, P)
            got = float(_new_recurrence(xs, ws, P))
            assert np.isfinite(got), name
            # a few float32 roundings per block over 56 blocks, relative to the
            # magnitude of the terms (the sum may cancel)
            scale = float(np.sum(np.abs(np.asarray(xs, np.float64) * ws * P)))
            tiny = 2.0 ** -126 * 2 ** 25                  # below what float32 products can hold
            assert abs(got - want) <= 1e-5 * scale + tiny, (name, got, want)
