"""GPU unit tests of the instructions the attention kernels rely on (needs an MI355X).

Sources: "SageAttention2 Technical Report" summary, 3.4 "Two-Level Accumulation: Mitigating the
Undocumented FP22 Accumulator" (probe the matrix core's accumulator: an input C carrying more
mantissa bits than the internal sum keeps, and a sum of products of spread magnitudes against
FP64), and "FP8 Quantization for P~V" (the E4M3 cast, round to nearest even, 448 the largest
value).

What the kernels assume, each checked here:
  * the output layout of the 32x32 MFMA accumulator (lane l, register r holds row
    8 (r / 4) + 4 (l / 32) + r % 4, column l % 32) and the pairing of the A and B operand bytes
    (a lane half's byte j of A meets the same lane half's byte j of B) -- the per-thread scale
    groups of K (4 per 64 keys) and the transposed V^ order follow from them;
  * the INT8 MFMA sums exactly;
  * the FP8 MFMA adds its C operand at full FP32 precision (so O accumulated through C is an
    FP32 buffer: the second level of the two-level accumulation);
  * the FP8 MFMA's internal sum of one step's 64 products is accurate to a small fraction of the
    largest product (the score error that the FP8-QK knob's parity margin allows for);
  * the kernels' E4M3 cast (clamp to +-448, then v_cvt_pk_fp8_f32) equals the oracle's E4M3
    codec on every FP32 input from 2^-27 to 2^18 of either sign, and on a random sample of all
    bit patterns (NaN: any NaN code);
  * the matrix cores reach a plausible share of their nominal dense rates.
"""
import sys

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_attention_amd import probe
    probe.load()


from quantized_attention_amd import probe  # noqa: E402

DEC = oracle.e4m3_decode_table()


def out_index():
    """(row, column) of every (lane, register) of the 32x32 accumulator, as the kernels assume."""
    lane = np.arange(64)[:, None]
    reg = np.arange(16)[None, :]
    return 8 * (reg // 4) + 4 * (lane // 32) + reg % 4, np.broadcast_to(lane % 32, (64, 16))


def host_product(a_val, b_val):
    """D[i][j] = sum over lane halves h and bytes j' of A[32h + i][j'] B[32h + j][j'] (FP64)."""
    A = np.concatenate([a_val[:32], a_val[32:]], axis=1)  # row i: half 0's bytes, then half 1's
    B = np.concatenate([b_val[:32], b_val[32:]], axis=1)
    return A @ B.T


def as_regs(D):
    r, c = out_index()
    return D[r, c]


def e4m3_codes_of(values):
    return oracle.e4m3_encode_f32(np.asarray(values, np.float32))


def test_int8_mfma_is_exact_in_the_assumed_layout():
    rng = np.random.default_rng(1)
    a = rng.integers(-127, 128, (64, 16)).astype(np.int8)
    b = rng.integers(-127, 128, (64, 16)).astype(np.int8)
    c = rng.integers(-2 ** 20, 2 ** 20, (64, 16)).astype(np.int32)
    d = probe.mfma_i8(*(torch.from_numpy(x).cuda() for x in (a, b, c))).cpu().numpy()
    want = as_regs(host_product(a.astype(np.int64), b.astype(np.int64))) + c
    assert np.array_equal(d.astype(np.int64), want)


def test_fp8_mfma_layout_on_exact_sums():
    """Small E4M3 values whose every partial sum is exact in any accumulator."""
    rng = np.random.default_rng(2)
    va = rng.choice([0.0, 1.0, -1.0, 2.0, -2.0, 0.5], (64, 32))
    vb = rng.choice([0.0, 1.0, -1.0, 2.0, -0.5], (64, 32))
    a, b = e4m3_codes_of(va), e4m3_codes_of(vb)
    assert np.array_equal(DEC[a], va) and np.array_equal(DEC[b], vb)
    c = np.zeros((64, 16), np.float32)
    d = probe.mfma_f8(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda(), torch.from_numpy(c).cuda())
    assert np.array_equal(d.cpu().numpy().astype(np.float64), as_regs(host_product(va, vb)))


def test_fp8_mfma_c_operand_passes_at_fp32():
    """A = B = 0: D must equal C bit for bit, for C with all 24 significant bits in use."""
    rng = np.random.default_rng(3)
    zero = torch.zeros((64, 32), dtype=torch.uint8, device="cuda")
    mant = rng.integers(0, 2 ** 23, (64, 16), dtype=np.int64) | 1  # odd: the last bit is set
    expo = rng.integers(100, 155, (64, 16), dtype=np.int64)
    sign = rng.integers(0, 2, (64, 16), dtype=np.int64)
    c = ((sign << 31) | (expo << 23) | mant).astype(np.uint32).view(np.float32)
    d = probe.mfma_f8(zero, zero, torch.from_numpy(c).cuda()).cpu().numpy()
    assert np.array_equal(d.view(np.uint32), c.view(np.uint32))
    # and C far above the products: D = C + sum, rounded once at C's magnitude
    va = np.full((64, 32), 2.0 ** -9)
    a = e4m3_codes_of(va)
    d = probe.mfma_f8(torch.from_numpy(a).cuda(), torch.from_numpy(a).cuda(),
                      torch.from_numpy(c).cuda()).cpu().numpy().astype(np.float64)
    exact = c.astype(np.float64) + 64 * 2.0 ** -18
    big = np.abs(c) >= 1.0  # there the sum 2^-12 lies far below C's last bit or near it
    tol = np.spacing(np.abs(exact).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(d - exact)[big] <= tol[big])


# The worst error of the FP8 MFMA's internal sum of one 64-product step, relative to the step's
# largest product, that the FP8-QK parity margin assumes (tests/test_gpu_qk_fp8.py, the oracle's
# qk_step_err).  Measured below: worst 2^-11.4 (the errors of 64 products aligned to the largest
# one and cut about 2^-17.5 below it add up), typical 2^-15.
FP8_MFMA_STEP_ERR = 2.0 ** -10


def test_fp8_mfma_internal_sum_precision():
    """64 products of spread magnitudes per output (random E4M3 values times powers of two from
    2^0 down to 2^-15 across the 64 products), 20 random trials: the error of D = A B (C = 0)
    against the exact FP64 sum, relative to the largest product of that output, stays within
    FP8_MFMA_STEP_ERR."""
    rng = np.random.default_rng(4)
    grid = DEC[(DEC > 0) & np.isfinite(DEC)]
    rels = []
    inexact = 0
    for trial in range(20):
        scale = 2.0 ** -rng.integers(0, 16, (64, 32))
        va = rng.choice(grid, (64, 32)) * rng.choice([-1.0, 1.0], (64, 32))
        va = DEC[e4m3_codes_of(va * scale)]
        vb = DEC[e4m3_codes_of(rng.choice(grid[grid <= 8], (64, 32)) * rng.choice([-1.0, 1.0], (64, 32)))]
        a, b = e4m3_codes_of(va), e4m3_codes_of(vb)
        c = torch.zeros((64, 16), dtype=torch.float32, device="cuda")
        d = probe.mfma_f8(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda(), c).cpu().numpy().astype(np.float64)
        exact = as_regs(host_product(DEC[a], DEC[b]))
        A = np.concatenate([DEC[a][:32], DEC[a][32:]], axis=1)
        B = np.concatenate([DEC[b][:32], DEC[b][32:]], axis=1)
        pmax = as_regs(np.max(np.abs(A)[:, None, :] * np.abs(B)[None, :, :], axis=-1))
        rels.append((np.abs(d - exact) / np.maximum(pmax, 1e-300)).ravel())
        inexact += int((d != exact.astype(np.float32)).sum())
    rel = np.concatenate(rels)
    say(f"fp8 mfma internal sum: worst error 2^{np.log2(rel.max()):.1f} of the largest product, median "
        f"2^{np.log2(max(np.median(rel), 1e-30)):.1f}; {inexact} of {rel.size} outputs differ from the correctly "
        f"rounded FP32 sum")
    assert rel.max() <= FP8_MFMA_STEP_ERR


def test_e4m3_cast_matches_oracle_codec():
    """Every FP32 value with exponent field 100 .. 145 (2^-27 up to 2^19), both signs, and 2^24
    random bit patterns over the whole range."""
    mismatch = 0
    total = 0
    for sign in (0, 1):
        for e0 in range(100, 146, 8):
            e1 = min(e0 + 8, 146)
            start = (sign << 31) | (e0 << 23)
            count = (e1 - e0) << 23
            got = probe.cvt_e4m3(start, count).cpu().numpy()
            x = (np.arange(count, dtype=np.uint64) + start).astype(np.uint32).view(np.float32)
            want = oracle.e4m3_encode_f32(x)
            mismatch += int((got != want).sum())
            total += count
            del x, want, got
    rng = np.random.default_rng(5)
    for _ in range(4):
        start = int(rng.integers(0, 2 ** 32 - 2 ** 22))
        got = probe.cvt_e4m3(start, 2 ** 22).cpu().numpy()
        x = (np.arange(2 ** 22, dtype=np.uint64) + start).astype(np.uint32).view(np.float32)
        want = oracle.e4m3_encode_f32(x)
        nan = np.isnan(x)
        assert np.all((got[nan] & 0x7F) == 0x7F)
        mismatch += int((got[~nan] != want[~nan]).sum())
        total += 2 ** 22
    say(f"e4m3 cast: {total} inputs, {mismatch} mismatches")
    assert mismatch == 0


def test_u8_conversion_rounds_to_nearest_even():
    """v_cvt_pk_u8_f32, which packs SageBwd's forward P codes (values 127 P / (the row's block max
    of P), in [0, 127]), rounds to nearest with ties to even, as the oracle's rint does: every
    FP32 value from 0 to 128 (all 1.12e9 bit patterns), against numpy's rint."""
    start, stop = 0, int(np.float32(128.0).view(np.uint32)) + 1
    mismatch, total = 0, 0
    step = 2 ** 24
    for a in range(start, stop, step):
        n = min(step, stop - a)
        got = probe.cvt_u8(a, n).cpu().numpy()
        x = (np.arange(n, dtype=np.uint64) + a).astype(np.uint32).view(np.float32)
        want = np.rint(x.astype(np.float64)).astype(np.uint8)
        mismatch += int((got != want).sum())
        total += n
        del x, want, got
    say(f"u8 conversion: {total} inputs in [0, 128], {mismatch} mismatches")
    assert mismatch == 0


@pytest.mark.parametrize("kind,nominal", [(0, 5000.0), (1, 5000.0), (2, 10100.0)])
def test_mfma_rates_are_plausible(kind, nominal):
    tops = probe.mfma_rate(kind)
    say(f"{probe.RATE_KINDS[kind][0]}: {tops:.0f} TOPS measured ({tops / nominal:.1%} of the nominal {nominal:.0f})")
    assert 0.3 * nominal < tops < 1.1 * nominal


def test_valu_rates():
    """Issue rates of the softmax's instructions relative to v_fma_f32 (the kernels' VALU budget
    counts v_exp_f32 and the FP8 and FP4 packs as two issue slots each): exp and the packs at
    most about half the FMA rate; exp interleaved with an equal number of FMAs takes at least 80%
    of the sum of their separate times (measured 88%: the exponentials are not hidden behind the
    arithmetic)."""
    rates = {k: probe.valu_rate(k) for k in probe.VALU_KINDS}
    fma = rates[0]
    for k, r in rates.items():
        say(f"{probe.VALU_KINDS[k][0]}: {r:.1f} wave instructions / ns ({r / fma:.2f} x v_fma_f32)")
    assert rates[1] / fma < 0.6 and rates[2] / fma < 0.6 and rates[3] / fma < 0.65
    t_mix = 1.0 / rates[5]                   # time per instruction of the interleaved mix
    t_sum = 0.5 / rates[1] + 0.5 / fma       # half of them exp, half fma, if they add up
    say(f"exp + fma interleaved: {t_mix / t_sum:.2f} of the sum of their separate times")
    assert t_mix >= 0.8 * t_sum


def test_hbm_reread_rates():
    """The preprocessing reads K and V twice (statistics, then quantization).  Running the second
    read right after the first, one group of heads at a time, would pay only if the Infinity
    Cache served a re-read much faster than HBM.  Measured here: cold reads of 128 and 256 MiB
    (after 2 GiB of other reads), the same buffer read again at once, and read again after 256
    MiB of writes in between; plus plain streaming writes.  Only plausibility is asserted; the
    printed rates are the evidence."""
    import torch
    MiB = 1 << 20
    A = torch.zeros(256 * MiB // 4, dtype=torch.float32, device="cuda")
    F = torch.zeros(2048 * MiB // 4, dtype=torch.float32, device="cuda")
    W = torch.zeros(256 * MiB // 4, dtype=torch.float32, device="cuda")
    med = lambda xs: sorted(xs)[len(xs) // 2]  # noqa: E731
    rates = []
    for size in (128 * MiB, 256 * MiB):
        cold, again, after = [], [], []
        for _ in range(3):
            probe.stream_rate(0, F, 2048 * MiB)  # evicts A from every cache
            cold.append(probe.stream_rate(0, A, size))
            again.append(probe.stream_rate(0, A, size))
            probe.stream_rate(1, W, 256 * MiB)
            after.append(probe.stream_rate(0, A, size))
        say(f"read {size // MiB} MiB: cold {med(cold):.2f} TB/s, again at once {med(again):.2f}, "
            f"again after 256 MiB of writes {med(after):.2f}")
        rates += cold + again + after
    writes = [probe.stream_rate(1, W, 256 * MiB) for _ in range(3)]
    say(f"write 256 MiB: {med(writes):.2f} TB/s")
    rates += writes
    assert all(0.5 < r < 30.0 for r in rates), rates
