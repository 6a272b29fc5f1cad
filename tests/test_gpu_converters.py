"""Exhaustive checks of the gfx950 conversion steps behind every code, scale
byte and bf16 output of the library, run through the library's own
converter-check entry point (the same device helpers the kernels call) and
compared with the oracle's format rules:

  * the NVFP4 GEMMs' exact dequantization: all 16 E2M1 codes times all 256
    E4M3 scale bytes through the fp4 -> fp16 and fp8 -> fp16 converters and the
    packed fp16 multiply, against e2m1 x e4m3 (every product is an fp16
    value);
  * the E2M1 -> fp32 decode of the dequantizer and the combine;
  * the MXFP8 GEMMs' exact dequantization: all 256 E8M0 scale bytes times
    all 256 E4M3 bytes through the fp8 -> bf16 scaled converter, against
    e4m3 x 2^(e - 127);
  * every finite fp32 input through the fp32 -> fp4 converter (nearest-even
    E2M1 with saturation and the sign kept), the +-448 clamp with the
    fp32 -> fp8 converter (MXFP8 nearest-even elements), the software E4M3
    encoder (block scales), the bf16 pair converter and the software bf16
    rounding, against the oracle's E2M1, E4M3 and bf16 nearest-even rules.

The sweeps: within one sign, each encoder's output is a monotone step function
of the fp32 bit pattern, and so is each oracle rule (nearest value on a sorted
grid). The GPU reports every pattern where its output changes; the test
evaluates the rule at both ends of every run of equal outputs. Equal at both
ends means equal on the whole run, so all 2^32 - 2^24 finite inputs are
covered. Formats: about 4.5 bits per value for NVFP4 (page "Thinking Machines
Details End-to-End 4-Bit Training for Inkling 2 Small", section "Background"),
E4M3 with E8M0 per 32 for the MXFP8 backward ("Key Takeaways")."""
import numpy as np
import pytest
import torch

import oracle
import precision_moe_numerics_amd as nvq
from gpu_util import host, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


CODES_LO, CODES_HI = 0x76543210, 0xFEDCBA98  # codes 0..7 and 8..15, element j in nibble j


def _e2m1(c):
    return np.float64(oracle.e2m1_decode(c))


def _e4m3(b):
    return np.float64(oracle.e4m3_decode(b))


def test_dequant_chain_fp4_times_e4m3_in_fp16():
    words = []
    for cw in (CODES_LO, CODES_HI):
        for k in range(64):
            sw = (4 * k) | ((4 * k + 1) << 8) | ((4 * k + 2) << 16) | ((4 * k + 3) << 24)
            words.append((cw, sw))
    w = np.array(words, dtype=np.uint32).view(np.int32)
    out = host(nvq.convert_probe(nvq.CVT_DQ_F16, to_dev(w))).view(np.uint16)
    checked, bad_scale, bad = 0, [], []
    for i, (cw, sw) in enumerate(words):
        for j in range(4):
            b = (sw >> (8 * j)) & 0xFF
            if (b & 0x7F) == 0x7F:
                continue  # NaN bytes are never produced
            s_ref = np.float16(_e4m3(b))
            assert np.float64(s_ref) == _e4m3(b)
            if out[i, j] != s_ref.view(np.uint16) and not (b & 0x80 and _e4m3(b) == 0):
                bad_scale.append((b, hex(out[i, j]), hex(s_ref.view(np.uint16))))
            for q in range(8):
                c = (cw >> (4 * q)) & 0xF
                v = _e2m1(c) * _e4m3(b)
                ref = np.float16(v)
                assert np.float64(ref) == v, "every product must be an fp16 value"
                got = out[i, 8 + 8 * j + q]
                if b & 0x80:
                    # negative scale bytes are never produced; compare values
                    ok = np.float64(np.uint16(got).view(np.float16)) == v
                else:
                    ok = got == ref.view(np.uint16)
                if not ok:
                    bad.append((c, b, hex(got), hex(ref.view(np.uint16))))
                checked += 1
    assert checked == 16 * 254
    assert not bad_scale, f"{len(bad_scale)} scale bytes: {bad_scale[:16]}"
    assert not bad, f"{len(bad)} of {checked} products differ (code, byte, got, want): {bad[:40]}"


def test_fp4_to_fp32_decode():
    w = np.array([CODES_LO, CODES_HI], dtype=np.uint32).view(np.int32)
    out = host(nvq.convert_probe(nvq.CVT_FP4_F32, to_dev(w)))
    ref = np.array([oracle.e2m1_decode(c) for c in range(16)], dtype=np.float32).reshape(2, 8)
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))  # -0.0 for code 8 included


def _runs(table, half):
    """(start pattern, end pattern exclusive, output) of every run of equal
    outputs among the finite patterns of one sign half."""
    o = table.view(np.uint32)
    first, cnt, pos, val = o[:, 0], o[:, 1], o[:, 2:10], o[:, 10:18]
    assert not (cnt & 0x80000000).any(), "a range overflowed, or the two values of a converter call disagreed"
    ts = np.arange(half * 32768, half * 32768 + 0x7F80)
    P = np.concatenate([(ts.astype(np.uint64) << 16)[:, None], pos[ts].astype(np.uint64)], axis=1)
    V = np.concatenate([first[ts][:, None], val[ts]], axis=1)
    mask = np.concatenate([np.ones((len(ts), 1), bool), np.arange(8)[None, :] < cnt[ts][:, None]], axis=1)
    P, V = P[mask], V[mask]
    keep = np.concatenate([[True], V[1:] != V[:-1]])
    P, V = P[keep], V[keep]
    end = np.uint64((half * 32768 + 0x7F80) << 16)
    return P, np.append(P[1:], end), V


def _f32(p):
    return float(np.array([p], dtype=np.uint64).astype(np.uint32).view(np.float32)[0])


def _sweep(which, rule, what, expect_runs):
    table = host(nvq.convert_probe(which))
    total = 0
    for half in (0, 1):
        starts, ends, vals = _runs(table, half)
        for s, e, v in zip(starts, ends, vals):
            lo, hi = rule(_f32(s)), rule(_f32(e - 1))
            assert lo == v and hi == v, (what, hex(int(s)), hex(int(e)), hex(int(v)), hex(lo), hex(hi))
        total += len(vals)
    print(f"{what}: {total} runs over all finite fp32 inputs, rule equal at both ends of each")
    assert total == expect_runs


def test_sweep_e2m1_converter():
    # 8 codes per sign (0 .. 6 and their negatives, -0 kept)
    _sweep(nvq.CVT_SCAN_E2M1, oracle.e2m1_rne, "fp32 -> E2M1 converter", 16)


def test_sweep_e4m3_converter_with_clamp():
    # 127 magnitudes (0 .. 448) per sign
    _sweep(nvq.CVT_SCAN_E4M3_HW, oracle.e4m3_rne_sat, "clamp + fp32 -> E4M3 converter", 254)


def test_sweep_e4m3_software_encoder():
    _sweep(nvq.CVT_SCAN_E4M3_SW, oracle.e4m3_rne_sat, "software E4M3 encoder", 254)


def _bf16_rule(x):
    return int(oracle.lib().o_f64_to_bf16_rne(float(x)))


@pytest.mark.parametrize("which,what", [(nvq.CVT_SCAN_BF16_HW, "bf16 pair converter"),
                                        (nvq.CVT_SCAN_BF16_SW, "software bf16 rounding")])
def test_sweep_bf16(which, what):
    # every finite bf16 value plus the rounding to infinity, per sign
    _sweep(which, _bf16_rule, what, 2 * (0x7F80 + 1))


def _sr_cases():
    """fp32 inputs around every E2M1 and E4M3 decision point (grid values,
    midpoints, binade edges, saturation, zero and subnormals, one and two ulps
    either side) and random values, each with the draws that sit at and next
    to its rounding threshold plus 0, 1, 2^15 and 65535."""
    g = np.random.default_rng(77)
    e2 = [0.0, 0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0, 7.0]
    e4 = [float(oracle.e4m3_decode(b)) for b in range(0x7F)] + [450.0, 464.0, 500.0, 2.0 ** -10, 2.0 ** -7]
    pts = []
    for v in e2 + e4 + [1e-30, 1.4e-45]:
        b = int(np.array([v], np.float32).view(np.uint32)[0])
        for db in (-2, -1, 0, 1, 2):
            if 0 <= b + db < 0x7F800000:
                pts.append(b + db)
    pts += list(np.array(g.uniform(0, 7, 3000), np.float32).view(np.uint32))
    pts += list(np.array(np.exp2(g.uniform(-12, 9, 3000)), np.float32).view(np.uint32))
    cases = []
    for b in pts:
        for sign in (0, 0x80000000):
            bb = int(b) | sign
            y = float(np.array([bb], np.uint32).view(np.float32)[0])
            draws = {0, 1, 0x8000, 0xFFFF, int(g.integers(0, 65536))}
            # thresholds: the draw count below f * 2^16 for both grids
            for th in (abs(y) * 131072.0, (abs(y) * 2.0 % 1.0) * 65536.0, (abs(y) % 1.0) * 65536.0):
                t = int(th)
                draws |= {max(0, min(65535, t + dd)) for dd in (-1, 0, 1)}
            for u in draws:
                cases.append((bb, u))
    return np.array(cases, dtype=np.uint32)


def test_stochastic_rounding_decisions_equal_the_oracle():
    """The integer stochastic-rounding decisions of the NVFP4 and MXFP8 SR
    encoders equal the oracle's o_e2m1_sr and o_e4m3_sr (the rule: round up
    iff the 16-bit draw is below the dropped fraction times 2^16) at and next
    to every threshold."""
    cases = _sr_cases()
    out = host(nvq.convert_probe(nvq.CVT_SR, to_dev(cases.view(np.int32)))).view(np.uint32)
    ys = cases[:, 0].view(np.float32)
    bad = []
    for (bb, u), y, o in zip(cases, ys, out):
        c, b = oracle.e2m1_sr(float(y), int(u)), oracle.e4m3_sr(float(y), int(u))
        if (o & 0xF) != c or ((o >> 8) & 0xFF) != b or ((o >> 16) & 0xF) != c or ((o >> 20) & 0xFF) != b \
                or (o >> 31):
            bad.append((hex(int(bb)), int(u), hex(int(o)), c, b))
    print(f"{len(cases)} (value, draw) pairs checked")
    assert not bad, f"{len(bad)} decisions differ (bits, draw, gpu, e2m1, e4m3): {bad[:10]}"


def test_e2m1_stochastic_converter_equals_the_rule_on_every_input():
    """The NVFP4 SR encoders take their E2M1 codes from the gfx950 stochastic
    converter (inputs below 1 rounded up to a multiple of 2^-17, one value per
    call, random operand ~(u << 16)). On the device, for every fp32 value
    with |y| <= 8 of both signs, its codes at draws 0 and 65535 and the first
    draw at which the code changes equal those of the software rule (checked
    against the oracle above); every draw is compared for every 65521st
    value."""
    cnt = host(nvq.convert_probe(nvq.CVT_SR_E2M1_SWEEP)).astype(np.int64)
    n_values = 2 * 0x41000001
    print(f"values with a decision {cnt[1]}, fully compared values {cnt[3]}")
    assert cnt[0] == 0, f"{cnt[0]} values differ"
    assert cnt[2] == 0, f"{cnt[2]} (value, draw) pairs differ"
    assert cnt[3] == -(-n_values // 65521)
    # every value in (0, 6) off the grid has a decision: most of the 2.18e9
    assert 2_100_000_000 < cnt[1] < n_values


def test_e4m3_stochastic_converter_equals_the_rule_on_every_input():
    """The MXFP8 SR requantizers take their E4M3 bytes from the gfx950
    stochastic fp8 converter (inputs below 2^-6 rounded up to a multiple of
    2^-25, above 448 clamped, random operand ~(u << 16) | 0xFFFF). On the
    device, for every fp32 value with |y| <= 512 of both signs, its bytes at
    draws 0 and 65535 and the first draw at which the byte changes equal those
    of the software rule (checked against the oracle above); every draw is
    compared for every 65521st value."""
    cnt = host(nvq.convert_probe(nvq.CVT_SR_E4M3_SWEEP)).astype(np.int64)
    n_values = 2 * 0x44000001
    print(f"values with a decision {cnt[1]}, fully compared values {cnt[3]}")
    assert cnt[0] == 0, f"{cnt[0]} values differ"
    assert cnt[2] == 0, f"{cnt[2]} (value, draw) pairs differ"
    assert cnt[3] == -(-n_values // 65521)
    assert 2_000_000_000 < cnt[1] < n_values


def test_mxfp8_operand_decode_to_bf16():
    """Every (E8M0 scale byte, E4M3 byte) pair through the MXFP8 GEMMs' operand
    decode: bit-exact bf16 of e4m3 * 2^(e - 127) for every scale byte in
    [3, 246] (the products then lie in bf16's range; 2^(e - 127) for e = 0 is
    passed as a zero float whose exponent field the converter reads) and every
    finite E4M3 byte. Outside that range the products need more than bf16's
    range; the test records how the converter rounds them."""
    got = host(nvq.convert_probe(nvq.CVT_DQ_MX_BF16)).view(np.uint16).astype(np.uint32)
    e4 = np.array([oracle.e4m3_decode(c) for c in range(256)])
    finite = np.isfinite(e4)
    assert finite.sum() == 254                      # 0x7F and 0xFF are NaN
    checked = 0
    for e in range(3, 247):
        prod = (e4[finite] * 2.0 ** (e - 127)).astype(np.float32)     # exact: at most 4 significant bits
        assert np.array_equal(prod.astype(np.float64), e4[finite] * 2.0 ** (e - 127))
        bits = prod.view(np.uint32)
        assert not (bits & 0xFFFF).any()            # exact in bf16
        assert np.array_equal(got[e][finite], bits >> 16), f"scale byte {e}"
        checked += int(finite.sum())
    # the rest of the table (products below bf16's subnormals or above its
    # range, NaN codes): recorded, not relied on (the quantizers never emit
    # NaN codes, and their scales stay in the exact range for bf16 inputs
    # whose block maximum is at least 2^-116)
    rne = 0
    for e in list(range(0, 3)) + list(range(247, 255)):
        prod = e4[finite] * 2.0 ** (e - 127)
        with np.errstate(over="ignore"):
            rne += int((got[e][finite] == oracle.f64_to_bf16_fast(prod).astype(np.uint32)).sum())
    nan_kept = sum(int((got[e][c] & 0x7F80) == 0x7F80 and (got[e][c] & 0x7F) != 0)
                   for e in range(3, 247) for c in (0x7F, 0xFF))
    print(f"MXFP8 operand decode: {checked} products bit-exact; outside the exact range {rne} of "
          f"{11 * 254} equal nearest-even bf16; NaN codes decoded to NaN {nan_kept} of {2 * 244} times", flush=True)


def test_e4m3_scale_pair_decode_to_f32():
    """Every pair of E4M3 bytes through the combine's block-scale decode (the
    fp8 -> fp32 pair converter at scale 1): both halves bit-equal to the
    oracle's E4M3 decode for all 254 finite bytes (subnormals, both signs, the
    largest 448), NaN for 0x7F and 0xFF, in either position of the pair."""
    got = host(nvq.convert_probe(nvq.CVT_E4M3_PAIR_F32))
    e4 = np.array([oracle.e4m3_decode(c) for c in range(256)], dtype=np.float64)
    idx = np.arange(65536)
    for half, byte in ((0, idx & 0xFF), (1, idx >> 8)):
        want = e4[byte]
        g = got[:, half].astype(np.float64)
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(g), nan), half
        assert np.array_equal(g[~nan], want[~nan]), half
        # -0 (0x80) keeps its sign
        assert np.array_equal(np.signbit(g[~nan]), np.signbit(want[~nan])), half
