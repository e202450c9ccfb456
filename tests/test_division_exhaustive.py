"""The quantize kernel's quotient equals IEEE binary32 division for every
pair of operands it can meet (every finite fp16 dividend, every positive
finite fp16 divisor): the coding rules divide by the stored scale ("Loading
a model in 4-bit", "Block-wise quantisation, stated exactly"), and the kernel
forms that quotient as a correctly rounded reciprocal plus Markstein's
correction.  The sweep (about 2e9 pairs) is plain C, compiled here with gcc
and run on the host CPU."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.slow
@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_markstein_quotient_is_ieee_for_all_fp16_pairs(tmp_path):
    exe = str(tmp_path / "markstein_sweep")
    subprocess.run(["gcc", "-O2", "-mfma", "-ffp-contract=off", "-fno-fast-math",
                    os.path.join(HERE, "native", "markstein_sweep.c"), "-lm", "-o", exe],
                   check=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    last = out.stdout.strip().splitlines()[-1]
    # 63488 finite fp16 dividends x 31743 positive finite fp16 divisors
    assert last == "pairs=2015299584 mismatches=0", out.stdout
    assert out.returncode == 0
    # the product by the reciprocal alone is not the IEEE quotient: the sweep
    # must see that
    bad = subprocess.run([exe, "uncorrected"], capture_output=True, text=True, timeout=600)
    n_bad = int(bad.stdout.strip().splitlines()[-1].split("mismatches=")[1])
    assert n_bad > 0


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_scale_quotients_and_reciprocal_are_ieee(tmp_path):
    """The INT4 scales divide by the constants 7 (sym: absmax / 7) and 15
    (asym: (hi - lo) / 15) before the fp16 rounding ("How 4-bit quantization
    works"; "INT4", "How it works"); the kernel forms these quotients with
    the constant reciprocal and Markstein's correction, and each group's
    reciprocal 1 / s from the hardware reciprocal and one Newton step.  Every
    operand they can meet is swept (about 1e9 values of hi - lo), in plain C
    on the host."""
    exe = str(tmp_path / "scale_div_sweep")
    subprocess.run(["gcc", "-O2", "-mfma", "-ffp-contract=off", "-fno-fast-math",
                    os.path.join(HERE, "native", "scale_div_sweep.c"), "-lm", "-o", exe],
                   check=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    lines = out.stdout.strip().splitlines()
    assert lines[-3] == "div7 operands=31744 mismatches=0", out.stdout
    assert lines[-2] == "div15 operands=1007681536 mismatches=0", out.stdout
    # the per-group reciprocal: 31743 positive fp16 s x 5 starting values
    assert lines[-1] == "rcp cases=158715 mismatches=0", out.stdout
    assert out.returncode == 0
    # without the correction steps the results differ: the sweep sees that
    bad = subprocess.run([exe, "uncorrected"], capture_output=True, text=True, timeout=600)
    counts = [int(l.split("mismatches=")[1]) for l in bad.stdout.strip().splitlines()[-3:]]
    assert all(c > 0 for c in counts)
