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
