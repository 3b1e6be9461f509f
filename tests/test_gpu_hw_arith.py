"""The gfx950 arithmetic facts the exact K decode of the decode-attention scores kernel and the
encoders rest on, checked exhaustively on the GPU by tests/native/hw_arith_check (built by build()):

* a BF16 pair summed by v_dot2_f32_bf16 against (1, 1), then rounded to BF16, equals the BF16
  rounding of the v_add_f32 sum, for every pair of +0 / finite normal BF16 values;
* v_fma_mix_f32 with the code as a binary16 denormal times s * 2^24 plus the binary16 minimum
  equals fma(code, s, m), for every finite non-negative binary16 scale, every code and 512
  minima;
* the encoders' three-instruction RN(x / 15) equals the IEEE division for every finite
  binary32 x >= +0;
* v_cvt_scalef32_pk_f32_fp8 with scale 1 gives the E4M3 value of both bytes, in either half of
  the word, for every pair of non-negative finite E4M3 bytes (the NVFP4 block scales).
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "native", "hw_arith_check")


@pytest.mark.gpu
def test_hw_arith_facts():
    assert os.path.exists(EXE), "tests/native/hw_arith_check is not built (run __graft_entry__.build())"
    print("running hw_arith_check", flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=90)
    sys.stdout.write(r.stdout)
    vals = {}
    for ln in r.stdout.split("\n"):
        parts = ln.split()
        for k, v in zip(parts[0::2], parts[1::2]):
            vals[k] = int(v)
    assert r.returncode == 0, r.stdout + r.stderr
    # every pair of the domain: (2 * 254 * 128 + 1)^2
    assert vals["dot2_pairs"] == (2 * 254 * 128 + 1) ** 2
    assert vals["dot2_bf16_mismatch"] == 0
    assert vals["fma_mix_cases"] == 0x7C00 * 512 * 16
    assert vals["fma_mix_mismatch"] == 0
    # every finite binary32 x >= +0
    assert vals["div15_cases"] == 0x7F800000
    assert vals["div15_mismatch"] == 0
    assert vals["e4m3_pairs"] == 127 * 127
    assert vals["e4m3_mismatch"] == 0

