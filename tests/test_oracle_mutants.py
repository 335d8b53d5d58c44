"""Plant plausible mistakes in a temporary copy of the oracle's C source and
check that each one fails at least one pin.  CPU only; the real oracle is not
touched."""
import os
import shutil
import subprocess
import tempfile

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, exact text in oracle.c, replacement)
MUTANTS = [
    ("scatter_pad_sign", "int64_t od = id * s - p + kd;", "int64_t od = id * s + p + kd;"),
    ("scatter_flipped_kernel", "wc[(kd * k + kh) * k + kw]", "wc[((k - 1 - kd) * k + kh) * k + kw]"),
    ("weight_cin_cout_swapped", "const float *wc = w + (ci * Cout + co) * k * k * k;",
     "const float *wc = w + (co * Cin + ci) * k * k * k;"),
    ("pool_divisor_squared", "double divisor = (double)(pk * pk * pk);", "double divisor = (double)(pk * pk);"),
    ("bias_after_scale2", "v = v + (bias ? (double)bias[co] : 0.0);\n            o[(dp * Hp + hp) * Wp + wp] = v * scale2;",
     "o[(dp * Hp + hp) * Wp + wp] = v * scale2 + (bias ? (double)bias[co] : 0.0);"),
    ("scale1_dropped", "for (int64_t i = 0; i < plane; ++i) Y[i] *= scale1;", ""),
    ("conv_bias_dropped", "if (conv_bias)\n            for (int64_t i = 0; i < plane; ++i) Y[i] += (double)conv_bias[co];\n        /* step 2 */", "/* step 2 */"),
    ("pool_window_stride_off", "Y[((dp * ps + a) * Ho + (hp * ps + b)) * Wo + (wp * ps + c)]",
     "Y[((dp * ps + a) * Ho + (hp * ps + b)) * Wo + (wp * ps + c - (wp > 0))]"),
    ("avgpool_no_pad_shift", "int64_t id = od * s - p + kd;", "int64_t id = od * s + kd;"),
    ("avgpool_divisor_count", "double div = count_include_pad ? (double)(k * k * k) : (double)cnt;",
     "double div = (double)cnt;"),
    ("convT1d_dilation_dropped", "int64_t o = i * s - p + dil * kk;", "int64_t o = i * s - p + kk;"),
    ("convT1d_flipped", "yc[o] += v * (double)wc[kk];", "yc[o] += v * (double)wc[K - 1 - kk];"),
    ("convT1d_weight_transposed", "const float *wc = w + (ci * Cout + co) * K;",
     "const float *wc = w + (co * Cin + ci) * K;"),
    ("out_len_no_dilation", "return (in - 1) * stride - 2 * pad + dilation * (k - 1) + out_pad + 1;",
     "return (in - 1) * stride - 2 * pad + (k - 1) + out_pad + 1;"),
    ("pool_len_ceil", "return floor_div(in + 2 * pad - k, stride) + 1;",
     "return floor_div(in + 2 * pad - k + stride - 1, stride) + 1;"),
]


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="oracle_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(workdir, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    path_c = os.path.join(workdir, f"{name}.c")
    path_so = os.path.join(workdir, f"lib{name}.so")
    with open(path_c, "w") as f:
        f.write(src.replace(old, new))
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC",
                    "-shared", "-w", "-o", path_so, path_c], check=True)
    lib = oracle.load_library(path_so)
    failed = []
    for pin in pins.ALL_PINS:
        if pin is pins.pin_flipped_conv1d_equivalence and failed:
            continue
        try:
            pin(lib=lib)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
