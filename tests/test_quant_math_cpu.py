"""The FP8 quantiser's arithmetic, checked on the CPU.

The kernel replaces the correctly rounded quotient fl32(w / s) by a product
with one FMA correction (t = w * rs, r = fma(-t, s, w), y = -fma(-r, rs, -t))
on rows whose scale s = fl32(amax / 448) is at least 2^-100.  The codes are
what must match: tests/native/quant_fma_codes.c checks every BF16 weight of
every such row (all positive finite BF16 amax, about 1.04e9 pairs) against the
division, both encoded by the oracle's E4M3FN encoder.  The hardware convert
the kernel encodes with is checked on the GPU (mtp_probe_fp8_convert)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_fma_quotient_gives_the_division_codes(tmp_path):
    exe = str(tmp_path / "quant_fma_codes")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-pthread",
                    os.path.join(ROOT, "tests", "native", "quant_fma_codes.c"),
                    os.path.join(ROOT, "oracle", "oracle.c"), "-o", exe, "-lm"], check=True)
    n = max(1, min(16, len(os.sched_getaffinity(0))))
    r = subprocess.run([exe, str(n)], capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout + r.stderr
    pairs = int(r.stdout.split()[1])
    assert pairs > 1_000_000_000, r.stdout
