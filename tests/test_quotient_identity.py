"""The fp8 dispatch kernel divides by the block scale with a reciprocal and one
remainder-correction step instead of an IEEE division per element.  This
checks, exhaustively over every bf16 input pair, that the shortcut yields the
same e4m3fn byte as the IEEE-rounded quotient the method specifies, with the
reciprocal correctly rounded and also one ulp below or above it (the device
takes it from v_rcp_f32 and a Newton step; the GPU parity tests then compare
the kernel itself against the oracle)."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("qid") / "quotient_identity")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math",
                    os.path.join(HERE, "quotient_identity.c"),
                    os.path.join(ROOT, "oracle", "ep_oracle.c"), "-o", exe, "-lm"], check=True)
    return exe


def _run_all(checker, stride, negatives):
    # the correctly rounded reciprocal and its two neighbours, in parallel
    procs = [subprocess.Popen([checker, stride, negatives, yoff], stdout=subprocess.PIPE, text=True)
             for yoff in ("0", "-1", "1")]
    for p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, out
        assert "differing bytes 0" in out, out


@pytest.mark.slow
def test_all_positive_pairs(checker):
    _run_all(checker, "1", "0")


def test_negative_pairs_strided(checker):
    _run_all(checker, "37", "1")
