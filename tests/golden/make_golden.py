"""Writes tests/golden/oracle_noise.txt from the CPU oracle only (regression fixture).

The pages print no worked example of the estimator, so the stored values are the oracle's own:
Philox4x32-10 words and the normals of channels 4q..4q+3 at fixed (seed, tag, draw, token, q),
chosen to cover zero and all-ones counter words. The words themselves are pinned independently
against rocRAND's engine (tests/test_oracle_generator.py); this file guards against accidental
changes of the oracle afterwards.

    python tests/golden/make_golden.py
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402

CASES = [
    (0, 0, 0, 0, 0),
    (1, 1, 0, 0, 0),
    (0x0D057002, 1, 63, 16383, 511),
    (0x0D057004, 0x100, 16383, 1023, 127),
    (0xFFFFFFFFFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF),
    (0x123456789ABCDEF0, 7, 12345, 678, 9),
]

if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_noise.txt")
    with open(out, "w") as f:
        f.write("# seed tag draw token q | w0 w1 w2 w3 | n(4q) n(4q+1) n(4q+2) n(4q+3)\n")
        f.write("# written by tests/golden/make_golden.py from the CPU oracle\n")
        for seed, tag, draw, token, q in CASES:
            w = oracle.noise_words(seed, tag, draw, token, q)
            n = [oracle.normal(seed, tag, draw, token, 4 * q + e) for e in range(4)]
            f.write("%d %d %d %d %d | %s | %s\n" % (seed, tag, draw, token, q,
                                                    " ".join(str(int(x)) for x in w),
                                                    " ".join(repr(float(x)) for x in n)))
    print(out)
