"""Memory-safety check of the float64 oracles (CPU only): both C oracles are
built with AddressSanitizer and run, in a child process that preloads the
sanitizer runtime, on small cases that reach every code path (zero and given
initial state, T = 1, lengths that are not a multiple of anything, the
backward pass, the sLSTM cell).  Any out-of-bounds access or use after free
aborts the child; its results must also equal those of the regular build."""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = textwrap.dedent(r"""
    import sys
    import numpy as np
    sys.path.insert(0, sys.argv[1])
    import oracle
    from oracle import slstm
    asan_m, asan_s = sys.argv[2], sys.argv[3]
    ref_m, san_m = oracle.Oracle(oracle.LIB), oracle.Oracle(asan_m)
    ref_s, san_s = slstm.SlstmOracle(slstm.LIB), slstm.SlstmOracle(asan_s)
    rng = np.random.default_rng(11)

    def same(a, b, what):
        for x, y in zip(a, b):
            x, y = np.asarray(x), np.asarray(y)
            assert x.shape == y.shape and np.allclose(x, y, rtol=0, atol=1e-12), what

    for T in (1, 7, 33):
        for state in (False, True):
            P, dk, dv = 3, 16, 24
            q, k = rng.normal(size=(P, T, dk)), rng.normal(size=(P, T, dk)) / 4
            v, o = rng.normal(size=(P, T, dv)), rng.normal(size=(P, T, dv))
            i, f = rng.normal(size=(P, T)), -np.log1p(np.exp(-rng.normal(3, 1, size=(P, T))))
            st = (rng.normal(size=(P, dk, dv)) * .1, rng.normal(size=(P, dk)) * .1,
                  rng.normal(size=P)) if state else (None, None, None)
            same(ref_m.forward(q, k, v, i, f, o, *st, threads=2),
                 san_m.forward(q, k, v, i, f, o, *st, threads=2), f"forward T={T} state={state}")
            dh = rng.normal(size=(P, T, dv))
            same(ref_m.backward(q, k, v, i, f, o, dh, *st, threads=2),
                 san_m.backward(q, k, v, i, f, o, dh, *st, threads=2), f"backward T={T} state={state}")
            B, H, d = 2, 2, 8
            gx, R = rng.normal(size=(B, H, T, 4, d)), rng.normal(size=(H, 4, d, d)) * .3
            sst = tuple(rng.normal(size=(B, H, d)) for _ in range(4)) if state else (None,) * 4
            if state:
                sst = (sst[0], np.abs(sst[1]) + 1, sst[2], sst[3])
            ra, (ca, na, ma, ha) = ref_s.forward(gx, R, *sst, threads=2)
            rb, (cb, nb, mb, hb) = san_s.forward(gx, R, *sst, threads=2)
            same((ra, ca, na, ma, ha), (rb, cb, nb, mb, hb), f"slstm T={T} state={state}")
    print("asan child OK")
""")


def test_oracles_under_address_sanitizer(tmp_path):
    import oracle
    from oracle import slstm
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True).stdout.strip()
    if not libasan or not os.path.exists(libasan):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    oracle.load()
    slstm.load()
    flags = ("-fsanitize=address", "-fno-omit-frame-pointer", "-g")
    am = oracle.build(out=str(tmp_path / "libmlstm_ref_asan.so"), extra_flags=flags)
    sm = str(tmp_path / "libslstm_ref_asan.so")
    subprocess.run(["gcc", "-std=c99", "-O1", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Werror", *flags,
                    slstm.SRC, "-o", sm, "-lm"], check=True)
    env = dict(os.environ, LD_PRELOAD=libasan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT, am, sm], env=env, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0 and "asan child OK" in r.stdout, r.stdout[-3000:] + r.stderr[-3000:]
