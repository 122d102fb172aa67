"""The library's host code under AddressSanitizer.

`tests/asan/host_asan.cpp` is linked with api.cpp compiled with the sanitizer
on host code only (`shared_prefix_scoring_amd/build.py` builds it beside the
library as `lib/duolm_host_asan`; device code is unchanged).  Every buffer it
hands to the library has exactly its stated size, so any read or write past
one, any use after free and (on the CPU) any leak aborts the run.
- CPU: the request packer on random structured requests (checked against a
  plain assembly of the same ids, on 0 to 64 threads) and its error paths.
- GPU: the executor -- planning, descriptor upload, graph cache, two lanes,
  independent mode, the packed host path, sessions and error paths -- on the
  tiny model, with scores compared across entry points bit for bit.
"""
import os
import subprocess

import pytest

import synth
import shared_prefix_scoring_amd as spa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "shared_prefix_scoring_amd", "lib", "duolm_host_asan")


def _run(args, asan_options, timeout):
    env = dict(os.environ, ASAN_OPTIONS=asan_options)
    return subprocess.run([EXE, *args], env=env, capture_output=True, text=True, timeout=timeout)


def test_packer_under_asan():
    if not os.path.exists(EXE):
        from shared_prefix_scoring_amd import build
        build.build()
    if not os.path.exists(EXE):
        pytest.skip("the toolchain could not build the host-sanitizer driver (see the build warning)")
    r = _run(["pack"], "detect_leaks=1:abort_on_error=1", 600)
    assert r.returncode == 0, r.stderr[-4000:]
    assert r.stdout.startswith("ok pack"), r.stdout


@pytest.mark.gpu
def test_executor_under_asan(tmp_path):
    assert os.path.exists(EXE), "build the library first (it builds the sanitizer driver beside it)"
    path = tmp_path / "tiny.duolmw"
    path.write_bytes(spa.weights_blob(synth.TINY, synth.make_weights(synth.TINY, seed=0)))
    # the HIP runtime keeps allocations until exit: leaks are not checked here
    r = _run(["score", str(path)], "detect_leaks=0:abort_on_error=1", 300)
    print(r.stdout.strip())
    assert r.returncode == 0, r.stderr[-4000:]
    assert r.stdout.startswith("ok score"), r.stdout
