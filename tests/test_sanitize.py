"""The host-side checks of libcachegen (csrc/cg_host.cpp) and the CPU oracle
under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

tests/native/fault_corpus.cpp feeds both truncated, bit-flipped, overwritten
and resized table images and blobs, bad parameters and bad controller inputs;
every case must end in an error code (or a decode flagged corrupt) with no
sanitizer report.  A planted out-of-bounds read in a throwaway program checks
that the sanitizer build does catch one here."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kv_cache_compression_anchor_amd", "csrc")
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer"]
ENV = dict(os.environ,
           ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")

pytestmark = pytest.mark.skipif(not (shutil.which("gcc") and shutil.which("g++")),
                                reason="needs gcc and g++")


def run(cmd, **kw):
    return subprocess.run(cmd, capture_output=True, text=True, env=ENV, timeout=300, **kw)


@pytest.fixture(scope="module")
def corpus_binary(tmp_path_factory):
    d = tmp_path_factory.mktemp("san")
    obj = str(d / "cgoracle.o")
    r = run(["gcc", "-std=gnu11", *SAN, "-ffp-contract=off", "-I", os.path.join(ROOT, "oracle"),
             "-c", os.path.join(ROOT, "oracle", "cgoracle.c"), "-o", obj])
    if r.returncode != 0 and "sanitize" in r.stderr:
        pytest.skip("no sanitizer runtime: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr
    exe = str(d / "fault_corpus")
    r = run(["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
             "-I", os.path.join(ROOT, "oracle"), os.path.join(CSRC, "cg_host.cpp"),
             os.path.join(ROOT, "tests", "native", "fault_corpus.cpp"), obj, "-lm", "-o", exe])
    assert r.returncode == 0, r.stderr
    return exe


def test_fault_corpus_is_clean_under_sanitizers(corpus_binary):
    r = run([corpus_binary])
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "fault corpus ok" in r.stdout
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-4000:]


def test_sanitizer_build_catches_a_planted_overread(tmp_path):
    src = tmp_path / "planted.c"
    src.write_text("#include <stdlib.h>\n"
                   "int main(int argc, char** argv) {\n"
                   "  (void)argv;\n"
                   "  int* a = (int*)malloc(4 * sizeof(int));\n"
                   "  for (int i = 0; i < 4; i++) a[i] = i;\n"
                   "  int s = a[3 + argc];  /* one past the end */\n"
                   "  free(a);\n"
                   "  return s == 12345;\n"
                   "}\n")
    exe = str(tmp_path / "planted")
    r = run(["gcc", *SAN, str(src), "-o", exe])
    if r.returncode != 0 and "sanitize" in r.stderr:
        pytest.skip("no sanitizer runtime")
    assert r.returncode == 0, r.stderr
    r = run([exe])
    # whichever sanitizer sees it first: ASan's heap check or UBSan's object size
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr or "runtime error: load" in r.stderr, r.stderr
