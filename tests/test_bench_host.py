"""Host-side checks of bench.py (CPU): the algorithmic byte counts behind the roofline figures,
worked out by hand from the tensor sizes, and the one-GPU contract."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_prefill_bytes_per_head_token():
    # q, k, alpha, b, v, w in bf16: 6 x 128 x 2 = 1536; o in fp32: 512; S0 read and S_T written
    # (2 x 128 x 128 x 4 = 131072) over T = 4096 tokens: 32
    assert bench.prefill_bytes_per_head_token(128, 128, 4096) == 1536 + 512 + 32
    assert bench.prefill_bytes_per_head_token(32, 32, 256) == 6 * 32 * 2 + 32 * 4 + 2 * 32 * 32 * 4 / 256
    # fp32 inputs: 6 x 128 x 4 = 3072, o 512, the states 32
    assert bench.prefill_bytes_per_head_token(128, 128, 4096, 4) == 3072 + 512 + 32


def test_decode_bytes_per_head():
    # the fp32 state read and written (2 x 65536), six bf16 vectors (1536), o in fp32 (512)
    assert bench.decode_bytes_per_head(128, 128) == 131072 + 1536 + 512 == 133120


def test_backward_bytes_per_head_token():
    # inputs 1536 (bf16), dO 512 (fp32), dq dk dalpha db dv dw 6 x 512 (fp32), S0 and dS_T read
    # and dS0 written amortised (3 x 65536 / 4096 = 48)
    assert bench.bwd_bytes_per_head_token(128, 128, 4096) == 1536 + 512 + 3072 + 48 == 5168


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_sources_digest_ignores_comments_and_layout_only():
    import bench
    a = 'int f(int x) { return x + 1; }  // one\n/* two */ const char* s = "// kept";\n'
    b = 'int f(int x)\n{\n    return x + 1;  /* changed comment */\n}\nconst char* s = "// kept";'
    c = 'int f(int x) { return x + 2; }\nconst char* s = "// kept";'
    d = 'int f(int x) { return x + 1; }\nconst char* s = "// changed";'
    assert bench._code_only(a).replace(" ", "") == bench._code_only(b).replace(" ", "")
    assert bench._code_only(a) != bench._code_only(c)
    assert bench._code_only(a) != bench._code_only(d)
    assert bench.sources_digest("split") != bench.sources_digest("fused")
