"""Host logic of the benchmark (CPU): the key that ties a PMC traffic record to its kernels'
code, and the algorithmic byte counts the roofline fractions divide by."""
import os
import shutil

import bench


def _copy_sources(tmp, kind):
    for f in bench._traffic_spec(kind)[1]:
        dst = os.path.join(tmp, f)
        os.makedirs(os.path.dirname(dst), exist_ok=True)
        shutil.copy(os.path.join(bench.ROOT, f), dst)


def test_traffic_key_ignores_comments_and_follows_code(tmp_path, monkeypatch):
    tmp = str(tmp_path)
    for kind in ("fa", "gateup"):
        _copy_sources(tmp, kind)
    monkeypatch.setattr(bench, "ROOT", tmp)
    base = {k: bench.kernel_source_hash(k) for k in ("fa", "gateup")}
    src = os.path.join(tmp, "session_decode_step_amd/csrc/attn.hip")
    text = open(src).read()
    # comments and blank space changed: the same key
    open(src, "w").write("// a note\n" + text.replace("\n\n", "\n\n  /* aside */\n\n", 1) + "\n   \n")
    assert bench.kernel_source_hash("fa") == base["fa"]
    # one constant of the code changed: another key, and the products' key is untouched
    assert "kFaMinChunk = 128;" in text
    open(src, "w").write(text.replace("kFaMinChunk = 128;", "kFaMinChunk = 256;"))
    assert bench.kernel_source_hash("fa") != base["fa"]
    assert bench.kernel_source_hash("gateup") == base["gateup"]


def test_algorithmic_bytes_of_the_headline_kernels():
    # fa_decode: each row's K and V once (fp16) plus q in and the output out (fp32)
    t = [4113] * 8
    assert bench.fa_algorithmic_bytes(t, 8, 32, 128) == sum(t) * 8 * 128 * 2 * 2 + 2 * 8 * 32 * 128 * 4
    # a Q4_0 matrix: 18 bytes per 32 weights
    assert bench.w_bytes("q4_0", 28672, 4096) == 28672 * 4096 * 18 // 32
    assert bench.w_bytes("q8_0", 32000, 2048) == 32000 * 2048 * 34 // 32
