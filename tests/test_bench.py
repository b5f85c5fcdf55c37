"""Host logic of bench.py (no GPU): the byte model, the code hash that ties the
committed counter traffic to the kernel code, and the one-GPU guard."""
import os
import subprocess
import sys

import bench
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_of_the_workloads():
    # 16 ranks x 256 tokens, h=7168, top-8, int8 rows: x + ids + rows + assist + counts + scales,
    # then the combine's bf16 rows + ids + assist + counts + weights + x_out
    d, c = bench.algorithmic_bytes(wl.BY_NAME["w16_h7168_bf16_q8"])
    assert (d, c) == (294273024, 529154048) and d + c == 823427072
    d8, c8 = bench.algorithmic_bytes(wl.BY_NAME["w8_h7168_fp16_uniform"])
    assert d8 + c8 == 66138112
    # the FP8 variant writes 1-byte codes too and ceil(7168/128) = 56 fp32 scales per row
    d3, c3 = bench.algorithmic_bytes(wl.BY_NAME["w16_h7168_bf16_fp8g128"])
    assert c3 == c
    assert d3 == 294273024 - 32768 * 4 + 32768 * 56 * 4
    # static int8: no row scales written, the 256 x 7168 fp32 coefficients read once
    d1, c1 = bench.algorithmic_bytes(wl.BY_NAME["w16_h7168_bf16_static_q8"])
    assert c1 == c and d1 == 294273024 - 32768 * 4 + 256 * 7168 * 4


def test_masked_and_special_bytes_count_only_rows_that_move():
    # brute force over the pairs: a row moves for an active pair of a real expert; a copy-expert pair makes the
    # combine read its token; x is read for tokens with a row; the mask is read by both calls; the const
    # experts' table is read once
    import numpy as np
    for name in ("w16_h7168_bf16_q8_pair_mask", "w16_h7168_bf16_q8_special"):
        w = wl.BY_NAME[name]
        inp = wl.make_inputs(w)
        N, K, h, E = w.num_tokens, w.topk, w.h, w.num_experts
        rows = copies = toks = 0
        for t in range(N):
            has = False
            for k in range(K):
                on = True if "mask" not in inp else bool(inp["mask"][t, k] if inp["mask"].ndim == 2
                                                           else inp["mask"][t])
                e = int(inp["ids"][t, k])
                if on and e < E:
                    rows += 1
                    has = True
                if on and E + w.zero_experts <= e < E + w.zero_experts + w.copy_experts:
                    copies += 1
            toks += has
        mb = inp["mask"].size if "mask" in inp else 0
        erc = w.ep_world * E * 4
        want_d = toks * h * 2 + N * K * 4 + mb + rows * h + rows * 12 + erc + rows * 4
        # the const experts' outputs are read once
        want_c = (rows * h * 2 + copies * h * 2 + w.const_experts * h * 2 + N * K * 4 + mb + rows * 12 + erc
                  + N * K * 4 + N * h * 2)
        assert bench.algorithmic_bytes(w, inp) == (want_d, want_c), name
        assert 0 < rows < w.rows


def test_code_hash_ignores_comments_and_spacing_only(tmp_path):
    a = tmp_path / "a.hip"
    a.write_text('const char *s = "x // y /* z */";  // note\nint f() { return 1; } /* block\ncomment */\n')
    b = tmp_path / "b.hip"
    b.write_text('const char *s = "x // y /* z */";\n\n// another note\nint f() {  return 1;  }\n')
    c = tmp_path / "c.hip"
    c.write_text('const char *s = "x // y /* z */";\nint f() { return 2; }\n')
    d = tmp_path / "d.hip"
    d.write_text('const char *s = "x // y";\nint f() { return 1; }\n')
    assert bench.code_hash(str(a)) == bench.code_hash(str(b))
    assert bench.code_hash(str(a)) != bench.code_hash(str(c))
    assert bench.code_hash(str(a)) != bench.code_hash(str(d))      # string contents count


def test_committed_traffic_matches_the_kernel_code():
    """profiles/ holds counter traffic for the kernels as they are now."""
    got = bench.counted_traffic(wl.BY_NAME["w16_h7168_bf16_q8"])
    assert got is not None, "the kernel code changed since the FETCH_SIZE / WRITE_SIZE runs"
    assert 1.0 <= got / 529154048 <= 1.02


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
