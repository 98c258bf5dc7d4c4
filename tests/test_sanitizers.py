"""Host AddressSanitizer / UndefinedBehaviorSanitizer runs (CPU only).

* The oracle's C code, built with gcc's ASan and UBSan, runs every function
  on small inputs (ragged tails, K above the block count, fp32 and bf16,
  windows, FP8 codes) and every invalid-argument path.
* The C-ABI library, its host code built with clang's ASan and UBSan (the
  device code is compiled as usual), runs every argument-validation and
  workspace-size path of the ABI tests plus a sweep of extreme sizes.  No GPU
  is touched: every call fails validation or only computes a size.

Each run happens in a child process with the sanitizer runtime preloaded and
halts on the first report, so a report fails the test.
"""
import glob
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_attention_index_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"


def _run_child(code, env_extra, timeout=300):
    env = dict(os.environ, **env_extra)
    r = subprocess.run([sys.executable, "-c", textwrap.dedent(code)], env=env,
                       capture_output=True, text=True, timeout=timeout)
    assert r.returncode == 0, f"child failed ({r.returncode}):\n{r.stdout[-4000:]}\n{r.stderr[-6000:]}"
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-6000:]
    return r.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.check_call([
        "gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
        "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
        "-o", lib, os.path.join(ROOT, "oracle", "msa_oracle.c"), "-lm"])
    asan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    out = _run_child(f"""
        import sys
        sys.path.insert(0, {ROOT!r})
        import numpy as np
        import oracle
        oracle._LIB = {lib!r}
        rng = np.random.default_rng(0)
        for (T, B, K, G, hkv, d, di) in [(300, 16, 5, 2, 2, 32, 24), (97, 64, 8, 4, 1, 64, 7),
                                         (1, 16, 1, 1, 1, 8, 1), (1000, 128, 3, 8, 2, 16, 128)]:
            ik = rng.standard_normal((T, di)).astype(np.float32)
            iq = rng.standard_normal((T, di)).astype(np.float32)
            km = oracle.pool(ik, B)
            oracle.pool_mean(ik, B)
            pos = np.arange(T, dtype=np.int64)
            for w in range(1, min(K, 3) + 1):
                sel, gr, ga, eb = oracle.select(iq, pos, km, B, K, window=w)
            rp, ql, sl = oracle.invert(sel, km.shape[0])
            oracle.counts(sel, pos, B)
            q = rng.standard_normal((T, G * hkv, d)).astype(np.float32)
            k = rng.standard_normal((hkv, T, d)).astype(np.float32)
            v = rng.standard_normal((hkv, T, d)).astype(np.float32)
            oracle.attend(q, k, v, pos, pos, sel, B, 0.3, oracle.F32)
            bits = lambda a: (a.view(np.uint32) >> 16).astype(np.uint16)
            oracle.attend(bits(q), bits(k), bits(v), pos, pos, sel, B, 0.3, oracle.BF16)
        codes = np.arange(256, dtype=np.uint8).reshape(2, 2, 64)
        oracle.dequant_e4m3(codes, np.ones((2, 2), np.float32))
        # invalid arguments are refused, never dereferenced
        L = oracle._load()
        assert L.oracle_pool(None, 10, 4, 16, None) != 0
        assert L.oracle_select_window(None, 1, None, None, 1, 4, 16, 4, 1, None, None, None,
                                      None) != 0
        bad = np.array([[5, 0]], np.int32)
        try:
            oracle.invert(bad, 3)
            raise SystemExit("invert accepted a block index out of range")
        except ValueError:
            pass
        try:
            oracle.attend(q, k, v, pos[:1], pos[:1], np.array([[999]], np.int32), B, 0.3,
                          oracle.F32)
            raise SystemExit("attend accepted a future block")
        except ValueError:
            pass
        print("oracle clean")
    """, {"LD_PRELOAD": asan, "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
          "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1", "OMP_NUM_THREADS": "4"})
    assert "oracle clean" in out


def test_abi_validation_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    runtimes = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not runtimes:
        pytest.skip("clang ASan runtime not available")
    srcs = ["msa_api.cpp", "pool.hip", "topk.hip", "invert.hip", "prefill.hip",
            "prefill_mfma.hip", "decode.hip"]
    procs, objs = [], []
    for s in srcs:
        obj = str(tmp_path / (os.path.splitext(s)[0] + ".o"))
        objs.append(obj)
        cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-sanitize-recover=all",
               "-Xarch_host", "-fno-omit-frame-pointer",
               f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "-c",
               os.path.join(CSRC, s), "-o", obj]
        procs.append(subprocess.Popen(cmd, stdout=subprocess.DEVNULL, stderr=subprocess.PIPE))
    for p, s in zip(procs, srcs):
        _, err = p.communicate(timeout=600)
        assert p.returncode == 0, f"{s}: {err.decode()[-3000:]}"
    lib = str(tmp_path / "libmsa_san.so")
    subprocess.check_call([CLANG, "-shared", "-fPIC", "-shared-libsan",
                           "-fsanitize=address,undefined", "-o", lib, *objs,
                           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    out = _run_child(f"""
        import sys
        sys.path.insert(0, {ROOT!r})
        sys.path.insert(0, {os.path.join(ROOT, 'tests')!r})
        import ctypes
        from block_sparse_attention_index_amd import ops
        ops.LIB_PATH = {lib!r}
        lib = ops.load()
        import test_abi
        n = 0
        for name in sorted(dir(test_abi)):
            if name.startswith("test_"):
                getattr(test_abi, name)(lib)
                n += 1
        # size queries over extreme arguments: defined behaviour, no overflow
        big = [1, 7, 4096, 1 << 20, 1 << 31, 1 << 40, (1 << 62)]
        for n_q in big:
            for B in (16, 512, 4096):
                for K in (1, 8, 64):
                    lib.msa_prefill_workspace_bytes(1, 0, n_q, 64, 128, B, K)
                    lib.msa_prefill_workspace_bytes(0, n_q, 7, 64, 256, B, K)
                    lib.msa_invert_workspace_bytes(n_q, K, 1 << 20)
                    lib.msa_topk_decode_workspace_bytes(1 << 16, n_q, K)
                    lib.msa_decode_step_workspace_bytes(1 << 16, n_q, 64, 128, B, K)
                    lib.msa_decode_workspace_bytes(1 << 16, 1 << 16, 128, B, K)
        # entry points with extreme sizes, fake pointers and an empty workspace:
        # every call is refused (bad shape, or workspace too small) before any launch
        P = ctypes.c_void_p(0x1000)
        for n_q in big + [-1, -(1 << 62)]:
            assert lib.msa_invert_selection(P, n_q, 8, 100, P, P, P, P, 0, None) in (-1, -3)
            assert lib.msa_sparse_gqa_prefill(P, P, P, 1, 1 << 62, n_q, n_q, 64, 8, 128, 64, P,
                                              16, P, P, P, 0.1, P, None, P, 0, None) in (-1, -3)
            c = (ctypes.c_int64 * 3)(0, n_q, 2 * n_q)
            lib.msa_prefill_varlen_workspace_bytes(1, 2, c, c, 64, 128, 128, 64, 8)
            assert lib.msa_prefill_varlen(P, P, P, P, P, 1, 2, c, c, 64, 8, 128, 128, 64, 8, 0.1,
                                          P, P, None, P, 0, None) in (-1, -3)
        print("abi clean", n)
    """, {"LD_PRELOAD": runtimes[0], "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
          "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1", "HIP_VISIBLE_DEVICES": ""})
    assert "abi clean" in out
