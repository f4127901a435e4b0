"""The combine's list-path kernels (link and merge, cut from csrc/combine.hip) built for the host
and run with each workgroup's threads as host threads and __syncthreads as a barrier over them,
under AddressSanitizer where the compiler has it.  Random arrival streams (retries, stale
generations, out-of-range tokens, several calls, multi-arrival tokens) against the oracle, bit
for bit on integer-toy rows with power-of-two weights (sums exact in any order, [NOTES]
numerical contract), for every vectors-per-thread variant of the merge.  On the host a wave
runs no faster than another, so a kernel that needs every wave of a workgroup to pass a point
before some other thread acts shows up here rather than as a rare GPU fault."""
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(HERE)
SRC = os.path.join(REPO, "asynchronous_moe_expert_amd", "csrc", "combine.hip")


def _kernels_source() -> str:
    src = open(SRC).read()
    a = src.index("template <typename T>\nstruct RowIO;")
    b = src.index("constexpr int kRelThreads")
    body = src[a:b]
    # empty asm statements only order the compiler's scheduling on the GPU; drop them
    return re.sub(r"asm volatile\(.*?\);", "/* (asm ordering statement) */", body, flags=re.S)


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    d = tmp_path_factory.mktemp("combine_host")
    open(d / "combine_kernels.inc", "w").write(_kernels_source())
    out = d / "combine_host"
    base = [gxx, "-std=c++20", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", f"-I{d}", f"-I{os.path.join(HERE, 'host_build')}",
            f"-I{os.path.join(REPO, 'include')}", f"-I{os.path.dirname(SRC)}", "-I/opt/rocm/include",
            os.path.join(HERE, "host_build", "combine_host.cpp"),
            "-o", str(out), "-lpthread"]
    r = subprocess.run(base[:2] + ["-fsanitize=address", "-fno-omit-frame-pointer"] + base[2:], capture_output=True,
                       text=True)
    if r.returncode != 0:  # (no AddressSanitizer runtime): plain build
        r = subprocess.run(base, capture_output=True, text=True)
    if r.returncode != 0:  # (a compiler that cannot build the kernels is a failure, not a skip)
        pytest.fail("host build failed: " + r.stderr[-1200:])
    return str(out)


def _stream(rng, T, K, extra):
    """Every (token, position) once in random order plus `extra` retries of delivered positions,
    stale generations and out-of-range tokens (as the GPU property test draws them)."""
    arr = [(t, j) for t in range(T) for j in range(K)]
    arr = [arr[i] for i in rng.permutation(len(arr))]
    stream = [(i, t, j, 0) for i, (t, j) in enumerate(arr)]
    for x in range(extra):
        kind = int(rng.integers(0, 3))
        t, j = arr[int(rng.integers(0, len(arr)))]
        item = (len(arr) + x, T + 3, j, 0) if kind == 2 else (len(arr) + x, t, j, 7 if kind == 1 else 0)
        stream.insert(int(rng.integers(0, len(stream) + 1)), item)
    return stream, len(arr) + extra


@pytest.mark.parametrize("H,K,T,calls,extra,seed", [
    (64, 4, 40, 3, 12, 1),      # one 8-element vector per thread
    (4096, 8, 12, 2, 8, 2),     # two per thread (the prefill hidden size)
    (8192, 3, 10, 2, 5, 3),     # four per thread
    (8200, 2, 6, 1, 3, 4),      # more than four per thread: every token through the list walk
    (64, 32, 3, 4, 30, 5),      # 32 positions: long lists, sort over several passes
])
def test_list_path_host_build(exe, tmp_path, H, K, T, calls, extra, seed):
    rng = np.random.default_rng(seed)
    stream, n_rows = _stream(rng, T, K, extra)
    rows = rng.integers(-64, 64, size=(n_rows, H)).astype(np.float32)
    w = (2.0 ** -rng.integers(0, 6, size=n_rows)).astype(np.float32)
    cuts = sorted(rng.choice(np.arange(1, len(stream)), min(calls - 1, len(stream) - 1), replace=False))
    parts = np.split(np.arange(len(stream)), cuts)
    T_cap = T
    d = str(tmp_path)
    open(os.path.join(d, "meta.txt"), "w").write(f"{T_cap} {H} {K} {len(parts)}\n")
    ocs = O.CombineState(T_cap, K)
    expect_rel, out_ref, err_ref = [], {}, 0
    for c, part in enumerate(parts):
        sel = [stream[i] for i in part]
        ri = np.array([x[0] for x in sel], np.int32)
        tok = np.array([x[1] for x in sel], np.int32)
        ks = np.array([x[2] for x in sel], np.int32)
        gen = np.array([x[3] for x in sel], np.uint32)
        p = os.path.join(d, f"c{c}_")
        open(p + "meta.txt", "w").write(f"{len(sel)} {n_rows}\n")
        rows.tofile(p + "rows")
        ri.tofile(p + "row_idx")
        tok.tofile(p + "tok")
        ks.tofile(p + "kslot")
        w[ri].tofile(p + "w")
        gen.tofile(p + "gen")
        out, rel, oerr = O.combine_release(ocs, rows.astype(np.float64), ri, tok, ks, w[ri], gen)
        expect_rel.append(np.asarray(rel, np.int32))
        out_ref.update({t: out[t] for t in rel})
        err_ref |= oerr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
    r = subprocess.run([exe, d], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stderr[-3000:]
    for c, rel in enumerate(expect_rel):
        got = np.fromfile(os.path.join(d, f"c{c}_rel.bin"), np.int32)
        assert np.array_equal(got, rel), f"release list of call {c}"
    out = np.fromfile(os.path.join(d, "out.bin"), np.float32).reshape(T_cap, H)
    for t, v in out_ref.items():
        assert np.array_equal(out[t], v.astype(np.float32)), f"released row of token {t}"
    assert np.array_equal(np.fromfile(os.path.join(d, "mask.bin"), np.uint32), ocs.mask[:T_cap])
    assert np.array_equal(np.fromfile(os.path.join(d, "tgen.bin"), np.uint32), ocs.tgen[:T_cap])
    assert int(np.fromfile(os.path.join(d, "err.bin"), np.uint32)[0]) == err_ref
