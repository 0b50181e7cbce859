"""The host C++ of the library (block list, argument validation, schedule
packing) built a second time with AddressSanitizer and UBSan by g++, and
driven through the same C ABI in a subprocess (CPU only).

The device kernels are replaced by stubs that return an error, so even
fully valid descriptors (with fake device addresses, never dereferenced)
exercise the whole host path, including schedule packing, under the
sanitizers.
"""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_distributed_amd", "csrc")

STUB = """
#include "kernels.h"
namespace mesh_attn {
hipError_t launch_tile_fwd_bf16(const TileParams&, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_tile_fwd_f32(const TileParams&, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_lse_merge(int, int64_t, int, int, const void*, const float*, void*, float*,
                            hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_tile_bwd_bf16(const BwdDqParams&, const BwdDkvParams&, int, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_bwd_delta(int64_t, int, int, const void*, const void*, float*, hipStream_t) {
    return hipErrorNoDevice;
}
}
"""

DRIVER = textwrap.dedent("""
    import ctypes, itertools, sys
    sys.path.insert(0, {root!r})
    import oracle
    from long_context_distributed_amd import _lib
    _lib.LIB_PATH = {lib!r}
    lib = _lib.load()
    n = ctypes.c_int32(0)
    for R, C in itertools.product(range(1, 7), repeat=2):
        arr = (_lib.Block * (R * C))()
        for r, c in itertools.product(range(R), range(C)):
            for causal, rot in itertools.product((0, 1), repeat=2):
                assert lib.mesh_attn_block_list(R, C, r, c, causal, rot, arr, R * C, ctypes.byref(n)) == 0
                got = [(b.q_slot, b.kv_slot, b.q_part, b.kv_part, b.kind) for b in arr]
                assert got == oracle.block_list_ref(R, C, r, c, causal, rot)
    FAKE = 0x100000
    def desc(blocks, dtype=0, L=64, nq=2, nkv=2, hq=4, hkv=2, d=128, scale=0.1):
        arr = (_lib.Block * max(1, len(blocks)))(*[_lib.Block(*b) for b in blocks])
        dd = _lib.TileDesc(dtype, L, nq, nkv, hq, hkv, d, scale, arr, len(blocks))
        dd._keep = arr
        return dd
    # valid descriptors reach the (stub) launch: full schedule packing under the sanitizers
    for (R, C, r, c) in [(2, 2, 0, 0), (4, 4, 2, 2), (8, 8, 4, 4), (16, 4, 8, 2), (8, 8, 0, 7)]:
        bl = oracle.block_list_ref(R, C, r, c, True, True)
        for dtype, d in ((0, 128), (1, 64), (1, 128)):
            st = lib.mesh_attn_tile_fwd(ctypes.byref(desc(bl, dtype=dtype, nq=C, nkv=R, d=d)),
                                        FAKE, FAKE, FAKE, FAKE, FAKE, None)
            assert st == _lib.ERR_HIP, st
        st = lib.mesh_attn_tile_bwd(ctypes.byref(desc(bl, nq=C, nkv=R)), *([FAKE] * 9), None)
        assert st == _lib.ERR_HIP, st
        assert lib.mesh_attn_tile_bwd(ctypes.byref(desc(bl, dtype=1, nq=C, nkv=R)), *([FAKE] * 9),
                                      None) == _lib.ERR_UNSUPPORTED
    # every invalid descriptor is rejected
    bl = oracle.block_list_ref(2, 2, 0, 0, True, True)
    for kw in (dict(dtype=7), dict(L=0), dict(nq=0), dict(nq=65), dict(hq=3), dict(scale=0.0),
               dict(d=96)):
        assert lib.mesh_attn_tile_fwd(ctypes.byref(desc(bl, **kw)), FAKE, FAKE, FAKE, FAKE, FAKE,
                                      None) < 0
    assert lib.mesh_attn_tile_fwd(ctypes.byref(desc(bl + [bl[0]])), FAKE, FAKE, FAKE, FAKE, FAKE,
                                  None) == _lib.ERR_INVALID
    big = [(s, j, s, 64 + j, 0) for s in range(32) for j in range(32)]   # 1024 blocks
    assert lib.mesh_attn_tile_fwd(ctypes.byref(desc(big, nq=32, nkv=32)), FAKE, FAKE, FAKE, FAKE,
                                  FAKE, None) == _lib.ERR_HIP
    assert lib.mesh_attn_lse_merge(8, 1 << 20, 128, 0, FAKE, FAKE, FAKE, FAKE, None) == _lib.ERR_HIP
    assert lib.mesh_attn_lse_merge(0, 16, 128, 0, FAKE, FAKE, FAKE, FAKE, None) == _lib.ERR_INVALID
    assert lib.mesh_attn_bwd_delta(1 << 20, 128, 0, FAKE, FAKE, FAKE, None) == _lib.ERR_HIP
    assert lib.mesh_attn_bwd_delta(16, 12, 0, FAKE, FAKE, FAKE, None) == _lib.ERR_INVALID
    # the greedy planner: equal to the oracle's plans, size queries, invalid costs
    import long_context_distributed_amd as mat
    costs = dict(recv_q_s=1.0, recv_kv_s=0.5, send_o_s=1.25, full_block_s=0.75, diag_block_s=0.375)
    for R, C in [(1, 1), (2, 2), (3, 5), (8, 8), (16, 4), (64, 1)]:
        for r, c in sorted(set([(0, 0), (R // 2, C // 2), (R - 1, C - 1)])):
            for causal, rot, delay in itertools.product((0, 1), repeat=3):
                got = mat.plan(R, C, r, c, causal, rot, costs, delay)
                want = oracle.greedy_plan_ref(R, C, r, c, causal, rot, costs, bool(delay))
                assert [(x["comm"], x["slot"], x["blocks"], x["end_s"]) for x in got] == \
                    [(x["comm"], x["slot"], x["blocks"], x["end_s"]) for x in want]
    pc = _lib.PlanCosts(1.0, 1.0, 1.0, -1.0, 1.0, 1)
    assert lib.mesh_attn_plan(2, 2, 0, 0, 1, 1, ctypes.byref(pc), None, 0, ctypes.byref(n), None, 0,
                              ctypes.byref(n)) == _lib.ERR_INVALID
    print("sanitized host path ok")
""")


def _runtime(name):
    out = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists("/opt/rocm/include/hip"),
                    reason="needs g++ and the HIP headers")
def test_host_code_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("sanitizer runtimes not installed")
    stub = tmp_path / "stub.cpp"
    stub.write_text(STUB)
    lib = tmp_path / "libmeshattn_sanitized.so"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fsanitize=address,undefined",
           "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "block_list.cpp"),
           os.path.join(CSRC, "plan.cpp"), str(stub), "-o", str(lib), "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    env = dict(os.environ, LD_PRELOAD=f"{asan} {ubsan}", ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-c", DRIVER.format(root=ROOT, lib=str(lib))],
                         capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "sanitized host path ok" in res.stdout
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr


THREADS_DRIVER = r"""
#include <atomic>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>

#include "mesh_attn.h"

static std::atomic<int> bad{0};

static void worker(int t) {
    mesh_attn_block blocks[MESH_ATTN_MAX_BLOCKS];
    int32_t n = 0;
    const int R = 4 + 2 * (t % 4), C = 4;
    void* fake = reinterpret_cast<void*>(0x100000);
    for (int it = 0; it < 2000; ++it) {
        // a valid block list, a valid tile (reaches the stub launch), an invalid tile
        if (mesh_attn_block_list(R, C, R / 2, C / 2, 1, 1, blocks, MESH_ATTN_MAX_BLOCKS, &n) !=
                MESH_ATTN_OK || n != R * C)
            ++bad;
        if (mesh_attn_last_error()[0] != 0) ++bad;
        mesh_attn_tile_desc d = {MESH_ATTN_BF16, 64, C, R, 4, 2, 128, 0.1f, blocks, n};
        if (mesh_attn_tile_fwd(&d, fake, fake, fake, fake, static_cast<float*>(fake), nullptr) !=
            MESH_ATTN_ERR_HIP)
            ++bad;
        if (mesh_attn_tile_bwd(&d, fake, fake, fake, fake, static_cast<float*>(fake),
                               static_cast<float*>(fake), static_cast<float*>(fake),
                               static_cast<float*>(fake), static_cast<float*>(fake), nullptr) !=
            MESH_ATTN_ERR_HIP)
            ++bad;
        d.part_len = 0;
        if (mesh_attn_tile_fwd(&d, fake, fake, fake, fake, static_cast<float*>(fake), nullptr) !=
            MESH_ATTN_ERR_INVALID)
            ++bad;
        if (std::strcmp(mesh_attn_last_error(), "tile_fwd: part_len must be >= 1") != 0) ++bad;
        mesh_attn_plan_costs pc = {1.0, 0.5, 1.0, 0.75, 0.375, 1};
        mesh_attn_plan_step steps[256];
        mesh_attn_block order[MESH_ATTN_MAX_BLOCKS];
        int32_t ns = 0, no = 0;
        if (mesh_attn_plan(R, C, R / 2, C / 2, 1, 1, &pc, steps, 256, &ns, order,
                           MESH_ATTN_MAX_BLOCKS, &no) != MESH_ATTN_OK ||
            ns < 1 || steps[ns - 1].end_s <= 0.0)
            ++bad;
    }
}

int main() {
    std::vector<std::thread> th;
    for (int t = 0; t < 8; ++t) th.emplace_back(worker, t);
    for (auto& x : th) x.join();
    std::printf("threads ok, bad=%d\n", bad.load());
    return bad.load() == 0 ? 0 : 1;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists("/opt/rocm/include/hip"),
                    reason="needs g++ and the HIP headers")
def test_host_code_under_tsan(tmp_path):
    """Eight native threads call the C ABI at once (valid and invalid tiles,
    block lists) with the host code built under ThreadSanitizer; each thread
    must see its own results and last-error text, and TSan must find no race."""
    if not _runtime("libtsan.so"):
        pytest.skip("ThreadSanitizer runtime not installed")
    (tmp_path / "stub.cpp").write_text(STUB)
    (tmp_path / "driver.cpp").write_text(THREADS_DRIVER)
    exe = tmp_path / "threads"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=thread", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "block_list.cpp"),
           os.path.join(CSRC, "plan.cpp"), str(tmp_path / "stub.cpp"), str(tmp_path / "driver.cpp"),
           "-o", str(exe),
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-pthread"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1:exitcode=66")
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "threads ok, bad=0" in res.stdout
    assert "ThreadSanitizer" not in res.stderr


def test_bench_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""
