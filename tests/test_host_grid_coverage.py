"""The kernels' work decomposition, checked exhaustively on the host.

A C++ driver links the library's host code (block list, validation, schedule
packing, work decomposition) and calls the same decoders the kernels call
(`decode_work_at`, `decode_key_block_at`, with `__host__ __device__`
qualifiers) for every workgroup and wave of the launch grids, over several
thousand tile shapes (mesh, tile, causal / rotated, partition length, head
counts and group sizes).  It checks that

  * every query row (Q slot, token, query head) of the tile is owned by
    exactly one lane of the forward grid (bf16 and f32 decompositions) and of
    the query-gradient grid, with the KV head of its group, and within its
    workgroup's token range (the bound of a DIAG block's keys);
  * every key (KV slot, token, KV head) is owned by exactly one lane of the
    key/value-gradient grid;
  * the packed schedules list exactly the non-SKIP blocks of each Q slot (in
    KV-slot order) and of each KV slot (in Q-slot order), and the Q-slot order
    is a permutation sorted by weight.

No GPU is needed: the launchers are stubs and nothing is launched.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_distributed_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

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

DRIVER = r"""
#include <cstdio>
#include <vector>

#include "kernels.h"
#include "tile_common.hpp"

using namespace mesh_attn;

static long fails = 0, plans = 0, rows_checked = 0;
#define CHECK(cond, ...)                                    \
    do {                                                    \
        if (!(cond)) {                                      \
            if (fails++ < 20) {                             \
                std::printf("FAIL %s:%d: ", what, __LINE__); \
                std::printf(__VA_ARGS__);                   \
                std::printf("\n");                          \
            }                                               \
        }                                                   \
    } while (0)

template <typename P>
static void cover_rows(const char* what, const P& p, int waves, const mesh_attn_tile_desc& d) {
    const int L = d.part_len, H = d.heads_q, G = d.heads_q / d.heads_kv;
    std::vector<int> cnt(static_cast<size_t>(d.n_q_slots) * L * H, 0);
    const int64_t n = tile_fwd_grid(p);
    for (int64_t lam = 0; lam < n; ++lam)
        for (int wv = 0; wv < waves; ++wv) {
            const dev::WorkItem w = dev::decode_work_at(p, static_cast<int>(lam), wv);
            CHECK(w.q_slot >= 0 && w.q_slot < d.n_q_slots, "q_slot %d", w.q_slot);
            CHECK(w.kv_head >= 0 && w.kv_head < d.heads_kv, "kv_head %d", w.kv_head);
            CHECK(w.head >= 0 && w.head < H && w.head / G == w.kv_head, "head %d kv_head %d",
                  w.head, w.kv_head);
            CHECK(w.wave_tok0 >= w.wg_tok0 && w.wg_tok_end <= L, "token range");
            if (w.q_slot < 0 || w.q_slot >= d.n_q_slots || w.head < 0 || w.head >= H) continue;
            for (int r = 0; r < p.wave_rows; ++r) {
                const int u = w.wave_tok0 + r;
                if (u >= L) continue;
                CHECK(u < w.wg_tok_end, "row %d past the workgroup's range %d", u, w.wg_tok_end);
                ++cnt[(static_cast<size_t>(w.q_slot) * L + u) * H + w.head];
            }
        }
    for (size_t i = 0; i < cnt.size(); ++i) CHECK(cnt[i] == 1, "row %zu owned %d times", i, cnt[i]);
    rows_checked += static_cast<long>(cnt.size());
}

static void cover_keys(const char* what, const BwdDkvParams& p, const mesh_attn_tile_desc& d) {
    const int L = d.part_len, H = d.heads_kv;
    std::vector<int> cnt(static_cast<size_t>(d.n_kv_slots) * L * H, 0);
    const int keys_per_wg = kBwdDkvWaves * kBwdRowsPerWave;
    const int64_t n = tile_bwd_dkdv_grid(p);
    for (int64_t lam = 0; lam < n; ++lam) {
        const dev::KeyBlock b = dev::decode_key_block_at(p, static_cast<int>(lam));
        CHECK(b.kv_slot >= 0 && b.kv_slot < d.n_kv_slots && b.kv_head >= 0 && b.kv_head < H &&
              b.key_block >= 0 && b.key_block * keys_per_wg < L, "key block decode");
        if (b.kv_slot < 0 || b.kv_slot >= d.n_kv_slots || b.kv_head < 0 || b.kv_head >= H) continue;
        for (int wv = 0; wv < kBwdDkvWaves; ++wv)
            for (int r = 0; r < kBwdRowsPerWave; ++r) {
                const int key = b.key_block * keys_per_wg + kBwdRowsPerWave * wv + r;
                if (key < L) ++cnt[(static_cast<size_t>(b.kv_slot) * L + key) * H + b.kv_head];
            }
    }
    for (size_t i = 0; i < cnt.size(); ++i) CHECK(cnt[i] == 1, "key %zu owned %d times", i, cnt[i]);
    rows_checked += static_cast<long>(cnt.size());
}

// The packed schedules against the block list itself.
static void check_schedules(const char* what, const TileSchedule& qs, const KvSchedule* ks,
                            const mesh_attn_tile_desc& d) {
    std::vector<int> kind(64 * 64, -1);
    for (int i = 0; i < d.n_blocks; ++i) kind[d.blocks[i].q_slot * 64 + d.blocks[i].kv_slot] = d.blocks[i].kind;
    std::vector<int> weight(d.n_q_slots, 0), seen(d.n_q_slots, 0);
    for (int s = 0; s < d.n_q_slots; ++s) {
        int e = qs.blk_off[s];
        for (int j = 0; j < d.n_kv_slots; ++j) {
            const int k = kind[s * 64 + j];
            if (k != MESH_ATTN_FULL && k != MESH_ATTN_DIAG) continue;
            CHECK(e < qs.blk_off[s + 1] && sched_entry(qs, e) == ((j << 2) | k), "Q-slot entry");
            ++e;
            weight[s] += k == MESH_ATTN_FULL ? 2 : 1;
        }
        CHECK(e == qs.blk_off[s + 1], "Q slot %d has extra entries", s);
    }
    for (int r = 0; r < d.n_q_slots; ++r) {
        const int s = qs.q_order[r];
        CHECK(s < d.n_q_slots && !seen[s], "q_order not a permutation");
        if (s < d.n_q_slots) seen[s] = 1;
        if (r > 0) CHECK(weight[qs.q_order[r - 1]] >= weight[s], "q_order not heaviest first");
    }
    if (ks == nullptr) return;
    for (int j = 0; j < d.n_kv_slots; ++j) {
        int e = ks->blk_off[j];
        for (int s = 0; s < d.n_q_slots; ++s) {
            const int k = kind[s * 64 + j];
            if (k != MESH_ATTN_FULL && k != MESH_ATTN_DIAG) continue;
            const uint32_t word = reinterpret_cast<const uint32_t*>(ks->blk)[e >> 2];
            CHECK(e < ks->blk_off[j + 1] && static_cast<int>((word >> (8 * (e & 3))) & 0xff) == ((s << 2) | k),
                  "KV-slot entry");
            ++e;
        }
        CHECK(e == ks->blk_off[j + 1], "KV slot %d has extra entries", j);
    }
}

int main() {
    const char* what = "plan";
    const int meshes[][4] = {{1, 1, 0, 0}, {2, 2, 1, 0}, {4, 4, 2, 2}, {3, 5, 1, 4},
                             {8, 8, 4, 4}, {16, 4, 8, 2}, {1, 8, 0, 3}, {8, 1, 5, 0}};
    const int lens[] = {1, 2, 31, 32, 33, 95, 96, 97, 255, 256, 257, 383, 384, 385, 1000};
    const int heads[][2] = {{1, 1}, {2, 2}, {3, 1}, {8, 2}, {5, 1}, {12, 2}, {7, 1},
                            {16, 2}, {12, 1}, {16, 1}, {48, 2}, {64, 1}};
    std::vector<mesh_attn_block> blocks(1024);
    for (const auto& m : meshes)
        for (int flags = 0; flags < 4; ++flags) {
            int32_t nb = 0;
            if (mesh_attn_block_list(m[0], m[1], m[2], m[3], flags & 1, (flags >> 1) & 1, blocks.data(),
                                     1024, &nb) != MESH_ATTN_OK) {
                std::printf("FAIL block list\n");
                return 1;
            }
            for (int L : lens)
                for (const auto& h : heads) {
                    // keep the enumeration to a few seconds: long partitions with small meshes
                    if (static_cast<long>(L) * h[0] * m[0] * m[1] > 400000) continue;
                    mesh_attn_tile_desc d = {MESH_ATTN_BF16, L, m[1], m[0], h[0], h[0] / h[1], 128,
                                             0.1f, blocks.data(), nb};
                    // one tile's Q slots are its mesh row (C), KV slots its mesh column (R)
                    TileParams p;
                    if (plan_tile_fwd("plan", d, p) != MESH_ATTN_OK) {
                        std::printf("FAIL plan_tile_fwd: %s\n", mesh_attn_last_error());
                        return 1;
                    }
                    what = "forward bf16";
                    cover_rows(what, p, kTileWavesBf16, d);
                    check_schedules(what, p.sched, nullptr, d);
                    BwdDqParams pq;
                    BwdDkvParams pk;
                    if (plan_tile_bwd("plan", d, pq, pk) != MESH_ATTN_OK) {
                        std::printf("FAIL plan_tile_bwd: %s\n", mesh_attn_last_error());
                        return 1;
                    }
                    what = "query gradient";
                    cover_rows(what, pq, kBwdDqWaves, d);
                    what = "key/value gradient";
                    cover_keys(what, pk, d);
                    check_schedules(what, pq.sched, &pk.sched, d);
                    d.dtype = MESH_ATTN_F32;
                    d.head_dim = 64;
                    if (plan_tile_fwd("plan", d, p) != MESH_ATTN_OK) {
                        std::printf("FAIL plan_tile_fwd f32: %s\n", mesh_attn_last_error());
                        return 1;
                    }
                    what = "forward f32";
                    cover_rows(what, p, kTileWavesF32, d);
                    plans += 4;
                    what = "plan";
                }
        }
    std::printf("plans %ld, rows and keys checked %ld, failures %ld\n", plans, rows_checked, fails);
    return fails == 0 ? 0 : 1;
}
"""


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_grid_covers_every_row_and_key_once(tmp_path):
    (tmp_path / "stub.cpp").write_text(STUB)
    (tmp_path / "driver.cpp").write_text(DRIVER)
    exe = tmp_path / "coverage"
    cmd = [HIPCC, "-std=c++17", "-O2", "-x", "hip", "--offload-arch=gfx950", "--cuda-host-only",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           str(tmp_path / "driver.cpp"), os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "block_list.cpp"),
           str(tmp_path / "stub.cpp"), "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    print(res.stdout[-2000:])
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-2000:]
    assert "failures 0" in res.stdout
