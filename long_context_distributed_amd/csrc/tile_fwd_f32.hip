// Tile forward, float32 inputs (head_dim 64 or 128), for gfx950 (MI355X).
//
// Same tile semantics as the bf16 kernel (Mesh-Attention tutorial page, "From
// 1-D ring to 2-D mesh"; online softmax as in the ring-attention page's
// log-sum-exp section) with float32 matrix-core math,
// v_mfma_f32_16x16x4_f32.
//
// Work decomposition, sized for small tiles as much as for large ones:
//   workgroup = 16 query rows of one query head; its KS waves split the keys:
//   wave w takes every KS-th 16-key tile of the Q slot's tile sequence (over
//   its FULL blocks, and its DIAG block up to the workgroup's last row).  Each
//   wave streams its own K/V tiles memory -> LDS by buffer-load DMA into two
//   buffers of its own (no barrier in the loop: a wave waits only for its own
//   loads), keeps its own (m, l, O), and the KS partials of every row are
//   merged through LDS at the end with log-sum-exp weights.
//
// Matrix-core formulation (16x16 outputs, K = 4 per MFMA; lane l holds
// A[l%16][l/16], B[l/16][l%16] and outputs rows 4*(l/16) + r, column l%16).
//   S^T = K Q^T per 16-key tile: k-index j = l/16 of MFMA (G, e) is dim
//     16G + 4j + e, so a lane reads 4 consecutive dims of its key (A) and of
//     its query row (B) with one 16-byte read and feeds them to 4 MFMAs.
//     The accumulator gives lane l the scores of keys 4*(l/16) + r of row
//     l%16: a row's 16 keys sit in the 4 lanes l%16 + 16j.
//   O^T += V^T P^T: k-step s contracts keys 4j + s, the key lane group j holds
//     in accumulator register s, so B is that register; output tile (h, e)
//     row i is dim 64h + 4i + e, so A (V[key][64h + 4i .. +3]) is again one
//     16-byte read per 4 MFMAs.
// LDS: K tiles row-major with 16-byte chunk c of key row n at c ^ (n & 15)
// (the 16 rows a 16-lane group reads land in distinct banks); V tiles
// row-major (a 16-lane group reads one whole row).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "tile_common.hpp"

// The DMA loads set M0 in inline assembly (see dma_tile); nothing else in
// this file uses M0.
#pragma clang diagnostic ignored "-Winline-asm"

namespace mesh_attn {
namespace {

using dev::kNegInf;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int RB = kWaveRowsF32;      // query rows per workgroup
constexpr int KS = kTileKeySplitF32;  // waves per workgroup, splitting the keys
constexpr int NT = KS * 64;
constexpr int BN = 16;                // keys per tile
constexpr int kRsrcWord3 = 0x00020000;  // buffer resource flags for gfx9 (raw, 32-bit)

static_assert(RB == 16 && kTileWavesF32 == 1, "one 16-row block per workgroup");

template <int D>
struct Shape {
    static constexpr int kRowBytes = D * 4;
    static constexpr int kTileBytes = BN * kRowBytes;  // one K or V tile
    static constexpr int kBufBytes = 2 * kTileBytes;   // K then V
    static constexpr int kWaveBytes = 2 * kBufBytes;   // two buffers per wave
    static constexpr int kLdsBytes = KS * kWaveBytes;
    static constexpr int kDma = kTileBytes / 1024;     // 1 KiB DMA loads per K (or V) tile
    static constexpr int kG = D / 16;                  // 16-dim groups
    // Merge area (reuses the tile buffers): O partials [KS][RB][D], then m and l [KS][RB].
    static_assert(KS * RB * D * 4 + 2 * KS * RB * 4 <= kLdsBytes, "merge area fits");
};

// Raw buffer descriptor of at most BN rows of `row_bytes` from `base`, of
// which `rows` exist (loads past them read zero); the last row is `last`
// bytes long.
__device__ __forceinline__ u32x4 tile_desc(const void* base, int rows, int row_bytes, int last) {
    const int r = rows < BN ? rows : BN;
    const int n = r > 0 ? (r - 1) * row_bytes + last : 0;
    const unsigned long long a = reinterpret_cast<unsigned long long>(base);
    return u32x4{static_cast<unsigned>(a), static_cast<unsigned>(a >> 32) & 0xffffu, static_cast<unsigned>(n),
                 static_cast<unsigned>(kRsrcWord3)};
}

// Value of x in lane (l ^ 16) and (l ^ 32) combined with the row's other lanes.
__device__ __forceinline__ float row_max4(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float row_sum4(float x) {
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
}

template <int D>
__global__ __launch_bounds__(NT, 2) void tile_fwd_f32_kernel(const TileParams p) {
    using S = Shape<D>;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[S::kLdsBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane >> 4, i16 = lane & 15;
    const int L = p.part_len;
    const dev::WorkItem w = dev::decode_work(p, 0);  // every wave shares the workgroup's rows
    const int u = w.wg_tok0 + i16;                  // this lane's query row (partition offset)
    const float c2 = p.scale_log2e;
    const int row_bytes = p.heads_kv * D * 4;
    const size_t slot_floats = (size_t)L * p.heads_kv * D;
    const float* kbase = reinterpret_cast<const float*>(p.k) + (size_t)w.kv_head * D;
    const float* vbase = reinterpret_cast<const float*>(p.v) + (size_t)w.kv_head * D;

    // Q fragments: row u, dims 16G + 4j .. +3 (zero past L).
    f32x4 qv[S::kG];
    {
        const float* qrow = reinterpret_cast<const float*>(p.q) +
                            ((size_t)(w.q_slot * L + min(u, L - 1)) * p.heads_q + w.head) * D + 4 * j;
#pragma unroll
        for (int G = 0; G < S::kG; ++G) {
            qv[G] = *reinterpret_cast<const f32x4*>(qrow + 16 * G);
            if (u >= L) qv[G] = f32x4{0.f, 0.f, 0.f, 0.f};
            // Await Q here, not at its first use inside the loop, where the
            // wait would also count the untracked tile DMA.
            asm volatile("" : "+v"(qv[G]));
        }
    }

    // Per-lane offsets: DMA sources within a tile, and the K / V reads.
    int gk[S::kDma], gv[S::kDma];
#pragma unroll
    for (int i = 0; i < S::kDma; ++i) {
        const int off = 1024 * i + 16 * lane;  // LDS byte within the tile
        const int row = off / S::kRowBytes, phys = (off % S::kRowBytes) >> 4;
        gk[i] = row * row_bytes + ((phys ^ (row & 15)) << 4);
        gv[i] = row * row_bytes + (phys << 4);
    }
    int kofs[S::kG];  // K read of key row i16, logical chunk 4G + j
#pragma unroll
    for (int G = 0; G < S::kG; ++G) kofs[G] = i16 * S::kRowBytes + (((4 * G + j) ^ i16) << 4);
    const int vofs = 4 * j * S::kRowBytes + (i16 << 4);  // V row 4j (+ s), chunk i16 (+ 16h)

    f32x4 o[4 * (D / 64)];
#pragma unroll
    for (int t = 0; t < 4 * (D / 64); ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = kNegInf, l = 0.0f;

    const unsigned lds_wave =
        static_cast<unsigned>(reinterpret_cast<uintptr_t>((LDS_AS unsigned char*)smem)) + wave * S::kWaveBytes;
    const LDS_AS unsigned char* wbuf = (const LDS_AS unsigned char*)smem + wave * S::kWaveBytes;

    const int b_beg = p.sched.blk_off[w.q_slot];
    const int b_end = p.sched.blk_off[w.q_slot + 1];
    auto tile_end = [&](int bi) { return (sched_entry(p.sched, bi) & 3) == kDiag ? w.wg_tok_end : L; };
    auto advance = [&](int& bi, int& n0, int steps) {
        for (int k = 0; k < steps && bi < b_end; ++k) {
            n0 += BN;
            if (n0 >= tile_end(bi)) {
                ++bi;
                n0 = 0;
            }
        }
    };
    // DMA of the K and V tile (block bi, keys n0 ..) into buffer b of this wave.
    auto dma_tile = [&](int bi, int n0, int b) {
        const size_t off = (size_t)(sched_entry(p.sched, bi) >> 2) * slot_floats + (size_t)n0 * p.heads_kv * D;
        const u32x4 kd = tile_desc(kbase + off, L - n0, row_bytes, D * 4);
        const u32x4 vd = tile_desc(vbase + off, L - n0, row_bytes, D * 4);
        const unsigned dst = lds_wave + b * S::kBufBytes;
#pragma unroll
        for (int i = 0; i < S::kDma; ++i) {
            const unsigned dk = __builtin_amdgcn_readfirstlane(dst + 1024 * i);
            const unsigned dv = __builtin_amdgcn_readfirstlane(dst + S::kTileBytes + 1024 * i);
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                         :: "s"(dk), "v"(gk[i]), "s"(kd) : "memory", "m0");
            asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                         :: "s"(dv), "v"(gv[i]), "s"(vd) : "memory", "m0");
        }
    };

    int cbi = b_beg, cn0 = 0;
    advance(cbi, cn0, wave);  // this wave's first tile
    int nbi = cbi, nn0 = cn0;
    advance(nbi, nn0, KS);    // and its next
    int buf = 0;
    if (cbi < b_end) dma_tile(cbi, cn0, 0);
    while (cbi < b_end) {
        const bool more = nbi < b_end;
        if (more) {
            dma_tile(nbi, nn0, buf ^ 1);
            asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * S::kDma) : "memory");  // this tile has landed
        } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        const LDS_AS unsigned char* kt = wbuf + buf * S::kBufBytes;
        const LDS_AS unsigned char* vt = kt + S::kTileBytes;

        // S^T for the 16 keys of this tile.
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int G = 0; G < S::kG; ++G) {
            const f32x4 ka = *reinterpret_cast<const LDS_AS f32x4*>(kt + kofs[G]);
#pragma unroll
            for (int e = 0; e < 4; ++e) s = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[e], qv[G][e], s, 0, 0, 0);
        }
        const bool diag = (sched_entry(p.sched, cbi) & 3) == kDiag;
        if ((diag && cn0 + BN - 1 > w.wg_tok0) || cn0 + BN > L) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = cn0 + 4 * j + r;
                if (key >= L || (diag && key > u)) s[r] = kNegInf;
            }
        }
        // Online softmax (exact running maximum per tile, base 2).
        const float mx = row_max4(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
        const float m_new = fmaxf(m, mx * c2);
        const float m_use = m_new == kNegInf ? 0.0f : m_new;
        const float alpha = dev::fast_exp2(m - m_use);
        m = m_new;
        l *= alpha;
#pragma unroll
        for (int t = 0; t < 4 * (D / 64); ++t) o[t] *= alpha;
        f32x4 pr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            pr[r] = dev::fast_exp2(__builtin_fmaf(s[r], c2, -m_use));
            l += pr[r];
        }
        // O^T += V^T P^T.
#pragma unroll
        for (int sk = 0; sk < 4; ++sk)
#pragma unroll
            for (int h = 0; h < D / 64; ++h) {
                const f32x4 va = *reinterpret_cast<const LDS_AS f32x4*>(vt + vofs + sk * S::kRowBytes + h * 256);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    o[4 * h + e] = __builtin_amdgcn_mfma_f32_16x16x4f32(va[e], pr[sk], o[4 * h + e], 0, 0, 0);
            }
        cbi = nbi;
        cn0 = nn0;
        advance(nbi, nn0, KS);
        buf ^= 1;
    }

    // Merge the KS partials of each row: O_w, m_w, l_w through LDS.
    const float l_row = row_sum4(l);
    __syncthreads();  // every wave is done with its tile buffers
    float* mo = reinterpret_cast<float*>(smem);       // [KS][RB][D]
    float* mm = mo + KS * RB * D;                      // [KS][RB]
    float* ml = mm + KS * RB;                          // [KS][RB]
#pragma unroll
    for (int h = 0; h < D / 64; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const f32x4 v4 = {o[4 * h][r], o[4 * h + 1][r], o[4 * h + 2][r], o[4 * h + 3][r]};
            *reinterpret_cast<f32x4*>(mo + (wave * RB + i16) * D + 64 * h + 16 * j + 4 * r) = v4;
        }
    if (j == 0) {
        mm[wave * RB + i16] = m;
        ml[wave * RB + i16] = l_row;
    }
    __syncthreads();
    constexpr int kQuads = RB * D / 4;
#pragma unroll
    for (int qd = tid; qd < kQuads; qd += NT) {
        const int row = qd / (D / 4), d4 = qd % (D / 4);
        float mt = kNegInf;
#pragma unroll
        for (int k = 0; k < KS; ++k) mt = fmaxf(mt, mm[k * RB + row]);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        float wsum = 0.0f;
        if (mt > kNegInf) {
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                const float wk = dev::fast_exp2(mm[k * RB + row] - mt);
                wsum += wk * ml[k * RB + row];
                acc += wk * *reinterpret_cast<const f32x4*>(mo + (k * RB + row) * D + 4 * d4);
            }
        }
        const int ur = w.wg_tok0 + row;
        if (ur < L) {
            const size_t q_row = (size_t)(w.q_slot * L + ur) * p.heads_q + w.head;
            const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.o) + q_row * D + 4 * d4) = acc * inv;
            if (d4 == 0) p.lse[q_row] = wsum > 0.0f ? (mt + __log2f(wsum)) * dev::kLn2 : kNegInf;
        }
    }
}

}  // namespace

hipError_t launch_tile_fwd_f32(const TileParams& p, int head_dim, hipStream_t stream) {
    if (p.wave_rows != RB) return hipErrorInvalidValue;
    const unsigned n_wg = static_cast<unsigned>(tile_fwd_grid(p));
    if (head_dim == 64)
        hipLaunchKernelGGL(tile_fwd_f32_kernel<64>, dim3(n_wg), dim3(NT), 0, stream, p);
    else if (head_dim == 128)
        hipLaunchKernelGGL(tile_fwd_f32_kernel<128>, dim3(n_wg), dim3(NT), 0, stream, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace mesh_attn
