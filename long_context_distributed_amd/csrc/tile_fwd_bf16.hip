// Tile forward, bf16 inputs, head_dim 128, for gfx950 (MI355X).
//
// One GPU's 2-D tile of the Q-KV matrix (Mesh-Attention tutorial page, "From
// 1-D ring to 2-D mesh"): for each Q slot, attention over the KV slots listed
// for it, FULL blocks entirely, DIAG blocks up to the diagonal, SKIP blocks
// not at all; the result is a partial output and log-sum-exp per query row.
//
// Work decomposition
//   workgroup = NW waves sharing one KV head (two per SIMD); each wave owns 32
//               query rows of one query head.  With GQA (G > 1) the waves of a
//               workgroup are the query heads of one KV group, so one K/V
//               stream from memory serves all of them.
//   K/V are streamed through LDS in tiles of 64 keys by the DMA path of
//   buffer loads (memory -> LDS without registers), into one of two buffers
//   while the waves compute on the other: one barrier per tile.  Rows past
//   the end of a partition read as zero through the buffer's range check.
//
// Matrix-core formulation (v_mfma_f32_32x32x16_bf16, 64-lane waves)
//   S^T = K Q^T: A = K tile (32 keys x 16 dims), B = Q^T (16 dims x 32 rows).
//     In the 32x32 accumulator, lane l holds query row l%32 and 16 keys,
//     key = 8*(i/4) + 4*(l/32) + i%4 for register i.  A query row thus lives
//     in one lane pair (l, l^32): the row max needs one cross-half exchange
//     (v_permlane32_swap) per 32 keys, the row sum one at the very end.
//   O^T += V^T P^T: A = V^T (32 dims x 16 keys), B = P^T straight from the
//     softmax registers (no shuffles).  The dot-product index of an MFMA only
//     has to be paired consistently between A and B, so B's keys follow the
//     accumulator order above and V^T is read in the same key order with the
//     LDS transpose read ds_read_b64_tr_b16: within 16 lanes, result lane j,
//     element p comes from source lane 4p + j/4, element j%4, so four lanes
//     reading 4-dim pieces of four key rows give every lane four keys of its
//     own dim.
//
// Online softmax with a lazy shift: a row keeps the shift m it used so far
// and only moves it (rescaling O and l) when a new score exceeds it by more
// than 2^8 in base 2; otherwise probabilities up to 2^8 are accumulated as
// they are.  The result is the same softmax, since O and l share the shift.
//
// LDS layouts (row-major, 16-byte chunks swizzled so that reads are free of
// bank conflicts; the DMA writes are contiguous per wave)
//   K: [64 keys][128 dims]; chunk c of key row n at chunk c ^ (n & 15).
//   V: [64 keys][128 dims]; chunk c of key row n at chunk c ^ (4 * (n & 3)).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "kernels.h"
#include "tile_common.hpp"

namespace mesh_attn {
namespace {

using dev::kNegInf;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_raw __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int D = 128;      // head dim
constexpr int BN = 64;      // keys per LDS tile
constexpr int NW = kTileWavesBf16;
constexpr int NT = NW * 64;
constexpr int kTileBytes = BN * D * 2;      // 16 KiB per K or V tile
constexpr int kBufBytes = 2 * kTileBytes;   // K then V
constexpr float kShiftSlack = 8.0f;         // base-2 headroom before the shift moves
constexpr int kRsrcWord3 = 0x00020000;      // buffer resource flags for gfx9 (raw, 32-bit)
constexpr int kDmaPerWave = 2 * kTileBytes / (NT * 16);  // 16-byte DMA loads per lane per tile

static_assert(kWaveRowsBf16 == 32, "one 32-row block per wave");
static_assert(2 * kTileBytes % (NT * 16) == 0, "DMA split");

typedef __amdgpu_buffer_rsrc_t Rsrc;
#define LDS_AS __attribute__((address_space(3)))

// Buffer resource over `rows` rows of `row_bytes` starting at base: loads
// from rows at or past `rows` return zero, with no branch.
__device__ __forceinline__ Rsrc rows_rsrc(const void* base, int rows, int row_bytes) {
    const int n = rows > 0 ? (rows - 1) * row_bytes + D * 2 : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kRsrcWord3);
}

// Per-thread constants of the DMA loader and of the LDS reads.
struct Lanes {
    // DMA: load i of this wave fills the 1 KiB region reg = wave + NW*i of a
    // buffer (regions 0..15 are K, 16..31 V); lane l of a region fills chunk
    // 64*reg + l, i.e. key row 4*(reg%16) + l/16, physical chunk l%16.
    int dma_gofs[kDmaPerWave];   // byte offset in the K or V tile (row, logical chunk)
    // readers
    int k_rofs[8];  // K fragment (key r32, chunk 2c+g), c = 0..7
    int v_rofs[4];  // V^T fragment, dims 32t + r32, keys 4g .. 4g+3 (+16ks, +8 for the upper half)
};

__device__ __forceinline__ void init_lanes(Lanes& ln, int tid, int wave, int row_bytes) {
    const int lane = tid & 63, g = lane >> 5, r32 = lane & 31;
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
        const int reg = wave + NW * i;          // 0..31
        const int row = 4 * (reg & 15) + (lane >> 4);
        const int phys = lane & 15;
        const int logical = reg < 16 ? (phys ^ (row & 15)) : (phys ^ (4 * (row & 3)));
        ln.dma_gofs[i] = row * row_bytes + logical * 16;
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) ln.k_rofs[c] = r32 * (D * 2) + (((2 * c + g) ^ (r32 & 15)) << 4);
    const int s16 = lane & 15, half = (lane >> 4) & 1;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int row = 4 * g + (s16 >> 2);
        const int chunk = 4 * (t ^ (s16 >> 2)) + 2 * half + ((s16 & 3) >> 1);
        ln.v_rofs[t] = row * (D * 2) + chunk * 16 + (s16 & 1) * 8;
    }
}

// Issues the DMA loads of keys n0..n0+63 (rows past the range read as zero)
// into LDS buffer `buf`.
__device__ __forceinline__ void dma_tile(const Lanes& ln, Rsrc kr, Rsrc vr, LDS_AS unsigned char* buf,
                                         int wave) {
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
        const int reg = wave + NW * i;
        const Rsrc r = reg < 16 ? kr : vr;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS_AS void*)(buf + reg * 1024), 16,
                                                 ln.dma_gofs[i], 0, 0, 0);
    }
}

struct State {
    bf16x8 qf[8];      // Q^T fragments, d-chunk c
    f32x16 o[4];       // O^T accumulators, dims 32t..32t+31
    float m;           // shift in use (scaled base-2 scores)
    float l;           // exponent sum over this lane's keys
};

__device__ __forceinline__ bf16x4 read_tr(const LDS_AS unsigned char* p) {
    const bf16x4_raw r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_raw*)p);
    return __builtin_bit_cast(bf16x4, r);
}

// Attention of the wave's 32 rows over the 64 keys n0.. held in LDS buffer `buf`.
template <bool MASK>
__device__ __forceinline__ void tile_math(State& st, const Lanes& ln, const LDS_AS unsigned char* buf,
                                          int n0, int L, bool diag, int wave_tok0, float c2) {
    const int lane = threadIdx.x & 63, g = lane >> 5, r32 = lane & 31;
    const LDS_AS unsigned char* sv = buf + kTileBytes;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        // S^T = K Q^T for keys n0+32h .. +31.
        f32x16 s;
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const bf16x8 ka = *reinterpret_cast<const LDS_AS bf16x8*>(buf + ln.k_rofs[c] + 8192 * h);
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, st.qf[c], s, 0, 0, 0);
        }

        if (MASK) {  // causal diagonal and ragged tail: hide keys after the query or past L
            const int u = wave_tok0 + r32;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int kk = n0 + 32 * h + 8 * (i >> 2) + 4 * g + (i & 3);
                if (kk >= L || (diag && kk > u)) s[i] = kNegInf;
            }
        }

        // Row maximum; move the shift only where a score outgrew it.
        float mx = kNegInf;
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
        const float m_cand = dev::max_with_partner(mx) * c2;
        const bool need = m_cand > st.m + kShiftSlack;
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
            const float m_new = need ? m_cand : st.m;
            const float alpha = need ? dev::fast_exp2(st.m - m_new) : 1.0f;
            st.m = m_new;
            st.l *= alpha;
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) st.o[t][i] *= alpha;
        }

        // P = exp2(S*c - m) in bf16, laid out as the B operand of the PV MFMAs.
        bf16x8 pb[2];
        const float shift = st.m == kNegInf ? 0.0f : st.m;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float pv = dev::fast_exp2(__builtin_fmaf(s[i], c2, -shift));
            st.l += pv;
            pb[i >> 3][i & 7] = static_cast<__bf16>(pv);
        }

        // O^T += V^T P^T, 16 keys per MFMA.
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int ks = 2 * h + kk;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const bf16x4 va = read_tr(sv + ln.v_rofs[t] + ks * 4096);
                const bf16x4 vb = read_tr(sv + ln.v_rofs[t] + ks * 4096 + 2048);
                const bf16x8 a8 = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
                st.o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a8, pb[kk], st.o[t], 0, 0, 0);
            }
        }
    }
}

__global__ __launch_bounds__(NT, 1) void tile_fwd_bf16_d128(const TileParams p) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem0[kBufBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char smem1[kBufBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps the schedule in SGPRs
    const int g = lane >> 5, r32 = lane & 31;
    const int L = p.part_len;
    const dev::WorkItem w = dev::decode_work(p, wave);
    const float c2 = p.scale_log2e;
    const int row_bytes = p.heads_kv * D * 2;
    const __bf16* kbase = reinterpret_cast<const __bf16*>(p.k) + (size_t)w.kv_head * D;
    const __bf16* vbase = reinterpret_cast<const __bf16*>(p.v) + (size_t)w.kv_head * D;
    const size_t slot_elems = (size_t)L * p.heads_kv * D;

    Lanes ln;
    init_lanes(ln, tid, wave, row_bytes);

    State st;
    {
        // Q rows of this wave (rows at or past L read as zero).
        const int qrow_bytes = p.heads_q * D * 2;
        const __bf16* q0 = reinterpret_cast<const __bf16*>(p.q) +
                           ((size_t)(w.q_slot * L + w.wave_tok0) * p.heads_q + w.head) * D;
        const Rsrc qr = rows_rsrc(q0, L - w.wave_tok0, qrow_bytes);
#pragma unroll
        for (int c = 0; c < 8; ++c)
            st.qf[c] = __builtin_bit_cast(
                bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qr, r32 * qrow_bytes + (16 * c + 8 * g) * 2,
                                                              0, 0));
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) st.o[t][i] = 0.0f;
    st.m = kNegInf;
    st.l = 0.0f;
    const int wave_last_tok = min(L, w.wave_tok0 + 32) - 1;

    const int b_beg = p.sched.blk_off[w.q_slot];
    const int b_end = p.sched.blk_off[w.q_slot + 1];

    // The tiles of this Q slot form one sequence over (block, key tile); the
    // next tile streams into the other LDS buffer while this one is computed.
    int bi = b_beg, n0 = 0;
    auto issue = [&](int bi_, int n0_, LDS_AS unsigned char* buf) {
        const size_t off = (size_t)(sched_entry(p.sched, bi_) >> 2) * slot_elems + (size_t)n0_ * p.heads_kv * D;
        dma_tile(ln, rows_rsrc(kbase + off, L - n0_, row_bytes),
                 rows_rsrc(vbase + off, L - n0_, row_bytes), buf, wave);
    };
    auto advance = [&](int& bi_, int& n0_) {
        n0_ += BN;
        const int end = (sched_entry(p.sched, bi_) & 3) == kDiag ? w.wg_tok_end : L;
        if (n0_ >= end) {
            ++bi_;
            n0_ = 0;
        }
    };

    if (b_beg < b_end) {
        issue(bi, n0, (LDS_AS unsigned char*)smem0);
        __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): this thread's DMA has landed
        __syncthreads();
        // One step: start the next tile's DMA into the other buffer, compute
        // on buffer BUF, wait for the DMA, barrier.  False after the last tile.
        auto step = [&](auto buf_tag) -> bool {
            constexpr int BUF = decltype(buf_tag)::value;
            LDS_AS unsigned char* cur = (LDS_AS unsigned char*)(BUF == 0 ? smem0 : smem1);
            LDS_AS unsigned char* nxt = (LDS_AS unsigned char*)(BUF == 0 ? smem1 : smem0);
            int nbi = bi, nn0 = n0;
            advance(nbi, nn0);
            const bool has_next = nbi < b_end;
            if (has_next) issue(nbi, nn0, nxt);
            const bool diag = (sched_entry(p.sched, bi) & 3) == kDiag;
            if (!(diag && n0 > wave_last_tok)) {
                if ((diag && n0 + BN - 1 > w.wave_tok0) || n0 + BN > L)
                    tile_math<true>(st, ln, cur, n0, L, diag, w.wave_tok0, c2);
                else
                    tile_math<false>(st, ln, cur, n0, L, diag, w.wave_tok0, c2);
            }
            if (!has_next) return false;
            __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0)
            __syncthreads();
            bi = nbi;
            n0 = nn0;
            return true;
        };
        while (step(std::integral_constant<int, 0>{}) && step(std::integral_constant<int, 1>{})) {
        }
    }

    // Epilogue: O = O_acc / l, lse = ln(2) * (m + log2 l); empty rows -> (0, -inf).
    const int u = w.wave_tok0 + r32;
    const float l_tot = dev::add_with_partner(st.l);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    if (u < L) {
        const size_t q_row = (size_t)(w.q_slot * L + u) * p.heads_q + w.head;
        __bf16* op = reinterpret_cast<__bf16*>(p.o) + q_row * D;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                bf16x4 ov;
#pragma unroll
                for (int j = 0; j < 4; ++j) ov[j] = static_cast<__bf16>(st.o[t][4 * ib + j] * inv);
                *reinterpret_cast<bf16x4*>(op + 32 * t + 8 * ib + 4 * g) = ov;
            }
        if (g == 0) p.lse[q_row] = l_tot > 0.0f ? (st.m + __log2f(l_tot)) * dev::kLn2 : kNegInf;
    }
}

}  // namespace

hipError_t launch_tile_fwd_bf16(const TileParams& p, int head_dim, hipStream_t stream) {
    if (head_dim != D || p.wave_rows != kWaveRowsBf16) return hipErrorInvalidValue;
    const unsigned n_wg = static_cast<unsigned>(p.n_q_slots) * p.n_tok_blocks * p.heads_kv *
                          p.n_head_groups;
    hipLaunchKernelGGL(tile_fwd_bf16_d128, dim3(n_wg), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mesh_attn
