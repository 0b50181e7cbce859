// Tile forward, bf16 inputs, head_dim 128, for gfx950 (MI355X).
//
// One GPU's 2-D tile of the Q-KV matrix (Mesh-Attention tutorial page, "From
// 1-D ring to 2-D mesh"): for each Q slot, attention over the KV slots listed
// for it, FULL blocks entirely, DIAG blocks up to the diagonal, SKIP blocks
// not at all; the result is a partial output and log-sum-exp per query row.
//
// Work decomposition
//   workgroup = 12 waves (three per SIMD) sharing one KV head; each wave owns
//               32 query rows of one query head.  With GQA (G > 1) the waves
//               of a workgroup are query heads of one KV group, so one K/V
//               stream from memory serves all of them.
//   K/V are streamed through LDS in tiles of 64 keys by the DMA path of
//   buffer loads (memory -> LDS without registers) into five buffers (all of
//   LDS); the waves meet at a barrier every second tile, where the DMA of the
//   next two tiles starts.  Rows past the end of a partition read as zero
//   through the buffer's range check.
//   Within a wave the work runs over 32-key halves with a software pipeline:
//   the QK^T MFMAs of half j+1 are issued next to the exponentials of half j
//   (at a raised wave priority, with the row maximum of half j+1), then the
//   PV MFMAs of half j.
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
// Online softmax with a checked shift: a row's exponentials are taken
// against a shift that starts at the exact maximum of the row's first 32
// keys.  O and l share the shift, so any shift gives the same softmax as
// long as nothing overflows; instead of a row maximum per 32 keys, each
// half's exponent sum is checked, and only when it exceeds 2^20 (or
// overflowed) does the wave take the rescue path: the shift moves to the
// half's exact row maximum, O and l are rescaled, and the half's
// exponentials are taken again.  Probabilities below 2^20 are accumulated
// as they are; fp32 and bf16 keep their relative precision at that scale.
//
// LDS layouts (row-major, 16-byte chunks swizzled so that reads are free of
// bank conflicts; the DMA writes are contiguous per wave)
//   K: [64 keys][128 dims]; chunk c of key row n at chunk c ^ (n & 15).
//   V: [64 keys][128 dims]; chunk c of key row n at chunk c ^ (4 * (n & 3)).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kernels.h"
#include "tile_common.hpp"

// The DMA loads set M0 in inline assembly (see dma_tile); nothing else in
// this file uses M0.
#pragma clang diagnostic ignored "-Winline-asm"

namespace mesh_attn {
namespace {

using dev::kNegInf;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_raw __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;      // head dim
constexpr int BN = 64;      // keys per LDS tile
constexpr int NW = kTileWavesBf16;
constexpr int NT = NW * 64;
constexpr int kNBuf = 5;                    // LDS tiles in flight (5 x 32 KiB = all of LDS)
constexpr int kTileBytes = BN * D * 2;      // 16 KiB per K or V tile
constexpr int kBufBytes = 2 * kTileBytes;   // K then V
constexpr float kHalfSumLimit = 1048576.0f;  // 2^20: a half's exponent sum above it moves the shift
constexpr int kRsrcWord3 = 0x00020000;      // buffer resource flags for gfx9 (raw, 32-bit)
constexpr int kDmaRegions = 2 * kTileBytes / 1024;       // 1 KiB DMA loads per tile
constexpr int kDmaPerWave = (kDmaRegions + NW - 1) / NW;  // per wave (the last may idle)

static_assert(kWaveRowsBf16 == 32, "one 32-row block per wave");

typedef __amdgpu_buffer_rsrc_t Rsrc;
#define LDS_AS __attribute__((address_space(3)))

// Byte range of a descriptor that serves at most `max_rows` rows of
// `row_bytes` from its base, of which `rows` exist: loads from rows at or past
// `rows` return zero, with no branch.  Clamping to the rows actually read
// keeps the range in 32 bits however long the partition is.
__device__ __forceinline__ int rows_range(int rows, int max_rows, int row_bytes) {
    const int r = rows < max_rows ? rows : max_rows;
    return r > 0 ? (r - 1) * row_bytes + D * 2 : 0;
}

__device__ __forceinline__ Rsrc rows_rsrc(const void* base, int rows, int max_rows, int row_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                             rows_range(rows, max_rows, row_bytes), kRsrcWord3);
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
        const int reg = min(wave + NW * i, kDmaRegions - 1);  // 0..31
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
        ln.v_rofs[t] = kTileBytes + row * (D * 2) + chunk * 16 + (s16 & 1) * 8;
    }
}

// Buffer descriptor words (base, range in bytes) for the DMA loads below.
__device__ __forceinline__ u32x4 rows_desc(const void* base, int rows, int max_rows, int row_bytes) {
    const unsigned long long a = reinterpret_cast<unsigned long long>(base);
    const int n = rows_range(rows, max_rows, row_bytes);
    return u32x4{static_cast<unsigned>(a), static_cast<unsigned>(a >> 32) & 0xffffu,
                 static_cast<unsigned>(n), static_cast<unsigned>(kRsrcWord3)};
}

// Issues the DMA loads of one K/V tile into LDS buffer `buf` (rows past the
// range read as zero).  Written as assembly on purpose: the compiler then
// does not model these LDS writes, so it does not make reads of the other
// buffers wait for them; completion is awaited explicitly (vmcnt) before the
// barrier that publishes the tile.  M0 holds the LDS destination.
__device__ __forceinline__ void dma_tile(const Lanes& ln, u32x4 kr, u32x4 vr, unsigned buf, int wave) {
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
        const int reg = wave + NW * i;
        if (reg >= kDmaRegions) break;
        const unsigned dst = __builtin_amdgcn_readfirstlane(buf + reg * 1024);
        if (reg < 16)
            asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                         :: "s"(dst), "v"(ln.dma_gofs[i]), "s"(kr) : "memory", "m0");
        else
            asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                         :: "s"(dst), "v"(ln.dma_gofs[i]), "s"(vr) : "memory", "m0");
    }
}

__device__ __forceinline__ bf16x4 read_tr(const LDS_AS unsigned char* p) {
    const bf16x4_raw r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_raw*)p);
    return __builtin_bit_cast(bf16x4, r);
}

// S^T = K Q^T for the 32 keys of half h of the tile in `buf`.
__device__ __forceinline__ f32x16 qk_half(const Lanes& ln, const bf16x8 (&qf)[8],
                                          const LDS_AS unsigned char* buf, int h) {
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const bf16x8 ka = *reinterpret_cast<const LDS_AS bf16x8*>(buf + ln.k_rofs[c] + 8192 * h);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[c], s, 0, 0, 0);
    }
    return s;
}

// O^T += V^T P^T for the 32 keys of half h of the tile in `buf`.
__device__ __forceinline__ void pv_half(const Lanes& ln, f32x16 (&o)[4], const bf16x8 (&pb)[2],
                                        const LDS_AS unsigned char* buf, int h) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const int ks = 2 * h + kk;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const bf16x4 va = read_tr(buf + ln.v_rofs[t] + ks * 4096);
            const bf16x4 vb = read_tr(buf + ln.v_rofs[t] + ks * 4096 + 2048);
            const bf16x8 a8 = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
            o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a8, pb[kk], o[t], 0, 0, 0);
        }
    }
}

// Causal diagonal and ragged tail: hide keys after the query or past L.
__device__ __forceinline__ void mask_half(f32x16& s, int key0, int L, bool diag, int u) {
    const int g = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int kk = key0 + 8 * (i >> 2) + 4 * g + (i & 3);
        if (kk >= L || (diag && kk > u)) s[i] = kNegInf;
    }
}

__device__ __forceinline__ float row_max(const f32x16& s) {
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
    return dev::max_with_partner(mx);
}

// P = exp2(S*c - shift) in bf16, laid out as the B operand of the PV
// MFMAs; returns this lane's sum of P over the half.
__device__ __forceinline__ float softmax_half(const f32x16& s, float c2, float shift, bf16x8 (&pb)[2]) {
    float h = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float pv = dev::fast_exp2(__builtin_fmaf(s[i], c2, -shift));
        h += pv;
        pb[i >> 3][i & 7] = static_cast<__bf16>(pv);
    }
    return h;
}

// Rescue path (wave-uniform, rare): a half's exponent sum outgrew the limit.
// The shift moves up to the half's exact row maximum (never down), O and l
// are rescaled, and the half's probabilities are taken again.
__device__ __forceinline__ void rescue_half(const f32x16& s, float c2, float& shift, float& l,
                                                      f32x16 (&o)[4], bf16x8 (&pb)[2], float& h) {
    const float cand = row_max(s) * c2;
    const float next = cand > shift ? cand : shift;
    const float alpha = dev::fast_exp2(shift - next);
    shift = next;
    l *= alpha;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[t][i] *= alpha;
    h = softmax_half(s, c2, shift, pb);
}

// Checks a half's exponent sum and folds it into l.
__device__ __forceinline__ void settle_half(const f32x16& s, float c2, float& shift, float& l, f32x16 (&o)[4],
                                            bf16x8 (&pb)[2], float h) {
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(!(h <= kHalfSumLimit)) != 0, 0))
        rescue_half(s, c2, shift, l, o, pb, h);
    l += h;
}

__global__ __launch_bounds__(NT, 1) void tile_fwd_bf16_d128(const TileParams p) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem[kNBuf * kBufBytes];

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
    const int u = w.wave_tok0 + r32;  // this lane's query offset in its partition

    Lanes ln;
    init_lanes(ln, tid, wave, row_bytes);

    bf16x8 qf[8];  // Q^T fragments, d-chunk c: q[u][h][16c + 8g .. +7] (zero past L)
    {
        const int qrow_bytes = p.heads_q * D * 2;
        const __bf16* q0 = reinterpret_cast<const __bf16*>(p.q) +
                           ((size_t)(w.q_slot * L + w.wave_tok0) * p.heads_q + w.head) * D;
        const Rsrc qr = rows_rsrc(q0, L - w.wave_tok0, 32, qrow_bytes);
#pragma unroll
        for (int c = 0; c < 8; ++c)
            qf[c] = __builtin_bit_cast(
                bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qr, r32 * qrow_bytes + (16 * c + 8 * g) * 2,
                                                              0, 0));
    }
    f32x16 o[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[t][i] = 0.0f;
    float shift = 0.0f;  // shift of the exponentials (scaled base-2 scores), uniform per row
    float l = 0.0f;      // exponent sum over this lane's keys

    const int b_beg = p.sched.blk_off[w.q_slot];
    const int b_end = p.sched.blk_off[w.q_slot + 1];

    // The tiles of this Q slot form one sequence over (block, key tile); tile
    // t lives in LDS buffer t % 5.  The work runs over 32-key halves j with a
    // software pipeline: the QK^T MFMAs of half j+1 are issued together with
    // the exponentials of half j, then come the row maximum of half j+1 and
    // the PV MFMAs of half j.  Stepping from an odd tile t into tile t+1, the
    // waves wait for their DMA of tiles t+1 and t+2 and meet at a barrier;
    // tile t's V is still read after it (the PV of its last half), so the DMA
    // started there, for tiles t+3 and t+4, goes into the buffers of tiles t-2
    // and t-1, which every wave finished before the barrier.
    auto tile_end = [&](int bi_) {
        return (sched_entry(p.sched, bi_) & 3) == kDiag ? w.wg_tok_end : L;
    };
    auto advance = [&](int& bi_, int& n0_) {
        n0_ += BN;
        if (n0_ >= tile_end(bi_)) {
            ++bi_;
            n0_ = 0;
        }
    };
    const unsigned lds0 = static_cast<unsigned>(reinterpret_cast<uintptr_t>((LDS_AS unsigned char*)smem));
    auto issue = [&](int bi_, int n0_, int buf_) {
        const size_t off = (size_t)(sched_entry(p.sched, bi_) >> 2) * slot_elems + (size_t)n0_ * p.heads_kv * D;
        dma_tile(ln, rows_desc(kbase + off, L - n0_, BN, row_bytes), rows_desc(vbase + off, L - n0_, BN, row_bytes),
                 lds0 + buf_ * kBufBytes, wave);
    };
    auto vmcnt0_barrier = [&]() {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };

    if (b_beg < b_end) {
        const LDS_AS unsigned char* lds = (const LDS_AS unsigned char*)smem;
        auto is_diag = [&](int bi_) { return (sched_entry(p.sched, bi_) & 3) == kDiag; };
        auto needs_mask = [&](bool diag_, int key0) {
            return (diag_ && key0 + 31 > w.wave_tok0) || key0 + 32 > L;
        };
        auto next_buf = [](int b) { return b == kNBuf - 1 ? 0 : b + 1; };
        // DMA cursor: the next tile to load and its buffer.
        int dbi = b_beg, dn0 = 0, dbuf = 0;
        auto issue_next = [&]() {
            if (dbi < b_end) {
                issue(dbi, dn0, dbuf);
                advance(dbi, dn0);
                dbuf = next_buf(dbuf);
            }
        };
        int bi = b_beg, n0 = 0;    // tile t
        bool dg = is_diag(bi);
        int bi1 = bi, n01 = n0;    // tile t+1
        advance(bi1, n01);
        int t = 0, buf = 0;
        issue_next();  // tiles 0 and 1
        issue_next();
        vmcnt0_barrier();
        issue_next();  // tiles 2 and 3
        issue_next();

        f32x16 s = qk_half(ln, qf, lds, 0);
        if (needs_mask(dg, n0)) mask_half(s, n0, L, dg, u);
        {
            const float m0 = row_max(s) * c2;
            shift = m0 == kNegInf ? 0.0f : m0;  // a row with no visible key yet keeps 0
        }

        // One pipeline step from half H of the tile in `cur` to the next half
        // (half 1 of the same tile, or half 0 of the next tile in `nxt`).
        auto step = [&](auto h_tag, const LDS_AS unsigned char* cur, const LDS_AS unsigned char* nxt,
                        bool mask_next, bool diag_next, int key0_next) {
            constexpr int H = decltype(h_tag)::value;
            // QK^T of the next half with the exponentials of this half at a
            // raised wave priority: the SIMD's arbiter then favours the wave
            // whose dependent QK chain is waiting to issue over the other two
            // waves' PV work.
            __builtin_amdgcn_s_setprio(1);
            f32x16 s_next = qk_half(ln, qf, nxt, H ^ 1);
            bf16x8 pb[2];
            const float h = softmax_half(s, c2, shift, pb);
            if (mask_next) mask_half(s_next, key0_next, L, diag_next, u);
            __builtin_amdgcn_s_setprio(0);
            settle_half(s, c2, shift, l, o, pb, h);
            // PV of this half.
            pv_half(ln, o, pb, cur, H);
            s = s_next;
        };

        for (;;) {
            const LDS_AS unsigned char* cur = lds + buf * kBufBytes;
            // Half 0 -> half 1 of tile t.
            step(std::integral_constant<int, 0>{}, cur, cur, needs_mask(dg, n0 + 32), dg, n0 + 32);
            if (bi1 >= b_end) break;
            // Into tile t+1.  Every second tile the waves wait for their DMA
            // (tiles t+1 and t+2 were loaded together) and meet at a barrier;
            // every wave has then finished tile t-1, so the buffers of tiles
            // t-2 and t-1 take tiles t+3 and t+4.
            if ((t & 1) == 1) {
                vmcnt0_barrier();
                issue_next();
                issue_next();
            }
            const int nbuf = next_buf(buf);
            const bool dg1 = is_diag(bi1);
            step(std::integral_constant<int, 1>{}, cur, lds + nbuf * kBufBytes, needs_mask(dg1, n01), dg1,
                 n01);
            buf = nbuf;
            ++t;
            bi = bi1;
            n0 = n01;
            dg = dg1;
            advance(bi1, n01);
        }
        // Second half of the last tile.
        bf16x8 pb[2];
        const float h = softmax_half(s, c2, shift, pb);
        settle_half(s, c2, shift, l, o, pb, h);
        pv_half(ln, o, pb, lds + buf * kBufBytes, 1);
    }

    // Epilogue: O = O_acc / l, lse = ln(2) * (shift + log2 l); empty rows -> (0, -inf).
    const float l_tot = dev::add_with_partner(l);
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
                for (int j = 0; j < 4; ++j) ov[j] = static_cast<__bf16>(o[t][4 * ib + j] * inv);
                *reinterpret_cast<bf16x4*>(op + 32 * t + 8 * ib + 4 * g) = ov;
            }
        if (g == 0) p.lse[q_row] = l_tot > 0.0f ? (shift + __log2f(l_tot)) * dev::kLn2 : kNegInf;
    }
}

}  // namespace

hipError_t launch_tile_fwd_bf16(const TileParams& p, int head_dim, hipStream_t stream) {
    if (head_dim != D || p.wave_rows != kWaveRowsBf16) return hipErrorInvalidValue;
    const unsigned n_wg = static_cast<unsigned>(tile_fwd_grid(p));
    hipLaunchKernelGGL(tile_fwd_bf16_d128, dim3(n_wg), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mesh_attn
