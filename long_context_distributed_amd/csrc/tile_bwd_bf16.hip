// Tile backward, bf16 inputs, head_dim 128, for gfx950 (MI355X).
//
// One tile's share of the attention gradients: for every visible pair of
// query row i and key j of the tile (same visibility as the forward),
//   P = exp(s - lse_i),  dV_j += P dO_i,  dS = P (dO_i . v_j - D_i),
//   dQ_i += scale dS k_j,  dK_j += scale dS q_i,
// with the rows' final lse and D = rowsum(dO * O) as inputs.  The pages aim
// Mesh-Attention at long-context training (tutorial page, greedy-scheduling
// section and closing summary) without giving the backward; this is the
// plain derivative of softmax attention.
//
// Two kernels, so that no gradient needs atomics:
//   tile_bwd_dq:   Q-stationary, the forward's work decomposition and K/V
//                  streaming; per 32 keys it recomputes S^T = K Q^T and
//                  dP^T = V dO^T and accumulates dQ^T += K^T dS^T.
//   tile_bwd_dkdv: KV-stationary; a workgroup owns 256 keys of one KV head
//                  (32 per wave; K in LDS, V in registers) and streams the
//                  query rows of every Q slot that sees them, 64 rows of one
//                  query head per stage (DMA into two LDS stages, one barrier
//                  per stage); per 32 rows it computes S = Q K^T and
//                  dP = dO V^T and accumulates dV^T += dO^T P and dK^T += Q^T dS.
// Each recomputes what the other needs (7 matrix products per pair instead
// of the 5 of the gradient formulas).
//
// Matrix-core use (v_mfma_f32_32x32x16_bf16).  In a 32x32 accumulator, lane l
// holds column l%32 and rows 8*(r/4) + 4*(l/32) + r%4 for register r.
//   dQ kernel: columns are query rows, so lse and D are one value per lane;
//     dQ^T's A operand K^T is read with ds_read_b64_tr_b16 in the same key
//     order as dS^T's registers (as V^T in the forward).
//   dK/dV kernel: columns are keys, rows are query rows, so lse and D enter
//     as the accumulators' initial values: S starts at -lse/scale and dP at
//     -D, then P = exp2(S * scale * log2 e) and dS = P * dP with no extra
//     per-element work.  dO^T and Q^T are read transposed in the register
//     order of P and dS.
//
// LDS tiles are row-major with 256-byte rows (128 bf16) and 16-byte chunks
// swizzled by swz(row) = 4*(row & 3) | ((row >> 2) & 3): both the 16-byte row
// reads (16 consecutive rows) and the transposed reads (4 rows x 64 bytes)
// then hit distinct banks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "tile_common.hpp"

// The DMA loads set M0 in inline assembly (see dma_1k); nothing else in this
// file uses M0.
#pragma clang diagnostic ignored "-Winline-asm"

namespace mesh_attn {
namespace {

using dev::kNegInf;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_raw __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t Rsrc;
#define LDS_AS __attribute__((address_space(3)))

constexpr int D = 128;
constexpr int kRowBytes = D * 2;           // one staged row
constexpr int kRsrcWord3 = 0x00020000;     // buffer resource flags for gfx9 (raw, 32-bit)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kPosInf = __builtin_inff();

static_assert(kBwdRowsPerWave == 32, "one 32-row (32-key) block per wave");

__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// Byte range of a descriptor that serves at most `max_rows` rows of
// `row_bytes` from its base, of which `rows` exist: reads of rows at or past
// `rows` return zero.  Clamping to the rows actually read keeps the range in
// 32 bits however long the partition is.
__device__ __forceinline__ int rows_range(int rows, int max_rows, int row_bytes) {
    const int r = rows < max_rows ? rows : max_rows;
    return r > 0 ? (r - 1) * row_bytes + kRowBytes : 0;
}

__device__ __forceinline__ Rsrc rows_rsrc(const void* base, int rows, int max_rows, int row_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                             rows_range(rows, max_rows, row_bytes), kRsrcWord3);
}

// The same as raw descriptor words, for the DMA loads.
__device__ __forceinline__ u32x4 rows_desc(const void* base, int rows, int max_rows, int row_bytes) {
    const unsigned long long a = reinterpret_cast<unsigned long long>(base);
    const int n = rows_range(rows, max_rows, row_bytes);
    return u32x4{static_cast<unsigned>(a), static_cast<unsigned>(a >> 32) & 0xffffu,
                 static_cast<unsigned>(n), static_cast<unsigned>(kRsrcWord3)};
}

// One DMA load: 64 lanes x 16 bytes from the buffer at per-lane offsets into
// the 1 KiB of LDS at `dst` (lane l to dst + 16 l).  Assembly so that the
// compiler does not make other LDS reads wait for it; completion is awaited
// (vmcnt) before the barrier that publishes the tile.
__device__ __forceinline__ void dma_1k(unsigned dst, int gofs, u32x4 desc) {
    const unsigned d = __builtin_amdgcn_readfirstlane(dst);
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(d), "v"(gofs), "s"(desc) : "memory", "m0");
}

__device__ __forceinline__ bf16x4 read_tr(const LDS_AS unsigned char* p) {
    const bf16x4_raw r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_raw*)p);
    return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 read_b128(const LDS_AS unsigned char* p) {
    return *reinterpret_cast<const LDS_AS bf16x8*>(p);
}

// Byte offsets of this lane's reads in a swizzled tile.
//   row[c]:   16-byte row read of row r32, chunk 2c+g (an A or B operand whose
//             lanes are rows and whose k-index runs along the row).
//   tr[t][e]: transposed read giving lane (dim 32t + l%32, g) four values of
//             rows 8e + 4g + 0..3; add 4096 per further 16 rows.
struct TileOffsets {
    int row[8];
    int tr[4][2];
};

__device__ __forceinline__ void init_offsets(TileOffsets& to, int lane) {
    const int g = lane >> 5, r32 = lane & 31;
#pragma unroll
    for (int c = 0; c < 8; ++c) to.row[c] = r32 * kRowBytes + (((2 * c + g) ^ swz(r32)) << 4);
    const int s16 = lane & 15, half = (lane >> 4) & 1, x = s16 >> 2, b = (s16 & 3) >> 1;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int row = 8 * e + 4 * g + x;
            const int chunk = (4 * t + 2 * half + b) ^ swz(row);
            to.tr[t][e] = row * kRowBytes + chunk * 16 + (s16 & 1) * 8;
        }
}

// A operand of 32 dims (32t ..) x 16 rows (16ks ..) of a tile, transposed.
__device__ __forceinline__ bf16x8 tr_frag(const TileOffsets& to, const LDS_AS unsigned char* tile,
                                          int t, int ks) {
    const bf16x4 a = read_tr(tile + to.tr[t][0] + ks * 4096);
    const bf16x4 b = read_tr(tile + to.tr[t][1] + ks * 4096);
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// ----------------------------------------------------------------------------
// Query-gradient kernel

constexpr int QW = kBwdDqWaves;
constexpr int QT = QW * 64;
constexpr int BN = 64;                          // keys per LDS tile
constexpr int kTileBytes = BN * kRowBytes;      // 16 KiB for K or V
constexpr int kBufBytes = 2 * kTileBytes;       // K then V
constexpr int kNBuf = 5;                        // tiles in flight (160 KiB)
constexpr int kDmaRegions = kBufBytes / 1024;   // 32 DMA loads per tile
constexpr int kDmaPerWave = kDmaRegions / QW;
static_assert(kDmaRegions % QW == 0, "DMA loads split evenly over the waves");

__global__ __launch_bounds__(QT, 1) void tile_bwd_dq_bf16_d128(const BwdDqParams p) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem[kNBuf * kBufBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, r32 = lane & 31;
    const int L = p.part_len;
    const dev::WorkItem w = dev::decode_work(p, wave);
    const float c2 = p.scale_log2e;
    const int row_bytes = p.heads_kv * kRowBytes;
    const __bf16* kbase = reinterpret_cast<const __bf16*>(p.k) + (size_t)w.kv_head * D;
    const __bf16* vbase = reinterpret_cast<const __bf16*>(p.v) + (size_t)w.kv_head * D;
    const size_t slot_elems = (size_t)L * p.heads_kv * D;
    const int u = w.wave_tok0 + r32;  // this lane's query offset in its partition
    const size_t q_row = (size_t)(w.q_slot * L + min(u, L - 1)) * p.heads_q + w.head;

    TileOffsets to;
    init_offsets(to, lane);
    int dma_gofs[kDmaPerWave];  // load i fills region wave + QW*i: rows 4*(reg%16) + l/16
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
        const int reg = wave + QW * i;
        const int row = 4 * (reg & 15) + (lane >> 4);
        dma_gofs[i] = row * row_bytes + (((lane & 15) ^ swz(row)) << 4);
    }

    // Q^T and dO^T fragments (B operands): row u, dims 16c + 8g .. +7.
    bf16x8 qf[8], dof[8];
    {
        const int qrow_bytes = p.heads_q * kRowBytes;
        const size_t first = ((size_t)(w.q_slot * L + w.wave_tok0) * p.heads_q + w.head) * D;
        const Rsrc qr = rows_rsrc(reinterpret_cast<const __bf16*>(p.q) + first, L - w.wave_tok0, 32, qrow_bytes);
        const Rsrc dr = rows_rsrc(reinterpret_cast<const __bf16*>(p.dout) + first, L - w.wave_tok0, 32,
                                  qrow_bytes);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int off = r32 * qrow_bytes + (16 * c + 8 * g) * 2;
            qf[c] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qr, off, 0, 0));
            dof[c] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(dr, off, 0, 0));
        }
    }
    // Per-row terms: exp2 shift lse*log2(e) (+inf: the row contributes nothing) and D.
    float lse2 = kPosInf, dlt = 0.0f;
    if (u < L) {
        const float ls = p.lse[q_row];
        if (ls > kNegInf) {
            lse2 = ls * kLog2e;
            dlt = p.delta[q_row];
        }
    }

    f32x16 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[t][i] = 0.0f;

    const int b_beg = p.sched.blk_off[w.q_slot];
    const int b_end = p.sched.blk_off[w.q_slot + 1];
    auto tile_end = [&](int bi_) { return (sched_entry(p.sched, bi_) & 3) == kDiag ? w.wg_tok_end : L; };
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
        const u32x4 kr = rows_desc(kbase + off, L - n0_, BN, row_bytes);
        const u32x4 vr = rows_desc(vbase + off, L - n0_, BN, row_bytes);
        const unsigned dst = lds0 + buf_ * kBufBytes;
#pragma unroll
        for (int i = 0; i < kDmaPerWave; ++i) {
            const int reg = wave + QW * i;
            dma_1k(dst + reg * 1024, dma_gofs[i], reg < 16 ? kr : vr);
        }
    };
    auto vmcnt0_barrier = [&]() {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };

    if (b_beg < b_end) {
        const LDS_AS unsigned char* lds = (const LDS_AS unsigned char*)smem;
        auto next_buf = [](int b) { return b == kNBuf - 1 ? 0 : b + 1; };
        int dbi = b_beg, dn0 = 0, dbuf = 0;  // DMA cursor
        auto issue_next = [&]() {
            if (dbi < b_end) {
                issue(dbi, dn0, dbuf);
                advance(dbi, dn0);
                dbuf = next_buf(dbuf);
            }
        };
        issue_next();  // tiles 0 and 1
        issue_next();
        vmcnt0_barrier();
        issue_next();  // tiles 2 and 3
        issue_next();

        int bi = b_beg, n0 = 0, buf = 0, t = 0;
        for (;;) {
            const bool dg = (sched_entry(p.sched, bi) & 3) == kDiag;
            const LDS_AS unsigned char* kt = lds + buf * kBufBytes;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int key0 = n0 + 32 * h;
                // S^T = K Q^T and dP^T = V dO^T for 32 keys, at a raised wave
                // priority so that the two MFMA chains issue ahead of the other
                // wave's VALU work (measured: ~3% faster for this kernel).
                __builtin_amdgcn_s_setprio(1);
                f32x16 s, dp;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    s[i] = 0.0f;
                    dp[i] = 0.0f;
                }
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_b128(kt + to.row[c] + 8192 * h), qf[c], s, 0, 0, 0);
                    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_b128(kt + kTileBytes + to.row[c] + 8192 * h),
                                                                 dof[c], dp, 0, 0, 0);
                }
                __builtin_amdgcn_s_setprio(0);
                if ((dg && key0 + 31 > w.wave_tok0) || key0 + 32 > L) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int kk = key0 + 8 * (i >> 2) + 4 * g + (i & 3);
                        if (kk >= L || (dg && kk > u)) s[i] = kNegInf;
                    }
                }
                // dS^T = P^T (dP^T - D), P^T = exp2(S^T c - lse log2 e)
                bf16x8 dsb[2];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float pv = dev::fast_exp2(__builtin_fmaf(s[i], c2, -lse2));
                    dsb[i >> 3][i & 7] = static_cast<__bf16>(pv * (dp[i] - dlt));
                }
                // dQ^T += K^T dS^T
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt)
                        acc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag(to, kt, tt, 2 * h + kk), dsb[kk],
                                                                          acc[tt], 0, 0, 0);
            }
            int bi1 = bi, n01 = n0;
            advance(bi1, n01);
            if (bi1 >= b_end) break;
            // Every second tile: wait for the DMA of the next two tiles and
            // meet at a barrier; every wave has then finished tiles t-1 and t,
            // so their buffers take tiles t+3 and t+4.
            if ((t & 1) == 1) {
                vmcnt0_barrier();
                issue_next();
                issue_next();
            }
            bi = bi1;
            n0 = n01;
            buf = next_buf(buf);
            ++t;
        }
    }

    // dQ = scale * dQ^T, float32, rows of this wave that exist.
    if (u < L) {
        float* op = p.dq + q_row * D;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                const f32x4 val = {acc[tt][4 * ib] * p.scale, acc[tt][4 * ib + 1] * p.scale,
                                   acc[tt][4 * ib + 2] * p.scale, acc[tt][4 * ib + 3] * p.scale};
                *reinterpret_cast<f32x4*>(op + 32 * tt + 8 * ib + 4 * g) = val;
            }
    }
}

// ----------------------------------------------------------------------------
// Key/value-gradient kernel

constexpr int KW = kBwdDkvWaves;
constexpr int KT = KW * 64;
constexpr int KB = KW * kBwdRowsPerWave;        // keys per workgroup
constexpr int kRows = 64;                       // query rows per stage (two 32-row blocks)
constexpr int kStageTile = kRows * kRowBytes;   // 16 KiB of Q or dO
constexpr int kTermOff = 2 * kStageTile;        // then -lse/scale and -D, one float per row each
constexpr int kStageBytes = kTermOff + 2 * kRows * 4;
constexpr int kNStage = 2;
constexpr int kKTileBytes = KB * kRowBytes;     // 64 KiB
constexpr int kStageRegions = 2 * kStageTile / 1024;    // DMA loads per stage (Q then dO)
constexpr int kStageDmaPerWave = kStageRegions / KW;
static_assert(kStageRegions % KW == 0, "stage DMA loads split evenly over the waves");
static_assert(KB * 16 % KT == 0, "K tile chunks split evenly over the threads");
static_assert(kRows == 64, "row terms are written by one wave, one lane per row");

__device__ __forceinline__ int kv_entry(const KvSchedule& s, int i) {
    const uint32_t word = reinterpret_cast<const uint32_t*>(s.blk)[i >> 2];
    return (word >> (8 * (i & 3))) & 0xff;
}

__global__ __launch_bounds__(KT, 1) void tile_bwd_dkdv_bf16_d128(const BwdDkvParams p) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem[kKTileBytes + kNStage * kStageBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, r32 = lane & 31;
    const int L = p.part_len;
    const int G = p.group;
    const dev::KeyBlock kbk = dev::decode_key_block_at(p, static_cast<int>(blockIdx.x));
    const int kv_head = kbk.kv_head;
    const int kb = kbk.key_block;
    const int kv_slot = kbk.kv_slot;
    const int key0 = kb * KB;               // first key of the workgroup (partition offset)
    const int kw0 = key0 + 32 * wave;       // first key of this wave
    const int key = kw0 + r32;              // this lane's key
    const int kv_row_bytes = p.heads_kv * kRowBytes;
    const int q_row_bytes = p.heads_q * kRowBytes;
    const float c2 = p.scale_log2e;
    const float neg_inv_scale = -1.0f / p.scale;

    LDS_AS unsigned char* lds = (LDS_AS unsigned char*)smem;
    LDS_AS unsigned char* ktile = lds;
    const unsigned stage0 = static_cast<unsigned>(reinterpret_cast<uintptr_t>(lds + kKTileBytes));

    TileOffsets to;
    init_offsets(to, lane);
    // Stage DMA: load i of this wave fills region reg = wave + KW*i (Q rows
    // 4*reg .. for reg < 16, dO rows 4*(reg-16) .. after), lane l to row
    // 4*(reg%16) + l/16, physical chunk l%16.
    int dma_gofs[kStageDmaPerWave];
#pragma unroll
    for (int i = 0; i < kStageDmaPerWave; ++i) {
        const int reg = wave + KW * i;
        const int row = 4 * (reg & 15) + (lane >> 4);
        dma_gofs[i] = row * q_row_bytes + (((lane & 15) ^ swz(row)) << 4);
    }

    // K tile of the workgroup's keys into LDS; V^T fragments (B operand of
    // dP = dO V^T: key r32 of this wave, dims 16c + 8g ..) into registers.
    const size_t kv_first = ((size_t)(kv_slot * L + key0) * p.heads_kv + kv_head) * D;
    {
        const Rsrc kr = rows_rsrc(reinterpret_cast<const __bf16*>(p.k) + kv_first, L - key0, KB, kv_row_bytes);
#pragma unroll
        for (int i = 0; i < KB * 16 / KT; ++i) {
            const int chunk_id = tid + KT * i;
            const int row = chunk_id >> 4, c = chunk_id & 15;
            const u32x4 val = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, row * kv_row_bytes + c * 16, 0, 0));
            *reinterpret_cast<LDS_AS u32x4*>(ktile + row * kRowBytes + ((c ^ swz(row)) << 4)) = val;
        }
    }
    bf16x8 vf[8];
    {
        const Rsrc vr = rows_rsrc(reinterpret_cast<const __bf16*>(p.v) + kv_first + (size_t)32 * wave * p.heads_kv * D,
                                  L - kw0, 32, kv_row_bytes);
#pragma unroll
        for (int c = 0; c < 8; ++c)
            vf[c] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(vr, r32 * kv_row_bytes + (16 * c + 8 * g) * 2, 0, 0));
        // Wait for V here: left to its first use inside the loop, the wait
        // counts the untracked stage DMA too and would stall every stage on
        // the next stage's loads.
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            u32x4 t = __builtin_bit_cast(u32x4, vf[c]);
            asm volatile("" : "+v"(t));
            vf[c] = __builtin_bit_cast(bf16x8, t);
        }
    }

    f32x16 dk[4], dv[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            dk[t][i] = 0.0f;
            dv[t][i] = 0.0f;
        }

    // Items: (entry e, row tile r0 of 64 rows, head hh), head innermost.  A
    // DIAG entry starts at row key0: earlier rows see none of these keys.
    const int e_beg = p.sched.blk_off[kv_slot];
    const int e_end = p.sched.blk_off[kv_slot + 1];
    auto first_row = [&](int e) { return (kv_entry(p.sched, e) & 3) == kDiag ? key0 : 0; };
    int e = e_beg, r0 = e_beg < e_end ? first_row(e_beg) : 0, hh = 0;
    auto step_item = [&](int& e_, int& r0_, int& hh_) {
        if (++hh_ == G) {
            hh_ = 0;
            r0_ += kRows;
            if (r0_ >= L) {
                ++e_;
                r0_ = e_ < e_end ? first_row(e_) : 0;
            }
        }
    };

    // Issues the loads of item (e_, r0_, hh_) into stage st: Q and dO rows by
    // DMA (rows at or past L read as zero), and, on wave 0, the rows' lse and
    // D into registers (one row per lane).  The row terms reach LDS through
    // store_terms once the current stage's work is done, so that wave 0 does
    // not wait for this stage's loads before its own matrix work.
    float ls_in = kNegInf, dl_in = 0.0f;
    int rr_in = 0;
    auto load_item = [&](int e_, int r0_, int hh_, int st) {
        const int s = kv_entry(p.sched, e_) >> 2;
        const int h = kv_head * G + hh_;
        const size_t first = ((size_t)(s * L + r0_) * p.heads_q + h) * D;
        const u32x4 qd = rows_desc(reinterpret_cast<const __bf16*>(p.q) + first, L - r0_, kRows, q_row_bytes);
        const u32x4 dd = rows_desc(reinterpret_cast<const __bf16*>(p.dout) + first, L - r0_, kRows, q_row_bytes);
        const unsigned dst = stage0 + st * kStageBytes;
#pragma unroll
        for (int i = 0; i < kStageDmaPerWave; ++i) {
            const int reg = wave + KW * i;
            dma_1k(dst + reg * 1024, dma_gofs[i], reg < 16 ? qd : dd);
        }
        if (wave == 0) {
            // Unconditional loads of an in-range row (the last one for rows
            // past L); store_terms decides what the row contributes.
            rr_in = r0_ + lane;
            const size_t qi = (size_t)(s * L + min(rr_in, L - 1)) * p.heads_q + h;
            ls_in = p.lse[qi];
            dl_in = p.delta[qi];
        }
    };
    // Row terms of the loaded item into stage st: -lse/scale (-inf for rows
    // that see nothing) and -D, one float per row (wave 0).
    auto store_terms = [&](int st) {
        if (wave == 0) {
            LDS_AS float* terms = reinterpret_cast<LDS_AS float*>(lds + kKTileBytes + st * kStageBytes + kTermOff);
            const bool live = rr_in < L && ls_in > kNegInf;
            terms[lane] = live ? ls_in * neg_inv_scale : kNegInf;
            terms[kRows + lane] = live ? -dl_in : 0.0f;
        }
    };
    auto vmcnt0_barrier = [&]() {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };

    const LDS_AS unsigned char* kw_tile = ktile + 32 * wave * kRowBytes;
    int st = 0;
    if (e < e_end) {
        load_item(e, r0, hh, 0);
        store_terms(0);
    }
    vmcnt0_barrier();  // K tile and stage 0

    while (e < e_end) {
        int e1 = e, r01 = r0, hh1 = hh;
        step_item(e1, r01, hh1);
        const bool more = e1 < e_end;
        // The other stage was last read before the previous barrier.
        if (more) load_item(e1, r01, hh1, st ^ 1);

        const LDS_AS unsigned char* base = lds + kKTileBytes + st * kStageBytes;
        const bool dg = (kv_entry(p.sched, e) & 3) == kDiag;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int rs = r0 + 32 * sub;          // first row of this 32-row block
            if (rs >= L) break;                    // uniform: past the partition
            const LDS_AS unsigned char* qb = base + sub * 32 * kRowBytes;
            const LDS_AS unsigned char* db = qb + kStageTile;
            const LDS_AS unsigned char* tb = base + kTermOff + 4 * 32 * sub;
            // S = Q K^T - lse/scale and dP = dO V^T - D (row terms as initial values).
            f32x16 s, dp;
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                const f32x4 a = *reinterpret_cast<const LDS_AS f32x4*>(tb + 4 * (8 * ib + 4 * g));
                const f32x4 b = *reinterpret_cast<const LDS_AS f32x4*>(tb + 4 * kRows + 4 * (8 * ib + 4 * g));
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    s[4 * ib + j] = a[j];
                    dp[4 * ib + j] = b[j];
                }
            }
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_b128(qb + to.row[c]), read_b128(kw_tile + to.row[c]), s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_b128(db + to.row[c]), vf[c], dp, 0, 0, 0);
            }
            if (kw0 + 31 >= L || (dg && kw0 + 31 > rs)) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int row = rs + 8 * (i >> 2) + 4 * g + (i & 3);
                    if (key >= L || (dg && key > row)) s[i] = kNegInf;
                }
            }
            bf16x8 pb[2], dsb[2];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float pv = dev::fast_exp2(s[i] * c2);
                pb[i >> 3][i & 7] = static_cast<__bf16>(pv);
                dsb[i >> 3][i & 7] = static_cast<__bf16>(pv * dp[i]);
            }
            // dV^T += dO^T P, dK^T += Q^T dS
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    dv[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag(to, db, t, kk), pb[kk], dv[t], 0, 0, 0);
                    dk[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag(to, qb, t, kk), dsb[kk], dk[t], 0, 0, 0);
                }
        }
        store_terms(st ^ 1);  // unused when this was the last item
        vmcnt0_barrier();  // the next stage has landed; this one is free
        st ^= 1;
        e = e1;
        r0 = r01;
        hh = hh1;
    }

    if (key < L) {
        const size_t orow = ((size_t)(kv_slot * L + key) * p.heads_kv + kv_head) * D;
        float* kp = p.dk + orow;
        float* vp = p.dv + orow;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                const int d0 = 32 * t + 8 * ib + 4 * g;
                *reinterpret_cast<f32x4*>(kp + d0) = f32x4{dk[t][4 * ib] * p.scale, dk[t][4 * ib + 1] * p.scale,
                                                           dk[t][4 * ib + 2] * p.scale, dk[t][4 * ib + 3] * p.scale};
                *reinterpret_cast<f32x4*>(vp + d0) = f32x4{dv[t][4 * ib], dv[t][4 * ib + 1], dv[t][4 * ib + 2],
                                                           dv[t][4 * ib + 3]};
            }
    }
}

}  // namespace

hipError_t launch_tile_bwd_bf16(const BwdDqParams& pq, const BwdDkvParams& pk, int head_dim,
                               hipStream_t stream) {
    if (head_dim != D || pq.wave_rows != kBwdRowsPerWave) return hipErrorInvalidValue;
    const unsigned n_wg_q = static_cast<unsigned>(tile_fwd_grid(pq));
    hipLaunchKernelGGL(tile_bwd_dq_bf16_d128, dim3(n_wg_q), dim3(QT), 0, stream, pq);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned n_wg_k = static_cast<unsigned>(tile_bwd_dkdv_grid(pk));
    hipLaunchKernelGGL(tile_bwd_dkdv_bf16_d128, dim3(n_wg_k), dim3(KT), 0, stream, pk);
    return hipGetLastError();
}

}  // namespace mesh_attn
