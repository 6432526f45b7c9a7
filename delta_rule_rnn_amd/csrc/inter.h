// inter.h -- K2: the sequential inter-chunk state pass (step a4) fused with
// the chunk output (step a5).
//
// Page keys: [KDA] "TileLang 实战：KDA 从零到一–Kimi Delta Attention";
// [SD] "TileLang 实战：KDA 从零到一--标量衰减"; [DPLR] "RNN的复兴04:线性注意力
// 并行计算DPLR".
//
// For each (batch, head), chunks in order, with S the [Dk, Dv] state
// (transpose of the pages' S) kept in fp32 MFMA accumulators:
//   Vnew = U - W S               (decay_la: Vnew = V)
//   O    = Q~ S + Aqk Vnew       (entry state read + intra-chunk term)
//   S   <- Diag(phi) S + Kbar^T Vnew
// ([DPLR] 5.3.5 standard KDA/GDN form; [KDA] 3.2 reference B; the state is
// updated only after the output used the entry state and the decay is
// applied before the accumulation, [SD] 5.2 ordering rules 1 and 2).
//
// Work split.  A workgroup owns one (b, h) chain and DVS = 16*NTN value
// columns (value columns evolve independently, [KDA] 3.4).  Its 4 waves split
// the rows: wave w produces 16 positions of Vnew and O (rows 32*(w/2) +
// prow(w%2, r)) and 32 key rows of S (rows 32w..32w+31).  Two LDS exchanges
// per chunk hand Vnew and S to every wave as natural B fragments.  The
// operands of the next NBUF-1 chunks are prefetched into registers while the
// current chunk computes.
//
// Block mapping: the NV = Dv/DVS workgroups of a chain read the same W, Q~,
// Kbar, Aqk; consecutive logical ids are placed on the same XCD (hardware
// dispatches workgroup i to XCD i % 8) so they share that XCD's L2.
#pragma once

#include <type_traits>

#include "common.h"

namespace dr {

template <typename T, int DK, int NTN>
struct InterOps {
    static constexpr int NKB = DK / 32;
    Frag<T> w[NKB];        // W rows of this wave's positions
    Frag<T> qt[NKB];       // Q~ rows of this wave's positions
    Frag<T> aqk[2];        // Aqk rows, key blocks 0..1
    Frag<T> kb[2][2];      // Kbar^T rows (half, key block) of this wave's S rows
    float u[NTN][4];       // U (or V) at this lane's 4 positions, per n-tile
    float phi[2][4];       // phi at this lane's S rows (half, i)
};

template <int KIND, typename T, int DK, int DV, int NTN>
__device__ __forceinline__ void inter_load(InterOps<T, DK, NTN>& op, const uint8_t* recb, int wave,
                                           int lane, int dv0)
{
    using R = Rec<T, DK, DV>;
    constexpr int C = kChunk;
    constexpr int NKB = DK / 32;
    constexpr bool DELTA = KIND != KIND_LA;
    const T* base = reinterpret_cast<const T*>(recb);
    // all blocks are in fragment order: lane l's 8 (or 4) elements are
    // contiguous and a wave-wide load is one contiguous run
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
        const size_t f = ((size_t)(wave * NKB + kb) * 64 + lane) * 8;
        if constexpr (DELTA) op.w[kb] = ld_frag(base + R::W + f);
        op.qt[kb] = ld_frag(base + R::QT + f);
    }
    // both key blocks: the record holds zeros above the diagonal, so the
    // block past this wave's positions contributes nothing
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) op.aqk[kb] = ld_frag(base + R::AQK + ((size_t)(wave * 2 + kb) * 64 + lane) * 8);
    if (NKB >= 4 || wave < NKB) {
        const float* phi = reinterpret_cast<const float*>(recb + R::PHI_BYTE);
        const int grp = lane >> 4;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                op.kb[half][kb] = ld_frag(base + R::KBT + ((size_t)((wave * 2 + half) * 2 + kb) * 64 + lane) * 8);
            ld4(phi + 32 * wave + 8 * grp + 4 * half, op.phi[half]);
        }
    }
#pragma unroll
    for (int n = 0; n < NTN; ++n)
        ld4(base + R::UT + ((size_t)((dv0 / 16 + n) * 4 + wave) * 64 + lane) * 4, op.u[n]);
}

template <int KIND, typename T, int DK, int DV, int NTN, int NBUF>
__global__ __launch_bounds__(kThreads) void inter_kernel(const uint8_t* __restrict__ ws,
                                                         const float* __restrict__ h0,
                                                         T* __restrict__ o, float* __restrict__ hT,
                                                         int Tlen, int H, int NT, int c0,
                                                         int nseg)
{
    using R = Rec<T, DK, DV>;
    constexpr int C = kChunk;
    constexpr int DVS = 16 * NTN;
    constexpr int NV = DV / DVS;
    constexpr int NKB = DK / 32;
    constexpr bool DELTA = KIND != KIND_LA;
    static_assert(DV % DVS == 0, "value split");

    // B-fragment exchange buffers: [block][n-tile][lane][8 slots]
    __shared__ __attribute__((aligned(16))) T sS[NKB][NTN][64][8];
    __shared__ __attribute__((aligned(16))) T sV[2][NTN][64][8];
    // per-wave output staging: 16 positions x 16*NTN columns, one row per
    // position, so the tile leaves as 16-byte row segments
    constexpr int LDO = 16 * NTN + 8;
    __shared__ __attribute__((aligned(16))) T sO[4][16][LDO];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, grp = lane >> 4;
    const int kbP = wave >> 1, halfP = wave & 1;
    const bool ownS = NKB >= 4 || wave < NKB;   // Dk = 128: every wave owns 32 state rows

    const int G = gridDim.x, bid = blockIdx.x;
    const int logical = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
    const int chain = logical / NV, slice = logical % NV;
    const int b = chain / H, h = chain % H;
    const int dv0 = slice * DVS;

    // ---- initial state --------------------------------------------------
    f32x4 S[2][NTN];
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int n = 0; n < NTN; ++n) {
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
            if (ownS && h0 != nullptr) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int dk = 32 * wave + 8 * grp + 4 * half + i;
                    s[i] = h0[(((size_t)b * H + h) * DK + dk) * DV + dv0 + 16 * n + r16];
                }
            }
            S[half][n] = s;
        }
    auto publish_state = [&]() {
        if (ownS) {
#pragma unroll
            for (int n = 0; n < NTN; ++n)
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    float tmp[4] = {S[half][n][0], S[half][n][1], S[half][n][2], S[half][n][3]};
                    st4(&sS[wave][n][lane][4 * half], tmp);
                }
        }
    };
    publish_state();
    lds_barrier();

    // this launch runs chunks c0 .. c0+nseg-1 of the chain (a segment; the
    // state enters through h0 and leaves through hT)
    const uint8_t* chain_rec = ws + (((size_t)b * H + h) * (size_t)NT + c0) * R::BYTES;
    // output rows are H*DV elements apart; orow0 = column dv0 of token 0
    const size_t ostride = (size_t)H * DV;
    T* const orow0 = o + (((size_t)b * Tlen + (size_t)c0 * C) * H + h) * DV + dv0;
    const int tlim = Tlen - c0 * C;   // valid positions from the segment start
    auto load = [&](InterOps<T, DK, NTN>& op, int c) {
        inter_load<KIND, T, DK, DV, NTN>(op, chain_rec + (size_t)c * R::BYTES, wave, lane, dv0);
    };

    // One chunk step with the operands in `cur` (loaded earlier).
    auto step = [&](int c, const InterOps<T, DK, NTN>& cur, auto guard_tag) {
        constexpr bool GUARD = decltype(guard_tag)::value;
        // entry-state fragments
        Frag<T> fS[NKB][NTN];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int n = 0; n < NTN; ++n) fS[kb][n] = ld_frag(&sS[kb][n][lane][0]);

        f32x4 P[NTN], O[NTN];
#pragma unroll
        for (int n = 0; n < NTN; ++n) {
            P[n] = f32x4{0.f, 0.f, 0.f, 0.f};
            O[n] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int n = 0; n < NTN; ++n) {
                if constexpr (DELTA) mma(P[n], cur.w[kb], fS[kb][n]);
                mma(O[n], cur.qt[kb], fS[kb][n]);
            }
        // Vnew at this lane's 4 positions
#pragma unroll
        for (int n = 0; n < NTN; ++n) {
            float vn[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) vn[i] = DELTA ? cur.u[n][i] - P[n][i] : cur.u[n][i];
            st4(&sV[kbP][n][lane][4 * halfP], vn);
        }
        lds_barrier();

        Frag<T> fV[2][NTN];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int n = 0; n < NTN; ++n) fV[kb][n] = ld_frag(&sV[kb][n][lane][0]);

        // intra-chunk term (Aqk is zero past the diagonal)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int n = 0; n < NTN; ++n) mma(O[n], cur.aqk[kb], fV[kb][n]);
        // store O.  The accumulator gives this lane 4 rows of one column; the
        // tile goes through this wave's own LDS staging area (no other wave
        // touches it, so no barrier) and leaves as 16-byte row segments.
        {
#pragma unroll
            for (int n = 0; n < NTN; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i) sO[wave][4 * grp + i][16 * n + r16] = from_f<T>(O[n][i]);
            constexpr int SEGS = 16 * NTN / 8;          // 8-element segments per row
#pragma unroll
            for (int it = lane; it < 16 * SEGS; it += 64) {
                const int rr = it / SEGS, sg = it % SEGS;
                // staging row rr holds position 32*kbP + prow(halfP, rr)
                const int pos = 32 * kbP + prow(halfP, rr);
                const Frag<T> f = ld_frag(&sO[wave][rr][8 * sg]);
                if (!GUARD || c * C + pos < tlim)
                    st_frag(orow0 + ((size_t)c * C + pos) * ostride + 8 * sg, f);
            }
        }
        // state update: decay first, then accumulate
        if (ownS) {
#pragma unroll
            for (int half = 0; half < 2; ++half)
#pragma unroll
                for (int n = 0; n < NTN; ++n) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) S[half][n][i] *= cur.phi[half][i];
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) mma(S[half][n], cur.kb[half][kb], fV[kb][n]);
                }
        }
        publish_state();
        lds_barrier();
    };

    // Operands are loaded NBUF-1 chunks ahead into a ring of register buffers.  Every load and
    // store inside the steady-state loop is unconditional (prefetch indices are
    // clamped to the last chunk, only the last chunk guards its output rows),
    // so the compiler can keep the prefetches in flight across steps instead of
    // draining the memory counter at control-flow joins.
    using Full = std::integral_constant<bool, false>;
    using Tail = std::integral_constant<bool, true>;
    const int last = nseg - 1;
    auto cl = [&](int c) { return c < last ? c : last; };
    static_assert(NBUF == 2 || NBUF == 3, "prefetch depth");
    if constexpr (NBUF == 3) {
        InterOps<T, DK, NTN> b0, b1, b2;
        int c = 0;
        if (nseg > 0) {
            load(b0, 0);
            load(b1, cl(1));
            for (; c + 3 <= last; c += 3) {
                load(b2, cl(c + 2)); step(c, b0, Full{});
                load(b0, cl(c + 3)); step(c + 1, b1, Full{});
                load(b1, cl(c + 4)); step(c + 2, b2, Full{});
            }
            if (c == last) {
                step(c, b0, Tail{});
            } else if (c + 1 == last) {
                step(c, b0, Full{});
                step(c + 1, b1, Tail{});
            } else {
                load(b2, c + 2);
                step(c, b0, Full{});
                step(c + 1, b1, Full{});
                step(c + 2, b2, Tail{});
            }
        }
    } else {
        InterOps<T, DK, NTN> b0, b1;
        int c = 0;
        if (nseg > 0) {
            load(b0, 0);
            for (; c + 2 <= last; c += 2) {
                load(b1, cl(c + 1)); step(c, b0, Full{});
                load(b0, cl(c + 2)); step(c + 1, b1, Full{});
            }
            if (c == last) {
                step(c, b0, Tail{});
            } else {
                load(b1, c + 1);
                step(c, b0, Full{});
                step(c + 1, b1, Tail{});
            }
        }
    }

    // ---- final state -----------------------------------------------------
    if (ownS && hT != nullptr) {
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int n = 0; n < NTN; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int dk = 32 * wave + 8 * grp + 4 * half + i;
                    hT[(((size_t)b * H + h) * DK + dk) * DV + dv0 + 16 * n + r16] = S[half][n][i];
                }
    }
}

}  // namespace dr
