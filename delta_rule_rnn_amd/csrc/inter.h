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
// columns (value columns evolve independently, [KDA] 3.4).  It has 8 waves:
//   recurrence waves 0..3 compute Vnew for 16 positions each (rows
//     32*(w/2) + prow(w%2, r)) and own 32 key rows of S (rows 32w..32w+31);
//   output waves 4..7 compute O for the same 16 positions of wave w-4.
// The output is off the recurrence's critical path: it only reads the state
// and Vnew that the recurrence waves publish in LDS.  Per chunk there are two
// barriers:
//   phase A (after the previous chunk's second barrier): sS holds the entry
//     state; recurrence waves form Vnew into sV, output waves form Q~ S;
//   barrier 1;
//   phase B: recurrence waves update S and publish it to sS (the output
//     waves finished reading sS before barrier 1); output waves add Aqk Vnew
//     (sV) and store O;
//   barrier 2.
// Each wave prefetches its own operands one chunk ahead into registers, and a
// ninth wave pulls the record lines of later chunks into L2 (PFD below).
//
// The output waves compute O^T = S^T Q~^T + Vnew^T Aqk^T (operands swapped):
// the accumulator then gives each lane 4 consecutive value columns of one
// position, which leave as one 8-byte (bf16) or 16-byte (fp32) store.
//
// Block mapping: the NV = Dv/DVS workgroups of a chain read the same W, Q~,
// Kbar, Aqk; consecutive logical ids are placed on the same XCD (hardware
// dispatches workgroup i to XCD i % 8) so they share that XCD's L2.
#pragma once

#include "common.h"

namespace dr {

constexpr int kInterThreads = 512;   // 4 recurrence + 4 output waves

// A workgroup of a C-token record chunk has NW = C/16 recurrence waves (16
// positions each) and as many output waves.  Recurrence wave w owns the S
// rows of its NH = 128/C 16-row groups g = NH*w + h (rows 32(g/2) +
// prow(g%2, .)), each reduced over the C/32 position blocks of Kbar^T.
template <int C2> struct InterShape {
    static constexpr int NW = C2 / 16, NH = 128 / C2, KQ = C2 / 32;
    static_assert(C2 == 64 || C2 == 128, "record chunk");
};

// Operands of one chunk for a recurrence wave.
template <typename T, int DK, int NTN, int C2 = kChunk>
struct RecurOps {
    static constexpr int NKB = DK / 32;
    using Sh = InterShape<C2>;
    Frag<T> w[NKB];               // W rows of this wave's positions
    Frag<T> kb[Sh::NH][Sh::KQ];   // Kbar^T rows (group, position block) of this wave's S rows
    Raw4<T> u[NTN];               // U (or V) at this lane's 4 positions, per n-tile
    float phi[Sh::NH][4];         // phi at this lane's S rows (group, i)
};

// Operands of one chunk for an output wave.
template <typename T, int DK, int C2 = kChunk>
struct OutOps {
    static constexpr int NKB = DK / 32;
    Frag<T> qt[NKB];                       // Q~ rows of this wave's positions
    Frag<T> aqk[InterShape<C2>::KQ];       // Aqk rows, key blocks
};

// All record blocks are in fragment order: lane l's 8 (or 4) elements are
// contiguous and a wave-wide load is one contiguous run.
template <int KIND, typename T, int DK, int DV, int NTN, int C2 = kChunk>
__device__ __forceinline__ void load_recur(RecurOps<T, DK, NTN, C2>& op, const uint8_t* recb, int wave,
                                           int lane, int dv0)
{
    using R = Rec<T, DK, DV, C2>;
    using Sh = InterShape<C2>;
    constexpr int NKB = DK / 32;
    const T* base = reinterpret_cast<const T*>(recb);
    if constexpr (KIND != KIND_LA) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
            op.w[kb] = ld_frag(base + R::W + ((size_t)(wave * NKB + kb) * 64 + lane) * 8);
    }
    if (Sh::NH * wave < 2 * NKB) {
        const float* phi = reinterpret_cast<const float*>(recb + R::PHI_BYTE);
        const int grp = lane >> 4;
#pragma unroll
        for (int hh = 0; hh < Sh::NH; ++hh) {
            const int g = Sh::NH * wave + hh;
#pragma unroll
            for (int kb = 0; kb < Sh::KQ; ++kb)
                op.kb[hh][kb] = ld_frag(base + R::KBT + ((size_t)(g * Sh::KQ + kb) * 64 + lane) * 8);
            ld4(phi + 32 * (g >> 1) + 8 * grp + 4 * (g & 1), op.phi[hh]);
        }
    }
#pragma unroll
    for (int n = 0; n < NTN; ++n)
        op.u[n].load(base + R::UT + ((size_t)((dv0 / 16 + n) * Sh::NW + wave) * 64 + lane) * 4);
}

template <typename T, int DK, int DV, int C2 = kChunk>
__device__ __forceinline__ void load_out(OutOps<T, DK, C2>& op, const uint8_t* recb, int wave, int lane)
{
    using R = Rec<T, DK, DV, C2>;
    constexpr int KQ = InterShape<C2>::KQ;
    constexpr int NKB = DK / 32;
    const T* base = reinterpret_cast<const T*>(recb);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
        op.qt[kb] = ld_frag(base + R::QT + ((size_t)(wave * NKB + kb) * 64 + lane) * 8);
    // every key block: the record holds zeros above the diagonal, so the
    // blocks past this wave's positions contribute nothing
#pragma unroll
    for (int kb = 0; kb < KQ; ++kb) op.aqk[kb] = ld_frag(base + R::AQK + ((size_t)(wave * KQ + kb) * 64 + lane) * 8);
}

// Asynchronous copy global -> LDS of BYTES bytes per lane from the lane's own
// address; lane l's bytes land at lds + l*BYTES (lds is the same for every
// lane).
template <int BYTES>
__device__ __forceinline__ void copy_to_lds_lane(const uint8_t* gsrc_lane, uint8_t* lds) {
    static_assert(BYTES == 4 || BYTES == 16, "copy width");
    const auto src = (const __attribute__((address_space(1))) void*)gsrc_lane;
    const auto dst = (__attribute__((address_space(3))) void*)lds;
    if constexpr (BYTES == 16) __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
    else __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
}

// Wait until this wave has no outstanding vector memory operation (the
// copies above count there until their data is in LDS).
__device__ __forceinline__ void wait_vm_all() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Body of the L2 prefetch wave: for every chunk step c of the workgroup
// (two barriers each, after the one that publishes the initial state), touch
// this workgroup's share of the record lines of chunk c+PFD: one 4-byte copy
// per 128-byte line into a scratch LDS word.  Lines are split between the NV
// workgroups of a chain, which share one XCD's L2.  The wave never reads the
// copies; it drains them before it ends.
template <typename T, int DK, int DV, int NV, int PFD>
__device__ __forceinline__ void l2_prefetch_wave(const uint8_t* chain_rec, int nseg, int slice, int lane,
                                                 uint8_t* sink)
{
    using R = Rec<T, DK, DV>;
    constexpr int LINES = (int)(R::BYTES / 128);
    constexpr int PER = (LINES + NV - 1) / NV;          // lines of this workgroup
    lds_barrier();   // initial state published
    for (int c = 0; c < nseg; ++c) {
        const int cp = c + PFD;
        if (cp < nseg) {
            const uint8_t* rec = chain_rec + (size_t)cp * R::BYTES;
#pragma unroll
            for (int i = 0; i < (PER + 63) / 64; ++i) {
                const int line = (i * 64 + lane) * NV + slice;
                if (i * 64 + lane < PER && line < LINES) copy_to_lds_lane<4>(rec + (size_t)line * 128, sink);
            }
        }
        lds_barrier();
        lds_barrier();
    }
    wait_vm_all();
}

// With PFD > 0 a ninth wave touches this workgroup's share of the record
// lines of chunk c+PFD while the others work on chunk c: one 4-byte copy per
// 128-byte line into a scratch LDS word, so the lines are in L2 by the time
// the compute waves load them.  The NV workgroups of a chain share the
// chain's L2 (same XCD) and split the lines between them.
template <int PFD, int C2 = kChunk>
constexpr int inter_threads() { return 2 * 64 * InterShape<C2>::NW + (PFD > 0 ? 64 : 0); }

// VARLEN: chains are (sequence, head) of packed sequences; seqinfo[i] =
// {first record slot, chunks, first token, tokens} of sequence i (written by
// varlen_table_kernel) replaces the dense layout's (Tlen, NT, c0, nseg).
//
// STATES (the backward's forward state pass): instead of o, write for every
// chunk its entry state S_c ([DK][DV] at states + r*DK*DV) and Vnew_c
// ([C][DV] at vnew + r*C*DV), both in the I/O type (rounded from the fp32
// accumulators) and slice-major (slc(), common.h), r the chunk's record
// index; the output
// waves only keep the barriers.  Rows of a ragged last chunk past the end
// get Vnew = 0 (their record rows are zero).
//
// C2 = 128 (sub-chunked 128-token records): 8 recurrence and 8 output waves,
// one 16-row group of S per recurrence wave; dense layout, no prefetch wave.
template <int KIND, typename T, int DK, int DV, int NTN, int PFD, bool VARLEN, bool STATES = false,
          int C2 = kChunk>
__global__ __launch_bounds__((inter_threads<PFD, C2>())) void inter_kernel(const uint8_t* __restrict__ ws,
                                                              const float* __restrict__ h0,
                                                              T* __restrict__ o, float* __restrict__ hT,
                                                              int Tlen, int H, int NT, int c0,
                                                              int nseg_arg,
                                                              const int4* __restrict__ seqinfo,
                                                              int maxchunks,
                                                              T* __restrict__ states = nullptr,
                                                              T* __restrict__ vnew = nullptr)
{
    using R = Rec<T, DK, DV, C2>;
    using Sh = InterShape<C2>;
    constexpr int C = C2;
    constexpr int NW = Sh::NW, NH = Sh::NH, KQ = Sh::KQ;
    constexpr int DVS = 16 * NTN;
    constexpr int NV = DV / DVS;
    constexpr int NKB = DK / 32;
    constexpr bool DELTA = KIND != KIND_LA;
    static_assert(DV % DVS == 0, "value split");
    static_assert(C2 == kChunk || (PFD == 0 && !VARLEN && !STATES), "128-token records: dense forward only");

    // B-fragment exchange buffers: [block][n-tile][lane][8 slots]
    __shared__ __attribute__((aligned(16))) T sS[NKB][NTN][64][8];
    __shared__ __attribute__((aligned(16))) T sV[KQ][NTN][64][8];

    const int tid = threadIdx.x, lane = tid & 63;
    const bool recur = tid < 64 * NW;            // waves 0..NW-1
    const int wave = (tid >> 6) & (NW - 1);      // position group of either role
    __shared__ __attribute__((aligned(16))) uint8_t sink[PFD > 0 ? 256 : 16];
    const int r16 = lane & 15, grp = lane >> 4;
    const int kbP = wave >> 1, halfP = wave & 1;
    const bool ownS = recur && NH * wave < 2 * NKB;   // Dk = 128: every recurrence wave

    const int G = gridDim.x, bid = blockIdx.x;
    const int logical = xcd_logical(bid, G);
    const int chain = logical / NV, slice = logical % NV;
    // packed sequences take chains head-major (chain = h * N + sequence), so
    // that each XCD's contiguous range of logical ids holds every sequence
    // for a few heads and the XCDs get equal token counts whatever the
    // lengths; the dense layout is (b, h) as stored
    const int nseq = G / (NV * H);
    const int b = VARLEN ? chain % nseq : chain / H, h = VARLEN ? chain / nseq : chain % H;
    const int dv0 = slice * DVS;

    // this launch runs nseg chunks of the chain from its record chain_rec on,
    // covering tokens tok0 .. tok0+tlim-1; the state enters through h0 and
    // leaves through hT
    int nseg, tlim;
    size_t tok0, rec0;     // rec0: record index of the launch's first chunk
    if constexpr (VARLEN) {
        const int4 si = seqinfo[b];   // b is the sequence here
        nseg = si.y;
        tok0 = (size_t)si.z;
        tlim = si.w;
        rec0 = (size_t)h * maxchunks + si.x;
    } else {
        nseg = nseg_arg;
        tok0 = (size_t)b * Tlen + (size_t)c0 * C;
        tlim = Tlen - c0 * C;
        rec0 = ((size_t)b * H + h) * (size_t)NT + c0;
    }
    const uint8_t* chain_rec = ws + rec0 * R::BYTES;

    auto fS_read = [&](Frag<T> (&fS)[NKB][NTN]) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int n = 0; n < NTN; ++n) fS[kb][n] = ld_frag(&sS[kb][n][lane][0]);
    };
    auto fV_read = [&](Frag<T> (&fV)[KQ][NTN]) {
#pragma unroll
        for (int kb = 0; kb < KQ; ++kb)
#pragma unroll
            for (int n = 0; n < NTN; ++n) fV[kb][n] = ld_frag(&sV[kb][n][lane][0]);
    };

    if constexpr (PFD > 0) {
        if (tid >= 2 * 64 * NW) {
            l2_prefetch_wave<T, DK, DV, NV, PFD>(chain_rec, nseg, slice, lane, sink);
            return;
        }
    }
    if (recur) {
        // ---- recurrence waves ---------------------------------------------
        // S rows of group g = NH*wave + half: 32(g/2) + 8(l/16) + 4(g%2) + i
        auto srow = [&](int half, int i) {
            const int g = NH * wave + half;
            return 32 * (g >> 1) + 8 * grp + 4 * (g & 1) + i;
        };
        f32x4 S[NH][NTN];
#pragma unroll
        for (int half = 0; half < NH; ++half)
#pragma unroll
            for (int n = 0; n < NTN; ++n) {
                f32x4 s = {0.f, 0.f, 0.f, 0.f};
                if (ownS && h0 != nullptr) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int dk = srow(half, i);
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
                    for (int half = 0; half < NH; ++half) {
                        const int g = NH * wave + half;
                        float tmp[4] = {S[half][n][0], S[half][n][1], S[half][n][2], S[half][n][3]};
                        st4(&sS[g >> 1][n][lane][4 * (g & 1)], tmp);
                    }
            }
        };
        publish_state();
        lds_barrier();

        using Ops = RecurOps<T, DK, NTN, C2>;
        auto load = [&](Ops& op, int c) {
            load_recur<KIND, T, DK, DV, NTN, C2>(op, chain_rec + (size_t)c * R::BYTES, wave, lane, dv0);
        };
        auto step = [&](int c, const Ops& cur, auto) {
            if constexpr (STATES) {
                // the chunk's entry state, as the final state is written
                if (ownS) {
                    T* sc = states + (rec0 + c) * (size_t)DK * DV;
#pragma unroll
                    for (int half = 0; half < NH; ++half)
#pragma unroll
                        for (int n = 0; n < NTN; ++n)
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                sc[slc(srow(half, i), dv0 + 16 * n + r16, DK)] = from_f<T>(S[half][n][i]);
                }
            }
            // phase A: Vnew at this lane's 4 positions
            f32x4 P[NTN];
#pragma unroll
            for (int n = 0; n < NTN; ++n) P[n] = f32x4{0.f, 0.f, 0.f, 0.f};
            if constexpr (DELTA) {
                Frag<T> fS[NKB][NTN];
                fS_read(fS);
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int n = 0; n < NTN; ++n) mma(P[n], cur.w[kb], fS[kb][n]);
            }
#pragma unroll
            for (int n = 0; n < NTN; ++n) {
                float vn[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) vn[i] = cur.u[n][i] - P[n][i];
                st4(&sV[kbP][n][lane][4 * halfP], vn);
                if constexpr (STATES) {
                    // positions 32(w/2) + 8(l/16) + 4(w%2) + i, the layout of U
                    T* vc = vnew + (rec0 + c) * (size_t)C * DV;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        vc[slc(32 * kbP + 8 * grp + 4 * halfP + i, dv0 + 16 * n + r16, C)] = from_f<T>(vn[i]);
                }
            }
            lds_barrier();
            // phase B: state update, decay first, then accumulate
            Frag<T> fV[KQ][NTN];
            fV_read(fV);
            if (ownS) {
#pragma unroll
                for (int half = 0; half < NH; ++half)
#pragma unroll
                    for (int n = 0; n < NTN; ++n) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) S[half][n][i] *= cur.phi[half][i];
#pragma unroll
                        for (int kb = 0; kb < KQ; ++kb) mma(S[half][n], cur.kb[half][kb], fV[kb][n]);
                    }
            }
            publish_state();
            lds_barrier();
        };
        prefetch_pair<Ops>(nseg, load, step);

        // ---- final state ---------------------------------------------------
        if (ownS && hT != nullptr) {
#pragma unroll
            for (int half = 0; half < NH; ++half)
#pragma unroll
                for (int n = 0; n < NTN; ++n)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int dk = srow(half, i);
                        hT[(((size_t)b * H + h) * DK + dk) * DV + dv0 + 16 * n + r16] = S[half][n][i];
                    }
        }
    } else if constexpr (STATES) {
        // no output: keep the recurrence waves' barriers (initial state, then
        // two per chunk)
        lds_barrier();
        for (int c = 0; c < nseg; ++c) {
            lds_barrier();
            lds_barrier();
        }
    } else {
        // ---- output waves ---------------------------------------------------
        lds_barrier();   // initial state published
        // this lane's output row: position pw(wave, r16), columns 4*grp.. of each n-tile
        const int pos = 32 * kbP + prow(halfP, r16);
        const size_t ostride = (size_t)H * DV;
        T* const orow = o + ((tok0 + pos) * H + h) * DV + dv0 + 4 * grp;

        using Ops = OutOps<T, DK, C2>;
        auto load = [&](Ops& op, int c) {
            load_out<T, DK, DV, C2>(op, chain_rec + (size_t)c * R::BYTES, wave, lane);
        };
        auto step = [&](int c, const Ops& cur, auto guard_tag) {
            constexpr bool GUARD = decltype(guard_tag)::value;
            // phase A: O^T = S^T Q~^T with the entry state
            f32x4 Ot[NTN];
#pragma unroll
            for (int n = 0; n < NTN; ++n) Ot[n] = f32x4{0.f, 0.f, 0.f, 0.f};
            {
                Frag<T> fS[NKB][NTN];
                fS_read(fS);
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int n = 0; n < NTN; ++n) mma(Ot[n], fS[kb][n], cur.qt[kb]);
            }
            lds_barrier();
            // phase B: intra-chunk term (Aqk is zero past the diagonal), store
            Frag<T> fV[KQ][NTN];
            fV_read(fV);
#pragma unroll
            for (int kb = 0; kb < KQ; ++kb)
#pragma unroll
                for (int n = 0; n < NTN; ++n) mma(Ot[n], fV[kb][n], cur.aqk[kb]);
            if (!GUARD || c * C + pos < tlim) {
#pragma unroll
                for (int n = 0; n < NTN; ++n) {
                    const float v4[4] = {Ot[n][0], Ot[n][1], Ot[n][2], Ot[n][3]};
                    st4(orow + (size_t)c * C * ostride + 16 * n, v4);
                }
            }
            lds_barrier();
        };
        prefetch_pair<Ops>(nseg, load, step);
    }
}

}  // namespace dr
