// seg.h -- the segment-parallel forward: three kernels that together compute
// the whole chunkwise forward (steps a1-a5) without writing per-chunk
// operand records to HBM.
//
// Page keys: [KDA] "TileLang 实战：KDA 从零到一–Kimi Delta Attention";
// [SD] "TileLang 实战：KDA 从零到一--标量衰减"; [GDN] "Gated DeltaNet";
// [DPLR] "RNN的复兴04:线性注意力并行计算DPLR".
//
// The chunks of each (batch, head) chain are grouped into NS segments of L
// consecutive chunks.  Every segment is evaluated independently from the
// augmented entry state X = [P | S] = [I | 0] ([Dk, Dk + Dv]): P is the
// transition from the segment's start (the product of the per-token maps
// S -> (I - beta k k^T) Diag(a) S, whose WY form is [DPLR] section 2), S the
// state reached from a zero entry state.  Per chunk, with U_bar = [0 | U]:
//   Y = U_bar - W X              (the chunk's pseudo values, [KDA] 3.2)
//   Z = Q~ X + Aqk Y             (entry-state read + intra-chunk term)
//   X <- Diag(phi) X + Kbar^T Y  (decay first, then the write, [SD] 5.2)
// Z's P columns are the chunk's effective queries q_eff, its S columns the
// chunk's output from a zero segment entry state.  With the entry states
// S_in[0] = h0, S_in[r+1] = M_r S_in[r] + N_r (X = [M_r | N_r] at the
// segment's end), the output is o = o_local + q_eff S_in[r].  This is the
// entry-state hand-off of the sequence-split (context-parallel) forward on
// [GDN] "前向计算的矩阵分解", applied inside one GPU.
//
// Kernels:
//   seg_kernel      one 512-thread workgroup per (b, h, segment): for each
//                   chunk in order, steps a1-a3 into LDS (as the chunk-
//                   parallel kernel computes them), then the state step above
//                   on MFMA with X in registers; o_local goes to o, q_eff to
//                   the workspace, [M | N] to the workspace at the end.
//   compose_kernel  per (chain, 16 value columns): the short sequential
//                   composition of the segment entry states; writes S_in^T
//                   (I/O dtype) per segment and the final state hT.
//   correct_kernel  chunk-parallel: o += q_eff S_in[segment] for every chunk
//                   of the segments after the first (the first segment
//                   starts from the true initial state).
#pragma once

#include "common.h"
#include "intra.h"

namespace dr {

constexpr int kSegThreads = 512;            // 8 waves, one workgroup per CU
constexpr int kSegTargetGroups = 256;       // segments are sized to give about this many workgroups

// LDS plan of seg_kernel (bytes).  Regions are reused across phases:
//   KP  K+ [C][LDK]                         P1 -> P4
//   KM  K- [C][LDK] (P1 -> P2), then U^T [DV][LDC] (P4 -> P5)
//   QP  Q~ [C][LDK]                         P1 -> P5
//   A   A fp32 [C][LDF] (P2 -> P3), then W [C][LDK] (P4 -> P5)
//   TT  per-group gate totals (P1), then T fp32 [C][LDF] (P3 -> P4)
//   VT  V^T [DV][LDC]                       P1 -> P4 (decay_la: -> P5)
//   KBT Kbar^T [DK][LDC]                    P1 -> P5
//   AQK Aqk [C][LDC]                        P2 -> P5
//   beta [C], gamma [C] (scalar gates), phi [DK] floats
template <int KIND, typename T, int DK, int DV>
struct SegCfg {
    static constexpr int C = kChunk;
    static constexpr int LDK = DK + 8;
    static constexpr int LDF = C + 4;
    static constexpr int LDC = C + 8;
    static constexpr int CPT = DK / 32;                  // channels per thread (elementwise steps)
    static constexpr int NCG = DK / CPT;                 // channel groups (32)
    static constexpr int NQ = kSegThreads / NCG;         // position groups (16)
    static constexpr int PL = C / NQ;                    // positions per thread (4)
    static constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
    static constexpr size_t SZ_CK = (size_t)C * LDK * sizeof(T);
    static constexpr size_t SZ_TC = (size_t)DK * LDC * sizeof(T);
    static constexpr size_t SZ_F = (size_t)C * LDF * sizeof(float);
    static constexpr size_t up16(size_t x) { return (x + 15) / 16 * 16; }
    static constexpr size_t R_KP = 0;
    static constexpr size_t R_KM = R_KP + up16(SZ_CK);
    static constexpr size_t R_QP = R_KM + up16(mx(SZ_CK, SZ_TC));
    static constexpr size_t R_A = R_QP + up16(SZ_CK);
    static constexpr size_t R_TT = R_A + up16(mx(SZ_F, SZ_CK));
    static constexpr size_t R_VT = R_TT + up16(mx(SZ_F, (size_t)NQ * DK * sizeof(float)));
    static constexpr size_t R_KBT = R_VT + up16(SZ_TC);
    static constexpr size_t R_AQK = R_KBT + up16(SZ_TC);
    static constexpr size_t R_BETA = R_AQK + up16((size_t)C * LDC * sizeof(T));
    static constexpr size_t R_GAM = R_BETA + C * sizeof(float);
    static constexpr size_t R_PHI = R_GAM + C * sizeof(float);
    static constexpr size_t BYTES = R_PHI + DK * sizeof(float);
    // state step: X columns per wave and 16-wide tiles per wave
    static constexpr int NCW = (DK + DV) / 8;
    static constexpr int NTW = NCW / 16;
    static_assert(DK == DV && (DK == 64 || DK == 128), "head size");
    static_assert(NQ * PL == C && PL == 4, "thread layout");
    static_assert(BYTES <= 160 * 1024, "LDS");
};

// Inputs of one chunk as a thread holds them (channels CPT*cg.., positions
// PL*qg..), loaded one chunk ahead.  Rows past the end of a ragged last chunk
// are loaded from the last valid row (every load unconditional) and zeroed
// where used.
template <int KIND, typename T, int DK, int DV>
struct SegIn {
    using Cfg = SegCfg<KIND, T, DK, DV>;
    using VT = typename VecOf<T, Cfg::CPT>::type;
    using VG = typename VecOf<float, Cfg::CPT>::type;
    VT kv[Cfg::PL], qv[Cfg::PL], vv[Cfg::PL];
    VG gv[KIND == KIND_KDA ? Cfg::PL : 1];
    float bt, gs;
};

template <int KIND, typename T, int DK, int DV>
__device__ __forceinline__ void seg_load(SegIn<KIND, T, DK, DV>& in, const T* __restrict__ q,
                                         const T* __restrict__ k, const T* __restrict__ v,
                                         const float* __restrict__ g, const float* __restrict__ beta,
                                         size_t row0, int nvalid, int H)
{
    using Cfg = SegCfg<KIND, T, DK, DV>;
    using In = SegIn<KIND, T, DK, DV>;
    using VT = typename In::VT;
    using VG = typename In::VG;
    constexpr int NCG = Cfg::NCG, PL = Cfg::PL, CPT = Cfg::CPT;
    const int tid = threadIdx.x, lane = tid & 63;
    const int last = nvalid - 1;
    const int ch0 = CPT * (tid % NCG), p0 = (tid / NCG) * PL;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        const size_t off = (row0 + (size_t)min(p0 + i, last) * H) * DK + ch0;
        if constexpr (KIND == KIND_KDA) in.gv[i] = ld_stream(reinterpret_cast<const VG*>(g + off));
        in.kv[i] = ld_stream(reinterpret_cast<const VT*>(k + off));
        in.qv[i] = ld_stream(reinterpret_cast<const VT*>(q + off));
    }
    if constexpr (KIND != KIND_KDA) in.gs = (tid < 64) ? ld_stream(g + row0 + (size_t)min(lane, last) * H) : 0.f;
    if constexpr (KIND != KIND_LA) in.bt = (tid < kChunk) ? ld_stream(beta + row0 + (size_t)min(tid, last) * H) : 0.f;
#pragma unroll
    for (int i = 0; i < PL; ++i)
        in.vv[i] = ld_stream(reinterpret_cast<const VT*>(v + (row0 + (size_t)min(p0 + i, last) * H) * DV + ch0));
}

// Pack two accumulator tiles (rows 8q..8q+3 and 8q+4..8q+7 of a 32-row block)
// into one natural B fragment of the I/O type.
template <typename T>
__device__ __forceinline__ Frag<T> pack_frag(const f32x4& lo, const f32x4& hi) {
    Frag<T> f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        frag_set(f, i, lo[i]);
        frag_set(f, 4 + i, hi[i]);
    }
    return f;
}

// ---------------------------------------------------------------------------
// Steps a1-a3 of one chunk into LDS (P0-P4).  On return (after a barrier)
// LDS holds Q~ (QP), W (A; delta kinds), U^T (KM; decay_la: V^T in VT), Kbar^T
// (KBT), Aqk (AQK) and phi (PHI) of the chunk.
template <int KIND, typename T, int DK, int DV, bool PRO>
__device__ __forceinline__ void seg_chunk_ops(const SegIn<KIND, T, DK, DV>& in, uint8_t* smem,
                                              unsigned* __restrict__ flags, int nvalid, const ProHead& ph)
{
    using Cfg = SegCfg<KIND, T, DK, DV>;
    constexpr int C = kChunk;
    constexpr bool DELTA = KIND != KIND_LA;
    constexpr bool PERCH = KIND == KIND_KDA;
    constexpr int LDK = Cfg::LDK, LDF = Cfg::LDF, LDC = Cfg::LDC;
    constexpr int NCG = Cfg::NCG, PL = Cfg::PL, NQ = Cfg::NQ, CPT = Cfg::CPT;
    constexpr int NKB = DK / 32;
    using In = SegIn<KIND, T, DK, DV>;
    using VT = typename In::VT;
    using VG = typename In::VG;

    T* sKp = reinterpret_cast<T*>(smem + Cfg::R_KP);
    T* sKm = reinterpret_cast<T*>(smem + Cfg::R_KM);
    T* sUt = reinterpret_cast<T*>(smem + Cfg::R_KM);
    T* sQp = reinterpret_cast<T*>(smem + Cfg::R_QP);
    float* sA = reinterpret_cast<float*>(smem + Cfg::R_A);
    T* sW = reinterpret_cast<T*>(smem + Cfg::R_A);
    float* sTot = reinterpret_cast<float*>(smem + Cfg::R_TT);
    float* sT = reinterpret_cast<float*>(smem + Cfg::R_TT);
    T* sVt = reinterpret_cast<T*>(smem + Cfg::R_VT);
    T* sKbT = reinterpret_cast<T*>(smem + Cfg::R_KBT);
    T* sAqk = reinterpret_cast<T*>(smem + Cfg::R_AQK);
    float* sBeta = reinterpret_cast<float*>(smem + Cfg::R_BETA);
    float* sGam = reinterpret_cast<float*>(smem + Cfg::R_GAM);
    float* sPhi = reinterpret_cast<float*>(smem + Cfg::R_PHI);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, grp = lane >> 4;

    // ---- P0: inputs, rows past the end of a ragged chunk zeroed ------------
    const int cg = tid % NCG, qg = tid / NCG, ch0 = CPT * cg, p0 = qg * PL;
    VT kv[PL], qv[PL], vv[PL];
    VG gv[PERCH ? PL : 1];
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        const bool ok = p0 + i < nvalid;
        kv[i] = ok ? in.kv[i] : VT{};
        qv[i] = ok ? in.qv[i] : VT{};
        vv[i] = ok ? in.vv[i] : VT{};
        if constexpr (PERCH) gv[i] = ok ? in.gv[i] : VG{};
    }
    if (tid < C) sBeta[tid] = (DELTA && tid < nvalid) ? (PRO ? pro_beta(ph, in.bt) : in.bt) : 0.f;
    // prologue: per-row factors of k and q (a row's DK channels sit in the 32
    // adjacent lanes of one half wave)
    float nk[PL], nq[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) nk[i] = nq[i] = 1.f;
    if constexpr (PRO) {
        if (ph.ops & PRO_QK_L2NORM) {
#pragma unroll
            for (int i = 0; i < PL; ++i) {
                float sk = 0.f, sq = 0.f;
#pragma unroll
                for (int j = 0; j < CPT; ++j) {
                    const float kk = (float)kv[i][j], qq = (float)qv[i][j];
                    sk += kk * kk;
                    sq += qq * qq;
                }
                sk = lane_group_sum<NCG>(sk);
                sq = lane_group_sum<NCG>(sq);
                nk[i] = 1.f / sqrtf(sk + kNormEps);
                nq[i] = 1.f / sqrtf(sq + kNormEps);
            }
        }
#pragma unroll
        for (int i = 0; i < PL; ++i) nq[i] *= ph.scale;
    }

    // ---- P1: a1 (gamma) + a2 (prep), V^T --------------------------------
    float gam[PL][CPT];
    float glast[CPT];
    if constexpr (PERCH) {
        float sc[CPT];
#pragma unroll
        for (int j = 0; j < CPT; ++j) sc[j] = 0.f;
#pragma unroll
        for (int i = 0; i < PL; ++i)
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                sc[j] += gv[i][j];
                gam[i][j] = sc[j];
            }
        {
            VG tot;
#pragma unroll
            for (int j = 0; j < CPT; ++j) tot[j] = sc[j];
            *reinterpret_cast<VG*>(sTot + qg * DK + ch0) = tot;
        }
        lds_barrier();
        float pre[CPT], all[CPT];
#pragma unroll
        for (int j = 0; j < CPT; ++j) pre[j] = all[j] = 0.f;
#pragma unroll
        for (int jq = 0; jq < NQ; ++jq) {
            const VG a = *reinterpret_cast<const VG*>(sTot + jq * DK + ch0);
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                if (jq < qg) pre[j] += a[j];
                all[j] += a[j];
            }
        }
#pragma unroll
        for (int j = 0; j < CPT; ++j) glast[j] = all[j] * kLog2e;
#pragma unroll
        for (int i = 0; i < PL; ++i)
#pragma unroll
            for (int j = 0; j < CPT; ++j) gam[i][j] = (pre[j] + gam[i][j]) * kLog2e;
    } else {
        if (wave == 0) {
            float x = (lane < nvalid) ? (PRO ? pro_gate(ph, in.gs) : in.gs) : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off, 64);
                if (lane >= off) x += y;
            }
            sGam[lane] = x * kLog2e;
        }
        lds_barrier();
#pragma unroll
        for (int i = 0; i < PL; ++i)
#pragma unroll
            for (int j = 0; j < CPT; ++j) gam[i][j] = sGam[p0 + i];
#pragma unroll
        for (int j = 0; j < CPT; ++j) glast[j] = sGam[C - 1];
    }
    {
        float phi[CPT];
#pragma unroll
        for (int j = 0; j < CPT; ++j) phi[j] = __builtin_amdgcn_exp2f(glast[j]);
        float kb[CPT][PL];
        float mxneg = 0.f;
#pragma unroll
        for (int i = 0; i < PL; ++i) {
            const int p = p0 + i;
            if constexpr (PERCH) {
                VT kp, km, qp;
#pragma unroll
                for (int j = 0; j < CPT; ++j) {
                    const float kk = (float)kv[i][j] * nk[i], qq = (float)qv[i][j] * nq[i];
                    const float e = __builtin_amdgcn_exp2f(gam[i][j]);
                    const float ei = __builtin_amdgcn_exp2f(-gam[i][j]);
                    mxneg = fmaxf(mxneg, -gam[i][j]);
                    kp[j] = from_f<T>(kk * e);
                    km[j] = from_f<T>(kk * ei);
                    qp[j] = from_f<T>(qq * e);
                    kb[j][i] = kk * (ei * phi[j]);
                }
                *reinterpret_cast<VT*>(sKp + p * LDK + ch0) = kp;
                *reinterpret_cast<VT*>(sKm + p * LDK + ch0) = km;
                *reinterpret_cast<VT*>(sQp + p * LDK + ch0) = qp;
            } else {
                // scalar gates: raw (normalised) k and q; the ratios
                // 2^(gamma_r - gamma_i) are applied where i <= r ([SD] 2.2)
                VT kn = kv[i], qn = qv[i];
                if constexpr (PRO) {
#pragma unroll
                    for (int j = 0; j < CPT; ++j) {
                        kn[j] = from_f<T>((float)kv[i][j] * nk[i]);
                        qn[j] = from_f<T>((float)qv[i][j] * nq[i]);
                    }
                }
                *reinterpret_cast<VT*>(sKp + p * LDK + ch0) = kn;
                *reinterpret_cast<VT*>(sQp + p * LDK + ch0) = qn;
                const float r = __builtin_amdgcn_exp2f(glast[0] - gam[i][0]) * nk[i];
#pragma unroll
                for (int j = 0; j < CPT; ++j) kb[j][i] = (float)kv[i][j] * r;
            }
        }
        // Kbar^T and V^T: PL consecutive positions of one channel per store
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            st4(sKbT + (ch0 + j) * LDC + p0, kb[j]);
            float vt[PL];
#pragma unroll
            for (int i = 0; i < PL; ++i) vt[i] = (float)vv[i][j];
            st4(sVt + (ch0 + j) * LDC + p0, vt);
        }
        if (qg == 0) {
#pragma unroll
            for (int j = 0; j < CPT; ++j) sPhi[ch0 + j] = phi[j];
        }
        if constexpr (PERCH) {
            if (flags) {
                const unsigned long long b16 = __ballot(mxneg >= 16.f);
                const unsigned long long b126 = __ballot(mxneg >= 126.f);
                if (lane == 0 && (b16 | b126)) atomicOr(flags, (b16 ? 1u : 0u) | (b126 ? 2u : 0u));
            }
        }
    }
    lds_barrier();

    // ---- P2: A (fp32, natural) and Aqk (natural, inclusive diagonal) -------
    {
        const T* kminus = PERCH ? sKm : sKp;
        constexpr int NA = DELTA ? 10 : 0;
        // items: NA lower tiles of A, 10 lower tiles of Aqk, and the two
        // upper tiles (0,1), (2,3) of Aqk that the state step's 32-wide key
        // blocks read (zero)
        for (int idx = wave; idx < NA + 12; idx += kSegThreads / 64) {
            if (idx >= NA + 10) {
                const int ti = idx == NA + 10 ? 0 : 2;
                T* dst = sAqk + (16 * ti) * LDC + 16 * (ti + 1);
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[(4 * grp + i) * LDC + r16] = from_f<T>(0.f);
                continue;
            }
            const bool isA = idx < NA;
            int ti, tj;
            lower_tile(isA ? idx : idx - NA, ti, tj);
            const T* arows = isA ? sKp : sQp;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const Frag<T> fa = ld_frag(arows + (16 * ti + r16) * LDK + 32 * kb + 8 * grp);
                const Frag<T> fb = ld_frag(kminus + (16 * tj + r16) * LDK + 32 * kb + 8 * grp);
                mma(acc, fa, fb);
            }
            const int col = 16 * tj + r16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * ti + 4 * grp + i;
                float ratio = 1.f;
                if constexpr (!PERCH) ratio = (col <= row) ? __builtin_amdgcn_exp2f(sGam[row] - sGam[col]) : 0.f;
                if (isA) sA[row * LDF + col] = (col < row) ? sBeta[row] * ratio * acc[i] : 0.f;
                else sAqk[row * LDC + col] = from_f<T>((col <= row) ? ratio * acc[i] : 0.f);
            }
        }
    }
    lds_barrier();
    if constexpr (!PERCH) {
        // scalar gates: Q~ = q 2^gamma in place (every reader of raw q is done)
#pragma unroll
        for (int i = 0; i < PL; ++i) {
            const int p = p0 + i;
            const float sc = __builtin_amdgcn_exp2f(sGam[p]);
            VT x = *reinterpret_cast<const VT*>(sQp + p * LDK + ch0);
#pragma unroll
            for (int j = 0; j < CPT; ++j) x[j] = from_f<T>((float)x[j] * sc);
            *reinterpret_cast<VT*>(sQp + p * LDK + ch0) = x;
        }
    }
    if constexpr (!DELTA) {
        lds_barrier();
        return;
    }

    // ---- P3: T = (I + A)^-1 ([GDN] "对角子块前代" and "合并相邻子块") ---------
    if (wave == 0) {
        const int blk = lane >> 4, col = lane & 15;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float* arow = sA + (16 * blk + r) * LDF + 16 * blk;
            float acc = (r == col) ? 1.f : 0.f;
#pragma unroll
            for (int j = 0; j < r; ++j) acc -= arow[j] * x[j];
            x[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sT[(16 * blk + r) * LDF + 16 * blk + col] = x[r];
        if ((blk & 1) == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sT[(16 * blk + r) * LDF + 16 * (blk + 1) + col] = 0.f;
        }
    }
    lds_barrier();
#pragma unroll
    for (int dist = 1; dist <= 3; ++dist) {
        if (wave < 4 - dist) {
            const int i = wave + dist, j = wave;
            f32x4 y = {0.f, 0.f, 0.f, 0.f};
            for (int m = j; m < i; ++m)
                y = mm16_lds(sA + 16 * i * LDF + 16 * m, LDF, sT + 16 * m * LDF + 16 * j, LDF, lane, y);
            const f32x4 z = mm16_acc(sT + 16 * i * LDF + 16 * i, LDF, y, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) sT[(16 * i + 4 * grp + e) * LDF + 16 * j + r16] = -z[e];
        }
        lds_barrier();
    }

    // ---- P4: [W | U] = T diag(beta) [K+ | V] ---------------------------------
    // (scalar gates: W = T diag(beta 2^gamma) K).  n-tiles of 16 columns:
    // waves 0-3 take W's, waves 4-7 U's.
    {
        constexpr int NTWt = DK / 16, NTUt = DV / 16;
        constexpr int PER = (NTWt + NTUt) / 8;
        static_assert(PER >= 1 && NTWt == 4 * PER, "n-tile split");
        const bool isW = wave < 4;
        const int nt0 = (wave & 3) * PER;
        Frag<T> fb[PER][2];
#pragma unroll
        for (int n = 0; n < PER; ++n) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (isW) {
                    const int col = 16 * (nt0 + n) + r16;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int p = 32 * kb + 8 * grp + j;
                        float s = to_f(sKp[p * LDK + col]);
                        if constexpr (!PERCH) s *= __builtin_amdgcn_exp2f(sGam[p]);
                        frag_set(fb[n][kb], j, s);
                    }
                } else {
                    fb[n][kb] = ld_frag(sVt + (16 * (nt0 + n) + r16) * LDC + 32 * kb + 8 * grp);
                }
            }
        }
        f32x4 acc[4][PER];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int n = 0; n < PER; ++n) acc[mt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (kb == 1 && mt < 2) continue;   // T is lower triangular
                Frag<T> fa;
                const float* src = sT + (16 * mt + r16) * LDF + 32 * kb + 8 * grp;
                const float* bsrc = sBeta + 32 * kb + 8 * grp;
#pragma unroll
                for (int j = 0; j < 8; ++j) frag_set(fa, j, src[j] * bsrc[j]);
#pragma unroll
                for (int n = 0; n < PER; ++n) mma(acc[mt][n], fa, fb[n][kb]);
            }
        }
        // W natural into the A region (A is dead after the merges); U^T into
        // the K- region (dead after P2): 4 consecutive positions per store
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int n = 0; n < PER; ++n) {
                const int col = 16 * (nt0 + n) + r16;
                if (isW) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) sW[(16 * mt + 4 * grp + i) * LDK + col] = from_f<T>(acc[mt][n][i]);
                } else {
                    const float u4[4] = {acc[mt][n][0], acc[mt][n][1], acc[mt][n][2], acc[mt][n][3]};
                    st4(sUt + col * LDC + 16 * mt + 4 * grp, u4);
                }
            }
    }
    lds_barrier();
}

// ---------------------------------------------------------------------------
// seg_kernel: one workgroup per (b, h, segment r), chunks r*L .. of the chain.
//   o     [B,T,H,DV] output; receives o_local (final for segment 0)
//   qeff  [B*H*NT][C][DK] effective queries of every chunk (segments >= 1 read)
//   xend  [B*H][NS][DK][DK+DV] fp32: [M_r | N_r] of every segment
// Segment 0 starts from S = h0 (or 0), so its o_local and N_0 are exact.
template <int KIND, typename T, int DK, int DV, bool PRO>
__global__ __launch_bounds__(kSegThreads, 1) void seg_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ g,
    const float* __restrict__ beta, const float* __restrict__ h0, T* __restrict__ o, T* __restrict__ qeff,
    float* __restrict__ xend, unsigned* __restrict__ flags, int Tlen, int H, int NT, int L, int NS, Prologue pro)
{
    using Cfg = SegCfg<KIND, T, DK, DV>;
    constexpr int C = kChunk;
    constexpr int NKB = DK / 32;
    constexpr int NCW = Cfg::NCW, NTW = Cfg::NTW;
    constexpr int LDK = Cfg::LDK, LDC = Cfg::LDC;
    constexpr bool DELTA = KIND != KIND_LA;
    __shared__ __attribute__((aligned(16))) uint8_t smem[Cfg::BYTES];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, grp = lane >> 4;
    const int r = blockIdx.x % NS;
    const int chain = blockIdx.x / NS;
    const int b = chain / H, h = chain % H;
    const int cbeg = r * L, cend = min(NT, cbeg + L);
    ProHead ph{};
    if constexpr (PRO) ph = pro_head(pro, h);

    // X columns of this wave: waves 0-3 hold P columns, 4-7 S columns
    const bool isS = wave >= 4;
    const int col0 = (wave & 3) * NCW;
    f32x4 X[NKB][2][NTW];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int n = 0; n < NTW; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 32 * kb + 8 * grp + 4 * hh + i, col = col0 + 16 * n + r16;
                    X[kb][hh][n][i] = (!isS && row == col) ? 1.f : 0.f;
                }
    if (isS && r == 0 && h0 != nullptr) {
        const float* h0c = h0 + (size_t)chain * DK * DV;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int n = 0; n < NTW; ++n)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        X[kb][hh][n][i] = h0c[(32 * kb + 8 * grp + 4 * hh + i) * DV + col0 + 16 * n + r16];
    }

    const T* sQp = reinterpret_cast<const T*>(smem + Cfg::R_QP);
    const T* sW = reinterpret_cast<const T*>(smem + Cfg::R_A);
    const T* sU = reinterpret_cast<const T*>(smem + (DELTA ? Cfg::R_KM : Cfg::R_VT));
    const T* sKbT = reinterpret_cast<const T*>(smem + Cfg::R_KBT);
    const T* sAqk = reinterpret_cast<const T*>(smem + Cfg::R_AQK);
    const float* sPhi = reinterpret_cast<const float*>(smem + Cfg::R_PHI);

    SegIn<KIND, T, DK, DV> in;
    auto row0_of = [&](int c) { return ((size_t)b * Tlen + (size_t)c * C) * H + h; };
    auto nvalid_of = [&](int c) { return min(C, Tlen - c * C); };
    if (cbeg < cend) seg_load<KIND, T, DK, DV>(in, q, k, v, g, beta, row0_of(cbeg), nvalid_of(cbeg), H);

    for (int c = cbeg; c < cend; ++c) {
        const int nvalid = nvalid_of(c);
        seg_chunk_ops<KIND, T, DK, DV, PRO>(in, smem, flags, nvalid, ph);
        // next chunk's inputs (clamped to the last chunk: unconditional loads)
        {
            const int cn = min(c + 1, cend - 1);
            seg_load<KIND, T, DK, DV>(in, q, k, v, g, beta, row0_of(cn), nvalid_of(cn), H);
        }

        // ---- P5: state step on this wave's NCW columns of X ----------------
        // Phases are kept apart with scheduling barriers so that only one
        // phase's operand fragments are in flight at a time; the bf16 copy of
        // X is re-formed where it is used (cheap packs) instead of being kept.
        auto xfrag = [&](int kb, int n) { return pack_frag<T>(X[kb][0][n], X[kb][1][n]); };
        // Y = U_bar - W X  (rows: positions 32 kbp + 8 grp + 4 hh + i)
        f32x4 Y[2][2][NTW];
#pragma unroll
        for (int kbp = 0; kbp < 2; ++kbp)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int n = 0; n < NTW; ++n) {
                    f32x4 u = {0.f, 0.f, 0.f, 0.f};
                    if (isS) {
                        float u4[4];
                        ld4(sU + (col0 + 16 * n + r16) * LDC + 32 * kbp + 8 * grp + 4 * hh, u4);
                        u = f32x4{u4[0], u4[1], u4[2], u4[3]};
                    }
                    Y[kbp][hh][n] = u;
                }
        if constexpr (DELTA) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                Frag<T> xf[NTW];
#pragma unroll
                for (int n = 0; n < NTW; ++n) xf[n] = xfrag(kb, n);
#pragma unroll
                for (int kbp = 0; kbp < 2; ++kbp)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        // negated W: the product accumulates U_bar - W X directly
                        Frag<T> fw = ld_frag(sW + (32 * kbp + prow(hh, r16)) * LDK + 32 * kb + 8 * grp);
                        fw = frag_neg(fw);
#pragma unroll
                        for (int n = 0; n < NTW; ++n) mma(Y[kbp][hh][n], fw, xf[n]);
                    }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        Frag<T> Yf[2][NTW];
#pragma unroll
        for (int kbp = 0; kbp < 2; ++kbp)
#pragma unroll
            for (int n = 0; n < NTW; ++n) Yf[kbp][n] = pack_frag<T>(Y[kbp][0][n], Y[kbp][1][n]);
        __builtin_amdgcn_sched_barrier(0);
        // Z^T = X^T Q~^T + Y^T Aqk^T, 32 positions at a time: lane (r16, grp)
        // holds columns col0 + 16 n + 4 grp + i of position 16 pt + r16;
        // stored as o_local (S waves) or q_eff (P waves, segments >= 1)
        // chunk bases are uniform; lanes add 32-bit offsets
        T* const ochunk = o + (((size_t)b * Tlen + (size_t)c * C) * H + h) * DV;
        T* const qchunk = qeff + ((size_t)chain * NT + c) * C * DK;
        const unsigned ocol = (unsigned)(col0 + 4 * grp);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            f32x4 Zt[NTW][2];
#pragma unroll
            for (int n = 0; n < NTW; ++n)
#pragma unroll
                for (int u = 0; u < 2; ++u) Zt[n][u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                Frag<T> xf[NTW];
#pragma unroll
                for (int n = 0; n < NTW; ++n) xf[n] = xfrag(kb, n);
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const Frag<T> fq = ld_frag(sQp + (16 * (2 * half + u) + r16) * LDK + 32 * kb + 8 * grp);
#pragma unroll
                    for (int n = 0; n < NTW; ++n) mma(Zt[n][u], xf[n], fq);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
#pragma unroll
                for (int kbp = 0; kbp <= half; ++kbp) {   // Aqk is zero above the diagonal
                    const Frag<T> fa = ld_frag(sAqk + (16 * (2 * half + u) + r16) * LDC + 32 * kbp + 8 * grp);
#pragma unroll
                    for (int n = 0; n < NTW; ++n) mma(Zt[n][u], Yf[kbp][n], fa);
                }
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int pos = 16 * (2 * half + u) + r16;
                if (isS) {
                    if (pos < nvalid) {
#pragma unroll
                        for (int n = 0; n < NTW; ++n) {
                            const float z4[4] = {Zt[n][u][0], Zt[n][u][1], Zt[n][u][2], Zt[n][u][3]};
                            st4(ochunk + ((unsigned)pos * (unsigned)(H * DV) + ocol + 16 * n), z4);
                        }
                    }
                } else if (r > 0) {
#pragma unroll
                    for (int n = 0; n < NTW; ++n) {
                        const float z4[4] = {Zt[n][u][0], Zt[n][u][1], Zt[n][u][2], Zt[n][u][3]};
                        st4(qchunk + ((unsigned)pos * DK + ocol + 16 * n), z4);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // X <- Diag(phi) X + Kbar^T Y
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                float ph4[4];
                ld4(sPhi + 32 * kb + 8 * grp + 4 * hh, ph4);
#pragma unroll
                for (int n = 0; n < NTW; ++n)
#pragma unroll
                    for (int i = 0; i < 4; ++i) X[kb][hh][n][i] *= ph4[i];
#pragma unroll
                for (int kbp = 0; kbp < 2; ++kbp) {
                    const Frag<T> fk = ld_frag(sKbT + (32 * kb + prow(hh, r16)) * LDC + 32 * kbp + 8 * grp);
#pragma unroll
                    for (int n = 0; n < NTW; ++n) mma(X[kb][hh][n], fk, Yf[kbp][n]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        lds_barrier();   // LDS operands are rewritten by the next chunk
    }

    // ---- segment end: [M | N] -------------------------------------------------
    float* xe = xend + ((size_t)chain * NS + r) * DK * (DK + DV) + (isS ? DK : 0) + col0 + r16;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int n = 0; n < NTW; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    xe[(size_t)(32 * kb + 8 * grp + 4 * hh + i) * (DK + DV) + 16 * n] = X[kb][hh][n][i];
}

// ---------------------------------------------------------------------------
// compose_kernel: per (chain, 16 value columns): S = N_0 (segment 0 began at
// the true initial state); for r = 1 .. NS-1: S_in[r] = S, written transposed
// in the I/O type for correct_kernel, then S <- M_r S + N_r.  Finally hT = S.
// fp32 throughout (FMA on the vector ALUs); 256 threads, thread t owns row
// t / 2 and 8 of the 16 columns.
constexpr int kComposeThreads = 256;
template <typename T, int DK, int DV>
__global__ __launch_bounds__(kComposeThreads) void compose_kernel(const float* __restrict__ xend,
                                                                  T* __restrict__ sinT, float* __restrict__ hT,
                                                                  int NS)
{
    static_assert(DK <= 128, "rows per thread");
    constexpr int NSL = DV / 16;
    constexpr int LDX = DK + DV;
    __shared__ __attribute__((aligned(16))) float sS[DK][16];
    const int tid = threadIdx.x;
    const int chain = blockIdx.x / NSL, c0 = (blockIdx.x % NSL) * 16;
    const int row = tid >> 1, half = tid & 1;
    const bool act = row < DK;
    const float* xe0 = xend + (size_t)chain * NS * DK * LDX;
    float s[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) s[j] = act ? xe0[(size_t)row * LDX + DK + c0 + 8 * half + j] : 0.f;
    for (int rr = 1; rr < NS; ++rr) {
        if (act) {
            T* dst = sinT + ((size_t)chain * NS + rr) * DV * DK;
#pragma unroll
            for (int j = 0; j < 8; ++j) dst[(size_t)(c0 + 8 * half + j) * DK + row] = from_f<T>(s[j]);
#pragma unroll
            for (int j = 0; j < 8; ++j) sS[row][8 * half + j] = s[j];
        }
        __syncthreads();
        const float* xe = xe0 + (size_t)rr * DK * LDX;
        float acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = act ? xe[(size_t)row * LDX + DK + c0 + 8 * half + j] : 0.f;
        if (act) {
            const float* mrow = xe + (size_t)row * LDX;
            for (int kk = 0; kk < DK; kk += 4) {
                const float4 m4 = *reinterpret_cast<const float4*>(mrow + kk);
                const float mv[4] = {m4.x, m4.y, m4.z, m4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int j = 0; j < 8; ++j) acc[j] = fmaf(mv[e], sS[kk + e][8 * half + j], acc[j]);
            }
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 8; ++j) s[j] = acc[j];
    }
    if (act && hT != nullptr) {
#pragma unroll
        for (int j = 0; j < 8; ++j) hT[((size_t)chain * DK + row) * DV + c0 + 8 * half + j] = s[j];
    }
}

// ---------------------------------------------------------------------------
// correct_kernel: o[c] += q_eff[c] S_in[r] for the chunks c of segments
// r >= 1.  One 256-thread workgroup per (chunk, chain) item; wave w owns the
// value columns DV/4 * w ..; lanes hold 4 consecutive columns of one
// position (O^T = S_in^T q_eff^T on MFMA).
template <typename T, int DK, int DV>
__global__ __launch_bounds__(kThreads) void correct_kernel(const T* __restrict__ qeff, const T* __restrict__ sinT,
                                                           T* __restrict__ o, int Tlen, int H, int NT, int L,
                                                           int NS)
{
    constexpr int C = kChunk;
    constexpr int NKB = DK / 32;
    constexpr int NTWc = DV / 64;          // 16-column tiles per wave
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, grp = lane >> 4;
    const int per = NT - L;                // corrected chunks per chain
    const int chain = blockIdx.x / per;
    const int c = L + blockIdx.x % per;
    const int r = c / L;
    const int b = chain / H, h = chain % H;
    const int nvalid = min(C, Tlen - c * C);
    const T* S = sinT + ((size_t)chain * NS + r) * DV * DK;
    const T* Q = qeff + ((size_t)chain * NT + c) * C * DK;
    f32x4 acc[NTWc][4];
#pragma unroll
    for (int n = 0; n < NTWc; ++n)
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc[n][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
        Frag<T> fs[NTWc];
#pragma unroll
        for (int n = 0; n < NTWc; ++n)
            fs[n] = ld_frag(S + (size_t)((DV / 4) * wave + 16 * n + r16) * DK + 32 * kb + 8 * grp);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
            const Frag<T> fq = ld_frag(Q + (size_t)(16 * pt + r16) * DK + 32 * kb + 8 * grp);
#pragma unroll
            for (int n = 0; n < NTWc; ++n) mma(acc[n][pt], fs[n], fq);
        }
    }
    T* orow = o + (((size_t)b * Tlen + (size_t)c * C) * H + h) * DV + (DV / 4) * wave + 4 * grp;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
        const int pos = 16 * pt + r16;
        if (pos < nvalid) {
#pragma unroll
            for (int n = 0; n < NTWc; ++n) {
                T* p = orow + (size_t)pos * H * DV + 16 * n;
                float cur[4];
                ld4(p, cur);
                const float z4[4] = {cur[0] + acc[n][pt][0], cur[1] + acc[n][pt][1], cur[2] + acc[n][pt][2],
                                     cur[3] + acc[n][pt][3]};
                st4(p, z4);
            }
        }
    }
}

}  // namespace dr
