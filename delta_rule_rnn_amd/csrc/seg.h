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

// LDS plan of seg_kernel (bytes).  Regions are reused across phases (P5 is
// the state step):
//   KP  K+ [C][LDK]                         P1 -> P5
//   KM  K- [C][LDK] (P1 -> P2), then T diag(beta) [C][LDC] in the I/O type
//       (P3 -> P5)
//   QP  Q~ [C][LDK]                         P1 -> P5
//   A   A fp32 [C][LDF]                     P2 -> P3
//   TT  per-group gate totals and their prefixes (P1), then T fp32 [C][LDF] (P3)
//   VT  V^T [DV][LDC]                       P1 -> P5
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
    static constexpr size_t R_VT = R_TT + up16(mx(SZ_F, (size_t)(NQ + 1) * DK * sizeof(float)));
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
                                         size_t row0, int nvalid, int H, int tid)
{
    using Cfg = SegCfg<KIND, T, DK, DV>;
    using In = SegIn<KIND, T, DK, DV>;
    using VT = typename In::VT;
    using VG = typename In::VG;
    constexpr int NCG = Cfg::NCG, PL = Cfg::PL, CPT = Cfg::CPT;
    const int lane = tid & 63;
    const int last = nvalid - 1;
    const int ch0 = CPT * (tid % NCG), p0 = (tid / NCG) * PL;
    // byte offsets from the chunk's first row (wave-uniform bases in scalar
    // registers): no 64-bit address per load
    const char* qc = reinterpret_cast<const char*>(q + row0 * DK);
    const char* kc = reinterpret_cast<const char*>(k + row0 * DK);
    const char* vc = reinterpret_cast<const char*>(v + row0 * DV);
    const char* gc = reinterpret_cast<const char*>(g + row0 * (KIND == KIND_KDA ? DK : 1));
    const char* bc = reinterpret_cast<const char*>(beta + row0);
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        const unsigned rr = (unsigned)min(p0 + i, last) * (unsigned)H;
        const unsigned ek = rr * (unsigned)DK + (unsigned)ch0;
        if constexpr (KIND == KIND_KDA) in.gv[i] = *reinterpret_cast<const VG*>(gc + ek * 4u);
        in.kv[i] = *reinterpret_cast<const VT*>(kc + ek * (unsigned)sizeof(T));
        in.qv[i] = *reinterpret_cast<const VT*>(qc + ek * (unsigned)sizeof(T));
    }
    // every thread loads (waves past the first re-read rows already fetched)
    // so that the loads are unconditional
    const unsigned rl = (unsigned)min(lane, last) * (unsigned)H * 4u;
    if constexpr (KIND != KIND_KDA) in.gs = *reinterpret_cast<const float*>(gc + rl);
    if constexpr (KIND != KIND_LA) in.bt = *reinterpret_cast<const float*>(bc + rl);
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        const unsigned ev = (unsigned)min(p0 + i, last) * (unsigned)(H * DV) + (unsigned)ch0;
        in.vv[i] = *reinterpret_cast<const VT*>(vc + ev * (unsigned)sizeof(T));
    }
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
// Steps a1-a3 of one chunk into LDS (P0-P3).  On return (after a barrier)
// LDS holds K+ (KP), Q~ (QP), V^T (VT), Kbar^T (KBT), Aqk (AQK), phi (PHI)
// and, for the delta kinds, T = (I + A)^-1 (TT, fp32), T diag(beta) in the
// I/O type (KM) and beta.  The state
// step forms the chunk's pseudo values as Y = T diag(beta) (U_bar - K+ X),
// the product U - W X of the UT transform taken in the other order, so W and
// U are never materialised.
template <int KIND, typename T, int DK, int DV, bool PRO, typename NF>
__device__ __forceinline__ void seg_chunk_ops(const SegIn<KIND, T, DK, DV>& in, uint8_t* smem,
                                              float& mxneg_seg, int nvalid, const ProHead& ph,
                                              int tid, NF&& next_loads)
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
    T* sQp = reinterpret_cast<T*>(smem + Cfg::R_QP);
    float* sA = reinterpret_cast<float*>(smem + Cfg::R_A);
    float* sTot = reinterpret_cast<float*>(smem + Cfg::R_TT);
    float* sT = reinterpret_cast<float*>(smem + Cfg::R_TT);
    T* sVt = reinterpret_cast<T*>(smem + Cfg::R_VT);
    T* sKbT = reinterpret_cast<T*>(smem + Cfg::R_KBT);
    T* sAqk = reinterpret_cast<T*>(smem + Cfg::R_AQK);
    float* sBeta = reinterpret_cast<float*>(smem + Cfg::R_BETA);
    float* sGam = reinterpret_cast<float*>(smem + Cfg::R_GAM);
    float* sPhi = reinterpret_cast<float*>(smem + Cfg::R_PHI);

    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar register)
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
                nk[i] = inv_sqrt(sk + kNormEps);
                nq[i] = inv_sqrt(sq + kNormEps);
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
        // exclusive prefix of the NQ = 16 group totals per channel, in place:
        // four adjacent lanes per channel take four groups each, then scan
        // across the four lanes; the channel's total goes to sAll
        static_assert(NQ == 16, "group scan");
        float* sAll = sTot + NQ * DK;
        if (tid < 4 * DK) {
            const int ch = tid >> 2, qq = tid & 3;
            float t[4], e[4], sum = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) t[i] = sTot[(4 * qq + i) * DK + ch];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                e[i] = sum;
                sum += t[i];
            }
            float x = sum;
            float y = __shfl_up(x, 1, 4);
            if (qq >= 1) x += y;
            y = __shfl_up(x, 2, 4);
            if (qq >= 2) x += y;
            const float excl = x - sum;
#pragma unroll
            for (int i = 0; i < 4; ++i) sTot[(4 * qq + i) * DK + ch] = excl + e[i];
            if (qq == 3) sAll[ch] = x;
        }
        lds_barrier();
        const VG pre = *reinterpret_cast<const VG*>(sTot + qg * DK + ch0);
        const VG all = *reinterpret_cast<const VG*>(sAll + ch0);
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
        // (V moves as stored, without a round trip through fp32).  The lanes
        // of one store hold channels CPT apart, rows whose addresses fall
        // on few LDS banks; at CPT = 4 each lane takes its channels in an
        // order rotated by (cg / 4) mod 4, so that one store's 64 lanes
        // spread over all banks
        const int rot = CPT == 4 ? (cg >> 2) & 3 : 0;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int jj = (j + rot) & (CPT - 1);
            float kr[PL];
            typename VecOf<T, 4>::type vt;
#pragma unroll
            for (int i = 0; i < PL; ++i) {
                float x = kb[0][i];
                T y = vv[i][0];
#pragma unroll
                for (int c = 1; c < CPT; ++c) {
                    x = jj == c ? kb[c][i] : x;
                    y = jj == c ? vv[i][c] : y;
                }
                kr[i] = x;
                vt[i] = y;
            }
            st4(sKbT + (ch0 + jj) * LDC + p0, kr);
            *reinterpret_cast<typename VecOf<T, 4>::type*>(sVt + (ch0 + jj) * LDC + p0) = vt;
        }
        if (qg == 0) {
#pragma unroll
            for (int j = 0; j < CPT; ++j) sPhi[ch0 + j] = phi[j];
        }
        if constexpr (PERCH) mxneg_seg = fmaxf(mxneg_seg, mxneg);
    }
    next_loads();
    lds_barrier();

    // ---- P2: A (fp32, natural) and Aqk (natural, inclusive diagonal) -------
    // The three lower 32x32 blocks (0,0), (1,0), (1,1) of each, one block per
    // wave (waves 0-2: A, waves 3-5: Aqk), four 16x16 tiles sharing their
    // operand loads; the diagonal blocks' upper tiles are written masked
    // (zero), so the state step can read Aqk in 32-wide key blocks.
    {
        const T* kminus = PERCH ? sKm : sKp;
        const int item = DELTA ? wave : wave + 3;   // decay_la: Aqk only (waves 0-2)
        if (item < 6) {
            const bool isA = item < 3;
            const int bi = item % 3;
            const int bI = bi == 0 ? 0 : 1, bJ = bi == 2 ? 1 : 0;   // (0,0) (1,0) (1,1)
            const T* arows = isA ? sKp : sQp;
            f32x4 acc[2][2];
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int v = 0; v < 2; ++v) acc[u][v] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                Frag<T> fa[2], fb[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    fa[u] = ld_frag(arows + (32 * bI + 16 * u + r16) * LDK + 32 * kb + 8 * grp);
                    fb[u] = ld_frag(kminus + (32 * bJ + 16 * u + r16) * LDK + 32 * kb + 8 * grp);
                }
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int v = 0; v < 2; ++v) mma(acc[u][v], fa[u], fb[v]);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int v = 0; v < 2; ++v) {
                    const int col = 32 * bJ + 16 * v + r16;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = 32 * bI + 16 * u + 4 * grp + i;
                        float ratio = 1.f;
                        if constexpr (!PERCH) ratio = (col <= row) ? __builtin_amdgcn_exp2f(sGam[row] - sGam[col]) : 0.f;
                        if (isA) sA[row * LDF + col] = (col < row) ? sBeta[row] * ratio * acc[u][v][i] : 0.f;
                        else sAqk[row * LDC + col] = from_f<T>((col <= row) ? ratio * acc[u][v][i] : 0.f);
                    }
                }
        }
    }
    lds_barrier();
    if constexpr (!PERCH) {
        // scalar gates: Q~ = q 2^gamma and K+ = k 2^gamma in place (every
        // reader of the raw rows is done)
#pragma unroll
        for (int i = 0; i < PL; ++i) {
            const int p = p0 + i;
            const float sc = __builtin_amdgcn_exp2f(sGam[p]);
            VT x = *reinterpret_cast<const VT*>(sQp + p * LDK + ch0);
            VT y = *reinterpret_cast<const VT*>(sKp + p * LDK + ch0);
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                x[j] = from_f<T>((float)x[j] * sc);
                y[j] = from_f<T>((float)y[j] * sc);
            }
            *reinterpret_cast<VT*>(sQp + p * LDK + ch0) = x;
            *reinterpret_cast<VT*>(sKp + p * LDK + ch0) = y;
        }
    }
    if constexpr (!DELTA) {
        lds_barrier();
        return;
    }

    // ---- P3: T = (I + A)^-1 ([GDN] "对角子块前代" and "合并相邻子块") ---------
    // Diagonal 16x16 blocks, one wave each: with N the block of A (strictly
    // lower, so N^16 = 0), (I + N)^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8).
    // The factors are powers of N and commute; the six dependent 16x16
    // products run on fp32 MFMA with the powers kept in an LDS block of T
    // that the later products never read (blocks (0,2), (0,3), (1,2), (1,3)).
    // T diag(beta) in the I/O type, row-major [C][LDC], over K- (dead after
    // P2): the state step's operand, written by the wave that finishes each
    // block
    T* sTb = reinterpret_cast<T*>(smem + Cfg::R_KM);
    static_assert((size_t)C * LDC * sizeof(T) <= Cfg::R_QP - Cfg::R_KM, "T diag(beta) fits K-");
    if (wave < 4) {
        const int blk = wave;
        float* Tb = sT + 16 * blk * LDF + 16 * blk;                             // the diagonal block
        float* Pw = sT + 16 * (blk >> 1) * LDF + 16 * (2 + (blk & 1));         // scratch block
        const float* Nb = sA + 16 * blk * LDF + 16 * blk;
        // T0 = I - N, in the accumulator layout (lane: column r16, rows 4 grp + i)
        f32x4 t;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 4 * grp + i;
            t[i] = (row == r16 ? 1.f : 0.f) - Nb[row * LDF + r16];
        }
        const float* P = Nb;
#pragma unroll
        for (int k = 0; k < 3; ++k) {
#pragma unroll
            for (int i = 0; i < 4; ++i) Tb[(4 * grp + i) * LDF + r16] = t[i];
            const f32x4 p2 = mm16_lds(P, LDF, P, LDF, lane, f32x4{0.f, 0.f, 0.f, 0.f});   // P <- P^2
#pragma unroll
            for (int i = 0; i < 4; ++i) Pw[(4 * grp + i) * LDF + r16] = p2[i];
            P = Pw;
            t = mm16_lds(Tb, LDF, Pw, LDF, lane, t);                                   // T <- T (I + P)
        }
        const float bc = sBeta[16 * blk + r16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            Tb[(4 * grp + i) * LDF + r16] = t[i];
            sTb[(16 * blk + 4 * grp + i) * LDC + 16 * blk + r16] = from_f<T>(t[i] * bc);
        }
    } else if (wave < 6) {
        // T01 and T23 are read by the 32-wide products below: zero
        float* z = sT + 16 * 2 * (wave - 4) * LDF + 16 * (2 * (wave - 4) + 1);
        T* zb = sTb + 16 * 2 * (wave - 4) * LDC + 16 * (2 * (wave - 4) + 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            z[(4 * grp + i) * LDF + r16] = 0.f;
            zb[(4 * grp + i) * LDC + r16] = from_f<T>(0.f);
        }
    }
    lds_barrier();
    // the 32-row diagonal halves, then the lower-left 32 x 32 block:
    // T10 = -T11 A10 T00 and T32 = -T33 A32 T22 (waves 0, 1); then
    // T[2:4][0:2] = -T[2:4][2:4] A[2:4][0:2] T[0:2][0:2], one 16 x 16 block
    // (i, j) per wave, the inner product Y = A[2:4][0:2] T[0:2][j] kept in
    // the wave's accumulators
    auto put = [&](int i, int j, const f32x4& z) {
        const float bc = sBeta[16 * j + r16];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sT[(16 * i + 4 * grp + e) * LDF + 16 * j + r16] = -z[e];
            sTb[(16 * i + 4 * grp + e) * LDC + 16 * j + r16] = from_f<T>(-z[e] * bc);
        }
    };
    if (wave < 2) {
        const int i = 2 * wave + 1, j = 2 * wave;
        const f32x4 y = mm16_lds(sA + 16 * i * LDF + 16 * j, LDF, sT + 16 * j * LDF + 16 * j, LDF, lane,
                                 f32x4{0.f, 0.f, 0.f, 0.f});
        put(i, j, mm16_acc(sT + 16 * i * LDF + 16 * i, LDF, y, lane));
    }
    lds_barrier();
    if (wave < 4) {
        const int i = 2 + (wave >> 1), j = wave & 1;
        auto yrow = [&](int r) {        // (A[2:4][0:2] T[0:2][j]) block row r
            f32x4 y = {0.f, 0.f, 0.f, 0.f};
            for (int m = j; m < 2; ++m)
                y = mm16_lds(sA + 16 * r * LDF + 16 * m, LDF, sT + 16 * m * LDF + 16 * j, LDF, lane, y);
            return y;
        };
        const f32x4 y2 = yrow(2);
        f32x4 z = mm16_acc(sT + 16 * i * LDF + 32, LDF, y2, lane);          // T(i, 2) Y(2)
        if (i == 3) {
            const f32x4 z3 = mm16_acc(sT + 48 * LDF + 48, LDF, yrow(3), lane);   // T(3, 3) Y(3)
#pragma unroll
            for (int e = 0; e < 4; ++e) z[e] += z3[e];
        }
        put(i, j, z);
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
    constexpr int LDK = Cfg::LDK, LDC = Cfg::LDC, LDF = Cfg::LDF;
    constexpr bool DELTA = KIND != KIND_LA;
    __shared__ __attribute__((aligned(16))) uint8_t smem[Cfg::BYTES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar register)
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
    const T* sKp = reinterpret_cast<const T*>(smem + Cfg::R_KP);
    const T* sV = reinterpret_cast<const T*>(smem + Cfg::R_VT);
    const T* sTb = reinterpret_cast<const T*>(smem + Cfg::R_KM);   // T diag(beta)
    const T* sKbT = reinterpret_cast<const T*>(smem + Cfg::R_KBT);
    const T* sAqk = reinterpret_cast<const T*>(smem + Cfg::R_AQK);
    const float* sPhi = reinterpret_cast<const float*>(smem + Cfg::R_PHI);

    float mxneg_seg = 0.f;   // largest chunk-local -gamma seen (gate-range flags)
    SegIn<KIND, T, DK, DV> in;
    auto row0_of = [&](int c) { return ((size_t)b * Tlen + (size_t)c * C) * H + h; };
    auto nvalid_of = [&](int c) { return min(C, Tlen - c * C); };
    // (cbeg < cend for every workgroup of the grid; the load stays
    // unconditional so that the compiler can count outstanding loads)
    seg_load<KIND, T, DK, DV>(in, q, k, v, g, beta, row0_of(cbeg), nvalid_of(cbeg), H, tid);
    {
        // As many stores as every chunk step issues after its loads, into an
        // empty range (the hardware drops them): the first chunk then sees
        // the same count of memory operations behind its inputs as every
        // later one, and the compiler waits for the inputs alone instead of
        // for everything outstanding.
        // (their data is the last loaded value, which keeps them behind the loads)
        const auto none = buffer_rsrc(o, 0u);
        const float z = (float)in.vv[Cfg::PL - 1][0];
        const float z4[4] = {z, z, z, z};
#pragma unroll
        for (int i = 0; i < 4 * NTW; ++i) buf_st4(none, 16u * i, (const T*)nullptr, z4);
    }

    for (int c = cbeg; c < cend; ++c) {
        const int nvalid = nvalid_of(c);
        // The thread index is re-read through an empty asm each chunk, so the
        // compiler recomputes the lane-dependent addresses inside the loop
        // instead of keeping dozens of them live across it (registers are
        // the scarce resource here: X alone takes 64 per lane).
        int tidv = threadIdx.x;
        asm volatile("" : "+v"(tidv));
        const int lane = tidv & 63, r16 = lane & 15, grp = lane >> 4;
        // next chunk's inputs (clamped to the last chunk: unconditional loads),
        // issued as soon as this chunk's are in LDS
        const int cn = min(c + 1, cend - 1);
        seg_chunk_ops<KIND, T, DK, DV, PRO>(in, smem, mxneg_seg, nvalid, ph, tidv, [&]() {
            seg_load<KIND, T, DK, DV>(in, q, k, v, g, beta, row0_of(cn), nvalid_of(cn), H, tidv);
        });

        // ---- P5: state step on this wave's NCW columns of X ----------------
        // The bf16 copy of X is re-formed where it is used (cheap packs)
        // instead of being kept in registers.
        auto xfrag = [&](int kb, int n) { return pack_frag<T>(X[kb][0][n], X[kb][1][n]); };
        // Y = T diag(beta) (U_bar - K+ X)  ([KDA] 3.2: U - W X with W = T diag(beta)
        // K+, U = T diag(beta) V), rows: positions 32 kbp + 8 grp + 4 hh + i.
        // decay_la: Y = U_bar.
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
                        ld4(sV + (col0 + 16 * n + r16) * LDC + 32 * kbp + 8 * grp + 4 * hh, u4);
                        u = f32x4{u4[0], u4[1], u4[2], u4[3]};
                    }
                    Y[kbp][hh][n] = u;
                }
        if constexpr (DELTA) {
            // R = U_bar - K+ X (in Y's registers)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                Frag<T> xf[NTW];
#pragma unroll
                for (int n = 0; n < NTW; ++n) xf[n] = xfrag(kb, n);
#pragma unroll
                for (int kbp = 0; kbp < 2; ++kbp)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        Frag<T> fk = ld_frag(sKp + (32 * kbp + prow(hh, r16)) * LDK + 32 * kb + 8 * grp);
                        fk = frag_neg(fk);
#pragma unroll
                        for (int n = 0; n < NTW; ++n) mma(Y[kbp][hh][n], fk, xf[n]);
                    }
            }
            Frag<T> Rf[2][NTW];
#pragma unroll
            for (int kbp = 0; kbp < 2; ++kbp)
#pragma unroll
                for (int n = 0; n < NTW; ++n) Rf[kbp][n] = pack_frag<T>(Y[kbp][0][n], Y[kbp][1][n]);
            // Y = (T diag(beta)) R; T is lower triangular
#pragma unroll
            for (int kbo = 0; kbo < 2; ++kbo)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
                    for (int n = 0; n < NTW; ++n) Y[kbo][hh][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kbi = 0; kbi <= kbo; ++kbi) {
                        const Frag<T> ft = ld_frag(sTb + (32 * kbo + prow(hh, r16)) * LDC + 32 * kbi + 8 * grp);
#pragma unroll
                        for (int n = 0; n < NTW; ++n) mma(Y[kbo][hh][n], ft, Rf[kbi][n]);
                    }
                }
        }
        Frag<T> Yf[2][NTW];
#pragma unroll
        for (int kbp = 0; kbp < 2; ++kbp)
#pragma unroll
            for (int n = 0; n < NTW; ++n) Yf[kbp][n] = pack_frag<T>(Y[kbp][0][n], Y[kbp][1][n]);
        // Z^T = X^T Q~^T + Y^T Aqk^T, 32 positions at a time: lane (r16, grp)
        // holds columns col0 + 16 n + 4 grp + i of position 16 pt + r16;
        // stored as o_local (S waves) or q_eff (P waves, segments >= 1)
        // chunk bases are uniform; lanes add 32-bit offsets.  o: rows past a
        // ragged chunk's end fall outside the resource and are dropped.
        const auto orsrc = buffer_rsrc(o + (((size_t)b * Tlen + (size_t)c * C) * H + h) * DV,
                                       (unsigned)(nvalid * H * DV * sizeof(T)));
        const auto qrsrc = buffer_rsrc(qeff + ((size_t)chain * NT + c) * C * DK, (unsigned)(C * DK * sizeof(T)));
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
                // every wave issues the same stores on every path (segment 0's
                // effective queries are written too, and never read)
                const unsigned pos = (unsigned)(16 * (2 * half + u) + r16);
                const auto rs = isS ? orsrc : qrsrc;
                const unsigned rowst = isS ? (unsigned)(H * DV) : (unsigned)DK;
#pragma unroll
                for (int n = 0; n < NTW; ++n) {
                    const float z4[4] = {Zt[n][u][0], Zt[n][u][1], Zt[n][u][2], Zt[n][u][3]};
                    buf_st4(rs, (pos * rowst + ocol + 16 * n) * (unsigned)sizeof(T), (const T*)nullptr, z4);
                }
            }
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
        }
        lds_barrier();   // LDS operands are rewritten by the next chunk
    }

    if constexpr (KIND == KIND_KDA) {
        if (flags) {
            const unsigned long long b16 = __ballot(mxneg_seg >= 16.f);
            const unsigned long long b126 = __ballot(mxneg_seg >= 126.f);
            if ((tid & 63) == 0 && (b16 | b126)) atomicOr(flags, (b16 ? 1u : 0u) | (b126 ? 2u : 0u));
        }
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
// fp32 MFMA (16x16x4) with fp32 operands; 256 threads, wave w owns the row
// tiles w*TPW .. of S (accumulators).  M_r does not depend on S, so the rows
// of the next segment's [M | N] are loaded into registers while the current
// product runs.
constexpr int kComposeThreads = 256;
template <typename T, int DK, int DV>
__global__ __launch_bounds__(kComposeThreads) void compose_kernel(const float* __restrict__ xend,
                                                                  T* __restrict__ sinT, float* __restrict__ hT,
                                                                  int NS)
{
    constexpr int LDX = DK + DV, NKB = DK / 32, NRT = DK / 16, TPW = NRT / 4;
    constexpr int LDT = DK + 4;      // padded row of S^T in LDS
    constexpr int NSL = DV / 16;
    static_assert(NRT % 4 == 0, "row tiles per wave");
    __shared__ __attribute__((aligned(16))) float sST[16 * LDT];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, grp = lane >> 4;
    // the NSL slices of a chain read the same [M | N]: consecutive logical
    // ids, so they share one XCD's L2
    const int lb = xcd_logical(blockIdx.x, gridDim.x);
    const int chain = lb / NSL, c0 = (lb % NSL) * 16;
    const float* xe0 = xend + (size_t)chain * NS * DK * LDX;
    struct Ops {
        Frag<float> m[TPW][NKB];   // rows of M_r (A fragments)
        float n[TPW][4];           // N_r at this lane's accumulator slots
    };
    auto trow = [&](int t) { return 16 * (wave * TPW + t); };
    auto load = [&](Ops& op, int rr) {
        const float* xe = xe0 + (size_t)rr * DK * LDX;
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
                op.m[t][kb] = ld_frag(xe + (size_t)(trow(t) + r16) * LDX + 32 * kb + 8 * grp);
#pragma unroll
            for (int i = 0; i < 4; ++i) op.n[t][i] = xe[(size_t)(trow(t) + 4 * grp + i) * LDX + DK + c0 + r16];
        }
    };
    f32x4 S[TPW];
    {
        Ops first;
        load(first, 0);
#pragma unroll
        for (int t = 0; t < TPW; ++t) S[t] = f32x4{first.n[t][0], first.n[t][1], first.n[t][2], first.n[t][3]};
    }
    Ops cur, nxt;
    if (NS > 1) load(cur, 1);
    for (int rr = 1; rr < NS; ++rr) {
        load(nxt, min(rr + 1, NS - 1));
        T* dst = sinT + ((size_t)chain * NS + rr) * DV * DK + (size_t)(c0 + r16) * DK;
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const float v4[4] = {S[t][0], S[t][1], S[t][2], S[t][3]};
            st4(dst + trow(t) + 4 * grp, v4);
            *reinterpret_cast<f32x4*>(sST + r16 * LDT + trow(t) + 4 * grp) = S[t];
        }
        lds_barrier();
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            f32x4 acc = {cur.n[t][0], cur.n[t][1], cur.n[t][2], cur.n[t][3]};
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) mma(acc, cur.m[t][kb], ld_frag(sST + r16 * LDT + 32 * kb + 8 * grp));
            S[t] = acc;
        }
        lds_barrier();
        cur = nxt;
    }
    if (hT != nullptr) {
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) hT[((size_t)chain * DK + trow(t) + 4 * grp + i) * DV + c0 + r16] = S[t][i];
    }
}

// ---------------------------------------------------------------------------
// correct_kernel: o[c] += q_eff[c] S_in[r] for the chunks c of segments
// r >= 1.  One 256-thread workgroup per (chain, segment r >= 1, group of
// kCorrChunks chunks of it): S_in^T (I/O dtype, [DV][DK]) is staged in LDS
// once; wave w owns the 16 positions 16 w .. of every chunk.  Per chunk the
// wave forms its [16][DV] correction on MFMA (O^T = S_in^T q_eff^T), parks
// it in its own fp32 LDS slab, and then reads, adds and writes o by whole
// rows, 16 bytes per lane (16 lanes cover a bf16 row of 128 values).  The
// next chunk's q_eff and o rows are loaded while the current one is
// processed.
constexpr int kCorrChunks = 8;
template <typename T, int DK, int DV>
__global__ __launch_bounds__(kThreads) void correct_kernel(const T* __restrict__ qeff, const T* __restrict__ sinT,
                                                           T* __restrict__ o, int Tlen, int H, int NT, int L,
                                                           int NS)
{
    constexpr int C = kChunk;
    constexpr int NKB = DK / 32;
    constexpr int NCT = DV / 16;           // 16-column tiles
    constexpr int LDS_ = DK + 8;           // padded row of S_in^T in LDS
    constexpr int LDO = DV + 4;            // padded row of a correction slab (floats)
    constexpr int EPL = 16 / sizeof(T);    // o elements per lane and access (16 bytes)
    constexpr int LPR = DV / EPL;          // lanes per o row
    constexpr int RPI = 64 / LPR;          // rows per wave-wide access
    constexpr int NIT = 16 / RPI;          // accesses for the wave's 16 rows
    static_assert(64 % LPR == 0 && 16 % RPI == 0, "row split");
    using V16 = typename VecOf<T, EPL>::type;
    __shared__ __attribute__((aligned(16))) T sS[DV * LDS_];
    __shared__ __attribute__((aligned(16))) float sO[4][16 * LDO];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, grp = lane >> 4;
    const int groups = (L + kCorrChunks - 1) / kCorrChunks;
    const int per = (NS - 1) * groups;
    // a segment's workgroups read the same S_in: consecutive logical ids,
    // so they share one XCD's L2
    const int lb = xcd_logical(blockIdx.x, gridDim.x);
    const int chain = lb / per;
    const int rem = lb % per;
    const int r = 1 + rem / groups;
    const int c0 = r * L + (rem % groups) * kCorrChunks;
    const int c1 = min(min(c0 + kCorrChunks, (r + 1) * L), NT);
    if (c0 >= c1) return;
    const int b = chain / H, h = chain % H;
    // S_in^T into LDS: 8 elements per thread and step
    const T* S = sinT + ((size_t)chain * NS + r) * DV * DK;
    for (int e = tid * 8; e < DV * DK; e += kThreads * 8) {
        const int row = e / DK, col = e % DK;
        st_frag(sS + row * LDS_ + col, ld_frag(S + e));
    }
    lds_barrier();
    float* slab = sO[wave];
    const int pos = 16 * wave + r16;
    const unsigned ostr = (unsigned)(H * DV);
    auto load_q = [&](Frag<T> (&fq)[NKB], int c) {
        const T* Q = qeff + ((size_t)chain * NT + c) * C * DK + (size_t)pos * DK + 8 * grp;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) fq[kb] = ld_frag(Q + 32 * kb);
    };
    auto orsrc_of = [&](int c) {
        return buffer_rsrc(o + (((size_t)b * Tlen + (size_t)c * C) * H + h) * DV,
                           (unsigned)(min(C, Tlen - c * C) * H * DV * sizeof(T)));
    };
    // this lane's o accesses: row 16 w + it*RPI + lane/LPR, elements
    // EPL*(lane%LPR) .. (rows past the end are dropped: read as zero, not
    // written)
    const int orow0 = 16 * wave + lane / LPR, ocol = EPL * (lane % LPR);
    auto ooff = [&](int it) { return ((unsigned)(orow0 + it * RPI) * ostr + (unsigned)ocol) * (unsigned)sizeof(T); };
    using U4 = unsigned __attribute__((ext_vector_type(4)));
    auto load_o = [&](U4 (&ov)[NIT], int c) {
        const auto rs = orsrc_of(c);
#pragma unroll
        for (int it = 0; it < NIT; ++it) ov[it] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)ooff(it), 0, 0);
    };
    Frag<T> fq[NKB];
    U4 on[NIT];
    load_q(fq, c0);
    load_o(on, c0);
    for (int c = c0; c < c1; ++c) {
        Frag<T> cur[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) cur[kb] = fq[kb];
        U4 oc[NIT];
#pragma unroll
        for (int it = 0; it < NIT; ++it) oc[it] = on[it];
        // (the last chunk reloads itself: the loads stay unconditional, and
        // the reload of o precedes this chunk's store)
        load_q(fq, min(c + 1, c1 - 1));
        load_o(on, min(c + 1, c1 - 1));
        f32x4 acc[NCT];
#pragma unroll
        for (int n = 0; n < NCT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int n = 0; n < NCT; ++n)
                mma(acc[n], ld_frag(sS + (16 * n + r16) * LDS_ + 32 * kb + 8 * grp), cur[kb]);
        // the wave's [16][DV] correction, row r16, columns 16n + 4(l/16) ..
#pragma unroll
        for (int n = 0; n < NCT; ++n) *reinterpret_cast<f32x4*>(slab + r16 * LDO + 16 * n + 4 * grp) = acc[n];
        // LDS accesses of one wave complete in order: the reads below see
        // the writes above (of other lanes of this wave)
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const auto rs = orsrc_of(c);
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const float* src = slab + (lane / LPR + it * RPI) * LDO + ocol;
            const V16 x = __builtin_bit_cast(V16, oc[it]);
            V16 y;
#pragma unroll
            for (int e = 0; e < EPL; ++e) y[e] = from_f<T>(to_f(x[e]) + src[e]);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(U4, y), rs, (int)ooff(it), 0, 0);
        }
        // the slab is rewritten for the next chunk only after these reads
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
}

}  // namespace dr
