// intra.h -- K1: chunk-parallel steps a1 (log2 cumsum), a2 (separable
// exponent prep) and a3 (UT transform), fused.  One 256-thread workgroup per
// (chunk, head, batch); everything stays in LDS until the chunk record is
// written.
//
// Page keys: [KDA] "TileLang 实战：KDA 从零到一–Kimi Delta Attention";
// [SD] "TileLang 实战：KDA 从零到一--标量衰减"; [GDN] "Gated DeltaNet";
// [DPLR] "RNN的复兴04:线性注意力并行计算DPLR".
//
// Per chunk (r, i = positions, d = key channel, gamma in log2 units):
//   a1  gamma_r = log2(e) * sum_{s<=r} g_s                 [KDA] section 0
//   a2  K+ = k 2^gamma, K- = k 2^-gamma, Q~ = q 2^gamma,
//       Kbar = k 2^(gamma_last - gamma), phi = 2^gamma_last  [KDA] 1.2, [DPLR] 5.3.4
//       (scalar gates keep raw k, q and apply the ratio 2^(gamma_r - gamma_i)
//        only where i <= r, [SD] 2.2)
//   a3  A = diag(beta) StrictLower(K+ K-^T) (bf16 MFMA, fp32 accumulate),
//       Aqk = Tril_incl(Q~ K-^T),
//       T = (I + A)^-1: the four 16x16 diagonal blocks by forward
//       substitution (one lane per column), the off-diagonal blocks by
//       T_ij = -T_ii sum_{j<=m<i} A_im T_mj on fp32 MFMA,
//       W = T diag(beta) K+, U = T diag(beta) V                [KDA] 3.2-3.3
#pragma once

#include "common.h"

namespace dr {

template <int KIND, typename T, int DK, int DV>
struct IntraCfg {
    static constexpr int C = kChunk;
    static constexpr int LDK = DK + 8;   // padded row (elements) of [C][DK] tiles
    static constexpr int LDF = C + 4;    // padded row (floats) of [C][C] fp32 tiles
    static constexpr int LDV = C + 8;    // padded row (elements) of [DV][C] tiles
    static constexpr size_t R_KP = 0;
    static constexpr size_t SZ_KP = (size_t)C * LDK * sizeof(T);
    static constexpr size_t SZ_VT = (size_t)DV * LDV * sizeof(T);
    static constexpr size_t SZ_F = (size_t)C * LDF * sizeof(float);
    static constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
    static constexpr size_t R_KM = R_KP + SZ_KP;                 // K-  | later beta*V^T
    static constexpr size_t R_QP = R_KM + mx(SZ_KP, SZ_VT);      // Q~  | later T (fp32)
    static constexpr size_t R_A = R_QP + mx(SZ_KP, SZ_F);        // A   | later W staging
    static constexpr size_t R_SMALL = R_A + mx(SZ_F, SZ_KP);
    // thread layout of the elementwise steps: CPT adjacent channels (one
    // 8-byte bf16 / 16-byte fp32 load) at PL consecutive positions
    static constexpr int CPT = DK / 32;         // channels per thread
    static constexpr int NCG = DK / CPT;        // channel groups (32)
    static constexpr int NQ = kThreads / NCG;   // position groups (8)
    static constexpr int PL = C / NQ;           // positions per group (8)
    static constexpr size_t R_BETA = R_SMALL;                        // [C] float
    static constexpr size_t R_GAM = R_BETA + C * sizeof(float);      // [C] float (scalar gates)
    static constexpr size_t R_TOT = R_GAM + C * sizeof(float);       // [NQ][DK] float
    static constexpr size_t BYTES = R_TOT + (size_t)NQ * DK * sizeof(float);
    static_assert(DK == 64 || DK == 128, "DK");
    static_assert(DV == DK, "DV == DK");
    static_assert(NQ * PL == C && PL == 8, "thread layout");
};

// Lower-triangular 16x16 tiles (ti >= tj) of a 64x64 matrix, in a fixed order.
__device__ __forceinline__ void lower_tile(int idx, int& ti, int& tj) {
    // 0:(0,0) 1:(1,0) 2:(1,1) 3:(2,0) 4:(2,1) 5:(2,2) 6:(3,0) 7:(3,1) 8:(3,2) 9:(3,3)
    ti = idx >= 6 ? 3 : idx >= 3 ? 2 : idx >= 1 ? 1 : 0;
    tj = idx - (ti * (ti + 1)) / 2;
}

// 16x16x16 fp32 product of two LDS blocks: Y = X[16x16] * Z[16x16]
// (natural reduction index 4*(lane/16) + s for step s).
__device__ __forceinline__ f32x4 mm16_lds(const float* X, int ldx, const float* Z, int ldz, int lane,
                                         f32x4 acc) {
    const int r = lane & 15, q = lane >> 4;
#pragma unroll
    for (int s = 0; s < 4; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(X[r * ldx + 4 * q + s], Z[(4 * q + s) * ldz + r], acc,
                                                   0, 0, 0);
    return acc;
}
// Y = X[16x16] (LDS) * Z where Z is a 16x16 accumulator tile in registers:
// step i uses accumulator element i, i.e. reduction index 4*(lane/16) + i.
__device__ __forceinline__ f32x4 mm16_acc(const float* X, int ldx, f32x4 Z, int lane) {
    const int r = lane & 15, q = lane >> 4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(X[r * ldx + 4 * q + i], Z[i], acc, 0, 0, 0);
    return acc;
}

// Inputs of one chunk as this thread holds them: channels CPT*cg .. +CPT-1
// (cg = tid % NCG) at positions qg*PL .. qg*PL+PL-1 (qg = tid / NCG), plus
// beta at position tid
// and, for scalar gates, the gate at position lane of wave 0.  Rows past the
// end of a ragged last chunk are loaded from the last valid row (so every load
// is unconditional) and replaced by zeros where they are used.
template <int KIND, typename T, int DK, int DV>
struct IntraIn {
    using Cfg = IntraCfg<KIND, T, DK, DV>;
    using VT = typename VecOf<T, Cfg::CPT>::type;
    using VG = typename VecOf<float, Cfg::CPT>::type;
    VT kv[Cfg::PL], qv[Cfg::PL], vv[Cfg::PL];
    VG gv[KIND == KIND_KDA ? Cfg::PL : 1];
    float bt, gs;
};

template <int KIND, typename T, int DK, int DV>
__device__ __forceinline__ void intra_load(IntraIn<KIND, T, DK, DV>& in, const T* __restrict__ q,
                                           const T* __restrict__ k, const T* __restrict__ v,
                                           const float* __restrict__ g, const float* __restrict__ beta,
                                           size_t row0, int nvalid, int H)
{
    using In = IntraIn<KIND, T, DK, DV>;
    using VT = typename In::VT;
    using VG = typename In::VG;
    constexpr int C = kChunk;
    constexpr int NCG = In::Cfg::NCG, PL = In::Cfg::PL, CPT = In::Cfg::CPT;
    const int tid = threadIdx.x & (kThreads - 1), lane = tid & 63;
    const int last = nvalid - 1;
    const int ch0 = CPT * (tid % NCG), p0 = (tid / NCG) * PL;
    // gates first, then k and q (step a1 needs them first), v last
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        const size_t off = (row0 + (size_t)min(p0 + i, last) * H) * DK + ch0;
        if constexpr (KIND == KIND_KDA) in.gv[i] = ld_stream(reinterpret_cast<const VG*>(g + off));
    }
    if constexpr (KIND != KIND_KDA) in.gs = (tid < 64) ? ld_stream(g + row0 + (size_t)min(lane, last) * H) : 0.f;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        const size_t off = (row0 + (size_t)min(p0 + i, last) * H) * DK + ch0;
        in.kv[i] = ld_stream(reinterpret_cast<const VT*>(k + off));
        in.qv[i] = ld_stream(reinterpret_cast<const VT*>(q + off));
    }
    if constexpr (KIND != KIND_LA) in.bt = (tid < C) ? ld_stream(beta + row0 + (size_t)min(tid, last) * H) : 0.f;
#pragma unroll
    for (int i = 0; i < PL; ++i)
        in.vv[i] = ld_stream(reinterpret_cast<const VT*>(v + (row0 + (size_t)min(p0 + i, last) * H) * DV + ch0));
}

// Steps a1-a3 (and the output operands) of one chunk from inputs already in
// registers (nvalid of its C rows are tokens); writes the chunk's record at
// recb.  With PRO, the input prologue (common.h) is applied to the loaded
// q, k, beta and scalar gates first.
//
// C2 = 128 (sub-chunked 128-token chunks, [KDA] 2.3): a 512-thread workgroup
// runs this body once per 64-row sub-chunk, threads 256*s .. 256*s+255 on
// sub-chunk s with the LDS regions at smem + s*Cfg::BYTES.  Each sub-chunk
// re-bases gamma at its own start, so K- never exceeds 2^(max -gamma) over
// 64 positions; the halves then exchange their gate totals and assemble the
// 128-row record (intra_merge below).
template <int KIND, typename T, int DK, int DV, bool PRO, int C2 = kChunk>
__device__ __forceinline__ void intra_chunk(const IntraIn<KIND, T, DK, DV>& in, uint8_t* smem_all,
                                            unsigned* __restrict__ flags,
                                            uint8_t* __restrict__ recb, int nvalid, const ProHead& ph)
{
    using Cfg = IntraCfg<KIND, T, DK, DV>;
    using R = Rec<T, DK, DV, C2>;
    constexpr int C = kChunk;
    constexpr bool SUB = C2 == 2 * kChunk;
    static_assert(C2 == kChunk || SUB, "record chunk");
    constexpr int KQ = C2 / 32, NW = C2 / 16;   // key blocks, position groups of the record
    constexpr bool DELTA = KIND != KIND_LA;
    constexpr bool PERCH = KIND == KIND_KDA;
    constexpr int LDK = Cfg::LDK, LDF = Cfg::LDF, LDV = Cfg::LDV;
    constexpr int NCG = Cfg::NCG, PL = Cfg::PL, NQ = Cfg::NQ, CPT = Cfg::CPT;
    using In = IntraIn<KIND, T, DK, DV>;
    using VT = typename In::VT;
    using VG = typename In::VG;

    // sub-chunk of this thread (0 unless SUB) and its LDS regions; sX: the
    // halves' gate totals (log2), [2][DK] floats after both regions
    const int half = SUB ? (int)(threadIdx.x >> 8) : 0;
    uint8_t* smem = smem_all + (SUB ? half * Cfg::BYTES : 0);
    float* sX = reinterpret_cast<float*>(smem_all + 2 * Cfg::BYTES);
    (void)sX;

    T* sKp = reinterpret_cast<T*>(smem + Cfg::R_KP);
    T* sKm = reinterpret_cast<T*>(smem + Cfg::R_KM);
    T* sVt = reinterpret_cast<T*>(smem + Cfg::R_KM);
    T* sQp = reinterpret_cast<T*>(smem + Cfg::R_QP);
    float* sT = reinterpret_cast<float*>(smem + Cfg::R_QP);
    float* sA = reinterpret_cast<float*>(smem + Cfg::R_A);
    T* sW = reinterpret_cast<T*>(smem + Cfg::R_A);
    float* sBeta = reinterpret_cast<float*>(smem + Cfg::R_BETA);
    float* sGam = reinterpret_cast<float*>(smem + Cfg::R_GAM);
    float* sTot = reinterpret_cast<float*>(smem + Cfg::R_TOT);

    const int tid = threadIdx.x & (kThreads - 1), lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, grp = lane >> 4;
    T* rW = reinterpret_cast<T*>(recb) + R::W;
    T* rQ = reinterpret_cast<T*>(recb) + R::QT;
    T* rKb = reinterpret_cast<T*>(recb) + R::KBT;
    T* rAqk = reinterpret_cast<T*>(recb) + R::AQK;
    T* rU = reinterpret_cast<T*>(recb) + R::UT;
    float* rPhi = reinterpret_cast<float*>(recb + R::PHI_BYTE);

    // ---- P0: this chunk's inputs (loaded one step ahead), rows past the end
    // of a ragged chunk zeroed
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
    // prologue: per-row factors of k and q (L2 normalisation, query scale).
    // A row's DK channels sit in the NCG = 32 adjacent lanes of one half
    // wave, so its sum of squares is a sum over that lane group.
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

    // ---- P1: a1 (gamma) + a2 (prep) -------------------------------------
    float gam[PL][CPT];
    float glast[CPT];
    if constexpr (PERCH) {
        // per-channel inclusive scan: each thread owns CPT channels x PL positions
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
                // last position of the chunk: (sum of the first NQ-1 group
                // totals) + last total, added in the same order as the last
                // group's own prefix + running sum
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
        // scalar gate: wave 0 scans the 64 positions
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
    // SUB: the other sub-chunk's gate totals
    float gother[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) gother[j] = 0.f;
    if constexpr (SUB) {
        if (PERCH ? qg == 0 : tid == 0) {
#pragma unroll
            for (int j = 0; j < CPT; ++j) sX[half * DK + ch0 + j] = glast[j];
        }
        lds_barrier();
#pragma unroll
        for (int j = 0; j < CPT; ++j) gother[j] = sX[(1 - half) * DK + (PERCH ? ch0 + j : 0)];
    }

    // Kbar of the merge (SUB, first sub-chunk): relative to the sub-chunk's
    // end, natural layout (this thread's CPT channels x PL positions)
    T kbl[SUB ? CPT : 1][SUB ? PL : 1];
    {
        // phi and Kbar of the record are relative to the record chunk's end
        // (for the first sub-chunk of a 128-token chunk, the totals of both)
        float phi[CPT], phl[CPT];
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            phl[j] = __builtin_amdgcn_exp2f(glast[j]);
            phi[j] = (SUB && half == 0) ? __builtin_amdgcn_exp2f(glast[j] + gother[j]) : phl[j];
        }
        (void)phl;
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
                    // Kbar = k 2^(gamma_last - gamma) = (k 2^-gamma) 2^gamma_last
                    kb[j][i] = kk * (ei * phi[j]);
                    if constexpr (SUB) kbl[j][i] = from_f<T>(kk * (ei * phl[j]));
                }
                *reinterpret_cast<VT*>(sKp + p * LDK + ch0) = kp;
                *reinterpret_cast<VT*>(sKm + p * LDK + ch0) = km;
                *reinterpret_cast<VT*>(sQp + p * LDK + ch0) = qp;
            } else {
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
                const float r = __builtin_amdgcn_exp2f(glast[0] - gam[i][0]) * nk[i];   // <= 1 (times nk)
                const float rc = (SUB && half == 0) ? r * __builtin_amdgcn_exp2f(gother[0]) : r;
#pragma unroll
                for (int j = 0; j < CPT; ++j) {
                    kb[j][i] = (float)kv[i][j] * rc;
                    if constexpr (SUB) kbl[j][i] = from_f<T>((float)kv[i][j] * r);
                }
            }
        }
        // Kbar in fragment order: channel ch is row prow(h, r) of key block
        // ch/32; each run of 8 positions is one 16-byte store
#pragma unroll
        for (int cc = 0; cc < CPT; ++cc) {
            const int ch = ch0 + cc, qq = ch & 31;
            const int wk = ch >> 5, hh = (qq >> 2) & 1, rr = 4 * (qq >> 3) + (qq & 3);
#pragma unroll
            for (int i0 = 0; i0 < PL; i0 += 8) {
                const int p = p0 + i0;
                Frag<T> f;
#pragma unroll
                for (int j = 0; j < 8; ++j) frag_set(f, j, kb[cc][i0 + j]);
                st_frag_stream(rKb + ((size_t)(((wk * 2 + hh) * KQ + (p >> 5) + 2 * half) * 64) + rr +
                                      16 * ((p & 31) >> 3)) * 8, f);
            }
        }
        if (qg == 0 && half == 0) {
            VG ph;
#pragma unroll
            for (int j = 0; j < CPT; ++j) ph[j] = phi[j];
            st_stream(reinterpret_cast<VG*>(rPhi + ch0), ph);
        }
        if constexpr (PERCH) {
            if (flags) {
                const unsigned long long b16 = __ballot(mxneg >= 16.f);
                const unsigned long long b126 = __ballot(mxneg >= 126.f);
                if (lane == 0 && (b16 | b126))
                    atomicOr(flags, (b16 ? 1u : 0u) | (b126 ? 2u : 0u));
            }
        }
        if constexpr (!DELTA) {
            // decay_la: the state pass reads V from the U slot (fragment order)
#pragma unroll
            for (int cc = 0; cc < CPT; ++cc) {
                const int ch = ch0 + cc;
                float vt[PL];
#pragma unroll
                for (int i = 0; i < PL; ++i) vt[i] = (float)vv[i][cc];
#pragma unroll
                for (int i = 0; i < PL; i += 4) {
                    const int p = p0 + i;
                    const int wv = 2 * (p >> 5) + ((p >> 2) & 1);
                    st4_stream(rU + ((size_t)(((ch >> 4) * NW + wv + 4 * half) * 64) + (ch & 15) +
                                     16 * ((p & 31) >> 3)) * 4, &vt[i]);
                }
            }
        }
    }
    lds_barrier();

    // ---- P2: A (natural layout, LDS) and Aqk (fragment order, record) ------
    {
        constexpr int NKB = DK / 32;
        constexpr int NA = DELTA ? 10 : 0;      // lower 16x16 tiles of A
        const T* kminus = PERCH ? sKm : sKp;
        // items: NA tiles of A, then the 6 nonzero 32x32 blocks (w, kb) of Aqk,
        // kb <= w/2, each computed transposed (keys x queries) with rows and
        // columns permuted so that the accumulators are fragment-ordered
        // (SUB: then 4 of the 8 blocks of Aqk10, below)
        constexpr int NX = SUB ? 4 : 0;
        for (int idx = wave; idx < NA + 6 + NX; idx += 4) {
            if (idx < NA) {
                int ti, tj;
                lower_tile(idx, ti, tj);
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    const Frag<T> fa = ld_frag(sKp + (16 * ti + r16) * LDK + 32 * kb + 8 * grp);
                    const Frag<T> fb = ld_frag(kminus + (16 * tj + r16) * LDK + 32 * kb + 8 * grp);
                    mma(acc, fa, fb);
                }
                const int col = 16 * tj + r16;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * ti + 4 * grp + i;
                    float ratio = 1.f;
                    if constexpr (!PERCH) ratio = (col < row) ? __builtin_amdgcn_exp2f(sGam[row] - sGam[col]) : 0.f;
                    sA[row * LDF + col] = (col < row) ? sBeta[row] * ratio * acc[i] : 0.f;
                }
            } else if (idx < NA + 6) {
                const int bI = idx - NA;   // (w, kb): (0,0) (1,0) (2,0) (2,1) (3,0) (3,1)
                const int w = bI < 2 ? bI : 2 + ((bI - 2) >> 1);
                const int kbk = bI < 2 ? 0 : ((bI - 2) & 1);
                const int query = pw(w, r16);
                f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
                for (int kd = 0; kd < NKB; ++kd) {
                    const Frag<T> fq = ld_frag(sQp + query * LDK + 32 * kd + 8 * grp);
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const Frag<T> fk = ld_frag(kminus + (32 * kbk + prow(hh, r16)) * LDK + 32 * kd + 8 * grp);
                        mma(acc[hh], fk, fq);   // [key][query]
                    }
                }
                Frag<T> out;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int key = 32 * kbk + 8 * grp + 4 * hh + i;
                        float val = 0.f;
                        if (key <= query) {
                            val = acc[hh][i];
                            if constexpr (!PERCH) val *= __builtin_amdgcn_exp2f(sGam[query] - sGam[key]);
                        }
                        frag_set(out, 4 * hh + i, val);
                    }
                st_frag_stream(rAqk + ((size_t)((w + 4 * half) * KQ + kbk + 2 * half) * 64 + lane) * 8, out);
            } else {
                // SUB: block (w1, kbk) of Aqk10 = Q~1 K-0^T, queries of the
                // second sub-chunk against keys of the first.  With gamma
                // based at the chunk start, Q~1 = (its sub-chunk's Q~) * phi0
                // <= 1 and K-0 stays within the first sub-chunk's range.
                const int bx = 4 * half + (idx - NA - 6);
                const int w1 = bx >> 1, kbk = bx & 1;
                const T* q1 = reinterpret_cast<const T*>(smem_all + Cfg::BYTES + Cfg::R_QP);
                const T* k0 = reinterpret_cast<const T*>(smem_all + (PERCH ? Cfg::R_KM : Cfg::R_KP));
                const float* gam0 = reinterpret_cast<const float*>(smem_all + Cfg::R_GAM);
                const float* gam1 = reinterpret_cast<const float*>(smem_all + Cfg::BYTES + Cfg::R_GAM);
                const int query = pw(w1, r16);
                f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
                for (int kd = 0; kd < NKB; ++kd) {
                    Frag<T> fq = ld_frag(q1 + query * LDK + 32 * kd + 8 * grp);
                    if constexpr (PERCH) {
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            frag_set(fq, j, frag_get(fq, j) * __builtin_amdgcn_exp2f(sX[32 * kd + 8 * grp + j]));
                    }
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const Frag<T> fk = ld_frag(k0 + (32 * kbk + prow(hh, r16)) * LDK + 32 * kd + 8 * grp);
                        mma(acc[hh], fk, fq);   // [key][query]
                    }
                }
                Frag<T> out;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int key = 32 * kbk + 8 * grp + 4 * hh + i;
                        float val = acc[hh][i];
                        if constexpr (!PERCH) val *= __builtin_amdgcn_exp2f(gam1[query] + sX[0] - gam0[key]);
                        frag_set(out, 4 * hh + i, val);
                    }
                st_frag_stream(rAqk + ((size_t)((4 + w1) * KQ + kbk) * 64 + lane) * 8, out);
            }
        }
        // the two blocks above the diagonal (w = 0, 1; kb = 1) are zero
        // (SUB: and, for the first sub-chunk's rows, both blocks of the second
        // sub-chunk's keys)
        {
            Frag<T> z;
#pragma unroll
            for (int j = 0; j < 8; ++j) frag_set(z, j, 0.f);
            if (tid < 128)
                st_frag_stream(rAqk + ((size_t)(((tid >> 6) + 4 * half) * KQ + 1 + 2 * half) * 64 + (tid & 63)) * 8, z);
            if (SUB && half == 0) {
#pragma unroll
                for (int kz = 2; kz < 4; ++kz)
                    st_frag_stream(rAqk + ((size_t)((tid >> 6) * KQ + kz) * 64 + (tid & 63)) * 8, z);
            }
        }
        // Q~ in fragment order, from the LDS copy (scalar gates scale it here)
        for (int e = tid; e < 4 * NKB * 64; e += kThreads) {
            const int l = e & 63, kq = (e >> 6) % NKB, w = (e >> 6) / NKB;
            const int row = pw(w, l & 15);
            Frag<T> f = ld_frag(sQp + row * LDK + 32 * kq + 8 * (l >> 4));
            if constexpr (!PERCH) {
                // (the second sub-chunk: gamma re-based to the chunk start)
                const float sc = __builtin_amdgcn_exp2f(sGam[row] + (half ? sX[0] : 0.f));
#pragma unroll
                for (int j = 0; j < 8; ++j) frag_set(f, j, frag_get(f, j) * sc);
            } else if (SUB && half == 1) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    frag_set(f, j, frag_get(f, j) * __builtin_amdgcn_exp2f(sX[32 * kq + 8 * (l >> 4) + j]));
            }
            st_frag_stream(rQ + ((size_t)e + (size_t)half * 4 * NKB * 64) * 8, f);
        }
    }
    if constexpr (!DELTA) return;
    lds_barrier();

    // ---- P3: T = (I + A)^-1 -----------------------------------------------
    if (wave == 0) {
        // diagonal blocks by forward substitution: lane = (block, column)
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
        if ((blk & 1) == 0) {   // T01 and T23 are read by the 32-wide product below
#pragma unroll
            for (int r = 0; r < 16; ++r) sT[(16 * blk + r) * LDF + 16 * (blk + 1) + col] = 0.f;
        }
    }
    {
        // beta * V, transposed into sVt[e][p] (the K- region is free now):
        // each thread writes its PL consecutive positions of CPT value channels
#pragma unroll
        for (int cc = 0; cc < CPT; ++cc) {
            float vt[PL];
#pragma unroll
            for (int i = 0; i < PL; ++i) vt[i] = sBeta[p0 + i] * (float)vv[i][cc];
            T* dst = sVt + (ch0 + cc) * LDV + p0;
#pragma unroll
            for (int i = 0; i < PL; i += 4) st4(dst + i, &vt[i]);
        }
    }
    lds_barrier();
    // off-diagonal blocks, by distance from the diagonal
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

    // ---- P4: [W | U] = T diag(beta) [K+ | V] --------------------------------
    {
        constexpr int NTW = DK / 16, NTN = (DK + DV) / 16, PER = NTN / 4, NKB = DK / 32;
        static_assert(NTN % 4 == 0 && (NTW % PER) == 0, "n-tile split");
        const int nt0 = wave * PER;
        const bool isW = nt0 < NTW;
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
                        float s = sBeta[p];
                        if constexpr (!PERCH) s *= __builtin_amdgcn_exp2f(sGam[p]);
                        frag_set(fb[n][kb], j, s * to_f(sKp[p * LDK + col]));
                    }
                } else {
                    const int e = 16 * (nt0 + n - NTW) + r16;
                    fb[n][kb] = ld_frag(sVt + e * LDV + 32 * kb + 8 * grp);
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
            // U rows are taken in the state pass's order (pw), W rows naturally
            const int arow = isW ? 16 * mt + r16 : pw(mt, r16);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (kb == 1 && mt < 2) continue;   // T is lower triangular
                Frag<T> fa;
                const float* src = sT + arow * LDF + 32 * kb + 8 * grp;
#pragma unroll
                for (int j = 0; j < 8; ++j) frag_set(fa, j, src[j]);
#pragma unroll
                for (int n = 0; n < PER; ++n) mma(acc[mt][n], fa, fb[n][kb]);
            }
        }
        // bf16: W is staged in LDS (the A region is free now) so the global
        // stores are 16-byte row segments
        auto stage_w = [&]() {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int n = 0; n < PER; ++n)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        sW[(16 * mt + 4 * grp + i) * LDK + 16 * (nt0 + n) + r16] = from_f<T>(acc[mt][n][i]);
        };
        auto copy_w = [&]() {
            // W in fragment order from the staged natural tile
            for (int e = tid; e < 4 * NKB * 64; e += kThreads) {
                const int l = e & 63, kq = (e >> 6) % NKB, w = (e >> 6) / NKB;
                st_frag_stream(rW + ((size_t)e + (size_t)half * 4 * NKB * 64) * 8,
                               ld_frag(sW + pw(w, l & 15) * LDK + 32 * kq + 8 * (l >> 4)));
            }
        };
        // fp32: 4-byte elements, stored straight from the accumulators into
        // their fragment-order slots.  (Staging these through LDS hit a
        // miscompile in this toolchain: two of the four row stores were merged
        // into one ds_write2_b32 whose first offset was encoded wrong at
        // Dk = 128.)
        auto direct_w = [&]() {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int n = 0; n < PER; ++n)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = 16 * mt + 4 * grp + i, col = 16 * (nt0 + n) + r16;
                        const int qq = row & 31;
                        const int wr = 2 * (row >> 5) + ((qq >> 2) & 1) + 4 * half, rr = 4 * (qq >> 3) + (qq & 3);
                        const size_t e = ((size_t)(wr * NKB + (col >> 5)) * 64 + rr + 16 * ((col & 31) >> 3)) * 8 + (col & 7);
                        rW[e] = from_f<T>(acc[mt][n][i]);
                    }
        };
        // U: m-tile mt holds the rows of state-pass wave mt, so each lane's 4
        // values are one fragment-order slot group
        auto store_u = [&]() {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int n = 0; n < PER; ++n) {
                    const int t = nt0 + n - NTW;
                    float vals[4] = {acc[mt][n][0], acc[mt][n][1], acc[mt][n][2], acc[mt][n][3]};
                    st4_stream(rU + ((size_t)(t * NW + mt + 4 * half) * 64 + lane) * 4, vals);
                }
        };
        if constexpr (!SUB) {
            if (isW) {
                if constexpr (sizeof(T) == 2) stage_w();
                else direct_w();
            } else {
                store_u();
            }
            if constexpr (sizeof(T) == 2) {
                lds_barrier();
                copy_w();
            }
        } else {
            // ---- SUB: the second sub-chunk's rows of the 128-row W and U.
            // Block elimination of (I + A) over the two sub-chunks gives
            // T10 = -T11 A10 T00 with A10 = diag(beta1) K+1 Kbar0^T (both
            // factors sub-chunk local), so with G = W1 Kbar0^T = T11 A10:
            //   W1 <- W1 Diag(phi0) - G W0,   U1 <- U1 - G U0
            // (W1, U1 of the second sub-chunk alone; W0, U0 of the first,
            // whose gamma base is already the chunk start).
            T* sW1 = reinterpret_cast<T*>(smem_all + Cfg::BYTES + Cfg::R_A);                // W1, natural rows
            T* sKb0 = reinterpret_cast<T*>(smem_all + Cfg::R_KP);                          // Kbar0, natural rows
            T* sWU0 = reinterpret_cast<T*>(smem_all + Cfg::R_KM);                          // [W0|U0] B fragments
            float* sG = reinterpret_cast<float*>(smem_all + Cfg::BYTES + Cfg::R_KP);      // G [64][LDF]
            static_assert((size_t)NTN * 2 * 64 * 8 * sizeof(T) <= Cfg::R_A - Cfg::R_KM, "[W0|U0] staging");
            static_assert((size_t)C * LDF * sizeof(float) <= Cfg::R_QP, "G staging");
            static_assert((size_t)C * LDK * sizeof(T) <= Cfg::R_SMALL - Cfg::R_A, "W staging");
            if (isW && (sizeof(T) == 2 || half == 1)) stage_w();
            lds_barrier();   // every P4 operand read done; W staged
            if (half == 0) {
#pragma unroll
                for (int i = 0; i < PL; ++i) {
                    VT x;
#pragma unroll
                    for (int cc = 0; cc < CPT; ++cc) x[cc] = kbl[cc][i];
                    *reinterpret_cast<VT*>(sKb0 + (p0 + i) * LDK + ch0) = x;
                }
                // natural B fragments over the positions: slots 0-3 from
                // m-tile 2kb, 4-7 from 2kb+1 (W: rows 32kb + 4(l/16) + i and
                // 32kb + 16 + ..., U: rows 32kb + 8(l/16) + j)
#pragma unroll
                for (int n = 0; n < PER; ++n)
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        Frag<T> f;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            frag_set(f, i, acc[2 * kb][n][i]);
                            frag_set(f, 4 + i, acc[2 * kb + 1][n][i]);
                        }
                        st_frag(sWU0 + ((size_t)((nt0 + n) * 2 + kb) * 64 + lane) * 8, f);
                    }
                // (copy_w is strided over all of the sub-chunk's threads)
                if constexpr (sizeof(T) == 2) copy_w();
                if (isW) {
                    if constexpr (sizeof(T) == 4) direct_w();
                } else {
                    store_u();
                }
            }
            lds_barrier();   // Kbar0 and [W0|U0] visible
            {
                // G = W1 Kbar0^T: 16 tiles over the 8 waves
                const int w8 = (int)(threadIdx.x >> 6);
#pragma unroll
                for (int tt = w8; tt < 16; tt += 8) {
                    const int ti = tt >> 2, tj = tt & 3;
                    f32x4 g4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb)
                        mma(g4, ld_frag(sW1 + (16 * ti + r16) * LDK + 32 * kb + 8 * grp),
                            ld_frag(sKb0 + (16 * tj + r16) * LDK + 32 * kb + 8 * grp));
#pragma unroll
                    for (int i = 0; i < 4; ++i) sG[(16 * ti + 4 * grp + i) * LDF + 16 * tj + r16] = g4[i];
                }
            }
            lds_barrier();   // G visible; W1 staging free
            if (half == 1) {
                if (isW) {
#pragma unroll
                    for (int n = 0; n < PER; ++n) {
                        const int col = 16 * (nt0 + n) + r16;
                        const float p0s = __builtin_amdgcn_exp2f(sX[PERCH ? col : 0]);
#pragma unroll
                        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                            for (int i = 0; i < 4; ++i) acc[mt][n][i] *= p0s;
                    }
                }
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const int grow = isW ? 16 * mt + r16 : pw(mt, r16);
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        // -G row grow, in the slot order of the fragments above
                        const float* gr = sG + grow * LDF + 32 * kb;
                        float gv8[8];
                        if (isW) {
                            ld4(gr + 4 * grp, gv8);
                            ld4(gr + 16 + 4 * grp, gv8 + 4);
                        } else {
                            ld4(gr + 8 * grp, gv8);
                            ld4(gr + 8 * grp + 4, gv8 + 4);
                        }
                        Frag<T> fa;
#pragma unroll
                        for (int j = 0; j < 8; ++j) frag_set(fa, j, -gv8[j]);
#pragma unroll
                        for (int n = 0; n < PER; ++n)
                            mma(acc[mt][n], fa, ld_frag(sWU0 + ((size_t)((nt0 + n) * 2 + kb) * 64 + lane) * 8));
                    }
                }
                if (isW) {
                    if constexpr (sizeof(T) == 2) stage_w();
                    else direct_w();
                } else {
                    store_u();
                }
            }
            if constexpr (sizeof(T) == 2) {
                lds_barrier();
                if (half == 1) copy_w();
            }
        }
    }
}

// One workgroup per item (chunk, head, batch) of chunks c0 .. c0+n-1,
// numbered heads fastest: the workgroups in flight at any time cover few
// chunks, so the rows of beta and of scalar gates that neighbouring heads
// share are fetched while still cached.  (Grouping a chunk's heads on one
// XCD, or numbering chunks fastest, measured slower.)
template <int KIND, typename T, int DK, int DV, bool PRO>
__global__ __launch_bounds__(kThreads, 2) void intra_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, uint8_t* __restrict__ ws,
    unsigned* __restrict__ flags, int Tlen, int H, int NT, int c0, int n, int B, Prologue pro)
{
    using Cfg = IntraCfg<KIND, T, DK, DV>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[Cfg::BYTES];
    const unsigned it = blockIdx.x;
    const int h = (int)(it % (unsigned)H);
    const unsigned t = it / (unsigned)H;
    const int c = c0 + (int)(t % (unsigned)n), b = (int)(t / (unsigned)n);
    const int nvalid = min(kChunk, Tlen - c * kChunk);
    IntraIn<KIND, T, DK, DV> in;
    intra_load<KIND, T, DK, DV>(in, q, k, v, g, beta, ((size_t)b * Tlen + (size_t)c * kChunk) * H + h, nvalid, H);
    ProHead ph{};
    if constexpr (PRO) ph = pro_head(pro, h);
    intra_chunk<KIND, T, DK, DV, PRO>(in, smem, flags,
                                      ws + (((size_t)b * H + h) * NT + c) * Rec<T, DK, DV>::BYTES, nvalid, ph);
}

// 128-token chunks of 64-row sub-chunks ([KDA] 2.3): one 512-thread
// workgroup per (chunk, head, batch), heads fastest; threads 256s .. 256s+255
// load and process sub-chunk s (intra_chunk with C2 = 128).
template <int KIND, typename T, int DK, int DV, bool PRO>
__global__ __launch_bounds__(2 * kThreads, 1) void intra128_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, uint8_t* __restrict__ ws,
    unsigned* __restrict__ flags, int Tlen, int H, int NT, int c0, int n, int B, Prologue pro)
{
    using Cfg = IntraCfg<KIND, T, DK, DV>;
    constexpr int C2 = 2 * kChunk;
    constexpr size_t BYTES = 2 * Cfg::BYTES + 2 * DK * sizeof(float);
    static_assert(BYTES <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(16))) uint8_t smem[BYTES];
    const unsigned it = blockIdx.x;
    const int h = (int)(it % (unsigned)H);
    const unsigned t = it / (unsigned)H;
    const int c = c0 + (int)(t % (unsigned)n), b = (int)(t / (unsigned)n);
    const int nv = min(C2, Tlen - c * C2);
    const int half = (int)(threadIdx.x >> 8);
    const int nvh = min(max(nv - kChunk * half, 0), kChunk);
    const size_t row_chunk = ((size_t)b * Tlen + (size_t)c * C2) * H + h;
    // an empty second sub-chunk loads the chunk's first row (and zeroes it)
    const size_t row0 = nvh > 0 ? row_chunk + (size_t)half * kChunk * H : row_chunk;
    IntraIn<KIND, T, DK, DV> in;
    intra_load<KIND, T, DK, DV>(in, q, k, v, g, beta, row0, max(nvh, 1), H);
    ProHead ph{};
    if constexpr (PRO) ph = pro_head(pro, h);
    intra_chunk<KIND, T, DK, DV, PRO, C2>(in, smem, flags,
                                          ws + (((size_t)b * H + h) * NT + c) * Rec<T, DK, DV, C2>::BYTES, nvh, ph);
}

// Packed sequences: one workgroup per (chunk slot, head), heads fastest.  The
// slot table written by varlen_table_kernel gives each chunk's first token
// and its valid rows; slots past the table's count exit at once.  Records go
// to index h * maxchunks + slot, so each sequence's chunks are contiguous for
// the state pass.
template <int KIND, typename T, int DK, int DV, bool PRO>
__global__ __launch_bounds__(kThreads, 2) void intra_varlen_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, uint8_t* __restrict__ ws,
    unsigned* __restrict__ flags, const int4* __restrict__ table, const int* __restrict__ total, int H,
    int maxchunks, Prologue pro)
{
    using Cfg = IntraCfg<KIND, T, DK, DV>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[Cfg::BYTES];
    const unsigned it = blockIdx.x;
    const int h = (int)(it % (unsigned)H), slot = (int)(it / (unsigned)H);
    if (slot >= *total) return;
    const int4 e = table[slot];     // {sequence, first token, valid rows, -}
    IntraIn<KIND, T, DK, DV> in;
    intra_load<KIND, T, DK, DV>(in, q, k, v, g, beta, (size_t)e.y * H + h, e.z, H);
    ProHead ph{};
    if constexpr (PRO) ph = pro_head(pro, h);
    intra_chunk<KIND, T, DK, DV, PRO>(in, smem, flags, ws + ((size_t)h * maxchunks + slot) * Rec<T, DK, DV>::BYTES,
                                      e.z, ph);
}

}  // namespace dr
