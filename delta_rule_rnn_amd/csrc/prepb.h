// prepb.h -- the backward's prep for bf16 I/O with the segment-parallel
// reverse pass and the bf16 gradient kernel: per chunk, gamma, phi, L,
// Aqk, T = (I + diag(beta) L)^-1 and W = T diag(beta) K+ from q, k, g, beta,
// written as the reverse pass's bf16 operands (RevRec: Kbar, Aqk^T, Q~^T,
// W^T) and the gradient kernel's fp32 arrays (T, L, phi; scalar gates also
// gamma and Aqk).
//
// Page keys as in backward.h: [KDA] "TileLang 实战：KDA 从零到一–Kimi Delta
// Attention" (sections 1.2 and 3.2-3.3: the separable exponents, the
// triangular solve and the WY products); [SD] "TileLang 实战：KDA 从零到一--标量
// 衰减" (the ratio form of scalar gates); [GDN] "Gated DeltaNet".
//
// The quantities and their precision are those of bwd_prep_kernel
// (backward.h): Aqk under per-channel gates is formed from split bf16
// operands (q 2^gamma and k 2^-gamma are off the bf16 grid; their high and
// low bf16 parts, three MFMAs per step, keep about 16 bits, which the small
// Aqk of nearly orthogonal rows needs), L on bf16 MFMA, T in fp32 (the
// diagonal blocks by forward substitution, the others by block distance on
// fp32 MFMA), W from bf16 M = diag(beta) K+ and T split into high and low
// parts.
//
// Layout: one 256-thread workgroup per (chunk, head), 77 KB of LDS at d =
// 128 so that two share a CU.  Each thread loads CPT = d/32 adjacent
// channels at 8 consecutive positions (one vector load per position), so
// Kbar leaves as one CPT-channel store per position and Q~^T as one 16-byte
// store per channel.  The four [C][d] bf16 LDS regions R0..R3 are reused:
//   R0  Q~ high (Aqk)           -> beta L fp32 [C][C+4] (T solve)
//   R1  Q~ low  (Aqk)           -> K+ (L)          -> block scratch (T solve)
//   R2  K- high (Aqk, L)        -> T fp32 [C][C+4] (T solve, W)
//   R3  K- low  (Aqk)           -> M^T = (diag(beta) K+)^T [d][C] (W)
// Scalar gates keep raw q in R0 and raw k in R2 (Aqk = (q k^T) 2^(gi - gj),
// L = (k k^T) 2^(gi - gj) on or below the diagonal).
#pragma once

#include "gradb.h"

namespace dr {
namespace bw {

constexpr int kPrepbThreads = 256;

template <int KIND, int DK>
struct PrepbSmem {
    static constexpr int LDK = DK + 8;               // bf16 row of a [C][DK] region
    static constexpr int LDQ = C + 8;                // bf16 row of a [DK][C] region
    static constexpr int LDF = C + 4;                // fp32 row of a [C][C] array
    static constexpr int mx(int a, int b) { return a > b ? a : b; }
    // one region: a [C][LDK] or [DK][LDQ] bf16 array, or a [C][LDF] fp32 one
    static constexpr int RB = mx(mx(C * LDK * 2, DK * LDQ * 2), C * LDF * 4);
    static constexpr int R0 = 0, R1 = RB, R2 = 2 * RB, R3 = 3 * RB;
    static constexpr int CPT = DK / 32, NQ = kPrepbThreads / 32, PL = C / NQ;
    static constexpr int TOT = 4 * RB;               // [NQ][DK] gate totals (kda)
    static constexpr int BETA = TOT + NQ * DK * 4, GAM = BETA + C * 4, BYTES = GAM + C * 4;
    static_assert(PL == 8, "eight positions per thread");
    static_assert(BYTES <= 80 * 1024, "two workgroups per CU");
};

template <int KIND, int DK>
__global__ __launch_bounds__(kPrepbThreads, 2) void bwd_prepb_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v, const float* __restrict__ g,
    const float* __restrict__ beta, float* __restrict__ prep, bf16* __restrict__ rrec, uint8_t* __restrict__ recs,
    int Tlen, int H, int NT, Pack pk)
{
    using P = Prep<DK>;
    using RR = RevRec<DK>;
    using SM = PrepbSmem<KIND, DK>;
    constexpr int LDK = SM::LDK, LDQ = SM::LDQ, LDF = SM::LDF, CPT = SM::CPT, NQ = SM::NQ, PL = SM::PL;
    constexpr bool DELTA = KIND != KIND_LA;
    constexpr bool PERCH = KIND == KIND_KDA;
    using VT = typename VecOf<bf16, CPT>::type;
    using VG = typename VecOf<float, CPT>::type;
    __shared__ __attribute__((aligned(16))) char smem[SM::BYTES];
    bf16* r0 = reinterpret_cast<bf16*>(smem + SM::R0);
    bf16* r1 = reinterpret_cast<bf16*>(smem + SM::R1);
    bf16* r2 = reinterpret_cast<bf16*>(smem + SM::R2);
    bf16* r3 = reinterpret_cast<bf16*>(smem + SM::R3);
    float* sTot = reinterpret_cast<float*>(smem + SM::TOT);
    float* sBeta = reinterpret_cast<float*>(smem + SM::BETA);
    float* sGam = reinterpret_cast<float*>(smem + SM::GAM);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, g4 = lane >> 4;
    ChunkLoc loc;
    if (!locate_chunk(pk, blockIdx.x, H, Tlen, NT, loc)) return;
    const int nvalid = loc.nvalid;
    const size_t row0 = loc.row0;
    float* out = prep + loc.ci * P::FLOATS;
    bf16* rr = rrec + loc.ci * RR::ELEMS;
    // the forward state pass's record of this chunk (its W, Kbar^T, U^T and
    // phi fields, in the fragment order that pass reads), or null
    using Rc = Rec<bf16, DK, DK>;
    uint8_t* recb = recs ? recs + loc.ci * Rc::BYTES : nullptr;
    bf16* rcW = recb ? reinterpret_cast<bf16*>(recb) + Rc::W : nullptr;
    bf16* rcKb = recb ? reinterpret_cast<bf16*>(recb) + Rc::KBT : nullptr;
    bf16* rcU = recb ? reinterpret_cast<bf16*>(recb) + Rc::UT : nullptr;

    // ---- inputs: channels ch0 .. ch0 + CPT - 1 at positions p0 .. p0 + 7;
    // rows past the end load the last valid row and are zeroed
    const int cg = tid % 32, qg = tid / 32, ch0 = CPT * cg, p0 = PL * qg;
    VT kv[PL], qv[PL], vv[PL];
    VG gv[PERCH ? PL : 1];
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        const size_t off = (row0 + (size_t)min(p0 + i, nvalid - 1) * H) * DK + ch0;
        if constexpr (PERCH) gv[i] = *reinterpret_cast<const VG*>(g + off);
        kv[i] = *reinterpret_cast<const VT*>(k + off);
        qv[i] = *reinterpret_cast<const VT*>(q + off);
    }
    // v only for the record (U = T diag(beta) V; decay_la: V itself)
    if (recb) {
#pragma unroll
        for (int i = 0; i < PL; ++i)
            vv[i] = *reinterpret_cast<const VT*>(v + (row0 + (size_t)min(p0 + i, nvalid - 1) * H) * DK + ch0);
    }
    if (tid < C) {
        const float bb = DELTA ? beta[row0 + (size_t)min(tid, nvalid - 1) * H] : 0.f;
        sBeta[tid] = tid < nvalid ? bb : 0.f;
    }
    if constexpr (!PERCH) {
        if (w == 0) {
            const float gs = g[row0 + (size_t)min(lane, nvalid - 1) * H];
            float x = lane < nvalid ? gs : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off, 64);
                if (lane >= off) x += y;
            }
            x *= kLog2e;
            sGam[lane] = x;
            out[P::GAM + lane] = x;
        }
    }
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        if (p0 + i >= nvalid) {
            kv[i] = VT{};
            qv[i] = VT{};
            vv[i] = VT{};
            if constexpr (PERCH) gv[i] = VG{};
        }
    }

    // ---- gamma (log2): per-channel cumsum over this thread's 8 positions,
    // then the totals of the position groups before it (kda); scalar gates
    // from the wave-0 scan
    float gam[PL][CPT], glast[CPT];
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
        VG tv;
#pragma unroll
        for (int j = 0; j < CPT; ++j) tv[j] = sc[j];
        *reinterpret_cast<VG*>(sTot + qg * DK + ch0) = tv;
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
        lds_barrier();
#pragma unroll
        for (int i = 0; i < PL; ++i)
#pragma unroll
            for (int j = 0; j < CPT; ++j) gam[i][j] = sGam[p0 + i];
#pragma unroll
        for (int j = 0; j < CPT; ++j) glast[j] = sGam[C - 1];
    }

    // ---- per element: Kbar (RevRec, natural), Q~^T (RevRec), phi; the
    // Aqk operands to LDS (kda: Q~ and K- split into high and low parts;
    // scalar gates: raw q and k)
    {
        float phi[CPT];
#pragma unroll
        for (int j = 0; j < CPT; ++j) phi[j] = __builtin_amdgcn_exp2f(glast[j]);
        float qt[CPT][PL], kbt[CPT][PL];
#pragma unroll
        for (int i = 0; i < PL; ++i) {
            const int p = p0 + i;
            VT kb;
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                const float kk = (float)kv[i][j], qq = (float)qv[i][j];
                const float e = __builtin_amdgcn_exp2f(gam[i][j]), ei = __builtin_amdgcn_exp2f(-gam[i][j]);
                qt[j][i] = qq * e;
                // Kbar = (k 2^-gamma) 2^gamma_last, as the prep's (scalar
                // gates: k 2^(gamma_last - gamma))
                kbt[j][i] = PERCH ? kk * ei * phi[j] : kk * __builtin_amdgcn_exp2f(glast[j] - gam[i][j]);
                kb[j] = (bf16)kbt[j][i];
            }
            *reinterpret_cast<VT*>(rr + RR::KB + (size_t)p * DK + ch0) = kb;
            if constexpr (PERCH) {
                VT qh, ql, kh, kl;
#pragma unroll
                for (int j = 0; j < CPT; ++j) {
                    const float km = (float)kv[i][j] * __builtin_amdgcn_exp2f(-gam[i][j]);
                    qh[j] = (bf16)qt[j][i];
                    ql[j] = (bf16)(qt[j][i] - (float)qh[j]);
                    kh[j] = (bf16)km;
                    kl[j] = (bf16)(km - (float)kh[j]);
                }
                *reinterpret_cast<VT*>(r0 + p * LDK + ch0) = qh;
                *reinterpret_cast<VT*>(r1 + p * LDK + ch0) = ql;
                *reinterpret_cast<VT*>(r2 + p * LDK + ch0) = kh;
                *reinterpret_cast<VT*>(r3 + p * LDK + ch0) = kl;
            } else {
                *reinterpret_cast<VT*>(r0 + p * LDK + ch0) = qv[i];
                *reinterpret_cast<VT*>(r2 + p * LDK + ch0) = kv[i];
            }
        }
        // Q~^T: this thread's eight positions of each channel, one store
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            bf16x8 x;
#pragma unroll
            for (int i = 0; i < PL; ++i) x[i] = (bf16)qt[j][i];
            *reinterpret_cast<bf16x8*>(rr + RR::QT + (size_t)(ch0 + j) * C + p0) = x;
        }
        if (qg == 0) {
            VG ph;
#pragma unroll
            for (int j = 0; j < CPT; ++j) ph[j] = phi[j];
            *reinterpret_cast<VG*>(out + P::PHI + ch0) = ph;
            if (recb) *reinterpret_cast<VG*>(reinterpret_cast<float*>(recb + Rc::PHI_BYTE) + ch0) = ph;
        }
        if (recb) {
            // the record's Kbar^T: channel ch is row prow(h, r) of key block
            // ch/32 there, and this thread's eight positions are one
            // fragment slot run (one 16-byte store per channel)
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                const int ch = ch0 + j, qq = ch & 31;
                const int wk = ch >> 5, hh = (qq >> 2) & 1, rl = 4 * (qq >> 3) + (qq & 3);
                bf16x8 x;
#pragma unroll
                for (int i = 0; i < PL; ++i) x[i] = (bf16)kbt[j][i];
                *reinterpret_cast<bf16x8*>(rcKb + ((size_t)((wk * 2 + hh) * (C / 32) + (p0 >> 5)) * 64 + rl +
                                                   16 * ((p0 & 31) >> 3)) * 8) = x;
            }
            if constexpr (!DELTA) {
                // decay_la: the state pass reads V from the U slot: U[32(w/2) +
                // 8(l/16) + 4(w%2) + i][16t + l%16], four positions per store
#pragma unroll
                for (int j = 0; j < CPT; ++j) {
                    const int ch = ch0 + j;
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf) {
                        bf16x4 x;
#pragma unroll
                        for (int i = 0; i < 4; ++i) x[i] = vv[4 * hf + i][j];
                        const int wv = 2 * (p0 >> 5) + hf;
                        *reinterpret_cast<bf16x4*>(rcU + ((size_t)((ch >> 4) * 4 + wv) * 64 + (ch & 15) +
                                                          16 * ((p0 & 31) >> 3)) * 4) = x;
                    }
                }
            }
        }
    }
    lds_barrier();

    // ---- Aqk over the ten tiles on or below the diagonal (tile ids w, w+4,
    // w+8), Aqk^T to RevRec (zeros for the six tiles above); scalar gates
    // also the fp32 Aqk of the lower tiles for the gradient kernel
#pragma unroll
    for (int t = 0; t < 3; ++t) {
        const int id = w + 4 * t;
        if (id < 10) {
            int it, jt;
            tile_lo(id, it, jt);
            f32x4 acc = zero4();
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks) {
                const int ko = 32 * ks + 8 * g4;
                const bf16x8 ah = ld8(r0 + (16 * it + l16) * LDK + ko), bh = ld8(r2 + (16 * jt + l16) * LDK + ko);
                acc = mf(ah, bh, acc);
                if constexpr (PERCH) {
                    acc = mf(ah, ld8(r3 + (16 * jt + l16) * LDK + ko), acc);
                    acc = mf(ld8(r1 + (16 * it + l16) * LDK + ko), bh, acc);
                }
            }
            const int j = 16 * jt + l16;
            f32x4 x;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * it + 4 * g4 + r;
                float a = j <= i ? acc[r] : 0.f;
                if constexpr (!PERCH) {
                    a *= j <= i ? __builtin_amdgcn_exp2f(sGam[i] - sGam[j]) : 0.f;
                    out[P::AQK + (size_t)i * C + j] = a;
                }
                x[r] = a;
            }
            *reinterpret_cast<bf16x4*>(rr + RR::AT + (size_t)j * C + 16 * it + 4 * g4) = pack4(x);
        }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int id = w + 4 * t;
        if (id < 6) {
            int it, jt;
            tile_up(id, it, jt);
            *reinterpret_cast<bf16x4*>(rr + RR::AT + (size_t)(16 * jt + l16) * C + 16 * it + 4 * g4) =
                pack4(zero4());
        }
    }
    if constexpr (!DELTA) return;
    lds_barrier();

    // ---- K+ (kda) to R1 for L; M^T = (diag(beta) K+)^T to R3 for W, eight
    // positions of a channel per store (scalar gates: K+ = k 2^gamma_r)
    {
        float mt[CPT][PL];
#pragma unroll
        for (int i = 0; i < PL; ++i) {
            const float bt = sBeta[p0 + i];
            VT kp;
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                const float x = (float)kv[i][j] * __builtin_amdgcn_exp2f(gam[i][j]);
                kp[j] = (bf16)x;
                mt[j][i] = bt * x;
            }
            if constexpr (PERCH) *reinterpret_cast<VT*>(r1 + (p0 + i) * LDK + ch0) = kp;
        }
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            bf16x8 x;
#pragma unroll
            for (int i = 0; i < PL; ++i) x[i] = (bf16)mt[j][i];
            *reinterpret_cast<bf16x8*>(r3 + (ch0 + j) * LDQ + p0) = x;
        }
    }
    lds_barrier();

    // ---- L = StrictLower(K+ K-^T) (scalar gates: (k k^T) 2^(gi - gj)): fp32
    // L of all sixteen tiles to the gradient kernel (zeros above), beta L to
    // R0 for the solve
    float* sA = reinterpret_cast<float*>(smem + SM::R0);
    {
        const bf16* kpl = PERCH ? r1 : r2;
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            const int id = w + 4 * t;
            if (id < 10) {
                int it, jt;
                tile_lo(id, it, jt);
                f32x4 acc = zero4();
#pragma unroll
                for (int ks = 0; ks < DK / 32; ++ks) {
                    const int ko = 32 * ks + 8 * g4;
                    acc = mf(ld8(kpl + (16 * it + l16) * LDK + ko), ld8(r2 + (16 * jt + l16) * LDK + ko), acc);
                }
                const int j = 16 * jt + l16;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * it + 4 * g4 + r;
                    float x = j < i ? acc[r] : 0.f;
                    if constexpr (!PERCH) x *= j < i ? __builtin_amdgcn_exp2f(sGam[i] - sGam[j]) : 0.f;
                    out[P::L + (size_t)i * C + j] = x;
                    sA[i * LDF + j] = sBeta[i] * x;
                }
            }
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int id = w + 4 * t;
            if (id < 6) {
                int it, jt;
                tile_up(id, it, jt);
#pragma unroll
                for (int r = 0; r < 4; ++r) out[P::L + (size_t)(16 * it + 4 * g4 + r) * C + 16 * jt + l16] = 0.f;
            }
        }
    }
    lds_barrier();

    // ---- T = (I + A)^-1, A = diag(beta) L, blocked over 16 x 16 blocks:
    // the diagonal blocks by forward substitution (wave 0, one column per
    // lane), the blocks above the diagonal zero (waves 1-3), then by block
    // distance T_ij = -T_ii sum_{j <= m < i} A_im T_mj on fp32 MFMA
    float* sT = reinterpret_cast<float*>(smem + SM::R2);
    float* sX = reinterpret_cast<float*>(smem + SM::R1);
    if (w == 0) {
        const int o = g4 * 16, jc = l16;
        float tc[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float s = 0.f;
#pragma unroll
            for (int m = 0; m < i; ++m) s += sA[(o + i) * LDF + o + m] * tc[m];
            tc[i] = i < jc ? 0.f : (i == jc ? 1.f : -s);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sT[(o + i) * LDF + o + jc] = tc[i];
    } else {
        for (int idx = tid - 64; idx < 6 * 256; idx += kPrepbThreads - 64) {
            int bi, bj;
            tile_up(idx >> 8, bi, bj);
            const int e = idx & 255;
            sT[(16 * bi + (e >> 4)) * LDF + 16 * bj + (e & 15)] = 0.f;
        }
    }
    lds_barrier();
#pragma unroll
    for (int dist = 1; dist < 4; ++dist) {
        const int bi = dist + w, bj = w;          // block (bi, bj), one per wave
        if (bi < 4) {
            f32x4 x = zero4();
            for (int m = bj; m < bi; ++m)
                x = mmk<16>(x, sA + 16 * bi * LDF + 16 * m, LDF, 1, sT + 16 * m * LDF + 16 * bj, LDF, 1, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) sX[w * 256 + (4 * g4 + r) * 16 + l16] = x[r];
        }
        lds_barrier();
        if (bi < 4) {
            const f32x4 y = mmk<16>(zero4(), sT + 16 * bi * LDF + 16 * bi, LDF, 1, sX + w * 256, 16, 1, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) sT[(16 * bi + 4 * g4 + r) * LDF + 16 * bj + l16] = -y[r];
        }
        lds_barrier();
    }
    // T to the gradient kernel, four elements per store
#pragma unroll
    for (int it_ = 0; it_ < (C * C) / (4 * kPrepbThreads); ++it_) {
        const int idx = tid + it_ * kPrepbThreads, r = idx >> 4, c4 = (idx & 15) * 4;
        *reinterpret_cast<f32x4*>(out + P::TI + (size_t)r * C + c4) = *reinterpret_cast<const f32x4*>(sT + r * LDF + c4);
    }

    // ---- the record's W and U^T (T split into bf16 high and low parts):
    // W^T = M^T T^T over tiles whose rows (channels) follow prow() and whose
    // columns (positions) follow pw(), so that a lane's two accumulators of a
    // key block are its fragment-order slot run of W; U = T (diag(beta) V)
    // with rows in pw() order, as the record's U^T slots
    if (recb) {
        // (beta V)^T to R0 (beta L, read by the solve, is dead)
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            bf16x8 x;
#pragma unroll
            for (int i = 0; i < PL; ++i) x[i] = (bf16)(sBeta[p0 + i] * (float)vv[i][j]);
            *reinterpret_cast<bf16x8*>(r0 + (ch0 + j) * LDQ + p0) = x;
        }
        lds_barrier();
        // the T row of position pos, k-step ks, split into high and low parts
        auto trow = [&](int pos, int ks, bf16x8& hi, bf16x8& lo) {
            const int ko = 32 * ks + 8 * g4;
            const f32x4 a0 = *reinterpret_cast<const f32x4*>(sT + pos * LDF + ko);
            const f32x4 a1 = *reinterpret_cast<const f32x4*>(sT + pos * LDF + ko + 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                hi[j] = (bf16)a0[j];
                hi[4 + j] = (bf16)a1[j];
                lo[j] = (bf16)(a0[j] - (float)hi[j]);
                lo[4 + j] = (bf16)(a1[j] - (float)hi[4 + j]);
            }
        };
        constexpr int NKB = DK / 32;
#pragma unroll 1
        for (int pi = w; pi < 4 * NKB; pi += 4) {
            const int wr = pi / NKB, kb = pi % NKB, pos = pw(wr, l16);
            f32x4 acc[2] = {zero4(), zero4()};
            for (int ks = 0; ks <= (wr >> 1); ++ks) {       // T[pos][j] = 0 for j > pos
                bf16x8 bh, bl;
                trow(pos, ks, bh, bl);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const bf16x8 a = ld8(r3 + (32 * kb + prow(h, l16)) * LDQ + 32 * ks + 8 * g4);
                    acc[h] = mf(a, bh, acc[h]);
                    acc[h] = mf(a, bl, acc[h]);
                }
            }
            bf16x8 f;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int r = 0; r < 4; ++r) f[4 * h + r] = (bf16)acc[h][r];
            *reinterpret_cast<bf16x8*>(rcW + ((size_t)(wr * NKB + kb) * 64 + lane) * 8) = f;
        }
#pragma unroll 1
        for (int ui = w; ui < 4 * (DK / 16); ui += 4) {
            const int wr = ui & 3, t = ui >> 2, pos = pw(wr, l16);
            f32x4 acc = zero4();
            for (int ks = 0; ks <= (wr >> 1); ++ks) {
                bf16x8 ah, al;
                trow(pos, ks, ah, al);
                const bf16x8 b = ld8(r0 + (16 * t + l16) * LDQ + 32 * ks + 8 * g4);
                acc = mf(ah, b, acc);
                acc = mf(al, b, acc);
            }
            *reinterpret_cast<bf16x4*>(rcU + ((size_t)(t * 4 + wr) * 64 + lane) * 4) = pack4(acc);
        }
    }

    // ---- W = T M over (C/16) x (DK/16) tiles, eight per wave (T split into
    // bf16 high and low parts; M^T rows from R3), W^T to RevRec
    constexpr int NDT = DK / 16;
#pragma unroll 1
    for (int t = w; t < 4 * NDT; t += 4) {
        const int it = t / NDT, dt = t % NDT;
        f32x4 acc = zero4();
        for (int ks = 0; ks <= (16 * it + 15) >> 5; ++ks) {     // T[i][j] = 0 for j > i
            const int ko = 32 * ks + 8 * g4;
            const f32x4 a0 = *reinterpret_cast<const f32x4*>(sT + (16 * it + l16) * LDF + ko);
            const f32x4 a1 = *reinterpret_cast<const f32x4*>(sT + (16 * it + l16) * LDF + ko + 4);
            bf16x8 ah, al;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                ah[j] = (bf16)a0[j];
                ah[4 + j] = (bf16)a1[j];
                al[j] = (bf16)(a0[j] - (float)ah[j]);
                al[4 + j] = (bf16)(a1[j] - (float)ah[4 + j]);
            }
            const bf16x8 b = ld8(r3 + (16 * dt + l16) * LDQ + ko);
            acc = mf(ah, b, acc);
            acc = mf(al, b, acc);
        }
        *reinterpret_cast<bf16x4*>(rr + RR::WT + (size_t)(16 * dt + l16) * C + 16 * it + 4 * g4) = pack4(acc);
    }
}

}  // namespace bw
}  // namespace dr
