// revseg.h -- the segment-parallel reverse state pass of the backward (bf16
// I/O, dense [B, T] layout).  Three kernels give the exit adjoints dS'_c,
// dVnew_c and dh0 that bwd_state_rev_kernel gives, without its value slices:
// each workgroup holds whole heads, so every chunk's operands are fetched
// once per pass instead of once per slice.
//
// Page keys: [GDN] "Gated DeltaNet" (section "反向传播：状态伴随与三角变换梯度":
// the state adjoint runs backwards over the chunks); [DPLR]
// "RNN的复兴04:线性注意力并行计算DPLR" (section 2: a run of chunks acts on
// the state through the product of their transitions).
//
// Per chunk, with D the adjoint of the chunk's exit state ([DK, DV]):
//   Y = Kbar D + Aqk^T dO               (dVnew)
//   D <- Diag(phi) D - W^T Y + Q~^T dO   (the adjoint of its entry state)
// an affine map of D.  The chunks of each chain are grouped into NS segments
// of L consecutive chunks (as the segment-parallel forward groups them).
//   rev_seg_kernel<MAPS>  one 512-thread workgroup per (chain, segment
//                         r >= 1): the segment's chunks backwards from the
//                         augmented X = [P | D] = [I | 0]; X at the segment's
//                         start is [Pi_r | N_r]: with E_r the adjoint that
//                         enters segment r from its right end, the adjoint
//                         at its start is Pi_r E_r + N_r.
//   rev_compose_kernel    per (chain, 16 value columns): E_{NS-1} = dhT (or
//                         0), E_{r-1} = Pi_r E_r + N_r; every E_r is written.
//   rev_seg_kernel<OUT>   one workgroup per (chain, segment): the segment's
//                         chunks backwards from D = E_r, storing dS'_c = D
//                         and dVnew_c = Y of every chunk (bf16, the I/O
//                         dtype), and dh0 (fp32: the D left at the start of
//                         segment 0).
// Products run on bf16 MFMA with fp32 accumulation: the chunk operands come
// as bf16 (bwd_prep_kernel's RevRec), X and Y are rounded to bf16 as they
// are read (as the forward's state products round S), X stays fp32 in the
// accumulators across the chunks.
#pragma once

#include "backward.h"
#include "seg.h"

namespace dr {
namespace bw {

constexpr int kRevThreads = 512;     // 8 waves, one workgroup per CU

// Per-wave columns of X, and the LDS plan (bytes) of rev_seg_kernel.
template <int DK, bool MAPS>
struct RevCfg {
    static constexpr int DV = DK;
    static constexpr int NCOL = MAPS ? DK + DV : DV;      // columns of X
    static constexpr int NTW = NCOL >= 256 ? 2 : 1;       // 16-column tiles per wave
    static constexpr int NCW = 16 * NTW;
    static constexpr int NACT = NCOL / NCW;               // waves that hold columns
    static constexpr int LDK = DK + 8, LDC = C + 8;       // padded rows (bf16 elements)
    static constexpr size_t R_KB = 0;                                  // Kbar  [C][LDK]
    static constexpr size_t R_AT = R_KB + (size_t)C * LDK * 2;        // Aqk^T [C][LDC]
    static constexpr size_t R_QT = R_AT + (size_t)C * LDC * 2;        // Q~^T  [DK][LDC]
    static constexpr size_t R_WT = R_QT + (size_t)DK * LDC * 2;       // W^T   [DK][LDC]
    static constexpr size_t R_DO = R_WT + (size_t)DK * LDC * 2;       // dO^T  [DV][LDC]
    static constexpr size_t R_PHI = R_DO + (size_t)DV * LDC * 2;      // phi   [DK] fp32
    static constexpr size_t BYTES = R_PHI + (size_t)DK * 4;
    static_assert(NACT <= kRevThreads / 64 && NCOL % NCW == 0 && (!MAPS || NACT % 2 == 0), "column split");
    static_assert(BYTES <= 160 * 1024, "LDS");
};

// One chunk's operands as the threads hold them between their load (one
// chunk ahead) and their store into LDS: the record in 16-byte units
// (consecutive threads, consecutive units: one contiguous read), two dO rows
// of eight channels, four values of phi.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
template <int KIND, int DK>
struct RevIn {
    using RR = RevRec<DK>;
    static constexpr bool DELTA = KIND != KIND_LA;
    static constexpr size_t ELEMS = DELTA ? RR::ELEMS : RR::WT;       // decay_la: no W
    static constexpr int NU = (int)(ELEMS / 8 / kRevThreads);
    static constexpr int NUD = (C / 2) * (DK / 8);                    // dO units (position pair, 8 channels)
    static_assert(NU * 8 * kRevThreads == (int)ELEMS, "record units per thread");
    static_assert(NUD <= kRevThreads && (RR::AT / 8) % kRevThreads == 0 && (RR::QT / 8) % kRevThreads == 0 &&
                      (RR::WT / 8) % kRevThreads == 0, "each unit step stays in one array");
    u32x4 rec[NU];
    u32x4 d0, d1;
    f32x4 phi;
};

// Loads of chunk c's operands into registers (every load unconditional:
// threads past the dO units and the phi lanes re-read valid addresses).
template <int KIND, int DK>
__device__ __forceinline__ void rev_load(RevIn<KIND, DK>& in, const bf16* __restrict__ rec,
                                         const float* __restrict__ prep_c, const bf16* __restrict__ dout,
                                         size_t drow0, int nvalid, int H, int tid) {
    using In = RevIn<KIND, DK>;
    constexpr int DV = DK;
    const u32x4* src = reinterpret_cast<const u32x4*>(rec);
#pragma unroll
    for (int j = 0; j < In::NU; ++j) in.rec[j] = src[tid + j * kRevThreads];
    const int u = tid % In::NUD;
    const int p = 2 * (u / (DV / 8)), c8 = u % (DV / 8);
    in.d0 = *reinterpret_cast<const u32x4*>(dout + (drow0 + (size_t)min(p, nvalid - 1) * H) * DV + 8 * c8);
    in.d1 = *reinterpret_cast<const u32x4*>(dout + (drow0 + (size_t)min(p + 1, nvalid - 1) * H) * DV + 8 * c8);
    in.phi = *reinterpret_cast<const f32x4*>(prep_c + Prep<DK>::PHI + 4 * (tid % (DK / 4)));
}

// The registers of rev_load into the LDS plan; dO rows past the end of a
// ragged chunk are zero.
template <int KIND, int DK, bool MAPS>
__device__ __forceinline__ void rev_stage(const RevIn<KIND, DK>& in, uint8_t* smem, int nvalid, int tid) {
    using Cfg = RevCfg<DK, MAPS>;
    using RR = RevRec<DK>;
    using In = RevIn<KIND, DK>;
    constexpr int DV = DK, LDK = Cfg::LDK, LDC = Cfg::LDC;
#pragma unroll
    for (int j = 0; j < In::NU; ++j) {
        const int u = tid + j * kRevThreads;      // unit of 8 elements; j * kRevThreads fixes the array
        constexpr int nkb = (int)(RR::AT / 8), nat = (int)((RR::QT - RR::AT) / 8), nqt = (int)((RR::WT - RR::QT) / 8);
        size_t off;
        if (j * kRevThreads < nkb) {
            off = Cfg::R_KB + ((size_t)(u / (DK / 8)) * LDK + 8 * (u % (DK / 8))) * 2;
        } else if (j * kRevThreads < nkb + nat) {
            const int v = u - nkb;
            off = Cfg::R_AT + ((size_t)(v / (C / 8)) * LDC + 8 * (v % (C / 8))) * 2;
        } else if (j * kRevThreads < nkb + nat + nqt) {
            const int v = u - nkb - nat;
            off = Cfg::R_QT + ((size_t)(v / (C / 8)) * LDC + 8 * (v % (C / 8))) * 2;
        } else {
            const int v = u - nkb - nat - nqt;
            off = Cfg::R_WT + ((size_t)(v / (C / 8)) * LDC + 8 * (v % (C / 8))) * 2;
        }
        *reinterpret_cast<u32x4*>(smem + off) = in.rec[j];
    }
    if (tid < In::NUD) {
        // dO^T: the pair (p, p+1) of each of the 8 channels as one 4-byte store
        const int p = 2 * (tid / (DV / 8)), c8 = tid % (DV / 8);
        const bf16x8 x0 = __builtin_bit_cast(bf16x8, in.d0), x1 = __builtin_bit_cast(bf16x8, in.d1);
        const bf16 z = (bf16)0.f;
        bf16* sDO = reinterpret_cast<bf16*>(smem + Cfg::R_DO);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            bf16x2 pr;
            pr[0] = p < nvalid ? x0[e] : z;
            pr[1] = p + 1 < nvalid ? x1[e] : z;
            *reinterpret_cast<bf16x2*>(sDO + (8 * c8 + e) * LDC + p) = pr;
        }
    }
    if (tid < DK / 4) *reinterpret_cast<f32x4*>(smem + Cfg::R_PHI + 16 * tid) = in.phi;
}

// rev_seg_kernel: one workgroup per (chain, segment r); MAPS: r = 1 .. NS-1
// (the grid holds chains * (NS - 1) workgroups), else r = 0 .. NS-1.
// Packed sequences (pk.table set): OUT only, NS = 1, the chains of
// locate_chain (a sequence without tokens writes dh0 = dhT).
//   rrec  RevRec (bf16) per chunk index;  prep: phi of every chunk (fp32)
//   ein   [chains][NS][DK][DV] fp32: E_r (OUT; with NS = 1 it is dhT, or
//         null for a zero exit adjoint)
//   xmap  [chains][NS][DK][2 DK] fp32: [Pi_r | N_r] (MAPS)
//   dhs   [chains * NT][DK][DV], dvn [chains * NT][C][DV] bf16 (OUT)
//   dh0   [chains][DK][DV] fp32 or null (OUT)
template <int KIND, int DK, bool MAPS>
__global__ __launch_bounds__(kRevThreads, 1) void rev_seg_kernel(
    const bf16* __restrict__ rrec, const float* __restrict__ prep, const bf16* __restrict__ dout,
    const float* __restrict__ ein, float* __restrict__ xmap, bf16* __restrict__ dhs, bf16* __restrict__ dvn,
    float* __restrict__ dh0, int Tlen, int H, int NT, int L, int NS, Pack pk)
{
    using Cfg = RevCfg<DK, MAPS>;
    using RR = RevRec<DK>;
    using P = Prep<DK>;
    constexpr int DV = DK, NKB = DK / 32, NTW = Cfg::NTW, NCW = Cfg::NCW, NACT = Cfg::NACT;
    constexpr int LDK = Cfg::LDK, LDC = Cfg::LDC;
    constexpr bool DELTA = KIND != KIND_LA;
    __shared__ __attribute__((aligned(16))) uint8_t smem[Cfg::BYTES];
    const bf16* sKb = reinterpret_cast<const bf16*>(smem + Cfg::R_KB);
    const bf16* sAT = reinterpret_cast<const bf16*>(smem + Cfg::R_AT);
    const bf16* sQT = reinterpret_cast<const bf16*>(smem + Cfg::R_QT);
    const bf16* sWT = reinterpret_cast<const bf16*>(smem + Cfg::R_WT);
    const bf16* sDO = reinterpret_cast<const bf16*>(smem + Cfg::R_DO);
    const float* sPhi = reinterpret_cast<const float*>(smem + Cfg::R_PHI);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, grp = lane >> 4;
    const int nsg = MAPS ? NS - 1 : NS;
    const int chain = blockIdx.x / nsg;
    const int r = blockIdx.x % nsg + (MAPS ? 1 : 0);
    const int h = chain % H;
    // the chain's chunks: per-chunk index ci0 + c, token rows (tok0 + c C + p) H + h
    size_t ci0, tok0;
    int tlim, cbeg, cend;
    if (pk.table) {
        const ChainLoc cl = locate_chain(pk, chain, H, Tlen, NT);
        ci0 = cl.ci0;
        tok0 = cl.tok0;
        tlim = cl.tlim;
        cbeg = 0;
        cend = cl.nseg;
    } else {
        ci0 = (size_t)chain * NT;
        tok0 = (size_t)(chain / H) * Tlen;
        tlim = Tlen;
        cbeg = r * L;
        cend = min(NT, cbeg + L);     // cbeg < cend: NS = ceil(NT / L)
    }
    // this wave's columns of X: MAPS: waves < NACT/2 hold P, the others D
    const bool active = wave < NACT;
    const bool isD = MAPS ? wave >= NACT / 2 : true;
    const int col0 = (MAPS ? wave % (NACT / 2) : wave) * NCW;

    f32x4 X[NKB][2][NTW];
    const float* e0 = ein ? ein + ((size_t)chain * NS + r) * DK * DV : nullptr;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int n = 0; n < NTW; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 32 * kb + 8 * grp + 4 * hh + i, col = col0 + 16 * n + r16;
                    if constexpr (MAPS) X[kb][hh][n][i] = (!isD && row == col) ? 1.f : 0.f;
                    else X[kb][hh][n][i] = (active && ein) ? e0[(size_t)row * DV + col] : 0.f;
                }

    auto drow0_of = [&](int c) { return (tok0 + (size_t)c * C) * H + h; };
    auto nvalid_of = [&](int c) { return min(C, tlim - c * C); };
    auto load = [&](RevIn<KIND, DK>& in, int c) {
        const size_t ci = ci0 + c;
        rev_load<KIND, DK>(in, rrec + ci * RR::ELEMS, prep + ci * P::FLOATS, dout, drow0_of(c), nvalid_of(c), H, tid);
    };
    RevIn<KIND, DK> in;
    if (cend > cbeg) load(in, cend - 1);    // (a packed sequence may have no tokens)
    for (int c = cend - 1; c >= cbeg; --c) {
        const size_t ci = ci0 + c;
        rev_stage<KIND, DK, MAPS>(in, smem, nvalid_of(c), tid);
        load(in, max(c - 1, cbeg));           // the next chunk (the last reloads itself)
        lds_barrier();
        if (active) {
            if constexpr (!MAPS) {
                // dS'_c: the adjoint of this chunk's exit state
                // (slice-major, slc())
                bf16* dst = dhs + ci * DK * DV;
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                        for (int n = 0; n < NTW; ++n)
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                dst[slc(32 * kb + 8 * grp + 4 * hh + i, col0 + 16 * n + r16, DK)] = (bf16)X[kb][hh][n][i];
            }
            // dO^T fragments of this wave's columns (D columns only)
            Frag<bf16> dof[2][NTW];
            // Y = Kbar X (+ Aqk^T dO), rows: positions 32 kbp + 8 grp + 4 hh + i
            f32x4 Y[2][2][NTW];
#pragma unroll
            for (int kbp = 0; kbp < 2; ++kbp)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int n = 0; n < NTW; ++n) Y[kbp][hh][n] = zero4();
            if (isD) {
#pragma unroll
                for (int kq = 0; kq < 2; ++kq)
#pragma unroll
                    for (int n = 0; n < NTW; ++n)
                        dof[kq][n] = ld_frag(sDO + (col0 + 16 * n + r16) * LDC + 32 * kq + 8 * grp);
                // Aqk^T is zero below its diagonal: key blocks kq >= kbp
#pragma unroll
                for (int kbp = 0; kbp < 2; ++kbp)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                        for (int kq = kbp; kq < 2; ++kq) {
                            const Frag<bf16> fa = ld_frag(sAT + (32 * kbp + prow(hh, r16)) * LDC + 32 * kq + 8 * grp);
#pragma unroll
                            for (int n = 0; n < NTW; ++n) mma(Y[kbp][hh][n], fa, dof[kq][n]);
                        }
            }
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                Frag<bf16> xf[NTW];
#pragma unroll
                for (int n = 0; n < NTW; ++n) xf[n] = pack_frag<bf16>(X[kb][0][n], X[kb][1][n]);
#pragma unroll
                for (int kbp = 0; kbp < 2; ++kbp)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const Frag<bf16> fk = ld_frag(sKb + (32 * kbp + prow(hh, r16)) * LDK + 32 * kb + 8 * grp);
#pragma unroll
                        for (int n = 0; n < NTW; ++n) mma(Y[kbp][hh][n], fk, xf[n]);
                    }
            }
            if constexpr (!MAPS) {
                // dVnew_c (rows past a ragged end are zero: Kbar's and
                // Aqk^T's are)
                bf16* dst = dvn + ci * C * DV;
#pragma unroll
                for (int kbp = 0; kbp < 2; ++kbp)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                        for (int n = 0; n < NTW; ++n)
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                dst[slc(32 * kbp + 8 * grp + 4 * hh + i, col0 + 16 * n + r16, C)] = (bf16)Y[kbp][hh][n][i];
            }
            // X <- Diag(phi) X - W^T Y (+ Q~^T dO)
            Frag<bf16> Yf[2][NTW];
#pragma unroll
            for (int kbp = 0; kbp < 2; ++kbp)
#pragma unroll
                for (int n = 0; n < NTW; ++n) Yf[kbp][n] = pack_frag<bf16>(Y[kbp][0][n], Y[kbp][1][n]);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const f32x4 ph4 = *reinterpret_cast<const f32x4*>(sPhi + 32 * kb + 8 * grp + 4 * hh);
#pragma unroll
                    for (int n = 0; n < NTW; ++n)
#pragma unroll
                        for (int i = 0; i < 4; ++i) X[kb][hh][n][i] *= ph4[i];
                    if constexpr (DELTA) {
#pragma unroll
                        for (int kbp = 0; kbp < 2; ++kbp) {
                            const Frag<bf16> fw =
                                frag_neg(ld_frag(sWT + (32 * kb + prow(hh, r16)) * LDC + 32 * kbp + 8 * grp));
#pragma unroll
                            for (int n = 0; n < NTW; ++n) mma(X[kb][hh][n], fw, Yf[kbp][n]);
                        }
                    }
                    if (isD) {
#pragma unroll
                        for (int kq = 0; kq < 2; ++kq) {
                            const Frag<bf16> fq = ld_frag(sQT + (32 * kb + prow(hh, r16)) * LDC + 32 * kq + 8 * grp);
#pragma unroll
                            for (int n = 0; n < NTW; ++n) mma(X[kb][hh][n], fq, dof[kq][n]);
                        }
                    }
                }
        }
        lds_barrier();   // the LDS operands are rewritten for the next chunk
    }
    if (!active) return;
    float* dst = nullptr;
    size_t ld = DV;
    if constexpr (MAPS) {
        dst = xmap + ((size_t)chain * NS + r) * DK * (2 * DK) + (isD ? DK : 0) + col0 + r16;
        ld = 2 * DK;
    } else {
        if (r != 0 || dh0 == nullptr) return;
        dst = dh0 + (size_t)chain * DK * DV + col0 + r16;
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int n = 0; n < NTW; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[(size_t)(32 * kb + 8 * grp + 4 * hh + i) * ld + 16 * n] = X[kb][hh][n][i];
}

// rev_compose_kernel: per (chain, 16 value columns c0..): E = dhT (or 0);
// ein[NS-1] = E; for r = NS-1 .. 1: E <- Pi_r E + N_r, ein[r-1] = E.  fp32
// MFMA (16x16x4) with fp32 operands; 256 threads, wave w owns the row tiles
// w*TPW .. of E (accumulators); the B operand, E's slice transposed, goes
// through LDS.
constexpr int kRevComposeThreads = 256;
template <int DK>
__global__ __launch_bounds__(kRevComposeThreads) void rev_compose_kernel(const float* __restrict__ xmap,
                                                                         const float* __restrict__ dhT,
                                                                         float* __restrict__ ein, int NS)
{
    constexpr int DV = DK, LDX = 2 * DK, NKB = DK / 32, NRT = DK / 16, TPW = NRT / 4, NSL = DV / 16;
    constexpr int LDT = DK + 4;
    static_assert(NRT % 4 == 0, "row tiles per wave");
    __shared__ __attribute__((aligned(16))) float sET[16 * LDT];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, grp = lane >> 4;
    // the NSL slices of a chain read the same maps: consecutive logical
    // ids, so they share one XCD's L2
    const int lb = xcd_logical(blockIdx.x, gridDim.x);
    const int chain = lb / NSL, c0 = (lb % NSL) * 16;
    auto trow = [&](int t) { return 16 * (wave * TPW + t); };
    f32x4 E[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            E[t][i] = dhT ? dhT[((size_t)chain * DK + trow(t) + 4 * grp + i) * DV + c0 + r16] : 0.f;
    auto put = [&](int rr) {
        float* e = ein + ((size_t)chain * NS + rr) * DK * DV + c0 + r16;
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) e[(size_t)(trow(t) + 4 * grp + i) * DV] = E[t][i];
    };
    put(NS - 1);
    for (int rr = NS - 1; rr >= 1; --rr) {
        const float* xm = xmap + ((size_t)chain * NS + rr) * DK * LDX;
#pragma unroll
        for (int t = 0; t < TPW; ++t) *reinterpret_cast<f32x4*>(sET + r16 * LDT + trow(t) + 4 * grp) = E[t];
        lds_barrier();
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            f32x4 acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = xm[(size_t)(trow(t) + 4 * grp + i) * LDX + DK + c0 + r16];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
                mma(acc, ld_frag(xm + (size_t)(trow(t) + r16) * LDX + 32 * kb + 8 * grp),
                    ld_frag(sET + r16 * LDT + 32 * kb + 8 * grp));
            E[t] = acc;
        }
        lds_barrier();
        put(rr - 1);
    }
}

}  // namespace bw
}  // namespace dr
