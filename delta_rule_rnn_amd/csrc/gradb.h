// gradb.h -- the gradient kernel of the backward for bf16 I/O: dq, dk, dv,
// dbeta and dg of every chunk, from the entry states S_c, Vnew_c and the exit
// adjoints dS'_c, dVnew_c (per-chunk arrays in bf16) and the prep's fp32
// gamma, phi, L, T (and Aqk for scalar gates).
//
// Page keys as in backward.h: [GDN] "Gated DeltaNet", section
// "反向传播：状态伴随与三角变换梯度" (the per-chunk gradients, the WY-
// representation backward through the triangular inverse, the gate gradient
// as a reverse cumulative sum inside each chunk); [KDA] "TileLang 实战：KDA
// 从零到一–Kimi Delta Attention" (the separable per-channel exponents).
//
// The chain rule is the one of bwd_grad_kernel (backward.h), with one
// change of route: P = N - M S (N = diag(beta) V, M = diag(beta) K+), the
// operand of dT = dVnew P^T, is formed as P = (I + diag(beta) L) Vnew.  Since
// Vnew = U - W S = T (N - M S) with T = (I + diag(beta) L)^-1, the two are the
// same matrix; this one is a C x C product over the value slice in place of
// a C x Dk one, and needs neither K+ nor S transposed in LDS.
//
// Layout for the MFMA (v_mfma_f32_16x16x32_bf16; fragment and accumulator
// conventions of common.h):
// - One 256-thread workgroup (four waves) per (chunk, head); about 78 KB of
//   LDS at d = 128, so that two workgroups share a CU and each one's waits
//   overlap the other's work.
// - Operands are bf16 in LDS (the per-chunk arrays and q, k, v, dO are bf16
//   already; T is split into high and low bf16 parts for the product that
//   reaches dv), each stored so that the product reads it along contiguous
//   elements, with rows padded by 16 bytes.
// - Wave w owns the key columns of column tiles w and w + 4 (d = 128; tile w
//   at d = 64) of every [C][Dk] result (all 64 rows).  Its tile rows are permuted by prow(): tile (s, h) row r holds
//   chunk row 32 s + prow(h, r), so a lane's accumulators of the two tiles of
//   block s hold rows 32 s + 8 (l/16) + 0..7 of its column, which is a
//   natural B fragment.  The later products over chunk positions (T^T dW,
//   dL K-, dL^T K+, dAqk K-, dAqk^T Q~) therefore take their B operands
//   from the wave's own registers (nW; K-, K+, Q~ formed per element), and
//   only their [C][C] A operands come from LDS.  The per-column sums of dg
//   (the gamma_last term and the reverse cumulative sum down the rows) stay
//   inside the wave.
// - [C][C] results are taken over the ten 16 x 16 tiles on or below the
//   diagonal (tile ids w, w + 4, w + 8 per wave); the six above it are
//   written as zeros, so every LDS operand is fully defined.
#pragma once

#include "backward.h"

namespace dr {
namespace bw {

constexpr int kGradbThreads = 256;

__device__ __forceinline__ bf16x8 ld8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ bf16x4 ld4b(const bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }
__device__ __forceinline__ f32x4 mf(const bf16x8& a, const bf16x8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 zero8() {
    bf16x8 z;
#pragma unroll
    for (int j = 0; j < 8; ++j) z[j] = (bf16)0.f;
    return z;
}
__device__ __forceinline__ bf16x4 pack4(f32x4 x) {
    bf16x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = (bf16)x[j];
    return o;
}
// Tile (it, jt) of the ten on or below the diagonal, id 0..9 in row order.
__device__ __forceinline__ void tile_lo(int id, int& it, int& jt) {
    it = id >= 6 ? 3 : id >= 3 ? 2 : id >= 1 ? 1 : 0;
    jt = id - it * (it + 1) / 2;
}
// Tile (it, jt) of the six above the diagonal, id 0..5.
__device__ __forceinline__ void tile_up(int id, int& it, int& jt) {
    it = id < 3 ? 0 : id < 5 ? 1 : 2;
    jt = id < 3 ? id + 1 : id < 5 ? id - 1 : 3;
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) float lds_f32;   // a float in LDS

// LDS regions (byte offsets) of one workgroup.
template <int KIND, int DK>
struct GradbSmem {
    static constexpr bool SCALAR = KIND != KIND_KDA;
    static constexpr int LC = C + 8;                 // bf16 row of a [*][C] array
    static constexpr int LS = kVS + 8;               // bf16 row of a [*][32] value slice
    static constexpr int CC = C * LC * 2;            // one [C][LC] bf16 array
    // phase 1 (value slices)
    static constexpr int TT = 0;                     // T^T, high part (kept through phase 2)
    static constexpr int TTL = TT + CC;              // T^T, low part
    static constexpr int LH = TTL + CC;              // L
    static constexpr int S = LH + CC;                // S slice  [DK][LS]
    static constexpr int DS = S + DK * LS * 2;       // dS' slice
    static constexpr int VN = DS + DK * LS * 2;      // Vnew slice [C][LS]
    static constexpr int DVN = VN + C * LS * 2;      // dVnew slice
    static constexpr int DO = DVN + C * LS * 2;      // dO slice
    static constexpr int VNT = DO + C * LS * 2;      // Vnew slice transposed [kVS][LC]
    static constexpr int DVNT = VNT + kVS * LC * 2;  // dVnew slice transposed
    static constexpr int END1 = DVNT + kVS * LC * 2;
    // phase 2: T (row-major), dT, Y^T, dL (G_L), dL^T, dAqk (G_Q), dAqk^T
    static constexpr int TR = TT + CC, DT = TR + CC, YT = DT + CC, DL = YT + CC, DLT = DL + CC, DAQ = DLT + CC,
                         DAQT = DAQ + CC, END2 = DAQT + CC;
    // phase 3: dq, dk (bf16) staged row-major over dL .. dAqk^T
    static constexpr int LQ = DK + 8;
    static constexpr int SQ = DL, SK = SQ + C * LQ * 2, END3 = SK + C * LQ * 2;
    static constexpr int BIG0 = END1 > END2 ? END1 : END2;
    static constexpr int BIG = BIG0 > END3 ? BIG0 : END3;
    // fp32 vectors.  dbeta partial slots [NDB][C], each row written by one
    // wave: the value-slice products (slot 0), dM per wave (1..4), dA per
    // wave (5..8); scalar gates: the pair terms' row and column sums per wave,
    // the per-element E row sums per wave, the gamma_last sums per wave
    static constexpr int NDB = 9;
    static constexpr int BT = BIG, GAM = BT + C * 4, PHI = GAM + C * 4, DPHI = PHI + DK * 4,
                         DB = DPHI + DK * 4, ER = DB + NDB * C * 4, EC = ER + (SCALAR ? 4 * C * 4 : 0),
                         RS = EC + (SCALAR ? 4 * C * 4 : 0), FP = RS + (SCALAR ? 4 * C * 4 : 0),
                         BYTES = FP + 16 * 4;
    // the zeroed slots: DB .. BYTES
    static constexpr int NZ = (BYTES - DB) / 4;
    static_assert(BYTES <= 80 * 1024, "two workgroups per CU");
};

template <int KIND, int DK>
__global__ __launch_bounds__(kGradbThreads, 2) void bwd_gradb_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const bf16* __restrict__ dout,
    const float* __restrict__ prep,
    const bf16* __restrict__ hs, const bf16* __restrict__ dhs, const bf16* __restrict__ vn,
    const bf16* __restrict__ dvn, bf16* __restrict__ dq, bf16* __restrict__ dk, bf16* __restrict__ dv,
    float* __restrict__ dg, float* __restrict__ dbeta, int Tlen, int H, int NT, Pack pk)
{
    using P = Prep<DK>;
    using SM = GradbSmem<KIND, DK>;
    constexpr int DV = DK, NCT = DK / 16, CTW = NCT / 4, NVS = DV / kVS, LC = SM::LC, LS = SM::LS;
    constexpr bool DELTA = KIND != KIND_LA;
    constexpr bool PERCH = KIND == KIND_KDA;
    static_assert(NCT % 4 == 0 && DV % kVS == 0, "column tiles per wave");
    __shared__ __attribute__((aligned(16))) char smem[SM::BYTES];
    auto B16 = [&](int off) { return reinterpret_cast<bf16*>(smem + off); };
    auto F32 = [&](int off) { return reinterpret_cast<float*>(smem + off); };
    float* sBt = F32(SM::BT);      // beta, zero past the end and for decay_la
    float* sGam = F32(SM::GAM);    // scalar gates: gamma per row
    float* sPhi = F32(SM::PHI);
    float* sDphi = F32(SM::DPHI);
    float* sDb = F32(SM::DB);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, g4 = lane >> 4;
    ChunkLoc loc;
    if (!locate_chunk(pk, blockIdx.x, H, Tlen, NT, loc)) return;
    const int nvalid = loc.nvalid;
    const size_t row0 = loc.row0, ci = loc.ci;
    const float* pc = prep + ci * P::FLOATS;
    // the wave's column tiles, w and w + 4 (d = 128): for each tile index c
    // the four waves hold 64 adjacent columns, so that their per-element
    // loads and dg stores of one tile take whole cache lines together; and
    // the chunk row of permuted tile (s, h) row l16
    auto ccol = [&](int c) { return 16 * (w + 4 * c) + l16; };
    auto prw = [&](int s, int h) { return 32 * s + prow(h, l16); };

    // ---- set-up: T^T (high, low), L, beta, gamma, phi; zeroed slots
    if constexpr (DELTA) {
        bf16* sTT = B16(SM::TT);
        bf16* sTTL = B16(SM::TTL);
        bf16* sLH = B16(SM::LH);
        f32x4 tv[4], lv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int idx = tid + j * kGradbThreads, r = idx >> 4, c4 = (idx & 15) * 4;
            tv[j] = *reinterpret_cast<const f32x4*>(pc + P::TI + r * C + c4);
            lv[j] = *reinterpret_cast<const f32x4*>(pc + P::L + r * C + c4);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int idx = tid + j * kGradbThreads, r = idx >> 4, c4 = (idx & 15) * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bf16 hi = (bf16)tv[j][e];
                sTT[(c4 + e) * LC + r] = hi;
                sTTL[(c4 + e) * LC + r] = (bf16)(tv[j][e] - (float)hi);
            }
            *reinterpret_cast<bf16x4*>(sLH + r * LC + c4) = pack4(lv[j]);
        }
    }
    if (tid < C) {
        const float bb = DELTA ? beta[row0 + (size_t)min(tid, nvalid - 1) * H] : 0.f;
        sBt[tid] = tid < nvalid ? bb : 0.f;
        if constexpr (!PERCH) sGam[tid] = pc[P::GAM + tid];
    }
    if (tid < DK) sPhi[tid] = pc[P::PHI + tid];
    for (int i = tid; i < SM::NZ; i += kGradbThreads) sDb[i] = 0.f;

    // ---- phase 1: value slices of 32 columns, one slice ahead in registers
    bf16* sS = B16(SM::S);
    bf16* sDS = B16(SM::DS);
    bf16* sVN = B16(SM::VN);
    bf16* sDVN = B16(SM::DVN);
    bf16* sDO = B16(SM::DO);
    bf16* sVNT = B16(SM::VNT);
    bf16* sDVNT = B16(SM::DVNT);
    constexpr int NUS = DK / 64;          // 16-byte units of a [DK][32] slice per thread
    bf16x8 rS[NUS], rDS[NUS], rVn, rDVn, rDO;
    bf16x4 rv[2];                         // v at (16 w + l16, 16 vt + 4 g4 .. +3)
    const int pp = tid >> 2, pc8 = (tid & 3) * 8;
    auto load_slice = [&](int dv0) {
#pragma unroll
        for (int j = 0; j < NUS; ++j) {
            const int u = tid + j * kGradbThreads, d = u >> 2, c8 = (u & 3) * 8;
            rS[j] = ld8(hs + ci * DK * DV + slc(d, dv0 + c8, DK));
            rDS[j] = ld8(dhs + ci * DK * DV + slc(d, dv0 + c8, DK));
        }
        rVn = ld8(vn + ci * C * DV + slc(pp, dv0 + pc8, C));
        rDVn = ld8(dvn + ci * C * DV + slc(pp, dv0 + pc8, C));
        rDO = ld8(dout + (row0 + (size_t)min(pp, nvalid - 1) * H) * DV + dv0 + pc8);
        if constexpr (DELTA) {
            const int r = 16 * w + l16;
#pragma unroll
            for (int vt = 0; vt < 2; ++vt)
                rv[vt] = ld4b(v + (row0 + (size_t)min(r, nvalid - 1) * H) * DV + dv0 + 16 * vt + 4 * g4);
        }
    };
    // accumulators: [C][DK] products over the wave's tiles (s, h, c); [C][C]
    // tiles of dAqk (ids w + 4 t) and of dT^T (column tile w, rows it >= w)
    f32x4 dQt[2][2][CTW], nW[2][2][CTW], dKb[2][2][CTW], dAq[3], dTt[4];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int c = 0; c < CTW; ++c) dQt[s][h][c] = nW[s][h][c] = dKb[s][h][c] = zero4();
#pragma unroll
    for (int t = 0; t < 3; ++t) dAq[t] = zero4();
#pragma unroll
    for (int t = 0; t < 4; ++t) dTt[t] = zero4();
    float dphi = 0.f, dbn = 0.f;
    load_slice(0);
    for (int sl = 0; sl < NVS; ++sl) {
        const int dv0 = sl * kVS;
        {
#pragma unroll
            for (int j = 0; j < NUS; ++j) {
                const int u = tid + j * kGradbThreads, d = u >> 2, c8 = (u & 3) * 8;
                *reinterpret_cast<bf16x8*>(sS + d * LS + c8) = rS[j];
                *reinterpret_cast<bf16x8*>(sDS + d * LS + c8) = rDS[j];
            }
            *reinterpret_cast<bf16x8*>(sVN + pp * LS + pc8) = rVn;
            *reinterpret_cast<bf16x8*>(sDVN + pp * LS + pc8) = rDVn;
            *reinterpret_cast<bf16x8*>(sDO + pp * LS + pc8) = pp < nvalid ? rDO : zero8();
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                sVNT[(pc8 + j) * LC + pp] = rVn[j];
                sDVNT[(pc8 + j) * LC + pp] = rDVn[j];
            }
            if constexpr (!DELTA) {
                // decay_la: dv = dVnew
                if (pp < nvalid) *reinterpret_cast<bf16x8*>(dv + (row0 + (size_t)pp * H) * DV + dv0 + pc8) = rDVn;
            }
        }
        bf16x4 cv[2] = {rv[0], rv[1]};
        lds_barrier();
        load_slice(min(sl + 1, NVS - 1) * kVS);
        if constexpr (DELTA) {
            bf16* sLH = B16(SM::LH);
            bf16* sTT = B16(SM::TT);
            bf16* sTTL = B16(SM::TTL);
            const int i0 = 16 * w;
            // P^T over the wave's position tile: P^T[v][i] = Vnew[i][v] + beta_i
            // (L Vnew)[i][v], rows v permuted (tile h row r: v = prow(h, r)) so
            // that the pair forms the A fragment of dT^T = P dVnew^T
            f32x4 pt[2] = {zero4(), zero4()};
            for (int sp = 0; sp <= (i0 + 15) >> 5; ++sp) {      // L[i][j] = 0 for j >= i
                const bf16x8 bl = ld8(sLH + (i0 + l16) * LC + 32 * sp + 8 * g4);
#pragma unroll
                for (int h = 0; h < 2; ++h) pt[h] = mf(ld8(sVNT + prow(h, l16) * LC + 32 * sp + 8 * g4), bl, pt[h]);
            }
            const float bi = sBt[i0 + l16];
            bf16x8 pb;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const bf16x4 x = ld4b(sVN + (i0 + l16) * LS + 8 * g4 + 4 * h);
#pragma unroll
                for (int r = 0; r < 4; ++r) pb[4 * h + r] = (bf16)((float)x[r] + bi * pt[h][r]);
            }
            // dT^T tiles (w, it), it >= w (dT strictly lower)
#pragma unroll
            for (int it = 0; it < 4; ++it)
                if (it >= w) dTt[it] = mf(pb, ld8(sDVN + (16 * it + l16) * LS + 8 * g4), dTt[it]);
            // dN^T = dVnew^T T (T split into high and low parts): lane holds
            // position 16 w + l16, value columns 16 vt + 4 g4 + r
#pragma unroll
            for (int vt = 0; vt < 2; ++vt) {
                f32x4 dn = zero4();
                for (int sp = i0 >> 5; sp < 2; ++sp) {           // T[i][r] = 0 for i < r
                    const bf16x8 a = ld8(sDVNT + (16 * vt + l16) * LC + 32 * sp + 8 * g4);
                    dn = mf(a, ld8(sTT + (i0 + l16) * LC + 32 * sp + 8 * g4), dn);
                    dn = mf(a, ld8(sTTL + (i0 + l16) * LC + 32 * sp + 8 * g4), dn);
                }
                const int r = i0 + l16;
                const float bt = sBt[r];
                float part = 0.f;
                f32x4 o;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    o[rr] = bt * dn[rr];
                    part += dn[rr] * (float)cv[vt][rr];
                }
                if (r < nvalid)
                    *reinterpret_cast<bf16x4*>(dv + (row0 + (size_t)r * H) * DV + dv0 + 16 * vt + 4 * g4) = pack4(o);
                dbn += part;
            }
        }
        {
            // dQ~ += dO S^T, nW += dVnew S^T, dKbar += Vnew dS'^T
            bf16x8 bS[CTW], bD[CTW];
#pragma unroll
            for (int c = 0; c < CTW; ++c) {
                bS[c] = ld8(sS + ccol(c) * LS + 8 * g4);
                bD[c] = ld8(sDS + ccol(c) * LS + 8 * g4);
            }
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int pr = prw(s, h);
                    const bf16x8 a1 = ld8(sDO + pr * LS + 8 * g4);
                    const bf16x8 a2 = ld8(sDVN + pr * LS + 8 * g4);
                    const bf16x8 a3 = ld8(sVN + pr * LS + 8 * g4);
#pragma unroll
                    for (int c = 0; c < CTW; ++c) {
                        dQt[s][h][c] = mf(a1, bS[c], dQt[s][h][c]);
                        nW[s][h][c] = mf(a2, bS[c], nW[s][h][c]);
                        dKb[s][h][c] = mf(a3, bD[c], dKb[s][h][c]);
                    }
                }
            // dAqk += dO Vnew^T over the wave's lower tiles
#pragma unroll
            for (int t = 0; t < 3; ++t) {
                const int id = w + 4 * t;
                if (id < 10) {
                    int it, jt;
                    tile_lo(id, it, jt);
                    dAq[t] = mf(ld8(sDO + (16 * it + l16) * LS + 8 * g4), ld8(sVN + (16 * jt + l16) * LS + 8 * g4),
                                dAq[t]);
                }
            }
        }
        {
            // dphi_d += sum over the slice of S .* dS' in row d: the wave's
            // DK/4 rows, 64 / (DK/4) lanes per row
            constexpr int DPW = DK / 4, LPD = 64 / DPW, VPL = kVS / LPD;
            const int d = w * DPW + lane / LPD, v0 = (lane % LPD) * VPL;
#pragma unroll
            for (int e = 0; e < VPL; e += 8) {
                const bf16x8 x = ld8(sS + d * LS + v0 + e), y = ld8(sDS + d * LS + v0 + e);
#pragma unroll
                for (int j = 0; j < 8; ++j) dphi += (float)x[j] * (float)y[j];
            }
        }
        lds_barrier();
    }

    // ---- phase 2 operands to LDS: dAqk (G_Q) and its transpose, dT, T
    bf16* sTR = B16(SM::TR);
    bf16* sDT = B16(SM::DT);
    bf16* sYT = B16(SM::YT);
    bf16* sDL = B16(SM::DL);
    bf16* sDLT = B16(SM::DLT);
    bf16* sDAQ = B16(SM::DAQ);
    bf16* sDAQT = B16(SM::DAQT);
    float* sER = F32(SM::ER);
    float* sEC = F32(SM::EC);
    // scalar gates: the pair terms c_ij = dX_ij X_ij add sum_j c_ij to E_i
    // and subtract sum_i c_ij from E_j; each wave's tiles have distinct row
    // and column tiles, so its row and column sums go to slots of its own
    auto pair_sums = [&](int it, int jt, const f32x4& cval) {
        float cs = 0.f;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const float rsum = row16_sum(cval[rr]);
            if (l16 == 0) sER[w * C + 16 * it + 4 * g4 + rr] += rsum;
            cs += cval[rr];
        }
        cs += __shfl_xor(cs, 16, 64);
        cs += __shfl_xor(cs, 32, 64);
        if (g4 == 0) sEC[w * C + 16 * jt + l16] += cs;
    };
#pragma unroll
    for (int t = 0; t < 3; ++t) {
        const int id = w + 4 * t;
        if (id < 10) {
            int it, jt;
            tile_lo(id, it, jt);
            const int j = 16 * jt + l16;
            f32x4 x, cval;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int i = 16 * it + 4 * g4 + rr;
                float a = j <= i ? dAq[t][rr] : 0.f;
                if constexpr (!PERCH) {
                    cval[rr] = a * pc[P::AQK + i * C + j];
                    a *= j <= i ? __builtin_amdgcn_exp2f(sGam[i] - sGam[j]) : 0.f;
                }
                x[rr] = a;
                sDAQ[i * LC + j] = (bf16)a;
            }
            *reinterpret_cast<bf16x4*>(sDAQT + j * LC + 16 * it + 4 * g4) = pack4(x);
            if constexpr (!PERCH) pair_sums(it, jt, cval);
        }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int id = w + 4 * t;
        if (id < 6) {
            int it, jt;
            tile_up(id, it, jt);
            const int j = 16 * jt + l16;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) sDAQ[(16 * it + 4 * g4 + rr) * LC + j] = (bf16)0.f;
            *reinterpret_cast<bf16x4*>(sDAQT + j * LC + 16 * it + 4 * g4) = pack4(zero4());
        }
    }
    // nW as B fragments of T^T dW: block sp, column tile c, rows 32 sp + 8 g4 + 4 h + r
    bf16x8 nWf[2][CTW];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int c = 0; c < CTW; ++c)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int r = 0; r < 4; ++r) nWf[s][c][4 * h + r] = (bf16)nW[s][h][c][r];
    if constexpr (DELTA) {
        // dT (row-major) from the dT^T tiles (w, it): lane holds dT[16 it + l16][16 w + 4 g4 + r]
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int i = 16 * it + l16;
            f32x4 x;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) x[rr] = (it >= w && 16 * w + 4 * g4 + rr < i) ? dTt[it][rr] : 0.f;
            *reinterpret_cast<bf16x4*>(sDT + i * LC + 16 * w + 4 * g4) = pack4(x);
        }
        // T row-major from T^T: 16 elements per thread
        {
            const bf16* sTT = B16(SM::TT);
            const int kr = tid >> 2, c0 = (tid & 3) * 16;
            const bf16x8 a = ld8(sTT + kr * LC + c0), b = ld8(sTT + kr * LC + c0 + 8);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                sTR[(c0 + j) * LC + kr] = a[j];
                sTR[(c0 + 8 + j) * LC + kr] = b[j];
            }
        }
        // dbeta from the value slices: the four lane groups' partials of row 16 w + l16
        dbn += __shfl_xor(dbn, 16, 64);
        dbn += __shfl_xor(dbn, 32, 64);
        if (g4 == 0) sDb[16 * w + l16] = dbn;
    }
    {
        constexpr int DPW = DK / 4, LPD = 64 / DPW;
        if constexpr (LPD >= 2) dphi += __shfl_xor(dphi, 1, 64);
        if constexpr (LPD >= 4) dphi += __shfl_xor(dphi, 2, 64);
        if (lane % LPD == 0) sDphi[w * DPW + lane / LPD] = dphi;
    }

    lds_barrier();

    // ---- phase 2b (it needs only dT, T, beta and L, so it runs before the
    // per-element phases): dA = -T^T dT T^T (strictly lower), dL = diag(beta) dA
    if constexpr (DELTA) {
        const bf16* sTT = B16(SM::TT);
        // L at this wave's dA elements (fp32, for the dbeta term)
        float lrc[3][4];
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            const int id = w + 4 * t;
            int it = 0, jt = 0;
            if (id < 10) tile_lo(id, it, jt);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                lrc[t][rr] = id < 10 ? pc[P::L + (16 * it + 4 * g4 + rr) * C + 16 * jt + l16] : 0.f;
        }
        // Y = dT T^T over the lower tiles, stored transposed
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            const int id = w + 4 * t;
            if (id < 10) {
                int it, jt;
                tile_lo(id, it, jt);
                f32x4 acc = zero4();
#pragma unroll
                for (int sp = 0; sp < 2; ++sp)
                    acc = mf(ld8(sDT + (16 * it + l16) * LC + 32 * sp + 8 * g4),
                             ld8(sTR + (16 * jt + l16) * LC + 32 * sp + 8 * g4), acc);
                *reinterpret_cast<bf16x4*>(sYT + (16 * jt + l16) * LC + 16 * it + 4 * g4) = pack4(acc);
            }
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int id = w + 4 * t;
            if (id < 6) {
                int it, jt;
                tile_up(id, it, jt);
                *reinterpret_cast<bf16x4*>(sYT + (16 * jt + l16) * LC + 16 * it + 4 * g4) = pack4(zero4());
            }
        }
        lds_barrier();
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            const int id = w + 4 * t;
            if (id < 10) {
                int it, jt;
                tile_lo(id, it, jt);
                f32x4 acc = zero4();
                for (int sp = it >> 1; sp < 2; ++sp)             // T^T[i][k] = 0 for k < i
                    acc = mf(ld8(sTT + (16 * it + l16) * LC + 32 * sp + 8 * g4),
                             ld8(sYT + (16 * jt + l16) * LC + 32 * sp + 8 * g4), acc);
                const int j = 16 * jt + l16;
                f32x4 xl, cval;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int i = 16 * it + 4 * g4 + rr;
                    const float da = j < i ? -acc[rr] : 0.f;
                    float dl = sBt[i] * da;
                    const float part = row16_sum(da * lrc[t][rr]);
                    if (l16 == 0) sDb[(5 + w) * C + i] = part;
                    if constexpr (!PERCH) {
                        cval[rr] = dl * lrc[t][rr];
                        dl *= j < i ? __builtin_amdgcn_exp2f(sGam[i] - sGam[j]) : 0.f;
                    }
                    xl[rr] = dl;
                    sDL[i * LC + j] = (bf16)dl;
                }
                *reinterpret_cast<bf16x4*>(sDLT + j * LC + 16 * it + 4 * g4) = pack4(xl);
                if constexpr (!PERCH) pair_sums(it, jt, cval);
            }
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int id = w + 4 * t;
            if (id < 6) {
                int it, jt;
                tile_up(id, it, jt);
                const int j = 16 * jt + l16;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) sDL[(16 * it + 4 * g4 + rr) * LC + j] = (bf16)0.f;
                *reinterpret_cast<bf16x4*>(sDLT + j * LC + 16 * it + 4 * g4) = pack4(zero4());
            }
        }
        lds_barrier();
    }

    // ---- per column tile c of the wave: the per-element values (rows
    // 32 s + 8 g4 + 4 h + r, column ccol(c)) e = 2^gamma, q, k; then per
    // 32-row block s (block 1 first, for the reverse cumulative sum of dg):
    // dq, dk and the log-gate adjoint E from the value-slice results, phase
    // 2a (dM = -T^T nW, B operand nW from registers), phase 2c (pairwise
    // products, B operands formed from the per-element values of both
    // blocks), then dg (kda) or E's row sums (scalar gates)
    // dq and dk of the last column tile stay in registers; those of the
    // others go to a lane-private stash in LDS (the phase 2b arrays T, dT,
    // Y^T are no longer read), 64 bytes per lane and tile
    bf16x8 lastq[2], lastk[2];
    bf16* sStash = B16(SM::TR) + (size_t)(w * (CTW > 1 ? CTW - 1 : 1) * 64 + lane) * 32;
    static_assert(4 * (CTW > 1 ? CTW - 1 : 1) * 64 * 64 <= 3 * SM::CC, "stash fits T, dT, Y^T");
    float* sRS = F32(SM::RS);      // scalar gates: E row sums, one slot per wave
    float fpw = 0.f;
    // lane bases of the fp32 vectors, kept opaque to the compiler: they lie
    // above 64 KB of LDS, past the 16-bit offset field of the LDS
    // instructions, so a constant address per row would take a register of
    // its own; from a base, each row is the instruction's offset.  Typed as
    // LDS pointers, so that the accesses stay LDS instructions (a generic
    // pointer through the asm would become flat accesses)
    lds_f32* sBtg = (lds_f32*)(sBt + 8 * g4);                 // rows 8 g4 + j
    lds_f32* sDbg = (lds_f32*)(sDb + (1 + w) * C + 8 * g4);   // the wave's dM slot
    lds_f32* sRSg = (lds_f32*)(sRS + w * C + 8 * g4);
    lds_f32* sPhc = (lds_f32*)(sPhi + 16 * w + l16);          // column 16 w + l16
    asm volatile("" : "+v"(sBtg), "+v"(sDbg), "+v"(sRSg), "+v"(sPhc));
    lds_f32* sGamg = sBtg + (SM::GAM - SM::BT) / 4;
    lds_f32* sDphc = sPhc + (SM::DPHI - SM::PHI) / 4;
#pragma unroll
    for (int c = 0; c < CTW; ++c) {
        const int d = ccol(c);
        // q and k of rows 32 s + 8 g4 + j (j = 4 h + r), kept as bf16 (exact)
        bf16x8 lq8[2], lk8[2];
        f32x4 ee[2][2], lg[2][2];
        {
            // byte offsets from the chunk's first row (wave-uniform bases), so
            // that no 64-bit address per row is kept in registers
            const char* qc = reinterpret_cast<const char*>(q + row0 * DK);
            const char* kc = reinterpret_cast<const char*>(k + row0 * DK);
            const char* gc = reinterpret_cast<const char*>(g + row0 * DK);
            const unsigned rowb = (unsigned)(H * DK * 2);
            // the column and row bases laundered per tile: offsets are
            // recomputed rather than kept from the previous tile
            int dl = d, rb = 8 * g4;
            asm volatile("" : "+v"(dl), "+v"(rb));
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        // rows past the end load the last valid row (every
                        // load unconditional) and are zeroed
                        const int row = 32 * s + rb + 4 * h + r;
                        const unsigned rc = (unsigned)min(row, nvalid - 1);
                        const unsigned ob = rc * rowb + (unsigned)dl * 2u;
                        const bf16 qv = *reinterpret_cast<const bf16*>(qc + ob);
                        const bf16 kv = *reinterpret_cast<const bf16*>(kc + ob);
                        lq8[s][4 * h + r] = row < nvalid ? qv : (bf16)0.f;
                        lk8[s][4 * h + r] = row < nvalid ? kv : (bf16)0.f;
                        if constexpr (PERCH) {
                            const unsigned og = (rc * (unsigned)(H * DK) + (unsigned)dl) * 4u;
                            const float gv = *reinterpret_cast<const float*>(gc + og);
                            lg[s][h][r] = row < nvalid ? gv : 0.f;
                        } else {
                            lg[s][h][r] = sGamg[32 * s + 4 * h + r];
                        }
                    }
        }
        // q and k stay packed, two rows per register (16 registers, not 32
        // of one element each): opaque words, unpacked where they are used
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            u32x4 pq = __builtin_bit_cast(u32x4, lq8[s]), pk = __builtin_bit_cast(u32x4, lk8[s]);
            asm volatile("" : "+v"(pq[0]), "+v"(pq[1]), "+v"(pq[2]), "+v"(pq[3]));
            asm volatile("" : "+v"(pk[0]), "+v"(pk[1]), "+v"(pk[2]), "+v"(pk[3]));
            lq8[s] = __builtin_bit_cast(bf16x8, pq);
            lk8[s] = __builtin_bit_cast(bf16x8, pk);
        }
        float gl;
        if constexpr (PERCH) {
            // gamma = log2(e) * cumsum of g down the column (rows past the
            // end add zero): the lane's eight rows of each block, then the
            // lane groups before it in the block, then block 0's total for
            // block 1
            float tot[2], ex[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                float run = 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    run += lg[s][j >> 2][j & 3];
                    lg[s][j >> 2][j & 3] = run;
                }
                float e0 = 0.f, t0 = 0.f;
#pragma unroll
                for (int gg = 0; gg < 4; ++gg) {
                    const float x = __shfl(run, l16 + 16 * gg, 64);
                    if (gg < g4) e0 += x;
                    t0 += x;
                }
                ex[s] = e0;
                tot[s] = t0;
            }
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        lg[s][h][r] = kLog2e * (lg[s][h][r] + ex[s] + (s == 1 ? tot[0] : 0.f));
            gl = kLog2e * (tot[0] + tot[1]);
        } else {
            gl = sGam[C - 1];
        }
        float fpart = 0.f;
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    ee[s][h][r] = __builtin_amdgcn_exp2f(lg[s][h][r]);
                    // Kbar = k 2^(gamma_last - gamma)
                    fpart += dKb[s][h][c][r] * (float)lk8[s][4 * h + r] * __builtin_amdgcn_exp2f(gl - lg[s][h][r]);
                }
        // B fragments of the pairwise products over both blocks sp
        bf16x8 fkm[2], fkp[2], fqt[2];
        if constexpr (PERCH) {
#pragma unroll
            for (int sp = 0; sp < 2; ++sp)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float e = ee[sp][h][r], kk = (float)lk8[sp][4 * h + r];
                        fkm[sp][4 * h + r] = (bf16)(kk * __builtin_amdgcn_rcpf(e));
                        fkp[sp][4 * h + r] = (bf16)(kk * e);
                        fqt[sp][4 * h + r] = (bf16)((float)lq8[sp][4 * h + r] * e);
                    }
        }
        float F = 0.f, all1 = 0.f;
        if constexpr (PERCH) {
            float fp = fpart;
            fp += __shfl_xor(fp, 16, 64);
            fp += __shfl_xor(fp, 32, 64);
            F = fp + sDphc[64 * c] * sPhc[64 * c];            // column d
        } else {
            fpw += fpart;
        }
#pragma unroll
        for (int s = 1; s >= 0; --s) {
            f32x4 aq[2], ak[2], aE[2];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float e = ee[s][h][r], kbf = __builtin_amdgcn_exp2f(gl - lg[s][h][r]);
                    const float qq = (float)lq8[s][4 * h + r], kk = (float)lk8[s][4 * h + r];
                    const float dqt = dQt[s][h][c][r], dkb = dKb[s][h][c][r];
                    // Q~ = q e, Kbar = k 2^(gamma_last - gamma)
                    aq[h][r] = dqt * e;
                    ak[h][r] = dkb * kbf;
                    aE[h][r] = dqt * qq * e - dkb * kk * kbf;
                }
            if constexpr (DELTA) {
                const bf16* sTT = B16(SM::TT);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int pr = prw(s, h);
                    f32x4 acc = zero4();
#pragma unroll
                    for (int sp = s; sp < 2; ++sp)               // T^T[r][i] = 0 for i < r
                        acc = mf(ld8(sTT + pr * LC + 32 * sp + 8 * g4), nWf[sp][c], acc);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int o = 32 * s + 4 * h + r;          // row 8 g4 + o
                        const float bt = sBtg[o];
                        const float dm = -acc[r], e = ee[s][h][r];
                        const float kp = (float)lk8[s][4 * h + r] * e;     // K+ = k e
                        // M = diag(beta) K+: dk += beta e dM, E += dM M, dbeta += dM K+
                        ak[h][r] += bt * e * dm;
                        aE[h][r] += dm * bt * kp;
                        // the wave's columns of the row: this tile's 16, added
                        // to the slot after the previous tiles' in order
                        const float part = row16_sum(dm * kp);
                        if (l16 == 0) sDbg[o] = (c == 0 ? 0.f : sDbg[o]) + part;
                    }
                }
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int pr = prw(s, h);
                if constexpr (PERCH) {
                    // dK+ += dL K-;  dK- = dL^T K+ + dAqk^T Q~;  dQ~ += dAqk K-
                    f32x4 dkp = zero4(), dqt = zero4(), dkm = zero4();
#pragma unroll
                    for (int sp = 0; sp <= s; ++sp) {            // dL, dAqk lower
                        dkp = mf(ld8(sDL + pr * LC + 32 * sp + 8 * g4), fkm[sp], dkp);
                        dqt = mf(ld8(sDAQ + pr * LC + 32 * sp + 8 * g4), fkm[sp], dqt);
                    }
#pragma unroll
                    for (int sp = s; sp < 2; ++sp) {
                        dkm = mf(ld8(sDLT + pr * LC + 32 * sp + 8 * g4), fkp[sp], dkm);
                        dkm = mf(ld8(sDAQT + pr * LC + 32 * sp + 8 * g4), fqt[sp], dkm);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float e = ee[s][h][r], kk = (float)lk8[s][4 * h + r];
                        const float qq = (float)lq8[s][4 * h + r];
                        // 1/e = 2^-gamma is normal in the gates' supported range
                        const float ei = __builtin_amdgcn_rcpf(e);
                        ak[h][r] += dkp[r] * e + dkm[r] * ei;
                        aq[h][r] += dqt[r] * e;
                        aE[h][r] += dkp[r] * (kk * e) - dkm[r] * (kk * ei) + dqt[r] * (qq * e);
                    }
                } else {
                    // G_L = dL .* Gamma, G_Q = dAqk .* Gamma (raw q, k):
                    // dk += G_L k + G_L^T k + G_Q^T q;  dq += G_Q k
                    f32x4 dkk = zero4(), dqq = zero4();
#pragma unroll
                    for (int sp = 0; sp <= s; ++sp) {
                        if constexpr (DELTA) dkk = mf(ld8(sDL + pr * LC + 32 * sp + 8 * g4), lk8[sp], dkk);
                        dqq = mf(ld8(sDAQ + pr * LC + 32 * sp + 8 * g4), lk8[sp], dqq);
                    }
#pragma unroll
                    for (int sp = s; sp < 2; ++sp) {
                        if constexpr (DELTA) dkk = mf(ld8(sDLT + pr * LC + 32 * sp + 8 * g4), lk8[sp], dkk);
                        dkk = mf(ld8(sDAQT + pr * LC + 32 * sp + 8 * g4), lq8[sp], dkk);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        ak[h][r] += dkk[r];
                        aq[h][r] += dqq[r];
                        // E's row sum over the wave's columns: this tile's 16,
                        // added to the slot after the previous tiles' in order
                        const float x = row16_sum(aE[h][r]);
                        const int o = 32 * s + 4 * h + r;          // row 8 g4 + o
                        if (l16 == 0) sRSg[o] = (c == 0 ? 0.f : sRSg[o]) + x;
                    }
                }
            }
            if constexpr (PERCH) {
                // dg down the column: reverse cumsum of E plus F.  The lane
                // holds rows 32 s + 8 g4 + j (j = 4 h + r): suffix sums inside
                // those eight, then the later lane groups' totals of this
                // block, and for block 0 all of block 1
                float run = 0.f;
#pragma unroll
                for (int j = 7; j >= 0; --j) {
                    run += aE[j >> 2][j & 3];
                    aE[j >> 2][j & 3] = run;
                }
                float later = 0.f, all = 0.f;
#pragma unroll
                for (int g = 3; g >= 0; --g) {
                    const float x = __shfl(run, l16 + 16 * g, 64);
                    if (g > g4) later += x;
                    all += x;
                }
                if (s == 0) later += all1;
                else all1 = all;
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = 32 * s + 8 * g4 + 4 * h + r;
                        if (row < nvalid)
                            *reinterpret_cast<float*>(reinterpret_cast<char*>(dg + row0 * DK) +
                                                      ((unsigned)row * (unsigned)(H * DK) + (unsigned)d) * 4u) =
                                aE[h][r] + later + F;
                    }
            }
            // dq, dk of rows 32 s + 8 g4 + 4 h + r, in the order (h, r)
            bf16x8 xq, xk;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    xq[4 * h + r] = (bf16)aq[h][r];
                    xk[4 * h + r] = (bf16)ak[h][r];
                }
            if (c == CTW - 1) {
                lastq[s] = xq;
                lastk[s] = xk;
            } else {
                bf16* st = sStash + (size_t)c * 64 * 32;
                *reinterpret_cast<bf16x8*>(st + 8 * s) = xq;
                *reinterpret_cast<bf16x8*>(st + 16 + 8 * s) = xk;
            }
        }
        // keeps the next column tile's loads from being hoisted into this
        // one (they would hold registers through its products)
        asm volatile("" ::: "memory");
    }
    if constexpr (!PERCH) {
        // the gamma_last sum, one slot per wave
        float* sFP = F32(SM::FP);
        const float fp = lane_group_sum<64>(fpw);
        if (lane == 0) sFP[w] = fp;
    }
    lds_barrier();

    // ---- phase 3: dq, dk staged row-major in LDS (over the dL .. dAqk^T
    // arrays, no longer read), then stored eight channels per access
    bf16* sQ = B16(SM::SQ);
    bf16* sK = B16(SM::SK);
    constexpr int LQ = SM::LQ;
#pragma unroll
    for (int c = 0; c < CTW; ++c) {
        bf16x8 xq[2], xk[2];
        if (c == CTW - 1) {
            xq[0] = lastq[0];
            xq[1] = lastq[1];
            xk[0] = lastk[0];
            xk[1] = lastk[1];
        } else {
            const bf16* st = sStash + (size_t)c * 64 * 32;
            xq[0] = ld8(st);
            xq[1] = ld8(st + 8);
            xk[0] = ld8(st + 16);
            xk[1] = ld8(st + 24);
        }
        const int d = ccol(c);
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int row = 32 * s + 8 * g4 + j;
                sQ[row * LQ + d] = xq[s][j];
                sK[row * LQ + d] = xk[s][j];
            }
    }
    lds_barrier();
    {
        constexpr int U8 = DK / 8;
#pragma unroll
        for (int it_ = 0; it_ < (C * U8) / kGradbThreads; ++it_) {
            const int idx = tid + it_ * kGradbThreads, r = idx / U8, d0 = (idx % U8) * 8;
            if (r < nvalid) {
                const size_t off = (row0 + (size_t)r * H) * DK + d0;
                *reinterpret_cast<bf16x8*>(dq + off) = ld8(sQ + r * LQ + d0);
                *reinterpret_cast<bf16x8*>(dk + off) = ld8(sK + r * LQ + d0);
            }
        }
    }
    if constexpr (!PERCH) {
      if (w == 0) {
        // scalar gates: row totals (per-element E, pair terms), then the
        // reverse cumulative sum over the 64 rows by lane shuffles
        const float* sRS = F32(SM::RS);
        const float* sFP = F32(SM::FP);
        const int r = lane;
        float t = 0.f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) t += sRS[ww * C + r];
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) t += sER[ww * C + r];
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) t -= sEC[ww * C + r];
        float dps = 0.f;
        for (int dd = 0; dd < DK; ++dd) dps += sDphi[dd];
        const float F = sFP[0] + sFP[1] + sFP[2] + sFP[3] + dps * sPhi[0];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_down(t, off, 64);
            if (r + off < 64) t += y;
        }
        if (r < nvalid) dg[row0 + (size_t)r * H] = t + F;
      }
    }
    if constexpr (DELTA) {
        if (tid < nvalid) {
            float db = 0.f;
#pragma unroll
            for (int j = 0; j < SM::NDB; ++j) db += sDb[j * C + tid];
            dbeta[row0 + (size_t)tid * H] = db;
        }
    }
}

}  // namespace bw
}  // namespace dr
