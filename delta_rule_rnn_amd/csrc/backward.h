// backward.h -- gradients of the chunkwise gated delta rule: three kernels
// here, after the forward state pass.
//
// Page keys: [KDA] "TileLang 实战：KDA 从零到一–Kimi Delta Attention";
// [SD] "TileLang 实战：KDA 从零到一--标量衰减"; [GDN] "Gated DeltaNet"
// (section "反向传播：状态伴随与三角变换梯度": the forward's operands are recomputed, the chunk entry
// states are rebuilt by a forward pass, the state adjoint runs backwards over
// the chunks, then the per-chunk gradients and the WY-representation backward
// go through the triangular inverse, and the gate gradient is a reverse
// cumulative sum inside each chunk).
//
// Chunk quantities (rows r, i, j = positions, d = key channel; kernel
// orientation, state S in R^{Dk x Dv}), as in the forward:
//   gamma = log2 cumsum of g;  e = 2^gamma;  phi = 2^gamma_last
//   Q~ = q e,  K+ = k e,  K- = k / e,  Kbar = k phi / e
//   L  = StrictLower(K+ K-^T)      (scalar gates: (k_i.k_j) 2^(gamma_i - gamma_j))
//   Aqk = TrilIncl(Q~ K-^T)        (scalar gates: (q_i.k_j) 2^(gamma_i - gamma_j))
//   T = (I + diag(beta) L)^-1,  W = T diag(beta) K+,  U = T diag(beta) V
//   Vnew = U - W S,  O = Q~ S + Aqk Vnew,  S' = diag(phi) S + Kbar^T Vnew
// and backwards, with dS' the adjoint of the exit state:
//   dVnew = Aqk^T dO + Kbar dS'              (state adjoint pass)
//   dS    = Q~^T dO + diag(phi) dS' - W^T dVnew
//   dQ~ = dO S^T,  dAqk = dO Vnew^T,  dKbar = Vnew dS'^T,  dphi = rowsum(S .* dS')
//   dW = -dVnew S^T,  dU = dVnew
//   dT = dW M^T + dU N^T  (M = diag(beta) K+, N = diag(beta) V),  dM = T^T dW,
//   dN = T^T dU,  dA = -T^T dT T^T (strictly lower),  dL = diag(beta) dA
// then through the separable exponents to dq, dk, dv, dbeta and the log-gate
// adjoint E; dg_s = sum_{r >= s} E_r + F with F the gamma_last terms (the
// ln 2 of d2^x/dx and the log2(e) of gamma cancel).
//
// Barriers are LDS-only (lds_barrier: wait for this wave's LDS operations,
// then s_barrier): threads of a workgroup exchange data through LDS only, and
// a full __syncthreads would also wait for every outstanding global load and
// store (prefetches and result stores included).
//
// The entry states S_c and Vnew_c of every chunk come first, from the
// forward's own two kernels (the chunk-parallel records, then the state pass
// in its STATES mode, fp32 state in accumulators).  The per-chunk state
// arrays (S_c, Vnew_c, and the exit adjoints dS'_c, dVnew_c) are stored in
// the I/O dtype, rounded from fp32 accumulators.  The kernels here keep
// their operands as fp32 in LDS, in natural row-major layout, and compute on
// fp32 MFMA (v_mfma_f32_16x16x4_f32), except for bf16 I/O: the prep's L and
// Aqk, and the gradient kernel's value-slice, pairwise and T products, run
// on bf16 MFMA (operands rounded as they are read, fp32 accumulation).  The
// I/O dtype otherwise only changes the loads of q, k, v, dO and the stores
// of dq, dk, dv.
//   bwd_prep_kernel     chunk-parallel: writes the natural fp32 chunk arrays
//                       (Aqk, L, T, phi, gamma, and for the value-slice
//                       reverse pass Q~, W, Kbar), or for the segment-
//                       parallel reverse pass its bf16 operands instead of
//                       the fp32 Q~, W, Kbar
//   bwd_state_rev_kernel   per (chain, 16 value columns), chunks in reverse:
//                       exit adjoints dS'_c, dVnew, and dh0 (fp32 I/O and
//                       packed sequences; bf16 I/O in the dense layout takes
//                       the segment-parallel pass of revseg.h)
//   bwd_grad_kernel     chunk-parallel: dq, dk, dv, dbeta, dg
#pragma once

#include "common.h"

namespace dr {
namespace bw {

constexpr int C = kChunk;
static_assert(C * C % 512 == 0 && C * 16 % 256 == 0, "strided loops assume exact trip counts");
constexpr int kVS = 32;            // value columns per state-pass workgroup / gradient slice
constexpr int LVS = kVS + 4;       // padded row of [*, 32] fp32 tiles
constexpr int LDC = C + 4;         // padded row of [C, C] fp32 tiles

// Natural fp32 arrays of one chunk of one (b, h), written by bwd_prep_kernel.
template <int DK>
struct Prep {
    static constexpr int DV = DK;
    static constexpr size_t QT = 0;                         // [C][DK]  Q~
    static constexpr size_t W = QT + (size_t)C * DK;        // [C][DK]  W
    static constexpr size_t KB = W + (size_t)C * DK;        // [C][DK]  Kbar
    static constexpr size_t AQK = KB + (size_t)C * DK;      // [C][C]   Aqk
    static constexpr size_t L = AQK + (size_t)C * C;        // [C][C]   L (strictly lower)
    static constexpr size_t TI = L + (size_t)C * C;         // [C][C]   T = (I + diag(beta) L)^-1
    static constexpr size_t PHI = TI + (size_t)C * C;       // [DK]     phi
    static constexpr size_t GAM = PHI + DK;                 // [C][DK] (kda) or [C]: gamma (log2)
    static constexpr size_t FLOATS = GAM + (size_t)C * DK;
};

// bf16 operands of one chunk for the segment-parallel reverse pass
// (revseg.h), written by bwd_prep_kernel for bf16 I/O in the layouts that
// pass stages into LDS: every product there reduces along contiguous
// elements.
template <int DK>
struct RevRec {
    static constexpr size_t KB = 0;                         // [C][DK]  Kbar
    static constexpr size_t AT = KB + (size_t)C * DK;       // [C][C]   Aqk^T: AT[i][j] = Aqk[j][i]
    static constexpr size_t QT = AT + (size_t)C * C;        // [DK][C]  Q~^T
    static constexpr size_t WT = QT + (size_t)DK * C;       // [DK][C]  W^T
    static constexpr size_t ELEMS = WT + (size_t)DK * C;    // bf16 elements
};

// Packed sequences (table == null: the dense [B, T] layout).  The chunk table
// and sequence descriptors are those of the packed forward
// (varlen_table_kernel): table[slot] = {sequence, first token, valid rows, -},
// seqinfo[n] = {first slot, chunks, first token, tokens}; per-chunk arrays
// are indexed h * maxchunks + slot.
// (struct Pack is declared in common.h, where the host code sees it too.)

// The chunk a chunk-parallel workgroup handles: its first token row (token
// index times H plus h), its valid rows and its per-chunk array index; false
// for a packed slot past the table's count.
struct ChunkLoc {
    size_t row0, ci;
    int nvalid;
};
__device__ __forceinline__ bool locate_chunk(const Pack& pk, unsigned it, int H, int Tlen, int NT, ChunkLoc& L) {
    const int h = (int)(it % (unsigned)H);
    const unsigned tt = it / (unsigned)H;
    if (pk.table) {
        const int slot = (int)tt;
        if (slot >= *pk.total) return false;
        const int4 e = pk.table[slot];
        L.row0 = (size_t)e.y * H + h;
        L.nvalid = e.z;
        L.ci = (size_t)h * pk.maxchunks + slot;
    } else {
        const int c = (int)(tt % (unsigned)NT), b = (int)(tt / (unsigned)NT);
        L.row0 = ((size_t)b * Tlen + (size_t)c * C) * H + h;
        L.nvalid = min(C, Tlen - c * C);
        L.ci = ((size_t)b * H + h) * NT + c;
    }
    return true;
}

// The (sequence or batch) * H + head index of logical chain lc out of
// nchains.  Packed sequences take chains head-major (lc = h * N + sequence),
// so that each XCD's contiguous range of logical ids (xcd_logical) holds
// every sequence for a few heads and the XCDs get equal token counts
// whatever the lengths; the dense layout keeps (b, h) order.
__device__ __forceinline__ int chain_of(const Pack& pk, int lc, int H, int nchains) {
    if (!pk.table) return lc;
    const int nseq = nchains / H;
    return (lc % nseq) * H + lc / nseq;
}

// The chain a state-pass workgroup follows: chunks ci0 + c*cstep for
// c = 0..nseg-1, tokens tok0 .. tok0 + tlim - 1 (token index; rows are
// token * H + h).
struct ChainLoc {
    size_t ci0, tok0;
    int nseg, tlim;
};
__device__ __forceinline__ ChainLoc locate_chain(const Pack& pk, int chain, int H, int Tlen, int NT) {
    const int b = chain / H, h = chain % H;
    ChainLoc L;
    if (pk.table) {
        const int4 si = pk.seqinfo[b];   // b is the sequence
        L.ci0 = (size_t)h * pk.maxchunks + si.x;
        L.nseg = si.y;
        L.tok0 = (size_t)si.z;
        L.tlim = si.w;
    } else {
        L.ci0 = (size_t)chain * NT;
        L.nseg = NT;
        L.tok0 = (size_t)b * Tlen;
        L.tlim = Tlen;
    }
    return L;
}

// acc[16x16] += A[16 x K] * B[K x 16] on fp32 MFMA, A(r, k) = A[r*ar + k*ak],
// B(k, c) = B[k*bk + c*bc].  At step k0 lane l supplies A(l%16, k0 + l/16)
// and B(k0 + l/16, l%16); the result is in the accumulator layout (lane l:
// rows 4*(l/16) + i, column l%16).  Wave-uniform control flow only.
template <int K>
__device__ __forceinline__ f32x4 mmk(f32x4 acc, const float* A, int ar, int ak, const float* B, int bk, int bc,
                                     int lane) {
    const int r = lane & 15, q = lane >> 4;
    const float* a = A + r * ar + q * ak;
    const float* b = B + q * bk + r * bc;
#pragma unroll 8
    for (int k0 = 0; k0 < K; k0 += 4)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[k0 * ak], b[k0 * bk], acc, 0, 0, 0);
    return acc;
}
// The same product with A contiguous along k (A(r, k) = A[r*ar + k]), read
// four k at a time: lane group q = l/16 takes the contiguous k range
// [q*K/4, (q+1)*K/4) instead of every fourth k (the sum is the same, in
// another order), so its A values arrive as 16-byte LDS reads.  ar and A
// must keep those reads 16-byte aligned.
template <int K>
__device__ __forceinline__ f32x4 mmk_a(f32x4 acc, const float* A, int ar, const float* B, int bk, int bc,
                                       int lane) {
    static_assert(K % 16 == 0, "k range per lane group");
    constexpr int KQ = K / 4;
    const int r = lane & 15, q = lane >> 4;
    const float* a = A + r * ar + q * KQ;
    const float* b = B + (q * KQ) * bk + r * bc;
#pragma unroll
    for (int s0 = 0; s0 < KQ; s0 += 4) {
        const f32x4 av = *reinterpret_cast<const f32x4*>(a + s0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j], b[(s0 + j) * bk], acc, 0, 0, 0);
    }
    return acc;
}
// Both operands contiguous along k (A(r, k) = A[r*ar + k], B(k, c) =
// B[c*bc + k]), both read four k at a time as above.
template <int K>
__device__ __forceinline__ f32x4 mmk_ab(f32x4 acc, const float* A, int ar, const float* B, int bc, int lane) {
    static_assert(K % 16 == 0, "k range per lane group");
    constexpr int KQ = K / 4;
    const int r = lane & 15, q = lane >> 4;
    const float* a = A + r * ar + q * KQ;
    const float* b = B + r * bc + q * KQ;
#pragma unroll
    for (int s0 = 0; s0 < KQ; s0 += 4) {
        const f32x4 av = *reinterpret_cast<const f32x4*>(a + s0);
        const f32x4 bv = *reinterpret_cast<const f32x4*>(b + s0);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j], bv[j], acc, 0, 0, 0);
    }
    return acc;
}
// The same product with both operands contiguous along k (A(r, k) =
// A[r*ar + k], B(k, c) = B[c*bc + k]) on bf16 MFMA (v_mfma_f32_16x16x32_bf16):
// lane l reads 8 consecutive fp32 values of row / column l%16 at k0 + 8*(l/16)
// (two 16-byte LDS reads each) and rounds them to bf16; fp32 accumulation.
// ar, bc and the pointers must keep those reads 16-byte aligned.
template <int K>
__device__ __forceinline__ f32x4 mmb(f32x4 acc, const float* A, int ar, const float* B, int bc, int lane) {
    const int r = lane & 15, q = lane >> 4;
    const float* a = A + r * ar + 8 * q;
    const float* b = B + r * bc + 8 * q;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 32) {
        const float4 a0 = *reinterpret_cast<const float4*>(a + k0), a1 = *reinterpret_cast<const float4*>(a + k0 + 4);
        const float4 b0 = *reinterpret_cast<const float4*>(b + k0), b1 = *reinterpret_cast<const float4*>(b + k0 + 4);
        const bf16x8 fa = {(bf16)a0.x, (bf16)a0.y, (bf16)a0.z, (bf16)a0.w, (bf16)a1.x, (bf16)a1.y, (bf16)a1.z, (bf16)a1.w};
        const bf16x8 fb = {(bf16)b0.x, (bf16)b0.y, (bf16)b0.z, (bf16)b0.w, (bf16)b1.x, (bf16)b1.y, (bf16)b1.z, (bf16)b1.w};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb, acc, 0, 0, 0);
    }
    return acc;
}
// Product with k contiguous in both operands, on the MFMA of the I/O dtype:
// bf16 operands for bf16 I/O (as the forward's products), fp32 otherwise.
template <typename T, int K>
__device__ __forceinline__ f32x4 mmc(f32x4 acc, const float* A, int ar, const float* B, int bc, int lane) {
    if constexpr (sizeof(T) == 2) return mmb<K>(acc, A, ar, B, bc, lane);
    else return mmk<K>(acc, A, ar, 1, B, 1, bc, lane);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
// bf16 MFMA (v_mfma_f32_16x16x32_bf16) over fp32 LDS operands of any
// layout: at step k0 lane l packs A(l%16, k0 + 8(l/16) + j) and
// B(k0 + 8(l/16) + j, l%16), j = 0..7, to bf16; fp32 accumulation.
// A(r, k) = A[r*ar + k*ak] (ACONT: ak = 1, read as two 16-byte loads, which
// needs ar and A 16-byte aligned); B(k, c) = B[k*bk + c*bc].
template <int K, bool ACONT>
__device__ __forceinline__ f32x4 mmb_g(f32x4 acc, const float* A, int ar, int ak, const float* B, int bk, int bc,
                                       int lane) {
    const int r = lane & 15, q = lane >> 4;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 32) {
        const int kk = k0 + 8 * q;
        float av[8], bv[8];
        if constexpr (ACONT) {
            const f32x4 a0 = *reinterpret_cast<const f32x4*>(A + r * ar + kk);
            const f32x4 a1 = *reinterpret_cast<const f32x4*>(A + r * ar + kk + 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) { av[j] = a0[j]; av[4 + j] = a1[j]; }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) av[j] = A[r * ar + (kk + j) * ak];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) bv[j] = B[(kk + j) * bk + r * bc];
        bf16x8 fa, fb;
#pragma unroll
        for (int j = 0; j < 8; ++j) { fa[j] = (bf16)av[j]; fb[j] = (bf16)bv[j]; }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb, acc, 0, 0, 0);
    }
    return acc;
}
// acc += A B on bf16 MFMA where B holds bf16 values exactly (slices of the
// per-chunk state arrays, stored in bf16 for bf16 I/O), so that it converts
// without loss, and A is fp32: split into bf16 high and low parts (x = hi +
// lo, lo = bf16(x - hi)), two MFMAs per step, about 16 significant bits;
// SPLIT false when A holds bf16 values too (one MFMA, exact).  Layouts as in
// mmb_g.
template <int K, bool ACONT, bool SPLIT>
__device__ __forceinline__ f32x4 mms(f32x4 acc, const float* A, int ar, int ak, const float* B, int bk, int bc,
                                     int lane) {
    const int r = lane & 15, q = lane >> 4;
#pragma unroll 1
    for (int k0 = 0; k0 < K; k0 += 32) {
        const int kk = k0 + 8 * q;
        float av[8];
        if constexpr (ACONT) {
            const f32x4 a0 = *reinterpret_cast<const f32x4*>(A + r * ar + kk);
            const f32x4 a1 = *reinterpret_cast<const f32x4*>(A + r * ar + kk + 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) { av[j] = a0[j]; av[4 + j] = a1[j]; }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) av[j] = A[r * ar + (kk + j) * ak];
        }
        bf16x8 ah, al, fb;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            ah[j] = (bf16)av[j];
            al[j] = (bf16)(av[j] - (float)ah[j]);
            fb[j] = (bf16)B[(kk + j) * bk + r * bc];
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, fb, acc, 0, 0, 0);
        if constexpr (SPLIT) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, fb, acc, 0, 0, 0);
    }
    return acc;
}
// The pairwise products of the gradient kernel on the MFMA of the I/O
// dtype: bf16 operands for bf16 I/O (as the value-slice products), fp32
// otherwise.  ACONT as in mmb_g; the fp32 form takes mmk_a when A is
// contiguous along k.
template <typename T, int K, bool ACONT>
__device__ __forceinline__ f32x4 mmp(f32x4 acc, const float* A, int ar, int ak, const float* B, int bk, int bc,
                                     int lane) {
    if constexpr (sizeof(T) == 2) return mmb_g<K, ACONT>(acc, A, ar, ak, B, bk, bc, lane);
    else if constexpr (ACONT) return mmk_a<K>(acc, A, ar, B, bk, bc, lane);
    else return mmk<K>(acc, A, ar, ak, B, bk, bc, lane);
}


// Four adjacent elements stored as one access (8 bytes bf16, 16 bytes fp32).
__device__ __forceinline__ void st4(bf16* p, f32x4 v) {
    bf16x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = (bf16)v[j];
    *reinterpret_cast<bf16x4*>(p) = o;
}
__device__ __forceinline__ void st4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
__device__ __forceinline__ int arow(int lane, int i) { return 4 * (lane >> 4) + i; }


// Cooperative copy of a [ROWS][COLS] fp32 block (row stride gs floats) into
// LDS (row stride ls floats, a multiple of 4) by NTHR threads.  The shape is
// known at compile time, so each thread issues up to 8 float4 loads before
// the first store (the loads' latencies overlap instead of adding up).
template <int ROWS, int COLS, int NTHR>
__device__ __forceinline__ void stage(float* dst, int ls, const float* __restrict__ src, size_t gs, int tid) {
    constexpr int PER = COLS / 4, N = ROWS * PER, IT = N / NTHR, BT = IT < 8 ? IT : 8;
    static_assert(COLS % 4 == 0 && N % NTHR == 0 && IT % BT == 0, "staging shape");
#pragma unroll
    for (int i0 = 0; i0 < IT; i0 += BT) {
        float4 buf[BT];
#pragma unroll
        for (int j = 0; j < BT; ++j) {
            const int idx = tid + (i0 + j) * NTHR, r = idx / PER, c4 = (idx % PER) * 4;
            buf[j] = *reinterpret_cast<const float4*>(src + r * gs + c4);
        }
#pragma unroll
        for (int j = 0; j < BT; ++j) {
            const int idx = tid + (i0 + j) * NTHR, r = idx / PER, c4 = (idx % PER) * 4;
            *reinterpret_cast<float4*>(dst + r * ls + c4) = buf[j];
        }
    }
}
// The two halves of a staging copy, for issuing the loads of several blocks
// before any of their LDS stores.  The source holds fp32 or bf16 (S); the
// LDS copy is fp32.
template <int ROWS, int COLS, int NTHR, typename S = float>
struct Staged {
    static constexpr int PER = COLS / 4, IT = ROWS * PER / NTHR;
    static_assert(COLS % 4 == 0 && (ROWS * PER) % NTHR == 0, "staging shape");
    // native 4-element vectors (not the float4 struct, whose copies become
    // memcpy and keep a loop-carried array out of registers)
    using V4 = typename VecOf<S, 4>::type;
    V4 v[IT];
    __device__ __forceinline__ void load(const S* __restrict__ src, size_t gs, int tid) {
#pragma unroll
        for (int j = 0; j < IT; ++j) {
            const int idx = tid + j * NTHR, r = idx / PER, c4 = (idx % PER) * 4;
            v[j] = *reinterpret_cast<const V4*>(src + r * gs + c4);
        }
    }
    __device__ __forceinline__ void store(float* dst, int ls, int tid) const {
#pragma unroll
        for (int j = 0; j < IT; ++j) {
            const int idx = tid + j * NTHR, r = idx / PER, c4 = (idx % PER) * 4;
            f32x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = (float)v[j][e];
            *reinterpret_cast<f32x4*>(dst + r * ls + c4) = x;
        }
    }
};
// fp32 LDS block to global memory (fp32 or bf16, four elements per access)
template <int ROWS, int COLS, int NTHR, typename D>
__device__ __forceinline__ void unstage(D* __restrict__ dst, size_t gs, const float* src, int ls, int tid) {
    constexpr int PER = COLS / 4, N = ROWS * PER, IT = N / NTHR;
    static_assert(COLS % 4 == 0 && N % NTHR == 0, "staging shape");
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int idx = tid + i * NTHR, r = idx / PER, c4 = (idx % PER) * 4;
        st4(dst + r * gs + c4, *reinterpret_cast<const f32x4*>(src + r * ls + c4));
    }
}

// ===========================================================================
constexpr int kPrepThreads = 512;
constexpr unsigned PREP_W_GAM = 1, PREP_W_AQK = 2;

// Prep: one 512-thread workgroup per (chunk, head, batch), heads fastest
// (one workgroup per CU by LDS: eight waves keep loads and products in
// flight together).
// ===========================================================================
template <int KIND, typename T, int DK>
struct PrepSmem {
    static constexpr int LDK = DK + 4;
    static constexpr size_t MAT = (size_t)C * LDK;
    static constexpr size_t SA = 0, SB = SA + MAT, SQ = SB + MAT, SL = SQ + MAT, ST = SL + (size_t)C * LDC;
    static constexpr size_t SBETA = ST + (size_t)C * LDC, SGAM = SBETA + C, SPHI = SGAM + C;
    static constexpr size_t FLOATS = SPHI + DK;
};

template <int KIND, typename T, int DK>
__global__ __launch_bounds__(kPrepThreads) void bwd_prep_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                       const float* __restrict__ g,
                                                       const float* __restrict__ beta, float* __restrict__ prep,
                                                       bf16* __restrict__ rrec, int Tlen, int H, int NT, Pack pk,
                                                       unsigned wmask)
{
    using P = Prep<DK>;
    using RR = RevRec<DK>;
    using SM = PrepSmem<KIND, T, DK>;
    constexpr int DV = DK, LDK = SM::LDK, NTH = kPrepThreads, NW = NTH / 64;
    constexpr bool DELTA = KIND != KIND_LA;
    constexpr bool PERCH = KIND == KIND_KDA;
    __shared__ __attribute__((aligned(16))) float smem[SM::FLOATS];
    float* sA = smem + SM::SA;     // kda: K+ (then M);  scalar: k (then M)
    float* sB = smem + SM::SB;     // kda: g, then K-
    float* sQ = smem + SM::SQ;     // q (kda: Q~)
    float* sL = smem + SM::SL;
    float* sT = smem + SM::ST;
    float* sBeta = smem + SM::SBETA;
    float* sGam = smem + SM::SGAM;
    float* sPhi = smem + SM::SPHI;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    ChunkLoc loc;
    if (!locate_chunk(pk, blockIdx.x, H, Tlen, NT, loc)) return;
    const int nvalid = loc.nvalid;
    const size_t row0 = loc.row0;   // token row of position 0
    float* out = prep + loc.ci * P::FLOATS;
    // the bf16 record of the segment-parallel reverse pass (null: not used);
    // with it, the fp32 Q~, W and Kbar (read only by the value-slice reverse
    // pass; the gradient kernel forms its own from q, k and gamma) are not
    // written
    bf16* rr = rrec ? rrec + loc.ci * RR::ELEMS : nullptr;
    // the per-channel gamma and Aqk arrays only where a later kernel reads
    // them (PREP_W_GAM: the gradient kernel with fp32 LDS operands;
    // PREP_W_AQK: the value-slice reverse pass, and scalar gates' gradient
    // kernels); the per-row gamma of scalar gates is always written
    const bool wgam = (wmask & PREP_W_GAM) != 0, waqk = (wmask & PREP_W_AQK) != 0;

    // ---- inputs, rows past the end of a ragged chunk zero
    #pragma unroll 8
    for (int it_ = 0; it_ < (C * DK) / NTH; ++it_) {
        const int idx = tid + it_ * NTH;
        const int r = idx / DK, d = idx % DK;
        // rows past the end load the last valid row (every load unconditional)
        const bool ok = r < nvalid;
        const size_t off = (row0 + (size_t)min(r, nvalid - 1) * H) * DK + d;
        const float kk = to_f(k[off]), qq = to_f(q[off]);
        sA[r * LDK + d] = ok ? kk : 0.f;
        sQ[r * LDK + d] = ok ? qq : 0.f;
        if constexpr (PERCH) {
            const float gg = g[off];
            sB[r * LDK + d] = ok ? gg : 0.f;
        }
    }
    if (tid < C) {
        const bool ok = tid < nvalid;
        const size_t rr = row0 + (size_t)min(tid, nvalid - 1) * H;
        const float bb = DELTA ? beta[rr] : 0.f;
        sBeta[tid] = ok ? bb : 0.f;
        if constexpr (!PERCH) {
            const float gg = g[rr];
            sGam[tid] = ok ? gg : 0.f;
        }
    }
    lds_barrier();

    // ---- gamma and the separable operands
    if constexpr (PERCH) {
        // cumsum down each column by NTH / DK threads, each over a block of
        // rows: block sums, then each block's running sum from the sum of the
        // blocks above it (sL is free until L is formed)
        constexpr int NB = NTH / DK, RB = C / NB;
        float* sBlk = sL;
        const int d = tid % DK, b = tid / DK;
        float bs = 0.f;
#pragma unroll
        for (int j = 0; j < RB; ++j) bs += sB[(b * RB + j) * LDK + d];
        sBlk[b * DK + d] = bs;
        lds_barrier();
        float run = 0.f;
#pragma unroll
        for (int b2 = 0; b2 < NB; ++b2)
            if (b2 < b) run += sBlk[b2 * DK + d];
        run *= kLog2e;
        for (int j = 0; j < RB; ++j) {
            const int r = b * RB + j;
            run += sB[r * LDK + d] * kLog2e;
            const float e = __builtin_amdgcn_exp2f(run), ei = __builtin_amdgcn_exp2f(-run);
            const float kk = sA[r * LDK + d];
            sA[r * LDK + d] = kk * e;
            sB[r * LDK + d] = kk * ei;
            sQ[r * LDK + d] *= e;
            if (wgam) out[P::GAM + (size_t)r * DK + d] = run;
        }
        if (b == NB - 1) {
            const float phi = __builtin_amdgcn_exp2f(run);
            sPhi[d] = phi;
            out[P::PHI + d] = phi;
        }
        lds_barrier();
        const float phi = sPhi[d];
        for (int j = 0; j < RB; ++j) {
            const int r = b * RB + j;
            const float kb = sB[r * LDK + d] * phi;
            if (rr) {
                rr[RR::KB + (size_t)r * DK + d] = (bf16)kb;
            } else {
                out[P::KB + (size_t)r * DK + d] = kb;
                out[P::QT + (size_t)r * DK + d] = sQ[r * LDK + d];
            }
        }
    } else {
        if (wave == 0) {
            float x = sGam[lane];
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off, 64);
                if (lane >= off) x += y;
            }
            x *= kLog2e;
            sGam[lane] = x;
            out[P::GAM + lane] = x;
        }
        lds_barrier();
        const float gl = sGam[C - 1];
        #pragma unroll 8
        for (int it_ = 0; it_ < (C * DK) / NTH; ++it_) {
            const int idx = tid + it_ * NTH;
            const int r = idx / DK, d = idx % DK;
            const float kb = sA[r * LDK + d] * __builtin_amdgcn_exp2f(gl - sGam[r]);
            if (rr) {
                rr[RR::KB + (size_t)r * DK + d] = (bf16)kb;
            } else {
                out[P::QT + (size_t)r * DK + d] = sQ[r * LDK + d] * __builtin_amdgcn_exp2f(sGam[r]);
                out[P::KB + (size_t)r * DK + d] = kb;
            }
        }
        if (tid < DK) {
            sPhi[tid] = __builtin_amdgcn_exp2f(gl);
            out[P::PHI + tid] = sPhi[tid];
        }
    }
    lds_barrier();
    if (rr) {
        // Q~^T for the reverse pass: 8 positions of one channel per 16-byte
        // store (scalar gates: Q~ = q 2^gamma formed here)
        static_assert((DK * (C / 8)) % NTH == 0, "Q~^T trip count");
        for (int u = tid; u < DK * (C / 8); u += NTH) {
            const int d = u / (C / 8), r0 = (u % (C / 8)) * 8;
            bf16x8 x;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float qv = sQ[(r0 + j) * LDK + d];
                if constexpr (!PERCH) qv *= __builtin_amdgcn_exp2f(sGam[r0 + j]);
                x[j] = (bf16)qv;
            }
            *reinterpret_cast<bf16x8*>(rr + RR::QT + (size_t)d * C + r0) = x;
        }
    }

    // ---- L and Aqk: 16 tiles each, 32 jobs over 4 waves
    for (int job = wave; job < 32; job += NW) {
        const bool isL = job < 16;
        const int t = job & 15, ti = t >> 2, tj = t & 3;
        f32x4 acc = zero4();
        if (ti >= tj && (isL ? DELTA : true)) {
            const float* Aop = isL ? sA : sQ;
            const float* Bop = PERCH ? sB : sA;
            // both operands run along the key channels (contiguous): bf16 MFMA
            // for bf16 I/O, as the forward's products, except Aqk under
            // per-channel gates: q 2^gamma and k 2^-gamma are off the bf16
            // grid, and rounding them loses the small Aqk of nearly orthogonal
            // rows, which reaches dVnew = Aqk^T dO + ... and through it dv
            // and dbeta; that product stays fp32
            if (PERCH && !isL)
                acc = mmk_ab<DK>(acc, Aop + ti * 16 * LDK, LDK, Bop + tj * 16 * LDK, LDK, lane);
            else
                acc = mmc<T, DK>(acc, Aop + ti * 16 * LDK, LDK, Bop + tj * 16 * LDK, LDK, lane);
        }
        bf16x4 at;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = ti * 16 + arow(lane, i), cc = tj * 16 + (lane & 15);
            float x = acc[i];
            if constexpr (!PERCH) x *= (cc <= r) ? __builtin_amdgcn_exp2f(sGam[r] - sGam[cc]) : 0.f;
            if (isL) {
                x = cc < r ? x : 0.f;
                sL[r * LDC + cc] = x;
                out[P::L + (size_t)r * C + cc] = x;
            } else {
                x = cc <= r ? x : 0.f;
                if (waqk) out[P::AQK + (size_t)r * C + cc] = x;
            }
            at[i] = (bf16)x;
        }
        // Aqk^T for the reverse pass: the lane's four rows are adjacent there
        if (!isL && rr)
            *reinterpret_cast<bf16x4*>(rr + RR::AT + (size_t)(tj * 16 + (lane & 15)) * C + ti * 16 + 4 * (lane >> 4)) = at;
    }
    lds_barrier();

    // ---- T = (I + diag(beta) L)^-1, blocked over 16 x 16 blocks:
    //   diagonal blocks T_ii = (I + A_ii)^-1 by forward substitution (one
    //   column per lane, in registers), then by block distance
    //   T_ij = -T_ii sum_{j <= m < i} A_im T_mj  (A = diag(beta) L)
    //   on fp32 MFMA, with sB (free after L and Aqk) as scratch
    if constexpr (DELTA) {
        if (wave == 0) {
            const int o = (lane >> 4) * 16, j = lane & 15;
            float t[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float sacc = 0.f;
#pragma unroll
                for (int m = 0; m < i; ++m) sacc += sL[(o + i) * LDC + o + m] * t[m];
                t[i] = i < j ? 0.f : (i == j ? 1.f : -sBeta[o + i] * sacc);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) sT[(o + i) * LDC + o + j] = t[i];
        } else {
            // zero blocks above the diagonal: 6 blocks of 256 over NTH - 64 threads
            for (int idx = tid - 64; idx < 6 * 256; idx += NTH - 64) {
                const int blk = idx >> 8, e = idx & 255;
                const int bi = blk < 3 ? 0 : (blk < 5 ? 1 : 2);
                const int bj = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
                sT[(bi * 16 + (e >> 4)) * LDC + bj * 16 + (e & 15)] = 0.f;
            }
        }
        lds_barrier();
        float* sX = sB;
#pragma unroll
        for (int dist = 1; dist < 4; ++dist) {
            const int i = dist + wave, j = wave;      // block (i, j), one per wave
            if (i < 4) {
                f32x4 x = zero4();
                for (int m = j; m < i; ++m)
                    x = mmk<16>(x, sL + i * 16 * LDC + m * 16, LDC, 1, sT + m * 16 * LDC + j * 16, LDC, 1, lane);
#pragma unroll
                for (int q = 0; q < 4; ++q) sX[wave * 256 + arow(lane, q) * 16 + (lane & 15)] = sBeta[i * 16 + arow(lane, q)] * x[q];
            }
            lds_barrier();
            if (i < 4) {
                const f32x4 y = mmk<16>(zero4(), sT + i * 16 * LDC + i * 16, LDC, 1, sX + wave * 256, 16, 1, lane);
#pragma unroll
                for (int q = 0; q < 4; ++q) sT[(i * 16 + arow(lane, q)) * LDC + j * 16 + (lane & 15)] = -y[q];
            }
            lds_barrier();
        }
        #pragma unroll 8
        for (int it_ = 0; it_ < (C * C) / NTH; ++it_) {
            const int idx = tid + it_ * NTH;
            out[P::TI + idx] = sT[(idx / C) * LDC + idx % C];
        }
    }

    // ---- M = diag(beta) K+ (in place), W = T M (the forward state pass
    // takes U, and Vnew, from the forward's own kernels)
    if constexpr (DELTA) {
        #pragma unroll 8
        for (int it_ = 0; it_ < (C * DK) / NTH; ++it_) {
            const int idx = tid + it_ * NTH;
            const int r = idx / DK, d = idx % DK;
            sA[r * LDK + d] *= PERCH ? sBeta[r] : sBeta[r] * __builtin_amdgcn_exp2f(sGam[r]);
        }
        lds_barrier();
        // (C/16) x (DK/16) tiles
        constexpr int NTL = 4 * (DK / 16);
        for (int t = wave; t < NTL; t += NW) {
            const int ti = t / (DK / 16), tj = t % (DK / 16);
            // T is lower triangular: the reduction stops at block ti
            f32x4 acc = zero4();
            for (int kb = 0; kb <= ti; ++kb)
                acc = mmk<16>(acc, sT + ti * 16 * LDC + kb * 16, LDC, 1, sA + kb * 16 * LDK + tj * 16, LDK, 1, lane);
            if (rr) {
                // W^T for the reverse pass
                bf16x4 wt;
#pragma unroll
                for (int i = 0; i < 4; ++i) wt[i] = (bf16)acc[i];
                *reinterpret_cast<bf16x4*>(rr + RR::WT + (size_t)(tj * 16 + (lane & 15)) * C + ti * 16 + 4 * (lane >> 4)) = wt;
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    out[P::W + (size_t)(ti * 16 + arow(lane, i)) * DK + tj * 16 + (lane & 15)] = acc[i];
            }
        }
    }
}

// ===========================================================================
// Reverse state pass: one workgroup per (chain, SV = 16 value columns)
// (value columns evolve independently, [KDA] section 3.4).  Consecutive
// logical ids -- the slices of one chain -- are placed on one XCD (hardware
// dispatches workgroup i to XCD i % 8) so they share its L2, and the lines
// of the chunk after the one in flight are pulled into L2 (one 4-byte
// LDS-DMA per 128-byte line into a scratch word).
// ===========================================================================
constexpr int kSV = 16;              // value columns per state-pass workgroup
// LDS row strides.  The tile product reads an operand either with the lane
// index along the row stride (A(r, k) = A[r*s + k]) or along the row (the k
// index strided: transposed A, and B).  With 64 four-byte banks the first is
// conflict-free for s = 4 (mod 64), the second for s = 16 (mod 64); each
// buffer is padded for the way it is read.
constexpr int LSV = kSV;             // [*][16] value-slice tiles, read with k strided

template <int DK>
struct StateSmem {
    static constexpr int LDN = DK + 4;     // [C][DK] read with the lane index along rows
    static constexpr int LDT = DK + 16;    // [C][DK] read transposed
    static constexpr int LCT = C + 16;     // [C][C] read transposed
    // reverse pass
    static constexpr size_t D = 0, KBN = D + (size_t)DK * LSV, QT = KBN + (size_t)C * LDN, WT = QT + (size_t)C * LDT,
                            AQK = WT + (size_t)C * LDT, DV = AQK + (size_t)C * LCT, DV2 = DV + (size_t)C * LSV,
                            DO = DV2 + (size_t)C * LSV,
                            RPHI = DO + (size_t)C * LSV, RSINK = RPHI + DK, REV = RSINK + 64;
};

// Pull the 128-byte lines of [rows][cols] fp32 blocks (row stride gs) into
// L2: one 4-byte LDS-DMA per line, spread over the workgroup's threads.
__device__ __forceinline__ void l2_touch(const float* __restrict__ src, size_t gs, int rows, int cols, int tid,
                                         int nthr, float* sink) {
    const int lpr = (cols * 4 + 127) / 128;    // lines per row (rows start 16-byte aligned)
    for (int idx = tid; idx < rows * lpr; idx += nthr) {
        const int r = idx / lpr, l = idx % lpr;
        const auto gp = (const __attribute__((address_space(1))) void*)(src + r * gs + 32 * l);
        __builtin_amdgcn_global_load_lds(gp, (__attribute__((address_space(3))) void*)sink, 4, 0, 0);
    }
}

// The reverse pass runs 8 waves, two per SIMD, so that one wave's LDS and
// memory waits overlap the other's products.  Each chunk's operands are
// loaded one step ahead into registers: Aqk, Kbar and dO right after the
// previous step's copies went to LDS in (A), Q~ and W after theirs in (B).
// Per chunk, three barriers separate: (A) Aqk, Kbar, dO to LDS; (B) the
// dVnew products, Q~ and W to LDS, the exit adjoint dS'_c stored; (C) the
// adjoint update in place, dVnew stored.
constexpr int kStateThreads = 512;

// acc += A (B1 + B2) with the layout of mmk: the B operand is the sum of two
// LDS tiles (the two halves of a split reduction), added as it is read.
template <int K>
__device__ __forceinline__ f32x4 mmk2(f32x4 acc, const float* A, int ar, int ak, const float* B1, const float* B2,
                                      int bk, int bc, int lane) {
    const int r = lane & 15, q = lane >> 4;
    const float* a = A + r * ar + q * ak;
    const int bo = q * bk + r * bc;
#pragma unroll 8
    for (int k0 = 0; k0 < K; k0 += 4)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[k0 * ak], B1[bo + k0 * bk] + B2[bo + k0 * bk], acc, 0, 0, 0);
    return acc;
}

// Reverse state pass, chunks in reverse: writes dS'_c (the exit-state adjoint
// of chunk c) and dVnew_c, and dh0.
template <int KIND, typename T, int DK>
__global__ __launch_bounds__(kStateThreads) void bwd_state_rev_kernel(const float* __restrict__ prep,
                                                                      const T* __restrict__ dout,
                                                                      const float* __restrict__ dhT,
                                                                      T* __restrict__ dhs,
                                                                      T* __restrict__ dvn,
                                                                      float* __restrict__ dh0, int Tlen, int H,
                                                                      int NT, Pack pk)
{
    using P = Prep<DK>;
    using SM = StateSmem<DK>;
    constexpr int DV = DK, LDN = SM::LDN, LDT = SM::LDT, LCT = SM::LCT, NVS = DV / kSV, NC = kStateThreads;
    constexpr bool DELTA = KIND != KIND_LA;
    // dVnew tile ti is split over waves ti and ti + 4: wave ti takes Aqk^T dO
    // and the first KS key channels of Kbar dS', wave ti + 4 the rest
    constexpr int KS = (DK - C) / 2;
    __shared__ __attribute__((aligned(16))) float smem[SM::REV];
    float* sD = smem + SM::D;         // dS'
    float* sKb = smem + SM::KBN;
    float* sQt = smem + SM::QT;
    float* sW = smem + SM::WT;
    float* sAqk = smem + SM::AQK;
    float* sDV = smem + SM::DV;       // dVnew = sDV + sDV2
    float* sDV2 = smem + SM::DV2;
    float* sDO = smem + SM::DO;
    float* sPhi = smem + SM::RPHI;
    float* sink = smem + SM::RSINK;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int logical = xcd_logical(blockIdx.x, gridDim.x);
    const int chain = chain_of(pk, logical / NVS, H, (int)gridDim.x / NVS), dv0 = (logical % NVS) * kSV;
    const int h = chain % H;
    const ChainLoc cl = locate_chain(pk, chain, H, Tlen, NT);
    constexpr int NDO = (C * kSV) / NC;
    Staged<C, C, NC> ga;
    Staged<C, DK, NC> gk, gq, gw;
    float xo[NDO];
    float ph = 0.f;
    // every load unconditional: rows of dO past the end read the last row
    auto load_a = [&](int c) {
        const float* pc = prep + (cl.ci0 + c) * P::FLOATS;
        ga.load(pc + P::AQK, C, tid);
        gk.load(pc + P::KB, DK, tid);
        ph = tid < DK ? pc[P::PHI + tid] : 0.f;
#pragma unroll
        for (int it_ = 0; it_ < NDO; ++it_) {
            const int idx = tid + it_ * NC, r = idx / kSV, cc = idx % kSV;
            xo[it_] = to_f(dout[((cl.tok0 + min(c * C + r, cl.tlim - 1)) * H + h) * DV + dv0 + cc]);
        }
    };
    auto load_b = [&](int c) {
        const float* pc = prep + (cl.ci0 + c) * P::FLOATS;
        gq.load(pc + P::QT, DK, tid);
        if constexpr (DELTA) gw.load(pc + P::W, DK, tid);
    };
    if (cl.nseg > 0) {
        load_a(cl.nseg - 1);
        load_b(cl.nseg - 1);
    }
#pragma unroll
    for (int it_ = 0; it_ < (DK * kSV) / NC; ++it_) {
        const int idx = tid + it_ * NC, r = idx / kSV, cc = idx % kSV;
        sD[r * LSV + cc] = dhT ? dhT[((size_t)chain * DK + r) * DV + dv0 + cc] : 0.f;
    }
    lds_barrier();
    for (int c = cl.nseg - 1; c >= 0; --c) {
        const size_t ci = cl.ci0 + c;
        const int cn = c > 0 ? c - 1 : 0;    // the next chunk (the last reloads itself)
        // (A) Aqk, Kbar, dO, phi to LDS; the next chunk's copies in flight
        ga.store(sAqk, LCT, tid);
        gk.store(sKb, LDN, tid);
        if (tid < DK) sPhi[tid] = ph;
#pragma unroll
        for (int it_ = 0; it_ < NDO; ++it_) {
            const int idx = tid + it_ * NC, r = idx / kSV, cc = idx % kSV;
            sDO[r * LSV + cc] = c * C + r < cl.tlim ? xo[it_] : 0.f;
        }
        load_a(cn);
        lds_barrier();
        // (B) dVnew = Aqk^T dO + Kbar dS': 4 tiles, two waves each; Q~ and W
        // (read only in (C)) to LDS, the next chunk's in flight; dS'_c out
        {
            const int ti = wave & 3;
            f32x4 acc = zero4();
            if (wave < 4) {
                acc = mmk<C>(acc, sAqk + ti * 16, 1, LCT, sDO, LSV, 1, lane);
                if constexpr (KS > 0) acc = mmk_a<KS>(acc, sKb + ti * 16 * LDN, LDN, sD, LSV, 1, lane);
            } else {
                acc = mmk_a<DK - KS>(acc, sKb + ti * 16 * LDN + KS, LDN, sD + KS * LSV, LSV, 1, lane);
            }
            float* dst = wave < 4 ? sDV : sDV2;
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[(ti * 16 + arow(lane, i)) * LSV + (lane & 15)] = acc[i];
            gq.store(sQt, LDT, tid);
            if constexpr (DELTA) gw.store(sW, LDT, tid);
            load_b(cn);
            constexpr int NS = (DK * kSV) / 4 < NC ? (DK * kSV) / 4 : NC;
            if (tid < NS) unstage<DK, kSV, NS>(dhs + ci * DK * DV + slc(0, dv0, DK), 32, sD, LSV, tid);
            // the lines of the chunk after the one in flight into L2
            if (c > 1) {
                const float* pn = prep + (ci - 2) * P::FLOATS;
                l2_touch(pn + P::AQK, C, C, C, tid, NC, sink);
                l2_touch(pn + P::KB, DK, C, DK, tid, NC, sink);
                l2_touch(pn + P::QT, DK, C, DK, tid, NC, sink);
                if constexpr (DELTA) l2_touch(pn + P::W, DK, C, DK, tid, NC, sink);
            }
        }
        lds_barrier();
        // (C) dS = Q~^T dO + diag(phi) dS' - W^T dVnew, in place, one tile
        // per wave; dVnew = sDV + sDV2 out
        {
            static_assert(DK / 16 <= 8, "one adjoint tile per wave");
            const int ti = wave;
            if (ti < DK / 16) {
                f32x4 acc;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = ti * 16 + arow(lane, i);
                    acc[i] = sPhi[r] * sD[r * LSV + (lane & 15)];
                }
                acc = mmk<C>(acc, sQt + ti * 16, 1, LDT, sDO, LSV, 1, lane);
                if constexpr (DELTA) {
                    const f32x4 wv = mmk2<C>(zero4(), sW + ti * 16, 1, LDT, sDV, sDV2, LSV, 1, lane);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i] -= wv[i];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) sD[(ti * 16 + arow(lane, i)) * LSV + (lane & 15)] = acc[i];
            }
            if (tid < (C * kSV) / 4) {
                const int r = tid / (kSV / 4), c4 = (tid % (kSV / 4)) * 4;
                const f32x4 x = *reinterpret_cast<const f32x4*>(sDV + r * LSV + c4);
                const f32x4 y = *reinterpret_cast<const f32x4*>(sDV2 + r * LSV + c4);
                st4(dvn + ci * C * DV + slc(r, dv0 + c4, C), x + y);
            }
        }
        lds_barrier();
    }
    if (dh0 && tid < 256) unstage<DK, kSV, 256>(dh0 + (size_t)chain * DK * DV + dv0, DV, sD, LSV, tid);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ===========================================================================
// Gradients: one 512-thread workgroup per (chunk, head, batch).
// ===========================================================================
template <int DK>
struct GradSmem {
    static constexpr int LDK = DK + 4;
    static constexpr size_t MAT = (size_t)C * LDK, SQ = (size_t)C * LDC;
    static constexpr size_t SL = (size_t)DK * LVS, VS = (size_t)C * LVS;
    // phase 1
    static constexpr size_t KP = 0;                 // K+ (kda) or k (scalar): persists
    static constexpr size_t TI = KP + MAT;          // T
    static constexpr size_t S1 = TI + SQ, DS1 = S1 + SL, VN1 = DS1 + SL, DVN1 = VN1 + VS, DO1 = DVN1 + VS,
                            V1 = DO1 + VS, P1 = V1 + VS, END1 = P1 + VS;
    // phase 2 (after phase 1): nW at TI + SQ; dT, Y at TI + SQ, TI + 2 SQ; dL, dAqk; then K- / raw q and Q~
    static constexpr size_t NW = TI + SQ, DT = TI + SQ, Y = TI + 2 * SQ, DL = TI + 3 * SQ, DAQK = TI + 4 * SQ,
                            KM = TI, QT = TI + 5 * SQ, END2 = QT + MAT;
    static constexpr size_t E = TI;                  // phase 3: E over the K- slot
    static constexpr size_t BIG = END1 > END2 ? END1 : END2;
    // reductions in a fixed order: dbeta partials [NDB][C], one slot per
    // source (the phase-1 value tiles' two column halves, the DK/16 column
    // tiles of phase 2a, the four column tiles of phase 2b), each written by
    // one wave; the column sums of dKbar * Kbar [8][16] per wave
    static constexpr int NDB = 2 + DK / 16 + 4;
    static constexpr size_t DB = BIG, SE = DB + (size_t)NDB * C, GAM = SE + C, PHI = GAM + C, FCOL = PHI + DK,
                            FP = FCOL + DK, DPHI = FP + 128, ROW = DPHI + DK, BT = ROW + C, FLOATS = BT + C;
    static_assert(FLOATS * 4 <= 160 * 1024, "LDS");
    static_assert(KM + MAT <= DL, "K- slot overlaps dL");
    static_assert(NW + MAT <= DL, "nW slot overlaps dL");
};

template <int KIND, typename T, int DK>
__global__ __launch_bounds__(512) void bwd_grad_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ beta,
    const T* __restrict__ dout, const float* __restrict__ prep, const T* __restrict__ hs,
    const T* __restrict__ dhs, const T* __restrict__ vn, const T* __restrict__ dvn,
    T* __restrict__ dq, T* __restrict__ dk, T* __restrict__ dv, float* __restrict__ dg, float* __restrict__ dbeta,
    int Tlen, int H, int NT, Pack pk)
{
    using P = Prep<DK>;
    using SM = GradSmem<DK>;
    constexpr int DV = DK, LDK = SM::LDK, NCT = DK / 16, NTL = 4 * NCT, OWN = NTL / 8, NVS = DV / kVS;
    constexpr bool DELTA = KIND != KIND_LA;
    constexpr bool PERCH = KIND == KIND_KDA;
    __shared__ __attribute__((aligned(16))) float smem[SM::FLOATS];
    float* sKp = smem + SM::KP;
    float* sT = smem + SM::TI;
    float* sDb = smem + SM::DB;
    float* sE = smem + SM::SE;
    float* sGam = smem + SM::GAM;
    float* sPhi = smem + SM::PHI;
    float* sF = smem + SM::FCOL;
    float* sFp = smem + SM::FP;
    float* sDphi = smem + SM::DPHI;
    float* sRow = smem + SM::ROW;
    float* sBt = smem + SM::BT;      // beta, zero past the end and for decay_la

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    ChunkLoc loc;
    if (!locate_chunk(pk, blockIdx.x, H, Tlen, NT, loc)) return;
    const int nvalid = loc.nvalid;
    const size_t row0 = loc.row0;
    const size_t ci = loc.ci;
    const float* pc = prep + ci * P::FLOATS;

    // owned tiles of every [C][DK] result: t = wave + 8 m
    auto trc = [&](int m, int& ti, int& tj) { const int t = wave + 8 * m; ti = t / NCT; tj = t % NCT; };
    // element (r, d) of owned tile m, accumulator slot i
    auto erow = [&](int m, int i) { int ti, tj; trc(m, ti, tj); return ti * 16 + arow(lane, i); };
    auto ecol = [&](int m) { int ti, tj; trc(m, ti, tj); return tj * 16 + (lane & 15); };
    // gamma (log2) and e = 2^gamma at element (r, d)
    auto gam_at = [&](int r, int d) { return PERCH ? pc[P::GAM + (size_t)r * DK + d] : sGam[r]; };
    auto in_at = [&](const T* __restrict__ x, int r, int d) {
        const float y = to_f(x[(row0 + (size_t)min(r, nvalid - 1) * H) * DK + d]);
        return r < nvalid ? y : 0.f;
    };

    // ---- set-up: K+ (or k), T, beta, gamma, phi
    // four adjacent channels per thread and access
#pragma unroll
    for (int it_ = 0; it_ < (C * DK) / (4 * 512); ++it_) {
        const int idx = tid + it_ * 512;
        const int r = idx / (DK / 4), d0 = (idx % (DK / 4)) * 4;
        const bool ok = r < nvalid;
        Raw4<T> xk;
        xk.load(k + (row0 + (size_t)min(r, nvalid - 1) * H) * DK + d0);
        f32x4 kp;
        if constexpr (PERCH) {
            const f32x4 gm = *reinterpret_cast<const f32x4*>(pc + P::GAM + (size_t)r * DK + d0);
#pragma unroll
            for (int j = 0; j < 4; ++j) kp[j] = (ok ? xk[j] : 0.f) * __builtin_amdgcn_exp2f(gm[j]);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) kp[j] = ok ? xk[j] : 0.f;
        }
        *reinterpret_cast<f32x4*>(sKp + r * LDK + d0) = kp;
    }
    if constexpr (DELTA) stage<C, C, 512>(sT, LDC, pc + P::TI, C, tid);
    if (tid < C) {
        const float bb = DELTA ? beta[row0 + (size_t)min(tid, nvalid - 1) * H] : 0.f;
        sBt[tid] = tid < nvalid ? bb : 0.f;
#pragma unroll
        for (int j = 0; j < SM::NDB; ++j) sDb[j * C + tid] = 0.f;
        sE[tid] = 0.f;
        sRow[tid] = 0.f;
        if constexpr (!PERCH) sGam[tid] = pc[P::GAM + tid];
    }
    if (tid < DK) {
        sPhi[tid] = pc[P::PHI + tid];
        sF[tid] = 0.f;
    }
    lds_barrier();
    auto beta_at = [&](int r) { return sBt[r]; };
    // row scale of M = diag(rs) K+ (scalar gates: K+ = k 2^gamma_r)
    auto mscale = [&](int r) { return PERCH ? beta_at(r) : beta_at(r) * __builtin_amdgcn_exp2f(sGam[r]); };

    // ---- phase 1: value slices
    f32x4 dQt[OWN], nW[OWN], dKb[OWN], dAqk[2], dT[2];
#pragma unroll
    for (int m = 0; m < OWN; ++m) dQt[m] = nW[m] = dKb[m] = zero4();
    dAqk[0] = dAqk[1] = dT[0] = dT[1] = zero4();
    float dphi = 0.f;
    float* s1 = smem + SM::S1;
    float* ds1 = smem + SM::DS1;
    float* vn1 = smem + SM::VN1;
    float* dvn1 = smem + SM::DVN1;
    float* do1 = smem + SM::DO1;
    float* v1 = smem + SM::V1;
    float* p1 = smem + SM::P1;
    // the value slices travel one slice ahead in registers: slice s+1 loads
    // during slice s's products (the last slice reloads itself, so that the
    // loads stay unconditional)
    Staged<DK, kVS, 512, T> g1, g2;
    Staged<C, kVS, 512, T> g3, g4;
    constexpr int NE = (C * kVS) / 512;
    float xd[NE], xv[NE];
    auto load_slice = [&](int dv0) {
        // one slice of the slice-major state arrays (slc()): contiguous
        g1.load(hs + ci * DK * DV + slc(0, dv0, DK), 32, tid);
        g2.load(dhs + ci * DK * DV + slc(0, dv0, DK), 32, tid);
        g3.load(vn + ci * C * DV + slc(0, dv0, C), 32, tid);
        g4.load(dvn + ci * C * DV + slc(0, dv0, C), 32, tid);
#pragma unroll
        for (int it_ = 0; it_ < NE; ++it_) {
            const int idx = tid + it_ * 512, r = idx / kVS, cc = idx % kVS;
            const size_t off = (row0 + (size_t)min(r, nvalid - 1) * H) * DV + dv0 + cc;
            xd[it_] = to_f(dout[off]);
            xv[it_] = to_f(v[off]);
        }
    };
    load_slice(0);
    for (int s = 0; s < NVS; ++s) {
        const int dv0 = s * kVS;
        {
            g1.store(s1, LVS, tid);
            g2.store(ds1, LVS, tid);
            g3.store(vn1, LVS, tid);
            g4.store(dvn1, LVS, tid);
#pragma unroll
            for (int it_ = 0; it_ < NE; ++it_) {
                const int idx = tid + it_ * 512, r = idx / kVS, cc = idx % kVS;
                do1[r * LVS + cc] = r < nvalid ? xd[it_] : 0.f;
                v1[r * LVS + cc] = r < nvalid ? xv[it_] : 0.f;
            }
        }
        lds_barrier();
        load_slice(min(s + 1, NVS - 1) * kVS);
        {
            const int ti = wave >> 1, tj = wave & 1;    // one [C][32] tile per wave
            if constexpr (DELTA) {
                // P = N - M S_s (N = diag(beta) V), and dN = T^T dVnew -> dv, dbeta
                // fp32 I/O: fp32 MFMA.  bf16 I/O: the S and dVnew slices hold
                // bf16 values, so bf16 MFMA with K+ (KDA; scalar gates: the
                // bf16 k itself) and T split into high and low parts keeps
                // about 16 bits of them (these products reach dv and dbeta)
                f32x4 x, dn;
                if constexpr (sizeof(T) == 2) {
                    x = mms<DK, true, PERCH>(zero4(), sKp + ti * 16 * LDK, LDK, 1, s1 + tj * 16, LVS, 1, lane);
                    dn = mms<C, false, true>(zero4(), sT + ti * 16, 1, LDC, dvn1 + tj * 16, LVS, 1, lane);
                } else {
                    x = mmk_a<DK>(zero4(), sKp + ti * 16 * LDK, LDK, s1 + tj * 16, LVS, 1, lane);
                    dn = mmk<C>(zero4(), sT + ti * 16, 1, LDC, dvn1 + tj * 16, LVS, 1, lane);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = ti * 16 + arow(lane, i), cc = tj * 16 + (lane & 15);
                    const float bt = beta_at(r), vv = v1[r * LVS + cc];
                    p1[r * LVS + cc] = bt * vv - mscale(r) * x[i];
                    if (r < nvalid) dv[(row0 + (size_t)r * H) * DV + dv0 + cc] = from_f<T>(bt * dn[i]);
                    float part = dn[i] * vv;
                    part = row16_sum(part);
                    // slot tj: this wave alone adds to it, slice after slice
                    if ((lane & 15) == 0) sDb[tj * C + r] += part;
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = ti * 16 + arow(lane, i), cc = tj * 16 + (lane & 15);
                    if (r < nvalid) dv[(row0 + (size_t)r * H) * DV + dv0 + cc] = from_f<T>(dvn1[r * LVS + cc]);
                }
            }
        }
        // dphi_d += sum over the slice of S .* dS' in row d: four lanes per
        // row, eight columns each, quad sum by DPP (every lane of the quad
        // keeps the row's total)
        if (tid < DK * 4) {
            const int d = tid >> 2, c0 = (tid & 3) * (kVS / 4);
            float part = 0.f;
#pragma unroll
            for (int e = 0; e < kVS / 4; e += 4) {
                const f32x4 a = *reinterpret_cast<const f32x4*>(s1 + d * LVS + c0 + e);
                const f32x4 b = *reinterpret_cast<const f32x4*>(ds1 + d * LVS + c0 + e);
                part += a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
            }
            part += dpp_peer<0xB1>(part);
            part += dpp_peer<0x4E>(part);
            dphi += part;
        }
        lds_barrier();
        // one product at a time (compiler barriers between them keep the
        // LDS operand loads of different products from piling up in registers)
#pragma unroll
        for (int m = 0; m < OWN; ++m) {
            int ti, tj;
            trc(m, ti, tj);
            dQt[m] = mmc<T, kVS>(dQt[m], do1 + ti * 16 * LVS, LVS, s1 + tj * 16 * LVS, LVS, lane);
            asm volatile("" ::: "memory");
        }
#pragma unroll
        for (int m = 0; m < OWN; ++m) {
            int ti, tj;
            trc(m, ti, tj);
            nW[m] = mmc<T, kVS>(nW[m], dvn1 + ti * 16 * LVS, LVS, s1 + tj * 16 * LVS, LVS, lane);
            asm volatile("" ::: "memory");
        }
#pragma unroll
        for (int m = 0; m < OWN; ++m) {
            int ti, tj;
            trc(m, ti, tj);
            dKb[m] = mmc<T, kVS>(dKb[m], vn1 + ti * 16 * LVS, LVS, ds1 + tj * 16 * LVS, LVS, lane);
            asm volatile("" ::: "memory");
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int t = wave + 8 * m, ti = t >> 2, tj = t & 3;
            dAqk[m] = mmc<T, kVS>(dAqk[m], do1 + ti * 16 * LVS, LVS, vn1 + tj * 16 * LVS, LVS, lane);
            if constexpr (DELTA)
                dT[m] = mmc<T, kVS>(dT[m], dvn1 + ti * 16 * LVS, LVS, p1 + tj * 16 * LVS, LVS, lane);
        }
        lds_barrier();
    }
    if (tid < DK * 4 && (tid & 3) == 0) sDphi[tid >> 2] = dphi;

    // ---- per-element accumulators: dq, dk, E (gamma adjoint, natural units)
    f32x4 aq[OWN], ak[OWN], aE[OWN];
    // e = 2^gamma at every owned element, kept for the later phases; the
    // element loads (gamma, q, k) are issued together, ahead of their use
    f32x4 ee[OWN];
    f32x4 lq[OWN], lk[OWN], lg[OWN];
    float lgl[OWN];
#pragma unroll
    for (int m = 0; m < OWN; ++m) {
        const int d = ecol(m);
        lgl[m] = PERCH ? pc[P::GAM + (size_t)(C - 1) * DK + d] : sGam[C - 1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = erow(m, i);
            lg[m][i] = gam_at(r, d);
            lq[m][i] = in_at(q, r, d);
            lk[m][i] = in_at(k, r, d);
        }
    }
    // sum of dKbar * Kbar over this lane's elements: every owned tile of a
    // wave has the same 16 columns (t = wave + 8m, NCT divides 8), so a lane
    // keeps one column d = ecol(0)
    float fpart = 0.f;
#pragma unroll
    for (int m = 0; m < OWN; ++m) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float gm = lg[m][i], e = __builtin_amdgcn_exp2f(gm);
            ee[m][i] = e;
            const float qq = lq[m][i], kk = lk[m][i];
            // Q~ = q e;  Kbar = k 2^(gamma_last - gamma)
            const float kbf = __builtin_amdgcn_exp2f(lgl[m] - gm);
            const float kbar = kk * kbf;
            aq[m][i] = dQt[m][i] * e;
            ak[m][i] = dKb[m][i] * kbf;
            aE[m][i] = dQt[m][i] * qq * e - dKb[m][i] * kbar;
            fpart += dKb[m][i] * kbar;
        }
    }
    static_assert(8 % NCT == 0, "owned tiles share their columns");
    // the four row groups of a column (lanes l, l+16, l+32, l+48)
    fpart += __shfl_xor(fpart, 16, 64);
    fpart += __shfl_xor(fpart, 32, 64);
    // one slot per contributing wave (waves w and w + NCT share columns)
    if constexpr (PERCH) {
        if (lane < 16) sFp[(wave / NCT) * DK + ecol(0)] = fpart;
    } else {
        fpart = row16_sum(fpart);
        if (lane == 0) sFp[wave] = fpart;
    }

    if constexpr (DELTA) {
        // ---- phase 2a: dM = T^T dW = -T^T nW
        float* sNW = smem + SM::NW;
#pragma unroll
        for (int m = 0; m < OWN; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) sNW[erow(m, i) * LDK + ecol(m)] = nW[m][i];
        lds_barrier();
#pragma unroll
        for (int m = 0; m < OWN; ++m) {
            int ti, tj;
            trc(m, ti, tj);
            const f32x4 acc = mmp<T, C, false>(zero4(), sT + ti * 16, 1, LDC, sNW + tj * 16, LDK, 1, lane);
            const int d = ecol(m);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = erow(m, i);
                const float dm = -acc[i];
                const float e = ee[m][i];
                const float kp = PERCH ? sKp[r * LDK + d] : sKp[r * LDK + d] * e;   // K+ = k e
                const float bt = beta_at(r);
                // M = diag(beta) K+ with K+ = k e:  dk += beta e dM,  E += dM M,  dbeta += dM K+
                ak[m][i] += bt * e * dm;
                aE[m][i] += dm * bt * kp;
                float part = dm * kp;
                part = row16_sum(part);
                if ((lane & 15) == 0) sDb[(2 + tj) * C + r] = part;
            }
        }
        lds_barrier();
        // ---- phase 2b: dA = -T^T dT T^T (strictly lower), dL = diag(beta) dA
        float* sDT = smem + SM::DT;
        float* sY = smem + SM::Y;
        float* sDL = smem + SM::DL;
        // L at this lane's dA elements, loaded ahead of the two products
        float lrc[2][4];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int t = wave + 8 * m, ti = t >> 2, tj = t & 3;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                lrc[m][i] = pc[P::L + (size_t)(ti * 16 + arow(lane, i)) * C + tj * 16 + (lane & 15)];
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int t = wave + 8 * m, ti = t >> 2, tj = t & 3;
#pragma unroll
            for (int i = 0; i < 4; ++i) sDT[(ti * 16 + arow(lane, i)) * LDC + tj * 16 + (lane & 15)] = dT[m][i];
        }
        lds_barrier();
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int t = wave + 8 * m, ti = t >> 2, tj = t & 3;
            f32x4 acc;
            if constexpr (sizeof(T) == 2) acc = mmb<C>(zero4(), sDT + ti * 16 * LDC, LDC, sT + tj * 16 * LDC, LDC, lane);
            else acc = mmk_ab<C>(zero4(), sDT + ti * 16 * LDC, LDC, sT + tj * 16 * LDC, LDC, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) sY[(ti * 16 + arow(lane, i)) * LDC + tj * 16 + (lane & 15)] = acc[i];
        }
        lds_barrier();
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int t = wave + 8 * m, ti = t >> 2, tj = t & 3;
            const f32x4 acc = mmp<T, C, false>(zero4(), sT + ti * 16, 1, LDC, sY + tj * 16, LDC, 1, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = ti * 16 + arow(lane, i), cc = tj * 16 + (lane & 15);
                const float da = cc < r ? -acc[i] : 0.f;
                sDL[r * LDC + cc] = beta_at(r) * da;
                float part = da * lrc[m][i];
                part = row16_sum(part);
                if ((lane & 15) == 0) sDb[(2 + NCT + tj) * C + r] = part;
            }
        }
    }
    // ---- dAqk (lower incl.) to LDS
    float* sDAqk = smem + SM::DAQK;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int t = wave + 8 * m, ti = t >> 2, tj = t & 3;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = ti * 16 + arow(lane, i), cc = tj * 16 + (lane & 15);
            sDAqk[r * LDC + cc] = cc <= r ? dAqk[m][i] : 0.f;
        }
    }
    lds_barrier();

    // ---- phase 2c: the pairwise products
    float* sKm = smem + SM::KM;     // kda: K-;  scalar: raw q
    float* sQt = smem + SM::QT;     // kda: Q~
    float* sDL = smem + SM::DL;
    // four adjacent channels per thread and access
    constexpr int DK4 = DK / 4;
    #pragma unroll 4
    for (int it_ = 0; it_ < (C * DK4) / 512; ++it_) {
        const int idx = tid + it_ * 512;
        const int r = idx / DK4, d0 = (idx % DK4) * 4;
        const bool ok = r < nvalid;
        const size_t go = (row0 + (size_t)min(r, nvalid - 1) * H) * DK + d0;
        Raw4<T> xq;
        xq.load(q + go);
        if constexpr (PERCH) {
            Raw4<T> xk;
            xk.load(k + go);
            const f32x4 gm = *reinterpret_cast<const f32x4*>(pc + P::GAM + (size_t)r * DK + d0);
            f32x4 km, qt;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                km[j] = (ok ? xk[j] : 0.f) * __builtin_amdgcn_exp2f(-gm[j]);
                qt[j] = (ok ? xq[j] : 0.f) * __builtin_amdgcn_exp2f(gm[j]);
            }
            *reinterpret_cast<f32x4*>(sKm + r * LDK + d0) = km;
            *reinterpret_cast<f32x4*>(sQt + r * LDK + d0) = qt;
        } else {
            f32x4 qv;
#pragma unroll
            for (int j = 0; j < 4; ++j) qv[j] = ok ? xq[j] : 0.f;
            *reinterpret_cast<f32x4*>(sKm + r * LDK + d0) = qv;
        }
    }
    // scalar gates: the pair terms c_ij = dX_ij X_ij go to a [C][C] matrix in
    // the Y slot (free in this phase), summed by rows and columns below
    float* sCx = smem + SM::Y;
    if constexpr (!PERCH) {
        // G = dX .* Gamma in place, and the log-gate terms of the pair products:
        // E_i += sum_j dX_ij X_ij,  E_j -= sum_i dX_ij X_ij  (X = L, Aqk)
        #pragma unroll 8
        for (int it_ = 0; it_ < (C * C) / 512; ++it_) {
            const int idx = tid + it_ * 512;
            const int r = idx / C, cc = idx % C;
            float contrib = 0.f;
            if (cc <= r) {
                const float gmm = __builtin_amdgcn_exp2f(sGam[r] - sGam[cc]);
                const float daq = sDAqk[r * LDC + cc];
                contrib += daq * pc[P::AQK + idx];
                sDAqk[r * LDC + cc] = daq * gmm;
                if constexpr (DELTA) {
                    const float dl = sDL[r * LDC + cc];
                    contrib += dl * pc[P::L + idx];
                    sDL[r * LDC + cc] = dl * gmm;
                }
            }
            sCx[r * LDC + cc] = contrib;
        }
    }
    lds_barrier();
    if constexpr (!PERCH) {
        // E_r = sum_{c <= r} c_rc - sum_{r' >= r} c_r'r, in a fixed order
        // (read in phase 3, after its barrier)
        if (tid < C) {
            float e = 0.f;
            for (int c2 = 0; c2 <= tid; ++c2) e += sCx[tid * LDC + c2];
            for (int r2 = tid; r2 < C; ++r2) e -= sCx[r2 * LDC + tid];
            sE[tid] = e;
        }
    }
    if constexpr (PERCH) {
        // dK+ += dL K-;  dK- = dL^T K+ + dAqk^T Q~;  dQ~ += dAqk K- (one
        // product at a time over the owned tiles, which keeps few results live)
#pragma unroll
        for (int m = 0; m < OWN; ++m) {
            int ti, tj;
            trc(m, ti, tj);
            const int d = ecol(m);
            const f32x4 dkp = mmp<T, C, true>(zero4(), sDL + ti * 16 * LDC, LDC, 1, sKm + tj * 16, LDK, 1, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = erow(m, i);
                ak[m][i] += dkp[i] * ee[m][i];
                aE[m][i] += dkp[i] * sKp[r * LDK + d];
            }
        }
#pragma unroll
        for (int m = 0; m < OWN; ++m) {
            int ti, tj;
            trc(m, ti, tj);
            const int d = ecol(m);
            f32x4 dkm = mmp<T, C, false>(zero4(), sDL + ti * 16, 1, LDC, sKp + tj * 16, LDK, 1, lane);
            dkm = mmp<T, C, false>(dkm, sDAqk + ti * 16, 1, LDC, sQt + tj * 16, LDK, 1, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = erow(m, i);
                ak[m][i] += dkm[i] / ee[m][i];
                aE[m][i] -= dkm[i] * sKm[r * LDK + d];
            }
        }
#pragma unroll
        for (int m = 0; m < OWN; ++m) {
            int ti, tj;
            trc(m, ti, tj);
            const int d = ecol(m);
            const f32x4 dqt = mmp<T, C, true>(zero4(), sDAqk + ti * 16 * LDC, LDC, 1, sKm + tj * 16, LDK, 1, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = erow(m, i);
                aq[m][i] += dqt[i] * ee[m][i];
                aE[m][i] += dqt[i] * sQt[r * LDK + d];
            }
        }
    }
#pragma unroll
    for (int m = 0; m < OWN; ++m) {
        int ti, tj;
        trc(m, ti, tj);
        if constexpr (PERCH) {
        } else {
            // raw k (sKp), raw q (sKm): dk += G_L k + G_L^T k + G_Q^T q;  dq += G_Q k
            f32x4 dkk = mmp<T, C, false>(zero4(), sDAqk + ti * 16, 1, LDC, sKm + tj * 16, LDK, 1, lane);
            if constexpr (DELTA) {
                dkk = mmp<T, C, true>(dkk, sDL + ti * 16 * LDC, LDC, 1, sKp + tj * 16, LDK, 1, lane);
                dkk = mmp<T, C, false>(dkk, sDL + ti * 16, 1, LDC, sKp + tj * 16, LDK, 1, lane);
            }
            const f32x4 dqq = mmp<T, C, true>(zero4(), sDAqk + ti * 16 * LDC, LDC, 1, sKp + tj * 16, LDK, 1, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ak[m][i] += dkk[i];
                aq[m][i] += dqq[i];
            }
        }
    }
    lds_barrier();

    // ---- phase 3: write dq, dk; E to LDS, then the reverse cumsum per column
    float* sEm = smem + SM::E;
    // dq, dk staged in LDS (the phase 2 buffers past E) so that they leave as
    // four adjacent channels per access
    float* sDq = smem + SM::Y;
    float* sDk = sDq + SM::MAT;
    static_assert(SM::Y >= SM::E + SM::MAT && SM::Y + 2 * SM::MAT <= SM::END2, "dq/dk staging");
#pragma unroll
    for (int m = 0; m < OWN; ++m) {
        const int d = ecol(m);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = erow(m, i);
            sEm[r * LDK + d] = aE[m][i];
            sDq[r * LDK + d] = aq[m][i];
            sDk[r * LDK + d] = ak[m][i];
        }
    }
    lds_barrier();
    {
        constexpr int DK4 = DK / 4;
#pragma unroll
        for (int it_ = 0; it_ < (C * DK4) / 512; ++it_) {
            const int idx = tid + it_ * 512;
            const int r = idx / DK4, d0 = (idx % DK4) * 4;
            if (r < nvalid) {
                const size_t off = (row0 + (size_t)r * H) * DK + d0;
                st4(dq + off, *reinterpret_cast<const f32x4*>(sDq + r * LDK + d0));
                st4(dk + off, *reinterpret_cast<const f32x4*>(sDk + r * LDK + d0));
            }
        }
    }
    if constexpr (PERCH) {
        // reverse cumsum down each column, 512 / DK threads per column, each
        // over a block of rows: block sums, then each block's scan from the
        // sum of the blocks below it
        constexpr int NB = 512 / DK, RB = C / NB;
        float* sBlk = smem + SM::KP;     // [NB][DK]: K+ is no longer read
        static_assert(SM::KP + NB * DK <= SM::E, "block sums overlap E");
        const int d = tid % DK, b = tid / DK;
        float bs = 0.f;
#pragma unroll
        for (int j = 0; j < RB; ++j) bs += sEm[(b * RB + j) * LDK + d];
        sBlk[b * DK + d] = bs;
        lds_barrier();
        float fsum = 0.f;
#pragma unroll
        for (int sl = 0; sl < 8 / NCT; ++sl) fsum += sFp[sl * DK + d];
        float acc = fsum + sDphi[d] * sPhi[d];
#pragma unroll
        for (int b2 = NB - 1; b2 > b; --b2) acc += sBlk[b2 * DK + d];
#pragma unroll
        for (int j = RB - 1; j >= 0; --j) {
            const int r = b * RB + j;
            acc += sEm[r * LDK + d];
            if (r < nvalid) dg[(row0 + (size_t)r * H) * DK + d] = acc;
        }
    } else {
        // row sums over the DK columns, 8 threads per row
        {
            const int r = tid >> 3, part0 = tid & 7;
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < DK / 8; ++j) s += sEm[r * LDK + part0 * (DK / 8) + j];
            s += __shfl_xor(s, 1, 64);
            s += __shfl_xor(s, 2, 64);
            s += __shfl_xor(s, 4, 64);
            if (part0 == 0) sRow[r] = s + sE[r];
        }
        if (tid == C) {
            float s = 0.f;
            for (int d = 0; d < DK; ++d) s += sDphi[d];
            sF[1] = s * sPhi[0];
        }
        lds_barrier();
        if (tid == 0) {
            float f0 = 0.f;
#pragma unroll
            for (int w = 0; w < 8; ++w) f0 += sFp[w];
            float acc = f0 + sF[1];
            for (int r = C - 1; r >= 0; --r) {
                acc += sRow[r];
                if (r < nvalid) dg[row0 + (size_t)r * H] = acc;
            }
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
