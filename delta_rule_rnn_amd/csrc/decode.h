// decode.h -- recurrent step for decoding: T new tokens per (batch, head),
// applied token by token to a state kept in HBM between calls.
//
// Page keys: [KDA] "TileLang 实战：KDA 从零到一–Kimi Delta Attention";
// [GDN] "Gated DeltaNet" (section "Recurrent 算法代码解析": the state split
// into value-column blocks over a parallel grid); [SD] "TileLang 实战：KDA
// 从零到一--标量衰减".
//
// Per token, with S the [Dk, Dv] state (transpose of the pages' S):
//   S <- Diag(a) S                         a = exp(g) per key channel (KDA) or
//                                          one scalar per token and head
//   delta kinds:  r = beta (v - S^T k),  S <- S + k r^T
//   decay_la:     S <- S + k v^T
//   o = S^T q                              (after the update, [KDA] 3.1;
//                                          evaluated as q.S_decayed + r q.k)
//
// Value columns evolve independently ([KDA] 3.4), so lane j of a wave owns
// state column dv0 + j: its Dk values stay in registers for all T tokens, the
// dot products over the key channels need no cross-lane reduction, and the
// state is read and written once per call with 256-byte row segments.  The
// token's k, q and gate are staged in LDS and read as broadcasts.  All
// arithmetic is fp32.  With PRO, the input prologue (common.h) is applied to
// each token's q, k, gate and beta as they are loaded.
#pragma once

#include "common.h"

namespace dr {

// At least two waves per SIMD (at most 256 VGPRs): the state column takes Dk
// registers and the compiler would otherwise also keep the staged key there.
// NTS: write the state back with non-temporal stores.  The host selects it
// when the state of the call is larger than half the last-level cache: the
// state is then not re-read from cache by the next call anyway, and the
// streaming stores keep it from evicting other data (measured +18% at 256
// sequences x 32 heads, d = 128).  Smaller states stay cache-resident between
// calls with ordinary stores.
template <int KIND, typename T, int DK, int DV, bool PRO, bool NTS>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void decode_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                    const T* __restrict__ v, const float* __restrict__ g,
                                                    const float* __restrict__ beta, float* __restrict__ state,
                                                    T* __restrict__ o, int Tlen, int H, Prologue pro)
{
    constexpr int NS = DV / 64;                 // workgroups per (b, h)
    constexpr bool DELTA = KIND != KIND_LA;
    constexpr bool PERCH = KIND == KIND_KDA;
    static_assert(DV % 64 == 0 && DK % 64 == 0, "decode layout");

    __shared__ __attribute__((aligned(16))) float sk[DK];
    __shared__ __attribute__((aligned(16))) float sq[DK];
    __shared__ __attribute__((aligned(16))) float sa[PERCH ? DK : 4];

    const int lane = threadIdx.x;
    const int chain = blockIdx.x / NS, slice = blockIdx.x % NS;
    const int b = chain / H, h = chain % H;
    const int col = slice * 64 + lane;
    float* st = state + (size_t)chain * DK * DV + col;
    ProHead ph{};
    if constexpr (PRO) ph = pro_head(pro, h);

    float S[DK];
#pragma unroll
    for (int d = 0; d < DK; ++d) S[d] = st[(size_t)d * DV];

    for (int t = 0; t < Tlen; ++t) {
        const size_t row = ((size_t)b * Tlen + t) * H + h;
        constexpr int NPL = DK / 64;     // channels per lane
        float kl[NPL], ql[NPL];
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
            kl[j] = to_f(k[row * DK + lane + 64 * j]);
            ql[j] = to_f(q[row * DK + lane + 64 * j]);
        }
        if constexpr (PRO) {
            // L2 normalisation over the DK channels (a butterfly over the
            // wave), then the query scale
            float nk = 1.f, nq = ph.scale;
            if (ph.ops & PRO_QK_L2NORM) {
                float sk2 = 0.f, sq2 = 0.f;
#pragma unroll
                for (int j = 0; j < NPL; ++j) {
                    sk2 += kl[j] * kl[j];
                    sq2 += ql[j] * ql[j];
                }
                sk2 = lane_group_sum<64>(sk2);
                sq2 = lane_group_sum<64>(sq2);
                nk = inv_sqrt(sk2 + kNormEps);
                nq *= inv_sqrt(sq2 + kNormEps);
            }
#pragma unroll
            for (int j = 0; j < NPL; ++j) {
                kl[j] *= nk;
                ql[j] *= nq;
            }
        }
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
            const int d = lane + 64 * j;
            sk[d] = kl[j];
            sq[d] = ql[j];
            if constexpr (PERCH) sa[d] = __builtin_amdgcn_exp2f(g[row * DK + d] * kLog2e);
        }
        const float a = PERCH ? 1.f : __builtin_amdgcn_exp2f((PRO ? pro_gate(ph, g[row]) : g[row]) * kLog2e);
        const float bt = DELTA ? (PRO ? pro_beta(ph, beta[row]) : beta[row]) : 0.f;
        const float vv = to_f(v[row * DV + col]);
        lds_barrier();

        // decay first, then the read-outs of the decayed state:
        //   kS = k . S,  qS = q . S,  qk = q . k
        // so that o = q . (S + k r) = qS + r qk needs no second pass over q
        // (groups of 16 channels with a compiler barrier between them, so the
        // broadcast LDS reads are not all hoisted into registers at once)
        float kS = 0.f, qS = 0.f, qk = 0.f;
#pragma unroll
        for (int d0 = 0; d0 < DK; d0 += 16) {
#pragma unroll
            for (int d = d0; d < d0 + 16; ++d) {
                S[d] *= PERCH ? sa[d] : a;
                kS += sk[d] * S[d];
                qS += sq[d] * S[d];
                qk += sq[d] * sk[d];
            }
            asm volatile("" ::: "memory");
        }
        const float r = DELTA ? bt * (vv - kS) : vv;
        const float oo = qS + r * qk;
#pragma unroll
        for (int d0 = 0; d0 < DK; d0 += 16) {
#pragma unroll
            for (int d = d0; d < d0 + 16; ++d) S[d] += sk[d] * r;
            asm volatile("" ::: "memory");
        }
        o[row * DV + col] = from_f<T>(oo);
        lds_barrier();   // the next token overwrites sk, sq, sa
    }

    // the row addresses of the store are formed here, not kept alive across
    // the token loop (the pointer passes through an empty asm)
    float* st_out = st;
    asm volatile("" : "+v"(st_out));
#pragma unroll
    for (int d = 0; d < DK; ++d) {
        if constexpr (NTS) __builtin_nontemporal_store(S[d], st_out + (size_t)d * DV);
        else st_out[(size_t)d * DV] = S[d];
    }
}

}  // namespace dr
