// prologue.h -- the input prologue as stand-alone elementwise kernels, for
// the backward through it (the forward fuses the prologue into its loads).
//
// Page: "Gated DeltaNet", sections "门控与 Head 映射" (beta = sigmoid(b),
// g = -exp(A_log) softplus(a + dt_bias)) and "加载 Token 与写入系数" (q, k divided
// by sqrt(sum of squares + 1e-6), q times the output scale), and the backward
// set of section "反向传播：状态伴随与三角变换梯度" (the gradients of the
// normalisation, the sigmoid and the gate generation, applied after the
// recurrence's own backward).
//
//   prologue_apply_kernel     raw q, k, g, beta -> the recurrence's inputs
//   prologue_backward_kernel  the recurrence's input gradients -> raw-input
//                             gradients (in place), dA_log and ddt_bias
//
// Chain rule per (token, head) row, y = x / n with n = sqrt(|x|^2 + 1e-6):
//   dq = scale (dq^ - y_q (y_q . dq^)) / n_q,   dk = (dk^ - y_k (y_k . dk^)) / n_k
//   db = s sigmoid(b) (1 - sigmoid(b)) dbeta^       (s = 2 with the doubling)
//   da = -exp(A_log) sigmoid(a + dt) dg^,  dA_log += g^ dg^,  ddt_bias += da
#pragma once

#include "common.h"

namespace dr {

constexpr int kProRows = 64;   // rows (tokens of one head) per workgroup

// One 256-thread workgroup per (head, block of kProRows rows of that head);
// each wave takes every fourth row.  A row's DK channels are spread over the
// 64 lanes (DK / 64 each).
template <typename T, int DK, bool PERCH>
__global__ __launch_bounds__(256) void prologue_apply_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                             const float* __restrict__ g,
                                                             const float* __restrict__ beta, T* __restrict__ qh,
                                                             T* __restrict__ kh, float* __restrict__ gh,
                                                             float* __restrict__ bh, long long rows_per_head, int H,
                                                             Prologue pro)
{
    constexpr int NPL = DK / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = blockIdx.x % H;
    const long long r0 = (long long)(blockIdx.x / H) * kProRows;
    const ProHead ph = pro_head(pro, h);
    for (int i = wave; i < kProRows; i += 4) {
        const long long tok = r0 + i;
        if (tok >= rows_per_head) break;
        const size_t row = (size_t)tok * H + h;
        float ql[NPL], kl[NPL];
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
            ql[j] = to_f(q[row * DK + lane + 64 * j]);
            kl[j] = to_f(k[row * DK + lane + 64 * j]);
            sq += ql[j] * ql[j];
            sk += kl[j] * kl[j];
        }
        float nq = ph.scale, nk = 1.f;
        if (ph.ops & PRO_QK_L2NORM) {
            sq = lane_group_sum<64>(sq);
            sk = lane_group_sum<64>(sk);
            nq *= inv_sqrt(sq + kNormEps);
            nk = inv_sqrt(sk + kNormEps);
        }
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
            qh[row * DK + lane + 64 * j] = from_f<T>(ql[j] * nq);
            kh[row * DK + lane + 64 * j] = from_f<T>(kl[j] * nk);
            if constexpr (PERCH) gh[row * DK + lane + 64 * j] = g[row * DK + lane + 64 * j];
        }
        if (lane == 0) {
            if constexpr (!PERCH) gh[row] = pro_gate(ph, g[row]);
            if (beta) bh[row] = pro_beta(ph, beta[row]);
        }
    }
}

// In place: dq, dk (DK per row, I/O dtype), dg (per-channel or one per row),
// dbeta (one per row) hold the gradients with respect to the recurrence's
// inputs and are overwritten with those with respect to the raw inputs.
// With gate generation, each workgroup (head h, row block j) writes its sums
// of the dA_log and ddt_bias terms to gpart[h * nblk + j] and
// gpart[(H + h) * nblk + j]; prologue_gate_sum_kernel adds them up.
template <typename T, int DK, bool PERCH>
__global__ __launch_bounds__(256) void prologue_backward_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                                const float* __restrict__ g,
                                                                const float* __restrict__ beta, T* __restrict__ dq,
                                                                T* __restrict__ dk, float* __restrict__ dg,
                                                                float* __restrict__ dbeta,
                                                                float* __restrict__ gpart, int nblk,
                                                                long long rows_per_head, int H, Prologue pro)
{
    constexpr int NPL = DK / 64;
    __shared__ float red[2][4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = blockIdx.x % H;
    const long long r0 = (long long)(blockIdx.x / H) * kProRows;
    const ProHead ph = pro_head(pro, h);
    const bool norm = ph.ops & PRO_QK_L2NORM;
    float accA = 0.f, accD = 0.f;
    for (int i = wave; i < kProRows; i += 4) {
        const long long tok = r0 + i;
        if (tok >= rows_per_head) break;
        const size_t row = (size_t)tok * H + h;
        float ql[NPL], kl[NPL], gq[NPL], gk[NPL];
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
            ql[j] = to_f(q[row * DK + lane + 64 * j]);
            kl[j] = to_f(k[row * DK + lane + 64 * j]);
            gq[j] = ph.scale * to_f(dq[row * DK + lane + 64 * j]);
            gk[j] = to_f(dk[row * DK + lane + 64 * j]);
            sq += ql[j] * ql[j];
            sk += kl[j] * kl[j];
        }
        if (norm) {
            sq = lane_group_sum<64>(sq);
            sk = lane_group_sum<64>(sk);
            const float iq = inv_sqrt(sq + kNormEps), ik = inv_sqrt(sk + kNormEps);
            float dotq = 0.f, dotk = 0.f;
#pragma unroll
            for (int j = 0; j < NPL; ++j) {
                dotq += ql[j] * iq * gq[j];
                dotk += kl[j] * ik * gk[j];
            }
            dotq = lane_group_sum<64>(dotq);
            dotk = lane_group_sum<64>(dotk);
#pragma unroll
            for (int j = 0; j < NPL; ++j) {
                gq[j] = (gq[j] - ql[j] * iq * dotq) * iq;
                gk[j] = (gk[j] - kl[j] * ik * dotk) * ik;
            }
        }
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
            dq[row * DK + lane + 64 * j] = from_f<T>(gq[j]);
            dk[row * DK + lane + 64 * j] = from_f<T>(gk[j]);
        }
        if (lane == 0) {
            if (beta && (ph.ops & PRO_BETA_SIGMOID)) {
                const float s = 1.f / (1.f + expf(-beta[row]));
                dbeta[row] = ((ph.ops & PRO_BETA_X2) ? 2.f : 1.f) * s * (1.f - s) * dbeta[row];
            }
            if constexpr (!PERCH) {
                if (ph.ops & PRO_GATE) {
                    const float a = g[row] + ph.gdt, dgh = dg[row];
                    const float da = -ph.gA / (1.f + expf(-a)) * dgh;
                    accA += -ph.gA * softplus_f(a) * dgh;   // g^ dg^
                    accD += da;
                    dg[row] = da;
                }
            }
        }
    }
    if constexpr (!PERCH) {
        if (ph.ops & PRO_GATE) {
            if (lane == 0) {
                red[0][wave] = accA;
                red[1][wave] = accD;
            }
            __syncthreads();
            if (threadIdx.x == 0) {
                const int j = (int)(blockIdx.x / H);
                gpart[(size_t)h * nblk + j] = red[0][0] + red[0][1] + red[0][2] + red[0][3];
                gpart[((size_t)H + h) * nblk + j] = red[1][0] + red[1][1] + red[1][2] + red[1][3];
            }
        }
    }
}

// dA_log[h] and ddt_bias[h] (when given) from the per-workgroup partials of
// prologue_backward_kernel, one workgroup per head, in a fixed order: each
// thread adds blocks tid, tid + 256, ... in turn, then the wave sums and
// the four wave totals in order.
__global__ __launch_bounds__(256) void prologue_gate_sum_kernel(const float* __restrict__ gpart, int nblk, int H,
                                                                float* __restrict__ dA_log,
                                                                float* __restrict__ ddt_bias)
{
    __shared__ float red[2][4];
    const int h = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const float* src = gpart + ((size_t)a * H + h) * nblk;
        float s = 0.f;
        for (int j = threadIdx.x; j < nblk; j += 256) s += src[j];
        s = lane_group_sum<64>(s);
        if (lane == 0) red[a][wave] = s;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        dA_log[h] = ((red[0][0] + red[0][1]) + red[0][2]) + red[0][3];
        if (ddt_bias) ddt_bias[h] = ((red[1][0] + red[1][1]) + red[1][2]) + red[1][3];
    }
}

}  // namespace dr
