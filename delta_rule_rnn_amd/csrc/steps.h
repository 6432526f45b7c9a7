// steps.h -- the first two steps as stand-alone kernels.  Both are
// bandwidth-bound elementwise/scan passes.
//
// Step a1, chunk-local log2 cumsum ("TileLang 实战：KDA 从零到一–Kimi Delta
// Attention" section 0; "07 · linear 路线（二）：衰减机制的演进" section 3.5):
//   gamma[cC + r] = log2(e) * sum_{s <= r} g[cC + s], restarting each chunk.
// Step a2, separable-exponent prep (same KDA page, section 1.2; "RNN的复兴04"
// section 5.3.4 for phi and Kbar):
//   kp = k 2^gamma, km = k 2^-gamma, qp = q 2^gamma,
//   kbar = k 2^(gamma_last - gamma), phi = 2^gamma_last.
#pragma once

#include "common.h"

namespace dr {

// One workgroup per (chunk, b*H + h).  D >= 2: thread d walks the chunk's
// positions for channel d (loads of consecutive channels are contiguous).
// D == 1: wave 0 scans the 64 positions with lane shuffles.
__global__ __launch_bounds__(kThreads) void cumsum_kernel(const float* __restrict__ g,
                                                          float* __restrict__ gamma, int Tlen, int H,
                                                          int D)
{
    constexpr int C = kChunk;
    const int c = blockIdx.x, bh = blockIdx.y;
    const int b = bh / H, h = bh % H;
    const int t0 = c * C;
    const int nvalid = min(C, Tlen - t0);
    const size_t row0 = ((size_t)b * Tlen + t0) * H + h;
    if (D == 1) {
        if (threadIdx.x < 64) {
            const int lane = threadIdx.x;
            float x = (lane < nvalid) ? g[row0 + (size_t)lane * H] : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off, 64);
                if (lane >= off) x += y;
            }
            if (lane < nvalid) gamma[row0 + (size_t)lane * H] = x * kLog2e;
        }
        return;
    }
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
        float s = 0.f;
        for (int p = 0; p < nvalid; ++p) {
            const size_t off = (row0 + (size_t)p * H) * D + d;
            s += g[off];
            gamma[off] = s * kLog2e;
        }
    }
}

// One thread per (token-head row, 8 channels).
template <typename T, int DK>
__global__ __launch_bounds__(kThreads) void prep_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const float* __restrict__ gamma,
    T* __restrict__ qp, T* __restrict__ kp, T* __restrict__ km, T* __restrict__ kbar,
    float* __restrict__ phi, unsigned* __restrict__ flags, int B, int Tlen, int H, int NT)
{
    constexpr int C = kChunk;
    constexpr int G8 = DK / 8;
    const size_t nitems = (size_t)B * Tlen * H * G8;
    const size_t it = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    bool f16 = false, f126 = false;
    if (it < nitems) {
        const int cg = (int)(it % G8);
        const size_t row = it / G8;                 // ((b*T + t)*H + h)
        const int h = (int)(row % H);
        const size_t bt = row / H;
        const int t = (int)(bt % Tlen);
        const int b = (int)(bt / Tlen);
        const int c = t / C;
        const int tl = min(Tlen, (c + 1) * C) - 1;  // last valid row of this chunk
        const size_t lrow = ((size_t)b * Tlen + tl) * H + h;
        const size_t off = row * DK + 8 * cg;
        const Frag<float> gm = ld_frag(gamma + off);
        const Frag<float> gl = ld_frag(gamma + lrow * DK + 8 * cg);
        Frag<T> fk = ld_frag(k + off), fq = ld_frag(q + off);
        Frag<T> okp, okm, oqp, okb;
        float mx = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float x = gm.v[j];
            const float e = __builtin_amdgcn_exp2f(x), ei = __builtin_amdgcn_exp2f(-x);
            const float kk = frag_get(fk, j), qq = frag_get(fq, j);
            mx = fmaxf(mx, -x);
            frag_set(okp, j, kk * e);
            frag_set(okm, j, kk * ei);
            frag_set(oqp, j, qq * e);
            frag_set(okb, j, kk * __builtin_amdgcn_exp2f(gl.v[j] - x));
        }
        if (kp) st_frag(kp + off, okp);
        if (km) st_frag(km + off, okm);
        if (qp) st_frag(qp + off, oqp);
        if (kbar) st_frag(kbar + off, okb);
        if (phi && t == c * C) {
            float* dst = phi + (((size_t)b * NT + c) * H + h) * DK + 8 * cg;
#pragma unroll
            for (int j = 0; j < 8; ++j) dst[j] = __builtin_amdgcn_exp2f(gl.v[j]);
        }
        f16 = mx >= 16.f;
        f126 = mx >= 126.f;
    }
    if (flags) {
        const unsigned long long b16 = __ballot(f16), b126 = __ballot(f126);
        if ((threadIdx.x & 63) == 0 && (b16 | b126)) atomicOr(flags, (b16 ? 1u : 0u) | (b126 ? 2u : 0u));
    }
}

// Packed sequences: from cu_seqlens (N+1 token offsets) build, in one
// workgroup, the table of chunks (slot -> {sequence, first token, valid rows})
// and per-sequence descriptors {first slot, chunks, first token, tokens}, the
// slot count in *total.  Offsets are clamped into [0, T] and kept
// non-decreasing, and slots beyond maxchunks are dropped, so every kernel
// stays in bounds whatever cu_seqlens holds; malformed offsets raise
// flag 0x4 (DR_FLAG_BAD_SEQLENS).
__global__ __launch_bounds__(1024) void varlen_table_kernel(const int* __restrict__ cu, int N, int T,
                                                            int maxchunks, int4* __restrict__ table,
                                                            int4* __restrict__ seqinfo, int* __restrict__ total,
                                                            unsigned* __restrict__ flags)
{
    __shared__ int wsum[16];
    __shared__ int carry_s;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    if (tid == 0) carry_s = 0;
    __syncthreads();
    bool bad = false;
    for (int base = 0; base < N; base += 1024) {
        const int i = base + tid;
        int s = 0, len = 0, nch = 0;
        if (i < N) {
            const int a = cu[i], e = cu[i + 1];
            s = min(max(a, 0), T);
            len = min(max(e, s), T) - s;
            nch = (len + kChunk - 1) / kChunk;
            bad = bad || a < 0 || e < a || e > T || (i == 0 && a != 0) || (i == N - 1 && e != T);
        }
        // inclusive scan of the chunk counts over the workgroup
        int x = nch;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        if (lane == 63) wsum[wid] = x;
        __syncthreads();
        int wpre = 0, btot = 0;
        for (int w = 0; w < 16; ++w) {
            if (w < wid) wpre += wsum[w];
            btot += wsum[w];
        }
        const int carry = carry_s;
        if (i < N) {
            const int first = carry + wpre + x - nch;
            const int off = min(first, maxchunks);
            const int nc = min(first + nch, maxchunks) - off;
            seqinfo[i] = make_int4(off, nc, s, len);
            for (int j = 0; j < nc; ++j)
                table[off + j] = make_int4(i, s + j * kChunk, min(kChunk, len - j * kChunk), 0);
        }
        __syncthreads();
        if (tid == 0) carry_s = carry + btot;
        __syncthreads();
    }
    if (tid == 0) *total = min(carry_s, maxchunks);
    if (flags && bad) atomicOr(flags, 4u);
}

// dst[i] = src ? src[i] : 0 for i < n (a fill that graph capture records as
// a kernel node).
// Debug fill: every 32-bit word of [p, p + 4 * n) set to all ones (a NaN
// as fp32, and two NaNs as bf16), grid-stride.
__global__ __launch_bounds__(256) void poison_kernel(uint32_t* __restrict__ p, size_t n)
{
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0xFFFFFFFFu;
}

__global__ __launch_bounds__(256) void copy_or_zero_kernel(float* __restrict__ dst, const float* __restrict__ src,
                                                           size_t n)
{
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

}  // namespace dr
