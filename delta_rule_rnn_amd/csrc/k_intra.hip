// k_intra.hip -- launchers of the chunk-parallel kernel (intra.h), dense and
// packed.
#include "host.h"
#include "intra.h"

namespace drh {

// ---- chunk-parallel kernel over chunks [c0, c0 + n) -----------------------
template <int KIND, typename E, int D, bool PRO>
dr_status launch_intra_t(const Problem& p, int c0, int n, hipStream_t st) {
    const long long items = (long long)p.B * n * p.H;
    if (items > 0x7fffffffLL) return DR_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((dr::intra_kernel<KIND, E, D, D, PRO>), dim3((unsigned)items), dim3(dr::kThreads), 0, st,
                       static_cast<const E*>(p.q), static_cast<const E*>(p.k), static_cast<const E*>(p.v),
                       p.g, p.beta, p.ws, p.flags, p.T, p.H, p.NT, c0, n, p.B, p.pro);
    return check_launch();
}

// 128-token chunks: one 512-thread workgroup per chunk (two sub-chunks)
template <int KIND, typename E, int D, bool PRO>
dr_status launch_intra128_t(const Problem& p, int c0, int n, hipStream_t st) {
    const long long items = (long long)p.B * n * p.H;
    if (items > 0x7fffffffLL) return DR_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((dr::intra128_kernel<KIND, E, D, D, PRO>), dim3((unsigned)items), dim3(2 * dr::kThreads), 0,
                       st, static_cast<const E*>(p.q), static_cast<const E*>(p.k), static_cast<const E*>(p.v),
                       p.g, p.beta, p.ws, p.flags, p.T, p.H, p.NT, c0, n, p.B, p.pro);
    return check_launch();
}

template <int KIND, bool PRO>
dr_status launch_intra_p(const Problem& p, int c0, int n, hipStream_t st) {
    if (p.C == kChunk128) {
        if (p.dtype == DR_BF16)
            return p.D == 64 ? launch_intra128_t<KIND, bf16, 64, PRO>(p, c0, n, st)
                             : launch_intra128_t<KIND, bf16, 128, PRO>(p, c0, n, st);
        if (p.D == 64) return launch_intra128_t<KIND, float, 64, PRO>(p, c0, n, st);
        return DR_ERR_UNSUPPORTED;
    }
    if (p.dtype == DR_BF16) {
        if (p.D == 64) return launch_intra_t<KIND, bf16, 64, PRO>(p, c0, n, st);
        return launch_intra_t<KIND, bf16, 128, PRO>(p, c0, n, st);
    }
    if (p.D == 64) return launch_intra_t<KIND, float, 64, PRO>(p, c0, n, st);
    return launch_intra_t<KIND, float, 128, PRO>(p, c0, n, st);
}

template <int KIND>
dr_status launch_intra_k(const Problem& p, int c0, int n, hipStream_t st) {
    return p.use_pro ? launch_intra_p<KIND, true>(p, c0, n, st) : launch_intra_p<KIND, false>(p, c0, n, st);
}

dr_status launch_intra(const Problem& p, int c0, int n, hipStream_t st) {
    if (n <= 0) return DR_OK;
    switch (p.kind) {
        case DR_KIND_KDA: return launch_intra_k<dr::KIND_KDA>(p, c0, n, st);
        case DR_KIND_GDN: return launch_intra_k<dr::KIND_GDN>(p, c0, n, st);
        default: return launch_intra_k<dr::KIND_LA>(p, c0, n, st);
    }
}

// ---- state pass + output over chunks [c0, c0 + n) ------------------------
// L2 prefetch distance of the state pass in chunks (0 = no prefetch wave);

template <int KIND, typename E, int D, bool PRO>
dr_status launch_intra_varlen_t(const Problem& p, hipStream_t st) {
    const long long items = (long long)p.maxchunks * p.H;
    if (items > 0x7fffffffLL) return DR_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((dr::intra_varlen_kernel<KIND, E, D, D, PRO>), dim3((unsigned)items), dim3(dr::kThreads), 0,
                       st, static_cast<const E*>(p.q), static_cast<const E*>(p.k), static_cast<const E*>(p.v), p.g,
                       p.beta, p.ws, p.flags, p.table, p.total, p.H, p.maxchunks, p.pro);
    return check_launch();
}
template <int KIND, bool PRO>
dr_status launch_intra_varlen_p(const Problem& p, hipStream_t st) {
    if (p.dtype == DR_BF16) {
        if (p.D == 64) return launch_intra_varlen_t<KIND, bf16, 64, PRO>(p, st);
        return launch_intra_varlen_t<KIND, bf16, 128, PRO>(p, st);
    }
    if (p.D == 64) return launch_intra_varlen_t<KIND, float, 64, PRO>(p, st);
    return launch_intra_varlen_t<KIND, float, 128, PRO>(p, st);
}
template <int KIND>
dr_status launch_intra_varlen_k(const Problem& p, hipStream_t st) {
    return p.use_pro ? launch_intra_varlen_p<KIND, true>(p, st) : launch_intra_varlen_p<KIND, false>(p, st);
}

dr_status launch_intra_varlen(const Problem& p, hipStream_t st) {
    switch (p.kind) {
        case DR_KIND_KDA: return launch_intra_varlen_k<dr::KIND_KDA>(p, st);
        case DR_KIND_GDN: return launch_intra_varlen_k<dr::KIND_GDN>(p, st);
        default: return launch_intra_varlen_k<dr::KIND_LA>(p, st);
    }
}

}  // namespace drh
