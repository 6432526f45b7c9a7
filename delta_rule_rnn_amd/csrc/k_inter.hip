// k_inter.hip -- launchers of the state-pass kernel (inter.h): the forward
// and the backward's state-writing mode.
#include "host.h"
#include "inter.h"

namespace drh {

// DR_INTER_PFD=0 switches it off for comparison.
template <int KIND, typename E, int D, int NTN, int PFD>
dr_status launch_inter_p(const Problem& p, const float* h0, float* hT, int c0, int n, hipStream_t st) {
    constexpr int NV = D / (16 * NTN);
    dim3 grid(p.B * p.H * NV);
    if (p.seqinfo) {
        // packed sequences: p.B is the sequence count
        hipLaunchKernelGGL((dr::inter_kernel<KIND, E, D, D, NTN, PFD, true>), grid, dim3(dr::inter_threads<PFD>()),
                           0, st, p.ws, h0, static_cast<E*>(p.o), hT, p.T, p.H, p.NT, 0, 0, p.seqinfo,
                           p.maxchunks);
    } else {
        hipLaunchKernelGGL((dr::inter_kernel<KIND, E, D, D, NTN, PFD, false>), grid, dim3(dr::inter_threads<PFD>()),
                           0, st, p.ws, h0, static_cast<E*>(p.o), hT, p.T, p.H, p.NT, c0, n, nullptr, 0);
    }
    return check_launch();
}

// The ninth (prefetch) wave lowers the register budget of every wave to 168;
// the fp32 and 64-column variants need more, so they run without it.
template <int KIND, typename E, int D, int NTN>
dr_status launch_inter_n(const Problem& p, const float* h0, float* hT, int c0, int n, hipStream_t st) {
    if constexpr (sizeof(E) == 2 && NTN <= 2)
        if (pick_pfd() != 0) return launch_inter_p<KIND, E, D, NTN, 2>(p, h0, hT, c0, n, st);
    return launch_inter_p<KIND, E, D, NTN, 0>(p, h0, hT, c0, n, st);
}

template <int KIND, typename E, int D>
dr_status launch_inter_t(const Problem& p, const float* h0, float* hT, int c0, int n, hipStream_t st) {
    const int ntn = pick_ntn(p.B * p.H, D);
    if (ntn == 1) return launch_inter_n<KIND, E, D, 1>(p, h0, hT, c0, n, st);
    // fp32 operands at 64 columns do not fit in registers: at most 32 columns
    if (ntn == 2 || sizeof(E) == 4) return launch_inter_n<KIND, E, D, 2>(p, h0, hT, c0, n, st);
    if constexpr (sizeof(E) == 2) return launch_inter_n<KIND, E, D, 4>(p, h0, hT, c0, n, st);
    return DR_ERR_UNSUPPORTED;
}

// 128-token records: 8 recurrence + 8 output waves, no prefetch wave; at
// most 32 value columns per workgroup (the 1024-thread workgroup leaves 128
// registers per lane)
template <int KIND, typename E, int D, int NTN>
dr_status launch_inter128_n(const Problem& p, const float* h0, float* hT, int c0, int n, hipStream_t st) {
    constexpr int NV = D / (16 * NTN);
    dim3 grid(p.B * p.H * NV);
    hipLaunchKernelGGL((dr::inter_kernel<KIND, E, D, D, NTN, 0, false, false, kChunk128>), grid,
                       dim3(dr::inter_threads<0, kChunk128>()), 0, st, p.ws, h0, static_cast<E*>(p.o), hT, p.T,
                       p.H, p.NT, c0, n, nullptr, 0, nullptr, nullptr);
    return check_launch();
}
template <int KIND, typename E, int D>
dr_status launch_inter128_t(const Problem& p, const float* h0, float* hT, int c0, int n, hipStream_t st) {
    if (sizeof(E) == 4 || pick_ntn(p.B * p.H, D) == 1) return launch_inter128_n<KIND, E, D, 1>(p, h0, hT, c0, n, st);
    return launch_inter128_n<KIND, E, D, 2>(p, h0, hT, c0, n, st);
}

template <int KIND>
dr_status launch_inter_k(const Problem& p, const float* h0, float* hT, int c0, int n, hipStream_t st) {
    if (p.C == kChunk128) {
        if (p.dtype == DR_BF16)
            return p.D == 64 ? launch_inter128_t<KIND, bf16, 64>(p, h0, hT, c0, n, st)
                             : launch_inter128_t<KIND, bf16, 128>(p, h0, hT, c0, n, st);
        if (p.D == 64) return launch_inter128_t<KIND, float, 64>(p, h0, hT, c0, n, st);
        return DR_ERR_UNSUPPORTED;
    }
    if (p.dtype == DR_BF16) {
        if (p.D == 64) return launch_inter_t<KIND, bf16, 64>(p, h0, hT, c0, n, st);
        return launch_inter_t<KIND, bf16, 128>(p, h0, hT, c0, n, st);
    }
    if (p.D == 64) return launch_inter_t<KIND, float, 64>(p, h0, hT, c0, n, st);
    return launch_inter_t<KIND, float, 128>(p, h0, hT, c0, n, st);
}

dr_status launch_inter(const Problem& p, const float* h0, float* hT, int c0, int n, hipStream_t st) {
    switch (p.kind) {
        case DR_KIND_KDA: return launch_inter_k<dr::KIND_KDA>(p, h0, hT, c0, n, st);
        case DR_KIND_GDN: return launch_inter_k<dr::KIND_GDN>(p, h0, hT, c0, n, st);
        default: return launch_inter_k<dr::KIND_LA>(p, h0, hT, c0, n, st);
    }
}

// mode (entry state and Vnew of every chunk, no output) over the records the
// chunk-parallel kernel wrote; slice width and prefetch as for the forward
template <int KIND, typename E, int D, int NTN, int PFD>
dr_status launch_states_p(const Problem& p, const float* h0, E* hs, E* vn, hipStream_t st) {
    constexpr int NV = D / (16 * NTN);
    dim3 grid(p.B * p.H * NV);
    if (p.seqinfo) {
        hipLaunchKernelGGL((dr::inter_kernel<KIND, E, D, D, NTN, PFD, true, true>), grid,
                           dim3(dr::inter_threads<PFD>()), 0, st, p.ws, h0, static_cast<E*>(nullptr),
                           static_cast<float*>(nullptr), p.T, p.H, p.NT, 0, 0, p.seqinfo, p.maxchunks, hs, vn);
    } else {
        hipLaunchKernelGGL((dr::inter_kernel<KIND, E, D, D, NTN, PFD, false, true>), grid,
                           dim3(dr::inter_threads<PFD>()), 0, st, p.ws, h0, static_cast<E*>(nullptr),
                           static_cast<float*>(nullptr), p.T, p.H, p.NT, 0, p.NT, nullptr, 0, hs, vn);
    }
    return check_launch();
}
template <int KIND, typename E, int D>
dr_status launch_states_t(const Problem& p, const float* h0, void* hs_, void* vn_, hipStream_t st) {
    E* hs = static_cast<E*>(hs_);
    E* vn = static_cast<E*>(vn_);
    const int ntn = pick_ntn(p.B * p.H, D);
    const bool pf = pick_pfd() != 0;
    if constexpr (sizeof(E) == 2) {
        if (ntn == 1) return pf ? launch_states_p<KIND, E, D, 1, 2>(p, h0, hs, vn, st)
                                : launch_states_p<KIND, E, D, 1, 0>(p, h0, hs, vn, st);
        if (ntn == 2) return pf ? launch_states_p<KIND, E, D, 2, 2>(p, h0, hs, vn, st)
                                : launch_states_p<KIND, E, D, 2, 0>(p, h0, hs, vn, st);
        return launch_states_p<KIND, E, D, 4, 0>(p, h0, hs, vn, st);
    } else {
        // fp32 operands at 64 columns do not fit in registers: at most 32 columns
        if (ntn == 1) return launch_states_p<KIND, E, D, 1, 0>(p, h0, hs, vn, st);
        return launch_states_p<KIND, E, D, 2, 0>(p, h0, hs, vn, st);
    }
}
dr_status launch_states(const Problem& p, const float* h0, void* hs, void* vn, hipStream_t st) {
    auto by_kind = [&](auto kind_tag) -> dr_status {
        constexpr int KIND = decltype(kind_tag)::value;
        if (p.dtype == DR_BF16)
            return p.D == 64 ? launch_states_t<KIND, bf16, 64>(p, h0, hs, vn, st)
                             : launch_states_t<KIND, bf16, 128>(p, h0, hs, vn, st);
        return p.D == 64 ? launch_states_t<KIND, float, 64>(p, h0, hs, vn, st)
                         : launch_states_t<KIND, float, 128>(p, h0, hs, vn, st);
    };
    switch (p.kind) {
        case DR_KIND_KDA: return by_kind(std::integral_constant<int, dr::KIND_KDA>{});
        case DR_KIND_GDN: return by_kind(std::integral_constant<int, dr::KIND_GDN>{});
        default: return by_kind(std::integral_constant<int, dr::KIND_LA>{});
    }
}

}  // namespace drh
