// k_seg.hip -- launchers of the segment-parallel forward (seg.h): the local
// segment pass, the entry-state composition and the output correction.
#include "host.h"
#include "seg.h"

namespace drh {

namespace {

template <int KIND, typename E, int D, bool PRO>
dr_status launch_seg_local_t(const Problem& p, const SegLayout& S, const float* h0, hipStream_t st) {
    const long long groups = (long long)p.B * p.H * S.NS;
    // the kernel addresses one chunk of o (C rows of H*D elements) with 32-bit offsets
    if (groups > 0x7fffffffLL || (long long)dr::kChunk * p.H * D * (long long)sizeof(E) > 0x7fffffffLL)
        return DR_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((dr::seg_kernel<KIND, E, D, D, PRO>), dim3((unsigned)groups), dim3(dr::kSegThreads), 0, st,
                       static_cast<const E*>(p.q), static_cast<const E*>(p.k), static_cast<const E*>(p.v), p.g,
                       p.beta, h0, static_cast<E*>(p.o), reinterpret_cast<E*>(p.ws + S.qeff),
                       reinterpret_cast<float*>(p.ws + S.xend), p.flags, p.T, p.H, p.NT, S.L, S.NS, p.pro);
    return check_launch();
}

template <int KIND, bool PRO>
dr_status launch_seg_local_p(const Problem& p, const SegLayout& S, const float* h0, hipStream_t st) {
    if (p.dtype == DR_BF16) {
        if (p.D == 64) return launch_seg_local_t<KIND, bf16, 64, PRO>(p, S, h0, st);
        return launch_seg_local_t<KIND, bf16, 128, PRO>(p, S, h0, st);
    }
    if (p.D == 64) return launch_seg_local_t<KIND, float, 64, PRO>(p, S, h0, st);
    return DR_ERR_UNSUPPORTED;
}

template <int KIND>
dr_status launch_seg_local_k(const Problem& p, const SegLayout& S, const float* h0, hipStream_t st) {
    return p.use_pro ? launch_seg_local_p<KIND, true>(p, S, h0, st) : launch_seg_local_p<KIND, false>(p, S, h0, st);
}

template <typename E, int D>
dr_status launch_compose_t(const Problem& p, const SegLayout& S, float* hT, hipStream_t st) {
    const long long groups = (long long)p.B * p.H * (D / 16);
    if (groups > 0x7fffffffLL) return DR_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((dr::compose_kernel<E, D, D>), dim3((unsigned)groups), dim3(dr::kComposeThreads), 0, st,
                       reinterpret_cast<const float*>(p.ws + S.xend), reinterpret_cast<E*>(p.ws + S.sint), hT, S.NS);
    return check_launch();
}

template <typename E, int D>
dr_status launch_correct_t(const Problem& p, const SegLayout& S, hipStream_t st) {
    const long long groups = (S.L + dr::kCorrChunks - 1) / dr::kCorrChunks;
    const long long items = (long long)p.B * p.H * (S.NS - 1) * groups;
    if (items <= 0) return DR_OK;
    if (items > 0x7fffffffLL) return DR_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((dr::correct_kernel<E, D, D>), dim3((unsigned)items), dim3(dr::kThreads), 0, st,
                       reinterpret_cast<const E*>(p.ws + S.qeff), reinterpret_cast<const E*>(p.ws + S.sint),
                       static_cast<E*>(p.o), p.T, p.H, p.NT, S.L, S.NS);
    return check_launch();
}

}  // namespace

dr_status launch_seg_local(const Problem& p, const SegLayout& S, const float* h0, hipStream_t st) {
    switch (p.kind) {
        case DR_KIND_KDA: return launch_seg_local_k<dr::KIND_KDA>(p, S, h0, st);
        case DR_KIND_GDN: return launch_seg_local_k<dr::KIND_GDN>(p, S, h0, st);
        default: return launch_seg_local_k<dr::KIND_LA>(p, S, h0, st);
    }
}

dr_status launch_seg_compose(const Problem& p, const SegLayout& S, float* hT, hipStream_t st) {
    if (S.NS <= 1 && hT == nullptr) return DR_OK;
    if (p.dtype == DR_BF16)
        return p.D == 64 ? launch_compose_t<bf16, 64>(p, S, hT, st) : launch_compose_t<bf16, 128>(p, S, hT, st);
    return p.D == 64 ? launch_compose_t<float, 64>(p, S, hT, st) : DR_ERR_UNSUPPORTED;
}

dr_status launch_seg_correct(const Problem& p, const SegLayout& S, hipStream_t st) {
    if (S.NS <= 1) return DR_OK;
    if (p.dtype == DR_BF16)
        return p.D == 64 ? launch_correct_t<bf16, 64>(p, S, st) : launch_correct_t<bf16, 128>(p, S, st);
    return p.D == 64 ? launch_correct_t<float, 64>(p, S, st) : DR_ERR_UNSUPPORTED;
}

}  // namespace drh
