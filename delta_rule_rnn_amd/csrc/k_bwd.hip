// k_bwd.hip -- launchers of the backward kernels (backward.h).
#include "host.h"
#include "backward.h"

namespace drh {

size_t bwd_prep_floats(int D) { return D == 64 ? dr::bw::Prep<64>::FLOATS : dr::bw::Prep<128>::FLOATS; }

template <int KIND, typename E, int D>
dr_status launch_backward_t(const BwdArgs& a, hipStream_t st) {
    using namespace dr::bw;
    float* prep = reinterpret_cast<float*>(a.ws + a.L.prep);
    float* hs = reinterpret_cast<float*>(a.ws + a.L.hs);
    float* dhs = reinterpret_cast<float*>(a.ws + a.L.dhs);
    float* vn = reinterpret_cast<float*>(a.ws + a.L.vn);
    float* dvn = reinterpret_cast<float*>(a.ws + a.L.dvn);
    const E* q = static_cast<const E*>(a.q);
    const E* k = static_cast<const E*>(a.k);
    const E* v = static_cast<const E*>(a.v);
    const E* dout = static_cast<const E*>(a.dout);
    const long long items = a.pk.table ? (long long)a.pk.maxchunks * a.H : (long long)a.B * a.NT * a.H;
    const long long slices = (long long)a.B * a.H * (D / kSV);
    if (items > 0x7fffffffLL || slices > 0x7fffffffLL) return DR_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((bwd_prep_kernel<KIND, E, D>), dim3((unsigned)items), dim3(kPrepThreads), 0, st, q, k, a.g, a.beta,
                       prep, a.T, a.H, a.NT, a.pk);
    dr_status s = check_launch();
    if (s != DR_OK) return s;
    hipLaunchKernelGGL((bwd_state_rev_kernel<KIND, E, D>), dim3((unsigned)slices), dim3(kStateThreads), 0, st, prep, dout, a.dhT,
                       dhs, dvn, a.dh0, a.T, a.H, a.NT, a.pk);
    if ((s = check_launch()) != DR_OK) return s;
    hipLaunchKernelGGL((bwd_grad_kernel<KIND, E, D>), dim3((unsigned)items), dim3(512), 0, st, q, k, v, a.beta, dout,
                       prep, hs, dhs, vn, dvn, static_cast<E*>(a.dq), static_cast<E*>(a.dk), static_cast<E*>(a.dv),
                       a.dg, a.dbeta, a.T, a.H, a.NT, a.pk);
    return check_launch();
}

// Workspace of the backward through the prologue: the recurrence's inputs

template <int KIND>
dr_status launch_backward_k(const BwdArgs& a, int D, int dtype, hipStream_t st) {
    if (dtype == DR_BF16) {
        if (D == 64) return launch_backward_t<KIND, bf16, 64>(a, st);
        return launch_backward_t<KIND, bf16, 128>(a, st);
    }
    if (D == 64) return launch_backward_t<KIND, float, 64>(a, st);
    return launch_backward_t<KIND, float, 128>(a, st);
}

// Backward for the dense layout (cu_seqlens == null, B batches) or packed
// sequences (cu_seqlens set, N sequences, B == 1), with or without a

dr_status launch_backward(int kind, const BwdArgs& a, int D, int dtype, hipStream_t st) {
    switch (kind) {
        case DR_KIND_KDA: return launch_backward_k<dr::KIND_KDA>(a, D, dtype, st);
        case DR_KIND_GDN: return launch_backward_k<dr::KIND_GDN>(a, D, dtype, st);
        default: return launch_backward_k<dr::KIND_LA>(a, D, dtype, st);
    }
}

}  // namespace drh
