// k_gradb.hip -- launchers of the bf16 backward kernels: the prep (prepb.h)
// and the gradient kernel (gradb.h).
#include "host.h"
#include "gradb.h"
#include "prepb.h"

namespace drh {

template <int KIND, int D>
dr_status launch_gradb(const BwdArgs& a, const float* prep, const bf16* hs, const bf16* dhs, const bf16* vn,
                       const bf16* dvn, hipStream_t st) {
    using namespace dr::bw;
    const long long items = a.pk.table ? (long long)a.pk.maxchunks * a.H : (long long)a.B * a.NT * a.H;
    if (items > 0x7fffffffLL) return DR_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((bwd_gradb_kernel<KIND, D>), dim3((unsigned)items), dim3(kGradbThreads), 0, st,
                       static_cast<const bf16*>(a.q), static_cast<const bf16*>(a.k), static_cast<const bf16*>(a.v),
                       a.g, a.beta, static_cast<const bf16*>(a.dout), prep, hs, dhs, vn, dvn, static_cast<bf16*>(a.dq),
                       static_cast<bf16*>(a.dk), static_cast<bf16*>(a.dv), a.dg, a.dbeta, a.T, a.H, a.NT, a.pk);
    return check_launch();
}

template <int KIND, int D>
dr_status launch_prepb(const BwdArgs& a, float* prep, bf16* rrec, uint8_t* recs, hipStream_t st) {
    using namespace dr::bw;
    const long long items = a.pk.table ? (long long)a.pk.maxchunks * a.H : (long long)a.B * a.NT * a.H;
    if (items > 0x7fffffffLL) return DR_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((bwd_prepb_kernel<KIND, D>), dim3((unsigned)items), dim3(kPrepbThreads), 0, st,
                       static_cast<const bf16*>(a.q), static_cast<const bf16*>(a.k), static_cast<const bf16*>(a.v),
                       a.g, a.beta, prep, rrec, recs, a.T, a.H, a.NT, a.pk);
    return check_launch();
}

#define DR_GRADB(KIND, D)                                                                                         \
    template dr_status launch_gradb<KIND, D>(const BwdArgs&, const float*, const bf16*, const bf16*, const bf16*, \
                                            const bf16*, hipStream_t);                                     \
    template dr_status launch_prepb<KIND, D>(const BwdArgs&, float*, bf16*, uint8_t*, hipStream_t);
DR_GRADB(dr::KIND_KDA, 64)
DR_GRADB(dr::KIND_KDA, 128)
DR_GRADB(dr::KIND_GDN, 64)
DR_GRADB(dr::KIND_GDN, 128)
DR_GRADB(dr::KIND_LA, 64)
DR_GRADB(dr::KIND_LA, 128)
#undef DR_GRADB

}  // namespace drh
