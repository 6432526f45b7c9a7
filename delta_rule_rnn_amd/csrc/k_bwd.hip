// k_bwd.hip -- launchers of the backward kernels (backward.h, revseg.h).
#include "host.h"
#include "backward.h"
#include "revseg.h"

namespace drh {

size_t bwd_prep_floats(int D) { return D == 64 ? dr::bw::Prep<64>::FLOATS : dr::bw::Prep<128>::FLOATS; }
size_t bwd_rrec_elems(int D) { return D == 64 ? dr::bw::RevRec<64>::ELEMS : dr::bw::RevRec<128>::ELEMS; }

namespace {

// The segment-parallel reverse pass (bf16 I/O): segment maps (segments
// 1 .. NS-1), their composition, then every segment from its exit adjoint;
// with one segment per chain (packed sequences, or chains that fill the GPU)
// only the last, from dhT.
template <int KIND, int D>
dr_status launch_rev_seg(const BwdArgs& a, const bf16* rrec, const float* prep, bf16* dhs, bf16* dvn,
                         hipStream_t st) {
    using namespace dr::bw;
    const long long chains = (long long)a.B * a.H;    // B: sequences for packed sequences
    const int NS = a.pk.table ? 1 : a.L.NS, L = a.L.L;
    const bf16* dout = static_cast<const bf16*>(a.dout);
    float* xmap = reinterpret_cast<float*>(a.ws + a.L.xmap);
    float* ein = reinterpret_cast<float*>(a.ws + a.L.ein);
    if (chains * NS > 0x7fffffffLL || chains * (D / 16) > 0x7fffffffLL) return DR_ERR_UNSUPPORTED;
    dr_status s;
    const float* e = a.dhT;       // one segment: it starts from dhT
    if (NS > 1) {
        hipLaunchKernelGGL((rev_seg_kernel<KIND, D, true>), dim3((unsigned)(chains * (NS - 1))), dim3(kRevThreads), 0,
                           st, rrec, prep, dout, ein, xmap, dhs, dvn, a.dh0, a.T, a.H, a.NT, L, NS, a.pk);
        if ((s = check_launch()) != DR_OK) return s;
        hipLaunchKernelGGL((rev_compose_kernel<D>), dim3((unsigned)(chains * (D / 16))), dim3(kRevComposeThreads), 0,
                           st, xmap, a.dhT, ein, NS);
        if ((s = check_launch()) != DR_OK) return s;
        e = ein;
    }
    hipLaunchKernelGGL((rev_seg_kernel<KIND, D, false>), dim3((unsigned)(chains * NS)), dim3(kRevThreads), 0, st,
                       rrec, prep, dout, e, xmap, dhs, dvn, a.dh0, a.T, a.H, a.NT, L, NS, a.pk);
    return check_launch();
}

}  // namespace

template <int KIND, typename E, int D>
dr_status launch_backward_t(const BwdArgs& a, hipStream_t st) {
    using namespace dr::bw;
    float* prep = reinterpret_cast<float*>(a.ws + a.L.prep);
    E* hs = reinterpret_cast<E*>(a.ws + a.L.hs);
    E* dhs = reinterpret_cast<E*>(a.ws + a.L.dhs);
    E* vn = reinterpret_cast<E*>(a.ws + a.L.vn);
    E* dvn = reinterpret_cast<E*>(a.ws + a.L.dvn);
    const E* q = static_cast<const E*>(a.q);
    const E* k = static_cast<const E*>(a.k);
    const E* v = static_cast<const E*>(a.v);
    const E* dout = static_cast<const E*>(a.dout);
    const long long items = a.pk.table ? (long long)a.pk.maxchunks * a.H : (long long)a.B * a.NT * a.H;
    const long long slices = (long long)a.B * a.H * (D / kSV);
    if (items > 0x7fffffffLL || slices > 0x7fffffffLL) return DR_ERR_UNSUPPORTED;
    // the segment-parallel reverse pass where its workspace is laid out
    // (bf16 I/O) unless the value-slice kernel is selected
    const bool seg = std::is_same<E, bf16>::value && a.L.NS > 0 && rev_seg_selected();
    bf16* rrec = seg ? reinterpret_cast<bf16*>(a.ws + a.L.rrec) : nullptr;
    // the gradient kernel with bf16 LDS operands forms per-channel gamma from
    // g itself; only scalar gates' gradient kernels and the value-slice
    // reverse pass read Aqk
    const bool gb = std::is_same<E, bf16>::value && gradb_selected();
    const bool perch = KIND == dr::KIND_KDA;
    const unsigned wmask = ((perch && gb) ? 0u : PREP_W_GAM) | ((perch && gb && seg) ? 0u : PREP_W_AQK);
    dr_status s;
    if constexpr (std::is_same<E, bf16>::value) {
        // the bf16 prep (two workgroups per CU) writes what the segment-
        // parallel reverse pass and the bf16 gradient kernel read
        if (gb && seg) s = launch_prepb<KIND, D>(a, prep, rrec, a.fwd ? a.ws + a.L.rec : nullptr, st);
    }
    if (!(gb && seg)) {
        if (a.fwd) return DR_ERR_UNSUPPORTED;     // only the bf16 prep writes the records
        hipLaunchKernelGGL((bwd_prep_kernel<KIND, E, D>), dim3((unsigned)items), dim3(kPrepThreads), 0, st, q, k, a.g,
                           a.beta, prep, rrec, a.T, a.H, a.NT, a.pk, wmask);
        s = check_launch();
    }
    // the forward state pass on the prep's records (bf16 prep path)
    if (s == DR_OK && a.fwd) s = launch_states(*a.fwd, a.h0, hs, vn, st);
    if (s != DR_OK) return s;
    if constexpr (std::is_same<E, bf16>::value) {
        if (seg) s = launch_rev_seg<KIND, D>(a, rrec, prep, dhs, dvn, st);
    }
    if (!seg) {
        hipLaunchKernelGGL((bwd_state_rev_kernel<KIND, E, D>), dim3((unsigned)slices), dim3(kStateThreads), 0, st, prep,
                           dout, a.dhT, dhs, dvn, a.dh0, a.T, a.H, a.NT, a.pk);
        s = check_launch();
    }
    if (s != DR_OK) return s;
    if constexpr (std::is_same<E, bf16>::value) {
        if (gb) return launch_gradb<KIND, D>(a, prep, hs, dhs, vn, dvn, st);
    }
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
