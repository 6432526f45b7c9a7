// k_misc.hip -- launchers of the decode, prologue and step kernels, and the
// step entry points of the C ABI (dr_chunk_cumsum, dr_kda_prep).
#include "host.h"
#include "decode.h"
#include "steps.h"
#include "prologue.h"

namespace drh {

template <int KIND, typename E, int D, bool PRO>
dr_status launch_decode_t(const DecodeArgs& a, hipStream_t st) {
    dim3 grid((unsigned)((long long)a.B * a.H * (D / 64)));
    const bool nts = (size_t)a.B * a.H * D * D * sizeof(float) > kDecodeStreamBytes;
    if (nts)
        hipLaunchKernelGGL((dr::decode_kernel<KIND, E, D, D, PRO, true>), grid, dim3(64), 0, st,
                           static_cast<const E*>(a.q), static_cast<const E*>(a.k), static_cast<const E*>(a.v), a.g,
                           a.beta, a.state, static_cast<E*>(a.o), a.T, a.H, a.pro);
    else
        hipLaunchKernelGGL((dr::decode_kernel<KIND, E, D, D, PRO, false>), grid, dim3(64), 0, st,
                           static_cast<const E*>(a.q), static_cast<const E*>(a.k), static_cast<const E*>(a.v), a.g,
                           a.beta, a.state, static_cast<E*>(a.o), a.T, a.H, a.pro);
    return check_launch();
}

template <int KIND, bool PRO>
dr_status launch_decode_p(const DecodeArgs& a, int D, int dtype, hipStream_t st) {
    if (dtype == DR_BF16) {
        if (D == 64) return launch_decode_t<KIND, bf16, 64, PRO>(a, st);
        return launch_decode_t<KIND, bf16, 128, PRO>(a, st);
    }
    if (D == 64) return launch_decode_t<KIND, float, 64, PRO>(a, st);
    return launch_decode_t<KIND, float, 128, PRO>(a, st);
}

template <int KIND>
dr_status launch_decode_k(const DecodeArgs& a, bool use_pro, int D, int dtype, hipStream_t st) {
    return use_pro ? launch_decode_p<KIND, true>(a, D, dtype, st) : launch_decode_p<KIND, false>(a, D, dtype, st);
}

dr_status launch_decode(int kind, const DecodeArgs& a, bool use_pro, int D, int dtype, hipStream_t st) {
    switch (kind) {
        case DR_KIND_KDA: return launch_decode_k<dr::KIND_KDA>(a, use_pro, D, dtype, st);
        case DR_KIND_GDN: return launch_decode_k<dr::KIND_GDN>(a, use_pro, D, dtype, st);
        default: return launch_decode_k<dr::KIND_LA>(a, use_pro, D, dtype, st);
    }
}

template <typename E, int D, bool PERCH>
dr_status launch_prologue_t(bool backward, const void* q, const void* k, const float* g, const float* beta, void* qh,
                            void* kh, float* gh, float* bh, void* dq, void* dk, float* dg, float* dbeta,
                            float* dA_log, float* ddt, int B, int T, int H, const dr::Prologue& pro, hipStream_t st,
                            float* gpart) {
    const long long rows = (long long)B * T;
    const long long nblk = (rows + dr::kProRows - 1) / dr::kProRows;
    const long long blocks = (long long)H * nblk;
    if (blocks > 0x7fffffffLL) return DR_ERR_UNSUPPORTED;
    const bool gate = backward && !PERCH && (pro.ops & dr::PRO_GATE);
    if (gate && !gpart) return DR_ERR_INVALID_ARG;
    if (!backward)
        hipLaunchKernelGGL((dr::prologue_apply_kernel<E, D, PERCH>), dim3((unsigned)blocks), dim3(256), 0, st,
                           static_cast<const E*>(q), static_cast<const E*>(k), g, beta, static_cast<E*>(qh),
                           static_cast<E*>(kh), gh, bh, rows, H, pro);
    else
        hipLaunchKernelGGL((dr::prologue_backward_kernel<E, D, PERCH>), dim3((unsigned)blocks), dim3(256), 0, st,
                           static_cast<const E*>(q), static_cast<const E*>(k), g, beta, static_cast<E*>(dq),
                           static_cast<E*>(dk), dg, dbeta, gpart, (int)nblk, rows, H, pro);
    if (gate) {
        if (check_launch() != DR_OK) return DR_ERR_HIP;
        hipLaunchKernelGGL(dr::prologue_gate_sum_kernel, dim3((unsigned)H), dim3(256), 0, st, gpart, (int)nblk, H,
                           dA_log, ddt);
    }
    return check_launch();
}

dr_status launch_prologue(bool backward, int kind, int D, int dtype, const void* q, const void* k, const float* g,
                          const float* beta, void* qh, void* kh, float* gh, float* bh, void* dq, void* dk, float* dg,
                          float* dbeta, float* dA_log, float* ddt, int B, int T, int H, const dr::Prologue& pro,
                          hipStream_t st, float* gpart) {
#define DR_PRO(E, DD, PC) \
    return launch_prologue_t<E, DD, PC>(backward, q, k, g, beta, qh, kh, gh, bh, dq, dk, dg, dbeta, dA_log, ddt, B, T, H, \
                                        pro, st, gpart)
    const bool perch = kind == DR_KIND_KDA;
    if (dtype == DR_BF16) {
        if (D == 64) { if (perch) DR_PRO(bf16, 64, true); else DR_PRO(bf16, 64, false); }
        if (perch) DR_PRO(bf16, 128, true); else DR_PRO(bf16, 128, false);
    }
    if (D == 64) { if (perch) DR_PRO(float, 64, true); else DR_PRO(float, 64, false); }
    if (perch) DR_PRO(float, 128, true); else DR_PRO(float, 128, false);
#undef DR_PRO
}

dr_status launch_varlen_table(const int* cu_seqlens, int N, int T, int maxchunks, int4* table, int4* seqinfo,
                              int* total, unsigned* flags, hipStream_t st) {
    hipLaunchKernelGGL(dr::varlen_table_kernel, dim3(1), dim3(1024), 0, st, cu_seqlens, N, T, maxchunks, table,
                       seqinfo, total, flags);
    return check_launch();
}

dr_status poison_workspace(void* ws, size_t bytes, hipStream_t st) {
    const char* e = getenv("DR_POISON_WORKSPACE");
    if (!e || e[0] != '1' || !ws || bytes < 4) return DR_OK;
    const size_t n = bytes / 4;
    const size_t blocks = std::min<size_t>((n + 255) / 256, 65536);
    hipLaunchKernelGGL(dr::poison_kernel, dim3((unsigned)blocks), dim3(256), 0, st, static_cast<uint32_t*>(ws), n);
    return check_launch();
}

dr_status launch_copy_or_zero(float* dst, const float* src, size_t n, hipStream_t st) {
    if (n == 0) return DR_OK;
    hipLaunchKernelGGL(dr::copy_or_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, dst, src, n);
    return check_launch();
}

}  // namespace drh

using namespace drh;

extern "C" {

dr_status dr_chunk_cumsum(const float* g, float* gamma, int B, int T, int H, int D, int C, void* stream) {
    if (B <= 0 || H <= 0 || T < 0 || D < 1 || D > 256) return DR_ERR_INVALID_ARG;
    if (C != dr::kChunk) return DR_ERR_UNSUPPORTED;
    if (T > 0 && (!g || !gamma || g == gamma)) return DR_ERR_INVALID_ARG;
    if (!aligned16(g) || !aligned16(gamma)) return DR_ERR_INVALID_ARG;
    const int NT = ceil_div(T, C);
    if (NT == 0) return DR_OK;
    dim3 grid(NT, B * H);
    hipLaunchKernelGGL(dr::cumsum_kernel, grid, dim3(dr::kThreads), 0, static_cast<hipStream_t>(stream), g,
                       gamma, T, H, D);
    return check_launch();
}

dr_status dr_kda_prep(const void* q, const void* k, const float* gamma, void* qp, void* kp, void* km,
                      void* kbar, float* phi, int B, int T, int H, int Dk, int C, int dtype, unsigned* flags,
                      void* stream) {
    if (B <= 0 || H <= 0 || T < 0) return DR_ERR_INVALID_ARG;
    if (dtype != DR_F32 && dtype != DR_BF16) return DR_ERR_INVALID_ARG;
    if ((Dk != 64 && Dk != 128) || C != dr::kChunk) return DR_ERR_UNSUPPORTED;
    if (T > 0 && (!q || !k || !gamma)) return DR_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, gamma, qp, kp, km, kbar, phi};
    for (const void* p : ptrs)
        if (!aligned16(p)) return DR_ERR_INVALID_ARG;
    const int NT = ceil_div(T, C);
    const size_t items = (size_t)B * T * H * (Dk / 8);
    if (items == 0) return DR_OK;
    const unsigned blocks = (unsigned)((items + dr::kThreads - 1) / dr::kThreads);
    hipStream_t st = static_cast<hipStream_t>(stream);
#define DR_PREP(TT, DD)                                                                                  \
    hipLaunchKernelGGL((dr::prep_kernel<TT, DD>), dim3(blocks), dim3(dr::kThreads), 0, st,            \
                       static_cast<const TT*>(q), static_cast<const TT*>(k), gamma, static_cast<TT*>(qp), \
                       static_cast<TT*>(kp), static_cast<TT*>(km), static_cast<TT*>(kbar), phi, flags, B, T, \
                       H, NT)
    if (dtype == DR_BF16) {
        if (Dk == 64) DR_PREP(bf16, 64); else DR_PREP(bf16, 128);
    } else {
        if (Dk == 64) DR_PREP(float, 64); else DR_PREP(float, 128);
    }
#undef DR_PREP
    return check_launch();
}

}  // extern "C"
