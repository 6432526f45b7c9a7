// deltarule.hip -- host side of the C ABI declared in include/deltarule.h:
// argument validation, workspace sizing and kernel dispatch for gfx950.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "../../include/deltarule.h"
#include "common.h"
#include "inter.h"
#include "intra.h"
#include "steps.h"

namespace {

using dr::bf16;

bool aligned16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

dr_status check_launch() {
    return hipGetLastError() == hipSuccess ? DR_OK : DR_ERR_HIP;
}

int ceil_div(int a, int b) { return (a + b - 1) / b; }

size_t record_bytes(int D, int dtype) {
    if (dtype == DR_BF16) return D == 64 ? dr::Rec<bf16, 64, 64>::BYTES : dr::Rec<bf16, 128, 128>::BYTES;
    return D == 64 ? dr::Rec<float, 64, 64>::BYTES : dr::Rec<float, 128, 128>::BYTES;
}

// Shared validation for the full forward and the fused step entry points.
dr_status validate(int kind, const void* q, const void* k, const void* v, const float* g,
                   const float* beta, int B, int T, int H, int Dk, int Dv, int C, int dtype) {
    if (kind < 0 || kind > 2) return DR_ERR_INVALID_ARG;
    if (B <= 0 || H <= 0 || T < 0) return DR_ERR_INVALID_ARG;
    if (dtype != DR_F32 && dtype != DR_BF16) return DR_ERR_INVALID_ARG;
    if (Dk <= 0 || Dv <= 0 || C <= 0) return DR_ERR_INVALID_ARG;
    if (Dk != Dv || (Dk != 64 && Dk != 128) || C != dr::kChunk) return DR_ERR_UNSUPPORTED;
    if ((long long)B * T * H * Dk > (1LL << 40)) return DR_ERR_INVALID_ARG;
    if (T > 0 && (!q || !k || !v || !g)) return DR_ERR_INVALID_ARG;
    if (T > 0 && kind != DR_KIND_DECAY_LA && !beta) return DR_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(beta))
        return DR_ERR_INVALID_ARG;
    return DR_OK;
}

template <int KIND, typename E, int D>
dr_status launch_intra(const void* q, const void* k, const void* v, const float* g, const float* beta,
                       int B, int T, int H, void* ws, unsigned* flags, hipStream_t st) {
    const int NT = ceil_div(T, dr::kChunk);
    if (NT == 0) return DR_OK;
    dim3 grid(NT, H, B);
    hipLaunchKernelGGL((dr::intra_kernel<KIND, E, D, D>), grid, dim3(dr::kThreads), 0, st,
                       static_cast<const E*>(q), static_cast<const E*>(k), static_cast<const E*>(v), g,
                       beta, static_cast<uint8_t*>(ws), flags, T, H, NT);
    return check_launch();
}

// Value columns per state-pass workgroup (16 * ntn).  Fewer columns per
// workgroup means more workgroups: with few (b, h) chains the narrow split
// fills the 256 CUs; with many chains wider slices cut the repeated reads of
// the shared W / Q~ / Kbar / Aqk operands.  DR_INTER_NTN (1, 2 or 4)
// overrides the choice for tuning.
int pick_ntn(int chains, int D) {
    if (const char* e = getenv("DR_INTER_NTN")) {
        const int v = atoi(e);
        if ((v == 1 || v == 2 || v == 4) && 16 * v <= D) return v;
    }
    const int cols = D / 16;                         // 16-column slices per chain
    if (chains * cols <= 512) return 1;              // <= 512 workgroups: narrowest
    if (chains * cols / 2 <= 512 || D == 64) return 2;
    return 4;
}

int pick_nbuf() {
    if (const char* e = getenv("DR_INTER_NBUF")) {
        const int v = atoi(e);
        if (v == 2 || v == 3) return v;
    }
    return 2;
}

template <int KIND, typename E, int D, int NTN, int NBUF>
dr_status launch_inter_n(const float* h0, void* o, float* hT, int B, int T, int H, const void* ws,
                         hipStream_t st) {
    const int NT = ceil_div(T, dr::kChunk);
    constexpr int NV = D / (16 * NTN);
    dim3 grid(B * H * NV);
    hipLaunchKernelGGL((dr::inter_kernel<KIND, E, D, D, NTN, NBUF>), grid, dim3(dr::kThreads), 0, st,
                       static_cast<const uint8_t*>(ws), h0, static_cast<E*>(o), hT, T, H, NT);
    return check_launch();
}

template <int KIND, typename E, int D>
dr_status launch_inter(const float* h0, void* o, float* hT, int B, int T, int H, const void* ws,
                       hipStream_t st) {
    const int ntn = pick_ntn(B * H, D);
    // fp32 operands are twice as large: one chunk of prefetch only
    const int nbuf = sizeof(E) == 4 ? 2 : pick_nbuf();
    if constexpr (sizeof(E) == 2) {
        if (nbuf == 3) {
            if (ntn == 1) return launch_inter_n<KIND, E, D, 1, 3>(h0, o, hT, B, T, H, ws, st);
            if (ntn == 2) return launch_inter_n<KIND, E, D, 2, 3>(h0, o, hT, B, T, H, ws, st);
            // 64 columns with three buffers does not fit in registers: two buffers
        }
    }
    if (ntn == 1) return launch_inter_n<KIND, E, D, 1, 2>(h0, o, hT, B, T, H, ws, st);
    if (ntn == 2) return launch_inter_n<KIND, E, D, 2, 2>(h0, o, hT, B, T, H, ws, st);
    return launch_inter_n<KIND, E, D, 4, 2>(h0, o, hT, B, T, H, ws, st);
}

template <int KIND>
dr_status dispatch_intra(int dtype, int D, const void* q, const void* k, const void* v, const float* g,
                         const float* beta, int B, int T, int H, void* ws, unsigned* flags,
                         hipStream_t st) {
    if (dtype == DR_BF16) {
        if (D == 64) return launch_intra<KIND, bf16, 64>(q, k, v, g, beta, B, T, H, ws, flags, st);
        return launch_intra<KIND, bf16, 128>(q, k, v, g, beta, B, T, H, ws, flags, st);
    }
    if (D == 64) return launch_intra<KIND, float, 64>(q, k, v, g, beta, B, T, H, ws, flags, st);
    return launch_intra<KIND, float, 128>(q, k, v, g, beta, B, T, H, ws, flags, st);
}

template <int KIND>
dr_status dispatch_inter(int dtype, int D, const float* h0, void* o, float* hT, int B, int T, int H,
                         const void* ws, hipStream_t st) {
    if (dtype == DR_BF16) {
        if (D == 64) return launch_inter<KIND, bf16, 64>(h0, o, hT, B, T, H, ws, st);
        return launch_inter<KIND, bf16, 128>(h0, o, hT, B, T, H, ws, st);
    }
    if (D == 64) return launch_inter<KIND, float, 64>(h0, o, hT, B, T, H, ws, st);
    return launch_inter<KIND, float, 128>(h0, o, hT, B, T, H, ws, st);
}

dr_status run_intra(int kind, const void* q, const void* k, const void* v, const float* g,
                    const float* beta, int B, int T, int H, int D, int dtype, void* ws, unsigned* flags,
                    hipStream_t st) {
    switch (kind) {
        case DR_KIND_KDA: return dispatch_intra<dr::KIND_KDA>(dtype, D, q, k, v, g, beta, B, T, H, ws, flags, st);
        case DR_KIND_GDN: return dispatch_intra<dr::KIND_GDN>(dtype, D, q, k, v, g, beta, B, T, H, ws, flags, st);
        default: return dispatch_intra<dr::KIND_LA>(dtype, D, q, k, v, g, nullptr, B, T, H, ws, flags, st);
    }
}

dr_status run_inter(int kind, const float* h0, void* o, float* hT, int B, int T, int H, int D, int dtype,
                    const void* ws, hipStream_t st) {
    switch (kind) {
        case DR_KIND_KDA: return dispatch_inter<dr::KIND_KDA>(dtype, D, h0, o, hT, B, T, H, ws, st);
        case DR_KIND_GDN: return dispatch_inter<dr::KIND_GDN>(dtype, D, h0, o, hT, B, T, H, ws, st);
        default: return dispatch_inter<dr::KIND_LA>(dtype, D, h0, o, hT, B, T, H, ws, st);
    }
}

dr_status forward(int kind, const void* q, const void* k, const void* v, const float* g,
                  const float* beta, const float* h0, void* o, float* hT, int B, int T, int H, int Dk,
                  int Dv, int C, int dtype, void* ws, size_t ws_bytes, unsigned* flags, void* stream) {
    dr_status s = validate(kind, q, k, v, g, beta, B, T, H, Dk, Dv, C, dtype);
    if (s != DR_OK) return s;
    if (T > 0 && !o) return DR_ERR_INVALID_ARG;
    if (!aligned16(o) || !aligned16(h0) || !aligned16(hT) || !aligned16(ws)) return DR_ERR_INVALID_ARG;
    const size_t need = dr_workspace_bytes(kind, B, T, H, Dk, Dv, C, dtype);
    if (T > 0 && (ws == nullptr || ws_bytes < need)) return DR_ERR_WORKSPACE;
    if (T == 0 && hT == nullptr) return DR_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (T > 0) {
        s = run_intra(kind, q, k, v, g, beta, B, T, H, Dk, dtype, ws, flags, st);
        if (s != DR_OK) return s;
    }
    return run_inter(kind, h0, o, hT, B, T, H, Dk, dtype, ws, st);
}

}  // namespace

extern "C" {

size_t dr_record_bytes(int Dk, int Dv, int C, int dtype) {
    if (Dk != Dv || (Dk != 64 && Dk != 128) || C != dr::kChunk) return 0;
    if (dtype != DR_F32 && dtype != DR_BF16) return 0;
    return record_bytes(Dk, dtype);
}

size_t dr_workspace_bytes(int kind, int B, int T, int H, int Dk, int Dv, int C, int dtype) {
    if (kind < 0 || kind > 2 || B <= 0 || H <= 0 || T < 0) return 0;
    const size_t rec = dr_record_bytes(Dk, Dv, C, dtype);
    if (rec == 0) return 0;
    return (size_t)B * H * (size_t)ceil_div(T, C) * rec;
}

dr_status kda_fwd(const void* q, const void* k, const void* v, const float* g, const float* beta,
                  const float* h0, void* o, float* hT, int B, int T, int H, int Dk, int Dv, int C,
                  int dtype, void* workspace, size_t workspace_bytes, unsigned* flags, void* stream) {
    return forward(DR_KIND_KDA, q, k, v, g, beta, h0, o, hT, B, T, H, Dk, Dv, C, dtype, workspace,
                   workspace_bytes, flags, stream);
}

dr_status gdn_fwd(const void* q, const void* k, const void* v, const float* g, const float* beta,
                  const float* h0, void* o, float* hT, int B, int T, int H, int Dk, int Dv, int C,
                  int dtype, void* workspace, size_t workspace_bytes, unsigned* flags, void* stream) {
    return forward(DR_KIND_GDN, q, k, v, g, beta, h0, o, hT, B, T, H, Dk, Dv, C, dtype, workspace,
                   workspace_bytes, flags, stream);
}

dr_status decay_la_fwd(const void* q, const void* k, const void* v, const float* g, const float* h0,
                       void* o, float* hT, int B, int T, int H, int Dk, int Dv, int C, int dtype,
                       void* workspace, size_t workspace_bytes, void* stream) {
    return forward(DR_KIND_DECAY_LA, q, k, v, g, nullptr, h0, o, hT, B, T, H, Dk, Dv, C, dtype, workspace,
                   workspace_bytes, nullptr, stream);
}

dr_status dr_intra(int kind, const void* q, const void* k, const void* v, const float* g, const float* beta,
                   int B, int T, int H, int Dk, int Dv, int C, int dtype, void* workspace,
                   size_t workspace_bytes, unsigned* flags, void* stream) {
    dr_status s = validate(kind, q, k, v, g, beta, B, T, H, Dk, Dv, C, dtype);
    if (s != DR_OK) return s;
    if (!aligned16(workspace)) return DR_ERR_INVALID_ARG;
    if (T > 0 && (!workspace || workspace_bytes < dr_workspace_bytes(kind, B, T, H, Dk, Dv, C, dtype)))
        return DR_ERR_WORKSPACE;
    return run_intra(kind, q, k, v, g, beta, B, T, H, Dk, dtype, workspace, flags,
                     static_cast<hipStream_t>(stream));
}

dr_status dr_inter(int kind, const float* h0, void* o, float* hT, int B, int T, int H, int Dk, int Dv,
                   int C, int dtype, const void* workspace, size_t workspace_bytes, void* stream) {
    if (kind < 0 || kind > 2 || B <= 0 || H <= 0 || T < 0) return DR_ERR_INVALID_ARG;
    if (dtype != DR_F32 && dtype != DR_BF16) return DR_ERR_INVALID_ARG;
    if (Dk != Dv || (Dk != 64 && Dk != 128) || C != dr::kChunk) return DR_ERR_UNSUPPORTED;
    if (T > 0 && !o) return DR_ERR_INVALID_ARG;
    if (!aligned16(o) || !aligned16(h0) || !aligned16(hT) || !aligned16(workspace)) return DR_ERR_INVALID_ARG;
    if (T > 0 && (!workspace || workspace_bytes < dr_workspace_bytes(kind, B, T, H, Dk, Dv, C, dtype)))
        return DR_ERR_WORKSPACE;
    if (T == 0 && hT == nullptr) return DR_OK;
    return run_inter(kind, h0, o, hT, B, T, H, Dk, dtype, workspace, static_cast<hipStream_t>(stream));
}

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

const char* dr_status_string(int status) {
    switch (status) {
        case DR_OK: return "ok";
        case DR_ERR_INVALID_ARG: return "invalid argument";
        case DR_ERR_UNSUPPORTED: return "unsupported size (Dk == Dv in {64, 128}, C == 64)";
        case DR_ERR_HIP: return "HIP launch failed";
        case DR_ERR_WORKSPACE: return "workspace missing or too small";
        default: return "unknown status";
    }
}

int dr_abi_version(void) { return 1; }

}  // extern "C"
