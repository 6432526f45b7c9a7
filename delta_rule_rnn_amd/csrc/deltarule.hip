// deltarule.hip -- host side of the C ABI declared in include/deltarule.h:
// argument validation, workspace sizing and kernel dispatch for gfx950.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "../../include/deltarule.h"
#include "common.h"
#include "inter.h"
#include "intra.h"
#include "decode.h"
#include "steps.h"
#include "backward.h"
#include "prologue.h"

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

// One forward problem: the arguments every launch needs.
struct Problem {
    int kind, dtype, D, B, T, H, NT;
    const void *q, *k, *v;
    const float *g, *beta;
    void* o;
    uint8_t* ws;
    unsigned* flags;
    // packed sequences only: B sequences, chunk table and descriptors in the
    // workspace (see varlen_layout)
    const int4* table = nullptr;
    const int4* seqinfo = nullptr;
    const int* total = nullptr;
    int maxchunks = 0;
    // input prologue (use_pro selects the kernels that apply it)
    dr::Prologue pro{0u, 1.f, nullptr, nullptr};
    bool use_pro = false;
};

// Checks a caller's prologue and converts it; *use is false when it is
// absent or does nothing (no ops, scale 1).
dr_status resolve_prologue(int kind, const dr_prologue* in, dr::Prologue* out, bool* use) {
    *use = false;
    *out = dr::Prologue{0u, 1.f, nullptr, nullptr};
    if (in == nullptr) return DR_OK;
    const unsigned known = DR_PRO_QK_L2NORM | DR_PRO_BETA_SIGMOID | DR_PRO_BETA_X2 | DR_PRO_GATE;
    if (in->ops & ~known) return DR_ERR_INVALID_ARG;
    if (!(in->scale == in->scale) || in->scale > 3.0e38f || in->scale < -3.0e38f) return DR_ERR_INVALID_ARG;
    if ((in->ops & DR_PRO_BETA_X2) && !(in->ops & DR_PRO_BETA_SIGMOID)) return DR_ERR_INVALID_ARG;
    if ((in->ops & (DR_PRO_BETA_SIGMOID | DR_PRO_BETA_X2)) && kind == DR_KIND_DECAY_LA) return DR_ERR_INVALID_ARG;
    if (in->ops & DR_PRO_GATE) {
        if (kind == DR_KIND_KDA) return DR_ERR_UNSUPPORTED;
        if (!in->A_log) return DR_ERR_INVALID_ARG;
        if ((reinterpret_cast<uintptr_t>(in->A_log) & 3u) || (reinterpret_cast<uintptr_t>(in->dt_bias) & 3u))
            return DR_ERR_INVALID_ARG;
    }
    static_assert(DR_PRO_QK_L2NORM == dr::PRO_QK_L2NORM && DR_PRO_BETA_SIGMOID == dr::PRO_BETA_SIGMOID &&
                      DR_PRO_BETA_X2 == dr::PRO_BETA_X2 && DR_PRO_GATE == dr::PRO_GATE,
                  "prologue bits");
    *out = dr::Prologue{in->ops, in->scale, (in->ops & DR_PRO_GATE) ? in->A_log : nullptr,
                        (in->ops & DR_PRO_GATE) ? in->dt_bias : nullptr};
    *use = in->ops != 0 || in->scale != 1.f;
    return DR_OK;
}

int device_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// Value columns per state-pass workgroup (16 * ntn): the widest slice that
// still gives every CU a workgroup.  Narrow slices multiply the reads of the
// operands all slices of a chain share (W, Q~, Kbar, Aqk); too few workgroups
// leave CUs idle.  DR_INTER_NTN (1, 2 or 4) overrides the choice for tuning.
int pick_ntn(int chains, int D) {
    if (const char* e = getenv("DR_INTER_NTN")) {
        const int v = atoi(e);
        if ((v == 1 || v == 2 || v == 4) && 16 * v <= D) return v;
    }
    const int cols = D / 16, cus = device_cus();
    int ntn = 4;
    while (ntn > 1 && (ntn > cols || (long long)chains * (cols / ntn) < cus)) ntn /= 2;
    return ntn;
}

int pick_pfd() {
    if (const char* e = getenv("DR_INTER_PFD")) {
        const int v = atoi(e);
        if (v == 0 || v == 2) return v;
    }
    return 2;
}

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

template <int KIND, bool PRO>
dr_status launch_intra_p(const Problem& p, int c0, int n, hipStream_t st) {
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

template <int KIND>
dr_status launch_inter_k(const Problem& p, const float* h0, float* hT, int c0, int n, hipStream_t st) {
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

Problem make_problem(int kind, const void* q, const void* k, const void* v, const float* g,
                     const float* beta, void* o, int B, int T, int H, int D, int dtype, void* ws,
                     unsigned* flags) {
    Problem p;
    p.kind = kind; p.dtype = dtype; p.D = D; p.B = B; p.T = T; p.H = H;
    p.NT = ceil_div(T, dr::kChunk);
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = kind == DR_KIND_DECAY_LA ? nullptr : beta;
    p.o = o; p.ws = static_cast<uint8_t*>(ws); p.flags = flags;
    return p;
}

// ---- the backward's forward state pass: the state-pass kernel in STATES
// mode (entry state and Vnew of every chunk, no output) over the records the
// chunk-parallel kernel wrote; slice width and prefetch as for the forward
template <int KIND, typename E, int D, int NTN, int PFD>
dr_status launch_states_p(const Problem& p, const float* h0, float* hs, float* vn, hipStream_t st) {
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
dr_status launch_states_t(const Problem& p, const float* h0, float* hs, float* vn, hipStream_t st) {
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
dr_status launch_states(const Problem& p, const float* h0, float* hs, float* vn, hipStream_t st) {
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

dr_status forward(int kind, const void* q, const void* k, const void* v, const float* g,
                  const float* beta, const float* h0, void* o, float* hT, int B, int T, int H, int Dk,
                  int Dv, int C, int dtype, void* ws, size_t ws_bytes, unsigned* flags, void* stream,
                  const dr_prologue* pro = nullptr) {
    dr_status s = validate(kind, q, k, v, g, beta, B, T, H, Dk, Dv, C, dtype);
    if (s != DR_OK) return s;
    dr::Prologue pr;
    bool use_pro;
    if ((s = resolve_prologue(kind, pro, &pr, &use_pro)) != DR_OK) return s;
    if (T > 0 && !o) return DR_ERR_INVALID_ARG;
    if (!aligned16(o) || !aligned16(h0) || !aligned16(hT) || !aligned16(ws)) return DR_ERR_INVALID_ARG;
    const size_t need = dr_workspace_bytes(kind, B, T, H, Dk, Dv, C, dtype);
    if (T > 0 && (ws == nullptr || ws_bytes < need)) return DR_ERR_WORKSPACE;
    if (T == 0 && hT == nullptr) return DR_OK;
    Problem p = make_problem(kind, q, k, v, g, beta, o, B, T, H, Dk, dtype, ws, flags);
    p.pro = pr;
    p.use_pro = use_pro;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (T == 0) return launch_inter(p, h0, hT, 0, 0, st);
    s = launch_intra(p, 0, p.NT, st);
    if (s != DR_OK) return s;
    return launch_inter(p, h0, hT, 0, p.NT, st);
}

// ---- packed sequences ---------------------------------------------------------
// Workspace of the varlen forward: records [H][maxchunks], then the chunk
// table [maxchunks] int4, the sequence descriptors [N] int4 and the slot
// count, each block 256-byte aligned.  maxchunks = ceil(T/C) + N bounds
// sum_i ceil(len_i / C).
struct VarlenLayout {
    size_t rec, table, seqinfo, total, bytes;
    int maxchunks;
};
VarlenLayout varlen_layout(int N, int T, int H, int D, int dtype) {
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    VarlenLayout L;
    L.maxchunks = ceil_div(T, dr::kChunk) + N;
    L.rec = 0;
    L.table = up((size_t)H * L.maxchunks * record_bytes(D, dtype));
    L.seqinfo = L.table + up((size_t)L.maxchunks * sizeof(int4));
    L.total = L.seqinfo + up((size_t)N * sizeof(int4));
    L.bytes = L.total + 256;
    return L;
}

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

dr_status forward_varlen(int kind, const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const int* cu_seqlens, int N, const float* h0, void* o, float* hT,
                         int T, int H, int Dk, int Dv, int C, int dtype, void* ws, size_t ws_bytes,
                         unsigned* flags, void* stream, const dr_prologue* pro = nullptr) {
    dr_status s = validate(kind, q, k, v, g, beta, 1, T, H, Dk, Dv, C, dtype);
    if (s != DR_OK) return s;
    dr::Prologue pr;
    bool use_pro;
    if ((s = resolve_prologue(kind, pro, &pr, &use_pro)) != DR_OK) return s;
    if (N < 1 || !cu_seqlens) return DR_ERR_INVALID_ARG;
    // grid sizes, checked before the chunk table is enqueued
    if ((long long)N * H * (Dv / 16) > 0x7fffffffLL ||
        ((long long)ceil_div(T, dr::kChunk) + N) * H > 0x7fffffffLL)
        return DR_ERR_UNSUPPORTED;
    if (T > 0 && !o) return DR_ERR_INVALID_ARG;
    if (!aligned16(o) || !aligned16(h0) || !aligned16(hT) || !aligned16(ws)) return DR_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return DR_ERR_INVALID_ARG;
    const VarlenLayout L = varlen_layout(N, T, H, Dk, dtype);
    if (!ws || ws_bytes < L.bytes) return DR_ERR_WORKSPACE;
    Problem p = make_problem(kind, q, k, v, g, beta, o, N, T, H, Dk, dtype, ws, flags);
    uint8_t* w = static_cast<uint8_t*>(ws);
    p.table = reinterpret_cast<const int4*>(w + L.table);
    p.seqinfo = reinterpret_cast<const int4*>(w + L.seqinfo);
    p.total = reinterpret_cast<const int*>(w + L.total);
    p.maxchunks = L.maxchunks;
    p.pro = pr;
    p.use_pro = use_pro;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(dr::varlen_table_kernel, dim3(1), dim3(1024), 0, st, cu_seqlens, N, T, L.maxchunks,
                       reinterpret_cast<int4*>(w + L.table), reinterpret_cast<int4*>(w + L.seqinfo),
                       reinterpret_cast<int*>(w + L.total), flags);
    if ((s = check_launch()) != DR_OK) return s;
    if (T > 0) {
        switch (kind) {
            case DR_KIND_KDA: s = launch_intra_varlen_k<dr::KIND_KDA>(p, st); break;
            case DR_KIND_GDN: s = launch_intra_varlen_k<dr::KIND_GDN>(p, st); break;
            default: s = launch_intra_varlen_k<dr::KIND_LA>(p, st); break;
        }
        if (s != DR_OK) return s;
    }
    if (T == 0 && hT == nullptr) return DR_OK;
    // the state pass reads nseg, tokens and record slots from the descriptors
    return launch_inter(p, h0, hT, 0, 0, st);
}

// ---- recurrent decode step --------------------------------------------------
struct DecodeArgs {
    const void *q, *k, *v;
    const float *g, *beta;
    float* state;
    void* o;
    int B, T, H;
    dr::Prologue pro;
};

// State sizes above half the MI355X last-level cache (256 MB) use streaming
// state stores (see decode.h).
constexpr size_t kDecodeStreamBytes = (size_t)128 << 20;

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

dr_status decode(int kind, const void* q, const void* k, const void* v, const float* g, const float* beta,
                 float* state, void* o, int B, int T, int H, int Dk, int Dv, int dtype, void* stream,
                 const dr_prologue* pro = nullptr) {
    // same argument rules as the forward, with the chunk size not involved
    dr_status s = validate(kind, q, k, v, g, beta, B, T, H, Dk, Dv, dr::kChunk, dtype);
    if (s != DR_OK) return s;
    dr::Prologue pr;
    bool use_pro;
    if ((s = resolve_prologue(kind, pro, &pr, &use_pro)) != DR_OK) return s;
    if (T > 0 && (!o || !state)) return DR_ERR_INVALID_ARG;
    if (!aligned16(o) || !aligned16(state)) return DR_ERR_INVALID_ARG;
    if (T == 0) return DR_OK;
    if ((long long)B * H * (Dv / 64) > 0x7fffffffLL) return DR_ERR_UNSUPPORTED;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const DecodeArgs a{q, k, v, g, kind == DR_KIND_DECAY_LA ? nullptr : beta, state, o, B, T, H, pr};
    switch (kind) {
        case DR_KIND_KDA: return launch_decode_k<dr::KIND_KDA>(a, use_pro, Dk, dtype, st);
        case DR_KIND_GDN: return launch_decode_k<dr::KIND_GDN>(a, use_pro, Dk, dtype, st);
        default: return launch_decode_k<dr::KIND_LA>(a, use_pro, Dk, dtype, st);
    }
}

// ---- backward ------------------------------------------------------------------
// Workspace: the natural fp32 chunk arrays of the prep kernel, then the entry
// states S_c [DK][DV], the exit adjoints dS'_c [DK][DV], Vnew_c and dVnew_c
// [C][DV] of every chunk, each block 256-byte aligned.
struct BwdLayout {
    size_t prep, hs, dhs, vn, dvn, rec, bytes;
};
// n = number of per-chunk entries (dense: B * H * ceil(T/C); packed:
// H * maxchunks)
// (the forward's chunk records come last: the forward state pass runs the
// forward's own two kernels over them)
BwdLayout bwd_layout_n(size_t n, int D, int dtype) {
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t pf = D == 64 ? dr::bw::Prep<64>::FLOATS : dr::bw::Prep<128>::FLOATS;
    BwdLayout L;
    L.prep = 0;
    L.hs = up(n * pf * 4);
    L.dhs = L.hs + up(n * D * D * 4);
    L.vn = L.dhs + up(n * D * D * 4);
    L.dvn = L.vn + up(n * dr::kChunk * D * 4);
    L.rec = L.dvn + up(n * dr::kChunk * D * 4);
    L.bytes = L.rec + up(n * record_bytes(D, dtype));
    return L;
}
BwdLayout bwd_layout(int B, int T, int H, int D, int dtype) {
    return bwd_layout_n((size_t)B * H * (size_t)ceil_div(T, dr::kChunk), D, dtype);
}

// B is the sequence count for packed sequences (pk.table set; T is then the
// packed token count and the tensors have a batch of one).
struct BwdArgs {
    const void *q, *k, *v, *dout;
    const float *g, *beta, *h0, *dhT;
    void *dq, *dk, *dv;
    float *dg, *dbeta, *dh0;
    int B, T, H, NT;
    uint8_t* ws;
    BwdLayout L;
    dr::bw::Pack pk;
};

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
// (q^, k^ in the I/O dtype, g^ and beta^ fp32), then the backward's own.
struct ProBwdLayout {
    size_t qh, kh, gh, bh, core, bytes;
};
// core: the bytes of what follows the prologue's part (the backward's own
// workspace, with the chunk table first for packed sequences)
ProBwdLayout probwd_layout(int kind, int B, int T, int H, int D, int dtype, size_t core) {
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t n = (size_t)B * T * H, esz = dtype == DR_BF16 ? 2 : 4;
    ProBwdLayout L;
    L.qh = 0;
    L.kh = up(n * D * esz);
    L.gh = L.kh + up(n * D * esz);
    L.bh = L.gh + up(n * (kind == DR_KIND_KDA ? D : 1) * 4);
    L.core = L.bh + up(n * 4);
    L.bytes = L.core + core;
    return L;
}

template <typename E, int D, bool PERCH>
dr_status launch_prologue_t(bool backward, const void* q, const void* k, const float* g, const float* beta, void* qh,
                            void* kh, float* gh, float* bh, void* dq, void* dk, float* dg, float* dbeta,
                            float* dA_log, float* ddt, int B, int T, int H, const dr::Prologue& pro, hipStream_t st) {
    const long long rows = (long long)B * T;
    const long long blocks = (long long)H * ((rows + dr::kProRows - 1) / dr::kProRows);
    if (blocks > 0x7fffffffLL) return DR_ERR_UNSUPPORTED;
    if (!backward)
        hipLaunchKernelGGL((dr::prologue_apply_kernel<E, D, PERCH>), dim3((unsigned)blocks), dim3(256), 0, st,
                           static_cast<const E*>(q), static_cast<const E*>(k), g, beta, static_cast<E*>(qh),
                           static_cast<E*>(kh), gh, bh, rows, H, pro);
    else
        hipLaunchKernelGGL((dr::prologue_backward_kernel<E, D, PERCH>), dim3((unsigned)blocks), dim3(256), 0, st,
                           static_cast<const E*>(q), static_cast<const E*>(k), g, beta, static_cast<E*>(dq),
                           static_cast<E*>(dk), dg, dbeta, dA_log, ddt, rows, H, pro);
    return check_launch();
}

dr_status launch_prologue(bool backward, int kind, int D, int dtype, const void* q, const void* k, const float* g,
                          const float* beta, void* qh, void* kh, float* gh, float* bh, void* dq, void* dk, float* dg,
                          float* dbeta, float* dA_log, float* ddt, int B, int T, int H, const dr::Prologue& pro,
                          hipStream_t st) {
#define DR_PRO(E, DD, PC) \
    return launch_prologue_t<E, DD, PC>(backward, q, k, g, beta, qh, kh, gh, bh, dq, dk, dg, dbeta, dA_log, ddt, B, T, H, pro, st)
    const bool perch = kind == DR_KIND_KDA;
    if (dtype == DR_BF16) {
        if (D == 64) { if (perch) DR_PRO(bf16, 64, true); else DR_PRO(bf16, 64, false); }
        if (perch) DR_PRO(bf16, 128, true); else DR_PRO(bf16, 128, false);
    }
    if (D == 64) { if (perch) DR_PRO(float, 64, true); else DR_PRO(float, 64, false); }
    if (perch) DR_PRO(float, 128, true); else DR_PRO(float, 128, false);
#undef DR_PRO
}

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
// prologue.  Workspace: [prologue part][chunk table (packed)][core].
dr_status backward_impl(int kind, const void* q, const void* k, const void* v, const float* g, const float* beta,
                        const int* cu_seqlens, int N, const float* h0, const void* dout, const float* dhT, void* dq,
                        void* dk, void* dv, float* dg, float* dbeta, float* dh0, float* dA_log, float* ddt_bias,
                        int B, int T, int H, int Dk, int Dv, int C, int dtype, const dr_prologue* prologue,
                        void* workspace, size_t workspace_bytes, unsigned* flags, void* stream) {
    dr_status s = validate(kind, q, k, v, g, beta, B, T, H, Dk, Dv, C, dtype);
    if (s != DR_OK) return s;
    dr::Prologue pr;
    bool use_pro;
    if ((s = resolve_prologue(kind, prologue, &pr, &use_pro)) != DR_OK) return s;
    const bool delta = kind != DR_KIND_DECAY_LA;
    const bool packed = cu_seqlens != nullptr;
    const int chains = packed ? N : B;
    const bool gate = use_pro && (pr.ops & dr::PRO_GATE);
    if (T > 0 && (!dout || !dq || !dk || !dv || !dg || (delta && !dbeta))) return DR_ERR_INVALID_ARG;
    if (gate && (!dA_log || (pr.dt_bias && !ddt_bias))) return DR_ERR_INVALID_ARG;
    const void* ptrs[] = {h0, dout, dhT, dq, dk, dv, dg, dbeta, dh0, workspace};
    for (const void* p : ptrs)
        if (!aligned16(p)) return DR_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(dA_log) & 3u) || (reinterpret_cast<uintptr_t>(ddt_bias) & 3u))
        return DR_ERR_INVALID_ARG;
    // grid sizes of the backward's kernels, checked before anything is enqueued
    const long long items = packed ? ((long long)ceil_div(T, dr::kChunk) + N) * H
                                   : (long long)B * ceil_div(T, dr::kChunk) * H;
    if ((long long)chains * H * (Dv / 16) > 0x7fffffffLL || items > 0x7fffffffLL) return DR_ERR_UNSUPPORTED;
    // workspace: [prologue part][chunk table (packed)][core]; every check
    // before the first launch
    VarlenLayout V{};
    size_t table_bytes = 0;
    BwdLayout L;
    if (packed) {
        V = varlen_layout(N, T, H, Dk, dtype);
        table_bytes = V.bytes - V.table;
        L = bwd_layout_n((size_t)H * V.maxchunks, Dk, dtype);
    } else {
        L = bwd_layout(B, T, H, Dk, dtype);
    }
    const size_t core_bytes = table_bytes + L.bytes;
    const ProBwdLayout PL = probwd_layout(kind, B, T, H, Dk, dtype, core_bytes);
    if (T > 0 && (!workspace || workspace_bytes < (use_pro ? PL.bytes : core_bytes))) return DR_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (gate) {
        // accumulated below (or left zero without tokens)
        hipLaunchKernelGGL(dr::copy_or_zero_kernel, dim3(((size_t)H + 255) / 256), dim3(256), 0, st, dA_log,
                           (const float*)nullptr, (size_t)H);
        if (ddt_bias)
            hipLaunchKernelGGL(dr::copy_or_zero_kernel, dim3(((size_t)H + 255) / 256), dim3(256), 0, st, ddt_bias,
                               (const float*)nullptr, (size_t)H);
        if ((s = check_launch()) != DR_OK) return s;
    }
    if (T == 0) {
        // no tokens: dh0 = dhT (or zero); nothing else to write
        if (!dh0) return DR_OK;
        const size_t n = (size_t)chains * H * Dk * Dv;
        hipLaunchKernelGGL(dr::copy_or_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, dh0, dhT, n);
        return check_launch();
    }
    uint8_t* w = static_cast<uint8_t*>(workspace);
    uint8_t* rest = use_pro ? w + PL.core : w;     // [chunk table][core]
    dr::bw::Pack pk{nullptr, nullptr, nullptr, 0};
    if (packed) {
        // the chunk table of the packed forward, rebased to this workspace
        int4* table = reinterpret_cast<int4*>(rest);
        int4* seqinfo = reinterpret_cast<int4*>(rest + (V.seqinfo - V.table));
        int* total = reinterpret_cast<int*>(rest + (V.total - V.table));
        hipLaunchKernelGGL(dr::varlen_table_kernel, dim3(1), dim3(1024), 0, st, cu_seqlens, N, T, V.maxchunks, table,
                           seqinfo, total, flags);
        if ((s = check_launch()) != DR_OK) return s;
        pk = dr::bw::Pack{table, seqinfo, total, V.maxchunks};
    }
    // the recurrence's inputs: the caller's, or the prologue's outputs
    const void *rq = q, *rk = k;
    const float *rg = g, *rb = delta ? beta : nullptr;
    if (use_pro) {
        void* qh = w + PL.qh;
        void* kh = w + PL.kh;
        float* gh = reinterpret_cast<float*>(w + PL.gh);
        float* bh = delta ? reinterpret_cast<float*>(w + PL.bh) : nullptr;
        s = launch_prologue(false, kind, Dk, dtype, q, k, g, rb, qh, kh, gh, bh, nullptr, nullptr, nullptr, nullptr,
                            nullptr, nullptr, B, T, H, pr, st);
        if (s != DR_OK) return s;
        rq = qh; rk = kh; rg = gh; rb = bh;
    }
    uint8_t* core = rest + table_bytes;
    {
        // forward state pass: the forward's chunk-parallel kernel writes the
        // chunk records, the state-pass kernel in STATES mode the entry
        // state and Vnew of every chunk (per-chunk arrays share the records'
        // index, dense and packed)
        Problem p = make_problem(kind, rq, rk, v, rg, rb, nullptr, chains, T, H, Dk, dtype, core + L.rec, nullptr);
        if (packed) {
            p.table = pk.table;
            p.seqinfo = pk.seqinfo;
            p.total = pk.total;
            p.maxchunks = pk.maxchunks;
        }
        s = packed ? launch_intra_varlen(p, st) : launch_intra(p, 0, p.NT, st);
        if (s != DR_OK) return s;
        s = launch_states(p, h0, reinterpret_cast<float*>(core + L.hs), reinterpret_cast<float*>(core + L.vn), st);
        if (s != DR_OK) return s;
    }
    BwdArgs a{rq, rk, v, dout, rg, rb, h0, dhT, dq, dk, dv, dg, delta ? dbeta : nullptr, dh0,
              chains, T, H, ceil_div(T, dr::kChunk), core, L, pk};
    switch (kind) {
        case DR_KIND_KDA: s = launch_backward_k<dr::KIND_KDA>(a, Dk, dtype, st); break;
        case DR_KIND_GDN: s = launch_backward_k<dr::KIND_GDN>(a, Dk, dtype, st); break;
        default: s = launch_backward_k<dr::KIND_LA>(a, Dk, dtype, st); break;
    }
    if (s != DR_OK || !use_pro) return s;
    // gradients with respect to the raw inputs, in place
    return launch_prologue(true, kind, Dk, dtype, q, k, g, delta ? beta : nullptr, nullptr, nullptr, nullptr,
                           nullptr, dq, dk, dg, delta ? dbeta : nullptr, dA_log, ddt_bias, B, T, H, pr, st);
}

}  // namespace

extern "C" {

size_t dr_backward_workspace_bytes(int kind, int B, int T, int H, int Dk, int Dv, int C, int dtype) {
    if (kind < 0 || kind > 2 || B <= 0 || H <= 0 || T < 0) return 0;
    if (dr_record_bytes(Dk, Dv, C, dtype) == 0) return 0;
    return bwd_layout(B, T, H, Dk, dtype).bytes;
}

dr_status dr_backward(int kind, const void* q, const void* k, const void* v, const float* g, const float* beta,
                      const float* h0, const void* dout, const float* dhT, void* dq, void* dk, void* dv, float* dg,
                      float* dbeta, float* dh0, int B, int T, int H, int Dk, int Dv, int C, int dtype,
                      void* workspace, size_t workspace_bytes, void* stream) {
    return dr_backward_prologue(kind, q, k, v, g, beta, h0, dout, dhT, dq, dk, dv, dg, dbeta, dh0, nullptr, nullptr,
                                B, T, H, Dk, Dv, C, dtype, nullptr, workspace, workspace_bytes, stream);
}

size_t dr_backward_prologue_workspace_bytes(int kind, int B, int T, int H, int Dk, int Dv, int C, int dtype) {
    if (kind < 0 || kind > 2 || B <= 0 || H <= 0 || T < 0) return 0;
    if (dr_record_bytes(Dk, Dv, C, dtype) == 0) return 0;
    return probwd_layout(kind, B, T, H, Dk, dtype, bwd_layout(B, T, H, Dk, dtype).bytes).bytes;
}

dr_status dr_backward_prologue(int kind, const void* q, const void* k, const void* v, const float* g,
                               const float* beta, const float* h0, const void* dout, const float* dhT, void* dq,
                               void* dk, void* dv, float* dg, float* dbeta, float* dh0, float* dA_log,
                               float* ddt_bias, int B, int T, int H, int Dk, int Dv, int C, int dtype,
                               const dr_prologue* prologue, void* workspace, size_t workspace_bytes, void* stream) {
    return backward_impl(kind, q, k, v, g, beta, nullptr, B, h0, dout, dhT, dq, dk, dv, dg, dbeta, dh0, dA_log,
                         ddt_bias, B, T, H, Dk, Dv, C, dtype, prologue, workspace, workspace_bytes, nullptr, stream);
}

size_t dr_backward_varlen_workspace_bytes(int kind, int N, int T, int H, int Dk, int Dv, int C, int dtype,
                                          int with_prologue) {
    if (kind < 0 || kind > 2 || N < 1 || H <= 0 || T < 0) return 0;
    if (dr_record_bytes(Dk, Dv, C, dtype) == 0) return 0;
    const VarlenLayout V = varlen_layout(N, T, H, Dk, dtype);
    const size_t core = (V.bytes - V.table) + bwd_layout_n((size_t)H * V.maxchunks, Dk, dtype).bytes;
    return with_prologue ? probwd_layout(kind, 1, T, H, Dk, dtype, core).bytes : core;
}

dr_status dr_backward_varlen(int kind, const void* q, const void* k, const void* v, const float* g,
                             const float* beta, const int* cu_seqlens, int N, const float* h0, const void* dout,
                             const float* dhT, void* dq, void* dk, void* dv, float* dg, float* dbeta, float* dh0,
                             float* dA_log, float* ddt_bias, int T, int H, int Dk, int Dv, int C, int dtype,
                             const dr_prologue* prologue, void* workspace, size_t workspace_bytes, unsigned* flags,
                             void* stream) {
    if (N < 1 || !cu_seqlens || (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u)) return DR_ERR_INVALID_ARG;
    return backward_impl(kind, q, k, v, g, beta, cu_seqlens, N, h0, dout, dhT, dq, dk, dv, dg, dbeta, dh0, dA_log,
                         ddt_bias, 1, T, H, Dk, Dv, C, dtype, prologue, workspace, workspace_bytes, flags, stream);
}

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
    const Problem p = make_problem(kind, q, k, v, g, beta, nullptr, B, T, H, Dk, dtype, workspace, flags);
    return launch_intra(p, 0, p.NT, static_cast<hipStream_t>(stream));
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
    const Problem p = make_problem(kind, nullptr, nullptr, nullptr, nullptr, nullptr, o, B, T, H, Dk, dtype,
                                   const_cast<void*>(workspace), nullptr);
    return launch_inter(p, h0, hT, 0, p.NT, static_cast<hipStream_t>(stream));
}

size_t dr_workspace_bytes_varlen(int kind, int N, int T, int H, int Dk, int Dv, int C, int dtype) {
    if (kind < 0 || kind > 2 || N < 1 || H <= 0 || T < 0) return 0;
    if (dr_record_bytes(Dk, Dv, C, dtype) == 0) return 0;
    return varlen_layout(N, T, H, Dk, dtype).bytes;
}

dr_status kda_fwd_varlen(const void* q, const void* k, const void* v, const float* g, const float* beta,
                         const int* cu_seqlens, int N, const float* h0, void* o, float* hT, int T, int H, int Dk,
                         int Dv, int C, int dtype, void* workspace, size_t workspace_bytes, unsigned* flags,
                         void* stream) {
    return forward_varlen(DR_KIND_KDA, q, k, v, g, beta, cu_seqlens, N, h0, o, hT, T, H, Dk, Dv, C, dtype,
                          workspace, workspace_bytes, flags, stream);
}

dr_status gdn_fwd_varlen(const void* q, const void* k, const void* v, const float* g, const float* beta,
                         const int* cu_seqlens, int N, const float* h0, void* o, float* hT, int T, int H, int Dk,
                         int Dv, int C, int dtype, void* workspace, size_t workspace_bytes, unsigned* flags,
                         void* stream) {
    return forward_varlen(DR_KIND_GDN, q, k, v, g, beta, cu_seqlens, N, h0, o, hT, T, H, Dk, Dv, C, dtype,
                          workspace, workspace_bytes, flags, stream);
}

dr_status decay_la_fwd_varlen(const void* q, const void* k, const void* v, const float* g, const int* cu_seqlens,
                              int N, const float* h0, void* o, float* hT, int T, int H, int Dk, int Dv, int C,
                              int dtype, void* workspace, size_t workspace_bytes, unsigned* flags, void* stream) {
    return forward_varlen(DR_KIND_DECAY_LA, q, k, v, g, nullptr, cu_seqlens, N, h0, o, hT, T, H, Dk, Dv, C, dtype,
                          workspace, workspace_bytes, flags, stream);
}

dr_status kda_decode(const void* q, const void* k, const void* v, const float* g, const float* beta,
                     float* state, void* o, int B, int T, int H, int Dk, int Dv, int dtype, void* stream) {
    return decode(DR_KIND_KDA, q, k, v, g, beta, state, o, B, T, H, Dk, Dv, dtype, stream);
}

dr_status gdn_decode(const void* q, const void* k, const void* v, const float* g, const float* beta,
                     float* state, void* o, int B, int T, int H, int Dk, int Dv, int dtype, void* stream) {
    return decode(DR_KIND_GDN, q, k, v, g, beta, state, o, B, T, H, Dk, Dv, dtype, stream);
}

dr_status decay_la_decode(const void* q, const void* k, const void* v, const float* g, float* state, void* o,
                          int B, int T, int H, int Dk, int Dv, int dtype, void* stream) {
    return decode(DR_KIND_DECAY_LA, q, k, v, g, nullptr, state, o, B, T, H, Dk, Dv, dtype, stream);
}

dr_status dr_forward(int kind, const void* q, const void* k, const void* v, const float* g, const float* beta,
                     const float* h0, void* o, float* hT, int B, int T, int H, int Dk, int Dv, int C, int dtype,
                     const dr_prologue* prologue, void* workspace, size_t workspace_bytes, unsigned* flags,
                     void* stream) {
    if (kind < 0 || kind > 2) return DR_ERR_INVALID_ARG;
    return forward(kind, q, k, v, g, kind == DR_KIND_DECAY_LA ? nullptr : beta, h0, o, hT, B, T, H, Dk, Dv, C,
                   dtype, workspace, workspace_bytes, flags, stream, prologue);
}

dr_status dr_forward_varlen(int kind, const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const int* cu_seqlens, int N, const float* h0, void* o, float* hT,
                            int T, int H, int Dk, int Dv, int C, int dtype, const dr_prologue* prologue,
                            void* workspace, size_t workspace_bytes, unsigned* flags, void* stream) {
    if (kind < 0 || kind > 2) return DR_ERR_INVALID_ARG;
    return forward_varlen(kind, q, k, v, g, kind == DR_KIND_DECAY_LA ? nullptr : beta, cu_seqlens, N, h0, o, hT,
                          T, H, Dk, Dv, C, dtype, workspace, workspace_bytes, flags, stream, prologue);
}

dr_status dr_decode(int kind, const void* q, const void* k, const void* v, const float* g, const float* beta,
                    float* state, void* o, int B, int T, int H, int Dk, int Dv, int dtype,
                    const dr_prologue* prologue, void* stream) {
    if (kind < 0 || kind > 2) return DR_ERR_INVALID_ARG;
    return decode(kind, q, k, v, g, kind == DR_KIND_DECAY_LA ? nullptr : beta, state, o, B, T, H, Dk, Dv, dtype,
                  stream, prologue);
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

int dr_abi_version(void) { return 5; }

}  // extern "C"
