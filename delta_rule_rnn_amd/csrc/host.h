// host.h -- host-side pieces shared by the library's translation units:
// argument checks, problem descriptors, workspace layouts and the launchers
// each kernel translation unit defines.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>

#include "../../include/deltarule.h"
#include "common.h"

namespace drh {

using dr::bf16;

inline bool aligned16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline dr_status check_launch() {
    return hipGetLastError() == hipSuccess ? DR_OK : DR_ERR_HIP;
}

// (in 64-bit arithmetic: a may be as large as INT_MAX)
inline int ceil_div(int a, int b) { return (int)(((long long)a + b - 1) / b); }

// The largest problem any entry point or size query accepts: B*T*H*D
// elements of one tensor at most 2^40 (evaluated in floating point, so that
// no product of the four ints can overflow).
inline bool within_limit(int B, int T, int H, int D) {
    return (double)B * (double)T * (double)H * (double)D <= 1099511627776.0;
}

// 128-token chunks (sub-chunked records) are built for the dense forward in
// bf16 at both head sizes and in fp32 at D = 64 (an fp32 D = 128 sub-chunk
// alone fills the LDS).
constexpr int kChunk128 = 2 * dr::kChunk;
inline bool chunk128_built(int D, int dtype) { return dtype == DR_BF16 || D == 64; }

inline size_t record_bytes(int D, int dtype, int C = dr::kChunk) {
    if (C == kChunk128) {
        if (dtype == DR_BF16)
            return D == 64 ? dr::Rec<bf16, 64, 64, kChunk128>::BYTES : dr::Rec<bf16, 128, 128, kChunk128>::BYTES;
        return D == 64 ? dr::Rec<float, 64, 64, kChunk128>::BYTES : dr::Rec<float, 128, 128, kChunk128>::BYTES;
    }
    if (dtype == DR_BF16) return D == 64 ? dr::Rec<bf16, 64, 64>::BYTES : dr::Rec<bf16, 128, 128>::BYTES;
    return D == 64 ? dr::Rec<float, 64, 64>::BYTES : dr::Rec<float, 128, 128>::BYTES;
}

// Shared validation for the full forward and the fused step entry points
// (allow128: the caller runs the dense forward, which also takes C = 128).
inline dr_status validate(int kind, const void* q, const void* k, const void* v, const float* g,
                   const float* beta, int B, int T, int H, int Dk, int Dv, int C, int dtype,
                   bool allow128 = false) {
    if (kind < 0 || kind > 2) return DR_ERR_INVALID_ARG;
    if (B <= 0 || H <= 0 || T < 0) return DR_ERR_INVALID_ARG;
    if (dtype != DR_F32 && dtype != DR_BF16) return DR_ERR_INVALID_ARG;
    if (Dk <= 0 || Dv <= 0 || C <= 0) return DR_ERR_INVALID_ARG;
    if (Dk != Dv || (Dk != 64 && Dk != 128)) return DR_ERR_UNSUPPORTED;
    if (C != dr::kChunk && !(allow128 && C == kChunk128 && chunk128_built(Dk, dtype))) return DR_ERR_UNSUPPORTED;
    if (!within_limit(B, T, H, Dk)) return DR_ERR_INVALID_ARG;
    if (T > 0 && (!q || !k || !v || !g)) return DR_ERR_INVALID_ARG;
    if (T > 0 && kind != DR_KIND_DECAY_LA && !beta) return DR_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(beta))
        return DR_ERR_INVALID_ARG;
    return DR_OK;
}

// One forward problem: the arguments every launch needs.
struct Problem {
    int kind, dtype, D, B, T, H, NT;
    int C = dr::kChunk;     // record chunk: 64, or 128 (sub-chunked)
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
inline dr_status resolve_prologue(int kind, const dr_prologue* in, dr::Prologue* out, bool* use) {
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

inline int device_cus() {
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
inline int pick_ntn(int chains, int D) {
    if (const char* e = getenv("DR_INTER_NTN")) {
        const int v = atoi(e);
        if ((v == 1 || v == 2 || v == 4) && 16 * v <= D) return v;
    }
    const int cols = D / 16, cus = device_cus();
    int ntn = 4;
    while (ntn > 1 && (ntn > cols || (long long)chains * (cols / ntn) < cus)) ntn /= 2;
    return ntn;
}

inline int pick_pfd() {
    if (const char* e = getenv("DR_INTER_PFD")) {
        const int v = atoi(e);
        if (v == 0 || v == 2) return v;
    }
    return 2;
}

inline Problem make_problem(int kind, const void* q, const void* k, const void* v, const float* g,
                     const float* beta, void* o, int B, int T, int H, int D, int dtype, void* ws,
                     unsigned* flags, int C = dr::kChunk) {
    Problem p;
    p.kind = kind; p.dtype = dtype; p.D = D; p.B = B; p.T = T; p.H = H;
    p.C = C;
    p.NT = ceil_div(T, C);
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = kind == DR_KIND_DECAY_LA ? nullptr : beta;
    p.o = o; p.ws = static_cast<uint8_t*>(ws); p.flags = flags;
    return p;
}


// Workspace of the varlen forward: records [H][maxchunks], then the chunk
// table [maxchunks] int4, the sequence descriptors [N] int4 and the slot
// count, each block 256-byte aligned.  maxchunks = ceil(T/C) + N bounds
// sum_i ceil(len_i / C).
struct VarlenLayout {
    size_t rec, table, seqinfo, total, bytes;
    int maxchunks;
};
inline VarlenLayout varlen_layout(int N, int T, int H, int D, int dtype) {
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

// bytes of the backward prep kernel's per-chunk arrays (floats), defined with
// the backward kernels
size_t bwd_prep_floats(int D);

// Segments of the chains: the chunks of each of `chains` chains grouped
// into NS segments of L consecutive chunks, so that chains * NS is about
// kSegGroups workgroups (one per CU); NS = 1 where the chains alone fill the
// GPU.  Used by the segment-parallel forward and the segment-parallel
// reverse pass of the backward; it depends only on the sizes.
constexpr int kSegGroups = 256;
struct SegPlan {
    int NS, L;
};
inline SegPlan seg_plan(long long chains, int NT) {
    SegPlan S{1, 1};
    if (NT > 1 && chains < kSegGroups) {
        const int want = (int)std::min<long long>(NT, (kSegGroups + chains - 1) / chains);
        S.L = ceil_div(NT, want);
        S.NS = ceil_div(NT, S.L);
    } else {
        S.L = std::max(NT, 1);
        S.NS = 1;
    }
    return S;
}

size_t bwd_rrec_elems(int D);   // k_bwd.hip
// Whether the segment-parallel reverse pass of the backward (revseg.h) is
// built for these sizes: bf16 I/O, the dense layout.
inline bool rev_seg_built(int D, int dtype) { return dtype == DR_BF16 && (D == 64 || D == 128); }
// The reverse pass the backward takes: the segment-parallel one where it is
// built, unless DR_BWD_REV=slices selects the value-slice kernel.
inline bool rev_seg_selected() {
    const char* e = getenv("DR_BWD_REV");
    return !(e != nullptr && strcmp(e, "slices") == 0);
}

// The gradient kernel the backward takes for bf16 I/O: the one with bf16
// LDS operands (gradb.h, two workgroups per CU), unless DR_BWD_GRAD=f32lds
// selects the one with fp32 LDS operands (backward.h; fp32 I/O always).
inline bool gradb_selected() {
    const char* e = getenv("DR_BWD_GRAD");
    return !(e != nullptr && strcmp(e, "f32lds") == 0);
}

// The backward takes the bf16 prep (prepb.h) for bf16 I/O where the
// segment-parallel reverse pass is built and selected and the bf16 gradient
// kernel is selected; that prep also writes the forward state pass's
// records, so the forward's chunk kernel does not run.
inline bool bwd_fused_prep(int D, int dtype) {
    return dtype == DR_BF16 && rev_seg_built(D, dtype) && rev_seg_selected() && gradb_selected();
}

// states S_c [DK][DV], the exit adjoints dS'_c [DK][DV], Vnew_c and dVnew_c
// [C][DV] of every chunk, in the I/O dtype, each block 256-byte aligned.
// Where the segment-parallel reverse pass is built: its bf16 chunk operands
// (RevRec), and for more than one segment per chain (dense layout) the
// segment maps [Pi_r | N_r] [chains][NS][D][2D] and the segment exit
// adjoints E_r [chains][NS][D][D] (fp32); packed sequences take one segment
// per chain.  NS = 0 where the pass is not built.
struct BwdLayout {
    size_t prep, hs, dhs, vn, dvn, rec, rrec, xmap, ein, bytes;
    int NS, L;
};
// n = number of per-chunk entries (dense: B * H * ceil(T/C); packed:
// H * maxchunks); chains and NT (dense) size the reverse pass's segments
// (the forward's chunk records come before them: the forward state pass runs
// the forward's own two kernels over them)
inline BwdLayout bwd_layout_n(size_t n, int D, int dtype, long long chains = 0, int NT = 0) {
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t pf = D == 64 ? bwd_prep_floats(64) : bwd_prep_floats(128);
    BwdLayout L;
    L.prep = 0;
    L.hs = up(n * pf * 4);
    const size_t esz = dtype == DR_BF16 ? 2 : 4;
    L.dhs = L.hs + up(n * D * D * esz);
    L.vn = L.dhs + up(n * D * D * esz);
    L.dvn = L.vn + up(n * dr::kChunk * D * esz);
    L.rec = L.dvn + up(n * dr::kChunk * D * esz);
    L.rrec = L.xmap = L.ein = L.bytes = L.rec + up(n * record_bytes(D, dtype));
    L.NS = L.L = 0;
    if (rev_seg_built(D, dtype)) {
        L.xmap = L.ein = L.bytes = L.rrec + up(n * bwd_rrec_elems(D) * 2);
        L.NS = 1;
        L.L = std::max(NT, 1);
        if (chains > 0) {
            const SegPlan S = seg_plan(chains, NT);
            L.NS = S.NS;
            L.L = S.L;
            if (S.NS > 1) {
                L.ein = L.xmap + up((size_t)chains * S.NS * D * 2 * D * 4);
                L.bytes = L.ein + up((size_t)chains * S.NS * D * D * 4);
            }
        }
    }
    return L;
}
inline BwdLayout bwd_layout(int B, int T, int H, int D, int dtype) {
    const int NT = ceil_div(T, dr::kChunk);
    return bwd_layout_n((size_t)B * H * (size_t)NT, D, dtype, (long long)B * H, NT);
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
    // bf16 prep path (bwd_fused_prep): the forward state pass's problem; the
    // prep writes that pass's records, which then runs between the prep and
    // the reverse pass.  Null: the caller has run the forward state pass.
    const Problem* fwd;
};

template <int KIND, int D>
dr_status launch_prepb(const BwdArgs& a, float* prep, bf16* rrec, uint8_t* recs, hipStream_t st);
template <int KIND, int D>
dr_status launch_gradb(const BwdArgs& a, const float* prep, const bf16* hs, const bf16* dhs, const bf16* vn,
                       const bf16* dvn, hipStream_t st);

struct ProBwdLayout {
    size_t qh, kh, gh, bh, core, bytes;
};
// core: the bytes of what follows the prologue's part (the backward's own
// workspace, with the chunk table first for packed sequences)
inline ProBwdLayout probwd_layout(int kind, int B, int T, int H, int D, int dtype, size_t core) {
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

// ---- segment-parallel forward (seg.h) ------------------------------------
// The chunks of every (b, h) chain are grouped into NS segments of L chunks
// (seg_plan).  Workspace: q_eff [B*H*NT][C][D] (I/O dtype), [M | N]
// [B*H][NS][D][2D] fp32, S_in^T [B*H][NS][D][D] (I/O dtype), each 256-aligned.
struct SegLayout {
    int NS, L;
    size_t qeff, xend, sint, bytes;
};
// Whether the segment kernel is built for these sizes (fp32 at D = 128
// does not fit its LDS plan).
inline bool seg_built(int D, int dtype) { return dtype == DR_BF16 || D == 64; }
// The path the forward entry points take: the segment-parallel one where it
// is built, unless DR_FWD_PATH=records selects the record path.
inline bool seg_supported(int D, int dtype) {
    const char* e = getenv("DR_FWD_PATH");
    return !(e != nullptr && e[0] == 'r') && seg_built(D, dtype);
}
inline SegLayout seg_layout(int B, int T, int H, int D, int dtype) {
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    SegLayout S{1, 1, 0, 0, 0, 0};
    const int NT = ceil_div(T, dr::kChunk);
    const long long chains = (long long)B * H;
    const SegPlan P = seg_plan(chains, NT);
    S.NS = P.NS;
    S.L = P.L;
    const size_t esz = dtype == DR_BF16 ? 2 : 4;
    S.qeff = 0;
    S.xend = up((size_t)chains * NT * dr::kChunk * D * esz);
    S.sint = S.xend + up((size_t)chains * S.NS * D * 2 * D * 4);
    S.bytes = S.sint + up((size_t)chains * S.NS * D * D * esz);
    return S;
}
dr_status launch_seg_local(const Problem& p, const SegLayout& S, const float* h0, hipStream_t st);  // k_seg.hip
dr_status launch_seg_compose(const Problem& p, const SegLayout& S, float* hT, hipStream_t st);     // k_seg.hip
dr_status launch_seg_correct(const Problem& p, const SegLayout& S, hipStream_t st);                // k_seg.hip

// The whole forward (dense layout), as dr_forward runs it (deltarule.hip).
dr_status forward(int kind, const void* q, const void* k, const void* v, const float* g, const float* beta,
                  const float* h0, void* o, float* hT, int B, int T, int H, int Dk, int Dv, int C, int dtype,
                  void* ws, size_t ws_bytes, unsigned* flags, void* stream, const dr_prologue* pro = nullptr);

// ---- launchers (one kernel family per translation unit) -------------------
dr_status launch_intra(const Problem& p, int c0, int n, hipStream_t st);           // k_intra.hip
dr_status launch_intra_varlen(const Problem& p, hipStream_t st);                   // k_intra.hip
dr_status launch_inter(const Problem& p, const float* h0, float* hT, int c0, int n, hipStream_t st);  // k_inter.hip
// S_c and Vnew_c of every chunk, in the I/O type
dr_status launch_states(const Problem& p, const float* h0, void* hs, void* vn, hipStream_t st);       // k_inter.hip
dr_status launch_backward(int kind, const BwdArgs& a, int D, int dtype, hipStream_t st);              // k_bwd.hip
dr_status launch_decode(int kind, const DecodeArgs& a, bool use_pro, int D, int dtype, hipStream_t st);  // k_misc.hip
dr_status launch_prologue(bool backward, int kind, int D, int dtype, const void* q, const void* k, const float* g,
                          const float* beta, void* qh, void* kh, float* gh, float* bh, void* dq, void* dk, float* dg,
                          float* dbeta, float* dA_log, float* ddt, int B, int T, int H, const dr::Prologue& pro,
                          hipStream_t st, float* gpart = nullptr);                                      // k_misc.hip
dr_status launch_varlen_table(const int* cu_seqlens, int N, int T, int maxchunks, int4* table, int4* seqinfo,
                              int* total, unsigned* flags, hipStream_t st);                              // k_misc.hip
dr_status launch_copy_or_zero(float* dst, const float* src, size_t n, hipStream_t st);                  // k_misc.hip
// Debug aid: with the environment variable DR_POISON_WORKSPACE=1, fills the
// first `bytes` of a workspace with NaN before an entry point's launches, so
// that a read of workspace the call never wrote shows as NaN in the results.
dr_status poison_workspace(void* ws, size_t bytes, hipStream_t st);                                     // k_misc.hip

}  // namespace drh
