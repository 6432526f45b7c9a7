// deltarule.hip -- host side of the C ABI declared in include/deltarule.h:
// argument validation, workspace sizing and kernel dispatch for gfx950.
#include "host.h"

namespace drh {

dr_status forward(int kind, const void* q, const void* k, const void* v, const float* g,
                  const float* beta, const float* h0, void* o, float* hT, int B, int T, int H, int Dk,
                  int Dv, int C, int dtype, void* ws, size_t ws_bytes, unsigned* flags, void* stream,
                  const dr_prologue* pro) {
    dr_status s = validate(kind, q, k, v, g, beta, B, T, H, Dk, Dv, C, dtype, true);
    if (s != DR_OK) return s;
    dr::Prologue pr;
    bool use_pro;
    if ((s = resolve_prologue(kind, pro, &pr, &use_pro)) != DR_OK) return s;
    if (T > 0 && !o) return DR_ERR_INVALID_ARG;
    if (!aligned16(o) || !aligned16(h0) || !aligned16(hT) || !aligned16(ws)) return DR_ERR_INVALID_ARG;
    const size_t need = dr_workspace_bytes(kind, B, T, H, Dk, Dv, C, dtype);
    if (T > 0 && (ws == nullptr || ws_bytes < need)) return DR_ERR_WORKSPACE;
    if (T == 0 && hT == nullptr) return DR_OK;
    Problem p = make_problem(kind, q, k, v, g, beta, o, B, T, H, Dk, dtype, ws, flags, C);
    p.pro = pr;
    p.use_pro = use_pro;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (T == 0) return launch_inter(p, h0, hT, 0, 0, st);
    if ((s = poison_workspace(ws, need, st)) != DR_OK) return s;
    if (C == dr::kChunk && seg_supported(Dk, dtype)) {
        // segment-parallel path: local segment pass, entry-state
        // composition (and hT), then the output correction
        const SegLayout S = seg_layout(B, T, H, Dk, dtype);
        if ((s = launch_seg_local(p, S, h0, st)) != DR_OK) return s;
        if ((s = launch_seg_compose(p, S, hT, st)) != DR_OK) return s;
        return launch_seg_correct(p, S, st);
    }
    s = launch_intra(p, 0, p.NT, st);
    if (s != DR_OK) return s;
    return launch_inter(p, h0, hT, 0, p.NT, st);
}

// One stage of the segment-parallel forward (0: local pass, 1: composition,
// 2: correction), for callers that time or split the stages.
dr_status forward_stage(int stage, int kind, const void* q, const void* k, const void* v, const float* g,
                        const float* beta, const float* h0, void* o, float* hT, int B, int T, int H, int Dk, int Dv,
                        int C, int dtype, const dr_prologue* pro, void* ws, size_t ws_bytes, unsigned* flags,
                        void* stream) {
    if (stage < 0 || stage > 2) return DR_ERR_INVALID_ARG;
    dr_status s = validate(kind, stage == 0 ? q : nullptr, k, v, g, beta, B, T, H, Dk, Dv, C, dtype);
    if (stage == 0 && s != DR_OK) return s;
    if (stage != 0 && (kind < 0 || kind > 2 || B <= 0 || H <= 0 || T < 0 || (dtype != DR_F32 && dtype != DR_BF16)))
        return DR_ERR_INVALID_ARG;
    if (Dk != Dv || (Dk != 64 && Dk != 128) || C != dr::kChunk || !seg_built(Dk, dtype)) return DR_ERR_UNSUPPORTED;
    dr::Prologue pr;
    bool use_pro;
    if ((s = resolve_prologue(kind, pro, &pr, &use_pro)) != DR_OK) return s;
    if (T > 0 && stage != 1 && !o) return DR_ERR_INVALID_ARG;
    if (!aligned16(o) || !aligned16(h0) || !aligned16(hT) || !aligned16(ws)) return DR_ERR_INVALID_ARG;
    const SegLayout S = seg_layout(B, T, H, Dk, dtype);
    if (T == 0) return DR_OK;
    if (ws == nullptr || ws_bytes < S.bytes) return DR_ERR_WORKSPACE;
    Problem p = make_problem(kind, q, k, v, g, beta, o, B, T, H, Dk, dtype, ws, flags);
    p.pro = pr;
    p.use_pro = use_pro;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (stage == 0) {
        // (the later stages read what stage 0 wrote: only stage 0 poisons)
        if ((s = poison_workspace(ws, S.bytes, st)) != DR_OK) return s;
        return launch_seg_local(p, S, h0, st);
    }
    if (stage == 1) return launch_seg_compose(p, S, hT, st);
    return launch_seg_correct(p, S, st);
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
    if ((s = poison_workspace(ws, L.bytes, st)) != DR_OK) return s;
    s = launch_varlen_table(cu_seqlens, N, T, L.maxchunks, reinterpret_cast<int4*>(w + L.table),
                            reinterpret_cast<int4*>(w + L.seqinfo), reinterpret_cast<int*>(w + L.total), flags, st);
    if (s != DR_OK) return s;
    if (T > 0 && (s = launch_intra_varlen(p, st)) != DR_OK) return s;
    if (T == 0 && hT == nullptr) return DR_OK;
    // the state pass reads nseg, tokens and record slots from the descriptors
    return launch_inter(p, h0, hT, 0, 0, st);
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
    return launch_decode(kind, a, use_pro, Dk, dtype, st);
}

// ---- backward ------------------------------------------------------------------

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
        if ((s = launch_copy_or_zero(dA_log, nullptr, (size_t)H, st)) != DR_OK) return s;
        if (ddt_bias && (s = launch_copy_or_zero(ddt_bias, nullptr, (size_t)H, st)) != DR_OK) return s;
    }
    if (T == 0) {
        // no tokens: dh0 = dhT (or zero); nothing else to write
        if (!dh0) return DR_OK;
        const size_t n = (size_t)chains * H * Dk * Dv;
        return launch_copy_or_zero(dh0, dhT, n, st);
    }
    uint8_t* w = static_cast<uint8_t*>(workspace);
    if ((s = poison_workspace(w, use_pro ? PL.bytes : core_bytes, st)) != DR_OK) return s;
    uint8_t* rest = use_pro ? w + PL.core : w;     // [chunk table][core]
    dr::bw::Pack pk{nullptr, nullptr, nullptr, 0};
    if (packed) {
        // the chunk table of the packed forward, rebased to this workspace
        int4* table = reinterpret_cast<int4*>(rest);
        int4* seqinfo = reinterpret_cast<int4*>(rest + (V.seqinfo - V.table));
        int* total = reinterpret_cast<int*>(rest + (V.total - V.table));
        if ((s = launch_varlen_table(cu_seqlens, N, T, V.maxchunks, table, seqinfo, total, flags, st)) != DR_OK)
            return s;
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
    // forward state pass: the forward's chunk-parallel kernel writes the
    // chunk records, the state-pass kernel in STATES mode the entry state and
    // Vnew of every chunk (per-chunk arrays share the records' index, dense
    // and packed).  On the bf16 prep path the prep writes the records the
    // state pass reads, and both run inside launch_backward.
    const bool fused = bwd_fused_prep(Dk, dtype);
    Problem p = make_problem(kind, rq, rk, v, rg, rb, nullptr, chains, T, H, Dk, dtype, core + L.rec, nullptr);
    {
        if (packed) {
            p.table = pk.table;
            p.seqinfo = pk.seqinfo;
            p.total = pk.total;
            p.maxchunks = pk.maxchunks;
        }
        if (!fused) {
            s = packed ? launch_intra_varlen(p, st) : launch_intra(p, 0, p.NT, st);
            if (s != DR_OK) return s;
            s = launch_states(p, h0, core + L.hs, core + L.vn, st);
            if (s != DR_OK) return s;
        }
    }
    BwdArgs a{rq, rk, v, dout, rg, rb, h0, dhT, dq, dk, dv, dg, delta ? dbeta : nullptr, dh0,
              chains, T, H, ceil_div(T, dr::kChunk), core, L, pk, fused ? &p : nullptr};
    s = launch_backward(kind, a, Dk, dtype, st);
    if (s != DR_OK || !use_pro) return s;
    // gradients with respect to the raw inputs, in place; the gate
    // parameters' per-workgroup partial sums go to the prologue's q slot
    // (its last reader, the gradient kernel, has run) and are summed in a
    // fixed order
    return launch_prologue(true, kind, Dk, dtype, q, k, g, delta ? beta : nullptr, nullptr, nullptr, nullptr,
                           nullptr, dq, dk, dg, delta ? dbeta : nullptr, dA_log, ddt_bias, B, T, H, pr, st,
                           reinterpret_cast<float*>(w + PL.qh));
}

}  // namespace drh

using namespace drh;

extern "C" {

size_t dr_backward_workspace_bytes(int kind, int B, int T, int H, int Dk, int Dv, int C, int dtype) {
    if (kind < 0 || kind > 2 || B <= 0 || H <= 0 || T < 0 || !within_limit(B, T, H, Dk)) return 0;
    if (C != dr::kChunk || dr_record_bytes(Dk, Dv, C, dtype) == 0) return 0;
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
    if (kind < 0 || kind > 2 || B <= 0 || H <= 0 || T < 0 || !within_limit(B, T, H, Dk)) return 0;
    if (C != dr::kChunk || dr_record_bytes(Dk, Dv, C, dtype) == 0) return 0;
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
    if (kind < 0 || kind > 2 || N < 1 || H <= 0 || T < 0 || !within_limit(1, T, H, Dk)) return 0;
    if (((long long)ceil_div(T, dr::kChunk) + N) * H > 0x7fffffffLL) return 0;
    if (C != dr::kChunk || dr_record_bytes(Dk, Dv, C, dtype) == 0) return 0;
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
    if (Dk != Dv || (Dk != 64 && Dk != 128)) return 0;
    if (dtype != DR_F32 && dtype != DR_BF16) return 0;
    if (C != dr::kChunk && !(C == kChunk128 && chunk128_built(Dk, dtype))) return 0;
    return record_bytes(Dk, dtype, C);
}

size_t dr_record_workspace_bytes(int kind, int B, int T, int H, int Dk, int Dv, int C, int dtype) {
    if (kind < 0 || kind > 2 || B <= 0 || H <= 0 || T < 0 || !within_limit(B, T, H, Dk)) return 0;
    const size_t rec = dr_record_bytes(Dk, Dv, C, dtype);
    if (rec == 0) return 0;
    return (size_t)B * H * (size_t)ceil_div(T, C) * rec;
}

size_t dr_segment_workspace_bytes(int kind, int B, int T, int H, int Dk, int Dv, int C, int dtype) {
    const size_t rec = dr_record_workspace_bytes(kind, B, T, H, Dk, Dv, C, dtype);
    if (rec == 0 || C != dr::kChunk || !seg_built(Dk, dtype)) return 0;
    return T == 0 ? 0 : seg_layout(B, T, H, Dk, dtype).bytes;
}

size_t dr_workspace_bytes(int kind, int B, int T, int H, int Dk, int Dv, int C, int dtype) {
    const size_t rec = dr_record_workspace_bytes(kind, B, T, H, Dk, Dv, C, dtype);
    if (rec == 0 || T == 0) return rec;
    return C == dr::kChunk && seg_supported(Dk, dtype) ? seg_layout(B, T, H, Dk, dtype).bytes : rec;
}

dr_status dr_forward_stage(int stage, int kind, const void* q, const void* k, const void* v, const float* g,
                           const float* beta, const float* h0, void* o, float* hT, int B, int T, int H, int Dk,
                           int Dv, int C, int dtype, const dr_prologue* prologue, void* workspace,
                           size_t workspace_bytes, unsigned* flags, void* stream) {
    return forward_stage(stage, kind, q, k, v, g, kind == DR_KIND_DECAY_LA ? nullptr : beta, h0, o, hT, B, T, H, Dk,
                         Dv, C, dtype, prologue, workspace, workspace_bytes, flags, stream);
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
    dr_status s = validate(kind, q, k, v, g, beta, B, T, H, Dk, Dv, C, dtype, true);
    if (s != DR_OK) return s;
    if (!aligned16(workspace)) return DR_ERR_INVALID_ARG;
    if (T > 0 && (!workspace || workspace_bytes < dr_record_workspace_bytes(kind, B, T, H, Dk, Dv, C, dtype)))
        return DR_ERR_WORKSPACE;
    const Problem p = make_problem(kind, q, k, v, g, beta, nullptr, B, T, H, Dk, dtype, workspace, flags, C);
    if ((s = poison_workspace(workspace, dr_record_workspace_bytes(kind, B, T, H, Dk, Dv, C, dtype),
                              static_cast<hipStream_t>(stream))) != DR_OK)
        return s;
    return launch_intra(p, 0, p.NT, static_cast<hipStream_t>(stream));
}

dr_status dr_inter(int kind, const float* h0, void* o, float* hT, int B, int T, int H, int Dk, int Dv,
                   int C, int dtype, const void* workspace, size_t workspace_bytes, void* stream) {
    if (kind < 0 || kind > 2 || B <= 0 || H <= 0 || T < 0) return DR_ERR_INVALID_ARG;
    if (dtype != DR_F32 && dtype != DR_BF16) return DR_ERR_INVALID_ARG;
    if (Dk != Dv || (Dk != 64 && Dk != 128) || dr_record_bytes(Dk, Dv, C, dtype) == 0) return DR_ERR_UNSUPPORTED;
    if (T > 0 && !o) return DR_ERR_INVALID_ARG;
    if (!aligned16(o) || !aligned16(h0) || !aligned16(hT) || !aligned16(workspace)) return DR_ERR_INVALID_ARG;
    if (T > 0 && (!workspace || workspace_bytes < dr_record_workspace_bytes(kind, B, T, H, Dk, Dv, C, dtype)))
        return DR_ERR_WORKSPACE;
    if (T == 0 && hT == nullptr) return DR_OK;
    const Problem p = make_problem(kind, nullptr, nullptr, nullptr, nullptr, nullptr, o, B, T, H, Dk, dtype,
                                   const_cast<void*>(workspace), nullptr, C);
    return launch_inter(p, h0, hT, 0, p.NT, static_cast<hipStream_t>(stream));
}

size_t dr_workspace_bytes_varlen(int kind, int N, int T, int H, int Dk, int Dv, int C, int dtype) {
    if (kind < 0 || kind > 2 || N < 1 || H <= 0 || T < 0 || !within_limit(1, T, H, Dk)) return 0;
    if (((long long)ceil_div(T, dr::kChunk) + N) * H > 0x7fffffffLL) return 0;
    if (C != dr::kChunk || dr_record_bytes(Dk, Dv, C, dtype) == 0) return 0;
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

const char* dr_status_string(int status) {
    switch (status) {
        case DR_OK: return "ok";
        case DR_ERR_INVALID_ARG: return "invalid argument";
        case DR_ERR_UNSUPPORTED:
            return "unsupported size (Dk == Dv in {64, 128}; C == 64, or C == 128 for the dense forward "
                   "except fp32 at Dk = 128)";
        case DR_ERR_HIP: return "HIP launch failed";
        case DR_ERR_WORKSPACE: return "workspace missing or too small";
        case DR_ERR_SCRATCH_LIMIT:
            return "problem needs more workspace than the library's static scratch array holds "
                   "(dr_noalloc_scratch_bytes()); call dr_forward with a caller workspace";
        default: return "unknown status";
    }
}

int dr_abi_version(void) { return 7; }

}  // extern "C"

