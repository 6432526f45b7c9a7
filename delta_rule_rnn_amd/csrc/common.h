// common.h -- shared device helpers for the gfx950 kernels: element types,
// MFMA operand fragments, and the chunk-record layout.
//
// MFMA operand fragments.  All matrix products use 16x16 output tiles and a
// reduction block of 32.  For one tile, lane l (0..63) owns row/column
// (l % 16) and the 8 reduction slots (l / 16, j), j = 0..7.  A fragment holds
// those 8 operand values; which reduction index a slot stands for is chosen
// by whoever fills the fragment, the same way for both operands (a dot
// product does not depend on the order of its terms).  "Natural" fragments
// use index 8*(l/16) + j.
//
//   bf16: one v_mfma_f32_16x16x32_bf16 per fragment pair.
//   fp32: eight v_mfma_f32_16x16x4_f32; instruction j consumes slot j of
//         every lane, so the reduction runs over the same 32 indices.
//
// Accumulator layout (both instruction shapes): lane l holds the four rows
// 4*(l/16) + i, i = 0..3, of column l % 16.  Two accumulator tiles whose rows
// are assigned with prow() form a natural B fragment over their 32 rows,
// which lets a product's result feed the next product without leaving
// registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace dr {

typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kChunk = 64;     // C
constexpr int kThreads = 256;  // 4 waves per workgroup
constexpr float kLog2e = 1.4426950408889634f;

enum Kind { KIND_KDA = 0, KIND_GDN = 1, KIND_LA = 2 };

// N contiguous elements as one vector value (ext_vector_type: element
// access with [], one load or store).
template <typename T, int N> struct VecOf;
template <int N> struct VecOf<bf16, N> { typedef __bf16 type __attribute__((ext_vector_type(N))); };
template <int N> struct VecOf<float, N> { typedef float type __attribute__((ext_vector_type(N))); };

template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { float v[8]; };

// Sums over aligned lane groups without the LDS crossbar: within each row of
// 16 lanes four DPP moves (swap neighbours, swap pairs -- quad sums --,
// mirror within 8 lanes, mirror within 16), then shuffles across rows.  The
// result is left in every lane of the group.  All lanes must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_peer(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_peer<0xB1>(v);     // quad_perm [1,0,3,2]
    v += dpp_peer<0x4E>(v);     // quad_perm [2,3,0,1]
    v += dpp_peer<0x141>(v);    // row_half_mirror
    v += dpp_peer<0x140>(v);    // row_mirror
    return v;
}
// Across rows: v_permlane16_swap / v_permlane32_swap of a value with
// itself leave the two rows (halves) of each pair in the two results, so
// their sum is the pair's total in every lane, without the LDS crossbar.
// Logical id of workgroup bid of a grid of G: the hardware dispatches
// workgroup i to XCD i mod 8, so when G is a multiple of 8 each XCD gets the
// contiguous logical range [x G/8, (x+1) G/8) and consecutive logical ids
// share one XCD's L2; otherwise the identity.
__device__ __forceinline__ int xcd_logical(int bid, int G) {
    return (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
}

template <int N>
__device__ __forceinline__ float lane_group_sum(float v) {
    static_assert(N == 16 || N == 32 || N == 64, "lane group");
    v = row16_sum(v);
    if constexpr (N >= 32) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    if constexpr (N >= 64) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    return v;
}
// 1 / sqrt(x) for the L2 norms (x >= the norm epsilon > 0): the hardware
// reciprocal square root, within an ulp or two of the rounded quotient
__device__ __forceinline__ float inv_sqrt(float x) { return __builtin_amdgcn_rsqf(x); }

__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f(float x) { return x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }

// ---- input prologue -------------------------------------------------------
// Optional elementwise pre-pass on the raw inputs, applied where the kernels
// load them (page "Gated DeltaNet": the gate and write strength of the layer's
// forward, section "门控与 Head 映射", and the token loads of the recurrent
// kernel, "加载 Token 与写入系数"):
//   PRO_QK_L2NORM     q, k <- x / sqrt(sum_d x_d^2 + 1e-6)   (per token, head)
//   (always)          q <- q * scale, after the normalisation
//   PRO_BETA_SIGMOID  beta <- 1 / (1 + exp(-beta)),  PRO_BETA_X2: doubled
//   PRO_GATE          scalar gates: g <- -exp(A_log[h]) * softplus(g + dt_bias[h])
enum : unsigned { PRO_QK_L2NORM = 1u, PRO_BETA_SIGMOID = 2u, PRO_BETA_X2 = 4u, PRO_GATE = 8u };
constexpr float kNormEps = 1e-6f;

struct Prologue {
    unsigned ops;
    float scale;
    const float* A_log;     // [H], PRO_GATE only
    const float* dt_bias;   // [H] or null
};

// The prologue's per-head constants: ops, query scale, exp(A_log[h]) and
// dt_bias[h].
struct ProHead {
    unsigned ops;
    float scale, gA, gdt;
};
__device__ __forceinline__ ProHead pro_head(const Prologue& p, int h) {
    ProHead r{p.ops, p.scale, 1.f, 0.f};
    if (p.ops & PRO_GATE) {
        r.gA = expf(p.A_log[h]);
        r.gdt = p.dt_bias ? p.dt_bias[h] : 0.f;
    }
    return r;
}
// log(1 + e^x) without overflow: max(x, 0) + log1p(e^-|x|)
__device__ __forceinline__ float softplus_f(float x) { return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x))); }
__device__ __forceinline__ float pro_gate(const ProHead& p, float a) {
    return (p.ops & PRO_GATE) ? -p.gA * softplus_f(a + p.gdt) : a;
}
__device__ __forceinline__ float pro_beta(const ProHead& p, float b) {
    if (!(p.ops & PRO_BETA_SIGMOID)) return b;
    // 1 / (1 + e^-b) from the hardware exp2 and reciprocal (e^-b = inf for
    // very negative b gives 0, as it should)
    const float s = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-b * kLog2e));
    return (p.ops & PRO_BETA_X2) ? 2.f * s : s;
}

__device__ __forceinline__ void mma(f32x4& c, const Frag<bf16>& a, const Frag<bf16>& b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& c, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
}

// 8 contiguous elements (16-byte aligned for bf16, 32-byte for fp32).
__device__ __forceinline__ Frag<bf16> ld_frag(const bf16* p) {
    Frag<bf16> f;
    f.v = *reinterpret_cast<const bf16x8*>(p);
    return f;
}
__device__ __forceinline__ Frag<float> ld_frag(const float* p) {
    Frag<float> f;
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    return f;
}
__device__ __forceinline__ void st_frag(bf16* p, const Frag<bf16>& f) {
    *reinterpret_cast<bf16x8*>(p) = f.v;
}
__device__ __forceinline__ void st_frag(float* p, const Frag<float>& f) {
    reinterpret_cast<float4*>(p)[0] = make_float4(f.v[0], f.v[1], f.v[2], f.v[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(f.v[4], f.v[5], f.v[6], f.v[7]);
}
// Negated fragment (sign flips; exact in either type).
__device__ __forceinline__ Frag<bf16> frag_neg(const Frag<bf16>& f) {
    Frag<bf16> r;
    r.v = -f.v;
    return r;
}
__device__ __forceinline__ Frag<float> frag_neg(const Frag<float>& f) {
    Frag<float> r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r.v[j] = -f.v[j];
    return r;
}
// fragment slot access
__device__ __forceinline__ float frag_get(const Frag<bf16>& f, int j) { return (float)f.v[j]; }
__device__ __forceinline__ float frag_get(const Frag<float>& f, int j) { return f.v[j]; }
__device__ __forceinline__ void frag_set(Frag<bf16>& f, int j, float x) { f.v[j] = (bf16)x; }
__device__ __forceinline__ void frag_set(Frag<float>& f, int j, float x) { f.v[j] = x; }

// Two adjacent elements as one 4-byte (bf16) or 8-byte (fp32) access.
template <typename T> struct Pair;
template <> struct Pair<bf16> {
    typedef bf16x2 type;
    __device__ static type zero() { type z; z[0] = (bf16)0.f; z[1] = (bf16)0.f; return z; }
    __device__ static type make(float a, float b) { type z; z[0] = (bf16)a; z[1] = (bf16)b; return z; }
    __device__ static float lo(type x) { return (float)x[0]; }
    __device__ static float hi(type x) { return (float)x[1]; }
};
template <> struct Pair<float> {
    typedef float2 type;
    __device__ static type zero() { return make_float2(0.f, 0.f); }
    __device__ static type make(float a, float b) { return make_float2(a, b); }
    __device__ static float lo(type x) { return x.x; }
    __device__ static float hi(type x) { return x.y; }
};

// Four contiguous elements (8-byte aligned for bf16).
__device__ __forceinline__ void ld4(const bf16* p, float* out) {
    const bf16x4 x = *reinterpret_cast<const bf16x4*>(p);
    out[0] = (float)x[0]; out[1] = (float)x[1]; out[2] = (float)x[2]; out[3] = (float)x[3];
}
__device__ __forceinline__ void ld4(const float* p, float* out) {
    const float4 x = *reinterpret_cast<const float4*>(p);
    out[0] = x.x; out[1] = x.y; out[2] = x.z; out[3] = x.w;
}
__device__ __forceinline__ void st4(bf16* p, const float* in) {
    bf16x4 x;
    x[0] = (bf16)in[0]; x[1] = (bf16)in[1]; x[2] = (bf16)in[2]; x[3] = (bf16)in[3];
    *reinterpret_cast<bf16x4*>(p) = x;
}
__device__ __forceinline__ void st4(float* p, const float* in) {
    *reinterpret_cast<float4*>(p) = make_float4(in[0], in[1], in[2], in[3]);
}

// Four contiguous elements kept in their storage type, so that a prefetch
// does not force an early wait for the load (the conversion to float happens
// at the use).
template <typename T> struct Raw4;
template <> struct Raw4<bf16> {
    bf16x4 v;
    __device__ void load(const bf16* p) { v = *reinterpret_cast<const bf16x4*>(p); }
    __device__ float operator[](int i) const { return (float)v[i]; }
};
template <> struct Raw4<float> {
    float4 v;
    __device__ void load(const float* p) { v = *reinterpret_cast<const float4*>(p); }
    __device__ float operator[](int i) const { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }
};

// Copy of four contiguous elements as one access (8 bytes for bf16, 16 for
// fp32; both addresses aligned to that size).
__device__ __forceinline__ void cp4(bf16* dst, const bf16* src) {
    *reinterpret_cast<bf16x4*>(dst) = *reinterpret_cast<const bf16x4*>(src);
}
__device__ __forceinline__ void cp4(float* dst, const float* src) {
    *reinterpret_cast<float4*>(dst) = *reinterpret_cast<const float4*>(src);
}

// Streaming (non-temporal) global accesses for data touched once: the
// chunk-parallel kernel's inputs and its record (measured a few percent
// faster than ordinary accesses there; the state pass, whose slices share
// the record through L2, keeps ordinary loads).  V is a 4-, 8- or 16-byte
// type; the access goes through a same-size vector of 32-bit words.
template <int N> struct WordsOf;
template <> struct WordsOf<4> { typedef unsigned type; };
template <> struct WordsOf<8> { typedef unsigned type __attribute__((ext_vector_type(2))); };
template <> struct WordsOf<16> { typedef unsigned type __attribute__((ext_vector_type(4))); };
template <typename V>
__device__ __forceinline__ V ld_stream(const V* p) {
    using U = typename WordsOf<sizeof(V)>::type;
    return __builtin_bit_cast(V, __builtin_nontemporal_load(reinterpret_cast<const U*>(p)));
}
template <typename V>
__device__ __forceinline__ void st_stream(V* p, const V& v) {
    using U = typename WordsOf<sizeof(V)>::type;
    __builtin_nontemporal_store(__builtin_bit_cast(U, v), reinterpret_cast<U*>(p));
}
__device__ __forceinline__ void st_frag_stream(bf16* p, const Frag<bf16>& f) {
    st_stream(reinterpret_cast<bf16x8*>(p), f.v);
}
__device__ __forceinline__ void st_frag_stream(float* p, const Frag<float>& f) {
    st_stream(reinterpret_cast<float4*>(p), make_float4(f.v[0], f.v[1], f.v[2], f.v[3]));
    st_stream(reinterpret_cast<float4*>(p) + 1, make_float4(f.v[4], f.v[5], f.v[6], f.v[7]));
}
__device__ __forceinline__ void st4_stream(bf16* p, const float* in) {
    bf16x4 x;
    x[0] = (bf16)in[0]; x[1] = (bf16)in[1]; x[2] = (bf16)in[2]; x[3] = (bf16)in[3];
    st_stream(reinterpret_cast<bf16x4*>(p), x);
}
__device__ __forceinline__ void st4_stream(float* p, const float* in) {
    st_stream(reinterpret_cast<float4*>(p), make_float4(in[0], in[1], in[2], in[3]));
}

// Buffer stores: a resource over [base, base + bytes) whose out-of-range
// lanes the hardware drops, so a store needs no branch on the row index (a
// branch around a store leaves the compiler unable to count outstanding
// memory operations, and it then waits for all of them at the next use of a
// prefetched load).  The third resource word is the raw 32-bit data format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// four consecutive elements (8 bytes bf16, 16 bytes fp32) at byte offset off
__device__ __forceinline__ void buf_st4(__amdgpu_buffer_rsrc_t r, unsigned off, const bf16* /*type tag*/,
                                        const float* in) {
    bf16x4 x;
    x[0] = (bf16)in[0]; x[1] = (bf16)in[1]; x[2] = (bf16)in[2]; x[3] = (bf16)in[3];
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, x), r, (int)off, 0, 0);
}
__device__ __forceinline__ Raw4<bf16> buf_ld4(__amdgpu_buffer_rsrc_t r, unsigned off, const bf16* /*type tag*/) {
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    Raw4<bf16> x;
    x.v = __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
    return x;
}
__device__ __forceinline__ Raw4<float> buf_ld4(__amdgpu_buffer_rsrc_t r, unsigned off, const float* /*type tag*/) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    Raw4<float> x;
    x.v = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
    return x;
}
__device__ __forceinline__ void buf_st4(__amdgpu_buffer_rsrc_t r, unsigned off, const float* /*type tag*/,
                                        const float* in) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    typedef float f32x4_ __attribute__((ext_vector_type(4)));
    const f32x4_ x = {in[0], in[1], in[2], in[3]};
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, (int)off, 0, 0);
}

// Workgroup barrier that orders LDS traffic only: waits for this wave's LDS
// operations, then meets the other waves.  Unlike __syncthreads() it does not
// wait for outstanding global loads and stores, so prefetches and record
// stores stay in flight across it.  Every barrier in these kernels exchanges
// LDS data only; global results are consumed by later kernels.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Row of a 32-row block held by row r (0..15) of its first (half = 0) or
// second (half = 1) 16-row tile, chosen so that the pair's accumulators form a
// natural B fragment: lane group q holds rows 8q..8q+3 (half 0) and
// 8q+4..8q+7 (half 1).
__device__ __forceinline__ int prow(int half, int r) { return 8 * (r >> 2) + 4 * half + (r & 3); }

// Chunk position held by row r of the state pass's wave w (w = 0..3): wave w
// owns the 16 positions of 32-block w/2 selected by prow(w%2, .).
__device__ __forceinline__ int pw(int w, int r) { return 32 * (w >> 1) + prow(w & 1, r); }

// The backward's per-chunk state arrays ([rows][D] matrices: the entry
// states S_c, Vnew_c and their adjoints) are stored slice-major: 32-column
// slices, each a contiguous [rows][32] block, so that a kernel reading one
// value slice takes whole cache lines.  Element (row, col) of a [rows][D]
// array:
__host__ __device__ constexpr size_t slc(int row, int col, int rows) {
    return (size_t)(col >> 5) * rows * 32 + (size_t)row * 32 + (col & 31);
}

// ---------------------------------------------------------------------------
// Chunk record: the operands the sequential pass streams, one record per
// (b, h, chunk).  Offsets in elements of the I/O type T except phi (float).
//
// Every block is stored in MFMA fragment order for the state pass, so one
// wave-wide load of 8 elements per lane reads a contiguous 64*8-element run
// (lane l, element j; NKB = DK/32; NW = C/16 position groups of 16; pw() and
// prow() above, with pw(w, r) = 32(w/2) + prow(w%2, r) for any w < NW):
//   W, QT  [w NW][kb NKB][l 64][j 8]     = X[pw(w, l%16)][32kb + 8(l/16) + j]
//   KBT    [w NKB][h 2][kb C/32][l][j 8] = Kbar[32kb + 8(l/16) + j][32w + prow(h, l%16)]
//   AQK    [w NW][kb C/32][l][j 8]       = Aqk[pw(w, l%16)][32kb + 8(l/16) + j]
//   UT     [t DV/16][w NW][l][i 4]       = U[32(w/2) + 8(l/16) + 4(w%2) + i][16t + l%16]
//   PHI    [DK] float
// C is 64, or 128 for the sub-chunked records of 128-token chunks.
// ---------------------------------------------------------------------------
template <typename T, int DK, int DV, int CH = kChunk>
struct Rec {
    static constexpr int C = CH;
    static constexpr size_t W = 0;                       // C*DK
    static constexpr size_t QT = W + (size_t)C * DK;     // C*DK
    static constexpr size_t KBT = QT + (size_t)C * DK;   // DK*C
    static constexpr size_t AQK = KBT + (size_t)DK * C;  // C*C
    static constexpr size_t UT = AQK + (size_t)C * C;    // DV*C
    static constexpr size_t END = UT + (size_t)DV * C;
    static constexpr size_t PHI_BYTE = END * sizeof(T);      // [DK] float
    static constexpr size_t BYTES = ((PHI_BYTE + DK * sizeof(float)) + 255) / 256 * 256;
};

// Runs step(i, ops, guard) for i = 0..n-1 with the operands of step i loaded
// one step ahead into a pair of register buffers.  Every load inside the
// steady-state loop is unconditional (the prefetch index is clamped to the
// last chunk) and only the last step gets the Tail guard tag, so the compiler
// can keep prefetches in flight across steps instead of draining the memory
// counter at control-flow joins.
template <typename Ops, typename Load, typename Step>
__device__ __forceinline__ void prefetch_pair(int n, Load&& load, Step&& step)
{
    using Full = std::integral_constant<bool, false>;
    using Tail = std::integral_constant<bool, true>;
    if (n <= 0) return;
    const int last = n - 1;
    auto cl = [&](int c) { return c < last ? c : last; };
    int c = 0;
    Ops b0, b1;
    load(b0, 0);
    for (; c + 2 <= last; c += 2) {
        load(b1, cl(c + 1)); step(c, b0, Full{});
        load(b0, cl(c + 2)); step(c + 1, b1, Full{});
    }
    if (c == last) {
        step(c, b0, Tail{});
    } else {
        load(b1, c + 1);
        step(c, b0, Full{});
        step(c + 1, b1, Tail{});
    }
}

// Packed-sequence chunk table as the backward kernels take it (written by
// varlen_table_kernel): table[slot] = {sequence, first token, valid rows, -},
// seqinfo[n] = {first slot, chunks, first token, tokens}, *total slots.
namespace bw {
struct Pack {
    const int4* table;
    const int4* seqinfo;
    const int* total;
    int maxchunks;
};
}  // namespace bw

}  // namespace dr
