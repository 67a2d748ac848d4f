// zsp_kernels.hip -- HIP kernels of libzsp for gfx950 (MI355X, CDNA4).
//
// Every kernel here is a stream over HBM with a few fp32 operations per
// byte: no contraction, so no MFMA. LDS holds data only in the range
// gather's span form (many short parameters), which realigns each rank's
// run of a span through it. Design points, each chosen by measurement on
// MI355X:
//
//  * One wavefront per workgroup, owning one 512-element tile of the index
//    space, or one half of it (shard launches of up to 16 ranks over long
//    pieces), or one span of two tiles (span gather). Small workgroups keep
//    more, shorter-lived waves in flight, which measured faster than
//    256-thread groups for these streams.
//  * Large shard launches cap the workgroups resident per CU (7 to 16,
//    through the LDS each reserves): fewer waves, each with 4-12 KiB of
//    loads in flight, let HBM serve the mixed read/write streams faster
//    than a full CU does. See shard_lds_pad.
//  * Lane l owns two 4-element quads of the tile, at 4*l and 256 + 4*l, so
//    every load and store instruction of the wave covers one contiguous run
//    (1 KiB for fp32 state, 512 B for bf16). Giving a lane 8 contiguous
//    elements instead makes each fp32 instruction touch every other 16 bytes
//    of a 2 KiB run, which measured ~5% slower.
//  * Every stream is touched once per launch, so global loads and stores
//    carry the non-temporal hint; that measured a further ~5%. The
//    exceptions are launches over short pieces (many parameters of a few
//    thousand elements): their gradient or source loads are ordinary ones,
//    and their tiles go to the XCDs in runs, so a cache line two
//    neighbouring tiles share is fetched once (xcd_run_tile).
//  * The optimizer state of the wave's quads is loaded before the gradients
//    so the state's latency overlaps the rank loop.
//  * The tile's parameter comes from a per-tile table: wave-uniform, so the
//    common single-parameter tile costs two scalar loads (a tile-aligned
//    gather reads one per-tile record instead: its piece's delta over long
//    pieces, the split and both deltas of at most two short pieces). A
//    launch can span any number of parameters -- thousands of small ones as
//    easily as one large one -- with no per-parameter launch.
//  * Gradient and parameter sources may sit at any 2-byte offset relative to
//    the quads (each parameter is padded on its own, so slices do not line
//    up). gfx9 global memory serves unaligned vector loads, so the fast path
//    stays one vector load per quad. Quads that cross a parameter or pad
//    boundary keep vector state access and mask per element (reading both
//    pieces' gradient vectors when they cross into the next piece); only
//    quads meeting three pieces or the edge of a launch's range go element
//    by element.
//  * The reduce over N_d ranks keeps each lane's 4 or 8 sums in registers
//    and adds rank r's values strictly after rank r-1's (fixed order,
//    bit-exact); the ranks are loaded 8 at a time (16 at a time for more
//    than 16 ranks), so 8 to 32 loads per lane are in flight.
//  * Floating point: built with -ffp-contract=off; division and square root
//    are the default correctly rounded expansions; bf16 narrowing is the
//    hardware round-to-nearest-even convert (v_cvt_pk_bf16_f32).
#include <hip/hip_runtime.h>

#include <atomic>
#include <type_traits>

#include "zsp_internal.hpp"

namespace zsp {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// Same vectors at the alignment of their element type: sources that start at
// any element offset.
typedef uint32_t u32x2_a2 __attribute__((ext_vector_type(2), aligned(2)));
typedef uint32_t u32x4_a2 __attribute__((ext_vector_type(4), aligned(2)));
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kQuad = 4;
constexpr int kHalf = kTile / 2;  // second quad of a lane is this far on

// Non-temporal accesses. One named function per pointer type rather than a
// template or overloads: both would lose the reduced alignment of the
// *_a2 / *_a4 typedefs (they are the same type as the aligned vector).
__device__ __forceinline__ u32x2 ldnt_x2_a2(const u32x2_a2* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ u32x4 ldnt_x4_a2(const u32x4_a2* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ u32x4 ld_x4_a2(const u32x4_a2* p) { return *p; }
__device__ __forceinline__ u32x4 ldnt_x4_a4(const u32x4_a4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ f32x4 ldnt_f32x4(const f32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void stnt(f32x4* p, f32x4 v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void stnt(u32x2* p, u32x2 v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void stnt(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    bf16x2 r;
    r.x = static_cast<__bf16>(a);
    r.y = static_cast<__bf16>(b);
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint16_t to_bf16(float a) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(a));
}

// 4 consecutive elements of a bf16 or fp32 source at base[off], any element
// offset; non-temporal unless TG (an ordinary, L2-allocating load).
template <typename GT, bool TG = false>
__device__ __forceinline__ void load4(const GT* base, uint32_t off, float (&x)[4]) {
    if constexpr (std::is_same<GT, uint16_t>::value) {
        const u32x2_a2* p = reinterpret_cast<const u32x2_a2*>(base + off);
        u32x2 u;
        if constexpr (TG) u = *p;
        else u = ldnt_x2_a2(p);
        x[0] = bf_lo(u.x); x[1] = bf_hi(u.x);
        x[2] = bf_lo(u.y); x[3] = bf_hi(u.y);
    } else {
        const u32x4_a4* p = reinterpret_cast<const u32x4_a4*>(base + off);
        u32x4 u;
        if constexpr (TG) u = *p;
        else u = ldnt_x4_a4(p);
        x[0] = __uint_as_float(u.x); x[1] = __uint_as_float(u.y);
        x[2] = __uint_as_float(u.z); x[3] = __uint_as_float(u.w);
    }
}

template <typename GT>
__device__ __forceinline__ float load1(const void* base, int64_t idx) {
    if constexpr (std::is_same<GT, uint16_t>::value)
        return __uint_as_float(uint32_t(static_cast<const uint16_t*>(base)[idx]) << 16);
    else
        return static_cast<const float*>(base)[idx];
}

__device__ __forceinline__ void ld_f32x4(const float* p, float (&x)[4]) {
    const f32x4 v = ldnt_f32x4(reinterpret_cast<const f32x4*>(p));
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}

__device__ __forceinline__ void st_f32x4(float* p, const float (&x)[4]) {
    stnt(reinterpret_cast<f32x4*>(p), f32x4{x[0], x[1], x[2], x[3]});
}

__device__ __forceinline__ void st_bf16x4(uint16_t* p, const float (&x)[4]) {
    stnt(reinterpret_cast<u32x2*>(p), u32x2{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])});
}

// Adam (Kingma & Ba, Algorithm 1) on one element, one fp32 rounding per
// operation in this order; must not be contracted into FMAs.
__device__ __forceinline__ void adam1(float& p, float& m, float& v, float g,
                                      const AdamScalars& h) {
    const float mn = h.b1 * m + h.omb1 * g;
    const float vn = h.b2 * v + h.omb2 * (g * g);
    const float mh = mn / h.bc1;
    const float vh = vn / h.bc2;
    const float den = __builtin_sqrtf(vh) + h.eps;
    const float upd = (h.lr * mh) / den;
    p = p - upd;
    m = mn;
    v = vn;
}

template <int CAP>
struct ShardArgs {
    const int64_t* e0;
    const PieceInfo* info;
    const int32_t* tile;
    int64_t tile_first, tile_end, e_begin, e_end;
    int64_t glen;  // elements of each gradient buffer
    float* master;
    float* m;
    float* v;
    uint16_t* work;
    float* acc;
    const void* src;
    AdamScalars hp;
    int32_t nd, shard_layout;
    const void* grads[CAP];
};

// Rank r's gradient pointer, read straight from the kernel-argument segment
// (scalar load; r is wave-uniform). Indexing the by-value argument's array
// through a reference can make the compiler copy the whole argument into
// per-lane scratch memory; addressing the segment directly never does. The
// argument struct is the kernel's only explicit argument, so it starts at
// offset 0 of the segment.
template <int CAP>
__device__ __forceinline__ const void* grad_ptr(int r) {
    const char* seg = (const char*)__builtin_amdgcn_kernarg_segment_ptr();
    return reinterpret_cast<const void* const*>(seg + offsetof(ShardArgs<CAP>, grads))[r];
}

constexpr bool uses_grads(int op) {
    return op == OP_REDUCE_SET || op == OP_REDUCE_ACC || op == OP_FUSED || op == OP_FUSED_ACC;
}
constexpr bool reads_acc(int op) {
    return op == OP_REDUCE_ACC || op == OP_FUSED_ACC || op == OP_ADAM;
}
constexpr bool is_reduce(int op) { return op == OP_REDUCE_SET || op == OP_REDUCE_ACC; }
constexpr bool is_adam(int op) { return op == OP_FUSED || op == OP_FUSED_ACC || op == OP_ADAM; }

// Sum over the N_d ranks, in rank order, of NQ quads per lane; quad h of
// rank r starts at element base[h] + off[h] of grads[r]. When base[] is
// wave-uniform the address is a scalar base plus a 32-bit lane offset. A
// batch's loads are all issued before its adds. TG: ordinary loads (see
// shard_kernel).
template <typename GT, int CAP, int NQ, bool TG>
__device__ __forceinline__ void reduce_quads(const ShardArgs<CAP>& a, const int64_t (&base)[NQ],
                                             const uint32_t (&off)[NQ],
                                             float (&g)[NQ][kQuad]) {
    // Ranks per batch of loads: 16 for the many-rank instantiations, whose
    // bytes are mostly gradient reads (+4.7% at N_d = 64 over 8, at 111
    // VGPRs; 32 spills), 8 otherwise (better at N_d = 8 and 16).
    constexpr int B = CAP >= 64 ? 16 : 8;
    const int nd = a.nd;
    int r0 = 0;
    for (; r0 + B <= nd; r0 += B) {
        float x[B][NQ][kQuad];
#pragma unroll
        for (int q = 0; q < B; ++q)
#pragma unroll
            for (int h = 0; h < NQ; ++h)
                load4<GT, TG>(static_cast<const GT*>(grad_ptr<CAP>(r0 + q)) + base[h], off[h],
                              x[q][h]);
#pragma unroll
        for (int q = 0; q < B; ++q) {
            const bool first = (r0 + q) == 0;
#pragma unroll
            for (int h = 0; h < NQ; ++h)
#pragma unroll
                for (int k = 0; k < kQuad; ++k) g[h][k] = first ? x[q][h][k] : g[h][k] + x[q][h][k];
        }
    }
    if (r0 < nd) {
        // Last, partial batch: every load is issued (ranks past the end
        // re-read the last rank, a cache hit) so none waits on a branch.
        float x[B][NQ][kQuad];
#pragma unroll
        for (int q = 0; q < B; ++q)
#pragma unroll
            for (int h = 0; h < NQ; ++h)
                load4<GT, TG>(static_cast<const GT*>(grad_ptr<CAP>(min(r0 + q, nd - 1))) + base[h],
                          off[h], x[q][h]);
#pragma unroll
        for (int q = 0; q < B; ++q) {
            if (r0 + q < nd) {
                const bool first = (r0 + q) == 0;
#pragma unroll
                for (int h = 0; h < NQ; ++h)
#pragma unroll
                    for (int k = 0; k < kQuad; ++k)
                        g[h][k] = first ? x[q][h][k] : g[h][k] + x[q][h][k];
            }
        }
    }
}

// One element's rank-order sum (per-element path); 8 ranks' loads are issued
// before their adds.
template <typename GT, int CAP>
__device__ __forceinline__ float reduce1(const ShardArgs<CAP>& a, int64_t sidx) {
    float g = 0.0f;
    for (int r0 = 0; r0 < a.nd; r0 += 8) {
        float x[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) x[q] = load1<GT>(grad_ptr<CAP>(min(r0 + q, a.nd - 1)), sidx);
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (r0 + q < a.nd) g = (r0 + q == 0) ? x[q] : g + x[q];
    }
    return g;
}

// NQ quads, each 4 in-range, non-pad elements of one piece. Quad h covers
// state elements Eb[h] + off[h] ...; its gradient starts at element
// gb[h] + off[h] of each rank's buffer and its flat parameter at
// ib[h] + off[h]. Eb[h] + off[h] is a multiple of 4, so every state access is
// an aligned 16-byte vector. With wave-uniform Eb/gb/ib (a tile inside one
// piece) every address is a scalar base plus the lane's 32-bit offset.
// Only quads with ok[h] store; the others' loads (in-range state, and
// whatever gb[h] names) are issued with the rest and their results dropped.
template <int OP, typename GT, int CAP, int NQ, bool TG>
__device__ __forceinline__ void quads_fast(const ShardArgs<CAP>& a, const int64_t (&Eb)[NQ],
                                           const int64_t (&gb)[NQ], const int64_t (&ib)[NQ],
                                           const uint32_t (&off)[NQ], const bool (&ok)[NQ]) {
    if constexpr (OP == OP_COPYIN) {
#pragma unroll
        for (int h = 0; h < NQ; ++h) {
            const GT* src = static_cast<const GT*>(a.src) + ib[h];
            float x[kQuad];
            load4<GT>(src, off[h], x);
            st_f32x4(a.master + Eb[h] + off[h], x);
            if constexpr (std::is_same<GT, uint16_t>::value) {
                const u32x2 raw = ldnt_x2_a2(reinterpret_cast<const u32x2_a2*>(src + off[h]));
                stnt(reinterpret_cast<u32x2*>(a.work + Eb[h] + off[h]), raw);
            } else {
                st_bf16x4(a.work + Eb[h] + off[h], x);
            }
            const float z[kQuad] = {0.0f, 0.0f, 0.0f, 0.0f};
            st_f32x4(a.m + Eb[h] + off[h], z);
            st_f32x4(a.v + Eb[h] + off[h], z);
        }
    } else {
        float p[NQ][kQuad], m[NQ][kQuad], v[NQ][kQuad], c[NQ][kQuad], g[NQ][kQuad];
        if constexpr (is_adam(OP)) {
#pragma unroll
            for (int h = 0; h < NQ; ++h) {
                ld_f32x4(a.master + Eb[h] + off[h], p[h]);
                ld_f32x4(a.m + Eb[h] + off[h], m[h]);
                ld_f32x4(a.v + Eb[h] + off[h], v[h]);
            }
        }
        if constexpr (reads_acc(OP)) {
#pragma unroll
            for (int h = 0; h < NQ; ++h) ld_f32x4(a.acc + Eb[h] + off[h], c[h]);
        }
        if constexpr (uses_grads(OP)) {
            reduce_quads<GT, CAP, NQ, TG>(a, gb, off, g);
        }
#pragma unroll
        for (int h = 0; h < NQ; ++h) {
#pragma unroll
            for (int k = 0; k < kQuad; ++k) {
                if constexpr (OP == OP_ADAM) g[h][k] = c[h][k];
                else if constexpr (reads_acc(OP)) g[h][k] = c[h][k] + g[h][k];
            }
        }
        if constexpr (is_reduce(OP)) {
#pragma unroll
            for (int h = 0; h < NQ; ++h)
                if (ok[h]) st_f32x4(a.acc + Eb[h] + off[h], g[h]);
        } else {
#pragma unroll
            for (int h = 0; h < NQ; ++h) {
#pragma unroll
                for (int k = 0; k < kQuad; ++k) adam1(p[h][k], m[h][k], v[h][k], g[h][k], a.hp);
                if (ok[h]) {
                    st_f32x4(a.master + Eb[h] + off[h], p[h]);
                    st_f32x4(a.m + Eb[h] + off[h], m[h]);
                    st_f32x4(a.v + Eb[h] + off[h], v[h]);
                    st_bf16x4(a.work + Eb[h] + off[h], p[h]);
                }
            }
        }
    }
}

// One quad of in-range pad elements.
template <int OP, int CAP>
__device__ __forceinline__ void quad_pad(const ShardArgs<CAP>& a, int64_t E) {
    const float z[kQuad] = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (OP == OP_COPYIN) {
        st_f32x4(a.master + E, z);
        st_f32x4(a.m + E, z);
        st_f32x4(a.v + E, z);
        stnt(reinterpret_cast<u32x2*>(a.work + E), u32x2{0u, 0u});
    } else if constexpr (is_reduce(OP)) {
        st_f32x4(a.acc + E, z);
    }
}

template <int OP, typename GT, int CAP>
__device__ __forceinline__ void elem_op(const ShardArgs<CAP>& a, int64_t e, bool valid,
                                        const PieceInfo& pi) {
    if constexpr (OP == OP_COPYIN) {
        float x = 0.0f;
        uint16_t w = 0;
        if (valid) {
            const int64_t s = e + pi.idelta;
            x = load1<GT>(a.src, s);
            if constexpr (std::is_same<GT, uint16_t>::value)
                w = static_cast<const uint16_t*>(a.src)[s];
            else
                w = to_bf16(x);
        }
        a.master[e] = x;
        a.work[e] = w;
        a.m[e] = 0.0f;
        a.v[e] = 0.0f;
    } else if constexpr (is_reduce(OP)) {
        float r = 0.0f;
        if (valid) {
            r = reduce1<GT>(a, a.shard_layout ? e : e + pi.gdelta);
            if constexpr (OP == OP_REDUCE_ACC) r = a.acc[e] + r;
        }
        a.acc[e] = r;
    } else {
        if (!valid) return;
        float g;
        if constexpr (OP == OP_ADAM) {
            g = a.acc[e];
        } else {
            g = reduce1<GT>(a, a.shard_layout ? e : e + pi.gdelta);
            if constexpr (OP == OP_FUSED_ACC) g = a.acc[e] + g;
        }
        float p = a.master[e], m = a.m[e], v = a.v[e];
        adam1(p, m, v, g, a.hp);
        a.master[e] = p;
        a.m[e] = m;
        a.v[e] = v;
        a.work[e] = to_bf16(p);
    }
}

// OUT: no element in range. FAST: 4 real elements of one piece, in range.
// PAD: 4 pad elements of one piece, in range. MIXED: in range, crossing a
// piece or pad boundary. SLOW: crossing the call's range boundary.
enum QuadKind : int { Q_OUT = 0, Q_FAST = 1, Q_PAD = 2, Q_SLOW = 3, Q_MIXED = 4 };

// Pieces of one tile, indexed from 0 (entry i is piece lo + i of the
// table): either the global table offset by lo, or a copy staged in LDS.
// Up to this many are staged; a tile holding more (parameters of a few
// elements per rank) searches the global table.
constexpr int kStage = 128;
// Tiles with fewer pieces than this search the global table directly (one or
// two cached loads); staging pays off only for more.
constexpr int kStageMin = 2;

// Local index of the piece holding element E among the n pieces whose starts
// are e0[0..n).
__device__ __forceinline__ int find_local(const int64_t* e0, int n, int64_t E) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (e0[mid] <= E) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

template <int CAP>
__device__ __forceinline__ int classify(const ShardArgs<CAP>& a, int64_t E, const PieceInfo& pi) {
    if (E >= a.e_end || E + kQuad <= a.e_begin) return Q_OUT;
    const bool inside = E >= a.e_begin && E + kQuad <= a.e_end;
    if (!inside) return Q_SLOW;
    if (E + kQuad <= pi.vend) return Q_FAST;
    if (E >= pi.vend && E + kQuad <= pi.end) return Q_PAD;
    return Q_MIXED;
}

// A quad inside the call's range whose elements are not all real elements
// of one piece: it crosses a piece boundary or the pad boundary. The state is
// still one aligned 16-byte vector per stream; each element finds its piece,
// all ranks' gradient loads of the 4 elements are issued together, and pad
// elements keep their state bit for bit (they are loaded and stored back).
template <int OP, typename GT, int CAP>
__device__ __forceinline__ void quad_mixed(const ShardArgs<CAP>& a, int64_t E, int p, PieceInfo pi,
                                           const PieceInfo* info) {
    // Pad elements read element 0 of the same buffer instead (always valid
    // memory, value discarded), so that every load is issued unconditionally:
    // loads under a per-lane condition each get their own wait.
    bool valid[kQuad];
    int64_t gs[kQuad], is[kQuad];
#pragma unroll
    for (int k = 0; k < kQuad; ++k) {
        const int64_t e = E + k;
        while (e >= pi.end) pi = info[++p];
        valid[k] = e < pi.vend;
        gs[k] = valid[k] ? (a.shard_layout ? e : e + pi.gdelta) : 0;
        is[k] = valid[k] ? e + pi.idelta : 0;
    }
    if constexpr (OP == OP_COPYIN) {
        float x[kQuad];
        uint32_t w[kQuad];
#pragma unroll
        for (int k = 0; k < kQuad; ++k) {
            const float xk = load1<GT>(a.src, is[k]);
            x[k] = valid[k] ? xk : 0.0f;
            if constexpr (std::is_same<GT, uint16_t>::value)
                w[k] = valid[k] ? (__float_as_uint(xk) >> 16) : 0u;
            else
                w[k] = to_bf16(x[k]);
        }
        st_f32x4(a.master + E, x);
        stnt(reinterpret_cast<u32x2*>(a.work + E), u32x2{w[0] | (w[1] << 16), w[2] | (w[3] << 16)});
        const float z[kQuad] = {0.0f, 0.0f, 0.0f, 0.0f};
        st_f32x4(a.m + E, z);
        st_f32x4(a.v + E, z);
    } else {
        float p4[kQuad], m4[kQuad], v4[kQuad], c4[kQuad], g[kQuad];
        u32x2 w_old{0u, 0u};
        if constexpr (is_adam(OP)) {
            ld_f32x4(a.master + E, p4);
            ld_f32x4(a.m + E, m4);
            ld_f32x4(a.v + E, v4);
            w_old = *reinterpret_cast<const u32x2*>(a.work + E);
        }
        if constexpr (reads_acc(OP)) ld_f32x4(a.acc + E, c4);
        if constexpr (uses_grads(OP)) {
#pragma unroll
            for (int k = 0; k < kQuad; ++k) g[k] = 0.0f;
            for (int r0 = 0; r0 < a.nd; r0 += 8) {
                float x[8][kQuad];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const void* gp = grad_ptr<CAP>(min(r0 + q, a.nd - 1));
#pragma unroll
                    for (int k = 0; k < kQuad; ++k) {
                        const float xk = load1<GT>(gp, gs[k]);
                        x[q][k] = valid[k] ? xk : 0.0f;
                    }
                }
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    if (r0 + q < a.nd)
#pragma unroll
                        for (int k = 0; k < kQuad; ++k)
                            g[k] = (r0 + q == 0) ? x[q][k] : g[k] + x[q][k];
            }
        }
#pragma unroll
        for (int k = 0; k < kQuad; ++k) {
            if constexpr (OP == OP_ADAM) g[k] = c4[k];
            else if constexpr (reads_acc(OP)) g[k] = c4[k] + g[k];
        }
        if constexpr (is_reduce(OP)) {
            float r[kQuad];
#pragma unroll
            for (int k = 0; k < kQuad; ++k) r[k] = valid[k] ? g[k] : 0.0f;
            st_f32x4(a.acc + E, r);
        } else {
#pragma unroll
            for (int k = 0; k < kQuad; ++k) {
                float pk = p4[k], mk = m4[k], vk = v4[k];
                adam1(pk, mk, vk, g[k], a.hp);
                if (valid[k]) {
                    p4[k] = pk;
                    m4[k] = mk;
                    v4[k] = vk;
                }
            }
            const uint32_t wn0 = pack_bf16(p4[0], p4[1]), wn1 = pack_bf16(p4[2], p4[3]);
            const uint32_t lo0 = valid[0] ? (wn0 & 0xffffu) : (w_old.x & 0xffffu);
            const uint32_t hi0 = valid[1] ? (wn0 & 0xffff0000u) : (w_old.x & 0xffff0000u);
            const uint32_t lo1 = valid[2] ? (wn1 & 0xffffu) : (w_old.y & 0xffffu);
            const uint32_t hi1 = valid[3] ? (wn1 & 0xffff0000u) : (w_old.y & 0xffff0000u);
            st_f32x4(a.master + E, p4);
            st_f32x4(a.m + E, m4);
            st_f32x4(a.v + E, v4);
            stnt(reinterpret_cast<u32x2*>(a.work + E), u32x2{lo0 | hi0, lo1 | hi1});
        }
    }
}

// A quad of a multi-piece tile lying wholly inside the call's range. Its
// elements before the end of the first element's piece read their gradient
// from gA on, the rest (the next piece) from gB on; valid has bit k set when
// element k is a real (non-pad) element. slow: the quad meets three pieces,
// or a read at gA or gB would leave the gradient buffers (possible only at
// their ends); quad_mixed then takes it.
struct QuadPlan {
    int64_t gA, gB;
    uint32_t valid, selB;
    bool slow;
};

// Bits of the elements k < x of a quad.
__device__ __forceinline__ uint32_t quad_below(int64_t x) {
    return x <= 0 ? 0u : x >= kQuad ? 0xfu : (1u << uint32_t(x)) - 1u;
}

template <int OP, int CAP>
__device__ __forceinline__ QuadPlan plan_quad(const ShardArgs<CAP>& a, int64_t E, int p,
                                              const PieceInfo& pi, const PieceInfo* info) {
    QuadPlan q{0, 0, 0u, 0u, false};
    const int64_t ga = a.shard_layout ? E : E + pi.gdelta;
    if (E + kQuad <= pi.end) {
        // One piece (its pad slots, if the quad has any, are in the buffers).
        q.gA = ga;
        q.gB = ga;
        q.valid = quad_below(pi.vend - E);
        return q;
    }
    const PieceInfo pn = info[p + 1];  // the tile holds E + 3, so it holds this piece
    const int64_t gb = a.shard_layout ? E : E + pn.gdelta;
    if (E + kQuad > pn.end || (uses_grads(OP) && (ga + kQuad > a.glen || gb < 0))) {
        q.slow = true;
        return q;
    }
    q.gA = ga;
    q.gB = gb;
    q.selB = 0xfu & ~quad_below(pi.end - E);
    q.valid = quad_below(pi.vend - E) | (q.selB & quad_below(pn.vend - E));
    return q;
}

// The rank-order sum for two planned quads whose elements may come from
// two pieces each: both reads go out for every rank of a batch of 4 before
// the adds, and each element takes the one its piece names.
template <typename GT, int CAP, bool TG>
__device__ __forceinline__ void reduce_two(const ShardArgs<CAP>& a, const QuadPlan (&q)[2],
                                           float (&g)[2][kQuad]) {
    constexpr int B = 4;
    const int nd = a.nd;
    for (int r0 = 0; r0 < nd; r0 += B) {
        float xa[B][2][kQuad], xb[B][2][kQuad];
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const GT* gp = static_cast<const GT*>(grad_ptr<CAP>(min(r0 + i, nd - 1)));
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                load4<GT, TG>(gp + q[h].gA, 0u, xa[i][h]);
                load4<GT, TG>(gp + q[h].gB, 0u, xb[i][h]);
            }
        }
#pragma unroll
        for (int i = 0; i < B; ++i) {
            if (r0 + i < nd) {
                const bool first = (r0 + i) == 0;
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int k = 0; k < kQuad; ++k) {
                        const float x = (q[h].selB >> k) & 1u ? xb[i][h][k] : xa[i][h][k];
                        g[h][k] = first ? x : g[h][k] + x;
                    }
            }
        }
    }
}

// Both quads of a lane of a multi-piece tile inside the call's range, as
// planned: one batch of state and gradient loads, then the stores of every
// real element (reduce ops also write 0 to pad slots of the accumulator).
// Pad elements of master, m and v are stored back unchanged; the bf16 copy is
// written element by element where a quad has pad elements. Slow quads are
// loaded with the rest and left alone.
template <int OP, typename GT, int CAP, bool TG>
__device__ __forceinline__ void quads_planned(const ShardArgs<CAP>& a, const int64_t (&E)[2],
                                              const QuadPlan (&q)[2]) {
    float p[2][kQuad], m[2][kQuad], v[2][kQuad], c[2][kQuad], g[2][kQuad];
    if constexpr (is_adam(OP)) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            ld_f32x4(a.master + E[h], p[h]);
            ld_f32x4(a.m + E[h], m[h]);
            ld_f32x4(a.v + E[h], v[h]);
        }
    }
    if constexpr (reads_acc(OP)) {
#pragma unroll
        for (int h = 0; h < 2; ++h) ld_f32x4(a.acc + E[h], c[h]);
    }
    if constexpr (uses_grads(OP)) {
        const bool two = (q[0].selB != 0u && q[0].gB != q[0].gA) ||
                         (q[1].selB != 0u && q[1].gB != q[1].gA);
        if (__any(two)) {
            reduce_two<GT, CAP, TG>(a, q, g);
        } else {
            const int64_t gb[2] = {q[0].gA, q[1].gA};
            const uint32_t off[2] = {0u, 0u};
            reduce_quads<GT, CAP, 2, TG>(a, gb, off, g);
        }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int k = 0; k < kQuad; ++k) {
            if constexpr (OP == OP_ADAM) g[h][k] = c[h][k];
            else if constexpr (reads_acc(OP)) g[h][k] = c[h][k] + g[h][k];
        }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (q[h].slow) continue;
        const uint32_t val = q[h].valid;
        if constexpr (is_reduce(OP)) {
            float r[kQuad];
#pragma unroll
            for (int k = 0; k < kQuad; ++k) r[k] = (val >> k) & 1u ? g[h][k] : 0.0f;
            st_f32x4(a.acc + E[h], r);
        } else {
            if (val == 0u) continue;
            float pn[kQuad], mn[kQuad], vn[kQuad];
#pragma unroll
            for (int k = 0; k < kQuad; ++k) {
                pn[k] = p[h][k];
                mn[k] = m[h][k];
                vn[k] = v[h][k];
                adam1(pn[k], mn[k], vn[k], g[h][k], a.hp);
                const bool ok = (val >> k) & 1u;
                pn[k] = ok ? pn[k] : p[h][k];
                mn[k] = ok ? mn[k] : m[h][k];
                vn[k] = ok ? vn[k] : v[h][k];
            }
            st_f32x4(a.master + E[h], pn);
            st_f32x4(a.m + E[h], mn);
            st_f32x4(a.v + E[h], vn);
            if (val == 0xfu) {
                st_bf16x4(a.work + E[h], pn);
            } else {
#pragma unroll
                for (int k = 0; k < kQuad; ++k)
                    if ((val >> k) & 1u) a.work[E[h] + k] = to_bf16(pn[k]);
            }
        }
    }
}

// One quad of any kind; p is the index of its piece in `info`.
template <int OP, typename GT, int CAP, bool TG>
__device__ __forceinline__ void quad_one(const ShardArgs<CAP>& a, int64_t E, int kind, int p,
                                         PieceInfo pi, const PieceInfo* info) {
    if (kind == Q_FAST) {
        const int64_t Eb[1] = {E};
        const int64_t gb[1] = {a.shard_layout ? E : E + pi.gdelta};
        const int64_t ib[1] = {E + pi.idelta};
        const uint32_t off[1] = {0u};
        const bool ok[1] = {true};
        quads_fast<OP, GT, CAP, 1, TG>(a, Eb, gb, ib, off, ok);
    } else if (kind == Q_PAD) {
        quad_pad<OP, CAP>(a, E);
    } else if (kind == Q_MIXED) {
        quad_mixed<OP, GT, CAP>(a, E, p, pi, info);
    } else if (kind == Q_SLOW) {
        // Only quads that cross the call's range boundary: element by element,
        // touching nothing outside the range.
        for (int k = 0; k < kQuad; ++k) {
            const int64_t e = E + k;
            if (e < a.e_begin || e >= a.e_end) continue;
            while (e >= pi.end) pi = info[++p];
            elem_op<OP, GT, CAP>(a, e, e < pi.vend, pi);
        }
    }
}

// Workgroups go to the 8 XCDs in turn (workgroup b to XCD b % 8), each XCD
// with an L2 of its own. Launches over short pieces give each XCD runs of
// kXcdRun consecutive tiles instead: a cache line that two neighbouring
// tiles share (a piece starts at any element offset) is then fetched once,
// into the L2 of the XCD that runs both. The grid is rounded up to whole
// rounds of 8 runs; xcd_run_tile maps workgroup b to its tile.
constexpr int kXcdRun = 16;

__device__ __forceinline__ int64_t xcd_run_tile(int64_t b) {
    const int64_t x = b % 8, i = b / 8;
    return ((i / kXcdRun) * 8 + x) * kXcdRun + (i % kXcdRun);
}

// W waves per tile: W = 1, the wave takes both quads of each lane; W = 2,
// workgroup 2i + h takes quad h (elements 256h .. 256h + 255) of tile i.
// TG: launches over short pieces. Their gradients are read with ordinary
// (L2-allocating) loads instead of non-temporal ones, and their tiles go
// to the XCDs in runs (xcd_run_tile): a tile's gradient runs start
// mid-line, and the line a run shares with the next tile's run is then
// still in that XCD's L2 when the next tile reads it. Runs of 16 tiles cut
// the 10,000-tensor fused step's read excess from +11.5% to +4.1% (all
// bytes: +7.7% to +2.7%) for 0.7% of its time.
template <int OP, typename GT, int CAP, int W, bool TG>
__global__ __launch_bounds__(kWaveLanes) void shard_kernel(const ShardArgs<CAP> a) {
    static_assert(W == 1 || W == 2, "one or two waves per tile");
    __shared__ int64_t s_e0[kStage];
    __shared__ PieceInfo s_info[kStage];
    const int lane = threadIdx.x;
    int64_t tile = a.tile_first + blockIdx.x / W;
    if constexpr (W == 1 && TG) {
        tile = a.tile_first + xcd_run_tile(blockIdx.x);
        if (tile >= a.tile_end) return;  // the grid is rounded up to 8 runs
    }
    const int hw = W == 2 ? int(blockIdx.x % 2) : 0;
    const int64_t E0 = tile * kTile + int64_t(lane) * kQuad;
    // Wave-uniform bracket of the tile's pieces (scalar loads).
    const int lo = a.tile[tile];
    const int hi = a.tile[tile + 1];
    if (lo == hi) {
        // Whole tile inside one piece: the common case for large parameters.
        const PieceInfo pi = a.info[lo];
        const int64_t T0 = tile * kTile;
        if (T0 >= a.e_begin && T0 + kTile <= a.e_end && T0 + kTile <= pi.vend) {
            // Every element real and in range: wave-uniform bases (scalar
            // registers) plus the lane's 32-bit offsets.
            const int64_t gbase = a.shard_layout ? T0 : T0 + pi.gdelta;
            if constexpr (W == 2) {
                const int64_t Eb[1] = {T0};
                const int64_t gb[1] = {gbase};
                const int64_t ib[1] = {T0 + pi.idelta};
                const uint32_t off[1] = {uint32_t(lane) * kQuad + uint32_t(hw) * uint32_t(kHalf)};
                const bool ok[1] = {true};
                quads_fast<OP, GT, CAP, 1, TG>(a, Eb, gb, ib, off, ok);
            } else {
                const int64_t Eb[2] = {T0, T0};
                const int64_t gb[2] = {gbase, gbase};
                const int64_t ib[2] = {T0 + pi.idelta, T0 + pi.idelta};
                const uint32_t off[2] = {uint32_t(lane) * kQuad, uint32_t(lane) * kQuad + kHalf};
                const bool ok[2] = {true, true};
                quads_fast<OP, GT, CAP, 2, TG>(a, Eb, gb, ib, off, ok);
            }
            return;
        }
    }
    // A tile at a piece, pad or range boundary. Several pieces: stage their
    // table in LDS with one coalesced load and search it there. A whole-tile
    // wave's two quads go through one call site (a loop kept rolled): each
    // copy of the update is long, and fewer copies keep the kernel within
    // the instruction cache.
    const int n = hi - lo + 1;
    const int64_t* e0 = a.e0 + lo;
    const PieceInfo* info = a.info + lo;
    if (n >= kStageMin && n <= kStage) {
        for (int i = lane; i < n; i += kWaveLanes) {
            s_e0[i] = e0[i];
            s_info[i] = info[i];
        }
        __syncthreads();
        e0 = s_e0;
        info = s_info;
    }
    if constexpr (W == 1 && OP != OP_COPYIN && CAP <= 16) {
        // Whole tile inside the call's range: both quads of a lane go out as
        // one batch of loads (each lane with its own addresses), a quad that
        // crosses into the next piece reading both pieces' gradients; only
        // quads meeting three pieces, or at the ends of the gradient
        // buffers, follow on their own. (Not for more than 16 ranks: the
        // registers it takes there would lower the waves per CU.)
        const int64_t T0 = tile * kTile;
        if (T0 >= a.e_begin && T0 + kTile <= a.e_end) {
            const int64_t E[2] = {E0, E0 + kHalf};
            const int pa = n == 1 ? 0 : find_local(e0, n, E[0]);
            const int pz = n == 1 ? 0 : find_local(e0, n, E[1]);
            const PieceInfo ia = info[pa], iz = info[pz];
            const QuadPlan q[2] = {plan_quad<OP>(a, E[0], pa, ia, info),
                                   plan_quad<OP>(a, E[1], pz, iz, info)};
            quads_planned<OP, GT, CAP, TG>(a, E, q);
#pragma unroll 1
            for (int h = 0; h < 2; ++h) {
                if (h ? q[1].slow : q[0].slow)
                    quad_mixed<OP, GT, CAP>(a, E[h], h ? pz : pa, h ? iz : ia, info);
            }
            return;
        }
    }
#pragma unroll 1
    for (int h = hw; h < hw + 3 - W; ++h) {  // both quads, or the wave's one
        const int64_t E = E0 + h * kHalf;
        const int p = n == 1 ? 0 : find_local(e0, n, E);
        const PieceInfo pi = info[p];
        quad_one<OP, GT, CAP, TG>(a, E, classify(a, E, pi), p, pi, info);
    }
}

struct GatherArgs {
    const int64_t* k0;
    const int64_t* delta;
    const int32_t* tile;
    const int64_t* tile_delta;  // per local tile, or NULL (k_first not tile-aligned)
    const int64_t* tile_pair;   // three per local tile, or NULL likewise
    int64_t k_first, count;
    const void* src;
    void* out;
};

// Element groups of 16 bytes: 8 bf16 contiguous per lane, or two fp32 quads
// per lane (at 4*l and 256 + 4*l), so each instruction stays contiguous.
template <typename T>
struct GatherShape {
    static constexpr int kGroup = 16 / sizeof(T);                       // elements per group
    static constexpr int kGroups = sizeof(T) == 2 ? 1 : 2;              // groups per lane
    static constexpr int kStride = sizeof(T) == 2 ? 0 : kHalf;          // between groups
    static constexpr int kLaneStep = kGroup;                            // lane offset
};

// N elements as one value (to bit-cast a 16-byte group into its elements).
template <typename T, int N>
struct ElemArray {
    T v[N];
};

// Tiles of the gather holding at most this many pieces read the pieces'
// starts and deltas with wave-uniform scalar loads and pick per lane with
// register selects: one scalar round trip, like a single-piece tile.
constexpr int kPick = 8;

// Gathers over short pieces (many parameters of a few thousand elements):
// a piece starts at any element offset, so its first and last cache lines
// are shared with the neighbouring pieces, which neighbouring tiles read.
// Such launches load their sources with ordinary (L2-allocating) loads and
// give each XCD runs of kXcdRun consecutive tiles (xcd_run_tile), so a shared
// line is fetched once into that XCD's L2. Long pieces keep non-temporal
// loads and the plain order: each line is read once.

template <bool SHORT>
__device__ __forceinline__ u32x4 ld_src(const u32x4_a2* p) {
    if constexpr (SHORT) return ld_x4_a2(p);
    else return ldnt_x4_a2(p);
}

// One tile of the gather: out[k] = src[K + delta(piece of K)], K = k_first
// + k, for the tile's k < count. s_k0 and s_delta: the wave's LDS for
// staging the pieces of a tile of many.
template <typename T, bool SHORT>
__device__ __forceinline__ void gather_tile(const GatherArgs& a, int64_t tile, int lane,
                                            int64_t* s_k0, int64_t* s_delta) {
    using S = GatherShape<T>;
    const int64_t kw = tile * kTile;  // local start of the wave's tile
    const T* src = static_cast<const T*>(a.src);
    T* out = static_cast<T*>(a.out);
    if (!SHORT && a.tile_delta && kw + kTile <= a.count) {
        // Long pieces, tile-aligned launch: one scalar load says whether the
        // whole tile is one run of one rank's slice, and gives that run's
        // delta, a round trip ahead of the data instead of two. Short-piece
        // launches read a record of their own (below).
        const int64_t d = a.tile_delta[tile];
        if (d != kNoTileDelta) {
            const T* sb = src + (a.k_first + kw + d);
            T* ob = out + kw;
#pragma unroll
            for (int h = 0; h < S::kGroups; ++h) {
                const uint32_t o = h * S::kStride + uint32_t(lane) * S::kLaneStep;
                stnt(reinterpret_cast<u32x4*>(ob + o),
                     ld_src<SHORT>(reinterpret_cast<const u32x4_a2*>(sb + o)));
            }
            return;
        }
    }
    if (SHORT && a.tile_pair) {
        // Short pieces, tile-aligned launch: one record gives the tile's (at
        // most two) pieces: the second's start and both deltas.
        const int64_t* rec = a.tile_pair + 3 * tile;
        const int64_t split = rec[0];
        if (split != kNoTileDelta) {
            const int64_t d0 = rec[1], d1 = rec[2];
#pragma unroll
            for (int h = 0; h < S::kGroups; ++h) {
                const int64_t k = kw + h * S::kStride + int64_t(lane) * S::kLaneStep;
                if (k >= a.count) continue;
                const int64_t K = a.k_first + k;
                if (k + S::kGroup <= a.count && (K + S::kGroup <= split || K >= split)) {
                    const int64_t d = K < split ? d0 : d1;
                    stnt(reinterpret_cast<u32x4*>(out + k),
                         ld_src<SHORT>(reinterpret_cast<const u32x4_a2*>(src + K + d)));
                } else {
                    // Crosses the split or the end: element by element, every
                    // load issued (clamped to the launch's last element).
                    T x[S::kGroup];
#pragma unroll
                    for (int i = 0; i < S::kGroup; ++i) {
                        const int64_t KK = min(K + i, a.k_first + a.count - 1);
                        x[i] = src[KK + (KK < split ? d0 : d1)];
                    }
                    if (k + S::kGroup <= a.count) {
                        stnt(reinterpret_cast<u32x4*>(out + k), __builtin_bit_cast(u32x4, x));
                    } else {
#pragma unroll
                        for (int i = 0; i < S::kGroup; ++i)
                            if (k + i < a.count) out[k + i] = x[i];
                    }
                }
            }
            return;
        }
    }
    const int64_t kw_last = a.k_first + min(kw + kTile, a.count) - 1;
    const int lo = a.tile[(a.k_first + kw) / kTile];
    const int hi = a.tile[kw_last / kTile + 1];
    const int n = hi - lo + 1;
    const int64_t* k0 = a.k0 + lo;
    const int64_t* delta = a.delta + lo;
    if (n == 1) {
        const int64_t next = k0[1], d = delta[0];
        if (kw + kTile <= a.count && a.k_first + kw + kTile <= next) {
            // The whole tile is one run of one rank's slice: scalar bases plus
            // the lane's 32-bit offsets.
            const T* sb = src + (a.k_first + kw + d);
            T* ob = out + kw;
#pragma unroll
            for (int h = 0; h < S::kGroups; ++h) {
                const uint32_t o = h * S::kStride + uint32_t(lane) * S::kLaneStep;
                stnt(reinterpret_cast<u32x4*>(ob + o),
                     ld_src<SHORT>(reinterpret_cast<const u32x4_a2*>(sb + o)));
            }
            return;
        }
    }
    if (n <= kPick) {
        // Few pieces: starts and deltas in scalar registers (indices clamped
        // so no load passes the table's end), picked per element by selects.
        int64_t sk[kPick + 1], sd[kPick];
#pragma unroll
        for (int i = 0; i <= kPick; ++i) sk[i] = k0[min(i, n)];
#pragma unroll
        for (int i = 0; i < kPick; ++i) sd[i] = delta[min(i, n - 1)];
        // next start and delta of the piece holding element K
        auto pick = [&](int64_t K, int64_t& next, int64_t& d) {
            next = sk[1];
            d = sd[0];
#pragma unroll
            for (int i = 1; i < kPick; ++i) {
                const bool c = i < n && sk[i] <= K;
                next = c ? sk[i + 1] : next;
                d = c ? sd[i] : d;
            }
        };
#pragma unroll
        for (int h = 0; h < S::kGroups; ++h) {
            const int64_t k = kw + h * S::kStride + int64_t(lane) * S::kLaneStep;
            if (k >= a.count) continue;
            const int64_t K = a.k_first + k;
            int64_t next, d;
            pick(K, next, d);
            if (k + S::kGroup <= a.count && K + S::kGroup <= next) {
                stnt(reinterpret_cast<u32x4*>(out + k),
                     ld_src<SHORT>(reinterpret_cast<const u32x4_a2*>(src + K + d)));
            } else {
                // Crosses a piece boundary or the end: each element picks its
                // own piece; every load is issued unconditionally.
                T x[S::kGroup];
#pragma unroll
                for (int i = 0; i < S::kGroup; ++i) {
                    const int64_t KK = min(K + i, a.k_first + a.count - 1);
                    int64_t nx, di;
                    pick(KK, nx, di);
                    x[i] = src[KK + di];
                }
                if (k + S::kGroup <= a.count) {
                    stnt(reinterpret_cast<u32x4*>(out + k), __builtin_bit_cast(u32x4, x));
                } else {
#pragma unroll
                    for (int i = 0; i < S::kGroup; ++i)
                        if (k + i < a.count) out[k + i] = x[i];
                }
            }
        }
        return;
    }
    if (n <= kStage) {
        // Many pieces: stage their starts and deltas in LDS.
        for (int i = lane; i <= n; i += kWaveLanes) s_k0[i] = k0[i];
        for (int i = lane; i < n; i += kWaveLanes) s_delta[i] = delta[i];
        __syncthreads();
        k0 = s_k0;
        delta = s_delta;
    }
#pragma unroll
    for (int h = 0; h < S::kGroups; ++h) {
        const int64_t k = kw + h * S::kStride + int64_t(lane) * S::kLaneStep;
        if (k >= a.count) continue;
        const int64_t K = a.k_first + k;
        int q = find_local(k0, n, K);
        int64_t next = k0[q + 1];
        int64_t d = delta[q];
        if (k + S::kGroup <= a.count && K + S::kGroup <= next) {
            // src may sit at any element offset; out + k is 16-byte aligned.
            const u32x4 x = ld_src<SHORT>(reinterpret_cast<const u32x4_a2*>(src + K + d));
            stnt(reinterpret_cast<u32x4*>(out + k), x);
        } else {
            for (int i = 0; i < S::kGroup; ++i) {
                const int64_t kk = k + i;
                if (kk >= a.count) break;
                const int64_t KK = K + i;
                while (KK >= next) {
                    ++q;
                    next = k0[q + 1];
                    d = delta[q];
                }
                out[kk] = src[KK + d];
            }
        }
    }
}

// One wave per tile (short-piece launches: XCD runs of kXcdRun tiles).
template <typename T, bool SHORT>
__global__ __launch_bounds__(kWaveLanes) void gather_kernel(const GatherArgs a) {
    __shared__ int64_t s_k0[kStage + 1];
    __shared__ int64_t s_delta[kStage];
    int64_t tile = blockIdx.x;
    if constexpr (SHORT) {
        tile = xcd_run_tile(tile);
        if (tile * kTile >= a.count) return;  // the grid is rounded up to 8 runs
    }
    gather_tile<T, SHORT>(a, tile, threadIdx.x, s_k0, s_delta);
}

// ---- Span gather (bf16 work copy, short pieces) ---------------------------
// One wave per span (see WaveSpan): it reads the span's record with scalar
// loads, loads every rank's run of the span as aligned 16-byte chunks and
// the span's pieces in one batch (ordinary loads: the first and last line
// of a run are shared with the neighbouring spans, which the same XCD runs),
// lands them in LDS, then writes the span's tiles with aligned 16-byte
// stores, each lane taking its 8 elements from LDS at the offset of their
// piece. Spans of two tiles measured fastest: larger spans leave fewer
// waves in flight, and waves that loop over spans (prefetching the next
// record and data) were slower still.
constexpr int kSpanPer = (kSpanChunks + kWaveLanes - 1) / kWaveLanes;  // chunks per lane
constexpr int kSegPer = (kSpanSegs + kWaveLanes - 1) / kWaveLanes;     // pieces per lane

struct SpanArgs {
    const WaveSpan* spans;
    const SpanSeg* segs;
    const uint16_t* src;
    uint16_t* out;
    int64_t span_first;
    int64_t nspan;
    int64_t k_first;
    int64_t count;
    int64_t src_elems;
};

// The record, read whole in one batch of 16-byte loads (scalar loads: the
// address is wave-uniform and nothing is stored before).
__device__ __forceinline__ WaveSpan load_span(const WaveSpan* p) {
    struct Words {
        u32x4 w[sizeof(WaveSpan) / 16];
    } words;
    const u32x4* rp = reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < int(sizeof(WaveSpan) / 16); ++i) words.w[i] = rp[i];
    return __builtin_bit_cast(WaveSpan, words);
}

// Source chunk of span chunk c: c + (first source chunk - first LDS chunk)
// of its run (the last run whose LDS start is at or below c).
template <typename Rec>
__device__ __forceinline__ int64_t span_chunk(const Rec& R, int c) {
    int64_t gd = R.chunk0;  // run 0 starts at LDS chunk 0
#pragma unroll
    for (int q = 1; q < kSpanRuns; ++q) {
        if (q >= R.nrun) break;
        gd = c >= R.lds0[q] ? R.chunk0 + R.dchunk[q - 1] - R.lds0[q] : gd;
    }
    return c + gd;
}

// A span's LDS image: every chunk of every run, then the pieces, in one
// batch of loads issued unconditionally (lanes past the end reload the last
// chunk or piece), then landed in LDS. src holds src_elems elements.
template <typename Rec>
__device__ __forceinline__ void span_land(const Rec& R, int lane, const uint16_t* src,
                                          int64_t src_elems, const SpanSeg* segs,
                                          u32x4* s_data, SpanSeg* s_seg) {
    const int chunks = R.chunks, nseg = R.nseg;
    const u32x4* src16 = reinterpret_cast<const u32x4*>(src);
    const int64_t whole = src_elems / kSpanChunkElems;  // chunks inside src (>= 1)
    u32x4 v[kSpanPer];
    bool tail = false;  // some chunk of this lane holds the end of src
#pragma unroll
    for (int j = 0; j < kSpanPer; ++j) {
        const int64_t gc = span_chunk(R, min(lane + j * kWaveLanes, chunks - 1));
        tail |= gc >= whole;
        v[j] = src16[min(gc, whole - 1)];
    }
    SpanSeg sg[kSegPer];
#pragma unroll
    for (int j = 0; j < kSegPer; ++j)
        sg[j] = segs[R.seg_first + min(lane + j * kWaveLanes, nseg - 1)];
    if (tail) {
        // a chunk holding the end of src: only its elements inside src
#pragma unroll
        for (int j = 0; j < kSpanPer; ++j) {
            const int64_t gc = span_chunk(R, min(lane + j * kWaveLanes, chunks - 1));
            if (gc >= whole) {
                uint16_t e[kSpanChunkElems];
#pragma unroll
                for (int k = 0; k < kSpanChunkElems; ++k) {
                    const int64_t x = gc * kSpanChunkElems + k;
                    e[k] = x < src_elems ? src[x] : uint16_t(0);
                }
                v[j] = __builtin_bit_cast(u32x4, e);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < kSegPer; ++j)
        if (lane + j * kWaveLanes < nseg) s_seg[lane + j * kWaveLanes] = sg[j];
#pragma unroll
    for (int j = 0; j < kSpanPer; ++j) {
        const int c = lane + j * kWaveLanes;
        if (c < chunks) s_data[c] = v[j];
    }
    __syncthreads();
}

// One lane's output chunk: the n (1 <= n) elements at span-local flat
// indices kl .. kl + min(n, 8) - 1, which meet pieces lo .. hi of the span,
// written to out (16-byte aligned) from the span's LDS image.
__device__ __forceinline__ void span_write8(const u32x4* s_data, const SpanSeg* s_seg, int kl,
                                            int lo, int hi, int n, uint16_t* out) {
    const uint32_t* s32 = reinterpret_cast<const uint32_t*>(s_data);
    const uint16_t* s16 = reinterpret_cast<const uint16_t*>(s_data);
    if (lo == hi && n >= kSpanChunkElems) {
        // One piece: the 8 elements are LDS elements p .. p + 7, read as the
        // dwords holding them (measured faster than whole 16-byte chunks and
        // a shift).
        const int p = kl + s_seg[lo].off;
        const int dw = p >> 1;
        u32x4 o;
        if ((p & 1) == 0) {
            o = u32x4{s32[dw], s32[dw + 1], s32[dw + 2], s32[dw + 3]};
        } else {
            const uint32_t d0 = s32[dw], d1 = s32[dw + 1], d2 = s32[dw + 2], d3 = s32[dw + 3],
                           d4 = s32[dw + 4];
            o = u32x4{__builtin_amdgcn_alignbyte(d1, d0, 2), __builtin_amdgcn_alignbyte(d2, d1, 2),
                      __builtin_amdgcn_alignbyte(d3, d2, 2), __builtin_amdgcn_alignbyte(d4, d3, 2)};
        }
        stnt(reinterpret_cast<u32x4*>(out), o);
        return;
    }
    // Several pieces, or fewer than 8 elements: each element finds its piece
    // (binary search, then forward); elements past the n-th read the last
    // one and are not stored.
    const int kl_last = kl + min(n, kSpanChunkElems) - 1;
    int q = lo;
    for (int h = hi; q < h;) {
        const int mid = (q + h + 1) >> 1;
        if (s_seg[mid].k <= kl) q = mid;
        else h = mid - 1;
    }
    uint16_t e[kSpanChunkElems];
#pragma unroll
    for (int k = 0; k < kSpanChunkElems; ++k) {
        const int K = min(kl + k, kl_last);
        while (q < hi && s_seg[q + 1].k <= K) ++q;
        e[k] = s16[K + s_seg[q].off];
    }
    if (n >= kSpanChunkElems) {
        stnt(reinterpret_cast<u32x4*>(out), __builtin_bit_cast(u32x4, e));
    } else {
#pragma unroll
        for (int k = 0; k < kSpanChunkElems; ++k)
            if (k < n) out[k] = e[k];
    }
}

__global__ __launch_bounds__(kWaveLanes) void gather_span_kernel(const SpanArgs a) {
    __shared__ u32x4 s_data[kSpanChunks];
    __shared__ SpanSeg s_seg[kSpanSegs];
    const int64_t sp = xcd_run_tile(blockIdx.x);
    if (sp >= a.nspan) return;  // the grid is rounded up to whole rounds of runs
    const WaveSpan R = load_span(a.spans + (a.span_first + sp));
    const int lane = threadIdx.x;
    const int64_t k_a = int64_t(R.tile0) * kTile;  // the span's first flat index
    span_land(R, lane, a.src, a.src_elems, a.segs, s_data, s_seg);

    const int64_t k_end = a.k_first + a.count;
    const int ntile = R.ntile;
    static_assert(kSpanTiles == 2, "the tile loop picks tseg[0] or tseg[1]");
    for (int tau = 0; tau < ntile; ++tau) {
        const int64_t K0 = k_a + int64_t(tau) * kTile;
        if (K0 + kTile <= a.k_first) continue;
        if (K0 >= k_end) break;
        // the tile's first and last piece (a select: no indexing of registers)
        const int ts = tau == 0 ? R.tseg[0] : R.tseg[1];
        const int kl = tau * int(kTile) + lane * kSpanChunkElems;
        const int64_t jo = k_a + kl - a.k_first;  // output index of the lane's first element
        if (jo < 0 || jo >= a.count) continue;  // (k_first is a multiple of kTile: jo >= 0)
        span_write8(s_data, s_seg, kl, ts & 0xff, ts >> 8, int(min(a.count - jo, int64_t(8))),
                    a.out + jo);
    }
}

// ---- Gather of a list of parameters into separate outputs ------------------
// A wave copies one tile of kTile elements of one output (two consecutive
// tiles in the record form of bf16 short-piece lists). A tile's record
// (TileRec) says where the tile's elements come from: a tile of a
// parameter whose slices hold kTile elements or more meets at most two
// ranks' slices, so two bases and a split describe it; a tile of a smaller
// parameter meets several, and each element group finds its rank by one
// division by the (small) shard length.

// The record of local tile kw / kTile of an output of a parameter with
// the given layout (element kw of the output is the tile's first).
__device__ __forceinline__ TileRec make_rec(void* out, int esz, int64_t shard_off, int64_t s,
                                            int64_t numel, int64_t S, int64_t kw) {
    TileRec r;
    r.out = static_cast<char*>(out) + kw * esz;
    // the rank whose slice holds element kw (a 32-bit division when both fit)
    const int64_t q = ((kw | s) >> 32) == 0 ? int64_t(uint32_t(kw) / uint32_t(s)) : kw / s;
    const int64_t rem = kw - q * s;
    r.step = S - s;
    r.base = shard_off + kw + q * r.step;  // q*S + shard_off + (kw - q*s)
    const int64_t cnt = min(kTile, numel - kw);
    if (s >= kTile) {
        r.split = static_cast<int32_t>(min(s - rem, kTile));
        r.count = static_cast<int32_t>(cnt);
    } else {
        r.split = -static_cast<int32_t>(s);
        r.count = static_cast<int32_t>(cnt | (rem << 16));
    }
    return r;
}

// Source offset (added to element k's own index) of local element k.
__device__ __forceinline__ int64_t rec_delta(const TileRec& rc, int k, int rem, uint32_t s) {
    if (rc.split >= 0) return rc.base + (k >= rc.split ? rc.step : 0);
    return rc.base + int64_t(uint32_t(rem + k) / s) * rc.step;
}

// One lane's share of a tile, loaded and not yet stored: its 16-byte groups
// (8 bf16, or two quads of fp32) and how many elements of each to store.
// Loading and storing apart lets a wave have several tiles' loads in
// flight before it stores any. The compiler reads this form's record in
// one scalar load; a copy that stored inside its per-group branch had the
// record's count read first and the rest after the branch, two round trips.
template <typename T>
struct RecGroups {
    u32x4 x[GatherShape<T>::kGroups];
    int n[GatherShape<T>::kGroups];  // elements to store (kGroup: the whole group)
    T* out;                          // the lane's first group; group h at + h * kStride
};

template <typename T, bool SHORT>
__device__ __forceinline__ RecGroups<T> load_rec_tile(const TileRec& rc, const T* src, int lane) {
    using Sh = GatherShape<T>;
    RecGroups<T> g;
    const bool many = rc.split < 0;
    const int count = many ? (rc.count & 0xffff) : rc.count;
    const int rem = many ? (rc.count >> 16) : 0;
    const uint32_t s = many ? uint32_t(-rc.split) : 1u;
    g.out = static_cast<T*>(rc.out) + lane * Sh::kLaneStep;
#pragma unroll
    for (int h = 0; h < Sh::kGroups; ++h) {
        const int o = h * Sh::kStride + lane * Sh::kLaneStep;
        g.n[h] = max(0, min(count - o, Sh::kGroup));
        g.x[h] = u32x4{0, 0, 0, 0};
        if (o >= count) continue;
        bool one;
        if (!many) one = o + Sh::kGroup <= rc.split || o >= rc.split;
        else one = uint32_t(rem + o) / s == uint32_t(rem + o + Sh::kGroup - 1) / s;
        if (g.n[h] == Sh::kGroup && one) {
            // the source may sit at any element offset
            const int64_t d = rec_delta(rc, o, rem, s);
            g.x[h] = ld_src<SHORT>(reinterpret_cast<const u32x4_a2*>(src + d + o));
        } else {
            // Crosses a slice boundary or the output's end: element by
            // element, every load issued (clamped to the last element).
            T x[Sh::kGroup];
#pragma unroll
            for (int i = 0; i < Sh::kGroup; ++i) {
                const int k = min(o + i, count - 1);
                x[i] = src[rec_delta(rc, k, rem, s) + k];
            }
            g.x[h] = __builtin_bit_cast(u32x4, x);
        }
    }
    return g;
}

template <typename T>
__device__ __forceinline__ void store_rec_tile(const RecGroups<T>& g) {
    using Sh = GatherShape<T>;
#pragma unroll
    for (int h = 0; h < Sh::kGroups; ++h) {
        T* out = g.out + h * Sh::kStride;  // 16-byte aligned
        if (g.n[h] == Sh::kGroup) {
            stnt(reinterpret_cast<u32x4*>(out), g.x[h]);
        } else if (g.n[h] > 0) {
            const auto x = __builtin_bit_cast(ElemArray<T, Sh::kGroup>, g.x[h]);
#pragma unroll
            for (int i = 0; i < Sh::kGroup; ++i)
                if (i < g.n[h]) out[i] = x.v[i];
        }
    }
}

// Copy one tile.
template <typename T, bool SHORT>
__device__ __forceinline__ void copy_rec_tile(const TileRec& rc, const T* src, int lane) {
    store_rec_tile(load_rec_tile<T, SHORT>(rc, src, lane));
}

// Short-piece lists give each XCD runs of kXcdRun consecutive tiles (see
// kXcdRun); returns the tile of workgroup `blk`, or -1 past the list.
template <bool SHORT>
__device__ __forceinline__ int64_t list_tile(int64_t blk, int64_t tiles) {
    if constexpr (SHORT) {
        const int64_t t = xcd_run_tile(blk);
        return t < tiles ? t : -1;
    } else {
        return blk;
    }
}

struct ListArgArgs {
    const void* src;
    int64_t S;
    int64_t tiles;
    int32_t n;
    int32_t esz;
    ArgEntry ents[kListArgMax];
    int32_t tile0[kListArgMax + 1];
};

// Argument form: the list's entries are in the kernel arguments. The wave
// counts, with scalar loads of the entries' first tiles, the entries that
// start after the first one at or below its tile, and reads that entry with
// one more scalar load: the argument segment stays in the scalar cache.
template <typename T, bool SHORT>
__global__ __launch_bounds__(kWaveLanes) void gather_list_args(const ListArgArgs a) {
    const int64_t b = list_tile<SHORT>(blockIdx.x, a.tiles);
    if (b < 0) return;
    const char* seg = (const char*)__builtin_amdgcn_kernarg_segment_ptr();
    const int32_t* t0 = reinterpret_cast<const int32_t*>(seg + offsetof(ListArgArgs, tile0));
    const ArgEntry* ents = reinterpret_cast<const ArgEntry*>(seg + offsetof(ListArgArgs, ents));
    // 16 first tiles per batch of scalar loads (the array has kListArgMax + 1
    // slots, so a batch never reads past it); tiles fit in 32 bits
    const int32_t bb = static_cast<int32_t>(b);
    int i = 0;
#pragma unroll
    for (int k0 = 0; k0 < kListArgMax; k0 += 16) {
        if (k0 >= a.n) break;
        int32_t v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = t0[k0 + j];
#pragma unroll
        for (int j = 0; j < 16; ++j) i += (k0 + j >= 1 && k0 + j < a.n && v[j] <= bb) ? 1 : 0;
    }
    const ArgEntry e = ents[i];
    const TileRec rc = make_rec(e.out, a.esz, e.shard_off, e.shard_len, e.numel, a.S,
                                (b - t0[i]) * kTile);
    copy_rec_tile<T, SHORT>(rc, static_cast<const T*>(a.src), threadIdx.x);
}

struct ListExpandArgs {
    const ListEntry* ents;
    const int32_t* coarse;
    const ParamInfo* params;
    TileRec* recs;
    int64_t S;
    int64_t t_begin;  // a multiple of 64
    int64_t t_end;
    int32_t n;
    int32_t esz;
};

// Staged form, first kernel: the records of tiles [t_begin, t_end), 64 per
// wave. The coarse index gives the entry of the wave's first tile; the
// wave's 64 tiles lie in that entry and at most 63 after it (every staged
// entry has a tile), whose first tiles the lanes load; each lane finds its
// own entry among them by a binary search over the lanes.
__global__ __launch_bounds__(kWaveLanes) void list_expand_kernel(const ListExpandArgs a) {
    const int lane = threadIdx.x;
    const int64_t b0 = a.t_begin + int64_t(blockIdx.x) * 64;
    const int64_t b = b0 + lane;
    const int i0 = a.coarse[b0 / 64];
    // lane l holds window entry i0 + l (past the list: its first tile reads
    // as unreachable)
    const ListEntry w = a.ents[min(i0 + lane, a.n - 1)];
    const int32_t t0 = i0 + lane < a.n ? w.tile0 : INT32_MAX;
    int j = 0;
    for (int st = 32; st > 0; st >>= 1) {
        const int c = j + st;
        const int32_t v = __shfl(t0, c < 64 ? c : 63);
        if (c < 64 && v <= b) j = c;
    }
    const int32_t id = __shfl(w.id, j);
    const int32_t tile0 = __shfl(w.tile0, j);
    const uint64_t o = uint64_t(reinterpret_cast<uintptr_t>(w.out));
    void* out = reinterpret_cast<void*>((uint64_t(uint32_t(__shfl(int(o >> 32), j))) << 32) |
                                        uint32_t(__shfl(int(uint32_t(o)), j)));
    if (b >= a.t_end) return;
    const ParamInfo p = a.params[id];
    const int64_t kw = (b - tile0) * kTile;
    a.recs[b - a.t_begin] = make_rec(out, a.esz, p.shard_off, p.shard_len, p.numel, a.S, kw);
}

// Tiles per wave of the record form: two for bf16 short-piece lists (one
// tile is 1 KB read and 1 KB written per wave, too little in flight while
// the waves of a many-tile list queue for dispatch), else one.
constexpr int list_rec_tiles(int esz, bool short_pieces) {
    return esz == 2 && short_pieces ? 2 : 1;
}

struct ListRecArgs {
    const TileRec* recs;
    const void* src;
    int64_t tiles;  // tiles of the chunk
};

// Staged form, second kernel: list_rec_tiles(sizeof(T), SHORT) consecutive
// records per wave, every tile's loads issued before any tile's stores
// (records past the chunk's last are clamped to it and not stored).
template <typename T, bool SHORT>
__global__ __launch_bounds__(kWaveLanes) void gather_list_recs(const ListRecArgs a) {
    constexpr int NT = list_rec_tiles(int(sizeof(T)), SHORT);
    const int64_t b = list_tile<SHORT>(blockIdx.x, (a.tiles + NT - 1) / NT);
    if (b < 0) return;
    const T* src = static_cast<const T*>(a.src);
    RecGroups<T> g[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j)
        g[j] = load_rec_tile<T, SHORT>(a.recs[min(NT * b + j, a.tiles - 1)], src, threadIdx.x);
#pragma unroll
    for (int j = 0; j < NT; ++j)
        if (NT * b + j < a.tiles) store_rec_tile(g[j]);
}

// Resident waves. With every CU full of shard waves, each touching a dozen
// streams, HBM serves the mix of reads and writes less efficiently than with
// fewer waves resident, as long as each wave has enough bytes in flight.
// The cap is set through the LDS each workgroup reserves (its piece tables
// plus padding), at totals measured on MI355X (160 KiB of LDS per CU).
// Half-tile waves (launches of up to 16 ranks over long pieces), by kind and
// by the bytes read per element: the fused step reading 40 or more (16 ranks
// with the accumulator) 23405 bytes, 7 workgroups per CU; a lighter fused
// step (8 ranks) 16384, 10 per CU; Adam alone 13312, 12 per CU; the reduce
// reading 24 or more (16 ranks) 13312, 12 per CU; a lighter reduce (8 ranks)
// 10240, 16 per CU. Whole-tile waves over short pieces, whose boundary tiles
// need more waves to hide their latency: 16384, 10 per CU, from 16 bytes per
// element. Lighter launches, launches of more than 16 ranks, launches too
// small to fill the chip several times, and the copy-in keep every wave.
constexpr size_t kLdsTunedPerCu = 163840;
constexpr size_t kLdsFusedHeavy = 23405;
constexpr size_t kLdsFused = 16384;
constexpr size_t kLdsAdamAlone = 13312;
constexpr size_t kLdsReduceHeavy = 13312;
constexpr size_t kLdsReduce = 10240;
constexpr size_t kLdsShortPieces = 16384;
constexpr int kHeavyFusedBytes = 40;
constexpr int kHeavyReduceBytes = 24;
constexpr int kShortCapBytes = 16;
constexpr int64_t kCapMinTiles = 8192;

size_t device_lds_per_cu() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
            hipSuccess)
            v = -1;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v > 0 ? size_t(v) : 0;
}

// Dynamic LDS that brings a shard workgroup (W waves per tile) to the
// reservation above, or 0.
template <int OP, typename GT, int CAP, int W>
size_t shard_lds_pad(const ShardLaunch& L, int64_t tiles) {
    if constexpr (CAP > 16 || OP == OP_COPYIN) {
        return 0;
    } else {
        if (tiles < kCapMinTiles || device_lds_per_cu() != kLdsTunedPerCu) return 0;
        const int grad = uses_grads(OP) ? L.nd * int(sizeof(GT)) : 0;
        const int bytes = grad + (is_adam(OP) ? 12 : 0) + (reads_acc(OP) ? 4 : 0);
        size_t total = 0;
        if constexpr (W == 1) {
            if (!L.short_pieces || bytes < kShortCapBytes) return 0;
            total = kLdsShortPieces;
        } else if constexpr (OP == OP_ADAM) {
            total = kLdsAdamAlone;
        } else if constexpr (is_adam(OP)) {
            total = bytes >= kHeavyFusedBytes ? kLdsFusedHeavy : kLdsFused;
        } else {
            total = bytes >= kHeavyReduceBytes ? kLdsReduceHeavy : kLdsReduce;
        }
        const size_t tables = kStage * (sizeof(int64_t) + sizeof(PieceInfo));
        return total > tables ? total - tables : 0;
    }
}

// Half-tile waves: shard launches of up to 16 ranks over long pieces (not
// the copy-in). Measured faster there under the caps above (+6-8% on the
// fused step, +1-6% on the reduce, +7% on Adam alone); whole-tile waves
// stay faster over short pieces and for more ranks.
template <int OP, int CAP>
constexpr bool kHalfTiles = CAP <= 16 && OP != OP_COPYIN;

// Ordinary gradient loads (TG) for launches over short pieces that read
// gradients, up to 16 ranks: 5656-5660 against 5494-5500 GB/s on the
// 10,000-tensor fused step (three alternating runs on one MI355X).
template <int OP, int CAP>
constexpr bool kTemporalShort = CAP <= 16 && uses_grads(OP);

// A launch's work-items (workgroups x 64) must fit in 32 bits.
constexpr int64_t kMaxBlocks = int64_t(UINT32_MAX) / kWaveLanes;

template <int OP, typename GT, int CAP>
hipError_t launch_t(const ShardLaunch& L, hipStream_t stream) {
    ShardArgs<CAP> a{};
    a.e0 = L.tab.e0;
    a.info = L.tab.info;
    a.tile = L.tab.tile;
    a.e_begin = L.e_begin;
    a.e_end = L.e_end;
    a.tile_first = L.e_begin / kTile;
    const int64_t tile_end = (L.e_end + kTile - 1) / kTile;
    a.tile_end = tile_end;
    a.master = L.master;
    a.m = L.m;
    a.v = L.v;
    a.work = L.work;
    a.acc = L.acc;
    a.src = L.src;
    a.hp = L.hp;
    a.nd = L.nd;
    a.shard_layout = L.shard_layout;
    a.glen = L.grad_len;
    if constexpr (uses_grads(OP)) {
        for (int r = 0; r < L.nd; ++r) a.grads[r] = L.grads[r];
    }
    const int64_t tiles = tile_end - a.tile_first;
    if (tiles <= 0) return hipSuccess;
    if constexpr (kHalfTiles<OP, CAP>) {
        if (!L.short_pieces && 2 * tiles <= kMaxBlocks) {
            const size_t lds_pad = shard_lds_pad<OP, GT, CAP, 2>(L, tiles);
            hipLaunchKernelGGL((shard_kernel<OP, GT, CAP, 2, false>),
                               dim3(static_cast<uint32_t>(2 * tiles)), dim3(kWaveLanes), lds_pad,
                               stream, a);
            return hipGetLastError();
        }
    }
    if (tiles > kMaxBlocks) return hipErrorInvalidValue;
    const size_t lds_pad = shard_lds_pad<OP, GT, CAP, 1>(L, tiles);
    if constexpr (kTemporalShort<OP, CAP>) {
        if (L.short_pieces) {
            const int64_t grid = (tiles + 8 * kXcdRun - 1) / (8 * kXcdRun) * (8 * kXcdRun);
            if (grid > kMaxBlocks) return hipErrorInvalidValue;
            hipLaunchKernelGGL((shard_kernel<OP, GT, CAP, 1, true>),
                               dim3(static_cast<uint32_t>(grid)), dim3(kWaveLanes), lds_pad,
                               stream, a);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((shard_kernel<OP, GT, CAP, 1, false>), dim3(static_cast<uint32_t>(tiles)),
                       dim3(kWaveLanes), lds_pad, stream, a);
    return hipGetLastError();
}

template <int OP, typename GT>
hipError_t launch_cap(const ShardLaunch& L, hipStream_t stream) {
    if constexpr (!uses_grads(OP)) {
        return launch_t<OP, GT, 1>(L, stream);
    } else {
        if (L.nd <= 16) return launch_t<OP, GT, 16>(L, stream);
        if (L.nd <= 64) return launch_t<OP, GT, 64>(L, stream);
        return launch_t<OP, GT, ZSP_MAX_RANKS>(L, stream);
    }
}

template <typename GT>
hipError_t launch_dtype(const ShardLaunch& L, ShardOp op, hipStream_t stream) {
    switch (op) {
        case OP_COPYIN: return launch_cap<OP_COPYIN, GT>(L, stream);
        case OP_REDUCE_SET: return launch_cap<OP_REDUCE_SET, GT>(L, stream);
        case OP_REDUCE_ACC: return launch_cap<OP_REDUCE_ACC, GT>(L, stream);
        case OP_FUSED: return launch_cap<OP_FUSED, GT>(L, stream);
        case OP_FUSED_ACC: return launch_cap<OP_FUSED_ACC, GT>(L, stream);
        case OP_ADAM: return launch_cap<OP_ADAM, GT>(L, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_shard_op(const ShardLaunch& L, ShardOp op, zsp_dtype dtype,
                           hipStream_t stream) {
    if (L.e_end <= L.e_begin) return hipSuccess;
    if (op == OP_ADAM) return launch_cap<OP_ADAM, float>(L, stream);
    if (dtype == ZSP_BF16) return launch_dtype<uint16_t>(L, op, stream);
    return launch_dtype<float>(L, op, stream);
}

hipError_t launch_gather(const GatherLaunch& L, zsp_dtype dtype, hipStream_t stream) {
    if (L.count <= 0) return hipSuccess;
    GatherArgs a{};
    a.k0 = L.tab.k0;
    a.delta = L.tab.delta;
    a.tile = L.tab.tile;
    a.tile_delta = L.tile_delta;
    a.tile_pair = L.tile_pair;
    a.k_first = L.k_first;
    a.count = L.count;
    a.src = L.src;
    a.out = L.out;
    if (L.nspan > 0 && dtype == ZSP_BF16) {
        SpanArgs sa{};
        sa.spans = L.tab.spans;
        sa.segs = L.tab.span_segs;
        sa.src = static_cast<const uint16_t*>(L.src);
        sa.out = static_cast<uint16_t*>(L.out);
        sa.span_first = L.span_first;
        sa.nspan = L.nspan;
        sa.k_first = L.k_first;
        sa.count = L.count;
        sa.src_elems = L.src_elems;
        const int64_t round = 8 * kXcdRun;  // one wave per span, XCD runs of spans
        const int64_t blocks = (L.nspan + round - 1) / round * round;
        if (blocks > kMaxBlocks) return hipErrorInvalidValue;
        hipLaunchKernelGGL(gather_span_kernel, dim3(static_cast<uint32_t>(blocks)),
                           dim3(kWaveLanes), 0, stream, sa);
        return hipGetLastError();
    }
    const int64_t tiles = (L.count + kTile - 1) / kTile;  // one wave per 512 outputs
    const int64_t runs = 8 * kXcdRun;
    const int64_t blocks = L.short_pieces ? (tiles + runs - 1) / runs * runs : tiles;
    if (blocks > kMaxBlocks) return hipErrorInvalidValue;
    const dim3 grid(static_cast<uint32_t>(blocks)), block(kWaveLanes);
    if (dtype == ZSP_BF16) {
        if (L.short_pieces)
            hipLaunchKernelGGL((gather_kernel<uint16_t, true>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((gather_kernel<uint16_t, false>), grid, block, 0, stream, a);
    } else {
        if (L.short_pieces)
            hipLaunchKernelGGL((gather_kernel<float, true>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((gather_kernel<float, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

namespace {

// Workgroups of a list launch of `waves` waves.
int64_t list_blocks(int64_t waves, bool short_pieces) {
    const int64_t runs = 8 * kXcdRun;
    return short_pieces ? (waves + runs - 1) / runs * runs : waves;
}

// Waves of the record form over `tiles` tiles.
int64_t rec_waves(int64_t tiles, int esz, bool short_pieces) {
    const int64_t nt = list_rec_tiles(esz, short_pieces);
    return (tiles + nt - 1) / nt;
}

template <typename T>
hipError_t launch_list_t(const ListLaunch& L, int esz, hipStream_t stream) {
    const dim3 block(kWaveLanes);
    if (L.n_args > 0) {
        ListArgArgs a{};
        a.src = L.src;
        a.S = L.S;
        a.tiles = L.tiles;
        a.n = L.n_args;
        a.esz = esz;
        for (int i = 0; i < L.n_args; ++i) a.ents[i] = L.args[i];
        for (int i = 0; i <= L.n_args; ++i) a.tile0[i] = L.arg_tile0[i];
        const int64_t blocks = list_blocks(L.tiles, L.short_pieces);
        if (blocks > kMaxBlocks) return hipErrorInvalidValue;
        if (L.short_pieces)
            hipLaunchKernelGGL((gather_list_args<T, true>), dim3(uint32_t(blocks)), block, 0,
                               stream, a);
        else
            hipLaunchKernelGGL((gather_list_args<T, false>), dim3(uint32_t(blocks)), block, 0,
                               stream, a);
        return hipGetLastError();
    }
    if (L.rec_cap <= 0 || L.rec_cap % 64 != 0) return hipErrorInvalidValue;
    if (L.mode != 0 && L.rec_cap < L.tiles) return hipErrorInvalidValue;
    if (L.mode == 2) {
        ListRecArgs g{};
        g.recs = L.recs;
        g.src = L.src;
        g.tiles = L.tiles;
        const int64_t blocks = list_blocks(rec_waves(L.tiles, esz, L.short_pieces), L.short_pieces);
        if (blocks > kMaxBlocks) return hipErrorInvalidValue;
        if (L.short_pieces)
            hipLaunchKernelGGL((gather_list_recs<T, true>), dim3(uint32_t(blocks)), block, 0,
                               stream, g);
        else
            hipLaunchKernelGGL((gather_list_recs<T, false>), dim3(uint32_t(blocks)), block, 0,
                               stream, g);
        return hipGetLastError();
    }
    for (int64_t t = 0; t < L.tiles; t += L.rec_cap) {
        const int64_t t_end = min(L.tiles, t + L.rec_cap);
        ListExpandArgs e{};
        e.ents = L.ents;
        e.coarse = L.coarse;
        e.params = L.params;
        e.recs = L.recs;
        e.S = L.S;
        e.t_begin = t;
        e.t_end = t_end;
        e.n = L.n_ents;
        e.esz = esz;
        const int64_t waves = (t_end - t + 63) / 64;
        hipLaunchKernelGGL(list_expand_kernel, dim3(uint32_t(waves)), block, 0, stream, e);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        if (L.mode == 1) continue;
        ListRecArgs g{};
        g.recs = L.recs;
        g.src = L.src;
        g.tiles = t_end - t;
        const int64_t blocks =
            list_blocks(rec_waves(t_end - t, esz, L.short_pieces), L.short_pieces);
        if (blocks > kMaxBlocks) return hipErrorInvalidValue;
        if (L.short_pieces)
            hipLaunchKernelGGL((gather_list_recs<T, true>), dim3(uint32_t(blocks)), block, 0,
                               stream, g);
        else
            hipLaunchKernelGGL((gather_list_recs<T, false>), dim3(uint32_t(blocks)), block, 0,
                               stream, g);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace

// Copy of a one-shot list's staging (entries and coarse index) from pinned
// host memory to the device: a kernel on the call's stream reads the host
// bytes once over the bus, where a copy-engine transfer made the next kernel
// wait on another engine (10,000-tensor list call: 86.7 against 97.5 us).
__global__ __launch_bounds__(256) void upload_kernel(const u32x4* src, u32x4* dst, int64_t n) {
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * 256)
        dst[i] = src[i];
}

hipError_t launch_upload(void* dst, const void* src, size_t bytes, hipStream_t stream) {
    if (bytes % 16 != 0) return hipErrorInvalidValue;
    const int64_t n = int64_t(bytes / 16);
    if (n == 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 1024);
    hipLaunchKernelGGL(upload_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream,
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n);
    return hipGetLastError();
}

hipError_t launch_gather_list(const ListLaunch& L, int esz, hipStream_t stream) {
    if (L.tiles <= 0) return hipSuccess;
    if (esz == 2) return launch_list_t<uint16_t>(L, esz, stream);
    if (esz == 4) return launch_list_t<float>(L, esz, stream);
    return hipErrorInvalidValue;
}

}  // namespace zsp
