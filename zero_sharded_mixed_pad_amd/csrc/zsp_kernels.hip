// zsp_kernels.hip -- HIP kernels of libzsp for gfx950 (MI355X, CDNA4).
//
// Every kernel here is a stream over HBM with a few fp32 operations per
// byte: no contraction, so no MFMA and no LDS for data. The design points:
//
//  * One wavefront owns one 512-element tile of the index space; lane l
//    handles 8 contiguous elements, so every state array moves as 16- or
//    32-byte vectors per lane (global_load/store_dwordx4), fully coalesced.
//  * The tile's parameter is found from a per-tile table (one or two cached
//    loads), so a launch can span any number of parameters -- thousands of
//    small ones as easily as one large one -- with no per-parameter launch.
//  * Gradient and parameter sources may sit at any 2-byte offset relative to
//    the 8-element groups (each parameter is padded on its own, so slices do
//    not line up). gfx9 global memory serves unaligned dwordx4 loads, so the
//    fast path stays one vector load per 8 elements; only groups that cross
//    a parameter or pad boundary take the per-element path.
//  * The reduce over N_d ranks keeps each lane's 8 sums in registers and adds
//    rank r's values strictly after rank r-1's (fixed order, bit-exact); the
//    ranks are loaded 8 at a time so 8 loads are in flight per lane.
//  * Floating point: built with -ffp-contract=off; division and square root
//    are the default correctly rounded expansions; bf16 narrowing is the
//    hardware round-to-nearest-even convert (v_cvt_pk_bf16_f32).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "zsp_internal.hpp"

namespace zsp {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct __attribute__((packed, aligned(2))) Unaligned16 {
    u32x4 v;
};

__device__ __forceinline__ u32x4 ld16u(const void* p) {
    return reinterpret_cast<const Unaligned16*>(p)->v;
}

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

template <typename GT>
__device__ __forceinline__ void load8(const void* base, int64_t idx, float (&x)[8]) {
    if constexpr (std::is_same<GT, uint16_t>::value) {
        const u32x4 u = ld16u(static_cast<const uint16_t*>(base) + idx);
        x[0] = bf_lo(u.x); x[1] = bf_hi(u.x);
        x[2] = bf_lo(u.y); x[3] = bf_hi(u.y);
        x[4] = bf_lo(u.z); x[5] = bf_hi(u.z);
        x[6] = bf_lo(u.w); x[7] = bf_hi(u.w);
    } else {
        const float* f = static_cast<const float*>(base) + idx;
        const u32x4 a = ld16u(f);
        const u32x4 b = ld16u(f + 4);
        x[0] = __uint_as_float(a.x); x[1] = __uint_as_float(a.y);
        x[2] = __uint_as_float(a.z); x[3] = __uint_as_float(a.w);
        x[4] = __uint_as_float(b.x); x[5] = __uint_as_float(b.y);
        x[6] = __uint_as_float(b.z); x[7] = __uint_as_float(b.w);
    }
}

template <typename GT>
__device__ __forceinline__ float load1(const void* base, int64_t idx) {
    if constexpr (std::is_same<GT, uint16_t>::value)
        return __uint_as_float(uint32_t(static_cast<const uint16_t*>(base)[idx]) << 16);
    else
        return static_cast<const float*>(base)[idx];
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

constexpr bool uses_grads(int op) {
    return op == OP_REDUCE_SET || op == OP_REDUCE_ACC || op == OP_FUSED || op == OP_FUSED_ACC;
}
constexpr bool reads_acc(int op) {
    return op == OP_REDUCE_ACC || op == OP_FUSED_ACC || op == OP_ADAM;
}
constexpr bool is_reduce(int op) { return op == OP_REDUCE_SET || op == OP_REDUCE_ACC; }

// Sum of the N_d ranks' values for 8 contiguous elements, rank order.
template <typename GT, int CAP>
__device__ __forceinline__ void reduce8(const ShardArgs<CAP>& a, int64_t sidx, float (&g)[8]) {
    const int nd = a.nd;
#pragma unroll
    for (int k = 0; k < 8; ++k) g[k] = 0.0f;
    int r0 = 0;
    for (; r0 + 8 <= nd; r0 += 8) {
        float x[8][8];
#pragma unroll
        for (int q = 0; q < 8; ++q) load8<GT>(a.grads[r0 + q], sidx, x[q]);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const bool first = (r0 + q) == 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) g[k] = first ? x[q][k] : g[k] + x[q][k];
        }
    }
    if (r0 < nd) {
        float x[8][8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (r0 + q < nd) load8<GT>(a.grads[r0 + q], sidx, x[q]);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            if (r0 + q < nd) {
                const bool first = (r0 + q) == 0;
#pragma unroll
                for (int k = 0; k < 8; ++k) g[k] = first ? x[q][k] : g[k] + x[q][k];
            }
        }
    }
}

template <typename GT, int CAP>
__device__ __forceinline__ float reduce1(const ShardArgs<CAP>& a, int64_t sidx) {
    float g = load1<GT>(a.grads[0], sidx);
    for (int r = 1; r < a.nd; ++r) g = g + load1<GT>(a.grads[r], sidx);
    return g;
}

__device__ __forceinline__ void st_f32x8(float* p, const float (&x)[8]) {
    f32x4* q = reinterpret_cast<f32x4*>(p);
    q[0] = f32x4{x[0], x[1], x[2], x[3]};
    q[1] = f32x4{x[4], x[5], x[6], x[7]};
}

__device__ __forceinline__ void ld_f32x8(const float* p, float (&x)[8]) {
    const f32x4* q = reinterpret_cast<const f32x4*>(p);
    const f32x4 a = q[0], b = q[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// 8 contiguous, in-range, non-pad elements of one piece starting at E
// (E is a multiple of 8, so every state access is an aligned vector).
template <int OP, typename GT, int CAP>
__device__ __forceinline__ void fast_group(const ShardArgs<CAP>& a, int64_t E,
                                           const PieceInfo& pi) {
    if constexpr (OP == OP_COPYIN) {
        const int64_t s = E + pi.idelta;
        float x[8];
        load8<GT>(a.src, s, x);
        st_f32x8(a.master + E, x);
        u32x4 w;
        if constexpr (std::is_same<GT, uint16_t>::value) {
            w = ld16u(static_cast<const uint16_t*>(a.src) + s);
        } else {
            w = u32x4{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]),
                      pack_bf16(x[6], x[7])};
        }
        *reinterpret_cast<u32x4*>(a.work + E) = w;
        const float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        st_f32x8(a.m + E, z);
        st_f32x8(a.v + E, z);
    } else {
        float g[8];
        if constexpr (uses_grads(OP)) {
            const int64_t s = a.shard_layout ? E : E + pi.gdelta;
            reduce8<GT>(a, s, g);
        }
        if constexpr (reads_acc(OP)) {
            float c[8];
            ld_f32x8(a.acc + E, c);
#pragma unroll
            for (int k = 0; k < 8; ++k) g[k] = (OP == OP_ADAM) ? c[k] : c[k] + g[k];
        }
        if constexpr (is_reduce(OP)) {
            st_f32x8(a.acc + E, g);
        } else {
            float p[8], m[8], v[8];
            ld_f32x8(a.master + E, p);
            ld_f32x8(a.m + E, m);
            ld_f32x8(a.v + E, v);
#pragma unroll
            for (int k = 0; k < 8; ++k) adam1(p[k], m[k], v[k], g[k], a.hp);
            st_f32x8(a.master + E, p);
            st_f32x8(a.m + E, m);
            st_f32x8(a.v + E, v);
            *reinterpret_cast<u32x4*>(a.work + E) =
                u32x4{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]),
                      pack_bf16(p[6], p[7])};
        }
    }
}

// 8 contiguous in-range pad elements.
template <int OP, int CAP>
__device__ __forceinline__ void pad_group(const ShardArgs<CAP>& a, int64_t E) {
    const float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if constexpr (OP == OP_COPYIN) {
        st_f32x8(a.master + E, z);
        st_f32x8(a.m + E, z);
        st_f32x8(a.v + E, z);
        *reinterpret_cast<u32x4*>(a.work + E) = u32x4{0u, 0u, 0u, 0u};
    } else if constexpr (is_reduce(OP)) {
        st_f32x8(a.acc + E, z);
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

template <int OP, typename GT, int CAP>
__global__ __launch_bounds__(kBlockThreads) void shard_kernel(const ShardArgs<CAP> a) {
    const int lane = threadIdx.x & (kWaveLanes - 1);
    const int64_t tile = a.tile_first + int64_t(blockIdx.x) * kWavesPerBlock +
                         (threadIdx.x / kWaveLanes);
    if (tile >= a.tile_end) return;
    const int64_t E = tile * kTile + int64_t(lane) * kElemsPerLane;
    if (E >= a.e_end || E + kElemsPerLane <= a.e_begin) return;

    // Piece holding E: the tile table brackets it, usually to one entry.
    int lo = a.tile[tile];
    int hi = a.tile[tile + 1];
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.e0[mid] <= E) lo = mid;
        else hi = mid - 1;
    }
    int p = lo;
    PieceInfo pi = a.info[p];

    const bool inside = E >= a.e_begin && E + kElemsPerLane <= a.e_end;
    if (inside && E + kElemsPerLane <= pi.vend) {
        fast_group<OP, GT, CAP>(a, E, pi);
    } else if (inside && E >= pi.vend && E + kElemsPerLane <= pi.end) {
        pad_group<OP, CAP>(a, E);
    } else {
        for (int k = 0; k < kElemsPerLane; ++k) {
            const int64_t e = E + k;
            if (e < a.e_begin || e >= a.e_end) continue;
            while (e >= pi.end) pi = a.info[++p];
            elem_op<OP, GT, CAP>(a, e, e < pi.vend, pi);
        }
    }
}

struct GatherArgs {
    const int64_t* k0;
    const int64_t* delta;
    const int32_t* tile;
    int64_t k_first, count;
    const void* src;
    void* out;
};

// out[k] = src[K + delta(piece of K)], K = k_first + k, k < count.
template <typename T>
__global__ __launch_bounds__(kBlockThreads) void gather_kernel(const GatherArgs a) {
    const int lane = threadIdx.x & (kWaveLanes - 1);
    const int64_t kw = (int64_t(blockIdx.x) * kWavesPerBlock + threadIdx.x / kWaveLanes) * kTile;
    if (kw >= a.count) return;
    const int64_t k = kw + int64_t(lane) * kElemsPerLane;
    if (k >= a.count) return;
    const int64_t K = a.k_first + k;
    const int64_t kw_last = a.k_first + min(kw + kTile, a.count) - 1;

    int lo = a.tile[(a.k_first + kw) / kTile];
    int hi = a.tile[kw_last / kTile + 1];
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.k0[mid] <= K) lo = mid;
        else hi = mid - 1;
    }
    int q = lo;
    int64_t next = a.k0[q + 1];
    int64_t d = a.delta[q];
    const T* src = static_cast<const T*>(a.src);
    T* out = static_cast<T*>(a.out);
    if (k + kElemsPerLane <= a.count && K + kElemsPerLane <= next) {
        if constexpr (sizeof(T) == 2) {
            *reinterpret_cast<u32x4*>(out + k) = ld16u(src + K + d);
        } else {
            u32x4* o = reinterpret_cast<u32x4*>(out + k);
            o[0] = ld16u(src + K + d);
            o[1] = ld16u(src + K + d + 4);
        }
    } else {
        for (int i = 0; i < kElemsPerLane; ++i) {
            const int64_t kk = k + i;
            if (kk >= a.count) break;
            const int64_t KK = K + i;
            while (KK >= next) {
                ++q;
                next = a.k0[q + 1];
                d = a.delta[q];
            }
            out[kk] = src[KK + d];
        }
    }
}

template <int OP, typename GT, int CAP>
hipError_t launch_t(const ShardLaunch& L, hipStream_t stream) {
    ShardArgs<CAP> a{};
    a.e0 = L.tab.e0;
    a.info = L.tab.info;
    a.tile = L.tab.tile;
    a.e_begin = L.e_begin;
    a.e_end = L.e_end;
    a.tile_first = L.e_begin / kTile;
    a.tile_end = (L.e_end + kTile - 1) / kTile;
    a.master = L.master;
    a.m = L.m;
    a.v = L.v;
    a.work = L.work;
    a.acc = L.acc;
    a.src = L.src;
    a.hp = L.hp;
    a.nd = L.nd;
    a.shard_layout = L.shard_layout;
    if constexpr (uses_grads(OP)) {
        for (int r = 0; r < L.nd; ++r) a.grads[r] = L.grads[r];
    }
    const int64_t waves = a.tile_end - a.tile_first;
    const int64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((shard_kernel<OP, GT, CAP>), dim3(static_cast<uint32_t>(blocks)),
                       dim3(kBlockThreads), 0, stream, a);
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
    a.k_first = L.k_first;
    a.count = L.count;
    a.src = L.src;
    a.out = L.out;
    const int64_t waves = (L.count + kTile - 1) / kTile;
    const int64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    if (dtype == ZSP_BF16)
        hipLaunchKernelGGL(gather_kernel<uint16_t>, dim3(static_cast<uint32_t>(blocks)),
                           dim3(kBlockThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(gather_kernel<float>, dim3(static_cast<uint32_t>(blocks)),
                           dim3(kBlockThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace zsp
