// Device side of librowred: the shared row-reduction core and the per-operator
// epilogues, written for gfx950 (CDNA4, 64-lane wavefronts).
//
// One worker (lane) of a row owns columns i = (chunk * W + w) * V + e and keeps
// them in private slot chunk * V + e (LuisaCompute notes, "Consecutive-worker
// reduction layout checkpoint", section "Implementation and semantics").
// The same map serves the load, the reduction and the store. When the row is
// an exact multiple of the plan's span every pack is one V-wide access;
// otherwise each pack loads the in-bounds V-wide window nearest to it and
// selects its columns, so no load is guarded by a branch, and stores of the
// one partial pack per worker are guarded element by element. Nothing is read
// or written past the row (meTile "Thread Ownership and Software Staging",
// section "Contiguous register memory": no speculative access beyond a ragged
// tensor).
//
// A row's partials combine in three levels, each in a fixed order so results
// are reproducible run to run:
//   1. a balanced tree over the worker's own slots (meTile page, section
//      "Register-tiled reductions");
//   2. a butterfly inside the row's lane segment of the wavefront: DPP
//      quad permutes and mirrors for distances 1..8, ds_swizzle for 16 and
//      two readlanes for 32 — every lane ends with the same value;
//   3. when a row spans several wavefronts, one float per wavefront in LDS,
//      one barrier, and every wavefront summing all partials itself (meTile
//      page, same section: private reduction scratch needs one barrier;
//      each sequential reduction gets its own scratch).
// Every lane takes part in every reduction; lanes without data contribute the
// operation's identity.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <type_traits>

#include "internal.h"

namespace rowred {

enum OpId { kRmsNorm = 0, kSum = 1, kSoftmax = 2, kLayerNorm = 3, kResidualLayerNorm = 4, kCrossEntropy = 5 };

// Storage types. float rows: packs of V consecutive floats at 4-byte
// alignment (row origins of odd-width rows are only dword aligned; gfx9
// vector memory instructions accept that). bfloat16 rows: packs of V
// bfloat16 loaded as 2V bytes with natural alignment (the planner admits
// V > 1 only when cols is a multiple of V and the pointers are 2V-byte
// aligned), widened to float exactly, and rounded back to nearest-even on
// the store (v_cvt_pk_bf16_f32).
typedef __bf16 bf16_t;
typedef float f32x2u __attribute__((ext_vector_type(2), aligned(4)));
typedef float f32x4u __attribute__((ext_vector_type(4), aligned(4)));
typedef unsigned short u16;
typedef unsigned int u32;
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <class T>
constexpr bool is_bf16 = __is_same(T, bf16_t);

// Cache policy of a launch (rr_plan.cache): rows are touched once, so their
// loads and stores may carry the non-temporal ("nt") hint, which keeps them
// from displacing useful lines and shortens the end-of-kernel write-back.
// Weights are shared by every row and must stay cached: their loads never
// take the hint. HINT bit 0: non-temporal stores; bit 1: non-temporal row
// loads.
constexpr int kHintNtStore = 1;
constexpr int kHintNtLoad = 2;
constexpr int hint_of_cache(int cache) { return cache == 0 ? 0 : (cache == 1 ? kHintNtStore : kHintNtStore | kHintNtLoad); }

// Overloads per access type (a template over the value type would lose the
// float typedefs' 4-byte alignment and assume natural vector alignment).
#define ROWRED_LDST(T)                                                                    \
    template <int HINT, bool STREAM>                                                      \
    __device__ __forceinline__ T ld(const T *p) {                                         \
        if constexpr (STREAM && (HINT & kHintNtLoad)) return __builtin_nontemporal_load(p); \
        else return *p;                                                                   \
    }                                                                                     \
    template <int HINT>                                                                   \
    __device__ __forceinline__ void st(T *p, T v) {                                       \
        if constexpr (HINT & kHintNtStore) __builtin_nontemporal_store(v, p);              \
        else *p = v;                                                                      \
    }
ROWRED_LDST(float)
ROWRED_LDST(f32x2u)
ROWRED_LDST(f32x4u)
ROWRED_LDST(u16)
ROWRED_LDST(u32)
ROWRED_LDST(u32x2)
ROWRED_LDST(u32x4)
#undef ROWRED_LDST

// bfloat16 <-> float: widening is exact (the bits are the float's top half).
__device__ __forceinline__ float u32_as_f32(u32 u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ float bf16_lo(u32 u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16_hi(u32 u) { return __builtin_bit_cast(float, u & 0xffff0000u); }
__device__ __forceinline__ u32 pack_bf16(float a, float b) {
    bf16x2 v;
    v.x = (bf16_t)a;
    v.y = (bf16_t)b;
    return __builtin_bit_cast(u32, v);
}
__device__ __forceinline__ u16 bf16_bits(float a) { return __builtin_bit_cast(u16, (bf16_t)a); }
// The float value of `a` rounded to bfloat16.
__device__ __forceinline__ float round_to_bf16(float a) { return __builtin_bit_cast(float, (u32)bf16_bits(a) << 16); }

// e^d for d <= 0 (a value minus its row maximum) on the hardware base-2
// exponential: 2^(d log2 e). Rounding the product adds at most |d| 2^-24
// relative error to the result, below 1.2e-6 for every term larger than 1e-9
// of the row's largest, on top of the instruction's own 1 ulp; -inf gives 0.
__device__ __forceinline__ float exp_nonpos(float d) { return __builtin_amdgcn_exp2f(d * 1.44269504088896341f); }

template <int V, int HINT = 0, bool STREAM = false>
__device__ __forceinline__ void load_pack(const float *__restrict__ p, float *d);
template <int V, int HINT = 0, bool STREAM = false>
__device__ __forceinline__ void load_pack(const bf16_t *__restrict__ p, float *d);

// Cross-entropy's target logit x[t] of a row, in two steps: the load always
// reads an in-row position (column 0 for a target outside [0, cols)), so no
// branch separates it from the loads around it, and target_or_nan, applied
// where the loss is formed, gives NaN for an out-of-range target. Using the
// value only there keeps the wait for it at the end.
template <class T>
__device__ __forceinline__ float target_raw(const T *row, int t, int cols) {
    float xt;
    load_pack<1>(row + ((t >= 0 && t < cols) ? t : 0), &xt);
    return xt;
}
__device__ __forceinline__ float target_or_nan(float raw, int t, int cols) {
    return (t >= 0 && t < cols) ? raw : __builtin_nanf("");
}

template <int V, int HINT, bool STREAM>
__device__ __forceinline__ void load_pack(const float *__restrict__ p, float *d) {
    if constexpr (V == 1) {
        d[0] = ld<HINT, STREAM>(p);
    } else if constexpr (V == 2) {
        f32x2u t = ld<HINT, STREAM>(reinterpret_cast<const f32x2u *>(p));
        d[0] = t.x;
        d[1] = t.y;
    } else {
        static_assert(V == 4, "float rows: V must be 1, 2 or 4");
        f32x4u t = ld<HINT, STREAM>(reinterpret_cast<const f32x4u *>(p));
        d[0] = t.x;
        d[1] = t.y;
        d[2] = t.z;
        d[3] = t.w;
    }
}

template <int V, int HINT, bool STREAM>
__device__ __forceinline__ void load_pack(const bf16_t *__restrict__ p, float *d) {
    if constexpr (V == 1) {
        d[0] = __builtin_bit_cast(float, (u32)ld<HINT, STREAM>(reinterpret_cast<const u16 *>(p)) << 16);
    } else if constexpr (V == 2) {
        const u32 t = ld<HINT, STREAM>(reinterpret_cast<const u32 *>(p));
        d[0] = bf16_lo(t);
        d[1] = bf16_hi(t);
    } else if constexpr (V == 4) {
        const u32x2 t = ld<HINT, STREAM>(reinterpret_cast<const u32x2 *>(p));
        d[0] = bf16_lo(t.x);
        d[1] = bf16_hi(t.x);
        d[2] = bf16_lo(t.y);
        d[3] = bf16_hi(t.y);
    } else {
        static_assert(V == 8, "bfloat16 rows: V must be 1, 2, 4 or 8");
        const u32x4 t = ld<HINT, STREAM>(reinterpret_cast<const u32x4 *>(p));
        d[0] = bf16_lo(t.x);
        d[1] = bf16_hi(t.x);
        d[2] = bf16_lo(t.y);
        d[3] = bf16_hi(t.y);
        d[4] = bf16_lo(t.z);
        d[5] = bf16_hi(t.z);
        d[6] = bf16_lo(t.w);
        d[7] = bf16_hi(t.w);
    }
}

template <int V, int HINT = 0>
__device__ __forceinline__ void store_pack(float *__restrict__ p, const float *d) {
    if constexpr (V == 1) {
        st<HINT>(p, d[0]);
    } else if constexpr (V == 2) {
        f32x2u t;
        t.x = d[0];
        t.y = d[1];
        st<HINT>(reinterpret_cast<f32x2u *>(p), t);
    } else {
        static_assert(V == 4, "float rows: V must be 1, 2 or 4");
        f32x4u t;
        t.x = d[0];
        t.y = d[1];
        t.z = d[2];
        t.w = d[3];
        st<HINT>(reinterpret_cast<f32x4u *>(p), t);
    }
}

template <int V, int HINT = 0>
__device__ __forceinline__ void store_pack(bf16_t *__restrict__ p, const float *d) {
    if constexpr (V == 1) {
        st<HINT>(reinterpret_cast<u16 *>(p), bf16_bits(d[0]));
    } else if constexpr (V == 2) {
        st<HINT>(reinterpret_cast<u32 *>(p), pack_bf16(d[0], d[1]));
    } else if constexpr (V == 4) {
        u32x2 t;
        t.x = pack_bf16(d[0], d[1]);
        t.y = pack_bf16(d[2], d[3]);
        st<HINT>(reinterpret_cast<u32x2 *>(p), t);
    } else {
        static_assert(V == 8, "bfloat16 rows: V must be 1, 2, 4 or 8");
        u32x4 t;
        t.x = pack_bf16(d[0], d[1]);
        t.y = pack_bf16(d[2], d[3]);
        t.z = pack_bf16(d[4], d[5]);
        t.w = pack_bf16(d[6], d[7]);
        st<HINT>(reinterpret_cast<u32x4 *>(p), t);
    }
}

template <int HINT>
__device__ __forceinline__ void store_one(float *p, float v) { st<HINT>(p, v); }
template <int HINT>
__device__ __forceinline__ void store_one(bf16_t *p, float v) { st<HINT>(reinterpret_cast<u16 *>(p), bf16_bits(v)); }

// Window layout of the pack of V columns that starts at column i0 of a row
// with `cols` columns (cols >= V), read without branches: the V-wide load
// always reads the in-bounds window that starts at window_start(i0, cols) =
// min(i0, cols - V), and slot e holds column window_start + e, which belongs
// to the pack when it is >= i0. A complete pack's window is the pack itself;
// the row's last, partial pack reads the row's final V columns and keeps the
// ones from i0 on; a pack past the row end keeps none. Slots that hold no
// column of the pack get `fill`. Nothing outside the row is read, and each
// slot costs one compare and one select.
template <int V>
__device__ __forceinline__ int window_start(int i0, int cols) { return i0 < cols - V ? i0 : cols - V; }

template <int V, int HINT = 0, bool STREAM = false, class T>
__device__ __forceinline__ void load_window(const T *__restrict__ row, int i0, int cols, float *d,
                                            float fill) {
    const int start = window_start<V>(i0, cols);
    const int lo = i0 - start;  // slots below lo hold columns of earlier packs
    float t[V];
    load_pack<V, HINT, STREAM>(row + start, t);
#pragma unroll
    for (int e = 0; e < V; ++e) d[e] = (e >= lo) ? t[e] : fill;
}

// Store of a pack held in the window layout: only the pack's own columns that
// lie before `end` (the row end, or a slice end on the split path) are written.
template <int V, int HINT = 0, class T>
__device__ __forceinline__ void store_guarded(T *__restrict__ row, int i0, int cols, int end, const float *d) {
    if (i0 + V <= end) {
        store_pack<V, HINT>(row + i0, d);  // complete pack: the window starts at i0
    } else {
        const int start = window_start<V>(i0, cols);
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const int j = start + e;
            if (j >= i0 && j < end) store_one<HINT>(row + j, d[e]);
        }
    }
}

// Load / store of one pack: plain V-wide access when the row is an exact
// multiple of the plan's span (every pack complete), else the guarded forms.
template <int V, bool EXACT, int HINT = 0, bool STREAM = false, class T>
__device__ __forceinline__ void load_slots(const T *__restrict__ row, int i0, int cols, float *d,
                                           float fill) {
    if constexpr (EXACT) load_pack<V, HINT, STREAM>(row + i0, d);
    else load_window<V, HINT, STREAM>(row, i0, cols, d, fill);
}

template <int V, bool EXACT, int HINT = 0, class T>
__device__ __forceinline__ void store_slots(T *__restrict__ row, int i0, int cols, const float *d) {
    if constexpr (EXACT) store_pack<V, HINT>(row + i0, d);
    else store_guarded<V, HINT>(row, i0, cols, cols, d);
}

// ---- combine operations ------------------------------------------------------

struct AddOp {
    template <class T>
    __device__ __forceinline__ T operator()(T a, T b) const { return a + b; }
};
struct MaxOp {
    __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
    __device__ __forceinline__ double operator()(double a, double b) const { return fmax(a, b); }
};

// Balanced tree over K (a power of two) values; overwrites t.
template <int K, class T, class Op>
__device__ __forceinline__ T tree_reduce(T *t, Op op) {
#pragma unroll
    for (int s = K / 2; s > 0; s /= 2) {
#pragma unroll
        for (int k = 0; k < s; ++k) t[k] = op(t[k], t[k + s]);
    }
    return t[0];
}

// ---- cross-lane moves ------------------------------------------------------------

// DPP controls: quad_perm [1,0,3,2] (lane ^ 1), quad_perm [2,3,0,1] (lane ^ 2),
// row_half_mirror (lane i of 8 reads 7 - i), row_mirror (lane i of 16 reads 15 - i).
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
// ds_swizzle bit-mask mode: and 0x1f, or 0, xor 0x10 (lane ^ 16 inside 32).
constexpr int kSwizzleXor16 = (0x10 << 10) | 0x1f;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 0xf, 0xf, false));
}
__device__ __forceinline__ float swizzle_xor16(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), kSwizzleXor16));
}
__device__ __forceinline__ float readlane(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// float64 values move as two 32-bit halves.
struct Halves {
    int lo, hi;
};
__device__ __forceinline__ Halves split(double v) {
    unsigned long long u = __builtin_bit_cast(unsigned long long, v);
    return Halves{(int)(u & 0xffffffffull), (int)(u >> 32)};
}
__device__ __forceinline__ double join(int lo, int hi) {
    unsigned long long u = ((unsigned long long)(unsigned)hi << 32) | (unsigned)lo;
    return __builtin_bit_cast(double, u);
}
template <int CTRL>
__device__ __forceinline__ double dpp(double v) {
    Halves h = split(v);
    return join(__builtin_amdgcn_update_dpp(0, h.lo, CTRL, 0xf, 0xf, false),
                __builtin_amdgcn_update_dpp(0, h.hi, CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ double swizzle_xor16(double v) {
    Halves h = split(v);
    return join(__builtin_amdgcn_ds_swizzle(h.lo, kSwizzleXor16),
                __builtin_amdgcn_ds_swizzle(h.hi, kSwizzleXor16));
}
__device__ __forceinline__ double readlane(double v, int lane) {
    Halves h = split(v);
    return join(__builtin_amdgcn_readlane(h.lo, lane), __builtin_amdgcn_readlane(h.hi, lane));
}

// Two float32 sums reduced together: one butterfly step and one LDS slot
// per wavefront carry both.
struct F2 {
    float a, b;
};
__device__ __forceinline__ F2 operator+(F2 x, F2 y) { return F2{x.a + y.a, x.b + y.b}; }
template <int CTRL>
__device__ __forceinline__ F2 dpp(F2 v) { return F2{dpp<CTRL>(v.a), dpp<CTRL>(v.b)}; }
__device__ __forceinline__ F2 swizzle_xor16(F2 v) { return F2{swizzle_xor16(v.a), swizzle_xor16(v.b)}; }
__device__ __forceinline__ F2 readlane(F2 v, int lane) { return F2{readlane(v.a, lane), readlane(v.b, lane)}; }

// Butterfly over aligned segments of SEG lanes (8, 16, 32 or 64). All lanes
// must be active. Afterwards every lane of a segment holds the same value:
// each step combines a lane with a partner holding the complementary half
// and the operations are commutative.
template <int SEG, class T, class Op>
__device__ __forceinline__ T segment_reduce(T v, Op op) {
    static_assert(SEG == 8 || SEG == 16 || SEG == 32 || SEG == 64, "segment of 8..64 lanes");
    v = op(v, dpp<kDppXor1>(v));
    v = op(v, dpp<kDppXor2>(v));
    v = op(v, dpp<kDppHalfMirror>(v));
    if constexpr (SEG >= 16) v = op(v, dpp<kDppMirror>(v));
    if constexpr (SEG >= 32) v = op(v, swizzle_xor16(v));
    if constexpr (SEG >= 64) v = op(readlane(v, 0), readlane(v, 32));
    return v;
}

// Lanes of one row and where they sit in the workgroup.
template <int SEG>
struct RowLanes {
    int W;            // workers per row
    int lane;         // worker index inside the row
    int row_in_group; // which of the group's rows
    int wave;         // wavefront index inside the group
    int first_wave;   // first wavefront of this row (ROW path)
    int waves;        // wavefronts per row (ROW path)

    __device__ __forceinline__ explicit RowLanes(const Args &a) {
        const int tid = threadIdx.x;
        if constexpr (SEG < 64) {
            W = SEG;
            lane = tid & (SEG - 1);
            row_in_group = tid / SEG;
            waves = 1;
        } else {
            W = a.lanes_per_row;
            lane = tid & (W - 1);
            row_in_group = tid >> a.log2_lanes;
            waves = W >> 6;
        }
        wave = tid >> 6;
        first_wave = row_in_group * waves;
    }
};

// Full row reduction: segment butterfly, then (rows wider than a wavefront)
// one partial per wavefront through `lds`, one barrier, fixed-order sum.
template <int SEG, class T, class Op>
__device__ __forceinline__ T row_reduce(T v, Op op, const RowLanes<SEG> &rl, T *lds) {
    v = segment_reduce<(SEG < 64 ? SEG : 64)>(v, op);
    if constexpr (SEG == 64) {
        if (rl.waves > 1) {
            if ((threadIdx.x & 63) == 0) lds[rl.wave] = v;
            __syncthreads();
            T acc = lds[rl.first_wave];
            for (int j = 1; j < rl.waves; ++j) acc = op(acc, lds[rl.first_wave + j]);
            v = acc;
        }
    }
    return v;
}

// ---- register-resident kernel ---------------------------------------------------
//
// OP: operator; V: floats per pack; NCHUNK: packs per worker (K = V*NCHUNK
// live floats); SEG: lanes per row when < 64 (several rows per wavefront), or
// 64 when a row takes lanes_per_row / 64 whole wavefronts; EXACT: the row
// length equals lanes_per_row * K, so every pack is complete; HINT: cache
// policy bits (see hint_of_cache); T: storage type of rows and weights
// (float or bfloat16; arithmetic is float either way).
template <int OP, int V, int NCHUNK, int SEG, bool EXACT, int HINT, class T>
__global__ void __launch_bounds__(1024) reg_kernel(const Args a) {
    constexpr int K = V * NCHUNK;
    const T *X = static_cast<const T *>(a.x);
    const T *R = static_cast<const T *>(a.residual);
    const T *Wt = static_cast<const T *>(a.w);
    const T *B = static_cast<const T *>(a.beta);
    T *Y = static_cast<T *>(a.y);
    T *H = static_cast<T *>(a.h_out);
    constexpr bool kMaxFirst = (OP == kSoftmax || OP == kCrossEntropy);
    __shared__ float lds0[16];
    __shared__ float lds1[16];
    __shared__ F2 lds2[16];
    __shared__ double ldsd[16];

    const RowLanes<SEG> rl(a);
    const int cols = a.cols;
    const int64_t row_raw = (int64_t)blockIdx.x * a.rows_per_group + rl.row_in_group;
    const bool row_ok = row_raw < a.rows;
    // Lanes of a group's missing last rows mirror the final row and store nothing.
    const int64_t row = row_ok ? row_raw : a.rows - 1;
    const int64_t off = row * (int64_t)cols;
    const int stride = rl.W * V;  // columns per chunk
    const int base = rl.lane * V;
    const float fill = kMaxFirst ? -INFINITY : 0.0f;

    // Cross-entropy: the target index is requested before the row, and the
    // target logit it points to right after the row's loads, so waiting for
    // the index holds back only the logit, not the row (fetching index and
    // logit as a dependent pair ahead of the row measured 2 % slower at
    // 1024x4096 on MI355X, 5 % in bfloat16, 9 % at bfloat16 4096x4096).
    int t_idx = 0;
    if constexpr (OP == kCrossEntropy) t_idx = a.targets[row];

    // ---- load: the worker's K floats stay in registers until the store.
    float v[K];
#pragma unroll
    for (int c = 0; c < NCHUNK; ++c)
        load_slots<V, EXACT, HINT, true>(X + off, c * stride + base, cols, &v[c * V], fill);
    float x_target = 0.0f;
    if constexpr (OP == kCrossEntropy) x_target = target_raw(X + off, t_idx, cols);
    if constexpr (OP == kResidualLayerNorm) {
        float r[K];
#pragma unroll
        for (int c = 0; c < NCHUNK; ++c)
            load_slots<V, EXACT, HINT, true>(R + off, c * stride + base, cols, &r[c * V], 0.0f);
        // h = x + residual at the tensors' precision (bfloat16 rows round it).
#pragma unroll
        for (int k = 0; k < K; ++k) v[k] = is_bf16<T> ? round_to_bf16(v[k] + r[k]) : v[k] + r[k];
        if (H != nullptr && row_ok) {
#pragma unroll
            for (int c = 0; c < NCHUNK; ++c) store_slots<V, EXACT, HINT>(H + off, c * stride + base, cols, &v[c * V]);
        }
    }

    if constexpr (OP == kRmsNorm) {
        float t[K];
#pragma unroll
        for (int k = 0; k < K; ++k) t[k] = v[k] * v[k];
        const float ss = row_reduce(tree_reduce<K>(t, AddOp{}), AddOp{}, rl, lds0);
        const float inv = rsqrtf(ss / (float)cols + a.eps);
        // The weights, which every row reads, are loaded after the reduction
        // rather than with the row: issued at the start, every group asks
        // for the same lines at once while the row loads are in flight
        // (measured on MI355X: 16384x8192 1.4-2 % faster this way, bfloat16
        // 1024x4096 8-15 %, bfloat16 16384x8192 1.4 % slower).
        float wv[K];
#pragma unroll
        for (int c = 0; c < NCHUNK; ++c) load_slots<V, EXACT>(Wt, c * stride + base, cols, &wv[c * V], 0.0f);
        if (row_ok) {
#pragma unroll
            for (int c = 0; c < NCHUNK; ++c) {
                float o[V];
#pragma unroll
                for (int e = 0; e < V; ++e) o[e] = v[c * V + e] * inv * wv[c * V + e];
                store_slots<V, EXACT, HINT>(Y + off, c * stride + base, cols, o);
            }
        }
    } else if constexpr (OP == kSum) {
        double t[K];
#pragma unroll
        for (int k = 0; k < K; ++k) t[k] = (double)v[k];
        const double s = row_reduce(tree_reduce<K>(t, AddOp{}), AddOp{}, rl, ldsd);
        if (row_ok && rl.lane == 0) a.row_out[row] = (float)s;
    } else if constexpr (OP == kSoftmax || OP == kCrossEntropy) {
        float t[K];
#pragma unroll
        for (int k = 0; k < K; ++k) t[k] = v[k];
        const float m = row_reduce(tree_reduce<K>(t, MaxOp{}), MaxOp{}, rl, lds0);
        // Missing columns hold -inf, so exp gives 0 there.
#pragma unroll
        for (int k = 0; k < K; ++k) v[k] = exp_nonpos(v[k] - m);
#pragma unroll
        for (int k = 0; k < K; ++k) t[k] = v[k];
        const float z = row_reduce(tree_reduce<K>(t, AddOp{}), AddOp{}, rl, lds1);
        if constexpr (OP == kSoftmax) {
            const float rz = 1.0f / z;
            if (row_ok) {
#pragma unroll
                for (int c = 0; c < NCHUNK; ++c) {
                    float o[V];
#pragma unroll
                    for (int e = 0; e < V; ++e) o[e] = v[c * V + e] * rz;
                    store_slots<V, EXACT, HINT>(Y + off, c * stride + base, cols, o);
                }
            }
        } else {
            if (row_ok && rl.lane == 0) a.row_out[row] = logf(z) + m - target_or_nan(x_target, t_idx, cols);
        }
    } else {
        static_assert(OP == kLayerNorm || OP == kResidualLayerNorm, "unknown operator");
        // Corrected two-pass statistics: the float32 mean m carries an
        // absolute error near 2^-24 |m|, which (x - mean) / sqrt(var + eps)
        // would amplify when the variance is small next to mean^2. The
        // deviations d = x - m are exact for x near m, so their sum gives
        // the correction c = sum(d) / n and the outputs use d - c; the
        // variance is sum(d^2) / n - c^2. Missing columns hold 0.
        float t[K];
#pragma unroll
        for (int k = 0; k < K; ++k) t[k] = v[k];
        const float m = row_reduce(tree_reduce<K>(t, AddOp{}), AddOp{}, rl, lds0) / (float)cols;
        // Deviations; slots past the row end must not count.
#pragma unroll
        for (int c = 0; c < NCHUNK; ++c) {
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const float d = v[c * V + e] - m;
                const int i0 = c * stride + base;
                v[c * V + e] = (EXACT || window_start<V>(i0, cols) + e >= i0) ? d : 0.0f;
            }
        }
        float t2[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            t[k] = v[k];
            t2[k] = v[k] * v[k];
        }
        // sum(d) and sum(d^2) in one reduction.
        const F2 cq = row_reduce(F2{tree_reduce<K>(t, AddOp{}), tree_reduce<K>(t2, AddOp{})}, AddOp{}, rl, lds2);
        const float corr = cq.a / (float)cols;
        const float q = cq.b / (float)cols;
        const float var = fmaxf(q - corr * corr, 0.0f);
        const float rstd = rsqrtf(var + a.eps);
#pragma unroll
        for (int k = 0; k < K; ++k) v[k] -= corr;
        if (row_ok) {
            // All gamma / beta packs are issued before the first store.
            float g[K], b[K];
#pragma unroll
            for (int c = 0; c < NCHUNK; ++c) {
                load_slots<V, EXACT>(Wt, c * stride + base, cols, &g[c * V], 0.0f);
                load_slots<V, EXACT>(B, c * stride + base, cols, &b[c * V], 0.0f);
            }
#pragma unroll
            for (int c = 0; c < NCHUNK; ++c) {
                float o[V];
#pragma unroll
                for (int e = 0; e < V; ++e) o[e] = v[c * V + e] * rstd * g[c * V + e] + b[c * V + e];
                store_slots<V, EXACT, HINT>(Y + off, c * stride + base, cols, o);
            }
        }
    }
}

// The value h (x, or x + residual at the tensors' precision) at flat position
// `pos`, read by every lane: the shift of the LayerNorms' sums (the row's
// first value on the streaming path, the slice's first value on the split
// path).
template <int OP, class T>
__device__ __forceinline__ float value_at(const Args &a, int64_t pos) {
    float h0;
    load_pack<1>(static_cast<const T *>(a.x) + pos, &h0);
    if constexpr (OP == kResidualLayerNorm) {
        float r0;
        load_pack<1>(static_cast<const T *>(a.residual) + pos, &r0);
        h0 = is_bf16<T> ? round_to_bf16(h0 + r0) : h0 + r0;
    }
    return h0;
}

// ---- streaming kernel for rows beyond the register budget ------------------------
//
// One row per workgroup, W = blockDim.x workers, the same ownership map with as
// many chunks as the row needs. Statistics take a single pass: softmax and
// cross-entropy keep a running (max, sum of exp) per lane, rescaling the sum
// when the max grows; LayerNorm merges each pack's (count, mean, M2) of the
// values shifted by the row's first value h0 (Chan's formula) and keeps a
// float64 running sum for the exact mean; lanes then merge in a fixed order.
// Passes over the row: RMSNorm 2, softmax 2, LayerNorm 2, cross-entropy 1,
// row sum 1. The first KEEP chunks of a lane (KEEP * V register slots) stay
// in registers between the two passes, and the next LDSC chunks in LDS, so
// the second pass re-reads only the rest of the row; every pack is read in
// bounds (a pack past the row end reads the row's last window and keeps none
// of it).
template <int OP, int V, int KEEP, int LDSC, int HINT, class T, bool DMA = false>
__device__ __forceinline__ void loop_row(const Args &a, const int64_t row) {
    const T *Wt = static_cast<const T *>(a.w);
    const T *B = static_cast<const T *>(a.beta);
    T *Y = static_cast<T *>(a.y);
    __shared__ float lds0[16];
    __shared__ float lds1[16];
    __shared__ double ldsd[16];
    __shared__ double ldsd2[16];
    const RowLanes<64> rl(a);
    const int cols = a.cols;
    const int64_t off = row * (int64_t)cols;
    const int stride = rl.W * V;
    const int base = rl.lane * V;
    const int nchunk = (cols + stride - 1) / stride;
    const T *xr = static_cast<const T *>(a.x) + off;
    const T *rr = (OP == kResidualLayerNorm) ? static_cast<const T *>(a.residual) + off : nullptr;
    constexpr int kKeep = KEEP > 0 ? KEEP * V : 1;
    float keep[kKeep];  // chunks 0 .. KEEP-1 of this lane
    // Chunks KEEP .. KEEP+LDSC-1 of this lane, in LDS (1024-lane groups only;
    // each lane reads back only the words it wrote, so no barrier is needed).
    // DMA: the chunks go from memory straight to LDS (global_load_lds, 16
    // bytes per lane, each wave's 64 lanes into one contiguous KiB), all of
    // them in flight at once with no registers held; each lane then reads its
    // own 16 bytes back. Only for 16-byte packs whose every window start is
    // 16-byte aligned, and one input row (not residual LayerNorm).
    static_assert(!DMA || (LDSC > 0 && V * sizeof(T) == 16 && OP != kResidualLayerNorm && KEEP * V <= 64),
                  "direct-to-LDS chunks: 16-byte packs of one input, at most 64 kept slots");
    // Register route: bfloat16 rows beside at most 64 register slots keep
    // these chunks as bfloat16 pairs, one 32-bit word per two values
    // (lossless: what is kept, x or h = bf16(x + residual), and the fill
    // values are bfloat16 numbers); float rows, and softmax beside 96 slots
    // (whose instance would spill with the packing), keep floats.
    constexpr bool kPacked = is_bf16<T> && !DMA && KEEP * V <= 64;
    __shared__ float lds_keep[(LDSC > 0 && !DMA && !kPacked) ? LDSC * V * 1024 : 1];
    __shared__ u32 lds_pk[(LDSC > 0 && kPacked) ? LDSC * (V / 2) * 1024 : 1];
    __shared__ u32x4 lds_dma[(LDSC > 0 && DMA) ? LDSC * 1024 : 1];
    static_assert(LDSC * 1024 * (DMA ? 16 : kPacked ? 2 * V : 4 * V) <= 144 * 1024,
                  "LDS-kept chunks: at most 144 KiB");
    auto lds_put = [&](int c, const float *d) {
        if constexpr (kPacked) {
#pragma unroll
            for (int e = 0; e < V / 2; ++e)
                lds_pk[((c - KEEP) * (V / 2) + e) * 1024 + threadIdx.x] = pack_bf16(d[2 * e], d[2 * e + 1]);
        } else {
#pragma unroll
            for (int e = 0; e < V; ++e) lds_keep[((c - KEEP) * V + e) * 1024 + threadIdx.x] = d[e];
        }
    };
    auto lds_get = [&](int c, float *d) {
        if constexpr (kPacked) {
#pragma unroll
            for (int e = 0; e < V / 2; ++e) {
                const u32 u = lds_pk[((c - KEEP) * (V / 2) + e) * 1024 + threadIdx.x];
                d[2 * e] = bf16_lo(u);
                d[2 * e + 1] = bf16_hi(u);
            }
        } else {
#pragma unroll
            for (int e = 0; e < V; ++e) d[e] = lds_keep[((c - KEEP) * V + e) * 1024 + threadIdx.x];
        }
    };
    const int ldsc = LDSC < nchunk - KEEP ? LDSC : (nchunk - KEEP > 0 ? nchunk - KEEP : 0);

    // Pack of the row's values (x, or x + residual for residual LayerNorm).
    // The last pass over the row may stream it past the caches (cache policy
    // 2); an earlier pass loads it normally so that the re-read can still
    // find it in the last-level cache.
    auto read_pass = [&](auto last, int i0, float *d, float fill) {
        constexpr bool kLast = decltype(last)::value;
        load_window<V, HINT, kLast>(xr, i0, cols, d, fill);
        if constexpr (OP == kResidualLayerNorm) {
            float r[V];
            load_window<V, HINT, kLast>(rr, i0, cols, r, 0.0f);
#pragma unroll
            for (int e = 0; e < V; ++e) d[e] = is_bf16<T> ? round_to_bf16(d[e] + r[e]) : d[e] + r[e];
        }
    };
    auto read_first = [&](int i0, float *d, float fill) { read_pass(std::false_type{}, i0, d, fill); };
    auto read = [&](int i0, float *d, float fill) { read_pass(std::true_type{}, i0, d, fill); };
    // First pass over the LDS-kept chunks: each is loaded, visited and
    // written to LDS. With one 1024-lane group per compute unit, one load in
    // flight per lane would leave the memory system idle between chunks, so
    // kLdsBatch chunks are loaded together where the registers allow it
    // (4 for LayerNorm's 32 kept slots, 2 for residual LayerNorm and for 64
    // slots, 1 beside the 96-slot softmax plan).
    constexpr int kLdsBatch = (KEEP * V <= 32 && OP != kResidualLayerNorm) ? 4 : (KEEP * V <= 64 ? 2 : 1);
    // The chunks beyond the kept ones, streamed in the first pass and re-read
    // in the second: with the group alone on its compute unit (LDS in use),
    // kLdsBatch (first pass) or 2 (second pass) loads are kept in flight.
    constexpr int kStreamBatch1 = LDSC > 0 ? kLdsBatch : 1;
    constexpr int kStreamBatch2 = (LDSC > 0 && kLdsBatch > 1) ? 2 : 1;
    auto stream_first = [&](auto visit, float fill) {
        int c = KEEP + ldsc;
        if constexpr (kStreamBatch1 > 1) {
            for (; c + kStreamBatch1 <= nchunk; c += kStreamBatch1) {
                float d[kStreamBatch1][V];
#pragma unroll
                for (int j = 0; j < kStreamBatch1; ++j) read_first((c + j) * stride + base, d[j], fill);
#pragma unroll
                for (int j = 0; j < kStreamBatch1; ++j) visit((c + j) * stride + base, d[j]);
            }
        }
        for (; c < nchunk; ++c) {
            float d[V];
            read_first(c * stride + base, d, fill);
            visit(c * stride + base, d);
        }
    };
    auto stream_second = [&](auto emit, float fill) {
        int c = KEEP + ldsc;
        if constexpr (kStreamBatch2 > 1) {
            for (; c + kStreamBatch2 <= nchunk; c += kStreamBatch2) {
                float d[kStreamBatch2][V];
#pragma unroll
                for (int j = 0; j < kStreamBatch2; ++j) read((c + j) * stride + base, d[j], fill);
#pragma unroll
                for (int j = 0; j < kStreamBatch2; ++j) emit((c + j) * stride + base, d[j]);
            }
        }
        for (; c < nchunk; ++c) {
            float d[V];
            read(c * stride + base, d, fill);
            emit(c * stride + base, d);
        }
    };
    // DMA form: issue every LDS chunk's load, then (after the kept chunks are
    // visited) read each back in the window layout (slots below the pack get
    // `fill`).
    auto dma_issue = [&] {
        if constexpr (DMA) {
            for (int c = KEEP; c < KEEP + ldsc; ++c) {
                const int start = window_start<V>(c * stride + base, cols);
                __builtin_amdgcn_global_load_lds(
                    (const __attribute__((address_space(1))) void *)(const void *)(xr + start),
                    (__attribute__((address_space(3))) void *)(void *)&lds_dma[(c - KEEP) * 1024 + (threadIdx.x & ~63u)],
                    16, 0, (HINT & kHintNtLoad) ? 2 : 0);
            }
        }
    };
    auto dma_read = [&](int c, float *d, float fill) {
        if constexpr (DMA) {
            const int i0 = c * stride + base;
            const int lo = i0 - window_start<V>(i0, cols);
            const u32x4 t = lds_dma[(c - KEEP) * 1024 + threadIdx.x];
            float v[V];
            if constexpr (is_bf16<T>) {
                v[0] = bf16_lo(t.x); v[1] = bf16_hi(t.x); v[2] = bf16_lo(t.y); v[3] = bf16_hi(t.y);
                v[4] = bf16_lo(t.z); v[5] = bf16_hi(t.z); v[6] = bf16_lo(t.w); v[7] = bf16_hi(t.w);
            } else {
                // Through a u32 value: a bit cast applied to a vector
                // element directly reads the vector's first element with
                // this compiler.
                v[0] = u32_as_f32(t.x); v[1] = u32_as_f32(t.y);
                v[2] = u32_as_f32(t.z); v[3] = u32_as_f32(t.w);
            }
#pragma unroll
            for (int e = 0; e < V; ++e) d[e] = (e >= lo) ? v[e] : fill;
        }
    };
    auto lds_chunks = [&](auto visit, float fill) {
        if constexpr (DMA) {
            // The compiler does not order LDS reads after these DMA loads
            // (measured: without this wait the reads return what LDS held
            // before), so wait for every outstanding vector memory operation
            // of the wave: vmcnt 0, expcnt and lgkmcnt left at their maxima.
            __builtin_amdgcn_s_waitcnt(0x0F70);
            asm volatile("" ::: "memory");
            for (int c = KEEP; c < KEEP + ldsc; ++c) {
                float d[V];
                dma_read(c, d, fill);
                visit(c * stride + base, d);
            }
            return;
        }
        int c = KEEP;
        if constexpr (LDSC > 0 && kLdsBatch > 1) {
            for (; c + kLdsBatch <= KEEP + ldsc; c += kLdsBatch) {
                float d[kLdsBatch][V];
#pragma unroll
                for (int j = 0; j < kLdsBatch; ++j) read_first((c + j) * stride + base, d[j], fill);
#pragma unroll
                for (int j = 0; j < kLdsBatch; ++j) {
                    visit((c + j) * stride + base, d[j]);
                    lds_put(c + j, d[j]);
                }
            }
        }
        for (; c < KEEP + ldsc; ++c) {
            float d[V];
            read_first(c * stride + base, d, fill);
            visit(c * stride + base, d);
            lds_put(c, d);
        }
    };
    // Softmax's first pass: the kept chunks are loaded into `keep` and handed
    // to visit_kept together, then the others are loaded into `d` and
    // visited one by one.
    auto first_pass_kept_together = [&](auto visit_kept, auto visit, float fill) {
#pragma unroll
        for (int c = 0; c < KEEP; ++c) read_first(c * stride + base, &keep[c * V], fill);
        dma_issue();
        visit_kept();
        lds_chunks(visit, fill);
        stream_first(visit, fill);
    };
    auto first_pass = [&](auto visit, float fill) {
#pragma unroll
        for (int c = 0; c < KEEP; ++c) read_first(c * stride + base, &keep[c * V], fill);
        dma_issue();
#pragma unroll
        for (int c = 0; c < KEEP; ++c) visit(c * stride + base, &keep[c * V]);
        lds_chunks(visit, fill);
        stream_first(visit, fill);
    };
    // Second pass: kept chunks come from registers (emit_kept), the others
    // are re-read (emit).
    auto second_pass_split = [&](auto emit_kept, auto emit, float fill) {
        // The kept chunks' column offsets are recomputed here from an opaque
        // copy of `base`, rather than held in registers from the first pass
        // alongside the kept values.
        int base2 = base;
        asm volatile("" : "+v"(base2));
#pragma unroll
        for (int c = 0; c < KEEP; ++c) {
            if (c < nchunk) {
                float d[V];
#pragma unroll
                for (int e = 0; e < V; ++e) d[e] = keep[c * V + e];
                emit_kept(c * stride + base2, d);
            }
        }
        for (int c = KEEP; c < KEEP + ldsc; ++c) {
            float d[V];
            if constexpr (DMA) {
                dma_read(c, d, fill);
            } else {
                lds_get(c, d);
            }
            emit(c * stride + base, d);
        }
        stream_second(emit, fill);
    };
    auto second_pass = [&](auto emit, float fill) {
#pragma unroll
        for (int c = 0; c < KEEP; ++c) {
            if (c < nchunk) {
                float d[V];
#pragma unroll
                for (int e = 0; e < V; ++e) d[e] = keep[c * V + e];
                emit(c * stride + base, d);
            }
        }
        for (int c = KEEP; c < KEEP + ldsc; ++c) {
            float d[V];
            if constexpr (DMA) {
                dma_read(c, d, fill);
            } else {
                lds_get(c, d);
            }
            emit(c * stride + base, d);
        }
        stream_second(emit, fill);
    };

    // Second pass of the LayerNorms, whose outputs need gamma and beta. Each
    // chunk's output needs AV weight values (load_aux), and
    // the stores of a chunk keep the compiler from issuing later chunks'
    // weight loads before them (they might alias), so a chunk-by-chunk pass
    // waits one cache round trip per chunk. Here the weights of a batch of
    // chunks are issued before any of that batch is stored: NBK chunks at a
    // time among the register-kept ones, NBL among the LDS-kept ones, NBS
    // among the streamed ones (whose row values are read in the same batch).
    auto second_pass_w = [&](auto nbk, auto nbl, auto nbs, auto av, auto load_aux, auto emit, float fill) {
        constexpr int NBK = decltype(nbk)::value, NBL = decltype(nbl)::value, NBS = decltype(nbs)::value;
        constexpr int AV = decltype(av)::value;
        // Kept chunks' offsets recomputed from an opaque copy of `base`
        // rather than held in registers since the first pass.
        int base2 = base;
        asm volatile("" : "+v"(base2));
#pragma unroll
        for (int c0 = 0; c0 < KEEP; c0 += NBK) {
            float aux[NBK][AV];
#pragma unroll
            for (int j = 0; j < NBK; ++j)
                if (c0 + j < KEEP && c0 + j < nchunk) load_aux((c0 + j) * stride + base2, aux[j]);
            // Keep the scheduler from moving the batch's arithmetic up between
            // its loads (it would reuse their registers and wait on each).
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < NBK; ++j) {
                if (c0 + j < KEEP && c0 + j < nchunk) {
                    float d[V];
#pragma unroll
                    for (int e = 0; e < V; ++e) d[e] = keep[(c0 + j) * V + e];
                    emit((c0 + j) * stride + base2, d, aux[j]);
                }
            }
        }
        auto lds_chunk = [&](int c, float *d) {
            if constexpr (DMA) {
                dma_read(c, d, fill);
            } else {
                lds_get(c, d);
            }
        };
        int c = KEEP;
        if constexpr (LDSC > 0) {
            for (; c + NBL <= KEEP + ldsc; c += NBL) {
                float aux[NBL][AV];
#pragma unroll
                for (int j = 0; j < NBL; ++j) load_aux((c + j) * stride + base, aux[j]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < NBL; ++j) {
                    float d[V];
                    lds_chunk(c + j, d);
                    emit((c + j) * stride + base, d, aux[j]);
                }
            }
            for (; c < KEEP + ldsc; ++c) {
                float aux[AV], d[V];
                load_aux(c * stride + base, aux);
                lds_chunk(c, d);
                emit(c * stride + base, d, aux);
            }
        }
        for (; c + NBS <= nchunk; c += NBS) {
            float d[NBS][V], aux[NBS][AV];
#pragma unroll
            for (int j = 0; j < NBS; ++j) read((c + j) * stride + base, d[j], fill);
#pragma unroll
            for (int j = 0; j < NBS; ++j) load_aux((c + j) * stride + base, aux[j]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < NBS; ++j) emit((c + j) * stride + base, d[j], aux[j]);
        }
        for (; c < nchunk; ++c) {
            float d[V], aux[AV];
            read(c * stride + base, d, fill);
            load_aux(c * stride + base, aux);
            emit(c * stride + base, d, aux);
        }
    };
    // Batches of at most 32 weight values (4 chunks of gamma and beta at
    // V = 4, 2 at V = 8), and streamed batches of at most 32 row and weight
    // values together (LayerNorm 4096x65536: float 0.5-1 % faster than
    // chunk by chunk, residual 1 %, bfloat16 1.5-2.2 %).
    auto weighted_pass = [&](auto av, auto load_aux, auto emit, float fill) {
        constexpr int AV = decltype(av)::value;
        constexpr int NB = 32 / AV < 1 ? 1 : (32 / AV > 4 ? 4 : 32 / AV);
        constexpr int NS = 32 / (V + AV) < 1 ? 1 : (32 / (V + AV) > 2 ? 2 : 32 / (V + AV));
        second_pass_w(std::integral_constant<int, NB>{}, std::integral_constant<int, NB>{},
                      std::integral_constant<int, NS>{}, av, load_aux, emit, fill);
    };

    if constexpr (OP == kRmsNorm) {
        float acc = 0.0f;
        first_pass([&](int, const float *d) {
            float t[V];
#pragma unroll
            for (int e = 0; e < V; ++e) t[e] = d[e] * d[e];
            acc += tree_reduce<V>(t, AddOp{});
        }, 0.0f);
        const float ss = row_reduce(acc, AddOp{}, rl, lds0);
        const float inv = rsqrtf(ss / (float)cols + a.eps);
        // Chunk by chunk: batching the weight loads as the LayerNorms do
        // measured 5 % slower here (4096x65536, float and bfloat16).
        second_pass([&](int i0, float *d) {
            float wv[V];
            load_window<V>(Wt, i0, cols, wv, 0.0f);
#pragma unroll
            for (int e = 0; e < V; ++e) d[e] = d[e] * inv * wv[e];
            store_guarded<V, HINT>(Y + off, i0, cols, cols, d);
        }, 0.0f);
    } else if constexpr (OP == kSum) {
        static_assert(KEEP == 0, "one pass: nothing to keep");
        double acc = 0.0;
        for (int c = 0; c < nchunk; ++c) {
            float d[V];
            read(c * stride + base, d, 0.0f);
            double t[V];
#pragma unroll
            for (int e = 0; e < V; ++e) t[e] = (double)d[e];
            acc += tree_reduce<V>(t, AddOp{});
        }
        const double s = row_reduce(acc, AddOp{}, rl, ldsd);
        if (rl.lane == 0) a.row_out[row] = (float)s;
    } else if constexpr (OP == kSoftmax || OP == kCrossEntropy) {
        static_assert(OP == kSoftmax || KEEP == 0, "one pass: nothing to keep");
        float m = -INFINITY, z = 0.0f;  // running max and sum of exp(x - m)
        auto visit = [&](int, const float *d) {
            float t[V];
#pragma unroll
            for (int e = 0; e < V; ++e) t[e] = d[e];
            const float mn = fmaxf(m, tree_reduce<V>(t, MaxOp{}));
            if (mn != -INFINITY) {  // missing columns hold -inf: exp gives 0
#pragma unroll
                for (int e = 0; e < V; ++e) t[e] = exp_nonpos(d[e] - mn);
                z = z * exp_nonpos(m - mn) + tree_reduce<V>(t, AddOp{});
                m = mn;
            }
        };
        // Softmax keeps exp(x - mk) rather than x in its register chunks, mk
        // being the lane's max over them, so the second pass scales them by
        // one factor instead of exponentiating again. They enter the online
        // (max, sum) first, as one pack: -inf (masked or missing columns)
        // becomes 0, NaN stays NaN.
        float mk = -INFINITY;
        if constexpr (OP == kSoftmax) {
            first_pass_kept_together([&] {
                if constexpr (KEEP > 0) {
                    static_assert(kKeep % 4 == 0, "kept slots fold into four accumulators");
                    float acc[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[j] = keep[j];
#pragma unroll
                    for (int i = 4; i < kKeep; ++i) acc[i % 4] = fmaxf(acc[i % 4], keep[i]);
                    mk = tree_reduce<4>(acc, MaxOp{});
                    // With mk = -inf every kept value is -inf (exp gives 0)
                    // or NaN, so any finite reference serves.
                    const float ref = mk == -INFINITY ? 0.0f : mk;
#pragma unroll
                    for (int i = 0; i < kKeep; ++i) keep[i] = exp_nonpos(keep[i] - ref);
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[j] = keep[j];
#pragma unroll
                    for (int i = 4; i < kKeep; ++i) acc[i % 4] += keep[i];
                    const float zk = tree_reduce<4>(acc, AddOp{});
                    const float mn = fmaxf(m, mk);
                    z = (m == -INFINITY ? 0.0f : z * exp_nonpos(m - mn)) +
                        (mk == -INFINITY ? 0.0f : zk * exp_nonpos(mk - mn));
                    m = mn;
                }
            }, visit, -INFINITY);
        } else {
            // Two packs per (max, sum) update: one rescaling exponential and
            // one max merge per 2V values instead of per V (cross-entropy
            // 2048x128256 -1 %, bf16 -1.5 to -5 %; four or eight packs measured
            // the same or slower).
            constexpr int U = 2;
            auto visit_u = [&](const float *d) {
                float t[U * V];
#pragma unroll
                for (int e = 0; e < U * V; ++e) t[e] = d[e];
                const float mn = fmaxf(m, tree_reduce<U * V>(t, MaxOp{}));
                if (mn != -INFINITY) {
#pragma unroll
                    for (int e = 0; e < U * V; ++e) t[e] = exp_nonpos(d[e] - mn);
                    z = z * exp_nonpos(m - mn) + tree_reduce<U * V>(t, AddOp{});
                    m = mn;
                }
            };
            int c = 0;
            for (; c + U <= nchunk; c += U) {
                float d[U * V];
#pragma unroll
                for (int u = 0; u < U; ++u) read((c + u) * stride + base, d + u * V, -INFINITY);
                visit_u(d);
            }
            for (; c < nchunk; ++c) {
                float d[V];
                read(c * stride + base, d, -INFINITY);
                visit(0, d);
            }
        }
        const float mrow = row_reduce(m, MaxOp{}, rl, lds0);
        const float zrow = row_reduce(m == -INFINITY ? 0.0f : z * exp_nonpos(m - mrow), AddOp{}, rl, lds1);
        if constexpr (OP == kSoftmax) {
            const float rz = 1.0f / zrow;
            // exp(x - mrow) / z for the kept chunks: their exp(x - mk) times
            // exp(mk - mrow) / z (0 where mk is -inf and the row is not).
            const float sk = exp_nonpos(mk - mrow) * rz;
            second_pass_split([&](int i0, float *d) {
#pragma unroll
                for (int e = 0; e < V; ++e) d[e] = d[e] * sk;
                store_guarded<V, HINT>(Y + off, i0, cols, cols, d);
            }, [&](int i0, float *d) {
#pragma unroll
                for (int e = 0; e < V; ++e) d[e] = exp_nonpos(d[e] - mrow) * rz;
                store_guarded<V, HINT>(Y + off, i0, cols, cols, d);
            }, -INFINITY);
        } else {
            // The target index and logit are fetched here, after the row:
            // requesting them before the first chunks (the index first, the
            // logit after two chunks) measured no faster on MI355X
            // (2048x128256, 8192x32769, float and bfloat16).
            if (rl.lane == 0) {
                const int t = a.targets[row];
                a.row_out[row] = logf(zrow) + mrow - target_or_nan(target_raw(xr, t, cols), t, cols);
            }
        }
    } else {
        static_assert(OP == kLayerNorm || OP == kResidualLayerNorm, "unknown operator");
        // Per lane, one pass over u = h - h0, the values shifted by the row's
        // first value h0: a running (count, mean, M2) merged pack by pack
        // with Chan's formula (the pack deviations and mean differences it
        // forms are exact for nearby values, so the lane's M2 stays accurate
        // in float32), and a float64 running sum of the packs' float32 sums
        // of u. The shift is what keeps this accurate when the variance is
        // small next to mean^2: u is of the order of the row's spread, not of
        // its mean, so the float32 sums and the running mean round at that
        // scale, and the row mean h0 + sum(u) / n the outputs subtract is
        // accurate to it. (An unshifted float32 mean would carry an error
        // near 2^-24 |mean| into every deviation, which (x - mean) /
        // sqrt(var + eps) amplifies.) Chan's weights k / (n + k) use the
        // hardware reciprocal: a 1-ulp error in a weight moves the merged
        // mean and M2 by far less than their own rounding.
        const float h0 = value_at<OP, T>(a, off);
        float n = 0.0f, mean = 0.0f, m2 = 0.0f;
        double sum = 0.0;
        // One pack: its values' shifted mean and M2 merged into the lane's
        // (count, mean, M2), and their shifted sum added to the float64
        // sum. FULL: all V columns lie in the row (every pack but the row's
        // last), so nothing is masked.
        auto add_pack = [&](auto full, int i0, const float *d, float k) {
            constexpr bool kFull = decltype(full)::value;
            const int start = window_start<V>(i0, cols);
            float t[V], u[V];
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const bool in = kFull || start + e >= i0;
                u[e] = in ? d[e] - h0 : 0.0f;
                t[e] = u[e];
            }
            const float ps = tree_reduce<V>(t, AddOp{});
            sum += (double)ps;
            const float pm = ps / k;
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const float dv = u[e] - pm;
                t[e] = (kFull || start + e >= i0) ? dv * dv : 0.0f;
            }
            const float pm2 = tree_reduce<V>(t, AddOp{});
            const float nn = n + k;
            const float delta = pm - mean;
            const float wk = k * __builtin_amdgcn_rcpf(nn);
            mean += delta * wk;
            m2 += pm2 + delta * delta * (n * wk);
            n = nn;
        };
        first_pass([&](int i0, const float *d) {
            const int left = cols - i0;
            if (left >= V) add_pack(std::true_type{}, i0, d, (float)V);
            else if (left > 0) add_pack(std::false_type{}, i0, d, (float)left);
        }, 0.0f);
        // Row mean (minus h0) from the float64 sums; the between-lane part of
        // the variance from each lane's mean (its float64 sum over its
        // count), in float64. The outputs take (h - h0) - mean in float32.
        const double rmean = row_reduce(sum, AddOp{}, rl, ldsd) / (double)cols;
        const double dv = n > 0.0f ? sum / (double)n - rmean : 0.0;  // lane mean minus row mean
        const double var = row_reduce((double)m2 + (double)n * dv * dv, AddOp{}, rl, ldsd2) / (double)cols;
        const float rstd = (float)(1.0 / sqrt(var + (double)a.eps));
        const float mu = (float)rmean;  // row mean minus h0
        T *hr = (OP == kResidualLayerNorm && a.h_out != nullptr) ? static_cast<T *>(a.h_out) + off : nullptr;
        // aux holds gamma (first V values) then beta.
        weighted_pass(std::integral_constant<int, 2 * V>{},
                      [&](int i0, float *gb) {  // windows as is, as for RMSNorm's w
                          const int st = window_start<V>(i0, cols);
                          load_pack<V>(Wt + st, gb);
                          load_pack<V>(B + st, gb + V);
                      },
                      [&](int i0, float *d, const float *gb) {
            if (hr != nullptr) store_guarded<V, HINT>(hr, i0, cols, cols, d);
#pragma unroll
            for (int e = 0; e < V; ++e) d[e] = ((d[e] - h0) - mu) * rstd * gb[e] + gb[V + e];
            store_guarded<V, HINT>(Y + off, i0, cols, cols, d);
        }, 0.0f);
    }
}

template <int OP, int V, int KEEP, int LDSC, int HINT, class T, bool DMA>
__global__ void __launch_bounds__(1024) loop_kernel(const Args a) {
    loop_row<OP, V, KEEP, LDSC, HINT, T, DMA>(a, blockIdx.x);
}

// ---- split rows: several workgroups per row ---------------------------------------
//
// For rows longer than one workgroup's register budget when there are too few
// rows to fill the chip. Row r is cut into S slices of W*K columns; workgroup
// (s, r) keeps slice s in registers (same ownership map inside the slice) and
// writes one partial per (row, slice) to the caller's workspace; a second
// launch merges the row's S partials in slice order (float64), re-reads its
// slice and writes the outputs. Partials:
//   RMSNorm: (sum x^2, -)          row sum: (sum x, -)
//   softmax / cross-entropy: (slice max m, sum exp(x - m))
//   LayerNorm: the slice's mean and M2 = sum (h - mean)^2, in float64, from
//   sums of h - c shifted by the slice's own first value c (so they round at
//   the scale of the row's spread, not of its mean); merged with Chan's
//   formula for combining (count, mean, M2) groups. The second launch reads
//   no input outside its own slice, so y may alias x: a shift shared by the
//   whole row would have to be re-read from x[row, 0], which the slice-0
//   workgroup of that launch may already have overwritten.

struct Partial2 {
    double a, b;
};

// Columns of slice s: [s * span, min((s + 1) * span, cols)).
__device__ __forceinline__ int slice_len(int s, int span, int cols) {
    const int left = cols - s * span;
    return left < span ? left : span;
}

template <int OP, int V, int NCHUNK, int HINT, class T>
__global__ void __launch_bounds__(1024) split_partial_kernel(const Args a) {
    constexpr int K = V * NCHUNK;
    __shared__ float lds0[16];
    __shared__ float lds1[16];
    __shared__ double ldsd[16];
    __shared__ double ldsd2[16];
    const RowLanes<64> rl(a);
    const int cols = a.cols;
    const int s = blockIdx.x;
    const int64_t row = blockIdx.y;
    const int64_t off = row * (int64_t)cols;
    const int span = rl.W * K;
    const int first = s * span;
    const int stride = rl.W * V;
    const int base = first + rl.lane * V;
    const T *xr = static_cast<const T *>(a.x) + off;
    constexpr bool kMaxFirst = (OP == kSoftmax || OP == kCrossEntropy);
    const float fill = kMaxFirst ? -INFINITY : 0.0f;
    const int end = first + slice_len(s, span, cols);  // slice end (exclusive)

    float v[K];
#pragma unroll
    for (int c = 0; c < NCHUNK; ++c) {
        const int i0 = c * stride + base;
        load_window<V, HINT, true>(xr, i0, cols, &v[c * V], fill);
        // Columns of the next slice belong to it, not to this one.
        const int start = window_start<V>(i0, cols);
#pragma unroll
        for (int e = 0; e < V; ++e)
            if (start + e >= end) v[c * V + e] = fill;
    }
    if constexpr (OP == kResidualLayerNorm) {
        const T *rr = static_cast<const T *>(a.residual) + off;
        T *hr = a.h_out ? static_cast<T *>(a.h_out) + off : nullptr;
#pragma unroll
        for (int c = 0; c < NCHUNK; ++c) {
            float r[V];
            const int i0 = c * stride + base;
            load_window<V, HINT, true>(rr, i0, cols, r, 0.0f);
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const float h = is_bf16<T> ? round_to_bf16(v[c * V + e] + r[e]) : v[c * V + e] + r[e];
                const int j = window_start<V>(i0, cols) + e;
                v[c * V + e] = (j >= i0 && j < end) ? h : 0.0f;
            }
            if (hr != nullptr) {
                float o[V];
#pragma unroll
                for (int e = 0; e < V; ++e) o[e] = v[c * V + e];
                // Only this slice's columns: the store is guarded by `end`.
                store_guarded<V, HINT>(hr, i0, cols, end, o);
            }
        }
    }

    Partial2 out = {0.0, 0.0};
    if constexpr (OP == kRmsNorm) {
        float t[K];
#pragma unroll
        for (int k = 0; k < K; ++k) t[k] = v[k] * v[k];
        out.a = (double)row_reduce(tree_reduce<K>(t, AddOp{}), AddOp{}, rl, lds0);
    } else if constexpr (OP == kSum) {
        double t[K];
#pragma unroll
        for (int k = 0; k < K; ++k) t[k] = (double)v[k];
        out.a = row_reduce(tree_reduce<K>(t, AddOp{}), AddOp{}, rl, ldsd);
    } else if constexpr (kMaxFirst) {
        float t[K];
#pragma unroll
        for (int k = 0; k < K; ++k) t[k] = v[k];
        const float m = row_reduce(tree_reduce<K>(t, MaxOp{}), MaxOp{}, rl, lds0);
        // A slice of -inf only (masked columns) has max -inf and sum 0.
        const float ref = m == -INFINITY ? 0.0f : m;
#pragma unroll
        for (int k = 0; k < K; ++k) t[k] = exp_nonpos(v[k] - ref);
        out.a = (double)m;
        out.b = (double)row_reduce(tree_reduce<K>(t, AddOp{}), AddOp{}, rl, lds1);
    } else {
        static_assert(OP == kLayerNorm || OP == kResidualLayerNorm, "unknown operator");
        // Inputs are not written during this launch (h_out may not alias
        // them), so the slice's first value reads the same in every lane.
        const double c0 = (double)value_at<OP, T>(a, off + first);
        double s1 = 0.0, s2 = 0.0;
#pragma unroll
        for (int c = 0; c < NCHUNK; ++c) {
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const int i0 = c * stride + base, j = window_start<V>(i0, cols) + e;
                const double dd = (j >= i0 && j < end) ? (double)v[c * V + e] - c0 : 0.0;
                s1 += dd;
                s2 += dd * dd;
            }
        }
        const double S1 = row_reduce(s1, AddOp{}, rl, ldsd);
        const double S2 = row_reduce(s2, AddOp{}, rl, ldsd2);
        const double n = (double)(end - first);
        out.a = c0 + S1 / n;                   // slice mean
        out.b = fmax(0.0, S2 - S1 * (S1 / n));  // slice M2
    }
    if (threadIdx.x == 0) static_cast<Partial2 *>(a.workspace)[row * gridDim.x + s] = out;
}

// Merge of the row's `slices` partials (slices of `span` columns), each lane
// taking every W-th one in slice order, then the fixed-order row reduction.
template <int OP>
__device__ __forceinline__ void merge_partials(const Partial2 *p, int slices, int span, int cols,
                                               const RowLanes<64> &rl, double *ldsd0, double *ldsd1,
                                               double &stat0, double &stat1) {
    if constexpr (OP == kRmsNorm || OP == kSum) {
        double acc = 0.0;
        for (int j = rl.lane; j < slices; j += rl.W) acc += p[j].a;
        stat0 = row_reduce(acc, AddOp{}, rl, ldsd0);
    } else if constexpr (OP == kSoftmax || OP == kCrossEntropy) {
        double m = -INFINITY;
        for (int j = rl.lane; j < slices; j += rl.W) m = fmax(m, p[j].a);
        m = row_reduce(m, MaxOp{}, rl, ldsd0);
        double z = 0.0;  // slices of -inf only add nothing
        for (int j = rl.lane; j < slices; j += rl.W)
            if (p[j].a != -INFINITY) z += p[j].b * exp(p[j].a - m);
        stat0 = m;
        stat1 = row_reduce(z, AddOp{}, rl, ldsd1);
    } else {
        // Chan's merge of (n_j, mean_j, M2_j): mean = sum n_j mean_j / n,
        // M2 = sum (M2_j + n_j (mean_j - mean)^2); var = M2 / n.
        double a1 = 0.0;
        for (int j = rl.lane; j < slices; j += rl.W) a1 += (double)slice_len(j, span, cols) * p[j].a;
        const double mean = row_reduce(a1, AddOp{}, rl, ldsd0) / (double)cols;
        double a2 = 0.0;
        for (int j = rl.lane; j < slices; j += rl.W) {
            const double d = p[j].a - mean;
            a2 += p[j].b + (double)slice_len(j, span, cols) * d * d;
        }
        stat0 = mean;
        stat1 = row_reduce(a2, AddOp{}, rl, ldsd1) / (double)cols;
    }
}

template <int OP, int V, int NCHUNK, int HINT, class T>
__global__ void __launch_bounds__(1024) split_final_kernel(const Args a) {
    constexpr int K = V * NCHUNK;
    __shared__ double ldsd0[16];
    __shared__ double ldsd1[16];
    const RowLanes<64> rl(a);
    const int cols = a.cols;
    const int s = blockIdx.x;
    const int64_t row = blockIdx.y;
    const int64_t off = row * (int64_t)cols;
    const int span = rl.W * K;
    const int slices = (cols + span - 1) / span;
    const int first = s * span;
    const int stride = rl.W * V;
    const int base = first + rl.lane * V;
    const int end = first + slice_len(s, span, cols);
    const Partial2 *p = static_cast<const Partial2 *>(a.workspace) + row * slices;
    // Cross-entropy: the target index is requested with the partials, so
    // only the logit it points to is fetched after the merge.
    int t_idx = 0;
    if constexpr (OP == kCrossEntropy) t_idx = a.targets[row];
    double stat0 = 0.0, stat1 = 0.0;
    merge_partials<OP>(p, slices, span, cols, rl, ldsd0, ldsd1, stat0, stat1);

    const T *xr = static_cast<const T *>(a.x) + off;
    if constexpr (OP == kSum) {
        if (threadIdx.x == 0) a.row_out[row] = (float)stat0;
        return;
    } else if constexpr (OP == kCrossEntropy) {
        if (threadIdx.x == 0) {
            const float xt = target_or_nan(target_raw(xr, t_idx, cols), t_idx, cols);
            a.row_out[row] = (float)(log(stat1) + stat0 - (double)xt);
        }
        return;
    } else {
        const T *Wt = static_cast<const T *>(a.w);
        const T *B = static_cast<const T *>(a.beta);
        T *Y = static_cast<T *>(a.y) + off;
        const T *rr = (OP == kResidualLayerNorm) ? static_cast<const T *>(a.residual) + off : nullptr;
        float scale = 0.0f, shift = 0.0f;
        if constexpr (OP == kRmsNorm) scale = (float)(1.0 / sqrt(stat0 / (double)cols + (double)a.eps));
        if constexpr (OP == kSoftmax) {
            shift = (float)stat0;
            scale = (float)(1.0 / stat1);
        }
        if constexpr (OP == kLayerNorm || OP == kResidualLayerNorm) scale = (float)(1.0 / sqrt(stat1 + (double)a.eps));
#pragma unroll
        for (int c = 0; c < NCHUNK; ++c) {
            const int i0 = c * stride + base;
            float d[V], w[V], b[V];
            load_window<V, HINT, true>(xr, i0, cols, d, 0.0f);
            if constexpr (OP == kResidualLayerNorm) {
                float r[V];
                load_window<V, HINT, true>(rr, i0, cols, r, 0.0f);
#pragma unroll
                for (int e = 0; e < V; ++e) d[e] = is_bf16<T> ? round_to_bf16(d[e] + r[e]) : d[e] + r[e];
            }
            if constexpr (OP == kRmsNorm) {
                load_window<V>(Wt, i0, cols, w, 0.0f);
#pragma unroll
                for (int e = 0; e < V; ++e) d[e] = d[e] * scale * w[e];
            } else if constexpr (OP == kSoftmax) {
#pragma unroll
                for (int e = 0; e < V; ++e) d[e] = exp_nonpos(d[e] - shift) * scale;
            } else {
                load_window<V>(Wt, i0, cols, w, 0.0f);
                load_window<V>(B, i0, cols, b, 0.0f);
#pragma unroll
                for (int e = 0; e < V; ++e) d[e] = (float)((double)d[e] - stat0) * scale * w[e] + b[e];
            }
            store_guarded<V, HINT>(Y, i0, cols, end, d);
        }
    }
}

// ---- host-side dispatch over the compiled instances -------------------------------

struct Launch {
    dim3 grid, block;
    hipStream_t stream;
    bool exact;
    int cache;
};

template <int OP, int V, int NCHUNK, int SEG, bool EXACT, class T>
int launch_reg_exact(const Args &a, const Launch &l) {
    switch (l.cache) {
        case 0: hipLaunchKernelGGL((reg_kernel<OP, V, NCHUNK, SEG, EXACT, hint_of_cache(0), T>), l.grid, l.block, 0, l.stream, a); break;
        case 1: hipLaunchKernelGGL((reg_kernel<OP, V, NCHUNK, SEG, EXACT, hint_of_cache(1), T>), l.grid, l.block, 0, l.stream, a); break;
        case 2: hipLaunchKernelGGL((reg_kernel<OP, V, NCHUNK, SEG, EXACT, hint_of_cache(2), T>), l.grid, l.block, 0, l.stream, a); break;
        default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

template <int OP, int V, int NCHUNK, int SEG, class T>
int launch_reg(const Args &a, const Launch &l) {
    return l.exact ? launch_reg_exact<OP, V, NCHUNK, SEG, true, T>(a, l)
                   : launch_reg_exact<OP, V, NCHUNK, SEG, false, T>(a, l);
}

// Chunk counts with at most 32 live values per lane.
template <int OP, int V, int SEG, class T>
int launch_by_chunks(int chunks, const Args &a, const Launch &l) {
    switch (chunks) {
        case 1: return launch_reg<OP, V, 1, SEG, T>(a, l);
        case 2: return launch_reg<OP, V, 2, SEG, T>(a, l);
        case 4: return launch_reg<OP, V, 4, SEG, T>(a, l);
        case 8:
            if constexpr (V * 8 <= 32) return launch_reg<OP, V, 8, SEG, T>(a, l);
            else return (int)hipErrorInvalidValue;
        default: return (int)hipErrorInvalidValue;
    }
}

// V = 1, 2, 4 for float rows; 1, 2, 4, 8 for bfloat16 rows (16 bytes at most).
template <int OP, int SEG, class T>
int launch_by_v(int v, int chunks, const Args &a, const Launch &l) {
    switch (v) {
        case 1: return launch_by_chunks<OP, 1, SEG, T>(chunks, a, l);
        case 2: return launch_by_chunks<OP, 2, SEG, T>(chunks, a, l);
        case 4: return launch_by_chunks<OP, 4, SEG, T>(chunks, a, l);
        case 8:
            if constexpr (is_bf16<T>) return launch_by_chunks<OP, 8, SEG, T>(chunks, a, l);
            else return (int)hipErrorInvalidValue;
        default: return (int)hipErrorInvalidValue;
    }
}

template <int OP, int V, int KEEP, int LDSC, class T, bool DMA>
int launch_loop_cache(const Args &a, const Launch &l) {
    switch (l.cache) {
        case 0: hipLaunchKernelGGL((loop_kernel<OP, V, KEEP, LDSC, hint_of_cache(0), T, DMA>), l.grid, l.block, 0, l.stream, a); break;
        case 1: hipLaunchKernelGGL((loop_kernel<OP, V, KEEP, LDSC, hint_of_cache(1), T, DMA>), l.grid, l.block, 0, l.stream, a); break;
        case 2: hipLaunchKernelGGL((loop_kernel<OP, V, KEEP, LDSC, hint_of_cache(2), T, DMA>), l.grid, l.block, 0, l.stream, a); break;
        default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

// LDS-kept chunks of bfloat16 rows go straight from memory to LDS when
// every window start is 16-byte aligned (row pointer aligned, cols a
// multiple of 8), the group has 1024 lanes, the row has one input and 32 or
// 64 slots are kept in registers (beside 96 the issue loop would spill);
// otherwise they pass through registers. Measured over the 2048x128256,
// 4096x65536 and 4096x49152 streaming cases: 2-3% faster for bfloat16, while
// float rows (four times as many 16-byte loads per row) ran 1-2.5% slower
// that way. LDS then holds the raw 16-byte packs, half the bytes of the
// widened floats the register route stores, so kDmaChunks of them (144 KiB
// of the 160 KiB a workgroup may allocate) fit where 4 widened ones did;
// that also lets RMSNorm's 64-slot plan (alone on its compute unit by its
// registers, which leave no room for the register route) keep chunks in
// LDS.
constexpr int kDmaChunks = 9;
template <int OP, int V, int KEEP, int LDSC, class T>
int launch_loop_keep(const Args &a, const Launch &l) {
    if constexpr (is_bf16<T> && V == 8 && KEEP > 0 && KEEP * V <= 64 && OP != kResidualLayerNorm &&
                  (LDSC > 0 || (OP == kRmsNorm && KEEP * V == 64))) {
        if (l.block.x == 1024 && (reinterpret_cast<uintptr_t>(a.x) & 15) == 0 && a.cols % V == 0)
            return launch_loop_cache<OP, V, KEEP, kDmaChunks, T, true>(a, l);
    }
    return launch_loop_cache<OP, V, KEEP, LDSC, T, false>(a, l);
}

// Streaming plans keep 0 or 32 register slots per lane (the two-pass
// operators at V >= 4: 32 / V chunks), 64 for RMSNorm and softmax, or 96 for
// softmax, whose instances still fit the 128 registers of a 1024-lane
// workgroup without spilling (the LayerNorms would spill at 64). A 1024-lane
// plan whose registers are full that way (softmax at 64 or 96 slots, the
// LayerNorms at 32) runs one workgroup per compute unit anyway, so it also
// keeps the next values of each lane in LDS: 32 floats (128 KiB), or 72
// bfloat16 values (144 KiB; 32 beside softmax's 96 slots): a 65536-column
// float LayerNorm row, or 131072 columns of softmax (a 128256-entry
// vocabulary), is then read once.
// (Float RMSNorm at 64 slots already holds a 65536-column row; with LDS
// added its instance would spill. bfloat16 RMSNorm at 64 slots takes 72
// values per lane into LDS straight from memory.)
template <int OP, int V, class T>
int launch_loop(int slots, const Args &a, const Launch &l) {
    if (slots == 0) return launch_loop_keep<OP, V, 0, 0, T>(a, l);
    constexpr bool kLn = OP == kLayerNorm || OP == kResidualLayerNorm;
    // LDS-kept chunks: 32 float values per lane (128 KiB), or 72 bfloat16
    // values (144 KiB) for bfloat16 rows.
    constexpr int kLds = (is_bf16<T> ? 72 : 32) / V;
    if constexpr (V >= 4 && OP != kSum && OP != kCrossEntropy) {
        if (slots == 32) {
            if (kLn && l.block.x == 1024) return launch_loop_keep<OP, V, 32 / V, (kLn ? kLds : 0), T>(a, l);
            return launch_loop_keep<OP, V, 32 / V, 0, T>(a, l);
        }
    }
    if constexpr (V >= 4 && (OP == kRmsNorm || OP == kSoftmax)) {
        if (slots == 64) return launch_loop_keep<OP, V, 64 / V, (OP == kSoftmax ? kLds : 0), T>(a, l);
    }
    if constexpr (V >= 4 && OP == kSoftmax) {
        // Beside 96 register slots the LDS chunks are loaded one at a time
        // (no registers to batch them), so more of them gained nothing; they
        // hold 32 values per lane.
        if (slots == 96) return launch_loop_keep<OP, V, 96 / V, 32 / V, T>(a, l);
    }
    return (int)hipErrorInvalidValue;
}

// Split rows: V = 4 (float) or 8 (bfloat16), K = 16 or 32, streaming hints.
template <int OP, class T>
int launch_split(const rr_plan &p, const Args &a, const Launch &l) {
    constexpr int V = is_bf16<T> ? 8 : 4;
    if (p.v != V || p.cache != 2) return (int)hipErrorInvalidValue;
    const int span = p.lanes_per_row * p.slots;
    const unsigned slices = (unsigned)((a.cols + span - 1) / span);
    const dim3 grid1(slices, (unsigned)a.rows);
    const dim3 grid2((OP == kSum || OP == kCrossEntropy) ? 1u : slices, (unsigned)a.rows);
    constexpr int H = hint_of_cache(2);
    if (p.slots == 16) {
        hipLaunchKernelGGL((split_partial_kernel<OP, V, 16 / V, H, T>), grid1, l.block, 0, l.stream, a);
        hipLaunchKernelGGL((split_final_kernel<OP, V, 16 / V, H, T>), grid2, l.block, 0, l.stream, a);
    } else if (p.slots == 32) {
        hipLaunchKernelGGL((split_partial_kernel<OP, V, 32 / V, H, T>), grid1, l.block, 0, l.stream, a);
        hipLaunchKernelGGL((split_final_kernel<OP, V, 32 / V, H, T>), grid2, l.block, 0, l.stream, a);
    } else {
        return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

// Launch `OP` on storage type T with a plan already checked by the planner.
template <int OP, class T>
int launch_op(const rr_plan &p, const Args &args, void *stream) {
    Args a = args;
    a.lanes_per_row = p.lanes_per_row;
    a.log2_lanes = __builtin_ctz((unsigned)p.lanes_per_row);
    a.rows_per_group = p.rows_per_group;
    const int64_t groups = (a.rows + p.rows_per_group - 1) / p.rows_per_group;
    Launch l;
    l.grid = dim3((unsigned)groups);
    l.block = dim3((unsigned)p.block);
    l.stream = reinterpret_cast<hipStream_t>(stream);
    l.exact = (int64_t)p.lanes_per_row * p.slots == (int64_t)a.cols;
    l.cache = p.cache;
    if (p.path == RR_PATH_SPLIT) return launch_split<OP, T>(p, a, l);
    if (p.path == RR_PATH_LOOP) {
        switch (p.v) {
            case 1: return launch_loop<OP, 1, T>(p.slots, a, l);
            case 2: return launch_loop<OP, 2, T>(p.slots, a, l);
            case 4: return launch_loop<OP, 4, T>(p.slots, a, l);
            case 8:
                if constexpr (is_bf16<T>) return launch_loop<OP, 8, T>(p.slots, a, l);
                else return (int)hipErrorInvalidValue;
            default: return (int)hipErrorInvalidValue;
        }
    }
    const int chunks = p.slots / p.v;
    switch (p.lanes_per_row) {
        case 8: return launch_by_v<OP, 8, T>(p.v, chunks, a, l);
        case 16: return launch_by_v<OP, 16, T>(p.v, chunks, a, l);
        case 32: return launch_by_v<OP, 32, T>(p.v, chunks, a, l);
        default: return launch_by_v<OP, 64, T>(p.v, chunks, a, l);
    }
}

}  // namespace rowred
