// quantize.hip -- absmax quantize kernels for gfx950:
//   x_q = sat(RNE(x / scale)),  scale = max(max|x|, floor) / qmax
// per tensor or per row, BF16/FP32 in, E4M3 / E5M2 / INT8 codes out.
//
// Definitions: AstrAI ops/fp8.py @5e76fbd (quantize_bf16 docstring: cast
// with fused amax, amax returned fresh; _fp8_quantize_cpu: x.float()/scale,
// amax clamped at 1e-12) and POPCORNBENCH "Kimi-K2.6 l2_p13" (reference
// model steps 2-4: amax clamp 1e-8, scale = amax/127, clamp +-127, ties to
// even).  The commit message on the AstrAI page motivates the last-workgroup
// epilogue: the step is published on device by the final workgroup of the
// reduction, with no extra launch and no host synchronization.
//
// Kernels
//   qz_amax   per-tensor current scaling, pass 1: HBM-streaming max|x| with
//             16-byte loads; on small grids the last workgroup publishes
//             amax and the step, on large ones each workgroup leaves its
//             maximum in the workspace.
//   qz_cast   pass 2 (or the only pass under delayed scaling, where it also
//             measures amax and publishes it, or updates the history ring,
//             from its last workgroup).  As pass 2 after per-workgroup
//             maxima, every workgroup reduces them and workgroup 0
//             publishes amax and the step.  As pass 2 it walks the tensor
//             from the end backwards, so it starts on the data pass 1 read
//             last, which the memory-side cache (256 MB) still holds.
//   qz_rows   per-row and row groups: one workgroup per group of rows
//             (one row for per-row scales); the group's second read hits
//             the cache, so HBM sees each element once.
#include "qdev.hpp"
#include "internal.hpp"

namespace ql {

typedef unsigned int u32v4 __attribute__((ext_vector_type(4)));

// Code stores of the cast pass of current scaling are non-temporal: the
// codes do not displace the input from the memory-side cache, from which
// that pass re-reads it (quantize of the large a: 127 -> 110 us); the GEMM
// that consumes the codes right after then reads them from HBM instead, and
// the whole forward step measured the same either way.  The single pass of
// delayed scaling, which re-reads nothing, stores through the caches (ring
// quantize of the large a: 78.5 -> 74.0 us).
template <bool NT>
__device__ __forceinline__ void store16_codes(uint8_t *dst, uint4 c)
{
    if constexpr (NT) __builtin_nontemporal_store(u32v4{c.x, c.y, c.z, c.w}, reinterpret_cast<u32v4 *>(dst));
    else *reinterpret_cast<uint4 *>(dst) = c;
}

// Whole-tensor kernels: at most one workgroup of 16 waves per CU.  That
// streams as fast as more, smaller workgroups (four waves per SIMD with four
// 32-byte units in flight per lane keep 32 MiB of reads outstanding) and
// keeps the end-of-grid election to 256 atomic pairs.
constexpr int QZ_THREADS = 1024;
constexpr int QZ_MAX_BLOCKS = 256;
static_assert(QZ_MAX_BLOCKS <= QZ_PARTS_PER_SLOT, "one workspace maximum per workgroup");
// Current scaling: amax passes of at least this many workgroups leave one
// maximum per workgroup in the workspace, which every workgroup of the cast
// pass reduces at its start (no election at the end of pass 1); smaller
// grids elect the last workgroup, which publishes before the cast starts.
constexpr int QZ_PARTS_MIN_BLOCKS = 64;
// Per-row / row-group kernel: one workgroup of 4 waves per group of rows.
constexpr int QZ_ROW_THREADS = 256;
constexpr int QZ_UNIT = 16;            // elements per vector unit
constexpr int QZ_UNROLL = 4;

enum : int { MODE_FLAT = 0, MODE_ROWS = 1, MODE_SCALAR = 2 };

// 16 consecutive input elements loaded with 16-byte loads.
template <typename T> struct Vec16;

template <> struct Vec16<uint16_t> {
    uint32_t w[8];
    __device__ __forceinline__ void load(const uint16_t *p)
    {
        const uint4 *q = reinterpret_cast<const uint4 *>(p);
        uint4 a = q[0], b = q[1];
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    }
    // The same with non-temporal loads (input read once: single-pass casts).
    __device__ __forceinline__ void load_nt(const uint16_t *p)
    {
        const u32v4 *q = reinterpret_cast<const u32v4 *>(p);
        const u32v4 a = __builtin_nontemporal_load(q), b = __builtin_nontemporal_load(q + 1);
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    }
    __device__ __forceinline__ float f(int i) const { return (i & 1) ? bf16_hi(w[i >> 1]) : bf16_lo(w[i >> 1]); }
    __device__ __forceinline__ uint32_t amax_bits() const
    {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) { uint32_t t = absbits_bf16_pair(w[i]); m = t > m ? t : m; }
        return m;
    }
};

template <> struct Vec16<float> {
    float v[16];
    __device__ __forceinline__ void load(const float *p)
    {
        const float4 *q = reinterpret_cast<const float4 *>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float4 a = q[i];
            v[4 * i] = a.x; v[4 * i + 1] = a.y; v[4 * i + 2] = a.z; v[4 * i + 3] = a.w;
        }
    }
    __device__ __forceinline__ void load_nt(const float *p)
    {
        const u32v4 *q = reinterpret_cast<const u32v4 *>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32v4 a = __builtin_nontemporal_load(q + i);
            v[4 * i] = __uint_as_float(a.x); v[4 * i + 1] = __uint_as_float(a.y);
            v[4 * i + 2] = __uint_as_float(a.z); v[4 * i + 3] = __uint_as_float(a.w);
        }
    }
    __device__ __forceinline__ float f(int i) const { return v[i]; }
    __device__ __forceinline__ uint32_t amax_bits() const
    {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) { uint32_t t = absbits_f32(v[i]); m = t > m ? t : m; }
        return m;
    }
};

template <typename T> __device__ __forceinline__ float load1(const T *x, int64_t i);
template <> __device__ __forceinline__ float load1<uint16_t>(const uint16_t *x, int64_t i) { return __uint_as_float((uint32_t)x[i] << 16); }
template <> __device__ __forceinline__ float load1<float>(const float *x, int64_t i) { return x[i]; }

template <int FMT, typename T>
__device__ __forceinline__ uint4 encode16(const Vec16<T> &u, const Divider &div)
{
    uint4 o;
    o.x = encode4<FMT>(div(u.f(0)), div(u.f(1)), div(u.f(2)), div(u.f(3)));
    o.y = encode4<FMT>(div(u.f(4)), div(u.f(5)), div(u.f(6)), div(u.f(7)));
    o.z = encode4<FMT>(div(u.f(8)), div(u.f(9)), div(u.f(10)), div(u.f(11)));
    o.w = encode4<FMT>(div(u.f(12)), div(u.f(13)), div(u.f(14)), div(u.f(15)));
    return o;
}

// The same with the quotient path fixed at compile time.
template <int FMT, bool FAST, typename T>
__device__ __forceinline__ uint4 encode16q(const Vec16<T> &u, const Divider &d)
{
    uint4 o;
    o.x = encode4<FMT>(d.q<FAST>(u.f(0)), d.q<FAST>(u.f(1)), d.q<FAST>(u.f(2)), d.q<FAST>(u.f(3)));
    o.y = encode4<FMT>(d.q<FAST>(u.f(4)), d.q<FAST>(u.f(5)), d.q<FAST>(u.f(6)), d.q<FAST>(u.f(7)));
    o.z = encode4<FMT>(d.q<FAST>(u.f(8)), d.q<FAST>(u.f(9)), d.q<FAST>(u.f(10)), d.q<FAST>(u.f(11)));
    o.w = encode4<FMT>(d.q<FAST>(u.f(12)), d.q<FAST>(u.f(13)), d.q<FAST>(u.f(14)), d.q<FAST>(u.f(15)));
    return o;
}

// Offsets of vector unit u in x and x_q for the two vector modes.
template <int MODE>
__device__ __forceinline__ void unit_offsets(const QzParams &p, int64_t u, int64_t &ox, int64_t &oq)
{
    if (MODE == MODE_FLAT) {
        ox = oq = u * QZ_UNIT;
    } else {
        int64_t row = u / p.units_per_row;
        int64_t c = (u - row * p.units_per_row) * QZ_UNIT;
        ox = row * p.ldx + c;
        oq = row * p.ldq + c;
    }
}

__device__ __forceinline__ void elem_offsets(const QzParams &p, int64_t e, int64_t &ox, int64_t &oq)
{
    int64_t row = e / p.cols, c = e - row * p.cols;
    ox = row * p.ldx + c;
    oq = row * p.ldq + c;
}

// Publish amax (floored) and fl32(amax/qmax).  NaN stays NaN.
__device__ __forceinline__ void publish(const QzParams &p, uint32_t bits, int64_t i)
{
    float a = __uint_as_float(bits);
    float amax = a < p.floor ? p.floor : a;
    if (p.amax_out) p.amax_out[i] = amax;
    if (p.scale_out) p.scale_out[i] = amax / p.qmax;      // IEEE division
}

// Finalize an amax history ring from the last workgroup (every thread of it
// calls this): hist[idx] = amax (floored), scale_used = the scale the cast
// used, ring scale = fl32(max(hist) / qmax) * 2^margin.  History values are
// non-negative floats, so their maximum is taken on the bit patterns.
__device__ __forceinline__ void ring_publish(const QzParams &p, uint32_t bits, uint32_t *red)
{
    const float a = __uint_as_float(bits);
    const float amax = a < p.floor ? p.floor : a;
    uint32_t m = absbits_f32(amax);
    for (int64_t i = threadIdx.x; i < p.hist_len; i += blockDim.x)
        if (i != p.ring_idx) { const uint32_t t = absbits_f32(p.ring[i]); m = t > m ? t : m; }
    m = block_max_u32(m, red);
    if (threadIdx.x == 0) {
        const float used = p.ring[p.hist_len];
        p.ring[p.ring_idx] = amax;
        if (p.scale_used) p.scale_used[0] = used;
        if (p.amax_out) p.amax_out[0] = amax;
        const float step = __uint_as_float(m) / p.qmax;           // IEEE division
        p.ring[p.hist_len] = __builtin_ldexpf(step, p.margin);
    }
}

// ---------------------------------------------------------------------------
// Pass 1 of per-tensor current scaling.
template <typename T, int MODE>
__global__ __launch_bounds__(QZ_THREADS) void qz_amax(QzPack pk)
{
    const QzParams &p = pk.t[blockIdx.y];
    const T *x = static_cast<const T *>(p.x);
    const int64_t gtid = (int64_t)blockIdx.x * QZ_THREADS + threadIdx.x;
    const int64_t gstride = (int64_t)gridDim.x * QZ_THREADS;
    uint32_t m = 0;
    if (MODE == MODE_SCALAR) {
        for (int64_t e = gtid; e < p.n_elems; e += gstride) {
            int64_t ox, oq;
            elem_offsets(p, e, ox, oq);
            uint32_t t = absbits_f32(load1<T>(x, ox));
            m = t > m ? t : m;
        }
    } else {
        int64_t u = gtid;
        for (; u + (QZ_UNROLL - 1) * gstride < p.n_units; u += QZ_UNROLL * gstride) {
            Vec16<T> v[QZ_UNROLL];
#pragma unroll
            for (int j = 0; j < QZ_UNROLL; ++j) {
                int64_t ox, oq;
                unit_offsets<MODE>(p, u + j * gstride, ox, oq);
                v[j].load(x + ox);
            }
#pragma unroll
            for (int j = 0; j < QZ_UNROLL; ++j) { uint32_t t = v[j].amax_bits(); m = t > m ? t : m; }
        }
        for (; u < p.n_units; u += gstride) {
            int64_t ox, oq;
            unit_offsets<MODE>(p, u, ox, oq);
            Vec16<T> v;
            v.load(x + ox);
            uint32_t t = v.amax_bits();
            m = t > m ? t : m;
        }
        if (MODE == MODE_FLAT)   // flat tail beyond the last whole unit
            for (int64_t e = p.n_units * QZ_UNIT + gtid; e < p.n_elems; e += gstride) {
                uint32_t t = absbits_f32(load1<T>(x, e));
                m = t > m ? t : m;
            }
    }
    __shared__ uint32_t red[QZ_THREADS / 64];
    m = block_max_u32(m, red);
    if (threadIdx.x == 0) {
        uint32_t bits;
        if (p.amax_part) p.amax_part[blockIdx.x] = m;
        else if (elect_last_max_n(p.ws, m, &bits, gridDim.x)) publish(p, bits, 0);
    }
}

// ---------------------------------------------------------------------------
// Cast with one step for the whole tensor.  MEASURE (delayed scaling): the
// step comes from the caller and amax is measured in the same pass.
template <typename T, int FMT, int MODE, bool MEASURE>
__global__ __launch_bounds__(QZ_THREADS) void qz_cast(QzPack pk)
{
    const QzParams &p = pk.t[blockIdx.y];
    const T *x = static_cast<const T *>(p.x);
    uint8_t *xq = static_cast<uint8_t *>(p.xq);
    float step;
    if (!MEASURE && p.amax_part) {
        // Current scaling after an amax pass of the same grid that left one
        // maximum per workgroup: every workgroup reduces them itself and
        // workgroup 0 publishes amax and the step, so no launch sits between
        // the two passes.
        uint32_t m = 0;
        for (int i = threadIdx.x; i < (int)gridDim.x; i += QZ_THREADS) m = p.amax_part[i] > m ? p.amax_part[i] : m;
        __shared__ uint32_t red0[QZ_THREADS / 64];
        m = block_max_u32(m, red0);
        const float a = __uint_as_float(m);
        const float amax = a < p.floor ? p.floor : a;       // NaN stays NaN
        step = amax / p.qmax;                                // IEEE division
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            if (p.amax_out) p.amax_out[0] = amax;
            p.scale_out[0] = step;
        }
    } else {
        step = p.scale_src[0];
    }
    const Divider div(step);
    const int64_t gtid = (int64_t)blockIdx.x * QZ_THREADS + threadIdx.x;
    const int64_t gstride = (int64_t)gridDim.x * QZ_THREADS;
    uint32_t m = 0;
    if (MODE == MODE_SCALAR) {
        for (int64_t e = gtid; e < p.n_elems; e += gstride) {
            int64_t ox, oq;
            elem_offsets(p, e, ox, oq);
            float v = load1<T>(x, ox);
            if (MEASURE) { uint32_t t = absbits_f32(v); m = t > m ? t : m; }
            xq[oq] = encode1<FMT>(div(v));
        }
    } else {
        // Unit u of the walk is unit n_units-1-u of the tensor in pass 2.
        auto phys = [&](int64_t u) { return MEASURE ? u : p.n_units - 1 - u; };
        // The quotient path is chosen once for the whole walk, so no element
        // carries a test for it.
        auto walk = [&](auto FASTC) {
            constexpr bool FAST = decltype(FASTC)::value;
            int64_t u = gtid;
            for (; u + (QZ_UNROLL - 1) * gstride < p.n_units; u += QZ_UNROLL * gstride) {
                Vec16<T> v[QZ_UNROLL];
                int64_t oq[QZ_UNROLL];
#pragma unroll
                for (int j = 0; j < QZ_UNROLL; ++j) {
                    int64_t ox;
                    unit_offsets<MODE>(p, phys(u + j * gstride), ox, oq[j]);
                    // A single-pass (delayed) cast reads its input once; the
                    // cast pass of current scaling reads it back from the
                    // memory-side cache.
                    if (MEASURE) v[j].load_nt(x + ox);
                    else v[j].load(x + ox);
                }
#pragma unroll
                for (int j = 0; j < QZ_UNROLL; ++j) {
                    if (MEASURE) { uint32_t t = v[j].amax_bits(); m = t > m ? t : m; }
                    store16_codes<!MEASURE>(xq + oq[j], encode16q<FMT, FAST>(v[j], div));
                }
            }
            for (; u < p.n_units; u += gstride) {
                int64_t ox, oq;
                unit_offsets<MODE>(p, phys(u), ox, oq);
                Vec16<T> v;
                v.load(x + ox);
                if (MEASURE) { uint32_t t = v.amax_bits(); m = t > m ? t : m; }
                store16_codes<!MEASURE>(xq + oq, encode16q<FMT, FAST>(v, div));
            }
        };
        if (div.fast) walk(std::true_type{});
        else walk(std::false_type{});
        if (MODE == MODE_FLAT)
            for (int64_t e = p.n_units * QZ_UNIT + gtid; e < p.n_elems; e += gstride) {
                float v = load1<T>(x, e);
                if (MEASURE) { uint32_t t = absbits_f32(v); m = t > m ? t : m; }
                xq[e] = encode1<FMT>(div(v));
            }
    }
    if (MEASURE) {
        __shared__ uint32_t red[QZ_THREADS / 64];
        __shared__ uint32_t last_bits;
        __shared__ int is_last;
        m = block_max_u32(m, red);
        if (threadIdx.x == 0) {
            uint32_t bits = 0;
            const bool last = elect_last_max_n(p.ws, m, &bits, gridDim.x);
            if (last && !p.ring) publish(p, bits, 0);
            is_last = last;
            last_bits = bits;
        }
        if (p.ring) {
            __syncthreads();
            if (is_last) ring_publish(p, last_bits, red);   // block-uniform branch
        }
    }
}

// ---------------------------------------------------------------------------
// Per-row and row groups: one workgroup per group.  Pass 1 reduces the
// group's amax, pass 2 re-reads the group (from cache) and casts it with the
// group's step (or the caller's step under delayed scaling).
template <typename T, int FMT, bool VEC, bool DELAYED>
__global__ __launch_bounds__(QZ_ROW_THREADS) void qz_rows(QzParams p)
{
    // Group g = blockIdx.x: rows [g*G, min((g+1)*G, rows)), G = group_rows
    // (1 for per-row scales).
    const int64_t grp = blockIdx.x;
    const int64_t r0 = grp * p.group_rows;
    const int64_t r1 = r0 + p.group_rows < p.rows ? r0 + p.group_rows : p.rows;
    // Narrow rows (fewer work items than threads) are covered several per
    // pass: thread t takes item t % W of row t / W, W items per row.
    const int64_t W = VEC ? p.units_per_row : p.cols;
    int64_t rpp = 1, tr = 0, tu = threadIdx.x, ustep = QZ_ROW_THREADS;
    if (W > 0 && W < QZ_ROW_THREADS) {
        const int w = (int)W;
        rpp = QZ_ROW_THREADS / w;
        tr = (int)threadIdx.x / w;
        tu = (int)threadIdx.x - (int)tr * w;
        ustep = w;
        if (tr >= rpp) tr = r1 - r0;                // idle threads
    }
    // A thread walks its items (r, u) in order, QZ_UNROLL at a time so that
    // their loads are all in flight together.
    auto next = [&](int64_t &r, int64_t &u) {
        u += ustep;
        if (u >= W) { u = tu; r += rpp; }
    };
    uint32_t m = 0;
    for (int64_t r = r0 + tr, u = tu; r < r1 && u < W;) {
        int64_t rr[QZ_UNROLL], uu[QZ_UNROLL];
        bool ok[QZ_UNROLL];
#pragma unroll
        for (int k = 0; k < QZ_UNROLL; ++k) {
            ok[k] = r < r1;
            rr[k] = r; uu[k] = u;
            if (ok[k]) next(r, u);
        }
        if (VEC) {
            Vec16<T> v[QZ_UNROLL];
#pragma unroll
            for (int k = 0; k < QZ_UNROLL; ++k)
                if (ok[k]) v[k].load(static_cast<const T *>(p.x) + rr[k] * p.ldx + uu[k] * QZ_UNIT);
#pragma unroll
            for (int k = 0; k < QZ_UNROLL; ++k)
                if (ok[k]) { const uint32_t t = v[k].amax_bits(); m = t > m ? t : m; }
        } else {
            float v[QZ_UNROLL];
#pragma unroll
            for (int k = 0; k < QZ_UNROLL; ++k)
                v[k] = ok[k] ? load1<T>(static_cast<const T *>(p.x) + rr[k] * p.ldx, uu[k]) : 0.0f;
#pragma unroll
            for (int k = 0; k < QZ_UNROLL; ++k) { const uint32_t t = absbits_f32(v[k]); m = t > m ? t : m; }
        }
    }
    __shared__ uint32_t red[QZ_ROW_THREADS / 64];
    m = block_max_u32(m, red);
    const float a = __uint_as_float(m);
    const float amax = a < p.floor ? p.floor : a;
    const float step = amax / p.qmax;                      // IEEE division
    if (threadIdx.x == 0) {
        if (p.amax_out) p.amax_out[grp] = amax;
        if (p.scale_out) p.scale_out[grp] = step;
    }
    const Divider div(DELAYED ? p.scale_src[grp] : step);
    // The quotient path is chosen once for the group's walk.
    auto walk = [&](auto FASTC) {
        constexpr bool FAST = decltype(FASTC)::value;
        for (int64_t r = r0 + tr, u = tu; r < r1 && u < W;) {
            int64_t rr[QZ_UNROLL], uu[QZ_UNROLL];
            bool ok[QZ_UNROLL];
#pragma unroll
            for (int k = 0; k < QZ_UNROLL; ++k) {
                ok[k] = r < r1;
                rr[k] = r; uu[k] = u;
                if (ok[k]) next(r, u);
            }
            if (VEC) {
                Vec16<T> v[QZ_UNROLL];
#pragma unroll
                for (int k = 0; k < QZ_UNROLL; ++k)
                    if (ok[k]) v[k].load(static_cast<const T *>(p.x) + rr[k] * p.ldx + uu[k] * QZ_UNIT);
#pragma unroll
                for (int k = 0; k < QZ_UNROLL; ++k)
                    if (ok[k])
                        *reinterpret_cast<uint4 *>(static_cast<uint8_t *>(p.xq) + rr[k] * p.ldq + uu[k] * QZ_UNIT) =
                            encode16q<FMT, FAST>(v[k], div);
            } else {
                float v[QZ_UNROLL];
#pragma unroll
                for (int k = 0; k < QZ_UNROLL; ++k)
                    v[k] = ok[k] ? load1<T>(static_cast<const T *>(p.x) + rr[k] * p.ldx, uu[k]) : 0.0f;
#pragma unroll
                for (int k = 0; k < QZ_UNROLL; ++k)
                    if (ok[k]) static_cast<uint8_t *>(p.xq)[rr[k] * p.ldq + uu[k]] = encode1<FMT>(div.q<FAST>(v[k]));
            }
        }
    };
    if (div.fast) walk(std::true_type{});
    else walk(std::false_type{});
}

// ---------------------------------------------------------------------------
// out_amax of a GEMM from its workgroups' maxima (|v| as FP32 bits).
__global__ __launch_bounds__(1024) void gemm_amax_finalize(const uint32_t *parts, int64_t n, float *out)
{
    uint32_t m = 0;
    for (int64_t i = threadIdx.x; i < n; i += 1024) m = parts[i] > m ? parts[i] : m;
    __shared__ uint32_t red[1024 / 64];
    m = block_max_u32(m, red);
    if (threadIdx.x == 0) out[0] = __uint_as_float(m);
}

hipError_t launch_amax_finalize(const GemmParams &p, int64_t nblocks, hipStream_t s)
{
    hipLaunchKernelGGL(gemm_amax_finalize, dim3(1), dim3(1024), 0, s, p.amax_part, nblocks, p.out_amax);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
__global__ void ws_fill_zero(uint32_t *ws, int64_t words)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < words) ws[i] = 0u;
}

// ---------------------------------------------------------------------------
// Host-side launchers.

static int blocks_for(int64_t work)
{
    int64_t b = (work + QZ_THREADS - 1) / QZ_THREADS;
    if (b < 1) b = 1;
    if (b > QZ_MAX_BLOCKS) b = QZ_MAX_BLOCKS;
    return (int)b;
}

static int64_t tensor_work(const QzParams &p, int mode)
{
    return mode == MODE_SCALAR ? p.n_elems : (p.n_units > 0 ? p.n_units : p.n_elems);
}

// ntensors (1 or 2) whole-tensor quantizes of the same mode and kind
// (current or delayed scaling), grid row y on tensor y.
template <typename T, int FMT, int MODE>
static hipError_t launch_tensor_pack(const QzPack &pk_in, int ntensors, hipStream_t s)
{
    int64_t work = tensor_work(pk_in.t[0], MODE);
    if (ntensors > 1 && tensor_work(pk_in.t[1], MODE) > work) work = tensor_work(pk_in.t[1], MODE);
    const dim3 grid(blocks_for(work), ntensors);
    // Delayed scaling is one launch: its last workgroup publishes.
    QzPack pk = pk_in;
    if (grid.x < QZ_PARTS_MIN_BLOCKS || pk.t[0].delayed) pk.t[0].amax_part = pk.t[1].amax_part = nullptr;
    if (pk.t[0].delayed) {
        hipLaunchKernelGGL((qz_cast<T, FMT, MODE, true>), grid, dim3(QZ_THREADS), 0, s, pk);
    } else {
        // With per-workgroup maxima the cast reduces them and publishes.
        hipLaunchKernelGGL((qz_amax<T, MODE>), grid, dim3(QZ_THREADS), 0, s, pk);
        hipLaunchKernelGGL((qz_cast<T, FMT, MODE, false>), grid, dim3(QZ_THREADS), 0, s, pk);
    }
    return hipGetLastError();
}

template <typename T, int FMT, int MODE>
static hipError_t launch_tensor_mode(const QzParams &p, hipStream_t s)
{
    return launch_tensor_pack<T, FMT, MODE>(QzPack{{p, p}}, 1, s);
}

template <typename T, int FMT>
static hipError_t launch_fmt(const QzParams &p, hipStream_t s)
{
    if (p.per_row) {
        if (p.rows == 0) return hipSuccess;
        const dim3 grid((unsigned)((p.rows + p.group_rows - 1) / p.group_rows));
        if (p.vec_rows) {
            if (p.delayed) hipLaunchKernelGGL((qz_rows<T, FMT, true, true>), grid, dim3(QZ_ROW_THREADS), 0, s, p);
            else hipLaunchKernelGGL((qz_rows<T, FMT, true, false>), grid, dim3(QZ_ROW_THREADS), 0, s, p);
        } else {
            if (p.delayed) hipLaunchKernelGGL((qz_rows<T, FMT, false, true>), grid, dim3(QZ_ROW_THREADS), 0, s, p);
            else hipLaunchKernelGGL((qz_rows<T, FMT, false, false>), grid, dim3(QZ_ROW_THREADS), 0, s, p);
        }
        return hipGetLastError();
    }
    switch (p.mode) {
    case MODE_FLAT: return launch_tensor_mode<T, FMT, MODE_FLAT>(p, s);
    case MODE_ROWS: return launch_tensor_mode<T, FMT, MODE_ROWS>(p, s);
    default: return launch_tensor_mode<T, FMT, MODE_SCALAR>(p, s);
    }
}

template <typename T, int FMT>
static hipError_t launch_pair_fmt(const QzParams &p0, const QzParams &p1, hipStream_t s)
{
    const bool pack = !p0.per_row && !p1.per_row && p0.mode == p1.mode && p0.delayed == p1.delayed && !p0.ring &&
                      !p1.ring && (p0.amax_part != nullptr) == (p1.amax_part != nullptr);
    if (!pack) {
        const hipError_t e = launch_fmt<T, FMT>(p0, s);
        return e != hipSuccess ? e : launch_fmt<T, FMT>(p1, s);
    }
    const QzPack pk{{p0, p1}};
    switch (p0.mode) {
    case MODE_FLAT: return launch_tensor_pack<T, FMT, MODE_FLAT>(pk, 2, s);
    case MODE_ROWS: return launch_tensor_pack<T, FMT, MODE_ROWS>(pk, 2, s);
    default: return launch_tensor_pack<T, FMT, MODE_SCALAR>(pk, 2, s);
    }
}

hipError_t launch_quantize_pair(const QzParams &p0, const QzParams &p1, int in_dt, int fmt, hipStream_t s)
{
    if (in_dt == DT_BF16) {
        if (fmt == FMT_E4M3) return launch_pair_fmt<uint16_t, FMT_E4M3>(p0, p1, s);
        if (fmt == FMT_E5M2) return launch_pair_fmt<uint16_t, FMT_E5M2>(p0, p1, s);
        return launch_pair_fmt<uint16_t, FMT_INT8>(p0, p1, s);
    }
    if (fmt == FMT_E4M3) return launch_pair_fmt<float, FMT_E4M3>(p0, p1, s);
    if (fmt == FMT_E5M2) return launch_pair_fmt<float, FMT_E5M2>(p0, p1, s);
    return launch_pair_fmt<float, FMT_INT8>(p0, p1, s);
}

hipError_t launch_quantize(const QzParams &p, int in_dt, int fmt, hipStream_t s)
{
    if (in_dt == DT_BF16) {
        if (fmt == FMT_E4M3) return launch_fmt<uint16_t, FMT_E4M3>(p, s);
        if (fmt == FMT_E5M2) return launch_fmt<uint16_t, FMT_E5M2>(p, s);
        return launch_fmt<uint16_t, FMT_INT8>(p, s);
    }
    if (fmt == FMT_E4M3) return launch_fmt<float, FMT_E4M3>(p, s);
    if (fmt == FMT_E5M2) return launch_fmt<float, FMT_E5M2>(p, s);
    return launch_fmt<float, FMT_INT8>(p, s);
}

hipError_t launch_ws_zero(void *ws, int64_t bytes, hipStream_t s)
{
    const int64_t words = bytes / 4;
    const unsigned blocks = (unsigned)((words + 255) / 256);
    hipLaunchKernelGGL(ws_fill_zero, dim3(blocks), dim3(256), 0, s, static_cast<uint32_t *>(ws), words);
    return hipGetLastError();
}

}  // namespace ql
