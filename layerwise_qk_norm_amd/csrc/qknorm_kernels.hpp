// Device code of the layerwise QK-Norm library (gfx950 / CDNA4, wave64).
//
// Method: "SwiftQK: Fast and Communication-Efficient Tensor Parallelism for
// Query-Key Normalization" -- Eq. (1) (RMSNorm over the full Q or K vector),
// Section III-A..D and Algorithm 1 (local sum of squares, scalar exchange
// overlapped with the x*gamma product, final scaling, persistent grid bounded
// by co-residency). Here the "ranks" are logical shards on one GPU: the
// shards of a token tile are workgroups of one grid that exchange their fp32
// partials through 64-bit slots in device memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qkn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Element formats. A "vector" is one 16-byte memory access.
struct Bf16 {
    using elem_t = uint16_t;
    static constexpr int kVec = 8;
};
struct F32 {
    using elem_t = float;
    static constexpr int kVec = 4;
};

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ void unpack(Bf16, const u32x4& v, float* f)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(v[i] << 16);
        f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void unpack(F32, const u32x4& v, float* f)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
}

// fp32 -> bf16 round to nearest even (gfx950 converts natively; NaN stays NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    __bf16 a = (__bf16)lo;
    __bf16 b = (__bf16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}
__device__ __forceinline__ u32x4 pack(Bf16, const float* f)
{
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    return v;
}
__device__ __forceinline__ u32x4 pack(F32, const float* f)
{
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(f[i]);
    return v;
}

__device__ __forceinline__ float to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ void from_f32(float v, uint16_t* p)
{
    __bf16 a = (__bf16)v;
    *p = __builtin_bit_cast(uint16_t, a);
}
__device__ __forceinline__ void from_f32(float v, float* p) { *p = v; }

// ---------------------------------------------------------------- memory

// Streaming 16-byte accesses: inputs are read once and outputs written once,
// so both are marked nontemporal.
__device__ __forceinline__ u32x4 ld_stream(const void* p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st_stream(void* p, const u32x4& v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ u32x4 ld_cached(const void* p)
{
    return *reinterpret_cast<const u32x4*>(p);
}

// Exchange slots: {tag (high 32 bits), fp32 partial (low 32 bits)} written and
// read as one 64-bit agent-scope atomic, so value and readiness arrive together
// and no separate fence is needed.
__device__ __forceinline__ void slot_publish(unsigned long long* s, uint32_t tag, float v)
{
    unsigned long long w = ((unsigned long long)tag << 32) | __float_as_uint(v);
    __hip_atomic_store(s, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long slot_read(const unsigned long long* s)
{
    return __hip_atomic_load(s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- reductions

// Sum over a full wave64 (EXEC must be all ones). Rows of 16 lanes reduce with
// DPP (xor 1, xor 2, half-mirror, mirror), leaving the row sum in every lane
// of the row; the four row sums are then added in lane order 0, 16, 32, 48.
// Fixed order, so results are bitwise reproducible.
__device__ __forceinline__ float wave_sum(float v)
{
#define QKN_DPP(ctrl) \
    __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), ctrl, 0xF, 0xF, false))
    v += QKN_DPP(0xB1);   // quad_perm [1,0,3,2]
    v += QKN_DPP(0x4E);   // quad_perm [2,3,0,1]
    v += QKN_DPP(0x141);  // row_half_mirror
    v += QKN_DPP(0x140);  // row_mirror
#undef QKN_DPP
    const int b = __builtin_bit_cast(int, v);
    float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
    float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
    float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
    return ((r0 + r1) + r2) + r3;
}

// ================================================================ fused kernel

struct FusedParams {
    const void* x[2];      // q, k            [T][H[i]]
    const void* gamma[2];  // gamma_q, gamma_k [H[i]]
    void* y[2];            // out_q, out_k    [T][H[i]]
    int64_t T;
    int64_t n_tiles;
    int32_t H[2];          // full widths (the RMS divisor)
    int32_t Wv[2];         // shard width in 16-byte vectors
    int32_t rows;          // tokens per tile
    int32_t n_shards;
    int32_t n_groups;
    int32_t xcd_map;
    float eps;
    uint32_t tag_base;     // tag of this call's first tile; tile i of a group uses tag_base + i
    unsigned long long* slots;  // [n_groups][2][n_shards][2*RMAX]
    uint32_t* fault;
    uint64_t spin_ticks;   // wall-clock ticks a comm wave may wait for one tile
    uint32_t test_flags;   // bit 0: never publish (forces the timeout path)
};

// Workgroup = 1 comm wave (wave 0) + NWD data waves. Every workgroup owns one
// logical shard and one group; a group is the n_shards workgroups that
// together cover a token tile (rows tokens x all columns of Q and of K).
// Data slots: a tile's Q part (rows x Wv[0] vectors) followed by its K part
// (rows x Wv[1] vectors), dealt to data threads round-robin, VPT per thread.
// The slot layout is the same for every tile, so gamma is loaded once.
template <class DT, int NWD, int VPT, int RMAX, bool PREFETCH>
__global__ void __launch_bounds__(64 * (NWD + 1))
fused_qknorm_kernel(FusedParams p)
{
    using elem_t = typename DT::elem_t;
    constexpr int EV = DT::kVec;
    constexpr int NSEG = 2 * RMAX;  // segments: (tensor, row) pairs of a tile
    constexpr int NDT = 64 * NWD;   // data threads

    __shared__ float red[NWD][NSEG];  // per-wave partial sums of squares
    __shared__ float rinv_s[NSEG];    // combined reciprocal RMS per segment

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // readfirstlane makes the wave index a scalar, so the comm/data split below
    // is a scalar branch: each wave executes only its own path's barriers.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int N = p.n_shards;
    const int rows = p.rows;

    // ---- decomposition (which shard, which group) -------------------------
    // With xcd_map, workgroups b and b' belong to one group only if
    // b % 8 == b' % 8: consecutive workgroup ids are dispatched round-robin to
    // the 8 XCDs, so a group's exchange stays inside one XCD's L2.
    int shard, group;
    {
        const int b = blockIdx.x;
        if (p.xcd_map) {
            const int j = b >> 3;
            shard = j % N;
            group = (j / N) * 8 + (b & 7);
        } else {
            shard = b % N;
            group = b / N;
        }
    }

    if (wave == 0) {
        // ================= comm wave: publish, acquire, combine =============
        const int kk = lane / NSEG;          // shard of the slot this lane watches
        const int sg = lane % NSEG;          // segment of that slot
        const bool seg_used = (sg % RMAX) < rows;
        const bool mine = seg_used && kk == shard && lane < N * NSEG;
        const bool peer = seg_used && kk != shard && lane < N * NSEG;
        const float Hf = (float)(sg < RMAX ? p.H[0] : p.H[1]);
        bool abandon = false;
        int it = 0;
        for (int64_t tile = group; tile < p.n_tiles; tile += p.n_groups, ++it) {
            __syncthreads();  // B1: data waves have written red[][]
            unsigned long long* slot =
                p.slots + ((size_t)(group * 2 + (it & 1)) * N) * NSEG + lane;
            const uint32_t want = p.tag_base + (uint32_t)it;
            float v = 0.f;
            if (mine) {
                float own = 0.f;
#pragma unroll
                for (int w = 0; w < NWD; ++w) own += red[w][sg];
                v = own;
                if (N > 1 && !(p.test_flags & 1u)) slot_publish(slot, want, own);
            }
            bool need = peer;
            if (N > 1 && !abandon) {
                const uint64_t t0 = wall_clock64();
                while (__any(need)) {
                    if (need) {
                        const unsigned long long w = slot_read(slot);
                        if ((uint32_t)(w >> 32) == want) {
                            v = __uint_as_float((uint32_t)w);
                            need = false;
                        }
                    }
                    if (!__any(need)) break;
                    if (wall_clock64() - t0 > p.spin_ticks) {
                        if (lane == 0) atomicOr(p.fault, 1u);
                        abandon = true;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
            }
            // S = sum over shards k = 0..N-1 in ascending order (same on every shard)
            float S = 0.f;
            for (int k2 = 0; k2 < N; ++k2) S += __shfl(v, k2 * NSEG + sg);
            if (lane < NSEG && seg_used) rinv_s[lane] = 1.0f / sqrtf(S / Hf + p.eps);
            __syncthreads();  // B2: rinv_s ready
        }
        return;
    }

    // ===================== data waves ========================================
    const int dt = tid - 64;  // data thread index
    const int dwave = wave - 1;
    const int V0 = rows * p.Wv[0];
    const int V = V0 + rows * p.Wv[1];

    // Static per-slot layout: element offset from the tile's first row, tensor,
    // segment, validity. gamma for the slot's columns is held in registers.
    int32_t off[VPT];
    int meta[VPT];  // bits 0..7 segment, bit 8 tensor 1, bit 9 valid
    u32x4 gam[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int v = dt + i * NDT;
        int t = 0, r = 0, c = 0;
        if (v < V0) {
            r = v / p.Wv[0];
            c = v - r * p.Wv[0];
        } else {
            t = 1;
            r = (v - V0) / p.Wv[1];
            c = (v - V0) - r * p.Wv[1];
        }
        const int col = (shard * p.Wv[t] + c) * EV;  // element column inside the row
        off[i] = r * p.H[t] + col;
        const bool valid = v < V;
        meta[i] = (t * RMAX + r) | (t << 8) | ((valid ? 1 : 0) << 9);
        gam[i] = valid ? ld_cached(static_cast<const elem_t*>(p.gamma[t]) + col) : u32x4{0, 0, 0, 0};
    }

    const elem_t* x0 = static_cast<const elem_t*>(p.x[0]);
    const elem_t* x1 = static_cast<const elem_t*>(p.x[1]);
    elem_t* y0 = static_cast<elem_t*>(p.y[0]);
    elem_t* y1 = static_cast<elem_t*>(p.y[1]);

    auto live = [&](int i, int64_t t0) {
        return (meta[i] & 512) && (t0 + ((meta[i] & 255) % RMAX) < p.T);
    };
    auto load_tile = [&](int64_t tile, u32x4 (&buf)[VPT]) {
        const int64_t t0 = tile * rows;
        const elem_t* b0 = x0 + t0 * p.H[0];
        const elem_t* b1 = x1 + t0 * p.H[1];
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            if (live(i, t0)) {
                const elem_t* src = ((meta[i] & 256) ? b1 : b0) + off[i];
                buf[i] = ld_stream(src);
            } else {
                buf[i] = u32x4{0, 0, 0, 0};
            }
        }
    };

    u32x4 cur[VPT];
    u32x4 nxt[VPT];
    int64_t tile = group;
    if (tile < p.n_tiles) load_tile(tile, cur);

    for (; tile < p.n_tiles; tile += p.n_groups) {
        const int64_t t0 = tile * rows;
        if (!PREFETCH && tile != group) load_tile(tile, cur);

        // ---- Phase A: local sums of squares (fp32) ---------------------------
        float acc[NSEG];
#pragma unroll
        for (int s = 0; s < NSEG; ++s) acc[s] = 0.f;
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            float f[EV];
            unpack(DT{}, cur[i], f);
            float sq = 0.f;
#pragma unroll
            for (int e = 0; e < EV; ++e) sq = fmaf(f[e], f[e], sq);
            const int sg = meta[i] & 255;
#pragma unroll
            for (int s = 0; s < NSEG; ++s) acc[s] += (sg == s) ? sq : 0.f;
        }
#pragma unroll
        for (int s = 0; s < NSEG; ++s) {
            if ((s % RMAX) < rows) {
                const float w = wave_sum(acc[s]);
                if (lane == 0) red[dwave][s] = w;
            }
        }
        __syncthreads();  // B1

        // ---- prefetch the next tile while the exchange is in flight -----------
        const int64_t next = tile + p.n_groups;
        if (PREFETCH && next < p.n_tiles) load_tile(next, nxt);

        // ---- Phase B (compute path): u = x * gamma, independent of the exchange
        float u[VPT][EV];
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            float f[EV], g[EV];
            unpack(DT{}, cur[i], f);
            unpack(DT{}, gam[i], g);
#pragma unroll
            for (int e = 0; e < EV; ++e) u[i][e] = f[e] * g[e];
        }
        __syncthreads();  // B2: rinv_s from the comm wave

        // ---- Phase C: y = u * rinv, one rounding to the output format ----------
        elem_t* o0 = y0 + t0 * p.H[0];
        elem_t* o1 = y1 + t0 * p.H[1];
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            if (live(i, t0)) {
                const float r = rinv_s[meta[i] & 255];
                float o[EV];
#pragma unroll
                for (int e = 0; e < EV; ++e) o[e] = u[i][e] * r;
                elem_t* dst = ((meta[i] & 256) ? o1 : o0) + off[i];
                st_stream(dst, pack(DT{}, o));
            }
        }
        if (PREFETCH) {
#pragma unroll
            for (int i = 0; i < VPT; ++i) cur[i] = nxt[i];
        }
    }
}

// ================================================================ split kernels

// Phase A alone: partials[s*T + t] = sum of x[t][j]^2 over shard s (fp32).
// One wave per (token, shard) item, items token-major; 4 waves per workgroup.
template <class DT, bool VEC>
__global__ void __launch_bounds__(256)
shard_sumsq_kernel(const void* x_, int64_t T, int32_t H, int32_t N, float* partials)
{
    using elem_t = typename DT::elem_t;
    constexpr int EV = DT::kVec;
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= T * N) return;  // wave-uniform
    const int64_t t = item / N;
    const int s = (int)(item - t * N);
    const int W = H / N;
    const elem_t* row = static_cast<const elem_t*>(x_) + t * H + (int64_t)s * W;
    float acc = 0.f;
    if (VEC) {
        const int Wv = W / EV;
        for (int v = lane; v < Wv; v += 64) {
            float f[EV];
            unpack(DT{}, ld_stream(row + v * EV), f);
#pragma unroll
            for (int e = 0; e < EV; ++e) acc = fmaf(f[e], f[e], acc);
        }
    } else {
        for (int j = lane; j < W; j += 64) {
            const float f = to_f32(row[j]);
            acc = fmaf(f, f, acc);
        }
    }
    acc = wave_sum(acc);
    if (lane == 0) partials[(int64_t)s * T + t] = acc;
}

// Phase B combine alone: rms_inv[t] = 1/sqrt(sum_s partials[s][t] / H + eps),
// shards added in ascending order.
__global__ void __launch_bounds__(256)
combine_scale_kernel(const float* partials, int64_t T, int32_t H, int32_t N, float eps,
                     float* rms_inv)
{
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= T) return;
    float S = 0.f;
    for (int s = 0; s < N; ++s) S += partials[(int64_t)s * T + t];
    rms_inv[t] = 1.0f / sqrtf(S / (float)H + eps);
}

// Phases B (x*gamma) and C alone: out = x * gamma * rms_inv. A workgroup
// covers `rpb` consecutive rows; its threads walk the rows' vectors linearly.
template <class DT, bool VEC>
__global__ void __launch_bounds__(256)
apply_scale_kernel(const void* x_, const void* g_, const float* rms_inv, int64_t T, int32_t H,
                   int32_t rpb, void* y_)
{
    using elem_t = typename DT::elem_t;
    constexpr int EV = DT::kVec;
    const elem_t* x = static_cast<const elem_t*>(x_);
    const elem_t* g = static_cast<const elem_t*>(g_);
    elem_t* y = static_cast<elem_t*>(y_);
    const int64_t r0 = (int64_t)blockIdx.x * rpb;
    const int unit = VEC ? EV : 1;
    const int per_row = H / unit;
    const int total = rpb * per_row;
    for (int v = threadIdx.x; v < total; v += 256) {
        const int rl = v / per_row;
        const int c = v - rl * per_row;
        const int64_t t = r0 + rl;
        if (t >= T) break;
        const float r = rms_inv[t];
        const int64_t base = t * H + (int64_t)c * unit;
        if (VEC) {
            float f[EV], gg[EV], o[EV];
            unpack(DT{}, ld_stream(x + base), f);
            unpack(DT{}, ld_cached(g + c * EV), gg);
#pragma unroll
            for (int e = 0; e < EV; ++e) o[e] = (f[e] * gg[e]) * r;
            st_stream(y + base, pack(DT{}, o));
        } else {
            const float o = (to_f32(x[base]) * to_f32(g[c])) * r;
            from_f32(o, y + base);
        }
    }
}

// ================================================================ copy ceiling

// Same access widths as the fused kernel (16-byte nontemporal loads and
// stores); bytes beyond the last full vector are copied one byte at a time.
__global__ void __launch_bounds__(256)
copy2_kernel(const void* a, const void* b, void* oa, void* ob, int64_t va, int64_t vb,
             int64_t ta, int64_t tb)
{
    const int64_t n = va + vb;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < n; v += stride) {
        if (v < va) {
            st_stream(static_cast<char*>(oa) + v * 16, ld_stream(static_cast<const char*>(a) + v * 16));
        } else {
            const int64_t w = v - va;
            st_stream(static_cast<char*>(ob) + w * 16, ld_stream(static_cast<const char*>(b) + w * 16));
        }
    }
    if (blockIdx.x == 0) {
        for (int64_t i = threadIdx.x; i < ta; i += 256)
            static_cast<char*>(oa)[va * 16 + i] = static_cast<const char*>(a)[va * 16 + i];
        for (int64_t i = threadIdx.x; i < tb; i += 256)
            static_cast<char*>(ob)[vb * 16 + i] = static_cast<const char*>(b)[vb * 16 + i];
    }
}

}  // namespace qkn
