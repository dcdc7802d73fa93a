// Measurement kernel: the copy skeleton of a fused launch. Kept apart from the
// fused kernels' source, which it shares nothing with but the helpers it includes.
#pragma once
#include "qknorm_ceilings.hpp"

namespace qkn {

// ================================================================ measurement

// Copy skeleton of a fused launch: the fused kernel's grid, workgroups (one
// wave that only passes the barriers plus `nwd` data waves), group and shard
// mapping, slot layout, tile stride loop, one barrier per iteration, pacing
// and one-tile prefetch, with no arithmetic and no exchange: each tile's bytes of
// x are stored unchanged to y (WIDEN: each byte zero-extended to a 16-bit
// word, the byte mix of E4M3 inputs with bf16 outputs). It measures what the
// persistent streaming structure itself can move.
struct SkeletonParams {
    const void* x[2];  // q, k  [T][H[i]]
    void* y[2];        // out_q, out_k
    int64_t T;
    int64_t n_tiles;
    int64_t nq;        // single-tensor tiles: tiles 0..nq-1 hold Q rows
    int32_t H[2];      // widths in elements
    int32_t Wv[2];     // shard widths in 16-byte vectors of x
    int32_t rows, nwd, n_shards, n_groups, xcd_map;
    int32_t in_bytes;  // element size of x
    uint32_t pace;     // the fused launch's pacing period (1/256 wall-clock ticks; 0: none)
    uint32_t stagger;  // 1 = group g's schedule starts g/n_groups periods late
};

template <int VPT, bool ST, bool WIDEN>
__global__ void __launch_bounds__(1024)
skeleton_kernel(SkeletonParams p)
{
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int N = p.n_shards;
    const int rows = p.rows;
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
    const int K = p.n_tiles > group ? (int)((p.n_tiles - 1 - group) / p.n_groups + 1) : 0;
    if (K == 0) return;
    if (wave == 0) {
        // passes the barriers, paced as the fused kernel's comm wave paces them
        const uint64_t t_entry = p.pace ? wall_clock64() : 0;
        const uint64_t phase = p.stagger ? (uint64_t)group * p.pace / (uint64_t)p.n_groups : 0;
        for (int k = 0; k <= K; ++k) {
            if (p.pace) {
                const uint64_t due = t_entry + (((uint64_t)k * p.pace + phase) >> 8);
                while (wall_clock64() < due) __builtin_amdgcn_s_sleep(1);
            }
            __syncthreads();
        }
        return;
    }
    const int dwave = wave - 1;
    const int ndt = 64 * p.nwd;
    const int ES = p.in_bytes;
    const int OS = WIDEN ? 2 * ES : ES;
    const int EV = 16 / ES;
    const int VQ = rows * p.Wv[0];
    const int VQp = ST ? VQ : (VQ + 63) & ~63;
    const int V = ST ? VQ : VQp + rows * p.Wv[1];
    constexpr uint32_t kOOB = 0x80000000u;
    uint32_t voff[VPT];                 // input byte offset from the tile's first row, or kOOB
    uint32_t poff[WIDEN ? VPT : 1][2];  // WIDEN: the lane's offsets for its two stores
    bool tk[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int vbase = i * ndt + dwave * 64;
        const int t = (!ST && vbase >= VQp) ? 1 : 0;
        // (valid, byte offset in x) of the slot's vector vbase + m
        auto locate = [&](int m, uint32_t& off) __attribute__((always_inline)) -> bool {
            const int v = vbase + m;
            const int u = t ? v - VQp : v;
            const int r = u / p.Wv[t];
            const int c = u - r * p.Wv[t];
            off = (uint32_t)((r * p.H[t] + (shard * p.Wv[t] + c) * EV) * ES);
            return t ? v < V : v < VQ;
        };
        uint32_t o;
        voff[i] = locate(lane, o) ? o : kOOB;
        tk[i] = t != 0;
        if constexpr (WIDEN) {
            // as in the fused kernel: store h covers the slot's vectors 32h..32h+31,
            // lanes 0-31 writing their first 16 output bytes, lanes 32-63 the second
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t oh;
                poff[i][h] = locate(32 * h + (lane & 31), oh) ? 2 * oh + 16 * (lane >> 5) : kOOB;
            }
        }
    }
    auto rsrc = [&](const void* base, int t, int eb) __attribute__((always_inline)) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                                 (int)(p.T * p.H[t] * eb), 0x00020000);
    };
    const __amdgpu_buffer_rsrc_t dxq = rsrc(p.x[0], 0, ES), dxk = rsrc(p.x[1], 1, ES);
    const __amdgpu_buffer_rsrc_t dyq = rsrc(p.y[0], 0, OS), dyk = rsrc(p.y[1], 1, OS);
    auto row_off = [&](int64_t tile, int t, int eb) __attribute__((always_inline)) -> uint32_t {
        int64_t t0 = tile * rows;
        t0 = t0 < p.T ? t0 : p.T;
        return (uint32_t)(t0 * p.H[t] * eb);
    };
    auto tile_of = [&](int k) __attribute__((always_inline)) -> int64_t { return group + (int64_t)k * p.n_groups; };
    // the tensor of each slot and the tile's byte offset in it (input, output)
    auto place = [&](int64_t tile, int i, int eb) __attribute__((always_inline)) -> uint32_t {
        if constexpr (ST) {
            const bool kt = tile >= p.nq;
            return row_off(kt ? tile - p.nq : tile, kt ? 1 : 0, eb);
        } else {
            return row_off(tile, tk[i] ? 1 : 0, eb);
        }
    };
    auto is_k = [&](int64_t tile, int i) __attribute__((always_inline)) -> bool {
        if constexpr (ST) return tile >= p.nq;
        else return tk[i];
    };
    auto load_tile = [&](int64_t tile, u32x4 (&buf)[VPT]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < VPT; ++i)
            buf[i] = __builtin_amdgcn_raw_buffer_load_b128(is_k(tile, i) ? dxk : dxq, voff[i] + place(tile, i, ES), 0, kNT);
    };
    auto store_tile = [&](int64_t tile, const u32x4 (&buf)[VPT]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const __amdgpu_buffer_rsrc_t d = is_k(tile, i) ? dyk : dyq;
            if constexpr (WIDEN) {
                const u32x4 w0 = widen_bytes(buf[i][0], buf[i][1]), w1 = widen_bytes(buf[i][2], buf[i][3]);
                u32x4 s0, s1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const auto sw = __builtin_amdgcn_permlane32_swap(w0[e], w1[e], false, false);
                    s0[e] = sw[0];
                    s1[e] = sw[1];
                }
                const uint32_t base = place(tile, i, OS);
                __builtin_amdgcn_raw_buffer_store_b128(s0, d, poff[i][0] + base, 0, kNT);
                __builtin_amdgcn_raw_buffer_store_b128(s1, d, poff[i][1] + base, 0, kNT);
            } else {
                __builtin_amdgcn_raw_buffer_store_b128(buf[i], d, voff[i] + place(tile, i, OS), 0, kNT);
            }
        }
    };
    u32x4 cur[VPT], nxt[VPT];
    if (p.pace && p.stagger) {
        const uint64_t due = wall_clock64() + (((uint64_t)group * p.pace / (uint64_t)p.n_groups) >> 8);
        while (wall_clock64() < due) __builtin_amdgcn_s_sleep(1);
    }
    load_tile(tile_of(0), cur);
    wait_vmcnt<0>();
    __syncthreads();
    for (int k = 0; k < K; ++k) {
        const bool more = k + 1 < K;
        if (more) load_tile(tile_of(k + 1), nxt);
        store_tile(tile_of(k), cur);
        __syncthreads();
        if (more) {
            // the loads before the stores just issued must be done; as in the
            // fused kernel, VPT stores may stay in flight (WIDEN: the first VPT
            // of its 2*VPT stores complete too)
            wait_vmcnt<VPT>();
#pragma unroll
            for (int i = 0; i < VPT; ++i) cur[i] = nxt[i];
        }
    }
}

}  // namespace qkn
