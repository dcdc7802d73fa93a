// Host runtime and C ABI of the layerwise QK-Norm library (see include/qknorm.h).
//
// Responsibilities: synchronous argument validation; launch planning (kernel
// variant, tile rows, a persistent grid bounded by co-residency -- "SwiftQK",
// Section III-D: at most B_res x N_CU workgroups so that every member of an
// exchange is resident); one workspace per (device, stream) holding the
// exchange slots and the fault word; kernel launches on the caller's stream.
#include "qknorm.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <type_traits>
#include <utility>

#include "qknorm_kernels.hpp"
#include "qknorm_skeleton.hpp"

namespace {

using qkn::Bf16;
using qkn::E4m3Bf16;
using qkn::E4m3E4m3;
using qkn::F32;
using qkn::FusedParams;

// ---------------------------------------------------------------- formats

// Element sizes of x, gamma and y of a format; `ev` columns per 16-byte
// vector of x, `kgam` 16-byte words of gamma per vector; `stats` statistics
// per token and shard (1: sum of squares; 2 for LayerNorm: also the sum) and
// `params` per-column vectors staged in LDS (gamma; LayerNorm: and beta).
struct Fmt {
    int in, gam, out, ev, kgam, stats, params;
};
bool fmt_valid(int f) { return f >= 0 && f < QKN_NUM_FORMATS; }
Fmt fmt_of(int f)
{
    switch (f) {
    case QKN_FMT_BF16: return {2, 2, 2, 8, 1, 1, 1};
    case QKN_FMT_F32: return {4, 4, 4, 4, 1, 1, 1};
    case QKN_FMT_E4M3_BF16: return {1, 2, 2, 16, 2, 1, 1};
    case QKN_FMT_E4M3_E4M3: return {1, 2, 1, 16, 2, 1, 1};
    case QKN_FMT_LN_BF16: return {2, 2, 2, 8, 1, 2, 2};
    default: return {4, 4, 4, 4, 1, 2, 2};  // QKN_FMT_LN_F32
    }
}
bool is_layernorm(int f) { return f == QKN_FMT_LN_BF16 || f == QKN_FMT_LN_F32; }
// format of an E4M3 call with output dtype `out` (QKN_BF16 or QKN_E4M3), or -1
int e4m3_fmt(int out)
{
    if (out == QKN_BF16) return QKN_FMT_E4M3_BF16;
    if (out == QKN_E4M3) return QKN_FMT_E4M3_E4M3;
    return -1;
}

// ---------------------------------------------------------------- variants

// Which formats instantiate a variant is decided by fused_fn_for below.
struct Variant {
    int vpt;          // 16-byte slots per data thread
    bool prefetch;    // next tile loaded during the exchange
    int lag;          // tiles between a tile's reduction and its scaling
    int max_threads;  // launch bound of the instantiation
};
constexpr Variant kVariants[QKN_NUM_VARIANTS] = {
    {1, true, 1, 1024},
    {2, true, 1, 1024},
    {3, true, 1, 1024},
    {4, true, 1, 1024},
    {6, true, 1, 768},
    {9, false, 1, 1024},  // fp32 only: no room for a prefetch buffer
    {1, true, 2, 1024},
    {2, true, 2, 1024},
    {3, true, 2, 768},
    {4, true, 2, 512},
    // bf16 single-tensor tiles only: four data waves and the comm wave, one
    // wave per SIMD, so no SIMD runs two data waves' arithmetic (reached
    // through the tuned table or QKN_OPT_FORCE_VARIANT, not the scored search)
    {5, true, 2, 320},
};

using FusedFn = void (*)(FusedParams);

// Instantiated variants per format. The 16-byte formats (bf16, fp32) have all
// but variant 5 (fp32 only); E4M3 vectors hold 16 columns, so their u
// registers double and only variants with up to 3 vectors per thread (lag 1)
// or 2 (lag 2) are instantiated.
template <class DT>
FusedFn fused_fn(int v)
{
    switch (v) {
    case 0: return qkn::fused_qknorm_kernel<DT, 1, true, 1, 1024>;
    case 1: return qkn::fused_qknorm_kernel<DT, 2, true, 1, 1024>;
    case 2: return qkn::fused_qknorm_kernel<DT, 3, true, 1, 1024>;
    case 3: return qkn::fused_qknorm_kernel<DT, 4, true, 1, 1024>;
    case 4: return qkn::fused_qknorm_kernel<DT, 6, true, 1, 768>;
    case 6: return qkn::fused_qknorm_kernel<DT, 1, true, 2, 1024>;
    case 7: return qkn::fused_qknorm_kernel<DT, 2, true, 2, 1024>;
    case 8: return qkn::fused_qknorm_kernel<DT, 3, true, 2, 768>;
    case 9: return qkn::fused_qknorm_kernel<DT, 4, true, 2, 512>;
    default: return nullptr;  // variant 10: single-tensor tiles only
    }
}
template <>
FusedFn fused_fn<F32>(int v)
{
    switch (v) {
    case 0: return qkn::fused_qknorm_kernel<F32, 1, true, 1, 1024>;
    case 1: return qkn::fused_qknorm_kernel<F32, 2, true, 1, 1024>;
    case 2: return qkn::fused_qknorm_kernel<F32, 3, true, 1, 1024>;
    case 3: return qkn::fused_qknorm_kernel<F32, 4, true, 1, 1024>;
    case 4: return qkn::fused_qknorm_kernel<F32, 6, true, 1, 768>;
    case 5: return qkn::fused_qknorm_kernel<F32, 9, false, 1, 1024>;
    case 6: return qkn::fused_qknorm_kernel<F32, 1, true, 2, 1024>;
    case 7: return qkn::fused_qknorm_kernel<F32, 2, true, 2, 1024>;
    case 8: return qkn::fused_qknorm_kernel<F32, 3, true, 2, 768>;
    case 9: return qkn::fused_qknorm_kernel<F32, 4, true, 2, 512>;
    default: return nullptr;
    }
}
// E4M3 launch bounds: variants 2 and 7 need more registers than 1024 threads allow
constexpr int kE4m3MaxThreads[QKN_NUM_VARIANTS] = {1024, 1024, 768, 0, 0, 0, 1024, 768, 0, 0, 0};
template <class DT>
FusedFn fused_fn_e4m3(int v)
{
    switch (v) {
    case 0: return qkn::fused_qknorm_kernel<DT, 1, true, 1, kE4m3MaxThreads[0]>;
    case 1: return qkn::fused_qknorm_kernel<DT, 2, true, 1, kE4m3MaxThreads[1]>;
    case 2: return qkn::fused_qknorm_kernel<DT, 3, true, 1, kE4m3MaxThreads[2]>;
    case 6: return qkn::fused_qknorm_kernel<DT, 1, true, 2, kE4m3MaxThreads[6]>;
    case 7: return qkn::fused_qknorm_kernel<DT, 2, true, 2, kE4m3MaxThreads[7]>;
    default: return nullptr;
    }
}
// LayerNorm (NORM = 1) for bf16 and fp32: every variant except 5, whose gamma
// and beta images would not fit in LDS
template <class DT>
FusedFn fused_fn_ln(int v)
{
    switch (v) {
    case 0: return qkn::fused_qknorm_kernel<DT, 1, true, 1, 1024, 1>;
    case 1: return qkn::fused_qknorm_kernel<DT, 2, true, 1, 1024, 1>;
    case 2: return qkn::fused_qknorm_kernel<DT, 3, true, 1, 1024, 1>;
    case 3: return qkn::fused_qknorm_kernel<DT, 4, true, 1, 1024, 1>;
    case 4: return qkn::fused_qknorm_kernel<DT, 6, true, 1, 512, 1>;
    case 6: return qkn::fused_qknorm_kernel<DT, 1, true, 2, 1024, 1>;
    case 7: return qkn::fused_qknorm_kernel<DT, 2, true, 2, 1024, 1>;
    case 8: return qkn::fused_qknorm_kernel<DT, 3, true, 2, 768, 1>;
    case 9: return qkn::fused_qknorm_kernel<DT, 4, true, 2, 512, 1>;
    default: return nullptr;
    }
}
FusedFn fused_fn_for(int fmt, int v)
{
    switch (fmt) {
    case QKN_FMT_BF16: return fused_fn<Bf16>(v);
    case QKN_FMT_F32: return fused_fn<F32>(v);
    case QKN_FMT_E4M3_BF16: return fused_fn_e4m3<E4m3Bf16>(v);
    case QKN_FMT_E4M3_E4M3: return fused_fn_e4m3<E4m3E4m3>(v);
    case QKN_FMT_LN_BF16: return fused_fn_ln<Bf16>(v);
    default: return fused_fn_ln<F32>(v);
    }
}
// Single-tensor tiles (Hq == Hk): the variants with 1-4 vectors per thread
// (E4M3: 1-3 with a one-tile lag, 1-2 with two), with the launch bounds of the
// format's mixed-tile kernels.
template <class DT, int NORM>
FusedFn fused_fn_st(int v)
{
    switch (v) {
    case 0: return qkn::fused_qknorm_kernel<DT, 1, true, 1, 1024, NORM, true>;
    case 1: return qkn::fused_qknorm_kernel<DT, 2, true, 1, 1024, NORM, true>;
    case 2: return qkn::fused_qknorm_kernel<DT, 3, true, 1, 1024, NORM, true>;
    case 3: return qkn::fused_qknorm_kernel<DT, 4, true, 1, 1024, NORM, true>;
    case 6: return qkn::fused_qknorm_kernel<DT, 1, true, 2, 1024, NORM, true>;
    case 7: return qkn::fused_qknorm_kernel<DT, 2, true, 2, 1024, NORM, true>;
    case 8: return qkn::fused_qknorm_kernel<DT, 3, true, 2, 768, NORM, true>;
    case 9: return qkn::fused_qknorm_kernel<DT, 4, true, 2, 512, NORM, true>;
    case 10:
        if constexpr (std::is_same<DT, Bf16>::value && NORM == 0)
            return qkn::fused_qknorm_kernel<DT, 5, true, 2, 320, NORM, true>;
        return nullptr;
    default: return nullptr;
    }
}
template <class DT>
FusedFn fused_fn_st_e4m3(int v)
{
    switch (v) {
    case 0: return qkn::fused_qknorm_kernel<DT, 1, true, 1, kE4m3MaxThreads[0], 0, true>;
    case 1: return qkn::fused_qknorm_kernel<DT, 2, true, 1, kE4m3MaxThreads[1], 0, true>;
    case 2: return qkn::fused_qknorm_kernel<DT, 3, true, 1, kE4m3MaxThreads[2], 0, true>;
    case 6: return qkn::fused_qknorm_kernel<DT, 1, true, 2, kE4m3MaxThreads[6], 0, true>;
    case 7: return qkn::fused_qknorm_kernel<DT, 2, true, 2, kE4m3MaxThreads[7], 0, true>;
    default: return nullptr;
    }
}
// kernel of a format, variant and tile layout (st: single-tensor tiles)
FusedFn fused_fn_layout(int fmt, int v, bool st)
{
    if (!st) return fused_fn_for(fmt, v);
    switch (fmt) {
    case QKN_FMT_BF16: return fused_fn_st<Bf16, 0>(v);
    case QKN_FMT_F32: return fused_fn_st<F32, 0>(v);
    case QKN_FMT_E4M3_BF16: return fused_fn_st_e4m3<E4m3Bf16>(v);
    case QKN_FMT_E4M3_E4M3: return fused_fn_st_e4m3<E4m3E4m3>(v);
    case QKN_FMT_LN_BF16: return fused_fn_st<Bf16, 1>(v);
    default: return fused_fn_st<F32, 1>(v);
    }
}
// Paced builds of the kernels the tuned table paces. On one schedule for every
// group (PACE = 1): bf16 variant 8 on mixed tiles (GQA), E4M3 -> bf16 variant 0
// on single-tensor tiles and 7 on mixed tiles, E4M3 -> E4M3 variant 7 on
// single-tensor tiles. Staggered (PACE = 2): bf16 variant 10 on single-tensor
// tiles (the prefill split one and two ways), E4M3 -> bf16 variant 7 on
// single-tensor tiles (split two ways) and LayerNorm bf16 variant 7 on
// single-tensor tiles (split two ways) and on mixed tiles. nullptr for every
// other kernel, which runs unpaced.
FusedFn paced_fn(int fmt, int v, bool st)
{
    if (fmt == QKN_FMT_BF16 && v == 10 && st) return qkn::fused_qknorm_kernel<Bf16, 5, true, 2, 320, 0, true, 2>;
    if (fmt == QKN_FMT_LN_BF16 && v == 7 && st) return qkn::fused_qknorm_kernel<Bf16, 2, true, 2, 1024, 1, true, 2>;
    if (fmt == QKN_FMT_LN_BF16 && v == 7 && !st) return qkn::fused_qknorm_kernel<Bf16, 2, true, 2, 1024, 1, false, 2>;
    if (fmt == QKN_FMT_BF16 && v == 8 && !st) return qkn::fused_qknorm_kernel<Bf16, 3, true, 2, 768, 0, false, 1>;
    if (fmt == QKN_FMT_E4M3_BF16 && v == 7 && st)
        return qkn::fused_qknorm_kernel<E4m3Bf16, 2, true, 2, kE4m3MaxThreads[7], 0, true, 2>;
    if (fmt == QKN_FMT_E4M3_BF16 && v == 0 && st)
        return qkn::fused_qknorm_kernel<E4m3Bf16, 1, true, 1, kE4m3MaxThreads[0], 0, true, 1>;
    if (fmt == QKN_FMT_E4M3_BF16 && v == 7 && !st)
        return qkn::fused_qknorm_kernel<E4m3Bf16, 2, true, 2, kE4m3MaxThreads[7], 0, false, 1>;
    if (fmt == QKN_FMT_E4M3_E4M3 && v == 7 && st)
        return qkn::fused_qknorm_kernel<E4m3E4m3, 2, true, 2, kE4m3MaxThreads[7], 0, true, 1>;
    return nullptr;
}
// Measurement ceilings: threads per workgroup of the one-shot copy and
// widening kernels (each thread moves one vector; one wave per workgroup
// measured fastest for both: 100.8 against 103.4 us with four waves for the
// prefill's 671 MB copy, 75.4 against 77.7 us for its E4M3 -> bf16 widening),
// and the largest tensor (output bytes) one launch of them takes.
constexpr int kCopyThreads = 64;
constexpr int kWidenThreads = 64;
constexpr int64_t kCeilingMaxBytes = (int64_t(1) << 31) - (int64_t(1) << 16);
using SkelFn = void (*)(qkn::SkeletonParams);
template <bool ST, bool WIDEN>
SkelFn skeleton_fn_vpt(int vpt)
{
    switch (vpt) {
    case 1: return qkn::skeleton_kernel<1, ST, WIDEN>;
    case 2: return qkn::skeleton_kernel<2, ST, WIDEN>;
    case 3: return qkn::skeleton_kernel<3, ST, WIDEN>;
    case 4: return WIDEN ? nullptr : qkn::skeleton_kernel<4, ST, false>;
    case 5: return WIDEN ? nullptr : qkn::skeleton_kernel<5, ST, false>;
    case 6: return WIDEN ? nullptr : qkn::skeleton_kernel<6, ST, false>;
    case 9: return WIDEN ? nullptr : qkn::skeleton_kernel<9, ST, false>;
    default: return nullptr;
    }
}
// the skeleton matching a fused launch's vectors per thread, tile layout and byte mix
SkelFn skeleton_fn(int vpt, bool st, bool widen)
{
    if (st) return widen ? skeleton_fn_vpt<true, true>(vpt) : skeleton_fn_vpt<true, false>(vpt);
    return widen ? skeleton_fn_vpt<false, true>(vpt) : skeleton_fn_vpt<false, false>(vpt);
}
// built for this format in some tile layout (variant 10: single-tensor tiles only)
bool variant_usable(int fmt, int v) { return fused_fn_for(fmt, v) != nullptr || fused_fn_layout(fmt, v, true) != nullptr; }
// paced builds on the staggered schedule (PACE = 2)
bool paced_staggered(int fmt, int v, bool st)
{
    return (fmt == QKN_FMT_BF16 && st && v == 10) || (fmt == QKN_FMT_LN_BF16 && v == 7) ||
           (fmt == QKN_FMT_E4M3_BF16 && st && v == 7);
}
bool is_e4m3(int fmt) { return fmt == QKN_FMT_E4M3_BF16 || fmt == QKN_FMT_E4M3_E4M3; }
// data waves a workgroup of variant v may have (launch bound / 64, minus the comm wave)
int max_data_waves(int fmt, int v)
{
    int t = is_e4m3(fmt) ? kE4m3MaxThreads[v] : kVariants[v].max_threads;
    if (is_layernorm(fmt) && v == 4) t = 512;  // gamma and beta need more registers
    return t / 64 - 1;
}

// dynamic LDS of a launch: gamma (and LayerNorm's beta) in slot order, kgam
// 16-byte words per slot each
size_t gamma_lds_bytes(int fmt, int v, int nwd, bool st = false)
{
    const Fmt f = fmt_of(fmt);
    // single-tensor tiles hold gamma_q's and gamma_k's images
    return (size_t)kVariants[v].vpt * 64 * nwd * 16 * f.kgam * f.params * (st ? 2 : 1);
}

// ---------------------------------------------------------------- options

// Plans are cached per (device, dtype, shape, alignment); any option change
// bumps g_opt_epoch, which invalidates every cached plan.
struct PlanKey {
    int dev, dtype, n_shards, aligned;
    int64_t T, Hq, Hk;
    uint64_t epoch;
    bool operator<(const PlanKey& o) const
    {
        return std::tie(dev, dtype, n_shards, aligned, T, Hq, Hk, epoch) <
               std::tie(o.dev, o.dtype, o.n_shards, o.aligned, o.T, o.Hq, o.Hk, o.epoch);
    }
};
uint64_t g_opt_epoch = 0;

struct Options {
    int64_t spin_ns = 1000000000;
    int64_t force_variant = -1;
    int64_t force_data_waves = 0;
    int64_t rows = 0;
    int64_t xcd_map = -1;
    int64_t cooperative = 0;
    int64_t max_groups = 0;
    int64_t force_split = 0;
    int64_t test_skip_publish = 0;
    int64_t split_vectors = 0;
    int64_t tile_layout = 0;
    int64_t wpc = 0;
    int64_t pace_gbs = -1;
};
Options g_opt;

thread_local std::string t_hip_error;

int hip_fail(hipError_t e, const char* what)
{
    char buf[256];
    std::snprintf(buf, sizeof buf, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
    t_hip_error = buf;
    return QKN_EHIP;
}
#define QKN_HIP(call)                                         \
    do {                                                      \
        hipError_t e_ = (call);                               \
        if (e_ != hipSuccess) return hip_fail(e_, #call);     \
    } while (0)

// ---------------------------------------------------------------- device info

struct DevInfo {
    int cu = 0;
    int wall_khz = 0;
    int lds_cu = 0;  // LDS bytes per CU, the most one workgroup can hold
    bool occ_done[QKN_NUM_FORMATS] = {};
    int occ[QKN_NUM_FORMATS][QKN_NUM_VARIANTS][QKN_MAX_DATA_WAVES + 1] = {};
    // single-tensor-tile kernels
    int occ_st[QKN_NUM_FORMATS][QKN_NUM_VARIANTS][QKN_MAX_DATA_WAVES + 1] = {};
};

std::mutex g_mu;
std::map<int, DevInfo> g_dev;

// Per device: a word of pinned, device-mapped host memory that a fused launch
// sets when an exchange times out, so that the host can see a fault without
// synchronising (qknorm_fault_pending); qknorm_check_fault clears it. Its device
// address sits next to each fault word (fault + 2) of the workspaces and of the
// no-allocation scratch; launches recorded under capture set the device fault
// word only.
struct FaultFlag {
    uint32_t* host = nullptr;
    uint32_t* dev = nullptr;
};
std::map<int, FaultFlag> g_flag;

// The current device's flag, allocated on first use outside stream capture
// (null while none exists).
FaultFlag* fault_flag(int dev, bool may_alloc)
{
    FaultFlag& f = g_flag[dev];
    if (!f.host && may_alloc) {
        void* h = nullptr;
        if (hipHostMalloc(&h, 64, hipHostMallocMapped | hipHostMallocCoherent) != hipSuccess) return &f;
        void* d = nullptr;
        if (hipHostGetDevicePointer(&d, h, 0) != hipSuccess) {
            (void)hipHostFree(h);
            return &f;
        }
        *static_cast<volatile uint32_t*>(h) = 0;
        f.host = static_cast<uint32_t*>(h);
        f.dev = static_cast<uint32_t*>(d);
    }
    return &f;
}

int device_info(int dev, int dtype, DevInfo** out)
{
    DevInfo& d = g_dev[dev];
    if (d.cu == 0) {
        QKN_HIP(hipDeviceGetAttribute(&d.cu, hipDeviceAttributeMultiprocessorCount, dev));
        QKN_HIP(hipDeviceGetAttribute(&d.wall_khz, hipDeviceAttributeWallClockRate, dev));
        if (d.wall_khz <= 0) d.wall_khz = 100000;
        QKN_HIP(hipDeviceGetAttribute(&d.lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev));
    }
    if (!d.occ_done[dtype]) {
        for (int layout = 0; layout < 2; ++layout) {
            const bool st = layout == 1;
            for (int v = 0; v < QKN_NUM_VARIANTS; ++v) {
                FusedFn fn = fused_fn_layout(dtype, v, st);
                bool usable = fn != nullptr;
                // data waves whose gamma (and beta) images fit the LDS next to the
                // kernel's own arrays; more cannot be launched
                int wfit = 0;
                if (usable) {
                    hipFuncAttributes fa;
                    QKN_HIP(hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(fn)));
                    const size_t room = (size_t)d.lds_cu > fa.sharedSizeBytes ? d.lds_cu - fa.sharedSizeBytes : 0;
                    for (int w = 1; w <= max_data_waves(dtype, v); ++w)
                        if (gamma_lds_bytes(dtype, v, w, st) <= room) wfit = w;
                    usable = wfit > 0;
                }
                if (usable) {
                    QKN_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                                (int)gamma_lds_bytes(dtype, v, wfit, st)));
                }
                for (int w = 0; w <= QKN_MAX_DATA_WAVES; ++w) {
                    int n = 0;
                    if (usable && w >= 1 && w <= wfit) {
                        QKN_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(
                            &n, reinterpret_cast<const void*>(fn), 64 * (w + 1),
                            gamma_lds_bytes(dtype, v, w, st)));
                    }
                    if (st) d.occ_st[dtype][v][w] = n;
                    else d.occ[dtype][v][w] = n;
                }
            }
        }
        d.occ_done[dtype] = true;
    }
    *out = &d;
    return QKN_OK;
}

// ---------------------------------------------------------------- workspace

struct Workspace {
    int device = -1;
    unsigned long long* slots = nullptr;
    size_t slot_entries = 0;
    uint32_t* fault = nullptr;
    uint32_t tag_base = 1;
    float* scratch = nullptr;  // split fallback: partials and rms_inv
    size_t scratch_floats = 0;
};

std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

// Stores the device's timeout flag address at fault + 2 (after the fault block
// was cleared on the same stream), where a timed-out launch finds it.
int bind_fault_flag(int dev, uint32_t* fault, hipStream_t stream)
{
    const FaultFlag* f = fault_flag(dev, true);
    if (!f->dev) return QKN_OK;  // no pinned memory: device fault word only
    QKN_HIP(hipMemcpyAsync(fault + 2, &f->dev, sizeof f->dev, hipMemcpyHostToDevice, stream));
    return QKN_OK;
}

int workspace_for(int dev, hipStream_t stream, Workspace** out)
{
    Workspace& w = g_ws[{dev, stream}];
    if (!w.fault) {
        w.device = dev;
        void* p = nullptr;
        if (hipMalloc(&p, 256) != hipSuccess) return QKN_ENOMEM;
        w.fault = static_cast<uint32_t*>(p);
        QKN_HIP(hipMemsetAsync(w.fault, 0, 256, stream));
        const int rc = bind_fault_flag(dev, w.fault, stream);
        if (rc) return rc;
    }
    *out = &w;
    return QKN_OK;
}

int ensure_slots(Workspace* w, size_t entries, hipStream_t stream)
{
    if (entries <= w->slot_entries) return QKN_OK;
    if (w->slots) {
        QKN_HIP(hipStreamSynchronize(stream));
        QKN_HIP(hipFree(w->slots));
        w->slots = nullptr;
        w->slot_entries = 0;
    }
    size_t n = std::max<size_t>(entries, 1 << 15);
    void* p = nullptr;
    if (hipMalloc(&p, n * sizeof(unsigned long long)) != hipSuccess) return QKN_ENOMEM;
    w->slots = static_cast<unsigned long long*>(p);
    w->slot_entries = n;
    QKN_HIP(hipMemsetAsync(w->slots, 0, n * sizeof(unsigned long long), stream));
    w->tag_base = 1;
    return QKN_OK;
}

int ensure_scratch(Workspace* w, size_t floats, hipStream_t stream)
{
    if (floats <= w->scratch_floats) return QKN_OK;
    if (w->scratch) {
        QKN_HIP(hipStreamSynchronize(stream));
        QKN_HIP(hipFree(w->scratch));
        w->scratch = nullptr;
        w->scratch_floats = 0;
    }
    void* p = nullptr;
    if (hipMalloc(&p, floats * sizeof(float)) != hipSuccess) return QKN_ENOMEM;
    w->scratch = static_cast<float*>(p);
    w->scratch_floats = floats;
    return QKN_OK;
}

// ---------------------------------------------------------------- static scratch

// The no-allocation entry point keeps its scratch in one file-scope device
// array instead of a workspace: 64-bit exchange slots, then a block holding the
// fault word, then fp32 statistics for the split fallback. Each device holds
// its own copy until the process ends. 2^18 slots hold every bf16 RMSNorm
// launch the planner can make on a device of 256 compute units (at most 16
// workgroups per CU, each with at most 2 x lag x 2 x rows = 64 slots).
constexpr size_t kStaticSlots = size_t(1) << 18;         // 2 MiB
constexpr size_t kStaticFaultWords = 32;                  // 256 B (fault word first)
constexpr size_t kStaticSplitFloats = size_t(1) << 18;    // 1 MiB
constexpr size_t kStaticWords = kStaticSlots + kStaticFaultWords + kStaticSplitFloats / 2;

}  // namespace

// Host code never passes the array's name to a kernel or a copy: in host code it
// is a stand-in, not a device address. Each device's address comes from
// hipGetSymbolAddress (static_scratch_for below).
static __device__ __align__(256) unsigned long long scratch[kStaticWords];

// Scratch of fused launches recorded under stream capture, laid out like
// `scratch`. Every recorded launch is preceded by a recorded fill kernel that
// zeroes the slots it uses, so each replay starts from cleared slots with tags
// counted from 1; eager calls (tags from a host counter) never use it. Bound by
// address only (graph_scratch_for below), since a capturing stream may not be
// synchronised.
static __device__ __align__(256) unsigned long long graph_scratch[kStaticWords];

namespace {

struct StaticScratch {
    unsigned long long* base = nullptr;  // this device's copy of `scratch`
    uint32_t tag_base = 1;               // tag of the next call's first tile
    unsigned long long* slots() const { return base; }
    uint32_t* fault() const { return reinterpret_cast<uint32_t*>(base + kStaticSlots); }
    float* split() const { return reinterpret_cast<float*>(base + kStaticSlots + kStaticFaultWords); }
};
std::map<int, StaticScratch> g_static;
// test hook (QKN_OPT_STATIC_SLOTS): slots of the static array a call may use, 0 = all
size_t g_static_slot_limit = 0;

std::map<int, StaticScratch> g_graph;  // per device: graph_scratch (tag_base unused)

int graph_scratch_for(int dev, StaticScratch** out)
{
    StaticScratch& s = g_graph[dev];
    if (!s.base) {
        void* p = nullptr;
        QKN_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(graph_scratch)));
        if (!p) return QKN_EHIP;
        s.base = static_cast<unsigned long long*>(p);
    }
    *out = &s;
    return QKN_OK;
}

int fill_words(unsigned long long* p, size_t n, hipStream_t stream)
{
    const unsigned blocks = (unsigned)std::max<size_t>(1, std::min<size_t>((n + 255) / 256, 2048));
    hipLaunchKernelGGL(qkn::fill_u64_kernel, dim3(blocks), dim3(256), 0, stream, p, (int64_t)n, 0ull);
    QKN_HIP(hipGetLastError());
    return QKN_OK;
}

// Binds the current device's copy of the array on its first use: the address
// from hipGetSymbolAddress (with that device current), every word cleared by a
// kernel on `stream`, and that stream synchronised once, so that a first call
// on another stream of the device also starts from cleared slots. Slot tags
// then start at 1, above the cleared words' 0.
int static_scratch_for(int dev, hipStream_t stream, StaticScratch** out)
{
    StaticScratch& s = g_static[dev];
    if (!s.base) {
        void* p = nullptr;
        QKN_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (!p) return QKN_EHIP;
        int rc = fill_words(static_cast<unsigned long long*>(p), kStaticWords, stream);
        if (rc) return rc;
        s.base = static_cast<unsigned long long*>(p);
        if ((rc = bind_fault_flag(dev, s.fault(), stream))) {
            s.base = nullptr;
            return rc;
        }
        QKN_HIP(hipStreamSynchronize(stream));
        s.tag_base = 1;
    }
    *out = &s;
    return QKN_OK;
}

// ---------------------------------------------------------------- validation

struct Range {
    uintptr_t lo, hi;
};
Range range_of(const void* p, int64_t bytes)
{
    uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return {a, a + (uintptr_t)bytes};
}
bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }
bool same(Range a, Range b) { return a.lo == b.lo && a.hi == b.hi; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int check_dims(int64_t T, int64_t H, int n_shards)
{
    if (T < 0 || H < 1 || H > (int64_t(1) << 28)) return QKN_EINVAL;
    if (n_shards < 1 || n_shards > QKN_MAX_SHARDS) return QKN_EINVAL;
    if (H % n_shards != 0) return QKN_EINVAL;
    return QKN_OK;
}
bool eps_ok(float eps) { return std::isfinite(eps) && eps >= 0.f; }


int current_device(int* dev)
{
    QKN_HIP(hipGetDevice(dev));
    return QKN_OK;
}

// ---------------------------------------------------------------- planning

// bpc[v * (QKN_MAX_DATA_WAVES + 1) + w]: co-resident workgroups per CU of
// variant v with w data waves (0 = not launchable).
// bpc: occupancy of the mixed-tile kernels; bpc_st: of the single-tensor-tile
// kernels (same layout), or null for none.
int plan(int dtype, int64_t T, int64_t Hq, int64_t Hk, int N, int cu, const int* bpc,
         const int* bpc_st, int aligned, qknorm_plan* out)
{
    std::memset(out, 0, sizeof *out);
    out->variant = -1;
    if (!fmt_valid(dtype)) return QKN_EINVAL;
    int rc = check_dims(T, Hq, N);
    if (rc) return rc;
    rc = check_dims(T, Hk, N);
    if (rc) return rc;
    if (cu < 1 || !bpc) return QKN_EINVAL;
    if (T == 0) return QKN_OK;
    const int ev = fmt_of(dtype).ev;
    const int64_t Wq = Hq / N, Wk = Hk / N;
    if (!aligned || Wq % ev || Wk % ev || g_opt.force_split) return QKN_OK;  // split kernels
    const int64_t wvq = Wq / ev, wvk = Wk / ev;
    // Tile layouts. Mixed: a tile is r tokens of Q and of K, Q's part padded to
    // whole waves, then K's. Single-tensor (RMSNorm in bf16 or fp32 with
    // Hq == Hk): a tile is r rows of one tensor, Q's tiles first, so there are
    // twice as many tiles and a tile's segments are its rows.
    const bool st_ok = Hq == Hk && bpc_st != nullptr && g_opt.tile_layout != 1;
    auto tile_vectors = [&](int64_t r, bool st) {
        return st ? r * wvq : ((r * wvq + 63) / 64) * 64 + r * wvk;
    };
    auto tiles_of = [&](int64_t r, bool st) { return (st ? 2 : 1) * ((T + r - 1) / r); };

    // Candidates (variant, data waves, rows, workgroups per CU). The tile must
    // fit the data threads' slots, and segments x statistics x N comm lanes
    // must fit one wave. Each candidate is scored by how far it lies, on a log
    // scale, from about 32 KB of tile loads plus stores in flight per CU and
    // about 8 waves per CU, with preferences for more rows per tile, fuller
    // slots and more vectors per thread, and against a one-tile lag when there
    // are peers to wait for. These general constants were fitted to the
    // timings of every candidate launch of 29 shapes of all four formats on
    // MI355X (mean 4.6 % from the best launch of each shape); streaming
    // batches split one or two ways use the refitted constants below.
    struct Best {
        int v = -1, w = 0, rows = 0, wpc = 0;
        bool st = false;
        double score = 0;
        int64_t wgs = 0;
    } best;
    // A two-tile lag only helps when there are peers to wait for.
    auto allowed = [&](int v) {
        const Variant& k = kVariants[v];
        if (!variant_usable(dtype, v)) return false;
        if (g_opt.force_variant >= 0) return v == g_opt.force_variant;
        if (v == 10) return false;
        return N > 1 || k.lag == 1;
    };
    const Fmt fm = fmt_of(dtype);
    // comm lanes: stats x segments x N slots in one wave (segments: 2 per token
    // for mixed tiles, 1 per row for single-tensor tiles)
    const int rows_cap = (int)std::min<int64_t>({(int64_t)qkn::kMaxRows, 32 / (N * fm.stats), T});
    const int rows_cap_st = (int)std::min<int64_t>({(int64_t)qkn::kMaxSeg, 64 / (N * fm.stats), T});
    const double batch = (double)T * (double)(wvq + wvk) * 16.0 * N;  // bytes read per call
    const double io = 1.0 + (double)fm.out / (double)fm.in;           // (loads + stores) / loads
    constexpr double kTarget = 32.0 * 1024;
    // A batch whose loads are smaller than the in-flight target is latency-bound:
    // a call takes one pass of a tile through a workgroup, so fewer vectors per
    // thread (the tile spread over more waves) shorten it, where in streaming
    // batches more vectors per thread help.
    const bool latency_bound = batch / cu < kTarget;
    // Streaming batches split one or two ways in bf16 or fp32 (RMSNorm and
    // LayerNorm) use constants refitted on the current kernels. For RMSNorm,
    // 22 such shapes (widths 1024-16384, 4096-65536 tokens, every candidate
    // timed with rotating buffer sets) put the rule's pick 4.5 % (at worst
    // 18 %) from each shape's best launch with the general constants, 1.4 %
    // (at worst 4.9 %) with a 40 KB in-flight target, 16 waves per CU and a
    // larger bonus per row. On shapes outside the fit they were faster for
    // RMSNorm (2.2 % in geomean) and for LayerNorm (up to 14 %).
    const bool refit = !latency_bound && N <= 2 &&
                       (dtype == QKN_FMT_BF16 || dtype == QKN_FMT_F32 || dtype == QKN_FMT_LN_BF16 ||
                        dtype == QKN_FMT_LN_F32);
    const double target = refit ? 40.0 * 1024 : kTarget;
    const double wave_target = refit ? 16.0 : 8.0;
    const double row_bonus = refit ? 0.4 : 0.2;
    auto consider = [&](int v, int w, int r, int wpc, bool st) {
        const Variant& k = kVariants[v];
        if (st && (!st_ok || r > rows_cap_st || !fused_fn_layout(dtype, v, true))) return;
        if (!st && !fused_fn_layout(dtype, v, false)) return;  // (variant 10: single-tensor tiles only)
        const int64_t tv = tile_vectors(r, st);
        if (w < 1 || w > max_data_waves(dtype, v) || (int64_t)64 * w * k.vpt < tv) return;
        const int b = (st ? bpc_st : bpc)[v * (QKN_MAX_DATA_WAVES + 1) + w];
        if (b <= 0 || wpc > b || (int64_t)b * cu < N) return;
        const int64_t tiles = tiles_of(r, st);
        const int64_t groups = std::min<int64_t>(tiles, (int64_t)wpc * cu / N);
        if (groups < 1) return;
        const int64_t wgs = groups * N;
        const double inflight = io * std::min((double)wgs * (double)(tv * 16), batch) / cu;
        const double waves = (double)wgs / cu * (w + 1);
        const double util = (double)tv / (double)(64 * w * k.vpt);
        double sc = std::fabs(std::log2(std::max(inflight, 1.0) / target)) +
                    0.5 * std::fabs(std::log2(std::max(waves, 0.1) / wave_target)) - row_bonus * r -
                    1.0 * util + (latency_bound ? 0.6 : -0.2) * std::log2((double)k.vpt);
        if (N > 1 && k.lag == 1) sc += 0.5;
        // latency-bound: every token also gets its own workgroup group if the
        // device can hold them
        if (latency_bound) sc += std::log2((double)(T * N) / (double)wgs);
        if (best.v < 0 || sc < best.score) {
            best.v = v;
            best.w = w;
            best.rows = r;
            best.wpc = wpc;
            best.st = st;
            best.score = sc;
            best.wgs = wgs;
        }
    };
    // Launches measured fastest on MI355X (every candidate timed with rotating
    // buffer sets) for the prefill-sized Q/K shards of the letter's models
    // (width 5120 split 1, 2, 4 or 8 ways; 5120/1024 split 4 ways), for bf16
    // and E4M3 activations and for LayerNorm, used for batches
    // of at least 4096 tokens when nothing is forced and the device can hold
    // them; the first fitting entry of a shape is taken. `xcd` 0: the launch
    // measured fastest with a group's members on different XCDs (narrow shards
    // and wide splits, where one slow XCD would otherwise hold back every group
    // placed on it); 1: members on one XCD.
    struct Tuned {
        int dtype, wq, wk, n, v, w, rows, wpc, st;
        int xcd = 1;
        int pace = 0;  // pacing rate in GB/s measured faster than none (0: none)
    };
    static const Tuned kTuned[] = {
        // single-tensor tiles first where they measured faster; the mixed-tile
        // entries after them serve when QKN_OPT_TILE_LAYOUT asks for mixed tiles
        {QKN_FMT_BF16, 5120, 5120, 1, 10, 4, 2, 1, 1, 1, 7100},
        {QKN_FMT_BF16, 5120, 5120, 1, 9, 5, 2, 1, 1},
        {QKN_FMT_BF16, 2560, 2560, 2, 10, 4, 4, 1, 1, 1, 7100},
        {QKN_FMT_BF16, 2560, 2560, 2, 9, 5, 4, 1, 1},
        {QKN_FMT_BF16, 1280, 1280, 4, 7, 11, 8, 1, 1, 0},
        {QKN_FMT_BF16, 640, 640, 8, 6, 8, 3, 3, 0, 0},
        {QKN_FMT_BF16, 640, 640, 8, 9, 3, 8, 2, 1},
        {QKN_FMT_BF16, 5120, 5120, 1, 3, 5, 1, 1, 0},
        {QKN_FMT_BF16, 2560, 2560, 2, 9, 5, 2, 1, 0},
        {QKN_FMT_BF16, 1280, 1280, 4, 9, 5, 4, 1, 0},
        {QKN_FMT_BF16, 640, 640, 8, 9, 3, 4, 2, 0},
        {QKN_FMT_BF16, 1280, 256, 4, 8, 2, 2, 4, 0, 0, 6700},
        {QKN_FMT_E4M3_BF16, 5120, 5120, 1, 0, 15, 3, 1, 1, 1, 6600},
        {QKN_FMT_E4M3_BF16, 1280, 1280, 4, 7, 3, 2, 3, 0, 0, 6600},
        {QKN_FMT_E4M3_BF16, 1280, 1280, 4, 7, 5, 8, 1, 1},
        {QKN_FMT_E4M3_BF16, 5120, 5120, 1, 2, 7, 2, 1, 0},
        {QKN_FMT_E4M3_BF16, 2560, 2560, 2, 7, 10, 8, 1, 1, 1, 6800},
        {QKN_FMT_E4M3_BF16, 2560, 2560, 2, 1, 10, 4, 1, 0, 0},
        {QKN_FMT_E4M3_BF16, 2560, 2560, 2, 7, 8, 3, 1, 0},
        {QKN_FMT_E4M3_BF16, 1280, 1280, 4, 6, 8, 3, 1, 0},
        {QKN_FMT_E4M3_BF16, 640, 640, 8, 7, 2, 3, 4, 0, 0, 6600},
        {QKN_FMT_E4M3_BF16, 1280, 256, 4, 7, 3, 4, 3, 0, 0},
        {QKN_FMT_E4M3_E4M3, 5120, 5120, 1, 6, 15, 3, 1, 1},
        {QKN_FMT_E4M3_E4M3, 2560, 2560, 2, 7, 10, 8, 1, 1, 1, 6600},
        {QKN_FMT_E4M3_E4M3, 5120, 5120, 1, 1, 15, 3, 1, 0},
        {QKN_FMT_E4M3_E4M3, 2560, 2560, 2, 7, 10, 4, 1, 0},
        {QKN_FMT_E4M3_E4M3, 1280, 1280, 4, 7, 3, 2, 3, 0},
        {QKN_FMT_E4M3_E4M3, 640, 640, 8, 7, 2, 3, 4, 0, 0},
        {QKN_FMT_E4M3_E4M3, 1280, 256, 4, 7, 3, 4, 3, 0},
        {QKN_FMT_LN_BF16, 5120, 5120, 1, 1, 10, 1, 1, 0},
        {QKN_FMT_LN_BF16, 2560, 2560, 2, 7, 10, 4, 1, 1, 1, 6900},
        {QKN_FMT_LN_BF16, 2560, 2560, 2, 7, 10, 2, 1, 0, 1, 6700},
        {QKN_FMT_LN_BF16, 1280, 1280, 4, 7, 10, 4, 1, 0},
        {QKN_FMT_LN_BF16, 640, 640, 8, 6, 5, 4, 4, 1, 0},
        {QKN_FMT_LN_BF16, 640, 640, 8, 7, 3, 2, 4, 0},
        {QKN_FMT_LN_BF16, 1280, 256, 4, 6, 12, 4, 2, 0, 0},
        {QKN_FMT_LN_F32, 2560, 2560, 2, 9, 5, 1, 2, 0},
    };
    const bool forced = g_opt.force_variant >= 0 || g_opt.rows > 0 || g_opt.force_data_waves > 0 || g_opt.wpc > 0 ||
                        g_opt.tile_layout == 2;
    bool tuned = false;
    bool tuned_xcd = true;
    int tuned_pace = 0;
    if (!forced && T >= 4096) {
        for (const Tuned& t : kTuned) {
            if (t.dtype == dtype && t.wq == Wq && t.wk == Wk && t.n == N &&
                t.rows <= (t.st ? rows_cap_st : rows_cap))
                consider(t.v, t.w, t.rows, t.wpc, t.st != 0);
            if (best.v >= 0) {  // the first entry that fits the device
                tuned = true;
                tuned_xcd = t.xcd != 0;
                tuned_pace = t.pace;
                break;
            }
        }
    }
    // the search below uses mixed tiles, or single-tensor tiles where
    // QKN_OPT_TILE_LAYOUT asks for them and the shape allows them
    const bool st_search = g_opt.tile_layout == 2 && st_ok;
    // E4M3 -> E4M3 over narrow shards (at most 160 vectors of Q and K per
    // token): every best launch timed (widths 2048-5120 over 2-8 shards, GQA)
    // ran three or four workgroups per CU, so the search starts there and
    // widens only if nothing fits.
    const bool narrow_e4 = dtype == QKN_FMT_E4M3_E4M3 && !forced && !latency_bound && N >= 2 && wvq + wvk <= 160;
    for (int pass = narrow_e4 ? 0 : 1; pass < 2 && best.v < 0; ++pass) {
        for (int v = 0; v < QKN_NUM_VARIANTS; ++v) {
            if (!allowed(v)) continue;
            const Variant& k = kVariants[v];
            if (st_search && !fused_fn_layout(dtype, v, true)) continue;
            for (int r = 1; r <= (st_search ? rows_cap_st : rows_cap); ++r) {
                if (g_opt.rows > 0 && r != g_opt.rows) continue;
                const int64_t tv = tile_vectors(r, st_search);
                int w = (int)((tv + 64 * k.vpt - 1) / (64 * k.vpt));
                if (g_opt.force_data_waves > 0) {
                    if (g_opt.force_data_waves < w) continue;
                    w = (int)g_opt.force_data_waves;
                }
                if (w < 1 || w > max_data_waves(dtype, v)) continue;
                const int b = (st_search ? bpc_st : bpc)[v * (QKN_MAX_DATA_WAVES + 1) + w];
                const int64_t tiles = tiles_of(r, st_search);
                for (int wpc = 1; wpc <= b; ++wpc) {
                    if (g_opt.wpc > 0 && wpc != g_opt.wpc) continue;
                    if (pass == 0 && wpc < 3) continue;
                    consider(v, w, r, wpc, st_search);
                    if ((int64_t)wpc * cu / N >= tiles) break;  // more would idle
                }
            }
        }
    }
    // Streaming RMSNorm shards split four or more ways ran faster on
    // single-tensor tiles in a sweep of 20 such shapes (bf16 and fp32, widths
    // 1024-16384 over N = 4 and 8, 16384 tokens): 18 faster, by up to 20 %,
    // with the scored mixed launch moved over unchanged but for twice the rows
    // per tile (the same bytes per tile, less Q's padding). With N = 1 or 2
    // the two layouts were within noise of each other, so mixed tiles stay;
    // wider splits were not measured.
    if (best.v >= 0 && !best.st && !tuned && !forced && g_opt.tile_layout == 0 && st_ok &&
        !latency_bound && N >= 4 && N <= 8 && (dtype == QKN_FMT_BF16 || dtype == QKN_FMT_F32) &&
        2 * best.rows <= rows_cap_st) {
        const Best mixed = best;
        best.v = -1;
        consider(mixed.v, mixed.w, 2 * mixed.rows, mixed.wpc, true);
        if (best.v < 0) best = mixed;
    }
    if (best.v < 0) {
        // nothing fits: residency failure if some variant would fit the shape
        // but not N co-resident workgroups; otherwise the split kernels
        for (int v = 0; v < QKN_NUM_VARIANTS; ++v) {
            const Variant& k = kVariants[v];
            if (!variant_usable(dtype, v)) continue;
            const int w = (int)((tile_vectors(1, false) + 64 * k.vpt - 1) / (64 * k.vpt));
            if (w >= 1 && w <= max_data_waves(dtype, v) && bpc[v * (QKN_MAX_DATA_WAVES + 1) + w] > 0 &&
                (int64_t)bpc[v * (QKN_MAX_DATA_WAVES + 1) + w] * cu < N)
                return QKN_ERESIDENCY;
        }
        return QKN_OK;
    }
    const int rows = best.rows;
    const int64_t n_tiles = tiles_of(rows, best.st);
    int64_t groups = best.wgs / N;
    if (g_opt.max_groups > 0) groups = std::min<int64_t>(groups, g_opt.max_groups);
    // a group's members share one XCD unless turned off (the option, the tuned
    // launch's measurement, or the rule below). Untuned streaming RMSNorm
    // shapes were timed with members on one XCD and spread (bf16 and fp32,
    // widths 1024-16384, 4096-65536 tokens, 2-8 shards): spread was faster on
    // 31 of 32 fp32 shapes split four or eight ways (by up to 14 %; 3 % slower on
    // the other), and never slower on the 12 bf16 shapes split four ways with
    // shard rows of at least 1 KiB (up to 10.5 % faster). Narrower bf16 shards
    // split four ways, bf16 split eight ways and splits of two gained or lost a
    // few percent from shape to shape (eight ways on one workgroup per CU: 2-5 %
    // slower spread), and LayerNorm and E4M3 likewise, so they keep one XCD.
    bool spread = !tuned_xcd;
    if (!tuned && !forced && !latency_bound && g_opt.xcd_map == -1)
        spread = (dtype == QKN_FMT_F32 && N >= 4 && N <= 8) ||
                 (dtype == QKN_FMT_BF16 && N == 4 && std::min(wvq, wvk) * 16 >= 1024);
    const bool want_xcd = g_opt.xcd_map == 1 || (g_opt.xcd_map == -1 && !spread);
    int xcd = 0;
    if (want_xcd && groups >= 8) {
        if (groups < n_tiles) groups -= groups % 8;  // capped: round to whole XCD sets
        xcd = (groups % 8 == 0) ? 1 : 0;
    }
    if (groups < 1) groups = 1;
    out->variant = best.v;
    out->threads = 64 * (best.w + 1);
    out->data_waves = best.w;
    out->slots = kVariants[best.v].vpt;
    out->rows = rows;
    out->n_tiles = n_tiles;
    out->n_groups = (int)groups;
    out->grid = (int)(groups * N);
    out->xcd_map = xcd;
    out->iters = (int)((n_tiles + groups - 1) / groups);
    out->st = best.st ? 1 : 0;
    // pacing: the tuned launch's measured rate unless the option sets one (0: off),
    // for kernels with a paced build
    out->pace_gbs = !paced_fn(dtype, best.v, best.st) ? 0
                    : g_opt.pace_gbs >= 0           ? (int)g_opt.pace_gbs
                    : tuned                         ? tuned_pace
                                                    : 0;
    return QKN_OK;
}

// Pacing period of a fused launch in 1/256 wall-clock ticks per iteration: the
// time the whole grid's bytes of one iteration (one tile's loads and stores per
// workgroup) take at the plan's pacing rate; 0 when the plan has none or runs
// two iterations or fewer.
uint32_t pace_period(const qknorm_plan& pl, int wv_q, int wv_k, const Fmt& f, int wall_khz)
{
    if (pl.pace_gbs <= 0 || pl.iters <= 2) return 0;
    const double tile_in = (double)pl.rows * (pl.st ? (double)wv_q : (double)(wv_q + wv_k)) * 16.0;
    const double per_iter = (double)pl.grid * tile_in * (1.0 + (double)f.out / (double)f.in);
    const double ticks = per_iter / ((double)pl.pace_gbs * 1e9) * (double)wall_khz * 1e3;
    return (uint32_t)std::min(ticks * 256.0, 4.0e9);
}

// ---------------------------------------------------------------- split launches

// 16-byte loads each lane of a split reduction issues at once: enough to cover
// a shard row of `row_bytes` in one pass (a wave loads 1 KiB per vector), at
// most 8; QKN_OPT_SPLIT_VECTORS overrides.
int reduce_vectors(int64_t row_bytes)
{
    if (g_opt.split_vectors > 0) return (int)g_opt.split_vectors;
    const int64_t need = (row_bytes + 1023) / 1024;
    return need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : 8;
}

template <class DT, bool STATS>
void launch_reduce_vec(int u, dim3 g, hipStream_t s, const void* x, int64_t T, int H, int N,
                       float* sums, float* sumsq)
{
    switch (u) {
    case 1: hipLaunchKernelGGL((qkn::shard_reduce_vec_kernel<DT, 1, STATS>), g, dim3(256), 0, s, x, T, H, N, sums, sumsq); break;
    case 2: hipLaunchKernelGGL((qkn::shard_reduce_vec_kernel<DT, 2, STATS>), g, dim3(256), 0, s, x, T, H, N, sums, sumsq); break;
    case 4: hipLaunchKernelGGL((qkn::shard_reduce_vec_kernel<DT, 4, STATS>), g, dim3(256), 0, s, x, T, H, N, sums, sumsq); break;
    default: hipLaunchKernelGGL((qkn::shard_reduce_vec_kernel<DT, 8, STATS>), g, dim3(256), 0, s, x, T, H, N, sums, sumsq); break;
    }
}

template <class DT>
void launch_sumsq_as(bool vec, dim3 g, dim3 b, hipStream_t s, const void* x, int64_t T, int H, int N,
                     float* partials)
{
    if (vec) launch_reduce_vec<DT, false>(reduce_vectors((int64_t)(H / N) * sizeof(typename DT::in_t)), g,
                                          s, x, T, H, N, nullptr, partials);
    else hipLaunchKernelGGL((qkn::shard_sumsq_kernel<DT>), g, b, 0, s, x, T, H, N, partials);
}

// fmt: any format whose input is x's format (only the input format matters)
int launch_sumsq(int fmt, const void* x, int64_t T, int64_t H, int N, float* partials,
                 hipStream_t s)
{
    const int64_t items = T * N;
    const int64_t blocks = (items + 3) / 4;
    if (blocks > 0x7fffffff) return QKN_EINVAL;
    const int W = (int)(H / N);
    const bool vec = aligned16(x) && ((int64_t)W * fmt_of(fmt).in) % 16 == 0;
    dim3 g((unsigned)blocks), b(256);
    switch (fmt) {
    case QKN_FMT_BF16: launch_sumsq_as<Bf16>(vec, g, b, s, x, T, (int)H, N, partials); break;
    case QKN_FMT_F32: launch_sumsq_as<F32>(vec, g, b, s, x, T, (int)H, N, partials); break;
    default: launch_sumsq_as<E4m3Bf16>(vec, g, b, s, x, T, (int)H, N, partials); break;
    }
    QKN_HIP(hipGetLastError());
    return QKN_OK;
}

int launch_combine(const float* partials, int64_t T, int64_t H, int N, float eps, float* rinv,
                   hipStream_t s)
{
    const int64_t blocks = (T + 255) / 256;
    if (blocks > 0x7fffffff) return QKN_EINVAL;
    hipLaunchKernelGGL(qkn::combine_scale_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       partials, T, (int)H, N, eps, rinv);
    QKN_HIP(hipGetLastError());
    return QKN_OK;
}

// 16-byte input vectors per thread of the one-pass apply kernels.
int apply_vectors() { return g_opt.split_vectors > 0 ? (int)std::min<int64_t>(g_opt.split_vectors, 4) : 2; }

// The one-pass apply kernels over T rows of `per_row` input vectors; LN
// selects the LayerNorm form (s0 = mean, s1 = rstd), else s0 = rms_inv.
template <class DT, bool LN>
int launch_apply_vec(hipStream_t s, const void* x, const void* g, const void* bt, const float* s0,
                     const float* s1, int64_t T, int64_t per_row, void* y)
{
    const int u = apply_vectors();
    const int64_t nvec = T * per_row;
    const int64_t blocks = (nvec + 256 * u - 1) / (256 * u);
    if (blocks > 0x7fffffff) return QKN_EINVAL;
    const dim3 gr((unsigned)blocks), b(256);
    const double inv = 1.0 / (double)per_row;
    switch (u) {
    case 1: hipLaunchKernelGGL((qkn::apply_vec_kernel<DT, 1, LN>), gr, b, 0, s, x, g, bt, s0, s1, nvec, (int)per_row, inv, y); break;
    case 2: hipLaunchKernelGGL((qkn::apply_vec_kernel<DT, 2, LN>), gr, b, 0, s, x, g, bt, s0, s1, nvec, (int)per_row, inv, y); break;
    default: hipLaunchKernelGGL((qkn::apply_vec_kernel<DT, 4, LN>), gr, b, 0, s, x, g, bt, s0, s1, nvec, (int)per_row, inv, y); break;
    }
    QKN_HIP(hipGetLastError());
    return QKN_OK;
}

template <class DT>
void launch_apply_as(dim3 gr, dim3 b, hipStream_t s, const void* x, const void* g,
                     const float* rinv, int64_t T, int H, int rpb, void* y)
{
    hipLaunchKernelGGL((qkn::apply_scale_kernel<DT>), gr, b, 0, s, x, g, rinv, T, H, rpb, y);
}

int launch_apply(int fmt, const void* x, const void* g, const float* rinv, int64_t T, int64_t H,
                 void* y, hipStream_t s)
{
    const Fmt f = fmt_of(fmt);
    // 16-byte paths need every row of x to be whole vectors (then gamma's and
    // y's rows are whole 16-byte words too: their elements are at least as wide)
    const bool vec = aligned16(x) && aligned16(g) && aligned16(y) && (H * f.in) % 16 == 0;
    if (vec) {
        const int64_t pr = H * f.in / 16;
        switch (fmt) {
        case QKN_FMT_BF16: return launch_apply_vec<Bf16, false>(s, x, g, nullptr, rinv, nullptr, T, pr, y);
        case QKN_FMT_F32: return launch_apply_vec<F32, false>(s, x, g, nullptr, rinv, nullptr, T, pr, y);
        case QKN_FMT_E4M3_BF16: return launch_apply_vec<E4m3Bf16, false>(s, x, g, nullptr, rinv, nullptr, T, pr, y);
        default: return launch_apply_vec<E4m3E4m3, false>(s, x, g, nullptr, rinv, nullptr, T, pr, y);
        }
    }
    const int64_t per_row = H;
    const int rpb = (int)std::max<int64_t>(1, std::min<int64_t>(64, 2048 / per_row));
    const int64_t blocks = (T + rpb - 1) / rpb;
    if (blocks > 0x7fffffff) return QKN_EINVAL;
    dim3 gr((unsigned)blocks), b(256);
    switch (fmt) {
    case QKN_FMT_BF16: launch_apply_as<Bf16>(gr, b, s, x, g, rinv, T, (int)H, rpb, y); break;
    case QKN_FMT_F32: launch_apply_as<F32>(gr, b, s, x, g, rinv, T, (int)H, rpb, y); break;
    case QKN_FMT_E4M3_BF16: launch_apply_as<E4m3Bf16>(gr, b, s, x, g, rinv, T, (int)H, rpb, y); break;
    default: launch_apply_as<E4m3E4m3>(gr, b, s, x, g, rinv, T, (int)H, rpb, y); break;
    }
    QKN_HIP(hipGetLastError());
    return QKN_OK;
}

template <class DT>
void launch_stats_as(bool vec, dim3 g, dim3 b, hipStream_t s, const void* x, int64_t T, int H,
                     int N, float* sums, float* sumsq)
{
    if (vec) launch_reduce_vec<DT, true>(reduce_vectors((int64_t)(H / N) * sizeof(typename DT::in_t)), g, s,
                                         x, T, H, N, sums, sumsq);
    else hipLaunchKernelGGL((qkn::shard_stats_kernel<DT>), g, b, 0, s, x, T, H, N, sums, sumsq);
}

int launch_stats(int fmt, const void* x, int64_t T, int64_t H, int N, float* sums, float* sumsq,
                 hipStream_t s)
{
    const int64_t blocks = (T * N + 3) / 4;
    if (blocks > 0x7fffffff) return QKN_EINVAL;
    const int W = (int)(H / N);
    const bool vec = aligned16(x) && ((int64_t)W * fmt_of(fmt).in) % 16 == 0;
    dim3 g((unsigned)blocks), b(256);
    if (fmt_of(fmt).in == 2) launch_stats_as<Bf16>(vec, g, b, s, x, T, (int)H, N, sums, sumsq);
    else launch_stats_as<F32>(vec, g, b, s, x, T, (int)H, N, sums, sumsq);
    QKN_HIP(hipGetLastError());
    return QKN_OK;
}

int launch_combine_stats(const float* sums, const float* sumsq, int64_t T, int64_t H, int N,
                         float eps, float* mean, float* rstd, hipStream_t s)
{
    const int64_t blocks = (T + 255) / 256;
    if (blocks > 0x7fffffff) return QKN_EINVAL;
    hipLaunchKernelGGL(qkn::combine_stats_kernel, dim3((unsigned)blocks), dim3(256), 0, s, sums,
                       sumsq, T, (int)H, N, eps, mean, rstd);
    QKN_HIP(hipGetLastError());
    return QKN_OK;
}

template <class DT>
void launch_norm_as(dim3 gr, dim3 b, hipStream_t s, const void* x, const void* g, const void* bt,
                    const float* mean, const float* rstd, int64_t T, int H, int rpb, void* y)
{
    hipLaunchKernelGGL((qkn::apply_norm_kernel<DT>), gr, b, 0, s, x, g, bt, mean, rstd, T, H, rpb, y);
}

int launch_apply_norm(int fmt, const void* x, const void* g, const void* bt, const float* mean,
                      const float* rstd, int64_t T, int64_t H, void* y, hipStream_t s)
{
    const Fmt f = fmt_of(fmt);
    const bool vec = aligned16(x) && aligned16(g) && (!bt || aligned16(bt)) && aligned16(y) &&
                     (H * f.in) % 16 == 0;
    if (vec) {
        const int64_t pr = H * f.in / 16;
        if (f.in == 2) return launch_apply_vec<Bf16, true>(s, x, g, bt, mean, rstd, T, pr, y);
        return launch_apply_vec<F32, true>(s, x, g, bt, mean, rstd, T, pr, y);
    }
    const int64_t per_row = H;
    const int rpb = (int)std::max<int64_t>(1, std::min<int64_t>(64, 2048 / per_row));
    const int64_t blocks = (T + rpb - 1) / rpb;
    if (blocks > 0x7fffffff) return QKN_EINVAL;
    dim3 gr((unsigned)blocks), b(256);
    if (f.in == 2) launch_norm_as<Bf16>(gr, b, s, x, g, bt, mean, rstd, T, (int)H, rpb, y);
    else launch_norm_as<F32>(gr, b, s, x, g, bt, mean, rstd, T, (int)H, rpb, y);
    QKN_HIP(hipGetLastError());
    return QKN_OK;
}

// ---------------------------------------------------------------- headwise

template <class DT>
void launch_headwise_as(int vh, dim3 g, hipStream_t s, const qkn::HeadwiseParams& p)
{
    switch (vh) {
    case 1: hipLaunchKernelGGL((qkn::headwise_kernel<DT, 1>), g, dim3(qkn::kHeadwiseThreads), 0, s, p); break;
    case 2: hipLaunchKernelGGL((qkn::headwise_kernel<DT, 2>), g, dim3(qkn::kHeadwiseThreads), 0, s, p); break;
    case 4: hipLaunchKernelGGL((qkn::headwise_kernel<DT, 4>), g, dim3(qkn::kHeadwiseThreads), 0, s, p); break;
    case 8: hipLaunchKernelGGL((qkn::headwise_kernel<DT, 8>), g, dim3(qkn::kHeadwiseThreads), 0, s, p); break;
    case 16: hipLaunchKernelGGL((qkn::headwise_kernel<DT, 16>), g, dim3(qkn::kHeadwiseThreads), 0, s, p); break;
    case 32: hipLaunchKernelGGL((qkn::headwise_kernel<DT, 32>), g, dim3(qkn::kHeadwiseThreads), 0, s, p); break;
    default: hipLaunchKernelGGL((qkn::headwise_kernel<DT, 64>), g, dim3(qkn::kHeadwiseThreads), 0, s, p); break;
    }
}

int headwise_fwd(int fmt, const void* q, const void* k, const void* gq, const void* gk, int64_t T,
                 int64_t hq, int64_t hk, int64_t D, float eps, void* oq, void* ok,
                 hipStream_t stream)
{
    t_hip_error.clear();
    if (T < 0 || hq < 1 || hk < 1 || D < 1 || hq * D > (int64_t(1) << 28) ||
        hk * D > (int64_t(1) << 28) || !eps_ok(eps))
        return QKN_EINVAL;
    if (T == 0) return QKN_OK;
    if (!q || !k || !gq || !gk || !oq || !ok) return QKN_EINVAL;
    const Fmt f = fmt_of(fmt);
    const int64_t Hq = hq * D, Hk = hk * D;
    const Range rq = range_of(q, T * Hq * f.in), rk = range_of(k, T * Hk * f.in);
    const Range rgq = range_of(gq, D * f.gam), rgk = range_of(gk, D * f.gam);
    const Range roq = range_of(oq, T * Hq * f.out), rok = range_of(ok, T * Hk * f.out);
    if (overlaps(roq, rok)) return QKN_EOVERLAP;
    if (overlaps(roq, rq) && !same(roq, rq)) return QKN_EOVERLAP;
    if (overlaps(rok, rk) && !same(rok, rk)) return QKN_EOVERLAP;
    if (overlaps(roq, rk) || overlaps(roq, rgq) || overlaps(roq, rgk)) return QKN_EOVERLAP;
    if (overlaps(rok, rq) || overlaps(rok, rgq) || overlaps(rok, rgk)) return QKN_EOVERLAP;
    qkn::HeadwiseParams p;
    std::memset(&p, 0, sizeof p);
    p.x[0] = q;
    p.x[1] = k;
    p.gamma[0] = gq;
    p.gamma[1] = gk;
    p.y[0] = oq;
    p.y[1] = ok;
    p.D = (int32_t)D;
    p.heads[0] = (int32_t)hq;
    p.heads[1] = (int32_t)hk;
    p.T = T;
    p.eps = eps;
    // 128-bit path: whole 16-byte vectors per head, a power of two of them (<= 64)
    const int64_t vh = D * f.in % 16 == 0 ? D * f.in / 16 : 0;
    const bool vec = vh >= 1 && vh <= 64 && (vh & (vh - 1)) == 0 && aligned16(q) && aligned16(k) &&
                     aligned16(gq) && aligned16(gk) && aligned16(oq) && aligned16(ok);
    if (vec) {
        p.nv[0] = T * Hq * f.in / 16;
        p.nv[1] = T * Hk * f.in / 16;
        constexpr int64_t W = qkn::kHeadwiseThreads;
        p.blocks_q = (p.nv[0] + W - 1) / W;
        const int64_t blocks = p.blocks_q + (p.nv[1] + W - 1) / W;
        if (blocks > 0x7fffffff) return QKN_EINVAL;
        if (f.in == 2) launch_headwise_as<Bf16>((int)vh, dim3((unsigned)blocks), stream, p);
        else launch_headwise_as<F32>((int)vh, dim3((unsigned)blocks), stream, p);
    } else {
        const int64_t blocks = (T * (hq + hk) + 3) / 4;
        if (blocks > 0x7fffffff) return QKN_EINVAL;
        if (f.in == 2) hipLaunchKernelGGL((qkn::headwise_scalar_kernel<Bf16>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((qkn::headwise_scalar_kernel<F32>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
    }
    QKN_HIP(hipGetLastError());
    return QKN_OK;
}

// ---------------------------------------------------------------- fused entry

// The fused entry point's split fallback (shapes the fused kernel does not
// take): the three split kernels per tensor, over token chunks whose fp32
// statistics fit the `floats` words at `buf` ((N+1) per token for RMSNorm,
// 2N+2 for LayerNorm). Rows are independent, so chunking changes no result.
int split_fallback(int dtype, const void* q, const void* k, const void* gq, const void* gk,
                   const void* bq, const void* bk, int64_t T, int64_t Hq, int64_t Hk, int N,
                   float eps, void* oq, void* ok, float* buf, size_t floats, hipStream_t stream)
{
    const Fmt f = fmt_of(dtype);
    const bool ln = is_layernorm(dtype);
    const size_t per_token = ln ? (size_t)(2 * N + 2) : (size_t)(N + 1);
    const int64_t chunk = std::min<int64_t>(T, (int64_t)(floats / per_token));
    if (chunk < 1) return QKN_ENOMEM;
    const void* xs[2] = {q, k};
    const void* gs[2] = {gq, gk};
    const void* bs[2] = {bq, bk};
    void* ys[2] = {oq, ok};
    const int64_t Hs[2] = {Hq, Hk};
    int rc = QKN_OK;
    for (int64_t t0 = 0; t0 < T; t0 += chunk) {
        const int64_t tc = std::min(chunk, T - t0);
        for (int i = 0; i < 2; ++i) {
            const void* x = static_cast<const char*>(xs[i]) + t0 * Hs[i] * f.in;
            void* y = static_cast<char*>(ys[i]) + t0 * Hs[i] * f.out;
            if (ln) {
                float* sums = buf;
                float* sumsq = sums + (size_t)N * tc;
                float* mean = sumsq + (size_t)N * tc;
                float* rstd = mean + tc;
                if ((rc = launch_stats(dtype, x, tc, Hs[i], N, sums, sumsq, stream))) return rc;
                if ((rc = launch_combine_stats(sums, sumsq, tc, Hs[i], N, eps, mean, rstd, stream))) return rc;
                if ((rc = launch_apply_norm(dtype, x, gs[i], bs[i], mean, rstd, tc, Hs[i], y, stream)))
                    return rc;
            } else {
                float* part = buf;
                float* rinv = buf + (size_t)N * tc;
                if ((rc = launch_sumsq(dtype, x, tc, Hs[i], N, part, stream))) return rc;
                if ((rc = launch_combine(part, tc, Hs[i], N, eps, rinv, stream))) return rc;
                if ((rc = launch_apply(dtype, x, gs[i], rinv, tc, Hs[i], y, stream))) return rc;
            }
        }
    }
    return QKN_OK;
}

// bq, bk: LayerNorm's beta (either may be null); null for the RMSNorm formats.
// noalloc: the scratch is this device's copy of the static array (no device
// memory is allocated), else the (device, stream) workspace.
int layerwise_fwd(int dtype, const void* q, const void* k, const void* gq, const void* gk,
                  const void* bq, const void* bk, int64_t T, int64_t Hq, int64_t Hk, int N,
                  float eps, void* oq, void* ok, hipStream_t stream, bool noalloc = false)
{
    t_hip_error.clear();
    int rc = check_dims(T, Hq, N);
    if (rc) return rc;
    if ((rc = check_dims(T, Hk, N))) return rc;
    if (!eps_ok(eps)) return QKN_EINVAL;
    if (T == 0) return QKN_OK;
    if (!q || !k || !gq || !gk || !oq || !ok) return QKN_EINVAL;
    const Fmt f = fmt_of(dtype);
    const Range rq = range_of(q, T * Hq * f.in), rk = range_of(k, T * Hk * f.in);
    const Range rgq = range_of(gq, Hq * f.gam), rgk = range_of(gk, Hk * f.gam);
    const Range roq = range_of(oq, T * Hq * f.out), rok = range_of(ok, T * Hk * f.out);
    if (overlaps(roq, rok)) return QKN_EOVERLAP;
    // in place needs the output to occupy exactly the input's bytes (same element size)
    if (overlaps(roq, rq) && !same(roq, rq)) return QKN_EOVERLAP;
    if (overlaps(rok, rk) && !same(rok, rk)) return QKN_EOVERLAP;
    if (overlaps(roq, rk) || overlaps(roq, rgq) || overlaps(roq, rgk)) return QKN_EOVERLAP;
    if (overlaps(rok, rq) || overlaps(rok, rgq) || overlaps(rok, rgk)) return QKN_EOVERLAP;
    if (bq || bk) {
        const Range rbq = range_of(bq, bq ? Hq * f.gam : 0), rbk = range_of(bk, bk ? Hk * f.gam : 0);
        if (overlaps(roq, rbq) || overlaps(roq, rbk) || overlaps(rok, rbq) || overlaps(rok, rbk))
            return QKN_EOVERLAP;
    }
    // The fused kernel addresses each tensor with 32-bit offsets into one buffer
    // descriptor: every tensor of a launch stays 64 KiB below 2^31 bytes, so
    // an unused lane's offset (2^31 + the tile's row offset + the store's word
    // offset) still fits in 32 bits. Longer batches run as consecutive launches
    // over token ranges (rows are independent, so the result is the same).
    // H <= 2^28 keeps tmax >= 1.
    const int64_t row_bytes = std::max(Hq, Hk) * std::max(f.in, f.out);
    const int64_t tmax = ((int64_t(1) << 31) - (int64_t(1) << 16)) / row_bytes;
    if (T > tmax) {
        for (int64_t t0 = 0; t0 < T; t0 += tmax) {
            const int64_t tc = std::min(tmax, T - t0);
            auto at = [&](const void* b, int64_t H, int e) {
                return static_cast<const void*>(static_cast<const char*>(b) + t0 * H * e);
            };
            rc = layerwise_fwd(dtype, at(q, Hq, f.in), at(k, Hk, f.in), gq, gk, bq, bk, tc, Hq, Hk,
                               N, eps, const_cast<void*>(at(oq, Hq, f.out)),
                               const_cast<void*>(at(ok, Hk, f.out)), stream, noalloc);
            if (rc) return rc;
        }
        return QKN_OK;
    }

    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    QKN_HIP(hipStreamIsCapturing(stream, &cap));
    // under capture: graph_scratch, a recorded clearing of the slots, tags from 1
    const bool captured = cap != hipStreamCaptureStatusNone;
    if (captured && g_opt.cooperative) return QKN_ECAPTURE;

    std::lock_guard<std::mutex> lock(g_mu);
    int dev = 0;
    if ((rc = current_device(&dev))) return rc;
    DevInfo* di = nullptr;
    if ((rc = device_info(dev, dtype, &di))) return rc;
    Workspace* ws = nullptr;
    StaticScratch* ss = nullptr;
    if (captured) {
        if ((rc = graph_scratch_for(dev, &ss))) return rc;
    } else if (noalloc) {
        if ((rc = static_scratch_for(dev, stream, &ss))) return rc;
    } else if ((rc = workspace_for(dev, stream, &ws))) {
        return rc;
    }
    const bool in_static = captured || noalloc;  // scratch in a static array

    const int aligned = aligned16(q) && aligned16(k) && aligned16(gq) && aligned16(gk) &&
                        aligned16(oq) && aligned16(ok) && (!bq || aligned16(bq)) &&
                        (!bk || aligned16(bk));
    static std::map<PlanKey, qknorm_plan> cache;
    const PlanKey key{dev, dtype, N, aligned, T, Hq, Hk, g_opt_epoch};
    qknorm_plan pl;
    auto hit = cache.find(key);
    if (hit != cache.end()) {
        pl = hit->second;
    } else {
        if ((rc = plan(dtype, T, Hq, Hk, N, di->cu, &di->occ[dtype][0][0], &di->occ_st[dtype][0][0], aligned,
                       &pl)))
            return rc;
        if (cache.size() > 4096) cache.clear();
        cache.emplace(key, pl);
    }

    if (pl.variant < 0) {
        // Shapes the fused kernel cannot hold in registers (or unaligned): the
        // same computation with the three split kernels, per tensor.
        if (in_static)
            return split_fallback(dtype, q, k, gq, gk, bq, bk, T, Hq, Hk, N, eps, oq, ok, ss->split(),
                                  kStaticSplitFloats, stream);
        const size_t need = (size_t)(is_layernorm(dtype) ? 2 * N + 2 : N + 1) * (size_t)T;
        if ((rc = ensure_scratch(ws, need, stream))) return rc;
        return split_fallback(dtype, q, k, gq, gk, bq, bk, T, Hq, Hk, N, eps, oq, ok, ws->scratch, need,
                              stream);
    }

    const size_t entries =
        (size_t)pl.n_groups * 2 * kVariants[pl.variant].lag * N * f.stats * 2 * pl.rows;
    unsigned long long* slots = nullptr;
    size_t slot_entries = 0;  // every slot the tags of this scratch have touched
    uint32_t* fault = nullptr;
    uint32_t* tag_base = nullptr;
    uint32_t graph_tag = 1;
    if (captured) {
        if (entries > kStaticSlots) return QKN_ESCRATCH;
        slots = ss->slots();
        fault = ss->fault();
        tag_base = &graph_tag;
        // recorded before the launch: every replay clears the slots it will use
        if ((rc = fill_words(slots, entries, stream))) return rc;
    } else if (noalloc) {
        const size_t usable = g_static_slot_limit ? std::min(g_static_slot_limit, kStaticSlots) : kStaticSlots;
        if (entries > usable) return QKN_ESCRATCH;
        slots = ss->slots();
        slot_entries = kStaticSlots;
        fault = ss->fault();
        tag_base = &ss->tag_base;
    } else {
        if ((rc = ensure_slots(ws, entries, stream))) return rc;
        slots = ws->slots;
        slot_entries = ws->slot_entries;
        fault = ws->fault;
        tag_base = &ws->tag_base;
    }
    if (!captured && (uint64_t)*tag_base + (uint64_t)pl.iters + 1 >= (uint64_t(1) << 32)) {
        // tags would wrap: clear every slot so no stale tag can match
        if ((rc = fill_words(slots, slot_entries, stream))) return rc;
        *tag_base = 1;
    }

    FusedParams p;
    std::memset(&p, 0, sizeof p);
    p.x[0] = q;
    p.x[1] = k;
    p.gamma[0] = gq;
    p.gamma[1] = gk;
    p.beta[0] = bq;
    p.beta[1] = bk;
    p.y[0] = oq;
    p.y[1] = ok;
    p.T = T;
    p.n_tiles = pl.n_tiles;
    p.H[0] = (int32_t)Hq;
    p.H[1] = (int32_t)Hk;
    p.Wv[0] = (int32_t)(Hq / N / f.ev);
    p.Wv[1] = (int32_t)(Hk / N / f.ev);
    p.rows = pl.rows;
    p.nwd = pl.data_waves;
    p.n_shards = N;
    p.n_groups = pl.n_groups;
    p.xcd_map = pl.xcd_map;
    p.eps = eps;
    p.tag_base = *tag_base;
    p.slots = slots;
    p.fault = fault;
    const double ticks = (double)g_opt.spin_ns * 1e-9 * (double)di->wall_khz * 1e3;
    p.spin_ticks = ticks < 1.0 ? 1 : (uint64_t)ticks;
    p.test_flags = g_opt.test_skip_publish ? 1u : 0u;
    p.nq = pl.st ? (T + pl.rows - 1) / pl.rows : 0;
    p.pace = pace_period(pl, p.Wv[0], p.Wv[1], f, di->wall_khz);
    *tag_base += (uint32_t)pl.iters;

    FusedFn fn = p.pace ? paced_fn(dtype, pl.variant, pl.st != 0) : fused_fn_layout(dtype, pl.variant, pl.st != 0);
    if (!fn) return QKN_EINVAL;
    const size_t lds = gamma_lds_bytes(dtype, pl.variant, pl.data_waves, pl.st != 0);
    if (g_opt.cooperative) {
        void* args[] = {&p};
        QKN_HIP(hipLaunchCooperativeKernel(reinterpret_cast<const void*>(fn), dim3(pl.grid),
                                           dim3(pl.threads), args, (unsigned)lds, stream));
    } else {
        hipLaunchKernelGGL(fn, dim3(pl.grid), dim3(pl.threads), (unsigned)lds, stream, p);
        QKN_HIP(hipGetLastError());
    }
    return QKN_OK;
}

int shard_sumsq(int dtype, const void* x, int64_t T, int64_t H, int N, float* partials,
                hipStream_t s)
{
    t_hip_error.clear();
    int rc = check_dims(T, H, N);
    if (rc) return rc;
    if (T == 0) return QKN_OK;
    if (!x || !partials) return QKN_EINVAL;
    if (overlaps(range_of(partials, (int64_t)N * T * 4), range_of(x, T * H * fmt_of(dtype).in)))
        return QKN_EOVERLAP;
    return launch_sumsq(dtype, x, T, H, N, partials, s);
}

int apply_scale(int dtype, const void* x, const void* g, const float* rinv, int64_t T, int64_t H,
                void* y, hipStream_t s)
{
    t_hip_error.clear();
    int rc = check_dims(T, H, 1);
    if (rc) return rc;
    if (T == 0) return QKN_OK;
    if (!x || !g || !rinv || !y) return QKN_EINVAL;
    const Fmt f = fmt_of(dtype);
    const Range ry = range_of(y, T * H * f.out), rx = range_of(x, T * H * f.in);
    if (overlaps(ry, rx) && !same(ry, rx)) return QKN_EOVERLAP;
    if (overlaps(ry, range_of(g, H * f.gam)) || overlaps(ry, range_of(rinv, T * 4))) return QKN_EOVERLAP;
    return launch_apply(dtype, x, g, rinv, T, H, y, s);
}

}  // namespace

// ================================================================ C ABI

extern "C" {

int qknorm_layerwise_fwd_bf16(const void* q, const void* k, const void* gamma_q, const void* gamma_k,
                              int64_t T, int64_t Hq, int64_t Hk, int n_shards, float eps,
                              void* out_q, void* out_k, hipStream_t stream)
{
    return layerwise_fwd(QKN_BF16, q, k, gamma_q, gamma_k, nullptr, nullptr, T, Hq, Hk, n_shards,
                         eps, out_q, out_k, stream);
}

int qknorm_layerwise_fwd_f32(const void* q, const void* k, const void* gamma_q, const void* gamma_k,
                             int64_t T, int64_t Hq, int64_t Hk, int n_shards, float eps,
                             void* out_q, void* out_k, hipStream_t stream)
{
    return layerwise_fwd(QKN_F32, q, k, gamma_q, gamma_k, nullptr, nullptr, T, Hq, Hk, n_shards,
                         eps, out_q, out_k, stream);
}

int qknorm_layerwise_fwd_bf16_noalloc(const void* q, const void* k, const void* gamma_q,
                                      const void* gamma_k, int64_t T, int64_t Hq, int64_t Hk,
                                      int n_shards, float eps, void* out_q, void* out_k,
                                      hipStream_t stream)
{
    return layerwise_fwd(QKN_FMT_BF16, q, k, gamma_q, gamma_k, nullptr, nullptr, T, Hq, Hk, n_shards,
                         eps, out_q, out_k, stream, true);
}

int qknorm_layerwise_fwd_e4m3(const void* q, const void* k, const void* gamma_q, const void* gamma_k,
                              int64_t T, int64_t Hq, int64_t Hk, int n_shards, float eps,
                              void* out_q, void* out_k, int out_dtype, hipStream_t stream)
{
    const int fmt = e4m3_fmt(out_dtype);
    if (fmt < 0) return QKN_EINVAL;
    return layerwise_fwd(fmt, q, k, gamma_q, gamma_k, nullptr, nullptr, T, Hq, Hk, n_shards, eps,
                         out_q, out_k, stream);
}

int qknorm_shard_sumsq_bf16(const void* x, int64_t T, int64_t H, int n_shards, float* partials,
                            hipStream_t stream)
{
    return shard_sumsq(QKN_BF16, x, T, H, n_shards, partials, stream);
}

int qknorm_shard_sumsq_e4m3(const void* x, int64_t T, int64_t H, int n_shards, float* partials,
                            hipStream_t stream)
{
    return shard_sumsq(QKN_FMT_E4M3_BF16, x, T, H, n_shards, partials, stream);
}

int qknorm_shard_sumsq_f32(const void* x, int64_t T, int64_t H, int n_shards, float* partials,
                           hipStream_t stream)
{
    return shard_sumsq(QKN_F32, x, T, H, n_shards, partials, stream);
}

int qknorm_combine_scale(const float* partials, int64_t T, int64_t H, int n_shards, float eps,
                         float* rms_inv, hipStream_t stream)
{
    t_hip_error.clear();
    int rc = check_dims(T, H, n_shards);
    if (rc) return rc;
    if (!eps_ok(eps)) return QKN_EINVAL;
    if (T == 0) return QKN_OK;
    if (!partials || !rms_inv) return QKN_EINVAL;
    if (overlaps(range_of(partials, (int64_t)n_shards * T * 4), range_of(rms_inv, T * 4)))
        return QKN_EOVERLAP;
    return launch_combine(partials, T, H, n_shards, eps, rms_inv, stream);
}

int qknorm_apply_scale_bf16(const void* x, const void* gamma, const float* rms_inv, int64_t T,
                            int64_t H, void* out, hipStream_t stream)
{
    return apply_scale(QKN_BF16, x, gamma, rms_inv, T, H, out, stream);
}

int qknorm_apply_scale_f32(const void* x, const void* gamma, const float* rms_inv, int64_t T,
                           int64_t H, void* out, hipStream_t stream)
{
    return apply_scale(QKN_F32, x, gamma, rms_inv, T, H, out, stream);
}

int qknorm_apply_scale_e4m3(const void* x, const void* gamma, const float* rms_inv, int64_t T,
                            int64_t H, void* out, int out_dtype, hipStream_t stream)
{
    const int fmt = e4m3_fmt(out_dtype);
    if (fmt < 0) return QKN_EINVAL;
    return apply_scale(fmt, x, gamma, rms_inv, T, H, out, stream);
}

int qknorm_layernorm_fwd_bf16(const void* q, const void* k, const void* gamma_q,
                              const void* gamma_k, const void* beta_q, const void* beta_k,
                              int64_t T, int64_t Hq, int64_t Hk, int n_shards, float eps,
                              void* out_q, void* out_k, hipStream_t stream)
{
    return layerwise_fwd(QKN_FMT_LN_BF16, q, k, gamma_q, gamma_k, beta_q, beta_k, T, Hq, Hk,
                         n_shards, eps, out_q, out_k, stream);
}

int qknorm_layernorm_fwd_f32(const void* q, const void* k, const void* gamma_q,
                             const void* gamma_k, const void* beta_q, const void* beta_k,
                             int64_t T, int64_t Hq, int64_t Hk, int n_shards, float eps,
                             void* out_q, void* out_k, hipStream_t stream)
{
    return layerwise_fwd(QKN_FMT_LN_F32, q, k, gamma_q, gamma_k, beta_q, beta_k, T, Hq, Hk,
                         n_shards, eps, out_q, out_k, stream);
}

static int shard_stats_entry(int fmt, const void* x, int64_t T, int64_t H, int N, float* sums,
                             float* sumsq, hipStream_t s)
{
    t_hip_error.clear();
    int rc = check_dims(T, H, N);
    if (rc) return rc;
    if (T == 0) return QKN_OK;
    if (!x || !sums || !sumsq) return QKN_EINVAL;
    const Range rx = range_of(x, T * H * fmt_of(fmt).in);
    const Range ra = range_of(sums, (int64_t)N * T * 4), rb = range_of(sumsq, (int64_t)N * T * 4);
    if (overlaps(ra, rx) || overlaps(rb, rx) || overlaps(ra, rb)) return QKN_EOVERLAP;
    return launch_stats(fmt, x, T, H, N, sums, sumsq, s);
}

int qknorm_shard_stats_bf16(const void* x, int64_t T, int64_t H, int n_shards, float* sums,
                            float* sumsq, hipStream_t stream)
{
    return shard_stats_entry(QKN_FMT_LN_BF16, x, T, H, n_shards, sums, sumsq, stream);
}

int qknorm_shard_stats_f32(const void* x, int64_t T, int64_t H, int n_shards, float* sums,
                           float* sumsq, hipStream_t stream)
{
    return shard_stats_entry(QKN_FMT_LN_F32, x, T, H, n_shards, sums, sumsq, stream);
}

int qknorm_combine_stats(const float* sums, const float* sumsq, int64_t T, int64_t H, int n_shards,
                         float eps, float* mean, float* rstd, hipStream_t stream)
{
    t_hip_error.clear();
    int rc = check_dims(T, H, n_shards);
    if (rc) return rc;
    if (!eps_ok(eps)) return QKN_EINVAL;
    if (T == 0) return QKN_OK;
    if (!sums || !sumsq || !mean || !rstd) return QKN_EINVAL;
    const Range ra = range_of(sums, (int64_t)n_shards * T * 4);
    const Range rb = range_of(sumsq, (int64_t)n_shards * T * 4);
    const Range rm = range_of(mean, T * 4), rr = range_of(rstd, T * 4);
    if (overlaps(rm, ra) || overlaps(rm, rb) || overlaps(rr, ra) || overlaps(rr, rb) ||
        overlaps(rm, rr))
        return QKN_EOVERLAP;
    return launch_combine_stats(sums, sumsq, T, H, n_shards, eps, mean, rstd, stream);
}

static int apply_norm_entry(int fmt, const void* x, const void* g, const void* b, const float* mean,
                            const float* rstd, int64_t T, int64_t H, void* y, hipStream_t s)
{
    t_hip_error.clear();
    int rc = check_dims(T, H, 1);
    if (rc) return rc;
    if (T == 0) return QKN_OK;
    if (!x || !g || !mean || !rstd || !y) return QKN_EINVAL;
    const Fmt f = fmt_of(fmt);
    const Range ry = range_of(y, T * H * f.out), rx = range_of(x, T * H * f.in);
    if (overlaps(ry, rx) && !same(ry, rx)) return QKN_EOVERLAP;
    if (overlaps(ry, range_of(g, H * f.gam)) || overlaps(ry, range_of(mean, T * 4)) ||
        overlaps(ry, range_of(rstd, T * 4)) || (b && overlaps(ry, range_of(b, H * f.gam))))
        return QKN_EOVERLAP;
    return launch_apply_norm(fmt, x, g, b, mean, rstd, T, H, y, s);
}

int qknorm_apply_norm_bf16(const void* x, const void* gamma, const void* beta, const float* mean,
                           const float* rstd, int64_t T, int64_t H, void* out, hipStream_t stream)
{
    return apply_norm_entry(QKN_FMT_LN_BF16, x, gamma, beta, mean, rstd, T, H, out, stream);
}

int qknorm_apply_norm_f32(const void* x, const void* gamma, const void* beta, const float* mean,
                          const float* rstd, int64_t T, int64_t H, void* out, hipStream_t stream)
{
    return apply_norm_entry(QKN_FMT_LN_F32, x, gamma, beta, mean, rstd, T, H, out, stream);
}

int qknorm_headwise_fwd_bf16(const void* q, const void* k, const void* gamma_q, const void* gamma_k,
                             int64_t T, int64_t heads_q, int64_t heads_k, int64_t head_dim,
                             float eps, void* out_q, void* out_k, hipStream_t stream)
{
    return headwise_fwd(QKN_FMT_BF16, q, k, gamma_q, gamma_k, T, heads_q, heads_k, head_dim, eps,
                        out_q, out_k, stream);
}

int qknorm_headwise_fwd_f32(const void* q, const void* k, const void* gamma_q, const void* gamma_k,
                            int64_t T, int64_t heads_q, int64_t heads_k, int64_t head_dim,
                            float eps, void* out_q, void* out_k, hipStream_t stream)
{
    return headwise_fwd(QKN_FMT_F32, q, k, gamma_q, gamma_k, T, heads_q, heads_k, head_dim, eps,
                        out_q, out_k, stream);
}

int qknorm_check_fault(hipStream_t stream)
{
    t_hip_error.clear();
    int dev = 0;
    int rc = current_device(&dev);
    if (rc) return rc;
    QKN_HIP(hipStreamSynchronize(stream));
    // the stream's workspace and the device's static scratch each hold a fault word
    uint32_t* faults[3] = {nullptr, nullptr, nullptr};
    {
        std::lock_guard<std::mutex> lock(g_mu);
        auto it = g_ws.find({dev, stream});
        if (it != g_ws.end()) faults[0] = it->second.fault;
        auto st = g_static.find(dev);
        if (st != g_static.end() && st->second.base) faults[1] = st->second.fault();
        auto gr = g_graph.find(dev);
        if (gr != g_graph.end() && gr->second.base) faults[2] = gr->second.fault();
    }
    bool timed_out = false;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        auto fl = g_flag.find(dev);
        if (fl != g_flag.end() && fl->second.host) {
            volatile uint32_t* h = fl->second.host;
            if (*h) timed_out = true;
            *h = 0;
        }
    }
    for (uint32_t* fault : faults) {
        if (!fault) continue;
        uint32_t h = 0;
        QKN_HIP(hipMemcpy(&h, fault, sizeof h, hipMemcpyDeviceToHost));
        if (h == 0) continue;
        QKN_HIP(hipMemset(fault, 0, sizeof h));
        timed_out = true;
    }
    return timed_out ? QKN_ETIMEOUT : QKN_OK;
}

int qknorm_fault_pending(void)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lock(g_mu);
    auto fl = g_flag.find(dev);
    if (fl == g_flag.end() || !fl->second.host) return 0;
    return *static_cast<volatile uint32_t*>(fl->second.host) != 0;
}

const uint32_t* qknorm_fault_flag(void)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return nullptr;
    std::lock_guard<std::mutex> lock(g_mu);
    return fault_flag(dev, true)->host;
}

const char* qknorm_strerror(int status)
{
    switch (status) {
    case QKN_OK: return "success";
    case QKN_EINVAL: return "invalid argument";
    case QKN_EOVERLAP: return "an output partially overlaps an input or another output";
    case QKN_ENOMEM: return "workspace allocation failed";
    case QKN_EHIP: return "HIP runtime error";
    case QKN_ERESIDENCY: return "the device cannot hold n_shards co-resident workgroups";
    case QKN_ETIMEOUT: return "a shard exchange timed out; outputs of that call are unspecified";
    case QKN_ECAPTURE: return "the cooperative launch option cannot be recorded under stream capture";
    case QKN_ESCRATCH: return "the call needs more exchange slots than the static scratch holds";
    default: return "unknown status";
    }
}

const char* qknorm_last_hip_error(void) { return t_hip_error.c_str(); }

int qknorm_max_coresident_workgroups(int dtype, int64_t Hq, int64_t Hk, int n_shards, int* out)
{
    t_hip_error.clear();
    if (!out || !fmt_valid(dtype)) return QKN_EINVAL;
    std::lock_guard<std::mutex> lock(g_mu);
    int dev = 0, rc = current_device(&dev);
    if (rc) return rc;
    DevInfo* di = nullptr;
    if ((rc = device_info(dev, dtype, &di))) return rc;
    qknorm_plan pl;
    if ((rc = plan(dtype, 1 << 20, Hq, Hk, n_shards, di->cu, &di->occ[dtype][0][0], &di->occ_st[dtype][0][0], 1,
                   &pl)))
        return rc;
    *out = pl.variant < 0 ? 0
                          : (pl.st ? di->occ_st[dtype][pl.variant][pl.data_waves]
                                   : di->occ[dtype][pl.variant][pl.data_waves]) * di->cu;
    return QKN_OK;
}

int qknorm_device_occupancy(int dtype, int* blocks_per_cu, int* cu_count)
{
    t_hip_error.clear();
    if (!blocks_per_cu || !cu_count || !fmt_valid(dtype)) return QKN_EINVAL;
    std::lock_guard<std::mutex> lock(g_mu);
    int dev = 0, rc = current_device(&dev);
    if (rc) return rc;
    DevInfo* di = nullptr;
    if ((rc = device_info(dev, dtype, &di))) return rc;
    // a variant built for single-tensor tiles only reports that kernel's occupancy
    for (int v = 0; v < QKN_NUM_VARIANTS; ++v) {
        const bool st_only = !fused_fn_layout(dtype, v, false) && fused_fn_layout(dtype, v, true);
        for (int w = 0; w <= QKN_MAX_DATA_WAVES; ++w)
            blocks_per_cu[v * (QKN_MAX_DATA_WAVES + 1) + w] = st_only ? di->occ_st[dtype][v][w] : di->occ[dtype][v][w];
    }
    *cu_count = di->cu;
    return QKN_OK;
}

int qknorm_release_workspace(void)
{
    std::lock_guard<std::mutex> lock(g_mu);
    int prev = 0;
    (void)hipGetDevice(&prev);
    for (auto& kv : g_ws) {
        Workspace& w = kv.second;
        (void)hipSetDevice(w.device);
        if (w.slots) (void)hipFree(w.slots);
        if (w.fault) (void)hipFree(w.fault);
        if (w.scratch) (void)hipFree(w.scratch);
    }
    g_ws.clear();
    (void)hipSetDevice(prev);
    return QKN_OK;
}

int qknorm_plan_fused(int dtype, int64_t T, int64_t Hq, int64_t Hk, int n_shards, int cu_count,
                      const int* blocks_per_cu, int aligned, qknorm_plan* out)
{
    if (!out) return QKN_EINVAL;
    // single-tensor-tile kernels occupy the device like the mixed-tile ones of
    // the same variant (same registers per wave; twice the LDS, never the limit
    // for the launches planned); the caller's table serves for both
    return plan(dtype, T, Hq, Hk, n_shards, cu_count, blocks_per_cu, blocks_per_cu, aligned, out);
}

int qknorm_set_option(int key, int64_t value)
{
    std::lock_guard<std::mutex> lock(g_mu);
    ++g_opt_epoch;
    switch (key) {
    case QKN_OPT_SPIN_LIMIT_NS: if (value < 1) return QKN_EINVAL; g_opt.spin_ns = value; return QKN_OK;
    case QKN_OPT_FORCE_VARIANT:
        if (value < -1 || value >= QKN_NUM_VARIANTS) return QKN_EINVAL;
        g_opt.force_variant = value; return QKN_OK;
    case QKN_OPT_ROWS:
        if (value < 0 || value > qkn::kMaxSeg) return QKN_EINVAL;
        g_opt.rows = value; return QKN_OK;
    case QKN_OPT_DATA_WAVES:
        if (value < 0 || value > QKN_MAX_DATA_WAVES) return QKN_EINVAL;
        g_opt.force_data_waves = value; return QKN_OK;
    case QKN_OPT_XCD_MAP: if (value < -1 || value > 1) return QKN_EINVAL; g_opt.xcd_map = value; return QKN_OK;
    case QKN_OPT_COOPERATIVE: g_opt.cooperative = value ? 1 : 0; return QKN_OK;
    case QKN_OPT_MAX_GROUPS: if (value < 0) return QKN_EINVAL; g_opt.max_groups = value; return QKN_OK;
    case QKN_OPT_FORCE_SPLIT: g_opt.force_split = value ? 1 : 0; return QKN_OK;
    case QKN_OPT_TEST_SKIP_PUBLISH: g_opt.test_skip_publish = value ? 1 : 0; return QKN_OK;
    case QKN_OPT_SPLIT_VECTORS:
        if (value != 0 && value != 1 && value != 2 && value != 4 && value != 8) return QKN_EINVAL;
        g_opt.split_vectors = value; return QKN_OK;
    case QKN_OPT_TILE_LAYOUT:
        if (value < 0 || value > 2) return QKN_EINVAL;
        g_opt.tile_layout = value; return QKN_OK;
    case QKN_OPT_WPC:
        if (value < 0 || value > 64) return QKN_EINVAL;
        g_opt.wpc = value; return QKN_OK;
    case QKN_OPT_PACE:
        if (value < -1 || value > 100000) return QKN_EINVAL;
        g_opt.pace_gbs = value; return QKN_OK;
    case QKN_OPT_STATIC_SLOTS:
        if (value < 0 || (uint64_t)value > kStaticSlots) return QKN_EINVAL;
        g_static_slot_limit = (size_t)value; return QKN_OK;
    default: return QKN_EINVAL;
    }
}

int64_t qknorm_get_option(int key)
{
    switch (key) {
    case QKN_OPT_SPIN_LIMIT_NS: return g_opt.spin_ns;
    case QKN_OPT_FORCE_VARIANT: return g_opt.force_variant;
    case QKN_OPT_ROWS: return g_opt.rows;
    case QKN_OPT_DATA_WAVES: return g_opt.force_data_waves;
    case QKN_OPT_XCD_MAP: return g_opt.xcd_map;
    case QKN_OPT_COOPERATIVE: return g_opt.cooperative;
    case QKN_OPT_MAX_GROUPS: return g_opt.max_groups;
    case QKN_OPT_FORCE_SPLIT: return g_opt.force_split;
    case QKN_OPT_TEST_SKIP_PUBLISH: return g_opt.test_skip_publish;
    case QKN_OPT_SPLIT_VECTORS: return g_opt.split_vectors;
    case QKN_OPT_TILE_LAYOUT: return g_opt.tile_layout;
    case QKN_OPT_WPC: return g_opt.wpc;
    case QKN_OPT_PACE: return g_opt.pace_gbs;
    case QKN_OPT_STATIC_SLOTS: return (int64_t)g_static_slot_limit;
    default: return INT64_MIN;
    }
}

int qknorm_bench_copy(const void* q, const void* k, void* out_q, void* out_k, int64_t bytes_q,
                      int64_t bytes_k, hipStream_t stream)
{
    t_hip_error.clear();
    if (bytes_q < 0 || bytes_k < 0) return QKN_EINVAL;
    if (bytes_q + bytes_k == 0) return QKN_OK;
    // a tensor of no bytes may come with a null pointer (empty tensors have none)
    if ((bytes_q && (!q || !out_q)) || (bytes_k && (!k || !out_k))) return QKN_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(out_q) || !aligned16(out_k)) return QKN_EINVAL;
    if (overlaps(range_of(out_q, bytes_q), range_of(q, bytes_q)) ||
        overlaps(range_of(out_q, bytes_q), range_of(k, bytes_k)) ||
        overlaps(range_of(out_k, bytes_k), range_of(q, bytes_q)) ||
        overlaps(range_of(out_k, bytes_k), range_of(k, bytes_k)) ||
        overlaps(range_of(out_q, bytes_q), range_of(out_k, bytes_k)))
        return QKN_EOVERLAP;
    if (bytes_q > kCeilingMaxBytes || bytes_k > kCeilingMaxBytes) return QKN_EINVAL;
    const uint32_t na = (uint32_t)(bytes_q / 16 * 16), nb = (uint32_t)(bytes_k / 16 * 16);
    const uint32_t wa = (na / 16 + kCopyThreads - 1) / kCopyThreads, wb = (nb / 16 + kCopyThreads - 1) / kCopyThreads;
    hipLaunchKernelGGL(qkn::copy_ceiling_kernel<kCopyThreads>, dim3(std::max(1u, wa + wb)), dim3(kCopyThreads), 0,
                       stream, q, k, out_q, out_k, na, nb, wa, (uint32_t)(bytes_q - na), (uint32_t)(bytes_k - nb));
    QKN_HIP(hipGetLastError());
    return QKN_OK;
}

int qknorm_bench_widen(const void* q, const void* k, void* out_q, void* out_k, int64_t bytes_q,
                       int64_t bytes_k, hipStream_t stream)
{
    t_hip_error.clear();
    if (bytes_q < 0 || bytes_k < 0) return QKN_EINVAL;
    if (bytes_q + bytes_k == 0) return QKN_OK;
    // a tensor of no bytes may come with a null pointer (empty tensors have none)
    if ((bytes_q && (!q || !out_q)) || (bytes_k && (!k || !out_k))) return QKN_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(out_q) || !aligned16(out_k)) return QKN_EINVAL;
    if (overlaps(range_of(out_q, 2 * bytes_q), range_of(q, bytes_q)) ||
        overlaps(range_of(out_q, 2 * bytes_q), range_of(k, bytes_k)) ||
        overlaps(range_of(out_k, 2 * bytes_k), range_of(q, bytes_q)) ||
        overlaps(range_of(out_k, 2 * bytes_k), range_of(k, bytes_k)) ||
        overlaps(range_of(out_q, 2 * bytes_q), range_of(out_k, 2 * bytes_k)))
        return QKN_EOVERLAP;
    if (2 * bytes_q > kCeilingMaxBytes || 2 * bytes_k > kCeilingMaxBytes) return QKN_EINVAL;
    const uint32_t na = (uint32_t)(bytes_q / 8 * 8), nb = (uint32_t)(bytes_k / 8 * 8);
    const uint32_t wa = (na / 8 + kWidenThreads - 1) / kWidenThreads, wb = (nb / 8 + kWidenThreads - 1) / kWidenThreads;
    hipLaunchKernelGGL(qkn::widen_ceiling_kernel<kWidenThreads>, dim3(std::max(1u, wa + wb)), dim3(kWidenThreads), 0,
                       stream, q, k, out_q, out_k, na, nb, wa, (uint32_t)(bytes_q - na), (uint32_t)(bytes_k - nb));
    QKN_HIP(hipGetLastError());
    return QKN_OK;
}

int qknorm_bench_skeleton(int dtype, const void* q, const void* k, void* out_q, void* out_k, int64_t T,
                          int64_t Hq, int64_t Hk, int n_shards, hipStream_t stream)
{
    t_hip_error.clear();
    if (!fmt_valid(dtype)) return QKN_EINVAL;
    int rc = check_dims(T, Hq, n_shards);
    if (rc) return rc;
    if ((rc = check_dims(T, Hk, n_shards))) return rc;
    if (T == 0) return QKN_OK;
    if (!q || !k || !out_q || !out_k) return QKN_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(out_q) || !aligned16(out_k)) return QKN_EINVAL;
    const Fmt f = fmt_of(dtype);
    const Range rq = range_of(q, T * Hq * f.in), rk = range_of(k, T * Hk * f.in);
    const Range roq = range_of(out_q, T * Hq * f.out), rok = range_of(out_k, T * Hk * f.out);
    if (overlaps(roq, rok) || overlaps(roq, rq) || overlaps(roq, rk) || overlaps(rok, rq) || overlaps(rok, rk))
        return QKN_EOVERLAP;
    // one launch: every tensor below 2^31 - 2^16 bytes (32-bit buffer offsets)
    if (T * std::max(Hq, Hk) * std::max(f.in, f.out) > (int64_t(1) << 31) - (int64_t(1) << 16)) return QKN_EINVAL;
    std::lock_guard<std::mutex> lock(g_mu);
    int dev = 0;
    if ((rc = current_device(&dev))) return rc;
    DevInfo* di = nullptr;
    if ((rc = device_info(dev, dtype, &di))) return rc;
    qknorm_plan pl;
    if ((rc = plan(dtype, T, Hq, Hk, n_shards, di->cu, &di->occ[dtype][0][0], &di->occ_st[dtype][0][0], 1, &pl)))
        return rc;
    if (pl.variant < 0) return QKN_EINVAL;  // the shape has no fused launch to mirror
    const SkelFn fn = skeleton_fn(kVariants[pl.variant].vpt, pl.st != 0, f.out == 2 * f.in);
    if (!fn) return QKN_EINVAL;
    qkn::SkeletonParams p;
    std::memset(&p, 0, sizeof p);
    p.x[0] = q;
    p.x[1] = k;
    p.y[0] = out_q;
    p.y[1] = out_k;
    p.T = T;
    p.n_tiles = pl.n_tiles;
    p.nq = pl.st ? (T + pl.rows - 1) / pl.rows : 0;
    p.H[0] = (int32_t)Hq;
    p.H[1] = (int32_t)Hk;
    p.Wv[0] = (int32_t)(Hq / n_shards / f.ev);
    p.Wv[1] = (int32_t)(Hk / n_shards / f.ev);
    p.rows = pl.rows;
    p.nwd = pl.data_waves;
    p.n_shards = n_shards;
    p.n_groups = pl.n_groups;
    p.xcd_map = pl.xcd_map;
    p.in_bytes = f.in;
    p.pace = pace_period(pl, p.Wv[0], p.Wv[1], f, di->wall_khz);
    p.stagger = p.pace && paced_staggered(dtype, pl.variant, pl.st != 0) ? 1u : 0u;
    hipLaunchKernelGGL(fn, dim3(pl.grid), dim3(pl.threads), 0, stream, p);
    QKN_HIP(hipGetLastError());
    return QKN_OK;
}

int qknorm_bench_fused(int dtype, const void* q, const void* k, const void* gamma_q,
                       const void* gamma_k, int64_t T, int64_t Hq, int64_t Hk, int n_shards,
                       float eps, void* out_q, void* out_k, int repeats, hipStream_t stream)
{
    if (!fmt_valid(dtype)) return QKN_EINVAL;
    if (repeats < 0) return QKN_EINVAL;
    for (int i = 0; i < repeats; ++i) {
        const int rc = layerwise_fwd(dtype, q, k, gamma_q, gamma_k, nullptr, nullptr, T, Hq, Hk,
                                     n_shards, eps, out_q, out_k, stream);
        if (rc) return rc;
    }
    return QKN_OK;
}

}  // extern "C"
