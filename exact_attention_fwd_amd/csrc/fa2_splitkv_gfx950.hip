// Split key/value attention for short query blocks (decoding) on gfx950, and
// the merge of partial results.
//
// What is computed: non-causal O = softmax(scale Q K^T) V and LSE for Nq
// query rows (typically a few new tokens) against Nk cached keys.  With few
// queries there are too few query tiles to fill 256 CUs, so the keys are
// split: each workgroup attends one query tile to one range of keys and
// leaves a partial result, normalised over its keys, with the log-sum-exp
// of its scores; a second kernel merges the parts,
//     LSE = M + ln sum_s exp(LSE_s - M),   O = sum_s exp(LSE_s - LSE) O_s,
// which is the online-softmax recurrence applied to whole parts ("3.6
// Attention I -- the memory problem and FlashAttention principles", 3.6.4;
// the result does not depend on how keys are grouped).  The pages name this
// scheme for decoding (3.6.9, 3.6.10) without giving its steps.
//
// Partial kernel: a workgroup is 4 waves sharing one tile of 32 queries; the
// waves take the 64-key tiles of the range in turn (wave w: tiles w, w+4, ..)
// and each keeps its own (m, l, acc).  K is loaded from global memory
// straight into the MFMA A-operand layout of S^T = K Q^T (no LDS); V goes
// through a per-wave LDS tile for the transposed read of O^T = V^T P^T.  A
// wave issues the loads of its next tile before computing the current one,
// and no workgroup barrier is needed until the end, where the four waves'
// states are merged through LDS.  With a single range the workgroup writes
// the final fp16 O and LSE itself.  The bound is HBM: every key and value is
// read once per query tile.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <cmath>

#include "fa2.h"
#include "fa2_device.h"
#include "fa2_launch.h"

namespace fa2 {
namespace {

using namespace dev;

template <int D>
struct SkvCfg {
    static_assert(D == 32 || D == 64 || D == 96 || D == 128, "head dim");
    static constexpr int kWaves = 4;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kQT = kQW;                    // queries per workgroup
    static constexpr int kRowBytes = D * 2;
    static constexpr int kChunks = D / 8;
    static constexpr int kTileBytes = kBK * kRowBytes; // one wave's V tile (= 32 x D fp32)
    static constexpr int kDSteps = D / 16;
    static constexpr int kDBlocks = D / 32;
    static constexpr int kWavesPerSimd = D >= 96 ? 1 : 2;
};

template <int D>
__global__ __launch_bounds__(SkvCfg<D>::kThreads)
__attribute__((amdgpu_waves_per_eu(SkvCfg<D>::kWavesPerSimd, SkvCfg<D>::kWavesPerSimd)))
void splitkv_partial_kernel(const _Float16* __restrict__ Q, const _Float16* __restrict__ K,
                            const _Float16* __restrict__ V, _Float16* __restrict__ O,
                            float* __restrict__ LSE, float* __restrict__ Opart,
                            float* __restrict__ Lpart, int Nq, int Nk, int n_qt, int n_splits,
                            int tiles_per_split, int rows, int n_wg, float c, uint32_t q_and,
                            uint32_t q_xor) {
    using C = SkvCfg<D>;
    __shared__ __attribute__((aligned(16))) unsigned char vbuf[C::kWaves][C::kTileBytes];
    __shared__ float m_s[C::kWaves][kQW], l_s[C::kWaves][kQW];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    // logical = ((bh * n_splits) + split) * n_qt + qt
    const int logical = xcd_logical_id(blockIdx.x, n_wg);
    const int qt = __builtin_amdgcn_readfirstlane(logical % n_qt);
    const int rest = __builtin_amdgcn_readfirstlane(logical / n_qt);
    const int split = __builtin_amdgcn_readfirstlane(rest % n_splits);
    const int bh = __builtin_amdgcn_readfirstlane(rest / n_splits);

    const int q0 = qt * C::kQT;
    const int my_q = q0 + l32;
    const auto rQ = make_rsrc(Q + size_t(bh) * Nq * D, uint32_t(Nq) * C::kRowBytes);
    const auto rK = make_rsrc(K + size_t(bh) * Nk * D, uint32_t(Nk) * C::kRowBytes);
    const auto rV = make_rsrc(V + size_t(bh) * Nk * D, uint32_t(Nk) * C::kRowBytes);

    h8 qf[C::kDSteps];
#pragma unroll
    for (int ds = 0; ds < C::kDSteps; ++ds) {
        u32x4 raw = __builtin_amdgcn_raw_buffer_load_b128(rQ, my_q * C::kRowBytes + 32 * ds + 16 * hi, 0, 0);
        qf[ds] = __builtin_bit_cast(h8, (raw & q_and) ^ q_xor);
    }

    const int n_tk = (Nk + kBK - 1) / kBK;
    const int t_end = min(n_tk, (split + 1) * tiles_per_split);
    unsigned char* vt = &vbuf[wave][0];
    const TrBase vtr(lane);

    // K of a tile in A-operand layout: block kb, d-step ds: key 32*kb + l32,
    // dims 16*ds + 8*hi .. +7.  V of a tile: row `lane`, every chunk.
    auto load_k = [&](h8 (&kf)[2][C::kDSteps], int t) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int ds = 0; ds < C::kDSteps; ++ds)
                kf[kb][ds] = __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(
                    rK, (t * kBK + 32 * kb + l32) * C::kRowBytes + 32 * ds + 16 * hi, 0, 0));
        }
    };
    u32x4 vs[C::kChunks];
    auto load_v = [&](int t) {
#pragma unroll
        for (int j = 0; j < C::kChunks; ++j)
            vs[j] = __builtin_amdgcn_raw_buffer_load_b128(rV, (t * kBK + lane) * C::kRowBytes + 16 * j, 0, 0);
    };

    float m2 = -INFINITY, lsum = 0.f;
    f32x16 acc[C::kDBlocks];
#pragma unroll
    for (int db = 0; db < C::kDBlocks; ++db) acc[db] = f32x16{};

    // One tile: V to LDS, next tile's loads, S^T, online softmax, O^T += V^T P^T.
    auto step = [&](int t, h8 (&kf)[2][C::kDSteps], h8 (&kf_next)[2][C::kDSteps]) {
#pragma unroll
        for (int j = 0; j < C::kChunks; ++j) *reinterpret_cast<u32x4*>(vt + lds_v_off(j, lane)) = vs[j];
        if (t + C::kWaves < t_end) {
            load_k(kf_next, t + C::kWaves);
            load_v(t + C::kWaves);
        }
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            f32x16 a = f32x16{};
#pragma unroll
            for (int ds = 0; ds < C::kDSteps; ++ds)
                a = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[kb][ds], qf[ds], a, 0, 0, 0);
            s[kb] = a;
        }
        if (t * kBK + kBK > Nk) {   // keys past Nk in the last tile
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (t * kBK + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3) >= Nk) s[kb][r] = -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 32; ++i) mx = __builtin_fmaxf(mx, s[i >> 4][i & 15]);
        const float m_new = __builtin_fmaxf(m2, c * pair_max(mx));
        const float sh = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m2 - sh);
        float ls = 0.f;
        h8 pf[4];
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i >> 4][i & 15], c, -sh));
            ls += p;
            pf[i >> 3][i & 7] = (_Float16)p;
        }
        lsum = alpha * lsum + ls;
        m2 = m_new;
#pragma unroll
        for (int db = 0; db < C::kDBlocks; ++db) acc[db] *= alpha;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int db = 0; db < C::kDBlocks; ++db)
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(read_tr_operand(vt, vtr, tr_imm(ks, db)),
                                                                 pf[ks], acc[db], 0, 0, 0);
        }
    };

    h8 kfa[2][C::kDSteps], kfb[2][C::kDSteps];
    int t = split * tiles_per_split + wave;
    if (t < t_end) {
        load_k(kfa, t);
        load_v(t);
    }
    for (; t + C::kWaves < t_end; t += 2 * C::kWaves) {
        step(t, kfa, kfb);
        step(t + C::kWaves, kfb, kfa);
    }
    if (t < t_end) step(t, kfa, kfb);

    // Merge the four waves: each leaves (m, l) per query and its acc (32 x D
    // fp32, row-major) in its own LDS tile, which it no longer reads.
    const float lt = pair_sum(lsum);
    if (hi == 0) {
        m_s[wave][l32] = m2;
        l_s[wave][l32] = lt;
    }
#pragma unroll
    for (int db = 0; db < C::kDBlocks; ++db) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const float4 x = make_float4(acc[db][4 * rr], acc[db][4 * rr + 1], acc[db][4 * rr + 2],
                                         acc[db][4 * rr + 3]);
            *reinterpret_cast<float4*>(vt + (l32 * D + 32 * db + 8 * rr + 4 * hi) * 4) = x;
        }
    }
    __syncthreads();
    // Thread -> (query qi, 8 columns): kThreads = 32 queries x (D/8) column groups
    // when D = 64; for other D the column groups are walked in a loop.
    constexpr int kGroups = D / 8;
    for (int item = tid; item < kQW * kGroups; item += C::kThreads) {
        const int qi = item / kGroups, cg = item % kGroups;
        float mw[C::kWaves], M = -INFINITY;
#pragma unroll
        for (int w = 0; w < C::kWaves; ++w) {
            mw[w] = m_s[w][qi];
            M = __builtin_fmaxf(M, mw[w]);
        }
        const float shm = M == -INFINITY ? 0.f : M;
        float L = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < C::kWaves; ++w) {
            const float e = __builtin_amdgcn_exp2f(mw[w] - shm);
            L += e * l_s[w][qi];
            const float* src = reinterpret_cast<const float*>(&vbuf[w][0]) + qi * D + 8 * cg;
#pragma unroll
            for (int k = 0; k < 8; ++k) o[k] += e * src[k];
        }
        const float inv = L > 0.f ? 1.0f / L : 0.f;
        const int q = q0 + qi;
        if (q >= Nq) continue;
        const size_t row = size_t(bh) * Nq + q;
        const float lse = L > 0.f ? (shm + __builtin_amdgcn_logf(L)) * kLn2 : -INFINITY;
        if (n_splits == 1) {
            h8 out;
#pragma unroll
            for (int k = 0; k < 8; ++k) out[k] = (_Float16)(o[k] * inv);
            *reinterpret_cast<h8*>(O + row * D + 8 * cg) = out;
            if (cg == 0) LSE[row] = lse;
        } else {
            float* dst = Opart + (size_t(split) * rows + row) * D + 8 * cg;
            *reinterpret_cast<float4*>(dst) = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
            *reinterpret_cast<float4*>(dst + 4) = make_float4(o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv);
            if (cg == 0) Lpart[size_t(split) * rows + row] = lse;
        }
    }
}

// Merge of n_parts partial results, one thread per (row, 8 columns).
template <int D>
__global__ __launch_bounds__(256) void lse_merge_kernel(const float* __restrict__ Opart,
                                                        const float* __restrict__ Lpart,
                                                        _Float16* __restrict__ O,
                                                        float* __restrict__ LSE, int n_parts,
                                                        int rows) {
    constexpr int kGroups = D / 8;
    const long gid = long(blockIdx.x) * 256 + threadIdx.x;
    if (gid >= long(rows) * kGroups) return;
    const int row = int(gid / kGroups), cg = int(gid % kGroups);
    float M = -INFINITY;
    for (int s = 0; s < n_parts; ++s) M = __builtin_fmaxf(M, Lpart[size_t(s) * rows + row]);
    const float sh = M == -INFINITY ? 0.f : M;
    float L = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < n_parts; ++s) {
        const float w = __builtin_amdgcn_exp2f((Lpart[size_t(s) * rows + row] - sh) * kLog2e);
        if (w == 0.f) continue;   // an empty part (LSE = -inf) may hold anything
        L += w;
        const float4* src = reinterpret_cast<const float4*>(Opart + (size_t(s) * rows + row) * D + 8 * cg);
        const float4 a = src[0], b = src[1];
        o[0] += w * a.x; o[1] += w * a.y; o[2] += w * a.z; o[3] += w * a.w;
        o[4] += w * b.x; o[5] += w * b.y; o[6] += w * b.z; o[7] += w * b.w;
    }
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    h8 out;
#pragma unroll
    for (int k = 0; k < 8; ++k) out[k] = (_Float16)(o[k] * inv);
    *reinterpret_cast<h8*>(O + size_t(row) * D + 8 * cg) = out;
    if (cg == 0) LSE[row] = L > 0.f ? sh + __builtin_amdgcn_logf(L) * kLn2 : -INFINITY;
}

template <int D>
hipError_t launch_merge_t(const float* opart, const float* lpart, void* o, float* lse,
                          int n_parts, int rows, hipStream_t stream) {
    const long threads = long(rows) * (D / 8);
    hipLaunchKernelGGL((lse_merge_kernel<D>), dim3(unsigned((threads + 255) / 256)), dim3(256), 0,
                       stream, opart, lpart, static_cast<_Float16*>(o), lse, n_parts, rows);
    return hipGetLastError();
}

template <int D>
hipError_t launch_splitkv_t(const void* q, const void* k, const void* v, void* o, float* lse,
                            void* ws, int BH, int Nq, int Nk, const SplitPlan& plan, float c,
                            uint32_t q_and, uint32_t q_xor, hipStream_t stream) {
    using C = SkvCfg<D>;
    const int n_qt = (Nq + C::kQT - 1) / C::kQT;
    const int n_wg = BH * n_qt * plan.n_splits;
    const int rows = BH * Nq;
    float* opart = static_cast<float*>(ws);
    float* lpart = opart ? opart + size_t(plan.n_splits) * rows * D : nullptr;
    hipLaunchKernelGGL((splitkv_partial_kernel<D>), dim3(n_wg), dim3(C::kThreads), 0, stream,
                       static_cast<const _Float16*>(q), static_cast<const _Float16*>(k),
                       static_cast<const _Float16*>(v), static_cast<_Float16*>(o), lse, opart,
                       lpart, Nq, Nk, n_qt, plan.n_splits, plan.tiles_per_split, rows, n_wg, c,
                       q_and, q_xor);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.n_splits == 1) return e;
    return launch_merge_t<D>(opart, lpart, o, lse, plan.n_splits, rows, stream);
}

}  // namespace

// Fixed scratch of fa2_fwd_splitkv_noalloc: the partial outputs and
// log-sum-exps of the key ranges, for callers that cannot allocate.  Every
// device that runs the library holds its own copy until the process ends.
// Host code never takes the array's name as a device address (on the host
// it names a stand-in): the address comes from hipGetSymbolAddress.
__device__ __align__(256) unsigned char scratch[FA2_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, void** out) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    int dev = cur;
    if (stream != nullptr && (e = hipStreamGetDevice(stream, &dev)) != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        // Once per device, with that device current.  Two threads racing
        // here look up the same address.
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t back = hipSetDevice(cur);
            if (e == hipSuccess) e = back;
        }
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_addr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

hipError_t launch_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                          void* ws, int BH, int Nq, int Nk, int d, float scale,
                          const SplitPlan& plan, hipStream_t stream) {
    const double a = std::fabs(static_cast<double>(scale));
    const bool zero = !(a >= 1.17549435082228751e-38);
    const float c = zero ? 1.0f : static_cast<float>(a * 1.4426950408889634);
    const uint32_t q_and = zero ? 0u : 0xffffffffu;
    const uint32_t q_xor = (!zero && scale < 0.f) ? 0x80008000u : 0u;
    switch (d) {
        case 32: return launch_splitkv_t<32>(q, k, v, o, lse, ws, BH, Nq, Nk, plan, c, q_and, q_xor, stream);
        case 64: return launch_splitkv_t<64>(q, k, v, o, lse, ws, BH, Nq, Nk, plan, c, q_and, q_xor, stream);
        case 96: return launch_splitkv_t<96>(q, k, v, o, lse, ws, BH, Nq, Nk, plan, c, q_and, q_xor, stream);
        case 128: return launch_splitkv_t<128>(q, k, v, o, lse, ws, BH, Nq, Nk, plan, c, q_and, q_xor, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_lse_merge(const float* opart, const float* lpart, void* o, float* lse,
                            int n_parts, int rows, int d, hipStream_t stream) {
    switch (d) {
        case 32: return launch_merge_t<32>(opart, lpart, o, lse, n_parts, rows, stream);
        case 64: return launch_merge_t<64>(opart, lpart, o, lse, n_parts, rows, stream);
        case 96: return launch_merge_t<96>(opart, lpart, o, lse, n_parts, rows, stream);
        case 128: return launch_merge_t<128>(opart, lpart, o, lse, n_parts, rows, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fa2
