// FlashAttention-1 loop order on gfx950: the comparator of the FA2 forward.
//
// Same result as fa2_fwd (O = softmax(scale Q K^T) V and LSE), computed in
// the order that "Implementing FlashAttention 1 and 2 forward in Triton"
// describes for FA1 (sections "parallelisation unit" and "output
// accumulation"): one workgroup per (batch, head); the key/value blocks are
// the outer loop and, for each of them, every query block is visited; after
// each key/value block the query block's output, already normalised, and its
// statistics (m, l) go back to global memory in fp32 and are read again for
// the next block; fp16 only at the very end.  The per-block update is the
// online-softmax recurrence with a normalised output ("3.6 Attention I",
// 3.6.4):
//     m_new = max(m, m~),  a = l e^(m - m_new),  b = e^(m~ - m_new),
//     l_new = a + b l~,    O_new = (a O + b P~ V) / l_new,
// with m~, P~ = e^(S - m~), l~ = rowsum P~ of the block.
//
// The building blocks are the FA2 kernel's (fa2_device.h): S^T = K Q^T with
// one query per lane, P reused from the accumulator as the B operand of
// O^T = V^T P^T, transposed V reads.  The key/value block is 128 keys (the
// block the Triton FA1 measured best), held in LDS for the whole inner loop
// and prefetched into registers one block ahead; the grid has only B*H
// workgroups, which is the structural difference the comparison is about.
// Head dim 64, the one the FA1 comparison is measured at.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "fa2_device.h"
#include "fa2_launch.h"

namespace fa2 {
namespace {

using namespace dev;

template <int D>
struct Fa1Cfg {
    static_assert(D == 64, "head dim");
    static constexpr int kWaves = 4;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kBM = kWaves * kQW;         // queries per inner step
    static constexpr int kSub = 2;                   // 64-key sub-tiles per key/value block
    static constexpr int kBN = kSub * kBK;           // keys per key/value block
    static constexpr int kRowBytes = D * 2;
    static constexpr int kChunks = D / 8;
    static constexpr int kTileBytes = kBK * kRowBytes;
    static constexpr int kDSteps = D / 16;
    static constexpr int kDBlocks = D / 32;
    static constexpr int kStage = kChunks / kWaves;  // chunks per thread per tensor and sub-tile
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(Fa1Cfg<D>::kThreads)
__attribute__((amdgpu_waves_per_eu(2, 2)))
void fa1_fwd_kernel(const _Float16* __restrict__ Q, const _Float16* __restrict__ K,
                    const _Float16* __restrict__ V, _Float16* __restrict__ O,
                    float* __restrict__ LSE, float* __restrict__ Ow, float* __restrict__ Mw,
                    float* __restrict__ Lw, int N, float c, uint32_t q_and, uint32_t q_xor) {
    using C = Fa1Cfg<D>;
    // sub-tile s of the key/value block: K chunk-major, V swizzled
    __shared__ __attribute__((aligned(16))) unsigned char kt_lds[C::kSub][C::kTileBytes];
    __shared__ __attribute__((aligned(16))) unsigned char vt_lds[C::kSub][C::kTileBytes];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    const int bh = blockIdx.x;

    const size_t head = size_t(bh) * size_t(N) * D;
    const uint32_t head_bytes = uint32_t(N) * C::kRowBytes;
    const auto rQ = make_rsrc(Q + head, head_bytes);
    const auto rK = make_rsrc(K + head, head_bytes);
    const auto rV = make_rsrc(V + head, head_bytes);
    const auto rO = make_rsrc(O + head, head_bytes);
    const auto rOw = make_rsrc(Ow + head, uint32_t(N) * D * 4);
    const auto rM = make_rsrc(Mw + size_t(bh) * N, uint32_t(N) * 4);
    const auto rL = make_rsrc(Lw + size_t(bh) * N, uint32_t(N) * 4);

    const int n_kt = (N + C::kBN - 1) / C::kBN;
    const int n_qt = (N + C::kBM - 1) / C::kBM;

    // Register staging of the next key/value block: thread (wave w, lane i)
    // moves chunks w + kWaves*j of row i of each 64-key sub-tile.
    u32x4 sk[C::kSub][C::kStage], sv[C::kSub][C::kStage];
    auto fetch = [&](int kt) {
#pragma unroll
        for (int s = 0; s < C::kSub; ++s) {
#pragma unroll
            for (int j = 0; j < C::kStage; ++j) {
                const int off = (kt * C::kBN + s * kBK + lane) * C::kRowBytes + (wave + C::kWaves * j) * 16;
                sk[s][j] = __builtin_amdgcn_raw_buffer_load_b128(rK, off, 0, 0);
                sv[s][j] = __builtin_amdgcn_raw_buffer_load_b128(rV, off, 0, 0);
            }
        }
    };
    auto put = [&]() {
#pragma unroll
        for (int s = 0; s < C::kSub; ++s) {
#pragma unroll
            for (int j = 0; j < C::kStage; ++j) {
                const int ch = wave + C::kWaves * j;
                *reinterpret_cast<u32x4*>(&kt_lds[s][0] + lds_k_off(ch, lane)) = sk[s][j];
                *reinterpret_cast<u32x4*>(&vt_lds[s][0] + lds_v_off(ch, lane)) = sv[s][j];
            }
        }
    };
    const int k_base = lds_k_off(hi, l32);
    const TrBase vtr(lane);

    fetch(0);
    for (int kt = 0; kt < n_kt; ++kt) {
        __syncthreads();   // every wave is done with the previous block
        put();
        __syncthreads();
        if (kt + 1 < n_kt) fetch(kt + 1);
        const int k0 = kt * C::kBN;
        // Causal: query blocks before this key block see none of its keys.
        const int qt_begin = CAUSAL ? k0 / C::kBM : 0;
        for (int qt = qt_begin; qt < n_qt; ++qt) {
            const int qw0 = qt * C::kBM + wave * kQW;
            if (qw0 >= N) continue;
            const int my_q = qw0 + l32;
            // the wave's last key block: later blocks hold only future keys
            const int kt_last = CAUSAL ? min(n_kt - 1, (qw0 + kQW - 1) / C::kBN) : n_kt - 1;
            if (kt > kt_last) continue;

            h8 qf[C::kDSteps];
#pragma unroll
            for (int ds = 0; ds < C::kDSteps; ++ds) {
                u32x4 raw = __builtin_amdgcn_raw_buffer_load_b128(rQ, my_q * C::kRowBytes + 32 * ds + 16 * hi, 0, 0);
                qf[ds] = __builtin_bit_cast(h8, (raw & q_and) ^ q_xor);
            }
            // S^T of the 128 keys: block b = 2*s + kb holds keys k0 + 32*b + 8*(r/4) + 4*hi + r%4.
            f32x16 st[2 * C::kSub];
#pragma unroll
            for (int s = 0; s < C::kSub; ++s) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    f32x16 acc = f32x16{};
#pragma unroll
                    for (int ds = 0; ds < C::kDSteps; ++ds) {
                        const h8 a = *reinterpret_cast<const h8*>(&kt_lds[s][0] + k_base + lds_k_off(2 * ds, 32 * kb));
                        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[ds], acc, 0, 0, 0);
                    }
                    st[2 * s + kb] = acc;
                }
            }
            if (k0 + C::kBN > N || (CAUSAL && k0 + C::kBN - 1 > qw0)) {
#pragma unroll
                for (int b = 0; b < 2 * C::kSub; ++b) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + 32 * b + 8 * (r >> 2) + 4 * hi + (r & 3);
                        if (key >= N || (CAUSAL && key > my_q)) st[b][r] = -INFINITY;
                    }
                }
            }
            // block statistics (scaled, base 2) and weights
            float mx = -INFINITY;
#pragma unroll
            for (int b = 0; b < 2 * C::kSub; ++b) {
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, st[b][r]);
            }
            const float mb = c * pair_max(mx);                 // m~ in log2 units
            const float shb = mb == -INFINITY ? 0.f : mb;
            float ls = 0.f;
            h8 pf[4 * C::kSub];
#pragma unroll
            for (int b = 0; b < 2 * C::kSub; ++b) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[b][r], c, -shb));
                    ls += p;
                    pf[2 * b + (r >> 3)][r & 7] = (_Float16)p;
                }
            }
            const float lb = pair_sum(ls);                     // l~
            // P~ V of the block: k-step ks covers keys 16*ks .. of the block.
            f32x16 pv[C::kDBlocks];
#pragma unroll
            for (int db = 0; db < C::kDBlocks; ++db) pv[db] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < 4 * C::kSub; ++ks) {
#pragma unroll
                for (int db = 0; db < C::kDBlocks; ++db)
                    pv[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        read_tr_operand(&vt_lds[ks / 4][0], vtr, tr_imm(ks % 4, db)), pf[ks], pv[db], 0, 0, 0);
            }
            // Merge with the stored (normalised) state of these queries.
            float m_old = -INFINITY, l_old = 0.f;
            if (kt > 0) {
                m_old = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rM, my_q * 4, 0, 0));
                l_old = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rL, my_q * 4, 0, 0));
            }
            const float m_new = __builtin_fmaxf(m_old, mb);
            const float sh = m_new == -INFINITY ? 0.f : m_new;
            const float a = l_old * __builtin_amdgcn_exp2f(m_old - sh);
            const float bw = __builtin_amdgcn_exp2f(mb - sh);
            const float l_new = a + bw * lb;
            const float inv = l_new > 0.f ? 1.0f / l_new : 0.f;
            // Lane's O elements: row my_q, columns 32*db + 8*(r/4) + 4*hi + r%4.
            const int o_off = my_q * D + 4 * hi;
            const bool last = kt == kt_last;
#pragma unroll
            for (int db = 0; db < C::kDBlocks; ++db) {
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int col = 32 * db + 8 * rr;
                    float pv4[4] = {0.f, 0.f, 0.f, 0.f};
                    if (kt > 0) {
                        const u32x4 raw = __builtin_amdgcn_raw_buffer_load_b128(rOw, (o_off + col) * 4, 0, 0);
#pragma unroll
                        for (int k = 0; k < 4; ++k) pv4[k] = __uint_as_float(raw[k]);
                    }
                    float nw[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) nw[k] = (a * pv4[k] + bw * pv[db][4 * rr + k]) * inv;
                    if (last) {
                        h4 out;
#pragma unroll
                        for (int k = 0; k < 4; ++k) out[k] = (_Float16)nw[k];
                        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, out), rO,
                                                              (o_off + col) * 2, 0, 0);
                    } else {
                        const u32x4 w = {__float_as_uint(nw[0]), __float_as_uint(nw[1]),
                                         __float_as_uint(nw[2]), __float_as_uint(nw[3])};
                        __builtin_amdgcn_raw_buffer_store_b128(w, rOw, (o_off + col) * 4, 0, 0);
                    }
                }
            }
            if (hi == 0 && my_q < N) {
                if (last) {
                    LSE[size_t(bh) * N + my_q] = (m_new + __builtin_amdgcn_logf(l_new)) * kLn2;
                } else {
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m_new), rM, my_q * 4, 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l_new), rL, my_q * 4, 0, 0);
                }
            }
        }
    }
}

template <int D, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, void* ws,
                  int BH, int N, float c, uint32_t q_and, uint32_t q_xor, hipStream_t stream) {
    using C = Fa1Cfg<D>;
    float* ow = static_cast<float*>(ws);
    float* mw = ow + size_t(BH) * N * D;
    float* lw = mw + size_t(BH) * N;
    hipLaunchKernelGGL((fa1_fwd_kernel<D, CAUSAL>), dim3(BH), dim3(C::kThreads), 0, stream,
                       static_cast<const _Float16*>(q), static_cast<const _Float16*>(k),
                       static_cast<const _Float16*>(v), static_cast<_Float16*>(o), lse, ow, mw,
                       lw, N, c, q_and, q_xor);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fa1(const void* q, const void* k, const void* v, void* o, float* lse, void* ws,
                      int BH, int N, int d, float scale, bool causal, hipStream_t stream) {
    // Scale handling as in the FA2 forward: |scale| below the smallest normal
    // float runs as 0 (Q cleared, c = 1); a negative scale flips Q's signs.
    const double a = std::fabs(static_cast<double>(scale));
    const bool zero = !(a >= 1.17549435082228751e-38);
    const float c = zero ? 1.0f : static_cast<float>(a * 1.4426950408889634);
    const uint32_t q_and = zero ? 0u : 0xffffffffu;
    const uint32_t q_xor = (!zero && scale < 0.f) ? 0x80008000u : 0u;
    if (d != 64) return hipErrorInvalidValue;
    return causal ? launch<64, true>(q, k, v, o, lse, ws, BH, N, c, q_and, q_xor, stream)
                  : launch<64, false>(q, k, v, o, lse, ws, BH, N, c, q_and, q_xor, stream);
}

}  // namespace fa2
