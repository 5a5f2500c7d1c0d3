// Backward pass of the attention forward for AMD MI355X (gfx950 / CDNA4).
//
// What is computed.  For the forward O = softmax(sigma Q K^T) V of one
// (batch, head), with causal masking when asked, and an upstream gradient
// dO, the gradients of <dO, O>:
//     P  = exp(sigma S - LSE)            S = Q K^T, LSE the forward's statistic
//     dV = P^T dO,   dP = dO V^T,   dS = P o (dP - delta),   delta_i = dO_i . O_i
//     dQ = sigma dS K,   dK = sigma dS^T Q.
// The N x N matrices S, P, dP, dS are never stored: every tile recomputes S
// and P from Q, K and the per-row LSE the forward kept ("3.6 Attention I --
// the memory problem and FlashAttention principles", 3.6.7: recompute instead
// of store, with only O(N) row statistics kept).  The formulas are the chain
// rule through the row softmax; delta_i equals sum_k P_ik dP_ik because
// O_i = sum_k P_ik V_k.
//
// Two kernels, no atomics, deterministic:
//  * dQ kernel -- grid over (query tile, batch*head) like the forward; each
//    wave owns 32 queries, holds Q^T and dO^T of them as MFMA B operands,
//    computes delta_i once (and writes it for the second kernel), then loops
//    over key tiles: S^T = K Q^T, dP^T = V dO^T, dS^T in registers,
//    dQ^T += K^T dS^T with K^T read from LDS through ds_read_b64_tr_b16.
//  * dK/dV kernel -- grid over (key tile, batch*head); each wave owns 32
//    keys, holds K^T and V^T of them, and loops over query tiles:
//    S = Q K^T, dP = dO V^T, P and dS in registers, dV^T += dO^T P and
//    dK^T += Q^T dS with Q^T and dO^T read transposed from LDS.
//  In both, an accumulator's register order is the B operand of the next
//  product (fa2_device.h), so P and dS never leave registers.
//  The dP products start their accumulation from -delta of their query rows
//  (except in the causal d = 128 kernel), so they return dP - delta and dS
//  is one multiply.
//  Tiles of 64 rows are double-buffered in LDS through registers (the next
//  tile's loads are issued before the current tile's products), one barrier
//  per tile.  Causal work stops at the diagonal; the tiles that cross it (and
//  the key tile that crosses N) are masked in a branch of their own, which
//  sets the exponent argument to -inf; causal grids take the longest tiles
//  first, a few heads at a time.  Rows past N read as zero through the per-head buffer resources,
//  which makes their contributions exactly zero, and their stores are
//  dropped.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>
#include <type_traits>

#include "fa2_device.h"
#include "fa2_launch.h"

namespace fa2 {
namespace {

using namespace dev;

template <int D>
struct BwdCfg {
    static_assert(D == 32 || D == 64 || D == 96 || D == 128, "head dim");
    static constexpr int kWaves = 4;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kRows = kWaves * kQW;         // queries (dQ) or keys (dK, dV) per workgroup
    // (D = 128 uses the software-pipelined dK/dV kernel below; measured 13-18 %
    // faster there, and slower at D = 96, where two waves share each SIMD.)
    static constexpr int kRowBytes = D * 2;
    static constexpr int kChunks = D / 8;              // 16-byte chunks per row
    static constexpr int kTileBytes = kBK * kRowBytes;
    static constexpr int kDSteps = D / 16;             // k-steps over the head dim
    static constexpr int kDBlocks = D / 32;            // 32-row blocks of a transposed accumulator
    static constexpr int kStage = kChunks / kWaves;    // staged chunks per thread per tensor and tile
    // The dK/dV kernel keeps K^T, V^T and two accumulators of D x 32 per
    // wave: at D = 128 that needs the registers of a whole SIMD.  The dQ
    // kernel fits four waves per SIMD at D = 32 (1-3 % faster than three) and
    // three at D = 64 (1-4 % faster than two; four spill there, 6 % slower).
    static constexpr int kWavesPerSimdQ = D <= 32 ? 4 : D <= 64 ? 3 : 2;
    static constexpr int kWavesPerSimdKV = D >= 128 ? 1 : D <= 32 ? 3 : 2;   // d = 32: three, 3-4 % faster
};

__device__ __forceinline__ f32x16 mfma(const h8& a, const h8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Per-lane bases of the plain A-operand reads (32 rows x 16 head-dim
// columns: row 32*blk + l32, chunk 2*ds + hi) from a swizzled tile.  The
// chunk's low bits are 2*(ds&1) + hi, so two bases cover every (ds, blk):
// the rest is the compile-time offset sw_imm(ds, blk).
struct SwBase {
    int b[2];
    __device__ __forceinline__ explicit SwBase(int lane) {
        const int l32 = lane & 31, hi = lane >> 5;
        b[0] = (hi * 64 + (l32 ^ (4 * hi))) << 4;
        b[1] = (hi * 64 + (l32 ^ (8 + 4 * hi))) << 4;
    }
};
__device__ __forceinline__ constexpr int sw_imm(int ds, int blk) { return (2 * ds * 64 + 32 * blk) << 4; }

// Stores a 32 x D transposed accumulator (rows of this lane = row `row`,
// columns 32*db + 8*(r/4) + 4*hi + r%4) as fp16 (RNE) after scaling by `mul`.
template <int D>
__device__ __forceinline__ void store_rows(__amdgpu_buffer_rsrc_t r, int row, int hi,
                                           const f32x16 (&acc)[D / 32], float mul) {
    const int base = row * D * 2 + 8 * hi;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            h4 out;
#pragma unroll
            for (int k = 0; k < 4; ++k) out[k] = (_Float16)(acc[db][4 * rr + k] * mul);
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, out), r,
                                                  base + 64 * db + 16 * rr, 0, 0);
        }
    }
}

// The same block as store_rows, restaged through a wave-private LDS region
// (used at D >= 96: +1 % at D = 96 and +5 % at D = 128 on the whole
// backward, measured in both run orders; no gain at D <= 64)
// of 32 rows x (2*D + 16) bytes and stored as 128-bit stores of whole row
// segments (64 lanes cover 1 KiB of consecutive output at D = 128) instead
// of 8 bytes in each of 32 rows per instruction.  `row0` is the first of
// the wave's 32 rows; the region must be free (the caller's barrier) and is
// free again on return.
template <int D>
__device__ __forceinline__ void store_rows_lds(__amdgpu_buffer_rsrc_t r, int row0, int lane,
                                               const f32x16 (&acc)[D / 32], float mul,
                                               unsigned char* region) {
    constexpr int kStride = 2 * D + 16;
    constexpr int kChunks = D / 8;
    const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            h4 out;
#pragma unroll
            for (int k = 0; k < 4; ++k) out[k] = (_Float16)(acc[db][4 * rr + k] * mul);
            *reinterpret_cast<h4*>(region + l32 * kStride + 64 * db + 16 * rr + 8 * hi) = out;
        }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the wave's writes are done
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < kQW * kChunks / 64; ++i) {
        const int row = (i * 64 + lane) / kChunks, ch = (i * 64 + lane) % kChunks;
        const u32x4 val = *reinterpret_cast<const u32x4*>(region + row * kStride + 16 * ch);
        __builtin_amdgcn_raw_buffer_store_b128(val, r, (row0 + row) * 2 * D + 16 * ch, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // the reads are done before the region is reused
    __builtin_amdgcn_wave_barrier();
}
template <int D>
constexpr int restage_bytes() { return 4 * kQW * (2 * D + 16); }

// ------------------------------------------------------------------ dQ
template <int D, bool CAUSAL>
__global__ __launch_bounds__(BwdCfg<D>::kThreads)
__attribute__((amdgpu_waves_per_eu(BwdCfg<D>::kWavesPerSimdQ, BwdCfg<D>::kWavesPerSimdQ)))
void fa2_bwd_dq_kernel(const _Float16* __restrict__ Q, const _Float16* __restrict__ K,
                       const _Float16* __restrict__ V, const _Float16* __restrict__ O,
                       const _Float16* __restrict__ dO, const float* __restrict__ LSE,
                       _Float16* __restrict__ dQ, float* __restrict__ Delta, int N,
                       int n_qtiles, int n_wg, float c2, float sigma, int group) {
    using C = BwdCfg<D>;
    // K tile swizzled (plain reads for S^T, transposed reads for dQ^T), V
    // tile chunk-major (plain reads for dP^T).
    // One LDS block (K tiles, then V tiles); the epilogue restages dQ in it.
    static_assert(restage_bytes<D>() <= 4 * C::kTileBytes, "restage fits");
    __shared__ __attribute__((aligned(16))) unsigned char lds[4 * C::kTileBytes];
    unsigned char* const kb0 = lds;
    unsigned char* const kb1 = lds + C::kTileBytes;
    unsigned char* const vb0 = lds + 2 * C::kTileBytes;
    unsigned char* const vb1 = lds + 3 * C::kTileBytes;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    const int logical = xcd_logical_id(blockIdx.x, n_wg);
    const HeadTile ht = head_tile_of(logical, n_qtiles, CAUSAL ? group : 1);   // causal: a few heads at a time
    const int bh = ht.bh;
    int qt = ht.rank;
    if (CAUSAL) qt = n_qtiles - 1 - qt;   // longest rows first
    const int q0 = qt * C::kRows;
    const size_t head = size_t(bh) * size_t(N) * D;
    const uint32_t head_bytes = uint32_t(N) * C::kRowBytes;
    const auto rQ = make_rsrc(Q + head, head_bytes);
    const auto rK = make_rsrc(K + head, head_bytes);
    const auto rV = make_rsrc(V + head, head_bytes);
    const auto rO = make_rsrc(O + head, head_bytes);
    const auto rdO = make_rsrc(dO + head, head_bytes);
    const auto rL = make_rsrc(LSE + size_t(bh) * N, uint32_t(N) * 4);
    const int my_q = q0 + wave * kQW + l32;

    // Q^T and dO^T fragments (B operands: lane = query my_q, dims
    // 16*ds + 8*hi + [0, 8)), and delta = dO . O of the query (the fp16
    // products are exact in fp32; the lane pair holds the two halves).
    h8 qf[C::kDSteps], dof[C::kDSteps];
    float dsum = 0.f;
#pragma unroll
    for (int ds = 0; ds < C::kDSteps; ++ds) {
        const int off = my_q * C::kRowBytes + 32 * ds + 16 * hi;
        qf[ds] = __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(rQ, off, 0, 0));
        dof[ds] = __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(rdO, off, 0, 0));
        const h8 of = __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(rO, off, 0, 0));
#pragma unroll
        for (int i = 0; i < 8; ++i) dsum = __builtin_fmaf((float)dof[ds][i], (float)of[i], dsum);
    }
    const float delta = pair_sum(dsum);
    const float lse2 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rL, my_q * 4, 0, 0)) * kLog2e;
    if (hi == 0 && my_q < N) Delta[size_t(bh) * N + my_q] = delta;
    // -delta in every element: the dP^T products accumulate onto it, so they
    // return dP - delta.  (Opaque to the compiler: kept in registers rather
    // than rebuilt from delta for every block.)
    f32x16 ndelta;
#pragma unroll
    for (int r = 0; r < 16; ++r) ndelta[r] = -delta;
    asm volatile("" : "+v"(ndelta));

    const int kv_end = CAUSAL ? min(N, q0 + C::kRows) : N;
    const int n_kt = (kv_end + kBK - 1) / kBK;
    // Tiles below n_full need no mask for any query of the workgroup.
    const int n_full = CAUSAL ? min(N / kBK, (q0 + 1) / kBK) : N / kBK;

    // Staging: thread (wave w, lane i) moves chunks w + kWaves*j of row i.
    u32x4 stk[C::kStage], stv[C::kStage];
    auto fetch = [&](int kt) {
#pragma unroll
        for (int j = 0; j < C::kStage; ++j) {
            const int off = (kt * kBK + lane) * C::kRowBytes + (wave + C::kWaves * j) * 16;
            stk[j] = __builtin_amdgcn_raw_buffer_load_b128(rK, off, 0, 0);
            stv[j] = __builtin_amdgcn_raw_buffer_load_b128(rV, off, 0, 0);
        }
    };
    auto put = [&](unsigned char* kb, unsigned char* vb) {
#pragma unroll
        for (int j = 0; j < C::kStage; ++j) {
            const int ch = wave + C::kWaves * j;
            *reinterpret_cast<u32x4*>(kb + lds_v_off(ch, lane)) = stk[j];
            *reinterpret_cast<u32x4*>(vb + lds_k_off(ch, lane)) = stv[j];
        }
    };
    const SwBase ksw(lane);
    const TrBase ktr(lane);
    const int v_base = lds_k_off(hi, l32);

    f32x16 acc[C::kDBlocks];
#pragma unroll
    for (int db = 0; db < C::kDBlocks; ++db) acc[db] = f32x16{};

    fetch(0);
    put(kb0, vb0);
    __syncthreads();
    for (int t = 0; t < n_kt; ++t) {
        const unsigned char* kb = (t & 1) ? kb1 : kb0;
        const unsigned char* vb = (t & 1) ? vb1 : vb0;
        const bool more = t + 1 < n_kt;
        if (more) fetch(t + 1);
        const bool masked = t >= n_full;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {   // 32 keys at a time
            f32x16 st = f32x16{}, dpt;   // dpt: dP^T - delta
#pragma unroll
            for (int ds = 0; ds < C::kDSteps; ++ds) {
                const h8 ak = *reinterpret_cast<const h8*>(kb + ksw.b[ds & 1] + sw_imm(ds, blk));
                st = mfma(ak, qf[ds], st);
                const h8 av = *reinterpret_cast<const h8*>(vb + v_base + lds_k_off(2 * ds, 32 * blk));
                dpt = mfma(av, dof[ds], ds == 0 ? ndelta : dpt);
            }
            // Register r of this lane: key t*64 + 32*blk + 8*(r/4) + 4*hi + r%4.
            // Exponent arguments; hidden keys (past N, or after the query
            // under the causal mask) get -inf, i.e. P = 0, in a branch of
            // their own that only the tiles crossing N or the diagonal take.
            float arg[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) arg[r] = __builtin_fmaf(st[r], c2, -lse2);
            if (masked) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = t * kBK + 32 * blk + 8 * (r >> 2) + 4 * hi + (r & 3);
                    if (key >= N || (CAUSAL && key > my_q)) arg[r] = -INFINITY;
                }
            }
            h8 dsf[2];
#pragma unroll
            for (int r = 0; r < 16; ++r)
                dsf[r >> 3][r & 7] = (_Float16)(__builtin_amdgcn_exp2f(arg[r]) * dpt[r]);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
                for (int db = 0; db < C::kDBlocks; ++db)
                    acc[db] = mfma(read_tr_operand(kb, ktr, tr_imm(2 * blk + kk, db)), dsf[kk], acc[db]);
            }
        }
        if (more) put((t & 1) ? kb0 : kb1, (t & 1) ? vb0 : vb1);
        __syncthreads();
    }
    if constexpr (D >= 96)
        store_rows_lds<D>(make_rsrc(dQ + head, head_bytes), my_q - l32, lane, acc, sigma,
                          lds + wave * kQW * (2 * D + 16));
    else
        store_rows<D>(make_rsrc(dQ + head, head_bytes), my_q, hi, acc, sigma);
}

// -------------------------------------------------------------- dK, dV
template <int D, bool CAUSAL>
__global__ __launch_bounds__(BwdCfg<D>::kThreads)
__attribute__((amdgpu_waves_per_eu(BwdCfg<D>::kWavesPerSimdKV, BwdCfg<D>::kWavesPerSimdKV)))
void fa2_bwd_dkdv_kernel(const _Float16* __restrict__ Q, const _Float16* __restrict__ K,
                         const _Float16* __restrict__ V, const _Float16* __restrict__ dO,
                         const float* __restrict__ LSE, const float* __restrict__ Delta,
                         _Float16* __restrict__ dK, _Float16* __restrict__ dV, int N,
                         int n_ktiles, int n_wg, float c2, float sigma, int group) {
    using C = BwdCfg<D>;
    // Q and dO tiles swizzled (plain reads for S and dP, transposed reads for
    // dK^T and dV^T); per-query log2-domain LSE and delta beside them.
    static_assert(restage_bytes<D>() <= 4 * C::kTileBytes, "restage fits");
    __shared__ __attribute__((aligned(16))) unsigned char lds[4 * C::kTileBytes];
    unsigned char* const qb0 = lds;
    unsigned char* const qb1 = lds + C::kTileBytes;
    unsigned char* const ob0 = lds + 2 * C::kTileBytes;
    unsigned char* const ob1 = lds + 3 * C::kTileBytes;
    __shared__ __attribute__((aligned(16))) float lb0[kBK], lb1[kBK], db0[kBK], db1[kBK];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    const int logical = xcd_logical_id(blockIdx.x, n_wg);
    const HeadTile ht = head_tile_of(logical, n_ktiles, CAUSAL ? group : 1);   // causal: tile 0 is the longest
    const int bh = ht.bh;
    const int kt = ht.rank;
    const int k0 = kt * C::kRows;
    const size_t head = size_t(bh) * size_t(N) * D;
    const uint32_t head_bytes = uint32_t(N) * C::kRowBytes;
    const auto rQ = make_rsrc(Q + head, head_bytes);
    const auto rK = make_rsrc(K + head, head_bytes);
    const auto rV = make_rsrc(V + head, head_bytes);
    const auto rdO = make_rsrc(dO + head, head_bytes);
    const auto rL = make_rsrc(LSE + size_t(bh) * N, uint32_t(N) * 4);
    const auto rD = make_rsrc(Delta + size_t(bh) * N, uint32_t(N) * 4);
    const int my_k = k0 + wave * kQW + l32;

    // K^T and V^T fragments (B operands: lane = key my_k, dims 16*ds + 8*hi + [0, 8)).
    h8 kf[C::kDSteps], vf[C::kDSteps];
#pragma unroll
    for (int ds = 0; ds < C::kDSteps; ++ds) {
        const int off = my_k * C::kRowBytes + 32 * ds + 16 * hi;
        kf[ds] = __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(rK, off, 0, 0));
        vf[ds] = __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(rV, off, 0, 0));
    }

    const int n_qt = (N + kBK - 1) / kBK;
    // Causal: queries before k0 see none of these keys; the query tiles that
    // overlap [k0, k0 + kRows) cross the diagonal and are masked.
    const int t0 = CAUSAL ? k0 / kBK : 0;
    const int t_mask_end = CAUSAL ? t0 + C::kRows / kBK : 0;

    u32x4 sq[C::kStage], so[C::kStage];
    float sl = 0.f, sd = 0.f;
    auto fetch = [&](int t) {
#pragma unroll
        for (int j = 0; j < C::kStage; ++j) {
            const int off = (t * kBK + lane) * C::kRowBytes + (wave + C::kWaves * j) * 16;
            sq[j] = __builtin_amdgcn_raw_buffer_load_b128(rQ, off, 0, 0);
            so[j] = __builtin_amdgcn_raw_buffer_load_b128(rdO, off, 0, 0);
        }
        if (wave == 0) sl = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rL, (t * kBK + lane) * 4, 0, 0)) * kLog2e;
        if (wave == 1) sd = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rD, (t * kBK + lane) * 4, 0, 0));
    };
    auto put = [&](unsigned char* qb, unsigned char* ob, float* lb, float* dbuf) {
#pragma unroll
        for (int j = 0; j < C::kStage; ++j) {
            const int ch = wave + C::kWaves * j;
            *reinterpret_cast<u32x4*>(qb + lds_v_off(ch, lane)) = sq[j];
            *reinterpret_cast<u32x4*>(ob + lds_v_off(ch, lane)) = so[j];
        }
        if (wave == 0) lb[lane] = sl;
        if (wave == 1) dbuf[lane] = -sd;   // -delta: the dP products accumulate onto it
    };
    const SwBase sw(lane);
    const TrBase tr(lane);

    f32x16 dk[C::kDBlocks], dv[C::kDBlocks];
#pragma unroll
    for (int db = 0; db < C::kDBlocks; ++db) {
        dk[db] = f32x16{};
        dv[db] = f32x16{};
    }

    fetch(t0);
    put(qb0, ob0, lb0, db0);
    __syncthreads();
    for (int t = t0; t < n_qt; ++t) {
        const bool odd = (t - t0) & 1;
        const unsigned char* qb = odd ? qb1 : qb0;
        const unsigned char* ob = odd ? ob1 : ob0;
        const float* lb = odd ? lb1 : lb0;
        const float* dlb = odd ? db1 : db0;
        const bool more = t + 1 < n_qt;
        if (more) fetch(t + 1);
        const bool masked = CAUSAL && t < t_mask_end;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {   // 32 queries at a time
            // -delta of the block's queries in the accumulator's register order.
            f32x16 nd;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 Dl = *reinterpret_cast<const float4*>(dlb + 32 * blk + 8 * g + 4 * hi);
                nd[4 * g] = Dl.x;
                nd[4 * g + 1] = Dl.y;
                nd[4 * g + 2] = Dl.z;
                nd[4 * g + 3] = Dl.w;
            }
            f32x16 s = f32x16{}, dp;   // dp: dP - delta
#pragma unroll
            for (int ds = 0; ds < C::kDSteps; ++ds) {
                const h8 aq = *reinterpret_cast<const h8*>(qb + sw.b[ds & 1] + sw_imm(ds, blk));
                s = mfma(aq, kf[ds], s);
                const h8 ao = *reinterpret_cast<const h8*>(ob + sw.b[ds & 1] + sw_imm(ds, blk));
                dp = mfma(ao, vf[ds], ds == 0 ? nd : dp);
            }
            // Register r = 4g + k of this lane: query t*64 + 32*blk + 8g + 4*hi + k.
            // Exponent arguments; under the causal mask the queries before
            // this key get -inf (P = 0) in a branch of its own that only the
            // tiles crossing the diagonal take.
            float arg[16];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 L = *reinterpret_cast<const float4*>(lb + 32 * blk + 8 * g + 4 * hi);
                const float lv[4] = {L.x, L.y, L.z, L.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) arg[4 * g + k] = __builtin_fmaf(s[4 * g + k], c2, -lv[k]);
            }
            if (masked) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (my_k > t * kBK + 32 * blk + 8 * (r >> 2) + 4 * hi + (r & 3)) arg[r] = -INFINITY;
            }
            h8 pf[2], dsf[2];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(arg[r]);
                pf[r >> 3][r & 7] = (_Float16)p;
                dsf[r >> 3][r & 7] = (_Float16)(p * dp[r]);
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
                for (int db = 0; db < C::kDBlocks; ++db) {
                    const int imm = tr_imm(2 * blk + kk, db);
                    dv[db] = mfma(read_tr_operand(ob, tr, imm), pf[kk], dv[db]);
                    dk[db] = mfma(read_tr_operand(qb, tr, imm), dsf[kk], dk[db]);
                }
            }
        }
        if (more) {
            if (odd) put(qb0, ob0, lb0, db0);
            else put(qb1, ob1, lb1, db1);
        }
        __syncthreads();
    }
    if constexpr (D >= 96) {
        unsigned char* const region = lds + wave * kQW * (2 * D + 16);
        store_rows_lds<D>(make_rsrc(dK + head, head_bytes), my_k - l32, lane, dk, sigma, region);
        store_rows_lds<D>(make_rsrc(dV + head, head_bytes), my_k - l32, lane, dv, 1.0f, region);
    } else {
        store_rows<D>(make_rsrc(dK + head, head_bytes), my_k, hi, dk, sigma);
        store_rows<D>(make_rsrc(dV + head, head_bytes), my_k, hi, dv, 1.0f);
    }
}

// ------------------------------------------------- dK, dV, software-pipelined
// At D = 128 the dK/dV kernel runs one wave per SIMD (its registers need a
// whole SIMD), so nothing hides one wave's VALU work behind another wave's
// MFMAs.  This variant pipelines it inside the wave, over 32-query blocks j:
// step j issues the dV/dK products of block j-1 and the S/dP products of
// block j+1 (independent of block j's softmax) slot by slot, with the P / dS
// arithmetic of block j spread between them.  S, dP, P and dS are
// double-buffered by block parity.  Query tiles (64 rows = 2 blocks) rotate
// through three LDS buffers: the tile read by block j-1's products is free
// after even step 2i, tile i+2 is stored during odd step 2i+1 and read from
// step 2i+3 on, so one barrier after every even step covers both hazards.
constexpr int kRing = 5;   // LDS operand reads run kRing - 1 products ahead

template <int D>
struct KvStream {
    using B = BwdCfg<D>;
    static constexpr int kPV = 4 * B::kDBlocks;   // dV and dK products of a block
    static constexpr int kQK = 2 * B::kDSteps;    // S and dP products of a block
    static constexpr int kSlots = kPV + kQK;
    static constexpr int kTile = kBK * B::kRowBytes;
    // Element pairs (2 of the 16 per lane) enter the three-stage VALU chain
    // (argument, exp2, dS and fp16 packing) in slots [0, kSlots - 2).
    static constexpr int pair_begin(int q) { return (q * (kSlots - 2)) / 8; }
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(BwdCfg<D>::kThreads)
__attribute__((amdgpu_waves_per_eu(1, 1)))
void fa2_bwd_dkdv_stream_kernel(const _Float16* __restrict__ Q, const _Float16* __restrict__ K,
                                const _Float16* __restrict__ V, const _Float16* __restrict__ dO,
                                const float* __restrict__ LSE, const float* __restrict__ Delta,
                                _Float16* __restrict__ dK, _Float16* __restrict__ dV, int N,
                                int n_ktiles, int n_wg, float c2, float sigma, int group) {
    using C = BwdCfg<D>;
    using S = KvStream<D>;
    __shared__ __attribute__((aligned(16))) unsigned char qbuf[3][S::kTile];
    __shared__ __attribute__((aligned(16))) unsigned char obuf[3][S::kTile];
    __shared__ __attribute__((aligned(16))) float lbuf[3][kBK], dbuf[3][kBK];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    const int logical = xcd_logical_id(blockIdx.x, n_wg);
    const HeadTile ht = head_tile_of(logical, n_ktiles, CAUSAL ? group : 1);   // causal: tile 0 is the longest
    const int bh = ht.bh;
    const int kt = ht.rank;
    const int k0 = kt * C::kRows;
    const size_t head = size_t(bh) * size_t(N) * D;
    const uint32_t head_bytes = uint32_t(N) * C::kRowBytes;
    const auto rQ = make_rsrc(Q + head, head_bytes);
    const auto rK = make_rsrc(K + head, head_bytes);
    const auto rV = make_rsrc(V + head, head_bytes);
    const auto rdO = make_rsrc(dO + head, head_bytes);
    const auto rL = make_rsrc(LSE + size_t(bh) * N, uint32_t(N) * 4);
    const auto rD = make_rsrc(Delta + size_t(bh) * N, uint32_t(N) * 4);
    const int kw0 = k0 + wave * kQW;       // first key of this wave
    const int my_k = kw0 + l32;

    h8 kf[C::kDSteps], vf[C::kDSteps];
#pragma unroll
    for (int ds = 0; ds < C::kDSteps; ++ds) {
        const int off = my_k * C::kRowBytes + 32 * ds + 16 * hi;
        kf[ds] = __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(rK, off, 0, 0));
        vf[ds] = __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(rV, off, 0, 0));
    }

    const int n_qt = (N + kBK - 1) / kBK;
    const int t0 = CAUSAL ? k0 / kBK : 0;        // first query tile that sees these keys
    const int nb = 2 * (n_qt - t0);              // 32-query blocks to walk

    // Staging of query tile t: chunks wave + kWaves*j of row `lane`, plus the
    // row's log2-domain LSE (wave 0) and delta (wave 1).
    u32x4 sq[C::kStage], so[C::kStage];
    float sl = 0.f, sd = 0.f;
    auto fetch = [&](int t) {
#pragma unroll
        for (int j = 0; j < C::kStage; ++j) {
            const int off = (t * kBK + lane) * C::kRowBytes + (wave + C::kWaves * j) * 16;
            sq[j] = __builtin_amdgcn_raw_buffer_load_b128(rQ, off, 0, 0);
            so[j] = __builtin_amdgcn_raw_buffer_load_b128(rdO, off, 0, 0);
        }
        if (wave == 0) sl = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rL, (t * kBK + lane) * 4, 0, 0)) * kLog2e;
        if (wave == 1) sd = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rD, (t * kBK + lane) * 4, 0, 0));
    };
    auto put = [&](int b) {
#pragma unroll
        for (int j = 0; j < C::kStage; ++j) {
            const int ch = wave + C::kWaves * j;
            *reinterpret_cast<u32x4*>(&qbuf[b][0] + lds_v_off(ch, lane)) = sq[j];
            *reinterpret_cast<u32x4*>(&obuf[b][0] + lds_v_off(ch, lane)) = so[j];
        }
        if (wave == 0) lbuf[b][lane] = sl;
        // Non-causal: -delta, onto which the dP products accumulate (measured
        // 2.5-5 % faster there; 3 % slower causal, which subtracts delta).
        if (wave == 1) dbuf[b][lane] = CAUSAL ? sd : -sd;
    };
    const SwBase sw(lane);
    const TrBase tr(lane);

    f32x16 dk[C::kDBlocks], dv[C::kDBlocks];
#pragma unroll
    for (int db = 0; db < C::kDBlocks; ++db) {
        dk[db] = f32x16{};
        dv[db] = f32x16{};
    }
    f32x16 s_[2], dp_[2];       // S and dP of the blocks of parity 0 / 1
    h8 pf[2][2], dsf[2][2];     // fp16 P and dS of the blocks of parity 0 / 1
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        pf[i][0] = pf[i][1] = dsf[i][0] = dsf[i][1] = h8{};
    }

    // Prologue: tiles t0 and t0+1 to LDS buffers 0 and 1; S and dP of block 0.
    fetch(t0);
    put(0);
    fetch(t0 + 1);
    put(1);
    __syncthreads();
    // -delta of the 16 query rows of block b's half of LDS buffer `buf`, in
    // the accumulator's register order (register 4g + k: row 32*half + 8g + 4*hi + k).
    auto neg_delta = [&](int buf, int half) {
        f32x16 nd;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4 Dv = *reinterpret_cast<const float4*>(&dbuf[buf][0] + 32 * half + 8 * g + 4 * hi);
            nd[4 * g] = Dv.x;
            nd[4 * g + 1] = Dv.y;
            nd[4 * g + 2] = Dv.z;
            nd[4 * g + 3] = Dv.w;
        }
        return nd;
    };
    {
        f32x16 a = f32x16{}, b = CAUSAL ? f32x16{} : neg_delta(0, 0);   // non-causal b: dP - delta
#pragma unroll
        for (int ds = 0; ds < C::kDSteps; ++ds) {
            a = mfma(*reinterpret_cast<const h8*>(&qbuf[0][0] + sw.b[ds & 1] + sw_imm(ds, 0)), kf[ds], a);
            b = mfma(*reinterpret_cast<const h8*>(&obuf[0][0] + sw.b[ds & 1] + sw_imm(ds, 0)), vf[ds], b);
        }
        s_[0] = a;
        dp_[0] = b;
    }

    // Step j (PAR = j & 1): products of block j-1 (dV, dK) and j+1 (S, dP),
    // softmax-side arithmetic of block j.
    auto step = [&](auto par_tag, int j) {
        constexpr int PAR = decltype(par_tag)::value;
        const int ti = j >> 1;                          // tile of block j, relative to t0
        // block j-1's tile; for j = 0 (no such block, P = dS = 0) tile 0,
        // whose contents are finite
        const int prev_buf = (j > 0 ? (j - 1) >> 1 : 0) % 3;
        const unsigned char* qb_prev = &qbuf[prev_buf][0];
        const unsigned char* ob_prev = &obuf[prev_buf][0];
        const unsigned char* qb_next = &qbuf[((j + 1) >> 1) % 3][0];
        const unsigned char* ob_next = &obuf[((j + 1) >> 1) % 3][0];
        const float* lb = &lbuf[ti % 3][0];
        constexpr int PREV = 1 - PAR;                  // parity of blocks j-1 and j+1
        // Non-causal: the dP products of block j+1 accumulate onto -delta of its rows.
        const f32x16 nd_next = CAUSAL ? f32x16{} : neg_delta(((j + 1) >> 1) % 3, PREV);
        // Row statistics of block j's 16 query rows of this lane (register r =
        // 4g + k: row 32*PAR + 8g + 4*hi + k of the tile).
        float Lr[16], Dr[16];   // Dr: delta (causal only)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4 L = *reinterpret_cast<const float4*>(lb + 32 * PAR + 8 * g + 4 * hi);
            Lr[4 * g] = L.x; Lr[4 * g + 1] = L.y; Lr[4 * g + 2] = L.z; Lr[4 * g + 3] = L.w;
            if (CAUSAL) {
                const float4 Dv = *reinterpret_cast<const float4*>(&dbuf[ti % 3][0] + 32 * PAR + 8 * g + 4 * hi);
                Dr[4 * g] = Dv.x; Dr[4 * g + 1] = Dv.y; Dr[4 * g + 2] = Dv.z; Dr[4 * g + 3] = Dv.w;
            }
        }
        const int q0 = (t0 + ti) * kBK + 32 * PAR;     // first query of block j
        const bool masked = CAUSAL && q0 < kw0 + kQW - 1;
        // j = 0 has no block j-1: its products run on P = dS = 0 (pf / dsf of
        // parity 1 start zeroed and are first written by block 1).

        h8 ring[kRing];
        auto read = [&](int p) {
            if (p < S::kPV) {
                const int kk = p / (2 * C::kDBlocks), rem = p % (2 * C::kDBlocks);
                const int db = rem >> 1, which = rem & 1;
                const int imm = tr_imm(2 * PREV + kk, db);
                ring[p % kRing] = read_tr_operand(which ? qb_prev : ob_prev, tr, imm);
            } else {
                const int a = p - S::kPV, ds = a >> 1, which = a & 1;
                ring[p % kRing] = *reinterpret_cast<const h8*>((which ? ob_next : qb_next) + sw.b[ds & 1] + sw_imm(ds, PREV));
            }
        };
        auto job = [&](int p) {
            const h8 a = ring[p % kRing];
            if (p < S::kPV) {
                const int kk = p / (2 * C::kDBlocks), rem = p % (2 * C::kDBlocks);
                const int db = rem >> 1, which = rem & 1;
                if (which) dk[db] = mfma(a, dsf[PREV][kk], dk[db]);
                else dv[db] = mfma(a, pf[PREV][kk], dv[db]);
            } else {
                const int q = p - S::kPV, ds = q >> 1, which = q & 1;
                if (which) dp_[PREV] = mfma(a, vf[ds], ds == 0 ? nd_next : dp_[PREV]);
                else s_[PREV] = mfma(a, kf[ds], ds == 0 ? f32x16{} : s_[PREV]);
            }
        };
        float arg[16], pe[16];
        auto pb = [&](int p) {    // first pair entering at slot p or later
            int q = 0;
            while (q < 8 && S::pair_begin(q) < p) ++q;
            return q;
        };
        auto valu = [&](int p) {
            // stage 3: dS, fp16 P and dS of the pairs that entered two slots ago
#pragma unroll
            for (int q = pb(p - 2); q < pb(p - 1); ++q) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int r = 2 * q + h;
                    const float d_ = CAUSAL ? pe[r] * (dp_[PAR][r] - Dr[r]) : pe[r] * dp_[PAR][r];
                    pf[PAR][r >> 3][r & 7] = (_Float16)pe[r];
                    dsf[PAR][r >> 3][r & 7] = (_Float16)d_;
                }
                pin(pf[PAR][q >> 2]);
                pin(dsf[PAR][q >> 2]);
            }
            // stage 2: exp2, causal mask
#pragma unroll
            for (int q = pb(p - 1); q < pb(p); ++q) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int r = 2 * q + h;
                    float e = __builtin_amdgcn_exp2f(arg[r]);
                    if (masked && my_k > q0 + 8 * (r >> 2) + 4 * hi + (r & 3)) e = 0.f;
                    pe[r] = e;
                    pin(pe[r]);
                }
            }
            // stage 1: scaled score minus the row's log2-domain LSE
#pragma unroll
            for (int q = pb(p); q < pb(p + 1); ++q) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int r = 2 * q + h;
                    arg[r] = __builtin_fmaf(s_[PAR][r], c2, -Lr[r]);
                    pin(arg[r]);
                }
            }
        };
        // Staging: an even step fetches tile ti+2 into registers (free since
        // the previous odd step stored theirs); the next, odd step stores it
        // into buffer (ti+2) % 3, whose old tile ti-1 was last read before the
        // barrier that ends the even step.
        if (PAR == 0) fetch(t0 + ti + 2);
#pragma unroll
        for (int p = 0; p < kRing - 1; ++p) read(p);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int p = 0; p < S::kSlots; ++p) {
            if (p + kRing - 1 < S::kSlots) read(p + kRing - 1);
            job(p);
            __builtin_amdgcn_sched_barrier(0);
            valu(p);
            if (PAR == 1 && p == S::kSlots / 2) put((ti + 2) % 3);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (PAR == 0) __syncthreads();
    };

    int j = 0;
    for (; j + 1 < nb; j += 2) {
        step(std::integral_constant<int, 0>{}, j);
        step(std::integral_constant<int, 1>{}, j + 1);
    }
    // nb is even: every block has been softmax'd; block nb-1 still owes its
    // dV / dK products.
    {
        const unsigned char* qb_prev = &qbuf[((nb - 1) >> 1) % 3][0];
        const unsigned char* ob_prev = &obuf[((nb - 1) >> 1) % 3][0];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int db = 0; db < C::kDBlocks; ++db) {
                const int imm = tr_imm(2 + kk, db);
                dv[db] = mfma(read_tr_operand(ob_prev, tr, imm), pf[1][kk], dv[db]);
                dk[db] = mfma(read_tr_operand(qb_prev, tr, imm), dsf[1][kk], dk[db]);
            }
        }
    }
    static_assert(restage_bytes<D>() <= 3 * S::kTile, "restage fits");
    __syncthreads();   // every wave is done with the query tiles
    unsigned char* const region = &qbuf[0][0] + wave * kQW * (2 * D + 16);
    store_rows_lds<D>(make_rsrc(dK + head, head_bytes), my_k - l32, lane, dk, sigma, region);
    store_rows_lds<D>(make_rsrc(dV + head, head_bytes), my_k - l32, lane, dv, 1.0f, region);
}

template <int D, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  const void* dout, void* dq, void* dk, void* dv, float* delta, int BH, int N,
                  float c2, float sigma, hipStream_t stream) {
    using C = BwdCfg<D>;
    const int n_tiles = (N + C::kRows - 1) / C::kRows;
    const int n_wg = n_tiles * BH;
    const auto* Q = static_cast<const _Float16*>(q);
    const auto* K = static_cast<const _Float16*>(k);
    const auto* V = static_cast<const _Float16*>(v);
    const auto* dO = static_cast<const _Float16*>(dout);
    // Causal grids: tiles of a few heads at a time, longest first (one
    // workgroup per SIMD-worth of waves: C::kWaves is 4).
    const int group_q = CAUSAL ? causal_group(n_tiles, n_wg, C::kWavesPerSimdQ) : 1;
    const int group_kv = CAUSAL ? causal_group(n_tiles, n_wg, C::kWavesPerSimdKV) : 1;
    hipLaunchKernelGGL((fa2_bwd_dq_kernel<D, CAUSAL>), dim3(n_wg), dim3(C::kThreads), 0, stream, Q,
                       K, V, static_cast<const _Float16*>(o), dO, lse, static_cast<_Float16*>(dq),
                       delta, N, n_tiles, n_wg, c2, sigma, group_q);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if constexpr (D == 128) {
        hipLaunchKernelGGL((fa2_bwd_dkdv_stream_kernel<D, CAUSAL>), dim3(n_wg), dim3(C::kThreads), 0,
                           stream, Q, K, V, dO, lse, static_cast<const float*>(delta),
                           static_cast<_Float16*>(dk), static_cast<_Float16*>(dv), N, n_tiles, n_wg,
                           c2, sigma, group_kv);
    } else {
        hipLaunchKernelGGL((fa2_bwd_dkdv_kernel<D, CAUSAL>), dim3(n_wg), dim3(C::kThreads), 0, stream,
                           Q, K, V, dO, lse, static_cast<const float*>(delta),
                           static_cast<_Float16*>(dk), static_cast<_Float16*>(dv), N, n_tiles, n_wg,
                           c2, sigma, group_kv);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv,
                      float* delta, int BH, int N, int d, float scale, bool causal,
                      hipStream_t stream) {
    // As in the forward, a |scale| below the smallest normal float is run as
    // scale 0 (uniform weights over the visible keys, zero dQ and dK).
    const double a = std::fabs(static_cast<double>(scale));
    const float sigma = a >= 1.17549435082228751e-38 ? scale : 0.0f;
    const float c2 = static_cast<float>(static_cast<double>(sigma) * 1.4426950408889634);
#define FA2_BWD_CASE(DD)                                                                        \
    case DD:                                                                                    \
        return causal ? launch<DD, true>(q, k, v, o, lse, dout, dq, dk, dv, delta, BH, N, c2,   \
                                         sigma, stream)                                         \
                      : launch<DD, false>(q, k, v, o, lse, dout, dq, dk, dv, delta, BH, N, c2,  \
                                          sigma, stream);
    switch (d) {
        FA2_BWD_CASE(32)
        FA2_BWD_CASE(64)
        FA2_BWD_CASE(96)
        FA2_BWD_CASE(128)
        default:
            return hipErrorInvalidValue;
    }
#undef FA2_BWD_CASE
}

}  // namespace fa2
