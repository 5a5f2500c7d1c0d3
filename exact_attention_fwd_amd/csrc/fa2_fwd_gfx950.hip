// FlashAttention-2 forward pass for AMD MI355X (gfx950 / CDNA4).
//
// What is computed ("3.6 Attention I -- the memory problem and FlashAttention
// principles", 3.6.4 and the tile loop of 3.6.6): for each query row the
// online-softmax state (running max m, running sum l, unnormalised output
// acc) is carried across key/value tiles; each tile updates
//     m_new = max(m, rowmax(S)),  alpha = exp(m - m_new),
//     P = exp(S - m_new),  l = alpha*l + rowsum(P),  acc = alpha*acc + P V,
// and the output is normalised once, O = acc / l, with LSE = m + ln l
// (3.6.7).  Causal attention skips key tiles entirely in the future and masks
// only the tiles that cross the diagonal (3.6.6).
//
// How it maps onto gfx950.  The CuTe write-up ("FlashAttention-2 from scratch
// in CuTe") describes an A100 design; the lessons kept from it are the grid
// over (Q tile, batch*head) with the Q tile resident, a one-tile-ahead K/V
// prefetch, 128-bit loads, bank-spread shared tiles and row-owning warps.
//
//  * One workgroup = 4 waves = 128 queries of one (batch, head).  Each wave
//    owns 32 whole query rows, so every row reduction stays inside the wave.
//  * The score tile is computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_f16 (A = 32 keys x 16 dims from LDS, B = Q^T held in
//    registers for the whole loop).  In the 32x32 accumulator a lane then
//    holds one query (column) and 16 of the 32 keys; the other 16 sit in lane
//    l^32.  Row max = 16 in-lane values + one v_permlane32_swap; the row sum
//    needs no cross-lane step until the epilogue.
//  * Exponentials are taken in base 2 with the scale folded in:
//    P = exp2(S*c - m2), c = |scale|*log2(e), m2 = c*max(S).
//  * The accumulator's register order is reused as the B operand of the PV
//    MFMA (O^T = V^T P^T), so P never leaves registers; V^T comes from LDS
//    through ds_read_b64_tr_b16, which returns four consecutive keys of one
//    head-dim column per lane.
//  * The key loop has a fast path and a general path.  The fast loop runs
//    unmasked tiles whose scaled row max stays within kLazy (log2 units) of
//    a lazily updated reference max m2: their weights exp2(S*c - m2) are at
//    most 2^kLazy, so acc and l need no rescale and no mask.  Everything
//    else (first tile, diagonal and tail tiles, a tile whose max outgrows
//    m2 + kLazy) takes the general path, which sets m2 to the running max as
//    in the recurrence and rescales acc and l by alpha = exp2(m2_old -
//    m2_new).  The softmax is the same: a row's common shift cancels.
//  * In the fast loop P and P V are software-pipelined over the 4 k-steps
//    of 16 keys: the MFMAs of one step overlap the LDS reads and the
//    exponentials of the next.
//  * K and V tiles (64 keys) are double-buffered in LDS.  The next tile's K
//    is fetched (128-bit buffer loads) before this tile's QK^T and written to
//    LDS after it; the next V is fetched then and written after this tile's
//    PV.  One barrier per tile.
//  * All global accesses are buffer instructions on a per-head resource
//    whose size is the head's N*d*2 bytes: rows past N read as zero and
//    stores past N are dropped by the hardware, so the tail needs no branch.
//  * Workgroup ids are remapped so that all Q tiles of one head run on the
//    same XCD (dispatch is round-robin over the 8 XCDs) and share its L2;
//    causal grids start with the longest rows.
//  * Occupancy: 3 waves per SIMD at d = 64, 2 at d = 128 (register bound).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>
#include <type_traits>

#include "fa2_launch.h"

namespace fa2 {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef __fp16 tr4 __attribute__((vector_size(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kQW = 32;             // query rows per wave
constexpr int kBQ = kWaves * kQW;   // query rows per workgroup
constexpr int kBK = 64;             // keys per K/V tile
constexpr float kLn2 = 0.69314718055994530942f;
// Largest growth of a row's scaled max (log2 units) the fast loop absorbs
// without rescaling: its fp16 weights stay <= 2^8.
constexpr float kLazy = 8.0f;
constexpr int kRsrcFlags = 0x00020000;   // raw buffer, 32-bit data format

template <int D>
struct Cfg {
    static constexpr int kRowBytes = D * 2;
    static constexpr int kChunks = D / 8;                     // 16-byte chunks per row
    static constexpr int kTileBytes = kBK * kRowBytes;
    static constexpr int kLoads = kBK * kChunks / kThreads;   // 16-byte loads per thread per tile
    static constexpr int kDSteps = D / 16;                    // k-steps of the S^T MFMA
    static constexpr int kDBlocks = D / 32;                   // 32-row blocks of O^T
    static constexpr int kLdsBytes = 4 * kTileBytes;          // {K, V} x 2 buffers
};

// LDS tile layouts, both in 16-byte chunks (8 fp16 of one row):
//  K: chunk-major, chunk c of key row r at (c * 64 + r) * 16.  A
//     ds_read_b128 quarter-wave reads one chunk of 16 consecutive keys,
//     256 contiguous bytes: every bank once.
//  V: chunk-major with an XOR swizzle of the row, chunk c of row r at
//     (c * 64 + (r ^ 4 * (c & 3))) * 16.  A ds_read_b64_tr_b16 half-wave
//     reads 4 rows x 4 chunks; the XOR moves the 4 chunk planes (1 KiB
//     apart, so on the same banks) onto 4 different 64-byte bank windows.
// Both keep every per-lane address a lane base plus a compile-time offset.
__device__ __forceinline__ int lds_k_off(int ch, int row) { return (ch * 64 + row) << 4; }
__device__ __forceinline__ int lds_v_off(int ch, int row) {
    return (ch * 64 + (row ^ ((ch & 3) << 2))) << 4;
}

__device__ __forceinline__ float pair_max(float x) {
    // v_permlane32_swap of x with itself: each lane sees its own value and
    // that of lane l^32 in the two results.
    auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

__device__ __forceinline__ h4 lds_read_tr(const unsigned char* p) {
    tr4 r = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
        (__attribute__((address_space(3))) tr4*)(p));
    return __builtin_bit_cast(h4, r);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcFlags);
}

// Occupancy: d = 64 fits 3 waves per SIMD (<= 168 VGPRs), d = 128 needs
// the 256 VGPRs of 2 waves per SIMD.
template <int D>
constexpr int kWavesPerEU = D == 64 ? 3 : 2;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(kWavesPerEU<D>, kWavesPerEU<D>)))
void fa2_fwd_kernel(const _Float16* __restrict__ Q, const _Float16* __restrict__ K,
                    const _Float16* __restrict__ V, _Float16* __restrict__ O,
                    float* __restrict__ LSE, int N, int n_qtiles, int n_wg, float c,
                    uint32_t q_sign) {
    using C = Cfg<D>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    // Workgroup -> (batch*head, Q tile).  Consecutive logical ids (the Q
    // tiles of one head) are placed on one XCD.
    const int wg = blockIdx.x;
    // readfirstlane keeps these (uniform) values in SGPRs, so the buffer
    // resources built from them are scalar.
    const int logical = (n_wg & 7) == 0 ? (wg & 7) * (n_wg >> 3) + (wg >> 3) : wg;
    const int bh = __builtin_amdgcn_readfirstlane(logical / n_qtiles);
    int qt = __builtin_amdgcn_readfirstlane(logical - bh * n_qtiles);
    if (CAUSAL) qt = n_qtiles - 1 - qt;
    const int q0 = qt * kBQ;
    const size_t head = size_t(bh) * size_t(N) * D;
    const uint32_t head_bytes = uint32_t(N) * C::kRowBytes;
    const auto rQ = make_rsrc(Q + head, head_bytes);
    const auto rK = make_rsrc(K + head, head_bytes);
    const auto rV = make_rsrc(V + head, head_bytes);

    const int qw0 = q0 + wave * kQW;   // first query of this wave
    const int my_q = qw0 + l32;        // the query this lane owns

    // Q^T operand: lane holds query my_q, dims 16*ds + 8*hi + [0, 8); rows
    // past N load as zero.
    h8 qf[C::kDSteps];
#pragma unroll
    for (int ds = 0; ds < C::kDSteps; ++ds) {
        u32x4 raw = __builtin_amdgcn_raw_buffer_load_b128(rQ, my_q * C::kRowBytes + 32 * ds + 16 * hi, 0, 0);
        raw ^= q_sign;   // scale < 0: softmax(s*S) = softmax(|s|*(-Q)K^T)
        qf[ds] = __builtin_bit_cast(h8, raw);
    }

    const int kv_end = CAUSAL ? min(N, q0 + kBQ) : N;
    const int n_kt = (kv_end + kBK - 1) / kBK;

    // Staging registers for one tensor (K or V) of the next tile: the next
    // K is fetched before this tile's QK^T and written to LDS after it; the
    // next V is fetched then and written after this tile's PV.
    // Wave w, instruction i moves rows 16*w + [0, 16) x chunks 4*i + [0, 4):
    // lane -> row 16*w + lane%16, chunk 4*i + lane/16.  Each row gives 64
    // contiguous bytes from memory; each quarter-wave writes 256 contiguous
    // LDS bytes.  Only the chunk depends on i, and (chunk & 3) does not, so
    // each address is one lane base plus a compile-time offset.
    u32x4 stage[C::kLoads];
    const int st_row = wave * 16 + (lane & 15);
    const int st_ch = lane >> 4;
    const int g_base = st_row * C::kRowBytes + st_ch * 16;
    const int k_st = lds_k_off(st_ch, st_row);
    const int v_st = lds_v_off(st_ch, st_row);
    static_assert(kWaves * 16 == kBK, "one 16-row band per wave");
    auto load_rows = [&](__amdgpu_buffer_rsrc_t rsrc, int kt) {
        const int voff = g_base + kt * C::kTileBytes;
#pragma unroll
        for (int i = 0; i < C::kLoads; ++i)
            stage[i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff + 64 * i, 0, 0);
    };
    auto store_rows = [&](unsigned char* dst, int lds_base) {
#pragma unroll
        for (int i = 0; i < C::kLoads; ++i)
            *reinterpret_cast<u32x4*>(dst + lds_base + (i << 12)) = stage[i];
    };
    auto kbuf_of = [&](int buf) { return smem + buf * 2 * C::kTileBytes; };
    auto vbuf_of = [&](int buf) { return smem + buf * 2 * C::kTileBytes + C::kTileBytes; };

    f32x16 oacc[C::kDBlocks];
#pragma unroll
    for (int db = 0; db < C::kDBlocks; ++db) oacc[db] = f32x16{};
    float m2 = -INFINITY;   // reference max of c*S for this query (log2 units)
    float lsum = 0.f;       // this lane's share of the running sum

    // Per-lane LDS read bases; the unrolled loops add compile-time offsets.
    // K (A operand of S^T): key 32*kb + l32, chunk 2*ds + hi.
    const int k_base = lds_k_off(hi, l32);
    // V^T (A operand of O^T) via ds_read_b64_tr_b16: lane = 16*g + 4*e + cc
    // reads keys 16*ks + 8*ab + 4*hi + e, columns 32*db + 16*(g&1) + 4*cc.
    // Chunk 4*db + tr_ch has (chunk & 3) == tr_ch, so the swizzle stays in
    // the base.
    const int tr_g = lane >> 4, tr_e = (lane >> 2) & 3, tr_c = lane & 3;
    const int tr_ch = 2 * (tr_g & 1) + (tr_c >> 1);
    const int v_base0 = lds_v_off(tr_ch, 4 * hi + tr_e) + (tr_c & 1) * 8;
    const int v_base1 = lds_v_off(tr_ch, 8 + 4 * hi + tr_e) + (tr_c & 1) * 8;

    // S^T = K Q^T for 64 keys x 32 queries: two 32x32 accumulators.
    auto qk_tile = [&](int buf, f32x16 (&s)[2]) {
        __builtin_amdgcn_s_setprio(1);
        const unsigned char* kbuf = kbuf_of(buf);
        s[0] = f32x16{};
        s[1] = f32x16{};
#pragma unroll
        for (int ds = 0; ds < C::kDSteps; ++ds) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const h8 a = *reinterpret_cast<const h8*>(kbuf + k_base + lds_k_off(2 * ds, 32 * kb));
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[ds], s[kb], 0, 0, 0);
            }
        }
        __builtin_amdgcn_s_setprio(0);
    };

    // Keys beyond N, and on diagonal tiles keys after the query, get -inf.
    // Register r of accumulator kb holds key k0 + 4*hi + off(kb, r) with a
    // compile-time off, so each test is one per-lane base against a constant.
    auto mask_tile = [&](int k0, f32x16 (&s)[2]) {
        const int past_end = k0 + 4 * hi - N;      // key >= N  <=>  past_end + off >= 0
        const int after_q = k0 + 4 * hi - my_q;    // key > q   <=>  after_q + off > 0
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
                const bool hidden = past_end >= -off || (CAUSAL && after_q > -off);
                if (hidden) s[kb][r] = -INFINITY;
            }
        }
    };

    // Row max of the tile's 64 scores of this lane's query: 32 in-lane values
    // as a shallow v_max3 tree, then one swap with lane l^32.
    auto tile_max = [&](const f32x16 (&s)[2]) {
        float t[11];
#pragma unroll
        for (int i = 0; i < 10; ++i) {
            const int r0 = 3 * i;
            t[i] = __builtin_fmaxf(__builtin_fmaxf(s[r0 >> 4][r0 & 15], s[(r0 + 1) >> 4][(r0 + 1) & 15]),
                                   s[(r0 + 2) >> 4][(r0 + 2) & 15]);
        }
        t[10] = __builtin_fmaxf(s[1][14], s[1][15]);
        const float u0 = __builtin_fmaxf(__builtin_fmaxf(t[0], t[1]), t[2]);
        const float u1 = __builtin_fmaxf(__builtin_fmaxf(t[3], t[4]), t[5]);
        const float u2 = __builtin_fmaxf(__builtin_fmaxf(t[6], t[7]), t[8]);
        const float u3 = __builtin_fmaxf(t[9], t[10]);
        return pair_max(__builtin_fmaxf(__builtin_fmaxf(u0, u1), __builtin_fmaxf(u2, u3)));
    };

    // P = exp2(c*S - shift) rounded to fp16 (RNE) as the B operands of the
    // PV MFMA; returns this lane's share of the row sum of the fp32 weights
    // (4 independent add chains).  Summing the fp16-rounded weights instead
    // would put up to 2^-12 relative error per term into l, which short
    // (causal) rows pass straight on to the LSE.
    auto exp_tile = [&](auto mask_tag, const f32x16 (&s)[2], float shift, h8 (&pf)[4]) {
        constexpr bool MASK = decltype(mask_tag)::value;
        float rsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float x = s[kb][r];
                float p = __builtin_amdgcn_exp2f(__builtin_fmaf(x, c, -shift));
                if constexpr (MASK) p = (x == -INFINITY) ? 0.f : p;
                rsum[r & 3] += p;
                pf[2 * kb + (r >> 3)][r & 7] = (_Float16)p;
            }
        }
        return (rsum[0] + rsum[1]) + (rsum[2] + rsum[3]);
    };

    // O^T += V^T P^T: 4 k-steps of 16 keys, D/32 row blocks.
    auto pv_tile = [&](int buf, const h8 (&pf)[4]) {
        const unsigned char* vbuf = vbuf_of(buf);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int db = 0; db < C::kDBlocks; ++db) {
                const int imm = ((4 * db) * 64 + 16 * ks) << 4;
                const h4 ta = lds_read_tr(vbuf + v_base0 + imm);
                const h4 tb = lds_read_tr(vbuf + v_base1 + imm);
                const h8 a = __builtin_shufflevector(ta, tb, 0, 1, 2, 3, 4, 5, 6, 7);
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[ks], oacc[db], 0, 0, 0);
            }
        }
        __builtin_amdgcn_s_setprio(0);
    };

    // Fast-loop P and P V, software-pipelined over the 4 k-steps of 16
    // keys: while the MFMAs of step ks run, the V^T operands of step ks+1
    // are read from LDS and its 8 weights per lane are exponentiated.
    auto exp_pv_pipelined = [&](int buf, const f32x16 (&s)[2], float shift) {
        const unsigned char* vbuf = vbuf_of(buf);
        float rsum[4] = {0.f, 0.f, 0.f, 0.f};
        auto exp_step = [&](int ks, h8& pk) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float x = s[ks >> 1][8 * (ks & 1) + j];
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(x, c, -shift));
                rsum[j & 3] += p;
                pk[j] = (_Float16)p;
            }
        };
        auto read_step = [&](int ks, h8 (&va)[C::kDBlocks]) {
#pragma unroll
            for (int db = 0; db < C::kDBlocks; ++db) {
                const int imm = ((4 * db) * 64 + 16 * ks) << 4;
                const h4 ta = lds_read_tr(vbuf + v_base0 + imm);
                const h4 tb = lds_read_tr(vbuf + v_base1 + imm);
                va[db] = __builtin_shufflevector(ta, tb, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        };
        h8 va[2][C::kDBlocks];
        h8 pk[2];
        read_step(0, va[0]);
        exp_step(0, pk[0]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks + 1 < 4) read_step(ks + 1, va[(ks + 1) & 1]);
#pragma unroll
            for (int db = 0; db < C::kDBlocks; ++db)
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[ks & 1][db], pk[ks & 1], oacc[db], 0, 0, 0);
            if (ks + 1 < 4) exp_step(ks + 1, pk[(ks + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
        }
        return (rsum[0] + rsum[1]) + (rsum[2] + rsum[3]);
    };

    // Causal: a tile entirely in this wave's future has no work; tiles that
    // cross the diagonal or the end of the sequence are masked.
    auto active = [&](int kt) { return !CAUSAL || kt * kBK <= qw0 + kQW - 1; };
    auto needs_mask = [&](int kt) {
        const int k0 = kt * kBK;
        return (CAUSAL && k0 + kBK - 1 > qw0) || (k0 + kBK > N);
    };

    load_rows(rK, 0);
    store_rows(kbuf_of(0), k_st);
    load_rows(rV, 0);
    store_rows(vbuf_of(0), v_st);
    __syncthreads();

    // The recurrence, with a lazily updated reference max m2.  Every tile
    // also moves the next tile into the other LDS buffers (past the last tile
    // the buffer loads return zeros and nothing reads them) and ends in one
    // barrier.
    //
    // Fast loop: unmasked tiles whose scaled row max stays within kLazy of
    // m2.  They take P = exp2(c*S - m2) <= 2^kLazy against the unchanged m2,
    // so acc and l need no rescale (alpha = 1) and no mask.
    // General path: everything else -- the first tile, diagonal and tail
    // tiles, and a tile whose max outgrows m2 + kLazy.  There m2 becomes the
    // running max exactly as in the recurrence, acc and l are rescaled by
    // alpha = exp2(m2_old - m2_new), and the loop is re-entered.
    // Both give the same softmax: only the common shift of a row differs.
    int kt = 0;
    f32x16 s[2];
    while (kt < n_kt) {
        bool mid_tile = false;   // left the fast loop after this tile's QK^T
        for (; kt < n_kt; ++kt) {
            if (!active(kt) || needs_mask(kt)) break;
            const int buf = kt & 1;
            load_rows(rK, kt + 1);
            qk_tile(buf, s);
            store_rows(kbuf_of(buf ^ 1), k_st);
            load_rows(rV, kt + 1);
            const float m2_tile = c * tile_max(s);
            if (__builtin_amdgcn_ballot_w64(m2_tile > m2 + kLazy)) {
                mid_tile = true;
                break;
            }
            lsum += exp_pv_pipelined(buf, s, m2);
            store_rows(vbuf_of(buf ^ 1), v_st);
            __syncthreads();
        }
        if (kt >= n_kt) break;

        const int buf = kt & 1;
        const bool act = active(kt);
        if (!mid_tile) {
            load_rows(rK, kt + 1);
            if (act) qk_tile(buf, s);
            store_rows(kbuf_of(buf ^ 1), k_st);
            load_rows(rV, kt + 1);
        }
        if (act) {
            const bool masked = needs_mask(kt);
            if (masked) mask_tile(kt * kBK, s);
            const float mx = tile_max(s);
            // A row with nothing visible yet keeps shift 0, so that
            // -inf - (-inf) never occurs; its weights are all zero.
            const float m2_tile = (mx == -INFINITY) ? -INFINITY : c * mx;
            const float m2_new = __builtin_fmaxf(m2, m2_tile);
            const float shift = (m2_new == -INFINITY) ? 0.f : m2_new;
            const float alpha = __builtin_amdgcn_exp2f(m2 - shift);
            m2 = m2_new;
#pragma unroll
            for (int db = 0; db < C::kDBlocks; ++db) oacc[db] *= alpha;
            h8 pf[4];
            // the masked variant is also right for unmasked tiles (no -inf)
            const float rs = exp_tile(std::true_type{}, s, shift, pf);
            lsum = alpha * lsum + rs;
            pv_tile(buf, pf);
        }
        store_rows(vbuf_of(buf ^ 1), v_st);
        __syncthreads();
        ++kt;
    }

    // Epilogue: one normalisation, fp16 (RNE) O, natural-log LSE.
    const float lt = pair_sum(lsum);
    const float inv = __builtin_amdgcn_rcpf(lt);
    const auto rO = make_rsrc(O + head, head_bytes);
    const int o_base = my_q * C::kRowBytes + 8 * hi;
#pragma unroll
    for (int db = 0; db < C::kDBlocks; ++db) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            h4 out;
#pragma unroll
            for (int t = 0; t < 4; ++t) out[t] = (_Float16)(oacc[db][4 * rr + t] * inv);
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, out), rO,
                                                  o_base + 64 * db + 16 * rr, 0, 0);
        }
    }
    if (hi == 0 && my_q < N) LSE[size_t(bh) * N + my_q] = (m2 + __builtin_amdgcn_logf(lt)) * kLn2;
}

template <int D, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                  int N, float c, uint32_t q_sign, hipStream_t stream) {
    using C = Cfg<D>;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&fa2_fwd_kernel<D, CAUSAL>),
        hipFuncAttributeMaxDynamicSharedMemorySize, C::kLdsBytes);
    if (attr != hipSuccess) return attr;
    const int n_qtiles = (N + kBQ - 1) / kBQ;
    const int n_wg = n_qtiles * BH;
    hipLaunchKernelGGL((fa2_fwd_kernel<D, CAUSAL>), dim3(n_wg), dim3(kThreads), C::kLdsBytes,
                       stream, static_cast<const _Float16*>(q), static_cast<const _Float16*>(k),
                       static_cast<const _Float16*>(v), static_cast<_Float16*>(o), lse, N,
                       n_qtiles, n_wg, c, q_sign);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                      int N, int d, float scale, bool causal, hipStream_t stream) {
    const float c = static_cast<float>(std::fabs(static_cast<double>(scale)) * 1.4426950408889634);
    const uint32_t q_sign = scale < 0.f ? 0x80008000u : 0u;
    if (d == 64) {
        return causal ? launch<64, true>(q, k, v, o, lse, BH, N, c, q_sign, stream)
                      : launch<64, false>(q, k, v, o, lse, BH, N, c, q_sign, stream);
    }
    return causal ? launch<128, true>(q, k, v, o, lse, BH, N, c, q_sign, stream)
                  : launch<128, false>(q, k, v, o, lse, BH, N, c, q_sign, stream);
}

}  // namespace fa2
