// FlashAttention-2 forward pass for AMD MI355X (gfx950 / CDNA4).
//
// What is computed ("3.6 Attention I -- the memory problem and FlashAttention
// principles", 3.6.4 and the tile loop of 3.6.6): for each query row the
// online-softmax state (running max m, running sum l, unnormalised output
// acc) is carried across key/value tiles; each tile updates
//     m_new = max(m, rowmax(S)),  alpha = exp(m - m_new),
//     P = exp(S - m_new),  l = alpha*l + rowsum(P),  acc = alpha*acc + P V,
// and the output is normalised once, O = acc / l, with LSE = m + ln l
// (3.6.7).  Causal attention stops at the diagonal and masks the tiles that
// cross it (3.6.6).
//
// How it maps onto gfx950.  The CuTe write-up ("FlashAttention-2 from scratch
// in CuTe") describes an A100 design; kept from it are the grid over
// (Q tile, batch*head) with the Q tile resident, a K/V prefetch ahead of use,
// 128-bit loads, bank-spread shared tiles and row-owning warps.
//
//  * Each wave owns 32 whole query rows, so every row reduction stays inside
//    the wave.  Head dims 32, 64, 96, 128 and 256 are compiled.  A workgroup
//    is 8 waves (256 queries of one (batch, head)) at d = 128 and at d = 64
//    (causal d = 64: once N >= 2048 and the grid fills the chip), and 4
//    waves (128 queries) otherwise: 8 waves halve the K/V staging per query,
//    while the smaller group wastes fewer masked keys on the diagonal of
//    short causal rows and fills the chip with small grids.  Two waves share
//    each SIMD; three at d = 32, whose registers allow it; one at d = 256,
//    where a wave's 32x256 fp32 accumulator needs the registers of a whole
//    SIMD.
//  * The score tile is computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_f16 (A = 32 keys x 16 dims from LDS, B = Q^T held in
//    registers for the whole loop).  In the 32x32 accumulator a lane then
//    holds one query (column) and 16 of the 32 keys; the other 16 sit in lane
//    l^32.  Row max = 16 in-lane values + one v_permlane32_swap; the row sum
//    needs no cross-lane step until the epilogue.
//  * Exponentials are taken in base 2 with the scale folded in:
//    P = exp2(S*c - m2), c = |scale|*log2(e) > 0, m2 a reference max of c*S.
//  * The accumulator's register order is reused as the B operand of the PV
//    MFMA (O^T = V^T P^T), so P never leaves registers; V^T comes from LDS
//    through ds_read_b64_tr_b16, which returns four consecutive keys of one
//    head-dim column per lane.
//  * Software pipeline over key tiles: iteration t runs, as one instruction
//    stream per wave, the MFMAs of P V for tile t-1 and of S^T for tile t+1
//    (both independent of tile t's softmax) interleaved slot by slot with the
//    softmax of tile t on the VALU.  The per-element VALU chain (scaled
//    score -> exp2 -> row sum and fp16 conversion) is itself pipelined across
//    slots, so no instruction waits on the one just issued.  S^T is
//    double-buffered in registers by tile parity; P is single-buffered: the
//    P V MFMAs come first in the stream and each 16-key chunk of P is
//    rewritten only after its last reader has issued.
//  * Lazy reference max, checked after the fact: the stream computes the
//    weights exp2(S*c - m2) against the row's current reference m2 without a
//    row max.  If every lane's 16 weights of the tile sum to at most
//    2^kLazy, each weight is at most 2^kLazy (safe in fp16) and m2 stays,
//    alpha = 1 (checking each lane's part needs no cross-lane step).
//    Otherwise (a weight may exceed 2^kLazy: the row max moved up, or m2 is
//    not finite) the wave redoes the tile with the recurrence step
//    itself: m2 := max(m2, scaled tile max), alpha = exp2(m2_old - m2_new),
//    weights recomputed.  A row's common shift cancels in the softmax, so
//    the result is the recurrence's; m2 starts at tile 0's max, and acc is
//    rescaled only when some row of the wave moved (ballot).
//  * K and V tiles (64 keys) are double-buffered in LDS and staged through
//    registers: each iteration writes the tiles fetched during the previous
//    one and fetches the next with 128-bit buffer loads, one LDS store or one
//    load per slot over the stream.  One barrier per tile (with the optional
//    ring of four tiles per tensor, one per two tiles).  Up to d = 96, and at
//    d = 128 with the ring of two, the last tile's iteration is a shorter
//    copy of the stream: no S^T of a next tile, no fetches; under the causal
//    mask a wave whose queries all precede that tile also skips its
//    (all-zero) softmax.  In an 8-wave
//    workgroup the waves 4-7, which lose issue arbitration to the older waves
//    0-3 on the same SIMD, run the stream at raised priority so the two
//    halves reach the barrier closer together.
//  * All global accesses are buffer instructions on a per-head resource
//    whose size is the head's N*d*2 bytes: rows past N read as zero and
//    stores past N are dropped by the hardware, so the tail needs no branch.
//  * Workgroup ids are remapped so that all Q tiles of one head run on the
//    same XCD (dispatch is round-robin over the 8 XCDs) and share its L2;
//    causal grids start with the longest rows, across small groups of heads.

// LDS tile layouts (fa2_device.h): V swizzled (chunk-major with an XOR of the
// row) for the transposing reads, K the same up to d = 128 and chunk-major at
// d = 256.  Both keep every per-lane address a lane base plus a compile-time
// offset.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>
#include <type_traits>

#include "fa2_device.h"
#include "fa2_launch.h"

namespace fa2 {
namespace {

using namespace dev;

// Compile-time tuning knobs.  The defaults are the measured choices;
// `bench.py --tile-sweep` rebuilds the library with other values and times
// them against each other.
#ifndef FA2_FWD_WAVES        // waves per workgroup at d = 64, 96, 128 (4 or 8); 0: Cfg's choice
#define FA2_FWD_WAVES 0
#endif
#ifndef FA2_FWD_KV_BUFS      // K/V tiles in LDS per tensor (2 or 4); 0: chosen at launch
#define FA2_FWD_KV_BUFS 0
#endif
#ifndef FA2_FWD_AHEAD        // LDS operand reads in flight ahead of the MFMAs; 0: Cfg's choice
#define FA2_FWD_AHEAD 0
#endif
#ifndef FA2_FWD_PRIO         // 8-wave groups: the younger half streams at raised priority
#define FA2_FWD_PRIO 1
#endif

// A tile keeps the row's reference max while each lane's weights in it sum
// to at most 2^kLazy, so every weight stays <= 2^8, far inside fp16 range.
constexpr float kLazyBound = 256.0f;   // 2^kLazy, kLazy = 8

template <int D, bool CAUSAL, int WV = 0>
struct Cfg {
    // Waves per workgroup (see the header): 8 at d = 128 and at non-causal
    // d = 64, 4 otherwise; causal d = 64 has both shapes (WV), chosen at
    // launch.  Two waves per SIMD; three at d = 32 (measured 6-7 % faster
    // non-causal than two); one at d = 256, whose registers need a SIMD each.
    static_assert(D == 32 || D == 64 || D == 96 || D == 128 || D == 256, "head dim");
    static constexpr int kWaves = (FA2_FWD_WAVES != 0 && (D == 64 || D == 128)) ? FA2_FWD_WAVES
                                  : WV != 0                                    ? WV
                                  : (D == 128 || (D == 64 && !CAUSAL))         ? 8 : 4;
    static_assert(kWaves == 4 || kWaves == 8, "waves per workgroup");
    static constexpr int kWavesPerSimd = D == 256 ? 1 : D == 32 ? 3 : 2;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kBQ = kWaves * kQW;               // query rows per workgroup
    static constexpr int kRowBytes = D * 2;
    static constexpr int kChunks = D / 8;                  // 16-byte chunks per row
    static constexpr int kTileBytes = kBK * kRowBytes;
    static constexpr int kDSteps = D / 16;                 // k-steps of the S^T MFMA
    static constexpr int kDBlocks = D / 32;                // 32-row blocks of O^T
    static constexpr int kStage = kChunks / kWaves;        // staged chunks per thread per tile
    static_assert(kChunks % kWaves == 0, "every chunk of a row staged by one wave");
    // K/V staging in row blocks (contiguous global segments, swizzled K) up
    // to d = 128; at d = 256 in chunk columns (see the kernel).
    static constexpr bool kRowStage = D <= 128;
    static constexpr int kPV = 4 * kDBlocks;               // P V MFMAs per tile
    static constexpr int kQK = 2 * kDSteps;                // S^T MFMAs per tile
    static constexpr int kSlots = kPV + kQK;               // one MFMA per slot
    // LDS operand reads in flight ahead of the MFMAs (measured best: 5 at
    // 8-wave d = 64 and at d = 256, 3 at d = 128, 4 elsewhere; 3..5 lie
    // within ~1 %).
    static constexpr int kAhead = FA2_FWD_AHEAD != 0                     ? FA2_FWD_AHEAD
                                  : (D == 64 && kWaves == 8) || D == 256 ? 5
                                  : D == 128                             ? 3 : 4;
    static_assert(kAhead >= 1 && kAhead <= 8, "read-ahead");
    // K/V tiles in LDS per tensor: a ring of 2, or of 4, which needs a
    // barrier only after every second tile (twice the LDS: 128 KiB at
    // d = 128; too much at d = 256, and at d = 96 it keeps a second
    // workgroup off the CU).  The launch picks the ring (pick_bufs);
    // kRing4 says whether the ring of 4 is compiled at all.
    static constexpr bool kRing4 = FA2_FWD_KV_BUFS == 4 ? (D != 96 && D != 256)
                                 : FA2_FWD_KV_BUFS == 0 && ((D == 64 && kWaves == 8) || D == 128);
    // Ring of 4 where measured faster (bench.py --tile-sweep, both run
    // orders): 8-wave d = 64 (+1.8 % at [4,32,2048,64]) and d = 128 once
    // a workgroup's key loop is long (+1 % at [2,16,16384,128], +2.7 % at
    // [1,16,65536,128] causal; -2 % at [4,32,2048,128]).
    static int pick_bufs(int N) {
        if (!kRing4) return 2;
        if (FA2_FWD_KV_BUFS == 4) return 4;
        return (D == 64 || N >= 8192) ? 4 : 2;
    }
    // Element pairs enter the three-stage VALU chain (scaled score, exp2,
    // sum + fp16) in slots [kE0, kE1); a pair's last stage runs two slots
    // after its first.
    static constexpr int kE0 = kDBlocks > 2 ? kDBlocks - 2 : 0;
    static constexpr int kE1 = kSlots - 2;
    static constexpr int pair_begin(int p) {
        return p <= kE0 ? 0 : p >= kE1 ? 16 : ((p - kE0) * 16) / (kE1 - kE0);
    }
    // P chunk ks (pairs 4ks .. 4ks+3) may be rewritten only after the last
    // P V MFMA that reads it (slot kDBlocks*ks + kDBlocks-1).
    static constexpr bool schedule_ok() {
        for (int p = 0; p < kSlots; ++p)
            for (int j = pair_begin(p); j < pair_begin(p + 1); ++j)
                if (p + 2 <= kDBlocks * (j / 4) + kDBlocks - 1) return false;
        // The staging stores take slots 0, 2, .., 4*kStage-2 and the loads
        // refilling the same registers slots 2*kStage+1, .., 6*kStage-1.
        return pair_begin(kSlots) == 16 && kStage >= 1 && 6 * kStage - 1 < kSlots;
    }
};

template <int D, bool CAUSAL, int NB, int WV>
__global__ __launch_bounds__((Cfg<D, CAUSAL, WV>::kThreads))
__attribute__((amdgpu_waves_per_eu(Cfg<D, CAUSAL, WV>::kWavesPerSimd, Cfg<D, CAUSAL, WV>::kWavesPerSimd)))
void fa2_fwd_kernel(const _Float16* __restrict__ Q, const _Float16* __restrict__ K,
                    const _Float16* __restrict__ V, _Float16* __restrict__ O,
                    float* __restrict__ LSE, int N, int n_qtiles, int n_wg, float c,
                    uint32_t q_and, uint32_t q_xor, int group) {
    using C = Cfg<D, CAUSAL, WV>;
    static_assert(C::schedule_ok(), "P chunk rewritten before its last reader");
    static_assert(NB == 2 || NB == 4, "K/V buffers");
    constexpr int kAhead = C::kAhead;
    // One LDS block: NB K tiles, then NB V tiles; after the key loop the
    // epilogue reuses it to restage O (kOutStride bytes per row).
    constexpr int kOutStride = C::kRowBytes + 16;
    constexpr int kLdsBytes = 2 * NB * C::kTileBytes > C::kWaves * kQW * kOutStride
                                  ? 2 * NB * C::kTileBytes
                                  : C::kWaves * kQW * kOutStride;
    __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];
    const auto kbuf = reinterpret_cast<unsigned char (*)[C::kTileBytes]>(lds);
    const auto vbuf = reinterpret_cast<unsigned char (*)[C::kTileBytes]>(lds + NB * C::kTileBytes);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    // Logical tile id: consecutive ids (the Q tiles of one head) go to one XCD.
    const int wg = blockIdx.x;
    const int logical = xcd_logical_id(wg, n_wg);
    // Causal grids take the query tiles longest first, a few heads at a
    // time (head_tile_of); the group is 1 otherwise.
    const HeadTile ht = head_tile_of(logical, n_qtiles, CAUSAL ? group : 1);
    const int bh = ht.bh;
    int qt = ht.rank;
    if (CAUSAL) qt = n_qtiles - 1 - qt;   // longest rows first
    const int q0 = qt * C::kBQ;
    const size_t head = size_t(bh) * size_t(N) * D;
    const uint32_t head_bytes = uint32_t(N) * C::kRowBytes;
    const auto rQ = make_rsrc(Q + head, head_bytes);
    const auto rK = make_rsrc(K + head, head_bytes);
    const auto rV = make_rsrc(V + head, head_bytes);

    const int qw0 = q0 + wave * kQW;   // first query of this wave
    const int my_q = qw0 + l32;        // the query this lane owns

    // Q^T fragments (B operand of S^T): lane holds query my_q, dims
    // 16*ds + 8*hi + [0,8).  q_and clears Q for a zero scale, q_xor flips its
    // sign for a negative one: softmax(s*S) = softmax(|s| * (-Q) K^T).
    // Loaded in the prologue after the first K/V loads (load_q below).
    h8 qf[C::kDSteps];
    auto load_q = [&]() {
#pragma unroll
        for (int ds = 0; ds < C::kDSteps; ++ds) {
            u32x4 raw = __builtin_amdgcn_raw_buffer_load_b128(rQ, my_q * C::kRowBytes + 32 * ds + 16 * hi, 0, 0);
            raw = (raw & q_and) ^ q_xor;
            qf[ds] = __builtin_bit_cast(h8, raw);
        }
    };

    const int kv_end = CAUSAL ? min(N, q0 + C::kBQ) : N;
    const int n_kt = (kv_end + kBK - 1) / kBK;
    // Tiles below n_full need no mask for any row of the workgroup.
    const int n_full = CAUSAL ? min(N / kBK, (q0 + 1) / kBK) : N / kBK;

    // Staging.  Load instruction n = w + kWaves*j (j < kStage) of wave w
    // moves one block of a tile.  Row blocks (d <= 128): kRi row segments of
    // kCi chunks -- 1 KiB of consecutive bytes when a row holds 8 or 16
    // chunks -- each 16-lane group taking 4 rows x 4 chunks, so its LDS
    // writes, both tiles in the swizzled layout, hit 16 distinct 16-byte bank
    // groups.  Chunk columns (d = 256, whose registers have no room for the
    // row block's addresses): chunk n of the 64 rows, one row per lane, K
    // chunk-major.
    u32x4 stk[C::kStage], stv[C::kStage];
    constexpr int kCi = (C::kChunks % 16 == 0) ? 16 : (C::kChunks % 8 == 0) ? 8 : 4;
    constexpr int kRi = 64 / kCi;
    constexpr int kCB = C::kChunks / kCi;
    const int st_r = ((lane >> 4) % (kRi / 4)) * 4 + (lane & 3);
    const int st_c = ((lane >> 4) / (kRi / 4)) * 4 + ((lane & 15) >> 2);
    auto st_row = [&](int j) {
        return C::kRowStage ? ((wave + C::kWaves * j) / kCB) * kRi + st_r : lane;
    };
    auto st_ch = [&](int j) {
        return C::kRowStage ? ((wave + C::kWaves * j) % kCB) * kCi + st_c : wave + C::kWaves * j;
    };
    auto fetch1 = [&](u32x4& dst, __amdgpu_buffer_rsrc_t r, int kt, int j) {
        dst = __builtin_amdgcn_raw_buffer_load_b128(
            r, (kt * kBK + st_row(j)) * C::kRowBytes + st_ch(j) * 16, 0, 0);
    };
    auto put_k1 = [&](unsigned char* buf, const u32x4& src, int j) {
        const int off = C::kRowStage ? lds_v_off(st_ch(j), st_row(j)) : lds_k_off(st_ch(j), st_row(j));
        *reinterpret_cast<u32x4*>(buf + off) = src;
    };
    auto put_v1 = [&](unsigned char* buf, const u32x4& src, int j) {
        *reinterpret_cast<u32x4*>(buf + lds_v_off(st_ch(j), st_row(j))) = src;
    };

    f32x16 oacc[C::kDBlocks];
#pragma unroll
    for (int db = 0; db < C::kDBlocks; ++db) oacc[db] = f32x16{};
    float m2 = -INFINITY;   // reference max of c*S for this query (log2 units)
    float lsum = 0.f;       // this lane's share of the running sum
    float alpha = 1.0f;     // rescale of acc owed by the next P V
    h8 pf[4];               // P of the last softmax'd tile, 4 chunks of 16 keys
#pragma unroll
    for (int i = 0; i < 4; ++i) pf[i] = h8{};
    f32x16 s0[2], s1[2];    // S^T of the even / odd tiles

    // Per-lane LDS read bases; the unrolled loops add compile-time offsets.
    // K (A operand of S^T): key 32*kb + l32, chunk 2*ds + hi.  Swizzled K
    // (row-block staging): chunk c of row r at (64c + (r ^ 4(c & 3))) * 16,
    // and c & 3 = 2*(ds & 1) + hi, so two lane bases cover every (ds, kb).
    const int k_base0 = C::kRowStage ? (hi * 64 + (l32 ^ (4 * hi))) << 4 : lds_k_off(hi, l32);
    const int k_base1 = C::kRowStage ? (hi * 64 + (l32 ^ (8 + 4 * hi))) << 4 : k_base0;
    auto k_off = [&](int ds, int kb) {
        return ((ds & 1) ? k_base1 : k_base0) + lds_k_off(2 * ds, 32 * kb);
    };
    // V^T (A operand of O^T) via ds_read_b64_tr_b16 (TrBase).
    const TrBase vt(lane);

    // Keys at or beyond N, and under the causal mask keys after the query,
    // get -inf.  Accumulator element (kb, r) is key k0 + 4hi + off with
    // off = 32kb + 8(r/4) + r%4, visible iff off <= lim for this lane's
    // limit (one compare and one select per element).
    auto mask_tile = [&](int k0, f32x16 (&s)[2]) {
        int lim = N - 1 - k0 - 4 * hi;                       // key < N
        if constexpr (CAUSAL) lim = min(lim, my_q - k0 - 4 * hi);   // key <= q
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
                if (off > lim) s[kb][r] = -INFINITY;
            }
        }
    };
    // Whether tile t needs mask_tile for this wave: beyond n_full (the
    // workgroup's bound) it does unless, under the causal mask, every key of
    // the tile is at or before this wave's first query and inside [0, N)
    // (wave-uniform).
    auto needs_mask = [&](int t) {
        return t >= n_full && (!CAUSAL || (t + 1) * kBK - 1 > qw0 || (t + 1) * kBK > N);
    };

    // Prologue.  The V buffer of tile -1 starts zeroed: the first
    // iteration's P V runs with P = 0 on it.  With a ring of 4, K(0..2) and
    // V(0) go to LDS and K(3), V(1) are fetched for the first iteration to
    // store; with 2, K(0), K(1) go to LDS and K(2), V(0) are fetched.  All
    // of these loads are issued together, before the first LDS store, so the
    // workgroup waits for one memory round trip, not two.  Q's loads come
    // after the K/V ones: the LDS stores and the first barrier wait only for
    // K/V (measured 0.6-2 % faster than Q first).
    for (int i = tid; i < C::kTileBytes / 16; i += C::kThreads)
        reinterpret_cast<u32x4*>(vbuf[NB - 1])[i] = u32x4{0u, 0u, 0u, 0u};
    if constexpr (NB == 4) {
        u32x4 t0[C::kStage], t1[C::kStage], t2[C::kStage], t3[C::kStage];
#pragma unroll
        for (int j = 0; j < C::kStage; ++j) {
            fetch1(t0[j], rK, 0, j);
            fetch1(t1[j], rK, 1, j);
            fetch1(t2[j], rK, 2, j);
            fetch1(t3[j], rV, 0, j);
        }
#pragma unroll
        for (int j = 0; j < C::kStage; ++j) {
            fetch1(stk[j], rK, 3, j);
            fetch1(stv[j], rV, 1, j);
        }
        load_q();
#pragma unroll
        for (int j = 0; j < C::kStage; ++j) {
            put_k1(kbuf[0], t0[j], j);
            put_k1(kbuf[1], t1[j], j);
            put_k1(kbuf[2], t2[j], j);
            put_v1(vbuf[0], t3[j], j);
        }
    } else {
        u32x4 t0[C::kStage], t1[C::kStage];
#pragma unroll
        for (int j = 0; j < C::kStage; ++j) {
            fetch1(t0[j], rK, 0, j);
            fetch1(t1[j], rK, 1, j);
        }
#pragma unroll
        for (int j = 0; j < C::kStage; ++j) {
            fetch1(stk[j], rK, 2, j);
            fetch1(stv[j], rV, 0, j);
        }
        load_q();
#pragma unroll
        for (int j = 0; j < C::kStage; ++j) {
            put_k1(kbuf[0], t0[j], j);
            put_k1(kbuf[1], t1[j], j);
        }
    }
    __syncthreads();
    {   // S^T of tile 0
#pragma unroll
        for (int ds = 0; ds < C::kDSteps; ++ds) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const h8 a = *reinterpret_cast<const h8*>(kbuf[0] + k_off(ds, kb));
                s0[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[ds], ds == 0 ? f32x16{} : s0[kb], 0, 0, 0);
            }
        }
    }
    // Reference max from tile 0, so the first iteration needs no correction.
    if (needs_mask(0)) mask_tile(0, s0);
    {
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 32; ++i) mx = __builtin_fmaxf(mx, s0[i >> 4][i & 15]);
        m2 = c * pair_max(mx);
    }
    __syncthreads();   // K buffer 0 is free before the first iteration refills it

    // Iteration t (PAR = t mod NB; tile x lives in buffer x mod NB).  It
    // reads K(t+1) (for S^T of the next tile) and V(t-1) (for P V of the
    // previous one).  Ring of 4: it stores K(t+3) and V(t+1), staged in
    // registers during iteration t-1, and fetches K(t+4), V(t+2); a barrier
    // follows every odd iteration, so a buffer is rewritten only after the
    // barrier that follows its last read, and read only after the barrier
    // that follows its store.  Ring of 2: it stores K(t+2), V(t), fetches
    // K(t+3), V(t+1), and every iteration ends with a barrier.  Loads past
    // the last tile read zeros or data that is never used.
    auto step = [&](auto par_tag, auto kind_tag, int t, f32x16 (&s_cur)[2], f32x16 (&s_next)[2]) {
        constexpr int PAR = decltype(par_tag)::value;
        // The last tile's iteration (LAST): there is no next tile, so it
        // issues no S^T products and no fetches, and stores only what a later
        // read needs.
        constexpr bool LAST = decltype(kind_tag)::value >= 1;
        // DEAD (causal): every key of the last tile comes after every query
        // of this wave, so its weights are all zero: only the P V of the
        // previous tile remains.
        constexpr bool DEAD = decltype(kind_tag)::value == 2;
        constexpr int kAheadK = NB == 4 ? 3 : 2, kAheadV = NB == 4 ? 1 : 0;
        unsigned char* kb_store = kbuf[(PAR + kAheadK) % NB];
        unsigned char* vb_store = vbuf[(PAR + kAheadV) % NB];
        const unsigned char* kb_read = kbuf[(PAR + 1) % NB];
        const unsigned char* vb_read = vbuf[(PAR + NB - 1) % NB];

        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
            for (int db = 0; db < C::kDBlocks; ++db) oacc[db] *= alpha;
        }
        if (!DEAD && needs_mask(t)) mask_tile(t * kBK, s_cur);

        // MFMA job p: p < kPV is P V (k-step p / kDBlocks, O^T block
        // p % kDBlocks), then S^T (d-step, key block).  Operands are read
        // kAhead jobs early into a ring.
        // The last iteration at d = 128 reads only one product ahead: its
        // extra copy of the stream then fits the registers (no spills).
        constexpr int kA = (LAST && D == 128) ? kAhead - 2 : kAhead;
        h8 ring[kA + 1];
        auto read = [&](int p) {
            if (p < C::kPV) {
                const int ks = p / C::kDBlocks, db = p % C::kDBlocks;
                ring[p % (kA + 1)] = read_tr_operand(vb_read, vt, tr_imm(ks, db));
            } else {
                const int j = p - C::kPV, ds = j >> 1, kb = j & 1;
                ring[p % (kA + 1)] = *reinterpret_cast<const h8*>(kb_read + k_off(ds, kb));
            }
        };
        auto mfma = [&](int p) {
            const h8 a = ring[p % (kA + 1)];
            if (p < C::kPV) {
                const int ks = p / C::kDBlocks, db = p % C::kDBlocks;
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[ks], oacc[db], 0, 0, 0);
            } else {
                const int j = p - C::kPV, ds = j >> 1, kb = j & 1;
                s_next[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[ds], ds == 0 ? f32x16{} : s_next[kb], 0, 0, 0);
            }
        };

        // Softmax of tile t against the current reference max, one slice per
        // slot; checked after the stream.
        const float shift = m2;
        float rsum[4];
        float arg[32], pe[32];
        auto sv = [&](int i) { return s_cur[i >> 4][i & 15]; };
        auto pb = [&](int p) { return p < 0 ? 0 : C::pair_begin(p); };
        auto valu = [&](int p) {
            // Stage 3: row sum and fp16 P of the pairs that entered two slots ago.
#pragma unroll
            for (int j = pb(p - 2); j < pb(p - 1); ++j) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int e = 2 * j + h;
                    rsum[e & 3] = e < 4 ? pe[e] : rsum[e & 3] + pe[e];
                    pf[e >> 3][e & 7] = (_Float16)pe[e];
                    pin(rsum[e & 3]);
                }
                pin(pf[j >> 2]);
            }
            // Stage 2: exp2 of the pairs that entered one slot ago.
#pragma unroll
            for (int j = pb(p - 1); j < pb(p); ++j) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int e = 2 * j + h;
                    pe[e] = __builtin_amdgcn_exp2f(arg[e]);
                    pin(pe[e]);
                }
            }
            // Stage 1: scaled, shifted scores of the pairs entering now.
#pragma unroll
            for (int j = pb(p); j < pb(p + 1); ++j) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int e = 2 * j + h;
                    arg[e] = __builtin_fmaf(sv(e), c, -shift);
                    pin(arg[e]);
                }
            }
        };

        // The stream: per slot, the LDS read kAhead jobs ahead, one MFMA,
        // the slot's VALU slice and at most one staging step: the K(t+2) and
        // V(t) chunks fetched last iteration go to LDS in slots 0, 2, ..,
        // then their registers are refilled with K(t+3) and V(t+1) in the odd
        // slots after that.  The scheduling barriers keep this order.
#pragma unroll
        for (int p = 0; p < kA; ++p) read(p);
        __builtin_amdgcn_sched_barrier(0);
        if (FA2_FWD_PRIO && C::kWaves == 8 && wave >= 4) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int p = 0; p < C::kSlots; ++p) {
            if (p + kA < (LAST ? C::kPV : C::kSlots)) read(p + kA);
            if (!LAST || p < C::kPV) mfma(p);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (!DEAD) valu(p);
            // (With a ring of two the last iteration still stores V of its
            // own tile, which the P V after the loop reads.)
            if constexpr (!LAST || NB == 2) {
                if (p % 2 == 0 && p / 2 >= C::kStage && p / 2 < 2 * C::kStage)
                    put_v1(vb_store, stv[p / 2 - C::kStage], p / 2 - C::kStage);
            }
            if constexpr (!LAST) {
                if (p % 2 == 0 && p / 2 < C::kStage) put_k1(kb_store, stk[p / 2], p / 2);
                const int q = p - 2 * C::kStage - 1;
                if (q >= 0 && q % 2 == 0 && q / 2 < C::kStage) fetch1(stk[q / 2], rK, t + kAheadK + 1, q / 2);
                if (q >= 0 && q % 2 == 0 && q / 2 >= C::kStage && q / 2 < 2 * C::kStage)
                    fetch1(stv[q / 2 - C::kStage], rV, t + kAheadV + 1, q / 2 - C::kStage);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
        // This lane's weights of the tile sum to at most 2^kLazy in every
        // lane: each weight is then <= 2^kLazy and the reference max stays.
        // (The first weight of each partial sum starts it, no add of 0.)  Otherwise
        // (the row max moved up, or m2 was still -inf) take the recurrence
        // step exactly: m2 := max(m2, tile max), rescale, recompute.
        if constexpr (DEAD) {
            alpha = 1.0f;
        } else {
            const float part = (rsum[0] + rsum[1]) + (rsum[2] + rsum[3]);
            if (__builtin_amdgcn_ballot_w64(!(part <= kLazyBound))) {
                float mx = -INFINITY;
#pragma unroll
                for (int i = 0; i < 32; ++i) mx = __builtin_fmaxf(mx, sv(i));
                const float m2_new = __builtin_fmaxf(m2, c * pair_max(mx));
                const float sh = m2_new == -INFINITY ? 0.f : m2_new;
                alpha = __builtin_amdgcn_exp2f(m2 - sh);
                m2 = m2_new;
                float r[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int e = 0; e < 32; ++e) {
                    const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sv(e), c, -sh));
                    r[e & 3] += pv;
                    pf[e >> 3][e & 7] = (_Float16)pv;
                }
                lsum = alpha * lsum + ((r[0] + r[1]) + (r[2] + r[3]));
            } else {
                alpha = 1.0f;
                lsum += part;
            }
        }
        if (NB == 2 || (PAR & 1)) __syncthreads();
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using Mid = std::integral_constant<int, 0>;
    using Last = std::integral_constant<int, 1>;
    using Dead = std::integral_constant<int, 2>;
    // Causal: this wave's queries all come before the last tile's keys.
    const bool dead = CAUSAL && qw0 + kQW <= (n_kt - 1) * kBK;
    int t = 0;
    // Up to d = 96, and at d = 128 with the ring of two, the last tile's
    // iteration is a LAST step (+0.6 to +1.8 % causal at d = 128, 0 to +0.7 %
    // non-causal).  With the ring of four at d = 128, and at d = 256, its
    // extra copy of the stream would spill hundreds of registers, so every
    // iteration there is a full one.
    const int n_main = n_kt - 1;   // iterations before the last tile's
    if constexpr (D > 128 || (D == 128 && NB == 4)) {
        if constexpr (NB == 4) {
            for (; t + 3 < n_kt; t += 4) {
                step(I0{}, Mid{}, t, s0, s1);
                step(I1{}, Mid{}, t + 1, s1, s0);
                step(I2{}, Mid{}, t + 2, s0, s1);
                step(I3{}, Mid{}, t + 3, s1, s0);
            }
            if (t < n_kt) step(I0{}, Mid{}, t, s0, s1);
            if (t + 1 < n_kt) step(I1{}, Mid{}, t + 1, s1, s0);
            if (t + 2 < n_kt) step(I2{}, Mid{}, t + 2, s0, s1);
        } else {
            for (; t + 1 < n_kt; t += 2) {
                step(I0{}, Mid{}, t, s0, s1);
                step(I1{}, Mid{}, t + 1, s1, s0);
            }
            if (t < n_kt) step(I0{}, Mid{}, t, s0, s1);
        }
    } else if constexpr (NB == 4) {
        for (; t + 3 < n_main; t += 4) {
            step(I0{}, Mid{}, t, s0, s1);
            step(I1{}, Mid{}, t + 1, s1, s0);
            step(I2{}, Mid{}, t + 2, s0, s1);
            step(I3{}, Mid{}, t + 3, s1, s0);
        }
        if (t < n_main) step(I0{}, Mid{}, t, s0, s1);
        if (t + 1 < n_main) step(I1{}, Mid{}, t + 1, s1, s0);
        if (t + 2 < n_main) step(I2{}, Mid{}, t + 2, s0, s1);
        if (CAUSAL && dead) {
            switch (n_main & 3) {
                case 0: step(I0{}, Dead{}, n_main, s0, s1); break;
                case 1: step(I1{}, Dead{}, n_main, s1, s0); break;
                case 2: step(I2{}, Dead{}, n_main, s0, s1); break;
                default: step(I3{}, Dead{}, n_main, s1, s0); break;
            }
        } else {
            switch (n_main & 3) {
                case 0: step(I0{}, Last{}, n_main, s0, s1); break;
                case 1: step(I1{}, Last{}, n_main, s1, s0); break;
                case 2: step(I2{}, Last{}, n_main, s0, s1); break;
                default: step(I3{}, Last{}, n_main, s1, s0); break;
            }
        }
    } else {
        for (; t + 1 < n_main; t += 2) {
            step(I0{}, Mid{}, t, s0, s1);
            step(I1{}, Mid{}, t + 1, s1, s0);
        }
        if (t < n_main) step(I0{}, Mid{}, t, s0, s1);
        if (CAUSAL && dead) {
            if (n_main & 1) step(I1{}, Dead{}, n_main, s1, s0);
            else step(I0{}, Dead{}, n_main, s0, s1);
        } else {
            if (n_main & 1) step(I1{}, Last{}, n_main, s1, s0);
            else step(I0{}, Last{}, n_main, s0, s1);
        }
    }

    // P V of the last tile.
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
        for (int db = 0; db < C::kDBlocks; ++db) oacc[db] *= alpha;
    }
    if (!dead) {
        // V(n_kt-1) was stored before the barrier that followed iteration
        // n_kt-2 or n_kt-1 (or in the prologue).
        const unsigned char* vb_read = vbuf[(n_kt - 1) % NB];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int db = 0; db < C::kDBlocks; ++db) {
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                    read_tr_operand(vb_read, vt, tr_imm(ks, db)), pf[ks], oacc[db], 0, 0, 0);
            }
        }
    }

    // Epilogue: one normalisation, fp16 (RNE) O, natural-log LSE.  O^T
    // element (db, r) of this lane is row my_q, column 32*db + 8*(r/4) +
    // 4*hi + r%4: written straight out, one instruction would cover 32 rows
    // with 16 bytes each.  The wave's 32 x D block goes through LDS instead
    // (rows kOutStride = 2*D + 16 bytes apart, so the 8-byte writes of a
    // half-wave fall on distinct banks) and leaves as 128-bit stores of
    // whole rows: 64 lanes cover 1 KiB of consecutive output.
    const float lt = pair_sum(lsum);
    const float inv = __builtin_amdgcn_rcpf(lt);
    const auto rO = make_rsrc(O + head, head_bytes);
    __syncthreads();   // every wave is done with the K/V tiles
    unsigned char* ob = lds + wave * kQW * kOutStride;
#pragma unroll
    for (int db = 0; db < C::kDBlocks; ++db) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            h4 out;
#pragma unroll
            for (int k = 0; k < 4; ++k) out[k] = (_Float16)(oacc[db][4 * rr + k] * inv);
            *reinterpret_cast<h4*>(ob + l32 * kOutStride + 64 * db + 16 * rr + 8 * hi) = out;
        }
    }
    // The block is read back by this wave only: its own LDS writes must have
    // completed (lgkmcnt(0)); no other wave is involved.
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < kQW * C::kChunks / 64; ++i) {
        const int row = (i * 64 + lane) / C::kChunks, ch = (i * 64 + lane) % C::kChunks;
        const u32x4 val = *reinterpret_cast<const u32x4*>(ob + row * kOutStride + 16 * ch);
        __builtin_amdgcn_raw_buffer_store_b128(val, rO, (qw0 + row) * C::kRowBytes + 16 * ch, 0, 0);
    }
    if (hi == 0 && my_q < N) LSE[size_t(bh) * N + my_q] = (m2 + __builtin_amdgcn_logf(lt)) * kLn2;
}

template <int D, bool CAUSAL, int WV>
hipError_t launch_w(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                    int N, float c, uint32_t q_and, uint32_t q_xor, hipStream_t stream) {
    using C = Cfg<D, CAUSAL, WV>;
    const int n_qtiles = (N + C::kBQ - 1) / C::kBQ;
    const int n_wg = n_qtiles * BH;
    const int group = CAUSAL ? causal_group(n_qtiles, n_wg, 4 * C::kWavesPerSimd / C::kWaves) : 1;
    const auto* qh = static_cast<const _Float16*>(q);
    const auto* kh = static_cast<const _Float16*>(k);
    const auto* vh = static_cast<const _Float16*>(v);
    auto* oh = static_cast<_Float16*>(o);
    if constexpr (C::kRing4) {
        if (C::pick_bufs(N) == 4) {
            hipLaunchKernelGGL((fa2_fwd_kernel<D, CAUSAL, 4, WV>), dim3(n_wg), dim3(C::kThreads), 0,
                               stream, qh, kh, vh, oh, lse, N, n_qtiles, n_wg, c, q_and, q_xor,
                               group);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((fa2_fwd_kernel<D, CAUSAL, 2, WV>), dim3(n_wg), dim3(C::kThreads), 0, stream,
                       qh, kh, vh, oh, lse, N, n_qtiles, n_wg, c, q_and, q_xor, group);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                  int N, float c, uint32_t q_and, uint32_t q_xor, hipStream_t stream) {
    if constexpr (D == 64 && CAUSAL) {
        // Causal d = 64: 8-wave groups (a ring of four, reads five ahead) once
        // rows are long and the grid of 256-query tiles still gives every one
        // of the 256 CUs a workgroup (measured +2 % at N = 2048, +4-5 % at
        // 4096, +7-8 % at 16384 and 65536); 4-wave groups below (-3 % at
        // N = 1024 with 8, -13 % at 512, and small grids leave CUs idle).
        const int64_t n8 = int64_t((N + 255) / 256) * BH;
        if (N >= 2048 && n8 >= 256)
            return launch_w<D, CAUSAL, 8>(q, k, v, o, lse, BH, N, c, q_and, q_xor, stream);
        return launch_w<D, CAUSAL, 4>(q, k, v, o, lse, BH, N, c, q_and, q_xor, stream);
    } else {
        return launch_w<D, CAUSAL, 0>(q, k, v, o, lse, BH, N, c, q_and, q_xor, stream);
    }
}

}  // namespace

hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                      int N, int d, float scale, bool causal, hipStream_t stream) {
    // A |scale| below the smallest normal float moves no score by a
    // representable amount in fp32 arithmetic: it is run as scale 0 (Q
    // cleared, c = 1: uniform weights over the visible keys).  Otherwise Q's
    // sign bits carry the sign of the scale and c = |scale| * log2(e) > 0.
    const double a = std::fabs(static_cast<double>(scale));
    const bool zero = !(a >= 1.17549435082228751e-38);
    const float c = zero ? 1.0f : static_cast<float>(a * 1.4426950408889634);
    const uint32_t q_and = zero ? 0u : 0xffffffffu;
    const uint32_t q_xor = (!zero && scale < 0.f) ? 0x80008000u : 0u;
    switch (d) {
        case 32:
            return causal ? launch<32, true>(q, k, v, o, lse, BH, N, c, q_and, q_xor, stream)
                          : launch<32, false>(q, k, v, o, lse, BH, N, c, q_and, q_xor, stream);
        case 64:
            return causal ? launch<64, true>(q, k, v, o, lse, BH, N, c, q_and, q_xor, stream)
                          : launch<64, false>(q, k, v, o, lse, BH, N, c, q_and, q_xor, stream);
        case 96:
            return causal ? launch<96, true>(q, k, v, o, lse, BH, N, c, q_and, q_xor, stream)
                          : launch<96, false>(q, k, v, o, lse, BH, N, c, q_and, q_xor, stream);
        case 128:
            return causal ? launch<128, true>(q, k, v, o, lse, BH, N, c, q_and, q_xor, stream)
                          : launch<128, false>(q, k, v, o, lse, BH, N, c, q_and, q_xor, stream);
        case 256:
            return causal ? launch<256, true>(q, k, v, o, lse, BH, N, c, q_and, q_xor, stream)
                          : launch<256, false>(q, k, v, o, lse, BH, N, c, q_and, q_xor, stream);
        default:
            return hipErrorInvalidValue;
    }
}

}  // namespace fa2
