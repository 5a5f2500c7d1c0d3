// Measurement probes for gfx950 (not part of the attention library's
// interface; bench.py --lds-probe, --valu-probe and --step-probe call them,
// and the forward bench lines take the step model's ceiling from here).
//
// LDS read bandwidth.  The forward kernels read every K tile with
// ds_read_b128 and every V tile with ds_read_b64_tr_b16, each wave the whole
// tile.  lds_read_probe measures what one CU's LDS delivers for those two
// instructions at a given number of waves per CU: every wave reads a 64 KiB
// LDS block again and again (16 reads per iteration, consecutive 16- or
// 8-byte lane segments, no bank conflicts), folding the data into one
// register so no read is dropped.
//
// VALU issue rate.  The softmax of a key tile is a stream of fp32 VALU
// instructions (fma, exp2, add, conversions).  valu_issue_probe times 16
// independent chains of one instruction kind (or a fixed mix) per wave, so
// that no instruction waits on the one before it: the cycles per
// instruction it reports are the wave's own issue rate (one wave per SIMD)
// or the SIMD's (several).
//
// A model of the forward's key step (d = 64 and 128).  step_model_probe
// runs, per wave, the MFMA work of one 64-key tile against 32 queries
// (d/8 S^T and d/8 P V products of v_mfma_f32_32x32x16_f16) with the
// softmax VALU work between them, in variants that add the real kernel's
// parts one at a time: MFMAs alone; S^T, then softmax, then P V in sequence;
// the software pipeline of the forward (P V of tile t-1 and S^T of tile t+1
// interleaved with tile t's softmax); the pipeline with its A operands read
// from LDS; that with a workgroup barrier every second tile; the sequential
// step with its A operands read from LDS; and the full pipeline with the
// next K/V tiles staged from HBM through registers, or by direct
// global-to-LDS loads.  No output is written and there is no prologue or
// epilogue, so the rates are ceilings for the corresponding kernel design on
// this chip, its clock under that load included.
//
// Wave 0 of workgroup 0 (LDS) or every wave (VALU, step model) reads the
// shader clock counter around its loop; the LDS probe and the step model
// also read the fixed 100 MHz counter, which gives the clock the CUs ran at.
// Where several waves share a SIMD it does not serve them evenly (the
// oldest runs ahead and finishes first), so per-SIMD rates come from the
// longest loop among each workgroup's waves, which started together, not
// from the mean of the waves' loop times.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace {

typedef __fp16 tr4 __attribute__((vector_size(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kLdsBytes = 65536;
constexpr int kRegion = 16384;   // four regions, a wave moves between them

template <int MODE>
__global__ void lds_read_probe(uint32_t* __restrict__ out, unsigned long long* __restrict__ clk,
                               int iters) {
    // kLdsBytes read, 32 KiB more only reserved (read once below), so that
    // no second workgroup fits on the CU.
    __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes + 32768];
    const int tid = threadIdx.x, nt = blockDim.x;
    for (int i = tid; i < (kLdsBytes + 32768) / 4; i += nt)
        reinterpret_cast<uint32_t*>(lds)[i] = uint32_t(i) * 2654435761u;
    __syncthreads();
    const int lane = tid & 63, wave = tid >> 6;
    uint32_t acc = 0;
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
        const int base = ((it * 7 + wave * 3) & 3) * kRegion;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if constexpr (MODE == 0) {
                // 16 bytes per lane, 1 KiB per instruction: base + 15 KiB + 1008 + 16 <= 64 KiB
                const u32x4 v = *reinterpret_cast<const u32x4*>(lds + base + j * 1024 + lane * 16);
                acc = (acc ^ v.x) ^ (v.y + v.z + v.w);
            } else {
                // 8 bytes per lane, 512 bytes per instruction
                const tr4 r = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                    (__attribute__((address_space(3))) tr4*)(lds + base + j * 512 + lane * 8));
                const u32x2 v = __builtin_bit_cast(u32x2, r);
                acc = acc ^ (v.x + v.y);
            }
        }
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    out[size_t(blockIdx.x) * nt + tid] = acc ^ reinterpret_cast<const uint32_t*>(lds + kLdsBytes)[tid & 8191];
    if (blockIdx.x == 0 && tid == 0) {
        clk[0] = t1 - t0;
        clk[1] = r1 - r0;
    }
}

// kind 0: v_add_f32 (VOP2), 1: v_fma_f32 (VOP3), 2: v_exp_f32, 3: exp2 + add,
// 4: exp2 + add + mul (the add and mul chains independent of the exp2 one).
template <int KIND>
__global__ void valu_issue_probe(const float* __restrict__ in, float* __restrict__ out,
                                 unsigned long long* __restrict__ clk, int iters) {
    // 96 KiB of LDS, written and read once: one workgroup per CU.
    __shared__ float resv[24576];
    float x[16], z[16], w[16];
    const int t = threadIdx.x;
    for (int i = t; i < 24576; i += blockDim.x) resv[i] = in[i & 1023];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        x[i] = in[(t + i) & 1023] + 1e-30f * resv[(t * 7 + i) % 24576];
        z[i] = in[(t + 3 * i + 1) & 1023];
        w[i] = in[(t + 5 * i + 2) & 1023];
    }
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if constexpr (KIND == 0) x[i] = x[i] + z[i];
            if constexpr (KIND == 1) x[i] = __builtin_fmaf(x[i], z[i], w[i]);
            if constexpr (KIND == 2) x[i] = __builtin_amdgcn_exp2f(x[i]);
            if constexpr (KIND == 3) {
                x[i] = __builtin_amdgcn_exp2f(x[i]);
                z[i] = z[i] + w[i];
            }
            if constexpr (KIND == 4) {
                x[i] = __builtin_amdgcn_exp2f(x[i]);
                z[i] = z[i] + w[i];
                w[i] = w[i] * z[i];
            }
        }
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += x[i] + z[i] + w[i];
    out[size_t(blockIdx.x) * blockDim.x + t] = s;
    if ((t & 63) == 0) {
        const size_t wv = size_t(blockIdx.x) * (blockDim.x >> 6) + (t >> 6);
        clk[2 * wv] = t0;
        clk[2 * wv + 1] = t1;
    }
}

// Keeps a register value live and opaque at this point of the stream (no
// instruction is emitted), so loop-invariant operands are not hoisted and
// identical products are not merged.
template <typename T>
__device__ __forceinline__ void opaque(T& x) { asm volatile("" : "+v"(x)); }

constexpr int kModelLds = 98304;  // 96 KiB: one workgroup per CU

// Fills the step model's K/V buffer: random fp16 pairs in [-2, 2) (a
// multiply-xorshift hash of the index), or the smooth pattern 1e-3*(i%256)
// as fp32 words.
__global__ void step_model_fill(uint32_t* __restrict__ p, size_t n_words, int random) {
    for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n_words; i += size_t(gridDim.x) * blockDim.x) {
        if (random) {
            uint32_t h = uint32_t(i) * 0x9E3779B1u ^ uint32_t(i >> 32);
            h ^= h >> 15;
            h *= 0x85EBCA77u;
            h ^= h >> 13;
            h *= 0xC2B2AE3Du;
            h ^= h >> 16;
            const _Float16 lo = (_Float16)(float(h & 0xFFFFu) * (4.0f / 65536.0f) - 2.0f);
            const _Float16 hi = (_Float16)(float(h >> 16) * (4.0f / 65536.0f) - 2.0f);
            p[i] = uint32_t(__builtin_bit_cast(uint16_t, lo)) | (uint32_t(__builtin_bit_cast(uint16_t, hi)) << 16);
        } else {
            p[i] = __builtin_bit_cast(uint32_t, 1e-3f * float(i & 255));
        }
    }
}

// The per-tile shape of the step at head dim D, as in the forward: D/32
// output blocks of 32 dims, 4*(D/32) P V products (16-key steps x blocks)
// and 2*(D/16) S^T products (2 key blocks x 16-dim steps), one product per
// slot; LDS operand reads kAhead products ahead (the forward's choice: 5 at
// 8-wave d = 64, 3 at d = 128).  Softmax element pairs enter the three-stage
// chain (scaled score, exp2, row sum and fp16 P) in slots [kE0, kE1), with
// the forward's spread, so all three stages end inside the tile's slots.
template <int D>
struct ModelShape {
    static constexpr int kDBlocks = D / 32;
    static constexpr int kPV = 4 * kDBlocks;
    static constexpr int kS = 2 * (D / 16);
    static constexpr int kSlots = kPV + kS;
    static constexpr int kAhead = D == 64 ? 5 : 3;
    static constexpr int kE0 = kDBlocks > 2 ? kDBlocks - 2 : 0;
    static constexpr int kE1 = kSlots - 2;
    static constexpr int pair_begin(int p) {
        return p <= kE0 ? 0 : p >= kE1 ? 16 : ((p - kE0) * 16) / (kE1 - kE0);
    }
    // P chunk ks (pairs 4ks .. 4ks+3) is rewritten only after its last
    // reader, the P V product in slot kDBlocks*ks + kDBlocks-1.
    static constexpr bool schedule_ok() {
        for (int p = 0; p < kSlots; ++p)
            for (int j = pair_begin(p); j < pair_begin(p + 1); ++j)
                if (p + 2 <= kDBlocks * (j / 4) + kDBlocks - 1) return false;
        return pair_begin(kSlots) == 16;
    }
};

// MODE 0: MFMAs only; 1: S^T, softmax, P V in sequence; 2: the pipelined
// step in registers; 3: 2 with A operands from LDS; 4: 3 with a barrier
// every second tile; 5: 1 with A operands from LDS; 6: 4 with the next K/V
// tiles staged as the forward stages them (128-bit loads from `kv` into
// registers, 128-bit LDS stores one tile later); 7: 4 with the same tiles
// staged by direct global-to-LDS loads instead.  D = 64 or 128; W waves per
// SIMD (256*W threads, one workgroup per CU).  `kv` holds 32 K/V tile pairs
// per group of eight workgroups that share an XCD, as the 256-query
// workgroups of one (batch, head) at N = 2048 share them.  The instruction
// stream, its dependences and the memory traffic follow the forward; the
// values do not (no result is meaningful).  The operands come from `in` and
// `kv`: small smooth numbers, or random fp16 values in [-2, 2) like the
// forward's N(0, 1) inputs (the chip's clock under an MFMA load depends on
// how many operand bits toggle).
template <int MODE, int D, int W>
__global__ __launch_bounds__(256 * W) void step_model_probe(const float* __restrict__ in,
                                                           const unsigned char* __restrict__ kv,
                                                           float* __restrict__ out,
                                                           unsigned long long* __restrict__ clk, int iters,
                                                           float c) {
    using M = ModelShape<D>;
    static_assert(M::schedule_ok(), "P chunk rewritten before its last reader");
    constexpr int kTile = 64 * D * 2;  // bytes of one K or V tile
    __shared__ __attribute__((aligned(16))) unsigned char lds[kModelLds];
    // Staged K/V tiles (modes 6, 7) land in an LDS object of their own: the
    // compiler then knows the direct loads cannot alias the operand reads and
    // waits for them only where asked (a ring of per-tile LDS objects would
    // give a kernel the same).
    __shared__ __attribute__((aligned(16))) unsigned char stage[MODE >= 6 ? 2 * kTile : 16];
    const int t = threadIdx.x, lane = t & 63;
    // Operand tiles: K at [0, 2 kTile) and V at [2 kTile, 4 kTile), two
    // tiles each (by tile parity), copied from the start of `kv`; the rest
    // only reserves the CU.
    for (int i = t; i < kTile; i += blockDim.x)
        reinterpret_cast<float*>(lds)[i] = reinterpret_cast<const float*>(kv)[i];
    h8 ak[2], av[2], qf[D / 16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        ak[0][i] = (_Float16)in[(t + i) & 1023];
        ak[1][i] = (_Float16)in[(t + 5 * i + 1) & 1023];
        av[0][i] = (_Float16)in[(t + 7 * i) & 1023];
        av[1][i] = (_Float16)in[(t + 9 * i + 2) & 1023];
#pragma unroll
        for (int j = 0; j < D / 16; ++j) qf[j][i] = (_Float16)in[(t + 3 * i + 11 * j) & 1023];
    }
    auto opaque_operands = [&]() {
        opaque(ak[0]); opaque(ak[1]); opaque(av[0]); opaque(av[1]);
#pragma unroll
        for (int j = 0; j < D / 16; ++j) opaque(qf[j]);
    };
    // A operand of S^T product (key block kb, dim step ds) and of P V
    // product (key step ks, output block db) of tile `par`: from registers
    // (modes 0-2) or from LDS (K: one 16-byte read per lane; V: two
    // transposing reads; 1 KiB per wave, consecutive lane segments).
    auto k_op = [&](int par, int kb, int ds) {
        if constexpr (MODE >= 3)
            return *reinterpret_cast<const h8*>(lds + par * kTile + (2 * ds + kb) * 1024 + lane * 16);
        else
            return ak[kb];
    };
    auto v_op = [&](int par, int ks, int db) {
        if constexpr (MODE >= 3) {
            const unsigned char* v = lds + (2 + par) * kTile + (M::kDBlocks * ks + db) * 1024 + lane * 8;
            const tr4 a = __builtin_amdgcn_ds_read_tr16_b64_v4f16((__attribute__((address_space(3))) tr4*)(v));
            const tr4 b = __builtin_amdgcn_ds_read_tr16_b64_v4f16((__attribute__((address_space(3))) tr4*)(v + 512));
            return __builtin_bit_cast(h8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
            return av[db & 1];
        }
    };
    f32x16 oacc[M::kDBlocks] = {};
    f32x16 s[2][2] = {};
    h8 pf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) pf[j] = av[j & 1];
    float m = 1.0f, lsum = 0.f;
    __syncthreads();
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    if constexpr (MODE == 0) {
        for (int it = 0; it < iters; ++it) {
            opaque_operands();
#pragma unroll
            for (int ds = 0; ds < D / 16; ++ds) {
                s[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ak[0], qf[ds], s[0][0], 0, 0, 0);
                s[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ak[1], qf[ds], s[0][1], 0, 0, 0);
            }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int db = 0; db < M::kDBlocks; ++db)
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[db & 1], pf[ks], oacc[db], 0, 0, 0);
        }
    } else if constexpr (MODE == 1 || MODE == 5) {
        for (int it = 0; it < iters; ++it) {
            opaque_operands();
            const int par = it & 1;
            f32x16 sc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(k_op(par, kb, 0), qf[0], f32x16{}, 0, 0, 0);
#pragma unroll
                for (int ds = 1; ds < D / 16; ++ds)
                    sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(k_op(par, kb, ds), qf[ds], sc[kb], 0, 0, 0);
            }
            float rs[4];
#pragma unroll
            for (int e = 0; e < 32; ++e) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e >> 4][e & 15], c, -m));
                rs[e & 3] = e < 4 ? p : rs[e & 3] + p;
                pf[e >> 3][e & 7] = (_Float16)p;
            }
            const float tot = (rs[0] + rs[1]) + (rs[2] + rs[3]);
            lsum += tot;
            m = tot > 256.f ? m + 1.f : m;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int db = 0; db < M::kDBlocks; ++db)
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(v_op(par, ks, db), pf[ks], oacc[db], 0, 0, 0);
        }
    } else {
        // Slot p of a tile: product p (p < kPV: P V with P of the previous
        // tile; then S^T of the next tile), then the three-stage softmax
        // chain on this tile's S^T: the pairs entering now get their scaled
        // score, those that entered one slot ago their exp2, those of two
        // slots ago go to the row sum and to fp16 P.
        constexpr bool kFromLds = MODE >= 3;
        constexpr int kA = M::kAhead;
        // K/V staging (modes 6, 7): each wave moves kN KiB of the workgroup's
        // 2*kTile bytes per tile, one 1 KiB instruction at a time.
        constexpr int kN = 2 * kTile / (1024 * 4 * W);
        const int wave = t >> 6;
        const unsigned char* src = kv + size_t((blockIdx.x & 7) + 8 * (blockIdx.x >> 6)) * 32 * 2 * kTile +
                                   wave * kN * 1024 + lane * 16;
        unsigned char* dst = stage + wave * kN * 1024;
        h8 st[kN];
#pragma unroll
        for (int i = 0; i < kN; ++i) st[i] = ak[i & 1];
        float arg[32], pe[32], rs[4];
        h8 ring[kA + 1];
        // One tile of parity PAR (a template parameter, so that S^T's two
        // register buffers are never indexed at run time).
        auto tile = [&](auto par_tag, int it) {
            constexpr int par = decltype(par_tag)::value;
            {
                opaque_operands();
                f32x16* scur = s[par];
                f32x16* snext = s[par ^ 1];
                auto operand = [&](int q) {
                    if (q < M::kPV) return v_op(par, q / M::kDBlocks, q % M::kDBlocks);
                    const int j = q - M::kPV;
                    return k_op(par ^ 1, j & 1, j >> 1);
                };
                auto pb = [&](int q) { return q < 0 ? 0 : M::pair_begin(q); };
                if constexpr (kFromLds) {
#pragma unroll
                    for (int q = 0; q < kA; ++q) ring[q % (kA + 1)] = operand(q);
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int p = 0; p < M::kSlots; ++p) {
                    if constexpr (kFromLds) {
                        if (p + kA < M::kSlots) ring[(p + kA) % (kA + 1)] = operand(p + kA);
                    }
                    if constexpr (MODE == 6) {
                        // as the forward: chunk i, loaded a tile ago, goes to LDS in
                        // slot 2i and its register is refilled in slot 2i + 1
                        if (p % 2 == 0 && p / 2 < kN)
                            *reinterpret_cast<h8*>(dst + (p / 2) * 1024 + lane * 16) = st[p / 2];
                        if (p % 2 == 1 && p / 2 < kN)
                            st[p / 2] = *reinterpret_cast<const h8*>(
                                src + size_t((it + par) & 31) * 2 * kTile + (p / 2) * 1024);
                    }
                    if constexpr (MODE == 7) {
                        if (p % 2 == 1 && p / 2 < kN)
                            __builtin_amdgcn_global_load_lds(
                                src + size_t((it + par) & 31) * 2 * kTile + (p / 2) * 1024,
                                (__attribute__((address_space(3))) void*)(dst + (p / 2) * 1024), 16, 0, 0);
                    }
                    const h8 a = kFromLds ? ring[p % (kA + 1)] : operand(p);
                    if (p < M::kPV) {
                        const int ks = p / M::kDBlocks, db = p % M::kDBlocks;
                        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[ks], oacc[db], 0, 0, 0);
                    } else {
                        const int j = p - M::kPV, ds = j >> 1, kb = j & 1;
                        snext[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            a, qf[ds], ds == 0 ? f32x16{} : snext[kb], 0, 0, 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int j = pb(p - 2); j < pb(p - 1); ++j) {
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const int e = 2 * j + h;
                            rs[e & 3] = e < 4 ? pe[e] : rs[e & 3] + pe[e];
                            pf[e >> 3][e & 7] = (_Float16)pe[e];
                            opaque(rs[e & 3]);
                        }
                        opaque(pf[j >> 2]);
                    }
#pragma unroll
                    for (int j = pb(p - 1); j < pb(p); ++j) {
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            pe[2 * j + h] = __builtin_amdgcn_exp2f(arg[2 * j + h]);
                            opaque(pe[2 * j + h]);
                        }
                    }
#pragma unroll
                    for (int j = pb(p); j < pb(p + 1); ++j) {
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const int e = 2 * j + h;
                            arg[e] = __builtin_fmaf(scur[e >> 4][e & 15], c, -m);
                            opaque(arg[e]);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                const float tot = (rs[0] + rs[1]) + (rs[2] + rs[3]);
                lsum += tot;
                m = tot > 256.f ? m + 1.f : m;
                if constexpr (MODE == 4) {
                    if (par == 1) __syncthreads();
                }
                if constexpr (MODE == 6) {
                    // LDS stores and reads done; the loads in flight may stay so
                    if (par == 1) {
                        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
                        __builtin_amdgcn_s_barrier();
                    }
                }
                if constexpr (MODE == 7) {
                    // the direct loads of the previous tile have landed; this tile's may stay in flight
                    if (par == 1) {
                        __builtin_amdgcn_s_waitcnt(0x0070 | kN);  // vmcnt(kN) lgkmcnt(0)
                        __builtin_amdgcn_s_barrier();
                    }
                }
            }
        };
        for (int it = 0; it < iters; it += 2) {
            tile(std::integral_constant<int, 0>{}, it);
            tile(std::integral_constant<int, 1>{}, it);
        }
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    // A real read of the LDS block keeps it allocated (and the CU reserved)
    // in every mode.
    float r = lsum + 1e-30f * reinterpret_cast<const float*>(lds)[t & 8191];
    if constexpr (MODE >= 6) {
        __syncthreads();
        r += 1e-30f * reinterpret_cast<const float*>(stage)[t];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        r += s[0][0][i] + s[0][1][i] + s[1][0][i] + s[1][1][i];
#pragma unroll
        for (int db = 0; db < M::kDBlocks; ++db) r += oacc[db][i];
    }
    out[size_t(blockIdx.x) * blockDim.x + t] = r;
    if (lane == 0) {
        const size_t wv = size_t(blockIdx.x) * (blockDim.x >> 6) + (t >> 6);
        clk[4 * wv] = t0;
        clk[4 * wv + 1] = t1;
        clk[4 * wv + 2] = r0;
        clk[4 * wv + 3] = r1;
    }
}

}  // namespace

// mode 0: ds_read_b128, mode 1: ds_read_b64_tr_b16.  `threads` per workgroup
// (a multiple of 64, at most 1024), `blocks` workgroups, `iters` loop trips,
// timed over `reps` launches after three untimed ones on the null stream.
// out[0] = ms per launch, out[1] = LDS bytes read per launch, out[2] = the
// shader clock in GHz seen by wave 0 of workgroup 0.  Returns 0, or the HIP
// error code (1 for invalid arguments).
extern "C" int fa2probe_lds_read(int mode, int threads, int blocks, int iters, int reps,
                                 double* out) {
    if (!out || (mode != 0 && mode != 1) || threads < 64 || threads > 1024 || threads % 64 ||
        blocks < 1 || iters < 1 || reps < 1)
        return 1;
    uint32_t* dout = nullptr;
    unsigned long long* dclk = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipError_t err = hipMalloc(&dout, sizeof(uint32_t) * size_t(blocks) * threads);
    if (err == hipSuccess) err = hipMalloc(&dclk, 2 * sizeof(unsigned long long));
    if (err == hipSuccess) err = hipEventCreate(&e0);
    if (err == hipSuccess) err = hipEventCreate(&e1);
    auto launch = [&]() {
        if (mode == 0)
            hipLaunchKernelGGL(lds_read_probe<0>, dim3(blocks), dim3(threads), 0, nullptr, dout, dclk, iters);
        else
            hipLaunchKernelGGL(lds_read_probe<1>, dim3(blocks), dim3(threads), 0, nullptr, dout, dclk, iters);
        return hipGetLastError();
    };
    for (int w = 0; w < 3 && err == hipSuccess; ++w) err = launch();
    if (err == hipSuccess) err = hipEventRecord(e0, nullptr);
    for (int r = 0; r < reps && err == hipSuccess; ++r) err = launch();
    if (err == hipSuccess) err = hipEventRecord(e1, nullptr);
    if (err == hipSuccess) err = hipEventSynchronize(e1);
    float ms = 0.f;
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, e0, e1);
    unsigned long long h[2] = {0, 0};
    if (err == hipSuccess) err = hipMemcpy(h, dclk, sizeof h, hipMemcpyDeviceToHost);
    if (err == hipSuccess) {
        out[0] = double(ms) / reps;
        out[1] = double(blocks) * (threads / 64) * double(iters) * 16.0 * (mode == 0 ? 1024.0 : 512.0);
        out[2] = h[1] ? double(h[0]) / (double(h[1]) / 100e6) / 1e9 : 0.0;
    }
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (dclk) (void)hipFree(dclk);
    if (dout) (void)hipFree(dout);
    return err == hipSuccess ? 0 : int(err);
}

// kind as valu_issue_probe; `threads` per workgroup (64 to 1024, whole
// waves), `blocks` workgroups, `iters` loop trips of 16 elements, after one
// untimed launch.  out[0] = shader-clock cycles per loop element per wave,
// the mean of the waves' own loop times (with several waves per SIMD the
// oldest runs ahead, so this mixes fast and starved waves); out[1] = cycles
// per element per SIMD: the longest loop among each workgroup's waves over
// the elements its waves issue per SIMD (threads / 256 waves when each
// workgroup fills one CU), mean over workgroups.  Returns 0, or the HIP
// error code (1 for invalid arguments).
extern "C" int fa2probe_valu_issue(int kind, int threads, int blocks, int iters, double* out) {
    if (!out || kind < 0 || kind > 4 || threads < 64 || threads > 1024 || threads % 64 ||
        blocks < 1 || iters < 1)
        return 1;
    const int wpb = threads / 64, waves = blocks * wpb;
    float* din = nullptr;
    float* dout = nullptr;
    unsigned long long* dclk = nullptr;
    hipError_t err = hipMalloc(&din, sizeof(float) * 1024);
    if (err == hipSuccess) err = hipMalloc(&dout, sizeof(float) * size_t(blocks) * threads);
    if (err == hipSuccess) err = hipMalloc(&dclk, 2 * sizeof(unsigned long long) * size_t(waves));
    float h_in[1024];
    for (int i = 0; i < 1024; ++i) h_in[i] = -1.0f - 0.001f * float(i);
    if (err == hipSuccess) err = hipMemcpy(din, h_in, sizeof h_in, hipMemcpyHostToDevice);
    for (int rep = 0; rep < 2 && err == hipSuccess; ++rep) {
        switch (kind) {
            case 0: hipLaunchKernelGGL(valu_issue_probe<0>, dim3(blocks), dim3(threads), 0, nullptr, din, dout, dclk, iters); break;
            case 1: hipLaunchKernelGGL(valu_issue_probe<1>, dim3(blocks), dim3(threads), 0, nullptr, din, dout, dclk, iters); break;
            case 2: hipLaunchKernelGGL(valu_issue_probe<2>, dim3(blocks), dim3(threads), 0, nullptr, din, dout, dclk, iters); break;
            case 3: hipLaunchKernelGGL(valu_issue_probe<3>, dim3(blocks), dim3(threads), 0, nullptr, din, dout, dclk, iters); break;
            default: hipLaunchKernelGGL(valu_issue_probe<4>, dim3(blocks), dim3(threads), 0, nullptr, din, dout, dclk, iters); break;
        }
        err = hipGetLastError();
        if (err == hipSuccess) err = hipDeviceSynchronize();
    }
    unsigned long long* h = nullptr;
    if (err == hipSuccess) {
        h = static_cast<unsigned long long*>(::operator new(2 * sizeof(unsigned long long) * size_t(waves)));
        err = hipMemcpy(h, dclk, 2 * sizeof(unsigned long long) * size_t(waves), hipMemcpyDeviceToHost);
    }
    if (err == hipSuccess) {
        const double elems = double(iters) * 16.0;
        double own = 0.0, span = 0.0;
        for (int b = 0; b < blocks; ++b) {
            unsigned long long longest = 0;
            for (int w = 0; w < wpb; ++w) {
                const unsigned long long d = h[2 * (size_t(b) * wpb + w) + 1] - h[2 * (size_t(b) * wpb + w)];
                own += double(d);
                longest = d > longest ? d : longest;
            }
            span += double(longest);
        }
        out[0] = own / waves / elems;
        out[1] = span / blocks / (elems * (threads / 256.0));
    }
    if (h) ::operator delete(h);
    if (dclk) (void)hipFree(dclk);
    if (dout) (void)hipFree(dout);
    if (din) (void)hipFree(din);
    return err == hipSuccess ? 0 : int(err);
}

namespace {
template <int MODE, int D, int W>
hipError_t launch_one(int blocks, const float* din, const unsigned char* kv, float* dout,
                      unsigned long long* dclk, int iters) {
    hipLaunchKernelGGL((step_model_probe<MODE, D, W>), dim3(blocks), dim3(256 * W), 0, nullptr, din, kv, dout,
                       dclk, iters, 0.18f);
    return hipGetLastError();
}
// Waves per SIMD each (mode, head dim) fits without spilling registers.
int step_model_max_waves(int mode, int d) {
    if (d == 64) return mode <= 1 ? 4 : (mode == 2 || mode == 5) ? 3 : 2;
    return mode <= 1 ? 3 : 2;
}
// The staging variants (modes 6 and 7) run at the forward's two waves per SIMD only.
int step_model_min_waves(int mode, int d) { return mode >= 6 || (d == 128 && mode == 4) ? 2 : 1; }
template <int D>
hipError_t launch_step_model(int mode, int w, int blocks, const float* din, const unsigned char* kv, float* dout,
                             unsigned long long* dclk, int iters) {
    switch (mode * 8 + w) {
        case 0 * 8 + 1: return launch_one<0, D, 1>(blocks, din, kv, dout, dclk, iters);
        case 0 * 8 + 2: return launch_one<0, D, 2>(blocks, din, kv, dout, dclk, iters);
        case 0 * 8 + 3: return launch_one<0, D, 3>(blocks, din, kv, dout, dclk, iters);
        case 0 * 8 + 4:
            if constexpr (D == 64) return launch_one<0, D, 4>(blocks, din, kv, dout, dclk, iters);
            break;
        case 1 * 8 + 1: return launch_one<1, D, 1>(blocks, din, kv, dout, dclk, iters);
        case 1 * 8 + 2: return launch_one<1, D, 2>(blocks, din, kv, dout, dclk, iters);
        case 1 * 8 + 3: return launch_one<1, D, 3>(blocks, din, kv, dout, dclk, iters);
        case 1 * 8 + 4:
            if constexpr (D == 64) return launch_one<1, D, 4>(blocks, din, kv, dout, dclk, iters);
            break;
        case 2 * 8 + 1: return launch_one<2, D, 1>(blocks, din, kv, dout, dclk, iters);
        case 2 * 8 + 2: return launch_one<2, D, 2>(blocks, din, kv, dout, dclk, iters);
        case 2 * 8 + 3:
            if constexpr (D == 64) return launch_one<2, D, 3>(blocks, din, kv, dout, dclk, iters);
            break;
        case 3 * 8 + 1: return launch_one<3, D, 1>(blocks, din, kv, dout, dclk, iters);
        case 3 * 8 + 2: return launch_one<3, D, 2>(blocks, din, kv, dout, dclk, iters);
        case 4 * 8 + 1:
            // (at d = 128 the compiler moves part of this variant's private
            // arrays into LDS, which the model does not intend)
            if constexpr (D == 64) return launch_one<4, D, 1>(blocks, din, kv, dout, dclk, iters);
            break;
        case 4 * 8 + 2: return launch_one<4, D, 2>(blocks, din, kv, dout, dclk, iters);
        case 5 * 8 + 1: return launch_one<5, D, 1>(blocks, din, kv, dout, dclk, iters);
        case 5 * 8 + 2: return launch_one<5, D, 2>(blocks, din, kv, dout, dclk, iters);
        case 5 * 8 + 3:
            if constexpr (D == 64) return launch_one<5, D, 3>(blocks, din, kv, dout, dclk, iters);
            break;
        case 6 * 8 + 2: return launch_one<6, D, 2>(blocks, din, kv, dout, dclk, iters);
        case 7 * 8 + 2: return launch_one<7, D, 2>(blocks, din, kv, dout, dclk, iters);
        default: break;
    }
    return hipErrorInvalidValue;
}
}  // namespace

// The step model.  d = 64 or 128; mode 0..7 as step_model_probe; random 1
// for random fp16 operands in [-2, 2), 0 for small smooth ones; w waves per
// SIMD, from 1 to what the registers allow without spills (d = 64: 4 for
// modes 0 and 1, 3 for modes 2 and 5, 2 for modes 3 and 4; d = 128: 3 for
// modes 0 and 1, 2 otherwise), and exactly 2 for modes 6 and 7 and for
// mode 4 at d = 128; `blocks` workgroups of 256*w threads (one per CU at a
// time), `iters` key tiles per wave (even), timed over `reps` launches after
// one untimed.  out[0] = ms per launch; out[1] = TFLOP/s of the MFMA work
// (d/4 products of 32x32x16 per tile and wave); out[2] = the shader clock in
// GHz (shader-clock counter against the 100 MHz one, over all waves); out[3]
// = MFMA busy: 32 cycles per product, per SIMD, over the longest wave loop of
// each workgroup in shader cycles, mean over workgroups (last launch).
// Returns 0, or the HIP error code (1 for invalid arguments).
extern "C" int fa2probe_step_model(int d, int mode, int w, int random, int blocks, int iters, int reps,
                                   double* out) {
    if (!out || (d != 64 && d != 128) || mode < 0 || mode > 7 || w < step_model_min_waves(mode, d) ||
        w > step_model_max_waves(mode, d) || (random != 0 && random != 1) || blocks < 1 || iters < 2 ||
        iters % 2 || reps < 1)
        return 1;
    const int wpb = 4 * w, waves = blocks * wpb, per_tile = d / 4;
    // 32 K/V tile pairs (64 keys x d, fp16, K then V) per group of eight workgroups
    const size_t kv_bytes = size_t(8 * ((blocks + 63) / 64)) * 32 * 2 * (64 * d * 2);
    float* din = nullptr;
    float* dout = nullptr;
    unsigned char* kv = nullptr;
    unsigned long long* dclk = nullptr;
    auto launch = [&]() {
        return d == 64 ? launch_step_model<64>(mode, w, blocks, din, kv, dout, dclk, iters)
                       : launch_step_model<128>(mode, w, blocks, din, kv, dout, dclk, iters);
    };
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipError_t err = hipMalloc(&din, sizeof(float) * 1024);
    if (err == hipSuccess) err = hipMalloc(&kv, kv_bytes);
    if (err == hipSuccess) {
        hipLaunchKernelGGL(step_model_fill, dim3(1024), dim3(256), 0, nullptr, reinterpret_cast<uint32_t*>(kv),
                           kv_bytes / 4, random);
        err = hipGetLastError();
    }
    if (err == hipSuccess) err = hipMalloc(&dout, sizeof(float) * size_t(blocks) * 256 * w);
    if (err == hipSuccess) err = hipMalloc(&dclk, 4 * sizeof(unsigned long long) * size_t(waves));
    if (err == hipSuccess) err = hipEventCreate(&e0);
    if (err == hipSuccess) err = hipEventCreate(&e1);
    float h_in[1024];
    uint32_t lcg = 12345u;
    for (int i = 0; i < 1024; ++i) {
        lcg = lcg * 1664525u + 1013904223u;
        h_in[i] = random ? float(lcg >> 8) * (4.0f / 16777216.0f) - 2.0f : 0.01f * (1.0f - 0.002f * float(i));
    }
    if (err == hipSuccess) err = hipMemcpy(din, h_in, sizeof h_in, hipMemcpyHostToDevice);
    if (err == hipSuccess) err = launch();
    if (err == hipSuccess) err = hipDeviceSynchronize();
    if (err == hipSuccess) err = hipEventRecord(e0, nullptr);
    for (int r = 0; r < reps && err == hipSuccess; ++r) err = launch();
    if (err == hipSuccess) err = hipEventRecord(e1, nullptr);
    if (err == hipSuccess) err = hipEventSynchronize(e1);
    float ms = 0.f;
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, e0, e1);
    unsigned long long* h = nullptr;
    if (err == hipSuccess) {
        h = static_cast<unsigned long long*>(::operator new(4 * sizeof(unsigned long long) * size_t(waves)));
        err = hipMemcpy(h, dclk, 4 * sizeof(unsigned long long) * size_t(waves), hipMemcpyDeviceToHost);
    }
    if (err == hipSuccess) {
        double cyc = 0.0, real = 0.0, busy = 0.0;
        for (int b = 0; b < blocks; ++b) {
            unsigned long long longest = 0;
            for (int i = 0; i < wpb; ++i) {
                const unsigned long long* c = h + 4 * (size_t(b) * wpb + i);
                cyc += double(c[1] - c[0]);
                real += double(c[3] - c[2]);
                longest = c[1] - c[0] > longest ? c[1] - c[0] : longest;
            }
            busy += double(w) * iters * per_tile * 32.0 / double(longest);
        }
        out[0] = double(ms) / reps;
        out[1] = double(waves) * iters * per_tile * 32768.0 / (out[0] * 1e-3) / 1e12;
        out[2] = real > 0.0 ? cyc / (real / 100e6) / 1e9 : 0.0;
        out[3] = busy / blocks;
    }
    if (h) ::operator delete(h);
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (dclk) (void)hipFree(dclk);
    if (dout) (void)hipFree(dout);
    if (kv) (void)hipFree(kv);
    if (din) (void)hipFree(din);
    return err == hipSuccess ? 0 : int(err);
}
