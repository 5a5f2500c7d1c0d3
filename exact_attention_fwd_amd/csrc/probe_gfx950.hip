// Measurement probes for gfx950 (not part of the attention library's
// interface; bench.py --lds-probe and --valu-probe call them).
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
// A model of the forward's d = 64 key step.  step_model_probe runs, per
// wave, the MFMA work of one 64-key tile against 32 queries (8 S^T and 8 P V
// products of v_mfma_f32_32x32x16_f16) with the softmax VALU work between
// them, in variants that add the real kernel's parts one at a time: MFMAs
// alone; S^T, then softmax, then P V in sequence; the software pipeline of
// the forward (P V of tile t-1 and S^T of tile t+1 interleaved with tile t's
// softmax); the pipeline with its A operands read from LDS; that with a
// workgroup barrier every second tile; and the sequential step with its A
// operands read from LDS.  Nothing is loaded
// from HBM and no K/V tile is staged, so the rates are ceilings for the
// corresponding kernel design on this chip, its clock under that load
// included.
//
// Wave 0 of workgroup 0 (LDS) or every wave (VALU, step model) reads the
// shader clock counter around its loop; the LDS probe and the step model
// also read the fixed 100 MHz counter, which gives the clock the CUs ran at.
// Where several waves share a SIMD it does not serve them evenly (the
// oldest runs ahead and finishes first), so per-SIMD rates come from the
// longest loop among each workgroup's waves, which started together, not
// from the mean of the waves' loop times.  Only a wave's own start and end
// counter values are compared: start values that the waves of one
// workgroup read right after a barrier were seen far apart.

#include <hip/hip_runtime.h>
#include <stdint.h>

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
constexpr int kModelAhead = 5;    // LDS operand reads in flight (the forward's 8-wave d = 64 choice)

// MODE 0: MFMAs only; 1: S^T, softmax, P V in sequence; 2: the pipelined
// step in registers; 3: 2 with A operands from LDS; 4: 3 with a barrier
// every second tile; 5: 1 with A operands from LDS.  W waves per SIMD
// (256*W threads, one workgroup per CU).
// Operand values are arbitrary (small fp16 numbers); only the instruction
// stream and its dependences follow the forward.
template <int MODE, int W>
__global__ __launch_bounds__(256 * W) void step_model_probe(const float* __restrict__ in, float* __restrict__ out,
                                                           unsigned long long* __restrict__ clk, int iters,
                                                           float c) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[kModelLds];
    const int t = threadIdx.x, lane = t & 63;
    // 32 KiB of operand tiles: K at [0, 16 KiB) and V at [16, 32 KiB), two
    // 8 KiB tiles each (by tile parity); the rest only reserves the CU.
    for (int i = t; i < 8192; i += blockDim.x)
        reinterpret_cast<float*>(lds)[i] = 1e-3f * float(i & 255);
    h8 ak[2], av[2], qf[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        ak[0][i] = (_Float16)(in[(t + i) & 1023] * 0.01f);
        ak[1][i] = (_Float16)(in[(t + 5 * i + 1) & 1023] * 0.01f);
        av[0][i] = (_Float16)(in[(t + 7 * i) & 1023] * 0.01f);
        av[1][i] = (_Float16)(in[(t + 9 * i + 2) & 1023] * 0.01f);
#pragma unroll
        for (int j = 0; j < 4; ++j) qf[j][i] = (_Float16)(in[(t + 3 * i + 11 * j) & 1023] * 0.01f);
    }
    auto opaque_operands = [&]() {
        opaque(ak[0]); opaque(ak[1]); opaque(av[0]); opaque(av[1]);
        opaque(qf[0]); opaque(qf[1]); opaque(qf[2]); opaque(qf[3]);
    };
    f32x16 oacc[2] = {};
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
            for (int j = 0; j < 4; ++j) {
                s[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ak[0], qf[j], s[0][0], 0, 0, 0);
                s[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ak[1], qf[j], s[0][1], 0, 0, 0);
                oacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[0], pf[j], oacc[0], 0, 0, 0);
                oacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[1], pf[j], oacc[1], 0, 0, 0);
            }
        }
    } else if constexpr (MODE == 1 || MODE == 5) {
        for (int it = 0; it < iters; ++it) {
            opaque_operands();
            // MODE 5: the A operands from LDS, as in the pipelined variant
            // (K: one 16-byte read per lane; V: two transposing reads).
            const unsigned char* kt = lds + (it & 1) * 8192 + lane * 16;
            const unsigned char* vt = lds + 16384 + (it & 1) * 8192 + lane * 8;
            auto k_op = [&](int kb, int ds) {
                if constexpr (MODE == 5) return *reinterpret_cast<const h8*>(kt + (ds * 2 + kb) * 1024);
                else return ak[kb];
            };
            auto v_op = [&](int ks, int db) {
                if constexpr (MODE == 5) {
                    const tr4 a = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                        (__attribute__((address_space(3))) tr4*)(vt + (ks * 2 + db) * 1024));
                    const tr4 b = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                        (__attribute__((address_space(3))) tr4*)(vt + (ks * 2 + db) * 1024 + 512));
                    return __builtin_bit_cast(h8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
                } else {
                    return av[db];
                }
            };
            f32x16 sc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(k_op(kb, 0), qf[0], f32x16{}, 0, 0, 0);
#pragma unroll
                for (int ds = 1; ds < 4; ++ds)
                    sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(k_op(kb, ds), qf[ds], sc[kb], 0, 0, 0);
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
            for (int ks = 0; ks < 4; ++ks) {
                oacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(v_op(ks, 0), pf[ks], oacc[0], 0, 0, 0);
                oacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(v_op(ks, 1), pf[ks], oacc[1], 0, 0, 0);
            }
        }
    } else {
        // Slot p (0..17) of a tile: MFMA p (p < 8: P V with P of the previous
        // tile, 8..15: S^T of the next tile), then the three-stage softmax
        // chain on this tile's S^T: pair p enters (scaled score), pair p-1
        // takes exp2, pair p-2 goes to the row sum and to fp16 P.
        constexpr bool kFromLds = MODE >= 3;
        float arg[32], pe[32], rs[4];
        h8 ring[kModelAhead + 1];
        for (int it = 0; it < iters; it += 2) {
#pragma unroll
            for (int par = 0; par < 2; ++par) {
                opaque_operands();
                f32x16* scur = s[par];
                f32x16* snext = s[par ^ 1];
                // Operand q of this tile: q < 8 from a V tile (two transposing
                // reads, 1 KiB per wave), else from a K tile (one 16-byte read
                // per lane); consecutive lane segments, no bank conflicts.
                auto read = [&](int q) {
                    if (q < 8) {
                        const unsigned char* v = lds + 16384 + par * 8192 + q * 1024 + lane * 8;
                        const tr4 a = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                            (__attribute__((address_space(3))) tr4*)(v));
                        const tr4 b = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                            (__attribute__((address_space(3))) tr4*)(v + 512));
                        ring[q % (kModelAhead + 1)] =
                            __builtin_bit_cast(h8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
                    } else {
                        ring[q % (kModelAhead + 1)] =
                            *reinterpret_cast<const h8*>(lds + (par ^ 1) * 8192 + (q - 8) * 1024 + lane * 16);
                    }
                };
                if constexpr (kFromLds) {
#pragma unroll
                    for (int q = 0; q < kModelAhead; ++q) read(q);
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int p = 0; p < 18; ++p) {
                    if constexpr (kFromLds) {
                        if (p + kModelAhead < 16) read(p + kModelAhead);
                    }
                    if (p < 8) {
                        const int ks = p >> 1, db = p & 1;
                        const h8 a = kFromLds ? ring[p % (kModelAhead + 1)] : av[db];
                        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[ks], oacc[db], 0, 0, 0);
                    } else if (p < 16) {
                        const int j = p - 8, ds = j >> 1, kb = j & 1;
                        const h8 a = kFromLds ? ring[p % (kModelAhead + 1)] : ak[kb];
                        snext[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            a, qf[ds], ds == 0 ? f32x16{} : snext[kb], 0, 0, 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    if (p >= 2) {
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const int e = 2 * (p - 2) + h;
                            rs[e & 3] = e < 4 ? pe[e] : rs[e & 3] + pe[e];
                            pf[e >> 3][e & 7] = (_Float16)pe[e];
                            opaque(rs[e & 3]);
                        }
                        if ((p - 2) % 4 == 3) opaque(pf[(p - 2) >> 2]);
                    }
                    if (p >= 1 && p <= 16) {
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const int e = 2 * (p - 1) + h;
                            pe[e] = __builtin_amdgcn_exp2f(arg[e]);
                            opaque(pe[e]);
                        }
                    }
                    if (p < 16) {
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const int e = 2 * p + h;
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
            }
        }
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    // A real read of the LDS block keeps it allocated (and the CU reserved)
    // in every mode.
    float r = lsum + 1e-30f * reinterpret_cast<const float*>(lds)[t & 8191];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        r += oacc[0][i] + oacc[1][i] + s[0][0][i] + s[0][1][i] + s[1][0][i] + s[1][1][i];
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
template <int MODE, int W>
hipError_t launch_step_model(int blocks, const float* din, float* dout, unsigned long long* dclk, int iters) {
    hipLaunchKernelGGL((step_model_probe<MODE, W>), dim3(blocks), dim3(256 * W), 0, nullptr, din, dout, dclk,
                       iters, 0.18f);
    return hipGetLastError();
}
hipError_t launch_step_model(int mode, int w, int blocks, const float* din, float* dout, unsigned long long* dclk,
                             int iters) {
    switch (mode * 8 + w) {
        case 0 * 8 + 1: return launch_step_model<0, 1>(blocks, din, dout, dclk, iters);
        case 0 * 8 + 2: return launch_step_model<0, 2>(blocks, din, dout, dclk, iters);
        case 0 * 8 + 3: return launch_step_model<0, 3>(blocks, din, dout, dclk, iters);
        case 0 * 8 + 4: return launch_step_model<0, 4>(blocks, din, dout, dclk, iters);
        case 1 * 8 + 1: return launch_step_model<1, 1>(blocks, din, dout, dclk, iters);
        case 1 * 8 + 2: return launch_step_model<1, 2>(blocks, din, dout, dclk, iters);
        case 1 * 8 + 3: return launch_step_model<1, 3>(blocks, din, dout, dclk, iters);
        case 1 * 8 + 4: return launch_step_model<1, 4>(blocks, din, dout, dclk, iters);
        case 2 * 8 + 1: return launch_step_model<2, 1>(blocks, din, dout, dclk, iters);
        case 2 * 8 + 2: return launch_step_model<2, 2>(blocks, din, dout, dclk, iters);
        case 2 * 8 + 3: return launch_step_model<2, 3>(blocks, din, dout, dclk, iters);
        case 3 * 8 + 1: return launch_step_model<3, 1>(blocks, din, dout, dclk, iters);
        case 3 * 8 + 2: return launch_step_model<3, 2>(blocks, din, dout, dclk, iters);
        case 4 * 8 + 1: return launch_step_model<4, 1>(blocks, din, dout, dclk, iters);
        case 4 * 8 + 2: return launch_step_model<4, 2>(blocks, din, dout, dclk, iters);
        case 5 * 8 + 1: return launch_step_model<5, 1>(blocks, din, dout, dclk, iters);
        case 5 * 8 + 2: return launch_step_model<5, 2>(blocks, din, dout, dclk, iters);
        default: return launch_step_model<5, 3>(blocks, din, dout, dclk, iters);
    }
}
}  // namespace

// The step model.  mode 0..5 as step_model_probe; w waves per SIMD (1 to 4
// for modes 0 and 1, 1 to 3 for modes 2 and 5, 1 or 2 for modes 3 and 4:
// what the registers allow without spills); `blocks` workgroups of 256*w threads (one per CU at a
// time), `iters` key tiles per wave (even), timed over `reps` launches after
// one untimed.  out[0] = ms per launch; out[1] = TFLOP/s of the MFMA work
// (16 products of 32x32x16 per tile and wave); out[2] = the shader clock in
// GHz (shader-clock counter against the 100 MHz one, over all waves);
// out[3] = MFMA busy: 32 cycles per product, per SIMD, over the longest
// wave loop of each workgroup in shader cycles, mean over workgroups (last
// launch).  Returns 0,
// or the HIP error code (1 for invalid arguments).
extern "C" int fa2probe_step_model(int mode, int w, int blocks, int iters, int reps, double* out) {
    const int max_w = mode <= 1 ? 4 : (mode == 2 || mode == 5) ? 3 : 2;
    if (!out || mode < 0 || mode > 5 || w < 1 || w > max_w || blocks < 1 || iters < 2 || iters % 2 ||
        reps < 1)
        return 1;
    const int wpb = 4 * w, waves = blocks * wpb;
    float* din = nullptr;
    float* dout = nullptr;
    unsigned long long* dclk = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipError_t err = hipMalloc(&din, sizeof(float) * 1024);
    if (err == hipSuccess) err = hipMalloc(&dout, sizeof(float) * size_t(blocks) * 256 * w);
    if (err == hipSuccess) err = hipMalloc(&dclk, 4 * sizeof(unsigned long long) * size_t(waves));
    if (err == hipSuccess) err = hipEventCreate(&e0);
    if (err == hipSuccess) err = hipEventCreate(&e1);
    float h_in[1024];
    for (int i = 0; i < 1024; ++i) h_in[i] = 1.0f - 0.002f * float(i);
    if (err == hipSuccess) err = hipMemcpy(din, h_in, sizeof h_in, hipMemcpyHostToDevice);
    if (err == hipSuccess) err = launch_step_model(mode, w, blocks, din, dout, dclk, iters);
    if (err == hipSuccess) err = hipDeviceSynchronize();
    if (err == hipSuccess) err = hipEventRecord(e0, nullptr);
    for (int r = 0; r < reps && err == hipSuccess; ++r) err = launch_step_model(mode, w, blocks, din, dout, dclk, iters);
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
            busy += double(w) * iters * 16.0 * 32.0 / double(longest);
        }
        out[0] = double(ms) / reps;
        out[1] = double(waves) * iters * 16.0 * 32768.0 / (out[0] * 1e-3) / 1e12;
        out[2] = real > 0.0 ? cyc / (real / 100e6) / 1e9 : 0.0;
        out[3] = busy / blocks;
    }
    if (h) ::operator delete(h);
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (dclk) (void)hipFree(dclk);
    if (dout) (void)hipFree(dout);
    if (din) (void)hipFree(din);
    return err == hipSuccess ? 0 : int(err);
}
