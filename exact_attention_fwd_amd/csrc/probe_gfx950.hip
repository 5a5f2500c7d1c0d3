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
// Wave 0 of workgroup 0 (LDS) or every wave (VALU) reads the shader clock
// counter around its loop; the LDS probe also reads the fixed 100 MHz
// counter, which gives the clock the CUs ran at.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __fp16 tr4 __attribute__((vector_size(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kLdsBytes = 65536;
constexpr int kRegion = 16384;   // four regions, a wave moves between them

template <int MODE>
__global__ void lds_read_probe(uint32_t* __restrict__ out, unsigned long long* __restrict__ clk,
                               int iters) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];
    const int tid = threadIdx.x, nt = blockDim.x;
    for (int i = tid; i < kLdsBytes / 4; i += nt)
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
    out[size_t(blockIdx.x) * nt + tid] = acc;
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
    float x[16], z[16], w[16];
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        x[i] = in[(t + i) & 1023];
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
    if ((t & 63) == 0) clk[size_t(blockIdx.x) * (blockDim.x >> 6) + (t >> 6)] = t1 - t0;
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
// untimed launch.  out[0] = shader-clock cycles per loop element per wave
// (averaged over every wave), out[1] = the same divided by the waves per
// SIMD (threads / 256 when each workgroup fills one CU).  Returns 0, or the
// HIP error code (1 for invalid arguments).
extern "C" int fa2probe_valu_issue(int kind, int threads, int blocks, int iters, double* out) {
    if (!out || kind < 0 || kind > 4 || threads < 64 || threads > 1024 || threads % 64 ||
        blocks < 1 || iters < 1)
        return 1;
    const int waves = blocks * (threads / 64);
    float* din = nullptr;
    float* dout = nullptr;
    unsigned long long* dclk = nullptr;
    hipError_t err = hipMalloc(&din, sizeof(float) * 1024);
    if (err == hipSuccess) err = hipMalloc(&dout, sizeof(float) * size_t(blocks) * threads);
    if (err == hipSuccess) err = hipMalloc(&dclk, sizeof(unsigned long long) * size_t(waves));
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
        h = static_cast<unsigned long long*>(::operator new(sizeof(unsigned long long) * size_t(waves)));
        err = hipMemcpy(h, dclk, sizeof(unsigned long long) * size_t(waves), hipMemcpyDeviceToHost);
    }
    if (err == hipSuccess) {
        double sum = 0.0;
        for (int i = 0; i < waves; ++i) sum += double(h[i]);
        const double per = sum / waves / (double(iters) * 16.0);
        out[0] = per;
        out[1] = per / (threads / 256.0);
    }
    if (h) ::operator delete(h);
    if (dclk) (void)hipFree(dclk);
    if (dout) (void)hipFree(dout);
    if (din) (void)hipFree(din);
    return err == hipSuccess ? 0 : int(err);
}
