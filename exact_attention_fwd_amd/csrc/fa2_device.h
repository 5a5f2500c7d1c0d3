// Device-side building blocks shared by the gfx950 attention kernels (forward
// and backward): vector types, the two LDS tile layouts, the cross-lane pair
// reductions of the 32x32 MFMA accumulator, the transposing LDS read and
// buffer resources.  Internal; not installed.
//
// Accumulator layout of v_mfma_f32_32x32x16_f16 (measured on the GPU before
// the kernels relied on it): lane l, register r holds row
// 8*(r/4) + 4*(l/32) + r%4 and column l%32 of the 32x32 result.  The A
// operand gives lane l row l%32 and k-elements 8*(l/32) .. +7, the B operand
// column l%32 and the same k-elements.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa2 {
namespace dev {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef __fp16 tr4 __attribute__((vector_size(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kQW = 32;                  // rows (queries or keys) owned by one wave
constexpr int kBK = 64;                  // rows per LDS tile
constexpr int kRsrcFlags = 0x00020000;   // raw buffer, 32-bit data format
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// LDS tile layouts, both in 16-byte chunks (8 fp16 of one row):
//  chunk-major: chunk c of row r at (c * 64 + r) * 16.  A ds_read_b128
//     quarter-wave reads one chunk of 16 consecutive rows, 256 contiguous
//     bytes: every bank once.
//  swizzled: chunk-major with an XOR of the row, chunk c of row r at
//     (c * 64 + (r ^ 4 * (c & 3))) * 16.  A ds_read_b64_tr_b16 half-wave
//     reads 4 rows x 4 chunks; the XOR moves the 4 chunk planes (1 KiB
//     apart, so on the same banks) onto 4 different 64-byte bank windows.
//     Reads of 16 consecutive rows of one chunk stay one contiguous 256-byte
//     block (the XOR permutes rows inside it).
__device__ __forceinline__ int lds_k_off(int ch, int row) { return (ch * 64 + row) << 4; }
__device__ __forceinline__ int lds_v_off(int ch, int row) {
    return (ch * 64 + (row ^ ((ch & 3) << 2))) << 4;
}

// max / sum of x over the lane pair (l, l^32) that shares an accumulator column.
__device__ __forceinline__ float pair_max(float x) {
    auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// ds_read_b64_tr_b16: four consecutive rows of one fp16 column per lane.
__device__ __forceinline__ h4 lds_read_tr(const unsigned char* p) {
    tr4 r = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
        (__attribute__((address_space(3))) tr4*)(p));
    return __builtin_bit_cast(h4, r);
}

// Per-lane bases of the transposed A-operand reads (rows x 16 of k, k running
// over tile rows) from a swizzled tile: lane = 16*g + 4*e + cc reads rows
// 16*ks + 8*ab + 4*hi + e of columns 32*db + 16*(g&1) + 4*cc.  Chunk
// 4*db + tr_ch has (chunk & 3) == tr_ch, so the swizzle stays in the base
// and (ks, db) add the compile-time offset tr_imm(ks, db).  The 8 k-elements
// of lane half hi are then tile rows 16*ks + 8*(j/4) + 4*hi + j%4, j < 8:
// exactly the rows that the accumulator registers 8*kk .. 8*kk+7 of a
// 32-row block hold, so an accumulator can be reused as the B operand.
struct TrBase {
    int b0, b1;
    __device__ __forceinline__ explicit TrBase(int lane) {
        const int hi = lane >> 5;
        const int tr_g = lane >> 4, tr_e = (lane >> 2) & 3, tr_c = lane & 3;
        const int tr_ch = 2 * (tr_g & 1) + (tr_c >> 1);
        b0 = lds_v_off(tr_ch, 4 * hi + tr_e) + (tr_c & 1) * 8;
        b1 = lds_v_off(tr_ch, 8 + 4 * hi + tr_e) + (tr_c & 1) * 8;
    }
};
__device__ __forceinline__ constexpr int tr_imm(int ks, int db) { return ((4 * db) * 64 + 16 * ks) << 4; }
__device__ __forceinline__ h8 read_tr_operand(const unsigned char* tile, const TrBase& tb, int imm) {
    const h4 a = lds_read_tr(tile + tb.b0 + imm);
    const h4 b = lds_read_tr(tile + tb.b1 + imm);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcFlags);
}

// Keeps a value computed at this point of the instruction stream: the empty
// volatile asm reads and redefines it, so the computation can be neither sunk
// nor hoisted past the neighbouring scheduling barriers.
template <typename T>
__device__ __forceinline__ void pin(T& x) { asm volatile("" : "+v"(x)); }

// Workgroup id -> logical tile id: when the grid is a multiple of 8,
// consecutive logical ids (the tiles of one head) go to one XCD (dispatch is
// round-robin over the 8 XCDs), so they share that XCD's L2.
__device__ __forceinline__ int xcd_logical_id(int wg, int n_wg) {
    return (n_wg & 7) == 0 ? (wg & 7) * (n_wg >> 3) + (wg >> 3) : wg;
}

// (batch*head, tile rank) of a logical id when each head has n_tiles tiles
// and the tiles are dealt `group` heads at a time, rank-major inside each
// group (group 1: head by head).  The launch sizes the group (causal_group)
// so the workgroups an XCD runs together take the same rank of a few heads.
struct HeadTile {
    int bh, rank;
};
__device__ __forceinline__ HeadTile head_tile_of(int logical, int n_tiles, int group) {
    if (group > 1) {
        const int g0 = logical / (group * n_tiles);
        const int i = logical - g0 * group * n_tiles;
        const int rank = i / group;
        return {__builtin_amdgcn_readfirstlane(g0 * group + (i - rank * group)),
                __builtin_amdgcn_readfirstlane(rank)};
    }
    const int bh = __builtin_amdgcn_readfirstlane(logical / n_tiles);
    return {bh, __builtin_amdgcn_readfirstlane(logical - bh * n_tiles)};
}

}  // namespace dev
}  // namespace fa2
