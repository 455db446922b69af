// Internal helpers of the gfx950 MoE kernels (device types, bf16 rounding,
// tile constants and the per-minibatch layout record).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef int intx4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Grouped-GEMM tile: 256 x 256 output per workgroup of eight waves (two per
// SIMD), each wave owning a 64 x 128 block of 2 x 4 MFMA 32x32 fragments;
// the tile kernels are in gemm_tile.hpp (bf16) and mx_tile.hpp (MXFP8).
constexpr int BM = 256;
constexpr int BN = 256;
// Each expert's padded rows start on a kSegRows boundary.  An expert's M tiles
// are BM rows, except its last, which has kSegRows when the expert's remaining
// rows fit in it (a half tile: its second row of fragments is skipped), so an
// expert pads to a multiple of 128 rows instead of 256.
constexpr int kSegRows = 128;

// The gate/up weights are packed so that every 64 output columns of the
// first GEMM hold 32 gate columns followed by the 32 up columns with the same
// intermediate index; a wave's neighbouring 32-wide fragments then carry g and
// u of the same element and SwiGLU is applied in registers.
constexpr int kGluGroup = 64;

// Largest expert count (router output range) and k the kernels accept.
constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 16;

// Per-minibatch layout record written by the layout kernel and read by the
// GEMM and combine kernels.  Experts are the E routed experts plus, when the
// shared expert is on, one more "expert" E that takes every token in order.
struct LayoutHeader {
    int32_t m_tiles;  // total M tiles over all experts
    int32_t rows;     // routed rows (T_mb * k)
    int32_t error;    // non-zero: an expert index was out of range
    int32_t prows;    // padded rows over all experts (a multiple of kSegRows)
};

// One entry of a layout table (tile and row starts, row counts), which an
// earlier launch wrote and no kernel changes while it is read: a scalar load,
// so waiting for it does not wait for the vector loads and stores in flight.
__device__ __forceinline__ int32_t ld_layout(const int32_t* p) {
    return *(const __attribute__((address_space(4))) int32_t*)p;
}

// Rows of M tile ml of an expert whose padded rows run from seg0 to seg1:
// BM, or kSegRows for a last tile that is a half tile.
__host__ __device__ __forceinline__ int tile_rows_of(int seg0, int seg1, int ml) {
    const int left = seg1 - seg0 - ml * BM;
    return left < BM ? left : BM;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __builtin_bit_cast(float, (uint32_t)h << 16);
}

__host__ __device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_cvoid;
typedef int intx8 __attribute__((ext_vector_type(8)));

// Scheduling masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMFMA = 0x008, kSchedVMEM = 0x020, kSchedDSRead = 0x100;

}  // namespace moe
