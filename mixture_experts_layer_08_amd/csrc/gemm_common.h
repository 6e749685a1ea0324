// Building blocks shared by the grouped-GEMM kernels (forward products and
// their backward): tile constants, operand and vector types, the direct
// global->LDS load, raw buffer stores, buffer descriptors, LDS swizzles and
// the activation functions.  Included by one translation unit each; every
// definition lives in an unnamed namespace.
#pragma once

#include <math.h>

#include "moe_common.h"

typedef int moe_i32x4_t __attribute__((ext_vector_type(4)));

#ifndef GEMM_WAVES
#define GEMM_WAVES 8
#endif
#ifndef GEMM_WAVES_N
#define GEMM_WAVES_N 4
#endif
#ifndef GEMM_GROUP
#define GEMM_GROUP 32  // tiles per L2 group: every row tile of an expert x a few column tiles
#endif

// Raw buffer stores (the tile epilogue): the descriptor's byte range ends at
// the last valid row, and the hardware drops stores past it.
__device__ void buffer_store_i16(short v, moe_i32x4_t rsrc, int voffset, int soffset,
                                 int aux) __asm("llvm.amdgcn.raw.buffer.store.i16");
__device__ void buffer_store_f32(float v, moe_i32x4_t rsrc, int voffset, int soffset,
                                 int aux) __asm("llvm.amdgcn.raw.buffer.store.f32");
__device__ void buffer_store_f32x4(moe::f32x4_t v, moe_i32x4_t rsrc, int voffset, int soffset,
                                   int aux) __asm("llvm.amdgcn.raw.buffer.store.v4f32");
typedef int moe_i32x2_t __attribute__((ext_vector_type(2)));
__device__ void buffer_store_i32x2(moe_i32x2_t v, moe_i32x4_t rsrc, int voffset, int soffset,
                                   int aux) __asm("llvm.amdgcn.raw.buffer.store.v2i32");
__device__ moe_i32x2_t buffer_load_i32x2(moe_i32x4_t rsrc, int voffset, int soffset,
                                         int aux) __asm("llvm.amdgcn.raw.buffer.load.v2i32");
__device__ moe::f32x4_t buffer_load_f32x4(moe_i32x4_t rsrc, int voffset, int soffset,
                                         int aux) __asm("llvm.amdgcn.raw.buffer.load.v4f32");
typedef int moe_i32x8_t __attribute__((ext_vector_type(8)));
// Scalar buffer load of eight consecutive dwords (wave-uniform offset; dwords
// past the descriptor's range read as zero).  It is counted by lgkmcnt, not
// vmcnt, so waiting for it never waits for the vector loads and stores in
// flight.
__device__ moe_i32x8_t s_buffer_load_i32x8(moe_i32x4_t rsrc, int offset,
                                           int aux) __asm("llvm.amdgcn.s.buffer.load.v8i32");
// cache policy of a buffer access (aux): system scope (sc0 sc1), which goes
// past the per-XCD L2 caches to memory
constexpr int kAuxSystem = 17;

namespace {

using namespace moe;

constexpr int kBM = 256;
constexpr int kBNMax = 256;  // widest B tile (two 128-column sub-tiles)
constexpr int kBK = 64;
constexpr int kNW = GEMM_WAVES;      // waves per workgroup
constexpr int kWN = GEMM_WAVES_N;    // waves across the B columns
constexpr int kWMn = kNW / kWN;      // waves across the rows
constexpr int kGThreads = kNW * 64;
constexpr int kStageA = kBM * kBK * 2;  // 32 KB

enum { MODE_SWIGLU = 0, MODE_GELU = 1, MODE_DOWN = 2 };

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) uint32_t lds_u32_t;

// buffer_load_dwordx4 ... lds: each lane's 16 bytes go to LDS at M0 + 16 * lane.
// Written as asm so the compiler does not add a wait for these LDS writes
// before unrelated LDS reads of the other stage; the instruction has no
// register outputs, and the kernel itself waits (vmcnt(0)) and barriers
// before any wave reads the stage the loads fill.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is reserved; nothing else in these kernels uses it
__device__ __forceinline__ void lds_dma16(i32x4_t rsrc, const void* lds, int voffset, int soffset) {
    // every scalar operand is wave-uniform; readfirstlane states it to the compiler
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void_t*)lds);
    rsrc.x = __builtin_amdgcn_readfirstlane(rsrc.x);
    rsrc.y = __builtin_amdgcn_readfirstlane(rsrc.y);
    rsrc.z = __builtin_amdgcn_readfirstlane(rsrc.z);
    rsrc.w = __builtin_amdgcn_readfirstlane(rsrc.w);
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen lds"
        :
        : "s"(m0), "v"(voffset), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soffset))
        : "memory", "m0");
}
// The same with the LDS destination as a 32-bit LDS address (computed once
// per kernel from the shared array, so no generic-pointer conversion per load).
__device__ __forceinline__ void lds_dma16_at(i32x4_t rsrc, uint32_t lds_addr, int voffset, int soffset) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
    rsrc.x = __builtin_amdgcn_readfirstlane(rsrc.x);
    rsrc.y = __builtin_amdgcn_readfirstlane(rsrc.y);
    rsrc.z = __builtin_amdgcn_readfirstlane(rsrc.z);
    rsrc.w = __builtin_amdgcn_readfirstlane(rsrc.w);
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen lds"
        :
        : "s"(m0), "v"(voffset), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soffset))
        : "memory", "m0");
}
#pragma clang diagnostic pop

// Buffer resource: 48-bit base, no stride, num_records bytes; loads past the
// end return zero and stores past it are dropped.  Every argument must be
// wave-uniform.
__device__ __forceinline__ i32x4_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4_t r;
    r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF);
    r.z = __builtin_amdgcn_readfirstlane((int)bytes);
    r.w = 0x00020000;
    return r;
}

// silu(g) = g * sigmoid(g), the reciprocal from v_rcp_f32 (1 ulp): the
// products' outputs are rounded to bf16 or feed fp32 sums, where an IEEE
// division's last bit does not show.
__device__ __forceinline__ float silu_f(float g) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}
__device__ __forceinline__ float gelu_f(float z) {
    return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
}

// Exchange inside lane pairs (CTRL 0xB1: lanes XOR 1) or pairs of pairs
// (CTRL 0x4E: lanes XOR 2) by DPP quad permutes: the lower lane of a pair
// keeps a and receives the partner's a into b; the upper lane keeps b and
// receives the partner's b into a.
template <int CTRL>
__device__ __forceinline__ void quad_xchg(uint32_t& a, uint32_t& b, bool upper) {
    const uint32_t got = (uint32_t)__builtin_amdgcn_mov_dpp((int)(upper ? a : b), CTRL, 0xF, 0xF, false);
    if (upper)
        a = got;
    else
        b = got;
}

// Stores of four rows of an MFMA 32 x 32 accumulator: in lanes 4m .. 4m+3,
// v[0..3] hold rows r .. r+3 of column c0 + (lane & 3).  Two exchange rounds
// (lane bit 0 with row bit 0, then lane bit 1 with row bit 1) leave lane
// 4m + j with row r + j, columns c0 .. c0+3, written with one 8-byte (bf16)
// or 16-byte (fp32) store.  Every lane of each quad must be active.
__device__ __forceinline__ void store_rows4_bf16(const float (&v)[4], i32x4_t rs, int voff,
                                                 int soff, int lane) {
    uint32_t w0 = __float_as_uint(v[0]), w1 = __float_as_uint(v[1]);
    uint32_t w2 = __float_as_uint(v[2]), w3 = __float_as_uint(v[3]);
    quad_xchg<0xB1>(w0, w1, lane & 1);
    quad_xchg<0xB1>(w2, w3, lane & 1);
    uint32_t p0 = pack_bf2(__uint_as_float(w0), __uint_as_float(w1));
    uint32_t p1 = pack_bf2(__uint_as_float(w2), __uint_as_float(w3));
    quad_xchg<0x4E>(p0, p1, lane & 2);
    moe_i32x2_t o;
    o.x = (int)p0;
    o.y = (int)p1;
    buffer_store_i32x2(o, rs, voff, soff, 0);
}
// The transpose alone (fp32): v[0..3] = rows r .. r+3 of column c0 + (lane
// & 3) in, row r + (lane & 3), columns c0 .. c0+3 out.
__device__ __forceinline__ void quad_transpose_f32(float (&v)[4], int lane) {
    uint32_t w0 = __float_as_uint(v[0]), w1 = __float_as_uint(v[1]);
    uint32_t w2 = __float_as_uint(v[2]), w3 = __float_as_uint(v[3]);
    quad_xchg<0xB1>(w0, w1, lane & 1);
    quad_xchg<0xB1>(w2, w3, lane & 1);
    quad_xchg<0x4E>(w0, w2, lane & 2);
    quad_xchg<0x4E>(w1, w3, lane & 2);
    v[0] = __uint_as_float(w0);
    v[1] = __uint_as_float(w1);
    v[2] = __uint_as_float(w2);
    v[3] = __uint_as_float(w3);
}
template <int AUX = 0>
__device__ __forceinline__ void store_rows4_f32(const float (&vin)[4], i32x4_t rs, int voff,
                                                int soff, int lane) {
    float v[4] = {vin[0], vin[1], vin[2], vin[3]};
    quad_transpose_f32(v, lane);
    f32x4_t o;
    o.x = v[0];
    o.y = v[1];
    o.z = v[2];
    o.w = v[3];
    // The whole offset goes in the vector operand, soffset stays 0: with a
    // register soffset, the compiler let the next VALU write the store's data
    // registers at once, and the first dword of some lanes' stores then held
    // the new value (measured wrong outputs).  With soffset 0 it pads the
    // store with the wait state a 16-byte store needs.
    buffer_store_f32x4(o, rs, voff + soff, 0, AUX);
}

// LDS swizzles (16-byte chunk index XOR).  A rows are 128 bytes: XOR with
// (row >> 1) & 7 puts any 16 consecutive rows of one chunk on distinct banks.
// B rows (one 128-column sub-tile) are 256 bytes: a transpose read serves 32
// lanes per pass, lanes 0-15 and 16-31 reading the same 4 rows at columns 16
// apart; XOR with 4 * (k & 3) sends the two halves to disjoint chunk sets.
__device__ __forceinline__ int swz_a(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int swz_b(int k) { return (k & 3) << 2; }

// Tile `logical` -> expert and row / column tile.  Inside an expert, tiles
// run in groups of every row tile times gn column tiles (about GEMM_GROUP
// tiles), column-fastest, so one XCD's run of tiles shares A rows and B
// panels in its L2.
__device__ __forceinline__ void map_tile(int logical, const int* s_pref, const int* s_mt, int E,
                                         int NT, int& e, int& m_tile, int& n_tile) {
    e = 0;
    while (e + 1 < E && s_pref[e + 1] <= logical) ++e;
    const int local = logical - s_pref[e];
    const int mt = s_mt[e];
    int gn = GEMM_GROUP / mt;
    if (gn < 1) gn = 1;
    if (gn > NT) gn = NT;
    const int grp = local / (mt * gn);
    int width = NT - grp * gn;
    if (width > gn) width = gn;
    const int rem = local - grp * mt * gn;
    m_tile = rem / width;
    n_tile = grp * gn + rem % width;
}

// Compute units of the current device (the persistent grids' size).
inline int num_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return 256;
    return n;
}

}  // namespace
