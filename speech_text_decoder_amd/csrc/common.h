// common.h - device helpers shared by the gfx950 kernels of the decoder block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define WAVE 64

// ------------------------------------------------------------ conversions
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    __bf16 h = (__bf16)f;  // round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
    return __builtin_bit_cast(uint16_t, h);
}

// v = hi + lo to about 16 significant bits: hi = bf16(v), lo = bf16(v - hi).
__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
    hi = f32_to_bf16_bits(v);
    lo = f32_to_bf16_bits(v - bf16_bits_to_f32(hi));
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// Storage-type tags: loads widen to fp32, stores round to nearest even.
struct F32 {
    typedef float T;
    static __device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ void st(float* p, int64_t i, float v) { p[i] = v; }
    static __device__ __forceinline__ float cvt(float v) { return v; }
};
struct BF16 {
    typedef uint16_t T;
    static __device__ __forceinline__ float ld(const uint16_t* p, int64_t i) { return bf16_bits_to_f32(p[i]); }
    static __device__ __forceinline__ void st(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16_bits(v); }
    static __device__ __forceinline__ float cvt(uint16_t v) { return bf16_bits_to_f32(v); }
};
struct F16 {
    typedef uint16_t T;
    static __device__ __forceinline__ float ld(const uint16_t* p, int64_t i) { return f16_bits_to_f32(p[i]); }
    static __device__ __forceinline__ void st(uint16_t* p, int64_t i, float v) { p[i] = f32_to_f16_bits(v); }
    static __device__ __forceinline__ float cvt(uint16_t v) { return f16_bits_to_f32(v); }
};

// 8 consecutive elements widened to fp32 (16-byte or 2x16-byte aligned loads).
__device__ __forceinline__ void load8(const uint16_t* p, float* o /*[8]*/, BF16) {
    u32x4 u = *reinterpret_cast<const u32x4*>(p);
    o[0] = __uint_as_float(u.x << 16); o[1] = __uint_as_float(u.x & 0xFFFF0000u);
    o[2] = __uint_as_float(u.y << 16); o[3] = __uint_as_float(u.y & 0xFFFF0000u);
    o[4] = __uint_as_float(u.z << 16); o[5] = __uint_as_float(u.z & 0xFFFF0000u);
    o[6] = __uint_as_float(u.w << 16); o[7] = __uint_as_float(u.w & 0xFFFF0000u);
}
__device__ __forceinline__ void load8(const uint16_t* p, float* o, F16) {
    u32x4 u = *reinterpret_cast<const u32x4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = f16_bits_to_f32((uint16_t)(w[i] & 0xFFFFu));
        o[2 * i + 1] = f16_bits_to_f32((uint16_t)(w[i] >> 16));
    }
}
__device__ __forceinline__ void load8(const float* p, float* o, F32) {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

// Access policies for fp32 data exchanged between workgroups. PlainMem uses
// ordinary loads and stores. PubMem ("publish") uses ordinary loads but
// device-scope relaxed atomic stores (sc1 on gfx950), which write through the
// writer's L2 to memory. The attention splits publish their partial records
// this way, wait for the stores to complete, then count themselves in; the last
// one of a (row, KV head) reads them all with device-scope loads and merges them.
struct PlainMem {
    static __device__ __forceinline__ float ld(const float* p) { return *p; }
    static __device__ __forceinline__ void ld8(const float* p, float* o) { load8(p, o, F32()); }
    static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
};
struct PubMem {
    static __device__ __forceinline__ float ld(const float* p) { return *p; }
    static __device__ __forceinline__ void ld8(const float* p, float* o) { load8(p, o, F32()); }
    static __device__ __forceinline__ void st(float* p, float v) {
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
};

// ------------------------------------------------------------ reductions
// Cross-lane moves stay in the VALU (no LDS round trip). Inside a 16-lane row,
// DPP: row_mirror pairs lane i with 15 - i, row_half_mirror i with 7 - i
// (within 8), quad_perm [2,3,0,1] i with i ^ 2 and [1,0,3,2] i with i ^ 1; each
// is a perfect matching that flips lane bit 3, 2, 1 and 0 respectively (the
// mirrors also flip the lower bits). Between rows, v_permlane16_swap and
// v_permlane32_swap (gfx950): with both operands the same register, result
// [0] holds the value of lane (l & ~16) (resp. ~32) and [1] that of lane
// (l | 16) (resp. | 32) - checked on the device.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
    return __builtin_amdgcn_update_dpp(0.f, v, CTRL, 0xF, 0xF, false);
}
constexpr int DPP_ROW_MIRROR = 0x140, DPP_ROW_HALF_MIRROR = 0x141, DPP_XOR2 = 0x4E, DPP_XOR1 = 0xB1;

__device__ __forceinline__ float xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
}
__device__ __forceinline__ float xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// Sum over the 8 (resp. 16) lanes of an aligned group; every lane gets it.
__device__ __forceinline__ float row8_sum(float v) {
    v += dpp_move<DPP_ROW_HALF_MIRROR>(v);
    v += dpp_move<DPP_XOR2>(v);
    v += dpp_move<DPP_XOR1>(v);
    return v;
}
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_move<DPP_ROW_MIRROR>(v);
    return row8_sum(v);
}

__device__ __forceinline__ float wave_sum(float v) {
    v = row16_sum(v);
    v += xor16(v);
    v += xor32(v);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
    return v;
}

// Sum over a block of NW waves through LDS; every thread gets the result.
template <int NW>
__device__ __forceinline__ float block_sum(float v, float* lds /*[NW]*/) {
    v = wave_sum(v);
    const int lane = threadIdx.x % WAVE, w = threadIdx.x / WAVE;
    __syncthreads();
    if (lane == 0) lds[w] = v;
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) s += lds[i];
    return s;
}

// Order-preserving map of a float to uint32 (larger float -> larger key);
// NaN maps to 0 so that it never wins a maximum.
__device__ __forceinline__ uint32_t float_order_key(float f) {
    if (f != f) return 0u;
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ------------------------------------------------------------ device clock stamps
// Kernel timing that also works inside HIP graphs. A timed launch gets a slot
// of kClockEntries (start, end) pairs; thread 0 of each workgroup stores its
// start and end ticks of the 100 MHz device clock (s_memrealtime) in the pair
// of its linear workgroup id, with plain stores: same-address atomics from
// thousands of workgroups would serialise and slow the kernel being timed.
// Bank 0 holds ids below kClockBank1; bank 1 (a second kernel launched under
// the same slot, e.g. a finishing pass) holds the rest. Ids beyond a bank's
// size are not recorded.
__device__ __forceinline__ uint64_t* clock_entry(uint64_t* slot, int bank) {
    const uint32_t id = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const uint32_t cap = bank ? (uint32_t)(sttd::kClockEntries - sttd::kClockBank1) : (uint32_t)sttd::kClockBank1;
    return id < cap ? slot + 2 * (size_t)((bank ? sttd::kClockBank1 : 0) + id) : nullptr;
}
__device__ __forceinline__ void clock_begin(uint64_t* slot, int bank = 0) {
    if (slot && threadIdx.x == 0) {
        uint64_t* e = clock_entry(slot, bank);
        if (e) e[0] = wall_clock64();
    }
}
__device__ __forceinline__ void clock_end(uint64_t* slot, int bank = 0) {
    if (slot && threadIdx.x == 0) {
        uint64_t* e = clock_entry(slot, bank);
        if (e) e[1] = wall_clock64();
    }
}

// ------------------------------------------------------------ device error word
__device__ __forceinline__ void record_error(uint32_t* err, uint32_t bit) {
    if (err) atomicOr(err, bit);
}
