// Device-side helpers shared by the gfx950 kernels of the quantized GEMV library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define QG_DEV __device__ __forceinline__

// Loads through the constant address space are selected as scalar (SMEM) loads
// whenever the address is wavefront-uniform: activation values shared by all 64
// rows of a wavefront land in SGPRs and feed the FMAs directly.
typedef const __attribute__((address_space(4))) float* qg_uniform_f32;

// Hide a value's bit pattern from the optimizer so that byte-wise conversions
// stay v_cvt_f32_ubyte{0..3} on the masked word instead of one bit-field extract
// per nibble.
QG_DEV uint32_t qg_opaque(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

QG_DEV float qg_ub0(uint32_t v) { return (float)(v & 0xffu); }
QG_DEV float qg_ub1(uint32_t v) { return (float)((v >> 8) & 0xffu); }
QG_DEV float qg_ub2(uint32_t v) { return (float)((v >> 16) & 0xffu); }
QG_DEV float qg_ub3(uint32_t v) { return (float)(v >> 24); }

QG_DEV float qg_half_lo(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu)); }
QG_DEV float qg_half_hi(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16)); }

QG_DEV float qg_readlane(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over each aligned group of 8 lanes; every lane of the group gets the same
// (bitwise identical) value.
QG_DEV float qg_sum8(float v) {
    v += __shfl_xor(v, 1, 64);
    v += __shfl_xor(v, 2, 64);
    v += __shfl_xor(v, 4, 64);
    return v;
}

// Sums of x over the eight 32-element sub-blocks of 256 activations: lane t holds
// x[4t..4t+3] (one float4 load, issued ahead of the weight loads it is consumed
// with so that waiting for it never waits for prefetched weights); lanes
// 8j..8j+7 cover sub-block j. Returns sub-block j's sum for j = 0..7 as
// wavefront-uniform values.
struct QgSub8 {
    float v[8];
};
QG_DEV float4 qg_x4(const float* __restrict__ xb, int lane) {
    return *reinterpret_cast<const float4*>(xb + 4 * lane);
}
QG_DEV QgSub8 qg_subblock_sums(const float4 xv) {
    float s = ((xv.x + xv.y) + xv.z) + xv.w;
    s = qg_sum8(s);
    QgSub8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r.v[j] = qg_readlane(s, 8 * j);
    return r;
}

// Q4_K 6-bit fields: four bytes of sub-scales / mins per word, as packed bytes.
//   sc[0..3] = low 6 bits of bytes 0..3, m[0..3] = low 6 bits of bytes 4..7,
//   sc[4..7] = low nibble of bytes 8..11 | top two bits of bytes 0..3 (as bits 4-5),
//   m[4..7]  = high nibble of bytes 8..11 | top two bits of bytes 4..7 (as bits 4-5).
struct QgScales {
    uint32_t sc03, sc47, m03, m47;
};
QG_DEV QgScales qg_q4k_scales(uint32_t s0, uint32_t s1, uint32_t s2) {
    QgScales r;
    r.sc03 = qg_opaque(s0 & 0x3f3f3f3fu);
    r.m03 = qg_opaque(s1 & 0x3f3f3f3fu);
    r.sc47 = qg_opaque((s2 & 0x0f0f0f0fu) | ((s0 >> 2) & 0x30303030u));
    r.m47 = qg_opaque(((s2 >> 4) & 0x0f0f0f0fu) | ((s1 >> 2) & 0x30303030u));
    return r;
}

// Agent-scope ticket: returns the counter's previous value (wavefront-uniform).
QG_DEV uint32_t qg_ticket(uint32_t* counter, int lane) {
    uint32_t old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)old);
}
QG_DEV void qg_ticket_reset(uint32_t* counter, int lane) {
    if (lane == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
