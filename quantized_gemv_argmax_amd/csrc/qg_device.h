// Device-side helpers shared by the gfx950 kernels of the quantized GEMV library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define QG_DEV __device__ __forceinline__

// Rows per packed tile. Sixteen rows are one DPP row of a wavefront.
#define QG_TILE_ROWS 16

// Loads through the constant address space are selected as scalar (SMEM) loads
// whenever the address is wavefront-uniform.
typedef const __attribute__((address_space(4))) float* qg_uniform_f32;

// Weight loads: read once per call, so they are marked non-temporal (streamed
// past the caches) unless QG_TEMPORAL_WEIGHTS is defined.
QG_DEV uint4 qg_stream_load(const uint4* p) {
#ifdef QG_TEMPORAL_WEIGHTS
    return *p;
#else
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    const u4 v = __builtin_nontemporal_load(reinterpret_cast<const u4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
#endif
}

// Hide a value's bit pattern from the optimizer so that byte-wise conversions
// stay v_cvt_f32_ubyte{0..3} on the masked word.
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

// ---------------------------------------------------------------------------
// DPP row broadcast (row_newbcast:L): every lane of a 16-lane DPP row reads the
// operand of lane L of its own row. Used to share activation registers across the
// 16 weight rows a DPP row processes, at no instruction cost.
//
// Hazard rule on gfx9: a VGPR written by a VALU instruction needs two wait states
// before any DPP instruction reads it (through any operand, the accumulator of
// v_dot2c included). The compiler cannot see inside inline assembly, so the
// blocks below schedule their own instructions to respect it: every mask is
// computed at least two instructions before the dot product that reads it, each
// accumulator is re-read at least two instructions after its last write, and the
// activation pairs are produced by qg_cvt_pairs*, which end with s_nop 1.
// A v_dot2c result read by an ordinary VALU instruction two instructions after
// the DPP dot product was observed stale on gfx950, so each block ends with
// s_nop 4 before the compiler's own code reads the accumulators.

// Broadcast of lane L of this DPP row (compiler-tracked, hazards handled by it).
template <int L>
QG_DEV float qg_bcast(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + L, 0xf, 0xf, true));
}

// Q4_K: one 16-byte quant segment (4 dwords, 32 weights) against the activation
// pairs of lanes LA (dwords 0, 1) and LB (dwords 2, 3) of this DPP row. For each
// dword: low nibbles of bytes 0,2 / 1,3 go to lo0 / lo1 with pairs x[r+0] / x[r+1],
// high nibbles of bytes 0,2 / 1,3 go to hi0 / hi1 with pairs x[r+2] / x[r+3]
// (r = 0 for dwords 0 and 2, r = 4 for dwords 1 and 3). The nibbles are masked in
// place and read as fp16 subnormals (q * 2^-24, high ones 16q * 2^-24).
template <int LA, int LB>
QG_DEV void qg_q4_seg_dot(float& lo0, float& hi0, float& lo1, float& hi1, const uint4 q, const uint32_t (&x)[8]) {
    uint32_t m0, m1, m2, m3, m4, m5, m6, m7, t;
    asm("v_and_b32 %4, 0xf000f, %13\n\t"
        "v_and_b32 %5, 0xf000f0, %13\n\t"
        "v_lshrrev_b32 %12, 8, %13\n\t"
        "v_and_b32 %6, 0xf000f, %12\n\t"
        "v_and_b32 %7, 0xf000f0, %12\n\t"
        "v_and_b32 %8, 0xf000f, %14\n\t"
        "v_and_b32 %9, 0xf000f0, %14\n\t"
        "v_lshrrev_b32 %12, 8, %14\n\t"
        "v_and_b32 %10, 0xf000f, %12\n\t"
        "v_and_b32 %11, 0xf000f0, %12\n\t"
        "v_dot2c_f32_f16_dpp %0, %17, %4 row_newbcast:%25 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %1, %19, %5 row_newbcast:%25 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %2, %18, %6 row_newbcast:%25 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %3, %20, %7 row_newbcast:%25 row_mask:0xf bank_mask:0xf\n\t"
        "v_and_b32 %4, 0xf000f, %15\n\t"
        "v_and_b32 %5, 0xf000f0, %15\n\t"
        "v_lshrrev_b32 %12, 8, %15\n\t"
        "v_and_b32 %6, 0xf000f, %12\n\t"
        "v_and_b32 %7, 0xf000f0, %12\n\t"
        "v_dot2c_f32_f16_dpp %0, %21, %8 row_newbcast:%25 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %1, %23, %9 row_newbcast:%25 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %2, %22, %10 row_newbcast:%25 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %3, %24, %11 row_newbcast:%25 row_mask:0xf bank_mask:0xf\n\t"
        "v_and_b32 %8, 0xf000f, %16\n\t"
        "v_and_b32 %9, 0xf000f0, %16\n\t"
        "v_lshrrev_b32 %12, 8, %16\n\t"
        "v_and_b32 %10, 0xf000f, %12\n\t"
        "v_and_b32 %11, 0xf000f0, %12\n\t"
        "v_dot2c_f32_f16_dpp %0, %17, %4 row_newbcast:%26 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %1, %19, %5 row_newbcast:%26 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %2, %18, %6 row_newbcast:%26 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %3, %20, %7 row_newbcast:%26 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %0, %21, %8 row_newbcast:%26 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %1, %23, %9 row_newbcast:%26 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %2, %22, %10 row_newbcast:%26 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot2c_f32_f16_dpp %3, %24, %11 row_newbcast:%26 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 4"
        : "+v"(lo0), "+v"(hi0), "+v"(lo1), "+v"(hi1), "=&v"(m0), "=&v"(m1), "=&v"(m2), "=&v"(m3), "=&v"(m4),
          "=&v"(m5), "=&v"(m6), "=&v"(m7), "=&v"(t)
        : "v"(q.x), "v"(q.y), "v"(q.z), "v"(q.w), "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]),
          "v"(x[6]), "v"(x[7]), "n"(LA), "n"(LB));
}

// Eight fp16x2 pairs (round to nearest even) from four float4, in the order
// (a.x,a.z) (a.y,a.w) (b.x,b.z) (b.y,b.w) (c...) (d...), then two wait states.
struct QgPairs8 {
    uint32_t p[8];
};
QG_DEV QgPairs8 qg_cvt_pairs(const float4 a, const float4 b, const float4 c, const float4 d) {
    QgPairs8 r;
    asm volatile(
        "v_cvt_pk_f16_f32 %0, %8, %10\n\t"
        "v_cvt_pk_f16_f32 %1, %9, %11\n\t"
        "v_cvt_pk_f16_f32 %2, %12, %14\n\t"
        "v_cvt_pk_f16_f32 %3, %13, %15\n\t"
        "v_cvt_pk_f16_f32 %4, %16, %18\n\t"
        "v_cvt_pk_f16_f32 %5, %17, %19\n\t"
        "v_cvt_pk_f16_f32 %6, %20, %22\n\t"
        "v_cvt_pk_f16_f32 %7, %21, %23\n\t"
        "s_nop 1"
        : "=&v"(r.p[0]), "=&v"(r.p[1]), "=&v"(r.p[2]), "=&v"(r.p[3]), "=&v"(r.p[4]), "=&v"(r.p[5]),
          "=&v"(r.p[6]), "=&v"(r.p[7])
        : "v"(a.x), "v"(a.y), "v"(a.z), "v"(a.w), "v"(b.x), "v"(b.y), "v"(b.z), "v"(b.w), "v"(c.x), "v"(c.y),
          "v"(c.z), "v"(c.w), "v"(d.x), "v"(d.y), "v"(d.z), "v"(d.w));
    return r;
}

// Four fp16x2 pairs from two float4: (a.x,a.z) (a.y,a.w) (b.x,b.z) (b.y,b.w),
// then two wait states.
struct QgPairs4 {
    uint32_t p[4];
};
QG_DEV QgPairs4 qg_cvt_pairs4(const float4 a, const float4 b) {
    QgPairs4 r;
    asm volatile(
        "v_cvt_pk_f16_f32 %0, %4, %6\n\t"
        "v_cvt_pk_f16_f32 %1, %5, %7\n\t"
        "v_cvt_pk_f16_f32 %2, %8, %10\n\t"
        "v_cvt_pk_f16_f32 %3, %9, %11\n\t"
        "s_nop 1"
        : "=&v"(r.p[0]), "=&v"(r.p[1]), "=&v"(r.p[2]), "=&v"(r.p[3])
        : "v"(a.x), "v"(a.y), "v"(a.z), "v"(a.w), "v"(b.x), "v"(b.y), "v"(b.z), "v"(b.w));
    return r;
}

// Sum over each quad of lanes (all four lanes get the same value).
QG_DEV float qg_quad_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xb1, 0xf, 0xf, true));  // [1,0,3,2]
    return v + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4e, 0xf, 0xf, true));  // [2,3,0,1]
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

// Sum of a value over the four DPP rows (lanes i, i+16, i+32, i+48).
QG_DEV float qg_sum_rows4(float v) {
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}

// ---------------------------------------------------------------------------
// fp16 matrix-core operands (v_mfma_f32_16x16x32_f16: lane l holds
// A[l % 16][8 (l / 16) + 0..7], B[8 (l / 16) + 0..7][l % 16] and
// D[4 (l / 16) + e][l % 16], e = 0..3).
typedef _Float16 qg_h8 __attribute__((ext_vector_type(8)));
typedef _Float16 qg_h2 __attribute__((ext_vector_type(2)));
typedef float qg_f4 __attribute__((ext_vector_type(4)));
typedef unsigned int qg_u4v __attribute__((ext_vector_type(4)));
typedef unsigned int qg_u2v __attribute__((ext_vector_type(2)));

// Sum of the eight fp16 values held in four packed pairs, in fp32 and a fixed
// order (a, b, c, d): each step is one v_dot2_f32_f16 against (1, 1), which adds
// both halves of a pair to the running sum. Used for the per-block activation
// sums, so that they are taken over exactly the values the dot products use.
QG_DEV float qg_sum_pairs4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const qg_h2 one = {(_Float16)1.0f, (_Float16)1.0f};
    float s = __builtin_amdgcn_fdot2(__builtin_bit_cast(qg_h2, a), one, 0.0f, false);
    s = __builtin_amdgcn_fdot2(__builtin_bit_cast(qg_h2, b), one, s, false);
    s = __builtin_amdgcn_fdot2(__builtin_bit_cast(qg_h2, c), one, s, false);
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(qg_h2, d), one, s, false);
}

// Q8_0 quant segments (16 int8 quants q) as signed fp16 subnormals q * 2^-24,
// two per word: per dword, the quants are biased to bytes (q ^ 0x80 = q + 128),
// bytes 0, 2 and then 1, 3 are moved into the low bytes of the two halves by one
// byte permutation each (selector byte 0x0c gives a zero byte), and one packed
// fp16 addition of -128 * 2^-24 (bits 0x8080) to both halves takes the bias off
// exactly, (q + 128) * 2^-24 - 128 * 2^-24 = q * 2^-24 being representable. So
// no activation sum is needed to remove a bias, and a product of the signed
// quants with the fp16 activations is exact: per dword 5 operations for 4
// weights. m[2d] holds bytes 0, 2 of dword d, m[2d + 1] bytes 1, 3.
QG_DEV uint32_t qg_f16x2_add(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(qg_h2, a) + __builtin_bit_cast(qg_h2, b));
}
QG_DEV void qg_q8_signed_masks(uint32_t (&m)[8], const uint4 q) {
    const uint32_t w[4] = {q.x ^ 0x80808080u, q.y ^ 0x80808080u, q.z ^ 0x80808080u, q.w ^ 0x80808080u};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        m[2 * d] = qg_f16x2_add(__builtin_amdgcn_perm(w[d], w[d], 0x0c020c00u), 0x80808080u);
        m[2 * d + 1] = qg_f16x2_add(__builtin_amdgcn_perm(w[d], w[d], 0x0c030c01u), 0x80808080u);
    }
}

// One Q8_0 quant segment of 16 weights: masked words m (2d: bytes 0, 2 of dword
// d; 2d + 1: bytes 1, 3) against the activation pairs x = ((x0, x2), (x1, x3),
// (x4, x6), (x5, x7)) of lane LA (dwords 0, 1) and lane LA + 1 (dwords 2, 3) of
// this DPP row. Opens with two wait states (masks and accumulators come from
// ordinary VALU code); TAIL blocks end with s_nop 4 before ordinary VALU code
// reads the accumulators.
#define QG_SEG8H_TEXT \
    "s_nop 1\n\t" \
    "v_dot2c_f32_f16_dpp %0, %12, %4 row_newbcast:%16 row_mask:0xf bank_mask:0xf\n\t" \
    "v_dot2c_f32_f16_dpp %1, %13, %5 row_newbcast:%16 row_mask:0xf bank_mask:0xf\n\t" \
    "v_dot2c_f32_f16_dpp %2, %14, %6 row_newbcast:%16 row_mask:0xf bank_mask:0xf\n\t" \
    "v_dot2c_f32_f16_dpp %3, %15, %7 row_newbcast:%16 row_mask:0xf bank_mask:0xf\n\t" \
    "v_dot2c_f32_f16_dpp %0, %12, %8 row_newbcast:%17 row_mask:0xf bank_mask:0xf\n\t" \
    "v_dot2c_f32_f16_dpp %1, %13, %9 row_newbcast:%17 row_mask:0xf bank_mask:0xf\n\t" \
    "v_dot2c_f32_f16_dpp %2, %14, %10 row_newbcast:%17 row_mask:0xf bank_mask:0xf\n\t" \
    "v_dot2c_f32_f16_dpp %3, %15, %11 row_newbcast:%17 row_mask:0xf bank_mask:0xf\n\t"
template <int LA, bool TAIL>
QG_DEV void qg_q8_seg8h_dot(float (&a)[4], const uint32_t (&m)[8], const uint4 x) {
    if constexpr (TAIL)
        asm(QG_SEG8H_TEXT "s_nop 4"
            : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3])
            : "v"(m[0]), "v"(m[1]), "v"(m[2]), "v"(m[3]), "v"(m[4]), "v"(m[5]), "v"(m[6]), "v"(m[7]), "v"(x.x),
              "v"(x.y), "v"(x.z), "v"(x.w), "n"(LA), "n"(LA + 1));
    else
        asm(QG_SEG8H_TEXT ""
            : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3])
            : "v"(m[0]), "v"(m[1]), "v"(m[2]), "v"(m[3]), "v"(m[4]), "v"(m[5]), "v"(m[6]), "v"(m[7]), "v"(x.x),
              "v"(x.y), "v"(x.z), "v"(x.w), "n"(LA), "n"(LA + 1));
}

// Two floats as an fp16 pair, rounded to nearest even.
QG_DEV uint32_t qg_pk_rne(float a, float b) {
    const qg_h2 h = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, h);
}

// Eight consecutive activations as an fp16 matrix-core operand in the order the
// masked quant dwords use: elements 0, 2, 1, 3, 4, 6, 5, 7 (bytes 0 and 2 of a
// dword, then bytes 1 and 3, of each of two dwords).
QG_DEV qg_h8 qg_a_operand(const float4 lo, const float4 hi) {
    const uint4 r = make_uint4(qg_pk_rne(lo.x, lo.z), qg_pk_rne(lo.y, lo.w), qg_pk_rne(hi.x, hi.z),
                               qg_pk_rne(hi.y, hi.w));
    return __builtin_bit_cast(qg_h8, r);
}

// All-ones fp16 operand: a product with it sums the other operand over K.
QG_DEV qg_h8 qg_ones_h8() {
    return __builtin_bit_cast(qg_h8, make_uint4(0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u));
}

// Byte k of a packed word, as float.
QG_DEV float qg_byte_f(uint32_t v, int k) { return (float)((v >> (8 * k)) & 0xffu); }

// Buffer-resource constants: raw buffer loads past a resource's range return
// zeros without a memory access; the cache policy bit marks streamed loads.
constexpr uint32_t kQgOutOfRange = 0x80000000u;  // >= every resource size used here
constexpr int kQgNonTemporal = 2;
constexpr int kQgRawBufferFlags = 0x00020000;

// ---------------------------------------------------------------------------
// Q6_K: one 16-byte segment of low quant bits (ql: 4 dwords, 32 weights: the low
// nibbles of run "lo", the high nibbles of run "hi", 64 weights further on) with
// the matching 16 bytes of high bits (qh), against the activation pairs of lanes
// LA (dwords 0, 1) and LB (dwords 2, 3). Each 6-bit quant is assembled in place
// in its byte: low four bits from ql, bits 2PP..2PP+1 (run lo) or 2PP+4..2PP+5
// (run hi) of qh as bits 4-5, by one bit-field insert with the 0x0F0F0F0F mask
// `m4` (a scalar register: the insert has no literal form); masking bytes 0, 2 /
// 1, 3 with 0x003F003F leaves two fp16 subnormals q * 2^-24. Accumulators: lo0 /
// lo1 take bytes 0, 2 / 1, 3 of run lo (pairs x[r+0] / x[r+1]), hi0 / hi1 those
// of run hi (pairs x[r+2] / x[r+3]), r = 0 for dwords 0 and 2, 4 for 1 and 3.
// Hazards as for qg_q4_seg_dot: all sixteen masks are built before the first dot
// product, accumulators rotate every four instructions, s_nop 4 at the end.
template <int LA, int LB, int PP>
QG_DEV void qg_q6_seg_dot(float& lo0, float& hi0, float& lo1, float& hi1, const uint4 ql, const uint4 qh,
                          const uint32_t (&x)[8], uint32_t m4) {
    uint32_t m[16], t0, t1, t2;
    if constexpr (PP == 0) {
        asm("v_lshlrev_b32 %20, 4, %27\n\t"
            "v_bfi_b32 %21, %39, %23, %20\n\t"
            "v_and_b32 %4, 0x3f003f, %21\n\t"
            "v_lshrrev_b32 %22, 8, %21\n\t"
            "v_and_b32 %5, 0x3f003f, %22\n\t"
            "v_lshrrev_b32 %20, 4, %23\n\t"
            "v_bfi_b32 %21, %39, %20, %27\n\t"
            "v_and_b32 %6, 0x3f003f, %21\n\t"
            "v_lshrrev_b32 %22, 8, %21\n\t"
            "v_and_b32 %7, 0x3f003f, %22\n\t"
            "v_lshlrev_b32 %20, 4, %28\n\t"
            "v_bfi_b32 %21, %39, %24, %20\n\t"
            "v_and_b32 %8, 0x3f003f, %21\n\t"
            "v_lshrrev_b32 %22, 8, %21\n\t"
            "v_and_b32 %9, 0x3f003f, %22\n\t"
            "v_lshrrev_b32 %20, 4, %24\n\t"
            "v_bfi_b32 %21, %39, %20, %28\n\t"
            "v_and_b32 %10, 0x3f003f, %21\n\t"
            "v_lshrrev_b32 %22, 8, %21\n\t"
            "v_and_b32 %11, 0x3f003f, %22\n\t"
            "v_lshlrev_b32 %20, 4, %29\n\t"
            "v_bfi_b32 %21, %39, %25, %20\n\t"
            "v_and_b32 %12, 0x3f003f, %21\n\t"
            "v_lshrrev_b32 %22, 8, %21\n\t"
            "v_and_b32 %13, 0x3f003f, %22\n\t"
            "v_lshrrev_b32 %20, 4, %25\n\t"
            "v_bfi_b32 %21, %39, %20, %29\n\t"
            "v_and_b32 %14, 0x3f003f, %21\n\t"
            "v_lshrrev_b32 %22, 8, %21\n\t"
            "v_and_b32 %15, 0x3f003f, %22\n\t"
            "v_lshlrev_b32 %20, 4, %30\n\t"
            "v_bfi_b32 %21, %39, %26, %20\n\t"
            "v_and_b32 %16, 0x3f003f, %21\n\t"
            "v_lshrrev_b32 %22, 8, %21\n\t"
            "v_and_b32 %17, 0x3f003f, %22\n\t"
            "v_lshrrev_b32 %20, 4, %26\n\t"
            "v_bfi_b32 %21, %39, %20, %30\n\t"
            "v_and_b32 %18, 0x3f003f, %21\n\t"
            "v_lshrrev_b32 %22, 8, %21\n\t"
            "v_and_b32 %19, 0x3f003f, %22\n\t"
            "v_dot2c_f32_f16_dpp %0, %31, %4 row_newbcast:%40 row_mask:0xf bank_mask:0xf\n\t"
            "v_dot2c_f32_f16_dpp %2, %32, %5 row_newbcast:%40 row_mask:0xf bank_mask:0xf\n\t"
            "v_dot2c_f32_f16_dpp %1, %33, %6 row_newbcast:%40 row_mask:0xf bank_mask:0xf\n\t"
            "v_dot2c_f32_f16_dpp %3, %34, %7 row_newbcast:%40 row_mask:0xf bank_mask:0xf\n\t"
            "v_dot2c_f32_f16_dpp %0, %35, %8 row_newbcast:%40 row_mask:0xf bank_mask:0xf\n\t"
            "v_dot2c_f32_f16_dpp %2, %36, %9 row_newbcast:%40 row_mask:0xf bank_mask:0xf\n\t"
            "v_dot2c_f32_f16_dpp %1, %37, %10 row_newbcast:%40 row_mask:0xf bank_mask:0xf\n\t"
            "v_dot2c_f32_f16_dpp %3, %38, %11 row_newbcast:%40 row_mask:0xf bank_mask:0xf\n\t"
            "v_dot2c_f32_f16_dpp %0, %31, %12 row_newbcast:%41 row_mask:0xf bank_mask:0xf\n\t"
            "v_dot2c_f32_f16_dpp %2, %32, %13 row_newbcast:%41 row_mask:0xf bank_mask:0xf\n\t"
            "v_dot2c_f32_f16_dpp %1, %33, %14 row_newbcast:%41 row_mask:0xf bank_mask:0xf\n\t"
            "v_dot2c_f32_f16_dpp %3, %34, %15 row_newbcast:%41 row_mask:0xf bank_mask:0xf\n\t"
            "v_dot2c_f32_f16_dpp %0, %35, %16 row_newbcast:%41 row_mask:0xf bank_mask:0xf\n\t"
            "v_dot2c_f32_f16_dpp %2, %36, %17 row_newbcast:%41 row_mask:0xf bank_mask:0xf\n\t"
            "v_dot2c_f32_f16_dpp %1, %37, %18 row_newbcast:%41 row_mask:0xf bank_mask:0xf\n\t"
            "v_dot2c_f32_f16_dpp %3, %38, %19 row_newbcast:%41 row_mask:0xf bank_mask:0xf\n\t"
            "s_nop 4"
            : "+v"(lo0), "+v"(hi0), "+v"(lo1), "+v"(hi1), "=&v"(m[0]), "=&v"(m[1]), "=&v"(m[2]), "=&v"(m[3]),
              "=&v"(m[4]), "=&v"(m[5]), "=&v"(m[6]), "=&v"(m[7]), "=&v"(m[8]), "=&v"(m[9]), "=&v"(m[10]),
              "=&v"(m[11]), "=&v"(m[12]), "=&v"(m[13]), "=&v"(m[14]), "=&v"(m[15]), "=&v"(t0), "=&v"(t1), "=&v"(t2)
            : "v"(ql.x), "v"(ql.y), "v"(ql.z), "v"(ql.w), "v"(qh.x), "v"(qh.y), "v"(qh.z), "v"(qh.w), "v"(x[0]),
              "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]), "s"(m4), "n"(LA),
              "n"(LB));
    } else {
        asm("v_lshlrev_b32 %20, 2, %27\n\t"
            "v_bfi_b32 %21, %39, %23, %20\n\t"
            "v_and_b32 %4, 0x3f003f, %21\n\t"
            "v_lshrrev_b32 %22, 8, %21\n\t"
            "v_and_b32 %5, 0x3f003f, %22\n\t"
            "v_lshrrev_b32 %20, 4, %23\n\t"
            "v_lshrrev_b32 %22, 2, %27\n\t"
            "v_bfi_b32 %21, %39, %20, %22\n\t"
            "v_and_b32 %6, 0x3f003f, %21\n\t"
            "v_lshrrev_b32 %22, 8, %21\n\t"
            "v_and_b32 %7, 0x3f003f, %22\n\t"
            "v_lshlrev_b32 %20, 2, %28\n\t"
            "v_bfi_b32 %21, %39, %24, %20\n\t"
            "v_and_b32 %8, 0x3f003f, %21\n\t"
            "v_lshrrev_b32 %22, 8, %21\n\t"
            "v_and_b32 %9, 0x3f003f, %22\n\t"
            "v_lshrrev_b32 %20, 4, %24\n\t"
            "v_lshrrev_b32 %22, 2, %28\n\t"
            "v_bfi_b32 %21, %39, %20, %22\n\t"
            "v_and_b32 %10, 0x3f003f, %21\n\t"
            "v_lshrrev_b32 %22, 8, %21\n\t"
            "v_and_b32 %11, 0x3f003f, %22\n\t"
            "v_lshlrev_b32 %20, 2, %29\n\t"
            "v_bfi_b32 %21, %39, %25, %20\n\t"
            "v_and_b32 %12, 0x3f003f, %21\n\t"
            "v_lshrrev_b32 %22, 8, %21\n\t"
            "v_and_b32 %13, 0x3f003f, %22\n\t"
            "v_lshrrev_b32 %20, 4, %25\n\t"
            "v_lshrrev_b32 %22, 2, %29\n\t"
            "v_bfi_b32 %21, %39, %20, %22\n\t"
            "v_and_b32 %14, 0x3f003f, %21\n\t"
            "v_lshrrev_b32 %22, 8, %21\n\t"
            "v_and_b32 %15, 0x3f003f, %22\n\t"
            "v_lshlrev_b32 %20, 2, %30\n\t"
            "v_bfi_b32 %21, %39, %26, %20\n\t"
            "v_and_b32 %16, 0x3f003f, %21\n\t"
            "v_lshrrev_b32 %22, 8, %21\n\t"
            "v_and_b32 %17, 0x3f003f, %22\n\t"
            "v_lshrrev_b32 %20, 4, %26\n\t"
            "v_lshrrev_b32 %22, 2, %30\n\t"
            "v_bfi_b32 %21, %39, %20, %22\n\t"
            "v_and_b32 %18, 0x3f003f, %21\n\t"
            "v_lshrrev_b32 %22, 8, %21\n\t"
            "v_and_b32 %19, 0x3f003f, %22\n\t"
            "v_dot2c_f32_f16_dpp %0, %31, %4 row_newbcast:%40 row_mask:0xf bank_mask:0xf\n\t"
            "v_dot2c_f32_f16_dpp %2, %32, %5 row_newbcast:%40 row_mask:0xf bank_mask:0xf\n\t"
            "v_dot2c_f32_f16_dpp %1, %33, %6 row_newbcast:%40 row_mask:0xf bank_mask:0xf\n\t"
            "v_dot2c_f32_f16_dpp %3, %34, %7 row_newbcast:%40 row_mask:0xf bank_mask:0xf\n\t"
            "v_dot2c_f32_f16_dpp %0, %35, %8 row_newbcast:%40 row_mask:0xf bank_mask:0xf\n\t"
            "v_dot2c_f32_f16_dpp %2, %36, %9 row_newbcast:%40 row_mask:0xf bank_mask:0xf\n\t"
            "v_dot2c_f32_f16_dpp %1, %37, %10 row_newbcast:%40 row_mask:0xf bank_mask:0xf\n\t"
            "v_dot2c_f32_f16_dpp %3, %38, %11 row_newbcast:%40 row_mask:0xf bank_mask:0xf\n\t"
            "v_dot2c_f32_f16_dpp %0, %31, %12 row_newbcast:%41 row_mask:0xf bank_mask:0xf\n\t"
            "v_dot2c_f32_f16_dpp %2, %32, %13 row_newbcast:%41 row_mask:0xf bank_mask:0xf\n\t"
            "v_dot2c_f32_f16_dpp %1, %33, %14 row_newbcast:%41 row_mask:0xf bank_mask:0xf\n\t"
            "v_dot2c_f32_f16_dpp %3, %34, %15 row_newbcast:%41 row_mask:0xf bank_mask:0xf\n\t"
            "v_dot2c_f32_f16_dpp %0, %35, %16 row_newbcast:%41 row_mask:0xf bank_mask:0xf\n\t"
            "v_dot2c_f32_f16_dpp %2, %36, %17 row_newbcast:%41 row_mask:0xf bank_mask:0xf\n\t"
            "v_dot2c_f32_f16_dpp %1, %37, %18 row_newbcast:%41 row_mask:0xf bank_mask:0xf\n\t"
            "v_dot2c_f32_f16_dpp %3, %38, %19 row_newbcast:%41 row_mask:0xf bank_mask:0xf\n\t"
            "s_nop 4"
            : "+v"(lo0), "+v"(hi0), "+v"(lo1), "+v"(hi1), "=&v"(m[0]), "=&v"(m[1]), "=&v"(m[2]), "=&v"(m[3]),
              "=&v"(m[4]), "=&v"(m[5]), "=&v"(m[6]), "=&v"(m[7]), "=&v"(m[8]), "=&v"(m[9]), "=&v"(m[10]),
              "=&v"(m[11]), "=&v"(m[12]), "=&v"(m[13]), "=&v"(m[14]), "=&v"(m[15]), "=&v"(t0), "=&v"(t1), "=&v"(t2)
            : "v"(ql.x), "v"(ql.y), "v"(ql.z), "v"(ql.w), "v"(qh.x), "v"(qh.y), "v"(qh.z), "v"(qh.w), "v"(x[0]),
              "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]), "s"(m4), "n"(LA),
              "n"(LB));
    }
}

// ---------------------------------------------------------------------------
// Top-k support. Per 16-lane group (one 16-row tile, one value per lane): the
// first maximum (larger value, then lower index) and sum over the group of
// exp(v - max), returned in every lane as (max, index bits, sum, 0). NaN counts
// as -inf; a lane with valid == false takes part as (-inf, INT_MAX) and adds
// nothing. A group whose maximum is -inf has sum 0.
QG_DEV bool qg_better(float v, int i, float bv, int bi) { return v > bv || (v == bv && i < bi); }

QG_DEV float4 qg_group16_stats(float v, int idx, bool valid) {
    if (!valid || v != v) v = -__builtin_huge_valf();
    if (!valid) idx = 0x7fffffff;
    float m = v;
    int mi = idx;
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) {
        const float om = __shfl_xor(m, off, 64);
        const int oi = __shfl_xor(mi, off, 64);
        if (qg_better(om, oi, m, mi)) {
            m = om;
            mi = oi;
        }
    }
    float e = (m == -__builtin_huge_valf()) ? 0.f : __expf(v - m);
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) e += __shfl_xor(e, off, 64);
    return make_float4(m, __builtin_bit_cast(float, mi), e, 0.f);
}

// Order-preserving map of a float to an unsigned key (larger float, larger key;
// -0 as +0, NaN as -inf) and its inverse.
QG_DEV uint32_t qg_ord(float v) {
    if (v != v) v = -__builtin_huge_valf();
    v = v + 0.0f;  // -0 -> +0
    const uint32_t b = __builtin_bit_cast(uint32_t, v);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
QG_DEV float qg_unord(uint32_t o) { return __builtin_bit_cast(float, (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o); }

// ---------------------------------------------------------------------------
// Q4_K against int8 activations: one 16-byte quant segment (4 dwords, 32 weights)
// and this lane's activation dwords x = (low run bytes 0-3, 4-7, high run bytes
// 0-3, 4-7), taken from lane LA for quant dwords 0, 1 and LB for 2, 3 by the DPP
// row broadcast. Low nibbles masked with 0x0F0F0F0F are four unsigned bytes (the
// quants of the low sub-block), the high nibbles likewise after a shift by 4;
// v_dot4c_i32_i8 adds four byte products to an int32 accumulator: lo0 / lo1 take
// dwords 0, 2 / 1, 3 of the low sub-block, hi0 / hi1 those of the high one. All
// masks come first; each accumulator is re-read four instructions after its last
// write; s_nop 4 at the end (as for qg_q4_seg_dot).
template <int LA, int LB>
QG_DEV void qg_q4_seg_dot_i8(int& lo0, int& hi0, int& lo1, int& hi1, const uint4 q, const uint32_t (&x)[4]) {
    uint32_t m0, m1, m2, m3, m4, m5, m6, m7, t;
    asm("v_and_b32 %4, 0x0f0f0f0f, %13\n\t"
        "v_lshrrev_b32 %12, 4, %13\n\t"
        "v_and_b32 %5, 0x0f0f0f0f, %12\n\t"
        "v_and_b32 %6, 0x0f0f0f0f, %14\n\t"
        "v_lshrrev_b32 %12, 4, %14\n\t"
        "v_and_b32 %7, 0x0f0f0f0f, %12\n\t"
        "v_and_b32 %8, 0x0f0f0f0f, %15\n\t"
        "v_lshrrev_b32 %12, 4, %15\n\t"
        "v_and_b32 %9, 0x0f0f0f0f, %12\n\t"
        "v_and_b32 %10, 0x0f0f0f0f, %16\n\t"
        "v_lshrrev_b32 %12, 4, %16\n\t"
        "v_and_b32 %11, 0x0f0f0f0f, %12\n\t"
        "v_dot4c_i32_i8_dpp %0, %17, %4 row_newbcast:%21 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %1, %19, %5 row_newbcast:%21 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %2, %18, %6 row_newbcast:%21 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %3, %20, %7 row_newbcast:%21 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %0, %17, %8 row_newbcast:%22 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %1, %19, %9 row_newbcast:%22 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %2, %18, %10 row_newbcast:%22 row_mask:0xf bank_mask:0xf\n\t"
        "v_dot4c_i32_i8_dpp %3, %20, %11 row_newbcast:%22 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 4"
        : "+v"(lo0), "+v"(hi0), "+v"(lo1), "+v"(hi1), "=&v"(m0), "=&v"(m1), "=&v"(m2), "=&v"(m3), "=&v"(m4),
          "=&v"(m5), "=&v"(m6), "=&v"(m7), "=&v"(t)
        : "v"(q.x), "v"(q.y), "v"(q.z), "v"(q.w), "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "n"(LA), "n"(LB));
}
