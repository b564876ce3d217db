// Device helpers shared by the LISA kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lisa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Two fp32 values -> packed bf16 bits (lo in bits 0..15), round to nearest
// even: one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2v_t));
}
// fp32 -> bf16 bits, round to nearest even.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return pack_bf16x2(f, 0.0f) & 0xFFFFu; }

// Element traits: storage type T is uint16_t (bf16 bit pattern) or float.
template <typename T> struct Elt;
template <> struct Elt<uint16_t> {
    static constexpr int kBytes = 2;
    __device__ static __forceinline__ float load(const uint16_t *p) { return bf16_bits_to_f32(*p); }
    __device__ static __forceinline__ float to_f32(uint16_t x) { return bf16_bits_to_f32(x); }
    __device__ static __forceinline__ uint16_t from_f32(float f) { return (uint16_t)f32_to_bf16_bits(f); }
};
template <> struct Elt<float> {
    static constexpr int kBytes = 4;
    __device__ static __forceinline__ float load(const float *p) { return *p; }
    __device__ static __forceinline__ float to_f32(float x) { return x; }
    __device__ static __forceinline__ float from_f32(float f) { return f; }
};

// A 16x16x32 MFMA operand fragment: 8 consecutive K-elements of one row (A)
// or one column (B) per lane.  Lane l covers row/column l%16 and K-elements
// 8*(l/16) .. 8*(l/16)+7.  bf16 uses one v_mfma_f32_16x16x32_bf16; fp32 uses
// eight v_mfma_f32_16x16x4_f32, element e of every lane forming the e-th
// K-slice.  Both produce the same accumulator layout: lane l holds
// D[4*(l/16)+r][l%16], r = 0..3.
template <typename T> struct Frag;
template <> struct Frag<uint16_t> {
    u32x4 v;
    __device__ __forceinline__ void zero() { v = u32x4{0u, 0u, 0u, 0u}; }
    __device__ __forceinline__ void load(const uint16_t *p) { v = *reinterpret_cast<const u32x4 *>(p); }
    // set from 8 fp32 values (rounded to bf16)
    __device__ __forceinline__ void set(const float *x) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    }
    __device__ __forceinline__ void set_bits(const uint16_t *x) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (uint32_t)x[2 * i] | ((uint32_t)x[2 * i + 1] << 16);
    }
};
template <> struct Frag<float> {
    f32x4 lo, hi;
    __device__ __forceinline__ void zero() { lo = f32x4{0, 0, 0, 0}; hi = lo; }
    __device__ __forceinline__ void load(const float *p) {
        lo = reinterpret_cast<const f32x4 *>(p)[0];
        hi = reinterpret_cast<const f32x4 *>(p)[1];
    }
    __device__ __forceinline__ void set(const float *x) {
        lo = f32x4{x[0], x[1], x[2], x[3]};
        hi = f32x4{x[4], x[5], x[6], x[7]};
    }
    __device__ __forceinline__ void set_bits(const float *x) { set(x); }
};

__device__ __forceinline__ f32x4 mma16(const Frag<uint16_t> &a, const Frag<uint16_t> &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a.v),
                                                   __builtin_bit_cast(bf16x8_t, b.v), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(const Frag<float> &a, const Frag<float> &b, f32x4 c) {
#pragma unroll
    for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[e], b.lo[e], c, 0, 0, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[e], b.hi[e], c, 0, 0, 0);
    return c;
}

// Total order on fp32 scores as unsigned keys: larger key = larger score;
// -0.0 and +0.0 map to the same key.
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (f == 0.0f) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Workgroups are dispatched round-robin over the 8 XCDs of the chip, each
// with its own L2.  Map the hardware block id to a logical id such that each
// XCD receives one contiguous range of logical ids (neighbouring logical
// blocks then share that XCD's L2).
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
    constexpr int X = 8;
    const int per = nblocks / X, rem = nblocks % X;
    const int xcd = bid % X, j = bid / X;
    return xcd * per + (xcd < rem ? xcd : rem) + j;
}

// Raw buffer access: a wave-uniform descriptor over [base, base + bytes).
// Loads whose byte offset falls outside return zeros, so tails and invalid
// rows need no branch; offsets are 32-bit VGPR values.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
// The base and size must be wave-uniform; readfirstlane makes that explicit so
// the descriptor lives in SGPRs (otherwise each load becomes a waterfall loop).
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void *p = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                             0x00020000 /* gfx9-family raw buffer word 3 */);
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t voff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0u, 0));
}
// The same with a wave-uniform part of the offset in soffset (an SGPR, so a
// constant part costs no VGPR).  Callers keep voff + soff inside the
// descriptor wherever the data is wanted; a zero-size descriptor reads zeros
// whatever the offsets.
__device__ __forceinline__ u32x4 buf_load16s(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
constexpr uint32_t kOffNone = 0x80000000u;  // an offset beyond every descriptor used here

// Fill a 16x16x32 fragment from a buffer: 8 consecutive elements at byte offset voff.
__device__ __forceinline__ void frag_buf_load(Frag<uint16_t> &f, rsrc_t r, uint32_t voff) {
    f.v = buf_load16(r, voff);
}
__device__ __forceinline__ void frag_buf_load(Frag<float> &f, rsrc_t r, uint32_t voff) {
    f.lo = __builtin_bit_cast(f32x4, buf_load16(r, voff));
    f.hi = __builtin_bit_cast(f32x4, buf_load16(r, voff + 16u));
}
__device__ __forceinline__ void frag_buf_load(Frag<uint16_t> &f, rsrc_t r, uint32_t voff, uint32_t soff) {
    f.v = buf_load16s(r, voff, soff);
}
__device__ __forceinline__ void frag_buf_load(Frag<float> &f, rsrc_t r, uint32_t voff, uint32_t soff) {
    f.lo = __builtin_bit_cast(f32x4, buf_load16s(r, voff, soff));
    f.hi = __builtin_bit_cast(f32x4, buf_load16s(r, voff + 16u, soff));
}

// gfx950 transposing LDS read (ds_read_b64_tr_b16): in each 16-lane block,
// lane l gets element l % 4 of the 4-element (8-byte) row piece addressed by
// lane 4e + l / 4, e = 0..3.  With lane j of the block addressing row
// (base + j / 4) at column 4 (j % 4) + c0, lane l receives rows base ..
// base + 3 of column c0 + l % 16: four consecutive K-elements of an MFMA
// operand read across rows of a row-major tile.
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
__device__ __forceinline__ u32x2 lds_read_tr16(const void *lds_byte_ptr) {
    lds_bf16x4_t *p = (lds_bf16x4_t *)(__attribute__((address_space(3))) unsigned char *)(
        (__attribute__((address_space(3))) void *)lds_byte_ptr);
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(p));
}

// Number of set bits of a 64-lane mask in the lanes below this one.
__device__ __forceinline__ uint32_t mbcnt64(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Make this wave's LDS writes visible to its own lanes before they read.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---- cross-lane helpers (DPP and gfx950 permlane swaps: VALU only, no LDS) --
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v),
                                                                 __builtin_bit_cast(int, v), CTRL,
                                                                 0xF, 0xF, false));
}
// The swaps return {v of this lane, v of lane^16 (or ^32)} in some order, so
// a symmetric combine of the two halves gives the pairwise result.
__device__ __forceinline__ float max_xor16(float v) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// over lanes l, l^16, l^32, l^48 (the four lane groups of a 16x16 MFMA tile)
__device__ __forceinline__ float wave_max_across16(float v) { return max_xor32(max_xor16(v)); }
__device__ __forceinline__ float wave_sum_across16(float v) { return sum_xor32(sum_xor16(v)); }

// over all 64 lanes
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_f32<0xB1>(v));   // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp_f32<0x4E>(v));   // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp_f32<0x141>(v));  // row_half_mirror
    v = fmaxf(v, dpp_f32<0x140>(v));  // row_mirror
    return wave_max_across16(v);
}
__device__ __forceinline__ float wave_min(float v) { return -wave_max(-v); }

// over the 16 lanes of each row (result in every lane of the row)
__device__ __forceinline__ float row_max(float v) {
    v = fmaxf(v, dpp_f32<0xB1>(v));   // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp_f32<0x4E>(v));   // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp_f32<0x141>(v));  // row_half_mirror
    v = fmaxf(v, dpp_f32<0x140>(v));  // row_mirror
    return v;
}
__device__ __forceinline__ float row_min(float v) { return -row_max(-v); }

__device__ __forceinline__ uint32_t max_u32_xor16(uint32_t v) {
    const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return max((uint32_t)p[0], (uint32_t)p[1]);
}
__device__ __forceinline__ uint32_t max_u32_xor32(uint32_t v) {
    const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return max((uint32_t)p[0], (uint32_t)p[1]);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_u32<0xB1>(v, v));
    v = max(v, dpp_u32<0x4E>(v, v));
    v = max(v, dpp_u32<0x141>(v, v));
    v = max(v, dpp_u32<0x140>(v, v));
    return max_u32_xor32(max_u32_xor16(v));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { return ~wave_max_u32(~v); }

// Inclusive prefix sum within each 16-lane row (row shifts; lanes shifted in
// from outside the row contribute 0).
__device__ __forceinline__ uint32_t row_inclusive_scan(uint32_t v) {
    v += dpp_u32<0x111>(0u, v);  // row_shr:1
    v += dpp_u32<0x112>(0u, v);  // row_shr:2
    v += dpp_u32<0x114>(0u, v);  // row_shr:4
    v += dpp_u32<0x118>(0u, v);  // row_shr:8
    return v;
}
// Lane 15 of each 16-lane row, broadcast to the whole row (row_newbcast:15).
__device__ __forceinline__ uint32_t row_broadcast15(uint32_t v) { return dpp_u32<0x15F>(0u, v); }

// Inclusive prefix sum over the 64 lanes of a wave (row shifts, then row
// broadcasts of lanes 15 and 31).
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
    v = row_inclusive_scan(v);
    v += dpp_u32<0x142, 0xA>(0u, v);  // row_bcast:15 into rows 1 and 3
    v += dpp_u32<0x143, 0xC>(0u, v);  // row_bcast:31 into rows 2 and 3
    return v;
}

// Exclusive prefix sum over a block of NT threads (NT multiple of 64, at
// most 64 waves).  `tmp` must hold NT/64 + 1 words; returns the exclusive
// prefix and the block total in *total.  Contains __syncthreads().
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *tmp, uint32_t *total) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t inc = wave_inclusive_scan(v);
    if (lane == 63) tmp[wave] = inc;
    __syncthreads();
    if (wave == 0) {
        const uint32_t x = lane < NW ? tmp[lane] : 0u;
        const uint32_t xs = wave_inclusive_scan(x);
        if (lane < NW) tmp[lane] = xs - x;
        if (lane == NW - 1) tmp[NW] = xs;
    }
    __syncthreads();
    const uint32_t res = tmp[wave] + inc - v;
    *total = tmp[NW];
    __syncthreads();
    return res;
}

}  // namespace lisa
