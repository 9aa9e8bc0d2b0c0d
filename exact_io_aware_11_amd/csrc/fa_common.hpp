// fa_common.hpp -- gfx950 building blocks shared by the attention kernels.
//
// MFMA operand conventions used throughout (wave64, v_mfma_f32_32x32x16_bf16
// and v_mfma_f32_32x32x2_f32):
//   lane l, i32 = l % 32, g = l / 32
//   A operand (M x K):  lane l holds row i32 and K-slots (g, j), j < 8 (bf16)
//                       or the single K-slot g (fp32).
//   B operand (K x N):  lane l holds column i32 and the same K-slots.
//   C/D (32 x 32 fp32): lane l, register r holds C[8*(r/4) + 4*g + r%4][i32].
// A contraction is correct for any assignment of real indices to K-slots as
// long as the A and B operands use the same one; the kernels exploit that to
// feed a C accumulator straight back in as a B operand without shuffles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// 2^x on the transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

// Round-to-nearest-even fp32 -> bf16 pair (v_cvt_pk_bf16_f32), packed in 32 bits.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// acc + lo + hi of a packed bf16 pair (v_dot2c_f32_bf16 against (1, 1)).
__device__ __forceinline__ float sum_bf16x2(uint32_t packed, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), one, acc, false);
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (nontemporal: the data is used once).
__device__ __forceinline__ uint4 load_stream16(const void* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;

// Buffer resource over [base, base + bytes) for raw buffer loads (stride 0,
// bounds-checked: bytes past the end read as zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// 16-byte buffer -> LDS copy (buffer_load_dwordx4 ... lds): lane l's 16 bytes,
// read at byte offset voff of the resource, land at lds_base + 16*l (checked
// with an in-bounds probe); lds_base must be wave-uniform.  Preferred over the
// global_ form: the compiler treats a global_load_lds as a FLAT access that may
// touch LDS and then forces every later LDS-read wait down to lgkmcnt(0) until
// the copy is known complete, which serialises read prefetching.  The buffer
// form is tracked on vmcnt only, so LDS reads keep partial lgkmcnt waits.
__device__ __forceinline__ void b2lds16(__amdgpu_buffer_rsrc_t r, uint32_t voff, void* lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, voff, 0, 0, 0);
}

// 4-byte buffer -> LDS copy (buffer_load_dword ... lds): lane l's word lands
// at lds_base + 4*l.
__device__ __forceinline__ void b2lds4(__amdgpu_buffer_rsrc_t r, uint32_t voff, void* lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 4, voff, 0, 0, 0);
}

// 16-byte global -> LDS copy that bypasses registers (global_load_lds_dwordx4).
// Lane l's 16 bytes land at lds_base + 16*l; lds_base must be wave-uniform.
__device__ __forceinline__ void g2lds16(const void* gsrc, void* lds_base) {
    __builtin_amdgcn_global_load_lds(gsrc, (lds_void*)lds_base, 16, 0, 0);
}

// 4-byte global -> LDS copy (global_load_lds_dword): lane l's word lands at
// lds_base + 4*l.
__device__ __forceinline__ void g2lds4(const void* gsrc, void* lds_base) {
    __builtin_amdgcn_global_load_lds(gsrc, (lds_void*)lds_base, 4, 0, 0);
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// local lane j supplies the address of 4 consecutive 16-bit elements; local
// lane i receives element i%4 of the rows supplied by local lanes 4e + i/4,
// e = 0..3.  With lane j pointing at row r0 + j/4, columns c0 + 4*(j%4) .. +3
// of a row-major tile, lane i receives column c0 + i of rows r0 .. r0+3.
__device__ __forceinline__ uint2 lds_read_tr16x4(const void* p) {
    const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
    return __builtin_bit_cast(uint2, r);
}

// Eight packed bf16 (one 16-byte chunk) -> one MFMA operand.
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// Element c (0..7) of four 16-byte rows r0..r3, packed as 4 x bf16 (one 8-byte
// store of a transposed tile row).
__device__ __forceinline__ uint2 column4(const uint4& r0, const uint4& r1, const uint4& r2,
                                         const uint4& r3, int c) {
    const uint32_t* a = reinterpret_cast<const uint32_t*>(&r0);
    const uint32_t* b = reinterpret_cast<const uint32_t*>(&r1);
    const uint32_t* e = reinterpret_cast<const uint32_t*>(&r2);
    const uint32_t* f = reinterpret_cast<const uint32_t*>(&r3);
    const int wi = c >> 1;
    uint32_t lo, hi;
    if (c & 1) {
        lo = (a[wi] >> 16) | (b[wi] & 0xffff0000u);
        hi = (e[wi] >> 16) | (f[wi] & 0xffff0000u);
    } else {
        lo = (a[wi] & 0xffffu) | (b[wi] << 16);
        hi = (e[wi] & 0xffffu) | (f[wi] << 16);
    }
    return make_uint2(lo, hi);
}

// Position of key (or query) k inside a transposed tile row, for the
// permutation that lets a 32x32 C accumulator be used directly as a
// K-slot-ordered B operand: within each group of 16, the 4-element quads are
// stored in the order 0, 2, 1, 3.
__device__ __forceinline__ int perm16(int k) {
    const int quad = (k >> 2) & 3;
    const int pq = (quad == 1) ? 2 : (quad == 2 ? 1 : quad);
    return (k & ~15) | (pq << 2) | (k & 3);
}

// Map the flat block id to (query head, query tile).  One sweep of BH
// consecutive ids covers every head once, so with a causal mask the most
// expensive (last) query tiles of all heads are issued first.  Within a sweep
// the G query heads that share a K/V head are NG = BH / G ids apart: the
// hardware deals blocks round-robin to the 8 XCDs, so when NG is a multiple
// of 8 a whole group -- and every tile of it -- runs on one XCD and shares
// that XCD's L2 copy of its K/V.  G = 1 gives bh = id % BH.
__device__ __forceinline__ void fwd_tile_of(int bid, int BH, int G, int nqt, bool causal,
                                            int& bh, int& qt) {
    const int j = bid % BH, NG = BH / G;
    bh = (j % NG) * G + j / NG;
    const int t = bid / BH;
    qt = causal ? (nqt - 1 - t) : t;
}

// Max / sum of x over lanes l and l ^ 32, in every lane: v_permlane32_swap of
// x with itself gives (x of lanes 0-31 twice, x of lanes 32-63 twice); the
// max or sum of its two results is the xor-32 reduction (checked with an
// in-bounds probe of the builtin).
__device__ __forceinline__ float xor32_max(float x) {
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// DPP sums inside a row of 16 lanes (quad_perm, half-mirror, mirror).
__device__ __forceinline__ float dpp_sum8(float v) {
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));  // [1,0,3,2]
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));  // [2,3,0,1]
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true)); // half mirror
    return v;
}
__device__ __forceinline__ float dpp_sum16(float v) {
    v = dpp_sum8(v);
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true)); // row mirror
    return v;
}

// XOR swizzles of the 16-byte chunks of an LDS tile row (2*D bytes, no
// padding), applied when the tile is copied in and when it is read.
//  k_swz: rows read one 16-byte chunk per lane by 32 consecutive rows.
//  v_swz: rows read with the transposing 8-byte read (4 rows x 32 bytes per
//         16-lane group).  D = 64, 128 or 256.
//  rt_swz: both patterns on the same tile (4*(row%4) + (row/4)%4).
template <int D>
__device__ __forceinline__ int k_swz(int row) { return row & (D / 8 - 1); }
template <int D>
__device__ __forceinline__ int v_swz(int row) {
    // rows of 256 or 512 bytes start in the same bank: shift rows r..r+3 of a
    // 4-row group by 64 bytes each; 128-byte rows pair up, shift by 64 bytes
    return D >= 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
}
template <int D>
__device__ __forceinline__ int rt_swz(int row) {
    return (4 * (row & 3) + ((row >> 2) & 3)) & (D / 8 - 1);
}

}  // namespace fa
